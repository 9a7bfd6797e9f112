// Split-KV paged decode of absorbed MLA on gfx950.
//
// Per work unit u = (sequence b, query i) the attention is, for all 128 heads
// at once (all heads share the cached latent, so this is a dense contraction):
//   S^T[t, h] = (c_KV[t] . q_abs[h] + k_R[t] . q_R[h]) * scale     (K = 576)
//   out_latent[h] = sum_t softmax_t(S[h, t]) * c_KV[t]            (K = 64 per page)
// ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 4, path B for the scores; the
// output stays in latent space and is up-projected by W_UV afterwards.)
//
// Work split: the 32-token tiles (half pages) of all units are laid end to end;
// workgroup g takes the contiguous range [g*chunk, (g+1)*chunk) of that list
// (chunk = ceil(total/W)), so every compute unit streams the same number of tiles
// whatever the length mix (the prefix sums of tiles per unit come from a wave scan
// inside each workgroup for up to 64 units, else from plan_kernel).  A unit that
// lies inside one range is finished in place; a unit cut by range borders leaves
// one normalised partial per piece (bf16, with an fp32 lse; slot 2g for the first
// segment of workgroup g, 2g+1 for its last), merged by log-sum-exp afterwards.
//
// Workgroup: 256 threads = 4 waves, one per SIMD.  Pages are processed as
// 32-token tiles (36 KiB) copied HBM -> LDS with direct 16-byte loads
// (global_load_lds_dwordx4) two tiles ahead into a 4-slot ring, plus two 8 KiB
// P buffers: the 160 KiB of LDS exactly.  Wave w computes the scores of heads
// 32w..32w+31 (its 32 queries live in 144 VGPRs) and the output of all heads
// for latent columns 128w..128w+127 (256 accumulator registers for the whole
// segment); see decode_kernel for the per-tile steps.
// LDS layout of a tile: a latent region of token rows (64 sixteen-byte chunks)
// and a RoPE region (8 chunks per token), each with an XOR swizzle of the chunk
// index that keeps both the row reads of QK (16 tokens, one chunk) and the
// 4-row transposing reads of PV free of bank conflicts.
//
// The same kernel decodes the MXFP8 cache of mxfp8.h (decode_kernel<true>): the
// tiles' codes and scales are staged per wave and dequantised to the bf16 tile
// layout above in a ring of 3 slots (see the constants kF8*); everything from the
// tile slot on is the bf16 kernel's.
#include <mutex>

#include "common.h"
#include "mxfp8.h"

namespace mla {

namespace {

constexpr int kThreads = 256;
// Tokens per tile: the cache streams in half pages, and the pages of all work units are
// split across workgroups in whole tiles.
constexpr int kTile = 32;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  const uint16_t* q_abs;
  const uint16_t* q_r;
  const uint16_t* kv;        // bf16 cache [num_pages, 64, 576], or
  const unsigned char* kv8;  // MXFP8 cache [num_pages, 64, 656] (rows of mxfp8.h)
  const int32_t* bt;
  const int32_t* seqlens;
  uint16_t* out_latent;
  float* lse;
  int32_t* cum;
  uint16_t* part_o;    // [2W, 128, 512] bf16 normalised partial outputs
  float* part_lse;
  int64_t num_pages;
  int last_page;     // min(num_pages, 2^31) - 1: page ids are int32, so clamps stay 32-bit
  int batch, s_q, max_blocks;
  int min_chunk;     // fewest tiles a workgroup takes (see split_chunk)
  float scale_log2;  // scale * log2(e)
};

// Tiles per workgroup range: the tiles split evenly over the W workgroups, but never
// fewer than min_chunk per workgroup (a workgroup's fixed costs -- its queries, its
// partial output and the merge of that partial -- then pay for enough tiles).
__device__ __forceinline__ int split_chunk(int total, int W, int min_chunk) {
  const int even = (total + W - 1) / W;
  return even > min_chunk ? even : min_chunk;
}

// Segment-aware split.  A workgroup pays about 20k cycles for every segment it starts
// (queries, first tiles, epilogue), as much as ~6 tiles of streaming; with equal tile
// counts a workgroup whose range spans two or three units finishes that much later than
// one inside a single unit, and the slowest sets the launch time (batch 64: 517k
// cycles against a 481k mean).  So the library's own split (min_chunk > 1) lays the units
// end to end on a cost line where each unit with tiles costs its tiles plus kSegCost, and
// cuts that line evenly: a range that takes in a unit start gets kSegCost fewer tiles.
// Kept to even splits where it cannot pay: ranges under kCostSplitMin tiles (the
// segment cost is then a large share of a range, and ranges shift by several tiles),
// and splits whose range boundaries already fall on unit starts (every workgroup has one
// segment; equal sequence lengths).  Explicit num_splits (min_chunk 1) split evenly.
// (kSegCost and kCostSplitMin are in common.h: the host checks bound the cost line.)
__device__ __forceinline__ int split_seg_cost(int even_chunk, bool aligned, int min_chunk) {
  return (min_chunk > 1 && even_chunk >= kCostSplitMin && !aligned) ? kSegCost : 0;
}

// LDS swizzles (the LDS has 64 banks of 4 bytes; a 16-byte read by 16 lanes, or
// an 8-byte transposing read by 32 lanes, moves 256 bytes per cycle).
// Latent rows (1024 B, a multiple of the bank width): chunk c of token t sits at
// position c ^ swz_lat(t), which spreads 16 consecutive tokens reading one chunk
// and the 4-token x 4-chunk blocks of the transposing reads over all banks.
__device__ __forceinline__ int swz_lat(int t) { return 4 * (t & 3) + ((t >> 2) & 3); }
// RoPE rows (128 B, two per bank row): chunk c of token t sits at c ^ swz_rope(t).
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 7; }

__device__ __forceinline__ int clamp_len(int L, int max_blocks) {
  return L < 0 ? 0 : (L > max_blocks * kPage ? max_blocks * kPage : L);
}

// Visible keys of unit u (query i of sequence b).
__device__ __forceinline__ int unit_visible(const DecodeArgs& a, int u) {
  const int b = u / a.s_q, i = u - b * a.s_q;
  return clamp_len(a.seqlens[b], a.max_blocks) - a.s_q + i + 1;
}

// ---------------------------------------------------------------------------- plan

// Up to this many work units (batch x queries), each decode workgroup computes the
// tile prefix sums itself and the plan kernel is not launched.
constexpr int kSelfPlanUnits = 64;

// Tiles of a work unit: its visible tokens in 32-token tiles (the work split's grain).
__device__ __forceinline__ int unit_tiles(int n_visible) {
  return n_visible > 0 ? (n_visible + kTile - 1) / kTile : 0;
}

// The split plan of U work units, plan[2U + 3] int32: plan[0..U] tile prefix sums
// (cum[u + 1] = cum[u] + ceil(visible_u / 32)), plan[U + 1 .. 2U + 1] the cost-line prefix
// sums (ccum[u + 1] = ccum[u] + tiles_u + seg if tiles_u > 0), plan[2U + 2] = seg (0 or
// kSegCost).  W is the decode's workgroup count.
__global__ __attribute__((amdgpu_flat_work_group_size(1024, 1024)))
void plan_kernel(DecodeArgs a, int32_t* cum, int W) {
  __shared__ int32_t warp_tot[16], warp_nz[16];
  __shared__ int32_t carry_s, carry_nz;
  const int U = a.batch * a.s_q;
  int32_t* ccum = cum + U + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { carry_s = 0; carry_nz = 0; cum[0] = 0; ccum[0] = 0; }
  __syncthreads();
  // pass 1: tile prefix sums into cum, prefix counts of units with tiles into ccum
  for (int base = 0; base < U; base += 1024) {
    const int u = base + tid;
    const int tiles = u < U ? unit_tiles(unit_visible(a, u)) : 0;
    int x = tiles, z = tiles > 0 ? 1 : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64), yz = __shfl_up(z, off, 64);
      if (lane >= off) { x += y; z += yz; }
    }
    if (lane == 63) { warp_tot[wave] = x; warp_nz[wave] = z; }
    __syncthreads();
    int before = carry_s, before_nz = carry_nz;
    for (int w = 0; w < wave; ++w) { before += warp_tot[w]; before_nz += warp_nz[w]; }
    if (u < U) { cum[u + 1] = before + x; ccum[u + 1] = before_nz + z; }
    __syncthreads();
    if (tid == 1023) { carry_s = before + x; carry_nz = before_nz + z; }
    __syncthreads();
  }
  // pass 2: do the even split's range boundaries all fall on unit starts?
  const int total = carry_s;
  const int chunk0 = split_chunk(total, W, a.min_chunk);
  int off_grid = 0;
  for (int u = tid; u < U; u += 1024)
    off_grid |= (cum[u + 1] > cum[u] && cum[u] % chunk0 != 0) ? 1 : 0;
  const int seg = split_seg_cost(chunk0, __syncthreads_or(off_grid) == 0, a.min_chunk);
  // pass 3: cost-line prefix sums
  for (int u = tid; u < U; u += 1024) ccum[u + 1] = cum[u + 1] + seg * ccum[u + 1];
  if (tid == 0) cum[2 * U + 2] = seg;
}

// ---------------------------------------------------------------------------- decode

// The pages are processed in tiles of 32 tokens (half a page, 36 KiB).  LDS:
// a ring of 4 tile slots (4 x 36 KiB) and two P buffers (2 x 8 KiB): the
// 160 KiB of LDS exactly.  Tile slot layout: latent region [32 tokens][1024 B]
// at offset 0, RoPE region [32 tokens][128 B] at offset 32768, both swizzled as
// above.
constexpr int kTileBytes = kTile * kRowBytes;        // 36864
constexpr int kRopeRegion = kTile * kLatent * 2;     // 32768
constexpr int kSlots = 4;
constexpr int kPBytes = kHeads * kTile * 2;          // 8192: P of one tile, [128 heads][32 tokens] bf16
constexpr int kLoadsPerTile = kTileBytes / 16 / kThreads;   // 9 direct loads per thread per tile
static_assert(kTileBytes % (16 * kThreads) == 0, "tile must split evenly over the workgroup");

// MXFP8 cache: a 32-token tile is 20 992 bytes in HBM.  LDS holds a ring of 3
// bf16 tile slots (the dequantised latent and the RoPE rows, laid out and swizzled
// as above) and a two-deep staging of the tile's codes and scale bytes.  Wave w
// loads the codes, scales and RoPE rows of tokens 8w .. 8w+7 and dequantises
// those rows itself, so staging needs no barrier: 4 code loads (two 512-byte rows
// each), 1 RoPE load, 1 four-byte-per-lane scale load.
constexpr int kF8Slots = 3;
constexpr int kF8TileBytes = kTile * kF8RowBytes;             // 20992
constexpr int kF8Stage = kTile * kLatent;                     // 16384 code bytes of a tile
constexpr int kF8ScaleStage = 4 * 256;                        // per wave: 32 lanes x 4 B, then a copy
constexpr int kF8StageOff = kF8Slots * kTileBytes;            // 110592
constexpr int kF8ScaleOff = kF8StageOff + 2 * kF8Stage;       // 143360
constexpr int kF8LdsBytes = kF8ScaleOff + 2 * kF8ScaleStage;  // 145408
constexpr int kF8LoadsPerTile = 6;   // the "s_waitcnt vmcnt(6)" below count these
static_assert(kF8LoadsPerTile == 6, "vmcnt literal");
static_assert(kF8LdsBytes % 1024 == 0 && kF8LdsBytes + 2 * kHeads * kTile * 2 <= 163840, "LDS budget");

// Tile copy HBM -> LDS: wave w copies the latent rows of tokens w, w+4, ...,
// w+28 (one 64-lane direct load per row, lane l = chunk position l) and the
// RoPE rows of tokens 8w .. 8w+7 (one load; lane l -> token 8w + l/8, chunk
// position l%8).  The per-lane global byte offsets below are constant.
struct TileLoadOffsets {
  uint32_t lat[4];   // latent row offset for tokens t with t % 16 == w + 4k
  uint32_t rope;     // RoPE offset relative to token 8w
};

__device__ __forceinline__ TileLoadOffsets tile_load_offsets(int lane, int wave_u) {
  TileLoadOffsets o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o.lat[k] = (uint32_t)((lane ^ swz_lat(wave_u + 4 * k)) * 16);
  o.rope = (uint32_t)((lane >> 3) * kRowBytes + kLatent * 2 + ((lane & 7) ^ ((4 * wave_u + (lane >> 4)) & 7)) * 16);
  return o;
}

// One 16-byte-per-lane direct load HBM -> LDS (global_load_lds_dwordx4): lane l
// reads sbase + voff and its 16 bytes land at LDS byte address lds + 16 l.
// Issued as inline asm so the compiler's wait-count model does not see the
// LDS write: it would otherwise wait for every load in flight (including the
// prefetch of the next tiles) before each LDS read.  The kernel waits for
// these loads itself with explicit vmcnt waits.  The leading s_nop covers the
// one wait state an M0 write needs before an LDS DMA instruction.  The cache
// is read once, so the loads are non-temporal: with `nt` the page stream runs
// at about 7.0 TB/s on MI355X, without it at about 6.2 TB/s.  No "memory"
// clobber: the load only writes a ring slot that no wave reads until a later
// tile barrier, and a volatile asm is never moved across that barrier.
__device__ __forceinline__ void dma_b128(const unsigned char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds));
}

// The same with 4 bytes per lane (global_load_lds_dword): lane l's bytes land at lds + 4 l.
__device__ __forceinline__ void dma_b32(const unsigned char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds));
}

// Query rows into a wave's LDS stage (the bf16-cache decode): the same 16-byte direct load
// without `nt` (the workgroups that share a unit read its queries again) and with a
// "memory" clobber, so that no LDS read of the stage moves across it.
__device__ __forceinline__ void dma_q_b128(const unsigned char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// The 9 direct loads of one tile.  Rows at or past `valid` (only in a
// sequence's last tile) are fetched from row 0 of the tile instead: they are
// masked out of the softmax, and loading finite data keeps 0 * V finite even
// when the unused rows of the cache hold NaN or Inf bit patterns.
__device__ __forceinline__ void issue_tile(const unsigned char* __restrict__ src, uint32_t lslot,
                                           const TileLoadOffsets& off, int wave_u, int lane, int valid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = wave_u + 4 * i;
    const int trow = t < valid ? t : 0;
    dma_b128(src + trow * kRowBytes, off.lat[i & 3], lslot + t * 1024);
  }
  const uint32_t ro = (8 * wave_u + (lane >> 3) < valid) ? 8 * wave_u * kRowBytes + off.rope
                                                          : (uint32_t)(kLatent * 2 + (lane & 7) * 16);
  dma_b128(src, ro, lslot + kRopeRegion + 1024 * wave_u);
}

// The lane id through an opaque move: address offsets derived from it are
// recomputed where they are used instead of being hoisted out of every loop
// and kept live (the registers are needed for the queries and accumulators).
__device__ __forceinline__ int opaque_lane() {
  int v = (int)__lane_id();
  asm volatile("v_mov_b32 %0, %0" : "+v"(v));
  return v;
}

// A per-step LDS address the compiler may not precompute: in the first step of a
// segment the slot numbers are constants, and without this the compiler would fold
// those addresses, hoist them out of the segment loop and, short of registers, spill
// them; their reloads then sit in the memory counter in front of the steady loop,
// whose counter waits it would have to tighten to zero on every step.  No instruction.
__device__ __forceinline__ uint32_t step_local(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// max(a, b, c) in one instruction (the compiler would quiet each operand first).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Softmax reference.  Each segment takes its per-head reference maximum from
// its first tile and keeps it: P = 2^(s - m_ref) in log2 units, so the O
// accumulators are never rescaled and any wave may accumulate any head.  A
// later score more than kHeadroom above the reference (P beyond 2^64, far
// outside real attention logits) makes the workgroup redo the segment once
// with the segment's true maximum as the reference, so the fp32 accumulators
// cannot overflow.
constexpr float kHeadroom = 64.0f;
// The bf16-cache decode stages a segment's queries through LDS in two rounds (k-steps
// 0..15 and 32..33, then 16..31 and 34..35), each wave in its own 18 KiB of ring slots 2
// and 3, which no load touches before the first step: 32 heads x 512 B of latent chunks,
// then 32 heads x 64 B of RoPE chunks.
constexpr int kQStageBytes = 18432;
constexpr int kQStageRope = 16384;
static_assert(2 * kTileBytes + 4 * kQStageBytes <= kSlots * kTileBytes, "query stage in slots 2 and 3");
// Code placement of the bf16-cache kernel's steady-state loop.  With the loop's first
// instruction at 28 mod 32 bytes (so at 28 or 60 mod 64) the batch-4 x 2-query workload
// measured 3-4% faster than at the other 4-byte offsets (a sweep of s_nop padding in the
// prologue, code otherwise identical; the two query units of a sequence then fetch 1.03x
// the cache bytes instead of up to 1.29x); batch 64 and the short workloads did not move.
// The cause is not known.  This many s_nop instructions, executed once per workgroup,
// put the loop there; a CPU test checks the offset in the compiled code.
constexpr int kLoopPadNops = 9;

// Scalar read of a value that no kernel of the launch writes (block table,
// sequence lengths, plan_kernel's prefix sums): through the constant address space
// the load is a scalar one, counted by lgkmcnt, so waiting for it never waits
// for the tile loads in flight (a vector load would, as those share vmcnt).
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// A workgroup's share of the work: tiles [start, end) of the tiles of all units laid
// end to end, unit u holding tile `start`, and ubeg, the first tile of unit u.  The
// ranges cut the cost line (see split_seg_cost) evenly: workgroup g takes cost positions
// [g chunk, (g + 1) chunk), chunk = split_chunk(T, W, min_chunk) over the line's length
// T; a cost position c in unit u's interval [C_u, C_u+1) is tile cum_u + max(0, c - C_u -
// seg).  With seg = 0 this is the even split of the tiles.
struct WorkRange {
  int start, end, u, ubeg;
};

// False when the workgroup has no tiles.  Up to kSelfPlanUnits units every wave scans
// the lengths itself (lane u holds unit u) and workgroup 0 publishes the plan (see
// plan_kernel) for the combine; more units read plan_kernel's array.
__device__ __forceinline__ bool work_range(const DecodeArgs& a, int lane, WorkRange& r) {
  const int U = a.batch * a.s_q;
  const int W = (int)gridDim.x;
  int total, T, seg, pex = 0, cpex = 0;   // pex, cpex: this lane's unit's tile and cost prefixes
  const bool self_plan = U <= kSelfPlanUnits;
  if (self_plan) {
    const int tiles = lane < U ? unit_tiles(unit_visible(a, lane)) : 0;
    int x = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    total = __builtin_amdgcn_readlane(x, 63);
    pex = x - tiles;
    const int chunk0 = split_chunk(total, W, a.min_chunk);
    seg = 0;
    cpex = pex;
    T = total;
    if (a.min_chunk > 1 && chunk0 >= kCostSplitMin) {   // short ranges skip the alignment test
      const bool aligned = __builtin_amdgcn_ballot_w64(tiles > 0 && pex % chunk0 != 0) == 0;
      seg = split_seg_cost(chunk0, aligned, a.min_chunk);
      const uint64_t nz = __builtin_amdgcn_ballot_w64(tiles > 0);
      cpex = pex + seg * __builtin_popcountll(nz & ((1ull << lane) - 1ull));
      T = total + seg * __builtin_popcountll(nz);
    }
    if (blockIdx.x == 0 && threadIdx.x < 64) {
      int32_t* ccum = a.cum + U + 1;
      if (lane < U) {
        a.cum[lane + 1] = x;
        ccum[lane + 1] = cpex + (tiles > 0 ? tiles + seg : 0);
      }
      if (lane == 0) {
        a.cum[0] = 0;
        ccum[0] = 0;
        a.cum[2 * U + 2] = seg;
      }
    }
  } else {
    total = ld_uniform(a.cum, U);
    T = ld_uniform(a.cum, 2 * U + 1);
    seg = ld_uniform(a.cum, 2 * U + 2);
  }
  if (total <= 0) return false;
  const int chunk = split_chunk(T, W, a.min_chunk);
  const int cs = blockIdx.x * chunk;
  if (cs >= T) return false;
  const int ce = min(T, cs + chunk);
  // the unit holding cost position c: the last with ccum <= c (units without tiles have
  // empty intervals, and one of them is never the last: the unit after it starts at the
  // same position, and c < T)
  int ue = 0, ce_base = 0, ce_tile0 = 0;
  if (self_plan) {
    // the prefix sums do not decrease, so u + 1 lanes have theirs at or below c
    r.u = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < U && cpex <= cs)) - 1;
    r.ubeg = __builtin_amdgcn_readlane(pex, r.u);
    r.start = r.ubeg + max(0, cs - __builtin_amdgcn_readlane(cpex, r.u) - seg);
    if (ce < T) {
      ue = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < U && cpex <= ce)) - 1;
      ce_tile0 = __builtin_amdgcn_readlane(pex, ue);
      ce_base = __builtin_amdgcn_readlane(cpex, ue);
    }
  } else {
    const int32_t* ccum = a.cum + U + 1;
    auto last_at_or_below = [&](int c) {
      int lo_u = 0, hi_u = U - 1;
      while (lo_u < hi_u) {
        const int mid = (lo_u + hi_u + 1) >> 1;
        if (ld_uniform(ccum, mid) <= c) lo_u = mid; else hi_u = mid - 1;
      }
      return lo_u;
    };
    r.u = last_at_or_below(cs);
    r.ubeg = ld_uniform(a.cum, r.u);
    r.start = r.ubeg + max(0, cs - ld_uniform(ccum, r.u) - seg);
    if (ce < T) {
      ue = last_at_or_below(ce);
      ce_tile0 = ld_uniform(a.cum, ue);
      ce_base = ld_uniform(ccum, ue);
    }
  }
  r.end = ce < T ? ce_tile0 + max(0, ce - ce_base - seg) : total;
  return r.start < r.end;
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Per 32-token tile k (one step) and wave w:
//   wait for tile k, barrier (P of tile k-1 visible); issue the loads of tile k+2;
//   QK  S^T[32 tokens, heads 32w..32w+31] over K = 576: 36 MFMAs in two chains
//       (even / odd k-steps), A = tile rows from LDS, B = queries in registers;
//   softmax of those heads for tile k, interleaved with
//   PV of tile k-1: O[all 128 heads, latent columns 128w..128w+127] += P . c_KV,
//       2 k-steps x 4 head blocks x 4 column blocks of 32x32x16 MFMAs;
//   P of tile k (bf16) -> LDS P buffer k%2.
// P is shared through LDS so that PV can be split by latent columns; that halves
// the PV operand traffic compared with every wave reading all 512 columns.
template <bool kF8>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeArgs a) {
  // 1024-byte alignment: tile slots and P buffers then start at multiples of 1024, so
  // adding a slot base never changes the low ten bits of an offset (see below).
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kF8 ? kF8LdsBytes : kSlots * kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char pbuf[2 * kPBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  WorkRange wr;
  if (!work_range(a, lane, wr)) return;
  if constexpr (!kF8) {
#pragma unroll
    for (int i = 0; i < kLoopPadNops; ++i) asm volatile("s_nop 0");
  }
  const int g = blockIdx.x;
  const int start = wr.start, end = wr.end;

  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;       // which half of the wave
  const int l32 = lane & 31;
  const uint32_t lbase = lds_addr(lds);

  // Lane constants of the address arithmetic, kept for the whole kernel:
  //   aql, arl: QK A-operand offsets within a tile slot of token l32, chunk hi of the
  //     latent row and of the RoPE row (swizzled); chunk 2q + hi sits at the offset
  //     XOR 32q (the swizzle XOR only moves the chunk index within bits 5..7);
  //   latl[k]: direct-load source offset of latent chunk position `lane` of a row t with
  //     t % 4 == w and (t / 4) % 4 == k;  ropel: RoPE source offset of this lane's row
  //     (token 8w + lane/8) and chunk position relative to the tile.
  // Byte offset of the tile slot of tile k (the bf16 cache rings 4 slots, the MXFP8 cache 3).
  auto slot_off = [](int k) -> uint32_t { return (uint32_t)((kF8 ? k % kF8Slots : (k & 3)) * kTileBytes); };
  uint32_t aql, arl, latl[4], ropel;
  {
    aql = l32 * 1024 + 16 * (hi ^ swz_lat(l32));
    arl = kRopeRegion + l32 * 128 + 16 * (hi ^ swz_rope(l32));
#pragma unroll
    for (int k = 0; k < 4; ++k) latl[k] = (uint32_t)((lane ^ swz_lat(wave_u + 4 * k)) * 16);
    ropel = (uint32_t)((8 * wave_u + (lane >> 3)) * kRowBytes + kLatent * 2 +
                       ((lane & 7) ^ ((4 * wave_u + (lane >> 4)) & 7)) * 16);
  }
  //   f8r, f8c, f8s (MXFP8 cache): tile source offsets of this lane's RoPE chunk (token
  //     8w + lane/8, chunk position lane%8, swizzled as the bf16 RoPE rows), code chunk
  //     (token 8w + lane/32, chunk lane%32; load i adds rows 2i: 1312 i bytes) and scale
  //     dword (token 8w + (lane%32)/4, bytes 4 (lane%4) .. +3; lanes 32..63 repeat 0..31).
  uint32_t f8r = 0, f8c = 0, f8s = 0;
  if constexpr (kF8) {
    f8r = (uint32_t)((8 * wave_u + (lane >> 3)) * kF8RowBytes + kF8Rope +
                     ((lane & 7) ^ ((4 * wave_u + (lane >> 4)) & 7)) * 16);
    f8c = (uint32_t)((8 * wave_u + (lane >> 5)) * kF8RowBytes + kF8Codes + 16 * (lane & 31));
    f8s = (uint32_t)((8 * wave_u + ((lane & 31) >> 2)) * kF8RowBytes + kF8Scales + 4 * (lane & 3));
  }
  //   offP0: PV A operand (P) of head l32, tokens 8hi .. +7 in a P buffer (k-step st:
  //     XOR 32st);  offV0: PV B operand (transposing reads) of column block 0, half 0,
  //     in a tile slot: token 8hi + e (e = (lane & 15) / 4), chunk 16w + cb; column
  //     block c, half r: XOR 64c + 16r.  Each XOR only touches bits 4..7.
  uint32_t offP0, offV0;
  {
    offP0 = l32 * 64 + 16 * (hi ^ ((l32 >> 2) & 3));
    const int eb = (lane & 15) >> 2;
    const int cb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    offV0 = (8 * hi + eb) * 1024 + 64 * eb + 16 * (cb ^ (2 * hi)) + 8 * (lane & 1) + 256 * wave_u;
  }

  int u = wr.u;
  // tiles of unit u (as the plan counts them)
  auto unit_tiles_at = [&](int uu) {
    const int bb = uu / a.s_q;
    return unit_tiles(clamp_len(ld_uniform(a.seqlens, bb), a.max_blocks) - a.s_q + (uu - bb * a.s_q) + 1);
  };

  // Tile offset of the first segment in its unit; -1 once that segment is done (every
  // later segment starts its unit, so the walker keeps no unit start across segments).
  int seg0_off = start - wr.ubeg;
  int pos = start;
  bool redo = false;              // re-run the current segment with m_redo as the reference
  float m_redo = -INFINITY;
  while (pos < end) {
    const int ubeg = pos - (seg0_off >= 0 ? seg0_off : 0);
    int uend = ubeg + unit_tiles_at(u);
    while (uend <= pos) {          // units without visible tokens (never the first)
      ++u;
      uend = ubeg + unit_tiles_at(u);
    }
    const int seg_end = min(end, uend);
    // tiles t0 .. t1-1 of the unit: tile t is rows 32 (t % 2) .. +31 of logical page t / 2
    const int t0 = pos - ubeg, t1 = seg_end - ubeg;
    const bool complete = (pos == ubeg) && (seg_end == uend);
    const int slot = complete ? -1 : 2 * g + (seg0_off >= 0 ? 0 : 1);

    const int b = u / a.s_q;
    const int n_vis = clamp_len(ld_uniform(a.seqlens, b), a.max_blocks) - a.s_q + (u - b * a.s_q) + 1;
    const int64_t bt_row = (int64_t)b * a.max_blocks;
    const int tok_begin = t0 * kTile;
    const int n_tiles = t1 - t0;   // every tile has a visible token
    const int last_page = (t1 - 1) >> 1;
    // Half of its page that the segment's tile k occupies.  Tiles past the segment's end
    // (the dummy loads of the last steps) take the first half of the last page, whose
    // row 0 is a visible token, so they never fetch a row past the sequence.
    auto tile_half = [&](int k) -> int { return k < n_tiles ? ((t0 + k) & 1) : 0; };
    auto tile_src = [&](int k) -> const unsigned char* {
      const int64_t phys = min(max(ld_uniform(a.bt, bt_row + ((t0 + k) >> 1)), 0), a.last_page);
      if constexpr (kF8) return a.kv8 + phys * (int64_t)kF8PageBytes + tile_half(k) * kF8TileBytes;
      else return (const unsigned char*)a.kv + phys * (int64_t)kPageBytes + tile_half(k) * kTileBytes;
    };
    auto tile_valid = [&](int k) { return min(kTile, n_vis - tok_begin - k * kTile); };
    auto issue = [&](int k) {
      if constexpr (kF8) {
        // RoPE rows straight into the bf16 slot; codes and scales into staging k & 1.
        // Rows past the sequence are loaded as they are (they lie in the same page) and
        // never reach a product: their latent is zeroed when dequantised and their
        // scores are masked.
        const unsigned char* src = tile_src(k);
        dma_b128(src, f8r, lbase + slot_off(k) + kRopeRegion + 1024 * wave_u);
        const uint32_t cd = lbase + kF8StageOff + (k & 1) * kF8Stage + 4096 * wave_u;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_b128(src + 2 * i * kF8RowBytes, f8c, cd + 1024 * i);
        dma_b32(src, f8s, lbase + kF8ScaleOff + (k & 1) * kF8ScaleStage + 256 * wave_u);
      } else {
        const TileLoadOffsets ldo = tile_load_offsets(opaque_lane(), wave_u);
        issue_tile(tile_src(k), lbase + (k & 3) * kTileBytes, ldo, wave_u, lane, tile_valid(k));
      }
    };
    // MXFP8: dequantise this wave's rows (tokens 8w .. 8w+7) of tile kc from staging
    // into the tile's bf16 slot; rows past the sequence become zeros.  Part j (0..3)
    // is staging load j: lane l holds row t = 8w + 2j + l/32, code chunk q = l%32
    // (latent values 16q .. 16q+15, block q/2), written as bf16 chunks 2q and 2q+1 of
    // row t.  With h = l/32, swz_lat(t) = 4 (2 (j & 1) + h) + ((2w + j/2) & 3), so the
    // byte offset of chunk 2q within the tile is 1024 (8w + 2j) + (f8l ^ u_j), where
    // f8l = 1024 h + (32q ^ 64h) is a lane constant and u_j = 128 (j & 1) + 16 ((2w + j/2) & 3)
    // is uniform; chunk 2q + 1 sits at that offset XOR 16.
    u32x4 f8v[4];
    uint32_t f8sc[4];
    // Per-tile lane addresses (set by f8_lanes, kept through the tile's dequantisation):
    // this lane's code chunk in the wave's staging, its scale byte (row l/32, block
    // (l%32)/2 of the wave's scale group) and f8l.
    uint32_t f8cb = 0, f8sb = 0, f8l = 0;
    auto f8_lanes = [&](int kc) {
      const uint32_t ln = (uint32_t)opaque_lane();
      f8cb = lbase + kF8StageOff + (kc & 1) * kF8Stage + 4096 * wave_u + 16u * ln;
      f8sb = lbase + kF8ScaleOff + (kc & 1) * kF8ScaleStage + 256 * wave_u + 16u * (ln >> 5) + ((ln & 31) >> 1);
      f8l = ((ln >> 5) << 10) | ((32u * (ln & 31)) ^ ((ln >> 5) << 6));
    };
    auto f8_read = [&](int j) {
      f8v[j] = __builtin_bit_cast(u32x4, lds_read_b128_at(f8cb + 1024 * j));
      f8sc[j] = *(MLA_LDS const unsigned char*)(uintptr_t)(f8sb + 32 * j);
    };
    // Half h of part j: codes 8h .. 8h+7 of the lane's chunk -> bf16 chunk 2q + h.
    auto f8_write = [&](uint32_t slot_base, int j, int h) {
      const uint32_t u = 128u * (j & 1) + 16u * ((2 * wave_u + (j >> 1)) & 3);
      const uint32_t addr = (slot_base + 1024 * (8 * wave_u + 2 * j) + (f8l ^ u)) ^ (16u * h);
      const float sc = mx_scale_f32(f8sc[j]);
      const u32x2 d0 = e4m3x4_to_bf16(f8v[j][2 * h], sc), d1 = e4m3x4_to_bf16(f8v[j][2 * h + 1], sc);
      *(MLA_LDS u32x4*)(uintptr_t)addr = u32x4{d0[0], d0[1], d1[0], d1[1]};
    };
    // Rows at or past `valid` (only in a segment's last tile) are overwritten with zeros.
    auto f8_zero_tail = [&](uint32_t slot_base, int valid) {
      const uint32_t ln = (uint32_t)opaque_lane();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 8 * wave_u + 2 * j + (int)(ln >> 5);
        const uint32_t u = 128u * (j & 1) + 16u * ((2 * wave_u + (j >> 1)) & 3);
        const uint32_t lo_addr = slot_base + 1024 * (8 * wave_u + 2 * j) + (f8l ^ u);
        if (t >= valid) {
          *(MLA_LDS u32x4*)(uintptr_t)lo_addr = u32x4{0u, 0u, 0u, 0u};
          *(MLA_LDS u32x4*)(uintptr_t)(lo_addr ^ 16u) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto f8_convert_all = [&](int kc) {
      f8_lanes(kc);
#pragma unroll
      for (int j = 0; j < 4; ++j) f8_read(j);
      const uint32_t sb = lbase + slot_off(kc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f8_write(sb, j, 0);
        f8_write(sb, j, 1);
      }
      if (tile_valid(kc) < kTile) f8_zero_tail(sb, tile_valid(kc));
    };

    // P buffer 1 stands for "P of tile -1" in the first step: zero it.  Its last
    // reader (the previous segment) is behind the end-of-segment barriers.
    *(u32x4*)(pbuf + kPBytes + 32 * tid) = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(pbuf + kPBytes + 32 * tid + 16) = u32x4{0u, 0u, 0u, 0u};

    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // earlier stores of this workgroup
    issue(0);
    if (n_tiles > 1) issue(1);
    if constexpr (kF8) {
      // tile 0 must be in bf16 before the first step; tile 1 may stay in flight
      if (n_tiles > 1) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      f8_convert_all(0);
      asm volatile("" ::: "memory");
    }

    // Queries of this wave's 32 heads as the MFMA B operand: lane l holds head
    // 32w + l32, columns 16ks + 8hi .. +7 (k-steps 0..31 latent, 32..35 RoPE).
    const int head = wave_u * 32 + l32;
    s16x8 q[36];
    if constexpr (kF8) {
      // lane offsets taken here (an opaque lane id): hoisted out of the segment loop they
      // would be spilled, and a reload between the loads waits for every load before it
      const int ln = opaque_lane();
      const int hq = wave_u * 32 + (ln & 31);
      const uint16_t* qa = a.q_abs + ((size_t)u * kHeads + hq) * kLatent + 8 * (ln >> 5);
      const uint16_t* qr = a.q_r + ((size_t)u * kHeads + hq) * kRope + 8 * (ln >> 5);
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) q[ks] = *(const s16x8*)(qa + 16 * ks);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) q[32 + ks] = *(const s16x8*)(qr + 16 * ks);
    } else {
      // Loaded straight into that layout, each load instruction touches 32 rows (one per
      // head) and the 36 of them take ~9k cycles to issue; staged through LDS, each direct
      // load copies 1 KiB of two heads' rows (8 cache lines) and the reads into the layout
      // are conflict-free.  Stage of a round, per head h (0..31 within the wave): latent
      // chunk c (16 B, 0..31 of the round) at 512h + 16 (c ^ (h & 15)); RoPE chunk c (0..3
      // of the round) at kQStageRope + 64h + 16 (c ^ f(h)), f(h) = ((h >> 1) ^ (h >> 3)) & 3.
      const uint32_t ln = (uint32_t)opaque_lane();
      const uint32_t ql = ln & 31, qh = ln >> 5;
      const uint32_t qst = lbase + 2 * kTileBytes + wave_u * kQStageBytes;
      const unsigned char* qa_w = (const unsigned char*)(a.q_abs + ((size_t)u * kHeads + wave_u * 32) * kLatent);
      const unsigned char* qr_w = (const unsigned char*)(a.q_r + ((size_t)u * kHeads + wave_u * 32) * kRope);
      // load i of the latent part: lanes 0..31 fill head 2i's 32 slots, lanes 32..63 head
      // 2i + 1's; slot s holds chunk s ^ (h & 15) = (l32 ^ hi) ^ 2 (i & 7)
      const uint32_t lat_v = 1024 * qh + 16 * (ql ^ qh);
      // load i of the RoPE part: lane l fills slot l & 3 of head 16i + l/4
      const uint32_t rh = ln >> 2;
      const uint32_t rope_v = 128 * rh + 16 * ((ln & 3) ^ (((rh >> 1) ^ (rh >> 3)) & 3));
      // reads: head l32, chunk 2k' + hi of the round at slot (2k' + hi) ^ (l32 & 15)
      const uint32_t lat_r = qst + 512 * ql + 16 * (qh ^ (ql & 15));
      const uint32_t fr = ((ql >> 1) ^ (ql >> 3)) & 3;
      const uint32_t rope_r = qst + kQStageRope + 64 * ql;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (r == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // round 0 read out
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dma_q_b128(qa_w + 2048 * i, (lat_v + 512 * r) ^ (32u * (i & 7)), qst + 1024 * i);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          dma_q_b128(qr_w + 2048 * i, (rope_v + 64 * r) ^ (32u * i), qst + kQStageRope + 1024 * i);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stage (and its tiles) in LDS
#pragma unroll
        for (int kp = 0; kp < 16; ++kp) q[16 * r + kp] = lds_read_b128_at(lat_r ^ (32u * kp));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) q[32 + 2 * r + kk] = lds_read_b128_at(rope_r + 16 * ((2 * kk + qh) ^ fr));
      }
      // read out before the first step, whose loads of tile 2 (any wave's) refill slot 2
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // O^T[column block c][head block hb], kept as o[hb][c]: the PV products take V^T as the A
    // operand and P^T as B (the same registers either way), so that register j of tile (hb, c)
    // is latent column 128w + 32c + 8(j/4) + 4hi + (j%4) of head 32hb + l32: each lane holds
    // runs of four consecutive columns of one head.
    f32x16 o[4][4];
    // Reference max (log2 units) of head 32w + l32: from the first tile, or the
    // segment's true maximum when the segment is being redone.
    float m_ref = redo ? m_redo : -INFINITY;
    float l_part = 0.f;        // this lane's share of that head's softmax denominator
    float m_seen = -INFINITY;  // largest score seen (log2 units); above m_ref + kHeadroom means overflow
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[hb][c][j] = 0.f;

    // Operands of the next step, prepared while the current one runs its PV stages:
    // QK A-operand addresses for tile slot kk & 3 (token l32, chunk 2ks + hi; latent
    // k-step 8p + q at aq[q] + 256p, RoPE k-step 32 + q at ar[q]) and the direct
    // loads of tile kn (source tile base, per-lane offsets, first LDS address).
    uint32_t aq[8], ar[4], dv[9];
    const unsigned char* dsrc;
    uint32_t m0n, m0c = 0, m0s = 0;   // LDS targets of the next tile's loads (m0c, m0s: MXFP8 codes, scales)
    int32_t bt_pref;
    // Each preparation comes in three parts so that it can be spread over stages.
    auto prep_qk = [&](int kk, int part) {
      const uint32_t cur_addr = lbase + slot_off(kk);
      // the MXFP8 variant has fewer registers to spare: it recomputes the lane offsets
      uint32_t ql = aql, rl = arl;
      if constexpr (kF8) {
        const int ln = opaque_lane(), t = ln & 31, h = ln >> 5;
        ql = t * 1024 + 16 * (h ^ swz_lat(t));
        rl = kRopeRegion + t * 128 + 16 * (h ^ swz_rope(t));
      }
      // cur_addr is a multiple of 1024: the XOR after the add only touches bits 5..7
      if (part < 2) {
        const uint32_t a0 = cur_addr + (kF8 ? ql : step_local(ql));
#pragma unroll
        for (int q2 = 4 * part; q2 < 4 * part + 4; ++q2) aq[q2] = a0 ^ (32u * q2);
      } else {
        const uint32_t r0 = cur_addr + (kF8 ? rl : step_local(rl));
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) ar[q2] = r0 ^ (32u * q2);
      }
    };
    auto prep_dma = [&](int kn, int32_t raw, int part) {
      if constexpr (kF8) {
        // per-lane source offsets are kernel constants: only bases change
        if (part != 0) return;
        const int32_t r = __builtin_amdgcn_readfirstlane(raw);
        const int64_t phys = min(max(r, 0), a.last_page);
        dsrc = a.kv8 + phys * (int64_t)kF8PageBytes + tile_half(kn) * kF8TileBytes;
        m0n = lbase + slot_off(kn) + kRopeRegion + 1024 * wave_u;
        m0c = lbase + kF8StageOff + (kn & 1) * kF8Stage + 4096 * wave_u;
        m0s = lbase + kF8ScaleOff + (kn & 1) * kF8ScaleStage + 256 * wave_u;
        return;
      }
      // past the end of the segment (valid <= 0) every row maps to row 0 of the page
      const int valid = tile_valid(kn);
      if (part == 0) {
        const int32_t r = __builtin_amdgcn_readfirstlane(raw);   // uniform: keeps the base in SGPRs
        const int64_t phys = min(max(r, 0), a.last_page);
        dsrc = (const unsigned char*)a.kv + phys * (int64_t)kPageBytes + tile_half(kn) * kTileBytes;
        m0n = lbase + (kn & 3) * kTileBytes + kRopeRegion + 1024 * wave_u;
        // rows at or past `valid` fetch the RoPE chunk of row 0 instead
        const uint32_t r_0 = (uint32_t)(kLatent * 2 + (lane & 7) * 16);
        const uint32_t keep = 0u - (uint32_t)(8 * wave_u + (lane >> 3) < valid);
        dv[0] = (ropel & keep) | (r_0 & ~keep);
      } else {
#pragma unroll
        for (int i = 4 * part - 4; i < 4 * part; ++i) {
          const int t = wave_u + 4 * i;
          dv[1 + i] = latl[i & 3] + (t < valid ? t * kRowBytes : 0);
        }
      }
    };
    {
      const int32_t raw2 = ld_uniform(a.bt, bt_row + min((t0 + 2) >> 1, last_page));
#pragma unroll
      for (int part = 0; part < 3; ++part) {
        prep_qk(0, part);
        prep_dma(2, raw2, part);
      }
    }

    // kFirst: the segment's first tile (sets the softmax reference); kLast: its last
    // tile (masks the keys past the end, issues no further loads).
    auto step = [&](const int k, auto first, auto last) __attribute__((always_inline)) {
      constexpr bool kFirst = decltype(first)::value;
      constexpr bool kMasked = decltype(last)::value;
      if constexpr (kF8) {
        // tile k was dequantised in the previous step (or before the first); the last
        // step drains the dummy loads issued past the end
        if (kMasked) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      } else {
        if (kMasked || kFirst) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerTile));   // tile k+1 may still be in flight
      }
      __syncthreads();   // tile k in LDS for all; P(k-1) visible; slot of tile k+2 and P buffer k%2 free

      // ---- scores S^T: 36 k-steps accumulated in one chain (dependent MFMAs on the same
      // registers issue back to back), the A operand read from LDS four k-steps ahead
      // through a ring of four registers, one LDS wait per pair of k-steps.
      // A operand, k-step ks: token l32 of the tile, chunk 2ks + hi:
      //   latent (ks = 8p + q < 32): aq[q] + 256p;  RoPE (ks = 32 + q): ar[q]
      // Written as one asm block so that the accumulator lives in VGPRs: the O
      // accumulators fill all 256 AGPRs, and compiler-selected MFMAs here would use
      // the AGPR form and shuttle O tiles between the register files every tile.
      // Hazards the block covers itself: the leading s_nop 1 separates a VALU write of
      // an operand from its MFMA read; the chain starts from the constant 0 and then
      // accumulates in place (same registers, back to back, no wait needed); a ring
      // register is refilled only after the MFMA reading it has issued (its A read is
      // at issue, the LDS return much later); the trailing 14 wait states exceed the 12
      // an 8-pass XDL result needs before a VALU or memory read.
      // The M0 steps of those loads are scalar adds, which write SCC: the blocks that
      // issue loads name SCC as clobbered, so no compare result is kept in it across them.
      // Except in a segment's last step the block also issues the 9 direct loads of
      // tile k+2, one after every fourth MFMA (RoPE rows first, M0 stepping through
      // the LDS rows), so their issue overlaps the MFMAs, and the scalar load of the
      // block-table entry of tile k+3's page (the block's final lgkmcnt(0) covers it;
      // an outstanding scalar load only makes its LDS waits stricter).  Past the end
      // of the segment those loads fetch row 0 of the segment's last page into the
      // free slot: a dummy that keeps every non-last step on one code path.  All
      // operand addresses were prepared during the previous step's PV stages.
      f32x16 sa;
      {
        s16x8 tq[4];
        if constexpr (!kMasked) {
          // the block-table entry of the page of tile k+3, for the next step's loads
          const int32_t* btp = a.bt + bt_row;
          const int bto = 4 * min((t0 + k + 3) >> 1, last_page);
          int32_t bt_next;
          uint32_t m0v = m0n;
          if constexpr (kF8) {
            uint32_t vtmp;   // source offset of code loads 1..3 (rows 2i further: 1312 i bytes)
            asm volatile(
                  "s_nop 1\n\t"
                  "s_load_dword %[btn], %[btp], %[bto]\n\t"
                  "ds_read_b128 %[t0], %[a0] offset:0\n\t"
                  "ds_read_b128 %[t1], %[a1] offset:0\n\t"
                  "ds_read_b128 %[t2], %[a2] offset:0\n\t"
                  "ds_read_b128 %[t3], %[a3] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q0], 0\n\tds_read_b128 %[t0], %[a4] offset:0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[vr], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q1], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q2], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:0\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q3], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q4], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:256\n\ts_mov_b32 m0, %[mc]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[vc], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q5], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q6], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:256\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q7], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q8], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:256\n\tv_add_u32 %[vt], 0x520, %[vc]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[vt], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q9], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q10], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:256\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q11], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q12], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:512\n\tv_add_u32 %[vt], 0xa40, %[vc]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[vt], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q13], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q14], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:512\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q15], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q16], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:512\n\tv_add_u32 %[vt], 0xf60, %[vc]\n\ts_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[vt], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q17], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q18], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:512\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q19], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q20], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:768\n\ts_mov_b32 m0, %[ms]\n\ts_nop 0\n\tglobal_load_lds_dword %[vs], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q21], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q22], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:768\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q23], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q24], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:768\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q25], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q26], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:768\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q27], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q28], %[sa]\n\tds_read_b128 %[t0], %[r0] offset:0\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q29], %[sa]\n\tds_read_b128 %[t1], %[r1] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q30], %[sa]\n\tds_read_b128 %[t2], %[r2] offset:0\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q31], %[sa]\n\tds_read_b128 %[t3], %[r3] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q32], %[sa]\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q33], %[sa]\n\t"
                  "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q34], %[sa]\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q35], %[sa]\n\t"
                  "s_nop 7\n\ts_nop 5"
                  : [sa] "=&v"(sa), [t0] "=&v"(tq[0]), [t1] "=&v"(tq[1]), [t2] "=&v"(tq[2]), [t3] "=&v"(tq[3]), [btn] "=&s"(bt_next), "+{m0}"(m0v), [vt] "=&v"(vtmp)
                  : [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]), [q5] "v"(q[5]),
                    [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]), [q10] "v"(q[10]), [q11] "v"(q[11]),
                    [q12] "v"(q[12]), [q13] "v"(q[13]), [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]),
                    [q18] "v"(q[18]), [q19] "v"(q[19]), [q20] "v"(q[20]), [q21] "v"(q[21]), [q22] "v"(q[22]), [q23] "v"(q[23]),
                    [q24] "v"(q[24]), [q25] "v"(q[25]), [q26] "v"(q[26]), [q27] "v"(q[27]), [q28] "v"(q[28]), [q29] "v"(q[29]),
                    [q30] "v"(q[30]), [q31] "v"(q[31]), [q32] "v"(q[32]), [q33] "v"(q[33]), [q34] "v"(q[34]), [q35] "v"(q[35]),
                    [a0] "v"(aq[0]), [a1] "v"(aq[1]), [a2] "v"(aq[2]), [a3] "v"(aq[3]), [a4] "v"(aq[4]), [a5] "v"(aq[5]), [a6] "v"(aq[6]), [a7] "v"(aq[7]),
                    [r0] "v"(ar[0]), [r1] "v"(ar[1]), [r2] "v"(ar[2]), [r3] "v"(ar[3]),
                    [src] "s"(dsrc), [btp] "s"(btp), [bto] "s"(bto), [vr] "v"(f8r), [vc] "v"(f8c), [vs] "v"(f8s), [mc] "s"(m0c), [ms] "s"(m0s)
                  : "memory", "scc");
          } else {
            asm volatile(
                  "s_nop 1\n\t"
                  "s_load_dword %[btn], %[btp], %[bto]\n\t"
                  "ds_read_b128 %[t0], %[a0] offset:0\n\t"
                  "ds_read_b128 %[t1], %[a1] offset:0\n\t"
                  "ds_read_b128 %[t2], %[a2] offset:0\n\t"
                  "ds_read_b128 %[t3], %[a3] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q0], 0\n\tds_read_b128 %[t0], %[a4] offset:0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d0], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q1], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q2], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:0\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q3], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q4], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:256\n\ts_add_u32 m0, m0, 0xffff8000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d1], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q5], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q6], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:256\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q7], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q8], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:256\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d2], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q9], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q10], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:256\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q11], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:256\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q12], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:512\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d3], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q13], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q14], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:512\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q15], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q16], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:512\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d4], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q17], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q18], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:512\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q19], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:512\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q20], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:768\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d5], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q21], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q22], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:768\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q23], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q24], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:768\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d6], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q25], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q26], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:768\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q27], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:768\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q28], %[sa]\n\tds_read_b128 %[t0], %[r0] offset:0\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d7], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q29], %[sa]\n\tds_read_b128 %[t1], %[r1] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q30], %[sa]\n\tds_read_b128 %[t2], %[r2] offset:0\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q31], %[sa]\n\tds_read_b128 %[t3], %[r3] offset:0\n\t"
                  "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q32], %[sa]\n\ts_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[d8], %[src] nt\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q33], %[sa]\n\t"
                  "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q34], %[sa]\n\t"
                  "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q35], %[sa]\n\t"
                  "s_nop 7\n\ts_nop 5"
                  : [sa] "=&v"(sa), [t0] "=&v"(tq[0]), [t1] "=&v"(tq[1]), [t2] "=&v"(tq[2]), [t3] "=&v"(tq[3]), [btn] "=&s"(bt_next), "+{m0}"(m0v)
                  : [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]), [q5] "v"(q[5]),
                    [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]), [q10] "v"(q[10]), [q11] "v"(q[11]),
                    [q12] "v"(q[12]), [q13] "v"(q[13]), [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]),
                    [q18] "v"(q[18]), [q19] "v"(q[19]), [q20] "v"(q[20]), [q21] "v"(q[21]), [q22] "v"(q[22]), [q23] "v"(q[23]),
                    [q24] "v"(q[24]), [q25] "v"(q[25]), [q26] "v"(q[26]), [q27] "v"(q[27]), [q28] "v"(q[28]), [q29] "v"(q[29]),
                    [q30] "v"(q[30]), [q31] "v"(q[31]), [q32] "v"(q[32]), [q33] "v"(q[33]), [q34] "v"(q[34]), [q35] "v"(q[35]),
                    [a0] "v"(aq[0]), [a1] "v"(aq[1]), [a2] "v"(aq[2]), [a3] "v"(aq[3]), [a4] "v"(aq[4]), [a5] "v"(aq[5]), [a6] "v"(aq[6]), [a7] "v"(aq[7]),
                    [r0] "v"(ar[0]), [r1] "v"(ar[1]), [r2] "v"(ar[2]), [r3] "v"(ar[3]),
                    [src] "s"(dsrc), [btp] "s"(btp), [bto] "s"(bto), [d0] "v"(dv[0]), [d1] "v"(dv[1]), [d2] "v"(dv[2]), [d3] "v"(dv[3]), [d4] "v"(dv[4]), [d5] "v"(dv[5]), [d6] "v"(dv[6]), [d7] "v"(dv[7]), [d8] "v"(dv[8])
                  : "memory", "scc");
          }
          bt_pref = bt_next;
        } else {
          asm volatile(
              "s_nop 1\n\t"
              "ds_read_b128 %[t0], %[a0] offset:0\n\t"
              "ds_read_b128 %[t1], %[a1] offset:0\n\t"
              "ds_read_b128 %[t2], %[a2] offset:0\n\t"
              "ds_read_b128 %[t3], %[a3] offset:0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q0], 0\n\tds_read_b128 %[t0], %[a4] offset:0\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q1], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q2], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:0\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q3], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q4], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:256\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q5], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:256\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q6], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:256\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q7], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:256\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q8], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:256\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q9], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:256\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q10], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:256\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q11], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:256\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q12], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:512\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q13], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:512\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q14], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:512\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q15], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:512\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q16], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:512\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q17], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:512\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q18], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:512\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q19], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:512\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q20], %[sa]\n\tds_read_b128 %[t0], %[a0] offset:768\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q21], %[sa]\n\tds_read_b128 %[t1], %[a1] offset:768\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q22], %[sa]\n\tds_read_b128 %[t2], %[a2] offset:768\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q23], %[sa]\n\tds_read_b128 %[t3], %[a3] offset:768\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q24], %[sa]\n\tds_read_b128 %[t0], %[a4] offset:768\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q25], %[sa]\n\tds_read_b128 %[t1], %[a5] offset:768\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q26], %[sa]\n\tds_read_b128 %[t2], %[a6] offset:768\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q27], %[sa]\n\tds_read_b128 %[t3], %[a7] offset:768\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q28], %[sa]\n\tds_read_b128 %[t0], %[r0] offset:0\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q29], %[sa]\n\tds_read_b128 %[t1], %[r1] offset:0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q30], %[sa]\n\tds_read_b128 %[t2], %[r2] offset:0\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q31], %[sa]\n\tds_read_b128 %[t3], %[r3] offset:0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t0], %[q32], %[sa]\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t1], %[q33], %[sa]\n\t"
              "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 %[sa], %[t2], %[q34], %[sa]\n\t"
              "v_mfma_f32_32x32x16_bf16 %[sa], %[t3], %[q35], %[sa]\n\t"
              "s_nop 7\n\ts_nop 5"
              : [sa] "=&v"(sa), [t0] "=&v"(tq[0]), [t1] "=&v"(tq[1]), [t2] "=&v"(tq[2]), [t3] "=&v"(tq[3])
              : [q0] "v"(q[0]), [q1] "v"(q[1]), [q2] "v"(q[2]), [q3] "v"(q[3]), [q4] "v"(q[4]), [q5] "v"(q[5]),
                [q6] "v"(q[6]), [q7] "v"(q[7]), [q8] "v"(q[8]), [q9] "v"(q[9]), [q10] "v"(q[10]), [q11] "v"(q[11]),
                [q12] "v"(q[12]), [q13] "v"(q[13]), [q14] "v"(q[14]), [q15] "v"(q[15]), [q16] "v"(q[16]), [q17] "v"(q[17]),
                [q18] "v"(q[18]), [q19] "v"(q[19]), [q20] "v"(q[20]), [q21] "v"(q[21]), [q22] "v"(q[22]), [q23] "v"(q[23]),
                [q24] "v"(q[24]), [q25] "v"(q[25]), [q26] "v"(q[26]), [q27] "v"(q[27]), [q28] "v"(q[28]), [q29] "v"(q[29]),
                [q30] "v"(q[30]), [q31] "v"(q[31]), [q32] "v"(q[32]), [q33] "v"(q[33]), [q34] "v"(q[34]), [q35] "v"(q[35]),
                [a0] "v"(aq[0]), [a1] "v"(aq[1]), [a2] "v"(aq[2]), [a3] "v"(aq[3]), [a4] "v"(aq[4]), [a5] "v"(aq[5]), [a6] "v"(aq[6]), [a7] "v"(aq[7]),
                [r0] "v"(ar[0]), [r1] "v"(ar[1]), [r2] "v"(ar[2]), [r3] "v"(ar[3])
              : "memory");
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- PV of tile k-1 (at k = 0: the zeroed P buffer 1 with the current, finite
      // tile as V, which adds exact zeros), interleaved with the softmax of tile k.
      // O^T += V^T P^T, operands as loaded (lane l32 + 32hi):
      //   P^T (B operand), head block hb, k-step st: head 32hb + l32, tokens 16st + 8hi + 0..7
      //     -> (pprev + offP0) XOR 32st, + 2048 hb
      //   V^T (A operand, transposing reads), half r, column block c: token 16st + 8hi + 4r + e,
      //     chunk 16w + 4c + cb, byte 8 (lane & 1) -> (vprev + offV0) XOR (64c + 16r), + 16384 st + 4096 r
      const unsigned char* vprev = lds + slot_off(k == 0 ? 0 : k - 1);
      const unsigned char* pprev = pbuf + ((k - 1) & 1) * kPBytes;
      const uint32_t vb = lds_addr(vprev) + (kF8 ? offV0 : step_local(offV0)), pb = lds_addr(pprev) + (kF8 ? offP0 : step_local(offP0));
      auto ld_v = [&](int st, int c) -> s16x8 {
        const s16x4 v0 = lds_read_tr4_at((vb ^ (64u * c)) + 16384 * st);
        const s16x4 v1 = lds_read_tr4_at((vb ^ (64u * c + 16u)) + 16384 * st + 4096);
        return s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      };
      auto ld_p = [&](int st, int hb) -> s16x8 { return lds_read_b128_at((pb ^ (32u * st)) + 2048 * hb); };
      s16x8 pa[4], bv[4], bvn;
      pa[0] = ld_p(0, 0);
      bv[0] = ld_v(0, 0);
#pragma unroll
      for (int c = 1; c < 4; ++c) bv[c] = ld_v(0, c);
#pragma unroll
      for (int hb = 1; hb < 4; ++hb) pa[hb] = ld_p(0, hb);

      // Scores of tile k, still unscaled (scale > 0 keeps the max).  Register j is
      // token 8(j/4) + 4hi + (j%4) of the tile.  Keys past the end of the sequence
      // (only in the segment's last tile) score -inf.
      float sc[16], xa[16], ex[16];
      float mx = -INFINITY;
      // Token 8(j/4) + 4hi + (j%4) is past the end when 4hi >= valid - 8(j/4) - (j%4): the
      // lane's 4hi (taken here, so it is not hoisted) against a uniform bound per register.
      // Comparing per-register token indices instead made the compiler keep sixteen lane
      // constants across the segment loop, spill them, and reload them one by one here.
      const int h4 = kMasked ? 4 * (opaque_lane() >> 5) : 0;
      auto score = [&](int j) {
        sc[j] = sa[j];
        if constexpr (kMasked) {
          if (h4 >= tile_valid(k) - (8 * (j >> 2) + (j & 3))) sc[j] = -INFINITY;
        }
        if (j & 1) mx = max3f(mx, sc[j - 1], sc[j]);
      };
      if constexpr (kFirst) {
        // The reference maximum is needed before the first weight: all scores first.
#pragma unroll
        for (int j = 0; j < 16; ++j) score(j);
        mx *= a.scale_log2;
        m_seen = fmaxf(m_seen, mx);
        const float mx_head = fmaxf(mx, __shfl_xor(mx, 32, 64));
        m_ref = redo ? m_ref : mx_head;   // a redo brings the segment's true maximum
      }
      __builtin_amdgcn_sched_barrier(0);

      // 32 stages, one PV MFMA each, fenced so that the order below is the issue order.
      // k-step 0 runs head-block-major: P register hb is reloaded with its k-step-1 value
      // right after its last use; V registers are refilled for k-step 1 after their last
      // use, the first k-step-1 column block going to the spare register bvn early.  k-step 1
      // runs column-block-major.  The softmax of tile k is software-pipelined over the
      // stages (score j at stage j, exponent argument at j+1, exponential at j+2, sum and
      // packing at j+3; in the first tile the scores are all done above), so each stage's
      // VALU work is independent and hides under its MFMA.
      constexpr int oB = kFirst ? 0 : 1;
      u32x2 pw[4];
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        if (st < 16) {
          const int hb = st >> 2, c = st & 3;
          o[hb][c] = mfma32(bv[c], pa[hb], o[hb][c]);
          if (c == 3) pa[hb] = ld_p(1, hb);
          if (st == 1) bvn = ld_v(1, 0);
          if (st >= 12 && st < 15) bv[st - 12] = ld_v(1, st - 11);
        } else {
          const int c = (st - 16) >> 2, hb = (st - 16) & 3;
          o[hb][c] = mfma32(c == 0 ? bvn : bv[c - 1], pa[hb], o[hb][c]);
        }
        if (!kFirst && st < 16) score(st);
        if (st >= oB && st < 16 + oB) xa[st - oB] = __builtin_fmaf(sc[st - oB], a.scale_log2, -m_ref);
        if (st >= oB + 1 && st < 17 + oB) ex[st - oB - 1] = __builtin_amdgcn_exp2f(xa[st - oB - 1]);
        if (st >= oB + 2 && st < 18 + oB) {
          const int j = st - oB - 2;
          l_part += ex[j];
          if (j & 1) pw[j >> 2][(j >> 1) & 1] = pack_bf16x2(ex[j - 1], ex[j]);
        }
        if (st == 20) {
          // P of tile k: tokens 8q + 4hi + 0..3 of head 32w + l32, chunk q at q ^ ((head >> 2) & 3).
          const int ln = opaque_lane(), ll = ln & 31;
          unsigned char* pk = pbuf + (k & 1) * kPBytes + (wave_u * 32 + ll) * 64 + 8 * (ln >> 5);
          const int sw = (ll >> 2) & 3;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) *(u32x2*)(pk + 16 * (qq ^ sw)) = pw[qq];
        }
        if (!kFirst && st == 21) m_seen = fmaxf(m_seen, mx * a.scale_log2);
        if constexpr (!kMasked) {
          if (st >= 22 && st < 25) prep_qk(k + 1, st - 22);
          if constexpr (kF8) {
            // Dequantisation of tile k+1 (its loads went out early in step k-1; tile k+2's
            // six are newer): lane addresses at stage 23, part j read at stage 24 + j and
            // its two halves converted and stored at stage 27 + j.
            if (st == 23) f8_lanes(k + 1);
            if (st == 24) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
            if (st >= 24 && st < 28) f8_read(st - 24);
            if (st == 25) prep_dma(k + 3, bt_pref, 0);
            if (st >= 27 && st < 31) {
              f8_write(lbase + slot_off(k + 1), st - 27, 0);
              f8_write(lbase + slot_off(k + 1), st - 27, 1);
            }
          } else {
            if (st >= 25 && st < 28) prep_dma(k + 3, bt_pref, st - 25);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kF8 && !kMasked) {
        if (tile_valid(k + 1) < kTile) f8_zero_tail(lbase + slot_off(k + 1), tile_valid(k + 1));
      }
    };

    int k = 0;
    if (n_tiles == 1) {
      step(0, Flag<true>{}, Flag<true>{});
    } else {
      step(0, Flag<true>{}, Flag<false>{});
      for (k = 1; k + 1 < n_tiles; ++k) step(k, Flag<false>{}, Flag<false>{});
      step(k, Flag<false>{}, Flag<true>{});
    }

    // PV of the last tile.
    __syncthreads();   // P of the last tile visible
    {
      const unsigned char* vlast = lds + slot_off(k);
      const unsigned char* plast = pbuf + (k & 1) * kPBytes;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s16x8 pa[4], bv[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) pa[hb] = lds_read_b128_at(((lds_addr(plast) + offP0) ^ (32u * st)) + 2048 * hb);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t vl = lds_addr(vlast) + offV0;
          const s16x4 v0 = lds_read_tr4_at((vl ^ (64u * c)) + 16384 * st);
          const s16x4 v1 = lds_read_tr4_at((vl ^ (64u * c + 16u)) + 16384 * st + 4096);
          bv[c] = s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int c = 0; c < 4; ++c) o[hb][c] = mfma32(bv[c], pa[hb], o[hb][c]);
      }
    }

    {
      // ---- end of segment: agree on a redo, publish row sums.  The ring slots are
      // free once every wave is past this barrier; slot 0 holds the scratch.
      __syncthreads();
      int* flags = (int*)lds;
      float* lsum = (float*)(lds + 256);   // 1 / (softmax denominator) of each head
      const bool any_over = __builtin_amdgcn_ballot_w64(m_seen > m_ref + kHeadroom) != 0;
      const float l_head = l_part + __shfl_xor(l_part, 32, 64);
      const float m_all = fmaxf(m_seen, __shfl_xor(m_seen, 32, 64));
      if (lane == 0) flags[wave_u] = any_over ? 1 : 0;
      if (hi == 0) lsum[head] = 1.f / l_head;   // one division per head, shared by the four waves
      __syncthreads();
      const bool again = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
      m_redo = m_all;         // the segment's true maximum: no score exceeds it on a redo
      // normalise and write.  Register j of tile (hb, c) is column 128w + 32c + 8(j/4) +
      // 4hi + (j%4) of head 32hb + l32, so each group of four registers becomes one 8-byte
      // bf16 write into a per-wave LDS stage of the wave's 128 columns of all 128 heads
      // (the ring is free now; row pitch 272 B puts the 32 heads of one write on distinct
      // bank pairs), read back as whole 16-byte row chunks: one store instruction then
      // writes four 256-byte row segments.
      if (!again) {
        const float lse2 = m_ref + __log2f(l_head);
        constexpr int kStagePitch = 272;
        static_assert(1024 + 4 * kHeads * kStagePitch <= (kF8 ? kF8LdsBytes : kSlots * kTileBytes),
                      "the stage fits in the ring below the P buffers");
        const int eln = opaque_lane(), el32 = eln & 31, ehi = eln >> 5;   // not kept live
        unsigned char* stage = lds + 1024 + wave_u * (kHeads * kStagePitch);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const float il = lsum[32 * hb + el32];
          unsigned char* srow = stage + (32 * hb + el32) * kStagePitch + 8 * ehi;
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *(u32x2*)(srow + 2 * (32 * c + 8 * q4)) =
                  u32x2{pack_bf16x2(o[hb][c][4 * q4] * il, o[hb][c][4 * q4 + 1] * il),
                        pack_bf16x2(o[hb][c][4 * q4 + 2] * il, o[hb][c][4 * q4 + 3] * il)};
        }
        // the wave reads back only what it wrote: LDS order within the wave suffices.
        // complete units go straight to out_latent, pieces of split units to their
        // partial slot; both as bf16
        const size_t obase = (size_t)(eln >> 4) * kLatent + wave_u * 128 + 8 * (eln & 15);
        uint16_t* ob = (slot < 0 ? a.out_latent + (size_t)u * kHeads * kLatent
                                 : a.part_o + (size_t)slot * kHeads * kLatent) + obase;
        const unsigned char* rrow = stage + (eln >> 4) * kStagePitch + 16 * (eln & 15);
#pragma unroll
        for (int i = 0; i < 32; ++i)
          *(u32x4*)(ob + (size_t)(4 * i) * kLatent) = *(const u32x4*)(rrow + 4 * i * kStagePitch);
        if (hi == 0) {
          if (slot < 0) {
            if (a.lse != nullptr) a.lse[(size_t)u * kHeads + head] = lse2 * kLn2;
          } else {
            a.part_lse[(size_t)slot * kHeads + head] = lse2;
          }
        }
      }
      __syncthreads();   // scratch read before the next segment refills the slots
      redo = again;      // a redo runs the same segment again (pos unchanged)
    }
    if (!redo) {
      pos = seg_end;
      ++u;                         // pos is now the next unit's start (or the range's end)
      seg0_off = -1;
    }
  }
}

// ---------------------------------------------------------------------------- stream (measurement)

// The memory side of decode_kernel<false> alone: the same work split, the same direct
// 16-byte non-temporal loads of the same 32-token tiles into the same 4-slot LDS ring,
// two tiles ahead, one workgroup barrier per tile -- and no arithmetic on the tiles.  Its
// time is the ceiling the decode's page stream can reach on the device.  So that every
// load is observable, thread t of each workgroup adds dword t of each tile's first row
// (the latent of the tile's first token, 256 dwords) into a 32-bit sum, stored at
// sums[block * 256 + t]: the sum over all threads and workgroups is the sum, over every
// tile of every unit, of its first row's latent dwords (mod 2^32).
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void stream_kernel(DecodeArgs a, uint32_t* __restrict__ sums) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kSlots * kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t acc = 0;
  WorkRange wr;
  if (work_range(a, lane, wr)) {
    const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lbase = lds_addr(lds);
    const TileLoadOffsets ldo = tile_load_offsets(lane, wave_u);
    int u = wr.u, pos = wr.start, seg0_off = wr.start - wr.ubeg;
    while (pos < wr.end) {
      const int ubeg = pos - (seg0_off >= 0 ? seg0_off : 0);
      int uend = ubeg;
      while (uend <= pos) {          // skips units without visible tokens
        const int bb = u / a.s_q;
        uend = ubeg + unit_tiles(clamp_len(ld_uniform(a.seqlens, bb), a.max_blocks) - a.s_q + (u - bb * a.s_q) + 1);
        if (uend <= pos) ++u;
      }
      const int seg_end = min(wr.end, uend);
      const int t0 = pos - ubeg, n_tiles = seg_end - pos;
      const int b = u / a.s_q;
      const int n_vis = clamp_len(ld_uniform(a.seqlens, b), a.max_blocks) - a.s_q + (u - b * a.s_q) + 1;
      const int64_t bt_row = (int64_t)b * a.max_blocks;
      auto issue = [&](int k) {
        const int64_t phys = min(max(ld_uniform(a.bt, bt_row + ((t0 + k) >> 1)), 0), a.last_page);
        const unsigned char* src = (const unsigned char*)a.kv + phys * (int64_t)kPageBytes + ((t0 + k) & 1) * kTileBytes;
        issue_tile(src, lbase + (k & 3) * kTileBytes, ldo, wave_u, lane, min(kTile, n_vis - (t0 + k) * kTile));
      };
      issue(0);
      if (n_tiles > 1) issue(1);
      for (int k = 0; k < n_tiles; ++k) {
        if (k + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerTile));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();   // tile k in LDS for all; the slot of tile k+2 was read two steps ago
        if (k + 2 < n_tiles) issue(k + 2);
        acc += *(MLA_LDS const uint32_t*)(uintptr_t)(lbase + (k & 3) * kTileBytes + 4 * tid);
      }
      __syncthreads();     // the next segment's first loads reuse the slots
      pos = seg_end;
      ++u;
      seg0_off = -1;
    }
  }
  sums[(size_t)blockIdx.x * kThreads + tid] = acc;
}

// ---------------------------------------------------------------------------- combine

// One workgroup of one wave per (work unit, 2 heads): lane l covers columns 4((l & 31)
// + 32v) .. +3 (v = 0..3) of head 2y + l/32, so each load instruction reads two
// contiguous 512-byte runs.  (Workgroups of one wave put more of them in flight at once:
// against 8 heads per workgroup of four waves the merge took 13% less time at batch 1,
// 6% at batch 16 and batch 4 x 2 queries, 1% at batch 64.)  Units
// finished in place are skipped; units without visible tokens get zeros and
// lse = -inf.  A split unit's fragments are merged in two passes: the lse of
// every fragment first (one fragment per lane of the head's half-wave), giving
// the largest lse m and each fragment's weight 2^(lse_f - m); then the partial
// outputs in batches of kCombineBatch fragments whose loads are all in flight
// together (the first batch already while the lse are awaited), accumulated in
// increasing fragment order (a fixed order: results do not depend on timing), and
// divided by the sum of the weights at the end.
constexpr int kCombineHeads = 2;
constexpr int kCombineBatch = 8;

__device__ __forceinline__ int fragment_slot(int gg, int g0, int chunk, int cbeg) {
  // The first fragment is a later segment of its workgroup when that workgroup's range
  // starts before the unit on the cost line (it then holds tiles of an earlier unit);
  // every later fragment is a first segment.
  return (gg == g0 && gg * chunk < cbeg) ? 2 * gg + 1 : 2 * gg;
}

__global__ __attribute__((amdgpu_flat_work_group_size(32 * kCombineHeads, 32 * kCombineHeads)))
void combine_kernel(DecodeArgs a, int W) {
  const int u = blockIdx.x;
  const int U = a.batch * a.s_q;
  const int T = ld_uniform(a.cum, 2 * U + 1), seg = ld_uniform(a.cum, 2 * U + 2);
  const int ubeg = ld_uniform(a.cum, u), uend = ld_uniform(a.cum, u + 1);
  const int cbeg = ld_uniform(a.cum, U + 1 + u);   // the unit's start on the cost line
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31;
  const int head = blockIdx.y * kCombineHeads + 2 * (tid >> 6) + (lane >> 5);
  const int col = 4 * l32;   // + 128 v
  uint16_t* dst = a.out_latent + ((size_t)u * kHeads + head) * kLatent + col;
  if (uend <= ubeg) {
#pragma unroll
    for (int v = 0; v < 4; ++v) *(u32x2*)(dst + 128 * v) = u32x2{0u, 0u};
    if (a.lse != nullptr && l32 == 0) a.lse[(size_t)u * kHeads + head] = -INFINITY;
    return;
  }
  // workgroups whose ranges hold the unit's first and last tiles (see work_range)
  const int chunk = split_chunk(T, W, a.min_chunk);
  const int g0 = (cbeg + seg) / chunk, g1 = (cbeg + seg + (uend - ubeg) - 1) / chunk;
  if (g0 == g1) return;
  const int F = g1 - g0 + 1;   // fragments of the unit, in workgroup order

  // Pass 1: lse of fragment f is read by lane f % 32 of the head's half-wave.  The first
  // 32 fragments' lse go out first and the first batch of partials right behind them (the
  // partials do not depend on the lse), so the wait for the lse leaves that batch in flight.
  auto frag_lse = [&](int f) {
    return f < F ? a.part_lse[(size_t)fragment_slot(g0 + f, g0, chunk, cbeg) * kHeads + head] : -INFINITY;
  };
  auto load_batch = [&](int f0, u32x2 (&x)[kCombineBatch][4]) {
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const int f = f0 + j < F ? f0 + j : F - 1;   // past the end: a valid fragment, weight 0
      const uint16_t* src =
          a.part_o + ((size_t)fragment_slot(g0 + f, g0, chunk, cbeg) * kHeads + head) * kLatent + col;
#pragma unroll
      for (int v = 0; v < 4; ++v) x[j][v] = __builtin_nontemporal_load((const u32x2*)(src + 128 * v));
    }
  };
  const float l_first = frag_lse(l32);
  asm volatile("" ::: "memory");   // the lse load is issued before the partial loads
  u32x2 x[kCombineBatch][4];
  load_batch(0, x);
  float m = l_first;
  for (int f0 = 32; f0 < F; f0 += 32) m = fmaxf(m, frag_lse(f0 + l32));
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 32));
  float wsum = l32 < F ? exp2f(l_first - m) : 0.f;
  for (int f0 = 32; f0 < F; f0 += 32) {
    const float l = frag_lse(f0 + l32);
    wsum += f0 + l32 < F ? exp2f(l - m) : 0.f;
  }
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off, 32);

  // Pass 2: the partial outputs, kCombineBatch fragments in flight at a time.
  auto widen = [](const u32x2& x) {
    return f32x4{bf2f((uint16_t)(x[0] & 0xFFFFu)), bf2f((uint16_t)(x[0] >> 16)), bf2f((uint16_t)(x[1] & 0xFFFFu)),
                 bf2f((uint16_t)(x[1] >> 16))};
  };
  f32x4 acc[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float wl = 0.f;   // weight of fragment f0 + l32 (this lane's), shared through the half-wave
  for (int f0 = 0; f0 < F; f0 += kCombineBatch) {
    if (f0 > 0) load_batch(f0, x);
    if ((f0 & 31) == 0) {
      const float l = f0 == 0 ? l_first : frag_lse(f0 + l32);
      wl = f0 + l32 < F ? exp2f(l - m) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const float w = __shfl(wl, ((f0 + j) & 31) + (lane & 32), 64);
      if (f0 + j < F) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] += widen(x[j][v]) * w;
      }
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    *(u32x2*)(dst + 128 * v) = u32x2{pack_bf16x2(acc[v][0] * inv, acc[v][1] * inv),
                                     pack_bf16x2(acc[v][2] * inv, acc[v][3] * inv)};
  if (a.lse != nullptr && l32 == 0) a.lse[(size_t)u * kHeads + head] = (m + __log2f(wsum)) * kLn2;
}

// ---------------------------------------------------------------------------- gather (test export)

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void gather_kernel(const uint16_t* __restrict__ kv, const int32_t* __restrict__ bt, const int32_t* __restrict__ seqlens,
                   uint16_t* __restrict__ dense, int max_blocks, int64_t num_pages) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(seqlens[b], max_blocks);
  int valid = L - j * kPage;
  valid = valid < 0 ? 0 : (valid > kPage ? kPage : valid);
  int64_t phys = valid > 0 ? bt[(size_t)b * max_blocks + j] : 0;
  phys = phys < 0 ? 0 : (phys >= num_pages ? num_pages - 1 : phys);
  const u32x4* src = (const u32x4*)(kv + phys * (int64_t)(kPage * kRow));
  u32x4* dst = (u32x4*)(dense + ((size_t)b * max_blocks * kPage + (size_t)j * kPage) * kRow);
  for (int c = threadIdx.x; c < kChunksPerPage; c += 256) {
    const int row = c / kChunksPerRow;
    dst[c] = row < valid ? src[c] : u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

hipError_t launch_decode(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv, const unsigned char* kv8,
                         const int32_t* bt, const int32_t* seqlens, uint16_t* out_latent, float* lse, int batch,
                         int s_q, int max_blocks, int64_t num_pages, float scale, int wgs, int min_chunk,
                         const DecodePlanView& plan, hipStream_t s, hipEvent_t ev_plan_done,
                         hipEvent_t ev_decode_done) {
  if (batch <= 0) return hipSuccess;
  DecodeArgs a{};
  a.min_chunk = min_chunk;
  a.q_abs = q_abs; a.q_r = q_r; a.kv = kv; a.kv8 = kv8; a.bt = bt; a.seqlens = seqlens;
  a.out_latent = out_latent; a.lse = lse; a.cum = plan.cum; a.part_o = plan.part_o; a.part_lse = plan.part_lse;
  a.num_pages = num_pages; a.batch = batch; a.s_q = s_q; a.max_blocks = max_blocks;
  a.last_page = (int)((num_pages < ((int64_t)1 << 31) ? num_pages : ((int64_t)1 << 31)) - 1);
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = hipSuccess;
  if (decode_launches_plan(batch * s_q)) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a, plan.cum, wgs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ev_plan_done != nullptr && (e = hipEventRecord(ev_plan_done, s)) != hipSuccess) return e;
  if (kv8 != nullptr)
    hipLaunchKernelGGL(decode_kernel<true>, dim3(wgs), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<false>, dim3(wgs), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_decode_done != nullptr && (e = hipEventRecord(ev_decode_done, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(batch * s_q, kHeads / kCombineHeads), dim3(32 * kCombineHeads), 0, s, a, wgs);
  return hipGetLastError();
}

bool decode_launches_plan(int units) { return units > kSelfPlanUnits; }

hipError_t launch_stream(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint32_t* sums, int batch,
                         int s_q, int max_blocks, int64_t num_pages, int wgs, int min_chunk, int32_t* cum,
                         hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  DecodeArgs a{};
  a.min_chunk = min_chunk;
  a.kv = kv; a.bt = bt; a.seqlens = seqlens; a.cum = cum;
  a.num_pages = num_pages; a.batch = batch; a.s_q = s_q; a.max_blocks = max_blocks;
  a.last_page = (int)((num_pages < ((int64_t)1 << 31) ? num_pages : ((int64_t)1 << 31)) - 1);
  if (decode_launches_plan(batch * s_q)) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a, cum, wgs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(stream_kernel, dim3(wgs), dim3(kThreads), 0, s, a, sums);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- allocation-free workspace

// The split-KV workspace of the allocation-free paged decode (prefix sums, partial lse
// and partial outputs, laid out as for a caller's workspace): a file-scope device array,
// one copy per device the library runs on, held until the process ends.  Every call on a
// device shares that device's copy; nothing in it needs clearing between calls (the
// decode writes every value it reads in the same call).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(unsigned char** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static unsigned char* dev_ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (dev_ptr[dev] == nullptr) {
    // the device's own address of its copy; the host-side name is only a stand-in
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    dev_ptr[dev] = static_cast<unsigned char*>(p);
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gather(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint16_t* dense, int batch,
                         int max_blocks, int64_t num_pages, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(max_blocks, batch), dim3(256), 0, s, kv, bt, seqlens, dense, max_blocks,
                     num_pages);
  return hipGetLastError();
}

}  // namespace mla
