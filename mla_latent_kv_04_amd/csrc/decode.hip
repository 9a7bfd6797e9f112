// Split-KV paged decode of absorbed MLA on gfx950.
//
// Per work unit u = (sequence b, query i) the attention is, for all 128 heads
// at once (all heads share the cached latent, so this is a dense contraction):
//   S^T[t, h] = (c_KV[t] . q_abs[h] + k_R[t] . q_R[h]) * scale     (K = 576)
//   out_latent[h] = sum_t softmax_t(S[h, t]) * c_KV[t]            (K = 64 per page)
// ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 4, path B for the scores; the
// output stays in latent space and is up-projected by W_UV afterwards.)
//
// Work split: the pages of all units are laid end to end; workgroup g takes the
// contiguous range [g*chunk, (g+1)*chunk) of that list (chunk = ceil(total/W)),
// so every compute unit streams the same number of pages whatever the length
// mix.  A unit that lies inside one range is finished in place; a unit cut by
// range borders leaves one normalised partial per piece (slot 2g for the first
// segment of workgroup g, 2g+1 for its last), merged by log-sum-exp afterwards.
//
// Workgroup: 256 threads = 4 waves, one per SIMD.  Each page (64 tokens x
// 1152 B = 72 KiB) is copied HBM -> LDS with direct 16-byte loads
// (global_load_lds_dwordx4), double buffered (2 x 72 KiB), plus a 16 KiB P
// buffer: the 160 KiB of LDS exactly.  Wave w computes the scores of heads
// 32w..32w+31 (its 32 queries live in 144 VGPRs) and the output of all heads
// for latent columns 128w..128w+127 (256 accumulator registers for the whole
// segment); see decode_kernel for the per-page steps.
// LDS layout of a page: a latent region of token rows (64 sixteen-byte chunks)
// and a RoPE region (8 chunks per token), each with an XOR swizzle of the chunk
// index that keeps both the row reads of QK (16 tokens, one chunk) and the
// 4-row transposing reads of PV free of bank conflicts.
#include "common.h"

namespace mla {

namespace {

constexpr int kThreads = 256;
constexpr int kLoadsPerThread = kChunksPerPage / kThreads;  // 18 direct loads per thread per page
static_assert(kChunksPerPage % kThreads == 0, "page must split evenly over the workgroup");
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  const uint16_t* q_abs;
  const uint16_t* q_r;
  const uint16_t* kv;
  const int32_t* bt;
  const int32_t* seqlens;
  uint16_t* out_latent;
  float* lse;
  const int32_t* cum;
  float* part_o;
  float* part_lse;
  int64_t num_pages;
  int batch, s_q, max_blocks;
  float scale_log2;  // scale * log2(e)
};

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

// Prefix sums of pages per work unit: cum[0] = 0, cum[u+1] = cum[u] + ceil(visible_u / 64).
__global__ __attribute__((amdgpu_flat_work_group_size(1024, 1024)))
void plan_kernel(DecodeArgs a, int32_t* cum) {
  __shared__ int32_t warp_tot[16];
  __shared__ int32_t carry_s;
  const int U = a.batch * a.s_q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { carry_s = 0; cum[0] = 0; }
  __syncthreads();
  for (int base = 0; base < U; base += 1024) {
    const int u = base + tid;
    int pages = 0;
    if (u < U) {
      const int n = unit_visible(a, u);
      pages = n > 0 ? (n + kPage - 1) / kPage : 0;
    }
    // inclusive scan inside the wave
    int x = pages;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) warp_tot[wave] = x;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += warp_tot[w];
    if (u < U) cum[u + 1] = before + x;
    __syncthreads();
    if (tid == 1023) carry_s = before + x;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------- decode

// LDS page buffer (73728 B): latent region [64 tokens][1024 B] at offset 0,
// RoPE region [64 tokens][128 B] at offset 65536, both swizzled as above.
constexpr int kRopeRegion = kPage * kLatent * 2;  // 65536

// Page copy HBM -> LDS: wave w copies the latent rows of tokens w, w+4, ...,
// w+60 (one 64-lane direct load per row, lane l = chunk position l) and the
// RoPE rows of tokens 16w .. 16w+15 (two loads; lane l -> token 8j + l/8,
// chunk position l%8).  The per-lane global byte offsets below are constant.
struct PageLoadOffsets {
  uint32_t lat[4];    // latent row offset for tokens t with t % 16 == w + 4k
  uint32_t rope[2];   // RoPE offsets (relative to token 8j) for j = 2w, 2w+1
};

__device__ __forceinline__ PageLoadOffsets page_load_offsets(int lane, int wave_u) {
  PageLoadOffsets o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o.lat[k] = (uint32_t)((lane ^ swz_lat(wave_u + 4 * k)) * 16);
  const int tr = lane >> 3, pr = lane & 7;
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) o.rope[j2] = (uint32_t)(tr * kRowBytes + kLatent * 2 + (pr ^ ((4 * j2 + (lane >> 4)) & 7)) * 16);
  return o;
}

// One 16-byte-per-lane direct load HBM -> LDS (global_load_lds_dwordx4): lane l
// reads sbase + voff and its 16 bytes land at LDS byte address lds + 16 l.
// Issued as inline asm so the compiler's wait-count model does not see the
// LDS write: it would otherwise wait for every load in flight (including the
// prefetch of the next page) before each LDS read.  The kernel waits for
// these loads itself with explicit vmcnt waits.  The leading s_nop covers the
// one wait state an M0 write needs before an LDS DMA instruction.  The cache
// is read once, so the loads are non-temporal: with `nt` the page stream runs
// at about 7.0 TB/s on MI355X, without it at about 6.2 TB/s.
// No "memory" clobber: the load only writes the LDS buffer that no wave reads
// until the next page barrier, and a volatile asm is never moved across that
// barrier; LDS reads of the current page may be scheduled around it freely.
__device__ __forceinline__ void dma_b128(const unsigned char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(MLA_LDS const void*)p;
}

// Rows at or past `valid` (only in a sequence's last page) are fetched from
// row 0 of the same page instead: they are masked out of the softmax, and
// loading finite data keeps 0 * V finite even when the unused rows of the
// cache hold NaN or Inf bit patterns.
__device__ __forceinline__ void issue_page(const unsigned char* __restrict__ src, unsigned char* buf,
                                           const PageLoadOffsets& off, int wave_u, int lane, int valid) {
  const uint32_t lbase = lds_addr(buf);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = wave_u + 4 * i;
    const int trow = t < valid ? t : 0;
    dma_b128(src + trow * kRowBytes, off.lat[i & 3], lbase + t * 1024);
  }
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) {
    const int j = 2 * wave_u + j2;
    const uint32_t ro = (8 * j + (lane >> 3) < valid) ? 8 * j * kRowBytes + off.rope[j2]
                                                       : (uint32_t)(kLatent * 2 + (lane & 7) * 16);
    dma_b128(src, ro, lbase + kRopeRegion + 1024 * j);
  }
}

// One of the 18 direct loads of a page (d = 0..15: latent row of token
// w + 4d; d = 16, 17: RoPE rows of tokens 8j .. 8j+7, j = 2w + d - 16).
__device__ __forceinline__ void issue_page_part(const unsigned char* __restrict__ src, uint32_t lbase,
                                                const PageLoadOffsets& off, int wave_u, int lane, int valid, int d) {
  if (d < 16) {
    const int t = wave_u + 4 * d;
    const int trow = t < valid ? t : 0;
    dma_b128(src + trow * kRowBytes, off.lat[d & 3], lbase + t * 1024);
  } else {
    const int j2 = d - 16, j = 2 * wave_u + j2;
    const uint32_t ro = (8 * j + (lane >> 3) < valid) ? 8 * j * kRowBytes + off.rope[j2]
                                                       : (uint32_t)(kLatent * 2 + (lane & 7) * 16);
    dma_b128(src, ro, lbase + kRopeRegion + 1024 * j);
  }
}

// The lane id through an opaque move: address offsets derived from it are
// recomputed where they are used instead of being hoisted out of every loop
// and kept live (the registers are needed for the queries and accumulators).
__device__ __forceinline__ int opaque_lane() {
  int v = (int)__lane_id();
  asm volatile("v_mov_b32 %0, %0" : "+v"(v));
  return v;
}

// Softmax reference.  Each segment takes its per-head reference maximum from
// its first page and keeps it: P = 2^(s - m_ref) in log2 units, so the O
// accumulators are never rescaled and any wave may accumulate any head.  A
// later score more than kHeadroom above the reference (P beyond 2^64, far
// outside real attention logits) makes the workgroup redo the segment once
// with the segment's true maximum as the reference, so the fp32 accumulators
// cannot overflow.
constexpr float kHeadroom = 64.0f;

// Per page (64 tokens) and wave w:
//   QK  S^T[64 tokens, heads 32w..32w+31] over K = 576 (72 MFMAs, A = page rows from
//       LDS, B = queries in registers); the next page's 18 direct loads are issued
//       between these MFMAs;
//   softmax of those 32 heads, P written as bf16 to the LDS P buffer [128 heads][64];
//   barrier;
//   PV  O[all 128 heads, latent columns 128w..128w+127] += P . c_KV (64 MFMAs, A = P
//       from LDS, B = page columns via transposing reads).
// Sharing P through LDS halves the PV operand traffic compared with every wave
// reading all 512 latent columns for its own heads.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kPageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[kHeads * kPage * 2];

  const int U = a.batch * a.s_q;
  const int total = a.cum[U];
  if (total <= 0) return;
  const int W = gridDim.x;
  const int chunk = (total + W - 1) / W;
  const int g = blockIdx.x;
  const int start = g * chunk;
  if (start >= total) return;
  const int end = min(total, start + chunk);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;       // which half of the wave
  const int l32 = lane & 31;
  const PageLoadOffsets ldo = page_load_offsets(lane, wave_u);

  // Largest u with cum[u] <= start (then cum[u+1] > start).
  int lo_u = 0, hi_u = U - 1;
  while (lo_u < hi_u) {
    const int mid = (lo_u + hi_u + 1) >> 1;
    if (a.cum[mid] <= start) lo_u = mid; else hi_u = mid - 1;
  }
  int u = lo_u;

  // P buffer row of this lane's head (writes): head 32w + l32, byte 8hi inside the chunk.
  const int pw_off = (wave_u * 32 + l32) * 128 + 8 * hi;
  const int ph = (l32 >> 1) & 7;

  bool first_seg = true;
  int pos = start;
  bool redo = false;              // re-run the current segment with m_redo as the reference
  float m_redo = -INFINITY;
  while (pos < end) {
    while (a.cum[u + 1] <= pos) ++u;
    const int ubeg = a.cum[u], uend = a.cum[u + 1];
    const int seg_end = min(end, uend);
    const int p0 = pos - ubeg, p1 = seg_end - ubeg;
    const bool complete = (pos == ubeg) && (seg_end == uend);
    const int slot = complete ? -1 : 2 * g + (first_seg ? 0 : 1);

    const int b = u / a.s_q;
    const int n_vis = unit_visible(a, u);
    const int32_t* bt_row = a.bt + (size_t)b * a.max_blocks;

    // Queries of this wave's 32 heads as the MFMA B operand: lane l holds head
    // 32w + l32, columns 16ks + 8hi .. +7 (k-steps 0..31 latent, 32..35 RoPE).
    const int head = wave_u * 32 + l32;
    const uint16_t* qa = a.q_abs + ((size_t)u * kHeads + head) * kLatent + 8 * hi;
    const uint16_t* qr = a.q_r + ((size_t)u * kHeads + head) * kRope + 8 * hi;
    s16x8 q[36];
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) q[ks] = *(const s16x8*)(qa + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[32 + ks] = *(const s16x8*)(qr + 16 * ks);

    auto page_src = [&](int p) -> const unsigned char* {
      int64_t phys = bt_row[p];
      phys = phys < 0 ? 0 : (phys >= a.num_pages ? a.num_pages - 1 : phys);
      return (const unsigned char*)a.kv + phys * (int64_t)kPageBytes;
    };

    f32x16 o[4][4];         // O[head block hb][column block c]
    // Reference max (log2 units) of head 32w + l32: from the first page, or the
    // segment's true maximum when the segment is being redone.
    float m_ref = redo ? m_redo : -INFINITY;
    float l_part = 0.f;       // this lane's share of that head's softmax denominator
    {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[hb][c][j] = 0.f;
      float m_seen = -INFINITY;
      bool overflow = false;

      {
        const unsigned char* src0 = page_src(p0);
        const uint32_t lb0 = lds_addr(lds);
#pragma unroll
        for (int d = 0; d < kLoadsPerThread; ++d) issue_page_part(src0, lb0, ldo, wave_u, lane, n_vis - p0 * kPage, d);
      }
      for (int p = p0; p < p1; ++p) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // this wave's loads of page p
        __syncthreads();                             // page p in LDS for all; page p-1 and P free
        const unsigned char* cur = lds + ((p - p0) & 1) * kPageBytes;
        const bool has_next = p + 1 < p1;
        const unsigned char* nsrc = page_src(has_next ? p + 1 : p);
        const uint32_t nbuf = lds_addr(lds + ((p + 1 - p0) & 1) * kPageBytes);
        const int nvalid = n_vis - (p + 1) * kPage;

        // ---- scores S^T: two 32-token blocks alternate (two accumulation chains);
        // LDS reads run kAhead MFMAs ahead; one next-page load per 4 MFMAs.
        // A operand, token block tb, k-step ks: token 32tb + l32, chunk 2ks + hi:
        //   latent (ks = 8p + q < 32): offA[q] + 256p + 32768tb;  RoPE (ks = 32 + q): offR[q] + 4096tb
        int offA[8], offR[4];
        {
          const int ln = opaque_lane(), lh = ln >> 5, ll = ln & 31;
          const int fa = swz_lat(ll), ga = swz_rope(ll);
#pragma unroll
          for (int q2 = 0; q2 < 8; ++q2) offA[q2] = ll * 1024 + 16 * ((2 * q2 + lh) ^ fa);
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) offR[q2] = kRopeRegion + ll * 128 + 16 * ((2 * q2 + lh) ^ ga);
        }
        f32x16 s0, s1;
#pragma unroll
        for (int j = 0; j < 16; ++j) { s0[j] = 0.f; s1[j] = 0.f; }
        {
          auto a_ptr = [&](int i) -> const s16x8* {
            const int tb = i & 1, ks = i >> 1;
            const unsigned char* pa = ks < 32 ? cur + offA[ks & 7] + 256 * (ks >> 3) + 32768 * tb
                                              : cur + offR[ks - 32] + 4096 * tb;
            return (const s16x8*)pa;
          };
          constexpr int kAhead = 4;
          s16x8 abuf[kAhead];
#pragma unroll
          for (int i = 0; i < kAhead; ++i) abuf[i] = *a_ptr(i);
#pragma unroll
          for (int i = 0; i < 72; ++i) {
            const s16x8 av = abuf[i % kAhead];
            if (i + kAhead < 72) abuf[i % kAhead] = *a_ptr(i + kAhead);
            if (i & 1) s1 = mfma32(av, q[i >> 1], s1);
            else s0 = mfma32(av, q[i >> 1], s0);
            if ((i & 3) == 3 && has_next) issue_page_part(nsrc, nbuf, ldo, wave_u, lane, nvalid, i >> 2);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);   // the first kAhead LDS reads
#pragma unroll
          for (int i = 0; i < 72; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            if (i + kAhead < 72) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then 1 LDS read
          }
        }
        __builtin_amdgcn_sched_barrier(0);

        // ---- softmax weights (base 2).  Register j of block tb is token
        // 32tb + 8(j/4) + 4hi + (j%4) of the page, head l32 of this wave.
        float x[32];
        const int tok0 = p * kPage;
        if (tok0 + kPage > n_vis) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int t = 8 * (j >> 2) + 4 * hi + (j & 3);
            x[j] = (tok0 + t < n_vis) ? s0[j] * a.scale_log2 : -INFINITY;
            x[16 + j] = (tok0 + 32 + t < n_vis) ? s1[j] * a.scale_log2 : -INFINITY;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) { x[j] = s0[j] * a.scale_log2; x[16 + j] = s1[j] * a.scale_log2; }
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 32; ++j) mx = fmaxf(mx, x[j]);
        m_seen = fmaxf(m_seen, mx);
        if (p == p0 && m_ref == -INFINITY) {   // first page (a redo arrives with m_ref set)
          m_ref = fmaxf(mx, __shfl_xor(mx, 32, 64));
        } else {
          overflow |= mx > m_ref + kHeadroom;
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) { x[j] = __builtin_amdgcn_exp2f(x[j] - m_ref); l_part += x[j]; }
        // P -> LDS: tokens 32tb + 8q + 4hi + 0..3 are registers 16tb + 4q + 0..3.
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            u32x2 w2;
            w2[0] = pack_bf16x2(x[16 * tb + 4 * qq], x[16 * tb + 4 * qq + 1]);
            w2[1] = pack_bf16x2(x[16 * tb + 4 * qq + 2], x[16 * tb + 4 * qq + 3]);
            *(u32x2*)(pbuf + pw_off + 16 * ((4 * tb + qq) ^ ph)) = w2;
          }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();   // P of all 128 heads visible

        // ---- O[all heads, columns 128w + ..] += P . c_KV over the page.
        // A operand (P), head block hb, k-step st: head 32hb + l32, tokens 16st + 8hi + 0..7
        //   -> offP[st] + 4096hb.  B operand (transposing read), half r, column block c
        //   (columns 128w + 32c ..): token 16st + 8hi + 4r + e, chunk 16w + 4c + cb, byte
        //   8 (lane & 1) -> offV[c][r] + 16384st + 4096r.
        int offP[4], offV[4][2];
        {
          const int ln = opaque_lane(), lh = ln >> 5, ll = ln & 31;
          const int pr = (ll >> 1) & 7;
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) offP[q2] = ll * 128 + 16 * ((2 * q2 + lh) ^ pr);
          const int eb = (ln & 15) >> 2;
          const int cb = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2)
#pragma unroll
            for (int r = 0; r < 2; ++r)
              offV[q2][r] = (8 * lh + eb) * 1024 + 64 * (q2 ^ eb) + 16 * (cb ^ (2 * lh + r)) + 8 * (ln & 1) + 256 * wave_u;
        }
        {
          // operands of k-step st: P tiles of the 4 head blocks, V tiles of the 4 column blocks
          auto load_ops = [&](int st, s16x8* pa, s16x8* bv) {
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) pa[hb] = *(const s16x8*)(pbuf + offP[st] + 4096 * hb);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const s16x4 lo = lds_read_tr4(cur + offV[c][0] + 16384 * st);
              const s16x4 h4 = lds_read_tr4(cur + offV[c][1] + 16384 * st + 4096);
              bv[c] = s16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
            }
          };
          s16x8 pa[2][4], bv[2][4];
          load_ops(0, pa[0], bv[0]);
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            if (st + 1 < 4) load_ops(st + 1, pa[(st + 1) & 1], bv[(st + 1) & 1]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int hb = 0; hb < 4; ++hb) o[hb][c] = mfma32(pa[st & 1][hb], bv[st & 1][c], o[hb][c]);
          }
          // reads of k-step st+1 (4 + 8) spread over the 16 MFMAs of k-step st
          __builtin_amdgcn_sched_group_barrier(0x100, 12, 1);
#pragma unroll
          for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
              if (st + 1 < 4 && m < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- end of pass: agree on a restart, publish row sums.  The page buffers
      // are free once every wave is past this barrier; they hold the scratch.
      __syncthreads();
      int* flags = (int*)lds;
      float* lsum = (float*)(lds + 256);
      const bool any_over = __builtin_amdgcn_ballot_w64(overflow) != 0;
      const float l_head = l_part + __shfl_xor(l_part, 32, 64);
      const float m_all = fmaxf(m_seen, __shfl_xor(m_seen, 32, 64));
      if (lane == 0) flags[wave_u] = any_over ? 1 : 0;
      if (hi == 0) lsum[head] = l_head;
      __syncthreads();
      const bool again = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
      m_redo = m_all;         // the segment's true maximum: no score exceeds it on a redo
      // normalise and write: O tile (hb, c), register j -> head 32hb + 8(j/4) + 4hi + (j%4),
      // column 128w + 32c + l32 (the lane part 4hi is folded into the base pointer so the
      // per-register row offsets are compile-time constants)
      if (!again) {
        const float lse2 = m_ref + __log2f(l_head);
        const float* lrow = lsum + 4 * hi;   // head 32hb + 8(j/4) + (j%4) from here
        const size_t obase = (size_t)(4 * hi) * kLatent + wave_u * 128 + l32;
        uint16_t* ob16 = a.out_latent + (size_t)u * kHeads * kLatent + obase;
        float* ob32 = a.part_o + (size_t)(slot < 0 ? 0 : slot) * kHeads * kLatent + obase;
  #pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          f32x16 il;
  #pragma unroll
          for (int j = 0; j < 16; ++j) il[j] = 1.f / lrow[32 * hb + 8 * (j >> 2) + (j & 3)];
  #pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x16 v = o[hb][c] * il;
            if (slot < 0) {
  #pragma unroll
              for (int j = 0; j < 16; ++j) ob16[(32 * hb + 8 * (j >> 2) + (j & 3)) * kLatent + 32 * c] = f2bf(v[j]);
            } else {
  #pragma unroll
              for (int j = 0; j < 16; ++j) ob32[(32 * hb + 8 * (j >> 2) + (j & 3)) * kLatent + 32 * c] = v[j];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (hi == 0) {
          if (slot < 0) {
            if (a.lse != nullptr) a.lse[(size_t)u * kHeads + head] = lse2 * kLn2;
          } else {
            a.part_lse[(size_t)slot * kHeads + head] = lse2;
          }
        }
      }
      __syncthreads();   // scratch read before the next segment refills the buffers
      redo = again;      // a redo runs the same segment again (pos unchanged)
    }
    if (!redo) {
      pos = seg_end;
      first_seg = false;
    }
  }
}

// ---------------------------------------------------------------------------- combine

// One workgroup per (work unit, 16 heads).  Units finished in place are
// skipped; units without visible tokens get zeros and lse = -inf; split units
// merge their partials in increasing workgroup order.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void combine_kernel(DecodeArgs a, int W) {
  const int u = blockIdx.x;
  const int U = a.batch * a.s_q;
  const int total = a.cum[U];
  const int ubeg = a.cum[u], uend = a.cum[u + 1];
  const int tid = threadIdx.x;
  const int head = blockIdx.y * 16 + (tid >> 4);
  const int c0 = (tid & 15) * 32;
  uint16_t* dst = a.out_latent + ((size_t)u * kHeads + head) * kLatent + c0;
  if (uend <= ubeg) {
#pragma unroll
    for (int v = 0; v < 4; ++v) *(u32x4*)(dst + 8 * v) = u32x4{0u, 0u, 0u, 0u};
    if (a.lse != nullptr && (tid & 15) == 0) a.lse[(size_t)u * kHeads + head] = -INFINITY;
    return;
  }
  const int chunk = (total + W - 1) / W;
  const int g0 = ubeg / chunk, g1 = (uend - 1) / chunk;
  if (g0 == g1) return;
  float m = -INFINITY;
  for (int gg = g0; gg <= g1; ++gg) {
    const int slot = (gg == g0 && gg * chunk < ubeg) ? 2 * gg + 1 : 2 * gg;
    m = fmaxf(m, a.part_lse[(size_t)slot * kHeads + head]);
  }
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.f;
  float wsum = 0.f;
  for (int gg = g0; gg <= g1; ++gg) {
    const int slot = (gg == g0 && gg * chunk < ubeg) ? 2 * gg + 1 : 2 * gg;
    const float w = exp2f(a.part_lse[(size_t)slot * kHeads + head] - m);
    wsum += w;
    const float* src = a.part_o + ((size_t)slot * kHeads + head) * kLatent + c0;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f32x4 x = *(const f32x4*)(src + 4 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * v + e] += w * x[e];
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[8 * v + 2 * e] * inv, acc[8 * v + 2 * e + 1] * inv);
    *(u32x4*)(dst + 8 * v) = w;
  }
  if (a.lse != nullptr && (tid & 15) == 0) a.lse[(size_t)u * kHeads + head] = (m + __log2f(wsum)) * kLn2;
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

hipError_t launch_decode(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv, const int32_t* bt,
                         const int32_t* seqlens, uint16_t* out_latent, float* lse, int batch, int s_q, int max_blocks,
                         int64_t num_pages, float scale, int wgs, const DecodePlanView& plan, hipStream_t s,
                         hipEvent_t ev_plan_done, hipEvent_t ev_decode_done) {
  if (batch <= 0) return hipSuccess;
  DecodeArgs a;
  a.q_abs = q_abs; a.q_r = q_r; a.kv = kv; a.bt = bt; a.seqlens = seqlens;
  a.out_latent = out_latent; a.lse = lse; a.cum = plan.cum; a.part_o = plan.part_o; a.part_lse = plan.part_lse;
  a.num_pages = num_pages; a.batch = batch; a.s_q = s_q; a.max_blocks = max_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a, plan.cum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_plan_done != nullptr && (e = hipEventRecord(ev_plan_done, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(decode_kernel, dim3(wgs), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_decode_done != nullptr && (e = hipEventRecord(ev_decode_done, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(batch * s_q, kHeads / 16), dim3(256), 0, s, a, wgs);
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint16_t* dense, int batch,
                         int max_blocks, int64_t num_pages, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(max_blocks, batch), dim3(256), 0, s, kv, bt, seqlens, dense, max_blocks,
                     num_pages);
  return hipGetLastError();
}

}  // namespace mla
