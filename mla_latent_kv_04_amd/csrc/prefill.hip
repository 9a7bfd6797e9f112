// Prefill of absorbed MLA on gfx950: the decompress branch.
//
// A chunk of M >= 256 new query tokens per sequence is cheaper to attend with
// the keys and values expanded per head than with matrix absorption
// ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 3: kPrefillThresh = 256,
// absorb below it and decompress above; section 6: the measured gain).  Two
// kernels:
//
//   decompress_kernel  K[b, h, t, :] = c_t . W_UK[h]^T,  V[b, h, t, :] = c_t . W_UV[h]
//                      for every cached token t < seqlens[b] ("DeepSeek的推理为什么
//                      比别人便宜一个数量级", leslieaibin.github.io, section "MLA":
//                      K = c . W_UK, V = c . W_UV), bf16 out, fp32 accumulation.
//   prefill_attention_kernel
//                      softmax((q_c . K_h + q_R . k_R) / sqrt(192)) . V_h with the
//                      chunk's causal rule (query i sees the first L - M + i + 1
//                      tokens), online softmax in fp32 (sheratonhq.com section 4
//                      for the score).
#include "prefill.h"

namespace mla {

namespace {

// ------------------------------------------------------------------ decompress

constexpr int kXWaves = 4;                     // waves per workgroup (one per SIMD)
constexpr int kXHalves = 2;                    // workgroups per head
constexpr int kXStreams = kXWaves * kXHalves;  // page streams per head
constexpr int kXSteps = kLatent / 16;          // MFMA k-steps over the latent
constexpr int kXAhead = 8;                     // k-steps of latent loads in flight ahead of their MFMAs
constexpr int kWPitchK = kLatent * 2 + 16;     // W_UK[h] in LDS as [n][k]: 1040 B rows, 4 banks apart
constexpr int kWPitchV = kDimC * 2;            // W_UV[h] in LDS as [k][n]: 256 B rows, 32-byte units swizzled
constexpr int kWBytes = kDimC * kWPitchK;      // 133 120 B, the larger layout
constexpr int kXStageRows = 16;                // output rows per staging round
constexpr int kXStage = kXStageRows * kDimC * 2;   // 4 KiB of output staging per wave
constexpr int kXBufFlags = 0x00020000;
static_assert(kLatent * kWPitchV <= kWBytes, "both weight layouts fit the LDS array");
static_assert(kWBytes + kXWaves * kXStage <= 160 * 1024, "weights and staging fit the LDS");
static_assert(kXSteps % kXAhead == 0, "the load ring restarts with every page");

struct DecompArgs {
  const uint16_t* kv;       // [num_pages, 64, 576]
  const int32_t* bt;        // [B, max_blocks]
  const int32_t* seqlens;   // [B]
  const uint16_t* w;        // W_UK [H, 128, 512] or W_UV [H, 512, 128]
  uint16_t* out;            // [B, H, max_len, 128]
  int64_t num_pages;
  int batch, max_blocks, max_len;
};

__device__ __forceinline__ int clamp_len(int L, int max_blocks) {
  const int cap = max_blocks * kPage;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// One head's expansion out^T[n, t] = sum_k W[n, k] c[t, k] over every cached page of
// every sequence.  Two workgroups per head (256 in all: one per compute unit), each
// with the head's whole weight matrix resident in LDS (W_UK[h] as [n][k], read with
// 16-byte loads; W_UV[h] as [k][n], read transposed), loaded once.  The pages of all
// sequences, in order, are dealt out to the 8 waves of the head's two workgroups in
// turn; a wave multiplies a page (64 tokens = 2 column blocks) by all 128 output
// columns (4 row blocks) of v_mfma_f32_32x32x16_bf16 over 32 k-steps.  The latent rows
// are the B operand and come straight from the cache into registers (16 bytes of one
// token per lane), kXAhead k-steps ahead of their MFMAs and across page boundaries, so
// the waves run without barriers once the weights are in.  A finished page goes out
// through a small per-wave LDS stage, 16 tokens at a time, so that every store
// instruction writes 1 KiB of the head's contiguous [token][128] output.
template <bool kIsV>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kXWaves, 64 * kXWaves), amdgpu_waves_per_eu(kXWaves / 4, kXWaves / 4)))
void decompress_kernel(DecompArgs a) {
  const int h = blockIdx.x / kXHalves;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = (blockIdx.x % kXHalves) * kXWaves + wave;
  __shared__ __attribute__((aligned(16))) unsigned char wt[kWBytes];
  __shared__ __attribute__((aligned(16))) unsigned char stages[kXWaves][kXStage];
  unsigned char* stage = stages[wave];

  // The head's weights: 8192 chunks of 16 bytes, all loads issued before the stores.
  {
    constexpr int kPer = kDimC * kLatent / 8 / (64 * kXWaves);
    const u32x4* src = reinterpret_cast<const u32x4*>(a.w + (size_t)h * kDimC * kLatent);
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = src[tid + 64 * kXWaves * i];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + 64 * kXWaves * i;
      // W_UV row k: 32-byte unit u of the row stored at unit u ^ 2 (k % 4), so that the
      // transposing reads of 4 consecutive rows by two lane groups hit distinct banks.
      const int k = c / 16, x = c % 16;
      const int off = kIsV ? k * kWPitchV + (((x >> 1) ^ (2 * (k & 3))) << 5) + (x & 1) * 16
                           : (c / 64) * kWPitchK + (c % 64) * 16;
      *(u32x4*)(wt + off) = v[i];
    }
  }
  __syncthreads();

  // Page walk (wave-uniform): page j of sequence b; the stream's pages are every
  // kXStreams-th (8th) page of the concatenation of all sequences' pages.
  struct Walk {
    int b, j, np;
  };
  auto pages_of = [&](int bb) { return (clamp_len(a.seqlens[bb], a.max_blocks) + kPage - 1) / kPage; };
  auto settle = [&](Walk& w) {
    while (w.b < a.batch && w.j >= w.np) {
      w.j -= w.np;
      ++w.b;
      w.np = w.b < a.batch ? pages_of(w.b) : 0;
    }
  };
  Walk cur{0, stream, pages_of(0)};
  settle(cur);
  if (cur.b >= a.batch) return;
  Walk nxt{cur.b, cur.j + kXStreams, cur.np};
  settle(nxt);
  // A page's rows as a buffer (a finished walk gives an empty one: its loads read zeros).
  auto page_rsrc = [&](const Walk& w) {
    int64_t page = w.b < a.batch ? a.bt[(size_t)w.b * a.max_blocks + w.j] : 0;
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.kv + (size_t)page * kPage * kRow), (short)0,
                                             w.b < a.batch ? kPageBytes : 0, kXBufFlags);
  };
  __amdgpu_buffer_rsrc_t rc = page_rsrc(cur), rn = page_rsrc(nxt);

  // B operand of column block nb at k-step ks: token 32 nb + lane % 32 of the page,
  // latent values 16 ks + 8 (lane / 32) .. +7.
  const uint32_t voff = (lane & 31) * kRowBytes + (lane >> 5) * 16;
  auto bload = [&](__amdgpu_buffer_rsrc_t r, int ks, int nb) {
    return __builtin_bit_cast(s16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, voff + nb * 32 * kRowBytes + ks * 32, 0, 0));
  };
  // A operand of row block m at k-step ks (output columns 32 m + lane % 32).
  // W_UV: rows 16 ks + 8 (lane / 32) + (lane % 16) / 4 (+4 for the second read), columns
  // 32 m + 16 g + 4 (lane % 4): 32-byte unit 2 m + g of the row, stored at unit
  // (2 m + g) ^ 2 (row % 4) = 2 (m ^ (row % 4)) + g (rows of one read share row % 4).
  const int g = (lane >> 4) & 1, s = lane & 15, r4 = (s >> 2) & 3;
  const unsigned char* abase = kIsV ? wt + (8 * (lane >> 5) + (s >> 2)) * kWPitchV + 32 * g + 8 * (s & 3)
                                    : wt + (lane & 31) * kWPitchK + 16 * (lane >> 5);
  auto aread = [&](int ks, int m) {
    if constexpr (kIsV) {
      const unsigned char* p = abase + 16 * ks * kWPitchV + 64 * (m ^ r4);
      const s16x4 lo = lds_read_tr4(p);
      const s16x4 hi = lds_read_tr4(p + 4 * kWPitchV);
      return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return *(const s16x8*)(abase + 32 * m * kWPitchK + 32 * ks);
    }
  };

  s16x8 bq[kXAhead][2];
#pragma unroll
  for (int ks = 0; ks < kXAhead; ++ks)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bq[ks][nb] = bload(rc, ks, nb);

  const f32x16 zero = {};
  while (true) {
    f32x16 acc[4][2];
    // weight operands two k-steps ahead (LDS latency exceeds one MFMA)
    s16x8 aop[3][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m = 0; m < 4; ++m) aop[ks][m] = aread(ks, m);
#pragma unroll
    for (int ks = 0; ks < kXSteps; ++ks) {
      if (ks + 2 < kXSteps) {
#pragma unroll
        for (int m = 0; m < 4; ++m) aop[(ks + 2) % 3][m] = aread(ks + 2, m);
      }
      const int slot = ks % kXAhead;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[m][nb] = mfma32(aop[ks % 3][m], bq[slot][nb], ks == 0 ? zero : acc[m][nb]);
      // refill the slot with the operand kXAhead k-steps on (the next page's first ones at the end)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        bq[slot][nb] = ks + kXAhead < kXSteps ? bload(rc, ks + kXAhead, nb) : bload(rn, ks + kXAhead - kXSteps, nb);
      __builtin_amdgcn_sched_barrier(0);
    }

    // D layout (32x32): lane l, register r -> row 8 (r / 4) + 4 (l / 32) + r % 4 (output column
    // within the row block), column l % 32 (token within the column block).  Four rounds of
    // 16 tokens through the wave's stage ([16 rows][256 B], 16-byte chunk c of row t stored
    // at chunk c ^ t): the 32 lanes holding the round's tokens write 8 bytes per register
    // quad, then all 64 lanes read 16 bytes each and store four consecutive tokens' rows
    // (1 KiB of the head's contiguous [token][128] block) per instruction.
    const int valid = clamp_len(a.seqlens[cur.b], a.max_blocks) - cur.j * kPage;
    uint16_t* dst_page = a.out + (((size_t)cur.b * kHeads + h) * a.max_len + cur.j * kPage) * kDimC;
#pragma unroll
    for (int rd = 0; rd < kPage / kXStageRows; ++rd) {
      constexpr int kRounds = 32 / kXStageRows;             // rounds per column block
      const int nb = rd / kRounds, sub = rd % kRounds;
      const int t = (lane & 31) - kXStageRows * sub;        // this lane's row in the round
      if (t >= 0 && t < kXStageRows) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x2 o;
            o[0] = pack_bf16x2(acc[m][nb][4 * q], acc[m][nb][4 * q + 1]);
            o[1] = pack_bf16x2(acc[m][nb][4 * q + 2], acc[m][nb][4 * q + 3]);
            const int chunk = 4 * m + q;                    // columns 8 chunk .. +7; this lane's 4 at +4 (l / 32)
            *(u32x2*)(stage + t * (kDimC * 2) + ((chunk ^ t) << 4) + 8 * (lane >> 5)) = o;
          }
      }
#pragma unroll
      for (int i = 0; i < kXStageRows / 4; ++i) {
        const int tr = 4 * i + (lane >> 4), c = lane & 15;
        const u32x4 v = *(const u32x4*)(stage + tr * (kDimC * 2) + ((c ^ tr) << 4));
        const int row = 32 * nb + kXStageRows * sub + tr;
        if (row < valid) *(u32x4*)(dst_page + (size_t)row * kDimC + 8 * c) = v;
      }
    }
    if (nxt.b >= a.batch) break;
    cur = nxt;
    rc = rn;
    nxt.j += kXStreams;
    settle(nxt);
    rn = page_rsrc(nxt);
  }
}

}  // namespace

hipError_t launch_decompress(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, const uint16_t* w_uk,
                             const uint16_t* w_uv, uint16_t* k_out, uint16_t* v_out, int batch, int max_blocks,
                             int max_len, int64_t num_pages, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  DecompArgs a;
  a.kv = kv;
  a.bt = bt;
  a.seqlens = seqlens;
  a.num_pages = num_pages;
  a.batch = batch;
  a.max_blocks = max_blocks;
  a.max_len = max_len;
  const dim3 grid(kHeads * kXHalves);
  a.w = w_uk;
  a.out = k_out;
  hipLaunchKernelGGL(decompress_kernel<false>, grid, dim3(64 * kXWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.w = w_uv;
  a.out = v_out;
  hipLaunchKernelGGL(decompress_kernel<true>, grid, dim3(64 * kXWaves), 0, s, a);
  return hipGetLastError();
}
}  // namespace mla

namespace mla {

namespace {

// ------------------------------------------------------------------ attention

constexpr int kAQW = 32;                 // queries per wave
constexpr int kAKeys = 64;               // keys per tile (one page)
constexpr int kAD = kDimC + kRope;       // 192: score dimension
constexpr int kKPitch = kAD * 2 + 16;    // 400 B: K tile rows [key][192]
constexpr int kVPitch = kDimC * 2 + 32;  // 288 B: V tile rows [key][128], 8 banks mod 32
constexpr int kKTile = kAKeys * kKPitch;
constexpr int kVTile = kAKeys * kVPitch;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDies = 8;                 // MI355X: 8 accelerator dies, each with its own L2
// Attention workgroup shape: waves (32 queries each) and LDS tile buffers.
constexpr int kAttnWaves = 8;
constexpr int kAttnBufs = 2;
// LDS operand reads issued this many MFMAs ahead of their use (key rows; value columns).
constexpr int kKeyAhead = 4;
constexpr int kValueAhead = 3;

struct AttnArgs {
  const uint16_t* q_c;      // [B, M, H, 128]
  const uint16_t* q_r;      // [B, M, H, 64]
  const uint16_t* k;        // [B, H, max_len, 128]
  const uint16_t* v;        // [B, H, max_len, 128]
  const uint16_t* kv;       // [num_pages, 64, 576] (k_R = columns 512..575)
  const int32_t* bt;        // [B, max_blocks]
  const int32_t* seqlens;   // [B]
  uint16_t* out;            // [B, M, H, 128]
  float* lse;               // [B, M, H] or null
  int64_t num_pages;
  int M, max_blocks, max_len;
  float scale_log2;         // softmax scale times log2(e)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_mfma_f32_32x32x16_bf16 with the accumulator in VGPRs (inline asm: a compiler-
// selected MFMA takes the AGPR form here and every VALU use of its result then costs
// a copy).  Hazards the asm covers itself: a leading s_nop separates a VALU write of
// an operand (or of the accumulator) from the MFMA's read; chains accumulate in place;
// the last MFMA of a chain carries 14 wait states, more than the 12 an 8-pass XDL
// result needs before a VALU read.
template <bool kZero, bool kLast>
__device__ __forceinline__ void mfma_v(f32x16& acc, const s16x8& a, const s16x8& b) {
  if constexpr (kZero && kLast)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\ts_nop 7\n\ts_nop 5"
                 : "=v"(acc) : "v"(a), "v"(b));
  else if constexpr (kZero)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
  else if constexpr (kLast)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 5"
                 : "+v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Uniform load through the scalar data cache (the block table is read-only here).
__device__ __forceinline__ int ld_scalar(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// One workgroup per (128-query tile, head, sequence).  Wave w owns queries
// i0 + 32 w .. +31.  Per 64-key tile (one page) it computes the transposed scores
// S^T[key, query] = K_tile . Q^T (v_mfma_f32_32x32x16_bf16: 2 key blocks x 12 k-steps
// over the 192 score dimensions, A = key rows from LDS, B = the wave's queries held
// in registers), so that each lane's accumulators belong to one query (lane % 32)
// and the online softmax needs one cross-lane exchange (lane ^ 32).  Then
// O^T[e, query] += V^T . P^T (4 column blocks x 4 k-steps; A = V columns through
// transposing LDS reads, B = the probabilities straight from the score registers,
// with the keys of each MFMA k-slot ordered as the score layout holds them).
// The next tile's loads are in flight in registers during the current tile's MFMAs
// and go to LDS between two barriers.  VALU work per tile is kept small: the scale is
// folded into the exponent's multiply-add, keys are masked only on tiles that
// reach past some query of the wave, and O is rescaled only when a running
// maximum of the wave actually grew.
template <int kW, int kBufs>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kW, 64 * kW), amdgpu_waves_per_eu(2, 2)))
void prefill_attention_kernel(AttnArgs a) {
  constexpr int kAQ = kAQW * kW;           // queries per workgroup
  constexpr int kT = 64 * kW;              // threads
  constexpr int kKH = 1024 / kT, kKR = 512 / kT, kVC = 1024 / kT;   // tile chunks per thread
  // Workgroups go round-robin over the 8 dies.  Ordinal o counts die-major, so each
  // die takes a contiguous run of (sequence, head) pairs with all their query tiles:
  // those tiles stream the same K/V rows at about the same time through one L2.
  // Within a pair the longest causal tiles come first.
  const int n_qt = (a.M + kAQ - 1) / kAQ;
  const int per_die = gridDim.x / kDies;
  const int ord = (blockIdx.x % kDies) * per_die + blockIdx.x / kDies;
  const int qt = n_qt - 1 - ord % n_qt;
  const int h = (ord / n_qt) % kHeads, b = ord / (n_qt * kHeads);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = clamp_len(a.seqlens[b], a.max_blocks);
  const int i0 = qt * kAQ;
  const int last_q = min(i0 + kAQ, a.M) - 1;
  const int p_last = L - a.M + last_q;                 // position of the tile's last query
  const int n_tiles = p_last >= 0 ? p_last / kAKeys + 1 : 0;

  // One LDS tile (44 KiB) so that two workgroups share a compute unit: while one
  // waits at a barrier or for its next tile, the other's MFMAs run.
  __shared__ __attribute__((aligned(16))) unsigned char kt[kBufs][kKTile];
  __shared__ __attribute__((aligned(16))) unsigned char vt[kBufs][kVTile];

  // This lane's query: i0 + 32 wave + lane % 32 (lanes l and l ^ 32 share it).
  const int qi = i0 + 32 * wave + (lane & 31);
  const bool q_ok = qi < a.M;
  const int qpos = L - a.M + qi;                       // keys t <= qpos are visible
  const int wave_first_pos = L - a.M + i0 + 32 * wave; // smallest query position of the wave
  const int g2 = lane >> 5;

  // Q^T operand: k-step ks covers score dimensions 16 ks + 8 g2 .. +7.
  s16x8 qop[kAD / 16];
  {
    const size_t row = ((size_t)b * a.M + (q_ok ? qi : 0)) * kHeads + h;
#pragma unroll
    for (int ks = 0; ks < kAD / 16; ++ks) {
      const int d = 16 * ks + 8 * g2;
      qop[ks] = d < kDimC ? *(const s16x8*)(a.q_c + row * kDimC + d)
                          : *(const s16x8*)(a.q_r + row * kRope + (d - kDimC));
    }
  }

  // Tile loads, as buffer loads whose per-lane byte offsets are fixed for the whole
  // loop (only the scalar base moves with the tile; no address temporaries for the
  // compiler to recycle while the loads are in flight).  Each buffer covers exactly
  // the tile's rows inside the sequence, so rows past it read as zeros.
  //   K_h: 64 rows x 16 chunks, 4 per thread; k_R: 64 rows x 8 chunks, 2 per thread;
  //   V_h: 64 rows x 16 chunks, 4 per thread.
  constexpr uint32_t kRowBytesKV = kDimC * 2;            // a head's keys (and values) are contiguous rows
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k) +
                               ((size_t)b * kHeads + h) * a.max_len * kDimC * 2;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v) +
                               ((size_t)b * kHeads + h) * a.max_len * kDimC * 2;
  uint32_t khoff[kKH], kroff[kKR], vvoff[kVC], khdst[kKH], krdst[kKR], vdst[kVC];
  static_assert(kKH == kVC, "K and V chunks share the loop below");
#pragma unroll
  for (int i = 0; i < kKH; ++i) {
    const int c = tid + kT * i, r = c / 16, x = c % 16;
    khoff[i] = r * kRowBytesKV + 16 * x;
    khdst[i] = r * kKPitch + 16 * x;
    vvoff[i] = r * kRowBytesKV + 16 * x;
    vdst[i] = r * kVPitch + 16 * x;
  }
#pragma unroll
  for (int i = 0; i < kKR; ++i) {
    const int c = tid + kT * i, r = c / 8, x = c % 8;
    kroff[i] = r * kRowBytes + 16 * x;
    krdst[i] = r * kKPitch + kDimC * 2 + 16 * x;
  }
  constexpr int kBufFlags = 0x00020000;
  u32x4 kreg[kKH + kKR], vreg[kVC];
  const int32_t* bt_row = a.bt + (size_t)b * a.max_blocks;
  auto load_tile = [&](int j, int raw_page) {
    const int t0 = j * kAKeys;
    const int valid = min(kAKeys, L - t0);
    const int64_t page = raw_page < 0 ? 0 : (raw_page >= a.num_pages ? a.num_pages - 1 : raw_page);
    const __amdgpu_buffer_rsrc_t kb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (size_t)t0 * kRowBytesKV), (short)0, valid * (int)kRowBytesKV, kBufFlags);
    const __amdgpu_buffer_rsrc_t vb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (size_t)t0 * kRowBytesKV), (short)0, valid * (int)kRowBytesKV, kBufFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.kv + (size_t)page * kPage * kRow + kLatent), (short)0, valid * kRowBytes, kBufFlags);
#pragma unroll
    for (int i = 0; i < kKH; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(kb, khoff[i], 0, 0);
#pragma unroll
    for (int i = 0; i < kKR; ++i) kreg[kKH + i] = __builtin_amdgcn_raw_buffer_load_b128(rb, kroff[i], 0, 0);
#pragma unroll
    for (int i = 0; i < kVC; ++i) vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(vb, vvoff[i], 0, 0);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kKH; ++i) *(u32x4*)(kt[buf] + khdst[i]) = kreg[i];
#pragma unroll
    for (int i = 0; i < kKR; ++i) *(u32x4*)(kt[buf] + krdst[i]) = kreg[kKH + i];
#pragma unroll
    for (int i = 0; i < kVC; ++i) *(u32x4*)(vt[buf] + vdst[i]) = vreg[i];
  };

  f32x16 o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[e][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;                // in scaled log2 units
  const float c1 = a.scale_log2;

  // Page ids come through scalar loads, one tile ahead of the loads that use them.
  int next_page = 0;
  if (n_tiles > 0) {
    load_tile(0, ld_scalar(bt_row));
    store_tile(0);
    if (n_tiles > 1) next_page = ld_scalar(bt_row + 1);
  }
  // Every load issued so far (queries, first tile) completes here: otherwise the
  // loop's wait counts, merged with this entry state, would make each tile wait for
  // the next tile's loads before its first MFMA.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = kBufs == 2 ? (j & 1) : 0;
    if (j + 1 < n_tiles) load_tile(j + 1, next_page);
    const unsigned char* K = kt[buf];
    const unsigned char* V = vt[buf];
    const int t0 = j * kAKeys;

    // S^T for key blocks mb = 0, 1: lane l, register r -> key 32 mb + 8 (r / 4) + 4 g2 + r % 4.
    // The 24 MFMAs run as one sequence (key block 0, then 1); each key-row operand is
    // read from LDS two MFMAs ahead of its use (the asm statements keep program order,
    // so the prefetch is written out).
    f32x16 s[2];
    {
      constexpr int kSteps = kAD / 16;
      const unsigned char* krow = K + (lane & 31) * kKPitch + 16 * g2;
      auto kread = [&](int n) {     // operand of MFMA n = (mb = n / 12, ks = n % 12)
        return *(const s16x8*)(krow + (n / kSteps) * 32 * kKPitch + (n % kSteps) * 32);
      };
      constexpr int kAhead = kKeyAhead;
      s16x8 kop[kAhead + 1];
#pragma unroll
      for (int n = 0; n < kAhead; ++n) kop[n] = kread(n);
#pragma unroll
      for (int n = 0; n < 2 * kSteps; ++n) {
        if (n + kAhead < 2 * kSteps) kop[(n + kAhead) % (kAhead + 1)] = kread(n + kAhead);
        const int mb = n / kSteps, ks = n % kSteps;
        const s16x8& ko = kop[n % (kAhead + 1)];
        if (ks == 0) mfma_v<true, false>(s[mb], ko, qop[ks]);
        else if (ks == kSteps - 1) mfma_v<false, true>(s[mb], ko, qop[ks]);
        else mfma_v<false, false>(s[mb], ko, qop[ks]);
      }
    }

    // Mask only where some key of the tile lies past some query of the wave.
    if (t0 + kAKeys - 1 > wave_first_pos) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + 32 * mb + 8 * (r >> 2) + 4 * g2 + (r & 3);
          s[mb][r] = key <= qpos ? s[mb][r] : -INFINITY;
        }
    }
    // Tile maximum of the raw scores (the scale is positive), then in scaled log2 units.
    float mt = max3f(s[0][0], s[0][1], s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mt = max3f(mt, s[0][r], s[0][r + 1]);
    mt = max3f(mt, s[0][15], s[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) mt = max3f(mt, s[1][r], s[1][r + 1]);
    mt = fmaxf(mt, s[1][15]);
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * c1;
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // Rescale O and l only when a running maximum of the wave grew.
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[e][r] *= alpha;
    }
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[mb][r], c1, -m_use));
        s[mb][r] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32);
    l_run += ps;

    // O^T += V^T . P^T.  k-step ks = (key block mb = ks / 2, half hf = ks % 2): slot i of
    // lane group g2 holds key 32 mb + 16 hf + 8 (i / 4) + 4 g2 + i % 4, i.e. score register
    // 8 hf + i.  The V^T operand gathers the same keys: two transposing reads of 4 rows.
    const int grp = (lane >> 4) & 1, sl = lane & 15;
    // V^T operand of MFMA n = (ks = n / 4, e = n % 4): rows 32 mb + 16 hf + 4 g2 + s / 4
    // (+8 for the second read), columns 32 e + 16 grp + 4 (s % 4); read one MFMA ahead.
    const unsigned char* vrow = V + (4 * g2 + (sl >> 2)) * kVPitch + (16 * grp + 4 * (sl & 3)) * 2;
    auto vread = [&](int n) {
      const int ks = n >> 2, e = n & 3;
      const unsigned char* p = vrow + (16 * ks) * kVPitch + 64 * e;
      const s16x4 lo = lds_read_tr4(p);
      const s16x4 hi = lds_read_tr4(p + 8 * kVPitch);
      return s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    s16x8 pops[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mb = ks >> 1, hf = ks & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w2 = pack_bf16x2(s[mb][8 * hf + 2 * i], s[mb][8 * hf + 2 * i + 1]);
        pops[ks][2 * i] = (short)(w2 & 0xFFFFu);
        pops[ks][2 * i + 1] = (short)(w2 >> 16);
      }
    }
    constexpr int kVA = kValueAhead;
    s16x8 vop[kVA + 1];
#pragma unroll
    for (int n = 0; n < kVA; ++n) vop[n] = vread(n);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      if (n + kVA < 16) vop[(n + kVA) % (kVA + 1)] = vread(n + kVA);
      const int ks = n >> 2, e = n & 3;
      if (ks == 3) mfma_v<false, true>(o[e], vop[n % (kVA + 1)], pops[ks]);
      else mfma_v<false, false>(o[e], vop[n % (kVA + 1)], pops[ks]);
    }

    // the page id two tiles ahead: its scalar load completes under the barrier
    if (j + 2 < n_tiles) next_page = ld_scalar(bt_row + j + 2);
    if constexpr (kBufs == 2) {
      if (j + 1 < n_tiles) store_tile(buf ^ 1);
      __syncthreads();
    } else {
      __syncthreads();
      if (j + 1 < n_tiles) store_tile(0);
      __syncthreads();
    }
  }

  if (!q_ok) return;
  // O^T layout: lane l, register r -> e = 32 blk + 8 (r / 4) + 4 g2 + r % 4, query lane % 32.
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* dst = a.out + (((size_t)b * a.M + qi) * kHeads + h) * kDimC;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2 w;
      w[0] = pack_bf16x2(o[e][4 * q] * inv, o[e][4 * q + 1] * inv);
      w[1] = pack_bf16x2(o[e][4 * q + 2] * inv, o[e][4 * q + 3] * inv);
      *(u32x2*)(dst + 32 * e + 8 * q + 4 * g2) = w;
    }
  if (a.lse != nullptr && g2 == 0)
    a.lse[((size_t)b * a.M + qi) * kHeads + h] = l_run > 0.f ? (m_run + __log2f(l_run)) / kLog2e : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_attention(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* k, const uint16_t* v,
                                    const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint16_t* out,
                                    float* lse, int batch, int M, int max_blocks, int max_len, int64_t num_pages,
                                    float scale, hipStream_t s) {
  if (batch <= 0 || M <= 0) return hipSuccess;
  AttnArgs a;
  a.q_c = q_c;
  a.q_r = q_r;
  a.k = k;
  a.v = v;
  a.kv = kv;
  a.bt = bt;
  a.seqlens = seqlens;
  a.out = out;
  a.lse = lse;
  a.num_pages = num_pages;
  a.M = M;
  a.max_blocks = max_blocks;
  a.max_len = max_len;
  a.scale_log2 = scale * kLog2e;
  // n_qt x 128 heads x batch workgroups: a multiple of the 8 dies since 128 is.
  constexpr int kW = kAttnWaves, kBufs = kAttnBufs;
  hipLaunchKernelGGL((prefill_attention_kernel<kW, kBufs>), dim3((M + kAQW * kW - 1) / (kAQW * kW) * kHeads * batch),
                     dim3(64 * kW), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
