// Prefill of absorbed MLA on gfx950: the decompress branch.
//
// A chunk of M >= 256 new query tokens per sequence is cheaper to attend with
// the keys and values expanded per head than with matrix absorption
// ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 3: kPrefillThresh = 256,
// absorb below it and decompress above; section 6: the measured gain).  Two
// kernels:
//
//   decompress_kernel  K[b, t, h, :] = c_t . W_UK[h]^T,  V[b, t, h, :] = c_t . W_UV[h]
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

constexpr int kDTok = 256;        // tokens per decompress workgroup
constexpr int kDK = 64;           // latent values per K-loop chunk
constexpr int kDPitchRow = kDK * 2 + 16;      // [row][k] tiles: rows 4 banks apart mod 64 for 16-byte reads
constexpr int kCCPR = kDK * 2 / 16;           // 16-byte chunks per [row][k] tile row
constexpr int kCRows = 512 / kCCPR;           // rows one pass of 512 threads covers
constexpr int kCP = kDTok / kCRows;           // passes per chunk (equal to kDK / 16, the V tile's)
constexpr int kDPitchV = 2 * kDimC * 2 + 32;  // [64 k][256 n] tile: 544 B = 8 banks mod 32 for transposing reads

struct DecompArgs {
  const uint16_t* kv;       // [num_pages, 64, 576]
  const int32_t* bt;        // [B, max_blocks]
  const int32_t* seqlens;   // [B]
  const uint16_t* w;        // W_UK [H, 128, 512] or W_UV [H, 512, 128]
  uint16_t* out;            // [B, max_len, H, 128]
  int64_t num_pages;
  int max_blocks, max_len;
};

__device__ __forceinline__ int clamp_len(int L, int max_blocks) {
  const int cap = max_blocks * kPage;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Computes the transposed product out^T[n, t] = sum_k W[n, k] c[t, k] for 256 tokens
// and the 256 output columns of two heads, so that each lane's accumulators hold
// consecutive output columns of one token (8-byte stores).  Eight waves: wave w
// owns head 2 hp + w / 4 (128 columns = 4 MFMA row blocks) and tokens
// 64 (w % 4) .. +63 (2 column blocks) of v_mfma_f32_32x32x16_bf16.  The A
// operand (weights) comes from LDS: for K row-major [n][k] (16-byte reads), for
// V [k][n] through transposing reads; the B operand (latent rows) from a
// [token][k] LDS tile.  Each kDK-wide chunk of the latent is loaded into
// registers while the previous one is multiplied.
template <bool kIsV>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512)))
void decompress_kernel(DecompArgs a) {
  const int hp = blockIdx.x, tb = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(a.seqlens[b], a.max_blocks);
  const int t0 = tb * kDTok;
  if (t0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  constexpr int kWBytes = kIsV ? kDK * kDPitchV : 2 * kDimC * kDPitchRow;
  __shared__ __attribute__((aligned(16))) unsigned char wt[kWBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ct[kDTok * kDPitchRow];

  static_assert(kCP == kDK / 16, "latent and weight chunks take the same number of passes");
  // Latent chunk loads: thread -> token row tid / kCCPR + kCRows i, 16 bytes at k 8 (tid % kCCPR).
  const uint16_t* crow[kCP];
#pragma unroll
  for (int i = 0; i < kCP; ++i) {
    const int t = t0 + tid / kCCPR + kCRows * i;
    const int tt = t < L ? t : 0;             // rows past the sequence read its token 0, never stored
    int64_t page = a.bt[(size_t)b * a.max_blocks + tt / kPage];
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    crow[i] = a.kv + ((size_t)page * kPage + (tt & (kPage - 1))) * kRow + 8 * (tid % kCCPR);
  }
  unsigned char* cdst = ct + (tid / kCCPR) * kDPitchRow + (tid % kCCPR) * 16;

  // Weight chunk loads.
  const uint16_t* wsrc[kCP];
  unsigned char* wdst[kCP];
#pragma unroll
  for (int i = 0; i < kCP; ++i) {
    if (!kIsV) {
      // W_UK rows n = tid / kCCPR + kCRows i of the head pair ([n][k], 16 bytes at k 8 (tid % kCCPR))
      const int n = tid / kCCPR + kCRows * i;
      wsrc[i] = a.w + ((size_t)(2 * hp + n / kDimC) * kDimC + (n % kDimC)) * kLatent + 8 * (tid % kCCPR);
      wdst[i] = wt + n * kDPitchRow + (tid % kCCPR) * 16;
    } else {
      // W_UV rows k = tid / 32 + 16 i of the chunk, 16 bytes of head 2 hp + (tid % 32) / 16 at e 8 (tid % 16)
      const int k = tid / 32 + 16 * i, nc = tid % 32;
      wsrc[i] = a.w + ((size_t)(2 * hp + nc / 16) * kLatent + k) * kDimC + 8 * (nc % 16);
      wdst[i] = wt + k * kDPitchV + nc * 16;
    }
  }

  u32x4 cv[kCP], wv[kCP];
  auto load_chunk = [&](int kc) {
    const int k0 = kc * kDK;
#pragma unroll
    for (int i = 0; i < kCP; ++i) cv[i] = *(const u32x4*)(crow[i] + k0);
#pragma unroll
    for (int i = 0; i < kCP; ++i) wv[i] = *(const u32x4*)(wsrc[i] + (kIsV ? (size_t)k0 * kDimC : (size_t)k0));
  };

  const int nh = wave / 4;            // head of the pair this wave computes
  const int tq = wave % 4;            // token quarter
  f32x16 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][n][j] = 0.f;

  load_chunk(0);
  for (int kc = 0; kc < kLatent / kDK; ++kc) {
    if (kc > 0) __syncthreads();
#pragma unroll
    for (int i = 0; i < kCP; ++i) *(u32x4*)(cdst + kCRows * i * kDPitchRow) = cv[i];
#pragma unroll
    for (int i = 0; i < kCP; ++i) *(u32x4*)wdst[i] = wv[i];
    __syncthreads();
    if (kc + 1 < kLatent / kDK) load_chunk(kc + 1);
    // keep the next chunk's loads ahead of this chunk's MFMAs (the scheduler would sink
    // them to their use, exposing the whole memory latency once per chunk)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kDK / 16; ++ks) {
      s16x8 bop[2];
#pragma unroll
      for (int n = 0; n < 2; ++n)
        bop[n] = *(const s16x8*)(ct + (64 * tq + 32 * n + (lane & 31)) * kDPitchRow + (16 * ks + 8 * (lane >> 5)) * 2);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        s16x8 aop;
        const int nrow = kDimC * nh + 32 * m;   // first output column of this row block
        if (!kIsV) {
          aop = *(const s16x8*)(wt + (nrow + (lane & 31)) * kDPitchRow + (16 * ks + 8 * (lane >> 5)) * 2);
        } else {
          // A[n][k] = W_UV[k][n]: rows k 16 ks + 8 (lane / 32) + 0..7 of column n, as two
          // transposing reads of 4 rows.  Within a 16-lane group, lane s reads row 4 e + s / 4
          // ... at columns 4 (s % 4): the group covers columns nrow + 16 (lane % 32 / 16) .. +15.
          const int g = (lane >> 4) & 1, s = lane & 15;
          const unsigned char* p = wt + (16 * ks + 8 * (lane >> 5) + (s >> 2)) * kDPitchV +
                                   (nrow + 16 * g + 4 * (s & 3)) * 2;
          const s16x4 lo = lds_read_tr4(p);
          const s16x4 hi = lds_read_tr4(p + 4 * kDPitchV);
          aop = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = mfma32(aop, bop[n], acc[m][n]);
      }
    }
  }

  // D layout (32x32): lane l, register j -> row 8 (j / 4) + 4 (l / 32) + j % 4 (output column
  // within the row block), column l % 32 (token within the column block).
  const int h = 2 * hp + nh;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int t = t0 + 64 * tq + 32 * n + (lane & 31);
    if (t >= L) continue;
    uint16_t* dst = a.out + (((size_t)b * a.max_len + t) * kHeads + h) * kDimC;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 o;
        o[0] = pack_bf16x2(acc[m][n][4 * q], acc[m][n][4 * q + 1]);
        o[1] = pack_bf16x2(acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]);
        *(u32x2*)(dst + 32 * m + 8 * q + 4 * (lane >> 5)) = o;
      }
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
  a.max_blocks = max_blocks;
  a.max_len = max_len;
  const dim3 grid(kHeads / 2, (max_len + kDTok - 1) / kDTok, batch);
  a.w = w_uk;
  a.out = k_out;
  hipLaunchKernelGGL(decompress_kernel<false>, grid, dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.w = w_uv;
  a.out = v_out;
  hipLaunchKernelGGL(decompress_kernel<true>, grid, dim3(512), 0, s, a);
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
  const uint16_t* k;        // [B, max_len, H, 128]
  const uint16_t* v;        // [B, max_len, H, 128]
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
  constexpr uint32_t kRowBytesKV = kHeads * kDimC * 2;   // 32 KiB between consecutive keys in K and V
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k) +
                               ((size_t)b * a.max_len * kHeads + h) * kDimC * 2;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v) +
                               ((size_t)b * a.max_len * kHeads + h) * kDimC * 2;
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
