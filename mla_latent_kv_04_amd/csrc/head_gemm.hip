// Per-head projections of absorbed MLA on MFMA (gfx950):
//   absorb:  q_abs[t, h, :] = q_c[t, h, :] . W_UK[h]       ([T,128] x [128,512] per head)
//   up-proj: out[t, h, :]   = out_latent[t, h, :] . W_UV[h] ([T,512] x [512,128] per head)
// ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 4, path B; "DeepSeek的推理为什么比别人便宜一个数量级",
// leslieaibin.github.io, section "MLA", V = c . W_UV.)
// Both contract over the rows of a row-major per-head weight.  At decode sizes (tens of
// tokens) the 16 MiB weight is read once and each of its bytes feeds only T products, so
// both kernels are bound by the memory reads, which here are all in flight from the
// kernel's start: a workgroup issues the loads of its weight slab and of a block of up to
// 64 tokens of activations together, stages both in LDS, computes from LDS, and writes its
// outputs through an LDS stage as whole 16-byte row chunks.
#include "common.h"

namespace mla {

namespace {

constexpr int kTB = 64;        // tokens per activation block
constexpr int kXcds = 8;       // dies of the device: consecutive workgroup ids go to different dies

// C[t, h, n] = sum_k A[t, h, k] * B[h, k, n];  A [T, H, K], B [H, K, N], C [T, H, N], all bf16.
// Workgroup = (column slab of NWG columns, head): S = N / NWG slabs per head; the S slabs of a
// head get workgroup ids on one die, so they read that head's activations through one L2.
// 4 waves, wave w owning columns 16 kNB w .. +16 kNB of the slab as 16-column MFMA blocks
// (v_mfma_f32_16x16x32_bf16), tokens in tiles of 16.
template <int K, int N, int NWG>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void head_gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
                      int T) {
  static_assert(NWG % 64 == 0 && N % NWG == 0 && K % 32 == 0, "tile shape");
  constexpr int S = N / NWG;
  static_assert(kHeads % kXcds == 0, "heads spread evenly over the dies");
  // Weight slab rows [K][NWG], pitch padded by 32 B: the four rows one 16-lane group of a
  // transposing read addresses start 8 banks apart.  Activation rows [kTB][K], pitch padded by
  // 16 B: the 16 rows one 16-byte read addresses start 4 banks apart (64 banks covered once).
  constexpr int kPitchW = NWG * 2 + 32;
  constexpr int kPitchA = K * 2 + 16;
  constexpr int kNB = NWG / 64;                 // 16-column blocks per wave
  constexpr int kWChunks = K * NWG * 2 / 16 / 256;
  constexpr int kAChunks = kTB * K * 2 / 16 / 256;
  static_assert(K * NWG * 2 % (16 * 256) == 0 && kTB * K * 2 % (16 * 256) == 0, "even split over the workgroup");
  constexpr int kOutPitch = NWG * 2 + 16;       // output stage rows [kTB][NWG] bf16
  static_assert(kTB * kOutPitch <= kTB * kPitchA, "the output stage reuses the activation block");
  __shared__ __attribute__((aligned(16))) unsigned char wt[K * kPitchW];
  __shared__ __attribute__((aligned(16))) unsigned char at[kTB * kPitchA];

  // die-aware ids: workgroup id = die + 8 (slab + S group), head = die + 8 group
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, r = bid / kXcds;
  const int slab = r % S, h = xcd + kXcds * (r / S);
  const int n0 = slab * NWG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWRow = NWG * 2 / 16;           // 16-byte chunks per weight slab row
  constexpr int kARow = K * 2 / 16;             // 16-byte chunks per activation row
  const uint16_t* Bh = B + (size_t)h * K * N + n0;

  // A operand of tile m, k-step ks: row 16 m + lane % 16, columns 32 ks + 8 (lane / 16) .. +7.
  const uint32_t a_lane = (uint32_t)((lane & 15) * kPitchA + 16 * (lane >> 4));
  // Transposing-read source of the weight: lane s of 16-lane group g addresses row 8 g + s / 4
  // (rows +4 for the second read) and columns 4 (s % 4) .. +3 of a 16-column block.
  const int g = lane >> 4, s = lane & 15;
  const unsigned char* tr_base = wt + (8 * g + (s >> 2)) * kPitchW + ((s & 3) * 4) * 2;

  for (int t0 = 0; t0 < T; t0 += kTB) {
    const int nt = T - t0 < kTB ? T - t0 : kTB;
    {
      // every load of the block in flight at once (the weight slab only with the first block);
      // activation rows past T are not loaded and their outputs are never stored
      u32x4 wv[kWChunks], av[kAChunks];
      if (t0 == 0) {
#pragma unroll
        for (int i = 0; i < kWChunks; ++i) {
          const int c = tid + 256 * i, k = c / kWRow, j = c % kWRow;
          wv[i] = __builtin_nontemporal_load((const u32x4*)(Bh + (size_t)k * N + j * 8));
        }
      }
#pragma unroll
      for (int i = 0; i < kAChunks; ++i) {
        const int c = tid + 256 * i, t = c / kARow, j = c % kARow;
        if (t < nt) av[i] = *(const u32x4*)(A + ((size_t)(t0 + t) * kHeads + h) * K + j * 8);
      }
      if (t0 > 0) __syncthreads();   // the previous block's output stage has been read
      if (t0 == 0) {
#pragma unroll
        for (int i = 0; i < kWChunks; ++i) {
          const int c = tid + 256 * i, k = c / kWRow, j = c % kWRow;
          *(u32x4*)(wt + k * kPitchW + j * 16) = wv[i];
        }
      }
#pragma unroll
      for (int i = 0; i < kAChunks; ++i) {
        const int c = tid + 256 * i, t = c / kARow, j = c % kARow;
        *(u32x4*)(at + t * kPitchA + j * 16) = t < nt ? av[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();

    // four independent accumulation chains per column block (one per token tile)
    constexpr int kTiles = kTB / 16;
    f32x4 acc[kTiles][kNB];
#pragma unroll
    for (int m = 0; m < kTiles; ++m)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[m][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t abase = lds_addr(at) + a_lane;
#pragma unroll 4
    for (int ks = 0; ks < K / 32; ++ks) {
      s16x8 b[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const unsigned char* p = tr_base + ks * 32 * kPitchW + (wave * kNB + nb) * 16 * 2;
        const s16x4 lo = lds_read_tr4(p);
        const s16x4 hi = lds_read_tr4(p + 4 * kPitchW);
        b[nb] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int m = 0; m < kTiles; ++m) {
        const s16x8 a = lds_read_b128_at(abase + m * 16 * kPitchA + ks * 64);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[m][nb] = mfma16(a, b[nb], acc[m][nb]);
      }
    }
    __syncthreads();   // every wave is done reading the activation block: it becomes the output stage

    // D layout of a 16x16 tile: lane l, register j -> row 4 (l / 16) + j, column l % 16.
#pragma unroll
    for (int m = 0; m < kTiles; ++m)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int col = (wave * kNB + nb) * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * m + 4 * (lane >> 4) + j;
          *(uint16_t*)(at + row * kOutPitch + col * 2) = f2bf(acc[m][nb][j]);
        }
      }
    __syncthreads();
    constexpr int kORow = NWG * 2 / 16;         // 16-byte chunks per output row of the slab
#pragma unroll
    for (int i = 0; i < kTB * kORow / 256; ++i) {
      const int c = tid + 256 * i, t = c / kORow, j = c % kORow;
      if (t < nt)
        *(u32x4*)(C + ((size_t)(t0 + t) * kHeads + h) * N + n0 + j * 8) = *(const u32x4*)(at + t * kOutPitch + j * 16);
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_abs, int tokens, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  constexpr int NWG = 128;
  hipLaunchKernelGGL((head_gemm_kernel<kDimC, kLatent, NWG>), dim3(kLatent / NWG * kHeads), dim3(256), 0, s, q_c,
                     w_uk, q_abs, tokens);
  return hipGetLastError();
}

hipError_t launch_up_proj(const uint16_t* ol, const uint16_t* w_uv, uint16_t* out, int tokens, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  constexpr int NWG = 64;
  hipLaunchKernelGGL((head_gemm_kernel<kLatent, kDimC, NWG>), dim3(kDimC / NWG * kHeads), dim3(256), 0, s, ol, w_uv,
                     out, tokens);
  return hipGetLastError();
}

}  // namespace mla
