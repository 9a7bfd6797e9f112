// Per-head projections of absorbed MLA on MFMA (gfx950):
//   absorb:  q_abs[t, h, :] = q_c[t, h, :] . W_UK[h]       ([T,128] x [128,512] per head)
//   up-proj: out[t, h, :]   = out_latent[t, h, :] . W_UV[h] ([T,512] x [512,128] per head)
// Both contract over the rows of a row-major per-head weight, so the weight's
// reduction dimension is strided in memory.  A workgroup stages a column slab
// of one head's weight in LDS once and feeds the MFMA B operand with
// transposing LDS reads (ds_read_b64_tr_b16), which deliver 4 consecutive
// rows of one column per lane.  For the small token counts of decode both
// kernels are bound by reading the 16 MiB weight from HBM.
#include "common.h"

namespace mla {

// C[t, h, n] = sum_k A[t, h, k] * B[h, k, n];  A [T, H, K], B [H, K, N], C [T, H, N], all bf16.
// Workgroup (blockIdx.x, blockIdx.y) = (column slab of NWG columns, head).  4 waves, each owning
// NWG/4 columns as 16-column MFMA blocks; tokens in tiles of 16 rows (v_mfma_f32_16x16x32_bf16).
template <int K, int N, int NWG>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void head_gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
                      int T) {
  static_assert(NWG % 64 == 0 && N % NWG == 0 && K % 32 == 0, "tile shape");
  // Row pitch padded by 32 B: the four rows one 16-lane group reads then start
  // 8 banks apart and cover all 32 LDS banks without conflict.
  constexpr int kPitch = NWG * 2 + 32;
  constexpr int kNB = NWG / 64;                 // 16-column blocks per wave
  constexpr int kChunksPerRowW = NWG * 2 / 16;  // 16-byte chunks per weight row
  __shared__ __attribute__((aligned(16))) unsigned char tile[K * kPitch];

  const int h = blockIdx.y;
  const int n0 = blockIdx.x * NWG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Stage the weight slab with every load in flight at once (a load-store loop
  // would pay one HBM round trip per iteration).
  constexpr int kChunks = K * kChunksPerRowW / 256;
  static_assert(K * kChunksPerRowW % 256 == 0, "slab must split evenly over the workgroup");
  const uint16_t* Bh = B + (size_t)h * K * N + n0;
  {
    u32x4 wv[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i, k = c / kChunksPerRowW, j = c % kChunksPerRowW;
      wv[i] = __builtin_nontemporal_load((const u32x4*)(Bh + (size_t)k * N + j * 8));
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i, k = c / kChunksPerRowW, j = c % kChunksPerRowW;
      *(u32x4*)(tile + k * kPitch + j * 16) = wv[i];
    }
  }

  // A operand of token tile m0 (rows m0 + lane % 16, columns 32ks + 8(lane / 16) .. +7),
  // all K/32 k-steps loaded together; rows past T read row 0 and are never stored.
  constexpr int kKS = K / 32;
  auto load_a = [&](int m0, s16x8 (&a)[kKS]) {
    const int arow = m0 + (lane & 15);
    const uint16_t* Ap = A + ((size_t)(arow < T ? arow : 0) * kHeads + h) * K + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) a[ks] = *(const s16x8*)(Ap + ks * 32);
  };
  s16x8 acur[kKS], anext[kKS];
  load_a(0, acur);
  __syncthreads();

  // Transposing-read source: lane s of 16-lane group g addresses row 8g + s/4
  // (rows +4 for the second read) and columns 4*(s%4) .. +3 of the block.
  const int g = lane >> 4, s = lane & 15;
  const unsigned char* tr_base = tile + (8 * g + (s >> 2)) * kPitch + ((s & 3) * 4) * 2;

  for (int m0 = 0; m0 < T; m0 += 16) {
    if (m0 + 16 < T) load_a(m0 + 16, anext);   // next tile's operand in flight during this tile
    f32x4 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const unsigned char* p = tr_base + ks * 32 * kPitch + (wave * kNB + nb) * 16 * 2;
        const s16x4 lo = lds_read_tr4(p);
        const s16x4 hi = lds_read_tr4(p + 4 * kPitch);
        const s16x8 b = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[nb] = mfma16(acur[ks], b, acc[nb]);
      }
    }
    // D layout of the 16x16 tile: lane l, register j -> row 4*(l/16) + j, column l % 16.
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int col = n0 + (wave * kNB + nb) * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = m0 + 4 * (lane >> 4) + j;
        if (row < T) C[((size_t)row * kHeads + h) * N + col] = f2bf(acc[nb][j]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) acur[ks] = anext[ks];
  }
}

hipError_t launch_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_abs, int tokens, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  constexpr int NWG = 128;
  hipLaunchKernelGGL((head_gemm_kernel<kDimC, kLatent, NWG>), dim3(kLatent / NWG, kHeads), dim3(256), 0, s, q_c,
                     w_uk, q_abs, tokens);
  return hipGetLastError();
}

hipError_t launch_up_proj(const uint16_t* ol, const uint16_t* w_uv, uint16_t* out, int tokens, hipStream_t s) {
  if (tokens <= 0) return hipSuccess;
  constexpr int NWG = 64;
  hipLaunchKernelGGL((head_gemm_kernel<kLatent, kDimC, NWG>), dim3(kDimC / NWG, kHeads), dim3(256), 0, s, ol, w_uv,
                     out, tokens);
  return hipGetLastError();
}

}  // namespace mla
