// Per-head projections of absorbed MLA on MFMA (gfx950):
//   absorb:  q_abs[t, h, :] = q_c[t, h, :] . W_UK[h]       ([T,128] x [128,512] per head)
//   up-proj: out[t, h, :]   = out_latent[t, h, :] . W_UV[h] ([T,512] x [512,128] per head)
// ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 4, path B; "DeepSeek的推理为什么比别人便宜一个数量级",
// leslieaibin.github.io, section "MLA", V = c . W_UV.)
// Both contract over the rows of a row-major per-head weight.  At decode sizes (tens of
// tokens) the 16 MiB weight is read once and each of its bytes feeds only T products, so
// both kernels are bound by the memory reads, which here are all in flight from the
// kernel's start: a workgroup issues the loads of its activation rows (straight into the
// registers that feed the MFMAs) and of its weight slab (staged in LDS) together, then
// computes, and writes its outputs through an LDS stage as whole 16-byte row chunks.
#include "common.h"

namespace mla {

namespace {

constexpr int kTB = 64;        // tokens per block: 16 per wave
constexpr int kXcds = 8;       // dies of the device: consecutive workgroup ids go to different dies

// C[t, h, n] = sum_k A[t, h, k] * B[h, k, n];  A [T, H, K], B [H, K, N], C [T, H, N], all bf16.
// Workgroup = (column slab of NWG columns, head): S = N / NWG slabs per head; the S slabs of a
// head get workgroup ids on one die, so they read that head's activations through one L2.
// Wave w owns tokens 16 w .. 16 w + 15 of each 64-token block and all NWG columns of the slab,
// as NWG / 16 blocks of v_mfma_f32_16x16x32_bf16 computing the transposed product
// C^T = B^T A^T: the weight (through transposing LDS reads) is the A operand, the wave's
// activation rows, held in registers, the B operand, and each lane's four results are four
// consecutive columns of one token (one 8-byte LDS write when staged).
template <int K, int N, int NWG>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void head_gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
                      int T) {
  static_assert(NWG % 16 == 0 && N % NWG == 0 && K % 32 == 0, "tile shape");
  static_assert(kHeads % kXcds == 0, "heads spread evenly over the dies");
  constexpr int S = N / NWG;
  constexpr int kNB = NWG / 16;                 // 16-column MFMA blocks per wave
  constexpr int kKS = K / 32;                   // k-steps
  // Weight slab rows [K][NWG], pitch padded by 32 B: the four rows one 16-lane group of a
  // transposing read addresses start 8 banks apart.
  constexpr int kPitchW = NWG * 2 + 32;
  constexpr int kWRow = NWG * 2 / 16;           // 16-byte chunks per weight slab row
  constexpr int kWChunks = K * kWRow / 256;
  static_assert(K * kWRow % 256 == 0, "the slab splits evenly over the workgroup");
  constexpr int kOutPitch = NWG * 2 + 16;       // output stage rows [kTB][NWG]
  constexpr int kORow = NWG * 2 / 16;           // 16-byte chunks per output row
  static_assert(kTB * kORow % 256 == 0, "the output block splits evenly over the workgroup");
  __shared__ __attribute__((aligned(16))) unsigned char wt[K * kPitchW];
  __shared__ __attribute__((aligned(16))) unsigned char st[kTB * kOutPitch];

  // die-aware ids: workgroup id = die + 8 (slab + S group), head = die + 8 group
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, r = bid / kXcds;
  const int slab = r % S, h = xcd + kXcds * (r / S);
  const int n0 = slab * NWG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* Bh = B + (size_t)h * K * N + n0;
  // Transposing-read source of the weight: lane s of 16-lane group g addresses row 8 g + s / 4
  // (rows +4 for the second read) and columns 4 (s % 4) .. +3 of a 16-column block, so lane l
  // receives rows 8 (l / 16) .. +7 of column l % 16: the A operand of W^T.
  const int g = lane >> 4, s = lane & 15;
  const unsigned char* tr_base = wt + (8 * g + (s >> 2)) * kPitchW + ((s & 3) * 4) * 2;

  for (int t0 = 0; t0 < T; t0 += kTB) {
    const int nt = T - t0 < kTB ? T - t0 : kTB;
    // B operand of k-step ks: token 16 wave + lane % 16, k = 32 ks + 8 (lane / 16) .. +7.
    // A token past T reads this block's first row instead; its results are never stored.
    const int row = 16 * wave + (lane & 15);
    const uint16_t* Ap = A + ((size_t)(t0 + (row < nt ? row : 0)) * kHeads + h) * K + 8 * (lane >> 4);
    s16x8 a[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) a[ks] = *(const s16x8*)(Ap + ks * 32);
    if (t0 == 0) {
      // the slab, with all its loads in flight at once (a load-store loop would pay one
      // memory round trip per iteration)
      u32x4 wv[kWChunks];
#pragma unroll
      for (int i = 0; i < kWChunks; ++i) {
        const int c = tid + 256 * i, k = c / kWRow, j = c % kWRow;
        wv[i] = __builtin_nontemporal_load((const u32x4*)(Bh + (size_t)k * N + j * 8));
      }
#pragma unroll
      for (int i = 0; i < kWChunks; ++i) {
        const int c = tid + 256 * i, k = c / kWRow, j = c % kWRow;
        *(u32x4*)(wt + k * kPitchW + j * 16) = wv[i];
      }
      __syncthreads();
    }

    f32x4 acc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const unsigned char* p = tr_base + ks * 32 * kPitchW + nb * 16 * 2;
        const s16x4 lo = lds_read_tr4(p);
        const s16x4 hi = lds_read_tr4(p + 4 * kPitchW);
        acc[nb] = mfma16(s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, a[ks], acc[nb]);
      }
    }
    // D layout of C^T: lane l, register j -> column 16 nb + 4 (l / 16) + j, token l % 16.
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int col = nb * 16 + 4 * (lane >> 4);
      *(u32x2*)(st + row * kOutPitch + col * 2) =
          u32x2{pack_bf16x2(acc[nb][0], acc[nb][1]), pack_bf16x2(acc[nb][2], acc[nb][3])};
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTB * kORow / 256; ++i) {
      const int c = tid + 256 * i, t = c / kORow, j = c % kORow;
      if (t < nt)
        *(u32x4*)(C + ((size_t)(t0 + t) * kHeads + h) * N + n0 + j * 8) = *(const u32x4*)(st + t * kOutPitch + j * 16);
    }
    __syncthreads();   // the stage is read before the next block's results land in it
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
