// Cache append of absorbed MLA on gfx950: the step that writes each new
// token's cache row before the decode reads it, and the matching rotation of
// the RoPE query.
//
//   row   = x . W_A,  W_A = [W_DKV | W_KR]  [d, 576]   (latent c and the
//           pre-rotation key, "DeepSeek的推理为什么比别人便宜一个数量级",
//           leslieaibin.github.io, section "MLA": c = x . W_DKV)
//   k_R   = RoPE(row[512:576]) with an fp32 table and fp32 multiply-add
//           ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 4 verification
//           paragraph; rope_compute_dtype fp32 in the section 3 plugin JSON)
//   cache[block_table[b][p / 64]][p % 64] = bf16(c || k_R),  p = seqlens[b] - s_q + i
//
// For decode-sized token counts the projection is bound by reading the 8 MiB
// weight: the contraction is split over the hidden dimension so that about one
// workgroup per compute unit streams its own 256 x 64 slab of W_A, and a second
// kernel sums the fp32 partials in a fixed order (bitwise reproducible), rotates
// the key in fp32, rounds once to bf16 and writes the row into its page.
#include "append.h"

namespace mla {

namespace {

constexpr int kSlabRows = 256;                 // hidden-state rows of W_A per pass
constexpr int kCols = 64;                      // output columns per workgroup
constexpr int kColBlocks = kRow / kCols;       // 9
constexpr int kTokens = 64;                    // tokens per workgroup: 4 waves x 16
constexpr int kXcds = 8;                       // MI355X: 8 accelerator dies, each with its own L2
constexpr int kTargetWgs = 256;                // one workgroup per compute unit

// Partial projection of one (token group, K split, column block) unit:
//   part[split][t][n0 .. n0 + 63] = sum over the split's hidden rows k of x[t][k] W_A[k][n].
// Units are numbered token group, then split, then column block, and handed out
// so that each die (workgroups go round-robin over the 8 dies) takes a
// contiguous run: the 9 column blocks that reuse one x slice then share an L2.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void append_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ part,
                        int T, int d, int splits, int slabs_per_split, int units, int per_die) {
  constexpr int kPitch = kCols * 2 + 32;       // 160 B: four rows a 16-lane group reads start 8 banks apart
  constexpr int kCPR = kCols * 2 / 16;         // 8 sixteen-byte chunks per weight row
  constexpr int kChunks = kSlabRows * kCPR / 256;
  constexpr int kKS = kSlabRows / 32;          // k-steps of v_mfma_f32_16x16x32_bf16 per slab
  __shared__ __attribute__((aligned(16))) unsigned char tile[kSlabRows * kPitch];

  const int q = (blockIdx.x % kXcds) * per_die + blockIdx.x / kXcds;
  if (q >= units) return;                      // whole workgroup: no barrier is skipped by half of it
  const int cb = q % kColBlocks;
  const int split = (q / kColBlocks) % splits;
  const int grp = q / (kColBlocks * splits);
  const int n0 = cb * kCols, m0 = grp * kTokens;
  const int k_begin = split * slabs_per_split * kSlabRows;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // A operand (x): row m0 + 16 wave + lane % 16, columns 32 ks + 8 (lane / 16) .. +7 of
  // the slab; rows past T read row 0 and are never stored.
  const int arow = m0 + 16 * wave + (lane & 15);
  const uint16_t* Ap = x + (size_t)(arow < T ? arow : 0) * d + k_begin + 8 * (lane >> 4);
  // Weight chunk i of this thread: slab row tid / 8 + 32 i, columns n0 + 8 (tid % 8) .. +7.
  const uint16_t* Wp = w + (size_t)(k_begin + tid / kCPR) * kRow + n0 + 8 * (tid % kCPR);
  unsigned char* wdst = tile + (tid / kCPR) * kPitch + (tid % kCPR) * 16;

  u32x4 wv[kChunks];
  s16x8 a[kKS];
  auto load_slab = [&](int s) {
    const size_t k0 = (size_t)s * kSlabRows;
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      wv[i] = __builtin_nontemporal_load((const u32x4*)(Wp + (k0 + 32 * i) * kRow));
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) a[ks] = *(const s16x8*)(Ap + k0 + 32 * ks);
  };

  // Transposing-read source: lane s of 16-lane group g addresses slab row 8g + s/4
  // (rows +4 for the second read) and columns 4 (s % 4) .. +3 of a 16-column block.
  const int g = lane >> 4, sl = lane & 15;
  const unsigned char* tr_base = tile + (8 * g + (sl >> 2)) * kPitch + (sl & 3) * 8;

  f32x4 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_slab(0);
  for (int s = 0; s < slabs_per_split; ++s) {
    if (s > 0) __syncthreads();                // every wave is done reading the previous slab
#pragma unroll
    for (int i = 0; i < kChunks; ++i) *(u32x4*)(wdst + 32 * i * kPitch) = wv[i];
    s16x8 acur[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) acur[ks] = a[ks];
    if (s + 1 < slabs_per_split) load_slab(s + 1);   // next slab in flight during this one
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const unsigned char* p = tr_base + ks * 32 * kPitch + nb * 32;
        const s16x4 lo = lds_read_tr4(p);
        const s16x4 hi = lds_read_tr4(p + 4 * kPitch);
        const s16x8 b = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[nb] = mfma16(acur[ks], b, acc[nb]);
      }
    }
  }

  // D layout of a 16x16 tile: lane l, register j -> row 4 (l / 16) + j, column l % 16.
  float* P = part + (size_t)split * T * kRow;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int col = n0 + 16 * nb + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + 16 * wave + 4 * (lane >> 4) + j;
      if (row < T) P[(size_t)row * kRow + col] = acc[nb][j];
    }
  }
}

// One workgroup per new token: sum the split partials in split order, rotate the
// last 64 values as 32 interleaved pairs with the position's fp32 table row,
// round to bf16 and write the row into its page.  Thread j owns columns 4j .. 4j + 3.
__global__ __attribute__((amdgpu_flat_work_group_size(192, 192)))
void append_finalize_kernel(const float* __restrict__ part, int splits, int T, const float* __restrict__ table,
                            int max_pos, const int32_t* __restrict__ bt, const int32_t* __restrict__ seqlens, int s_q,
                            int max_blocks, int64_t num_pages, uint16_t* __restrict__ kv) {
  const int t = blockIdx.x;
  const int b = t / s_q, i = t - b * s_q;
  const int p = seqlens[b] - s_q + i;
  if (p < 0 || p >= max_pos || (p >> 6) >= max_blocks) return;
  const int page = bt[(size_t)b * max_blocks + (p >> 6)];
  if (page < 0 || page >= num_pages) return;
  const int j = threadIdx.x;
  if (j >= kRow / 4) return;

  const float* src = part + (size_t)t * kRow + 4 * j;
  const size_t stride = (size_t)T * kRow;
  f32x4 acc = *(const f32x4*)src;
#pragma unroll 4
  for (int s = 1; s < splits; ++s) acc += *(const f32x4*)(src + s * stride);

  if (j >= kLatent / 4) {
    // columns 512 + 4r .. +3 hold pairs 2r and 2r + 1 of the key
    const int r = j - kLatent / 4;
    const float* row = table + (size_t)p * kRope;
    const float c0 = row[2 * r], c1 = row[2 * r + 1];
    const float s0 = row[kRope / 2 + 2 * r], s1 = row[kRope / 2 + 2 * r + 1];
    const f32x4 v = acc;
    acc[0] = v[0] * c0 - v[1] * s0;
    acc[1] = v[0] * s0 + v[1] * c0;
    acc[2] = v[2] * c1 - v[3] * s1;
    acc[3] = v[2] * s1 + v[3] * c1;
  }
  u32x2 out;
  out[0] = pack_bf16x2(acc[0], acc[1]);
  out[1] = pack_bf16x2(acc[2], acc[3]);
  *(u32x2*)(kv + ((size_t)page * kPage + (p & (kPage - 1))) * kRow + 4 * j) = out;
}

// q_r [T, H, 64] rotated in place.  One workgroup per token; thread tid always owns
// pairs 4 (tid % 8) .. +3 of a head (16 bytes), so it loads its table entries once.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope_q_kernel(uint16_t* __restrict__ q_r, const float* __restrict__ table, const int32_t* __restrict__ seqlens,
                   int s_q, int heads, int max_pos) {
  const int t = blockIdx.x;
  const int b = t / s_q, i = t - b * s_q;
  const int p = seqlens[b] - s_q + i;
  if (p < 0 || p >= max_pos) return;
  const int qd = threadIdx.x & 7;
  const f32x4 c = *(const f32x4*)(table + (size_t)p * kRope + 4 * qd);
  const f32x4 sn = *(const f32x4*)(table + (size_t)p * kRope + kRope / 2 + 4 * qd);
  uint16_t* base = q_r + (size_t)t * heads * kRope;
  for (int ch = threadIdx.x; ch < heads * (kRope / 8); ch += 256) {
    u32x4 v = *(const u32x4*)(base + 8 * ch);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf2f((uint16_t)(v[k] & 0xFFFFu)), bb = bf2f((uint16_t)(v[k] >> 16));
      v[k] = pack_bf16x2(a * c[k] - bb * sn[k], a * sn[k] + bb * c[k]);
    }
    *(u32x4*)(base + 8 * ch) = v;
  }
}

// table[p] = [cos(p theta_0) .. cos(p theta_31) | sin(p theta_0) .. sin(p theta_31)],
// theta_i = base^(-2i/64): angles, cosines and sines in fp64, each entry rounded once to fp32.
__global__ void rope_table_kernel(float* __restrict__ table, int max_pos, double base) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= max_pos * (kRope / 2)) return;
  const int p = idx / (kRope / 2), i = idx % (kRope / 2);
  const double theta = pow(base, -2.0 * i / kRope);
  const double ang = (double)p * theta;
  table[(size_t)p * kRope + i] = (float)cos(ang);
  table[(size_t)p * kRope + kRope / 2 + i] = (float)sin(ang);
}

}  // namespace

AppendPlan plan_append(int tokens, int d_model) {
  AppendPlan pl{};
  const int slabs = d_model / kSlabRows;
  const int groups = (tokens + kTokens - 1) / kTokens;
  const int base_units = kColBlocks * groups;
  int splits = slabs;
  for (int s = 1; s <= slabs; ++s) {
    if (slabs % s == 0 && (int64_t)base_units * s >= kTargetWgs) {
      splits = s;
      break;
    }
  }
  pl.splits = splits;
  pl.slabs_per_split = slabs / splits;
  pl.units = base_units * splits;
  pl.part_bytes = (size_t)splits * tokens * kRow * sizeof(float);
  return pl;
}

hipError_t launch_append(const uint16_t* x, const uint16_t* w_a, const float* table, const int32_t* bt,
                         const int32_t* seqlens, uint16_t* kv, float* part, int batch, int s_q, int d_model,
                         int max_blocks, int64_t num_pages, int max_pos, hipStream_t s) {
  const int T = batch * s_q;
  if (T <= 0) return hipSuccess;
  const AppendPlan pl = plan_append(T, d_model);
  const int per_die = (pl.units + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(append_gemm_kernel, dim3(per_die * kXcds), dim3(256), 0, s, x, w_a, part, T, d_model, pl.splits,
                     pl.slabs_per_split, pl.units, per_die);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_finalize_kernel, dim3(T), dim3(192), 0, s, part, pl.splits, T, table, max_pos, bt, seqlens,
                     s_q, max_blocks, num_pages, kv);
  return hipGetLastError();
}

hipError_t launch_rope_q(uint16_t* q_r, const float* table, const int32_t* seqlens, int batch, int s_q, int heads,
                         int max_pos, hipStream_t s) {
  const int T = batch * s_q;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_q_kernel, dim3(T), dim3(256), 0, s, q_r, table, seqlens, s_q, heads, max_pos);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* table, int max_pos, double base, hipStream_t s) {
  if (max_pos <= 0) return hipSuccess;
  const int n = max_pos * (kRope / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, max_pos, base);
  return hipGetLastError();
}

}  // namespace mla
