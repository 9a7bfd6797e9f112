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
// workgroup per compute unit streams its own 32 KiB slab of W_A and writes an
// fp32 partial; while its weight loads are in flight each workgroup also rotates
// a share of the RoPE query of the same tokens.  A second kernel sums the
// partials in split order (bitwise reproducible), rotates the key in fp32,
// rounds once to bf16 and writes the rows into their pages.  (Summing in the
// last-arriving workgroup of each column block instead was measured slower:
// the arrival ticket and the device-scope release/acquire it needs cost more
// than the second launch.)  When the token count alone fills the device the
// contraction is not split and the first kernel writes the rows itself.
#include "append.h"
#include "mxfp8.h"

namespace mla {

namespace {

constexpr int kSlabBytes = 32768;              // W_A bytes each workgroup stages per pass
constexpr int kTokens = 64;                    // tokens per workgroup: 4 waves x 16
constexpr int kXcds = 8;                       // MI355X: 8 accelerator dies, each with its own L2
constexpr int kTargetWgs = 256;                // one workgroup per compute unit
constexpr int kQEarly = 2;                     // q_R chunks per thread rotated under the weight loads

struct AppendArgs {
  const uint16_t* x;        // [T, d]
  const uint16_t* w;        // [d, 576]
  const float* table;       // [max_pos, 64]
  const int32_t* bt;        // [B, max_blocks]
  const int32_t* seqlens;   // [B]
  uint16_t* kv;             // [num_pages, 64, 576] (bf16 cache) or null
  unsigned char* kv8;       // [num_pages, 64, 656] (MXFP8 cache) or null
  uint16_t* q_r;            // [T, heads, 64] or null
  float* part;              // [splits, T, 576] when splits > 1
  int64_t num_pages;
  int T, d, s_q, max_blocks, max_pos, heads;
  int splits, slabs_per_split, units, per_die;
  int direct;               // the projection kernel writes the rows itself (bf16 cache, one split)
};

// Position of token t (p = seqlens[b] - s_q + i) and its cache row index
// page * 64 + p % 64, or -1 when that slot or its table row does not exist.
__device__ __forceinline__ int64_t slot_of(const AppendArgs& a, int t, int* pos) {
  const int b = t / a.s_q, i = t - b * a.s_q;
  const int p = a.seqlens[b] - a.s_q + i;
  *pos = p;
  if (p < 0 || p >= a.max_pos || (p >> 6) >= a.max_blocks) return -1;
  const int page = a.bt[(size_t)b * a.max_blocks + (p >> 6)];
  if (page < 0 || page >= a.num_pages) return -1;
  return (int64_t)page * kPage + (p & (kPage - 1));
}

// Rotates the four pairs held in a 16-byte chunk of bf16 (pair k = halves of word k).
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 v, const f32x4& c, const f32x4& sn) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = bf2f((uint16_t)(v[k] & 0xFFFFu)), x1 = bf2f((uint16_t)(v[k] >> 16));
    v[k] = pack_bf16x2(x0 * c[k] - x1 * sn[k], x0 * sn[k] + x1 * c[k]);
  }
  return v;
}

// One 16-byte chunk of q_R: chunk idx covers pairs 4 (idx % 8) .. +3 of head
// (idx / 8) % heads of token idx / (8 heads).
struct QChunk {
  u32x4 v;
  f32x4 c, sn;
  uint16_t* dst;
};

__device__ __forceinline__ bool load_q_chunk(const AppendArgs& a, size_t idx, QChunk& qc) {
  const size_t per_token = (size_t)a.heads * (kRope / 8);
  if (idx >= (size_t)a.T * per_token) return false;
  const int t = (int)(idx / per_token);
  const int b = t / a.s_q, i = t - b * a.s_q;
  const int p = a.seqlens[b] - a.s_q + i;
  if (p < 0 || p >= a.max_pos) return false;
  const int qd = (int)(idx & 7);
  qc.dst = a.q_r + idx * 8;
  qc.v = *(const u32x4*)qc.dst;
  qc.c = *(const f32x4*)(a.table + (size_t)p * kRope + 4 * qd);
  qc.sn = *(const f32x4*)(a.table + (size_t)p * kRope + kRope / 2 + 4 * qd);
  return true;
}

// One (token group, K split, column block) unit per workgroup:
//   partial[t][n0 .. n0 + kCols - 1] = sum over the split's hidden rows k of x[t][k] W_A[k][n].
// The workgroup stages a 32 KiB slab of W_A (kR rows of kCols columns) and the
// matching x slab (64 tokens x kR hidden values, loaded a whole 1 KiB row segment
// per instruction) in LDS; the MFMA B operand comes from transposing LDS reads,
// the A operand from plain 16-byte LDS reads, each wave owning 16 tokens.
// Narrow column blocks mean fewer K splits for the same slab size, hence fewer
// fp32 partials, at the price of re-reading x (from L2) once per column block.
// Units are numbered token group, then split, then column block, and handed out
// so that each die (workgroups go round-robin over the 8 dies) takes a
// contiguous run: column blocks that reuse one x slice, and that share the
// 128-byte lines of W_A rows, then share an L2.
template <int kCols>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void append_kernel(AppendArgs a) {
  static_assert(kCols == 32 || kCols == 64, "column block");
  constexpr int kR = kSlabBytes / (kCols * 2);           // slab rows: 512, 256
  // Row pitch: the four rows one 16-lane group reads in a transposing read must
  // start 8 LDS banks apart (pitch = 8 or 24 banks mod 32) to cover all 32 banks.
  constexpr int kPitch = kCols == 32 ? 96 : 160;
  // x slab rows (one token each) padded by 16 bytes: the 8 rows one group of 8 lanes
  // reads with a 16-byte read then start 4 banks apart.
  constexpr int kXPitch = kR * 2 + 16;
  constexpr int kXCPR = kR * 2 / 16;                      // 16-byte chunks per x slab row
  constexpr int kXChunks = kTokens * kXCPR / 256;         // per thread: 16, 8
  constexpr int kCPR = kCols * 2 / 16;                    // 16-byte chunks per weight row
  constexpr int kChunks = kR * kCPR / 256;                // 8 per thread
  constexpr int kNB = kCols / 16;                         // 16-column MFMA blocks per wave
  constexpr int kColBlocks = kRow / kCols;
  __shared__ __attribute__((aligned(16))) unsigned char tile[kR * kPitch];
  __shared__ __attribute__((aligned(16))) unsigned char xs[kTokens * kXPitch];

  const int q = (blockIdx.x % kXcds) * a.per_die + blockIdx.x / kXcds;
  if (q >= a.units) return;                    // whole workgroup: no barrier is skipped by half of it
  const int cb = q % kColBlocks;
  const int split = (q / kColBlocks) % a.splits;
  const int grp = q / (kColBlocks * a.splits);
  const int n0 = cb * kCols, m0 = grp * kTokens;
  const int k_begin = split * a.slabs_per_split * kR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T;

  // q_R chunks of this thread (issued first: waiting for them leaves the W_A loads in flight).
  const size_t q_stride = (size_t)a.units * 256;
  QChunk qe[kQEarly];
  bool qok[kQEarly];
#pragma unroll
  for (int k = 0; k < kQEarly; ++k)
    qok[k] = a.q_r != nullptr && load_q_chunk(a, (size_t)q * 256 + tid + k * q_stride, qe[k]);

  // x chunk i of this thread: slab row (token) tid / kXCPR + (256 / kXCPR) i, 16 bytes at
  // hidden offset 8 (tid % kXCPR); tokens past T read token 0 and are never stored.
  constexpr int kXRowStep = 256 / kXCPR;
  const uint16_t* Xp[kXChunks];
#pragma unroll
  for (int i = 0; i < kXChunks; ++i) {
    const int row = m0 + tid / kXCPR + kXRowStep * i;
    Xp[i] = a.x + (size_t)(row < T ? row : 0) * a.d + k_begin + 8 * (tid % kXCPR);
  }
  unsigned char* xdst = xs + (tid / kXCPR) * kXPitch + (tid % kXCPR) * 16;
  // Weight chunk i of this thread: slab row tid / kCPR + (256 / kCPR) i, 16 bytes at column
  // n0 + 8 (tid % kCPR).
  constexpr int kRowStep = 256 / kCPR;
  const uint16_t* Wp = a.w + (size_t)(k_begin + tid / kCPR) * kRow + n0 + 8 * (tid % kCPR);
  unsigned char* wdst = tile + (tid / kCPR) * kPitch + (tid % kCPR) * 16;

  u32x4 wv[kChunks], xv[kXChunks];
  auto load_slab = [&](int s) {
    const size_t k0 = (size_t)s * kR;
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      wv[i] = __builtin_nontemporal_load((const u32x4*)(Wp + (k0 + kRowStep * i) * kRow));
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) xv[i] = *(const u32x4*)(Xp[i] + k0);
  };
  load_slab(0);

#pragma unroll
  for (int k = 0; k < kQEarly; ++k)
    if (qok[k]) *(u32x4*)qe[k].dst = rotate_chunk(qe[k].v, qe[k].c, qe[k].sn);

  // Transposing-read source: lane s of 16-lane group g addresses slab row 8g + s/4
  // (rows +4 for the second read) and columns 4 (s % 4) .. +3 of a 16-column block.
  const int g = lane >> 4, sl = lane & 15;
  const unsigned char* tr_base = tile + (8 * g + (sl >> 2)) * kPitch + (sl & 3) * 8;
  // A operand: token 16 wave + lane % 16, hidden offsets 32 ks + 8 (lane / 16) .. +7.
  const unsigned char* a_base = xs + (16 * wave + (lane & 15)) * kXPitch + 16 * (lane >> 4);

  f32x4 acc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = 0; s < a.slabs_per_split; ++s) {
    if (s > 0) __syncthreads();                // every wave is done reading the previous slab
#pragma unroll
    for (int i = 0; i < kChunks; ++i) *(u32x4*)(wdst + kRowStep * i * kPitch) = wv[i];
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) *(u32x4*)(xdst + kXRowStep * i * kXPitch) = xv[i];
    if (s + 1 < a.slabs_per_split) load_slab(s + 1);   // next slab in flight during this one
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kR / 32; ++ks) {
      const s16x8 av = *(const s16x8*)(a_base + ks * 64);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const unsigned char* p = tr_base + ks * 32 * kPitch + nb * 32;
        const s16x4 lo = lds_read_tr4(p);
        const s16x4 hi = lds_read_tr4(p + 4 * kPitch);
        const s16x8 b = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[nb] = mfma16(av, b, acc[nb]);
      }
    }
  }

  // D layout of a 16x16 tile: lane l, register j -> row 4 (l / 16) + j, column l % 16.
  if (a.direct) {
    // The sum is complete: rotate key pairs (columns 2i, 2i + 1 sit in lanes l, l ^ 1) and
    // store each pair of bf16 from its even lane.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + 16 * wave + 4 * (lane >> 4) + j;
      int p = 0;
      const int64_t dst = row < T ? slot_of(a, row, &p) : -1;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int col = n0 + 16 * nb + (lane & 15);
        float v = acc[nb][j];
        const float other = __shfl_xor(v, 1);
        if (col >= kLatent && dst >= 0) {
          const int pr = (col - kLatent) >> 1;
          const float c = a.table[(size_t)p * kRope + pr], sn = a.table[(size_t)p * kRope + kRope / 2 + pr];
          v = (lane & 1) ? other * sn + v * c : v * c - other * sn;
        }
        const float partner = __shfl_xor(v, 1);
        if (dst >= 0 && !(lane & 1)) *(uint32_t*)(a.kv + dst * kRow + col) = pack_bf16x2(v, partner);
      }
    }
  } else {
    float* P = a.part + (size_t)split * T * kRow;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int col = n0 + 16 * nb + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = m0 + 16 * wave + 4 * (lane >> 4) + j;
        if (row < T) P[(size_t)row * kRow + col] = acc[nb][j];
      }
    }
  }

  // q_R chunks beyond the first kQEarly per thread (only when tokens outnumber the units' threads).
  if (a.q_r != nullptr) {
    for (size_t idx = (size_t)q * 256 + tid + kQEarly * q_stride; idx < (size_t)T * a.heads * (kRope / 8);
         idx += q_stride) {
      QChunk qc;
      if (load_q_chunk(a, idx, qc)) *(u32x4*)qc.dst = rotate_chunk(qc.v, qc.c, qc.sn);
    }
  }
}

// One wave per (new token, 64-column block): lane l sums the split partials of
// column 64 cb + l in split order, all loads of up to kBatch splits issued before
// the first addition; in the last block (the key) lanes 2i and 2i + 1 hold pair
// i, exchange values and rotate it with the position's fp32 table row; then the
// value is rounded to bf16 and each pair is stored from its even lane.
template <bool kF8>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void append_finalize_kernel(AppendArgs a) {
  constexpr int kBatch = 16;
  const int t = blockIdx.x, cb = blockIdx.y, lane = threadIdx.x;
  int p = 0;
  const int64_t dst = slot_of(a, t, &p);
  if (dst < 0) return;
  const int col = 64 * cb + lane;
  const float* src = a.part + (size_t)t * kRow + col;
  const size_t stride = (size_t)a.T * kRow;
  float v[kBatch];
#pragma unroll
  for (int sp = 0; sp < kBatch; ++sp)
    if (sp < a.splits) v[sp] = src[sp * stride];
  float acc = v[0];
#pragma unroll
  for (int sp = 1; sp < kBatch; ++sp)
    if (sp < a.splits) acc += v[sp];
  for (int sp = kBatch; sp < a.splits; ++sp) acc += src[sp * stride];

  float other = __shfl_xor(acc, 1);
  if (col >= kLatent) {
    const int pr = (col - kLatent) >> 1;
    const float c = a.table[(size_t)p * kRope + pr], sn = a.table[(size_t)p * kRope + kRope / 2 + pr];
    acc = (lane & 1) ? other * sn + acc * c : acc * c - other * sn;
    other = __shfl_xor(acc, 1);
  }
  if constexpr (!kF8) {
    if (!(lane & 1)) *(uint32_t*)(a.kv + dst * kRow + col) = pack_bf16x2(acc, other);
  } else {
    unsigned char* row = a.kv8 + dst * kF8RowBytes;
    if (col >= kLatent) {
      if (!(lane & 1)) *(uint32_t*)(row + kF8Rope + 2 * (col - kLatent)) = pack_bf16x2(acc, other);
      return;
    }
    // MXFP8 latent: each half-wave is one block of 32 values; its largest magnitude
    // sets the scale, then pairs are coded in the even lanes and four codes are
    // stored as one dword from every fourth lane.
    float amax = fabsf(acc);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const int sb = mx_scale_byte(amax);
    const float x = ldexpf(acc, 127 - sb), xo = ldexpf(other, 127 - sb);
    const uint32_t pk = e4m3_pack2<false>(0u, x, xo);          // even lanes: (this, next) codes
    const uint32_t pk2 = __shfl_xor(pk, 2);
    if ((lane & 3) == 0) *(uint32_t*)(row + kF8Codes + col) = (pk & 0xFFFFu) | (pk2 << 16);
    if ((lane & 31) == 0) row[kF8Scales + col / 32] = (unsigned char)sb;
  }
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

// bf16 cache rows -> MXFP8 cache rows.  One wave per row: lane l holds latent values
// 8l .. 8l+7 (block l / 4), so a block's four lanes find its largest magnitude with
// two exchanges; every lane stores its 8 codes (the wave writes the 512-byte code
// run), the first lane of each block its scale byte, lanes 0..7 the 128 bytes of k_R.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void quantize_mxfp8_kernel(const uint16_t* __restrict__ kv, unsigned char* __restrict__ kv8, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* src = kv + row * kRow;
  unsigned char* dst = kv8 + row * kF8RowBytes;
  const u32x4 v = *(const u32x4*)(src + 8 * lane);
  float f[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf2f((uint16_t)(v[k] & 0xFFFFu));
    f[2 * k + 1] = bf2f((uint16_t)(v[k] >> 16));
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int sb = mx_scale_byte(amax);
  uint32_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    c[h] = e4m3_pack2<false>(0u, ldexpf(f[4 * h], 127 - sb), ldexpf(f[4 * h + 1], 127 - sb));
    c[h] = e4m3_pack2<true>(c[h], ldexpf(f[4 * h + 2], 127 - sb), ldexpf(f[4 * h + 3], 127 - sb));
  }
  *(u32x2*)(dst + kF8Codes + 8 * lane) = u32x2{c[0], c[1]};
  if ((lane & 3) == 0) dst[kF8Scales + lane / 4] = (unsigned char)sb;
  if (lane < 8) *(u32x4*)(dst + kF8Rope + 16 * lane) = *(const u32x4*)(src + kLatent + 8 * lane);
}

}  // namespace

AppendPlan plan_append(int tokens, int d_model, bool mxfp8) {
  AppendPlan pl{};
  const int groups = (tokens + kTokens - 1) / kTokens;
  // One token group (decode): 32-column blocks halve the fp32 partials of 64-column
  // ones; more groups (prefill-sized): 64-column blocks read x fewer times.
  const int cols = groups == 1 && d_model % 512 == 0 ? 32 : 64;
  const int rows = kSlabBytes / (cols * 2);
  const int slabs = d_model / rows;
  const int base_units = (kRow / cols) * groups;
  int splits = slabs;
  for (int s = 1; s <= slabs; ++s) {
    if (slabs % s == 0 && (int64_t)base_units * s >= kTargetWgs) {
      splits = s;
      break;
    }
  }
  pl.cols = cols;
  pl.splits = splits;
  pl.slabs_per_split = slabs / splits;
  pl.units = base_units * splits;
  // the MXFP8 cache always takes the partial-sum kernel (it holds the block quantiser)
  pl.part_bytes = splits > 1 || mxfp8 ? (size_t)splits * tokens * kRow * sizeof(float) : 0;
  return pl;
}

hipError_t launch_append(const uint16_t* x, const uint16_t* w_a, const float* table, const int32_t* bt,
                         const int32_t* seqlens, uint16_t* kv, unsigned char* kv8, uint16_t* q_r, int heads,
                         unsigned char* ws, int batch, int s_q, int d_model, int max_blocks, int64_t num_pages,
                         int max_pos, hipStream_t s, hipEvent_t ev_proj_done) {
  const int T = batch * s_q;
  if (T <= 0) return ev_proj_done != nullptr ? hipEventRecord(ev_proj_done, s) : hipSuccess;
  const bool f8 = kv8 != nullptr;
  const AppendPlan pl = plan_append(T, d_model, f8);
  AppendArgs a;
  a.x = x;
  a.w = w_a;
  a.table = table;
  a.bt = bt;
  a.seqlens = seqlens;
  a.kv = kv;
  a.kv8 = kv8;
  a.q_r = q_r;
  a.part = reinterpret_cast<float*>(ws);
  a.num_pages = num_pages;
  a.T = T;
  a.d = d_model;
  a.s_q = s_q;
  a.max_blocks = max_blocks;
  a.max_pos = max_pos;
  a.heads = q_r != nullptr ? heads : 0;
  a.splits = pl.splits;
  a.slabs_per_split = pl.slabs_per_split;
  a.units = pl.units;
  a.per_die = (pl.units + kXcds - 1) / kXcds;
  a.direct = pl.splits == 1 && !f8;
  const dim3 grid(a.per_die * kXcds);
  if (pl.cols == 32)
    hipLaunchKernelGGL(append_kernel<32>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev_proj_done != nullptr) e = hipEventRecord(ev_proj_done, s);
  if (e != hipSuccess || a.direct) return e;
  if (f8)
    hipLaunchKernelGGL(append_finalize_kernel<true>, dim3(T, kRow / 64), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(append_finalize_kernel<false>, dim3(T, kRow / 64), dim3(64), 0, s, a);
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

hipError_t launch_quantize_mxfp8(const uint16_t* kv, unsigned char* kv8, int64_t num_pages, hipStream_t s) {
  const int64_t rows = num_pages * kPage;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, kv, kv8, rows);
  return hipGetLastError();
}

}  // namespace mla
