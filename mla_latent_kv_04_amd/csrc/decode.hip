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
// Workgroup: 256 threads = 4 waves, one per SIMD; wave w owns heads 32w..32w+31.
// Each page (64 tokens x 1152 B = 72 KiB) is copied HBM -> LDS with direct
// 16-byte loads (global_load_lds_dwordx4), double buffered (2 x 72 KiB of the
// 160 KiB LDS).  Per page and wave:
//   QK: 2 token blocks x 36 k-steps of v_mfma_f32_32x32x16_bf16, A = page rows
//       (ds_read_b128), B = the wave's 32 queries held in 144 VGPRs;
//   softmax: fp32, base 2, one head per lane pair (lanes l and l^32);
//   PV: 16 column blocks x 4 k-steps, A = P (bf16, straight from the score
//       registers), B = page columns via transposing LDS reads; O stays in 256
//       accumulator registers for the whole segment.
// LDS layout of a page: token-major rows of 72 sixteen-byte chunks, chunk c of
// token t stored at position c ^ swz(t); swz spreads both the row reads of QK
// (8 tokens, same chunk) and the 4-row transposing reads of PV over all banks.
#include "common.h"

namespace mla {

namespace {

constexpr int kThreads = 256;
constexpr int kLoadsPerThread = kChunksPerPage / kThreads;  // 18
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

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

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
// RoPE region [64 tokens][128 B] at offset 65536.  Inside each token row the
// 16-byte chunk c is stored at position c ^ swz(t & 7) (only the low 3 bits of
// the chunk index change), so 8 consecutive tokens reading one chunk, and the
// 4-token x 2-chunk blocks of a transposing read, hit 32 distinct banks.
constexpr int kRopeRegion = kPage * kLatent * 2;  // 65536

// Page copy HBM -> LDS: wave w copies the latent rows of tokens w, w+4, ...,
// w+60 (one 64-lane direct load per row, lane l = chunk position l) and the
// RoPE rows of tokens 16w .. 16w+15 (two loads; lane l -> token 8j + l/8,
// chunk position l%8).  The per-lane global offsets below are constant.
struct PageLoadOffsets {
  uint32_t lat_even;  // latent row offset for tokens t with t % 8 == w
  uint32_t lat_odd;   // ... t % 8 == w + 4
  uint32_t rope;      // RoPE offset inside a group of 8 tokens
};

__device__ __forceinline__ PageLoadOffsets page_load_offsets(int lane, int wave_u) {
  PageLoadOffsets o;
  o.lat_even = (uint32_t)((lane ^ swz(wave_u)) * 16);
  o.lat_odd = (uint32_t)((lane ^ swz(wave_u + 4)) * 16);
  const int tr = lane >> 3, pr = lane & 7;
  o.rope = (uint32_t)(tr * kRowBytes + kLatent * 2 + (pr ^ swz(tr)) * 16);
  return o;
}

// Rows at or past `valid` (only in a sequence's last page) are fetched from
// row 0 of the same page instead: they are masked out of the softmax, and
// loading finite data keeps 0 * V finite even when the unused rows of the
// cache hold NaN or Inf bit patterns.
__device__ __forceinline__ void issue_page(const unsigned char* __restrict__ src, unsigned char* buf,
                                           const PageLoadOffsets& off, int wave_u, int lane, int valid) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = wave_u + 4 * i;
    const uint32_t lo = (i & 1) ? off.lat_odd : off.lat_even;
    const int trow = t < valid ? t : 0;
    __builtin_amdgcn_global_load_lds((const void*)(src + trow * kRowBytes + lo), (MLA_LDS void*)(buf + t * 1024), 16,
                                     0, 0);
  }
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) {
    const int j = 2 * wave_u + j2;
    const uint32_t ro = (8 * j + (lane >> 3) < valid) ? 8 * j * kRowBytes + off.rope
                                                       : (uint32_t)(kLatent * 2 + (lane & 7) * 16);
    __builtin_amdgcn_global_load_lds((const void*)(src + ro), (MLA_LDS void*)(buf + kRopeRegion + 1024 * j), 16, 0, 0);
  }
}

// Softmax reference.  Each segment takes its per-head reference maximum from
// its first page and keeps it: P = 2^(s - m_ref) in log2 units, so the O
// accumulators are never rescaled.  A later score more than kHeadroom above
// the reference (P beyond 2^64, far outside real attention logits) makes the
// workgroup restart the segment with the larger reference, so the fp32
// accumulators cannot overflow.
constexpr float kHeadroom = 64.0f;

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kPageBytes];

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

  // Lane-constant parts of the LDS read addresses (byte offsets inside a page buffer).
  // QK A operand (token block tb, k-step ks = 4p + qq): token 32tb + l32, chunk 2ks + hi
  //   -> l32*1024 + 32*(qq ^ (sa >> 1)) + 16*(hi ^ (sa & 1)) + 128p + 32768tb.
  const int sa = swz(l32);
  int offA[4], offR[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int in_grp = 32 * (qq ^ (sa >> 1)) + 16 * (hi ^ (sa & 1));
    offA[qq] = l32 * 1024 + in_grp;
    offR[qq] = kRopeRegion + l32 * 128 + in_grp;
  }
  // PV B operand (transposing read), k-step kk (tokens 16kk..16kk+15), half r, column
  // block nb = 2p + qq: token 16kk + 8r + tb_b, chunk 4nb + cb, byte 8(lane & 1)
  //   -> tb_b*1024 + 64*(qq ^ (sb >> 2)) + 16*(cb ^ (sb & 3)) + 8(lane & 1) + 128p + (16kk + 8r)*1024.
  const int tb_b = 4 * hi + ((lane & 15) >> 2);
  const int sb = swz(tb_b);
  const int cb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int offB[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) offB[qq] = tb_b * 1024 + 64 * (qq ^ (sb >> 2)) + 16 * (cb ^ (sb & 3)) + 8 * (lane & 1);

  bool first_seg = true;
  int pos = start;
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

    f32x16 o[16];
    float m_ref = -INFINITY, l_run = 0.f;

    auto page_src = [&](int p) -> const unsigned char* {
      int64_t phys = bt_row[p];
      phys = phys < 0 ? 0 : (phys >= a.num_pages ? a.num_pages - 1 : phys);
      return (const unsigned char*)a.kv + phys * (int64_t)kPageBytes;
    };

    for (;;) {  // runs once unless a score leaves the headroom (then restarts with a larger reference)
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[nb][j] = 0.f;
      l_run = 0.f;
      bool restart = false;

      issue_page(page_src(p0), lds, ldo, wave_u, lane, n_vis - p0 * kPage);
      for (int p = p0; p < p1; ++p) {
        const unsigned char* cur = lds + ((p - p0) & 1) * kPageBytes;
        if (p + 1 < p1) {
          issue_page(page_src(p + 1), lds + ((p + 1 - p0) & 1) * kPageBytes, ldo, wave_u, lane,
                     n_vis - (p + 1) * kPage);
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerThread));
        } else {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        __syncthreads();

        // ---- scores S^T for the page: two 32-token blocks
        f32x16 s0, s1;
#pragma unroll
        for (int j = 0; j < 16; ++j) { s0[j] = 0.f; s1[j] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          const int qq = ks & 3;
          const unsigned char* pa0 = ks < 32 ? cur + offA[qq] + 128 * (ks >> 2) : cur + offR[qq];
          const s16x8 a0 = *(const s16x8*)(pa0);
          const s16x8 a1 = *(const s16x8*)(pa0 + (ks < 32 ? 32768 : 4096));
          s0 = mfma32(a0, q[ks], s0);
          s1 = mfma32(a1, q[ks], s1);
        }

        // ---- softmax weights (base 2).  Register j of block tb is token
        // 32tb + 8(j/4) + 4hi + (j%4) of the page, head l32 of this wave.
        const int tok0 = p * kPage;
        float x[32];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int t = 8 * (j >> 2) + 4 * hi + (j & 3);
          x[j] = (tok0 + t < n_vis) ? s0[j] * a.scale_log2 : -INFINITY;
          x[16 + j] = (tok0 + 32 + t < n_vis) ? s1[j] * a.scale_log2 : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 32; ++j) mx = fmaxf(mx, x[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (p == p0) {
          m_ref = fmaxf(m_ref, mx);
        } else if (__builtin_amdgcn_ballot_w64(mx > m_ref + kHeadroom) != 0) {
          m_ref = fmaxf(m_ref, mx);
          restart = true;
        }
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) { x[j] = __builtin_amdgcn_exp2f(x[j] - m_ref); rs += x[j]; }
        rs += __shfl_xor(rs, 32, 64);
        l_run += rs;

        // ---- P (bf16) as the MFMA A operand: k-step kk = 2tb + j2 uses registers
        // 8j2 .. 8j2+7 of block tb, i.e. tokens 16kk + 8(j/4) + 4hi + j%4.
        s16x8 pa[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[8 * kk + 2 * e], x[8 * kk + 2 * e + 1]);
          pa[kk] = __builtin_bit_cast(s16x8, w);
        }

        // ---- O += P . c_KV over the page (16 column blocks of 32).
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int nb = 0; nb < 16; ++nb) {
            const unsigned char* pb = cur + offB[nb & 1] + 128 * (nb >> 1) + 16 * kk * 1024;
            const s16x4 lo = lds_read_tr4(pb);
            const s16x4 hi4 = lds_read_tr4(pb + 8 * 1024);
            const s16x8 bv = s16x8{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            o[nb] = mfma32(pa[kk], bv, o[nb]);
          }
        }
        // Workgroup-uniform restart decision, taken at the barrier that also
        // frees this page buffer.
        const int any_restart = __syncthreads_or(restart ? 1 : 0);
        if (any_restart) {
          restart = true;
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // drain the prefetch before reusing the buffers
          __syncthreads();
          break;
        }
      }
      if (!restart) break;
    }

    // ---- write the segment's result
    const float inv_l = 1.f / l_run;
    const float lse2 = m_ref + __log2f(l_run);
    f32x16 il;
#pragma unroll
    for (int j = 0; j < 16; ++j) il[j] = __shfl(inv_l, 8 * (j >> 2) + 4 * hi + (j & 3), 64);
    if (slot < 0) {
      uint16_t* ob = a.out_latent + ((size_t)u * kHeads + wave_u * 32) * kLatent + l32;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) {
        const f32x16 v = o[nb] * il;
#pragma unroll
        for (int j = 0; j < 16; ++j) ob[(size_t)(8 * (j >> 2) + 4 * hi + (j & 3)) * kLatent + nb * 32] = f2bf(v[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (a.lse != nullptr && hi == 0) a.lse[(size_t)u * kHeads + head] = lse2 * kLn2;
    } else {
      float* ob = a.part_o + ((size_t)slot * kHeads + wave_u * 32) * kLatent + l32;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) {
        const f32x16 v = o[nb] * il;
#pragma unroll
        for (int j = 0; j < 16; ++j) ob[(size_t)(8 * (j >> 2) + 4 * hi + (j & 3)) * kLatent + nb * 32] = v[j];
        __builtin_amdgcn_sched_barrier(0);
      }
      if (hi == 0) a.part_lse[(size_t)slot * kHeads + head] = lse2;
    }
    pos = seg_end;
    first_seg = false;
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
