// Internal definitions shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// DeepSeek MLA dimensions (the mla_config.h constants of "撕开 DeepSeek MLA 源码",
// sheratonhq.com section 3).
constexpr int kHeads = 128;
constexpr int kDimC = 128;             // d_hc, content head dim
constexpr int kLatent = 512;           // d_c
constexpr int kRope = 64;              // d_R
constexpr int kRow = kLatent + kRope;  // 576 elements per cached token
constexpr int kRowBytes = kRow * 2;    // 1152
constexpr int kPage = 64;              // tokens per page
constexpr int kPageBytes = kPage * kRowBytes;     // 73728
constexpr int kChunksPerRow = kRowBytes / 16;      // 72 sixteen-byte chunks
constexpr int kChunksPerPage = kPage * kChunksPerRow;  // 4608

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and leaves the export and LDS/scalar counters unconstrained
// (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14]).
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return ((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Two fp32 -> packed pair of bf16 (low half = a).
// Round-to-nearest-even of two floats into one register (a in the low half); a
// two-element vector conversion maps onto the single packed conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ f32x16 mfma32(const s16x8& a, const s16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const s16x8& a, const s16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Transposing LDS read of 4 bf16.  Within each group of 16 lanes, lane i
// receives element (i % 4) of the 8-byte rows addressed by lanes 4e + i/4,
// e = 0..3: the 16 lanes address a 4 x 16 block (row e = lanes 4e..4e+3, each
// giving 4 consecutive columns) and lane i gets column i.
__device__ __forceinline__ s16x4 lds_read_tr4(const void* lds_byte_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(lds_byte_ptr));
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(MLA_LDS const void*)p;
}

// The same reads at a 32-bit LDS byte address.
__device__ __forceinline__ s16x4 lds_read_tr4_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(uintptr_t)addr);
}
__device__ __forceinline__ s16x8 lds_read_b128_at(uint32_t addr) {
  return *(MLA_LDS const s16x8*)(uintptr_t)addr;
}

// Fewest 32-token tiles a decode workgroup takes when the caller lets the library size
// the split (num_splits = 0); an explicit num_splits splits the tiles evenly.  A
// workgroup pays a fixed cost per range (its queries, its partial output and that
// partial's merge) that only a few tiles amortise: measured on MI355X at batch 1 and
// 2048 tokens (64 tiles), decode plus merge takes 30 us with 4 tiles per workgroup
// (16 workgroups), 32 us with 2 and 39-40 us with 1; larger workloads, whose even split
// already gives 8 or more tiles per compute unit, are unaffected.
constexpr int kAutoMinChunk = 4;
// The segment-aware split (decode_kernel's work_range): a segment start counts as this
// many tiles on the cost line, for ranges of at least kCostSplitMin tiles.
constexpr int kSegCost = 6;
constexpr int kCostSplitMin = 48;
// Most workgroups a decode split uses (num_splits is at most 2^16).
constexpr int kMaxSplits = 1 << 16;

// Host-side launch helpers (defined in the kernel translation units).
struct DecodePlanView {
  int32_t* cum;       // [2 units + 3] the split plan: tile and cost-line prefix sums, segment cost
  uint16_t* part_o;   // [2 * wgs, 128, 512] normalised partial outputs, bf16
  float* part_lse;    // [2 * wgs, 128] log2-domain lse of the partials
};

hipError_t launch_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_abs, int tokens,
                           hipStream_t s);
hipError_t launch_up_proj(const uint16_t* ol, const uint16_t* w_uv, uint16_t* out, int tokens, hipStream_t s);
// Exactly one of kv (bf16 cache) and kv8 (MXFP8 cache) is non-null.
hipError_t launch_decode(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv, const unsigned char* kv8,
                         const int32_t* bt, const int32_t* seqlens, uint16_t* out_latent, float* lse, int batch,
                         int s_q, int max_blocks, int64_t num_pages, float scale, int wgs, int min_chunk,
                         const DecodePlanView& plan, hipStream_t s, hipEvent_t ev_plan_done = nullptr,
                         hipEvent_t ev_decode_done = nullptr);
// Whether a decode of this many (sequence, query) units launches the separate
// prefix-sum kernel (smaller ones compute the sums inside every decode workgroup).
bool decode_launches_plan(int units);
// The decode's page stream alone (same split, loads and LDS ring, no arithmetic); sums
// [wgs * 256] receive per-thread sums of the tiles' first-row dwords.  cum: [units + 1].
hipError_t launch_stream(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint32_t* sums, int batch,
                         int s_q, int max_blocks, int64_t num_pages, int wgs, int min_chunk, int32_t* cum,
                         hipStream_t s);
// Size of the device array that backs the allocation-free paged decode: a workspace for
// up to 256 split-KV workgroups (2 x 256 partial outputs of 128 x 512 bf16 = 64 MiB, their
// lse) and up to 65 536 (sequence, query) units of prefix sums.
constexpr size_t kNoAllocScratchBytes = (size_t)68 << 20;
// That array's address on the current device (looked up once per device).
hipError_t noalloc_scratch(unsigned char** ptr);
hipError_t launch_gather(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint16_t* dense, int batch,
                         int max_blocks, int64_t num_pages, hipStream_t s);

}  // namespace mla
