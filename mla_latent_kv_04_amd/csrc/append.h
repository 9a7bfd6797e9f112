// Host-side launch interface of the cache-append kernels (append.hip).
#pragma once

#include "common.h"

namespace mla {

// Split of the cache-append projection over the hidden dimension (a pure function
// of the token count and hidden size, so workspace sizing and launch agree).
struct AppendPlan {
  int cols;             // output columns per projection workgroup (32 or 64)
  int splits;           // partial sums per output value
  int slabs_per_split;  // 32 KiB slabs of W_A per split
  int units;            // workgroups of the projection kernel that do work
  size_t part_bytes;    // fp32 partials [splits, tokens, 576] (0 if splits == 1 and the cache is bf16)
};

AppendPlan plan_append(int tokens, int d_model, bool mxfp8);

// Exactly one of kv (bf16 cache) and kv8 (MXFP8 cache) is non-null.
hipError_t launch_append(const uint16_t* x, const uint16_t* w_a, const float* table, const int32_t* bt,
                         const int32_t* seqlens, uint16_t* kv, unsigned char* kv8, uint16_t* q_r, int heads,
                         unsigned char* ws, int batch, int s_q, int d_model, int max_blocks, int64_t num_pages,
                         int max_pos, hipStream_t s, hipEvent_t ev_proj_done = nullptr);
hipError_t launch_quantize_mxfp8(const uint16_t* kv, unsigned char* kv8, int64_t num_pages, hipStream_t s);
hipError_t launch_rope_q(uint16_t* q_r, const float* table, const int32_t* seqlens, int batch, int s_q, int heads,
                         int max_pos, hipStream_t s);
hipError_t launch_rope_table(float* table, int max_pos, double base, hipStream_t s);

}  // namespace mla
