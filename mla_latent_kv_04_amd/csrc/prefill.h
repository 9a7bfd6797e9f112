// Host-side launch interface of the prefill (decompress branch) kernels (prefill.hip).
#pragma once

#include "common.h"

namespace mla {

// K, V [batch, H, max_len, 128] bf16 (each head's keys contiguous) for every cached token
// t < seqlens[b] (rows past a sequence's length are left as they were); max_len >= max_blocks * 64.
hipError_t launch_decompress(const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, const uint16_t* w_uk,
                             const uint16_t* w_uv, uint16_t* k_out, uint16_t* v_out, int batch, int max_blocks,
                             int max_len, int64_t num_pages, hipStream_t s);

// out [batch, M, H, 128] bf16 and lse [batch, M, H] fp32 (may be null) of the M-token chunk.
hipError_t launch_prefill_attention(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* k, const uint16_t* v,
                                    const uint16_t* kv, const int32_t* bt, const int32_t* seqlens, uint16_t* out,
                                    float* lse, int batch, int M, int max_blocks, int max_len, int64_t num_pages,
                                    float scale, hipStream_t s);

}  // namespace mla
