/*
 * Absorbed Multi-Head Latent Attention (MLA) decode over a paged latent cache,
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (stated in the pages' terms):
 *   - Each cached token stores one row of 576 bf16 values: the latent c_KV
 *     (512) followed by the decoupled RoPE key k_R (64), 1152 bytes per token
 *     per layer ("撕开 DeepSeek MLA 源码", sheratonhq.com, section 1).
 *   - Rows live in pages of 64 tokens; a block table maps a sequence's logical
 *     page j to a physical page (same page, section 3: page_size 64 in the
 *     mla_plugin JSON; section 5: the page-table base feeds 16-byte loads).
 *   - W_UK is folded into the query: q_abs = q_c . W_UK[h] (section 4, path B,
 *     contraction 'qhd,hdc->qhc').  Scores are (q_abs . c_KV + q_R . k_R) times
 *     1/sqrt(d_hc + d_R) = 1/sqrt(192) (section 4).  Softmax, then P . c_KV in
 *     latent space, then the up-projection through W_UV ("DeepSeek的推理为什么
 *     比别人便宜一个数量级", leslieaibin.github.io, section "MLA": V = c . W_UV).
 *
 * Fixed dimensions: num_heads H = 128, d_hc = 128, d_c = 512, d_R = 64,
 * page_size = 64 (the mla_config.h constants and mla_plugin JSON, sheratonhq.com
 * section 3).  Other values return MLA_ERR_UNSUPPORTED.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 *   - All tensor pointers are DEVICE pointers (HIP device memory of the current
 *     device); parameter structs and size outputs are HOST pointers.
 *   - The caller owns every buffer.  The library allocates nothing on these
 *     calls and keeps no pointer after returning.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *     enqueue work on it and return; nothing is synchronised.
 *   - Host-side checks run before any launch and return an error without
 *     touching the GPU: NULL pointers, unsupported dimensions, pointers not
 *     16-byte aligned (MLA_ERR_MISALIGNED; the pages report misaligned-address
 *     faults for 16-byte vector loads from an unaligned cache or page table,
 *     sheratonhq.com section 5), a workspace that is too small.  A failed
 *     launch returns MLA_ERR_HIP.  mla_last_error() then gives a thread-local
 *     message.  No C++ exception crosses this interface.
 *   - Values in device memory cannot be checked without a synchronisation and
 *     are preconditions: s_q <= seqlens[b] <= max_blocks_per_seq * 64, and the
 *     block-table entries of pages that cover tokens [0, seqlens[b]) lie in
 *     [0, num_pages).  Entries past those pages, and cache rows at or past
 *     seqlens[b], are never read.  Violations never make the kernels read
 *     outside kv_blocks or block_table (lengths are clamped to the table row and
 *     page ids to [0, num_pages)); the affected outputs are then unspecified.
 *     A sequence with fewer visible tokens than 1 gets out_latent = 0 and
 *     lse = -inf.
 */
#ifndef MLA_KV04_H
#define MLA_KV04_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, bad field */
  MLA_ERR_MISALIGNED = 2,  /* a tensor pointer is not 16-byte aligned */
  MLA_ERR_UNSUPPORTED = 3, /* a dimension other than the fixed ones above */
  MLA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  MLA_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} mla_status;

/* Decode-step description (host struct).  The pages' plugin JSON names the
 * same fields: num_heads, page_size, kv_cache_dtype bf16 (sheratonhq.com §3). */
typedef struct mla_decode_params {
  int32_t batch;              /* B >= 0 sequences */
  int32_t s_q;                /* new query tokens per sequence, 1 .. 256: 1 for
                                 a decode step, 2 for a two-token verify step,
                                 more for a short prefill chunk; query i of
                                 sequence b sees tokens t <= seqlens[b] - s_q + i
                                 (longer chunks: mla_prefill) */
  int32_t num_heads;          /* must be 128 */
  int32_t page_size;          /* must be 64 */
  int32_t max_blocks_per_seq; /* row length of block_table, >= 1 */
  int32_t num_splits;         /* 0: one decode workgroup per compute unit of the
                                 current device; > 0: exactly this many (the
                                 split plan changes, the result stays within
                                 rounding) */
  int64_t num_pages;          /* physical pages in kv_blocks, >= 1 */
  float scale;                /* softmax scale on (q_abs.c + q_R.k_R); > 0,
                                 1/sqrt(192) for the DeepSeek dimensions */
  int32_t reserved;           /* must be 0 */
} mla_decode_params;

/* q_abs[t, h, :] = q_c[t, h, :] . W_UK[h]  (bf16 in, fp32 accumulate, RNE to bf16).
 * q_c [tokens, H, 128], w_uk [H, 128, 512], q_abs [tokens, H, 512].  tokens >= 0
 * (0 is a no-op).  sheratonhq.com section 4, path B. */
mla_status mla_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_abs,
                        int32_t tokens, int32_t num_heads, void* stream);

/* Workspace bytes needed by mla_decode_paged (fused = 0) or mla_decode
 * (fused = 1) for these parameters: the split plan (tile and cost prefix sums
 * per (sequence, query) unit), the
 * normalised partial outputs and lse of sequences split across workgroups,
 * and, when fused, q_abs and out_latent.  The pages size the cache by its
 * 64-token pages of 1152-byte rows (sheratonhq.com sections 1 and 3) and say
 * nothing of a split over the sequence; the split-KV workspace is this
 * library's.  With p->num_splits == 0 the current device's compute-unit count
 * is queried (a HIP call).  Returns 0 when p is invalid (including
 * 2 * batch * s_q * max_blocks_per_seq > 2^31 - 1: the sums of 32-token tiles
 * over sequences are 32-bit) or the query fails. */
size_t mla_decode_workspace_size(const mla_decode_params* p, int32_t fused);

/* Paged decode in latent space (split-KV over pages, log-sum-exp merge):
 * scores (q_abs . c_KV + q_R . k_R) * scale over the rows the block table
 * names (sheratonhq.com section 4, path B; section 3, page_size 64; section 5,
 * the page table feeding 16-byte loads), softmax, and P . c_KV kept in latent
 * space for the later W_UV projection (leslieaibin.github.io section "MLA").
 *   q_abs       [B, s_q, H, 512] bf16   absorbed content query
 *   q_r         [B, s_q, H, 64]  bf16   RoPE query (already rotated)
 *   kv_blocks   [num_pages, 64, 576] bf16, row = c_KV[512] || k_R[64]
 *   block_table [B, max_blocks_per_seq] int32 physical page ids
 *   seqlens     [B] int32, tokens in the cache per sequence (including the
 *               s_q new ones)
 *   out_latent  [B, s_q, H, 512] bf16  softmax(scores) . c_KV
 *   lse         [B, s_q, H] fp32, natural log of the softmax denominator of the
 *               scaled scores; may be NULL
 *   workspace   device scratch of >= mla_decode_workspace_size(p, 0) bytes,
 *               16-byte aligned; contents need no initialisation.
 * Calls that share a workspace must be ordered on one stream. */
mla_status mla_decode_paged(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv_blocks,
                            const int32_t* block_table, const int32_t* seqlens, uint16_t* out_latent,
                            float* lse, const mla_decode_params* p, void* workspace,
                            size_t workspace_bytes, void* stream);

/* out[t, h, :] = out_latent[t, h, :] . W_UV[h]  (bf16 in, fp32 accumulate, RNE).
 * out_latent [tokens, H, 512], w_uv [H, 512, 128], out [tokens, H, 128].
 * leslieaibin.github.io section "MLA" (V = c . W_UV) with the token sum moved
 * before the projection. */
mla_status mla_up_proj(const uint16_t* out_latent, const uint16_t* w_uv, uint16_t* out,
                       int32_t tokens, int32_t num_heads, void* stream);

/* Fused decode step: absorb -> paged decode -> merge -> up-projection; the
 * same function as expanding K = c . W_UK[h] and V = c . W_UV[h] per head and
 * running plain attention (sheratonhq.com section 4, paths A and B;
 * leslieaibin.github.io section "MLA").
 *   q_c [B, s_q, H, 128], q_r [B, s_q, H, 64], w_uk [H, 128, 512],
 *   w_uv [H, 512, 128], out [B, s_q, H, 128] bf16, lse as above (may be NULL).
 * workspace >= mla_decode_workspace_size(p, 1) bytes (holds q_abs and
 * out_latent as well). */
mla_status mla_decode(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk,
                      const uint16_t* w_uv, const uint16_t* kv_blocks, const int32_t* block_table,
                      const int32_t* seqlens, uint16_t* out, float* lse, const mla_decode_params* p,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Test export of the page gather: dense[b, t, :] = kv_blocks[block_table[b][t / 64], t % 64, :]
 * for t < seqlens[b]; rows t in [seqlens[b], max_blocks_per_seq * 64) are zero
 * (the paging of sheratonhq.com section 3, page_size 64, and the page-table
 * lookup of section 5).  dense [B, max_blocks_per_seq * 64, 576] bf16. */
mla_status mla_gather_kv(const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens,
                         uint16_t* dense, const mla_decode_params* p, void* stream);

/* ---------------------------------------------------------------- cache append
 *
 * Each decode step first appends its new tokens to the cache
 * ("DeepSeek的推理为什么比别人便宜一个数量级", leslieaibin.github.io, the decode
 * loop of the closing summary): the hidden state x is compressed to the latent
 * c = x . W_DKV, d -> d_c = 512 (same page, section "MLA", first step; d = 7168
 * for DeepSeek, kHiddenDim in sheratonhq.com section 3), and the 64-value key
 * k_R, shared by all heads (sheratonhq.com section 1), is rotated with RoPE
 * computed from an fp32 precomputed table with fp32 multiply-add
 * (sheratonhq.com section 4, verification paragraph; rope_compute_dtype fp32
 * in the section 3 plugin JSON).  Where the pages are silent this library
 * takes k_R = RoPE(x . W_KR) from the same x, passes W_DKV and W_KR as one
 * matrix W_A = [W_DKV | W_KR] [d, 576], applies no normalisation to c, and
 * rotates the interleaved pairs (2i, 2i + 1), i = 0..31.
 *
 * New token i (0 <= i < s_q) of sequence b has position p = seqlens[b] - s_q + i
 * (seqlens counts the new tokens, as for the decode) and its row goes to row
 * p % 64 of page block_table[b][p / 64]. */

typedef struct mla_append_params {
  int32_t batch;              /* B >= 0 sequences */
  int32_t s_q;                /* new tokens per sequence, >= 1 */
  int32_t d_model;            /* hidden size d: a multiple of 256, <= 65536 (7168 for DeepSeek) */
  int32_t page_size;          /* must be 64 */
  int32_t max_blocks_per_seq; /* row length of block_table, >= 1 */
  int32_t max_pos;            /* rows of rope_table, >= 1 */
  int64_t num_pages;          /* physical pages in kv_blocks, >= 1 */
  int32_t num_heads;          /* heads of q_r when mla_append_kv is given one: 1..4096 (128 for DeepSeek) */
  int32_t reserved;           /* must be 0 */
} mla_append_params;

/* Workspace bytes needed by mla_append_kv and mla_append_kv_mxfp8: the fp32
 * partial sums of the split projection, splits x tokens x 576 x 4 bytes (2 MiB
 * for 64 tokens and d = 7168; with the projection not split, tokens x 576 x 4,
 * which only the MXFP8 cache uses).  Returns 0 when p is invalid.  No HIP call. */
size_t mla_append_workspace_size(const mla_append_params* p);

/* Writes the new tokens' cache rows (and, optionally, rotates their RoPE query):
 * two kernel launches (one when the token count alone fills the device).
 *   x           [B, s_q, d] bf16 hidden states of the new tokens
 *   w_a         [d, 576] bf16, columns 0..511 = W_DKV, 512..575 = W_KR
 *   rope_table  [max_pos, 64] fp32, row p = cos(p theta_0..31) then
 *               sin(p theta_0..31) (mla_rope_table writes one; any table of
 *               this layout works, e.g. a rescaled one)
 *   block_table [B, max_blocks_per_seq] int32, seqlens [B] int32 (as for decode)
 *   kv_blocks   [num_pages, 64, 576] bf16, updated in place: only the rows of
 *               the new tokens are written, c in 0..511 and k_R in 512..575,
 *               each the fp32 result rounded once to bf16 (nearest, even)
 *   q_r         [B, s_q, num_heads, 64] bf16 or NULL: when given, rotated in
 *               place exactly as mla_rope_q does (same positions and table)
 *   workspace   >= mla_append_workspace_size(p) bytes, 16-byte aligned, no
 *               initialisation needed; calls sharing it must be ordered on one
 *               stream.
 * Accumulation is fp32 in a fixed order: repeated calls give identical bits.
 * A token whose position is negative, >= max_pos or past the block-table row,
 * or whose page id is outside [0, num_pages), is not written (device values are
 * preconditions; nothing outside the buffers is touched).  Tokens of one call
 * must not share a slot. */
mla_status mla_append_kv(const uint16_t* x, const uint16_t* w_a, const float* rope_table,
                         const int32_t* block_table, const int32_t* seqlens, uint16_t* kv_blocks, uint16_t* q_r,
                         const mla_append_params* p, void* workspace, size_t workspace_bytes, void* stream);

/* Rotates the RoPE query in place with the key's rotation at the same position:
 * q_r [B, s_q, num_heads, 64] bf16, token i of sequence b at p = seqlens[b] - s_q + i,
 * every head turned by the angles of table row p (fp32 multiply-add, one RNE
 * rounding to bf16).  Tokens with p < 0 or p >= max_pos are left unchanged.
 * 1 <= num_heads <= 4096.  sheratonhq.com section 4 (fp32 RoPE). */
mla_status mla_rope_q(uint16_t* q_r, const float* rope_table, const int32_t* seqlens, int32_t batch, int32_t s_q,
                      int32_t num_heads, int32_t max_pos, void* stream);

/* Fills rope_table [max_pos, 64] fp32: entry (p, i) = cos(p theta_i) and entry
 * (p, 32 + i) = sin(p theta_i), theta_i = base^(-2i/64), with the angle, cosine
 * and sine evaluated in double precision and each entry rounded once to fp32
 * (an fp32 angle would carry a phase error at long positions, the failure
 * sheratonhq.com section 4 attributes to low-precision RoPE).  base > 1
 * (10000 is the usual value). */
mla_status mla_rope_table(float* rope_table, int32_t max_pos, double base, void* stream);

/* ---------------------------------------------------------------- prefill
 *
 * A chunk of s_q new tokens per sequence whose rows are already in the cache
 * (seqlens counts them; query i sees the first seqlens[b] - s_q + i + 1 tokens).
 * Short chunks are cheapest with matrix absorption, long ones with the keys and
 * values expanded per head ("decompress"): K_h = c . W_UK[h]^T and
 * V_h = c . W_UV[h] for every cached token ("DeepSeek的推理为什么比别人便宜一个数量级",
 * leslieaibin.github.io, section "MLA"), then plain attention with the 192-wide
 * score q_c . K_h + q_R . k_R.  The pages switch branches at
 * kPrefillThresh = 256 query rows (sheratonhq.com section 3; section 6 reports
 * the gain).  Both branches compute the same function. */

typedef struct mla_prefill_params {
  int32_t batch;              /* B >= 0 sequences */
  int32_t s_q;                /* chunk length M >= 1 (at most 256 on the absorbed branch) */
  int32_t num_heads;          /* must be 128 */
  int32_t page_size;          /* must be 64 */
  int32_t max_blocks_per_seq; /* row length of block_table, >= 1 */
  int32_t mode;               /* 0: decompress when s_q >= threshold, else absorb;
                                 1: always absorb; 2: always decompress */
  int64_t num_pages;          /* physical pages in kv_blocks, >= 1 */
  float scale;                /* 1/sqrt(192) for the DeepSeek dimensions */
  int32_t threshold;          /* 0: 256 (the pages' kPrefillThresh); else 1 .. 257 */
  int32_t reserved;           /* must be 0 */
} mla_prefill_params;

/* Workspace bytes of mla_prefill: on the decompress branch the expanded K and V,
 * each [batch, 128 heads, max_blocks_per_seq * 64, 128] bf16 (32 KiB per token slot),
 * K at offset 0 and V at the size of one rounded up to 256 bytes; rows at or past
 * seqlens[b] are left as they were.  On the absorbed branch what mla_decode
 * needs.  0 when p is invalid. */
size_t mla_prefill_workspace_size(const mla_prefill_params* p);

/* Attention output of the chunk's queries.
 *   q_c [B, s_q, 128, 128], q_r [B, s_q, 128, 64] (rotated), w_uk [128, 128, 512],
 *   w_uv [128, 512, 128], kv_blocks / block_table / seqlens as for decode,
 *   out [B, s_q, 128, 128] bf16, lse [B, s_q, 128] fp32 (may be NULL).
 * Decompress branch: bf16 K and V (fp32 accumulation), fp32 scores and online
 * softmax, fp32 accumulation of P . V with P rounded to bf16.  Absorbed branch:
 * exactly mla_decode.  Workspace contents need no initialisation; calls sharing
 * it must be ordered on one stream.  Preconditions on device values as for
 * decode; a query with no visible token gets out = 0, lse = -inf. */
mla_status mla_prefill(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk, const uint16_t* w_uv,
                       const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens, uint16_t* out,
                       float* lse, const mla_prefill_params* p, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---------------------------------------------------------------- MXFP8 latent cache
 *
 * The pages keep the latent cache at four bits (NVFP4) and gather it with
 * 16-byte vector loads at byte offsets of half the element index, which needs a
 * 16-byte aligned page-table base ("撕开 DeepSeek MLA 源码", sheratonhq.com,
 * section 5); they give neither the element code nor the scale layout.  This
 * library's low-precision cache is the CDNA4-native analogue, OCP MXFP8:
 *   - latent codes: OCP E4M3 (bias 7, no infinities, largest 448, 0x7F/0xFF NaN);
 *   - blocks of 32 consecutive latent values share one E8M0 scale byte s,
 *     value 2^(s - 127); a block's scale is the smallest power of two 2^X with
 *     max |v| <= 448 * 2^X (no element saturates), X in [-127, 127], s = 0 for an
 *     all-zero block; codes are v / 2^X rounded to nearest, ties to even;
 *   - k_R stays bf16.
 * Row of one token, MLA_MXFP8_ROW_BYTES = 656 bytes (every part 16-byte aligned):
 *   bytes [0, 512) codes, [512, 528) the 16 scale bytes, [528, 656) k_R as 64 bf16.
 * A page is 64 rows (41 984 bytes, against 73 728 for bf16: 41/72); paging and
 * block tables are the bf16 cache's.  kv_mxfp8 pointers are 16-byte aligned.
 * Dequantisation (code value times 2^(s - 127)) is exact in bf16 for normal
 * results, so the decode over an MXFP8 cache is the bf16 decode over the
 * dequantised cache, with the same accumulation and the same outputs contract. */
#define MLA_MXFP8_ROW_BYTES 656

/* kv_mxfp8 [num_pages, 64, 656] from kv_blocks [num_pages, 64, 576] bf16, every
 * row (finite inputs; the result for a row holding NaN or Inf is unspecified).
 * num_pages >= 0 (0 is a no-op).  Deterministic: a pure function of the row. */
mla_status mla_quantize_kv_mxfp8(const uint16_t* kv_blocks, uint8_t* kv_mxfp8, int64_t num_pages, void* stream);

/* mla_decode_paged over an MXFP8 cache: same arguments, parameters, workspace
 * (mla_decode_workspace_size(p, 0)) and outputs; kv_mxfp8 [num_pages, 64, 656]. */
mla_status mla_decode_paged_mxfp8(const uint16_t* q_abs, const uint16_t* q_r, const uint8_t* kv_mxfp8,
                                  const int32_t* block_table, const int32_t* seqlens, uint16_t* out_latent,
                                  float* lse, const mla_decode_params* p, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* mla_decode (fused step) over an MXFP8 cache: same arguments and workspace
 * (mla_decode_workspace_size(p, 1)). */
mla_status mla_decode_mxfp8(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk,
                            const uint16_t* w_uv, const uint8_t* kv_mxfp8, const int32_t* block_table,
                            const int32_t* seqlens, uint16_t* out, float* lse, const mla_decode_params* p,
                            void* workspace, size_t workspace_bytes, void* stream);

/* mla_append_kv into an MXFP8 cache: the same rows (fp32 sums in the same fixed
 * order, k_R rotated in fp32 and rounded once to bf16), with the latent of each
 * row quantised from its fp32 values as above.  Always two kernel launches;
 * workspace >= mla_append_workspace_size(p) bytes. */
mla_status mla_append_kv_mxfp8(const uint16_t* x, const uint16_t* w_a, const float* rope_table,
                               const int32_t* block_table, const int32_t* seqlens, uint8_t* kv_mxfp8,
                               uint16_t* q_r, const mla_append_params* p, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Benchmark timing hook.  After mla_profile_enable(1), every mla_decode_paged
 * and mla_decode call (either cache format) on any stream records HIP events around each of its
 * kernels (up to 65536 calls; the library creates those events once and keeps
 * them).  mla_profile_collect waits for the recorded calls and, for kernel k of
 * [absorb, plan, decode, combine, up-projection], writes to launches[k] the
 * number of calls that launched it and to ms[k] the summed milliseconds of
 * those launches (host arrays of 5; a paged call launches no absorb or
 * up-projection, and with at most 64 sequence-query units no plan kernel, so
 * those stay 0), the number of calls to *calls, and clears the record.
 * mla_profile_enable(0) stops recording.  Off by default; not for code under
 * graph capture. */
mla_status mla_profile_enable(int32_t enable);
mla_status mla_profile_collect(double* ms, int32_t* launches, int32_t* calls);

/* The same hook for mla_append_kv and mla_append_kv_mxfp8 calls (recorded while mla_profile_enable(1) is
 * in force, up to 65536 calls): writes the summed milliseconds of [projection
 * kernel, partial-sum kernel] to ms[0..1] (host array of 2; the second is 0 for
 * calls whose projection is not split) and the number of calls to *calls, and
 * clears that record. */
mla_status mla_profile_collect_append(double* ms, int32_t* calls);

/* The same for decompress-branch mla_prefill calls: ms[0] = decompress kernels,
 * ms[1] = attention kernel. */
mla_status mla_profile_collect_prefill(double* ms, int32_t* calls);

/* mla_decode_paged without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments (less the workspace), kernels and results as
 * mla_decode_paged on the same parameters; the workspace is a device array built
 * into the library, one copy per device, looked up on the first call on each device
 * and held until the process ends: 68 MiB, enough for at most 256 split-KV
 * workgroups (num_splits, or the device's compute units when 0) and 65 536
 * (sequence, query) units.  Larger parameters return MLA_ERR_UNSUPPORTED.  Allocates
 * nothing.  All calls on one device share that device's array: calls that may overlap
 * on one device (different streams, different threads) race and must be ordered by
 * the caller.  bf16 cache only. */
mla_status mla_decode_paged_noalloc(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv_blocks,
                                    const int32_t* block_table, const int32_t* seqlens, uint16_t* out_latent,
                                    float* lse, const mla_decode_params* p, void* stream);

/* Decode workgroups (split-KV ranges) that mla_decode_paged, mla_decode and
 * mla_stream_pages launch for these parameters: p->num_splits when > 0, else the
 * current device's compute-unit count (a HIP call).  0 when p is invalid. */
int32_t mla_decode_num_workgroups(const mla_decode_params* p);

/* Measurement of the page stream alone.  The pages call decode memory-bound: its
 * arithmetic intensity sits far below the roofline ridge, so HBM bandwidth sets its
 * speed (sheratonhq.com section 1).  This call reads exactly the cache rows
 * mla_decode_paged reads for the same arguments, with the same work split, the same
 * 16-byte direct loads into the same LDS ring and the same per-tile workgroup
 * barrier, and does no arithmetic on them: its time is the stream-read ceiling of the
 * decode on the device.  So that every load is observable, thread t of workgroup g
 * writes to sums[g * 256 + t] the 32-bit sum (mod 2^32) of dword t of the first row
 * of every 32-token tile the workgroup streams (the tile's first token's latent,
 * 256 dwords); the sum of all of sums[] is therefore the sum, over every tile of
 * every (sequence, query) unit, of that row's latent dwords.
 *   kv_blocks, block_table, seqlens, p: as for mla_decode_paged (p->scale unused)
 *   sums       [mla_decode_num_workgroups(p) * 256] uint32, 4-byte aligned
 *   workspace  >= mla_decode_workspace_size(p, 0) bytes (the split plan) */
mla_status mla_stream_pages(const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens,
                            uint32_t* sums, const mla_decode_params* p, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Number of compute units of the current device (a HIP call). */
mla_status mla_device_cu_count(int32_t* num_cus);

/* Static text for a status code; never NULL. */
const char* mla_status_string(mla_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_KV04_H */
