// C-ABI entry points: host-side validation, workspace layout, kernel launches.
// Nothing here allocates device memory or synchronises; every call enqueues on
// the caller's stream and returns.
#include <stdarg.h>
#include <string.h>

#include <array>
#include <cstdio>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "mla.h"
#include "common.h"
#include "append.h"
#include "prefill.h"

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mla_status ok() {
  g_last_error.clear();
  return MLA_OK;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Query tokens per sequence the absorbed decode accepts: beyond the prefill
// threshold the decompress branch (mla_prefill) is the one to use.
constexpr int kMaxDecodeSq = 256;
constexpr int kPrefillThreshold = 256;

mla_status check_params(const mla_decode_params* p) {
  if (p == nullptr) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->s_q < 1 || p->s_q > kMaxDecodeSq)
    return fail(MLA_ERR_UNSUPPORTED, "s_q %d (supported: 1 .. %d)", p->s_q, kMaxDecodeSq);
  if (p->num_heads != mla::kHeads) return fail(MLA_ERR_UNSUPPORTED, "num_heads %d (supported: 128)", p->num_heads);
  if (p->page_size != mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size %d (supported: 64)", p->page_size);
  if (p->max_blocks_per_seq < 1) return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", p->max_blocks_per_seq);
  if (p->max_blocks_per_seq > (1 << 24)) return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  if (p->num_splits < 0 || p->num_splits > mla::kMaxSplits) return fail(MLA_ERR_INVALID_ARG, "num_splits %d", p->num_splits);
  if (p->num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages %lld < 1", (long long)p->num_pages);
  if (!(p->scale > 0.f) || p->scale > 1e30f) return fail(MLA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (p->reserved != 0) return fail(MLA_ERR_INVALID_ARG, "reserved must be 0");
  if ((int64_t)p->batch * p->s_q > (1 << 24)) return fail(MLA_ERR_INVALID_ARG, "batch * s_q too large");
  // The kernels sum 32-token tiles per (sequence, query) unit in 32-bit integers, on a
  // cost line where each unit also counts kSegCost tiles; a unit has at most 2 *
  // max_blocks_per_seq tiles, and a range start may pass the line's end by one range
  // (at most kMaxSplits), so this bounds every prefix sum and range position.
  const int64_t line = (int64_t)p->batch * p->s_q * ((int64_t)p->max_blocks_per_seq * 2 + mla::kSegCost);
  if (line + mla::kMaxSplits > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARG,
                "batch * s_q * (max_blocks_per_seq * 2 + %d) + %d = %lld exceeds 2^31 - 1 (tile prefix sums)",
                mla::kSegCost, mla::kMaxSplits, (long long)(line + mla::kMaxSplits));
  return MLA_OK;
}

mla_status resolve_wgs(const mla_decode_params* p, int* wgs) {
  if (p->num_splits > 0) {
    *wgs = p->num_splits;
    return MLA_OK;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
  if (cus <= 0) return fail(MLA_ERR_HIP, "device reports %d compute units", cus);
  *wgs = cus;
  return MLA_OK;
}

// Fewest tiles per decode workgroup: the library's choice when it sizes the split, none
// beyond an even split when the caller fixes num_splits.
int min_chunk(const mla_decode_params* p) { return p->num_splits > 0 ? 1 : mla::kAutoMinChunk; }

struct WsLayout {
  size_t cum, part_lse, part_o, q_abs, out_latent, total;
};

WsLayout layout(const mla_decode_params* p, int wgs, bool fused) {
  const size_t units = (size_t)p->batch * p->s_q;
  WsLayout L;
  size_t off = 0;
  L.cum = off;   // the split plan: tile and cost-line prefix sums and the segment cost
  off += round_up((2 * (units + 1) + 1) * sizeof(int32_t));
  L.part_lse = off;
  off += round_up((size_t)2 * wgs * mla::kHeads * sizeof(float));
  L.part_o = off;
  off += round_up((size_t)2 * wgs * mla::kHeads * mla::kLatent * 2);
  L.q_abs = off;
  if (fused) off += round_up(units * mla::kHeads * mla::kLatent * 2);
  L.out_latent = off;
  if (fused) off += round_up(units * mla::kHeads * mla::kLatent * 2);
  L.total = off;
  return L;
}


// Opt-in kernel timing for benchmarks: HIP events recorded on the caller's
// stream around each kernel of a decode call.  Slot layout: 0 start,
// 1 absorb done, 2 plan done, 3 decode done, 4 combine done, 5 up-proj done.
// `ran` has bit k set when kernel k (absorb, plan, decode, combine, up-proj) was
// launched by the call: an interval with no kernel in it is only event overhead
// and is left out of the sums.
constexpr int kProfKernels = 5;
struct ProfCall {
  std::array<hipEvent_t, kProfKernels + 1> ev{};
  unsigned ran = 0;
};
struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::deque<ProfCall> ev;   // a deque: entries handed out stay where they are
  size_t used = 0;
  // cache-append calls: 0 start, 1 projection done, 2 partial sums done
  std::vector<std::array<hipEvent_t, 3>> aev;
  size_t aused = 0;
  // decompress-branch prefill calls: 0 start, 1 decompress done, 2 attention done
  std::vector<std::array<hipEvent_t, 3>> pev;
  size_t pused = 0;
};
Profiler g_prof;
constexpr size_t kMaxProfiledCalls = 1 << 16;
constexpr unsigned kRanAbsorb = 1u, kRanPlan = 2u, kRanDecode = 4u, kRanCombine = 8u, kRanUpProj = 16u;

ProfCall* prof_slot() {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.enabled || g_prof.used >= kMaxProfiledCalls) return nullptr;
  if (g_prof.used == g_prof.ev.size()) {
    ProfCall c;
    for (auto& x : c.ev)
      if (hipEventCreate(&x) != hipSuccess) return nullptr;
    g_prof.ev.push_back(c);
  }
  ProfCall* c = &g_prof.ev[g_prof.used++];
  c->ran = 0;
  return c;
}

hipEvent_t* prof_triple_slot(std::vector<std::array<hipEvent_t, 3>>& v, size_t& used) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.enabled || used >= kMaxProfiledCalls) return nullptr;
  if (used == v.size()) {
    std::array<hipEvent_t, 3> e{};
    for (auto& x : e)
      if (hipEventCreate(&x) != hipSuccess) return nullptr;
    v.push_back(e);
  }
  return v[used++].data();
}

mla_status collect_triples(std::vector<std::array<hipEvent_t, 3>>& v, size_t& used, double* ms, int32_t* calls) {
  if (ms == nullptr || calls == nullptr) return fail(MLA_ERR_INVALID_ARG, "NULL output pointer");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  ms[0] = ms[1] = 0.0;
  for (size_t i = 0; i < used; ++i) {
    auto& e = v[i];
    hipError_t r = hipEventSynchronize(e[2]);
    if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize");
    for (int k = 0; k < 2; ++k) {
      float t = 0.f;
      r = hipEventElapsedTime(&t, e[k], e[k + 1]);
      if (r != hipSuccess) return hip_fail(r, "hipEventElapsedTime");
      ms[k] += t;
    }
  }
  *calls = (int32_t)used;
  used = 0;
  return ok();
}

hipEvent_t* prof_append_slot() { return prof_triple_slot(g_prof.aev, g_prof.aused); }

mla_status run_paged(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv, const unsigned char* kv8,
                     const int32_t* bt, const int32_t* seqlens, uint16_t* out_latent, float* lse,
                     const mla_decode_params* p, unsigned char* ws, const WsLayout& L, int wgs, hipStream_t s,
                     ProfCall* pc) {
  hipEvent_t* ev = pc ? pc->ev.data() : nullptr;
  mla::DecodePlanView plan;
  plan.cum = reinterpret_cast<int32_t*>(ws + L.cum);
  plan.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  plan.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o);
  hipError_t e = mla::launch_decode(q_abs, q_r, kv, kv8, bt, seqlens, out_latent, lse, p->batch, p->s_q,
                                    p->max_blocks_per_seq, p->num_pages, p->scale, wgs, min_chunk(p), plan, s,
                                    ev ? ev[2] : nullptr, ev ? ev[3] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (ev != nullptr && (e = hipEventRecord(ev[4], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (pc != nullptr && p->batch > 0)
    pc->ran |= kRanDecode | kRanCombine | (mla::decode_launches_plan(p->batch * p->s_q) ? kRanPlan : 0u);
  return MLA_OK;
}

mla_status check_append(const mla_append_params* p) {
  if (p == nullptr) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->s_q < 1) return fail(MLA_ERR_INVALID_ARG, "s_q %d < 1", p->s_q);
  if ((int64_t)p->batch * p->s_q > (1 << 24)) return fail(MLA_ERR_INVALID_ARG, "batch * s_q too large");
  if (p->d_model < 256 || p->d_model % 256 != 0 || p->d_model > (1 << 16))
    return fail(MLA_ERR_UNSUPPORTED, "d_model %d (supported: multiples of 256 up to 65536)", p->d_model);
  if (p->page_size != mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size %d (supported: 64)", p->page_size);
  if (p->max_blocks_per_seq < 1 || p->max_blocks_per_seq > (1 << 24))
    return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq %d", p->max_blocks_per_seq);
  if (p->max_pos < 1 || p->max_pos > (1 << 26)) return fail(MLA_ERR_INVALID_ARG, "max_pos %d", p->max_pos);
  if (p->num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages %lld < 1", (long long)p->num_pages);
  if (p->num_heads < 1 || p->num_heads > 4096) return fail(MLA_ERR_INVALID_ARG, "num_heads %d", p->num_heads);
  if (p->reserved != 0) return fail(MLA_ERR_INVALID_ARG, "reserved must be 0");
  return MLA_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

mla_status check_prefill(const mla_prefill_params* p) {
  if (p == nullptr) return fail(MLA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch %d < 0", p->batch);
  if (p->s_q < 1 || p->s_q > (1 << 20)) return fail(MLA_ERR_INVALID_ARG, "s_q %d", p->s_q);
  if ((int64_t)p->batch * p->s_q > (1 << 24)) return fail(MLA_ERR_INVALID_ARG, "batch * s_q too large");
  if (p->num_heads != mla::kHeads) return fail(MLA_ERR_UNSUPPORTED, "num_heads %d (supported: 128)", p->num_heads);
  if (p->page_size != mla::kPage) return fail(MLA_ERR_UNSUPPORTED, "page_size %d (supported: 64)", p->page_size);
  if (p->max_blocks_per_seq < 1 || p->max_blocks_per_seq > (1 << 20))
    return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_seq %d", p->max_blocks_per_seq);
  if (p->num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages %lld < 1", (long long)p->num_pages);
  if (!(p->scale > 0.f) || p->scale > 1e30f) return fail(MLA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (p->mode < 0 || p->mode > 2) return fail(MLA_ERR_INVALID_ARG, "mode %d (0 auto, 1 absorb, 2 decompress)", p->mode);
  if (p->threshold < 0 || p->threshold > kMaxDecodeSq + 1)
    return fail(MLA_ERR_INVALID_ARG, "threshold %d (0 .. %d)", p->threshold, kMaxDecodeSq + 1);
  if (p->reserved != 0) return fail(MLA_ERR_INVALID_ARG, "reserved must be 0");
  const int thr = p->threshold > 0 ? p->threshold : kPrefillThreshold;
  const bool absorb = p->mode == 1 || (p->mode == 0 && p->s_q < thr);
  if (absorb && p->s_q > kMaxDecodeSq)
    return fail(MLA_ERR_UNSUPPORTED, "s_q %d on the absorbed branch (at most %d)", p->s_q, kMaxDecodeSq);
  if (!absorb && (int64_t)p->batch * p->max_blocks_per_seq * mla::kPage * mla::kHeads > ((int64_t)1 << 40))
    return fail(MLA_ERR_INVALID_ARG, "expanded K/V too large");
  return MLA_OK;
}

bool prefill_absorbs(const mla_prefill_params* p) {
  const int thr = p->threshold > 0 ? p->threshold : kPrefillThreshold;
  return p->mode == 1 || (p->mode == 0 && p->s_q < thr);
}

mla_decode_params absorbed_params(const mla_prefill_params* p) {
  mla_decode_params d{};
  d.batch = p->batch;
  d.s_q = p->s_q;
  d.num_heads = p->num_heads;
  d.page_size = p->page_size;
  d.max_blocks_per_seq = p->max_blocks_per_seq;
  d.num_splits = 0;
  d.num_pages = p->num_pages;
  d.scale = p->scale;
  d.reserved = 0;
  return d;
}

// Bytes of one expanded tensor (K or V): [batch, max_blocks * 64, 128, 128] bf16.
size_t expanded_bytes(const mla_prefill_params* p) {
  return round_up((size_t)p->batch * p->max_blocks_per_seq * mla::kPage * mla::kHeads * mla::kDimC * 2);
}

}  // namespace

extern "C" {

size_t mla_append_workspace_size(const mla_append_params* p) {
  if (check_append(p) != MLA_OK) return 0;
  const int T = p->batch * p->s_q;
  // the MXFP8 plan always has partials and is otherwise the bf16 one: enough for both
  const size_t part = T > 0 ? round_up(mla::plan_append(T, p->d_model, true).part_bytes) : 0;
  return part > 0 ? part : 16;
}

}  // extern "C"

namespace {

mla_status append_impl(const uint16_t* x, const uint16_t* w_a, const float* rope_table, const int32_t* block_table,
                       const int32_t* seqlens, uint16_t* kv_blocks, unsigned char* kv8, uint16_t* q_r,
                       const mla_append_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_append(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return ok();
  if (!x || !w_a || !rope_table || !block_table || !seqlens || (!kv_blocks && !kv8) || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(x) || !aligned16(w_a) || !aligned16(rope_table) || !aligned16(kv_blocks) || !aligned16(kv8) ||
      !aligned16(workspace) || !aligned4(block_table) || !aligned4(seqlens) || !aligned16(q_r))
    return fail(MLA_ERR_MISALIGNED, "tensor or workspace not aligned (16 B; block_table and seqlens 4 B)");
  const size_t need = mla_append_workspace_size(p);
  if (workspace_bytes < need) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = prof_append_slot();
  hipError_t e;
  if (ev != nullptr && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = mla::launch_append(x, w_a, rope_table, block_table, seqlens, kv_blocks, kv8, q_r, p->num_heads,
                         static_cast<unsigned char*>(workspace), p->batch, p->s_q, p->d_model,
                         p->max_blocks_per_seq, p->num_pages, p->max_pos, s, ev ? ev[1] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  if (ev != nullptr && (e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return ok();
}

}  // namespace

extern "C" {

mla_status mla_append_kv(const uint16_t* x, const uint16_t* w_a, const float* rope_table,
                         const int32_t* block_table, const int32_t* seqlens, uint16_t* kv_blocks, uint16_t* q_r,
                         const mla_append_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  return append_impl(x, w_a, rope_table, block_table, seqlens, kv_blocks, nullptr, q_r, p, workspace,
                     workspace_bytes, stream);
}

mla_status mla_append_kv_mxfp8(const uint16_t* x, const uint16_t* w_a, const float* rope_table,
                               const int32_t* block_table, const int32_t* seqlens, uint8_t* kv_mxfp8,
                               uint16_t* q_r, const mla_append_params* p, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return append_impl(x, w_a, rope_table, block_table, seqlens, nullptr, kv_mxfp8, q_r, p, workspace,
                     workspace_bytes, stream);
}

mla_status mla_quantize_kv_mxfp8(const uint16_t* kv_blocks, uint8_t* kv_mxfp8, int64_t num_pages, void* stream) {
  if (num_pages < 0 || num_pages > ((int64_t)1 << 31) / mla::kPage)
    return fail(MLA_ERR_INVALID_ARG, "num_pages %lld", (long long)num_pages);
  if (num_pages == 0) return ok();
  if (!kv_blocks || !kv_mxfp8) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(kv_blocks) || !aligned16(kv_mxfp8)) return fail(MLA_ERR_MISALIGNED, "tensor not 16-byte aligned");
  hipError_t e = mla::launch_quantize_mxfp8(kv_blocks, kv_mxfp8, num_pages, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return ok();
}

mla_status mla_rope_q(uint16_t* q_r, const float* rope_table, const int32_t* seqlens, int32_t batch, int32_t s_q,
                      int32_t num_heads, int32_t max_pos, void* stream) {
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (s_q < 1) return fail(MLA_ERR_INVALID_ARG, "s_q %d < 1", s_q);
  if ((int64_t)batch * s_q > (1 << 24)) return fail(MLA_ERR_INVALID_ARG, "batch * s_q too large");
  if (num_heads < 1 || num_heads > 4096) return fail(MLA_ERR_INVALID_ARG, "num_heads %d", num_heads);
  if (max_pos < 1 || max_pos > (1 << 26)) return fail(MLA_ERR_INVALID_ARG, "max_pos %d", max_pos);
  if (batch == 0) return ok();
  if (!q_r || !rope_table || !seqlens) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_r) || !aligned16(rope_table) || !aligned4(seqlens))
    return fail(MLA_ERR_MISALIGNED, "tensor not aligned (16 B; seqlens 4 B)");
  hipError_t e = mla::launch_rope_q(q_r, rope_table, seqlens, batch, s_q, num_heads, max_pos,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope_q launch");
  return ok();
}

mla_status mla_rope_table(float* rope_table, int32_t max_pos, double base, void* stream) {
  if (max_pos < 1 || max_pos > (1 << 26)) return fail(MLA_ERR_INVALID_ARG, "max_pos %d", max_pos);
  if (!(base > 1.0) || base > 1e30) return fail(MLA_ERR_INVALID_ARG, "base must be finite and > 1");
  if (!rope_table) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(rope_table)) return fail(MLA_ERR_MISALIGNED, "rope_table not 16-byte aligned");
  hipError_t e = mla::launch_rope_table(rope_table, max_pos, base, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope_table launch");
  return ok();
}

const char* mla_status_string(mla_status s) {
  // A C caller may pass any int; in C++ an enum object holding a value outside the
  // enumerators' range may not be read as the enum, so its bytes are read as an int.
  int32_t code;
  static_assert(sizeof(s) == sizeof(code), "mla_status is int-sized");
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_MISALIGNED: return "MLA_ERR_MISALIGNED";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

mla_status mla_device_cu_count(int32_t* num_cus) {
  if (num_cus == nullptr) return fail(MLA_ERR_INVALID_ARG, "num_cus is NULL");
  mla_decode_params p{};
  p.num_splits = 0;
  int w = 0;
  mla_status st = resolve_wgs(&p, &w);
  if (st != MLA_OK) return st;
  *num_cus = w;
  return ok();
}

mla_status mla_absorb_q(const uint16_t* q_c, const uint16_t* w_uk, uint16_t* q_abs, int32_t tokens,
                        int32_t num_heads, void* stream) {
  if (tokens < 0) return fail(MLA_ERR_INVALID_ARG, "tokens %d < 0", tokens);
  if (num_heads != mla::kHeads) return fail(MLA_ERR_UNSUPPORTED, "num_heads %d (supported: 128)", num_heads);
  if (tokens == 0) return ok();
  if (!q_c || !w_uk || !q_abs) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_c) || !aligned16(w_uk) || !aligned16(q_abs)) return fail(MLA_ERR_MISALIGNED, "tensor not 16-byte aligned");
  hipError_t e = mla::launch_absorb_q(q_c, w_uk, q_abs, tokens, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "absorb_q launch");
  return ok();
}

mla_status mla_up_proj(const uint16_t* out_latent, const uint16_t* w_uv, uint16_t* out, int32_t tokens,
                       int32_t num_heads, void* stream) {
  if (tokens < 0) return fail(MLA_ERR_INVALID_ARG, "tokens %d < 0", tokens);
  if (num_heads != mla::kHeads) return fail(MLA_ERR_UNSUPPORTED, "num_heads %d (supported: 128)", num_heads);
  if (tokens == 0) return ok();
  if (!out_latent || !w_uv || !out) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(out_latent) || !aligned16(w_uv) || !aligned16(out)) return fail(MLA_ERR_MISALIGNED, "tensor not 16-byte aligned");
  hipError_t e = mla::launch_up_proj(out_latent, w_uv, out, tokens, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "up_proj launch");
  return ok();
}

size_t mla_decode_workspace_size(const mla_decode_params* p, int32_t fused) {
  if (check_params(p) != MLA_OK) return 0;
  int wgs = 0;
  if (resolve_wgs(p, &wgs) != MLA_OK) return 0;
  return layout(p, wgs, fused != 0).total;
}

}  // extern "C"

namespace {

mla_status decode_paged_impl(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv_blocks,
                             const unsigned char* kv8, const int32_t* block_table, const int32_t* seqlens,
                             uint16_t* out_latent, float* lse, const mla_decode_params* p, void* workspace,
                             size_t workspace_bytes, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return ok();
  if (!q_abs || !q_r || (!kv_blocks && !kv8) || !block_table || !seqlens || !out_latent)
    return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_abs) || !aligned16(q_r) || !aligned16(kv_blocks) || !aligned16(kv8) || !aligned16(block_table) ||
      !aligned16(out_latent) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(seqlens) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_MISALIGNED, "tensor or workspace not aligned (16 B; seqlens and lse 4 B)");
  int wgs = 0;
  st = resolve_wgs(p, &wgs);
  if (st != MLA_OK) return st;
  const WsLayout L = layout(p, wgs, false);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  ProfCall* pc = prof_slot();
  if (pc != nullptr) {
    hipError_t e = hipEventRecord(pc->ev[0], s);
    if (e == hipSuccess) e = hipEventRecord(pc->ev[1], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  st = run_paged(q_abs, q_r, kv_blocks, kv8, block_table, seqlens, out_latent, lse, p,
                 static_cast<unsigned char*>(workspace), L, wgs, s, pc);
  if (st == MLA_OK && pc != nullptr) {
    hipError_t e = hipEventRecord(pc->ev[5], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return st == MLA_OK ? ok() : st;
}

mla_status decode_fused_impl(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk, const uint16_t* w_uv,
                             const uint16_t* kv_blocks, const unsigned char* kv8, const int32_t* block_table,
                             const int32_t* seqlens, uint16_t* out, float* lse, const mla_decode_params* p,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return ok();
  if (!q_c || !q_r || !w_uk || !w_uv || (!kv_blocks && !kv8) || !block_table || !seqlens || !out)
    return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_c) || !aligned16(q_r) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(kv_blocks) ||
      !aligned16(kv8) ||
      !aligned16(block_table) || !aligned16(out) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(seqlens) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_MISALIGNED, "tensor or workspace not aligned (16 B; seqlens and lse 4 B)");
  int wgs = 0;
  st = resolve_wgs(p, &wgs);
  if (st != MLA_OK) return st;
  const WsLayout L = layout(p, wgs, true);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int tokens = p->batch * p->s_q;
  uint16_t* q_abs = reinterpret_cast<uint16_t*>(ws + L.q_abs);
  uint16_t* ol = reinterpret_cast<uint16_t*>(ws + L.out_latent);
  ProfCall* pc = prof_slot();
  hipEvent_t* ev = pc ? pc->ev.data() : nullptr;
  hipError_t e;
  if (ev != nullptr && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = mla::launch_absorb_q(q_c, w_uk, q_abs, tokens, s);
  if (e != hipSuccess) return hip_fail(e, "absorb_q launch");
  if (ev != nullptr && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  st = run_paged(q_abs, q_r, kv_blocks, kv8, block_table, seqlens, ol, lse, p, ws, L, wgs, s, pc);
  if (st != MLA_OK) return st;
  e = mla::launch_up_proj(ol, w_uv, out, tokens, s);
  if (e != hipSuccess) return hip_fail(e, "up_proj launch");
  if (ev != nullptr && (e = hipEventRecord(ev[5], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (pc != nullptr) pc->ran |= kRanAbsorb | kRanUpProj;
  return ok();
}

}  // namespace

extern "C" {

mla_status mla_decode_paged(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv_blocks,
                            const int32_t* block_table, const int32_t* seqlens, uint16_t* out_latent, float* lse,
                            const mla_decode_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_paged_impl(q_abs, q_r, kv_blocks, nullptr, block_table, seqlens, out_latent, lse, p, workspace,
                           workspace_bytes, stream);
}

mla_status mla_decode_paged_mxfp8(const uint16_t* q_abs, const uint16_t* q_r, const uint8_t* kv_mxfp8,
                                  const int32_t* block_table, const int32_t* seqlens, uint16_t* out_latent,
                                  float* lse, const mla_decode_params* p, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_paged_impl(q_abs, q_r, nullptr, kv_mxfp8, block_table, seqlens, out_latent, lse, p, workspace,
                           workspace_bytes, stream);
}

mla_status mla_decode(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk, const uint16_t* w_uv,
                      const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens, uint16_t* out,
                      float* lse, const mla_decode_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_fused_impl(q_c, q_r, w_uk, w_uv, kv_blocks, nullptr, block_table, seqlens, out, lse, p, workspace,
                           workspace_bytes, stream);
}

mla_status mla_decode_mxfp8(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk, const uint16_t* w_uv,
                            const uint8_t* kv_mxfp8, const int32_t* block_table, const int32_t* seqlens,
                            uint16_t* out, float* lse, const mla_decode_params* p, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_fused_impl(q_c, q_r, w_uk, w_uv, nullptr, kv_mxfp8, block_table, seqlens, out, lse, p, workspace,
                           workspace_bytes, stream);
}

size_t mla_prefill_workspace_size(const mla_prefill_params* p) {
  if (check_prefill(p) != MLA_OK) return 0;
  if (prefill_absorbs(p)) {
    const mla_decode_params d = absorbed_params(p);
    return mla_decode_workspace_size(&d, 1);
  }
  return p->batch == 0 ? 16 : 2 * expanded_bytes(p);
}

mla_status mla_prefill(const uint16_t* q_c, const uint16_t* q_r, const uint16_t* w_uk, const uint16_t* w_uv,
                       const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens, uint16_t* out,
                       float* lse, const mla_prefill_params* p, void* workspace, size_t workspace_bytes,
                       void* stream) {
  mla_status st = check_prefill(p);
  if (st != MLA_OK) return st;
  if (prefill_absorbs(p)) {
    const mla_decode_params d = absorbed_params(p);
    return mla_decode(q_c, q_r, w_uk, w_uv, kv_blocks, block_table, seqlens, out, lse, &d, workspace,
                      workspace_bytes, stream);
  }
  if (p->batch == 0) return ok();
  if (!q_c || !q_r || !w_uk || !w_uv || !kv_blocks || !block_table || !seqlens || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_c) || !aligned16(q_r) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(kv_blocks) ||
      !aligned16(out) || !aligned16(workspace) || !aligned4(block_table) || !aligned4(seqlens) || !aligned4(lse))
    return fail(MLA_ERR_MISALIGNED, "tensor or workspace not aligned (16 B; block_table, seqlens and lse 4 B)");
  const size_t need = mla_prefill_workspace_size(p);
  if (workspace_bytes < need) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* kbuf = static_cast<uint16_t*>(workspace);
  uint16_t* vbuf = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(workspace) + expanded_bytes(p));
  const int max_len = p->max_blocks_per_seq * mla::kPage;
  hipEvent_t* ev = prof_triple_slot(g_prof.pev, g_prof.pused);
  hipError_t e;
  if (ev != nullptr && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = mla::launch_decompress(kv_blocks, block_table, seqlens, w_uk, w_uv, kbuf, vbuf, p->batch,
                             p->max_blocks_per_seq, max_len, p->num_pages, s);
  if (e != hipSuccess) return hip_fail(e, "decompress launch");
  if (ev != nullptr && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = mla::launch_prefill_attention(q_c, q_r, kbuf, vbuf, kv_blocks, block_table, seqlens, out, lse, p->batch,
                                    p->s_q, p->max_blocks_per_seq, max_len, p->num_pages, p->scale, s);
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  if (ev != nullptr && (e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return ok();
}

mla_status mla_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.enabled = enable != 0;
  g_prof.used = 0;
  g_prof.aused = 0;
  g_prof.pused = 0;
  return ok();
}

mla_status mla_profile_collect(double* ms, int32_t* launches, int32_t* calls) {
  if (ms == nullptr || launches == nullptr || calls == nullptr) return fail(MLA_ERR_INVALID_ARG, "NULL output pointer");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int k = 0; k < kProfKernels; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  for (size_t i = 0; i < g_prof.used; ++i) {
    auto& c = g_prof.ev[i];
    hipError_t r = hipEventSynchronize(c.ev[kProfKernels]);
    if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize");
    for (int k = 0; k < kProfKernels; ++k) {
      if (!(c.ran & (1u << k))) continue;
      float t = 0.f;
      r = hipEventElapsedTime(&t, c.ev[k], c.ev[k + 1]);
      if (r != hipSuccess) return hip_fail(r, "hipEventElapsedTime");
      ms[k] += t;
      ++launches[k];
    }
  }
  *calls = (int32_t)g_prof.used;
  g_prof.used = 0;
  return ok();
}

mla_status mla_profile_collect_append(double* ms, int32_t* calls) {
  return collect_triples(g_prof.aev, g_prof.aused, ms, calls);
}

mla_status mla_profile_collect_prefill(double* ms, int32_t* calls) {
  return collect_triples(g_prof.pev, g_prof.pused, ms, calls);
}

mla_status mla_gather_kv(const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens,
                         uint16_t* dense, const mla_decode_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return ok();
  if (!kv_blocks || !block_table || !seqlens || !dense) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(kv_blocks) || !aligned16(dense) || (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seqlens) & 3u))
    return fail(MLA_ERR_MISALIGNED, "tensor not aligned");
  hipError_t e = mla::launch_gather(kv_blocks, block_table, seqlens, dense, p->batch, p->max_blocks_per_seq,
                                    p->num_pages, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

mla_status mla_decode_paged_noalloc(const uint16_t* q_abs, const uint16_t* q_r, const uint16_t* kv_blocks,
                                    const int32_t* block_table, const int32_t* seqlens, uint16_t* out_latent,
                                    float* lse, const mla_decode_params* p, void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return ok();
  int wgs = 0;
  st = resolve_wgs(p, &wgs);
  if (st != MLA_OK) return st;
  const WsLayout L = layout(p, wgs, false);
  if (L.total > mla::kNoAllocScratchBytes)
    return fail(MLA_ERR_UNSUPPORTED,
                "allocation-free decode: %d workgroups and %d units need %zu bytes of workspace, above the "
                "built-in %zu (at most 256 workgroups and 65536 sequence-query units)",
                wgs, p->batch * p->s_q, L.total, mla::kNoAllocScratchBytes);
  unsigned char* ws = nullptr;
  const hipError_t e = mla::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  return decode_paged_impl(q_abs, q_r, kv_blocks, nullptr, block_table, seqlens, out_latent, lse, p, ws, L.total,
                           stream);
}

int32_t mla_decode_num_workgroups(const mla_decode_params* p) {
  if (check_params(p) != MLA_OK) return 0;
  int wgs = 0;
  if (resolve_wgs(p, &wgs) != MLA_OK) return 0;
  return wgs;
}

mla_status mla_stream_pages(const uint16_t* kv_blocks, const int32_t* block_table, const int32_t* seqlens,
                            uint32_t* sums, const mla_decode_params* p, void* workspace, size_t workspace_bytes,
                            void* stream) {
  mla_status st = check_params(p);
  if (st != MLA_OK) return st;
  if (p->batch == 0) return ok();
  if (!kv_blocks || !block_table || !seqlens || !sums) return fail(MLA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(kv_blocks) || !aligned16(block_table) || !aligned16(workspace) || !aligned4(sums) ||
      (reinterpret_cast<uintptr_t>(seqlens) & 3u))
    return fail(MLA_ERR_MISALIGNED, "tensor or workspace not aligned (16 B; sums and seqlens 4 B)");
  int wgs = 0;
  st = resolve_wgs(p, &wgs);
  if (st != MLA_OK) return st;
  const WsLayout L = layout(p, wgs, false);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  hipError_t e = mla::launch_stream(kv_blocks, block_table, seqlens, sums, p->batch, p->s_q, p->max_blocks_per_seq,
                                    p->num_pages, wgs, min_chunk(p),
                                    reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) + L.cum),
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream launch");
  return ok();
}

}  // extern "C"
