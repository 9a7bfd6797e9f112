// Host-side argument validation of the C ABI, run under AddressSanitizer and
// UndefinedBehaviorSanitizer (the library's host code and this driver are built with
// -fsanitize=address,undefined on the host side only; no kernel is ever launched).
// Every call below must be rejected, or sized, on the host before any GPU work; the
// program exits non-zero on the first unexpected status and the sanitizers abort on
// any memory error or undefined behaviour along the way (signed overflow in the size
// arithmetic, out-of-range shifts, misaligned accesses, bad format strings).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mla.h"

static int g_checks = 0, g_failures = 0;

static void expect(const char* what, int got, int want) {
  ++g_checks;
  if (got != want) {
    ++g_failures;
    std::printf("FAIL %s: status %d (%s), expected %d (%s); last error: %s\n", what, got,
                mla_status_string((mla_status)got), want, mla_status_string((mla_status)want), mla_last_error());
  }
}

static void expect_true(const char* what, bool ok) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::printf("FAIL %s\n", what);
  }
}

// Fake device addresses: validation rejects every call before anything dereferences them.
static void* const A = reinterpret_cast<void*>(0x10000);
static void* const MIS = reinterpret_cast<void*>(0x10008);

static mla_decode_params params() {
  mla_decode_params p;
  std::memset(&p, 0, sizeof p);
  p.batch = 2;
  p.s_q = 1;
  p.num_heads = 128;
  p.page_size = 64;
  p.max_blocks_per_seq = 4;
  p.num_splits = 8;
  p.num_pages = 8;
  p.scale = 0.0721687836f;
  return p;
}

static int paged(const mla_decode_params* p, void* ws = A, size_t ws_bytes = size_t(1) << 30) {
  auto* u16 = static_cast<uint16_t*>(A);
  auto* i32 = static_cast<int32_t*>(A);
  return mla_decode_paged(u16, u16, u16, i32, i32, u16, nullptr, p, ws, ws_bytes, nullptr);
}

int main() {
  // status strings, including an unknown code
  expect_true("status string of MLA_OK", std::strcmp(mla_status_string(MLA_OK), "MLA_OK") == 0);
  expect_true("status string of an unknown code", std::strcmp(mla_status_string((mla_status)99), "MLA_ERR_UNKNOWN") == 0);

  // decode parameters, one bad field at a time
  struct Bad {
    const char* what;
    void (*set)(mla_decode_params&);
    int status;
  } bad[] = {
      {"s_q 0", [](mla_decode_params& p) { p.s_q = 0; }, MLA_ERR_UNSUPPORTED},
      {"s_q 257", [](mla_decode_params& p) { p.s_q = 257; }, MLA_ERR_UNSUPPORTED},
      {"num_heads 64", [](mla_decode_params& p) { p.num_heads = 64; }, MLA_ERR_UNSUPPORTED},
      {"page_size 16", [](mla_decode_params& p) { p.page_size = 16; }, MLA_ERR_UNSUPPORTED},
      {"batch -1", [](mla_decode_params& p) { p.batch = -1; }, MLA_ERR_INVALID_ARG},
      {"batch INT32_MIN", [](mla_decode_params& p) { p.batch = INT32_MIN; }, MLA_ERR_INVALID_ARG},
      {"max_blocks 0", [](mla_decode_params& p) { p.max_blocks_per_seq = 0; }, MLA_ERR_INVALID_ARG},
      {"max_blocks INT32_MAX", [](mla_decode_params& p) { p.max_blocks_per_seq = INT32_MAX; }, MLA_ERR_INVALID_ARG},
      {"num_pages 0", [](mla_decode_params& p) { p.num_pages = 0; }, MLA_ERR_INVALID_ARG},
      {"num_pages INT64_MIN", [](mla_decode_params& p) { p.num_pages = INT64_MIN; }, MLA_ERR_INVALID_ARG},
      {"scale 0", [](mla_decode_params& p) { p.scale = 0.f; }, MLA_ERR_INVALID_ARG},
      {"scale NaN", [](mla_decode_params& p) { p.scale = std::nanf(""); }, MLA_ERR_INVALID_ARG},
      {"scale inf", [](mla_decode_params& p) { p.scale = INFINITY; }, MLA_ERR_INVALID_ARG},
      {"num_splits -2", [](mla_decode_params& p) { p.num_splits = -2; }, MLA_ERR_INVALID_ARG},
      {"num_splits INT32_MAX", [](mla_decode_params& p) { p.num_splits = INT32_MAX; }, MLA_ERR_INVALID_ARG},
      {"reserved 1", [](mla_decode_params& p) { p.reserved = 1; }, MLA_ERR_INVALID_ARG},
      {"batch * s_q over 2^24", [](mla_decode_params& p) { p.batch = INT32_MAX; p.s_q = 256; }, MLA_ERR_INVALID_ARG},
      {"tiles over 2^31", [](mla_decode_params& p) { p.batch = 4096; p.s_q = 2; p.max_blocks_per_seq = 1 << 17; },
       MLA_ERR_INVALID_ARG},
  };
  for (const Bad& b : bad) {
    mla_decode_params p = params();
    b.set(p);
    expect(b.what, paged(&p), b.status);
    expect_true(b.what, mla_last_error()[0] != '\0');
    expect_true("workspace size of bad params is 0", mla_decode_workspace_size(&p, 0) == 0);
  }
  expect("NULL params", paged(nullptr), MLA_ERR_INVALID_ARG);
  expect_true("workspace size of NULL params is 0", mla_decode_workspace_size(nullptr, 1) == 0);

  // the largest accepted sizes: the workspace arithmetic stays in range
  {
    mla_decode_params p = params();
    p.batch = 4096;
    p.s_q = 2;
    p.max_blocks_per_seq = 131064;   // 8192 units x (2 x 131064 + 6) + 65536 <= 2^31 - 1
    p.num_splits = 1 << 16;
    const size_t need = mla_decode_workspace_size(&p, 0);
    expect_true("largest accepted decode has a workspace size", need > 0);
    expect_true("the fused call needs more", mla_decode_workspace_size(&p, 1) > need);
    expect("workspace one byte short", paged(&p, A, need - 1), MLA_ERR_WORKSPACE);
  }

  // pointers: NULL and misaligned tensors, small and missing workspaces
  {
    mla_decode_params p = params();
    auto* u16 = static_cast<uint16_t*>(A);
    auto* i32 = static_cast<int32_t*>(A);
    auto* mis = static_cast<uint16_t*>(MIS);
    expect("NULL q_r", mla_decode_paged(u16, nullptr, u16, i32, i32, u16, nullptr, &p, A, 1 << 30, nullptr),
           MLA_ERR_INVALID_ARG);
    expect("misaligned kv_blocks", mla_decode_paged(u16, u16, mis, i32, i32, u16, nullptr, &p, A, 1 << 30, nullptr),
           MLA_ERR_MISALIGNED);
    const size_t need = mla_decode_workspace_size(&p, 0);
    expect_true("workspace size", need > 0);
    expect("NULL workspace", paged(&p, nullptr, need), MLA_ERR_WORKSPACE);
    expect("empty batch is a no-op", [&] {
      mla_decode_params e = params();
      e.batch = 0;
      return mla_decode_paged(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &e, nullptr, 0, nullptr);
    }(), MLA_OK);
  }

  // projections
  {
    auto* u16 = static_cast<uint16_t*>(A);
    expect("absorb tokens -1", mla_absorb_q(u16, u16, u16, -1, 128, nullptr), MLA_ERR_INVALID_ARG);
    expect("absorb tokens INT32_MIN", mla_absorb_q(u16, u16, u16, INT32_MIN, 128, nullptr), MLA_ERR_INVALID_ARG);
    expect("absorb heads 96", mla_absorb_q(u16, u16, u16, 4, 96, nullptr), MLA_ERR_UNSUPPORTED);
    expect("up-proj misaligned", mla_up_proj(static_cast<uint16_t*>(MIS), u16, u16, 4, 128, nullptr),
           MLA_ERR_MISALIGNED);
    expect("absorb nothing", mla_absorb_q(nullptr, nullptr, nullptr, 0, 128, nullptr), MLA_OK);
  }

  // cache append parameters
  {
    mla_append_params p;
    std::memset(&p, 0, sizeof p);
    p.batch = 2;
    p.s_q = 1;
    p.d_model = 7168;
    p.page_size = 64;
    p.max_blocks_per_seq = 4;
    p.max_pos = 1024;
    p.num_pages = 8;
    p.num_heads = 128;
    expect_true("append workspace size", mla_append_workspace_size(&p) > 0);
    mla_append_params q = p;
    q.d_model = 7000;
    expect_true("append d_model 7000 has no workspace", mla_append_workspace_size(&q) == 0);
    q = p;
    q.d_model = INT32_MAX;
    expect_true("append d_model INT32_MAX has no workspace", mla_append_workspace_size(&q) == 0);
    q = p;
    q.batch = INT32_MAX;
    q.s_q = INT32_MAX;
    expect_true("append batch * s_q overflow has no workspace", mla_append_workspace_size(&q) == 0);
    expect_true("append NULL params has no workspace", mla_append_workspace_size(nullptr) == 0);
  }

  // prefill parameters
  {
    mla_prefill_params p;
    std::memset(&p, 0, sizeof p);
    p.batch = 2;
    p.s_q = 300;
    p.num_heads = 128;
    p.page_size = 64;
    p.max_blocks_per_seq = 16;
    p.num_pages = 32;
    p.scale = 0.0721687836f;
    expect_true("prefill workspace size", mla_prefill_workspace_size(&p) > 0);
    mla_prefill_params q = p;
    q.threshold = 258;
    expect_true("prefill threshold 258 has no workspace", mla_prefill_workspace_size(&q) == 0);
    q = p;
    q.max_blocks_per_seq = INT32_MAX;
    expect_true("prefill huge table has no workspace", mla_prefill_workspace_size(&q) == 0);
    q = p;
    q.mode = 7;
    expect_true("prefill mode 7 has no workspace", mla_prefill_workspace_size(&q) == 0);
  }

  // RoPE helpers
  {
    expect("rope table max_pos 0", mla_rope_table(static_cast<float*>(A), 0, 10000.0, nullptr), MLA_ERR_INVALID_ARG);
    expect("rope table base NaN", mla_rope_table(static_cast<float*>(A), 16, std::nan(""), nullptr),
           MLA_ERR_INVALID_ARG);
  }

  std::printf("%s: %d checks, %d failures\n", g_failures ? "FAILED" : "ok", g_checks, g_failures);
  return g_failures ? 1 : 0;
}
