// Argument fuzz of the C ABI (include/gdn.h), for a host build with
// AddressSanitizer and UndefinedBehaviorSanitizer: every entry point is called
// with a valid base shape and one defect at a time (null pointers, bad or
// extreme sizes, unsupported dtypes and tile sizes, short or misaligned
// workspaces, bad parameters), and must return a non-OK status with a
// message, without touching the device buffers (the pointers passed are host
// addresses that the library must not read) and without a sanitizer report.
// The workspace-size queries must return 0 for bad arguments and must not
// overflow for extreme ones.  Exit status 0 when every check holds.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"

namespace {

int g_checks = 0, g_failures = 0;

void expect_error(gdn_status_t st, const char* what) {
  ++g_checks;
  const char* msg = gdn_last_error();
  if (st == GDN_OK || msg == nullptr || msg[0] == '\0') {
    ++g_failures;
    std::printf("FAIL %s: status %d (%s), message \"%s\"\n", what, int(st), gdn_status_string(st), msg ? msg : "(null)");
  }
}

void expect_zero(size_t v, const char* what) {
  ++g_checks;
  if (v != 0) {
    ++g_failures;
    std::printf("FAIL %s: %zu, expected 0\n", what, v);
  }
}

// dummy host buffers standing in for device pointers (never read)
alignas(256) unsigned char g_buf[4096];
alignas(256) unsigned char g_buf2[4096];  // a second buffer where two must not overlap
void* P = g_buf;
const float* F = reinterpret_cast<const float*>(g_buf);
float* FW = reinterpret_cast<float*>(g_buf);
const int32_t* I = reinterpret_cast<const int32_t*>(g_buf);

gdn_shape_t base() { return gdn_shape_t{2, 64, 2, 4, 32, 32, GDN_DTYPE_BF16}; }

// the prefill entry points, each with the same tensors
gdn_status_t scan(const gdn_shape_t* s, const void* q, const void* k, const void* v, const float* g, const float* b,
                  const int32_t* cu, void* out, float* so) {
  return gdn_prefill_scan(s, q, k, v, g, b, cu, nullptr, out, so, nullptr);
}
gdn_status_t blockwise(const gdn_shape_t* s, const void* q, const void* k, const void* v, const float* g,
                       const float* b, const int32_t* cu, void* out, float* so) {
  return gdn_prefill_scan_blockwise(s, q, k, v, g, b, cu, nullptr, out, so, 16, nullptr);
}
gdn_status_t chunked(const gdn_shape_t* s, const void* q, const void* k, const void* v, const float* g,
                     const float* b, const int32_t* cu, void* out, float* so) {
  return gdn_prefill_chunked(s, q, k, v, g, b, cu, nullptr, out, so, 64, P, size_t(1) << 40, nullptr);
}
gdn_status_t segmented(const gdn_shape_t* s, const void* q, const void* k, const void* v, const float* g,
                       const float* b, const int32_t* cu, void* out, float* so) {
  return gdn_prefill_segmented(s, q, k, v, g, b, cu, nullptr, out, so, 64, 128, P, size_t(1) << 40, nullptr);
}
gdn_status_t noalloc(const gdn_shape_t* s, const void* q, const void* k, const void* v, const float* g,
                     const float* b, const int32_t* cu, void* out, float* so) {
  return gdn_prefill_segmented_noalloc(s, q, k, v, g, b, cu, nullptr, out, so, 64, 128, nullptr);
}

typedef gdn_status_t (*prefill_fn)(const gdn_shape_t*, const void*, const void*, const void*, const float*,
                                   const float*, const int32_t*, void*, float*);

void fuzz_prefill(prefill_fn fn, const char* name) {
  char what[160];
  auto run = [&](const gdn_shape_t* s, const char* defect, const void* q = g_buf, const void* k = g_buf,
                 const void* v = g_buf, const float* g = F, const float* b = F, const int32_t* cu = I,
                 void* out = g_buf, float* so = FW) {
    std::snprintf(what, sizeof what, "%s: %s", name, defect);
    expect_error(fn(s, q, k, v, g, b, cu, out, so), what);
  };
  gdn_shape_t s = base();
  run(nullptr, "shape NULL");
  run(&s, "q NULL", nullptr);
  run(&s, "k NULL", g_buf, nullptr);
  run(&s, "v NULL", g_buf, g_buf, nullptr);
  run(&s, "g NULL", g_buf, g_buf, g_buf, nullptr);
  run(&s, "beta NULL", g_buf, g_buf, g_buf, F, nullptr);
  run(&s, "cu_seqlens NULL", g_buf, g_buf, g_buf, F, F, nullptr);
  run(&s, "out NULL", g_buf, g_buf, g_buf, F, F, I, nullptr);
  run(&s, "state_out NULL", g_buf, g_buf, g_buf, F, F, I, g_buf, nullptr);
  const struct { int field; int32_t value; const char* defect; } bad[] = {
      {0, 0, "num_seqs 0"},          {0, -1, "num_seqs -1"},        {0, INT_MIN, "num_seqs INT_MIN"},
      {1, -1, "total_tokens -1"},    {1, INT_MIN, "total_tokens INT_MIN"},
      {2, 0, "h_qk 0"},              {2, -2, "h_qk -2"},            {3, 6, "h_v not a multiple of h_qk"},
      {3, 0, "h_v 0"},               {3, INT_MAX, "h_v INT_MAX"},   {4, 24, "d_k 24"},
      {4, 256, "d_k 256"},           {4, 0, "d_k 0"},               {5, 8, "d_v 8"},
      {5, 512, "d_v 512"},           {5, -32, "d_v -32"},           {6, 7, "io_dtype 7"},
      {6, -1, "io_dtype -1"},
  };
  for (const auto& c : bad) {
    gdn_shape_t t = base();
    int32_t* f[] = {&t.num_seqs, &t.total_tokens, &t.h_qk, &t.h_v, &t.d_k, &t.d_v};
    if (c.field < 6) *f[c.field] = c.value;
    else t.io_dtype = static_cast<gdn_dtype_t>(c.value);
    run(&t, c.defect);
  }
  // sizes whose products overflow 32 bits
  gdn_shape_t t = base();
  t.total_tokens = INT_MAX, t.h_qk = 64, t.h_v = 1024, t.d_k = 128, t.d_v = 128;
  run(&t, "total_tokens INT_MAX with 1024 value heads");
  t = base();
  t.num_seqs = INT_MAX;
  run(&t, "num_seqs INT_MAX");
}

void fuzz_chunked_extras() {
  gdn_shape_t s = base();
  const size_t need = gdn_prefill_chunked_workspace(&s, 64);
  ++g_checks;
  if (need == 0) {
    ++g_failures;
    std::printf("FAIL chunked workspace query of a valid shape returned 0\n");
  }
  expect_error(gdn_prefill_chunked(&s, P, P, P, F, F, I, nullptr, P, FW, 48, P, need, nullptr), "chunked: chunk 48");
  expect_error(gdn_prefill_chunked(&s, P, P, P, F, F, I, nullptr, P, FW, 0, P, need, nullptr), "chunked: chunk 0");
  expect_error(gdn_prefill_chunked(&s, P, P, P, F, F, I, nullptr, P, FW, -64, P, need, nullptr), "chunked: chunk -64");
  expect_error(gdn_prefill_chunked(&s, P, P, P, F, F, I, nullptr, P, FW, 64, nullptr, need, nullptr),
               "chunked: workspace NULL");
  expect_error(gdn_prefill_chunked(&s, P, P, P, F, F, I, nullptr, P, FW, 64, g_buf + 16, need, nullptr),
               "chunked: workspace misaligned");
  expect_error(gdn_prefill_chunked(&s, P, P, P, F, F, I, nullptr, P, FW, 64, P, need - 1, nullptr),
               "chunked: workspace one byte short");
  expect_zero(gdn_prefill_chunked_workspace(nullptr, 64), "chunked workspace: shape NULL");
  expect_zero(gdn_prefill_chunked_workspace(&s, 40), "chunked workspace: chunk 40");
  gdn_shape_t t = base();
  t.h_v = 3;
  expect_zero(gdn_prefill_chunked_workspace(&t, 64), "chunked workspace: h_v not a multiple of h_qk");
  t = base();
  t.total_tokens = INT_MAX, t.h_qk = 64, t.h_v = 64, t.d_k = 128;
  const size_t big = gdn_prefill_chunked_workspace(&t, 16);  // must not wrap around
  ++g_checks;
  if (big != 0 && big < (size_t(INT_MAX) / 16) * 64) {
    ++g_failures;
    std::printf("FAIL chunked workspace of INT_MAX tokens, 64 heads: %zu (wrapped)\n", big);
  }

  const size_t seg = gdn_prefill_segmented_workspace(&s, 64, 128);
  expect_error(gdn_prefill_segmented(&s, P, P, P, F, F, I, nullptr, P, FW, 64, 100, P, seg, nullptr),
               "segmented: segment not a multiple of the chunk");
  expect_error(gdn_prefill_segmented(&s, P, P, P, F, F, I, nullptr, P, FW, 64, 0, P, seg, nullptr),
               "segmented: segment 0");
  expect_error(gdn_prefill_segmented(&s, P, P, P, F, F, I, nullptr, P, FW, 64, -128, P, seg, nullptr),
               "segmented: segment -128");
  expect_error(gdn_prefill_segmented(&s, P, P, P, F, F, I, nullptr, P, FW, 64, 128, P, seg - 1, nullptr),
               "segmented: workspace one byte short");
  expect_error(gdn_prefill_segmented(&s, P, P, P, F, F, I, nullptr, P, FW, 64, 128, nullptr, seg, nullptr),
               "segmented: workspace NULL");
  expect_zero(gdn_prefill_segmented_workspace(&s, 64, 100), "segmented workspace: segment not a multiple");
  expect_zero(gdn_prefill_segmented_workspace(&s, 64, 0), "segmented workspace: segment 0");
  expect_zero(gdn_prefill_segmented_workspace(nullptr, 64, 128), "segmented workspace: shape NULL");
  expect_error(gdn_prefill_segmented_noalloc(&s, P, P, P, F, F, I, nullptr, P, FW, 64, INT_MAX / 64 * 64, nullptr),
               "noalloc: segment beyond the static scratch");
  expect_error(gdn_prefill_segmented_noalloc(&s, P, P, P, F, F, I, nullptr, P, FW, 48, 96, nullptr),
               "noalloc: chunk 48");

  expect_error(gdn_prefill_scan_blockwise(&s, P, P, P, F, F, I, nullptr, P, FW, 0, nullptr), "blockwise: block 0");
  expect_error(gdn_prefill_scan_blockwise(&s, P, P, P, F, F, I, nullptr, P, FW, 6, nullptr), "blockwise: block 6");
  expect_error(gdn_prefill_scan_blockwise(&s, P, P, P, F, F, I, nullptr, P, FW, -8, nullptr), "blockwise: block -8");
}

void fuzz_decode() {
  char what[128];
  auto plain = [&](int32_t b, int32_t hqk, int32_t hv, int32_t dk, int32_t dv, int dt, const char* defect,
                   const void* q = g_buf, const float* g = F, const float* sin = F, void* out = g_buf,
                   float* so = FW) {
    std::snprintf(what, sizeof what, "decode: %s", defect);
    expect_error(gdn_decode_step(b, hqk, hv, dk, dv, static_cast<gdn_dtype_t>(dt), q, P, P, g, F, sin, out, so,
                                 nullptr),
                 what);
  };
  plain(0, 2, 4, 32, 32, 1, "batch 0");
  plain(-1, 2, 4, 32, 32, 1, "batch -1");
  plain(1, 0, 4, 32, 32, 1, "h_qk 0");
  plain(1, 3, 4, 32, 32, 1, "h_v not a multiple of h_qk");
  plain(1, 2, 4, 48, 32, 1, "d_k 48");
  plain(1, 2, 4, 32, 4, 1, "d_v 4");
  plain(1, 2, 4, 32, 32, 3, "io_dtype 3");
  plain(INT_MAX, 64, 1024, 128, 128, 1, "batch INT_MAX, 1024 heads");
  plain(1, 2, 4, 32, 32, 1, "q NULL", nullptr);
  plain(1, 2, 4, 32, 32, 1, "g NULL", g_buf, nullptr);
  plain(1, 2, 4, 32, 32, 1, "state_in NULL", g_buf, F, nullptr);
  plain(1, 2, 4, 32, 32, 1, "out NULL", g_buf, F, F, nullptr);
  plain(1, 2, 4, 32, 32, 1, "state_out NULL", g_buf, F, F, g_buf, nullptr);

  gdn_decode_fused_params_t bad_eps{nullptr, nullptr, nullptr, -1.f, 1e-6f};
  gdn_decode_fused_params_t nan_eps{nullptr, nullptr, nullptr, 1e-6f, NAN};
  gdn_decode_fused_params_t inf_eps{nullptr, nullptr, nullptr, INFINITY, 1e-6f};
  expect_error(gdn_decode_step_fused(1, 2, 4, 32, 32, GDN_DTYPE_BF16, P, P, P, F, F, &bad_eps, F, P, FW, nullptr),
               "fused decode: qk_eps -1");
  expect_error(gdn_decode_step_fused(1, 2, 4, 32, 32, GDN_DTYPE_BF16, P, P, P, F, F, &nan_eps, F, P, FW, nullptr),
               "fused decode: norm_eps NaN");
  expect_error(gdn_decode_step_fused(1, 2, 4, 32, 32, GDN_DTYPE_BF16, P, P, P, F, F, &inf_eps, F, P, FW, nullptr),
               "fused decode: qk_eps inf");
  expect_error(gdn_decode_step_fused(0, 2, 4, 32, 32, GDN_DTYPE_BF16, P, P, P, F, F, nullptr, F, P, FW, nullptr),
               "fused decode: batch 0");
  expect_error(gdn_decode_step_fused(1, 2, 4, 32, 32, GDN_DTYPE_BF16, nullptr, P, P, F, F, nullptr, F, P, FW,
                                     nullptr),
               "fused decode: q_raw NULL");
  expect_error(gdn_decode_step_fused(1, 2, 4, 32, 32, GDN_DTYPE_BF16, P, P, P, F, F, nullptr, nullptr, P, FW,
                                     nullptr),
               "fused decode: state_in NULL");
}

void fuzz_moe() {
  const gdn_moe_shape_t ok{8, 64, 256, 256};
  const struct { gdn_moe_shape_t s; const char* defect; } bad[] = {
      {{0, 64, 256, 256}, "num_experts 0"},     {{-1, 64, 256, 256}, "num_experts -1"},
      {{8, -1, 256, 256}, "rows -1"},           {{8, 64, 100, 256}, "k 100"},
      {{8, 64, 256, 100}, "n 100"},             {{8, 64, 0, 256}, "k 0"},
      {{8, 64, 256, -128}, "n -128"},           {{INT_MAX, INT_MAX, 1 << 30, 1 << 30}, "every size near INT_MAX"},
  };
  char what[128];
  for (const auto& c : bad) {
    std::snprintf(what, sizeof what, "moe q4: %s", c.defect);
    expect_error(gdn_moe_gemm_q4(&c.s, P, I, g_buf, P, P, P, nullptr), what);
    std::snprintf(what, sizeof what, "dequant q4: %s", c.defect);
    expect_error(gdn_dequant_q4(&c.s, g_buf, P, P, P, nullptr), what);
    std::snprintf(what, sizeof what, "moe bf16: %s", c.defect);
    expect_error(gdn_moe_gemm_bf16(&c.s, P, I, P, P, nullptr), what);
    std::snprintf(what, sizeof what, "pack q4: %s", c.defect);
    expect_error(gdn_moe_pack_q4(&c.s, g_buf, g_buf2, nullptr), what);
    std::snprintf(what, sizeof what, "moe q4 packed: %s", c.defect);
    expect_error(gdn_moe_gemm_q4_packed(&c.s, P, I, g_buf, P, P, P, nullptr), what);
  }
  expect_error(gdn_moe_pack_q4(nullptr, g_buf, g_buf2, nullptr), "pack q4: shape NULL");
  expect_error(gdn_moe_pack_q4(&ok, nullptr, g_buf2, nullptr), "pack q4: codes NULL");
  expect_error(gdn_moe_pack_q4(&ok, g_buf, nullptr, nullptr), "pack q4: packed NULL");
  expect_error(gdn_moe_pack_q4(&ok, g_buf, g_buf, nullptr), "pack q4: packed equals codes");
  expect_error(gdn_moe_gemm_q4_packed(&ok, P, I, nullptr, P, P, P, nullptr), "moe q4 packed: codes NULL");
  expect_error(gdn_moe_gemm_q4_packed(&ok, P, I, g_buf, P, P, g_buf + 8, nullptr), "moe q4 packed: y misaligned");
  expect_error(gdn_moe_gemm_q4(nullptr, P, I, g_buf, P, P, P, nullptr), "moe q4: shape NULL");
  expect_error(gdn_moe_gemm_q4(&ok, nullptr, I, g_buf, P, P, P, nullptr), "moe q4: x NULL");
  expect_error(gdn_moe_gemm_q4(&ok, P, nullptr, g_buf, P, P, P, nullptr), "moe q4: offsets NULL");
  expect_error(gdn_moe_gemm_q4(&ok, P, I, nullptr, P, P, P, nullptr), "moe q4: codes NULL");
  expect_error(gdn_moe_gemm_q4(&ok, P, I, g_buf, nullptr, P, P, nullptr), "moe q4: scales NULL");
  expect_error(gdn_moe_gemm_q4(&ok, P, I, g_buf, P, nullptr, P, nullptr), "moe q4: biases NULL");
  expect_error(gdn_moe_gemm_q4(&ok, P, I, g_buf, P, P, nullptr, nullptr), "moe q4: y NULL");
  expect_error(gdn_dequant_q4(&ok, g_buf, P, P, nullptr, nullptr), "dequant q4: weights NULL");
  expect_error(gdn_moe_gemm_bf16(&ok, P, I, nullptr, P, nullptr), "moe bf16: weights NULL");
}

void fuzz_attention() {
  const gdn_attn_shape_t ok{1, 16, 2, 128, 4096};
  const gdn_attn_params_t pok{0.0884f, GDN_ATTN_AUTO, 0, 0};
  char what[128];
  const struct { gdn_attn_shape_t s; const char* defect; } bad_s[] = {
      {{0, 16, 2, 128, 4096}, "batch 0"},            {{1, 15, 2, 128, 4096}, "h_q not a multiple of h_kv"},
      {{1, 16, 0, 128, 4096}, "h_kv 0"},             {{1, 16, 2, 96, 4096}, "head_dim 96"},
      {{1, 16, 2, 128, 0}, "max_context 0"},          {{1, 16, 2, 128, (1 << 24) + 1}, "max_context past 2^24"},
      {{INT_MAX, 1 << 20, 1, 256, 1 << 24}, "every size near its limit"},
  };
  for (const auto& c : bad_s) {
    std::snprintf(what, sizeof what, "attention: %s", c.defect);
    expect_error(gdn_attention_decode(&c.s, &pok, P, P, P, I, P, P, size_t(1) << 40, nullptr), what);
    std::snprintf(what, sizeof what, "attention workspace: %s", c.defect);
    expect_zero(gdn_attention_decode_workspace(&c.s, &pok), what);
  }
  const struct { gdn_attn_params_t p; const char* defect; } bad_p[] = {
      {{NAN, GDN_ATTN_AUTO, 0, 0}, "scale NaN"},           {{INFINITY, GDN_ATTN_AUTO, 0, 0}, "scale inf"},
      {{0.1f, 5, 0, 0}, "layout 5"},                       {{0.1f, -1, 0, 0}, "layout -1"},
      {{0.1f, GDN_ATTN_AUTO, 3, 0}, "heads_per_group 3"},  {{0.1f, GDN_ATTN_AUTO, 16, 0}, "heads_per_group 16"},
      {{0.1f, GDN_ATTN_FIXED_BLOCK, 0, 5000}, "num_blocks 5000"},
      {{0.1f, GDN_ATTN_FIXED_BLOCK, 0, -1}, "num_blocks -1"},
  };
  for (const auto& c : bad_p) {
    std::snprintf(what, sizeof what, "attention: %s", c.defect);
    expect_error(gdn_attention_decode(&ok, &c.p, P, P, P, I, P, P, size_t(1) << 40, nullptr), what);
  }
  expect_error(gdn_attention_decode(nullptr, &pok, P, P, P, I, P, P, 0, nullptr), "attention: shape NULL");
  expect_error(gdn_attention_decode(&ok, nullptr, P, P, P, I, P, P, 0, nullptr), "attention: params NULL");
  expect_error(gdn_attention_decode(&ok, &pok, nullptr, P, P, I, P, P, 0, nullptr), "attention: q NULL");
  expect_error(gdn_attention_decode(&ok, &pok, P, P, P, nullptr, P, P, 0, nullptr), "attention: lens NULL");
  expect_error(gdn_attention_decode(&ok, &pok, P, P, P, I, nullptr, P, 0, nullptr), "attention: out NULL");
  const gdn_attn_params_t fixed{0.0884f, GDN_ATTN_FIXED_BLOCK, 8, 64};
  const size_t need = gdn_attention_decode_workspace(&ok, &fixed);
  ++g_checks;
  if (need == 0) {
    ++g_failures;
    std::printf("FAIL attention workspace of a valid fixed-block call returned 0\n");
  }
  expect_error(gdn_attention_decode(&ok, &fixed, P, P, P, I, P, P, need - 1, nullptr),
               "attention: workspace one byte short");
  expect_error(gdn_attention_decode(&ok, &fixed, P, P, P, I, P, nullptr, need, nullptr), "attention: workspace NULL");
  expect_zero(gdn_attention_decode_workspace(nullptr, &fixed), "attention workspace: shape NULL");
}

void fuzz_misc() {
  const int codes[] = {GDN_OK, GDN_ERR_INVALID, GDN_ERR_UNSUPPORTED, GDN_ERR_LAUNCH, 4, -1, 1 << 30};
  for (int c : codes) {
    ++g_checks;
    const char* s = gdn_status_string(static_cast<gdn_status_t>(c));
    if (s == nullptr || s[0] == '\0') {
      ++g_failures;
      std::printf("FAIL gdn_status_string(%d) is empty\n", c);
    }
  }
  ++g_checks;
  if (gdn_profile_collect(nullptr, nullptr, 0) != 0) {
    ++g_failures;
    std::printf("FAIL gdn_profile_collect with nothing recorded\n");
  }
}

}  // namespace

int main() {
  fuzz_prefill(scan, "scan");
  fuzz_prefill(blockwise, "scan_blockwise");
  fuzz_prefill(chunked, "chunked");
  fuzz_prefill(segmented, "segmented");
  fuzz_prefill(noalloc, "segmented_noalloc");
  fuzz_chunked_extras();
  fuzz_decode();
  fuzz_moe();
  fuzz_attention();
  fuzz_misc();
  std::printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
