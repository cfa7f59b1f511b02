// C ABI of libgdn.so (declared in include/gdn.h): host-side validation and
// dispatch.  Nothing here touches device memory; every check happens before
// the first launch, and a failed check enqueues nothing.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gdn_internal.hpp"

namespace {

thread_local std::string g_last_error;

gdn_status_t fail(gdn_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gdn_status_t ok() {
  g_last_error.clear();
  return GDN_OK;
}

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// The int32 an enum object of the ABI holds.  A C caller may store any int
// there, and reading a value outside the enumerators through the C++ enum
// type is undefined, so the bytes are copied instead.
template <typename E>
int32_t enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int32_t), "the ABI's enums are int-sized");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by all entry points.  Sizes are bounded so that every
// element index of the largest tensor fits in int32 arithmetic on the
// (sequence, head, row) granularity the kernels use.
gdn_status_t check_dims(int n, int t, int h_qk, int h_v, int d_k, int d_v, int32_t io, const char* what) {
  if (n < 1) return fail(GDN_ERR_INVALID, "%s: num_seqs/batch must be >= 1 (got %d)", what, n);
  if (t < 0) return fail(GDN_ERR_INVALID, "%s: total_tokens must be >= 0 (got %d)", what, t);
  if (h_qk < 1 || h_v < 1 || h_v % h_qk != 0)
    return fail(GDN_ERR_INVALID, "%s: h_v (%d) must be a positive multiple of h_qk (%d)", what, h_v, h_qk);
  if (io != GDN_DTYPE_F32 && io != GDN_DTYPE_BF16)
    return fail(GDN_ERR_INVALID, "%s: io_dtype must be GDN_DTYPE_F32 or GDN_DTYPE_BF16", what);
  if (!supported_dim(d_k) || !supported_dim(d_v))
    return fail(GDN_ERR_UNSUPPORTED, "%s: d_k=%d, d_v=%d; supported sizes are 16, 32, 64, 128", what, d_k, d_v);
  const long long rows = (long long)n * h_v * d_v;
  if (rows > (1ll << 30)) return fail(GDN_ERR_UNSUPPORTED, "%s: num_seqs * h_v * d_v too large", what);
  if ((long long)t * h_v > (1ll << 31) - 1 || (long long)t * h_qk > (1ll << 31) - 1)
    return fail(GDN_ERR_UNSUPPORTED, "%s: total_tokens * heads exceeds int32", what);
  return GDN_OK;
}

gdn_status_t check_ptrs(const char* what, std::initializer_list<std::pair<const char*, const void*>> ps) {
  for (auto& p : ps) {
    if (!p.second) return fail(GDN_ERR_INVALID, "%s: %s is NULL", what, p.first);
    if (!aligned16(p.second)) return fail(GDN_ERR_INVALID, "%s: %s is not 16-byte aligned", what, p.first);
  }
  return GDN_OK;
}

gdn_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

gdn::Dims dims_of(const gdn_shape_t* s) {
  return gdn::Dims{s->num_seqs, s->total_tokens, s->h_qk, s->h_v, s->d_k, s->d_v,
                   enum_bits(s->io_dtype) == GDN_DTYPE_BF16};
}

gdn_status_t check_prefill(const gdn_shape_t* s, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu, const float* state_in, const void* out,
                           const float* state_out, const char* what) {
  if (!s) return fail(GDN_ERR_INVALID, "%s: shape is NULL", what);
  gdn_status_t st =
      check_dims(s->num_seqs, s->total_tokens, s->h_qk, s->h_v, s->d_k, s->d_v, enum_bits(s->io_dtype), what);
  if (st != GDN_OK) return st;
  // with no tokens the per-token tensors are never read or written and may be NULL
  if (s->total_tokens > 0) {
    st = check_ptrs(what, {{"q", q}, {"k", k}, {"v", v}, {"g", g}, {"beta", beta}, {"out", out}});
    if (st != GDN_OK) return st;
  } else {
    for (const void* p : {q, k, v, static_cast<const void*>(g), static_cast<const void*>(beta), out})
      if (p && !aligned16(p)) return fail(GDN_ERR_INVALID, "%s: a token tensor is not 16-byte aligned", what);
  }
  st = check_ptrs(what, {{"cu_seqlens", cu}, {"state_out", state_out}});
  if (st != GDN_OK) return st;
  if (state_in && !aligned16(state_in)) return fail(GDN_ERR_INVALID, "%s: state_in is not 16-byte aligned", what);
  if (out && (out == q || out == k || out == v || out == state_in || out == state_out))
    return fail(GDN_ERR_INVALID, "%s: out aliases another tensor", what);
  return GDN_OK;
}

// ---------------------------------------------------------------- profiling
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfRecord> g_prof;

}  // namespace

namespace gdn {

Prof::Prof(const char* name, hipStream_t st) : name_(name), st_(st) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  if (hipEventCreate(&start_) != hipSuccess) {
    start_ = nullptr;
    return;
  }
  if (hipEventRecord(start_, st_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    start_ = nullptr;
  }
}

Prof::~Prof() {
  if (!start_) return;
  hipEvent_t stop = nullptr;
  if (hipEventCreate(&stop) != hipSuccess || hipEventRecord(stop, st_) != hipSuccess) {
    if (stop) (void)hipEventDestroy(stop);
    (void)hipEventDestroy(start_);
    return;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({name_, start_, stop});
}

}  // namespace gdn

extern "C" {

gdn_status_t gdn_profile_enable(int enabled) {
  g_prof_on.store(enabled != 0);
  return ok();
}

int gdn_profile_collect(const char** names, float* ms, int cap) {
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof);
  }
  int n = int(recs.size()), rc = n;
  for (int i = 0; i < n; ++i) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, recs[i].start, recs[i].stop) != hipSuccess) rc = -1;
    if (i < cap) {
      if (names) names[i] = recs[i].name;
      if (ms) ms[i] = t;
    }
    (void)hipEventDestroy(recs[i].start);
    (void)hipEventDestroy(recs[i].stop);
  }
  return rc;
}


const char* gdn_status_string(gdn_status_t status) {
  switch (enum_bits(status)) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID: return "GDN_ERR_INVALID";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH";
  }
  return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

gdn_status_t gdn_prefill_scan(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const int32_t* cu_seqlens,
                              const float* state_in, void* out, float* state_out, void* stream) {
  gdn_status_t st =
      check_prefill(shape, q, k, v, g, beta, cu_seqlens, state_in, out, state_out, "gdn_prefill_scan");
  if (st != GDN_OK) return st;
  return launched(gdn::launch_scan(dims_of(shape), q, k, v, g, beta, cu_seqlens, state_in, out, state_out,
                                   static_cast<hipStream_t>(stream)),
                  "gdn_prefill_scan");
}

gdn_status_t gdn_prefill_scan_blockwise(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                                        const float* g, const float* beta, const int32_t* cu_seqlens,
                                        const float* state_in, void* out, float* state_out, int32_t state_block,
                                        void* stream) {
  const char* what = "gdn_prefill_scan_blockwise";
  gdn_status_t st = check_prefill(shape, q, k, v, g, beta, cu_seqlens, state_in, out, state_out, what);
  if (st != GDN_OK) return st;
  if (state_block < 1 || state_block % 4 != 0)
    return fail(GDN_ERR_INVALID, "%s: state_block must be a positive multiple of 4 (got %d)", what, state_block);
  return launched(gdn::launch_scan(dims_of(shape), q, k, v, g, beta, cu_seqlens, state_in, out, state_out,
                                   static_cast<hipStream_t>(stream), state_block),
                  what);
}

size_t gdn_prefill_chunked_workspace(const gdn_shape_t* shape, int32_t chunk_size) {
  if (!shape || (chunk_size != 16 && chunk_size != 32 && chunk_size != 64)) return 0;
  if (check_dims(shape->num_seqs, shape->total_tokens, shape->h_qk, shape->h_v, shape->d_k, shape->d_v,
                 enum_bits(shape->io_dtype), "gdn_prefill_chunked_workspace") != GDN_OK)
    return 0;
  return gdn::chunked_workspace_bytes(dims_of(shape), chunk_size);
}

gdn_status_t gdn_prefill_chunked(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const int32_t* cu_seqlens,
                                 const float* state_in, void* out, float* state_out, int32_t chunk_size,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "gdn_prefill_chunked";
  gdn_status_t st = check_prefill(shape, q, k, v, g, beta, cu_seqlens, state_in, out, state_out, what);
  if (st != GDN_OK) return st;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
    return fail(GDN_ERR_UNSUPPORTED, "%s: chunk_size %d; supported sizes are 16, 32, 64", what, chunk_size);
  const gdn::Dims d = dims_of(shape);
  // the prep runs one workgroup per (chunk, value head), indexed in int
  if (gdn::chunked_max_chunks(d, chunk_size) * size_t(d.h_v) > size_t(1u << 31) - 8)
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many chunks", what);
  const size_t need = gdn::chunked_workspace_bytes(d, chunk_size);
  if (!workspace) return fail(GDN_ERR_INVALID, "%s: workspace is NULL", what);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GDN_ERR_INVALID, "%s: workspace is not 256-byte aligned", what);
  if (workspace_bytes < need)
    return fail(GDN_ERR_INVALID, "%s: workspace has %zu bytes, needs %zu", what, workspace_bytes, need);
  return launched(gdn::launch_chunked(d, chunk_size, q, k, v, g, beta, cu_seqlens, state_in, out, state_out,
                                      workspace, static_cast<hipStream_t>(stream)),
                  what);
}

size_t gdn_prefill_segmented_workspace(const gdn_shape_t* shape, int32_t chunk_size, int32_t segment_tokens) {
  if (!shape || (chunk_size != 0 && chunk_size != 16 && chunk_size != 32 && chunk_size != 64)) return 0;
  if (segment_tokens < 1 || (chunk_size > 0 && segment_tokens % chunk_size != 0)) return 0;
  if (check_dims(shape->num_seqs, shape->total_tokens, shape->h_qk, shape->h_v, shape->d_k, shape->d_v,
                 enum_bits(shape->io_dtype), "gdn_prefill_segmented_workspace") != GDN_OK)
    return 0;
  return gdn::segmented_workspace_bytes(dims_of(shape), chunk_size, segment_tokens);
}

namespace {
// Checks shared by the segmented prefill and its allocation-free variant.
gdn_status_t check_segmented(const gdn_shape_t* shape, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, const float* state_in, const void* out,
                             const float* state_out, int32_t chunk_size, int32_t segment_tokens, const char* what) {
  gdn_status_t st = check_prefill(shape, q, k, v, g, beta, cu_seqlens, state_in, out, state_out, what);
  if (st != GDN_OK) return st;
  if (chunk_size != 0 && chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
    return fail(GDN_ERR_UNSUPPORTED, "%s: chunk_size %d; supported are 0 (direct scan), 16, 32, 64", what,
                chunk_size);
  if (segment_tokens < 1) return fail(GDN_ERR_INVALID, "%s: segment_tokens must be >= 1", what);
  if (chunk_size > 0 && segment_tokens % chunk_size != 0)
    return fail(GDN_ERR_INVALID, "%s: segment_tokens (%d) must be a multiple of chunk_size (%d)", what,
                segment_tokens, chunk_size);
  const gdn::Dims d = dims_of(shape);
  if (chunk_size > 0) {
    gdn::Dims dw = d;
    dw.total_tokens = d.total_tokens < segment_tokens ? d.total_tokens : segment_tokens;
    if (gdn::chunked_max_chunks(dw, chunk_size) * size_t(d.h_v) > size_t(1u << 31) - 8)
      return fail(GDN_ERR_UNSUPPORTED, "%s: too many chunks per segment", what);
  }
  return GDN_OK;
}
}  // namespace

gdn_status_t gdn_prefill_segmented(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const int32_t* cu_seqlens,
                                   const float* state_in, void* out, float* state_out, int32_t chunk_size,
                                   int32_t segment_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "gdn_prefill_segmented";
  gdn_status_t st = check_segmented(shape, q, k, v, g, beta, cu_seqlens, state_in, out, state_out, chunk_size,
                                    segment_tokens, what);
  if (st != GDN_OK) return st;
  const gdn::Dims d = dims_of(shape);
  const size_t need = gdn::segmented_workspace_bytes(d, chunk_size, segment_tokens);
  if (!workspace) return fail(GDN_ERR_INVALID, "%s: workspace is NULL", what);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GDN_ERR_INVALID, "%s: workspace is not 256-byte aligned", what);
  if (workspace_bytes < need)
    return fail(GDN_ERR_INVALID, "%s: workspace has %zu bytes, needs %zu", what, workspace_bytes, need);
  return launched(gdn::launch_segmented(d, chunk_size, segment_tokens, q, k, v, g, beta, cu_seqlens, state_in, out,
                                        state_out, workspace, static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_prefill_segmented_noalloc(const gdn_shape_t* shape, const void* q, const void* k, const void* v,
                                           const float* g, const float* beta, const int32_t* cu_seqlens,
                                           const float* state_in, void* out, float* state_out, int32_t chunk_size,
                                           int32_t segment_tokens, void* stream) {
  const char* what = "gdn_prefill_segmented_noalloc";
  gdn_status_t st = check_segmented(shape, q, k, v, g, beta, cu_seqlens, state_in, out, state_out, chunk_size,
                                    segment_tokens, what);
  if (st != GDN_OK) return st;
  const gdn::Dims d = dims_of(shape);
  const size_t need = gdn::segmented_workspace_bytes(d, chunk_size, segment_tokens);
  if (need > size_t(GDN_STATIC_SCRATCH_BYTES))
    return fail(GDN_ERR_INVALID,
                "%s: these shapes need %zu bytes of scratch per segment of %d tokens; the static scratch holds %zu "
                "(use fewer segment_tokens)",
                what, need, segment_tokens, size_t(GDN_STATIC_SCRATCH_BYTES));
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  hipError_t e = gdn::static_scratch(&scratch, &scratch_bytes);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s: static scratch address: %s", what, hipGetErrorString(e));
  if (scratch_bytes < need) return fail(GDN_ERR_INVALID, "%s: static scratch too small", what);
  return launched(gdn::launch_segmented(d, chunk_size, segment_tokens, q, k, v, g, beta, cu_seqlens, state_in, out,
                                        state_out, scratch, static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_decode_step(int32_t batch, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                             gdn_dtype_t io_dtype, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* state_in, void* out, float* state_out,
                             void* stream) {
  const char* what = "gdn_decode_step";
  gdn_status_t st = check_dims(batch, batch, h_qk, h_v, d_k, d_v, enum_bits(io_dtype), what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"q", q}, {"k", k}, {"v", v}, {"g", g}, {"beta", beta}, {"state_in", state_in},
                         {"out", out}, {"state_out", state_out}});
  if (st != GDN_OK) return st;
  if (out == q || out == k || out == v || out == state_in || out == state_out)
    return fail(GDN_ERR_INVALID, "%s: out aliases another tensor", what);
  const gdn::Dims d{batch, batch, h_qk, h_v, d_k, d_v, enum_bits(io_dtype) == GDN_DTYPE_BF16};
  return launched(gdn::launch_decode(d, q, k, v, g, beta, state_in, out, state_out,
                                     static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_decode_step_fused(int32_t batch, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                                   gdn_dtype_t io_dtype, const void* q_raw, const void* k_raw, const void* v,
                                   const float* g_raw, const float* beta_raw,
                                   const gdn_decode_fused_params_t* params, const float* state_in, void* out,
                                   float* state_out, void* stream) {
  const char* what = "gdn_decode_step_fused";
  gdn_status_t st = check_dims(batch, batch, h_qk, h_v, d_k, d_v, enum_bits(io_dtype), what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"q_raw", q_raw}, {"k_raw", k_raw}, {"v", v}, {"g_raw", g_raw}, {"beta_raw", beta_raw},
                         {"state_in", state_in}, {"out", out}, {"state_out", state_out}});
  if (st != GDN_OK) return st;
  if (out == q_raw || out == k_raw || out == v || out == state_in || out == state_out)
    return fail(GDN_ERR_INVALID, "%s: out aliases another tensor", what);
  gdn_decode_fused_params_t p{nullptr, nullptr, nullptr, 1e-6f, 1e-6f};
  if (params) p = *params;
  for (const void* a : {static_cast<const void*>(p.gate_bias), static_cast<const void*>(p.gate_scale),
                        static_cast<const void*>(p.norm_weight)})
    if (a && (reinterpret_cast<uintptr_t>(a) & 3u) != 0)
      return fail(GDN_ERR_INVALID, "%s: gate_bias, gate_scale and norm_weight must be 4-byte aligned", what);
  if (!(p.qk_eps >= 0.f && p.qk_eps <= 3.0e38f) || !(p.norm_eps >= 0.f && p.norm_eps <= 3.0e38f))
    return fail(GDN_ERR_INVALID, "%s: qk_eps and norm_eps must be finite and >= 0", what);
  const gdn::Dims d{batch, batch, h_qk, h_v, d_k, d_v, enum_bits(io_dtype) == GDN_DTYPE_BF16};
  return launched(gdn::launch_decode_fused(d, q_raw, k_raw, v, g_raw, beta_raw, p.gate_bias, p.gate_scale,
                                           p.norm_weight, p.qk_eps, p.norm_eps, state_in, out, state_out,
                                           static_cast<hipStream_t>(stream)),
                  what);
}

static gdn_status_t check_moe(const gdn_moe_shape_t* s, const char* what) {
  if (!s) return fail(GDN_ERR_INVALID, "%s: shape is NULL", what);
  if (s->num_experts < 1) return fail(GDN_ERR_INVALID, "%s: num_experts must be >= 1", what);
  if (s->num_experts > 4096) return fail(GDN_ERR_UNSUPPORTED, "%s: at most 4096 experts", what);
  if (s->rows < 0) return fail(GDN_ERR_INVALID, "%s: rows must be >= 0", what);
  if (s->k < 128 || s->k % 128 != 0)
    return fail(GDN_ERR_UNSUPPORTED, "%s: k (%d) must be a positive multiple of 128", what, s->k);
  if (s->n < 128 || s->n % 128 != 0)
    return fail(GDN_ERR_UNSUPPORTED, "%s: n (%d) must be a positive multiple of 128", what, s->n);
  // the grid: one workgroup per (64-row block slot, 128-column block)
  const long long slots = (((long long)s->rows + (long long)s->num_experts * 63) / 64 + 7) / 8 * 8;
  if (slots * (s->n / 128) > (1ll << 31) - 1)
    return fail(GDN_ERR_UNSUPPORTED, "%s: (rows + 63 num_experts) / 64 (rounded up to 8) * n / 128 exceeds int32",
                what);
  if ((long long)s->rows * s->k > (1ll << 31) - 1 || (long long)s->rows * s->n > (1ll << 40))
    return fail(GDN_ERR_UNSUPPORTED, "%s: rows * k must stay below 2^31", what);
  return GDN_OK;
}

gdn_status_t gdn_moe_gemm_q4(const gdn_moe_shape_t* shape, const void* x, const int32_t* expert_offsets,
                             const uint8_t* codes, const void* scales, const void* biases, void* y, void* stream) {
  const char* what = "gdn_moe_gemm_q4";
  gdn_status_t st = check_moe(shape, what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"expert_offsets", expert_offsets}, {"codes", codes}, {"scales", scales},
                         {"biases", biases}});
  if (st != GDN_OK) return st;
  if (shape->rows > 0) {
    st = check_ptrs(what, {{"x", x}, {"y", y}});
    if (st != GDN_OK) return st;
    if (y == x) return fail(GDN_ERR_INVALID, "%s: y aliases x", what);
  }
  return launched(gdn::launch_moe_gemm(shape->num_experts, shape->rows, shape->n, shape->k, x, expert_offsets, codes,
                                       scales, biases, y, true, false, static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_moe_pack_q4(const gdn_moe_shape_t* shape, const uint8_t* codes, uint8_t* packed, void* stream) {
  const char* what = "gdn_moe_pack_q4";
  gdn_status_t st = check_moe(shape, what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"codes", codes}, {"packed", packed}});  // non-NULL, 16-byte aligned
  if (st != GDN_OK) return st;
  const size_t bytes = size_t(shape->num_experts) * size_t(shape->n) * size_t(shape->k / 2);
  const uintptr_t a = reinterpret_cast<uintptr_t>(codes), b = reinterpret_cast<uintptr_t>(packed);
  if (a < b + bytes && b < a + bytes) return fail(GDN_ERR_INVALID, "%s: packed overlaps codes", what);
  return launched(gdn::launch_pack_q4(shape->num_experts, shape->n, shape->k, codes, packed,
                                      static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_moe_gemm_q4_packed(const gdn_moe_shape_t* shape, const void* x, const int32_t* expert_offsets,
                                    const uint8_t* packed_codes, const void* scales, const void* biases, void* y,
                                    void* stream) {
  const char* what = "gdn_moe_gemm_q4_packed";
  gdn_status_t st = check_moe(shape, what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"expert_offsets", expert_offsets}, {"packed_codes", packed_codes}, {"scales", scales},
                         {"biases", biases}});
  if (st != GDN_OK) return st;
  if (shape->rows > 0) {
    st = check_ptrs(what, {{"x", x}, {"y", y}});
    if (st != GDN_OK) return st;
    if (y == x) return fail(GDN_ERR_INVALID, "%s: y aliases x", what);
  }
  return launched(gdn::launch_moe_gemm(shape->num_experts, shape->rows, shape->n, shape->k, x, expert_offsets,
                                       packed_codes, scales, biases, y, true, true, static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_dequant_q4(const gdn_moe_shape_t* shape, const uint8_t* codes, const void* scales,
                            const void* biases, void* weights, void* stream) {
  const char* what = "gdn_dequant_q4";
  gdn_status_t st = check_moe(shape, what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"codes", codes}, {"scales", scales}, {"biases", biases}, {"weights", weights}});
  if (st != GDN_OK) return st;
  return launched(gdn::launch_dequant_q4(shape->num_experts, shape->n, shape->k, codes, scales, biases, weights,
                                         static_cast<hipStream_t>(stream)),
                  what);
}

gdn_status_t gdn_moe_gemm_bf16(const gdn_moe_shape_t* shape, const void* x, const int32_t* expert_offsets,
                               const void* weights, void* y, void* stream) {
  const char* what = "gdn_moe_gemm_bf16";
  gdn_status_t st = check_moe(shape, what);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"expert_offsets", expert_offsets}, {"weights", weights}});
  if (st != GDN_OK) return st;
  if (shape->rows > 0) {
    st = check_ptrs(what, {{"x", x}, {"y", y}});
    if (st != GDN_OK) return st;
    if (y == x) return fail(GDN_ERR_INVALID, "%s: y aliases x", what);
  }
  return launched(gdn::launch_moe_gemm(shape->num_experts, shape->rows, shape->n, shape->k, x, expert_offsets,
                                       weights, nullptr, nullptr, y, false, false, static_cast<hipStream_t>(stream)),
                  what);
}

// ---------------------------------------------------------------- decode attention
struct AttnPlan {
  gdn::AttnDims d;
  float scale;
  bool fixed_block;
  int hp, nb;
};

// Compute units of the current device (256 on MI355X, also the fallback).
static int device_cu_count() {
  static std::atomic<int> cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 16) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 16) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static gdn_status_t attn_plan(const gdn_attn_shape_t* s, const gdn_attn_params_t* p, const char* what,
                              AttnPlan& plan) {
  if (!s) return fail(GDN_ERR_INVALID, "%s: shape is NULL", what);
  if (s->batch < 1) return fail(GDN_ERR_INVALID, "%s: batch must be >= 1", what);
  if (s->h_kv < 1 || s->h_q < s->h_kv || s->h_q % s->h_kv != 0)
    return fail(GDN_ERR_INVALID, "%s: h_q (%d) must be a positive multiple of h_kv (%d)", what, s->h_q, s->h_kv);
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256)
    return fail(GDN_ERR_UNSUPPORTED, "%s: head_dim %d; supported sizes are 64, 128, 256", what, s->head_dim);
  if (s->max_context < 1 || s->max_context > (1 << 24))
    return fail(GDN_ERR_INVALID, "%s: max_context must be in [1, 2^24] (got %d)", what, s->max_context);
  if ((long long)s->batch * s->h_q > (1ll << 24))
    return fail(GDN_ERR_UNSUPPORTED, "%s: batch * h_q too large", what);
  gdn_attn_params_t d{1.0f / std::sqrt(float(s->head_dim)), GDN_ATTN_AUTO, 0, 0};
  if (p) d = *p;
  if (!std::isfinite(d.scale)) return fail(GDN_ERR_INVALID, "%s: scale must be finite", what);
  const int group = s->h_q / s->h_kv;
  int hp = d.heads_per_group;
  if (hp == 0) {
    hp = 8;
    while (group % hp) hp /= 2;
  } else if ((hp != 1 && hp != 2 && hp != 4 && hp != 8) || group % hp) {
    return fail(GDN_ERR_INVALID, "%s: heads_per_group %d must be 0, or 1, 2, 4 or 8 dividing h_q / h_kv = %d",
                what, d.heads_per_group, group);
  }
  const long long base = (long long)s->batch * s->h_kv * (group / hp);
  // automatic part count: one workgroup per compute unit, parts of at least 32 positions
  const long long n_cu = device_cu_count();
  const int nb_auto = int(std::max(1ll, std::min({(n_cu + base - 1) / base, (s->max_context + 31ll) / 32, 4096ll})));
  bool fixed;
  switch (d.layout) {
    case GDN_ATTN_GENERAL: fixed = false; break;
    case GDN_ATTN_FIXED_BLOCK: fixed = true; break;
    case GDN_ATTN_AUTO: fixed = nb_auto > 1; break;
    default: return fail(GDN_ERR_INVALID, "%s: layout %d is not a gdn_attn_layout_t", what, d.layout);
  }
  int nb = 1;
  if (fixed) {
    if (d.num_blocks < 0 || d.num_blocks > std::min(s->max_context, 4096))
      return fail(GDN_ERR_INVALID, "%s: num_blocks must be in [0, min(max_context, 4096)] (got %d)", what,
                  d.num_blocks);
    nb = d.num_blocks > 0 ? d.num_blocks : nb_auto;
  }
  if (base * nb > (1ll << 31) - 1) return fail(GDN_ERR_UNSUPPORTED, "%s: too many workgroups", what);
  plan.d = gdn::AttnDims{s->batch, s->h_q, s->h_kv, s->head_dim, s->max_context};
  plan.scale = d.scale;
  plan.fixed_block = fixed;
  plan.hp = hp;
  plan.nb = nb;
  return GDN_OK;
}

size_t gdn_attention_decode_workspace(const gdn_attn_shape_t* shape, const gdn_attn_params_t* params) {
  AttnPlan plan;
  if (attn_plan(shape, params, "gdn_attention_decode_workspace", plan) != GDN_OK) return 0;
  return plan.fixed_block ? gdn::attn_workspace_bytes(plan.d, plan.nb) : 0;
}

gdn_status_t gdn_attention_decode(const gdn_attn_shape_t* shape, const gdn_attn_params_t* params, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* context_lens, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "gdn_attention_decode";
  AttnPlan plan;
  gdn_status_t st = attn_plan(shape, params, what, plan);
  if (st != GDN_OK) return st;
  st = check_ptrs(what, {{"q", q}, {"k_cache", k_cache}, {"v_cache", v_cache}, {"out", out}});
  if (st != GDN_OK) return st;
  if (!context_lens) return fail(GDN_ERR_INVALID, "%s: context_lens is NULL", what);
  if (reinterpret_cast<uintptr_t>(context_lens) & 3u)
    return fail(GDN_ERR_INVALID, "%s: context_lens is not 4-byte aligned", what);
  if (out == q || out == k_cache || out == v_cache || out == context_lens)
    return fail(GDN_ERR_INVALID, "%s: out aliases an input", what);
  if (plan.fixed_block) {
    const size_t need = gdn::attn_workspace_bytes(plan.d, plan.nb);
    if (!workspace) return fail(GDN_ERR_INVALID, "%s: workspace is NULL", what);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(GDN_ERR_INVALID, "%s: workspace is not 256-byte aligned", what);
    if (workspace_bytes < need)
      return fail(GDN_ERR_INVALID, "%s: workspace has %zu bytes, needs %zu", what, workspace_bytes, need);
  }
  return launched(gdn::launch_attn_decode(plan.d, plan.scale, plan.fixed_block, plan.hp, plan.nb, q, k_cache,
                                          v_cache, context_lens, out, workspace, static_cast<hipStream_t>(stream)),
                  what);
}

}  // extern "C"
