// Host-side launcher declarations shared by the C ABI (gdn_api.cpp) and the
// kernel translation units.  Every launcher assumes its arguments were
// validated by the caller and only enqueues work on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Optional per-kernel timing: while profiling is enabled, a Prof object
// records a hipEvent on `st` when constructed and another when destroyed, so
// a launch placed between the two is timed on its own stream.
class Prof {
 public:
  Prof(const char* name, hipStream_t st);
  ~Prof();
  Prof(const Prof&) = delete;
  Prof& operator=(const Prof&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  hipEvent_t start_ = nullptr;
};

struct Dims {
  int num_seqs, total_tokens, h_qk, h_v, d_k, d_v;
  bool bf16;  // io dtype: bf16 if true, fp32 otherwise
};

// Decode: `batch` sequences, one token each.
hipError_t launch_decode(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* s_in, void* out, float* s_out, hipStream_t st);

// Decode with the q/k L2 norms, the gate and beta activations and the
// per-head RMS output norm folded in; gate_bias, gate_scale and norm_weight
// may be null.
hipError_t launch_decode_fused(const Dims& d, const void* q, const void* k, const void* v, const float* g_raw,
                               const float* b_raw, const float* gate_bias, const float* gate_scale,
                               const float* norm_weight, float qk_eps, float norm_eps, const float* s_in,
                               void* out, float* s_out, hipStream_t st);

// Prefill by direct token scan.  sblock > 0 builds the blockwise ablation:
// the state goes to s_out and back every sblock tokens.
hipError_t launch_scan(const Dims& d, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const int32_t* cu, const float* s_in, void* out, float* s_out,
                       hipStream_t st, int sblock = 0);

// Chunked prefill: workspace layout and the three launches.
size_t chunked_max_chunks(const Dims& d, int chunk);
size_t chunked_workspace_bytes(const Dims& d, int chunk);
hipError_t launch_chunked(const Dims& d, int chunk, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const int32_t* cu, const float* s_in, void* out,
                          float* s_out, void* workspace, hipStream_t st);

// Prefill in windows of L packed tokens with the state carried through
// s_out; chunk 0 selects the direct scan.  The workspace holds the window's
// offsets and, for the chunked path, one window's chunked workspace.
size_t segmented_workspace_bytes(const Dims& d, int chunk, int L);
hipError_t launch_segmented(const Dims& d, int chunk, int L, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const int32_t* cu, const float* s_in, void* out,
                            float* s_out, void* workspace, hipStream_t st);

// Device address and size of the static scratch array on the current device
// (taken once per device; the array lives in gdn_noalloc.hip).
hipError_t static_scratch(void** ptr, size_t* bytes);

// Grouped expert GEMM: y[r] = W_e x[r] over expert row groups; q4 selects
// 4-bit group-affine weights rebuilt in the kernel, else bf16 weights;
// packed, codes in the layout launch_pack_q4 writes.
hipError_t launch_moe_gemm(int n_exp, int m, int n, int k, const void* x, const int32_t* offsets,
                           const void* weights, const void* scales, const void* biases, void* y, bool q4,
                           bool packed, hipStream_t st);
// 4-bit codes [E, N, K / 2] rewritten in 1 KiB (16-row, 128-k) tiles.
hipError_t launch_pack_q4(int n_exp, int n, int k, const void* codes, void* packed, hipStream_t st);
// The whole bf16 weight matrix [E, N, K] from 4-bit codes.
hipError_t launch_dequant_q4(int n_exp, int n, int k, const void* codes, const void* scales, const void* biases,
                             void* w, hipStream_t st);

// Decode attention over a grouped-query KV cache: hp query heads per
// workgroup; the fixed-block layout splits each context into nb equal parts
// whose partial results go to the workspace and are merged by a second kernel.
struct AttnDims {
  int batch, h_q, h_kv, head_dim, t_max;
};
size_t attn_workspace_bytes(const AttnDims& d, int nb);
hipError_t launch_attn_decode(const AttnDims& d, float scale, bool fixed_block, int hp, int nb, const void* q,
                              const void* k, const void* v, const int32_t* lens, void* out, void* workspace,
                              hipStream_t st);

}  // namespace gdn
