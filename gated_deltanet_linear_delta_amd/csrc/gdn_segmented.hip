// Prefill of a long packed batch in bounded token windows.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// "Bounding scratch memory by chunking the prompt": a long prompt is run as a
// sequence of bounded segments instead of keeping temporaries for every token
// at once; the recurrent state carries the context from one segment to the
// next, so the output does not change, and peak scratch memory is set by the
// segment, not by the prompt.
//
// Here the packed tokens [0, T) are cut into windows of L tokens.  Within a
// window each sequence's tokens form a (possibly empty) sub-sequence:
// cu_w[n] = clamp(cu[n], w0, w1) - w0, computed on the device so cu_seqlens
// never leaves it.  The window runs through the chunked path (or the direct
// scan) with the inputs offset by w0 tokens; its state comes from state_in
// for the first window and from state_out, in place, afterwards.  Sequences
// absent from a window keep their state (the kernels skip an in-place copy).
// The chunked workspace is sized for one window and reused by every window,
// in stream order.
#include <algorithm>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

__global__ __launch_bounds__(256) void window_offsets_kernel(int N, int T, int w0, int w1,
                                                             const int32_t* __restrict__ cu, int32_t* __restrict__ cu_w) {
  for (int n = threadIdx.x; n <= N; n += 256) {
    int c = cu[n];
    c = c < 0 ? 0 : (c > T ? T : c);
    c = c < w0 ? w0 : (c > w1 ? w1 : c);
    cu_w[n] = c - w0;
  }
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

static Dims window_dims(const Dims& d, int L) {
  Dims w = d;
  w.total_tokens = std::min(d.total_tokens, L);
  return w;
}

size_t segmented_workspace_bytes(const Dims& d, int chunk, int L) {
  const size_t offs = round256(size_t(d.num_seqs + 1) * sizeof(int32_t));
  return offs + (chunk > 0 ? chunked_workspace_bytes(window_dims(d, L), chunk) : 0);
}

hipError_t launch_segmented(const Dims& d, int chunk, int L, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const int32_t* cu, const float* s_in, void* out,
                            float* s_out, void* workspace, hipStream_t st) {
  const size_t esz = d.bf16 ? 2 : 4;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  int32_t* cu_w = reinterpret_cast<int32_t*>(base);
  void* chunk_ws = base + round256(size_t(d.num_seqs + 1) * sizeof(int32_t));
  int w0 = 0;
  do {  // at least one window, so that T = 0 still writes state_out
    const int w1 = int(std::min<long long>(d.total_tokens, (long long)w0 + L));
    {
      Prof prof("window_offsets", st);
      hipLaunchKernelGGL(window_offsets_kernel, dim3(1), dim3(256), 0, st, d.num_seqs, d.total_tokens, w0, w1, cu,
                         cu_w);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    Dims dw = d;
    dw.total_tokens = w1 - w0;
    const size_t tq = size_t(w0) * d.h_qk * d.d_k * esz, tv = size_t(w0) * d.h_v * d.d_v * esz;
    const size_t tg = size_t(w0) * d.h_v;
    const void* qw = static_cast<const uint8_t*>(q) + tq;
    const void* kw = static_cast<const uint8_t*>(k) + tq;
    const void* vw = static_cast<const uint8_t*>(v) + tv;
    void* ow = static_cast<uint8_t*>(out) + tv;
    const float* sw = w0 == 0 ? s_in : s_out;
    e = chunk > 0 ? launch_chunked(dw, chunk, qw, kw, vw, g + tg, beta + tg, cu_w, sw, ow, s_out, chunk_ws, st)
                  : launch_scan(dw, qw, kw, vw, g + tg, beta + tg, cu_w, sw, ow, s_out, st);
    if (e != hipSuccess) return e;
    w0 = w1;
  } while (w0 < d.total_tokens);
  return hipSuccess;
}

}  // namespace gdn
