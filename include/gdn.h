/*
 * gdn.h -- C ABI of libgdn.so: the gated delta rule on MI355X (gfx950).
 *
 * The operation.  Perplexity, "Optimizing on-device inference for Apple
 * Silicon", section "Qwen creates three distinct workload shapes", describes a
 * Gated DeltaNet layer: a fixed-size recurrent state per head, a learned gate
 * that decides how much of the old state is kept, and a delta update from the
 * current token, each token depending on the previous state; prefill walks the
 * tokens directly or regroups them into blocks.  Section "Keeping the
 * recurrent state on chip" fixes the precisions: state and gate fp32, query
 * and key activations bf16.  The recurrence computed here, per sequence and
 * per value head h, is the gated delta rule
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with S a d_v x d_k fp32 matrix.  Value head h reads query/key head
 * h / (h_v / h_qk) (contiguous groups).  Apart from gdn_decode_step_fused
 * (below), the library applies no softplus, sigmoid, normalisation or scaling
 * to q, k, v, g or beta: callers pass g as the log of the decay (finite,
 * normally <= 0) and beta as the write strength.
 *
 * Conventions shared by every entry point.
 *  - All tensor pointers are DEVICE pointers allocated and owned by the
 *    caller; the library never allocates or frees device memory and keeps no
 *    pointer after returning.  (The one device buffer of its own is the
 *    static scratch array of gdn_prefill_segmented_noalloc, which comes with
 *    the library's code on each device.)  Layouts are dense row-major, last index
 *    fastest:
 *        q, k        [T, h_qk, d_k]        io_dtype
 *        v, out      [T, h_v,  d_v]        io_dtype
 *        g, beta     [T, h_v]              fp32
 *        cu_seqlens  [num_seqs + 1]        int32, cu[0] = 0, cu[N] = T,
 *                                          non-decreasing (zero-length
 *                                          sequences allowed)
 *        state_in,
 *        state_out   [num_seqs, h_v, d_v, d_k]  fp32 (d_k fastest)
 *    Pointers must be 16-byte aligned.  When total_tokens is 0, q, k, v, g,
 *    beta and out are not accessed and may be NULL.
 *  - state_in may be NULL (zero initial state).  state_out may be the same
 *    pointer as state_in (in place); no other output may alias any input.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    runs asynchronously.  A call returns after validating its arguments on
 *    the host and enqueueing kernels; it never synchronises the device.
 *  - Errors: arguments are checked on the host before anything is enqueued;
 *    on failure the call returns GDN_ERR_INVALID or GDN_ERR_UNSUPPORTED and
 *    enqueues nothing.  cu_seqlens lives on the device and its contents are
 *    not checked on the host; kernels clamp every offset to [0, T], so a
 *    malformed cu_seqlens gives meaningless results but no out-of-bounds
 *    access.  A launch failure returns GDN_ERR_LAUNCH.  gdn_last_error()
 *    gives a message for the last failing call on the calling thread.
 *  - Supported sizes: d_k, d_v in {16, 32, 64, 128}; h_v a positive multiple
 *    of h_qk.  Results are deterministic (no atomics).
 *  - Outputs in bf16 are rounded to nearest even from fp32.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID = 1,     /* null pointer, bad shape, misalignment, workspace too small */
  GDN_ERR_UNSUPPORTED = 2, /* well-formed but outside the built sizes (d_k, d_v, chunk) */
  GDN_ERR_LAUNCH = 3       /* the HIP runtime reported an error while enqueueing */
} gdn_status_t;

typedef enum {
  GDN_DTYPE_F32 = 0,  /* q, k, v, out in fp32 */
  GDN_DTYPE_BF16 = 1  /* q, k, v, out in bf16 */
} gdn_dtype_t;

typedef struct {
  int32_t num_seqs;     /* N >= 1 packed sequences */
  int32_t total_tokens; /* T = cu_seqlens[N] >= 0 */
  int32_t h_qk;         /* query/key heads, >= 1 */
  int32_t h_v;          /* value heads, a multiple of h_qk */
  int32_t d_k;          /* key dimension: 16, 32, 64 or 128 */
  int32_t d_v;          /* value dimension: 16, 32, 64 or 128 */
  gdn_dtype_t io_dtype; /* dtype of q, k, v and out */
} gdn_shape_t;

/*
 * Prefill by direct token scan: each state row stays in registers for the
 * whole sequence and the tokens are walked in order (section "Keeping the
 * recurrent state on chip": the state is loaded once, carried through the
 * scan, and written back once).  Writes out[T, h_v, d_v] and
 * state_out[N, h_v, d_v, d_k].
 */
gdn_status_t gdn_prefill_scan(const gdn_shape_t* shape,
                              const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              const int32_t* cu_seqlens, const float* state_in,
                              void* out, float* state_out, void* stream);

/*
 * The ablation of section "Keeping the recurrent state on chip": with
 * register residency switched off the pages fall back to a blockwise scan,
 * which moves the state through memory every block and stops the cooperating
 * threads at barriers.  This is gdn_prefill_scan with the state's home in
 * state_out: every state_block tokens of a sequence each lane stores its part
 * of the state there, the workgroup meets at a barrier, and the lane reads it
 * back.  The arithmetic is the resident scan's, so out and state_out equal
 * gdn_prefill_scan's bit for bit; only the time differs.  Each round trip
 * moves 2 * h_v * d_v * d_k * 4 bytes per sequence.  state_block must be a
 * positive multiple of 4 (the scan walks tokens in blocks of 4).
 */
gdn_status_t gdn_prefill_scan_blockwise(const gdn_shape_t* shape,
                                        const void* q, const void* k, const void* v,
                                        const float* g, const float* beta,
                                        const int32_t* cu_seqlens, const float* state_in,
                                        void* out, float* state_out, int32_t state_block,
                                        void* stream);

/*
 * Bytes of device workspace gdn_prefill_chunked needs for this shape and
 * chunk size (0 if the shape or chunk size is invalid).  The bound depends
 * on num_seqs, total_tokens, h_qk, h_v, d_k, io_dtype and chunk_size.
 */
size_t gdn_prefill_chunked_workspace(const gdn_shape_t* shape, int32_t chunk_size);

/*
 * Prefill in blocks of chunk_size tokens (section "Qwen creates three
 * distinct workload shapes": the updates regrouped into blocks to expose
 * matrix operations).  Same tensors and results as gdn_prefill_scan, up to
 * rounding.  Chunks start at each sequence's first token; the last one may
 * be short.  chunk_size must be 16, 32 or 64.  `workspace` is caller-owned
 * device memory of at least gdn_prefill_chunked_workspace() bytes, 256-byte
 * aligned; its contents on entry do not matter and are garbage on exit.
 * Calls that share a workspace must be ordered on one stream.
 */
gdn_status_t gdn_prefill_chunked(const gdn_shape_t* shape,
                                 const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const int32_t* cu_seqlens, const float* state_in,
                                 void* out, float* state_out,
                                 int32_t chunk_size, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Bytes of device workspace gdn_prefill_segmented needs (0 if an argument is
 * invalid): the window's offsets, (num_seqs + 1) int32 rounded up to 256
 * bytes, plus, for chunk_size > 0, gdn_prefill_chunked_workspace of a batch of
 * min(total_tokens, segment_tokens) tokens.  It grows with segment_tokens,
 * not with the prompt.
 */
size_t gdn_prefill_segmented_workspace(const gdn_shape_t* shape, int32_t chunk_size, int32_t segment_tokens);

/*
 * Prefill of a long packed batch in bounded segments (section "Bounding
 * scratch memory by chunking the prompt": the prompt runs as a sequence of
 * bounded segments, the recurrent state carries the context from one to the
 * next, and the output does not change while peak scratch memory is set by
 * the segment).  The packed tokens are cut into windows of segment_tokens;
 * each sequence's tokens inside a window run through the chunked path
 * (chunk_size 16, 32 or 64; segment_tokens a multiple of it) or the direct
 * scan (chunk_size 0).  The state starts from state_in and passes from window
 * to window through state_out, in place.  Same tensors as gdn_prefill_chunked.
 * Results equal one gdn_prefill_chunked (or gdn_prefill_scan) call up to
 * rounding.  For a single sequence they are bit for bit the same when the
 * windows cut at the boundaries of the blocks the path walks: always for the
 * chunked path, and for the scan when segment_tokens is a multiple of 4.  The workspace must be
 * 256-byte aligned and at least gdn_prefill_segmented_workspace() bytes.
 */
gdn_status_t gdn_prefill_segmented(const gdn_shape_t* shape,
                                   const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const int32_t* cu_seqlens, const float* state_in,
                                   void* out, float* state_out,
                                   int32_t chunk_size, int32_t segment_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gdn_prefill_segmented with its workspace taken from a static device array
 * of GDN_STATIC_SCRATCH_BYTES bytes instead of a caller buffer.  The library
 * holds that array on every device it runs on until the process ends; the
 * call allocates nothing.  Arguments, results and errors are those of
 * gdn_prefill_segmented (the same kernels, so out and state_out are equal to
 * its results bit for bit), except that a call whose
 * gdn_prefill_segmented_workspace(shape, chunk_size, segment_tokens) exceeds
 * GDN_STATIC_SCRATCH_BYTES returns GDN_ERR_INVALID and enqueues nothing (use
 * fewer segment_tokens: at 32 value heads of 128 x 128, chunk 64, a
 * 2048-token segment needs about 45 MiB).  All calls on one device share the
 * array, which keeps whatever the last call left in it: calls that may
 * overlap on one device (other streams, other threads) race and must be
 * ordered by the caller.
 */
#define GDN_STATIC_SCRATCH_BYTES (64u << 20)

gdn_status_t gdn_prefill_segmented_noalloc(const gdn_shape_t* shape,
                                           const void* q, const void* k, const void* v,
                                           const float* g, const float* beta,
                                           const int32_t* cu_seqlens, const float* state_in,
                                           void* out, float* state_out,
                                           int32_t chunk_size, int32_t segment_tokens, void* stream);

/*
 * One recurrent step for each of `batch` sequences (section "Decode: minimize
 * bytes moved per token": one step per new token, bound by the bytes moved).
 * Tensors: q, k [batch, h_qk, d_k]; v, out [batch, h_v, d_v] (io_dtype);
 * g, beta [batch, h_v] fp32; state_in, state_out [batch, h_v, d_v, d_k] fp32.
 * state_in must not be NULL; state_out may equal state_in (in place).
 */
gdn_status_t gdn_decode_step(int32_t batch, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                             gdn_dtype_t io_dtype,
                             const void* q, const void* k, const void* v,
                             const float* g, const float* beta,
                             const float* state_in, void* out, float* state_out, void* stream);

/*
 * Optional parts of the fused decode step.  The three pointers are DEVICE
 * pointers (fp32, 4-byte aligned) or NULL; NULL selects the default noted.
 */
typedef struct {
  const float* gate_bias;   /* [h_v], added to g_raw before softplus; NULL = zeros */
  const float* gate_scale;  /* [h_v], multiplies the softplus;          NULL = ones  */
  const float* norm_weight; /* [d_v], multiplies the normalised output; NULL = ones  */
  float qk_eps;             /* finite, >= 0 */
  float norm_eps;           /* finite, >= 0 */
} gdn_decode_fused_params_t;

/*
 * One decode step with the work on either side of the recurrent update folded
 * into the same kernel (section "Reduce state and intermediate traffic": the
 * decode path fuses the preparation of queries and keys, and the recurrent
 * update with its normalisation, so that no intermediate value goes through
 * memory).  The pages name neither the preparation nor the norm; this call
 * computes, per sequence b, value head h (query/key head j = h / (h_v / h_qk)):
 *
 *     q = q_raw / sqrt(sum(q_raw^2) + qk_eps)        over d_k, fp32, not rounded
 *     k = k_raw / sqrt(sum(k_raw^2) + qk_eps)
 *     g = -gate_scale[h] * softplus(g_raw + gate_bias[h]),   beta = sigmoid(beta_raw)
 *     the gdn_decode_step update of state with q, k, v, g, beta, giving o
 *     out = o / sqrt(mean(o^2) + norm_eps) * norm_weight     over d_v
 *
 * Tensors and layouts as gdn_decode_step: q_raw, k_raw [batch, h_qk, d_k] and
 * v, out [batch, h_v, d_v] in io_dtype; g_raw, beta_raw [batch, h_v] fp32;
 * state_in, state_out [batch, h_v, d_v, d_k] fp32 (state_out may equal
 * state_in).  `params` is a HOST pointer read during the call, or NULL for
 * {NULL, NULL, NULL, 1e-6, 1e-6}.  With qk_eps = 0 an all-zero q_raw or k_raw
 * gives NaN, as does an all-zero output with norm_eps = 0.
 */
gdn_status_t gdn_decode_step_fused(int32_t batch, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                                   gdn_dtype_t io_dtype,
                                   const void* q_raw, const void* k_raw, const void* v,
                                   const float* g_raw, const float* beta_raw,
                                   const gdn_decode_fused_params_t* params,
                                   const float* state_in, void* out, float* state_out, void* stream);

/*
 * Expert GEMM on 4-bit group-affine weights (section "Dequantize the weights
 * during the matrix multiplication": each weight is a 4-bit code, each group
 * of 64 weights shares a bf16 scale and bias that rebuild it, the matrix unit
 * consumes bf16, accumulation is fp32 and the output bf16; section "Keep
 * expert routing on the GPU": the activation rows routed to an expert are
 * stored together).  Shapes:
 *     x        [rows, k]        bf16, rows grouped by expert
 *     expert_offsets [num_experts + 1] int32, device; expert e owns rows
 *              expert_offsets[e] .. expert_offsets[e + 1] - 1 (empty allowed,
 *              non-decreasing, from 0 to rows; clamped on the device)
 *     codes    [num_experts, n, k / 2] uint8: byte i of row (e, c) holds
 *              the codes of k = 2 i (low nibble) and k = 2 i + 1 (high)
 *     scales, biases [num_experts, n, k / 64] bf16: one per group of 64 k
 *     y        [rows, n]        bf16
 * Weight (e, c, k) = bf16(scale * code + bias), the product and sum formed by
 * one fp32 fma and rounded once (nearest even); y[r, c] = sum_k x[r, k] *
 * weight(e, c, k) for the expert e of row r, fp32 accumulation (in an order
 * of its own).  k is a positive multiple of 128, n of 128; at most 4096
 * experts; rows * k below 2^31.  With rows = 0, x and y may be NULL.
 */
typedef struct {
  int32_t num_experts;  /* E >= 1 */
  int32_t rows;         /* total routed activation rows, >= 0 */
  int32_t k;            /* contraction size, a multiple of 128 */
  int32_t n;            /* output columns, a multiple of 128 */
} gdn_moe_shape_t;

/* The fused form: each weight tile is rebuilt in registers as it is used; the
 * bf16 matrix never exists in memory. */
gdn_status_t gdn_moe_gemm_q4(const gdn_moe_shape_t* shape, const void* x, const int32_t* expert_offsets,
                             const uint8_t* codes, const void* scales, const void* biases, void* y,
                             void* stream);

/* Codes rewritten for the load path of the fused form (the same section: the
 * GEMM reads each weight tile's codes once; here each tile's codes become one
 * contiguous 1 KiB block, so that one load instruction covers whole cache lines
 * instead of 16 rows k / 2 bytes apart).  A one-time step when weights are
 * loaded.  codes [num_experts, n, k / 2] uint8 as above; packed, the same
 * number of bytes, receives block b = (e * n / 16 + t) * k / 128 + u (16-row
 * tile t, 128-k super-slab u) at byte 1024 b, its 16 bytes at 16 (16 g + c)
 * (g = 0..3, c = 0..15) being bytes 64 u + 16 g .. 64 u + 16 g + 15 of row
 * 16 t + c of expert e.  Both device pointers 16-byte aligned and not
 * overlapping; shape as for gdn_moe_gemm_q4 (rows and x unused). */
gdn_status_t gdn_moe_pack_q4(const gdn_moe_shape_t* shape, const uint8_t* codes, uint8_t* packed, void* stream);

/* gdn_moe_gemm_q4 reading codes packed by gdn_moe_pack_q4 (16-byte aligned);
 * y is bit-identical to gdn_moe_gemm_q4 on the same unpacked codes. */
gdn_status_t gdn_moe_gemm_q4_packed(const gdn_moe_shape_t* shape, const void* x, const int32_t* expert_offsets,
                                    const uint8_t* packed_codes, const void* scales, const void* biases, void* y,
                                    void* stream);

/* The pages' ablation, first half: rebuild the whole bf16 matrix
 * weights [num_experts, n, k] in memory (the same rounding as the fused form). */
gdn_status_t gdn_dequant_q4(const gdn_moe_shape_t* shape, const uint8_t* codes, const void* scales,
                            const void* biases, void* weights, void* stream);

/* The ablation, second half: the same grouped GEMM reading bf16 weights
 * [num_experts, n, k].  With weights from gdn_dequant_q4 it returns exactly
 * gdn_moe_gemm_q4's y. */
gdn_status_t gdn_moe_gemm_bf16(const gdn_moe_shape_t* shape, const void* x, const int32_t* expert_offsets,
                               const void* weights, void* y, void* stream);

/*
 * Decode attention over a grouped-query KV cache (sections "Pack query heads
 * to reuse KV rows" and "Switch attention layouts at long contexts": in a
 * decode step of a full-attention layer each query head reads its KV head's
 * whole cache; eight query heads share one KV head in the model described
 * there, each head holds 256 values, and past 32K positions a fixed-block
 * layout splits the cache into equal parts processed in parallel).  Per
 * sequence b and query head h, with j = h / (h_q / h_kv) and
 * n = context_lens[b]:
 *
 *     o[b, h] = sum_{t < n} softmax_t(scale * q[b, h] . k[b, j, t]) v[b, j, t]
 *
 * and o[b, h] = 0 when n = 0.  The caller has already written the current
 * token's key and value at position n - 1.  Scores, the softmax and the sums
 * are fp32 (products of bf16 inputs are exact); the output is rounded once to
 * bf16.  Shapes (dense, last index fastest, 16-byte aligned):
 *     q              [batch, h_q, head_dim]              bf16
 *     k_cache,
 *     v_cache        [batch, h_kv, max_context, head_dim] bf16
 *     context_lens   [batch] int32, device, 4-byte aligned; each value is
 *                    clamped to [0, max_context] on the device
 *     out            [batch, h_q, head_dim]              bf16, aliasing no input
 * head_dim is 64, 128 or 256; h_q is a multiple of h_kv; max_context is at
 * most 2^24.
 *
 * Scheduling, which changes no value beyond fp32 summation order:
 *  - heads_per_group query heads of one KV head share a workgroup, which
 *    loads each key and value row once for all of them (1, 2, 4 or 8,
 *    dividing h_q / h_kv; 0 = the largest of those that divides it).  The
 *    output bytes do not depend on it.
 *  - GDN_ATTN_GENERAL: one workgroup per (sequence, KV head, head pack)
 *    walks the whole context; no workspace.  GDN_ATTN_FIXED_BLOCK: each
 *    context is cut into num_blocks equal parts (0 = chosen from the shape
 *    and the device's compute-unit count), one workgroup each, and a second
 *    kernel merges the parts; it needs gdn_attention_decode_workspace()
 *    bytes of 256-byte aligned device workspace.  The automatic part count
 *    is min(ceil(CUs / (batch * h_kv * packs)), ceil(max_context / 32)),
 *    with CUs the current device's compute units and packs = h_q / h_kv /
 *    heads_per_group.  GDN_ATTN_AUTO takes the fixed-block layout when that
 *    count exceeds 1, i.e. when one workgroup per head pack would leave
 *    compute units idle.
 */
typedef enum {
  GDN_ATTN_AUTO = 0,
  GDN_ATTN_GENERAL = 1,
  GDN_ATTN_FIXED_BLOCK = 2
} gdn_attn_layout_t;

typedef struct {
  int32_t batch;        /* sequences, >= 1 */
  int32_t h_q;          /* query heads, a multiple of h_kv */
  int32_t h_kv;         /* KV heads, >= 1 */
  int32_t head_dim;     /* 64, 128 or 256 */
  int32_t max_context;  /* cache positions per (sequence, KV head), 1 .. 2^24 */
} gdn_attn_shape_t;

typedef struct {
  float scale;              /* multiplies q . k; finite */
  int32_t layout;           /* a gdn_attn_layout_t */
  int32_t heads_per_group;  /* 0, 1, 2, 4 or 8 */
  int32_t num_blocks;       /* fixed-block parts per context, 0 = automatic, at most min(max_context, 4096) */
} gdn_attn_params_t;

/* Workspace bytes for these arguments (0 when the general layout is chosen).
 * `params` is a HOST pointer, or NULL for {1 / sqrt(head_dim), AUTO, 0, 0}.
 * Returns 0 for invalid arguments as well; gdn_attention_decode reports them. */
size_t gdn_attention_decode_workspace(const gdn_attn_shape_t* shape, const gdn_attn_params_t* params);

gdn_status_t gdn_attention_decode(const gdn_attn_shape_t* shape, const gdn_attn_params_t* params, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* context_lens, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing for benchmarks and profiling.  While enabled (process-wide),
 * every kernel the library enqueues is bracketed by two hipEvents recorded on
 * the stream it is launched on.  Off by default; when off, no events are
 * created or recorded.
 */
gdn_status_t gdn_profile_enable(int enabled);

/*
 * Elapsed times of the kernels recorded since the last collect, in launch
 * order.  The caller must have synchronised the streams involved.  Copies up
 * to `cap` records (names are static strings owned by the library), frees
 * every recorded event and returns the number of records available (which may
 * exceed cap; the excess is dropped).  Returns -1 if an event query fails.
 */
int gdn_profile_collect(const char** names, float* ms, int cap);

/* Static, human-readable name of a status code ("GDN_OK", ...). */
const char* gdn_status_string(gdn_status_t status);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
