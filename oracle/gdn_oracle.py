"""Plain fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE ONLY.  This module is the checker that the HIP path is
measured against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The library path
(``gated_deltanet_linear_delta_amd``) never imports, calls or falls back to it,
and this module imports nothing from the library: the two share no code.

What it computes
----------------
Source: Perplexity, "Optimizing on-device inference for Apple Silicon"
(Slovak and Spanish editions of the same post).

* Section "Qwen creates three distinct workload shapes" (sk: "Qwen vytvára
  tri rôzne tvary pracovného zaťaženia"; es: "Qwen crea tres formas de carga
  de trabajo distintas") describes a Gated DeltaNet layer as a fixed-size
  recurrent state, a learned gate that sets how much of the old state is kept,
  and a delta update that folds in the current token; every token depends on
  the state left by the previous one.  Prefill may walk the tokens carrying
  the state, or regroup the updates into blocks; both evaluate the same
  computation.
* Section "Keeping the recurrent state on chip" (es: "Mantener el estado
  recurrente en el chip") says the state is a matrix, and that the state and
  its gate are fp32 while query/key activations are bf16.
* Section "Bounding scratch memory by chunking the prompt" (es: "Limitar la
  memoria temporal mediante la fragmentación de mensajes") says the state is
  carried from one prompt segment to the next without changing the output.

The pages give the recurrence in prose only.  The equation used here is the
gated delta rule, the plainest formula that fits that prose:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t                       (post-update state)
    alpha_t = exp(g_t)                  (g is the log-gate, passed in)

per sequence and per value head, with S a [d_v, d_k] matrix (row index over
d_v, column index over d_k).  With H_qk query/key heads shared by H_v value
heads, value head h reads query/key head h // (H_v / H_qk) (contiguous
groups).  The prefill and decode functions apply no softplus, sigmoid, q/k
normalisation or q scaling: those belong to the caller, and the inputs
arrive already prepared.  gated_delta_decode_fused is the one exception: it
takes raw inputs and applies those steps itself (readings in its docstring).

Every input is widened exactly to fp64 (bf16 and fp32 values are exactly
representable) and every step runs in fp64.

Parity status: each public function is pinned by ``tests/test_oracle.py``
(brute force on the literal matrix form, exact rational arithmetic, the delta
invariant, closed forms for pure decay / constancy / orthonormal keys, a
hand-worked fixture in ``tests/golden/``, and agreement of the two forms
below).  The fused decode step is pinned by its own hand-worked fixture
(three cases covering both norms, the gate and beta activations and both
epsilons), closed forms of softplus and sigmoid, and its scale invariances.
The grouped GEMM on 4-bit weights is pinned by a hand-worked fixture (which
fixes the nibble order and the bf16 rounding of a rebuilt weight), a
brute-force triple loop, closed forms and the definition of bf16 rounding.
Decode attention is pinned by a hand-worked fixture, closed forms (uniform
scores give the mean value, a dominant key selects its value, two keys give
a logistic weight), invariance to a shift of all scores and head sharing.
No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "qk_head_of",
    "gated_delta_recurrence",
    "gated_delta_decode_step",
    "gated_delta_chunk_form",
    "softplus",
    "sigmoid",
    "gated_delta_decode_fused",
    "round_bf16",
    "dequantize_q4",
    "grouped_gemm_q4",
    "decode_attention",
]


def qk_head_of(h_v: int, h_qk: int) -> np.ndarray:
    """Query/key head read by each value head: contiguous groups of
    ``h_v // h_qk`` value heads share one query/key head.

    The pages describe head sharing only for the attention layers (section
    "Qwen creates three distinct workload shapes": several query heads share
    each key/value head).  For the recurrent layer the same contiguous-group
    convention is taken.
    """
    if h_qk <= 0 or h_v % h_qk != 0:
        raise ValueError(f"h_v={h_v} must be a positive multiple of h_qk={h_qk}")
    return np.arange(h_v) // (h_v // h_qk)


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_inputs(q, k, v, g, beta, cu_seqlens, state_in):
    q, k, v, g, beta = (_as_f64(a) for a in (q, k, v, g, beta))
    if q.ndim != 3 or k.shape != q.shape:
        raise ValueError("q and k must both be [T, H_qk, d_k]")
    T, h_qk, d_k = q.shape
    if v.ndim != 3 or v.shape[0] != T:
        raise ValueError("v must be [T, H_v, d_v]")
    h_v, d_v = v.shape[1], v.shape[2]
    if g.shape != (T, h_v) or beta.shape != (T, h_v):
        raise ValueError("g and beta must be [T, H_v]")
    if not np.all(np.isfinite(g)):
        raise ValueError("g (log-gate) must be finite")
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must be non-decreasing, start at 0 and end at T")
    n = cu.size - 1
    if state_in is None:
        s0 = np.zeros((n, h_v, d_v, d_k), dtype=np.float64)
    else:
        s0 = _as_f64(state_in)
        if s0.shape != (n, h_v, d_v, d_k):
            raise ValueError(f"state_in must be [{n}, {h_v}, {d_v}, {d_k}]")
    return q, k, v, g, beta, cu, s0, qk_head_of(h_v, h_qk)


def gated_delta_recurrence(q, k, v, g, beta, cu_seqlens=None, state_in=None):
    """Token-by-token gated delta rule over a packed, ragged batch (fp64).

    Follows the prose of "Qwen creates three distinct workload shapes" (walk
    the tokens and carry the state) and "Keeping the recurrent state on chip"
    (the state is a matrix) with the gated delta rule stated in the module
    header.  The update is applied in its expanded rank-one form

        p = S k,  u = beta (v - alpha p),  S <- alpha S + u k^T,  o = S q,

    which is the same algebra as alpha S (I - beta k k^T) + beta v k^T.

    Args (widened to fp64):
      q, k: [T, H_qk, d_k]; v: [T, H_v, d_v]; g, beta: [T, H_v]
      cu_seqlens: [N+1] token offsets of the packed sequences (None = one
        sequence of length T); zero-length sequences are allowed.
      state_in: [N, H_v, d_v, d_k] or None (zeros).
    Returns:
      o: [T, H_v, d_v] fp64, state_out: [N, H_v, d_v, d_k] fp64.
    """
    q, k, v, g, beta, cu, s0, qmap = _check_inputs(q, k, v, g, beta, cu_seqlens, state_in)
    T, h_v, d_v = v.shape
    o = np.zeros((T, h_v, d_v), dtype=np.float64)
    s_out = np.empty_like(s0)
    for n in range(cu.size - 1):
        S = s0[n].copy()  # [H_v, d_v, d_k]
        for t in range(int(cu[n]), int(cu[n + 1])):
            kt = k[t, qmap]  # [H_v, d_k]
            qt = q[t, qmap]
            alpha = np.exp(g[t])  # [H_v]
            p = np.einsum("hij,hj->hi", S, kt)
            u = beta[t][:, None] * (v[t] - alpha[:, None] * p)
            S = alpha[:, None, None] * S + u[:, :, None] * kt[:, None, :]
            o[t] = np.einsum("hij,hj->hi", S, qt)
        s_out[n] = S
    return o, s_out


def gated_delta_decode_step(q, k, v, g, beta, state):
    """One recurrent step per sequence for a batch of B sequences (fp64).

    Decode runs one step of the recurrence per new token; its cost is the
    bytes moved per token (section "Decode: minimize bytes moved per token",
    es: "Decodificación: minimizar los bytes transferidos por token").

    Args: q, k: [B, H_qk, d_k]; v: [B, H_v, d_v]; g, beta: [B, H_v];
          state: [B, H_v, d_v, d_k].
    Returns: o [B, H_v, d_v], new state [B, H_v, d_v, d_k] (fp64).
    """
    q = _as_f64(q)
    B = q.shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    return gated_delta_recurrence(q, k, v, g, beta, cu_seqlens=cu, state_in=state)


def softplus(x):
    """softplus(x) = log(1 + e^x) in fp64, evaluated as logaddexp(0, x)."""
    return np.logaddexp(0.0, _as_f64(x))


def sigmoid(x):
    """sigmoid(x) = 1 / (1 + e^-x) in fp64, evaluated as exp(-softplus(-x))."""
    return np.exp(-np.logaddexp(0.0, -_as_f64(x)))


def gated_delta_decode_fused(q_raw, k_raw, v, g_raw, beta_raw, state, gate_bias=None, gate_scale=None,
                             norm_weight=None, qk_eps=1e-6, norm_eps=1e-6):
    """One decode step with the work on either side of the update folded in
    (fp64).

    Section "Reduce state and intermediate traffic" (es: "Reducir el tráfico
    de estados y elementos intermedios") lists, among the chains the decode
    path fuses so that no intermediate goes through memory, the preparation
    of queries and keys and the recurrent update together with its
    normalisation.  The pages name neither the preparation nor the norm; the
    readings taken here are:

      q = q_raw / sqrt(sum(q_raw^2) + qk_eps)          per (sequence, qk head), over d_k
      k = k_raw / sqrt(sum(k_raw^2) + qk_eps)
      g = -gate_scale[h] * softplus(g_raw + gate_bias[h])   (so alpha = exp(g) is in (0, 1])
      beta = sigmoid(beta_raw)
      o, S' = one step of the gated delta rule (gated_delta_decode_step)
      out = o / sqrt(mean(o^2) + norm_eps) * norm_weight    per (sequence, v head), over d_v

    gate_bias, gate_scale: [H_v] or None (zeros, ones); norm_weight: [d_v] or
    None (ones).  Args otherwise as gated_delta_decode_step, with the raw
    (pre-activation) q, k, g and beta.  Returns (out [B, H_v, d_v], new state).
    """
    q_raw, k_raw, v, g_raw, beta_raw = (_as_f64(a) for a in (q_raw, k_raw, v, g_raw, beta_raw))
    h_v, d_v = v.shape[1], v.shape[2]
    bias = np.zeros(h_v) if gate_bias is None else _as_f64(gate_bias)
    scale = np.ones(h_v) if gate_scale is None else _as_f64(gate_scale)
    w = np.ones(d_v) if norm_weight is None else _as_f64(norm_weight)
    q = q_raw / np.sqrt(np.sum(q_raw * q_raw, axis=-1, keepdims=True) + qk_eps)
    k = k_raw / np.sqrt(np.sum(k_raw * k_raw, axis=-1, keepdims=True) + qk_eps)
    g = -scale[None, :] * softplus(g_raw + bias[None, :])
    beta = sigmoid(beta_raw)
    o, s_new = gated_delta_decode_step(q, k, v, g, beta, state)
    out = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + norm_eps) * w
    return out, s_new


def gated_delta_chunk_form(q, k, v, g, beta, chunk_size, cu_seqlens=None, state_in=None):
    """Blockwise evaluation of the same recurrence (fp64), used only to
    self-check the token loop.

    Section "Qwen creates three distinct workload shapes" says the updates can
    be regrouped into blocks that expose matrix operations and evaluate the
    same computation.  The pages print no block formula; this is the one that
    follows from unrolling the recurrence inside a block of n tokens that
    starts from state S0.  With gamma_r = exp(G_r), unrolling gives
    S_r = gamma_r S0 + sum_{i<=r} (gamma_r / gamma_i) u_i k_i^T and
    u_r = beta_r (v_r - alpha_r S_{r-1} k_r); substituting the first into the
    second yields the triangular system (I + A) U = diag(beta) V -
    diag(beta gamma) K S0^T below, and o_r = S_r q_r gives O:

      G_r   = sum_{i<=r} g_i           (log-decay inside the block)
      A_ri  = beta_r exp(G_r - G_i) (k_r . k_i)        for i < r, else 0
      U     = (I + A)^{-1} (diag(beta) V - diag(beta exp(G)) K S0^T)
      O     = diag(exp(G)) Q S0^T + (M * Q K^T) U,  M_ri = exp(G_r - G_i), i <= r
      S_end = exp(G_{n-1}) S0 + (diag(exp(G_{n-1} - G)) U)^T K

    Blocks start at each sequence's first token; the last one may be short.
    ``np.linalg.solve`` serves as the triangular solve.
    """
    if chunk_size < 1:
        raise ValueError("chunk_size must be >= 1")
    q, k, v, g, beta, cu, s0, qmap = _check_inputs(q, k, v, g, beta, cu_seqlens, state_in)
    T, h_v, d_v = v.shape
    o = np.zeros((T, h_v, d_v), dtype=np.float64)
    s_out = np.empty_like(s0)
    for n in range(cu.size - 1):
        for h in range(h_v):
            S = s0[n, h].copy()  # [d_v, d_k]
            j = qmap[h]
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk_size):
                c1 = min(c0 + chunk_size, int(cu[n + 1]))
                Kc, Qc, Vc = k[c0:c1, j], q[c0:c1, j], v[c0:c1, h]
                bc, G = beta[c0:c1, h], np.cumsum(g[c0:c1, h])
                nb = c1 - c0
                D = G[:, None] - G[None, :]
                lower_strict = np.tril(np.ones((nb, nb), dtype=bool), -1)
                lower = np.tril(np.ones((nb, nb), dtype=bool), 0)
                decay = np.where(lower, np.exp(np.where(lower, D, 0.0)), 0.0)
                A = np.where(lower_strict, bc[:, None] * decay * (Kc @ Kc.T), 0.0)
                rhs = bc[:, None] * Vc - (bc * np.exp(G))[:, None] * (Kc @ S.T)
                U = np.linalg.solve(np.eye(nb) + A, rhs)
                o[c0:c1, h] = np.exp(G)[:, None] * (Qc @ S.T) + (decay * (Qc @ Kc.T)) @ U
                S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * U).T @ Kc
            s_out[n, h] = S
    return o, s_out


# ---------------------------------------------------------------- expert GEMM on 4-bit weights
# Section "Dequantize the weights during the matrix multiplication" (es:
# "Descuantificar los pesos durante la multiplicación de matrices"): each
# expert weight is a 4-bit integer code, every group of 64 weights shares a
# bf16 scale and a bf16 bias that reconstruct its values, the matrix unit
# consumes bf16 operands, so the weights are rebuilt in bf16 before the
# multiplication; accumulation is fp32 and the output bf16.  Section "Keep
# expert routing on the GPU" says the activation rows routed to each expert
# are stored together; a grouped GEMM multiplies each expert's rows by that
# expert's matrix.  Readings taken: a weight is scale * code + bias with code
# in 0..15 (affine); groups run along the contraction index k; codes are
# packed two to a byte along k, the even k in the low nibble; the rebuilt
# weight is rounded once to bf16 (nearest, ties to even).


def round_bf16(x):
    """Round to the nearest bfloat16 value (ties to even), returned as fp64.
    Values must be finite and exactly representable in fp32 (rounding
    happens from the fp32 value, which the checks here hold exactly)."""
    f = np.asarray(x, dtype=np.float64)
    f32 = f.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), f):
        raise ValueError("round_bf16: value not exactly representable in fp32")
    u = f32.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rest = u & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    r = ((keep + up.astype(np.uint64)) << np.uint64(16)).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def dequantize_q4(codes, scales, biases, group=64):
    """Rebuild bf16 weights from 4-bit group-affine codes.

    codes: uint8 [..., N, K / 2], two codes per byte, k = 2 i in the low
    nibble of byte i and k = 2 i + 1 in the high nibble; scales, biases:
    [..., N, K / group] (bf16 values).  Returns [..., N, K] fp64 holding the
    bf16-rounded weights scale * code + bias.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0x0F).astype(np.float64)
    hi = (codes >> 4).astype(np.float64)
    q = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], 2 * codes.shape[-1])
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=-1)
    b = np.repeat(np.asarray(biases, dtype=np.float64), group, axis=-1)
    if s.shape != q.shape:
        raise ValueError("scales and biases must hold one value per group of codes")
    return round_bf16(s * q + b)  # the product and sum are exact in fp64


def grouped_gemm_q4(x, codes, scales, biases, expert_offsets, group=64):
    """Grouped GEMM over experts with 4-bit group-affine weights (fp64).

    x: [M, K] activation rows, grouped by expert: rows
    expert_offsets[e] .. expert_offsets[e + 1] - 1 go to expert e (empty
    groups allowed); codes [E, N, K / 2], scales and biases [E, N, K / group].
    Returns y [M, N] with y[r] = W_e x[r] for the expert e owning row r, W_e
    the rebuilt bf16 weights of dequantize_q4, in fp64.
    """
    x = _as_f64(x)
    off = np.asarray(expert_offsets, dtype=np.int64)
    w = dequantize_q4(codes, scales, biases, group)  # [E, N, K]
    E, N, K = w.shape
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    if off.shape != (E + 1,) or off[0] != 0 or off[-1] != x.shape[0] or np.any(np.diff(off) < 0):
        raise ValueError("expert_offsets must be non-decreasing, start at 0 and end at M")
    y = np.zeros((x.shape[0], N), dtype=np.float64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            y[a:b] = x[a:b] @ w[e].T
    return y


# ---------------------------------------------------------------- decode attention over a KV cache
# Sections "Pack query heads to reuse KV rows" and "Switch attention layouts
# at long contexts" (es: "Empaquetar los cabezales de consulta para reutilizar
# las filas KV", "Cambiar los diseños de atención en contextos largos"; sk:
# "Zbaľovanie hláv dopytu na opätovné použitie riadkov KV", "Prepínanie
# rozložení pozornosti pri dlhých kontextoch"): a decode step of a
# full-attention layer reads the whole KV cache; eight query heads share one
# KV head (grouped-query attention, 16 query and 2 KV heads in the model the
# pages describe), each head holds 256 values, and a fixed-block layout splits
# the cache into equal parts processed in parallel.  Packing and the block
# layout change how the work is scheduled, not what is computed.  Readings
# taken: softmax attention with the scale passed in by the caller; query head
# h reads KV head h // (h_q / h_kv) (contiguous groups); sequence b attends to
# its first context_lens[b] cached positions, which include the current
# token's key and value; an empty context gives a zero output.


def decode_attention(q, k_cache, v_cache, context_lens, scale):
    """One decode step of softmax attention over a KV cache (fp64).

    q: [B, H_q, d]; k_cache, v_cache: [B, H_kv, T_max, d];
    context_lens: [B] (0 <= len <= T_max).  Returns o [B, H_q, d] with
    o[b, h] = sum_t softmax_t(scale * q[b, h] . k[b, j, t]) v[b, j, t] over
    t < context_lens[b], j = h // (H_q / H_kv); zero where the context is empty.
    """
    q, k_cache, v_cache = (_as_f64(a) for a in (q, k_cache, v_cache))
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    if h_kv <= 0 or h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    lens = np.asarray(context_lens, dtype=np.int64)
    if lens.shape != (B,) or np.any(lens < 0) or np.any(lens > k_cache.shape[2]):
        raise ValueError("context_lens must be in [0, T_max]")
    group = h_q // h_kv
    o = np.zeros((B, h_q, d))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(h_q):
            j = h // group
            s = scale * (k_cache[b, j, :n] @ q[b, h])
            w = np.exp(s - s.max())
            o[b, h] = (w / w.sum()) @ v_cache[b, j, :n]
    return o
