"""Seeded synthetic inputs for the gated delta rule.

This module only draws random numbers and prepares them the way a caller of
the layer would (L2-normalised q/k, beta = sigmoid(.), g = -softplus(.),
bf16 rounding of the activations).  It holds none of the recurrence's
arithmetic, so both the HIP path and the fp64 oracle can be fed from it.

Workload shapes follow the layer described in Perplexity, "Optimizing
on-device inference for Apple Silicon", section "Qwen creates three distinct
workload shapes" (a recurrent layer with a fixed-size per-head state) and
section "Keeping the recurrent state on chip" (fp32 state and gate, bf16
query/key activations).  The pages give no head counts for this layer; the
named workloads at the end fix them (16 query/key heads shared by 32 value
heads, d_k = d_v = 128).

All arrays are numpy: activations are float32 arrays whose values are exactly
representable in the requested io dtype (bf16 values are produced by
round-to-nearest-even), gates and state are float32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Inputs", "DecodeInputs", "RawDecodeInputs", "round_to_bf16", "make_prefill", "make_decode",
           "make_decode_raw", "MoeInputs", "make_moe", "AttentionInputs", "make_attention", "attention_device",
           "tiny_fp32_prefill", "decode_1000_steps", "prefill_4096", "prefill_131072", "ragged_32_then_decode"]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 values that are exactly representable in bfloat16.  Inputs must be
    finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _io(x: np.ndarray, io_dtype: str) -> np.ndarray:
    if io_dtype == "bf16":
        return round_to_bf16(x)
    if io_dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"io_dtype must be 'bf16' or 'f32', not {io_dtype!r}")


@dataclass
class Inputs:
    """A packed prefill batch.  Shapes: q, k [T, h_qk, d_k]; v [T, h_v, d_v];
    g, beta [T, h_v]; cu_seqlens [N+1] int32; state_in [N, h_v, d_v, d_k] or
    None."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    state_in: np.ndarray | None
    io_dtype: str
    chunk_size: int = 64
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        T, h_qk, d_k = self.q.shape
        return dict(num_seqs=len(self.cu_seqlens) - 1, total_tokens=T, h_qk=h_qk,
                    h_v=self.v.shape[1], d_k=d_k, d_v=self.v.shape[2])


@dataclass
class DecodeInputs:
    """``steps`` decode steps for B sequences: q, k [steps, B, h_qk, d_k];
    v [steps, B, h_v, d_v]; g, beta [steps, B, h_v]; state [B, h_v, d_v, d_k]."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    state: np.ndarray
    io_dtype: str
    meta: dict = field(default_factory=dict)


def _draw_gate(rng, shape, shift):
    beta_raw = rng.standard_normal(shape)
    g_raw = rng.standard_normal(shape)
    beta = _sigmoid(beta_raw).astype(np.float32)
    g = (-_softplus(g_raw + shift)).astype(np.float32)
    return g, beta


def make_prefill(lengths, h_qk, h_v, d_k, d_v, io_dtype="bf16", gate_shift=0.0,
                 state_std=None, seed=0, chunk_size=64, rng=None) -> Inputs:
    """Draw a packed batch of sequences with the given lengths.

    Draw order: q, k, v (standard normal, float32), beta_raw, g_raw (float64),
    then the initial state (normal with standard deviation ``state_std``; no
    state if None).  q and k are L2-normalised per (token, head) before
    rounding to the io dtype; beta = sigmoid(beta_raw),
    g = -softplus(g_raw + gate_shift).
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = [int(x) for x in lengths]
    if any(x < 0 for x in lengths):
        raise ValueError("lengths must be >= 0")
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = _io(_unit_rows(rng.standard_normal((T, h_qk, d_k), dtype=np.float32)), io_dtype)
    k = _io(_unit_rows(rng.standard_normal((T, h_qk, d_k), dtype=np.float32)), io_dtype)
    v = _io(rng.standard_normal((T, h_v, d_v), dtype=np.float32), io_dtype)
    g, beta = _draw_gate(rng, (T, h_v), gate_shift)
    state = None
    if state_std is not None:
        state = (rng.standard_normal((len(lengths), h_v, d_v, d_k), dtype=np.float32)
                 * np.float32(state_std)).astype(np.float32)
    return Inputs(q, k, v, g, beta, cu, state, io_dtype, chunk_size,
                  dict(lengths=lengths, gate_shift=gate_shift, state_std=state_std, seed=seed))


def make_decode(steps, batch, h_qk, h_v, d_k, d_v, io_dtype="bf16", gate_shift=0.0,
                state_std=0.02, seed=0, rng=None, state=None) -> DecodeInputs:
    """Draw ``steps`` decode steps at batch ``batch``.  Draw order: the
    initial state (unless given), then q, k, v, beta_raw, g_raw as arrays of
    shape [steps, batch, ...]."""
    rng = np.random.default_rng(seed) if rng is None else rng
    if state is None:
        state = (rng.standard_normal((batch, h_v, d_v, d_k), dtype=np.float32)
                 * np.float32(state_std)).astype(np.float32)
    q = _io(_unit_rows(rng.standard_normal((steps, batch, h_qk, d_k), dtype=np.float32)), io_dtype)
    k = _io(_unit_rows(rng.standard_normal((steps, batch, h_qk, d_k), dtype=np.float32)), io_dtype)
    v = _io(rng.standard_normal((steps, batch, h_v, d_v), dtype=np.float32), io_dtype)
    g, beta = _draw_gate(rng, (steps, batch, h_v), gate_shift)
    return DecodeInputs(q, k, v, g, beta, np.ascontiguousarray(state, dtype=np.float32), io_dtype,
                        dict(steps=steps, batch=batch, gate_shift=gate_shift, seed=seed))


@dataclass
class RawDecodeInputs:
    """One decode step for B sequences with raw (unprepared) activations, for
    the fused step: q_raw, k_raw [B, h_qk, d_k]; v [B, h_v, d_v]; g_raw,
    beta_raw [B, h_v]; state [B, h_v, d_v, d_k]; per-head gate_bias and
    gate_scale [h_v]; norm_weight [d_v]."""

    q_raw: np.ndarray
    k_raw: np.ndarray
    v: np.ndarray
    g_raw: np.ndarray
    beta_raw: np.ndarray
    state: np.ndarray
    gate_bias: np.ndarray
    gate_scale: np.ndarray
    norm_weight: np.ndarray
    io_dtype: str
    meta: dict = field(default_factory=dict)


def make_decode_raw(batch, h_qk, h_v, d_k, d_v, io_dtype="bf16", state_std=0.02, seed=0,
                    rng=None) -> RawDecodeInputs:
    """Draw one fused decode step.  Draw order: state (normal, standard
    deviation ``state_std``), q_raw, k_raw, v (standard normal, rounded to the
    io dtype, q and k NOT normalised), g_raw, beta_raw (standard normal),
    gate_bias (normal, mean 2, sd 0.5), gate_scale (uniform [0.5, 1.5]),
    norm_weight (normal, mean 1, sd 0.2).  All float32."""
    rng = np.random.default_rng(seed) if rng is None else rng
    f = np.float32
    state = (rng.standard_normal((batch, h_v, d_v, d_k), dtype=f) * f(state_std)).astype(f)
    q = _io(rng.standard_normal((batch, h_qk, d_k), dtype=f), io_dtype)
    k = _io(rng.standard_normal((batch, h_qk, d_k), dtype=f), io_dtype)
    v = _io(rng.standard_normal((batch, h_v, d_v), dtype=f), io_dtype)
    g_raw = rng.standard_normal((batch, h_v), dtype=f)
    beta_raw = rng.standard_normal((batch, h_v), dtype=f)
    gate_bias = (2.0 + 0.5 * rng.standard_normal(h_v)).astype(f)
    gate_scale = rng.uniform(0.5, 1.5, size=h_v).astype(f)
    norm_weight = (1.0 + 0.2 * rng.standard_normal(d_v)).astype(f)
    return RawDecodeInputs(q, k, v, g_raw, beta_raw, state, gate_bias, gate_scale, norm_weight, io_dtype,
                           dict(batch=batch, seed=seed, state_std=state_std))


@dataclass
class MoeInputs:
    """A grouped expert GEMM on 4-bit group-affine weights.  x [M, K] (rows
    grouped by expert; bf16 values in float32); expert_offsets [E + 1] int32;
    codes [E, N, K / 2] uint8 (even k in the low nibble); scales, biases
    [E, N, K / 64] (bf16 values in float32); token_of_row [M]: the token each
    row was routed from."""

    x: np.ndarray
    expert_offsets: np.ndarray
    codes: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    token_of_row: np.ndarray
    meta: dict = field(default_factory=dict)


def make_moe(tokens, num_experts=256, top_k=8, k=2048, n=1024, weight_std=0.02, skew=0.3, seed=0,
             rng=None) -> MoeInputs:
    """Route ``tokens`` tokens to ``top_k`` of ``num_experts`` experts and draw
    4-bit expert weights.

    Draw order: per-expert popularity (normal, standard deviation ``skew``),
    per-(token, expert) routing
    noise (normal; each token takes the top_k largest popularity + noise, so
    experts receive uneven row counts), token activations (standard normal,
    rounded to bf16), codes (uniform nibbles), then per group the range of a
    quantized N(0, weight_std) weight group (6 weight_std times U[0.8, 1.2])
    giving scale = bf16(range / 15) and bias = bf16(-range / 2 + a shift
    uniform in +-scale).  Rows are the routed tokens' activations, grouped by
    expert and in token order within an expert.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    pop = skew * rng.standard_normal(num_experts)
    noise = rng.standard_normal((tokens, num_experts))
    choice = np.argsort(-(pop[None, :] + noise), axis=1, kind="stable")[:, :top_k]  # [tokens, top_k]
    xt = round_to_bf16(rng.standard_normal((tokens, k), dtype=np.float32))
    expert_of = choice.reshape(-1)
    token_of = np.repeat(np.arange(tokens), top_k)
    order = np.lexsort((token_of, expert_of))  # by expert, then token
    counts = np.bincount(expert_of, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    token_of_row = token_of[order]
    codes = rng.integers(0, 256, size=(num_experts, n, k // 2), dtype=np.uint8)
    rngs = (6.0 * weight_std * rng.uniform(0.8, 1.2, size=(num_experts, n, k // 64))).astype(np.float32)
    scales = round_to_bf16(rngs / np.float32(15.0))
    shift = rng.uniform(-1.0, 1.0, size=rngs.shape).astype(np.float32) * scales
    biases = round_to_bf16(-rngs / np.float32(2.0) + shift)
    return MoeInputs(xt[token_of_row], offsets, codes, scales, biases, token_of_row,
                     dict(tokens=tokens, num_experts=num_experts, top_k=top_k, k=k, n=n, skew=skew, seed=seed))


@dataclass
class AttentionInputs:
    """One decode step of grouped-query attention over a KV cache (sections
    "Pack query heads to reuse KV rows" and "Switch attention layouts at long
    contexts": 16 query heads, 2 KV heads, 256 values per head in the model
    described there).  q [B, h_q, d]; k_cache, v_cache [B, h_kv, T_max, d]
    (bf16 values in float32 arrays); context_lens [B]; scale 1 / sqrt(d)."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    context_lens: np.ndarray
    scale: float


def make_attention(context_lens, h_q=16, h_kv=2, head_dim=256, max_context=None, seed=0, rng=None):
    """Entries N(0, 1) rounded to bf16, so that scale * q . k is about N(0, 1);
    positions past a context hold random values too (they must not be read)."""
    rng = rng or np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    B = len(lens)
    T = int(max_context if max_context is not None else max(1, int(lens.max(initial=1))))
    q = round_to_bf16(rng.standard_normal((B, h_q, head_dim), dtype=np.float32))
    k = round_to_bf16(rng.standard_normal((B, h_kv, T, head_dim), dtype=np.float32))
    v = round_to_bf16(rng.standard_normal((B, h_kv, T, head_dim), dtype=np.float32))
    return AttentionInputs(q, k, v, lens, 1.0 / math.sqrt(head_dim))


def attention_device(context_lens, h_q=16, h_kv=2, head_dim=256, max_context=None, seed=0, device="cuda"):
    """The same distribution drawn on the device (for caches of hundreds of
    MiB): returns bf16 torch tensors q, k_cache, v_cache, int32 context_lens
    and the scale."""
    import torch

    lens = [int(x) for x in context_lens]
    T = int(max_context if max_context is not None else max(1, max(lens)))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B = len(lens)
    q = torch.randn((B, h_q, head_dim), generator=gen, device=device).to(torch.bfloat16)
    k = torch.empty((B, h_kv, T, head_dim), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for t in (k, v):  # drawn a slice at a time to bound the fp32 temporary
        for b in range(B):
            for j in range(h_kv):
                t[b, j] = torch.randn((T, head_dim), generator=gen, device=device).to(torch.bfloat16)
    cl = torch.tensor(lens, dtype=torch.int32, device=device)
    return q, k, v, cl, 1.0 / math.sqrt(head_dim)


def ragged_lengths(rng, n, lo=256, hi=8192):
    """Sequence lengths log-uniform in [lo, hi], rounded to integers."""
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


# The five named workloads.  Each draws from its own seed (1000 .. 1004).
def tiny_fp32_prefill():
    """T = 64, 2 query/key and 2 value heads, d = 16, fp32, chunk 16, zero initial state."""
    return make_prefill([64], 2, 2, 16, 16, "f32", 0.0, None, rng=np.random.default_rng(1000), chunk_size=16)


def decode_1000_steps(decode_steps: int | None = None):
    """B = 1, 16 query/key heads shared by 32 value heads, d = 128, bf16, an
    N(0, 0.02) state carried over 1000 steps (or ``decode_steps``)."""
    steps = 1000 if decode_steps is None else decode_steps
    return make_decode(steps, 1, 16, 32, 128, 128, "bf16", 0.0, 0.02, rng=np.random.default_rng(1001))


def prefill_4096():
    """One 4096-token prompt, 16 / 32 heads, d = 128, bf16, gate shift 2, chunk 64, zero initial state."""
    return make_prefill([4096], 16, 32, 128, 128, "bf16", 2.0, None, rng=np.random.default_rng(1002), chunk_size=64)


def prefill_131072():
    """One 131072-token prompt, otherwise as prefill_4096."""
    return make_prefill([131072], 16, 32, 128, 128, "bf16", 2.0, None, rng=np.random.default_rng(1003),
                        chunk_size=64)


def ragged_32_then_decode(decode_steps: int | None = None):
    """32 sequences, lengths log-uniform in [256, 8192], each with an N(0, 0.02)
    initial state, then 256 decode steps (or ``decode_steps``) at B = 32.
    Returns (Inputs, DecodeInputs)."""
    rng = np.random.default_rng(1004)
    lengths = ragged_lengths(rng, 32)
    pre = make_prefill(lengths, 16, 32, 128, 128, "bf16", 2.0, 0.02, rng=rng, chunk_size=64)
    steps = 256 if decode_steps is None else decode_steps
    dec = make_decode(steps, 32, 16, 32, 128, 128, "bf16", 2.0, rng=rng,
                      state=np.zeros((32, 32, 128, 128), np.float32))
    return pre, dec
