"""Error measures of the GPU parity tests (numpy only, so that oracle
workers in other processes can import it without torch).

Three measures are taken on every (sequence, value head) slice of outputs
(over all its tokens, or all its decode steps) and of final states, and a
check passes when the worst slice is within each bound:

* Frobenius: ||x - r||_F / ||r||_F.  The tolerance proper: 1e-5 for fp32
  inputs, 3e-3 for bf16 inputs with fp32 state.  Rounding the exact result to
  bf16 alone costs about 1.5e-3 on it.
* max norm: ||x - r||_max / ||r||_max, the largest elementwise error against
  the largest reference element of the slice.  bf16 rounding (8 significant
  bits, to nearest) puts at most 2^-8 |r| on one element, so rounding alone
  stays below 2^-8 (3.9e-3) on this measure; the kernels' own rounding (the
  state rounded once to bf16 in its products with K and Q, P rounded once,
  the split operands to 2^-17) reaches outputs damped by the chunk decay and
  adds well under that.  Bound: 1e-2 for bf16, 1e-5 for fp32 inputs (where
  the fp32 path rounds nothing to bf16).
* per token: ||x_t - r_t|| / max(||r_t||, RMS), with RMS the slice's
  root-mean-square row norm.  bf16 rounding contributes at most 2^-8 ||r_t||
  to a row; the products' rounding scales with the state, hence with RMS
  rather than with the token's own norm, which may be small.  Bound: 1e-2
  for bf16, 1e-5 for fp32.  A single token that is entirely wrong scores
  about 1 on this measure whatever the sequence length, while it moves the
  Frobenius measure of a 131072-token slice by only about 2.8e-3.
"""
import numpy as np

TOL = {"f32": 1e-5, "bf16": 3e-3}       # relative Frobenius, per slice
TOL_MAX = {"f32": 1e-5, "bf16": 1e-2}   # max norm, per slice
TOL_TOK = {"f32": 1e-5, "bf16": 1e-2}   # per token, against max(token norm, slice RMS)


class Errors:
    """Worst slice errors of one comparison, on the three measures."""

    def __init__(self, frob=0.0, maxn=0.0, tok=0.0):
        self.frob, self.maxn, self.tok = float(frob), float(maxn), float(tok)

    def merge(self, other: "Errors") -> "Errors":
        return Errors(max(self.frob, other.frob), max(self.maxn, other.maxn), max(self.tok, other.tok))

    def ok(self, io_dtype: str) -> bool:
        return self.frob <= TOL[io_dtype] and self.maxn <= TOL_MAX[io_dtype] and self.tok <= TOL_TOK[io_dtype]

    def __repr__(self):
        return f"frob {self.frob:.3e} max {self.maxn:.3e} tok {self.tok:.3e}"


def _ratio(num, den):
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def seq_errors(o, r) -> Errors:
    """Errors of one sequence's outputs o, r [L, H, d] (tokens, heads, values),
    each head a slice."""
    o = np.asarray(o, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.shape[0] == 0:
        return Errors()
    d = o - r
    rn = np.sqrt(np.sum(r * r, axis=(0, 2)))                      # [H]
    frob = _ratio(np.sqrt(np.sum(d * d, axis=(0, 2))), rn)
    maxn = _ratio(np.max(np.abs(d), axis=(0, 2)), np.max(np.abs(r), axis=(0, 2)))
    rms = rn / np.sqrt(r.shape[0])                                 # [H]
    row_r = np.sqrt(np.sum(r * r, axis=2))                         # [L, H]
    row_d = np.sqrt(np.sum(d * d, axis=2))
    tok = _ratio(row_d, np.maximum(row_r, rms[None, :]))
    return Errors(frob.max(), maxn.max(), tok.max())


def out_errors(o, r, cu) -> Errors:
    """Worst (sequence, head) errors of packed [T, H, d] outputs."""
    e = Errors()
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            e = e.merge(seq_errors(o[a:b], r[a:b]))
    return e


def state_errors(s, r) -> Errors:
    """Worst (sequence, head) errors of [N, H, dv, dk] states; the per-token
    measure is taken over the state's rows."""
    s = np.asarray(s, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    e = Errors()
    for n in range(r.shape[0]):
        # rows of the state play the part of tokens: [dv, H, dk]
        e = e.merge(seq_errors(np.transpose(s[n], (1, 0, 2)), np.transpose(r[n], (1, 0, 2))))
    return e


def max_rel_out(o, r, cu):
    """Largest per-(sequence, head) relative Frobenius error of [T, H, d] outputs."""
    return out_errors(o, r, cu).frob


def max_rel_state(s, r):
    """Largest per-(sequence, head) relative Frobenius error of [N, H, dv, dk] states."""
    return state_errors(s, r).frob
