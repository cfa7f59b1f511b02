"""Oracle comparisons spread over the host's cores.

At the long and ragged workloads the fp64 token loop of the oracle runs for
minutes on one core; (sequence, query/key head group) items are independent,
so they run in a pool of fresh Python processes (the spawn start method: the
workers import numpy, the oracle and metrics.py, never torch or the GPU).
Each item carries its inputs and the GPU's results for that item, and the
worker returns the error measures only.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np


def host_workers(cap: int = 16) -> int:
    """Worker processes for oracle pools: the cores this process may run on,
    at most ``cap``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def pool_map(fn, items, workers: int | None = None):
    """fn over items in a spawn-started process pool, results in order."""
    workers = workers or host_workers()
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        return list(pool.imap(fn, items, chunksize=1))


def check_prefill_item(item: dict) -> dict:
    """Oracle and error measures for one item: a sequence's tokens for a
    group of value heads (q, k [L, h_qk, dk]; v [L, h_v, dv]; g, beta
    [L, h_v]; state_in [1, h_v, dv, dk] or None) against the GPU's outputs
    o [L, h_v, dv] and final state s [1, h_v, dv, dk].  With a "dec" entry
    (q, k, v, g, beta per step [steps, 1, ...], the GPU's decode outputs o
    [steps, h_v, dv] and final state s) the decode steps continue from the
    oracle's final state."""
    from metrics import seq_errors, state_errors
    from oracle import gated_delta_decode_step, gated_delta_recurrence

    o_ref, s_ref = gated_delta_recurrence(item["q"], item["k"], item["v"], item["g"], item["beta"],
                                          state_in=item.get("state_in"))
    res = {"out": seq_errors(item["o"], o_ref), "state": state_errors(item["s"], s_ref)}
    if res["out"].tok > 0.1:  # name the wrong tokens and heads, for the failure message
        o = np.asarray(item["o"], dtype=np.float64)
        d = np.sqrt(np.sum((o - o_ref) ** 2, axis=2))
        rn = np.sqrt(np.sum(o_ref ** 2, axis=2))
        rms = np.sqrt(np.mean(rn ** 2, axis=0))
        bad = np.argwhere(d > 0.1 * np.maximum(rn, rms[None, :]))
        res["bad_tokens"] = f"{len(bad)} (token, head) rows, first {bad[:8].tolist()}, tokens {bad[:, 0].min()}..{bad[:, 0].max()}"

    dec = item.get("dec")
    if dec is not None:
        S = s_ref
        steps = dec["q"].shape[0]
        od_ref = np.zeros((steps,) + s_ref.shape[1:3])
        for t in range(steps):
            ot, S = gated_delta_decode_step(dec["q"][t], dec["k"][t], dec["v"][t], dec["g"][t], dec["beta"][t], S)
            od_ref[t] = ot[0]
        res["dec_out"] = seq_errors(dec["o"], od_ref)
        res["dec_state"] = state_errors(dec["s"], S)
    res["tag"] = item.get("tag")
    return res
