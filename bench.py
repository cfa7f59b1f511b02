#!/usr/bin/env python3
"""Benchmark of the gated delta rule layer core on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Headline: chunked prefill of one 4096-token sequence (16 query/key heads shared
by 32 value heads, d_k = d_v = 128, bf16 q/k/v, fp32 gate and state, chunk 64).
One step is one gdn_prefill_chunked call over that prompt with every input
already resident in device memory; value = 4096 / (seconds per step).  The
same JSON line also carries:
  decode      one gdn_decode_step per token: B=1 with the state carried in
              place (it stays cache-resident), and B=32 "cold", rotating over
              eight state sets (512 MiB, twice the 256 MB Infinity Cache) so
              each step streams its state from HBM; timed by replaying a HIP
              graph of captured steps, and per kernel with HIP events;
  decode_fused  gdn_decode_step_fused (q/k L2 norms, gate and beta
              activations and the per-head RMS output norm in the decode
              kernel) at the same two batches, beside the same step
              unfused (torch prologue and epilogue around gdn_decode_step);
  scan        gdn_prefill_scan over the same 4096-token prompt (the
              direct-scan alternative, kept for the crossover);
  crossover   scan against chunked on one sequence of 64 ... 131072 tokens,
              50 timed calls each after 10 warm-ups, in alternating order,
              with medians, p10 and p90 (the scan skipped at 131072);
  state_residency_ablation  the first 2048 tokens through the resident scan
              and through gdn_prefill_scan_blockwise (state to memory and
              back every 32 or 16 tokens), with the state bytes moved;
  ragged_prefill  32 sequences with the ragged workload's lengths (about
              73k tokens, drawn on the device) through the chunked path and
              the scan: tokens/s, MFMA and HBM fractions;
  moe_gemm_q4  the expert GEMM on 4-bit group-affine weights (256 experts,
              top 8, K = 2048, N = 1024) at 512- and 2048-token prompts:
              rebuilt in the GEMM (codes as given, and repacked into 1 KiB
              tiles) against the two-pass ablation, with the HBM and MFMA
              fractions of the fused kernel;
  attention_decode  one decode step of grouped-query attention (16 query
              heads on 2 KV heads, 256 values per head, bf16 cache drawn on
              the device) at contexts of 32K, 64K and 128K positions: the
              fixed-block layout with all 8 query heads of a group packed in
              a workgroup, beside the pages' two ablations (one query head
              per workgroup; the general layout, one workgroup per head pack
              over the whole context) and the pages' own pack of 4; timed by
              graph replay, with per-kernel HIP event times and the cache's
              HBM fraction;
  segmented_prefill  a 131072-token prompt (drawn on the device) chunked in
              one call and through gdn_prefill_segmented in 8192- and
              4096-token segments: time, workspace, and output equality;
  roofline    for the longest kernel of the chunked call: algorithmic bytes
              per launch over its mean duration, from HIP events that the
              library records on the launch stream while profiling is on;
  cpu_baseline  the fp64 oracle timed on this host's cores: a process pool,
              one process per core (at most 16), over (sequence, value head)
              items of bounded samples of the four bf16 workloads, and the
              oracle as it stands (all heads in one process) on one core.
  traffic     HBM bytes per launch of that kernel as the FETCH_SIZE and
              WRITE_SIZE counters saw them (profiles/, scaled by the same
              counters on a copy of known size), or null once the kernel
              source differs from the one the counters were taken on.
--prefill-only runs just the headline calls and one 512 MiB device copy (the
counter calibration), for counter runs under rocprofv3; --attention-counters
runs just three eager decode-attention calls at 32K and 128K and the same copy.
Before the W warmup steps the headline step runs untimed for 0.25 s so that
the GPU clocks have settled; the timed region is exactly K steps.
Prints exactly one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s

T, HQK, HV, DK, DV, CHUNK = 4096, 16, 32, 128, 128, 64
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_sweep_T4096_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "gated_deltanet_linear_delta_amd", "csrc", "gdn_chunked.hip")
MFMA_FILE = os.path.join(ROOT, "profiles", "chunk_prefill_T4096_mfma.md")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_traffic.md")
DECODE_SOURCE = os.path.join(ROOT, "gated_deltanet_linear_delta_amd", "csrc", "gdn_decode.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_flops(t, hv=HV, hqk=HQK, dk=DK, dv=DV, c=CHUNK):
    """Useful flops of the chunked form per call: the inter-chunk products
    (K S^T, Q S^T, state update: 6 dk dv), the Gram products counted once per
    query/key head (2 C dk Hqk/Hv), the causal halves of the C x C products
    with U (C dv each for T Y and QKm U) and of T's construction (C dk), and
    the triangular inverse (C^2 / 3), per token and value head."""
    return t * hv * (6 * dk * dv + 2 * c * dk * hqk / hv + c * dk + 2 * c * dv + c * c / 3)


def kernel_bytes(name, t, n_seqs, state_in):
    """Algorithmic HBM bytes of one launch: each of the kernel's inputs from
    the caller read once, each output written once (bf16 activations, fp32
    gate, beta and state).  The prep kernel consumes q, k, g and beta; the
    sweep consumes v (and the prep's per-chunk operands, which are not
    algorithmic) and writes o and the state."""
    qk = t * 2 * HQK * DK * 2
    vo = t * HV * DV * 2
    gb = t * 2 * HV * 4
    st = n_seqs * HV * DV * DK * 4
    if name == "chunk_sweep":
        return 2 * vo + st * (2 if state_in else 1)
    if name == "chunk_prep":
        return qk + gb
    if name == "chunk_table":
        return 4 * (n_seqs + 1)
    if name == "scan":
        return qk + 2 * vo + gb + st * (2 if state_in else 1)
    raise KeyError(name)


def decode_bytes(b):
    return b * (2 * HV * DV * DK * 4 + 2 * HQK * DK * 2 + 2 * HV * DV * 2 + 2 * HV * 4)


def source_digest(path):
    import hashlib
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def profile_fields(path, source):
    """The machine-readable `- key: value` lines of a committed counter
    summary, if it was taken on the current source of its kernel; else None."""
    try:
        with open(path) as fh:
            fields = dict(line.strip("- \n").split(": ", 1) for line in fh if line.startswith("- ") and ": " in line)
        return fields if fields.get("source_sha256") == source_digest(source) else None
    except OSError:
        return None


def measured_traffic():
    """HBM bytes of one chunked-prefill call (prep and sweep launches) from the
    committed counter summary, if it was taken on the current kernel source;
    else None."""
    f = profile_fields(TRAFFIC_FILE, KERNEL_SOURCE)
    try:
        return sum(int(f[k]) for k in ("prep_fetch_bytes_per_launch", "prep_write_bytes_per_launch",
                                       "fetch_bytes_per_launch", "write_bytes_per_launch")) if f else None
    except (KeyError, ValueError):
        return None


def counter_figures():
    """Counter-derived figures from the committed rocprofv3 summaries (each
    None unless taken on the current kernel source): the prefill kernels'
    MFMA busy fractions and executed bf16 MFMA flops, and the HBM bytes of
    the plain and the fused decode step at B = 1 and B = 32 (FETCH_SIZE +
    WRITE_SIZE, copy-calibrated)."""
    out = {}
    m = profile_fields(MFMA_FILE, KERNEL_SOURCE)
    for key in ("prep_mfma_busy", "sweep_mfma_busy", "call_mfma_busy"):
        out[key] = float(m[key]) if m and key in m else None
    for key in ("prep_bf16_mfma_flops", "sweep_bf16_mfma_flops"):
        out[key] = int(m[key]) if m and key in m else None
    d = profile_fields(DECODE_TRAFFIC_FILE, DECODE_SOURCE)
    for key in ("b1_bytes_per_step", "b32_bytes_per_step", "fused_b1_bytes_per_step", "fused_b32_bytes_per_step"):
        out["decode_" + key] = int(d[key]) if d and key in d else None
    out["source"] = "profiles/chunk_prefill_T4096_mfma.md, profiles/decode_step_traffic.md"
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def mean_by_name(records):
    acc = {}
    for name, ms in records:
        acc.setdefault(name, []).append(ms)
    return {k: (float(np.mean(v)), len(v)) for k, v in acc.items()}


def _oracle_item(item):
    """CPU baseline worker: the fp64 oracle on one (sequence, value head) item
    (prefill tokens, or decode steps one at a time).  Runs in a spawn-started
    process that imports numpy and the oracle only."""
    from oracle import gated_delta_decode_step, gated_delta_recurrence
    if item["kind"] == "prefill":
        gated_delta_recurrence(item["q"], item["k"], item["v"], item["g"], item["beta"], state_in=item["s0"])
    else:
        S = item["s0"]
        for t in range(item["q"].shape[0]):
            _, S = gated_delta_decode_step(item["q"][t], item["k"][t], item["v"][t], item["g"][t],
                                           item["beta"][t], S)
    return 0


def _host_cores(cap=16):
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_baseline_leg(log_fn):
    """The fp64 oracle on the host cores: a process pool, one process per core,
    over (sequence, value head) items, on bounded samples of the four bf16
    workloads, plus the oracle as it stands (all heads in one process) on one
    core.  Tokens/s per workload."""
    import multiprocessing as mp
    from gated_deltanet_linear_delta_amd.workloads import make_decode, make_prefill, ragged_lengths

    def f32(a):
        return np.ascontiguousarray(a, dtype=np.float32)

    def prefill_items(inp, seqs):
        G = inp.v.shape[1] // inp.q.shape[1]
        cu = inp.cu_seqlens
        for n in seqs:
            a, b = int(cu[n]), int(cu[n + 1])
            for h in range(inp.v.shape[1]):
                j = h // G
                yield {"kind": "prefill", "q": f32(inp.q[a:b, j:j + 1]), "k": f32(inp.k[a:b, j:j + 1]),
                       "v": f32(inp.v[a:b, h:h + 1]), "g": f32(inp.g[a:b, h:h + 1]),
                       "beta": f32(inp.beta[a:b, h:h + 1]),
                       "s0": None if inp.state_in is None else f32(inp.state_in[n:n + 1, h:h + 1])}

    def decode_items(dec):
        G = dec.v.shape[2] // dec.q.shape[2]
        for h in range(dec.v.shape[2]):
            j = h // G
            yield {"kind": "decode", "q": f32(dec.q[:, :, j:j + 1]), "k": f32(dec.k[:, :, j:j + 1]),
                   "v": f32(dec.v[:, :, h:h + 1]), "g": f32(dec.g[:, :, h:h + 1]), "beta": f32(dec.beta[:, :, h:h + 1]),
                   "s0": f32(dec.state[:, h:h + 1])}

    cores = _host_cores()
    rng4 = np.random.default_rng(1004)
    lens4 = ragged_lengths(rng4, 32)
    cases = {
        "decode_1000_steps": ("decode", make_decode(1000, 1, HQK, HV, DK, DV, "bf16", 0.0, 0.02,
                                                   rng=np.random.default_rng(1001)), None,
                              "all 1000 steps, 32 value heads"),
        "prefill_4096": ("prefill", make_prefill([4096], HQK, HV, DK, DV, "bf16", 2.0, None,
                                                 rng=np.random.default_rng(1002)), [0],
                         "all 4096 tokens, 32 value heads"),
        "prefill_131072": ("prefill", make_prefill([32768], HQK, HV, DK, DV, "bf16", 2.0, None,
                                                   rng=np.random.default_rng(1003)), [0],
                           "the first 32768 tokens (same distributions), 32 value heads"),
        "ragged_32_then_decode": ("prefill", make_prefill(lens4[:16], HQK, HV, DK, DV, "bf16", 2.0, 0.02,
                                                          rng=np.random.default_rng(1004)), list(range(16)),
                                  f"prefill of 16 of the 32 sequences ({int(sum(lens4[:16]))} tokens, "
                                  "the workload's first sixteen lengths), 32 value heads"),
    }
    per = {}
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_item, [{"kind": "decode", "q": np.zeros((1, 1, 1, 4), np.float32),
                                 "k": np.zeros((1, 1, 1, 4), np.float32), "v": np.zeros((1, 1, 1, 4), np.float32),
                                 "g": np.zeros((1, 1, 1), np.float32), "beta": np.zeros((1, 1, 1), np.float32),
                                 "s0": np.zeros((1, 1, 4, 4), np.float32)}] * cores)  # start the workers
        for name, (kind, inp, seqs, what) in cases.items():
            items = list(decode_items(inp) if kind == "decode" else prefill_items(inp, seqs))
            tokens = inp.q.shape[0] * (inp.q.shape[1] if kind == "decode" else 1)
            t0 = time.perf_counter()
            pool.map(_oracle_item, items, chunksize=1)
            el = time.perf_counter() - t0
            per[name] = {"tokens_per_s": round(tokens / el, 1), "seconds": round(el, 2), "items": len(items),
                         "sample": what}
            log_fn(f"cpu baseline {name}: {per[name]}")
    # the oracle as it stands, on one core: all heads vectorised in one process
    from oracle import gated_delta_recurrence
    inp2 = cases["prefill_4096"][1]
    n_tok = 512
    t0 = time.perf_counter()
    gated_delta_recurrence(inp2.q[:n_tok], inp2.k[:n_tok], inp2.v[:n_tok], inp2.g[:n_tok], inp2.beta[:n_tok])
    el1 = time.perf_counter() - t0
    single = {"tokens_per_s": round(n_tok / el1, 1), "seconds": round(el1, 2),
              "sample": f"the first {n_tok} tokens of the 4096-token prompt, all 32 value heads in one process"}
    return {"value": per["prefill_4096"]["tokens_per_s"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"prefill_4096: {per['prefill_4096']['sample']}, fp64 NumPy token loop, one process per "
                      f"core over {per['prefill_4096']['items']} (sequence, value head) items "
                      f"({per['prefill_4096']['seconds']} s)",
            "per_workload": per, "single_core": single, "host_cpus": os.cpu_count(), "host_cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scan", action="store_true")
    ap.add_argument("--no-moe", action="store_true", help="skip the 4-bit expert GEMM leg")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 131072-token segmented-prefill and the ragged-batch legs")
    ap.add_argument("--no-attention", action="store_true", help="skip the decode-attention leg")
    ap.add_argument("--prefill-only", action="store_true", help="headline calls and the copy calibration only")
    ap.add_argument("--attention-counters", action="store_true",
                    help="eager decode-attention calls at 32K and 128K and the copy calibration only")
    ap.add_argument("--moe-counters", action="store_true",
                    help="eager 4-bit expert GEMM calls at 512 and 2048 tokens and the copy calibration only")
    ap.add_argument("--decode-counters", action="store_true",
                    help="eager decode steps (B=1 and B=32, state sets rotating past the Infinity Cache) and the "
                         "copy calibration only")
    ap.add_argument("--no-crossover", action="store_true", help="skip the scan-vs-chunked prompt-length sweep")
    ap.add_argument("--crossover-reps", type=int, default=50, help="timed calls per kernel and prompt length")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer core has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_linear_delta_amd import gdn
    from gated_deltanet_linear_delta_amd.workloads import make_decode, prefill_4096

    gdn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup

    def copy_calibration():
        src = torch.ones(1 << 28, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 536870912 bytes read, 536870912 written")

    if args.moe_counters:
        # counter runs: three eager calls of the fused expert GEMM per prompt
        # size (the bench leg's inputs), three more on the packed codes, then
        # the calibration copy
        from gated_deltanet_linear_delta_amd.workloads import make_moe
        for tok in (512, 2048):
            mi = make_moe(tok, num_experts=256, top_k=8, k=2048, n=1024, seed=5000 + tok)
            bfd = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)
            xm, offm = bfd(mi.x), torch.from_numpy(mi.expert_offsets.astype(np.int32)).to(dev)
            cm, sm, bm = torch.from_numpy(mi.codes).to(dev), bfd(mi.scales), bfd(mi.biases)
            ym = torch.empty((xm.shape[0], 1024), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                gdn.moe_gemm_q4(xm, offm, cm, sm, bm, y=ym)
            pm = gdn.moe_pack_q4(cm)
            for _ in range(3):
                gdn.moe_gemm_q4_packed(xm, offm, pm, sm, bm, y=ym)
            torch.cuda.synchronize()
            log(f"expert GEMM at {tok} tokens: three calls, then three on packed codes")
            del xm, offm, cm, pm, sm, bm, ym
            torch.cuda.empty_cache()
        copy_calibration()
        print(json.dumps({"moe_counters": True}), flush=True)
        return

    if args.decode_counters:
        # counter runs: eager steps (no graphs), each batch rotating over state
        # sets larger than the Infinity Cache, so every step streams its state
        # from HBM; then the calibration copy
        for B, n_sets in ((1, 256), (32, 8)):
            dec = make_decode(n_sets, B, HQK, HV, DK, DV, "bf16", 2.0 if B > 1 else 0.0, 0.02, seed=1001 + B)
            bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)
            dq, dk_, dv_ = bf(dec.q), bf(dec.k), bf(dec.v)
            dg, db = torch.from_numpy(dec.g).to(dev), torch.from_numpy(dec.beta).to(dev)
            states = [torch.from_numpy(dec.state).to(dev).clone() for _ in range(n_sets)]
            dout = torch.empty((B, HV, DV), dtype=torch.bfloat16, device=dev)
            for i in range(2 * n_sets):
                s_ = i % n_sets
                gdn.decode_step(dq[s_], dk_[s_], dv_[s_], dg[s_], db[s_], states[s_], out=dout, state_out=states[s_])
            torch.cuda.synchronize()
            log(f"decode B={B}: {2 * n_sets} eager steps over {n_sets} state sets")
            del states, dq, dk_, dv_, dg, db, dout
            torch.cuda.empty_cache()
        # the fused step over the same rotation (raw q/k/g/beta, per-head
        # gate parameters and norm weight)
        from gated_deltanet_linear_delta_amd.workloads import make_decode_raw
        for B, n_sets in ((1, 256), (32, 8)):
            rng = np.random.default_rng(2001 + B)
            sets = [make_decode_raw(B, HQK, HV, DK, DV, "bf16", 0.02, rng=rng) for _ in range(n_sets)]
            bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)
            f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
            dq = [bf(r.q_raw) for r in sets]
            dk_ = [bf(r.k_raw) for r in sets]
            dv_ = [bf(r.v) for r in sets]
            dg = [f32(r.g_raw) for r in sets]
            db = [f32(r.beta_raw) for r in sets]
            states = [f32(r.state) for r in sets]
            bias, scale, w = f32(sets[0].gate_bias), f32(sets[0].gate_scale), f32(sets[0].norm_weight)
            dout = torch.empty((B, HV, DV), dtype=torch.bfloat16, device=dev)
            for i in range(2 * n_sets):
                s_ = i % n_sets
                gdn.decode_step_fused(dq[s_], dk_[s_], dv_[s_], dg[s_], db[s_], states[s_], gate_bias=bias,
                                      gate_scale=scale, norm_weight=w, out=dout, state_out=states[s_])
            torch.cuda.synchronize()
            log(f"fused decode B={B}: {2 * n_sets} eager steps over {n_sets} state sets")
            del sets, states, dq, dk_, dv_, dg, db, dout
            torch.cuda.empty_cache()
        copy_calibration()
        print(json.dumps({"decode_counters": True}), flush=True)
        return

    if args.attention_counters:
        # counter runs: graph replays are left out (rocprofv3's counter
        # collection does not survive them); three eager calls per context of
        # the fixed-block layout with packs of 8, then the calibration copy
        from gated_deltanet_linear_delta_amd.workloads import attention_device
        for TA in (32768, 131072):
            qa, ka, va, cla, sca = attention_device([TA], seed=TA)
            oa = torch.empty_like(qa)
            wsa = gdn.alloc_workspace(gdn.attention_decode_workspace_bytes(1, 16, 2, 256, TA, sca, "fixed_block", 8),
                                      dev)
            for _ in range(3):
                gdn.attention_decode(qa, ka, va, cla, sca, layout="fixed_block", heads_per_group=8, out=oa,
                                     workspace=wsa)
            torch.cuda.synchronize()
            log(f"attention at {TA}: three calls")
            del qa, ka, va, oa, wsa
            torch.cuda.empty_cache()
        copy_calibration()
        print(json.dumps({"attention_counters": True}), flush=True)
        return

    # ------------------------------------------------------------ inputs
    log("generating the 4096-token prefill workload")
    inp = prefill_4096()

    def io(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(dev)

    q, k, v = io(inp.q), io(inp.k), io(inp.v)
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    cu = torch.tensor(inp.cu_seqlens, dtype=torch.int32, device=dev)
    out = torch.empty((T, HV, DV), dtype=torch.bfloat16, device=dev)
    st = torch.empty((1, HV, DV, DK), dtype=torch.float32, device=dev)
    ws = gdn.alloc_workspace(gdn.chunked_workspace_bytes(1, T, HQK, HV, DK, DV, gdn.GDN_DTYPE_BF16, CHUNK), dev)

    def prefill():
        gdn.prefill_chunked(q, k, v, g, beta, cu, None, out=out, state_out=st, chunk_size=CHUNK, workspace=ws)

    # ------------------------------------------------------------ headline: chunked prefill
    # The GPU raises its clocks over the first milliseconds of sustained work;
    # run the step untimed for a quarter second first, so that the W warmup
    # and K timed steps see the steady state.
    settle_start = time.perf_counter()
    while time.perf_counter() - settle_start < 0.25:
        for _ in range(20):
            prefill()
        torch.cuda.synchronize()
    for _ in range(W):
        prefill()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        prefill()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    log(f"chunked prefill: {ms_step * 1e3:.1f} us per call (wall, {K} calls)")

    # per-call distribution: HIP events around each call, max(50, K) calls
    n_ev = max(50, K)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for e0, e1 in evs:
        e0.record()
        prefill()
        e1.record()
    torch.cuda.synchronize()
    call_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    call_stats = {"calls": n_ev, "median_us": round(float(np.median(call_us)), 2),
                  "p10_us": round(float(np.percentile(call_us, 10)), 2),
                  "p90_us": round(float(np.percentile(call_us, 90)), 2)}
    log(f"chunked prefill per call (events): {call_stats}")

    gdn.profile_enable(True)
    for _ in range(K):
        prefill()
    torch.cuda.synchronize()
    gdn.profile_enable(False)
    per_kernel = mean_by_name(gdn.profile_collect())
    call_ms = sum(m for m, _ in per_kernel.values())
    log("chunked kernels (HIP events): " + ", ".join(f"{n} {m * 1e3:.1f} us" for n, (m, _) in per_kernel.items()))
    # The roofline unit is the whole call (prep + sweep, the two launches of one
    # gdn_prefill_chunked): HIP events around each call leave the launches
    # back to back, while events between the two kernels add a barrier that
    # costs the sweep about 5 us (rocprofv3 reads it 10 % below the per-kernel
    # events above).
    dom = "chunk_prep+chunk_sweep"
    dom_ms = call_stats["median_us"] * 1e-3
    dom_bytes = kernel_bytes("chunk_prep", T, 1, False) + kernel_bytes("chunk_sweep", T, 1, False)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    flops = prefill_flops(T)
    mfma_util = flops / (ms_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)

    if args.prefill_only:
        # counter calibration: one device copy of exactly 512 MiB each way
        src = torch.ones(1 << 28, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 536870912 bytes read, 536870912 written")
        print(json.dumps({"prefill_only": True, "ms_per_step": round(ms_step, 5),
                          "kernels_us": {n: round(m * 1e3, 2) for n, (m, _) in per_kernel.items()}}), flush=True)
        return

    # ------------------------------------------------------------ decode
    def replay_us(step, steps_per_graph):
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(steps_per_graph):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        reps = max(2, 2000 // steps_per_graph)
        t1 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t1) * 1e6 / (reps * steps_per_graph)

    def decode_leg(B, n_sets, steps_per_graph, seed):
        dec = make_decode(n_sets, B, HQK, HV, DK, DV, "bf16", 2.0 if B > 1 else 0.0, 0.02, seed=seed)
        dq, dk_, dv_ = io(dec.q), io(dec.k), io(dec.v)
        dg = torch.from_numpy(dec.g).to(dev)
        db = torch.from_numpy(dec.beta).to(dev)
        states = [torch.from_numpy(dec.state).to(dev).clone() for _ in range(n_sets)]
        dout = torch.empty((B, HV, DV), dtype=torch.bfloat16, device=dev)

        def step(i):
            s = i % n_sets
            gdn.decode_step(dq[s], dk_[s], dv_[s], dg[s], db[s], states[s], out=dout, state_out=states[s])

        for i in range(2 * n_sets):
            step(i)
        torch.cuda.synchronize()
        # per-kernel durations from HIP events
        gdn.profile_enable(True)
        for i in range(steps_per_graph):
            step(i)
        torch.cuda.synchronize()
        gdn.profile_enable(False)
        kern = mean_by_name(gdn.profile_collect())["decode"][0]
        # launch-free step time: replay a captured graph of steps
        us = replay_us(step, steps_per_graph)
        nbytes = decode_bytes(B)
        return {
            "batch": B,
            "state_sets": n_sets,
            "us_per_step_graph": round(us, 3),
            "kernel_us": round(kern * 1e3, 3),
            "tokens_per_s": round(B / (us * 1e-6), 1),
            "bytes_per_step": nbytes,
            # launch-free step time from graph replay (it matches the rocprofv3
            # kernel average; HIP events around one short kernel add overhead)
            "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_frac_event_timed": round(nbytes / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }

    def fused_leg(B, n_sets, steps_per_graph, seed):
        """gdn_decode_step_fused from raw q/k/g/beta, and for comparison the same
        step unfused: torch prologue (L2 norms, softplus, sigmoid), the plain
        gdn_decode_step, torch RMS norm epilogue, each intermediate in memory."""
        from gated_deltanet_linear_delta_amd.workloads import make_decode_raw
        rng = np.random.default_rng(seed)
        sets = [make_decode_raw(B, HQK, HV, DK, DV, "bf16", 0.02, rng=rng) for _ in range(n_sets)]
        t = lambda x: torch.from_numpy(x).to(dev)
        dq = [io(r.q_raw) for r in sets]
        dk_ = [io(r.k_raw) for r in sets]
        dv_ = [io(r.v) for r in sets]
        dg = [t(r.g_raw) for r in sets]
        db = [t(r.beta_raw) for r in sets]
        states = [t(r.state).clone() for r in sets]
        bias, scale, w = t(sets[0].gate_bias), t(sets[0].gate_scale), t(sets[0].norm_weight)
        dout = torch.empty((B, HV, DV), dtype=torch.bfloat16, device=dev)
        eps = 1e-6

        def fused(i):
            s = i % n_sets
            gdn.decode_step_fused(dq[s], dk_[s], dv_[s], dg[s], db[s], states[s], gate_bias=bias, gate_scale=scale,
                                  norm_weight=w, qk_eps=eps, norm_eps=eps, out=dout, state_out=states[s])

        def unfused(i):
            s = i % n_sets
            qf, kf = dq[s].float(), dk_[s].float()
            qn = (qf * torch.rsqrt((qf * qf).sum(-1, keepdim=True) + eps)).to(torch.bfloat16)
            kn = (kf * torch.rsqrt((kf * kf).sum(-1, keepdim=True) + eps)).to(torch.bfloat16)
            g = -scale * torch.nn.functional.softplus(dg[s] + bias)
            beta = torch.sigmoid(db[s])
            o, _ = gdn.decode_step(qn, kn, dv_[s], g, beta, states[s], state_out=states[s])
            of = o.float()
            dout.copy_(of * torch.rsqrt((of * of).mean(-1, keepdim=True) + eps) * w)

        for i in range(2 * n_sets):
            fused(i)
            unfused(i)
        torch.cuda.synchronize()
        gdn.profile_enable(True)
        for i in range(steps_per_graph):
            fused(i)
        torch.cuda.synchronize()
        gdn.profile_enable(False)
        kern = mean_by_name(gdn.profile_collect())["decode_fused"][0]
        us = replay_us(fused, steps_per_graph)
        us_unfused = replay_us(unfused, steps_per_graph)
        nbytes = decode_bytes(B) + 2 * HV * 4 + DV * 4
        return {
            "batch": B,
            "state_sets": n_sets,
            "us_per_step_graph": round(us, 3),
            "kernel_us": round(kern * 1e3, 3),
            "tokens_per_s": round(B / (us * 1e-6), 1),
            "bytes_per_step": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "unfused_us_per_step_graph": round(us_unfused, 3),
            "fusion_speedup": round(us_unfused / us, 2),
        }

    log("decode legs")
    dec_b1 = decode_leg(1, 1, 200, 1001)
    dec_b1_cold = decode_leg(1, 256, 256, 1001)
    dec_b32 = decode_leg(32, 8, 64, 1004)
    dec_b32_warm = decode_leg(32, 1, 64, 1004)  # one 64 MiB state set: it stays in the Infinity Cache
    log(f"decode B=1: {dec_b1}")
    log(f"decode B=1 cold: {dec_b1_cold}")
    log(f"decode B=32 cold: {dec_b32}")
    log(f"decode B=32 warm: {dec_b32_warm}")
    fused_b1 = fused_leg(1, 1, 200, 2001)
    fused_b1_cold = fused_leg(1, 256, 256, 2001)
    fused_b32 = fused_leg(32, 8, 64, 2004)
    log(f"fused decode B=1: {fused_b1}")
    log(f"fused decode B=1 cold: {fused_b1_cold}")
    log(f"fused decode B=32 cold: {fused_b32}")

    # ------------------------------------------------------------ direct scan
    scan = None
    if not args.no_scan:
        outs, sts = torch.empty_like(out), torch.empty_like(st)
        for _ in range(2):
            gdn.prefill_scan(q, k, v, g, beta, cu, None, out=outs, state_out=sts)
        torch.cuda.synchronize()
        gdn.profile_enable(True)
        n_scan = max(3, K // 10)
        t2 = time.perf_counter()
        for _ in range(n_scan):
            gdn.prefill_scan(q, k, v, g, beta, cu, None, out=outs, state_out=sts)
        torch.cuda.synchronize()
        scan_wall = (time.perf_counter() - t2) * 1e3 / n_scan
        gdn.profile_enable(False)
        scan_ms = mean_by_name(gdn.profile_collect())["scan"][0]
        scan = {"ms_per_call": round(scan_wall, 4), "kernel_ms": round(scan_ms, 4),
                "tokens_per_s": round(T / (scan_wall * 1e-3), 1),
                "chunked_speedup": round(scan_wall / ms_step, 2)}
        log(f"direct scan: {scan}")

    # ------------------------------------------------------------ scan vs chunked over prompt length
    # One sequence of T tokens (16 q/k and 32 v heads, d = 128, bf16, inputs
    # drawn on the device with the workloads' distributions), both kernels,
    # 10 untimed calls each, then reps rounds whose order alternates (scan
    # first in even rounds, chunked first in odd ones), each call timed by
    # HIP events; median, p10 and p90 per kernel.  The scan is skipped at
    # 131072 tokens (about 30 ms a call).
    crossover = None
    if not args.no_crossover and not args.no_scan:
        crossover = {"reps": args.crossover_reps, "warmup": 10, "lengths": {}}
        gen = torch.Generator(device=dev)
        for TC in (64, 256, 1024, 4096, 16384, 65536, 131072):
            gen.manual_seed(7000 + TC)
            unit = lambda x: (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
            qC = unit(torch.randn((TC, HQK, DK), generator=gen, device=dev))
            kC = unit(torch.randn((TC, HQK, DK), generator=gen, device=dev))
            vC = torch.randn((TC, HV, DV), generator=gen, device=dev).to(torch.bfloat16)
            bC = torch.sigmoid(torch.randn((TC, HV), generator=gen, device=dev))
            gC = -torch.nn.functional.softplus(torch.randn((TC, HV), generator=gen, device=dev) + 2.0)
            cuC = torch.tensor([0, TC], dtype=torch.int32, device=dev)
            oC = torch.empty((TC, HV, DV), dtype=torch.bfloat16, device=dev)
            sC = torch.empty((1, HV, DV, DK), dtype=torch.float32, device=dev)
            wsC = gdn.alloc_workspace(gdn.chunked_workspace_bytes(1, TC, HQK, HV, DK, DV, gdn.GDN_DTYPE_BF16, CHUNK),
                                      dev)
            calls = {"chunked": lambda: gdn.prefill_chunked(qC, kC, vC, gC, bC, cuC, None, out=oC, state_out=sC,
                                                             chunk_size=CHUNK, workspace=wsC)}
            if TC < 131072:
                calls["scan"] = lambda: gdn.prefill_scan(qC, kC, vC, gC, bC, cuC, None, out=oC, state_out=sC)
            for fn in calls.values():
                for _ in range(10):
                    fn()
            torch.cuda.synchronize()
            times = {name: [] for name in calls}
            names = list(calls)
            for r in range(args.crossover_reps):
                order = names if r % 2 == 0 else names[::-1]
                evs = []
                for name in order:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    calls[name]()
                    e1.record()
                    evs.append((name, e0, e1))
                torch.cuda.synchronize()
                for name, e0, e1 in evs:
                    times[name].append(e0.elapsed_time(e1) * 1e3)
            res = {}
            for name, ts in times.items():
                ts = np.array(ts)
                med = float(np.median(ts))
                res[name] = {"median_us": round(med, 2), "p10_us": round(float(np.percentile(ts, 10)), 2),
                             "p90_us": round(float(np.percentile(ts, 90)), 2),
                             "tokens_per_s": round(TC / (med * 1e-6), 1)}
            if "scan" in res:
                res["chunked_speedup"] = round(res["scan"]["median_us"] / res["chunked"]["median_us"], 3)
            crossover["lengths"][str(TC)] = res
            log(f"crossover T={TC}: {res}")
            del qC, kC, vC, bC, gC, oC, sC, wsC
            torch.cuda.empty_cache()
        # the shortest measured length from which on the chunked form is faster at every measured length
        sp = {int(t): r["chunked_speedup"] for t, r in crossover["lengths"].items() if "chunked_speedup" in r}
        crossover["chunked_faster_from_tokens"] = next(
            (t for t in sorted(sp) if all(sp[u] > 1.0 for u in sp if u >= t)), None)

    # ------------------------------------------------------------ state on chip vs blockwise
    # The pages' ablation: a 2K-token prompt, the register-resident scan against
    # a blockwise scan that moves the state through memory every block.
    ablation = None
    if not args.no_scan:
        T2 = 2048
        q2, k2, v2 = q[:T2], k[:T2], v[:T2]
        g2, b2 = g[:T2].contiguous(), beta[:T2].contiguous()
        cu2 = torch.tensor([0, T2], dtype=torch.int32, device=dev)
        o2, s2 = torch.empty((T2, HV, DV), dtype=torch.bfloat16, device=dev), torch.empty_like(st)

        def time_call(fn, n=5):
            fn()
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t3) * 1e3 / n

        state_bytes = HV * DV * DK * 4
        ablation = {"prompt_tokens": T2,
                    "resident_ms": round(time_call(lambda: gdn.prefill_scan(q2, k2, v2, g2, b2, cu2, None, out=o2,
                                                                             state_out=s2)), 4)}
        for blk in (32, 16):
            ms = time_call(lambda: gdn.prefill_scan_blockwise(q2, k2, v2, g2, b2, cu2, None, out=o2, state_out=s2,
                                                              state_block=blk))
            trips = (T2 - 1) // blk
            ablation[f"blockwise_{blk}"] = {"ms": round(ms, 4), "state_round_trips": trips,
                                            "state_mib_moved": round(trips * 2 * state_bytes / 2**20, 1),
                                            "slowdown": round(ms / ablation["resident_ms"], 3)}
        log(f"state residency ablation: {ablation}")

    # ------------------------------------------------------------ ragged batch
    # 32 sequences with the ragged workload's lengths (log-uniform in [256,
    # 8192], the same seeded draw), inputs drawn on the device with its
    # distributions and a per-sequence N(0, 0.02) initial state: the regime
    # where many sequences fill the chip.
    ragged = None
    if not args.no_long:
        from gated_deltanet_linear_delta_amd.workloads import ragged_lengths
        lengths = ragged_lengths(np.random.default_rng(1004), 32)
        cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        TR, NR = int(cu_np[-1]), len(lengths)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1004)
        unit = lambda x: (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        qR = unit(torch.randn((TR, HQK, DK), generator=gen, device=dev))
        kR = unit(torch.randn((TR, HQK, DK), generator=gen, device=dev))
        vR = torch.randn((TR, HV, DV), generator=gen, device=dev).to(torch.bfloat16)
        bR = torch.sigmoid(torch.randn((TR, HV), generator=gen, device=dev))
        gR = -torch.nn.functional.softplus(torch.randn((TR, HV), generator=gen, device=dev) + 2.0)
        s0R = 0.02 * torch.randn((NR, HV, DV, DK), generator=gen, device=dev)
        cuR = torch.from_numpy(cu_np).to(dev)
        oR, sR = torch.empty((TR, HV, DV), dtype=torch.bfloat16, device=dev), torch.empty_like(s0R)
        wsR = gdn.alloc_workspace(gdn.chunked_workspace_bytes(NR, TR, HQK, HV, DK, DV, gdn.GDN_DTYPE_BF16, CHUNK), dev)
        chunked_call = lambda: gdn.prefill_chunked(qR, kR, vR, gR, bR, cuR, s0R, out=oR, state_out=sR,
                                                   chunk_size=CHUNK, workspace=wsR)
        for _ in range(3):
            chunked_call()
        torch.cuda.synchronize()
        gdn.profile_enable(True)
        n_r = 10
        t3 = time.perf_counter()
        for _ in range(n_r):
            chunked_call()
        torch.cuda.synchronize()
        ms_r = (time.perf_counter() - t3) * 1e3 / n_r
        gdn.profile_enable(False)
        kr = {n_: round(m_ * 1e3, 2) for n_, (m_, _) in mean_by_name(gdn.profile_collect()).items()}
        nbytes = TR * (2 * HQK * DK * 2 + 2 * HV * DV * 2 + 2 * HV * 4) + NR * HV * DV * DK * 4 * 2
        ragged = {"sequences": NR, "tokens": TR, "chunked_ms": round(ms_r, 4),
                  "tokens_per_s": round(TR / (ms_r * 1e-3), 1), "kernels_us": kr,
                  "mfma_util": round(prefill_flops(TR) / (ms_r * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                  "algorithmic_bytes": nbytes,
                  "hbm_frac": round(nbytes / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if not args.no_scan:
            gdn.prefill_scan(qR, kR, vR, gR, bR, cuR, s0R, out=oR, state_out=sR)
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            for _ in range(3):
                gdn.prefill_scan(qR, kR, vR, gR, bR, cuR, s0R, out=oR, state_out=sR)
            torch.cuda.synchronize()
            ragged["scan_ms"] = round((time.perf_counter() - t3) * 1e3 / 3, 4)
        del qR, kR, vR, bR, gR, s0R, oR, sR, wsR
        torch.cuda.empty_cache()
        log(f"ragged batch: {ragged}")

    # ------------------------------------------------------------ expert GEMM on 4-bit weights
    # The pages' other ablation: 4-bit group-affine expert weights rebuilt
    # inside the grouped GEMM against rebuilding the whole bf16 matrix in
    # memory first.  256 experts, top 8, one projection K = 2048 -> N = 1024,
    # at prompts of 512 and 2048 tokens.
    moe = None
    if not args.no_moe:
        from gated_deltanet_linear_delta_amd.workloads import make_moe
        moe = {}
        for tok in (512, 2048):
            mi = make_moe(tok, num_experts=256, top_k=8, k=2048, n=1024, seed=5000 + tok)
            bfd = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(dev)
            xm, offm = bfd(mi.x), torch.from_numpy(mi.expert_offsets.astype(np.int32)).to(dev)
            cm, sm, bm = torch.from_numpy(mi.codes).to(dev), bfd(mi.scales), bfd(mi.biases)
            ym = torch.empty((xm.shape[0], 1024), dtype=torch.bfloat16, device=dev)
            wm = torch.empty((256, 1024, 2048), dtype=torch.bfloat16, device=dev)
            pm = gdn.moe_pack_q4(cm)  # codes in the tiled layout (a one-time step at weight load)
            fused = lambda: gdn.moe_gemm_q4(xm, offm, cm, sm, bm, y=ym)
            fused_packed = lambda: gdn.moe_gemm_q4_packed(xm, offm, pm, sm, bm, y=ym)
            two_pass = lambda: (gdn.dequant_q4(cm, sm, bm, weights=wm), gdn.moe_gemm_bf16(xm, offm, wm, y=ym))
            for fn in (fused, fused_packed, two_pass, fused, fused_packed):
                for _ in range(3):
                    fn()
            torch.cuda.synchronize()
            res = {}
            for name, fn in (("fused", fused), ("fused_packed", fused_packed), ("two_pass", two_pass)):
                # wall time per call with profiling off (best of 5 runs of 20 calls), then the
                # kernels' own durations from a separate pass with HIP events
                best = float("inf")
                for _ in range(5):
                    t3 = time.perf_counter()
                    for _ in range(20):
                        fn()
                    torch.cuda.synchronize()
                    best = min(best, (time.perf_counter() - t3) * 1e6 / 20)
                res[name + "_us"] = round(best, 2)
                gdn.profile_enable(True)
                for _ in range(20):
                    fn()
                torch.cuda.synchronize()
                gdn.profile_enable(False)
                res[name + "_kernels_us"] = {n_: round(m_ * 1e3, 2) for n_, (m_, _) in
                                             mean_by_name(gdn.profile_collect()).items()}
            M = int(xm.shape[0])
            nbytes = cm.numel() + 2 * 2 * sm.numel() + 2 * xm.numel() + 2 * ym.numel() + 4 * offm.numel()
            kern = res["fused_kernels_us"]["moe_gemm_q4"]
            kern_p = res["fused_packed_kernels_us"]["moe_gemm_q4_packed"]
            res.update({"packed_hbm_frac": round(nbytes / (kern_p * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "packed_speedup": round(res["fused_us"] / res["fused_packed_us"], 3),"routed_rows": M, "rows_per_expert_max": int(np.diff(mi.expert_offsets).max()),
                        "algorithmic_bytes": nbytes,
                        "hbm_gbs": round(nbytes / (kern * 1e-6) / 1e9, 1),
                        "hbm_frac": round(nbytes / (kern * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "tflops": round(2.0 * M * 2048 * 1024 / (kern * 1e-6) / 1e12, 1),
                        "mfma_util": round(2.0 * M * 2048 * 1024 / (kern * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                        "fusion_speedup": round(res["two_pass_us"] / res["fused_us"], 2)})
            moe[f"tokens_{tok}"] = res
            del xm, cm, pm, sm, bm, ym, wm
        torch.cuda.empty_cache()
        log(f"expert GEMM on 4-bit weights: {moe}")

    # ------------------------------------------------------------ decode attention at long contexts
    # One decode step of the attention layer at the pages' long contexts:
    # fixed-block with packed query heads (the library's choice), the
    # unpacked and general-layout ablations, and packs of 4.
    attention = None
    if not args.no_attention:
        from gated_deltanet_linear_delta_amd.workloads import attention_device
        attention = {"shape": {"batch": 1, "h_q": 16, "h_kv": 2, "head_dim": 256, "cache": "bf16"}}
        variants = (("fixed_block_packed8", "fixed_block", 8), ("fixed_block_packed4", "fixed_block", 4),
                    ("fixed_block_unpacked", "fixed_block", 1), ("general_packed8", "general", 8))
        for TA in (32768, 65536, 131072):
            qa, ka, va, cla, sca = attention_device([TA], seed=TA)
            oa = torch.empty_like(qa)
            cache_bytes = 2 * ka.numel() * 2
            res = {"cache_bytes": cache_bytes}
            for name, layout, hp in variants:
                wsa = gdn.alloc_workspace(gdn.attention_decode_workspace_bytes(1, 16, 2, 256, TA, sca, layout, hp, 0),
                                          dev)

                def att(_i=0):
                    gdn.attention_decode(qa, ka, va, cla, sca, layout=layout, heads_per_group=hp, out=oa,
                                         workspace=wsa)

                att()
                torch.cuda.synchronize()
                gdn.profile_enable(True)
                for _ in range(5):
                    att()
                torch.cuda.synchronize()
                gdn.profile_enable(False)
                kern = {n_: round(m_ * 1e3, 2) for n_, (m_, _) in mean_by_name(gdn.profile_collect()).items()}
                slow = layout == "general"
                per_graph = 2 if slow else 20
                graph = torch.cuda.CUDAGraph()
                sa = torch.cuda.Stream()
                sa.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(sa):
                    with torch.cuda.graph(graph, stream=sa):
                        for _ in range(per_graph):
                            att()
                torch.cuda.current_stream().wait_stream(sa)
                graph.replay()
                torch.cuda.synchronize()
                reps = 5 if slow else 50
                t3 = time.perf_counter()
                for _ in range(reps):
                    graph.replay()
                torch.cuda.synchronize()
                us = (time.perf_counter() - t3) * 1e6 / (reps * per_graph)
                res[name] = {"us": round(us, 2), "kernels_us": kern,
                             "cache_gbs": round(cache_bytes / (us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(cache_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
                del graph, wsa
            best = res["fixed_block_packed8"]["us"]
            res["packing_speedup"] = round(res["fixed_block_unpacked"]["us"] / best, 3)
            res["fixed_block_speedup"] = round(res["general_packed8"]["us"] / best, 3)
            attention[f"context_{TA}"] = res
            log(f"decode attention at {TA}: {res}")
            del qa, ka, va, oa
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ bounded prompt segments
    # One 131072-token prompt (the long workload's shape; inputs drawn on the
    # device with the same distributions), chunked in one call with a
    # whole-prompt workspace, and in segments with a per-segment workspace.
    segmented = None
    if not args.no_long:
        TL = 131072
        gen = torch.Generator(device=dev)
        gen.manual_seed(1003)

        def unit_bf16(shape):
            x = torch.randn(shape, generator=gen, device=dev)
            return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

        qL, kL = unit_bf16((TL, HQK, DK)), unit_bf16((TL, HQK, DK))
        vL = torch.randn((TL, HV, DV), generator=gen, device=dev).to(torch.bfloat16)
        bL = torch.sigmoid(torch.randn((TL, HV), generator=gen, device=dev))
        gL = -torch.nn.functional.softplus(torch.randn((TL, HV), generator=gen, device=dev) + 2.0)
        cuL = torch.tensor([0, TL], dtype=torch.int32, device=dev)
        oL = torch.empty((TL, HV, DV), dtype=torch.bfloat16, device=dev)
        sL = torch.empty_like(st)
        full_ws = gdn.chunked_workspace_bytes(1, TL, HQK, HV, DK, DV, gdn.GDN_DTYPE_BF16, CHUNK)
        wsL = gdn.alloc_workspace(full_ws, dev)

        def timed(fn, n=5):
            fn()
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t3) * 1e3 / n

        segmented = {"prompt_tokens": TL, "whole_prompt": {
            "ms": round(timed(lambda: gdn.prefill_chunked(qL, kL, vL, gL, bL, cuL, None, out=oL, state_out=sL,
                                                          chunk_size=CHUNK, workspace=wsL)), 3),
            "workspace_mib": round(full_ws / 2**20, 1)}}
        o_ref = oL.clone()
        for L in (8192, 4096):
            need = gdn.segmented_workspace_bytes(1, TL, HQK, HV, DK, DV, gdn.GDN_DTYPE_BF16, CHUNK, L)
            ms = timed(lambda: gdn.prefill_segmented(qL, kL, vL, gL, bL, cuL, None, out=oL, state_out=sL,
                                                     chunk_size=CHUNK, segment_tokens=L, workspace=wsL))
            torch.cuda.synchronize()
            segmented[f"segments_{L}"] = {"ms": round(ms, 3), "workspace_mib": round(need / 2**20, 1),
                                          "output_equal": bool(torch.equal(oL, o_ref))}
        segmented["tokens_per_s_whole"] = round(TL / (segmented["whole_prompt"]["ms"] * 1e-3), 1)
        del qL, kL, vL, bL, gL, oL, wsL, o_ref
        torch.cuda.empty_cache()
        log(f"segmented long prompt: {segmented}")

    # ------------------------------------------------------------ measured roofs
    # The box's practical roofs beside the data-sheet peaks: a 1 GiB device
    # copy (read and written once) and a bf16 8192^3 GEMM through torch.mm
    # (the vendor library), each the median of 20 event-timed runs after 5
    # untimed ones.
    def measured_roofs():
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]

        def median_s(fn):
            for _ in range(5):
                fn()
            for e0, e1 in ev:
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3

        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        copy_gbs = 2 * src.numel() * 4 / median_s(lambda: dst.copy_(src)) / 1e9
        del src, dst
        n = 8192
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        gemm_tflops = 2 * n ** 3 / median_s(lambda: torch.mm(a, b, out=c)) / 1e12
        del a, b, c
        torch.cuda.empty_cache()
        return {"copy_gbs": round(copy_gbs, 1), "gemm_bf16_tflops": round(gemm_tflops, 1),
                "prefill_hbm_frac_of_copy": round(achieved / copy_gbs, 4),
                "prefill_mfma_frac_of_gemm": round(flops / (ms_step * 1e-3) / (gemm_tflops * 1e12), 4),
                "decode_b32_frac_of_copy": round(dec_b32["hbm_gbs"] / copy_gbs, 4),
                "method": "1 GiB fp32 device-to-device copy (torch copy_, the runtime's copy kernel) and bf16 "
                          "8192^3 torch.mm, medians of 20 HIP-event-timed runs"}

    roofs = measured_roofs()
    log(f"measured roofs: {roofs}")

    # ------------------------------------------------------------ CPU baseline: the oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_leg(log)
        log(f"cpu baseline: {cpu}")

    line = {
        "metric": "GDN prefill tokens/s @T=4096 (MFMA util) + decode tokens/s (HBM GB/s frac)",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gated delta rule chunked prefill, 1 x 4096 tokens, 16 qk / 32 v heads, "
                               "d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 gate/state, zero initial state",
                   "batch": 1, "seq_len": T, "h_qk": HQK, "h_v": HV, "d_k": DK, "d_v": DV, "chunk": CHUNK},
        "mfma_util": round(mfma_util, 4),
        "algorithmic_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        # the same count with the Gram products formed per value head instead of
        # once per query/key head (140,629 instead of 132,437 flop per token and
        # value head at this shape)
        "mfma_util_dense": round(prefill_flops(T, hqk=HV) / (ms_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
        "kernels_us": {n: round(m * 1e3, 2) for n, (m, _) in per_kernel.items()},
        "call_us_events": call_stats,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "algorithmic_bytes": dom_bytes, "kernel_us": round(dom_ms * 1e3, 2),
                     "mfma_busy": counter_figures()["call_mfma_busy"]},
        # from the committed rocprofv3 counter summaries (None when taken on another kernel source)
        "counters": counter_figures(),
        "measured_roofs": roofs,
        "decode": {"b1_warm": dec_b1, "b1_cold": dec_b1_cold, "b32_cold": dec_b32, "b32_warm": dec_b32_warm},
        "decode_fused": {"b1_warm": fused_b1, "b1_cold": fused_b1_cold, "b32_cold": fused_b32},
        "state_residency_ablation": ablation,
        "segmented_prefill": segmented,
        "ragged_prefill": ragged,
        "moe_gemm_q4": moe,
        "attention_decode": attention,
        "scan": scan,
        "crossover": crossover,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
