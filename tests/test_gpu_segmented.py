"""GPU tests of the bounded prompt-segment driver (gdn_prefill_segmented) and
of the blockwise-scan ablation (gdn_prefill_scan_blockwise).

Perplexity's "Optimizing on-device inference for Apple Silicon", section
"Bounding scratch memory by chunking the prompt", runs a long prompt in bounded
segments with the recurrent state carried between them and the output
unchanged; section "Keeping the recurrent state on chip" compares the
register-resident scan with a blockwise scan that moves the state through
memory every block.  So:

- segmented == one call, bit for bit, where the windows cut at the blocks
  the path walks (one sequence; chunks, or 4-token blocks for the scan), and
  within tolerance of the oracle where they do not;
- segmented ragged batches == the fp64 oracle within tolerance (windows then
  move the chunk boundaries of sequences that straddle them);
- blockwise scan == resident scan, bit for bit, for every block size.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import make_prefill, prefill_4096, tiny_fp32_prefill
from oracle import gated_delta_recurrence

from helpers import dev_prefill, host, out_errors, state_errors

pytestmark = pytest.mark.gpu


def one_call(d, chunk):
    if chunk == 0:
        return gdn.prefill_scan(**d)
    return gdn.prefill_chunked(**d, chunk_size=chunk)


@pytest.mark.parametrize("chunk,L", [(64, 64), (64, 256), (32, 96), (16, 1024), (0, 4), (0, 100)])
def test_segmented_single_sequence_bit_exact(chunk, L):
    inp = make_prefill([1000], 2, 4, 64, 64, "bf16", 1.0, 0.05, seed=500 + L)
    d = dev_prefill(inp)
    o1, s1 = one_call(d, chunk)
    o2, s2 = gdn.prefill_segmented(**d, chunk_size=chunk, segment_tokens=L)
    torch.cuda.synchronize()
    print(f"segmented chunk={chunk} L={L}: max |diff| out {float((o1.float() - o2.float()).abs().max()):.3e}",
          flush=True)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_segmented_scan_unaligned_vs_oracle():
    inp = make_prefill([1000], 2, 4, 64, 64, "f32", 1.0, 0.05, seed=501)
    d = dev_prefill(inp)
    o, s = gdn.prefill_segmented(**d, chunk_size=0, segment_tokens=7)
    torch.cuda.synchronize()
    o_ref, s_ref = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.state_in)
    eo, es = out_errors(host(o), o_ref, inp.cu_seqlens), state_errors(host(s), s_ref)
    print(f"segmented scan L=7: out {eo}; state {es}", flush=True)
    assert eo.ok("f32") and es.ok("f32"), (eo, es)


@pytest.mark.parametrize("chunk", [0, 16, 64])
def test_segmented_ragged_vs_oracle(chunk):
    lengths = [300, 0, 1000, 77, 513, 1, 129]
    inp = make_prefill(lengths, 2, 4, 128, 64, "bf16", 2.0, 0.02, seed=77)
    d = dev_prefill(inp)
    L = 256
    o, s = gdn.prefill_segmented(**d, chunk_size=chunk, segment_tokens=L)
    torch.cuda.synchronize()
    o_ref, s_ref = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.state_in)
    eo, es = out_errors(host(o), o_ref, inp.cu_seqlens), state_errors(host(s), s_ref)
    print(f"segmented ragged chunk={chunk} L={L}: out {eo}; state {es}", flush=True)
    assert eo.ok("bf16") and es.ok("bf16"), (eo, es)


def test_segmented_fp32_in_place_and_empty():
    inp = make_prefill([40, 0, 90], 2, 2, 16, 32, "f32", 0.0, 0.1, seed=9, chunk_size=16)
    d = dev_prefill(inp)
    s_io = d["state_in"].clone()
    o, s = gdn.prefill_segmented(**dict(d, state_in=s_io), state_out=s_io, chunk_size=16, segment_tokens=32)
    torch.cuda.synchronize()
    assert s.data_ptr() == s_io.data_ptr()
    o_ref, s_ref = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.state_in)
    eo, es = out_errors(host(o), o_ref, inp.cu_seqlens), state_errors(host(s), s_ref)
    print(f"segmented fp32 in place: out {eo}; state {es}", flush=True)
    assert eo.ok("f32") and es.ok("f32"), (eo, es)
    # an empty prompt still writes state_out (= state_in), for both paths
    e = make_prefill([0, 0], 2, 2, 16, 32, "f32", 0.0, 0.1, seed=10)
    de = dev_prefill(e)
    for chunk in (0, 16):
        _, se = gdn.prefill_segmented(**de, chunk_size=chunk, segment_tokens=16)
        torch.cuda.synchronize()
        assert torch.equal(se, de["state_in"])


def test_segmented_4096_prompt_bit_exact():
    # the 4096-token prompt in 1024-token segments equals one chunked call
    inp = prefill_4096()
    d = dev_prefill(inp)
    o1, s1 = gdn.prefill_chunked(**d, chunk_size=64)
    o2, s2 = gdn.prefill_segmented(**d, chunk_size=64, segment_tokens=1024)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("block", [4, 16, 32, 64, 100])
def test_blockwise_scan_equals_resident(block):
    inp = make_prefill([200, 0, 333, 64], 2, 4, 128, 32, "bf16", 1.0, 0.05, seed=40 + block)
    d = dev_prefill(inp)
    o1, s1 = gdn.prefill_scan(**d)
    o2, s2 = gdn.prefill_scan_blockwise(**d, state_block=block)
    s_io = d["state_in"].clone()
    o3, s3 = gdn.prefill_scan_blockwise(**dict(d, state_in=s_io), state_out=s_io, state_block=block)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)


def test_blockwise_scan_fp32_vs_oracle():
    inp = tiny_fp32_prefill()
    d = dev_prefill(inp)
    o, s = gdn.prefill_scan_blockwise(**d, state_block=8)
    torch.cuda.synchronize()
    o_ref, s_ref = gated_delta_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.state_in)
    eo, es = out_errors(host(o), o_ref, inp.cu_seqlens), state_errors(host(s), s_ref)
    print(f"blockwise scan fp32: out {eo}; state {es}", flush=True)
    assert eo.ok("f32") and es.ok("f32"), (eo, es)
