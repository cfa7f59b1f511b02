"""Every entry point captured in a HIP graph gives, on each replay, the bytes
of the same call made eagerly.

The library launches kernels only (no memsets, copies or allocations), so a
captured call must replay exactly.  Each graph is replayed three times, with
eager library calls and unrelated torch work between the replays and a
synchronisation after each, and every replay is compared with the eager
result.  The benchmark times decode and attention this way.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_delta_amd import gdn
from gated_deltanet_linear_delta_amd.workloads import make_attention, make_decode, make_moe, make_prefill

from helpers import dev_prefill, f32, torch_io

pytestmark = pytest.mark.gpu


def check_replays(call, outputs):
    """call(outs) runs the library into the tensors outs; outputs() makes a fresh set."""
    ref = outputs()
    call(ref)
    torch.cuda.synchronize()
    outs = outputs()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(outs)  # warm-up on the capture stream
        side.synchronize()
        for t in outs:
            t.zero_()
        with torch.cuda.graph(graph, stream=side):
            call(outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        other = outputs()
        call(other)  # eager work between the replays
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        for a, b in zip(other, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("chunk", [0, 64])
def test_graph_prefill(chunk):
    inp = make_prefill([300, 0, 129], 4, 8, 128, 128, "bf16", 1.0, 0.02, seed=31)
    d = dev_prefill(inp)
    T = inp.q.shape[0]
    ws = gdn.alloc_workspace(gdn.chunked_workspace_bytes(3, T, 4, 8, 128, 128, gdn.GDN_DTYPE_BF16, 64)) \
        if chunk else None

    def outputs():
        return [torch.empty((T, 8, 128), dtype=torch.bfloat16, device="cuda"),
                torch.empty((3, 8, 128, 128), dtype=torch.float32, device="cuda")]

    def call(o):
        if chunk:
            gdn.prefill_chunked(**d, out=o[0], state_out=o[1], chunk_size=chunk, workspace=ws)
        else:
            gdn.prefill_scan(**d, out=o[0], state_out=o[1])

    check_replays(call, outputs)


def test_graph_segmented():
    inp = make_prefill([700, 50], 4, 8, 128, 128, "bf16", 1.0, 0.02, seed=32)
    d = dev_prefill(inp)
    T = inp.q.shape[0]
    ws = gdn.alloc_workspace(gdn.segmented_workspace_bytes(2, T, 4, 8, 128, 128, gdn.GDN_DTYPE_BF16, 64, 256))

    def outputs():
        return [torch.empty((T, 8, 128), dtype=torch.bfloat16, device="cuda"),
                torch.empty((2, 8, 128, 128), dtype=torch.float32, device="cuda")]

    check_replays(lambda o: gdn.prefill_segmented(**d, out=o[0], state_out=o[1], chunk_size=64,
                                                  segment_tokens=256, workspace=ws), outputs)


@pytest.mark.parametrize("fused", [False, True])
def test_graph_decode(fused):
    dec = make_decode(1, 8, 16, 32, 128, 128, "bf16", 2.0, 0.02, seed=33)
    q, k, v = (torch_io(x[0], "bf16") for x in (dec.q, dec.k, dec.v))
    g, beta, s0 = f32(dec.g[0]), f32(dec.beta[0]), f32(dec.state)

    def outputs():
        return [torch.empty((8, 32, 128), dtype=torch.bfloat16, device="cuda"),
                torch.empty((8, 32, 128, 128), dtype=torch.float32, device="cuda")]

    def call(o):
        if fused:
            gdn.decode_step_fused(q, k, v, g, beta, s0, out=o[0], state_out=o[1])
        else:
            gdn.decode_step(q, k, v, g, beta, s0, out=o[0], state_out=o[1])

    check_replays(call, outputs)


def test_graph_moe():
    m = make_moe(200, num_experts=16, top_k=4, k=256, n=256, seed=34)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()
    x, off = bf(m.x), torch.from_numpy(m.expert_offsets.astype(np.int32)).cuda()
    c, s, b = torch.from_numpy(m.codes).cuda(), bf(m.scales), bf(m.biases)
    check_replays(lambda o: gdn.moe_gemm_q4(x, off, c, s, b, y=o[0]),
                  lambda: [torch.empty((x.shape[0], 256), dtype=torch.bfloat16, device="cuda")])
    # the code pack and the GEMM on packed codes, captured together
    check_replays(lambda o: gdn.moe_gemm_q4_packed(x, off, gdn.moe_pack_q4(c, packed=o[1]), s, b, y=o[0]),
                  lambda: [torch.empty((x.shape[0], 256), dtype=torch.bfloat16, device="cuda"),
                           torch.empty_like(c)])


@pytest.mark.parametrize("layout", ["general", "fixed_block"])
def test_graph_attention(layout):
    inp = make_attention([3000, 17, 0], 16, 2, 256, None, seed=35)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()
    q, k, v = bf(inp.q), bf(inp.k_cache), bf(inp.v_cache)
    cl = torch.tensor(inp.context_lens, dtype=torch.int32, device="cuda")
    ws = gdn.alloc_workspace(gdn.attention_decode_workspace_bytes(3, 16, 2, 256, k.shape[2], inp.scale, layout))
    check_replays(lambda o: gdn.attention_decode(q, k, v, cl, inp.scale, layout=layout, out=o[0], workspace=ws),
                  lambda: [torch.empty_like(q)])
