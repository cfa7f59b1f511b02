"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/gdn.h declares, sizes the workspace, and rejects bad
arguments with the documented status before enqueueing anything."""
import ctypes
import os
import re

import pytest

from gated_deltanet_linear_delta_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        from gated_deltanet_linear_delta_amd import build
        build.build()
    return gdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header(lib):
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in [(0, "GDN_OK"), (1, "GDN_ERR_INVALID"), (2, "GDN_ERR_UNSUPPORTED"), (3, "GDN_ERR_LAUNCH")]:
        assert lib.gdn_status_string(code).decode() == name
    assert lib.gdn_status_string(99).decode() == "GDN_ERR_UNKNOWN"


def shape(**kw):
    base = dict(num_seqs=1, total_tokens=4096, h_qk=16, h_v=32, d_k=128, d_v=128, io_dtype=gdn.GDN_DTYPE_BF16)
    base.update(kw)
    return gdn.GdnShape(**base)


def expected_workspace(n, t, h_v, c, bf16=True, h_qk=16, dk=128):
    """The per-slot (first token, length) table, padded to 256 bytes, then
    per (slot, value head), for (T + N (C - 1)) / C slots: P = K^T diag(dec) T
    as d_k / 16 row blocks x max(C, 32) / 32 token slabs (one 1 KiB plane
    each, two in fp32), the 16-row x 32-column fragments of the lower
    triangle of R = QKm T (1, 2 or 6 for C = 16, 32, 64; split into two 1 KiB
    planes each) and 3 C fp32 scalars, padded to 256 bytes; then per (slot,
    query/key head) Q and K as C / 16 row blocks x max(d_k, 32) / 32 slabs."""
    r256 = lambda x: (x + 255) // 256 * 256
    max_chunks = (t + n * (c - 1)) // c
    nf = {16: 1, 32: 2, 64: 6}[c]
    tpl = 1 if bf16 else 2
    per = r256((dk // 16) * (max(c, 32) // 32) * tpl * 1024 + nf * 2 * 1024 + 3 * c * 4)
    qk = 2 * (c // 16) * (max(dk, 32) // 32) * tpl * 1024
    return r256(8 * max_chunks) + max_chunks * h_v * per + max_chunks * h_qk * qk


def test_workspace_size(lib):
    s = shape()
    assert lib.gdn_prefill_chunked_workspace(ctypes.byref(s), 64) == expected_workspace(1, 4096, 32, 64)
    assert expected_workspace(1, 4096, 32, 64) == 512 + 64 * 32 * 29440 + 64 * 16 * 32768
    s32 = shape(io_dtype=gdn.GDN_DTYPE_F32)
    assert lib.gdn_prefill_chunked_workspace(ctypes.byref(s32), 64) == expected_workspace(1, 4096, 32, 64, False)
    assert lib.gdn_prefill_chunked_workspace(ctypes.byref(s), 48) == 0
    assert lib.gdn_prefill_chunked_workspace(None, 64) == 0
    assert lib.gdn_prefill_chunked_workspace(ctypes.byref(shape(h_v=24)), 64) == 0
    s2 = shape(num_seqs=32, total_tokens=73000)
    for c in (16, 32, 64):
        assert lib.gdn_prefill_chunked_workspace(ctypes.byref(s2), c) == expected_workspace(32, 73000, 32, c)


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation first


def prefill_args(s, **over):
    a = dict(q=FAKE, k=FAKE + 256, v=FAKE + 512, g=FAKE + 768, beta=FAKE + 1024, cu=FAKE + 1280,
             state_in=None, out=FAKE + 1536, state_out=FAKE + 1792)
    a.update(over)
    return [ctypes.byref(s) if s is not None else None, a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"],
            a["state_in"], a["out"], a["state_out"]]


@pytest.mark.parametrize("case,status", [
    (dict(s=None), 1),
    (dict(s=shape(h_v=24)), 1),
    (dict(s=shape(num_seqs=0)), 1),
    (dict(s=shape(total_tokens=-1)), 1),
    (dict(s=shape(d_k=48)), 2),
    (dict(s=shape(d_v=256)), 2),
    (dict(s=shape(io_dtype=7)), 1),
    (dict(s=shape(), q=None), 1),
    (dict(s=shape(), beta=FAKE + 4), 1),
    (dict(s=shape(), out=FAKE), 1),
    (dict(s=shape(), state_in=FAKE + 8), 1),
])
def test_prefill_rejects(lib, case, status):
    s = case.pop("s")
    args = prefill_args(s, **case)
    assert lib.gdn_prefill_scan(*args, None) == status
    assert lib.gdn_last_error().decode() != ""
    assert lib.gdn_prefill_chunked(*args, 64, FAKE + 4096, 1 << 40, None) == status


def test_chunked_rejects_chunk_and_workspace(lib):
    s = shape()
    args = prefill_args(s)
    need = lib.gdn_prefill_chunked_workspace(ctypes.byref(s), 64)
    assert lib.gdn_prefill_chunked(*args, 128, FAKE + 4096, need, None) == 2
    assert lib.gdn_prefill_chunked(*args, 64, None, need, None) == 1
    assert lib.gdn_prefill_chunked(*args, 64, FAKE + 4096 + 16, need, None) == 1
    assert lib.gdn_prefill_chunked(*args, 64, FAKE + 4096, need - 1, None) == 1
    assert "needs" in lib.gdn_last_error().decode()


def test_decode_rejects(lib):
    p = [FAKE + 256 * i for i in range(8)]
    ok = [1, 16, 32, 128, 128, gdn.GDN_DTYPE_BF16]
    assert lib.gdn_decode_step(0, 16, 32, 128, 128, 1, *p, None) == 1
    assert lib.gdn_decode_step(1, 16, 24, 128, 128, 1, *p, None) == 1
    assert lib.gdn_decode_step(1, 16, 32, 96, 128, 1, *p, None) == 2
    bad = list(p)
    bad[5] = None  # state_in is required for decode
    assert lib.gdn_decode_step(*ok, *bad, None) == 1
    bad = list(p)
    bad[6] = p[5]  # out aliases state_in
    assert lib.gdn_decode_step(*ok, *bad, None) == 1


def test_decode_fused_rejects(lib):
    p = [FAKE + 256 * i for i in range(5)]  # q_raw, k_raw, v, g_raw, beta_raw
    st_in, out, st_out = FAKE + 2048, FAKE + 2304, FAKE + 2560
    ok = [1, 16, 32, 128, 128, gdn.GDN_DTYPE_BF16]
    P = gdn.GdnFusedParams

    def call(dims=ok, ptrs=p, params=None, s_in=st_in, o=out, s_out=st_out):
        pr = ctypes.byref(params) if params is not None else None
        return lib.gdn_decode_step_fused(*dims, *ptrs, pr, s_in, o, s_out, None)

    assert call(dims=[0, 16, 32, 128, 128, 1]) == 1
    assert call(dims=[1, 16, 24, 128, 128, 1]) == 1
    assert call(dims=[1, 16, 32, 128, 96, 1]) == 2
    assert call(ptrs=[p[0], None] + p[2:]) == 1          # k_raw missing
    assert call(s_in=None) == 1                           # state_in is required
    assert call(o=st_in) == 1                             # out aliases state_in
    assert call(params=P(None, None, None, -1.0, 1e-6)) == 1
    assert call(params=P(None, None, None, 1e-6, float("nan"))) == 1
    assert call(params=P(None, None, None, 1e-6, float("inf"))) == 1
    assert call(params=P(FAKE + 3072 + 2, None, None, 1e-6, 1e-6)) == 1  # misaligned gate_bias
    assert "aligned" in lib.gdn_last_error().decode()


def test_segmented_workspace_size(lib):
    s = shape(total_tokens=131072)
    r256 = lambda x: (x + 255) // 256 * 256
    # offsets for N + 1 sequences, then one window's chunked workspace
    for L in (4096, 8192):
        assert lib.gdn_prefill_segmented_workspace(ctypes.byref(s), 64, L) == r256(8) + expected_workspace(1, L, 32, 64)
    assert lib.gdn_prefill_segmented_workspace(ctypes.byref(s), 0, 1000) == 256      # direct scan: offsets only
    # a window never exceeds the prompt
    assert lib.gdn_prefill_segmented_workspace(ctypes.byref(shape(total_tokens=100)), 64, 8192) == \
        256 + expected_workspace(1, 100, 32, 64)
    s2 = shape(num_seqs=32, total_tokens=73000)
    assert lib.gdn_prefill_segmented_workspace(ctypes.byref(s2), 32, 8192) == r256(33 * 4) + \
        expected_workspace(32, 8192, 32, 32)
    # bounded: the segmented workspace at T = 131072 is a small fraction of the whole-prompt one
    assert lib.gdn_prefill_segmented_workspace(ctypes.byref(s), 64, 8192) * 15 < \
        lib.gdn_prefill_chunked_workspace(ctypes.byref(s), 64)
    for c, L in ((64, 100), (48, 4096), (64, 0), (0, 0), (16, -16)):
        assert lib.gdn_prefill_segmented_workspace(ctypes.byref(s), c, L) == 0
    assert lib.gdn_prefill_segmented_workspace(None, 64, 4096) == 0


def test_segmented_and_blockwise_reject(lib):
    s = shape()
    args = prefill_args(s)
    need = lib.gdn_prefill_segmented_workspace(ctypes.byref(s), 64, 1024)
    ws = FAKE + 4096
    assert lib.gdn_prefill_segmented(*args, 48, 1024, ws, need, None) == 2
    assert lib.gdn_prefill_segmented(*args, 64, 1000, ws, need, None) == 1     # not a multiple of the chunk
    assert lib.gdn_prefill_segmented(*args, 64, 0, ws, need, None) == 1
    assert lib.gdn_prefill_segmented(*args, 64, 1024, None, need, None) == 1
    assert lib.gdn_prefill_segmented(*args, 64, 1024, ws + 16, need, None) == 1
    assert lib.gdn_prefill_segmented(*args, 64, 1024, ws, need - 1, None) == 1
    assert "needs" in lib.gdn_last_error().decode()
    bad = prefill_args(shape(d_k=48))
    assert lib.gdn_prefill_segmented(*bad, 64, 1024, ws, 1 << 40, None) == 2
    assert lib.gdn_prefill_scan_blockwise(*args, 0, None) == 1
    assert lib.gdn_prefill_scan_blockwise(*args, 6, None) == 1      # not a multiple of 4
    assert lib.gdn_prefill_scan_blockwise(*prefill_args(s, out=FAKE), 16, None) == 1  # out aliases q
    assert lib.gdn_prefill_scan_blockwise(*bad, 16, None) == 2


def test_empty_prompt_token_tensors_may_be_null(lib):
    # T = 0: q, k, v, g, beta and out are never touched, so NULL passes validation;
    # cu_seqlens and state_out are still required.  Only validation runs here: the
    # calls below fail on a later check (workspace) or on purpose, before any launch.
    s = shape(total_tokens=0)
    nul = [ctypes.byref(s), None, None, None, None, None, FAKE, None, None, FAKE + 256]
    assert lib.gdn_prefill_chunked(*nul, 64, None, 0, None) == 1
    assert "workspace" in lib.gdn_last_error().decode()
    nul_cu = list(nul)
    nul_cu[6] = None
    assert lib.gdn_prefill_chunked(*nul_cu, 64, FAKE + 4096, 1 << 40, None) == 1
    assert "cu_seqlens" in lib.gdn_last_error().decode()
    mis = list(nul)
    mis[1] = FAKE + 8
    assert lib.gdn_prefill_chunked(*mis, 64, FAKE + 4096, 1 << 40, None) == 1
    assert "aligned" in lib.gdn_last_error().decode()


def test_moe_rejects(lib):
    S = gdn.GdnMoeShape
    p = [FAKE + 256 * i for i in range(6)]  # x, offsets, codes, scales, biases, y
    ok = S(8, 100, 256, 256)
    assert lib.gdn_moe_gemm_q4(None, *p, None) == 1
    assert lib.gdn_moe_gemm_q4(ctypes.byref(S(0, 100, 256, 256)), *p, None) == 1
    assert lib.gdn_moe_gemm_q4(ctypes.byref(S(8, -1, 256, 256)), *p, None) == 1
    assert lib.gdn_moe_gemm_q4(ctypes.byref(S(8, 100, 192, 256)), *p, None) == 2    # k not a multiple of 128
    assert lib.gdn_moe_gemm_q4(ctypes.byref(S(5000, 100, 256, 256)), *p, None) == 2  # too many experts
    assert lib.gdn_moe_gemm_q4(ctypes.byref(S(8, 100, 256, 192)), *p, None) == 2    # n not a multiple of 128
    assert lib.gdn_moe_gemm_q4(ctypes.byref(ok), None, *p[1:], None) == 1            # x missing with rows > 0
    assert lib.gdn_moe_gemm_q4(ctypes.byref(ok), p[0], None, *p[2:], None) == 1      # offsets missing
    assert lib.gdn_moe_gemm_q4(ctypes.byref(ok), *p[:5], p[0], None) == 1           # y aliases x
    assert lib.gdn_moe_gemm_q4(ctypes.byref(ok), p[0] + 8, *p[1:], None) == 1       # misaligned x
    assert "aligned" in lib.gdn_last_error().decode()
    assert lib.gdn_dequant_q4(ctypes.byref(ok), p[2], p[3], p[4], None, None) == 1   # weights missing
    assert lib.gdn_moe_gemm_bf16(ctypes.byref(S(8, 100, 100, 256)), p[0], p[1], p[2], p[5], None) == 2
    assert lib.gdn_moe_gemm_bf16(ctypes.byref(ok), p[0], p[1], None, p[5], None) == 1
    # packed codes: the pack and the packed GEMM validate like the others
    big = 8 * 256 * 128  # bytes of the codes at the ok shape
    assert lib.gdn_moe_pack_q4(None, p[2], p[2] + big, None) == 1
    assert lib.gdn_moe_pack_q4(ctypes.byref(S(8, 100, 192, 256)), p[2], p[2] + big, None) == 2
    assert lib.gdn_moe_pack_q4(ctypes.byref(ok), None, p[2] + big, None) == 1
    assert lib.gdn_moe_pack_q4(ctypes.byref(ok), p[2], None, None) == 1
    assert lib.gdn_moe_pack_q4(ctypes.byref(ok), p[2], p[2] + 8 + big, None) == 1   # misaligned
    assert lib.gdn_moe_pack_q4(ctypes.byref(ok), p[2], p[2] + big - 1024, None) == 1  # overlaps codes
    assert "overlaps" in lib.gdn_last_error().decode()
    assert lib.gdn_moe_gemm_q4_packed(ctypes.byref(S(8, 100, 256, 192)), *p, None) == 2
    assert lib.gdn_moe_gemm_q4_packed(ctypes.byref(ok), p[0], p[1], None, *p[3:], None) == 1
    assert lib.gdn_moe_gemm_q4_packed(ctypes.byref(ok), *p[:5], p[0], None) == 1     # y aliases x


def attn_ws_expected(B, h_q, d, nb):
    """part_o [B, h_q, nb, d] fp32 padded to 256 bytes, then (max, sum) pairs."""
    rows = B * h_q * nb
    return (rows * d * 4 + 255) // 256 * 256 + rows * 8


def test_attention_workspace_size(lib):
    A, P = gdn.GdnAttnShape, gdn.GdnAttnParams
    s = A(1, 16, 2, 256, 32768)
    fixed = P(0.0625, gdn.GDN_ATTN_FIXED_BLOCK, 8, 128)
    assert lib.gdn_attention_decode_workspace(ctypes.byref(s), ctypes.byref(fixed)) == attn_ws_expected(1, 16, 256, 128)
    general = P(0.0625, gdn.GDN_ATTN_GENERAL, 0, 0)
    assert lib.gdn_attention_decode_workspace(ctypes.byref(s), ctypes.byref(general)) == 0
    # the automatic choice: fixed blocks when (batch x KV heads x packs) leaves compute units idle
    auto = lib.gdn_attention_decode_workspace(ctypes.byref(s), None)
    # (compute units / 2 groups parts, at least 32 positions each: 128 on a 256-CU device)
    assert auto in [attn_ws_expected(1, 16, 256, nb) for nb in range(2, 1025)]
    assert lib.gdn_attention_decode_workspace(ctypes.byref(A(1, 16, 2, 256, 32)), None) == 0  # one part anyway
    assert lib.gdn_attention_decode_workspace(ctypes.byref(A(512, 16, 2, 256, 4096)), None) == 0  # enough groups
    assert lib.gdn_attention_decode_workspace(ctypes.byref(A(1, 16, 2, 256, 64)), None) == attn_ws_expected(1, 16, 256, 2)
    assert lib.gdn_attention_decode_workspace(ctypes.byref(A(1, 16, 2, 96, 4096)), None) == 0  # invalid -> 0


def test_attention_rejects(lib):
    A, P = gdn.GdnAttnShape, gdn.GdnAttnParams
    p = [FAKE + 256 * i for i in range(6)]  # q, k, v, lens, out, workspace
    s = A(1, 16, 2, 256, 1024)
    ws = attn_ws_expected(1, 16, 256, 4)
    fixed = P(0.0625, gdn.GDN_ATTN_FIXED_BLOCK, 0, 4)

    def call(shape=s, params=fixed, ptrs=p, nbytes=ws):
        return lib.gdn_attention_decode(None if shape is None else ctypes.byref(shape),
                                        None if params is None else ctypes.byref(params), *ptrs[:5], ptrs[5],
                                        nbytes, None)
    assert call(shape=None) == 1
    assert call(shape=A(0, 16, 2, 256, 1024)) == 1
    assert call(shape=A(1, 12, 8, 256, 1024)) == 1                 # h_q not a multiple of h_kv
    assert call(shape=A(1, 16, 2, 96, 1024)) == 2                  # head size not built
    assert call(shape=A(1, 16, 2, 256, 0)) == 1
    assert call(shape=A(1, 16, 2, 256, (1 << 24) + 1)) == 1
    assert call(params=P(float("nan"), 2, 0, 4)) == 1
    assert call(params=P(0.1, 7, 0, 4)) == 1                       # not a layout
    assert call(params=P(0.1, 2, 3, 4)) == 1                       # 3 heads per workgroup
    assert call(params=P(0.1, 2, 16, 4)) == 1                      # more than 8
    assert call(shape=A(1, 12, 2, 256, 1024), params=P(0.1, 2, 4, 4)) == 1  # 4 does not divide 6
    assert call(params=P(0.1, 2, 0, 1025)) == 1                    # more parts than positions
    assert call(params=P(0.1, 2, 0, -1)) == 1
    for i in range(5):                                             # each pointer missing
        ptrs = list(p)
        ptrs[i] = None
        assert call(ptrs=ptrs) == 1
    ptrs = list(p)
    ptrs[0] += 8                                                   # misaligned q
    assert call(ptrs=ptrs) == 1 and "aligned" in lib.gdn_last_error().decode()
    ptrs = list(p)
    ptrs[3] += 2                                                   # misaligned context_lens
    assert call(ptrs=ptrs) == 1
    ptrs = list(p)
    ptrs[4] = ptrs[1]                                              # out aliases the key cache
    assert call(ptrs=ptrs) == 1
    ptrs = list(p)
    ptrs[5] = None
    assert call(ptrs=ptrs) == 1                                    # workspace missing
    ptrs[5] = FAKE + 128
    assert call(ptrs=ptrs) == 1                                    # not 256-byte aligned
    assert call(nbytes=ws - 1) == 1
    assert "needs" in lib.gdn_last_error().decode()
