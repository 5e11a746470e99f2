"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/attn.h declares, and rejects every invalid argument with the
documented code before any HIP call (fake device addresses are never touched).
"""
import ctypes
import math
import os
import re

import pytest

import tiled_attention_forward_attn_amd as tafa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

A = 0x10000          # fake, 16-byte aligned device addresses, far apart
GAP = 1 << 36


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", src, flags=re.M)


def header_codes():
    src = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_(?:OK|E_\w+))\s*=\s*(-?\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tafa.LIB_PATH):
        pytest.fail("libmi355attn.so is not built (run __graft_entry__.build())")
    return tafa.load()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == {"attn_fwd", "attn_fp8_quantize", "attn_lse_merge", "attn_decode",
                          "attn_decode_workspace_bytes", "attn_decode_paged", "attn_decode_noalloc",
                          "attn_fp8_quantize_rotated", "attn_strerror", "attn_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tafa.SIGNATURES)


def test_version_and_strerror(lib):
    assert tafa.version() == 10700
    codes = header_codes()
    assert codes["ATTN_OK"] == 0
    texts = {tafa.strerror(c) for c in codes.values()}
    assert len(texts) == len(codes)              # every code has its own text
    assert tafa.strerror(12345) == "unknown error code"


def fwd_args(**kw):
    a = dict(q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, B=2, H=3, N=300, d=128,
             causal=0, window=-1, scale=0.125, dtype=0, dq=None, dk=None, dv=None, stream=None)
    a.update(kw)
    return a


def call_fwd(lib, **kw):
    a = fwd_args(**kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                        a["causal"], a["window"], a["scale"], a["dtype"], a["dq"], a["dk"], a["dv"],
                        a["stream"])


E = header_codes()


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), "ATTN_E_SHAPE"), (dict(H=-2), "ATTN_E_SHAPE"), (dict(N=-5), "ATTN_E_SHAPE"),
    (dict(N=(1 << 23) + 1), "ATTN_E_SHAPE"), (dict(B=1 << 13, H=1 << 12), "ATTN_E_SHAPE"),
    (dict(d=96), "ATTN_E_HEADDIM"), (dict(d=512), "ATTN_E_HEADDIM"), (dict(d=0), "ATTN_E_HEADDIM"),
    (dict(d=256, dtype=1, dq=A + 5 * GAP, dk=A + 6 * GAP, dv=A + 7 * GAP), "ATTN_E_HEADDIM"),
    (dict(d=256, dtype=2, dv=A + 7 * GAP), "ATTN_E_HEADDIM"),
    (dict(d=256, N=(1 << 22) + 1, B=1, H=1), "ATTN_E_SHAPE"),  # 32-bit descriptor range at d = 256
    (dict(dtype=3), "ATTN_E_DTYPE"), (dict(dtype=-1), "ATTN_E_DTYPE"),
    (dict(q=None), "ATTN_E_NULL"), (dict(k=None), "ATTN_E_NULL"), (dict(v=None), "ATTN_E_NULL"),
    (dict(o=None), "ATTN_E_NULL"), (dict(lse=None), "ATTN_E_NULL"),
    (dict(dtype=1), "ATTN_E_NULL"),
    (dict(dtype=1, dq=A + 5 * GAP, dk=A + 6 * GAP), "ATTN_E_NULL"),
    (dict(causal=2), "ATTN_E_WINDOW"), (dict(causal=-1), "ATTN_E_WINDOW"),
    (dict(window=-2), "ATTN_E_WINDOW"),
    (dict(scale=math.inf), "ATTN_E_SCALE"), (dict(scale=math.nan), "ATTN_E_SCALE"),
    (dict(q=A + 8), "ATTN_E_ALIGN"), (dict(o=A + 3 * GAP + 4), "ATTN_E_ALIGN"),
    (dict(lse=A + 4 * GAP + 2), "ATTN_E_ALIGN"),
    (dict(dtype=1, dq=A + 5 * GAP + 1, dk=A + 6 * GAP, dv=A + 7 * GAP), "ATTN_E_ALIGN"),
    (dict(o=A), "ATTN_E_ALIAS"), (dict(o=A + GAP + 1024), "ATTN_E_ALIAS"),
    (dict(lse=A + 2 * GAP + 64), "ATTN_E_ALIAS"), (dict(lse=A + 3 * GAP + 16), "ATTN_E_ALIAS"),
    (dict(dtype=1, dq=A + 3 * GAP, dk=A + 6 * GAP, dv=A + 7 * GAP), "ATTN_E_ALIAS"),
    # dtype 2 (q, k bf16; v E4M3): only descale_v is required
    (dict(dtype=2), "ATTN_E_NULL"), (dict(dtype=2, dq=A + 5 * GAP, dk=A + 6 * GAP), "ATTN_E_NULL"),
    (dict(dtype=2, dv=A + 7 * GAP + 2), "ATTN_E_ALIGN"),
    (dict(dtype=2, dv=A + 3 * GAP + 64), "ATTN_E_ALIAS"),
    (dict(dtype=2, dv=A + 7 * GAP, o=A + 2 * GAP + 1024), "ATTN_E_ALIAS"),
])
def test_attn_fwd_rejects(lib, kw, code):
    assert call_fwd(lib, **kw) == E[code]


def test_attn_fwd_empty_problem_is_ok(lib):
    for kw in (dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=None, o=None, d=77)):
        assert call_fwd(lib, **kw) == E["ATTN_OK"]


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


# These calls pass validation with fake addresses and reach the launch, which
# fails cleanly only where there is no GPU.
@pytest.mark.skipif(not _no_gpu(), reason="fake device addresses would reach a real kernel")
def test_attn_fwd_output_right_after_input_is_not_alias(lib):
    # q occupies [A, A + 2*3*300*128*2); o starting right after it is legal
    qbytes = 2 * 3 * 300 * 128 * 2
    rc = call_fwd(lib, o=A + qbytes + (16 - qbytes % 16) % 16)
    assert rc != E["ATTN_E_ALIAS"]


@pytest.mark.skipif(not _no_gpu(), reason="fake device addresses would reach a real kernel")
def test_fp8_pv_checks_v_at_one_byte_per_element(lib):
    # dtype 2's v holds 1 byte per element: o right after that extent is legal,
    # while the same placement overlaps a bf16 v
    vbytes = 2 * 3 * 300 * 128
    o = A + 2 * GAP + vbytes
    assert call_fwd(lib, dtype=2, dv=A + 7 * GAP, o=o) != E["ATTN_E_ALIAS"]
    assert call_fwd(lib, dtype=0, o=o) == E["ATTN_E_ALIAS"]


def call_quant(lib, x=A, x8=A + GAP, ds=A + 2 * GAP, B=2, H=3, N=300, d=128, per_tensor=0):
    return lib.attn_fp8_quantize(x, x8, ds, B, H, N, d, per_tensor, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), "ATTN_E_SHAPE"), (dict(N=(1 << 23) + 1), "ATTN_E_SHAPE"),
    (dict(d=32), "ATTN_E_HEADDIM"), (dict(d=256), "ATTN_E_HEADDIM"),
    (dict(x=None), "ATTN_E_NULL"), (dict(x8=None), "ATTN_E_NULL"), (dict(ds=None), "ATTN_E_NULL"),
    (dict(per_tensor=2), "ATTN_E_DTYPE"),
    (dict(x=A + 8), "ATTN_E_ALIGN"), (dict(x8=A + GAP + 4), "ATTN_E_ALIGN"),
    (dict(ds=A + 2 * GAP + 2), "ATTN_E_ALIGN"),
    (dict(x8=A + 64), "ATTN_E_ALIAS"), (dict(ds=A + GAP + 128), "ATTN_E_ALIAS"),
])
def test_quantize_rejects(lib, kw, code):
    assert call_quant(lib, **kw) == E[code]


def test_quantize_empty_problem_is_ok(lib):
    assert call_quant(lib, N=0, x=None) == E["ATTN_OK"]


def test_binding_checks_before_calling(lib):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tafa.fwd(q, q, q)                        # CPU tensors are refused by the binding
    with pytest.raises(ValueError):
        tafa.quantize(q)


def test_binding_buffer_check_refuses_host_memory():
    # the check every caller-supplied output, descale and workspace goes
    # through: a host tensor for a device pointer is refused (the shape and
    # dtype refusals are exercised on the GPU, where device tensors exist)
    import torch
    t = torch.zeros(2, 3, dtype=torch.float32)
    with pytest.raises(ValueError, match="must be on"):
        tafa._check_buf("out", t, (2, 3), (torch.float32,), torch.device("cuda:0"))
    with pytest.raises(ValueError, match="must be a torch.Tensor"):
        tafa._check_buf("lse", [0.0], (1,), (torch.float32,), torch.device("cuda:0"))
    with pytest.raises(ValueError, match="workspace"):
        tafa._workspace(torch.zeros(16, dtype=torch.uint8), 16, torch.device("cuda:0"))


def call_merge(lib, op=A, lp=A + GAP, o=A + 2 * GAP, lse=A + 3 * GAP, R=3, B=2, H=3, N=300, d=128):
    return lib.attn_lse_merge(op, lp, o, lse, R, B, H, N, d, None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), "ATTN_E_SHAPE"), (dict(R=4097), "ATTN_E_SHAPE"), (dict(B=-1), "ATTN_E_SHAPE"),
    (dict(N=(1 << 23) + 1), "ATTN_E_SHAPE"),
    (dict(d=32), "ATTN_E_HEADDIM"), (dict(d=96), "ATTN_E_HEADDIM"),
    (dict(op=None), "ATTN_E_NULL"), (dict(lp=None), "ATTN_E_NULL"), (dict(o=None), "ATTN_E_NULL"),
    (dict(lse=None), "ATTN_E_NULL"),
    (dict(op=A + 4), "ATTN_E_ALIGN"), (dict(o=A + 2 * GAP + 8), "ATTN_E_ALIGN"),
    (dict(lp=A + GAP + 2), "ATTN_E_ALIGN"), (dict(lse=A + 3 * GAP + 1), "ATTN_E_ALIGN"),
    (dict(o=A + 1024), "ATTN_E_ALIAS"), (dict(lse=A + GAP + 64), "ATTN_E_ALIAS"),
    (dict(lse=A + 2 * GAP + 4096), "ATTN_E_ALIAS"),
])
def test_lse_merge_rejects(lib, kw, code):
    assert call_merge(lib, **kw) == E[code]


def test_lse_merge_empty_problem_is_ok(lib):
    assert call_merge(lib, N=0, op=None, d=77) == E["ATTN_OK"]


WS = A + 5 * GAP


def call_decode(lib, q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, B=2, H=3,
                Nq=4, Nk=1000, d=128, causal=1, scale=0.125, splits=8, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(B, H, Nq, d, splits)
    return lib.attn_decode(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, splits, ws, ws_bytes, None)


def test_decode_workspace_bytes(lib):
    assert lib.attn_decode_workspace_bytes(2, 3, 4, 128, 8) == 8 * 2 * 3 * 4 * (4 * 128 + 4)
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 64, 1) == 64 * 4 + 4
    for args in ((2, 3, 33, 128, 8), (2, 3, 4, 96, 8), (2, 3, 4, 128, 0), (-1, 3, 4, 128, 8),
                 (2, 3, 0, 128, 8)):
        assert lib.attn_decode_workspace_bytes(*args) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Nq=33), "ATTN_E_SHAPE"), (dict(Nk=3), "ATTN_E_SHAPE"), (dict(splits=0), "ATTN_E_SHAPE"),
    (dict(splits=4097), "ATTN_E_SHAPE"), (dict(B=-1), "ATTN_E_SHAPE"), (dict(Nk=(1 << 23) + 1), "ATTN_E_SHAPE"),
    (dict(d=256, ws_bytes=1 << 30), "ATTN_E_HEADDIM"),
    (dict(q=None), "ATTN_E_NULL"), (dict(v=None), "ATTN_E_NULL"), (dict(lse=None), "ATTN_E_NULL"),
    (dict(causal=2), "ATTN_E_WINDOW"), (dict(scale=math.inf), "ATTN_E_SCALE"),
    (dict(k=A + GAP + 8), "ATTN_E_ALIGN"), (dict(lse=A + 4 * GAP + 2), "ATTN_E_ALIGN"),
    (dict(ws=None), "ATTN_E_WORKSPACE"), (dict(ws=WS + 8), "ATTN_E_WORKSPACE"),
    (dict(ws_bytes=16), "ATTN_E_WORKSPACE"),
    (dict(o=A + GAP + 4096), "ATTN_E_ALIAS"), (dict(ws=A + 2 * GAP + 1024), "ATTN_E_ALIAS"),
    (dict(lse=WS + 64), "ATTN_E_ALIAS"), (dict(o=A + 4 * GAP - 64), "ATTN_E_ALIAS"),
])
def test_decode_rejects(lib, kw, code):
    assert call_decode(lib, **kw) == E[code]


def test_decode_empty_problem_is_ok(lib):
    assert call_decode(lib, Nq=0, q=None, ws=None, ws_bytes=0) == E["ATTN_OK"]


def call_paged(lib, q=A, kc=A + GAP, vc=A + 2 * GAP, table=A + 6 * GAP, lens=A + 7 * GAP,
               o=A + 3 * GAP, lse=A + 4 * GAP, B=2, H=3, Nq=4, d=128, num_pages=100, page_size=64,
               max_pages=40, causal=1, scale=0.125, splits=8, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(B, H, Nq, d, splits)
    return lib.attn_decode_paged(q, kc, vc, table, lens, o, lse, B, H, Nq, d, num_pages, page_size,
                                 max_pages, causal, scale, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=16), "ATTN_E_SHAPE"), (dict(page_size=96), "ATTN_E_SHAPE"),
    (dict(page_size=8192), "ATTN_E_SHAPE"), (dict(num_pages=0), "ATTN_E_SHAPE"),
    (dict(max_pages=0), "ATTN_E_SHAPE"), (dict(max_pages=(1 << 23) // 64 + 1), "ATTN_E_SHAPE"),
    (dict(Nq=33), "ATTN_E_SHAPE"), (dict(splits=0), "ATTN_E_SHAPE"), (dict(B=-1), "ATTN_E_SHAPE"),
    (dict(d=256, ws_bytes=1 << 30), "ATTN_E_HEADDIM"),
    (dict(q=None), "ATTN_E_NULL"), (dict(kc=None), "ATTN_E_NULL"), (dict(table=None), "ATTN_E_NULL"),
    (dict(lens=None), "ATTN_E_NULL"), (dict(lse=None), "ATTN_E_NULL"),
    (dict(causal=2), "ATTN_E_WINDOW"), (dict(scale=math.nan), "ATTN_E_SCALE"),
    (dict(vc=A + 2 * GAP + 8), "ATTN_E_ALIGN"), (dict(table=A + 6 * GAP + 2), "ATTN_E_ALIGN"),
    (dict(lens=A + 7 * GAP + 1), "ATTN_E_ALIGN"),
    (dict(ws=None), "ATTN_E_WORKSPACE"), (dict(ws_bytes=16), "ATTN_E_WORKSPACE"),
    (dict(o=A + GAP + 4096), "ATTN_E_ALIAS"), (dict(lse=A + 6 * GAP + 16), "ATTN_E_ALIAS"),
    (dict(ws=A + 7 * GAP), "ATTN_E_ALIAS"), (dict(o=A + 4 * GAP - 64), "ATTN_E_ALIAS"),
])
def test_decode_paged_rejects(lib, kw, code):
    assert call_paged(lib, **kw) == E[code]


def test_decode_paged_empty_problem_is_ok(lib):
    assert call_paged(lib, Nq=0, q=None, ws=None, ws_bytes=0) == E["ATTN_OK"]
    assert call_paged(lib, B=0, table=None, lens=None, ws=None, ws_bytes=0) == E["ATTN_OK"]


def call_noalloc(lib, q=A, k=A + GAP, v=A + 2 * GAP, o=A + 3 * GAP, lse=A + 4 * GAP, B=2, H=3, Nq=4,
                 Nk=1000, d=128, causal=1, scale=0.125, splits=8):
    return lib.attn_decode_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, splits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Nq=33), "ATTN_E_SHAPE"), (dict(Nk=3), "ATTN_E_SHAPE"), (dict(splits=0), "ATTN_E_SHAPE"),
    (dict(B=-1), "ATTN_E_SHAPE"), (dict(d=256), "ATTN_E_HEADDIM"),
    (dict(q=None), "ATTN_E_NULL"), (dict(lse=None), "ATTN_E_NULL"),
    (dict(causal=2), "ATTN_E_WINDOW"), (dict(scale=math.nan), "ATTN_E_SCALE"),
    (dict(k=A + GAP + 8), "ATTN_E_ALIGN"), (dict(o=A + GAP + 4096), "ATTN_E_ALIAS"),
    # splits * B * H * Nq * (4 d + 4) = 8 * 1024 * 32 * 516 bytes > 16 MiB: refused before any HIP call
    (dict(B=32, H=32, Nq=32, Nk=4096), "ATTN_E_SCRATCH"),
])
def test_decode_noalloc_rejects(lib, kw, code):
    assert call_noalloc(lib, **kw) == E[code]


def test_decode_noalloc_scratch_limit(lib):
    # the largest call that fits the static buffer is accepted by the checks
    # (not launched here: the sizes alone decide), one more split is refused
    limit = 16 << 20
    assert tafa.NOALLOC_SCRATCH_BYTES == limit
    need = lib.attn_decode_workspace_bytes(4, 8, 32, 128, 31)      # 31 * 1024 * 516 bytes
    assert need <= limit < lib.attn_decode_workspace_bytes(4, 8, 32, 128, 32)
    assert call_noalloc(lib, B=4, H=8, Nq=32, Nk=4096, splits=32) == E["ATTN_E_SCRATCH"]
    assert call_noalloc(lib, Nq=0, q=None) == E["ATTN_OK"]


def call_rot(lib, x=A, x8=A + GAP, ds=A + 2 * GAP, signs=A + 3 * GAP, B=2, H=3, N=300, d=128, pt=0):
    return lib.attn_fp8_quantize_rotated(x, x8, ds, signs, B, H, N, d, pt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(signs=None), "ATTN_E_NULL"), (dict(x=None), "ATTN_E_NULL"),
    (dict(signs=A + 3 * GAP + 4), "ATTN_E_ALIGN"), (dict(x8=A + GAP + 4), "ATTN_E_ALIGN"),
    (dict(d=256), "ATTN_E_HEADDIM"), (dict(d=96), "ATTN_E_HEADDIM"), (dict(N=-1), "ATTN_E_SHAPE"),
    (dict(pt=2), "ATTN_E_DTYPE"),
    (dict(signs=A + GAP + 64), "ATTN_E_ALIAS"), (dict(signs=A + 2 * GAP), "ATTN_E_ALIAS"),
])
def test_quantize_rotated_rejects(lib, kw, code):
    assert call_rot(lib, **kw) == E[code]


def test_quantize_rotated_empty_problem_is_ok(lib):
    assert call_rot(lib, N=0, x=None, signs=None) == E["ATTN_OK"]
