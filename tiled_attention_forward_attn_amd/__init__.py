"""Python binding of the MI355X tiled attention forward library.

Argument marshalling only: every step of the attention forward pass and of the
fp8 quantiser runs in the HIP kernels of libmi355attn.so, reached through its
C ABI (include/attn.h). PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or fails to load, every call
raises.

    o, lse = fwd(q, k, v, causal=False, window=-1, scale=None)      # bf16
    q8, dq = quantize(q); k8, dk = quantize(k); v8, dv = quantize(v)
    o, lse = fwd(q8, k8, v8, descales=(dq, dk, dv))                  # fp8
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmi355attn.so"
LIB_PATH = os.path.join(_HERE, LIB_NAME)
BLOCK_ROWS = 128                      # rows per fp8 scaling block

DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1
DTYPE_FP8_PV = 2

_lib: ctypes.CDLL | None = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

# name -> (restype, argtypes); mirrors include/attn.h
SIGNATURES = {
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _vp]),
    "attn_fp8_quantize": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_fp8_quantize_rotated": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_lse_merge": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_decode_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "attn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp,
                         ctypes.c_size_t, _vp]),
    "attn_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                               _f, _i, _vp, ctypes.c_size_t, _vp]),
    "attn_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_strerror": (ctypes.c_char_p, [_i]),
    "attn_version": (_i, []),
}


class AttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what} failed with code {code}: {strerror(code)}")


def load() -> ctypes.CDLL:
    """Load libmi355attn.so (built in-tree by build.py); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m tiled_attention_forward_attn_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load().attn_strerror(code).decode()


def version() -> int:
    return load().attn_version()


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_4d(name: str, t: torch.Tensor):
    if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 4-D [B, H, N, d] CUDA tensor")


def _check_buf(name: str, t: torch.Tensor, shape, dtypes, device: torch.device):
    """A caller-supplied output or auxiliary tensor must be exactly what the
    kernels read or write through its pointer: on the inputs' device,
    contiguous, of this shape and dtype. Raises ValueError otherwise (before
    any launch)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(map(str, dtypes))}, got {t.dtype}")


def _is_fp8(t: torch.Tensor) -> bool:
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        window: int = -1, scale: float | None = None, descales=None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """Attention forward through attn_fwd. Returns (o bf16 [B,H,N,d], lse fp32 [B,H,N]).

    q, k, v all bf16 (dtype 0); all E4M3 codes (uint8 / float8_e4m3fn) with
    descales=(dq, dk, dv) fp32 [B, H, ceil(N/128)] (dtype 1); or q, k bf16 and
    v E4M3 codes with descales=(None, None, dv) (dtype 2: scores in bf16, P
    and V in E4M3). scale=None means 1/sqrt(d).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_4d(name, t)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    B, H, N, d = q.shape
    q8, k8, v8 = _is_fp8(q), _is_fp8(k), _is_fp8(v)
    bf = [t.dtype == torch.bfloat16 for t in (q, k, v)]
    if q8 and k8 and v8:
        dtype = DTYPE_FP8_E4M3
    elif bf[0] and bf[1] and v8:
        dtype = DTYPE_FP8_PV
    elif all(bf):
        dtype = DTYPE_BF16
    else:
        raise ValueError("q, k, v must be all bf16, all E4M3 codes, or bf16 q, k with E4M3 v")
    if dtype != DTYPE_BF16:
        if descales is None or len(descales) != 3 or descales[2] is None:
            raise ValueError("E4M3 inputs need descales=(dq, dk, dv) (dq, dk None when q, k are bf16)")
        if dtype == DTYPE_FP8_E4M3 and (descales[0] is None or descales[1] is None):
            raise ValueError("all-E4M3 inputs need dq and dk")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = descales if dtype != DTYPE_BF16 else (None, None, None)
    if dtype == DTYPE_FP8_PV:
        dq = dk = None
    nsb = -(-N // BLOCK_ROWS)
    for name, t in (("descale_q", dq), ("descale_k", dk), ("descale_v", dv)):
        if t is not None:
            _check_buf(name, t, (B, H, nsb), (torch.float32,), q.device)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check_buf("out", out, (B, H, N, d), (torch.bfloat16,), q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_buf("lse", lse, (B, H, N), (torch.float32,), q.device)
    rc = load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                         int(causal), int(window), float(scale), dtype,
                         _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd")
    return out, lse


def quantize(x: torch.Tensor, per_tensor: bool = False, out: torch.Tensor | None = None,
             descale: torch.Tensor | None = None, stream=None,
             rotation_signs: torch.Tensor | None = None):
    """bf16 [B,H,N,d] -> (E4M3 codes uint8 [B,H,N,d], fp32 descale [B,H,ceil(N/128)]).

    rotation_signs: int8 [d] on x's device; when given, the rows are rotated
    first (attn_fp8_quantize_rotated, incoherent processing). Quantise Q and K
    with the same signs; V without."""
    _check_4d("x", x)
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    B, H, N, d = x.shape
    if rotation_signs is not None:
        _check_buf("rotation_signs", rotation_signs, (d,), (torch.int8,), x.device)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    else:
        _check_buf("out", out, (B, H, N, d), (torch.uint8, torch.float8_e4m3fn), x.device)
    if descale is None:
        descale = torch.empty((B, H, -(-N // BLOCK_ROWS)), dtype=torch.float32, device=x.device)
    else:
        _check_buf("descale", descale, (B, H, -(-N // BLOCK_ROWS)), (torch.float32,), x.device)
    if rotation_signs is None:
        rc = load().attn_fp8_quantize(_ptr(x), _ptr(out), _ptr(descale), B, H, N, d,
                                      int(per_tensor), _stream(stream))
        what = "attn_fp8_quantize"
    else:
        rc = load().attn_fp8_quantize_rotated(_ptr(x), _ptr(out), _ptr(descale), _ptr(rotation_signs),
                                              B, H, N, d, int(per_tensor), _stream(stream))
        what = "attn_fp8_quantize_rotated"
    if rc != 0:
        raise AttnError(rc, what)
    return out, descale


def merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, out: torch.Tensor | None = None,
          lse: torch.Tensor | None = None, stream=None):
    """Merge partial results over disjoint key sets through attn_lse_merge.

    o_parts fp32 [R, B, H, N, d], lse_parts fp32 [R, B, H, N] (natural-log
    softmax denominators) -> (o bf16 [B, H, N, d], lse fp32 [B, H, N])."""
    if o_parts.dim() != 5 or lse_parts.dim() != 4 or o_parts.shape[:4] != lse_parts.shape:
        raise ValueError("o_parts must be [R, B, H, N, d] and lse_parts [R, B, H, N]")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts and lse_parts must be fp32")
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if lse_parts.device != o_parts.device:
        raise ValueError("o_parts and lse_parts must be on the same device")
    R, B, H, N, d = o_parts.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=o_parts.device)
    else:
        _check_buf("out", out, (B, H, N, d), (torch.bfloat16,), o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    else:
        _check_buf("lse", lse, (B, H, N), (torch.float32,), o_parts.device)
    rc = load().attn_lse_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse), R, B, H, N, d,
                               _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_lse_merge")
    return out, lse


MAX_DECODE_Q = 32


def _workspace(ws: torch.Tensor | None, need: int, device: torch.device) -> torch.Tensor:
    """The decode workspace: allocated here when not given; a caller's must be
    a contiguous device tensor on the inputs' device (its byte size goes to the
    C ABI, which rejects one that is too small)."""
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return ws


def default_splits(B: int, H: int, Nk: int) -> int:
    """Key chunks per (b, h) for attn_decode: about 2048 single-wave
    workgroups in all, each chunk at least 256 keys."""
    return max(1, min(-(-2048 // max(1, B * H)), -(-Nk // 256), 4096))


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
           scale: float | None = None, splits: int | None = None,
           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None, stream=None):
    """Decode attention through attn_decode: q bf16 [B, H, Nq, d] (Nq <= 32,
    the sequence's last positions) against k, v bf16 [B, H, Nk, d].
    Returns (o bf16 [B, H, Nq, d], lse fp32 [B, H, Nq]). The workspace (device
    bytes) is allocated here when not given."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_4d(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if splits is None:
        splits = default_splits(B, H, Nk)
    lib = load()
    need = lib.attn_decode_workspace_bytes(B, H, Nq, d, splits)
    workspace = _workspace(workspace, need, q.device)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check_buf("out", out, (B, H, Nq, d), (torch.bfloat16,), q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        _check_buf("lse", lse, (B, H, Nq), (torch.float32,), q.device)
    rc = lib.attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d,
                         int(causal), float(scale), int(splits), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_decode")
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20     # ATTN_NOALLOC_SCRATCH_BYTES


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                   scale: float | None = None, splits: int | None = None,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None, stream=None):
    """decode() through attn_decode_noalloc: the library keeps the partials in
    its own static device buffer, so the C call allocates nothing (out and lse
    are allocated here when not given). Calls that overlap on one device race
    on that buffer."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_4d(name, t)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if splits is None:
        splits = default_splits(B, H, Nk)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check_buf("out", out, (B, H, Nq, d), (torch.bfloat16,), q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        _check_buf("lse", lse, (B, H, Nq), (torch.float32,), q.device)
    rc = load().attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d,
                                    int(causal), float(scale), int(splits), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_decode_noalloc")
    return out, lse


def decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_table: torch.Tensor, seq_lens: torch.Tensor, *, causal: bool = False,
                 scale: float | None = None, splits: int | None = None,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, stream=None):
    """Decode attention through attn_decode_paged: q bf16 [B, H, Nq, d] against
    the paged pools k_cache, v_cache bf16 [num_pages, H, page_size, d], with
    block_table int32 [B, max_pages] and seq_lens int32 [B] on the device.
    Returns (o bf16 [B, H, Nq, d], lse fp32 [B, H, Nq]). splits defaults to the
    value for the longest sequence the table can address."""
    _check_4d("q", q)
    _check_4d("k_cache", k_cache)
    _check_4d("v_cache", v_cache)
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    B, H, Nq, d = q.shape
    num_pages, page_size = k_cache.shape[0], k_cache.shape[2]
    if k_cache.shape != (num_pages, H, page_size, d) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, H, page_size, d] with q's H and d")
    for name, t, shape in (("block_table", block_table, None), ("seq_lens", seq_lens, (B,))):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous int32 tensor on q's device")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    if not (q.device == k_cache.device == v_cache.device):
        raise ValueError("q, k_cache and v_cache must be on the same device")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if splits is None:
        splits = default_splits(B, H, max_pages * page_size)
    lib = load()
    need = lib.attn_decode_workspace_bytes(B, H, Nq, d, splits)
    workspace = _workspace(workspace, need, q.device)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check_buf("out", out, (B, H, Nq, d), (torch.bfloat16,), q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        _check_buf("lse", lse, (B, H, Nq), (torch.float32,), q.device)
    rc = lib.attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                               _ptr(seq_lens), _ptr(out), _ptr(lse), B, H, Nq, d, num_pages,
                               page_size, max_pages, int(causal), float(scale), int(splits),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_decode_paged")
    return out, lse


__all__ = ["fwd", "quantize", "merge", "decode", "decode_paged", "decode_noalloc", "default_splits", "load", "strerror", "version", "AttnError", "LIB_PATH",
           "SIGNATURES", "BLOCK_ROWS", "DTYPE_BF16", "DTYPE_FP8_E4M3", "DTYPE_FP8_PV"]
