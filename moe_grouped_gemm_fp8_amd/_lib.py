"""ctypes binding of libfg8.so (the C ABI declared in include/fg8.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  PyTorch provides device memory and the current stream.  If the
library has not been built this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfg8.so")

FG8_OK, FG8_EINVAL, FG8_EUNSUPPORTED, FG8_EHIP = 0, 1, 2, 3
OUT_F32, OUT_BF16 = 0, 1
SCALE_KINDS = {"1x128": 0, "128x128": 1, "mx": 2, "1x128_t": 3}

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_ptr = ctypes.c_void_p

_SIGNATURES = {
    "fp8_quantize": [_c_ptr, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr],
    "fp8_quantize_bf16": [_c_ptr, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr],
    "gemm_fp8_blockscaled": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int, _c_i64, _c_i64,
                             _c_i64, _c_ptr, ctypes.c_size_t, _c_ptr],
    "gemm_fp8_blockscaled_noalloc": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int,
                                     _c_i64, _c_i64, _c_i64, _c_ptr],
    "grouped_gemm_fp8_contiguous": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int,
                                    _c_i64, _c_i64, _c_i64, _c_i32, _c_ptr],
    "grouped_gemm_fp8_contiguous_swiglu": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                           _c_i64, _c_i64, _c_i64, _c_i32, _c_ptr],
    "grouped_gemm_fp8_kgrouped": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int,
                                  _c_i32, _c_i64, _c_i64, _c_i64, _c_ptr],
    "grouped_gemm_fp8_masked": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int,
                                _c_i32, _c_i64, _c_i64, _c_i64, _c_ptr],
    "gemm_mxfp8": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int, _c_i32, _c_i64,
                   _c_i64, _c_i64, _c_ptr],
    "grouped_gemm_mxfp8_contiguous": [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, ctypes.c_int,
                                      _c_i64, _c_i64, _c_i64, _c_i32, _c_ptr],
    "moe_contiguous_layout_fp8": [_c_ptr, _c_i32, _c_i64, _c_i64, _c_ptr, _c_i32, _c_i32, _c_i64,
                                  _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr],
    "fg8_moe_capacity": [_c_i64, _c_i32, _c_i32],
    "fg8_gemm_workspace_bytes": [_c_i64, _c_i64, _c_i64],
    "fg8_tile_choice": [_c_i32, _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_ptr],
    "fg8_last_error": [],
    "fg8_version": [],
}
_RESTYPES = {"fg8_gemm_workspace_bytes": ctypes.c_size_t, "fg8_last_error": ctypes.c_char_p,
             "fg8_moe_capacity": ctypes.c_int64}

_lib = None
_lock = threading.Lock()


class Fg8Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"fg8 status {status}: {message}")
        self.status = status


def lib():
    """Load libfg8.so once.  Raises if it is missing: the HIP path has no
    substitute."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is not built; run "
                                       "`python -m moe_grouped_gemm_fp8_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                for name, args in _SIGNATURES.items():
                    fn = getattr(L, name)
                    fn.argtypes = args
                    fn.restype = _RESTYPES.get(name, ctypes.c_int)
                _lib = L
    return _lib


def _check(status):
    if status != FG8_OK:
        raise Fg8Error(status, lib().fg8_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _fp8(t, name):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return _dev(t, torch.uint8, name)


def _out_code(dtype):
    if dtype == torch.float32:
        return OUT_F32
    if dtype == torch.bfloat16:
        return OUT_BF16
    raise TypeError("output dtype must be float32 or bfloat16")


def version() -> int:
    return lib().fg8_version()


def tile_choice(mode, m, n, k, groups=1, num_cus=None):
    """The tiling the library picks for a GEMM of this shape (fg8_tile_choice;
    mode 0 dense, 1 contiguous, 2 masked, 3 K-grouped): dict of bm, bn,
    splits, grid, raster.  num_cus defaults to the current device's."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    out = (ctypes.c_int32 * 5)()
    _check(lib().fg8_tile_choice(mode, m, n, k, groups, num_cus, ctypes.cast(out, ctypes.c_void_p)))
    return dict(zip(("bm", "bn", "splits", "grid", "raster"), list(out)))


# --------------------------------------------------------------- quantize
def fp8_quantize(x, kind="1x128", q=None, scales=None):
    """x float32 or bfloat16 [..., rows, cols] -> (q uint8, scales); see fg8.h
    for layouts ("1x128_t": groups of 128 rows, q [..., cols, rows]).  A
    bfloat16 source quantizes exactly like its float32 value."""
    bf16 = x.dtype == torch.bfloat16
    _dev(x, torch.bfloat16 if bf16 else torch.float32, "x")
    code = SCALE_KINDS[kind]
    *lead, rows, cols = x.shape
    batch = 1
    for d in lead:
        batch *= d
    if q is None:
        shape = (*lead, cols, rows) if kind == "1x128_t" else x.shape
        q = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        if kind == "1x128_t":
            scales = torch.empty((*lead, rows // 128, cols), dtype=torch.float32, device=x.device)
        elif kind == "1x128":
            scales = torch.empty((*lead, cols // 128, rows), dtype=torch.float32, device=x.device)
        elif kind == "128x128":
            scales = torch.empty((*lead, -(-rows // 128), cols // 128), dtype=torch.float32,
                                 device=x.device)
        else:
            scales = torch.empty((*lead, rows, cols // 32), dtype=torch.uint8, device=x.device)
    fn = lib().fp8_quantize_bf16 if bf16 else lib().fp8_quantize
    _check(fn(_ptr(x), batch, rows, cols, code, _ptr(q), _ptr(scales), _stream()))
    return q, scales


# --------------------------------------------------------------- GEMMs
def gemm_workspace_bytes(m, n, k) -> int:
    return int(lib().fg8_gemm_workspace_bytes(m, n, k))


_ws_cache = {}


def _workspace(nbytes, device):
    """A zero-initialised workspace per (device, stream); the kernels leave its
    counters at zero, so it is reused as is."""
    if nbytes == 0:
        return None
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def gemm_fp8_blockscaled(a, sa, b, sb, out_dtype=torch.bfloat16, out=None, workspace=None):
    """D [m, n] = A B^T with a [m, k] e4m3, sa [k/128, m], b [n, k], sb [ceil(n/128), k/128]."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.float32, "sa"); _dev(sb, torch.float32, "sb")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or sa.shape != (k // 128, m) or sb.shape != (-(-n // 128), k // 128):
        raise ValueError("operand shapes disagree")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    need = gemm_workspace_bytes(m, n, k)
    ws = workspace if workspace is not None else _workspace(need, a.device)
    _check(lib().gemm_fp8_blockscaled(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out),
                                      _out_code(out.dtype), m, n, k, _ptr(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(),
                                      _stream()))
    return out


def gemm_fp8_blockscaled_noalloc(a, sa, b, sb, out_dtype=torch.bfloat16, out=None):
    """gemm_fp8_blockscaled without a workspace: the split-K scratch is the
    library's static per-GPU array (see fg8.h).  `out` must be given by
    callers that cannot allocate; calls that overlap on one GPU race."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.float32, "sa"); _dev(sb, torch.float32, "sb")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or sa.shape != (k // 128, m) or sb.shape != (-(-n // 128), k // 128):
        raise ValueError("operand shapes disagree")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    if out.shape != (m, n):
        raise ValueError("output shape disagrees")
    _check(lib().gemm_fp8_blockscaled_noalloc(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out),
                                              _out_code(out.dtype), m, n, k, _stream()))
    return out


def grouped_gemm_fp8_contiguous(a, sa, b, sb, block_expert, out_dtype=torch.bfloat16, out=None):
    """Contiguous layout: a [m_total, k], sa [k/128, m_total], b [E, n, k],
    sb [E, ceil(n/128), k/128], block_expert int32 [m_total/128]."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.float32, "sa"); _dev(sb, torch.float32, "sb")
    _dev(block_expert, torch.int32, "block_expert")
    m, k = a.shape
    E, n, kb = b.shape
    if kb != k or sa.shape != (k // 128, m) or sb.shape != (E, -(-n // 128), k // 128) \
            or block_expert.shape != (m // 128,):
        raise ValueError("operand shapes disagree")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    _check(lib().grouped_gemm_fp8_contiguous(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                             _ptr(block_expert), _ptr(out), _out_code(out.dtype),
                                             m, n, k, E, _stream()))
    return out


def grouped_gemm_fp8_contiguous_swiglu(a, sa, b, sb, block_expert, q_out=None, s_out=None):
    """The contiguous grouped GEMM with W1 (rows interleaved in 128-row gate /
    up blocks, see fg8.h) and the SiLU-gated activation plus its 1x128
    quantization fused into the epilogue: a [m_total, k], sa [k/128, m_total],
    b [E, n, k], sb [E, n/128, k/128], block_expert int32 [m_total/128] ->
    (q_out uint8 [m_total, n/2], s_out float32 [n/256, m_total]).  Rows of
    skipped blocks (expert id out of range) are left as they were."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.float32, "sa"); _dev(sb, torch.float32, "sb")
    _dev(block_expert, torch.int32, "block_expert")
    m, k = a.shape
    E, n, kb = b.shape
    if kb != k or sa.shape != (k // 128, m) or sb.shape != (E, -(-n // 128), k // 128) \
            or block_expert.shape != (m // 128,):
        raise ValueError("operand shapes disagree")
    if q_out is None:
        q_out = torch.empty((m, n // 2), dtype=torch.uint8, device=a.device)
    if s_out is None:
        s_out = torch.empty((n // 256, m), dtype=torch.float32, device=a.device)
    _dev(q_out, torch.uint8, "q_out"); _dev(s_out, torch.float32, "s_out")
    if q_out.shape != (m, n // 2) or s_out.shape != (n // 256, m):
        raise ValueError("output shapes disagree")
    _check(lib().grouped_gemm_fp8_contiguous_swiglu(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                                    _ptr(block_expert), _ptr(q_out), _ptr(s_out),
                                                    m, n, k, E, _stream()))
    return q_out, s_out


def grouped_gemm_fp8_kgrouped(a, sa, b, sb, k_offsets, out_dtype=torch.float32, out=None):
    """Weight-gradient layout: a [m, k_total], sa [k_total/128, m], b [n, k_total],
    sb [k_total/128, n] (1x128 along K on both), k_offsets int32 [G + 1]
    (device) -> d [G, m, n] with d[g] = A[:, K_g] B[:, K_g]^T."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.float32, "sa"); _dev(sb, torch.float32, "sb")
    _dev(k_offsets, torch.int32, "k_offsets")
    m, k = a.shape
    n = b.shape[0]
    G = k_offsets.shape[0] - 1
    if b.shape != (n, k) or sa.shape != (k // 128, m) or sb.shape != (k // 128, n) or G < 1:
        raise ValueError("operand shapes disagree")
    if out is None:
        out = torch.empty((G, m, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    if out.shape != (G, m, n):
        raise ValueError("output shape disagrees")
    _check(lib().grouped_gemm_fp8_kgrouped(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(k_offsets),
                                           _ptr(out), _out_code(out.dtype), G, m, n, k, _stream()))
    return out


def grouped_gemm_fp8_masked(a, sa, b, sb, valid_rows, out_dtype=torch.bfloat16, out=None):
    """Masked layout: a [E, cap, k], sa [E, k/128, cap], b [E, n, k],
    sb [E, ceil(n/128), k/128], valid_rows int32 [E] (device).  Rows at or
    past valid_rows[e] of `out` are left as they were."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.float32, "sa"); _dev(sb, torch.float32, "sb")
    _dev(valid_rows, torch.int32, "valid_rows")
    E, cap, k = a.shape
    n = b.shape[1]
    if b.shape != (E, n, k) or sa.shape != (E, k // 128, cap) \
            or sb.shape != (E, -(-n // 128), k // 128) or valid_rows.shape != (E,):
        raise ValueError("operand shapes disagree")
    if out is None:
        out = torch.zeros((E, cap, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    _check(lib().grouped_gemm_fp8_masked(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(valid_rows),
                                         _ptr(out), _out_code(out.dtype), E, cap, n, k, _stream()))
    return out


def gemm_mxfp8(a, sa, b, sb, valid_rows=None, out_dtype=torch.bfloat16, out=None):
    """MXFP8: a [G, m, k], sa uint8 [G, m, k/32], b [G, n, k], sb uint8 [G, n, k/32],
    valid_rows None or int32 [G] (device)."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.uint8, "sa"); _dev(sb, torch.uint8, "sb")
    G, m, k = a.shape
    n = b.shape[1]
    if b.shape != (G, n, k) or sa.shape != (G, m, k // 32) or sb.shape != (G, n, k // 32):
        raise ValueError("operand shapes disagree")
    if valid_rows is not None:
        _dev(valid_rows, torch.int32, "valid_rows")
    if out is None:
        alloc = torch.empty if valid_rows is None else torch.zeros
        out = alloc((G, m, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    _check(lib().gemm_mxfp8(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(valid_rows), _ptr(out),
                            _out_code(out.dtype), G, m, n, k, _stream()))
    return out


def grouped_gemm_mxfp8_contiguous(a, sa, b, sb, block_expert, out_dtype=torch.bfloat16, out=None):
    """Contiguous layout with MXFP8 operands: a [m_total, k], sa uint8
    [m_total, k/32], b [E, n, k], sb uint8 [E, n, k/32], block_expert int32
    [m_total/128]."""
    _fp8(a, "a"); _fp8(b, "b")
    _dev(sa, torch.uint8, "sa"); _dev(sb, torch.uint8, "sb")
    _dev(block_expert, torch.int32, "block_expert")
    m, k = a.shape
    E, n, kb = b.shape
    if kb != k or sa.shape != (m, k // 32) or sb.shape != (E, n, k // 32) \
            or block_expert.shape != (m // 128,):
        raise ValueError("operand shapes disagree")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _dev(out, out.dtype, "out")
    _check(lib().grouped_gemm_mxfp8_contiguous(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                                               _ptr(block_expert), _ptr(out),
                                               _out_code(out.dtype), m, n, k, E, _stream()))
    return out


# --------------------------------------------------------------- MoE routing
def moe_capacity(tokens, topk, num_experts) -> int:
    """Rows of a contiguous layout that hold any routing of these sizes."""
    return int(lib().fg8_moe_capacity(tokens, topk, num_experts))


def moe_contiguous_layout_fp8(x, topk_ids, num_experts, m_cap=None, out=None):
    """x float32 or bfloat16 [tokens, hidden], topk_ids int32 [tokens, topk]
    (device) -> dict of q uint8 [m_cap, hidden], sa [hidden/128, m_cap],
    block_expert int32 [m_cap/128], row_token int32 [m_cap], token_row int32
    [tokens, topk], expert_offsets int32 [E + 1], expert_counts int32 [E], all
    on the device: the operands of grouped_gemm_fp8_contiguous plus the row
    map and its inverse.  `out`, a
    dict like the one returned, gives the buffers to fill."""
    bf16 = x.dtype == torch.bfloat16
    _dev(x, torch.bfloat16 if bf16 else torch.float32, "x")
    _dev(topk_ids, torch.int32, "topk_ids")
    tokens, hidden = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != tokens:
        raise ValueError("topk_ids must be [tokens, topk]")
    topk = topk_ids.shape[1]
    if m_cap is None:
        m_cap = moe_capacity(tokens, topk, num_experts)
    dev = x.device
    shapes = {"q": ((m_cap, hidden), torch.uint8), "sa": ((hidden // 128, m_cap), torch.float32),
              "block_expert": ((m_cap // 128,), torch.int32), "row_token": ((m_cap,), torch.int32),
              "token_row": ((tokens, topk), torch.int32),
              "expert_offsets": ((num_experts + 1,), torch.int32),
              "expert_counts": ((num_experts,), torch.int32)}
    if out is not None:
        for name, (shape, dtype) in shapes.items():
            _dev(out[name], dtype, name)
            if tuple(out[name].shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
    else:
        out = {name: torch.empty(shape, dtype=dtype, device=dev)
               for name, (shape, dtype) in shapes.items()}
    _check(lib().moe_contiguous_layout_fp8(
        _ptr(x), int(bf16), tokens, hidden, _ptr(topk_ids), topk, num_experts, m_cap,
        _ptr(out["q"]), _ptr(out["sa"]), _ptr(out["block_expert"]), _ptr(out["row_token"]),
        _ptr(out["token_row"]), _ptr(out["expert_offsets"]), _ptr(out["expert_counts"]),
        _stream()))
    return out
