"""Python binding of libmoegmm.so: the routed-expert W4A16 grouped matmul for
MI355X (gfx950).

Thin ctypes marshalling over the C ABI in include/moe_gmm.h: every function
takes torch CUDA tensors, passes their device pointers and the current HIP
stream, allocates outputs with torch, and raises on a non-zero status.  All
arithmetic runs in the library's HIP kernels; there is no fallback path.  The
library is loaded on first use and its absence is an error.
"""

import ctypes
import os

import torch

__all__ = [
    "MXFP4", "NVFP4", "W_BF16", "F32", "BF16", "GMM_AUTO", "GMM_STREAM", "GMM_TILED", "ACT_NONE", "ACT_SILU_MUL",
    "MoeGmmError", "library", "route_sort", "route_sort_workspace_bytes", "packed_weight_bytes", "mxfp4_encode",
    "moe_gmm", "moe_combine", "mxfp4_to_nvfp4", "debug_decode", "bf16_encode",
    "mxfp4_quantize", "moe_gmm_w4a4",
]

MXFP4, NVFP4, W_BF16 = 0, 1, 2
F32, BF16 = 0, 1
GMM_AUTO, GMM_STREAM, GMM_TILED = 0, 1, 2
ACT_NONE, ACT_SILU_MUL = 0, 1

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoegmm.so")
_lib = None

_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route_sort_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "moe_route_sort": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_sort_noalloc": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_packed_weight_bytes": (_sz, [ctypes.c_int, _i32, _i32, _i32]),
    "mxfp4_encode": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_bf16_encode": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "moe_mxfp4_quantize": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "moe_gmm_w4a4": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp,
                                    ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "moe_gmm": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _i32,
                               _vp, ctypes.c_int, _vp]),
    "moe_gmm_ex": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _i32,
                                  _vp, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_gmm_act": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _i32,
                                   _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_combine": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _i32, _i32, _i32, _vp,
                                   ctypes.c_int, _vp]),
    "moe_mxfp4_to_nvfp4": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_debug_decode": (ctypes.c_int, [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _vp]),
    "moe_calib_mfma_bf16": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "moe_calib_hbm_read": (ctypes.c_int, [_vp, _sz, _i32, _vp, _vp]),
    "moe_calib_mfma_parts": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _sz, _vp, _sz, ctypes.c_float, _i32, _i32,
                                            _vp, _vp]),
}


class MoeGmmError(RuntimeError):
    pass


def library():
    """The loaded libmoegmm.so (ctypes.CDLL).  torch is imported first so the
    library binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MoeGmmError(
                "libmoegmm.so is not built (%s); run python -m moe_grouped_gemm_route_amd.build"
                % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        msg = library().moe_status_string(status).decode()
        raise MoeGmmError("libmoegmm status %d: %s" % (status, msg))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoeGmmError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise MoeGmmError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise MoeGmmError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise MoeGmmError("%s must have %d dims" % (name, ndim))
    return t


def _bits16(t, name):
    """bf16 tensors (or their uint16/int16 bit views) as a 16-bit view."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return _dev(t, torch.int16, name)


def route_sort_workspace_bytes(T, k, E):
    """moe_route_sort_workspace_bytes: device workspace bytes of a route sort
    of T tokens x k slots over E experts (0 when none is needed)."""
    return int(library().moe_route_sort_workspace_bytes(T, k, E))


def route_sort(topk_ids, E, ws=None):
    """moe_route_sort.  topk_ids [T, k] int32 -> dict of int32 tensors
    group_offsets [E+1], sorted_token, sorted_pair, pair_row [T*k] and
    err_count [1].  ws: a device tensor of at least
    route_sort_workspace_bytes(T, k, E) bytes, or None to allocate one."""
    _dev(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    out = {
        "group_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "sorted_token": torch.empty(T * k, dtype=torch.int32, device=dev),
        "sorted_pair": torch.empty(T * k, dtype=torch.int32, device=dev),
        "pair_row": torch.empty(T * k, dtype=torch.int32, device=dev),
        "err_count": torch.empty(1, dtype=torch.int32, device=dev),
    }
    need = route_sort_workspace_bytes(T, k, E)
    if ws is None and need > 0:
        ws = torch.empty((need + 3) // 4, dtype=torch.int32, device=dev)
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
            raise MoeGmmError("ws must be a contiguous CUDA (HIP) tensor")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(library().moe_route_sort(
        _ptr(topk_ids), T, k, E, _ptr(out["group_offsets"]), _ptr(out["sorted_token"]),
        _ptr(out["sorted_pair"]), _ptr(out["pair_row"]), _ptr(out["err_count"]), _ptr(ws), ws_bytes,
        _stream()))
    return out


def packed_weight_bytes(fmt, E, N, K):
    n = library().moe_packed_weight_bytes(fmt, E, N, K)
    if n == 0:
        raise MoeGmmError("unsupported weight shape E=%d N=%d K=%d" % (E, N, K))
    return n


def mxfp4_encode(codes, scales, tensor_scale=None, fmt=MXFP4, err_count=None):
    """mxfp4_encode.  codes [E, N, K/2] uint8, scales [E, N, K/32] (MXFP4) or
    [E, N, K/16] (NVFP4) uint8, tensor_scale [E] float32 (NVFP4 only).
    Returns the packed uint8 buffer.  err_count: an optional [1] int32 device
    tensor that receives the number of scale values outside the exact-decode
    domain."""
    _dev(codes, torch.uint8, "codes", 3)
    _dev(scales, torch.uint8, "scales", 3)
    E, N, K2 = codes.shape
    K = 2 * K2
    per = 32 if fmt == MXFP4 else 16
    if tuple(scales.shape) != (E, N, K // per):
        raise MoeGmmError("scales must be [E, N, K/%d]" % per)
    if fmt == NVFP4:
        _dev(tensor_scale, torch.float32, "tensor_scale", 1)
    packed = torch.empty(packed_weight_bytes(fmt, E, N, K), dtype=torch.uint8, device=codes.device)
    if err_count is not None:
        _dev(err_count, torch.int32, "err_count", 1)
    _check(library().mxfp4_encode(fmt, _ptr(codes), _ptr(scales), _ptr(tensor_scale), E, N, K,
                                  _ptr(packed), _ptr(err_count), _stream()))
    return packed


def bf16_encode(weights):
    """moe_bf16_encode.  weights [E, N, K] bfloat16 (or its int16/uint16 bit
    view) -> the packed uint8 buffer of the bf16 comparison arm."""
    wb = _bits16(weights, "weights")
    if wb.dim() != 3:
        raise MoeGmmError("weights must be [E, N, K]")
    E, N, K = wb.shape
    packed = torch.empty(packed_weight_bytes(W_BF16, E, N, K), dtype=torch.uint8, device=wb.device)
    _check(library().moe_bf16_encode(_ptr(wb), E, N, K, _ptr(packed), _stream()))
    return packed


def moe_gmm(packed, fmt, E, N, K, x, group_offsets, M, row_index=None, out_dtype=F32,
            kernel=GMM_AUTO, out=None, act=ACT_NONE):
    """moe_gmm_act.  x: bf16 [T, K] (gathered through row_index) or [M, K].
    Returns y [M, N] (act=ACT_NONE) or [M, N/2] (act=ACT_SILU_MUL), float32 or
    bfloat16."""
    _dev(packed, torch.uint8, "packed", 1)
    xb = _bits16(x, "x")
    _dev(group_offsets, torch.int32, "group_offsets", 1)
    if group_offsets.numel() != E + 1:
        raise MoeGmmError("group_offsets must have E+1 entries")
    if xb.dim() != 2 or xb.shape[1] != K:
        raise MoeGmmError("x must be [rows, K]")
    if row_index is None:
        if xb.shape[0] < M:
            raise MoeGmmError("x must have M rows when row_index is None")
    else:
        _dev(row_index, torch.int32, "row_index", 1)
        if row_index.numel() < M:
            raise MoeGmmError("row_index must have M entries")
    if packed.numel() < packed_weight_bytes(fmt, E, N, K):
        raise MoeGmmError("packed buffer too small")
    dt = torch.float32 if out_dtype == F32 else torch.bfloat16
    cols = N // 2 if act == ACT_SILU_MUL else N
    if out is None:
        out = torch.empty((M, cols), dtype=dt, device=packed.device)
    else:
        _dev(out, dt, "out", 2)
        if tuple(out.shape) != (M, cols):
            raise MoeGmmError("out must be [M, %d]" % cols)
    _check(library().moe_gmm_act(_ptr(packed), fmt, E, N, K, _ptr(xb), xb.shape[0], _ptr(row_index),
                                 _ptr(group_offsets), M, _ptr(out), out_dtype, act, kernel,
                                 _stream()))
    return out


def mxfp4_quantize(x):
    """moe_mxfp4_quantize.  x bf16 [R, K] -> (codes [R, K/2] uint8, scales
    [R, K/32] uint8)."""
    xb = _bits16(x, "x")
    if xb.dim() != 2 or xb.shape[1] % 32:
        raise MoeGmmError("x must be [R, K] with K a multiple of 32")
    R, K = xb.shape
    codes = torch.empty((R, K // 2), dtype=torch.uint8, device=xb.device)
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device=xb.device)
    _check(library().moe_mxfp4_quantize(_ptr(xb), R, K, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def moe_gmm_w4a4(packed, E, N, K, xq_codes, xq_scales, group_offsets, M, row_index=None,
                 out_dtype=F32, act=ACT_NONE, out=None, fmt=MXFP4, err_count=None):
    """moe_gmm_w4a4.  xq_codes [rows, K/2], xq_scales [rows, K/32] from
    mxfp4_quantize; packed MXFP4 or NVFP4 (power-of-two block scales)
    weights.  Returns y [M, N] or [M, N/2].  err_count: an optional [1] int32
    device tensor that receives the NVFP4 weight blocks whose scales do not
    qualify."""
    _dev(packed, torch.uint8, "packed", 1)
    _dev(xq_codes, torch.uint8, "xq_codes", 2)
    _dev(xq_scales, torch.uint8, "xq_scales", 2)
    _dev(group_offsets, torch.int32, "group_offsets", 1)
    rows = xq_codes.shape[0]
    if tuple(xq_codes.shape) != (rows, K // 2) or tuple(xq_scales.shape) != (rows, K // 32):
        raise MoeGmmError("xq_codes must be [rows, K/2] and xq_scales [rows, K/32]")
    if group_offsets.numel() != E + 1:
        raise MoeGmmError("group_offsets must have E+1 entries")
    if row_index is None:
        if rows < M:
            raise MoeGmmError("the activations must have M rows when row_index is None")
    else:
        _dev(row_index, torch.int32, "row_index", 1)
        if row_index.numel() < M:
            raise MoeGmmError("row_index must have M entries")
    if packed.numel() < packed_weight_bytes(fmt, E, N, K):
        raise MoeGmmError("packed buffer too small")
    dt = torch.float32 if out_dtype == F32 else torch.bfloat16
    cols = N // 2 if act == ACT_SILU_MUL else N
    if out is None:
        out = torch.empty((M, cols), dtype=dt, device=packed.device)
    else:
        _dev(out, dt, "out", 2)
        if tuple(out.shape) != (M, cols):
            raise MoeGmmError("out must be [M, %d]" % cols)
    if err_count is not None:
        _dev(err_count, torch.int32, "err_count", 1)
    _check(library().moe_gmm_w4a4(_ptr(packed), fmt, E, N, K, _ptr(xq_codes), _ptr(xq_scales), rows,
                                  _ptr(row_index), _ptr(group_offsets), M, _ptr(out), out_dtype, act,
                                  _ptr(err_count), _stream()))
    return out


def moe_combine(y, topk_weights, pair_row, out_dtype=F32):
    """moe_combine.  y [rows, N] float32/bfloat16, topk_weights [T, k] float32,
    pair_row [T*k] int32 -> out [T, N]."""
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise MoeGmmError("y must be float32 or bfloat16")
    _dev(y, y.dtype, "y", 2)
    _dev(topk_weights, torch.float32, "topk_weights", 2)
    _dev(pair_row, torch.int32, "pair_row", 1)
    T, k = topk_weights.shape
    N = y.shape[1]
    if pair_row.numel() != T * k:
        raise MoeGmmError("pair_row must have T*k entries")
    dt = torch.float32 if out_dtype == F32 else torch.bfloat16
    out = torch.empty((T, N), dtype=dt, device=y.device)
    _check(library().moe_combine(_ptr(y), F32 if y.dtype == torch.float32 else BF16,
                                 _ptr(topk_weights), _ptr(pair_row), T, k, N, _ptr(out),
                                 out_dtype, _stream()))
    return out


def mxfp4_to_nvfp4(scales):
    """moe_mxfp4_to_nvfp4.  scales [E, N, K/32] uint8 E8M0 ->
    (block_scales [E, N, K/16] uint8 E4M3, tensor_scale [E] float32,
    err_count [1] int32)."""
    _dev(scales, torch.uint8, "scales", 3)
    E, N, KB = scales.shape
    bs = torch.empty((E, N, 2 * KB), dtype=torch.uint8, device=scales.device)
    ts = torch.empty(E, dtype=torch.float32, device=scales.device)
    err = torch.empty(1, dtype=torch.int32, device=scales.device)
    _check(library().moe_mxfp4_to_nvfp4(_ptr(scales), E, N, 32 * KB, _ptr(bs), _ptr(ts),
                                        _ptr(err), _stream()))
    return bs, ts, err


def debug_decode(packed, fmt, E, N, K):
    """moe_debug_decode -> dense bf16 bit patterns [E, N, K] (int16 view)."""
    _dev(packed, torch.uint8, "packed", 1)
    w = torch.empty((E, N, K), dtype=torch.int16, device=packed.device)
    _check(library().moe_debug_decode(_ptr(packed), fmt, E, N, K, _ptr(w), _stream()))
    return w


def calib_mfma_bf16(a, b, blocks, iters):
    """moe_calib_mfma_bf16: blocks workgroups of 4 waves, each wave issuing
    iters * 128 bf16 MFMAs (16x16x32) on register-resident fragments taken
    from a ([blocks*256*8*8] bf16 bits) and b ([blocks*256*4*8]).  Returns the
    [blocks*256] f32 sums; FLOPs = blocks * 4 * iters * 128 * 16384."""
    a = _bits16(a, "a")
    b = _bits16(b, "b")
    lanes = blocks * 256
    if a.numel() < lanes * 64 or b.numel() < lanes * 32:
        raise MoeGmmError("calib_mfma_bf16: a needs %d and b %d bf16 values" % (lanes * 64, lanes * 32))
    out = torch.empty(lanes, dtype=torch.float32, device=a.device)
    _check(library().moe_calib_mfma_bf16(_ptr(a), _ptr(b), blocks, iters, _ptr(out), _stream()))
    return out


PARTS_LDS_A, PARTS_CODES, PARTS_STAGE, PARTS_BARRIER, PARTS_REG_DECODE, PARTS_CODES_XOR = 1, 2, 4, 8, 16, 32


def calib_mfma_parts(parts, rows16, a, b, codes, x, scale, blocks, chunks):
    """moe_calib_mfma_parts: the tiled kernel's wave tile (rows16 row subtiles
    x 4 column subtiles) over chunks 128-deep chunks per wave, with the data
    movement named by parts (PARTS_* bits).  a and b as for calib_mfma_bf16;
    codes and x are device buffers (any dtype) of the code stream and the
    staging source.  Returns the [blocks*256] f32 sums; FLOPs = blocks * 4 *
    chunks * 4 * rows16 * 4 * 16384."""
    a = _bits16(a, "a")
    b = _bits16(b, "b")
    lanes = blocks * 256
    if a.numel() < lanes * 64 or b.numel() < lanes * 32:
        raise MoeGmmError("calib_mfma_parts: a needs %d and b %d bf16 values" % (lanes * 64, lanes * 32))
    for name, t in (("codes", codes), ("x", x)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise MoeGmmError("%s must be a contiguous CUDA (HIP) tensor" % name)
    out = torch.empty(lanes, dtype=torch.float32, device=a.device)
    _check(library().moe_calib_mfma_parts(parts, rows16, _ptr(a), _ptr(b), _ptr(codes),
                                          codes.numel() * codes.element_size(), _ptr(x),
                                          x.numel() * x.element_size(), float(scale), blocks, chunks, _ptr(out),
                                          _stream()))
    return out


def calib_hbm_read(src, blocks):
    """moe_calib_hbm_read: blocks workgroups of 256 threads stream the device
    buffer src (16-byte aligned, a multiple of 16 bytes) with 16-byte loads.
    Returns the [blocks * 256] uint32 XOR partials (as int32 bits)."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise MoeGmmError("src must be a contiguous CUDA (HIP) tensor")
    nbytes = src.numel() * src.element_size()
    out = torch.empty(blocks * 256, dtype=torch.int32, device=src.device)
    _check(library().moe_calib_hbm_read(_ptr(src), nbytes, blocks, _ptr(out), _stream()))
    return out
