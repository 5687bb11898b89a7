"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/moe_gmm.h declares, and rejects bad arguments before any
HIP call (so nothing is launched)."""

import ctypes
import os
import re

import pytest

import moe_grouped_gemm_route_amd as moe
from moe_grouped_gemm_route_amd.synth import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_gmm.h")

OK, ERR_NULL, ERR_SHAPE, ERR_FORMAT = 0, 1, 2, 3
FAKE = ctypes.c_void_p(1 << 20)          # never dereferenced: calls fail validation first
FAKE_ALIGNED = ctypes.c_void_p(1 << 30)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return moe.library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"moe_route_sort", "mxfp4_encode", "moe_gmm", "moe_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe._SIGNATURES)


def test_status_strings(lib):
    for s in range(6):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def test_packed_bytes(lib):
    for c in CONFIGS.values():
        E, N, K = c["E"], c["N"], c["K"]
        mx = lib.moe_packed_weight_bytes(0, E, N, K)
        # codes 4 bits each + one scale byte per 32 weights (K/128 chunks padded to groups of 4)
        groups = -(-(K // 128) // 4)
        assert mx == E * N * K // 2 + E * (N // 16) * groups * 256
        nv = lib.moe_packed_weight_bytes(1, E, N, K)
        groups = -(-(K // 128) // 2)
        # + the tensor scales and one flag word per 16-column subtile, each padded to 256 bytes
        assert nv == (E * N * K // 2 + E * (N // 16) * groups * 256 + ((4 * E + 255) // 256) * 256
                      + ((4 * E * (N // 16) + 255) // 256) * 256)
    assert lib.moe_packed_weight_bytes(0, 8, 512, 100) == 0
    assert lib.moe_packed_weight_bytes(0, 8, 48, 256) == 0
    assert lib.moe_packed_weight_bytes(7, 8, 512, 256) == 0


def _ws_formula(T, k, E):
    """The workspace size the header documents: none up to 4,096 pairs, else
    4 E bytes per segment of max(1024, ceil(M / 64) rounded up to 512)
    pairs."""
    M = T * k
    if M <= 4096:
        return 0
    s = max(1024, -(-(-(-M // 64)) // 512) * 512)
    return 4 * E * -(-M // s)


def test_route_sort_workspace_bytes(lib):
    f = lib.moe_route_sort_workspace_bytes
    for T, k, E in [(64, 2, 8), (64, 6, 256), (256, 6, 256), (682, 6, 256), (4096, 1, 1024),
                    (4097, 1, 256), (4096, 6, 256), (1 << 21, 8, 1024), (1 << 22, 4, 256),
                    (3000, 8, 1024), (100000, 7, 3)]:
        assert f(T, k, E) == _ws_formula(T, k, E), (T, k, E)
    assert f(4096, 6, 256) == 24 * 256 * 4            # the 4,096-token prefill: 24 segments
    assert f(4097, 1, 256) == 5 * 256 * 4
    assert f(1 << 21, 8, 1024) == 64 * 1024 * 4       # the largest accepted problem: 256 KiB
    assert f(0, 6, 256) == 0 and f(4, 2, 1025) == 0 and f(1 << 22, 8, 8) == 0


def test_route_sort_validation(lib):
    f = lib.moe_route_sort
    assert f(None, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_NULL
    assert f(FAKE, 0, 2, 8, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_SHAPE
    assert f(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_SHAPE
    assert f(FAKE, 4, 2, 1025, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_SHAPE
    assert f(FAKE, 1 << 22, 8, 8, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ERR_SHAPE
    need = lib.moe_route_sort_workspace_bytes(4096, 6, 256)
    assert f(FAKE, 4096, 6, 256, FAKE, FAKE, FAKE, FAKE, None, None, need, None) == ERR_NULL
    assert f(FAKE, 4096, 6, 256, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 4, None) == ERR_SHAPE
    assert f(FAKE, 4096, 6, 256, FAKE, FAKE, FAKE, FAKE, None, ctypes.c_void_p((1 << 20) + 2), need,
             None) == ERR_SHAPE


def test_encode_validation(lib):
    f = lib.mxfp4_encode
    assert f(0, None, FAKE, None, 8, 512, 256, FAKE_ALIGNED, None, None) == ERR_NULL
    assert f(0, FAKE, FAKE, None, 8, 512, 96, FAKE_ALIGNED, None, None) == ERR_SHAPE
    assert f(2, FAKE, FAKE, None, 8, 512, 256, FAKE_ALIGNED, None, None) == ERR_FORMAT
    assert f(1, FAKE, FAKE, None, 8, 512, 256, FAKE_ALIGNED, None, None) == ERR_NULL      # NVFP4 needs tensor scales
    assert f(0, FAKE, FAKE, FAKE, 8, 512, 256, FAKE_ALIGNED, None, None) == ERR_FORMAT    # MXFP4 takes none
    assert f(0, FAKE, FAKE, None, 8, 512, 256, ctypes.c_void_p((1 << 30) + 16), None, None) == ERR_SHAPE


def test_gmm_validation(lib):
    f = lib.moe_gmm_ex
    args = lambda **kw: [kw.get("packed", FAKE_ALIGNED), kw.get("fmt", 0), kw.get("E", 8),
                         kw.get("N", 512), kw.get("K", 256), kw.get("x", FAKE_ALIGNED),
                         kw.get("x_rows", 128), None,
                         kw.get("off", FAKE), kw.get("M", 128), kw.get("y", FAKE),
                         kw.get("dt", 0), kw.get("kernel", 0), None]
    assert f(*args(packed=None)) == ERR_NULL
    assert f(*args(y=None)) == ERR_NULL
    assert f(*args(off=None)) == ERR_NULL
    assert f(*args(K=200)) == ERR_SHAPE
    assert f(*args(N=500)) == ERR_SHAPE
    assert f(*args(E=0)) == ERR_SHAPE
    assert f(*args(E=1025)) == ERR_SHAPE            # the tile scan covers 1024 experts
    assert f(*args(M=0)) == ERR_SHAPE
    assert f(*args(M=(1 << 24) + 1)) == ERR_SHAPE
    assert f(*args(fmt=3)) == ERR_FORMAT
    assert f(*args(dt=2)) == ERR_FORMAT
    assert f(*args(kernel=3)) == ERR_FORMAT
    assert f(*args(packed=ctypes.c_void_p((1 << 30) + 128))) == ERR_SHAPE
    assert f(*args(x_rows=0)) == ERR_SHAPE
    assert f(*args(x_rows=127)) == ERR_SHAPE        # band input needs x_rows >= M
    assert f(*args(x_rows=1 << 22, K=512)) == ERR_SHAPE   # 4 GiB of activations
    # every byte offset stays below the lane offset that reads zeros (2^31 - 64 KiB)
    assert f(*args(x_rows=0x7FFF0000 // 8192 + 1, K=4096)) == ERR_SHAPE
    assert f(*args(E=1, N=64, K=0x7FFF0000 // 8 + 128)) == ERR_SHAPE     # a wave's code range
    assert lib.moe_gmm(None, 0, 8, 512, 256, FAKE, 128, None, FAKE, 128, FAKE, 0, None) == ERR_NULL


def test_gmm_grid_within_dispatch_limit(lib):
    # one expert of 2^30 columns: an accepted weight shape whose grids pass
    # the 2^32 - 1 work-items of a dispatch (16,777,215 workgroups of 256)
    ex, act, g = lib.moe_gmm_ex, lib.moe_gmm_act, lib.moe_gmm_w4a4
    N = 1 << 30
    assert lib.moe_packed_weight_bytes(0, 1, N, 128) > 0
    # streaming: 8 tile slots x 2^22 column groups of 256
    assert ex(FAKE_ALIGNED, 0, 1, N, 128, FAKE_ALIGNED, 1, None, FAKE, 1, FAKE, 0, 1, None) == ERR_SHAPE
    # with the fused activation: 8 x 2^22 groups of 128 gated columns
    assert act(FAKE_ALIGNED, 0, 1, N, 128, FAKE_ALIGNED, 1, None, FAKE, 1, FAKE, 0, 1, 1, None) == ERR_SHAPE
    # tiled: (ceil(M / 128) + 1) x 2^22 passes the limit from M = 385 rows
    assert ex(FAKE_ALIGNED, 0, 1, N, 128, FAKE_ALIGNED, 385, None, FAKE, 385, FAKE, 0, 2, None) == ERR_SHAPE
    assert g(FAKE_ALIGNED, 0, 1, N, 128, FAKE_ALIGNED, FAKE, 385, None, FAKE, 385, FAKE, 0, 0, None,
             None) == ERR_SHAPE


def test_bf16_arm_validation(lib):
    assert lib.moe_packed_weight_bytes(2, 8, 512, 256) == 8 * 512 * 256 * 2
    assert lib.mxfp4_encode(2, FAKE, FAKE, None, 8, 512, 256, FAKE_ALIGNED, None, None) == ERR_FORMAT
    assert lib.moe_bf16_encode(None, 8, 512, 256, FAKE_ALIGNED, None) == ERR_NULL
    assert lib.moe_bf16_encode(FAKE, 8, 512, 200, FAKE_ALIGNED, None) == ERR_SHAPE
    assert lib.moe_bf16_encode(FAKE, 8, 512, 256, ctypes.c_void_p((1 << 30) + 16), None) == ERR_SHAPE
    # a wave's code range (four 4 KiB-per-chunk subtiles of bf16 weights,
    # eight 1 KiB-per-chunk subtiles of MXFP4 / NVFP4) stays below the lane
    # offset the kernels use to read zeros, 2^31 - 64 KiB
    assert lib.moe_packed_weight_bytes(2, 1, 64, 0x7FFF0000 // 16384 * 128) > 0
    assert lib.moe_packed_weight_bytes(2, 1, 64, 0x7FFF0000 // 16384 * 128 + 128) == 0
    assert lib.moe_packed_weight_bytes(2, 1, 64, 1 << 25) == 0
    assert lib.moe_packed_weight_bytes(0, 1, 128, 0x7FFF0000 // 8192 * 128) > 0
    assert lib.moe_packed_weight_bytes(0, 1, 128, 0x7FFF0000 // 8192 * 128 + 128) == 0
    assert lib.moe_packed_weight_bytes(0, 1, 128, 1 << 26) == 0
    assert lib.moe_bf16_encode(FAKE, 1, 64, 1 << 25, FAKE_ALIGNED, None) == ERR_SHAPE
    ex = lib.moe_gmm_ex
    assert ex(FAKE_ALIGNED, 2, 1, 64, 1 << 25, FAKE_ALIGNED, 1, None, FAKE, 1, FAKE, 0, 2, None) == ERR_SHAPE
    act = lib.moe_gmm_act
    assert act(FAKE_ALIGNED, 2, 8, 512, 256, FAKE_ALIGNED, 128, None, FAKE, 128, FAKE, 0, 1, 0, None) == 4


def test_w4a4_validation(lib):
    q = lib.moe_mxfp4_quantize
    assert q(None, 4, 64, FAKE_ALIGNED, FAKE, None) == ERR_NULL
    assert q(FAKE_ALIGNED, 4, 48, FAKE_ALIGNED, FAKE, None) == ERR_SHAPE
    assert q(FAKE_ALIGNED, 0, 64, FAKE_ALIGNED, FAKE, None) == ERR_SHAPE
    assert q(ctypes.c_void_p((1 << 30) + 2), 4, 64, FAKE_ALIGNED, FAKE, None) == ERR_SHAPE
    g = lib.moe_gmm_w4a4
    args = lambda **kw: [kw.get("packed", FAKE_ALIGNED), kw.get("fmt", 0), kw.get("E", 8), kw.get("N", 512),
                         kw.get("K", 256),
                         kw.get("qc", FAKE_ALIGNED), FAKE, kw.get("rows", 128), None, FAKE, 128,
                         FAKE, kw.get("dt", 0), kw.get("act", 0), None, None]
    assert g(*args(packed=None)) == ERR_NULL
    assert g(*args(qc=None)) == ERR_NULL
    assert g(*args(K=200)) == ERR_SHAPE
    assert g(*args(rows=100)) == ERR_SHAPE          # band input needs M rows
    assert g(*args(act=3)) == ERR_FORMAT
    assert g(*args(dt=5)) == ERR_FORMAT
    assert g(*args(N=192, act=1)) == ERR_SHAPE
    assert g(*args(qc=ctypes.c_void_p((1 << 30) + 8))) == ERR_SHAPE
    assert g(*args(fmt=2)) == 4                     # bf16 weights: unsupported
    assert g(*args(fmt=5)) == ERR_FORMAT
    assert g(*args(fmt=1, K=200)) == ERR_SHAPE
    assert g(*args(E=1025)) == ERR_SHAPE
    assert g(*args(rows=0x7FFF0000 // 2048 + 1, K=4096)) == ERR_SHAPE   # codes past 2^31 - 64 KiB


def test_gmm_act_validation(lib):
    f = lib.moe_gmm_act
    args = lambda **kw: [kw.get("packed", FAKE_ALIGNED), 0, kw.get("E", 8), kw.get("N", 512),
                         kw.get("K", 256), FAKE_ALIGNED, 128, None, FAKE, 128, FAKE, 0,
                         kw.get("act", 1), kw.get("kernel", 0), None]
    assert f(*args(act=2)) == ERR_FORMAT
    assert f(*args(act=-1)) == ERR_FORMAT
    assert f(*args(N=192)) == ERR_SHAPE                 # halves must be 64-column multiples
    assert f(*args(packed=None)) == ERR_NULL
    assert f(*args(N=1 << 17, K=1 << 17, E=1)) == ERR_SHAPE   # code range past 32-bit offsets
    assert f(*args(N=4096, K=(0x7FFF0000 // (130 * 1024) + 1) * 128, E=1)) == ERR_SHAPE


def test_combine_validation(lib):
    f = lib.moe_combine
    assert f(FAKE_ALIGNED, 0, FAKE, FAKE, 4, 2, 6, FAKE_ALIGNED, 0, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, 0, FAKE, FAKE, 4, 0, 8, FAKE_ALIGNED, 0, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, 5, FAKE, FAKE, 4, 2, 8, FAKE_ALIGNED, 0, None) == ERR_FORMAT
    assert f(None, 0, FAKE, FAKE, 4, 2, 8, FAKE_ALIGNED, 0, None) == ERR_NULL


def test_cast_and_debug_decode_validation(lib):
    assert lib.moe_mxfp4_to_nvfp4(None, 1, 16, 64, FAKE, FAKE, None, None) == ERR_NULL
    assert lib.moe_mxfp4_to_nvfp4(FAKE, 1, 16, 48, FAKE, FAKE, None, None) == ERR_SHAPE
    assert lib.moe_debug_decode(FAKE_ALIGNED, 0, 1, 64, 100, FAKE, None) == ERR_SHAPE
    assert lib.moe_debug_decode(None, 0, 1, 64, 128, FAKE, None) == ERR_NULL


def test_calib_validation(lib):
    f = lib.moe_calib_mfma_bf16
    assert f(None, FAKE_ALIGNED, 1, 1, FAKE_ALIGNED, None) == ERR_NULL
    assert f(FAKE_ALIGNED, FAKE_ALIGNED, 1, 1, None, None) == ERR_NULL
    assert f(FAKE_ALIGNED, FAKE_ALIGNED, 0, 1, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, FAKE_ALIGNED, 65536, 1, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, FAKE_ALIGNED, 1, 0, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, FAKE_ALIGNED, 1, (1 << 20) + 1, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(ctypes.c_void_p((1 << 30) + 8), FAKE_ALIGNED, 1, 1, FAKE_ALIGNED, None) == ERR_SHAPE


def test_calib_parts_validation(lib):
    f = lib.moe_calib_mfma_parts
    A = FAKE_ALIGNED
    ok = dict(parts=0, rows16=8, a=A, b=A, codes=A, codes_bytes=1 << 20, x=A, x_bytes=8192, scale=1.0,
              blocks=4, chunks=2, out=A)

    def call(**kw):
        d = dict(ok, **kw)
        return f(d["parts"], d["rows16"], d["a"], d["b"], d["codes"], d["codes_bytes"], d["x"], d["x_bytes"],
                 ctypes.c_float(d["scale"]), d["blocks"], d["chunks"], d["out"], None)

    for name in ("a", "b", "codes", "x", "out"):
        assert call(**{name: None}) == ERR_NULL
    for parts in (3, 5, 6, 64, -1, 1 | 2 | 4 | 8):
        assert call(parts=parts) == ERR_SHAPE
    assert call(rows16=7) == ERR_SHAPE
    assert call(blocks=0) == ERR_SHAPE
    assert call(blocks=65536) == ERR_SHAPE
    assert call(chunks=0) == ERR_SHAPE
    assert call(chunks=3) == ERR_SHAPE
    assert call(chunks=(1 << 24) + 2) == ERR_SHAPE
    assert call(codes_bytes=4 * 4096 - 1) == ERR_SHAPE        # a wave region under 4 KiB
    assert call(blocks=1, codes_bytes=4 << 31) == ERR_SHAPE   # a wave region of 2 GiB
    assert call(x_bytes=4096) == ERR_SHAPE
    assert call(x_bytes=8192 + 512) == ERR_SHAPE
    assert call(x_bytes=1 << 31) == ERR_SHAPE
    assert call(a=ctypes.c_void_p((1 << 30) + 8)) == ERR_SHAPE
    assert call(x=ctypes.c_void_p((1 << 30) + 8)) == ERR_SHAPE


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(moe.MoeGmmError):
        moe.route_sort(torch.zeros((4, 2), dtype=torch.int32), 8)


def test_route_sort_noalloc_validation(lib):
    f = lib.moe_route_sort_noalloc
    assert f(None, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_NULL
    assert f(FAKE, 4, 2, 8, FAKE, None, FAKE, FAKE, None, None) == ERR_NULL
    assert f(FAKE, 0, 2, 8, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert f(FAKE, 4, 2, 1025, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert f(FAKE, 1 << 22, 8, 8, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE


def test_calib_hbm_read_validation(lib):
    f = lib.moe_calib_hbm_read
    assert f(None, 1 << 20, 64, FAKE_ALIGNED, None) == ERR_NULL
    assert f(FAKE_ALIGNED, 1 << 20, 64, None, None) == ERR_NULL
    assert f(FAKE_ALIGNED, 8, 64, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, (1 << 20) + 4, 64, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, 1 << 20, 0, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(FAKE_ALIGNED, 1 << 20, 65536, FAKE_ALIGNED, None) == ERR_SHAPE
    assert f(ctypes.c_void_p((1 << 30) + 8), 1 << 20, 64, FAKE_ALIGNED, None) == ERR_SHAPE
