"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Integer and index results are compared bit for bit; decoded weights are
compared exactly (every decoded value is representable in bf16); f32 matmul
outputs to max|gpu - oracle| / max|oracle| <= 1e-5; bf16 outputs to one bf16
ulp of the oracle.  Full-size workloads are checked on sampled outputs, which
the oracle computes one dot product at a time, plus properties that hold at
any size (kernel configurations agree bitwise, NVFP4 built by the lossless
cast equals MXFP4 bitwise, repeated runs are bitwise identical).
"""

import numpy as np
import pytest
import torch

import moe_grouped_gemm_route_amd as moe
import oracle
from moe_grouped_gemm_route_amd.synth import (make_config, make_ep_share, make_problem, make_tokens_problem,
                                              random_bf16_bits)
from gpu_util import (DEV, REL_TOL, bf16_bits_to_f64, bf16_ulp, oracle_gmm_bands, rel_err, run_gpu,
                      to_dev, weights_for)

pytestmark = pytest.mark.gpu

KERNELS = [moe.GMM_STREAM, moe.GMM_TILED]


def _route_check(ids, E, ws=None):
    ref = oracle.route_sort(ids, E)
    got = moe.route_sort(to_dev(ids), E, ws=ws)
    torch.cuda.synchronize()
    for key in ("group_offsets", "sorted_token", "sorted_pair", "pair_row"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    assert int(got["err_count"].item()) == ref["err_count"]


# ---------------------------------------------------------------- decode ---

def test_debug_decode_all_codes_mxfp4():
    E, N, K = 2, 64, 512
    rng = np.random.default_rng(100)
    codes = np.tile(np.arange(256, dtype=np.uint8), E * N * K // 2 // 256).reshape(E, N, K // 2)
    codes = rng.permuted(codes, axis=2)
    scales = rng.integers(2, 253, size=(E, N, K // 32)).astype(np.uint8)
    scales[0, 0, :4] = [2, 127, 252, 126]
    packed = moe.mxfp4_encode(to_dev(codes), to_dev(scales), None, moe.MXFP4)
    w = moe.debug_decode(packed, moe.MXFP4, E, N, K).cpu().numpy()
    ref = oracle.decode_mxfp4(codes, scales)
    got = bf16_bits_to_f64(w)
    assert np.array_equal(got, ref)


def test_debug_decode_nvfp4_general_e4m3():
    E, N, K = 2, 64, 256
    rng = np.random.default_rng(101)
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    bs = rng.integers(0, 0x7F, size=(E, N, K // 16)).astype(np.uint8)   # every finite positive E4M3
    bs[0, 0, :] = np.arange(16)                                          # subnormals and zero
    ts = np.array([1.0, 1.0], dtype=np.float32)
    packed = moe.mxfp4_encode(to_dev(codes), to_dev(bs), to_dev(ts), moe.NVFP4)
    w = moe.debug_decode(packed, moe.NVFP4, E, N, K).cpu().numpy()
    ref = oracle.decode_nvfp4(codes, bs, ts)
    assert np.array_equal(bf16_bits_to_f64(w), ref)


def test_nvfp4_cast_gpu_matches_oracle():
    p = make_problem(T=8, k=2, E=4, K=512, N=64, seed=102, exp_range=(-12, 5))
    bs_ref, ts_ref = oracle.mxfp4_to_nvfp4(p["scales"])
    bs, ts, err = moe.mxfp4_to_nvfp4(to_dev(p["scales"]))
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(ts.cpu().numpy(), ts_ref)
    assert err.item() == 0
    bad = p["scales"].copy()
    bad[1, 3, 2] = bad[1].max() - 18                  # below k_max - 17: not castable
    _, _, err = moe.mxfp4_to_nvfp4(to_dev(bad))
    assert err.item() == 1


def test_nvfp4_cast_experts_with_tiny_kmax():
    # largest E8M0 byte 5 and an all-zero expert: subnormal tensor scales,
    # bit for bit as the oracle's cast
    rng = np.random.default_rng(103)
    sc = rng.integers(0, 6, size=(3, 16, 8)).astype(np.uint8)
    sc[0, 0, 0] = 5
    sc[1] = 0
    sc[2] = rng.integers(120, 138, size=(16, 8)).astype(np.uint8)
    bs_ref, ts_ref = oracle.mxfp4_to_nvfp4(sc)
    bs, ts, err = moe.mxfp4_to_nvfp4(to_dev(sc))
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), ts_ref.view(np.uint32))
    assert err.item() == 0


def test_encode_counts_scales_outside_exact_domain():
    # E8M0 bytes 0, 1, 253, 254 and 255 planted in an MXFP4 tensor, E4M3 NaN
    # bytes and a non-finite tensor scale in an NVFP4 one: each is counted;
    # in-domain tensors count zero
    rng = np.random.default_rng(104)
    E, N, K = 2, 64, 256
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(2, 253, size=(E, N, K // 32)).astype(np.uint8)
    err = torch.full((1,), 77, dtype=torch.int32, device=DEV)
    moe.mxfp4_encode(to_dev(codes), to_dev(scales), None, moe.MXFP4, err_count=err)
    assert err.item() == 0
    bad = scales.copy()
    bad[0, 0, 0], bad[0, 5, 3], bad[1, 63, 7], bad[1, 9, 2], bad[0, 40, 6] = 0, 1, 253, 254, 255
    moe.mxfp4_encode(to_dev(codes), to_dev(bad), None, moe.MXFP4, err_count=err)
    assert err.item() == 5
    bs = rng.integers(0, 0x7F, size=(E, N, K // 16)).astype(np.uint8)
    ts = np.array([1.0, 0.25], dtype=np.float32)
    moe.mxfp4_encode(to_dev(codes), to_dev(bs), to_dev(ts), moe.NVFP4, err_count=err)
    assert err.item() == 0
    bs[1, 2, 3], bs[0, 7, 15] = 0x7F, 0xFF
    ts[1] = np.inf
    moe.mxfp4_encode(to_dev(codes), to_dev(bs), to_dev(ts), moe.NVFP4, err_count=err)
    assert err.item() == 3


# ------------------------------------------------------------ route sort ---

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_route_sort_configs(cfg):
    from moe_grouped_gemm_route_amd.synth import CONFIGS
    c = CONFIGS[cfg]
    p = make_problem(T=c["T"], k=c["k"], E=c["E"], K=32, N=1, seed=cfg, routing=c["routing"],
                     empty_experts=c.get("empty_experts", ()))
    _route_check(p["topk_ids"], c["E"])


def test_route_sort_edge_cases():
    _route_check(np.zeros((1, 1), dtype=np.int32), 1)                       # single pair, E = 1
    _route_check(np.full((300, 4), 5, dtype=np.int32), 8)                   # all on one expert
    rng = np.random.default_rng(7)
    ids = rng.integers(-3, 260, size=(777, 6)).astype(np.int32)            # invalid ids dropped
    _route_check(ids, 256)
    _route_check(rng.integers(0, 1024, size=(3000, 8)).astype(np.int32), 1024)
    _route_check(rng.integers(0, 3, size=(5000, 1)).astype(np.int32), 3)


def test_route_sort_unit_boundaries():
    # around the one-workgroup limit (4,096 pairs) and the segments of the
    # two-kernel path: a ragged last segment of one pair, segments of 4,608
    # pairs (262,145 pairs: sub-segments of 576 pairs, two id batches per
    # wave), 1,024 experts (two per scan thread), more than 32 segments (two
    # batches of count-table rows), one expert, and dropped ids spread over
    # the segments
    rng = np.random.default_rng(9)
    for M, E in [(4096, 256), (4097, 256), (4097, 1), (8191, 7), (24576, 256), (262145, 1024),
                 (262145, 600)]:
        ids = rng.integers(0, E, size=(M, 1), dtype=np.int32)
        _route_check(ids, E)
        bad = ids.copy()
        bad[rng.random(bad.shape) < 0.1] = E + 3
        bad[rng.random(bad.shape) < 0.05] = -1
        _route_check(bad, E)
    _route_check(np.full((6000, 4), 9, dtype=np.int32), 16)                # one band
    _route_check(np.full((6000, 4), 99, dtype=np.int32), 16)               # every pair dropped


def test_route_sort_workspace_needs_no_clearing():
    # the count table is written in full before it is read: a workspace full
    # of stale values, passed explicitly and reused, gives the same result
    rng = np.random.default_rng(10)
    ids = rng.integers(0, 256, size=(4096, 6), dtype=np.int32)
    need = moe.route_sort_workspace_bytes(4096, 6, 256)
    assert need == 24 * 256 * 4
    ws = torch.randint(-2 ** 31, 2 ** 31 - 1, (need // 4,), dtype=torch.int32, device=DEV)
    _route_check(ids, 256, ws=ws)
    _route_check(rng.integers(0, 256, size=(1000, 6), dtype=np.int32), 256, ws=ws)
    with pytest.raises(moe.MoeGmmError):
        moe.route_sort(to_dev(ids), 256, ws=ws[:-1])


def test_route_sort_max_pairs():
    # the largest pair count the call accepts (T * k = 2^24): E = 1024 with
    # uniform ids, and E = 256 with a skewed id mix (a quarter of the pairs on
    # expert 0), against the oracle's stable sort, bit for bit
    rng = np.random.default_rng(8)
    ids = rng.integers(0, 1024, size=(1 << 21, 8), dtype=np.int32)
    _route_check(ids, 1024)
    ids = rng.integers(0, 256, size=(1 << 22, 4), dtype=np.int32)
    ids[rng.random(ids.shape) < 0.25] = 0
    _route_check(ids, 256)


# ------------------------------------------------------------------- gmm ---

SMALL = [
    # T, k, E, K, N, routing, band input, empty experts
    dict(T=64, k=2, E=8, K=256, N=512, routing="uniform", empty=(7,)),
    dict(T=200, k=4, E=16, K=1024, N=320, routing="zipf", empty=(3,)),
    dict(T=37, k=3, E=5, K=384, N=192, routing="uniform", x_rows=111),
    dict(T=300, k=1, E=1, K=128, N=64, routing="uniform"),
    dict(T=1, k=1, E=4, K=128, N=256, routing="uniform"),
    # mean band >= 4 rows with N a multiple of 128: the stream kernel's
    # eight-subtile waves, with the last workgroup's waves partly past N
    dict(T=160, k=4, E=12, K=512, N=384, routing="zipf", empty=(5,)),
    dict(T=96, k=2, E=16, K=256, N=640, routing="uniform"),
]


def _small(i):
    c = SMALL[i]
    return make_problem(T=c["T"], k=c["k"], E=c["E"], K=c["K"], N=c["N"], seed=200 + i,
                        routing=c["routing"], empty_experts=c.get("empty", ()),
                        x_rows=c.get("x_rows"), exp_range=(-6, -2))


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_gmm_small_full_oracle(case, fmt, kernel):
    p = _small(case)
    w, packed = weights_for(p, fmt)
    r, y = run_gpu(p, packed, fmt, kernel=kernel)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.gmm(p["x"], ref_r["sorted_token"] if p["gather"] else None,
                     ref_r["group_offsets"], w)
    got = y.cpu().numpy()
    assert np.array_equal(r["group_offsets"].cpu().numpy(), ref_r["group_offsets"])
    assert rel_err(got, ref) <= REL_TOL


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_gmm_kernels_agree_bitwise_and_bf16_output(case):
    p = _small(case)
    w, packed = weights_for(p, "mxfp4")
    _, ys = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_STREAM)
    _, yt = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED)
    r, yb = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED, out_dtype=moe.BF16)
    _, yb2 = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_STREAM, out_dtype=moe.BF16)
    assert torch.equal(ys, yt)
    assert torch.equal(yb.view(torch.int16), yb2.view(torch.int16))
    assert torch.equal(yb, ys.to(torch.bfloat16))            # bf16 = RNE of the f32 sum
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.gmm(p["x"], ref_r["sorted_token"] if p["gather"] else None,
                     ref_r["group_offsets"], w)
    got = yb.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref))


# Band sizes that reach every specialised walk: the stream kernel's one- and
# two-subtile tiles (1..16, 17..32 rows, several 32-row tiles) and the tiled
# kernel's 1..8 valid 16-row subtiles, whole and ragged 128-row tiles, and an
# empty expert.  N = 320 leaves three of the four waves of the last tiled
# column block without columns.
BANDS = [1, 15, 16, 17, 31, 32, 33, 48, 0, 64, 80, 96, 112, 127, 128, 129, 200, 5]


def _banded_problem(seed, fmt_scales=(-6, -2), N=320):
    E = len(BANDS)
    p = make_problem(T=sum(BANDS), k=1, E=E, K=256, N=N, seed=seed, exp_range=fmt_scales)
    rng = np.random.default_rng(seed + 1)
    ids = np.repeat(np.arange(E, dtype=np.int32), BANDS)
    rng.shuffle(ids)
    p["topk_ids"] = ids.reshape(-1, 1)
    return p


@pytest.mark.parametrize("fmt,N", [("mxfp4", 320), ("nvfp4", 320), ("mxfp4", 384), ("mxfp4", 4096)])
def test_gmm_every_band_shape(fmt, N):
    # N = 384 and 4096 send the MXFP4 streaming choice through the split
    # kernel (the mean band is over 4 rows): its bands of more than 64 rows as
    # LDS-tiled units, 65 .. 200 rows, and the others as eight-subtile
    # streaming waves; at N = 384 the grid is one round of workgroups and the
    # tiled units cover 64 rows, at N = 4096 they cover 128; f32 and bf16
    # output
    p = _banded_problem(260, N=N)
    w, packed = weights_for(p, fmt)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    assert np.array_equal(np.diff(ref_r["group_offsets"]), BANDS)
    ref = oracle.gmm(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w)
    ys = []
    for kernel in KERNELS:
        _, y = run_gpu(p, packed, fmt, kernel=kernel)
        assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
        ys.append(y)
        _, yb = run_gpu(p, packed, fmt, kernel=kernel, out_dtype=moe.BF16)
        assert torch.equal(yb, y.to(torch.bfloat16))
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("kernel", KERNELS)
def test_gmm_nvfp4_general_e4m3_scales(kernel):
    # NVFP4 weights whose per-16 scales are arbitrary E4M3 values (not only
    # the powers of two the lossless cast produces), mixed per chunk
    p = make_problem(T=96, k=4, E=8, K=512, N=256, seed=250, routing="zipf")
    rng = np.random.default_rng(251)
    bs = rng.integers(0x20, 0x50, size=(8, 256, 32)).astype(np.uint8)
    bs[:, :, 8:16] &= 0xF8                        # some chunks hold only powers of two
    p["block_scales"] = bs
    p["tensor_scale"] = np.ldexp(1.0, rng.integers(-4, 4, size=8)).astype(np.float32)
    w, packed = weights_for(p, "nvfp4")
    _, y = run_gpu(p, packed, "nvfp4", kernel=kernel)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.gmm(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w)
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("act", [moe.ACT_NONE, moe.ACT_SILU_MUL])
def test_gmm_nvfp4_scale_kinds_mixed_across_waves(act, kernel):
    # per expert: only powers of two (the cast's scales); general E4M3 scales
    # in one 16-column strip only (one wave of a workgroup decodes them, the
    # others do not); a few zero scales among powers of two
    E, N = 9, 384
    p = make_problem(T=96, k=4, E=E, K=512, N=N, seed=252, routing="zipf")
    rng = np.random.default_rng(253)
    bs = (rng.integers(1, 16, size=(E, N, 32)) << 3).astype(np.uint8)   # 2^-6 .. 2^8
    for e in range(E):
        if e % 3 == 1:
            c0 = 16 * (e % (N // 16))
            bs[e, c0:c0 + 16] = rng.integers(0x20, 0x50, size=(16, 32))
        elif e % 3 == 2:
            bs[e, rng.integers(0, N, 5), rng.integers(0, 32, 5)] = 0
    p["block_scales"] = bs
    p["tensor_scale"] = np.ldexp(1.0, rng.integers(-4, 4, size=E)).astype(np.float32)
    w, packed = weights_for(p, "nvfp4")
    _, y = run_gpu(p, packed, "nvfp4", kernel=kernel, act=act)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.gmm(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w)
    if act == moe.ACT_SILU_MUL:
        ref = oracle.silu_mul(ref)
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL


# ---------------------------------------- fused gate/up activation ---

def _act_problems():
    banded = _banded_problem(270)
    banded["N"] = 384
    banded["codes"] = np.ascontiguousarray(
        np.random.default_rng(271).integers(0, 256, size=(banded["E"], 384, 128), dtype=np.uint8))
    banded["scales"] = (np.random.default_rng(272).integers(-6, -1, size=(banded["E"], 384, 8))
                        + 127).astype(np.uint8)
    gathered = make_problem(T=96, k=4, E=8, K=512, N=512, seed=273, routing="zipf")
    return [banded, gathered]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("case", [0, 1])
def test_gmm_silu_mul_full_oracle(case, fmt, kernel):
    p = _act_problems()[case]
    w, packed = weights_for(p, fmt)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.silu_mul(oracle.gmm(p["x"], ref_r["sorted_token"] if p["gather"] else None,
                                     ref_r["group_offsets"], w))
    _, y = run_gpu(p, packed, fmt, kernel=kernel, act=moe.ACT_SILU_MUL)
    assert tuple(y.shape) == (p["T"] * p["k"], p["N"] // 2)
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
    _, yb = run_gpu(p, packed, fmt, kernel=kernel, act=moe.ACT_SILU_MUL, out_dtype=moe.BF16)
    assert torch.equal(yb, y.to(torch.bfloat16))              # bf16 = RNE of the f32 value
    got = yb.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref))


def test_gmm_silu_mul_kernels_agree_bitwise():
    for p in _act_problems():
        _, packed = weights_for(p, "mxfp4")
        _, ys = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_STREAM, act=moe.ACT_SILU_MUL)
        _, yt = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED, act=moe.ACT_SILU_MUL)
        assert torch.equal(ys, yt)


def test_layer_chain_small():
    # route -> w13 with the fused activation (bf16) -> w2 on the band-ordered
    # activation (f32) -> combine, each stage against the oracle on the
    # previous GPU stage's output
    p = make_problem(T=80, k=3, E=8, K=256, N=512, seed=280, routing="zipf")
    H, D = p["N"] // 2, p["K"]
    rng = np.random.default_rng(281)
    w2c = rng.integers(0, 256, size=(p["E"], D, H // 2), dtype=np.uint8)
    w2s = (rng.integers(-6, -1, size=(p["E"], D, H // 32)) + 127).astype(np.uint8)
    w13, p13 = weights_for(p, "mxfp4")
    pk2 = moe.mxfp4_encode(to_dev(w2c), to_dev(w2s), None, moe.MXFP4)
    r, h = run_gpu(p, p13, "mxfp4", out_dtype=moe.BF16, act=moe.ACT_SILU_MUL)
    M = p["T"] * p["k"]
    y2 = moe.moe_gmm(pk2, moe.MXFP4, p["E"], D, H, h, r["group_offsets"], M)
    out = moe.moe_combine(y2, to_dev(p["topk_weights"]), r["pair_row"])
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref_h = oracle.silu_mul(oracle.gmm(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w13))
    got_h = h.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_h - ref_h) <= bf16_ulp(ref_h))
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_y2 = oracle.gmm(h_bits, None, ref_r["group_offsets"], {"fmt": "mxfp4", "codes": w2c, "scales": w2s})
    assert rel_err(y2.cpu().numpy(), ref_y2) <= REL_TOL
    ref_out = oracle.combine(y2.cpu().numpy(), p["topk_weights"], ref_r["pair_row"])
    assert rel_err(out.cpu().numpy(), ref_out) <= REL_TOL


# ------------------------------------------------ bf16 comparison arm ---

def _bf16_weights(E, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((E, N, K), dtype=np.float32) * 0.05
    return (x.view(np.uint32) >> 16).astype(np.uint16)         # truncation: any bf16 will do


def test_bf16_encode_round_trip():
    wb = _bf16_weights(3, 192, 384, 290)
    packed = moe.bf16_encode(to_dev(wb))
    back = moe.debug_decode(packed, moe.W_BF16, 3, 192, 384)
    assert np.array_equal(back.cpu().numpy().view(np.uint16), wb)


@pytest.mark.parametrize("case", [0, 1, 2, 3])
def test_gmm_bf16_weights_full_oracle(case):
    # both kernels on bf16 weights: every band shape (N = 320), a Zipf
    # problem, band input, and N = 384 with a 512-deep K
    p = [_banded_problem(291), _small(1), _small(2), _small(5)][case]
    wb = _bf16_weights(p["E"], p["N"], p["K"], 292 + case)
    packed = moe.bf16_encode(to_dev(wb))
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.gmm(p["x"], ref_r["sorted_token"] if p["gather"] else None, ref_r["group_offsets"],
                     {"fmt": "bf16", "weights": wb})
    _, ys = run_gpu(p, packed, "bf16", kernel=moe.GMM_STREAM)
    _, yt = run_gpu(p, packed, "bf16", kernel=moe.GMM_TILED)
    assert rel_err(ys.cpu().numpy(), ref) <= REL_TOL
    assert torch.equal(ys, yt)
    _, yb = run_gpu(p, packed, "bf16", kernel=moe.GMM_TILED, out_dtype=moe.BF16)
    assert torch.equal(yb, ys.to(torch.bfloat16))


@pytest.mark.parametrize("kernel", KERNELS)
def test_gmm_bf16_of_decoded_mxfp4_is_bitwise_mxfp4(kernel):
    # the bf16 arm on the decoded MXFP4 weights issues the same MFMAs on the
    # same operands: the two outputs are equal bit for bit
    p = _banded_problem(295)
    _, packed = weights_for(p, "mxfp4")
    dec = moe.debug_decode(packed, moe.MXFP4, p["E"], p["N"], p["K"])
    pb = moe.bf16_encode(dec)
    _, y4 = run_gpu(p, packed, "mxfp4", kernel=kernel)
    _, y16 = run_gpu(p, pb, "bf16", kernel=kernel)
    assert torch.equal(y4, y16)


# --------------------------------------------------------------- W4A4 ---

def _special_rows():
    # blocks that exercise every rounding tie, saturation, zero and -0
    # blocks, bf16 subnormals and the largest finite magnitudes
    from moe_grouped_gemm_route_amd.synth import f32_to_bf16_bits
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 0.3, -0.25, -5.0, 4.0, 0.0]
    rows = np.zeros((6, 64), dtype=np.float32)
    rows[0, :len(ties)] = ties
    rows[1, :len(ties)] = np.array(ties) * 2.0 ** -20
    rows[2, 1] = -0.0
    rows[2, 33] = 3.0e38
    rows[2, 34] = -1.0e38
    rows[3, :8] = np.float32(2.0 ** -130) * np.arange(1, 9)      # bf16 subnormals
    rows[4] = np.random.default_rng(300).standard_normal(64) * 1e-3
    rows[5, 32:] = -np.abs(np.random.default_rng(301).standard_normal(32))
    return f32_to_bf16_bits(rows)


@pytest.mark.parametrize("which", ["special", "random"])
def test_mxfp4_quantize_matches_oracle(which):
    if which == "special":
        bits = _special_rows()
    else:
        p = make_problem(T=300, k=1, E=1, K=512, N=64, seed=302)
        bits = p["x"]
    codes, scales = moe.mxfp4_quantize(to_dev(bits))
    rc, rs = oracle.quantize_mxfp4_rows(bits)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _w4a4_ref(p, w):
    qc, qs = oracle.quantize_mxfp4_rows(p["x"])
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    return oracle.gmm_w4a4(qc, qs, ref_r["sorted_token"] if p["gather"] else None,
                           ref_r["group_offsets"], w)


def _run_w4a4(p, packed, out_dtype=moe.F32, act=moe.ACT_NONE, fmt=moe.MXFP4, err_count=None):
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    qc, qs = moe.mxfp4_quantize(to_dev(p["x"]))
    return moe.moe_gmm_w4a4(packed, p["E"], p["N"], p["K"], qc, qs, r["group_offsets"], p["T"] * p["k"],
                            row_index=r["sorted_token"] if p["gather"] else None,
                            out_dtype=out_dtype, act=act, fmt=fmt, err_count=err_count)


@pytest.mark.parametrize("case", ["banded", "gathered", "band_input"])
def test_gmm_w4a4_full_oracle(case):
    if case == "banded":
        p = _banded_problem(310)
    elif case == "gathered":
        p = make_problem(T=96, k=4, E=8, K=512, N=512, seed=311, routing="zipf")
    else:
        p = _small(2)
    w, packed = weights_for(p, "mxfp4")
    ref = _w4a4_ref(p, w)
    y = _run_w4a4(p, packed)
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
    yb = _run_w4a4(p, packed, out_dtype=moe.BF16)
    assert torch.equal(yb, y.to(torch.bfloat16))
    if p["N"] % 128 == 0:
        ya = _run_w4a4(p, packed, act=moe.ACT_SILU_MUL)
        assert rel_err(ya.cpu().numpy(), oracle.silu_mul(ref)) <= REL_TOL


@pytest.mark.parametrize("E", [1000, 1024])
def test_gmm_most_experts(E):
    # the largest expert counts the tile scans cover (64 lanes of up to 16
    # experts; 1000 leaves the last lane partial), every expert's band
    # checked whole, through both W4A16 kernels and the W4A4 kernel
    p = make_problem(T=700, k=4, E=E, K=256, N=128, seed=330 + E, routing="zipf", empty_experts=(0, E - 1))
    w, packed = weights_for(p, "mxfp4")
    ref_r = oracle.route_sort(p["topk_ids"], E)
    ref = oracle.gmm(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w)
    ys = []
    for kernel in KERNELS:
        _, y = run_gpu(p, packed, "mxfp4", kernel=kernel)
        assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
        ys.append(y)
    assert torch.equal(ys[0], ys[1])
    yq = _run_w4a4(p, packed)
    assert rel_err(yq.cpu().numpy(), _w4a4_ref(p, w)) <= REL_TOL


def test_gmm_w4a4_thin_tiles_every_call():
    # many tiles of 1..16 rows make chunks short, so each chunk's wait meets
    # its loads still in flight; every call must give the oracle's output
    # and the same bits (a wait that trusted the order in which the 4-byte
    # direct-to-LDS scale loads land once gave one wrong 16-column subtile
    # in some tiles, differently from call to call)
    p = make_problem(T=700, k=4, E=1024, K=256, N=128, seed=1354, routing="zipf", empty_experts=(0, 1023))
    w, packed = weights_for(p, "mxfp4")
    ref = _w4a4_ref(p, w)
    ys = [_run_w4a4(p, packed) for _ in range(6)]
    for y in ys:
        assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
        assert torch.equal(y, ys[0])


@pytest.mark.parametrize("case", ["banded", "gathered", "band_input"])
def test_gmm_w4a4_nvfp4_weights(case):
    # NVFP4 weights from the lossless cast (both E4M3 halves of a block one
    # equal power of two) through the W4A4 kernel: the oracle's W4A4 matmul
    # on the NVFP4 decode within the bound, and bitwise the output of the
    # MXFP4 weights the cast came from, for every output form; no block is
    # counted
    if case == "banded":
        p = _banded_problem(312)
    elif case == "gathered":
        p = make_problem(T=96, k=4, E=8, K=512, N=512, seed=313, routing="zipf", exp_range=(-12, 3))
    else:
        p = _small(2)
    w_nv, packed_nv = weights_for(p, "nvfp4")
    _, packed_mx = weights_for(p, "mxfp4")
    err = torch.full((1,), -5, dtype=torch.int32, device=DEV)
    y = _run_w4a4(p, packed_nv, fmt=moe.NVFP4, err_count=err)
    assert err.item() == 0
    assert rel_err(y.cpu().numpy(), _w4a4_ref(p, w_nv)) <= REL_TOL
    assert torch.equal(y, _run_w4a4(p, packed_mx))
    for odt, act in ((moe.BF16, moe.ACT_NONE), (moe.F32, moe.ACT_SILU_MUL), (moe.BF16, moe.ACT_SILU_MUL)):
        if act == moe.ACT_SILU_MUL and p["N"] % 128:
            continue
        a = _run_w4a4(p, packed_nv, out_dtype=odt, act=act, fmt=moe.NVFP4)
        b = _run_w4a4(p, packed_mx, out_dtype=odt, act=act)
        assert torch.equal(a, b), (odt, act)


def test_gmm_w4a4_nvfp4_counts_blocks_that_do_not_qualify():
    # blocks whose two E4M3 scales differ or are not a power of two are
    # counted once each (every expert has one tile here), whatever the number
    # of waves that read them; blocks of experts with no rows are not used
    p = make_problem(T=24, k=2, E=6, K=256, N=128, seed=314, empty_experts=(5,))
    bs, ts = oracle.mxfp4_to_nvfp4(p["scales"])
    bad = bs.copy()
    planted = [(0, 3, 2, 0x39, 0x38), (1, 100, 5, 0x40, 0x48), (2, 17, 0, 0x00, 0x00), (4, 127, 7, 0x38, 0x30),
               (5, 0, 0, 0x39, 0x39)]          # the last in the empty expert 5
    for e, n, j, lo, hi in planted:
        bad[e, n, 2 * j], bad[e, n, 2 * j + 1] = lo, hi
    packed = moe.mxfp4_encode(to_dev(p["codes"]), to_dev(bad), to_dev(ts), moe.NVFP4)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    _run_w4a4(p, packed, fmt=moe.NVFP4, err_count=err)
    assert err.item() == 4
    _run_w4a4(p, packed, fmt=moe.NVFP4, err_count=err, act=moe.ACT_SILU_MUL, out_dtype=moe.BF16)
    assert err.item() == 4


@pytest.mark.slow
def test_config5_w4a4_nvfp4_equals_mxfp4_bitwise():
    # the NVFP4 workload (config 5, scales from the library's own cast)
    # through the W4A4 kernel equals the MXFP4 weights' output bit for bit
    p = make_config(5)
    _, packed_mx = weights_for(p, "mxfp4")
    bs, ts, err = moe.mxfp4_to_nvfp4(to_dev(p["scales"]))
    assert err.item() == 0
    packed_nv = moe.mxfp4_encode(to_dev(p["codes"]), bs, ts, moe.NVFP4)
    cnt = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    a = _run_w4a4(p, packed_nv, fmt=moe.NVFP4, err_count=cnt)
    b = _run_w4a4(p, packed_mx)
    assert cnt.item() == 0
    assert torch.equal(a, b)
    del packed_mx, packed_nv


def test_w4a4_layer_chain_small():
    # the W4A4 layer: route -> quantize x -> w13 with the fused activation
    # (bf16) -> quantize h -> w2 on the band-ordered activation (f32) ->
    # combine, each stage against the oracle on the previous GPU stage's output
    p = make_problem(T=80, k=3, E=8, K=256, N=512, seed=320, routing="zipf")
    H, D = p["N"] // 2, p["K"]
    rng = np.random.default_rng(321)
    w2c = rng.integers(0, 256, size=(p["E"], D, H // 2), dtype=np.uint8)
    w2s = (rng.integers(-6, -1, size=(p["E"], D, H // 32)) + 127).astype(np.uint8)
    w13, p13 = weights_for(p, "mxfp4")
    pk2 = moe.mxfp4_encode(to_dev(w2c), to_dev(w2s), None, moe.MXFP4)
    M = p["T"] * p["k"]
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    qc, qs = moe.mxfp4_quantize(to_dev(p["x"]))
    h = moe.moe_gmm_w4a4(p13, p["E"], p["N"], p["K"], qc, qs, r["group_offsets"], M,
                         row_index=r["sorted_token"], out_dtype=moe.BF16, act=moe.ACT_SILU_MUL)
    qhc, qhs = moe.mxfp4_quantize(h)
    y2 = moe.moe_gmm_w4a4(pk2, p["E"], D, H, qhc, qhs, r["group_offsets"], M)
    out = moe.moe_combine(y2, to_dev(p["topk_weights"]), r["pair_row"])
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref_h = oracle.silu_mul(_w4a4_ref(p, w13))
    got_h = h.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_h - ref_h) <= bf16_ulp(ref_h))
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_qc, ref_qs = oracle.quantize_mxfp4_rows(h_bits)
    assert np.array_equal(qhc.cpu().numpy(), ref_qc) and np.array_equal(qhs.cpu().numpy(), ref_qs)
    ref_y2 = oracle.gmm_w4a4(ref_qc, ref_qs, None, ref_r["group_offsets"],
                             {"fmt": "mxfp4", "codes": w2c, "scales": w2s})
    assert rel_err(y2.cpu().numpy(), ref_y2) <= REL_TOL
    ref_out = oracle.combine(y2.cpu().numpy(), p["topk_weights"], ref_r["pair_row"])
    assert rel_err(out.cpu().numpy(), ref_out) <= REL_TOL


def test_gmm_rows_past_bands_untouched_and_canary():
    # dropped pairs leave rows [group_offsets[E], M) unwritten; nothing is
    # written past the end of y
    p = make_problem(T=50, k=2, E=6, K=256, N=128, seed=300)
    p["topk_ids"][3, 1] = 99
    p["topk_ids"][10, 0] = -1
    w, packed = weights_for(p, "mxfp4")
    M, N = p["T"] * p["k"], p["N"]
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    for kernel in KERNELS:
        buf = torch.full((M + 4, N), 12345.0, dtype=torch.float32, device="cuda")
        moe.moe_gmm(packed, moe.MXFP4, p["E"], N, p["K"], to_dev(p["x"]), r["group_offsets"],
                    M, row_index=r["sorted_token"], kernel=kernel, out=buf[:M])
        got = buf.cpu().numpy()
        assert np.all(got[M - 2:] == 12345.0)
        ref_r = oracle.route_sort(p["topk_ids"], p["E"])
        ref = oracle.gmm(p["x"], np.maximum(ref_r["sorted_token"], 0), ref_r["group_offsets"], w)
        assert rel_err(got[:M - 2], ref[:M - 2]) <= REL_TOL


def test_all_pairs_dropped():
    # every id outside [0, E): every band is empty, so no tile runs and y is
    # left untouched by both kernels, the fused activation and W4A4; combine
    # of all-dropped pairs gives zeros
    p = make_problem(T=40, k=3, E=8, K=256, N=256, seed=330)
    p["topk_ids"][:] = p["E"]
    p["topk_ids"][::2, 1] = -5
    M, N, K, E = p["T"] * p["k"], p["N"], p["K"], p["E"]
    r = moe.route_sort(to_dev(p["topk_ids"]), E)
    assert int(r["err_count"].item()) == M
    assert torch.all(r["group_offsets"] == 0) and torch.all(r["pair_row"] == -1)
    _, packed = weights_for(p, "mxfp4")
    x = to_dev(p["x"])
    for kernel in KERNELS:
        for act in (moe.ACT_NONE, moe.ACT_SILU_MUL):
            cols = N // 2 if act == moe.ACT_SILU_MUL else N
            buf = torch.full((M, cols), 777.0, dtype=torch.float32, device="cuda")
            moe.moe_gmm(packed, moe.MXFP4, E, N, K, x, r["group_offsets"], M, row_index=r["sorted_token"],
                        kernel=kernel, act=act, out=buf)
            torch.cuda.synchronize()
            assert torch.all(buf == 777.0)
    qc, qs = moe.mxfp4_quantize(x)
    buf = torch.full((M, N), 777.0, dtype=torch.float32, device="cuda")
    moe.moe_gmm_w4a4(packed, E, N, K, qc, qs, r["group_offsets"], M, row_index=r["sorted_token"], out=buf)
    out = moe.moe_combine(buf, to_dev(p["topk_weights"]), r["pair_row"])
    torch.cuda.synchronize()
    assert torch.all(buf == 777.0)
    assert torch.all(out == 0.0)


def test_gmm_deterministic():
    p = _small(1)
    _, packed = weights_for(p, "mxfp4")
    for kernel in KERNELS:
        _, a = run_gpu(p, packed, "mxfp4", kernel=kernel)
        _, b = run_gpu(p, packed, "mxfp4", kernel=kernel)
        assert torch.equal(a, b)


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 3, 17, 64, 300, 1024]))
        k = min(int(rng.integers(1, 9)), E)          # top-k picks distinct experts
        T = int(rng.integers(1, max(2, 3000 // k)))
        out.append(dict(T=T, k=k, E=E, K=int(rng.choice([128, 256, 384, 640])),
                        N=int(rng.choice([64, 128, 192, 320, 512])),
                        routing=str(rng.choice(["uniform", "zipf"])),
                        band=bool(rng.integers(0, 2)), seed=700 + i))
    return out


@pytest.mark.parametrize("shape", _random_shapes(12, 77), ids=lambda c: "E%d_T%d_k%d_K%d_N%d_%s%s" % (
    c["E"], c["T"], c["k"], c["K"], c["N"], c["routing"], "_band" if c["band"] else ""))
def test_gmm_random_shapes_all_kernels(shape):
    # seeded shapes across the expert counts, band sizes, K (odd and even
    # chunk counts) and N the kernels handle: both W4A16 kernels and the W4A4
    # kernel against the oracle, each twice (same bits), the two W4A16
    # kernels bit for bit
    c = shape
    p = make_problem(T=c["T"], k=c["k"], E=c["E"], K=c["K"], N=c["N"], seed=c["seed"], routing=c["routing"],
                     x_rows=c["T"] * c["k"] if c["band"] else None, exp_range=(-6, -2))
    w, packed = weights_for(p, "mxfp4")
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.gmm(p["x"], ref_r["sorted_token"] if p["gather"] else None, ref_r["group_offsets"], w)
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    ys = []
    for kernel in KERNELS:
        _, a = run_gpu(p, packed, "mxfp4", kernel=kernel, routed=r)
        _, b = run_gpu(p, packed, "mxfp4", kernel=kernel, routed=r)
        assert rel_err(a.cpu().numpy(), ref) <= REL_TOL
        assert torch.equal(a, b)
        ys.append(a)
    assert torch.equal(ys[0], ys[1])
    ref4 = _w4a4_ref(p, w)
    q = [_run_w4a4(p, packed) for _ in range(2)]
    assert rel_err(q[0].cpu().numpy(), ref4) <= REL_TOL
    assert torch.equal(q[0], q[1])


@pytest.mark.parametrize("shape", _random_shapes(8, 78), ids=lambda c: "E%d_T%d_k%d_K%d_N%d_%s%s" % (
    c["E"], c["T"], c["k"], c["K"], c["N"], c["routing"], "_band" if c["band"] else ""))
def test_gmm_random_shapes_nvfp4_and_activation(shape):
    # the same kind of shapes with NVFP4 weights whose E4M3 block scales are
    # arbitrary (a quarter of the subtiles) or powers of two, through both
    # W4A16 kernels; the fused gate/up activation where N allows it
    c = shape
    p = make_problem(T=c["T"], k=c["k"], E=c["E"], K=c["K"], N=c["N"], seed=c["seed"], routing=c["routing"],
                     x_rows=c["T"] * c["k"] if c["band"] else None, exp_range=(-6, -2))
    rng = np.random.default_rng(c["seed"] + 1)
    E, N, K = c["E"], c["N"], c["K"]
    bs = (rng.integers(2, 15, size=(E, N, K // 16)) << 3).astype(np.uint8)        # powers of two
    general = rng.random((E, N // 16)) < 0.25
    gen_bytes = rng.integers(0x28, 0x48, size=(E, N, K // 16)).astype(np.uint8)
    bs = np.where(np.repeat(general, 16, axis=1)[:, :, None], gen_bytes, bs)
    p["block_scales"] = bs
    p["tensor_scale"] = np.ldexp(1.0, rng.integers(-3, 3, size=E)).astype(np.float32)
    w, packed = weights_for(p, "nvfp4")
    ref_r = oracle.route_sort(p["topk_ids"], E)
    ref = oracle.gmm(p["x"], ref_r["sorted_token"] if p["gather"] else None, ref_r["group_offsets"], w)
    r = moe.route_sort(to_dev(p["topk_ids"]), E)
    ys = []
    for kernel in KERNELS:
        _, y = run_gpu(p, packed, "nvfp4", kernel=kernel, routed=r)
        assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
        ys.append(y)
    assert torch.equal(ys[0], ys[1])
    if N % 128 == 0:
        refa = oracle.silu_mul(ref)
        acts = []
        for kernel in KERNELS:
            _, ya = run_gpu(p, packed, "nvfp4", kernel=kernel, routed=r, act=moe.ACT_SILU_MUL)
            assert rel_err(ya.cpu().numpy(), refa) <= REL_TOL
            acts.append(ya)
        assert torch.equal(acts[0], acts[1])


# ------------------------------------------------- full-size workloads ---

def _sample(M_valid, N, n, seed):
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, M_valid, size=n)
    cols = rng.integers(0, N, size=n)
    rows[:8] = [0, M_valid - 1] * 4
    cols[:8] = [0, N - 1, 0, N - 1, 1, N - 2, 15, 16]
    return rows, cols


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_gmm_config_sampled(cfg):
    p = make_config(cfg)
    fmt = "nvfp4" if cfg == 5 else "mxfp4"
    w, packed = weights_for(p, fmt)
    out_dtype = moe.BF16 if p["out"] == "bf16" else moe.F32
    r, y = run_gpu(p, packed, fmt, out_dtype=out_dtype)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    assert np.array_equal(r["sorted_token"].cpu().numpy(), ref_r["sorted_token"])
    M = p["T"] * p["k"]
    rows, cols = _sample(M, p["N"], 3000, 400 + cfg)
    ri = ref_r["sorted_token"] if p["gather"] else None
    ref = oracle.gmm_sampled(p["x"], ri, ref_r["group_offsets"], w, rows, cols)
    got = y.float().cpu().numpy()[rows, cols].astype(np.float64)
    if out_dtype == moe.BF16:
        assert np.all(np.abs(got - ref) <= bf16_ulp(ref))
        _, y32 = run_gpu(p, packed, fmt, routed=r)
        got = y32.cpu().numpy()[rows, cols]
    assert rel_err(got, ref) <= REL_TOL
    if cfg == 1:
        full = oracle.gmm(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w)
        _, y32 = run_gpu(p, packed, fmt, routed=r)
        assert rel_err(y32.cpu().numpy(), full) <= REL_TOL


@pytest.mark.slow
@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 4])
def test_gmm_silu_mul_config_sampled(cfg):
    p = make_config(cfg)
    w, packed = weights_for(p, "mxfp4")
    r, y = run_gpu(p, packed, "mxfp4", act=moe.ACT_SILU_MUL)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    M, H = p["T"] * p["k"], p["N"] // 2
    rows, cols = _sample(M, H, 2000, 450 + cfg)
    g = oracle.gmm_sampled(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w, rows, cols)
    u = oracle.gmm_sampled(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w, rows, cols + H)
    ref = oracle.silu(g) * u
    got = y.cpu().numpy()[rows, cols].astype(np.float64)
    assert rel_err(got, ref) <= REL_TOL


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_gmm_config_full_output(cfg):
    # every output element of the full-size decode workloads against the
    # whole oracle: f32 output to the 1e-5 bound, and for config 2 (timed with
    # bf16 output) the bf16 output as well.  A bf16 output is the RNE of the
    # f32 sum, so it equals the f32 output's RNE bit for bit and lies within
    # one bf16 ulp of the oracle plus the f32 sum's own 1e-5 max|ref| bound
    # (the second term governs outputs whose sum cancels to near zero)
    p = make_config(cfg)
    fmt = "nvfp4" if cfg == 5 else "mxfp4"
    w, packed = weights_for(p, fmt)
    r, y32 = run_gpu(p, packed, fmt)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    assert np.array_equal(r["group_offsets"].cpu().numpy(), ref_r["group_offsets"])
    ri = ref_r["sorted_token"] if p["gather"] else None
    bands = oracle_gmm_bands(p["x"], ri, ref_r["group_offsets"], w)
    off = ref_r["group_offsets"]
    ref = np.concatenate([bands[e] for e in sorted(bands)])
    assert ref.shape == (int(off[-1]), p["N"]) and off[-1] == p["T"] * p["k"]
    assert rel_err(y32.cpu().numpy(), ref) <= REL_TOL
    if p["out"] == "bf16":
        _, yb = run_gpu(p, packed, fmt, out_dtype=moe.BF16, routed=r)
        assert torch.equal(yb, y32.to(torch.bfloat16))
        got = yb.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + REL_TOL * np.max(np.abs(ref)))


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 3])
def test_gmm_ep_share_full_output(cfg):
    # one GPU's share of the decode workloads under expert parallelism over 8
    # GPUs (experts e % 8 == 0, local ids e // 8, one top-1 row per pair
    # routed to them): 54 gathered rows over 32 experts for w13, 319
    # band-ordered rows for w2 with the Zipf head band of 201 rows (the split
    # kernel's tiled units).  Every output against the whole oracle, and the
    # tiled kernel bit for bit equal
    p = make_ep_share(cfg, gpus=8, rank=0)
    assert p["E"] == 32 and p["k"] == 1
    w, packed = weights_for(p, "mxfp4")
    r, y = run_gpu(p, packed, "mxfp4")
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    assert np.array_equal(r["group_offsets"].cpu().numpy(), ref_r["group_offsets"])
    assert np.array_equal(r["sorted_token"].cpu().numpy(), ref_r["sorted_token"])
    ri = ref_r["sorted_token"] if p["gather"] else None
    bands = oracle_gmm_bands(p["x"], ri, ref_r["group_offsets"], w)
    ref = np.concatenate([bands[e] for e in sorted(bands)])
    assert ref.shape == (p["T"], p["N"])
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
    _, yt = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED, routed=r)
    assert torch.equal(yt, y)


@pytest.mark.parametrize("cfg", [2, 3])
def test_gmm_batch1_decode_full_output(cfg):
    # one token (six routed rows) with the config's weights: the streaming
    # choice gets at most one wave per SIMD and runs two-subtile waves with
    # four chunks in flight (K = 4096 and 2048: 32 and 16 chunks, both with a
    # ragged last round of the ring).  Every output against the oracle, the
    # bf16 output equal to the f32 one's RNE, and the tiled kernel bit for
    # bit equal
    p = make_tokens_problem(cfg, 1)
    assert p["T"] * p["k"] == 6
    w, packed = weights_for(p, "mxfp4")
    r, y = run_gpu(p, packed, "mxfp4")
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ri = ref_r["sorted_token"] if p["gather"] else None
    bands = oracle_gmm_bands(p["x"], ri, ref_r["group_offsets"], w)
    ref = np.concatenate([bands[e] for e in sorted(bands)])
    assert ref.shape == (6, p["N"])
    assert rel_err(y.cpu().numpy(), ref) <= REL_TOL
    _, yb = run_gpu(p, packed, "mxfp4", out_dtype=moe.BF16, routed=r)
    assert torch.equal(yb, y.to(torch.bfloat16))
    _, yt = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED, routed=r)
    assert torch.equal(yt, y)
    if cfg == 2:
        # the w13 of a batch-1 layer: the fused activation on the same path,
        # each wave one gate and one up subtile
        ref_h = oracle.silu_mul(ref)
        _, h = run_gpu(p, packed, "mxfp4", act=moe.ACT_SILU_MUL, routed=r)
        assert tuple(h.shape) == (6, p["N"] // 2)
        assert rel_err(h.cpu().numpy(), ref_h) <= REL_TOL
        _, ht = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED, act=moe.ACT_SILU_MUL, routed=r)
        assert torch.equal(ht, h)


@pytest.mark.slow
def test_gmm_config4_whole_experts():
    # every output of 32 whole experts' bands (every eighth expert) of the
    # 4,096-token prefill, f32 output
    p = make_config(4)
    w, packed = weights_for(p, "mxfp4")
    r, y = run_gpu(p, packed, "mxfp4")
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    off = ref_r["group_offsets"]
    experts = list(range(0, p["E"], 8))
    bands = oracle_gmm_bands(p["x"], ref_r["sorted_token"], off, w, experts)
    yh = y.cpu().numpy()
    got = np.concatenate([yh[off[e]:off[e + 1]] for e in experts])
    ref = np.concatenate([bands[e] for e in experts])
    assert ref.shape[0] >= 32 * 64
    assert rel_err(got, ref) <= REL_TOL


@pytest.mark.slow
def test_gmm_w4a4_config4_whole_experts():
    # W4A4 on the 4,096-token prefill: every output of 8 whole experts' bands
    # (over 3,000,000 outputs) against the oracle's W4A4 grouped matmul on its
    # own quantization of the token rows those bands read
    p = make_config(4)
    w, packed = weights_for(p, "mxfp4")
    y = _run_w4a4(p, packed)
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    off = ref_r["group_offsets"]
    experts = list(range(3, p["E"], 32))
    qc, qs = oracle.quantize_mxfp4_rows(p["x"])
    bands = oracle_gmm_bands(None, ref_r["sorted_token"], off, w, experts, quantized=(qc, qs))
    yh = y.cpu().numpy()
    got = np.concatenate([yh[off[e]:off[e + 1]] for e in experts])
    ref = np.concatenate([bands[e] for e in experts])
    assert ref.size >= 3000
    assert rel_err(got, ref) <= REL_TOL


@pytest.mark.slow
@pytest.mark.parametrize("kernel", KERNELS)
def test_gmm_largest_activation_matrix(kernel):
    # the activations at the limit the call accepts (every byte offset below
    # the lane offset that reads zeros): 262,136 token rows x 4096 bf16 =
    # 2^31 - 64 KiB, every row its own expert band entry (top-1 of 8); the
    # rows of the last tokens are checked
    K, N, E = 4096, 256, 8
    T = 0x7FFF0000 // (2 * K)
    p = make_problem(T=1, k=1, E=E, K=K, N=N, seed=470)
    rng = np.random.default_rng(471)
    p["x"] = random_bf16_bits(rng, (T, K))
    p["topk_ids"] = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    p["T"] = T
    w, packed = weights_for(p, "mxfp4")
    print("largest activation matrix: T=%d K=%d kernel=%d" % (T, K, kernel), flush=True)
    r, y = run_gpu(p, packed, "mxfp4", kernel=kernel)
    ref_r = oracle.route_sort(p["topk_ids"], E)
    assert np.array_equal(r["group_offsets"].cpu().numpy(), ref_r["group_offsets"])
    rows, cols = _sample(T, N, 1500, 472)
    rows[8:24] = ref_r["pair_row"][T - 16:]                   # the last 16 tokens' rows
    ref = oracle.gmm_sampled(p["x"], ref_r["sorted_token"], ref_r["group_offsets"], w, rows, cols)
    got = y.cpu().numpy()[rows, cols].astype(np.float64)
    assert rel_err(got, ref) <= REL_TOL


def test_gmm_w4a4_largest_activation_codes():
    # W4A4 at the limit the call accepts for its activation codes: 1,048,544
    # token rows x 2048 code bytes = 2^31 - 64 KiB (random codes and E8M0
    # scales), every row its own band entry (top-1 of 8), gathered through
    # row_index; the rows of the last tokens are among the samples
    from oracle.formats import decode_mxfp4
    K, N, E = 4096, 256, 8
    T = 0x7FFF0000 // (K // 2)
    p = make_problem(T=1, k=1, E=E, K=K, N=N, seed=480)
    rng = np.random.default_rng(481)
    qc = rng.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
    qs = (rng.integers(-4, 1, size=(T, K // 32)) + 127).astype(np.uint8)
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    w, packed = weights_for(p, "mxfp4")
    print("largest W4A4 activation codes: T=%d K=%d" % (T, K), flush=True)
    r = moe.route_sort(to_dev(ids), E)
    y = moe.moe_gmm_w4a4(packed, E, N, K, to_dev(qc), to_dev(qs), r["group_offsets"], T,
                         row_index=r["sorted_token"])
    ref_r = oracle.route_sort(ids, E)
    assert np.array_equal(r["group_offsets"].cpu().numpy(), ref_r["group_offsets"])
    rows, cols = _sample(T, N, 1500, 482)
    rows[8:24] = ref_r["pair_row"][T - 16:]                   # the last 16 tokens' rows
    off = ref_r["group_offsets"]
    ref = np.empty(len(rows))
    for i, (row, col) in enumerate(zip(rows, cols)):
        e = int(np.searchsorted(off, row, side="right") - 1)
        src = int(ref_r["sorted_token"][row])
        xa = decode_mxfp4(qc[src], qs[src])
        wc = decode_mxfp4(p["codes"][e, col], p["scales"][e, col])
        ref[i] = float(np.dot(xa, wc))
    got = y.cpu().numpy()[rows, cols].astype(np.float64)
    assert rel_err(got, ref) <= REL_TOL


def test_config5_nvfp4_equals_mxfp4_bitwise():
    p = make_config(5)
    _, packed_mx = weights_for(p, "mxfp4")
    # NVFP4 scales produced on the GPU by the library's own lossless cast
    bs, ts, err = moe.mxfp4_to_nvfp4(to_dev(p["scales"]))
    assert err.item() == 0
    packed_nv = moe.mxfp4_encode(to_dev(p["codes"]), bs, ts, moe.NVFP4)
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    for kernel in KERNELS:
        _, a = run_gpu(p, packed_mx, "mxfp4", kernel=kernel, routed=r)
        _, b = run_gpu(p, packed_nv, "nvfp4", kernel=kernel, routed=r)
        assert torch.equal(a, b)
    del packed_mx, packed_nv


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 4])
def test_full_size_kernels_agree_bitwise(cfg):
    p = make_config(cfg)
    _, packed = weights_for(p, "mxfp4")
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    _, a = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_STREAM, routed=r)
    _, b = run_gpu(p, packed, "mxfp4", kernel=moe.GMM_TILED, routed=r)
    assert torch.equal(a, b)


# --------------------------------------------------------------- combine ---

@pytest.mark.parametrize("ydt", [moe.F32, moe.BF16])
def test_combine_matches_oracle(ydt):
    p = make_problem(T=256, k=6, E=32, K=128, N=512, seed=500, routing="zipf")
    p["topk_ids"][5, 2] = -7                          # a dropped pair
    rng = np.random.default_rng(501)
    M = p["T"] * p["k"]
    yf = rng.standard_normal((M, p["N"])).astype(np.float32)
    y = to_dev(yf)
    if ydt == moe.BF16:
        y = y.to(torch.bfloat16)
        yf = y.float().cpu().numpy()
    r = moe.route_sort(to_dev(p["topk_ids"]), p["E"])
    out = moe.moe_combine(y, to_dev(p["topk_weights"]), r["pair_row"]).cpu().numpy()
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    ref = oracle.combine(yf, p["topk_weights"], ref_r["pair_row"])
    assert rel_err(out, ref) <= REL_TOL


@pytest.mark.slow
def test_combine_strides_past_its_grid_cap():
    # 2^23 + 4096 tokens of 512 columns (k = 1): 2^30 + 2^19 four-column
    # quads, more than the 2^22 workgroups of 256 threads the launch is capped
    # at, so the last 4,096 tokens come from each thread's second stride.
    # Every output against the closed form of one slot, RNE_bf16(f32(w * y)),
    # and 96 tokens on both sides of the stride against the oracle.
    T, N = (1 << 23) + 4096, 512
    g = torch.Generator(device=DEV).manual_seed(520)
    y = torch.randn((T, N), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    w = torch.rand((T, 1), generator=g, device=DEV, dtype=torch.float32) + 0.5
    pair_row = torch.randperm(T, generator=g, device=DEV).to(torch.int32)
    out = moe.moe_combine(y, w, pair_row, out_dtype=moe.BF16)
    torch.cuda.synchronize()
    step = 1 << 20
    for t0 in range(0, T, step):
        sl = slice(t0, min(T, t0 + step))
        ref = (w[sl] * y[pair_row[sl].long()].float()).to(torch.bfloat16)
        assert torch.equal(out[sl], ref), t0
        del ref
    toks = np.concatenate([np.arange(0, 32), np.arange((1 << 23) - 32, (1 << 23) + 32), np.arange(T - 32, T)])
    pr = pair_row.cpu().numpy()
    rows = pr[toks]
    got = out[torch.from_numpy(toks).to(DEV)].float().cpu().numpy()
    ref = oracle.combine(y[torch.from_numpy(rows).long().to(DEV)].float().cpu().numpy(),
                         w[torch.from_numpy(toks).to(DEV)].cpu().numpy(),
                         np.arange(len(toks), dtype=np.int32))
    # one bf16 rounding (after an f32 one) of the exact product
    assert np.all(np.abs(got - ref) <= bf16_ulp(ref))


@pytest.mark.slow
def test_config3_w2_then_combine():
    p = make_config(3)
    w, packed = weights_for(p, "mxfp4")
    r, y = run_gpu(p, packed, "mxfp4")
    out = moe.moe_combine(y, to_dev(p["topk_weights"]), r["pair_row"]).cpu().numpy()
    ref_r = oracle.route_sort(p["topk_ids"], p["E"])
    # the oracle combine over oracle rows needed by the sampled tokens only
    rng = np.random.default_rng(503)
    toks = rng.choice(p["T"], size=12, replace=False)
    cols = np.arange(0, p["N"], 37)
    k = p["k"]
    rows = np.array([ref_r["pair_row"][t * k + j] for t in toks for j in range(k)])
    rr, cc = np.repeat(rows, len(cols)), np.tile(cols, len(rows))
    yref = oracle.gmm_sampled(p["x"], None, ref_r["group_offsets"], w, rr, cc).reshape(len(rows), len(cols))
    ref = np.zeros((len(toks), len(cols)))
    for i, t in enumerate(toks):
        for j in range(k):
            ref[i] += float(p["topk_weights"][t, j]) * yref[i * k + j]
    assert rel_err(out[np.ix_(toks, cols)], ref) <= REL_TOL


# ----------------------------------------------------- graph capture ---
@pytest.mark.parametrize("w4a4", [False, True])
def test_graph_capture_layer_replays_match_eager(w4a4):
    # one routed-expert layer (route sort into a caller workspace, w13 with
    # the fused activation, w2, combine; the W4A4 layer also quantizes x and
    # h) captured once in a HIP graph, then replayed on new routing,
    # activations and router weights copied into the captured inputs: every
    # replay equals the eager calls on the same inputs bit for bit, with eager
    # work and host synchronisations between the replays.  No call of the
    # path records a memset or an allocation of its own.
    E, K, N, T, k = 8, 256, 512, 80, 3
    H, M = N // 2, T * k
    probs = [make_problem(T=T, k=k, E=E, K=K, N=N, seed=320 + i, routing="zipf" if i % 2 else "uniform")
             for i in range(5)]
    _, pk13 = weights_for(probs[0], "mxfp4")
    rng = np.random.default_rng(330)
    w2c = rng.integers(0, 256, size=(E, K, H // 2), dtype=np.uint8)
    w2s = (rng.integers(-6, -1, size=(E, K, H // 32)) + 127).astype(np.uint8)
    pk2 = moe.mxfp4_encode(to_dev(w2c), to_dev(w2s), None, moe.MXFP4)
    ids, x, tw = to_dev(probs[0]["topk_ids"]), to_dev(probs[0]["x"]), to_dev(probs[0]["topk_weights"])
    ws = torch.empty(moe.route_sort_workspace_bytes(T, k, E) // 4 + 1, dtype=torch.int32, device=DEV)

    def layer():
        r = moe.route_sort(ids, E, ws=ws)
        if w4a4:
            qc, qs = moe.mxfp4_quantize(x)
            h = moe.moe_gmm_w4a4(pk13, E, N, K, qc, qs, r["group_offsets"], M, row_index=r["sorted_token"],
                                 out_dtype=moe.BF16, act=moe.ACT_SILU_MUL)
            hc, hs = moe.mxfp4_quantize(h)
            y2 = moe.moe_gmm_w4a4(pk2, E, K, H, hc, hs, r["group_offsets"], M)
        else:
            h = moe.moe_gmm(pk13, moe.MXFP4, E, N, K, x, r["group_offsets"], M, row_index=r["sorted_token"],
                            out_dtype=moe.BF16, act=moe.ACT_SILU_MUL)
            y2 = moe.moe_gmm(pk2, moe.MXFP4, E, K, H, h, r["group_offsets"], M)
        return moe.moe_combine(y2, tw, r["pair_row"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g = layer()
    torch.cuda.synchronize()
    for i, p in enumerate(probs):
        ids.copy_(to_dev(p["topk_ids"]))
        x.copy_(to_dev(p["x"]))
        tw.copy_(to_dev(p["topk_weights"]))
        ref = layer()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), i
        assert bool(torch.isfinite(ref).all())


# ------------------------------------------------------- calibration ---
def test_calib_mfma_closed_form():
    # all-ones A with B = 1 or 2: every 16x16x32 MFMA adds 32 * b to each of
    # a lane's 4 accumulator elements; a lane holds 32 tiles and each
    # iteration runs 4 rounds, so its sum is 128 * 128 * iters * b (exact)
    blocks, iters = 3, 5
    a = torch.full((blocks * 256 * 64,), 1.0, dtype=torch.bfloat16, device="cuda")
    for bv in (1.0, 2.0):
        b = torch.full((blocks * 256 * 32,), bv, dtype=torch.bfloat16, device="cuda")
        out = moe.calib_mfma_bf16(a, b, blocks, iters)
        torch.cuda.synchronize()
        assert torch.all(out == 16384.0 * iters * bv)



def test_calib_parts_closed_form():
    # all-ones A, B, staging source and decoded codes (byte 0x22: two e2m1
    # codes of 1.0, scale 1): every MFMA adds 32 to each of a lane's 4
    # accumulator elements, so a lane's sum is 4 * rows16 * 4 * 32 * 4 *
    # chunks = 2048 * rows16 * chunks whatever data movement runs beside it
    # (the code stream wraps inside each wave's 8 KiB region, the staging
    # inside 8 KiB); the register-decode part decodes changing codes, so its
    # sums are only finite
    blocks, chunks = 3, 10
    a = torch.full((blocks * 256 * 64,), 1.0, dtype=torch.bfloat16, device="cuda")
    b = torch.full((blocks * 256 * 32,), 1.0, dtype=torch.bfloat16, device="cuda")
    codes = torch.full((blocks * 4 * 8192,), 0x22, dtype=torch.uint8, device="cuda")
    x = torch.full((4096,), 1.0, dtype=torch.bfloat16, device="cuda")
    P = moe
    for rows16 in (8, 6):
        for parts in (0, P.PARTS_LDS_A, P.PARTS_CODES, P.PARTS_STAGE, P.PARTS_BARRIER, P.PARTS_CODES_XOR,
                      P.PARTS_LDS_A | P.PARTS_CODES | P.PARTS_STAGE):
            out = moe.calib_mfma_parts(parts, rows16, a, b, codes, x, 1.0, blocks, chunks)
            torch.cuda.synchronize()
            assert torch.all(out == 2048.0 * rows16 * chunks), (parts, rows16, out[:4])
        out = moe.calib_mfma_parts(P.PARTS_REG_DECODE, rows16, a, b, codes, x, 1.0, blocks, chunks)
        torch.cuda.synchronize()
        assert torch.all(torch.isfinite(out))


def test_calib_hbm_read_closed_form():
    # the XOR of every thread's partial is the XOR of the buffer's 32-bit
    # words: regions of unequal length, bytes past the last whole 1 KiB run,
    # fewer runs than waves, and no whole run at all
    rng = np.random.default_rng(105)
    for nbytes, blocks in (((1 << 22) + 48, 7), ((1 << 22) + 2048 + 32, 5), (4096, 3), (48, 2)):
        buf = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
        out = moe.calib_hbm_read(torch.from_numpy(buf.view(np.int32)).to(DEV), blocks)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(buf)
