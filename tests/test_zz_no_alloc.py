"""moe_route_sort_noalloc (the route sort for callers that cannot allocate)
against moe_route_sort with a caller workspace, through the C ABI: every
output bit for bit, on consecutive calls that share the library's per-GPU
count table, the later ones smaller (the table keeps the earlier call's
contents, which must not leak into the result)."""

import ctypes

import numpy as np
import pytest
import torch

import moe_grouped_gemm_route_amd as moe

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(ids, E):
    T, k = ids.shape
    M = T * k
    out = {key: torch.full((M,), -7, dtype=torch.int32, device=DEV)
           for key in ("sorted_token", "sorted_pair", "pair_row")}
    out["group_offsets"] = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    out["err_count"] = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = moe.library().moe_route_sort_noalloc(
        _ptr(ids), T, k, E, _ptr(out["group_offsets"]), _ptr(out["sorted_token"]),
        _ptr(out["sorted_pair"]), _ptr(out["pair_row"]), _ptr(out["err_count"]), stream)
    assert st == 0, moe.library().moe_status_string(st)
    return out


def test_noalloc_route_sort_matches_workspace_call():
    torch.cuda.set_device(0)
    rng = np.random.default_rng(301)
    # two-kernel path (24 segments of 256 experts, then 8 of 1,024 experts,
    # with dropped ids), then the one-workgroup path that needs no table
    cases = [(4096, 6, 256, 0.0), (1000, 8, 1024, 0.05), (64, 6, 256, 0.0)]
    for T, k, E, drop in cases:
        ids = rng.integers(0, E, size=(T, k), dtype=np.int32)
        ids[rng.random(ids.shape) < drop] = E + 1
        d_ids = torch.from_numpy(ids).to(DEV)
        got = _noalloc(d_ids, E)
        ref = moe.route_sort(d_ids, E)
        torch.cuda.synchronize()
        for key in ("group_offsets", "sorted_token", "sorted_pair", "pair_row", "err_count"):
            assert torch.equal(got[key], ref[key]), (T, k, E, key)
