"""The grouped weight gradient for expert shapes (dr_grouped_wgrad): private
token slots whose partials stay in registers, merged in slot order.

It must give the bits of the materialised-partials path
(dr_grouped_splitk_gemm_tn + dr_grouped_splitk_reduce), whose partials and
reduce are pinned to the oracle elsewhere; here it is also checked against
the oracle directly: the oracle's slot tree over the GPU's own slot partials
gives exactly its bits, and dW lies within 1e-4 * sum |x dy| of the exact fp64
product (bitwise-determinism interview note, multiple-writers row: one
private slot per writer, merged in a fixed order).  All calls go through the
C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_bits_equal, dev, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dr():
    require_gpu()
    import bitwise_deterministic_fp32_amd as m
    m.dr_set_launch_params(reset=True)
    yield m
    m.dr_set_launch_params(reset=True)


CASES = [
    # seed, M, N, group offsets, split_tokens
    (1, 512, 256, [0, 1000, 1000, 2999, 3000], 256),   # 4, 0, 8 and 1 slots: an empty group, a one-token group
    (2, 256, 128, [0, 4500, 5000], 128),               # 36 slots (5 chunks: the chunk-sum merge) and 4
    (3, 264, 136, [0, 700, 1500], 100),                # ragged M and N tiles; slots of 100 tokens (partial stages)
    (4, 256, 128, [0, 17, 33, 1000], 2048),            # every group one slot, shorter than a stage
    (5, 7168, 256, [0, 640, 1900], 512),               # the expert hidden size
    (6, 8, 8, [0, 5, 300], 64),                        # one 8 x 8 corner of a tile: the rest of it zeros
]


def _inputs(seed, M, N, off):
    K = off[-1]
    rng = np.random.default_rng(seed)
    X = workloads.bf16_bits(rng.standard_normal((K, M)).astype(np.float32))
    dY = workloads.bf16_bits(rng.standard_normal((K, N)).astype(np.float32))
    return K, X, dY


@pytest.mark.parametrize("seed,M,N,off,split", CASES)
def test_grouped_wgrad_matches_materialised_path_and_oracle(dr, seed, M, N, off, split):
    say(f"grouped wgrad M={M} N={N} offsets={off} split={split}")
    K, X, dY = _inputs(seed, M, N, off)
    Xd, dYd, offd = dev_bf16(X), dev_bf16(dY), dev(np.array(off, np.int32))
    out, ws = dr.dr_grouped_wgrad(Xd, dYd, offd, split)
    dr.dr_workspace_status(ws)
    got = host(out)
    # the materialised path: every slot partial in memory, then the reduce
    P, so, wsg = dr.dr_grouped_splitk_gemm_tn(Xd, dYd, offd, split)
    ref = host(dr.dr_grouped_splitk_reduce(P, so, wsg))
    assert_bits_equal(got, ref, "grouped wgrad vs materialised partials")
    # the oracle's slot tree over the GPU's slot partials gives the same bits
    so_h = host(so)
    want_so, _ = oracle.grouped_slots(off, split)
    assert np.array_equal(so_h, want_so)
    nslots = int(so_h[-1])
    Ph = host(P[:nslots]) if nslots else np.zeros((0, M, N), np.float32)
    assert_bits_equal(got, oracle.grouped_splitk_reduce(Ph, so_h), "grouped wgrad vs oracle tree")
    # and dW within the split-K tolerance of the exact product, group by group
    for g in range(len(off) - 1):
        a, b = off[g], off[g + 1]
        if a == b:
            assert np.all(got[g] == 0) and not np.signbit(got[g]).any()
            continue
        exact, A = oracle.splitk_reference(X[a:b], dY[a:b])
        assert np.all(np.abs(got[g].astype(np.float64) - exact) <= 1e-4 * A), g


def test_grouped_wgrad_launch_invariance(dr):
    K, X, dY = _inputs(7, 512, 256, [0, 2500, 2600, 4000])
    off = dev(np.array([0, 2500, 2600, 4000], np.int32))
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    say("grouped wgrad launch invariance")
    ref, _ = dr.dr_grouped_wgrad(Xd, dYd, off, 128)
    ref = host(ref)
    try:
        for grid in (1, 3, 7, 64, 300):
            dr.dr_set_launch_params(grid_blocks=grid)
            got, _ = dr.dr_grouped_wgrad(Xd, dYd, off, 128)
            assert_bits_equal(host(got), ref, f"grid {grid}")
    finally:
        dr.dr_set_launch_params(reset=True)
    # a garbage-filled workspace and output change nothing
    ws = torch.full((dr.dr_grouped_wgrad_workspace_size(K, 3, 128, 512, 256),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    out = torch.full((3, 512, 256), float("nan"), device="cuda")
    dr.dr_grouped_wgrad(Xd, dYd, off, 128, out=out, ws=ws)
    assert_bits_equal(host(out), ref, "poisoned workspace")


def test_grouped_wgrad_bad_offsets_fail_closed(dr):
    K, X, dY = _inputs(8, 256, 128, [0, 300, 600])
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    out = torch.full((2, 256, 128), 7.0, device="cuda")
    say("grouped wgrad bad offsets")
    for bad in ([0, 400, 300], [0, 300, 601], [-1, 300, 600]):
        _, ws = dr.dr_grouped_wgrad(Xd, dYd, dev(np.array(bad, np.int32)), 64, out=out)
        with pytest.raises(dr.DetReduceError):
            dr.dr_workspace_status(ws)
        assert torch.all(out == 7.0)
