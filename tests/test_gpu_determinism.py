"""Bitwise repeatability, launch invariance and batch invariance of the
deterministic paths, compared byte for byte through fingerprints and host
copies, plus the negative control on the atomic baselines and the
fail-closed behaviour on bad device data.

The pages' harness semantics are mirrored: replays under contention from a side
stream, input sizes large enough that many workgroups compete for the same
outputs, and a negative control proving the comparison is sensitive
(Megatron-LM determinism reference, section 4.4; bitwise comparison of section
4.5)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_bits_equal, dev, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def dr():
    require_gpu()
    import bitwise_deterministic_fp32_amd as m
    m.dr_set_launch_params(reset=True)
    yield m
    m.dr_set_launch_params(reset=True)


class Contention:
    """Keeps a side stream busy with bandwidth and MFMA work during replays."""

    def __init__(self):
        self.stream = torch.cuda.Stream()
        self.a = torch.randn(4096, 4096, device="cuda", dtype=torch.float32)
        self.buf = torch.empty(64 << 20, dtype=torch.float32, device="cuda")

    def __enter__(self):
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            for _ in range(4):
                self.buf.copy_(self.buf.flip(0))
                self.a = self.a @ self.a * 1e-3
        return self

    def __exit__(self, *exc):
        torch.cuda.synchronize()


@pytest.fixture(scope="module")
def contention():
    require_gpu()
    return Contention()


def replay_fingerprints(dr, fn, replays=REPLAYS, contention=None):
    out = []
    for r in range(replays):
        if contention is not None and r % 2 == 1:
            with contention:
                t = fn()
        else:
            t = fn()
        out.append(dr.fingerprint_value(t))
    return out


# ---------------------------------------------------------------------------
# inputs (moderate sizes: many workgroups per destination)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def moe(dr):
    inp = workloads.moe_inputs(11, 2048, 256, 8, 2048, "bf16", zipf_bias_s=1.2)
    _, _, inv = dr.dr_sort_by_dest(dev(inp.expert_ids.reshape(-1)), 256)
    return inp, dev_bf16(inp.rows), inv.view(inp.T, inp.k), dev(inp.gates)


@pytest.fixture(scope="module")
def dk(dr):
    inp = workloads.sparse_attn_inputs(13, Q=1024, K=8192, S=256, H=128)
    return inp, dev_bf16(inp.src), dev(inp.index), dev(inp.out0)


# ---------------------------------------------------------------------------
# repeatability and the negative control
# ---------------------------------------------------------------------------
def test_combine_replays_bit_exact(dr, moe, contention):
    say("combine replays")
    inp, rows, row_of, gates = moe
    fps = replay_fingerprints(dr, lambda: dr.dr_combine(rows, row_of, gates), contention=contention)
    assert len(set(fps)) == 1, fps


def test_index_add_replays_bit_exact(dr, dk, contention):
    say("index_add replays")
    inp, src, index, out0 = dk

    def run():
        out = out0.clone()
        dr.dr_index_add(out, src, index)
        return out
    fps = replay_fingerprints(dr, run, contention=contention)
    assert len(set(fps)) == 1, fps


def test_sort_replays_bit_exact(dr, dk, contention):
    say("sort replays")
    inp, src, index, out0 = dk
    fps = replay_fingerprints(dr, lambda: dr.dr_sort_by_dest(index, inp.D)[0], contention=contention)
    assert len(set(fps)) == 1


def test_splitk_replays_bit_exact(dr, contention):
    say("splitk replays")
    inp = workloads.splitk_inputs(17, 4096, 1024, 24, 16)
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    fps = replay_fingerprints(dr, lambda: dr.dr_splitk_reduce(dr.dr_splitk_gemm_tn(X, dY, 16)), contention=contention)
    assert len(set(fps)) == 1


def test_atomic_baselines_are_nondeterministic(dr, dk, moe):
    """Negative control: with many writers per element the atomic paths change bits
    between replays, so the byte comparison above is able to see an order change."""
    say("atomic negative control")
    inp, src, index, out0 = dk

    def run_index_add():
        out = out0.clone()
        dr.dr_index_add_atomic(out, src, index)
        return out
    fps = replay_fingerprints(dr, run_index_add, replays=6)
    assert len(set(fps)) > 1, "index_add_atomic gave identical bits in every replay"
    # and the deterministic answer is within rounding of the atomic one
    det = out0.clone()
    dr.dr_index_add(det, src, index)
    at = run_index_add()
    torch.testing.assert_close(det, at, rtol=1e-4, atol=1e-4)

    inp2, rows, row_of, gates = moe

    def run_combine():
        out = torch.zeros(inp2.T, inp2.H, dtype=torch.float32, device="cuda")
        dr.dr_combine_atomic(rows, row_of, gates, out=out)
        return out
    fps = replay_fingerprints(dr, run_combine, replays=6)
    assert len(set(fps)) > 1, "combine_atomic gave identical bits in every replay"


# ---------------------------------------------------------------------------
# launch invariance: grid size, tile size and sort tile never change a bit
# ---------------------------------------------------------------------------
def test_index_add_launch_invariance(dr, dk):
    inp, src, index, out0 = dk
    ref = None
    for grid in (0, 1, 7, 64, 1000):
        for tc in (3, 4, 5, 6, 7):
            for st in (8, 10, 12, 13):
                if grid not in (0, 7) and (tc, st) != (5, 12):
                    continue
                cif = 1 + (tc + st + grid) % 2
                say(f"index_add launch grid={grid} tile=2^{tc} sort_tile=2^{st} chunks_in_flight={cif}")
                dr.dr_set_launch_params(grid_blocks=grid, tile_chunks_log2=tc, sort_tile_log2=st,
                                        chunks_in_flight=cif)
                try:
                    out = out0.clone()
                    dr.dr_index_add(out, src, index)
                    fp = dr.fingerprint_value(out)
                finally:
                    dr.dr_set_launch_params(reset=True)
                ref = fp if ref is None else ref
                assert fp == ref, (grid, tc, st)


@pytest.mark.parametrize("H", [128, 384])
def test_sparse_attn_dk_launch_invariance_and_replays(dr, H):
    """Grid, tile and sort-tile sizes never change a bit; with a grid of one or
    seven workgroups every wavefront walks many items (and with H = 384 the
    items of a tile's three column slices), so the look-ahead across items is
    exercised.  The first result is also the oracle's."""
    inp = workloads.sparse_attn_dk_inputs(31, 600, 400, 32, H, s=1.1)
    Q, dS, idx = dev_bf16(inp.Q), dev(inp.dS), dev(inp.key_idx)
    ref = None
    for grid, tc, st in ((0, 5, 0), (7, 3, 8), (1000, 7, 12), (0, 4, 13), (0, 6, 10), (1, 5, 0), (0, 5, 0)):
        say(f"sparse_attn_dk H={H} launch grid={grid} tile=2^{tc} sort_tile={st}")
        dr.dr_set_launch_params(grid_blocks=grid, tile_chunks_log2=tc, sort_tile_log2=st)
        try:
            dK = dev(inp.dK0)
            dr.dr_sparse_attn_dk(dK, Q, dS, idx)
            fp = dr.fingerprint_value(dK)
        finally:
            dr.dr_set_launch_params(reset=True)
        if ref is None:
            assert_bits_equal(host(dK), oracle.sparse_attn_dk(inp.dK0, inp.Q, inp.dS, inp.key_idx), "sparse_attn_dk")
        ref = fp if ref is None else ref
        assert fp == ref, (grid, tc, st)
    # a reused plan (scales read by source id) on small grids
    perm, seg, _ = dr.dr_sort_by_dest(idx.reshape(-1).contiguous(), 400, want_inv=False)
    for grid in (1, 7):
        say(f"sparse_attn_dk H={H} reused plan grid={grid}")
        dr.dr_set_launch_params(grid_blocks=grid)
        try:
            dK = dev(inp.dK0)
            dr.dr_sparse_attn_dk(dK, Q, dS, idx, perm=perm, seg_offsets=seg)
            fp = dr.fingerprint_value(dK)
        finally:
            dr.dr_set_launch_params(reset=True)
        assert fp == ref, ("reused plan", grid)


def test_sort_launch_invariance(dr, dk):
    inp, src, index, out0 = dk
    ref = None
    for st in (8, 9, 10, 11, 12, 13):
        dr.dr_set_launch_params(sort_tile_log2=st)
        try:
            p, s, i = dr.dr_sort_by_dest(index, inp.D)
            fp = (dr.fingerprint_value(p), dr.fingerprint_value(s), dr.fingerprint_value(i))
        finally:
            dr.dr_set_launch_params(reset=True)
        ref = fp if ref is None else ref
        assert fp == ref, st


def test_fingerprint_grid_invariance(dr):
    t = dev(workloads.normal_f32(5, 0, (1 << 20) + 3))
    ref = dr.fingerprint_value(t)
    for grid in (1, 3, 64, 1024, 8192):
        dr.dr_set_launch_params(grid_blocks=grid)
        try:
            assert dr.fingerprint_value(t) == ref, grid
        finally:
            dr.dr_set_launch_params(reset=True)


def test_splitk_grid_invariance(dr):
    """Persistent split-K workgroups may take any share of the (split, tile)
    items: the partials, and so the reduced result, keep their bits."""
    say("splitk grid invariance")
    inp = workloads.splitk_inputs(23, 3000, 200, 24, 5)  # ragged M tile and a short last stage
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    ref = host(dr.dr_splitk_gemm_tn(X, dY, 5))
    for grid in (1, 3, 17, 1000):
        dr.dr_set_launch_params(grid_blocks=grid)
        try:
            got = host(dr.dr_splitk_gemm_tn(X, dY, 5))
        finally:
            dr.dr_set_launch_params(reset=True)
        assert_bits_equal(got, ref, f"grid {grid}")


# ---------------------------------------------------------------------------
# batch invariance
# ---------------------------------------------------------------------------
def test_combine_batch_invariance(dr, moe):
    """A token's bytes are the same alone, in any subset, or in the full batch."""
    say("combine batch invariance")
    inp, rows, row_of, gates = moe
    full = host(dr.dr_combine(rows, row_of, gates))
    rng = np.random.default_rng(3)
    for size in (1, 2, 17, 1000):
        sel = np.sort(rng.choice(inp.T, size, replace=False))
        idx = dev(sel.astype(np.int64))
        sub = host(dr.dr_combine(rows, row_of[idx].contiguous(), gates[idx].contiguous()))
        assert_bits_equal(sub, full[sel], f"subset of {size}")


def test_index_add_batch_invariance(dr, dk):
    """A destination row's bytes depend only on its own ordered contributions."""
    say("index_add batch invariance")
    inp, src, index, out0 = dk
    full = out0.clone()
    dr.dr_index_add(full, src, index)
    idx_h = inp.index
    keep = (idx_h % 5 == 0) | (idx_h < 20)
    kept_rows = np.unique(idx_h[keep])
    sel = dev(np.nonzero(keep)[0].astype(np.int64))
    part = out0.clone()
    dr.dr_index_add(part, src[sel].contiguous(), index[sel].contiguous())
    rows = dev(kept_rows.astype(np.int64))
    assert_bits_equal(host(part[rows]), host(full[rows]), "kept rows")


def test_splitk_batch_invariance(dr):
    """A dW row depends only on its own column of X: column subsets give equal rows,
    whatever the M tiling of the launch."""
    say("splitk batch invariance")
    inp = workloads.splitk_inputs(19, 2048, 512, 24, 8)
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    full = host(dr.dr_splitk_reduce(dr.dr_splitk_gemm_tn(X, dY, 8)))
    for cols in (np.arange(0, 512, 7), np.array([5]), np.arange(100, 163)):
        c = dev(cols.astype(np.int64))
        sub = host(dr.dr_splitk_reduce(dr.dr_splitk_gemm_tn(X[:, c].contiguous(), dY, 8)))
        assert_bits_equal(sub, full[cols], f"{len(cols)} columns")


def test_combine_ep_size_invariance(dr, moe):
    """The order key is the row (expert), not the slot: permuting each token's slots,
    as a different expert-parallel layout would, gives the same bytes."""
    inp, rows, row_of, gates = moe
    full = host(dr.dr_combine(rows, row_of, gates))
    p = dev(np.random.default_rng(4).permutation(inp.k).astype(np.int64))
    alt = host(dr.dr_combine(rows, row_of[:, p].contiguous(), gates[:, p].contiguous()))
    assert_bits_equal(alt, full, "slot permutation")


# ---------------------------------------------------------------------------
# fail closed on bad device data
# ---------------------------------------------------------------------------
def test_index_add_out_of_range_leaves_out_untouched(dr, dk):
    say("index_add fail closed")
    inp, src, index, out0 = dk
    bad = index.clone()
    bad[12345] = inp.D  # one index out of range
    out = out0.clone()
    _, ws = dr.dr_index_add(out, src, bad)
    with pytest.raises(dr.DetReduceError) as e:
        dr.dr_workspace_status(ws)
    assert e.value.status == 4
    assert dr.fingerprint_value(out) == dr.fingerprint_value(out0)
    bad[12345] = -1
    _, ws = dr.dr_index_add(out, src, bad)
    with pytest.raises(dr.DetReduceError):
        dr.dr_workspace_status(ws)
    assert dr.fingerprint_value(out) == dr.fingerprint_value(out0)
    # the same workspace is usable again for a good call
    dr.dr_index_add(out, src, index, ws=ws)
    dr.dr_workspace_status(ws)


def test_index_add_bad_plan_is_refused(dr, dk):
    say("index_add bad plan")
    inp, src, index, out0 = dk
    perm, seg, _ = dr.dr_sort_by_dest(index, inp.D, want_inv=False)
    seg_h = host(seg)
    d_long = int(np.argmax(np.diff(seg_h)))  # a segment with at least two rows
    lo = int(seg_h[d_long])
    for corrupt in ("seg", "perm", "order", "duplicate"):
        p, s = perm.clone(), seg.clone()
        if corrupt == "seg":
            s[100] = s[101] + 1  # not monotone
        elif corrupt == "perm":
            p[0], p[-1] = p[-1].clone(), p[0].clone()  # rows in the wrong segments
        elif corrupt == "order":
            p[lo], p[lo + 1] = p[lo + 1].clone(), p[lo].clone()  # right segment, wrong source order
        else:
            p[lo + 1] = p[lo].clone()  # a source row twice, another never
        out = out0.clone()
        _, ws = dr.dr_index_add(out, src, index, perm=p, seg_offsets=s)
        with pytest.raises(dr.DetReduceError) as e:
            dr.dr_workspace_status(ws)
        assert e.value.status == 6, corrupt
        assert dr.fingerprint_value(out) == dr.fingerprint_value(out0)


def test_sort_out_of_range_reports(dr):
    dest = dev(np.array([0, 1, 2, 9, 1], np.int32))
    ws = torch.empty(dr.dr_sort_workspace_size(5, 9), dtype=torch.uint8, device="cuda")
    dr.dr_sort_by_dest(dest, 9, ws=ws)
    with pytest.raises(dr.DetReduceError):
        dr.dr_workspace_status(ws)
    src = dev(np.array([0, 1, 7, 2, 1], np.int32))
    ws2 = torch.empty(dr.dr_sort_workspace_size(5, 10, 5), dtype=torch.uint8, device="cuda")
    dr.dr_sort_by_dest(dest, 10, src, 5, ws=ws2)
    with pytest.raises(dr.DetReduceError):
        dr.dr_workspace_status(ws2)


def test_combine_bad_row_poisons_token_only(dr):
    rows = dev(np.ones((10, 8), np.float32))
    row_of = dev(np.array([[0, 1], [2, 10], [3, 4]], np.int32))
    gates = dev(np.ones((3, 2), np.float32))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = host(dr.dr_combine(rows, row_of, gates, dev_status=status))
    assert np.all(out[0] == 2.0) and np.all(out[2] == 2.0)
    assert np.all(np.isnan(out[1]))
    with pytest.raises(dr.DetReduceError):
        dr.dr_read_status(status)


# ---------------------------------------------------------------------------
# special values stay bit-exact run to run (GPU vs GPU)
# ---------------------------------------------------------------------------
def test_signed_zero_and_nan_replay(dr):
    n, H = 5000, 16
    rng = np.random.default_rng(9)
    index = rng.integers(0, 40, n).astype(np.int32)
    src = rng.standard_normal((n, H)).astype(np.float32)
    src[::7] = -0.0
    src[5, 3] = np.float32("nan")
    out0 = np.zeros((40, H), np.float32)
    out0[::3] = -0.0
    res = []
    for _ in range(3):
        out = dev(out0)
        dr.dr_index_add(out, dev(src), dev(index))
        res.append(host(out).view(np.uint32).copy())
    assert all(np.array_equal(res[0], r) for r in res)
    # a row whose contributions are all -0.0 on a -0.0 destination stays -0.0
    z_out = dev(np.full((2, 4), -0.0, np.float32))
    dr.dr_index_add(z_out, dev(np.full((9, 4), -0.0, np.float32)), dev(np.zeros(9, np.int32)))
    assert (host(z_out).view(np.uint32) == 0x80000000).all()
    want = oracle.index_add(np.full((2, 4), -0.0, np.float32), np.full((9, 4), -0.0, np.float32), np.zeros(9, np.int32))
    assert_bits_equal(host(z_out), want, "signed zeros")
