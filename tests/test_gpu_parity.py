"""Parity of every deterministic entry point with the CPU oracle, element by
element, on seeded inputs at sizes the oracle finishes in seconds.  The sizes
span several workgroup tiles and end in ragged tails.  All calls go through the
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
    return m


# ---------------------------------------------------------------------------
# sort
# ---------------------------------------------------------------------------
SORT_CASES = [
    # (n, num_dests, with_src, src_bound, distribution)
    (0, 5, False, 0, "uniform"),
    (1, 1, False, 0, "uniform"),
    (1000, 1, False, 0, "uniform"),
    (4095, 7, False, 0, "uniform"),
    (100003, 300, False, 0, "zipf"),
    (100003, 65536, False, 0, "zipf"),
    (70001, 131072, False, 0, "zipf"),
    (50000, 256, True, 50000, "uniform"),
    (30000, 1000, True, 7, "uniform"),  # many duplicate (dest, src) pairs: ties by position
]


@pytest.mark.parametrize("n,D,with_src,src_bound,dist", SORT_CASES)
def test_sort_matches_oracle(dr, n, D, with_src, src_bound, dist):
    say(f"sort n={n} D={D} src={with_src}")
    rng = np.random.default_rng(n + D)
    if dist == "zipf":
        dest = np.minimum(rng.zipf(1.2, n) - 1, D - 1).astype(np.int32)
    else:
        dest = rng.integers(0, D, n).astype(np.int32)
    src = rng.integers(0, src_bound, n).astype(np.int32) if with_src else None
    perm, seg, inv = dr.dr_sort_by_dest(dev(dest), D, None if src is None else dev(src), src_bound)
    want_perm, want_seg, want_inv = oracle.sort_by_dest(dest, D, src)
    assert np.array_equal(host(perm), want_perm)
    assert np.array_equal(host(seg), want_seg)
    assert np.array_equal(host(inv), want_inv)


@pytest.mark.parametrize("sort_tile_log2", [12, 13])
@pytest.mark.parametrize("n,D,with_src,src_bound,dist", [
    (100003, 65536, False, 0, "zipf"),
    (20001, 512, False, 0, "uniform"),      # one 9-bit pass whose bins equal D
    (50000, 256, True, 50000, "uniform"),   # source ids staged through LDS
    (30000, 1000, True, 7, "uniform"),
])
def test_sort_large_tiles_match_oracle(dr, sort_tile_log2, n, D, with_src, src_bound, dist):
    """The largest tiles (32 keys per thread) and a ragged last tile."""
    say(f"sort n={n} D={D} src={with_src} tile=2^{sort_tile_log2}")
    rng = np.random.default_rng(n + D + 1)
    if dist == "zipf":
        dest = np.minimum(rng.zipf(1.2, n) - 1, D - 1).astype(np.int32)
    else:
        dest = rng.integers(0, D, n).astype(np.int32)
    src = rng.integers(0, src_bound, n).astype(np.int32) if with_src else None
    dr.dr_set_launch_params(sort_tile_log2=sort_tile_log2)
    try:
        perm, seg, inv = dr.dr_sort_by_dest(dev(dest), D, None if src is None else dev(src), src_bound)
    finally:
        dr.dr_set_launch_params(reset=True)
    want_perm, want_seg, want_inv = oracle.sort_by_dest(dest, D, src)
    assert np.array_equal(host(perm), want_perm)
    assert np.array_equal(host(seg), want_seg)
    assert np.array_equal(host(inv), want_inv)


BOUNDARY_SORT_CASES = [
    # (n, num_dests, distribution): sizes around the 1 K / 8 K tile steps,
    # one to four digit passes, and a single repeated key
    (1, 1, "uniform"),
    (63, 5, "uniform"),
    (64, 256, "uniform"),
    (65, 257, "zipf"),
    (1025, 65536, "zipf"),
    (4097, 2, "uniform"),
    (8191, 300, "zipf"),
    (8192, 65536, "uniform"),
    (8193, 65536, "zipf"),
    (20000, 1 << 20, "uniform"),   # three 7-bit passes
    (32767, 1 << 25, "uniform"),   # four passes
    (32768, 65536, "zipf"),
    (32768, 7, "same"),            # every key equal: the identity permutation
    (32769, 65536, "zipf"),
]


@pytest.mark.parametrize("n,D,dist", BOUNDARY_SORT_CASES)
def test_sort_tile_boundaries_match_oracle(dr, n, D, dist):
    """Sizes one below, at and one above tile multiples, with the default tile
    and with 2^10-key tiles, equal the oracle."""
    say(f"sort n={n} D={D} {dist}")
    rng = np.random.default_rng(3 * n + D)
    if dist == "zipf":
        dest = np.minimum(rng.zipf(1.2, n) - 1, D - 1).astype(np.int32)
    elif dist == "same":
        dest = np.full(n, D - 1, np.int32)
    else:
        dest = rng.integers(0, D, n).astype(np.int32)
    want_perm, want_seg, want_inv = oracle.sort_by_dest(dest, D, None)
    for tile in (0, 10):
        dr.dr_set_launch_params(sort_tile_log2=tile)
        try:
            perm, seg, inv = dr.dr_sort_by_dest(dev(dest), D)
        finally:
            dr.dr_set_launch_params(reset=True)
        assert np.array_equal(host(perm), want_perm), f"perm, sort tile {tile}"
        assert np.array_equal(host(seg), want_seg), f"seg_offsets, sort tile {tile}"
        assert np.array_equal(host(inv), want_inv), f"inv_perm, sort tile {tile}"


@pytest.mark.parametrize("bad_value", [-1, 100])
def test_index_add_rejects_bad_index(dr, bad_value):
    """An index outside [0, D), here the last of a ragged tile, sets the status
    and leaves out untouched."""
    say(f"index_add with a bad index {bad_value}")
    rng = np.random.default_rng(5)
    n, D, H = 3000, 100, 64
    index = rng.integers(0, D, n).astype(np.int32)
    index[2999] = bad_value
    out0 = workloads.normal_f32(5, 0, D * H).reshape(D, H)
    o = dev(out0)
    src = workloads.normal_f32(5, 1, n * H).reshape(n, H)
    _, ws = dr.dr_index_add(o, dev(src), dev(index))
    with pytest.raises(dr.DetReduceError):
        dr.dr_workspace_status(ws)
    assert_bits_equal(host(o), out0, "out after a bad index")


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------
def _row_of(dr, expert_ids, E):
    """Expert-major row of each (token, slot): the dispatch sort's inverse permutation."""
    T, k = expert_ids.shape
    _, _, inv = dr.dr_sort_by_dest(dev(expert_ids.reshape(-1)), E)
    return inv.view(T, k)


@pytest.mark.parametrize("T,E,k,H,rows_dtype", [
    (256, 8, 2, 128, "f32"),     # the tiny configuration itself
    (1000, 64, 8, 1000, "bf16"),  # 2 column slices, the second one ragged
    (333, 64, 6, 7168, "bf16"),
    (257, 16, 1, 64, "f32"),
    (300, 128, 13, 136, "bf16"),  # k > 8: chunk tree
    (100, 128, 64, 256, "f32"),
])
def test_combine_matches_oracle(dr, T, E, k, H, rows_dtype):
    say(f"combine T={T} E={E} k={k} H={H} {rows_dtype}")
    inp = workloads.moe_inputs(77 + k, T, E, k, H, rows_dtype, zipf_bias_s=1.2)
    row_of_dev = _row_of(dr, inp.expert_ids, E)
    _, _, inv = oracle.sort_by_dest(inp.expert_ids.reshape(-1), E)
    row_of = inv.reshape(T, k)
    assert np.array_equal(host(row_of_dev), row_of)
    rows = dev(inp.rows) if rows_dtype == "f32" else dev_bf16(inp.rows)
    out = dr.dr_combine(rows, row_of_dev, dev(inp.gates))
    want = oracle.combine(inp.rows, row_of, inp.gates)
    assert_bits_equal(host(out), want, "combine")


def test_combine_order_example_fp32(dr):
    """The fp32 analogue of the pages' order example through combine: gates 1, rows [1, x, x]
    in row order give (1+x)+x; rows [x, x, 1] give (x+x)+1."""
    x = np.float32(3 * 2.0 ** -26)
    rows = np.array([[1.0] * 4, [x] * 4, [x] * 4, [x] * 4, [x] * 4, [1.0] * 4], np.float32)
    row_of = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    gates = np.ones((2, 3), np.float32)
    out = host(dr.dr_combine(dev(rows), dev(row_of), dev(gates)))
    assert out.view(np.uint32)[0, 0] == 0x3F800000
    assert out.view(np.uint32)[1, 0] == 0x3F800001


# ---------------------------------------------------------------------------
# index_add
# ---------------------------------------------------------------------------
def _index_add_case(seed, n, D, H, src_dtype, dist):
    rng = np.random.default_rng(seed)
    if dist == "zipf":
        index = np.minimum(rng.zipf(1.1, n) - 1, D - 1).astype(np.int32)
    elif dist == "hot":
        index = np.where(rng.random(n) < 0.5, 3, rng.integers(0, D, n)).astype(np.int32)
    else:
        index = rng.integers(0, D, n).astype(np.int32)
    if src_dtype == "bf16":
        src = workloads.normal_bf16(seed, 1, n * H).reshape(n, H)
    else:
        src = workloads.normal_f32(seed, 1, n * H).reshape(n, H)
    out0 = workloads.normal_f32(seed, 2, D * H).reshape(D, H)
    return index, src, out0


@pytest.mark.parametrize("n,D,H,src_dtype,dist", [
    (0, 10, 128, "bf16", "uniform"),
    (1, 10, 128, "bf16", "uniform"),
    (20000, 4096, 128, "bf16", "zipf"),     # long segments: many multi-tile rows
    (20001, 50, 128, "f32", "hot"),         # one destination with ~10000 rows
    (3000, 131072, 4096, "bf16", "zipf"),   # embedding-like: mostly singletons
    (5000, 300, 136, "f32", "uniform"),     # ragged lane group (34 pieces)
    (4000, 2000, 24, "bf16", "zipf"),       # a row narrower than one lane group
    (30000, 40, 136, "bf16", "hot"),        # long segments merged over a partial second 128-column slice
    (30001, 40, 132, "f32", "hot"),         # the same with fp32 rows (4 columns in the last slice)
])
def test_index_add_matches_oracle(dr, n, D, H, src_dtype, dist):
    say(f"index_add n={n} D={D} H={H} {src_dtype} {dist}")
    index, src, out0 = _index_add_case(n + D + H, n, D, H, src_dtype, dist)
    out = dev(out0.copy())
    s = dev(src) if src_dtype == "f32" else dev_bf16(src)
    _, ws = dr.dr_index_add(out, s, dev(index))
    dr.dr_workspace_status(ws)
    want = oracle.index_add(out0, src, index)
    assert_bits_equal(host(out), want, "index_add")


def test_index_add_deep_tile_merge(dr):
    """With tiles of 2^3 chunks (64 rows), 2^22 rows make the host's bound ask
    tilecombine for 17 levels, its deepest counter form; the hot destination
    (half the rows, about 32,768 tiles) merges its partial rows through it,
    and the result and the kept fingerprint equal the oracle's."""
    n, D, H = (1 << 22) + 5, 1000, 8
    say(f"index_add deep tile merge n={n} D={D} H={H} tile=2^3")
    index, src, out0 = _index_add_case(77, n, D, H, "bf16", "hot")
    dr.dr_set_launch_params(tile_chunks_log2=3)
    try:
        out = dev(out0)
        dr.dr_index_add(out, dev_bf16(src), dev(index))
        got = host(out)
    finally:
        dr.dr_set_launch_params(reset=True)
    assert_bits_equal(got, oracle.index_add(out0, src, index, threads=8), "index_add deep tile merge")
    # the same with the fingerprint kept current
    h0 = oracle.fingerprint(out0)
    h = torch.tensor([h0 - (1 << 64) if h0 >= (1 << 63) else h0], dtype=torch.int64, device="cuda")
    dr.dr_set_launch_params(tile_chunks_log2=3)
    try:
        out = dev(out0)
        dr.dr_index_add_fingerprinted(out, dev_bf16(src), dev(index), h)
        got2 = host(out)
    finally:
        dr.dr_set_launch_params(reset=True)
    assert_bits_equal(got2, got, "fingerprinted")
    assert (int(h.item()) & ((1 << 64) - 1)) == oracle.fingerprint(got), "kept fingerprint"


@pytest.mark.parametrize("D", [10, 4096, 131072])
def test_index_add_empty_with_dirty_workspace(dr, D):
    """No contributions, one or two sort passes, a workspace full of 0xFF bytes:
    the call must clear its own status and plan state and leave out untouched."""
    say(f"index_add n=0 D={D} dirty workspace")
    H = 128
    out0 = workloads.normal_f32(D, 2, D * H).reshape(D, H)
    out = dev(out0.copy())
    src = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    index = torch.empty((0,), dtype=torch.int32, device="cuda")
    ws = torch.full((dr.dr_index_add_workspace_size(0, D, H),), 0xFF, dtype=torch.uint8, device="cuda")
    dr.dr_index_add(out, src, index, ws=ws)
    dr.dr_workspace_status(ws)
    assert_bits_equal(host(out), out0, "index_add with no contributions")


def test_index_add_reused_plan(dr):
    say("index_add reused plan")
    index, src, out0 = _index_add_case(5, 30000, 1000, 128, "bf16", "zipf")
    perm, seg, _ = dr.dr_sort_by_dest(dev(index), 1000, want_inv=False)
    out = dev(out0.copy())
    _, ws = dr.dr_index_add(out, dev_bf16(src), dev(index), perm=perm, seg_offsets=seg)
    dr.dr_workspace_status(ws)
    assert_bits_equal(host(out), oracle.index_add(out0, src, index), "index_add with plan")


def _hash_tensor(v: int):
    return torch.tensor([v - (1 << 64) if v >= (1 << 63) else v], dtype=torch.int64, device="cuda")


def _hash_value(t) -> int:
    return int(t.item()) & ((1 << 64) - 1)


@pytest.mark.parametrize("n,D,H,src_dtype,dist", [
    (20001, 50, 128, "f32", "hot"),         # long segments: tile partials and tilecombine rewrite rows
    (3000, 131072, 4096, "bf16", "zipf"),   # embedding-like: mostly singletons
    (5000, 300, 136, "f32", "uniform"),     # ragged lane group
    (4000, 2000, 24, "bf16", "zipf"),       # a row narrower than one lane group
    (0, 70, 64, "f32", "uniform"),          # nothing to add: the hash stays
])
def test_index_add_fingerprinted_matches_oracle(dr, n, D, H, src_dtype, dist):
    """The incremental fingerprint equals the oracle's fingerprint of the whole updated destination."""
    say(f"index_add_fingerprinted n={n} D={D} H={H} {src_dtype} {dist}")
    index, src, out0 = _index_add_case(n + D + H + 1, n, D, H, src_dtype, dist)
    out = dev(out0.copy())
    h = _hash_tensor(oracle.fingerprint(out0))
    s = dev(src) if src_dtype == "f32" else dev_bf16(src)
    _, ws = dr.dr_index_add_fingerprinted(out, s, dev(index), h)
    dr.dr_workspace_status(ws)
    want = oracle.index_add(out0, src, index)
    assert_bits_equal(host(out), want, "index_add_fingerprinted")
    assert _hash_value(h) == oracle.fingerprint(want)
    # a reused plan and other launch shapes give the same hash; a second call keeps it current
    perm, seg, _ = dr.dr_sort_by_dest(dev(index), D, want_inv=False)
    if n == 0:
        perm = seg = None  # an empty plan has no storage to pass
    dr.dr_set_launch_params(grid_blocks=37, tile_chunks_log2=3)
    try:
        dr.dr_index_add_fingerprinted(out, s, dev(index), h, perm=perm, seg_offsets=seg)
    finally:
        dr.dr_set_launch_params(reset=True)
    want2 = oracle.index_add(want, src, index)
    assert_bits_equal(host(out), want2, "second call")
    assert _hash_value(h) == oracle.fingerprint(want2) == dr.fingerprint_value(out)


def test_index_add_fingerprinted_fails_closed(dr):
    index, src, out0 = _index_add_case(77, 3000, 100, 64, "f32", "uniform")
    index[1234] = 100  # out of range
    out = dev(out0.copy())
    h0 = oracle.fingerprint(out0)
    h = _hash_tensor(h0)
    _, ws = dr.dr_index_add_fingerprinted(out, dev(src), dev(index), h)
    with pytest.raises(dr.DetReduceError):
        dr.dr_workspace_status(ws)
    assert_bits_equal(host(out), out0, "untouched")
    assert _hash_value(h) == h0


def test_phase_events_time_the_reduction(dr):
    """The measurement hook records the caller's events around the reduction kernels and changes no bit."""
    index, src, out0 = _index_add_case(91, 50000, 3000, 256, "bf16", "zipf")
    want = oracle.index_add(out0, src, index)
    out = dev(out0.copy())
    b_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dr.dr_set_phase_events(b_, e_)
    try:
        _, ws = dr.dr_index_add(out, dev_bf16(src), dev(index))
    finally:
        dr.dr_set_phase_events()
    dr.dr_workspace_status(ws)
    assert_bits_equal(host(out), want, "index_add with phase events")
    assert b_.elapsed_time(e_) > 0


def test_index_add_order_example_fp32(dr):
    """old value added last: out0 = 1, contributions [x, x] -> 1 + 2^-23."""
    x = np.float32(3 * 2.0 ** -26)
    out = dev(np.ones((2, 4), np.float32))
    dr.dr_index_add(out, dev(np.full((2, 4), x, np.float32)), dev(np.array([1, 1], np.int32)))
    o = host(out).view(np.uint32)
    assert (o[1] == 0x3F800001).all() and (o[0] == 0x3F800000).all()


# ---------------------------------------------------------------------------
# sparse-attention key gradient (contributions formed in the reduce)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nq,topk,H,K,q_dtype", [
    (300, 16, 128, 512, "bf16"),
    (257, 7, 64, 100, "f32"),      # ragged chunks, fp32 query rows
    (1000, 64, 128, 300, "bf16"),  # keys chosen by up to 1000 queries: several tiles per key
    (3, 5, 8, 9, "bf16"),          # tiny, most keys untouched
    (500, 24, 384, 1000, "bf16"),  # three 128-column slices; top-k not a power of two
    (200, 12, 136, 50, "bf16"),    # a second slice of 8 columns
    (2000, 40, 136, 200, "bf16"),  # keys of several tiles merged over that partial slice
])
def test_sparse_attn_dk_matches_oracle(dr, nq, topk, H, K, q_dtype):
    say(f"sparse_attn_dk nq={nq} topk={topk} H={H} K={K} {q_dtype}")
    inp = workloads.sparse_attn_dk_inputs(nq + K, nq, K, topk, H, s=1.1)
    Qh = inp.Q if q_dtype == "bf16" else workloads.bf16_to_f32(inp.Q)
    Q = dev_bf16(Qh) if q_dtype == "bf16" else dev(Qh)
    dS, idx = dev(inp.dS), dev(inp.key_idx)
    dK = dev(inp.dK0)
    dr.dr_sparse_attn_dk(dK, Q, dS, idx)
    want = oracle.sparse_attn_dk(inp.dK0, Qh, inp.dS, inp.key_idx)
    assert_bits_equal(host(dK), want, "sparse_attn_dk")
    # the same bits as index_add over contributions materialised by torch (fp32 products)
    q_of = torch.arange(nq * topk, device="cuda") // topk
    contrib = (dS.reshape(-1, 1) * Q.float()[q_of]).contiguous()
    ref = dev(inp.dK0)
    dr.dr_index_add(ref, contrib, idx.reshape(-1).contiguous())
    assert_bits_equal(host(ref), want, "index_add over materialised contributions")
    # a reused plan gives the same bits
    perm, seg, _ = dr.dr_sort_by_dest(idx.reshape(-1).contiguous(), K, want_inv=False)
    dK2 = dev(inp.dK0)
    dr.dr_sparse_attn_dk(dK2, Q, dS, idx, perm=perm, seg_offsets=seg)
    assert_bits_equal(host(dK2), want, "reused plan")


@pytest.mark.parametrize("nq", [(1 << 24) - 1, 1 << 24])
def test_sparse_attn_dk_at_the_row_offset_limit(dr, nq):
    """The bf16 LDS form forms row byte offsets with 24-bit multiplies, so it takes
    sources of fewer than 2^24 rows; 2^24 rows go to the generic form.  Both sides
    of that limit, with the last query rows selected, equal the oracle bit for bit."""
    say(f"sparse_attn_dk row-offset limit nq={nq}")
    H, K, topk = 8, 1000, 1
    rng = np.random.default_rng(24 + nq % 7)
    key_idx = rng.integers(0, K, size=(nq, topk), dtype=np.int32)
    key_idx[-3:, 0] = K - 1  # the last source rows land on one key
    Qh = workloads.normal_bf16(31, 0, nq * H).reshape(nq, H)
    dS = workloads.normal_f32(31, 1, nq * topk, 0.1).reshape(nq, topk)
    dK0 = workloads.normal_f32(31, 2, K * H).reshape(K, H)
    dK = dev(dK0)
    dr.dr_sparse_attn_dk(dK, dev_bf16(Qh), dev(dS), dev(key_idx))
    want = oracle.sparse_attn_dk(dK0, Qh, dS, key_idx, threads=8)
    assert_bits_equal(host(dK), want, f"sparse_attn_dk nq={nq}")


def test_sparse_attn_dk_bad_key_leaves_dk_untouched(dr):
    inp = workloads.sparse_attn_dk_inputs(5, 64, 128, 8, 64, s=1.1)
    bad = inp.key_idx.copy()
    bad[10, 3] = 128
    dK = dev(inp.dK0)
    _, ws = dr.dr_sparse_attn_dk(dK, dev_bf16(inp.Q), dev(inp.dS), dev(bad))
    with pytest.raises(dr.DetReduceError):
        dr.dr_workspace_status(ws)
    assert_bits_equal(host(dK), inp.dK0, "dK after a bad key")


# ---------------------------------------------------------------------------
# split-K
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S,count", [
    (9, 4096),     # two chunks of 8 splits, the second a single split
    (16, 1001),    # count not a multiple of 4: one element per lane group
    (17, 4096),    # three chunks: the tree pads the fourth with -0.0
    (64, 7168 * 24 // 4),
    (100, 2052),   # 13 chunks on 16 lanes
    (300, 1000),   # 38 chunks on 64 lanes
    (512, 256),    # 64 chunks, the widest lane group
    (513, 260),    # 65 chunks: one thread walks the chunks
])
def test_splitk_reduce_split_counts(dr, S, count):
    """The reduce stage alone over given partials (wide magnitude range, signed
    zeros), for split counts on both reduce paths; bit-exact to the oracle's tree."""
    say(f"splitk_reduce S={S} count={count}")
    rng = np.random.default_rng(S * 7919 + count)
    P = (rng.standard_normal((S, count)) * np.exp2(rng.integers(-20, 20, (S, count)))).astype(np.float32)
    P[rng.random((S, count)) < 0.01] = np.float32(-0.0)
    got = host(dr.dr_splitk_reduce(dev(P)))
    assert_bits_equal(got, oracle.splitk_reduce(P), f"splitk_reduce S={S}")


@pytest.mark.parametrize("S,count", [
    (64, 7168 * 24),  # a lane per chunk, hashed as stored
    (1, 4096),        # one thread per 4 elements, hashed as stored
    (600, 4096),      # more than 64 chunks: one thread walks them
    (9, 1001),        # count not a multiple of 4: hashed after the reduce
    (5, 0),
    (16, 4),
])
def test_splitk_reduce_fingerprinted(dr, S, count):
    """The reduce with its fingerprint equals dr_splitk_reduce and
    dr_fingerprint, and the oracle's tree and fingerprint, bit for bit."""
    say(f"splitk_reduce_fingerprinted S={S} count={count}")
    rng = np.random.default_rng(S * 31 + count)
    P = (rng.standard_normal((S, count)) * np.exp2(rng.integers(-20, 20, (S, count)))).astype(np.float32)
    P[rng.random((S, count)) < 0.01] = np.float32(-0.0)
    h = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.full((dr.dr_splitk_reduce_fingerprinted_workspace_size(S, count),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    got = dr.dr_splitk_reduce_fingerprinted(dev(P), h, ws=ws)
    want = oracle.splitk_reduce(P)
    assert_bits_equal(host(got), want, f"splitk_reduce_fingerprinted S={S}")
    assert _hash_value(h) == oracle.fingerprint(want), "fused fingerprint differs from the oracle's"
    h2 = dr.dr_fingerprint(dr.dr_splitk_reduce(dev(P)))
    assert _hash_value(h) == _hash_value(h2), "fused fingerprint differs from dr_fingerprint"


@pytest.mark.parametrize("K,M,N,splits", [
    (1024, 256, 24, 4),
    (1000, 200, 24, 7),     # ragged splits and a ragged M tile
    (777, 72, 40, 5),       # two N tiles, ragged
    (256, 64, 1, 1),
    (300, 1, 24, 3),
    (2000, 136, 24, 3),     # three 256-token stages per split, the last one short
    (1500, 128, 20, 1),     # six stages; N not a multiple of 8 (scalar dY staging)
    (600, 64, 36, 2),       # second N tile of 4 columns
    (5000, 1000, 32, 3),    # streaming kernel: four 256-column M tiles, the last 232 wide
    (4100, 520, 8, 9),      # streaming kernel: N = 8, a 4-token tail stage per split
    (700, 2056, 16, 2),     # streaming kernel: nine M tiles, the last 8 wide
    (120, 64, 16, 40),      # streaming kernel: 3-token splits (one short k-step each)
])
def test_splitk_matches_oracle(dr, K, M, N, splits):
    say(f"splitk K={K} M={M} N={N} S={splits}")
    inp = workloads.splitk_inputs(K + M + N, K, M, N, splits)
    partials = dr.dr_splitk_gemm_tn(dev_bf16(inp.X), dev_bf16(inp.dY), splits)
    dW = dr.dr_splitk_reduce(partials)
    P = host(partials)
    # reduce stage: bit-exact against the oracle's tree over the same partials
    assert_bits_equal(host(dW), oracle.splitk_reduce(P), "splitk_reduce")
    # partials and result within the tolerance of the exact fp64 sums
    Pexact = oracle.splitk_partials(inp.X, inp.dY, splits)
    c = -(-K // splits)
    for s in range(splits):
        _, A = oracle.splitk_reference(inp.X[s * c:(s + 1) * c], inp.dY[s * c:(s + 1) * c])
        assert np.all(np.abs(P[s] - Pexact[s]) <= 1e-4 * A + 1e-30), s
    exact, A = oracle.splitk_reference(inp.X, inp.dY)
    assert np.all(np.abs(host(dW) - exact) <= 1e-4 * A + 1e-30)


@pytest.mark.parametrize("K,M,N,splits", [(1000, 200, 24, 7), (5000, 1000, 32, 3), (4100, 520, 8, 9),
                                           (120, 64, 16, 40), (16384, 7168, 24, 64)])
def test_splitk_stream_kernel_matches_tile_kernel(dr, K, M, N, splits):
    """Thin-N partials come from the streaming kernel by default; forcing the
    general tile kernel must give the same bits (both take the same MFMA steps
    of 16 tokens from each split's first token)."""
    say(f"splitk stream vs tile K={K} M={M} N={N} S={splits}")
    inp = workloads.splitk_inputs(K + 3 * M + N, K, M, N, splits)
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    got = {}
    for mode in (1, 2):
        dr.dr_set_launch_params(splitk_stream=mode)
        try:
            got[mode] = host(dr.dr_splitk_gemm_tn(X, dY, splits))
        finally:
            dr.dr_set_launch_params(reset=True)
    assert_bits_equal(got[1], got[2], "stream vs tile partials")


# ---------------------------------------------------------------------------
# grouped split with private slots; the dispatch permute
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,M,N,offsets,split", [
    (2000, 136, 24, [0, 0, 700, 701, 1999, 2000], 256),   # empty, one-token and multi-stage slots
    (1000, 64, 40, list(range(0, 1001, 50)), 37),          # many groups, two N tiles, ragged slots
    (600, 72, 20, [0, 600], 600),                           # one group, one slot, scalar dY staging
    (900, 128, 24, [100, 300, 300, 800], 128),             # tokens outside every group are ignored
])
def test_grouped_splitk_matches_oracle(dr, K, M, N, offsets, split):
    say(f"grouped splitk K={K} M={M} N={N} groups={len(offsets) - 1} split={split}")
    inp = workloads.splitk_inputs(K + M + split, K, M, N, 1)
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    off = np.array(offsets, np.int32)
    P, so, ws = dr.dr_grouped_splitk_gemm_tn(X, dY, dev(off), split)
    dr.dr_workspace_status(ws)
    want_so, ranges = oracle.grouped_slots(off, split)
    assert np.array_equal(host(so), want_so)
    S = int(want_so[-1])
    Ph = host(P)[:S]
    exact = oracle.grouped_splitk_partials(inp.X, inp.dY, off, split)
    for s_, (a, b) in enumerate(ranges):
        _, A = oracle.splitk_reference(inp.X[a:b], inp.dY[a:b])
        assert np.all(np.abs(Ph[s_] - exact[s_]) <= 1e-4 * A + 1e-30), s_
    dW = dr.dr_grouped_splitk_reduce(P, so, ws)
    # reduce stage: bit-exact against the oracle's per-group tree over the same partials
    assert_bits_equal(host(dW), oracle.grouped_splitk_reduce(Ph, want_so), "grouped reduce")
    for g in range(len(offsets) - 1):
        e, A = oracle.splitk_reference(inp.X[off[g]:off[g + 1]], inp.dY[off[g]:off[g + 1]])
        assert np.all(np.abs(host(dW)[g] - e) <= 1e-4 * A + 1e-30), g


def test_grouped_splitk_grid_invariance_and_bad_offsets(dr):
    inp = workloads.splitk_inputs(91, 1500, 200, 24, 1)
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    off = dev(np.array([0, 10, 10, 900, 1500], np.int32))
    ref = None
    for grid in (0, 1, 7, 1000):
        dr.dr_set_launch_params(grid_blocks=grid)
        try:
            P, so, ws = dr.dr_grouped_splitk_gemm_tn(X, dY, off, 100)
            S = int(host(so)[-1])
            got = host(dr.dr_grouped_splitk_reduce(P, so, ws)), host(P)[:S]
        finally:
            dr.dr_set_launch_params(reset=True)
        if ref is None:
            ref = got
        assert_bits_equal(got[0], ref[0], f"grid {grid}")
        assert_bits_equal(got[1], ref[1], f"grid {grid} partials")
    # offsets that run backwards or past K are refused, and out is left alone
    for bad in ([0, 10, 5, 1500], [0, 10, 900, 1501], [-1, 10, 900, 1500]):
        P, so, ws = dr.dr_grouped_splitk_gemm_tn(X, dY, dev(np.array(bad, np.int32)), 100)
        with pytest.raises(dr.DetReduceError) as e:
            dr.dr_workspace_status(ws)
        assert e.value.status == 6, bad
        out = torch.full((3, 200, 24), 7.0, device="cuda")
        dr.dr_grouped_splitk_reduce(P, so, ws, out=out)
        assert bool((out == 7.0).all()), bad


@pytest.mark.parametrize("T,E,k,H,dtype", [(300, 16, 4, 256, "bf16"), (1000, 64, 8, 7168, "bf16"),
                                            (77, 5, 1, 36, "f32")])
def test_permute_rows_matches_oracle(dr, T, E, k, H, dtype):
    say(f"permute T={T} E={E} k={k} H={H}")
    inp = workloads.moe_inputs(T + E + k, T, E, k, H, dtype, zipf_bias_s=1.2)
    rows = workloads.normal_f32(T, 3, T * H).reshape(T, H)
    x = dev_bf16(workloads.bf16_bits(rows)) if dtype == "bf16" else dev(rows)
    perm, _, inv = dr.dr_sort_by_dest(dev(inp.expert_ids.reshape(-1)), E)
    want = oracle.permute_rows(host(x.view(torch.int16) if dtype == "bf16" else x), host(perm), k)
    for inv_perm in (None, inv):  # output order, token order
        out = dr.dr_permute_rows(x, perm, k, inv_perm=inv_perm)
        got = host(out.view(torch.int16) if dtype == "bf16" else out)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_permute_rows_bad_entry(dr):
    x = dev(np.arange(40, dtype=np.float32).reshape(10, 4))
    perm = dev(np.array([0, 3, 25, 7], np.int32))  # 25 // 2 = 12 is not a row
    out = torch.full((4, 4), -1.0, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dr.dr_permute_rows(x, perm, 2, out=out, dev_status=status)
    with pytest.raises(dr.DetReduceError):
        dr.dr_read_status(status)
    o = host(out)
    assert (o[2] == -1.0).all() and o[1].tolist() == [4.0, 5.0, 6.0, 7.0]
    # an inverse that perm does not invert: those rows are refused, the rest are copied
    perm = dev(np.array([1, 0, 3, 2], np.int32))
    inv = dev(np.array([1, 0, 3, 3], np.int32))   # w = 3 claims row 3, which perm gives to w = 2; row 2 is left
    out = torch.full((4, 4), -1.0, device="cuda")
    status.zero_()
    dr.dr_permute_rows(x, perm, 2, inv_perm=inv, out=out, dev_status=status)
    with pytest.raises(dr.DetReduceError):
        dr.dr_read_status(status)
    o = host(out)
    assert o[0].tolist() == [0.0, 1.0, 2.0, 3.0] and o[1].tolist() == [0.0, 1.0, 2.0, 3.0]
    assert o[3].tolist() == [4.0, 5.0, 6.0, 7.0] and (o[2] == -1.0).all()


def test_splitk_reduce_ragged_counts(dr):
    for S, count in [(1, 5), (3, 7), (64, 172032), (100, 1001), (9, 4)]:
        say(f"splitk_reduce S={S} count={count}")
        P = workloads.normal_f32(S + count, 0, S * count).reshape(S, count)
        out = dr.dr_splitk_reduce(dev(P))
        assert_bits_equal(host(out), oracle.splitk_reduce(P), f"splitk_reduce S={S}")


# ---------------------------------------------------------------------------
# fingerprint
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nbytes", [0, 8, 16, 24, 40, 1000, 4096, 1 << 20, (1 << 22) + 24])
def test_fingerprint_matches_oracle(dr, nbytes):
    say(f"fingerprint nbytes={nbytes}")
    rng = np.random.default_rng(nbytes)
    data = rng.integers(0, 256, nbytes, dtype=np.uint8)
    t = dev(data)
    assert dr.fingerprint_value(t) == oracle.fingerprint(data)


def test_fingerprint_odd_lengths_and_dtypes(dr):
    rng = np.random.default_rng(1)
    for n in [1, 3, 5, 7, 9, 1001]:  # int16 tensors: 2n bytes, tails of 2, 6, 10, 14, 18 bytes
        a = rng.integers(-30000, 30000, n).astype(np.int16)
        assert dr.fingerprint_value(dev(a)) == oracle.fingerprint(a)
    f = workloads.normal_f32(3, 0, 12345)
    assert dr.fingerprint_value(dev(f)) == oracle.fingerprint(f)
    z = np.zeros(4, np.float32)
    nz = z.copy()
    nz[2] = -0.0
    assert dr.fingerprint_value(dev(z)) != dr.fingerprint_value(dev(nz))


@pytest.mark.parametrize("T,E,k,H,rows_dtype", [
    (1000, 64, 8, 1000, "bf16"),
    (257, 16, 1, 64, "f32"),
    (300, 128, 13, 136, "bf16"),
    (9000, 64, 8, 1024, "bf16"),   # over 1024 partials: the one-workgroup wide final sum
    (270000, 16, 9, 64, "f32"),    # over 65536 partials: the two-level final sum
])
def test_combine_fingerprinted_matches_separate_calls(dr, T, E, k, H, rows_dtype):
    say(f"combine_fingerprinted T={T} k={k} H={H} {rows_dtype}")
    inp = workloads.moe_inputs(91 + k, T, E, k, H, rows_dtype, zipf_bias_s=1.2)
    row_of = _row_of(dr, inp.expert_ids, E)
    rows = dev(inp.rows) if rows_dtype == "f32" else dev_bf16(inp.rows)
    gates = dev(inp.gates)
    out, h = dr.dr_combine_fingerprinted(rows, row_of, gates)
    ref = dr.dr_combine(rows, row_of, gates)
    assert_bits_equal(host(out), host(ref), "fused combine output")
    hv = int(h.item()) & ((1 << 64) - 1)
    assert hv == dr.fingerprint_value(ref)
    assert hv == oracle.fingerprint(host(ref))
    # a poisoned token is hashed as written
    bad = row_of.clone()
    bad[T // 2, 0] = inp.T * inp.k + 5
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out2, h2 = dr.dr_combine_fingerprinted(rows, bad, gates, dev_status=status)
    assert np.isnan(host(out2)[T // 2]).all()
    assert int(h2.item()) & ((1 << 64) - 1) == oracle.fingerprint(host(out2))


# ---------------------------------------------------------------------------
# workspace contents
# ---------------------------------------------------------------------------
def _filled(nbytes, byte):
    return torch.full((max(int(nbytes), 16),), byte, dtype=torch.uint8, device="cuda")


def test_results_do_not_depend_on_workspace_contents(dr):
    """Every entry point that takes a workspace gives the same bytes (and a clear
    status) whether its workspace starts as zeros or as 0xFF bytes, and whatever
    its outputs held before: no call may read state it has not written itself."""
    say("workspace contents: sort, index_add, sparse_attn_dk, combine_fingerprinted, grouped split, decode, fingerprint")
    runs = {}
    for byte in (0x00, 0xFF):
        got = {}
        # sort: two destination passes with source ids, and one pass
        rng = np.random.default_rng(1)
        dest = dev(np.minimum(rng.zipf(1.2, 30000) - 1, 1999).astype(np.int32))
        src = dev(rng.integers(0, 30000, 30000).astype(np.int32))
        for D, s_ids, bound in ((2000, src, 30000), (256, None, 0)):
            ws = _filled(dr.dr_sort_workspace_size(30000, D, bound), byte)
            perm = torch.full((30000,), -7, dtype=torch.int32, device="cuda")
            seg = torch.full((D + 1,), -7, dtype=torch.int32, device="cuda")
            p, sg, inv = dr.dr_sort_by_dest(torch.minimum(dest, torch.tensor(D - 1, device="cuda", dtype=torch.int32)),
                                            D, s_ids, bound, perm=perm, seg_offsets=seg, ws=ws)
            dr.dr_workspace_status(ws)
            got[f"sort{D}"] = (host(p), host(sg), host(inv))
        # index_add with its own sort (two passes), plain and fingerprinted
        index, srcr, out0 = _index_add_case(3, 20000, 4096, 128, "bf16", "zipf")
        for fp in (False, True):
            out = dev(out0.copy())
            ws = _filled(dr.dr_index_add_workspace_size(20000, 4096, 128), byte)
            if fp:
                h = _hash_tensor(oracle.fingerprint(out0))
                dr.dr_index_add_fingerprinted(out, dev_bf16(srcr), dev(index), h, ws=ws)
                got["index_add_fp_hash"] = _hash_value(h)
            else:
                dr.dr_index_add(out, dev_bf16(srcr), dev(index), ws=ws)
            dr.dr_workspace_status(ws)
            got[f"index_add{fp}"] = host(out)
        # fused sparse-attention key gradient
        inp = workloads.sparse_attn_dk_inputs(5, Q=256, K=2048, S=32, H=128)
        dK = dev(inp.dK0.copy())
        ws = _filled(dr.dr_sparse_attn_dk_workspace_size(256, 32, 2048, 128), byte)
        dr.dr_sparse_attn_dk(dK, dev_bf16(inp.Q), dev(inp.dS), dev(inp.key_idx), ws=ws)
        dr.dr_workspace_status(ws)
        got["sparse_attn_dk"] = host(dK)
        # combine with its fingerprint
        m = workloads.moe_inputs(9, 300, 64, 8, 520, "bf16", zipf_bias_s=1.2)
        row_of = _row_of(dr, m.expert_ids, 64)
        ws = _filled(dr.dr_combine_fingerprinted_workspace_size(torch.bfloat16, 520, 300), byte)
        out, h = dr.dr_combine_fingerprinted(dev_bf16(m.rows), row_of, dev(m.gates), ws=ws)
        got["combine"] = (host(out), _hash_value(h))
        # grouped split: slot table, partials and per-group reduce
        sk = workloads.splitk_inputs(11, 2000, 200, 24, 1)
        off = dev(np.array([0, 700, 700, 1500, 2000], np.int32))
        ws = _filled(dr.dr_grouped_splitk_workspace_size(2000, 4, 256), byte)
        P, so, ws = dr.dr_grouped_splitk_gemm_tn(dev_bf16(sk.X), dev_bf16(sk.dY), off, 256, ws=ws)
        dr.dr_workspace_status(ws)
        got["grouped"] = (host(so), host(dr.dr_grouped_splitk_reduce(P, so, ws)))
        # decode attention
        di = workloads.decode_inputs(13, B=3, Lmax=1000, Hq=8, Hkv=2, D=128)
        ws = _filled(dr.dr_decode_attention_workspace_size(3, 8, 1000, 256, 128), byte)
        st = torch.zeros(1, dtype=torch.int32, device="cuda")  # decode reports device errors here only
        o = dr.dr_decode_attention(dev_bf16(di.q), dev_bf16(di.k), dev_bf16(di.v), dev(di.lens), di.scale, 256,
                                   ws=ws, dev_status=st)
        dr.dr_read_status(st)
        got["decode"] = host(o)
        # fingerprint
        data = dev(np.arange(1 << 18, dtype=np.int32))
        ws = _filled(dr.dr_fingerprint_workspace_size(1 << 20), byte)
        got["fingerprint"] = _hash_value(dr.dr_fingerprint(data, ws=ws))
        runs[byte] = got
    for key in runs[0x00]:
        a, b = runs[0x00][key], runs[0xFF][key]
        a = a if isinstance(a, tuple) else (a,)
        b = b if isinstance(b, tuple) else (b,)
        for x, y in zip(a, b):
            if isinstance(x, np.ndarray):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), key
            else:
                assert x == y, key
