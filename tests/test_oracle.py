"""Pins for the CPU oracle, checked against facts the pages and mathematics fix.

Each test compares the oracle with something that is not the oracle: a value
printed on the pages, a closed form, a textbook special case computed with
numpy float32 scalars, an independent formulation of the same tree, an fp64
error bound, brute force on tiny inputs, or a library routine.
"""
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import read_golden

F32 = np.float32
U = 2.0 ** -24  # unit roundoff of binary32


def bits32(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def from_bits32(b: int) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------------------
# Independent formulations of the tree (numpy float32; none calls the oracle)
# ---------------------------------------------------------------------------
def lr_sum(v):
    """Textbook left-to-right float32 sum starting from the first element."""
    v = np.asarray(v, dtype=F32)
    s = F32(v[0])
    for x in v[1:]:
        s = F32(s + F32(x))
    return s


def stride_doubling(sums):
    """Pairwise tree by stride doubling over leaves padded with -0.0 to a power of two."""
    s = np.asarray(sums, dtype=F32)
    size = 1
    while size < s.size:
        size *= 2
    s = np.concatenate([s, np.full(size - s.size, -0.0, dtype=F32)])
    while s.size > 1:
        s = (s[0::2] + s[1::2]).astype(F32)
    return F32(s[0])


def chunk_sums(v):
    v = np.asarray(v, dtype=F32)
    return [lr_sum(v[i:i + 8]) for i in range(0, v.size, 8)]


def padded_tree(v):
    return stride_doubling(chunk_sums(v))


def binary_counter_tree(v):
    """Streaming form: push chunk sums on a binary counter, fold from the right at the end."""
    stack = []  # list of (level, value), levels strictly decreasing
    for s in chunk_sums(v):
        level = 0
        while stack and stack[-1][0] == level:
            _, left = stack.pop()
            s = F32(left + s)
            level += 1
        stack.append((level, s))
    acc = stack.pop()[1]
    while stack:
        acc = F32(stack.pop()[1] + acc)
    return acc


def tiled_tree(v, m):
    """Aligned tiles of 2^m chunks reduced on their own, then the pairwise tree over tile sums."""
    cs = chunk_sums(v)
    width = 2 ** m
    tiles = [stride_doubling(cs[i:i + width]) for i in range(0, len(cs), width)]
    return stride_doubling(tiles)


def mixed_values(rng, n):
    """Mixed-magnitude float32 values (exponents spread over ~40 binades), both signs."""
    mant = rng.standard_normal(n)
    expo = rng.integers(-20, 20, n)
    return (mant * 2.0 ** expo).astype(F32)


# ---------------------------------------------------------------------------
# The pages' worked example and its fp32 analogue
# ---------------------------------------------------------------------------
def test_bf16_worked_example(golden_dir):
    g = read_golden(os.path.join(golden_dir, "bf16_order_example.txt"))
    x_bits = int(g["x_bits"], 16)
    one_bits = int(g["one_bits"], 16)
    # the fixture's bit patterns encode the page's printed numbers
    assert float(workloads.bf16_to_f32(np.array([x_bits], np.uint16))[0]) == float(g["x_value"]) == 3 * 2.0 ** -10
    names = {"x": x_bits, "one": one_bits}
    for order in ("order_a", "order_b"):
        seq = np.array([names[s] for s in g[order + "_inputs"].split(",")], dtype=np.uint16)
        got = oracle.tree_sum_bf16(seq)
        assert got == int(g[order + "_bits"], 16), (order, hex(got))
        assert float(workloads.bf16_to_f32(np.array([got], np.uint16))[0]) == float(g[order + "_value"])


def test_fp32_analogue_of_worked_example():
    # x = 3*2^-26 is below half an ulp of 1.0 (2^-24) but x+x = 1.5*2^-24 is above it.
    x = F32(3 * 2.0 ** -26)
    assert bits32(oracle.tree_sum_f32([1.0, x, x])) == 0x3F800000
    assert bits32(oracle.tree_sum_f32([x, x, 1.0])) == 0x3F800001


# ---------------------------------------------------------------------------
# Tree: special cases, formulations, bound
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("L", list(range(1, 9)))
def test_tree_up_to_eight_is_left_to_right(L):
    rng = np.random.default_rng(L)
    for _ in range(50):
        v = mixed_values(rng, L)
        assert bits32(oracle.tree_sum_f32(v)) == bits32(lr_sum(v))


@pytest.mark.parametrize("m", range(0, 7))
def test_tree_full_power_of_two_chunks_is_pairwise(m):
    rng = np.random.default_rng(100 + m)
    L = 8 * 2 ** m
    for _ in range(10):
        v = mixed_values(rng, L)
        # textbook pairwise summation over the 2^m chunk sums
        s = [lr_sum(v[i:i + 8]) for i in range(0, L, 8)]
        while len(s) > 1:
            s = [F32(s[i] + s[i + 1]) for i in range(0, len(s), 2)]
        assert bits32(oracle.tree_sum_f32(v)) == bits32(s[0])


LENGTHS = list(range(1, 301)) + [511, 512, 513, 1000, 4345, 8192]


def test_tree_shape_equivalent_formulations():
    """The oracle's recursive split equals padded stride doubling, the binary counter,
    and every aligned 2^m-chunk tiling (the property that makes any grid give the same bits)."""
    rng = np.random.default_rng(7)
    for L in LENGTHS:
        v = mixed_values(rng, L)
        want = bits32(oracle.tree_sum_f32(v))
        assert bits32(padded_tree(v)) == want, L
        assert bits32(binary_counter_tree(v)) == want, L
        if L in (37, 129, 300, 513, 4345):
            for m in range(0, 7):
                assert bits32(tiled_tree(v, m)) == want, (L, m)


def test_midpoint_tree_is_a_different_reading():
    """Negative control for the shape test: a midpoint split disagrees for some length."""
    def midpoint(s):
        if len(s) == 1:
            return s[0]
        h = (len(s) + 1) // 2
        return F32(midpoint(s[:h]) + midpoint(s[h:]))
    rng = np.random.default_rng(8)
    differs = 0
    for L in range(17, 200):
        v = mixed_values(rng, L)
        differs += bits32(midpoint(chunk_sums(v))) != bits32(oracle.tree_sum_f32(v))
    assert differs > 0


def test_tree_error_bound_fp64():
    rng = np.random.default_rng(9)
    for L in [1, 2, 7, 8, 9, 63, 64, 65, 1000, 4096, 5000]:
        for _ in range(5):
            v = mixed_values(rng, L)
            exact = math.fsum(float(x) for x in v)
            absum = math.fsum(abs(float(x)) for x in v)
            C = (L + 7) // 8
            depth = (min(L, 8) - 1) + (math.ceil(math.log2(C)) if C > 1 else 0)
            gamma = depth * U / (1 - depth * U)
            got = float(oracle.tree_sum_f32(v))
            assert abs(got - exact) <= gamma * absum + 1e-45, (L, got, exact)


def test_tree_brute_force_tiny_exact_cases():
    # sums of small integers are exact in float32 whatever the order
    rng = np.random.default_rng(10)
    for L in range(1, 120):
        v = rng.integers(-1000, 1000, L).astype(F32)
        assert float(oracle.tree_sum_f32(v)) == float(v.astype(np.float64).sum())


def test_tree_subnormals_kept():
    tiny = from_bits32(1)  # 2^-149
    got = oracle.tree_sum_f32(np.full(20, tiny, dtype=F32))
    assert bits32(got) == 20  # 20 * 2^-149, exact, not flushed


def test_tree_signed_zero():
    assert bits32(oracle.tree_sum_f32([-0.0])) == 0x80000000
    assert bits32(oracle.tree_sum_f32([-0.0] * 13)) == 0x80000000
    assert bits32(oracle.tree_sum_f32([-0.0, 0.0])) == 0


def test_tree_permutation_sensitive():
    """The tree is a fixed order: permuting inputs may change bits (pages: order decides the last bit)."""
    rng = np.random.default_rng(11)
    changed = 0
    for _ in range(200):
        v = mixed_values(rng, 64)
        changed += bits32(oracle.tree_sum_f32(v)) != bits32(oracle.tree_sum_f32(rng.permutation(v)))
    assert changed > 0


def test_order_demo_diagnostic():
    """The four orders of the pages' demo (sequential, pairwise, 4-block split, shuffled) over
    mixed-magnitude fp32 values; the spread is reported as (max-min)/ulp(max).  Over many draws
    some spread is nonzero, which is what the replay tests rely on to see an order change."""
    rng = np.random.default_rng(12)
    spreads = []
    for _ in range(200):
        v = mixed_values(rng, 16)
        a = lr_sum(v)
        b = stride_doubling(v)
        c = lr_sum([lr_sum(v[i:i + 4]) for i in range(0, 16, 4)])
        d = lr_sum(rng.permutation(v))
        r = np.array([a, b, c, d], dtype=F32)
        hi = r[np.argmax(np.abs(r))]
        ulp = np.spacing(np.abs(hi))
        spreads.append(float((r.max() - r.min()) / ulp))
    assert max(spreads) > 0


# ---------------------------------------------------------------------------
# Sort
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("with_src", [False, True])
def test_sort_brute_force(with_src):
    rng = np.random.default_rng(20)
    for trial in range(30):
        n = int(rng.integers(0, 300))
        D = int(rng.integers(1, 40))
        dest = rng.integers(0, D, n).astype(np.int32)
        src = rng.integers(0, 50, n).astype(np.int32) if with_src else None
        perm, seg, inv = oracle.sort_by_dest(dest, D, src)
        key = (lambda i: (dest[i], src[i], i)) if with_src else (lambda i: (dest[i], i))
        want = sorted(range(n), key=key)
        assert list(perm) == want
        assert list(inv[perm]) == list(range(n))
        counts = np.bincount(dest, minlength=D)
        assert list(seg) == [0] + list(np.cumsum(counts))


def test_sort_rejects_out_of_range():
    with pytest.raises(oracle.OracleError):
        oracle.sort_by_dest(np.array([0, 5], np.int32), 5)
    with pytest.raises(oracle.OracleError):
        oracle.sort_by_dest(np.array([-1], np.int32), 5)


# ---------------------------------------------------------------------------
# index_add / scatter-reduce
# ---------------------------------------------------------------------------
def test_index_add_short_segments_match_sequential_add_at():
    """With a zero destination and at most 8 contributions per row, the defined order is the
    plain sequential index_add in source order (numpy's unbuffered add.at)."""
    rng = np.random.default_rng(30)
    D, H = 64, 16
    index = np.repeat(np.arange(D, dtype=np.int32), rng.integers(0, 9, D))
    index = rng.permutation(index).astype(np.int32)
    src = mixed_values(rng, index.size * H).reshape(-1, H)
    want = np.zeros((D, H), F32)
    np.add.at(want, index, src)
    got = oracle.index_add(np.zeros((D, H), F32), src, index)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_index_add_old_value_added_last():
    # out0 = 1, contributions [x, x] with x = 3*2^-26: 1 + (x + x) = 1 + 2^-23, whereas
    # adding the old value first would give (1 + x) + x = 1.
    x = F32(3 * 2.0 ** -26)
    out0 = np.ones((2, 1), F32)
    got = oracle.index_add(out0, np.array([[x], [x]], F32), np.array([1, 1], np.int32))
    assert bits32(got[1, 0]) == 0x3F800001
    assert bits32(got[0, 0]) == 0x3F800000  # untouched row


def test_index_add_bf16_source_is_exact_widening():
    rng = np.random.default_rng(31)
    D, H, n = 16, 8, 100
    index = rng.integers(0, D, n).astype(np.int32)
    f = rng.standard_normal((n, H)).astype(F32)
    b = workloads.bf16_bits(f)
    w = workloads.bf16_to_f32(b)
    got_b = oracle.index_add(np.zeros((D, H), F32), b, index)
    got_f = oracle.index_add(np.zeros((D, H), F32), w, index)
    assert np.array_equal(got_b.view(np.uint32), got_f.view(np.uint32))


def test_index_add_untouched_rows_and_fp64_bound():
    rng = np.random.default_rng(32)
    D, H, n = 200, 24, 5000
    index = np.minimum(rng.zipf(1.3, n) - 1, D - 1).astype(np.int32)
    src = mixed_values(rng, n * H).reshape(n, H)
    out0 = mixed_values(rng, D * H).reshape(D, H)
    got = oracle.index_add(out0, src, index)
    counts = np.bincount(index, minlength=D)
    untouched = counts == 0
    assert untouched.any()
    assert np.array_equal(got[untouched].view(np.uint32), out0[untouched].view(np.uint32))
    exact = out0.astype(np.float64).copy()
    np.add.at(exact, index, src.astype(np.float64))
    absum = np.abs(out0.astype(np.float64))
    np.add.at(absum, index, np.abs(src.astype(np.float64)))
    for d in np.nonzero(~untouched)[0]:
        L = counts[d]
        C = (L + 7) // 8
        depth = (min(L, 8) - 1) + (math.ceil(math.log2(C)) if C > 1 else 0) + 1
        gamma = depth * U / (1 - depth * U)
        assert np.all(np.abs(got[d] - exact[d]) <= gamma * absum[d] + 1e-45)


def test_scatter_reduce_permutation_invariant():
    """Presenting the same (dest, src_id, value) triples in another input order gives the same bits."""
    rng = np.random.default_rng(33)
    D, H, n = 50, 8, 2000
    dest = rng.integers(0, D, n).astype(np.int32)
    sid = rng.permutation(n).astype(np.int32)
    src = mixed_values(rng, n * H).reshape(n, H)
    out0 = mixed_values(rng, D * H).reshape(D, H)
    a = oracle.scatter_reduce(out0, src, dest, sid)
    p = rng.permutation(n)
    b = oracle.scatter_reduce(out0, src[p], dest[p], sid[p])
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_index_add_batch_invariance():
    """A row's bytes depend only on its own ordered contributions."""
    rng = np.random.default_rng(34)
    D, H, n = 40, 8, 600
    index = rng.integers(0, D, n).astype(np.int32)
    src = mixed_values(rng, n * H).reshape(n, H)
    out0 = mixed_values(rng, D * H).reshape(D, H)
    full = oracle.index_add(out0, src, index)
    keep = (index % 3 == 0) | (index == 7)   # drop every contribution of the other rows
    part = oracle.index_add(out0, src[keep], index[keep])
    rows = np.unique(index[keep])
    assert np.array_equal(full[rows].view(np.uint32), part[rows].view(np.uint32))
    # the listed-destination entry point agrees with the full computation
    sub = oracle.index_add(out0, src, index, dests=[3, 7, 0, 39])
    assert np.array_equal(sub.view(np.uint32), full[[3, 7, 0, 39]].view(np.uint32))


# ---------------------------------------------------------------------------
# Combine
# ---------------------------------------------------------------------------
def _expert_major_rows(expert_ids):
    """Row index of each (token, slot) in the expert-major layout, stable by token (brute force)."""
    T, k = expert_ids.shape
    order = sorted(range(T * k), key=lambda a: (expert_ids.flat[a], a))
    row_of = np.empty(T * k, np.int32)
    row_of[order] = np.arange(T * k)
    return row_of.reshape(T, k)


# ---------------------------------------------------------------------------
# Sparse-attention key gradient (contributions formed on the fly)
# ---------------------------------------------------------------------------
def _sparse_case(seed, nq, topk, H, num_keys, bf16):
    rng = np.random.default_rng(seed)
    Qf = rng.standard_normal((nq, H)).astype(F32)
    Q = workloads.bf16_bits(Qf) if bf16 else Qf
    dS = (0.1 * rng.standard_normal((nq, topk))).astype(F32)
    key_idx = np.stack([rng.choice(num_keys, topk, replace=False) for _ in range(nq)]).astype(np.int32)
    dK0 = rng.standard_normal((num_keys, H)).astype(F32)
    return Q, dS, key_idx, dK0


@pytest.mark.parametrize("bf16", [False, True])
def test_sparse_attn_dk_is_index_add_of_rounded_products(bf16):
    """The fused form equals index_add over contributions that numpy forms as
    float32 products (each element one IEEE rounding), source id q*topk + j."""
    Q, dS, key_idx, dK0 = _sparse_case(70 + bf16, 300, 16, 24, 64, bf16)
    nq, topk = key_idx.shape
    Qf = (Q.astype(np.uint32) << 16).view(F32) if bf16 else Q
    q_of = np.arange(nq * topk) // topk
    contrib = dS.reshape(-1, 1) * Qf[q_of]
    assert contrib.dtype == F32
    want = oracle.index_add(dK0, contrib, key_idx.reshape(-1))
    got = oracle.sparse_attn_dk(dK0, Q, dS, key_idx)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    keys = np.array([0, 5, 63, 17], np.int32)
    assert np.array_equal(oracle.sparse_attn_dk(dK0, Q, dS, key_idx, keys=keys).view(np.uint32),
                          want[keys].view(np.uint32))


def test_sparse_attn_dk_closed_forms():
    # one query per key: dK = dK0 + fl32(dS * Q), element by element
    rng = np.random.default_rng(72)
    nq, H = 20, 8
    Q = rng.standard_normal((nq, H)).astype(F32)
    dS = rng.standard_normal((nq, 1)).astype(F32)
    key_idx = np.arange(nq, dtype=np.int32).reshape(nq, 1)[::-1].copy()
    dK0 = rng.standard_normal((nq, H)).astype(F32)
    want = dK0.copy()
    for q in range(nq):
        want[key_idx[q, 0]] = dK0[key_idx[q, 0]] + dS[q, 0] * Q[q]
    got = oracle.sparse_attn_dk(dK0, Q, dS, key_idx)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # the order is by query: three queries select key 0 with rows 1, x, x (x = 3 * 2^-26)
    # and unit score gradients; T(1, x, x) = 1 but T(x, x, 1) = 1 + 2^-23
    x = F32(3 * 2.0 ** -26)
    dS1 = np.ones((3, 1), F32)
    idx = np.zeros((3, 1), np.int32)
    zero = np.zeros((1, 1), F32)
    assert bits32(oracle.sparse_attn_dk(zero, np.array([[1.0], [x], [x]], F32), dS1, idx)[0, 0]) == 0x3F800000
    assert bits32(oracle.sparse_attn_dk(zero, np.array([[x], [x], [1.0]], F32), dS1, idx)[0, 0]) == 0x3F800001
    # keys no query selected are untouched, and an out-of-range key is refused
    with pytest.raises(Exception):
        oracle.sparse_attn_dk(zero, np.ones((1, 1), F32), dS1[:1], np.array([[1]], np.int32))


def test_combine_k2_closed_form():
    inp = workloads.make("tiny_moe_combine")
    row_of = _expert_major_rows(inp.expert_ids)
    got = oracle.combine(inp.rows, row_of, inp.gates)
    T, H = inp.T, inp.H
    want = np.empty((T, H), F32)
    for t in range(T):
        a, b = (0, 1) if row_of[t, 0] < row_of[t, 1] else (1, 0)
        for h in range(H):
            pa = F32(inp.gates[t, a] * inp.rows[row_of[t, a], h])
            pb = F32(inp.gates[t, b] * inp.rows[row_of[t, b], h])
            want[t, h] = F32(pa + pb)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("k", [1, 3, 8, 13, 20, 64])
def test_combine_general_k(k):
    rng = np.random.default_rng(40 + k)
    T, H = 37, 12
    R = T * k + 5
    rows = mixed_values(rng, R * H).reshape(R, H)
    row_of = rng.permutation(R)[:T * k].astype(np.int32).reshape(T, k)
    gates = rng.random((T, k)).astype(F32)
    got = oracle.combine(rows, row_of, gates)
    for t in range(T):
        order = np.argsort(row_of[t], kind="stable")
        for h in range(H):
            prods = [F32(gates[t, j] * rows[row_of[t, j], h]) for j in order]
            want = lr_sum(prods) if k <= 8 else padded_tree(prods)
            assert bits32(got[t, h]) == bits32(want)
    # slot order does not matter: the order is by row index
    p = rng.permutation(k)
    again = oracle.combine(rows, row_of[:, p], gates[:, p])
    assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
    # token subsets give the same bytes as the full batch
    sub = oracle.combine(rows, row_of, gates, tokens=[5, 0, 36])
    assert np.array_equal(sub.view(np.uint32), got[[5, 0, 36]].view(np.uint32))


def test_combine_bf16_rows_and_bound():
    inp = workloads.make("moe_combine", T=64, E=16, H=64)
    row_of = _expert_major_rows(inp.expert_ids)
    got = oracle.combine(inp.rows, row_of, inp.gates)
    y = workloads.bf16_to_f32(inp.rows).astype(np.float64)
    g = inp.gates.astype(np.float64)
    exact = np.einsum("tk,tkh->th", g, y[row_of])
    absum = np.einsum("tk,tkh->th", np.abs(g), np.abs(y[row_of]))
    gamma = 8 * U / (1 - 8 * U)  # one product rounding plus 7 adds
    assert np.all(np.abs(got - exact) <= gamma * absum + 1e-45)


# ---------------------------------------------------------------------------
# Split-K
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 5, 8, 9, 13, 64, 100])
def test_splitk_reduce_tree(S):
    rng = np.random.default_rng(50 + S)
    P = mixed_values(rng, S * 33).reshape(S, 33)
    got = oracle.splitk_reduce(P)
    for e in range(33):
        want = lr_sum(P[:, e]) if S <= 8 else padded_tree(P[:, e])
        assert bits32(got[e]) == bits32(want)


def test_splitk_reference_against_matmul():
    inp = workloads.make("splitk_mhc", K=300, M=40, N=24, splits=7)
    exact, absum = oracle.splitk_reference(inp.X, inp.dY)
    x = workloads.bf16_to_f32(inp.X).astype(np.float64)
    y = workloads.bf16_to_f32(inp.dY).astype(np.float64)
    want = x.T @ y
    want_abs = np.abs(x).T @ np.abs(y)
    assert np.allclose(exact, want, rtol=0, atol=1e-12 * want_abs.max())
    assert np.allclose(absum, want_abs, rtol=1e-13, atol=0)
    P = oracle.splitk_partials(inp.X, inp.dY, 7)
    c = -(-300 // 7)
    for s in range(7):
        lo, hi = s * c, min(300, (s + 1) * c)
        assert np.allclose(P[s], x[lo:hi].T @ y[lo:hi], rtol=0, atol=1e-12 * want_abs.max())
    assert np.allclose(P.sum(axis=0), exact, rtol=0, atol=1e-12 * want_abs.max())


# ---------------------------------------------------------------------------
# Grouped split with private slots; the dispatch permute
# ---------------------------------------------------------------------------
def test_grouped_slots_brute_force():
    """Slots cut each group from its first token; empty groups own no slot."""
    off = [0, 0, 5, 5, 6, 14]
    so, rng = oracle.grouped_slots(off, 3)
    assert so.tolist() == [0, 0, 2, 2, 3, 6]
    assert rng.tolist() == [[0, 3], [3, 5], [5, 6], [6, 9], [9, 12], [12, 14]]
    so, rng = oracle.grouped_slots([0, 4], 4)
    assert so.tolist() == [0, 1] and rng.tolist() == [[0, 4]]


def test_grouped_splitk_reference_and_reduce():
    rng = np.random.default_rng(81)
    K, M, N = 200, 12, 5
    X = workloads.bf16_bits(rng.standard_normal((K, M)).astype(F32))
    dY = workloads.bf16_bits(rng.standard_normal((K, N)).astype(F32))
    off = np.array([0, 37, 37, 120, 200], np.int32)
    x = workloads.bf16_to_f32(X).astype(np.float64)
    y = workloads.bf16_to_f32(dY).astype(np.float64)
    so, ranges = oracle.grouped_slots(off, 16)
    P = oracle.grouped_splitk_partials(X, dY, off, 16)
    for s, (a, b) in enumerate(ranges):
        assert np.allclose(P[s], x[a:b].T @ y[a:b], rtol=0, atol=1e-12)
    # each group's slots sum to that group's matmul
    for g in range(4):
        want = x[off[g]:off[g + 1]].T @ y[off[g]:off[g + 1]]
        assert np.allclose(P[so[g]:so[g + 1]].sum(axis=0), want, rtol=0, atol=1e-11)
    # the reduce: up to 8 slots left to right in float32; an empty group is zero
    Pf = P.astype(F32)
    out = oracle.grouped_splitk_reduce(Pf, so)
    assert np.array_equal(out[1], np.zeros((M, N), F32)) and so[2] == so[1]
    g0 = Pf[so[0]:so[1]]
    assert g0.shape[0] == 3
    assert np.array_equal(out[0].view(np.uint32), ((g0[0] + g0[1]) + g0[2]).view(np.uint32))
    assert np.array_equal(out[3], oracle.splitk_reduce(Pf[so[3]:so[4]]))


def test_permute_rows_brute_force():
    x = np.arange(5 * 3, dtype=np.int32).reshape(5, 3)
    perm = np.array([4, 0, 9, 3, 1, 2, 8, 5, 7, 6], np.int32)   # a permutation of 5 tokens x 2 slots
    out = oracle.permute_rows(x, perm, 2)
    for r in range(10):
        assert out[r].tolist() == x[perm[r] // 2].tolist()


@pytest.mark.parametrize("seed,T,E,k", [(1, 40, 6, 2), (2, 257, 32, 8), (3, 9, 64, 4), (4, 100, 3, 3)])
def test_permute_rows_expert_blocks_hold_tokens_in_ascending_order(seed, T, E, k):
    """The dispatch layout the DeepSeek-V4 book fixes (ch. 9, section 3.2): the
    rows routed to one expert sit together, experts in id order, and within an
    expert's block the tokens are in ascending original token order.  The
    expected layout is built by brute force from the (expert, token) pairs
    sorted with Python's sort; nothing divides a permutation index by k."""
    rng = np.random.default_rng(seed)
    expert_ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, 5)).astype(F32)
    x[:, 0] = np.arange(T)              # a token's row carries its own id
    pairs = sorted((int(expert_ids[t, j]), t) for t in range(T) for j in range(k))
    want = np.stack([x[t] for _, t in pairs])
    perm, seg, _ = oracle.sort_by_dest(expert_ids.reshape(-1), E)
    got = oracle.permute_rows(x, perm, k)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # block by block: expert e owns rows [seg[e], seg[e+1]), exactly its tokens, ascending
    for e in range(E):
        block = got[seg[e]:seg[e + 1], 0].astype(np.int64)
        tokens = sorted(t for t in range(T) if e in expert_ids[t])
        assert block.tolist() == tokens


# ---------------------------------------------------------------------------
# Decode attention (by definition)
# ---------------------------------------------------------------------------
def test_decode_attention_against_torch_sdpa_and_closed_forms():
    import torch
    rng = np.random.default_rng(90)
    B, Hq, Hkv, D, Lmax = 3, 8, 2, 16, 40
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Lmax, Hkv, D))
    vc = rng.standard_normal((B, Lmax, Hkv, D))
    lens = np.array([40, 1, 17], np.int32)
    scale = 0.25
    out, A = oracle.decode_attention(q, kc, vc, lens, scale)
    for b in range(B):
        L = lens[b]
        kk = torch.from_numpy(kc[b, :L]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)   # [Hq, L, D]
        vv = torch.from_numpy(vc[b, :L]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        qq = torch.from_numpy(q[b]).unsqueeze(1)                                          # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)[:, 0]
        assert np.allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)
    # one cached token: the value row itself; equal scores: the mean of the values
    assert np.allclose(out[1], vc[1, 0].repeat(Hq // Hkv, axis=0), rtol=0, atol=1e-15)
    z, _ = oracle.decode_attention(np.zeros((1, 2, D)), kc[:1], vc[:1], np.array([5], np.int32), 1.0)
    assert np.allclose(z[0, 0], vc[0, :5, 0].mean(axis=0), rtol=0, atol=1e-14)
    # |out| <= A, and an empty sequence gives zeros
    assert np.all(np.abs(out) <= A + 1e-15)
    e, _ = oracle.decode_attention(q[:1], kc[:1], vc[:1], np.array([0], np.int32), scale)
    assert np.all(e == 0)
    # hand example: scores ln 3 and 0 give weights 3/4 and 1/4
    qh = np.array([[[1.0, 0.0]]])
    kh = np.array([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    vh = np.array([[[[4.0, -8.0]], [[8.0, 16.0]]]])
    oh, _ = oracle.decode_attention(qh, kh, vh, np.array([2], np.int32), float(np.log(3.0)))
    assert np.allclose(oh[0, 0], [5.0, -2.0], rtol=0, atol=1e-14)
    # key/value pairs in any order give the same result (a softmax-weighted average)
    perm = rng.permutation(40)
    o2, _ = oracle.decode_attention(q[:1], kc[:1, perm], vc[:1, perm], np.array([40], np.int32), scale)
    assert np.allclose(o2[0], out[0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Fingerprint
# ---------------------------------------------------------------------------
def test_splitmix64_published_outputs(golden_dir):
    g = read_golden(os.path.join(golden_dir, "splitmix64_seed0.txt"))
    gamma = int(g["gamma"], 16)
    for i in (1, 2, 3):
        assert oracle.splitmix64_mix((i * gamma) % 2 ** 64) == int(g[str(i)], 16)


def test_fingerprint_of_zero_bytes_is_the_splitmix64_sequence(golden_dir):
    """All-zero words turn every term into a published SplitMix64 output, so the
    fingerprint of 8*w zero bytes is mix(8*w) plus the first w outputs."""
    g = read_golden(os.path.join(golden_dir, "splitmix64_seed0.txt"))
    outs = [int(g[str(i)], 16) for i in (1, 2, 3)]
    for w in (1, 2, 3):
        want = (oracle.splitmix64_mix(8 * w) + sum(outs[:w])) % 2 ** 64
        assert oracle.fingerprint(np.zeros(8 * w, np.uint8)) == want


def test_fingerprint_of_chosen_words_hits_published_outputs(golden_dir):
    """A data word w_i = (i+1)*gamma XOR (j+1)*gamma turns term i into the
    published output j+1.  Words are assembled little-endian and a short last
    word is zero-padded, so the bytes below (and a 3-byte zero tail) fix the
    XOR, the word index, the byte order and the padding against published
    values."""
    g = read_golden(os.path.join(golden_dir, "splitmix64_seed0.txt"))
    gamma = int(g["gamma"], 16)
    outs = {i: int(g[str(i)], 16) for i in (1, 2, 3)}
    M = 2 ** 64

    def words_to_bytes(ws):
        return np.frombuffer(b"".join(int(w).to_bytes(8, "little") for w in ws), np.uint8).copy()

    for targets in ([2], [3], [1, 3], [3, 1], [2, 2, 2], [3, 1, 2]):
        ws = [((i + 1) * gamma % M) ^ (j * gamma % M) for i, j in enumerate(targets)]
        data = words_to_bytes(ws)
        want = (oracle.splitmix64_mix(len(data)) + sum(outs[j] for j in targets)) % M
        assert oracle.fingerprint(data) == want, targets
        # a zero tail shorter than a word is padded into one more zero word
        i = len(targets)
        tail = np.concatenate([data, np.zeros(3, np.uint8)])
        want_tail = (oracle.splitmix64_mix(len(tail)) + sum(outs[j] for j in targets)
                     + oracle.splitmix64_mix((i + 1) * gamma % M)) % M
        assert oracle.fingerprint(tail) == want_tail, targets


def test_fingerprint_properties():
    rng = np.random.default_rng(60)
    data = rng.integers(0, 256, 1003, dtype=np.uint8)
    h = oracle.fingerprint(data)
    assert oracle.fingerprint(data) == h
    for pos in (0, 7, 8, 500, 1002):
        for bit in (0, 7):
            d2 = data.copy()
            d2[pos] ^= 1 << bit
            assert oracle.fingerprint(d2) != h
    # +0.0 and -0.0 differ; swapping two distinct words is seen; length is part of the hash
    assert oracle.fingerprint(np.array([0.0], F32)) != oracle.fingerprint(np.array([-0.0], F32))
    w = rng.integers(0, 2 ** 63, 16, dtype=np.int64)
    w2 = w.copy()
    w2[[3, 9]] = w2[[9, 3]]
    assert oracle.fingerprint(w) != oracle.fingerprint(w2)
    assert oracle.fingerprint(np.zeros(1, np.uint8)) != oracle.fingerprint(np.zeros(2, np.uint8))
    assert oracle.fingerprint(np.zeros(0, np.uint8)) == oracle.splitmix64_mix(0) == 0


# ---------------------------------------------------------------------------
# Generators (shared inputs): bf16 rounding against a library routine
# ---------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(70)
    f = np.concatenate([rng.standard_normal(100000).astype(F32),
                        mixed_values(rng, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], F32)])
    ours = workloads.bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generators_are_seeded():
    a = workloads.make("tiny_moe_combine")
    b = workloads.make("tiny_moe_combine")
    assert np.array_equal(a.rows, b.rows) and np.array_equal(a.gates, b.gates)
    assert np.array_equal(a.expert_ids, b.expert_ids)
    for t in range(a.T):
        assert len(set(a.expert_ids[t])) == a.k
    assert np.allclose(a.gates.sum(axis=1), 1.0, atol=1e-6)


# ---------------------------------------------------------------------------
# Host threads divide the row loop only
# ---------------------------------------------------------------------------
def test_oracle_threads_do_not_change_bits():
    """The oracle's multi-threaded form hands contiguous destination (or token)
    ranges to threads; every row is computed from its own inputs, so the bytes
    equal the single-threaded result for any thread count."""
    rng = np.random.default_rng(95)
    D, H, n = 300, 16, 6000
    index = np.minimum(rng.zipf(1.2, n) - 1, D - 1).astype(np.int32)
    src = workloads.bf16_bits(mixed_values(rng, n * H).reshape(n, H))
    out0 = mixed_values(rng, D * H).reshape(D, H)
    one = oracle.index_add(out0, src, index)
    for t in (2, 3, 8, 64):
        assert np.array_equal(oracle.index_add(out0, src, index, threads=t).view(np.uint32), one.view(np.uint32))
    nq, topk, K = 200, 16, 97
    key_idx = np.stack([rng.choice(K, topk, replace=False) for _ in range(nq)]).astype(np.int32)
    Q = workloads.bf16_bits(rng.standard_normal((nq, H)).astype(F32))
    dS = mixed_values(rng, nq * topk).reshape(nq, topk)
    dk0 = mixed_values(rng, K * H).reshape(K, H)
    one = oracle.sparse_attn_dk(dk0, Q, dS, key_idx)
    for t in (2, 7):
        assert np.array_equal(oracle.sparse_attn_dk(dk0, Q, dS, key_idx, threads=t).view(np.uint32),
                              one.view(np.uint32))
    inp = workloads.make("moe_combine", T=64, E=16, H=64)
    row_of = _expert_major_rows(inp.expert_ids)
    one = oracle.combine(inp.rows, row_of, inp.gates)
    for t in (2, 5, 16):
        assert np.array_equal(oracle.combine(inp.rows, row_of, inp.gates, threads=t).view(np.uint32),
                              one.view(np.uint32))
