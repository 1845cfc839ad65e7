"""Seeded random sweeps: many small shapes per entry point, each under random
launch parameters, compared with the oracle (bit for bit, or to the split-K
tolerance).  Sizes stay small so that the oracle takes milliseconds."""
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


def _launch(dr, rng):
    dr.dr_set_launch_params(grid_blocks=int(rng.choice([0, 1, 5, 64, 700])),
                            tile_chunks_log2=int(rng.integers(3, 8)),
                            sort_tile_log2=int(rng.choice([0, 8, 9, 10, 11, 12, 13])),
                            chunks_in_flight=int(rng.integers(1, 3)))


def _dest(rng, n, D):
    kind = rng.integers(0, 3)
    if kind == 0:
        return rng.integers(0, D, n).astype(np.int32)
    if kind == 1:
        return np.minimum(rng.zipf(1.3, n) - 1, D - 1).astype(np.int32)
    return np.full(n, rng.integers(0, D), np.int32)  # one hot destination


def test_random_sort_and_index_add(dr):
    rng = np.random.default_rng(2024)
    for case in range(24):
        n = int(rng.choice([0, 1, 7, 100, 1000, 5000, 20000]))
        D = int(rng.choice([1, 3, 64, 300, 4096, 70000]))
        bf16 = bool(rng.integers(0, 2))
        H = int(rng.choice([8, 16, 24, 136, 520])) if bf16 else int(rng.choice([4, 12, 128, 260]))
        dest = _dest(rng, n, D)
        say(f"random index_add case {case}: n={n} D={D} H={H} bf16={bf16}")
        _launch(dr, rng)
        try:
            srcf = rng.standard_normal((n, H)).astype(np.float32)
            src_h = workloads.bf16_bits(srcf) if bf16 else srcf
            out0 = rng.standard_normal((D, H)).astype(np.float32)
            out = dev(out0)
            _, ws = dr.dr_index_add(out, dev_bf16(src_h) if bf16 else dev(src_h), dev(dest))
            dr.dr_workspace_status(ws)
            perm, seg, inv = dr.dr_sort_by_dest(dev(dest), D)
        finally:
            dr.dr_set_launch_params(reset=True)
        assert_bits_equal(host(out), oracle.index_add(out0, src_h, dest), f"index_add case {case}")
        wp, ws_, wi = oracle.sort_by_dest(dest, D)
        assert np.array_equal(host(perm), wp) and np.array_equal(host(seg), ws_) and np.array_equal(host(inv), wi)


def test_random_combine(dr):
    rng = np.random.default_rng(2025)
    for case in range(16):
        T = int(rng.choice([1, 5, 100, 700]))
        E = int(rng.choice([4, 16, 256]))
        k = int(rng.integers(1, min(E, 20) + 1))
        bf16 = bool(rng.integers(0, 2))
        H = int(rng.choice([8, 64, 520, 1024])) if bf16 else int(rng.choice([4, 36, 256]))
        say(f"random combine case {case}: T={T} E={E} k={k} H={H} bf16={bf16}")
        inp = workloads.moe_inputs(3000 + case, T, E, k, H, "bf16" if bf16 else "f32", zipf_bias_s=1.2)
        _, _, inv = dr.dr_sort_by_dest(dev(inp.expert_ids.reshape(-1)), E)
        row_of = inv.view(T, k)
        rows = dev_bf16(inp.rows) if bf16 else dev(inp.rows)
        out, h = dr.dr_combine_fingerprinted(rows, row_of, dev(inp.gates))
        want = oracle.combine(inp.rows, host(row_of), inp.gates)
        assert_bits_equal(host(out), want, f"combine case {case}")
        assert int(h.item()) & ((1 << 64) - 1) == oracle.fingerprint(want)


def test_random_sparse_attn_dk_and_grouped(dr):
    rng = np.random.default_rng(2026)
    for case in range(10):
        nq = int(rng.choice([1, 9, 200, 800]))
        K = int(rng.choice([16, 100, 1000]))
        topk = int(rng.integers(1, min(K, 64) + 1))
        H = int(rng.choice([8, 64, 128]))
        say(f"random sparse_attn_dk case {case}: nq={nq} keys={K} topk={topk} H={H}")
        inp = workloads.sparse_attn_dk_inputs(4000 + case, nq, K, topk, H)
        _launch(dr, rng)
        try:
            dK = dev(inp.dK0)
            dr.dr_sparse_attn_dk(dK, dev_bf16(inp.Q), dev(inp.dS), dev(inp.key_idx))
        finally:
            dr.dr_set_launch_params(reset=True)
        assert_bits_equal(host(dK), oracle.sparse_attn_dk(inp.dK0, inp.Q, inp.dS, inp.key_idx), f"dK case {case}")
    for case in range(8):
        Kt = int(rng.choice([50, 700, 3000]))
        M = int(rng.choice([1, 64, 100, 256]))
        N = int(rng.choice([1, 8, 24, 40]))
        G = int(rng.integers(1, 12))
        cuts = np.sort(rng.integers(0, Kt + 1, G - 1))
        off = np.concatenate([[0], cuts, [Kt]]).astype(np.int32)
        split = int(rng.choice([16, 100, 256, 1000]))
        say(f"random grouped case {case}: K={Kt} M={M} N={N} groups={G} split={split}")
        inp = workloads.splitk_inputs(5000 + case, Kt, M, N, 1)
        P, so, ws = dr.dr_grouped_splitk_gemm_tn(dev_bf16(inp.X), dev_bf16(inp.dY), dev(off), split)
        dr.dr_workspace_status(ws)
        want_so, _ = oracle.grouped_slots(off, split)
        assert np.array_equal(host(so), want_so)
        Ph = host(P)[:int(want_so[-1])]
        dW = dr.dr_grouped_splitk_reduce(P, so, ws)
        assert_bits_equal(host(dW), oracle.grouped_splitk_reduce(Ph, want_so), f"grouped reduce case {case}")
        for g in range(G):
            e, A = oracle.splitk_reference(inp.X[off[g]:off[g + 1]], inp.dY[off[g]:off[g + 1]])
            assert np.all(np.abs(host(dW)[g] - e) <= 1e-4 * A + 1e-30), (case, g)


def test_random_decode_attention(dr):
    """Random batches, head groupings, lengths, chunk sizes and cache layouts against the oracle within the
    derived bound; each batch's first sequence alone must give the same bits."""
    from tests.test_gpu_decode import check_against_oracle
    rng = np.random.default_rng(2027)
    for case in range(12):
        B = int(rng.integers(1, 7))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.integers(1, 5))
        Lmax = int(rng.integers(1, 1500))
        lens = rng.integers(0, Lmax + 1, B)
        if rng.random() < 0.3:
            lens[0] = Lmax
        chunk = int(rng.choice([64, 128, 192, 512, 1024, 1 << 20]))
        head_major = bool(rng.integers(0, 2))
        say(f"decode random {case}: B={B} G={G} Hkv={Hkv} Lmax={Lmax} lens={lens.tolist()} chunk={chunk} "
            f"head_major={head_major}")
        inp = workloads.decode_inputs(3000 + case, B, Lmax, G * Hkv, Hkv, 128, lens)
        q, k, v, L = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev(inp.lens)
        if head_major:
            k, v = k.permute(0, 2, 1, 3).contiguous(), v.permute(0, 2, 1, 3).contiguous()
        got = host(dr.dr_decode_attention(q, k, v, L, inp.scale, chunk, head_major=head_major))
        check_against_oracle(inp, got, chunk)
        one = host(dr.dr_decode_attention(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(),
                                          L[:1].contiguous(), inp.scale, chunk, head_major=head_major))
        assert_bits_equal(one[0], got[0], f"case {case}: first sequence alone")
