"""Decode attention with a fixed KV partition: parity with the fp64 oracle
within a bound derived from the fp32 arithmetic, and bitwise invariance of a
sequence's output to the batch around it (DeepSeek-V4 book ch. 9, section
2.1).  All calls go through the C ABI (the ctypes binding)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_bits_equal, dev, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def dr():
    require_gpu()
    import bitwise_deterministic_fp32_amd as m
    m.dr_set_launch_params(reset=True)
    return m


def to_dev(inp):
    return dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev(inp.lens)


def tolerance(inp, want, A, kv_chunk, b, h):
    """First-order bound on |fp32 result - exact|, per column of output row (b, h).

    Weights.  With s_j the exact scores and w_j = softmax(s)_j, an fp32
    evaluation sees weights w_j e^{d_j} / sum_k w_k e^{d_k} for some errors d_j,
    so to first order out' - out = sum_j w_j d_j (v_j - out), bounded per column
    by sum_j w_j |d_j| |v_jc - out_c|.  A score is a sum of 128 exact bf16
    products rounded in fp32 (at most 129 u S_j, S_j = scale * sum_i |q_i k_ji|),
    then scaled by a rounded scale * log2(e) (2 u S_j, the log2(e) and ln 2
    factors cancel); the exponent t_j - m is rounded (u (S_j + S_max)); the
    running-maximum rescales inside a chunk and the chunk factors of the merge
    are exponents of rounded differences of maxima (2 u S_max each).  So
    |d_j| <= u (132 S_j + 6 S_max) =: d_j.  Exactly, out' - out =
    (1/Z) sum_j w_j (d_j + r(d_j)) (v_j - out) with Z = sum_k w_k e^{d_k} and
    r(x) = e^x - 1 - x (the terms constant in j cancel, since
    sum_j w_j (v_j - out) = 0), which gives the factor `second` below.

    Sums.  Every other step is a sum of non-negative weights or of weight *
    value products along a chain of at most d roundings (d = 5 kv_chunk / 64 in
    a lane, 6 in the butterfly and the wave merge, one per chunk in the merge,
    one for the division), each within 2 u of the hardware exp2 factors:
    u (4 d + 32) A_c with A_c = sum_j w_j |v_jc| >= |out_c|.

    Keeping the per-token and per-column terms (rather than the largest S_j and
    |v_j| + |out|) makes the bound tight enough that one dropped or doubled
    cached token of average weight falls outside it at 16,384 tokens
    (test_decode_bound_sees_a_dropped_or_doubled_token)."""
    L = int(inp.lens[b])
    if L == 0:
        return np.zeros(inp.D)
    g = inp.Hq // inp.Hkv
    q = workloads.bf16_to_f32(inp.q[b, h]).astype(np.float64)
    k = workloads.bf16_to_f32(inp.k[b, :L, h // g]).astype(np.float64)
    v = workloads.bf16_to_f32(inp.v[b, :L, h // g]).astype(np.float64)
    s = inp.scale * (k @ q)
    w = np.exp(s - s.max())
    w /= w.sum()
    S = inp.scale * (np.abs(k) @ np.abs(q))
    d_j = U * (132.0 * S + 6.0 * S.max())
    D, d_min = float(d_j.max()), float(d_j.min())
    # exact remainder of the expansion: e^x = 1 + x + r(x), |r(x)| <= x^2 e^|x| / 2, and the normaliser 1/Z <= e^D
    second = np.exp(D) * (1.0 + 0.5 * D * D * np.exp(D) / d_min)
    score_term = second * ((w * d_j) @ np.abs(v - want[b, h]))
    nc = -(-L // kv_chunk)
    d = 5 * min(kv_chunk, L) // 64 + 5 + 6 + nc + 1
    return score_term + A[b, h] * U * (4.0 * d + 32.0)


def worst_ratio(inp, got, kv_chunk, rows=None):
    """max over the rows and columns of |got - exact| / bound (<= 1 passes)."""
    want, A = oracle.decode_attention(inp.q, inp.k, inp.v, inp.lens, inp.scale)
    rows = rows if rows is not None else [(b, h) for b in range(inp.B) for h in range(inp.Hq)]
    worst = 0.0
    for b, h in rows:
        tol = tolerance(inp, want, A, kv_chunk, b, h)
        err = np.abs(got[b, h].astype(np.float64) - want[b, h])
        if int(inp.lens[b]) == 0:
            worst = max(worst, 0.0 if np.all(got[b, h] == 0) else np.inf)
            continue
        worst = max(worst, float((err / tol).max()))
    return worst


def check_against_oracle(inp, got, kv_chunk, rows=None):
    want, A = oracle.decode_attention(inp.q, inp.k, inp.v, inp.lens, inp.scale)
    assert np.all(np.isfinite(got)), "NaN cache rows past a sequence's length reached the output"
    rows = rows if rows is not None else [(b, h) for b in range(inp.B) for h in range(inp.Hq)]
    worst = 0.0
    for b, h in rows:
        tol = tolerance(inp, want, A, kv_chunk, b, h)
        err = np.abs(got[b, h].astype(np.float64) - want[b, h])
        assert np.all(err <= tol), (b, h, float(err.max()), float(tol.max()))
        if int(inp.lens[b]) == 0:
            assert np.all(got[b, h] == 0)
        nz = A[b, h] > 0
        if nz.any():
            worst = max(worst, float((err[nz] / A[b, h][nz]).max()))
    return worst


DECODE_CASES = [
    # (B, Lmax, Hq, Hkv, lens, kv_chunk)
    (4, 300, 32, 8, None, 64),                       # several chunks, ragged ends
    (3, 1000, 8, 8, [1000, 999, 1], 256),            # one query head per KV head; length = capacity
    (2, 700, 4, 2, [700, 333], 1 << 20),             # one chunk: the whole sequence in one workgroup
    (5, 2100, 64, 8, [0, 1, 16, 64, 2100], 512),     # empty sequence, block-aligned lengths
    (2, 520, 16, 1, [520, 17], 128),                 # sixteen query heads on one KV head
    (2, 5000, 32, 8, [4999, 5000], 512),             # ten chunks
    (3, 900, 16, 4, [63, 65, 900], 64),              # lengths around one 64-token round
]


def head_major(t):
    return t.permute(0, 2, 1, 3).contiguous()


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,lens,kv_chunk", DECODE_CASES)
def test_decode_attention_matches_oracle(dr, B, Lmax, Hq, Hkv, lens, kv_chunk):
    say(f"decode B={B} Lmax={Lmax} Hq={Hq} Hkv={Hkv} lens={lens} chunk={kv_chunk}")
    inp = workloads.decode_inputs(7 + B + Lmax, B, Lmax, Hq, Hkv, 128, lens)
    q, k, v, L = to_dev(inp)
    got = host(dr.dr_decode_attention(q, k, v, L, inp.scale, kv_chunk))
    worst = check_against_oracle(inp, got, kv_chunk)
    say(f"  worst |err| / A = {worst:.3g}")
    # the head-major cache layout gives the same bits
    hm = host(dr.dr_decode_attention(q, head_major(k), head_major(v), L, inp.scale, kv_chunk, head_major=True))
    assert_bits_equal(hm, got, "head-major layout")


def test_decode_attention_is_batch_invariant(dr):
    """A sequence's output bits do not depend on the other sequences, its
    position, the batch size or the cache capacity."""
    inp = workloads.decode_inputs(31, 6, 1500, 32, 8, 128, [1500, 7, 640, 1, 1111, 0])
    q, k, v, L = to_dev(inp)
    chunk = 256
    say("decode batch invariance: full batch")
    full = host(dr.dr_decode_attention(q, k, v, L, inp.scale, chunk))
    for b in range(inp.B):
        say(f"  sequence {b} alone")
        one = host(dr.dr_decode_attention(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(),
                                          L[b:b + 1].contiguous(), inp.scale, chunk))
        assert_bits_equal(one[0], full[b], f"sequence {b} alone")
    say("  reversed batch")
    rev = host(dr.dr_decode_attention(q.flip(0).contiguous(), k.flip(0).contiguous(), v.flip(0).contiguous(),
                                      L.flip(0).contiguous(), inp.scale, chunk))
    assert_bits_equal(rev[::-1], full, "reversed batch")
    say("  larger cache capacity")
    pad = torch.full((inp.B, 2500 - inp.Lmax, inp.Hkv, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    big = host(dr.dr_decode_attention(q, torch.cat([k, pad], 1).contiguous(), torch.cat([v, pad], 1).contiguous(),
                                      L, inp.scale, chunk))
    assert_bits_equal(big, full, "capacity 2500")
    say("  head-major layout, larger capacity")
    bigh = host(dr.dr_decode_attention(q, head_major(torch.cat([k, pad], 1)), head_major(torch.cat([v, pad], 1)), L,
                                       inp.scale, chunk, head_major=True))
    assert_bits_equal(bigh, full, "head-major, capacity 2500")
    say("  repeated runs")
    h0 = dr.fingerprint_value(torch.from_numpy(full).cuda())
    for _ in range(3):
        again = dr.dr_decode_attention(q, k, v, L, inp.scale, chunk)
        assert dr.fingerprint_value(again) == h0


def test_occupancy_chosen_split_moves_the_bits(dr):
    """The deliberately batch-variant baseline: a split-KV heuristic picks a
    different partition for a different batch size, and the same sequence's
    output bits change with it."""
    inp = workloads.decode_inputs(32, 64, 4096, 32, 8, 128, [4096] * 64)
    q, k, v, L = to_dev(inp)
    c_small = dr.dr_decode_attention_occupancy_chunk(1, 8, 4096)
    c_large = dr.dr_decode_attention_occupancy_chunk(64, 8, 4096)
    say(f"decode occupancy chunks: batch 1 -> {c_small}, batch 64 -> {c_large}")
    assert c_small != c_large
    alone = host(dr.dr_decode_attention(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(),
                                        L[:1].contiguous(), inp.scale, c_small))
    batched = host(dr.dr_decode_attention(q, k, v, L, inp.scale, c_large))
    assert not np.array_equal(alone[0].view(np.uint32), batched[0].view(np.uint32))
    # the fixed partition gives one answer for both, and both answers are within the bound
    fixed_alone = host(dr.dr_decode_attention(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(),
                                              L[:1].contiguous(), inp.scale, 512))
    fixed_batched = host(dr.dr_decode_attention(q, k, v, L, inp.scale, 512))
    assert_bits_equal(fixed_alone[0], fixed_batched[0], "fixed partition")
    sub = dataclasses.replace(inp, B=1, q=inp.q[:1], k=inp.k[:1], v=inp.v[:1], lens=inp.lens[:1])
    check_against_oracle(sub, alone, c_small)
    check_against_oracle(sub, fixed_alone, 512)


def test_decode_attention_bad_length_fails_closed(dr):
    inp = workloads.decode_inputs(33, 3, 1000, 8, 2, 128, [5, 3, 9])
    q, k, v, _ = to_dev(inp)
    lens = dev(np.array([5, -1, 1001], np.int32))
    out = torch.full((3, 8, 128), 7.0, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("decode bad lengths")
    dr.dr_decode_attention(q, k, v, lens, inp.scale, 64, out=out, dev_status=status)
    with pytest.raises(dr.DetReduceError):
        dr.dr_read_status(status)
    got = host(out)
    assert np.all(got[1:] == 7.0)
    inp.lens = np.array([5, 0, 0], np.int32)
    check_against_oracle(inp, got, 64, rows=[(0, h) for h in range(8)])


def test_decode_attention_peaked_and_flat_weights(dr):
    """Scores scaled up 16x (weights close to one-hot) and identical keys (uniform weights: the output is the
    mean of the value rows) stay within the bound."""
    inp = workloads.decode_inputs(34, 3, 900, 16, 4, 128, [900, 333, 64])
    inp.q = workloads.bf16_bits(workloads.bf16_to_f32(inp.q) * 16.0)  # exact: a power of two
    q, k, v, L = to_dev(inp)
    say("decode peaked weights")
    got = host(dr.dr_decode_attention(q, k, v, L, inp.scale, 128))
    check_against_oracle(inp, got, 128)
    say("decode flat weights")
    flat = dataclasses.replace(inp, k=np.broadcast_to(inp.k[:, :1], inp.k.shape).copy())
    for b in range(flat.B):
        flat.k[b, flat.lens[b]:] = workloads.BF16_NAN
    got = host(dr.dr_decode_attention(q, dev_bf16(flat.k), v, L, inp.scale, 128))
    check_against_oracle(flat, got, 128)
    want_mean = workloads.bf16_to_f32(inp.v[0, :900]).astype(np.float64).mean(axis=0)  # [Hkv, D]
    assert np.allclose(got[0], np.repeat(want_mean, 4, axis=0), rtol=0, atol=1e-5)


def test_decode_bound_sees_a_dropped_or_doubled_token(dr):
    """Negative control of the decode check at full length: the GPU output of a
    16,384-token sequence passes against the oracle, and fails against the
    oracle recomputed with one cached token dropped or doubled.  The tokens are
    taken near the start, a chunk boundary, the middle and the end, each the
    one among 64 neighbours whose weight is closest to the average weight 1/L
    (for the query head that weighs it most): a token of far less than average
    weight moves the output by less than rounding, and no tolerance can see it."""
    L, chunk = 16384, 512
    inp = workloads.decode_inputs(35, 1, L, 32, 8, 128, [L])
    q, k, v, lens = to_dev(inp)
    say("decode negative control: 16,384 tokens")
    got = host(dr.dr_decode_attention(q, k, v, lens, inp.scale, chunk))
    assert worst_ratio(inp, got, chunk) <= 1.0
    g = inp.Hq // inp.Hkv
    kv_head = 3
    heads = list(range(kv_head * g, kv_head * g + g))
    qf = workloads.bf16_to_f32(inp.q[0, heads]).astype(np.float64)                # [g, D]
    kf = workloads.bf16_to_f32(inp.k[0, :, kv_head]).astype(np.float64)           # [L, D]
    s = inp.scale * (kf @ qf.T)                                                    # [L, g]
    w = np.exp(s - s.max(axis=0))
    w /= w.sum(axis=0)
    rows = [(0, h) for h in heads]
    for start in (0, chunk - 32, L // 2, L - 64):
        j = start + int(np.argmin(np.abs(w[start:start + 64].max(axis=1) * L - 1.0)))
        for kind in ("dropped", "doubled"):
            if kind == "dropped":
                kk = np.delete(inp.k, j, axis=1)
                vv = np.delete(inp.v, j, axis=1)
            else:
                kk = np.insert(inp.k, j, inp.k[:, j], axis=1)
                vv = np.insert(inp.v, j, inp.v[:, j], axis=1)
            bad = dataclasses.replace(inp, Lmax=kk.shape[1], k=kk, v=vv,
                                      lens=np.array([kk.shape[1]], np.int32))
            ratio = worst_ratio(bad, got, chunk, rows=rows)
            say(f"  token {j} {kind} (weight x L = {float(w[j].max()) * L:.2f}): worst |err| / bound = {ratio:.2f}")
            assert ratio > 1.0, (j, kind, ratio)
