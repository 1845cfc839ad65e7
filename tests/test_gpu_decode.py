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


def tolerance(inp, A, kv_chunk, b, h):
    """First-order bound on |fp32 result - exact| for output row (b, h).

    A score is a sum of 128 exact bf16 products rounded in fp32, then scaled:
    its error is at most 129 u S with S = scale * sum_i |q_i k_i|, which moves
    the normalised weights by a relative 2 * 129 u S (after the log2(e) and
    ln 2 factors cancel); rounding the exponent t - m adds u |t - m| <= 2 u S.
    Every other step is a sum of non-negative weights or of weight * value
    products along a chain of at most d roundings (d = 5 kv_chunk / 64 in a
    lane, 6 in the butterfly and the wave merge, one per chunk in the merge,
    one for the division), each within 2 u of the hardware exp2 factors.
    Everything is relative to A = sum_j w_j |v_j| >= |out|."""
    L = int(inp.lens[b])
    if L == 0:
        return np.zeros(inp.D)
    g = inp.Hq // inp.Hkv
    q = workloads.bf16_to_f32(inp.q[b, h]).astype(np.float64)
    k = workloads.bf16_to_f32(inp.k[b, :L, h // g]).astype(np.float64)
    S = inp.scale * float((np.abs(k) @ np.abs(q)).max())
    nc = -(-L // kv_chunk)
    d = 5 * min(kv_chunk, L) // 64 + 5 + 6 + nc + 1
    return A[b, h] * U * (270.0 * S + 4.0 * d + 32.0)


def check_against_oracle(inp, got, kv_chunk, rows=None):
    want, A = oracle.decode_attention(inp.q, inp.k, inp.v, inp.lens, inp.scale)
    assert np.all(np.isfinite(got)), "NaN cache rows past a sequence's length reached the output"
    rows = rows if rows is not None else [(b, h) for b in range(inp.B) for h in range(inp.Hq)]
    worst = 0.0
    for b, h in rows:
        tol = tolerance(inp, A, kv_chunk, b, h)
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
