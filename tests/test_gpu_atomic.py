"""The atomicAdd baselines: what the deterministic paths replace.

The pages' default path adds every contribution with a hardware atomic (the
Megatron-LM determinism reference, section 3.1, op catalog: `scatter_add_` and
`index_add_` in the MoE unpermute and the embedding backward; DeepSeek-V4 book
ch. 9, glossary, "atomicAdd").  Its sum is correct only to rounding, and its
last bits follow the arrival order.  So each baseline is checked two ways:

- its result lies within the fp64 error bound of a sum taken in SOME order,
  against the exact value and against the oracle's ordered result;
- replays change its bits (the negative control of the reference's harness,
  section 4.4: the strict comparison must be able to see an order change).

All calls go through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import dev, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def gamma(k: int) -> float:
    return k * U / (1 - k * U)


@pytest.fixture(scope="module")
def dr():
    require_gpu()
    import bitwise_deterministic_fp32_amd as m
    m.dr_set_launch_params(reset=True)
    return m


def replay_fingerprints(dr, fn, replays=6):
    return [dr.fingerprint_value(fn()) for _ in range(replays)]


def test_combine_atomic_within_bound_of_exact_and_oracle(dr):
    """k atomic adds of rounded products into a zeroed row: a sum of k rounded
    terms in some order, so |atomic - exact| <= gamma_k * sum |g y| per element."""
    inp = workloads.moe_inputs(61, 1024, 64, 8, 1024, "bf16", zipf_bias_s=1.2)
    say("combine_atomic: 1024 tokens x top-8, hidden 1024")
    _, _, inv = dr.dr_sort_by_dest(dev(inp.expert_ids.reshape(-1)), inp.E)
    row_of = host(inv).reshape(inp.T, inp.k)
    rows, gates = dev_bf16(inp.rows), dev(inp.gates)
    out = torch.zeros(inp.T, inp.H, dtype=torch.float32, device="cuda")
    dr.dr_combine_atomic(rows, inv.view(inp.T, inp.k), gates, out=out)
    got = host(out).astype(np.float64)
    y = workloads.bf16_to_f32(inp.rows).astype(np.float64)[row_of]          # [T, k, H]
    g = inp.gates.astype(np.float64)[:, :, None]
    exact = (g * y).sum(axis=1)
    absum = np.abs(g * y).sum(axis=1)
    tol = gamma(inp.k) * absum
    assert np.all(np.abs(got - exact) <= tol)
    want = oracle.combine(inp.rows, row_of, inp.gates).astype(np.float64)
    assert np.all(np.abs(got - want) <= 2 * tol)
    say(f"  max |atomic - oracle| / sum|gy| = {float((np.abs(got - want) / np.maximum(absum, 1e-300)).max()):.3g}")


def test_index_add_atomic_within_bound_of_exact_and_oracle(dr):
    """L atomic adds into a preset row: the old value and L rows summed in some
    order, so |atomic - exact| <= gamma_L * (|old| + sum |v|); untouched rows
    keep their bits."""
    inp = workloads.sparse_attn_inputs(62, Q=512, K=4096, S=64, H=128)
    say("index_add_atomic: 32,768 rows into 4096 keys")
    out = dev(inp.out0)
    dr.dr_index_add_atomic(out, dev_bf16(inp.src), dev(inp.index))
    got = host(out)
    counts = np.bincount(inp.index, minlength=inp.D)
    untouched = counts == 0
    assert np.array_equal(got[untouched].view(np.uint32), inp.out0[untouched].view(np.uint32))
    v = workloads.bf16_to_f32(inp.src).astype(np.float64)
    exact = inp.out0.astype(np.float64)
    np.add.at(exact, inp.index, v)
    absum = np.abs(inp.out0.astype(np.float64))
    np.add.at(absum, inp.index, np.abs(v))
    tol = np.array([gamma(max(int(c), 1)) for c in counts])[:, None] * absum
    assert np.all(np.abs(got.astype(np.float64) - exact) <= tol)
    want = oracle.index_add(inp.out0, inp.src, inp.index).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - want) <= 2 * tol)


def test_splitk_atomic_within_tolerance_of_exact(dr):
    """Each split's tile added atomically into a zeroed dW: within the
    1e-4 * sum |x y| tolerance of the split-K contract, and within twice that of
    the ordered split-K result."""
    inp = workloads.splitk_inputs(63, 4096, 1024, 24, 64)
    say("splitk_gemm_tn_atomic: K 4096, M 1024, N 24, 64 splits")
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    out = torch.zeros(inp.M, inp.N, dtype=torch.float32, device="cuda")
    dr.dr_splitk_gemm_tn_atomic(X, dY, inp.splits, out=out)
    got = host(out).astype(np.float64)
    exact, A = oracle.splitk_reference(inp.X, inp.dY)
    assert np.all(np.abs(got - exact) <= 1e-4 * A)
    det = host(dr.dr_splitk_reduce(dr.dr_splitk_gemm_tn(X, dY, inp.splits))).astype(np.float64)
    assert np.all(np.abs(got - det) <= 2e-4 * A)


def test_splitk_atomic_negative_control(dr):
    """64 splits adding into each dW element: replays of the atomic path change
    bits, while the ordered path's replays do not."""
    inp = workloads.splitk_inputs(64, 8192, 2048, 24, 64)
    X, dY = dev_bf16(inp.X), dev_bf16(inp.dY)
    say("splitk atomic negative control")

    def atomic():
        out = torch.zeros(inp.M, inp.N, dtype=torch.float32, device="cuda")
        dr.dr_splitk_gemm_tn_atomic(X, dY, inp.splits, out=out)
        return out
    fps = replay_fingerprints(dr, atomic)
    assert len(set(fps)) > 1, "splitk_gemm_tn_atomic gave identical bits in every replay"
    det = replay_fingerprints(dr, lambda: dr.dr_splitk_reduce(dr.dr_splitk_gemm_tn(X, dY, inp.splits)), replays=3)
    assert len(set(det)) == 1, det
