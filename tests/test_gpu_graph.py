"""The entry points launch only kernels on the caller's stream (no memset, copy
or synchronisation), so a step can be captured once in a HIP graph and
replayed.  Each graph here is replayed several times, with other eager work
and synchronisations between the replays, and every replay must give the
bits of the eager calls."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import assert_bits_equal, dev, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dr():
    require_gpu()
    import bitwise_deterministic_fp32_amd as m
    m.dr_set_launch_params(reset=True)
    return m


def capture(fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_moe_step_graph(dr):
    say("graph: dispatch sort + fingerprinting combine")
    inp = workloads.moe_inputs(41, 1000, 64, 8, 1024, "bf16", 1.2)
    T, E, k, H = inp.T, inp.E, inp.k, inp.H
    keys = dev(inp.expert_ids.reshape(-1).copy())
    rows, gates = dev_bf16(inp.rows), dev(inp.gates)
    n = T * k
    perm, seg, inv = (torch.empty(n, dtype=torch.int32, device="cuda"), torch.empty(E + 1, dtype=torch.int32,
                      device="cuda"), torch.empty(n, dtype=torch.int32, device="cuda"))
    ws_sort = torch.empty(dr.dr_sort_workspace_size(n, E), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    fp = torch.empty(1, dtype=torch.int64, device="cuda")
    ws_c = torch.empty(dr.dr_combine_fingerprinted_workspace_size(rows.dtype, H, T), dtype=torch.uint8,
                       device="cuda")

    def step():
        dr.dr_sort_by_dest(keys, E, perm=perm, seg_offsets=seg, inv_perm=inv, ws=ws_sort)
        dr.dr_combine_fingerprinted(rows, inv.view(T, k), gates, out=out, out_hash=fp, ws=ws_c)

    step()
    want_out, want_fp, want_inv = host(out).copy(), int(fp.item()), host(inv).copy()
    g = capture(step)
    for r in range(3):
        out.fill_(7.0)
        inv.zero_()
        fp.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(host(out), want_out, f"replay {r}")
        assert int(fp.item()) == want_fp and np.array_equal(host(inv), want_inv)
        dr.dr_combine(rows, inv.view(T, k), gates)  # eager work between replays
        torch.cuda.synchronize()


def test_decode_attention_graph(dr):
    say("graph: decode attention")
    inp = workloads.decode_inputs(42, 5, 1300, 32, 8, 128, [1300, 5, 700, 0, 1024])
    q, k, v, L = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), dev(inp.lens)
    out = torch.empty(5, 32, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(dr.dr_decode_attention_workspace_size(5, 32, 1300, 256), dtype=torch.uint8, device="cuda")
    call = lambda: dr.dr_decode_attention(q, k, v, L, inp.scale, 256, out=out, ws=ws)
    call()
    want = host(out).copy()
    g = capture(call)
    for r in range(3):
        out.fill_(-1.0)
        ws.fill_(0xFF)  # stale partials must not leak into a replay
        g.replay()
        assert_bits_equal(host(out), want, f"replay {r}")
        dr.dr_decode_attention(q[:2].contiguous(), k[:2].contiguous(), v[:2].contiguous(), L[:2].contiguous(),
                               inp.scale, 64)
        torch.cuda.synchronize()


def test_index_add_graph(dr):
    say("graph: index_add (internal sort and plan) on a reset destination")
    rng = np.random.default_rng(43)
    n, D, H = 20000, 3000, 256
    index = dev(np.minimum(rng.zipf(1.3, n) - 1, D - 1).astype(np.int32))
    src = dev_bf16(workloads.normal_bf16(43, 1, n * H).reshape(n, H))
    out0 = dev(workloads.normal_f32(43, 2, D * H).reshape(D, H))
    out = out0.clone()
    ws = torch.empty(dr.dr_index_add_workspace_size(n, D, H), dtype=torch.uint8, device="cuda")
    call = lambda: dr.dr_index_add(out, src, index, ws=ws)
    call()
    want = host(out).copy()
    g = capture(call)
    for r in range(3):
        out.copy_(out0)
        ws.fill_(0xFF)
        g.replay()
        assert_bits_equal(host(out), want, f"replay {r}")
        dr.dr_workspace_status(ws)
        dr.dr_index_add(out0.clone(), src[:100].contiguous(), index[:100].contiguous())
        torch.cuda.synchronize()


def test_splitk_graph(dr):
    say("graph: split-K partials + ordered reduce")
    sk = workloads.splitk_inputs(44, 4096, 1000, 24, 16)
    X, dY = dev_bf16(sk.X), dev_bf16(sk.dY)
    P = torch.empty(16, 1000, 24, dtype=torch.float32, device="cuda")
    dW = torch.empty(1000, 24, dtype=torch.float32, device="cuda")

    def call():
        dr.dr_splitk_gemm_tn(X, dY, 16, partials=P)
        dr.dr_splitk_reduce(P, out=dW)

    call()
    want = host(dW).copy()
    g = capture(call)
    for r in range(3):
        dW.fill_(3.0)
        P.fill_(float("nan"))
        g.replay()
        assert_bits_equal(host(dW), want, f"replay {r}")
        dr.dr_splitk_gemm_tn(X[:256].contiguous(), dY[:256].contiguous(), 1)
        torch.cuda.synchronize()


def test_splitk_reduce_fingerprinted_graph(dr):
    """The split-K step with the fused reduce and fingerprint, replayed from a graph."""
    say("graph: split-K partials + reduce with its fingerprint")
    sk = workloads.splitk_inputs(46, 4096, 1000, 24, 64)
    X, dY = dev_bf16(sk.X), dev_bf16(sk.dY)
    P = torch.empty(64, 1000, 24, dtype=torch.float32, device="cuda")
    dW = torch.empty(1000, 24, dtype=torch.float32, device="cuda")
    h = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(dr.dr_splitk_reduce_fingerprinted_workspace_size(64, 1000 * 24), dtype=torch.uint8,
                     device="cuda")

    def call():
        dr.dr_splitk_gemm_tn(X, dY, 64, partials=P)
        dr.dr_splitk_reduce_fingerprinted(P, h, out=dW, ws=ws)

    call()
    want = host(dW).copy()
    want_h = int(h.item())
    assert want_h == int(dr.dr_fingerprint(dW).item())
    g = capture(call)
    for r in range(3):
        dW.fill_(3.0)
        P.fill_(float("nan"))
        h.fill_(0)
        ws.fill_(0xFF)
        g.replay()
        assert_bits_equal(host(dW), want, f"replay {r}")
        assert int(h.item()) == want_h, f"replay {r}: fingerprint"
        dr.dr_splitk_gemm_tn(X[:256].contiguous(), dY[:256].contiguous(), 1)
        torch.cuda.synchronize()


def test_index_add_fingerprinted_graph(dr):
    """The destination's fingerprint stays current over eager calls and over graph replays."""
    say("graph: index_add_fingerprinted, accumulating")
    rng = np.random.default_rng(45)
    n, D, H = 8000, 40000, 512
    index = dev(np.minimum(rng.zipf(1.1, n) - 1, D - 1).astype(np.int32))
    src = dev_bf16(workloads.normal_bf16(45, 1, n * H).reshape(n, H))
    out = dev(workloads.normal_f32(45, 2, D * H).reshape(D, H))
    h = torch.empty(1, dtype=torch.int64, device="cuda")
    dr.dr_fingerprint(out, out=h)
    ws = torch.empty(dr.dr_index_add_workspace_size(n, D, H), dtype=torch.uint8, device="cuda")
    call = lambda: dr.dr_index_add_fingerprinted(out, src, index, h, ws=ws)
    for i in range(8):
        call()
        torch.cuda.synchronize()
        assert (int(h.item()) & ((1 << 64) - 1)) == dr.fingerprint_value(out), f"eager call {i}"
    g = capture(call)
    for r in range(6):
        g.replay()
        torch.cuda.synchronize()
        assert (int(h.item()) & ((1 << 64) - 1)) == dr.fingerprint_value(out), f"replay {r}"
