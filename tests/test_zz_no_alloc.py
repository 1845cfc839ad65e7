"""The no-allocation combine, dr_combine_fingerprinted_noalloc, against the
workspace entry point it is a variant of, dr_combine_fingerprinted: the same
output bits and the same fingerprint, call after call.  The calls run in a row
with shrinking inputs, so each one starts from the scratch the one before left
behind.  All calls go through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import assert_bits_equal, dev, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # seed, tokens, experts, top-k, hidden, row dtype
    (81, 4096, 64, 8, 7168, "bf16"),   # 28,672 wavefronts, 3,584 partials: the one-workgroup wide sum
    (82, 1000, 32, 12, 1024, "bf16"),  # k > 8: four wavefronts per workgroup
    (83, 300, 16, 3, 256, "f32"),      # smaller again
]


def test_noalloc_combine_matches_the_workspace_entry_point():
    require_gpu()
    import bitwise_deterministic_fp32_amd as dr
    dr.dr_set_launch_params(reset=True)
    for seed, T, E, k, H, dt in CASES:
        say(f"noalloc combine: T={T} E={E} k={k} H={H} {dt}")
        inp = workloads.moe_inputs(seed, T, E, k, H, dt, zipf_bias_s=1.2)
        _, _, inv = dr.dr_sort_by_dest(dev(inp.expert_ids.reshape(-1)), E)
        rows = dev_bf16(inp.rows) if dt == "bf16" else dev(inp.rows)
        row_of, gates = inv.view(T, k), dev(inp.gates)
        want, want_h = dr.dr_combine_fingerprinted(rows, row_of, gates)
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        h = torch.zeros(1, dtype=torch.int64, device="cuda")
        for rep in range(2):
            dr.dr_combine_fingerprinted_noalloc(rows, row_of, gates, out=out, out_hash=h)
            assert_bits_equal(host(out), host(want), f"noalloc combine T={T} rep {rep}")
            assert int(h.item()) == int(want_h.item()), (T, rep)
        assert int(h.item()) & ((1 << 64) - 1) == dr.fingerprint_value(out)
