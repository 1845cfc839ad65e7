"""Restart replay: inputs saved to disk and replayed by a fresh process give
the same output bytes (compared by fingerprint) as the run that saved them.

This is the restart-replay gate of the bitwise-determinism interview note
("how to verify: three gates"): a run restored from disk must continue with
identical bits.  The replaying process shares nothing with the first one but
the files (no warm caches, no allocator state, another HIP context)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fresh_process_replay_gives_identical_fingerprints(tmp_path):
    require_gpu()
    from tests.replay_child import run_all
    moe = workloads.moe_inputs(71, 1024, 64, 8, 1024, "bf16", zipf_bias_s=1.2)
    ia = workloads.sparse_attn_inputs(72, Q=512, K=4096, S=64, H=128)
    dk = workloads.sparse_attn_dk_inputs(73, Q=1024, K=8192, S=64)
    sk = workloads.splitk_inputs(74, 4096, 1024, 24, 16)
    arrays = {
        "moe_E": np.array(moe.E), "moe_T": np.array(moe.T), "moe_k": np.array(moe.k),
        "moe_expert_ids": moe.expert_ids.reshape(-1), "moe_rows": moe.rows, "moe_gates": moe.gates,
        "ia_out0": ia.out0, "ia_src": ia.src, "ia_index": ia.index,
        "dk_dK0": dk.dK0, "dk_Q": dk.Q, "dk_dS": dk.dS, "dk_key_idx": dk.key_idx,
        "sk_X": sk.X, "sk_dY": sk.dY, "sk_splits": np.array(sk.splits),
    }
    for name, a in arrays.items():
        np.save(tmp_path / (name + ".npy"), a, allow_pickle=False)
    say("replay: first run in this process")
    first = {k: str(v) for k, v in run_all(lambda name: np.load(tmp_path / (name + ".npy"))).items()}
    torch.cuda.synchronize()
    say("replay: fresh child process")
    r = subprocess.run([sys.executable, os.path.join(HERE, "replay_child.py"), str(tmp_path)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    child = json.loads(r.stdout.strip().splitlines()[-1])
    assert child == first, (child, first)
    assert first["combine"] == first["combine_fused_hash"]
