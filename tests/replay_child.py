"""Child process of the restart-replay test: loads the inputs a parent saved
to disk, runs the deterministic paths on the GPU through the C ABI, and prints
the fingerprints of their outputs as one JSON line.  Run as
``python tests/replay_child.py <dir>``."""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bitwise_deterministic_fp32_amd as dr  # noqa: E402


def run_all(load) -> dict:
    """The replayed step: the same calls in the parent and the child."""
    def dev(name):
        return torch.from_numpy(np.ascontiguousarray(load(name))).cuda()

    def dev_bf16(name):
        return torch.from_numpy(np.ascontiguousarray(load(name)).view(np.int16)).view(torch.bfloat16).cuda()

    fps = {}
    E, T, k = int(load("moe_E")), int(load("moe_T")), int(load("moe_k"))
    _, _, inv = dr.dr_sort_by_dest(dev("moe_expert_ids"), E)
    out, h = dr.dr_combine_fingerprinted(dev_bf16("moe_rows"), inv.view(T, k), dev("moe_gates"))
    fps["combine"] = dr.fingerprint_value(out)
    fps["combine_fused_hash"] = int(h.item()) & ((1 << 64) - 1)
    out = dev("ia_out0")
    dr.dr_index_add(out, dev_bf16("ia_src"), dev("ia_index"))
    fps["index_add"] = dr.fingerprint_value(out)
    dK = dev("dk_dK0")
    dr.dr_sparse_attn_dk(dK, dev_bf16("dk_Q"), dev("dk_dS"), dev("dk_key_idx"))
    fps["sparse_attn_dk"] = dr.fingerprint_value(dK)
    splits = int(load("sk_splits"))
    dW = dr.dr_splitk_reduce(dr.dr_splitk_gemm_tn(dev_bf16("sk_X"), dev_bf16("sk_dY"), splits))
    fps["splitk"] = dr.fingerprint_value(dW)
    return fps


def main(folder: str) -> None:
    fps = run_all(lambda name: np.load(os.path.join(folder, name + ".npy")))
    torch.cuda.synchronize()
    print(json.dumps({k: str(v) for k, v in fps.items()}), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
