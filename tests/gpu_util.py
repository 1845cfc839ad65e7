"""Helpers for the GPU tests: host <-> device transfers and byte comparisons.
Nothing here computes any part of the reduction."""
import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def say(msg: str) -> None:
    """Progress line naming the case, flushed before the GPU work it announces."""
    print(msg, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bfloat16 bit patterns (uint16) to a device bf16 tensor, bit for bit."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint8)


def assert_bits_equal(got, want, what=""):
    got, want = np.ascontiguousarray(got), np.ascontiguousarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gb, wb = bits(got), bits(want)
    if not np.array_equal(gb, wb):
        bad = np.argwhere(gb != wb)
        first = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements differ; first at {first}: "
                             f"got {got[first]!r} ({gb[first]:#x}) want {want[first]!r} ({wb[first]:#x})")
