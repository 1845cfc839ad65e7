"""Host-side checks of the Python binding, run without a GPU.

A caller-supplied buffer of the wrong shape, size, dtype or device would be an
out-of-bounds access on the device, so the binding refuses it before anything
reaches the library.  Here host tensors stand in for device tensors (the
placement check is replaced for the test) and the library's compute entry
points are replaced by a stub that fails the test if it is reached; the
size queries still go to the real library.  A call with correct arguments
reaches the stub ("reached the library")."""
import pytest
import torch

import bitwise_deterministic_fp32_amd as m

REACHED = "reached the library"


class _NoLaunch:
    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name.endswith("_workspace_size") or name in ("dr_grouped_splitk_max_slots", "dr_status_string",
                                                         "dr_last_error"):
            return getattr(self.real, name)
        raise AssertionError(f"{name} {REACHED}")


@pytest.fixture
def b(monkeypatch):
    def host_dev(t, name, dtypes=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtypes is not None and t.dtype not in dtypes:
            raise TypeError(f"{name} has dtype {t.dtype}")
        return t
    monkeypatch.setattr(m, "_dev", host_dev)
    monkeypatch.setattr(m, "lib", _NoLaunch(m.lib))
    return m


def reaches(fn):
    with pytest.raises(AssertionError, match=REACHED):
        fn()


def f32(*s):
    return torch.zeros(*s, dtype=torch.float32)


def i32(*s):
    return torch.zeros(*s, dtype=torch.int32)


def i64(*s):
    return torch.zeros(*s, dtype=torch.int64)


def bf16(*s):
    return torch.zeros(*s, dtype=torch.bfloat16)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def test_splitk_reduce_checks(b):
    P = f32(4, 6, 8)
    reaches(lambda: b.dr_splitk_reduce(P, out=f32(6, 8)))
    with pytest.raises(ValueError):
        b.dr_splitk_reduce(P, out=f32(6, 7))
    need = b.dr_splitk_reduce_fingerprinted_workspace_size(4, 48)
    reaches(lambda: b.dr_splitk_reduce_fingerprinted(P, i64(1), out=f32(48), ws=u8(need)))
    with pytest.raises(ValueError):
        b.dr_splitk_reduce_fingerprinted(P, i64(2), ws=u8(need))          # hash of two elements
    with pytest.raises(TypeError):
        b.dr_splitk_reduce_fingerprinted(P, i64(1), ws=f32(need))         # workspace not bytes
    with pytest.raises(ValueError):
        b.dr_splitk_reduce_fingerprinted(P, i64(1), ws=u8(need - 1))      # workspace too small
    with pytest.raises(ValueError):
        b.dr_splitk_reduce_fingerprinted(P, i64(1), out=f32(47), ws=u8(need))
    with pytest.raises(ValueError):
        b.dr_splitk_reduce_fingerprinted(P, torch.zeros(1, dtype=torch.int64, device="meta"), ws=u8(need))


def test_splitk_gemm_checks(b):
    X, dY = bf16(512, 64), bf16(512, 24)
    reaches(lambda: b.dr_splitk_gemm_tn(X, dY, 4, partials=f32(4, 64, 24)))
    with pytest.raises(ValueError):
        b.dr_splitk_gemm_tn(X, bf16(511, 24), 4)                          # dY rows differ from K
    with pytest.raises(ValueError):
        b.dr_splitk_gemm_tn(X, dY, 4, partials=f32(3, 64, 24))
    reaches(lambda: b.dr_splitk_gemm_tn_atomic(X, dY, 4, out=f32(64, 24)))
    with pytest.raises(ValueError):
        b.dr_splitk_gemm_tn_atomic(X, dY, 4, out=f32(24, 64))


def test_combine_checks(b):
    rows, row_of, gates = bf16(40, 16), i32(10, 4), f32(10, 4)
    reaches(lambda: b.dr_combine(rows, row_of, gates, out=f32(10, 16)))
    with pytest.raises(ValueError):
        b.dr_combine(rows, row_of, gates, out=f32(10, 8))
    with pytest.raises(ValueError):
        b.dr_combine(rows, row_of, f32(10, 3))
    with pytest.raises(ValueError):
        b.dr_combine_atomic(rows, row_of, gates, out=f32(9, 16))
    with pytest.raises(ValueError):
        b.dr_combine_fingerprinted(rows, row_of, gates, out_hash=i64(3))
    with pytest.raises(ValueError):
        b.dr_combine(rows, row_of, gates, dev_status=i32(0))


def test_index_add_checks(b):
    out, src, index = f32(20, 8), bf16(50, 8), i32(50)
    reaches(lambda: b.dr_index_add(out, src, index))
    reaches(lambda: b.dr_index_add(out, src, index, perm=i32(50), seg_offsets=i32(21)))
    with pytest.raises(ValueError):
        b.dr_index_add(out, bf16(50, 16), index)                          # rows of another width
    with pytest.raises(ValueError):
        b.dr_index_add(out, src, index, perm=i32(49), seg_offsets=i32(21))
    with pytest.raises(ValueError):
        b.dr_index_add(out, src, index, perm=i32(50), seg_offsets=i32(20))
    with pytest.raises(ValueError):
        b.dr_index_add(out, src, index, perm=i32(50))                     # half a plan
    need = b.dr_index_add_workspace_size(50, 20, 8)
    with pytest.raises(ValueError):
        b.dr_index_add(out, src, index, ws=u8(need - 1))
    with pytest.raises(ValueError):
        b.dr_index_add_fingerprinted(out, src, index, i64(2))
    with pytest.raises(ValueError):
        b.dr_index_add_atomic(out, bf16(49, 8), index)
    with pytest.raises(ValueError):
        b.dr_index_add(out, src, torch.zeros(50, dtype=torch.int32, device="meta"))


def test_sparse_attn_dk_checks(b):
    dK, Q, dS, idx = f32(30, 8), bf16(6, 8), f32(6, 4), i32(6, 4)
    reaches(lambda: b.dr_sparse_attn_dk(dK, Q, dS, idx))
    with pytest.raises(ValueError):
        b.dr_sparse_attn_dk(dK, Q, f32(6, 5), idx)
    with pytest.raises(ValueError):
        b.dr_sparse_attn_dk(dK, bf16(5, 8), dS, idx)
    with pytest.raises(ValueError):
        b.dr_sparse_attn_dk(dK, Q, dS, idx, perm=i32(24), seg_offsets=i32(30))


def test_sort_permute_checks(b):
    dest = i32(100)
    reaches(lambda: b.dr_sort_by_dest(dest, 7))
    with pytest.raises(ValueError):
        b.dr_sort_by_dest(dest, 7, perm=i32(99))
    with pytest.raises(ValueError):
        b.dr_sort_by_dest(dest, 7, seg_offsets=i32(7))
    with pytest.raises(ValueError):
        b.dr_sort_by_dest(dest, 7, inv_perm=i32(101))
    with pytest.raises(ValueError):
        b.dr_sort_by_dest(dest, 7, src_id=i32(50), src_id_bound=8)
    x = bf16(25, 16)
    reaches(lambda: b.dr_permute_rows(x, i32(100), 4, out=bf16(100, 16)))
    with pytest.raises(ValueError):
        b.dr_permute_rows(x, i32(100), 4, out=bf16(99, 16))
    with pytest.raises(ValueError):
        b.dr_permute_rows(x, i32(100), 4, inv_perm=i32(10))


def test_grouped_decode_fingerprint_checks(b):
    X, dY, off = bf16(600, 64), bf16(600, 32), i32(5)
    S = b.dr_grouped_splitk_max_slots(600, 4, 128)
    reaches(lambda: b.dr_grouped_splitk_gemm_tn(X, dY, off, 128))
    with pytest.raises(ValueError):
        b.dr_grouped_splitk_gemm_tn(X, dY, off, 128, partials=f32(S - 1, 64, 32))
    with pytest.raises(ValueError):
        b.dr_grouped_splitk_gemm_tn(X, dY, off, 128, slot_offsets=i32(4))
    with pytest.raises(ValueError):
        b.dr_grouped_splitk_reduce(f32(S, 64, 32), i32(5), u8(256), out=f32(3, 64, 32))
    with pytest.raises(ValueError):
        b.dr_grouped_splitk_reduce(f32(S, 64, 32), i32(5), u8(16))
    q, kc, lens = bf16(2, 8, 128), bf16(2, 64, 2, 128), i32(2)
    reaches(lambda: b.dr_decode_attention(q, kc, kc, lens, 0.1, 64))
    with pytest.raises(ValueError):
        b.dr_decode_attention(q, kc, kc, lens, 0.1, 64, out=f32(2, 8, 64))
    with pytest.raises(ValueError):
        b.dr_fingerprint(f32(10), out=i64(2))
    with pytest.raises(ValueError):
        b.dr_fingerprint(f32(10), ws=u8(8))
