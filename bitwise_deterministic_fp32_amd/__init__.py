"""Python binding of libdetreduce: argument marshalling only.

Every function here has the name of the C entry point it calls
(include/detreduce.h).  It checks tensor placement and dtypes, allocates the
outputs and workspaces it is not given (torch is used for device memory and
streams only), and passes raw pointers and the current HIP stream to the
library.  All arithmetic happens in the HIP kernels of libdetreduce.so; there
is no fallback.  Importing this package fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "DetReduceError", "LIB_PATH", "lib", "declared_functions",
    "dr_status_string", "dr_last_error", "dr_version", "dr_set_launch_params", "dr_set_phase_events",
    "dr_sort_workspace_size", "dr_sort_by_dest",
    "dr_combine", "dr_combine_atomic", "dr_combine_fingerprinted_workspace_size", "dr_combine_fingerprinted",
    "dr_combine_fingerprinted_noalloc",
    "dr_index_add_workspace_size", "dr_index_add", "dr_index_add_fingerprinted", "dr_index_add_atomic",
    "dr_sparse_attn_dk_workspace_size", "dr_sparse_attn_dk",
    "dr_splitk_gemm_tn", "dr_splitk_gemm_tn_atomic", "dr_splitk_reduce",
    "dr_splitk_reduce_fingerprinted_workspace_size", "dr_splitk_reduce_fingerprinted",
    "dr_grouped_splitk_max_slots", "dr_grouped_splitk_workspace_size", "dr_grouped_splitk_gemm_tn",
    "dr_grouped_splitk_reduce", "dr_grouped_wgrad_workspace_size", "dr_grouped_wgrad", "dr_permute_rows",
    "dr_decode_attention_workspace_size", "dr_decode_attention", "dr_decode_attention_occupancy_chunk",
    "dr_fingerprint_workspace_size", "dr_fingerprint", "fingerprint_value",
    "dr_workspace_status", "dr_read_status",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdetreduce.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "detreduce.h")

DR_F32, DR_BF16 = 0, 1
_STATUS_BYTES = 256  # the status block at the start of every workspace
_DTYPES = {torch.float32: DR_F32, torch.bfloat16: DR_BF16}


class DetReduceError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        self.status = status
        super().__init__(f"{what}: {_status_name(status)}: {detail}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bitwise_deterministic_fp32_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "dr_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "dr_last_error": ([], ctypes.c_char_p),
        "dr_version": ([], i32),
        "dr_set_launch_params": ([vp], ctypes.c_int),
        "dr_set_phase_events": ([vp, vp], ctypes.c_int),
        "dr_sort_workspace_size": ([i64, i32, i32], sz),
        "dr_sort_by_dest": ([vp, vp, i32, i64, i32, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "dr_combine": ([vp, ctypes.c_int, i64, i64, vp, vp, i64, i32, vp, vp, vp], ctypes.c_int),
        "dr_combine_atomic": ([vp, ctypes.c_int, i64, i64, vp, vp, i64, i32, vp, vp, vp], ctypes.c_int),
        "dr_combine_fingerprinted_workspace_size": ([ctypes.c_int, i64, i64], sz),
        "dr_combine_fingerprinted": ([vp, ctypes.c_int, i64, i64, vp, vp, i64, i32, vp, vp, vp, sz, vp, vp],
                                     ctypes.c_int),
        "dr_combine_fingerprinted_noalloc": ([vp, ctypes.c_int, i64, i64, vp, vp, i64, i32, vp, vp, vp, vp],
                                             ctypes.c_int),
        "dr_index_add_workspace_size": ([i64, i32, i64], sz),
        "dr_index_add": ([vp, i32, i64, vp, ctypes.c_int, i64, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "dr_index_add_fingerprinted": ([vp, i32, i64, vp, ctypes.c_int, i64, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "dr_index_add_atomic": ([vp, i32, i64, vp, ctypes.c_int, i64, vp, vp, vp], ctypes.c_int),
        "dr_sparse_attn_dk_workspace_size": ([i64, i32, i32, i64], sz),
        "dr_sparse_attn_dk": ([vp, i32, i64, vp, ctypes.c_int, vp, vp, i64, i32, vp, vp, vp, sz, vp], ctypes.c_int),
        "dr_splitk_gemm_tn": ([vp, vp, i64, i64, i64, i32, vp, vp], ctypes.c_int),
        "dr_splitk_gemm_tn_atomic": ([vp, vp, i64, i64, i64, i32, vp, vp], ctypes.c_int),
        "dr_splitk_reduce": ([vp, i32, i64, vp, vp], ctypes.c_int),
        "dr_splitk_reduce_fingerprinted_workspace_size": ([i32, i64], sz),
        "dr_splitk_reduce_fingerprinted": ([vp, i32, i64, vp, vp, vp, sz, vp], ctypes.c_int),
        "dr_grouped_splitk_max_slots": ([i64, i32, i32], i64),
        "dr_grouped_splitk_workspace_size": ([i64, i32, i32], sz),
        "dr_grouped_splitk_gemm_tn": ([vp, vp, i64, i64, i64, vp, i32, i32, vp, i64, vp, vp, sz, vp], ctypes.c_int),
        "dr_grouped_splitk_reduce": ([vp, i64, vp, i32, i64, vp, vp, vp], ctypes.c_int),
        "dr_grouped_wgrad_workspace_size": ([i64, i32, i32, i64, i64], sz),
        "dr_grouped_wgrad": ([vp, vp, i64, i64, i64, vp, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "dr_permute_rows": ([vp, i64, i64, vp, vp, i64, i32, vp, vp, vp], ctypes.c_int),
        "dr_decode_attention_workspace_size": ([i64, i32, i32, i32, i64], sz),
        "dr_decode_attention": ([vp, vp, vp, vp, ctypes.c_int, vp, i64, i32, i32, i64, i32, ctypes.c_float, i32, vp, sz,
                                 vp, vp],
                                ctypes.c_int),
        "dr_decode_attention_occupancy_chunk": ([i64, i32, i32], i32),
        "dr_fingerprint_workspace_size": ([i64], sz),
        "dr_fingerprint": ([vp, i64, vp, vp, sz, vp], ctypes.c_int),
        "dr_workspace_status": ([vp, vp], ctypes.c_int),
        "dr_read_status": ([vp, vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def declared_functions() -> list[str]:
    """Names of the functions that include/detreduce.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dr_[a-z0-9_]+)\s*\(", text)))


def _status_name(s: int) -> str:
    return lib.dr_status_string(s).decode()


def dr_status_string(s: int) -> str:
    return _status_name(s)


def dr_last_error() -> str:
    return lib.dr_last_error().decode()


def dr_version() -> int:
    return int(lib.dr_version())


def _check(status: int, what: str) -> None:
    if status != 0:
        raise DetReduceError(status, what, dr_last_error())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtypes=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


class _LaunchParams(ctypes.Structure):
    _fields_ = [("grid_blocks", ctypes.c_int32), ("tile_chunks_log2", ctypes.c_int32),
                ("sort_tile_log2", ctypes.c_int32), ("chunks_in_flight", ctypes.c_int32),
                ("splitk_stream", ctypes.c_int32)]


def dr_set_launch_params(grid_blocks: int = 0, tile_chunks_log2: int = 0, sort_tile_log2: int = 0,
                         chunks_in_flight: int = 0, splitk_stream: int = 0, reset: bool = False) -> None:
    """Thread-local launch overrides (tests of launch invariance); reset=True restores defaults."""
    if reset:
        _check(lib.dr_set_launch_params(None), "dr_set_launch_params")
        return
    p = _LaunchParams(grid_blocks, tile_chunks_log2, sort_tile_log2, chunks_in_flight, splitk_stream)
    _check(lib.dr_set_launch_params(ctypes.byref(p)), "dr_set_launch_params")


def dr_set_phase_events(reduce_begin=None, reduce_end=None) -> None:
    """Thread-local hook: index_add-family calls record these torch.cuda.Events (enable_timing=True) around
    their ordered reduction kernels.  No arguments turns it off."""
    def handle(e):
        if e is None:
            return None
        if not e.cuda_event:
            e.record()  # torch creates the underlying event at its first record
        return e.cuda_event
    _check(lib.dr_set_phase_events(handle(reduce_begin), handle(reduce_end)), "dr_set_phase_events")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _sized(t: torch.Tensor, name: str, device, dtypes=None, shape=None, numel=None, min_numel=None) -> torch.Tensor:
    """A caller-supplied buffer: on `device`, contiguous, of the given dtype and
    exactly `shape` (or `numel` elements, or at least `min_numel`).  A buffer
    too small for what the kernels write would be an out-of-bounds access on the
    device, so every mismatch is refused here, before anything is launched."""
    _dev(t, name, dtypes)
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")
    return t


def _ws(ws, need: int, device, name: str = "ws") -> torch.Tensor:
    """A workspace: the caller's (a uint8 tensor on `device`, its numel is the
    byte count passed on) or a new one of `need` bytes."""
    if ws is None:
        return _workspace(need, device)
    return _sized(ws, name, device, (torch.uint8,), min_numel=need)


def _status_buf(dev_status, device):
    if dev_status is not None:
        _sized(dev_status, "dev_status", device, (torch.int32,), min_numel=1)
    return dev_status


def _hash_buf(h, name: str, device) -> torch.Tensor:
    return _sized(h, name, device, (torch.int64,), numel=1)


# ---------------------------------------------------------------------------
def dr_sort_workspace_size(n: int, num_dests: int, src_id_bound: int = 0) -> int:
    return int(lib.dr_sort_workspace_size(n, num_dests, src_id_bound))


def dr_sort_by_dest(dest, num_dests: int, src_id=None, src_id_bound: int = 0, *, perm=None, seg_offsets=None,
                    inv_perm=None, want_inv: bool = True, ws=None, stream=None):
    """Stable sort by (dest, src_id).  Returns (perm, seg_offsets, inv_perm or None)."""
    _dev(dest, "dest", (torch.int32,))
    n = dest.numel()
    dev = dest.device
    if src_id is not None:
        _sized(src_id, "src_id", dev, (torch.int32,), numel=n)
    i32 = (torch.int32,)
    perm = _sized(perm, "perm", dev, i32, numel=n) if perm is not None else \
        torch.empty(n, dtype=torch.int32, device=dev)
    seg_offsets = _sized(seg_offsets, "seg_offsets", dev, i32, numel=num_dests + 1) if seg_offsets is not None \
        else torch.empty(num_dests + 1, dtype=torch.int32, device=dev)
    if inv_perm is None and want_inv:
        inv_perm = torch.empty(n, dtype=torch.int32, device=dev)
    elif inv_perm is not None:
        _sized(inv_perm, "inv_perm", dev, i32, numel=n)
    need = dr_sort_workspace_size(n, num_dests, src_id_bound if src_id is not None else 0)
    ws = _ws(ws, need, dev)
    _check(lib.dr_sort_by_dest(_p(dest), _p(src_id), src_id_bound, n, num_dests, _p(perm), _p(seg_offsets),
                               _p(inv_perm), _p(ws), ws.numel(), _stream(stream)), "dr_sort_by_dest")
    return perm, seg_offsets, inv_perm


def _combine_args(rows, row_of, gates):
    _dev(rows, "rows", tuple(_DTYPES))
    _sized(row_of, "row_of", rows.device, (torch.int32,))
    _sized(gates, "gates", rows.device, (torch.float32,))
    if rows.dim() != 2 or row_of.dim() != 2 or gates.shape != row_of.shape:
        raise ValueError("rows must be [R, H]; row_of and gates [T, k]")
    return rows.shape[0], rows.shape[1], row_of.shape[0], row_of.shape[1]


def _combine_out(out, rows, T, H):
    if out is None:
        return torch.empty(T, H, dtype=torch.float32, device=rows.device)
    return _sized(out, "out", rows.device, (torch.float32,), shape=(T, H))


def dr_combine(rows, row_of, gates, *, out=None, dev_status=None, stream=None):
    """out[t] = ordered tree over fl32(gate * row) of the token's k rows (written)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    out = _combine_out(out, rows, T, H)
    _status_buf(dev_status, rows.device)
    _check(lib.dr_combine(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k, _p(out),
                          _p(dev_status), _stream(stream)), "dr_combine")
    return out


def dr_combine_fingerprinted_workspace_size(rows_dtype, hidden: int, T: int) -> int:
    return int(lib.dr_combine_fingerprinted_workspace_size(_DTYPES[rows_dtype], hidden, T))


def dr_combine_fingerprinted(rows, row_of, gates, *, out=None, out_hash=None, ws=None, dev_status=None, stream=None):
    """dr_combine plus the fingerprint of its output, hashed as it is stored.  Returns (out, out_hash)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    out = _combine_out(out, rows, T, H)
    out_hash = _hash_buf(out_hash, "out_hash", rows.device) if out_hash is not None else \
        torch.empty(1, dtype=torch.int64, device=rows.device)
    ws = _ws(ws, dr_combine_fingerprinted_workspace_size(rows.dtype, H, T), rows.device)
    _status_buf(dev_status, rows.device)
    _check(lib.dr_combine_fingerprinted(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k, _p(out),
                                        _p(out_hash), _p(ws), ws.numel(), _p(dev_status), _stream(stream)),
           "dr_combine_fingerprinted")
    return out, out_hash


def dr_combine_fingerprinted_noalloc(rows, row_of, gates, *, out, out_hash, dev_status=None, stream=None):
    """dr_combine_fingerprinted with the library's static scratch instead of a workspace (nothing is
    allocated, here or in the library: the caller passes out and out_hash).  Returns (out, out_hash)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    _sized(out, "out", rows.device, (torch.float32,), shape=(T, H))
    _hash_buf(out_hash, "out_hash", rows.device)
    _status_buf(dev_status, rows.device)
    _check(lib.dr_combine_fingerprinted_noalloc(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k,
                                                _p(out), _p(out_hash), _p(dev_status), _stream(stream)),
           "dr_combine_fingerprinted_noalloc")
    return out, out_hash


def dr_combine_atomic(rows, row_of, gates, *, out, dev_status=None, stream=None):
    """Nondeterministic baseline: atomically adds each fl32(gate * row) into out (caller zeroes it)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    _sized(out, "out", rows.device, (torch.float32,), shape=(T, H))
    _status_buf(dev_status, rows.device)
    _check(lib.dr_combine_atomic(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k, _p(out),
                                 _p(dev_status), _stream(stream)), "dr_combine_atomic")
    return out


# ---------------------------------------------------------------------------
def dr_index_add_workspace_size(n: int, num_dests: int, hidden: int) -> int:
    return int(lib.dr_index_add_workspace_size(n, num_dests, hidden))


def _index_add_args(out, src, index, perm, seg_offsets):
    _dev(out, "out", (torch.float32,))
    if out.dim() != 2:
        raise ValueError("out must be [num_dests, hidden]")
    D, H = out.shape
    _sized(index, "index", out.device, (torch.int32,))
    n = index.numel()
    _sized(src, "src", out.device, tuple(_DTYPES), shape=(n, H))
    _plan_args(perm, seg_offsets, n, D, out.device)
    return D, H, n


def _plan_args(perm, seg_offsets, n, D, device):
    if (perm is None) != (seg_offsets is None):
        raise ValueError("perm and seg_offsets must both be given or both be None")
    if perm is not None:
        _sized(perm, "perm", device, (torch.int32,), numel=n)
        _sized(seg_offsets, "seg_offsets", device, (torch.int32,), numel=D + 1)


def dr_index_add(out, src, index, *, perm=None, seg_offsets=None, ws=None, stream=None):
    """out[d] += ordered tree of src rows i with index[i] == d (in place).  Returns (out, ws)."""
    D, H, n = _index_add_args(out, src, index, perm, seg_offsets)
    ws = _ws(ws, dr_index_add_workspace_size(n, D, H), out.device)
    _check(lib.dr_index_add(_p(out), D, H, _p(src), _DTYPES[src.dtype], n, _p(index), _p(perm), _p(seg_offsets),
                            _p(ws), ws.numel(), _stream(stream)), "dr_index_add")
    return out, ws


def dr_index_add_fingerprinted(out, src, index, inout_hash, *, perm=None, seg_offsets=None, ws=None, stream=None):
    """dr_index_add that moves inout_hash (an int64 device tensor of one element holding the fingerprint of
    out) to the fingerprint of the updated out.  Returns (out, ws)."""
    D, H, n = _index_add_args(out, src, index, perm, seg_offsets)
    _hash_buf(inout_hash, "inout_hash", out.device)
    ws = _ws(ws, dr_index_add_workspace_size(n, D, H), out.device)
    _check(lib.dr_index_add_fingerprinted(_p(out), D, H, _p(src), _DTYPES[src.dtype], n, _p(index), _p(perm),
                                          _p(seg_offsets), _p(inout_hash), _p(ws), ws.numel(), _stream(stream)),
           "dr_index_add_fingerprinted")
    return out, ws


def dr_sparse_attn_dk_workspace_size(num_queries: int, topk: int, num_keys: int, head_dim: int) -> int:
    return int(lib.dr_sparse_attn_dk_workspace_size(num_queries, topk, num_keys, head_dim))


def dr_sparse_attn_dk(dK, Q, dS, key_idx, *, perm=None, seg_offsets=None, ws=None, stream=None):
    """dK[key] += ordered tree of fl32(dS[q, j] * Q[q]) over the (q, j) that selected key (in place).
    Returns (dK, ws)."""
    _dev(dK, "dK", (torch.float32,))
    _sized(key_idx, "key_idx", dK.device, (torch.int32,))
    if dK.dim() != 2 or key_idx.dim() != 2:
        raise ValueError("dK must be [num_keys, head_dim] and key_idx [num_queries, topk]")
    K, H = dK.shape
    nq, topk = key_idx.shape
    _sized(Q, "Q", dK.device, tuple(_DTYPES), shape=(nq, H))
    _sized(dS, "dS", dK.device, (torch.float32,), shape=(nq, topk))
    _plan_args(perm, seg_offsets, nq * topk, K, dK.device)
    ws = _ws(ws, dr_sparse_attn_dk_workspace_size(nq, topk, K, H), dK.device)
    _check(lib.dr_sparse_attn_dk(_p(dK), K, H, _p(Q), _DTYPES[Q.dtype], _p(dS), _p(key_idx), nq, topk, _p(perm),
                                 _p(seg_offsets), _p(ws), ws.numel(), _stream(stream)), "dr_sparse_attn_dk")
    return dK, ws


def dr_index_add_atomic(out, src, index, *, dev_status=None, stream=None):
    D, H, n = _index_add_args(out, src, index, None, None)
    _status_buf(dev_status, out.device)
    _check(lib.dr_index_add_atomic(_p(out), D, H, _p(src), _DTYPES[src.dtype], n, _p(index), _p(dev_status),
                                   _stream(stream)), "dr_index_add_atomic")
    return out


# ---------------------------------------------------------------------------
def _gemm_args(X, dY):
    _dev(X, "X", (torch.bfloat16,))
    if X.dim() != 2 or dY.dim() != 2:
        raise ValueError("X must be [K, M] and dY [K, N]")
    _sized(dY, "dY", X.device, (torch.bfloat16,))
    if dY.shape[0] != X.shape[0]:
        raise ValueError(f"X and dY must have the same number of rows (tokens), got {X.shape[0]} and {dY.shape[0]}")
    return X.shape[0], X.shape[1], dY.shape[1]


def dr_splitk_gemm_tn(X, dY, splits: int, *, partials=None, stream=None):
    """partials[s] = X_s^T dY_s (bf16 MFMA into fp32), one private buffer per split."""
    K, M, N = _gemm_args(X, dY)
    partials = _sized(partials, "partials", X.device, (torch.float32,), shape=(splits, M, N)) \
        if partials is not None else torch.empty(splits, M, N, dtype=torch.float32, device=X.device)
    _check(lib.dr_splitk_gemm_tn(_p(X), _p(dY), K, M, N, splits, _p(partials), _stream(stream)), "dr_splitk_gemm_tn")
    return partials


def dr_splitk_gemm_tn_atomic(X, dY, splits: int, *, out, stream=None):
    """Nondeterministic baseline: adds every split's X_s^T dY_s into out [M, N] with fp32 atomics."""
    K, M, N = _gemm_args(X, dY)
    _sized(out, "out", X.device, (torch.float32,), shape=(M, N))
    _check(lib.dr_splitk_gemm_tn_atomic(_p(X), _p(dY), K, M, N, splits, _p(out), _stream(stream)),
           "dr_splitk_gemm_tn_atomic")
    return out


def _reduce_args(partials):
    _dev(partials, "partials", (torch.float32,))
    if partials.dim() < 1 or partials.shape[0] < 1:
        raise ValueError("partials must be [S, ...] with S >= 1")
    S = partials.shape[0]
    return S, partials.numel() // S


def _reduce_out(out, partials, count):
    if out is None:
        return torch.empty(partials.shape[1:], dtype=torch.float32, device=partials.device)
    return _sized(out, "out", partials.device, (torch.float32,), numel=count)


def dr_splitk_reduce(partials, *, out=None, stream=None):
    """out = ordered tree over the split axis of partials [S, ...]."""
    S, count = _reduce_args(partials)
    out = _reduce_out(out, partials, count)
    _check(lib.dr_splitk_reduce(_p(partials), S, count, _p(out), _stream(stream)), "dr_splitk_reduce")
    return out


def dr_splitk_reduce_fingerprinted_workspace_size(splits: int, count: int) -> int:
    return lib.dr_splitk_reduce_fingerprinted_workspace_size(splits, count)


def dr_splitk_reduce_fingerprinted(partials, out_hash, *, out=None, ws=None, stream=None):
    """dr_splitk_reduce that also writes dr_fingerprint(out) to out_hash (int64 [1] on the device)."""
    S, count = _reduce_args(partials)
    _hash_buf(out_hash, "out_hash", partials.device)
    out = _reduce_out(out, partials, count)
    ws = _ws(ws, dr_splitk_reduce_fingerprinted_workspace_size(S, count), partials.device)
    _check(lib.dr_splitk_reduce_fingerprinted(_p(partials), S, count, _p(out), _p(out_hash), _p(ws), ws.numel(),
                                              _stream(stream)), "dr_splitk_reduce_fingerprinted")
    return out


def dr_grouped_splitk_max_slots(K: int, num_groups: int, split_tokens: int) -> int:
    return int(lib.dr_grouped_splitk_max_slots(K, num_groups, split_tokens))


def dr_grouped_splitk_workspace_size(K: int, num_groups: int, split_tokens: int) -> int:
    return int(lib.dr_grouped_splitk_workspace_size(K, num_groups, split_tokens))


def dr_grouped_splitk_gemm_tn(X, dY, group_offsets, split_tokens: int, *, partials=None, slot_offsets=None, ws=None,
                              stream=None):
    """Private slot partials X_s^T dY_s of every group's token slots.  Returns (partials, slot_offsets, ws)."""
    K, M, N = _gemm_args(X, dY)
    _sized(group_offsets, "group_offsets", X.device, (torch.int32,), min_numel=2)
    G = group_offsets.numel() - 1
    S = dr_grouped_splitk_max_slots(K, G, split_tokens)
    if partials is None:
        partials = torch.empty(S, M, N, dtype=torch.float32, device=X.device)
    else:
        _sized(partials, "partials", X.device, (torch.float32,))
        if partials.dim() != 3 or tuple(partials.shape[1:]) != (M, N) or partials.shape[0] < S:
            raise ValueError(f"partials must be [>= {S}, {M}, {N}], got {tuple(partials.shape)}")
    slot_offsets = _sized(slot_offsets, "slot_offsets", X.device, (torch.int32,), numel=G + 1) \
        if slot_offsets is not None else torch.empty(G + 1, dtype=torch.int32, device=X.device)
    ws = _ws(ws, dr_grouped_splitk_workspace_size(K, G, split_tokens), X.device)
    _check(lib.dr_grouped_splitk_gemm_tn(_p(X), _p(dY), K, M, N, _p(group_offsets), G, split_tokens, _p(partials),
                                         partials.shape[0], _p(slot_offsets), _p(ws), ws.numel(), _stream(stream)),
           "dr_grouped_splitk_gemm_tn")
    return partials, slot_offsets, ws


def dr_grouped_splitk_reduce(partials, slot_offsets, ws, *, out=None, stream=None):
    """out[g] = ordered tree over group g's slots (zero for an empty group); ws is the workspace the
    partials' call filled (it holds the slot table)."""
    _dev(partials, "partials", (torch.float32,))
    if partials.dim() < 1:
        raise ValueError("partials must be [slots, ...]")
    _sized(slot_offsets, "slot_offsets", partials.device, (torch.int32,), min_numel=2)
    _sized(ws, "ws", partials.device, (torch.uint8,), min_numel=_STATUS_BYTES)
    G = slot_offsets.numel() - 1
    count = partials[0].numel() if partials.shape[0] else 0
    if out is None:
        out = torch.empty((G,) + tuple(partials.shape[1:]), dtype=torch.float32, device=partials.device)
    else:
        _sized(out, "out", partials.device, (torch.float32,), numel=G * count)
    _check(lib.dr_grouped_splitk_reduce(_p(partials), partials.shape[0], _p(slot_offsets), G, count, _p(out),
                                        _p(ws), _stream(stream)), "dr_grouped_splitk_reduce")
    return out


def dr_grouped_wgrad_workspace_size(K: int, num_groups: int, split_tokens: int, M: int, N: int) -> int:
    return int(lib.dr_grouped_wgrad_workspace_size(K, num_groups, split_tokens, M, N))


def dr_grouped_wgrad(X, dY, group_offsets, split_tokens: int, *, out=None, ws=None, stream=None):
    """out[g] = ordered tree over group g's slot partials X_s^T dY_s (large M, N; partials kept in registers).
    Returns (out, ws)."""
    K, M, N = _gemm_args(X, dY)
    _sized(group_offsets, "group_offsets", X.device, (torch.int32,), min_numel=2)
    G = group_offsets.numel() - 1
    if out is None:
        out = torch.empty(G, M, N, dtype=torch.float32, device=X.device)
    else:
        _sized(out, "out", X.device, (torch.float32,), shape=(G, M, N))
    ws = _ws(ws, dr_grouped_wgrad_workspace_size(K, G, split_tokens, M, N), X.device)
    _check(lib.dr_grouped_wgrad(_p(X), _p(dY), K, M, N, _p(group_offsets), G, split_tokens, _p(out), _p(ws),
                                ws.numel(), _stream(stream)), "dr_grouped_wgrad")
    return out, ws


def dr_permute_rows(rows, perm, k: int, *, inv_perm=None, out=None, dev_status=None, stream=None):
    """out[r] = rows[perm[r] // k] (the expert-major copy of the token rows); with inv_perm the copies
    run in token order."""
    _dev(rows, "rows")
    if rows.dim() < 1:
        raise ValueError("rows must be [tokens, ...]")
    _sized(perm, "perm", rows.device, (torch.int32,))
    n = perm.numel()
    if inv_perm is not None:
        _sized(inv_perm, "inv_perm", rows.device, (torch.int32,), numel=n)
    row_bytes = rows[0].numel() * rows.element_size() if rows.shape[0] else 0
    shape = (n,) + tuple(rows.shape[1:])
    if out is None:
        out = torch.empty(shape, dtype=rows.dtype, device=rows.device)
    else:
        _sized(out, "out", rows.device, (rows.dtype,), shape=shape)
    _status_buf(dev_status, rows.device)
    _check(lib.dr_permute_rows(_p(rows), row_bytes, rows.shape[0], _p(perm), _p(inv_perm), n, k, _p(out),
                               _p(dev_status), _stream(stream)), "dr_permute_rows")
    return out


# ---------------------------------------------------------------------------
def dr_decode_attention_workspace_size(batch: int, num_q_heads: int, max_seq_len: int, kv_chunk: int,
                                       head_dim: int = 128) -> int:
    return int(lib.dr_decode_attention_workspace_size(batch, num_q_heads, max_seq_len, kv_chunk, head_dim))


DR_KV_TOKEN_MAJOR, DR_KV_HEAD_MAJOR = 0, 1


def dr_decode_attention(q, k_cache, v_cache, seq_lens, scale: float, kv_chunk: int, *, head_major: bool = False,
                        out=None, ws=None, dev_status=None, stream=None):
    """Decode attention of q [B, Hq, D] (bf16) over the caches (bf16; [B, Lmax, Hkv, D], or [B, Hkv, Lmax, D]
    with head_major) with a fixed KV partition of kv_chunk tokens; returns fp32 [B, Hq, D]."""
    _dev(q, "q", (torch.bfloat16,))
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _sized(t, name, q.device, (torch.bfloat16,))
    _sized(seq_lens, "seq_lens", q.device, (torch.int32,))
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, D] and the caches 4-D of one shape")
    B, Hq, D = q.shape
    Lmax, Hkv = (k_cache.shape[2], k_cache.shape[1]) if head_major else (k_cache.shape[1], k_cache.shape[2])
    if k_cache.shape[0] != B or k_cache.shape[3] != D or seq_lens.numel() != B:
        raise ValueError("batch or head_dim mismatch")
    out = _sized(out, "out", q.device, (torch.float32,), shape=(B, Hq, D)) if out is not None else \
        torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    ws = _ws(ws, dr_decode_attention_workspace_size(B, Hq, Lmax, kv_chunk, D), q.device)
    _status_buf(dev_status, q.device)
    layout = DR_KV_HEAD_MAJOR if head_major else DR_KV_TOKEN_MAJOR
    _check(lib.dr_decode_attention(_p(out), _p(q), _p(k_cache), _p(v_cache), layout, _p(seq_lens), B, Hq, Hkv, D,
                                   Lmax, float(scale), kv_chunk, _p(ws), ws.numel(), _p(dev_status),
                                   _stream(stream)),
           "dr_decode_attention")
    return out


def dr_decode_attention_occupancy_chunk(batch: int, num_kv_heads: int, max_seq_len: int) -> int:
    """The batch-dependent kv_chunk of an occupancy-driven split-KV heuristic (a deliberately batch-variant
    baseline)."""
    return int(lib.dr_decode_attention_occupancy_chunk(batch, num_kv_heads, max_seq_len))


# ---------------------------------------------------------------------------
def dr_fingerprint_workspace_size(nbytes: int) -> int:
    return int(lib.dr_fingerprint_workspace_size(nbytes))


def dr_fingerprint(t, *, out=None, ws=None, stream=None):
    """Device-side 64-bit fingerprint of t's bytes in logical order (an int64 tensor of one element)."""
    _dev(t, "tensor")
    nbytes = t.numel() * t.element_size()
    out = _hash_buf(out, "out", t.device) if out is not None else torch.empty(1, dtype=torch.int64, device=t.device)
    ws = _ws(ws, dr_fingerprint_workspace_size(nbytes), t.device)
    _check(lib.dr_fingerprint(_p(t), nbytes, _p(out), _p(ws), ws.numel(), _stream(stream)), "dr_fingerprint")
    return out


def fingerprint_value(t, stream=None) -> int:
    """The fingerprint as an unsigned Python int (synchronises)."""
    return int(dr_fingerprint(t, stream=stream).item()) & ((1 << 64) - 1)


def dr_workspace_status(ws, stream=None) -> None:
    """Raises DetReduceError if the device status word of a sort/index_add workspace is set."""
    _check(lib.dr_workspace_status(_p(ws), _stream(stream)), "device status")


def dr_read_status(dev_status, stream=None) -> None:
    _check(lib.dr_read_status(_p(dev_status), _stream(stream)), "device status")
