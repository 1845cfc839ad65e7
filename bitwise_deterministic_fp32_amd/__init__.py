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
    "dr_index_add_workspace_size", "dr_index_add", "dr_index_add_fingerprinted", "dr_index_add_atomic",
    "dr_sparse_attn_dk_workspace_size", "dr_sparse_attn_dk",
    "dr_splitk_gemm_tn", "dr_splitk_gemm_tn_atomic", "dr_splitk_reduce",
    "dr_splitk_reduce_fingerprinted_workspace_size", "dr_splitk_reduce_fingerprinted",
    "dr_grouped_splitk_max_slots", "dr_grouped_splitk_workspace_size", "dr_grouped_splitk_gemm_tn",
    "dr_grouped_splitk_reduce", "dr_permute_rows",
    "dr_decode_attention_workspace_size", "dr_decode_attention", "dr_decode_attention_occupancy_chunk",
    "dr_fingerprint_workspace_size", "dr_fingerprint", "fingerprint_value",
    "dr_workspace_status", "dr_read_status",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdetreduce.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "detreduce.h")

DR_F32, DR_BF16 = 0, 1
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
                ("sort_tile_log2", ctypes.c_int32), ("chunks_in_flight", ctypes.c_int32)]


def dr_set_launch_params(grid_blocks: int = 0, tile_chunks_log2: int = 0, sort_tile_log2: int = 0,
                         chunks_in_flight: int = 0, reset: bool = False) -> None:
    """Thread-local launch overrides (tests of launch invariance); reset=True restores defaults."""
    if reset:
        _check(lib.dr_set_launch_params(None), "dr_set_launch_params")
        return
    p = _LaunchParams(grid_blocks, tile_chunks_log2, sort_tile_log2, chunks_in_flight)
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
        _dev(src_id, "src_id", (torch.int32,))
    perm = perm if perm is not None else torch.empty(n, dtype=torch.int32, device=dev)
    seg_offsets = seg_offsets if seg_offsets is not None else torch.empty(num_dests + 1, dtype=torch.int32, device=dev)
    if inv_perm is None and want_inv:
        inv_perm = torch.empty(n, dtype=torch.int32, device=dev)
    need = dr_sort_workspace_size(n, num_dests, src_id_bound if src_id is not None else 0)
    ws = ws if ws is not None else _workspace(need, dev)
    _check(lib.dr_sort_by_dest(_p(dest), _p(src_id), src_id_bound, n, num_dests, _p(perm), _p(seg_offsets),
                               _p(inv_perm), _p(ws), ws.numel(), _stream(stream)), "dr_sort_by_dest")
    return perm, seg_offsets, inv_perm


def _combine_args(rows, row_of, gates):
    _dev(rows, "rows", tuple(_DTYPES))
    _dev(row_of, "row_of", (torch.int32,))
    _dev(gates, "gates", (torch.float32,))
    if rows.dim() != 2 or row_of.dim() != 2 or gates.shape != row_of.shape:
        raise ValueError("rows must be [R, H]; row_of and gates [T, k]")
    return rows.shape[0], rows.shape[1], row_of.shape[0], row_of.shape[1]


def dr_combine(rows, row_of, gates, *, out=None, dev_status=None, stream=None):
    """out[t] = ordered tree over fl32(gate * row) of the token's k rows (written)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    out = out if out is not None else torch.empty(T, H, dtype=torch.float32, device=rows.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.dr_combine(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k, _p(out),
                          _p(dev_status), _stream(stream)), "dr_combine")
    return out


def dr_combine_fingerprinted_workspace_size(rows_dtype, hidden: int, T: int) -> int:
    return int(lib.dr_combine_fingerprinted_workspace_size(_DTYPES[rows_dtype], hidden, T))


def dr_combine_fingerprinted(rows, row_of, gates, *, out=None, out_hash=None, ws=None, dev_status=None, stream=None):
    """dr_combine plus the fingerprint of its output, hashed as it is stored.  Returns (out, out_hash)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    out = out if out is not None else torch.empty(T, H, dtype=torch.float32, device=rows.device)
    _dev(out, "out", (torch.float32,))
    out_hash = out_hash if out_hash is not None else torch.empty(1, dtype=torch.int64, device=rows.device)
    ws = ws if ws is not None else _workspace(dr_combine_fingerprinted_workspace_size(rows.dtype, H, T), rows.device)
    _check(lib.dr_combine_fingerprinted(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k, _p(out),
                                        _p(out_hash), _p(ws), ws.numel(), _p(dev_status), _stream(stream)),
           "dr_combine_fingerprinted")
    return out, out_hash


def dr_combine_atomic(rows, row_of, gates, *, out, dev_status=None, stream=None):
    """Nondeterministic baseline: atomically adds each fl32(gate * row) into out (caller zeroes it)."""
    R, H, T, k = _combine_args(rows, row_of, gates)
    _dev(out, "out", (torch.float32,))
    _check(lib.dr_combine_atomic(_p(rows), _DTYPES[rows.dtype], R, H, _p(row_of), _p(gates), T, k, _p(out),
                                 _p(dev_status), _stream(stream)), "dr_combine_atomic")
    return out


# ---------------------------------------------------------------------------
def dr_index_add_workspace_size(n: int, num_dests: int, hidden: int) -> int:
    return int(lib.dr_index_add_workspace_size(n, num_dests, hidden))


def dr_index_add(out, src, index, *, perm=None, seg_offsets=None, ws=None, stream=None):
    """out[d] += ordered tree of src rows i with index[i] == d (in place).  Returns (out, ws)."""
    _dev(out, "out", (torch.float32,))
    _dev(src, "src", tuple(_DTYPES))
    _dev(index, "index", (torch.int32,))
    D, H = out.shape
    n = index.numel()
    if src.shape != (n, H):
        raise ValueError(f"src must be [{n}, {H}], got {tuple(src.shape)}")
    ws = ws if ws is not None else _workspace(dr_index_add_workspace_size(n, D, H), out.device)
    _check(lib.dr_index_add(_p(out), D, H, _p(src), _DTYPES[src.dtype], n, _p(index), _p(perm), _p(seg_offsets),
                            _p(ws), ws.numel(), _stream(stream)), "dr_index_add")
    return out, ws


def dr_index_add_fingerprinted(out, src, index, inout_hash, *, perm=None, seg_offsets=None, ws=None, stream=None):
    """dr_index_add that moves inout_hash (an int64 device tensor of one element holding the fingerprint of
    out) to the fingerprint of the updated out.  Returns (out, ws)."""
    _dev(out, "out", (torch.float32,))
    _dev(src, "src", tuple(_DTYPES))
    _dev(index, "index", (torch.int32,))
    _dev(inout_hash, "inout_hash", (torch.int64,))
    if inout_hash.numel() != 1:
        raise ValueError("inout_hash must hold one element")
    D, H = out.shape
    n = index.numel()
    if src.shape != (n, H):
        raise ValueError(f"src must be [{n}, {H}], got {tuple(src.shape)}")
    ws = ws if ws is not None else _workspace(dr_index_add_workspace_size(n, D, H), out.device)
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
    _dev(Q, "Q", tuple(_DTYPES))
    _dev(dS, "dS", (torch.float32,))
    _dev(key_idx, "key_idx", (torch.int32,))
    K, H = dK.shape
    nq, topk = key_idx.shape
    if Q.shape != (nq, H) or dS.shape != (nq, topk):
        raise ValueError(f"Q must be [{nq}, {H}] and dS [{nq}, {topk}], got {tuple(Q.shape)} and {tuple(dS.shape)}")
    ws = ws if ws is not None else _workspace(dr_sparse_attn_dk_workspace_size(nq, topk, K, H), dK.device)
    _check(lib.dr_sparse_attn_dk(_p(dK), K, H, _p(Q), _DTYPES[Q.dtype], _p(dS), _p(key_idx), nq, topk, _p(perm),
                                 _p(seg_offsets), _p(ws), ws.numel(), _stream(stream)), "dr_sparse_attn_dk")
    return dK, ws


def dr_index_add_atomic(out, src, index, *, dev_status=None, stream=None):
    _dev(out, "out", (torch.float32,))
    _dev(src, "src", tuple(_DTYPES))
    _dev(index, "index", (torch.int32,))
    D, H = out.shape
    n = index.numel()
    _check(lib.dr_index_add_atomic(_p(out), D, H, _p(src), _DTYPES[src.dtype], n, _p(index), _p(dev_status),
                                   _stream(stream)), "dr_index_add_atomic")
    return out


# ---------------------------------------------------------------------------
def dr_splitk_gemm_tn(X, dY, splits: int, *, partials=None, stream=None):
    """partials[s] = X_s^T dY_s (bf16 MFMA into fp32), one private buffer per split."""
    _dev(X, "X", (torch.bfloat16,))
    _dev(dY, "dY", (torch.bfloat16,))
    K, M = X.shape
    N = dY.shape[1]
    partials = partials if partials is not None else torch.empty(splits, M, N, dtype=torch.float32, device=X.device)
    _dev(partials, "partials", (torch.float32,))
    _check(lib.dr_splitk_gemm_tn(_p(X), _p(dY), K, M, N, splits, _p(partials), _stream(stream)), "dr_splitk_gemm_tn")
    return partials


def dr_splitk_gemm_tn_atomic(X, dY, splits: int, *, out, stream=None):
    _dev(X, "X", (torch.bfloat16,))
    _dev(dY, "dY", (torch.bfloat16,))
    _dev(out, "out", (torch.float32,))
    K, M = X.shape
    N = dY.shape[1]
    _check(lib.dr_splitk_gemm_tn_atomic(_p(X), _p(dY), K, M, N, splits, _p(out), _stream(stream)),
           "dr_splitk_gemm_tn_atomic")
    return out


def dr_splitk_reduce(partials, *, out=None, stream=None):
    """out = ordered tree over the split axis of partials [S, ...]."""
    _dev(partials, "partials", (torch.float32,))
    S = partials.shape[0]
    count = partials.numel() // S
    out = out if out is not None else torch.empty(partials.shape[1:], dtype=torch.float32, device=partials.device)
    _dev(out, "out", (torch.float32,))
    _check(lib.dr_splitk_reduce(_p(partials), S, count, _p(out), _stream(stream)), "dr_splitk_reduce")
    return out


def dr_splitk_reduce_fingerprinted_workspace_size(splits: int, count: int) -> int:
    return lib.dr_splitk_reduce_fingerprinted_workspace_size(splits, count)


def dr_splitk_reduce_fingerprinted(partials, out_hash, *, out=None, ws=None, stream=None):
    """dr_splitk_reduce that also writes dr_fingerprint(out) to out_hash (int64 [1] on the device)."""
    _dev(partials, "partials", (torch.float32,))
    _dev(out_hash, "out_hash", (torch.int64,))
    S = partials.shape[0]
    count = partials.numel() // S
    out = out if out is not None else torch.empty(partials.shape[1:], dtype=torch.float32, device=partials.device)
    _dev(out, "out", (torch.float32,))
    need = dr_splitk_reduce_fingerprinted_workspace_size(S, count)
    ws = ws if ws is not None else _workspace(need, partials.device)
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
    _dev(X, "X", (torch.bfloat16,))
    _dev(dY, "dY", (torch.bfloat16,))
    _dev(group_offsets, "group_offsets", (torch.int32,))
    K, M = X.shape
    N = dY.shape[1]
    G = group_offsets.numel() - 1
    S = dr_grouped_splitk_max_slots(K, G, split_tokens)
    partials = partials if partials is not None else torch.empty(S, M, N, dtype=torch.float32, device=X.device)
    slot_offsets = slot_offsets if slot_offsets is not None else torch.empty(G + 1, dtype=torch.int32,
                                                                            device=X.device)
    ws = ws if ws is not None else _workspace(dr_grouped_splitk_workspace_size(K, G, split_tokens), X.device)
    _dev(partials, "partials", (torch.float32,))
    _check(lib.dr_grouped_splitk_gemm_tn(_p(X), _p(dY), K, M, N, _p(group_offsets), G, split_tokens, _p(partials),
                                         partials.shape[0], _p(slot_offsets), _p(ws), ws.numel(), _stream(stream)),
           "dr_grouped_splitk_gemm_tn")
    return partials, slot_offsets, ws


def dr_grouped_splitk_reduce(partials, slot_offsets, ws, *, out=None, stream=None):
    """out[g] = ordered tree over group g's slots (zero for an empty group)."""
    _dev(partials, "partials", (torch.float32,))
    G = slot_offsets.numel() - 1
    count = partials[0].numel() if partials.shape[0] else 0
    out = out if out is not None else torch.empty((G,) + tuple(partials.shape[1:]), dtype=torch.float32,
                                                  device=partials.device)
    _check(lib.dr_grouped_splitk_reduce(_p(partials), partials.shape[0], _p(slot_offsets), G, count, _p(out),
                                        _p(ws), _stream(stream)), "dr_grouped_splitk_reduce")
    return out


def dr_permute_rows(rows, perm, k: int, *, inv_perm=None, out=None, dev_status=None, stream=None):
    """out[r] = rows[perm[r] // k] (the expert-major copy of the token rows); with inv_perm the copies
    run in token order."""
    _dev(perm, "perm", (torch.int32,))
    if rows.device.type != "cuda" or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous CUDA tensor")
    n = perm.numel()
    row_bytes = rows[0].numel() * rows.element_size() if rows.shape[0] else 0
    out = out if out is not None else torch.empty((n,) + tuple(rows.shape[1:]), dtype=rows.dtype, device=rows.device)
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
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, name, (torch.bfloat16,))
    _dev(seq_lens, "seq_lens", (torch.int32,))
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, D] and the caches 4-D of one shape")
    B, Hq, D = q.shape
    Lmax, Hkv = (k_cache.shape[2], k_cache.shape[1]) if head_major else (k_cache.shape[1], k_cache.shape[2])
    if k_cache.shape[0] != B or k_cache.shape[3] != D or seq_lens.numel() != B:
        raise ValueError("batch or head_dim mismatch")
    out = out if out is not None else torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    ws = ws if ws is not None else _workspace(dr_decode_attention_workspace_size(B, Hq, Lmax, kv_chunk, D), q.device)
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
    out = out if out is not None else torch.empty(1, dtype=torch.int64, device=t.device)
    ws = ws if ws is not None else _workspace(dr_fingerprint_workspace_size(nbytes), t.device)
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
