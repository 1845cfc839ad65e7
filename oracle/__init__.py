"""Python access to the CPU oracle (oracle.c) through ctypes.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
CPU-baseline leg import this package.  The product library and its Python
binding never import it, and it imports nothing from them.

All functions take and return numpy arrays on the host.  bfloat16 data is
passed as its raw 16-bit patterns (uint16 arrays).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Flags that keep float arithmetic exactly IEEE binary32 with round-to-nearest:
# no contraction into fused multiply-add, no reassociation, no excess precision.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-msse2", "-mfpmath=sse", "-pthread", "-Wall", "-Wextra"]

F32, BF16 = 0, 1
ERRORS = {0: "ok", 1: "bad argument", 4: "index out of range", 6: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i64, i32, vp, u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64
        L.oracle_tree_sum_f32.argtypes = [vp, i64, vp]
        L.oracle_tree_sum_bf16.argtypes = [vp, i64, vp]
        L.oracle_sort_by_dest.argtypes = [vp, vp, i64, i32, vp, vp, vp]
        L.oracle_scatter_reduce.argtypes = [vp, i32, i64, vp, ctypes.c_int, i64, vp, vp, vp, i64, i32]
        L.oracle_combine.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, i64, i32, vp, i64, vp, i32]
        L.oracle_sparse_attn_dk.argtypes = [vp, i32, i64, vp, ctypes.c_int, vp, vp, i64, i32, vp, i64, i32]
        L.oracle_splitk_reduce.argtypes = [vp, i32, i64, vp]
        L.oracle_splitk_reference.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        L.oracle_splitk_partials.argtypes = [vp, vp, i64, i64, i64, i32, vp]
        L.oracle_splitmix64_mix.argtypes = [u64]
        L.oracle_splitmix64_mix.restype = u64
        L.oracle_fingerprint.argtypes = [vp, i64]
        L.oracle_fingerprint.restype = u64
        for name in ("oracle_tree_sum_f32", "oracle_tree_sum_bf16", "oracle_sort_by_dest",
                     "oracle_scatter_reduce", "oracle_combine", "oracle_sparse_attn_dk", "oracle_splitk_reduce",
                     "oracle_splitk_reference", "oracle_splitk_partials"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what}: {ERRORS.get(rc, rc)}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def tree_sum_f32(v) -> np.float32:
    v = _c(v, np.float32)
    out = np.zeros(1, np.float32)
    _check(lib().oracle_tree_sum_f32(_ptr(v), v.size, _ptr(out)), "tree_sum_f32")
    return out[0]


def tree_sum_bf16(bits) -> int:
    v = _c(bits, np.uint16)
    out = np.zeros(1, np.uint16)
    _check(lib().oracle_tree_sum_bf16(_ptr(v), v.size, _ptr(out)), "tree_sum_bf16")
    return int(out[0])


def sort_by_dest(dest, num_dests: int, src_id=None):
    """Returns (perm, seg_offsets, inv_perm) as int32 arrays."""
    dest = _c(dest, np.int32)
    n = dest.size
    src = None if src_id is None else _c(src_id, np.int32)
    perm = np.empty(n, np.int32)
    seg = np.empty(num_dests + 1, np.int32)
    inv = np.empty(n, np.int32)
    _check(lib().oracle_sort_by_dest(_ptr(dest), _ptr(src), n, num_dests, _ptr(perm), _ptr(seg), _ptr(inv)),
           "sort_by_dest")
    return perm, seg, inv


def _dtype_code(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported source dtype {a.dtype}")


def scatter_reduce(out0, src, index, src_id=None, dests=None, threads: int = 1):
    """out[d] = out0[d] + T(contributions of d in (src_id, position) order).

    out0: float32 [D, H].  src: float32 or uint16 (bf16 bits) [n, H].
    dests: optional list of destination ids; then only those rows are returned
    (shape [len(dests), H]) and out0 is only read at those rows.
    threads: host threads sharing the destination rows (the result does not
    depend on it).
    """
    out0 = np.asarray(out0, dtype=np.float32)
    D, H = out0.shape
    src = np.ascontiguousarray(src)
    index = _c(index, np.int32)
    n = index.size
    assert src.shape == (n, H), (src.shape, n, H)
    sid = None if src_id is None else _c(src_id, np.int32)
    if dests is None:
        out = np.array(out0, dtype=np.float32, copy=True, order="C")
        dl, nd = None, 0
    else:
        dl = _c(dests, np.int32)
        nd = dl.size
        out = np.ascontiguousarray(out0[dl], dtype=np.float32)
    _check(lib().oracle_scatter_reduce(_ptr(out), D, H, _ptr(src), _dtype_code(src), n, _ptr(index),
                                       _ptr(sid), _ptr(dl), nd, int(threads)), "scatter_reduce")
    return out


def index_add(out0, src, index, dests=None, threads: int = 1):
    """torch-style index_add_(0, index, src) in the defined order (source id = row i)."""
    return scatter_reduce(out0, src, index, None, dests, threads)


def sparse_attn_dk(dK0, Q, dS, key_idx, keys=None, threads: int = 1):
    """dK[key] = dK0[key] + T(fl32(dS[q, j] * Q[q]) over the (q, j) with key_idx[q, j] == key, in order of
    q * topk + j).  Q: float32 or uint16 (bf16 bits) [nq, H]; dS: float32 [nq, topk]; key_idx: int32 [nq, topk].
    keys: optional list of keys; then only those rows are returned."""
    dK0 = np.asarray(dK0, dtype=np.float32)
    num_keys, H = dK0.shape
    Q = np.ascontiguousarray(Q)
    dS = _c(dS, np.float32)
    key_idx = _c(key_idx, np.int32)
    nq, topk = key_idx.shape
    assert Q.shape == (nq, H) and dS.shape == (nq, topk), (Q.shape, dS.shape, key_idx.shape)
    if keys is None:
        out = np.array(dK0, dtype=np.float32, copy=True, order="C")
        kl, nk = None, 0
    else:
        kl = _c(keys, np.int32)
        nk = kl.size
        out = np.ascontiguousarray(dK0[kl], dtype=np.float32)
    _check(lib().oracle_sparse_attn_dk(_ptr(out), num_keys, H, _ptr(Q), _dtype_code(Q), _ptr(dS), _ptr(key_idx),
                                       nq, topk, _ptr(kl), nk, int(threads)), "sparse_attn_dk")
    return out


def combine(rows, row_of, gates, tokens=None, threads: int = 1):
    """out[t] = T(fl32(gate*row) over the token's slots, ordered by row index)."""
    rows = np.ascontiguousarray(rows)
    R, H = rows.shape
    row_of = _c(row_of, np.int32)
    gates = _c(gates, np.float32)
    T, k = row_of.shape
    if tokens is None:
        tl, nt = None, T
    else:
        tl = _c(tokens, np.int64)
        nt = tl.size
    out = np.empty((nt, H), np.float32)
    _check(lib().oracle_combine(_ptr(rows), _dtype_code(rows), R, H, _ptr(row_of), _ptr(gates), T, k,
                                _ptr(tl), nt if tl is not None else 0, _ptr(out), int(threads)), "combine")
    return out


def splitk_reduce(partials):
    """partials: float32 [S, ...] -> float32 [...] reduced over the split axis by T."""
    p = _c(partials, np.float32)
    S = p.shape[0]
    count = p.size // S
    out = np.empty(p.shape[1:], np.float32)
    _check(lib().oracle_splitk_reduce(_ptr(p), S, count, _ptr(out)), "splitk_reduce")
    return out


def splitk_reference(X, dY):
    """fp64 (exact, absum) of X^T dY for bf16-bit inputs X [K, M], dY [K, N]."""
    X = _c(X, np.uint16)
    dY = _c(dY, np.uint16)
    K, M = X.shape
    N = dY.shape[1]
    exact = np.empty((M, N), np.float64)
    absum = np.empty((M, N), np.float64)
    _check(lib().oracle_splitk_reference(_ptr(X), _ptr(dY), K, M, N, _ptr(exact), _ptr(absum)),
           "splitk_reference")
    return exact, absum


def splitk_partials(X, dY, splits: int):
    X = _c(X, np.uint16)
    dY = _c(dY, np.uint16)
    K, M = X.shape
    N = dY.shape[1]
    P = np.empty((splits, M, N), np.float64)
    _check(lib().oracle_splitk_partials(_ptr(X), _ptr(dY), K, M, N, splits, _ptr(P)), "splitk_partials")
    return P


def grouped_slots(group_offsets, split_tokens: int):
    """The private slots of a grouped split: group g owns tokens
    [off[g], off[g+1]), cut into consecutive slots of split_tokens tokens from
    its first token (the last one short).  Returns (slot_offsets [G+1],
    slot token ranges [S, 2]), slots in (group, position) order."""
    off = np.asarray(group_offsets, dtype=np.int64)
    G = off.size - 1
    slot_off = [0]
    ranges = []
    for g in range(G):
        t = int(off[g])
        while t < off[g + 1]:
            ranges.append((t, min(int(off[g + 1]), t + split_tokens)))
            t += split_tokens
        slot_off.append(len(ranges))
    return np.array(slot_off, np.int32), np.array(ranges, np.int64).reshape(-1, 2)


def grouped_splitk_partials(X, dY, group_offsets, split_tokens: int):
    """fp64 (exact for bf16 inputs) X_s^T dY_s of every private slot s [S, M, N]."""
    X = _c(X, np.uint16)
    dY = _c(dY, np.uint16)
    _, ranges = grouped_slots(group_offsets, split_tokens)
    M, N = X.shape[1], dY.shape[1]
    P = np.empty((len(ranges), M, N), np.float64)
    for s, (a, b) in enumerate(ranges):
        P[s] = splitk_partials(X[a:b], dY[a:b], 1)[0]
    return P


def grouped_splitk_reduce(partials, slot_offsets):
    """out[g] = T(partials[slot_offsets[g]], ..., partials[slot_offsets[g+1]-1]) in slot order;
    a group with no slot (no tokens) has the zero gradient."""
    p = _c(partials, np.float32)
    so = np.asarray(slot_offsets, dtype=np.int64)
    G = so.size - 1
    out = np.zeros((G,) + p.shape[1:], np.float32)
    for g in range(G):
        if so[g + 1] > so[g]:
            out[g] = splitk_reduce(p[so[g]:so[g + 1]])
    return out


def permute_rows(x, perm, k: int):
    """Dispatch-side stable permute: out[r] = x[perm[r] // k] (bytes copied)."""
    x = np.ascontiguousarray(x)
    perm = np.asarray(perm, dtype=np.int64)
    return x[perm // k].copy()


def decode_attention(q, k_cache, v_cache, seq_lens, scale: float):
    """Decode attention, the operation that a batch-invariant decode kernel
    must evaluate with a KV partition that does not depend on the batch
    (DeepSeek-V4 book ch. 9, section 2.1, giving up occupancy-chosen split-KV).
    By its definition, in fp64: for sequence b and query
    head h (key/value head h // (Hq // Hkv)), with s_j = scale * q.k_j over the
    sequence's first seq_lens[b] cache rows,
        out[b, h] = sum_j softmax(s)_j v_j,     A[b, h] = sum_j softmax(s)_j |v_j|
    (A bounds the rounding error of any fp32 evaluation).  A sequence with no
    cached token has out = 0.  q: [B, Hq, D]; caches: [B, Lmax, Hkv, D]; float32
    or uint16 (bf16 bits)."""
    def f64(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            a = (a.astype(np.uint32) << 16).view(np.float32)
        return a.astype(np.float64)
    q = f64(q)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_cache).shape[2]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    A = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        kc, vc = f64(k_cache[b, :L]), f64(v_cache[b, :L])   # one sequence's cached rows
        for h in range(Hq):
            kk, vv = kc[:, h // g], vc[:, h // g]
            s_ = scale * (kk @ q[b, h])
            p_ = np.exp(s_ - s_.max())
            p_ /= p_.sum()
            out[b, h] = p_ @ vv
            A[b, h] = p_ @ np.abs(vv)
    return out, A


def splitmix64_mix(z: int) -> int:
    return int(lib().oracle_splitmix64_mix(ctypes.c_uint64(z & ((1 << 64) - 1))))


def fingerprint(data) -> int:
    """Fingerprint of an array's bytes in logical (C-contiguous) order."""
    b = np.ascontiguousarray(data)
    raw = b.view(np.uint8).reshape(-1) if b.size else np.zeros(0, np.uint8)
    buf = raw if raw.size else np.zeros(1, np.uint8)
    return int(lib().oracle_fingerprint(_ptr(buf), raw.size))
