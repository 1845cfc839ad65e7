"""Seeded synthetic inputs for the five ordered scatter-reduce workloads.

This module is shared by the GPU tests, the bench and the CPU oracle's callers.
It draws inputs only: routing choices, gates, Zipf-distributed indices and
normal samples.  It performs none of the reduction's arithmetic (no sort of
contributions, no segment sums, no products) so that it can feed both sides of
a parity check without tying them together.

Every array is a pure function of (seed, shape parameters).  Large draws are
split into fixed blocks, each with its own PCG64 stream derived from
``SeedSequence([seed, tag, block])``, so the bits do not depend on how many
threads generate them.

Workload shapes follow the pages' use cases:
  * MoE token combine after expert computation (DeepSeek-V4 book, ch. 9,
    section 3.2 "MoE backward"; Megatron-LM determinism reference, section 3.1
    op catalog, MoE token unpermute row),
  * sparse-attention backward key gradient (DeepSeek-V4 book, ch. 9,
    section 3.1),
  * embedding gradient (Megatron-LM determinism reference, section 3.1,
    vocab-parallel embedding row),
  * thin split-K contraction with per-split buffers (DeepSeek-V4 book, ch. 9,
    section 3.3 "mHC backward"),
  * decode attention over a KV cache (DeepSeek-V4 book, ch. 9, section 2.1);
    the pages give no attention shape, so a common grouped-query one is used.
No public dataset is involved; these synthetic draws stand in for activations
and gradients of a real model.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_BLOCK = 1 << 22  # elements per independently seeded block


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _block_rng(seed: int, tag: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, block])))


def normal_f32(seed: int, tag: int, n: int, scale: float = 1.0) -> np.ndarray:
    """n samples of N(0, scale^2) as float32, generated block-wise in threads."""
    out = np.empty(n, dtype=np.float32)
    nblocks = (n + _BLOCK - 1) // _BLOCK

    def fill(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        rng = _block_rng(seed, tag, b)
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if scale != 1.0:
            out[lo:hi] *= np.float32(scale)

    if nblocks <= 1:
        for b in range(nblocks):
            fill(b)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16.  Inputs must be finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16_bits expects finite inputs")
    u = a.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    n = flat_u.size

    def conv(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        x = flat_u[lo:hi]
        flat_o[lo:hi] = ((x + np.uint32(0x7FFF) + ((x >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)

    nblocks = (n + _BLOCK - 1) // _BLOCK
    if nblocks <= 1:
        for b in range(nblocks):
            conv(b)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(conv, range(nblocks)))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tag: int, n: int, scale: float = 1.0) -> np.ndarray:
    return bf16_bits(normal_f32(seed, tag, n, scale))


def zipf_weights(count: int, s: float) -> np.ndarray:
    """Unnormalised weights (id+1)^-s for ids 0..count-1 (float64)."""
    return np.arange(1, count + 1, dtype=np.float64) ** (-s)


# --------------------------------------------------------------------------
# MoE combine (configurations "tiny MoE combine" and "MoE unpermute/combine")
# --------------------------------------------------------------------------
@dataclass
class MoeInputs:
    T: int
    E: int
    k: int
    H: int
    rows_dtype: str                   # "f32" or "bf16"
    expert_ids: np.ndarray            # int32 [T, k], distinct per token
    gates: np.ndarray                 # float32 [T, k]
    rows: np.ndarray                  # float32 [T*k, H] or uint16 (bf16 bits) [T*k, H]
    meta: dict = field(default_factory=dict)


def moe_routing(seed: int, T: int, E: int, k: int, zipf_bias_s: float | None) -> tuple[np.ndarray, np.ndarray]:
    """Top-k routing with softmax gates over the chosen logits.

    logits = N(0,1) [T, E] (+ bias_e = -s*ln(e+1) when a Zipf bias is given);
    the k largest logits per token are chosen (ties go to the lower expert id),
    and the gates are the softmax of the chosen logits, rounded to float32.
    """
    rng = _block_rng(seed, 1, 0)
    logits = rng.standard_normal((T, E))
    if zipf_bias_s is not None:
        logits = logits + (-zipf_bias_s * np.log(np.arange(1, E + 1, dtype=np.float64)))[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(logits, order, axis=1)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    gates = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int32), gates


def moe_inputs(seed: int, T: int, E: int, k: int, H: int, rows_dtype: str,
               zipf_bias_s: float | None = None) -> MoeInputs:
    """Expert outputs are N(0,1) rows, one per (token, slot) assignment.

    The rows are laid out in the expert-major order that the dispatch sort
    defines; the values themselves are i.i.d., so they are drawn here without
    reference to that order, and the caller builds ``row_of`` with its own sort.
    """
    expert_ids, gates = moe_routing(seed, T, E, k, zipf_bias_s)
    if rows_dtype == "f32":
        rows = normal_f32(seed, 2, T * k * H).reshape(T * k, H)
    elif rows_dtype == "bf16":
        rows = normal_bf16(seed, 2, T * k * H).reshape(T * k, H)
    else:
        raise ValueError(rows_dtype)
    return MoeInputs(T, E, k, H, rows_dtype, expert_ids, gates, rows)


# --------------------------------------------------------------------------
# Sparse-attention backward key-gradient index_add
# --------------------------------------------------------------------------
@dataclass
class IndexAddInputs:
    n: int
    D: int
    H: int
    src_dtype: str
    index: np.ndarray      # int32 [n]
    src: np.ndarray        # uint16 bf16 bits [n, H] or float32 [n, H]
    out0: np.ndarray       # float32 [D, H] initial destination contents
    meta: dict = field(default_factory=dict)


def sparse_attn_keys(seed: int, Q: int, K: int, S: int, s: float) -> np.ndarray:
    """Per query, S distinct key ids drawn without replacement with P ~ (id+1)^-s.

    Gumbel-top-k: the S largest log(w) + Gumbel noise.  Each query's ids are
    returned in ascending order.  int32 [Q, S].
    """
    logw = np.log(zipf_weights(K, s))
    out = np.empty((Q, S), dtype=np.int32)
    qb = 64

    def fill(b: int) -> None:
        lo, hi = b * qb, min(Q, (b + 1) * qb)
        rng = _block_rng(seed, 3, b)
        u = rng.random((hi - lo, K))
        g = logw[None, :] - np.log(-np.log(u))
        top = np.argpartition(-g, S - 1, axis=1)[:, :S]
        out[lo:hi] = np.sort(top, axis=1)

    nb = (Q + qb - 1) // qb
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(nb)))
    return out


def sparse_attn_inputs(seed: int, Q: int = 8192, K: int = 65536, S: int = 512, H: int = 128,
                       s: float = 1.1, src_scale: float = 0.1) -> IndexAddInputs:
    """Contribution i = q*S + j carries dK-row gradient of query q to key index[i]."""
    keys = sparse_attn_keys(seed, Q, K, S, s)
    n = Q * S
    src = normal_bf16(seed, 4, n * H, src_scale).reshape(n, H)
    out0 = normal_f32(seed, 5, K * H).reshape(K, H)
    return IndexAddInputs(n, K, H, "bf16", keys.reshape(-1), src, out0, {"Q": Q, "S": S})


@dataclass
class SparseAttnDkInputs:
    nq: int
    num_keys: int
    H: int
    key_idx: np.ndarray    # int32 [nq, topk]
    Q: np.ndarray          # uint16 bf16 bits [nq, H]
    dS: np.ndarray         # float32 [nq, topk]
    dK0: np.ndarray        # float32 [num_keys, H]


def sparse_attn_dk_inputs(seed: int, Q: int = 8192, K: int = 65536, S: int = 512, H: int = 128,
                          s: float = 1.1, ds_scale: float = 0.1) -> SparseAttnDkInputs:
    """The same key selection as sparse_attn_inputs, with the query rows (bf16
    N(0,1)) and score gradients (fp32 N(0, ds_scale^2)) instead of
    materialised contribution rows."""
    keys = sparse_attn_keys(seed, Q, K, S, s)
    q = normal_bf16(seed, 11, Q * H).reshape(Q, H)
    ds = normal_f32(seed, 12, Q * S, ds_scale).reshape(Q, S)
    dk0 = normal_f32(seed, 5, K * H).reshape(K, H)
    return SparseAttnDkInputs(Q, K, H, keys, q, ds, dk0)


def embedding_grad_inputs(seed: int, tokens: int = 8 * 4096, V: int = 131072, H: int = 4096,
                          s: float = 1.1, preset_out: bool = True) -> IndexAddInputs:
    """Token ids i.i.d. with P ~ (id+1)^-s; bf16 upstream gradients N(0,1)."""
    rng = _block_rng(seed, 6, 0)
    w = zipf_weights(V, s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    ids = np.searchsorted(cdf, rng.random(tokens), side="right").astype(np.int32)
    np.minimum(ids, V - 1, out=ids)
    src = normal_bf16(seed, 7, tokens * H).reshape(tokens, H)
    out0 = normal_f32(seed, 8, V * H).reshape(V, H) if preset_out else np.zeros((V, H), np.float32)
    return IndexAddInputs(tokens, V, H, "bf16", ids, src, out0, {})


# --------------------------------------------------------------------------
# Split-K thin contraction
# --------------------------------------------------------------------------
@dataclass
class SplitKInputs:
    K: int
    M: int
    N: int
    splits: int
    X: np.ndarray    # uint16 bf16 bits [K, M]
    dY: np.ndarray   # uint16 bf16 bits [K, N]


def splitk_inputs(seed: int, K: int = 16384, M: int = 7168, N: int = 24, splits: int = 64) -> SplitKInputs:
    X = normal_bf16(seed, 9, K * M).reshape(K, M)
    dY = normal_bf16(seed, 10, K * N).reshape(K, N)
    return SplitKInputs(K, M, N, splits, X, dY)


# --------------------------------------------------------------------------
# Grouped expert weight gradient
# --------------------------------------------------------------------------
@dataclass
class GroupedWgradInputs:
    K: int
    M: int
    N: int
    split_tokens: int
    group_offsets: np.ndarray  # int32 [G + 1]
    X: np.ndarray              # uint16 bf16 bits [K, M]: the experts' token rows, expert-major
    dY: np.ndarray             # uint16 bf16 bits [K, N]: the gradient of the expert layer's output


def grouped_wgrad_inputs(seed: int, experts: int = 8, M: int = 7168, N: int = 2048, split_tokens: int = 2048,
                         T: int = 16384, E: int = 256, k: int = 8, zipf_bias_s: float = 1.2) -> GroupedWgradInputs:
    """The hottest `experts` experts of the MoE routing (one GPU's share at expert parallelism E / experts),
    with their token counts from that routing; X and dY bf16 N(0,1)."""
    expert_ids, _ = moe_routing(seed, T, E, k, zipf_bias_s)
    counts = np.bincount(expert_ids.reshape(-1), minlength=E)[:experts]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    K = int(off[-1])
    X = normal_bf16(seed, 17, K * M).reshape(K, M)
    dY = normal_bf16(seed, 18, K * N).reshape(K, N)
    return GroupedWgradInputs(K, M, N, split_tokens, off, X, dY)


# --------------------------------------------------------------------------
# The five named configurations (full sizes); seed = 1000 + configuration number
# --------------------------------------------------------------------------
CONFIGS = {
    "tiny_moe_combine": dict(kind="moe", seed=1001, T=256, E=8, k=2, H=128, rows_dtype="f32", zipf_bias_s=None),
    "moe_combine": dict(kind="moe", seed=1002, T=16384, E=256, k=8, H=7168, rows_dtype="bf16", zipf_bias_s=1.2),
    "sparse_attn_dk": dict(kind="sparse_attn", seed=1003, Q=8192, K=65536, S=512, H=128, s=1.1),
    "embedding_grad": dict(kind="embedding", seed=1004, tokens=32768, V=131072, H=4096, s=1.1),
    "splitk_mhc": dict(kind="splitk", seed=1005, K=16384, M=7168, N=24, splits=64),
    "decode_attention": dict(kind="decode", seed=1006, B=64, Lmax=16384, Hq=32, Hkv=8, D=128),
}


# --------------------------------------------------------------------------
# Decode attention
# --------------------------------------------------------------------------
BF16_NAN = 0x7FC0  # fills cache rows past a sequence's length: they must never be read


@dataclass
class DecodeInputs:
    B: int
    Lmax: int
    Hq: int
    Hkv: int
    D: int
    scale: float
    lens: np.ndarray   # int32 [B]
    q: np.ndarray      # uint16 bf16 bits [B, Hq, D]
    k: np.ndarray      # uint16 bf16 bits [B, Lmax, Hkv, D]
    v: np.ndarray


def decode_inputs(seed: int, B: int = 64, Lmax: int = 16384, Hq: int = 32, Hkv: int = 8, D: int = 128,
                  lens=None) -> DecodeInputs:
    """Sequence lengths uniform in [1, Lmax] (unless given); q, K and V bf16
    N(0,1); scale 1/sqrt(D).  Cache rows at or past a sequence's length hold
    NaN."""
    if lens is None:
        lens = _block_rng(seed, 13, 0).integers(1, Lmax + 1, size=B)
    lens = np.asarray(lens, np.int32)
    q = normal_bf16(seed, 14, B * Hq * D).reshape(B, Hq, D)
    k = normal_bf16(seed, 15, B * Lmax * Hkv * D).reshape(B, Lmax, Hkv, D)
    v = normal_bf16(seed, 16, B * Lmax * Hkv * D).reshape(B, Lmax, Hkv, D)
    for b in range(B):
        k[b, lens[b]:] = BF16_NAN
        v[b, lens[b]:] = BF16_NAN
    return DecodeInputs(B, Lmax, Hq, Hkv, D, float(1.0 / np.sqrt(D)), lens, q, k, v)


def make(name: str, **overrides):
    """Build the inputs of a named configuration, optionally with smaller shapes."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    seed = cfg.pop("seed")
    if kind == "moe":
        return moe_inputs(seed, cfg["T"], cfg["E"], cfg["k"], cfg["H"], cfg["rows_dtype"], cfg["zipf_bias_s"])
    if kind == "sparse_attn":
        return sparse_attn_inputs(seed, cfg["Q"], cfg["K"], cfg["S"], cfg["H"], cfg["s"])
    if kind == "embedding":
        return embedding_grad_inputs(seed, cfg["tokens"], cfg["V"], cfg["H"], cfg["s"], cfg.get("preset_out", True))
    if kind == "splitk":
        return splitk_inputs(seed, cfg["K"], cfg["M"], cfg["N"], cfg["splits"])
    if kind == "decode":
        return decode_inputs(seed, cfg["B"], cfg["Lmax"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg.get("lens"))
    raise ValueError(kind)
