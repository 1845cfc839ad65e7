"""CPU checks of the C-ABI library: it loads, exports every function the header
declares, and refuses bad arguments synchronously, before any GPU work (fail
closed).  No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bitwise_deterministic_fp32_amd", "libdetreduce.so")
HEADER = os.path.join(ROOT, "include", "detreduce.h")

DR_OK, DR_ERR_INVALID_ARGUMENT, DR_ERR_UNSUPPORTED, DR_ERR_WORKSPACE_TOO_SMALL = 0, 1, 2, 3
FAKE = 0x7F0000000000  # a 256-byte aligned address that is never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        build_module().build()
    L = ctypes.CDLL(LIB)
    L.dr_last_error.restype = ctypes.c_char_p
    L.dr_status_string.restype = ctypes.c_char_p
    return L


def build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_detreduce_build",
                                                  os.path.join(ROOT, "bitwise_deterministic_fp32_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dr_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared()
    for required in ("dr_sort_by_dest", "dr_combine", "dr_index_add", "dr_splitk_reduce", "dr_fingerprint",
                     "dr_combine_fingerprinted", "dr_sparse_attn_dk", "dr_decode_attention", "dr_index_add_fingerprinted",
                     "dr_combine_atomic", "dr_index_add_atomic", "dr_splitk_gemm_tn", "dr_splitk_gemm_tn_atomic"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(dr_\w+)$", out, flags=re.M))
    missing = [n for n in declared() if n not in exported]
    assert not missing, missing
    for n in declared():
        assert getattr(lib, n) is not None


def test_phase_events_hook(lib):
    f = lib.dr_set_phase_events
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, None) == DR_OK
    assert f(FAKE, None) == DR_ERR_INVALID_ARGUMENT
    assert f(None, FAKE) == DR_ERR_INVALID_ARGUMENT


def test_status_strings(lib):
    for code in range(7):
        assert lib.dr_status_string(code).decode().startswith("DR_")
    assert lib.dr_version() >= 100


def _err(lib):
    return lib.dr_last_error().decode()


def test_combine_rejects_bad_arguments(lib):
    f = lib.dr_combine
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    # hidden not a multiple of 8 for bf16
    assert f(FAKE, 1, 10, 100, FAKE, FAKE, 4, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT
    assert "multiple of 8" in _err(lib)
    # unknown dtype
    assert f(FAKE, 7, 10, 128, FAKE, FAKE, 4, 2, FAKE, None, None) == DR_ERR_UNSUPPORTED
    # k out of range
    assert f(FAKE, 0, 10, 128, FAKE, FAKE, 4, 65, FAKE, None, None) == DR_ERR_UNSUPPORTED
    assert f(FAKE, 0, 10, 128, FAKE, FAKE, 4, 0, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT
    # misaligned rows / out
    assert f(FAKE + 4, 0, 10, 128, FAKE, FAKE, 4, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE, 0, 10, 128, FAKE, FAKE, 4, 2, FAKE + 8, None, None) == DR_ERR_INVALID_ARGUMENT
    # null pointers with T > 0
    assert f(FAKE, 0, 10, 128, None, FAKE, 4, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT


def test_index_add_rejects_bad_arguments(lib):
    f = lib.dr_index_add
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    lib.dr_index_add_workspace_size.restype = ctypes.c_size_t
    lib.dr_index_add_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64]
    need = lib.dr_index_add_workspace_size(1000, 64, 128)
    assert need > 0
    # workspace too small
    assert f(FAKE, 64, 128, FAKE, 1, 1000, FAKE, None, None, FAKE, need - 1, None) == DR_ERR_WORKSPACE_TOO_SMALL
    # only one of perm / seg_offsets
    assert f(FAKE, 64, 128, FAKE, 1, 1000, FAKE, FAKE, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    # hidden not a multiple of 4 for fp32
    assert f(FAKE, 64, 130, FAKE, 0, 1000, FAKE, None, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    # bad sizes
    assert f(FAKE, 0, 128, FAKE, 1, 1000, FAKE, None, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE, 64, 128, FAKE, 1, -1, FAKE, None, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE, 64, 128, FAKE, 1, 1 << 31, FAKE, None, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    # misaligned workspace or out
    assert f(FAKE, 64, 128, FAKE, 1, 1000, FAKE, None, None, FAKE + 4, need, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE + 4, 64, 128, FAKE, 1, 1000, FAKE, None, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    # the fingerprinted form also needs an aligned hash word
    g = lib.dr_index_add_fingerprinted
    g.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    assert g(FAKE, 64, 128, FAKE, 1, 1000, FAKE, None, None, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    assert g(FAKE, 64, 128, FAKE, 1, 1000, FAKE, None, None, FAKE + 4, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    assert g(FAKE, 64, 128, FAKE, 1, 1000, FAKE, None, None, FAKE, FAKE, need - 1, None) == DR_ERR_WORKSPACE_TOO_SMALL
    assert g(FAKE, 64, 130, FAKE, 0, 1000, FAKE, None, None, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT


def test_sparse_attn_dk_rejects_bad_arguments(lib):
    f = lib.dr_sparse_attn_dk
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.dr_sparse_attn_dk_workspace_size.restype = ctypes.c_size_t
    lib.dr_sparse_attn_dk_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    lib.dr_index_add_workspace_size.restype = ctypes.c_size_t
    lib.dr_index_add_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64]
    need = lib.dr_sparse_attn_dk_workspace_size(100, 16, 512, 128)
    # the index_add workspace plus the two buffers the sort moves the 1600 scales through
    assert need >= lib.dr_index_add_workspace_size(1600, 512, 128) + 2 * 1600 * 4
    ok_args = (FAKE, 512, 128, FAKE, 1, FAKE, FAKE, 100, 16, None, None, FAKE, need, None)

    def call(**kw):
        names = ["dK", "K", "H", "Q", "dt", "dS", "idx", "nq", "topk", "perm", "seg", "ws", "wsb", "s"]
        args = dict(zip(names, ok_args))
        args.update(kw)
        return f(*[args[n] for n in names])

    assert call(wsb=need - 1) == DR_ERR_WORKSPACE_TOO_SMALL
    assert call(topk=0) == DR_ERR_INVALID_ARGUMENT
    assert call(nq=-1) == DR_ERR_INVALID_ARGUMENT
    assert call(nq=1 << 27, topk=16) == DR_ERR_INVALID_ARGUMENT      # 2^31 contributions
    assert call(dS=None) == DR_ERR_INVALID_ARGUMENT
    assert call(dS=FAKE + 2) == DR_ERR_INVALID_ARGUMENT
    assert call(Q=FAKE + 8) == DR_ERR_INVALID_ARGUMENT               # 16-byte aligned rows
    assert call(H=132) == DR_ERR_INVALID_ARGUMENT                    # bf16 rows need 8 | head_dim
    assert call(dt=5) == DR_ERR_UNSUPPORTED
    assert call(perm=FAKE) == DR_ERR_INVALID_ARGUMENT                # perm without seg_offsets
    assert call(K=0) == DR_ERR_INVALID_ARGUMENT


def test_grouped_splitk_and_permute_reject_bad_arguments(lib):
    lib.dr_grouped_splitk_max_slots.restype = ctypes.c_int64
    lib.dr_grouped_splitk_max_slots.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    assert lib.dr_grouped_splitk_max_slots(1000, 4, 256) == 3 + 4
    lib.dr_grouped_splitk_workspace_size.restype = ctypes.c_size_t
    lib.dr_grouped_splitk_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    need = lib.dr_grouped_splitk_workspace_size(1000, 4, 256)
    g = lib.dr_grouped_splitk_gemm_tn
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    ok = dict(X=FAKE, dY=FAKE, K=1000, M=64, N=24, off=FAKE, G=4, split=256, P=FAKE, slots=7, so=FAKE, ws=FAKE,
              wsb=need, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return g(*a.values())

    assert call(slots=6) == DR_ERR_WORKSPACE_TOO_SMALL        # fewer partial slots than the bound
    assert call(wsb=need - 1) == DR_ERR_WORKSPACE_TOO_SMALL
    assert call(G=0) == DR_ERR_INVALID_ARGUMENT
    assert call(G=65536) == DR_ERR_INVALID_ARGUMENT
    assert call(split=0) == DR_ERR_INVALID_ARGUMENT
    assert call(X=FAKE + 2) == DR_ERR_INVALID_ARGUMENT
    assert call(off=None) == DR_ERR_INVALID_ARGUMENT
    assert call(K=0) == DR_ERR_INVALID_ARGUMENT
    r = lib.dr_grouped_splitk_reduce
    r.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert r(FAKE, 7, FAKE, 0, 100, FAKE, FAKE, None) == DR_ERR_INVALID_ARGUMENT
    assert r(FAKE + 4, 7, FAKE, 4, 100, FAKE, FAKE, None) == DR_ERR_INVALID_ARGUMENT  # 4 | count: 16-byte rows
    assert r(FAKE, 7, FAKE, 4, 100, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT
    p = lib.dr_permute_rows
    p.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert p(FAKE, 24, 10, FAKE, None, 20, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT      # row_bytes % 16
    assert p(FAKE, 32, 10, FAKE, None, 20, 0, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT      # k
    assert p(FAKE + 8, 32, 10, FAKE, None, 20, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT  # alignment
    assert p(FAKE, 32, 10, FAKE, FAKE + 2, 20, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT  # alignment
    assert p(FAKE, 32, 10, None, None, 20, 2, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT
    assert p(None, 32, 10, None, None, 0, 2, None, None, None) == DR_OK                         # nothing to do


def test_decode_attention_rejects_bad_arguments(lib):
    f = lib.dr_decode_attention
    f.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int64, ctypes.c_int32,
                                                                             ctypes.c_int32, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    ws_size = lib.dr_decode_attention_workspace_size
    ws_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    ws_size.restype = ctypes.c_size_t
    need = ws_size(4, 32, 1000, 256, 128)
    assert need == 256 + 4 * 32 * 4 * (8 + 128 * 4)      # status block + one slot per (sequence, head, chunk)
    assert ws_size(4, 32, 1000, 100, 128) == 0 and ws_size(4, 32, 1000, 256, 64) == 0

    def call(**kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, layout=0, lens=FAKE, B=4, hq=32, hkv=8, D=128, L=1000, scale=0.1,
                 chunk=256, ws=FAKE, ws_bytes=need, status=None)
        a.update(kw)
        return f(a["out"], a["q"], a["k"], a["v"], a["layout"], a["lens"], a["B"], a["hq"], a["hkv"], a["D"], a["L"],
                 a["scale"], a["chunk"], a["ws"], a["ws_bytes"], a["status"], None)
    assert call(D=64) == DR_ERR_INVALID_ARGUMENT               # head_dim 128 only
    assert call(layout=2) == DR_ERR_INVALID_ARGUMENT           # unknown cache layout
    assert call(hq=24) == DR_ERR_INVALID_ARGUMENT              # 24 / 8 = 3 heads per KV head
    assert call(hq=20, hkv=6) == DR_ERR_INVALID_ARGUMENT       # not a multiple
    assert call(chunk=96) == DR_ERR_INVALID_ARGUMENT           # not a multiple of 64
    assert call(chunk=1 << 21) == DR_ERR_INVALID_ARGUMENT
    assert call(L=0) == DR_ERR_INVALID_ARGUMENT
    assert call(L=(1 << 30) + 1) == DR_ERR_INVALID_ARGUMENT
    assert call(scale=float("nan")) == DR_ERR_INVALID_ARGUMENT
    assert call(scale=float("inf")) == DR_ERR_INVALID_ARGUMENT
    assert call(q=None) == DR_ERR_INVALID_ARGUMENT
    assert call(out=FAKE + 4) == DR_ERR_INVALID_ARGUMENT        # 16-byte alignment
    assert call(k=FAKE + 8) == DR_ERR_INVALID_ARGUMENT
    assert call(status=FAKE + 2) == DR_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=need - 1) == DR_ERR_WORKSPACE_TOO_SMALL
    assert call(B=1 << 28, hkv=8, hq=32, L=1 << 20, chunk=64) == DR_ERR_INVALID_ARGUMENT   # grid too large
    assert call(B=0, q=None, k=None, v=None, out=None, lens=None, ws=None) == DR_OK      # nothing to do
    oc = lib.dr_decode_attention_occupancy_chunk
    oc.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    oc.restype = ctypes.c_int32
    assert oc(0, 8, 1000) == 0 and oc(4, 0, 1000) == 0


def test_sort_rejects_bad_arguments(lib):
    f = lib.dr_sort_by_dest
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.dr_sort_workspace_size.restype = ctypes.c_size_t
    lib.dr_sort_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    need = lib.dr_sort_workspace_size(5000, 300, 0)
    assert f(FAKE, None, 0, 5000, 300, FAKE, FAKE, None, FAKE, need - 1, None) == DR_ERR_WORKSPACE_TOO_SMALL
    assert f(FAKE, None, 0, 5000, 0, FAKE, FAKE, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE, FAKE, 0, 5000, 300, FAKE, FAKE, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT  # src bound
    assert f(None, None, 0, 5000, 300, FAKE, FAKE, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT


def test_splitk_rejects_bad_arguments(lib):
    f = lib.dr_splitk_gemm_tn
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    # 10 tokens in 4 splits of 3 tokens: the last split is non-empty (9 < 10) -> accepted shape;
    # 10 tokens in 6 splits of 2: split 5 starts at 10 -> empty -> rejected
    assert f(FAKE, FAKE, 10, 64, 24, 6, FAKE, None) == DR_ERR_INVALID_ARGUMENT
    assert "empty split" in _err(lib)
    assert f(FAKE, FAKE, 10, 64, 24, 0, FAKE, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE + 2, FAKE, 16384, 7168, 24, 64, FAKE, None) == DR_ERR_INVALID_ARGUMENT
    g = lib.dr_splitk_reduce
    g.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert g(FAKE, 0, 100, FAKE, None) == DR_ERR_INVALID_ARGUMENT
    assert g(FAKE + 4, 64, 100, FAKE, None) == DR_ERR_INVALID_ARGUMENT


def test_fingerprint_rejects_bad_arguments(lib):
    f = lib.dr_fingerprint
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.dr_fingerprint_workspace_size.restype = ctypes.c_size_t
    need = lib.dr_fingerprint_workspace_size(ctypes.c_int64(100))
    assert f(FAKE + 4, 100, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE, 100, FAKE, FAKE, need - 1, None) == DR_ERR_WORKSPACE_TOO_SMALL
    assert f(FAKE, -1, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT


def test_launch_params_validation(lib):
    class P(ctypes.Structure):
        _fields_ = [("grid_blocks", ctypes.c_int32), ("tile_chunks_log2", ctypes.c_int32),
                    ("sort_tile_log2", ctypes.c_int32), ("chunks_in_flight", ctypes.c_int32),
                    ("splitk_stream", ctypes.c_int32)]
    lib.dr_set_launch_params.argtypes = [ctypes.c_void_p]
    assert lib.dr_set_launch_params(ctypes.byref(P(0, 2, 0, 0, 0))) == DR_ERR_INVALID_ARGUMENT
    assert lib.dr_set_launch_params(ctypes.byref(P(0, 0, 20, 0, 0))) == DR_ERR_INVALID_ARGUMENT
    assert lib.dr_set_launch_params(ctypes.byref(P(-1, 0, 0, 0, 0))) == DR_ERR_INVALID_ARGUMENT
    assert lib.dr_set_launch_params(ctypes.byref(P(0, 0, 0, 3, 0))) == DR_ERR_INVALID_ARGUMENT
    assert lib.dr_set_launch_params(ctypes.byref(P(0, 0, 0, 0, 3))) == DR_ERR_INVALID_ARGUMENT
    lib.dr_index_add_workspace_size.restype = ctypes.c_size_t
    lib.dr_index_add_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64]
    default = lib.dr_index_add_workspace_size(100000, 1000, 128)
    assert lib.dr_set_launch_params(ctypes.byref(P(64, 3, 10, 1, 2))) == DR_OK
    # smaller tiles need more partial-row space
    assert lib.dr_index_add_workspace_size(100000, 1000, 128) > default
    assert lib.dr_set_launch_params(None) == DR_OK
    assert lib.dr_index_add_workspace_size(100000, 1000, 128) == default


def test_kernels_have_no_fused_multiply_add():
    """The defined order forbids contraction: the gfx950 assembly of every kernel
    source holds no fused or packed fp32 multiply-add instruction."""
    build = build_module()
    csrc = os.path.join(ROOT, "bitwise_deterministic_fp32_amd", "csrc")
    bad = re.compile(r"\b(v_fma\w*|v_fmac\w*|v_fmamk\w*|v_fmaak\w*|v_pk_fma\w*|v_pk_add_f32|v_pk_mul_f32|v_mad_f32|v_mac_f32)\b")
    for src in build.SOURCES:
        if not src.endswith(".hip"):
            continue
        asm = subprocess.run([build.hipcc(), *build.FLAGS, "--cuda-device-only", "-S", os.path.join(csrc, src),
                              "-o", "-"], capture_output=True, text=True, check=True).stdout
        found = sorted(set(bad.findall(asm)))
        if src == "decode.hip":
            # attention has no defined summation tree; its kernel fuses products by explicit fmaf calls
            # (its order is still fixed), but packed fp32 forms stay out
            found = [x for x in found if x.startswith(("v_pk_", "v_mad_", "v_mac_"))]
        assert not found, (src, found)
        assert "scratch_store" not in asm, src   # no kernel spills registers to scratch


def test_splitk_reduce_fingerprinted_rejects_bad_arguments(lib):
    """Argument checks of the reduce with its fingerprint fail before any launch."""
    lib.dr_splitk_reduce_fingerprinted_workspace_size.restype = ctypes.c_size_t
    lib.dr_splitk_reduce_fingerprinted_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64]
    need = lib.dr_splitk_reduce_fingerprinted_workspace_size(64, 7168 * 24)
    assert need >= lib.dr_splitk_reduce_fingerprinted_workspace_size(64, 0) > 0
    f = lib.dr_splitk_reduce_fingerprinted
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    n = 7168 * 24
    assert f(FAKE, 0, n, FAKE, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT        # no splits
    assert f(FAKE, 64, -1, FAKE, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT      # negative count
    assert f(None, 64, n, FAKE, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT       # null partials
    assert f(FAKE + 4, 64, n, FAKE, FAKE, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT   # misaligned partials
    assert f(FAKE, 64, n, FAKE, None, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT       # null out_hash
    assert f(FAKE, 64, n, FAKE, FAKE + 4, FAKE, need, None) == DR_ERR_INVALID_ARGUMENT   # misaligned out_hash
    assert f(FAKE, 64, n, FAKE, FAKE, None, need, None) == DR_ERR_INVALID_ARGUMENT       # null workspace
    assert f(FAKE, 64, n, FAKE, FAKE, FAKE, need - 1, None) == DR_ERR_WORKSPACE_TOO_SMALL
    assert f(FAKE, 1 << 27, n, FAKE, FAKE, FAKE, need, None) == DR_ERR_UNSUPPORTED


def test_combine_fingerprinted_noalloc_rejects_before_any_device_work(lib):
    """The no-allocation combine checks its arguments and its scratch bound
    before it looks up the static scratch or launches anything: a call whose
    scratch would exceed the 1 MiB static array is refused as unsupported."""
    f = lib.dr_combine_fingerprinted_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    bf16 = 1
    # too big for the static scratch: 200,000 tokens of 7168 bf16 columns (2.8 M wavefronts at k = 8)
    assert f(FAKE, bf16, 10 ** 6, 7168, FAKE, FAKE, 200_000, 8, FAKE, FAKE, None, None) == DR_ERR_UNSUPPORTED
    assert b"scratch" in lib.dr_last_error()
    # k > 8 halves the workgroup, so the bound is reached at half the tokens
    assert f(FAKE, bf16, 10 ** 6, 7168, FAKE, FAKE, 60_000, 16, FAKE, FAKE, None, None) == DR_ERR_UNSUPPORTED
    # the usual argument checks come first
    assert f(FAKE, bf16, 100, 7168, FAKE, FAKE, 10, 8, FAKE, None, None, None) == DR_ERR_INVALID_ARGUMENT  # no hash
    assert f(FAKE, bf16, 100, 7168, FAKE, FAKE, 10, 8, FAKE, FAKE + 4, None, None) == DR_ERR_INVALID_ARGUMENT
    assert f(FAKE, bf16, 100, 7, FAKE, FAKE, 10, 8, FAKE, FAKE, None, None) == DR_ERR_INVALID_ARGUMENT  # hidden % 8
    assert f(FAKE, 7, 100, 7168, FAKE, FAKE, 10, 8, FAKE, FAKE, None, None) == DR_ERR_UNSUPPORTED  # dtype
    assert f(FAKE, bf16, 100, 7168, FAKE, FAKE, 10, 65, FAKE, FAKE, None, None) == DR_ERR_UNSUPPORTED  # k > 64


def test_grouped_wgrad_rejects_bad_arguments(lib):
    lib.dr_grouped_wgrad_workspace_size.restype = ctypes.c_size_t
    lib.dr_grouped_wgrad_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                                    ctypes.c_int64]
    need = lib.dr_grouped_wgrad_workspace_size(4096, 4, 256, 512, 256)
    assert need > 256
    f = lib.dr_grouped_wgrad
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    ok = [FAKE, FAKE, 4096, 512, 256, FAKE, 4, 256, FAKE, FAKE, need, None]

    def call(**kw):
        a = list(ok)
        names = ["X", "dY", "K", "M", "N", "off", "G", "split", "out", "ws", "ws_bytes", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)
    assert call(X=None) == DR_ERR_INVALID_ARGUMENT
    assert call(K=0) == DR_ERR_INVALID_ARGUMENT
    assert call(G=0) == DR_ERR_INVALID_ARGUMENT
    assert call(G=70000) == DR_ERR_INVALID_ARGUMENT
    assert call(split=0) == DR_ERR_INVALID_ARGUMENT
    assert call(M=500) == DR_ERR_UNSUPPORTED          # not a multiple of 8
    assert call(N=20) == DR_ERR_UNSUPPORTED
    assert call(M=(1 << 23) + 8) == DR_ERR_UNSUPPORTED  # a stage's byte range must fit 32 bits
    assert call(N=(1 << 23) + 8) == DR_ERR_UNSUPPORTED
    assert call(X=FAKE + 8) == DR_ERR_INVALID_ARGUMENT  # 16-byte alignment
    assert call(ws_bytes=need - 1) == DR_ERR_WORKSPACE_TOO_SMALL
    assert call(K=(1 << 31) - 100) == DR_ERR_UNSUPPORTED
