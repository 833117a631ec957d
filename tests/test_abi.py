"""The C-ABI library: it loads, exports every entry point include/fa.h
declares, and rejects bad arguments before any HIP call (so these checks run
on a host without a GPU; no compute call is made here)."""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

needs_lib = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libfa.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert header_functions() == sorted(_lib.EXPORTS)


def header_signatures():
    """name -> list of C parameter types, from the declarations in include/fa.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    sigs = {}
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M):
        params = [" ".join(p.split()) for p in m.group(2).split(",")]
        types = []
        for p in params:
            p = re.sub(r"\b\w+$", "", p).strip()   # drop the parameter name
            types.append(p)
        sigs[m.group(1)] = types
    return sigs


def _ctype_of(c_type):
    if c_type == "const long long*":
        return ctypes.POINTER(ctypes.c_longlong)
    if "*" in c_type:
        return ctypes.c_void_p
    return {"int": ctypes.c_int, "float": ctypes.c_float, "size_t": ctypes.c_size_t,
            "unsigned": ctypes.c_uint, "unsigned long long": ctypes.c_ulonglong}[c_type]


@needs_lib
def test_binding_argtypes_match_header():
    """Every ctypes prototype in the binding has the header's parameter count
    and kinds (pointer, int, unsigned, unsigned long long, float, size_t), so a change of the C signature
    cannot be marshalled wrongly."""
    lib = _lib.load()
    sigs = header_signatures()
    assert sorted(sigs) == sorted(_lib.EXPORTS)
    for name, types in sigs.items():
        want = [_ctype_of(t) for t in types if t != "void"]
        got = list(getattr(lib, name).argtypes)
        assert got == want, (name, got, want)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    names = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in header_functions():
        assert re.search(rf"\bT {name}$", names, flags=re.M), name


@needs_lib
def test_strerror():
    for st in (0, -1, -2, -3, -4, -5):
        assert isinstance(fa.fa_strerror(st), str) and fa.fa_strerror(st)
    assert fa.fa_strerror(12345) == "unknown status"


@needs_lib
def test_workspace_size(monkeypatch):
    monkeypatch.delenv("FA_DQ_MODE", raising=False)
    rows = 1 * 32 * 8192
    # the smallest workspace: the two per-row statistics (recompute method)
    bf = fa.fa_bwd_workspace_bytes(1, 32, 8192, 128, fa.FA_BF16)
    assert bf == 2 * rows * 4
    f32 = fa.fa_bwd_workspace_bytes(1, 1, 128, 64, fa.FA_FP32)
    assert f32 == 2 * 512
    assert fa.fa_bwd_workspace_bytes(1, 1, 100, 64, fa.FA_BF16) % 256 == 0
    assert fa.fa_bwd_workspace_bytes(0, 1, 128, 64, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 128, 80, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_bytes(1, 2, 100, 96, fa.FA_BF16) == round_up(200 * 4) * 2
    # with FA_DQ_MODE=atomic it holds the fp32 accumulator too
    monkeypatch.setenv("FA_DQ_MODE", "atomic")
    assert fa.fa_bwd_workspace_bytes(1, 32, 8192, 128, fa.FA_BF16) == 2 * rows * 4 + rows * 128 * 4
    assert fa.fa_bwd_workspace_bytes(1, 2, 100, 96, fa.FA_BF16) == round_up(200 * 4) * 2   # no atomic d = 96


def handoff_head_bytes(N, causal):
    """The dS buffer's bytes per head: query block i (64 rows) keeps 4 KB per
    32-key slice, 2i + 2 slices causal, ceil(N / 32) otherwise."""
    nqb, nks = -(-N // 64), -(-N // 32)
    return 4096 * sum((2 * i + 2) if causal else nks for i in range(nqb))


@needs_lib
@pytest.mark.parametrize("B,H,N,d", [(1, 32, 8192, 128), (2, 3, 100, 64), (1, 1, 1, 96), (1, 2, 4099, 256),
                                     (4, 16, 1024, 64)])
def test_workspace_size_per_method(B, H, N, d):
    rows = B * H * N
    stats = 2 * round_up(rows * 4)
    for causal in (0, 1):
        ws = lambda m, dt=fa.FA_BF16: fa.fa_bwd_workspace_size(B, H, N, d, causal, dt, m)
        assert ws(fa.FA_DQ_RECOMPUTE) == stats
        assert ws(fa.FA_DQ_HANDOFF) == stats + round_up(B * H * handoff_head_bytes(N, causal)) + 4096
        assert ws(fa.FA_DQ_ATOMIC) == (stats + round_up(rows * d * 4) if d in (64, 128) else 0)
        # fp32 has only the recompute kernels
        assert ws(fa.FA_DQ_HANDOFF, fa.FA_FP32) == 0
        assert ws(fa.FA_DQ_RECOMPUTE, fa.FA_FP32) == stats
        assert ws(7) == 0
    # the causal buffer keeps about half of the (query, key) pairs
    assert (fa.fa_bwd_workspace_size(1, 1, 8192, 128, 1, fa.FA_BF16, fa.FA_DQ_HANDOFF)
            < 0.51 * fa.fa_bwd_workspace_size(1, 1, 8192, 128, 0, fa.FA_BF16, fa.FA_DQ_HANDOFF))
    assert fa.fa_bwd_workspace_size(0, 1, 128, 64, 0, fa.FA_BF16, fa.FA_DQ_HANDOFF) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 128, 64, 2, fa.FA_BF16, fa.FA_DQ_HANDOFF) == 0


@needs_lib
def test_dq_method_follows_the_workspace(monkeypatch):
    """fa_bwd takes the dS hand-off exactly when the workspace holds its
    buffer, the recompute otherwise; FA_DQ_MODE forces one (atomic only where
    that method exists, never with dropout)."""
    monkeypatch.delenv("FA_DQ_MODE", raising=False)
    for (B, H, N, d) in ((1, 32, 8192, 128), (2, 3, 100, 64), (1, 2, 4099, 256), (1, 1, 17, 96)):
        for causal in (0, 1):
            need = fa.fa_bwd_workspace_size(B, H, N, d, causal, fa.FA_BF16, fa.FA_DQ_HANDOFF)
            m = lambda ws, drop=0: fa.fa_bwd_dq_method(B, H, N, d, causal, fa.FA_BF16, ws, drop)
            assert m(need) == fa.FA_DQ_HANDOFF and m(need + 1) == fa.FA_DQ_HANDOFF
            assert m(need - 1) == fa.FA_DQ_RECOMPUTE and m(0) == fa.FA_DQ_RECOMPUTE
            assert m(need, 1) == fa.FA_DQ_HANDOFF and m(need - 1, 1) == fa.FA_DQ_RECOMPUTE
            assert fa.fa_bwd_dq_method(B, H, N, d, causal, fa.FA_FP32, need, 0) == fa.FA_DQ_RECOMPUTE
    monkeypatch.setenv("FA_DQ_MODE", "recompute")
    assert fa.fa_bwd_dq_method(1, 1, 128, 64, 1, fa.FA_BF16, 1 << 40, 0) == fa.FA_DQ_RECOMPUTE
    monkeypatch.setenv("FA_DQ_MODE", "atomic")
    assert fa.fa_bwd_dq_method(1, 1, 128, 64, 1, fa.FA_BF16, 0, 0) == fa.FA_DQ_ATOMIC
    assert fa.fa_bwd_dq_method(1, 1, 128, 64, 1, fa.FA_BF16, 1 << 40, 1) == fa.FA_DQ_HANDOFF
    assert fa.fa_bwd_dq_method(1, 1, 128, 96, 1, fa.FA_BF16, 1 << 40, 0) == fa.FA_DQ_HANDOFF
    # rejected arguments
    assert fa.fa_bwd_dq_method(0, 1, 128, 64, 1, fa.FA_BF16, 0, 0) == -1
    assert fa.fa_bwd_dq_method(1, 1, 128, 80, 1, fa.FA_BF16, 0, 0) == -2
    assert fa.fa_bwd_dq_method(1, 1, 128, 64, 2, fa.FA_BF16, 0, 0) == -1
    assert fa.fa_bwd_dq_method(1, 1, 128, 64, 1, fa.FA_BF16, 0, 2) == -1
    assert fa.fa_bwd_dq_method(1, 1, 128, 64, 1, fa.FA_FP32, 0, 1) == -2


P = 0x10000  # a non-null, 256-byte aligned stand-in address; never dereferenced


def round_up(x, a=256):
    return -(-x // a) * a


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, causal=0, scale=0.125, stream=None,
             dtype=fa.FA_BF16, layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    return fa.fa_fwd(**a)


def bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, dO=P, lse=P, dq=P, dk=P, dv=P, B=1, H=1, N=128, d=64, causal=0,
             scale=0.125, workspace=P, workspace_bytes=1 << 30, stream=None, dtype=fa.FA_BF16,
             layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    return fa.fa_bwd(**a)


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1), (dict(causal=2), -1),
    (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1), (dict(d=80), -2), (dict(d=512), -2),
    (dict(dtype=7), -2),
    (dict(q=P + 8), -1), (dict(lse=P + 2), -1),
    (dict(B=1024, H=1024, N=4096, d=128), -2),
    (dict(layout=2), -1), (dict(layout=-1), -1),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), -1), (dict(dq=None), -1), (dict(dk=None), -1), (dict(dv=None), -1),
    (dict(N=-5), -1), (dict(d=32), -2), (dict(scale=float("-inf")), -1),
    (dict(workspace=None), -3), (dict(workspace_bytes=1000), -3), (dict(workspace=P + 16), -3),
    (dict(dv=P + 4), -1), (dict(layout=7), -1),
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def dense_strides(B, H, N, d, layout=fa.FA_LAYOUT_BHND):
    if layout == fa.FA_LAYOUT_BNHD:
        return [N * H * d, d, H * d]
    return [H * N * d, N * d, d]


def fwd_strided(strides=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=3, N=128, d=64, causal=0, scale=0.125, stream=None,
             dtype=fa.FA_BF16)
    a.update(kw)
    if strides is None:
        strides = dense_strides(a["B"], a["H"], a["N"], a["d"]) * 4
    return fa.fa_fwd_strided(strides=strides, **a)


def bwd_strided(strides=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, dO=P, lse=P, dq=P, dk=P, dv=P, B=2, H=3, N=128, d=64, causal=0,
             scale=0.125, workspace=P, workspace_bytes=1 << 30, stream=None, dtype=fa.FA_BF16)
    a.update(kw)
    if strides is None:
        strides = dense_strides(a["B"], a["H"], a["N"], a["d"]) * 8
    return fa.fa_bwd_strided(strides=strides, **a)


def _set(strides, tensor, values):
    s = list(strides)
    s[3 * tensor:3 * tensor + 3] = values
    return s


D = dense_strides(2, 3, 128, 64)


@needs_lib
@pytest.mark.parametrize("strides,kw,status", [
    (None, dict(q=None), -1), (None, dict(d=80), -2), (None, dict(N=0), -1), (None, dict(q=P + 8), -1),
    (None, dict(dtype=fa.FA_FP32, d=512), -2),
    (_set(D * 4, 0, [D[0], D[1], -64]), {}, -1),           # negative row stride
    (_set(D * 4, 1, [D[0], D[1], 68]), {}, -1),            # k rows 136 bytes apart: not 16-byte aligned
    (_set(D * 4, 2, [D[0], 4, D[2]]), {}, -1),             # v head stride of 8 bytes
    (_set(D * 4, 0, [1 << 41, D[1], D[2]]), {}, -1),       # beyond 2^40
    (_set(D * 4, 0, [D[0], D[1], 1 << 23]), {}, -1),       # 128 rows of 2^24 bytes: 2^31
    (_set(D * 4, 3, [0, D[1], D[2]]), {}, -1),             # o: two batches on the same rows
    (_set(D * 4, 3, [D[0], D[1], 32]), {}, -1),            # o rows of 64 elements 32 apart
    (_set(D * 4, 3, [D[0], 64, 64]), {}, -1),              # o: heads and rows interleave onto each other
])
def test_fwd_strided_rejects(strides, kw, status):
    assert fwd_strided(strides, **kw) == status


def test_fwd_strided_rejects_a_null_stride_array():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfa.so not built")
    lib = _lib.load()
    assert lib.fa_fwd_strided(P, P, P, P, P, 1, 1, 128, 64, 0, 0.125, None, None, fa.FA_BF16) == -1
    with pytest.raises(ValueError):
        fa.fa_fwd_strided(P, P, P, P, P, 1, 1, 128, 64, 0, 0.125, [0] * 11, None, fa.FA_BF16)


@needs_lib
@pytest.mark.parametrize("strides,kw,status", [
    (None, dict(dv=None), -1), (None, dict(workspace=None), -3), (None, dict(workspace_bytes=100), -3),
    (_set(D * 8, 4, [D[0], D[1], 12]), {}, -1),            # dO rows 24 bytes apart
    (_set(D * 8, 5, [D[0], 0, D[2]]), {}, -1),             # dq: every head on the same rows
    (_set(D * 8, 7, [D[0], D[1], 0]), {}, -1),             # dv: every row on one row
    (_set(D * 8, 6, [D[0], D[1], 4]), dict(dtype=fa.FA_FP32), -1),   # fp32 dk rows of 64 overlapping
    (_set(D * 8, 6, [D[0], D[1], 6]), dict(dtype=fa.FA_FP32), -1),   # fp32 stride of 24 bytes
])
def test_bwd_strided_rejects(strides, kw, status):
    assert bwd_strided(strides, **kw) == status


@needs_lib
def test_bwd_workspace_boundary():
    need = fa.fa_bwd_workspace_bytes(1, 1, 128, 64, fa.FA_BF16)
    assert bwd(workspace_bytes=need - 1) == -3


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        _lib.load()


def splitkv(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=4, Nk=1000, d=128, causal=1, scale=0.125,
             num_splits=0, workspace=P, workspace_bytes=1 << 30, stream=None, dtype=fa.FA_BF16,
             layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    return fa.fa_fwd_splitkv(**a)


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(Nq=0), -1), (dict(Nk=0), -1), (dict(Nq=1001), -1), (dict(causal=2), -1),
    (dict(num_splits=-1), -1), (dict(num_splits=1025), -1), (dict(layout=3), -1),
    (dict(scale=float("nan")), -1), (dict(d=80), -2), (dict(dtype=fa.FA_FP32), -2), (dict(dtype=5), -2),
    (dict(q=P + 8), -1), (dict(workspace=None), -3), (dict(workspace_bytes=100), -3),
    (dict(workspace=P + 64), -3), (dict(B=64, H=64, Nk=1 << 20), -2),
])
def test_splitkv_rejects(kw, status):
    assert splitkv(**kw) == status


@needs_lib
def test_splitkv_noncausal_allows_more_queries_than_keys_and_sizes_workspace():
    # the query count may exceed the key count when not causal: only the
    # workspace check stops this call (a null-free, too-small workspace)
    assert splitkv(causal=0, Nq=2000, workspace_bytes=10) == -3
    rows, tile = 1 * 2 * 4, 32
    for ns in (1, 3, 7):
        n = fa.fa_fwd_splitkv_workspace_bytes(1, 2, 4, 1000, 128, ns)
        tiles = (1000 + tile - 1) // tile
        per = -(-tiles // ns)
        used = -(-tiles // per)
        r = lambda x: -(-x // 256) * 256
        assert n == r(used * rows * 128 * 4) + r(used * rows * 4), ns
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 4, 1000, 80, 0) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 4, 1000, 128, 2000) == 0


def fwd8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=256, d=128, causal=1, scale=0.125, descale_q=0.5,
             descale_k=0.5, descale_v=0.5, stream=None, layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    return fa.fa_fwd_fp8(**a)


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(lse=None), -1), (dict(N=0), -1), (dict(causal=3), -1),
    (dict(scale=float("-inf")), -1), (dict(descale_q=0.0), -1), (dict(descale_k=-1.0), -1),
    (dict(descale_v=float("inf")), -1), (dict(descale_q=float("nan")), -1), (dict(layout=2), -1),
    (dict(d=80), -2), (dict(d=512), -2), (dict(k=P + 4), -1), (dict(o=P + 2), -1),
    (dict(scale=1e30, descale_q=1e30, descale_k=1e30), -1),
])
def test_fp8_rejects(kw, status):
    assert fwd8(**kw) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(Nq=0), -1), (dict(Nq=1001), -1), (dict(num_splits=-2), -1),
    (dict(descale_v=0.0), -1), (dict(d=512), -2), (dict(d=80), -2), (dict(layout=4), -1), (dict(workspace=None), -3),
    (dict(workspace_bytes=64), -3),
])
def test_splitkv_fp8_rejects(kw, status):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=4, Nk=1000, d=128, causal=1, scale=0.125, descale_q=1.0,
             descale_k=1.0, descale_v=1.0, num_splits=0, workspace=P, workspace_bytes=1 << 30, stream=None,
             layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    assert fa.fa_fwd_splitkv_fp8(**a) == status


@needs_lib
def test_splitkv_fp8_workspace_uses_64_key_tiles():
    tiles = -(-1000 // 64)
    for ns in (1, 4, 9):
        per = -(-tiles // ns)
        used = -(-tiles // per)
        r = lambda x: -(-x // 256) * 256
        for d in (64, 96, 128, 256):
            assert fa.fa_fwd_splitkv_fp8_workspace_bytes(1, 2, 4, 1000, d, ns) == r(used * 8 * d * 4) + r(used * 8 * 4)
    assert fa.fa_fwd_splitkv_fp8_workspace_bytes(1, 2, 4, 1000, 80, 0) == 0


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(N=0), -1), (dict(causal=2), -1), (dict(scale=float("nan")), -1),
    (dict(drop_t=-1), -1), (dict(drop_t=256), -1), (dict(layout=3), -1), (dict(d=80), -2), (dict(v=P + 8), -1),
])
def test_fwd_dropout_rejects(kw, status):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=64, d=128, causal=1, scale=0.125, drop_t=26, seed=7,
             offset=0, stream=None, layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    assert fa.fa_fwd_dropout(**a) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), -1), (dict(dk=None), -1), (dict(H=0), -1), (dict(drop_t=300), -1), (dict(d=32), -2),
    (dict(workspace=None), -3), (dict(workspace_bytes=1023), -3), (dict(workspace=P + 16), -3),
    (dict(lse=P + 2), -1),
])
def test_bwd_dropout_rejects(kw, status):
    a = dict(q=P, k=P, v=P, o=P, dO=P, lse=P, dq=P, dk=P, dv=P, B=1, H=2, N=64, d=128, causal=1, scale=0.125,
             drop_t=26, seed=(1 << 63) + 5, offset=3, workspace=P,
             workspace_bytes=fa.fa_bwd_workspace_bytes(1, 2, 64, 128, fa.FA_BF16), stream=None,
             layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    assert fa.fa_bwd_dropout(**a) == status


def test_drop_threshold_rounds_to_256ths():
    assert fa.drop_threshold(0.0) == 0
    assert fa.drop_threshold(0.1) == 26
    assert fa.drop_threshold(0.25) == 64
    assert fa.drop_threshold(255 / 256) == 255
    for bad in (-0.01, 0.999, 1.0):
        with pytest.raises(ValueError):
            fa.drop_threshold(bad)


@needs_lib
def test_tensors_of_2_pow_31_elements_are_unsupported():
    """The kernels index a tensor's elements within 31 bits per call; the
    largest accepted shape is tested on the GPU (63 x 32 x 8192 x 128)."""
    big = dict(q=P, k=P, v=P, o=P, lse=P, B=64, H=32, N=8192, d=128, causal=1, scale=0.125, stream=None,
               dtype=fa.FA_BF16, layout=fa.FA_LAYOUT_BHND)
    assert fa.fa_fwd(**big) == -2
    assert fa.fa_fwd(**dict(big, B=1, H=1, N=1 << 24)) == -2   # one head of 2^24 rows x 128
    assert fa.fa_fwd_dropout(q=P, k=P, v=P, o=P, lse=P, B=64, H=32, N=8192, d=128, causal=1, scale=0.125, drop_t=0,
                             seed=0, offset=0, stream=None, layout=fa.FA_LAYOUT_BHND) == -2


@needs_lib
def test_head_dim_256_in_every_call():
    """d = 256 exists for the bf16 and fp32 forward and backward, the
    dropout calls, the bf16 split-key-range forward and the two FP8
    forwards."""
    base = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=64, d=256, causal=1, scale=0.0625, stream=None,
                layout=fa.FA_LAYOUT_BHND)
    assert fa.fa_fwd(**dict(base, q=None), dtype=fa.FA_FP32) == -1   # d = 256 fp32 passes the shape check
    assert fa.fa_fwd(**dict(base, q=None), dtype=fa.FA_BF16) == -1   # d = 256 bf16 passes the shape check
    assert fa.fa_bwd_workspace_bytes(1, 2, 64, 256, fa.FA_BF16) > 0
    assert fa.fa_bwd_workspace_bytes(1, 2, 64, 256, fa.FA_FP32) > 0
    assert fa.fa_fwd_dropout(**dict(base, o=None), drop_t=26, seed=1, offset=0) == -1   # shape accepted
    assert fa.fa_fwd_fp8(**dict(base, q=None), descale_q=1.0, descale_k=1.0, descale_v=1.0) == -1   # shape accepted
    # split: 64 keys are 2 tiles, fewer than the 4 a range takes at least, so one range: O and LSE
    # partials of 4 rows x 2 heads
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 2, 4, 64, 256, 0) == round_up(1 * 2 * 4 * 256 * 4) + 256
    # FP8: 64 keys are one 64-key tile, so one range as well
    assert fa.fa_fwd_splitkv_fp8_workspace_bytes(1, 2, 4, 64, 256, 0) == round_up(1 * 2 * 4 * 256 * 4) + 256
    sk = dict(q=None, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=4, Nk=64, d=256, causal=1, scale=0.0625, num_splits=0,
              workspace=P, workspace_bytes=1 << 20, stream=None, dtype=fa.FA_BF16, layout=fa.FA_LAYOUT_BHND)
    assert fa.fa_fwd_splitkv(**sk) == -1   # the shape passes; the null q is rejected
    assert fa.fa_fwd_splitkv(**dict(sk, q=P, dtype=fa.FA_FP32)) == -2



@needs_lib
@pytest.mark.parametrize("kw", [dict(seed=-1), dict(seed=1 << 64), dict(offset=-1), dict(offset=1 << 32)])
def test_dropout_seed_and_offset_out_of_range_raise(kw):
    """ctypes would wrap these silently into another mask; the binding raises
    before the C call."""
    fwd = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=64, d=128, causal=1, scale=0.125, drop_t=26, seed=7,
               offset=0, stream=None, layout=fa.FA_LAYOUT_BHND)
    with pytest.raises(ValueError):
        fa.fa_fwd_dropout(**dict(fwd, **kw))
    bwd = dict(fwd, dO=P, dq=P, dk=P, dv=P, workspace=P, workspace_bytes=1 << 20)
    with pytest.raises(ValueError):
        fa.fa_bwd_dropout(**dict(bwd, **kw))


def test_buffer_checks_of_the_binding():
    """Caller-supplied outputs, statistics and workspaces are checked for
    shape, dtype, contiguity and device before their pointers are used (host
    tensors stand in for device ones here)."""
    import torch
    from exact_tiled_attention_online_amd import _lib
    dev = torch.device("cpu")
    good = torch.empty((1, 2, 64), dtype=torch.float32)
    assert _lib._check_buf(good, (1, 2, 64), torch.float32, dev, "lse") is good
    for bad in (torch.empty((1, 2, 63), dtype=torch.float32), torch.empty((1, 2, 64), dtype=torch.bfloat16),
                torch.empty((1, 64, 2), dtype=torch.float32).transpose(1, 2), torch.empty((2, 64)),
                torch.empty((1, 2, 64), dtype=torch.float32, device="meta")):
        with pytest.raises(ValueError):
            _lib._check_buf(bad, (1, 2, 64), torch.float32, dev, "lse")
    ws = torch.empty(4096, dtype=torch.uint8)
    assert _lib._check_ws(ws, dev) is ws
    for bad in (torch.empty(1024, dtype=torch.float32), ws[::2], torch.empty(4096, dtype=torch.uint8, device="meta")):
        with pytest.raises(ValueError):
            _lib._check_ws(bad, dev)
    assert _lib._check_uint((1 << 64) - 1, 64, "seed") == (1 << 64) - 1
    assert _lib._check_uint(0, 32, "offset") == 0


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1), (dict(B=0), -1), (dict(Nq=0), -1),
    (dict(causal=2), -1), (dict(scale=float("nan")), -1), (dict(d=80), -2), (dict(d=512), -2), (dict(dtype=fa.FA_FP32), -2),
    (dict(causal=1, Nq=2000, Nk=1000), -1), (dict(num_splits=-1), -1), (dict(num_splits=5000), -1),
    (dict(layout=5), -1), (dict(q=P + 8), -1),
    # more partial results than the static scratch holds: 64 ranges x 4096 rows x (128 + 1) floats
    (dict(B=1, H=64, Nq=64, Nk=8192, num_splits=64), -5),
])
def test_splitkv_noalloc_rejects(kw, status):
    """The no-allocation split forward checks every argument of
    fa_fwd_splitkv, and the scratch bound, before any HIP call (no GPU here:
    a call that got past the checks would fail with FA_ERR_HIP instead)."""
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=4, Nk=1000, d=128, causal=1, scale=0.125, num_splits=0,
             stream=None, dtype=fa.FA_BF16, layout=fa.FA_LAYOUT_BHND)
    a.update(kw)
    assert fa.fa_fwd_splitkv_noalloc(**a) == status


@needs_lib
def test_splitkv_noalloc_bound_is_the_workspace_size():
    """The largest call it takes is the one whose fa_fwd_splitkv workspace fits
    FA_SPLITKV_NOALLOC_MAX_BYTES."""
    assert _lib.FA_SPLITKV_NOALLOC_MAX_BYTES == 32 * 1024 * 1024
    n = fa.fa_fwd_splitkv_workspace_bytes(1, 64, 64, 8192, 128, 64)
    assert n > _lib.FA_SPLITKV_NOALLOC_MAX_BYTES
    assert fa.fa_fwd_splitkv_workspace_bytes(8, 32, 1, 16384, 128, 0) < _lib.FA_SPLITKV_NOALLOC_MAX_BYTES
    header = open(HEADER).read()
    assert "#define FA_SPLITKV_NOALLOC_MAX_BYTES (32u * 1024u * 1024u)" in header


def test_split_conveniences_check_the_cache_geometry():
    """forward_splitkv / forward_splitkv_fp8 take a key/value cache only with
    q's batch, heads and head dim (checked on shapes, before any launch)."""
    class Shape:
        def __init__(self, shape):
            self.shape = shape

    q = Shape((2, 4, 3, 128))
    _lib._check_kv_heads(q, Shape((2, 4, 1000, 128)), fa.FA_LAYOUT_BHND)
    for bad in ((2, 1, 1000, 128), (2, 4, 1000, 64), (1, 4, 1000, 128)):
        with pytest.raises(ValueError):
            _lib._check_kv_heads(q, Shape(bad), fa.FA_LAYOUT_BHND)
    # [B, N, H, d]: heads are the third dimension
    _lib._check_kv_heads(Shape((2, 3, 4, 128)), Shape((2, 1000, 4, 128)), fa.FA_LAYOUT_BNHD)
    with pytest.raises(ValueError):
        _lib._check_kv_heads(Shape((2, 3, 4, 128)), Shape((2, 1000, 1, 128)), fa.FA_LAYOUT_BNHD)


@needs_lib
@pytest.mark.parametrize("scale", [-0.125, -1e-30, 0.0, -0.0, 1e-40, 3.0e38])
def test_any_finite_scale_passes_the_checks(scale):
    """Any finite scale is accepted (the checks then reach the null pointer
    that follows them): negative, zero, subnormal and huge values."""
    assert fwd(scale=scale, o=None) == -1
    assert bwd(scale=scale, dq=None) == -1
    assert fwd(scale=scale, d=80) == -2            # the shape check ran past the scale
    assert bwd(scale=scale, d=80) == -2
