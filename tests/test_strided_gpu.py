"""GPU parity of the strided entry points (fa_fwd_strided, fa_bwd_strided)
through the C ABI.

The strided calls run the kernels of fa_fwd / fa_bwd with per-tensor row
addresses, so on the same values they must give bitwise the same O, LSE, dQ,
dK and dV as the dense calls; the dense calls are compared with the fp64
oracle elsewhere, and here once more on the packed case.  Inputs are views
into one packed projection buffer [B, N, 3, H, d (+ pad)], with the
gradients written into a packed gradient buffer of the same form; padding
between rows holds a sentinel that no call may overwrite (the kernels write
exactly d elements per row).
"""
import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import compare, log, oracle_heads, run_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0   # exactly representable in bf16 and fp32


def _torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _packed(arrays, dtype, pad, shape=None):
    """A [B, N, len(arrays), H, d + pad] device buffer holding the [B,H,N,d]
    arrays (None: left as sentinel; `shape` gives (B, H, N, d) when every
    slot is None) with the sentinel in the padding, and [B,H,N,d] views of
    its slots."""
    import torch
    B, H, N, d = shape if shape is not None else next(a.shape for a in arrays if a is not None)
    buf = torch.full((B, N, len(arrays), H, d + pad), SENTINEL, dtype=_torch_dtype(dtype), device="cuda")
    views = []
    for i, a in enumerate(arrays):
        view = buf[:, :, i, :, :d].permute(0, 2, 1, 3)
        if a is not None:
            view.copy_(to_dev(a, dtype))
        views.append(view)
    return buf, views


def _pad_untouched(buf, d):
    import torch
    if buf.shape[-1] == d:
        return True
    return bool(torch.all(buf[..., d:] == SENTINEL).item())


CASES = [(dtype, d, causal, n, m)
         for dtype in ("bf16", "fp32")
         for d in (64, 96, 128, 256)
         for causal in (False, True)
         for n in (200, 513)
         for m in ((fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE) if dtype == "bf16" else (fa.FA_DQ_RECOMPUTE,))]


@pytest.mark.parametrize("dtype,d,causal,n,method", CASES)
def test_packed_qkv_is_bitwise_the_dense_run(dtype, d, causal, n, method):
    import torch
    log(f"strided packed: {dtype} d={d} causal={causal} N={n} method={method}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 3, n, d), seed=4100 + n + d, dtype=dtype)
    scale = gen.default_scale(d)
    dense = run_gpu(x, dtype, causal, scale, method=method)["_dev"]

    pad = 8
    qkv, (q, k, v) = _packed([x["q"], x["k"], x["v"]], dtype, pad)
    qkv_before = qkv.clone()
    obuf, (o,) = _packed([None], dtype, pad, x["q"].shape)
    # dO as a [B,N,H,d] tensor seen as [B,H,N,d]
    do = to_dev(x["do"], dtype, fa.FA_LAYOUT_BNHD).permute(0, 2, 1, 3)
    o_ret, lse = fa.forward_strided(q, k, v, causal, scale, out=o)
    gbuf, grads = _packed([None, None, None], dtype, pad, x["q"].shape)
    dq, dk, dv = fa.backward_strided(q, k, v, o, do, lse, causal, scale, grads=grads, method=method)
    torch.cuda.synchronize()

    assert o_ret.data_ptr() == o.data_ptr()
    assert torch.equal(o, dense["o_dev"]), "O differs from the dense run"
    assert torch.equal(lse, dense["lse_dev"]), "LSE differs from the dense run"
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(got, dense[name + "_dev"]), f"{name} differs from the dense run"
    assert torch.equal(qkv, qkv_before), "the packed inputs were written"
    assert _pad_untouched(obuf, d) and _pad_untouched(gbuf, d), "a write reached the padding between rows"


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("fp32", 96)])
def test_packed_qkv_against_the_oracle(dtype, d):
    log(f"strided oracle: {dtype} d={d}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, 300, d), seed=4300 + d, dtype=dtype)
    scale = gen.default_scale(d)
    _, (q, k, v) = _packed([x["q"], x["k"], x["v"]], dtype, 0)
    _, (do,) = _packed([x["do"]], dtype, 8)
    o, lse = fa.forward_strided(q, k, v, True, scale)
    dq, dk, dv = fa.backward_strided(q, k, v, o, do, lse, True, scale)
    got = {"o": to_np(o), "lse": to_np(lse), "dq": to_np(dq), "dk": to_np(dk), "dv": to_np(dv)}
    want = oracle_heads(x, True, scale, heads=None)
    for (b, h), wv in want.items():
        compare({n: got[n][b, h] for n in wv}, wv, dtype, where=f"strided {dtype} d={d} head ({b},{h})")


def test_keys_and_values_broadcast_over_the_batch():
    """k, v with batch stride 0 (one key/value set shared by every batch)
    give the dense run on the expanded copies, bitwise."""
    import torch
    log("strided broadcast k, v")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(3, 2, 257, 128), seed=4401, dtype="bf16")
    for n in ("k", "v"):
        x[n] = np.broadcast_to(x[n][:1], x[n].shape).copy()
    scale = gen.default_scale(128)
    dense = run_gpu(x, "bf16", True, scale)["_dev"]
    q = to_dev(x["q"], "bf16")
    k1, v1 = to_dev(x["k"][:1], "bf16"), to_dev(x["v"][:1], "bf16")
    k, v = k1.expand(3, -1, -1, -1), v1.expand(3, -1, -1, -1)
    assert k.stride(0) == 0
    o, lse = fa.forward_strided(q, k, v, True, scale)
    do = to_dev(x["do"], "bf16")
    dq, dk, dv = fa.backward_strided(q, k, v, o, do, lse, True, scale)
    torch.cuda.synchronize()
    for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(got, dense[name + "_dev"]), f"{name} differs from the dense run"


def test_every_tensor_in_its_own_layout():
    """q [B,N,H,d], k [B,H,N,d], v a packed slot, o padded [B,H,N,d+8], dO
    [B,N,H,d], dq [B,N,H,d], dk padded, dv a packed slot: bitwise the dense
    run, across a ragged tail and the non-causal mask."""
    import torch
    log("strided mixed layouts")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 2, 333, 64), seed=4501, dtype="bf16")
    scale = gen.default_scale(64)
    dense = run_gpu(x, "bf16", False, scale)["_dev"]
    bnhd = fa.FA_LAYOUT_BNHD
    q = to_dev(x["q"], "bf16", bnhd).permute(0, 2, 1, 3)
    k = to_dev(x["k"], "bf16")
    _, (v,) = _packed([x["v"]], "bf16", 0)
    obuf, (o,) = _packed([None], "bf16", 8, x["q"].shape)
    do = to_dev(x["do"], "bf16", bnhd).permute(0, 2, 1, 3)
    dq = torch.empty((2, 333, 2, 64), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    kbuf = torch.full((2, 2, 333, 72), SENTINEL, dtype=torch.bfloat16, device="cuda")
    dk = kbuf[..., :64]
    vbuf, (dv, _) = _packed([None, None], "bf16", 8, x["q"].shape)
    _, lse = fa.forward_strided(q, k, v, False, scale, out=o)
    fa.backward_strided(q, k, v, o, do, lse, False, scale, grads=(dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(o, dense["o_dev"]) and torch.equal(lse, dense["lse_dev"])
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(got, dense[name + "_dev"]), f"{name} differs from the dense run"
    assert _pad_untouched(obuf, 64) and _pad_untouched(kbuf, 64) and _pad_untouched(vbuf, 64)


def test_single_row_single_head():
    """B = H = N = 1: the strides of one-entry dimensions never enter an
    address (the binding passes 0 for them)."""
    import torch
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 1, 1, 64), seed=4601, dtype="bf16")
    scale = gen.default_scale(64)
    dense = run_gpu(x, "bf16", True, scale)["_dev"]
    _, (q, k, v) = _packed([x["q"], x["k"], x["v"]], "bf16", 8)
    o, lse = fa.forward_strided(q, k, v, True, scale)
    dq, dk, dv = fa.backward_strided(q, k, v, o, to_dev(x["do"], "bf16"), lse, True, scale)
    torch.cuda.synchronize()
    for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(got, dense[name + "_dev"]), name


def test_binding_rejects_views_without_contiguous_rows():
    import torch
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")[..., ::2]
    with pytest.raises(ValueError):
        fa.forward_strided(q, q, q, False, 0.125)
    t = torch.zeros((2, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError):   # an output whose batches land on the same rows
        fa.forward_strided(t, t, t, False, 0.125, out=t[:1].expand(2, -1, -1, -1))
