"""The library under HIP graph capture: it allocates nothing, sets no memory
with hipMemset and only enqueues kernels on the caller's stream, so a whole
forward + backward step (and the split-key-range forward) can be captured
once and replayed.  Each replay is checked bit for bit against the eager
result (the default path is deterministic), with other eager work and
synchronisations between the replays."""
import math

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def _step_tensors(B, H, N, d, seed):
    import torch
    x = gen.make_inputs(gen.workload("c3"), shape=(B, H, N, d), seed=seed)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = fa.workspace(q)
    return dict(q=q, k=k, v=v, do=do, o=o, dq=dq, dk=dk, dv=dv, lse=lse, ws=ws)


def _enqueue_step(t, B, H, N, d, causal, scale, stream):
    P = lambda n: t[n].data_ptr()
    s = stream.cuda_stream
    st = fa.fa_fwd(P("q"), P("k"), P("v"), P("o"), P("lse"), B, H, N, d, causal, scale, s, fa.FA_BF16,
                   fa.FA_LAYOUT_BHND)
    assert st == 0, fa.fa_strerror(st)
    st = fa.fa_bwd(P("q"), P("k"), P("v"), P("o"), P("do"), P("lse"), P("dq"), P("dk"), P("dv"), B, H, N, d,
                   causal, scale, P("ws"), t["ws"].numel(), s, fa.FA_BF16, fa.FA_LAYOUT_BHND)
    assert st == 0, fa.fa_strerror(st)


def _snapshot(t):
    return {n: t[n].clone() for n in ("o", "lse", "dq", "dk", "dv")}


@pytest.mark.parametrize("causal", [False, True])
def test_captured_step_replays_bitwise(causal):
    import torch
    B, H, N, d = 1, 4, 1000, 128
    scale = 1.0 / math.sqrt(d)
    log(f"[graph] fwd+bwd B={B} H={H} N={N} d={d} causal={causal}")
    t = _step_tensors(B, H, N, d, seed=8)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _enqueue_step(t, B, H, N, d, causal, scale, side)
    torch.cuda.synchronize()
    want = _snapshot(t)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _enqueue_step(t, B, H, N, d, causal, scale, torch.cuda.current_stream())
    other = _step_tensors(1, 2, 300, 64, seed=9)
    for rep in range(3):
        for n in ("o", "lse", "dq", "dk", "dv"):
            t[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        # unrelated eager work between the replays
        with torch.cuda.stream(side):
            _enqueue_step(other, 1, 2, 300, 64, True, 0.125, side)
        torch.cuda.synchronize()
        for n, ref in want.items():
            assert torch.equal(t[n], ref), (rep, n)


def test_captured_splitkv_replays_bitwise():
    import torch
    B, H, Nq, Nk, d = 2, 3, 4, 3000, 128
    scale = 1.0 / math.sqrt(d)
    log("[graph] split-key-range forward")
    x = gen.make_decode_inputs(B, H, Nq, Nk, d, seed=12)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    ws = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0), dtype=torch.uint8, device=q.device)
    fa.forward_splitkv(q, k, v, True, scale, out=o, lse=lse, ws=ws)
    torch.cuda.synchronize()
    want_o, want_l = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward_splitkv(q, k, v, True, scale, out=o, lse=lse, ws=ws)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(lse, want_l), rep


def test_captured_dropout_step_replays_bitwise():
    """The dropout forward + backward regenerate their mask from (seed,
    offset) in every kernel and keep no state between calls, so a captured
    step replays to the same bits; a step captured with another offset gives
    another mask."""
    import torch
    B, H, N, d = 1, 4, 777, 128
    scale = 1.0 / math.sqrt(d)
    log(f"[graph] dropout fwd+bwd B={B} H={H} N={N} d={d}")
    t = _step_tensors(B, H, N, d, seed=21)

    def enqueue(offset):
        fa.forward_dropout(t["q"], t["k"], t["v"], True, scale, 0.125, 77, offset, out=t["o"], lse=t["lse"])
        fa.backward_dropout(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], True, scale, 0.125, 77, offset,
                            ws=t["ws"], grads=(t["dq"], t["dk"], t["dv"]))

    enqueue(5)
    torch.cuda.synchronize()
    want = _snapshot(t)
    enqueue(6)
    torch.cuda.synchronize()
    other = _snapshot(t)
    assert not torch.equal(other["o"], want["o"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue(5)
    for rep in range(3):
        for n in ("o", "lse", "dq", "dk", "dv"):
            t[n].fill_(float("nan"))
        t["ws"].fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, ref in want.items():
            assert torch.equal(t[n], ref), (rep, n)


def test_captured_fp8_forward_and_d256_step_replay_bitwise():
    """The FP8 forward and the d = 256 forward + backward enqueue kernels
    only, so captured calls replay to the eager bits."""
    import torch
    log("[graph] FP8 forward and d = 256 step")
    x8 = gen.make_fp8_inputs((1, 4, 700, 128), seed=88)
    q8, k8, v8 = (torch.from_numpy(x8[n]).cuda() for n in ("q8", "k8", "v8"))
    o8 = torch.empty((1, 4, 700, 128), dtype=torch.bfloat16, device="cuda")
    l8 = torch.empty((1, 4, 700), dtype=torch.float32, device="cuda")

    def fp8():
        fa.forward_fp8(q8, k8, v8, x8["descale_q"], x8["descale_k"], x8["descale_v"], True, 128 ** -0.5,
                       out=o8, lse=l8)

    t = _step_tensors(1, 2, 600, 256, seed=89)

    def d256():
        _enqueue_step(t, 1, 2, 600, 256, True, 1.0 / 16.0, torch.cuda.current_stream())

    fp8()
    d256()
    torch.cuda.synchronize()
    want = (o8.clone(), l8.clone(), _snapshot(t))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8()
        d256()
    for rep in range(3):
        o8.fill_(float("nan"))
        l8.fill_(float("nan"))
        for n in ("o", "lse", "dq", "dk", "dv"):
            t[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o8, want[0]) and torch.equal(l8, want[1]), rep
        for n, ref in want[2].items():
            assert torch.equal(t[n], ref), (rep, n)
