"""fa_fwd_splitkv_noalloc (through the C ABI): the split-key-range forward
with its partial results in the library's static device array gives the same
bits as fa_fwd_splitkv with a caller workspace, on two calls in a row (the
second with a smaller input, so the array still holds the first call's
partials), and meets the oracle bar; a call needing more than the array holds
returns FA_ERR_SCRATCH and leaves its outputs untouched."""
import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import _lib
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import log, to_dev, to_np
from oracle import ref

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, causal, scale, num_splits, o, lse):
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    s = torch.cuda.current_stream()
    return fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                                     Nq, Nk, d, causal, scale, num_splits, s.cuda_stream, fa.FA_BF16,
                                     fa.FA_LAYOUT_BHND)


# (B, H, Nq, Nk, d, causal, num_splits): the second case is smaller in every
# dimension, so a stale partial of the first call would show if it were read
CASES = [(4, 8, 40, 3000, 128, True, 0), (2, 3, 5, 700, 64, False, 3)]


def test_noalloc_matches_the_workspace_form_on_two_calls():
    import torch
    for B, H, Nq, Nk, d, causal, ns in CASES:
        log(f"[noalloc] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} num_splits={ns}")
        x = gen.make_decode_inputs(B, H, Nq, Nk, d, seed=Nq + Nk)
        q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
        scale = d ** -0.5
        o_ws, l_ws = fa.forward_splitkv(q, k, v, causal, scale, num_splits=ns)
        o = torch.full_like(q, 7.0)
        lse = torch.full((B, H, Nq), 7.0, dtype=torch.float32, device=q.device)
        st = _noalloc(q, k, v, causal, scale, ns, o, lse)
        assert st == _lib.FA_OK, fa.fa_strerror(st)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws) and torch.equal(lse, l_ws), "differs from fa_fwd_splitkv"
        got_o, got_l = to_np(o), to_np(lse)
        for b, h in ((0, 0), (B - 1, H - 1)):
            want = ref.forward_rect(x["q"], x["k"], x["v"], scale, causal, heads=[(b, h)])[(b, h)]
            tol = 2e-2 * max(1e-2, float(np.abs(want["o"]).max()))
            assert float(np.abs(got_o[b, h] - want["o"]).max()) <= tol
            assert float(np.abs(got_l[b, h] - want["lse"]).max()) <= 1e-3


def test_noalloc_rejects_more_than_its_scratch():
    import torch
    B, H, Nq, Nk, d, ns = 1, 64, 64, 8192, 128, 64
    need = fa.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, ns)
    assert need > _lib.FA_SPLITKV_NOALLOC_MAX_BYTES
    log(f"[noalloc] over the limit: {need} bytes needed")
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, Nq), 7.0, dtype=torch.float32, device="cuda")
    assert _noalloc(q, k, k, True, 0.1, ns, o, lse) == _lib.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
