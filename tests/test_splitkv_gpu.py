"""GPU parity of the split-key-range forward (fa_fwd_splitkv, through the C
ABI) against the fp64 oracle's rectangular forward: Nq queries against Nk
keys, the queries being the last Nq positions under the causal mask.

Small and ragged shapes are compared element by element on every head; the
decode workload (8 x 32 heads, 1 query against 16384 cached keys) runs at its
full size in the launch configuration the benchmark uses and is compared on
sampled heads.  Bar: bf16 O within 2e-2 * max|ref| per head, LSE within 1e-3.
"""
import math

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import compare, log, to_dev, to_np
from oracle import ref

pytestmark = pytest.mark.gpu


def run_split(x, causal, scale, num_splits=0, layout=0):
    import torch
    q, k, v = (to_dev(x[n], "bf16", layout) for n in ("q", "k", "v"))
    o, lse = fa.forward_splitkv(q, k, v, causal, scale, num_splits=num_splits, layout=layout)
    torch.cuda.synchronize()
    return {"o": to_np(o, layout), "lse": to_np(lse)}


def check_all_heads(x, causal, scale, got, where):
    want = ref.forward_rect(x["q"], x["k"], x["v"], scale, causal, heads=None)
    o, lse = want
    B, H = o.shape[:2]
    for b in range(B):
        for h in range(H):
            compare({"o": got["o"][b, h], "lse": got["lse"][b, h]}, {"o": o[b, h], "lse": lse[b, h]}, "bf16",
                    names=("o", "lse"), where=f"{where} head ({b},{h})")


CASES = [
    # B, H, Nq, Nk, d, causal, num_splits
    (2, 3, 1, 1000, 128, True, 0),
    (2, 3, 1, 1000, 128, False, 3),
    (1, 4, 7, 513, 64, True, 0),
    (1, 4, 7, 513, 64, False, 1),
    (2, 2, 32, 4096, 128, True, 0),
    (1, 2, 33, 2000, 128, True, 5),
    (1, 2, 100, 100, 64, True, 0),
    (1, 2, 100, 100, 128, False, 4),
    (1, 1, 64, 8192, 128, True, 1024),
    (3, 2, 5, 31, 128, True, 0),
    (2, 2, 3, 777, 96, True, 0),
    (1, 3, 40, 500, 96, False, 2),
    (1, 1, 1, 1, 64, True, 0),
    (2, 3, 1, 1000, 256, True, 0),
    (1, 2, 33, 777, 256, False, 3),
    (1, 2, 100, 100, 256, True, 0),
    (1, 1, 7, 4099, 256, True, 1024),
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,ns", CASES)
def test_splitkv_matches_oracle(B, H, Nq, Nk, d, causal, ns):
    log(f"[splitkv] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={ns}")
    x = gen.make_decode_inputs(B, H, Nq, Nk, d, seed=900 + Nq + Nk + d)
    scale = 1.0 / math.sqrt(d)
    got = run_split(x, causal, scale, ns)
    check_all_heads(x, causal, scale, got, f"splitkv Nq{Nq} Nk{Nk} d{d} c{int(causal)} s{ns}")


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_bnhd_layout_and_split_counts(causal):
    log(f"[splitkv-bnhd] causal={causal}")
    x = gen.make_decode_inputs(2, 3, 9, 700, 128, seed=4321, sigma_qk=2.0)
    scale = 0.1
    results = [run_split(x, causal, scale, ns, layout) for ns in (1, 2, 6, 0)
               for layout in (fa.FA_LAYOUT_BHND, fa.FA_LAYOUT_BNHD)]
    for r in results:
        check_all_heads(x, causal, scale, r, f"bnhd/splits c{int(causal)}")
    # the layout changes addresses only: same split count, same bits
    for i in range(0, len(results), 2):
        for n in ("o", "lse"):
            assert np.array_equal(results[i][n], results[i + 1][n])


def test_splitkv_square_causal_agrees_with_fa_fwd():
    import torch
    log("[splitkv-square]")
    w = gen.workload("c3")
    x = gen.make_inputs(w, shape=(1, 4, 1024, 128), seed=77)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    o1, l1 = fa.forward(q, k, v, True, w.scale)
    o2, l2 = fa.forward_splitkv(q, k, v, True, w.scale)
    torch.cuda.synchronize()
    want = ref.forward_rect(x["q"], x["k"], x["v"], w.scale, True)
    for got in ({"o": to_np(o1), "lse": to_np(l1)}, {"o": to_np(o2), "lse": to_np(l2)}):
        for h in range(4):
            compare({"o": got["o"][0, h], "lse": got["lse"][0, h]},
                    {"o": want[0][0, h], "lse": want[1][0, h]}, "bf16", names=("o", "lse"), where=f"square h{h}")


def test_decode_workload_full_size_sampled_heads():
    import torch
    w = gen.DECODE
    log(f"[decode-full] {w.name}")
    x = gen.make_decode_inputs(w.B, w.H, w.Nq, w.Nk, w.d, seed=w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    got = run_split(x, w.causal, w.scale)
    assert np.isfinite(got["o"]).all() and np.isfinite(got["lse"]).all()
    heads = [(0, 0), (3, 17), (7, 31)]
    want = ref.forward_rect(x["q"], x["k"], x["v"], w.scale, w.causal, heads=heads)
    for (b, h), r in want.items():
        compare({"o": got["o"][b, h], "lse": got["lse"][b, h]}, r, "bf16", names=("o", "lse"),
                where=f"decode head ({b},{h})")
    torch.cuda.empty_cache()


def test_maximum_size_decode_sampled_heads():
    """The split forward at the largest key/value cache the ABI takes for
    8 x 32 heads: one query against Nk = 65535 keys, d = 128 (2.15e9 - 32768
    elements per K and V tensor), bf16 and FP8 (codes of the same values'
    kind); three whole heads against the oracle."""
    import torch
    B, H, Nq, Nk, d = 8, 32, 1, 65535, 128
    assert B * H * Nk * d < 2 ** 31 and B * H * (Nk + 1) * d >= 2 ** 31
    scale, ds = 1.0 / math.sqrt(d), 2.0 ** -5
    log(f"[decode max size] B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    g = torch.Generator(device="cuda").manual_seed(65535)
    q = torch.randn((B, H, Nq, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    k, v = (torch.randn((B, H, Nk, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
            for _ in range(2))
    o, lse = fa.forward_splitkv(q, k, v, True, scale)
    torch.cuda.synchronize()
    heads = ((0, 0), (3, 20), (B - 1, H - 1))
    for b, h in heads:
        want = ref.forward_rect(*(t[b, h].float().cpu().numpy()[None, None] for t in (q, k, v)), scale, True,
                                heads=[(0, 0)])[(0, 0)]
        errs = compare({"o": to_np(o[b, h]), "lse": to_np(lse[b, h])}, want, "bf16", names=("o", "lse"),
                       where=f"decode max size head ({b},{h})")
        log(f"  bf16 head ({b},{h}) max errors {errs}")
    del k, v
    torch.cuda.empty_cache()

    def codes(shape):
        x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
        x.mul_(1.0 / ds).clamp_(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)

    q8, k8, v8 = codes((B, H, Nq, d)), codes((B, H, Nk, d)), codes((B, H, Nk, d))
    o8, lse8 = fa.forward_splitkv_fp8(q8, k8, v8, ds, ds, ds, True, scale)
    torch.cuda.synchronize()
    for b, h in heads:
        qh, kh, vh = (gen.e4m3_to_f32(t[b, h].cpu().numpy()).astype(np.float64) * ds for t in (q8, k8, v8))
        o_ref, lse_ref = ref.head_forward_rect(qh, kh, vh, scale, True)
        # the FP8 bound: P rounded to e4m3 for the P V product
        tol_o = (2.0 ** -4 + Nk * 2.0 ** -17) * float(np.abs(vh).max()) + 2.0 ** -9 * float(np.abs(o_ref).max())
        err_o = float(np.abs(to_np(o8[b, h]) - o_ref).max())
        err_l = float(np.abs(to_np(lse8[b, h]) - lse_ref).max())
        assert err_l <= 1e-3 and err_o <= tol_o, (b, h, err_o, tol_o, err_l)
        log(f"  fp8 head ({b},{h}) O err {err_o:.3e} (bound {tol_o:.3e}), LSE err {err_l:.2e}")
    del q8, k8, v8, o8, lse8
    torch.cuda.empty_cache()
