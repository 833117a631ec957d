"""Host-side checks of the seeded input recipe (no attention arithmetic here)."""
import numpy as np
import pytest

from exact_tiled_attention_online_amd import inputs as gen


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, -2.5e-38, 3.3895314e38], np.float32)])
    # exact ties: bf16 mantissa boundaries with the low 16 bits = 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000) + (0x3F80 << 16)
    x = np.concatenate([x, ties.view(np.float32)])
    ours = gen.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == theirs).all()
    assert (gen.round_bf16(x) == torch.from_numpy(x).to(torch.bfloat16).float().numpy()).all()


def test_inputs_are_seeded_and_shaped():
    w = gen.workload("c1")
    a = gen.make_inputs(w)
    b = gen.make_inputs(w)
    for name in ("q", "k", "v", "do"):
        assert a[name].shape == w.shape and a[name].dtype == np.float32
        assert (a[name] == b[name]).all()
    assert not (a["q"] == a["k"]).all()


def test_bf16_inputs_are_representable_and_spread():
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, 64, 64))
    for name, t in x.items():
        assert (gen.round_bf16(t) == t).all()
    w5 = gen.workload("c5")
    y = gen.make_inputs(w5, shape=(1, 1, 4096, 128))
    assert 1.9 < y["q"].std() < 2.1 and 0.95 < y["v"].std() < 1.05


def test_workload_table():
    assert [w.name.split("_")[0] for w in gen.WORKLOADS] == ["c1", "c2", "c3", "c4", "c5"]
    c4 = gen.workload("c4")
    fwd, bwd = c4.flops()
    assert fwd == 4 * 32 * 8192 ** 2 * 128 / 2 and bwd == 10 * 32 * 8192 ** 2 * 128 / 2
    assert c4.scale == 1 / np.sqrt(128)


def test_decode_inputs_recipe():
    from exact_tiled_attention_online_amd import inputs as gen
    x = gen.make_decode_inputs(2, 3, 4, 50, 64, seed=9)
    assert x["q"].shape == (2, 3, 4, 64) and x["k"].shape == (2, 3, 50, 64) and x["v"].shape == (2, 3, 50, 64)
    y = gen.make_decode_inputs(2, 3, 4, 50, 64, seed=9)
    for n in ("q", "k", "v"):
        np.testing.assert_array_equal(x[n], y[n])
        np.testing.assert_array_equal(gen.round_bf16(x[n]), x[n])
    w = gen.DECODE
    assert w.Nq <= w.Nk and w.kv_bytes() == 2 * w.B * w.H * w.Nk * w.d * 2
