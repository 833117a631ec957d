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


def test_e4m3_table_follows_the_ocp_definition():
    t = gen.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    assert t[0x80] == 0.0 and np.signbit(t[0x80]) and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(np.delete(t, [0x7F, 0xFF])).all()
    assert (np.diff(t[:0x7F]) > 0).all()                 # positive codes are ordered
    # normal values: (1 + m/8) * 2^(e-7)
    for code in (0x09, 0x3C, 0x55, 0x7A):
        e, m = (code >> 3) & 15, code & 7
        assert t[code] == (1 + m / 8) * 2.0 ** (e - 7)


def test_e4m3_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = gen.e4m3_bits(gen.e4m3_to_f32(codes))
    np.testing.assert_array_equal(back[codes != 0x80], codes[codes != 0x80])   # -0 keeps its sign
    assert back[codes == 0x80][0] == 0x80
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 500.0, -1.0625, np.nan], dtype=np.float32)
    assert list(gen.e4m3_bits(x)) == [0x38, 0x3A, 0x00, 0x01, 0x7F, 0xB8, 0x7F]


def test_e4m3_matches_torch_float8():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s for s in (0.001, 0.1, 3.0, 80.0)])
    x = np.clip(x, -448, 448)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(gen.e4m3_bits(x), want)


def test_fp8_inputs_recipe():
    x = gen.make_fp8_inputs((1, 2, 300, 128), seed=4)
    for n in ("q", "k", "v"):
        assert x[n + "8"].dtype == np.uint8 and x[n + "8"].shape == (1, 2, 300, 128)
        np.testing.assert_array_equal(x[n], gen.e4m3_to_f32(x[n + "8"]) * np.float32(x["descale_" + n]))
        assert np.isfinite(x[n]).all() and np.abs(x[n]).max() <= 448 * x["descale_" + n]
    y = gen.make_fp8_inputs((1, 2, 300, 128), seed=4)
    np.testing.assert_array_equal(x["k8"], y["k8"])
