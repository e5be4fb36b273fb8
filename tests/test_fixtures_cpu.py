"""The seeded input generators: bfloat16 rounding against the IEEE definition worked in 64-bit
integers and against values whose roundings are known by hand, and the threaded weight draw
against a serial draw from the same seeds."""
import numpy as np
import pytest

import fixtures as F
from fixtures import synth as S


def _round_u64(a):
    w = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((w + 0x7FFF + ((w >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_rounding_known_values():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties go to 1 + 2^-6
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.0, 0.0, -0.0,
                  3.3895313892515355e38, 1e-40], np.float32)
    # 1e-40 is the subnormal 0x000116C2: its low half is below the tie, so it drops to 0x00010000
    want = np.array([1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -2.0, 0.0, -0.0, 3.3895313892515355e38,
                     float(np.uint32(0x00010000).view(np.float32))], np.float64)
    got = F.to_bf16_values(x).astype(np.float64)
    assert np.array_equal(got, want.astype(np.float32).astype(np.float64))
    assert np.signbit(got[6])
    assert F.to_bf16_bits(np.float32([1.0]))[0] == 0x3F80


@pytest.mark.parametrize("seed", range(3))
def test_bf16_rounding_matches_64_bit_definition(seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # plus exact ties and the largest finite values
    ties = (rng.integers(0, 2**16, 1000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    ext = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x00008000, 0x80008000], np.uint32)
    x = np.concatenate([x, ties.view(np.float32), ext.view(np.float32)])
    x = x[np.isfinite(x)]
    ref = _round_u64(x)
    assert np.array_equal(F.to_bf16_bits(x), ref)
    assert np.array_equal(F.to_bf16_values(x).view(np.uint32), ref.astype(np.uint32) << 16)


def test_bf16_rounding_non_finite_inputs():
    x = np.array([np.inf, -np.inf, 1.5], np.float32)
    assert np.array_equal(F.to_bf16_bits(x), _round_u64(x))
    v = F.to_bf16_values(x)
    assert np.isposinf(v[0]) and np.isneginf(v[1]) and v[2] == 1.5


def test_rounding_leaves_its_input_alone():
    x = np.float32([1 + 2**-8 + 2**-20, 2.5])
    keep = x.copy()
    F.to_bf16_values(x), F.to_bf16_bits(x)
    assert np.array_equal(x, keep)


@pytest.mark.parametrize("cfg", ["tiny", "small_bf16"])
def test_threaded_layer_weights_equal_a_serial_draw(cfg):
    sh = F.get_config(cfg).shape
    d, hq, hkv, dh, f = sh.d_model, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.ffn_dim
    dims = {"q": (hq * dh, d), "k": (hkv * dh, d), "v": (hkv * dh, d), "o": (d, hq * dh),
            "gate": (f, d), "up": (f, d), "down": (d, f)}
    for layer in range(1, sh.n_layers + 1):
        w = F.layer_weights(sh, layer)
        for j, (n, dm) in enumerate(dims.items()):
            ref = F.rng(1, layer, j).standard_normal(dm, dtype=np.float32) * np.float32(0.02)
            if sh.dtype == "bf16":
                ref = (_round_u64(ref).astype(np.uint32) << 16).view(np.float32)
            assert np.array_equal(w["w_" + n], ref), (cfg, layer, n)
    assert S._TENSOR_ID == {n: j for j, n in enumerate(dims)}


def test_int8_quantizer_hand_worked_rows():
    # row 0: max |w| = 1.27 -> s = 0.01; 0.025 / 0.01 = 2.5 exactly in binary? it is not, so use
    # a power-of-two scale: row 1 has max 127 -> s = 1 and exact halves round to even
    w = np.array([[1.27, -0.5, 0.004, 0.0],
                  [127.0, 2.5, 3.5, -2.5],
                  [0.0, 0.0, 0.0, 0.0],
                  [-63.5, 0.25, 0.75, 1.0]], np.float32)
    q, s = F.quantize_int8_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert s[1] == 1.0 and q[1].tolist() == [127, 2, 4, -2]          # ties to even
    assert q[0, 0] == 127 and q[0, 1] == -50 and q[0, 2] == 0 and q[0, 3] == 0
    assert s[2] == 0.0 and q[2].tolist() == [0, 0, 0, 0]              # an all-zero row
    assert s[3] == np.float32(63.5) / np.float32(127) and q[3, 0] == -127
    assert q[3].tolist() == [-127, 0, 2, 2]                           # 0.5 -> 0, 1.5 -> 2, 2.0 -> 2


def test_int8_quantizer_bounds_on_random_rows():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((300, 97)).astype(np.float32) * np.float32(0.02)
    q, s = F.quantize_int8_rows(w)
    assert np.abs(q).max() == 127
    assert (np.abs(q).max(axis=1) == 127).all()                        # every row's max maps to +-127
    err = np.abs(w - q.astype(np.float64) * s[:, None])
    assert (err <= s[:, None] * (0.5 + 1e-6)).all()                    # within half a step


def test_int8_layer_weights_quantize_the_float32_draws():
    sh = F.get_config("small_bf16").shape
    wq = F.layer_weights_int8(sh, 2)
    ref = F.rng(1, 2, 4).standard_normal((sh.ffn_dim, sh.d_model), dtype=np.float32) * np.float32(0.02)
    q, s = F.quantize_int8_rows(ref)
    assert np.array_equal(wq["q_gate"], q) and np.array_equal(wq["s_gate"], s)
    assert wq["q_q"].shape == (sh.n_q_heads * sh.head_dim, sh.d_model)
    assert wq["q_down"].shape == (sh.d_model, sh.ffn_dim) and wq["s_down"].shape == (sh.d_model,)


def test_oracle_dequantize():
    import oracle as O
    wq = {"q_" + n: np.array([[127, -2], [0, 5]], np.int8) for n in ("q", "k", "v", "o", "gate", "up", "down")}
    wq.update({"s_" + n: np.array([0.5, 0.25], np.float32) for n in ("q", "k", "v", "o", "gate", "up", "down")})
    wq["g_attn"] = wq["g_ffn"] = np.ones(2, np.float32)
    w = O.dequantize(wq)
    assert w["w_gate"].tolist() == [[63.5, -1.0], [0.0, 1.25]] and w["w_down"].dtype == np.float32
