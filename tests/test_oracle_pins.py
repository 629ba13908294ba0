"""Pins of the oracle's building blocks against values fixed independently of
it: library routines, closed forms, brute force, hand-derived examples."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import river_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_from_f32_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.4e38, 1e-30], np.float32),
        # exact ties between two bf16 values (lower 16 bits 0x8000), odd and even
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], np.uint32).view(np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = ro.bf16_from_f32(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _bf16_exact(v):
    """Nearest bf16 to a float64 value by exact rational arithmetic (ties even)."""
    if v == 0:
        return 0.0
    f = Fraction(v)
    sgn = -1 if f < 0 else 1
    f = abs(f)
    e = math.floor(math.log2(f))
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    k = f / ulp
    lo = math.floor(k)
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sgn * float(lo * ulp)


def test_bf16_from_f64_exact_rounding():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    # values one float64 ulp either side of a bf16 tie: float32 double rounding
    # would get some of these wrong
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 5.0 + 2.0 ** -6])
    x = np.concatenate([x, ties, np.nextafter(ties, 0), np.nextafter(ties, 10)])
    got = ro.bf16_from_f64(x)
    want = np.array([_bf16_exact(v) for v in x])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- quantiser
def test_quantizer_hand_worked_examples():
    with open(os.path.join(GOLDEN, "quant_worked_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        w = np.array([e["w"]], np.float32)
        q, s, z = ro.quantize_int4(w, e["group"])
        assert q[0].tolist() == e["q"], e["name"]
        assert float(s[0, 0]) == e["s"], e["name"]
        assert float(z[0, 0]) == e["z"], e["name"]
        wh = ro.dequantize_int4(q, s, z, e["group"])
        assert wh[0].tolist() == e["w_hat"], e["name"]


def test_quantizer_error_bound_and_code_range():
    rng = np.random.default_rng(2)
    for group in (4, 64, 128):
        w = torch.from_numpy(rng.standard_normal((48, 4 * group)).astype(np.float32) * 0.02)
        w = w.to(torch.bfloat16).float().numpy()
        q, s, z = ro.quantize_int4(w, group)
        assert q.dtype == np.uint8 and q.max() <= 15
        wh = ro.dequantize_int4(q, s, z, group)
        err = np.abs(wh - w).reshape(48, 4, group)
        # half a step, plus what bf16 rounding of s and z can add: s carries a
        # relative error up to 2^-9 over 15 steps, z up to half its bf16 ulp
        zulp = np.abs(z) * 2.0 ** -8 + 1e-30
        bound = s * (0.5 + 15 * 2.0 ** -9 + zulp) + 1e-7
        assert np.all(err <= bound[..., None])
        # every group uses both ends of the code range
        qg = q.reshape(48, 4, group)
        assert np.all(qg.min(-1) <= 1) and np.all(qg.max(-1) >= 14)


def test_quantizer_groups_run_along_input_columns():
    # a matrix that is constant on each (row, column group) is reproduced exactly,
    # and only if the groups are taken along the input dimension
    group = 8
    vals = np.array([[0.5, -1.0, 2.0], [0.25, 4.0, -0.125]], np.float32)
    w = np.repeat(vals, group, axis=1)
    q, s, z = ro.quantize_int4(w, group)
    assert np.array_equal(ro.dequantize_int4(q, s, z, group), w)
    assert s.shape == (2, 3)


def test_quantizer_rejects_ragged_groups():
    with pytest.raises(ValueError):
        ro.quantize_int4(np.zeros((2, 10), np.float32), 4)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    eps = 1e-5
    c = 0.37
    h = np.full((1, 16), c)
    g = np.linspace(0.5, 2.0, 16)
    want = g * c / math.sqrt(c * c + eps)
    assert np.allclose(ro.rmsnorm(h, g, eps)[0], want, rtol=1e-14)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 64))
    y = ro.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)
    assert np.allclose(ro.rmsnorm(5.0 * x, np.ones(64), 0.0), y, rtol=1e-12)


# ---------------------------------------------------------------- RoPE
def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(4)
    D, theta = 16, 500000.0
    pos = np.array([0, 1, 7, 300, 16383])
    x = rng.standard_normal((len(pos), 3, D))
    cos, sin = ro.rope_tables(pos, D, theta)
    got = ro.apply_rope(x, cos, sin)
    # rotate-half RoPE as complex multiplication: (x_i + j x_{i+D/2}) e^{j pos theta^(-2i/D)}
    half = D // 2
    zc = x[..., :half] + 1j * x[..., half:]
    freq = np.array([theta ** (-2.0 * i / D) for i in range(half)])
    rot = np.exp(1j * pos[:, None, None] * freq[None, None, :])
    zr = zc * rot
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_rope_properties():
    rng = np.random.default_rng(5)
    D, theta = 64, 500000.0
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    c0, s0 = ro.rope_tables([0], D, theta)
    assert np.array_equal(ro.apply_rope(q, c0, s0), q)  # identity at position 0
    c, s = ro.rope_tables([123], D, theta)
    assert np.isclose(np.linalg.norm(ro.apply_rope(q, c, s)), np.linalg.norm(q), rtol=1e-13)

    def dot(m, n):
        cm, sm = ro.rope_tables([m], D, theta)
        cn, sn = ro.rope_tables([n], D, theta)
        return float(np.sum(ro.apply_rope(q, cm, sm) * ro.apply_rope(k, cn, sn)))
    assert np.isclose(dot(10, 3), dot(107, 100), rtol=1e-10)
    assert np.isclose(dot(5, 5), float(np.sum(q * k)), rtol=1e-12)


# ---------------------------------------------------------------- attention
def _attention_brute(q, kc, vc, start, n):
    B, _, Hq, D = q.shape
    Hkv = kc.shape[1]
    out = np.zeros_like(q, dtype=np.float64)
    for b in range(B):
        for i in range(n):
            p = start + i
            for h in range(Hq):
                j = h // (Hq // Hkv)
                sc = [sum(q[b, i, h, d] * kc[b, j, t, d] for d in range(D)) / math.sqrt(D) for t in range(p + 1)]
                mx = max(sc)
                e = [math.exp(v - mx) for v in sc]
                tot = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[t] / tot * vc[b, j, t, d] for t in range(p + 1))
    return out


@pytest.mark.parametrize("start,n", [(0, 5), (4, 1), (7, 1), (2, 3)])
def test_attention_matches_brute_force(start, n):
    rng = np.random.default_rng(6 + start)
    B, Hq, Hkv, D, S = 2, 4, 2, 4, 10
    q = rng.standard_normal((B, n, Hq, D))
    kc = rng.standard_normal((B, Hkv, S, D))
    vc = rng.standard_normal((B, Hkv, S, D))
    got = ro.attention(q, kc, vc, start, n)
    want = _attention_brute(q, kc, vc, start, n)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, S = 1, 2, 1, 8, 6
    kc = np.tile(rng.standard_normal((1, 1, 1, D)), (B, Hkv, S, 1))  # all keys equal
    vc = rng.standard_normal((B, Hkv, S, D))
    q = rng.standard_normal((B, 1, Hq, D))
    out = ro.attention(q, kc, vc, 4, 1)
    assert np.allclose(out[0, 0, 0], vc[0, 0, :5].mean(axis=0), rtol=1e-12)
    out0 = ro.attention(q, kc, vc, 0, 1)  # a single visible position
    assert np.allclose(out0[0, 0, 1], vc[0, 0, 0], rtol=1e-14)


# ---------------------------------------------------------------- cosine, silu, linear, greedy
def test_cosine_closed_forms():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 33))
    assert np.allclose(ro.cosine_rows(x, x), 1.0)
    assert np.allclose(ro.cosine_rows(x, -x), -1.0)
    assert np.allclose(ro.cosine_rows(x, 3.5 * x + 0.0), 1.0)
    a = np.array([[1.0, 0.0], [1.0, 1.0]])
    b = np.array([[0.0, 2.0], [1.0, 0.0]])
    assert np.allclose(ro.cosine_rows(a, b), [0.0, 1 / math.sqrt(2)])
    assert ro.cosine_rows(np.zeros((1, 3)), np.ones((1, 3)))[0] == 0.0


def test_silu_closed_forms():
    assert ro.silu(np.array(0.0)) == 0.0
    assert np.isclose(ro.silu(np.array(40.0)), 40.0)
    assert np.isclose(ro.silu(np.array(1.0)), 1.0 / (1.0 + math.exp(-1.0)))


def test_linear_is_row_major_weight_product():
    x = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 1.0]])  # [N=2][K=3]
    assert ro.linear(x, w).tolist() == [[1.0, 5.0]]


def test_greedy_lowest_index_on_ties():
    assert ro.greedy(np.array([[1.0, 3.0, 3.0, 2.0]])).tolist() == [1]


# ---------------------------------------------------------------- one layer, closed form
def test_layer_with_only_value_and_output_paths():
    """With q = k = 0 and a single visible position, attention returns v, so the
    layer is h + (expand_gqa(x Wv^T)) Wo^T (+ 0 MLP when W_down = 0)."""
    s = ro.Shape(1, 8, 4, 2, 2, 16, 10, 4, False)
    rng = np.random.default_rng(9)

    def bf(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    lw = {
        "attn_norm": np.ones(8, np.float32), "mlp_norm": np.ones(8, np.float32),
        "wq": np.zeros((8, 8), np.float32), "wk": np.zeros((4, 8), np.float32),
        "wv": bf(rng.standard_normal((4, 8))), "wo": bf(rng.standard_normal((8, 8))),
        "w_gate": bf(rng.standard_normal((16, 8))), "w_up": bf(rng.standard_normal((16, 8))),
        "w_down": np.zeros((8, 16), np.float32),
    }
    h = rng.standard_normal((1, 1, 8))
    kc = np.zeros((1, 2, 4, 2))
    vc = np.zeros((1, 2, 4, 2))
    out = ro.decoder_layer(s, lw, h, 0, kc, vc)
    x = ro.bf16_from_f64(h[0, 0] / math.sqrt(np.mean(h[0, 0] ** 2) + s.eps))
    v = ro.bf16_from_f64(lw["wv"].astype(np.float64) @ x)           # [Hkv*D] = kv heads 0,1
    o = np.concatenate([v[0:2], v[0:2], v[2:4], v[2:4]])             # q heads 0,1 -> kv 0; 2,3 -> kv 1
    want = h[0, 0] + lw["wo"].astype(np.float64) @ ro.bf16_from_f64(o)
    assert np.allclose(out[0, 0], want, rtol=1e-12, atol=1e-12)
    assert np.allclose(vc[0, :, 0].reshape(-1), v)                   # this position's slot holds v


def test_kv_bytes_reproduce_printed_memory_figures():
    """bf16 parameters plus one bf16 cache reproduce the original model's peak
    memory at 16K and 64K tokens as printed; River-LLM grows by the same amount
    between those contexts, i.e. it keeps a single cache."""
    with open(os.path.join(GOLDEN, "memory_pages.json")) as f:
        g = json.load(f)
    s = ro.Shape(32, 4096, 32, 8, 128, 14336, 128256, 128, False)
    per_layer = (s.Hq + 2 * s.Hkv) * s.Dh * s.d + s.d * s.Hq * s.Dh + 3 * s.F * s.d + 2 * s.d
    params = 2 * s.V * s.d + s.L * per_layer + s.d
    orc = ro.RiverOracle.__new__(ro.RiverOracle)
    orc.s = s
    kvb = orc.kv_bytes_per_token()
    assert kvb == 131072
    gib = 2.0 ** 30
    assert round((2 * params + 16384 * kvb) / gib, 2) == g["original_16k"]
    assert round((2 * params + 65536 * kvb) / gib, 2) == g["original_64k"]
    assert round(g["river_64k"] - g["river_16k"], 2) == round((65536 - 16384) * kvb / gib, 2)
