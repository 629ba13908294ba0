"""Pins of the stage-by-stage checker (tests/teacher_forcing.py), on the CPU.

* the oracle's own stored activations pass;
* a second correct implementation -- the oracle with every product taken in
  float32 instead of float64 -- passes too (the allowances are wide enough for
  a different summation order), although its free-running logits differ from
  the float64 oracle's;
* each planted mistake (a value off by two ulps, two heads swapped, a
  residual scaled by 1e-4, a backbone layer run where the exit copy should be,
  a key from the wrong position, a drifted cosine, a wrong exit decision, a
  logit off by 1e-3 of the spread) is caught.
"""
import numpy as np
import pytest

import synth
from oracle import river_oracle as ro
from teacher_forcing import check_pass

TAU = 0.5


def _f32_linear(x, w):
    return (np.asarray(x, np.float32) @ np.asarray(w, np.float32).T).astype(np.float64)


def run_recorded(tiny_np, shape, B, T, steps, tau, linear=None):
    """Oracle passes with their stored activations, as the checker takes them."""
    saved = ro.linear
    if linear is not None:
        ro.linear = linear
    try:
        orc = ro.RiverOracle(shape.as_dict(), tiny_np, B, T + steps)
        orc.build_exit_layers("int4")
        toks = synth.make_tokens(shape, B, T, seed=0).numpy()
        passes = []
        res = orc.prefill(toks, tau, record=True)
        passes.append((res, T, 0, orc.k_cache.copy(), orc.v_cache.copy()))
        nxt = res["next"]
        for step in range(steps):
            res = orc.decode_step(nxt, tau, record=True)
            passes.append((res, 1, T + step, orc.k_cache.copy(), orc.v_cache.copy()))
            nxt = res["next"]
    finally:
        ro.linear = saved
    return orc, passes


def as_record(res, B, n):
    R = B * n
    layers = [{k: np.array(v, dtype=np.float64).reshape(R, -1) for k, v in d.items()}
              for d in res["layers"]]
    return layers, np.array(res["h_final"], dtype=np.float64).reshape(R, -1)


def check(orc, tiny_np, shape, res, B, n, start, kc, vc, tau, mutate=None):
    layers, h_out = as_record(res, B, n)
    trace = list(res["trace"]) + [float("nan")] * shape.n_layers   # copies
    logits = np.array(res["logits"], dtype=np.float64)
    nxt = np.array(res["next"])
    E = res["E"]
    kc = kc.copy()
    vc = vc.copy()
    ctx = {"layers": layers, "h_out": h_out, "trace": trace, "logits": logits, "kc": kc, "vc": vc,
           "E": E}
    lwf = lambda l, ex: orc.exit_layers[l] if ex else tiny_np["layers"][l]
    ctx["lw"] = lwf
    if mutate:
        mutate(ctx)
    w_lm = tiny_np["embed"] if tiny_np["lm_head"] is None else tiny_np["lm_head"]
    return check_pass(orc.s, ctx["lw"], ctx["E"], ctx["layers"], ctx["h_out"], ctx["kc"], ctx["vc"],
                      B, n, start, ctx["trace"], tau, ctx["logits"], nxt, tiny_np["final_norm"], w_lm)


@pytest.fixture(scope="module")
def recorded(tiny_np):
    shape = synth.TINY
    orc, passes = run_recorded(tiny_np, shape, 2, 9, 2, TAU)
    assert any(p[0]["E"] < shape.n_layers for p in passes), "no exit in the fixture"
    return orc, passes


def test_oracle_record_passes(tiny_np, recorded):
    orc, passes = recorded
    for res, n, start, kc, vc in passes:
        check(orc, tiny_np, synth.TINY, res, 2, n, start, kc, vc, TAU)


def test_float32_products_pass(tiny_np):
    """A different correct implementation passes stage by stage."""
    shape = synth.TINY
    orc32, passes = run_recorded(tiny_np, shape, 2, 9, 2, TAU, linear=_f32_linear)
    for res, n, start, kc, vc in passes:
        check(orc32, tiny_np, shape, res, 2, n, start, kc, vc, TAU)


def _ulp(x):
    e = np.floor(np.log2(np.abs(x)))
    return 2.0 ** (e - 7)


def _bump_u(ctx):
    u = ctx["layers"][1]["u"]
    i = np.argmax(np.abs(u[0]))
    u[0, i] += 2 * _ulp(u[0, i]) * np.sign(u[0, i])


def _swap_heads(ctx):
    q = ctx["layers"][0]["q"]
    D = synth.TINY.head_dim
    a = q[:, 0:D].copy()
    q[:, 0:D] = q[:, D:2 * D]
    q[:, D:2 * D] = a


def _scale_hmid(ctx):
    ctx["layers"][2]["h_mid"] *= 1.0 + 1e-4


def _backbone_for_exit(ctx):
    lw = ctx["lw"]
    ctx["lw"] = lambda l, ex: lw(l, False)


def _key_from_other_position(ctx):
    kc = ctx["kc"]
    kc[0, 0, :, 3] = kc[0, 0, :, 4]


def _cos_drift(ctx):
    ctx["trace"][0] += 1e-4


def _wrong_decision(ctx):
    ctx["E"] = synth.TINY.n_layers


def _logit_off(ctx):
    lg = ctx["logits"]
    lg[0, 5] += 1e-3 * np.std(lg[0])


@pytest.mark.parametrize("mutate", [_bump_u, _swap_heads, _scale_hmid, _backbone_for_exit,
                                    _key_from_other_position, _cos_drift, _wrong_decision,
                                    _logit_off])
def test_planted_mistakes_are_caught(tiny_np, recorded, mutate):
    orc, passes = recorded
    # the prefill pass (exit taken in it) for most mistakes
    for res, n, start, kc, vc in passes:
        if res["E"] < synth.TINY.n_layers:
            break
    with pytest.raises(AssertionError):
        check(orc, tiny_np, synth.TINY, res, 2, n, start, kc, vc, TAU, mutate=mutate)
