"""Pins of the oracle's prior-art KV strategies (speed comparators for the
KV-shared exit; the lead page's section 2 describes them in a sentence each):
kv_mask (layers past the exit are skipped, later tokens leave out the K/V
that are missing), propagate (layers past the exit only compute their K/V
from the exit state), mono (skipped as well, the exit layer never increases
along the sequence), recompute (skipped, and the missing K/V are computed by
running the earlier positions through a layer when a later pass reaches it)."""
import math

import numpy as np
import pytest

import synth
from oracle import river_oracle as ro
from test_oracle_invariants import B, T, prompt, textbook_last_logits

STRATS = ("kv_mask", "propagate", "mono", "recompute")


def make(tiny_np, strat, max_seq=T + 6):
    o = ro.RiverOracle(synth.TINY.as_dict(), tiny_np, B, max_seq)
    o.build_exit_layers(ro.EXIT_INT4)
    o.set_kv_strategy(strat)
    return o


def run(o, taus):
    res = [o.prefill(prompt(), taus[0])]
    for tau in taus[1:]:
        res.append(o.decode_step(res[-1]["next"], tau))
    return res


@pytest.mark.parametrize("strat", STRATS)
def test_no_exit_is_the_river(tiny_np, strat):
    """tau > 1 never exits: every strategy is the backbone, bit for bit."""
    a, b = make(tiny_np, "river"), make(tiny_np, strat)
    ra, rb = run(a, [1.5] * 4), run(b, [1.5] * 4)
    for x, y in zip(ra, rb):
        assert x["E"] == y["E"] == synth.TINY.n_layers
        assert np.array_equal(x["logits"], y["logits"])
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.v_cache, b.v_cache)


@pytest.mark.parametrize("strat", STRATS)
def test_exit_after_layer0_is_a_one_layer_model(tiny_np, strat):
    """tau < -1 exits after layer 0 at every pass: the logits are those of
    the one-layer model (layer 0, final norm, LM head), computed by the
    independent textbook forward on the whole sequence."""
    o = make(tiny_np, strat)
    res = run(o, [-1.5] * 4)
    assert all(r["E"] == 1 for r in res)
    s1 = ro.Shape(**synth.shrink(synth.TINY, n_layers=1).as_dict())
    p = prompt()
    seqs = [list(p[b]) + [int(r["next"][b]) for r in res[:-1]] for b in range(B)]
    for step, r in enumerate(res):
        for b in range(B):
            want = textbook_last_logits(s1, lambda l: tiny_np["layers"][0], tiny_np["embed"],
                                        tiny_np["final_norm"], tiny_np["lm_head"], seqs[b][:T + step])
            assert np.max(np.abs(r["logits"][b] - want)) <= 1e-6 * np.std(want), (strat, step, b)


def test_propagate_writes_deeper_kv_from_the_exit_state(tiny_np):
    """propagate, exit after layer 0: the cache of each deeper layer l at a
    position holds bf16(RoPE(x W_k^T)) and bf16(x W_v^T) with
    x = bf16(rmsnorm(h_1, g_l)), h_1 the state after layer 0 (taken here
    from the river oracle run to layer 0 only)."""
    o = make(tiny_np, "propagate")
    o.prefill(prompt(), -1.5)
    ref = ro.RiverOracle(synth.shrink(synth.TINY, n_layers=1).as_dict(),
                         {**tiny_np, "layers": tiny_np["layers"][:1]}, B, T + 6)
    ref.build_exit_layers(ro.EXIT_INT4)
    h1 = ref.prefill(prompt(), 2.0)["h_final"]                 # [B, T, d]
    s = o.s
    D, Hkv = s.Dh, s.Hkv
    half = D // 2
    for l in range(1, s.L):
        w = tiny_np["layers"][l]
        for b in range(B):
            for t in range(T):
                r = h1[b, t]
                x = ro.bf16_from_f64(r / math.sqrt(np.dot(r, r) / s.d + s.eps) * w["attn_norm"])
                k = x @ w["wk"].astype(np.float64).T
                v = ro.bf16_from_f64(x @ w["wv"].astype(np.float64).T)
                for j in range(Hkv):
                    kk = k[j * D:(j + 1) * D]
                    z = (kk[:half] + 1j * kk[half:]) * np.exp(1j * t * s.theta ** (-2.0 * np.arange(half) / D))
                    kr = ro.bf16_from_f64(np.concatenate([z.real, z.imag]))
                    assert np.allclose(o.k_cache[l, b, j, t], kr, rtol=2 ** -7, atol=1e-9), (l, b, t, j)
                    assert np.allclose(o.v_cache[l, b, j, t], v[j * D:(j + 1) * D], rtol=2 ** -7, atol=1e-9)


def test_kv_mask_leaves_out_missing_positions(tiny_np):
    """kv_mask: a prompt that exits after layer 0 leaves no K/V at layers
    1..; a decode step that runs every layer (tau > 1) then attends only to
    itself there, so its attention output at those layers is its own value
    vector for every query head (a softmax over one position)."""
    o = make(tiny_np, "kv_mask")
    r0 = o.prefill(prompt(), -1.5)
    r1 = o.decode_step(r0["next"], 1.5, record=True)
    assert r1["E"] == o.s.L
    s = o.s
    for l in range(1, s.L):
        att = r1["layers"][l]["attn"].reshape(B, s.Hq, s.Dh)
        for b in range(B):
            for h in range(s.Hq):
                j = (h * s.Hkv) // s.Hq
                assert np.array_equal(att[b, h], o.v_cache[l, b, j, T]), (l, b, h)
    # layer 0 holds every position: there the step attends to the whole prompt
    att0 = r1["layers"][0]["attn"].reshape(B, s.Hq, s.Dh)
    assert not np.array_equal(att0[0, 0], o.v_cache[0, 0, 0, T])


def test_mono_exit_layer_never_increases(tiny_np):
    """mono: after a pass that exits at E, a step whose test would not fire
    (tau > 1) still exits at E; a later step may exit earlier, never later."""
    o = make(tiny_np, "mono")
    res = run(o, [0.5, 1.5, 1.5, -1.5, 1.5])
    E = [r["E"] for r in res]
    assert E[0] < o.s.L
    assert E[1] == E[2] == E[0]
    assert E[3] == 1 and E[4] == 1
    assert all(b <= a for a, b in zip(E, E[1:]))
    # the river with the same taus goes back to the full depth
    rr = run(make(tiny_np, "river"), [0.5, 1.5, 1.5, -1.5, 1.5])
    assert rr[1]["E"] == o.s.L


def test_recompute_completes_to_the_backbone(tiny_np):
    """recompute with forced exits: after every pass, each (layer, position)
    that the position's depth covers holds exactly the K/V of the plain
    backbone decoder fed the same tokens, the depth never grows along the
    sequence, and a pass that runs every layer completes the whole cache and
    gives the backbone's logits."""
    L = synth.TINY.n_layers
    plan = [2, 1, 3, 1, 2, L]
    o = make(tiny_np, "recompute", max_seq=T + len(plan) + 1)
    bb = make(tiny_np, "river", max_seq=T + len(plan) + 1)
    r = o.prefill(prompt(), 0.5, force_E=1)
    rb = bb.prefill(prompt(), 0.5, force_E=L)
    nxt = r["next"]

    def same_where_deep(upto):
        for p in range(upto):
            for l in range(int(o.depth[p])):
                for a, b in ((o.k_cache, bb.k_cache), (o.v_cache, bb.v_cache)):
                    assert np.allclose(a[l, :, :, p], b[l, :, :, p], rtol=1e-12, atol=1e-12), (l, p)

    same_where_deep(T)
    assert np.all(o.depth[:T] == 1)
    for i, fe in enumerate(plan):
        r = o.decode_step(nxt, 0.5, force_E=fe)
        rb = bb.decode_step(nxt, 0.5, force_E=L)
        pos = T + i
        assert o.depth[pos] == fe
        assert np.all(np.diff(o.depth[:pos + 1]) <= 0), o.depth[:pos + 1]
        # every earlier position now holds at least this pass's depth
        assert np.all(o.depth[:pos + 1] >= fe)
        same_where_deep(pos + 1)
        nxt = r["next"]
    assert np.all(o.depth[:T + len(plan)] == L)
    assert np.allclose(r["logits"], rb["logits"], rtol=1e-12, atol=1e-12)


def test_recompute_batches_only_missing_rows(tiny_np):
    """After a prompt that exits at 2, a pass that runs 3 layers recomputes
    layer 2 for every prompt position and nothing at layers 0 and 1 (their
    cached K/V stay bit for bit); the positions' depth becomes 3."""
    o = make(tiny_np, "recompute")
    r = o.prefill(prompt(), 0.5, force_E=2)
    k0 = o.k_cache.copy()
    o.decode_step(r["next"], 0.5, force_E=3)
    assert np.array_equal(o.k_cache[:2, :, :, :T], k0[:2, :, :, :T])
    assert not np.array_equal(o.k_cache[2, :, :, :T], k0[2, :, :, :T])
    assert np.all(o.depth[:T + 1] == 3)
