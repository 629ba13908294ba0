"""Invariants the lead page fixes for the river, checked on the oracle.

* an exit layer is a copy of its layer (section 3): unquantised copies must
  reproduce the backbone exactly, whatever the decisions;
* the exit test is the batch minimum of the state-transition similarity
  compared with tau, "exceeds" read as strict, with no re-check after an exit
  (section 4): tau > 1 never exits, tau < -1 always exits after layer 0;
* exit layers write K/V into the original layer's cache slot (section 3);
* prefill takes one decision for the whole prompt (section 5).
"""
import math

import numpy as np
import pytest

import synth
from oracle import river_oracle as ro

B, T, STEPS = 2, 12, 4


def make(tiny_np, mode=ro.EXIT_INT4, max_seq=T + STEPS + 1):
    o = ro.RiverOracle(synth.TINY.as_dict(), tiny_np, B, max_seq)
    o.build_exit_layers(mode)
    return o


def prompt():
    return synth.make_tokens(synth.TINY, B, T, seed=0).numpy()


# ---------------------------------------------------------------------------
# Independent textbook forward: no KV cache, the whole sequence recomputed
# layer by layer with a causal mask, every position with its own weights.
# ---------------------------------------------------------------------------
def textbook_last_logits(s, weights_of_layer, embed, final_norm, w_lm, seq):
    bf = ro.bf16_from_f64
    h = embed[np.asarray(seq)].astype(np.float64)            # [P, d]
    P = h.shape[0]
    D, Hq, Hkv = s.Dh, s.Hq, s.Hkv
    half = D // 2
    for l in range(s.L):
        w = weights_of_layer(l)
        x = np.stack([bf(r / math.sqrt(np.dot(r, r) / s.d + s.eps) * w["attn_norm"]) for r in h])
        q = x @ w["wq"].astype(np.float64).T
        k = x @ w["wk"].astype(np.float64).T
        v = bf(x @ w["wv"].astype(np.float64).T)
        for p in range(P):
            for heads, vec in ((Hq, q), (Hkv, k)):
                for hh in range(heads):
                    a = vec[p, hh * D:hh * D + half].copy()
                    b = vec[p, hh * D + half:(hh + 1) * D].copy()
                    for i in range(half):
                        ang = p * s.theta ** (-2.0 * i / D)
                        vec[p, hh * D + i] = a[i] * math.cos(ang) - b[i] * math.sin(ang)
                        vec[p, hh * D + half + i] = b[i] * math.cos(ang) + a[i] * math.sin(ang)
        q, k = bf(q), bf(k)
        o = np.zeros((P, Hq * D))
        for p in range(P):
            for hh in range(Hq):
                j = hh // (Hq // Hkv)
                qs = q[p, hh * D:(hh + 1) * D]
                sc = np.array([qs @ k[t, j * D:(j + 1) * D] for t in range(p + 1)]) / math.sqrt(D)
                e = np.exp(sc - sc.max())
                o[p, hh * D:(hh + 1) * D] = (e / e.sum()) @ v[:p + 1, j * D:(j + 1) * D]
        h = h + bf(o) @ w["wo"].astype(np.float64).T
        x2 = np.stack([bf(r / math.sqrt(np.dot(r, r) / s.d + s.eps) * w["mlp_norm"]) for r in h])
        g = x2 @ w["w_gate"].astype(np.float64).T
        u = bf(g / (1.0 + np.exp(-g)) * (x2 @ w["w_up"].astype(np.float64).T))
        h = h + u @ w["w_down"].astype(np.float64).T
    r = h[-1]
    xf = bf(r / math.sqrt(np.dot(r, r) / s.d + s.eps) * final_norm)
    return xf @ w_lm.astype(np.float64).T


def run_sequence(o, tau, steps=STEPS, force=None):
    res = [o.prefill(prompt(), tau, force_E=force)]
    for _ in range(steps):
        res.append(o.decode_step(res[-1]["next"], tau, force_E=force))
    return res


def sequences(res):
    p = prompt()
    return [list(p[b]) + [int(r["next"][b]) for r in res[:-1]] for b in range(B)]


@pytest.mark.parametrize("tau,which", [(1.5, "backbone"), (-1.5, "exit_after_0")])
def test_decisions_at_extreme_tau_match_textbook_forward(tiny_np, tau, which):
    o = make(tiny_np)
    res = run_sequence(o, tau)
    want_E = o.s.L if which == "backbone" else 1
    assert all(r["E"] == want_E for r in res)

    def weights_of_layer(l):
        if which == "backbone" or l == 0:
            return tiny_np["layers"][l]
        return o.exit_layers[l]
    seqs = sequences(res)
    for step, r in enumerate(res):
        for b in range(B):
            seq = seqs[b][:T + step]
            want = textbook_last_logits(o.s, weights_of_layer, tiny_np["embed"], tiny_np["final_norm"],
                                        tiny_np["lm_head"], seq)
            got = r["logits"][b]
            assert np.max(np.abs(got - want)) <= 1e-6 * np.std(want), (step, b)


def test_copy_mode_exit_layers_reproduce_backbone_exactly(tiny_np):
    o1 = make(tiny_np, ro.EXIT_COPY)
    o2 = make(tiny_np, ro.EXIT_COPY)
    a = run_sequence(o1, 0.3)
    b = run_sequence(o2, 2.0)
    assert any(r["E"] < o1.s.L for r in a)            # decisions did fire
    assert all(r["E"] == o1.s.L for r in b)
    for ra, rb in zip(a, b):
        assert np.array_equal(ra["logits"], rb["logits"])
    assert np.array_equal(o1.k_cache, o2.k_cache) and np.array_equal(o1.v_cache, o2.v_cache)


def test_int4_exit_changes_the_result(tiny_np):
    # the quantised bank really is used once an exit fires
    a = run_sequence(make(tiny_np), -1.5, steps=1)
    b = run_sequence(make(tiny_np), 1.5, steps=1)
    assert not np.allclose(a[0]["logits"], b[0]["logits"])


def test_trace_is_batch_min_and_no_recheck(tiny_np):
    o = make(tiny_np)
    r0 = o.prefill(prompt(), 2.0, record=True)
    # prefill: the minimum over all B*T prompt rows, one entry per tested layer
    ins = [d["h_in"] for d in r0["layers"]] + [r0["h_final"]]
    assert len(r0["trace"]) == o.s.L - 1
    for l, m in enumerate(r0["trace"]):
        c = ro.cosine_rows(ins[l].reshape(-1, o.s.d), ins[l + 1].reshape(-1, o.s.d))
        assert m == c.min() and c.size == B * T
    r = o.decode_step(r0["next"], 2.0, record=True)
    ins = [d["h_in"] for d in r["layers"]] + [r["h_final"]]
    for l, m in enumerate(r["trace"]):
        c = ro.cosine_rows(ins[l].reshape(-1, o.s.d), ins[l + 1].reshape(-1, o.s.d))
        assert c.size == B and m == c.min()
    # once the exit fires after layer E-1, no deeper layer is tested: the trace holds E entries
    o2 = make(tiny_np)
    o2.prefill(prompt(), 2.0)
    tau = np.float32(r["trace"][1]) - np.float32(1e-6)   # fires at layer 1 at the latest
    r2 = o2.decode_step(r0["next"], float(tau))
    assert r2["E"] <= 2 and len(r2["trace"]) == r2["E"]


def test_exceeds_is_strict(tiny_np):
    o = make(tiny_np)
    o.prefill(prompt(), 2.0)
    probe = o.decode_step(np.array([5, 6]), 2.0)
    m0 = np.float32(probe["trace"][0])
    for tau, fires in ((m0, False), (np.nextafter(m0, np.float32(-2)), True)):
        o2 = make(tiny_np)
        o2.prefill(prompt(), 2.0)
        r = o2.decode_step(np.array([5, 6]), float(tau))
        assert (r["E"] == 1) == fires


def test_exit_kv_lands_in_the_backbone_slot(tiny_np):
    o = make(tiny_np)
    o.prefill(prompt(), 2.0)
    canary = 1234.5
    pos = o.pos
    o.k_cache[:, :, :, pos:] = canary
    o.v_cache[:, :, :, pos:] = canary
    before_k, before_v = o.k_cache.copy(), o.v_cache.copy()
    r = o.decode_step(np.array([7, 9]), -1.5, record=True)    # exits after layer 0
    assert r["E"] == 1
    changed = (o.k_cache != before_k) | (o.v_cache != before_v)
    expect = np.zeros_like(changed)
    expect[:, :B, :, pos, :] = True
    assert np.array_equal(changed, expect)
    # the slots hold the K/V the used path produces from the recorded layer inputs
    for l in range(o.s.L):
        lw = tiny_np["layers"][l] if l < r["E"] else o.exit_layers[l]
        x = ro.bf16_from_f64(ro.rmsnorm(r["layers"][l]["h_in"][:, 0], lw["attn_norm"], o.s.eps))
        k = ro.linear(x, lw["wk"]).reshape(B, 1, o.s.Hkv, o.s.Dh)
        v = ro.linear(x, lw["wv"]).reshape(B, o.s.Hkv, o.s.Dh)
        c, s_ = ro.rope_tables([pos], o.s.Dh, o.s.theta)
        k = ro.bf16_from_f64(ro.apply_rope(k, c, s_))[:, 0]
        assert np.array_equal(o.k_cache[l, :B, :, pos], k)
        assert np.array_equal(o.v_cache[l, :B, :, pos], ro.bf16_from_f64(v))


def test_force_E_replays_a_decision(tiny_np):
    a, b = make(tiny_np), make(tiny_np)
    ra = run_sequence(a, 0.5, steps=2)
    rb = [b.prefill(prompt(), 0.5, force_E=ra[0]["E"])]
    for r in ra[1:]:
        rb.append(b.decode_step(rb[-1]["next"], 0.5, force_E=r["E"]))
    for x, y in zip(ra, rb):
        assert np.array_equal(x["logits"], y["logits"])


def test_call_order_and_bounds(tiny_np):
    o = ro.RiverOracle(synth.TINY.as_dict(), tiny_np, B, T + 1)
    with pytest.raises(RuntimeError):
        o.prefill(prompt(), 0.5)
    o.build_exit_layers()
    with pytest.raises(RuntimeError):
        o.decode_step(np.array([1, 2]), 0.5)
    r = o.prefill(prompt(), 0.5)
    o.decode_step(r["next"], 0.5)
    with pytest.raises(ValueError):
        o.decode_step(r["next"], 0.5)   # cache full
