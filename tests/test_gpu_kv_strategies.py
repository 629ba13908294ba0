"""GPU parity of the earlier fixes for the missing K/V of early-exited tokens
(kv mask, state propagation, mono-decreasing exit), the speed comparators of
"River-LLM: Large Language Model Seamless Exit Based on KV Share", section 2,
against the oracle's same strategies (RiverOracle.set_kv_strategy).

Same bar as the method's own parity: exit decisions identical except inside
the 1e-3 window around tau (the oracle then replays the GPU's decision),
logits within 2e-2 x std of the oracle's row, K/V cosine >= 0.999 for every
slot the strategy writes (layers below E for kv mask and mono, every layer
for propagation).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import river_oracle as ro
from test_gpu_parity import (_river, check_decision, compare_kv, compare_logits, kv_numpy, tiny,  # noqa: F401
                             LOGIT_TOL)

pytestmark = pytest.mark.gpu


def compare_kv_layers(gk, gv, orc, layers, B, positions):
    for l in layers:
        compare_kv(gk[l:l + 1], gv[l:l + 1], _Sub(orc, l), 1, B, positions)


class _Sub:
    """An oracle view holding one layer of its cache."""
    def __init__(self, orc, l):
        self.k_cache = orc.k_cache[l:l + 1]
        self.v_cache = orc.v_cache[l:l + 1]


def snapshot(orc):
    """The oracle's sequence state (a replayed pass must start from it: the
    recompute strategy moves earlier positions' states and depths)."""
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in vars(orc).items()
            if k in ("k_cache", "v_cache", "depth", "h_state", "pos_E", "pos", "last_E")}


def restore(orc, snap):
    for k, v in snap.items():
        setattr(orc, k, v.copy() if isinstance(v, np.ndarray) else v)


def compare_kv_deep(gk, gv, orc, L, B, upto):
    """Every (layer, position) the oracle's depth covers (recompute)."""
    for p in range(upto):
        compare_kv_layers(gk, gv, orc, range(int(orc.depth[p])), B, [p])


def run_strategy(tiny, strategy, tau, steps, B=2, T=32, gemv="auto", graph=True):
    rv = _river()
    s = synth.TINY
    L = s.n_layers
    max_seq = T + steps
    print(f"[kv-strategy] {strategy} tau={tau} B={B} T={T} gemv={gemv} graph={graph}", flush=True)
    r = rv.River(s, tiny["cuda"], B, max_seq)
    r.use_graph(graph)
    r.gemv_mode(gemv)
    r.kv_strategy(strategy)
    r.build_exit_layers("int4")
    orc = ro.RiverOracle(s.as_dict(), tiny["np"], B, max_seq)
    orc.set_kv_strategy(strategy)
    orc.build_exit_layers("int4")
    toks = synth.make_tokens(s, B, T, seed=1)
    gl, gn = r.prefill(toks.cuda(), tau)
    st = r.exit_stats()
    o = orc.prefill(toks.numpy(), tau)
    if check_decision(st["last_E"], st["last_trace"], o, tau, L):
        o = orc.prefill(toks.numpy(), tau, force_E=st["last_E"])
    compare_logits(gl.cpu().numpy(), o["logits"])
    E = st["last_E"]
    written = range(L) if strategy in ("river", "propagate") else range(E)
    gk, gv = kv_numpy(r, L, B, T)
    compare_kv_layers(gk, gv, orc, written, B, range(T))
    Es = [E]
    nxt = o["next"]
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(steps):
        tok.copy_(torch.from_numpy(nxt.astype(np.int32)))
        gl, gn = r.decode_step(tok, tau)
        st = r.exit_stats()
        snap = snapshot(orc)
        o = orc.decode_step(nxt, tau)
        if check_decision(st["last_E"], st["last_trace"], o, tau, L):
            restore(orc, snap)
            o = orc.decode_step(nxt, tau, force_E=st["last_E"])
        compare_logits(gl.cpu().numpy(), o["logits"])
        for b in range(B):
            g = int(gn[b])
            assert o["logits"][b, g] >= o["logits"][b].max() - LOGIT_TOL * np.std(o["logits"][b])
        E = st["last_E"]
        pos = T + step
        written = range(L) if strategy in ("river", "propagate") else range(E)
        gk, gv = kv_numpy(r, L, B, pos + 1)
        compare_kv_layers(gk, gv, orc, written, B, [pos])
        if strategy == "recompute":
            compare_kv_deep(gk, gv, orc, L, B, pos + 1)
        Es.append(E)
        nxt = o["next"]
    r.close()
    return Es


@pytest.mark.parametrize("strategy", ["kv_mask", "propagate", "mono"])
@pytest.mark.parametrize("tau", [0.5, -1.5, 1.5])
def test_strategy_parity_tiny(tiny, strategy, tau):
    L = synth.TINY.n_layers
    Es = run_strategy(tiny, strategy, tau, steps=12)
    if tau > 1:
        assert all(e == L for e in Es)
    if tau < -1:
        assert all(e == 1 for e in Es)
    if strategy == "mono":
        assert all(a >= b for a, b in zip(Es[1:], Es[2:])), Es


@pytest.mark.parametrize("tau", [0.5, -1.5, 1.5, 0.9])
def test_recompute_parity_tiny(tiny, tau):
    """One sequence (the recompute comparator runs batch 1)."""
    L = synth.TINY.n_layers
    Es = run_strategy(tiny, "recompute", tau, steps=12, B=1, T=33)
    if tau > 1:
        assert all(e == L for e in Es)
    if tau < -1:
        assert all(e == 1 for e in Es)


@pytest.mark.parametrize("strategy", ["kv_mask", "propagate", "mono"])
def test_strategy_parity_dot_gemv_batch1(tiny, strategy):
    run_strategy(tiny, strategy, 0.5, steps=6, B=1, T=37, gemv="dot")


@pytest.mark.parametrize("strategy", ["kv_mask", "propagate", "mono"])
def test_strategy_parity_mfma_gemv_eager(tiny, strategy):
    run_strategy(tiny, strategy, 0.5, steps=6, B=4, T=29, gemv="mfma", graph=False)


def test_kv_mask_varied_exits(tiny):
    """Exits forced per step so that the mask has holes at several depths;
    the oracle follows the same forced exits."""
    rv = _river()
    s = synth.TINY
    L = s.n_layers
    B, T = 2, 24
    plan = [L, 1, 2, L, 3, 1, L, 2]
    r = rv.River(s, tiny["cuda"], B, T + len(plan))
    r.kv_strategy("kv_mask")
    r.build_exit_layers("int4")
    orc = ro.RiverOracle(s.as_dict(), tiny["np"], B, T + len(plan))
    orc.set_kv_strategy("kv_mask")
    orc.build_exit_layers("int4")
    toks = synth.make_tokens(s, B, T, seed=2)
    r.force_exit_layer(2)
    gl, _ = r.prefill(toks.cuda(), 0.5)
    o = orc.prefill(toks.numpy(), 0.5, force_E=2)
    compare_logits(gl.cpu().numpy(), o["logits"])
    nxt = o["next"]
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    for step, fe in enumerate(plan):
        r.force_exit_layer(fe)
        tok.copy_(torch.from_numpy(nxt.astype(np.int32)))
        gl, _ = r.decode_step(tok, 0.5)
        o = orc.decode_step(nxt, 0.5, force_E=fe)
        compare_logits(gl.cpu().numpy(), o["logits"])
        gk, gv = kv_numpy(r, L, B, T + step + 1)
        compare_kv_layers(gk, gv, orc, range(fe), B, [T + step])
        nxt = o["next"]
    r.close()


@pytest.mark.parametrize("B", [1, 2])
def test_strategies_agree_without_exit(tiny, B):
    """With no exit (tau above 1) every strategy runs the same layers: the
    logits are bitwise those of the method (recompute: one sequence)."""
    rv = _river()
    s = synth.TINY
    outs = []
    for strategy in rv.KV_STRATEGIES:
        if strategy == "recompute" and B != 1:
            continue
        r = rv.River(s, tiny["cuda"], B, 40)
        r.kv_strategy(strategy)
        r.build_exit_layers("int4")
        lg, nx = r.prefill(synth.make_tokens(s, B, 32, seed=0).cuda(), 1.5)
        seq = [lg.clone()]
        for _ in range(4):
            lg, nx = r.decode_step(nx.clone(), 1.5)
            seq.append(lg.clone())
        outs.append(torch.stack(seq).cpu())
        r.close()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_strategy_option_rejects(tiny):
    rv = _river()
    s = synth.TINY
    r = rv.River(s, tiny["cuda"], 2, 40)
    r.build_exit_layers("int4")
    with pytest.raises(rv.RiverError):
        r.set_option(rv.RIVER_OPT_KV_STRATEGY, 5)
    r.kv_strategy("kv_mask")
    r.attn_kind("valu")
    _, nx = r.prefill(synth.make_tokens(s, 2, 32, seed=0).cuda(), 0.5)
    with pytest.raises(rv.RiverError):
        r.decode_step(nx.clone(), 0.5)
    # recompute: one sequence only
    r.attn_kind("mfma")
    r.kv_strategy("recompute")
    with pytest.raises(rv.RiverError):
        r.prefill(synth.make_tokens(s, 2, 32, seed=0).cuda(), 0.5)
    r.close()


def run_forced(shape, w_dev, w_np, strategy, B, T, plan, chunk=0, prefill_E=None, attn="mfma"):
    """Exits forced per pass (prefill at prefill_E, then plan[i] at decode step
    i) on both sides; logits and the K/V slots the strategy writes compared."""
    rv = _river()
    L = len(w_dev["layers"])
    max_seq = T + len(plan)
    sh = synth.shrink(shape, n_layers=L)
    print(f"[kv-strategy] forced {strategy} {shape.name} L={L} B={B} T={T} chunk={chunk} plan={plan}",
          flush=True)
    r = rv.River(sh, w_dev, B, max_seq)
    r.kv_strategy(strategy)
    r.attn_kind(attn)
    if chunk:
        r.set_option(rv.RIVER_OPT_ATTN_CHUNK, chunk)
    r.build_exit_layers("int4")
    orc = ro.RiverOracle(sh.as_dict(), w_np, B, max_seq)
    orc.set_kv_strategy(strategy)
    orc.build_exit_layers("int4")
    toks = synth.make_tokens(sh, B, T, seed=2)
    pe = L if prefill_E is None else prefill_E
    r.force_exit_layer(pe)
    gl, _ = r.prefill(toks.cuda(), 0.5)
    o = orc.prefill(toks.numpy(), 0.5, force_E=pe)
    compare_logits(gl.cpu().numpy(), o["logits"])
    nxt = o["next"]
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    for step, fe in enumerate(plan):
        r.force_exit_layer(fe)
        tok.copy_(torch.from_numpy(nxt.astype(np.int32)))
        gl, _ = r.decode_step(tok, 0.5)
        o = orc.decode_step(nxt, 0.5, force_E=fe)
        compare_logits(gl.cpu().numpy(), o["logits"])
        written = range(L) if strategy == "propagate" else range(fe)
        gk, gv = kv_numpy(r, L, B, T + step + 1)
        compare_kv_layers(gk, gv, orc, written, B, [T + step])
        if strategy == "recompute":
            compare_kv_deep(gk, gv, orc, L, B, T + step + 1)
        nxt = o["next"]
    r.close()


@pytest.mark.parametrize("attn", ["mfma", "valu"])
def test_recompute_forced_exits_tiny(tiny, attn):
    """A prompt that exits after layer 0, then passes deeper and shallower:
    150 pending rows at once (every prompt position through layers 1..3),
    then a few rows at a time, on both attention kernels."""
    L = synth.TINY.n_layers
    run_forced(synth.TINY, tiny["cuda"], tiny["np"], "recompute", 1, 150, [2, L, 1, 3, 2, 1, 1, L],
               prefill_E=1, attn=attn)


@pytest.mark.parametrize("strategy", ["kv_mask", "propagate"])
def test_forced_exits_split_attention_tiny(tiny, strategy):
    """150 cached positions in 64-position chunks: the mask and the skipped
    layers across several attention splits."""
    L = synth.TINY.n_layers
    run_forced(synth.TINY, tiny["cuda"], tiny["np"], strategy, 2, 150, [L, 1, 3, 2, L, 1], chunk=64,
               prefill_E=2)


def run_forced_tf(shape, w_dev, hw, strategy, B, T, plan, chunk=0, prefill_E=None):
    """As run_forced, with every pass checked stage by stage with the oracle
    fed the stored activations (the bar of the full-shape parity tests: a
    free-running float64 oracle drifts from any bf16 implementation by about
    one bf16 ulp of the final state per layer, ~2e-2 of the logit spread on a
    128k vocabulary), and the free-running oracle beside it for the K/V
    cosine bar on the slots the strategy writes."""
    from teacher_forcing import Report, check_pass
    from test_gpu_parity_full import kv_cos
    rv = _river()
    L = len(w_dev["layers"])
    max_seq = T + len(plan)
    sh = synth.shrink(shape, n_layers=L)
    print(f"[kv-strategy] forced+tf {strategy} {shape.name} L={L} B={B} T={T} chunk={chunk} plan={plan}",
          flush=True)
    r = rv.River(sh, w_dev, B, max_seq)
    r.kv_strategy(strategy)
    if chunk:
        r.set_option(rv.RIVER_OPT_ATTN_CHUNK, chunk)
    r.build_exit_layers("int4")
    orc = ro.RiverOracle(sh.as_dict(), hw, B, max_seq)
    orc.set_kv_strategy(strategy)
    orc.build_exit_layers("int4")
    lw = lambda l, ex: orc.exit_layers[l] if ex else hw["layers"][l]
    w_lm = hw["embed"] if hw["lm_head"] is None else hw["lm_head"]
    rep = Report()
    toks = synth.make_tokens(sh, B, T, seed=2)
    pe = L if prefill_E is None else prefill_E
    pos_E = [pe] * T
    r.force_exit_layer(pe)
    gl, gn = r.prefill(toks.cuda(), 0.5)
    orc.prefill(toks.numpy(), 0.5, force_E=pe)
    r.record(B)
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = gn.cpu().numpy().astype(np.int64)
    for step, fe in enumerate(plan):
        pos = T + step
        r.force_exit_layer(fe)
        tok.copy_(torch.from_numpy(nxt.astype(np.int32)))
        gl, gn = r.decode_step(tok, 0.5)
        st = r.exit_stats()
        assert st["last_E"] == fe
        pos_E.append(fe)
        layers, h_out = r.read_record(B)
        k, v = r.kv_views()
        kc = k[:L, :B, :, :pos + 1].double().cpu().numpy()
        vc = v[:L, :B, :, :pos + 1].double().cpu().numpy()
        check_pass(orc.s, lw, fe, layers, h_out, kc, vc, B, 1, pos, st["last_trace"], 0.5,
                   gl.double().cpu().numpy(), gn.cpu().numpy(), hw["final_norm"], w_lm, rep,
                   strategy=strategy, pos_E=pos_E, forced=True)
        orc.decode_step(nxt, 0.5, force_E=fe)
        written = L if strategy == "propagate" else fe
        kv_cos(kc[:written], vc[:written], orc, written, B, pos, pos + 1)
        if strategy == "recompute":
            for p in range(pos + 1):
                dp = int(orc.depth[p])
                kv_cos(kc[:dp], vc[:dp], orc, dp, B, p, p + 1)
        nxt = gn.cpu().numpy().astype(np.int64)
    print(f"[kv-strategy] worst: {rep.worst}", flush=True)
    r.close()


@pytest.fixture(scope="module")
def w8b3():
    from test_gpu_parity_full import host_weights
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=3)
    return w, host_weights(w)


@pytest.mark.parametrize("strategy", ["kv_mask", "propagate", "mono", "recompute"])
def test_forced_exits_8b_layer_shapes(w8b3, strategy):
    """Head dim 128, 4 query heads per K/V head, the full vocabulary: the
    decode kernels at the benchmark's launch shapes under each strategy."""
    w, hw = w8b3
    plan, pe = ([1, 3, 2, 1, 1, 3], 1) if strategy == "recompute" else ([3, 1, 2, 1, 3], 3)
    run_forced_tf(synth.LLAMA_8B, w, hw, strategy, 1, 40, plan, chunk=0, prefill_E=pe)


def test_forced_exits_8b_split_mask(w8b3):
    w, hw = w8b3
    run_forced_tf(synth.LLAMA_8B, w, hw, "kv_mask", 2, 140, [1, 3, 2, 3], chunk=64, prefill_E=2)


@pytest.mark.parametrize("strategy", ["kv_mask", "propagate", "mono"])
def test_strategy_prefill_batch16_tiny(strategy):
    """Prefill of more than 8 rows per position (the batched-row path) under
    each comparator: logits and the written K/V against the oracle's same
    strategy (decode steps of more than 8 rows take only the method)."""
    rv = _river()
    s = synth.TINY
    L = s.n_layers
    B, T = 16, 20
    w = synth.make_weights(s, seed=0)
    from conftest import np_weights
    from test_gpu_parity import to_cuda
    r = rv.River(s, to_cuda(w), B, T + 2)
    r.kv_strategy(strategy)
    r.build_exit_layers("int4")
    orc = ro.RiverOracle(s.as_dict(), np_weights(w), B, T + 2)
    orc.set_kv_strategy(strategy)
    orc.build_exit_layers("int4")
    toks = synth.make_tokens(s, B, T, seed=3)
    for fe in (None, 1, 2):
        r.force_exit_layer(-1 if fe is None else fe)
        r.reset()
        gl, _ = r.prefill(toks.cuda(), 0.5)
        st = r.exit_stats()
        o = orc.prefill(toks.numpy(), 0.5, force_E=fe)
        if fe is None and check_decision(st["last_E"], st["last_trace"], o, 0.5, L):
            o = orc.prefill(toks.numpy(), 0.5, force_E=st["last_E"])
        compare_logits(gl.cpu().numpy(), o["logits"])
        E = st["last_E"]
        written = range(L) if strategy == "propagate" else range(E)
        gk, gv = kv_numpy(r, L, B, T)
        compare_kv_layers(gk, gv, orc, written, B, range(T))
    with pytest.raises(rv.RiverError):
        r.decode_step(torch.zeros(B, dtype=torch.int32, device="cuda"), 0.5)
    r.close()


def test_recompute_state_buffer_rules(tiny):
    """The recompute comparator's state buffer: too small or misaligned ->
    RIVER_E_BAD_SIZE; no buffer, or a decode step after the buffer was
    replaced without a new prefill -> RIVER_E_STATE."""
    import ctypes
    rv = _river()
    s = synth.TINY
    r = rv.River(s, tiny["cuda"], 1, 40)
    r.build_exit_layers("int4")
    lib = r.lib
    small = torch.empty(40 * s.d_model - 1, dtype=torch.float32, device="cuda")
    assert lib.river_set_kv_state(r.ctx, ctypes.c_void_p(small.data_ptr()), small.numel() * 4) == \
        rv.RIVER_E_BAD_SIZE
    big = torch.empty(40 * s.d_model + 8, dtype=torch.float32, device="cuda")
    assert lib.river_set_kv_state(r.ctx, ctypes.c_void_p(big.data_ptr() + 4), 40 * s.d_model * 4) == \
        rv.RIVER_E_BAD_SIZE
    r.set_option(rv.RIVER_OPT_KV_STRATEGY, rv.KV_STRATEGIES.index("recompute"))
    with pytest.raises(rv.RiverError):      # no buffer attached
        r.prefill(synth.make_tokens(s, 1, 16, seed=0).cuda(), 0.5)
    r.kv_strategy("recompute")              # attaches one
    _, nx = r.prefill(synth.make_tokens(s, 1, 16, seed=0).cuda(), 0.5)
    r.decode_step(nx.clone(), 0.5)
    assert lib.river_set_kv_state(r.ctx, ctypes.c_void_p(big.data_ptr()), big.numel() * 4) == 0
    with pytest.raises(rv.RiverError):      # a new buffer starts no sequence
        r.decode_step(nx.clone(), 0.5)
    r.close()
