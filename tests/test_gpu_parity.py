"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Rules (from the method's target accuracy):
  * int4 codes, scales and zeros: bit-exact;
  * per-layer exit decisions identical except where |min cos - tau| < 1e-3
    (the oracle then replays the GPU's decision with force_E);
  * logits: max |diff| <= 2e-2 * std of the oracle's logits of that row, with
    both sides fed the same (oracle-greedy) tokens;
  * K/V: cosine >= 0.999 with the oracle's, per (layer, row, position).
"""
import math

import numpy as np
import pytest
import torch

import synth
from conftest import np_weights
from oracle import river_oracle as ro

pytestmark = pytest.mark.gpu

WINDOW = 1e-3
LOGIT_TOL = 2e-2
KV_COS = 0.999


def _river():
    from early_exit_kv_amd import river as rv
    return rv


def to_cuda(w):
    return {
        "embed": w["embed"].cuda(), "final_norm": w["final_norm"].cuda(),
        "lm_head": None if w["lm_head"] is None else w["lm_head"].cuda(),
        "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w["layers"]],
    }


@pytest.fixture(scope="module")
def tiny():
    w = synth.make_weights(synth.TINY, seed=0)
    return {"cpu": w, "np": np_weights(w), "cuda": to_cuda(w)}


def kv_numpy(r, L, B, upto):
    k, v = r.kv_views()
    return (k[:L, :B, :, :upto].float().cpu().numpy(), v[:L, :B, :, :upto].float().cpu().numpy())


def check_decision(gpu_E, gpu_trace, orc_res, tau, L):
    """Same E, or a differing decision whose deciding cosine sits inside the window."""
    oE = orc_res["E"]
    if gpu_E == oE:
        return False
    first = min(gpu_E, oE) - 1          # the layer where one side exited and the other did not
    m = orc_res["trace"][first] if first < len(orc_res["trace"]) else gpu_trace[first]
    assert abs(m - tau) < WINDOW, f"decisions differ outside the window: gpu E={gpu_E} oracle E={oE} m={m}"
    return True


def compare_logits(gl, ol):
    gl = np.asarray(gl, dtype=np.float64)
    for b in range(ol.shape[0]):
        tol = LOGIT_TOL * np.std(ol[b])
        err = np.max(np.abs(gl[b] - ol[b]))
        assert err <= tol, f"row {b}: max|dlogit|={err} > {tol}"


def compare_kv(gk, gv, orc, L, B, positions):
    for l in range(L):
        for b in range(B):
            for p in positions:
                for name, g, o in (("K", gk, orc.k_cache), ("V", gv, orc.v_cache)):
                    a = g[l, b, :, p].reshape(-1).astype(np.float64)
                    c = o[l, b, :, p].reshape(-1)
                    cos = a @ c / max(np.linalg.norm(a) * np.linalg.norm(c), 1e-30)
                    assert cos >= KV_COS, f"{name} l={l} b={b} p={p} cos={cos}"


def run_parity(tiny, tau, steps, mode="int4", graph=True, B=2, T=32):
    rv = _river()
    s = synth.TINY
    max_seq = T + steps
    print(f"[parity] tiny tau={tau} mode={mode} graph={graph} B={B} T={T} steps={steps}", flush=True)
    r = rv.River(s, tiny["cuda"], B, max_seq, copy_bank=(mode == "copy"))
    r.use_graph(graph)
    r.build_exit_layers(mode)
    orc = ro.RiverOracle(s.as_dict(), tiny["np"], B, max_seq)
    orc.build_exit_layers(mode)
    toks = synth.make_tokens(s, B, T, seed=0)
    gl, gn = r.prefill(toks.cuda(), tau)
    st = r.exit_stats()
    o = orc.prefill(toks.numpy(), tau)
    if check_decision(st["last_E"], st["last_trace"], o, tau, s.n_layers):
        o = orc.prefill(toks.numpy(), tau, force_E=st["last_E"])
    compare_logits(gl.cpu().numpy(), o["logits"])
    gk, gv = kv_numpy(r, s.n_layers, B, T)
    compare_kv(gk, gv, orc, s.n_layers, B, range(T))
    Es = [st["last_E"]]
    nxt = o["next"]
    tok_buf = torch.empty(B, dtype=torch.int32, device="cuda")
    for step in range(steps):
        tok_buf.copy_(torch.from_numpy(nxt.astype(np.int32)))
        gl, gn = r.decode_step(tok_buf, tau)
        st = r.exit_stats()
        o = orc.decode_step(nxt, tau)
        if check_decision(st["last_E"], st["last_trace"], o, tau, s.n_layers):
            orc.pos -= 1
            o = orc.decode_step(nxt, tau, force_E=st["last_E"])
        compare_logits(gl.cpu().numpy(), o["logits"])
        # greedy token of the GPU must be an argmax of the oracle within tolerance
        for b in range(B):
            g = int(gn[b])
            assert o["logits"][b, g] >= o["logits"][b].max() - LOGIT_TOL * np.std(o["logits"][b])
        pos = T + step
        gk, gv = kv_numpy(r, s.n_layers, B, pos + 1)
        compare_kv(gk, gv, orc, s.n_layers, B, [pos])
        # traces agree on the layers both sides tested
        for l, m in enumerate(o["trace"]):
            gm = st["last_trace"][l]
            if not math.isnan(gm):
                assert abs(gm - m) < 2e-3, (step, l, gm, m)
        Es.append(st["last_E"])
        nxt = o["next"]
    stats = r.exit_stats()
    r.close()
    return Es, stats


def test_quantizer_bit_exact_tiny(tiny):
    rv = _river()
    s = synth.TINY
    r = rv.River(s, tiny["cuda"], 2, 48)
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    for l in range(s.n_layers):
        for i, name in enumerate(rv.LINEAR_NAMES):
            words, sz = r.exit_linear_packed(l, i)
            q, sc, z = rv.unpack_int4(words.cpu().numpy(), sz.cpu().numpy(), s.group_size)
            oq, osc, oz = ro.quantize_int4(tiny["np"]["layers"][l][name], s.group_size)
            assert np.array_equal(q, oq), (l, name)
            assert np.array_equal(sc.view(np.uint32), osc.view(np.uint32)), (l, name)
            assert np.array_equal(z.view(np.uint32), oz.view(np.uint32)), (l, name)
    r.close()


@pytest.mark.parametrize("tau", [0.5, -1.5, 1.5])
def test_decode_parity_tiny(tiny, tau):
    Es, stats = run_parity(tiny, tau, steps=16)
    L = synth.TINY.n_layers
    if tau > 1:
        assert all(e == L for e in Es)
    if tau < -1:
        assert all(e == 1 for e in Es)
    assert stats["n_decode_steps"] == 16 and sum(stats["decode_hist"]) == 16
    assert stats["n_prefill"] == 1


def test_decode_parity_tiny_eager(tiny):
    run_parity(tiny, 0.5, steps=4, graph=False)


def test_parity_batch1_ragged_prompt(tiny):
    # a prompt length that is not a multiple of any tile, one row
    run_parity(tiny, 0.5, steps=3, B=1, T=37)


def test_copy_mode_equals_backbone_on_gpu(tiny):
    rv = _river()
    s = synth.TINY
    outs = []
    for tau in (0.3, 1.5):
        r = rv.River(s, tiny["cuda"], 2, 40, copy_bank=True)
        r.build_exit_layers("copy")
        toks = synth.make_tokens(s, 2, 32, seed=0).cuda()
        lg, nx = r.prefill(toks, tau)
        seq = [lg.clone()]
        Es = []
        for _ in range(6):
            lg, nx = r.decode_step(nx.clone(), tau)
            seq.append(lg.clone())
            Es.append(r.exit_stats()["last_E"])
        k, v = r.kv_views()
        outs.append((torch.stack(seq).cpu(), k.clone().cpu(), v.clone().cpu(), Es))
        r.close()
    assert any(e < s.n_layers for e in outs[0][3])
    assert all(e == s.n_layers for e in outs[1][3])
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])


@pytest.mark.parametrize("B", [2, 16])
def test_decode_steps_match_single_steps_bitwise(tiny, B):
    """river_decode_steps (several steps per call, tokens fed back on the
    device, one recorded graph per call shape) against the same steps one
    call each: identical next tokens, last logits, K/V cache and exit
    histogram.  Four calls of two steps over two alternating next-token
    buffers, so the fourth replays the second's graph; also eager."""
    rv = _river()
    s = synth.TINY
    toks = synth.make_tokens(s, B, 32, seed=0).cuda()

    def single():
        r = rv.River(s, tiny["cuda"], B, 48)
        r.build_exit_layers("int4")
        _, nx = r.prefill(toks, 0.5)
        outs = []
        for _ in range(8):
            lg, nx = r.decode_step(nx.clone(), 0.5)
            outs.append(nx.clone())
        torch.cuda.synchronize()
        k, v = r.kv_views()
        st = r.exit_stats()
        res = (torch.stack(outs).cpu(), lg.cpu(), k.clone().cpu(), v.clone().cpu(),
               (st["decode_hist"], st["pos"], st["n_decode_steps"]))
        r.close()
        return res

    def multi(graph):
        r = rv.River(s, tiny["cuda"], B, 48)
        r.use_graph(graph)
        r.build_exit_layers("int4")
        _, nx = r.prefill(toks, 0.5)
        ring = [torch.empty((2, B), dtype=torch.int32, device="cuda") for _ in range(2)]
        logits = torch.empty((B, s.vocab), dtype=torch.float32, device="cuda")
        ring[1][1].copy_(nx)
        outs = []
        for c in range(4):
            src, dst = ring[(c + 1) % 2][1], ring[c % 2]
            r.decode_steps(src, 2, 0.5, logits=logits, next_tok=dst)
            torch.cuda.synchronize()   # eager host work between replays
            outs.append(dst.clone())
        k, v = r.kv_views()
        st = r.exit_stats()
        res = (torch.cat(outs).cpu(), logits.cpu(), k.clone().cpu(), v.clone().cpu(),
               (st["decode_hist"], st["pos"], st["n_decode_steps"]))
        r.close()
        return res

    ref = single()
    for graph in (True, False):
        got = multi(graph)
        assert torch.equal(got[0], ref[0]), f"graph={graph}: next tokens"
        assert torch.equal(got[1], ref[1]), f"graph={graph}: last logits"
        assert torch.equal(got[2], ref[2]) and torch.equal(got[3], ref[3]), f"graph={graph}: K/V cache"
        assert got[4] == ref[4], f"graph={graph}: exit histogram, position, step count"


def test_graph_replay_matches_eager_bitwise(tiny):
    rv = _river()
    s = synth.TINY
    res = []
    for graph in (True, False):
        r = rv.River(s, tiny["cuda"], 2, 48)
        r.use_graph(graph)
        r.build_exit_layers("int4")
        toks = synth.make_tokens(s, 2, 32, seed=0).cuda()
        lg, nx = r.prefill(toks, 0.5)
        tok = torch.empty(2, dtype=torch.int32, device="cuda")
        seq = []
        for _ in range(8):
            tok.copy_(nx)
            lg, nx = r.decode_step(tok, 0.5)
            torch.cuda.synchronize()   # eager host work between replays
            seq.append(lg.clone())
        k, v = r.kv_views()
        res.append((torch.stack(seq).cpu(), k.clone().cpu(), r.exit_stats()["decode_hist"]))
        r.close()
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
    assert res[0][2] == res[1][2]


def test_exit_kv_lands_in_backbone_slot_on_gpu(tiny):
    rv = _river()
    s = synth.TINY
    B, T = 2, 32
    r = rv.River(s, tiny["cuda"], B, 40)
    r.build_exit_layers("int4")
    toks = synth.make_tokens(s, B, T, seed=0).cuda()
    _, nx = r.prefill(toks, -1.5)
    k, v = r.kv_views()
    canary = 1234.0
    k[:, :, :, T:] = canary
    v[:, :, :, T:] = canary
    before_k, before_v = k.clone(), v.clone()
    r.decode_step(nx.clone(), -1.5)     # exits after layer 0: layers 1.. are exit layers
    torch.cuda.synchronize()
    assert r.exit_stats()["last_E"] == 1
    changed = (k != before_k) | (v != before_v)
    expect = torch.zeros_like(changed)
    expect[:, :B, :, T, :] = True
    # every element of the written slots changes from the canary, nothing else moves
    assert torch.equal(changed, expect)
    r.close()


def test_forced_exit_layers(tiny):
    """force_E = L runs the original model; force_E = 0 every layer quantised;
    each matches the oracle with the same forcing."""
    rv = _river()
    s = synth.TINY
    for fe in (0, s.n_layers, 2):
        r = rv.River(s, tiny["cuda"], 2, 40)
        r.build_exit_layers("int4")
        r.force_exit_layer(fe)
        orc = ro.RiverOracle(s.as_dict(), tiny["np"], 2, 40)
        orc.build_exit_layers("int4")
        toks = synth.make_tokens(s, 2, 32, seed=0)
        gl, gn = r.prefill(toks.cuda(), 0.5)
        o = orc.prefill(toks.numpy(), 0.5, force_E=fe)
        compare_logits(gl.cpu().numpy(), o["logits"])
        tok = torch.from_numpy(o["next"].astype(np.int32)).cuda()
        gl, gn = r.decode_step(tok, 0.5)
        o = orc.decode_step(o["next"], 0.5, force_E=fe)
        compare_logits(gl.cpu().numpy(), o["logits"])
        st = r.exit_stats()
        assert st["last_E"] == fe and st["decode_hist"][fe] == 1
        r.close()


def test_gpu_error_paths(tiny):
    rv = _river()
    s = synth.TINY
    r = rv.River(s, tiny["cuda"], 2, 34)
    r.build_exit_layers("int4")
    toks = synth.make_tokens(s, 2, 32, seed=0).cuda()
    with pytest.raises(rv.RiverError) as e:
        r.prefill(synth.make_tokens(s, 3, 8).cuda(), 0.5)   # B > max_batch
    assert e.value.code == rv.RIVER_E_RANGE
    with pytest.raises(rv.RiverError) as e:
        r.prefill(synth.make_tokens(s, 2, 35).cuda(), 0.5)  # T > max_seq
    assert e.value.code == rv.RIVER_E_RANGE
    _, nx = r.prefill(toks, 0.5)
    r.decode_step(nx.clone(), 0.5)
    r.decode_step(nx.clone(), 0.5)
    with pytest.raises(rv.RiverError) as e:
        r.decode_step(nx.clone(), 0.5)                      # cache full (34 positions)
    assert e.value.code == rv.RIVER_E_RANGE
    bad = torch.tensor([5, s.vocab + 7], dtype=torch.int32, device="cuda")
    r.reset()
    r.prefill(toks, 0.5)
    r.decode_step(bad, 0.5)
    assert r.exit_stats()["token_errors"] == 1
    r.close()


def test_record_and_kernel_timing_entry_points(tiny):
    """Activation record: too small a buffer is refused before any launch, and
    recording does not change what a step computes; kernel timing returns a
    positive time and refuses classes it cannot time alone."""
    rv = _river()
    s = synth.TINY
    toks = synth.make_tokens(s, 2, 8, seed=0).cuda()
    outs = []
    for rec in (False, True):
        r = rv.River(s, tiny["cuda"], 2, 12)
        r.build_exit_layers("int4")
        if rec:
            r.record(2)                                       # room for 2 rows only
            with pytest.raises(rv.RiverError) as e:
                r.prefill(toks, 0.5)                          # 16 rows
            assert e.value.code == rv.RIVER_E_BAD_SIZE
            r.record(16)
        gl, nx = r.prefill(toks, 0.5)
        g2, _ = r.decode_step(nx.clone(), 0.5)
        outs.append((gl.cpu(), g2.cpu()))
        if rec:
            layers, h_out = r.read_record(2)
            assert len(layers) == s.n_layers and h_out.shape == (2, s.d_model)
            assert np.all(np.isfinite(h_out))
            for kind in ("qkv", "attn", "o", "gateup", "down"):
                t = r.time_kernel(kind, reps=3)
                assert 0.0 < t < 1e5, (kind, t)
            with pytest.raises(rv.RiverError) as e:
                r.time_kernel("lm_head")
            assert e.value.code == rv.RIVER_E_INVALID_ARG
        r.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_tau_sweep_replays_one_graph(tiny):
    """tau lives in the control block: decode steps with different tau replay
    the same recorded step and take each tau's decision (tau > 1 never exits,
    tau < -1 exits after the first layer), bit for bit as eager launches do."""
    rv = _river()
    s = synth.TINY
    L = s.n_layers
    toks = synth.make_tokens(s, 2, 16, seed=0).cuda()
    taus = [2.0, -1.5, 0.5, 2.0, -1.5]
    runs = []
    for graph in (True, False):
        r = rv.River(s, tiny["cuda"], 2, 16 + len(taus))
        r.use_graph(graph)
        r.build_exit_layers("int4")
        _, nx = r.prefill(toks, 0.5)
        tok = torch.empty(2, dtype=torch.int32, device="cuda")
        lg = torch.empty((2, s.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty(2, dtype=torch.int32, device="cuda")
        tok.copy_(nx)
        out = []
        for tau in taus:
            r.decode_step(tok, tau, logits=lg, next_tok=nxt)
            out.append((r.exit_stats()["last_E"], lg.cpu().clone()))
            tok.copy_(nxt)
        r.close()
        runs.append(out)
    for (eg, lg_g), (ee, lg_e), tau in zip(runs[0], runs[1], taus):
        assert eg == ee, (tau, eg, ee)
        assert torch.equal(lg_g, lg_e), tau
        if tau > 1:
            assert eg == L
        if tau < -1:
            assert eg == 1
