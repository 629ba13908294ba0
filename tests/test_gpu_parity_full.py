"""GPU parity at the real layer shapes of the Llama-3.2-1B and Llama-3.1-8B
workloads, plus the code paths the tiny decoder never reaches (split-K decode
attention over a long context, batch 8).

The decoders here keep every per-layer shape and the full vocabulary, so each
kernel runs in the launch configuration the benchmark times; only the number
of layers and the prompt length are cut so that the float64 oracle finishes in
seconds.

Rules: every pass is checked stage by stage with the oracle fed the stored
activations (tests/teacher_forcing.py: q, K/V, attention, residuals, SwiGLU
product, exit cosines and decisions, logits -- the logits bar max|dlogit| <=
2e-2 * std included); a free-running oracle fed only the same tokens runs
beside it for the exit decisions (identical unless |min cos - tau| < 1e-3)
and the K/V cosine bar (>= 0.999).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import river_oracle as ro
from teacher_forcing import Report, check_pass
from test_gpu_parity import KV_COS, check_decision

pytestmark = pytest.mark.gpu


def _river():
    from early_exit_kv_amd import river as rv
    return rv


def host_weights(w, dtype=np.float64):
    """Device bf16 weights -> host arrays (exact bf16 values) for the oracle."""
    def cv(t):
        return None if t is None else t.float().cpu().numpy().astype(dtype)
    return {"embed": cv(w["embed"]), "final_norm": cv(w["final_norm"]), "lm_head": cv(w["lm_head"]),
            "layers": [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]]}


def parity_run(shape, w_dev, B, T, steps, tau, mode="int4", gemv="auto", attn="mfma", chunk=0,
               check_prefill=True, free_running=True):
    """Prefill + decode steps on the GPU with every pass checked stage by stage
    (teacher forcing at each stored activation), and a free-running oracle
    beside it for the exit decisions and the K/V cosine bar.

    chunk: positions per decode-attention workgroup (0: the library's choice).
    check_prefill=False: the prefill pass is not checked stage by stage (the
    decode steps still are, against the cache the GPU's prefill left: the
    attention of each step over every stored position included).
    free_running=False: no free-running oracle (for prompts too long for the
    float64 oracle to prefill in seconds).
    """
    rv = _river()
    max_seq = T + steps
    L = len(w_dev["layers"])
    print(f"[parity-full] {shape.name} L={L} B={B} T={T} steps={steps} tau={tau} attn={attn} "
          f"chunk={chunk} gemv={gemv}", flush=True)
    sh = synth.shrink(shape, n_layers=L)
    r = rv.River(sh, w_dev, B, max_seq)
    r.gemv_mode(gemv)
    r.attn_kind(attn)
    if chunk:
        r.set_option(rv.RIVER_OPT_ATTN_CHUNK, chunk)
    r.build_exit_layers(mode)
    r.record(B * T if check_prefill else 0)
    hw = host_weights(w_dev)
    orc = ro.RiverOracle(sh.as_dict(), hw, B, max_seq)
    orc.build_exit_layers(mode)
    lw = lambda l, ex: orc.exit_layers[l] if ex else hw["layers"][l]
    w_lm = hw["embed"] if hw["lm_head"] is None else hw["lm_head"]
    rep = Report()

    def check(gl, gn, st, n, start):
        layers, h_out = r.read_record(B * n)
        k, v = r.kv_views()
        kc = k[:L, :B, :, :start + n].double().cpu().numpy()
        vc = v[:L, :B, :, :start + n].double().cpu().numpy()
        check_pass(orc.s, lw, st["last_E"], layers, h_out, kc, vc, B, n, start, st["last_trace"], tau,
                   gl.double().cpu().numpy(), gn.cpu().numpy(), hw["final_norm"], w_lm, rep)
        return kc, vc

    toks = synth.make_tokens(sh, B, T, seed=0)
    gl, gn = r.prefill(toks.cuda(), tau)
    st = r.exit_stats()
    if check_prefill:
        kc, vc = check(gl, gn, st, T, 0)
    else:
        r.record(B)
    if free_running:
        if not check_prefill:
            k, v = r.kv_views()
            kc = k[:L, :B, :, :T].double().cpu().numpy()
            vc = v[:L, :B, :, :T].double().cpu().numpy()
        o = orc.prefill(toks.numpy(), tau)
        if check_decision(st["last_E"], st["last_trace"], o, tau, L):
            o = orc.prefill(toks.numpy(), tau, force_E=st["last_E"])
        kv_cos(kc, vc, orc, L, B, 0, T)
    Es = [st["last_E"]]
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = gn.cpu().numpy().astype(np.int64)
    for step in range(steps):
        tok.copy_(torch.from_numpy(nxt.astype(np.int32)))
        gl, gn = r.decode_step(tok, tau)
        st = r.exit_stats()
        kc, vc = check(gl, gn, st, 1, T + step)
        if free_running:
            o = orc.decode_step(nxt, tau)
            if check_decision(st["last_E"], st["last_trace"], o, tau, L):
                orc.pos -= 1
                o = orc.decode_step(nxt, tau, force_E=st["last_E"])
            kv_cos(kc, vc, orc, L, B, T + step, T + step + 1)
        Es.append(st["last_E"])
        nxt = gn.cpu().numpy().astype(np.int64)
    print(f"[parity-full] worst: {rep.worst}", flush=True)
    r.close()
    return Es


def kv_cos(kc, vc, orc, L, B, p0, p1):
    """Free-running K/V (the oracle fed only the same tokens): cosine per
    (layer, row, position) at least KV_COS."""
    for l in range(L):
        for b in range(B):
            for p in range(p0, p1):
                for name, g, o in (("K", kc, orc.k_cache), ("V", vc, orc.v_cache)):
                    a = g[l, b, :, p].reshape(-1)
                    c = o[l, b, :, p].reshape(-1)
                    cos = a @ c / max(np.linalg.norm(a) * np.linalg.norm(c), 1e-30)
                    assert cos >= KV_COS, f"{name} l={l} b={b} p={p} cos={cos}"


@pytest.fixture(scope="module")
def w8b():
    return synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=3)


@pytest.fixture(scope="module")
def w1b():
    return synth.make_weights(synth.LLAMA_1B, seed=0, device="cuda", n_layers=3)


@pytest.mark.parametrize("which", ["1b", "8b"])
def test_quantizer_bit_exact_full_layer(which, w8b, w1b):
    rv = _river()
    shape = synth.LLAMA_8B if which == "8b" else synth.LLAMA_1B
    w = w8b if which == "8b" else w1b
    sh = synth.shrink(shape, n_layers=1)
    wl = dict(w)
    wl["layers"] = w["layers"][:1]
    print(f"[parity-full] quantizer {which}", flush=True)
    r = rv.River(sh, wl, 1, 8)
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    for i, name in enumerate(rv.LINEAR_NAMES):
        words, sz = r.exit_linear_packed(0, i)
        q, sc, z = rv.unpack_int4(words.cpu().numpy(), sz.cpu().numpy(), sh.group_size)
        oq, osc, oz = ro.quantize_int4(wl["layers"][0][name].float().cpu().numpy(), sh.group_size)
        assert np.array_equal(q, oq), name
        assert np.array_equal(sc.view(np.uint32), osc.view(np.uint32)), name
        assert np.array_equal(z.view(np.uint32), oz.view(np.uint32)), name
    r.close()


@pytest.mark.parametrize("tau", [0.5, -1.5])
def test_decode_parity_8b_layer_shapes(w8b, tau):
    Es = parity_run(synth.LLAMA_8B, w8b, B=1, T=12, steps=3, tau=tau)
    if tau < -1:
        assert all(e == 1 for e in Es)


def test_decode_parity_8b_mfma_gemv(w8b):
    """Every decode linear on the matrix-core GEMV."""
    parity_run(synth.LLAMA_8B, w8b, B=1, T=12, steps=3, tau=0.5, gemv="mfma")


def test_decode_parity_1b_layer_shapes_tied(w1b):
    parity_run(synth.LLAMA_1B, w1b, B=1, T=12, steps=3, tau=0.5)


def test_decode_parity_8b_layer_shapes_batch8(w8b):
    """8 rows per step: RMSNorm and the exit test as row kernels, q|k|v and
    gate|up on the batched-row GEMM, o and down on the matrix-core GEMV."""
    w = dict(w8b)
    w["layers"] = w8b["layers"][:2]
    parity_run(synth.LLAMA_8B, w, B=8, T=6, steps=2, tau=0.3)


@pytest.mark.parametrize("tau", [0.5, -1.5])
def test_decode_parity_row_path_ragged(tau):
    """5 and 7 rows per step, the fewest and a ragged count on the row-kernel
    path (the batched-row GEMM's 16-row tile mostly padding), on the tiny
    decoder (group size 64) with the exit taken and never taken."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    for B in (5, 7):
        Es = parity_run(synth.TINY, w, B=B, T=6, steps=3, tau=tau)
        if tau < -1:
            assert all(e == 1 for e in Es)


def test_decode_parity_8b_layer_shapes_batch32(w8b):
    """32 rows per step: every linear on the batched-row MFMA GEMM (split K,
    last-workgroup reduction), RMSNorm and the exit test as row kernels."""
    w = dict(w8b)
    w["layers"] = w8b["layers"][:2]
    parity_run(synth.LLAMA_8B, w, B=32, T=4, steps=2, tau=0.3)


@pytest.mark.parametrize("tau", [0.5, -1.5])
def test_decode_parity_tiny_batch16(tau):
    """16 rows per step on the tiny decoder (group size 64)."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    Es = parity_run(synth.TINY, w, B=16, T=8, steps=3, tau=tau)
    if tau < -1:
        assert all(e == 1 for e in Es)


def test_decode_parity_tiny_batch64_max_rows():
    """64 rows per step, the most the batched-row GEMM takes (four 16-row
    blocks per workgroup), and 37 rows: a ragged last block."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    parity_run(synth.TINY, w, B=64, T=6, steps=2, tau=0.5)
    parity_run(synth.TINY, w, B=37, T=5, steps=2, tau=0.5)


def test_prefill_parity_8b_split_k_o_down(w8b):
    """A 500-token prompt on two 8B-shape layers: the prefill GEMM's o and
    down run 256 workgroups of 64-row tiles (the last block ragged, 52
    rows), so K is split in two halves and pgemm_reduce_kernel adds the
    partial tiles and runs the residual epilogue; every stage of the prefill
    and one decode step is checked against the oracle."""
    w = dict(w8b)
    w["layers"] = w8b["layers"][:2]
    parity_run(synth.LLAMA_8B, w, B=1, T=500, steps=1, tau=0.5)


def test_decode_parity_lm_head_split_reduce():
    """The batched LM head with K split: a 2,048-wide decoder with a
    1,100-token vocabulary (nine 128-column blocks, the last partial) at 24
    rows (two splits) and 40 rows (four splits); the reduce kernel takes eight
    column blocks per workgroup, so one full group of blocks and one ragged
    group of a single partial block."""
    sh = synth.shrink(synth.LLAMA_1B, name="1b-layers-small-vocab", n_layers=2, vocab=1100)
    w = synth.make_weights(sh, seed=3, device="cuda")
    parity_run(sh, w, B=24, T=4, steps=2, tau=0.5)
    parity_run(sh, w, B=40, T=4, steps=2, tau=0.5)


def test_split_attention_long_context_tiny():
    """A context of several hundred positions splits the decode attention over
    workgroups and merges the splits in the last one; B=8 fills the GEMV's
    widest batch tile."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    parity_run(synth.TINY, w, B=8, T=700, steps=3, tau=0.5)


def test_prefill_ragged_rows_tiny():
    """B*T rows that end inside a GEMM tile, one row per batch element."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    parity_run(synth.TINY, w, B=3, T=45, steps=2, tau=0.5)


def test_prefill_ragged_rows_tiny_mfma_gemv():
    """Three rows per decode step (padded to four) on the matrix-core GEMV."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    parity_run(synth.TINY, w, B=3, T=45, steps=2, tau=0.5, gemv="mfma")


def test_decode_parity_8b_batch8_mfma_gemv(w8b):
    """Eight rows: q|k|v, o and gate|up on the matrix-core GEMV, the down
    projection (its rows too wide for LDS) on the dot-product GEMV."""
    w = dict(w8b)
    w["layers"] = w8b["layers"][:2]
    parity_run(synth.LLAMA_8B, w, B=8, T=6, steps=2, tau=0.3, gemv="mfma")


def test_decode_parity_8b_dot_gemv(w8b):
    """Every decode linear on the dot-product GEMV."""
    parity_run(synth.LLAMA_8B, w8b, B=1, T=12, steps=3, tau=0.5, gemv="dot")


def test_split_attention_long_context_tiny_valu():
    """The vector-ALU decode attention on the same long context."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    parity_run(synth.TINY, w, B=8, T=700, steps=3, tau=0.5, attn="valu")


def test_decode_parity_8b_valu_attention(w8b):
    """The vector-ALU decode attention at head dim 128."""
    parity_run(synth.LLAMA_8B, w8b, B=1, T=12, steps=3, tau=0.5, attn="valu")
