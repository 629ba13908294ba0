"""Prefill attention on long prompts: the matrix-core (flash-style) kernel and
the vector-ALU one against the exact causal softmax.

A prefill is run with the activation record on; for sampled query rows
(every row of the first and the last query block, the rows around block
boundaries, and a random sample) and every query head, the stored bf16
attention output must be a round-to-nearest-even of a value within the fp32
allowance of the exact float64 softmax(q K^T / sqrt(Dh)) V computed from the
stored q and the K/V the prefill wrote into the cache (the same rule as the
stage-by-stage check of every pass).  The prompts span many 64-row query
blocks and 32-key tiles, with a ragged last block.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import river_oracle as ro
from teacher_forcing import attention_row, bf16_interval_ok

pytestmark = pytest.mark.gpu


def _rv():
    from early_exit_kv_amd import river as rv
    return rv


def check_prefill_attention(shape, w, B, T, attn, n_random=48, seed=5):
    rv = _rv()
    print(f"[prefill-attn] {shape.name} B={B} T={T} attn={attn}", flush=True)
    sh = synth.shrink(shape, n_layers=len(w["layers"]))
    r = rv.River(sh, w, B, T + 1)
    r.attn_kind(attn)
    r.build_exit_layers("int4")
    r.record(B * T)
    toks = synth.make_tokens(sh, B, T, seed=seed)
    r.prefill(toks.cuda(), 0.5, want_logits=False)
    layers, _ = r.read_record(B * T)
    k, v = r.kv_views()
    L = len(w["layers"])
    rng = np.random.default_rng(seed)
    rows_t = np.unique(np.concatenate([np.arange(0, min(T, 66)), np.arange(max(0, T - 66), T),
                                       [t for t in (127, 128, 129, 1023, 1024, 2047, 2048) if t < T],
                                       rng.choice(T, min(T, n_random), replace=False)]))
    scale = 1.0 / np.sqrt(sh.head_dim)
    Hq, Hkv, Dh = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    worst = 0
    for l in range(L):
        kc = k[l, :B, :, :T].double().cpu().numpy()
        vc = v[l, :B, :, :T].double().cpu().numpy()
        q = layers[l]["q"].reshape(B, T, Hq, Dh)
        att = layers[l]["attn"].reshape(B, T, Hq, Dh)
        for b in range(B):
            for t in rows_t:
                for h in range(Hq):
                    j = (h * Hkv) // Hq
                    e, bnd = attention_row(q[b, t, h], kc[b, j, :t + 1], vc[b, j, :t + 1], scale)
                    ok = bf16_interval_ok(att[b, t, h], e, bnd)
                    assert ok.all(), (l, b, int(t), h, float(np.max(np.abs(att[b, t, h] - e))))
                    worst = max(worst, float(np.max(np.abs(att[b, t, h] - e) / (np.abs(e) + 1e-3))))
    r.close()
    print(f"[prefill-attn] rows checked {len(rows_t)} x {B} x {Hq} heads x {L} layers; worst rel {worst:.2e}",
          flush=True)


@pytest.mark.parametrize("attn", ["mfma", "valu"])
def test_prefill_attention_8b_shape_3000(attn):
    """Head dim 128, four query heads per kv head: 47 query blocks (the last
    of 56 rows), 94 key tiles."""
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1)
    check_prefill_attention(synth.LLAMA_8B, w, B=1, T=3000, attn=attn)


def test_prefill_attention_8b_shape_two_rows():
    """Two prompts of 1,100 positions: the batch index of the cache and q."""
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1)
    check_prefill_attention(synth.LLAMA_8B, w, B=2, T=1100, attn="mfma", n_random=24)


def test_prefill_attention_tiny_1500():
    """Head dim 64, two query heads per kv head, four prompts of 1,500 (192
    workgroups with both heads, so one query head per workgroup)."""
    w = synth.make_weights(synth.TINY, seed=0, device="cuda", n_layers=2)
    check_prefill_attention(synth.TINY, w, B=4, T=1500, attn="mfma", n_random=32)


@pytest.mark.parametrize("T", [512, 1100])
def test_prefill_attention_8b_shape_split_heads(T):
    """One short prompt: with all four query heads of a kv head per workgroup
    the grid would hold 64 (T=512) or 144 (T=1,100) workgroups, fewer than
    CUs, so each workgroup takes one (T=512) or two (T=1,100) of them."""
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1)
    check_prefill_attention(synth.LLAMA_8B, w, B=1, T=T, attn="mfma", n_random=32)
