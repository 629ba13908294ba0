"""Backbone offloading (lead page, section 5: deep backbone layers leave device
memory, the exit layers stay resident).

The seven linears of the offloaded layers live in pinned host memory; the
kernels read them over the host link only when the device-side decision runs
the layer on its backbone (tau > 1 never exits, so every layer is read), and
the first kernel after a pending exit test streams the exit copy first when
the backbone is off device.  Checked stage by stage against the oracle
(tests/teacher_forcing.py) with the same rules as every other pass, and bit
for bit against the same decoder with every weight in device memory: the
kernels and the order of every sum are the same, only where the bytes come
from differs.
"""
import numpy as np
import pytest
import torch

import synth
from test_gpu_parity_full import parity_run

pytestmark = pytest.mark.gpu


def _rv():
    from early_exit_kv_amd import river as rv
    return rv


@pytest.fixture(scope="module")
def tiny_w():
    return synth.make_weights(synth.TINY, seed=0, device="cuda")


@pytest.mark.parametrize("tau", [2.0, 0.5, -1.5])
def test_offloaded_tiny_parity(tiny_w, tau):
    """Layers 1..3 of the tiny decoder offloaded: tau 2 reads every offloaded
    backbone every step, -1.5 exits after layer 0 (layer 1's first kernel
    guesses the exit copy and keeps it), 0.5 mixes."""
    rv = _rv()
    w = rv.offload_layers(tiny_w, 1)
    assert not w["layers"][1]["wq"].is_cuda and w["layers"][1]["wq"].is_pinned()
    Es = parity_run(synth.TINY, w, B=2, T=32, steps=3, tau=tau)
    if tau > 1:
        assert all(e == synth.TINY.n_layers for e in Es)
    if tau < -1:
        assert all(e == 1 for e in Es)


def test_offloaded_8b_layer_shapes_backbone_read(  ):
    """8B layer shapes, layer 1 of 2 offloaded, tau 2: the 436 MB backbone of
    layer 1 is read from host memory at every pass."""
    rv = _rv()
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=2)
    wo = rv.offload_layers(w, 1)
    del w
    Es = parity_run(synth.LLAMA_8B, wo, B=1, T=12, steps=2, tau=2.0)
    assert all(e == 2 for e in Es)


@pytest.mark.parametrize("tau", [2.0, 0.5, -1.5])
def test_offloaded_equals_resident_bitwise(tiny_w, tau):
    """Recorded decode steps (HIP graphs) with layers 2..3 offloaded give the
    same logits, tokens, decisions and K/V bit for bit as the resident
    decoder."""
    rv = _rv()
    s = synth.TINY
    toks = synth.make_tokens(s, 2, 16, seed=0).cuda()
    outs = []
    for w in (tiny_w, rv.offload_layers(tiny_w, 2)):
        r = rv.River(s, w, 2, 24)
        r.build_exit_layers("int4")
        lg0, nx = r.prefill(toks, tau)
        tok = torch.empty(2, dtype=torch.int32, device="cuda")
        lg = torch.empty((2, s.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty(2, dtype=torch.int32, device="cuda")
        tok.copy_(nx)
        res = [(lg0.cpu(), nx.cpu(), r.exit_stats()["last_E"])]
        for _ in range(4):
            r.decode_step(tok, tau, logits=lg, next_tok=nxt)
            res.append((lg.cpu().clone(), nxt.cpu().clone(), r.exit_stats()["last_E"]))
            tok.copy_(nxt)
        k, v = r.kv_views()
        res.append((k[:, :2, :, :21].cpu().clone(), v[:, :2, :, :21].cpu().clone(), 0))
        r.close()
        outs.append(res)
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and a[2] == b[2]
