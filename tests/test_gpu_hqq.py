"""The HQQ-style exit bank (RIVER_EXIT_HQQ): codes, scales and zeros bit for
bit against the oracle's quantize_int4_hqq at group sizes 32, 64, 128 and
256 (every linear of an 8B-shape layer among them), and decode parity of an
HQQ bank against the oracle built with the same refinement."""
import numpy as np
import pytest
import torch

import synth
from oracle import river_oracle as ro
from test_gpu_parity_full import parity_run

pytestmark = pytest.mark.gpu


def _rv():
    from early_exit_kv_amd import river as rv
    return rv


def bit_exact(shape, w):
    rv = _rv()
    sh = synth.shrink(shape, n_layers=1)
    wl = dict(w)
    wl["layers"] = w["layers"][:1]
    print(f"[hqq] {shape.name} G={shape.group_size}", flush=True)
    r = rv.River(sh, wl, 1, 8)
    r.build_exit_layers("hqq")
    torch.cuda.synchronize()
    for i, name in enumerate(rv.LINEAR_NAMES):
        words, sz = r.exit_linear_packed(0, i)
        q, sc, z = rv.unpack_int4(words.cpu().numpy(), sz.cpu().numpy(), sh.group_size)
        oq, osc, oz = ro.quantize_int4_hqq(wl["layers"][0][name].float().cpu().numpy(), sh.group_size)
        assert np.array_equal(sc.view(np.uint32), osc.view(np.uint32)), name
        assert np.array_equal(z.view(np.uint32), oz.view(np.uint32)), (name, int((z != oz).sum()))
        assert np.array_equal(q, oq), (name, int((q != oq).sum()))
    r.close()


@pytest.mark.parametrize("G", [32, 64, 256])
def test_hqq_bank_bit_exact_tiny(G):
    shape = synth.shrink(synth.TINY, group_size=G)
    bit_exact(shape, synth.make_weights(shape, seed=0, device="cuda", n_layers=1))


def test_hqq_bank_bit_exact_8b_layer():
    bit_exact(synth.LLAMA_8B, synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1))


@pytest.mark.parametrize("tau", [0.5, -1.5])
def test_decode_parity_hqq_tiny(tau):
    w = synth.make_weights(synth.TINY, seed=0, device="cuda")
    parity_run(synth.TINY, w, B=2, T=32, steps=3, tau=tau, mode="hqq")


def test_decode_parity_hqq_8b_layer_shapes():
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=2)
    parity_run(synth.LLAMA_8B, w, B=1, T=12, steps=2, tau=-1.5, mode="hqq")
