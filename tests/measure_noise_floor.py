"""How far two correct implementations of the decoder drift apart.

Runs the oracle twice on the same seeded inputs, once with every linear in
float64 and once with every linear in float32 (numpy sgemm), everything else
unchanged, and reports the logits difference of a prefill and of the first
decode step as rms and max relative to the logit spread.  Both runs follow the
method exactly; the difference is what the bf16 storage points make of a
different summation order, i.e. the floor under any free-running comparison.

    python tests/measure_noise_floor.py 8b 3 12 int4 0

(shape, layers, prompt length, exit mode, forced exit layer E.)  Test
infrastructure: tests/test_noise_floor.py asserts what these figures show.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import river_oracle as ro  # noqa: E402


def _f32_linear(x, w):
    return (np.asarray(x, np.float32) @ np.asarray(w, np.float32).T).astype(np.float64)


def floor(which, L, T, mode, fe, verbose=False):
    """{'prefill': (rms/std, max/std), 'decode': (...)} of the float64- vs
    float32-product oracles on the first L layers of a shape."""
    shape = {"8b": synth.LLAMA_8B, "1b": synth.LLAMA_1B, "tiny": synth.TINY}[which]
    w = synth.make_weights(shape, seed=0, device="cpu", n_layers=L)
    sh = synth.shrink(shape, n_layers=L)
    cv = lambda t: None if t is None else t.float().numpy()
    hw = {"embed": cv(w["embed"]), "final_norm": cv(w["final_norm"]), "lm_head": cv(w["lm_head"]),
          "layers": [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]]}
    del w
    toks = synth.make_tokens(sh, 1, T, seed=0).numpy()
    out = {}
    f64 = ro.linear
    for name, fn in (("f64", f64), ("f32", _f32_linear)):
        ro.linear = fn
        try:
            orc = ro.RiverOracle(sh.as_dict(), hw, 1, T + 4)
            orc.build_exit_layers(mode)
            t0 = time.time()
            o = orc.prefill(toks, 0.5, force_E=fe)
            o2 = orc.decode_step(o["next"], 0.5, force_E=fe)
        finally:
            ro.linear = f64
        out[name] = (o["logits"][0], o2["logits"][0])
        if verbose:
            print(f"{name}: {time.time() - t0:.1f} s", flush=True)
    res = {}
    for i, nm in enumerate(("prefill", "decode")):
        a, b = out["f64"][i], out["f32"][i]
        d = np.abs(a - b)
        res[nm] = (float(np.sqrt(np.mean(d ** 2)) / a.std()), float(d.max() / a.std()))
    return res


def main():
    which, L, T, mode, fe = sys.argv[1], int(sys.argv[2]), int(sys.argv[3]), sys.argv[4], int(sys.argv[5])
    for nm, (rms, mx) in floor(which, L, T, mode, fe, verbose=True).items():
        print(f"{which} L={L} T={T} {mode} E={fe} {nm}: rms/std {rms:.2e} max/std {mx:.4f}")


if __name__ == "__main__":
    main()
