import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def np_weights(w):
    """torch bf16 weight dict -> float32 numpy dict (exact bf16 values)."""
    def cv(t):
        return None if t is None else t.float().cpu().numpy()
    return {
        "embed": cv(w["embed"]), "final_norm": cv(w["final_norm"]), "lm_head": cv(w["lm_head"]),
        "layers": [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]],
    }


@pytest.fixture(scope="session")
def tiny_np():
    import synth
    return np_weights(synth.make_weights(synth.TINY, seed=0))
