"""river_debug_linear_noalloc: the entry point for callers that cannot
allocate.  It runs the same kernels as river_debug_linear with the batched-row
GEMM's split-K partial tiles in the library's static scratch array, so its
output must equal river_debug_linear's bit for bit, and both must lie within
the fp32 accumulation bound of the float64 product (the bar of every linear
core).  Two calls in a row, the second with fewer rows, show that nothing left
in the shared scratch by the first call leaks into the second.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import river_oracle as ro

pytestmark = pytest.mark.gpu


def _rv():
    from early_exit_kv_amd import river as rv
    return rv


def _bound_check(x, y, wh):
    x64 = x.float().numpy().astype(np.float64)
    y_ref = ro.linear(x64, wh)
    bound = x64.shape[1] * 2.0 ** -24 * (np.abs(x64) @ np.abs(wh).T)
    d = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    assert np.all(d <= bound), float(np.max(d - bound))


@pytest.fixture(scope="module")
def ctx8b_rows():
    rv = _rv()
    sh = synth.shrink(synth.LLAMA_8B, n_layers=1)
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1)
    r = rv.River(sh, w, 64, 8)
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    yield sh, w, r
    r.close()


@pytest.mark.parametrize("use_exit", [1, 0])
def test_noalloc_linear_matches_debug_linear_8b(ctx8b_rows, use_exit):
    sh, w, r = ctx8b_rows
    g = torch.Generator(device="cpu").manual_seed(99)
    for i, name in enumerate(("w_down", "w_gate", "wq", "wo")):
        li = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down").index(name)
        N, K = r.linear_shape(li)
        wb = w["layers"][0][name].float().cpu().numpy()
        if use_exit:
            q, s, z = ro.quantize_int4(wb, sh.group_size)
            wh = ro.dequantize_int4(q, s, z, sh.group_size).astype(np.float64)
        else:
            wh = wb.astype(np.float64)
        for M in (64, 20):     # the second call has fewer rows than the first
            print(f"[noalloc] 8b {name} M={M} exit={use_exit}", flush=True)
            x = torch.randn((M, K), generator=g).to(torch.bfloat16)
            xd = x.cuda()
            y_na = r.debug_linear(0, li, use_exit, xd, noalloc=True)
            y_ws = r.debug_linear(0, li, use_exit, xd)
            torch.cuda.synchronize()
            assert torch.equal(y_na, y_ws), (name, M)
            _bound_check(x, y_na, wh)


def test_noalloc_linear_rejects_partials_beyond_the_scratch():
    """A linear whose 64-row partial tiles exceed the 32 MiB array is refused
    before any launch (gate with 16,640 rows at K = 4096: 130 column blocks x
    8 splits x 64 x 128 floats = 34.1 MB); the workspace entry point runs it."""
    rv = _rv()
    sh = synth.shrink(synth.LLAMA_8B, n_layers=1, ffn_dim=16640, vocab=1024)
    w = synth.make_weights(sh, seed=0, device="cuda", n_layers=1)
    r = rv.River(sh, w, 64, 8)
    r.build_exit_layers("int4")
    x = torch.randn((64, sh.d_model)).to(torch.bfloat16).cuda()
    print("[noalloc] oversize partials", flush=True)
    with pytest.raises(rv.RiverError) as e:
        r.debug_linear(0, 4, 1, x, noalloc=True)
    assert e.value.code == rv.RIVER_E_BAD_SIZE
    r.debug_linear(0, 4, 1, x)
    torch.cuda.synchronize()
    r.close()
