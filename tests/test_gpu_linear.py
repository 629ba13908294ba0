"""Per-linear GPU parity: each weight-streaming core (the GEMV used at decode
batch sizes, the MFMA GEMM used for prefill rows) against the oracle's float64
product with the same weights, at the real layer shapes.

The debug entry point river_debug_linear runs one linear of one layer with a
plain fp32 output, so a wrong index, a dropped group term or a mis-ordered
nibble shows up here on its own instead of as a drift of the final logits.

Tolerance, from the arithmetic: both sides see the same bf16 inputs and the
same weights (bf16, or the int4 codes with their bf16 scale/zero), so the only
difference is the fp32 accumulation order of the kernel.  Its error is at most
K * 2^-24 * sum|x w| (the standard bound for a length-K sum); the rms error
over a row is far smaller and is checked against 1e-5 of the rms output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import river_oracle as ro

pytestmark = pytest.mark.gpu

LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def _ref(x64, w64):
    y = ro.linear(x64, w64)
    bound = x64.shape[1] * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T)
    return y, bound


@pytest.fixture(scope="module")
def ctx8b():
    from early_exit_kv_amd import river as rv
    sh = synth.shrink(synth.LLAMA_8B, n_layers=1)
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1)
    r = rv.River(sh, w, 1, 8)
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    yield sh, w, r
    r.close()


@pytest.fixture(scope="module")
def ctx8b_rows():
    """Context made for up to 64 rows per step: 9..64 rows run on the
    batched-row MFMA GEMM of decode steps."""
    from early_exit_kv_amd import river as rv
    sh = synth.shrink(synth.LLAMA_8B, n_layers=1)
    w = synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=1)
    r = rv.River(sh, w, 64, 8)
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    yield sh, w, r
    r.close()


@pytest.mark.parametrize("M", [1, 8, 40, 300])
@pytest.mark.parametrize("use_exit", [0, 1])
def test_linear_cores_8b(ctx8b, M, use_exit):
    check_linears(ctx8b, M, use_exit)


@pytest.mark.parametrize("M", [1, 2, 3, 8])
@pytest.mark.parametrize("use_exit", [0, 1])
def test_linear_mfma_gemv_8b(ctx8b, M, use_exit):
    """The matrix-core GEMV of decode steps (where it fits) on the same shapes."""
    _, _, r = ctx8b
    r.gemv_mode("mfma")
    try:
        check_linears(ctx8b, M, use_exit)
    finally:
        r.gemv_mode("auto")


@pytest.mark.parametrize("M", [1, 2, 3, 8])
@pytest.mark.parametrize("use_exit", [0, 1])
def test_linear_dot_gemv_8b(ctx8b, M, use_exit):
    """The dot-product GEMV on the same shapes."""
    _, _, r = ctx8b
    r.gemv_mode("dot")
    try:
        check_linears(ctx8b, M, use_exit)
    finally:
        r.gemv_mode("auto")


@pytest.mark.parametrize("M", [9, 32, 33, 64])
@pytest.mark.parametrize("use_exit", [0, 1])
def test_linear_batched_rows_8b(ctx8b_rows, M, use_exit):
    check_linears(ctx8b_rows, M, use_exit)


@pytest.mark.parametrize("use_exit", [0, 1])
def test_linear_wide_prefill_8b(ctx8b, use_exit):
    """4,100 rows: the prefill GEMM with 256-column blocks (from 4,096 rows),
    32 full row blocks and a ragged one of 4 rows; the oracle product is taken
    on 96 sampled rows, every row of the ragged block among them."""
    M = 4100
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([np.arange(M - 4, M), np.arange(0, 8), [127, 128, 2047, 4095],
                                     rng.choice(M, 80, replace=False)]))
    check_linears(ctx8b, M, use_exit, rows=rows)


def check_linears(ctx, M, use_exit, rows=None):
    sh, w, r = ctx
    g = torch.Generator(device="cpu").manual_seed(1234 + M)
    worst = []
    for i, name in enumerate(LINEARS):
        N, K = r.linear_shape(i)
        x = torch.randn((M, K), generator=g).to(torch.bfloat16)
        wb = w["layers"][0][name].float().cpu().numpy()
        if use_exit:
            q, s, z = ro.quantize_int4(wb, sh.group_size)
            wh = ro.dequantize_int4(q, s, z, sh.group_size).astype(np.float64)
        else:
            wh = wb.astype(np.float64)
        x64 = x.float().numpy().astype(np.float64)
        if rows is not None:
            x64 = x64[rows]
        y_ref, bound = _ref(x64, wh)
        print(f"[linear] 8b {name} M={M} exit={use_exit}", flush=True)
        y = r.debug_linear(0, i, use_exit, x.cuda())
        torch.cuda.synchronize()
        y = y.cpu().numpy().astype(np.float64)
        if rows is not None:
            y = y[rows]
        d = np.abs(y - y_ref)
        rel = np.sqrt(np.mean(d ** 2)) / np.sqrt(np.mean(y_ref ** 2))
        worst.append((name, float(rel), float(np.max(d / (bound + 1e-30)))))
        assert np.all(d <= bound), (name, M, use_exit, float(np.max(d - bound)))
        assert rel < 1e-5, (name, M, use_exit, rel)
    print(worst, flush=True)
