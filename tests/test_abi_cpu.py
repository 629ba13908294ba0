"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every declared entry point, sizes and layouts follow their closed
forms, and invalid calls return their status codes before touching the GPU."""
import ctypes
import os
import re

import pytest

import synth
from early_exit_kv_amd import river as rv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rv.LIB_PATH):
        pytest.fail("libriver.so is not built (run early_exit_kv_amd/build.py)")
    return rv.load_library()


def declared_functions():
    with open(os.path.join(ROOT, "include", "river.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(river_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names, "no declarations found"
    assert set(names) == set(rv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_covers_codes(lib):
    for code in range(7):
        assert lib.river_strerror(code).decode() not in ("", "unknown status")
    assert lib.river_strerror(99).decode() == "unknown status"


@pytest.mark.parametrize("name", ["tiny", "1b", "8b"])
def test_query_sizes_closed_forms(lib, name):
    wl = synth.WORKLOADS[name]
    s = wl.shape
    cfg = rv.make_config(s, wl.batch, wl.max_seq)
    sz = rv.query_sizes(cfg)
    # one shared cache: L * 2 (K and V) * Hkv * Dh * 2 bytes per token and row
    per_token = s.n_layers * 2 * s.n_kv_heads * s.head_dim * 2
    assert sz.kv_cache_bytes == per_token * wl.batch * wl.max_seq
    if name == "8b":
        assert per_token == 131072
    # int4 bank: half a byte per weight plus 4 bytes (bf16 scale + zero) per group
    lin = [(s.n_q_heads * s.head_dim, s.d_model), (s.n_kv_heads * s.head_dim, s.d_model),
           (s.n_kv_heads * s.head_dim, s.d_model), (s.d_model, s.n_q_heads * s.head_dim),
           (s.ffn_dim, s.d_model), (s.ffn_dim, s.d_model), (s.d_model, s.ffn_dim)]
    exact = s.n_layers * sum(n * k // 2 + n * (k // s.group_size) * 4 for n, k in lin)
    assert exact <= sz.exit_bank_bytes <= exact + s.n_layers * 14 * 256
    copy = s.n_layers * sum(n * k * 2 for n, k in lin)
    assert copy <= sz.exit_bank_copy_bytes <= copy + s.n_layers * 7 * 256
    if name == "8b":
        # per layer: 436,207,616 bf16 bytes against 115,867,648 packed bytes
        assert copy // s.n_layers == 436207616
        assert exact // s.n_layers == 115867648


def test_exit_bank_offsets_tile_the_bank(lib):
    s = synth.TINY
    cfg = rv.make_config(s, 2, 48)
    sz = rv.query_sizes(cfg)
    spans = []
    for layer in range(s.n_layers):
        for lin in range(7):
            co, so = rv.exit_bank_offsets(cfg, layer, lin)
            n, k = [(256, 256), (128, 256), (128, 256), (256, 256), (1024, 256), (1024, 256),
                    (256, 1024)][lin]
            assert co % 256 == 0 and so % 256 == 0
            spans.append((co, co + n * k // 2))
            spans.append((so, so + n * (k // s.group_size) * 4))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= sz.exit_bank_bytes


def test_invalid_configs(lib):
    s = synth.TINY
    out = rv.RiverSizes()
    bad = rv.make_config(s, 2, 48)
    bad.n_layers = 0
    assert lib.river_query_sizes(ctypes.byref(bad), ctypes.byref(out)) == rv.RIVER_E_INVALID_ARG
    bad = rv.make_config(s, 2, 48)
    bad.n_kv_heads = 3
    assert lib.river_query_sizes(ctypes.byref(bad), ctypes.byref(out)) == rv.RIVER_E_INVALID_ARG
    bad = rv.make_config(s, 2, 48)
    bad.group_size = 48   # not a power of two
    assert lib.river_query_sizes(ctypes.byref(bad), ctypes.byref(out)) == rv.RIVER_E_UNIMPLEMENTED
    bad = rv.make_config(s, 2, 48)
    bad.rope_theta = float("nan")
    assert lib.river_query_sizes(ctypes.byref(bad), ctypes.byref(out)) == rv.RIVER_E_INVALID_ARG
    assert lib.river_query_sizes(None, ctypes.byref(out)) == rv.RIVER_E_INVALID_ARG


def _fake_ctx(lib, cfg, shrink=None):
    """A context over fake (never dereferenced) device pointers: river_init
    touches no device memory, so its validation runs on a machine without GPU."""
    sz = rv.query_sizes(cfg)
    layers = (rv.RiverLayerW * cfg.n_layers)()
    for i in range(cfg.n_layers):
        for name, _ in rv.RiverLayerW._fields_:
            setattr(layers[i], name, 0x1000)
    w = rv.RiverWeights(0x1000, 0x1000, 0x1000, layers)
    given = rv.RiverSizes(sz.exit_bank_bytes, sz.exit_bank_copy_bytes, sz.kv_cache_bytes,
                          sz.workspace_bytes, sz.control_bytes)
    if shrink:
        setattr(given, shrink, getattr(given, shrink) - 1)
    ctx = ctypes.c_void_p()
    P = ctypes.c_void_p(0x1000)
    st = lib.river_init(ctypes.byref(cfg), ctypes.byref(w), P, P, P, P, ctypes.byref(given), None,
                        ctypes.byref(ctx))
    return st, ctx


def test_init_checks_sizes_and_pointers(lib):
    cfg = rv.make_config(synth.TINY, 2, 48)
    for field in ("exit_bank_bytes", "kv_cache_bytes", "workspace_bytes", "control_bytes"):
        st, _ = _fake_ctx(lib, cfg, shrink=field)
        assert st == rv.RIVER_E_BAD_SIZE, field
    ctx = ctypes.c_void_p()
    sz = rv.query_sizes(cfg)
    assert lib.river_init(ctypes.byref(cfg), None, None, None, None, None, ctypes.byref(sz), None,
                          ctypes.byref(ctx)) == rv.RIVER_E_INVALID_ARG
    # untied model without an LM head
    layers = (rv.RiverLayerW * cfg.n_layers)()
    for i in range(cfg.n_layers):
        for name, _ in rv.RiverLayerW._fields_:
            setattr(layers[i], name, 0x1000)
    w = rv.RiverWeights(0x1000, 0x1000, None, layers)
    P = ctypes.c_void_p(0x1000)
    assert lib.river_init(ctypes.byref(cfg), ctypes.byref(w), P, P, P, P, ctypes.byref(sz), None,
                          ctypes.byref(ctx)) == rv.RIVER_E_INVALID_ARG


def test_call_order_and_argument_errors_enqueue_nothing(lib):
    cfg = rv.make_config(synth.TINY, 2, 48)
    st, ctx = _fake_ctx(lib, cfg)
    assert st == rv.RIVER_OK and ctx
    tok = ctypes.c_void_p(0x2000)
    try:
        # prefill / decode before the exit layers exist
        assert lib.river_prefill(ctx, tok, 2, 8, ctypes.c_float(0.5), None, None) == rv.RIVER_E_STATE
        assert lib.river_decode_step(ctx, tok, ctypes.c_float(0.5), None, None) == rv.RIVER_E_STATE
        # non-finite tau and null tokens are rejected first
        for t in (float("nan"), float("inf")):
            assert lib.river_prefill(ctx, tok, 2, 8, ctypes.c_float(t), None, None) == rv.RIVER_E_INVALID_ARG
            assert lib.river_decode_step(ctx, tok, ctypes.c_float(t), None, None) == rv.RIVER_E_INVALID_ARG
        assert lib.river_prefill(ctx, None, 2, 8, ctypes.c_float(0.5), None, None) == rv.RIVER_E_INVALID_ARG
        # several steps per call: 1..64 steps, and a next-token buffer to chain them through
        nx = ctypes.c_void_p(0x3000)
        for n in (0, -1, 65):
            assert lib.river_decode_steps(ctx, n, tok, ctypes.c_float(0.5), None, nx) == rv.RIVER_E_INVALID_ARG
        assert lib.river_decode_steps(ctx, 2, tok, ctypes.c_float(0.5), None, None) == rv.RIVER_E_INVALID_ARG
        assert lib.river_decode_steps(ctx, 2, tok, ctypes.c_float(float("nan")), None, nx) == rv.RIVER_E_INVALID_ARG
        assert lib.river_decode_steps(ctx, 4, tok, ctypes.c_float(0.5), None, nx) == rv.RIVER_E_STATE
        assert lib.river_build_exit_layers(ctx, 7) == rv.RIVER_E_INVALID_ARG
        assert lib.river_exit_stats(ctx, None) == rv.RIVER_E_INVALID_ARG
        st_out = rv.RiverExitStats()
        assert lib.river_exit_stats(ctx, ctypes.byref(st_out)) == rv.RIVER_E_STATE
        # options
        assert lib.river_set_option(ctx, rv.RIVER_OPT_GRAPH, 2) == rv.RIVER_E_INVALID_ARG
        assert lib.river_set_option(ctx, rv.RIVER_OPT_FORCE_E, cfg.n_layers + 1) == rv.RIVER_E_RANGE
        assert lib.river_set_option(ctx, rv.RIVER_OPT_FORCE_E, -1) == rv.RIVER_OK
        assert lib.river_set_option(ctx, 99, 0) == rv.RIVER_E_INVALID_ARG
        assert lib.river_reset(ctx) == rv.RIVER_OK
        # the copy bank is larger than what was handed over
        assert lib.river_build_exit_layers(ctx, rv.RIVER_EXIT_COPY) == rv.RIVER_E_BAD_SIZE
    finally:
        lib.river_destroy(ctx)
    lib.river_destroy(None)  # a no-op


def test_product_path_has_no_cpu_fallback(monkeypatch):
    import torch
    monkeypatch.setattr(torch.cuda, "is_available", lambda: False)
    with pytest.raises(RuntimeError):
        rv.River(synth.TINY, {"layers": []}, 2, 48)


def test_unpack_int4_layout():
    import numpy as np
    # byte i of word w: column 8w+i in the low nibble, column 8w+i+4 in the high one
    codes = (np.arange(16, dtype=np.uint8).reshape(1, 16) * 7) % 16
    words = np.zeros((1, 2), dtype=np.int64)
    for c in range(16):
        w, j = divmod(c, 8)
        words[0, w] |= int(codes[0, c]) << (8 * (j % 4) + 4 * (j // 4))
    sz = np.array([[(0x3F80 | (0x40A0 << 16))]], dtype=np.int64)  # s = 1.0, z = 5.0
    got, s, z = rv.unpack_int4(words, sz, 16)
    assert np.array_equal(got, codes) and s[0, 0] == 1.0 and z[0, 0] == 5.0
