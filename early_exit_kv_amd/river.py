"""Thin ctypes binding of libriver.so (the C ABI in include/river.h).

Argument marshalling only: every step of the decoder runs in the HIP kernels
of libriver.so.  PyTorch supplies device memory and the HIP stream.  There is
no CPU fallback: without the built library or a GPU this module raises.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libriver.so")

RIVER_OK, RIVER_E_INVALID_ARG, RIVER_E_BAD_SIZE, RIVER_E_STATE = 0, 1, 2, 3
RIVER_E_RANGE, RIVER_E_HIP, RIVER_E_UNIMPLEMENTED = 4, 5, 6
RIVER_EXIT_INT4, RIVER_EXIT_COPY, RIVER_EXIT_HQQ = 1, 2, 3
RIVER_OPT_GRAPH, RIVER_OPT_FORCE_E, RIVER_OPT_PROFILE, RIVER_OPT_ATTN_CHUNK, RIVER_OPT_GEMV = 1, 2, 3, 4, 5
RIVER_OPT_ATTN, RIVER_OPT_KV_STRATEGY = 6, 7
KV_STRATEGIES = ("river", "kv_mask", "propagate", "mono", "recompute")
KERNEL_KINDS = ("begin", "qkv", "attn", "o", "gateup", "down", "lm_head",
                "p_norm", "p_gemm", "p_attn", "p_cos")
RIVER_MAX_LAYERS = 256
LINEAR_NAMES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")

# names of every entry point include/river.h declares
EXPORTS = (
    "river_query_sizes", "river_exit_bank_offsets", "river_init", "river_build_exit_layers",
    "river_prefill", "river_decode_step", "river_decode_steps", "river_exit_stats", "river_set_option",
    "river_reset", "river_destroy", "river_strerror", "river_profile_read",
    "river_debug_linear", "river_record_bytes", "river_set_record", "river_time_kernel",
    "river_debug_linear_noalloc", "river_set_kv_state",
)


class RiverError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__(f"{what}: {_lib_strerror(code)} (status {code})")


class RiverConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("tied_embeddings", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("max_batch", ctypes.c_int32), ("max_seq", ctypes.c_int32),
    ]


class RiverLayerW(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class RiverWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(RiverLayerW))]


class RiverSizes(ctypes.Structure):
    _fields_ = [("exit_bank_bytes", ctypes.c_size_t), ("exit_bank_copy_bytes", ctypes.c_size_t),
                ("kv_cache_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
                ("control_bytes", ctypes.c_size_t)]


class RiverKernelTime(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class RiverExitStats(ctypes.Structure):
    _fields_ = [
        ("prefill_hist", ctypes.c_int64 * (RIVER_MAX_LAYERS + 1)),
        ("decode_hist", ctypes.c_int64 * (RIVER_MAX_LAYERS + 1)),
        ("n_prefill", ctypes.c_int64), ("n_decode_steps", ctypes.c_int64),
        ("mean_exit_layer", ctypes.c_double), ("last_E", ctypes.c_int32), ("pos", ctypes.c_int32),
        ("token_errors", ctypes.c_int32),
        ("last_trace", ctypes.c_float * RIVER_MAX_LAYERS),
    ]


_LIB = None


def load_library(path=LIB_PATH):
    """Load libriver.so and declare the C signatures; raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run early_exit_kv_amd/build.py")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, f32, i64 = ctypes.c_int32, ctypes.c_float, ctypes.c_int64
    sig = {
        "river_query_sizes": (ctypes.c_int, [ctypes.POINTER(RiverConfig), ctypes.POINTER(RiverSizes)]),
        "river_exit_bank_offsets": (ctypes.c_int, [ctypes.POINTER(RiverConfig), i32, i32, i32,
                                                   ctypes.POINTER(ctypes.c_size_t),
                                                   ctypes.POINTER(ctypes.c_size_t)]),
        "river_init": (ctypes.c_int, [ctypes.POINTER(RiverConfig), ctypes.POINTER(RiverWeights), P, P,
                                      P, P, ctypes.POINTER(RiverSizes), P, ctypes.POINTER(P)]),
        "river_build_exit_layers": (ctypes.c_int, [P, i32]),
        "river_prefill": (ctypes.c_int, [P, P, i32, i32, f32, P, P]),
        "river_decode_step": (ctypes.c_int, [P, P, f32, P, P]),
        "river_decode_steps": (ctypes.c_int, [P, i32, P, f32, P, P]),
        "river_exit_stats": (ctypes.c_int, [P, ctypes.POINTER(RiverExitStats)]),
        "river_set_option": (ctypes.c_int, [P, i32, i64]),
        "river_reset": (ctypes.c_int, [P]),
        "river_destroy": (None, [P]),
        "river_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "river_profile_read": (ctypes.c_int, [P, ctypes.POINTER(RiverKernelTime)]),
        "river_debug_linear": (ctypes.c_int, [P, i32, i32, i32, P, i32, P]),
        "river_debug_linear_noalloc": (ctypes.c_int, [P, i32, i32, i32, P, i32, P]),
        "river_record_bytes": (ctypes.c_int, [ctypes.POINTER(RiverConfig), i32, ctypes.POINTER(ctypes.c_size_t)]),
        "river_set_record": (ctypes.c_int, [P, P, ctypes.c_size_t]),
        "river_time_kernel": (ctypes.c_int, [P, i32, i32, ctypes.POINTER(ctypes.c_double)]),
        "river_set_kv_state": (ctypes.c_int, [P, P, ctypes.c_size_t]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _lib_strerror(code):
    try:
        return load_library().river_strerror(code).decode()
    except Exception:  # the message is best effort
        return "?"


def _check(code, what):
    if code != RIVER_OK:
        raise RiverError(code, what)


def make_config(shape, max_batch, max_seq):
    """RiverConfig from a shape object/dict with the usual field names."""
    s = shape.as_dict() if hasattr(shape, "as_dict") else dict(shape)
    return RiverConfig(
        s["n_layers"], s["d_model"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn_dim"],
        s["vocab"], float(s.get("rms_eps", 1e-5)), float(s.get("rope_theta", 500000.0)),
        int(bool(s["tied_embeddings"])), s["group_size"], int(max_batch), int(max_seq))


def query_sizes(cfg):
    out = RiverSizes()
    _check(load_library().river_query_sizes(ctypes.byref(cfg), ctypes.byref(out)), "river_query_sizes")
    return out


def exit_bank_offsets(cfg, layer, linear, copy_layout=False):
    co, so = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().river_exit_bank_offsets(ctypes.byref(cfg), layer, linear, int(copy_layout),
                                                  ctypes.byref(co), ctypes.byref(so)),
           "river_exit_bank_offsets")
    return co.value, so.value


def record_bytes(cfg, rows):
    out = ctypes.c_size_t(0)
    _check(load_library().river_record_bytes(ctypes.byref(cfg), int(rows), ctypes.byref(out)),
           "river_record_bytes")
    return out.value


def _align256(n):
    return (n + 255) // 256 * 256


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


class River:
    """One decoder instance: borrowed weights, caller-owned device buffers
    (allocated here with torch), and the library context."""

    def __init__(self, shape, weights, max_batch, max_seq, copy_bank=False, device="cuda"):
        self.lib = load_library()
        if not torch.cuda.is_available():
            raise RuntimeError("river needs a GPU: torch.cuda.is_available() is False")
        self.shape = shape
        self.cfg = make_config(shape, max_batch, max_seq)
        self.sizes = query_sizes(self.cfg)
        dev = torch.device(device)
        bank = self.sizes.exit_bank_copy_bytes if copy_bank else self.sizes.exit_bank_bytes
        self.bank = torch.empty(bank, dtype=torch.uint8, device=dev)
        self.kv = torch.zeros(self.sizes.kv_cache_bytes // 2, dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(self.sizes.workspace_bytes, dtype=torch.uint8, device=dev)
        self.control = torch.zeros(self.sizes.control_bytes, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.Stream(device=dev)
        self.w = weights  # keep the borrowed tensors alive
        c = self.cfg
        for t in self._all_weight_tensors():
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise ValueError("weights must be contiguous bf16 tensors")
            if not t.is_cuda and not t.is_pinned():
                raise ValueError("weights must be CUDA tensors (or, for offloaded backbone "
                                 "linears, pinned host tensors)")
        for t in (weights["embed"], weights["final_norm"], weights.get("lm_head")):
            if t is not None and not t.is_cuda:
                raise ValueError("embedding, final norm and LM head must be CUDA tensors")
        n = c.n_layers
        self._layers = (RiverLayerW * n)()
        for i, lw in enumerate(weights["layers"]):
            for name, _ in RiverLayerW._fields_:
                t = lw[name]
                if not t.is_cuda and name in ("attn_norm", "mlp_norm"):
                    raise ValueError("norm gains must be CUDA tensors")
                setattr(self._layers[i], name, t.data_ptr() if t.is_cuda else device_address(t))
        rw = RiverWeights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                          weights["lm_head"].data_ptr() if weights.get("lm_head") is not None else None,
                          self._layers)
        sizes = RiverSizes(bank, self.sizes.exit_bank_copy_bytes, self.sizes.kv_cache_bytes,
                           self.sizes.workspace_bytes, self.sizes.control_bytes)
        self.ctx = ctypes.c_void_p()
        _check(self.lib.river_init(ctypes.byref(c), ctypes.byref(rw), _ptr(self.bank), _ptr(self.kv),
                                   _ptr(self.ws), _ptr(self.control), ctypes.byref(sizes),
                                   ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(self.ctx)),
               "river_init")
        self.batch = None

    def _all_weight_tensors(self):
        w = self.w
        yield w["embed"]
        yield w["final_norm"]
        if w.get("lm_head") is not None:
            yield w["lm_head"]
        for lw in w["layers"]:
            for name, _ in RiverLayerW._fields_:
                yield lw[name]

    # -- stream plumbing: the library runs on self.stream, ordered after the
    #    caller's current stream and before anything the caller enqueues next
    def _enter(self):
        self.stream.wait_stream(torch.cuda.current_stream())

    def _leave(self):
        torch.cuda.current_stream().wait_stream(self.stream)

    def _call(self, fn, what, *args):
        self._enter()
        try:
            _check(fn(self.ctx, *args), what)
        finally:
            self._leave()

    # -- API -----------------------------------------------------------------
    def build_exit_layers(self, mode="int4"):
        m = {"int4": RIVER_EXIT_INT4, "copy": RIVER_EXIT_COPY, "hqq": RIVER_EXIT_HQQ}[mode]
        self._call(self.lib.river_build_exit_layers, "river_build_exit_layers", m)
        self.mode = mode

    def prefill(self, tokens, tau, want_logits=True, logits=None, next_tok=None):
        B, T = tokens.shape
        tokens = tokens.to(torch.int32).contiguous()
        if logits is None and want_logits:
            logits = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        if next_tok is None:
            next_tok = torch.empty((B,), dtype=torch.int32, device=tokens.device)
        self._call(self.lib.river_prefill, "river_prefill", _ptr(tokens), B, T, ctypes.c_float(tau),
                   _ptr(logits), _ptr(next_tok))
        self.batch = B
        return logits, next_tok

    def decode_step(self, tokens, tau, want_logits=True, logits=None, next_tok=None):
        # the C ABI reads int32 ids in place; a converted copy would be a new
        # pointer, and so a new recorded graph, on every step
        if (not isinstance(tokens, torch.Tensor) or tokens.dtype != torch.int32 or not tokens.is_cuda
                or tokens.dim() != 1 or not tokens.is_contiguous()):
            raise ValueError("decode_step: tokens must be a contiguous int32 CUDA tensor of shape [B]")
        if self.batch is not None and tokens.shape[0] != self.batch:
            raise ValueError(f"decode_step: {tokens.shape[0]} tokens for a batch of {self.batch}")
        for name, t, dt in (("logits", logits, torch.float32), ("next_tok", next_tok, torch.int32)):
            if t is not None and (t.dtype != dt or not t.is_cuda or not t.is_contiguous()):
                raise ValueError(f"decode_step: {name} must be a contiguous {dt} CUDA tensor")
        B = tokens.shape[0]
        if logits is None and want_logits:
            logits = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        if next_tok is None:
            next_tok = torch.empty((B,), dtype=torch.int32, device=tokens.device)
        self._call(self.lib.river_decode_step, "river_decode_step", _ptr(tokens), ctypes.c_float(tau),
                   _ptr(logits), _ptr(next_tok))
        return logits, next_tok

    def decode_steps(self, tokens, n, tau, want_logits=True, logits=None, next_tok=None):
        """n decode steps in one call (river_decode_steps), the next tokens fed
        back on the device: returns (logits of the last step, next tokens
        [n, B])."""
        if (not isinstance(tokens, torch.Tensor) or tokens.dtype != torch.int32 or not tokens.is_cuda
                or tokens.dim() != 1 or not tokens.is_contiguous()):
            raise ValueError("decode_steps: tokens must be a contiguous int32 CUDA tensor of shape [B]")
        B = tokens.shape[0]
        if self.batch is not None and B != self.batch:
            raise ValueError(f"decode_steps: {B} tokens for a batch of {self.batch}")
        n = int(n)
        if next_tok is None:
            next_tok = torch.empty((n, B), dtype=torch.int32, device=tokens.device)
        if (next_tok.dtype != torch.int32 or not next_tok.is_cuda or not next_tok.is_contiguous()
                or tuple(next_tok.shape) != (n, B)):
            raise ValueError(f"decode_steps: next_tok must be a contiguous int32 CUDA tensor of shape [{n}, {B}]")
        if logits is None and want_logits:
            logits = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        if logits is not None and (logits.dtype != torch.float32 or not logits.is_cuda or not logits.is_contiguous()):
            raise ValueError("decode_steps: logits must be a contiguous float32 CUDA tensor")
        self._call(self.lib.river_decode_steps, "river_decode_steps", n, _ptr(tokens), ctypes.c_float(tau),
                   _ptr(logits), _ptr(next_tok))
        return logits, next_tok

    def exit_stats(self):
        st = RiverExitStats()
        self._call(self.lib.river_exit_stats, "river_exit_stats", ctypes.byref(st))
        L = self.cfg.n_layers
        return {
            "decode_hist": [st.decode_hist[e] for e in range(L + 1)],
            "prefill_hist": [st.prefill_hist[e] for e in range(L + 1)],
            "n_decode_steps": st.n_decode_steps, "n_prefill": st.n_prefill,
            "mean_exit_layer": st.mean_exit_layer, "last_E": st.last_E, "pos": st.pos,
            "token_errors": st.token_errors,
            "last_trace": [st.last_trace[l] for l in range(L)],
        }

    def set_option(self, option, value):
        _check(self.lib.river_set_option(self.ctx, option, ctypes.c_int64(value)), "river_set_option")

    def use_graph(self, on=True):
        self.set_option(RIVER_OPT_GRAPH, 1 if on else 0)

    def force_exit_layer(self, e):
        """-1: decide with tau; e in 0..L: layers < e backbone, the rest exit layers."""
        self.set_option(RIVER_OPT_FORCE_E, e)

    def gemv_mode(self, mode):
        """Kernel of decode linears of <= 8 rows: "auto" (per linear), "dot"
        (dot-product GEMV) or "mfma" (matrix-core GEMV where it fits)."""
        self.set_option(RIVER_OPT_GEMV, {"auto": 0, "dot": 1, "mfma": 2}[mode])

    def kv_strategy(self, name):
        """Layers at and past the exit: "river" (exit layers, the method) or a
        comparator: "kv_mask", "propagate", "mono", "recompute" (see
        include/river.h; "recompute" attaches a state buffer of max_seq rows)."""
        if name == "recompute" and getattr(self, "kv_state", None) is None:
            c = self.cfg
            self.kv_state = torch.empty(c.max_seq * c.d_model, dtype=torch.float32, device=self.ws.device)
            _check(self.lib.river_set_kv_state(self.ctx, _ptr(self.kv_state), self.kv_state.numel() * 4),
                   "river_set_kv_state")
        self.set_option(RIVER_OPT_KV_STRATEGY, KV_STRATEGIES.index(name))

    def attn_kind(self, kind):
        """Attention kernels (decode and prefill): "mfma" (matrix cores) or "valu"."""
        self.set_option(RIVER_OPT_ATTN, {"mfma": 0, "valu": 1}[kind])

    def profile(self, on=True):
        """Time every kernel with HIP events (decode steps then launch eagerly)."""
        self.set_option(RIVER_OPT_PROFILE, 1 if on else 0)

    def profile_read(self):
        """{kind: (launches, total_ms)} accumulated since the previous read."""
        arr = (RiverKernelTime * len(KERNEL_KINDS))()
        self._call(self.lib.river_profile_read, "river_profile_read", arr)
        return {k: (arr[i].launches, arr[i].total_ms) for i, k in enumerate(KERNEL_KINDS)}

    def debug_linear(self, layer, linear, use_exit, x, y=None, noalloc=False):
        """y = x W^T (fp32 [M][N]) for one linear through the production cores.
        noalloc=True calls river_debug_linear_noalloc (partial tiles in the
        library's static scratch); pass y to reuse an output buffer."""
        N, K = self.linear_shape(linear)
        x = x.to(torch.bfloat16).contiguous()
        assert x.shape[1] == K
        if y is None:
            y = torch.empty((x.shape[0], N), dtype=torch.float32, device=x.device)
        assert y.dtype == torch.float32 and y.is_contiguous() and y.shape == (x.shape[0], N)
        fn, name = ((self.lib.river_debug_linear_noalloc, "river_debug_linear_noalloc") if noalloc
                    else (self.lib.river_debug_linear, "river_debug_linear"))
        self._call(fn, name, layer, linear, int(use_exit), _ptr(x), x.shape[0], _ptr(y))
        return y

    def time_kernel(self, kind, reps=20):
        """Mean execution time (us) of one decode kernel class, launched back to
        back for every layer from a replayed graph (see river_time_kernel)."""
        k = KERNEL_KINDS.index(kind) if isinstance(kind, str) else int(kind)
        out = ctypes.c_double(0.0)
        self._call(self.lib.river_time_kernel, "river_time_kernel", k, int(reps), ctypes.byref(out))
        return out.value

    def record(self, max_rows):
        """Switch the activation record on for passes of up to max_rows rows
        (max_rows=0 switches it off)."""
        if max_rows <= 0:
            _check(self.lib.river_set_record(self.ctx, None, 0), "river_set_record")
            self.rec = None
            return
        n = record_bytes(self.cfg, max_rows)
        self.rec = torch.zeros(n, dtype=torch.uint8, device=self.ws.device)
        _check(self.lib.river_set_record(self.ctx, _ptr(self.rec), n), "river_set_record")

    def read_record(self, rows):
        """Arrays of the last pass with `rows` rows: a list of per-layer dicts
        (h_in, q, attn, h_mid, u) and the final residual, as float64 numpy."""
        torch.cuda.synchronize()
        c = self.cfg
        qd = c.n_q_heads * c.head_dim
        fields = (("h_in", c.d_model, 4), ("q", qd, 2), ("attn", qd, 2), ("h_mid", c.d_model, 4),
                  ("u", c.ffn_dim, 2))
        buf = self.rec

        def arr(off, width, nbytes):
            v = buf[off:off + rows * width * nbytes]
            t = v.view(torch.float32) if nbytes == 4 else v.view(torch.bfloat16).float()
            return t.reshape(rows, width).cpu().double().numpy()

        layers, off = [], 0
        for _ in range(c.n_layers):
            d = {}
            for name, width, nb in fields:
                d[name] = arr(off, width, nb)
                off += _align256(rows * width * nb)
            layers.append(d)
        return layers, arr(off, c.d_model, 4)

    def reset(self):
        _check(self.lib.river_reset(self.ctx), "river_reset")

    def close(self):
        if self.ctx:
            self.lib.river_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- views of the caller-owned buffers (layouts from include/river.h) -----
    def kv_views(self):
        c = self.cfg
        kv = self.kv.view(2, c.n_layers, c.max_batch, c.n_kv_heads, c.max_seq, c.head_dim)
        return kv[0], kv[1]

    def exit_linear_packed(self, layer, linear):
        """(codes uint32 [N][K/8], sz uint32 [N][K/G]) tensors viewing the bank."""
        N, K = self.linear_shape(linear)
        co, so = exit_bank_offsets(self.cfg, layer, linear)
        words = self.bank[co:co + N * (K // 8) * 4].view(torch.int32).view(N, K // 8)
        G = self.cfg.group_size
        sz = self.bank[so:so + N * (K // G) * 4].view(torch.int32).view(N, K // G)
        return words, sz

    def linear_shape(self, linear):
        c = self.cfg
        qd, kd = c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim
        return [(qd, c.d_model), (kd, c.d_model), (kd, c.d_model), (c.d_model, qd),
                (c.ffn_dim, c.d_model), (c.ffn_dim, c.d_model), (c.d_model, c.ffn_dim)][linear]


_HIP = None


def device_address(t):
    """Device-side address of a pinned host tensor (hipHostGetDevicePointer)."""
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipHostGetDevicePointer.restype = ctypes.c_int
        _HIP.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
    out = ctypes.c_void_p()
    rc = _HIP.hipHostGetDevicePointer(ctypes.byref(out), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0 or not out.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({rc}): is the tensor pinned?")
    return out.value


def offload_layers(weights, first_layer):
    """Backbone offloading (lead page, section 5): a copy of the weight dict in
    which the seven linear matrices of layers >= first_layer are pinned host
    tensors (the device reads them over the host link only when it runs that
    layer on its backbone).  Norm gains, embedding and LM head stay where they
    are.  Drop the caller's references to the original tensors of those
    layers to release their device memory."""
    out = {k: v for k, v in weights.items() if k != "layers"}
    out["layers"] = []
    for l, lw in enumerate(weights["layers"]):
        nl = dict(lw)
        if l >= first_layer:
            for name in LINEAR_NAMES:
                h = torch.empty(lw[name].shape, dtype=lw[name].dtype, pin_memory=True)
                h.copy_(lw[name])
                nl[name] = h
        out["layers"].append(nl)
    return out


def unpack_int4(words, sz, group):
    """Host-side unpacking of the packed exit layout (include/river.h):
    returns codes uint8 [N][K], scale and zero as float32 [N][K/G]."""
    import numpy as np
    w = np.asarray(words, dtype=np.int64) & 0xFFFFFFFF
    N, KW = w.shape
    codes = np.empty((N, KW * 8), dtype=np.uint8)
    for j in range(8):   # byte i: column i low nibble, column i + 4 high nibble
        shift = 8 * j if j < 4 else 8 * (j - 4) + 4
        codes[:, j::8] = ((w >> shift) & 0xF).astype(np.uint8)
    z32 = np.asarray(sz, dtype=np.int64) & 0xFFFFFFFF
    s = ((z32 & 0xFFFF).astype(np.uint32) << 16).view(np.float32)
    z = ((z32 >> 16).astype(np.uint32) << 16).view(np.float32)
    return codes, s, z


def tau_is_valid(tau):
    return math.isfinite(tau)
