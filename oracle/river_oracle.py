"""Plain CPU oracle of the KV-shared early-exit decoder (River-LLM).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  It shares no code with the HIP path
and must never be used as a fallback for it.

What it computes follows the lead page ("River-LLM: Large Language Model
Seamless Exit Based on KV Share", arXiv:2604.18396):

* section 3 (KV-shared exit river): beside each decoder layer sits an *exit
  layer*, a full copy of that layer's parameters that is then quantised to
  4-bit weights with 16-bit activations (W4A16), built without training; the
  exit layer writes its K/V into the slot of the shared cache that belongs to
  the original layer, so later tokens never find a missing entry;
* section 4 (exit decision): at each layer the state-transition similarity
  between that layer's input and output is taken per token; if its minimum
  over the batch exceeds tau, the rest of the layers run as exit layers, and
  no deeper layer checks again;
* section 5 (prefill / generation): prefill takes one sequence-level decision
  for all prompt tokens, generation decides once per generated position.

Arithmetic: float64 for the forward pass.  Activations that the method keeps
in 16 bits (the "A16" of W4A16) are rounded to bf16 at the points where the
decoder stores them: the RMSNorm outputs that feed a linear layer, q/k/v
after RoPE (k and v are what the cache holds), the attention output, and the
SwiGLU product.  The residual stream stays wide.  The quantiser follows its
definition in float32, because its result is an integer code that both sides
must reach in the same precision.

Readings where the pages are silent (all stated again where they are used):
the similarity is the cosine between the residual stream entering a layer and
the one leaving it; "exceeds" is a strict ``>``; the test runs after each
backbone layer except the last; the quantiser is asymmetric min-max
round-to-nearest with a float zero point per (output row, group of G inputs),
the parameter form of HQQ, without HQQ's refinement step.
"""
import math

import numpy as np

EXIT_INT4 = "int4"
EXIT_COPY = "copy"
EXIT_HQQ = "hqq"


# --------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even)
# --------------------------------------------------------------------------
def bf16_from_f32(x):
    """Round float32 values to the nearest bf16 value (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32)
    return np.where(np.isnan(x), x, out)


def bf16_from_f64(x):
    """Round float64 values to the nearest bf16 value in one step (no double
    rounding through float32); float64 out.  Exact for results in the normal
    range of bf16, which is all this decoder produces."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    drop = np.uint64(45)  # 52 fraction bits of float64 minus 7 of bf16
    lsb = (u >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    mask = ~np.uint64((1 << 45) - 1)
    r = ((u + half + lsb) & mask).view(np.float64)
    # beyond bf16's largest finite value the rounding goes to infinity
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


# --------------------------------------------------------------------------
# Exit-layer construction: copy, then 4-bit quantisation
# (lead page, section 3: copy the layer's parameters in full, then quantise
#  to W4A16; the page names HQQ as the default quantiser)
# --------------------------------------------------------------------------
def quantize_int4(w, group):
    """Asymmetric 4-bit quantisation of a row-major weight matrix.

    For each output row and each group of ``group`` consecutive input columns
    (all float32, every operation separately rounded):
        lo, hi = min, max of the group
        s = bf16(fl(hi - lo) / 15), and s = 1 when that is 0
        z = bf16(fl(-lo / s))
        q = clamp(round_half_even(fl(fl(w / s) + z)), 0, 15)
    Returns (q uint8 [N,K], s float32 [N,K/G], z float32 [N,K/G]); s and z hold
    bf16 values.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % group:
        raise ValueError("group size must divide the number of columns")
    wg = w.reshape(n, k // group, group)
    lo = wg.min(axis=-1)
    hi = wg.max(axis=-1)
    s = bf16_from_f32((hi - lo) / np.float32(15.0))
    s = np.where(s == np.float32(0.0), np.float32(1.0), s).astype(np.float32)
    z = bf16_from_f32(-lo / s)
    t = wg / s[..., None]
    t = t + z[..., None]
    q = np.clip(np.rint(t), 0, 15).astype(np.uint8)
    return q.reshape(n, k), s, z


# HQQ-style refinement of the zero point.  The page names HQQ as its default
# quantiser but gives none of its steps; these are the published defaults of
# the half-quadratic solver (beta 10, growth kappa 1.01, 20 rounds), with the
# l1 norm (p = 1) as the sparsity-promoting error norm: its proximal step is a
# plain soft threshold, so every step is a separately rounded float32
# operation and both sides reach the same codes bit for bit (HQQ's p < 1 needs
# a power function, which no two math libraries round alike).
HQQ_ITERS = 20
HQQ_BETA = 10.0
HQQ_KAPPA = 1.01


def tree_sum_f32(x):
    """Sum over the last axis (a power of two) in a fixed pairwise order, in
    float32: the two halves are added element-wise, then the two halves of
    that, down to a single value."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    if n & (n - 1):
        raise ValueError("the tree sum takes a power-of-two length")
    while n > 1:
        n //= 2
        x = x[..., :n] + x[..., n:2 * n]
    return x[..., 0]


def quantize_int4_hqq(w, group, iters=HQQ_ITERS, beta=HQQ_BETA, kappa=HQQ_KAPPA):
    """4-bit quantisation with an HQQ-style refinement of the zero point.

    Starts from the min-max quantiser (quantize_int4: scale s and zero z), then
    alternates, for ``iters`` rounds, per (row, group), in float32 with every
    operation separately rounded and zf = z to begin with:
        q  = clamp(round_half_even(fl(fl(w / s) + zf)), 0, 15)   quantise
        e  = fl(w - fl(fl(q - zf) * s))                          residual
        we = sign(e) * max(fl(|e| - fl(1 / beta)), 0)            proximal step of |.|_1
        zf = fl(tree_sum(fl(q - fl(fl(w - we) / s))) / G)        closed-form zero
        beta = fl(beta * kappa)
    (half-quadratic splitting: the error variable we absorbs the sparse large
    residuals, the zero is the least-squares fit of the rest).  The scale keeps
    its min-max value; the zero is stored as bf16(zf) and the codes are taken
    once more with the stored scale and zero.  iters = 0 is quantize_int4.
    Returns (q uint8 [N,K], s float32 [N,K/G], z float32 [N,K/G]).
    """
    q0, s, z = quantize_int4(w, group)
    if iters == 0:
        return q0, s, z
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    wg = w.reshape(n, k // group, group)
    sg = s[..., None]
    zf = z.astype(np.float32)
    b = np.float32(beta)
    kap = np.float32(kappa)
    inv_g = np.float32(1.0) / np.float32(group)       # a power of two: exact
    for _ in range(iters):
        q = np.clip(np.rint((wg / sg) + zf[..., None]), 0, 15).astype(np.float32)
        e = wg - (q - zf[..., None]) * sg
        thr = np.float32(1.0) / b
        we = np.sign(e) * np.maximum(np.abs(e) - thr, np.float32(0.0))
        t = q - (wg - we) / sg
        zf = (tree_sum_f32(t) * inv_g).astype(np.float32)
        b = np.float32(b * kap)
    zb = bf16_from_f32(zf)
    q = np.clip(np.rint((wg / sg) + zb[..., None]), 0, 15).astype(np.uint8)
    return q.reshape(n, k), s, zb


def dequantize_int4(q, s, z, group):
    """w_hat = fl(fl(q - z) * s) in float32 (the W ~ s (q - z) form)."""
    n, k = q.shape
    qg = q.reshape(n, k // group, group).astype(np.float32)
    wh = (qg - z[..., None]) * s[..., None]
    return wh.reshape(n, k).astype(np.float32)


# --------------------------------------------------------------------------
# Decoder pieces (Llama-style layer: pre-norm attention and SwiGLU MLP)
# --------------------------------------------------------------------------
def rmsnorm(h, gain, eps):
    """h / sqrt(mean(h^2) + eps) * gain, over the last axis, float64."""
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope_tables(positions, head_dim, theta):
    """cos/sin [n, head_dim/2] of angle pos * theta^(-2i/head_dim), float64."""
    half = head_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x, cos, sin):
    """Rotate-half RoPE: pair (i, i + D/2) turned by the angle of index i.
    x [..., n, H, D]; cos/sin [n, D/2]."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c = cos[:, None, :]
    s = sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(a):
    return a / (1.0 + np.exp(-a))


def cosine_rows(a, b):
    """Per-row cosine a.b / max(|a||b|, 1e-8), clamped to [-1, 1], float64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    num = np.sum(a * b, axis=-1)
    den = np.maximum(np.sqrt(np.sum(a * a, axis=-1)) * np.sqrt(np.sum(b * b, axis=-1)), 1e-8)
    return np.clip(num / den, -1.0, 1.0)


def linear(x, w):
    """x @ w^T in float64 (w is a row-major [N][K] matrix)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


class Shape:
    """Decoder hyper-parameters (names follow the usual Llama notation)."""

    def __init__(self, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim,
                 vocab, group_size, tied_embeddings, rms_eps=1e-5, rope_theta=500000.0, **_):
        self.L, self.d, self.Hq, self.Hkv, self.Dh = n_layers, d_model, n_q_heads, n_kv_heads, head_dim
        self.F, self.V, self.G = ffn_dim, vocab, group_size
        self.tied = bool(tied_embeddings)
        self.eps, self.theta = float(rms_eps), float(rope_theta)


def attention(q, kc, vc, start, n, present=None):
    """Causal GQA attention for n new rows at positions start..start+n-1.

    q [B, n, Hq, D]; kc/vc [B, Hkv, S, D] already hold the new keys/values.
    Query head h reads kv head floor(h * Hkv / Hq).  Scores q.k / sqrt(D),
    softmax with its maximum subtracted, float64.  Returns [B, n, Hq, D].
    ``present`` (bool per position, or None for all): earlier positions whose
    keys/values this layer does not hold are left out (the KV-mask strategy).
    """
    B, _, Hq, D = q.shape
    Hkv = kc.shape[1]
    end = start + n
    out = np.empty((B, n, Hq, D), dtype=np.float64)
    rows = np.arange(n)[:, None] + start
    cols = np.arange(end)[None, :]
    masked = cols > rows
    if present is not None:
        masked = masked | ~np.asarray(present[:end], dtype=bool)[None, :]
    for b in range(B):
        for h in range(Hq):
            j = (h * Hkv) // Hq
            k = kc[b, j, :end].astype(np.float64)
            v = vc[b, j, :end].astype(np.float64)
            sc = (q[b, :, h].astype(np.float64) @ k.T) / math.sqrt(D)
            sc = np.where(masked, -np.inf, sc)
            sc = sc - sc.max(axis=-1, keepdims=True)
            p = np.exp(sc)
            p = p / p.sum(axis=-1, keepdims=True)
            out[b, :, h] = p @ v
    return out


def layer_kv(shape, lw, h, start, kc, vc):
    """Keys and values of one layer for h [B, n, d] at positions
    start..start+n-1 (RMSNorm, the k and v projections, RoPE on k), written
    into this layer's cache slots; the layer's attention and MLP do not run
    (the state-propagation strategy's deeper layers)."""
    B, n, d = h.shape
    Hkv, D = shape.Hkv, shape.Dh
    x = bf16_from_f64(rmsnorm(h, lw["attn_norm"], shape.eps))
    k = linear(x, lw["wk"]).reshape(B, n, Hkv, D)
    v = linear(x, lw["wv"]).reshape(B, n, Hkv, D)
    cos, sin = rope_tables(np.arange(start, start + n), D, shape.theta)
    kc[:, :, start:start + n] = bf16_from_f64(apply_rope(k, cos, sin)).transpose(0, 2, 1, 3)
    vc[:, :, start:start + n] = bf16_from_f64(v).transpose(0, 2, 1, 3)


def decoder_layer(shape, lw, h, start, kc, vc, rec=None, present=None):
    """One decoder layer on h [B, n, d] at positions start..start+n-1.

    ``lw`` holds float32 copies of the layer weights (backbone or exit copy).
    Writes the new K/V into kc/vc [B, Hkv, S, D] (this layer's slots of the
    shared cache) and returns the residual stream after the layer (float64).
    If ``rec`` is a dict, the stored activations are put in it (q after RoPE,
    attention output, residual after the attention block, SwiGLU product).
    """
    B, n, d = h.shape
    Hq, Hkv, D = shape.Hq, shape.Hkv, shape.Dh
    x = bf16_from_f64(rmsnorm(h, lw["attn_norm"], shape.eps))
    q = linear(x, lw["wq"]).reshape(B, n, Hq, D)
    k = linear(x, lw["wk"]).reshape(B, n, Hkv, D)
    v = linear(x, lw["wv"]).reshape(B, n, Hkv, D)
    cos, sin = rope_tables(np.arange(start, start + n), D, shape.theta)
    q = bf16_from_f64(apply_rope(q, cos, sin))
    k = bf16_from_f64(apply_rope(k, cos, sin))
    v = bf16_from_f64(v)
    kc[:, :, start:start + n] = k.transpose(0, 2, 1, 3)
    vc[:, :, start:start + n] = v.transpose(0, 2, 1, 3)
    o = bf16_from_f64(attention(q, kc, vc, start, n, present)).reshape(B, n, Hq * D)
    h1 = h + linear(o, lw["wo"])
    x2 = bf16_from_f64(rmsnorm(h1, lw["mlp_norm"], shape.eps))
    u = bf16_from_f64(silu(linear(x2, lw["w_gate"])) * linear(x2, lw["w_up"]))
    if rec is not None:
        rec.update(h_in=h.copy(), q=q.reshape(B, n, Hq * D), attn=o.copy(), h_mid=h1.copy(), u=u.copy())
    return h1 + linear(u, lw["w_down"])


def lm_head(shape, h, final_norm, w_lm):
    """logits = bf16(rmsnorm(h, final_norm)) @ W_lm^T, float64 [.., V]."""
    x = bf16_from_f64(rmsnorm(h, final_norm, shape.eps))
    return linear(x, w_lm)


def greedy(logits):
    """argmax over the vocabulary; the lowest index wins ties."""
    return np.argmax(logits, axis=-1).astype(np.int64)


# --------------------------------------------------------------------------
# The river: backbone layers, exit layers, shared cache, exit controller
# --------------------------------------------------------------------------
class RiverOracle:
    """KV-shared early-exit decoder on the CPU.

    weights: dict with float32 numpy arrays (bf16 values):
      embed [V,d], final_norm [d], lm_head [V,d] or None (tied to embed),
      layers: list of dicts attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down.
    """

    LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")

    def __init__(self, shape, weights, max_batch, max_seq):
        self.s = shape if isinstance(shape, Shape) else Shape(**shape)
        self.w = weights
        self.max_batch, self.max_seq = int(max_batch), int(max_seq)
        self.exit_layers = None
        self.exit_codes = None   # per layer: name -> (q, s, z) in int4 mode
        s = self.s
        kv_shape = (s.L, self.max_batch, s.Hkv, self.max_seq, s.Dh)
        self.k_cache = np.zeros(kv_shape, dtype=np.float64)
        self.v_cache = np.zeros(kv_shape, dtype=np.float64)
        self.strategy = "river"
        self.reset()

    # -- build ------------------------------------------------------------
    def build_exit_layers(self, mode=EXIT_INT4):
        """One exit layer per decoder layer: a copy of all its parameters,
        with the seven linear matrices quantised in int4 mode (min-max) or hqq
        mode (min-max, then the HQQ-style zero refinement); norm gains are
        copied as they are.  Embedding, final norm and LM head get no copy."""
        if mode not in (EXIT_INT4, EXIT_COPY, EXIT_HQQ):
            raise ValueError(mode)
        quant = quantize_int4_hqq if mode == EXIT_HQQ else quantize_int4
        self.exit_layers, self.exit_codes = [], []
        for lw in self.w["layers"]:
            ex, codes = {}, {}
            for name, arr in lw.items():
                if name in self.LINEARS and mode in (EXIT_INT4, EXIT_HQQ):
                    q, sc, z = quant(arr, self.s.G)
                    codes[name] = (q, sc, z)
                    ex[name] = dequantize_int4(q, sc, z, self.s.G)
                else:
                    ex[name] = np.array(arr, dtype=np.float32, copy=True)
            self.exit_layers.append(ex)
            self.exit_codes.append(codes)

    # What happens to the layers at and past the exit (E .. L-1):
    #   river      they run as their exit layers and write K/V into the shared
    #              cache (the method of the lead page, section 3);
    #   and, as speed comparators, three of the prior fixes the page's
    #   section 2 describes for the missing K/V of early-exited tokens:
    #   kv_mask    they are skipped; deeper layers of later tokens leave out
    #              the positions whose K/V they do not hold;
    #   propagate  they only compute their K/V from the exit state (their own
    #              RMSNorm gain, k and v projections and RoPE), no attention
    #              and no MLP;
    #   mono       they are skipped, and the exit layer never increases along
    #              the sequence: a decode step also exits on reaching the
    #              previous pass's E, so every layer a token runs holds K/V
    #              for all earlier positions.
    #   recompute  they are skipped; each position keeps its state at its
    #              exit, and when a later pass runs layer l, the earlier
    #              positions that lack layer l's K/V run layer l (backbone)
    #              as extra rows of that pass, their state advancing with it.
    #              A position's depth (the layers it holds K/V for) is the
    #              largest E of the passes from its own on, so it never grows
    #              along the sequence and the rows missing at layer l are the
    #              last positions before the current one.
    #   In every strategy but river the logits come from the exit state.
    KV_STRATEGIES = ("river", "kv_mask", "propagate", "mono", "recompute")

    def set_kv_strategy(self, name):
        if name not in self.KV_STRATEGIES:
            raise ValueError(name)
        self.strategy = name

    def reset(self):
        self.pos = 0
        self.batch = None
        self.last_E = self.s.L
        self.pos_E = np.full(self.max_seq, self.s.L, dtype=np.int64)
        # recompute: each position's depth and its state at the input of
        # that depth's layer
        self.depth = np.full(self.max_seq, self.s.L, dtype=np.int64)
        self.h_state = np.zeros((self.max_batch, self.max_seq, self.s.d), dtype=np.float64)

    # -- one pass over all layers ------------------------------------------
    def _run(self, tokens, start, tau, force_E, record):
        s = self.s
        B, n = tokens.shape
        h = self.w["embed"][tokens].astype(np.float64)        # [B, n, d]
        strat = getattr(self, "strategy", "river")
        # mono: a decode step exits at the latest on reaching the previous E
        cap = self.last_E if (strat == "mono" and start > 0) else s.L
        exited = False
        E = s.L
        trace = []
        inputs = []
        for l in range(s.L):
            if force_E is not None:
                use_exit = l >= force_E
            else:
                use_exit = exited
            if use_exit and strat != "river":
                # past the exit: skipped, or (propagate) only this layer's K/V
                # from the exit state; the residual stream stays as it is
                if strat == "propagate":
                    layer_kv(s, self.w["layers"][l], h, start, self.k_cache[l, :B], self.v_cache[l, :B])
                continue
            lw = self.exit_layers[l] if use_exit else self.w["layers"][l]
            rec = {} if record else None
            present = None
            if strat == "kv_mask":
                present = self.pos_E > l                       # earlier positions holding layer l
                present[start:] = True
            pend = np.nonzero(self.depth[:start] <= l)[0] if strat == "recompute" else ()
            if len(pend):
                # the earlier positions without layer l's K/V go through layer
                # l together with this pass's rows
                q0 = int(pend[0])
                assert np.array_equal(pend, np.arange(q0, start)), "missing rows are not a suffix"
                rows = np.concatenate([self.h_state[:B, q0:start], h], axis=1)
                out = decoder_layer(s, lw, rows, q0, self.k_cache[l, :B], self.v_cache[l, :B], rec)
                self.h_state[:B, q0:start] = out[:, :start - q0]
                self.depth[q0:start] = l + 1
                h_out = out[:, start - q0:]
                if record:
                    rec = {k: v[:, start - q0:] for k, v in rec.items()}
            else:
                h_out = decoder_layer(s, lw, h, start, self.k_cache[l, :B], self.v_cache[l, :B], rec, present)
            if record:
                inputs.append(rec)
            if force_E is None:
                if not exited and l < s.L - 1:
                    # batch minimum of the per-token state-transition similarity
                    m = float(cosine_rows(h.reshape(-1, s.d), h_out.reshape(-1, s.d)).min())
                    trace.append(m)
                    # the decision is taken in float32, like the device's
                    if np.float32(m) > np.float32(tau) or l + 1 >= cap:
                        exited = True
                        E = l + 1
            h = h_out
        if force_E is not None:
            E = int(force_E)
        self.last_E = E
        self.pos_E[start:start + n] = E
        self.depth[start:start + n] = E
        self.h_state[:B, start:start + n] = h
        w_lm = self.w["embed"] if self.w["lm_head"] is None else self.w["lm_head"]
        logits = lm_head(s, h[:, -1], self.w["final_norm"], w_lm)
        res = {"logits": logits, "next": greedy(logits), "E": E, "trace": trace, "h_final": h}
        if record:
            res["layers"] = inputs
        return res

    def prefill(self, tokens, tau, force_E=None, record=False):
        """Sequence-level exit: one decision per layer for all B*T prompt rows
        (the minimum runs over every row).  Logits of each row's last position."""
        if self.exit_layers is None:
            raise RuntimeError("build_exit_layers first")
        tokens = np.asarray(tokens, dtype=np.int64)
        B, T = tokens.shape
        if B > self.max_batch or T > self.max_seq:
            raise ValueError("prefill exceeds the cache")
        self.reset()
        res = self._run(tokens, 0, tau, force_E, record)
        self.pos = T
        self.batch = B
        return res

    def decode_step(self, tokens, tau, force_E=None, record=False):
        """Token-level exit for one generated position (all B rows share it)."""
        if self.exit_layers is None or self.batch is None:
            raise RuntimeError("prefill first")
        tokens = np.asarray(tokens, dtype=np.int64).reshape(-1, 1)
        if tokens.shape[0] != self.batch:
            raise ValueError("batch size differs from the prefill's")
        if self.pos + 1 > self.max_seq:
            raise ValueError("cache full")
        res = self._run(tokens, self.pos, tau, force_E, record)
        res["pos"] = self.pos
        self.pos += 1
        return res

    def kv_bytes_per_token(self, dtype_bytes=2):
        """Bytes the single shared cache holds per token (K and V, all layers)."""
        s = self.s
        return s.L * 2 * s.Hkv * s.Dh * dtype_bytes
