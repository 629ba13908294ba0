"""Stage-by-stage check of one pass of the decoder, with every stage of the
oracle fed the activations the implementation under test stored.

Why teacher forcing at every stored activation: the decoder keeps its
activations in bf16 (the A16 of W4A16).  Two correct implementations whose
fp32 sums differ only in order round a few elements the other way; each later
bf16 rounding turns such a difference of a few 1e-7 into whole ulps, so after
two or three layers the logits of any two correct implementations differ by
about one bf16 ulp of the normalised final state, which on a 128k vocabulary
is already ~2e-2 of the logit spread.  Feeding the oracle the stored values
instead checks every stage on its own, and tightly:

* a stored bf16 value must be a round-to-nearest-even of a value within an
  allowance ``b`` of the exact (float64) result computed from the teacher-
  forced inputs: ``bf16(e - b) <= g <= bf16(e + b)``;
* a stored fp32 value must lie within ``b`` of the exact result;
* ``b`` is an fp32 evaluation allowance: 8 sqrt(K) 2^-24 sum|x||w| for a
  length-K product (the probabilistic sqrt(K) bound with a wide margin), plus
  the effect of inputs that the implementation normalises internally and may
  round to the other bf16 neighbour when the exact value sits within 1e-5
  (relative) of a rounding midpoint.

The oracle's pieces (RMSNorm, linear, RoPE, attention, SiLU, LM head) come
from ``oracle.river_oracle``; the allowances are written here.
"""
import numpy as np

from oracle import river_oracle as ro

U32 = 2.0 ** -24      # unit roundoff of fp32
C_ACC = 8.0           # margin on the sqrt(K) accumulation bound
DELTA_NORM = 1e-5     # relative evaluation error allowed for a normalised input
COS_TOL = 1e-5        # fp32 cosine vs exact cosine of the same stored states
LOGIT_BAR = 2e-2      # max |dlogit| <= LOGIT_BAR * std(logits)


def bf16_interval_ok(g, e, b):
    lo = ro.bf16_from_f64(e - b)
    hi = ro.bf16_from_f64(e + b)
    return (g >= lo) & (g <= hi)


def flip_size(x):
    """For exact normalised values x: how far the bf16 value an fp32
    evaluation may store can sit from bf16(x) (0 unless x is within
    DELTA_NORM of a rounding midpoint)."""
    xr = ro.bf16_from_f64(x)
    a = ro.bf16_from_f64(x - DELTA_NORM * np.abs(x))
    c = ro.bf16_from_f64(x + DELTA_NORM * np.abs(x))
    return xr, np.maximum(np.abs(a - xr), np.abs(c - xr))


def product(x, w, fl=None):
    """Exact x @ w^T and its fp32 allowance (x stored values; fl flip sizes)."""
    w = np.asarray(w)
    y = ro.linear(x, w)
    aw = np.abs(w).astype(np.float32)
    k = w.shape[1]
    b = C_ACC * np.sqrt(k) * U32 * (np.abs(x).astype(np.float32) @ aw.T).astype(np.float64)
    if fl is not None:
        b = b + (fl.astype(np.float32) @ aw.T).astype(np.float64)
    return y, b


class Report:
    def __init__(self):
        self.worst = {}

    def bf16(self, name, g, e, b):
        ok = bf16_interval_ok(g, e, b)
        if not np.all(ok):
            i = np.unravel_index(np.argmin(ok), ok.shape)
            raise AssertionError(f"{name}: {int((~ok).sum())} of {ok.size} stored bf16 values outside "
                                 f"the allowance; first at {i}: got {g[i]!r}, exact {e[i]!r}, b {b[i]!r}")
        # share of values stored as the other neighbour of the exact result
        self._note(name + " flips", np.array([np.mean(g != ro.bf16_from_f64(e))]))

    def f32(self, name, g, e, b):
        d = np.abs(g - e)
        bad = d > b
        if np.any(bad):
            i = np.unravel_index(np.argmax(d - b), d.shape)
            raise AssertionError(f"{name}: {int(bad.sum())} of {d.size} fp32 values outside the "
                                 f"allowance; worst at {i}: got {g[i]!r}, exact {e[i]!r}, b {b[i]!r}")
        self._note(name, d / (b + 1e-30))

    def _note(self, name, r):
        key = name.split("[")[0] + (" flips" if name.endswith(" flips") else "")
        self.worst[key] = max(self.worst.get(key, 0.0), float(np.max(r)) if r.size else 0.0)


def rope_allowance(y, b, pos, D, theta):
    """RoPE on exact products y [R, H, D] (rotate-half pairs) with allowance b."""
    cos, sin = ro.rope_tables(pos, D, theta)
    e = ro.apply_rope(y, cos, sin)
    half = D // 2
    c = np.abs(cos)[:, None, :]
    s = np.abs(sin)[:, None, :]
    b0, b1 = b[..., :half], b[..., half:]
    y0, y1 = np.abs(y[..., :half]), np.abs(y[..., half:])
    rb = np.concatenate([c * b0 + s * b1, c * b1 + s * b0], axis=-1)
    rb = rb + 4 * U32 * np.concatenate([y0 + y1, y0 + y1], axis=-1)
    return e, rb


def attention_row(q, k, v, scale):
    """Exact softmax(q k^T scale) v of one query row over the stored keys and
    values k, v [n][Dh] (float64), and its fp32 evaluation allowance: the
    score error (accumulation bound plus the exponential's few ulps) carried
    through the softmax, the accumulation of the n products, the final
    rounding."""
    n = k.shape[0]
    sc = (k @ q) * scale
    m = sc.max()
    w = np.exp(sc - m)
    pr = w / w.sum()
    o = pr @ v
    ds = C_ACC * np.sqrt(k.shape[1]) * U32 * scale * (np.abs(k) @ np.abs(q)) + 4e-6 * (1.0 + np.abs(sc - m))
    b = 2.0 * (pr * ds) @ np.abs(v - o) + C_ACC * np.sqrt(n) * U32 * (pr @ np.abs(v)) + 2 * U32 * np.abs(o)
    return o, b


def check_pass(shape, layer_weights, E, rec_layers, h_out, kc, vc, B, n, start, trace, tau,
               logits, nxt, final_norm, w_lm, report=None, strategy="river", pos_E=None, forced=False,
               cap=None):
    """Check one prefill (n = T rows per sequence, start = 0) or decode step
    (n = 1, start = position) of the implementation under test.

    layer_weights(l, use_exit) -> dict of float32 arrays (the oracle's backbone
    or exit copy); rec_layers / h_out: the stored activations (rows ordered
    b-major, float64); kc, vc: the stored cache [L][B][Hkv][S][D] (float64);
    trace: the per-layer batch-min cosines the implementation recorded.

    strategy: what the layers from E on did.  "river": ran as exit layers;
    "kv_mask" / "mono": skipped (nothing stored, the final state is the exit
    state), and under "kv_mask" the attention of layer l leaves out the
    earlier positions p with pos_E[p] <= l; "propagate": only their K/V,
    from the exit state with the backbone's norm gain and k/v projections.
    forced: E was forced (no exit test ran); cap: under "mono", the E at which
    the pass exits whatever the cosine (the previous pass's E).
    """
    s = shape
    rep = report or Report()
    R = B * n
    L = s.L
    qd, kd = s.Hq * s.Dh, s.Hkv * s.Dh
    pos = np.tile(np.arange(start, start + n), B)           # position of each row
    bidx = np.repeat(np.arange(B), n)
    end = start + n
    skip = strategy != "river"
    last_run = E if skip else L                              # layers that ran in full
    for l in range(L):
        use_exit = l >= E
        if skip and use_exit:
            if strategy == "propagate":
                lw = layer_weights(l, False)
                xr, fl = flip_size(ro.rmsnorm(h_out, lw["attn_norm"], s.eps))
                yk, bk = product(xr, lw["wk"], fl)
                yv, bv = product(xr, lw["wv"], fl)
                ek, rk = rope_allowance(yk.reshape(R, s.Hkv, s.Dh), bk.reshape(R, s.Hkv, s.Dh), pos, s.Dh,
                                        s.theta)
                tag = f"layer {l} (propagated K/V)"
                rep.bf16(f"k[{tag}]", kc[l, bidx, :, pos], ek, rk)
                rep.bf16(f"v[{tag}]", vc[l, bidx, :, pos], yv.reshape(R, s.Hkv, s.Dh),
                         bv.reshape(R, s.Hkv, s.Dh) + 2 * U32 * np.abs(yv.reshape(R, s.Hkv, s.Dh)))
            continue
        lw = layer_weights(l, use_exit)
        st = rec_layers[l]
        h_in = st["h_in"]
        h_next = rec_layers[l + 1]["h_in"] if l + 1 < last_run else h_out
        tag = f"layer {l} ({'exit' if use_exit else 'backbone'})"

        # RMSNorm -> q|k|v -> RoPE; q stored, k/v in the cache slot of layer l
        xr, fl = flip_size(ro.rmsnorm(h_in, lw["attn_norm"], s.eps))
        yq, bq = product(xr, lw["wq"], fl)
        yk, bk = product(xr, lw["wk"], fl)
        yv, bv = product(xr, lw["wv"], fl)
        eq, rq = rope_allowance(yq.reshape(R, s.Hq, s.Dh), bq.reshape(R, s.Hq, s.Dh), pos, s.Dh, s.theta)
        ek, rk = rope_allowance(yk.reshape(R, s.Hkv, s.Dh), bk.reshape(R, s.Hkv, s.Dh), pos, s.Dh, s.theta)
        rep.bf16(f"q[{tag}]", st["q"].reshape(R, s.Hq, s.Dh), eq, rq)
        gk = kc[l, bidx, :, pos]                              # [R, Hkv, D]
        gv = vc[l, bidx, :, pos]
        rep.bf16(f"k[{tag}]", gk, ek, rk)
        rep.bf16(f"v[{tag}]", gv, yv.reshape(R, s.Hkv, s.Dh),
                 bv.reshape(R, s.Hkv, s.Dh) + 2 * U32 * np.abs(yv.reshape(R, s.Hkv, s.Dh)))

        # causal GQA attention over the stored cache, from the stored q
        q = st["q"].reshape(R, s.Hq, s.Dh)
        scale = 1.0 / np.sqrt(s.Dh)
        eo = np.empty((R, s.Hq, s.Dh))
        bo = np.empty((R, s.Hq, s.Dh))
        for r in range(R):
            b, p = bidx[r], pos[r]
            keep = np.arange(p + 1)
            if strategy == "kv_mask":
                keep = keep[(keep >= start) | (np.asarray(pos_E)[:p + 1] > l)]
            for h in range(s.Hq):
                j = (h * s.Hkv) // s.Hq
                eo[r, h], bo[r, h] = attention_row(q[r, h], kc[l, b, j, keep], vc[l, b, j, keep], scale)
        rep.bf16(f"attn[{tag}]", st["attn"].reshape(R, s.Hq, s.Dh), eo, bo)

        # o projection + residual (fp32 stored)
        yo, bo2 = product(st["attn"], lw["wo"])
        e1 = h_in + yo
        rep.f32(f"h_mid[{tag}]", st["h_mid"], e1, bo2 + 2 * U32 * (np.abs(h_in) + np.abs(e1)))

        # RMSNorm -> gate|up -> SwiGLU (bf16 stored)
        xr2, fl2 = flip_size(ro.rmsnorm(st["h_mid"], lw["mlp_norm"], s.eps))
        g, bg = product(xr2, lw["w_gate"], fl2)
        up, bu = product(xr2, lw["w_up"], fl2)
        sig = 1.0 / (1.0 + np.exp(-g))
        si = g * sig
        eu = si * up
        dsi = sig * (1.0 + g * (1.0 - sig))
        buu = np.abs(up * dsi) * bg + np.abs(si) * bu + bg * bu + 6 * U32 * np.abs(eu)
        rep.bf16(f"u[{tag}]", st["u"], eu, buu)

        # down projection + residual
        yd, bd = product(st["u"], lw["w_down"])
        e2 = st["h_mid"] + yd
        rep.f32(f"h_out[{tag}]", h_next, e2, bd + 2 * U32 * (np.abs(st["h_mid"]) + np.abs(e2)))

        # exit test after backbone layers except the last
        if l < L - 1 and l < E and not forced:
            cos = ro.cosine_rows(h_in, h_next)
            m = float(cos.min())
            gm = float(trace[l])
            assert abs(gm - m) <= COS_TOL, f"{tag}: recorded min cos {gm} vs {m} from the stored states"
            exited = l == E - 1
            if exited and E != cap:
                assert m > tau - COS_TOL, f"{tag}: exited with min cos {m} <= tau {tau}"
            else:
                assert m <= tau + COS_TOL, f"{tag}: did not exit with min cos {m} > tau {tau}"
    if E < L and not forced:
        assert E >= 1 and (E - 1) < len(trace), f"exit layer E={E} without a test before it"

    # final RMSNorm + LM head on the last row of every sequence
    last = np.arange(B) * n + (n - 1)
    xr, fl = flip_size(ro.rmsnorm(h_out[last], final_norm, s.eps))
    el, bl = product(xr, w_lm, fl)
    bl = bl + 2 * U32 * np.abs(el)
    rep.f32("logits", logits, el, bl)
    for b in range(B):
        d = np.max(np.abs(logits[b] - el[b]))
        assert d <= LOGIT_BAR * np.std(el[b]), f"row {b}: max|dlogit| {d} > {LOGIT_BAR} * std"
        gi = int(nxt[b])
        assert gi == int(np.argmax(logits[b])), f"row {b}: next {gi} is not the argmax of the logits"
        assert el[b, gi] + bl[b, gi] >= np.max(el[b] - bl[b]), f"row {b}: next {gi} is not a possible argmax"
    return rep
