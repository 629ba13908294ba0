#!/usr/bin/env python
"""Decode throughput of the KV-shared early-exit decoder on one MI355X.

One "step" is one token-level-exit decode step of the whole decoder (embedding,
every layer as backbone or exit layer, the exit test after each backbone
layer, LM head and argmax) for the batch, on synthetic seeded inputs resident
in HBM.  Default workload: the Llama-3.1-8B shape at batch 1 after a
512-token prompt, tau = 0.5.

Prints one JSON line with the throughput, a roofline object for the kernel
class that takes the most time (algorithmic bytes per launch over its mean
launch duration, timed with HIP events on the library's stream), and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s, 8B-shape KV-shared exit, τ=0.5; HBM GB/s as % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch decode steps without HIP graphs")
    ap.add_argument("--steps-per-launch", type=int, default=1,
                    help="decode steps per library call (river_decode_steps; with graphs, one "
                         "recorded graph of that many steps); 1 = one step per call")
    ap.add_argument("--tau-sweep", action="store_true",
                    help="instead of the benchmark line: for each tau of the workload (or --taus) "
                         "the exit histogram, decode tokens/s, the exit-decision share of the step, "
                         "exit/backbone layer time and exit/backbone K/V cosine, as one JSON line")
    ap.add_argument("--taus", type=str, default=None,
                    help="comma-separated taus for --tau-sweep and --kv-strategies")
    ap.add_argument("--kv-strategies", action="store_true",
                    help="instead of the benchmark line: decode tokens/s and exit histogram of the "
                         "method and of the four earlier K/V fixes it is compared with (kv mask, "
                         "state propagation, mono-decreasing exit, batching recompute) at each tau, "
                         "as one JSON line")
    ap.add_argument("--exit-mode", default="int4", choices=["int4", "hqq"],
                    help="exit bank of --tau-sweep: min-max int4, or int4 with the HQQ-style zero refinement")
    ap.add_argument("--offload-from", type=int, default=None,
                    help="backbone offloading: the linears of layers >= this one in pinned host "
                         "memory; prints decode tokens/s at --tau and with every layer on its "
                         "backbone, and the device bytes, as one JSON line")
    ap.add_argument("--exit-gemm-only", action="store_true",
                    help="run only the int4 exit-layer GEMMs at the batch-32 prefill shape (for "
                         "hardware-counter runs) and print their rate")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB three times (a plain "
                         "copy kernel of known size, to scale hardware byte counters)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# Algorithmic bytes per launch (what each kernel must move, nothing it avoids)
# ----------------------------------------------------------------------------
def linear_bytes(N, K, G, exit_int4):
    if exit_int4:
        return N * K // 2 + N * (K // G) * 4   # packed codes + bf16 scale/zero
    return N * K * 2


def kind_bytes(shape, B, kind, exit_path, ctx_len):
    s = shape
    d, F, G = s.d_model, s.ffn_dim, s.group_size
    qd, kd = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    if kind == "qkv":
        return (linear_bytes(qd + 2 * kd, d, G, exit_path) + B * d * 4 + B * (qd + 2 * kd) * 2)
    if kind == "attn":
        return B * kd * 2 * 2 * ctx_len + B * qd * 2 * 2
    if kind == "o":
        return linear_bytes(d, qd, G, exit_path) + B * qd * 2 + B * d * 4 * 2
    if kind == "gateup":
        return linear_bytes(2 * F, d, G, exit_path) + B * d * 4 + B * F * 2
    if kind == "down":
        return linear_bytes(d, F, G, exit_path) + B * F * 2 + B * d * 4 * 3
    if kind == "lm_head":
        return s.vocab * d * 2 + B * d * 4 + B * s.vocab * 4
    if kind == "begin":
        return B * d * 2 + B * d * 4
    return 0


def step_bytes(shape, B, E, ctx_len):
    tot = kind_bytes(shape, B, "begin", False, 0) + kind_bytes(shape, B, "lm_head", False, 0)
    for layer in range(shape.n_layers):
        ex = layer >= E
        for k in ("qkv", "attn", "o", "gateup", "down"):
            tot += kind_bytes(shape, B, k, ex, ctx_len)
    return tot


def mean_kind_bytes(shape, B, kind, hist, positions):
    """Mean algorithmic bytes per launch of `kind` over steps whose E values
    are given by `hist` (count per E) and whose context lengths are `positions`."""
    L = shape.n_layers
    steps = sum(hist)
    if steps == 0:
        return 0.0
    mean_ctx = sum(positions) / len(positions)
    if kind in ("lm_head", "begin"):
        return float(kind_bytes(shape, B, kind, False, mean_ctx))
    tot = 0.0
    for E, n in enumerate(hist):
        if n == 0:
            continue
        for layer in range(L):
            tot += n * kind_bytes(shape, B, kind, layer >= E, mean_ctx)
    return tot / (steps * L)


# ----------------------------------------------------------------------------
def cpu_baseline(shape, weights, B, T, mean_E):
    """The oracle, as it stands, on a bounded sample: one backbone layer, one
    exit layer (quantised by the oracle itself) and the LM head of the same
    workload, for one decode position after a T-token context; the step time is
    assembled as mean_E backbone layers + (L - mean_E) exit layers + LM head."""
    import numpy as np
    from oracle import river_oracle as ro
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    s = ro.Shape(**shape.as_dict())
    lw = {k: v.float().cpu().numpy() for k, v in weights["layers"][0].items()}
    ex = dict(lw)
    for name in ro.RiverOracle.LINEARS:
        q, sc, z = ro.quantize_int4(lw[name], s.G)
        ex[name] = ro.dequantize_int4(q, sc, z, s.G)
    lm = (weights["lm_head"] if weights["lm_head"] is not None else weights["embed"]).float().cpu().numpy()
    fn = weights["final_norm"].float().cpu().numpy()
    rng = np.random.default_rng(0)
    S = T + 1
    kc = ro.bf16_from_f64(rng.standard_normal((B, s.Hkv, S, s.Dh)))
    vc = ro.bf16_from_f64(rng.standard_normal((B, s.Hkv, S, s.Dh)))
    h = rng.standard_normal((B, 1, s.d)) * 0.5
    # the three pieces timed in turn until about 10 s of CPU work (at most 20
    # rounds), each piece's mean taken
    t_bb = t_ex = t_lm = 0.0
    rounds = 0
    while rounds < 20 and (rounds == 0 or t_bb + t_ex + t_lm < 10.0):
        t0 = time.perf_counter()
        ro.decoder_layer(s, lw, h, T, kc, vc)
        t_bb += time.perf_counter() - t0
        t0 = time.perf_counter()
        ro.decoder_layer(s, ex, h, T, kc, vc)
        t_ex += time.perf_counter() - t0
        t0 = time.perf_counter()
        ro.lm_head(s, h[:, -1], fn, lm)
        t_lm += time.perf_counter() - t0
        rounds += 1
    total = t_bb + t_ex + t_lm
    t_bb, t_ex, t_lm = t_bb / rounds, t_ex / rounds, t_lm / rounds
    step = mean_E * t_bb + (s.L - mean_E) * t_ex + t_lm
    return {
        "value": round(B / step, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"float64 numpy oracle, extrapolated: one decode position at context {T}; {rounds} rounds "
                   f"({total:.1f} s of CPU work) of 1 backbone layer (mean {t_bb:.2f} s), 1 int4 exit layer "
                   f"({t_ex:.2f} s) and the LM head ({t_lm:.2f} s); step = {mean_E:.2f} x backbone + "
                   f"{s.L - mean_E:.2f} x exit + LM head = {step:.2f} s; cores = the BLAS thread pool's size"),
    }


class DecodeLoop:
    """Greedy decode steps with the next tokens fed back on the device, `per`
    steps per library call (river_decode_steps: with graphs on, one recorded
    graph of `per` steps, so the graph launch is paid once per `per` steps);
    a remainder runs one step per call.  Next tokens land in two [per][B]
    buffers used in turn; a call reads its first tokens from the last row of
    the other buffer, so the calls hit the same two recorded graphs."""

    def __init__(self, r, B, vocab, dev, per):
        import torch
        self.r, self.per = r, max(1, int(per))
        self.ring = [torch.empty((self.per, B), dtype=torch.int32, device=dev) for _ in range(2)]
        self.logits = torch.empty((B, vocab), dtype=torch.float32, device=dev)
        self.cur = 0

    def start(self, first):
        """The tokens of the next step (e.g. the prefill's next tokens)."""
        self.ring[0][self.per - 1].copy_(first)
        self.cur = 0

    def run(self, n, tau):
        while n > 0:
            src, dst = self.ring[self.cur][self.per - 1], self.ring[1 - self.cur]
            if self.per > 1 and n >= self.per:
                self.r.decode_steps(src, self.per, tau, logits=self.logits, next_tok=dst)
                n -= self.per
            else:
                self.r.decode_step(src, tau, logits=self.logits, next_tok=dst[self.per - 1])
                n -= 1
            self.cur = 1 - self.cur


def timed_steps(r, loop, tau, W, K):
    """W warm-up and K timed decode steps (graph replays): seconds for the K
    and the histogram of E over the K."""
    import torch

    loop.run(W, tau)
    h0 = r.exit_stats()["decode_hist"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop.run(K, tau)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    h1 = r.exit_stats()["decode_hist"]
    return el, [a - b for a, b in zip(h1, h0)]


def kv_cosines(r, tokens, shape, n_rows):
    """Exit-layer K/V against backbone K/V for the same layer input: for each
    layer l a prefill with layers < l on the backbone and l.. on their exit
    copies (forced E = l) writes the exit layer's K/V for the input the
    backbone layers produced, compared with the all-backbone prefill's K/V of
    that layer.  Cosine per (layer, row, position) over all kv heads."""
    import torch
    L = shape.n_layers
    B, T = tokens.shape
    k, v = r.kv_views()

    def prefill_kv(e):
        r.force_exit_layer(e)
        r.reset()
        r.prefill(tokens, 0.5, want_logits=False)
        torch.cuda.synchronize()
        return k[:, :B, :, :T].float().clone(), v[:, :B, :, :T].float().clone()

    kb, vb = prefill_kv(L)
    per_layer = []
    for l in range(L):
        ke, ve = prefill_kv(l)
        cs = []
        for a, b in ((ke[l], kb[l]), (ve[l], vb[l])):
            a = a.permute(0, 2, 1, 3).reshape(B * T, -1)
            b = b.permute(0, 2, 1, 3).reshape(B * T, -1)
            cs.append(torch.nn.functional.cosine_similarity(a, b, dim=1))
        per_layer.append((float(cs[0].mean()), float(cs[0].min()), float(cs[1].mean()), float(cs[1].min())))
        del ke, ve
    r.force_exit_layer(-1)
    return {
        "k_mean": round(sum(x[0] for x in per_layer) / L, 5), "k_min": round(min(x[1] for x in per_layer), 5),
        "v_mean": round(sum(x[2] for x in per_layer) / L, 5), "v_min": round(min(x[3] for x in per_layer), 5),
        "per_layer_k_mean": [round(x[0], 5) for x in per_layer],
        "per_layer_v_mean": [round(x[2], 5) for x in per_layer],
        "rows_positions": f"{B} x {T}",
    }


def exit_gemm_rate(r, dev, reps=3):
    """The int4 exit GEMMs at the batch-32 prefill shape (32 x 1024 rows):
    each of layer 0's seven linears through the production prefill GEMM (plain
    fp32 output), timed with events after one warm-up call."""
    import torch
    M = 32 * 1024
    g = torch.Generator(device="cpu").manual_seed(7)
    flop = ms_tot = 0.0
    for li in range(7):
        N_, K_ = r.linear_shape(li)
        x = (torch.randn((M, K_), generator=g) * 0.5).to(torch.bfloat16).to(dev)
        r.debug_linear(0, li, 1, x)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            y = r.debug_linear(0, li, 1, x)
        ev1.record()
        torch.cuda.synchronize()
        ms_tot += ev0.elapsed_time(ev1) / reps
        flop += 2.0 * M * N_ * K_
        del x, y
    tf = flop / (ms_tot * 1e-3) / 1e12
    return {"rows": M, "total_ms": round(ms_tot, 3), "tflops": round(tf, 1),
            "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "what": "the 7 int4 exit-layer linears of one layer at 32 x 1024 rows "
                    "(batch-32 prefill shape), prefill GEMM with fp32 output, "
                    "2*M*N*K flop over their event time"}


def offload_measure(args):
    """Decode with the backbone linears of layers >= k in pinned host memory:
    tokens/s at tau (the exit copies in HBM serve the layers past the exit)
    and with every layer forced onto its backbone (E = L: every offloaded
    layer crosses the host link each step), plus device memory in use."""
    import torch
    import synth
    from early_exit_kv_amd import river as rv
    wl = synth.WORKLOADS[args.workload]
    shape, B, T = wl.shape, wl.batch, wl.prompt
    tau = 0.5 if args.tau is None else args.tau
    k, K, W = args.offload_from, args.steps, args.warmup
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.make_weights(shape, seed=0, device=dev)
    wo = rv.offload_layers(w, k)
    del w
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    tokens = synth.make_tokens(shape, B, T, seed=0).to(dev)
    r = rv.River(shape, wo, B, T + W + K + 8)
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    dev_bytes = torch.cuda.memory_allocated(dev)
    weights_dev = sum(t.numel() * 2 for t in r._all_weight_tensors() if t.is_cuda)
    weights_host = sum(t.numel() * 2 for t in r._all_weight_tensors() if not t.is_cuda)
    loop = DecodeLoop(r, B, shape.vocab, dev, args.steps_per_launch)
    out = {"what": "backbone offloading", "workload": wl.name, "offload_from_layer": k, "tau": tau,
           "device_weight_bytes": weights_dev, "host_weight_bytes": weights_host,
           "exit_bank_bytes": r.sizes.exit_bank_bytes, "kv_cache_bytes": r.sizes.kv_cache_bytes,
           "workspace_bytes": r.sizes.workspace_bytes, "torch_allocated_bytes": dev_bytes}
    for name, fe, n in (("decide", -1, K), ("all_backbone", shape.n_layers, max(2, K // 64))):
        r.force_exit_layer(fe)
        r.reset()
        _, nxt = r.prefill(tokens, tau, want_logits=False)
        loop.start(nxt)
        el, hist = timed_steps(r, loop, tau, min(W, n), n)
        out[name] = {"steps": n, "decode_tok_s": round(B * n / el, 3), "ms_per_step": round(el / n * 1e3, 3),
                     "exit_hist": {str(e): c for e, c in enumerate(hist) if c}}
        print(f"[offload] {name}: {out[name]}", file=sys.stderr, flush=True)
    r.force_exit_layer(-1)
    r.close()
    print(json.dumps(out))


def tau_sweep(args):
    """Per tau: exit histogram, decode tokens/s; then the exit-decision share
    of the step, exit/backbone layer time and exit/backbone K/V cosine."""
    import torch
    import synth
    from early_exit_kv_amd import river as rv

    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    B, T = wl.batch, wl.prompt
    taus = [float(t) for t in args.taus.split(",")] if args.taus else list(wl.taus)
    K, W = args.steps, args.warmup
    L = shape.n_layers
    print(f"[sweep] workload {wl.name} B={B} T={T} steps={K} warmup={W} taus={taus}", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    weights = synth.make_weights(shape, seed=0, device=dev)
    tokens = synth.make_tokens(shape, B, T, seed=0).to(dev)
    r = rv.River(shape, weights, B, T + W + K + 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r.build_exit_layers(args.exit_mode)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0
    loop = DecodeLoop(r, B, shape.vocab, dev, args.steps_per_launch)
    r.prefill(tokens, taus[0], want_logits=False)   # untimed: first launches load code
    torch.cuda.synchronize()
    rows = []
    for tau in taus:
        r.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, nxt = r.prefill(tokens, tau, want_logits=False)
        torch.cuda.synchronize()
        prefill_s = time.perf_counter() - t0
        pE = r.exit_stats()["last_E"]
        loop.start(nxt)
        el, hist_all = timed_steps(r, loop, tau, W, K)
        mean_E = sum(e * n for e, n in enumerate(hist_all)) / max(1, sum(hist_all))
        pos = T + W + K / 2
        byts = sum(n * step_bytes(shape, B, e, pos) for e, n in enumerate(hist_all)) / max(1, sum(hist_all))
        rows.append({"tau": tau, "prefill_E": pE, "prefill_tok_s": round(B * T / prefill_s, 1),
                     "decode_tok_s": round(B * K / el, 2), "ms_per_step": round(el / K * 1e3, 4),
                     "exit_hist": {str(e): n for e, n in enumerate(hist_all) if n},
                     "mean_exit_layer": round(mean_E, 3),
                     "step_hbm_frac": round(byts / (el / K) / 1e9 / HBM_PEAK_GBS, 4)})
        print(f"[sweep] tau={tau}: {rows[-1]}", file=sys.stderr, flush=True)

    # X6: the exit decision's share of a step: the same steps with the
    # decision fixed on the host at the E the device took (no test, no flag
    # reads) against the steps that decide on the device
    ref = rows[len(rows) // 2]
    E_ref = max(ref["exit_hist"], key=lambda e: ref["exit_hist"][e])
    tau_ref = ref["tau"]
    x6 = {}
    for name, fe in (("device_decision", -1), ("forced_same_E", int(E_ref))):
        r.force_exit_layer(fe)
        r.reset()
        _, nxt = r.prefill(tokens, tau_ref, want_logits=False)
        loop.start(nxt)
        x6[name + "_ms"] = round(timed_steps(r, loop, tau_ref, W, K)[0] / K * 1e3, 4)
    r.force_exit_layer(-1)
    x6["tau"] = tau_ref
    x6["E"] = int(E_ref)
    x6["share"] = round((x6["device_decision_ms"] - x6["forced_same_E_ms"]) / x6["device_decision_ms"], 5)

    # X7: per-layer time of the backbone layer against the exit layer, from
    # the per-class kernel times with every layer forced to one form
    x7 = {}
    r.reset()
    r.prefill(tokens, 0.5, want_logits=False)
    for name, fe in (("backbone_layer_us", L), ("exit_layer_us", 0)):
        r.force_exit_layer(fe)
        x7[name] = round(sum(r.time_kernel(k, reps=10) for k in ("qkv", "attn", "o", "gateup", "down")), 3)
    r.force_exit_layer(-1)
    x7["ratio"] = round(x7["backbone_layer_us"] / x7["exit_layer_us"], 3)
    d, F, G = shape.d_model, shape.ffn_dim, shape.group_size
    qd, kd = shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
    nk = [(qd + 2 * kd, d), (d, qd), (2 * F, d), (d, F)]
    x7["byte_ratio"] = round(sum(linear_bytes(n, k, G, False) for n, k in nk) /
                             sum(linear_bytes(n, k, G, True) for n, k in nk), 3)

    # X8: exit-layer K/V against backbone K/V for the same layer input
    Tk = min(T, 128)
    x8 = kv_cosines(r, tokens[:, :Tk].contiguous(), shape, B)
    r.close()
    out = {"what": "tau sweep", "workload": wl.name, "exit_mode": args.exit_mode,
           "build_exit_layers_s": round(build_s, 4), "batch": B, "prompt": T, "steps": K, "warmup": W,
           "config": f"decoder L={L} d={d} {shape.n_q_heads}q/{shape.n_kv_heads}kv heads x {shape.head_dim} "
                     f"FFN {F} vocab {shape.vocab}, int4 g{G} exit layers",
           "sweep": rows, "x6_exit_decision": x6, "x7_layer_time": x7, "x8_kv_cosine": x8}
    print(json.dumps(out))


def strategy_sweep(args):
    """Per tau and per K/V strategy of the layers past the exit: decode
    tokens/s, the exit histogram and the mean exit layer."""
    import torch
    import synth
    from early_exit_kv_amd import river as rv

    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    B, T = wl.batch, wl.prompt
    taus = [float(t) for t in args.taus.split(",")] if args.taus else list(wl.taus)
    K, W = args.steps, args.warmup
    print(f"[strategies] workload {wl.name} B={B} T={T} steps={K} warmup={W} taus={taus}", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    weights = synth.make_weights(shape, seed=0, device=dev)
    tokens = synth.make_tokens(shape, B, T, seed=0).to(dev)
    r = rv.River(shape, weights, B, T + W + K + 2)
    r.build_exit_layers("int4")
    # one step per call for every strategy: the recompute comparator sizes
    # each step's launches on the host, and the others are timed alike
    loop = DecodeLoop(r, B, shape.vocab, dev, 1)
    rows = []
    for tau in taus:
        for strategy in rv.KV_STRATEGIES:
            r.kv_strategy(strategy)
            r.reset()
            _, nxt = r.prefill(tokens, tau, want_logits=False)
            pE = r.exit_stats()["last_E"]
            loop.start(nxt)
            el, hist = timed_steps(r, loop, tau, W, K)
            mean_E = sum(e * n for e, n in enumerate(hist)) / max(1, sum(hist))
            row = {"tau": tau, "strategy": strategy, "prefill_E": pE,
                   "decode_tok_s": round(B * K / el, 2), "ms_per_step": round(el / K * 1e3, 4),
                   "exit_hist": {str(e): n for e, n in enumerate(hist) if n},
                   "mean_exit_layer": round(mean_E, 3)}
            if strategy == "recompute":
                row["launch"] = "eager, exit layer read back after every step"
            else:
                # the same steps launched eagerly (the recompute comparator's mode)
                r.use_graph(False)
                r.reset()
                _, nxt = r.prefill(tokens, tau, want_logits=False)
                loop.start(nxt)
                el2, _ = timed_steps(r, loop, tau, W, K)
                r.use_graph(True)
                row["launch"] = "graph"
                row["decode_tok_s_eager"] = round(B * K / el2, 2)
            rows.append(row)
            print(f"[strategies] {rows[-1]}", file=sys.stderr, flush=True)
    r.close()
    print(json.dumps({"what": "K/V strategies past the exit", "workload": wl.name, "batch": B, "prompt": T,
                      "steps": K, "warmup": W, "rows": rows}))


def main():
    args = parse()
    if args.kv_strategies:
        if args.gpus != 1:
            print("the strategy sweep runs on one GPU", file=sys.stderr)
            sys.exit(2)
        strategy_sweep(args)
        return
    if args.tau_sweep:
        if args.gpus != 1:
            print("the tau sweep runs on one GPU", file=sys.stderr)
            sys.exit(2)
        tau_sweep(args)
        return
    if args.offload_from is not None:
        offload_measure(args)
        return
    if args.exit_gemm_only:
        import torch
        import synth
        from early_exit_kv_amd import river as rv
        dev = torch.device("cuda:0")
        shape = synth.LLAMA_8B
        w1 = synth.make_weights(shape, seed=0, device=dev, n_layers=1)
        r = rv.River(synth.shrink(shape, n_layers=1), w1, 1, 8)
        r.build_exit_layers("int4")
        print(json.dumps({"exit_gemm_b32": exit_gemm_rate(r, dev)}))
        r.close()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path runs on a single GPU; sharding across GPUs is designed, not built).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from early_exit_kv_amd import river as rv

    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    B, T = wl.batch, wl.prompt
    tau = args.tau if args.tau is not None else wl.taus[len(wl.taus) // 2 if len(wl.taus) > 1 else 0]
    if args.workload == "8b":
        tau = 0.5 if args.tau is None else args.tau
    K, W = args.steps, args.warmup
    max_seq = T + W + K + 2   # + the profiled step and the slot kernel timing writes
    print(f"[bench] workload {wl.name} B={B} T={T} steps={K} warmup={W} tau={tau}", file=sys.stderr,
          flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    weights = synth.make_weights(shape, seed=0, device=dev)
    tokens = synth.make_tokens(shape, B, T, seed=0).to(dev)
    r = rv.River(shape, weights, B, max_seq)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r.build_exit_layers("int4")
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t0

    # one untimed prefill first (the first launch of each kernel loads its
    # code), then the timed one from a reset cache
    r.prefill(tokens, tau, want_logits=False)
    torch.cuda.synchronize()
    r.reset()
    t0 = time.perf_counter()
    _, nxt = r.prefill(tokens, tau, want_logits=False)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    st0 = r.exit_stats()
    prefill_E = st0["last_E"]

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    r.use_graph(not args.eager)

    loop = DecodeLoop(r, B, shape.vocab, dev, args.steps_per_launch)
    loop.start(nxt)

    def run(n):
        loop.run(n, tau)

    run(W)
    torch.cuda.synchronize()
    hist0 = r.exit_stats()["decode_hist"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(K)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    hist1 = r.exit_stats()["decode_hist"]
    hist = [a - b for a, b in zip(hist1, hist0)]
    mean_E = sum(e * n for e, n in enumerate(hist)) / max(1, sum(hist))
    positions = [T + W + i + 1 for i in range(K)]
    tok_s = B * K / elapsed
    ms_step = elapsed / K * 1e3
    avg_step_bytes = sum(n * step_bytes(shape, B, e, sum(positions) / K) for e, n in enumerate(hist)) / K
    step_gbs = avg_step_bytes / (elapsed / K) / 1e9

    # the same decode steps with the decision fixed: E = L is the original
    # model (every layer on its backbone), E = 0 the statically quantised one
    # (every layer on its int4 copy); the pages report River against both
    baselines = None
    if not args.no_baselines:
        baselines = {}
        for name, e in (("original", shape.n_layers), ("full_int4", 0)):
            r.force_exit_layer(e)
            r.reset()
            _, nxt_b = r.prefill(tokens, tau, want_logits=False)
            loop.start(nxt_b)
            run(W)                         # same positions as the timed River steps
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run(K)
            torch.cuda.synchronize()
            baselines[name] = round(B * K / (time.perf_counter() - t0), 2)
        r.force_exit_layer(-1)
        r.reset()
        _, nxt_b = r.prefill(tokens, tau, want_logits=False)
        loop.start(nxt_b)
        run(W + K)                         # back to the state the profiling below expects
        baselines["river_vs_original"] = round(tok_s / baselines["original"], 3)
        baselines["river_vs_full_int4"] = round(tok_s / baselines["full_int4"], 3)

    roofline = None
    kinds = {}
    if not args.no_profile:
        # Layer kernels: each class launched back to back for all layers from a
        # replayed graph, with the exit mix of the timed steps (force_E = the
        # E they took), timed by events around the replays on the library's
        # stream.  LM head and begin: one eager step with events around each
        # kernel (a single launch per step, so the gap in front is included).
        E_mix = max(range(len(hist)), key=lambda e: hist[e])
        mix = [0] * len(hist)
        mix[E_mix] = 1
        r.force_exit_layer(E_mix)
        for kind in ("qkv", "attn", "o", "gateup", "down"):
            avg_us = r.time_kernel(kind, reps=20)
            mb = mean_kind_bytes(shape, B, kind, mix, [T + W + K + 1])
            kinds[kind] = {"launches_per_step": shape.n_layers, "avg_us": round(avg_us, 3),
                           "avg_bytes": int(mb), "gbs": round(mb / (avg_us * 1e-6) / 1e9, 1),
                           "timing": "graph replay, back to back"}
        r.force_exit_layer(-1)
        r.profile(True)
        r.profile_read()
        run(1)
        times = r.profile_read()
        r.profile(False)
        for kind in ("begin", "lm_head"):
            n, ms = times[kind]
            mb = mean_kind_bytes(shape, B, kind, hist, positions)
            avg_us = ms / max(n, 1) * 1e3
            kinds[kind] = {"launches_per_step": 1, "avg_us": round(avg_us, 3), "avg_bytes": int(mb),
                           "gbs": round(mb / (avg_us * 1e-6) / 1e9, 1), "timing": "eager, events around"}
        dom = max(kinds, key=lambda k: kinds[k]["avg_us"] * kinds[k]["launches_per_step"])
        dk = kinds[dom]
        achieved = dk["avg_bytes"] / (dk["avg_us"] * 1e-6) / 1e9
        from early_exit_kv_amd.profiling import load_traffic
        traffic = load_traffic(os.path.join(ROOT, "profiles", f"{dom}_{wl.name}_traffic.json"))
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": None if traffic is None else int(traffic),
                    "kernel": dom, "algorithmic_bytes": dk["avg_bytes"], "avg_us": dk["avg_us"]}

    prefill_gemm = None
    if not args.no_profile:
        # prefill GEMMs with every layer on its exit copy (forced E = 0): the
        # int4-dequant MFMA GEMMs at M = B*T rows, timed with events
        r.reset()
        r.force_exit_layer(0)
        r.profile(True)
        r.profile_read()
        r.prefill(tokens, tau, want_logits=False)
        times = r.profile_read()
        r.profile(False)
        r.force_exit_layer(-1)
        n, ms = times["p_gemm"]
        s_ = shape
        qd, kd = s_.n_q_heads * s_.head_dim, s_.n_kv_heads * s_.head_dim
        nk = ((qd + 2 * kd) * s_.d_model + s_.d_model * qd + 2 * s_.ffn_dim * s_.d_model
              + s_.d_model * s_.ffn_dim)
        flop = 2.0 * B * T * nk * s_.n_layers
        tflops = flop / (ms * 1e-3) / 1e12
        prefill_gemm = {"rows": B * T, "launches": n, "total_ms": round(ms, 3),
                        "tflops": round(tflops, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                        "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                        "what": "all q|k|v, o, gate|up, down GEMMs of a prefill with every layer on "
                                "its int4 exit copy (forced E=0), 2*M*N*K flop over their event time"}

    exit_gemm_b32 = None
    if not args.no_profile and shape.d_model >= 2048:
        exit_gemm_b32 = exit_gemm_rate(r, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, weights, B, T, mean_E)

    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) weights, uniform tokens)",
        "config": {"workload": f"{wl.name}: decoder L={shape.n_layers} d={shape.d_model} "
                               f"{shape.n_q_heads}q/{shape.n_kv_heads}kv heads x {shape.head_dim} "
                               f"FFN {shape.ffn_dim} vocab {shape.vocab}",
                   "batch": B, "prompt": T, "tau": tau, "exit_layers": "int4 g%d" % shape.group_size,
                   "graphs": not args.eager, "steps_per_launch": args.steps_per_launch},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_hbm_gbs": round(step_gbs, 1), "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "mean_exit_layer": round(mean_E, 3), "exit_hist": {str(e): n for e, n in enumerate(hist) if n},
        "prefill_tok_s": round(B * T / prefill_s, 1), "prefill_E": prefill_E,
        "build_exit_layers_s": round(build_s, 4), "kernels": kinds, "prefill_exit_gemm": prefill_gemm,
        "exit_gemm_b32": exit_gemm_b32,
        "baselines_tok_s": baselines,
    }
    r.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
