"""Benchmark: GPTQ linear layers end to end on one MI355X.

Headline workload: the attention-projection layer -- W 4096 x 4096 bf16
~ N(0, 0.02), 262144 calibration tokens (128 x 2048) of low-rank + noise
activations with 1% outlier channels x20, 4-bit, group 128, block 128,
percdamp 0.01.  Synthetic, seeded; inputs are resident in HBM before timing
starts.

One step = the whole hot path: zero S, S += X^T X over all tokens, then
quantize the layer (H, dead fix, damping, R = chol(H^-1) upper, column loop
with lazy block updates, unpermute + pack), outputs in HBM.

Prints one JSON line.  `roofline` covers the dominant kernel (the statistics
call), timed live with HIP events on the stream the library launches on;
`phase_rooflines` covers the factorisation, the column chain and the lazy
update, from the library's own per-phase event tracing over extra steps;
`workloads` times the other layer shapes of the pages' workloads (one
line each, inputs resident); `cpu_baseline` is the float64 oracle on a
bounded sample of the headline layer on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 (matrix)
PEAK_FP64_TFLOPS = 78.6         # MI355X fp64
PEAK_HBM_GBS = 8000.0

METRIC = "seconds per linear layer (4096x4096, 262144 tok, 4-bit g128); % MFMA/HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=128 * 2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="token sample for the oracle's statistics")
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="row sample for the oracle's column loop")
    ap.add_argument("--workloads", default="all",
                    help="comma list of extra workloads to time (tiny, mlp_up, mlp_down, "
                         "large_attn, large_fc1, large_fc2, block), 'all' or 'none'")
    ap.add_argument("--phase", choices=("layer", "hessian"), default="layer",
                    help="'hessian' times only the statistics call (for counter passes)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB "
                         "(a plain copy kernel of known size for scaling HBM counters)")
    return ap.parse_args()


def kernel_source_hash(name):
    with open(os.path.join(ROOT, "post_weight_quantization_15_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(src_hash):
    """HBM bytes per launch of the statistics kernels from the committed
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "hessian_attn_proj_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def tensor_sha(t):
    import torch
    b = t.detach().contiguous().view(torch.uint8) if t.dtype != torch.uint8 else t
    return hashlib.sha256(b.cpu().numpy().tobytes()).hexdigest()


def host_info():
    import numpy
    import scipy
    info = {"affinity_cores": len(os.sched_getaffinity(0)),
            "numpy": numpy.__version__, "scipy": scipy.__version__,
            "python": platform.python_version()}
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{k: p.get(k) for k in ("internal_api", "num_threads", "version")}
                        for p in threadpool_info()]
    except Exception:       # noqa: BLE001
        info["blas"] = None
    try:
        with open("/proc/meminfo") as f:
            kb = int(f.readline().split()[1])
        info["host_ram_gib"] = round(kb / 2 ** 20, 1)
    except OSError:
        info["host_ram_gib"] = None
    return info


def cpu_baseline(W, X, params, n_tokens, cpu_tokens, cpu_rows):
    """The oracle as it stands, on a bounded sample, scaled to one layer."""
    import numpy as np
    import oracle as orc
    info = host_info()
    threads = [b.get("num_threads") or 1 for b in (info.get("blas") or [])] or [1]
    m, d = W.shape
    Xs = X[:cpu_tokens].float().cpu().numpy()
    t0 = time.perf_counter()
    S_part = orc.hessian_sum(Xs)
    t_stats_s = time.perf_counter() - t0
    t_stats = t_stats_s * (n_tokens / Xs.shape[0])
    S = S_part * (n_tokens / Xs.shape[0])       # stand-in statistics for timing
    t0 = time.perf_counter()
    H, perm, dead, damp = orc.prepare(S, n_tokens, params["percdamp"], params["act_order"])
    R, damp = orc.factor(H, damp)
    t_factor = time.perf_counter() - t0
    Wr = W[:cpu_rows].double().cpu().numpy()
    t0 = time.perf_counter()
    Wp = Wr.copy()
    Wp[:, dead] = 0.0
    Wp = Wp[:, perm]
    out = orc.quantize_columns(Wp, R, params["bits"], params["group_size"],
                               params["blocksize"],
                               orc.fit_grid(Wr, params["bits"]) if params["group_size"] == -1 else None)
    codes = np.empty_like(out["codes"])
    codes[:, perm] = out["codes"]
    orc.pack_codes(codes, params["bits"])
    t_loop_s = time.perf_counter() - t0
    t_loop = t_loop_s * (m / Wr.shape[0])
    total = t_stats + t_factor + t_loop
    return {"value": round(total, 3), "unit": "s per layer (extrapolated)",
            "cores": int(max(threads)), "kind": "oracle",
            "sample": (f"extrapolated: statistics measured on {Xs.shape[0]} of {n_tokens} tokens "
                       f"({t_stats_s:.2f} s) x{n_tokens / Xs.shape[0]:g}; factor at full d={d} "
                       f"({t_factor:.2f} s, measured); column loop + packing on {Wr.shape[0]} of {m} "
                       f"rows ({t_loop_s:.2f} s) x{m / Wr.shape[0]:g}"),
            "phases_s": {"stats": round(t_stats, 2), "factor": round(t_factor, 2),
                         "loop": round(t_loop, 2)},
            "host": info}


def time_layer(gq, torch, W, X, params, steps, warmup, shared=None):
    """Whole-path time of one layer (statistics + quantize), inputs resident."""
    dev = W.device
    m, d = W.shape
    N = X.shape[0]
    S = torch.zeros(d, d, dtype=torch.float32, device=dev)
    hws = torch.empty(max(gq.gptq_hessian_workspace_bytes(d, N), 1), dtype=torch.uint8, device=dev)
    qws = torch.empty(gq.gptq_workspace_bytes(m, d, **params), dtype=torch.uint8, device=dev)

    def step():
        S.zero_()
        gq.gptq_hessian_accumulate(S, X, ws=hws)
        return gq.gptq_quantize_layer(W, S, N, ws=qws, **params)

    return timed_and_traced(gq, torch, step, steps, warmup)


def timed_and_traced(gq, torch, step, steps, warmup):
    """Seconds per step over `steps` untraced steps after `warmup`, then one
    traced step for the per-phase split (milliseconds per phase)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    gq.gptq_trace_enable(True)
    gq.gptq_trace_read(reset=True)
    step()
    torch.cuda.synchronize()
    tr = gq.gptq_trace_read(reset=True)
    gq.gptq_trace_enable(False)
    return sec, {k: round(v[0], 3) for k, v in tr.items()}


def time_block(gq, torch, B, steps, warmup):
    """The decoder block's seven linears in order; q/k/v share one factor,
    gate/up another."""
    dev = B["q"]["W"].device
    p = B["q"]["params"]

    def stats(X):
        d = X.shape[1]
        S = torch.zeros(d, d, dtype=torch.float32, device=dev)
        gq.gptq_hessian_accumulate(S, X)
        return S

    def step():
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            X = B[names[0]]["X"]
            S = stats(X)
            if len(names) > 1:
                R, perm, dead, _ = gq.gptq_cholesky_inverse(S, X.shape[0], p["percdamp"],
                                                           p["act_order"])
                for nm in names:
                    gq.gptq_quantize_layer(B[nm]["W"], None, 0, R=R, perm=perm, dead=dead, **p)
            else:
                gq.gptq_quantize_layer(B[names[0]]["W"], S, X.shape[0], **p)

    return timed_and_traced(gq, torch, step, steps, warmup)


def workloads(gq, torch, synth, names, dev):
    """One timed line per extra workload (1 warm-up, 2 steps each)."""
    out = {}
    for name in names:
        t0 = time.perf_counter()
        if name == "tiny":
            L = synth.tiny_layer(dev)
            sec, ph = time_layer(gq, torch, L["W"], L["X"], L["params"], 2, 1)
            cfg = "tiny layer 128x256, 512 fp32 tokens, 4-bit per-row"
        elif name in ("mlp_up", "mlp_down"):
            P = synth.mlp_pair(dev)
            L = P[name.split("_")[1]]
            sec, ph = time_layer(gq, torch, L["W"], L["X"], L["params"], 2, 1)
            cfg = (f"MLP {name.split('_')[1]} {L['W'].shape[0]}x{L['W'].shape[1]}, "
                   "262144 tokens, 3-bit g128 act-order")
            del P
        elif name.startswith("large_"):
            which = name.split("_")[1]
            L = synth.large_model_layer(which, dev)
            sec, ph = time_layer(gq, torch, L["W"], L["X"], L["params"], 2, 1)
            cfg = f"d_model-12288 {which} {L['W'].shape[0]}x{L['W'].shape[1]}, 262144 tokens, 4-bit per-row"
        elif name == "block":
            B = synth.decoder_block(dev)
            sec, ph = time_block(gq, torch, B, 2, 1)
            cfg = ("decoder block: q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008, "
                   "131072 tokens, 2-bit g64 act-order (seven linears)")
            del B
        else:
            raise ValueError(name)
        out[name] = {"s": round(sec, 5), "config": cfg, "phases_traced_ms": ph,
                     "wall_s_incl_inputs": round(time.perf_counter() - t0, 1)}
        L = None
        torch.cuda.empty_cache()
        print(f"# workload {name}: {sec * 1e3:.2f} ms", file=sys.stderr, flush=True)
    return out


def _event_ms(torch, fn, reps):
    """Mean milliseconds of fn() over reps calls, HIP events on the current
    stream (the one the library launches on)."""
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def next_rows(gq, torch, synth, dev):
    """The rows after the core path, each timed: the dequantizing matmul
    against HBM (the packed weights are its traffic), the quantizer variants
    and the layer-by-layer driver on the attention-projection shape."""
    out = {}
    # ---- dequantizing matmul: fc1-shaped weights (49152 x 12288), random
    # codes (the kernel's time does not depend on their values)
    m, d, g = 49152, 12288, 128
    ng = d // g
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    dq = []
    for bits in (4, 3, 2):
        words = -(-d * bits // 32)
        qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (m, words), dtype=torch.int32,
                           device=dev, generator=gen)
        sc32 = torch.rand(m, ng, device=dev, generator=gen) * 0.01 + 0.001
        zp = torch.randint(0, 2 ** bits, (m, ng), dtype=torch.uint8, device=dev,
                           generator=gen)
        gi = (torch.arange(d, device=dev) // g).to(torch.int32)
        for n in (1, 8):
            X = torch.randn(n, d, device=dev, generator=gen).to(torch.bfloat16)
            Y = torch.empty(n, m, device=dev)
            for sc in (sc32, sc32.half()):
                ms = _event_ms(torch, lambda: gq.gptq_dequant_matmul(X, qw, sc, zp, gi, bits, g,
                                                                    Y=Y), 20)
                byts = (qw.numel() * 4 + sc.numel() * sc.element_size() + zp.numel() + gi.numel() * 4
                        + X.numel() * 2 + Y.numel() * 4)
                gbs = byts / (ms * 1e-3) / 1e9
                dq.append({"bits": bits, "tokens": n, "scales": str(sc.dtype).split(".")[-1],
                           "ms": round(ms, 4), "bytes": byts, "GB/s": round(gbs, 1),
                           "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        del qw, sc32, zp
    out["dequant_matmul"] = {"shape": f"{m}x{d} g{g}, bf16 activations, fp32 out",
                             "bound": "hbm", "peak_GB/s": PEAK_HBM_GBS, "runs": dq}
    torch.cuda.empty_cache()
    # ---- the same product at many activation rows (matrix cores): the
    # layer-by-layer driver's propagation shape, 65536 tokens x 4096 x 4096
    n, m, d = 65536, 4096, 4096
    X = torch.randn(n, d, device=dev, generator=gen).to(torch.bfloat16)
    Y = torch.empty(n, m, device=dev)
    gm = []
    for bits, g in ((4, 128), (4, -1), (2, 128), (8, 128)):
        ng = 1 if g == -1 else d // g
        qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (m, d * bits // 32), dtype=torch.int32,
                           device=dev, generator=gen)
        sc = torch.rand(m, ng, device=dev, generator=gen) * 0.01 + 0.001
        zp = torch.randint(0, 2 ** bits, (m, ng), dtype=torch.uint8, device=dev, generator=gen)
        gi = (torch.zeros(d, device=dev) if g == -1 else
              torch.arange(d, device=dev) // g).to(torch.int32)
        ms = _event_ms(torch, lambda: gq.gptq_dequant_matmul(X, qw, sc, zp, gi, bits, g, Y=Y), 3)
        tf = 2.0 * n * m * d / (ms * 1e-3) / 1e12
        gm.append({"bits": bits, "group_size": g, "ms": round(ms, 3), "TFLOP/s": round(tf, 1),
                   "frac_bf16": round(tf / PEAK_BF16_TFLOPS, 4)})
        del qw, sc, zp, gi
    out["dequant_gemm"] = {"shape": f"{n} tokens x {m}x{d}, bf16 activations, fp32 out",
                           "bound": "mfma", "peak_TFLOP/s": PEAK_BF16_TFLOPS, "runs": gm}
    del X, Y
    torch.cuda.empty_cache()
    # ---- quantizer variants on the attention-projection layer (S given)
    L = synth.attn_proj_layer(dev)
    W, X = L["W"], L["X"]
    n_tok = X.shape[0]
    S = torch.zeros(W.shape[1], W.shape[1], device=dev)
    gq.gptq_hessian_accumulate(S, X)
    base = dict(L["params"])
    var = {}
    for name, extra in (("minmax g128 (metric)", {}), ("symmetric g128", {"grid": "symmetric"}),
                        ("static g128 act-order", {"static_groups": True, "act_order": True}),
                        ("ternary g8", {"grid": "symmetric", "bits": 2, "group_size": 8}),
                        ("8-bit row", {"bits": 8, "group_size": -1})):
        p = dict(base, **extra)
        var[name] = round(_event_ms(torch, lambda: gq.gptq_quantize_layer(W, S, n_tok, **p), 3), 3)
    out["variants_quantize_ms"] = {"workload": "4096x4096, S of 262144 tokens given", **var}
    # ---- layer-by-layer driver: four 4096 x 4096 layers, ReLU between
    Ws = [W] + [synth.normal_weight(4096, 4096, 0.02, 8, f"stack/{i}", dev) for i in range(3)]
    Xs = X[:65536].contiguous()
    ms = _event_ms(torch, lambda: gq.gptq_quantize_stack(Ws, Xs, base, "relu"), 2)
    out["stack_driver"] = {"workload": "4 layers 4096x4096, 65536 tokens, 4-bit g128, ReLU",
                           "ms": round(ms, 3), "ms_per_layer": round(ms / 4, 3)}
    return out


def phase_rooflines(ph, m, d, N, bits, gsize, bsize):
    """Per-phase achieved rates against the published peaks, from the
    library's per-phase event tracing (milliseconds per layer)."""
    nb = -(-d // bsize)
    ng = 1 if gsize == -1 else -(-d // gsize)
    out = []
    f_ms = ph["factor"]
    out.append({"phase": "factor (fp64 reverse Cholesky + triangular inverse)",
                "bound": "mfma", "unit": "TFLOP/s", "peak": PEAK_FP64_TFLOPS,
                "algorithmic": f"2 d^3 / 3 = {2 * d ** 3 / 3:.4e} flop",
                "ms": round(f_ms, 4),
                "achieved": round(2 * d ** 3 / 3 / (f_ms * 1e-3) / 1e12, 2)})
    # the column chain's contract bytes: the fp32 working block read, E
    # written, the codes, R's diagonal blocks and the grids
    chain_bytes = m * d * (4 + 4) + m * d * bits / 8 + nb * 128 * 128 * 4 + m * ng * 5
    c_ms = ph["chain"]
    out.append({"phase": "column chain (in-block quantize + OBS feedback)",
                "bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
                "algorithmic": f"{chain_bytes:.4e} bytes (fp32 block in, E out, codes, R blocks, grids)",
                "ms": round(c_ms, 4),
                "achieved": round(chain_bytes / (c_ms * 1e-3) / 1e9, 1)})
    # the lazy kernels' share of m b^2 n_b (n_b - 1): the library updates the
    # tail once per batch of four blocks (K = 4b); the share of a batch's
    # later blocks in its own columns is applied inside the chain kernels
    kb = 4 * bsize
    lazy_flops = sum(2.0 * m * min(kb, d - s0) * max(0, d - s0 - kb)
                     for s0 in range(0, d, kb))
    l_ms = ph["lazy"]
    out.append({"phase": "lazy block update (fp32 MFMA)",
                "bound": "mfma", "unit": "TFLOP/s", "peak": PEAK_FP32_TFLOPS,
                "algorithmic": f"2 m K sum(d - i2) over batches of K = 4b = {kb} columns "
                               f"= {lazy_flops:.4e} flop (of m b^2 n_b (n_b - 1) = "
                               f"{2.0 * m * bsize * bsize * nb * (nb - 1) / 2.0:.4e}; the rest "
                               "runs in the chain kernels)",
                "ms": round(l_ms, 4),
                "achieved": round(lazy_flops / (l_ms * 1e-3) / 1e12, 2)})
    for o in out:
        o["frac"] = round(o["achieved"] / o["peak"], 4)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer "
              "path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch
    import post_weight_quantization_15_amd as gq
    import synth

    dev = torch.device("cuda:0")
    gq.load_library()
    L = synth.attn_proj_layer(dev, n=args.tokens)
    W, X, params = L["W"], L["X"], L["params"]
    m, d = W.shape
    N = X.shape[0]
    S = torch.zeros(d, d, dtype=torch.float32, device=dev)
    hws = torch.empty(max(gq.gptq_hessian_workspace_bytes(d, N), 1), dtype=torch.uint8, device=dev)
    qws = torch.empty(gq.gptq_workspace_bytes(m, d, **params), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        S.zero_()
        if ev:
            ev[0].record()
        gq.gptq_hessian_accumulate(S, X, ws=hws)
        if ev:
            ev[1].record()
        out = None
        if args.phase == "layer":
            out = gq.gptq_quantize_layer(W, S, N, ws=qws, **params)
        if ev:
            ev[2].record()
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if args.copy_probe_mib > 0:
        nb = args.copy_probe_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_step = elapsed * 1e3 / args.steps
    hess_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    quant_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    flops = float(N) * d * (d + 1)                 # symmetric X^T X
    achieved = flops / (hess_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(kernel_source_hash("k_hessian.hip"))
    roofline = {"kernel": "gptq_hessian_accumulate (bf16 MFMA split-K + fixed-order reduce)",
                "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic,
                "algorithmic": f"N*d*(d+1) = {flops:.4e} flop per launch"}
    line = {
        "metric": METRIC, "value": round(ms_step / 1e3, 6), "unit": "s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"attention-projection layer {m}x{d}, {N} tokens, "
                               f"{params['bits']}-bit g{params['group_size']}"
                               + ("" if args.phase == "layer" else " (statistics only)"),
                   "m": m, "d": d, "tokens": N, **params},
        "phases_ms": {"hessian": round(hess_ms, 4), "quantize": round(quant_ms, 4)},
        "roofline": roofline,
    }
    if args.phase == "layer":
        # per-phase times from the library's event tracing (extra steps, not
        # part of the headline timing)
        gq.gptq_trace_enable(True)
        gq.gptq_trace_read(reset=True)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        tr = gq.gptq_trace_read(reset=True)
        gq.gptq_trace_enable(False)
        ph = {k: v[0] / 2 for k, v in tr.items()}
        line["phases_traced_ms"] = {k: round(v, 4) for k, v in ph.items()}
        line["phase_rooflines"] = phase_rooflines(ph, m, d, N, params["bits"],
                                                  params["group_size"], params["blocksize"])
        line["inputs_sha256"] = {"W": tensor_sha(W), "X": tensor_sha(X)}
    names = ([] if args.workloads == "none" or args.phase != "layer" else
             ["tiny", "mlp_up", "mlp_down", "large_attn", "large_fc1", "large_fc2", "block"]
             if args.workloads == "all" else args.workloads.split(","))
    if names:
        del S, hws, qws
        Wc, Xc = W.cpu(), X.cpu()
        del L, W, X
        torch.cuda.empty_cache()
        line["workloads"] = workloads(gq, torch, synth, names, dev)
        line["next_rows"] = next_rows(gq, torch, synth, dev)
        W, X = Wc, Xc
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W, X, params, N, args.cpu_tokens, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
