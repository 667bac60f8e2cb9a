"""Benchmark of the activation-sparse decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--headline-only]

Headline workload: the Llama-3-8B-shaped SwiGLU MLP (d_model 4096, d_ff 14336,
bf16 weights ~ N(0, 0.02^2)), batch 1, Student-t(3) decode tokens, thresholds
calibrated on 256 synthetic calibration vectors by the library's own GPU
calibration kernel, 50% sparsity on both the gate/up input and the down input.
A step is one decode token through L independent MLP layers (distinct 352 MB
weight buffers, so no layer is still resident in the 256 MB Infinity Cache when
it runs again).  value = achieved GB/s of active-row bytes (the weight rows of
surviving inputs only) over the whole sparse MLP.

Also reported, each with the fp64 CPU oracle timed on a bounded sample beside it:
the dense baseline (same kernels over every row), the dominant kernel's roofline
from HIP events recorded around it on its own stream, a sparsity sweep, and one
entry per hot-path step (calibration, threshold GEMV, top-k / rank blend, GLASS
local signal + static-mask MLP, MoE router + routed + shared experts, 16-token
batches on the matrix cores, the full decoder block, the small fp16 MLP).
Sub-benchmarks are timed as HIP-graph replays of sequences rotating over weight
copies (launch overhead excluded, caches not reused across a copy's uses).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

METRIC = "µs/layer and achieved HBM GB/s (active-row bytes) vs dense GEMV at 50% sparsity"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
SWEEP = (0.0, 0.25, 0.40, 0.50, 0.65)
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--sparsity", type=float, default=0.5)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--rows", default="", help="comma-separated row names to run (default: all)")
    ap.add_argument("--traffic-run", action="store_true",
                    help="counter run: a 256 MiB device copy (known bytes) then 16 headline sparse-MLP calls")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def r4(x):
    return None if x is None else round(float(x), 4)


# ============================================================================ helpers
class Ctx:
    def __init__(self, torch, asg, L, datagen, dev):
        self.torch, self.asg, self.L, self.datagen, self.dev = torch, asg, L, datagen, dev
        self.stream = torch.cuda.current_stream(dev).cuda_stream

    def graph_us(self, fn_list, reps=20, warmup=2):
        """Capture fn_list (callables issuing library calls) once into a HIP graph and
        time `reps` replays; returns microseconds per callable."""
        torch = self.torch
        for f in fn_list[:warmup]:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fn_list[:1]:
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s, capture_error_mode="relaxed"):
            for f in fn_list:
                f()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = self.L.HipEvent(), self.L.HipEvent()
        st = torch.cuda.current_stream().cuda_stream
        a.record(st)
        for _ in range(reps):
            g.replay()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_ms(b) * 1e3 / (reps * len(fn_list))


def cpu_time(fn, seconds, max_n=1000):
    n = 0
    t0 = time.perf_counter()
    while True:
        fn(n)
        n += 1
        el = time.perf_counter() - t0
        if el > seconds or n >= max_n:
            return el / n * 1e6, n, el


def cores():
    return len(os.sched_getaffinity(0))


# ============================================================================ headline
def headline(a, C):
    torch, asg, L, datagen, dev = C.torch, C.asg, C.L, C.datagen, C.dev
    shape = datagen.CFG2
    d, f = shape.d_model, shape.d_ff
    row_gu, row_d = 2 * f * 2, d * 2
    t0 = time.time()
    wgu, wd = datagen.mlp_weights_input_major(2, 0, shape)
    w0 = asg.MLPWeights(wgu.to(dev), wd.to(dev))
    del wgu, wd
    layers = [w0] + [asg.MLPWeights(w0.w_gate_up.clone(), w0.w_down.clone()) for _ in range(a.layers - 1)]
    calib = datagen.student_t((256, d), datagen.seed_for(2, 0, "calib")).to(dev)
    n_tok = 64
    toks = datagen.student_t((n_tok, d), datagen.seed_for(2, 0, "decode")).to(dev)
    torch.cuda.synchronize()
    log(f"llama mlp weights ready in {time.time() - t0:.1f}s ({a.layers} layers)")

    def calibrate(s):
        if s <= 0:
            return float("-inf"), float("-inf")
        t_x = float(asg.as_calibrate_threshold(calib, s).item())
        hs = []
        for b in range(0, 256, 16):
            _, dbg = asg.as_sparse_swiglu_mlp(calib[b:b + 16], w0, t_x, float("-inf"), debug=True)
            hs.append(dbg["h"].clone())
        t_h = float(asg.as_calibrate_threshold(torch.cat(hs), s).item())
        return t_x, t_h

    def active_bytes(t_x, t_h):
        out = []
        for i in range(n_tok):
            _, dbg = asg.as_sparse_swiglu_mlp(toks[i:i + 1], w0, t_x, t_h, debug=True)
            nx = int((toks[i].float().abs() > t_x).sum().item())
            nh = int((dbg["h"][0].abs() > t_h).sum().item())
            out.append((nx * row_gu, nh * row_d, nx, nh))
        return out

    def run(t_x, t_h, flags, steps, warmup, per_kernel):
        evs = [[L.HipEvent() for _ in range(3)] for _ in range(steps * a.layers)] if per_kernel else []
        Y = torch.empty((1, d), dtype=torch.float32, device=dev)
        warm = [asg.api.prepare_sparse_swiglu_mlp(toks[(s * a.layers + l) % n_tok], w, t_x, t_h, Y, flags=flags)
                for s in range(warmup) for l, w in enumerate(layers)]
        calls = [asg.api.prepare_sparse_swiglu_mlp(toks[(s * a.layers + l) % n_tok], w, t_x, t_h, Y, flags=flags,
                                                   events=evs[s * a.layers + l] if per_kernel else None)
                 for s in range(steps) for l, w in enumerate(layers)]
        for c in warm:
            c()
        torch.cuda.synchronize()
        e0, e1 = L.HipEvent(), L.HipEvent()
        e0.record(C.stream)
        for c in calls:
            c()
        e1.record(C.stream)
        torch.cuda.synchronize()
        total_ms = e0.elapsed_ms(e1)
        k1 = k2 = None
        if per_kernel:
            k1 = np.array([e[0].elapsed_ms(e[1]) for e in evs]) * 1e3
            k2 = np.array([e[1].elapsed_ms(e[2]) for e in evs]) * 1e3
        used = [(s * a.layers + l) % n_tok for s in range(steps) for l in range(a.layers)]
        return total_ms, k1, k2, used

    res = {}
    sweep = SWEEP if not a.no_sweep else (a.sparsity,)
    if a.sparsity not in sweep:
        sweep = tuple(sweep) + (a.sparsity,)
    for s in sweep:
        t_x, t_h = calibrate(s)
        ab = active_bytes(t_x, t_h)
        total_ms, _, _, used = run(t_x, t_h, a.flags, a.steps, a.warmup, per_kernel=False)
        calls = a.steps * a.layers
        bytes_tot = sum(ab[t][0] + ab[t][1] for t in used)
        r = dict(sparsity=s, t_x=t_x, t_h=t_h, us_per_layer=total_ms * 1e3 / calls,
                 gbs=bytes_tot / (total_ms * 1e-3) / 1e9,
                 realized_sparsity_x=1 - np.mean([ab[t][2] for t in used]) / d,
                 realized_sparsity_h=1 - np.mean([ab[t][3] for t in used]) / f,
                 active_mb_per_layer=bytes_tot / calls / 1e6, total_ms=total_ms)
        if abs(s - a.sparsity) < 1e-9:
            _, k1, k2, used_k = run(t_x, t_h, a.flags, a.steps, 2, per_kernel=True)
            b1 = np.array([ab[t][0] for t in used_k], dtype=np.float64)
            r["stage1_us"], r["stage2_us"] = float(k1.mean()), float(k2.mean())
            r["stage1_gbs"] = float(b1.sum() / (k1.sum() * 1e-6) / 1e9)
            r["stage1_bytes_per_launch"] = float(b1.mean())
            # the same step with the down stage's slices adding into Y atomically (no
            # deterministic combine); reported beside the headline, not as it
            at_ms, _, _, _ = run(t_x, t_h, a.flags | L.AS_FLAG_ATOMIC_SPLITK, a.steps, a.warmup, per_kernel=False)
            r["atomic_us_per_layer"] = at_ms * 1e3 / calls
            r["atomic_gbs"] = bytes_tot / (at_ms * 1e-3) / 1e9
        res[s] = r
        log(f"s={s:.2f} {r['us_per_layer']:.2f} us/layer {r['gbs']:.0f} GB/s (active {r['active_mb_per_layer']:.1f} MB)")
    dense_ms, _, _, _ = run(0.0, 0.0, a.flags | L.AS_FLAG_FORCE_DENSE, a.steps, a.warmup, per_kernel=False)
    _, dk1, dk2, _ = run(0.0, 0.0, a.flags | L.AS_FLAG_FORCE_DENSE, a.steps, 2, per_kernel=True)
    dense_us = dense_ms * 1e3 / (a.steps * a.layers)
    dense_at_ms, _, _, _ = run(0.0, 0.0, a.flags | L.AS_FLAG_FORCE_DENSE | L.AS_FLAG_ATOMIC_SPLITK, a.steps, a.warmup,
                               per_kernel=False)
    dense_at_us = dense_at_ms * 1e3 / (a.steps * a.layers)
    dense_bytes = d * row_gu + f * row_d
    log(f"dense {dense_us:.2f} us/layer {dense_bytes / (dense_us * 1e-6) / 1e9:.0f} GB/s")
    m = res[a.sparsity]
    out = {
        "metric": METRIC,
        "value": round(m["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(m["total_ms"] / a.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped SwiGLU MLP layer 4096->14336->4096, bf16 weights, batch 1, "
                               "Student-t(3) tokens, 50% sparsity on gate/up and down inputs",
                   "d_model": d, "d_ff": f, "weights": "bf16", "sparsity": a.sparsity,
                   "layers_per_step": a.layers, "tokens": n_tok},
        "us_per_layer": round(m["us_per_layer"], 3),
        "dense_us_per_layer": round(dense_us, 3),
        "dense_gbs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
        "speedup_vs_dense": round(dense_us / m["us_per_layer"], 3),
        "frac_of_peak_layer": round(m["gbs"] / PEAK_HBM_GBS, 4),
        "atomic_splitk": {"us_per_layer": round(m["atomic_us_per_layer"], 3), "gbs": round(m["atomic_gbs"], 1),
                          "dense_us_per_layer": round(dense_at_us, 3),
                          "speedup_vs_dense": round(dense_at_us / m["atomic_us_per_layer"], 3),
                          "note": "AS_FLAG_ATOMIC_SPLITK: down-stage slices add into fp32 Y with atomics "
                                  "(not bitwise reproducible); value above is the deterministic path"},
        "stage_us": {"gate_up": round(m["stage1_us"], 3), "down": round(m["stage2_us"], 3),
                     "dense_gate_up": round(float(dk1.mean()), 3), "dense_down": round(float(dk2.mean()), 3)},
        "roofline": {"bound": "hbm", "kernel": "gather_gemv_kernel: gate/up row gather (split-K partials left for the down prologue, which applies SwiGLU)",
                     "achieved": round(m["stage1_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(m["stage1_gbs"] / PEAK_HBM_GBS, 4),
                     "bytes_per_launch": m["stage1_bytes_per_launch"], "us_per_launch": round(m["stage1_us"], 3),
                     "traffic": traffic_from_profiles()},
        "sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in res[s].items()
                   if k in ("sparsity", "us_per_layer", "gbs", "realized_sparsity_x", "realized_sparsity_h",
                            "active_mb_per_layer")} for s in sorted(res)],
    }
    del layers, w0
    torch.cuda.empty_cache()
    return out, m["t_x"], m["t_h"]


def traffic_from_profiles():
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter runs,
    when they were taken on the current kernel sources (else null)."""
    p = os.path.join(HERE, "profiles", "gather_gemv_llama_mlp_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
        if rec.get("source_sha256") != kernel_source_hash():
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:
        return None


def kernel_source_hash():
    h = hashlib.sha256()
    for fn in ("gather_gemv_impl.hpp", "common.hpp"):
        h.update(open(os.path.join(HERE, "activation_sparse_gemv_amd", "csrc", fn), "rb").read())
    return h.hexdigest()


def cpu_baseline_headline(t_x, t_h, seconds):
    import torch
    from activation_sparse_gemv_amd import datagen
    from oracle import teal
    shape = datagen.CFG2
    wgu, wd = datagen.mlp_weights_input_major(2, 0, shape)
    Wg, Wu, Wd = (wgu[:, 0, :].to(torch.float64).numpy(), wgu[:, 1, :].to(torch.float64).numpy(),
                  wd.to(torch.float64).numpy())
    del wgu, wd
    toks = datagen.student_t((64, shape.d_model), datagen.seed_for(2, 0, "decode")).to(torch.float64).numpy()
    active = [0]

    def one(i):
        r = teal.swiglu_mlp_threshold(toks[i % 64], Wg, Wu, Wd, t_x, t_h)
        # the active-row bytes of this token, counted as the GPU path counts them (bf16 rows)
        active[0] += int(r["m1"].sum()) * 2 * shape.d_ff * 2 + int(r["m2"].sum()) * shape.d_model * 2

    us, n, el = cpu_time(one, seconds, max_n=100000)
    return {"value": round(active[0] / el / 1e9, 3), "unit": "GB/s", "cores": cores(), "kind": "oracle",
            "us_per_layer": round(us, 1),
            "sample": f"{n} decode tokens through one 4096->14336->4096 threshold MLP (fp64 numpy, same "
                      f"thresholds and tokens as the GPU run), {el:.1f} s; value = the active-row bytes "
                      f"(bf16 rows of the kept inputs) of those tokens per second; fp64 weight conversion "
                      f"not timed"}


# ============================================================================ per-row sub-benchmarks
def row_calibrate(C, cpu):
    torch, asg, datagen = C.torch, C.asg, C.datagen
    pool = datagen.student_t((256, 14336), 7001).to(C.dev)
    fns = [lambda: asg.as_calibrate_threshold(pool, 0.5) for _ in range(4)]
    us = C.graph_us(fns, reps=5)
    mb = pool.numel() * 2 / 1e6
    r = {"step": "a1 threshold calibration (nearest-rank order statistic, grid-wide 4-pass radix select)",
         "shape": "pool 256 x 14336 bf16", "us": r4(us), "pool_mb": mb,
         "gbs_4_passes": r4(4 * mb * 1e6 / (us * 1e-6) / 1e9),
         "note": "offline, once per model; four histogram launches over the pool and one select launch"}
    if cpu:
        from oracle import teal
        P = pool.cpu().to(torch.float64).numpy()
        cu, n, _ = cpu_time(lambda i: teal.calibrate_threshold(P, 0.5), 3.0, 20)
        r["cpu_oracle_us"], r["cpu_cores"] = r4(cu), cores()
    return r


def row_gemv(C, cpu):
    torch, asg, datagen = C.torch, C.asg, C.datagen
    out = []
    for K, N, tag in ((14336, 4096, "down-shaped 14336->4096"), (4096, 4096, "o-proj 4096->4096"),
                      (4096, 6144, "qkv 4096->6144")):
        W = [datagen.normal((K, N), 7100 + K + N).to(C.dev)]
        W += [W[0].clone() for _ in range(int(np.ceil(600e6 / (K * N * 2))))]
        calib = datagen.student_t((256, K), 7200 + K)
        x = datagen.student_t((16, K), 7300 + K).to(C.dev)
        t = float(asg.as_calibrate_threshold(calib.to(C.dev), 0.5).item())
        nnz = float((x.float().abs() > t).sum(dim=1).float().mean().item())
        Y = torch.empty((1, N), dtype=torch.float32, device=C.dev)
        fs = [lambda w=w, i=i: asg.as_threshold_gemv(x[i % 16], w, t, Y=Y) for i, w in enumerate(W * 2)]
        fd = [lambda w=w, i=i: asg.as_dense_gemv(x[i % 16], w, Y=Y) for i, w in enumerate(W * 2)]
        us, usd = C.graph_us(fs), C.graph_us(fd)
        ab = nnz * N * 2
        r = {"shape": tag, "sparsity": 0.5, "us": r4(us), "dense_us": r4(usd), "speedup": r4(usd / us),
             "active_mb": r4(ab / 1e6), "gbs": r4(ab / (us * 1e-6) / 1e9), "frac_hbm": r4(ab / (us * 1e-6) / 8e12),
             "dense_gbs": r4(K * N * 2 / (usd * 1e-6) / 1e9)}
        if cpu and K == 14336:
            from oracle import teal
            W64 = W[0].cpu().to(torch.float64).numpy()
            X64 = x.cpu().to(torch.float64).numpy()
            cu, n, _ = cpu_time(lambda i: teal.masked_gemv(X64[i % 16], W64, t), 3.0, 200)
            r["cpu_oracle_us"], r["cpu_cores"] = r4(cu), cores()
        out.append(r)
        del W
    return {"step": "a2+a3 fused mask/compaction + row-gather GEMV (split-K)", "cases": out}


def row_topk(C, cpu):
    torch, asg, datagen = C.torch, C.asg, C.datagen
    n, k = 14336, 7168
    loc = torch.from_numpy(np.abs(np.random.default_rng(1).standard_t(3, n)).astype(np.float32)).to(C.dev)
    prior = datagen.uniform01((n,), datagen.seed_for(4, 0, "prior")).to(C.dev)
    ub = C.graph_us([lambda: asg.as_topk_mask(loc, k, prior=prior, lam=0.5) for _ in range(4)])
    h = torch.from_numpy(np.abs(np.random.default_rng(2).standard_t(3, (128, 768))).astype(np.float32)).to(C.dev)
    uv = C.graph_us([lambda: asg.as_topk_mask(h, 77) for _ in range(4)])
    r = {"step": "a6 exact top-k (LDS radix select, index tie-break) and GLASS rank blend",
         "blend_n14336_k7168_us": r4(ub), "value_128rows_n768_k77_us": r4(uv),
         "note": "blend = two ordinal rankings (chunked counting, four values per thread) + LDS-staged radix select; once per prompt"}
    if cpu:
        from oracle import topk
        L64, P64 = loc.cpu().double().numpy(), prior.cpu().double().numpy()
        cu, _, _ = cpu_time(lambda i: topk.glass_topk(L64, P64, 0.5, k), 3.0, 100)
        H64 = h.cpu().double().numpy()
        cv, _, _ = cpu_time(lambda i: [topk.value_topk(H64[j], 77) for j in range(128)], 3.0, 100)
        r.update(cpu_oracle_blend_us=r4(cu), cpu_oracle_value_us=r4(cv), cpu_cores=cores())
    return r


def row_glass(C, cpu):
    torch, asg, L, datagen = C.torch, C.asg, C.L, C.datagen
    c = datagen.CFG4
    d, f, k = c["d_model"], c["d_ff"], c["keep"]
    W = datagen.mlp_weights_neuron_major(4, 0, d, f)
    Wd = W.to(C.dev)
    copies = [asg.MLPWeights(Wd, None, L.AS_MLP_NEURON_SET)] + \
             [asg.MLPWeights(Wd.clone(), None, L.AS_MLP_NEURON_SET) for _ in range(3)]
    prompt = datagen.student_t((c["prompt"], d), datagen.seed_for(4, 0, "prompt")).to(C.dev)
    prior = datagen.uniform01((f,), datagen.seed_for(4, 0, "prior")).to(C.dev)
    toks = datagen.student_t((16, d), datagen.seed_for(4, 0, "decode")).to(C.dev)
    u_loc = C.graph_us([lambda w=w: asg.as_glass_local_signal(prompt, w) for w in copies])
    loc = asg.as_glass_local_signal(prompt, copies[0])
    _, idx = asg.as_topk_mask(loc, k, prior=prior, lam=c["lam"])
    idx = idx.contiguous()
    Y = torch.empty((1, d), dtype=torch.float32, device=C.dev)
    fs = [lambda w=w, i=i: asg.as_sparse_swiglu_mlp(toks[i % 16], w, neuron_idx=idx, Y=Y)
          for i, w in enumerate(copies * 3)]
    fd = [lambda w=w, i=i: asg.as_sparse_swiglu_mlp(toks[i % 16], w, flags=L.AS_FLAG_FORCE_DENSE, Y=Y)
          for i, w in enumerate(copies * 3)]
    us, usd = C.graph_us(fs), C.graph_us(fd)
    ab = k * 3 * d * 2
    flops = 2 * c["prompt"] * d * 2 * f
    lw = 2 * f * d * 2
    r = {"step": "a7 GLASS static neuron set: local signal (MFMA prefill) + rank-blend top-k + neuron-set SwiGLU",
         "shape": "d_model 4096, d_ff 14336, keep 7168, bf16, batch 1",
         "decode_us": r4(us), "dense_us": r4(usd), "speedup": r4(usd / us), "active_mb": r4(ab / 1e6),
         "gbs": r4(ab / (us * 1e-6) / 1e9), "frac_hbm": r4(ab / (us * 1e-6) / 8e12),
         "local_signal_us_128_tokens": r4(u_loc),
         # 128 tokens: 128 flops per weight byte, below the bf16 ridge (~312), so the
         # weight stream (gate + up rows of every neuron) bounds it
         "local_signal_bound": "hbm",
         "local_signal_weight_mb": r4(lw / 1e6),
         "local_signal_gbs": r4(lw / (u_loc * 1e-6) / 1e9),
         "local_signal_frac_hbm": r4(lw / (u_loc * 1e-6) / 8e12),
         "local_signal_tflops": r4(flops / (u_loc * 1e-6) / 1e12),
         "local_signal_frac_mfma_bf16": r4(flops / (u_loc * 1e-6) / 1e12 / PEAK_BF16_TFLOPS)}
    if cpu:
        from oracle import glass
        Wg, Wu, Wdn = (W[:, j].to(torch.float64).numpy() for j in range(3))
        I = idx.cpu().numpy()
        T = toks.cpu().double().numpy()
        cu, _, _ = cpu_time(lambda i: glass.neuron_set_mlp(T[i % 16], Wg, Wu, Wdn, I), 4.0, 100)
        r.update(cpu_oracle_us=r4(cu), cpu_cores=cores())
    del copies, Wd
    torch.cuda.empty_cache()
    return r


class _LazyF64:
    """Index-on-demand fp64 view of a stacked bf16 expert tensor (oracle sample only)."""

    def __init__(self, t):
        self.t, self.c = t, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.c:
            self.c[e] = self.t[e].to("cpu").double().numpy()
        return self.c[e]


def row_moe(C, cpu):
    torch, asg, L, datagen = C.torch, C.asg, C.L, C.datagen
    c = datagen.CFG5
    w = datagen.moe_weights(5, 0, n_experts=c["n_experts"], d_model=c["d_model"], d_ff_e=c["d_ff_e"],
                            d_ff_shared=c["d_ff_shared"])
    d = c["d_model"]

    def mk(src):
        return asg.MoEWeights(src["w_gate_up"], src["w_down"], src["w_router"],
                              asg.MLPWeights(src["s_gate_up"], src["s_down"]))
    dev0 = {k: v.to(C.dev) for k, v in w.items()}
    copies = [mk(dev0)] + [mk({k: v.clone() for k, v in dev0.items()}) for _ in range(2)]
    cases = []
    for T in c["tokens"]:
        X = datagen.student_t((T, d), datagen.seed_for(5, T, "decode")).to(C.dev)
        fs = [lambda ww=ww: asg.moe_layer(X, ww, c["top"], c["keep"]) for ww in copies * 2]
        fd = [lambda ww=ww: asg.moe_layer(X, ww, c["top"], c["keep"], flags=L.AS_FLAG_FORCE_DENSE)
              for ww in copies * 2]
        fa = [lambda ww=ww: asg.moe_layer(X, ww, c["top"], c["keep"], flags=L.AS_FLAG_ATOMIC_SPLITK)
              for ww in copies * 2]
        us, usd = C.graph_us(fs, reps=10), C.graph_us(fd, reps=10)
        fda = [lambda ww=ww: asg.moe_layer(X, ww, c["top"], c["keep"],
                                           flags=L.AS_FLAG_FORCE_DENSE | L.AS_FLAG_ATOMIC_SPLITK)
               for ww in copies * 2]
        usa, usda = C.graph_us(fa, reps=10), C.graph_us(fda, reps=10)
        _, dbg = asg.moe_layer(X, copies[0], c["top"], c["keep"], debug=True)
        ids = dbg["ids"].cpu().numpy()
        touched = len(np.unique(ids))
        e_gu = c["d_ff_e"] * 2 * d * 2
        down_rows = sum(len(np.unique(np.concatenate([dbg["keep"][t, j].cpu().numpy()
                                                      for t in range(T) for j in range(c["top"])
                                                      if ids[t, j] == e]))) for e in np.unique(ids))
        ab = touched * e_gu + down_rows * d * 2 + (2 * d * c["d_ff_shared"] + c["d_ff_shared"] * d) * 2 + \
            d * c["n_experts"] * 2
        dense_b = touched * (e_gu + c["d_ff_e"] * d * 2) + (3 * d * c["d_ff_shared"]) * 2 + d * c["n_experts"] * 2
        cases.append({"tokens": T, "experts_touched": touched, "us": r4(us), "dense_us": r4(usd),
                      "speedup": r4(usd / us),
                      "atomic_splitk": {"us": r4(usa), "dense_us": r4(usda), "speedup": r4(usda / usa)},
                      "active_mb": r4(ab / 1e6), "dense_mb": r4(dense_b / 1e6),
                      "gbs": r4(ab / (us * 1e-6) / 1e9), "frac_hbm": r4(ab / (us * 1e-6) / 8e12)})
        log(f"moe T={T}: {us:.1f} us (dense {usd:.1f}); atomic split-K {usa:.1f} (dense {usda:.1f})")
    r = {"step": "a8+a9 MoE layer: router GEMV + top-8/softmax, dense shared expert, routed experts "
                 "(dense gate/up scoring, exact top-77 of 768, gathered down rows)",
         "shape": "128 experts, d_model 2048, d_ff_e 768, shared d_ff 4096, bf16", "cases": cases}
    if cpu:
        from oracle import moe as omoe
        ow = {"w_router": w["w_router"].double().numpy(), "w_gate_up": _LazyF64(w["w_gate_up"]),
              "w_down": _LazyF64(w["w_down"]), "s_gate_up": w["s_gate_up"].double().numpy(),
              "s_down": w["s_down"].double().numpy()}
        X1 = datagen.student_t((1, d), datagen.seed_for(5, 1, "decode")).double().numpy()
        omoe.moe_layer(X1, ow, c["top"], c["keep"])          # warm the lazy fp64 experts
        cu, _, _ = cpu_time(lambda i: omoe.moe_layer(X1, ow, c["top"], c["keep"]), 4.0, 100)
        r.update(cpu_oracle_us_T1=r4(cu), cpu_cores=cores())
    del copies, dev0
    torch.cuda.empty_cache()
    return r


def row_batch16(C, cpu, t_x, t_h):
    torch, asg, L, datagen = C.torch, C.asg, C.L, C.datagen
    shape = datagen.CFG2
    wgu, wd = datagen.mlp_weights_input_major(2, 0, shape)
    w0 = asg.MLPWeights(wgu.to(C.dev), wd.to(C.dev))
    copies = [w0] + [asg.MLPWeights(w0.w_gate_up.clone(), w0.w_down.clone()) for _ in range(3)]
    X = datagen.student_t((16, shape.d_model), datagen.seed_for(2, 2, "decode")).to(C.dev)
    Y = torch.empty((16, shape.d_model), dtype=torch.float32, device=C.dev)
    us = C.graph_us([lambda w=w: asg.as_sparse_swiglu_mlp(X, w, t_x, t_h, Y=Y) for w in copies * 2])
    usd = C.graph_us([lambda w=w: asg.as_sparse_swiglu_mlp(X, w, flags=L.AS_FLAG_FORCE_DENSE, Y=Y)
                      for w in copies * 2])
    usa = C.graph_us([lambda w=w: asg.as_sparse_swiglu_mlp(X, w, t_x, t_h, flags=L.AS_FLAG_ATOMIC_SPLITK, Y=Y)
                      for w in copies * 2])
    usda = C.graph_us([lambda w=w: asg.as_sparse_swiglu_mlp(X, w, flags=L.AS_FLAG_FORCE_DENSE | L.AS_FLAG_ATOMIC_SPLITK,
                                                            Y=Y) for w in copies * 2])
    _, dbg = asg.as_sparse_swiglu_mlp(X, w0, t_x, t_h, debug=True)
    ux = int((X.float().abs() > t_x).any(dim=0).sum().item())
    uh = int((dbg["h"].abs() > t_h).any(dim=0).sum().item())
    ab = ux * 2 * shape.d_ff * 2 + uh * shape.d_model * 2
    del copies, w0
    torch.cuda.empty_cache()
    return {"step": "a10 16-token batch on the matrix cores (MFMA gathered skinny GEMM), Llama MLP, 50% thresholds",
            "us": r4(us), "dense_us": r4(usd), "speedup": r4(usd / us),
            "atomic_splitk": {"us": r4(usa), "dense_us": r4(usda), "speedup": r4(usda / usa)},
            "union_rows_x": ux, "union_rows_h": uh, "active_mb": r4(ab / 1e6),
            "gbs": r4(ab / (us * 1e-6) / 1e9), "frac_hbm": r4(ab / (us * 1e-6) / 8e12),
            "note": "with per-token thresholds the union of active rows over 16 tokens covers nearly every row"}


def row_block(C, cpu):
    torch, asg, L, datagen = C.torch, C.asg, C.L, C.datagen
    from oracle import block as oblock, teal
    out = []
    for layer in (0, 31):
        s = datagen.cfg3_sparsity(layer)
        wqkv, wo = datagen.attn_weights(3, layer)
        wgu, wd = datagen.mlp_weights_input_major(3, layer, datagen.CFG2)
        kc, vc = datagen.kv_cache(3, layer)
        bw = asg.BlockWeights(wqkv.to(C.dev), wo.to(C.dev), asg.MLPWeights(wgu.to(C.dev), wd.to(C.dev)))
        bw2 = asg.BlockWeights(bw.w_qkv.clone(), bw.w_o.clone(),
                               asg.MLPWeights(bw.mlp.w_gate_up.clone(), bw.mlp.w_down.clone()))
        kcd, vcd = kc.to(C.dev), vc.to(C.dev)
        # thresholds: GPU calibration on 64 synthetic vectors, pools taken sequentially through the block
        calib = datagen.student_t((64, 4096), datagen.seed_for(3, layer, "calib")).to(C.dev)
        t = dict(qkv=float("-inf"), o=float("-inf"), gate_up=float("-inf"), down=float("-inf"))
        for key, pk in (("qkv", "xn"), ("o", "o"), ("gate_up", "xn2"), ("down", "h")):
            pool = torch.stack([asg.as_decoder_block(calib[i], bw, kcd, vcd, t, debug=True)[1][pk]
                                for i in range(64)])
            t[key] = float(asg.as_calibrate_threshold(pool, s).item())
        x = datagen.student_t((8, 4096), datagen.seed_for(3, layer, "decode")).to(C.dev)
        Y = torch.empty(4096, dtype=torch.float32, device=C.dev)
        fs = [lambda w=w, i=i: asg.as_decoder_block(x[i % 8], w, kcd, vcd, t, Y=Y) for i, w in enumerate([bw, bw2] * 3)]
        fd = [lambda w=w, i=i: asg.as_decoder_block(x[i % 8], w, kcd, vcd, t, flags=L.AS_FLAG_FORCE_DENSE, Y=Y)
              for i, w in enumerate([bw, bw2] * 3)]
        us, usd = C.graph_us(fs), C.graph_us(fd)
        # active bytes from the GPU's own intermediates of one token
        _, g = asg.as_decoder_block(x[0], bw, kcd, vcd, t, debug=True)
        nx = int((g["xn"].abs() > t["qkv"]).sum().item())
        no = int((g["o"].abs() > t["o"]).sum().item())
        nx2 = int((g["xn2"].abs() > t["gate_up"]).sum().item())
        nh = int((g["h"].abs() > t["down"]).sum().item())
        ab = (nx * 6144 + no * 4096 + nx2 * 2 * 14336 + nh * 4096) * 2 + 2 * kc.numel() * 2
        dense_b = (4096 * 6144 + 4096 * 4096 + 4096 * 28672 + 14336 * 4096) * 2 + 2 * kc.numel() * 2
        r = {"layer": layer, "sparsity": r4(s), "us": r4(us), "dense_us": r4(usd), "speedup": r4(usd / us),
             "active_mb_incl_kv": r4(ab / 1e6), "dense_mb": r4(dense_b / 1e6),
             "gbs": r4(ab / (us * 1e-6) / 1e9), "frac_hbm": r4(ab / (us * 1e-6) / 8e12)}
        if cpu:
            W = dict(wqkv=wqkv.double().numpy(), wo=wo.double().numpy(), wgu=wgu.double().numpy(),
                     wd=wd.double().numpy(), kc=kc.double().numpy(), vc=vc.double().numpy())
            X = x.cpu().double().numpy()
            to = dict(qkv=t["qkv"], o=t["o"], gu=t["gate_up"], d=t["down"])
            cu, _, _ = cpu_time(lambda i: oblock.decoder_block(X[i % 8], W["wqkv"], W["wo"], W["wgu"], W["wd"],
                                                               W["kc"], W["vc"], to), 4.0, 50)
            r.update(cpu_oracle_us=r4(cu), cpu_cores=cores())
            del W
        out.append(r)
        log(f"block layer {layer}: {us:.1f} us (dense {usd:.1f})")
        del bw, bw2
        torch.cuda.empty_cache()
    return {"step": "a11 decoder block (RMSNorm, thresholded qkv / o / MLP projections, dense GQA attention "
                    "over 2048 cached keys)", "shape": "Llama-3-8B block, 32/8 heads, bf16, batch 1",
            "cases": out, "model_step_estimate_us": r4(np.mean([c["us"] for c in out]) * 32)}


def row_small(C, cpu):
    torch, asg, L, datagen = C.torch, C.asg, C.L, C.datagen
    from oracle import teal
    shape = datagen.CFG1
    wgu, wd = datagen.mlp_weights_input_major(1, 0, shape)
    w = asg.MLPWeights(wgu.to(C.dev), wd.to(C.dev))
    calib = datagen.laplace((256, shape.d_model), datagen.seed_for(1, 0, "calib"), dtype="f16")
    t_x, t_h, _ = teal.calibrate_mlp(calib.double().numpy(), wgu[:, 0, :].double().numpy(),
                                     wgu[:, 1, :].double().numpy(), 0.5, 0.5)
    toks = datagen.laplace((64, shape.d_model), datagen.seed_for(1, 0, "decode"), dtype="f16").to(C.dev)
    Y = torch.empty((1, shape.d_model), dtype=torch.float32, device=C.dev)
    us = C.graph_us([lambda i=i: asg.as_sparse_swiglu_mlp(toks[i], w, float(t_x), float(t_h), Y=Y)
                     for i in range(16)])
    usd = C.graph_us([lambda i=i: asg.as_sparse_swiglu_mlp(toks[i], w, flags=L.AS_FLAG_FORCE_DENSE, Y=Y)
                      for i in range(16)])
    r = {"step": "small SwiGLU 512->2048->512, fp16 weights, 50%/50% (latency bound: 6.3 MB dense)",
         "us": r4(us), "dense_us": r4(usd), "speedup": r4(usd / us)}
    if cpu:
        Wg, Wu, Wd = (wgu[:, 0, :].double().numpy(), wgu[:, 1, :].double().numpy(), wd.double().numpy())
        T = toks.cpu().double().numpy()
        cu, _, _ = cpu_time(lambda i: teal.swiglu_mlp_threshold(T[i % 64], Wg, Wu, Wd, t_x, t_h), 2.0, 2000)
        r.update(cpu_oracle_us=r4(cu), cpu_cores=cores())
    return r


def traffic_run(C):
    """For rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes: one plain device copy of
    256 MiB (the counters' scale reference), then 16 sparse MLP calls of the headline
    workload rotating over 8 layer copies; prints the active bytes of each call."""
    torch, asg, datagen = C.torch, C.asg, C.datagen
    src = torch.empty(256 << 20, dtype=torch.uint8, device=C.dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    shape = datagen.CFG2
    d, f = shape.d_model, shape.d_ff
    wgu, wd = datagen.mlp_weights_input_major(2, 0, shape)
    w0 = asg.MLPWeights(wgu.to(C.dev), wd.to(C.dev))
    layers = [w0] + [asg.MLPWeights(w0.w_gate_up.clone(), w0.w_down.clone()) for _ in range(7)]
    calib = datagen.student_t((256, d), datagen.seed_for(2, 0, "calib")).to(C.dev)
    toks = datagen.student_t((64, d), datagen.seed_for(2, 0, "decode")).to(C.dev)
    t_x = float(asg.as_calibrate_threshold(calib, 0.5).item())
    hs = [asg.as_sparse_swiglu_mlp(calib[b:b + 16], w0, t_x, float("-inf"), debug=True)[1]["h"].clone()
          for b in range(0, 256, 16)]
    t_h = float(asg.as_calibrate_threshold(torch.cat(hs), 0.5).item())
    torch.cuda.synchronize()
    for i in range(16):
        y, dbg = asg.as_sparse_swiglu_mlp(toks[i], layers[i % 8], t_x, t_h, debug=True)
        torch.cuda.synchronize()
        nx = int((toks[i].float().abs() > t_x).sum().item())
        nh = int((dbg["h"][0].abs() > t_h).sum().item())
        print(json.dumps({"call": i, "gate_up_active_bytes": nx * 2 * f * 2, "down_active_bytes": nh * d * 2}),
              flush=True)
    print(json.dumps({"copy_bytes": src.numel(), "kernel_source_sha256": kernel_source_hash()}), flush=True)


# ============================================================================ main
def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding is described, not implemented)"}))
        sys.exit(2)
    import torch
    sys.path.insert(0, HERE)
    import activation_sparse_gemv_amd as asg
    from activation_sparse_gemv_amd import _lib as L
    from activation_sparse_gemv_amd import datagen
    L.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    C = Ctx(torch, asg, L, datagen, dev)
    if a.traffic_run:
        traffic_run(C)
        return
    out, t_x, t_h = headline(a, C)
    cpu = not a.no_cpu_baseline
    if not a.headline_only:
        rows = {}
        for name, fn in (("a1_calibrate", lambda: row_calibrate(C, cpu)), ("a2_a3_gemv", lambda: row_gemv(C, cpu)),
                         ("a6_topk", lambda: row_topk(C, cpu)), ("a7_glass", lambda: row_glass(C, cpu)),
                         ("a8_a9_moe", lambda: row_moe(C, cpu)),
                         ("a10_batch16_mfma", lambda: row_batch16(C, cpu, t_x, t_h)),
                         ("a11_block", lambda: row_block(C, cpu)), ("small_mlp_fp16", lambda: row_small(C, cpu))):
            if a.rows and name not in a.rows.split(","):
                continue
            t0 = time.time()
            rows[name] = fn()
            log(f"row {name} done in {time.time() - t0:.1f}s")
        out["rows"] = rows
    if cpu:
        out["cpu_baseline"] = cpu_baseline_headline(t_x, t_h, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
