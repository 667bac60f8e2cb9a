"""Phase timelines of the one-token sparse SwiGLU MLP (Llama-3-8B shape) and of
the decode attention (n_ctx 2048, 32 query / 8 kv heads).

    python -m activation_sparse_gemv_amd.build --timeline
    python -m activation_sparse_gemv_amd.timeline [--sparsity 0.5] [--reps 8] [--out FILE]
    python -m activation_sparse_gemv_amd.timeline --attention [--reps 8] [--out FILE]

Loads libactsparse_timeline.so (the opt-in build whose kernels write the device's
100 MHz clock at phase boundaries, include/actsparse_timeline.h) instead of
libactsparse.so, runs the 4096 -> 14336 -> 4096 bf16 MLP at batch 1 over eight
rotating weight copies (2.8 GB, beyond the 256 MB last-level cache), and prints,
per launch, the distribution over workgroups of each phase: the fused
mask-and-gather design of the TEAL slides (slide 11) split into what a workgroup
waits for and what it streams.  The stamps add a few instructions per phase; the
layer time of this build is printed beside the table for comparison with the
product library.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import _lib as L

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_TL = os.path.join(PKG, "libactsparse_timeline.so")
TICK_US = 0.01          # s_memrealtime: 100 MHz

GU_PHASES = [
    ("start after the first workgroup", lambda g, t0: g[:, 0] - t0),
    ("x arrived (load of the whole input)", lambda g, t0: g[:, 8] - g[:, 0]),
    ("mask scan over the input", lambda g, t0: g[:, 9] - g[:, 8]),
    ("split points of the list", lambda g, t0: g[:, 11] - g[:, 9]),
    ("row list written (thread 0's wave)", lambda g, t0: g[:, 12] - g[:, 11]),
    ("barrier after the list", lambda g, t0: g[:, 13] - g[:, 12]),
    ("second barrier (prologue end)", lambda g, t0: g[:, 1] - g[:, 13]),
    ("main loop (row gather)", lambda g, t0: g[:, 2] - g[:, 1]),
    ("slot reduction", lambda g, t0: g[:, 3] - g[:, 2]),
    ("partial tile stored", lambda g, t0: g[:, 4] - g[:, 3]),
    ("end", lambda g, t0: g[:, 4] - t0),
]
DN_PHASES = [
    ("start after the first gate/up workgroup", lambda d, t0: d[:, 0] - t0),
    ("gate/up partials arrived", lambda d, t0: d[:, 8] - d[:, 0]),
    ("sum + SwiGLU staged in LDS", lambda d, t0: d[:, 9] - d[:, 8]),
    ("h exports", lambda d, t0: d[:, 10] - d[:, 9]),
    ("mask + row list in LDS", lambda d, t0: d[:, 1] - d[:, 10]),
    ("main loop (row gather)", lambda d, t0: d[:, 2] - d[:, 1]),
    ("slot reduction", lambda d, t0: d[:, 3] - d[:, 2]),
    ("partial tile stored", lambda d, t0: d[:, 4] - d[:, 3]),
    ("tile counter", lambda d, t0: d[:, 5] - d[:, 4]),
    ("end (counter returned)", lambda d, t0: d[:, 5] - t0),
]


def _stats(x):
    x = np.asarray(x, dtype=np.float64) * TICK_US
    return np.median(x), np.percentile(x, 10), np.percentile(x, 90), x.max()


def summarize(runs):
    """runs: list of (gate/up stamps [G1, 16], down stamps [G2, 16]) of single calls."""
    rows_gu = {k: [] for k, _ in GU_PHASES}
    rows_dn = {k: [] for k, _ in DN_PHASES}
    extra = {"gap": [], "span": [], "combine": [], "gu_rows": [], "dn_rows": [], "gu_last": [], "dn_main_last": []}
    for g, d in runs:
        g = g[g[:, 0] > 0]
        d = d[d[:, 0] > 0]
        t0 = g[:, 0].min()
        for k, f in GU_PHASES:
            rows_gu[k].append(f(g, t0))
        for k, f in DN_PHASES:
            rows_dn[k].append(f(d, t0))
        last = d[d[:, 6] > 0]
        extra["combine"].append(last[:, 6] - last[:, 5])
        extra["gap"].append([d[:, 0].min() - g[:, 4].max()])
        extra["span"].append([max(d[:, 5].max(), last[:, 6].max() if len(last) else 0) - t0])
        extra["gu_rows"].append(g[:, 7])
        extra["dn_rows"].append(d[:, 7])
        extra["gu_last"].append([g[:, 4].max() - t0])
        extra["dn_main_last"].append([d[:, 2].max() - t0])
    cat = lambda v: np.concatenate([np.asarray(a, dtype=np.float64) for a in v])
    return ({k: _stats(cat(v)) for k, v in rows_gu.items()}, {k: _stats(cat(v)) for k, v in rows_dn.items()},
            {k: cat(v) for k, v in extra.items()}, len(runs[0][0][runs[0][0][:, 0] > 0]),
            len(runs[0][1][runs[0][1][:, 0] > 0]))


def breakdown(runs):
    """Main-loop medians of each launch by XCD (workgroup index mod 8: the hardware
    deals workgroups to the eight XCDs in turn) and by dispatch half (the first half
    of a launch's workgroups take the CUs first; the second half share those CUs as
    younger waves), and the launch's streaming rate: rows gathered x row bytes over
    the span from the first main-loop start to the last main-loop end."""
    out = []
    for k, (name, row_bytes) in enumerate((("gate/up", 2 * 14336 * 2 // 56), ("down", 4096 * 2 // 32))):
        mains, idx, rate = [], [], []
        for r in runs:
            g = r[k]
            live = g[:, 0] > 0
            g = g[live]
            ids = np.nonzero(live)[0]
            mains.append((g[:, 2] - g[:, 1]) * TICK_US)
            idx.append(ids)
            span = (g[:, 2].max() - g[:, 1].min()) * TICK_US
            rate.append(g[:, 7].sum() * row_bytes / (span * 1e-6) / 1e12)
        m, i = np.concatenate(mains), np.concatenate(idx)
        n = int(i.max()) + 1
        xcd = " / ".join(f"{np.median(m[i % 8 == x]):.2f}" for x in range(8))
        half = f"{np.median(m[i < n // 2]):.2f} / {np.median(m[i >= n // 2]):.2f}"
        out.append(f"- {name} main loop, median µs by XCD 0..7: {xcd}; by dispatch half (first / second): "
                   f"{half}; rows x row bytes over the main-loop span: {np.median(rate):.2f} TB/s")
    return out


def table(title, stats):
    out = [f"| {title} | median us | p10 | p90 | max |", "|---|---|---|---|---|"]
    for k, (m, a, b, c) in stats.items():
        out.append(f"| {k} | {m:.2f} | {a:.2f} | {b:.2f} | {c:.2f} |")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--sparsity", type=float, default=0.5)
    ap.add_argument("--reps", type=int, default=8)
    ap.add_argument("--out", default=None, help="also write the markdown summary here")
    ap.add_argument("--attention", action="store_true", help="time the decode attention's phases instead")
    a = ap.parse_args(argv)
    if a.attention:
        return attention_main(a, argv)
    if not os.path.exists(LIB_TL):
        raise SystemExit(f"{LIB_TL} not built: python -m activation_sparse_gemv_amd.build --timeline")
    L.LIB_PATH = LIB_TL
    import torch
    from . import api as asg
    from . import datagen
    lib = L.load()
    lib.as_phase_timeline_arm.restype = ctypes.c_int
    lib.as_phase_timeline_arm.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    dev = "cuda:0"
    shape = datagen.CFG2
    d = shape.d_model
    wgu, wd = datagen.mlp_weights_input_major(2, 0, shape)
    w0 = asg.MLPWeights(wgu.to(dev), wd.to(dev))
    del wgu, wd
    layers = [w0] + [asg.MLPWeights(w0.w_gate_up.clone(), w0.w_down.clone()) for _ in range(7)]
    calib = datagen.student_t((256, d), datagen.seed_for(2, 0, "calib")).to(dev)
    toks = datagen.student_t((64, d), datagen.seed_for(2, 0, "decode")).to(dev)
    t_x = float(asg.as_calibrate_threshold(calib, a.sparsity).item())
    hs = []
    for b in range(0, 256, 16):
        _, dbg = asg.as_sparse_swiglu_mlp(calib[b:b + 16], w0, t_x, float("-inf"), debug=True)
        hs.append(dbg["h"].clone())
    t_h = float(asg.as_calibrate_threshold(torch.cat(hs), a.sparsity).item())
    Y = torch.empty((1, d), dtype=torch.float32, device=dev)
    words = 2 * 16 * 4096
    buf = torch.zeros(words, dtype=torch.int64, device=dev)
    lines = [f"# Phase timeline: sparse SwiGLU MLP 4096 -> 14336 -> 4096, bf16, batch 1, "
             f"sparsity {a.sparsity} (MI355X)", "",
             "Command (from the repository root):", "", "```",
             "python -m activation_sparse_gemv_amd.build --timeline",
             "python -m activation_sparse_gemv_amd.timeline " + " ".join(argv if argv is not None else sys.argv[1:]),
             "```", "",
             "Per-workgroup phase durations from the 100 MHz device clock, pooled over "
             f"{a.reps} single calls, each issued behind 8 calls on the other weight copies "
             "(eight 352 MB copies rotate, so no call finds its rows in the 256 MB cache).", ""]
    for name, tx, th in (("sparse", t_x, t_h), ("dense", float("-inf"), float("-inf"))):
        calls = [asg.prepare_sparse_swiglu_mlp(toks[i % 64], layers[i % 8], tx, th, Y) for i in range(48)]
        for c in calls:
            c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per_layer = []
        for _ in range(5):
            e0.record()
            for c in calls:
                c()
            e1.record()
            torch.cuda.synchronize()
            per_layer.append(e0.elapsed_time(e1) * 1e3 / len(calls))
        runs = []
        for rep in range(a.reps):
            buf.zero_()
            c = asg.prepare_sparse_swiglu_mlp(toks[5 + rep], layers[(3 + rep) % 8], tx, th, Y)
            for c2 in calls[:8]:
                c2()
            # arming is host-side: the armed call queues behind the eight in flight
            L.check(lib.as_phase_timeline_arm(ctypes.c_void_p(buf.data_ptr()), words), "as_phase_timeline_arm")
            c()
            torch.cuda.synchronize()
            tl = buf.cpu().numpy().reshape(2, words // 32, 16)
            runs.append((tl[0].copy(), tl[1].copy()))
        gu, dn, ex, n1, n2 = summarize(runs)
        br = breakdown(runs)
        lines += [f"## {name}", "",
                  f"- layer time of this build: {np.median(per_layer):.2f} us (median of 5 x 48 back-to-back calls)",
                  f"- one call from the first gate/up workgroup to the last down workgroup: median "
                  f"{np.median(ex['span']) * TICK_US:.2f} us",
                  f"- gate/up launch: {n1} workgroups, rows per workgroup median {np.median(ex['gu_rows']):.0f}; "
                  f"last one ends at {np.median(ex['gu_last']) * TICK_US:.2f} us (median over calls)",
                  f"- gap from the last gate/up workgroup to the first down workgroup: "
                  f"{np.median(ex['gap']) * TICK_US:.2f} us",
                  f"- down launch: {n2} workgroups, rows per workgroup median {np.median(ex['dn_rows']):.0f}; "
                  f"last main loop ends at {np.median(ex['dn_main_last']) * TICK_US:.2f} us; "
                  f"combine of the last workgroup per tile {np.median(ex['combine']) * TICK_US:.2f} us", ""]
        lines += table("gate/up phase", gu) + [""] + table("down phase", dn) + [""] + br + [""]
        print("\n".join(lines[-(len(gu) + len(dn) + len(br) + 15):]), flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")


ATT_PHASES = [
    ("workgroup start (after the first)", lambda g, t0: g[:, 0] - t0),
    ("scores computed (query and K rows arrived)", lambda g, t0: g[:, 1] - t0),
    ("chunk maximum known (first barrier)", lambda g, t0: g[:, 2] - t0),
    ("wave partial outputs in LDS (second barrier)", lambda g, t0: g[:, 3] - t0),
    ("chunk record stored and complete", lambda g, t0: g[:, 4] - t0),
    ("arrival counter returned", lambda g, t0: g[:, 5] - t0),
]
ATT_MERGE = [
    ("merge weights ready (statistics loaded)", lambda g, t0: g[:, 6] - t0),
    ("output stored", lambda g, t0: g[:, 7] - t0),
]


def attention_main(a, argv):
    """Decode attention at n_ctx 2048, 32/8 heads, head_dim 128: per-workgroup phase
    times from the first workgroup's entry, for calls on one cache (its 8.4 MB stay
    in the last-level cache) and on 40 rotating caches (336 MB, from HBM)."""
    if not os.path.exists(LIB_TL):
        raise SystemExit(f"{LIB_TL} not built: python -m activation_sparse_gemv_amd.build --timeline")
    L.LIB_PATH = LIB_TL
    import torch
    from . import api as asg
    from . import datagen
    lib = L.load()
    lib.as_attention_timeline_arm.restype = ctypes.c_int
    lib.as_attention_timeline_arm.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    dev = "cuda:0"
    c3 = datagen.CFG3_ATTN
    n_q, n_kv, hd, n_ctx = c3["n_q"], c3["n_kv"], c3["head_dim"], c3["n_ctx"]
    caches = []
    for i in range(40):
        kc, vc = datagen.kv_cache(3, i, n_ctx=n_ctx, n_kv=n_kv, head_dim=hd)
        caches.append((kc.to(dev), vc.to(dev)))
    q = datagen.normal((n_q, hd), datagen.seed_for(3, 0, 91), std=1.0, dtype="f32").to(dev)
    kn = datagen.normal((n_kv, hd), datagen.seed_for(3, 0, 92), std=1.0, dtype="f32").to(dev)
    vn = datagen.normal((n_kv, hd), datagen.seed_for(3, 0, 93), std=1.0, dtype="f32").to(dev)
    words = 16 * 4096
    buf = torch.zeros(words, dtype=torch.int64, device=dev)
    lines = ["# Phase timeline: decode attention, n_ctx 2048, 32 query / 8 kv heads, head_dim 128 (MI355X)", "",
             "Command (from the repository root):", "", "```",
             "python -m activation_sparse_gemv_amd.build --timeline",
             "python -m activation_sparse_gemv_amd.timeline " + " ".join(argv if argv is not None else sys.argv[1:]),
             "```", "",
             "Times in us from the first workgroup's entry (100 MHz device clock stamped by thread 0 of every "
             f"workgroup), pooled over {a.reps} single calls, each issued behind 8 calls on other caches. "
             "The last two rows are the merging workgroup of each kv head only.", ""]
    for name, rot in (("one cache (warm: last-level cache)", False), ("40 rotating caches (cold: HBM)", True)):
        for i in range(8):
            asg.as_gqa_decode_attention(q, kn, vn, *caches[i])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(64):
            asg.as_gqa_decode_attention(q, kn, vn, *caches[(i % 40) if rot else 0])
        e1.record()
        torch.cuda.synchronize()
        per_call = e0.elapsed_time(e1) * 1e3 / 64
        chunk, merge = {k: [] for k, _ in ATT_PHASES}, {k: [] for k, _ in ATT_MERGE}
        n_wg = 0
        for rep in range(a.reps):
            buf.zero_()
            for i in range(8):
                asg.as_gqa_decode_attention(q, kn, vn, *caches[(8 + rep * 3 + i) % 40 if rot else 0])
            L.check(lib.as_attention_timeline_arm(ctypes.c_void_p(buf.data_ptr()), words),
                    "as_attention_timeline_arm")
            asg.as_gqa_decode_attention(q, kn, vn, *caches[(rep * 5) % 40 if rot else 0])
            torch.cuda.synchronize()
            g = buf.cpu().numpy().reshape(-1, 16)
            g = g[g[:, 0] > 0].astype(np.float64)
            n_wg = len(g)
            t0 = g[:, 0].min()
            for k, f in ATT_PHASES:
                chunk[k].append(f(g, t0))
            m = g[g[:, 7] > 0]
            for k, f in ATT_MERGE:
                merge[k].append(f(m, t0))
        cat = lambda v: np.concatenate([np.asarray(x, dtype=np.float64) for x in v])
        st = {k: _stats(cat(v)) for k, v in chunk.items()}
        st.update({k: _stats(cat(v)) for k, v in merge.items()})
        lines += [f"## {name}", "",
                  f"- {n_wg} workgroups (8 kv heads x chunks of 64 cached keys); eager back-to-back calls "
                  f"(events; host-bound, the binding's per-call work included): {per_call:.2f} us per call", ""]
        lines += table("phase (us from the first entry)", st) + [""]
        print("\n".join(lines[-(len(st) + 6):]), flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
