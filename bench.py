"""Throughput of the DFlash 2 per-cycle draft-block path on one MI355X.

One step = one whole cycle over one batch of synthetic inputs, replayed from a
HIP graph: 20 two-tap conv sites (each its own x, x_{-1} and tap weights),
top-16 over the drafter's block logits, pair scores (gathered bf16 MFMA
projections + bilinear epilogue), the Viterbi path, and greedy verification
against the target's logits.  Default workload: 32 requests, block 16
(15 drafts), vocabulary 151,936, hidden 5120, rank 256.

Prints one JSON line.  value = draft blocks per second (requests x cycles /
s) for the whole step; per-kernel times come from HIP events recorded on the
launch stream by the library's timing hook; the roofline object describes the
kernel with the largest time per step; hbm_frac is the cycle's algorithmic
HBM bytes (logits, target logits, gathered embedding rows, context rows,
selector weights and, with the conv sites, their x, x_prev, W and y) per
second against the 8 TB/s peak, for the step and every sweep point;
cpu_baseline times the CPU oracle on a bounded sample of the same workload.
`tables` reports the same cycles with the pair scores read from per-token
A/B tables built once per weight set (dflash2_selector_tables, timed on its
own as `build_ms`); the headline value projects the embedding rows every
cycle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/s (topk+select+verify) at B=1/8/32, block 8/16; % HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

STRESS = "b64_blk16_v262144_stress"
KERNEL_TAGS = ["conv_gemm", "conv_epilogue", "topk_chunk", "topk_merge", "project_gemm", "h_gemm",
               "proj_reduce", "pair_epilogue", "path", "argmax_part", "greedy_final",
               "sumexp_part", "residual_fused", "residual_chunk", "residual_find"]
EVICT_BYTES = 1 << 30          # written between cold replays: 4x the 256 MB Infinity Cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b32_blk16_v151936_conv")
    ap.add_argument("--no-sweep", action="store_true", help="skip the batch x block sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tables", action="store_true", help="skip the per-token table cycles")
    ap.add_argument("--no-kernel-profile", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache replays")
    ap.add_argument("--no-heads", action="store_true",
                    help="skip the fused LM-head legs (drafter top-16, target greedy verification)")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="requests the oracle recomputes (0: all of the batch)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this size (counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_cycle(w, dev, E=None, conv=True, tables=False, fused=False):
    import torch
    import synth
    from draft_selection_bf16_amd.cycle import ConvSite, Cycle
    z, tok, _ = synth.drafter_logits(w, device=dev)
    Z = synth.target_logits(w, z, tok, device=dev)
    if E is None:
        E = synth.embeddings(w, device=dev)
    wa, wb, wh = synth.selector_weights(w, device=dev)
    h = synth.context_hidden(w, device=dev)
    last = synth.last_tokens(w, device=dev)
    sites = []
    if conv:
        for s in range(w.conv_sites):
            x, xp, wt, bs = synth.conv_site(w, s, device=dev)
            sites.append(ConvSite(x, xp, wt, bs, torch.empty(x.shape, dtype=torch.bfloat16, device=dev)))
    cyc = Cycle(logits=z, target=Z, emb=E, h=h, w_a=wa, w_b=wb, w_h=wh, last_tok=last, K=w.K,
                path_mode=w.path_mode, verify=w.verify, tau=w.tau if w.tau > 0 else 1.0,
                conv_sites=sites, seed=w.seed, tables=tables, fused=fused)
    return cyc, E


def time_graph(cyc, steps, warmup):
    import torch
    for _ in range(warmup):
        cyc.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        cyc.replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall


def replay_spread(cyc, n):
    """Median and 90th percentile of single replays (events around each
    replay; outside the timed region)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        cyc.replay()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return dict(median=round(ms[n // 2], 5), p90=round(ms[min(n - 1, (9 * n) // 10)], 5), n=n)


def cold_replays(cyc, n, evict):
    """Median and 90th percentile of single replays, each after `evict` (a
    1 GiB buffer) has been overwritten, so that no input of the cycle is
    left in the Infinity Cache or the L2s; the fill runs outside the events."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in ev:
        evict.fill_(1)
        a.record()
        cyc.replay()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return dict(median_us=round(1e3 * ms[n // 2], 2), p90_us=round(1e3 * ms[min(n - 1, (9 * n) // 10)], 2), n=n)


def heads_leg(dev, steps):
    """The fused LM-head kernels at the benchmark's shapes: the drafter's
    top-16 from its hidden states (dflash2_lm_head_topk; logits h E^T never
    stored) and greedy and rejection verification from the target's hidden
    states (dflash2_verify_greedy_head, dflash2_verify_reject_head).  Per call: HIP events around `steps`
    back-to-back calls; per kernel: the library's timing hook.  MFMA
    fraction = 2 rows V d flops per call against the dense bf16 peak."""
    import torch
    import synth
    import draft_selection_bf16_amd as df2
    out = {}
    E = None
    for name in ("b32_blk16_v151936_conv", "b1_blk8_v151936"):
        w = synth.WORKLOADS[name]
        if E is None or E.shape[0] != w.V:
            E = synth.embeddings(w, device=dev)
        d, V = w.d, w.V
        rows = w.B * w.T
        h = synth.context_hidden(w, device=dev).reshape(rows, d)
        idx = torch.empty((rows, 16), dtype=torch.int32, device=dev)
        val = torch.empty((rows, 16), dtype=torch.float32, device=dev)
        wsb = torch.empty(max(1, df2.dflash2_lm_head_topk_workspace_bytes(rows, V, d, 16)), dtype=torch.uint8,
                          device=dev)
        g = torch.Generator().manual_seed(5)
        ht = torch.randn(w.B, w.T + 1, d, generator=g).to(torch.bfloat16).to(dev)
        path = torch.randint(0, V, (w.B, w.T), generator=g, dtype=torch.int32).to(dev)
        acc = torch.empty((w.B,), dtype=torch.int32, device=dev)
        otok = torch.empty((w.B, w.T + 1), dtype=torch.int32, device=dev)
        wsv = torch.empty(max(1, df2.dflash2_verify_greedy_head_workspace_bytes(w.B, w.T, V, d)),
                          dtype=torch.uint8, device=dev)
        # rejection verification: 16 candidates per position, q uniform over
        # them, the drafted token one of them
        cand = torch.randint(0, V, (w.B, w.T, 16), generator=g, dtype=torch.int32).to(dev)
        qq = torch.full((w.B, w.T, 16), 1.0 / 16, dtype=torch.float32, device=dev)
        rank = torch.randint(0, 16, (w.B, w.T), generator=g, dtype=torch.int32).to(dev)
        rpath = torch.gather(cand, 2, rank.long()[..., None])[..., 0].contiguous()
        seed = torch.tensor([7], dtype=torch.int64, device=dev)
        wsr = torch.empty(max(1, df2.dflash2_verify_reject_head_workspace_bytes(w.B, w.T, V, d, 16)),
                          dtype=torch.uint8, device=dev)
        calls = {"lm_head_topk": (lambda: df2.dflash2_lm_head_topk(h, E, 16, idx, val, wsb), rows,
                                  ("lmhead_topk", "lmhead_merge")),
                 "verify_greedy_head": (lambda: df2.dflash2_verify_greedy_head(ht, E, path, acc, otok, wsv),
                                        w.B * (w.T + 1), ("head_argmax", "greedy_head_final")),
                 "verify_reject_head": (lambda: df2.dflash2_verify_reject_head(ht, E, rpath, rank, cand, qq, 1.0,
                                                                               seed, acc, otok, wsr),
                                        w.B * (w.T + 1), ("head_stats", "head_row_reduce", "head_decide",
                                                          "head_block_logits", "head_draw"))}
        res = {}
        for key, (fn, nrows, tags) in calls.items():
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            us = 1e3 * a.elapsed_time(b) / steps
            kern = {}
            for tag in tags:
                df2.dflash2_profile_start(tag, steps)
                for _ in range(steps):
                    fn()
                ms = df2.dflash2_profile_stop(steps)
                kern[tag] = round(1e3 * sum(ms) / max(1, len(ms)), 2)
            flops = 2 * nrows * V * d
            tf = flops / (us * 1e-6) / 1e12
            res[key] = dict(rows=nrows, us_per_call=round(us, 2), kernels_us=kern, tflops=round(tf, 1),
                            mfma_frac=round(tf / BF16_PEAK_TFLOPS, 4),
                            lm_head_read_tbs=round(V * d * 2 / (us * 1e-6) / 1e12, 2))
        out[name] = res
        del h, idx, val, wsb, ht, path, acc, otok, wsv, cand, qq, rank, rpath, seed, wsr
    del E
    torch.cuda.empty_cache()
    return out


def profile_kernels(cyc, steps):
    """Per-launch durations of each kernel tag over `steps` eager cycles."""
    import torch
    import draft_selection_bf16_amd as df2
    out = {}
    per_step_launch = {"conv_gemm": len(cyc.conv_sites), "conv_epilogue": len(cyc.conv_sites)}
    for tag in KERNEL_TAGS:
        n_per = per_step_launch.get(tag, 1)
        if n_per == 0:
            continue
        torch.cuda.synchronize()
        df2.dflash2_profile_start(tag, steps * n_per)
        for _ in range(steps):
            cyc.run()
        ms = df2.dflash2_profile_stop(steps * n_per)
        if ms:
            out[tag] = dict(launches_per_step=len(ms) / steps, avg_us=1e3 * sum(ms) / len(ms),
                            us_per_step=1e3 * sum(ms) / steps)
    return out


def cycle_bytes(w, conv, esz=2, tables=False):
    """Algorithmic HBM bytes of one cycle: the drafter and target logits, the
    gathered embedding rows of the candidates and last tokens, the context
    rows and the three selector weights, and, with the conv sites, each
    site's x, x_prev, W and y.  With per-token tables the candidates' and
    last tokens' fp32 table rows and W_H replace the embedding rows and the
    three weights."""
    B, T, K, V, d, r = w.B, w.T, w.K, w.V, w.d, w.r
    by = B * T * V * esz + B * (T + 1) * V * esz
    if tables:
        by += (B * T * K + B) * 2 * r * 4 + B * T * d * 2 + r * d * 2
    else:
        by += (B * T * K + B + B * T) * d * 2 + 3 * r * d * 2
    if conv and w.conv_sites:
        L, G2 = w.block, 2 * (d // 16)
        by += w.conv_sites * (2 * B * L * d * 2 + B * d * 2 + G2 * d * 2)
    return by


def hbm_frac(w, conv, us, tables=False):
    return round(cycle_bytes(w, conv, tables=tables) / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)


def tables_leg(w, E, dev, steps, warmup, with_sweep):
    """The cycle with per-token A/B tables: the one-off table build, the step
    with and without the conv sites, per-kernel times and (with the sweep)
    the other batch x block points."""
    import torch
    import draft_selection_bf16_amd as df2
    out = {}
    cyc, _ = build_cycle(w, dev, E=E, conv=True, tables=True)
    wa, wb = cyc.w_a, cyc.w_b
    tab = torch.empty_like(cyc.tab)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    df2.dflash2_selector_tables(E, wa, wb, tab)
    a.record()
    for _ in range(3):
        df2.dflash2_selector_tables(E, wa, wb, tab)
    b.record()
    torch.cuda.synchronize()
    build_ms = a.elapsed_time(b) / 3
    out["build_ms"] = round(build_ms, 3)
    out["build_tflops"] = round(2 * w.V * w.d * 2 * w.r / (build_ms * 1e-3) / 1e12, 1)
    out["table_bytes"] = w.V * 2 * w.r * 4
    del tab
    cyc.capture()
    ms, _ = time_graph(cyc, steps, warmup)
    out["ms_per_step"] = round(ms, 5)
    out["value"] = round(w.B / (ms / 1e3), 1)
    out["hbm_frac"] = hbm_frac(w, True, ms * 1e3, tables=True)
    out["kernels"] = {k: round(v["avg_us"], 2) for k, v in profile_kernels(cyc, min(steps, 50)).items()}
    del cyc
    cyc_nc, _ = build_cycle(w, dev, E=E, conv=False, tables=True)
    cyc_nc.capture(conv=False)
    ms_nc, _ = time_graph(cyc_nc, steps, warmup)
    del cyc_nc
    out["us_per_cycle_without_conv"] = round(ms_nc * 1e3, 2)
    out["value_without_conv"] = round(w.B / (ms_nc / 1e3), 1)
    out["hbm_frac_without_conv"] = hbm_frac(w, False, ms_nc * 1e3, tables=True)
    if with_sweep:
        import synth
        sw = {}
        for name in ("b1_blk8_v151936", "b8_blk8_v151936_sampled", "b32_blk8_v151936",
                     "b1_blk16_v151936", "b8_blk16_v151936"):
            ws_ = synth.WORKLOADS[name]
            c2, _ = build_cycle(ws_, dev, E=E, conv=False, tables=True)
            c2.capture(conv=False)
            m2, _ = time_graph(c2, steps, warmup)
            sw[name] = dict(us_per_cycle=round(m2 * 1e3, 2), blocks_per_s=round(ws_.B / (m2 / 1e3), 1))
            del c2
        out["sweep"] = sw
    return out


def algorithmic(w, tag, esz=2):
    """(bytes, flops) one launch of `tag` must move / compute."""
    B, T, K, V, d, r = w.B, w.T, w.K, w.V, w.d, w.r
    G2 = 2 * (d // 16)
    L = w.block
    if tag == "topk_chunk":
        return B * T * V * esz + B * T * K * 8, 0
    if tag in ("argmax_part", "sumexp_part"):
        return B * (T + 1) * V * esz, 0
    if tag == "project_gemm":
        mc = B * T * K
        outs = mc * 2 * r + B * r + B * T * r
        return (mc + B + B * T) * d * 2 + 3 * r * d * 2 + 4 * outs, 2 * d * outs
    if tag == "conv_gemm":
        return B * L * d * 2 + G2 * d * 2, 2 * B * L * d * G2
    if tag == "conv_epilogue":
        return 2 * B * L * d * 2 + B * d * 2, 4 * B * L * d
    return None, None


def roofline_of(w, tag, avg_us):
    by, fl = algorithmic(w, tag)
    if by is None:
        return None
    t = avg_us * 1e-6
    if fl and fl / by > (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9):
        ach = fl / t / 1e12
        return dict(kernel=tag, bound="mfma", achieved=round(ach, 2), peak=BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / BF16_PEAK_TFLOPS, 4), traffic=None,
                    algorithmic_flops=fl, algorithmic_bytes=by, avg_us=round(avg_us, 2))
    ach = by / t / 1e9
    return dict(kernel=tag, bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4), traffic=None, algorithmic_bytes=by,
                avg_us=round(avg_us, 2))


COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters_b32_blk16_v151936_conv.txt")
TRACE = os.path.join(ROOT, "profiles", "cycle_b32_blk16_v151936_conv_kernel_trace.txt")

def source_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "draft_selection_bf16_amd")
    # the kernels are their sources plus the compiler flags they are built with
    for f in sorted(glob.glob(os.path.join(pkg, "csrc", "*"))) + [os.path.join(pkg, "build.py")]:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(tag):
    """HBM bytes per launch of `tag` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None
    when the summary is missing or the kernel sources changed since."""
    if not os.path.exists(COUNTERS):
        return None
    kv, rows = {}, {}
    for line in open(COUNTERS):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("kernel "):
            parts = line.split()
            rows[parts[1]] = {k: float(v) for k, v in (p.split("=") for p in parts[2:])}
        elif "=" in line:
            k, v = (x.strip() for x in line.split("=", 1))
            kv[k] = v
    if kv.get("source_sha256") != source_hash() or tag not in rows:
        return None
    r = rows[tag]
    return int(1024 * (r["fetch_kib"] * float(kv["fetch_factor"]) +
                       r["write_kib"] * float(kv["write_factor"])))


def trace_avg_us(tag):
    """Average duration (us) of kernel `tag` in the committed rocprofv3
    kernel-trace summary of the benchmark cycle, or None when the summary is
    missing or the kernel sources changed since it was taken."""
    if not os.path.exists(TRACE):
        return None
    sha, avg = None, None
    for line in open(TRACE):
        line = line.strip()
        if line.startswith("# source_sha256"):
            sha = line.split("=", 1)[1].strip()
        elif line and not line.startswith("#"):
            parts = line.split()
            if parts[0] == tag and len(parts) >= 3:
                avg = float(parts[2])
    if sha != source_hash():
        return None
    return avg


def cpu_baseline(cyc, w, nreq, min_seconds=10.0, max_reps=4, one_core_req=1):
    """The oracle's cycle for `nreq` of the requests (all 20 conv sites on
    those requests, top-16, pair scores, Viterbi, greedy verification),
    repeated until about `min_seconds` of oracle time (at most `max_reps`
    passes)."""
    import numpy as np
    import torch
    import oracle
    nreq = w.B if nreq <= 0 or nreq > w.B else nreq
    rows = list(range(nreq))
    # host copies (not timed)
    z = cyc.logits[rows].cpu()
    Z = cyc.target[rows].cpu()
    h = cyc.h[rows].cpu()
    last = cyc.last_tok[rows].cpu().numpy()
    wa, wb, wh = cyc.w_a.cpu(), cyc.w_b.cpu(), cyc.w_h.cpu()
    sites = [(s.x[rows].cpu(), s.x_prev[rows].cpu(), s.w.cpu(),
              None if s.base is None else s.base.cpu()) for s in cyc.conv_sites]
    torch.cuda.synchronize()

    def one_pass():
        t0 = time.perf_counter()
        for x, xp, wt, bs in sites:
            oracle.dynconv2(x, xp, wt, bs)
        idx, val = oracle.topk(z, w.K)
        t1 = time.perf_counter()
        # embedding rows of the oracle's own candidates (a gather; not timed)
        uniq, inv = np.unique(np.concatenate([idx.ravel(), last]), return_inverse=True)
        sub = cyc.emb[torch.from_numpy(uniq).to(cyc.emb.device).long()].cpu()
        ridx = inv[: idx.size].reshape(idx.shape).astype(np.int32)
        rlast = inv[idx.size:].astype(np.int32)
        t2 = time.perf_counter()
        S = oracle.pair_scores(ridx, val, rlast, sub, h, wa, wb, wh)
        p = oracle.path(S, idx, oracle.PATH_VITERBI)
        oracle.verify_greedy(Z, p["tok"])
        t3 = time.perf_counter()
        return (t1 - t0) + (t3 - t2)

    secs, reps = one_pass(), 1
    while secs < min_seconds and reps < max_reps:
        secs += one_pass()
        reps += 1
    cores = oracle.num_threads()
    out = dict(value=round(nreq * reps / secs, 4), unit="blocks/s", cores=cores,
               kind="oracle", seconds=round(secs, 2),
               sample=f"{reps} pass(es) over {nreq} of {w.B} requests of {w.name}: 20 conv sites, "
                      f"top-16, pair scores, Viterbi path, greedy verify (embedding-row gather "
                      f"excluded)")
    # the same oracle on one core, over `one_core_req` requests
    n1 = max(1, min(one_core_req, nreq))
    rows = rows[:n1]
    z, Z, h, last = z[:n1], Z[:n1], h[:n1], last[:n1]
    sites = [(x[:n1], xp[:n1], wt, bs) for x, xp, wt, bs in sites]
    oracle.set_num_threads(1)
    try:
        s1 = one_pass()
    finally:
        oracle.set_num_threads(cores)
    out["one_core"] = dict(value=round(n1 / s1, 4), unit="blocks/s", cores=1, seconds=round(s1, 2),
                           sample=f"1 pass over {n1} request(s) of {w.name}, same steps")
    import platform
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out["host"] = dict(cpu=cpu, os_cpu_count=os.cpu_count(), machine=platform.machine())
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              f"multi-GPU form (every request is independent: shard the batch, one process per GPU)", file=sys.stderr)
        sys.exit(2)
    log("importing torch")
    import torch
    import synth
    import draft_selection_bf16_amd as df2

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    df2.lib()
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS[args.workload]
    log(f"building inputs for {w.name}")
    cyc, E = build_cycle(w, dev)
    cyc.run()
    torch.cuda.synchronize()
    cyc.capture()
    log("timing the full cycle")
    ms, wall = time_graph(cyc, args.steps, args.warmup)
    value = w.B / (ms / 1e3)
    spread = replay_spread(cyc, min(args.steps, 100))
    evict = None if args.no_cold else torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    cold = None if evict is None else cold_replays(cyc, min(args.steps, 50), evict)

    # the same cycle without the conv sites (top-K + select + verify only)
    cyc_nc, _ = build_cycle(w, dev, E=E, conv=False)
    cyc_nc.capture(conv=False)
    ms_nc, _ = time_graph(cyc_nc, args.steps, args.warmup)

    kernels = {}
    roof = None
    if not args.no_kernel_profile:
        log("per-kernel event timing")
        kernels = profile_kernels(cyc, min(args.steps, 50))
        dom = max(kernels, key=lambda k: kernels[k]["us_per_step"])
        roof = roofline_of(w, dom, kernels[dom]["avg_us"])
        if roof is not None and w.name == "b32_blk16_v151936_conv":
            roof["traffic"] = measured_traffic(dom)
            # the same kernel's average duration in the committed rocprofv3
            # trace of this command, and the fraction it gives
            tus = trace_avg_us(dom)
            if tus:
                rt = roofline_of(w, dom, tus)
                roof["trace"] = dict(avg_us=round(tus, 2), achieved=rt["achieved"], frac=rt["frac"])
        for k, v in kernels.items():
            rl = roofline_of(w, k, v["avg_us"])
            if rl:
                v["roofline"] = {kk: rl[kk] for kk in ("bound", "achieved", "unit", "frac")}

    sweep = {}
    if not args.no_sweep:
        log("sweep")
        for name in ("b1_blk8_v151936", "b8_blk8_v151936_sampled", "b32_blk8_v151936",
                     "b1_blk16_v151936", "b8_blk16_v151936"):
            ws_ = synth.WORKLOADS[name]
            c2, _ = build_cycle(ws_, dev, E=E, conv=False)
            c2.capture(conv=False)
            m2, _ = time_graph(c2, args.steps, args.warmup)
            sweep[name] = dict(B=ws_.B, block=ws_.block, path=ws_.path_mode, verify=ws_.verify,
                               us_per_cycle=round(m2 * 1e3, 2), blocks_per_s=round(ws_.B / (m2 / 1e3), 1),
                               hbm_frac=hbm_frac(ws_, False, m2 * 1e3))
            if evict is not None:
                cr = cold_replays(c2, min(args.steps, 50), evict)
                sweep[name]["cold"] = dict(cr, hbm_frac=hbm_frac(ws_, False, cr["median_us"]))
            del c2
            if ws_.B == 1 and ws_.verify == "greedy":
                # the same cycle as one persistent launch (dflash2_cycle_fused)
                c2, _ = build_cycle(ws_, dev, E=E, conv=False, fused=True)
                c2.capture(conv=False)
                m2, _ = time_graph(c2, args.steps, args.warmup)
                sweep[name]["fused_us_per_cycle"] = round(m2 * 1e3, 2)
                sweep[name]["fused_status"] = int(c2.status.item())
                del c2
        sweep[w.name + " (no conv)"] = dict(B=w.B, block=w.block, us_per_cycle=round(ms_nc * 1e3, 2),
                                            blocks_per_s=round(w.B / (ms_nc / 1e3), 1),
                                            hbm_frac=hbm_frac(w, False, ms_nc * 1e3))
        if evict is not None:
            cr = cold_replays(cyc_nc, min(args.steps, 50), evict)
            sweep[w.name + " (no conv)"]["cold"] = dict(cr, hbm_frac=hbm_frac(w, False, cr["median_us"]))
        if w.name != STRESS:
            # the stress cycle (64 requests, vocabulary 262,144, half greedy and half
            # rejection verification), with and without its 20 conv sites
            ws_ = synth.WORKLOADS[STRESS]
            E4 = None
            for conv in (True, False):
                c2, E4 = build_cycle(ws_, dev, E=E4, conv=conv)
                c2.capture(conv=conv)
                m2, _ = time_graph(c2, args.steps, args.warmup)
                sweep[STRESS + ("" if conv else " (no conv)")] = dict(
                    B=ws_.B, block=ws_.block, path=ws_.path_mode, verify=ws_.verify,
                    conv_sites=ws_.conv_sites if conv else 0, us_per_cycle=round(m2 * 1e3, 2),
                    blocks_per_s=round(ws_.B / (m2 / 1e3), 1), hbm_frac=hbm_frac(ws_, conv, m2 * 1e3))
                del c2
            del E4

    del cyc_nc
    heads = None
    if not args.no_heads:
        log("fused LM-head legs")
        heads = heads_leg(dev, min(args.steps, 20))

    tabs = None
    if not args.no_tables:
        log("per-token tables")
        tabs = tables_leg(w, E, dev, args.steps, args.warmup, not args.no_sweep)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(cyc, w, args.cpu_sample)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "block": w.block, "draft_tokens": w.T,
                   "candidates": w.K, "vocab": w.V, "hidden": w.d, "rank": w.r,
                   "conv_sites": w.conv_sites, "path": w.path_mode, "verify": w.verify,
                   "step": "20 x dynconv2 + topk + pair_scores + path + verify, one HIP graph"},
        "tokens_scored_per_s": round(w.B * w.T * w.K / (ms / 1e3), 1),
        # scored (predecessor, candidate) pairs: K at the first position (from
        # the last verified token), K x K at each later one
        "pair_scores_per_s": round(w.B * (w.K + (w.T - 1) * w.K * w.K) / (ms / 1e3), 1),
        "value_without_conv": round(w.B / (ms_nc / 1e3), 1),
        "hbm_frac": hbm_frac(w, True, ms * 1e3),
        "hbm_frac_without_conv": hbm_frac(w, False, ms_nc * 1e3),
        "replay_ms": spread,
        "cold_replay": None if cold is None else dict(cold, hbm_frac=hbm_frac(w, True, cold["median_us"])),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "sweep": sweep,
        "tables": tabs,
        "heads": heads,
        "wall_s_timed": round(wall, 3),
    }
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
