#!/usr/bin/env python3
"""Benchmark: one global-attention layer of the VGGT Aggregator at S = 100 frames.

A step is one full call of the block -- range guards + QKV projection with QK
LayerNorm and 2D RoPE + attention core + output projection -- over
X[100, 1031, 1024] bf16 (N = 103,100 tokens, d = 1024, H = 16, Dh = 64), with
every input already resident in HBM.  Prints ONE JSON line:

  value        algorithmic TFLOP/s of the whole layer (4 N^2 d + 8 N d^2 FLOP)
  ms_per_step  ms per layer
  roofline     the attention-core kernel alone, timed on the call's stream
               with HIP events, against the dense fp16/bf16 MFMA peak
  cpu_baseline the fp64 NumPy oracle timed on this host on a bounded sample
  extra        ms/layer of the other block modes and frame counts

Inputs are seeded synthetic data (X ~ N(0,1), weights ~ N(0,1/d), gamma ~
1+N(0,0.1), beta ~ N(0,0.1)); there are no trained weights.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "global-attention ms/layer + TFLOP/s (frac of bf16 MFMA peak) at S frames, 1 GPU"


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_kernel_s100_global_hbm_bytes.md")


def attention_source_hash() -> str:
    """Hash of the attention kernel's code: its sources without // comments
    and blank lines, so that comment edits keep the recorded counters valid."""
    h = hashlib.sha256()
    for f in ("attention.hip", "common.h"):
        with open(os.path.join(ROOT, "vggt_global_attention_amd", "csrc", f)) as fh:
            code = [line.split("//", 1)[0].rstrip() for line in fh.read().splitlines()]
        h.update("\n".join(c for c in code if c.strip()).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when the attention sources changed since the counters were taken."""
    try:
        kv = dict(line.split(": ", 1) for line in open(TRAFFIC_PROFILE).read().splitlines()
                  if line.startswith(("traffic_bytes_per_launch:", "attention_source_sha256_16:")))
    except OSError:
        return None
    if kv.get("attention_source_sha256_16", "").strip() != attention_source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="s100")
    ap.add_argument("--mode", default="global",
                    choices=["global", "frame", "register", "subsampled", "merged"])
    ap.add_argument("--sub", default="3x3", help="subsampled mode: windows sub_h x sub_w")
    ap.add_argument("--merge", default="4,2,3,12",
                    help="merged mode: frames per block, window rows, window columns, merges per block")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other modes / sizes")
    ap.add_argument("--cpu-rows", type=int, default=8192, help="query rows in the CPU sample")
    ap.add_argument("--only-stage", default=None, choices=["prep", "qkv", "core", "out"],
                    help="time one stage in a loop (for profilers) and print its ms")
    ap.add_argument("--cpu-full", action="store_true",
                    help="instead of the layer: time the fp64 oracle on whole workloads "
                         "(tiny, s24, s500, s100; s300 on a row sample) on this host")
    ap.add_argument("--hbm", action="store_true",
                    help="instead of the layer: HBM-bound kernels (register-mode patch copy, "
                         "residual update) at 500 frames, warm and after a 512 MB cache scrub")
    ap.add_argument("--descriptors", type=int, default=0, metavar="PER_FRAME",
                    help="instead of the layer: descriptor attention of the workload's tokens "
                         "against PER_FRAME cached descriptors per frame")
    ap.add_argument("--schedule", default=None, metavar="S_LIST",
                    help="instead of the layer: time the 24-layer attention-only schedule and "
                         "record its peak device memory at these frame counts, e.g. 1,25,100")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    ap.add_argument("--graph", action="store_true",
                    help="with --schedule: also time the forward captured into a HIP graph "
                         "(frame counts up to 100)")
    ap.add_argument("--power", action="store_true",
                    help="instead of the layer: socket power and shader clock (amd-smi) while "
                         "the workload's layer runs on its inputs and on zero q/k/v operands")
    return ap.parse_args()


def gpu_inputs(w):
    import torch
    from vggt_global_attention_amd import synth
    inp = synth.make_inputs(w)
    keys = ("X", "Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")
    return inp, {k: inp[k].to("cuda").contiguous() for k in keys}


def time_block(w, mode, d, steps, warmup, sub=(1, 1), rows=None, operands="fp16", inplace=False):
    """ms per full call and ms per attention-core stage, both with HIP events
    on the stream the library launches on (torch's current stream).  rows =
    (begin, count): the query-row window of the global block instead.
    inplace (register mode): Y = X on a copy of X, so the patch rows stay
    where they are and only the special rows are written."""
    import torch
    from vggt_global_attention_amd import api
    from vggt_global_attention_amd import binding as B
    X = d["X"].clone() if inplace else d["X"]
    args = (X, d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"], d["k_beta"])
    if rows is not None:
        blk = api.RowsBlock(d["X"], w.H, w.grid_h, w.grid_w, rows[0], rows[1])
        Y = torch.empty((rows[1], w.d), dtype=d["X"].dtype, device=d["X"].device)
    else:
        if mode == "merged":
            blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w, merge=sub)
        else:
            blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w, sub=sub, operands=operands)
        Y = X if inplace else torch.empty_like(d["X"])
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        blk(*args, Y=Y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        blk(*args, Y=Y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    # attention core alone: the workspace holds q/k/v from the calls above; the
    # core overwrites q with O, so rerun the QKV stage (untimed) before each core.
    core = 0.0
    for i in range(steps):
        blk.stage(B.STAGE_QKV, *args, Y)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        blk.stage(B.STAGE_CORE, *args, Y)
        c1.record(stream)
        torch.cuda.synchronize()
        core += c0.elapsed_time(c1)
    return ms_step, core / steps


def loop_stage(w, mode, d, stage, steps, sub=(1, 1)):
    import torch
    from vggt_global_attention_amd import api
    from vggt_global_attention_amd import binding as B
    st = {"prep": B.STAGE_PREP, "qkv": B.STAGE_QKV, "core": B.STAGE_CORE, "out": B.STAGE_OUT}
    if mode == "merged":
        blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w, merge=sub)
    else:
        blk = api.Block(mode, d["X"], w.H, w.grid_h, w.grid_w, sub=sub)
    args = (d["X"], d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"], d["k_beta"])
    Y = torch.empty_like(d["X"])
    blk(*args, Y=Y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if stage == "core":
            blk.stage(B.STAGE_QKV, *args, Y)
        blk.stage(st[stage], *args, Y)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_descriptor(w, d, per_frame, steps, warmup):
    """Descriptor attention: the S*T tokens attend to per_frame * S cached
    descriptors.  Times the append of all descriptors (one chunk), the full
    attend call and its attention-core stage (HIP events on the call's
    stream)."""
    import torch
    from vggt_global_attention_amd import binding as B
    from vggt_global_attention_amd import synth
    from vggt_global_attention_amd.descriptor import DescriptorCache
    M = per_frame * w.S
    D = synth.make_descriptors(w, M, 0).to("cuda")
    cache = DescriptorCache(w.d, w.H, M)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    wts = (d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"])
    Y = torch.empty_like(d["X"])
    for _ in range(warmup):
        cache.reset()
        cache.append(D, d["Wqkv"], d["k_gamma"], d["k_beta"])
        cache.attend(d["X"], w.grid_h, w.grid_w, *wts, Y=Y)
    torch.cuda.synchronize()
    app = att = core = 0.0
    for _ in range(steps):
        cache.reset()
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        cache.append(D, d["Wqkv"], d["k_gamma"], d["k_beta"])
        e1.record(stream)
        cache.attend(d["X"], w.grid_h, w.grid_w, *wts, Y=Y)
        e2.record(stream)
        cache.attend_stage(B.STAGE_QKV, d["X"], w.grid_h, w.grid_w, *wts, Y)
        c0, c1 = ev(), ev()
        c0.record(stream)
        cache.attend_stage(B.STAGE_CORE, d["X"], w.grid_h, w.grid_w, *wts, Y)
        c1.record(stream)
        torch.cuda.synchronize()
        app += e0.elapsed_time(e1)
        att += e1.elapsed_time(e2)
        core += c0.elapsed_time(c1)
    app, att, core = app / steps, att / steps, core / steps
    attn_flop = 4.0 * w.N * M * w.d
    gemm_flop = 4.0 * M * w.d ** 2 + 4.0 * w.N * w.d ** 2   # K, V of the descriptors; q, Wo
    return {"descriptors": M, "per_frame": per_frame, "append_ms": app, "attend_ms": att,
            "core_ms": core, "core_tflops": attn_flop / core / 1e9,
            "tflops": (attn_flop + gemm_flop) / (app + att) / 1e9}


def hbm_kernels(steps):
    """GB/s of the HBM-bound kernels at 500 frames (X: 1.06 GB): the register
    block's patch copy (the call with Y != X minus the in-place call) and the
    residual update, each timed warm (back to back) and cold (a 512 MB write,
    twice the 256 MB Infinity Cache, before every call)."""
    import torch
    from vggt_global_attention_amd import api, configs, synth
    from vggt_global_attention_amd import schedule as S
    w = configs.WORKLOADS["s500"]
    inp, d = gpu_inputs(w)
    stream = torch.cuda.current_stream()
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, cold):
        tot = 0.0
        for _ in range(steps):
            if cold:
                scrub.fill_(1)
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / steps

    args = [d[k] for k in ("Wqkv", "Wo", "q_gamma", "q_beta", "k_gamma", "k_beta")]
    blk = api.Block("register", d["X"], w.H, w.grid_h, w.grid_w)
    Xi = d["X"].clone()
    Y = torch.empty_like(d["X"])
    out = {}
    copy_bytes = 2.0 * w.S * (w.T - 17) * w.d * 2
    for cold in (False, True):
        blk(d["X"], *args, Y=Y)
        blk(Xi, *args, Y=Xi)
        torch.cuda.synchronize()
        full = timed(lambda: blk(d["X"], *args, Y=Y), cold)
        inplace = timed(lambda: blk(Xi, *args, Y=Xi), cold)
        ms = full - inplace
        out[f"patch_copy_s500_{'cold' if cold else 'warm'}"] = {
            "bytes": copy_bytes, "ms": ms, "gbs": copy_bytes / ms / 1e6,
            "register_call_ms": full, "register_call_inplace_ms": inplace}
    del Xi, Y
    # reference: the runtime's own device-to-device copy of the same tensor
    Xc = torch.empty_like(d["X"])
    xbytes = 2.0 * w.N * w.d * 2
    for cold in (False, True):
        Xc.copy_(d["X"])
        torch.cuda.synchronize()
        ms = timed(lambda: Xc.copy_(d["X"]), cold)
        out[f"torch_copy_s500_{'cold' if cold else 'warm'}"] = {
            "bytes": xbytes, "ms": ms, "gbs": xbytes / ms / 1e6}
    del Xc
    gamma = torch.full((w.d,), 0.5, dtype=torch.float32, device="cuda")
    Yr = d["X"].flip(0).contiguous()
    Z = torch.empty_like(d["X"])
    res_bytes = 3.0 * w.N * w.d * 2
    for cold in (False, True):
        S.residual(d["X"], Yr, gamma, Z=Z)
        torch.cuda.synchronize()
        ms = timed(lambda: S.residual(d["X"], Yr, gamma, Z=Z), cold)
        out[f"residual_s500_{'cold' if cold else 'warm'}"] = {
            "bytes": res_bytes, "ms": ms, "gbs": res_bytes / ms / 1e6}
    return out


def schedule_forward(w, spec, steps, warmup, ls=1e-5, graph=False):
    """ms per attention-only forward of `spec` and the peak device memory of
    the run (torch's allocator high-water mark: input, state, kept states,
    workspace and the weights of every block).  graph: also the forward
    captured once into a HIP graph (torch.cuda.CUDAGraph) and replayed, which
    removes the host launch cost of its ~400 kernels (into its own state
    buffer, after the memory figure is taken)."""
    import torch
    from vggt_global_attention_amd import schedule as S
    from vggt_global_attention_amd import synth
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    blocks = [{k: v.to("cuda") for k, v in b.items()}
              for b in synth.make_block_weights(w, 2 * spec.n_layers, ls)]
    wbytes = sum(t.numel() * t.element_size() for b in blocks for t in b.values())
    X = synth.make_inputs(w)["X"].to("cuda")
    sch = S.Schedule(X, w.H, w.grid_h, w.grid_w, blocks, spec)
    caches = sch.alloc_caches(X)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        sch(X, state=X, caches=caches)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        sch(X, state=X, caches=caches)     # in place: the state overwrites the input
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    peak = torch.cuda.max_memory_allocated() - base
    flop = 0.0
    for l in range(spec.n_layers):
        mode = spec.inter_mode(l)
        flop += w.flop("frame") + w.flop(mode, spec.merge if mode == "merged" else spec.sub)
    out = {"S": w.S, "N": w.N, "ms_per_forward": ms, "tflops": flop / ms / 1e9,
           "peak_bytes": peak, "peak_gb": peak / 1e9, "weights_bytes": wbytes,
           "state_bytes": X.numel() * 2, "caches_bytes": caches.numel() * 2,
           "workspace_bytes": sch.workspace.numel(), "flop_per_forward": flop,
           "inter_modes": [spec.inter_mode(l) for l in range(spec.n_layers)]}
    if graph:
        state = torch.empty_like(X)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            sch(X, state=state, caches=caches)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            sch(X, state=state, caches=caches)
        for _ in range(max(warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out["ms_per_forward_graph"] = e0.elapsed_time(e1) / steps
        del g, state
    del sch, caches, X, blocks
    torch.cuda.empty_cache()
    return out


def schedule_sweep(frames, steps, warmup, graph=False):
    from vggt_global_attention_amd import configs
    from vggt_global_attention_amd import schedule as S
    variants = {"vggt": S.ScheduleSpec(),
                # AVGGT: the first third of the layers as frame attention, the
                # remaining global layers subsampled with 3 x 3 windows
                "avggt_early8_sub3x3": S.ScheduleSpec(early_frame=8, sub=(3, 3)),
                # HTTM: every global layer with merging in blocks of 4 frames x
                # 2 x 3 cells, 12 of a block's 18 sources merged
                "httm_F4w2x3r12": S.ScheduleSpec(merge=(4, 2, 3, 12))}
    rows = []
    for n in frames:
        w = configs.custom(f"s{n}", S=n, grid_h=26, grid_w=39, d=1024, H=16, cid=70)
        for vname, spec in variants.items():
            print(f"[bench] schedule {vname} S={n}", file=sys.stderr, flush=True)
            st = steps if n <= 100 else 1
            r = schedule_forward(w, spec, st, min(warmup, 1) if n > 100 else warmup,
                                 graph=graph and n <= 100)
            r["variant"] = vname
            rows.append(r)
            gtxt = (f", graph replay {r['ms_per_forward_graph']:.1f} ms"
                    if "ms_per_forward_graph" in r else "")
            print(f"[bench]   {r['ms_per_forward']:.1f} ms{gtxt}, peak {r['peak_gb']:.2f} GB",
                  file=sys.stderr, flush=True)
    return rows


def power_run(w, d, steps):
    """Median socket power and shader clock, sampled with `amd-smi metric -p -c`
    from a thread, while the layer runs back to back: idle, on the workload's
    inputs, and on zero operands (Wqkv = 0, beta = 0: q = k = v = 0, every P
    equal) -- the same kernels and instruction stream with no operand
    toggling."""
    import statistics
    import subprocess
    import threading
    import time
    import torch
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                out = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"],
                                     capture_output=True, text=True, timeout=10).stdout
                g = json.loads(out)
                g = g["gpu_data"][0] if isinstance(g, dict) else g[0]
                clk = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_")]
                samples.append((time.time(), float(g["power"]["socket_power"]["value"]),
                                sum(clk) / len(clk)))
            except (OSError, ValueError, KeyError, IndexError, TypeError,
                    subprocess.SubprocessError):
                pass
            time.sleep(0.2)

    z = dict(d)
    z["Wqkv"] = torch.zeros_like(d["Wqkv"])
    z["q_beta"] = torch.zeros_like(d["q_beta"])
    z["k_beta"] = torch.zeros_like(d["k_beta"])
    th = threading.Thread(target=sample, daemon=True)
    th.start()
    rows = []
    for name, inp in (("idle", None), ("synthetic inputs", d), ("zero operands", z)):
        print(f"[bench] power: {name}", file=sys.stderr, flush=True)
        t0 = time.time()
        ms = core = None
        if inp is None:
            time.sleep(2.0)
        else:
            ms, core = time_block(w, "global", inp, steps, 3)
        t1 = time.time()
        sel = [s for s in samples if t0 + 0.5 < s[0] < t1 - 0.2]
        rows.append({"case": name, "ms_per_layer": ms, "core_ms": core, "samples": len(sel),
                     "socket_power_w": statistics.median(s[1] for s in sel) if sel else None,
                     "gfx_clock_mhz": statistics.median(s[2] for s in sel) if sel else None})
    stop.set()
    th.join()
    return rows


def host_info():
    """CPU model, logical CPUs and NumPy's BLAS, for the oracle timing."""
    import platform
    import numpy as np
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "blas": blas}


def cpu_baseline(w, inp, n_rows, outputs=None):
    """The fp64 oracle on a bounded sample of the same layer: k/v for all N
    tokens, then q, attention and output projection for n_rows query rows.
    outputs: {name: Y [S, T, d] on the host} of GPU calls on the same inputs,
    whose errors on the sampled rows are reported (relL1 = sum|err| /
    sum|ref|, max|err| / max|ref|, mean|err| / max|ref|)."""
    import numpy as np
    import torch
    import oracle
    from vggt_global_attention_amd import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    threads = max(1, min(threads, os.cpu_count() or 1))
    os.environ["ORACLE_THREADS"] = str(threads)
    p = oracle.OracleParams(
        Wqkv=inp["Wqkv"].to(torch.float64).numpy(), Wo=inp["Wo"].to(torch.float64).numpy(),
        q_gamma=inp["q_gamma"].double().numpy(), q_beta=inp["q_beta"].double().numpy(),
        k_gamma=inp["k_gamma"].double().numpy(), k_beta=inp["k_beta"].double().numpy(),
        H=w.H, grid_h=w.grid_h, grid_w=w.grid_w)
    X = inp["X"].to(torch.float64).numpy()
    rows = synth.sample_rows(w, n_rows).numpy()
    t0 = time.perf_counter()
    ref = oracle.global_attention_rows(X, p, rows, threads=threads)
    dt = time.perf_counter() - t0
    errors = {}
    for name, Y in (outputs or {}).items():
        y = Y.reshape(-1, w.d)[torch.from_numpy(rows)].to(torch.float64).numpy()
        err = np.abs(y - ref)
        errors[name] = {"relL1": float(err.sum() / np.abs(ref).sum()),
                        "max_over_max": float(err.max() / np.abs(ref).max()),
                        "mean_over_max": float(err.mean() / np.abs(ref).max())}
    n, d = w.N, w.d
    flop = 4.0 * n * d * d + len(rows) * (2.0 * d * d + 4.0 * n * d + 2.0 * d * d)
    full_s = dt * (w.flop("global") / flop)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host": host_info(),
            "sample": f"{w.name} global layer: k/v for all {n} tokens + {len(rows)} sampled query "
                      f"rows (q, attention over all keys, Wo); {flop / 1e12:.3f} TFLOP in {dt:.1f} s; "
                      f"full layer extrapolates to {full_s:.0f} s",
            "ms_per_step_extrapolated": full_s * 1e3,
            "sample_errors": errors}


def cpu_full():
    """Wall time of the fp64 oracle (all host threads) on whole workloads:
    tiny and s24 in frame and global mode, s500 in frame and register mode,
    the s100 global layer, and s300 global on 1,024 sampled query rows
    (extrapolated linearly in the rows)."""
    import oracle
    import torch
    from vggt_global_attention_amd import configs, synth
    threads = max(1, os.cpu_count() or 1)
    os.environ["ORACLE_THREADS"] = str(threads)
    runs = []
    for name, mode in (("tiny", "frame"), ("tiny", "global"), ("s24", "frame"), ("s24", "global"),
                       ("s500", "frame"), ("s500", "register"), ("s100", "global"),
                       ("s300", "global_rows")):
        w = configs.WORKLOADS[name]
        inp = synth.make_inputs(w)
        p = oracle.OracleParams(
            Wqkv=inp["Wqkv"].to(torch.float64).numpy(), Wo=inp["Wo"].to(torch.float64).numpy(),
            q_gamma=inp["q_gamma"].double().numpy(), q_beta=inp["q_beta"].double().numpy(),
            k_gamma=inp["k_gamma"].double().numpy(), k_beta=inp["k_beta"].double().numpy(),
            H=w.H, grid_h=w.grid_h, grid_w=w.grid_w)
        X = inp["X"].to(torch.float64).numpy()
        print(f"[bench] oracle {name} {mode}", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        if mode == "global_rows":
            rows = synth.sample_rows(w, 1024).numpy()
            oracle.global_attention_rows(X, p, rows, threads=threads)
            dt = time.perf_counter() - t0
            runs.append({"workload": name, "mode": "global", "seconds": dt,
                         "sample_rows": int(len(rows)),
                         "seconds_extrapolated": dt * w.N / len(rows)})
        else:
            getattr(oracle, f"{mode}_attention")(X, p, threads=threads)
            runs.append({"workload": name, "mode": mode, "seconds": time.perf_counter() - t0})
        print(f"[bench]   {runs[-1]['seconds']:.1f} s", file=sys.stderr, flush=True)
    return {"oracle_full": runs, "threads": threads, "host": host_info()}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1",
                          "requested_gpus": a.gpus}))
        sys.exit(2)
    import torch
    from vggt_global_attention_amd import configs
    from vggt_global_attention_amd import binding as B
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    B.lib()  # fails loudly without the HIP library
    if a.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n, "copies": 3}))
        return
    if a.hbm:
        print(json.dumps({"hbm_kernels": hbm_kernels(a.steps), "peak_gbs": PEAK_HBM_GBS}),
              flush=True)
        return
    if a.cpu_full:
        print(json.dumps(cpu_full()), flush=True)
        return
    if a.schedule:
        frames = [int(x) for x in a.schedule.split(",")]
        rows = schedule_sweep(frames, a.steps, a.warmup, graph=a.graph)
        print(json.dumps({"schedule_sweep": rows, "layers": 24,
                          "register_layers": [2, 6, 9, 14, 20], "cached_layers": [4, 11, 17, 23],
                          "shape": "T=1031 (26x39 patches + 17), d=1024, H=16, bf16 state",
                          "data": "synthetic (seeded; no trained weights)"}), flush=True)
        return
    w = configs.WORKLOADS[a.workload]
    sub = (1, 1)
    if a.mode == "subsampled":
        sub = tuple(int(x) for x in a.sub.lower().split("x"))
    elif a.mode == "merged":
        sub = tuple(int(x) for x in a.merge.split(","))
    print(f"[bench] generating inputs for {w.name} (S={w.S}, N={w.N})", file=sys.stderr, flush=True)
    inp, d = gpu_inputs(w)
    if a.power:
        print(json.dumps({"power": power_run(w, d, a.steps), "workload": w.name}), flush=True)
        return
    if a.descriptors:
        r = time_descriptor(w, d, a.descriptors, a.steps, a.warmup)
        r["workload"] = w.name
        print(json.dumps({"descriptor_attention": r}), flush=True)
        return
    if a.only_stage:
        ms = loop_stage(w, a.mode, d, a.only_stage, a.steps, sub)
        print(json.dumps({"stage": a.only_stage, "mode": a.mode, "workload": w.name,
                          "ms_per_iter_wall": ms}))
        return
    print(f"[bench] timing {a.mode} ({a.warmup} warmup + {a.steps} steps)", file=sys.stderr, flush=True)
    ms, core_ms = time_block(w, a.mode, d, a.steps, a.warmup, sub)
    # global layer: its output with fp16 and with bf16 attention operands, for
    # the error report of the CPU baseline leg (after the timed region)
    outputs = {}
    if a.mode == "global" and not a.no_cpu:
        from vggt_global_attention_amd import api
        args = (d["X"], d["Wqkv"], d["Wo"], d["q_gamma"], d["q_beta"], d["k_gamma"], d["k_beta"])
        for ops in ("fp16", "bf16"):
            blk = api.Block("global", d["X"], w.H, w.grid_h, w.grid_w, operands=ops)
            outputs[f"{ops}_operands"] = blk(*args).cpu()
            del blk
        torch.cuda.empty_cache()
    flop = w.flop(a.mode, sub)
    attn_flop = w.attention_flop(a.mode, sub)
    achieved = attn_flop / (core_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": flop / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in/out; bf16 MFMA projections, fp16 MFMA attention, fp32 accumulate",
        "data": "synthetic (seeded; no trained weights)",
        "config": {"workload": f"{a.mode} attention layer, S={w.S} frames x T={w.T} tokens "
                               f"({w.grid_h}x{w.grid_w} patches + 17 special), N={w.N}, "
                               f"d={w.d}, H={w.H}, Dh={w.Dh}",
                   "S": w.S, "T": w.T, "N": w.N, "d": w.d, "H": w.H, "mode": a.mode,
                   "flop_per_step": flop},
        "frac_of_peak": flop / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "attn_kernel (attention core)",
                     "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_TFLOPS,
                     "traffic": recorded_traffic() if (a.workload, a.mode) == ("s100", "global") else None,
                     "traffic_unit": "bytes per launch (FETCH_SIZE*2.0 + WRITE_SIZE*1.0)",
                     "flop_per_launch": attn_flop, "ms_per_launch": core_ms},
    }
    if a.mode == "merged":
        out["config"]["merge"] = list(sub)
        out["config"]["merged_tokens"] = w.merged_tokens(*sub)
        out["roofline"]["kernel"] = "CORE stage: merge + attn_kernel<W> + unmerge"
    if a.mode == "subsampled":
        out["config"]["sub"] = list(sub)
        out["config"]["kept_keys"] = w.kept_keys(*sub)
        out["roofline"]["kernel"] = "CORE stage: K/V gather + discarded sums + attn_kernel<SGA>"
    if not a.no_extra and a.workload == "s100" and a.mode == "global":
        extra = {}
        httm = (4, 2, 3, 12)   # 4-frame runs, 2 x 3 windows, 12 of 18 sources merged
        # (mode, sub / merge parameters, attention operand type)
        runs = (("s24", (("global", (1, 1), "fp16"), ("frame", (1, 1), "fp16"))),
                ("s500", (("frame", (1, 1), "fp16"), ("frame", (1, 1), "bf16"),
                          ("register", (1, 1), "fp16"), ("register", (1, 1), "fp16", "inplace"))),
                ("s100", (("global", (1, 1), "bf16"), ("subsampled", (3, 3), "fp16"),
                          ("merged", httm, "fp16"))),
                ("s300", (("global", (1, 1), "fp16"), ("subsampled", (3, 3), "fp16"),
                          ("merged", httm, "fp16"))))
        for name, modes in runs:
            ww = configs.WORKLOADS[name]
            dd = d if name == a.workload else gpu_inputs(ww)[1]
            for mode, esub, ops, *flags in modes:
                print(f"[bench] extra {name} {mode} {esub} {ops} {' '.join(flags)}", file=sys.stderr,
                      flush=True)
                m2, c2 = time_block(ww, mode, dd, max(3, a.steps // 2), 2, esub, operands=ops,
                                    inplace="inplace" in flags)
                key = f"{name}_{mode}"
                if mode == "subsampled":
                    key += f"{esub[0]}x{esub[1]}"
                elif mode == "merged":
                    key += "_F{}w{}x{}r{}".format(*esub)
                if ops == "bf16":
                    key += "_bf16ops"
                if "inplace" in flags:
                    key += "_inplace"
                # merged mode: FLOP of the attention over the merged tokens
                # (the merge and unmerge kernels run inside core_ms)
                extra[key] = {"ms_per_layer": m2, "tflops": ww.flop(mode, esub) / m2 / 1e9,
                              "core_ms": c2,
                              "core_tflops": ww.attention_flop(mode, esub) / c2 / 1e9}
                if mode == "subsampled":
                    extra[key]["kept_keys"] = ww.kept_keys(*esub)
                if mode == "merged":
                    extra[key]["merged_tokens"] = ww.merged_tokens(*esub)
                if key.endswith("register_inplace") and key[:-len("_inplace")] in extra:
                    # the patch-row copy: the out-of-place call minus the in-place one
                    # (HBM-bound; 2 bytes read + 2 written per patch element)
                    pb = 4.0 * ww.S * (ww.T - 17) * ww.d
                    pm = extra[key[:-len("_inplace")]]["ms_per_layer"] - m2
                    extra[f"{name}_register_patch_copy"] = {"bytes": pb, "ms": pm,
                                                           "gbs": pb / pm / 1e6 if pm > 0 else None,
                                                           "peak_gbs": 8000.0}
            if dd is not d:
                del dd
            torch.cuda.empty_cache()
        # one GPU's share of a query-row split over 8 GPUs: N/8 queries, all N keys
        share = (w.N + 7) // 8
        print("[bench] extra s100 global rows share 1/8", file=sys.stderr, flush=True)
        m2, c2 = time_block(w, "global", d, max(3, a.steps // 2), 2, rows=(3 * share, share))
        attn = 4.0 * share * w.N * w.d
        gemm = 4.0 * w.N * w.d ** 2 + 4.0 * share * w.d ** 2  # k, v for all; q and Wo for the share
        extra["s100_global_rows_share1of8"] = {"ms_per_layer": m2, "tflops": (attn + gemm) / m2 / 1e9,
                                               "core_ms": c2, "core_tflops": attn / c2 / 1e9,
                                               "query_rows": share, "key_rows": w.N}
        print("[bench] extra s100 descriptor attention, 64 per frame", file=sys.stderr, flush=True)
        extra["s100_descriptor64"] = time_descriptor(w, d, 64, max(3, a.steps // 2), 2)
        from vggt_global_attention_amd import schedule as S
        print("[bench] extra s100 24-layer attention-only forward", file=sys.stderr, flush=True)
        del d
        torch.cuda.empty_cache()
        r = schedule_forward(w, S.ScheduleSpec(), 2, 1)
        extra["s100_schedule24"] = {k: r[k] for k in ("ms_per_forward", "tflops", "peak_gb",
                                                      "flop_per_forward")}
        out["extra"] = extra
    if not a.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_rows, outputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
