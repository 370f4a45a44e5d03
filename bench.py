#!/usr/bin/env python3
"""Decode-step benchmark of HOT/COLD cascade attention on one MI355X.

One step = the whole hot path over one batch: one COLD append per request
(host allocator), copy-on-write page copies (none without forks), per-step
dispatch, then cascade attention (bf16 MFMA prefix contraction over the HOT
slab, paged suffix pass over COLD, log-sum-exp merge) with the step's new
K/V fused in: the paged pass reads each request's new token from the step's
K/V tensor, and the merge lands it in its slot and advances the device block
tables and lengths (spkv_decode_step_append; --separate-append uses one
spkv_append_tokens launch before spkv_decode_step instead).  Inputs are
seeded synthetic tensors already resident in HBM.

Default workload: the Llama-3.1-8B-shaped layer (B = 64, Hq = 32, Hkv = 8,
d = 128, bf16, Lp = 16384, Ls ~ U[256, 2048] growing by one token per step,
COLD page size 1 with shuffled slots).

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: the library runs the
step on one GPU.
"""
from __future__ import annotations

import argparse
import gc
import json
import subprocess
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "cascade decode-attn KV-tokens/s per step + % HBM roofline, Lp=16K 8B shape"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C1", choices=["C0", "C1", "C2", "C3", "C4"])
    ap.add_argument("--lp", type=int, default=None, help="override the prefix length (C3 sweep)")
    ap.add_argument("--mode", default="step", choices=["step", "cascade", "dense"],
                    help="step: dispatcher decides (default); cascade/dense: force a backend")
    ap.add_argument("--page-size", type=int, default=None, help="override the COLD page size")
    ap.add_argument("--contiguous", action="store_true", help="COLD pages handed out in order (no shuffle)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing sample")
    ap.add_argument("--cold-runs", type=int, default=50,
                    help="timed runs of the cold-cache protocol (0: skip); 10 untimed runs precede them")
    ap.add_argument("--flush-mib", type=int, default=1024, help="bytes written before each cold-cache run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-launch", type=int, default=1, choices=(0, 1, 2),
                    help="spkv_dispatch_params.single_launch of the timed steps")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured read and MFMA ceilings (spkv_probe_read / spkv_probe_mfma)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM traffic per launch (written by profile_step.py)")
    ap.add_argument("--sweep-lp", default=None, metavar="L1,L2,...",
                    help="time cascade and dense attention at each prefix length (C3 crossover sweep) and exit")
    ap.add_argument("--sweep-batch", default=None, metavar="B1,B2,...",
                    help="time cascade and dense attention at each number of requests sharing the prefix "
                         "(at the configuration's or --lp's prefix length) and exit")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="after the timed steps, this many steps through the HIP-graph entry point "
                         "(spkv_graph_decode_step_append), timed the same way (0: skip)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append the step's K/V with its own launch (spkv_append_tokens) before the decode step")
    ap.add_argument("--layers", type=int, default=1,
                    help="with L > 1: a decode step over L layers (one layer-strided HOT and COLD allocation, "
                         "shared slots); own JSON line")
    ap.add_argument("--admission-sweep", default=None, metavar="F1,F2,...",
                    help="time the multi-agent batch with the HOT pool at each fraction of the total prefix "
                         "length (groups that do not fit fall back to COLD) and exit")
    ap.add_argument("--layout-study", action="store_true",
                    help="time the prefix storage layouts (HOT slab cascade / HOT slab flat / private COLD copies) and exit")
    ap.add_argument("--layout-batch", type=int, default=256, help="requests sharing the prefix in --layout-study")
    ap.add_argument("--layout-variant", default=None, choices=["hot_cascade", "hot_flat", "private_flat"],
                    help="only this variant of --layout-study (one per counter run)")
    ap.add_argument("--multistep", action="store_true",
                    help="the multi-agent run (C4 recipe): 32 decode steps with forks at step 8 and releases at "
                         "step 24, per-group vs batch-global dispatch, COLD page size 1 and 16; one JSON line")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 5 times (counter calibration) and exit")
    ap.add_argument("--other-configs", default="C2,C3@16384,C4", metavar="LIST",
                    help="configurations also measured (in child processes, short runs) by the default C1 step "
                         "run and reported under 'other_configs'; 'none' for none")
    return ap.parse_args()


def other_configs(args, ceilings=None) -> dict:
    """Short step-mode runs of further configurations, each in a child process
    (its own pools and GPU context, one after the other): per configuration
    ms per step, GPU ms per step, KV-tokens/s, the launches' durations and
    fractions, and the step roofline."""
    res = {}
    for item in [x for x in args.other_configs.split(",") if x and x != "none"]:
        cfg, _, lp = item.partition("@")
        cmd = [sys.executable, os.path.abspath(__file__), "--config", cfg, "--mode", "step", "--steps", "10",
               "--warmup", "3", "--no-cpu-baseline", "--cold-runs", "0", "--graph-steps", "0", "--other-configs", "none",
               "--no-ceilings", "--single-launch", str(args.single_launch)]
        if lp:
            cmd += ["--lp", lp]
        print(f"[bench] other configuration {item}", file=sys.stderr, flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            res[item] = {"error": f"exit {r.returncode}", "stderr_tail": r.stderr[-400:]}
            continue
        d = json.loads(lines[-1])
        res[item] = {"workload": d["config"]["workload"], "ms_per_step": d["ms_per_step"],
                     "gpu_ms_per_step": d["gpu_ms_per_step"], "value": d["value"], "unit": d["unit"],
                     "kernels": {k: {f: v[f] for f in ("avg_us", "hbm_frac", "mfma_frac") if f in v}
                                 for k, v in d["kernels"].items()},
                     "roofline": {k: d["roofline"].get(k) for k in ("kernel", "bound", "frac", "traffic_frac")},
                     "step_roofline": d["step_roofline"]["frac"],
                     "two_launches_gpu_ms_per_step": (d.get("two_launches") or {}).get("gpu_ms_per_step")}
        if ceilings:
            for k, v in d["kernels"].items():
                res[item]["kernels"][k]["frac_of_read_ceiling"] = round(v["gbps"] / ceilings["read_gbps"], 4)
    return res


def copy_probe(mib: int) -> int:
    """A plain device-to-device copy of known size: MIB MiB read and MIB MiB written per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
    return 0


def measure_ceilings(torch, R, read_mib: int = 4096, reps: int = 10, mfma_iters: int = 20000):
    """What this device achieves beside its published peaks: the best of
    `reps` launches of a streaming read over `read_mib` MiB (well beyond the
    caches) and of a bf16 MFMA loop on every SIMD, each timed with events on
    the current stream (the one the probes launch on)."""
    from shared_prefix_paged_amd import lib as _lib
    import ctypes as C
    cus = C.c_int32()
    R.check(_lib.spkv_device_cus(C.byref(cus)))
    buf = torch.empty(read_mib << 20, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    sink = torch.zeros(int(cus.value) * 16 * 4, dtype=torch.int32, device="cuda:0")   # a word per wave
    waves = int(cus.value) * 8                   # two waves per SIMD
    fsink = torch.empty(waves, dtype=torch.float32, device="cuda:0")

    def best_ms(launch):
        launch()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    read_ms = best_ms(lambda: R.probe_read(buf, sink))
    mfma_ms = best_ms(lambda: R.probe_mfma(waves, mfma_iters, fsink))
    torch.cuda.synchronize()
    nbytes = buf.numel()
    flops = 8.0 * 32 * 32 * 16 * 2 * waves * mfma_iters
    del buf
    return {"read_gbps": round(nbytes / read_ms / 1e6, 1), "read_bytes": nbytes,
            "mfma_bf16_tflops": round(flops / mfma_ms / 1e9, 1), "mfma_waves": waves, "mfma_iters": mfma_iters,
            "note": f"best of {reps} launches each: spkv_probe_read (block-contiguous 32 KB chunks, 8 "
                    f"nontemporal 16-byte loads in flight per lane, 16 blocks of 256 per CU, a plain store per "
                    f"wave) and spkv_probe_mfma (8 independent "
                    f"32x32x16 bf16 MFMA chains per wave, 2 waves per SIMD)"}


def quiet_gc() -> None:
    """Collect once, then keep every object alive so far out of later
    collections: a full collection over the setup's objects otherwise stalls
    the host for tens of ms inside a timed region (the GPU queue runs dry)."""
    gc.collect()
    gc.freeze()


def sweep_lp(args) -> int:
    """Attention time of both backends (forced) and the dispatcher's choice at
    each prefix length (--sweep-lp) or at each number of requests sharing the
    prefixes (--sweep-batch, at the configuration's or --lp's prefix length);
    one JSON line.  Same workload recipe at every point (the configuration's
    heads and suffix-length distribution)."""
    import numpy as np
    import torch
    import workloads as W
    from shared_prefix_paged_amd import runtime as R
    from shared_prefix_paged_amd import _abi as A
    from hip_setup import setup_single_step

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg0 = W.CONFIGS[args.config]
    rows = []
    if args.sweep_batch:
        points = [(args.lp, int(x)) for x in args.sweep_batch.split(",")]
    else:
        points = [(int(x), None) for x in args.sweep_lp.split(",")]
    for lp, nb in points:
        wl = W.make_workload(cfg0, prefix_len=lp, batch=nb, extra_steps=4)
        cfg = wl.cfg
        st = setup_single_step(wl, device=dev)
        B = wl.batch
        out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
        lse = torch.empty((B, cfg.num_q_heads), dtype=torch.float32, device=dev)
        ws = torch.empty(st.batch.workspace_size(), dtype=torch.uint8, device=dev)
        G = cfg.num_q_heads // cfg.num_kv_heads
        rec = {"lp": int(max(wl.group_prefix_len)) if len(wl.group_prefix_len) else 0, "batch": B,
               "m_eff": int(max(np.bincount(wl.group_of[wl.group_of >= 0])) * G) if (wl.group_of >= 0).any() else 0,
               "kv_tokens": int(sum(wl.prefix_len_of(b) + int(wl.suffix_len[b]) for b in range(B)))}
        for name, mode in (("cascade", A.SPKV_MODE_FORCE_CASCADE), ("dense", A.SPKV_MODE_FORCE_DENSE),
                           ("dispatch", A.SPKV_MODE_PER_GROUP)):
            params = R.default_params(mode)
            quiet_gc()
            for _ in range(3):
                _, _, choice = R.decode_step(st.batch, st.pools, params, ws, out, lse)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = max(1, args.steps)
            e0.record()
            for _ in range(n):
                R.decode_step(st.batch, st.pools, params, ws, out, lse)
            e1.record()
            torch.cuda.synchronize()
            rec[f"{name}_us"] = round(1e3 * e0.elapsed_time(e1) / n, 2)
            if name == "dispatch":
                rec["dispatch_choice"] = "cascade" if len(choice) and choice[0] else "dense"
        rec["best"] = "cascade" if rec["cascade_us"] < rec["dense_us"] else "dense"
        print(f"[sweep] {json.dumps(rec)}", file=sys.stderr, flush=True)
        rows.append(rec)
        del st, ws, out, lse
        torch.cuda.empty_cache()
    key = "batch" if args.sweep_batch else "lp"
    cross = [r[key] for r in rows if r["best"] == "cascade"]
    print(json.dumps({"metric": f"attention time per step, cascade vs dense, by {'batch' if key == 'batch' else 'prefix length'}",
                      "unit": "us", "config": {"workload": f"{args.config} recipe, {key} swept",
                                               "steps_per_point": max(1, args.steps)},
                      "rows": rows, f"cascade_wins_from_{key}": min(cross) if cross else None,
                      "dispatch_agrees": all(r["dispatch_choice"] == r["best"] for r in rows)}), flush=True)
    return 0


def layout_study(args) -> int:
    """The storage layout in isolation, at B requests sharing an Lp-token
    prefix (Llama-3.1-8B layer shape): the prefix stored once in the HOT slab
    and read once by the prefix contraction (cascade); stored once but
    re-read for every request by the paged pass (flat over the shared rows);
    and copied into every request's own COLD pages (flat over private copies,
    the layout of a pool without a shared level).  Warm and cold-cache
    attention times and algorithmic bytes; one JSON line.  Timing only: pool
    contents are random on the device (the paths are parity-tested on the
    oracle's inputs elsewhere)."""
    import numpy as np
    import torch
    from shared_prefix_paged_amd import runtime as R
    from shared_prefix_paged_amd import _abi as A

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, d = args.layout_batch, 32, 8, 128
    Lp = args.lp or 8192
    kvb = 2 * Hkv * d * 2
    rng = np.random.Generator(np.random.PCG64(105))
    ls = rng.integers(256, 2048, size=B, endpoint=True).astype(np.int64)   # COLD suffix per request
    gen = torch.Generator(device=dev)
    gen.manual_seed(105)
    q = torch.randn((B, Hq, d), generator=gen, device=dev).to(torch.bfloat16)

    def build(private: bool):
        lengths = ls + (Lp if private else 0)
        pages = int(lengths.sum()) + 32 * B
        cp = R.ColdPool(pages, 1, rng.permutation(pages).astype(np.int32))   # shuffled P = 1 slots
        seqs = [cp.seq_new() for _ in range(B)]
        for t in range(int(lengths.max())):
            cp.append_batch([s for s, n in zip(seqs, lengths) if n > t])
        tables, lens = cp.block_tables(seqs, int(lengths.max()))
        pools = R.KVPools.allocate(1 if private else Lp, pages, Hkv, d, torch.bfloat16, dev)
        for t in (pools.k_hot, pools.v_hot, pools.k_cold, pools.v_cold):
            t.normal_(generator=gen)
        if private:
            batch = R.DecodeBatch(q, [-1] * B, [], [], tables, lens, 1, Hkv)
        else:
            batch = R.DecodeBatch(q, [0] * B, [0], [Lp], tables, lens, 1, Hkv)
        return cp, pools, batch

    variants = {"hot_cascade": (False, A.SPKV_MODE_FORCE_CASCADE),
                "hot_flat": (False, A.SPKV_MODE_FORCE_DENSE),
                "private_flat": (True, A.SPKV_MODE_FORCE_DENSE)}
    pick = [args.layout_variant] if args.layout_variant else list(variants)
    scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
    clean = torch.zeros(args.flush_mib << 20, dtype=torch.uint8, device=dev)
    attn_ids = (A.SPKV_KERNEL_PREFIX, A.SPKV_KERNEL_FLAT, A.SPKV_KERNEL_MERGE, A.SPKV_KERNEL_PAGED_PREFIX)
    kname = {A.SPKV_KERNEL_PREFIX: "prefix_mfma", A.SPKV_KERNEL_FLAT: "flat_paged", A.SPKV_KERNEL_MERGE: "merge",
             A.SPKV_KERNEL_PAGED_PREFIX: "paged_prefix"}
    res = {}
    built = {}
    for name in pick:
        private, mode = variants[name]
        if private not in built:
            built.clear()
            torch.cuda.empty_cache()
            built[private] = build(private)
        cp, pools, batch = built[private]
        params = R.default_params(mode)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(batch.workspace_size(), dtype=torch.uint8, device=dev)
        quiet_gc()
        for _ in range(3):
            R.decode_step(batch, pools, params, ws, out, lse)
        torch.cuda.synchronize()
        with R.KernelTimer() as kt:
            for _ in range(args.steps):
                R.decode_step(batch, pools, params, ws, out, lse)
            torch.cuda.synchronize()
            per = {k: kt.read(k) for k in attn_ids}
        warm = 1e3 * sum(v[0] for v in per.values()) / args.steps
        cold = []
        for i in range(args.cold_runs):
            scratch.fill_(i & 1)
            clean.view(torch.int64).sum()
            torch.cuda.synchronize()
            with R.KernelTimer() as kc:
                R.decode_step(batch, pools, params, ws, out, lse)
                torch.cuda.synchronize()
                cold.append(1e3 * sum(kc.read(k)[0] for k in attn_ids))
        assert torch.isfinite(out).all()
        tokens = int(B * Lp + ls.sum())
        stored = (Lp if not private else B * Lp) * kvb            # prefix bytes held in HBM
        read = (Lp if mode == A.SPKV_MODE_FORCE_CASCADE else B * Lp) * kvb + int(ls.sum()) * kvb
        res[name] = {"warm_us": round(warm, 2), "cold_median_us": round(float(np.median(cold)), 2) if cold else None,
                     "kernels_us": {kname[k]: round(1e3 * v[0] / max(1, v[1]), 2) for k, v in per.items() if v[1]},
                     "kv_bytes_read": read, "prefix_bytes_stored": stored,
                     "kv_tokens_per_s_warm": round(tokens / (warm * 1e-6), 1)}
        print(f"[layout] {name}: {json.dumps(res[name])}", file=sys.stderr, flush=True)
        del ws, out, lse
    print(json.dumps({"metric": "attention time per step by prefix storage layout", "unit": "us",
                      "config": {"workload": f"B={B} requests sharing Lp={Lp}, Hq={Hq}, Hkv={Hkv}, d={d}, bf16, "
                                             "Ls~U[256, 2048], shuffled P = 1 COLD slots",
                                 "steps": args.steps, "cold_runs": args.cold_runs,
                                 "flush_bytes": args.flush_mib << 20},
                      "variants": res}), flush=True)
    return 0


def multi_layer(args) -> int:
    """A decode step over L layers of one model, the layers sharing one HOT
    and one COLD allocation with the GraniKV paper's layer stride (Section
    3.2: head h of layer l of a slab at row base*Hkv*L + l*Lp*Hkv + h*Lp; COLD
    layer-major with the same slots in every layer): one host append per step,
    one copy-on-write launch for all layers, then per layer the K/V write and
    the attention call.  The step touches L times one layer's K/V, far more
    than the caches hold, so nothing is reused from the previous step.  One
    JSON line: KV tokens attended per second over all layers, and per-layer
    times."""
    import numpy as np
    import torch
    import workloads as W
    from shared_prefix_paged_amd import runtime as R
    from shared_prefix_paged_amd import _abi as A
    from hip_setup import setup_single_step, to_device

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    L = args.layers
    total_steps = args.warmup + 2 * args.steps + 1
    wl = W.make_workload(W.CONFIGS[args.config], prefix_len=args.lp, page_size=args.page_size,
                         extra_steps=max(32, total_steps + 1))
    cfg = wl.cfg
    B, Hq, Hkv, d, P = wl.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    st = setup_single_step(wl, device=dev, max_blocks=(int(wl.suffix_len.max()) + total_steps + P - 1) // P + 1,
                           num_layers=L)
    batch, cold, pools = st.batch, st.cold, st.pools
    per_layer = [pools.at_layer(li) for li in range(L)]
    cold_views = [pools.cold_layer(li) for li in range(L)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(106)
    qs = [torch.randn((B, Hq, d), generator=gen, device=dev).to(pools.k_cold.dtype) for _ in range(L)]
    kv_new = []
    for s_ in range(total_steps):
        dr = W.step_draws(cfg, s_, B)
        kv_new.append((to_device(dr.k_new, cfg.dtype, dev), to_device(dr.v_new, cfg.dtype, dev)))
    seqs = np.asarray(st.seqs, dtype=np.int32)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(batch.workspace_size(), dtype=torch.uint8, device=dev)
    params = R.default_params(A.SPKV_MODE_PER_GROUP)
    lp_of = np.array([wl.prefix_len_of(b) for b in range(B)], dtype=np.int64)
    mb = batch.max_blocks
    state = {"i": 0}

    def one_step():
        i = state["i"]
        slots, cows = cold.append_batch(seqs)
        k, v = kv_new[i]
        if cows:                                   # one launch copies the pages in every layer
            R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device=dev), pools.k_cold, pools.v_cold,
                          cold.num_pages, P, Hkv, d, num_layers=L)
        for li in range(L):
            kc, vc = cold_views[li]
            # layer 0 also appends to the (shared) device block tables and lengths
            R.append_tokens(k, v, slots, kc, vc, pools.cold_slots, P, Hkv, d,
                            tables=batch.tables if li == 0 else None, max_blocks=mb if li == 0 else 0,
                            lens=batch.lens if li == 0 else None)
        batch.lens_h += 1
        for li in range(L):
            batch.struct.q = qs[li].data_ptr()
            R.decode_step(batch, per_layer[li], params, ws, out, lse)
        state["i"] = i + 1
        return L * int(np.sum(lp_of + batch.lens_h))

    quiet_gc()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tokens = 0
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        tokens += one_step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    with R.KernelTimer() as kt:
        for _ in range(args.steps):
            one_step()
        torch.cuda.synchronize()
        per = {name: kt.read(k) for name, k in (("prefix_mfma", A.SPKV_KERNEL_PREFIX), ("flat_paged", A.SPKV_KERNEL_FLAT),
                                                ("paged_prefix", A.SPKV_KERNEL_PAGED_PREFIX),
                                                ("merge", A.SPKV_KERNEL_MERGE), ("append", A.SPKV_KERNEL_CACHE))}
    assert torch.isfinite(out).all()
    print(json.dumps({
        "metric": f"decode-step attention over {L} layers, KV-tokens/s", "value": round(tokens / wall, 1),
        "unit": "KV-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 4), "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "us_per_layer": round(1e3 * gpu_ms / args.steps / L, 2), "higher_is_better": True, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} layer shape x {L} layers (one HOT and one COLD allocation, "
                               "layer-strided slabs, shared slots)",
                   "layers": L, "batch": B, "prefix_len": [int(x) for x in wl.group_prefix_len], "page_size": P},
        "kernels_avg_us": {k: round(1e3 * v[0] / v[1], 2) for k, v in per.items() if v[1]},
        "hbm_bytes_held": int(sum(t.numel() * t.element_size()
                                  for t in (pools.k_hot, pools.v_hot, pools.k_cold, pools.v_cold)))}), flush=True)
    return 0


def multistep(args) -> int:
    """The heterogeneous multi-agent run as the GraniKV paper measures it
    (Section 4.5 Table 4, Appendix B.8b Table 21: several prefix groups,
    per-group dispatch against one batch-global decision): the C4 recipe (8
    groups x 16 requests, Lp_g ~ U[2048, 16384], Ls ~ U[128, 4096], Llama-3.1-8B
    layer), 32 decode steps; before the appends of step 8 the first request of
    every group forks (COLD fork + HOT reference), at step 24 those parents are
    released; every step appends one token per live request (host allocator,
    copy-on-write copies, the new K/V fused into the step).  The schedule runs
    once per (page size, dispatch mode) from the same initial state, so both
    modes see identical pools.  Per run: attention time per step (sum of the
    attention kernels' event durations) and KV tokens attended; one JSON line.
    Timing only (the same schedule is parity-checked against the oracle by the
    GPU tests)."""
    import numpy as np
    import torch
    import workloads as W
    from shared_prefix_paged_amd import runtime as R
    from shared_prefix_paged_amd import _abi as A
    from hip_setup import setup_single_step, to_device

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    steps, fork_step, release_step = 32, 8, 24
    attn_ids = (A.SPKV_KERNEL_PREFIX, A.SPKV_KERNEL_FLAT, A.SPKV_KERNEL_MERGE, A.SPKV_KERNEL_PAGED_PREFIX)
    runs = {}
    for P in (1, 16):
        wl = W.make_workload(W.CONFIGS["C4"], page_size=P, extra_steps=40)
        cfg = wl.cfg
        B, Hq, Hkv, d = wl.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        mb = (int(wl.suffix_len.max()) + steps + P - 1) // P + 2
        draws = []
        n_live = B
        for s_ in range(steps):
            n_live += 8 if s_ == fork_step else (-8 if s_ == release_step else 0)
            dr = W.step_draws(cfg, s_, n_live)
            draws.append((to_device(dr.k_new, cfg.dtype, dev), to_device(dr.v_new, cfg.dtype, dev),
                          to_device(dr.q, cfg.dtype, dev)))
        for mode_name, mode in (("per_group", A.SPKV_MODE_PER_GROUP), ("batch_global", A.SPKV_MODE_BATCH_GLOBAL)):
            st = setup_single_step(wl, device=dev, max_blocks=mb)
            hot, cold, pools = st.hot, st.cold, st.pools
            group_of = {b: int(wl.group_of[b]) for b in range(B)}
            live = list(range(B))
            parents = []
            params = R.default_params(mode)
            out = torch.empty((B + 8, Hq, d), dtype=torch.float32, device=dev)
            lse = torch.empty((B + 8, Hq), dtype=torch.float32, device=dev)
            ws = None
            batch = None
            recs = []
            quiet_gc()
            for s_ in range(steps):
                if s_ == fork_step:
                    firsts = {}
                    for b in sorted(live):
                        firsts.setdefault(group_of[b], b)
                    for g in sorted(firsts):
                        c = cold.fork(firsts[g])
                        hot.incref(st.bases[g])
                        group_of[c] = g
                        live.append(c)
                        parents.append(firsts[g])
                if s_ == release_step:
                    for p in parents:
                        cold.release(p)
                        hot.decref(st.bases[group_of[p]])
                        live.remove(p)
                live.sort()
                if batch is None or s_ in (fork_step, release_step):
                    tables, lens = cold.block_tables(live, mb)
                    batch = R.DecodeBatch(draws[s_][2], [group_of[b] for b in live], st.bases, wl.group_prefix_len,
                                          tables, lens, P, Hkv)
                    ws = torch.empty(batch.workspace_size(), dtype=torch.uint8, device=dev)
                k_new, v_new, q = draws[s_]
                slots, cows = cold.append_batch(live)
                if cows:
                    R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device=dev), pools.k_cold, pools.v_cold,
                                  cold.num_pages, P, Hkv, d)
                batch.lens_h += 1
                batch.struct.q = q.data_ptr()
                n = len(live)
                with R.KernelTimer() as kt:
                    _, _, choice = R.decode_step_append(batch, pools, params, ws, k_new, v_new, slots, out[:n],
                                                        lse[:n])
                    torch.cuda.synchronize()
                    us = 1e3 * sum(kt.read(k)[0] for k in attn_ids)
                tokens = int(sum(int(wl.group_prefix_len[group_of[b]]) if group_of[b] >= 0 else 0 for b in live)
                             + int(batch.lens_h.sum()))
                recs.append({"step": s_, "live": n, "cow_pairs": len(cows), "groups_cascade": int(np.sum(choice)),
                             "attention_us": round(us, 2), "kv_tokens": tokens})
            assert torch.isfinite(out).all()
            t = np.array([r["attention_us"] for r in recs])
            tok = np.array([r["kv_tokens"] for r in recs])
            runs[f"P{P}/{mode_name}"] = {
                "mean_attention_us": round(float(t.mean()), 2),
                "kv_tokens_per_s": round(float(tok.sum() / (t.sum() * 1e-6)), 1),
                "steps_0_7_us": round(float(t[:fork_step].mean()), 2),
                "steps_8_23_us": round(float(t[fork_step:release_step].mean()), 2),
                "steps_24_31_us": round(float(t[release_step:].mean()), 2),
                "cow_pairs": int(sum(r["cow_pairs"] for r in recs)),
                "groups_cascade_per_step": sorted({r["groups_cascade"] for r in recs}),
                "per_step": recs}
            print(f"[multistep] P={P} {mode_name}: {runs[f'P{P}/{mode_name}']['mean_attention_us']} us/step "
                  f"{runs[f'P{P}/{mode_name}']['kv_tokens_per_s']:.3g} KV-tok/s", file=sys.stderr, flush=True)
            del st, batch, ws, out, lse
            torch.cuda.empty_cache()
    ratio = {f"P{P}": round(runs[f"P{P}/batch_global"]["mean_attention_us"] / runs[f"P{P}/per_group"]["mean_attention_us"], 3)
             for P in (1, 16)}
    print(json.dumps({"metric": "multi-agent decode: attention time per step, per-group vs batch-global dispatch",
                      "unit": "us", "config": {"workload": "C4 recipe: 8 groups x 16 requests, Lp_g~U[2048, 16384], "
                                                           "Ls~U[128, 4096], Hq=32, Hkv=8, d=128, bf16, shuffled slots; "
                                                           "32 steps, forks at 8, releases at 24"},
                      "speedup_per_group_over_batch_global": ratio, "runs": runs}), flush=True)
    return 0


def admission_sweep(args) -> int:
    """HOT admission under pressure, at the multi-agent shape (8 prefix groups
    x 16 requests, Lp_g ~ U[2048, 16384], Ls ~ U[128, 4096], the Llama-3.1-8B
    layer): the HOT pool holds a fraction f of the groups' total prefix
    length; groups are admitted first fit in group order, and a group that
    does not fit keeps its prefix in every member's own COLD pages (the COLD
    fallback) and takes the flat pass.  Per f: groups admitted, prefix bytes
    stored, attention time per step (per-group dispatch, warm), KV tokens/s.
    One JSON line.  Timing only: pool contents are random on the device."""
    import numpy as np
    import torch
    import workloads as W
    from shared_prefix_paged_amd import runtime as R
    from shared_prefix_paged_amd import _abi as A
    from shared_prefix_paged_amd import OutOfMemory

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS["C4"]
    B, Hq, Hkv, d, ng = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.num_groups
    kvb = 2 * Hkv * d * 2
    rng = np.random.Generator(np.random.PCG64(cfg.seed))    # the recipe's first draws: prefix, then suffix lengths
    lp = rng.integers(*cfg.prefix_range, size=ng, endpoint=True).astype(np.int64)
    ls = rng.integers(*cfg.suffix_range, size=B, endpoint=True).astype(np.int64)
    gof0 = np.minimum(np.arange(B) // (B // ng), ng - 1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(107)
    q = torch.randn((B, Hq, d), generator=gen, device=dev).to(torch.bfloat16)
    params = R.default_params(A.SPKV_MODE_PER_GROUP)
    rows = []
    for f in [float(x) for x in args.admission_sweep.split(",")]:
        cap = int(f * int(lp.sum()))
        hot = R.HotPool(max(cap, 1))
        bases = {}
        for g in range(ng):
            try:
                bases[g] = hot.alloc(int(lp[g]))
            except OutOfMemory:
                pass                                         # COLD fallback for this group
        admitted = sorted(bases)
        gid = {g: i for i, g in enumerate(admitted)}
        group_of = [gid.get(int(g), -1) for g in gof0]
        lengths = np.array([ls[b] + (0 if int(gof0[b]) in bases else lp[gof0[b]]) for b in range(B)], np.int64)
        pages = int(lengths.sum()) + 32 * B
        cp = R.ColdPool(pages, 1, rng.permutation(pages).astype(np.int32))
        seqs = [cp.seq_new() for _ in range(B)]
        for t in range(int(lengths.max())):
            cp.append_batch([sq for sq, n in zip(seqs, lengths) if n > t])
        tables, lens = cp.block_tables(seqs, int(lengths.max()))
        pools = R.KVPools.allocate(max(cap, 1), pages, Hkv, d, torch.bfloat16, dev)
        for t in (pools.k_hot, pools.v_hot, pools.k_cold, pools.v_cold):
            t.normal_(generator=gen)
        batch = R.DecodeBatch(q, group_of, [bases[g] for g in admitted], [int(lp[g]) for g in admitted], tables,
                              lens, 1, Hkv)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(batch.workspace_size(), dtype=torch.uint8, device=dev)
        quiet_gc()
        for _ in range(3):
            _, _, choice = R.decode_step(batch, pools, params, ws, out, lse)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            R.decode_step(batch, pools, params, ws, out, lse)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / args.steps
        assert torch.isfinite(out).all()
        tokens = int(lengths.sum() + sum(lp[g] for g in gof0 if int(g) in bases))
        rec = {"hot_fraction": f, "groups_admitted": len(admitted), "groups_cascade": int(np.sum(choice)),
               "hot_prefix_bytes": int(sum(lp[g] for g in admitted) * kvb),
               "private_prefix_bytes": int(sum(lp[gof0[b]] for b in range(B) if int(gof0[b]) not in bases) * kvb),
               "attention_us": round(us, 2), "kv_tokens_per_s": round(tokens / (us * 1e-6), 1)}
        print(f"[admission] {json.dumps(rec)}", file=sys.stderr, flush=True)
        rows.append(rec)
        del batch, pools, ws, out, lse, cp, hot
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "attention time per step by HOT pool size (COLD fallback for groups that do not fit)",
                      "unit": "us", "config": {"workload": f"{cfg.name} lengths: B={B}, {ng} groups, Hq={Hq}, "
                                                           f"Hkv={Hkv}, d={d}, bf16, shuffled P = 1 slots",
                                               "prefix_lengths": [int(x) for x in lp], "steps": args.steps},
                      "rows": rows}), flush=True)
    return 0


def source_digest() -> str:
    """Digest of the sources that decide what the kernels read and write
    (probes.hip holds only the measurement probes)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "shared_prefix_paged_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f == "probes.hip":
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str, config: str, mode: str, kernel: str):
    """HBM bytes per launch of `kernel` from calibrated FETCH_SIZE + WRITE_SIZE
    counters, if they were taken on the current sources; else None."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources") != source_digest():
        return None
    rec = t.get("runs", {}).get(f"{config}/{mode}", {}).get(kernel)
    return None if rec is None else rec.get("traffic_bytes")


def kv_bytes_per_token(hkv, d, esz):
    return 2 * hkv * d * esz


def main():
    args = parse()
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.sweep_lp or args.sweep_batch:
        return sweep_lp(args)
    if args.layout_study:
        return layout_study(args)
    if args.layers > 1:
        return multi_layer(args)
    if args.multistep:
        return multistep(args)
    if args.admission_sweep:
        return admission_sweep(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import workloads as W
    from shared_prefix_paged_amd import runtime as R
    from shared_prefix_paged_amd import _abi as A
    from hip_setup import setup_single_step, to_device

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.config]
    cold_warm = 10 if args.cold_runs > 0 else 0
    graph_steps = max(0, args.graph_steps)
    total_steps = args.warmup + 4 * args.steps + 1 + cold_warm + max(0, args.cold_runs) + \
        (graph_steps + 3 if graph_steps else 0)
    wl = W.make_workload(cfg, prefix_len=args.lp, page_size=args.page_size, extra_steps=max(32, total_steps + 1))
    if args.contiguous:
        wl.free_order = None
    cfg = wl.cfg
    B, Hq, Hkv, d, P = wl.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    esz = 2 if cfg.dtype == "bf16" else 4
    kvb = kv_bytes_per_token(Hkv, d, esz)
    max_len0 = int(wl.suffix_len.max())
    st = setup_single_step(wl, device=dev, max_blocks=(max_len0 + total_steps + P - 1) // P + 1)
    batch, pools, cold = st.batch, st.pools, st.cold
    mb = batch.max_blocks
    print(f"[bench] {cfg.name}: B={B} Hq={Hq} Hkv={Hkv} d={d} {cfg.dtype} Lp={list(wl.group_prefix_len)} "
          f"sum(Ls)={int(wl.suffix_len.sum())} P={P}", file=sys.stderr, flush=True)

    # Per-step inputs (fresh K/V of the decoded token, fresh Q), resident on the device.
    k_steps, v_steps, q_steps = [], [], []
    for s in range(total_steps):
        dr = W.step_draws(cfg, s, B)
        k_steps.append(to_device(dr.k_new, cfg.dtype, dev))
        v_steps.append(to_device(dr.v_new, cfg.dtype, dev))
        q_steps.append(to_device(dr.q, cfg.dtype, dev))
    seqs = np.asarray(st.seqs, dtype=np.int32)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(batch.workspace_size(), dtype=torch.uint8, device=dev)
    mode = {"step": A.SPKV_MODE_PER_GROUP, "cascade": A.SPKV_MODE_FORCE_CASCADE,
            "dense": A.SPKV_MODE_FORCE_DENSE}[args.mode]
    params = R.default_params(mode)
    params.single_launch = args.single_launch
    lp_of = np.array([wl.prefix_len_of(b) for b in range(B)], dtype=np.int64)
    state = {"i": 0, "choice": None}
    separate = args.separate_append or cfg.dtype != "bf16"     # the fused step is bf16 only

    host = {"append_s": 0.0, "call_s": 0.0, "n": 0}

    def one_step(flush=None, graph=None):
        i = state["i"]
        h0 = time.perf_counter()
        slots, cows = cold.append_batch(seqs)                       # host allocator
        host["append_s"] += time.perf_counter() - h0
        if cows:
            R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device=dev), pools.k_cold, pools.v_cold,
                          cold.num_pages, P, Hkv, d)
        if separate:
            # new K/V to their slots + device block tables, one launch (slots travel in the launch)
            R.append_tokens(k_steps[i], v_steps[i], slots, pools.k_cold, pools.v_cold, pools.cold_slots, P, Hkv, d,
                            tables=batch.tables, max_blocks=mb, lens=batch.lens)
        batch.lens_h += 1                                            # host mirror of the lengths
        batch.struct.q = q_steps[i].data_ptr()
        if flush is not None:
            flush()                                                  # outside the event window
        h1 = time.perf_counter()
        if graph is not None:
            _, _, choice, inst = graph.decode_step_append(batch, pools, params, ws, k_steps[i], v_steps[i], slots,
                                                          out, lse)
            state["instantiations"] = state.get("instantiations", 0) + int(inst)
        elif separate:
            _, _, choice = R.decode_step(batch, pools, params, ws, out, lse)
        else:
            _, _, choice = R.decode_step_append(batch, pools, params, ws, k_steps[i], v_steps[i], slots, out, lse)
        host["call_s"] += time.perf_counter() - h1                  # dispatch + plan + launches (asynchronous)
        host["n"] += 1
        state["choice"] = choice
        state["i"] = i + 1
        return int(np.sum(lp_of + batch.lens_h))                     # logical KV tokens attended

    quiet_gc()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    host.update(append_s=0.0, call_s=0.0, n=0)

    # ---- timed region: exactly `steps` steps --------------------------------
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tokens = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        tokens += one_step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / args.steps
    value = tokens / wall
    host_step = {"append_batch_us": round(1e6 * host["append_s"] / host["n"], 2),
                 "decode_call_us": round(1e6 * host["call_s"] / host["n"], 2)}
    # The dispatcher and the plan alone (host only, pure): the per-step
    # decision of the GraniKV paper's Section 3.6 and the split plan.
    reps = 2000
    hd0 = time.perf_counter()
    for _ in range(reps):
        R.dispatch(batch, params)
    hd1 = time.perf_counter()
    for _ in range(reps):
        batch.plan()
    hd2 = time.perf_counter()
    from shared_prefix_paged_amd import lib as _lib
    for _ in range(reps):
        _lib.spkv_version()
    hd3 = time.perf_counter()
    host_step["dispatch_us"] = round(1e6 * (hd1 - hd0) / reps, 3)
    host_step["plan_us"] = round(1e6 * (hd2 - hd1) / reps, 3)
    host_step["empty_ctypes_call_us"] = round(1e6 * (hd3 - hd2) / reps, 3)
    host_step["note"] = ("decode_call_us: host time of the spkv call that dispatches, plans and enqueues the step's "
                         "kernels (they run asynchronously); dispatch_us / plan_us: spkv_dispatch and "
                         "spkv_plan_query alone, each from Python through ctypes (call overhead included; "
                         "empty_ctypes_call_us is a call that does nothing, for comparison)")

    # ---- per-kernel durations from HIP events on the launch stream ----------
    # (the plan's per-request partial-state counts are recorded at every step
    # for the byte accounting below)
    per_step = []
    with R.KernelTimer() as kt:
        for _ in range(args.steps):
            one_step()
            choice = state["choice"]
            casc = list(map(int, choice)) if len(choice) else None
            fp, pp = batch.plan_parts(casc)
            per_step.append((batch.lens_h.copy(), fp, pp, [int(c) for c in choice]))
        torch.cuda.synchronize()
    kt_ms = {k: kt.read(k) for k in (A.SPKV_KERNEL_PREFIX, A.SPKV_KERNEL_FLAT, A.SPKV_KERNEL_MERGE,
                                     A.SPKV_KERNEL_CACHE, A.SPKV_KERNEL_PAGED_PREFIX)}
    # The same steps again with the paged pass and the prefix contraction as
    # two launches (params.single_launch = 0), when the step above ran them as
    # one: each kernel's own duration and roofline, beside the single launch's.
    # (GPU time per step without per-kernel events first, then the kernels.)
    kt2_ms, gpu2_ms = None, None
    if kt_ms[A.SPKV_KERNEL_PAGED_PREFIX][1] > 0:
        params.single_launch = 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            one_step()
        e1.record()
        torch.cuda.synchronize()
        gpu2_ms = e0.elapsed_time(e1) / args.steps
        with R.KernelTimer() as kt2:
            for _ in range(args.steps):
                one_step()
            torch.cuda.synchronize()
        kt2_ms = {k: kt2.read(k) for k in (A.SPKV_KERNEL_PREFIX, A.SPKV_KERNEL_FLAT, A.SPKV_KERNEL_MERGE)}
        params.single_launch = args.single_launch

    # ---- the same steps through the HIP-graph entry point: host time of the
    # call (record, update the graph's kernel nodes in place, launch) and GPU
    # time per step, next to the direct call's figures above.
    graph_res = None
    if graph_steps and not separate:
        g = R.StepGraph()
        for _ in range(3):
            one_step(graph=g)
        torch.cuda.synchronize()
        host.update(append_s=0.0, call_s=0.0, n=0)
        state["instantiations"] = 0
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tg = time.perf_counter()
        g0.record()
        for _ in range(graph_steps):
            one_step(graph=g)
        g1.record()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - tg
        graph_res = {"steps": graph_steps, "ms_per_step": round(1e3 * gwall / graph_steps, 4),
                     "gpu_ms_per_step": round(g0.elapsed_time(g1) / graph_steps, 4),
                     "graph_call_us": round(1e6 * host["call_s"] / host["n"], 2),
                     "direct_call_us": host_step["decode_call_us"],
                     "instantiations": int(state["instantiations"]),
                     "note": "graph_call_us: host time of spkv_graph_decode_step_append (record the step, update the "
                             "instantiated graph's kernel nodes, launch); instantiations: steps whose launches "
                             "differed from the graph's (re-instantiated instead of updated)"}
        g.close()

    # ---- cold-cache protocol: the last-level cache (256 MB) and the L2s are
    # flushed by a large write (then a read of another buffer, so the flush's
    # dirty lines are written back beforehand) before each timed run; the
    # flush completes before the attention call, and a run's time is the sum
    # of its attention kernels' event durations (host planning and the append
    # are outside it).
    cold_res = None
    if args.cold_runs > 0:
        scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
        clean = torch.zeros(args.flush_mib << 20, dtype=torch.uint8, device=dev)
        fill = [0]

        def flush():
            # the write evicts every cached line; reading a second buffer then
            # writes those dirty lines back and leaves clean ones, so no
            # write-back of the flush lands inside the timed window
            fill[0] ^= 1
            scratch.fill_(fill[0])
            clean.view(torch.int64).sum()

        for _ in range(cold_warm):
            one_step(flush)
        torch.cuda.synchronize()
        times, toks = [], []
        attn_ids = (A.SPKV_KERNEL_PREFIX, A.SPKV_KERNEL_FLAT, A.SPKV_KERNEL_MERGE, A.SPKV_KERNEL_PAGED_PREFIX)

        def flush_and_wait():
            flush()
            torch.cuda.synchronize()

        for _ in range(args.cold_runs):
            with R.KernelTimer() as ktc:
                toks.append(one_step(flush_and_wait))
                torch.cuda.synchronize()
                times.append(1e3 * sum(ktc.read(k)[0] for k in attn_ids))
        del scratch, clean
        t = np.array(times)
        med = float(np.median(t))
        cold_res = {"runs": args.cold_runs, "flush_bytes": args.flush_mib << 20,
                "median_us": round(med, 2), "p10_us": round(float(np.percentile(t, 10)), 2),
                "p90_us": round(float(np.percentile(t, 90)), 2),
                "kv_tokens_per_s": round(float(np.median(toks)) / (med * 1e-6), 1),
                "window": "sum of the attention kernels' event durations, after a write of flush_bytes "
                          "and a read of as many other bytes have completed",
                "warm_attention_us": None}
    choice = [int(c) for c in state["choice"]]
    n_casc = sum(choice)
    backend = "cascade" if choice and n_casc == len(choice) else ("dense" if n_casc == 0 else
                                                                  f"mixed: {n_casc} of {len(choice)} groups cascade")
    plan = batch.plan(choice if choice else None)

    # Algorithmic bytes / FLOPs of one launch, averaged over the profiled steps
    # (the lengths grow by one token per step).  Paged pass: K and V rows of
    # every token it attends, block-table entries of its COLD tokens, the
    # query rows once per partial state, and the partial states it writes.
    # Prefix pass: the HOT slab once, member queries, partial states.  Merge:
    # every partial state, then O and LSE.
    rows = B * Hq
    flat_b, prefix_b, prefix_f, merge_b = [], [], [], []
    for L, fp, pp, ch in per_step:
        # the per-group choice: members of a group that takes the flat pass read its prefix there
        flat_member = np.array([g >= 0 and not ch[g] for g in wl.group_of], dtype=bool)
        Lf = L + np.where(flat_member, lp_of, 0)
        part_bytes = Hq * int(fp.sum()) * (d + 1) * 4
        flat_b.append(int(Lf.sum()) * kvb + 4 * int(np.sum(-(-L // P))) + Hq * int(fp.sum()) * d * esz + part_bytes)
        pb = pf = ppart = 0.0
        if any(ch):
            for g, lp in enumerate(wl.group_prefix_len):
                members = np.flatnonzero(wl.group_of == g)
                if lp <= 0 or len(members) == 0 or not ch[g]:
                    continue
                npf = int(pp[members[0]])
                pb += int(lp) * kvb + len(members) * Hq * d * esz + len(members) * Hq * npf * (d + 1) * 4
                ppart += len(members) * Hq * npf * (d + 1) * 4
                pf += 4.0 * len(members) * Hq * int(lp) * d
        prefix_b.append(pb)
        prefix_f.append(pf)
        # (fused step: the merge also reads the new tokens' K/V and writes them to their slots)
        merge_b.append(part_bytes + ppart + rows * (d + 1) * 4 + (0 if separate else 2 * B * kvb))
    flat_bytes, prefix_bytes = float(np.mean(flat_b)), float(np.mean(prefix_b))
    prefix_flops, merge_bytes = float(np.mean(prefix_f)), float(np.mean(merge_b))

    # Launch classes: the paged pass and the prefix contraction as two
    # launches, or as one paged_prefix launch (both roles' bytes and FLOPs).
    classes = (("prefix_mfma", A.SPKV_KERNEL_PREFIX, prefix_bytes, prefix_flops),
               ("flat_paged", A.SPKV_KERNEL_FLAT, flat_bytes, 0.0),
               ("paged_prefix", A.SPKV_KERNEL_PAGED_PREFIX, flat_bytes + prefix_bytes, prefix_flops),
               ("merge", A.SPKV_KERNEL_MERGE, merge_bytes, 0.0))

    def kernel_table(ms_by_class):
        table = {}
        for name, kid, nbytes, flops in classes:
            if kid not in ms_by_class:
                continue
            ms, n = ms_by_class[kid]
            if n == 0:
                continue
            avg_us = 1e3 * ms / n
            table[name] = {"avg_us": round(avg_us, 3), "launches": n,
                           "alg_bytes": int(nbytes), "gbps": round(nbytes / avg_us / 1e3, 1),
                           "hbm_frac": round(nbytes / avg_us / 1e3 / HBM_PEAK_GBPS, 4)}
            if flops:
                table[name]["tflops"] = round(flops / avg_us / 1e6, 2)
                table[name]["mfma_frac"] = round(flops / avg_us / 1e6 / BF16_PEAK_TFLOPS, 4)
            tr = measured_traffic(args.traffic, traffic_key, args.mode, name)
            if tr:
                table[name]["traffic_bytes"] = int(tr)
                table[name]["traffic_frac"] = round(tr / avg_us / 1e3 / HBM_PEAK_GBPS, 4)
        return table

    traffic_key = args.config if args.lp is None else f"{args.config}@{args.lp}"
    kernels = kernel_table(kt_ms)
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    dk = kernels[dom]
    if dk.get("mfma_frac", 0.0) > dk["hbm_frac"]:
        roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(dk["tflops"] / BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        roofline = {"bound": "hbm", "achieved": dk["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(dk["gbps"] / HBM_PEAK_GBPS, 4), "traffic": None}
    roofline["kernel"] = dom
    two_launches = None
    if kt2_ms is not None:
        two_launches = {"kernels": kernel_table(kt2_ms), "gpu_ms_per_step": round(gpu2_ms, 4),
                        "note": "the same steps with spkv_dispatch_params.single_launch = 0: the paged pass and "
                                "the prefix contraction as separate launches (each kernel's own roofline)"}
    roofline["traffic"] = measured_traffic(args.traffic, traffic_key, args.mode, dom)
    if roofline["traffic"]:
        # HBM bytes the counters saw (L2 <-> fabric) over the same duration:
        # for the flat pass over a shared slab the algorithmic bytes count every
        # request's re-read of the prefix, most of which the caches serve.
        tg = roofline["traffic"] / dk["avg_us"] / 1e3
        roofline["traffic_gbps"] = round(tg, 1)
        roofline["traffic_frac"] = round(tg / HBM_PEAK_GBPS, 4)
    attn_us = sum(k["avg_us"] for k in kernels.values())
    if cold_res is not None:
        cold_res["warm_attention_us"] = round(attn_us, 2)
    # Step roofline: T* = sum over kernels of max(bytes / HBM peak, flops / MFMA peak).
    # Per role (the paged pass, the prefix contraction, the merge), whether
    # the first two ran as one launch or two.
    t_star = 0.0
    ran = set(kernels)
    for names, nbytes, flops in ((("prefix_mfma", "paged_prefix"), prefix_bytes, prefix_flops),
                                 (("flat_paged", "paged_prefix"), flat_bytes, 0.0),
                                 (("merge",), merge_bytes, 0.0)):
        if ran.intersection(names):
            t_star += max(nbytes / (HBM_PEAK_GBPS * 1e3), flops / (BF16_PEAK_TFLOPS * 1e6))
    step_roofline = {"t_star_us": round(t_star, 2), "t_measured_us": round(attn_us, 2),
                     "frac": round(t_star / attn_us, 4) if attn_us > 0 else None,
                     "note": "T* = sum over kernels of max(alg bytes / 8 TB/s, alg flops / 2.5 PFLOP/s); "
                             "T measured = sum of per-kernel event durations (warm)"}
    if cold_res is not None:
        cold_res["step_roofline_frac"] = round(t_star / cold_res["median_us"], 4)

    # ---- measured ceilings: each launch against what the device achieves ----
    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(torch, R)
        for tab in [kernels] + ([two_launches["kernels"]] if two_launches else []):
            for k in tab.values():
                k["frac_of_read_ceiling"] = round(k["gbps"] / ceilings["read_gbps"], 4)
                if "tflops" in k:
                    k["frac_of_mfma_ceiling"] = round(k["tflops"] / ceilings["mfma_bf16_tflops"], 4)
        roofline["measured_peak"] = ceilings["read_gbps"] if roofline["bound"] == "hbm" \
            else ceilings["mfma_bf16_tflops"]
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / roofline["measured_peak"], 4)

    # ---- oracle on the host cores, bounded sample ---------------------------
    cpu = cpu_1t = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)
        cpu_1t = cpu_baseline(wl, args.cpu_seconds / 2, threads=1)

    # ---- the other configurations (the default C1 step run only) ------------
    others = None
    if args.config == "C1" and args.lp is None and args.mode == "step" and args.other_configs not in ("", "none"):
        others = other_configs(args, ceilings)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one decode step, B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, {cfg.dtype}, "
                        f"Lp={list(map(int, wl.group_prefix_len))}, Ls~U{list(cfg.suffix_range)} (+1 per step), "
                        f"COLD page size {P}, {'contiguous' if args.contiguous else 'shuffled'} slots",
            "batch": B, "prefix_len": [int(x) for x in wl.group_prefix_len], "page_size": P,
            "slots": "contiguous" if args.contiguous else "shuffled",
            "backend": backend, "mode": args.mode,
            "append": "separate launch" if separate else "fused into the step",
        },
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "attention_us_per_step": round(attn_us, 2),
        "kv_tokens_per_s_attention": round(tokens / args.steps / (attn_us * 1e-6), 1),
        "kernels": kernels,
        "host": host_step,
        "two_launches": two_launches,
        "graph": graph_res,
        "plan": {f: int(getattr(plan, f)) for f, _ in plan._fields_},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "ceilings": ceilings,
        "cold_cache": cold_res,
        "cpu_baseline": cpu,
        "cpu_baseline_1t": cpu_1t,
        "other_configs": others,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(wl, budget_s: float, threads=None):
    """The oracle, untuned, on the host cores: fp64 attention per request
    (decode_request over the logical concatenation of prefix and suffix),
    cycling over the workload's requests until the budget is spent.  Each
    group's prefix is widened to float64 once, before the clock starts (it is
    shared by the group's requests); a request's own suffix and queries are
    widened inside the timed loop.  threads=1 limits the BLAS pools to one
    thread."""
    import contextlib
    from oracle.attention import decode_request, widen
    limit = contextlib.nullcontext()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        if threads is not None:
            limit = threadpool_limits(limits=threads)
        pool = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        pool = os.cpu_count() or 1
    cores = 1 if threads == 1 else min(pool, len(os.sched_getaffinity(0)))
    cfg = wl.cfg
    scale = 1.0 / float(cfg.head_dim) ** 0.5
    pk = [widen(k, cfg.dtype) for k in wl.prefix_k]
    pv = [widen(v, cfg.dtype) for v in wl.prefix_v]
    done, tokens = 0, 0
    order = list(range(wl.batch))
    with limit:
        t0 = time.perf_counter()
        while done == 0 or time.perf_counter() - t0 < budget_s:
            b = order[done % len(order)]
            g = int(wl.group_of[b])
            sk, sv = wl.suffix_kv(b)
            decode_request(widen(wl.q[b], cfg.dtype), pk[g] if g >= 0 else None, pv[g] if g >= 0 else None,
                           widen(sk, cfg.dtype), widen(sv, cfg.dtype), scale, cfg.group_size)
            tokens += wl.prefix_len_of(b) + int(wl.suffix_len[b])
            done += 1
        el = time.perf_counter() - t0
    return {"value": round(tokens / el, 1), "unit": "KV-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} requests ({done / wl.batch:.2f} passes over the {wl.batch} requests of the same "
                      f"workload, all query heads, prefix + suffix; each group's prefix widened to fp64 once "
                      f"beforehand), fp64 numpy, {el:.1f} s"}


if __name__ == "__main__":
    sys.exit(main())
