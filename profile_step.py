"""Profiles the decode step of bench.py with rocprofv3 (on a machine with the GPU).

    python profile_step.py [--config C1] [--lp N] [--mode step|cascade|dense] [--out DIR]

Runs, each as its own rocprofv3 process (program directly after ``--``, from
/tmp with TMPDIR=/tmp, under a hard time limit):

  1. ``--kernel-trace --stats`` over ``bench.py`` (the timed command itself);
  2. ``--pmc FETCH_SIZE`` and 3. ``--pmc WRITE_SIZE`` over a short bench run;
  4./5. the same two counters over ``bench.py --copy-probe 256``, a plain
     device copy that reads and writes 256 MiB, to turn counter readings into
     bytes (factor = known bytes / counter reading);
  6./7. two passes of shader-sequencer counters over a short bench run: MFMA
     busy cycles and bf16 MFMA operations (the prefix contraction), VALU, LDS
     and bank-conflict cycles (every kernel).

Writes ``profiles/<config>_<mode>_kernel_stats.md`` (per-kernel durations),
``profiles/<config>_<mode>_traffic.md`` (counter readings, factors, bytes per
launch), ``profiles/<config>_<mode>_counters.md`` (MFMA and LDS counters)
and updates ``profiles/traffic.json``, which bench.py reads for its roofline
``traffic`` field while the kernel sources are unchanged.  Raw rocprofv3 output
stays in --out.  This script itself never touches the GPU.

With ``--layout`` it profiles ``bench.py --layout-study`` instead: the study's
warm and cold times (one plain run), then ``--pmc FETCH_SIZE`` over each
storage variant alone and over the copy probe, giving the HBM bytes each
layout reads per step; writes ``profiles/layout_study.md``.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNELS = {"flat_kernel": "flat_paged", "prefix_mfma_kernel": "prefix_mfma", "merge_kernel": "merge",
           "paged_prefix_kernel": "paged_prefix", "paged_prefix_co_kernel": "paged_prefix"}
COPY_MIB = 256
NUM_CUS, SIMDS_PER_CU, NUM_XCC = 256, 4, 8
# Counter passes: at most 8 SQ and 2 GRBM counters each (one hardware pass).
SQ_PASSES = (
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_BUSY_CU_CYCLES",
     "SQ_WAVE_CYCLES", "SQ_WAVES", "GRBM_GUI_ACTIVE"),
    ("SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE",
     "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY"),
)


def kernel_key(name: str):
    base = name.replace("(anonymous namespace)::", "")
    base = base.split("<")[0].split("(")[0].replace("void ", "").strip()
    return KERNELS.get(base)


def rocprof(args, out_dir, tag, prog, limit=240):
    cmd = ["rocprofv3"] + args + ["-f", "csv", "-d", os.path.join(out_dir, tag), "-o", tag, "--",
                                  sys.executable] + prog
    env = dict(os.environ, TMPDIR="/tmp")
    print(f"[profile] {tag}: {' '.join(cmd)}", flush=True)
    with open(os.path.join(out_dir, tag + ".log"), "w") as log:
        r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT, timeout=limit)
    files = glob.glob(os.path.join(out_dir, tag, "**", f"{tag}_*.csv"), recursive=True)
    # rocprofv3 may end with a signal after the program has finished and its
    # results are complete; the csv files decide.
    if not files:
        raise RuntimeError(f"{tag}: rocprofv3 exited {r.returncode} without results")
    return cmd, files


def counter_means(files, counter):
    sums, counts = {}, {}
    for f in files:
        if not f.endswith("counter_collection.csv"):
            continue
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = kernel_key(r["Kernel_Name"]) or r["Kernel_Name"]
            sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    return {k: (sums[k] / counts[k], counts[k]) for k in sums}


def layout_profile(a, prof_dir):
    bench = os.path.join(ROOT, "bench.py")
    study = [bench, "--layout-study", "--steps", "10", "--cold-runs", "10"]
    print(f"[profile] layout study: {' '.join(study)}", flush=True)
    r = subprocess.run([sys.executable] + study, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                       text=True, timeout=400)
    if r.returncode != 0:
        raise RuntimeError(f"layout study exited {r.returncode}")
    times = json.loads(r.stdout.strip().splitlines()[-1])
    c_copy, f_copy = rocprof(["--pmc", "FETCH_SIZE"], a.out, "fetch_size_copy", [bench, "--copy-probe", str(COPY_MIB)],
                             limit=120)
    kib, _ = max(counter_means(f_copy, "FETCH_SIZE").values(), key=lambda v: v[0])
    factor = (COPY_MIB << 20) / (kib * 1024.0)
    rows, cmds = [], [c_copy]
    for v, rec in times["variants"].items():
        c, f = rocprof(["--pmc", "FETCH_SIZE"], a.out, f"fetch_size_{v}",
                       [bench, "--layout-study", "--layout-variant", v, "--steps", "3", "--cold-runs", "0"], limit=240)
        cmds.append(c)
        m = counter_means(f, "FETCH_SIZE")
        per_step = sum(m[k][0] for k in dict.fromkeys(KERNELS.values()) if k in m) * 1024 * factor
        rows.append((v, rec, per_step))
    rel = lambda c: " ".join(os.path.relpath(x, ROOT) if x.startswith(ROOT) else x for x in c)
    md = ["# Prefix storage layout in isolation", "",
          f"Workload: {times['config']['workload']}. The same decode-step attention with the shared prefix",
          "(1) stored once in the HOT slab and read once by the prefix contraction (cascade), (2) stored once in",
          "the HOT slab but re-read for every request by the paged pass (flat), (3) copied into every request's own",
          "COLD pages (flat over private copies: a pool without a shared level). Warm: mean of the attention kernels'",
          f"event durations over {times['config']['steps']} back-to-back steps; cold: median over",
          f"{times['config']['cold_runs']} runs, each after a {times['config']['flush_bytes'] >> 20} MiB flush.",
          "HBM read per step: FETCH_SIZE of the attention kernels (one rocprofv3 run per variant), scaled by the",
          f"same counter over a {COPY_MIB} MiB device copy ({factor * 1024:.1f} bytes per KiB read).", "",
          "| variant | prefix bytes stored | algorithmic K/V bytes read | HBM read (FETCH_SIZE) | warm us | cold us | "
          "kernels (warm, us) |", "|---|---|---|---|---|---|---|"]
    for v, rec, hbm in rows:
        ks = ", ".join(f"{k} {t}" for k, t in rec["kernels_us"].items())
        md.append(f"| {v} | {rec['prefix_bytes_stored'] / 1e6:.1f} MB | {rec['kv_bytes_read'] / 1e9:.3f} GB | "
                  f"{hbm / 1e9:.3f} GB | {rec['warm_us']} | {rec['cold_median_us']} | {ks} |")
    md += ["", "Commands: the study (repo root) and the counter runs (from /tmp, TMPDIR=/tmp):", "", "```",
           "python " + rel(study)] + [rel(c) for c in cmds] + ["```", ""]
    open(os.path.join(prof_dir, "layout_study.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps({v: {"hbm_read_bytes": int(h), "warm_us": rec["warm_us"]} for v, rec, h in rows}), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", default="C1")
    ap.add_argument("--mode", default="step")
    ap.add_argument("--lp", type=int, default=None, help="override the prefix length (C3 sweep points)")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "profile"), help="raw rocprofv3 output")
    ap.add_argument("--prof-dir", default=os.path.join(ROOT, "profiles"), help="where the summaries go")
    ap.add_argument("--layout", action="store_true", help="profile bench.py --layout-study instead of the step")
    a = ap.parse_args()
    os.makedirs(a.out, exist_ok=True)
    prof_dir = os.path.abspath(a.prof_dir)
    os.makedirs(prof_dir, exist_ok=True)
    if a.layout:
        return layout_profile(a, prof_dir)
    bench = os.path.join(ROOT, "bench.py")
    run = [bench, "--config", a.config, "--mode", a.mode, "--no-cpu-baseline", "--cold-runs", "0", "--graph-steps", "0",
           "--other-configs", "none", "--no-ceilings"]
    name = f"{a.config.lower()}_{a.mode}"
    cfg_key = a.config
    if a.lp is not None:
        run += ["--lp", str(a.lp)]
        name = f"{a.config.lower()}_lp{a.lp}_{a.mode}"
        cfg_key = f"{a.config}@{a.lp}"

    # 1. kernel trace + stats of the bench command
    cmd, files = rocprof(["--kernel-trace", "--stats"], a.out, "stats",
                         run + ["--steps", str(a.steps), "--warmup", str(a.warmup)])
    stats = [f for f in files if f.endswith("kernel_stats.csv")]
    lines = [f"# Kernel durations: {a.config}, mode {a.mode}", "",
             "rocprofv3 kernel trace of one bench.py run (every kernel of the warmup, timed and",
             "per-kernel-timing steps). Command, run from /tmp with TMPDIR=/tmp:", "", "```",
             " ".join(os.path.relpath(c, ROOT) if c.startswith(ROOT) else c for c in cmd), "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    avg_ns = {}
    for r in csv.DictReader(open(stats[0])):
        k = kernel_key(r["Name"])
        if k:
            avg_ns[k] = float(r["AverageNs"])
        n = r["Name"].replace("(anonymous namespace)::", "").replace("|", "/")
        n = n.split("(")[0] if "<" not in n else n.split(">(")[0] + ">"
        lines.append(f"| `{n[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    open(os.path.join(prof_dir, f"{name}_kernel_stats.md"), "w").write("\n".join(lines) + "\n")

    # 2-5. HBM traffic counters, calibrated on a copy of known size
    short = run + ["--steps", "3", "--warmup", "1"]
    readings, cmds = {}, {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        c1, f1 = rocprof(["--pmc", counter], a.out, f"{counter.lower()}_bench", short, limit=120)
        c2, f2 = rocprof(["--pmc", counter], a.out, f"{counter.lower()}_copy", [bench, "--copy-probe", str(COPY_MIB)],
                         limit=120)
        readings[counter] = (counter_means(f1, counter), counter_means(f2, counter))
        cmds[counter] = (c1, c2)
    factors = {}
    for counter, (_, copy) in readings.items():
        kib, _ = max(copy.values(), key=lambda v: v[0])        # the copy kernel: the largest reading
        factors[counter] = (COPY_MIB << 20) / (kib * 1024.0)
    runs = {}
    for k in dict.fromkeys(KERNELS.values()):
        f = readings["FETCH_SIZE"][0].get(k)
        w = readings["WRITE_SIZE"][0].get(k)
        if f is None or w is None:
            continue
        runs[k] = {"fetch_kib": round(f[0], 1), "write_kib": round(w[0], 1), "dispatches": f[1],
                   "traffic_bytes": int(f[0] * 1024 * factors["FETCH_SIZE"] + w[0] * 1024 * factors["WRITE_SIZE"])}
    sys.path.insert(0, ROOT)
    from importlib import util
    spec = util.spec_from_file_location("bench_mod", bench)
    bm = util.module_from_spec(spec)
    spec.loader.exec_module(bm)                                # for source_digest only (no GPU use)
    tpath = os.path.join(prof_dir, "traffic.json")
    try:
        t = json.load(open(tpath if os.path.exists(tpath) else os.path.join(ROOT, "profiles", "traffic.json")))
    except (OSError, ValueError):
        t = {}
    if t.get("sources") != bm.source_digest():
        t = {"sources": bm.source_digest(), "runs": {}}
    t["runs"][f"{cfg_key}/{a.mode}"] = runs
    t["factors"] = factors
    json.dump(t, open(tpath, "w"), indent=1, sort_keys=True)
    md = [f"# HBM traffic per launch: {a.config}, mode {a.mode}", "",
          f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each in its own rocprofv3 run, scaled by",
          f"the same counter over a plain {COPY_MIB} MiB device copy (reads and writes {COPY_MIB} MiB).", "",
          "| counter | copy reading (KiB) | factor (bytes per KiB read) |", "|---|---|---|"]
    for counter, (_, copy) in readings.items():
        kib, _ = max(copy.values(), key=lambda v: v[0])
        md.append(f"| {counter} | {kib:.1f} | {factors[counter] * 1024:.1f} |")
    md += ["", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | dispatches | traffic (MB per launch) |",
           "|---|---|---|---|---|"]
    for k, r in runs.items():
        md.append(f"| {k} | {r['fetch_kib']} | {r['write_kib']} | {r['dispatches']} | {r['traffic_bytes'] / 1e6:.1f} |")
    md += ["", "Commands (from /tmp, TMPDIR=/tmp):", "", "```"]
    for counter, (c1, c2) in cmds.items():
        for c in (c1, c2):
            md.append(" ".join(os.path.relpath(x, ROOT) if x.startswith(ROOT) else x for x in c))
    md += ["```", "", f"Kernel sources digest: {t['sources']}"]
    open(os.path.join(prof_dir, f"{name}_traffic.md"), "w").write("\n".join(md) + "\n")

    # 6-7. shader-sequencer counters (MFMA, VALU, LDS) per kernel
    sq, sq_cmds = {}, []
    for i, counters in enumerate(SQ_PASSES):
        c, f = rocprof(["--pmc"] + list(counters), a.out, f"sq{i + 1}_bench", short, limit=120)
        sq_cmds.append(c)
        for counter in counters:
            for k, (v, _) in counter_means(f, counter).items():
                sq.setdefault(k, {})[counter] = v
    cm = [f"# Shader counters per launch: {a.config}, mode {a.mode}", "",
          "Means per dispatch over a short bench run, summed over the chip's shader engines and XCDs.",
          f"Derived: kernel cycles = GRBM_GUI_ACTIVE / {NUM_XCC} (one reading per XCD); MFMA busy =",
          f"SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x {NUM_CUS} CUs x {SIMDS_PER_CU} SIMDs); bf16 MFMA rate =",
          "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / average duration (kernel trace) against 2.5 PFLOP/s;",
          "LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
          "| kernel | avg us | MFMA busy | bf16 MFMA TFLOP/s | % of peak | VALU insts | LDS insts | "
          "bank-conflict share |", "|---|---|---|---|---|---|---|---|"]
    for k in dict.fromkeys(KERNELS.values()):
        v = sq.get(k)
        if not v:
            continue
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / NUM_XCC
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * NUM_CUS * SIMDS_PER_CU) if cyc > 0 else 0.0
        t = avg_ns.get(k, 0.0) * 1e-9
        tf = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / t / 1e12 if t > 0 else 0.0
        lds = v.get("SQ_LDS_IDX_ACTIVE", 0.0)
        bc = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds > 0 else 0.0
        cm.append(f"| {k} | {t * 1e6:.2f} | {100 * busy:.1f} % | {tf:.1f} | {100 * tf / 2500:.1f} % | "
                  f"{v.get('SQ_INSTS_VALU', 0):.0f} | {v.get('SQ_INSTS_LDS', 0):.0f} | {100 * bc:.1f} % |")
    cm += ["", "Raw means per dispatch:", "", "| kernel | counter | value |", "|---|---|---|"]
    for k in dict.fromkeys(KERNELS.values()):
        for counter, val in sorted(sq.get(k, {}).items()):
            cm.append(f"| {k} | {counter} | {val:.1f} |")
    cm += ["", "Commands (from /tmp, TMPDIR=/tmp):", "", "```"]
    cm += [" ".join(os.path.relpath(x, ROOT) if x.startswith(ROOT) else x for x in c) for c in sq_cmds]
    cm += ["```", "", f"Kernel sources digest: {bm.source_digest()}"]
    open(os.path.join(prof_dir, f"{name}_counters.md"), "w").write("\n".join(cm) + "\n")
    print(json.dumps(runs), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
