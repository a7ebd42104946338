"""Benchmark of the tiered-KV decode step on one MI355X.

One step = append the new token's K/V, split-K attention over every live
row of every layer, chunk merge, the Eq. 1 score update, and -- every Delta
steps -- the reassignment (rank, label, changed-row lists, row moves).  The
workload is the 7B-shaped one: 32 layers, 32 query / 32 kv heads, head_dim
128, bf16, batch 1, 2200 prefilled positions, 512 decode steps, Delta = 64,
HBM ratio 0.5, eviction 0.03, protected 200 prompt + 4 sinks + 128 recent,
T1 staging resident in HBM.  Inputs are seeded synthetic (Gaussian with
planted heavy hitters) and sit in HBM before the timed region starts.

Prints one JSON line.  Extra fields: the split-K kernel's roofline (live K/V
bytes per launch / launch time, HIP events on the launch stream), the
stream-staging leg (T1 rows copied from pinned host memory one layer ahead
of attention; H2D GB/s against the pinned H2D bandwidth measured here), the
CPU oracle timed on a bounded sample of the same workload, and the parity of
the GPU with the oracle over that sample (sampled outputs, final scores,
every reassignment's labels).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
STAGING_LAYERS = 4  # HBM slots of the stream-staging leg (two layers per copy)
KERNEL_SRC = os.path.join(ROOT, "decode_attention_tkv_amd", "csrc", "attn.hip")
def attention_kernel(w, args):
    """Which pass of the split-K kernel a workload's decode steps take: bf16
    caches with one query head per kv head, or four or more (unless the
    vector pass is asked for), use the matrix cores; every other shape the
    vector units."""
    if w.dtype == "bf16" and (w.q_heads == w.kv_heads or w.q_heads >= 4 * w.kv_heads) and not args.vector_pass:
        return "k_attn_chunk (split-K attention, matrix-core pass)"
    return "k_attn_chunk (split-K attention, vector pass)"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_chunk_7b_traffic.txt")
COPY_BYTES = 1 << 30  # plain device copy used to scale the HBM byte counters
METRIC = "decode steps/sec (attn+scoring, all layers) at 7B shape; achieved HBM GB/s %peak"


def _dev(a, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def load_inputs(w, steps, torch):
    heavy, u = w.heavy_mask(), w.unit_vector()
    k0 = _dev(w.kv(0, 0, w.prefill, heavy, u), w.dtype, torch)
    v0 = _dev(w.kv(1, 0, w.prefill, heavy, u), w.dtype, torch)
    kn = w.kv(0, w.prefill, steps, heavy, u)
    vn = w.kv(1, w.prefill, steps, heavy, u)
    # [steps][L][B][Hkv][d] so that each step's rows are one contiguous block
    kn = _dev(np.ascontiguousarray(np.moveaxis(kn, 2, 0)), w.dtype, torch)
    vn = _dev(np.ascontiguousarray(np.moveaxis(vn, 2, 0)), w.dtype, torch)
    q = _dev(w.q(0, steps, u), w.dtype, torch)
    return k0, v0, kn, vn, q


CHUNK = 0  # split-K rows per work-group (0: the library's default for the shape)
EXTRA_FLAGS = 0  # TKV_FLAG_* added to every handle (e.g. the vector pass for grouped-query heads)


def run_decode(w, inputs, warmup, steps, torch, tkv, staging_layers=0, time_kernels=True, sync_reassign=False,
               samples=(), scored_prefill=None, layer_hbm=None):
    """Prefill, `warmup` untimed steps, then `steps` timed steps.  Returns
    (seconds, stats before, stats after).  sync_reassign: drain the stream
    before and after every reassignment of the timed steps and put the
    per-call wall times (ms) under after["reassign_synced_ms"].  samples:
    0-based steps whose outputs are copied to the host (a synchronisation
    each; for untimed runs), under after["samples"]; the last step's output
    is always under after["last_out"].  scored_prefill: the prompt's queries
    [L][B][n][Hq][d] to prefill with scores instead of the plain placement.
    layer_hbm: per-layer HBM ratios (tkv_options.layer_hbm), or None."""
    k0, v0, kn, vn, q = inputs
    c = tkv.TieredKV.for_workload(w, staging_layers=staging_layers, time_kernels=time_kernels, chunk=CHUNK,
                                  extra_flags=EXTRA_FLAGS, layer_hbm=layer_hbm)
    if scored_prefill is not None:
        c.prefill_scored(k0, v0, scored_prefill)
    else:
        c.prefill(k0, v0)
    h = c.h
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lib = tkv.lib()
    optr = out.data_ptr()
    kp = [kn[t].data_ptr() for t in range(warmup + steps)]
    vp = [vn[t].data_ptr() for t in range(warmup + steps)]
    qp = [q[t].data_ptr() for t in range(warmup + steps)]

    synced = []
    sampled = {}

    def step(t):
        # append + attention of every layer (+ the pending Eq. 1 update) in one call
        rc = lib.tkv_decode_step(h, kp[t], vp[t], qp[t], optr, stream)
        if rc == 0 and t in samples:
            sampled[t] = out.cpu().numpy()
        if rc == 0 and (t + 1) % w.delta == 0:
            if sync_reassign and t >= warmup:
                # the caller's stream only: the write-back of rows entering T1 runs on the
                # library's own stream, beside the next steps
                cur = torch.cuda.current_stream()
                cur.synchronize()
                r0 = time.perf_counter()
                rc = lib.tkv_reassign(h, stream)
                cur.synchronize()
                synced.append((time.perf_counter() - r0) * 1e3)
            else:
                rc = lib.tkv_reassign(h, stream)
        if rc != 0:
            raise tkv.TkvError(rc, lib.tkv_last_error(h).decode())

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    before = c.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        step(t)
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    after = c.stats()
    after["reassign_synced_ms"] = synced
    after["samples"] = sampled
    after["last_out"] = out.cpu().numpy()
    c.close()
    return secs, before, after


def pinned_h2d_gbs(torch, mb=256, reps=20):
    src = torch.empty(mb << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(mb << 20, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    return (mb << 20) / float(np.median(times)) / 1e9


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def _pmc_rows(d):
    """Rows of a rocprofv3 counter_collection.csv under directory d."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    return list(csv.DictReader(open(files[0])))


def summarize_pmc(fetch_dir, write_dir):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of
    `bench.py --pmc-probe` into the traffic summary under profiles/."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(d) if r.get("Counter_Name") == counter]
        attn = [float(r["Counter_Value"]) for r in rows if "k_attn_chunk" in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()
                and "k_" not in r["Kernel_Name"]]
        if not attn or not copy:
            raise SystemExit("%s: attention or copy dispatches missing" % counter)
        copy_kib = max(copy)          # the 1 GiB copy is the largest copy dispatch
        factor = (COPY_BYTES / 1024.0) / copy_kib
        out[counter] = {"attn_kib_mean": sum(attn) / len(attn), "dispatches": len(attn),
                        "copy_kib": copy_kib, "factor": factor,
                        "bytes_per_launch": sum(attn) / len(attn) * 1024.0 * factor}
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    # live K/V bytes per dispatch of the probe: 8 + 24 steps from the 7b prefill, none evicted yet
    import tkvsynth
    w = tkvsynth.CONFIGS["7b"]
    n_disp = out["FETCH_SIZE"]["dispatches"]
    kv = sum((w.prefill + 1 + t) * w.kv_bytes_per_token() * w.batch for t in range(n_disp)) / n_disp
    lines = ["# k_attn_chunk HBM traffic, 7b workload (rocprofv3 counters)", "",
             "Commands (one MI355X, repo root; each counter in its own run):", "",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o pmc -- python bench.py --pmc-probe" % fetch_dir,
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o pmc -- python bench.py --pmc-probe" % write_dir,
             "    python bench.py --summarize-pmc %s %s" % (fetch_dir, write_dir), "",
             "`--pmc-probe` runs 8 warmup + 24 decode steps of the 7b workload, then one plain 1 GiB device",
             "copy (torch copy_) whose counter reading scales KiB to bytes (factor = 1 GiB / counted).", "",
             "| Counter | attention dispatches | mean KiB / dispatch | copy KiB (1 GiB copy) | scale | bytes / launch |",
             "|---|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[c]
        lines.append("| %s | %d | %.0f | %.0f | %.4f | %.4g |" % (c, o["dispatches"], o["attn_kib_mean"], o["copy_kib"],
                                                                o["factor"], o["bytes_per_launch"]))
    lines += ["", "Live K/V bytes per dispatch of the probe (algorithmic): %.6g" % kv,
              "", "traffic_bytes_per_launch: %.6g" % total,
              "traffic_over_kv_bytes: %.6f" % (total / kv),
              "kernel_source_sha256_16: %s" % kernel_hash()]
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    open(TRAFFIC_FILE, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_traffic(kv_bytes_per_launch):
    """Counter-derived HBM bytes per split-K launch (the probe's traffic-to-
    live-K/V ratio applied to this run's launches), if the counters were
    taken on this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = dict(l.split(": ", 1) for l in open(TRAFFIC_FILE).read().splitlines() if ": " in l and not l.startswith("|"))
    if kv.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["traffic_over_kv_bytes"]) * kv_bytes_per_launch
    except (KeyError, ValueError):
        return None


def gpu_trace(w, inputs, n_steps, torch, tkv, sample_every=16):
    """The first n_steps decode steps on a fresh handle, recorded for the
    oracle to follow: outputs at sampled steps, the fp32 scores each
    reassignment ranks by, the labels it produced, and the final scores."""
    k0, v0, kn, vn, q = inputs
    c = tkv.TieredKV.for_workload(w)
    c.prefill(k0, v0)
    out = torch.empty((w.layers, w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    tr = {"outs": {}, "ranks": [], "labels": []}
    for t in range(n_steps):
        c.append(kn[t], vn[t])
        c.decode_attn(q[t], out)
        if t % sample_every == 0 or t == n_steps - 1:
            tr["outs"][t] = out.cpu().numpy()
        if (t + 1) % w.delta == 0:
            n = w.prefill + t + 1
            tr["ranks"].append(c.read_scores()[:, :n])
            c.reassign()
            tr["labels"].append(c.read_tiers()[:, :n])
    tr["s"] = c.read_scores()
    c.close()
    return tr


def cpu_baseline(w, n_steps, trace=None):
    """The oracle as it stands, on the host cores: prefill untimed, then
    n_steps decode steps with a reassignment every Delta steps.  Given the
    GPU's trace of the same steps, the oracle ranks on the GPU's fp32 scores
    (the labelling decision is taken in the kernel's precision) and, after
    the timed loop, the two runs are compared."""
    import oracle
    heavy, u = w.heavy_mask(), w.unit_vector()
    o = oracle.OracleTKV.for_workload(w)
    o.prefill(w.values(w.kv(0, 0, w.prefill, heavy, u)), w.values(w.kv(1, 0, w.prefill, heavy, u)))
    kn = w.values(w.kv(0, w.prefill, n_steps, heavy, u))
    vn = w.values(w.kv(1, w.prefill, n_steps, heavy, u))
    q = w.values(w.q(0, n_steps, u))
    refs, labels = {}, []
    live_rows = 0  # live rows attended, summed over steps and sequences
    t0 = time.perf_counter()
    for t in range(n_steps):
        o.append(kn[:, :, t], vn[:, :, t])
        live_rows += int(np.count_nonzero(o.tier[:, : o.n] < 3))
        ref = o.attend(q[t])
        if trace is not None and t in trace["outs"]:
            refs[t] = ref
        if (t + 1) % w.delta == 0:
            ranks = trace["ranks"][len(labels)] if trace is not None else None
            new, _ = o.reassign(rank_scores=ranks)
            labels.append(new)
    secs = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    res = {"value": n_steps / secs, "unit": "steps/s", "cores": threads, "kind": "oracle",
           # the live K/V bytes those steps attend (the GPU roofline's algorithmic bytes) per second
           "kv_gbs": live_rows * w.kv_bytes_per_token() / secs / 1e9,
           "sample": "%s workload, prefill %d, decode steps 1..%d incl. %d reassignment(s); fp64 C "
                     "attention (OpenMP) + numpy scoring/tiering; %.1f s"
                     % (w.name, w.prefill, n_steps, n_steps // w.delta, secs)}
    if trace is None:
        return res, None
    n = o.n
    out_err = max(float(np.max(np.abs(trace["outs"][t] - refs[t]))) for t in refs)
    g = trace["s"][:, :n].astype(np.float64)
    r = o.s[:, :n]
    m = r > 0
    s_rel = float(np.max(np.abs(g[m] - r[m]) / r[m])) if m.any() else 0.0
    same = all(np.array_equal(a, b) for a, b in zip(trace["labels"], labels))
    tol = 5e-3 if w.dtype == "bf16" else 1e-5
    parity = {"steps": n_steps, "sampled_steps": len(refs), "out_max_abs": out_err, "out_tol": tol,
              "score_max_rel": s_rel, "score_tol": 1e-4, "reassignments": len(labels),
              "labels_bit_exact": same, "ok": bool(out_err <= tol and s_rel <= 1e-4 and same)}
    return res, parity


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_steps_per_s(w, n_steps):
    """The oracle alone over the first n_steps decode steps (prefill untimed)."""
    import oracle
    heavy, u = w.heavy_mask(), w.unit_vector()
    o = oracle.OracleTKV.for_workload(w)
    o.prefill(w.values(w.kv(0, 0, w.prefill, heavy, u)), w.values(w.kv(1, 0, w.prefill, heavy, u)))
    kn = w.values(w.kv(0, w.prefill, n_steps, heavy, u))
    vn = w.values(w.kv(1, w.prefill, n_steps, heavy, u))
    q = w.values(w.q(0, n_steps, u))
    t0 = time.perf_counter()
    for t in range(n_steps):
        o.append(kn[:, :, t], vn[:, :, t])
        o.attend(q[t])
        if (t + 1) % w.delta == 0:
            o.reassign()
    return n_steps / (time.perf_counter() - t0)


def single_thread_oracle(name, n_steps, timeout=120):
    """oracle_steps_per_s in a child process limited to one OpenMP thread (the
    child touches no GPU)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-only", name, str(n_steps)],
                           env=env, capture_output=True, text=True, timeout=timeout)
        if r.returncode != 0:
            return {"error": (r.stderr or "")[-300:]}
        return json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:  # reported, never fatal to the bench line
        return {"error": str(e)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="7b")
    ap.add_argument("--chunk", type=int, default=0, help="split-K rows per work-group: 128, 256 or 512 (0: default)")
    ap.add_argument("--vector-pass", action="store_true",
                    help="bf16 heads (one, or 4 or more, per kv head) on the vector units instead of the matrix cores")
    ap.add_argument("--stream-steps", type=int, default=64, help="timed steps of the stream-staging leg (0: skip)")
    ap.add_argument("--staging-layers", type=int, default=STAGING_LAYERS,
                    help="HBM staging slots S of the stream-staging leg (2 .. layers - 1)")
    ap.add_argument("--cpu-steps", type=int, default=192,
                    help="steps of the CPU oracle baseline and of the parity check beside it (0: skip)")
    ap.add_argument("--baseline-steps", type=int, default=None,
                    help="timed steps of each baseline policy on the same engine (default: --steps; 0: skip)")
    ap.add_argument("--prefill-reps", type=int, default=3,
                    help="timed runs of the plain and the scored prefill of the workload's cache (0: skip)")
    ap.add_argument("--no-drained-leg", dest="drained_leg", action="store_false",
                    help="skip the run that times each reassignment with the stream drained around it")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short run for counter collection: 8 + 24 steps, then one 1 GiB device copy")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc runs of --pmc-probe")
    ap.add_argument("--no-full-run", dest="full_run", action="store_false",
                    help="skip the legs over the workload's whole decode (every reassignment)")
    ap.add_argument("--single-thread-steps", type=int, default=12,
                    help="decode steps of the one-thread oracle runs (tiny: its whole decode; 0: skip)")
    ap.add_argument("--oracle-only", nargs=2, metavar=("WORKLOAD", "STEPS"),
                    help="(internal) time the oracle alone on the host and print one JSON line")
    args = ap.parse_args()
    if args.oracle_only:
        import tkvsynth
        name, n = args.oracle_only[0], int(args.oracle_only[1])
        w = tkvsynth.CONFIGS[name]
        n = min(n, w.steps)
        print(json.dumps({"workload": name, "steps": n, "steps_per_s": oracle_steps_per_s(w, n),
                          "threads": int(os.environ.get("OMP_NUM_THREADS", "0") or 0)}))
        return
    global CHUNK, EXTRA_FLAGS
    CHUNK = args.chunk
    EXTRA_FLAGS = 32 if args.vector_pass else 0  # TKV_FLAG_VECTOR_PASS
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the tiered-KV decode path has no multi-GPU leg "
              "(sequences would shard one per GPU with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_tkv_amd as tkv
    import tkvsynth

    if args.pmc_probe:
        args.warmup, args.steps, args.stream_steps, args.cpu_steps, args.baseline_steps = 8, 24, 0, 0, 0
        args.prefill_reps = 0
    base = tkvsynth.CONFIGS[args.workload]
    total = args.warmup + args.steps
    # the workload's own decode length, stretched if more steps are asked for
    w = base if total <= base.steps else base.replace(steps=total)
    print("[bench] drawing inputs for %s (%d steps)" % (w.name, w.steps), file=sys.stderr, flush=True)
    inputs = load_inputs(w, w.steps, torch)
    torch.cuda.synchronize()

    print("[bench] resident staging: %d warmup + %d timed steps" % (args.warmup, args.steps),
          file=sys.stderr, flush=True)
    secs, before, after = run_decode(w, inputs, args.warmup, args.steps, torch, tkv)
    if args.pmc_probe:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] pmc probe done", file=sys.stderr, flush=True)
        return
    kern_ms = after["attn_kernel_ms"] - before["attn_kernel_ms"]
    launches = after["attn_kernel_launches"] - before["attn_kernel_launches"]
    kv_bytes = after["attn_kv_bytes"] - before["attn_kv_bytes"]
    steps_per_s = args.steps / secs
    achieved = kv_bytes / (kern_ms / 1e3) / 1e9
    step_gbs = kv_bytes / secs / 1e9

    result = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": secs / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "%s: %d layers, %d q / %d kv heads, head_dim %d, %s, batch %d, cache %d -> %d, "
                               "delta %d, hbm %.2f, evict %.2f, protect %d prompt + %d sinks + %d recent, "
                               "resident T1 staging" % (w.name, w.layers, w.q_heads, w.kv_heads, w.head_dim,
                                                        w.dtype, w.batch, w.prefill, w.prefill + total, w.delta,
                                                        w.hbm_ratio, w.evict_ratio, w.prompt, w.sinks, w.recent),
                   "timed_steps": "%d..%d" % (args.warmup + 1, total),
                   "reassignments_timed": int(after["reassigns"] - before["reassigns"])},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(kv_bytes / launches),
                     "kernel": attention_kernel(w, args),
                     "avg_launch_us": kern_ms / launches * 1e3, "launches": launches,
                     "kv_bytes_per_launch": kv_bytes / launches},
        "step_hbm_gbs": step_gbs,
        "step_hbm_frac": step_gbs / HBM_PEAK_GBS,
        # Host wall time inside tkv_reassign.  The call waits for the tier counts, so it also
        # covers draining the decode steps still queued on the stream when it was made.  None
        # when the timed window holds no reassignment.
        "reassign_wall_ms_per_call": ((after["reassign_ms"] - before["reassign_ms"])
                                      / (after["reassigns"] - before["reassigns"])
                                      if after["reassigns"] > before["reassigns"] else None),
    }
    # The cost of one reassignment on its own: the same run with the stream drained before and
    # after each reassignment call, so the call's wall time is its host work plus its GPU work.
    if args.drained_leg and result["config"]["reassignments_timed"] > 0:
        print("[bench] reassignment cost, stream drained around each call", file=sys.stderr, flush=True)
        _, _, rs = run_decode(w, inputs, args.warmup, args.steps, torch, tkv, time_kernels=False,
                              sync_reassign=True)
        result["reassign_ms_per_call_drained"] = float(np.median(rs["reassign_synced_ms"]))

    # The workload's whole decode (every reassignment of it), whatever --steps is: once timed as
    # the headline is, once with the stream drained around each reassignment (its cost on its own)
    # and with outputs sampled for the stream-staging comparison below.
    full_samples = {}
    wf = base if base.steps >= w.steps else w
    # the stream-staging windows (below): the first reassignment (after step delta) mid-window, and
    # the steady state from the step after it; their last steps are compared with this run's
    ns = args.stream_steps
    first_warm, steady_warm = max(0, w.delta - ns // 2), w.delta + 1
    stream_last = (first_warm + ns - 1, steady_warm + ns - 1) if ns > 0 else ()
    if args.full_run:
        print("[bench] full run: %d steps, every reassignment" % wf.steps, file=sys.stderr, flush=True)
        finputs = inputs if wf is w else load_inputs(wf, wf.steps, torch)
        fsecs, fb, fa = run_decode(wf, finputs, 0, wf.steps, torch, tkv)
        fk_ms = fa["attn_kernel_ms"] - fb["attn_kernel_ms"]
        fkv = fa["attn_kv_bytes"] - fb["attn_kv_bytes"]
        nre = fa["reassigns"] - fb["reassigns"]
        result["full_run"] = {
            "steps": wf.steps, "timed_steps": "1..%d" % wf.steps, "reassignments": int(nre),
            "steps_per_s": wf.steps / fsecs, "ms_per_step": fsecs / wf.steps * 1e3,
            "kernel_frac": fkv / (fk_ms / 1e3) / 1e9 / HBM_PEAK_GBS if fk_ms > 0 else None,
            "step_hbm_frac": fkv / fsecs / 1e9 / HBM_PEAK_GBS,
            "reassign_ms_per_call_in_stream": (fa["reassign_ms"] - fb["reassign_ms"]) / nre if nre else None}
        _, _, fr = run_decode(wf, finputs, 0, wf.steps, torch, tkv, time_kernels=False, sync_reassign=True,
                              samples={t for t in stream_last if t < wf.steps})
        full_samples = fr["samples"]
        result["full_run"]["reassign_ms_per_call_drained"] = (float(np.median(fr["reassign_synced_ms"]))
                                                              if fr["reassign_synced_ms"] else None)
        result["full_run"]["reassign_ms_drained_each"] = [round(x, 3) for x in fr["reassign_synced_ms"]]
        if "reassign_ms_per_call_drained" not in result and fr["reassign_synced_ms"]:
            result["reassign_ms_per_call_drained"] = result["full_run"]["reassign_ms_per_call_drained"]
        if finputs is not inputs:
            del finputs

    if args.stream_steps > 0:
        # Stream staging: each step copies every layer's T1 rows from pinned host memory into
        # one of S HBM slots, ahead of the attention that reads them.  Three
        # windows of --stream-steps steps: the first reassignment after a plain prefill (whose
        # positional first placement leaves most rows to re-tier), the steady state (the next
        # window, ending after the next reassignment), and the first reassignment after a
        # scored prefill (rows placed by the prompt's own scores from the start).
        pinned = pinned_h2d_gbs(torch)
        ws = base if base.steps >= steady_warm + ns else base.replace(steps=steady_warm + ns)
        sinputs = inputs if ws.steps <= w.steps else load_inputs(ws, ws.steps, torch)

        def window(warm, scored=None, label=""):
            print("[bench] stream staging (S=%d) %s: steps %d..%d" % (args.staging_layers, label, warm + 1, warm + ns),
                  file=sys.stderr, flush=True)
            ssecs, sb, sa = run_decode(ws, sinputs, warm, ns, torch, tkv, staging_layers=args.staging_layers,
                                       scored_prefill=scored)
            h2d = sa["h2d_bytes"] - sb["h2d_bytes"]
            return sa, {"timed_steps": "%d..%d" % (warm + 1, warm + ns),
                        "reassignments": int(sa["reassigns"] - sb["reassigns"]),
                        "steps_per_s": ns / ssecs, "h2d_gbs": h2d / ssecs / 1e9,
                        "h2d_frac_of_pinned": (h2d / ssecs / 1e9) / pinned, "h2d_bytes_per_step": h2d / ns,
                        # max(H2D time at the pinned rate, resident step time) / stream step time: 1.0
                        # means the layer-ahead copies hide the compute completely (or the reverse)
                        "overlap_efficiency": max(h2d / ns / (pinned * 1e9), secs / args.steps) / (ssecs / ns)}

        sa1, first = window(first_warm, label="first reassignment")
        sa2, steady = window(steady_warm, label="steady state")
        scored = None
        qb = ws.prefill * ws.layers * ws.batch * ws.q_heads * ws.head_dim * ws.elem_bytes
        if qb <= (8 << 30):
            qp = _dev(np.ascontiguousarray(np.moveaxis(ws.q(ws.steps, ws.prefill, ws.unit_vector()), 0, 2)),
                      ws.dtype, torch)
            _, scored = window(first_warm, scored=qp, label="first reassignment, scored prefill")
            del qp
        # Proposition 1 on the wire: stream staging must give the resident run's outputs bit for bit
        cmp = {}
        for t, o in ((first_warm + ns - 1, sa1["last_out"]), (steady_warm + ns - 1, sa2["last_out"])):
            if t in full_samples:
                cmp[str(t + 1)] = bool(np.array_equal(o, full_samples[t]))
        result["stream_staging"] = dict(steady, **{
            "staging_layers": args.staging_layers, "steps": ns, "pinned_h2d_gbs": pinned,
            "window": "steady state: steps %s, after the first reassignment and holding the next"
                      % steady["timed_steps"],
            "first_reassignment_window": first, "scored_prefill_window": scored,
            "outputs_bitwise_equal_resident": cmp,
            "hbm_kv_bytes_allocated": sa2["hbm_bytes"], "full_cache_bytes": sa2["full_cache_bytes"]})
        if cmp and not all(cmp.values()):
            raise SystemExit("stream staging outputs differ from the resident run: %s" % cmp)
        if sinputs is not inputs:
            del sinputs

    if args.baseline_steps is None:
        args.baseline_steps = args.steps
    if args.baseline_steps > 0:
        # the same engine under other policies, same inputs and step window
        result["baselines"] = {}
        policies = (("full cache (all rows in T0)", dict(hbm_ratio=1.0, evict_ratio=0.0), None),
                    ("eviction only, heavy hitters (no T1)", dict(no_t1=True), None),
                    ("sinks + recent window", dict(hbm_ratio=0.0, no_t1=True, prompt=0), None))
        if w.batch > 1:
            policies += (("one HBM budget for the batch", dict(shared_hbm=True), None),)
        # per-layer budgets: the first half of the layers 0.2 below the workload's ratio, the
        # rest 0.2 above (the same mean; the same rows evicted)
        half = w.layers // 2
        lo, hi = max(0.0, w.hbm_ratio - 0.2), min(1.0, w.hbm_ratio + 0.2)
        policies += (("per-layer HBM budgets (%d layers at %.2f, %d at %.2f)" % (half, lo, w.layers - half, hi), {},
                      [lo] * half + [hi] * (w.layers - half)),)
        result["baselines"]["tiered (this line)"] = {
            "steps_per_s": steps_per_s, "live_rows_per_seq_at_end":
                (after["tier_count"][0] + after["tier_count"][1] + after["tier_count"][2]) / w.batch,
            "t0_rows_at_end": after["tier_count"][0],
            "hbm_ratio": w.hbm_ratio, "evict_ratio": w.evict_ratio, "no_t1": False,
            "kernel_gbs": achieved, "host_bytes": after["host_bytes"]}
        for name, kw, layer_hbm in policies:
            print("[bench] baseline %s: %d timed steps" % (name, args.baseline_steps), file=sys.stderr, flush=True)
            wb = w.replace(**kw)
            bsecs, bb, ba = run_decode(wb, inputs, args.warmup, args.baseline_steps, torch, tkv, layer_hbm=layer_hbm)
            # (with per-layer budgets tier_count counts (layer, position) rows)
            per = w.batch * (w.layers if layer_hbm else 1)
            live = (ba["tier_count"][0] + ba["tier_count"][1] + ba["tier_count"][2]) / per
            kb = ba["attn_kv_bytes"] - bb["attn_kv_bytes"]
            km = ba["attn_kernel_ms"] - bb["attn_kernel_ms"]
            result["baselines"][name] = {
                "steps_per_s": args.baseline_steps / bsecs, "live_rows_per_seq_at_end": live,
                "t0_rows_at_end": ba["tier_count"][0] / (w.layers if layer_hbm else 1),
                "hbm_ratio": wb.hbm_ratio if not layer_hbm else sum(layer_hbm) / len(layer_hbm),
                "evict_ratio": wb.evict_ratio, "no_t1": wb.no_t1,
                "kernel_gbs": kb / (km / 1e3) / 1e9 if km > 0 else None,
                "host_bytes": ba["host_bytes"]}

    q_bytes = w.prefill * w.layers * w.batch * w.q_heads * w.head_dim * w.elem_bytes
    if args.prefill_reps > 0 and q_bytes > (8 << 30):
        result["prefill"] = {"skipped": "the prompt's queries would take %.0f GB of host memory" % (q_bytes / 1e9)}
    elif args.prefill_reps > 0:
        # the step before the decode path: fill the cache, with and without the prompt's scores
        print("[bench] prefill: plain and scored, %d runs each" % args.prefill_reps, file=sys.stderr, flush=True)
        qp = _dev(np.ascontiguousarray(np.moveaxis(w.q(w.steps, w.prefill, w.unit_vector()), 0, 2)), w.dtype, torch)
        times = {}
        for scored in (False, True):
            ts = []
            for _ in range(args.prefill_reps + 1):  # the first run warms up
                c = tkv.TieredKV.for_workload(w)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                if scored:
                    c.prefill_scored(inputs[0], inputs[1], qp)
                else:
                    c.prefill(inputs[0], inputs[1])
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
                c.close()
            times[scored] = float(np.median(ts[1:])) * 1e3
        del qp
        result["prefill"] = {"positions": w.prefill, "plain_ms": times[False], "scored_ms": times[True],
                             "scoring_and_replacement_ms": times[True] - times[False],
                             "note": "plain: first placement + T1 rows to pinned host memory; scored adds the "
                                     "prompt's causal attention scores and one full re-placement"}

    args.cpu_steps = min(args.cpu_steps, w.steps)
    if args.cpu_steps > 0:
        print("[bench] parity trace: %d GPU steps" % args.cpu_steps, file=sys.stderr, flush=True)
        trace = gpu_trace(w, inputs, args.cpu_steps, torch, tkv)
        print("[bench] cpu baseline: oracle, %d steps" % args.cpu_steps, file=sys.stderr, flush=True)
        result["cpu_baseline"], result["parity"] = cpu_baseline(w, args.cpu_steps, trace)
        result["cpu_baseline"]["cpu_model"] = cpu_model()
        if args.single_thread_steps > 0:
            print("[bench] one-thread oracle: tiny and %s" % w.name, file=sys.stderr, flush=True)
            import tkvsynth as _ts
            result["cpu_baseline"]["single_thread"] = {
                "tiny": single_thread_oracle("tiny", _ts.CONFIGS["tiny"].steps),
                w.name: single_thread_oracle(w.name, args.single_thread_steps)}
        if not result["parity"]["ok"]:
            print(json.dumps(result), flush=True)
            raise SystemExit("parity with the oracle failed: %s" % result["parity"])

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
