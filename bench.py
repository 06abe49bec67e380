"""Benchmark: block-sparse attention forward at the Wan 2.1 14B attention shape.

One step = one inference call of the hot path on the GPU: look up the mask
set of the timestep in the resident bank and run the block-sparse forward on
Q, K, V as they lie ([B, H, L, d]; persistent launch, longest-row-first
order).  Inputs are resident in HBM before the timed region starts.  The
roofline figures are for the attention kernel, timed with events on the
launch stream around the call (which also enqueues a 4-microsecond
queue-reset kernel).  The metric is effective kept-block
throughput: 4 * block^2 * d FLOP per kept (query block, key block) tile,
counting full tiles, divided by the step time.  Also reported: the dense
forward on the same inputs (speedup = t_dense / t_sparse, the ratio the pages
print), the offline calibration steps (block mass, compile, work order) and
the float64 CPU oracle timed on a bounded sample of the same workload, and
the sustained matrix-core rate this GPU reaches with zero and with random
bf16 operands (the built `mfma_rate` probe, run after the timed work in its
own process): under random operands the clock drops to stay within power,
which bounds any matrix-core-bound kernel below the vendor figure.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
       python bench.py --copy-probe 1024   (plain copy, for counter scaling)
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective kept-block TFLOPS (frac of bf16 MFMA peak) + speedup vs dense, Wan shape"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 matrix peak (vendor figure)
COUNTERS = os.path.join(ROOT, "profiles", "attn_sparse_wan_counters.json")
KERNEL_SOURCES = ["block_sparse_attention_calibatt_amd/csrc/attn_fwd.hip",
                  "block_sparse_attention_calibatt_amd/csrc/tiles.h"]


def speedup(t_dense, t_method):
    """Time ratio at equal shape, the definition behind every speedup the pages print."""
    return t_dense / t_method


def tile_flops(block, d):
    return 4.0 * block * block * d


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload):
    """Bytes per launch from the committed counter summary, if it covers this
    workload and matches the current kernel source: (traffic, extra), where
    traffic counts what L2 fetched from and wrote to the memory side
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain copy
    of known size) and extra holds the memory-side request counters of the
    same launch.  Both include reads the MALL serves, so they bound HBM bytes
    from above."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, None
    if c.get("kernel_source_hash") != kernel_source_hash() or not c.get("workload", "").startswith(workload + ":"):
        return None, None
    extra = {k: c[k] for k in ("memory_side_read_bytes_per_launch", "memory_side_write_bytes_per_launch",
                               "compulsory_bytes_per_launch") if k in c}
    return c.get("traffic_bytes_per_launch"), (extra or None)


def mfma_rate():
    """Sustained matrix-core rate with zero and with random bf16 operands (the built probe), or None."""
    exe = os.path.join(ROOT, "block_sparse_attention_calibatt_amd", "mfma_rate")
    if not os.path.exists(exe):
        return None
    import subprocess
    try:
        res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        return json.loads(res.stdout.strip().splitlines()[-1]) if res.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def copy_probe(mb):
    import torch
    n = mb * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}))


def host_info():
    """The host the CPU figures come from: logical CPUs, the ones this process
    may run on, the CPU model and the memory size."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["affinity"] = None
    model = mem = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        with open("/proc/meminfo") as f:
            kb = next((int(ln.split()[1]) for ln in f if ln.startswith("MemTotal")), None)
            mem = round(kb / (1 << 20), 1) if kb else None
    except OSError:
        pass
    info["cpu_model"] = model
    info["ram_gib"] = mem
    return info


def _oracle_worker(job):
    """One worker of the CPU baseline: the float64 oracle on whole query blocks
    of its heads, in order, until its time budget is spent."""
    folder, heads, budget_s, block, scale, seq_len, nqb, d = job
    import oracle
    q, k, v = (np.load(os.path.join(folder, n + ".npy"), mmap_mode="r") for n in ("q", "k", "v"))
    rp = np.load(os.path.join(folder, "rp.npy"))
    ci = np.load(os.path.join(folder, "ci.npy"))
    t0 = time.time()
    n, flops = 0, 0.0
    for h in heads:
        for qb in range(nqb):
            if time.time() - t0 >= budget_s:
                return t0, time.time(), n, flops
            oracle.sparse_attention_rows(q, k, v, rp, ci, block, scale, seq_len, [(0, h, qb)])
            r = h * nqb + qb
            flops += tile_flops(block, d) * int(rp[r + 1] - rp[r])
            n += 1
    return t0, time.time(), n, flops


def cpu_baseline(q, k, v, rp, ci, cfg, budget_s, workers=None):
    """The float64 oracle on the same inputs and mask, as a pool over heads:
    one process per usable core (at most 16 and at most H), each with one BLAS
    thread, worker i taking heads i, i + W, ... and their query blocks in
    order until budget_s elapses.  The processes are started fresh (spawn),
    read the inputs from memory-mapped files, and run after the GPU work."""
    import multiprocessing as mp
    import shutil
    import tempfile
    from concurrent.futures import ProcessPoolExecutor
    host = host_info()
    usable = host["affinity"] or host["nproc"] or 1
    W = max(1, min(usable, 16, cfg.H) if workers is None else workers)
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    folder = tempfile.mkdtemp(prefix="calibatt_cpu_", dir=shm)
    saved = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        for n, a in (("q", q), ("k", k), ("v", v), ("rp", rp), ("ci", ci)):
            np.save(os.path.join(folder, n + ".npy"), np.ascontiguousarray(a))
        for n in saved:
            os.environ[n] = "1"
        jobs = [(folder, list(range(i, cfg.H, W)), budget_s, cfg.block, cfg.scale, cfg.S, cfg.nqb, cfg.d)
                for i in range(W)]
        # (a pool that raises if a worker dies, instead of starting new ones)
        with ProcessPoolExecutor(max_workers=W, mp_context=mp.get_context("spawn")) as pool:
            res = list(pool.map(_oracle_worker, jobs))
    finally:
        for n, val in saved.items():
            if val is None:
                os.environ.pop(n, None)
            else:
                os.environ[n] = val
        shutil.rmtree(folder, ignore_errors=True)
    t_start = min(r[0] for r in res)
    t_end = max(r[1] for r in res)
    n = sum(r[2] for r in res)
    flops = sum(r[3] for r in res)
    dt = t_end - t_start
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": W, "kind": "oracle",
            "sample": f"{n} of {cfg.rows} query blocks of the same inputs and mask, float64, {W} processes "
                      f"x 1 BLAS thread over heads (worker i: heads i, i+{W}, ..., blocks in order), "
                      f"{dt:.1f} s wall",
            "host": host}


def cpu_extra(q, k, v, cfg, budget_s):
    """The float64 oracle on the dense call and on the calibration pooling, each on
    whole query blocks in order until budget_s elapses, scaled to one full call."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except ImportError:
        threads = None
    out = {"process": "this one, serial over query blocks", "blas_threads": threads}
    nkv = cfg.nkb_valid
    rp = (np.arange(cfg.rows + 1) * nkv).astype(np.int32)
    ci = np.tile(np.arange(nkv), cfg.rows).astype(np.int32)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and n < cfg.rows:
        oracle.sparse_attention_rows(q, k, v, rp, ci, cfg.block, cfg.scale, cfg.S, [(0, n // cfg.nqb, n % cfg.nqb)])
        n += 1
    dt = time.perf_counter() - t0
    rate = tile_flops(cfg.block, cfg.d) * nkv * n / dt
    out["dense"] = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s",
                    "est_full_call_s": round(tile_flops(cfg.block, cfg.d) * nkv * cfg.rows / rate, 1),
                    "sample": f"{n} of {cfg.rows} query blocks in order, all keys, {dt:.1f} s"}
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and n < cfg.rows:
        h, qb = n // cfg.nqb, n % cfg.nqb
        oracle.block_mass_rows(q[0, h], k[0, h], cfg.block, cfg.scale, cfg.S, qb)
        n += 1
    dt = time.perf_counter() - t0
    out["block_mass"] = {"rows_per_s": round(n / dt, 3), "est_per_prompt_s": round(cfg.rows * dt / n, 1),
                         "sample": f"{n} of {cfg.rows} pooled query-block rows in order, {dt:.1f} s"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="wan", choices=["wan", "wan720", "mochi", "imbalance", "calib"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-calib", action="store_true")
    ap.add_argument("--no-anchor", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the block-sparse forward "
              "shards by head with no exchange, see the design notes", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch
    import synth
    import block_sparse_attention_calibatt_amd as cal

    cal.load()
    cfg = synth.get_config(args.config)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    calib_pipeline = None
    if cfg.name == "calib":
        # the mask comes from calibration on the GPU: pooled mass of each
        # prompt, top ceil(keep_frac * nkb) blocks per row, agreement of
        # ceil(rho * P) prompts, CSR; inference then runs on another input
        P = len(cfg.prompt_seeds)
        keep = -(-cfg.nkb * cfg.keep_frac.numerator // cfg.keep_frac.denominator)
        agree = -(-P * cfg.rho.numerator // cfg.rho.denominator)
        lse = torch.empty(cfg.B * cfg.H * cfg.L, dtype=torch.float32, device=dev)
        masses = torch.empty((P, cfg.H, cfg.nqb, cfg.nkb), dtype=torch.float32, device=dev)
        mws = torch.empty(cal.calibatt_block_mass_ws_bytes(cfg.B, cfg.H, cfg.L, cfg.block), dtype=torch.uint8,
                          device=dev)
        # every prompt's Q and K go to the GPU first (host generation leaves the
        # GPU idle, and a pooling timed right after an idle gap runs inside the
        # clock's ramp); then one untimed pooling, and the prompts back to back
        prompts = []
        for seed in cfg.prompt_seeds:
            qp, kp = synth.gen_qk(cfg, seed)
            prompts.append(tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (qp, kp)))
            del qp, kp
        cal.calibatt_block_mass_single_pass(prompts[0][0], prompts[0][1], cfg.block, cfg.scale, lse, masses[0], cfg.S,
                                            ws=mws)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for p, (Qp, Kp) in enumerate(prompts):
            cal.calibatt_block_mass_single_pass(Qp, Kp, cfg.block, cfg.scale, lse, masses[p], cfg.S, ws=mws)
        c1.record()
        torch.cuda.synchronize()
        pool_ms = c0.elapsed_time(c1)
        del prompts
        t_c = time.perf_counter()
        crp, cci = cal.calibatt_compile_masks(masses, keep, agree, cfg.nkb_valid)
        compile_ms = (time.perf_counter() - t_c) * 1e3
        sets = [(crp.cpu().numpy(), cci.cpu().numpy())]
        calib_pipeline = {"prompts": P, "keep_per_row": int(keep), "min_agree": int(agree),
                          "block_mass_ms_all_prompts": round(pool_ms, 2),
                          "compile_ms_incl_sync": round(compile_ms, 3),
                          "kept_blocks": int(cci.numel())}
        del masses, lse, mws
        q, k, v = synth.gen_qkv(cfg, cfg.infer_seed)
    else:
        q, k, v = synth.gen_qkv(cfg)
        sets = [synth.csr_for_config(cfg, t) for t in range(cfg.n_sets)]
    Q, K, V = (torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (q, k, v))
    O = torch.empty_like(Q)
    bank = cal.MaskBank(sets, cfg.H, cfg.nqb, cfg.nkb_valid, dev)
    qws = cal.new_queue(dev)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    stream = torch.cuda.current_stream(dev)

    def step(i):
        rp, ci, wo, _ = bank.lookup(i % len(bank))
        cal.calibatt_sparse_attn_fwd(Q, K, V, O, rp, ci, cfg.block, cfg.scale, cfg.S, wo, qws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    nnz_steps = [int(bank.nnz[i % len(bank)]) for i in range(args.steps)]
    flops = tile_flops(cfg.block, cfg.d) * cfg.B * float(np.mean(nnz_steps))
    value = flops / (ms * 1e-3) / 1e12
    achieved = float(np.mean([tile_flops(cfg.block, cfg.d) * cfg.B * n / (t * 1e-3) / 1e12
                              for n, t in zip(nnz_steps, launch_ms)]))
    density = float(np.mean(bank.nnz)) / (cfg.rows * cfg.nkb_valid)

    extra = {}
    if calib_pipeline is not None:
        extra["calibration_pipeline"] = calib_pipeline
    # one cold launch: L2 and MALL flushed by a 512 MB scratch write first
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    scratch.fill_(1)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rp0, ci0, wo0, _ = bank.lookup(0)
    c0.record(stream)
    cal.calibatt_sparse_attn_fwd(Q, K, V, O, rp0, ci0, cfg.block, cfg.scale, cfg.S, wo0, qws)
    c1.record(stream)
    torch.cuda.synchronize()
    del scratch
    extra["launch_ms_stats"] = {
        "median": round(float(np.median(launch_ms)), 4),
        "min": round(float(np.min(launch_ms)), 4),
        "cold_after_512MB_write": round(c0.elapsed_time(c1), 4),
    }

    if not args.no_sweep and cfg.name == "wan":
        # time vs kept density: the structured Wan masks (band + frame + position
        # + random fill) at several targets, and uniform random masks below
        # the structured floor.  Every mask is made on the host first, and the
        # points are timed back to back after the step has run again for a
        # while: after an idle gap (host work) the clock ramps up anew, and a
        # short low-density launch would be timed inside that ramp.
        sweep = []
        rng = np.random.default_rng(7)
        cases = [("random", 0.05), ("random", 0.10), ("random", 0.20), ("structured", 0.30),
                 ("structured", 0.50), ("structured", 0.70), ("structured", 0.90)]
        sbanks = []
        for kind, target in cases:
            m = (synth.random_csr(rng, cfg.H, cfg.nqb, cfg.nkb_valid, target) if kind == "random"
                 else synth.wan_csr(cfg, 0, target=target))
            sbanks.append((kind, cal.MaskBank([m], cfg.H, cfg.nqb, cfg.nkb_valid, dev, validate=False)))
        for i in range(25):
            step(i)
        for kind, sb in sbanks:
            srp, sci, swo, _ = sb.lookup(0)
            for _ in range(2):
                cal.calibatt_sparse_attn_fwd(Q, K, V, O, srp, sci, cfg.block, cfg.scale, cfg.S, swo, qws)
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(5):
                cal.calibatt_sparse_attn_fwd(Q, K, V, O, srp, sci, cfg.block, cfg.scale, cfg.S, swo, qws)
            s1.record(stream)
            torch.cuda.synchronize()
            t_ms = s0.elapsed_time(s1) / 5
            nnz = int(sb.nnz[0])
            sweep.append({"mask": kind, "density": round(nnz / (cfg.rows * cfg.nkb_valid), 4), "ms": round(t_ms, 4),
                          "tflops": round(tile_flops(cfg.block, cfg.d) * cfg.B * nnz / (t_ms * 1e-3) / 1e12, 1)})
        del sbanks
        extra["time_vs_density"] = sweep
        slope, icpt = np.polyfit([p["density"] for p in sweep], [p["ms"] for p in sweep], 1)
        extra["time_vs_density_fit"] = {"intercept_ms": round(float(icpt), 4), "ms_per_unit_density": round(float(slope), 3)}

    if not args.no_dense:
        for _ in range(2):
            cal.calibatt_dense_attn_fwd(Q, K, V, O, cfg.block, cfg.scale, cfg.S, qws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nd = 5
        e0.record(stream)
        for _ in range(nd):
            cal.calibatt_dense_attn_fwd(Q, K, V, O, cfg.block, cfg.scale, cfg.S, qws)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / nd
        dense_flops = tile_flops(cfg.block, cfg.d) * cfg.B * cfg.rows * cfg.nkb_valid
        extra["dense_ms"] = round(dense_ms, 4)
        extra["dense_tflops"] = round(dense_flops / (dense_ms * 1e-3) / 1e12, 2)
        extra["speedup_vs_dense"] = round(speedup(dense_ms, ms), 3)

    if not args.no_anchor and cfg.grid is not None:
        # anchor rows (spatial-repetition heads) for every head: the workload
        # of the pages' anchor-row table
        F, R, C = cfg.grid
        heads = list(range(cfg.H))
        nkv = cfg.nkb_valid
        rows_out = {}
        for ka in (15, 10, 5, 4, 3):
            aws = torch.empty(cal.calibatt_anchor_ws_bytes(cfg.B, cfg.H, F, C, ka, cfg.d), dtype=torch.uint8,
                              device=dev)
            for _ in range(2):
                cal.calibatt_anchor_attn_fwd(Q, K, V, O, heads, cfg.grid, ka, cfg.scale, cfg.S, qws, ws=aws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            na = 5
            e0.record(stream)
            for _ in range(na):
                cal.calibatt_anchor_attn_fwd(Q, K, V, O, heads, cfg.grid, ka, cfg.scale, cfg.S, qws, ws=aws)
            e1.record(stream)
            torch.cuda.synchronize()
            a_ms = e0.elapsed_time(e1) / na
            lq = -(-(F * ka * C) // 128) * 128
            a_flops = tile_flops(128, cfg.d) * cfg.B * cfg.H * (lq // 128) * nkv
            rows_out[f"k{ka}"] = {
                "ms": round(a_ms, 4),
                "row_sparsity": round(1 - ka / R, 4),
                "speedup_vs_dense": round(speedup(extra["dense_ms"], a_ms), 2) if "dense_ms" in extra else None,
                "anchor_tile_tflops": round(a_flops / (a_ms * 1e-3) / 1e12, 1),
                "parts_per_row": cal.calibatt_anchor_parts(cfg.B, cfg.H, cfg.grid, ka, cfg.L, cfg.S, cfg.d,
                                                           torch.cuda.get_device_properties(dev).multi_processor_count),
            }
            del aws
        extra["anchor_rows_all_heads"] = rows_out

    if not args.no_calib:
        # offline calibration steps on one prompt at this shape, then compile of 8 prompts' masses
        lse = torch.empty(cfg.B * cfg.H * cfg.L, dtype=torch.float32, device=dev)
        mass = torch.empty((8, cfg.H, cfg.nqb, cfg.nkb), dtype=torch.float32, device=dev)
        cal.calibatt_block_mass(Q, K, cfg.block, cfg.scale, lse, mass[0], cfg.S)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        for p in range(8):
            cal.calibatt_block_mass(Q, K, cfg.block, cfg.scale, lse, mass[p], cfg.S)
        e[1].record(stream)
        torch.cuda.synchronize()
        # the single-pass pooling of the same 8 prompts
        mws = torch.empty(cal.calibatt_block_mass_ws_bytes(cfg.B, cfg.H, cfg.L, cfg.block), dtype=torch.uint8,
                          device=dev)
        mass1 = torch.empty_like(mass)
        cal.calibatt_block_mass_single_pass(Q, K, cfg.block, cfg.scale, lse, mass1[0], cfg.S, ws=mws)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for p in range(8):
            cal.calibatt_block_mass_single_pass(Q, K, cfg.block, cfg.scale, lse, mass1[p], cfg.S, ws=mws)
        s1.record(stream)
        torch.cuda.synchronize()
        single_ms = s0.elapsed_time(s1) / 8
        single_diff = float(((mass1 - mass).abs() / mass.abs().clamp_min(1e-30)).max())
        del mass1, mws
        t_c = time.perf_counter()
        rp, ci = cal.calibatt_compile_masks(mass, cfg.nkb // 4, 4, cfg.nkb_valid)
        compile_s = time.perf_counter() - t_c
        t_c = time.perf_counter()
        rp_e, ci_e = cal.calibatt_compile_masks_energy(mass, 0.05, 4, cfg.nkb_valid)
        energy_s = time.perf_counter() - t_c
        wo = torch.empty(cfg.rows + 9, dtype=torch.int32, device=dev)
        e[2].record(stream)
        cal.calibatt_build_schedule(rp, cfg.H, cfg.nqb, wo)
        e[3].record(stream)
        torch.cuda.synchronize()
        pool_ms = e[0].elapsed_time(e[1]) / 8
        # the single pass makes one score product per (query, key): 2*B*H*S^2*d FLOP per prompt
        single_tf = 2.0 * cfg.B * cfg.H * cfg.S * cfg.S * cfg.d / (single_ms * 1e-3) / 1e12
        extra["calib"] = {
            "block_mass_ms_per_prompt": round(pool_ms, 3),
            "block_mass_qk_tflops": round(2 * 2.0 * cfg.B * cfg.H * cfg.S * cfg.S * cfg.d / (pool_ms * 1e-3) / 1e12, 2),
            "block_mass_single_pass_ms_per_prompt": round(single_ms, 3),
            "block_mass_single_pass_max_rel_diff": single_diff,
            "block_mass_single_pass_roofline": {"bound": "mfma", "achieved": round(single_tf, 1), "peak": PEAK_BF16_TFLOPS,
                                                "unit": "TFLOP/s", "frac": round(single_tf / PEAK_BF16_TFLOPS, 4)},
            "compile_ms_8_prompts_incl_sync": round(compile_s * 1e3, 3),
            "schedule_ms": round(e[2].elapsed_time(e[3]), 4),
            "compiled_density": round(ci.numel() / (cfg.rows * cfg.nkb_valid), 4),
            "energy_compile_ms_8_prompts_incl_sync": round(energy_s * 1e3, 3),
            "energy_compiled_density_eps_0.05": round(ci_e.numel() / (cfg.rows * cfg.nkb_valid), 4),
        }

    if not args.no_calib:
        # timestep sharing of 24 drifting Wan-shaped mask sets (IoU, runs, shared masks)
        tsets = synth.drifting_sets(cfg if cfg.name == "wan" else synth.get_config("wan"), 24)
        tbank = cal.MaskBank(tsets, cfg.H, cfg.nqb, cfg.nkb_valid, dev)
        tbank.share(0.95, cfg.nkb)
        torch.cuda.synchronize()
        t_s = time.perf_counter()
        sb = tbank.share(0.95, cfg.nkb)
        share_s = time.perf_counter() - t_s
        extra.setdefault("calib", {})["share_24_sets_tau_0.95"] = {
            "ms_incl_syncs": round(share_s * 1e3, 3), "shared_sets": sb.n_sets,
            "runs": [int(x) for x in sb.cluster_of]}
        # interval skip lists of the same 24 sets: trimmed, and merged at the 95th percentile
        sk = {}
        for pct in (100, 95):
            tbank.encode_skip_lists(pct, cfg.nkb)
            torch.cuda.synchronize()
            t_s = time.perf_counter()
            lists = tbank.encode_skip_lists(pct, cfg.nkb)
            enc_s = time.perf_counter() - t_s
            kept = int(lists.decode().nnz.sum())
            sk[f"merge_{pct}"] = {"encode_ms_incl_sync": round(enc_s * 1e3, 3), "width": lists.width,
                                  "widest": lists.widest, "MB": round(lists.size_bytes / 1e6, 2),
                                  "kept_blocks": kept, "kept_before": int(tbank.nnz.sum())}
        extra["calib"]["skip_lists_24_sets"] = sk

    if not args.no_calib and cfg.grid is not None:
        # spatial-similarity score of every head of one prompt
        sws = torch.empty(cal.calibatt_similarity_ws_bytes(cfg.B, cfg.H, cfg.L), dtype=torch.uint8, device=dev)
        sim = cal.calibatt_spatial_similarity(Q, K, cfg.scale, cfg.grid, cfg.S, ws=sws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            cal.calibatt_spatial_similarity(Q, K, cfg.scale, cfg.grid, cfg.S, sim=sim, ws=sws)
        e1.record(stream)
        torch.cuda.synchronize()
        sim_ms = e0.elapsed_time(e1) / 3
        # the same with the log-sum-exp of this prompt's single-pass pooling
        slse = torch.empty(cfg.B * cfg.H * cfg.L, dtype=torch.float32, device=dev)
        smass = torch.empty((cfg.B, cfg.H, cfg.nqb, cfg.nkb), dtype=torch.float32, device=dev)
        cal.calibatt_block_mass_single_pass(Q, K, cfg.block, cfg.scale, slse, smass, cfg.S)
        e0.record(stream)
        for _ in range(3):
            cal.calibatt_spatial_similarity(Q, K, cfg.scale, cfg.grid, cfg.S, sim=sim, ws=sws, lse=slse)
        e1.record(stream)
        torch.cuda.synchronize()
        sim_reuse_ms = e0.elapsed_time(e1) / 3
        del slse, smass
        # three score products per tile: the log-sum-exp pass and the two rows of each pair
        sim_flops = 3 * tile_flops(128, cfg.d) / 2 * cfg.B * cfg.H * cfg.nqb * cfg.nkb_valid
        extra.setdefault("calib", {})["spatial_similarity"] = {
            "ms_per_prompt": round(sim_ms, 3),
            "ms_per_prompt_with_pooling_lse": round(sim_reuse_ms, 3),
            "qk_tflops": round(sim_flops / (sim_ms * 1e-3) / 1e12, 1),
            "max_score": round(float(sim.max()), 4),
            "mean_score": round(float(sim.mean()), 4),
        }

    # the probe runs in its own process, after the timed work
    peak_probe = None if args.no_peak_probe else mfma_rate()
    mix = (peak_probe or {}).get("pooling_mix_cycles_per_wave_tile")
    if mix and "calib" in extra and cfg.block == 128 and cfg.d == 128:
        # the single pass's bound from the probe: per SIMD, its wave-tiles
        # (4 waves per 128-query block, one per 128-key tile) at the probe's
        # cycles per wave-tile for products and vector work together, at
        # the probe's clock; the pass runs its own clock, so this is a rate
        # bound in cycles more than in time
        wave_tiles = cfg.B * cfg.H * cfg.nqb * 4 * cfg.nkb_valid / (4 * peak_probe["cus"])
        bound_ms = wave_tiles * mix["both"] / (mix["clock_ghz"][2] * 1e9) * 1e3
        measured = extra["calib"]["block_mass_single_pass_ms_per_prompt"]
        extra["calib"]["block_mass_single_pass_mix_bound"] = {
            "bound": "matrix and vector issue on one SIMD (probe)", "wave_tiles_per_simd": round(wave_tiles),
            "cycles_per_wave_tile": mix["both"], "probe_clock_ghz": mix["clock_ghz"][2],
            "ms_at_probe_clock": round(bound_ms, 3), "frac": round(bound_ms / measured, 4)}

    cpu = cpu_more = None
    if not args.no_cpu:
        rp0, ci0 = sets[0]
        cpu = cpu_baseline(q, k, v, rp0, ci0, cfg, args.cpu_seconds)
        cpu_more = cpu_extra(q, k, v, cfg, args.cpu_seconds / 2.5)

    traffic = traffic_from_profile(cfg.name)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} H={cfg.H} L={cfg.L} (valid {cfg.S}) d={cfg.d} "
                        f"block={cfg.block}, {len(bank)} mask set(s), mean kept density {density:.4f}",
            "global_batch": cfg.B,
            "seq_len": cfg.S,
            "parallelism": "single GPU",
            "kept_blocks_per_step": float(np.mean(nnz_steps)),
            "launch": "persistent grid; heads spread over 8 per-XCD partitions longest first, rows longest first, atomic queue per partition with stealing",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic[0],
            "traffic_kind": "bytes L2 exchanged with the memory side per launch (FETCH_SIZE and WRITE_SIZE "
                            "scaled by a 1 GiB copy); includes reads the MALL serves, an upper bound on HBM bytes",
            "traffic_counters": traffic[1],
            "kernel": "attn_fwd_pp_kernel<128,false,false,false>",
            "avg_launch_ms": round(float(np.mean(launch_ms)), 4),
            "measured_mfma_rate": peak_probe,
            "frac_of_random_operand_rate": (round(achieved / peak_probe["random_operands_tflops"], 4)
                                            if peak_probe else None),
        },
        "cpu_baseline": cpu,
        "cpu_oracle_other_calls": cpu_more,
        "wall_s_timed": round(wall, 3),
        "input_setup_s": round(gen_s, 2),
    }
    line.update(extra)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
