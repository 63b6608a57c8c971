"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one split-K decode pass of the 16-stream workload (16 streams x 1
query row, 32/4 heads, head dim 256, bf16 K/V, depths U[1024, 32768] drawn
from seed, slices of 1024 keys): the decode kernel over every (stream, kv head,
slice) followed by the log-sum-exp combine.  `value` is the decode K/V stream
rate in GB/s (algorithmic bytes: every visible K and V row read once).

The same run times every other workload of the hot path on its own inputs,
each with its kernel alone and with the combine that follows it, as absolute
GB/s, TFLOP/s and tokens/s and as a fraction of its binding roof (the larger of
bytes / 8 TB/s and flops / 2.5 PFLOP/s):
  * the int8 verify-window decode (16 streams x 16 rows, 48/4 heads, depths
    12000 and 32000, slices of 2048), with causal windows and with each window
    a 16-node binary tree;
  * the split-K decode with e4m3 K/V rows and fp32 row scales;
  * the maskless selected-key prefill (2048 rows at positions 30000..32047,
    16/2 heads, 512 block ids per row over 4-cell blocks; 4*D flops per visited
    (row, head, key)) and the selected-key decode (16 rows, one per sequence of a
    unified cache, the key range split 32 ways, then the combine);
  * the tiny dense decode and the semantic-edge mask prefill (its 4096 keys
    split 8 ways, then the combine; the unsplit call, 64 work-groups, beside it);
  * measured roofs: a 1 GiB device copy (also the calibration of the memory
    counters), a bf16 8192^3 matmul, the issue rate of the two bf16 matrix-core
    product shapes the kernels use, and a gather probe that reads exactly the
    K/V blocks the selected-key prefill gathers; the selected-key prefill is
    also timed right after a 512 MiB write (cold Infinity Cache).
Then the FP64 oracle is timed on the host cores on bounded samples of the
split-K decode, the selected-key prefill and the depth-32000 verify decode.

Prints ONE JSON line.  Inputs are seeded synthetic data (no dataset).
"""

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
SEL_DECODE_SPLITS = 32         # key-range splits of the selected-key decode rows (16 rows x 2 kv heads each)
EDGE_SPLITS = 8                # key-range splits of the semantic-edge mask prefill (64 work-groups unsplit)

# HBM bytes of one decode launch on the split-K workload, from two rocprofv3 --pmc
# runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
# by what the same counter reads for the 1 GiB device copy (FETCH_SIZE reads half
# the copied bytes: factor 2.0; WRITE_SIZE reads them all: factor 1.0).  The
# figures describe the decode kernel's sources as they were when measured (the
# SHA-256 below); once those change they are stale and `traffic` is null.
DECODE_TRAFFIC = {"sources_sha256": "b25c9ae5cc3f49cd77d80eb004dd937cd2a10546ab478bdee629efb985e3441c",
                  "fetch_bytes": 592472.0 * 1024 * 2.0,
                  "write_bytes": 9701.48 * 1024 * 1.0}
# the files the decode kernel is built from
DECODE_SOURCES = ["arch.h", "common.h", "device_cache.h", "internal.h", "mfma_kernel.h", "lean_kernel.h", "mfma_decode.hip"]


def kernel_sources_sha256():
    """SHA-256 over the decode kernel's source files (names and contents, in order)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "split_flash_attention_amd", "csrc")
    for f in DECODE_SOURCES:
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_traffic():
    t = DECODE_TRAFFIC
    if t is None or t["sources_sha256"] != kernel_sources_sha256():
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def _tree_windows(np, gen):
    wl = gen.config5(32000)
    return dataclasses.replace(wl, tree_parent=np.tile(gen.heap_parents(16), (16, 1)).astype(np.int32),
                               name="int8_tree_verify_decode_d32000")


# decode workloads --only can time alone: name -> (np, gen) -> (workload, description)
ONLY = {
    "verify_decode_d12000": lambda np, gen: (gen.config5(12000), "int8 verify: 16 streams x 16-row causal windows, "
                                             "48/4 heads, D=256, depth 12000, slices of 2048"),
    "verify_decode_d32000": lambda np, gen: (gen.config5(32000), "int8 verify: 16 streams x 16-row causal windows, "
                                             "48/4 heads, D=256, depth 32000, slices of 2048"),
    "tree_verify_decode_d32000": lambda np, gen: (_tree_windows(np, gen), "int8 verify as at depth 32000, each "
                                                  "window a 16-node binary tree in heap order"),
    "fp8_decode": lambda np, gen: (gen.config2(kv_dtype="fp8"), "split-K decode as the headline with e4m3 K/V "
                                   "rows + fp32 row scales"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=sorted(ONLY) + ["sel_prefill"], default=None,
                    help="time one workload alone (for profiling) and print its figures")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle(fn, warmup, torch, min_s=0.3):
    """Untimed calls of `fn` before a measurement: at least `warmup` of them and at
    least `min_s` seconds of them, so that the clocks have left their idle state
    after the host-side generation of the workload."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 1
    while n < warmup or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed(fn, steps, torch):
    """Average ms of `fn` over `steps` back-to-back calls, HIP events on the current
    stream (the stream the library launches on)."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def timed_each(fn, n, torch):
    """Per-call ms of `fn` over n calls (HIP events around each call): (median, min)."""
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(s)
    for i in range(n):
        fn()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    d = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    return statistics.median(d), min(d)


def timed_cold(fn, flush, n, torch):
    """Median ms of `fn` right after `flush` (a write larger than the Infinity Cache)."""
    s = torch.cuda.current_stream()
    d = []
    for _ in range(n):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        torch.cuda.synchronize()
        d.append(e0.elapsed_time(e1))
    return statistics.median(d)


def roof_frac(nbytes, flops, ms):
    """Fraction of the binding roof: max(bytes / HBM peak, flops / MFMA peak) / time."""
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    return t_roof / (ms * 1e-3)


def decode_work(wl, np):
    """Algorithmic bytes (each visible K and V row once, row scales included) and flops
    (4*D per visited (row, query head, key)) of a decode workload."""
    row_bytes = wl.head_dim * (1 if wl.kv_dtype in ("i8", "fp8") else 2 if wl.kv_dtype != "f32" else 4)
    if wl.kv_dtype in ("i8", "fp8"):
        row_bytes += 4
    kv_len = np.asarray(wl.kv_len, np.int64)
    nbytes = int(kv_len.sum()) * wl.n_head_kv * row_bytes * 2
    R = wl.n_row
    keys = 0
    for n in kv_len:
        for r in range(R):
            if wl.tree_parent is not None:
                keys += int(n) - R + (r + 1).bit_length()          # binary heap: depth of node r + 1
            elif wl.causal:
                keys += int(n) - R + r + 1
            else:
                keys += int(n)
    flops = 4.0 * wl.head_dim * wl.n_head_q * keys
    return nbytes, flops


def time_decode(name, wl, steps, warmup, sa, hip_run, torch, np, workload_text):
    """Kernel-only and with-combine timings of one decode workload, after `warmup`
    untimed steps of it."""
    d = hip_run.DecodeDev(wl, "cuda", poison_outputs=False)
    a, c = d.args(), d.combine_args()

    def kernel():
        sa.sel_attn_decode(a)

    def step():
        sa.sel_attn_decode(a)
        sa.sel_attn_split_combine(c)

    settle(step, warmup, torch)
    ms_k = timed(kernel, steps, torch)
    ms_s = timed(step, steps, torch)
    k_med, k_min = timed_each(kernel, steps, torch)
    nbytes, flops = decode_work(wl, np)
    rows = wl.n_stream * wl.n_row
    out = {"workload": workload_text,
           "kernel_ms": round(ms_k, 5), "kernel_ms_median": round(k_med, 5), "kernel_ms_min": round(k_min, 5),
           "step_ms": round(ms_s, 5),
           "kv_bytes": nbytes, "gflop": round(flops / 1e9, 3),
           "gbs": round(nbytes / (ms_k * 1e-3) / 1e9, 2),
           "tflops": round(flops / (ms_k * 1e-3) / 1e12, 2),
           "hbm_peak_frac": round(nbytes / (ms_k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "mfma_peak_frac": round(flops / (ms_k * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "binding_roof_frac": round(roof_frac(nbytes, flops, ms_k), 4),
           "binding_roof_frac_step": round(roof_frac(nbytes, flops, ms_s), 4),
           "tokens_per_s": round(rows / (ms_s * 1e-3), 1),
           "decode_path": sa.decode_path(a)}
    del d
    return out


def gather_roof(wl, k, v, torch, np):
    """Achievable gather bandwidth for the selected-key workload's own access pattern:
    the probe reads exactly the K and V blocks the kernel gathers (one kv head's 4 x 512 B
    rows of each selected block), one (row, kv head) unit per wave in list order as the
    kernel does, and nothing else."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "tests", "probe", "libgather_probe.so"))
    lib.gather_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n_blocks = -(-wl.n_kv // wl.block_size)
    hkv = wl.n_head_kv
    ents, starts = [], [0]
    for r in range(wl.n_row):
        ids = wl.sel[r].astype(np.int64)
        ids = np.unique(ids[(ids >= 0) & (ids < n_blocks)])
        for g in range(hkv):
            kv_pair = np.stack([ids * hkv + g, (ids + n_blocks) * hkv + g], axis=1).reshape(-1)
            ents.append(kv_pair)                            # K block, then V block (V follows K)
            starts.append(starts[-1] + kv_pair.size)
    idx = torch.from_numpy(np.concatenate(ents).astype(np.int32)).cuda()
    ustart = torch.tensor(starts, dtype=torch.int32).cuda()
    n_units = len(starts) - 1
    kv = torch.cat([k.reshape(-1), v.reshape(-1)])          # [K cache][V cache], 16-bit elements
    row_bytes = wl.head_dim * 2
    groups = 1024
    out = torch.empty(groups * 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    per_unroll = {}
    for unroll in (4, 8, 16):
        def run():
            rc = lib.gather_probe(kv.data_ptr(), idx.data_ptr(), ustart.data_ptr(), n_units, hkv,
                                  wl.block_size * hkv * row_bytes, row_bytes, wl.block_size,
                                  hkv * row_bytes, out.data_ptr(), groups, unroll, stream)
            assert rc == 0, rc
        run()
        ms = timed_each(run, 10, torch)[1]
        per_unroll[unroll] = idx.numel() * wl.block_size * row_bytes / (ms * 1e-3) / 1e9
    return max(per_unroll.values()), per_unroll


def sel_cells(wl, np):
    """Visited cells of a selection workload: unique valid ids x block size, summed over rows."""
    n = 0
    for r in range(wl.n_row):
        ids = wl.sel[r]
        ok = (ids >= 0) & (ids.astype(np.int64) * wl.block_size < wl.n_kv)
        n += np.unique(ids[ok]).size * wl.block_size
    return n


def host_info():
    """The host the oracle runs on: core counts and the BLAS behind numpy."""
    info = {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        info["blas"] = [{"api": p.get("internal_api"), "threads": p.get("num_threads"),
                         "version": p.get("version")} for p in pools]
        info["threads"] = max([p.get("num_threads", 1) for p in pools] + [1])
    except Exception:
        info["threads"] = info["affinity_cpus"]
    return info


def cpu_baseline(wl2, wl3, wl5, np, budget_s=8.0):
    """The FP64 oracle (as it stands) on bounded samples: the split-K decode by whole
    streams, the selected-key prefill by rows, the verify decode by whole streams,
    each repeated in order until `budget_s` has passed."""
    import oracle
    res = {}
    # split-K decode: GB/s of K/V
    cells = n_calls = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = n_calls % wl2.n_stream
        sl = slice(b, b + 1)
        oracle.decode(q=wl2.q[sl], k=wl2.k[sl], v=wl2.v[sl], kv_dtype=wl2.kv_dtype, kv_len=wl2.kv_len[sl],
                      causal=wl2.causal, scale=wl2.scale)
        cells += int(wl2.kv_len[b])
        n_calls += 1
    dt = time.perf_counter() - t0
    res["split_k_decode"] = {"value": round(cells * wl2.n_head_kv * wl2.head_dim * 4 / dt / 1e9, 4),
                             "unit": "GB/s",
                             "sample": f"{n_calls} single-stream passes over the 16 streams in order, "
                                       f"{cells} cells x 32 query heads, {dt:.1f} s"}
    # selected-key prefill: TFLOP/s
    done = flops = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        r = done % wl3.n_row
        oracle.prefill(q=wl3.q, k=wl3.k, v=wl3.v, kv_dtype=wl3.kv_dtype, scale=wl3.scale, q_pos=wl3.q_pos,
                       sel=wl3.sel, block_size=wl3.block_size, rows=[r])
        ids = wl3.sel[r]
        ok = (ids >= 0) & (ids.astype(np.int64) * wl3.block_size < wl3.n_kv)
        flops += 4.0 * wl3.head_dim * wl3.n_head_q * np.unique(ids[ok]).size * wl3.block_size
        done += 1
    dt = time.perf_counter() - t0
    res["selected_key_prefill"] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                                   "sample": f"{done} of the 2048 rows in order, {dt:.1f} s"}
    # verify decode at depth 32000: TFLOP/s
    done = 0
    flops = 0.0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = done % wl5.n_stream
        sl = slice(b, b + 1)
        oracle.decode(q=wl5.q[sl], k=wl5.k[sl], v=wl5.v[sl], kv_dtype=wl5.kv_dtype, kv_len=wl5.kv_len[sl],
                      causal=True, scale=wl5.scale, k_scale=wl5.k_scale[sl], v_scale=wl5.v_scale[sl])
        n = int(wl5.kv_len[b])
        flops += sum(4.0 * wl5.head_dim * wl5.n_head_q * (n - wl5.n_row + r + 1) for r in range(wl5.n_row))
        done += 1
    dt = time.perf_counter() - t0
    res["int8_verify_decode_d32000"] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                                        "sample": f"{done} single-stream passes (16 rows x 48 heads), {dt:.1f} s"}
    return res


def time_sel_prefill(wl3, steps, warmup, sa, hip_run, torch, np):
    """The selected-key prefill workload: kernel timings (warm, one by one, and after a
    write that evicts the Infinity Cache) and its gather roof."""
    d3 = hip_run.PrefillDev(wl3, "cuda", poison_outputs=False)
    a3 = d3.args()

    def prefill():
        sa.sel_attn_prefill(a3)

    settle(prefill, warmup, torch)
    ms_prefill = timed(prefill, steps, torch)
    pre_med, pre_min = timed_each(prefill, steps, torch)
    flush_buf = torch.empty(1 << 27, dtype=torch.float32, device="cuda")       # 512 MiB
    ms_prefill_cold = timed_cold(prefill, lambda: flush_buf.fill_(0.5), 5, torch)
    del flush_buf
    gather_gbs, per_unroll = gather_roof(wl3, d3.k, d3.v, torch, np)
    n_cells = sel_cells(wl3, np)
    flops3 = 4.0 * wl3.head_dim * wl3.n_head_q * n_cells
    gather3 = n_cells * wl3.n_head_kv * wl3.head_dim * 2 * 2
    tflops3 = flops3 / (ms_prefill * 1e-3) / 1e12
    return {"workload": "2048 rows x 512 block ids (4-cell blocks), 16/2 heads, D=256, bf16",
            "ms": round(ms_prefill, 5), "ms_median": round(pre_med, 5),
            "ms_min": round(pre_min, 5), "ms_cold": round(ms_prefill_cold, 5),
            "gflop": round(flops3 / 1e9, 3),
            "tflops": round(tflops3, 3),
            "mfma_peak_frac": round(tflops3 / BF16_PEAK_TFLOPS, 5),
            "gathered_gbs": round(gather3 / (ms_prefill * 1e-3) / 1e9, 2),
            "gather_roof_gbs": round(gather_gbs, 1),
            "gather_roof_frac": round(gather3 / (ms_prefill * 1e-3) / 1e9 / gather_gbs, 4),
            "gather_probe_gbs_by_blocks_in_flight": {str(k): round(v, 1) for k, v in per_unroll.items()},
            "tokens_per_s": round(wl3.n_row / (ms_prefill * 1e-3), 1),
            "prefill_path": sa.prefill_path(a3)}


def memory_roofs(torch):
    """Read bandwidth (GB/s) of each level of the memory hierarchy, from the window
    probe: random 1 KiB chunks of a resident window of 16 KiB (L1), 2 MiB (L2 of each
    accelerator die), 64 MiB (Infinity Cache) and 2 GiB (HBM)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "tests", "probe", "libgather_probe.so"))
    lib.window_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    groups, iters = 2048, 1024
    out = torch.empty(groups * 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, kib in (("l1_16KiB", 16), ("l2_2MiB", 2048), ("infinity_cache_64MiB", 65536),
                      ("hbm_2GiB", 2 << 20)):
        buf = torch.ones(kib * 256, dtype=torch.float32, device="cuda")

        def run():
            rc = lib.window_read_probe(buf.data_ptr(), kib, iters, out.data_ptr(), groups, stream)
            assert rc == 0, rc
        for _ in range(3):
            run()
        ms = timed_each(run, 10, torch)[0]
        res[name] = round(groups * 4 * iters * 1024 / (ms * 1e-3) / 1e9, 1)
        del buf
    return res


def mfma_rates(torch):
    """Issue rate of the two bf16 matrix-core shapes the kernels use, from the MFMA
    probe: 256 work-groups of one wave per SIMD, 4 independent accumulator chains
    (throughput) and 1 chain (a dependent chain, as in a tile's score products).
    Returns {shape: {chains: (TFLOP/s over the chip, core cycles per product)}}."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "tests", "probe", "libmfma_probe.so"))
    lib.mfma_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    groups, iters = 256, 4096
    out = torch.empty(groups * 256, dtype=torch.float32, device="cuda")
    ticks = torch.empty(groups, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for shape, name, flop in ((32, "32x32x16_bf16", 32768.0), (16, "16x16x32_bf16", 16384.0)):
        res[name] = {}
        for chains in (4, 1):
            def run():
                rc = lib.mfma_rate_probe(shape, chains, iters, groups, out.data_ptr(), ticks.data_ptr(), stream)
                assert rc == 0, rc
            run()
            ms = timed_each(run, 5, torch)[0]
            torch.cuda.synchronize()
            cyc = float(ticks.double().median().item()) / (iters * chains)
            tflops = groups * 4 * iters * chains * flop / (ms * 1e-3) / 1e12
            res[name][f"chains_{chains}"] = {"tflops": round(tflops, 1), "cycles_per_product": round(cyc, 2)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import split_flash_attention_amd as sa
    from tests import hip_run
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sa.lib()

    if args.only == "sel_prefill":
        out = time_sel_prefill(gen.config3(), args.steps, args.warmup, sa, hip_run, torch, np)
        out["memory_read_gbs"] = memory_roofs(torch)
        print(json.dumps({"workload": args.only, args.only: out}), flush=True)
        return
    if args.only:
        wl, text = ONLY[args.only](np, gen)
        out = time_decode(args.only, wl, args.steps, args.warmup, sa, hip_run, torch, np, text)
        print(json.dumps({"workload": args.only, args.only: out}), flush=True)
        return

    # ---- the headline workload (host generation, then resident in HBM) ----------
    log("generating the split-K decode workload")
    wl2 = gen.config2()
    d2 = hip_run.DecodeDev(wl2, "cuda", poison_outputs=False)
    a2 = d2.args()
    c2 = d2.combine_args()

    def step():
        sa.sel_attn_decode(a2)
        sa.sel_attn_split_combine(c2)

    def decode_only():
        sa.sel_attn_decode(a2)

    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps -------------------------------------------
    log("timing the split-K decode")
    ms_step = timed(step, args.steps, torch)
    ms_decode = timed(decode_only, args.steps, torch)
    dec_med, dec_min = timed_each(decode_only, args.steps, torch)

    cells = int(np.asarray(wl2.kv_len, np.int64).sum())
    kv_bytes = cells * wl2.n_head_kv * wl2.head_dim * 2 * 2          # K and V, bf16
    gbs_step = kv_bytes / (ms_step * 1e-3) / 1e9
    gbs_kernel = kv_bytes / (ms_decode * 1e-3) / 1e9

    result = {
        "metric": "decode KV GB/s (% HBM peak) + sel-prefill TFLOP/s, GQA h256 at 32k depth",
        "value": round(gbs_step, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, depths U[1024,32768])",
        "config": {"workload": "split-K decode: 16 streams x 1 row, 32/4 heads, head dim 256, bf16 K/V, "
                               "depths U[1024,32768], slices of 1024, LSE combine",
                   "kv_bytes_per_step": kv_bytes, "decode_path": sa.decode_path(a2),
                   "hbm_peak_frac_step": round(gbs_step / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(gbs_kernel, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs_kernel / HBM_PEAK_GBS, 4),
                     "traffic": decode_traffic(),
                     "kernel": "decode (lean_attn_kernel<0, 2, 256, 2, false, false>: decode, bf16, D=256)",
                     "kernel_ms": round(ms_decode, 5),
                     "kernel_ms_median": round(dec_med, 5), "kernel_ms_min": round(dec_min, 5)},
        "tokens_per_s": round(wl2.n_stream / (ms_step * 1e-3), 1),
    }

    # ---- the other decode workloads ----------------------------------------------
    log("generating and timing the int8 verify-window decode at depth 12000")
    wl5a = gen.config5(12000)
    result["verify_decode_d12000"] = time_decode(
        "5a", wl5a, args.steps, args.warmup, sa, hip_run, torch, np,
        "int8 verify: 16 streams x 16-row causal windows, 48/4 heads, D=256, depth 12000, slices of 2048")
    del wl5a
    log("generating and timing the int8 verify-window decode at depth 32000 (chain and tree windows)")
    wl5 = gen.config5(32000)
    result["verify_decode_d32000"] = time_decode(
        "5b", wl5, args.steps, args.warmup, sa, hip_run, torch, np,
        "int8 verify: 16 streams x 16-row causal windows, 48/4 heads, D=256, depth 32000, slices of 2048")
    wl5t = dataclasses.replace(wl5, tree_parent=np.tile(gen.heap_parents(16), (16, 1)).astype(np.int32),
                               name="int8_tree_verify_decode_d32000")
    result["tree_verify_decode_d32000"] = time_decode(
        "5t", wl5t, args.steps, args.warmup, sa, hip_run, torch, np,
        "int8 verify as at depth 32000, each window a 16-node binary tree in heap order")
    del wl5t
    log("generating and timing the split-K decode with e4m3 K/V")
    wl2f = gen.config2(kv_dtype="fp8")
    result["fp8_decode"] = time_decode(
        "2f", wl2f, args.steps, args.warmup, sa, hip_run, torch, np,
        "split-K decode as the headline with e4m3 K/V rows + fp32 row scales")
    del wl2f

    # ---- selected-key prefill and decode ------------------------------------------
    log("selected-key prefill")
    wl3 = gen.config3()
    result["sel_prefill"] = time_sel_prefill(wl3, args.steps, args.warmup, sa, hip_run, torch, np)
    log("selected-key decode")
    wl6 = gen.sel_decode()
    d6 = hip_run.PrefillDev(wl6, "cuda", n_splits=SEL_DECODE_SPLITS, poison_outputs=False)
    a6 = d6.args()
    c6 = sa.combine_args(part_o=d6.part_o, part_ml=d6.part_ml, out=d6.out.view(1, *d6.out.shape))

    def sel_decode():
        sa.sel_attn_prefill(a6)
        sa.sel_attn_split_combine(c6)

    def sel_decode_kernel():
        sa.sel_attn_prefill(a6)

    settle(sel_decode, args.warmup, torch)
    ms_sd = timed(sel_decode, args.steps, torch)
    ms_sdk = timed(sel_decode_kernel, args.steps, torch)
    sd_med, sd_min = timed_each(sel_decode, args.steps, torch)
    cells6 = sel_cells(wl6, np)
    flops6 = 4.0 * wl6.head_dim * wl6.n_head_q * cells6
    gather6 = cells6 * wl6.n_head_kv * wl6.head_dim * 2 * 2
    result["sel_decode"] = {"workload": f"16 rows x 512 block ids (4-cell blocks), 16/2 heads, D=256, bf16, "
                                        f"N=32048, {SEL_DECODE_SPLITS} key-range splits + combine",
                            "kernel_ms": round(ms_sdk, 5), "step_ms": round(ms_sd, 5),
                            "step_ms_median": round(sd_med, 5), "step_ms_min": round(sd_min, 5),
                            "tflops": round(flops6 / (ms_sd * 1e-3) / 1e12, 3),
                            "gathered_gbs": round(gather6 / (ms_sd * 1e-3) / 1e9, 2),
                            "tokens_per_s": round(wl6.n_row / (ms_sd * 1e-3), 1)}
    del d6

    # ---- small workloads and measured roofs ---------------------------------------
    log("small workloads and roofs")
    wl1 = gen.config1()
    d1 = hip_run.DecodeDev(wl1, "cuda", poison_outputs=False)
    a1, c1 = d1.args(), d1.combine_args()

    def step1():
        sa.sel_attn_decode(a1)
        sa.sel_attn_split_combine(c1)

    step1()
    c1_med, c1_min = timed_each(step1, args.steps, torch)
    result["dense_decode_tiny"] = {"workload": "1 row, 4/1 heads, D=256, 64 fp32 keys, decode + combine",
                                   "us_median": round(c1_med * 1e3, 2), "us_min": round(c1_min * 1e3, 2)}
    small4 = {}
    for name, wl4 in (("4", gen.config4()), ("4c", gen.config4(nan=False))):
        # the timed launch: 8 key-range splits (512 work-groups), then the combine
        d4 = hip_run.PrefillDev(wl4, "cuda", n_splits=EDGE_SPLITS, poison_outputs=False)
        a4, c4 = d4.args(), sa.combine_args(part_o=d4.part_o, part_ml=d4.part_ml,
                                            out=d4.out.view(1, *d4.out.shape), sinks=d4.sinks)

        def step4():
            sa.sel_attn_prefill(a4)
            sa.sel_attn_split_combine(c4)

        settle(step4, args.warmup, torch)
        small4[name] = timed_each(step4, args.steps, torch)
        del d4
        if name == "4":
            d4u = hip_run.PrefillDev(wl4, "cuda", poison_outputs=False)
            a4u = d4u.args()
            sa.sel_attn_prefill(a4u)
            small4["4u"] = timed_each(lambda: sa.sel_attn_prefill(a4u), args.steps, torch)
            del d4u
    result["semantic_edge_prefill"] = {"workload": "256 rows x 4096 keys, 16/4 heads, D=128, fp16, softcap, "
                                                   f"ALiBi, F32 mask (with NaN K / control without), "
                                                   f"{EDGE_SPLITS} key-range splits + combine",
                                       "us_median": round(small4["4"][0] * 1e3, 2),
                                       "us_median_control": round(small4["4c"][0] * 1e3, 2),
                                       "us_median_unsplit": round(small4["4u"][0] * 1e3, 2)}
    copy_src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")     # 1 GiB
    copy_dst = torch.empty_like(copy_src)
    copy_src.fill_(1.0)
    copy_dst.copy_(copy_src)
    ms_copy = timed(lambda: copy_dst.copy_(copy_src), max(3, args.steps // 4), torch)
    del copy_src, copy_dst
    mm_a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    mm_b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    mm_c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
    torch.matmul(mm_a, mm_b, out=mm_c)
    ms_mm = timed_each(lambda: torch.matmul(mm_a, mm_b, out=mm_c), 10, torch)[1]
    del mm_a, mm_b, mm_c
    copy_gbs = 2 * (1 << 28) * 4 / (ms_copy * 1e-3) / 1e9
    result["roofs"] = {"hbm_peak_gbs": HBM_PEAK_GBS, "bf16_mfma_peak_tflops": BF16_PEAK_TFLOPS,
                       "copy_gbs": round(copy_gbs, 1),
                       "bf16_matmul_tflops": round(2.0 * 8192 ** 3 / (ms_mm * 1e-3) / 1e12, 1),
                       "sel_gather_gbs": result["sel_prefill"]["gather_roof_gbs"],
                       "mfma_rates": mfma_rates(torch)}
    result["copy_gbs"] = round(copy_gbs, 1)

    if not args.no_cpu_baseline:
        log("timing the FP64 oracle on samples")
        info = host_info()
        cb = cpu_baseline(wl2, wl3, wl5, np)
        head = cb["split_k_decode"]
        result["cpu_baseline"] = {"value": head["value"], "unit": head["unit"], "cores": int(info["threads"]),
                                  "kind": "oracle", "sample": "split-K decode workload: " + head["sample"],
                                  "others": {k: v for k, v in cb.items() if k != "split_k_decode"},
                                  "host": info}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
