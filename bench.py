"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--verify]

One step = one split-K decode pass of the 16-stream workload (16 streams x 1
query row, 32/4 heads, head dim 256, bf16 K/V, depths U[1024, 32768] drawn
from seed, slices of 1024 keys): the decode kernel over every (stream, kv head,
slice) followed by the log-sum-exp combine.  `value` is the decode K/V stream
rate in GB/s (algorithmic bytes: every visible K and V row read once).

The same run also times the maskless selected-key prefill (2048 rows at
positions 30000..32047, 16/2 heads, head dim 256, bf16, 512 block ids per row
over 4-cell blocks) and reports its TFLOP/s (4*D flops per visited (row, head,
key)), the selected-key decode (16 rows, one per sequence of a unified cache, with
the same lists and block size, the key range split 32 ways, then the combine),
and a plain device copy of 1 GiB (the achievable copy rate, and the
calibration for the memory counters).  Beside them: per-launch median and
minimum times, the selected-key prefill right after a 512 MiB write (cold
Infinity Cache), measured roofs (a bf16 8192^3 matmul, and a gather probe that
reads exactly the K/V blocks the selected-key prefill gathers), the tiny dense
decode and the semantic-edge mask prefill.  `--verify` adds the int8
verify-window decode (16 streams x 16 rows, 48/4 heads, depth 32000, slices of
2048) with chain and tree windows, and the split-K decode with e4m3 K/V rows.

Prints ONE JSON line.  Inputs are seeded synthetic data (no dataset).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
SEL_DECODE_SPLITS = 32         # key-range splits of the selected-key decode rows (16 rows x 2 kv heads each)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

# HBM bytes of one decode launch on the split-K workload, from two rocprofv3 --pmc
# runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled
# by what the same counter reads for the 1 GiB device copy (FETCH_SIZE reads half
# the copied bytes: factor 2.0; WRITE_SIZE reads them all: factor 1.0).  The
# figures describe the decode kernel's sources as they were when measured (the
# SHA-256 below); once those change they are stale and `traffic` is null.
DECODE_TRAFFIC = {"sources_sha256": "7273fdf1521d6310c25d72804953745323174e3fc50f00013c325ad4d132b1cf",
                  "fetch_bytes": 592916.47 * 1024 * 2.0,
                  "write_bytes": 10594.20 * 1024 * 1.0}
# the files the decode kernel is built from
DECODE_SOURCES = ["arch.h", "common.h", "internal.h", "mfma_kernel.h", "lean_kernel.h", "mfma_decode.hip"]


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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--verify", action="store_true", help="also time the int8 verify-window decode")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def timed(fn, steps, torch):
    """Average ms of `fn` over `steps` back-to-back calls, HIP events on the current stream."""
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
    import statistics
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
    import statistics
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
    best = 0.0
    for unroll in (4, 8, 16):
        def run():
            rc = lib.gather_probe(kv.data_ptr(), idx.data_ptr(), ustart.data_ptr(), n_units, hkv,
                                  wl.block_size * hkv * row_bytes, row_bytes, wl.block_size,
                                  hkv * row_bytes, out.data_ptr(), groups, unroll, stream)
            assert rc == 0, rc
        run()
        ms = timed_each(run, 10, torch)[1]
        best = max(best, idx.numel() * wl.block_size * row_bytes / (ms * 1e-3) / 1e9)
    return best


def cpu_baseline_decode(wl, min_seconds=12.0):
    """The FP64 oracle (as it stands) on a bounded sample of the decode workload:
    its streams one at a time, in order, until `min_seconds` have passed."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cells = 0
    n_calls = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        b = n_calls % wl.n_stream
        sl = slice(b, b + 1)
        oracle.decode(q=wl.q[sl], k=wl.k[sl], v=wl.v[sl], kv_dtype=wl.kv_dtype, kv_len=wl.kv_len[sl],
                      causal=wl.causal, scale=wl.scale)
        cells += int(wl.kv_len[b])
        n_calls += 1
    # (the whole workload takes about 1.4 s on 16 cores, so the sample repeats it)
    dt = time.perf_counter() - t0
    nbytes = cells * wl.n_head_kv * wl.head_dim * 2 * 2
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"split-K decode workload: {n_calls} single-stream passes over its 16 streams "
                      f"in order, {cells} cells x 32 query heads, {dt:.1f} s"}


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

    # ---- inputs (host generation, then resident in HBM) --------------------------
    log("generating the split-K decode workload")
    wl2 = gen.config2()
    d2 = hip_run.DecodeDev(wl2, "cuda", poison_outputs=False)
    a2 = d2.args()
    c2 = d2.combine_args()
    log("generating the selected-key prefill workload")
    wl3 = gen.config3()
    d3 = hip_run.PrefillDev(wl3, "cuda", poison_outputs=False)
    a3 = d3.args()
    log("generating the selected-key decode workload")
    wl6 = gen.sel_decode()
    d6 = hip_run.PrefillDev(wl6, "cuda", n_splits=SEL_DECODE_SPLITS, poison_outputs=False)
    a6 = d6.args()
    c6 = sa.combine_args(part_o=d6.part_o, part_ml=d6.part_ml, out=d6.out.view(1, *d6.out.shape))
    copy_src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")     # 1 GiB
    copy_dst = torch.empty_like(copy_src)
    copy_src.fill_(1.0)

    def step():
        sa.sel_attn_decode(a2)
        sa.sel_attn_split_combine(c2)

    def decode_only():
        sa.sel_attn_decode(a2)

    def prefill():
        sa.sel_attn_prefill(a3)

    def copy():
        copy_dst.copy_(copy_src)

    def sel_decode():
        sa.sel_attn_prefill(a6)
        sa.sel_attn_split_combine(c6)

    log("warmup")
    for _ in range(args.warmup):
        step()
        prefill()
        sel_decode()
        copy()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps -------------------------------------------
    log("timing")
    ms_step = timed(step, args.steps, torch)
    ms_decode = timed(decode_only, args.steps, torch)
    ms_prefill = timed(prefill, args.steps, torch)
    ms_copy = timed(copy, max(3, args.steps // 4), torch)
    ms_sd = timed(sel_decode, args.steps, torch)
    dec_med, dec_min = timed_each(decode_only, args.steps, torch)
    pre_med, pre_min = timed_each(prefill, args.steps, torch)
    sd_med, sd_min = timed_each(sel_decode, args.steps, torch)

    # ---- more figures: cold selected-key prefill, measured roofs, the small workloads --
    log("cold runs, roofs and the small workloads")
    flush_buf = torch.empty(1 << 27, dtype=torch.float32, device="cuda")       # 512 MiB
    ms_prefill_cold = timed_cold(prefill, lambda: flush_buf.fill_(0.5), 5, torch)
    del flush_buf
    gather_gbs = gather_roof(wl3, d3.k, d3.v, torch, np)
    mm_a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    mm_b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16).contiguous()
    mm_c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
    torch.matmul(mm_a, mm_b, out=mm_c)
    ms_mm = timed_each(lambda: torch.matmul(mm_a, mm_b, out=mm_c), 10, torch)[1]
    matmul_tflops = 2.0 * 8192 ** 3 / (ms_mm * 1e-3) / 1e12
    del mm_a, mm_b, mm_c
    wl1 = gen.config1()
    d1 = hip_run.DecodeDev(wl1, "cuda", poison_outputs=False)
    a1, c1 = d1.args(), d1.combine_args()

    def step1():
        sa.sel_attn_decode(a1)
        sa.sel_attn_split_combine(c1)

    step1()
    c1_med, c1_min = timed_each(step1, args.steps, torch)
    small4 = {}
    for name, wl4 in (("4", gen.config4()), ("4c", gen.config4(nan=False))):
        d4 = hip_run.PrefillDev(wl4, "cuda", poison_outputs=False)
        a4 = d4.args()
        sa.sel_attn_prefill(a4)
        small4[name] = timed_each(lambda: sa.sel_attn_prefill(a4), args.steps, torch)
        del d4

    cells = int(np.asarray(wl2.kv_len, np.int64).sum())
    kv_bytes = cells * wl2.n_head_kv * wl2.head_dim * 2 * 2          # K and V, bf16
    gbs_step = kv_bytes / (ms_step * 1e-3) / 1e9
    gbs_kernel = kv_bytes / (ms_decode * 1e-3) / 1e9

    # selected-key prefill work: 4*D flops per visited (row, query head, key)
    n_cells = 0
    for r in range(wl3.n_row):
        ids = wl3.sel[r]
        ok = (ids >= 0) & (ids.astype(np.int64) * wl3.block_size < wl3.n_kv)
        n_cells += np.unique(ids[ok]).size * wl3.block_size
    flops3 = 4.0 * wl3.head_dim * wl3.n_head_q * n_cells
    gather3 = n_cells * wl3.n_head_kv * wl3.head_dim * 2 * 2
    tflops3 = flops3 / (ms_prefill * 1e-3) / 1e12

    def sel_cells(wl):
        n = 0
        for r in range(wl.n_row):
            ids = wl.sel[r]
            ok = (ids >= 0) & (ids.astype(np.int64) * wl.block_size < wl.n_kv)
            n += np.unique(ids[ok]).size * wl.block_size
        return n

    cells6 = sel_cells(wl6)
    flops6 = 4.0 * wl6.head_dim * wl6.n_head_q * cells6
    gather6 = cells6 * wl6.n_head_kv * wl6.head_dim * 2 * 2

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
                     "kernel": "decode (lean_attn_kernel<0, 2, 256>: decode, bf16, D=256)",
                     "kernel_ms": round(ms_decode, 5),
                     "kernel_ms_median": round(dec_med, 5), "kernel_ms_min": round(dec_min, 5)},
        "sel_prefill": {"workload": "2048 rows x 512 block ids (4-cell blocks), 16/2 heads, D=256, bf16",
                        "ms": round(ms_prefill, 5), "ms_median": round(pre_med, 5),
                        "ms_min": round(pre_min, 5), "ms_cold": round(ms_prefill_cold, 5),
                        "tflops": round(tflops3, 3),
                        "mfma_peak_frac": round(tflops3 / BF16_PEAK_TFLOPS, 5),
                        "gathered_gbs": round(gather3 / (ms_prefill * 1e-3) / 1e9, 2),
                        "gather_roof_gbs": round(gather_gbs, 1),
                        "gather_roof_frac": round(gather3 / (ms_prefill * 1e-3) / 1e9 / gather_gbs, 4),
                        "tokens_per_s": round(wl3.n_row / (ms_prefill * 1e-3), 1),
                        "prefill_path": sa.prefill_path(a3)},
        "sel_decode": {"workload": f"16 rows x 512 block ids (4-cell blocks), 16/2 heads, D=256, bf16, "
                                   f"N=32048, {SEL_DECODE_SPLITS} key-range splits + combine",
                       "ms": round(ms_sd, 5), "ms_median": round(sd_med, 5), "ms_min": round(sd_min, 5),
                       "tflops": round(flops6 / (ms_sd * 1e-3) / 1e12, 3),
                       "gathered_gbs": round(gather6 / (ms_sd * 1e-3) / 1e9, 2),
                       "tokens_per_s": round(wl6.n_row / (ms_sd * 1e-3), 1)},
        "dense_decode_tiny": {"workload": "1 row, 4/1 heads, D=256, 64 fp32 keys, decode + combine",
                              "us_median": round(c1_med * 1e3, 2), "us_min": round(c1_min * 1e3, 2)},
        "semantic_edge_prefill": {"workload": "256 rows x 4096 keys, 16/4 heads, D=128, fp16, softcap, "
                                              "ALiBi, F32 mask (with NaN K / control without)",
                                  "us_median": round(small4["4"][0] * 1e3, 2),
                                  "us_median_control": round(small4["4c"][0] * 1e3, 2)},
        "roofs": {"hbm_peak_gbs": HBM_PEAK_GBS, "bf16_mfma_peak_tflops": BF16_PEAK_TFLOPS,
                  "copy_gbs": round(2 * copy_src.numel() * 4 / (ms_copy * 1e-3) / 1e9, 1),
                  "bf16_matmul_tflops": round(matmul_tflops, 1),
                  "sel_gather_gbs": round(gather_gbs, 1)},
        "copy_gbs": round(2 * copy_src.numel() * 4 / (ms_copy * 1e-3) / 1e9, 1),
        "tokens_per_s": round(wl2.n_stream / (ms_step * 1e-3), 1),
    }

    if args.verify:
        log("generating the int8 verify-window workload at depth 12000")
        wl5a = gen.config5(12000)
        d5a = hip_run.DecodeDev(wl5a, "cuda", poison_outputs=False)
        a5a, c5a = d5a.args(), d5a.combine_args()

        def step5a():
            sa.sel_attn_decode(a5a)
            sa.sel_attn_split_combine(c5a)

        step5a()
        ms5a = timed(step5a, args.steps, torch)
        bytes5a = int(np.asarray(wl5a.kv_len, np.int64).sum()) * wl5a.n_head_kv * (wl5a.head_dim + 4) * 2
        flops5a = sum(4.0 * wl5a.head_dim * wl5a.n_head_q * wl5a.n_stream * (int(wl5a.kv_len[0]) - wl5a.n_row + r + 1)
                      for r in range(wl5a.n_row))
        result["verify_decode_d12000"] = {"workload": "int8 verify: 16 streams x 16 rows, 48/4 heads, D=256, depth 12000",
                                          "ms": round(ms5a, 5), "gbs": round(bytes5a / (ms5a * 1e-3) / 1e9, 2),
                                          "tflops": round(flops5a / (ms5a * 1e-3) / 1e12, 2),
                                          "tokens_per_s": round(wl5a.n_stream * wl5a.n_row / (ms5a * 1e-3), 1)}
        del d5a
        log("generating the int8 verify-window workload at depth 32000")
        wl5 = gen.config5(32000)
        d5 = hip_run.DecodeDev(wl5, "cuda", poison_outputs=False)
        a5, c5 = d5.args(), d5.combine_args()

        def step5():
            sa.sel_attn_decode(a5)
            sa.sel_attn_split_combine(c5)

        step5()
        ms5 = timed(step5, args.steps, torch)
        cells5 = int(np.asarray(wl5.kv_len, np.int64).sum())
        bytes5 = cells5 * wl5.n_head_kv * (wl5.head_dim + 4) * 2
        flops5 = 0.0
        for r in range(wl5.n_row):
            flops5 += 4.0 * wl5.head_dim * wl5.n_head_q * wl5.n_stream * (int(wl5.kv_len[0]) - wl5.n_row + r + 1)
        roof5 = max(bytes5 / (HBM_PEAK_GBS * 1e9), flops5 / (BF16_PEAK_TFLOPS * 1e12)) * 1e3   # ms
        result["verify_decode"] = {"workload": "int8 verify: 16 streams x 16 rows, 48/4 heads, D=256, depth 32000",
                                   "ms": round(ms5, 5), "gbs": round(bytes5 / (ms5 * 1e-3) / 1e9, 2),
                                   "hbm_peak_frac": round(bytes5 / (ms5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "tflops": round(flops5 / (ms5 * 1e-3) / 1e12, 2),
                                   "mfma_peak_frac": round(flops5 / (ms5 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                   "binding_roof_frac": round(roof5 / ms5, 4),
                                   "tokens_per_s": round(wl5.n_stream * wl5.n_row / (ms5 * 1e-3), 1)}
        del d5
        log("generating the int8 tree verify-window workload")
        wl5t = gen.config5(32000, tree="heap")
        d5t = hip_run.DecodeDev(wl5t, "cuda", poison_outputs=False)
        a5t, c5t = d5t.args(), d5t.combine_args()

        def step5t():
            sa.sel_attn_decode(a5t)
            sa.sel_attn_split_combine(c5t)

        step5t()
        ms5t = timed(step5t, args.steps, torch)
        # visible keys of heap node r: the cached prefix plus floor(log2(r + 1)) + 1 window nodes
        flops5t = 0.0
        for r in range(wl5t.n_row):
            vis = int(wl5t.kv_len[0]) - wl5t.n_row + (r + 1).bit_length()
            flops5t += 4.0 * wl5t.head_dim * wl5t.n_head_q * wl5t.n_stream * vis
        result["tree_verify_decode"] = {"workload": "int8 verify as above, each window a 16-node binary "
                                                    "tree in heap order",
                                        "ms": round(ms5t, 5), "gbs": round(bytes5 / (ms5t * 1e-3) / 1e9, 2),
                                        "tflops": round(flops5t / (ms5t * 1e-3) / 1e12, 2)}
        del d5t
        log("generating the split-K decode workload with e4m3 K/V")
        wl2f = gen.config2(kv_dtype="fp8")
        d2f = hip_run.DecodeDev(wl2f, "cuda", poison_outputs=False)
        a2f, c2f = d2f.args(), d2f.combine_args()

        def step2f():
            sa.sel_attn_decode(a2f)
            sa.sel_attn_split_combine(c2f)

        step2f()
        ms2f = timed(step2f, args.steps, torch)
        bytes2f = cells * wl2f.n_head_kv * (wl2f.head_dim + 4) * 2         # e4m3 rows + fp32 scales
        result["fp8_decode"] = {"workload": "split-K decode as above with e4m3 K/V rows + fp32 row scales",
                                "ms": round(ms2f, 5), "gbs": round(bytes2f / (ms2f * 1e-3) / 1e9, 2),
                                "hbm_peak_frac": round(bytes2f / (ms2f * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "tokens_per_s": round(wl2f.n_stream / (ms2f * 1e-3), 1)}
        del d2f

    if not args.no_cpu_baseline:
        log("timing the FP64 oracle on a sample")
        result["cpu_baseline"] = cpu_baseline_decode(wl2)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
