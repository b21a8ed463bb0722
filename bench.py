"""Benchmark of paged decode attention on one MI355X: the five workloads.

    python bench.py [--steps K] [--warmup W] [--workload all|decode7b|mixed|beam|gqa|...]
                    [--partition P] [--algo auto|wave|mfma] [--no-cpu-baseline]
                    [--calib-copy-mib M]

The default (--workload all) prints ONE JSON line.  Its `value` is the
headline: the 7B-shape decode step (64 sequences, 32 query heads = 32 KV
heads, head_dim 128, 16-token blocks, contexts uniform on [128, 2048], each
including the token being decoded; a pool of ceil(1.25 x the blocks needed)
whose free list starts as a seeded permutation; q/K/V drawn N(0, 1) in fp32
and rounded to bf16).  One step (timed, inputs resident in HBM) is one
launch of the decode step kernel: it writes each sequence's new K/V rows at
its last position through the block table and attends every key, that row
included (2,048-token partitions cover every context, so there is no split
and no reduce).  The three-launch form (reshape_and_cache through the slot
mapping -> split-K decode -> partition reduce) is timed beside it as
`three_launch_step`.  `value` is step algorithmic bytes (K/V rows every
sequence attends to, q, out, the table entries and lengths read, the new
rows written) per second.  `roofline` is the step kernel's, from HIP events
on its stream.

The same line carries the other four workloads as keys of their own, each
with its step time, per-kernel times (mean, median, p10, p90), its own
roofline, the sampled error against the CPU oracle and the oracle timed on a
bounded sample:
  c3_mixed     continuous-batching step: 48 decode sequences (contexts
               U[64, 4096]) + 4 chunked-prefill sequences of 512 causal rows
               over 0/512/1024/1536 cached tokens, with reshape_and_cache of
               the 2,096 new rows; prefill reported in TFLOP/s against the
               bf16 matrix peak;
  c4_beam      16 requests sharing a 1,024-token prefix, 1-200 own tokens,
               beam width 4: copy_blocks of the shared partial tails +
               reshape_and_cache + decode; its K/V working set is cache
               resident, so the HBM roofline uses unique bytes and the
               logical bytes (shared blocks once per beam) are reported
               separately against no HBM bound;
  c5_gqa_bf16  16 sequences, 64 query heads over 8 KV heads (group 8,
               matrix cores), head_dim 128, contexts U[8192, 32768], bf16
               KV: split-K decode that appends the current token's rows in
               the same launch, + reduce, with the partition the library
               picks for these lengths (pkv_decode_partition_tokens: the
               shortest whose workgroups fill one round of the resident
               ones; --partition overrides it);
  c5_gqa_int8  the same with int8 KV and per-block fp32 scales (the pool is
               the library's block encoder output over the bf16 pool; the
               current token goes in by quantise-on-write, then decode +
               reduce).

Timing: W untimed warm-up steps, then K steps back to back between two
device synchronisations (the step time), then a second pass of K steps, each
after a 512 MB read that flushes the caches, with HIP events on the launch
stream around every kernel (the per-kernel times).

Other --workload values print the line of one workload on its own (and the
kernels that no default line covers: int8/4-bit storage, swapping, prefix
caching, long-document prefill).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/f16 matrix peak, published
BLOCK = 16
METRIC = "paged decode attention: KV GB/s (% of HBM peak) + tokens/s at 7B shape"
PAGE_ALLOC_P99_BAR_US = 1000.0   # cnnetsun.cn section 4.2: page allocation P99 < 1 ms

# HBM traffic of a workload's main kernel per launch, from two rocprofv3
# --pmc passes over the bench (FETCH_SIZE scaled by 1 / the factor that a
# known-size copy kernel shows in the same run, WRITE_SIZE as read), with the
# profile that records the counts.  Valid only while the kernel sources hash
# to the measured value; a changed kernel reports null.
# HBM bytes per step of the dominant kernel(s), from rocprofv3 counter runs:
# FETCH_SIZE scaled by 1 / 0.500041 (a 1 GiB torch.bitwise_not in the same
# process reads as 524,331 KiB) plus WRITE_SIZE (exact for the same copy).
# Reported only while the kernel sources hash to the value they were taken on.
_SHA = "f48f9e8ac13d99de29020f47717904dc89d5ee1d"
TRAFFIC = {
    "decode7b": {"bytes_per_launch": 1120485706, "sources_sha1": _SHA, "partition_tokens": 2048,
                 "profile": "profiles/decode_wave_7b_bf16_p2048_step_kernel_trace.md"},
    "gqa-bf16": {"bytes_per_launch": 1544128461, "sources_sha1": _SHA, "partition_tokens": 6448,
                 "profile": "profiles/decode_mfma_gqa_long_bf16_kernel_trace.md"},
    "gqa-int8": {"bytes_per_launch": 828921235, "sources_sha1": _SHA, "partition_tokens": 2048,
                 "profile": "profiles/decode_mfma_gqa_long_int8_kernel_trace.md"},
    "gqa-int4": {"bytes_per_launch": 446596696, "sources_sha1": _SHA, "partition_tokens": 1504,
                 "profile": "profiles/decode_mfma_gqa_long_int4_kernel_trace.md"},
}
KERNEL_SOURCES = ("decode_wave.hip", "decode_mfma.hip", "reduce.hip", "attention_common.h",
                  "device_common.h", "mfma_common.h")


def kernel_sources_sha1() -> str:
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_366_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_of(name: str, part: int):
    """(bytes per step of the roofline's kernels or None, where the figure
    comes from)."""
    t = TRAFFIC.get(name)
    if t is None:
        return None, "not measured for this workload"
    if t["partition_tokens"] != part:
        return None, f"measured at {t['partition_tokens']}-token partitions, not {part}"
    if t["sources_sha1"] != kernel_sources_sha1():
        return None, (f"stale: kernel sources changed since the counter run in {t['profile']}")
    return t["bytes_per_launch"], (f"rocprofv3 --pmc FETCH_SIZE (scaled by the calibration copy) "
                                   f"+ WRITE_SIZE, {t['profile']}")


# ---------------------------------------------------------------------------
# host-side helpers
# ---------------------------------------------------------------------------
def W_blocks(n, block_size: int = BLOCK) -> int:
    return -(-int(n) // block_size)


def to_dev_bf16(x, torch):
    from synth import workloads as W
    bits = W.storage_array(x, "bf16").view(np.int16)
    return torch.from_numpy(bits).to("cuda").view(torch.bfloat16)


def stats_ms(xs):
    a = np.asarray(xs, np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90))}


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover - informational only
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        blas = None
    return {"cpu_model": model, "host_cores_visible": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas_threads": blas}


class OracleClock:
    """Wall and CPU time of the oracle calls made through it."""

    def __init__(self):
        self.wall = 0.0
        self.cpu = 0.0

    def __call__(self, fn, *args, **kw):
        c0, t0 = time.process_time(), time.perf_counter()
        r = fn(*args, **kw)
        self.wall += time.perf_counter() - t0
        self.cpu += time.process_time() - c0
        return r

    def baseline(self, nbytes: float, sample: str, **extra):
        """The oracle's rate over its sample, as KV GB/s on the workload's own
        byte rule (the K/V rows the sampled sequences attend to)."""
        wall = max(self.wall, 1e-9)
        return {"value": nbytes / wall / 1e9, "unit": "GB/s",
                "cores": max(1, int(math.ceil(self.cpu / wall - 0.05))), "kind": "oracle",
                "sample": sample, "seconds": self.wall, **extra, **host_info()}


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
FLUSH_BYTES = 512 << 20   # twice the 256 MB memory-side cache of an MI355X
_flush_buf = None


def flush_caches(torch) -> None:
    """Reads FLUSH_BYTES of device memory, which evicts from the L2 caches and
    the memory-side cache whatever a previous kernel left there.  A read, not
    a write: a write would leave the caches full of dirty lines, and the next
    kernel's reads would pay for writing them back."""
    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    _flush_buf.amax()


def run_timed(torch, step, steps: int, warmup: int, nseg: int):
    """Warm up, then time `steps` calls of step(None) between two device
    synchronisations: the step's own launches only, nothing recorded between
    them.  A second pass of `steps` calls then has step record nseg + 1
    events on the launch stream around its kernels, with a 512 MB read
    before each call (outside the events) so that every call starts with
    cold caches; an event between two kernels adds a few microseconds of its
    own, so that pass gives the per-kernel durations but not the step time.
    Returns (ms per step of the first pass, [per-segment ms lists of the
    second])."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush_caches(torch)
        step(evs[i])
    torch.cuda.synchronize()
    segs = [[e[j].elapsed_time(e[j + 1]) for e in evs] for j in range(nseg)]
    return wall * 1e3 / steps, segs


def calibration_kernel(torch, mib: int) -> None:
    """An elementwise kernel that reads and writes exactly mib MiB."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()


def base_result(a, metric, value, unit, ms_per_step, dtype, config):
    return {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": config,
    }


def roofline(kernel, bound, achieved, peak, unit, traffic=None, traffic_source=None):
    r = {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
         "frac": achieved / peak, "traffic": traffic}
    if traffic_source is not None:
        r["traffic_source"] = traffic_source
    return r


def free_device(torch):
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# 7B-shape decode (the headline line)
# ---------------------------------------------------------------------------
class Workload:
    """7B-shape decode batch, built through the library's block manager."""

    def __init__(self, seed: int = 1, num_seqs: int = 64, heads: int = 32, head_dim: int = 128,
                 len_range=(128, 2048), block_size: int = BLOCK):
        import paged_kv_cache_366_amd as pkv
        from synth import workloads as W

        rng = np.random.default_rng(seed)
        self.S, self.H, self.D, self.bs = num_seqs, heads, head_dim, block_size
        bs = block_size
        lens = W.draw_lengths(rng, num_seqs, *len_range)
        nb = W.pool_size(lens, 1.25, bs)
        perm = W.draw_permutation(rng, nb)
        t0 = time.perf_counter()
        bm = pkv.pkv_bm_create(nb, bs, perm)
        seqs = [pkv.pkv_seq_create(bm, int(n) - 1) for n in lens]
        t1 = time.perf_counter()
        slots, cow = pkv.pkv_seq_append_batch(bm, seqs)
        self.max_blocks = int(max(W.blocks_for(n, bs) for n in lens))
        tables, lens_bm = pkv.pkv_seq_export(bm, seqs, self.max_blocks)
        t2 = time.perf_counter()
        assert len(cow) == 0 and np.array_equal(lens_bm, lens)
        self.host_bm = {"create_us": (t1 - t0) * 1e6, "append_export_us": (t2 - t1) * 1e6}
        self.bm, self.seqs, self.perm = bm, seqs, perm
        q = W.draw_normal(rng, (num_seqs, heads, head_dim), "bf16")
        kc, vc, _, _ = W.draw_paged_kv(rng, tables, lens, nb, heads, head_dim, "bf16", bs)
        self.lens, self.tables, self.slots, self.q = lens, tables, slots, q
        self.kc_full, self.vc_full = kc, vc          # with the current token (oracle side)
        blk, row = slots // bs, slots % bs
        self.new_k = kc[blk, :, row, :].copy()       # [S, H, D]
        self.new_v = vc[blk, :, row, :].copy()
        self.num_blocks = nb
        self.scale = np.float32(1.0 / math.sqrt(head_dim))

    # algorithmic bytes (bf16 everywhere, fp32 output)
    def kv_bytes(self) -> int:
        return int(self.lens.astype(np.int64).sum()) * self.H * self.D * 2 * 2

    def main_kernel_bytes(self) -> int:
        tbl = int(sum(W_blocks(n, self.bs) for n in self.lens)) * 4
        return self.kv_bytes() + self.S * self.H * self.D * 2 + tbl + self.S * 4

    def step_bytes(self) -> int:
        """The step's algorithmic bytes: every K/V row the sequences attend
        (the new token's read once, from its input rows), q, tables and
        lengths, the fp32 output, and the new rows written to their slots."""
        out = self.S * self.H * self.D * 4
        new_rows = self.S * self.H * self.D * 2 * 2
        return self.main_kernel_bytes() + out + new_rows


def cpu_baseline(wl: Workload, min_seconds: float = 10.0, max_reps: int = 40):
    """The oracle over the whole batch, repeated until at least min_seconds."""
    from oracle import attention as A

    clock = OracleClock()
    reps = 0
    out = None
    while reps < max_reps and (clock.wall < min_seconds or reps == 0):
        out = clock(A.decode, wl.q, wl.kc_full, wl.vc_full, wl.tables, wl.lens, wl.scale,
                    block_size=wl.bs)
        reps += 1
    per_call = clock.wall / reps
    res = clock.baseline(
        wl.kv_bytes() * reps,
        f"full batch ({wl.S} sequences, {int(wl.lens.sum())} context tokens) x {reps} passes of "
        f"the float64 oracle, {per_call:.2f} s per pass",
        tokens_per_s=wl.S / per_call)
    return res, out


def allocation_latency(pkv, wl: Workload, rounds: int = 40):
    """Page-allocation latency inside the library on the 7B-shape pool: each
    round creates the batch's 64 sequences at their cached lengths, appends
    their current token, and frees them; the library times every call that
    takes blocks (64 creates and one batch append per round)."""
    bm = pkv.pkv_bm_create(wl.num_blocks, wl.bs, wl.perm)
    try:
        for _ in range(rounds):
            seqs = [pkv.pkv_seq_create(bm, int(n) - 1) for n in wl.lens]
            pkv.pkv_seq_append_batch(bm, seqs)
            for s_ in seqs:
                pkv.pkv_seq_free(bm, s_)
        lat = pkv.pkv_bm_latency_get(bm)
    finally:
        pkv.pkv_bm_destroy(bm)
    lat["bar_p99_us"] = PAGE_ALLOC_P99_BAR_US
    lat["meets_bar"] = bool(lat["p99_us"] < PAGE_ALLOC_P99_BAR_US)
    lat["workload"] = (f"{rounds} rounds of: create the 64 sequences of the 7B-shape batch "
                       f"({wl.num_blocks}-block pool), append one token each, free them")
    return lat


def bench_decode7b(a, torch, pkv, algo):
    print("[bench] building the 7B-shape decode workload on the host", file=sys.stderr, flush=True)
    wl = Workload(seed=a.seed, block_size=a.block_size)
    dev = "cuda"
    kc = to_dev_bf16(wl.kc_full, torch)
    vc = to_dev_bf16(wl.vc_full, torch)
    blk = torch.from_numpy((wl.slots // wl.bs).astype(np.int64)).to(dev)
    row = torch.from_numpy((wl.slots % wl.bs).astype(np.int64)).to(dev)
    kc[blk, :, row, :] = float("nan")     # the step's cache write must fill these
    vc[blk, :, row, :] = float("nan")
    q = to_dev_bf16(wl.q, torch)
    new_k = to_dev_bf16(wl.new_k, torch)
    new_v = to_dev_bf16(wl.new_v, torch)
    slots = torch.from_numpy(wl.slots.astype(np.int32)).to(dev)
    tables = torch.from_numpy(wl.tables).to(dev)
    lens = torch.from_numpy(wl.lens).to(dev)
    max_ctx = int(wl.lens.max())
    part = a.partition if a.partition_set else 2048
    out = torch.empty((wl.S, wl.H, wl.D), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(pkv.pkv_decode_step_workspace_bytes(wl.S, wl.H, wl.D, max_ctx, part), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # One launch per step: the attention kernel appends each sequence's new
    # K/V rows at its last position and attends with them (2,048-token
    # partitions cover every context, so no split and no reduce).
    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        pkv.pkv_paged_attention_decode_step(out, q, new_k, new_v, kc, vc, tables, lens, max_ctx,
                                            float(wl.scale), part, algo, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    print(f"[bench] warmup {a.warmup}, timing {a.steps} steps", file=sys.stderr, flush=True)
    ms_per_step, (main_ms,) = run_timed(torch, step, a.steps, a.warmup, 1)
    if a.calib_copy_mib:
        calibration_kernel(torch, a.calib_copy_mib)
    got = out.cpu().numpy().astype(np.float64)

    # the same step as three launches (reshape_and_cache, split-K decode with
    # 1,536-token partitions, reduce), for comparison
    if a.no_compare:
        return finish_decode7b(a, torch, pkv, wl, kc, vc, ws, got, ms_per_step, main_ms, part,
                               None)
    sep_part = 1536
    ws3 = torch.empty(max(pkv.pkv_decode_workspace_bytes(wl.S, wl.H, wl.D, max_ctx, sep_part), 1),
                      dtype=torch.uint8, device=dev)
    out3 = torch.empty_like(out)

    def step3(ev):
        if ev is not None:
            ev[0].record(stream)
        pkv.pkv_reshape_and_cache(new_k, new_v, kc, vc, slots)
        if ev is not None:
            ev[1].record(stream)
        pkv.pkv_paged_attention_decode_partials(out3, q, kc, vc, tables, lens, max_ctx,
                                                float(wl.scale), sep_part, algo, workspace=ws3)
        if ev is not None:
            ev[2].record(stream)
        pkv.pkv_paged_attention_reduce(out3, lens, max_ctx, sep_part, ws3)
        if ev is not None:
            ev[3].record(stream)

    ms3, (rc_ms, main3_ms, red_ms) = run_timed(torch, step3, a.steps, a.warmup, 3)
    three = {
        "ms_per_step": ms3, "partition_tokens": sep_part,
        "kernel_ms": {"reshape_and_cache": stats_ms(rc_ms), "decode_main": stats_ms(main3_ms),
                      "reduce": stats_ms(red_ms)},
        "max_abs_diff_vs_one_launch": float((out3 - out).abs().max())}
    del ws3
    return finish_decode7b(a, torch, pkv, wl, kc, vc, ws, got, ms_per_step, main_ms, part, three)


def finish_decode7b(a, torch, pkv, wl, kc, vc, ws, got, ms_per_step, main_ms, part, three):
    main_avg = float(np.mean(main_ms))
    step_bytes = wl.step_bytes()
    achieved = step_bytes / (main_avg * 1e-3) / 1e9
    traffic, tsrc = traffic_of("decode7b", part) if wl.bs == BLOCK else (None, "not measured")
    result = base_result(a, METRIC, step_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s", ms_per_step,
                         "bf16", {
        "workload": "7B-shape paged decode, bf16 KV and q, fp32 accumulate: 64 sequences, "
                    f"32 heads MHA, head_dim 128, block_size {wl.bs}, contexts U[128, 2048], "
                    "pool 1.25x, random placement; step = append of each sequence's new K/V "
                    "rows + decode attention, one launch",
        "num_seqs": wl.S, "heads": wl.H, "head_dim": wl.D, "block_size": wl.bs,
        "context_tokens": int(wl.lens.sum()), "num_blocks": wl.num_blocks,
        "partition_tokens": part, "algo": a.algo, "seed": a.seed})
    result.update({
        "tokens_per_s": wl.S / (ms_per_step * 1e-3),
        "hbm_frac_step": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernel_ms": {"decode_step": stats_ms(main_ms)},
        "bytes": {"step": step_bytes, "kv": wl.kv_bytes(),
                  "new_rows_written": wl.S * wl.H * wl.D * 2 * 2},
        "roofline": roofline("decode_wave_kernel (append + attention, one launch per step)",
                             "hbm", achieved, HBM_PEAK_GBS, "GB/s", traffic, tsrc),
        "three_launch_step": three,
        "host_block_manager_us": wl.host_bm,
        "page_allocation_latency": allocation_latency(pkv, wl),
        "block_manager": {k: v for k, v in pkv.pkv_bm_stats_get(wl.bm).items()
                          if k in ("num_blocks", "used_blocks", "logical_blocks", "waste_slots")},
        "cpu_baseline": None,
    })
    del kc, vc, ws
    free_device(torch)
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on the same batch", file=sys.stderr, flush=True)
        cb, ref = cpu_baseline(wl, min_seconds=a.oracle_seconds)
        result["cpu_baseline"] = cb
        result["max_abs_err_vs_oracle"] = float(np.abs(got - ref).max())
    pkv.pkv_bm_destroy(wl.bm)
    return result


# ---------------------------------------------------------------------------
# long-context grouped-query decode
# ---------------------------------------------------------------------------
def owned_blocks(c, W):
    """(block, filled rows) of every block some sequence of case c owns."""
    return [(int(c.block_tables[s_, j]), int(min(BLOCK, n - BLOCK * j)))
            for s_, n in enumerate(c.context_lens) for j in range(W.blocks_for(n))]


def coded_rows(c, cache, s_, qmax):
    """Rows [0, n) of sequence s_ for every KV head as the oracle's block
    encoder codes them (codes x scale, float64), from the host pool."""
    from oracle import quantize as Q
    from synth import workloads as W
    n = int(c.context_lens[s_])
    out = np.empty((n, cache.shape[1], cache.shape[3]), np.float64)
    for j in range(W.blocks_for(n)):
        f = min(BLOCK, n - BLOCK * j)
        b = c.block_tables[s_, j]
        for g in range(cache.shape[1]):
            codes, sc = Q.quantize_tile(cache[b, g], f, qmax)
            out[BLOCK * j:BLOCK * j + f, g] = codes[:f].astype(np.float64) * np.float64(sc)
    return out


def gqa_case():
    from synth import workloads as W
    print("[bench] building the long-context GQA workload on the host", file=sys.stderr,
          flush=True)
    return W.gqa_long_decode(seed=4)


def bench_gqa(a, torch, pkv, algo, kv: str, c=None, sample_seqs: int = 6):
    from oracle import attention as A
    from oracle import quantize as Q
    from synth import workloads as W
    if c is None:
        c = gqa_case()
    int8, int4 = kv == "int8", kv == "int4"
    dev = "cuda"
    if int8 or int4:
        # the int8 / 4-bit pool is the library's block encoder output over
        # the bf16 pool (built before the timed region)
        sk, sv = to_dev_bf16(c.k_cache, torch), to_dev_bf16(c.v_cache, torch)
        nb_, hkv_, D_ = c.num_blocks, c.kv_heads, c.head_dim
        width = D_ if int8 else D_ // 2
        kc = torch.zeros((nb_, hkv_, BLOCK, width), dtype=torch.int8 if int8 else torch.uint8,
                         device=dev)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((nb_, hkv_), dtype=torch.float32, device=dev)
        vs = torch.zeros_like(ks)
        own = owned_blocks(c, W)
        encode = pkv.pkv_quantize_blocks if int8 else pkv.pkv_quantize_blocks_int4
        encode(sk, sv, kc, vc, ks, vs,
               torch.from_numpy(np.array([b for b, _ in own], np.int32)).to(dev),
               torch.from_numpy(np.array([f for _, f in own], np.int32)).to(dev))
        torch.cuda.synchronize()
        del sk, sv
    else:
        kc, vc = to_dev_bf16(c.k_cache, torch), to_dev_bf16(c.v_cache, torch)
        ks = vs = None
    q = to_dev_bf16(c.q, torch)
    tables = torch.from_numpy(c.block_tables).to(dev)
    lens = torch.from_numpy(c.context_lens).to(dev)
    S, hq, D = c.q.shape
    hkv = c.kv_heads
    max_ctx = int(c.context_lens.max())
    # the library's partition for these lengths and this kernel: the
    # shortest whose workgroups fit one round of the resident ones
    kv_code = pkv.PKV_I8 if int8 else pkv.PKV_I4 if int4 else pkv.PKV_BF16
    part = a.partition if a.partition_set else pkv.pkv_decode_partition_tokens(
        c.context_lens, pkv.PKV_BF16, kv_code, hq, hkv, D, BLOCK, c.num_blocks, algo)
    out = torch.empty((S, hq, D), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(pkv.pkv_decode_step_workspace_bytes(S, hq, D, max_ctx, part), 1),
                     dtype=torch.uint8, device=dev)
    scaled = int8 or int4
    # the step's cache write: each sequence's current token (the last
    # position) goes to its slot, into the int8 or 4-bit pool through
    # quantise-on-write (its block's scale already covers it, so the write is
    # the same every step) or into the bf16 pool
    last = c.context_lens - 1
    slot_h = np.array([c.block_tables[s_][p // BLOCK] * BLOCK + p % BLOCK
                       for s_, p in enumerate(last)], np.int32)
    new_k = to_dev_bf16(c.k_cache[slot_h // BLOCK, :, slot_h % BLOCK, :], torch)
    new_v = to_dev_bf16(c.v_cache[slot_h // BLOCK, :, slot_h % BLOCK, :], torch)
    slots_d = torch.from_numpy(slot_h).to(dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # bf16: the attention launch appends the current token's rows itself
    # (pkv_paged_attention_decode_step), then the reduce kernel merges the
    # partitions: two launches.  int8 / 4-bit: quantise-on-write of
    # the current token, the attention launch, the reduce: three.
    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        if int8:
            pkv.pkv_reshape_and_cache_int8(new_k, new_v, kc, vc, ks, vs, slots_d)
        elif int4:
            pkv.pkv_reshape_and_cache_int4(new_k, new_v, kc, vc, ks, vs, slots_d)
        if ev is not None:
            ev[1].record(stream)
        if scaled:
            pkv.pkv_paged_attention_decode(out, q, kc, vc, tables, lens, max_ctx, float(c.scale),
                                           part, algo, k_scale=ks, v_scale=vs, workspace=ws)
        else:
            pkv.pkv_paged_attention_decode_step(out, q, new_k, new_v, kc, vc, tables, lens,
                                                max_ctx, float(c.scale), part, algo,
                                                workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    print(f"[bench] GQA {kv}: warmup {a.warmup}, timing {a.steps} steps", file=sys.stderr,
          flush=True)
    ms_per_step, (wr_ms, main_ms) = run_timed(torch, step, a.steps, a.warmup, 2)
    tokens = int(c.context_lens.astype(np.int64).sum())
    bits = 8 if int8 else 4 if int4 else 16
    kvb = tokens * hkv * D * bits // 8 * 2
    nblk = sum(W.blocks_for(n) for n in c.context_lens)
    # attention: every K/V row attended (the current token's once), q, table
    # entries, lengths, scales, and the fp32 output
    main_bytes = (kvb + S * hq * D * 2 + nblk * 4 + S * 4 + (nblk * hkv * 8 if scaled else 0)
                  + S * hq * D * 4)
    # + the cache write: the current token's rows written in the pool's type
    # (and scales); quantise-on-write also reads its bf16 rows
    wr_bytes = (S * hkv * D * bits // 8 * 2 + (S * hkv * 8 if scaled else 0)
                + (S * hkv * D * 2 * 2 if scaled else 0))
    step_bytes = main_bytes + wr_bytes
    main_avg = float(np.mean(main_ms))
    # the attention launch(es): main kernel + reduce (the append included for bf16)
    achieved = (main_bytes + (0 if scaled else wr_bytes)) / (main_avg * 1e-3) / 1e9
    got = out.cpu().numpy()
    del kc, vc, ws, ks, vs
    free_device(torch)
    # sampled parity of this run's output against the oracle, whole sequences
    # (every query head), from the host pool; the oracle encodes int8 / 4-bit
    # tiles itself.  The same calls are the CPU baseline's sample.
    rng = np.random.default_rng(1)
    G = hq // hkv
    clock = OracleClock()
    err = 0.0
    pick = rng.choice(S, min(sample_seqs, S), replace=False)
    for s_ in pick:
        n = int(c.context_lens[s_])
        if scaled:
            qmax = Q.INT8_MAX if int8 else Q.INT4_MAX
            K = clock(coded_rows, c, c.k_cache, s_, qmax)
            V = clock(coded_rows, c, c.v_cache, s_, qmax)
        else:
            K = clock(A.gather, c.k_cache, c.block_tables[s_], n, BLOCK)
            V = clock(A.gather, c.v_cache, c.block_tables[s_], n, BLOCK)
        for h_ in range(hq):
            ref = clock(A.attend, c.q[s_, h_], K[:, h_ // G], V[:, h_ // G], c.scale)
            err = max(err, float(np.abs(got[s_, h_] - ref).max()))
    sample_tokens = int(sum(int(c.context_lens[s_]) for s_ in pick))
    kv_text = {"int8": "int8 KV (block encoder output) with per-block fp32 scales",
               "int4": "4-bit KV (block encoder output) with per-block fp32 scales",
               "bf16": "bf16 KV"}[kv]
    traffic, tsrc = traffic_of(f"gqa-{kv}", part)
    result = base_result(a, METRIC, step_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s", ms_per_step,
                         "bf16" if kv == "bf16" else f"{kv}-kv/bf16", {
        "workload": f"long-context GQA decode, {kv_text}: "
                    "16 sequences, 64 query heads over 8 KV heads, head_dim 128, "
                    "contexts U[8192, 32768]; step = cache write of each sequence's current "
                    "token (bf16: inside the attention launch; codes: quantise-on-write) + "
                    f"split-K decode with {part}-token partitions ("
                    + ("set by --partition" if a.partition_set else
                       "the library's choice for these lengths and this kernel")
                    + ") + reduce kernel",
        "context_tokens": tokens, "partition_tokens": part, "algo": a.algo})
    result.update({
        "tokens_per_s": S / (ms_per_step * 1e-3),
        "kernel_ms": ({"cache_write_" + kv: stats_ms(wr_ms), "decode_and_reduce": stats_ms(main_ms)}
                      if scaled else {"append_decode_and_reduce": stats_ms(main_ms)}),
        "bytes": {"step": step_bytes, "decode_main": main_bytes, "kv": kvb},
        "kv_gbs_step": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": roofline(("decode_mfma_kernel" if algo != pkv.PKV_ALGO_WAVE
                              else "decode_wave_kernel") + " + reduce_kernel"
                             + ("" if scaled else " (append in the main kernel)"), "hbm",
                             achieved, HBM_PEAK_GBS, "GB/s", traffic, tsrc),
        "max_abs_err_vs_oracle_sampled": err,
        "cpu_baseline": None if a.no_cpu_baseline else clock.baseline(
            sample_tokens * hkv * D * bits // 8 * 2,
            f"{len(pick)} whole sequences ({sample_tokens} tokens, all {hq} query heads) of the "
            "batch through the float64 oracle" + (" (with its own block encoder)" if scaled
                                                 else "")),
    })
    return result


# ---------------------------------------------------------------------------
# continuous-batching mixed step: decode sequences + prefill chunks
# ---------------------------------------------------------------------------
def bench_mixed(a, torch, pkv, algo):
    from oracle import attention as A
    from synth import workloads as W
    print("[bench] building the mixed-step workload on the host", file=sys.stderr, flush=True)
    ms = W.mixed_step(seed=2)
    dev = "cuda"
    nb, hkv, D, hq = ms.num_blocks, ms.kv_heads, ms.head_dim, ms.q_heads
    bm = pkv.pkv_bm_create(nb, BLOCK, ms.perm)
    kc = torch.full((nb, hkv, BLOCK, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = kc.clone()
    seqs = []
    for s_ in range(len(ms.prior)):
        sid = pkv.pkv_seq_create(bm, int(ms.prior[s_]))
        if ms.prior[s_]:
            sl = pkv.pkv_seq_slots(bm, sid, 0, int(ms.prior[s_]))
            pkv.pkv_reshape_and_cache(to_dev_bf16(ms.prior_k[s_], torch),
                                      to_dev_bf16(ms.prior_v[s_], torch), kc, vc,
                                      torch.from_numpy(sl).to(dev))
        seqs.append(sid)
    t0 = time.perf_counter()
    slots = np.concatenate([pkv.pkv_seq_append(bm, sid, int(ms.new[s_]))[0]
                            for s_, sid in enumerate(seqs)])
    lens_all = ms.prior + ms.new
    tables, lens = pkv.pkv_seq_export(bm, seqs, W.blocks_for(int(lens_all.max())))
    host_us = (time.perf_counter() - t0) * 1e6
    dec = np.flatnonzero(ms.new == 1)
    pre = np.flatnonzero(ms.new > 1)
    starts = np.concatenate([[0], np.cumsum(ms.new)])
    rows_p = np.concatenate([np.arange(starts[s_], starts[s_ + 1]) for s_ in pre])
    qdev = to_dev_bf16(ms.q, torch)
    q_d = qdev[torch.from_numpy(starts[dec]).to(dev)].contiguous()
    q_p = qdev[torch.from_numpy(rows_p).to(dev)].contiguous()
    new_k, new_v = to_dev_bf16(ms.new_k, torch), to_dev_bf16(ms.new_v, torch)
    slots_d = torch.from_numpy(slots.astype(np.int32)).to(dev)
    t_d = torch.from_numpy(np.ascontiguousarray(tables[dec])).to(dev)
    l_d = torch.from_numpy(np.ascontiguousarray(lens[dec])).to(dev)
    t_p = torch.from_numpy(np.ascontiguousarray(tables[pre])).to(dev)
    l_p = torch.from_numpy(np.ascontiguousarray(lens[pre])).to(dev)
    qsl = np.concatenate([[0], np.cumsum(ms.new[pre])]).astype(np.int32)
    qsl_d = torch.from_numpy(qsl).to(dev)
    mc_d, mc_p, mq = int(lens[dec].max()), int(lens[pre].max()), int(ms.new[pre].max())
    part = a.partition if a.partition_set else pkv.pkv_decode_partition_tokens(
        lens[dec], pkv.PKV_BF16, pkv.PKV_BF16, hq, hkv, D, BLOCK, nb, algo)
    out_d = torch.empty(q_d.shape, dtype=torch.float32, device=dev)
    out_p = torch.empty(q_p.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(max(pkv.pkv_decode_workspace_bytes(len(dec), hq, D, mc_d, part), 1),
                     dtype=torch.uint8, device=dev)
    ppart = (a.prefill_partition if a.prefill_partition is not None else
             pkv.pkv_prefill_partition_tokens(ms.new[pre], lens[pre], hq))
    ws_p = torch.empty(max(pkv.pkv_prefill_workspace_bytes(len(rows_p), hq, D, mc_p, ppart), 1),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        pkv.pkv_reshape_and_cache(new_k, new_v, kc, vc, slots_d)
        if ev is not None:
            ev[1].record(stream)
        pkv.pkv_paged_attention_decode_partials(out_d, q_d, kc, vc, t_d, l_d, mc_d,
                                                float(ms.scale), part, algo, workspace=ws)
        pkv.pkv_paged_attention_reduce(out_d, l_d, mc_d, part, ws)
        if ev is not None:
            ev[2].record(stream)
        pkv.pkv_paged_attention_prefill(out_p, q_p, kc, vc, t_p, qsl_d, l_p, mq, mc_p,
                                        float(ms.scale), partition_tokens=ppart, workspace=ws_p)
        if ev is not None:
            ev[3].record(stream)

    print(f"[bench] mixed step: warmup {a.warmup}, timing {a.steps} steps", file=sys.stderr,
          flush=True)
    ms_per_step, (rc_ms, dec_ms, pre_ms) = run_timed(torch, step, a.steps, a.warmup, 3)
    T = int(ms.new.sum())
    kv_dec = int(lens[dec].astype(np.int64).sum()) * hkv * D * 4
    kv_pre = int(lens[pre].astype(np.int64).sum()) * hkv * D * 4
    rc_bytes = T * hkv * D * 2 * 2 * 2
    dec_bytes = kv_dec + len(dec) * hq * D * (2 + 4)
    pre_bytes = kv_pre + len(rows_p) * hq * D * (2 + 4)
    step_bytes = rc_bytes + dec_bytes + pre_bytes
    flops = 0
    for s_ in pre:
        n, ql = int(lens[s_]), int(ms.new[s_])
        flops += sum(n - ql + i + 1 for i in range(ql)) * hq * D * 4
    pre_avg = float(np.mean(pre_ms))
    dec_avg = float(np.mean(dec_ms))
    got_p, got_d = out_p.cpu().numpy(), out_d.cpu().numpy()
    pkv.pkv_bm_destroy(bm)
    del kc, vc, ws, ws_p
    free_device(torch)

    # sampled parity against the oracle over each sequence's logical rows
    # (the cached prior rows, then the step's new rows), from the host draws.
    # The same calls are the CPU baseline's sample.
    def logical(s_):
        K = np.concatenate([ms.prior_k[s_], ms.new_k[starts[s_]:starts[s_ + 1]]])
        V = np.concatenate([ms.prior_v[s_], ms.new_v[starts[s_]:starts[s_ + 1]]])
        return K.astype(np.float64), V.astype(np.float64)

    rng = np.random.default_rng(0)
    G = hq // hkv
    clock, clock_p = OracleClock(), OracleClock()
    err_d = err_p = 0.0
    dec_pick = rng.choice(len(dec), 24, replace=False)
    for j in dec_pick:
        s_ = dec[j]
        K, V = clock(logical, s_)
        for h_ in range(hq):
            ref = clock(A.attend, ms.q[starts[s_], h_], K[:, h_ // G], V[:, h_ // G], ms.scale)
            err_d = max(err_d, float(np.abs(got_d[j, h_] - ref).max()))
    dec_tokens = int(sum(int(lens[dec[j]]) for j in dec_pick))
    pre_flops = 0
    for j, s_ in enumerate(pre):
        n, ql = int(lens[s_]), int(ms.new[s_])
        K, V = clock_p(logical, s_)
        for i in (0, ql // 2, ql - 1):
            P = n - ql + i
            for h_ in range(hq):
                ref = clock_p(A.attend, ms.q[rows_p[qsl[j] + i], h_], K[:P + 1, h_ // G],
                              V[:P + 1, h_ // G], ms.scale)
                err_p = max(err_p, float(np.abs(got_p[qsl[j] + i, h_] - ref).max()))
                pre_flops += 4 * D * (P + 1)
    traffic, tsrc = traffic_of("mixed-decode", part)
    result = base_result(a, METRIC, step_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s", ms_per_step,
                         "bf16", {
        "workload": "continuous-batching mixed step, bf16: 48 decode sequences (contexts "
                    "U[64, 4096]) + 4 prefill chunks of 512 causal rows over 0/512/1024/1536 "
                    "cached tokens; 32 heads x 128; step = reshape_and_cache of 2096 rows + "
                    "decode + reduce + chunked prefill",
        "partition_tokens": part, "prefill_partition_tokens": ppart,
        "algo": a.algo})
    result.update({
        "tokens_per_s": (len(dec) + len(rows_p)) / (ms_per_step * 1e-3),
        "kernel_ms": {"reshape_and_cache": stats_ms(rc_ms), "decode_and_reduce": stats_ms(dec_ms),
                      "prefill": stats_ms(pre_ms)},
        "bytes": {"step": step_bytes, "decode": dec_bytes, "prefill_unique": pre_bytes,
                  "reshape_and_cache": rc_bytes},
        "kv_gbs_decode": dec_bytes / (dec_avg * 1e-3) / 1e9,
        "prefill_gflop": flops / 1e9,
        "prefill_tflops": flops / (pre_avg * 1e-3) / 1e12,
        "roofline": roofline("decode_wave_kernel + reduce (decode part)", "hbm",
                             dec_bytes / (dec_avg * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", traffic,
                             tsrc),
        "roofline_prefill": roofline("prefill_mfma_kernel", "mfma",
                                     flops / (pre_avg * 1e-3) / 1e12, BF16_MFMA_PEAK_TFLOPS,
                                     "TFLOP/s"),
        "host_block_manager_us": {"append_export_us": host_us},
        "max_abs_err_vs_oracle_sampled": max(err_d, err_p),
        "max_abs_err_vs_oracle_sampled_parts": {"decode": err_d, "prefill": err_p},
        "cpu_baseline": None if a.no_cpu_baseline else clock.baseline(
            dec_tokens * hkv * D * 4,
            f"24 decode sequences ({dec_tokens} tokens, all {hq} heads) through the float64 "
            f"oracle (value); 3 rows of each prefill chunk, all heads (prefill_tflops)",
            prefill_seconds=clock_p.wall,
            prefill_tflops=pre_flops / max(clock_p.wall, 1e-9) / 1e12),
    })
    return result


# ---------------------------------------------------------------------------
# shared prefix + beam search with copy-on-write
# ---------------------------------------------------------------------------
def bench_beam(a, torch, pkv, algo):
    from oracle import attention as A
    from synth import workloads as W
    print("[bench] building the shared-prefix beam workload on the host", file=sys.stderr,
          flush=True)
    bc = W.beam_cow(seed=3)
    dev = "cuda"
    nb, hkv, D, hq = bc.num_blocks, bc.kv_heads, bc.head_dim, bc.q_heads
    bm = pkv.pkv_bm_create(nb, BLOCK, bc.perm)
    kc = torch.full((nb, hkv, BLOCK, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = kc.clone()

    def write(sl, k, v):
        pkv.pkv_reshape_and_cache(to_dev_bf16(k, torch), to_dev_bf16(v, torch), kc, vc,
                                  torch.from_numpy(np.asarray(sl, np.int32)).to(dev))

    root = pkv.pkv_seq_create(bm, bc.prefix_len)
    write(pkv.pkv_seq_slots(bm, root, 0, bc.prefix_len), bc.prefix_k, bc.prefix_v)
    reqs = []
    for r, n in enumerate(bc.request_lens):
        s_ = pkv.pkv_seq_fork(bm, root)
        write(pkv.pkv_seq_append(bm, s_, int(n))[0], bc.req_k[r], bc.req_v[r])
        reqs.append(s_)
    pkv.pkv_seq_free(bm, root)
    beams = []
    for s_ in reqs:
        beams += [pkv.pkv_seq_fork(bm, s_) for _ in range(bc.beam_width - 1)] + [s_]
    t0 = time.perf_counter()
    slots, pairs = pkv.pkv_seq_append_batch(bm, beams)
    mb = W.blocks_for(bc.prefix_len + int(bc.request_lens.max()) + 1)
    tables, lens = pkv.pkv_seq_export(bm, beams, mb)
    host_us = (time.perf_counter() - t0) * 1e6
    stats = pkv.pkv_bm_stats_get(bm)
    # beams share the prompt's blocks (the block manager counts them): K/V
    # loads stay cached, so a block read by one beam serves the others
    load_policy = pkv.PKV_KV_CACHED if stats["shared_blocks"] > 0 else 0
    pairs_d = torch.from_numpy(np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)).to(dev)
    slots_d = torch.from_numpy(slots.astype(np.int32)).to(dev)
    bk, bv = to_dev_bf16(bc.beam_k, torch), to_dev_bf16(bc.beam_v, torch)
    q = to_dev_bf16(bc.q, torch)
    t_d, l_d = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    S = len(beams)
    mc = int(lens.max())
    # the 64 beams' contexts are nearly equal (1,025-1,225 tokens) and fill
    # the GPU unsplit, so one partition per context is the default here
    part = a.partition if a.partition_set else 0
    out = torch.empty((S, hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(pkv.pkv_decode_workspace_bytes(S, hq, D, mc, part), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        pkv.pkv_copy_blocks(kc, vc, pairs_d)
        pkv.pkv_reshape_and_cache(bk, bv, kc, vc, slots_d)
        if ev is not None:
            ev[1].record(stream)
        pkv.pkv_paged_attention_decode_partials(out, q, kc, vc, t_d, l_d, mc, float(bc.scale),
                                                part, algo | load_policy, workspace=ws)
        pkv.pkv_paged_attention_reduce(out, l_d, mc, part, ws)
        if ev is not None:
            ev[2].record(stream)

    print(f"[bench] beams: warmup {a.warmup}, timing {a.steps} steps", file=sys.stderr,
          flush=True)
    ms_per_step, (cow_ms, dec_ms) = run_timed(torch, step, a.steps, a.warmup, 2)
    logical = int(lens.astype(np.int64).sum()) * hkv * D * 4
    unique_blocks = len(set(int(b) for s_ in range(S) for b in tables[s_, :W.blocks_for(lens[s_])]))
    unique = unique_blocks * hkv * BLOCK * D * 4
    dec_avg = float(np.mean(dec_ms))
    got = out.cpu().numpy()
    pkv.pkv_bm_destroy(bm)
    del kc, vc, ws
    free_device(torch)
    # sampled parity over each beam's logical rows (prefix, the request's own
    # tokens, the beam's token) from the host draws; the CPU baseline's sample
    rng = np.random.default_rng(0)
    clock = OracleClock()
    err = 0.0
    pick = rng.choice(S, 32, replace=False)

    def logical_rows(b):
        r = b // bc.beam_width
        K = np.concatenate([bc.prefix_k, bc.req_k[r], bc.beam_k[b:b + 1]]).astype(np.float64)
        V = np.concatenate([bc.prefix_v, bc.req_v[r], bc.beam_v[b:b + 1]]).astype(np.float64)
        return K, V

    for b in pick:
        K, V = clock(logical_rows, int(b))
        assert K.shape[0] == lens[b]
        for h_ in range(hq):
            ref = clock(A.attend, bc.q[b, h_], K[:, h_], V[:, h_], bc.scale)
            err = max(err, float(np.abs(got[b, h_] - ref).max()))
    sample_tokens = int(sum(int(lens[b]) for b in pick))
    result = base_result(a, METRIC, unique / (dec_avg * 1e-3) / 1e9, "GB/s (unique K/V)",
                         ms_per_step, "bf16", {
        "workload": "shared-prefix beam search with copy-on-write, bf16: 16 requests sharing a "
                    "1024-token prefix, 1-200 own tokens, beam width 4; step = copy_blocks of the "
                    "shared partial tails + reshape_and_cache of 64 tokens + decode + reduce",
        "partition_tokens": part, "algo": a.algo, "cow_pairs": int(len(pairs)),
        "kv_loads": "cached" if load_policy else "pool-size rule"})
    result.update({
        "tokens_per_s": S / (ms_per_step * 1e-3),
        "kernel_ms": {"copy_blocks_and_reshape": stats_ms(cow_ms),
                      "decode_and_reduce": stats_ms(dec_ms)},
        "bytes": {"logical_kv": logical, "unique_kv": unique},
        "note": "the unique K/V working set (each shared block once) fits the 256 MB "
                "memory-side cache; roofline is unique bytes against HBM, logical bytes (shared "
                "blocks once per beam) are the cache-served rate",
        "roofline": roofline("decode_wave_kernel + reduce (unique K/V bytes)", "hbm",
                             unique / (dec_avg * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
        "logical_kv_gbs": {"bound": "cache", "achieved": logical / (dec_avg * 1e-3) / 1e9,
                           "unit": "GB/s"},
        "block_manager": {"append_export_us": host_us, **stats},
        "max_abs_err_vs_oracle_sampled": err,
        "cpu_baseline": None if a.no_cpu_baseline else clock.baseline(
            sample_tokens * hkv * D * 4,
            f"32 beams ({sample_tokens} logical tokens, all {hq} heads) through the float64 "
            "oracle; value in logical K/V bytes"),
    })
    return result


# ---------------------------------------------------------------------------
# int8 storage of a long-context pool (whole blocks)
# ---------------------------------------------------------------------------
def bench_quantize(a, torch, pkv, bits: int = 8):
    from synth import workloads as W
    print("[bench] building the long-context pool on the host", file=sys.stderr, flush=True)
    c = W.gqa_long_decode(seed=4)
    dev = "cuda"
    nb, hkv, D = c.num_blocks, c.kv_heads, c.head_dim
    owned = owned_blocks(c, W)
    blocks = torch.from_numpy(np.array([b for b, _ in owned], np.int32)).to(dev)
    filled_h = np.array([f for _, f in owned], np.int32)
    filled = torch.from_numpy(filled_h).to(dev)
    sk, sv = to_dev_bf16(c.k_cache, torch), to_dev_bf16(c.v_cache, torch)
    if bits == 8:
        dk = torch.zeros((nb, hkv, BLOCK, D), dtype=torch.int8, device=dev)
        encode = pkv.pkv_quantize_blocks
    else:
        dk = torch.zeros((nb, hkv, BLOCK, D // 2), dtype=torch.uint8, device=dev)
        encode = pkv.pkv_quantize_blocks_int4
    dv = torch.zeros_like(dk)
    ks = torch.zeros((nb, hkv), dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        encode(sk, sv, dk, dv, ks, vs, blocks, filled)
        if ev is not None:
            ev[1].record(stream)

    ms_per_step, (q_ms,) = run_timed(torch, step, a.steps, a.warmup, 1)
    rows = int(filled_h.sum())
    nlisted = len(owned)
    # read the filled rows of K and V once (bf16), write every row's codes
    # and one fp32 scale per (block, head), K and V
    nbytes = (rows * hkv * D * 2 * 2 + nlisted * hkv * BLOCK * D * bits // 8 * 2
              + nlisted * hkv * 4 * 2)
    avg = float(np.mean(q_ms))
    name = "int8" if bits == 8 else "4-bit"
    result = base_result(a, METRIC, nbytes / (ms_per_step * 1e-3) / 1e9, "GB/s", ms_per_step,
                         "bf16->int8" if bits == 8 else "bf16->int4", {
        "workload": f"{name} storage of a long-context pool: every owned block of 16 sequences x "
                    f"8 KV heads x 128, contexts U[8192, 32768], bf16 -> {name} codes + "
                    "per-(block, head) fp32 scales",
        "blocks": nlisted})
    result.update({
        "kernel_ms": {"quantize_blocks" + ("" if bits == 8 else "_int4"): avg},
        "bytes": {"per_call": nbytes},
        "roofline": roofline("quantize_blocks_kernel", "hbm", nbytes / (avg * 1e-3) / 1e9,
                             HBM_PEAK_GBS, "GB/s"),
        "cpu_baseline": None,
    })
    return result


# ---------------------------------------------------------------------------
# preemption by swapping: blocks device -> pinned host -> device
# ---------------------------------------------------------------------------
def bench_swap(a, torch, pkv):
    from synth import workloads as W
    print("[bench] building the 7B-shape pool on the host", file=sys.stderr, flush=True)
    wl = Workload(seed=a.seed)
    dev = "cuda"
    kc, vc = to_dev_bf16(wl.kc_full, torch), to_dev_bf16(wl.vc_full, torch)
    # the 16 longest sequences are preempted: all their blocks go to host memory
    order = np.argsort(-wl.lens)[:16]
    own = np.concatenate([wl.tables[s_, :W.blocks_for(wl.lens[s_])] for s_ in order]).astype(np.int32)
    n = len(own)
    shape = (n,) + tuple(kc.shape[1:])
    hk = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    out_pairs = np.stack([own, np.arange(n, dtype=np.int32)], 1)
    in_pairs = np.stack([np.arange(n, dtype=np.int32), own], 1)
    # staging for 256 blocks per round (64 MiB): gather/scatter on the
    # device, long runs over PCIe
    ws = torch.empty(pkv.pkv_swap_workspace_bytes(256, kc.shape[1], kc.shape[3], BLOCK,
                                                  pkv.PKV_BF16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        pkv.pkv_swap_blocks(hk, hv, kc, vc, out_pairs, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        pkv.pkv_swap_blocks(kc, vc, hk, hv, in_pairs, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    pkv.pkv_swap_stats_get(reset=True)
    ms_per_step, (out_ms, in_ms) = run_timed(torch, step, a.steps, a.warmup, 2)
    swap_stats = pkv.pkv_swap_stats_get(reset=True)   # warm-up and timed steps
    nbytes = n * int(np.prod(kc.shape[1:])) * 2 * 2          # K and V, one direction
    o, i_ = float(np.mean(out_ms)), float(np.mean(in_ms))
    result = base_result(a, METRIC, 2 * nbytes / (ms_per_step * 1e-3) / 1e9, "GB/s", ms_per_step,
                         "bf16", {
        "workload": "preemption by swapping at the 7B shape: every block of the 16 longest "
                    "sequences (32 heads x 128, bf16) to pinned host memory and back",
        "blocks": n})
    result.update({
        "kernel_ms": {"swap_out": o, "swap_in": i_},
        "bytes": {"per_direction": nbytes},
        "gbs": {"device_to_host": nbytes / (o * 1e-3) / 1e9, "host_to_device": nbytes / (i_ * 1e-3) / 1e9},
        "roofline": None,
        "note": "DMA over PCIe; the pages quote 32-64 GB/s for PCIe (kongchang.com, section "
                "on preemption)",
        "swap_stats": swap_stats,
        "swapped_blocks_per_s": (swap_stats["blocks_to_host"] + swap_stats["blocks_to_device"])
        / ((a.steps + a.warmup) * ms_per_step * 1e-3),
        "cpu_baseline": None,
    })
    return result


# ---------------------------------------------------------------------------
# prefix caching: admission of requests that share a system prompt
# ---------------------------------------------------------------------------
def bench_prefix(a, torch, pkv, algo):
    from synth import workloads as W
    print("[bench] building the shared-system-prompt workload on the host", file=sys.stderr,
          flush=True)
    c = W.prefix_sharing(seed=6, draw_q=False, pool_factor=2.2)
    dev = "cuda"
    R, nb, hkv, D, hq = len(c.prompts), c.num_blocks, c.kv_heads, c.head_dim, c.q_heads
    lens = np.array([len(p) for p in c.prompts], np.int32)
    bm = pkv.pkv_bm_create(nb, BLOCK, c.perm)
    kc = torch.full((nb, hkv, BLOCK, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = kc.clone()
    kd = [to_dev_bf16(k, torch) for k in c.k]
    vd = [to_dev_bf16(v, torch) for v in c.v]
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    qd = [torch.randn((int(n), hq, D), generator=g, device=dev).to(torch.bfloat16) for n in lens]

    def i32d(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)

    # request 0 computes the system prompt and publishes it
    sid0, _ = pkv.pkv_seq_create_cached(bm, c.prompts[0])
    pkv.pkv_reshape_and_cache(kd[0], vd[0], kc, vc, i32d(pkv.pkv_seq_slots(bm, sid0, 0, int(lens[0]))))
    pkv.pkv_seq_publish(bm, sid0, c.prompts[0])
    rest = list(range(1, R))
    # host cost of admission: create from tokens + slot lookup, then free
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        ids = []
        for r in rest:
            sid, cached = pkv.pkv_seq_create_cached(bm, c.prompts[r])
            pkv.pkv_seq_slots(bm, sid, cached, int(lens[r]) - cached)
            ids.append(sid)
        for sid in ids:
            pkv.pkv_seq_free(bm, sid)
    admit_us = (time.perf_counter() - t0) * 1e6 / (reps * len(rest))
    # the admitted batch, with the cache and (same requests, same pool) without
    sids, cached = zip(*[pkv.pkv_seq_create_cached(bm, c.prompts[r]) for r in rest])
    plain = [pkv.pkv_seq_create(bm, int(lens[r])) for r in rest]
    stats = pkv.pkv_bm_prefix_stats(bm)
    mb = W.blocks_for(int(lens.max()))

    def batch(seq_ids, starts):
        rows = [int(lens[r]) - st for r, st in zip(rest, starts)]
        slots = np.concatenate([pkv.pkv_seq_slots(bm, sid, st, n)
                                for sid, st, n in zip(seq_ids, starts, rows)])
        tables, _ = pkv.pkv_seq_export(bm, list(seq_ids), mb)
        qsl = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        return {
            "k": torch.cat([kd[r][st:] for r, st in zip(rest, starts)]),
            "v": torch.cat([vd[r][st:] for r, st in zip(rest, starts)]),
            "q": torch.cat([qd[r][st:] for r, st in zip(rest, starts)]),
            "slots": i32d(slots), "tables": i32d(tables), "qsl": i32d(qsl),
            "lens": i32d(lens[rest]), "rows": rows, "max_q": max(rows),
            "tables_h": tables, "qsl_h": qsl,
        }

    hit = batch(sids, cached)
    full = batch(plain, [0] * len(rest))
    for b in (hit, full):
        b["out"] = torch.empty(b["q"].shape, dtype=torch.float32, device=dev)
        b["ws"] = torch.empty(max(pkv.pkv_prefill_workspace_bytes(
            b["q"].shape[0], hq, D, int(lens.max()), a.prefill_partition or 0), 1),
            dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    mc = int(lens.max())
    torch.cuda.synchronize()

    def run(b):
        pkv.pkv_reshape_and_cache(b["k"], b["v"], kc, vc, b["slots"])
        pkv.pkv_paged_attention_prefill(b["out"], b["q"], kc, vc, b["tables"], b["qsl"], b["lens"],
                                        b["max_q"], mc, float(c.scale),
                                        partition_tokens=a.prefill_partition or 0, workspace=b["ws"])

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        run(hit)
        if ev is not None:
            ev[1].record(stream)
        run(full)
        if ev is not None:
            ev[2].record(stream)

    ms_per_step, (hit_ms, full_ms) = run_timed(torch, step, a.steps, a.warmup, 2)
    h_avg, f_avg = float(np.mean(hit_ms)), float(np.mean(full_ms))
    prompt_tokens = int(lens[rest].sum())
    # the cached rows give the same result as computing them
    diff = 0.0
    got_h, got_f = hit["out"].cpu().numpy(), full["out"].cpu().numpy()
    for j, r in enumerate(rest):
        a_, n_ = int(hit["qsl_h"][j]), hit["rows"][j]
        b_ = int(full["qsl_h"][j]) + cached[j]
        diff = max(diff, float(np.abs(got_h[a_:a_ + n_] - got_f[b_:b_ + n_]).max()))
    from oracle import attention as A
    rng = np.random.default_rng(0)
    err = 0.0
    for j in rng.choice(len(rest), 4, replace=False):
        r, n = rest[j], int(lens[rest[j]])
        K = c.k[r].astype(np.float64)     # the request's rows, as written
        V = c.v[r].astype(np.float64)
        for i in (0, hit["rows"][j] - 1):
            P = cached[j] + i
            h_ = int(rng.integers(0, hq))
            qrow = qd[r][P, h_].float().cpu().numpy()
            ref = A.attend(qrow, K[:P + 1, h_ // (hq // hkv)], V[:P + 1, h_ // (hq // hkv)],
                           c.scale)
            err = max(err, float(np.abs(got_h[int(hit["qsl_h"][j]) + i, h_] - ref).max()))
    flops = sum(sum(range(int(n) - rows + 1, int(n) + 1)) * hq * D * 4
                for n, rows in zip(lens[rest], hit["rows"]))
    saved = sum(cached) * hkv * D * 2 * 2
    pkv.pkv_bm_destroy(bm)
    result = base_result(a, METRIC, prompt_tokens / (h_avg * 1e-3), "prompt tokens/s (effective)",
                         ms_per_step, "bf16", {
        "workload": "prefix caching at the 7B shape (32 heads x 128, bf16): 31 requests sharing "
                    "a 1024-token system prompt already in the cache, 64-256 own tokens each; "
                    "admission = reshape_and_cache + prefill of the uncached rows, against the "
                    "same requests computed in full",
        "requests": len(rest), "prefill_partition_tokens": a.prefill_partition or 0})
    result.update({
        "kernel_ms": {"with_prefix_cache": h_avg, "without": f_avg},
        "speedup": f_avg / h_avg,
        "rows": {"computed": int(sum(hit["rows"])), "without_cache": int(sum(full["rows"]))},
        "prefix_cache": {**stats, "cached_tokens": int(sum(cached)),
                         "kv_bytes_not_stored": saved, "admit_us_per_request": admit_us},
        "roofline": roofline("prefill_mfma_kernel + reshape_and_cache (cached step)", "mfma",
                             flops / (h_avg * 1e-3) / 1e12, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"),
        "max_abs_diff_cached_vs_full": diff,
        "max_abs_err_vs_oracle_sampled": err,
        "cpu_baseline": None,
    })
    return result


# ---------------------------------------------------------------------------
# chunked prefill of a long document: short chunks over long cached contexts
# ---------------------------------------------------------------------------
def bench_prefill_long(a, torch, pkv, algo):
    from synth import workloads as W
    print("[bench] building the long-context prefill workload on the host", file=sys.stderr,
          flush=True)
    # 4 documents of 16,384 tokens whose last 64 tokens form this step's chunk
    c = W.prefill_case(7, 32, 32, 128, [(16384 - 64, 64)] * 4, dtype="bf16")
    dev = "cuda"
    D, hq = 128, 32
    kc, vc = to_dev_bf16(c.k_cache, torch), to_dev_bf16(c.v_cache, torch)
    q = to_dev_bf16(c.q, torch)
    t = torch.from_numpy(c.block_tables).to(dev)
    l = torch.from_numpy(c.context_lens).to(dev)
    qsl = torch.from_numpy(c.query_start_loc).to(dev)
    mc, mq = int(c.context_lens.max()), 64
    # the library's key partition for these chunks (split so that two
    # workgroups per compute unit are busy), unless --prefill-partition
    part = (a.prefill_partition if a.prefill_partition is not None else
            pkv.pkv_prefill_partition_tokens(np.diff(c.query_start_loc), c.context_lens, hq))
    out_s = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out_n = torch.empty_like(out_s)
    ws = torch.empty(max(pkv.pkv_prefill_workspace_bytes(q.shape[0], hq, D, mc, part), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        pkv.pkv_paged_attention_prefill(out_s, q, kc, vc, t, qsl, l, mq, mc, float(c.scale),
                                        partition_tokens=part, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        pkv.pkv_paged_attention_prefill(out_n, q, kc, vc, t, qsl, l, mq, mc, float(c.scale))
        if ev is not None:
            ev[2].record(stream)

    ms_per_step, (split_ms, plain_ms) = run_timed(torch, step, a.steps, a.warmup, 2)
    s_avg, n_avg = float(np.mean(split_ms)), float(np.mean(plain_ms))
    flops = sum(sum(range(16384 - 64 + 1, 16384 + 1)) for _ in range(4)) * hq * D * 4
    kv_bytes = 4 * 16384 * hq * D * 2 * 2
    from oracle import attention as A
    got = out_s.cpu().numpy()
    rng = np.random.default_rng(0)
    err = 0.0
    for s_ in range(4):
        K = A.gather(c.k_cache, c.block_tables[s_], 16384, BLOCK)
        V = A.gather(c.v_cache, c.block_tables[s_], 16384, BLOCK)
        for i in (0, 63):
            h_ = int(rng.integers(0, hq))
            P = 16384 - 64 + i
            ref = A.attend(c.q[64 * s_ + i, h_], K[:P + 1, h_], V[:P + 1, h_], c.scale)
            err = max(err, float(np.abs(got[64 * s_ + i, h_] - ref).max()))
    result = base_result(a, METRIC, kv_bytes / (s_avg * 1e-3) / 1e9, "GB/s (K/V read)", ms_per_step,
                         "bf16", {
        "workload": "chunked prefill of long documents, bf16: 4 sequences of 16,384 tokens whose "
                    "last 64 form the chunk, 32 heads x 128; split-K prefill (key partitions + "
                    "reduce) against the same call without partitions",
        "prefill_partition_tokens": part})
    result.update({
        "kernel_ms": {"split": s_avg, "no_split": n_avg},
        "speedup": n_avg / s_avg,
        "roofline": roofline("prefill_mfma_kernel + reduce (split-K)", "hbm",
                             kv_bytes / (s_avg * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
        "mfma_tflops": flops / (s_avg * 1e-3) / 1e12,
        "max_abs_diff_split_vs_not": float((out_s - out_n).abs().max()),
        "max_abs_err_vs_oracle_sampled": err,
        "cpu_baseline": None,
    })
    return result


WORKLOADS = ("all", "decode7b", "mixed", "beam", "gqa", "gqa-int8", "gqa-int4", "quantize",
             "quantize-int4", "swap", "prefix", "prefill-long")

# keys of a workload line kept when it is nested in the default line
SUB_KEYS = ("value", "unit", "ms_per_step", "dtype", "config", "tokens_per_s", "kernel_ms",
            "bytes", "kv_gbs_step", "kv_gbs_decode", "prefill_gflop", "prefill_tflops",
            "roofline", "roofline_prefill", "logical_kv_gbs", "note", "block_manager",
            "max_abs_err_vs_oracle_sampled", "max_abs_err_vs_oracle_sampled_parts",
            "cpu_baseline")


def nested(line: dict) -> dict:
    return {k: line[k] for k in SUB_KEYS if k in line}


def bench_all(a, torch, pkv, algo):
    """The headline line with the other four workloads nested in it."""
    t0 = time.perf_counter()
    result = bench_decode7b(a, torch, pkv, algo)
    free_device(torch)
    result["c3_mixed"] = nested(bench_mixed(a, torch, pkv, algo))
    free_device(torch)
    result["c4_beam"] = nested(bench_beam(a, torch, pkv, algo))
    free_device(torch)
    c = gqa_case()
    result["c5_gqa_bf16"] = nested(bench_gqa(a, torch, pkv, algo, "bf16", c))
    free_device(torch)
    result["c5_gqa_int8"] = nested(bench_gqa(a, torch, pkv, algo, "int8", c))
    free_device(torch)
    result["bench_wall_s"] = time.perf_counter() - t0
    return result


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=WORKLOADS, default="all",
                    help="all: the headline 7B decode line with the mixed-step, beam and "
                         "long-context GQA (bf16, int8) workloads nested in it; the others "
                         "print one workload's line")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-K partition size in tokens (0 = no split) for every workload "
                         "run; default 2048 for the 7B step (no split), 0 for the beam "
                         "workload, the library's choice (pkv_decode_partition_tokens) for the "
                         "mixed step and the long-context GQA workloads")
    ap.add_argument("--algo", choices=("auto", "wave", "mfma"), default="auto")
    ap.add_argument("--prefill-partition", type=int, default=None,
                    help="key partition size of chunked prefill in tokens (0 = no split); "
                         "default: the library's choice (pkv_prefill_partition_tokens) for the "
                         "mixed step and long documents, no split for prefix admission")
    ap.add_argument("--block-size", type=int, default=BLOCK, choices=(16, 32, 64, 128),
                    help="KV block size of the decode7b workload (16 is the headline line)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="7B step: skip the three-launch comparison (for profiling one kernel)")
    ap.add_argument("--oracle-seconds", type=float, default=8.0,
                    help="least CPU time of the headline's oracle baseline (whole-batch passes)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one elementwise kernel that reads and writes this many MiB "
                         "(a known-size kernel for scaling rocprofv3 byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the library has no "
              "multi-GPU mode", file=sys.stderr)
        return 2
    a.partition_set = a.partition is not None
    if a.partition is None:
        # each workload chooses its own split-K partition unless --partition
        # is given: 2,048 tokens (no split) for the 7B step, none for beams,
        # the library's choice for the mixed step's decode part and for
        # long-context GQA
        a.partition = 0

    import torch
    import paged_kv_cache_366_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    pkv.load()
    algo = {"auto": pkv.PKV_ALGO_AUTO, "wave": pkv.PKV_ALGO_WAVE, "mfma": pkv.PKV_ALGO_MFMA}[a.algo]
    if a.workload == "all":
        result = bench_all(a, torch, pkv, algo)
    elif a.workload == "decode7b":
        result = bench_decode7b(a, torch, pkv, algo)
    elif a.workload == "mixed":
        result = bench_mixed(a, torch, pkv, algo)
    elif a.workload == "beam":
        result = bench_beam(a, torch, pkv, algo)
    elif a.workload in ("quantize", "quantize-int4"):
        result = bench_quantize(a, torch, pkv, 8 if a.workload == "quantize" else 4)
    elif a.workload == "swap":
        result = bench_swap(a, torch, pkv)
    elif a.workload == "prefix":
        result = bench_prefix(a, torch, pkv, algo)
    elif a.workload == "prefill-long":
        result = bench_prefill_long(a, torch, pkv, algo)
    else:
        result = bench_gqa(a, torch, pkv, algo, {"gqa": "bf16", "gqa-int8": "int8",
                                                 "gqa-int4": "int4"}[a.workload])
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
