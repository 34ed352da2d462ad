"""Benchmark of the paged KV write + paged attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

One step = the whole hot path over one batch of the decode workload
(64 sequences, Hq 32, Hkv 8, head_dim 128, page_size 16, bf16 KV, context
lengths U{512..4096}, 65536-page pools): the slot-mapping write of the 64 new
tokens, then paged decode attention (split-K partitions + log-sum-exp merge)
over every sequence's pages.  Inputs are resident in HBM before timing starts.
Each timed step is preceded, outside its timed region, by a 1 GiB device fill
that evicts L2 and the 256 MB Infinity Cache, so KV reads come from HBM.  Every
step is timed with a pair of HIP events on the stream the kernels run on.

The printed JSON line carries:
  value        decode KV-read GB/s of the step: algorithmic bytes / step time,
  roofline     the split-K decode kernel (the step's dominant kernel), timed
               alone with HIP events the library records around it, against
               the 8 TB/s HBM peak; decode_call has the whole attention call,
  prefill, ... the other workloads (chunked prefill TFLOP/s against the bf16
               MFMA peak, shared-prefix decode, fp8 long-context decode, and
               both decode workloads at their 8-way head shard: 1 KV head),
  stream_ceiling  a plain read-only kernel over the same pages (context),
  cpu_baseline the CPU oracle on the same decode workload (headline value),
               and on sampled parts of the prefill and long fp8 decode
               workloads, write and attention timed separately.
Algorithmic bytes count each sequence's K and V rows once per KV head, plus q,
out and the block_table entries read; flops count causally visible (query,
key) pairs, 4 * D per pair per head.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6  # dense: 256 CU x 4096 flop/clk x 2.4 GHz
# Core clock the chip sustains under the prefill kernel's MFMA + exp load:
# rocprofv3 --pmc GRBM_GUI_ACTIVE per XCD over the kernel's traced duration
# (about 528K cycles in 265 us, profiles/prefill_bf16_b8_n512.md).  The
# MFMA peak at that clock is the one the kernel can reach on this load.
PREFILL_SUSTAINED_CLOCK_GHZ = 2.0
NOMINAL_CLOCK_GHZ = 2.4
METRIC = "decode KV-read GB/s (% of HBM peak) + prefill TFLOP/s (% MFMA peak), 1 GPU"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
CALIB_BYTES = 256 << 20


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


_TOKEN_RE = re.compile(rb'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def _code_only(src: bytes) -> bytes:
    """C++ source without its comments, whitespace runs collapsed: what the
    compiler sees (string and character literals are kept as written)."""
    text = _TOKEN_RE.sub(lambda m: m.group(0) if m.group(0)[:1] in b"\"'" else b" ", src)
    return re.sub(rb"\s+", b" ", text).strip()


def kernel_source_hash() -> str:
    """Hash of the library's sources as code (comments and layout ignored), so
    that counters taken on one build stay attached to it through comment edits."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.join(ROOT, "paged_kv_cache_243_amd", "csrc"))):
        with open(os.path.join(ROOT, "paged_kv_cache_243_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()))
    return h.hexdigest()[:16]


def decode_kernel_bytes(w) -> int:
    """Algorithmic bytes of the split-K decode kernel alone: K+V rows once per
    (sequence, KV head), q and the block_table entries it reads (its partial
    results are an implementation artefact and are not counted)."""
    cfg = w.cfg
    esz = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[cfg.kv_dtype]
    qsz = 4 if cfg.q_dtype == "f32" else 2
    lens = w.seq_lens.cpu().numpy().astype(int)
    kv = int(lens.sum()) * cfg.hkv * cfg.head_dim * esz * 2
    q = w.q.shape[0] * cfg.hq * cfg.head_dim * qsz
    table = int(sum(-(-l // cfg.page_size) for l in lens)) * 8
    scales = 2 * cfg.hkv * 4 if cfg.kv_dtype == "fp8_e4m3fn" else 0
    return int(kv + q + table + scales)


def decode_bytes(w) -> int:
    """K+V rows once per (sequence, KV head), q, out, block_table entries read."""
    cfg = w.cfg
    esz = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[cfg.kv_dtype]
    qsz = 4 if cfg.q_dtype == "f32" else 2
    lens = w.seq_lens.cpu().numpy().astype(int)
    kv = int(lens.sum()) * cfg.hkv * cfg.head_dim * esz * 2
    T = w.q.shape[0]
    qo = 2 * T * cfg.hq * cfg.head_dim * qsz
    table = int(sum(-(-l // cfg.page_size) for l in lens)) * 8
    scales = 2 * cfg.hkv * 4 if cfg.kv_dtype == "fp8_e4m3fn" else 0
    return int(kv + qo + table + scales)


def unique_decode_bytes(w) -> int:
    """Distinct pages touched (shared pages once) x page bytes for K and V."""
    cfg = w.cfg
    esz = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[cfg.kv_dtype]
    bt = w.block_table.cpu().numpy()
    lens = w.seq_lens.cpu().numpy().astype(int)
    pages = set()
    for b in range(bt.shape[0]):
        pages.update(bt[b, :-(-lens[b] // cfg.page_size)].tolist())
    return int(len(pages) * cfg.page_size * cfg.hkv * cfg.head_dim * esz * 2)


def prefill_flops(w) -> int:
    """4 * D * Hq per causally visible (query, key) pair: QK^T and PV."""
    cfg = w.cfg
    lens = w.seq_lens.cpu().numpy().astype(int)
    qsl = w.query_start_loc.cpu().numpy().astype(int)
    pairs = 0
    for b in range(len(lens)):
        n = qsl[b + 1] - qsl[b]
        P = lens[b] - n
        pairs += n * P + n * (n + 1) // 2
    return int(4 * cfg.head_dim * cfg.hq * pairs)


def write_bytes(w) -> int:
    esz = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[w.cfg.kv_dtype]
    T = w.k_new.shape[0]
    return int(2 * 2 * T * w.cfg.hkv * w.cfg.head_dim * esz + 8 * T)


def fp8_write_bytes(T: int, hkv: int, d: int) -> int:
    """Algorithmic bytes of one quantising write: bf16 K and V rows read, fp8
    codes written, slots and the two scale vectors read."""
    return int(2 * T * hkv * d * (2 + 1) + 8 * T + 2 * 4 * hkv)


class Fp8WriteRunner:
    """Quantising write of the chunked-prefill workload's 4096 new bf16 K/V
    rows into fp8 pools of the same geometry (65536 pages), with per-head
    scales amax / 448 of the rows."""

    def __init__(self, pkv, w, torch):
        self.pkv, self.w = pkv, w
        shape = w.key_pool.shape
        self.kp = torch.zeros(shape, dtype=torch.uint8, device=w.k_new.device)
        self.vp = torch.zeros(shape, dtype=torch.uint8, device=w.k_new.device)
        self.ks = (w.k_new.float().abs().amax(dim=(0, 2)) / 448).contiguous()
        self.vs = (w.v_new.float().abs().amax(dim=(0, 2)) / 448).contiguous()

    def write(self):
        w = self.w
        self.pkv.paged_kv_write_fp8(w.k_new, w.v_new, w.slot_mapping, self.kp, self.vp, self.ks, self.vs)

    def attend(self, kernel_events=None):
        pass


class Runner:
    """Write + attention of one workload with preallocated buffers: two calls
    (paged_kv_write, then paged_attention), or with fused=True the one call
    paged_kv_write_attention (write() then does nothing)."""

    def __init__(self, pkv, w, torch, shared_prefix_pages=0, fused=False):
        self.pkv, self.w, self.torch = pkv, w, torch
        self.shared = shared_prefix_pages
        self.fused = fused
        self.kp, self.vp = w.key_pool, w.value_pool  # written in place each step (same rows)
        self.out = torch.empty_like(w.q)
        need = pkv.paged_attention_workspace_size(w.q, w.key_pool, w.block_table,
                                                  max_query_len=w.max_query_len,
                                                  split_tokens=w.split_tokens,
                                                  shared_prefix_pages=shared_prefix_pages)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.q.device)

    def write(self):
        if self.fused:
            return
        w = self.w
        self.pkv.paged_kv_write(w.k_new, w.v_new, w.slot_mapping, self.kp, self.vp)

    def attend(self, kernel_events=None):
        w = self.w
        if self.fused:
            self.pkv.paged_kv_write_attention(w.k_new, w.v_new, w.slot_mapping, self.kp, self.vp, w.q,
                                              w.block_table, w.seq_lens, w.query_start_loc, w.scale, self.out,
                                              k_scale=w.k_scale, v_scale=w.v_scale,
                                              max_query_len=w.max_query_len, split_tokens=w.split_tokens,
                                              workspace=self.ws, timing_events=kernel_events,
                                              shared_prefix_pages=self.shared)
            return
        self.pkv.paged_attention(w.q, self.kp, self.vp, w.block_table, w.seq_lens, w.query_start_loc,
                                 w.scale, self.out, k_scale=w.k_scale, v_scale=w.v_scale,
                                 max_query_len=w.max_query_len, split_tokens=w.split_tokens,
                                 workspace=self.ws, timing_events=kernel_events,
                                 shared_prefix_pages=self.shared)


class Times:
    """Per-step HIP event times (ms): write, attention call, its main attention
    kernel alone (events the library records on the same stream), whole step."""

    def __init__(self, write, attn, kernel, step, wall):
        self.write, self.attn, self.kernel, self.step, self.wall = write, attn, kernel, step, wall


def time_steps(runner, torch, steps, warmup, flush, progress="", kernel_events=True, mid_event=False):
    """Time `steps` steps after `warmup` untimed ones; the cache flush, when
    given, runs before each step outside its timed region.  With
    kernel_events the library also records a HIP event pair around the main
    attention kernel, and with mid_event one more event separates the write
    from the attention call (each event packet lengthens the step by a few
    microseconds, so whole-step figures come from a pass with events at the
    step's ends only)."""
    for _ in range(warmup):
        runner.write()
        runner.attend()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        e = ev[i]
        e[0].record()
        runner.write()
        if mid_event:
            e[1].record()
        runner.attend(kernel_events=(e[3], e[4]) if kernel_events else None)
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = Times(write=[e[0].elapsed_time(e[1]) for e in ev] if mid_event else None,
              attn=[e[1 if mid_event else 0].elapsed_time(e[2]) for e in ev],
              kernel=[e[3].elapsed_time(e[4]) for e in ev] if kernel_events else None,
              step=[e[0].elapsed_time(e[2]) for e in ev], wall=wall)
    if progress:
        extra = f", main kernel {statistics.median(t.kernel):.4f} ms" if kernel_events else ""
        log(f"{progress}: {steps} steps, median step {statistics.median(t.step):.4f} ms{extra}")
    return t


def time_graph_steps(runner, torch, steps, warmup, flush, progress=""):
    """The same write + attention step captured once as a HIP graph (torch's
    stream capture of the library's launches) and replayed: one replay per
    step, the cache flush before each outside the timed region, HIP events
    around each replay.  Returns the per-step times (ms)."""
    for _ in range(warmup):
        runner.write()
        runner.attend()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        runner.write()
        runner.attend()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        ev[i][0].record()
        g.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    if progress:
        log(f"{progress} (HIP graph): {steps} steps, median step {statistics.median(ms):.4f} ms")
    del g
    return ms


def time_workload(runner, torch, steps, warmup, flush, progress):
    """Timed passes: whole steps with events at their ends only; for the
    two-call form, the write and the attention call apart (an event between
    them); the main kernel alone (events around it)."""
    plain = time_steps(runner, torch, steps, warmup, flush, progress + " (steps)", kernel_events=False)
    split = None
    if not getattr(runner, "fused", False):
        split = time_steps(runner, torch, steps, 1, flush, progress + " (write | attention)", kernel_events=False,
                           mid_event=True)
    kern = time_steps(runner, torch, steps, 1, flush, progress + " (main kernel)", kernel_events=True)
    return plain, split, kern


def traffic_from_profile(kernel: str):
    """Counter-derived HBM bytes per launch from the committed rocprofv3 PMC
    summary, or None when the kernels changed since the counters were taken."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if prof.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = prof.get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("traffic_bytes_per_launch")


def fp8_prefill_config(W):
    """The chunked-prefill workload (8 x 512 new tokens on up to 8192 old) with fp8 E4M3FN pools."""
    import dataclasses
    c = W.CONFIGS[3]
    return dataclasses.replace(c, name=c.name + "-fp8", kv_dtype="fp8_e4m3fn")


def tp_shard(W, cid: int, tp: int):
    """Workload `cid` of the workloads module with the heads one GPU holds under a `tp`-way head split."""
    return W.head_shard(W.CONFIGS[cid], tp)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, limit_s=10.0):
    """Median of 3 wall-clock runs of fn(), or 1 run when it takes longer
    than limit_s; returns (seconds, runs)."""
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if times[-1] > limit_s:
            break
    return statistics.median(times), len(times)


def cpu_oracle_leg(w, sel_tokens=None):
    """The oracle as it stands (fp64, OpenMP over (sequence, KV head)) on a
    workload already resident in host copies: the write of all new tokens and
    the attention of the selected query rows (all when None), timed
    separately.  Returns (write_s, attention_s, threads, runs)."""
    import oracle
    from paged_kv_cache_243_amd import workloads as W
    S = W.to_numpy_storage
    threads = len(os.sched_getaffinity(0))
    kp0, vp0 = S(w.key_pool), S(w.value_pool)
    k, v, sm = S(w.k_new), S(w.v_new), S(w.slot_mapping)
    q, bt, sl, qsl = S(w.q), S(w.block_table), S(w.seq_lens), S(w.query_start_loc)
    ks = None if w.k_scale is None else S(w.k_scale)
    vs = None if w.v_scale is None else S(w.v_scale)
    kp, vp = kp0.copy(), vp0.copy()
    t_write, runs_w = _timed(lambda: oracle.paged_kv_write(k, v, sm, kp, vp))
    t_attn, runs_a = _timed(lambda: oracle.paged_attention(q, w.q_dtype, kp, vp, w.kv_dtype, bt, sl, qsl, w.scale,
                                                           ks, vs, sel_tokens=sel_tokens, threads=threads))
    return t_write, t_attn, threads, min(runs_w, runs_a)


def cpu_baseline_decode(w):
    """Headline CPU baseline: the whole decode step of the timed workload (the
    write of its 64 tokens and the attention of all 64 rows)."""
    tw, ta, threads, runs = cpu_oracle_leg(w)
    return {"value": round(decode_bytes(w) / (tw + ta) / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "ms_per_step": round((tw + ta) * 1e3, 1), "write_ms": round(tw * 1e3, 2),
            "attention_ms": round(ta * 1e3, 1), "cpu": _cpu_model(),
            "sample": f"the full decode step of the timed workload ({w.cfg.batch} sequences: write of "
                      f"{w.k_new.shape[0]} tokens, then attention of every row), fp64, write and attention "
                      f"timed separately, median of {runs} runs"}


def cpu_baseline_prefill(w, every: int = 8):
    """Chunked prefill: the write of all 4096 new tokens, then attention of
    every `every`-th query row (all heads), GFLOP/s over the sampled rows'
    causally visible pairs."""
    import numpy as np
    sel = np.arange(0, w.q.shape[0], every, dtype=np.int64)
    tw, ta, threads, runs = cpu_oracle_leg(w, sel)
    lens = w.seq_lens.cpu().numpy().astype(np.int64)
    qsl = w.query_start_loc.cpu().numpy().astype(np.int64)
    seq = np.searchsorted(qsl, sel, side="right") - 1
    pos = lens[seq] - (qsl[seq + 1] - qsl[seq]) + (sel - qsl[seq])
    flops = int(4 * w.cfg.head_dim * w.cfg.hq * int((pos + 1).sum()))
    return {"value": round(flops / ta / 1e9, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "attention_ms": round(ta * 1e3, 1), "write_ms": round(tw * 1e3, 2),
            "write_GBps": round(write_bytes(w) / tw / 1e9, 3), "flop_sampled": flops,
            "sample": f"the write of all {w.k_new.shape[0]} new tokens, then attention of every {every}th query "
                      f"row ({len(sel)} of {w.q.shape[0]} rows, all heads), fp64, median of {runs} runs"}


def cpu_baseline_long_decode(w, every: int = 2):
    """Long-context fp8 decode: the write of the 16 new tokens, then attention
    of every `every`-th sequence's row; GB/s over those sequences' K/V bytes."""
    import numpy as np
    sel = np.arange(0, w.q.shape[0], every, dtype=np.int64)
    tw, ta, threads, runs = cpu_oracle_leg(w, sel)
    lens = w.seq_lens.cpu().numpy().astype(np.int64)
    kv_bytes = int(lens[sel].sum()) * w.cfg.hkv * w.cfg.head_dim * 2
    return {"value": round(kv_bytes / ta / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "attention_ms": round(ta * 1e3, 1), "write_ms": round(tw * 1e3, 2), "kv_bytes_sampled": kv_bytes,
            "sample": f"the write of all {w.k_new.shape[0]} new tokens, then attention of one sequence in {every} "
                      f"({len(sel)} of {w.q.shape[0]}, {int(lens[sel].sum())} positions), fp64 on fp8 codes "
                      f"dequantised exactly, median of {runs} runs"}


def stream_ceiling(w, torch, flush, steps: int) -> dict:
    """Practical HBM ceiling: a plain read-only kernel (bench_ceiling.hip)
    streaming exactly the K and V pages the decode workload reads, in the
    same order and access shape, with no compute; HIP events around each
    call, the cache flushed before each."""
    import ctypes
    import numpy as np
    from paged_kv_cache_243_amd import build as Bd
    if not os.path.exists(Bd.CEILING_OUT):
        Bd.build_ceiling()
    lib = ctypes.CDLL(Bd.CEILING_OUT)
    lib.stream_read_pages.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                              ctypes.c_void_p, ctypes.c_void_p]
    lib.stream_read_pages.restype = ctypes.c_int
    cfg = w.cfg
    bt = w.block_table.cpu().numpy()
    lens = w.seq_lens.cpu().numpy().astype(np.int64)
    pages = np.concatenate([bt[b, :-(-int(lens[b]) // cfg.page_size)] for b in range(len(lens))])
    pages_t = torch.as_tensor(pages, dtype=torch.int64, device=w.q.device)
    page_bytes = cfg.page_size * cfg.hkv * cfg.head_dim * w.key_pool.element_size()
    moved = int(len(pages)) * page_bytes * 2
    out = {"kernel": "stream_read_kernel (bench_ceiling.hip)", "bytes": moved,
           "pages": int(len(pages)), "page_bytes": page_bytes}
    stream = torch.cuda.current_stream()
    for wgs in (256, 1024):
        sink = torch.empty(wgs * 8, dtype=torch.int32, device=w.q.device)
        call = lambda: lib.stream_read_pages(w.key_pool.data_ptr(), w.value_pool.data_ptr(), pages_t.data_ptr(),
                                             len(pages), page_bytes, wgs, sink.data_ptr(),
                                             ctypes.c_void_p(stream.cuda_stream))
        assert call() == 0
        ms = []
        for _ in range(steps):
            if flush is not None:
                flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        med = statistics.median(ms)
        out[f"workgroups_{wgs}"] = {"ms_median": round(med, 5), "GBps": round(moved / (med * 1e-3) / 1e9, 1),
                                    "frac_of_hbm_peak": round(moved / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def csr_unpack_timing(pkv, w, torch, steps: int) -> dict:
    """The decode workload's metadata given in the packed page-list form
    (kv_indptr, kv_indices, kv_last_page_len) and unpacked on the GPU into
    block_table [64, 256] and seq_lens; HIP events around each call."""
    import numpy as np
    bt0 = w.block_table.cpu().numpy()
    sl0 = w.seq_lens.cpu().numpy()
    n = (sl0 + 15) // 16
    indptr = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int64, device=w.q.device)
    indices = torch.as_tensor(np.concatenate([bt0[b, :n[b]] for b in range(len(n))]), device=w.q.device)
    last = torch.as_tensor(sl0 - (n - 1) * 16, dtype=torch.int64, device=w.q.device)
    bt = torch.empty_like(w.block_table)
    sl = torch.empty_like(w.seq_lens)
    call = lambda: pkv.paged_block_table_from_csr(indptr, indices, last, bt, sl, page_size=16, pad_page=0)
    for _ in range(3):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    moved = int(indptr.numel() * 8 + indices.numel() * 8 + last.numel() * 8 + bt.numel() * 8 + sl.numel() * 8)
    return {"workload": "decode workload's metadata (64 sequences, 256-entry rows) unpacked from the packed "
                        "page list", "kernel": "csr_to_block_table_kernel",
            "call_us_median": round(ms[len(ms) // 2] * 1e3, 2), "bytes": moved,
            "note": "HIP events around one call from Python: bound by the binding's launch cost; the kernel "
                    "alone runs in about 3 us (rocprofv3)"}


def host_control_plane_timing() -> dict:
    """Host cost of one decode step's bookkeeping in the C++ control plane for
    the decode workload's shape: 64 sequences of U{512..4096} tokens in a
    65536-page pool, each appending one token, then the step metadata built
    (block_table [64, 272], seq_lens, query_start_loc)."""
    import numpy as np
    from paged_kv_cache_243_amd.host import PagePool
    rng = np.random.default_rng(243_002)
    pool = PagePool(65536, 16)
    seqs = []
    for _ in range(64):
        s = pool.create()
        pool.append(s, int(rng.integers(511, 4096)))
        seqs.append(s)
    pool.confirm(np.concatenate([pool.pages(s) for s in seqs]))
    n_new = np.ones(64, dtype=np.int64)
    times = []
    for _ in range(200):
        t0 = time.perf_counter()
        pool.append_batch(seqs, n_new)
        pool.build_step(seqs, n_new, 272, 65535)
        times.append(time.perf_counter() - t0)
    times.sort()
    return {"workload": "64 sequences append one token each (one batched call), then the step metadata is "
                        "built (block_table [64, 272]); C++ control plane called from Python",
            "us_per_step_median": round(times[len(times) // 2] * 1e6, 1)}


def _counter_means(run_dir: str, counter: str) -> dict:
    """(mean, dispatches, largest) of `counter` per dispatch, by kernel name,
    over the rocprofv3 counter-collection CSVs under run_dir."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v), max(v)) for k, v in vals.items()}


def write_traffic(fetch_dir: str, write_dir: str) -> int:
    """profiles/traffic.json from the FETCH_SIZE and WRITE_SIZE runs of
    `--profile-workload decode` (the one-call step): each counter (KiB per
    dispatch) is scaled by the factor that maps it, on the 256 MiB device copy
    the profile run launches first, to the copy's true size."""
    from paged_kv_cache_243_amd import workloads as W
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    kib = CALIB_BYTES / 1024

    def calib(table):
        # the largest device copy dispatch is the 256 MiB calibration copy
        copies = [v[2] for k, v in table.items() if "copyBuffer" in k]
        if not copies:
            raise SystemExit("no calibration copy in the counter run")
        return max(copies)
    f_cal, w_cal = calib(fetch), calib(write)
    ff, wf = kib / f_cal, kib / w_cal
    key = next(k for k in fetch if "decode_kernel<2, 128>" in k)
    w2 = W.generate(2, "cpu")
    alg = decode_kernel_bytes(w2) + write_bytes(w2)
    fb = fetch[key][0] * 1024 * ff
    wb = write[key][0] * 1024 * wf
    out = {
        "kernel_source_hash": kernel_source_hash(),
        "note": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each "
                "scaled by the factor that maps the same counter on a 256 MiB device copy to its true size",
        "calibration": {"copy_bytes": CALIB_BYTES, "FETCH_SIZE_KiB": round(f_cal, 1),
                        "WRITE_SIZE_KiB": round(w_cal, 1), "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "kernels": {"decode_kernel<2,128>": {
            "workload": "the one-call paged decode step, bf16, B=64, Hq=32, Hkv=8, D=128, L_b ~ U{512..4096} "
                        "(the split-K pass also writes the 64 new rows)",
            "FETCH_SIZE_KiB_mean": round(fetch[key][0], 1), "WRITE_SIZE_KiB_mean": round(write[key][0], 1),
            "dispatches": fetch[key][1],
            "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
            "traffic_bytes_per_launch": int(fb + wb), "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round((fb + wb) / alg, 4)}},
    }
    with open(PROFILE_TRAFFIC, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out["kernels"]), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="time only the decode workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--profile-workload",
                    choices=["decode", "decode_2calls", "prefill", "prefill_fp8", "shared", "sharedplain", "fp8",
                             "fp8write", "csr", "decode_tp8", "fp8_tp8", "prefill_tp8"],
                    help="time one workload only and print its median times (for profiler runs); decode and fp8 "
                         "run the one-call step the headline times")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(no GPU) write profiles/traffic.json from the rocprofv3 FETCH_SIZE and WRITE_SIZE "
                         "counter runs of --profile-workload decode")
    args = ap.parse_args(argv)

    if args.write_traffic:
        return write_traffic(*args.write_traffic)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    # Kernel arguments in device memory (a HIP runtime option, read when the
    # runtime starts): a launch's first loads of its arguments then stay on
    # the device instead of reaching into host memory.  The one-call decode
    # step measured about 3 us faster with it (interleaved processes).  A
    # value the caller set is kept, and the line reports the one used.
    os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")
    import torch
    import paged_kv_cache_243_amd as pkv
    from paged_kv_cache_243_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pkv.load()
    dev = torch.device("cuda:0")
    flush = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    if args.profile_workload == "csr":
        print(json.dumps(csr_unpack_timing(pkv, W.generate(2, dev), torch, args.steps)), flush=True)
        return 0
    if args.profile_workload == "fp8write":
        w = W.generate(3, dev)
        t = time_steps(Fp8WriteRunner(pkv, w, torch), torch, args.steps, args.warmup, flush, "fp8 write",
                       kernel_events=False, mid_event=True)
        print(json.dumps({"workload": "quantising fp8 write of 4096 bf16 K/V rows (Hkv 8, D 128)",
                          "write_ms_median": statistics.median(t.write),
                          "write_ms_mean": statistics.fmean(t.write)}), flush=True)
        return 0
    if args.profile_workload:
        cid = {"decode": 2, "decode_2calls": 2, "prefill": 3, "prefill_fp8": 3, "shared": 4, "sharedplain": 4,
               "fp8": 5, "decode_tp8": 2, "fp8_tp8": 5, "prefill_tp8": 3}[args.profile_workload]
        if args.profile_workload == "prefill_fp8":
            w = W.generate(fp8_prefill_config(W), dev)
        else:
            w = W.generate(tp_shard(W, cid, 8) if args.profile_workload.endswith("_tp8") else cid, dev)
        # calibration for hardware byte counters: a plain device copy of known
        # size (256 MiB read + 256 MiB written), launched once
        calib = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        torch.empty_like(calib).copy_(calib)
        del calib
        pages = w.cfg.shared_prefix_tokens // w.cfg.page_size if args.profile_workload == "shared" else 0
        fused = args.profile_workload in ("decode", "fp8")
        t = time_steps(Runner(pkv, w, torch, shared_prefix_pages=pages, fused=fused), torch, args.steps,
                       args.warmup, flush, args.profile_workload, mid_event=not fused)
        print(json.dumps({"workload": w.cfg.name, "form": "one call" if fused else "two calls",
                          "write_ms_median": statistics.median(t.write) if t.write else None,
                          "attention_ms_median": statistics.median(t.attn),
                          "main_kernel_ms_median": statistics.median(t.kernel),
                          "main_kernel_ms_mean": statistics.fmean(t.kernel),
                          "step_ms_median": statistics.median(t.step)}), flush=True)
        return 0

    # ---- headline: decode workload, write + attention per step, as the one
    # call paged_kv_write_attention (one kernel pass writes and attends, then
    # the merge); the two separate calls are timed beside it
    log("generating the bf16 decode workload (64 sequences of 512-4096 positions)")
    w2 = W.generate(2, dev)
    r2 = Runner(pkv, w2, torch, fused=True)
    r2s = Runner(pkv, w2, torch)
    t2, _, k2 = time_workload(r2, torch, args.steps, args.warmup, flush, "decode bf16, one call")
    t2s, c2s, k2s = time_workload(r2s, torch, args.steps, args.warmup, flush, "decode bf16, two calls")
    g2 = time_graph_steps(r2, torch, args.steps, args.warmup, flush, "decode bf16, one call")
    bytes2 = decode_bytes(w2)
    kbytes2 = decode_kernel_bytes(w2) + write_bytes(w2)  # the fused kernel also moves the new rows
    step_ms = statistics.median(t2.step)
    attn_ms = statistics.median(c2s.attn)
    kern_ms = statistics.fmean(k2.kernel)
    achieved = kbytes2 / (kern_ms * 1e-3) / 1e9
    warm = time_steps(r2s, torch, max(5, args.steps // 3), 2, None, kernel_events=False, mid_event=True)
    result = {
        "metric": METRIC,
        "value": round(bytes2 / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "runtime": {"HIP_FORCE_DEV_KERNARG": os.environ.get("HIP_FORCE_DEV_KERNARG")},
        "config": {
            "workload": "paged decode, bf16 KV: write 1 new token per sequence, then split-K decode "
                        "attention over each sequence's pages",
            "form": "paged_kv_write_attention (the write and the attention as one call)",
            "batch": w2.cfg.batch, "q_heads": w2.cfg.hq, "kv_heads": w2.cfg.hkv,
            "head_dim": w2.cfg.head_dim, "page_size": w2.cfg.page_size, "num_pages": w2.cfg.num_pages,
            "context_lengths": "U{512..4096}", "kv_dtype": "bf16", "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel<2,128> (split-K decode pass, writing the new rows)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile("decode_kernel<2,128>"),
            "algorithmic_bytes_per_launch": kbytes2,
            "launch_ms_mean": round(kern_ms, 5),
            "launch_ms_median": round(statistics.median(k2.kernel), 5),
            "launch_ms_min": round(min(k2.kernel), 5),
            "launches_timed": len(k2.kernel),
        },
        "two_calls": {
            "form": "paged_kv_write, then paged_attention",
            "step_ms_median": round(statistics.median(t2s.step), 5),
            "step_GBps": round(bytes2 / (statistics.median(t2s.step) * 1e-3) / 1e9, 1),
            "step_frac_of_hbm_peak": round(bytes2 / (statistics.median(t2s.step) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "write_ms_median": round(statistics.median(c2s.write), 5),
            "decode_kernel_ms_mean": round(statistics.fmean(k2s.kernel), 5),
            "decode_kernel_GBps": round(decode_kernel_bytes(w2) / (statistics.fmean(k2s.kernel) * 1e-3) / 1e9, 1),
        },
        "decode_call": {
            "kernels": "decode_kernel + merge_kernel (paged_attention)",
            "algorithmic_bytes": bytes2,
            "ms_median": round(attn_ms, 5),
            "ms_min": round(min(c2s.attn), 5),
            "GBps": round(bytes2 / (attn_ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(bytes2 / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_warm_median": round(statistics.median(warm.attn), 5),
        },
        "graph_step": {
            "form": "the same one-call step captured once as a HIP graph and replayed",
            "ms_median": round(statistics.median(g2), 5),
            "GBps": round(bytes2 / (statistics.median(g2) * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(bytes2 / (statistics.median(g2) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "timed_loop_wall_s": round(t2.wall, 4),
    }
    if not args.no_extra:
        result["csr_unpack"] = csr_unpack_timing(pkv, w2, torch, args.steps)
        log("streaming-read ceiling over the decode workload's pages")
        result["stream_ceiling"] = stream_ceiling(w2, torch, flush, args.steps)
    del r2, r2s
    cpu = {}

    if not args.no_extra:
        extra = {}
        # chunked prefill
        log("generating the chunked-prefill workload (8 x 512 new tokens)")
        w3 = W.generate(3, dev)
        r3 = Runner(pkv, w3, torch)
        t3, c3, kt3 = time_workload(r3, torch, max(5, args.steps // 2), args.warmup, flush, "prefill bf16")
        fl = prefill_flops(w3)
        a3 = statistics.median(c3.attn)
        k3 = statistics.fmean(kt3.kernel)
        # quantising fp8 write of the same 4096 new rows
        fw = time_steps(Fp8WriteRunner(pkv, w3, torch), torch, args.steps, args.warmup, flush,
                        "fp8 quantising write", kernel_events=False, mid_event=True)
        fw_ms = statistics.median(fw.write)
        fw_bytes = fp8_write_bytes(w3.k_new.shape[0], w3.cfg.hkv, w3.cfg.head_dim)
        extra["fp8_quantising_write"] = {
            "workload": "4096 new bf16 K/V rows (Hkv 8, head_dim 128) quantised to E4M3FN with per-head "
                        "scales and scattered into 65536-page fp8 pools",
            "kernel": "slot_scatter_fp8_kernel",
            "bound": "hbm", "unit": "GB/s",
            "algorithmic_bytes": fw_bytes,
            "ms_median": round(fw_ms, 5),
            "achieved": round(fw_bytes / (fw_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "frac": round(fw_bytes / (fw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        extra["prefill"] = {
            "workload": "chunked causal prefill, bf16: 8 sequences x 512 new tokens on U{0..8192} old "
                        "context, Hq 32, Hkv 8, head_dim 128",
            "kernel": "prefill_kernel<2,128,1>",
            "bound": "mfma", "unit": "TFLOP/s",
            "achieved": round(fl / (k3 * 1e-3) / 1e12, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "frac": round(fl / (k3 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "sustained_clock_GHz": PREFILL_SUSTAINED_CLOCK_GHZ,
            "frac_of_peak_at_sustained_clock": round(fl / (k3 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS
                                                     * NOMINAL_CLOCK_GHZ / PREFILL_SUSTAINED_CLOCK_GHZ, 4),
            "sustained_clock_source": "rocprofv3 GRBM_GUI_ACTIVE per XCD over the traced kernel duration",
            "flop_per_launch": fl,
            "launch_ms_mean": round(k3, 5),
            "call_ms_median": round(a3, 5),
            "call_TFLOPs": round(fl / (a3 * 1e-3) / 1e12, 2),
            "write_ms_median": round(statistics.median(c3.write), 5),
            "write_GBps": round(write_bytes(w3) / (statistics.median(c3.write) * 1e-3) / 1e9, 1),
            "step_ms_median": round(statistics.median(t3.step), 5),
        }
        del r3
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on the chunked-prefill workload (sampled rows)")
            cpu["prefill"] = cpu_baseline_prefill(w3)
        del w3
        torch.cuda.empty_cache()
        # the same chunked prefill over fp8 E4M3FN pools (per-head scales)
        log("generating the chunked-prefill workload with fp8 KV")
        w3f = W.generate(fp8_prefill_config(W), dev)
        r3f = Runner(pkv, w3f, torch)
        t3f, c3f, kt3f = time_workload(r3f, torch, max(5, args.steps // 2), args.warmup, flush, "prefill fp8 KV")
        k3f = statistics.fmean(kt3f.kernel)
        fl3f = prefill_flops(w3f)
        extra["prefill_fp8_kv"] = {
            "workload": "the chunked causal prefill over fp8 E4M3FN pools with per-head scales (codes widened "
                        "exactly to bf16, bf16 MFMA)",
            "kernel": "prefill_kernel<1,128,1>",
            "bound": "mfma", "unit": "TFLOP/s",
            "achieved": round(fl3f / (k3f * 1e-3) / 1e12, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "frac": round(fl3f / (k3f * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "flop_per_launch": fl3f,
            "launch_ms_mean": round(k3f, 5),
            "call_ms_median": round(statistics.median(c3f.attn), 5),
            "step_ms_median": round(statistics.median(t3f.step), 5),
        }
        del r3f, w3f
        torch.cuda.empty_cache()
        # shared-prefix decode
        log("generating the shared-prefix decode workload (256 sequences on a 2048-position prefix)")
        w4 = W.generate(4, dev)
        pages4 = w4.cfg.shared_prefix_tokens // w4.cfg.page_size
        r4 = Runner(pkv, w4, torch, shared_prefix_pages=pages4)
        t4 = time_steps(r4, torch, args.steps, args.warmup, flush, "shared-prefix decode", kernel_events=False,
                        mid_event=True)
        r4p = Runner(pkv, w4, torch)
        t4p = time_steps(r4p, torch, args.steps, args.warmup, flush, "shared-prefix decode, plain call",
                         kernel_events=False, mid_event=True)
        a4 = statistics.median(t4.attn)
        a4p = statistics.median(t4p.attn)
        extra["shared_prefix_decode"] = {
            "workload": "256 sequences sharing 128 prefix pages + U{0..512} private tokens, Hq 64, Hkv 8",
            "form": f"shared_prefix_pages={pages4}: one launch whose first workgroups run the split-K decode of the "
                    f"private positions and the rest the prefix once as MFMA tiles, then the merge",
            "unit": "GB/s",
            "logical_GBps": round(decode_bytes(w4) / (a4 * 1e-3) / 1e9, 1),
            "unique_GBps": round(unique_decode_bytes(w4) / (a4 * 1e-3) / 1e9, 1),
            "attention_ms_median": round(a4, 5),
            "step_ms_median": round(statistics.median(t4.step), 5),
            "plain_call_attention_ms_median": round(a4p, 5),
            "plain_call_logical_GBps": round(decode_bytes(w4) / (a4p * 1e-3) / 1e9, 1),
        }
        del r4p
        del r4, w4
        torch.cuda.empty_cache()
        # long-context fp8 decode
        log("generating the long-context fp8 decode workload (16 sequences of 32k-128k positions)")
        w5 = W.generate(5, dev)
        r5 = Runner(pkv, w5, torch, fused=True)
        t5, _, kt5 = time_workload(r5, torch, args.steps, args.warmup, flush, "fp8 long decode")
        g5 = time_graph_steps(r5, torch, args.steps, args.warmup, flush, "fp8 long decode")
        k5 = statistics.fmean(kt5.kernel)
        b5 = decode_bytes(w5)
        kb5 = decode_kernel_bytes(w5) + write_bytes(w5)  # the fused kernel also moves the new rows
        extra["fp8_long_decode"] = {
            "workload": "16 sequences, U{32768..131072} positions, fp8 E4M3FN KV with per-head scales, "
                        "Hq 64, Hkv 8, split_tokens 2048: the (sequence, 32-position unit) list cut into "
                        "equal stream-K ranges (their count set by split_tokens), merged per sequence by "
                        "log-sum-exp",
            "form": "paged_kv_write_attention (the write and the attention as one call)",
            "kernel": "decode_kernel<1,128> (split-K decode pass, writing the new rows)",
            "bound": "hbm", "unit": "GB/s",
            "achieved": round(kb5 / (k5 * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "frac": round(kb5 / (k5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": kb5,
            "launch_ms_mean": round(k5, 5),
            "step_ms_median": round(statistics.median(t5.step), 5),
            "step_GBps": round(b5 / (statistics.median(t5.step) * 1e-3) / 1e9, 1),
            "step_frac_of_hbm_peak": round(b5 / (statistics.median(t5.step) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "graph_step_ms_median": round(statistics.median(g5), 5),
            "graph_step_GBps": round(b5 / (statistics.median(g5) * 1e-3) / 1e9, 1),
            "graph_step_frac_of_hbm_peak": round(b5 / (statistics.median(g5) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        del r5
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on the long-context fp8 decode workload (sampled sequences)")
            cpu["long_fp8_decode"] = cpu_baseline_long_decode(w5)
        del w5
        torch.cuda.empty_cache()
        # the two decode workloads at their 8-way tensor-parallel shard: one KV
        # head (and its query heads) per GPU, all sequences and positions
        shards = {}
        for cid, key in ((2, "decode_bf16"), (5, "long_decode_fp8")):
            log(f"generating the 8-way head shard of the {key} workload")
            ws = W.generate(tp_shard(W, cid, 8), dev)
            rs = Runner(pkv, ws, torch)
            ts, cs, kts = time_workload(rs, torch, args.steps, args.warmup, flush, f"{key}, 8-way head shard")
            ks = statistics.fmean(kts.kernel)
            kbs = decode_kernel_bytes(ws)
            shards[key] = {
                "q_heads": ws.cfg.hq, "kv_heads": ws.cfg.hkv, "kv_dtype": ws.cfg.kv_dtype,
                "algorithmic_bytes_per_launch": kbs,
                "launch_ms_mean": round(ks, 5),
                "achieved_GBps": round(kbs / (ks * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(kbs / (ks * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "call_ms_median": round(statistics.median(cs.attn), 5),
            }
            del rs, ws
            torch.cuda.empty_cache()
        extra["tp8_shard_decode"] = {
            "workload": "the bf16 decode workload and the long-context fp8 decode with the query and KV "
                        "heads of one GPU of an 8-way head split (1 KV head); not the headline",
            "kernel": "decode_kernel (one-wave parts, 8 per workgroup)",
            **shards,
        }
        result.update(extra)

    if not args.no_extra:
        result["host_control_plane"] = host_control_plane_timing()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the decode workload")
        result["cpu_baseline"] = {**cpu_baseline_decode(w2), **cpu}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
