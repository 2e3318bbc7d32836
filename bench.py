"""Benchmark: K4V2 g128 quantize-append + scale-folded paged decode attention.

One step = quantise-append of the new token of every sequence, then one decode
step of attention over the packed cache (every row of the hot path), on the
Qwen3-32B-shaped workload: 8 sequences x 16384 cached tokens (+1 appended),
64 query / 8 KV heads, head_dim 128, 16-token pages in a random block table.
Synthetic seeded inputs (kvq_inputs); no model weights or datasets.

Timing: inputs resident in HBM; W untimed warm-up steps, then K timed steps
bracketed by torch.cuda.synchronize().  Each step runs on the next of R
copies of the pool (R x 109 MB, more than the 256 MB Infinity Cache), so
every decode reads its 109 MB from HBM.  A step is two C-ABI calls on one
stream: kvq_append_decode_partials (the split kernel, which also encodes each
sequence's new token into its page before reading it; the dominant kernel)
and kvq_decode_combine.  The timed steps carry no events.

roofline.achieved: after the timed steps and --kernel-warmup untimed
launches (the shader clock ramps back up for ~10 ms after the idle gap of a
sync), --kernel-launches back-to-back launches of the split kernel alone
(same arguments, same pool rotation) run between two HIP events recorded on
the launch stream; their elapsed time over the launch count is the kernel's
average launch duration.  Per-launch kernel
events (kvq_set_split_kernel_events, hipExtLaunchKernel's start/stop events)
are available with --event-every N, but each timed launch then runs a few
microseconds longer than an untimed one, so they are not the default.

roofline.traffic: HBM bytes per launch of the split kernel from rocprofv3
FETCH_SIZE and WRITE_SIZE counter runs, each scaled by the factor the same
counter reads for a device-to-device copy of known size.  The figures are
read from profiles/decode_kernel_qwen3_32b_16k_traffic.txt and reported only
while the kernel sources still hash to the value recorded there (null
otherwise).  --copy-probe-mb adds the calibration copy to a run.

Prints one JSON line.  N > 1 GPUs is not supported: this build measures one
GPU's share (see the design notes for how the path shards).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "K4V2 decode-attention KV GB/s and % of HBM peak; quantize-append tokens/s"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, vendor figure
KV_BYTES_PER_TOKEN_HEAD = 104
APPEND_BYTES_PER_TOKEN_HEAD = 512 + 104


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=6, help="pool copies cycled to defeat the Infinity Cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the oracle sample (default: min(16, cpu count)); one group each")
    ap.add_argument("--no-append-bench", action="store_true")
    ap.add_argument("--no-fp16-baseline", action="store_true",
                    help="skip the uncompressed fp16 cache decode on the same workload")
    ap.add_argument("--no-mixed-window", action="store_true",
                    help="skip the fp16 sink + recent window beside the K4V2 history")
    ap.add_argument("--no-presets", action="store_true",
                    help="skip the k4v4 / k8v2 / k8v4 / k3v3 presets on the same workload")
    ap.add_argument("--preset-list", default="",
                    help="comma-separated preset:page_tokens legs to run instead of the default list "
                         "(e.g. k4v2_g128:64)")
    ap.add_argument("--no-multi-query", action="store_true",
                    help="skip the multi-row (speculative draft) decode on the same cache")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the labelled warm-cache timing of the split kernel")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the decode of the other workload shapes (Qwen3-4B, Qwen3-30B-A3B, Llama-3.1-70B)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the measured read ceilings (kvq_stream_read_probe, kvq_page_walk_probe)")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--kernel-launches", type=int, default=200,
                    help="back-to-back split-kernel launches timed for roofline.achieved")
    ap.add_argument("--kernel-warmup", type=int, default=400,
                    help="untimed split-kernel launches right before the timed ones (shader clock ramp)")
    ap.add_argument("--dist-blocks", type=int, default=100,
                    help="blocks timed for the per-step median and p10/p90 (0: skip)")
    ap.add_argument("--dist-block-steps", type=int, default=10,
                    help="steps per distribution block (one event between blocks)")
    ap.add_argument("--event-every", type=int, default=0,
                    help="also time the split kernel with kernel events on every N-th timed step (0: off)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_qwen3_32b_16k_traffic.txt")
DECODE_SOURCES = [os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "csrc", f)
                  for f in ("kvq_decode.hip", "kvq_decode_common.h", "kvq_device.h", "kvq_quant.h")] + \
                 [os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "build.py")]   # compile flags


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """(bytes per launch, note) from the committed counter summary, or (None,
    reason) when it is missing or the kernel changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    rec = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256") != decode_source_hash():
        return None, "kernel changed since the counters were taken"
    try:
        return int(rec["fetch_bytes_per_launch"]) + int(rec["write_bytes_per_launch"]), \
            f"fetch {rec['fetch_bytes_per_launch']} + write {rec['write_bytes_per_launch']} B (scaled)"
    except (KeyError, ValueError):
        return None, "malformed counter summary"


class HipEvents:
    """Timing events from the HIP runtime the process already uses (the one
    libkvq is linked against), through ctypes."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def record(self, i, stream_ptr):
        if self.hip.hipEventRecord(self.ev[i], ctypes.c_void_p(stream_ptr)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        t = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(t), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


class DecodeCall:
    """Pre-marshalled C-ABI calls (one ctypes call per kernel launch)."""

    def __init__(self, kvq, lib, fmt, stream_ptr):
        self.kvq, self.lib, self.fmt, self.stream = kvq, lib, ctypes.byref(fmt), ctypes.c_void_p(stream_ptr)

    def append_args(self, k, v, slots, cache):
        P = ctypes.c_void_p
        return (self.fmt, P(k.data_ptr()), P(v.data_ptr()), ctypes.c_int64(k.stride(0)),
                ctypes.c_int64(v.stride(0)), P(slots.data_ptr()), ctypes.c_int64(k.shape[0]),
                ctypes.c_int32(k.shape[1]), P(cache.data_ptr()), ctypes.c_int64(cache.shape[0]), self.stream)

    def fused_args(self, k, v, q, cache, bt, lens, max_len, ws, pps):
        P = ctypes.c_void_p
        return (self.fmt, P(k.data_ptr()), P(v.data_ptr()), ctypes.c_int64(k.stride(0)),
                ctypes.c_int64(v.stride(0)), P(q.data_ptr()), P(cache.data_ptr()), ctypes.c_int64(cache.shape[0]),
                P(bt.data_ptr()), ctypes.c_int32(bt.shape[1]), P(lens.data_ptr()), ctypes.c_int32(q.shape[0]),
                ctypes.c_int32(q.shape[1]), ctypes.c_int32(cache.shape[1]), ctypes.c_int32(max_len),
                ctypes.c_float(1.0 / math.sqrt(128)), P(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                ctypes.c_int32(pps), self.stream)

    def partials_args(self, q, cache, bt, lens, max_len, ws, pps):
        P = ctypes.c_void_p
        return (self.fmt, P(q.data_ptr()), P(cache.data_ptr()), ctypes.c_int64(cache.shape[0]),
                P(bt.data_ptr()), ctypes.c_int32(bt.shape[1]), P(lens.data_ptr()), ctypes.c_int32(q.shape[0]),
                ctypes.c_int32(q.shape[1]), ctypes.c_int32(cache.shape[1]), ctypes.c_int32(max_len),
                ctypes.c_float(1.0 / math.sqrt(128)), P(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                ctypes.c_int32(pps), self.stream)

    def combine_args(self, out, lens, num_q_heads, num_kv_heads, max_len, ws, pps):
        P = ctypes.c_void_p
        return (self.fmt, P(out.data_ptr()), 0 if out.dtype.itemsize == 2 else 1, P(lens.data_ptr()),
                ctypes.c_int32(lens.numel()), ctypes.c_int32(num_q_heads), ctypes.c_int32(num_kv_heads),
                ctypes.c_int32(max_len), P(ws.data_ptr()), ctypes.c_size_t(ws.numel()), ctypes.c_int32(pps),
                self.stream)


def clock_warmup(fn, argl, ms_per_call, args):
    """Untimed launches worth about as much GPU time as the headline's
    --kernel-warmup launches (~25 us each), so that a timed kernel loop starts
    with the shader clock out of the ramp that follows an idle gap."""
    n = int(min(400, max(20, math.ceil(args.kernel_warmup * 0.025 / max(ms_per_call, 1e-3)))))
    if args.kernel_warmup <= 0:
        n = 0
    bad = 0
    for i in range(n):
        bad |= fn(*argl[i % len(argl)])
    return bad


def read_ceiling(torch, lib, dev, stream, nbytes, copies, launches):
    """The plain streaming-read rate of this device (kvq_stream_read_probe):
    `copies` buffers of the decode's KV bytes read in turn, back to back (the
    same rotation through more memory than the 256 MB Infinity Cache holds
    as the decode's pool copies), and a 2 GiB read for the steady state."""
    nb = (nbytes + 15) // 16 * 16
    bufs = [torch.zeros(nb, dtype=torch.uint8, device=dev) for _ in range(copies)]
    big = torch.zeros(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    fn = lib.kvq_stream_read_probe
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    args = [(P(b.data_ptr()), ctypes.c_size_t(nb), P(sink.data_ptr()), sp) for b in bufs]
    big_args = (P(big.data_ptr()), ctypes.c_size_t(big.numel()), P(sink.data_ptr()), sp)
    torch.cuda.synchronize()
    bad = 0
    for i in range(5):
        bad |= fn(*args[i % copies])
    ev = HipEvents(4)
    ev.record(0, stream.cuda_stream)
    for i in range(launches):
        bad |= fn(*args[i % copies])
    ev.record(1, stream.cuda_stream)
    nbig = 10
    for i in range(nbig):
        bad |= fn(*big_args)
    ev.record(2, stream.cuda_stream)
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("kvq_stream_read_probe failed")
    us = ev.elapsed_ms(0, 1) / launches * 1e3
    big_us = ev.elapsed_ms(1, 2) / nbig * 1e3
    ev.close()
    del bufs, big
    return {"kernel": "stream_read_kernel", "bytes_per_launch": nb, "us_per_launch": round(us, 3),
            "GBps": round(nb / us / 1e3, 1), "steady_2GiB_GBps": round((2 << 30) / big_us / 1e3, 1),
            "launches": launches}


def page_walk_ceiling(torch, lib, fmt, dev, stream, pools, bt, lens, B, Hkv, max_len, pps, launches):
    """The decode's own page walk without its arithmetic (kvq_page_walk_probe):
    the same pool copies, block table, sequence lengths and split size, the
    same work decomposition and bytes, launched back to back.  The rate of
    the decode's access pattern (random page regions), beside the plain
    sequential read."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    P = ctypes.c_void_p
    sp = P(stream.cuda_stream)
    fn = lib.kvq_page_walk_probe
    args = [(ctypes.byref(fmt), P(p.data_ptr()), ctypes.c_int64(p.shape[0]), P(bt.data_ptr()),
             ctypes.c_int32(bt.shape[1]), P(lens.data_ptr()), ctypes.c_int32(B), ctypes.c_int32(Hkv),
             ctypes.c_int32(max_len), ctypes.c_int32(pps), P(sink.data_ptr()), sp) for p in pools]
    torch.cuda.synchronize()
    bad = 0
    for i in range(5):
        bad |= fn(*args[i % len(args)])
    ev = HipEvents(2)
    ev.record(0, stream.cuda_stream)
    for i in range(launches):
        bad |= fn(*args[i % len(args)])
    ev.record(1, stream.cuda_stream)
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("kvq_page_walk_probe failed")
    us = ev.elapsed_ms(0, 1) / launches * 1e3
    ev.close()
    return {"kernel": "page_walk_kernel", "us_per_launch": round(us, 3), "launches": launches,
            "pages_per_split": pps}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, groups: int, threads: int):
    """The oracle (plain C) on a bounded sample of the same workload: `groups`
    (sequence, KV head) groups of 16385 tokens, each quantise-appended and
    decoded for its 8 query heads, run on `threads` host threads at once (the
    oracle's C calls release the GIL; groups are independent).  Also times one
    group on one thread."""
    import concurrent.futures as cf
    import numpy as np
    import kvq_inputs as inp
    import oracle
    n = int(inp.final_lens(w)[0])
    pages = -(-n // 16)
    units = [(b, h) for b in range(w.num_seqs) for h in range(w.num_kv_heads)][:groups]
    kv = {b: inp.sequence_kv(w, b, 0, n) for b in sorted({b for b, _ in units})}
    q = inp.queries(w).numpy()
    pools = {u: np.zeros((pages, 1, 1664), np.uint8) for u in units}
    bt = np.arange(pages, dtype=np.int32)[None]
    slots = np.arange(n, dtype=np.int64)

    def append(u):
        b, h = u
        k, v = kv[b]
        oracle.quantize_append(k[:, h:h + 1].numpy(), v[:, h:h + 1].numpy(), slots, pools[u])

    def decode(u):
        b, h = u
        oracle.decode_attention(pools[u], bt, np.array([n]), q[b:b + 1, h * w.gqa:(h + 1) * w.gqa],
                                1 / math.sqrt(128))

    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(append, units))
        t1 = time.perf_counter()
        list(ex.map(decode, units))
        t2 = time.perf_counter()
    t3 = time.perf_counter()
    decode(units[0])
    t4 = time.perf_counter()
    kv_bytes = len(units) * n * KV_BYTES_PER_TOKEN_HEAD
    return {
        "value": kv_bytes / (t2 - t1) / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "oracle_form": "plain-definition oracle as written for parity: every cached token is dequantised "
                       "and un-rotated by a dense fp64 128x128 Hadamard product (16384 multiply-adds per "
                       "vector, not an O(896) FWHT), then fp64 softmax(q.k) v; not a tuned CPU decode",
        "sample": f"{len(units)} (sequence, KV head) groups of qwen3_32b_16k, {n} tokens each: quantise-append, "
                  f"then decode of {w.gqa} query heads per group (fp64 plain definition), one group per thread",
        "seconds": round(t2 - t0, 2),
        "append_tokens_per_s": len(units) * n / (t1 - t0) / w.num_kv_heads,
        "single_thread_value": n * KV_BYTES_PER_TOKEN_HEAD / (t4 - t3) / 1e9,
        "host_cpu": cpu_model(),
        "host_threads_available": os.cpu_count(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by (sequence, KV head) with no exchange, see the design notes", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import kvq_inputs as inp
    import quantized_decode_attention_quantize_amd as kvq

    dev = torch.device("cuda:0")
    lib = kvq.load()
    if args.copy_probe_mb > 0:
        # calibration for the byte counters: one plain copy of known size
        src = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fmt = kvq.format_from_string("kvarn_k4v2_g128")
    stream = torch.cuda.current_stream()
    call = DecodeCall(kvq, lib, fmt, stream.cuda_stream)

    w = inp.workload("qwen3_32b_16k")
    B, Hq, Hkv = w.num_seqs, w.num_q_heads, w.num_kv_heads
    ctx = w.context
    n = ctx + 1
    bt_np, num_pages = inp.page_table(w)
    bt = torch.from_numpy(bt_np).to(dev)
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)

    # fill one pool with the 16384 cached tokens of every sequence, then copy it
    base = torch.zeros((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    for b in range(B):
        k, v = inp.sequence_kv(w, b, 0, ctx, device=dev)
        kvq.quantize_append(k, v, torch.from_numpy(inp.slot_mapping(bt_np, b, 0, ctx)).to(dev), base)
    pools = [base] + [base.clone() for _ in range(args.replicas - 1)]
    new_k, new_v = [], []
    for b in range(B):
        k, v = inp.sequence_kv(w, b, ctx, 1, device=dev)
        new_k.append(k)
        new_v.append(v)
    new_k = torch.cat(new_k).contiguous()       # [B][Hkv][128]: token ctx of every sequence
    new_v = torch.cat(new_v).contiguous()
    q = inp.queries(w, 0, device=dev).contiguous()
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    pps = args.pages_per_split
    ws = kvq.alloc_workspace(B, Hq, Hkv, n, pps)
    torch.cuda.synchronize()

    part_args = [call.fused_args(new_k, new_v, q, p, bt, lens, n, ws, pps) for p in pools]
    comb_args = call.combine_args(out, lens, Hq, Hkv, n, ws, pps)
    part_fn, comb_fn = lib.kvq_append_decode_partials, lib.kvq_decode_combine

    set_events = lib.kvq_set_split_kernel_events

    def step(i, ev=None):
        r = i % len(pools)
        if ev is not None:
            set_events(hev.ev[2 * ev], hev.ev[2 * ev + 1])
        st = part_fn(*part_args[r])
        if ev is not None:
            set_events(None, None)
        st |= comb_fn(*comb_args)
        return st

    for i in range(args.warmup):
        if step(i):
            raise RuntimeError("kvq call failed during warm-up")
    torch.cuda.synchronize()
    sampled = {}
    if args.event_every > 0:
        sampled = {i: k for k, i in enumerate(range(0, args.steps, args.event_every))}
    hev = HipEvents(2 * len(sampled) + 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bad = 0
    for i in range(args.steps):
        bad |= step(args.warmup + i, sampled.get(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if bad:
        raise RuntimeError("kvq call failed in the timed region")
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # the split kernel alone, back to back, between two events on its stream,
    # after --kernel-warmup untimed launches: after an idle gap (the sync
    # above) the shader clock ramps back up over ~10 ms, and the first ~400
    # launches measured ~8% slower than the ones after them
    nl = max(1, args.kernel_launches)
    nw = max(0, args.kernel_warmup)
    k0 = args.warmup + args.steps
    for i in range(nw):
        bad |= part_fn(*part_args[(k0 + i) % len(pools)])
    kl0 = 2 * len(sampled)
    hev.record(kl0, stream.cuda_stream)
    for i in range(nl):
        bad |= part_fn(*part_args[(k0 + nw + i) % len(pools)])
    hev.record(kl0 + 1, stream.cuda_stream)
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("kvq call failed in the kernel-only launches")
    dec_avg_ms = hev.elapsed_ms(kl0, kl0 + 1) / nl
    ev_ms = [hev.elapsed_ms(2 * k, 2 * k + 1) for k in range(len(sampled))]
    hev.close()

    # spread of the per-step time: --dist-blocks blocks of --dist-block-steps
    # steps each, one event between consecutive blocks (each event adds its
    # own marker gap, ~1/block_steps of it per step); per-step time of a block
    # = its elapsed time / block_steps.  The same for the split kernel alone.
    dist = kdist = None
    if args.dist_blocks > 0:
        nb, bs = args.dist_blocks, max(1, args.dist_block_steps)

        def blocks(fn_block):
            he = HipEvents(nb + 1)
            he.record(0, stream.cuda_stream)
            failed = 0
            for k in range(nb):
                failed |= fn_block(k)
                he.record(k + 1, stream.cuda_stream)
            torch.cuda.synchronize()
            if failed:
                raise RuntimeError("kvq call failed in the distribution blocks")
            per = np.array([he.elapsed_ms(k, k + 1) / bs for k in range(nb)])
            he.close()
            return {"median_ms": round(float(np.median(per)), 5),
                    "p10_ms": round(float(np.percentile(per, 10)), 5),
                    "p90_ms": round(float(np.percentile(per, 90)), 5),
                    "mean_ms": round(float(per.mean()), 5), "blocks": nb, "steps_per_block": bs}

        base_i = args.warmup + args.steps + nw + nl
        dist = blocks(lambda k: sum(step(base_i + k * bs + j) for j in range(bs)))
        kdist = blocks(lambda k: sum(part_fn(*part_args[(base_i + k * bs + j) % len(pools)]) for j in range(bs)))
    # labelled warm figure: the same launches on one pool copy, whose 109 MB
    # stay in the 256 MB Infinity Cache between launches (not the headline)
    warm_ms = None
    if not args.no_warm:
        hw = HipEvents(2)
        for i in range(5):
            part_fn(*part_args[0])
        hw.record(0, stream.cuda_stream)
        for i in range(nl):
            bad |= part_fn(*part_args[0])
        hw.record(1, stream.cuda_stream)
        torch.cuda.synchronize()
        if bad:
            raise RuntimeError("kvq call failed in the warm launches")
        warm_ms = hw.elapsed_ms(0, 1) / nl
        hw.close()
    # output quality of the benchmark step: relative MSE against exact
    # attention over the unquantised keys and values (sampled sequences)
    quality_ref = attention_reference(torch, inp, w, q, QUALITY_SEQS)
    step(0)
    torch.cuda.synchronize()
    out_rel_mse = rel_mse(out, quality_ref)
    traffic, traffic_note = recorded_traffic()
    ceiling = walk = None
    if not args.no_read_ceiling:
        ceiling = read_ceiling(torch, lib, dev, stream, B * n * Hkv * KV_BYTES_PER_TOKEN_HEAD, len(pools), nl)
        walk = page_walk_ceiling(torch, lib, fmt, dev, stream, pools, bt, lens, B, Hkv, n,
                                 pps or kvq.decode_pages_per_split(B, Hq, Hkv, n), nl)

    kv_bytes = B * n * Hkv * KV_BYTES_PER_TOKEN_HEAD
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (dec_avg_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded kvq_inputs; no model weights)",
        "config": {"workload": "qwen3_32b_16k", "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": 128, "context": n, "page": 16, "format": "kvq-k4v2-g128 v1",
                   "step": "append 1 token/seq fused into the decode split kernel + combine",
                   "pool_replicas": len(pools),
                   "pages_per_split": pps or kvq.decode_pages_per_split(B, Hq, Hkv, n)},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "output_rel_mse": float(f"{out_rel_mse:.4e}"),
        "output_rel_mse_note": f"sum |out - exact|^2 / sum |exact|^2, sequences {list(QUALITY_SEQS)}, all heads; "
                               "exact = fp32 attention over the unquantised fp16 keys and values",
        "ms_per_step_median": None if dist is None else dist["median_ms"],
        "ms_per_step_p10": None if dist is None else dist["p10_ms"],
        "ms_per_step_p90": None if dist is None else dist["p90_ms"],
        "step_distribution": dist,
        "decode_kernel_ms": round(dec_avg_ms, 5),
        "decode_kernel_distribution": kdist,
        "decode_kernel_launches_timed": nl,
        "decode_kernel_launches_warmup": nw,
        "warm_cache_decode_kernel_ms": None if warm_ms is None else round(warm_ms, 5),
        "warm_cache_note": "one pool copy re-read back to back (resident in the 256 MB Infinity Cache); "
                           "not HBM-bound, not the roofline figure",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "decode_kernel", "bytes_per_launch": kv_bytes, "traffic_note": traffic_note},
    }
    if ceiling:
        # the same bytes read front to back by a plain streaming kernel on this
        # device: the rate the decode's page walk is measured against
        ceiling["decode_frac_of_it"] = round(achieved / ceiling["GBps"], 4)
        result["roofline"]["measured_read_ceiling"] = ceiling
    if walk:
        # the decode's own reads (same pages, order and decomposition) with
        # no arithmetic: the ceiling of its access pattern
        walk["bytes_per_launch"] = kv_bytes
        walk["GBps"] = round(kv_bytes / walk["us_per_launch"] / 1e3, 1)
        walk["decode_frac_of_it"] = round(achieved / walk["GBps"], 4)
        result["roofline"]["measured_page_walk_ceiling"] = walk

    if ev_ms:
        result["kernel_events_in_steps"] = {
            "samples": len(ev_ms), "mean_ms": round(float(np.mean(ev_ms)), 5),
            "p10_p90_ms": [round(float(np.percentile(ev_ms, 10)), 5), round(float(np.percentile(ev_ms, 90)), 5)]}

    if not args.no_fp16_baseline:
        result["fp16_baseline"] = fp16_baseline(torch, inp, kvq, lib, dev, stream, args, ms_per_step)

    if not args.no_workloads:
        result["other_workloads"] = [workload_bench(torch, inp, kvq, lib, dev, stream, args, name)
                                     for name in ("qwen3_4b_64k", "qwen3_30b_a3b_128k", "llama31_70b_128k")]

    if not args.no_multi_query:
        result["multi_query"] = multi_query_bench(torch, inp, kvq, lib, dev, stream, args, pools, bt, lens, n)

    if not args.no_mixed_window:
        result["mixed_window"] = mixed_window(torch, inp, kvq, lib, dev, stream, args)

    if not args.no_presets:
        legs = (("k4v4_g128", 16), ("k4v2_g128_pb", 16), ("k8v2_g128", 16), ("k8v4_g128", 16),
                ("k3v3_g128", 16), ("k4v2_g128", 32), ("k4v2_g128", 64), ("k4v2_g128", 128))
        if args.preset_list:
            legs = [(x.split(":")[0], int(x.split(":")[1]) if ":" in x else 16)
                    for x in args.preset_list.split(",")]
        result["presets"] = [preset_bench(torch, inp, kvq, lib, dev, stream, args, p, pt,
                                          ref=quality_ref if pt == 16 else None) for p, pt in legs]

    if not args.no_append_bench:
        result.update(append_bench(torch, inp, kvq, call, dev))

    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        result["cpu_baseline"] = cpu_baseline(w, threads, threads)

    print(json.dumps(result), flush=True)


def fp16_baseline(torch, inp, kvq, lib, dev, stream, args, k4v2_ms_per_step):
    """The same decode (8 x 16385 tokens, 64 / 8 heads) over the uncompressed
    fp16 cache: 512 bytes per token per KV head instead of 104.  Each step is
    the split kernel + the combine; the split kernel alone is then timed back
    to back between two events, as for K4V2."""
    import numpy as np
    w = inp.workload("qwen3_32b_16k")
    B, Hq, Hkv = w.num_seqs, w.num_q_heads, w.num_kv_heads
    n = w.context + 1
    f16 = kvq.format_from_string("fp16")
    bt_np, num_pages = inp.page_table(w)
    bt = torch.from_numpy(bt_np).to(dev)
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    base = torch.zeros((num_pages, Hkv, kvq.page_bytes(f16)), dtype=torch.uint8, device=dev)
    for b in range(B):
        k, v = inp.sequence_kv(w, b, 0, n, device=dev)
        kvq.quantize_append(k, v, torch.from_numpy(inp.slot_mapping(bt_np, b, 0, n)).to(dev), base, fmt=f16)
    pools = [base, base.clone()]          # 2 x 537 MB: no step finds its pool in the 256 MB cache
    q = inp.queries(w, 0, device=dev).contiguous()
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    ws = kvq.alloc_workspace(B, Hq, Hkv, n, fmt=f16)
    call = DecodeCall(kvq, lib, f16, stream.cuda_stream)
    part = [call.partials_args(q, p, bt, lens, n, ws, 0) for p in pools]
    comb = call.combine_args(out, lens, Hq, Hkv, n, ws, 0)
    pf, cfn = lib.kvq_decode_partials, lib.kvq_decode_combine
    steps = max(20, args.steps // 2)
    for i in range(5):
        pf(*part[i % 2]); cfn(*comb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if pf(*part[i % 2]) | cfn(*comb):
            raise RuntimeError("fp16 decode call failed")
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    hev = HipEvents(2)
    nl = max(1, args.kernel_launches // 2)
    bad = clock_warmup(pf, part, ms, args)
    hev.record(0, stream.cuda_stream)
    for i in range(nl):
        bad |= pf(*part[i % 2])
    hev.record(1, stream.cuda_stream)
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError("fp16 decode call failed")
    kern = hev.elapsed_ms(0, 1) / nl
    hev.close()
    fp16_bytes = B * n * Hkv * 512
    return {"workload": "qwen3_32b_16k, fp16 cache (512 B per token-head)", "ms_per_step": round(ms, 5),
            "split_kernel_ms": round(kern, 5),
            "kernel_GBps": round(fp16_bytes / (kern * 1e-3) / 1e9, 2),
            "kernel_pct_hbm_peak": round(100 * fp16_bytes / (kern * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "k4v2_step_speedup": round(ms / k4v2_ms_per_step, 3)}


def workload_bench(torch, inp, kvq, lib, dev, stream, args, name):
    """Decode (split kernel + combine, no append) over another workload's K4V2
    cache at full size, inputs resident in HBM; the split kernel alone is also
    timed back to back.  The Llama-shaped prompt is one sequence of 131072
    tokens; the others hold 4 x 131072 and 32 ragged sequences of 32K-64K."""
    import numpy as np
    w = inp.workload(name)
    B, Hq, Hkv = w.num_seqs, w.num_q_heads, w.num_kv_heads
    lens_np = inp.seq_lens(w)
    bt_np, num_pages = inp.page_table(w)
    fmt = kvq.format_from_string("k4v2_g128")
    cache = torch.zeros((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    for b in range(B):
        n = int(lens_np[b])
        for s0 in range(0, n, 32768):          # bounded chunks of generated fp16 rows
            cnt = min(32768, n - s0)
            k, v = inp.sequence_kv(w, b, s0, cnt, device=dev)
            kvq.quantize_append(k, v, torch.from_numpy(inp.slot_mapping(bt_np, b, s0, cnt)).to(dev), cache)
            del k, v
    pools = [cache]
    kv_bytes = int(lens_np.sum()) * Hkv * KV_BYTES_PER_TOKEN_HEAD
    if kv_bytes < 3 * (256 << 20):             # keep the pools beyond the 256 MB cache
        pools += [cache.clone() for _ in range(-(-3 * (256 << 20) // kv_bytes) - 1)]
    bt = torch.from_numpy(bt_np).to(dev)
    lens = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    q = inp.queries(w, 0, device=dev).contiguous()
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    ws = kvq.alloc_workspace(B, Hq, Hkv, L)
    call = DecodeCall(kvq, lib, fmt, stream.cuda_stream)
    part = [call.partials_args(q, p, bt, lens, L, ws, 0) for p in pools]
    comb = call.combine_args(out, lens, Hq, Hkv, L, ws, 0)
    pf, cfn = lib.kvq_decode_partials, lib.kvq_decode_combine
    for i in range(5):
        pf(*part[i % len(pools)]); cfn(*comb)
    torch.cuda.synchronize()
    steps = max(20, args.steps // 4)
    t0 = time.perf_counter()
    for i in range(steps):
        if pf(*part[i % len(pools)]) | cfn(*comb):
            raise RuntimeError(f"{name} decode failed")
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    hev = HipEvents(2)
    nl = max(1, args.kernel_launches // 4)
    bad = clock_warmup(pf, part, ms, args)
    hev.record(0, stream.cuda_stream)
    for i in range(nl):
        bad |= pf(*part[i % len(pools)])
    hev.record(1, stream.cuda_stream)
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError(f"{name} decode failed")
    kern = hev.elapsed_ms(0, 1) / nl
    hev.close()
    del pools, cache
    return {"workload": name, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "tokens": int(lens_np.sum()), "kv_bytes": kv_bytes, "ms_per_call": round(ms, 5),
            "call_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 2), "split_kernel_ms": round(kern, 5),
            "kernel_GBps": round(kv_bytes / (kern * 1e-3) / 1e9, 2),
            "kernel_pct_hbm_peak": round(100 * kv_bytes / (kern * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "pages_per_split": kvq.decode_pages_per_split(B, Hq, Hkv, L)}


def multi_query_bench(torch, inp, kvq, lib, dev, stream, args, pools, bt, lens, n):
    """kvq_decode_attention_mq (split kernel + combine) on the K4V2 cache of
    the main workload: q_len causal query rows per sequence, with the
    workload's 64 query heads (G = 8) and with 32 (G = 4, where two rows fill
    the 8-column MFMA group one row leaves half empty)."""
    import numpy as np
    B, Hkv = lens.numel(), pools[0].shape[1]
    fmt = kvq.format_from_string("k4v2_g128")
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    fn = lib.kvq_decode_attention_mq
    res = []
    rng = np.random.default_rng(20260605 + 77)
    for hq, m in ((64, 1), (64, 2), (64, 4), (32, 1), (32, 2)):
        q = torch.from_numpy(rng.standard_normal((B, m, hq, 128)).astype(np.float16)).to(dev)
        out = torch.empty((B, m, hq, 128), dtype=torch.float16, device=dev)
        wsb = kvq.decode_workspace_bytes_mq(B, m, hq, Hkv, n)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        argl = [(ctypes.byref(fmt), P(out.data_ptr()), 0, P(q.data_ptr()), i32(m), P(p.data_ptr()), i64(p.shape[0]),
                 P(bt.data_ptr()), i32(bt.shape[1]), P(lens.data_ptr()), i32(B), i32(hq), i32(Hkv), i32(n),
                 ctypes.c_float(1.0 / math.sqrt(128)), P(ws.data_ptr()), ctypes.c_size_t(wsb), i32(0),
                 P(stream.cuda_stream)) for p in pools]
        for i in range(5):
            fn(*argl[i % len(pools)])
        torch.cuda.synchronize()
        steps = max(20, args.steps // 2)
        t0 = time.perf_counter()
        for i in range(steps):
            if fn(*argl[i % len(pools)]):
                raise RuntimeError("multi-row decode failed")
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        kv_bytes = B * n * Hkv * KV_BYTES_PER_TOKEN_HEAD
        res.append({"num_q_heads": hq, "q_len": m, "ms_per_call": round(ms, 5),
                    "query_rows_per_s": round(B * m / (ms * 1e-3), 1),
                    "kv_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 2)})
    return res


def attention_reference(torch, inp, w, q, seqs):
    """Exact attention of the sampled sequences over their unquantised fp16
    keys and values (fp32 matmuls; a quality measure, not a timed step):
    {b: [Hq][128] float32}.  q: fp16 [B][Hq][128] on the device."""
    ref = {}
    n = w.context + 1
    G = w.num_q_heads // w.num_kv_heads
    for b in seqs:
        k, v = inp.sequence_kv(w, b, 0, n, device=q.device)
        kf = k.float().permute(1, 0, 2).contiguous()          # [Hkv][n][128]
        vf = v.float().permute(1, 0, 2).contiguous()
        qb = q[b].float().view(w.num_kv_heads, G, 128)
        p = torch.softmax(torch.matmul(qb, kf.transpose(1, 2).contiguous()) / math.sqrt(128), dim=-1)
        ref[b] = torch.matmul(p, vf).reshape(w.num_q_heads, 128)
        del k, v, kf, vf, p
    return ref


def rel_mse(out, ref):
    """sum |out - ref|^2 / sum |ref|^2 over the sampled sequences."""
    num = sum(float(((out[b].float() - r) ** 2).sum()) for b, r in ref.items())
    den = sum(float((r ** 2).sum()) for r in ref.values())
    return num / den


QUALITY_SEQS = (0, 5)


def preset_bench(torch, inp, kvq, lib, dev, stream, args, preset, page_tokens=16, ref=None):
    """The benchmark step (fused append + decode split kernel, then the
    combine) on the same workload with another preset's bit widths or page
    size; the split kernel alone is then timed back to back between two
    events.  Page-balanced keys take no fused append: every sequence's
    16385 tokens are written with its pages (whole-page blocks), and the
    step is the split kernel + combine.  With ref, the output's relative MSE
    against exact attention on the sampled sequences."""
    import numpy as np
    w = inp.workload("qwen3_32b_16k")
    B, Hq, Hkv = w.num_seqs, w.num_q_heads, w.num_kv_heads
    ctx, n = w.context, w.context + 1
    fmt = kvq.format_from_string(preset, page_tokens=page_tokens)
    balanced = fmt.key_norm == kvq.KEY_NORM_PAGE
    region = kvq.page_bytes(fmt)
    if page_tokens == 16:
        bt_np, num_pages = inp.page_table(w)
    else:        # a random permutation of pages of page_tokens tokens
        per_seq = -(-n // page_tokens)
        num_pages = B * per_seq
        perm = np.random.default_rng(20260605 + page_tokens).permutation(num_pages).astype(np.int32)
        bt_np = perm.reshape(B, per_seq)
    bt = torch.from_numpy(bt_np).to(dev)
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    base = torch.zeros((num_pages, Hkv, region), dtype=torch.uint8, device=dev)
    nk, nv = [], []
    for b in range(B):
        k, v = inp.sequence_kv(w, b, 0, n, device=dev)
        m = n if balanced else ctx
        t = np.arange(m)
        slots = bt_np[b, t // page_tokens].astype(np.int64) * page_tokens + t % page_tokens
        kvq.quantize_append(k[:m], v[:m], torch.from_numpy(slots).to(dev), base, fmt=fmt)
        nk.append(k[ctx:])
        nv.append(v[ctx:])
        del k, v
    nk, nv = torch.cat(nk).contiguous(), torch.cat(nv).contiguous()
    # copies cycled so that each launch reads a pool the 256 MB Infinity Cache
    # does not hold: at least 640 MB in all
    copies = max(3, -(-640_000_000 // base.numel()))
    pools = [base] + [base.clone() for _ in range(copies - 1)]
    q = inp.queries(w, 0, device=dev).contiguous()
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    ws = kvq.alloc_workspace(B, Hq, Hkv, n, fmt=fmt)
    call = DecodeCall(kvq, lib, fmt, stream.cuda_stream)
    if balanced:
        part = [call.partials_args(q, p, bt, lens, n, ws, 0) for p in pools]
        pf = lib.kvq_decode_partials
    else:
        part = [call.fused_args(nk, nv, q, p, bt, lens, n, ws, 0) for p in pools]
        pf = lib.kvq_append_decode_partials
    comb = call.combine_args(out, lens, Hq, Hkv, n, ws, 0)
    cfn = lib.kvq_decode_combine
    steps = max(20, args.steps // 2)
    for i in range(5):
        pf(*part[i % len(part)]); cfn(*comb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if pf(*part[i % len(part)]) | cfn(*comb):
            raise RuntimeError(f"{preset} decode call failed")
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    hev = HipEvents(2)
    nl = max(1, args.kernel_launches // 2)
    bad = clock_warmup(pf, part, ms, args)
    hev.record(0, stream.cuda_stream)
    for i in range(nl):
        bad |= pf(*part[i % len(part)])
    hev.record(1, stream.cuda_stream)
    torch.cuda.synchronize()
    if bad:
        raise RuntimeError(f"{preset} decode call failed")
    kern = hev.elapsed_ms(0, 1) / nl
    hev.close()
    quality = None
    if ref is not None:
        pf(*part[0])
        cfn(*comb)
        torch.cuda.synchronize()
        quality = rel_mse(out, ref)
    per_token_head = region // page_tokens       # bytes per (token, KV head)
    kv_bytes = B * n * Hkv * per_token_head
    del pools, base
    r = {"preset": preset, "page_tokens": page_tokens, "bytes_per_token_head": per_token_head,
         "ms_per_step": round(ms, 5),
         "step_GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 2), "split_kernel_ms": round(kern, 5),
         "kernel_GBps": round(kv_bytes / (kern * 1e-3) / 1e9, 2),
         "kernel_pct_hbm_peak": round(100 * kv_bytes / (kern * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
         "output_rel_mse": None if quality is None else float(f"{quality:.4e}")}
    if balanced:
        r["step"] = "decode split kernel + combine (the new token written with its page; no fused append)"
    return r


def mixed_window(torch, inp, kvq, lib, dev, stream, args, sink=4, recent=124):
    """The same decode with each sequence's first `sink` and last `recent`
    tokens uncompressed in an fp16 cache and the other 16257 in K4V2: K4V2
    partials, rotated fp16 partials, one combine (three launches per step)."""
    import numpy as np
    w = inp.workload("qwen3_32b_16k")
    B, Hq, Hkv = w.num_seqs, w.num_q_heads, w.num_kv_heads
    n = w.context + 1
    nf = sink + recent
    nh = n - nf
    f16 = kvq.format_from_string("fp16")
    k4 = kvq.format_from_string("k4v2_g128")
    bt_np, num_pages = inp.page_table(w)
    hp = -(-nh // 16)
    bt_h = torch.from_numpy(np.ascontiguousarray(bt_np[:, :hp])).to(dev)
    cache_h = torch.zeros((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    pf = -(-nf // 16)
    bt_f = torch.arange(B * pf, dtype=torch.int32, device=dev).view(B, pf)
    cache_f = torch.zeros((B * pf, Hkv, 8192), dtype=torch.uint8, device=dev)
    for b in range(B):
        k, v = inp.sequence_kv(w, b, 0, n, device=dev)
        kw = torch.cat([k[:sink], k[n - recent:]]).contiguous()
        vw = torch.cat([v[:sink], v[n - recent:]]).contiguous()
        kvq.quantize_append(kw, vw, torch.from_numpy(inp.slot_mapping(bt_f.cpu().numpy(), b, 0, nf)).to(dev),
                            cache_f, fmt=f16)
        kh, vh = k[sink:n - recent].contiguous(), v[sink:n - recent].contiguous()
        kvq.quantize_append(kh, vh, torch.from_numpy(inp.slot_mapping(bt_np, b, 0, nh)).to(dev), cache_h)
    pools = [cache_h] + [cache_h.clone() for _ in range(5)]
    q = inp.queries(w, 0, device=dev).contiguous()
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    lens_h = torch.full((B,), nh, dtype=torch.int32, device=dev)
    lens_f = torch.full((B,), nf, dtype=torch.int32, device=dev)
    s_h = kvq.decode_split_slots(B, Hq, Hkv, nh, fmt=k4)
    s_f = kvq.decode_split_slots(B, Hq, Hkv, nf, fmt=f16)
    total = s_h + s_f
    ws = torch.empty((kvq.slots_workspace_bytes(B, Hq, total),), dtype=torch.uint8, device=dev)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sc = ctypes.c_float(1.0 / math.sqrt(128))

    def part_args(fmt, cache, bt, lens, L, off):
        return (ctypes.byref(fmt), P(q.data_ptr()), P(cache.data_ptr()), i64(cache.shape[0]), P(bt.data_ptr()),
                i32(bt.shape[1]), P(lens.data_ptr()), i32(B), i32(Hq), i32(Hkv), i32(L), sc, P(ws.data_ptr()),
                ctypes.c_size_t(ws.numel()), i32(0), i32(off), i32(total), i32(1), P(stream.cuda_stream))
    ah = [part_args(k4, p, bt_h, lens_h, nh, 0) for p in pools]
    af = part_args(f16, cache_f, bt_f, lens_f, nf, s_h)
    ac = (P(out.data_ptr()), 0, i32(B), i32(Hq), P(ws.data_ptr()), ctypes.c_size_t(ws.numel()), i32(total), i32(1),
          P(stream.cuda_stream))
    fp, fc = lib.kvq_decode_partials_slots, lib.kvq_decode_combine_slots
    steps = max(20, args.steps)
    for i in range(10):
        fp(*ah[i % 6]); fp(*af); fc(*ac)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st = fp(*ah[i % 6]) | fp(*af) | fc(*ac)
        if st:
            raise RuntimeError("mixed-window decode failed")
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kv_bytes = B * Hkv * (nh * KV_BYTES_PER_TOKEN_HEAD + nf * 512)
    return {"workload": f"qwen3_32b_16k, {sink} sink + {recent} recent tokens fp16, {nh} K4V2",
            "ms_per_step": round(ms, 5), "GBps": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
            "kv_bytes": kv_bytes, "launches_per_step": 3}


APPEND_COUNTERS_FILE = os.path.join(ROOT, "profiles", "append_staged_llama31_70b_128k_counters.txt")
APPEND_SOURCES = [os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "csrc", f)
                  for f in ("kvq_append.hip", "kvq_device.h", "kvq_quant.h")] + \
                 [os.path.join(ROOT, "quantized_decode_attention_quantize_amd", "build.py")]
# MI355X vector ALU: 256 CUs x 4 SIMDs x 16 lanes, one 32-bit lane-op per lane per clock
# (fp32 add, mul, compare, integer, conversion) at 2.4 GHz
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def recorded_append_counters():
    """(fields, note) from the committed append counter summary, or (None,
    reason) when it is missing or the append sources changed since."""
    if not os.path.exists(APPEND_COUNTERS_FILE):
        return None, "no counter summary"
    rec = {}
    with open(APPEND_COUNTERS_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in APPEND_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    if rec.get("kernel_source_sha256") != h.hexdigest():
        return None, "kernel changed since the counters were taken"
    try:
        return {k: int(rec[k]) for k in ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                         "valu_instructions_per_launch")}, "rocprofv3 counters (scaled bytes)"
    except (KeyError, ValueError):
        return None, "malformed counter summary"


def append_bench(torch, inp, kvq, call, dev):
    """Bulk quantise-append of the Llama-3.1-70B-shaped 131072-token prompt
    (8 KV heads) in one call; tokens/s of the prompt.  Each of the timed
    launches is bracketed by HIP events on the launch stream; the headline is
    their mean, with the median and p10/p90 beside it (the encoder is
    ALU-heavy and the shader clock falls over a run of launches)."""
    import numpy as np
    w = inp.workload("llama31_70b_128k")
    T = w.context
    bt_np, num_pages = inp.page_table(w)
    k, v = inp.sequence_kv(w, 0, 0, T, device=dev)
    slots = torch.from_numpy(inp.slot_mapping(bt_np, 0, 0, T)).to(dev)
    cache = torch.zeros((num_pages, w.num_kv_heads, 1664), dtype=torch.uint8, device=dev)
    args = call.append_args(k, v, slots, cache)
    fn = kvq.load().kvq_quantize_append
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn(*args)
    reps = 20
    hev = HipEvents(2 * reps)
    torch.cuda.synchronize()
    for r in range(reps):
        hev.record(2 * r, stream.cuda_stream)
        if fn(*args):
            raise RuntimeError("kvq_quantize_append failed")
        hev.record(2 * r + 1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms_all = np.array([hev.elapsed_ms(2 * r, 2 * r + 1) for r in range(reps)])
    hev.close()
    ms = float(ms_all.mean())
    moved = T * w.num_kv_heads * APPEND_BYTES_PER_TOKEN_HEAD
    counters, note = recorded_append_counters()
    roof = {"kernel": "quantize_append_staged", "bound": "alu", "unit": "lane-op/s",
            "peak": VALU_PEAK_LANE_OPS, "achieved": None, "frac": None,
            "hbm_bytes_per_launch": moved, "hbm_GBps": round(moved / (ms * 1e-3) / 1e9, 2),
            "hbm_frac": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None, "counters_note": note}
    if counters:
        lane_ops = counters["valu_instructions_per_launch"] * 64
        roof.update({"valu_instructions_per_launch": counters["valu_instructions_per_launch"],
                     "achieved": round(lane_ops / (ms * 1e-3), 1),
                     "frac": round(lane_ops / (ms * 1e-3) / VALU_PEAK_LANE_OPS, 4),
                     "traffic": counters["fetch_bytes_per_launch"] + counters["write_bytes_per_launch"]})
    return {"append_tokens_per_s": round(T / (ms * 1e-3), 1),
            "append_config": {"workload": "llama31_70b_128k prefill", "tokens": T,
                              "num_kv_heads": w.num_kv_heads, "kernel_ms": round(ms, 5),
                              "kernel_ms_median": round(float(np.median(ms_all)), 5),
                              "kernel_ms_p10": round(float(np.percentile(ms_all, 10)), 5),
                              "kernel_ms_p90": round(float(np.percentile(ms_all, 90)), 5),
                              "launches": reps,
                              "GBps": round(moved / (ms * 1e-3) / 1e9, 2),
                              "pct_hbm_peak": round(100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                              "roofline": roof}}


if __name__ == "__main__":
    main()
