#!/usr/bin/env python3
"""Benchmark: NVFP4 paged decode attention on one MI355X -- effective KV GB/s (% of HBM peak) + tokens/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config long|batch32|ragged|mixed|extend|prefill|write|gather|tiny|sweep]

One step is one decode step of the workload's hot path, inputs already resident in HBM:
  long     split-K NVFP4 decode + log-sum-exp merge, 4 x 131072 tokens, 8 KV / 64 query heads (default);
           two cache copies (1.2 GB) rotate, so no step reads a cache the previous step read
  batch32  same path, 32 x 4096 tokens, 8 / 32 heads; three cache copies rotate so that every
           step reads a cache not touched by the previous two (the 256 MB last-level cache holds one)
  ragged   64 ragged sequences, fused quantize-append of one token per sequence + decode (two
           cache copies rotate)
  mixed    28 layers, FP8 at layers 0, 25, 26, 27 and NVFP4 elsewhere, 44 x 8192 tokens
  extend   per NVFP4 layer of the mixed stack: 16384-token prefix -> FP8 workspace + 2048-token
           chunk quantize-append (24 layers per step)
  prefill  per NVFP4 layer: one-pass NVFP4 cache + FP8 copy write of a prompt and causal attention
           over the copy
  write    quantize-on-write of the ragged batch's whole cache (512,723 tokens x 8 kv heads, bf16 K
           and V) into a fresh NVFP4 pool; the per-tensor scale reduction is timed apart
  gather   the extend path's prefix gather alone: one NVFP4 layer's 16384-token prefix -> FP8 workspace
  tiny     1 x 256 tokens (latency-bound)
  sweep    precision studies (per-layer NVFP4 vs FP8 sensitivity, per-tensor scale variants)

The timed region is exactly K steps between two device synchronisations, with nothing else in it.
Right after it, the dominant kernel is timed on its own: for decode, 40 more steps whose split
kernel's dispatch records a HIP event pair (the long workload rotates two cache copies, batch32
three); for extend and prefill, the attention launches of two more steps between events on the
launch stream.  Effective KV GB/s =
NVFP4 (or FP8) bytes the step must read (144 B per token and KV head; 256 B for FP8) / step time.
The CPU baseline times the fp64 oracle (one thread per worker) on a bounded sample of the same
workload: dequantize + attention for the decode configs and the mixed stack (each layer in its
precision), the whole per-(layer, kv head) pipeline for extend, and for prefill the prompt's write
plus a block of query rows whose attention time is scaled to the whole prompt by its flop ratio.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16 matrix-core peak of MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="long", choices=["long", "batch32", "ragged", "mixed", "extend", "prefill",
                                                         "write", "gather", "tiny", "sweep"])
    ap.add_argument("--pages-per-split", type=int, default=0, help="force the split size (0 = planner)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000     # hipEventDisableSystemFence (hip_runtime_api.h)


class HipEventPairs:
    """K pairs of raw hipEvent_t from the HIP runtime the library runs on (timing plumbing only)."""

    def __init__(self, n):
        import ctypes
        self._ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")       # the runtime torch has already loaded
        self.start = [ctypes.c_void_p() for _ in range(n)]
        self.stop = [ctypes.c_void_p() for _ in range(n)]
        # timing-only events: no system-scope fence (cache writeback and invalidation) when they are
        # recorded, which would otherwise lengthen the bracketed kernel and the work after it
        for e in self.start + self.stop:
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, i, which, stream):
        """hipEventRecord of start (which == 0) or stop event i on the raw stream handle."""
        ev = (self.start if which == 0 else self.stop)[i]
        if self.hip.hipEventRecord(ev, self._ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self):
        ms = self._ct.c_float()
        out = []
        for a, b in zip(self.start, self.stop):
            if self.hip.hipEventSynchronize(b) != 0 or self.hip.hipEventElapsedTime(self._ct.byref(ms), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for e in self.start + self.stop:
            self.hip.hipEventDestroy(e)


KERNEL_SAMPLES = 40    # decode configs: launches timed one by one after the headline loop

# Worker processes of the CPU baseline: one per core of the process's affinity set, at most 16 --
# the host-CPU share one GPU gets on the machines the benchmark runs on (a pool wider than that
# share would be time-sliced, not faster).
CPU_WORKER_CAP = 16


def host_cpu():
    """CPU model (from /proc/cpuinfo), cores in the affinity set, and the worker count used."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0))
    return {"model": model, "affinity_cores": avail, "workers": max(1, min(avail, CPU_WORKER_CAP)),
            "worker_cap": CPU_WORKER_CAP,
            "cap_reason": "one spawned worker per affinity core, at most 16: the host-CPU share of one GPU"}

# HBM traffic of one decode step (one decode_split_kernel launch, merge included) on the long workload, from
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch, one counter per run) scaled by
# the factors a plain 1 GiB device copy gives (x2.000 / x1.000).  Valid only for the kernel sources
# (the decode file and the headers it includes, hashed together) and the split plan they were taken
# with; reported as null otherwise.
TRAFFIC = {
    "long": {"source_sha256": "fee6281dd19eaf7d4fa29e105df3dff8e37ae6031ca0c2b3352b6b397c023ed5", "plan": [2, 512],
             "kernels": {"decode_split_kernel": (296438.7, 4304.0)},
             "fetch_factor": 2.0, "write_factor": 1.0},
}


DECODE_SOURCES = ("nvkv_decode.hip", "nvkv_device.h", "nvkv_launch.h")


def decode_source_sha256():
    """sha256 over the decode kernel's sources, concatenated in DECODE_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_paged_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stream_read_ceiling(nv, nbytes, dev, reps=20):
    """Streaming-read rate of the device in GB/s: the library's read probe (coalesced 16-byte loads
    over the whole GPU) on a buffer of max(nbytes, 768 MiB) -- larger than the 256 MB last-level
    cache -- timed with events on the launch stream around each of `reps` launches."""
    import torch
    n = max(int(nbytes), 768 << 20) // 16 * 16
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)     # every 16-byte chunk folds to 0
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(5):
        nv.read_probe(buf, sink)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in pairs:
        e0.record()
        nv.read_probe(buf, sink)
        e1.record()
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in pairs) / reps
    del buf
    return {"value": round(n / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "bytes": n, "us_per_read": round(ms * 1e3, 2),
            "method": f"nvkv_read_probe, mean of {reps} launches"}


# ------------------------------------------------------------------------------------------------
def build_layer_cache(nv, wl, layer, dev, fp8=False):
    """Upload one layer's cached K/V and write it into a new pool with the library's kernels."""
    import torch
    from bit_paged_kv_amd import paged
    k = torch.cat([wl.kv("k", b, layer) for b in range(wl.batch)]).to(dev)
    v = torch.cat([wl.kv("v", b, layer) for b in range(wl.batch)]).to(dev)
    slots = torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(dev)
    if fp8:
        pool, s1, s2 = paged.build_fp8_cache(k, v, slots, wl.num_pages)
    else:
        pool, s1, s2 = paged.build_nvfp4_cache(k, v, slots, wl.num_pages)
    del k, v
    return pool, s1, s2


def _cpu_units(args):
    """One pool worker: the oracle's decode (fp64 dequantize + attention, one thread) on the given
    (sequence, kv head) units; returns (KV bytes, seconds spent in the oracle)."""
    cfg_index, units, budget_s = args
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import attention as o_att
    from oracle import nvfp4 as o_nv
    wl = workloads.config(cfg_index)
    g = wl.group
    q = wl.q().float().numpy()
    done_bytes, spent = 0, 0.0
    with threadpool_limits(limits=1):
        for b, hks in units:
            k = wl.kv("k", b).float().numpy()
            v = wl.kv("v", b).float().numpy()
            gk = o_nv.global_scale(k)
            gv = o_nv.global_scale(v)
            for hk in hks:
                ck, sk = o_nv.quantize_blocks(k[:, hk], gk)      # cache contents (not timed)
                cv, sv = o_nv.quantize_blocks(v[:, hk], gv)
                t0 = time.perf_counter()
                kh = o_nv.dequantize_blocks(ck, sk, gk)[:, None]
                vh = o_nv.dequantize_blocks(cv, sv, gv)[:, None]
                o_att.decode_attention_one(q[b, hk * g:(hk + 1) * g], kh, vh, wl.sm_scale)
                spent += time.perf_counter() - t0
                done_bytes += k.shape[0] * 144
                if spent >= budget_s:
                    return done_bytes, spent
    return done_bytes, spent


def cpu_baseline(cfg_index, budget_s=6.0):
    """Time the oracle's decode on (sequence, kv head) units of the workload, one unit list per host
    core (a process pool of fresh interpreters, at most 16; each regenerates its sequences from the
    seeded generator, untimed), each worker stopping after ~budget_s of oracle time; returns the
    summed per-worker KV GB/s."""
    import multiprocessing as mp

    import workloads
    wl = workloads.config(cfg_index)
    cores = max(1, min(host_cpu()["workers"], wl.batch * wl.h_kv))
    all_units = [(b, hk) for b in range(wl.batch) for hk in range(wl.h_kv)]
    jobs = []
    n = len(all_units)
    for w in range(cores):
        mine = all_units[w * n // cores:(w + 1) * n // cores]    # contiguous: few sequences per worker
        by_seq = {}
        for b, hk in mine:
            by_seq.setdefault(b, []).append(hk)
        jobs.append((cfg_index, sorted(by_seq.items()), budget_s))
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_cpu_units, jobs)
    total = sum(r[0] for r in res)
    rate = sum(r[0] / r[1] for r in res if r[1] > 0)
    spent = sum(r[1] for r in res)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{total} KV bytes of (sequence, kv head) units of {int(wl.seq_lens.min())}..{int(wl.seq_lens.max())}-token sequences "
                      f"(fp64 dequantize + softmax attention for {wl.group} query heads each), {spent:.1f} s of oracle "
                      f"time over {cores} single-threaded workers; rate summed over workers; host "
                      f"{host_cpu()['model']}", "host": host_cpu()}


def _cpu_mixed_units(args):
    """One pool worker, 28-layer stack: the oracle's decode of (layer, sequence) units over all kv
    heads, each layer in its own precision (NVFP4: dequantize blocks; FP8: dequantize E4M3 x s);
    returns (KV bytes, seconds spent in the oracle)."""
    cfg_index, units, budget_s = args
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import attention as o_att
    from oracle import fp8 as o_fp8
    from oracle import nvfp4 as o_nv
    wl = workloads.config(cfg_index)
    g = wl.group
    qs = {}
    done_bytes, spent = 0, 0.0
    with threadpool_limits(limits=1):
        for layer, b in units:
            if layer not in qs:
                qs[layer] = wl.q(layer).float().numpy()
            q = qs[layer][b]
            k = wl.kv("k", b, layer).float().numpy()
            v = wl.kv("v", b, layer).float().numpy()
            fp8 = wl.is_fp8(layer)
            if fp8:                                   # cache contents (not timed); scales of this sequence
                sk, sv = o_fp8.fp8_scale(k), o_fp8.fp8_scale(v)
                ck, cv = o_fp8.fp8_quantize(k, sk), o_fp8.fp8_quantize(v, sv)
            else:
                gk, gv = o_nv.global_scale(k), o_nv.global_scale(v)
            for hk in range(wl.h_kv):
                if not fp8:
                    nk, nsk = o_nv.quantize_blocks(k[:, hk], gk)
                    nvv, nsv = o_nv.quantize_blocks(v[:, hk], gv)
                t0 = time.perf_counter()
                if fp8:
                    kh = o_fp8.fp8_dequantize(ck[:, hk], sk)[:, None]
                    vh = o_fp8.fp8_dequantize(cv[:, hk], sv)[:, None]
                else:
                    kh = o_nv.dequantize_blocks(nk, nsk, gk)[:, None]
                    vh = o_nv.dequantize_blocks(nvv, nsv, gv)[:, None]
                o_att.decode_attention_one(q[hk * g:(hk + 1) * g], kh, vh, wl.sm_scale)
                spent += time.perf_counter() - t0
                done_bytes += k.shape[0] * (256 if fp8 else 144)
                if spent >= budget_s:
                    return done_bytes, spent
    return done_bytes, spent


def _cpu_extend_units(args):
    """One pool worker, extend or prefill of the stack's NVFP4 layers: the oracle's pipeline for
    (layer, kv head) units with the head's query group; returns (step bytes, seconds of oracle time
    for the whole unit, attention flops of the whole unit, seconds measured).

    extend: NVFP4 prefix -> FP8 workspace, chunk -> FP8 rows after it, causal attention of the
    2048-row chunk over prefix || chunk, chunk -> NVFP4; all timed.
    prefill: the prompt -> NVFP4 and the FP8 copy (timed), then causal attention of a block of
    `rows` query rows whose mean visible-key count equals the prompt's (timed); the whole prompt's
    attention time is that block's time scaled by the flop ratio."""
    cfg_index, mode, units, budget_s, rows = args
    import torch
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import attention as o_att
    from oracle import fp8 as o_fp8
    from oracle import nvfp4 as o_nv
    wl = workloads.config(cfg_index)
    g = wl.group
    prefix, chunk = wl.extend_prefix, wl.extend_chunk
    if mode == "extend":
        ext = workloads.Workload(name="extend", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                                 seq_lens=[prefix + chunk], chan=wl.chan)
        gen = torch.Generator().manual_seed(wl.seed * 7 + 5)
        q_all = torch.randn((chunk, wl.h_q, 128), generator=gen).to(torch.bfloat16).float().numpy()
    else:
        ext = workloads.Workload(name="prefill", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                                 seq_lens=[prefix], chan=wl.chan)
        gen = torch.Generator().manual_seed(wl.seed * 7 + 6)
        q_all = torch.randn((prefix, wl.h_q, 128), generator=gen).to(torch.bfloat16).float().numpy()
    done_bytes, est, flops, spent = 0, 0.0, 0, 0.0
    cur = None
    with threadpool_limits(limits=1):
        for layer, hk in units:
            if cur is None or cur[0] != layer:
                k = ext.kv("k", 0, layer, length=prefix).float().numpy()
                v = ext.kv("v", 0, layer, length=prefix).float().numpy()
                cur = (layer, k, v, o_nv.global_scale(k), o_nv.global_scale(v))
            _, k, v, gk, gv = cur
            s_wk, s_wv = np.float32(6.0 * gk), np.float32(6.0 * gv)
            qg = q_all[:, hk * g:(hk + 1) * g]
            if mode == "extend":
                ck = wl.chunk("k", layer).float().numpy()[:, hk]
                cv = wl.chunk("v", layer).float().numpy()[:, hk]
                pk, psk = o_nv.quantize_blocks(k[:, hk], gk)          # the cached prefix (not timed)
                pv, psv = o_nv.quantize_blocks(v[:, hk], gv)
                t0 = time.perf_counter()
                wk = np.concatenate([o_fp8.nvfp4_to_fp8_workspace(pk, psk, gk, s_wk), o_fp8.fp8_quantize(ck, s_wk)])
                wv = np.concatenate([o_fp8.nvfp4_to_fp8_workspace(pv, psv, gv, s_wv), o_fp8.fp8_quantize(cv, s_wv)])
                o_att.extend_attention_one(qg, o_fp8.fp8_dequantize(wk, s_wk)[:, None],
                                           o_fp8.fp8_dequantize(wv, s_wv)[:, None], prefix, wl.sm_scale)
                o_nv.quantize_blocks(ck, gk)
                o_nv.quantize_blocks(cv, gv)
                dt = time.perf_counter() - t0
                spent += dt
                est += dt
                done_bytes += prefix * (144 + 256) + chunk * (512 + 144)
                flops += 4 * 128 * g * (chunk * prefix + chunk * (chunk + 1) // 2)
            else:
                n = prefix
                t0 = time.perf_counter()
                o_nv.quantize_blocks(k[:, hk], gk)
                o_nv.quantize_blocks(v[:, hk], gv)
                wk, wv = o_fp8.fp8_quantize(k[:, hk], s_wk), o_fp8.fp8_quantize(v[:, hk], s_wv)
                t1 = time.perf_counter()
                r0 = (n - rows) // 2
                o_att.extend_attention_one(qg[r0:r0 + rows], o_fp8.fp8_dequantize(wk[:r0 + rows], s_wk)[:, None],
                                           o_fp8.fp8_dequantize(wv[:r0 + rows], s_wv)[:, None], r0, wl.sm_scale)
                t2 = time.perf_counter()
                full = n * (n + 1) // 2
                sample = rows * r0 + rows * (rows + 1) // 2
                spent += t2 - t0
                est += (t1 - t0) + (t2 - t1) * full / sample
                done_bytes += n * (512 + 144 + 256)
                flops += 4 * 128 * g * full
            if spent >= budget_s:
                break
    return done_bytes, est, flops, spent


def _cpu_write_units(args):
    """One pool worker, quantize-on-write: the oracle's NVFP4 block quantizer (fp32, one thread) on
    (sequence, kv head) units' K and V; returns (bytes as the kernel counts them, seconds)."""
    cfg_index, units, budget_s = args
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import nvfp4 as o_nv
    wl = workloads.config(cfg_index)
    done_bytes, spent = 0, 0.0
    with threadpool_limits(limits=1):
        for b, hks in units:
            k = wl.kv("k", b).float().numpy()
            v = wl.kv("v", b).float().numpy()
            gk, gv = o_nv.global_scale(k), o_nv.global_scale(v)      # this sequence's scales (not timed)
            for hk in hks:
                t0 = time.perf_counter()
                o_nv.quantize_blocks(k[:, hk], gk)
                o_nv.quantize_blocks(v[:, hk], gv)
                spent += time.perf_counter() - t0
                done_bytes += k.shape[0] * (512 + 144)
                if spent >= budget_s:
                    return done_bytes, spent
    return done_bytes, spent


def cpu_baseline_write(cfg_index, budget_s=6.0):
    """The oracle's quantizer timed on (sequence, kv head) units of the workload's cache, one unit list
    per host core (at most 16 spawned workers, ~budget_s of oracle time each); summed GB/s."""
    import multiprocessing as mp

    import workloads
    wl = workloads.config(cfg_index)
    cores = host_cpu()["workers"]
    # units spread over the batch so that every worker sees long and short sequences
    all_units = [(b, hk) for hk in range(wl.h_kv) for b in range(wl.batch)]
    jobs = []
    for w in range(cores):
        by_seq = {}
        for b, hk in all_units[w::cores]:
            by_seq.setdefault(b, []).append(hk)
        jobs.append((cfg_index, sorted(by_seq.items()), budget_s))
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_cpu_write_units, jobs)
    total = sum(r[0] for r in res)
    rate = sum(r[0] / r[1] for r in res if r[1] > 0)
    spent = sum(r[1] for r in res)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{total} bytes (bf16 K+V read, NVFP4 written) of (sequence, kv head) units of the ragged "
                      f"cache (fp32 NVFP4 block quantizer of K and V; scales of the unit's sequence), {spent:.1f} s of "
                      f"oracle time over {cores} single-threaded workers; rate summed over workers; host "
                      f"{host_cpu()['model']}", "host": host_cpu()}


def _cpu_gather_units(args):
    """One pool worker, prefix gather: the oracle's NVFP4 -> FP8 workspace transcode of K and V on
    (layer, kv head) units of the extend prefix; returns (bytes as the kernel counts them, seconds)."""
    cfg_index, units, budget_s = args
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import fp8 as o_fp8
    from oracle import nvfp4 as o_nv
    wl = workloads.config(cfg_index)
    prefix = wl.extend_prefix
    ext = workloads.Workload(name="extend", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                             seq_lens=[prefix + wl.extend_chunk], chan=wl.chan)
    done_bytes, spent, cur = 0, 0.0, None
    with threadpool_limits(limits=1):
        for layer, hk in units:
            if cur is None or cur[0] != layer:
                k = ext.kv("k", 0, layer, length=prefix).float().numpy()
                v = ext.kv("v", 0, layer, length=prefix).float().numpy()
                cur = (layer, k, v, o_nv.global_scale(k), o_nv.global_scale(v))
            _, k, v, gk, gv = cur
            ck, sk = o_nv.quantize_blocks(k[:, hk], gk)              # the cached prefix (not timed)
            cv, sv = o_nv.quantize_blocks(v[:, hk], gv)
            t0 = time.perf_counter()
            o_fp8.nvfp4_to_fp8_workspace(ck, sk, gk, np.float32(6.0 * gk))
            o_fp8.nvfp4_to_fp8_workspace(cv, sv, gv, np.float32(6.0 * gv))
            spent += time.perf_counter() - t0
            done_bytes += prefix * (144 + 256)
            if spent >= budget_s:
                break
    return done_bytes, spent


def cpu_baseline_gather(cfg_index, budget_s=6.0):
    """The oracle's prefix transcode timed on (layer, kv head) units, one unit list per host core (at
    most 16 spawned workers, ~budget_s of oracle time each); summed GB/s."""
    import multiprocessing as mp

    import workloads
    wl = workloads.config(cfg_index)
    cores = host_cpu()["workers"]
    all_units = [(layer, hk) for layer in range(wl.layers) if not wl.is_fp8(layer) for hk in range(wl.h_kv)]
    n = len(all_units)
    jobs = [(cfg_index, all_units[w * n // cores:(w + 1) * n // cores], budget_s) for w in range(cores)]
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_cpu_gather_units, jobs)
    total = sum(r[0] for r in res)
    rate = sum(r[0] / r[1] for r in res if r[1] > 0)
    spent = sum(r[1] for r in res)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{total} bytes (NVFP4 read, FP8 written) of (layer, kv head) units of the 16384-token extend "
                      f"prefix (fp32 transcode of K and V), {spent:.1f} s of oracle time over {cores} single-threaded "
                      f"workers; rate summed over workers; host {host_cpu()['model']}", "host": host_cpu()}


def cpu_baseline_stack(cfg_index, mode, budget_s=6.0, rows=1024):
    """The oracle timed on the mixed stack (mode "mixed", KV GB/s) or on the extend / prefill step of
    its NVFP4 layers (step GB/s, plus the oracle's attention TFLOP/s), one unit list per host core
    (at most 16 spawned workers, each stopping after ~budget_s of oracle time)."""
    import multiprocessing as mp

    import workloads
    wl = workloads.config(cfg_index)
    cores = host_cpu()["workers"]
    if mode == "mixed":
        all_units = [(layer, b) for b in range(wl.batch) for layer in range(wl.layers)]
    else:
        all_units = [(layer, hk) for layer in range(wl.layers) if not wl.is_fp8(layer) for hk in range(wl.h_kv)]
    jobs = []
    n = len(all_units)
    for w in range(cores):
        mine = all_units[w * n // cores:(w + 1) * n // cores]
        jobs.append((cfg_index, mine, budget_s) if mode == "mixed" else (cfg_index, mode, mine, budget_s, rows))
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_cpu_mixed_units if mode == "mixed" else _cpu_extend_units, jobs)
    host = host_cpu()["model"]
    if mode == "mixed":
        total = sum(r[0] for r in res)
        rate = sum(r[0] / r[1] for r in res if r[1] > 0)
        spent = sum(r[1] for r in res)
        return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{total} KV bytes of (layer, sequence) units taken in layer order per sequence (each "
                          f"layer in its own precision, FP8 scales of the unit's sequence; fp64 dequantize + "
                          f"softmax attention over 8 kv heads), {spent:.1f} s of oracle time over {cores} "
                          f"single-threaded workers; rate summed over workers; host {host}", "host": host_cpu()}
    total = sum(r[0] for r in res)
    rate = sum(r[0] / r[1] for r in res if r[1] > 0)
    tflops = sum(r[2] / r[1] for r in res if r[1] > 0) / 1e12
    spent = sum(r[3] for r in res)
    what = ("the whole per-(layer, kv head) pipeline: prefix gather to FP8, chunk append, causal attention of "
            "2048 chunk rows x 4 query heads over 18432 keys, chunk quantize-append" if mode == "extend" else
            f"the prompt's NVFP4 + FP8 write, then causal attention of {rows} query rows x 4 query heads whose "
            f"mean key count is the prompt's, the whole prompt's attention time taken as that block's time x the "
            f"flop ratio")
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "attention_tflops": round(tflops, 6),
            "sample": f"{total} step bytes of (layer, kv head) units ({what}; fp64), {spent:.1f} s of oracle "
                      f"time over {cores} single-threaded workers; rate summed over workers; host {host}",
            "host": host_cpu()}


# ------------------------------------------------------------------------------------------------
def precision_studies(nv, workloads, dev):
    """The per-layer NVFP4-vs-FP8 sensitivity sweep over the 28-layer stack's synthetic K/V (batch 4
    x 8192 tokens, the stack's per-layer channel scales and outlier channels), and the per-tensor
    scale variants on one layer; prints one JSON line."""
    import torch
    import studies as analysis
    base = workloads.config(4)
    wl = workloads.Workload(name="sweep", seed=base.seed, batch=4, h_kv=base.h_kv, h_q=base.h_q,
                            seq_lens=[8192] * 4, chan=base.chan, layers=base.layers, fp8_layers=base.fp8_layers)
    pt = torch.from_numpy(wl.page_table).to(dev)
    sl = torch.from_numpy(wl.total_lens.astype(np.int32)).to(dev)
    slots = torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(dev)
    t0 = time.perf_counter()
    rows = []
    for layer in range(wl.layers):
        k = torch.cat([wl.kv("k", b, layer) for b in range(wl.batch)]).to(dev)
        v = torch.cat([wl.kv("v", b, layer) for b in range(wl.batch)]).to(dev)
        L = {"q": wl.q(layer).to(dev), "k": k, "v": v}
        r = analysis.layer_sensitivity([L], slots, wl.num_pages, pt, sl, wl.sm_scale, wl.h_kv)[0]
        r["layer"] = layer
        rows.append(r)
        if layer == 1:
            variants = analysis.gscale_variants(L["q"], k, v, slots, wl.num_pages, pt, sl, wl.sm_scale, wl.h_kv,
                                                calib_tokens=1024)
        log(f"layer {layer}: NVFP4 vs FP8 rel-L2 {r['nvfp4_vs_fp8']['rel_l2']:.3e}, {time.perf_counter() - t0:.1f} s")
    order = sorted(range(len(rows)), key=lambda i: -rows[i]["nvfp4_vs_bf16"]["rel_l2"])
    print(json.dumps({"study": "per-layer NVFP4 sensitivity and per-tensor scale variants",
                      "data": "synthetic (seeded; 28-layer stack's per-layer channel scales, batch 4 x 8192)",
                      "layers": rows, "most_sensitive_first": order, "gscale_variants_layer1": variants}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the library has no multi-GPU path, "
                                   "so --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import bit_paged_kv_amd as nv
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.config
    if name == "sweep":
        precision_studies(nv, workloads, dev)
        return
    index = {"tiny": 0, "batch32": 1, "long": 2, "ragged": 3, "write": 3, "mixed": 4, "extend": 4, "prefill": 4,
             "gather": 4}[name]
    wl = workloads.config(index)
    stream = torch.cuda.current_stream(dev)
    t_setup = time.perf_counter()

    # ---- build the step ------------------------------------------------------------------------
    att_flops = 0            # extend: attention flops per launch
    if name in ("long", "batch32", "tiny", "ragged"):
        # copies rotate so that no step reads a pool the 256 MB last-level cache may still hold
        copies = 3 if name in ("batch32", "tiny") else 2
        pools = []
        for c in range(copies):
            pool, gk, gv = build_layer_cache(nv, wl, 0, dev)
            pools.append(pool)
        log(f"cache built in {time.perf_counter() - t_setup:.1f} s ({copies} copies)")
        pt = torch.from_numpy(wl.page_table).to(dev)
        sl = torch.from_numpy(wl.total_lens.astype(np.int32)).to(dev)
        plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()),
                              args.pages_per_split)
        q = wl.q().to(dev)
        out = torch.empty((wl.batch, wl.h_q, 128), dtype=torch.float32, device=dev)
        ws = nv.alloc_decode_workspace(wl.batch, wl.h_q, wl.h_kv, plan[1], dev)
        new_k = wl.new_token("k").to(dev) if wl.append else None
        new_v = wl.new_token("v").to(dev) if wl.append else None
        step_bytes = wl.kv_bytes_nvfp4()
        calls = [nv.prepare_nvfp4_decode(q, pool, gk, gv, pt, sl, wl.sm_scale, plan, wl.h_kv, new_k=new_k,
                                         new_v=new_v, out=out, workspace=ws)[0] for pool in pools]
        counter = [0]

        def step(events=None, i=0):
            call = calls[counter[0] % len(calls)]
            if events is None:
                call.run()
            else:
                call.run_timed(events.start[i], events.stop[i])
            counter[0] += 1
        timed_kernel = "decode_split_kernel<PageNv4>"
        kernel_bytes = step_bytes
        desc = (f"{name}: batch {wl.batch}, context {int(wl.seq_lens[0]) if name != 'ragged' else 'ragged'}, "
                f"{wl.h_kv} KV / {wl.h_q} query heads, head_dim 128, page 16, NVFP4 cache, "
                f"{plan[1]} pieces of equal cost (at least {plan[0]} pages; paired 9:7 per compute unit when the "
                f"lengths are equal), split streams merged in-kernel")
        extra = {"batch": wl.batch, "context_tokens": int(wl.total_lens.sum()), "kv_heads": wl.h_kv,
                 "q_heads": wl.h_q, "head_dim": 128, "page_size": 16, "cache": "nvfp4",
                 "pages_per_split": plan[0], "num_splits": plan[1], "cache_copies_rotated": copies,
                 "fused_append": bool(wl.append)}
        tokens_per_step = wl.batch
    elif name == "write":
        # quantize-on-write of a whole cache: the ragged batch's 512,723 cached tokens x 8 kv heads,
        # bf16 K and V, into a fresh NVFP4 pool at the page table's slots (misaligned sequence starts);
        # the per-tensor scales are computed once beforehand, as a prefill would
        k, v, slots = (torch.cat([wl.kv("k", b) for b in range(wl.batch)]).to(dev),
                       torch.cat([wl.kv("v", b) for b in range(wl.batch)]).to(dev),
                       torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(dev))
        n_tok = k.shape[0]
        g_k, g_v = nv.global_scale(k), nv.global_scale(v)
        gk, gv = float(g_k.item()), float(g_v.item())
        pool = nv.alloc_nvfp4_pool(wl.num_pages, wl.h_kv, dev)
        call = nv.prepare_nvfp4_quantize_append(k, v, slots, gk, gv, pool)
        log(f"write inputs ready in {time.perf_counter() - t_setup:.1f} s")

        def step(events=None, i=0):
            call.run()
        # reads 2 x 256 B of bf16 and writes 2 x 72 B per (token, kv head)
        step_bytes = n_tok * wl.h_kv * (512 + 144)
        timed_kernel = None
        kernel_bytes = None
        desc = (f"write: NVFP4 quantize-on-write of {n_tok} tokens x {wl.h_kv} kv heads (the ragged batch's cache, "
                f"bf16 K and V) into a paged pool")
        extra = {"tokens": n_tok, "kv_heads": wl.h_kv, "head_dim": 128, "page_size": 16, "sequences": wl.batch}
        tokens_per_step = n_tok
    elif name == "gather":
        # the extend path's prefix gather alone: one NVFP4 layer's 16384-token prefix (8 kv heads, a
        # permuted page table) transcoded into the dense FP8 workspace, one launch per step
        layer = next(l for l in range(wl.layers) if not wl.is_fp8(l))
        prefix = wl.extend_prefix
        ext = workloads.Workload(name="extend", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                                 seq_lens=[prefix + wl.extend_chunk], chan=wl.chan)
        from bit_paged_kv_amd import paged
        slots = torch.from_numpy(ext.slots(0, 0, prefix)).to(dev)
        pool, gk_l, gv_l = paged.build_nvfp4_cache(ext.kv("k", 0, layer, length=prefix).to(dev),
                                                   ext.kv("v", 0, layer, length=prefix).to(dev), slots, ext.num_pages)
        pt = torch.from_numpy(ext.page_table).to(dev)
        prefix_lens = torch.tensor([prefix], dtype=torch.int32, device=dev)
        offs = torch.tensor([0, prefix], dtype=torch.int32, device=dev)
        k_ws = torch.empty((prefix, wl.h_kv, 128), dtype=torch.uint8, device=dev)
        v_ws = torch.empty_like(k_ws)
        call = nv.prepare_dequant_to_workspace(pool, gk_l, gv_l, pt, prefix_lens, offs, prefix, 6.0 * gk_l,
                                               6.0 * gv_l, wl.h_kv, k_ws, v_ws)
        log(f"gather inputs ready in {time.perf_counter() - t_setup:.1f} s")

        def step(events=None, i=0):
            call.run()
        # reads 2 x 72 B of NVFP4 and writes 2 x 128 B of FP8 per (token, kv head)
        step_bytes = prefix * wl.h_kv * (144 + 256)
        timed_kernel = None
        kernel_bytes = None
        desc = (f"gather: NVFP4 prefix of {prefix} tokens x {wl.h_kv} kv heads (one layer of the 28-layer stack, "
                f"permuted pages) -> dense FP8 workspace")
        extra = {"prefix": prefix, "kv_heads": wl.h_kv, "head_dim": 128, "page_size": 16}
        tokens_per_step = prefix
    elif name == "mixed":
        pt = torch.from_numpy(wl.page_table).to(dev)
        sl = torch.from_numpy(wl.total_lens.astype(np.int32)).to(dev)
        plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()),
                              args.pages_per_split)
        layers = []
        for layer in range(wl.layers):
            fp8 = wl.is_fp8(layer)
            pool, s1, s2 = build_layer_cache(nv, wl, layer, dev, fp8=fp8)
            layers.append(dict(precision=nv.PREC_FP8 if fp8 else nv.PREC_NVFP4, q=wl.q(layer).to(dev), pool=pool,
                               k_gscale=s1, v_gscale=s2,
                               out=torch.empty((wl.batch, wl.h_q, 128), dtype=torch.float32, device=dev)))
            log(f"layer {layer} ({'FP8' if fp8 else 'NVFP4'}) cache built, {time.perf_counter() - t_setup:.1f} s")
        log(f"28-layer cache built in {time.perf_counter() - t_setup:.1f} s")
        ws = nv.alloc_decode_workspace(wl.batch, wl.h_q, wl.h_kv, plan[1], dev)
        n_fp8 = len(wl.fp8_layers)
        step_bytes = (wl.layers - n_fp8) * wl.kv_bytes_nvfp4() + n_fp8 * wl.kv_bytes_fp8()

        call = nv.prepare_decode_layers(layers, pt, sl, wl.sm_scale, plan, wl.h_kv, workspace=ws)

        def step(events=None, i=0):
            call.run()
        timed_kernel = None
        kernel_bytes = None
        desc = (f"mixed: 28 layers (FP8 at {list(wl.fp8_layers)}), batch {wl.batch}, context 8192, "
                f"8 KV / 32 query heads, split-K {plan[1]} x {plan[0]} pages")
        extra = {"batch": wl.batch, "context_tokens": int(wl.total_lens.sum()), "layers": wl.layers,
                 "fp8_layers": list(wl.fp8_layers), "kv_heads": wl.h_kv, "q_heads": wl.h_q,
                 "pages_per_split": plan[0], "num_splits": plan[1]}
        tokens_per_step = wl.batch
    elif name == "prefill":
        # per NVFP4 layer of the stack: a 16384-token prompt written once into the NVFP4 cache and the
        # dense FP8 copy (one pass), then causal BF16-Q x FP8-KV attention over the copy
        ext = workloads.Workload(name="prefill", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                                 seq_lens=[wl.extend_prefix], chan=wl.chan)
        nlayers = [l for l in range(wl.layers) if not wl.is_fp8(l)]
        n_tok = wl.extend_prefix
        slots = torch.from_numpy(ext.slots(0, 0, n_tok)).to(dev)
        offs = torch.tensor([0, n_tok], dtype=torch.int32, device=dev)
        zero = torch.zeros(1, dtype=torch.int32, device=dev)
        gen = torch.Generator().manual_seed(wl.seed * 7 + 6)
        q_all = torch.randn((n_tok, wl.h_q, 128), generator=gen).to(torch.bfloat16).to(dev)
        att_out = torch.empty((n_tok, wl.h_q, 128), dtype=torch.float32, device=dev)
        k_ws = torch.empty((n_tok, wl.h_kv, 128), dtype=torch.uint8, device=dev)    # shared by layers
        v_ws = torch.empty_like(k_ws)
        layer_calls = []
        for layer in nlayers:
            k = ext.kv("k", 0, layer).to(dev)
            v = ext.kv("v", 0, layer).to(dev)
            gk_l = float(nv.global_scale(k).item())
            gv_l = float(nv.global_scale(v).item())
            pool = nv.alloc_nvfp4_pool(ext.num_pages, wl.h_kv, dev)
            s_wk, s_wv = 6.0 * gk_l, 6.0 * gv_l
            layer_calls.append((
                nv.prepare_nvfp4_prefill_write(k, v, slots, gk_l, gv_l, pool, s_wk, s_wv, k_ws, v_ws),
                nv.prepare_fp8_extend_attn(q_all, offs, k_ws, v_ws, offs, zero, s_wk, s_wv, wl.sm_scale, wl.h_kv,
                                           n_tok, 0, out=att_out)[0]))
            log(f"layer {layer} prompt ready, {time.perf_counter() - t_setup:.1f} s")
        att_events = []

        def step(events=None, i=0):
            for write, attend in layer_calls:
                write.run()
                if events is not None:
                    k = len(att_events)
                    events.record(k, 0, stream.cuda_stream)
                    attend.run()
                    events.record(k, 1, stream.cuda_stream)
                    att_events.append(k)
                else:
                    attend.run()
        # bytes of the write: read bf16 K+V (512 B per token-head), write NVFP4 (144 B) and FP8 (256 B)
        step_bytes = len(layer_calls) * wl.h_kv * n_tok * (512 + 144 + 256)
        att_flops = 4 * 128 * wl.h_q * (n_tok * (n_tok + 1) // 2)
        timed_kernel = "extend_attn_kernel"
        kernel_bytes = None
        desc = (f"prefill: {len(layer_calls)} NVFP4 layers x (16384-token prompt -> NVFP4 cache + FP8 copy in one pass, "
                f"causal attention of 32 query heads over the FP8 copy), 8 KV heads")
        extra = {"layers": len(layer_calls), "prompt": n_tok, "kv_heads": wl.h_kv, "q_heads": wl.h_q}
        tokens_per_step = n_tok
    else:  # extend
        ext = workloads.Workload(name="extend", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                                 seq_lens=[wl.extend_prefix + wl.extend_chunk], chan=wl.chan)
        nlayers = [l for l in range(wl.layers) if not wl.is_fp8(l)]
        prefix, chunk = wl.extend_prefix, wl.extend_chunk
        pt = torch.from_numpy(ext.page_table).to(dev)
        from bit_paged_kv_amd import paged
        caches = []
        slots = torch.from_numpy(ext.slots(0, 0, prefix)).to(dev)
        for layer in nlayers:
            k = ext.kv("k", 0, layer, length=prefix).to(dev)
            v = ext.kv("v", 0, layer, length=prefix).to(dev)
            pool, gk_l, gv_l = paged.build_nvfp4_cache(k, v, slots, ext.num_pages)
            ck = wl.chunk("k", layer).to(dev)
            cv = wl.chunk("v", layer).to(dev)
            caches.append((pool, gk_l, gv_l, ck, cv))
            del k, v
            log(f"layer {layer} prefix cache built, {time.perf_counter() - t_setup:.1f} s")
        log(f"extend caches built in {time.perf_counter() - t_setup:.1f} s")
        chunk_slots = torch.from_numpy(ext.slots(0, prefix, prefix + chunk)).to(dev)
        prefix_lens = torch.tensor([prefix], dtype=torch.int32, device=dev)
        offs = torch.tensor([0, prefix], dtype=torch.int32, device=dev)
        k_ws = torch.empty((prefix + chunk, wl.h_kv, 128), dtype=torch.uint8, device=dev)   # shared by layers
        v_ws = torch.empty_like(k_ws)

        chunk_offs = torch.tensor([0, chunk], dtype=torch.int32, device=dev)
        gen = torch.Generator().manual_seed(wl.seed * 7 + 5)
        q_chunk = torch.randn((chunk, wl.h_q, 128), generator=gen).to(torch.bfloat16).to(dev)   # N(0,1) queries
        att_out = torch.empty((chunk, wl.h_q, 128), dtype=torch.float32, device=dev)
        layer_calls = []
        for pool, gk_l, gv_l, ck, cv in caches:
            s_wk, s_wv = 6.0 * gk_l, 6.0 * gv_l       # the layer's FP8 scale amax / 448
            layer_calls.append((
                nv.prepare_dequant_to_workspace(pool, gk_l, gv_l, pt, prefix_lens, offs, prefix, s_wk, s_wv, wl.h_kv,
                                                k_ws, v_ws),
                nv.prepare_fp8_workspace_append(ck, cv, chunk_offs, offs, prefix_lens, chunk, prefix, s_wk, s_wv,
                                                wl.h_kv, k_ws, v_ws),
                nv.prepare_fp8_extend_attn(q_chunk, chunk_offs, k_ws, v_ws, offs, prefix_lens, s_wk, s_wv,
                                           wl.sm_scale, wl.h_kv, chunk, prefix, out=att_out)[0],
                nv.prepare_nvfp4_quantize_append(ck, cv, chunk_slots, gk_l, gv_l, pool)))
        att_events = []

        def step(events=None, i=0):
            for gather, append, attend, quantize in layer_calls:
                gather.run()
                append.run()
                if events is not None:
                    k = len(att_events)
                    events.record(k, 0, stream.cuda_stream)
                    attend.run()
                    events.record(k, 1, stream.cuda_stream)
                    att_events.append(k)
                else:
                    attend.run()
                quantize.run()
        # bytes: read prefix NVFP4 (144 B/token/head), write FP8 workspace (256 B), read chunk bf16 (512 B),
        # write chunk NVFP4 (144 B)
        step_bytes = len(caches) * wl.h_kv * (prefix * (144 + 256) + chunk * (512 + 144))
        # attention flops per launch: 4 * 128 per (query row, head, visible key)
        att_flops = 4 * 128 * wl.h_q * (chunk * prefix + chunk * (chunk + 1) // 2)
        timed_kernel = "extend_attn_kernel"
        kernel_bytes = None
        desc = (f"extend: {len(caches)} NVFP4 layers x (16384-token prefix -> shared FP8 workspace, 2048-token chunk "
                f"-> FP8 workspace, causal attention of the chunk's 32 query heads over prefix || chunk, chunk "
                f"quantize-append), 8 KV heads")
        extra = {"layers": len(caches), "prefix": prefix, "chunk": chunk, "kv_heads": wl.h_kv, "q_heads": wl.h_q}
        tokens_per_step = chunk

    # ---- warm up, then time exactly K steps -------------------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the headline region holds nothing but the K steps: no per-launch events inside it
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_gpu_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"

    # ---- the dominant kernel's own duration, right after the headline region ---------------------
    split_only = None
    if timed_kernel == "extend_attn_kernel":
        # two more steps, each attention launch between timing-only events on its launch stream
        att_events.clear()
        events = HipEventPairs(2 * len(layer_calls))
        for _ in range(2):
            step(events)
        torch.cuda.synchronize()
        kms = events.elapsed_ms()
        events.close()
        kernel_ms = sum(kms) / len(kms)
        achieved = att_flops / (kernel_ms * 1e-3) / 1e12
        bound, peak, unit = "mfma", MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        timing = (f"{timed_kernel}: mean of {len(kms)} launches in 2 steps after the timed region (min "
                  f"{min(kms) * 1e3:.1f} us, max {max(kms) * 1e3:.1f} us), timing-only HIP events (no system "
                  f"fence) recorded on the launch stream around each launch")
    elif timed_kernel:
        # The decode step is one kernel launch (the last piece of each split stream merges it).  The
        # roofline unit is the step: its duration comes from the HIP events around the K timed steps
        # (on the launch stream), which hold nothing else; a kernel trace of the same command shows
        # the launches back to back.
        kernel_ms = step_gpu_ms
        achieved = kernel_bytes / (kernel_ms * 1e-3) / 1e9
        # the kernel by itself, for reference: KERNEL_SAMPLES more steps whose kernel dispatch records
        # timing-only events (the recording itself adds a few microseconds inside the bracket)
        events = HipEventPairs(KERNEL_SAMPLES)
        for i in range(KERNEL_SAMPLES):
            step(events, i)
        torch.cuda.synchronize()
        kms = events.elapsed_ms()
        events.close()
        srt = sorted(kms)
        split_only = {"kernel": "decode_split_kernel<PageNv4>", "mean_us": round(sum(kms) / len(kms) * 1e3, 2),
                      "median_us": round(srt[len(srt) // 2] * 1e3, 2), "min_us": round(srt[0] * 1e3, 2),
                      "max_us": round(srt[-1] * 1e3, 2), "samples": len(kms),
                      "method": "hipEvents (no system fence) recorded by the kernel's own dispatch, in "
                                f"{KERNEL_SAMPLES} steps after the timed region; the recording adds a few us"}
        timed_kernel = "decode step: decode_split_kernel<PageNv4> (split streams merged in-kernel)"
        timing = (f"HIP events on the launch stream around the {args.steps} timed steps, divided by "
                  f"{args.steps}: the step's kernels back to back, nothing else in the region")
    else:
        kernel_ms = step_gpu_ms
        achieved = step_bytes / (kernel_ms * 1e-3) / 1e9
        timed_kernel = "whole step"
        timing = "HIP events on the launch stream around the K timed steps, divided by K"
    if name in ("long", "batch32", "tiny", "ragged"):
        assert torch.isfinite(out).all().item(), "non-finite decode output"
    log(f"{args.steps} steps: wall {ms_per_step:.4f} ms/step, events {step_gpu_ms:.4f} ms/step, "
        f"{value:.1f} GB/s ({value / HBM_PEAK_GBS:.1%} of 8 TB/s); {timed_kernel} {kernel_ms * 1e3:.1f} us "
        f"-> {achieved:.1f} {unit} ({achieved / peak:.1%} of {peak:.0f})")

    gscale = None
    if name == "write":
        # the per-tensor scale reduction over the same K and V (amax of 2 x 1.01 GB of bf16), timed apart
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nv.global_scale(k, out=g_k)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            nv.global_scale(k, out=g_k)
            nv.global_scale(v, out=g_v)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gb = 2 * n_tok * wl.h_kv * 128 * 2
        assert (float(g_k.item()), float(g_v.item())) == (gk, gv)
        gscale = {"us_for_k_and_v": round(us, 2), "bytes": gb, "GB/s": round(gb / (us * 1e-6) / 1e9, 1)}
        log(f"global scale of K and V: {us:.1f} us, {gscale['GB/s']} GB/s")

    # the device's streaming-read rate, for the decode configs (after the timed region)
    ceiling = None
    if bound == "hbm":
        ceiling = stream_read_ceiling(nv, step_bytes if name != "mixed" else wl.kv_bytes_nvfp4(), dev)
        log(f"streaming-read ceiling {ceiling['value']} GB/s; step at {100.0 * value / ceiling['value']:.1f} %, "
            f"kernel at {100.0 * achieved / ceiling['value']:.1f} % of it")

    cpu = None
    if not args.no_cpu_baseline and name in ("long", "batch32", "ragged", "tiny"):
        cpu = cpu_baseline(index)
        log(f"cpu baseline {cpu['value']} GB/s")
    elif not args.no_cpu_baseline and name == "gather":
        cpu = cpu_baseline_gather(index)
        log(f"cpu baseline {cpu['value']} GB/s")
    elif not args.no_cpu_baseline and name == "write":
        cpu = cpu_baseline_write(index)
        log(f"cpu baseline {cpu['value']} GB/s")
    elif not args.no_cpu_baseline and name in ("mixed", "extend", "prefill"):
        # mixed: the untimed cache preparation (quantizing each unit's K/V) takes ~25x the timed decode,
        # so its workers stop after 1 s of oracle time to keep the run within a minute
        cpu = cpu_baseline_stack(index, name, budget_s=1.0 if name == "mixed" else 6.0)
        log(f"cpu baseline {cpu['value']} GB/s" +
            (f", attention {cpu['attention_tflops']} TFLOP/s" if "attention_tflops" in cpu else ""))

    traffic, traffic_detail = None, None
    t = TRAFFIC.get(name)
    if t is not None and timed_kernel.startswith("decode step"):
        if decode_source_sha256() == t["source_sha256"] and list(plan) == t["plan"]:
            rd = sum(f for f, _ in t["kernels"].values()) * 1024 * t["fetch_factor"]
            wr = sum(w for _, w in t["kernels"].values()) * 1024 * t["write_factor"]
            traffic = round(rd + wr)
            traffic_detail = {"read_bytes": round(rd), "write_bytes": round(wr),
                              "algorithmic_read_bytes": kernel_bytes,
                              "per_kernel_kib_fetch_write": {k: list(v) for k, v in t["kernels"].items()},
                              "source": "rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE per dispatch x copy calibration"}
        else:
            traffic_detail = "kernel source or split plan changed since the counters were taken"
    res = {
        "metric": "NVFP4 paged decode attn: effective KV GB/s (% of HBM peak) + tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded; see workloads/)",
        "config": {"workload": desc, **extra},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_per_step / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": step_bytes,
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": timed_kernel,
                     "kernel_us": round(kernel_ms * 1e3, 2),
                     ("flops_per_launch" if bound == "mfma" else "bytes_per_launch"):
                         att_flops if bound == "mfma" else (kernel_bytes or step_bytes),
                     "traffic_detail": traffic_detail, "timing": timing},
        "cpu_baseline": cpu,
    }
    if gscale is not None:
        res["global_scale"] = gscale
    if split_only is not None:
        res["roofline"]["kernel_events"] = split_only
    if ceiling is not None:
        res["stream_read_ceiling"] = ceiling
        res["pct_of_stream_read_ceiling"] = round(100.0 * value / ceiling["value"], 2)
        res["roofline"]["frac_of_stream_read_ceiling"] = round(achieved / ceiling["value"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
