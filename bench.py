"""Benchmark of one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: append each sequence's newest K/V row
(pkv_kv_append), then paged decode attention over every cached token
(pkv_paged_decode_attn: the decode kernel and, for split contexts, the partition merge).
The latent workload calls pkv_paged_decode_attn_mla, the verify workload (several query
tokens per sequence, each appended) pkv_paged_decode_attn_multi, and --cascade on the
shared-prefix workload pkv_paged_decode_attn_cascade.  Inputs are seeded synthetic
tensors already resident in HBM when timing starts.

Steps rotate over --layers independent copies of the KV cache (one per layer, as in a
real model), so the 256 MB last-level cache cannot carry one step's KV into the next.

Prints one JSON line.  `value` is KV GB/s for the whole step (algorithmic KV bytes read
per step / step time); decode tokens/s (query tokens per second) is reported beside it.
`roofline` covers the attention call (decode + merge kernels of one call), timed with HIP
events on the stream the library launches on; a shared prefix is counted once there.
`cpu_baseline` is the fp64 oracle timed on a bounded sample of the same workload on this
host.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--cascade] [--graph] [--no-cpu]
                  [--flush]
"""

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: KV GB/s read & % of MI355X HBM peak; decode tokens/s"
HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0              # MI355X dense bf16 / fp16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gqa": ["paged_kv_cache_288_amd/csrc/gqa_stream.hip", "paged_kv_cache_288_amd/csrc/gqa_ring_body.hpp",
            "paged_kv_cache_288_amd/csrc/gqa_stream_body.hpp",
            "paged_kv_cache_288_amd/csrc/gqa_decode.hip", "paged_kv_cache_288_amd/csrc/gqa_tile.hpp",
            "paged_kv_cache_288_amd/csrc/gqa_multi.hip", "paged_kv_cache_288_amd/csrc/gqa_multi_ring_body.hpp",
            "paged_kv_cache_288_amd/csrc/gqa_multi_body.hpp",
            "paged_kv_cache_288_amd/csrc/pkv_device.hpp"],
    "mla": ["paged_kv_cache_288_amd/csrc/mla_stream.hip", "paged_kv_cache_288_amd/csrc/gqa_stream.hip",
            "paged_kv_cache_288_amd/csrc/gqa_stream_body.hpp", "paged_kv_cache_288_amd/csrc/gqa_tile.hpp",
            "paged_kv_cache_288_amd/csrc/pkv_device.hpp"],
    "multi": ["paged_kv_cache_288_amd/csrc/gqa_multi.hip", "paged_kv_cache_288_amd/csrc/gqa_multi_body.hpp",
              "paged_kv_cache_288_amd/csrc/gqa_multi_ring_body.hpp", "paged_kv_cache_288_amd/csrc/gqa_ring_body.hpp",
              "paged_kv_cache_288_amd/csrc/gqa_tile.hpp", "paged_kv_cache_288_amd/csrc/pkv_device.hpp"],
    "cascade": ["paged_kv_cache_288_amd/csrc/gqa_cascade.hip", "paged_kv_cache_288_amd/csrc/gqa_stream_body.hpp",
                "paged_kv_cache_288_amd/csrc/gqa_multi_body.hpp", "paged_kv_cache_288_amd/csrc/gqa_tile.hpp",
                "paged_kv_cache_288_amd/csrc/pkv_device.hpp"],
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text):
    """Source text without comments and blank lines: what the compiler sees of it."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_hash(kind):
    """Hash of the kernel sources' code (comments ignored), keying stored counter data."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def kv_bytes(w):
    """Algorithmic KV bytes one decode call reads: every cached token's K and V row once
    (the latent row once for MLA)."""
    if w.kind == "mla":
        per_token = w.d * w.elem_bytes
    else:
        per_token = 2 * w.Hkv * w.d * w.elem_bytes
    return int(w.context_lens.astype(np.int64).sum()) * per_token


def kv_unique_bytes(w):
    """KV bytes stored for the batch: a shared prefix counted once, then every sequence's
    own tokens (what has to come from HBM at least once per call)."""
    per_token = kv_bytes(w) // max(int(w.context_lens.astype(np.int64).sum()), 1)
    prefix = w.meta.get("prefix_blocks", 0) * w.bs
    own = int((w.context_lens.astype(np.int64) - prefix).sum())
    return (prefix + own) * per_token


def traffic_for(workload_name, kind):
    """Measured HBM bytes per call from committed counter runs, if they were taken on
    the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload_name)
    if not e or e.get("kernel_hash") != kernel_hash(kind):
        return None
    return e.get("bytes_per_call")


def kernel_family(w):
    """Kernel sources a workload runs on: the latent kernels, the multi-token kernel, or the
    single-token GQA kernels."""
    if w.kind == "mla":
        return "mla"
    return "multi" if w.q_len > 1 else "gqa"


def kernel_label(w, pkv, ps, cascade=False):
    if cascade:
        return ("pkv_paged_decode_attn_cascade call (cascade_kernel: tails and shared prefix "
                "in one launch, then cascade_merge_kernel)")
    if w.q_len > 1:
        ring = w.kv_dtype == "bf16" and w.d == 128 and (w.Hq // w.Hkv) * w.q_len <= 32
        return ("pkv_paged_decode_attn_multi call (%s + multi_merge_kernel)"
                % ("gqa_multi_ring_kernel" if ring else "gqa_multi_kernel"))
    if w.kind == "mla":
        if ps == 0 and w.Hq % 64 == 0 and w.Hq <= 128:
            return "pkv_paged_decode_attn_mla call, balanced mode (mla_split_kernel + stream_merge_kernel<512>)"
        if ps == 0 and w.Hq % 32 == 0 and w.Hq <= 128:
            return "pkv_paged_decode_attn_mla call, balanced mode (mla_stream_kernel + stream_merge_kernel<512>)"
        return "pkv_paged_decode_attn_mla call, partitioned (mla_decode_kernel + partition_merge_kernel<512>)"
    if pkv.decode_partition_size(w.B, w.Hkv, w.max_context_len, ps) == 0:
        # the merge: stream_merge_long_kernel when segments average more than 16 pieces
        merge = "stream_merge_kernel / stream_merge_long_kernel"
        if w.kv_dtype == "bf16" and w.d == 128:
            return ("pkv_paged_decode_attn call, balanced mode (gqa_multi_ring_kernel<1>, one query "
                    "row per sequence, + %s)" % merge)
        if w.d == 128:
            return ("pkv_paged_decode_attn call, balanced mode (gqa_multi_kernel<128, 1, true>, one "
                    "query row per sequence, + %s)" % merge)
        return "pkv_paged_decode_attn call, balanced mode (gqa_ring_kernel + %s)" % merge
    return "pkv_paged_decode_attn call, partitioned (gqa_decode_kernel + partition_merge_kernel)"


def read_ceiling():
    """Achievable read bandwidth on this GPU, measured in the same run by the library's
    streaming-read probe (a child process, started before this process touches the GPU):
    the best scattered 4 KiB-chunk and grid-stride rates with nontemporal loads."""
    exe = os.path.join(ROOT, "paged_kv_cache_288_amd", "read_ceiling")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    except (OSError, subprocess.TimeoutExpired):
        return None
    chunk = [float(m) for m in re.findall(r"scattered 4 KiB chunks, loads=nontemporal.*: ([0-9.]+) GB/s", r.stdout)]
    stream = [float(m) for m in re.findall(r"^loads=nontemporal.*: ([0-9.]+) GB/s", r.stdout, re.M)]
    if r.returncode != 0 or not chunk:
        return None
    return {"scattered_4KiB_nt_GBs": max(chunk), "grid_stride_nt_GBs": max(stream) if stream else None,
            "probe": "paged_kv_cache_288_amd/read_ceiling (4 GiB buffer, constant and random data)"}


class TimingEvent:
    """A HIP event for timing only (hipEventDisableSystemFence): recording it does not write
    back and invalidate the caches, as an ordinary event does (the HIP documentation gives
    this flag for events that only measure time, for more accurate timings).  Recorded on the
    stream the library launches on (torch's current stream)."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import ctypes
        import torch
        rc = self._lib().hipEventRecord(self._ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if getattr(self, "_ev", None) is not None and self._hip is not None:
            self._hip.hipEventDestroy(self._ev)
            self._ev = None


def cpu_model_name():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.TimeoutExpired):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, target_s=15.0):
    """Time the fp64 oracle on the first sequences of the workload (one thread)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:
        limiter = None
    order = list(range(w.B))
    done, tokens, t_total = 0, 0, 0.0
    while done < len(order) and t_total < target_s:
        b = order[done]
        L = int(w.context_lens[b])
        n = -(-L // w.bs)
        ids = w.block_table[b, :n]
        t0 = time.perf_counter()
        q = oracle.bf16_bits_to_f64(w.q[b:b + 1])
        table = np.arange(n)[None, :]
        if w.q_len > 1:
            K = oracle.decode_kv_bits(w.k_pool[ids], w.kv_dtype, w.k_scale)
            V = oracle.decode_kv_bits(w.v_pool[ids], w.kv_dtype, w.v_scale)
            oracle.multi_token_decode_attention(q, K, V, table, w.context_lens[b:b + 1], w.scale)
        elif w.kind == "mla":
            kv = oracle.bf16_bits_to_f64(w.k_pool[ids])
            oracle.mla_decode_attention(q, kv, table, w.context_lens[b:b + 1], w.scale, w.d_v)
        else:
            K = oracle.decode_kv_bits(w.k_pool[ids], w.kv_dtype, w.k_scale)
            V = oracle.decode_kv_bits(w.v_pool[ids], w.kv_dtype, w.v_scale)
            oracle.paged_decode_attention(q, K, V, table, w.context_lens[b:b + 1], w.scale)
        t_total += time.perf_counter() - t0
        tokens += L
        done += 1
    per_token = kv_bytes(w) / int(w.context_lens.astype(np.int64).sum())
    if limiter is not None:
        limiter.unregister()
    return {
        "value": round(tokens * per_token / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model_name(),
        "threads": ("one: BLAS and OpenMP pools limited to 1 thread with threadpoolctl"
                    if limiter is not None else "one (threadpoolctl unavailable; numpy default)"),
        "kind": "oracle",
        "sample": f"first {done} of {w.B} sequences ({tokens} cached tokens, all {w.Hq} "
                  f"query heads x {w.q_len} query tokens), gather + fp64 attention, "
                  f"{t_total:.1f} s",
        "decode_tokens_per_s": round(done * w.q_len / t_total, 4),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa70b")
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--layers", type=int, default=4,
                    help="copies of the KV cache the steps rotate over (one step = one layer)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--flush", action="store_true",
                    help="write 512 MiB of scratch before every step (outside the call's events)")
    ap.add_argument("--append-fp8", action="store_true",
                    help="FP8 workloads: append the new rows as bf16 through the quantizing append")
    ap.add_argument("--cascade", action="store_true",
                    help="shared-prefix workloads: attend through pkv_paged_decode_attn_cascade")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step's append and attention call as captured graphs")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling probe run before the benchmark")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps (steady clocks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (to scale memory counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path "
                          "has no multi-GPU mode"}))
        sys.exit(2)

    import torch
    import paged_kv_cache_288_amd as pkv
    from paged_kv_cache_288_amd.workloads import make_workload

    if not os.path.exists(pkv.library_path()):
        from paged_kv_cache_288_amd import build as _b
        _b.build(verbose=False)
    ceiling = None if args.no_ceiling else read_ceiling()
    pkv.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"

    t0 = time.time()
    w = make_workload(args.workload)
    log(f"workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} bs={w.bs} "
        f"{w.kv_dtype} sum(L)={int(w.context_lens.sum())} (generated in {time.time() - t0:.1f} s)")

    def put(a):
        if a is None:
            return None
        a = a.view(np.int16) if a.dtype == np.uint16 else a
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, kp0, vp0 = put(w.q), put(w.k_pool), put(w.v_pool)
    kps = [kp0] + [kp0.clone() for _ in range(args.layers - 1)]
    vps = [vp0] + [None if vp0 is None else vp0.clone() for _ in range(args.layers - 1)]
    bt, cl = put(w.block_table), put(w.context_lens)
    ks, vs = put(w.k_scale), put(w.v_scale)
    nk, nv, slots = put(w.new_k), put(w.new_v), put(w.slot_mapping)
    multi = w.q_len > 1
    cascade = bool(args.cascade)
    if cascade and (multi or w.kind != "gqa" or not w.meta.get("prefix_blocks")):
        sys.exit("--cascade needs a single-token GQA workload with a shared prefix")
    out = torch.empty((w.B, w.q_len, w.Hq, w.d_v) if multi else (w.B, w.Hq, w.d_v),
                      dtype=torch.float32, device=dev)
    ps = w.partition_size if args.partition is None else args.partition
    if cascade:
        pb = w.meta["prefix_blocks"]
        plen = pb * w.bs
        prefix_t = put(np.ascontiguousarray(w.block_table[0, :pb]))
        tail_np = np.ascontiguousarray(w.block_table[:, pb:])
        tail_t = put(tail_np)
        tail_lens_np = (w.context_lens - plen).astype(np.int32)
        tail_l = put(tail_lens_np)
        max_tail = int(tail_lens_np.max())
        nbytes = pkv.cascade_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, plen, max_tail)
    elif multi:
        nbytes = pkv.multi_workspace_bytes(w.B, w.q_len, w.Hq, w.Hkv, w.d, w.max_context_len)
    elif w.kind == "mla":
        nbytes = pkv.mla_workspace_bytes(w.B, w.Hq, w.d_v, w.max_context_len, ps)
    else:
        nbytes = pkv.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.max_context_len, ps)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.flush else None
    torch.cuda.synchronize()

    def attend(kp, vp):
        if cascade:
            pkv.paged_decode_attn_cascade(out, q, kp, vp, prefix_t, plen, tail_t, tail_l, w.scale,
                                          max_tail, kv_dtype=w.kv_dtype, k_scale=ks,
                                          v_scale=vs, workspace=ws)
        elif multi:
            pkv.paged_decode_attn_multi(out, q, kp, vp, bt, cl, w.scale, w.max_context_len,
                                        workspace=ws)
        elif w.kind == "mla":
            pkv.paged_decode_attn_mla(out, q, kp, bt, cl, w.scale, w.max_context_len, d_v=w.d_v,
                                      partition_size=ps, workspace=ws)
        else:
            pkv.paged_decode_attn(out, q, kp, vp, bt, cl, w.scale, w.max_context_len,
                                  kv_dtype=w.kv_dtype, k_scale=ks, v_scale=vs,
                                  partition_size=ps, workspace=ws)

    append_fp8 = args.append_fp8 and w.kv_dtype == "fp8"
    if append_fp8:
        # the new rows as bf16 values (their stored codes decoded), quantized again on append
        nk16 = (nk.view(torch.float8_e4m3fn).float() * ks[None, :, None]).to(torch.bfloat16)
        nv16 = (nv.view(torch.float8_e4m3fn).float() * vs[None, :, None]).to(torch.bfloat16)

    def append(kp, vp):
        if append_fp8:
            pkv.kv_append_fp8(kp, vp, nk16, nv16, ks, vs, slots)
        else:
            pkv.kv_append(kp, vp, nk, nv, slots, kv_dtype=w.kv_dtype)

    def step(i, ev=None):
        kp, vp = kps[i % args.layers], vps[i % args.layers]
        if flush_buf is not None:
            flush_buf.fill_(1)
        append(kp, vp)
        if ev is not None:
            ev[0].record()
        attend(kp, vp)
        if ev is not None:
            ev[1].record()

    if args.graph:
        # all cache copies' steps (append + attention each) captured as one graph, replayed
        # once per `layers` steps, as a model step over several layers would be; the
        # replays run the same kernels as the eager steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            pkv.graph_begin()
            for i in range(args.layers):
                append(kps[i], vps[i])
                attend(kps[i], vps[i])
            graph = pkv.graph_end()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        if args.steps % args.layers or args.warmup % args.layers or args.flush:
            sys.exit("--graph needs --steps and --warmup multiples of --layers, and no --flush")

        def step(i, ev=None):  # noqa: F811  (the graph-replay step)
            if i % args.layers == 0:
                graph.launch()

    # Bring the GPU to its steady clocks first: after the host-side workload generation the
    # device has been idle for seconds, and a handful of steps is not enough for its clocks
    # and power state to settle (the first steps then run up to ~20 % slower).  These steps
    # are untimed, like the W warmup steps that follow.
    settle_steps = 0
    t_settle = time.time() + max(args.settle_s, 0.0)
    while time.time() < t_settle:
        for _ in range(args.layers):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    if args.graph:  # no events inside a replay: the step time (append + attention) stands in
        call_ms = np.full(args.steps, total_ms / args.steps)
    else:
        call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_per_step = total_ms / args.steps

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    kvb = kv_bytes(w)
    kvu = kv_unique_bytes(w)
    shared = kvu != kvb
    call_avg = float(call_ms.mean())
    # HBM roofline on the bytes that must come from HBM: a shared prefix once
    achieved = kvu / (call_avg * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
    }
    if w.kind == "mla":
        # The latent case is a dense contraction on the matrix cores (scores over d_qk and
        # p.V over d_v for every query head and cached token), but at about 240 flop per
        # byte it sits below the ridge point of 8 TB/s and 2.5 PFLOP/s (312 flop/B): the
        # binding roof is the larger of the two minimum times, and the fraction is that
        # time over the call's.  Both rates are reported.
        flops = float(w.context_lens.astype(np.int64).sum()) * w.Hq * 2 * (w.d + w.d_v)
        tflops = flops / (call_avg * 1e-3) / 1e12
        t_hbm = kvu / (HBM_PEAK_GBS * 1e9)
        t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        hbm_bound = t_hbm >= t_mfma
        roofline = {
            "bound": "hbm" if hbm_bound else "mfma",
            "achieved": round(achieved, 2) if hbm_bound else round(tflops, 2),
            "peak": HBM_PEAK_GBS if hbm_bound else MFMA_BF16_PEAK_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round(max(t_hbm, t_mfma) / (call_avg * 1e-3), 4),
            "t_hbm_us": round(t_hbm * 1e6, 2),
            "t_mfma_us": round(t_mfma * 1e6, 2),
            "algorithmic_flops_per_call": flops,
            "hbm_achieved_GBs": round(achieved, 2),
            "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
            "mfma_achieved_TFLOPs": round(tflops, 2),
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        }
    elif multi:
        # q_len * G query rows share each K/V row: scores and p.V on the matrix cores, still
        # below the ridge point, so the call is priced against HBM; the MFMA share beside it
        flops = float(w.context_lens.astype(np.int64).sum()) * w.Hq * w.q_len * 2 * (w.d + w.d_v)
        tflops = flops / (call_avg * 1e-3) / 1e12
        roofline.update({
            "algorithmic_flops_per_call": flops,
            "mfma_achieved_TFLOPs": round(tflops, 2),
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        })
    result = {
        "metric": METRIC,
        "value": round(kvb / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.d, "block_size": w.bs, "kv_dtype": w.kv_dtype,
            "context_tokens": int(w.context_lens.sum()),
            "max_context_len": w.max_context_len,
            "partition_size": int(pkv.decode_partition_size(w.B, w.Hkv, w.max_context_len, ps))
            if w.kind != "mla" else ps,
            "kv_bytes_per_step": kvb, "flush_between_steps": bool(args.flush),
            "cache_copies_rotated": args.layers, "graph_replay": bool(args.graph),
            "quantizing_append": bool(append_fp8), "query_tokens_per_sequence": w.q_len,
            "cascade": cascade, "settle_s": args.settle_s, "settle_steps": settle_steps,
        },
        "decode_tokens_per_s": round(w.B * w.q_len / (ms_per_step * 1e-3), 1),
        **({"decode_tokens_per_s_80_layers_kv_attention_only_excludes_weights":
            round(w.B * w.q_len / (ms_per_step * 1e-3) / 80, 1)}
           if (w.kind, w.Hq, w.Hkv, w.d) == ("gqa", 64, 8, 128) else {}),
        "hbm_peak_frac_step": round(kvb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            **roofline,
            "traffic": traffic_for(w.name + ("+cascade" if cascade else ""),
                                   "cascade" if cascade else kernel_family(w)),
            "kernel": kernel_label(w, pkv, ps, cascade),
            "call_ms_avg": round(call_avg, 5),
            "call_ms_median": round(float(np.median(call_ms)), 5),
            "call_ms_p90": round(float(np.percentile(call_ms, 90)), 5),
            "algorithmic_bytes_per_call": kvu,
            **({"logical_bytes_per_call": kvb,
                "logical_GBs": round(kvb / (call_avg * 1e-3) / 1e9, 2)} if shared else {}),
        },
        "read_ceiling": ceiling,
        "cpu_baseline": None,
    }
    if ceiling:
        result["roofline"]["frac_of_measured_read_ceiling"] = round(
            achieved / ceiling["scattered_4KiB_nt_GBs"], 4)
    if not args.no_cpu:
        log("timing the oracle on a sample (one core)...")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
