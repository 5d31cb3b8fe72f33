"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic input already in
HBM: compress every layer's keys and values into the packed planes, then run
one decode-attention step (query prep, split-K attention, combine) per layer
straight from the packed cache.  The decode launches of all layers are
replayed from one captured HIP graph (--eager-decode launches them one by one).

Prints ONE JSON line.  `value` is decode-attention throughput in GB/s of
packed KV read (packed K + V bytes of all layers / decode time of the step);
keys and values compressed per second are reported beside it.  `roofline`
covers the split-K decode-attention kernel: algorithmic bytes per launch /
its mean launch duration (HIP events recorded by libtq around each launch on
the launch stream, in a separate pass after the timed region) against the
8 TB/s HBM peak.  `cpu_baseline` times the
fp64 oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--key-format full|first-stage|q8_0|q4_0]
                    [--rotation dense|hadamard|hadamard2] [--layout flat|paged] [--block-size N]
                    [--eager-decode] [--no-cpu-baseline] [--scores] [--calib-read] [--calib-mfma]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


SPIN_CYCLES = 40_000_000     # ~20 ms: covers the host enqueue time of the profiled steps


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3, and until 1.5 s of steps have run, so "
                         "that the GPU's clocks have settled under load)")
    ap.add_argument("--workload", default="asym-d256",
                    help="workload name (default: asym-d256, the largest single-GPU cache, 7.1 GB packed)")
    ap.add_argument("--key-format", choices=["full", "first-stage", "q8_0", "q4_0"], default="full",
                    help="full: Lloyd-Max codes + QJL signs (the default); first-stage: codes and "
                         "||k|| only (qjl_m = 0); q8_0 / q4_0: the rotated 8-bit / 4-bit block formats "
                         "(comparison workload)")
    ap.add_argument("--rotation", choices=["dense", "hadamard", "hadamard2"], default=None,
                    help="override the workload's rotation (hadamard2: two Walsh-Hadamard rounds)")
    ap.add_argument("--layout", choices=["flat", "paged"], default="flat",
                    help="flat: one contiguous cache per call (the default); paged: the same tokens in a "
                         "block pool behind a shuffled block table, written with tq_append_* and read with "
                         "tq_attend_decode_paged")
    ap.add_argument("--block-size", type=int, default=64)
    ap.add_argument("--splits", type=int, default=0,
                    help="split count of the decode (0: the library's plan)")
    ap.add_argument("--eager-decode", action="store_true",
                    help="launch the per-layer decode kernels one by one from the host instead of replaying "
                         "them from a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (to calibrate HBM byte counters)")
    ap.add_argument("--calib-read", action="store_true",
                    help="run only the streaming-read calibration program (the practical HBM read ceiling)")
    ap.add_argument("--calib-mfma", action="store_true",
                    help="run only the matrix-core calibration program (sustained bf16 / f16 / i8 MFMA rates)")
    ap.add_argument("--scores", action="store_true",
                    help="time only tq_scores (query prep + raw scores [B, Hq, T]) over every layer's packed "
                         "keys and print its own JSON line")
    return ap.parse_args()


def calib_copy(torch):
    """A plain copy kernel of known size: reads and writes 1 GiB per launch."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                      "launches": 15, "copy_GBps": round(2 * n / dt / 1e9, 1)}), flush=True)


class Layer:
    """Inputs, formats and packed planes of one layer (flat, or a block pool
    behind a seeded shuffled block table)."""

    def __init__(self, w, layer, tq, W, torch, paged_block=0, splits=0):
        self.cb = tq.tq_build_codebook(w.d, w.k_bits)
        self.rot = tq.tq_make_rotation(w.rotation_seed(layer), w.d, w.rot)
        self.kf = tq.KeyFormat(w.d, w.k_bits, self.cb, self.rot, qjl_m=w.qjl_m)
        self.bf = tq.BlockFormat(w.d, w.block_bits, self.rot) if w.block_bits else None
        self.vf = tq.ValueFormat(w.d, w.v_bits, w.group)
        self.k = W.make_keys(w, layer, device="cuda")
        self.v = W.make_values(w, layer, device="cuda")
        self.q = W.make_queries(w, layer, device="cuda")
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
        self.lay = None
        if paged_block:
            import numpy as np
            maxb = (w.T + paged_block - 1) // paged_block
            perm = np.random.default_rng(w.seed * 7 + layer).permutation(w.B * maxb).astype(np.int32)
            self.lay = tq.CacheLayout(maxb * paged_block, torch.full((w.B,), w.T, dtype=torch.int32, device="cuda"),
                                      torch.from_numpy(perm.reshape(w.B, maxb)).cuda(), paged_block, w.B * maxb)
            self.pos0 = torch.zeros(w.B, dtype=torch.int32, device="cuda")
            self.kc = tq.alloc_layout_key_cache(self.kf, self.lay, w.B, w.Hkv)
            self.vc = tq.alloc_layout_value_cache(self.vf, self.lay, w.B, w.Hkv)
            cap = self.lay.capacity
        else:
            self.kc = (tq.alloc_block_cache(self.bf, w.B, w.Hkv, w.T) if self.bf
                       else tq.alloc_key_cache(self.kf, w.B, w.Hkv, w.T))
            self.vc = tq.alloc_value_cache(self.vf, w.B, w.Hkv, w.T)
            cap = w.T
        self.splits = splits or tq.tq_attend_splits(self.kf, w.B, w.Hq, w.Hkv, cap)
        if self.bf:     # same split plan as the TurboQuant keys of this shape
            n = tq.tq_attend_block_workspace_bytes(self.bf, w.B, w.Hq, w.Hkv, cap, self.splits)
        else:
            n = (tq.tq_attend_workspace_bytes(self.kf, w.B, w.Hq, w.Hkv, cap, self.splits) if self.lay is None
                 else tq.tq_attend_paged_workspace_bytes(self.kf, w.B, w.Hq, w.Hkv, self.lay, self.splits))
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def compress_keys(self, tq):
        if self.bf:
            tq.tq_compress_keys_block(self.bf, self.k, self.kc)
        elif self.lay is None:
            tq.tq_compress_keys(self.kf, self.k, self.kc)
        else:
            tq.tq_append_keys(self.kf, self.k, self.lay, self.pos0, self.kc)

    def compress_values(self, tq):
        if self.lay is None:
            tq.tq_compress_values(self.vf, self.v, self.vc)
        else:
            tq.tq_append_values(self.vf, self.v, self.lay, self.pos0, self.vc)

    def decode(self, tq, w):
        if self.bf:
            tq.tq_attend_decode_block(self.bf, self.vf, self.q, self.kc, self.vc, w.Hkv, w.T, out=self.out,
                                      ws=self.ws, n_splits=self.splits)
        elif self.lay is None:
            tq.tq_attend_decode(self.kf, self.vf, self.q, self.kc, self.vc, w.Hkv, w.T, out=self.out, ws=self.ws,
                                n_splits=self.splits)
        else:
            tq.tq_attend_decode_paged(self.kf, self.vf, self.q, self.kc, self.vc, w.Hkv, self.lay, out=self.out,
                                      ws=self.ws, n_splits=self.splits)


def scores_only(w, layers, tq, torch, steps):
    """tq_scores over every layer's packed keys: key planes read plus fp32
    scores written, per second (HIP events around the timed layer passes)."""
    for L in layers:
        L.compress_keys(tq)
    out = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tq.tq_scores_workspace_bytes(layers[0].kf, w.B, w.Hq), 16), dtype=torch.uint8,
                     device="cuda")

    def one_pass():
        for L in layers:
            tq.tq_scores(L.kf, L.q, L.kc, w.Hkv, w.T, out=out, ws=ws)

    for _ in range(3):
        one_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        one_pass()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    key_bytes = w.layers * w.B * w.Hkv * w.T * w.key_bytes()
    score_bytes = w.layers * w.B * w.Hq * w.T * 4
    return {"mode": "scores", "workload": w.name, "layers": w.layers, "steps": steps,
            "tq_scores_ms_per_step": round(ms, 4), "key_bytes": key_bytes, "score_bytes": score_bytes,
            "GBps": round((key_bytes + score_bytes) / (ms * 1e-3) / 1e9, 1),
            "hbm_fraction": round((key_bytes + score_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def measured_traffic(w):
    """HBM bytes per launch of the split-K attention kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for a plain 1 GiB copy), or None when there is no summary
    for this workload or the kernel source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{w.name}.txt")
    src = os.path.join(ROOT, "attention_decode_amd", "csrc", "k_attend_mfma.hip")
    try:
        fields = {}
        for line in open(path):
            if ":" in line and not line.startswith("#") and not line.startswith("tq::"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("kernel_source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
        return (float(fields["attend_fetch_kib"]) * float(fields["fetch_factor"])
                + float(fields["attend_write_kib"]) * float(fields["write_factor"])) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def read_ceiling():
    """The streaming-read ceiling measured on this GPU model (GB/s), from the
    committed calibration summary (bench.py --calib-read), or None."""
    try:
        for line in open(os.path.join(ROOT, "profiles", "hbm_read_ceiling.txt")):
            if line.startswith("{"):
                return float(json.loads(line)["read_GBps"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def _oracle_leg(w, small, rot, k, v, q, seconds: float):
    """The oracle on (sequence 0, KV head h) units of `small` until the time
    budget: keys compressed, values compressed, then decode attention of the
    unit's G query heads over the oracle-packed unit."""
    import oracle as O

    key_time = val_time = dec_time = 0.0
    vectors = 0
    h = 0
    t_start = time.perf_counter()
    while h < small.Hkv and (h == 0 or time.perf_counter() - t_start < seconds):
        t0 = time.perf_counter()
        ok = O.compress_keys(k[h], w.k_bits, rot)
        t1 = time.perf_counter()
        ov = O.compress_values(v[h], w.v_bits, w.group)
        t2 = time.perf_counter()
        O.attend(q[h * w.G:(h + 1) * w.G], ok, w.k_bits, rot, ov, w.v_bits, w.group)
        t3 = time.perf_counter()
        key_time += t1 - t0
        val_time += t2 - t1
        dec_time += t3 - t2
        vectors += small.T
        h += 1
    packed = vectors * (w.key_bytes() + w.value_bytes())
    return {"decode_GBps": packed / dec_time / 1e9, "keys_compressed_per_s": vectors / key_time,
            "values_compressed_per_s": vectors / val_time, "units": h, "seconds": round(time.perf_counter() - t_start, 2)}


def cpu_baseline(w, seconds: float):
    """The oracle (as is) on a bounded sample of the workload, on all the host
    cores this process may use and then on one core: (sequence, KV head) units
    of up to 8192 tokens, each compressed (keys, then values) and attended by
    its G query heads.  The OpenMP thread count is set through the runtime the
    oracle links (omp_set_num_threads), between the legs."""
    import ctypes
    import oracle as O
    from attention_decode_amd import workloads as W

    allowed = len(os.sched_getaffinity(0))
    threads = min(int(os.environ.get("OMP_NUM_THREADS", allowed)), allowed)
    small = w.with_T(min(w.T, 8192), B=1, layers=1)
    rot = O.rotation(w.rotation_seed(0), w.d, w.rot, m=w.qjl_m)
    O.codebook(w.d, w.k_bits)
    k = W.make_keys(small, 0).double().numpy()[0]
    v = W.make_values(small, 0).double().numpy()[0]
    q = W.make_queries(small, 0).double().numpy()[0]
    gomp = ctypes.CDLL("libgomp.so.1")      # the OpenMP runtime liboracle.so is linked with
    gomp.omp_set_num_threads(threads)
    many = _oracle_leg(w, small, rot, k, v, q, 0.6 * seconds)
    gomp.omp_set_num_threads(1)
    one = _oracle_leg(w, small, rot, k, v, q, 0.4 * seconds)
    gomp.omp_set_num_threads(threads)
    return {
        "value": round(many["decode_GBps"], 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"{many['units']} (sequence, KV head) units x {small.T} tokens of {w.name} on {threads} threads, "
                  f"{one['units']} on 1 thread: fp64 oracle key and value compression, then decode attention of "
                  f"{w.G} query heads over the unit (GB/s of packed KV read)",
        "keys_compressed_per_s": round(many["keys_compressed_per_s"], 1),
        "values_compressed_per_s": round(many["values_compressed_per_s"], 1),
        "one_core": {"value": round(one["decode_GBps"], 5), "unit": "GB/s", "cores": 1,
                     "keys_compressed_per_s": round(one["keys_compressed_per_s"], 1),
                     "values_compressed_per_s": round(one["values_compressed_per_s"], 1)},
        "nproc": os.cpu_count(), "affinity_cores": allowed,
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence / KV head with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.calib_read or args.calib_mfma:
        import subprocess
        name = "calib_read" if args.calib_read else "calib_mfma"
        prog = os.path.join(ROOT, "attention_decode_amd", name)
        if not os.path.exists(prog):
            sys.exit(f"{name} is not built (python -m attention_decode_amd.build)")
        sys.exit(subprocess.call([prog]))
    import torch
    import attention_decode_amd as tq
    from attention_decode_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calib_copy:
        calib_copy(torch)
        return
    w = W.WORKLOADS[args.workload]
    if args.rotation and args.rotation != w.rot:
        w = replace(w, name=f"{w.name}-{args.rotation}", rot=args.rotation)
    if args.key_format == "first-stage":
        w = replace(w, name=w.name + "-first-stage", qjl=False)
    elif args.key_format in ("q8_0", "q4_0"):
        w = replace(w, name=f"{w.name}-{args.key_format}", block_bits=8 if args.key_format == "q8_0" else 4)
    if w.block_bits and args.layout != "flat":
        sys.exit("the block key formats run on the flat layout only")
    print(f"[bench] setting up {w.name}: layers={w.layers} B={w.B} Hkv={w.Hkv} Hq={w.Hq} T={w.T} d={w.d}",
          file=sys.stderr, flush=True)
    paged = args.block_size if args.layout == "paged" else 0
    if paged and (paged < 32 or paged & (paged - 1)):
        sys.exit("--block-size must be a power of two, at least 32")
    if paged:
        w = replace(w, name=f"{w.name}-paged{paged}")
    if args.scores and (w.block_bits or paged):
        sys.exit("--scores times tq_scores on the flat TurboQuant key planes only")
    layers = [Layer(w, l, tq, W, torch, paged, args.splits) for l in range(w.layers)]
    torch.cuda.synchronize()
    if args.scores:
        print(json.dumps(scores_only(w, layers, tq, torch, args.steps)), flush=True)
        return
    stream = torch.cuda.current_stream()

    def step(ev=None, eager=False):
        if ev:
            ev[0].record(stream)
        for L in layers:
            L.compress_keys(tq)
        if ev:
            ev[1].record(stream)
        for L in layers:
            L.compress_values(tq)
        if ev:
            ev[2].record(stream)
        if decode_graph is not None and not eager:
            decode_graph.replay()
        else:
            for L in layers:
                L.decode(tq, w)
        if ev:
            ev[3].record(stream)

    decode_graph = None
    # Warm-up: the GPU takes tens of milliseconds of sustained load to reach
    # its steady clocks, far more than three steps of a small cache, so by
    # default the warm-up runs for at least 1.5 s (and three steps).
    n_warm = 0
    t_warm = time.perf_counter()
    while args.warmup is None or n_warm < args.warmup:
        step()
        n_warm += 1
        if args.warmup is None and n_warm >= 3:
            torch.cuda.synchronize()
            if time.perf_counter() - t_warm >= 1.5:
                break
    torch.cuda.synchronize()
    # The per-layer decode launches (q-prep, split-K attention, merge for every
    # layer) are captured once into a HIP graph and replayed each step: at the
    # microsecond kernels of a small cache the host's launch path, not the GPU,
    # would otherwise set the pace.  The first replay must reproduce the eager
    # outputs bit for bit.
    if not args.eager_decode:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for L in layers:
                L.decode(tq, w)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        eager_out = [L.out.clone() for L in layers]
        decode_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(decode_graph):
            for L in layers:
                L.decode(tq, w)
        for L in layers:
            L.out.zero_()
        decode_graph.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(L.out, o) for L, o in zip(layers, eager_out)):
            sys.exit("graph replay of the decode launches differs from the eager launches")
        del eager_out

    print("[bench] warmup done", file=sys.stderr, flush=True)

    # timed region: the compress launches, then the decode graph (or the eager
    # decode launches); phase boundaries marked by stream events only
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-kernel launch durations: a separate pass with libtq's per-launch events.
    # The pass is queued behind one short spin kernel (torch.cuda._sleep), so
    # that the host runs ahead of the GPU and each launch's event pair brackets
    # the kernel rather than the host's launch latency (which matters for the
    # microsecond kernels of the per-layer decode).
    # One unrecorded step follows the spin, so that the recorded ones run at
    # the clocks of a busy GPU.
    spin = getattr(torch.cuda, "_sleep", None)
    tq.tq_profile_read("")
    if spin is not None:
        spin(SPIN_CYCLES)
    step(eager=True)
    tq.tq_profile_enable(True)
    for _ in range(max(1, min(args.steps, 5))):
        step(eager=True)
    torch.cuda.synchronize()
    tq.tq_profile_enable(False)
    attn_ms, attn_n = tq.tq_profile_read("tq_attend_splitk")
    qp_ms, qp_n = tq.tq_profile_read("tq_qprep")
    mg_ms, mg_n = tq.tq_profile_read("tq_merge_splits")
    kq_ms, kq_n = tq.tq_profile_read("tq_compress_keys")
    vq_ms, vq_n = tq.tq_profile_read("tq_compress_values")
    tq.tq_profile_read("")

    k_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    v_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    d_ms = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    ceiling = read_ceiling()
    packed = w.packed_bytes()
    vectors = w.vectors()
    value = packed / (d_ms * 1e-3) / 1e9
    # split-K attention kernel: algorithmic bytes per launch = packed K + V
    # planes of one layer + the queries read + the outputs written.  The
    # workspace traffic of the launch (score operands and per-query scales read
    # by every workgroup of a unit, split partials written for the merge) is
    # reported beside it, not counted.
    per_layer_keys = w.B * w.Hkv * w.T
    splits = layers[0].splits
    in_bytes = 4 if w.dtype == "float32" else 2
    q_bytes = w.B * w.Hq * w.d * in_bytes
    out_bytes = w.B * w.Hq * w.d * 4
    attn_bytes = per_layer_keys * (w.key_bytes() + w.value_bytes()) + q_bytes + out_bytes
    overhead = {"split_partials_written": w.B * w.Hq * splits * (w.d + 2) * 4 if splits > 1 else 0,
                "query_prep_rows": w.B * w.Hq * 2 * w.d * 4}
    attn_avg_s = attn_ms * 1e-3 / max(attn_n, 1)
    achieved = attn_bytes / attn_avg_s / 1e9
    # key compressor: algorithmic flops per key 2 d^2 (dense rotation; d log2 d
    # adds for a Walsh-Hadamard one) + 2 m d (QJL projection) against the bf16
    # matrix-core peak, and its HBM bytes (key read, planes written)
    import math
    kq_avg_s = kq_ms * 1e-3 / max(kq_n, 1)
    rot_flop = 2 * w.d * w.d if w.rot == "dense" else w.d * int(math.log2(w.d)) * (2 if w.rot == "hadamard2" else 1)
    key_flop = rot_flop + 2 * w.qjl_m * w.d
    key_io = in_bytes * w.d + w.key_bytes()
    kq_tflops = per_layer_keys * key_flop / kq_avg_s / 1e12 if kq_n else None
    kq_gbps = per_layer_keys * key_io / kq_avg_s / 1e9 if kq_n else None
    result = {
        "metric": "decode attention GB/s of packed KV read (% of HBM peak); keys compressed/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and statistics of the workload, no model weights)",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.B, "kv_heads": w.Hkv,
                   "q_heads": w.Hq, "tokens": w.T, "head_dim": w.d, "input_dtype": w.dtype,
                   "k_bits": (f"{w.block_bits} (rotated block format, fp16 scale per 32)" if w.block_bits
                              else f"{w.k_bits}+1 (Lloyd-Max + QJL sign)" if w.qjl
                              else f"{w.k_bits} (Lloyd-Max only, first-stage format)"), "rotation": w.rot,
                   "v_bits": w.v_bits, "v_group": w.group, "attn_splits": splits},
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "decode_launch": "eager" if decode_graph is None else "hip-graph",
        "decode_ms_per_step": round(d_ms, 4),
        "compress_keys_ms_per_step": round(k_ms, 4),
        "compress_values_ms_per_step": round(v_ms, 4),
        "keys_compressed_per_s": vectors / (k_ms * 1e-3),
        "values_compressed_per_s": vectors / (v_ms * 1e-3),
        "packed_bytes_per_step": packed,
        "roofline": {"bound": "hbm", "kernel": "tq_attend_splitk", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w), "bytes_per_launch": attn_bytes,
                     "bytes_per_launch_terms": {"packed_kv": per_layer_keys * (w.key_bytes() + w.value_bytes()),
                                                "queries": q_bytes, "outputs": out_bytes},
                     "workspace_overhead_bytes": overhead,
                     "avg_launch_us": round(attn_avg_s * 1e6, 3), "launches": attn_n,
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": round(achieved / ceiling, 4) if ceiling else None},
        "compress_keys_roofline": None if not kq_n else {
            "kernel": "tq_compress_keys", "bound": "mfma", "flop_per_key": key_flop,
            "achieved": round(kq_tflops, 2), "peak": 2500.0, "unit": "TFLOP/s", "frac": round(kq_tflops / 2500.0, 4),
            "hbm_GBps": round(kq_gbps, 1), "hbm_frac": round(kq_gbps / HBM_PEAK_GBS, 4),
            "keys_per_launch": per_layer_keys, "avg_launch_us": round(kq_avg_s * 1e6, 2)},
        "kernel_avg_us": {"tq_compress_keys": round(kq_ms * 1e3 / max(kq_n, 1), 3),
                          "tq_compress_values": round(vq_ms * 1e3 / max(vq_n, 1), 3),
                          "tq_qprep": round(qp_ms * 1e3 / max(qp_n, 1), 3),
                          "tq_attend_splitk": round(attn_avg_s * 1e6, 3),
                          "tq_merge_splits": round(mg_ms * 1e3 / max(mg_n, 1), 3) if mg_n else None},
    }
    if packed < (256 << 20):
        # The packed cache of all layers fits the 256 MB MALL, so the decode
        # above reads it largely from there.  Cold figure: before each decode
        # phase, a 512 MiB read evicts it; median over five phases.
        flush = torch.ones((512 << 20) // 4, device="cuda")
        cold = []
        for _ in range(5):
            flush.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            if decode_graph is not None:
                decode_graph.replay()
            else:
                for L in layers:
                    L.decode(tq, w)
            c1.record(stream)
            cold.append((c0, c1))
        torch.cuda.synchronize()
        cold_ms = sorted(a.elapsed_time(b) for a, b in cold)[len(cold) // 2]
        del flush
        result["decode_cold"] = {"ms_per_step": round(cold_ms, 4), "GBps": round(packed / (cold_ms * 1e-3) / 1e9, 2),
                                 "flush_bytes": 512 << 20}
    if paged:
        # one decode step's append: one new token per sequence into every layer's pool
        pos = torch.full((w.B,), w.T - 1, dtype=torch.int32, device="cuda")
        ones = [(L.k[:, :, -1:].contiguous(), L.v[:, :, -1:].contiguous()) for L in layers]
        torch.cuda.synchronize()
        tq.tq_profile_enable(True)
        tq.tq_profile_read("")
        for _ in range(10):
            for L, (k1, v1) in zip(layers, ones):
                tq.tq_append_keys(L.kf, k1, L.lay, pos, L.kc)
                tq.tq_append_values(L.vf, v1, L.lay, pos, L.vc)
        torch.cuda.synchronize()
        tq.tq_profile_enable(False)
        ak_ms, ak_n = tq.tq_profile_read("tq_compress_keys")
        av_ms, av_n = tq.tq_profile_read("tq_compress_values")
        result["append_one_token_us"] = {"keys_per_layer": round(ak_ms * 1e3 / max(ak_n, 1), 3),
                                         "values_per_layer": round(av_ms * 1e3 / max(av_n, 1), 3),
                                         "tokens_per_call": w.B * w.Hkv}
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
