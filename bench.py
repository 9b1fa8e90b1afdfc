"""Benchmark: canonical-Huffman exponent coding on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c1|c3|c4|c5]

A step is one pass of the whole hot path over the workload: exponent histogram,
codebook build, block sizes and scan, bit-pack encode (with the one host read of
the two size totals), and a decode.  The default workload is c2 (BF16 [4096,4096],
N(0, 1/64), one codebook per tensor, max code length 32).

To keep the reads honest against the 256 MB Infinity Cache, the step rotates over
R copies of the input and its containers (>= 1 GiB of traffic in flight): step i
encodes copy i % R and decodes copy (i + R/2) % R, which was encoded half a
rotation earlier and has been evicted since.

After the K steps, decodes run back to back over the rotation between two events,
at least 20 times; the median per-launch time is `decode_ms`, the time the roofline
uses.
The device-side encode chain is timed the same way (`encode_chain_ms`), and so are
whole compress() calls, host share included (`compress_ms_back_to_back`).
The JSON line reports decode throughput (BF16 bytes out / decode time) as `value`,
with encode throughput, compression ratio, the decode kernel's HBM roofline and
the CPU oracle's decode throughput on the host as extra fields.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode GB/s (BF16 out) and % HBM roofline; encode GB/s; compression ratio"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5", "c2-low", "c4-low"])
    p.add_argument("--copies", type=int, default=0, help="rotation depth (0 = enough for 1 GiB)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--overlap", action="store_true",
                   help="c3 only: measure how much per-layer decode hides behind the layer's GEMMs")
    p.add_argument("--layers", type=int, default=32,
                   help="c3 only: decode the first N transformer layers (and the lm_head) instead of all 32")
    p.add_argument("--overlap-layers", type=int, default=8)
    p.add_argument("--overlap-reps", type=int, default=5)
    p.add_argument("--overlap-batches", type=int, nargs="+", default=[1, 16, 128, 1024, 4096])
    p.add_argument("--overlap-wgs", type=int, nargs="+", default=[0, 256, 128, 64],
                   help="caps on the decode's resident workgroups to try (0 = default)")
    p.add_argument("--codec", default="huffman", choices=["huffman", "zf"],
                   help="zf: the dominant-range codec (2048-element blocks, 3 dense bit planes, outlier records)")
    p.add_argument("--shared-codebook", action="store_true",
                   help="c3 only: one model-wide codebook over all 225 tensors instead of one per tensor")
    p.add_argument("--kv-slots", action="store_true",
                   help="c5 only: fill the K/V cache online into fixed compressed slots, then decode slots on demand")
    p.add_argument("--kv-bits", type=float, default=3.5, help="slot stream capacity in bits per element")
    p.add_argument("--fp4-scales", action="store_true",
                   help="E8M0 block scales of MX-FP4 weights for the Llama-3-8B-shaped set, Huffman-coded whole byte")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--reps", type=int, default=25, help="timed repetitions (median reported; at least 20)")
    p.add_argument("--no-layer-call", action="store_true",
                   help="c2 only: skip the Llama-3-8B-shaped layer-call sub-record")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run plain device copies of 256 MiB (reference for HBM byte counters)")
    return p.parse_args()


DECODE_SOURCES = ("lossless_float_compression_amd/csrc/zx_decode.hip", "lossless_float_compression_amd/csrc/zx_common.h")
ZF_SOURCES = ("lossless_float_compression_amd/csrc/zx_zf.hip", "lossless_float_compression_amd/csrc/zx_common.h")


def decode_source_hash(sources=DECODE_SOURCES) -> str:
    """Hash of a decode kernel's sources with comments and blank space removed, so
    that only a change of the code itself invalidates counters taken on it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        src = open(os.path.join(ROOT, f), encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


# workload names used in the committed profile summaries
WORKLOAD_SLUG = {"c1": "bf16_1024x1024", "c2": "bf16_4096x4096", "c3": "llama3_8b_shaped_layer",
                 "c4": "fp8_e4m3_8192x8192", "c5": "bf16_kv_cache",
                 "c2-low": "bf16_4096x4096_low_entropy", "c4-low": "fp8_e4m3_8192x8192_low_entropy"}


def decode_kernel_name(cs) -> str:
    """Which decode kernel the library launches for a batch of containers (the same
    rule as its host code: per-block codebooks take k_decode_fast_blocks; a batch with a container
    under 2.3 bits per code, or of E8M0 scales, takes the fast decode's low-entropy mode)."""
    cs = [c for c in cs if c.n]
    if any(c.per_block for c in cs):
        return "k_decode_fast_blocks (per-block codebooks)"
    if any(c.dtype == 2 or 10 * c.total_bits < 23 * c.n for c in cs):
        return "k_decode_fast (low-entropy mode)"
    return "k_decode_fast"


def profiled_traffic(cfg: str, kernel: str = "k_decode", sources=DECODE_SOURCES):
    """HBM bytes per decode launch (FETCH_SIZE and WRITE_SIZE counters scaled by a plain
    copy of known size) from the committed counter summary, or None when there is none
    or the decode kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{WORKLOAD_SLUG[cfg]}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != decode_source_hash(sources):
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """Plain device-to-device copies of exactly 256 MiB (read 256 MiB, write 256 MiB)."""
    import torch
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied 5 x 268435456 bytes", flush=True)


def decode_alg_bytes(c) -> int:
    """Bytes the decode must move: every container array it reads plus the output."""
    read = (c.signmant.numel() + c.total_bits // 8 + c.gaps.numel() + c.seg_desc.numel() * 4
            + c.block_bitoff.numel() * 8 + c.block_seg.numel() * 4 + c.lengths.numel() + c.degenerate.numel() * 2)
    return int(read + c.raw_bytes())


def make_input(cfg):
    import torch
    import workloads
    if cfg == "c1":
        return workloads.c1().cuda(), "c1: BF16 [1024,1024] N(0,0.02) seed 0, one codebook, 64K blocks", None
    if cfg == "c2":
        return (workloads.c2().cuda(),
                "c2: BF16 [4096,4096] N(0,1/sqrt(4096)), one codebook per tensor, max code length 32", None)
    if cfg == "c4":
        q, scale = workloads.c4()
        return (q.cuda(), "c4: FP8 E4M3FN [8192,8192] N(0,1)*448/amax, one codebook, nibble sign+mantissa", scale)
    if cfg == "c2-low":
        return (workloads.low_entropy(workloads.BF16).cuda(),
                "BF16 [4096,4096] low-entropy exponents (one value at p 0.85, geometric tail), one codebook", None)
    if cfg == "c4-low":
        return (workloads.low_entropy(workloads.FP8).cuda(),
                "FP8 E4M3FN [8192,8192] low-entropy exponents (one value at p 0.85, geometric tail), one codebook", 1.0)
    raise ValueError(cfg)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads() -> int:
    """Host threads for the threaded oracle: the cores this process may use, at most 16
    (one GPU's share of the host on the GPU machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _timed_reps(fn, seconds: float, min_reps: int = 3):
    """Run fn until `seconds` have passed (at least min_reps times); return (median s, reps, last result)."""
    ts, out = [], None
    t_end = time.perf_counter() + seconds
    while len(ts) < min_reps or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        out = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), len(ts), out


def cpu_baseline(x_cpu_bits: np.ndarray, dtype: int, seconds: float):
    """The oracle as it stands, on this host, on the same tensor: its bit-serial decode of
    the tensor's container on T threads over independent 65536-element blocks (the
    reported value), then on one thread, and its single-threaded encode."""
    return cpu_baseline_parts([(x_cpu_bits, dtype, False)], seconds, f"full tensor ({x_cpu_bits.size} elements)")


def cpu_baseline_parts(parts, seconds: float, sample: str):
    """cpu_baseline over a sample of several tensors, each (raw bits, dtype, per_block)
    with its own container: the times of the parts add up, and the rates are the
    sample's raw bytes over those sums."""
    import oracle
    oracle.build(force=False)
    T = host_threads()
    share = seconds / 3 / max(len(parts), 1)
    t_enc = t_dec1 = t_decT = 0.0
    n_enc = n_dec1 = n_decT = 0
    nb = nblk = 0
    for bits, dtype, per_block in parts:
        te, ne, c = _timed_reps(lambda: oracle.encode(dtype, bits, per_block=per_block), share, min_reps=1)
        t1, n1, y1 = _timed_reps(lambda: oracle.decode(c), share, min_reps=1)
        tT, nT, yT = _timed_reps(lambda: oracle.decode_threaded(c, T), share)
        assert np.array_equal(y1, bits) and np.array_equal(yT, bits)
        t_enc += te; t_dec1 += t1; t_decT += tT
        n_enc += ne; n_dec1 += n1; n_decT += nT
        nb += bits.nbytes
        nblk += c.nblocks
    return {"value": round(nb / t_decT / 1e9, 4), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": (f"{sample}, {nblk} blocks of 65536: bit-serial oracle decode on {T} threads over contiguous "
                       f"block ranges ({n_decT} timed runs, medians summed over the {len(parts)} container(s)); "
                       f"single-thread decode ({n_dec1} runs) and encode ({n_enc} runs) likewise"),
            "decode_1thread_GBps": round(nb / t_dec1 / 1e9, 4),
            "encode_1thread_GBps": round(nb / t_enc / 1e9, 4),
            "cpu_model": cpu_model(), "host_threads_available": os.cpu_count()}


def exponent_stats(x_bits: np.ndarray, dtype: int, c) -> dict:
    """Entropy of the exponent histogram, mean and longest code length, input hash."""
    import hashlib
    e = ((x_bits >> 7) & 0xFF) if dtype == 0 else ((x_bits >> 3) & 0xF) if dtype == 1 else x_bits
    h = np.bincount(e.astype(np.int64), minlength=256 if dtype != 1 else 16).astype(np.float64)
    p = h[h > 0] / h.sum()
    return {"exponent_entropy_bits": round(float(-(p * np.log2(p)).sum()), 5),
            "mean_code_bits": round(c.total_bits / c.n, 5),
            "max_code_bits": int(c.lengths.max().item()),
            "input_sha256": hashlib.sha256(x_bits.tobytes()).hexdigest()}


def median_launch_ms(launch, n_per_rep: int, reps: int = 25, warmup: int = 5):
    """hipEvents around `n_per_rep` back-to-back launches (one rotation), `reps` times after
    `warmup` untimed reps; returns (median, mean) per-launch milliseconds."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for i in range(n_per_rep):
            launch(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        for i in range(n_per_rep):
            launch(i)
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) / n_per_rep for a, b in ev])
    return float(np.median(per)), float(per.mean())


def encode_chain(cs, xs):
    """A launcher for the device-side encode chain of copy k: zx_encode_plan (histogram,
    codebook, block sizes, totals, canonical codes, decode table) and zx_encode_coded, through the C ABI into
    preallocated buffers with the sizes already known (the same work compress() does,
    without its one host wait for the totals and without allocation)."""
    import ctypes
    import torch
    import lossless_float_compression_amd as zx
    L = zx.lib()
    P = ctypes.c_void_p
    sptr = P(torch.cuda.current_stream().cuda_stream)
    bufs = []
    for c, x in zip(cs, xs):
        flat = x.reshape(-1).view(torch.int16 if c.dtype == zx.BF16 else torch.uint8)
        nb = zx.nblocks_of(c.n)
        A = zx.alphabet(c.dtype)
        d = dict(flat=flat, th=torch.empty(A, dtype=torch.int32, device="cuda"),
                 cd=torch.empty(A, dtype=torch.int32, device="cuda"),
                 bh=torch.empty((max(nb, 1), A), dtype=torch.int32, device="cuda"),
                 ln=torch.empty((1, A), dtype=torch.uint8, device="cuda"),
                 dg=torch.empty(1, dtype=torch.int16, device="cuda"),
                 bo=torch.empty(nb + 1, dtype=torch.int64, device="cuda"),
                 bs=torch.empty(nb + 1, dtype=torch.int32, device="cuda"),
                 tot=torch.empty(2, dtype=torch.int64, device="cuda"),
                 dt=torch.empty(zx.zx_decode_table_bytes(), dtype=torch.uint8, device="cuda"),
                 sm=torch.empty_like(c.signmant), st=torch.empty_like(c.stream), sd=torch.empty_like(c.seg_desc),
                 gp=torch.empty_like(c.gaps), err=torch.zeros(1, dtype=torch.int32, device="cuda"))
        bufs.append((c, {k: (v if not torch.is_tensor(v) else P(v.data_ptr())) for k, v in d.items()}, d))

    def launch(k):
        c, p, _ = bufs[k % len(bufs)]
        st = 0
        st |= L.zx_encode_plan(c.dtype, p["flat"], c.n, 32, p["bh"], p["th"], p["ln"], p["dg"], p["bo"], p["bs"],
                               p["tot"], None, 0, p["dt"], p["cd"], p["err"], sptr)
        st |= L.zx_encode_coded(c.dtype, p["flat"], c.n, p["ln"], p["cd"], p["dg"], p["bo"], p["bs"], c.total_bits,
                                c.nsegs, p["sm"], p["st"], p["sd"], p["gp"], p["err"], sptr)
        assert st == 0, "encode chain call failed"

    def check():
        for c, _, d in bufs:
            assert int(d["err"].item()) == 0
            assert torch.equal(d["st"], c.stream) and torch.equal(d["gp"], c.gaps) and torch.equal(d["sm"], c.signmant)
            assert torch.equal(d["dt"], c.dtab) and torch.equal(d["bo"], c.block_bitoff)

    return launch, check


def encode_alg_bytes(c) -> int:
    """Bytes the encode must move: the input read once, every container array written."""
    return int(c.raw_bytes() + c.nbytes() - 64)


def layer_call_record(n_layers: int = 4, reps: int = 25):
    """One transformer-layer call of the Llama-3-8B-shaped set (7 tensors, one batched
    decode), rotating over layers 0..n_layers-1 so the reads come from HBM (4 layers
    move about 2.9 GB, over 10 times the 256 MB Infinity Cache); median of `reps`."""
    import ctypes
    import torch
    import workloads
    import lossless_float_compression_amd as zx
    per = len(workloads.C3_SHAPES)
    layers = []
    for l in range(n_layers):
        grp = []
        for j in range(per):
            x = workloads.c3_tensor(l * per + j)
            grp.append(zx.compress(x))
            del x
        layers.append(grp)
    outs = [zx.empty_output(c) for c in layers[0]]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    L = zx.lib()
    arrs = [(zx.zx_container * per)(*[c.container() for c in grp]) for grp in layers]
    optrs = (ctypes.c_void_p * per)(*[o.data_ptr() for o in outs])
    eptr = ctypes.c_void_p(err.data_ptr())
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(i):
        assert L.zx_decode_block_batch(arrs[i % n_layers], optrs, per, eptr, sptr) == 0

    med, mean = median_launch_ms(launch, n_layers, reps=reps)
    assert int(err.item()) == 0
    for grp_i in (0, n_layers - 1):     # outputs of the last call of each layer equal their inputs
        launch(grp_i)
        torch.cuda.synchronize()
        for j, o in enumerate(outs):
            assert torch.equal(o.view(torch.int16).reshape(-1), workloads.c3_tensor(grp_i * per + j).reshape(-1))
    alg = sum(decode_alg_bytes(c) for c in layers[0])
    raw = sum(c.raw_bytes() for c in layers[0])
    ach = alg / (med * 1e-3) / 1e9
    return {"workload": f"Llama-3-8B-shaped BF16 layer call (q,k,v,o,gate,up,down; 218,103,808 elements), "
                        f"rotating over layers 0-{n_layers - 1}",
            "layer_decode_ms": round(med, 5), "layer_decode_ms_mean": round(mean, 5),
            "decode_GBps": round(raw / (med * 1e-3) / 1e9, 2),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBPS, 4), "alg_bytes_per_launch": int(alg),
                         "traffic": profiled_traffic("c3"), "kernel": decode_kernel_name(layers[0])},
            "segments_per_call": int(sum(c.nsegs for c in layers[0])),
            "reps": reps}


def bench_single(args):
    import torch
    import lossless_float_compression_amd as zx

    x0, desc, scale = make_input(args.config)
    raw_bytes = x0.numel() * x0.element_size()
    c_probe = zx.compress(x0)
    per_copy_traffic = decode_alg_bytes(c_probe) + raw_bytes * 2
    R = args.copies or max(4, 2 * math.ceil((1 << 30) / per_copy_traffic / 2))
    xs = [x0.clone() for _ in range(R)]
    cs = [zx.compress(x) for x in xs]
    outs = [zx.empty_output(c) for c in cs]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    half = R // 2

    def step(i, ev=None):
        # decode first: its container was encoded half a rotation ago, so the decode
        # starts as soon as the previous step's encode kernels drain
        k_enc = i % R
        k_dec = (i + half) % R
        if ev is not None:
            ev[0].record(stream)
        zx.decompress(cs[k_dec], out=outs[k_dec], err=err)
        if ev is not None:
            ev[1].record(stream)
        cs[k_enc] = zx.compress(xs[k_enc], fp8_scale=scale)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_dec_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    enc_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    # decode launches back to back over the rotation (each copy cold in the caches),
    # events around each rotation: per-launch figures without event overhead.  The
    # containers are marshalled once, so the host enqueues launches faster than the
    # GPU runs them and the events see no host gaps.
    import ctypes
    lib = zx.lib()
    conts = [c.container() for c in cs]
    optrs = [ctypes.c_void_p(o.data_ptr()) for o in outs]
    eptr = ctypes.c_void_p(err.data_ptr())
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def dec_launch(i):
        k = i % R
        assert lib.zx_decode(ctypes.byref(conts[k]), optrs[k], eptr, sptr) == 0

    reps = max(20, args.reps)
    dec_med, dec_mean = median_launch_ms(dec_launch, R, reps=reps)
    # the device-side encode chain alone, back to back over the rotation
    enc_launch, enc_check = encode_chain(cs, xs)
    enc_med, _ = median_launch_ms(enc_launch, R, reps=reps)
    enc_check()

    # whole compress() calls back to back over the rotation (each waits for its own
    # totals on the host, so this includes the host's share of every call)
    def compress_launch(i):
        cs[i % R] = zx.compress(xs[i % R], fp8_scale=scale)

    cmp_med, _ = median_launch_ms(compress_launch, R, reps=reps)
    # correctness at full size, outside the timed region
    assert int(err.item()) == 0, "decoder reported a corrupt container"
    for k in range(R):
        y = zx.decompress(cs[k])
        assert torch.equal(y.reshape(-1).view(x0.dtype), xs[k].reshape(-1)), f"copy {k} did not round-trip"
    c = cs[0]
    alg = decode_alg_bytes(c)
    achieved = alg / (dec_med * 1e-3) / 1e9
    enc_alg = encode_alg_bytes(c)
    enc_e2e_ms = float(np.median(enc_ms))
    # context only: the same tensor kept in pinned host memory and copied to the device
    # per use, the offloading alternative the pages compare against
    pinned = torch.empty(raw_bytes, dtype=torch.uint8, pin_memory=True)
    dev_buf = torch.empty(raw_bytes, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dev_buf.copy_(pinned, non_blocking=True)
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0.record(stream)
    for _ in range(20):
        dev_buf.copy_(pinned, non_blocking=True)
    h1.record(stream)
    torch.cuda.synchronize()
    h2d_gbps = raw_bytes * 20 / (h0.elapsed_time(h1) * 1e-3) / 1e9
    del pinned, dev_buf
    from bench_big import copy_context_GBps
    xb = x0.reshape(-1).cpu().numpy()
    xb = xb.view(np.uint16) if c.dtype == 0 else xb.view(np.uint8)
    res = {
        "metric": METRIC,
        "value": round(raw_bytes / (dec_med * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": desc, "elements": c.n, "raw_bytes": raw_bytes, "rotation_copies": R,
                   "segments": c.nsegs, "timing": f"median over {reps} reps of {R} back-to-back launches"},
        "decode_ms": round(dec_med, 5),
        "decode_ms_mean": round(dec_mean, 5),
        "decode_ms_in_step": round(float(step_dec_ms.mean()), 5),
        "encode_ms": round(enc_e2e_ms, 5),
        "encode_GBps": round(raw_bytes / (enc_e2e_ms * 1e-3) / 1e9, 2),
        "compress_ms_back_to_back": round(cmp_med, 5),
        "encode_chain_ms": round(enc_med, 5),
        "encode_chain_GBps": round(raw_bytes / (enc_med * 1e-3) / 1e9, 2),
        "encode_roofline": {"bound": "hbm", "alg_bytes": enc_alg, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "chain_achieved": round(enc_alg / (enc_med * 1e-3) / 1e9, 1),
                            "chain_frac": round(enc_alg / (enc_med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "end_to_end_frac": round(enc_alg / (enc_e2e_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "ratio": round(c.nbytes() / raw_bytes, 5),
        "exponent_bits_per_element": round(c.total_bits / c.n, 5),
        **exponent_stats(xb, c.dtype, c),
        "context_h2d_copy_GBps": round(h2d_gbps, 2),
        "context_d2d_copy_GBps": copy_context_GBps(alg),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": profiled_traffic(args.config),
                     "kernel": decode_kernel_name([c]), "alg_bytes_per_launch": alg},
    }
    if args.config == "c2" and not args.no_layer_call:
        del xs, cs, outs
        torch.cuda.empty_cache()
        res["llama3_8b_layer_call"] = layer_call_record()
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(xb, c.dtype, args.cpu_seconds)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the codec needs no collectives: each GPU decodes its own shard)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        calibrate_copy()
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.overlap and args.config != "c3":
        print("--overlap applies to --config c3", file=sys.stderr)
        sys.exit(2)
    if args.kv_slots and args.config != "c5":
        print("--kv-slots applies to --config c5", file=sys.stderr)
        sys.exit(2)
    if args.codec == "huffman" and args.config in ("c1", "c2", "c4", "c2-low", "c4-low") and not args.fp4_scales:
        res = bench_single(args)
    else:
        import bench_big
        res = bench_big.run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
