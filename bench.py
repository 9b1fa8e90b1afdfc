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

After the K steps, max(K, 100) decodes run back to back over the rotation between
two events; their average launch time is `decode_ms`, the time the roofline uses.
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
    p.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--copies", type=int, default=0, help="rotation depth (0 = enough for 1 GiB)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--overlap", action="store_true",
                   help="c3 only: measure how much per-layer decode hides behind the layer's GEMMs")
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
    p.add_argument("--cpu-seconds", type=float, default=10.0)
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
                 "c4": "fp8_e4m3_8192x8192", "c5": "bf16_kv_cache"}


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
    raise ValueError(cfg)


def cpu_baseline(x_cpu_bits: np.ndarray, dtype: int, seconds: float):
    """The oracle (single-threaded, as it stands) decoding the same tensor's container."""
    import oracle
    oracle.build(force=False)
    c = oracle.encode(dtype, x_cpu_bits)
    reps = 0
    t0 = time.perf_counter()
    while True:
        y = oracle.decode(c)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    assert np.array_equal(y, x_cpu_bits)
    gbps = reps * x_cpu_bits.nbytes / el / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"full tensor ({x_cpu_bits.size} elements), bit-serial oracle decode repeated {reps}x "
                      f"over {el:.1f} s on one host core"}


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
    # two events around all of them: the per-launch average without event overhead.
    # The containers are marshalled once, so the host enqueues launches faster than
    # the GPU runs them and the events see no host gaps.
    import ctypes
    lib = zx.lib()
    conts = [c.container() for c in cs]
    optrs = [ctypes.c_void_p(o.data_ptr()) for o in outs]
    eptr = ctypes.c_void_p(err.data_ptr())
    sptr = ctypes.c_void_p(stream.cuda_stream)
    n_launch = max(args.steps, 100)
    for k in range(R):
        assert lib.zx_decode(ctypes.byref(conts[k]), optrs[k], eptr, sptr) == 0
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    bad = 0
    for i in range(n_launch):
        k = i % R
        bad |= lib.zx_decode(ctypes.byref(conts[k]), optrs[k], eptr, sptr)
    d1.record(stream)
    torch.cuda.synchronize()
    assert bad == 0, "zx_decode returned an error status"
    dec_avg = d0.elapsed_time(d1) / n_launch
    # correctness at full size, outside the timed region
    assert int(err.item()) == 0, "decoder reported a corrupt container"
    for k in range(R):
        y = zx.decompress(cs[k])
        assert torch.equal(y.reshape(-1).view(x0.dtype), xs[k].reshape(-1)), f"copy {k} did not round-trip"
    c = cs[0]
    alg = decode_alg_bytes(c)
    achieved = alg / (dec_avg * 1e-3) / 1e9
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
    res = {
        "metric": METRIC,
        "value": round(raw_bytes / (dec_avg * 1e-3) / 1e9, 2),
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
        "config": {"workload": desc, "elements": c.n, "raw_bytes": raw_bytes, "rotation_copies": R},
        "decode_ms": round(dec_avg, 5),
        "decode_ms_in_step": round(float(step_dec_ms.mean()), 5),
        "encode_ms": round(float(enc_ms.mean()), 5),
        "encode_GBps": round(raw_bytes / (float(enc_ms.mean()) * 1e-3) / 1e9, 2),
        "ratio": round(c.nbytes() / raw_bytes, 5),
        "exponent_bits_per_element": round(c.total_bits / c.n, 5),
        "context_h2d_copy_GBps": round(h2d_gbps, 2),
        "context_d2d_copy_GBps": copy_context_GBps(alg),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": profiled_traffic(args.config),
                     "kernel": "k_decode", "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        xb = x0.reshape(-1).cpu().numpy()
        xb = xb.view(np.uint16) if c.dtype == 0 else xb.view(np.uint8)
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
    if args.codec == "huffman" and args.config in ("c1", "c2", "c4") and not args.fp4_scales:
        res = bench_single(args)
    else:
        import bench_big
        res = bench_big.run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
