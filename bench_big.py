"""Large workloads for bench.py (--config c3 | c5).

c3: Llama-3-8B-shaped BF16 weight set (32 layers x {q,k,v,o,gate,up,down} + lm_head),
    one codebook per tensor; a step decodes the whole set as 33 calls, one
    zx_decode_block_batch per transformer layer (7 tensors) and one for the lm_head.
c5: BF16 K/V cache [2, 32, 8, 32768, 128] (2^31 elements), one codebook per
    65536-element block; a step decodes the whole cache.

Inputs are drawn on the GPU with seeded generators (workloads.py), compressed once
(the encode is timed separately on a subset), then decoded repeatedly.  The
decoded outputs are compared with the inputs on the device after timing.
"""
from __future__ import annotations

import time

import numpy as np
import torch

import workloads
import lossless_float_compression_amd as zx

HBM_PEAK_GBPS = 8000.0
METRIC = "decode GB/s (BF16 out) and % HBM roofline; encode GB/s; compression ratio"


def _alg_bytes(c) -> int:
    read = (c.signmant.numel() + c.total_bits // 8 + c.gaps.numel() + c.seg_desc.numel() * 4
            + c.block_bitoff.numel() * 8 + c.block_seg.numel() * 4 + c.lengths.numel() + c.degenerate.numel() * 2)
    return int(read + c.raw_bytes())


def _traffic(cfg):
    from bench import profiled_traffic
    return profiled_traffic(cfg)


def decode_kernel_name(cs):
    from bench import decode_kernel_name as name
    return name(cs)


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def copy_context_GBps(traffic: int) -> float:
    """Context for a roofline fraction: device-to-device copies (hipMemcpyAsync, the
    runtime's blit kernel) that each move `traffic` bytes, half read and half written,
    rotated over at least 1 GiB of buffers and timed back to back like the decode
    launches: the rate a copy-shaped kernel reaches at this transfer size, in the
    same bytes-moved unit as roofline.achieved."""
    half = max(traffic // 2 // 256 * 256, 256)
    R = max(2, -(-(1 << 30) // (2 * half)))
    src = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(R)]
    dst = [torch.empty_like(a) for a in src]
    for a, b in zip(src, dst):
        a.fill_(1)
        b.copy_(a)
    n = max(100, R)
    e0, e1 = _events(2)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        dst[i % R].copy_(src[i % R])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    del src, dst
    return round(2 * half / (ms * 1e-3) / 1e9, 1)


def run_c3(args):
    names = workloads.c3_names()
    n_layers = min(getattr(args, "layers", workloads.C3_LAYERS), workloads.C3_LAYERS)
    per_layer = len(workloads.C3_SHAPES)
    # the first n_layers layers and the lm_head (all of the set by default)
    idx = list(range(n_layers * per_layer)) + [len(names) - 1]
    t0 = time.time()
    comps, raw_total, enc_ms = [], 0, []
    e = _events(2)
    shared = getattr(args, "shared_codebook", False)
    cb = zx.build_shared_codebook(workloads.c3_tensor(i) for i in idx) if shared else None
    for i in idx:
        x = workloads.c3_tensor(i)
        raw_total += x.numel() * 2
        if i < per_layer:  # time the encode of layer 0 (its 7 tensors), after one untimed call
            zx.compress(x, codebook=cb)
            torch.cuda.synchronize()
            e[0].record()
            c = zx.compress(x, codebook=cb)
            e[1].record()
            torch.cuda.synchronize()
            enc_ms.append((e[0].elapsed_time(e[1]), x.numel() * 2))
        else:
            c = zx.compress(x, codebook=cb)
        comps.append(c)
        del x
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    groups = [comps[l * per_layer:(l + 1) * per_layer] for l in range(n_layers)] + [[comps[-1]]]
    outs = [[zx.empty_output(c) for c in groups[0]], [zx.empty_output(c) for c in groups[0]]]
    out_head = zx.empty_output(comps[-1])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(evs=None):
        for g, grp in enumerate(groups):
            o = [out_head] if g == n_layers else outs[g % 2]
            if evs is not None:
                evs[g][0].record()
            zx.decompress_batch(grp, o, err=err)
            if evs is not None:
                evs[g][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[_events(2) for _ in groups] for _ in range(args.steps)]
    t1 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    layer_ms = np.array([[ev[g][0].elapsed_time(ev[g][1]) for g in range(n_layers)] for ev in evs])
    head_ms = np.array([ev[n_layers][0].elapsed_time(ev[n_layers][1]) for ev in evs])
    assert int(err.item()) == 0
    # correctness: decode every tensor again and compare with a regenerated input
    for i, c in zip(idx, comps):
        y = zx.decompress(c)
        assert torch.equal(y.view(torch.int16), workloads.c3_tensor(i)), f"tensor {i} did not round-trip"
        del y
    dec_ms = float(layer_ms.sum(1).mean() + head_ms.mean())
    layer_alg = sum(_alg_bytes(c) for c in groups[0])
    layer_raw = sum(c.raw_bytes() for c in groups[0])
    lay_avg = float(layer_ms.mean())
    achieved = layer_alg / (lay_avg * 1e-3) / 1e9
    comp_bytes = sum(c.nbytes() for c in comps)
    enc_t = sum(m for m, _ in enc_ms)
    enc_b = sum(b for _, b in enc_ms)
    return {
        "metric": METRIC, "value": round(raw_total / (dec_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "c3: Llama-3-8B-shaped BF16 weights, " + ("one model-wide codebook" if shared else
                                                                             "one codebook per tensor") + ", one batched call per layer",
                   "elements": int(raw_total // 2), "raw_bytes": int(raw_total), "calls_per_step": len(groups),
                   "layers": n_layers, "segments_per_layer_call": int(sum(c.nsegs for c in groups[0]))},
        "decode_ms": round(dec_ms, 4), "layer_decode_ms": round(lay_avg, 5), "lm_head_decode_ms": round(float(head_ms.mean()), 5),
        "layer_decode_GBps": round(layer_raw / (lay_avg * 1e-3) / 1e9, 2),
        "encode_GBps_layer0": round(enc_b / (enc_t * 1e-3) / 1e9, 2),
        "ratio": round(comp_bytes / raw_total, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": _traffic("c3"), "kernel": decode_kernel_name(groups[0]) + " (one layer call)",
                     "alg_bytes_per_launch": int(layer_alg)},
        "context_d2d_copy_GBps": copy_context_GBps(int(layer_alg)),
        "setup_s": round(setup_s, 1),
        **({} if args.no_cpu else {"cpu_baseline": _c3_cpu_baseline(args)}),
    }


def _c3_cpu_baseline(args):
    """The oracle on layer 0 (its seven tensors, one codebook each): a bounded sample of
    the set, copied from the device."""
    from bench import cpu_baseline_parts
    parts = [(workloads.c3_tensor(i).cpu().numpy().view(np.uint16).reshape(-1), 0, False)
             for i in range(len(workloads.C3_SHAPES))]
    return cpu_baseline_parts(parts, args.cpu_seconds, "layer 0 (7 tensors, 218,103,808 elements)")


def _c5_cpu_baseline(args):
    """The oracle on one (kv, layer) slab of the cache, one codebook per block: a bounded
    sample of the cache, copied from the device."""
    from bench import cpu_baseline_parts
    x = workloads.c5_slab(0, 0).cpu().numpy().view(np.uint16).reshape(-1)
    return cpu_baseline_parts([(x, 0, True)], args.cpu_seconds,
                              f"one [8, 32768, 128] slab (kv 0, layer 0; {x.size} elements, one codebook per block)")


def run_c5(args):
    t0 = time.time()
    x = workloads.c5()
    raw = x.numel() * 2
    torch.cuda.synchronize()
    # encode: the first call also allocates; the figure is the mean of the calls after it
    c = zx.compress(x, per_block=True)
    torch.cuda.synchronize()
    enc = []
    for _ in range(3):
        e = _events(2)
        e[0].record()
        c = zx.compress(x, per_block=True)
        e[1].record()
        torch.cuda.synchronize()
        enc.append(e[0].elapsed_time(e[1]))
    enc_ms = float(np.mean(enc))
    setup_s = time.time() - t0
    out = zx.empty_output(c)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(args.warmup):
        zx.decompress(c, out=out, err=err)
    torch.cuda.synchronize()
    reps = max(args.steps, 20)
    evs = [_events(2) for _ in range(reps)]
    t1 = time.perf_counter()
    for k in range(reps):
        evs[k][0].record()
        zx.decompress(c, out=out, err=err)
        evs[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    dec = np.array([a.elapsed_time(b) for a, b in evs])
    assert int(err.item()) == 0
    assert torch.equal(out.view(torch.int16), x), "K/V cache did not round-trip"
    dec_ms = float(np.median(dec))
    alg = _alg_bytes(c)
    achieved = alg / (dec_ms * 1e-3) / 1e9
    from bench import encode_alg_bytes
    enc_alg = encode_alg_bytes(c)
    return {
        "metric": METRIC, "value": round(raw / (dec_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "c5: BF16 K/V [2,32,8,32768,128], 0.5*t(5) with 4/128 channels x20, one codebook per 64K block",
                   "elements": int(x.numel()), "raw_bytes": int(raw)},
        "decode_ms": round(dec_ms, 4), "decode_ms_mean": round(float(dec.mean()), 4),
        "timing": f"median of {reps} launches, events around each",
        "encode_ms": round(enc_ms, 4),
        "encode_GBps": round(raw / (enc_ms * 1e-3) / 1e9, 2),
        "encode_roofline": {"bound": "hbm", "alg_bytes": int(enc_alg), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "achieved": round(enc_alg / (enc_ms * 1e-3) / 1e9, 1),
                            "frac": round(enc_alg / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "ratio": round(c.nbytes() / raw, 5), "exponent_bits_per_element": round(c.total_bits / c.n, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": _traffic("c5"), "kernel": decode_kernel_name([c]),
                     "alg_bytes_per_launch": int(alg)},
        "context_d2d_copy_GBps": copy_context_GBps(int(alg)),
        "setup_s": round(setup_s, 1),
        **({} if args.no_cpu else {"cpu_baseline": _c5_cpu_baseline(args)}),
    }


def run_overlap(args):
    """Per-layer decode hidden behind the consumer: layer l+1 is decoded on a side
    stream into the other of two scratch buffer sets while the 7 GEMMs of layer l
    (y = x W^T, x of `batch` tokens, BF16) run on the main stream.  For each batch
    size: decode alone, GEMMs alone (on decoded weights) and the pipelined loop,
    per layer, averaged over the layers after the first."""
    from lossless_float_compression_amd.pipeline import LayerPipeline
    n_layers = args.overlap_layers
    per_layer = len(workloads.C3_SHAPES)
    comps, raw_layer = [], 0
    for i in range(n_layers * per_layer):
        x = workloads.c3_tensor(i)
        if i < per_layer:
            raw_layer += x.numel() * 2
        comps.append(zx.compress(x))
        del x
    layers = [comps[l * per_layer:(l + 1) * per_layer] for l in range(n_layers)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pipe = LayerPipeline(layers, depth=2, err=err)
    main = torch.cuda.current_stream()
    shapes = list(workloads.C3_SHAPES.values())
    results = []
    for batch in args.overlap_batches:
        g = torch.Generator(device="cuda")
        g.manual_seed(7_000_000 + batch)
        xs = [torch.randn((batch, shp[1]), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
              for shp in shapes]
        ys = [torch.empty((batch, shp[0]), device="cuda", dtype=torch.bfloat16) for shp in shapes]

        def consumer(l, w):
            for j in range(per_layer):
                torch.matmul(xs[j], w[j].view(torch.bfloat16).t(), out=ys[j])

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = _events(2)
            e0.record(main)
            for _ in range(args.overlap_reps):
                fn()
            e1.record(main)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.overlap_reps / n_layers

        def decode_only():
            for l in range(n_layers):
                pipe.start(l)
                pipe.acquire(l, main)
                pipe.release(l, main)

        dec = [pipe.bufs[0]]
        pipe.start(0)
        dec_w = pipe.acquire(0, main)
        pipe.release(0, main)

        def gemm_only():
            for l in range(n_layers):
                consumer(l, dec_w)

        def pipelined():
            pipe.run(consumer, main)

        pipe.max_workgroups = 0
        t_dec = timed(decode_only)
        t_mm = timed(gemm_only)
        flops = 2.0 * batch * sum(o * i for o, i in shapes)
        row = {"batch": batch, "decode_ms": round(t_dec, 4), "gemm_ms": round(t_mm, 4),
               "gemm_TFLOPs": round(flops / (t_mm * 1e-3) / 1e12, 1), "pipelined": []}
        for wgs in args.overlap_wgs:
            pipe.max_workgroups = wgs
            t_pipe = timed(pipelined)
            # the share of the (uncapped) decode time that no longer adds to the layer time
            hidden = (t_dec + t_mm - t_pipe) / t_dec if t_dec > 0 else 0.0
            row["pipelined"].append({"decode_workgroups": wgs or "default (all resident slots)", "ms": round(t_pipe, 4),
                                     "hidden_frac": round(hidden, 3)})
        pipe.max_workgroups = 0
        row["hidden_frac"] = max(p["hidden_frac"] for p in row["pipelined"])
        results.append(row)
        del xs, ys, dec
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the pipeline's buffers after a run hold the last two layers: compare them
    for l in (n_layers - 2, n_layers - 1):
        pipe.start(l)
        w = pipe.acquire(l, main)
        for j in range(per_layer):
            assert torch.equal(w[j].view(torch.int16), workloads.c3_tensor(l * per_layer + j)), "pipeline decode mismatch"
        pipe.release(l, main)
    torch.cuda.synchronize()
    return {
        "metric": "per-layer decode hidden behind the consumer GEMMs (decode of layer l+1 on a second stream "
                  "into double-buffered scratch while layer l multiplies)",
        "value": results[-1]["hidden_frac"], "unit": "fraction of decode time hidden", "n_gpus": 1,
        "steps": args.overlap_reps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"c3 layers 0..{n_layers - 1}: 7 GEMMs per layer, y = x W^T",
                   "layer_raw_bytes": int(raw_layer), "batches": list(args.overlap_batches)},
        "results": results,
    }


def run_kv_slots(args):
    """K/V cache [2, 32, 8, 32768, 128] filled online into fixed compressed slots.

    The cache grows by 512 tokens at a time; each such step completes one 65536-
    element block in every (kv, layer, head) slab, 512 blocks in all, which one
    zx_kv_encode_slots call compresses into their slots (no host synchronisation).
    The 512 new blocks are first gathered into a contiguous staging buffer (where a
    serving loop would have written the new tokens), outside the timed region.
    Then reused blocks are decoded on demand: all 64 blocks of every slab of one
    layer (2 x 8 x 64 = 1024 slots) in one zx_kv_decode_slots launch."""
    from lossless_float_compression_amd.kvslots import KVSlotPool
    t0 = time.time()
    x = workloads.c5()                                   # int16 [2, 32, 8, 32768, 128]
    raw = x.numel() * 2
    nb_tok = 32768 // 512
    xv = x.view(2, 32, 8, nb_tok, 512 * 128)             # block (kv, layer, head, t)
    n_slabs = 2 * 32 * 8
    pool = KVSlotPool(n_slabs * nb_tok, bits_per_elem=args.kv_bits)
    stage = torch.empty((n_slabs, 512 * 128), dtype=torch.int16, device="cuda")
    slab_ids = torch.arange(n_slabs, dtype=torch.int32, device="cuda")
    status = torch.empty((nb_tok, n_slabs), dtype=torch.int32, device="cuda")
    # slot of block (slab, t) = slab * nb_tok + t
    ev = [_events(2) for _ in range(nb_tok)]
    pool.append(xv[:, :, :, 0].reshape(n_slabs, -1).contiguous(), slab_ids * nb_tok, status=status[0])   # warm-up
    torch.cuda.synchronize()
    for t in range(nb_tok):
        stage.copy_(xv[:, :, :, t].reshape(n_slabs, -1))
        sid = slab_ids * nb_tok + t
        ev[t][0].record()
        pool.append(stage, sid, status=status[t])
        ev[t][1].record()
    torch.cuda.synchronize()
    app_ms = np.array([a.elapsed_time(b) for a, b in ev])
    st = status.cpu().numpy()
    overflow = int((st == 6).sum())
    assert ((st == 0) | (st == 6)).all(), "append reported an error"
    setup_s = time.time() - t0
    blk_raw = n_slabs * 65536 * 2
    # decode on demand: every block of layer 5 (both kv, 8 heads, 64 blocks each)
    layer = 5
    slots = [((kv * 32 + layer) * 8 + h) * nb_tok + t for kv in range(2) for h in range(8) for t in range(nb_tok)]
    fits = [s for s in slots if st[s % nb_tok, s // nb_tok] == 0]
    out = torch.empty((len(fits), 65536), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    fits_t = torch.tensor(fits, dtype=torch.int32, device="cuda")
    for _ in range(args.warmup):
        pool.decode(fits_t, out=out, err=err)
    torch.cuda.synchronize()
    dev = []
    for _ in range(args.steps):
        e = _events(2)
        e[0].record()
        pool.decode(fits_t, out=out, err=err)
        e[1].record()
        torch.cuda.synchronize()
        dev.append(e[0].elapsed_time(e[1]))
    assert int(err.item()) == 0
    ref = x.view(2, 32, 8, nb_tok, 65536)
    for i, s in enumerate(fits):
        slab, t = divmod(s, nb_tok)
        kv, rest = divmod(slab, 256)
        l, h = divmod(rest, 8)
        assert torch.equal(out[i].view(torch.int16), ref[kv, l, h, t]), f"slot {s} did not round-trip"
    dec_ms = float(np.mean(dev))
    app = float(app_ms[1:].mean()) if nb_tok > 1 else float(app_ms.mean())
    used_bits = pool.block_bitoff[:, 1].sum().item()
    # bytes the stored blocks occupy in their slots (the rest of each slot is reserve)
    nseg_sum = pool.block_seg[:, 1].sum().item()
    words = ((pool.block_bitoff[:, 1] + 31) // 32).sum().item()
    stored = pool.n_slots * (pool.sizes.sm_bytes + pool.sizes.alphabet + 2 + 16 + 8) + words * 4 + nseg_sum * (64 + 8)
    # algorithmic bytes of an append: raw blocks read, sign/mantissa bytes, code bits and
    # gap bytes written (one gap byte per 128 code bits)
    app_alg = blk_raw + n_slabs * 65536 + (used_bits / 8 + used_bits / 128) * n_slabs / pool.n_slots
    return {
        "metric": "K/V append: raw GB/s compressed into fixed slots per 512-token step; on-demand slot decode GB/s",
        "value": round(blk_raw / (app * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "c5 K/V cache [2,32,8,32768,128] filled 512 tokens at a time into one slot per "
                               "65536-element block", "slots": pool.n_slots, "cap_words": pool.cap_words,
                   "blocks_per_append": n_slabs},
        "append_ms": round(app, 4), "append_blocks": n_slabs,
        "append_roofline": {"bound": "hbm", "achieved": round(app_alg / (app * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(app_alg / (app * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "overflow_blocks": overflow,
        "decode_slots": len(fits), "decode_ms": round(dec_ms, 4),
        "decode_GBps": round(len(fits) * 65536 * 2 / (dec_ms * 1e-3) / 1e9, 2),
        "pool_bytes": pool.nbytes(), "pool_ratio": round(pool.nbytes() / pool.raw_bytes(), 5),
        "stored_ratio": round(stored / pool.raw_bytes(), 5),
        "setup_s": round(setup_s, 1),
    }


def _zf_traffic(cfg):
    from bench import ZF_SOURCES, profiled_traffic
    return profiled_traffic(cfg, "k_zf_decode", ZF_SOURCES)


def _zf_alg_bytes(c) -> int:
    """Algorithmic bytes of one dominant-range decode: the container read, the output written."""
    nb = c.lb.numel()
    return int(c.signmant.numel() + c.planes.numel() + 2 * c.nrecords + nb + 8 * (nb + 1) + c.raw_bytes())


def _zf_inputs(cfg):
    """(list of device tensors decoded per step, description) for the dominant-range bench."""
    import bench
    if cfg in ("c1", "c2", "c4"):
        x, desc, _ = bench.make_input(cfg)
        return [x], desc
    if cfg == "c5":
        return [workloads.c5()], "c5: BF16 K/V [2,32,8,32768,128], 0.5*t(5) with 4/128 channels x20"
    # c3: layer 0's seven tensors (the per-layer decode unit)
    per_layer = len(workloads.C3_SHAPES)
    return [workloads.c3_tensor(i) for i in range(per_layer)], "c3: Llama-3-8B-shaped BF16, layer 0 (7 tensors)"


def run_zf(args):
    """Dominant-range codec (ZipFloat page, 3.1-3.3) on the same workloads as the
    Huffman codec: decode launches back to back over copies rotating through >= 1 GiB
    (one launch per tensor; a c3 step is layer 0's seven tensors), encode timed after
    one untimed call, ratio of all container bytes to the raw tensor."""
    t0 = time.time()
    xs0, desc = _zf_inputs(args.config)
    raw = sum(x.numel() * x.element_size() for x in xs0)
    cs0 = [zx.compress_zf(x) for x in xs0]
    alg = sum(_zf_alg_bytes(c) for c in cs0)
    R = max(2, -(-(1 << 30) // (alg + raw)))
    if raw * R > (24 << 30):
        R = 1
    copies = [xs0] + [[x.clone() for x in xs0] for _ in range(R - 1)]
    cs = [cs0] + [[zx.compress_zf(x) for x in xs] for xs in copies[1:]]
    outs = [[torch.empty_like(x) for x in xs] for xs in copies]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # encode: one untimed call per tensor, then the timed ones
    torch.cuda.synchronize()
    enc = []
    for _ in range(3):
        e = _events(2)
        e[0].record()
        for x in xs0:
            zx.compress_zf(x)
        e[1].record()
        torch.cuda.synchronize()
        enc.append(e[0].elapsed_time(e[1]))
    enc_ms = float(np.mean(enc[1:]))
    import ctypes
    L = zx.lib()
    conts = [[c.container() for c in cc] for cc in cs]
    optrs = [[ctypes.c_void_p(o.data_ptr()) for o in oo] for oo in outs]
    eptr = ctypes.c_void_p(err.data_ptr())
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step(k):
        bad = 0
        for c, o in zip(conts[k % R], optrs[k % R]):
            bad |= L.zx_zf_decode(ctypes.byref(c), o, eptr, sptr)
        return bad

    for k in range(max(args.warmup, R)):
        step(k)
    torch.cuda.synchronize()
    n_launch = max(args.steps, 100)
    d0, d1 = _events(2)
    d0.record()
    bad = 0
    for k in range(n_launch):
        bad |= step(k)
    d1.record()
    torch.cuda.synchronize()
    assert bad == 0 and int(err.item()) == 0
    dec_ms = d0.elapsed_time(d1) / n_launch
    for xs, oo in zip(copies, outs):
        for x, o in zip(xs, oo):
            assert torch.equal(o.view(x.dtype), x), "dominant-range decode did not round-trip"
    comp = sum(c.nbytes() for c in cs0)
    recs = sum(c.nrecords for c in cs0)
    n_el = sum(c.n for c in cs0)
    achieved = alg / (dec_ms * 1e-3) / 1e9
    return {
        "metric": "dominant-range codec: decode GB/s (output) and % HBM roofline; encode GB/s; compression ratio",
        "value": round(raw / (dec_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": n_launch,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
        "data": "synthetic", "config": {"workload": desc, "codec": "dominant-range (2048-element blocks, l_b = MD - 6)",
                                        "elements": int(n_el), "raw_bytes": int(raw), "rotation_copies": R},
        "decode_ms": round(dec_ms, 5), "encode_ms": round(enc_ms, 5),
        "encode_GBps": round(raw / (enc_ms * 1e-3) / 1e9, 2),
        "ratio": round(comp / raw, 5), "outlier_fraction": round(recs / n_el, 6),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": _zf_traffic(args.config),
                     "kernel": "k_zf_decode",
                     "alg_bytes_per_launch": int(alg // len(cs0))},
        "context_d2d_copy_GBps": copy_context_GBps(int(alg // len(cs0))),
        "setup_s": round(time.time() - t0, 1),
    }


def run_fp4_scales(args):
    """E8M0 block scales of MX-FP4 weights (every tensor of the Llama-3-8B-shaped set,
    blocks of 32 inputs; 2.3e8 bytes) as one tensor with one codebook: decode launches
    back to back over copies rotating through >= 1 GiB, encode after one untimed call."""
    t0 = time.time()
    x0 = workloads.fp4_scales_c3().view(torch.float8_e8m0fnu)
    raw = x0.numel()
    c0 = zx.compress(x0)
    alg0 = _alg_bytes(c0)
    R = max(2, -(-(1 << 30) // (alg0 + raw)))
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    cs = [c0] + [zx.compress(x) for x in xs[1:]]
    outs = [zx.empty_output(c) for c in cs]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    enc = []
    for _ in range(3):
        e = _events(2)
        e[0].record()
        zx.compress(x0)
        e[1].record()
        torch.cuda.synchronize()
        enc.append(e[0].elapsed_time(e[1]))
    enc_ms = float(np.mean(enc[1:]))
    setup_s = time.time() - t0
    import ctypes
    L = zx.lib()
    conts = [c.container() for c in cs]
    optrs = [ctypes.c_void_p(o.data_ptr()) for o in outs]
    eptr = ctypes.c_void_p(err.data_ptr())
    sptr = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for k in range(max(args.warmup, R)):
        assert L.zx_decode(ctypes.byref(conts[k % R]), optrs[k % R], eptr, sptr) == 0
    torch.cuda.synchronize()
    n_launch = max(args.steps, 100)
    d0, d1 = _events(2)
    d0.record()
    bad = 0
    for k in range(n_launch):
        bad |= L.zx_decode(ctypes.byref(conts[k % R]), optrs[k % R], eptr, sptr)
    d1.record()
    torch.cuda.synchronize()
    assert bad == 0 and int(err.item()) == 0
    dec_ms = d0.elapsed_time(d1) / n_launch
    for x, o in zip(xs, outs):
        assert torch.equal(o.view(torch.uint8), x.view(torch.uint8)), "scale bytes did not round-trip"
    achieved = alg0 / (dec_ms * 1e-3) / 1e9
    return {
        "metric": "E8M0 block-scale codec: decode GB/s (output) and % HBM roofline; encode GB/s; compression ratio",
        "value": round(raw / (dec_ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": n_launch,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "E8M0 scales of MX-FP4 blocks of 32 for the Llama-3-8B-shaped set (N(0,1/sqrt(fan_in))), "
                               "one tensor, one codebook", "elements": int(raw), "raw_bytes": int(raw), "rotation_copies": R},
        "decode_ms": round(dec_ms, 5), "encode_ms": round(enc_ms, 5),
        "encode_GBps": round(raw / (enc_ms * 1e-3) / 1e9, 2),
        "ratio": round(c0.nbytes() / raw, 5), "bits_per_element": round(c0.total_bits / c0.n, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "k_decode_fast<E8M0> (low-entropy mode)",
                     "alg_bytes_per_launch": int(alg0)},
        "context_d2d_copy_GBps": copy_context_GBps(int(alg0)),
        "setup_s": round(setup_s, 1),
    }


def run(args):
    if getattr(args, "fp4_scales", False):
        return run_fp4_scales(args)
    if getattr(args, "codec", "huffman") == "zf":
        return run_zf(args)
    if getattr(args, "kv_slots", False):
        return run_kv_slots(args)
    if getattr(args, "overlap", False):
        return run_overlap(args)
    if args.config == "c3":
        return run_c3(args)
    return run_c5(args)
