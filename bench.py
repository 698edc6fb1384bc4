#!/usr/bin/env python3
"""Benchmark of the lossless BF16 weight codec on one MI355X.

One step = the whole hot path over one synthetic weight set already resident
in HBM: batched encode (plane split + histogram + 12-bit table, chunked rANS
encode, seek-table scan, compaction) followed by batched fused decode back to
BF16.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

With --fused-gemm M it measures instead the decode fused with its consumer
(Y += X W^T from the compressed weights, M rows of X) against torch's BF16
batched GEMM on the uncompressed weights and against decode-then-GEMM, on
the expert down projections of the MoE set by default, and prints that
line.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
DEFAULT_WORKLOAD = "moe-experts-bf16"  # the largest single-GPU set (22.5 GB)
FUSED_DEFAULT_WORKLOAD = "moe-w2-bf16"
STAGES = ["split_hist", "rans_encode", "scan", "compact"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None,
                   help=f"weight set (default {DEFAULT_WORKLOAD}; with --fused-gemm {FUSED_DEFAULT_WORKLOAD})")
    p.add_argument("--layout", default=None, choices=["bf16", "bf16r", "fp16", "fp16r", "fp32", "fp8e4m3", "fp8e5m2"],
                   help="plane layout (default: the set's own type; fp16* store the set as IEEE half, "
                        "fp8* as FP8 scaled per tensor)")
    p.add_argument("--tensor-table", action="store_true", help="one frequency table per tensor")
    p.add_argument("--raw-fallback", action="store_true", help="store chunks that do not shrink raw")
    p.add_argument("--crc", action="store_true", help="a CRC-32 per chunk, written by encode, checked by decode")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU work for the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the round-trip check before timing")
    p.add_argument("--cold-reps", type=int, default=5,
                   help="decode-only repetitions after a 1 GiB write that evicts the Infinity Cache and L2 "
                        "(and as many back-to-back warm ones); 0 skips both")
    p.add_argument("--fused-gemm", type=int, default=0, metavar="M",
                   help="measure the fused decode + GEMM with M rows of X (default set moe-w2-bf16)")
    p.add_argument("--copy-ref", action="store_true",
                   help="after timing, launch one plain device copy of 256 MiB (read 256 MiB, write 256 MiB): "
                        "the reference for scaling hardware byte counters taken over this run")
    return p.parse_args()


COPY_REF_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest():
    """sha256 over the HIP sources: measured traffic holds only for the
    kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lossless_weight_compression_bf16_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the counter passes recorded in
    profiles/traffic.json, or None when none match these sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest():
        return None
    return rec.get("traffic_bytes")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, xs, target_s, layout, opts):
    """The oracle, as it stands, on a bounded sample of the same set: with
    one thread per host core available (at most 16), and with one thread on a
    smaller piece of the same sample.  The sample is the set's first tensors,
    passed over again while less than target_s seconds have been spent (a
    small set is timed over several passes)."""
    import oracle
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(16, avail))
    # calibrate on a piece that gives every thread several chunks
    probe = xs[0][: min(xs[0].size, 4 * threads * 65536)]
    t = time.perf_counter()
    e = oracle.encode(probe, layout, threads=threads, opts=opts)
    oracle.decode(e, threads=threads)
    rate = probe.size / max(time.perf_counter() - t, 1e-6)  # elements / s, round trip
    want = max(int(rate * target_s), 1)
    sample, count = [], 0
    for x in xs:
        if count >= want and sample:
            break
        take = x if count + x.size <= 2 * want else x[: max(want - count, 65536)]
        sample.append(take)
        count += take.size
    t_enc = t_dec = 0.0
    nbytes = 0
    passes = 0
    while passes == 0 or t_enc + t_dec < target_s:
        for x in sample:
            t = time.perf_counter()
            e = oracle.encode(x, layout, threads=threads, opts=opts)
            t_enc += time.perf_counter() - t
            t = time.perf_counter()
            y, _ = oracle.decode(e, threads=threads)
            t_dec += time.perf_counter() - t
            assert np.array_equal(y, x)
            nbytes += x.size * w.elem_bytes
        passes += 1
    total = t_enc + t_dec
    # one thread, on the first ~1/threads of the same sample (whole chunks)
    one = sample[0][: max(65536, (count // threads) // 65536 * 65536)]
    t = time.perf_counter()
    e = oracle.encode(one, layout, threads=1, opts=opts)
    t1_enc = time.perf_counter() - t
    t = time.perf_counter()
    y, _ = oracle.decode(e, threads=1)
    t1_dec = time.perf_counter() - t
    assert np.array_equal(y, one)
    b1 = one.size * w.elem_bytes
    return {
        "value": nbytes / total / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {len(sample)} tensor(s) of {w.name}, {count} elements "
                  f"({count * w.elem_bytes / 1e6:.1f} MB), {passes} pass(es), encode + decode, {threads} threads",
        "encode_GBps": nbytes / t_enc / 1e9,
        "decode_GBps": nbytes / t_dec / 1e9,
        "seconds": total,
        "one_thread": {"value": b1 / (t1_enc + t1_dec) / 1e9, "encode_GBps": b1 / t1_enc / 1e9,
                       "decode_GBps": b1 / t1_dec / 1e9, "elements": int(one.size)},
        "host_cpus": avail,
        "cpu_model": cpu_model(),
    }


def coded_symbols(layout, seg):
    """The coded byte of each element under a plane layout (for reporting)."""
    if layout == "fp32":
        return ((seg.view(np.uint32) >> 23) & 0xFF).astype(np.uint8)
    if layout.startswith("fp8"):
        return ((seg.view(np.uint8) >> 3) & 0xF).astype(np.uint8)  # the exponent's top 4 bits
    v = seg.view(np.uint16)
    if layout == "bf16r":
        return ((v >> 7) & 0xFF).astype(np.uint8)
    if layout == "fp16r":
        return (((v >> 7) & 0xF8) | ((v >> 13) & 0x04) | ((v >> 8) & 0x03)).astype(np.uint8)
    return (v >> 8).astype(np.uint8)


def coded_plane_entropy(xs, tables, seek, layout, tensor_table, max_chunks=4096):
    """Bits per coded symbol over a strided sample of chunks: the empirical
    entropy of each chunk's coded bytes, their cross-entropy under the chunk's
    12-bit table (the ideal rANS length for that table), and the payload the
    encoder actually produced (states, words and padding)."""
    C = seek.size - 1
    stride = max(1, -(-C // max_chunks))
    h_emp = h_q = 0.0
    syms = pay = 0
    k = 0
    for ti, x in enumerate(xs):
        for c0 in range(0, x.size, 65536):
            if k % stride == 0:
                seg = x[c0:c0 + 65536]
                sym = coded_symbols(layout, seg)
                cnt = np.bincount(sym, minlength=256).astype(np.float64)
                nz = cnt > 0
                f = tables[ti if tensor_table else k].astype(np.float64)
                h_emp += float(-(cnt[nz] * np.log2(cnt[nz] / seg.size)).sum())
                h_q += float(-(cnt[nz] * np.log2(f[nz] / 4096.0)).sum())
                syms += seg.size
                pay += int(seek[k + 1] - seek[k])
            k += 1
    return {"H_emp": round(h_emp / syms, 4), "H_q": round(h_q / syms, 4),
            "payload_bits": round(8.0 * pay / syms, 4),
            "chunks_sampled": -(-C // stride), "chunk_stride": stride}


def fused_gemm_main(args):
    """Decode fused with its consumer against BF16 GEMM and decode-then-GEMM."""
    import torch
    import lossless_weight_compression_bf16_amd as wc
    from lossless_weight_compression_bf16_amd import _binding as B, codec, gemm as G, synthetic as S

    wc.lib()
    dev = torch.device("cuda:0")
    name = args.workload or FUSED_DEFAULT_WORKLOAD
    w = S.workload(name)
    if w.dtype != "bf16":
        raise SystemExit("the fused decode + GEMM takes BF16 sets")
    m = int(args.fused_gemm)
    shapes = [(int(r), int(c)) for r, c in w.shapes]
    T = len(shapes)
    log(f"[fused] generating {w.name}: {T} matrices, {w.n} elements; m = {m}")
    bits = S.set_bits(w)
    # W stacked per shape (bmm operands), each matrix a contiguous view
    groups = {}
    for i, sh in enumerate(shapes):
        groups.setdefault(sh, []).append(i)
    wstack, ws = {}, [None] * T
    for sh, idx in groups.items():
        st = torch.empty((len(idx),) + sh, dtype=torch.int16, device=dev)
        for j, i in enumerate(idx):
            st[j].copy_(torch.from_numpy(bits[i].view(np.int16)).view(sh))
            ws[i] = st[j].view(torch.bfloat16)
        wstack[sh] = st.view(torch.bfloat16)
    g = np.random.default_rng(12345)
    xb = [S.f32_to_bf16_bits(g.standard_normal(m * c).astype(np.float32)).reshape(m, c) for _, c in shapes]
    xs = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in xb]
    xt = {sh: torch.stack([xs[i].t() for i in idx]).contiguous() for sh, idx in groups.items()}  # G x K x m
    yflat = torch.zeros(sum(m * r for r, _ in shapes), dtype=torch.float32, device=dev)
    ys, off = [], 0
    for r, _ in shapes:
        ys.append(yflat[off:off + m * r].view(m, r))
        off += m * r
    log("[fused] encoding (tile order, and row-major for decode-then-GEMM)")
    et = G.encode_weights(ws)
    er = codec.encode_batch([x.view(-1) for x in ws])
    dstack = {sh: torch.empty_like(wstack[sh]) for sh in groups}
    douts = [None] * T
    for sh, idx in groups.items():
        for j, i in enumerate(idx):
            douts[i] = dstack[sh][j].view(-1)
    ns = [r * c for r, c in shapes]
    fmt = B.format_word("bf16")
    h_segs, tot = B.wc_plan_batch(fmt, ns)
    d_segs = codec.segments_to_device(h_segs, T, dev)
    h_g = G.gemm_descriptors(xs, ys, shapes)
    d_g = G.descriptors_to_device(h_g, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    bufs = et.batch.buffers()
    stream = torch.cuda.current_stream()

    def fused():
        yflat.zero_()
        B.wc_decode_gemm_batch(fmt, h_segs, d_segs, T, h_g, d_g, m, bufs, err, stream)

    def bf16_gemm():
        return [torch.bmm(wstack[sh], xt[sh]) for sh in groups]

    def decode_then_gemm():
        codec.decode_batch(er, outs=douts, check=False)
        return [torch.bmm(dstack[sh], xt[sh]) for sh in groups]

    # before timing: both encodings round-trip bit for bit, and the fused Y
    # agrees with torch's BF16 GEMM of the uncompressed weights (whose output
    # is rounded to BF16: relative differences of a few 2^-9 are expected;
    # the element-wise parity against the oracle is in the test suite)
    fused()
    torch.cuda.synchronize()
    if int(err.item()):
        raise RuntimeError(f"device error bits {int(err.item()):#x}")
    for a, b in zip(G.decode_weights(et), ws):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    yt = decode_then_gemm()
    torch.cuda.synchronize()
    for sh in groups:
        assert torch.equal(dstack[sh].view(torch.int16), wstack[sh].view(torch.int16))
    worst = 0.0
    for (sh, idx), y_b in zip(groups.items(), yt):
        for j, i in enumerate(idx):
            ref = y_b[j].t().float()
            worst = max(worst, float((ys[i] - ref).abs().max() / ref.abs().max().clamp_min(1e-30)))
    if worst > 2.0 ** -6:
        raise RuntimeError(f"fused Y differs from the BF16 GEMM by {worst:.3g} of its largest value")
    log(f"[fused] checked: both encodings round-trip; fused Y within {worst:.2e} of the BF16 GEMM")

    def timed(fn, K, W):
        for _ in range(W):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in ev]
        return float(np.mean(t)), float(np.median(t)), float(min(t))

    K, W = args.steps, args.warmup
    f_ms = timed(fused, K, W)
    b_ms = timed(bf16_gemm, K, W)
    d_ms = timed(decode_then_gemm, K, W)
    dec_only = timed(lambda: codec.decode_batch(er, outs=douts, check=False), K, W)
    C = int(tot.num_chunks)
    payload_bytes = int(et.batch.payload.numel())
    raw_w = 2 * int(tot.n)
    alg = (payload_bytes + int(tot.raw_bytes) + int(tot.table_bytes) + 8 * (C + 1)
           + sum(2 * m * c for _, c in shapes) + sum(4 * m * r for r, _ in shapes))
    achieved = alg / (f_ms[0] / 1e3) / 1e9
    flops = sum(2.0 * m * r * c for r, c in shapes)
    result = {
        "metric": "fused decode+GEMM: BF16 weight GB/s consumed (Y = X W^T from compressed W)",
        "value": round(raw_w / (f_ms[0] / 1e3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(f_ms[0], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "m": m, "matrices": T, "elements": int(tot.n), "chunks": C},
        "ratio": round(et.ratio, 5),
        "fused_ms": {"mean": round(f_ms[0], 5), "median": round(f_ms[1], 5), "min": round(f_ms[2], 5)},
        "bf16_gemm_ms": {"mean": round(b_ms[0], 5), "median": round(b_ms[1], 5), "min": round(b_ms[2], 5),
                         "kind": f"torch.bmm per shape ({len(groups)} launches), uncompressed BF16 weights"},
        "decode_then_gemm_ms": {"mean": round(d_ms[0], 5), "median": round(d_ms[1], 5),
                                "min": round(d_ms[2], 5)},
        "decode_only_ms": round(dec_only[0], 5),
        "fused_vs_bf16": round(b_ms[0] / f_ms[0], 4),
        "fused_vs_decode_then_gemm": round(d_ms[0] / f_ms[0], 4),
        "bf16_gemm_weight_GBps": round(raw_w / (b_ms[0] / 1e3) / 1e9, 2),
        "tflops": round(flops / (f_ms[0] / 1e3) / 1e12, 3),
        "roofline": {"kernel": "decode_gemm", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "alg_bytes": alg},
        "max_rel_diff_vs_bf16_gemm": round(worst, 6),
    }
    if not args.no_cpu_baseline:
        log("[fused] timing the oracle on host cores")
        result["cpu_baseline"] = fused_cpu_baseline(w, bits, xb, shapes)
    print(json.dumps(result), flush=True)


def fused_cpu_baseline(w, bits, xb, shapes):
    """The oracle as it stands on the first matrix: decode of its tile-ordered
    stream (all host cores, at most 16), the inverse tile order, and the
    double-precision X W^T (one thread)."""
    import oracle
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(16, avail))
    r, c = shapes[0]
    tiles = oracle.tile_order(bits[0].reshape(r, c))
    e = oracle.encode(tiles, "bf16", threads=threads)
    t = time.perf_counter()
    y, _ = oracle.decode(e, threads=threads)
    wmat = oracle.tile_order(y, True, (r, c))
    oracle.gemm_bf16(xb[0], wmat)
    dt = time.perf_counter() - t
    assert np.array_equal(wmat.reshape(-1), bits[0])
    return {"value": 2 * r * c / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"matrix 0 of {w.name} ({r} x {c}), m = {xb[0].shape[0]}: decode ({threads} threads), "
                      f"inverse tile order and double-precision X W^T (1 thread)",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the codec shards by "
              "whole tensors with no exchange on decode, and no multi-GPU path is built here.",
              file=sys.stderr)
        sys.exit(2)
    if args.fused_gemm:
        if not 1 <= args.fused_gemm <= 64:
            raise SystemExit("--fused-gemm takes 1 to 64 rows")
        fused_gemm_main(args)
        return

    import torch
    import lossless_weight_compression_bf16_amd as wc
    from lossless_weight_compression_bf16_amd import _binding as B, codec, synthetic as S

    wc.lib()
    dev = torch.device("cuda:0")
    w = S.workload(args.workload or DEFAULT_WORKLOAD)
    layout = args.layout or w.dtype
    if layout.startswith("fp16"):
        w = S.with_dtype(w, "fp16")
    elif layout.startswith("fp8"):
        w = S.with_dtype(w, layout)
    elif (layout == "fp32") != (w.dtype == "fp32"):
        raise SystemExit(f"layout {layout} does not fit the {w.dtype} set {w.name}")
    opts = ((B.WC_OPT_TENSOR_TABLE if args.tensor_table else 0) | (B.WC_OPT_RAW_FALLBACK if args.raw_fallback else 0)
            | (B.WC_OPT_CRC32 if args.crc else 0))
    fmt = B.format_word(layout) | opts
    log(f"[bench] generating {w.name}: {len(w.shapes)} tensors, {w.n} elements")
    t0 = time.perf_counter()
    xs = S.set_bits(w)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; uploading")
    ity = {4: torch.int32, 2: torch.int16, 1: torch.uint8}[w.elem_bytes]
    nty = {4: np.int32, 2: np.int16, 1: np.uint8}[w.elem_bytes]
    ins = [torch.from_numpy(x.view(nty)).to(dev) for x in xs]
    outs = [torch.empty_like(t) for t in ins]
    ns = [t.numel() for t in ins]

    h_in, tot = B.wc_plan_batch(fmt, ns)
    h_out, _ = B.wc_plan_batch(fmt, ns)
    for i in range(len(ins)):
        h_in[i].ptr = ins[i].data_ptr()
        h_out[i].ptr = outs[i].data_ptr()
    d_in = codec.segments_to_device(h_in, len(ins), dev)
    d_out = codec.segments_to_device(h_out, len(ins), dev)
    raw = torch.empty(tot.raw_bytes, dtype=torch.uint8, device=dev)
    tables = torch.empty(max(tot.table_bytes // 2, 8), dtype=torch.int16, device=dev)
    seek = torch.empty(tot.num_chunks + 1, dtype=torch.int64, device=dev)
    payload = torch.empty(tot.payload_capacity, dtype=torch.uint8, device=dev)
    scratch = torch.empty(tot.scratch_bytes, dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    crc = torch.empty(max(int(tot.num_chunks), 1), dtype=torch.int32, device=dev) if args.crc else None
    enc_bufs = B.make_buffers(raw, tables, seek, payload, tot.payload_capacity, crc)
    stream = torch.cuda.current_stream()
    C = int(tot.num_chunks)
    n = int(tot.n)
    raw_in_bytes = n * w.elem_bytes

    K, W = args.steps, args.warmup
    # per step: 5 stage events recorded inside wc_encode_batch, 2 around the decode
    evs = [B.HipEvents(7) for _ in range(max(K, 1))]

    def step(i=None):
        sev = evs[i] if i is not None else None
        B.wc_encode_batch(fmt, h_in, d_in, len(ins), enc_bufs, scratch, scratch.numel(), err,
                          stream, sev)
        if sev is not None:
            sev.record(5, stream)
        dec_bufs = B.make_buffers(raw, tables, seek, payload, payload_bytes, crc)
        B.wc_decode_batch(fmt, h_out, d_out, len(outs), dec_bufs, err, stream)
        if sev is not None:
            sev.record(6, stream)

    # one encode first, so every decode (warm-up included) is given the
    # payload's real size, which selects the decoder variant
    B.wc_encode_batch(fmt, h_in, d_in, len(ins), enc_bufs, scratch, scratch.numel(), err, stream, None)
    torch.cuda.synchronize()
    payload_bytes = int(seek[-1].item())
    for _ in range(max(W, 1)):
        step()
    torch.cuda.synchronize()
    if int(err.item()):
        raise RuntimeError(f"device error bits {int(err.item()):#x}")
    checked = None
    if not args.no_check:
        for a, b in zip(ins, outs):
            if not torch.equal(a, b):
                raise RuntimeError("round trip is not bit-exact")
        checked = True
        log("[bench] round trip bit-exact")
    table_bytes = int(tot.table_bytes)
    compressed = int(tot.raw_bytes + table_bytes + seek.numel() * 8 + payload_bytes + tot.crc_bytes)
    ratio = compressed / raw_in_bytes

    # timed region: K steps with nothing but the codec's launches in them
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(K):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K
    if int(err.item()):
        raise RuntimeError(f"device error bits {int(err.item()):#x}")
    # per-kernel times: K more steps with events between the kernels
    # (outside the timed region; the events add their own small gaps)
    torch.cuda.synchronize()
    t_ev0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    ms_step_events = (time.perf_counter() - t_ev0) * 1e3 / K
    if int(err.item()):
        raise RuntimeError(f"device error bits {int(err.item()):#x}")

    per_step = {s: [evs[i].elapsed_ms(j, j + 1) for i in range(K)] for j, s in enumerate(STAGES)}
    per_step["rans_decode"] = [evs[i].elapsed_ms(5, 6) for i in range(K)]
    stage_ms = {s: sum(per_step[s]) / K for s in STAGES}
    dec_ms = sum(per_step["rans_decode"]) / K
    enc_ms = sum(stage_ms.values())

    # algorithmic bytes (the minimum the method moves), per launch
    side = payload_bytes + table_bytes + 8 * (C + 1)
    raw_plane = int(tot.raw_bytes)
    # the raw plane is written by the encoder for the 16-bit layouts, by the
    # split pass for FP32 and FP8
    raw_by_encoder = layout not in ("fp32", "fp8e4m3", "fp8e5m2")
    alg = {
        "rans_decode": side + raw_plane + raw_in_bytes,           # read compressed + raw plane, write BF16
        "encode_total": raw_in_bytes + raw_plane + side,          # read BF16, write raw plane + compressed
        "split_hist": raw_in_bytes + table_bytes + (0 if raw_by_encoder else raw_plane),
        "rans_encode": raw_in_bytes + table_bytes + payload_bytes + (raw_plane if raw_by_encoder else 0),
        "compact": 2 * payload_bytes,
    }
    times = {"split_hist": stage_ms["split_hist"], "rans_encode": stage_ms["rans_encode"],
             "scan": stage_ms["scan"], "compact": stage_ms["compact"], "rans_decode": dec_ms}
    dominant = max(times, key=times.get)
    dom_bytes = alg.get(dominant, 0)
    dom_ms = times[dominant]
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9 if dom_ms > 0 else 0.0

    kernels = {}
    for k, t in times.items():
        entry = {"ms": round(t, 5), "ms_median": round(float(np.median(per_step[k])), 5),
                 "ms_min": round(min(per_step[k]), 5)}
        if k in alg and t > 0:
            entry["alg_GBps"] = round(alg[k] / (t / 1e3) / 1e9, 2)
            entry["hbm_frac"] = round(alg[k] / (t / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)
        kernels[k] = entry

    result = {
        "metric": "rANS decode/encode GB/s of BF16 weights + % HBM roofline; compression ratio",
        "value": round(raw_in_bytes / (ms_step / 1e3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_with_kernel_events": round(ms_step_events, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": w.name, "tensors": len(w.shapes), "elements": n,
                   "raw_bytes": raw_in_bytes, "chunks": C, "weights": w.dtype,
                   "layout": layout, "tensor_table": bool(args.tensor_table),
                   "raw_fallback": bool(args.raw_fallback), "crc32": bool(args.crc)},
        "ratio": round(ratio, 5),
        "round_trip_bit_exact": checked,
        "encode_GBps": round(raw_in_bytes / (enc_ms / 1e3) / 1e9, 3),
        "decode_GBps": round(raw_in_bytes / (dec_ms / 1e3) / 1e9, 3),
        "decode_hbm_frac": round(alg["rans_decode"] / (dec_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "encode_hbm_frac": round(alg["encode_total"] / (enc_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels": kernels,
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dominant, w.name), "alg_bytes": int(dom_bytes)},
    }
    # decode alone, warm (back to back) and cold (after a 1 GiB write that
    # evicts the 256 MB Infinity Cache and the L2s)
    if args.cold_reps > 0:
        flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
        dec_bufs = B.make_buffers(raw, tables, seek, payload, payload_bytes, crc)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        warm, cold = [], []
        for mode in ("warm", "cold"):
            for _ in range(args.cold_reps):
                if mode == "cold":
                    flush.fill_(1)
                ev[0].record(stream)
                B.wc_decode_batch(fmt, h_out, d_out, len(outs), dec_bufs, err, stream)
                ev[1].record(stream)
                torch.cuda.synchronize()
                (warm if mode == "warm" else cold).append(ev[0].elapsed_time(ev[1]))
        del flush
        if int(err.item()):
            raise RuntimeError(f"device error bits {int(err.item()):#x}")
        for mode, ts in (("warm", warm), ("cold", cold)):
            med = float(np.median(ts))
            result[f"decode_{mode}"] = {
                "ms_median": round(med, 5), "ms_min": round(min(ts), 5), "reps": len(ts),
                "hbm_frac_median": round(alg["rans_decode"] / (med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
    result["entropy"] = coded_plane_entropy(
        xs, tables.cpu().numpy().view(np.uint16)[: table_bytes // 2].reshape(-1, 256),
        seek.cpu().numpy().view(np.uint64), layout, args.tensor_table)

    # achievable bandwidth on this GPU: a plain device copy, 1 GiB each way
    # (larger than the 256 MB Infinity Cache), in the same run
    csrc = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(3)
    cdst = torch.empty_like(csrc)
    torch.add(csrc, 0, out=cdst)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    c0.record(stream)
    for _ in range(reps):
        torch.add(csrc, 0, out=cdst)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / reps
    result["copy_GBps"] = round(2 * csrc.numel() * 4 / (copy_ms / 1e3) / 1e9, 1)
    result["decode_vs_copy"] = round(alg["rans_decode"] / (dec_ms / 1e3) / 1e9 / result["copy_GBps"], 4)
    del csrc, cdst
    if args.copy_ref:
        src = torch.empty(COPY_REF_BYTES // 4, dtype=torch.int32, device=dev).fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 0, out=dst)  # the plain copy kernel of known size
        torch.cuda.synchronize()
        log(f"[bench] copy reference: {COPY_REF_BYTES} B read, {COPY_REF_BYTES} B written")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(w, xs, args.cpu_seconds, layout, opts)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
