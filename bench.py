#!/usr/bin/env python3
"""Encode & decode throughput of e4m3 entropy coding on one MI355X.

One step = the whole hot path over one synthetic shard, all on the GPU:
  byte_histogram (distribution monitor) -> pmf_kl against the calibration
  average -> for each codec of the workload: entropy_encode, entropy_decode.
The codebooks are built once from calibration shards before timing (the
single-stage design builds them off the critical path).

value = uncompressed bytes round-tripped per second (codecs x N / step time).
The timed steps record HIP events only around the dominant encode/decode
kernel (its average duration gives the roofline figure); the per-op
breakdown under "kernels" comes from an untimed pass with events around
every op, since each recorded event adds a few microseconds of queue time.

Prints ONE JSON line.  Options: --workload {ffn1,tiny_qlc,ffn2,grad,batch,bf16}.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode & decode GB/s (uncompressed e4m3) on 1 MI355X, % HBM roofline; compression %"
HBM_PEAK_GBPS = 8000.0

WORKLOAD_TEXT = {
    "tiny_qlc": "tiny base-scheme QLC: 2^20 e4m3 bytes, N(0,1), seed 0; codebook from a 2^20 calibration draw (seed 1)",
    "ffn1": "FFN1-activation-like shard 4096x16384 e4m3 (64 MiB): N(0,0.5^2) with 1% N(0,8^2) outliers, seed 2; "
            "codebooks from 8 calibration shards of 2^22 (seeds 100-107)",
    "ffn2": "FFN2-input-like shard 4096x16384 e4m3 (64 MiB): 0.25*GELU(N(0,1)), seed 3; calibration seeds 100-107",
    "grad": "gradient-like shard 2048x16384 e4m3 (32 MiB): Laplace(0,0.02)*2^(6+e) per 128 block, seed 4; "
            "calibration seeds 100-107",
    "batch": "64 shards x 4 MiB FFN1-like e4m3 (256 MiB), sigma~U(0.4,0.6), seeds 1000-1063",
    "bf16": "BF16 exponent coding (seven frequent exponents in 3-bit codes, the rest escaped): 2^25 BF16 values "
            "(64 MiB) of N(0, 0.02^2), seed 5, chunks of 16384 values, table from sigma",
}
CODECS = {
    "tiny_qlc": ["qlc"],
    "ffn1": ["qlc", "huffman"],
    "ffn2": ["qlc_adapted", "qlc", "qlc_opt", "huffman"],
    "grad": ["eg", "qlc", "qlc_opt", "huffman"],
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="ffn1", choices=list(WORKLOAD_TEXT))
    p.add_argument("--sets", type=int, default=3, help="buffer sets rotated per step (defeats the 256 MB MALL)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--copy-ref", action="store_true", help="also run plain device copies (counter calibration)")
    p.add_argument("--verbose", action="store_true")
    return p.parse_args()


def log(args, *a):
    if args.verbose:
        print(*a, file=sys.stderr, flush=True)


def make_codebook(ec, name, counts):
    if name == "qlc":
        return ec.Codebook.qlc(counts)
    if name == "qlc_adapted":
        return ec.Codebook.qlc(counts, *ec.QLC_ADAPTED)
    if name == "qlc_opt":   # the cheapest layout with four code lengths
        return ec.Codebook.qlc(counts, *ec.qlc_optimal_area_layout(counts, 4))
    if name == "huffman":
        return ec.Codebook.huffman(counts)
    if name == "eg":
        return ec.Codebook.exp_golomb(counts, -1)
    raise KeyError(name)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "lossless_entropy_coding_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file, workload, op):
    """Measured HBM bytes per launch from a committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    cur = source_hash(kernel_file)
    for line in open(path):
        m = re.match(r"^traffic\s+(\S+)\s+src=(\S+)\s+bytes=(\d+)", line)
        if m and m.group(1) == op and m.group(2) == cur:
            return int(m.group(3))
    return None


# ---------------------------------------------------------------- CPU leg

def cpu_baseline(x, counts, codec_names, chunk, calib_rows):
    """The oracle as it stands (single-threaded C + Python), timed on the
    host over the same step on the same shard."""
    from oracle import codebooks as cbm
    from oracle import stats
    from oracle import stream as st
    builders = {
        "qlc": lambda c: cbm.qlc_codebook(c),
        "qlc_adapted": lambda c: cbm.qlc_codebook(c, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX),
        "qlc_opt": lambda c: cbm.qlc_codebook(c, *cbm.qlc_optimal_areas(c, 4)),
        "huffman": lambda c: cbm.huffman_codebook(c),
        "eg": lambda c: cbm.eg_codebook(c),
    }
    cbs = [builders[n](counts) for n in codec_names]
    t0 = time.perf_counter()
    h = stats.histogram(x)
    stats.kl_bits(h, counts, q_add=1)
    for cb in cbs:
        s = st.encode_stream(x, cb, chunk)
        y = st.decode_stream(s, cb)
        assert np.array_equal(y, x)
    dt = time.perf_counter() - t0
    return dict(value=round(len(codec_names) * x.size / dt / 1e9, 5), unit="GB/s", cores=1, kind="oracle",
                sample="one full step on the same %d-byte shard (histogram, KL, %s encode+decode), "
                       "single-threaded, %.1f s, host %s" % (x.size, "/".join(codec_names), dt,
                                                             platform.processor() or platform.machine()))


# ---------------------------------------------------------------- GPU leg

def run_single(args, ec, torch):
    import synth
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    codec_names = CODECS[args.workload]
    C = w.chunk_symbols
    t = time.perf_counter()
    x = synth.workload(args.workload)
    calib = synth.calibration_shards(args.workload)
    log(args, "data %.1f s, sha256 %s" % (time.perf_counter() - t, synth.sha256(x)[:16]))
    N = x.size

    # calibration (off the critical path): GPU histograms, host codebook build
    calib_d = torch.from_numpy(calib).to(dev)
    rows_d = ec.byte_histogram(calib_d)
    pooled_d = ec.byte_histogram(calib_d.view(-1))[0]
    avg_pmf_d = ec.pmf_average(rows_d)
    torch.cuda.synchronize()
    counts = [int(c) for c in pooled_d.cpu().numpy().astype(np.uint64)]
    t = time.perf_counter()
    cbs = [make_codebook(ec, n, counts) for n in codec_names]
    build_us = (time.perf_counter() - t) * 1e6
    del calib_d

    x_d = torch.from_numpy(x).to(dev)
    sets = []
    for i in range(args.sets):
        xi = x_d if i == 0 else x_d.clone()
        bufs = []
        for cb in cbs:
            cap = ec.max_encoded_bytes(cb, N, C)
            bufs.append(dict(s=torch.empty(cap, dtype=torch.uint8, device=dev),
                             y=torch.empty(N, dtype=torch.uint8, device=dev),
                             n=torch.zeros(1, dtype=torch.int64, device=dev)))
        sets.append(dict(x=xi, bufs=bufs, hist=torch.empty((1, 256), dtype=torch.int64, device=dev),
                         kl=torch.empty(1, dtype=torch.float32, device=dev)))
    status = torch.zeros(2 * len(cbs), dtype=torch.int32, device=dev)
    nops = 2 + 2 * len(cbs)

    op_names = ["byte_histogram", "pmf_kl"]
    for n in codec_names:
        op_names += ["%s_encode" % n, "%s_decode" % n]

    def step(S, events=None, only=None):
        # events[k] is recorded before op k (and events[nops] after the last
        # op); with `only`, just the two events around op `only`
        def rec(k):
            if events is not None and (only is None or k in (only, only + 1)):
                events[k].record()
        rec(0)
        ec.byte_histogram(S["x"], out=S["hist"])
        rec(1)
        ec.pmf_kl(S["hist"], pooled_d, q_add=1, out=S["kl"])
        rec(2)
        for j, cb in enumerate(cbs):
            B = S["bufs"][j]
            ec.encode(cb, S["x"], C, out=B["s"], out_len=B["n"], status=status[2 * j:2 * j + 1])
            rec(3 + 2 * j)
            ec.decode(cb, B["s"], N, out=B["y"], status=status[2 * j + 1:2 * j + 2], in_len=B["s"].numel())
            rec(4 + 2 * j)

    def new_events():
        return [[torch.cuda.Event(enable_timing=True) for _ in range(nops + 1)] for _ in range(args.steps)]

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # per-op breakdown: an untimed pass with events around every op (each
    # event costs a few microseconds of queue time, so the timed steps below
    # record only the two around the dominant kernel)
    evs = new_events()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    per_op = {o: [e[k].elapsed_time(e[k + 1]) * 1e3 for e in evs] for k, o in enumerate(op_names)}   # us
    dominant = max((o for o in op_names if o.endswith("code")), key=lambda o: statistics.mean(per_op[o]))
    dom_k = op_names.index(dominant)

    # the timed steps
    evs = new_events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i], only=dom_k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_us = [e[dom_k].elapsed_time(e[dom_k + 1]) * 1e3 for e in evs]

    if args.copy_ref:   # plain copies of N bytes, for the hardware-counter scale factor
        dst = torch.empty_like(x_d)
        for _ in range(5):
            dst.copy_(sets[-1]["x"])
        torch.cuda.synchronize()

    # correctness of what was timed
    st = status.cpu().numpy()
    if st.any():
        raise SystemExit("device status bits set: %s" % st)
    for S in sets:
        for B in S["bufs"]:
            if not torch.equal(B["y"], S["x"]):
                raise SystemExit("round trip mismatch")
    hist_ok = np.array_equal(sets[0]["hist"].cpu().numpy()[0], np.bincount(x, minlength=256))

    stream_len = [int(B["n"].item()) for B in sets[0]["bufs"]]
    kernels = {}
    for o in op_names:
        us = statistics.mean(per_op[o])
        d = dict(us=round(us, 2), us_median=round(statistics.median(per_op[o]), 2))
        if o == "byte_histogram":
            moved = N + 256 * 8
        elif o.endswith("_encode") or o.endswith("_decode"):
            j = codec_names.index(o.rsplit("_", 1)[0])
            moved = N + stream_len[j]
        else:
            moved = 2 * 256 * 8
        d["GBps_uncompressed"] = round(N / us / 1e3, 1) if o != "pmf_kl" else None
        d["hbm_GBps"] = round(moved / us / 1e3, 1)
        d["roofline_frac"] = round(moved / us / 1e3 / HBM_PEAK_GBPS, 4)
        kernels[o] = d

    compression = {}
    idx = ec.index_bytes(N, C)
    for j, n in enumerate(codec_names):
        payload = stream_len[j] - idx
        compression[n] = dict(stream_bytes=stream_len[j], payload_pct=round(100 * (1 - payload / N), 3),
                              stream_pct=round(100 * (1 - stream_len[j] / N), 3),
                              max_code_len=cbs[j].max_len)
        if n == "qlc_opt":
            compression[n]["layout"] = ec.qlc_optimal_area_layout(counts, 4)

    ms_per_step = wall / args.steps * 1e3
    value = len(codec_names) * N / (wall / args.steps) / 1e9
    j = codec_names.index(dominant.rsplit("_", 1)[0])
    moved = N + stream_len[j]
    kfile = "decode.hip" if dominant.endswith("decode") else "encode.hip"
    traffic = load_traffic(kfile, args.workload, dominant)
    avg_us = statistics.mean(dom_us)   # measured inside the timed steps
    roofline = dict(kernel=dominant, bound="hbm", achieved=round(moved / avg_us / 1e3, 1),
                    peak=HBM_PEAK_GBPS, unit="GB/s", frac=round(moved / avg_us / 1e3 / HBM_PEAK_GBPS, 4),
                    traffic=traffic, algorithmic_bytes=moved, avg_us=round(avg_us, 2))

    kl = float(sets[0]["kl"].item())
    out = dict(metric=METRIC, value=round(value, 2), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="u8", data="synthetic",
               config=dict(workload=WORKLOAD_TEXT[args.workload], name=args.workload, n_bytes=N, chunk_symbols=C,
                           codecs=codec_names, buffer_sets=args.sets,
                           step="byte_histogram + pmf_kl + per codec entropy_encode + entropy_decode"),
               roofline=roofline, kernels=kernels,
               kernels_note="per-op event times from an untimed pass with events around every op",
               compression=compression,
               extra=dict(kl_bits_vs_calibration=kl, histogram_exact=hist_ok, codebook_build_us=round(build_us, 1),
                          avg_pmf_top=float(avg_pmf_d.max().item()), numpy=np.__version__,
                          input_sha256=synth.sha256(x)[:16]))
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x, counts, codec_names, C, None)
    else:
        out["cpu_baseline"] = None
    return out


def run_batch(args, ec, torch):
    """64 x 4 MiB shards: single-stage (one fixed avg-PMF Huffman codebook)
    against three-stage (per-shard histogram, per-shard codebook, codebook
    lengths embedded in each stream), the codebooks built on the GPU
    (three_stage) or on the host after a copy of the histograms
    (three_stage_host)."""
    import synth
    dev = torch.device("cuda:0")
    C = 16384
    t = time.perf_counter()
    x = synth.batch_shards(64, 1 << 22)
    calib = synth.calibration_shards("ffn1")
    log(args, "data %.1f s" % (time.perf_counter() - t))
    S, n = x.shape
    x_d = torch.from_numpy(x).to(dev)
    pooled_d = ec.byte_histogram(torch.from_numpy(calib).to(dev).view(-1))[0]
    torch.cuda.synchronize()
    counts = [int(c) for c in pooled_d.cpu().numpy()]
    fixed = ec.Codebook.huffman(counts)
    stride = max(ec.max_encoded_bytes(fixed, n, C, True), ec.own_max_encoded_bytes(n, C, True))
    stride = (stride + 255) // 256 * 256 + 4096
    out = torch.empty((S, stride), dtype=torch.uint8, device=dev)
    y = torch.empty((S, n), dtype=torch.uint8, device=dev)
    lens = torch.zeros(S, dtype=torch.int64, device=dev)
    status = torch.zeros(S, dtype=torch.int32, device=dev)
    hist = torch.empty((S, 256), dtype=torch.int64, device=dev)
    kl = torch.empty(S, dtype=torch.float32, device=dev)
    tables = torch.empty((S, ec.device_codebook_bytes()), dtype=torch.uint8, device=dev)
    rtables = torch.empty_like(tables)

    def single():
        ec.byte_histogram(x_d, out=hist)
        ec.pmf_kl(hist, pooled_d, q_add=1, out=kl)
        ec.encode_batch(fixed, x_d, C, out=out, out_len=lens, status=status)
        ec.decode_batch(fixed, out, n, out=y, status=status)

    def three():
        ec.byte_histogram(x_d, out=hist)                                  # frequency analysis
        ec.build_huffman_device(hist, out=tables, status=status)          # codebook generation
        ec.encode_batch_device(tables, x_d, C, embed_lengths=True, out=out, out_len=lens, status=status)
        # the receiver rebuilds each codebook from the lengths its stream carries
        ec.huffman_tables_from_streams(out, out=rtables, status=status)
        ec.decode_batch_device(rtables, out, n, out=y, status=status)

    def three_host():
        ec.byte_histogram(x_d, out=hist)
        h = hist.cpu().numpy()          # histograms -> host
        cbs = [ec.Codebook.huffman([int(c) for c in row]) for row in h]
        ec.encode_batch(cbs, x_d, C, embed_lengths=True, out=out, out_len=lens, status=status)
        ec.decode_batch(cbs, out, n, out=y, status=status)
        return cbs

    res = {}
    for name, fn in (("single_stage", single), ("three_stage", three), ("three_stage_host", three_host)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            keep = fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        if status.cpu().numpy().any() or not torch.equal(y, x_d):
            raise SystemExit("batch round trip failed (%s)" % name)
        L = lens.cpu().numpy()
        res[name] = dict(ms_per_step=round(dt * 1e3, 4), GBps=round(S * n / dt / 1e9, 2),
                         stream_pct=round(100 * (1 - L.sum() / (S * n)), 3))
        del keep
    klv = kl.cpu().numpy()
    value = res["single_stage"]["GBps"]
    return dict(metric=METRIC, value=value, unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=res["single_stage"]["ms_per_step"], higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="u8", data="synthetic",
                config=dict(workload=WORKLOAD_TEXT["batch"], name="batch", n_bytes=S * n, chunk_symbols=C,
                            codecs=["huffman"], step="histogram + KL + batch encode + batch decode"),
                paths=res, kl_bits=dict(min=float(klv.min()), max=float(klv.max()), mean=float(klv.mean())),
                roofline=None, cpu_baseline=None)


def run_bf16(args, ec, torch):
    """BF16 exponent coding: one step = bf16_exp_encode + bf16_exp_decode of
    one 64 MiB tensor."""
    import synth
    dev = torch.device("cuda:0")
    w = synth.BF16_WORKLOAD
    n, chunk = w["n"], w["chunk"]
    x = synth.bf16_draw(w["seed"], n, w["sigma"])
    table = ec.bf16_exp_table_from_sigma(w["sigma"])
    x_d = torch.from_numpy(x.view(np.int16)).to(dev)
    sets = []
    for i in range(args.sets):
        sets.append(dict(x=x_d if i == 0 else x_d.clone(),
                         s=torch.empty(ec.bf16_exp_max_encoded_bytes(n, chunk), dtype=torch.uint8, device=dev),
                         y=torch.empty(n, dtype=torch.bfloat16, device=dev),
                         n=torch.zeros(1, dtype=torch.int64, device=dev)))
    status = torch.zeros(2, dtype=torch.int32, device=dev)

    def step(S, ev=None):
        if ev:
            ev[0].record()
        ec.bf16_exp_encode(table, S["x"], chunk, out=S["s"], out_len=S["n"], status=status[0:1])
        if ev:
            ev[1].record()
        ec.bf16_exp_decode(S["s"], n, out=S["y"], status=status[1:2])
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    enc_us = statistics.mean(e[0].elapsed_time(e[1]) * 1e3 for e in evs)
    dec_us = statistics.mean(e[1].elapsed_time(e[2]) * 1e3 for e in evs)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.copy_ref:   # plain copies of the input, for the hardware-counter scale factor
        dst = torch.empty_like(x_d)
        for _ in range(5):
            dst.copy_(sets[-1]["x"])
        torch.cuda.synchronize()
    if status.cpu().numpy().any():
        raise SystemExit("device status bits set: %s" % status.cpu().numpy())
    for S in sets:
        if not torch.equal(S["y"].view(torch.int16), S["x"]):
            raise SystemExit("bf16 round trip mismatch")
    L = int(sets[0]["n"].item())
    moved = 2 * n + L
    dom, dom_us = ("bf16_exp_decode", dec_us) if dec_us >= enc_us else ("bf16_exp_encode", enc_us)
    kernels = {o: dict(us=round(u, 2), GBps_uncompressed=round(2 * n / u / 1e3, 1),
                       roofline_frac=round(moved / u / 1e3 / HBM_PEAK_GBPS, 4))
               for o, u in (("bf16_exp_encode", enc_us), ("bf16_exp_decode", dec_us))}
    return dict(metric=METRIC, value=round(2 * n / (wall / args.steps) / 1e9, 2), unit="GB/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=round(wall / args.steps * 1e3, 4),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="u16", data="synthetic",
                config=dict(workload=WORKLOAD_TEXT["bf16"], name="bf16", n_bytes=2 * n, chunk_values=chunk,
                            table=list(table), step="bf16_exp_encode + bf16_exp_decode"),
                roofline=dict(kernel=dom, bound="hbm", achieved=round(moved / dom_us / 1e3, 1), peak=HBM_PEAK_GBPS,
                              unit="GB/s", frac=round(moved / dom_us / 1e3 / HBM_PEAK_GBPS, 4),
                              traffic=load_traffic("bf16exp.hip", "bf16", dom),
                              algorithmic_bytes=moved, avg_us=round(dom_us, 2)),
                kernels=kernels, compression=dict(stream_bytes=L, stream_pct=round(100 * (1 - L / (2 * n)), 3)),
                cpu_baseline=None)


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py: this engine runs on one GPU; --gpus %d is not supported (multi-GPU sharding is a "
              "design note only)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import lossless_entropy_coding_amd as ec
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    ec.lib()
    if args.workload == "batch":
        out = run_batch(args, ec, torch)
    elif args.workload == "bf16":
        out = run_bf16(args, ec, torch)
    else:
        out = run_single(args, ec, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
