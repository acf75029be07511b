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

With no --workload the headline is the 64 MiB FFN1-like shard and
extra.configs carries every workload: the tiny base-scheme QLC case, FFN1,
FFN2, the gradient shard and the 64 x 4 MiB batch (single-stage and
three-stage paths), each with per-op times, a roofline object and the CPU
oracle timed on one core and on all cores.  A plain 64 MiB device copy is
timed in the same run as the practical bandwidth ceiling.

All host-side work (synthetic data, CPU oracle legs) runs before the GPU is
first touched, so the process pools fork from a process without GPU state.

Prints ONE JSON line.  --workload NAME runs just that workload (profiling).
"""

from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import multiprocessing as mp
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
CONFIG_ORDER = ["tiny_qlc", "ffn1", "ffn2", "grad", "batch"]
HEADLINE = "ffn1"
BATCH_SHARDS, BATCH_SHARD_N, BATCH_CHUNK = 64, 1 << 22, 16384

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
    "batch": ["huffman"],
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None, choices=list(WORKLOAD_TEXT),
                   help="run only this workload (default: headline FFN1 plus every workload under extra.configs)")
    p.add_argument("--extra-steps", type=int, default=20, help="timed steps per workload under extra.configs")
    p.add_argument("--sets", type=int, default=3, help="buffer sets rotated per step (defeats the 256 MB MALL)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baselines")
    p.add_argument("--cpu-workers", type=int, default=0,
                   help="processes for the all-core oracle leg (default: OMP_NUM_THREADS, else the CPUs this "
                        "process may run on)")
    p.add_argument("--copy-ref", action="store_true",
                   help="accepted for older recorded commands; the 64 MiB copy now runs in every run")
    p.add_argument("--verbose", action="store_true")
    return p.parse_args()


def log(args, *a):
    if args.verbose:
        print(*a, file=sys.stderr, flush=True)


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


def roofline_obj(kernel, moved, avg_us, traffic, copy_gbps):
    achieved = moved / avg_us / 1e3
    return dict(kernel=kernel, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=traffic, algorithmic_bytes=moved,
                avg_us=round(avg_us, 2), copy_ceiling_GBps=copy_gbps,
                frac_of_copy=round(achieved / copy_gbps, 4) if copy_gbps else None)


@contextlib.contextmanager
def fork_pool(n):
    """A fork pool whose workers leave on their own (close, then join) rather
    than by SIGTERM: under rocprofv3 a forked worker carries the profiler's
    signal handler, and a worker terminated by signal can hang in it, which
    leaves the parent waiting forever in the pool's shutdown."""
    pool = mp.get_context("fork").Pool(n)
    try:
        yield pool
        pool.close()
    except BaseException:
        pool.terminate()
        raise
    finally:
        pool.join()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_workers(args):
    if args.cpu_workers > 0:
        return args.cpu_workers
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


# ---------------------------------------------------------------- host data

def _gen(task):
    import synth
    kind = task[0]
    if kind == "x":
        return synth.workload(task[1])
    if kind == "calib":                     # one calibration shard of a workload
        w = synth.WORKLOADS[task[1]]
        return synth.draw(w.calib_recipe, task[2], w.calib_n)
    if kind == "batch":                     # one shard of the multi-shard batch
        return synth.batch_shards(1, BATCH_SHARD_N, first_seed=1000 + task[1])[0]
    if kind == "bf16":
        w = synth.BF16_WORKLOAD
        return synth.bf16_draw(w["seed"], w["n"], w["sigma"])
    raise KeyError(kind)


def make_data(names, workers):
    """Synthetic inputs of the named workloads, drawn in a process pool."""
    import synth
    tasks = []
    for n in names:
        if n == "batch":
            tasks += [("batch", i) for i in range(BATCH_SHARDS)]
            tasks += [("calib", "ffn1", s) for s in synth.WORKLOADS["ffn1"].calib_seeds]
        elif n == "bf16":
            tasks.append(("bf16",))
        else:
            tasks.append(("x", n))
            tasks += [("calib", n, s) for s in synth.WORKLOADS[n].calib_seeds]
    # the long draws first, so they do not end up last on one worker
    order = sorted(range(len(tasks)), key=lambda i: tasks[i][0] not in ("x", "bf16"))
    with fork_pool(min(workers, len(tasks))) as pool:
        got = pool.map(_gen, [tasks[i] for i in order], chunksize=1)
    res = dict(zip([tasks[i] for i in order], got))
    data = {}
    for n in names:
        if n == "batch":
            data[n] = dict(x=np.stack([res[("batch", i)] for i in range(BATCH_SHARDS)]),
                           calib=np.stack([res[("calib", "ffn1", s)] for s in synth.WORKLOADS["ffn1"].calib_seeds]))
        elif n == "bf16":
            data[n] = dict(x=res[("bf16",)])
        else:
            data[n] = dict(x=res[("x", n)],
                           calib=np.stack([res[("calib", n, s)] for s in synth.WORKLOADS[n].calib_seeds]))
    return data


# ---------------------------------------------------------------- CPU leg
#
# The oracle as it stands: plain Python around the bit-serial C encoder and
# decoder.  Single core: one process over a bounded sample of the shard.
# All cores: the shard split into contiguous ranges of whole chunks (whole
# shards for the batch), one process per range, each running the same step
# on its range as a stream of its own; the wall time is the slowest range.

_CPU = {}


def _oracle_codebook(name, counts):
    from oracle import codebooks as cbm
    if name == "qlc":
        return cbm.qlc_codebook(counts)
    if name == "qlc_adapted":
        return cbm.qlc_codebook(counts, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX)
    if name == "qlc_opt":
        return cbm.qlc_codebook(counts, *cbm.qlc_optimal_areas(counts, 4))
    if name == "huffman":
        return cbm.huffman_codebook(counts)
    if name == "eg":
        return cbm.eg_codebook(counts)
    raise KeyError(name)


def _cpu_step(name, lo, hi):
    """One step of the oracle over bytes [lo, hi) of a workload (over shards
    [lo, hi) for the batch); returns its duration in seconds."""
    from oracle import stats
    from oracle import stream as st
    d = _CPU[name]
    t0 = time.perf_counter()
    parts = [d["x"][i] for i in range(lo, hi)] if name == "batch" else [d["x"][lo:hi]]
    for x in parts:
        h = stats.histogram(x)
        stats.kl_bits(h, d["counts"], q_add=1)
        for cb in d["cbs"]:
            s = st.encode_stream(x, cb, d["chunk"])
            if not np.array_equal(st.decode_stream(s, cb), x):
                raise RuntimeError("oracle round trip failed (%s)" % name)
    return time.perf_counter() - t0


def cpu_baselines(data, names, workers, sample_bytes=8 << 20):
    """{workload: cpu_baseline object}: one core over a bounded sample, all
    cores over the whole shard."""
    import synth
    from oracle import _clib, stats
    _clib.lib()                       # load the C core once, before the fork
    plan = {}
    for n in names:
        d = data[n]
        counts = [int(c) for c in stats.histogram(d["calib"].reshape(-1))]
        chunk = BATCH_CHUNK if n == "batch" else synth.WORKLOADS[n].chunk_symbols
        _CPU[n] = dict(x=d["x"], counts=counts, chunk=chunk,
                       cbs=[_oracle_codebook(c, counts) for c in CODECS[n]])
        if n == "batch":
            units, unit_bytes = BATCH_SHARDS, BATCH_SHARD_N
        else:
            units, unit_bytes = d["x"].size // chunk, chunk
            if d["x"].size % chunk:
                units += 1
        plan[n] = (units, unit_bytes)
    out = {}
    model = cpu_model()
    with fork_pool(workers) as pool:
        for n in names:
            units, ub = plan[n]
            N = data[n]["x"].size
            k = len(CODECS[n])
            # one core, bounded sample (whole chunks / shards from the start)
            s_units = max(1, min(units, sample_bytes // ub))
            hi = s_units if n == "batch" else min(N, s_units * ub)
            one = _cpu_step(n, 0, hi)
            s_bytes = s_units * ub if n == "batch" else hi
            # all cores, whole workload
            P = min(workers, units)
            cuts = [units * i // P for i in range(P + 1)]
            ranges = [(n, cuts[i], cuts[i + 1]) if n == "batch" else
                      (n, cuts[i] * ub, min(N, cuts[i + 1] * ub)) for i in range(P)]
            t0 = time.perf_counter()
            pool.starmap(_cpu_step, ranges, chunksize=1)
            wall = time.perf_counter() - t0
            out[n] = dict(
                value=round(k * N / wall / 1e9, 5), unit="GB/s", cores=P, kind="oracle",
                sample="the whole %d-byte workload, one step (histogram, KL, %s encode+decode) split over %d "
                       "processes by contiguous %s; wall %.2f s; CPU %s"
                       % (N, "/".join(CODECS[n]), P, "shards" if n == "batch" else "chunk ranges", wall, model),
                one_core=dict(value=round(k * s_bytes / one / 1e9, 5), unit="GB/s", cores=1,
                              sample="the first %d bytes, one step, %.2f s" % (s_bytes, one)),
                cpu_model=model)
    _CPU.clear()
    return out


# ---------------------------------------------------------------- GPU legs

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


class GpuEvent:
    """A HIP event recorded on torch's current stream (the stream every
    library call here runs on), created without the system-scope fence
    (hipEventDisableSystemFence).  torch.cuda.Event records with that fence:
    each record then held the GPU idle for about 5 us between two kernels in
    the profiled steps, which the timed step would count."""
    _hip = None
    _flags = 0x20000000   # hipEventDisableSystemFence (timing stays enabled)

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            import ctypes
            import lossless_entropy_coding_amd as ec
            ec.lib()
            rts = [p for p in ec._hip_runtimes_mapped() if os.path.exists(p)]
            if len(rts) != 1:
                raise SystemExit("expected one mapped HIP runtime, found %s" % rts)
            h = ctypes.CDLL(rts[0])   # the runtime torch and libec already use
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._e = ctypes.c_void_p()
        if self._rt().hipEventCreateWithFlags(ctypes.byref(self._e), self._flags) != 0:
            raise SystemExit("hipEventCreateWithFlags failed")

    def record(self):
        import lossless_entropy_coding_amd as ec
        if self._rt().hipEventRecord(self._e, ec._stream(None)) != 0:   # torch's current stream
            raise SystemExit("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        if self._rt().hipEventElapsedTime(ctypes.byref(ms), self._e, end._e) != 0:
            raise SystemExit("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._e:
            self._hip.hipEventDestroy(self._e)


def ev_us(a, b):
    return a.elapsed_time(b) * 1e3


def copy_ceiling(torch, x_d, reps=30, pairs=3):
    """Plain device-to-device copies of x_d's size (read N, write N),
    rotating over `pairs` source/destination pairs so that the working set
    (pairs x 2N) exceeds the 256 MB last-level cache: mean event time and
    GB/s moved."""
    srcs = [x_d] + [x_d.clone() for _ in range(pairs - 1)]
    dsts = [torch.empty_like(x_d) for _ in range(pairs)]
    for i in range(2 * pairs):
        dsts[i % pairs].copy_(srcs[i % pairs])
    torch.cuda.synchronize()
    evs = [(GpuEvent(), GpuEvent()) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        dsts[i % pairs].copy_(srcs[i % pairs])
        b.record()
    torch.cuda.synchronize()
    if not all(torch.equal(d, x_d) for d in dsts):
        raise SystemExit("device copy mismatch")
    us = statistics.mean(ev_us(a, b) for a, b in evs)
    nb = x_d.numel() * x_d.element_size()
    return dict(bytes=nb, us=round(us, 2), GBps=round(2 * nb / us / 1e3, 1), buffer_pairs=pairs)


def run_single(name, d, args, ec, torch, steps, warmup, copy_gbps):
    import synth
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    codec_names = CODECS[name]
    C = w.chunk_symbols
    x, calib = d["x"], d["calib"]
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
    # one read of the input per encode: the histogram's pass also sizes every
    # codec's chunks (the codebooks are fixed before the data is seen), when
    # the shapes allow it
    n_chunks = (N + C - 1) // C
    try:
        _, sz = ec.byte_histogram_sized(x_d, cbs, C)
        for j, cb in enumerate(cbs):
            ec.encode_sized(cb, x_d, C, sz[j, 0])
        one_read = True
    except ec.ECError:
        one_read = False
    torch.cuda.synchronize()
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
                         kl=torch.empty(1, dtype=torch.float32, device=dev),
                         sizes=torch.empty((len(cbs), 1, max(n_chunks, 1)), dtype=torch.int32, device=dev)))
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
        if one_read:
            ec.byte_histogram_sized(S["x"], cbs, C, out=S["hist"], sizes=S["sizes"])
        else:
            ec.byte_histogram(S["x"], out=S["hist"])
        rec(1)
        ec.pmf_kl(S["hist"], pooled_d, q_add=1, out=S["kl"])
        rec(2)
        for j, cb in enumerate(cbs):
            B = S["bufs"][j]
            if one_read:
                ec.encode_sized(cb, S["x"], C, S["sizes"][j, 0], out=B["s"], out_len=B["n"],
                                status=status[2 * j:2 * j + 1])
            else:
                ec.encode(cb, S["x"], C, out=B["s"], out_len=B["n"], status=status[2 * j:2 * j + 1])
            rec(3 + 2 * j)
            ec.decode(cb, B["s"], N, out=B["y"], status=status[2 * j + 1:2 * j + 2], in_len=B["s"].numel())
            rec(4 + 2 * j)

    def new_events():
        return [[GpuEvent() for _ in range(nops + 1)] for _ in range(steps)]

    for i in range(warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # per-op breakdown: an untimed pass with events around every op (each
    # event costs a few microseconds of queue time, so the timed steps below
    # record only the two around the dominant kernel)
    evs = new_events()
    for i in range(steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    per_op = {o: [ev_us(e[k], e[k + 1]) for e in evs] for k, o in enumerate(op_names)}
    dominant = max((o for o in op_names if o.endswith("code")), key=lambda o: statistics.mean(per_op[o]))
    dom_k = op_names.index(dominant)

    # the timed steps
    evs = new_events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % len(sets)], evs[i], only=dom_k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_us = [ev_us(e[dom_k], e[dom_k + 1]) for e in evs]

    # correctness of what was timed
    st = status.cpu().numpy()
    if st.any():
        raise SystemExit("device status bits set (%s): %s" % (name, st))
    for S in sets:
        for B in S["bufs"]:
            if not torch.equal(B["y"], S["x"]):
                raise SystemExit("round trip mismatch (%s)" % name)
    # the two-pass entropy_encode (a sizing read, then the packer), for
    # reference: its streams equal the timed ones
    two_pass = {}
    if one_read:
        S = sets[0]
        for j, cb in enumerate(cbs):
            B = S["bufs"][j]
            ref, ref_len, _ = ec.encode(cb, S["x"], C)
            evs2 = [(GpuEvent(), GpuEvent()) for _ in range(steps)]
            for a, b in evs2:
                a.record()
                ec.encode(cb, S["x"], C, out=ref, out_len=ref_len)
                b.record()
            torch.cuda.synchronize()
            L = int(ref_len.item())
            if L != int(B["n"].item()) or not torch.equal(ref[:L], B["s"][:L]):
                raise SystemExit("two-pass and one-read streams differ (%s)" % name)
            two_pass[codec_names[j]] = round(statistics.mean(ev_us(a, b) for a, b in evs2), 2)
    hist_ok = np.array_equal(sets[0]["hist"].cpu().numpy()[0], np.bincount(x, minlength=256))

    stream_len = [int(B["n"].item()) for B in sets[0]["bufs"]]
    kernels = {}
    for o in op_names:
        us = statistics.mean(per_op[o])
        dd = dict(us=round(us, 2), us_median=round(statistics.median(per_op[o]), 2))
        if o == "byte_histogram":
            moved = N + 256 * 8
        elif o.endswith("_encode") or o.endswith("_decode"):
            j = codec_names.index(o.rsplit("_", 1)[0])
            moved = N + stream_len[j]
        else:
            moved = 2 * 256 * 8
        dd["GBps_uncompressed"] = round(N / us / 1e3, 1) if o != "pmf_kl" else None
        dd["hbm_GBps"] = round(moved / us / 1e3, 1)
        dd["roofline_frac"] = round(moved / us / 1e3 / HBM_PEAK_GBPS, 4)
        kernels[o] = dd

    compression = {}
    idx = ec.index_bytes(N, C)
    for j, n in enumerate(codec_names):
        payload = stream_len[j] - idx
        compression[n] = dict(stream_bytes=stream_len[j], payload_pct=round(100 * (1 - payload / N), 3),
                              stream_pct=round(100 * (1 - stream_len[j] / N), 3),
                              max_code_len=cbs[j].max_len)
        if n == "qlc_opt":
            compression[n]["layout"] = ec.qlc_optimal_area_layout(counts, 4)

    j = codec_names.index(dominant.rsplit("_", 1)[0])
    kfile = "decode.hip" if dominant.endswith("decode") else "encode.hip"
    roofline = roofline_obj(dominant, N + stream_len[j], statistics.mean(dom_us),
                            load_traffic(kfile, name, dominant), copy_gbps)
    res = dict(value=round(len(codec_names) * N / (wall / steps) / 1e9, 2), unit="GB/s", steps=steps,
               warmup=warmup, ms_per_step=round(wall / steps * 1e3, 4), n_bytes=N, chunk_symbols=C,
               codecs=codec_names, workload=WORKLOAD_TEXT[name],
               step=("byte_histogram_sized (the histogram's read also sizes every codec's chunks) + pmf_kl + per "
                     "codec entropy_encode_sized (reads the input once) + entropy_decode" if one_read else
                     "byte_histogram + pmf_kl + per codec entropy_encode + entropy_decode"),
               two_pass_encode_us=two_pass or None,
               roofline=roofline, kernels=kernels, compression=compression,
               kl_bits_vs_calibration=float(sets[0]["kl"].item()), histogram_exact=hist_ok,
               codebook_build_us=round(build_us, 1), avg_pmf_top=float(avg_pmf_d.max().item()))
    return res


def run_batch(d, args, ec, torch, steps, warmup, copy_gbps):
    """64 x 4 MiB shards: single-stage (one fixed avg-PMF Huffman codebook)
    against three-stage (per-shard histogram, per-shard codebook, codebook
    lengths embedded in each stream), the codebooks built on the GPU
    (three_stage) or on the host after a copy of the histograms
    (three_stage_host)."""
    dev = torch.device("cuda:0")
    C = BATCH_CHUNK
    x, calib = d["x"], d["calib"]
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

    # each path is a list of (op name, callable); the host path's codebook
    # build is one op that includes the copy of the histograms to the host
    # single stage: the histogram's read also sizes the fixed codebook's chunks
    bsizes = torch.empty((1, S, (n + C - 1) // C), dtype=torch.int32, device=dev)
    single = [("byte_histogram", lambda: ec.byte_histogram_sized(x_d, [fixed], C, out=hist, sizes=bsizes)),
              ("pmf_kl", lambda: ec.pmf_kl(hist, pooled_d, q_add=1, out=kl)),
              ("huffman_encode_batch", lambda: ec.encode_batch_sized(fixed, x_d, C, bsizes[0], out=out, out_len=lens,
                                                                     status=status)),
              ("huffman_decode_batch", lambda: ec.decode_batch(fixed, out, n, out=y, status=status))]
    three = [("byte_histogram", lambda: ec.byte_histogram(x_d, out=hist)),                 # frequency analysis
             ("build_huffman_device", lambda: ec.build_huffman_device(hist, out=tables, status=status)),
             ("encode_batch_device", lambda: ec.encode_batch_device(tables, x_d, C, embed_lengths=True, out=out,
                                                                    out_len=lens, status=status)),
             # the receiver rebuilds each codebook from the lengths its stream carries
             ("huffman_tables_from_streams", lambda: ec.huffman_tables_from_streams(out, out=rtables,
                                                                                    status=status)),
             ("decode_batch_device", lambda: ec.decode_batch_device(rtables, out, n, out=y, status=status))]
    host_cbs = []

    def host_build():
        h = hist.cpu().numpy()          # histograms -> host
        host_cbs[:] = [ec.Codebook.huffman([int(c) for c in row]) for row in h]

    three_host = [("byte_histogram", lambda: ec.byte_histogram(x_d, out=hist)),
                  ("host_codebooks", host_build),
                  ("encode_batch", lambda: ec.encode_batch(host_cbs, x_d, C, embed_lengths=True, out=out,
                                                           out_len=lens, status=status)),
                  ("decode_batch", lambda: ec.decode_batch(host_cbs, out, n, out=y, status=status))]

    def check(label):
        if status.cpu().numpy().any() or not torch.equal(y, x_d):
            raise SystemExit("batch round trip failed (%s)" % label)

    res, per_shard = {}, {}
    for label, ops in (("single_stage", single), ("three_stage", three), ("three_stage_host", three_host)):
        for _ in range(warmup):
            for _, f in ops:
                f()
        torch.cuda.synchronize()
        # per-op breakdown (untimed pass, events around every op)
        evs = [[GpuEvent() for _ in range(len(ops) + 1)] for _ in range(steps)]
        for e in evs:
            for k, (_, f) in enumerate(ops):
                e[k].record()
                f()
            e[len(ops)].record()
        torch.cuda.synchronize()
        check(label)
        per_op = {o: statistics.mean(ev_us(e[k], e[k + 1]) for e in evs) for k, (o, _) in enumerate(ops)}
        # timed steps: events around the decode only (last op)
        dk = len(ops) - 1
        evs = [(GpuEvent(), GpuEvent()) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in evs:
            for k, (_, f) in enumerate(ops):
                if k == dk:
                    a.record()
                f()
            b.record()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        check(label)
        L = lens.cpu().numpy().astype(np.int64)
        moved_dec = S * n + int(L.sum())
        dec_us = statistics.mean(ev_us(a, b) for a, b in evs)
        kernels = {}
        for o, us in per_op.items():
            kk = dict(us=round(us, 2))
            if "code" in o and "codebook" not in o and "tables" not in o:
                kk["hbm_GBps"] = round(moved_dec / us / 1e3, 1)
                kk["roofline_frac"] = round(moved_dec / us / 1e3 / HBM_PEAK_GBPS, 4)
            elif o == "byte_histogram":
                kk["hbm_GBps"] = round(S * n / us / 1e3, 1)
                kk["roofline_frac"] = round(S * n / us / 1e3 / HBM_PEAK_GBPS, 4)
            kernels[o] = kk
        res[label] = dict(ms_per_step=round(dt * 1e3, 4), GBps=round(S * n / dt / 1e9, 2),
                          stream_pct=round(100 * (1 - L.sum() / (S * n)), 3), kernels=kernels,
                          decode_roofline=roofline_obj(ops[dk][0], moved_dec, dec_us, None, copy_gbps))
        per_shard[label] = [round(100 * (1 - int(v) / n), 3) for v in L]
    klv = kl.cpu().numpy().astype(np.float64)
    diff = np.array(per_shard["three_stage"]) - np.array(per_shard["single_stage"])
    ss = res["single_stage"]
    # the dominant kernel of the single-stage step, with its own event time
    dom = max(("huffman_encode_batch", "huffman_decode_batch"), key=lambda o: ss["kernels"][o]["us"])
    roof = ss["decode_roofline"] if dom == "huffman_decode_batch" else roofline_obj(
        dom, ss["decode_roofline"]["algorithmic_bytes"], ss["kernels"][dom]["us"], None, copy_gbps)
    roof["traffic"] = load_traffic("decode.hip" if dom.endswith("decode_batch") else "encode.hip", "batch", dom)
    return dict(value=ss["GBps"], unit="GB/s", steps=steps, warmup=warmup, ms_per_step=ss["ms_per_step"],
                n_bytes=S * n, chunk_symbols=C, codecs=["huffman"], workload=WORKLOAD_TEXT["batch"],
                step=("single stage: byte_histogram_sized (also sizes the chunks) + pmf_kl + batch encode (sized, "
                      "one read) + batch decode (64 shards)"),
                roofline=roof, paths=res,
                per_shard=dict(kl_bits_vs_average=[round(float(v), 6) for v in klv],
                               single_stage_stream_pct=per_shard["single_stage"],
                               three_stage_stream_pct=per_shard["three_stage"],
                               three_minus_single_pct=dict(mean=round(float(diff.mean()), 4),
                                                           max=round(float(diff.max()), 4))),
                kl_bits=dict(min=float(klv.min()), max=float(klv.max()), mean=float(klv.mean())))


def run_bf16(d, args, ec, torch, steps, warmup, copy_gbps):
    """BF16 exponent coding: one step = bf16_exp_encode + bf16_exp_decode of
    one 64 MiB tensor."""
    import synth
    dev = torch.device("cuda:0")
    w = synth.BF16_WORKLOAD
    n, chunk = w["n"], w["chunk"]
    x = d["x"]
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

    for i in range(warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    evs = [[GpuEvent() for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    enc_us = statistics.mean(ev_us(e[0], e[1]) for e in evs)
    dec_us = statistics.mean(ev_us(e[1], e[2]) for e in evs)
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
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
    return dict(value=round(2 * n / (wall / steps) / 1e9, 2), unit="GB/s", steps=steps, warmup=warmup,
                ms_per_step=round(wall / steps * 1e3, 4), n_bytes=2 * n, chunk_values=chunk,
                workload=WORKLOAD_TEXT["bf16"], table=list(table), step="bf16_exp_encode + bf16_exp_decode",
                roofline=roofline_obj(dom, moved, dom_us, load_traffic("bf16exp.hip", "bf16", dom), copy_gbps),
                kernels=kernels, compression=dict(stream_bytes=L, stream_pct=round(100 * (1 - L / (2 * n)), 3)))


def run_gpu(name, d, args, ec, torch, steps, warmup, copy_gbps):
    if name == "batch":
        return run_batch(d, args, ec, torch, steps, warmup, copy_gbps)
    if name == "bf16":
        return run_bf16(d, args, ec, torch, steps, warmup, copy_gbps)
    return run_single(name, d, args, ec, torch, steps, warmup, copy_gbps)


def line(name, r, args, cpu):
    """The one JSON line, headed by workload `name`'s result r."""
    cfg = dict(workload=r["workload"], name=name, n_bytes=r["n_bytes"], step=r["step"])
    for k in ("chunk_symbols", "chunk_values", "codecs", "table"):
        if k in r:
            cfg[k] = r[k]
    cfg["buffer_sets"] = args.sets
    out = dict(metric=METRIC, value=r["value"], unit="GB/s", n_gpus=1, steps=r["steps"], warmup=r["warmup"],
               ms_per_step=r["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="u16" if name == "bf16" else "u8", data="synthetic", config=cfg, roofline=r["roofline"])
    for k in ("kernels", "compression", "paths", "per_shard", "two_pass_encode_us"):
        if k in r and r[k] is not None:
            out[k] = r[k]
    out["cpu_baseline"] = cpu.get(name)
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py: this engine runs on one GPU; --gpus %d is not supported (multi-GPU sharding is a "
              "design note only)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    names = [args.workload] if args.workload else CONFIG_ORDER
    workers = cpu_workers(args)

    # host side first: no GPU state exists yet when the pools fork
    t = time.perf_counter()
    data = make_data(names, workers)
    log(args, "data %.1f s" % (time.perf_counter() - t))
    cpu = {}
    if not args.no_cpu:
        t = time.perf_counter()
        cpu = cpu_baselines(data, [n for n in names if n != "bf16"], workers)
        log(args, "cpu baselines %.1f s" % (time.perf_counter() - t))

    import torch
    import lossless_entropy_coding_amd as ec
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    ec.lib()
    # the practical ceiling: a plain copy of 64 MiB on the device
    flat = np.ascontiguousarray(data[names[0]]["x"]).reshape(-1).view(np.uint8)
    if flat.size >= 1 << 26:
        probe = torch.from_numpy(flat[:1 << 26].copy()).to("cuda:0")
    else:
        probe = torch.zeros(1 << 26, dtype=torch.uint8, device="cuda:0")
    copy = copy_ceiling(torch, probe)
    del probe
    copy_gbps = copy["GBps"]

    head = args.workload or HEADLINE
    results = {}
    for n in names:
        t = time.perf_counter()
        full = n == head
        results[n] = run_gpu(n, data[n], args, ec, torch, args.steps if full else min(args.steps, args.extra_steps),
                             args.warmup if full else min(args.warmup, 5), copy_gbps)
        log(args, "%s %.1f s" % (n, time.perf_counter() - t))
        torch.cuda.empty_cache()

    out = line(head, results[head], args, cpu)
    out["roofline"]["copy_ceiling"] = copy
    extra = dict(numpy=np.__version__, copy_ceiling=copy)
    if not args.workload:
        confs = {}
        for n in names:
            r = dict(results[n])
            r["cpu_baseline"] = cpu.get(n)
            confs[n] = r
        extra["configs"] = confs
        extra["configs_note"] = ("every workload of the run; the %s entry is the headline above. Per-op times come "
                                 "from an untimed pass with events around every op; roofline.avg_us from events "
                                 "around the dominant kernel inside the timed steps" % head)
    else:
        r = results[head]
        for k in ("kl_bits_vs_calibration", "histogram_exact", "codebook_build_us", "avg_pmf_top", "kl_bits"):
            if k in r:
                extra[k] = r[k]
    out["extra"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
