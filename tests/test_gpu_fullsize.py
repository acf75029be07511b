"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: one preallocated output buffer of ``max_encoded_bytes``,
decode told the whole buffer length, chunks of the workload's size.

Every stream is compared byte for byte with the oracle's (the oracle's C
encoder finishes a 64 MiB shard in a few seconds); the decoded bytes must
equal the input and the histograms must equal the oracle's.  The 256 MiB
multi-shard batch checks every shard's histogram, round trip and stream
against the oracle, for the fixed codebook and for per-shard codebooks built
on the host and on the GPU.
"""

import functools

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"

CASES = [("tiny_qlc", "qlc"),
         ("ffn1", "qlc"), ("ffn1", "huffman"), ("ffn1", "qlc_opt"),
         ("ffn2", "qlc_adapted"), ("ffn2", "qlc"), ("ffn2", "huffman"), ("ffn2", "qlc_opt"), ("ffn2", "qlc_free"),
         ("grad", "eg"), ("grad", "qlc"), ("grad", "huffman"), ("grad", "qlc_opt")]


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


@functools.lru_cache(maxsize=1)
def _workload(name):
    x = synth.workload(name)
    counts = [int(c) for c in stats.histogram(synth.calibration_shards(name).reshape(-1))]
    return x, counts


def _codebooks(ec, name, counts):
    if name == "qlc":
        return ec.Codebook.qlc(counts), cbm.qlc_codebook(counts)
    if name == "qlc_adapted":
        return (ec.Codebook.qlc(counts, *ec.QLC_ADAPTED),
                cbm.qlc_codebook(counts, cbm.QLC_ADAPTED_AREAS, cbm.QLC_ADAPTED_SUFFIX))
    if name in ("qlc_opt", "qlc_free"):
        L = 4 if name == "qlc_opt" else 8
        layout = ec.qlc_optimal_area_layout(counts, L)
        assert layout == cbm.qlc_optimal_areas(counts, L)
        return ec.Codebook.qlc(counts, *layout), cbm.qlc_codebook(counts, *cbm.qlc_optimal_areas(counts, L))
    if name == "huffman":
        return ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)
    if name == "eg":
        return ec.Codebook.exp_golomb(counts, -1), cbm.eg_codebook(counts)
    raise KeyError(name)


@pytest.mark.parametrize("workload,codec", CASES)
def test_full_size_stream_matches_oracle(ec, workload, codec):
    print("case", workload, codec, flush=True)
    x, counts = _workload(workload)
    C = synth.WORKLOADS[workload].chunk_symbols
    N = x.size
    cb, ocb = _codebooks(ec, codec, counts)
    x_d = torch.from_numpy(x).to(DEV)

    hist = torch.empty((1, 256), dtype=torch.int64, device=DEV)
    ec.byte_histogram(x_d, out=hist)
    cap = ec.max_encoded_bytes(cb, N, C)
    s = torch.empty(cap, dtype=torch.uint8, device=DEV)
    y = torch.empty(N, dtype=torch.uint8, device=DEV)
    n = torch.zeros(1, dtype=torch.int64, device=DEV)
    status = torch.zeros(2, dtype=torch.int32, device=DEV)
    ec.encode(cb, x_d, C, out=s, out_len=n, status=status[0:1])
    ec.decode(cb, s, N, out=y, status=status[1:2], in_len=cap)
    torch.cuda.synchronize()

    assert status.cpu().numpy().tolist() == [0, 0]
    assert np.array_equal(hist.cpu().numpy()[0].astype(np.uint64), stats.histogram(x))
    want = st.encode_stream(x, ocb, C)
    L = int(n.item())
    assert L == len(want)
    got = s[:L].cpu().numpy().tobytes()
    if got != want:
        g = np.frombuffer(got, np.uint8)
        w = np.frombuffer(want, np.uint8)
        first = int(np.flatnonzero(g != w)[0])
        pytest.fail("stream differs from the oracle's first at byte %d of %d" % (first, L))
    assert torch.equal(y, x_d)


@pytest.mark.parametrize("mode", ["fixed", "per_shard_host", "per_shard_device"])
def test_full_size_batch_matches_oracle(ec, mode):
    print("case batch %s" % mode, flush=True)
    per_shard = mode != "fixed"
    x, counts = _workload("batch")
    S, n = 64, 1 << 22
    x = x.reshape(S, n)
    C = synth.WORKLOADS["batch"].chunk_symbols
    x_d = torch.from_numpy(x).to(DEV)
    hist = torch.empty((S, 256), dtype=torch.int64, device=DEV)
    ec.byte_histogram(x_d, out=hist)
    torch.cuda.synchronize()
    h = hist.cpu().numpy()
    for i in range(S):
        assert np.array_equal(h[i].astype(np.uint64), stats.histogram(x[i])), i
    if per_shard:
        rows = [[int(c) for c in r] for r in h]
    else:
        rows = [counts] * S
    y = torch.empty((S, n), dtype=torch.uint8, device=DEV)
    lens = torch.zeros(S, dtype=torch.int64, device=DEV)
    status = torch.zeros(S, dtype=torch.int32, device=DEV)
    if mode == "per_shard_device":
        # the bench's three-stage step: histogram rows -> device codebooks
        stride = (ec.own_max_encoded_bytes(n, C, True) + 255) // 256 * 256 + 4096
        out = torch.empty((S, stride), dtype=torch.uint8, device=DEV)
        tables, _ = ec.build_huffman_device(hist, status=status)
        ec.encode_batch_device(tables, x_d, C, embed_lengths=True, out=out, out_len=lens, status=status)
        ec.decode_batch_device(tables, out, n, out=y, status=status)
    else:
        cbs = [ec.Codebook.huffman(r) for r in rows] if per_shard else ec.Codebook.huffman(counts)
        worst = max(ec.max_encoded_bytes(c, n, C, True) for c in (cbs if per_shard else [cbs]))
        stride = (worst + 255) // 256 * 256 + 4096
        out = torch.empty((S, stride), dtype=torch.uint8, device=DEV)
        ec.encode_batch(cbs, x_d, C, embed_lengths=per_shard, out=out, out_len=lens, status=status)
        ec.decode_batch(cbs, out, n, out=y, status=status)
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any()
    assert torch.equal(y, x_d)
    L = lens.cpu().numpy()
    got = out.cpu().numpy()
    for i in range(S):   # every shard's stream
        want = st.encode_stream(x[i], cbm.huffman_codebook(rows[i]), C, embed_lengths=per_shard)
        assert int(L[i]) == len(want), i
        assert got[i, : int(L[i])].tobytes() == want, i
