"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact on streams, decoded bytes and histograms; PMF averages and KL
divergences within 1e-5 relative (fp32 GPU vs fp64 oracle).
"""

import numpy as np
import pytest

import synth
from oracle import codebooks as cbm
from oracle import stats
from oracle import stream as st

from _util import deep_counts, padding_flips

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


DEV = "cuda:0"


def _calib_counts(recipe="normal", seed=1, n=1 << 18):
    return [int(c) for c in stats.histogram(synth.draw(recipe, seed, n))]


def _pair(ec, name, counts):
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
    if name == "eg0":
        return ec.Codebook.exp_golomb(counts, 0), cbm.eg_codebook(counts, 0)
    if name == "eg8":
        return ec.Codebook.exp_golomb(counts, 8), cbm.eg_codebook(counts, 8)
    raise KeyError(name)


def _gpu_encode(ec, cb, x, C):
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV) if x.size else torch.zeros(16, dtype=torch.uint8,
                                                                                      device=DEV)[:0]
    out, out_len, status = ec.encode(cb, xd, C)
    torch.cuda.synchronize()
    L = int(out_len.item())
    return out[:L].cpu().numpy().tobytes(), int(status.item())


def _gpu_decode(ec, cb, stream_bytes, n):
    d = torch.frombuffer(bytearray(stream_bytes), dtype=torch.uint8).to(DEV)
    y, status = ec.decode(cb, d, n)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(status.item())


CODECS = ["qlc", "qlc_adapted", "qlc_opt", "qlc_free", "huffman", "eg", "eg0", "eg8"]
SIZES = [(1, 256), (255, 4096), (256, 256), (257, 256), (4095, 4096), (4096, 4096), (4097, 4096),
         (3 * 4096 + 17, 4096), (16384 * 3 + 999, 16384), (100_000, 1024), (70_001, 8192), (50_000, 12288)]


@pytest.mark.parametrize("n,C", SIZES)
@pytest.mark.parametrize("name", CODECS)
def test_stream_and_round_trip_match_oracle(ec, name, n, C):
    print("case", name, n, C, flush=True)
    counts = _calib_counts()
    cb, ocb = _pair(ec, name, counts)
    x = synth.draw("ffn1", 7 + n, n)
    want = st.encode_stream(x, ocb, C)
    got, status = _gpu_encode(ec, cb, x, C)
    assert status == 0
    assert got == want
    y, dstatus = _gpu_decode(ec, cb, want, n)
    assert dstatus == 0
    assert np.array_equal(y, x)


@pytest.mark.parametrize("C", [256, 4096, 16384])
@pytest.mark.parametrize("layout_kind", ["optimal", "empty_areas"])
def test_qlc_layout_with_three_bit_codes_and_empty_areas(ec, C, layout_kind):
    # one symbol holds almost everything: the cheapest layout gives it a
    # 3-bit code (an area of suffix width 0); the second layout also leaves
    # areas 1, 2 and 4-7 empty, so their prefixes are never codewords.  The
    # data mixes long runs of that symbol with every other byte.
    print("case qlc spike layout", layout_kind, C, flush=True)
    counts = [1] * 256
    counts[0x40] = 1 << 40
    if layout_kind == "optimal":
        layout = ec.qlc_optimal_area_layout(counts, 4)
        assert layout == cbm.qlc_optimal_areas(counts, 4)
    else:
        layout = ((1, 0, 0, 255, 0, 0, 0, 0), (0, 0, 0, 8, 0, 0, 0, 0))
    assert layout[1][0] == 0
    cb, ocb = ec.Codebook.qlc(counts, *layout), cbm.qlc_codebook(counts, *layout)
    assert ocb.length[0x40] == 3
    rng = np.random.default_rng(C)
    n = 5 * C + 77
    x = np.full(n, 0x40, dtype=np.uint8)
    pos = rng.choice(n, n // 9, replace=False)
    x[pos] = rng.integers(0, 256, pos.size, dtype=np.uint8)
    x[: 3 * 256] = np.arange(3 * 256) % 256
    want = st.encode_stream(x, ocb, C)
    got, status = _gpu_encode(ec, cb, x, C)
    assert status == 0 and got == want
    y, dstatus = _gpu_decode(ec, cb, want, n)
    assert dstatus == 0 and np.array_equal(y, x)


@pytest.mark.parametrize("r,profile", [(0.9973, (8, 8, 0)), (0.9907, (7, 10, 3)), (0.979, (6, 13, 7)),
                                       (0.9757, (5, 14, 8)), (0.9116, (4, 17, 9))])
def test_huffman_length_profiles(ec, r, profile):
    # Codebooks of one length only, of lengths up to 10 and 13 bits (every
    # code in the decoder's 13-bit table), and with 14- and 17-bit codes
    # (longer codes than the table covers); runs of the longest codes at odd
    # offsets.
    print("case huffman profile", profile, flush=True)
    counts = [int(1e4 * r ** s) for s in range(256)]
    ocb = cbm.huffman_codebook(counts)
    lo, hi = min(ocb.length), max(ocb.length)
    assert (lo, hi, max(min(hi - 1, 12) - lo + 1, 0)) == profile
    cb = ec.Codebook.huffman(counts)
    rng = np.random.default_rng(int(r * 1e4))
    p = np.array(counts, dtype=np.float64) + 1
    n = 150_000
    x = rng.choice(256, size=n, p=p / p.sum()).astype(np.uint8)
    x[:512] = np.arange(512) % 256                      # every code, the longest included
    rare = np.argsort(ocb.length)[-8:]                  # runs of the longest codes at odd offsets
    for k, at in enumerate((1031, 5000, 77_777, 120_003)):
        x[at:at + 40] = rare[(np.arange(40) + k) % 8]
    for C in (4096, 16384):
        want = st.encode_stream(x, ocb, C)
        got, status = _gpu_encode(ec, cb, x, C)
        assert status == 0 and got == want
        y, dstatus = _gpu_decode(ec, cb, want, n)
        assert dstatus == 0 and np.array_equal(y, x)


def test_empty_input(ec):
    counts = _calib_counts()
    for name in ("qlc", "huffman", "eg"):
        cb, ocb = _pair(ec, name, counts)
        x = np.zeros(0, dtype=np.uint8)
        want = st.encode_stream(x, ocb, 16384)
        got, status = _gpu_encode(ec, cb, x, 16384)
        assert status == 0 and got == want
        y, dstatus = _gpu_decode(ec, cb, want, 0)
        assert dstatus == 0 and y.size == 0


@pytest.mark.parametrize("name", CODECS)
def test_all_symbols_and_one_repeated_symbol(ec, name):
    counts = _calib_counts()
    cb, ocb = _pair(ec, name, counts)
    for x in (np.tile(np.arange(256, dtype=np.uint8), 97), np.full(40000, 0x7E, dtype=np.uint8),
              np.full(40000, np.argmax(ocb.length), dtype=np.uint8)):
        want = st.encode_stream(x, ocb, 4096)
        got, status = _gpu_encode(ec, cb, x, 4096)
        assert status == 0 and got == want
        y, dstatus = _gpu_decode(ec, cb, want, x.size)
        assert dstatus == 0 and np.array_equal(y, x)


@pytest.mark.parametrize("depth", [24, 25, 33, 39, 40])
def test_deep_huffman_codes(ec, depth):
    counts = [int(c) for c in deep_counts(depth)]
    cb, ocb = ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)
    assert ocb.max_len == depth
    rng = np.random.default_rng(depth)
    x = rng.integers(0, 256, 60000).astype(np.uint8)
    x[::7] = np.argmax(ocb.length)                 # the deepest code, often
    x[3::11] = 0                                   # and the shortest
    want = st.encode_stream(x, ocb, 16384)
    got, status = _gpu_encode(ec, cb, x, 16384)
    assert status == 0 and got == want
    y, dstatus = _gpu_decode(ec, cb, want, x.size)
    assert dstatus == 0 and np.array_equal(y, x)


@pytest.mark.parametrize("C", [4096, 16384, 65536])
@pytest.mark.parametrize("depth", [20, 26, 27])
def test_chunks_of_mixed_code_length(ec, C, depth):
    """Chunks of short codes next to chunks of the deepest code: one launch
    has chunks whose packed bits fit the encoder's LDS stage and chunks that
    do not, and rows whose code pairs span more than 32 bits."""
    counts = [int(c) for c in deep_counts(depth)]
    cb, ocb = ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)
    assert ocb.max_len == depth
    deepest, shortest = int(np.argmax(ocb.length)), int(np.argmin(ocb.length))
    rng = np.random.default_rng(C + depth)
    parts = [np.full(C, shortest), np.full(C, deepest), rng.integers(0, 256, C),
             np.where(rng.random(C) < 0.5, deepest, shortest), np.full(C // 2 + 37, deepest)]
    x = np.concatenate(parts).astype(np.uint8)
    want = st.encode_stream(x, ocb, C)
    got, status = _gpu_encode(ec, cb, x, C)
    assert status == 0 and got == want
    y, dstatus = _gpu_decode(ec, cb, want, x.size)
    assert dstatus == 0 and np.array_equal(y, x)


@pytest.mark.parametrize("C", [4096, 16384])
@pytest.mark.parametrize("codec", ["huffman", "eg0"])
def test_sub_chunks_that_outrun_the_ring(ec, C, codec):
    """Sub-chunks of different code-length profiles side by side, so that one
    wave holds lanes the decoder's LDS ring keeps up with and lanes whose long
    codes (more than 16 bits a symbol over 32 symbols) outrun it and decode
    again from global memory: long codes in the first half, in the second
    half, throughout, short ones, and a mix."""
    if codec == "huffman":
        counts = [int(c) for c in deep_counts(20)]
        cb, ocb = ec.Codebook.huffman(counts), cbm.huffman_codebook(counts)
        length = np.array(ocb.length)
        long_, mid, short = (int(np.flatnonzero(length == l)[0]) for l in (20, 12, 3))
    else:   # order-0 Exp-Golomb: ranks 128..255 take 15-17 bits
        counts = [int(c) for c in np.arange(256, 0, -1)]
        cb, ocb = ec.Codebook.exp_golomb(counts, 0), cbm.eg_codebook(counts, 0)
        r2s = ocb.rank_to_sym
        long_, mid, short = r2s[255], r2s[40], r2s[0]
    rng = np.random.default_rng(C)
    kinds = [
        np.full(256, short),                                         # short
        np.concatenate([np.full(128, long_), np.full(128, short)]),  # long first half
        np.concatenate([np.full(128, short), np.full(128, long_)]),  # long second half
        np.full(256, long_),                                         # long throughout
        np.full(256, mid),                                           # middling
        rng.integers(0, 256, 256),                                   # mixed
    ]
    pick = rng.integers(0, len(kinds), 3 * C // 256 + 5)
    x = np.concatenate([kinds[k] for k in pick] + [np.full(77, long_)]).astype(np.uint8)
    print("case ring overrun", codec, C, x.size, flush=True)
    want = st.encode_stream(x, ocb, C)
    got, status = _gpu_encode(ec, cb, x, C)
    assert status == 0 and got == want
    y, dstatus = _gpu_decode(ec, cb, want, x.size)
    assert dstatus == 0 and np.array_equal(y, x)


def test_encode_is_deterministic(ec):
    counts = _calib_counts()
    cb, _ = _pair(ec, "huffman", counts)
    x = torch.from_numpy(synth.draw("ffn1", 3, 1 << 22)).to(DEV)
    ref = None
    for _ in range(10):
        out, out_len, status = ec.encode(cb, x, 16384)
        torch.cuda.synchronize()
        s = out[: int(out_len.item())].clone()
        if ref is None:
            ref = s
        assert int(status.item()) == 0 and torch.equal(s, ref)


def test_calls_on_two_streams_at_once(ec):
    """Histograms and encodes enqueued on two streams with no ordering between
    them (the library's scratch is kept per stream): every result equals the
    same call made alone."""
    counts = _calib_counts()
    cb, _ = _pair(ec, "huffman", counts)
    xs = [torch.from_numpy(synth.draw(r, 60 + k, (8 << 20) + 4096 * k)).to(DEV) for k, r in enumerate(["ffn1", "grad"])]
    ref = []
    for x in xs:
        out, out_len, status = ec.encode(cb, x, 16384)
        ref.append(out[: int(out_len.item())].cpu())
        assert int(status.item()) == 0
    hist_ref = [stats.histogram(x.cpu().numpy()) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty(ec.max_encoded_bytes(cb, x.numel(), 16384), dtype=torch.uint8, device=DEV) for x in xs]
    lens = [torch.zeros(1, dtype=torch.int64, device=DEV) for _ in xs]
    sts = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in xs]
    hists = [torch.zeros((1, 256), dtype=torch.int64, device=DEV) for _ in xs]
    torch.cuda.synchronize()
    for rep in range(4):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                ec.byte_histogram(xs[k], out=hists[k])
                ec.encode(cb, xs[k], 16384, out=outs[k], out_len=lens[k], status=sts[k])
        torch.cuda.synchronize()
        for k in range(2):
            L = int(lens[k].item())
            assert int(sts[k].item()) == 0 and L == ref[k].numel(), (rep, k)
            assert torch.equal(outs[k][:L].cpu(), ref[k]), (rep, k)
            assert np.array_equal(hists[k].cpu().numpy()[0].astype(np.uint64), hist_ref[k]), (rep, k)


@pytest.mark.parametrize("segs,seg_n", [(1, 1000), (3, 4 << 20), (8, 12345), (2, 1 << 16)])
def test_histogram_matches_oracle(ec, segs, seg_n):
    x = np.stack([synth.draw("ffn2", 50 + s, seg_n) for s in range(segs)])
    h = ec.byte_histogram(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.uint64)
    for s in range(segs):
        assert np.array_equal(got[s], stats.histogram(x[s]))


def test_pmf_average_and_kl_match_oracle(ec):
    rows = [stats.histogram(synth.draw("ffn1", 100 + s, 1 << 20)) for s in range(8)]
    shards = [stats.histogram(synth.batch_shards(1, 1 << 20, first_seed=1000 + i)[0]) for i in range(6)]
    rows_t = torch.from_numpy(np.stack(rows).astype(np.int64)).to(DEV)
    avg = ec.pmf_average(rows_t)
    pooled = sum(r.astype(np.int64) for r in rows)
    p_t = torch.from_numpy(np.stack(shards).astype(np.int64)).to(DEV)
    q_t = torch.from_numpy(pooled.astype(np.int64)).to(DEV)
    kl = ec.pmf_kl(p_t, q_t, q_add=1)
    kl0 = ec.pmf_kl(rows_t[:1], rows_t[0], q_add=0)
    torch.cuda.synchronize()
    want_avg = stats.average_pmf(rows)
    got_avg = avg.cpu().numpy().astype(np.float64)
    for s in range(256):
        if want_avg[s] > 0:
            assert abs(got_avg[s] - want_avg[s]) <= 1e-5 * want_avg[s]
        else:
            assert got_avg[s] == 0
    got_kl = kl.cpu().numpy().astype(np.float64)
    for i, sh in enumerate(shards):
        want = stats.kl_bits(sh, pooled, q_add=1)
        assert want > 0 and abs(got_kl[i] - want) <= 1e-5 * want, (i, got_kl[i], want)
    assert abs(float(kl0.item())) <= 1e-7       # D(P || P) = 0


def test_kl_with_counts_beyond_2_to_31_matches_oracle(ec):
    # row totals past 2^31 take the kernel's double-precision ratio branch
    rng = np.random.default_rng(9)
    q = rng.integers(1 << 30, 1 << 34, 256).astype(np.int64)
    # (deviations of 2^18 and more: at smaller ones the fp64 oracle's own
    # rounding, about 1e-17 bits, nears 1e-5 of the divergence)
    rows = [q + rng.integers(-(1 << d), 1 << d, 256) for d in (18, 22, 28)]
    p_t = torch.from_numpy(np.stack(rows)).to(DEV)
    kl = ec.pmf_kl(p_t, torch.from_numpy(q).to(DEV), q_add=0).cpu().numpy().astype(np.float64)
    for i, r in enumerate(rows):
        assert r.sum() >= 1 << 31
        want = stats.kl_bits(r, q)
        assert want > 0 and abs(kl[i] - want) <= 1e-5 * want, (i, kl[i], want)


def test_kl_closed_forms(ec):
    p = np.zeros(256, np.int64)
    q = np.zeros(256, np.int64)
    p[0], p[1] = 300_000, 700_000
    q[0], q[1] = 400_000, 600_000
    kl = ec.pmf_kl(torch.from_numpy(p).to(DEV), torch.from_numpy(q).to(DEV))
    torch.cuda.synchronize()
    want = 0.3 * np.log2(0.3 / 0.4) + 0.7 * np.log2(0.7 / 0.6)
    assert abs(float(kl.item()) - want) <= 1e-5 * want
    q[1] = 0     # a hole in Q under mass of P: infinite
    kl = ec.pmf_kl(torch.from_numpy(p).to(DEV), torch.from_numpy(q).to(DEV))
    torch.cuda.synchronize()
    assert np.isinf(float(kl.item()))


@pytest.mark.parametrize("per_segment", [False, True])
@pytest.mark.parametrize("embed", [False, True])
def test_batch_matches_oracle(ec, per_segment, embed):
    S, seg_n, C = 5, 70_000, 16384
    x = np.stack([synth.draw("ffn1", 200 + s, seg_n) for s in range(S)])
    if per_segment:
        cnts = [[int(c) for c in stats.histogram(x[s])] for s in range(S)]
    else:
        cnts = [_calib_counts("ffn1", 100)] * S
    cbs = [ec.Codebook.huffman(c) for c in cnts]
    ocbs = [cbm.huffman_codebook(c) for c in cnts]
    xd = torch.from_numpy(x).to(DEV)
    out, out_len, status = ec.encode_batch(cbs, xd, C, embed_lengths=embed)
    torch.cuda.synchronize()
    lens = out_len.cpu().numpy()
    assert (status.cpu().numpy() == 0).all()
    for s in range(S):
        want = st.encode_stream(x[s], ocbs[s], C, embed_lengths=embed)
        assert out[s, : int(lens[s])].cpu().numpy().tobytes() == want
    y, dstatus = ec.decode_batch(cbs, out, seg_n)
    torch.cuda.synchronize()
    assert (dstatus.cpu().numpy() == 0).all()
    assert np.array_equal(y.cpu().numpy(), x)


@pytest.mark.parametrize("chunks", [4095, 4096, 4097, 5000])
@pytest.mark.parametrize("name", ["qlc", "huffman", "eg"])
def test_streams_around_the_placement_switch(ec, name, chunks):
    # up to 4096 chunks a stream the pack launch places the chunks itself;
    # beyond, a separate scan launch does: both must give the oracle's stream
    print("case chunks", name, chunks, flush=True)
    C = 256
    n = chunks * C - 7
    counts = _calib_counts()
    cb, ocb = _pair(ec, name, counts)
    x = synth.draw("ffn1", 31 + chunks, n)
    want = st.encode_stream(x, ocb, C)
    got, status = _gpu_encode(ec, cb, x, C)
    assert status == 0
    assert got == want
    y, dstatus = _gpu_decode(ec, cb, want, n)
    assert dstatus == 0 and np.array_equal(y, x)


def test_batch_exp_golomb_of_mixed_orders(ec):
    # order 1 codes fit two to a 32-bit window (at most 16 bits), order 0
    # codes do not (up to 17 bits): the decoder's mode must suit every
    # segment of the batch, not just the first
    counts = _calib_counts()
    S, seg_n, C = 3, 50_000, 4096
    ks = [1, 0, 5]
    cbs = [ec.Codebook.exp_golomb(counts, k) for k in ks]
    ocbs = [cbm.eg_codebook(counts, k) for k in ks]
    assert [max(o.length) for o in ocbs][:2] == [16, 17]
    x = np.stack([synth.draw("ffn1", 300 + s, seg_n) for s in range(S)])
    x[1, :256] = np.arange(256)
    x[1, 300:340] = ocbs[1].rank_to_sym[255]   # back-to-back 17-bit codes in segment 1
    xd = torch.from_numpy(x).to(DEV)
    out, out_len, status = ec.encode_batch(cbs, xd, C)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    lens = out_len.cpu().numpy()
    for s in range(S):
        assert out[s, : int(lens[s])].cpu().numpy().tobytes() == st.encode_stream(x[s], ocbs[s], C)
    y, dstatus = ec.decode_batch(cbs, out, seg_n)
    torch.cuda.synchronize()
    assert (dstatus.cpu().numpy() == 0).all()
    assert np.array_equal(y.cpu().numpy(), x)


@pytest.mark.parametrize("n,C", [(200_000, 4096), (5000 * 256, 256)])
def test_capacity_overflow_reports_required_length(ec, n, C):
    counts = _calib_counts()
    cb, ocb = _pair(ec, "qlc", counts)
    x = synth.draw("ffn1", 11, n)
    want = st.encode_stream(x, ocb, C)
    xd = torch.from_numpy(x).to(DEV)
    cap = (len(want) - 1000) // 16 * 16
    big = torch.full((cap + 8192,), 0xCD, dtype=torch.uint8, device=DEV)
    out, guard = big[:cap], big[cap:]
    _, out_len, status = ec.encode(cb, xd, C, out=out)
    torch.cuda.synchronize()
    assert int(status.item()) & ec.S_CAPACITY
    assert int(out_len.item()) == len(want)
    assert bool((guard == 0xCD).all())
    with pytest.raises(ec.ECError):       # cannot even hold the index
        ec.encode(cb, xd, C, out=torch.empty(100, dtype=torch.uint8, device=DEV))


def test_corruption_and_header_errors_are_reported(ec):
    counts = _calib_counts()
    x = synth.draw("ffn1", 12, 100_000)
    for name in ("qlc", "huffman", "eg"):
        cb, ocb = _pair(ec, name, counts)
        s = bytearray(st.encode_stream(x, ocb, 4096))
        h = st.parse_header(bytes(s))
        rng = np.random.default_rng(0)
        for _ in range(8):
            t = bytearray(s)
            pos = h["payload_offset"] + int(rng.integers(0, h["payload_bytes"]))
            t[pos] ^= 1 << int(rng.integers(0, 8))
            y, status = _gpu_decode(ec, cb, bytes(t), x.size)
            assert status & ec.S_CORRUPT or not np.array_equal(y, x)
        t = bytearray(s)
        t[0] ^= 1
        assert _gpu_decode(ec, cb, bytes(t), x.size)[1] & ec.S_BAD_HEADER
        same_codec_other, _ = _pair(ec, name, _calib_counts("ffn2", 5))
        assert _gpu_decode(ec, same_codec_other, bytes(s), x.size)[1] & ec.S_CODEBOOK_MISMATCH
        other_codec, _ = _pair(ec, "huffman" if name != "huffman" else "qlc", counts)
        assert _gpu_decode(ec, other_codec, bytes(s), x.size)[1] & ec.S_CODEBOOK_MISMATCH
        # a stream cut short: the header no longer fits the buffer
        d = torch.frombuffer(bytearray(s), dtype=torch.uint8).to(DEV)
        _, status = ec.decode(cb, d, x.size, in_len=len(s) - 16)
        torch.cuda.synchronize()
        assert int(status.item()) & ec.S_BAD_HEADER
        # index pointing past the payload
        t = bytearray(s)
        t[64 + 8 * 3: 64 + 8 * 4] = (h["payload_bytes"] + 4096).to_bytes(8, "little")
        assert _gpu_decode(ec, cb, bytes(t), x.size)[1] & ec.S_CORRUPT
        # wrong n
        d = torch.frombuffer(bytearray(s), dtype=torch.uint8).to(DEV)
        _, status = ec.decode(cb, d, x.size - 1)
        torch.cuda.synchronize()
        assert int(status.item()) & ec.S_BAD_HEADER


@pytest.mark.parametrize("n,C", [(100_000, 4096), (70_001, 16384)])
def test_a_set_padding_bit_is_corrupt(ec, n, C):
    # the oracle rejects any set bit between a chunk's last code and its end
    counts = _calib_counts()
    x = synth.draw("ffn1", 13, n)
    for name in ("qlc", "huffman", "eg"):
        cb, ocb = _pair(ec, name, counts)
        s = st.encode_stream(x, ocb, C)
        flips = padding_flips(s)
        assert len(flips) >= 2
        for where, t in flips:
            with pytest.raises(st.CorruptStream):
                st.decode_stream(t, ocb)
            y, status = _gpu_decode(ec, cb, t, n)
            assert status & ec.S_CORRUPT, (name, where)
        y, status = _gpu_decode(ec, cb, s, n)
        assert status == 0 and np.array_equal(y, x)


def test_qlc_unused_suffix_is_corrupt(ec):
    counts = _calib_counts()
    cb, ocb = _pair(ec, "qlc", counts)
    x = np.zeros(256, dtype=np.uint8) + ocb.rank_to_sym[0]    # 256 six-bit zero codes
    s = bytearray(st.encode_stream(x, ocb, 256))
    h = st.parse_header(bytes(s))
    po = h["payload_offset"]
    # first code -> area 7 (prefix 111) with suffix 255 (>= 168: not a codeword)
    word = int.from_bytes(s[po:po + 4], "little") | (0b11111111111 << 21)
    s[po:po + 4] = word.to_bytes(4, "little")
    y, status = _gpu_decode(ec, cb, bytes(s), x.size)
    assert status & ec.S_CORRUPT
