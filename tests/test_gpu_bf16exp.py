"""GPU parity of the BF16 exponent coder: streams byte-identical to the
oracle's, decodes equal to the input, at small and ragged sizes, with many
escapes, at the full 64 MiB workload in the benchmark's launch
configuration, and the capacity and corruption reports."""

import numpy as np
import pytest

import synth
from oracle import bf16exp as bx

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ec():
    import lossless_entropy_coding_amd as ec
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ec.lib()
    return ec


def _to_dev(x):
    t = torch.empty(max(x.size, 8), dtype=torch.int16, device=DEV)[: x.size]
    if x.size:
        t.copy_(torch.from_numpy(x.view(np.int16)))
    return t


def _round(ec, x, table, chunk, cap=None):
    xd = _to_dev(x)
    out = None if cap is None else torch.full((cap,), 0xCD, dtype=torch.uint8, device=DEV)
    out, out_len, status = ec.bf16_exp_encode(table, xd, chunk, out=out)
    torch.cuda.synchronize()
    return out, int(out_len.item()), int(status.item())


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 2047, 2048, 2049, 16383, 16384, 16385, 50_000, 100_003])
@pytest.mark.parametrize("chunk", [2048, 16384])
def test_stream_and_round_trip_match_oracle(ec, n, chunk):
    print("case bf16", n, chunk, flush=True)
    rng = np.random.default_rng(n + chunk)
    x = synth.bf16_draw(20 + n, n, 0.02)
    if n > 20:   # some values far outside the table: escapes
        k = n // 20
        x[rng.choice(n, k, replace=False)] = rng.integers(0, 1 << 16, k, dtype=np.uint16)
    table = bx.table_from_sigma(0.02)
    want = bx.encode(x, table, chunk)
    out, L, status = _round(ec, x, table, chunk)
    assert status == 0 and L == len(want)
    assert out[:L].cpu().numpy().tobytes() == want
    y, dstatus = ec.bf16_exp_decode(out[:L], n)
    torch.cuda.synchronize()
    assert int(dstatus.item()) == 0
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_every_value_escaped_and_every_code(ec):
    # uniform random bit patterns: almost all exponents escape; then a
    # shard whose values cycle through the seven table exponents
    x = np.random.default_rng(1).integers(0, 1 << 16, 70_001, dtype=np.uint16)
    table = [1, 2, 3, 200, 201, 202, 250]
    for data in (x, bx.join(np.array(table * 10_000, dtype=np.uint8), np.arange(70_000, dtype=np.uint8))):
        want = bx.encode(data, table, 16384)
        out, L, status = _round(ec, data, table, 16384)
        assert status == 0 and out[:L].cpu().numpy().tobytes() == want
        y, dstatus = ec.bf16_exp_decode(out[:L], data.size)
        torch.cuda.synchronize()
        assert int(dstatus.item()) == 0
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), data)


def test_full_size_workload(ec):
    w = synth.BF16_WORKLOAD
    print("case bf16 full size", w, flush=True)
    x = synth.bf16_draw(w["seed"], w["n"], w["sigma"])
    table = ec.bf16_exp_table_from_sigma(w["sigma"])
    assert list(table) == bx.table_from_sigma(w["sigma"])
    want = bx.encode(x, table, w["chunk"])
    out, L, status = _round(ec, x, table, w["chunk"])
    assert status == 0 and L == len(want)
    assert out[:L].cpu().numpy().tobytes() == want
    y, dstatus = ec.bf16_exp_decode(out, w["n"], in_len=out.numel())
    torch.cuda.synchronize()
    assert int(dstatus.item()) == 0
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_capacity_overflow(ec):
    x = np.random.default_rng(2).integers(0, 1 << 16, 40_000, dtype=np.uint16)
    table = bx.table_from_sigma(0.02)
    want = bx.encode(x, table, 16384)
    cap = (len(want) - 777) // 16 * 16
    big = torch.full((cap + 4096,), 0xCD, dtype=torch.uint8, device=DEV)
    out, out_len, status = ec.bf16_exp_encode(table, _to_dev(x), 16384, out=big[:cap])
    torch.cuda.synchronize()
    assert int(status.item()) & ec.S_CAPACITY
    assert int(out_len.item()) == len(want)
    assert bool((big[cap:] == 0xCD).all())
    with pytest.raises(ec.ECError):     # cannot hold the sections before the escapes
        ec.bf16_exp_encode(table, _to_dev(x), 16384, out=torch.empty(1000, dtype=torch.uint8, device=DEV))
    with pytest.raises(ec.ECError):     # table entries must differ
        ec.bf16_exp_encode([1, 1, 2, 3, 4, 5, 6], _to_dev(x), 16384)


def test_bad_header_and_corrupt_index_are_reported(ec):
    n = 30_000
    x = synth.bf16_draw(3, n, 0.02)
    x[::97] = 0x7F00                      # escapes
    table = bx.table_from_sigma(0.02)
    good = bytearray(bx.encode(x, table, 2048))

    def dec(b, n_=n, in_len=None):
        d = torch.frombuffer(bytearray(b), dtype=torch.uint8).to(DEV)
        _, st = ec.bf16_exp_decode(d, n_, in_len=in_len)
        torch.cuda.synchronize()
        return int(st.item())

    assert dec(good) == 0
    assert dec(good, n_=n - 1) & ec.S_BAD_HEADER             # wrong length
    bad = bytearray(good)
    bad[0] ^= 1                                                 # magic
    assert dec(bad) & ec.S_BAD_HEADER
    assert dec(good, in_len=len(good) - 1) & ec.S_BAD_HEADER   # escapes beyond in_len
    bad = bytearray(good)
    off = 64 + 8 * 3                                            # esc_off[3] one higher
    v = int.from_bytes(bad[off:off + 8], "little") + 1
    bad[off:off + 8] = v.to_bytes(8, "little")
    assert dec(bad) & ec.S_CORRUPT
