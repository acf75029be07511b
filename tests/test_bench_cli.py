"""bench.py's host logic that runs without a GPU: more than one GPU is
refused with a message (this engine runs on one GPU), and the measured HBM
traffic is taken from a committed profile only while the kernel source it
was measured on is unchanged."""

import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    bench = _bench()
    csrc = tmp_path / "lossless_entropy_coding_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "decode.hip").write_bytes(b"kernel source v1\n")
    h1 = hashlib.sha256(b"kernel source v1\n").hexdigest()[:16]
    (tmp_path / "profiles" / "traffic_w.txt").write_text(
        "# header\n| table | row |\n"
        "traffic huffman_decode src=%s bytes=123456\n"
        "traffic qlc_decode src=0000000000000000 bytes=999\n" % h1)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("decode.hip", "w", "huffman_decode") == 123456
    assert bench.load_traffic("decode.hip", "w", "qlc_decode") is None       # another source
    assert bench.load_traffic("decode.hip", "w", "eg_decode") is None        # no line
    assert bench.load_traffic("decode.hip", "other", "huffman_decode") is None   # no file
    (csrc / "decode.hip").write_bytes(b"kernel source v2\n")                 # the kernel changed
    assert bench.load_traffic("decode.hip", "w", "huffman_decode") is None


def test_committed_traffic_lines_are_well_formed():
    prof = os.path.join(ROOT, "profiles")
    for name in os.listdir(prof):
        if not name.startswith("traffic_"):
            continue
        lines = [l.split() for l in open(os.path.join(prof, name)) if l.startswith("traffic ")]
        assert lines, name
        for _, op, srcf, nbytes in lines:
            assert srcf.startswith("src=") and len(srcf) == 4 + 16 and nbytes.startswith("bytes=")
            assert int(nbytes[6:]) > 0
            # op names as bench.py reports them (per codec, batch paths, device builds)
            assert op.endswith(("_encode", "_decode", "_batch", "_device", "_streams")) or op == "byte_histogram", \
                (name, op)
