"""Host-side checks that need no GPU: argument validation of the device
append and demand-mapped cache entry points (they return before any HIP
call), and bench.py's algorithmic byte count, traffic records, read-ceiling
records and one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

from native import ensure_built
from paged_kv_cache_191_amd import kvpaged as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def setup_module(_):
    ensure_built()


def _append(L=None, **kw):
    a = dict(k=None, v=None, nb=None, bt=None, stride=4, ctx=None, S=2,
             kc=None, vc=None, N=8, B=16, hkv=2, d=128)
    a.update(kw)
    return L(a["k"], a["v"], a["nb"], a["bt"], a["stride"], a["ctx"], a["S"],
             a["kc"], a["vc"], a["N"], a["B"], a["hkv"], a["d"])


def test_append_token_argument_errors():
    lib = kv.lib()

    def call(dtype=kv.KV_BF16, **kw):
        return _append(lambda *x: lib.kv_append_token(*x, dtype, None), **kw)

    assert call(S=0) == kv.KV_OK                     # nothing to do
    assert call() == kv.KV_EINVAL                    # NULL pointers
    for bad in (dict(S=-1), dict(stride=0), dict(N=0), dict(B=0),
                dict(hkv=0), dict(d=0)):
        assert call(**bad) == kv.KV_EINVAL, bad
        assert "bad shape" in kv.kv_last_error()
    assert call(dtype=7) == kv.KV_EINVAL
    assert "dtype" in kv.kv_last_error()


def test_append_token_fp8_argument_errors():
    lib = kv.lib()

    def call(ks=1.0, vs=1.0, **kw):
        return _append(lambda *x: lib.kv_append_token_fp8(*x, ks, vs, None),
                       **kw)

    assert call(S=0) == kv.KV_OK
    assert call(d=12) == kv.KV_EINVAL                # D % 8 != 0
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0),
                   (float("nan"), 1.0)):
        assert call(ks=ks, vs=vs) == kv.KV_EINVAL
        assert "scale" in kv.kv_last_error()
    assert call() == kv.KV_EINVAL                    # NULL pointers


def test_vcache_prefetch_and_sync_reject_null():
    lib = kv.lib()
    assert lib.kv_vcache_prefetch(None, 0, 16) == kv.KV_EINVAL
    assert lib.kv_vcache_sync(None) == kv.KV_EINVAL


def test_decode_bytes_counts_each_term_once():
    sys.path.insert(0, ROOT)
    import bench
    ctx = np.array([35, 16, 1, 100])
    hq, hkv, d, B = 8, 8, 64, 16
    kvb = int(ctx.sum()) * hkv * d * 2 * 4      # K and V, fp32 (4 B)
    qo = 2 * 4 * hq * d * 4
    table = (3 + 1 + 1 + 7) * 4                  # blocks per sequence x 4 B
    want = kvb + qo + table + 4 * 4
    assert bench.decode_bytes(ctx, hq, hkv, d, B, True, esize=4) == want
    assert bench.decode_bytes(ctx, hq, hkv, d, B, False, esize=4) == \
        want - table
    # a 32-token shared prefix counts once over the four sequences
    ctx2 = ctx + 32
    shared = bench.decode_bytes(ctx2, hq, hkv, d, B, True, esize=4,
                                shared=32)
    full = bench.decode_bytes(ctx2, hq, hkv, d, B, True, esize=4)
    assert full - shared == 3 * 32 * hkv * d * 2 * 4
    # fp8 K/V: one byte per value, q/o unchanged
    fp8 = bench.decode_bytes(ctx, hq, hkv, d, B, True, esize=2, kv_esize=1)
    assert fp8 == int(ctx.sum()) * hkv * d * 2 + 2 * 4 * hq * d * 2 + \
        table + 16


def test_traffic_records_parse():
    # Each record holds measured and algorithmic bytes per launch and the
    # hashes of its sources; bench.py reports the measured bytes only while
    # the hashes match (else None).
    sys.path.insert(0, ROOT)
    import bench
    for w, path in bench.TRAFFIC_PROFILES.items():
        # decode records count one launch; the prefill record a whole pass,
        # whose 64-query blocks each re-read their chunk's keys (so more
        # traffic over the algorithmic bytes is expected there)
        unit = "pass" if w in bench.PASS_PROFILES else "launch"
        hi = 3.0 if unit == "pass" else 1.3
        vals = {}
        hashes = 0
        for line in open(path):
            if line.startswith((f"traffic_bytes_per_{unit}:",
                                f"algorithmic_bytes_per_{unit}:")):
                k, v = line.split(":")
                vals[k] = int(v)
            hashes += line.startswith("source_sha256 ")
        assert hashes >= 2, w
        ratio = vals[f"traffic_bytes_per_{unit}"] / \
            vals[f"algorithmic_bytes_per_{unit}"]
        assert 1.0 <= ratio < hi, (w, ratio)
        t = bench.recorded_traffic(w)
        assert t is None or t == vals[f"traffic_bytes_per_{unit}"]
    assert bench.recorded_traffic("no_such_workload") is None


def test_read_ceilings_attach_to_decode_records(monkeypatch):
    # Each HBM record with a byte count gets the plain-read rate of its byte
    # count (layouts whose bytes differ by less than 1 MiB share one
    # measurement); MFMA records and records without a byte count are left
    # alone.
    sys.path.insert(0, ROOT)
    import bench
    calls = []

    def fake_plain_read(nbytes, device):
        calls.append(nbytes)
        nb = int(nbytes) // 16 * 16
        return {"bytes": nb, "us": 100.0, "GBps": 6400.0 if nb > 5e8 else
                6000.0, "workgroups_per_cu": 2}

    monkeypatch.setattr(bench, "plain_read", fake_plain_read)
    rl = {
        "paged": bench.roofline_record("hbm", 5880.0, 8000.0, "GB/s",
                                       bytes_per_launch=640109829),
        "contig": bench.roofline_record("hbm", 5900.0, 8000.0, "GB/s",
                                        bytes_per_launch=640070707),
        "fp8": bench.roofline_record("hbm", 4800.0, 8000.0, "GB/s",
                                     bytes_per_launch=320598892),
        "copy": bench.roofline_record("hbm", 3800.0, 8000.0, "GB/s"),
        "prefill": bench.roofline_record("mfma", 1200.0, 2500.0, "TFLOP/s"),
    }
    out = bench.add_read_ceilings(rl, None)
    assert calls == [640109829, 320598892]
    assert sorted(int(k) for k in out) == [320598880, 640109824]
    assert rl["paged"]["plain_read_GBps"] == 6400.0
    assert rl["contig"]["plain_read_GBps"] == 6400.0
    assert rl["paged"]["frac_of_plain_read"] == round(5880.0 / 6400.0, 4)
    assert rl["fp8"]["frac_of_plain_read"] == round(4800.0 / 6000.0, 4)
    assert "plain_read_GBps" not in rl["copy"]
    assert "plain_read_GBps" not in rl["prefill"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_noalloc_decode_rejects_oversized_workspace():
    """paged_attn_decode_noalloc refuses a shape whose workspace exceeds its
    16 MiB scratch before touching any device (forced here by a huge chunk
    count; host logic only, in a child process so that the override is read
    fresh)."""
    code = (
        "import ctypes\n"
        "from paged_kv_cache_191_amd import kvpaged as kv\n"
        "f = kv.lib().paged_attn_decode_noalloc\n"
        "p = ctypes.c_void_p(16)\n"
        "st = f(p, p, p, p, 4, p, 4, p, 64, 2, 32, 8, 128, 16, 0.1, "
        "kv.KV_BF16, None)\n"
        "print(st, kv.kv_last_error())\n")
    env = dict(os.environ, KVPAGED_DECODE_CHUNKS="100000")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    st, msg = r.stdout.split(" ", 1)
    assert int(st) == kv.KV_EINVAL
    assert "scratch" in msg
