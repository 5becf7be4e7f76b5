"""The bench's byte counts and pool figures (CPU): what roofline.achieved,
value and the block-manager fields divide by, checked against hand-worked
cases and the pages' 13B figure."""
import os
import subprocess
import sys

import numpy as np

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_bytes_13b_token():
    """One token of the 13B shape (40 heads x 128, fp16) is 20 KiB of K+V per
    layer; over the model's 40 layers that is the 800 KiB per token the pages
    print (polomodov.tech "vLLM and PagedAttention" slide 5)."""
    total, kv = bench.decode_bytes([1], 40, 128, 2, 16)
    assert kv == 40 * 128 * 2 * 2
    assert kv * 40 == 800 * 1024
    # + q and out (one row each), one table entry, one context length
    assert total == kv + 2 * 40 * 128 * 2 + 4 + 4


def test_decode_bytes_counts_shared_blocks_per_sequence():
    ctx = [20, 18]
    total, kv = bench.decode_bytes(ctx, 2, 64, 2, 16)
    assert kv == 38 * 2 * 64 * 2 * 2
    assert total == kv + 2 * 2 * 2 * 64 * 2 + (2 + 2) * 4 + 2 * 4


def test_unique_kv_bytes_counts_shared_blocks_once():
    """Block 5 is shared by both sequences (16 tokens each); 6 holds 4 tokens of
    sequence 0, 7 holds 2 of sequence 1: 22 distinct token rows."""
    tables = np.array([[5, 6, 99], [5, 7, 99]], np.int32)
    assert bench.unique_kv_bytes(tables, [20, 18], 2, 64, 2, 16) == 22 * 2 * 64 * 2 * 2
    # a shared block counts the most tokens any sequence uses in it
    tables = np.array([[5, 99], [5, 99]], np.int32)
    assert bench.unique_kv_bytes(tables, [3, 9], 1, 64, 2, 16) == 9 * 64 * 2 * 2


def test_step_bytes():
    ctx = [10, 33]
    dec, _ = bench.decode_bytes(ctx, 4, 64, 2, 16)
    # + the cache write (read k, v; write both) + slots + one CoW copy of a block
    assert bench.step_bytes(ctx, 4, 64, 2, 16, 1) == \
        dec + 4 * 2 * 4 * 64 * 2 + 8 * 2 + 2 * 2 * 4 * 16 * 64 * 2


def test_block_manager_stats():
    class BM:
        def seq_len(self, s):
            return {0: 17, 1: 16, 2: 40}[s]

    class Eng:
        bm, NB = BM(), 100

    class WL:
        bs = 16
    tables = np.array([[5, 6, 99], [5, 99, 99], [7, 8, 9]], np.int32)
    st = bench.block_manager_stats(Eng(), [0, 1, 2], tables, WL())
    assert st["logical_blocks"] == 2 + 1 + 3
    assert st["blocks_in_use"] == 5
    assert st["useful_kv_fraction"] == round(73 / 96, 4)
    assert st["sharing_saving"] == round(1 - 5 / 6, 4)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_record_only_for_the_profiled_source(tmp_path, monkeypatch):
    """The roofline's traffic comes from a committed counter record only while
    the kernel sources hash to the values the counters were taken on."""
    import hashlib
    import json
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source v1")
    rec = {"sources": ["k.hip"],
           "source_sha256": hashlib.sha256(b"kernel source v1").hexdigest(),
           "traffic_bytes_per_launch": 1003.0, "algorithmic_bytes_per_launch": 1000,
           "summary": "profiles/x.md"}
    (tmp_path / "profiles" / "decode_w_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.load_traffic("decode_w")
    assert got["traffic_bytes_per_launch"] / got["algorithmic_bytes_per_launch"] == 1.003
    src.write_bytes(b"kernel source v2")          # the kernel changed since the counters
    assert bench.load_traffic("decode_w") is None
    assert bench.load_traffic("decode_missing") is None
