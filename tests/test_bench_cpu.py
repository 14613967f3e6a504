"""Host-side logic of bench.py, without a GPU: the one-GPU contract, the
algorithmic byte counts the roofline line divides by, and the rule that a
committed counter record is only reported for the kernel source it was taken on.
"""
import hashlib
import json
import os
import shutil
import subprocess
import sys

import bench
from compressed_sparse_attention_csa_amd import accounting as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_scan_bytes_per_launch():
    # 4 queries x (262,144 fp8 keys of 64 B + 4,096 page scales of 4 B + 4 indexer query heads of 64 bf16
    # + 4 head weights of 4 B)
    per_q = 262144 * 64 + 4096 * 4 + 4 * 64 * 2 + 4 * 4
    assert bench.scan_bytes_per_launch() == 4 * per_q == 67176512


def test_step_bytes_add_up():
    # per query: its key stream and page scales, q^I, w and the Top-K row written; then per layer the
    # gathered fp8 K and V rows with their page scales, the bf16 window rows, q, out and the Top-K row read
    attend = 1024 * 2 * (128 + 4) + 128 * 2 * 128 * 2 + 2 * 64 * 128 * 2 + 1024 * 4
    assert A.attend_bytes(1024, 128, 128, 64, "fp8", "bf16") == attend
    per_q = 262144 * 64 + 4096 * 4 + 4 * 64 * 2 + 4 * 4 + 1024 * 4 + 4 * attend
    assert bench.step_bytes() == 4 * per_q == 73156672


def test_traffic_record_gated_by_kernel_source(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "compressed_sparse_attention_csa_amd", "csrc", "index.hip")
    rec = {"source_sha256": None, "bytes_per_launch": 123456, "scope": "read + write"}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "compressed_sparse_attention_csa_amd" / "csrc").mkdir(parents=True)
    shutil.copy(src, tmp_path / "compressed_sparse_attention_csa_amd" / "csrc" / "index.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = tmp_path / "profiles" / "index_scan_1m_decode_traffic.json"
    rec["source_sha256"] = sha
    path.write_text(json.dumps(rec))
    assert bench.traffic_from_profiles() == (123456, "read + write")
    rec["source_sha256"] = "0" * 64            # taken on another source: not reported
    path.write_text(json.dumps(rec))
    assert bench.traffic_from_profiles() == (None, None)
    path.unlink()                              # no record
    assert bench.traffic_from_profiles() == (None, None)


def test_compress_bytes_of_one_token_appends():
    # fp8 pages, bf16 rows and window ring (R = 128), r = 4, with the indexer.
    # Token 11 closes block 2 (entry 2, slot 2 of page 0): the new row's gate/K/V,
    # rows 8-10 back from block staging, the row into the ring, the projection
    # (128 x 64 fp32), page 0's two earlier entries from fp32 staging, all three
    # entries' K/V/indexer codes and the three page scales, the new entry's staging.
    row = 3 * 128 * 2
    closing = row + 3 * row + 2 * 128 * 2 + 128 * 64 * 4 + 2 * 320 * 4 + 3 * 320 + 3 * 4 + 320 * 4
    assert A.compress_bytes(11, 1, 4, 128, 64, "fp8", "bf16", 128) == closing == 41164
    # token 12 opens block 3: the row in, into block staging and into the ring
    assert A.compress_bytes(12, 1, 4, 128, 64, "fp8", "bf16", 128) == row + row + 2 * 128 * 2
    # the entry that fills page 0 (slot 63) leaves no staging behind
    full = row + 3 * row + 512 + 128 * 64 * 4 + 63 * 320 * 4 + 64 * 320 + 3 * 4
    assert A.compress_bytes(255, 1, 4, 128, 64, "fp8", "bf16", 128) == full
    # bf16 pages write only the new entry
    assert A.compress_bytes(11, 1, 4, 128, 64, "bf16", "bf16", 128) == row + 3 * row + 512 + 128 * 64 * 4 + 320 * 2


def test_attend_bytes_per_launch():
    # 4 queries, one layer: gathered fp8 K/V rows with page scales, bf16 window rows, q, out, Top-K row
    assert bench.attend_bytes_per_launch() == 4 * (1024 * 2 * (128 + 4) + 128 * 2 * 128 * 2 + 2 * 64 * 128 * 2
                                                   + 1024 * 4) == 1490944
