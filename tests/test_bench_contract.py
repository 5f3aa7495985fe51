"""CPU checks of bench.py's contract that need no GPU.

* ``--gpus N`` with N > 1 exits with a message (one GPU only);
* the algorithmic byte and flop counts it divides by, checked against the
  figures of the target workloads (packed weights + scales + zero points +
  activations + output; 2 M N K);
* the traffic record under profiles/ is read only when its kernel hash
  matches the kernel source.
"""
import json
import os
import subprocess
import sys

import bench
from weight_only_int4_unpack_amd import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_and_flops():
    W = synthetic.WORKLOADS
    assert bench.alg_bytes(W["decode_m1"]) == 46002176
    assert bench.alg_bytes(W["decode_m5"]) == 46182400
    assert bench.alg_bytes(W["k2112"]) == 5944832
    assert bench.alg_bytes(W["prefill"]) == 138231808
    assert bench.alg_bytes(W["sweep_pc16"]) == 8660992
    assert bench.flops(W["prefill"]) == 365072220160
    assert bench.flops(W["decode_m5"]) == 891289600


def test_traffic_record_is_tied_to_the_kernel_source(tmp_path):
    rec = {"decode_m1+decode_m5": {"bytes_per_launch": 123, "kernel_sha": bench.kernel_source_hash()}}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(rec))
    assert bench.load_traffic(str(p), "decode_m1+decode_m5", bench.kernel_source_hash()) == 123
    assert bench.load_traffic(str(p), "decode_m1+decode_m5", "0" * 16) is None
    assert bench.load_traffic(str(p), "prefill", bench.kernel_source_hash()) is None
