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


def test_traffic_summary_reads_the_rocprof_counter_files(tmp_path):
    # two counter passes in rocprofv3's CSV form: the 256 MiB calibration copy
    # and the two decode instantiations (rows rounded up to 4 and 8), each
    # counter summed over its instances; FETCH_SIZE reads half the bytes
    from weight_only_int4_unpack_amd import traffic
    dec = ("void w4a16::(anonymous namespace)::decode_kernel<w4a16::(anonymous namespace)::BF16, "
           "false, 1, true, 4, {mt}, false>(w4a16::DecodeParams)")
    kib = {"FETCH_SIZE": {"copy": 131072.0, 4: 22000.0, 8: 24000.0},
           "WRITE_SIZE": {"copy": 262144.0, 4: 700.0, 8: 3600.0}}
    for counter, vals in kib.items():
        d = tmp_path / counter
        d.mkdir()
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        did = 0
        for key, v in vals.items():
            name = "__amd_rocclr_copyBuffer" if key == "copy" else dec.format(mt=key)
            for _ in range(3):
                did += 1
                rows += [f'{did},"{name}",{counter},{v / 2}'] * 2   # two instances
        (d / "bench_counter_collection.csv").write_text("\n".join(rows) + "\n")
    rec = traffic.summarise(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"))
    r = rec["decode_m1+decode_m5"]
    assert r["calibration"]["fetch_scale"] == 2.0 and r["calibration"]["write_scale"] == 1.0
    assert r["read_bytes"] == {"M=1": 22000 * 2048, "M=5": 24000 * 2048}
    assert r["write_bytes"] == {"M=1": 700 * 1024, "M=5": 3600 * 1024}
    assert r["bytes_per_launch"] == (22000 * 2048 + 700 * 1024 + 24000 * 2048 + 3600 * 1024) // 2
    assert r["kernel_sha"] == bench.kernel_source_hash()
