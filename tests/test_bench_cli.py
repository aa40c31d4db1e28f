"""Host-side checks of bench.py: the one-GPU guard, and the stored counter
traffic keyed by workload names that the bench actually emits (a renamed
workload would otherwise silently report "traffic": null)."""
import json
import os
import subprocess
import sys

import coli_synth as cs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_keys_name_emitted_workloads():
    sys.path.insert(0, ROOT)
    import bench
    names = set()
    for cfg in cs.CONFIGS.values():
        for bits in (4, 8, 2):
            names.add(cfg.name + (f" int{bits} weights" if bits != 4 else ""))
    kernels = {"dec_gateup", "pf_gateup", "pack_fp8_gateup"}
    for (kernel, workload), nbytes in bench.TRAFFIC.items():
        assert kernel in kernels, kernel
        assert nbytes > 0
        if kernel == "pack_fp8_gateup":
            assert workload.startswith("pack_fp8 layer H"), workload
        else:
            assert workload in names, workload
