"""bench.py on the CPU: the one-GPU rule of its command line, and the HBM counter record it
reports as roofline.traffic (profiles/lrkv_decode_c1_traffic.json)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ALG_BYTES = 2 * 2 * 8 * 4096 * (128 + 16 * 56)  # eq 9 at B=8, T=4096, H=16, d_h=128, r=56


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_traffic_record_is_consistent():
    with open(os.path.join(ROOT, "profiles", "lrkv_decode_c1_traffic.json")) as f:
        rec = json.load(f)
    cal = rec["calibration"]
    cnt = rec["counters_kib_per_dispatch"]
    split = next(k for k in cnt if k.startswith("decode_split_kernel") and k.endswith("true>"))
    merge = next(k for k in cnt if k.startswith("merge_expand_kernel"))
    # HBM bytes of one call = (FETCH_SIZE x the copy calibration + WRITE_SIZE) KiB, split +
    # merge (the record holds the counters to 0.1 KiB and the factor to four decimals)
    per = lambda k: (cnt[k]["FETCH_SIZE"] * cal["fetch_factor"] + cnt[k]["WRITE_SIZE"]) * 1024
    assert abs(per(split) + per(merge) - rec["hbm_bytes_per_call"]) <= 1e-4 * ALG_BYTES
    # the cache is read once: at least the algorithmic bytes, and not much more
    assert ALG_BYTES <= rec["hbm_bytes_split_kernel"] <= 1.1 * ALG_BYTES
    assert rec["hbm_bytes_per_call"] <= 1.1 * ALG_BYTES
