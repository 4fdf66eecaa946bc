"""Host-side checks of bench.py (no GPU): the one-GPU guard, the contract line,
the fractions of the probes, and the algorithmic FLOP and byte counts against
counts taken independently from the workload definitions."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_contract_line_carries_the_required_keys():
    class Args:
        steps, warmup = 7, 3

    res = dict(value=12.5, unit="GB/s", ms_per_step=0.25, config={"workload": "a workload"},
               roofline={"unit": "GB/s", "achieved": 12.5}, cpu_baseline={"value": 1.0})
    line = bench.contract_line(Args, res, "c2")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 7 and line["warmup"] == 3
    assert line["config"]["workload_name"] == "c2" and line["config"]["workload"] == "a workload"
    assert line["data"] == "synthetic" and line["higher_is_better"] is True
    json.dumps(line)


def test_fractions_of_the_probes():
    probes = dict(hbm_read_gbs=6400.0, hbm_copy_gbs=5000.0, mfma_bf16_tflops=2400.0)
    dec = {"roofline": {"unit": "GB/s", "achieved": 3200.0}}
    bench.against_probes(dec, probes)
    assert dec["roofline"]["frac_of_probe"] == 0.5 and dec["roofline"]["frac_of_copy_probe"] == 0.64
    # an extend at 1,000 FLOP/B: the MFMA probe bounds it
    ext = {"roofline": {"unit": "TFLOP/s", "achieved": 600.0, "tflops": 600.0, "achieved_gbs": 600.0}}
    bench.against_probes(ext, probes)
    assert ext["roofline"]["frac_of_probe"] == 0.25
    assert ext["roofline"]["attainable_tflops_of_probes"] == 2400.0
    # at 100 FLOP/B the read probe bounds it: 100 x 6.4 TB/s = 640 TFLOP/s
    low = {"roofline": {"unit": "GB/s", "achieved": 3200.0, "tflops": 320.0, "achieved_gbs": 3200.0}}
    bench.against_probes(low, probes)
    assert low["roofline"]["attainable_tflops_of_probes"] == 640.0
    assert low["roofline"]["frac_of_attainable_of_probes"] == 0.5


def test_extend_flops_count_every_window_pair():
    from sliding_window_attention_swa_amd import workloads as W
    wl = W.c3_extend_bf16()
    flops, ext_bytes, store_bytes, keys = bench.extend_counts(wl)
    pairs = sum(min(i, wl.window) + 1 for b in range(wl.batch)
                for i in range(int(wl.prefix_lens[b]), int(wl.seq_lens[b])))
    assert flops == pairs * wl.q_heads * wl.head_dim * 4 == 34_628_173_824  # the 34.63 GFLOP of C3
    total_q = wl.q.shape[0]
    assert ext_bytes > 2 * total_q * wl.q_heads * wl.head_dim * 2 + keys * wl.kv_heads * wl.head_dim * 2 * 2
    assert store_bytes == total_q * wl.kv_heads * wl.head_dim * 2 * 2 * 2 + total_q * 8


def test_decode_bytes_count_the_window():
    from sliding_window_attention_swa_amd import workloads as W
    wl = W.c2_decode_bf16()
    dec, store, translate, fused, flops = bench.decode_bytes(wl, "bf16")
    keys = np.minimum(wl.seq_lens.astype(np.int64), wl.window + 1)
    kv = int(keys.sum()) * wl.kv_heads * wl.head_dim * 2 * 2
    assert kv == 33_816_576  # every C2 request holds a full window of 129 keys
    assert dec == kv + wl.batch * wl.q_heads * wl.head_dim * (2 + 2) + int(keys.sum()) * 4 + (wl.batch + 1) * 4
    assert fused and store == wl.batch * wl.kv_heads * wl.head_dim * 2 * 2 + wl.batch * 8
    assert flops == int(keys.sum()) * wl.q_heads * wl.head_dim * 4
