"""Host-side logic of bench.py (no GPU): the one-GPU guard and the algorithmic
bytes and flops that the roofline fractions divide by, restated from the layer's
shapes."""
import os
import subprocess
import sys

import numpy as np

import bench
from int4_routed_expert_moe_amd import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_work_from_the_shapes():
    """K2.5 decode (T=64, H=7168, I=2048, top-8) with 291 active experts: gate and
    up are 2 x 2048 x 7168 int4 weights (half a byte each) plus one 2-byte scale
    per 32 of them, per expert; x is read once in bf16, h (512 slot rows x 2048)
    written once."""
    cfg = synthetic.WORKLOADS[2]
    counts = np.zeros(cfg["E"], np.int64)
    counts[:291] = 1
    work, _, _, active = bench.algorithmic_work(cfg, counts, cfg["shared_I"])
    assert active == 291
    per_expert_gu = 2 * 2048 * 7168 // 2 + 2 * 2048 * (7168 // 32) * 2
    assert per_expert_gu == 16_515_072
    gu_bytes, gu_flops = work["moe_int4_grouped_swiglu"]
    assert gu_bytes == 291 * per_expert_gu + 64 * 7168 * 2 + 512 * 2048 * 2 == 4_808_900_608
    assert gu_flops == 2 * 512 * 2 * 7168 * 2048
    d_bytes, d_flops = work["moe_int4_grouped_down"]
    assert d_bytes == 291 * (7168 * 2048 // 2 + 7168 * (2048 // 32) * 2) + 512 * 2048 * 2 + 512 * 7168 * 2
    assert d_flops == 2 * 512 * 2048 * 7168


def test_exact_work_counts_int8_activations_and_fp32_outputs():
    cfg = synthetic.WORKLOADS[4]
    counts = np.ones(cfg["E"], np.int64)
    work, _, _, active = bench.algorithmic_work(cfg, counts, None)
    T, H, I, S = cfg["T"], cfg["H"], cfg["I"], cfg["T"] * cfg["k"]
    assert active == cfg["E"]
    gu_bytes, _ = work["moe_int4_grouped_swiglu"]
    # int8 codes and an fp32 scale per group of 32, in and out
    assert gu_bytes == (cfg["E"] * (2 * I * H // 2 + 2 * I * (H // 32) * 2) + T * H + T * (H // 32) * 4
                        + S * I + S * (I // 32) * 4)
    d_bytes, _ = work["moe_int4_grouped_down"]
    assert d_bytes == cfg["E"] * (H * I // 2 + H * (I // 32) * 2) + S * I + S * (I // 32) * 4 + S * H * 4
