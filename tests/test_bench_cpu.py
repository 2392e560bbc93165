"""CPU checks of the benchmark's own arithmetic: the algorithmic bytes and flops its roofline
fractions divide by, written out from the layer's shapes, and its one-GPU refusal."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_moe_layer_sigmoid_amd import inputs as I  # noqa: E402


def test_gate_up_bytes_bf16_headline():
    """Every routed expert active: W13 of 257 experts (2I x d bf16), x once (T x d), h once
    (T(K+1) x I): the 15,300,820,992 bytes the headline roofline uses."""
    c = I.V3_BF16
    want = 257 * (2 * 2048) * 7168 * 2 + 4096 * 7168 * 2 + 4096 * 9 * 2048 * 2
    assert want == 15_300_820_992
    assert bench.gate_up_bytes(c, np.ones(256, dtype=np.int64), False) == want
    # an expert with no rows contributes no weight bytes
    counts = np.ones(256, dtype=np.int64)
    counts[:10] = 0
    assert bench.gate_up_bytes(c, counts, False) == want - 10 * (2 * 2048) * 7168 * 2


def test_gate_up_bytes_fp8_counts_scales():
    c = I.V3_FP8
    T, d, i2 = c.T, c.d, 2 * c.inter
    w = 257 * (i2 * d + (i2 // 128) * (d // 128) * 4)
    a = T * d + T * (d // 128) * 4
    h = T * 9 * c.inter + T * 9 * (c.inter // 128) * 4
    assert bench.gate_up_bytes(c, np.ones(256, dtype=np.int64), True) == w + a + h
    # E8M0 codes are one byte each
    w8 = 257 * (i2 * d + (i2 // 128) * (d // 128))
    a8 = T * d + T * (d // 128)
    h8 = T * 9 * c.inter + T * 9 * (c.inter // 128)
    assert bench.gate_up_bytes(c, np.ones(256, dtype=np.int64), True, 1) == w8 + a8 + h8


def test_down_and_combine_bytes():
    c = I.V3_BF16
    w = 257 * 7168 * 2048 * 2
    h = 4096 * 9 * 2048 * 2
    y = 4096 * 8 * 7168 * 2 + 4096 * 7168 * 4
    assert bench.down_bytes(c, np.ones(256, dtype=np.int64), False) == w + h + y
    assert bench.combine_bytes(c) == 4096 * 8 * 7168 * 2 + 4096 * 7168 * 4 + 4096 * 7168 * 2


def test_layer_and_backward_flops():
    """Router 2 T d N plus 3 SwiGLU products of 2 d I flops each per token and expert (K
    routed + 1 shared); the backward is twice that (Dgrad and Wgrad)."""
    c = I.V3_BF16
    f = 2 * 4096 * 7168 * 256 + 3 * 2 * 7168 * 2048 * 4096 * 9
    assert bench.layer_flops(c) == f
    assert bench.backward_flops(c) == 2 * f


def test_roofline_bound_from_arithmetic_intensity():
    """The gate/up roofline is taken against the matrix cores only above the ridge point of its
    dtype's peak (bf16 2.5 PFLOP/s / 8 TB/s = 312.5 flop/B, E4M3 625): the bf16 T = 4096
    headline (141 flop/B) and the E4M3 decode step are HBM-bound, the E4M3 T = 16384 layer
    (1085 flop/B) is matrix-core-bound; the fractions divide by the matching peak."""
    for cfg, fp8, bound in ((I.V3_BF16, False, "hbm"), (I.V3_FP8, True, "mfma"), (I.V3_DECODE, True, "hbm")):
        flop = 4 * cfg.rows * cfg.d * cfg.inter
        nbytes = bench.gate_up_bytes(cfg, np.ones(256, dtype=np.int64), fp8)
        r = bench.gate_up_roofline(flop, nbytes, 2.0, fp8)
        assert r["bound"] == bound, cfg.name
        if bound == "hbm":
            assert r["unit"] == "GB/s" and abs(r["frac"] - nbytes / 2e-3 / 8e12) < 1e-4
        else:
            assert r["unit"] == "TFLOP/s" and abs(r["frac"] - flop / 2e-3 / 5e15) < 1e-4
    assert bench.gate_up_roofline(312.6e9, 1e9, 1.0, False)["bound"] == "mfma"
    assert bench.gate_up_roofline(312.4e9, 1e9, 1.0, False)["bound"] == "hbm"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
