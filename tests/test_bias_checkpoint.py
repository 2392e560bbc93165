"""Checkpoint / resume of the bias loop, on the CPU: the decode-shaped run (T = 256 fresh tokens
per step, 256 experts, top-8, Zipf-skewed starting bias, gamma = 0.001) driven by the oracle's
routing and bias rule for 100 steps straight through, against 50 steps, a save of the bias
state to a file, the bias overwritten, a restore and 50 steps more.  The two final biases must
be bit-identical.  (The GPU counterpart runs the device layer the same way.)"""
import os
import tempfile
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_moe_layer_sigmoid_amd import inputs as I
from sparse_moe_layer_sigmoid_amd.state import load_bias_state, save_bias_state


def _oracle_steps(cfg, wr64, layer, start, stop):
    for step in range(start, stop):
        x = I.gen_x(cfg, step=step).double().numpy()
        b = layer.bias.numpy()
        r = O.route(x, wr64, b, cfg.top_k)
        nb = O.bias_update(b, O.expert_counts(r["idx"], cfg.n_experts), cfg.T, cfg.top_k, cfg.gamma)
        layer.bias.copy_(torch.from_numpy(nb))


def test_bias_loop_checkpoint_resume():
    cfg = I.V3_DECODE
    wr64 = I.gen_router(cfg).double().numpy()
    b0 = I.gen_bias(cfg)
    straight = SimpleNamespace(bias=b0.clone())
    _oracle_steps(cfg, wr64, straight, 0, cfg.steps)
    resumed = SimpleNamespace(bias=b0.clone())
    half = cfg.steps // 2
    _oracle_steps(cfg, wr64, resumed, 0, half)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "bias_state.safetensors")
        save_bias_state(path, resumed, step=half)
        resumed.bias.fill_(float("nan"))
        start = load_bias_state(path, resumed)
    assert start == half
    _oracle_steps(cfg, wr64, resumed, start, cfg.steps)
    assert np.array_equal(resumed.bias.numpy().view(np.uint32), straight.bias.numpy().view(np.uint32))
    assert not np.array_equal(straight.bias.numpy(), b0.numpy())   # the loop really moved the bias


def test_bias_state_rejects_wrong_shape():
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "s.safetensors")
        save_bias_state(path, SimpleNamespace(bias=torch.zeros(16)), step=3)
        with pytest.raises(ValueError):
            load_bias_state(path, SimpleNamespace(bias=torch.zeros(32)))
        ok = SimpleNamespace(bias=torch.ones(16))
        assert load_bias_state(path, ok) == 3 and bool((ok.bias == 0).all())
