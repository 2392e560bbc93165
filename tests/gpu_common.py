"""Shared helpers of the GPU parity tests: device transfer, metrics, tie-window checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O

TIE_WINDOW = 1e-6   # tokens whose oracle z gap is below this may legitimately pick differently
BF16_TOL = 1e-2     # max |out - ref| / rms(ref), bf16 path
FP8_TOL = 3e-2      # same, fp8 path


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype in (torch.bfloat16, torch.float16) \
        else t.detach().cpu().numpy().astype(np.float64)


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms) if ref.size else 0.0


def check_route(gpu_idx, gpu_gate, gpu_counts, gpu_scores, r, n_experts, top_k):
    """Compare a GPU routing with the oracle's.  Returns the mask of tie-window tokens.

    Outside the tie window: the expert sets are identical and the gates agree within 1e-6.
    Inside it: the GPU's set must still be a valid top-K, i.e. every pick has an oracle z
    within the window of the K-th best.  The counts must equal the histogram of the GPU's
    own indices, and the oracle's counts when no token is in the window."""
    gi = gpu_idx.cpu().numpy()
    gg = gpu_gate.cpu().numpy().astype(np.float64)
    gc = gpu_counts.cpu().numpy()
    T = gi.shape[0]
    if gpu_scores is not None:
        # soundness of the device's refinement rule: a token is recomputed in fp64 when its
        # fp32 margin is under 4e-6, so fp32 affinities must stay within 2e-6 of the truth
        ds = np.max(np.abs(gpu_scores.cpu().numpy().astype(np.float64) - r["s"])) if T else 0.0
        say(f"  max |s_gpu - s_oracle| = {ds:.3e}")
        assert ds < 2e-6, f"affinity error {ds} breaks the refinement argument"
    tie = (r["margin"] < TIE_WINDOW) | (r["group_margin"] < TIE_WINDOW)
    n_diff = sum(set(gi[t]) != set(r["idx"][t]) for t in range(T))
    say(f"  tokens in the tie window: {int(tie.sum())}; tokens whose expert set differs from the oracle's: {n_diff}")
    for t in range(T):
        assert len(set(gi[t])) == top_k and gi[t].min() >= 0 and gi[t].max() < n_experts
        assert abs(gg[t].sum() - 1.0) < top_k * 2.0 ** -23
        if not tie[t]:
            assert set(gi[t]) == set(r["idx"][t]), (t, gi[t], r["idx"][t])
            want = dict(zip(r["idx"][t], r["gate"][t]))
            for e, g in zip(gi[t], gg[t]):
                assert abs(g - want[e]) <= 1e-6, (t, e, g, want[e])
        else:
            zk = np.sort(r["z"][t][list(r["idx"][t])])[0]
            assert all(r["z"][t][e] >= zk - TIE_WINDOW for e in gi[t]), (t, gi[t])
    assert np.array_equal(gc, np.bincount(gi.ravel(), minlength=n_experts))
    if not tie.any():
        assert np.array_equal(gc, O.expert_counts(r["idx"], n_experts))
    return tie


def check_permutation_properties(offs, sorted_token, pair_pos, idx, n_experts):
    """Properties of a permutation that hold for any input: offsets are the exclusive scan
    of the loads, every pair's row points back to its token, each expert's rows are in token
    order, and the shared segment is the identity."""
    off = offs.cpu().numpy()
    st = sorted_token.cpu().numpy()
    pp = pair_pos.cpu().numpy()
    gi = idx.cpu().numpy()
    T, K = gi.shape
    counts = np.bincount(gi.ravel(), minlength=n_experts)
    assert off[0] == 0 and np.array_equal(np.diff(off[:n_experts + 1]), counts)
    assert off[n_experts + 1] == T * K + T
    assert np.all(st[pp.ravel()] == np.repeat(np.arange(T), K))
    assert len(np.unique(pp)) == T * K
    for e in range(n_experts):
        seg = st[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert (gi[seg] == e).any(axis=1).all()
    assert np.array_equal(st[T * K:], np.arange(T))
