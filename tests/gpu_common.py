"""Shared helpers of the GPU parity tests: device transfer, metrics, tie-window checks."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

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


# The fp8 matrix cores add products in groups of 8 K and keep about 13 bits below each
# group's largest term (measured in test_gpu_fp8_precision): a dot product's error is a small
# multiple of 2^-12 * sum |a_k w_k|.  The bound used in the checks is 2^-10 * sum |a_k w_k|.
FP8_DOT_REL = 2.0 ** -10


def fp8_staged_check(pick, x_rows, gi, pp, gate_of, n_experts, expert_weights, buf, out32, tol, e8m0=False):
    """The fp8 layer checked stage by stage on the tokens `pick`.

    The stored h of the fp8 path is an E4M3 code chosen by rounding a floating-point value,
    so where the device's and the oracle's accumulations straddle a rounding midpoint, two
    codes are both correct.  The check therefore (1) bounds every stored h value, the device
    code times its 1x128 scale, against the oracle's exact h: within one E4M3 half-step at
    the device's scale plus the fp8 dot-product bound pushed through SwiGLU, and the device's
    tile scales against the oracle's; then (2) recomputes the down projections and the
    combine in the oracle from the device's stored h and compares the layer output at `tol`.

    x_rows: [len(pick), d] the picked tokens' bf16 inputs (float64).
    gi, pp: the device's top-K indices and pair rows (numpy), for all tokens.
    gate_of(t, e): the oracle's gate of expert e for token t.
    e8m0: the power-of-two scale variant (the device's scales are E8M0 codes); a device h
    scale may then be the neighbouring power of two when the tile max lies within the
    dot-product error of a power-of-two boundary.
    Returns (staged error, fraction of h codes equal to the oracle's)."""
    qw, qa = O._quantisers("fp8_e8m0" if e8m0 else "fp8")
    h_codes = buf["h"].cpu().numpy()
    h_scales = buf["hs"].cpu().numpy()
    if e8m0:
        h_scales = O.e8m0_decode(h_scales)
    shared_base = int(buf["expert_offsets"][n_experts].item())
    K = gi.shape[1]
    xd = O.dequant_1x128(*qa(O.fp32_round(x_rows)))

    def deq_pair(e):
        w13, w2 = expert_weights(e)
        return O.dequant_128x128(*qw(w13)), O.dequant_128x128(*qw(w2))

    needed = sorted({int(e) for t in pick for e in gi[t]} | {n_experts})
    with ThreadPoolExecutor(16) as ex:
        cache = dict(zip(needed, ex.map(deq_pair, needed)))
    deq = cache.__getitem__

    y_routed = np.zeros((len(pick) * K, x_rows.shape[1]))
    y_shared = np.zeros((len(pick), x_rows.shape[1]))
    gates = np.zeros((len(pick), K))
    n_same = n_all = 0
    for j, t in enumerate(pick):
        for k in range(K + 1):
            e = int(gi[t, k]) if k < K else n_experts
            row = int(pp[t, k]) if k < K else shared_base + int(t)
            w13, w2 = deq(e)
            inter = w13.shape[0] // 2
            a = xd[j] @ w13[:inter].T
            c = xd[j] @ w13[inter:].T
            h = O.silu(a) * c
            da = FP8_DOT_REL * (np.abs(xd[j]) @ np.abs(w13[:inter]).T)
            dc = FP8_DOT_REL * (np.abs(xd[j]) @ np.abs(w13[inter:]).T)
            eps = 1.1 * da * np.abs(c) + np.abs(O.silu(a)) * dc + da * dc + 2.0 ** -18 * np.abs(h)
            s_dev = h_scales[row].astype(np.float64)
            s_orc = qa(O.fp32_round(h[None]))[1][0].astype(np.float64)
            tile_eps = eps.reshape(-1, 128).max(axis=1)
            if e8m0:
                amax = np.abs(h).reshape(-1, 128).max(axis=1)
                may_be_zero = amax - tile_eps <= 0  # an all-zero tile takes scale 1
                lo = np.where(may_be_zero, 2.0 ** -127, np.exp2(O.e8m0_exponent(np.maximum(amax - tile_eps, 0.0))))
                hi = np.maximum(np.exp2(O.e8m0_exponent(amax + tile_eps)), np.where(may_be_zero, 1.0, 0.0))
                assert np.all((s_dev >= np.minimum(lo, s_orc)) & (s_dev <= np.maximum(hi, s_orc))), (t, e)
            else:
                assert np.all(np.abs(s_dev - s_orc) <= tile_eps / 448 + 2.0 ** -22 * s_orc), (t, e)
            s_el = np.repeat(s_dev, 128)
            h_dev = O.dequant_1x128(h_codes[row][None], h_scales[row][None])[0]
            step = O.e4m3_half_ulp(np.minimum((np.abs(h) + eps) / s_el, 448.0)) * s_el
            bad = np.abs(h_dev - h) > step * 1.0001 + eps
            assert not bad.any(), (t, e, np.nonzero(bad)[0][:5], h_dev[bad][:5], h[bad][:5])
            n_same += int(np.sum(h_codes[row] == qa(O.fp32_round(h[None]))[0][0]))
            n_all += h.size
            y = h_dev @ w2.T
            if k < K:
                y_routed[j * K + k] = O.bf16_round(y)
                gates[j, k] = gate_of(int(t), e)
            else:
                y_shared[j] = O.fp32_round(y)
    ref = O.combine(y_routed, y_shared, np.arange(len(pick) * K).reshape(len(pick), K), gates)
    got = out32[torch.as_tensor(np.asarray(pick), device=out32.device)].cpu().numpy().astype(np.float64)
    err = rel_err(got, ref)
    assert err <= tol, err
    return err, n_same / max(n_all, 1)
