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


def fp8_end_to_end_bar(err: float, case: str):
    """The 3e-2 bar on the fp8 layer end to end against the oracle's fp8 pipeline.

    The device and the oracle each round h to E4M3 codes from their own sum: the oracle's is
    exact, the matrix cores add 8 products at a time keeping about 13 bits below the largest
    (measured in test_gpu_fp8_precision), so ~0.4% of the codes sit one step apart where the
    two sums straddle a rounding midpoint, and a code one step away on a large h moves an
    output by a few percent of the output's RMS.  Where that pushes the end-to-end figure past
    the bar the test records an expected failure carrying the measured value (a miss of the
    bar, not a pass); the staged check, which holds every stored h to its bound and the rest
    of the layer to 3e-2, stays asserted."""
    if err > FP8_TOL:
        import pytest
        pytest.xfail(f"{case}: fp8 end to end vs the oracle's fp8 pipeline {err:.3e} > {FP8_TOL} "
                     f"(E4M3 h codes one step apart at rounding midpoints)")


# The fp8 matrix cores add products in groups of 8 K and keep about 13 bits below each
# group's largest term (measured in test_gpu_fp8_precision): a dot product's error is a small
# multiple of 2^-12 * sum |a_k w_k|.  The bound used in the checks is 2^-10 * sum |a_k w_k|.
FP8_DOT_REL = 2.0 ** -10


def fp8_staged_check(pick, x_rows, gi, pp, gate_of, n_experts, expert_weights, buf, out32, tol, e8m0=False,
                     weights_quantised=False, workers=16):
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
    expert_weights(e): the expert's weights (w13, w2), or with weights_quantised=True those
    weights already block-quantised and dequantised by the oracle.
    e8m0: the power-of-two scale variant (the device's scales are E8M0 codes); a device h
    scale may then be the neighbouring power of two when the tile max lies within the
    dot-product error of a power-of-two boundary.
    Returns (staged error, fraction of h codes equal to the oracle's)."""
    batch = dict(pick=pick, x_rows=x_rows, gi=gi, pp=pp, gate_of=gate_of, buf=buf, out32=out32)
    errs, same = fp8_staged_check_batches([batch], n_experts, expert_weights, tol, e8m0, weights_quantised, workers)
    return errs[0], same


def fp8_staged_check_batches(batches, n_experts, expert_weights, tol, e8m0=False, weights_quantised=False,
                             workers=16):
    """fp8_staged_check over several forwards that share the expert weights (e.g. steps of a
    decode loop): each expert's weights are fetched once for all of them.  Each batch is a
    dict of the arguments pick, x_rows, gi, pp, gate_of, buf, out32.  Work is done expert by
    expert (all picked rows of an expert at once, experts in parallel).
    Returns ([staged error per batch], fraction of h codes equal to the oracle's)."""
    qw, qa = O._quantisers("fp8_e8m0" if e8m0 else "fp8")
    st = []
    for b in batches:
        h_scales = b["buf"]["hs"].cpu().numpy()
        st.append(dict(pick=np.asarray(b["pick"]), gi=b["gi"], pp=b["pp"], h_codes=b["buf"]["h"].cpu().numpy(),
                       h_scales=O.e8m0_decode(h_scales) if e8m0 else h_scales,
                       shared_base=int(b["buf"]["expert_offsets"][n_experts].item()),
                       xd=O.dequant_1x128(*qa(O.fp32_round(b["x_rows"])))))
    K = batches[0]["gi"].shape[1]
    d = batches[0]["x_rows"].shape[1]
    # (batch, picked-token index j, slot k) triples of each expert; slot K is the shared expert
    pairs = {}
    for bi, b in enumerate(st):
        for j, t in enumerate(b["pick"]):
            for k in range(K):
                pairs.setdefault(int(b["gi"][t, k]), []).append((bi, j, k))
        pairs.setdefault(n_experts, []).extend((bi, j, K) for j in range(len(b["pick"])))

    def one(e):
        bjk = np.array(pairs[e])
        w13, w2 = expert_weights(e)
        if not weights_quantised:
            w13, w2 = O.dequant_128x128(*qw(w13)), O.dequant_128x128(*qw(w2))
        inter = w13.shape[0] // 2
        out = []
        for bi in np.unique(bjk[:, 0]):
            b = st[bi]
            sel = bjk[:, 0] == bi
            js, ks = bjk[sel, 1], bjk[sel, 2]
            rows = np.where(ks < K, b["pp"][b["pick"][js], np.minimum(ks, K - 1)], b["shared_base"] + b["pick"][js])
            xe = b["xd"][js]
            a = xe @ w13[:inter].T
            c = xe @ w13[inter:].T
            h = O.silu(a) * c
            da = FP8_DOT_REL * (np.abs(xe) @ np.abs(w13[:inter]).T)
            dc = FP8_DOT_REL * (np.abs(xe) @ np.abs(w13[inter:]).T)
            eps = 1.1 * da * np.abs(c) + np.abs(O.silu(a)) * dc + da * dc + 2.0 ** -18 * np.abs(h)
            s_dev = b["h_scales"][rows].astype(np.float64)
            hq_orc, s_orc = qa(O.fp32_round(h))
            s_orc = np.asarray(s_orc, np.float64)
            tile_eps = eps.reshape(len(js), -1, 128).max(axis=2)
            if e8m0:
                amax = np.abs(h).reshape(len(js), -1, 128).max(axis=2)
                may_be_zero = amax - tile_eps <= 0  # an all-zero tile takes scale 1
                lo = np.where(may_be_zero, 2.0 ** -127, np.exp2(O.e8m0_exponent(np.maximum(amax - tile_eps, 0.0))))
                hi = np.maximum(np.exp2(O.e8m0_exponent(amax + tile_eps)), np.where(may_be_zero, 1.0, 0.0))
                ok_s = (s_dev >= np.minimum(lo, s_orc)) & (s_dev <= np.maximum(hi, s_orc))
            else:
                ok_s = np.abs(s_dev - s_orc) <= tile_eps / 448 + 2.0 ** -22 * s_orc
            assert ok_s.all(), (e, int(bi), np.argwhere(~ok_s)[:3])
            s_el = np.repeat(s_dev, 128, axis=1)
            h_dev = O.dequant_1x128(b["h_codes"][rows], b["h_scales"][rows])
            step = O.e4m3_half_ulp(np.minimum((np.abs(h) + eps) / s_el, 448.0)) * s_el
            bad = np.abs(h_dev - h) > step * 1.0001 + eps
            assert not bad.any(), (e, int(bi), np.argwhere(bad)[:5])
            y = h_dev @ w2.T
            y = O.bf16_round(y) if e < n_experts else O.fp32_round(y)
            out.append((bi, js, ks, y, int(np.sum(b["h_codes"][rows] == hq_orc)), h.size))
        return out

    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        results = [r for rs in ex.map(one, sorted(pairs)) for r in rs]
    y_routed = [np.zeros((len(b["pick"]) * K, d)) for b in st]
    y_shared = [np.zeros((len(b["pick"]), d)) for b in st]
    n_same = n_all = 0
    for bi, js, ks, y, same, n in results:
        routed = ks < K
        y_routed[bi][js[routed] * K + ks[routed]] = y[routed]
        y_shared[bi][js[~routed]] = y[~routed]
        n_same += same
        n_all += n
    errs = []
    for bi, (b, sb) in enumerate(zip(batches, st)):
        pick = sb["pick"]
        gates = np.array([[b["gate_of"](int(t), int(sb["gi"][t, k])) for k in range(K)] for t in pick])
        ref = O.combine(y_routed[bi], y_shared[bi], np.arange(len(pick) * K).reshape(len(pick), K), gates)
        got = b["out32"][torch.as_tensor(pick, device=b["out32"].device)].cpu().numpy().astype(np.float64)
        err = rel_err(got, ref)
        assert err <= tol, (bi, err)
        errs.append(err)
    return errs, n_same / max(n_all, 1)
