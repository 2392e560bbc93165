"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with its pin.
``test_oracle_pins.py`` runs them; ``test_oracle_mutations.py`` plants plausible mistakes
in the oracle and checks that at least one pin fails for each.

What the pins rest on:
* library routines: torch's bfloat16 and float8_e4m3fn conversions, torch.sigmoid,
  torch.nn.functional.silu and matmul, numpy bincount / stable argsort;
* the OCP E4M3FN format's published constants (max 448, min subnormal 2^-9, ...);
* brute force over all K-subsets / all expert pairs on tiny inputs;
* closed forms (hand-computed bias steps, exactly representable fp8 products);
* invariants the pages fix ("DeepSeek-V3 Technical Report" wiki summary,
  "DeepSeekMoE と補助損失なしの負荷分散": K distinct experts per token, gates from the
  normalised original affinities so they sum to one and do not depend on the bias,
  overloaded -> -gamma, underloaded -> +gamma, no token dropped).
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

from oracle import moe_oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ storage formats


def pin_bf16_round_vs_torch():
    r = _rng(1)
    v = (r.standard_normal(20000) * np.exp2(r.integers(-30, 30, 20000))).astype(np.float32)
    # exact midpoints between neighbouring bf16 values (ties must go to even)
    b = torch.from_numpy(r.standard_normal(4000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    mid = (b.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, mid, -mid, np.float32([0.0, 1.0, -2.5])])
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = O.bf16_round(v)
    assert np.array_equal(got, ref), "bf16 rounding differs from torch"


def pin_e4m3_constants():
    d = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0          # largest finite
    assert d[0x01] == 2.0 ** -9                            # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9                        # largest subnormal
    assert d[0x08] == 2.0 ** -6                            # smallest normal
    assert d[0x38] == 1.0 and d[0x39] == 1.125 and d[0x40] == 2.0
    assert d[0x00] == 0.0 and np.signbit(d[0x80])
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(np.isnan(d)) == 2                        # no other NaN, no infinities
    assert np.all(np.isfinite(d[~np.isnan(d)]))


def pin_e4m3_vs_torch():
    r = _rng(2)
    v = np.concatenate([
        r.uniform(-448, 448, 50000),
        r.standard_normal(50000) * np.exp2(r.integers(-12, 8, 50000)),
    ]).astype(np.float32)
    pos = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)     # exact in fp32
    v = np.concatenate([v, mids, -mids, pos.astype(np.float32)])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(v)
    assert np.array_equal(got, ref), "E4M3 encode differs from torch.float8_e4m3fn"


def pin_e4m3_roundtrip_ties_saturation():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)
    pos = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    for c in range(126):  # midpoint between code c and c+1 goes to the even one
        m = (pos[c] + pos[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert O.e4m3_encode(m) == want, (c, m)
        # just off the midpoint goes to the nearer one
        assert O.e4m3_encode(np.nextafter(m, 0)) == c
        assert O.e4m3_encode(np.nextafter(m, 1e9)) == c + 1
    assert O.e4m3_encode(449.0) == 0x7E and O.e4m3_encode(1e30) == 0x7E
    assert O.e4m3_encode(-500.0) == 0xFE
    assert O.e4m3_encode(-1e-6) == 0x80 and O.e4m3_encode(1e-6) == 0x00


def pin_quant_1x128_properties():
    r = _rng(3)
    x = r.standard_normal((37, 512)).astype(np.float32)
    x[5, 128:256] = 0.0                                     # an all-zero tile
    x[7, 300] = 250.0                                       # an outlier tile
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    q, s = O.quant_1x128(x)
    assert q.shape == x.shape and s.shape == (37, 4) and s.dtype == np.float32
    t = np.abs(x).reshape(37, 4, 128)
    amax = t.max(axis=2)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(448)))
    assert s[5, 1] == 1.0 and np.all(q[5, 128:256] == 0)
    # the element equal to the tile max maps to +/-448 exactly
    j = np.argmax(t, axis=2)
    for rr in range(37):
        for c in range(4):
            if nz[rr, c]:
                assert (q[rr, c * 128 + j[rr, c]] & 0x7F) == 0x7E
    # quantise-dequantise error <= half an E4M3 step at |x|/s, times s
    deq = O.dequant_1x128(q, s)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    bound = O.e4m3_half_ulp(x / sc) * sc
    assert np.all(np.abs(deq - x) <= bound * (1 + 1e-6))


def pin_quant_exact_layouts():
    """Tiles/blocks whose values are E4M3 numbers times a per-tile power of two quantise
    exactly, so dequant(quant(x)) == x; distinct scales per tile/block catch any mix-up of
    which scale belongs to which tile (a transposed scale index, a wrong tile width)."""
    r = _rng(4)
    pos = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    rows, cols = 6, 384
    codes = r.integers(0, 127, size=(rows, cols))
    vals = pos[codes] * np.where(r.random((rows, cols)) < 0.5, -1, 1)
    e = r.integers(-6, 4, size=(rows, cols // 128))
    x = vals.reshape(rows, 3, 128).copy()
    x[:, :, 0] = 448.0                                     # pin every tile's amax
    x = x * np.exp2(e)[:, :, None]
    x = x.reshape(rows, cols)
    q, s = O.quant_1x128(x)
    assert np.array_equal(s, np.exp2(e).astype(np.float32))
    assert np.array_equal(O.dequant_1x128(q, s), x)
    # 128x128 blocks of a [256, 384] weight, each with its own power-of-two scale
    n, k = 256, 384
    codes = r.integers(0, 127, size=(n, k))
    w = (pos[codes] * np.where(r.random((n, k)) < 0.5, -1, 1)).reshape(2, 128, 3, 128)
    eb = r.integers(-9, -3, size=(2, 3))
    w[:, 0, :, 0] = 448.0
    w = (w * np.exp2(eb)[:, None, :, None]).reshape(n, k)
    qw, sw = O.quant_128x128(w)
    assert np.array_equal(sw, np.exp2(eb).astype(np.float32))
    assert np.array_equal(O.dequant_128x128(qw, sw), w)
    # exact GEMM of exactly-representable operands: integer arithmetic gives the result
    # (every tile holds a 7, so s = 7/448 = 2^-6 and the codes are exact)
    a_int = r.integers(-7, 8, size=(4, k))
    b_int = r.integers(-7, 8, size=(5, k))
    a_int[:, ::128] = 7
    b_int[:, ::128] = -7
    qa, sa = O.quant_1x128(a_int.astype(np.float32))
    qb, sb = O.quant_1x128(b_int.astype(np.float32))
    got = O.dequant_1x128(qa, sa) @ O.dequant_1x128(qb, sb).T
    assert np.array_equal(got, (a_int @ b_int.T).astype(np.float64))


# ------------------------------------------------------------------ power-of-two (E8M0) scales


def _smallest_pow2_exponent(amax: float) -> int:
    """Brute force over every exponent of the E8M0 range, in exact rational arithmetic."""
    from fractions import Fraction
    if amax == 0:
        return 0
    a = Fraction(float(amax))
    for k in range(-127, 128):
        if a <= 448 * Fraction(2) ** k:
            return k
    raise AssertionError("amax beyond 448 * 2^127")


def pin_e8m0_exponent_bruteforce():
    """The scale exponent is the smallest k with amax <= 448 * 2^k (clamped at -127),
    checked against an exhaustive search at boundaries and on random magnitudes."""
    r = _rng(11)
    vals = [0.0, 1.0, 448.0, 224.0, 3.5, 1.75, 3.4e38, 2.0 ** -149, 2.0 ** -126, 1e-38]
    for k in (-127, -60, -9, -1, 0, 1, 7, 60, 119):
        b = 448.0 * 2.0 ** k
        vals += [b, float(np.nextafter(np.float32(b), np.float32(np.inf))),
                 float(np.nextafter(np.float32(b), np.float32(0)))]
    vals += list((r.random(300) * 2.0 ** r.integers(-140, 120, 300)).astype(np.float32).astype(np.float64))
    vals = np.array(vals, dtype=np.float64)
    got = O.e8m0_exponent(vals)
    want = np.array([_smallest_pow2_exponent(v) for v in vals])
    assert np.array_equal(got, want), vals[got != want][:5]


def pin_e8m0_format_constants():
    """E8M0 (OCP microscaling scale format): unsigned 8-bit exponent, bias 127, 0xFF = NaN."""
    assert O.e8m0_decode(np.uint8(127)) == 1.0 and O.e8m0_decode(np.uint8(128)) == 2.0
    assert O.e8m0_decode(np.uint8(0)) == 2.0 ** -127 and O.e8m0_decode(np.uint8(254)) == 2.0 ** 127
    assert np.isnan(O.e8m0_decode(np.uint8(255)))


def pin_quant_e8m0_exact_layouts():
    """Tiles of E4M3 numbers times a per-tile power of two, whose largest magnitude lies in
    (224, 448] * 2^e, get code e + 127 and quantise exactly; distinct exponents per tile /
    block catch a scale attached to the wrong tile.  A max just above 448 * 2^e moves to
    code e + 128."""
    r = _rng(12)
    pos = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    rows, cols = 6, 384
    vals = pos[r.integers(0, 121, size=(rows, cols))] * np.where(r.random((rows, cols)) < 0.5, -1, 1)
    e = r.integers(-20, 20, size=(rows, cols // 128))
    x = vals.reshape(rows, 3, 128).copy()
    x[:, :, 5] = np.where(r.random((rows, 3)) < 0.5, 448.0, -240.0)   # amax in (224, 448]
    x = (x * np.exp2(e)[:, :, None]).reshape(rows, cols)
    q, c = O.quant_1x128_e8m0(x)
    assert c.dtype == np.uint8 and np.array_equal(c.astype(np.int64), e + 127)
    assert np.array_equal(O.dequant_1x128(q, O.e8m0_decode(c)), x)
    x2 = x.copy()
    x2[0, 5] = 448.0 * 2.0 ** e[0, 0] * (1 + 2.0 ** -20)
    _, c2 = O.quant_1x128_e8m0(x2)
    assert int(c2[0, 0]) == e[0, 0] + 128 and np.array_equal(c2[1:], c[1:])
    n, k = 256, 384
    w = (pos[r.integers(0, 121, size=(n, k))] * np.where(r.random((n, k)) < 0.5, -1, 1)).reshape(2, 128, 3, 128)
    eb = r.integers(-12, -2, size=(2, 3))
    w[:, 3, :, 7] = -288.0
    w = (w * np.exp2(eb)[:, None, :, None]).reshape(n, k)
    qw, cw = O.quant_128x128_e8m0(w)
    assert np.array_equal(cw.astype(np.int64), eb + 127)
    assert np.array_equal(O.dequant_128x128(qw, O.e8m0_decode(cw)), w)


def pin_quant_e8m0_against_fp32_rule():
    """The power-of-two scale is the fp32 scale amax / 448 rounded up to a power of two
    (so 1 <= s_pow2 / s_fp32 < 2), and the round trip stays within half an E4M3 step."""
    r = _rng(13)
    x = r.standard_normal((29, 512)).astype(np.float32)
    x[3, 100] = 900.0
    x[4, 128:256] = 0.0
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    _, s32 = O.quant_1x128(x)
    q, c = O.quant_1x128_e8m0(x)
    s2 = O.e8m0_decode(c)
    ratio = s2 / s32.astype(np.float64)
    nz = np.abs(x).reshape(29, 4, 128).max(axis=2) > 0
    assert np.all((ratio[nz] >= 1) & (ratio[nz] < 2)) and np.all(c[~nz] == 127)
    deq = O.dequant_1x128(q, s2)
    sc = np.repeat(s2, 128, axis=1)
    assert np.all(np.abs(deq - x) <= O.e4m3_half_ulp(x / sc) * sc)


def pin_fp8_e8m0_layer_close_to_exact():
    """The power-of-two-scale fp8 layer approximates the exact layer about as well as the
    fp32-scale one (at most one bit of headroom lost per tile)."""
    r = _rng(14)
    T, d, N, I = 16, 256, 4, 128
    x = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    wr = r.standard_normal((N, d)) * 0.05
    b = np.zeros(N, np.float32)
    w13 = r.standard_normal((N + 1, 2 * I, d)) * 0.05
    w2 = r.standard_normal((N + 1, d, I)) * 0.05
    ex, _, _ = O.forward(x, wr, b, w13, w2, 2, precision="exact")
    f8, _, _ = O.forward(x, wr, b, w13, w2, 2, precision="fp8")
    e8, _, _ = O.forward(x, wr, b, w13, w2, 2, precision="fp8_e8m0")
    rms = np.sqrt(np.mean(ex ** 2))
    err8 = np.sqrt(np.mean((e8 - ex) ** 2)) / rms
    assert err8 < 0.1 and np.max(np.abs(e8 - ex)) / rms < 0.4
    assert err8 < 2.0 * np.sqrt(np.mean((f8 - ex) ** 2)) / rms
    assert not np.array_equal(e8, f8)  # the scale rule really differs


# ------------------------------------------------------------------ routing


def _tiny_router(seed, T=24, d=32, N=8, scale=1.0):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    w = r.standard_normal((N, d)) * 0.3 * scale
    b = r.uniform(-0.05, 0.05, N).astype(np.float32)
    return x, w, b


def pin_route_bruteforce():
    """Top-K by z equals the K-subset of largest total z (all subsets enumerated); gates
    are the subset's sigmoid affinities (torch.sigmoid) over their sum."""
    for seed in range(4):
        x, w, b = _tiny_router(seed)
        K = 3
        r = O.route(x, w, b, K)
        s_ref = torch.sigmoid(torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
        z_ref = s_ref + b.astype(np.float64)
        assert np.allclose(r["s"], s_ref, rtol=0, atol=1e-15)
        for t in range(x.shape[0]):
            best = max(itertools.combinations(range(w.shape[0]), K),
                       key=lambda S: sum(z_ref[t, list(S)]))
            assert set(r["idx"][t]) == set(best)
            assert len(set(r["idx"][t])) == K
            # descending z order
            assert all(z_ref[t, r["idx"][t][i]] >= z_ref[t, r["idx"][t][i + 1]] for i in range(K - 1))
            g = s_ref[t, list(r["idx"][t])]
            assert np.allclose(r["gate"][t], g / g.sum(), rtol=0, atol=1e-15)
            assert abs(r["gate"][t].sum() - 1.0) < 1e-14


def pin_route_bias_only_selects():
    x, w, b = _tiny_router(11)
    K = 2
    r0 = O.route(x, w, b, K)
    # a constant shift of every bias changes nothing
    r1 = O.route(x, w, b + np.float32(0.25), K)
    assert np.array_equal(r0["idx"], r1["idx"]) and np.allclose(r0["gate"], r1["gate"], atol=1e-15)
    # forcing expert j: it is picked for every token and its gate is still s_j / sum s
    j = 5
    bf = b.copy()
    bf[j] = 10.0
    rf = O.route(x, w, bf, K)
    s = torch.sigmoid(torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
    for t in range(x.shape[0]):
        assert rf["idx"][t][0] == j
        sel = list(rf["idx"][t])
        assert np.allclose(rf["gate"][t], s[t, sel] / s[t, sel].sum(), atol=1e-15)
    # two bias vectors that give the same selection give bit-identical gates
    rb = O.route(x, w, b * np.float32(1.0001), K)
    same = np.all(np.sort(rb["idx"], 1) == np.sort(r0["idx"], 1), axis=1)
    assert same.any()
    for t in np.nonzero(same)[0]:
        g0 = dict(zip(r0["idx"][t], r0["gate"][t]))
        g1 = dict(zip(rb["idx"][t], rb["gate"][t]))
        assert all(g0[e] == g1[e] for e in g0)


def pin_route_special_cases():
    x, w, b = _tiny_router(12)
    N = w.shape[0]
    r = O.route(x, w, b, N)                         # K = N: every expert, gates = s / sum s
    s = torch.sigmoid(torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
    for t in range(x.shape[0]):
        g = dict(zip(r["idx"][t], r["gate"][t]))
        assert np.allclose([g[e] for e in range(N)], s[t] / s[t].sum(), atol=1e-15)
    # one group is the ungrouped router
    ra = O.route(x, w, b, 3)
    rg = O.route(x, w, b, 3, n_group=1, topk_group=1)
    assert np.array_equal(ra["idx"], rg["idx"])
    # keeping every group is the ungrouped router too
    rk = O.route(x, w, b, 3, n_group=4, topk_group=4)
    assert np.array_equal(ra["idx"], rk["idx"])
    # exact ties: equal z -> the lower index first
    xt = np.zeros((1, 4))
    wt = np.zeros((6, 4))
    rt = O.route(xt, wt, np.zeros(6, np.float32), 3)
    assert list(rt["idx"][0]) == [0, 1, 2] and np.allclose(rt["gate"][0], 1 / 3)


def pin_route_groups_bruteforce():
    """Group-limited routing: group score = the best pair sum inside the group (all pairs
    enumerated), the topk_group best groups kept, then the best K-subset inside them."""
    for seed in range(3):
        x, w, b = _tiny_router(20 + seed, T=16, N=12)
        n_group, topk_group, K = 4, 2, 3
        r = O.route(x, w, b, K, n_group, topk_group)
        s = torch.sigmoid(torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
        z = s + b.astype(np.float64)
        gs = 12 // n_group
        for t in range(x.shape[0]):
            score = [max(z[t, g * gs + i] + z[t, g * gs + j] for i, j in itertools.combinations(range(gs), 2))
                     for g in range(n_group)]
            kept = max(itertools.combinations(range(n_group), topk_group),
                       key=lambda G: sum(score[g] for g in G))
            allowed = [e for g in kept for e in range(g * gs, (g + 1) * gs)]
            best = max(itertools.combinations(allowed, K), key=lambda S: sum(z[t, list(S)]))
            assert set(r["idx"][t]) == set(best), (seed, t)
            assert all((e // gs) in kept for e in r["idx"][t])


# ------------------------------------------------------------------ permutation, counts


def pin_counts_and_permute():
    r = _rng(5)
    T, K, N = 50, 3, 7
    idx = np.stack([r.permutation(N)[:K] for _ in range(T)])
    counts = O.expert_counts(idx, N)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=N))
    assert counts.sum() == T * K
    off, st, pp = O.permute(idx, N, 1)
    assert off[0] == 0 and np.array_equal(np.diff(off[:N + 1]), np.bincount(idx.ravel(), minlength=N))
    assert off[N + 1] == T * K + T
    order = np.argsort(idx.ravel(), kind="stable")          # expert-major, token order
    assert np.array_equal(st[:T * K], order // K)
    inv = np.empty(T * K, dtype=np.int64)
    inv[order] = np.arange(T * K)
    assert np.array_equal(pp.ravel(), inv)
    assert np.array_equal(st[T * K:], np.arange(T))
    for t in range(T):
        for k in range(K):
            assert st[pp[t, k]] == t


def pin_bias_update_closed_form():
    # N = 4 experts, T = 2 tokens, K = 2: mean load 1.  Loads 2, 1, 1, 0.
    b = np.float32([0.5, -0.25, 0.0, 1.0])
    got = O.bias_update(b, np.array([2, 1, 1, 0]), T=2, top_k=2, gamma=0.125)
    assert np.array_equal(got, np.float32([0.375, -0.25, 0.0, 1.125]))
    # balanced loads leave every bias (bit pattern included) alone
    bz = np.float32([-0.0, 0.1, -3.0, 7.5])
    got = O.bias_update(bz, np.array([1, 1, 1, 1]), T=2, top_k=2, gamma=0.001)
    assert np.array_equal(got.view(np.uint32), bz.view(np.uint32))
    # fl32(0.1f - 0.001f) = 0x3DCAC083 (found by exact rational arithmetic on the two floats)
    got = O.bias_update(np.float32([0.1, 0.1]), np.array([2, 0]), T=2, top_k=1, gamma=0.001)
    assert got.view(np.uint32)[0] == 0x3DCAC083 and got[1] > np.float32(0.1)


# ------------------------------------------------------------------ FFN and the layer


def _tiny_layer(seed, T=20, d=24, N=6, I=10, scale=0.3):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N, d)) * scale
    b = r.uniform(-0.05, 0.05, N).astype(np.float32)
    w13 = r.standard_normal((N + 1, 2 * I, d)) * scale
    w2 = r.standard_normal((N + 1, d, I)) * scale
    return x, wr, b, w13, w2


def pin_single_expert_is_plain_swiglu():
    """N = K = 1: the layer is two SwiGLU MLPs added (torch silu / matmul, float64)."""
    x, wr, b, w13, w2 = _tiny_layer(6, N=1)
    I = w13.shape[1] // 2
    out, r, _ = O.forward(x, wr, b, w13, w2, top_k=1)
    X = torch.from_numpy(x)

    def mlp(e):
        W1, W3 = torch.from_numpy(w13[e, :I]), torch.from_numpy(w13[e, I:])
        return (torch.nn.functional.silu(X @ W1.T) * (X @ W3.T)) @ torch.from_numpy(w2[e]).T

    ref = (mlp(0) + mlp(1)).numpy()
    assert np.allclose(r["gate"], 1.0)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def pin_dense_equals_sparse():
    for seed, (ng, tg) in zip(range(3), [(1, 1), (3, 2), (2, 1)]):
        x, wr, b, w13, w2 = _tiny_layer(30 + seed)
        dense, r = O.forward_dense(x, wr, b, w13, w2, top_k=2, n_group=ng, topk_group=tg)
        sparse, _, _ = O.forward(x, wr, b, w13, w2, top_k=2, n_group=ng, topk_group=tg)
        assert np.allclose(dense, sparse, rtol=0, atol=1e-12)


def pin_combine_closed_form():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    sh = np.array([[0.5, 0.25], [-1.0, 1.0]])
    pp = np.array([[2, 0], [1, 2]])
    g = np.array([[0.75, 0.25], [0.5, 0.5]])
    out = O.combine(y, sh, pp, g)
    assert np.array_equal(out, np.array([[75.75, 150.75], [54.0, 111.0]]))


def pin_fp8_layer_close_to_exact():
    """The fp8 model is an approximation of the exact layer: small relative error."""
    r = _rng(7)
    T, d, N, I = 16, 256, 4, 128
    x = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    wr = r.standard_normal((N, d)) * 0.05
    b = np.zeros(N, np.float32)
    w13 = r.standard_normal((N + 1, 2 * I, d)) * 0.05
    w2 = r.standard_normal((N + 1, d, I)) * 0.05
    ex, _, _ = O.forward(x, wr, b, w13, w2, 2, precision="exact")
    f8, _, _ = O.forward(x, wr, b, w13, w2, 2, precision="fp8")
    bf, _, _ = O.forward(x, wr, b, w13, w2, 2, precision="bf16")
    rms = np.sqrt(np.mean(ex ** 2))
    # E4M3 keeps 3 mantissa bits (relative step 1/16 .. 1/8): a few percent RMS error
    assert np.sqrt(np.mean((f8 - ex) ** 2)) / rms < 0.1
    assert np.max(np.abs(f8 - ex)) / rms < 0.4
    assert np.max(np.abs(bf - ex)) / rms < 0.03
    assert np.max(np.abs(f8 - ex)) > np.max(np.abs(bf - ex))  # fp8 really quantises


# ------------------------------------------------------------------ backward


def _fd_check(seed, n_group=1, topk_group=1, K=2):
    """Central finite differences of the (pinned) dense forward against ``backward`` along
    random directions in x, W_r, W13 and W2.  The selection must not change within the step,
    which is asserted."""
    x, wr, b, w13, w2 = _tiny_layer(seed, T=9, d=12, N=8, I=6, scale=0.4)
    r = _rng(seed + 100)
    d_out = r.standard_normal((9, 12))
    g = O.backward(x, wr, b, w13, w2, K, d_out, n_group, topk_group)
    params = {"x": x, "wr": wr, "w13": w13, "w2": w2}
    grads = {"x": g["dx"], "wr": g["dw_router"], "w13": g["dw13"], "w2": g["dw2"]}

    def loss(p):
        out, rr = O.forward_dense(p["x"], p["wr"], b, p["w13"], p["w2"], K, n_group, topk_group)
        return float(np.sum(d_out * out)), rr["idx"]

    _, idx0 = loss(params)
    eps = 1e-6
    for name in params:
        for _ in range(3):
            v = r.standard_normal(params[name].shape)
            hi = dict(params, **{name: params[name] + eps * v})
            lo = dict(params, **{name: params[name] - eps * v})
            lh, ih = loss(hi)
            ll, il = loss(lo)
            assert np.array_equal(ih, idx0) and np.array_equal(il, idx0), "selection moved"
            fd = (lh - ll) / (2 * eps)
            an = float(np.sum(grads[name] * v))
            assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (name, fd, an)


def pin_backward_finite_differences():
    _fd_check(21)


def pin_backward_finite_differences_groups():
    _fd_check(22, n_group=4, topk_group=2, K=3)


def pin_backward_closed_forms():
    """K = N = 1: the single gate is 1 whatever the affinity, so the router gets no gradient;
    the shared expert's gradients are those of a plain SwiGLU FFN, checked against torch
    autograd of the textbook form (float64)."""
    x, wr, b, w13, w2 = _tiny_layer(23, T=5, d=8, N=1, I=4, scale=0.5)
    d_out = _rng(24).standard_normal((5, 8))
    g = O.backward(x, wr, b, w13, w2, 1, d_out)
    assert np.all(g["du"] == 0) and np.all(g["dw_router"] == 0)
    xt = torch.tensor(x, requires_grad=True)
    w13t = torch.tensor(w13[1], requires_grad=True)
    w2t = torch.tensor(w2[1], requires_grad=True)
    a, c = xt @ w13t[:4].T, xt @ w13t[4:].T
    out = (torch.nn.functional.silu(a) * c) @ w2t.T
    (out * torch.tensor(d_out)).sum().backward()
    assert np.allclose(g["dw13"][1], w13t.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw2"][1], w2t.grad.numpy(), rtol=1e-12, atol=1e-12)


def pin_backward_bf16_model_close_to_exact():
    """The bf16-storage model of the backward is a small perturbation of the exact gradients."""
    x, wr, b, w13, w2 = _tiny_layer(25, T=16, d=32, N=6, I=16, scale=0.3)
    d_out = _rng(26).standard_normal((16, 32))
    ex = O.backward(x, wr, b, w13, w2, 2, d_out)
    bf = O.backward(x, wr, b, w13, w2, 2, d_out, precision="bf16")
    for k in ("dx", "dw_router", "dw13", "dw2"):
        e = np.max(np.abs(bf[k] - ex[k])) / np.sqrt(np.mean(ex[k] ** 2))
        assert 0 < e < 0.05, (k, e)


def pin_backward_fp8_model_close_to_exact():
    """The fp8 model of the backward approximates the exact gradients (E4M3 keeps 3 mantissa
    bits: a few percent of RMS; a dropped term, a wrong operand or a misplaced scale would not)
    and is not the bf16 model.  Which axis each operand is quantised along is a reading of the
    pages that this closeness cannot tell apart; the GPU parity tests hold the device to it."""
    r = _rng(27)
    T, d, N, I = 40, 256, 4, 128
    x = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    wr = r.standard_normal((N, d)) * 0.05
    b = np.zeros(N, np.float32)
    w13 = r.standard_normal((N + 1, 2 * I, d)) * 0.05
    w2 = r.standard_normal((N + 1, d, I)) * 0.05
    d_out = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    ex = O.backward(x, wr, b, w13, w2, 2, d_out)
    f8 = O.backward(x, wr, b, w13, w2, 2, d_out, precision="fp8")
    bf = O.backward(x, wr, b, w13, w2, 2, d_out, precision="bf16")
    for k in ("dx", "dw_router", "dw13", "dw2"):
        rms = np.sqrt(np.mean(ex[k] ** 2))
        e8 = np.sqrt(np.mean((f8[k] - ex[k]) ** 2)) / rms
        assert 0.001 < e8 < 0.12, (k, e8)
        assert not np.array_equal(f8[k], bf[k])


def pin_route_margins_bruteforce():
    """The tie margins that decide which tokens the parity tests exclude: ``margin`` is the
    gap between the K-th and the (K+1)-th largest z among the allowed experts, and
    ``group_margin`` the gap between the last kept and the best dropped group score.  Checked
    against a full sort of z (torch.sigmoid affinities) and an enumeration of every pair
    inside each group, with the group limit on and off, and K = N (no (K+1)-th: +inf)."""
    for seed in range(3):
        x, w, b = _tiny_router(40 + seed, T=12, N=12)
        s = torch.sigmoid(torch.from_numpy(x) @ torch.from_numpy(w).T).numpy()
        z = s + b.astype(np.float64)
        for K in (1, 3):
            r = O.route(x, w, b, K)
            for t in range(x.shape[0]):
                zs = np.sort(z[t])[::-1]
                assert abs(r["margin"][t] - (zs[K - 1] - zs[K])) <= 1e-15
                assert r["group_margin"][t] == np.inf
        n_group, topk_group, K = 4, 2, 3
        gs = 12 // n_group
        r = O.route(x, w, b, K, n_group, topk_group)
        for t in range(x.shape[0]):
            score = sorted((max(z[t, g * gs + i] + z[t, g * gs + j] for i, j in itertools.combinations(range(gs), 2))
                            for g in range(n_group)), reverse=True)
            assert abs(r["group_margin"][t] - (score[topk_group - 1] - score[topk_group])) <= 1e-15
            kept = set(int(e) // gs for e in r["idx"][t])
            allowed = np.sort(np.concatenate([z[t, g * gs:(g + 1) * gs] for g in range(n_group)
                                              if g in kept or len(kept) < topk_group]))[::-1]
            if len(kept) == topk_group:
                assert abs(r["margin"][t] - (allowed[K - 1] - allowed[K])) <= 1e-15
    x, w, b = _tiny_router(43, N=6)
    assert np.all(O.route(x, w, b, 6)["margin"] == np.inf)


def pin_e4m3_half_ulp_neighbours():
    """Half the E4M3 spacing, at every positive code and at the midpoint of every pair of
    neighbouring codes, equals half the distance between the two neighbours (the format's
    spacing read off its value table); at 448 it is half the gap down to 416."""
    pos = O.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    gap = np.diff(pos)                                   # 126 gaps between codes 0..126
    assert np.array_equal(O.e4m3_half_ulp(pos[:126]), gap / 2)
    assert np.array_equal(O.e4m3_half_ulp(-pos[:126]), gap / 2)
    assert np.array_equal(O.e4m3_half_ulp((pos[:126] + pos[1:]) / 2), gap / 2)
    assert O.e4m3_half_ulp(448.0) == (448.0 - 416.0) / 2
    assert O.e4m3_half_ulp(2.0 ** -6) == 2.0 ** -10 and O.e4m3_half_ulp(2.0 ** -7) == 2.0 ** -10


def pin_forward_bf16_storage_handbuilt():
    """The bf16 storage model of the forward on a hand-built expert whose values are exact
    in float64, so every rounding it applies is visible in the result.

    x = [1, 0]; W1 rows give a = [40, 48], for which silu(a) = a exactly in float64
    (exp(-40) < 2^-54); W3 rows give c = [1 + 2^-6 + 2^-9, -(1/2 + 2^-9)], so
    h = [40.703125, -24.09375] (binary 101000.101101 and -11000.00011), whose bf16 values are
    40.75 and -24.125.  W2 = [[1, 1], [1/2, 1/4]] gives y = [16.625, 14.34375] from the stored
    h (16.609375 and 14.328125 from the exact h).  The routed expert's y is stored in bf16
    (14.34375 = 1110.01011: a tie, to the even 14.375), the shared expert's in float32, and
    with one routed expert at gate 1 the output is their sum: [33.25, 28.71875]."""
    x = np.array([[1.0, 0.0]])
    w13 = np.array([[40.0, 0.0], [48.0, 0.0], [1.017578125, 0.0], [-0.501953125, 0.0]])
    w2 = np.array([[1.0, 1.0], [0.5, 0.25]])
    out, ex = O.forward_sparse(x, np.array([[0]]), np.array([[1.0]]), 1, lambda e: (w13, w2), "bf16")
    assert np.array_equal(ex["y_routed"][0], [16.625, 14.375])
    assert np.array_equal(ex["y_shared"][0], [16.625, 14.34375])
    assert np.array_equal(out[0], [33.25, 28.71875])
    y, h = O.expert_rows(x, w13, w2, "bf16", return_h=True)
    assert np.array_equal(h[0], [40.75, -24.125]) and np.array_equal(y[0], [16.625, 14.34375])
    ex_out, _ = O.forward_sparse(x, np.array([[0]]), np.array([[1.0]]), 1, lambda e: (w13, w2), "exact")
    assert np.array_equal(ex_out[0], [33.21875, 28.65625])


def pin_forward_fp8_storage_handbuilt():
    """The FP8 model of the forward on a hand-built expert (d = I = 128) whose tile scales are
    exact, so only the E4M3 roundings the pages' scheme applies move the result.

    x = [1.03125, 7, 0, ...]: tile amax 7 -> s = 7/448 = 2^-6; 1.03125 / s = 66 rounds to the
    E4M3 value 64, so the expert sees x = [1, 7, 0, ...].  W1 column 0 = a = [64, 40, 48, 40]
    (block amax 112 -> s = 1/4, exact), W3 column 0 = c = [7, 0.4375, 0.4375, 1.75] (block amax
    7 -> s = 2^-6, exact); silu(a) = a, so h = a c = [448, 17.5, 21, 70, 0, ...].  Its 1x128
    tile has amax 448 -> s = 1, and E4M3 stores [448, 18, 20, 72]: 17.5 -> 18 (spacing 2),
    21 -> 20 (a tie, to the even mantissa), 70 -> 72 (spacing 8).  W2 picks y = [h1, h2, h3,
    h0 + h1/4] = [18, 20, 72, 452.5]; the routed copy is stored in bf16 (452.5 -> 452), the
    shared one in float32, so out = [36, 40, 144, 904.5]."""
    d = inter = 128
    x = np.zeros((1, d))
    x[0, 0], x[0, 1] = 1.03125, 7.0
    w13 = np.zeros((2 * inter, d))
    w2 = np.zeros((d, inter))
    w13[0, 2], w13[inter, 2] = 112.0, 7.0
    w13[:4, 0] = [64, 40, 48, 40]
    w13[inter:inter + 4, 0] = [7, 0.4375, 0.4375, 1.75]
    w2[127, 127] = 7.0
    w2[0, 1] = w2[1, 2] = w2[2, 3] = w2[3, 0] = 1.0
    w2[3, 1] = 0.25
    out, ex = O.forward_sparse(x, np.array([[0]]), np.array([[1.0]]), 1, lambda e: (w13, w2), "fp8")
    assert np.array_equal(ex["y_routed"][0, :4], [18, 20, 72, 452])
    assert np.array_equal(ex["y_shared"][0, :4], [18, 20, 72, 452.5])
    assert np.array_equal(out[0, :4], [36, 40, 144, 904.5]) and not np.any(out[0, 4:])


def pin_backward_bf16_storage_handbuilt():
    """The bf16 storage model of the backward on a hand-built layer (T = 1, d = I = 2, N = K = 2
    plus the shared expert, all three experts with the same weights).

    Router: x = [1, 0], router rows [0, 0] and [40, 0] -> s = [1/2, 1] (sigmoid(40) = 1 in
    float64), so the gates are 2/3 (expert 1) and 1/3 (expert 0).  Experts: a = [40, 48]
    (silu(a) = a, sigmoid(a) = 1), c = [3/4, 1 + 2^-6 + 2^-9] -> h = [30, 48.84375], stored
    in bf16 as [30, 48.75].  d_out = [1, 1/2].
    Expert 0: dy = bf16(fl32(d_out / 3)) = [0.333984375, 0.1669921875] (1/3 = 0.0101010...b
    rounds up at its 8th bit), so dW2 = dy^T h = [[10.01953125, 16.28173828125],
    [5.009765625, 8.140869140625]].  W2 = [[1, 1/2], [1/4, 1]] gives dh = dy W2 =
    [0.375732421875, 0.333984375]; da = bf16(dh c) = [0.28125, 0.33984375] (from
    0.2817993... and 0.3398551...), dc = bf16(dh a) = [15, 16] (from 15.029296875 and
    16.03125); dW13 column 0 is [da | dc] (x = [1, 0]).
    dx: the routed rows' contributions dac W13 are stored in bf16 (expert 0: 55.09375 -> 55,
    expert 1: 110.1875 -> 110), the shared expert's (165.09375) in float64, and the router
    term is zero (both experts return the same y, so the gates' gradient cancels):
    dx = [330.09375, 0]."""
    x = np.array([[1.0, 0.0]])
    wr = np.array([[0.0, 0.0], [40.0, 0.0]])
    w13 = np.zeros((3, 4, 2))
    w13[:, :, 0] = [40, 48, 0.75, 1.017578125]
    w2 = np.zeros((3, 2, 2))
    w2[:] = [[1, 0.5], [0.25, 1]]
    g = O.backward(x, wr, np.zeros(2, np.float32), w13, w2, 2, np.array([[1.0, 0.5]]), precision="bf16")
    assert np.array_equal(g["route"]["idx"], [[1, 0]])
    assert np.array_equal(g["dw2"][0], [[10.01953125, 16.28173828125], [5.009765625, 8.140869140625]])
    assert np.array_equal(g["dw13"][0][:, 0], [0.28125, 0.33984375, 15.0, 16.0])
    assert np.array_equal(g["dw13"][2][:, 0], [0.84375, 1.015625, 45.0, 48.0])
    assert np.array_equal(g["dx"], [[330.09375, 0.0]]) and np.all(g["du"] == 0)


def pin_backward_fp8_storage_handbuilt():
    """The FP8 model of the backward on a hand-built layer: T = 3, d = I = 128, one routed
    expert (K = 1, gate 1) plus the shared one, both with the same weights.  Every scale of
    the Dgrad path is exact, so the E4M3 roundings there show as exact binary fractions; the
    Wgrad tiles use fl32(v / 448) scales, given below as the exact float32 values.

    Inputs: x rows [1, 7], [1.5, 7], [1.03125, 7] (then zeros); their 1x128 tiles have
    s = 2^-6 and the third rounds 66 -> 64, i.e. to [1, 7].  W1 column 0 = [64, 40], W3
    column 0 = [7, 15/32] (block scales 1/4 and 2^-6, exact).  h = silu(a) c with a = 64 x0,
    40 x0 and c = 7 x0, 15/32 x0: token rows [448, 18.75] -> E4M3 [448, 18] (s = 1) and
    [1008, 42.1875] -> [1008, 40.5] (s = 2.25, 42.1875 / 2.25 = 18.75 -> 18).
    d_out rows [7, 0.8125], [7, 0.53125], [7, 0.5]; dy = d_out (gate 1, bf16 values).
    Dgrad: dy is quantised 1x128 (s = 2^-6: 0.53125 -> 0.5, a tie to the even code 32); W2 = 1/4 at (0, 0), 1 at
    (1, 1) -> dh = [7/4, dy1]; da = bf16(dh c), dc = bf16(dh a): token 0 da = [12.25,
    0.380859375], dc = [112, 32.5].  [da | dc] is quantised per 1x128 tile: da's s = 7/256
    (0.380859375 -> 14 * 7/256 = 0.3828125), dc's s = 1/4 (32.5 -> 32); dac W13 gives
    1598.3125 for token 0, stored in bf16 (1600) for the routed rows, so dx[0, 0] = 3198.3125;
    dx[:, 2] = bf16(112 da0) + 112 da0.
    Wgrad (the tokens are the reduction axis; every Wgrad operand here spans one tile):
    dy^T row 0 = [7, 7, 7] is exact; row 1 = [0.8125, 0.53125, 0.5] has s_dy = fl32(0.8125 /
    448) and codes [448, 288, 288] (0.53125 / s_dy = 292.9, 0.5 / s_dy = 275.7).  h^T (bf16 of
    the stored h) is one 128x128 block: rows [448, 1008, 448] and [18, 40.5, 18], amax 1008 ->
    s = 2.25, 448 -> 432 (199.1 -> 192 of that scale).  x^T is one block with s = 2^-6, its
    row 0 [1, 1.5, 1.03125] -> [1, 1.5, 1].  [da | dc]^T rows are 1x128 tiles along the
    tokens: da0 = [12.25, 18.375, 12.25] (s = 21/512: 12.25 -> 11.8125), da1 = [0.380859375,
    0.3515625, 0.234375] and dc1 = [32.5, 30, 20] (codes [448, 416, 288] of s_da = fl32(
    0.380859375 / 448) and s_dc = fl32(32.5 / 448)), dc0 = [112, 168, 112] (s = 3/8: 112 -> 108).
    So dW2[1, 0] = s_dy (448 * 432 + 288 * 1008 + 288 * 432) and dW13[I + 1, 0] =
    s_dc (448 * 1 + 416 * 1.5 + 288 * 1)."""
    d = inter = 128
    x = np.zeros((3, d))
    x[:, 0] = [1.0, 1.5, 1.03125]
    x[:, 1] = 7.0
    w13 = np.zeros((2, 2 * inter, d))
    w2 = np.zeros((2, d, inter))
    w13[:, 0, 0], w13[:, 1, 0], w13[:, 0, 2] = 64, 40, 112
    w13[:, inter, 0], w13[:, inter + 1, 0] = 7, 0.46875
    w2[:, 0, 0], w2[:, 1, 1], w2[:, 127, 127] = 0.25, 1, 7
    d_out = np.zeros((3, d))
    d_out[:, 0] = 7
    d_out[:, 1] = [0.8125, 0.53125, 0.5]
    g = O.backward(x, np.zeros((1, d)), np.zeros(1, np.float32), w13, w2, 1, d_out, precision="fp8")
    s_dy = float.fromhex("0x1.db6db6p-10")     # fl32(0.8125 / 448)
    s_da = float.fromhex("0x1.bdb6dcp-11")     # fl32(0.380859375 / 448)
    s_dc = float.fromhex("0x1.292492p-4")      # fl32(32.5 / 448)
    assert np.float32(0.8125 / 448) == s_dy and np.float32(0.380859375 / 448) == s_da \
        and np.float32(32.5 / 448) == s_dc
    assert np.array_equal(g["dx"][:, [0, 2]], [[3198.3125, 2748.0], [4764.828125, 4122.0], [3171.21875, 2748.0]])
    assert not np.any(g["dx"][:, 1]) and not np.any(g["dx"][:, 3:])
    assert np.array_equal(g["dw2"][0][:2, :2], [[7 * (432 + 1008 + 432), 7 * (18 + 40.5 + 18)],
                                                [s_dy * (448 * 432 + 288 * 1008 + 288 * 432),
                                                 s_dy * (448 * 18 + 288 * 40.5 + 288 * 18)]])
    assert np.array_equal(g["dw13"][0][[0, 1, inter, inter + 1]][:, :2],
                          [[11.8125 + 18.375 * 1.5 + 11.8125, 7 * (11.8125 + 18.375 + 11.8125)],
                           [s_da * (448 + 416 * 1.5 + 288), 7 * s_da * (448 + 416 + 288)],
                           [108 + 168 * 1.5 + 108, 7 * (108 + 168 + 108)],
                           [s_dc * (448 + 416 * 1.5 + 288), 7 * s_dc * (448 + 416 + 288)]])
    # the shared expert has the same weights and sees dy = d_out (bf16 values already)
    assert np.array_equal(g["dw2"][1], g["dw2"][0]) and np.array_equal(g["dw13"][1], g["dw13"][0])

    # The router's gradient reads the stored h through the gates' gradient: T = 1, two routed
    # experts (K = 2) with gates 1/3 and 2/3 (router rows [0] and [40] on x0 = 1: s = 1/2 and 1).
    # Both hold h = [448, 17.5] -> E4M3 [448, 18] (s = 1); expert 0's W2 returns y0 = h1, expert
    # 1's y0 = h0 / 4 = 112; d_out = [1, 0, ...].  dgate = [18, 112], their gate-weighted sum is
    # 242/3, and du0 = (18 - 242/3) / (3/2) * s0 (1 - s0) = -94/9 (with h1 = 17.5 it would be
    # -10.5); du1 = 0 (s1 = 1).  dW_r[0] = du0 x.
    x = np.zeros((1, d))
    x[0, 0], x[0, 1] = 1.0, 7.0
    wr = np.zeros((2, d))
    wr[1, 0] = 40.0
    w13 = np.zeros((3, 2 * inter, d))
    w13[:, 0, 0], w13[:, 1, 0], w13[:, 0, 2] = 64, 40, 112
    w13[:, inter, 0], w13[:, inter + 1, 0] = 7, 0.4375
    w2 = np.zeros((3, d, inter))
    w2[:, 127, 127] = 7
    w2[0, 0, 1] = 1.0
    w2[1, 0, 0] = 0.25
    d_out = np.zeros((1, d))
    d_out[0, 0] = 1.0
    g = O.backward(x, wr, np.zeros(2, np.float32), w13, w2, 2, d_out, precision="fp8")
    assert np.array_equal(g["route"]["idx"], [[1, 0]]) and np.array_equal(g["dgate"], [[112.0, 18.0]])
    assert abs(g["du"][0, 1] + 94 / 9) < 1e-12 and g["du"][0, 0] == 0
    assert np.allclose(g["dw_router"][0, :2], [-94 / 9, -7 * 94 / 9], rtol=0, atol=1e-11)


def pin_block_quantisation_idempotent():
    """Quantising block-quantised weights again gives them back: the block max is +-448 s
    exactly, so the scale is s again and every value is its own code (fp32 and power-of-two
    scales); the fp8 layer on such weights with re-quantisation skipped is the same layer."""
    r = _rng(15)
    w = torch.from_numpy((r.standard_normal((256, 384)) * 0.02).astype(np.float32)).to(torch.bfloat16).double().numpy()
    for qfn in (O.quant_128x128, O.quant_128x128_e8m0):
        q, s = qfn(w)
        sv = O.e8m0_decode(s) if qfn is O.quant_128x128_e8m0 else s
        w1 = O.dequant_128x128(q, sv)
        q2, s2 = qfn(w1)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)
    x, wr, b, w13, w2 = _tiny_layer(16, T=12, d=128, N=3, I=128, scale=0.05)
    rr = O.route(x, wr, b, 2)
    full, _ = O.forward_sparse(x, rr["idx"], rr["gate"], 3, lambda e: (w13[e], w2[e]), "fp8")
    deq = lambda m: O.dequant_128x128(*O.quant_128x128(m))
    pre, _ = O.forward_sparse(x, rr["idx"], rr["gate"], 3, lambda e: (deq(w13[e]), deq(w2[e])), "fp8",
                              weights_quantised=True)
    assert np.array_equal(full, pre)


def pin_fp32_round_closed_forms():
    """IEEE binary32 round-to-nearest-even at points worked out from the format: [1, 2) has
    spacing 2^-23, so 1 + 2^-24 is a tie that goes to the even neighbour 1, 1 + 3 * 2^-25 lies
    above the midpoint and goes to 1 + 2^-23, and (1 + 2^-23) + 2^-24 is a tie whose even
    neighbour is 1 + 2^-22; [2^24, 2^25) has spacing 2, so 2^24 + 1 ties to 2^24 and 2^24 + 3 to
    2^24 + 4.  The same with the sign flipped."""
    cases = [(1 + 2.0 ** -24, 1.0), (1 + 2.0 ** -25, 1.0), (1 + 3 * 2.0 ** -25, 1 + 2.0 ** -23),
             (1 + 2.0 ** -23 + 2.0 ** -24, 1 + 2.0 ** -22), (2.0 ** 24 + 1, 2.0 ** 24), (2.0 ** 24 + 3, 2.0 ** 24 + 4),
             (0.1, 13421773 * 2.0 ** -27)]
    for v, want in cases:
        assert O.fp32_round(v) == want and O.fp32_round(-v) == -want, (v, want)


def pin_quant_negative_extreme():
    """A tile or block whose largest magnitude is a negative value: the scale comes from |x|.
    Tile [-3.5, 1.75, 0.4375, 0, ...]: amax 3.5 -> s = 3.5 / 448 = 2^-7 (power-of-two rule: the
    same 2^-7), the values scale to -448, 224, 56, all E4M3 numbers, so the negative extreme
    is stored as code 0xFE and every value comes back exactly.  The same values in one
    128x128 weight block."""
    x = np.zeros((1, 128))
    x[0, :3] = [-3.5, 1.75, 0.4375]
    q, s = O.quant_1x128(x)
    assert s[0, 0] == np.float32(2.0 ** -7) and q[0, 0] == 0xFE
    assert np.array_equal(O.dequant_1x128(q, s), x)
    q8, c8 = O.quant_1x128_e8m0(x)
    assert c8[0, 0] == 127 - 7 and q8[0, 0] == 0xFE
    w = np.zeros((128, 128))
    w[5, 9], w[0, 0], w[127, 127] = -3.5, 1.75, 0.4375
    qw, sw = O.quant_128x128(w)
    assert sw[0, 0] == np.float32(2.0 ** -7) and qw[5, 9] == 0xFE
    assert np.array_equal(O.dequant_128x128(qw, sw), w)
    qw8, cw8 = O.quant_128x128_e8m0(w)
    assert cw8[0, 0] == 127 - 7 and qw8[5, 9] == 0xFE


def pin_forward_h_quantised_from_fp32():
    """The fp8 paths quantise h as the float32 value the kernels form.  Hand-built expert
    (d = I = 128, weights given as already quantised): x = e_0, W1 column 0 = [64, 64, 0, ...],
    W3 column 0 = [7, (1.0625 + 2^-30) / 64, 0, ...]; silu(64) = 64 in float64, so h = [448,
    1.0625 + 2^-30, 0, ...], whose tile (amax 448) has scale 1 under both scale rules.  In
    float32 h_1 is 1.0625, the midpoint between the E4M3 neighbours 1 and 1.125, and rounds to
    the even one, 1; the float64 value lies above the midpoint and would give 1.125."""
    d = inter = 128
    rows = np.zeros((1, d))
    rows[0, 0] = 1.0
    w13 = np.zeros((2 * inter, d))
    w2 = np.zeros((d, inter))
    w13[0, 0] = w13[1, 0] = 64.0
    w13[inter, 0] = 7.0
    w13[inter + 1, 0] = (1.0625 + 2.0 ** -30) / 64
    for prec in ("fp8", "fp8_e8m0"):
        _, h = O.expert_rows(rows, w13, w2, prec, return_h=True, weights_quantised=True)
        assert h[0, 0] == 448.0 and h[0, 1] == 1.0 and not np.any(h[0, 2:]), prec


def pin_layer_flops():
    # DeepSeek-V3 shape: 9 of 257 experts per token; 2*7168*256 + 6*7168*2048*9 per token
    assert O.layer_flops(1, 7168, 256, 8, 2048) == 796_393_472


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
