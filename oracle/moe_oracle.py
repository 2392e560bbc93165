"""Plain CPU oracle of the DeepSeekMoE layer forward (sigmoid routing, aux-loss-free bias).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module: only the
test-suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library; it is a slow, obviously
correct NumPy restatement of what the layer computes, in float64 unless a step is
defined in a lower precision (the fp8 codec, the fp32 bias add).

Sources (the pages this follows; cited by page title and section):

* [TR]  "DeepSeek-V3 Technical Report" (wiki summary, notes.yuuk.io), sections
  "DeepSeekMoE と補助損失なしの負荷分散" (shared + routed experts, N_s = 1, N_r = 256,
  K_r = 8, sigmoid gating, gates from the normalised selected affinities, per-expert bias
  b_i used for routing only, the +/- gamma load rule, no token dropping, node limit M = 4)
  and "FP8 混合精度訓練" (1x128 activation tiles, 128x128 weight blocks, online amax
  scaling, E4M3 everywhere, promotion to FP32 every N_C = 128 elements, gating kept in
  high precision).
* [PFN] "Vol.25 DeepSeek-V3の技術とその影響" (preferred.jp), section
  "MoEの歴史とDeepSeekMoE-V3の特徴": one always-on shared expert plus 8 of 256 routed
  experts per token, whose results are combined; "学習と推論の課題と解決策" (values of a
  1x128 / 128x128 tile can share an exponent) and "ハードウェアデザインへの提案" (requests
  for quantisation support in hardware), with [TR] "考察" (native tile / block quantisation
  in the matrix unit) -- the power-of-two scale variant below.

Readings taken where the pages are silent:

* affinity s = sigmoid(x . e_i) with e_i the i-th router row and no router bias vector;
* selection on z = s + b, larger z first, equal z -> lower expert index;
* gates g = s_S / sum(s_S) with no extra scaling (they sum to one);
* expert FFN = SwiGLU: W2 (silu(W1 x) * (W3 x)); W13 rows [0, I) are W1, [I, 2I) are W3;
* output = shared expert + sum_k g_k FFN_k(x), no residual;
* group-limited routing (stand-in for the node limit): groups of N/n_group contiguous
  experts, group score = sum of the two largest z, keep the topk_group best groups (equal
  scores -> lower group index), then top-K inside them;
* bias step b <- b + fl32(-gamma * sign(load - T K / N)), sign(0) = 0, compared in
  integers as load * N vs T * K;
* E4M3 = OCP E4M3FN (bias 7, max 448, no infinities); q = RNE(fl32(v / s)) with
  s = fl32(amax / 448), saturating at +/-448, amax = 0 -> s = 1; the sign bit of q is the
  sign bit of v (so a negative value that rounds to zero gives code 0x80);
* power-of-two variant: the tile scale is the smallest 2^k with amax / 2^k <= 448
  (k in [-127, 127], k = 0 for an all-zero tile), stored as the E8M0 code k + 127, and
  q = RNE(v / 2^k) (an exact division).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0

# --------------------------------------------------------------------------------------
# Rounding helpers (definitions of the storage formats; not shared with the GPU side)
# --------------------------------------------------------------------------------------


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits), ties to even.

    Written from the definition of the format: |v| = m * 2^e with m in [0.5, 1); keep
    round_half_even(m * 2^8) * 2^(e - 8).  Works for float32 or float64 input and returns
    float64 holding bf16-representable values.  (Overflow past the bf16 range is not
    handled; the layer never produces such values.)
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def fp32_round(a) -> np.ndarray:
    """Round to the nearest float32 value (IEEE RNE), returned as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# E4M3 (OCP E4M3FN) codec.  [TR] "FP8 混合精度訓練" -> "E4M3 統一".
# --------------------------------------------------------------------------------------


def _e4m3_positive_table() -> np.ndarray:
    """Values of the 127 non-negative finite codes 0x00..0x7E, in code order.

    Code = (E << 3) | M.  E = 0: subnormal, value M * 2^-9.  E >= 1: (1 + M/8) * 2^(E-7).
    Code 0x7F (E = 15, M = 7) is NaN; there is no infinity.
    """
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        E, M = code >> 3, code & 7
        vals[code] = M * 2.0 ** -9 if E == 0 else (1.0 + M / 8.0) * 2.0 ** (E - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()
# all 256 codes: bit 7 is the sign, 0x7F / 0xFF are NaN
_E4M3_ALL = np.concatenate([_E4M3_POS, [np.nan], -_E4M3_POS, [np.nan]])


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes (a lookup in the table of all 256 codes)."""
    return _E4M3_ALL[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Encode real values (taken exactly as given) to E4M3 codes.

    Round to nearest, ties to the even code (the one whose mantissa LSB is 0); magnitudes
    at or above 448 saturate to 448; NaN -> 0x7F (with the input's sign bit).
    From the format's definition: |v| lies in the binade [2^e, 2^(e+1)), whose 8 values are
    spaced 2^(e-3); below 2^-6 the subnormals keep the spacing 2^-9 of the lowest binade
    (e = -6).  n = RNE(|v| / 2^(e-3)) (an exact division) is then 8..16 in a binade (16 being
    the first value of the next one) or 0..8 below it, and the code (E << 3) | M, with
    value (1 + M/8) 2^(E-7) for E >= 1 and M 2^-9 for E = 0, is (e + 6) * 8 + n.
    """
    v = np.asarray(v)
    if v.dtype != np.float32:
        v = v.astype(np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    _, e = np.frexp(a)                       # a = f 2^e, f in [0.5, 1): binade exponent e - 1
    e = np.where(a < 2.0 ** -6, -6, e - 1)
    n = np.rint(np.ldexp(a, 3 - e))          # round half to even
    code = (e + 6) * 8 + n
    code = np.where((a >= E4M3_MAX) | (code > 126), 126, code)
    code = np.where(nan, 0x7F, code).astype(np.uint8)
    return np.where(sign, code | 0x80, code).astype(np.uint8)


def e4m3_half_ulp(v) -> np.ndarray:
    """Half the E4M3 spacing at magnitude |v| (|v| <= 448).

    The spacing is 2^(floor(log2|v|) - 3) for |v| >= 2^-6 and 2^-9 below.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)


def _tile_scale(amax32: np.ndarray) -> np.ndarray:
    """s = fl32(amax / 448) in IEEE float32; an all-zero tile gets s = 1."""
    s = (amax32.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)


def quant_1x128(x):
    """Online 1x128 tile quantisation of activations.  [TR] "FP8 混合精度訓練" ->
    "細粒度量子化" (activation tiles 1x128) and "オンライン量子化" (scale from the
    tile's current max |x|).

    x: [rows, cols] values representable in float32 (cols % 128 == 0).
    Returns (q uint8 [rows, cols], s float32 [rows, cols // 128]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    rows, cols = x32.shape
    assert cols % 128 == 0
    t = x32.reshape(rows, cols // 128, 128)
    amax = np.max(np.abs(t), axis=2)
    s = _tile_scale(amax)
    v = (t / s[:, :, None]).astype(np.float32)  # IEEE float32 division
    q = e4m3_encode(v).reshape(rows, cols)
    return q, s


def quant_128x128(w):
    """128x128 block quantisation of a weight matrix [n, k] (n, k % 128 == 0).
    [TR] "FP8 混合精度訓練" -> "細粒度量子化" (weights per 128x128 block).
    Returns (q uint8 [n, k], s float32 [n // 128, k // 128])."""
    w32 = np.asarray(w, dtype=np.float32)
    n, k = w32.shape
    assert n % 128 == 0 and k % 128 == 0
    b = w32.reshape(n // 128, 128, k // 128, 128)
    amax = np.max(np.abs(b), axis=(1, 3))
    s = _tile_scale(amax)
    v = (b / s[:, None, :, None]).astype(np.float32)
    q = e4m3_encode(v).reshape(n, k)
    return q, s


def dequant_1x128(q, s) -> np.ndarray:
    rows, cols = q.shape
    return (e4m3_decode(q).reshape(rows, cols // 128, 128) * s.astype(np.float64)[:, :, None]).reshape(rows, cols)


def dequant_128x128(q, s) -> np.ndarray:
    n, k = q.shape
    v = e4m3_decode(q).reshape(n // 128, 128, k // 128, 128)
    return (v * s.astype(np.float64)[:, None, :, None]).reshape(n, k)


# --------------------------------------------------------------------------------------
# Power-of-two tile scales (a shared exponent per tile, stored as an E8M0 code).
# [PFN] "学習と推論の課題と解決策": inside a 1x128 or 128x128 tile the values can share one
# exponent; [TR] "考察" and [PFN] "ハードウェアデザインへの提案": the authors ask for tile /
# block quantisation supported natively by the matrix unit.  Reading: the tile's scale is
# the smallest power of two 2^k with amax / 2^k <= 448 (the fp32 rule s = amax / 448 rounded
# up to a power of two), k clamped to [-127, 127]; an all-zero tile gets k = 0.  The code is
# k + 127 (E8M0: value 2^(code - 127)).  Dividing by 2^k is exact, so q = RNE_E4M3(x / 2^k).
# --------------------------------------------------------------------------------------

E8M0_BIAS = 127


def e8m0_exponent(amax) -> np.ndarray:
    """k = the smallest integer with amax <= 448 * 2^k, clamped to [-127, 127]; 0 for amax = 0.

    A first guess from log2 is corrected by the two exact comparisons of the definition
    (448 * 2^k is exact in float64), so the result does not depend on log2's rounding."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    with np.errstate(divide="ignore"):
        k = np.where(pos, np.ceil(np.log2(np.where(pos, a, 1.0) / E4M3_MAX)), 0.0)
    for _ in range(2):
        k = np.where(pos & (a > E4M3_MAX * np.exp2(k)), k + 1, k)          # 2^k too small
        k = np.where(pos & (a <= E4M3_MAX * np.exp2(k - 1)), k - 1, k)     # 2^(k-1) suffices
    return np.clip(k, -127, 127).astype(np.int64)


def e8m0_decode(codes) -> np.ndarray:
    """Value of E8M0 codes 0..254: 2^(code - 127) (code 255 is NaN and never produced)."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2((c - E8M0_BIAS).astype(np.float64)))


def quant_1x128_e8m0(x):
    """1x128 tile quantisation with a power-of-two scale per tile (see above).
    Returns (q uint8 [rows, cols], codes uint8 [rows, cols // 128])."""
    x64 = np.asarray(x, dtype=np.float64)
    rows, cols = x64.shape
    assert cols % 128 == 0
    t = x64.reshape(rows, cols // 128, 128)
    k = e8m0_exponent(np.max(np.abs(t), axis=2))
    q = e4m3_encode(t / np.exp2(k)[:, :, None]).reshape(rows, cols)
    return q, (k + E8M0_BIAS).astype(np.uint8)


def quant_128x128_e8m0(w):
    """128x128 block quantisation with a power-of-two scale per block.
    Returns (q uint8 [n, k], codes uint8 [n // 128, k // 128])."""
    w64 = np.asarray(w, dtype=np.float64)
    n, kk = w64.shape
    assert n % 128 == 0 and kk % 128 == 0
    b = w64.reshape(n // 128, 128, kk // 128, 128)
    k = e8m0_exponent(np.max(np.abs(b), axis=(1, 3)))
    q = e4m3_encode(b / np.exp2(k)[:, None, :, None]).reshape(n, kk)
    return q, (k + E8M0_BIAS).astype(np.uint8)


# --------------------------------------------------------------------------------------
# Routing.  [TR] "DeepSeekMoE と補助損失なしの負荷分散".
# --------------------------------------------------------------------------------------


def sigmoid(u):
    u = np.asarray(u, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-u))


def _rank_desc(values: np.ndarray, ids: np.ndarray):
    """Order candidates by value descending, equal values by id ascending; NaN last."""
    key = np.where(np.isnan(values), -np.inf, values)
    order = sorted(range(len(ids)), key=lambda j: (-key[j], ids[j]))
    return [int(ids[j]) for j in order], [float(key[j]) for j in order]


def route(x, w_router, bias, top_k: int, n_group: int = 1, topk_group: int = 1):
    """Affinity, bias-adjusted selection and gates for every token.

    s_{t,i} = sigmoid(x_t . e_i); z_{t,i} = s_{t,i} + b_i; S_t = the top_k experts by z
    (restricted to the topk_group best groups when n_group > 1); gates are the selected
    ORIGINAL affinities s normalised to sum to one -- the bias only decides selection.

    Returns a dict with idx [T, K] (descending z), gate [T, K], s [T, N], z [T, N], and the
    tie margins used by parity tests: ``margin`` (z of the K-th pick minus the best
    non-picked allowed z) and ``group_margin`` (score of the last kept group minus the best
    dropped group; +inf without groups).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)
    T = x.shape[0]
    N = w.shape[0]
    assert 1 <= top_k <= N and N % n_group == 0
    gsz = N // n_group
    if n_group > 1:
        assert gsz >= 2 and 1 <= topk_group <= n_group and top_k <= topk_group * gsz
    s = sigmoid(x @ w.T)
    z = s + b[None, :]
    idx = np.zeros((T, top_k), dtype=np.int64)
    gate = np.zeros((T, top_k), dtype=np.float64)
    margin = np.full(T, np.inf)
    gmargin = np.full(T, np.inf)
    for t in range(T):
        allowed = np.arange(N)
        if n_group > 1:
            gscore = np.empty(n_group)
            for g in range(n_group):
                zz = np.sort(np.where(np.isnan(z[t, g * gsz:(g + 1) * gsz]), -np.inf,
                                      z[t, g * gsz:(g + 1) * gsz]))[::-1]
                gscore[g] = zz[0] + zz[1]
            gorder, gvals = _rank_desc(gscore, np.arange(n_group))
            kept = sorted(gorder[:topk_group])
            if topk_group < n_group:
                gmargin[t] = gvals[topk_group - 1] - gvals[topk_group]
            allowed = np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in kept])
        order, vals = _rank_desc(z[t, allowed], allowed)
        sel = order[:top_k]
        if top_k < len(order):
            margin[t] = vals[top_k - 1] - vals[top_k]
        idx[t] = sel
        ss = s[t, sel]
        gate[t] = ss / ss.sum()
    return {"idx": idx, "gate": gate, "s": s, "z": z, "margin": margin, "group_margin": gmargin}


# --------------------------------------------------------------------------------------
# Load histogram, permutation, combine, bias update.
# --------------------------------------------------------------------------------------


def expert_counts(idx, n_experts: int) -> np.ndarray:
    """load_i = number of (token, slot) pairs routed to expert i over the whole batch
    ([TR] "DeepSeekMoE と補助損失なしの負荷分散": the load is monitored over the batch)."""
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in np.asarray(idx).reshape(-1):
        counts[e] += 1
    return counts


def permute(idx, n_experts: int, n_shared: int = 1):
    """Expert-major, token-ascending order of all (token, slot) pairs (a counting sort),
    followed by one segment of all T tokens in order for the shared expert.

    Returns (offsets [n_experts + n_shared + 1], sorted_token [T*(K+n_shared)],
    pair_pos [T, K]) with sorted_token[pair_pos[t, k]] == t.
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    counts = expert_counts(idx, n_experts)
    offsets = np.zeros(n_experts + n_shared + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    for j in range(n_shared):
        offsets[n_experts + j + 1] = offsets[n_experts + j] + T
    cursor = offsets[:n_experts].copy()
    sorted_token = np.zeros(T * (K + n_shared), dtype=np.int64)
    pair_pos = np.zeros((T, K), dtype=np.int64)
    for t in range(T):
        for k in range(K):
            e = idx[t, k]
            pos = cursor[e]
            cursor[e] += 1
            sorted_token[pos] = t
            pair_pos[t, k] = pos
    for j in range(n_shared):
        base = offsets[n_experts + j]
        sorted_token[base:base + T] = np.arange(T)
    return offsets, sorted_token, pair_pos


def combine(y_routed, y_shared, pair_pos, gate) -> np.ndarray:
    """out_t = y_shared[t] + sum_k gate[t, k] * y_routed[pair_pos[t, k]] (float64).
    ([PFN] "MoEの歴史とDeepSeekMoE-V3の特徴": the chosen experts' results come back and are
    merged with the always-on shared expert; [TR] "DualPipe パイプライン並列化": the
    combine stage.)"""
    y_routed = np.asarray(y_routed, dtype=np.float64)
    pair_pos = np.asarray(pair_pos)
    gate = np.asarray(gate, dtype=np.float64)
    T, K = pair_pos.shape
    out = np.zeros((T, y_routed.shape[1]))
    for k in range(K):
        out += gate[:, k:k + 1] * y_routed[pair_pos[:, k]]
    if y_shared is not None:
        out += np.asarray(y_shared, dtype=np.float64)
    return out


def bias_update(bias, counts, T: int, top_k: int, gamma: float) -> np.ndarray:
    """Aux-loss-free bias step ([TR] "DeepSeekMoE と補助損失なしの負荷分散"): an overloaded
    expert's bias drops by gamma, an underloaded one's rises by gamma, an expert exactly at
    the mean load T*K/N is left alone.  One float32 add per expert."""
    bias32 = np.asarray(bias, dtype=np.float32)
    counts = np.asarray(counts, dtype=np.int64)
    N = bias32.shape[0]
    diff = counts * N - int(T) * int(top_k)  # load - mean, scaled by N, in integers
    step = np.where(diff > 0, np.float32(-gamma), np.float32(gamma)).astype(np.float32)
    moved = (bias32 + step).astype(np.float32)
    return np.where(diff == 0, bias32, moved).astype(np.float32)


# --------------------------------------------------------------------------------------
# Expert FFN and the whole layer.
# --------------------------------------------------------------------------------------


def silu(a):
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def swiglu_hidden(x_rows, w13) -> np.ndarray:
    """h = silu(x W1^T) * (x W3^T) with W1 = w13[:I], W3 = w13[I:] (float64)."""
    I = w13.shape[0] // 2
    w13 = np.asarray(w13, dtype=np.float64)
    a = x_rows @ w13[:I].T
    c = x_rows @ w13[I:].T
    return silu(a) * c


def swiglu_ffn(x_rows, w13, w2) -> np.ndarray:
    """Expert FFN: W2 (silu(W1 x) * (W3 x)), float64, no intermediate rounding."""
    return swiglu_hidden(np.asarray(x_rows, dtype=np.float64), w13) @ np.asarray(w2, np.float64).T


def forward_dense(x, w_router, bias, w13, w2, top_k, n_group=1, topk_group=1):
    """The layer as a dense masked mixture over ALL experts (tiny shapes only):
    out_t = FFN_shared(x_t) + sum_i G_{t,i} FFN_i(x_t), G zero outside the selection.
    w13: [N+1, 2I, d], w2: [N+1, d, I]; the shared expert is index N."""
    x = np.asarray(x, dtype=np.float64)
    N = np.asarray(w_router).shape[0]
    r = route(x, w_router, bias, top_k, n_group, topk_group)
    T = x.shape[0]
    G = np.zeros((T, N))
    for t in range(T):
        G[t, r["idx"][t]] = r["gate"][t]
    out = swiglu_ffn(x, w13[N], w2[N])
    for i in range(N):
        out = out + G[:, i:i + 1] * swiglu_ffn(x, w13[i], w2[i])
    return out, r


def forward_sparse(x, idx, gate, n_experts: int, expert_weights, precision: str = "exact", workers: int = 1,
                   weights_quantised: bool = False):
    """The layer computed the sparse way: permute, per-expert FFN on gathered rows, combine.

    idx, gate: [T, K] routing decisions and gates (from ``route``).
    expert_weights(e) -> (w13_e [2I, d], w2_e [d, I]) for e in 0..n_experts, where
    e == n_experts is the shared expert.
    precision:
      "exact" -- float64 throughout;
      "bf16"  -- models the stored bfloat16 intermediates: h and the routed expert outputs
                 are rounded to bf16, the shared expert output to float32;
      "fp8"   -- models the FP8 path of [TR] "FP8 混合精度訓練": x quantised per 1x128
                 tile, weights per 128x128 block, h (as float32) re-quantised per 1x128
                 tile along I, products accumulated exactly (float64 stands in for the
                 FP32 promotion every 128 elements), routed outputs rounded to bf16,
                 shared output to float32;
      "fp8_e8m0" -- the same with power-of-two tile scales (``quant_1x128_e8m0``,
                 ``quant_128x128_e8m0``).
    workers > 1 evaluates the experts concurrently (same arithmetic, for large inputs).
    weights_quantised (fp8 precisions): expert_weights(e) already returns the weights after
    their 128x128 block quantisation (dequantised values), so they are not quantised again
    (for callers that quantise each expert once and reuse it; quantising such values again
    would give them back unchanged).
    Returns (out [T, d] float64, extras dict with the permutation and per-row outputs).
    """
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    gate = np.asarray(gate, dtype=np.float64)
    T, K = idx.shape
    offsets, sorted_token, pair_pos = permute(idx, n_experts, 1)
    if precision in ("fp8", "fp8_e8m0"):
        xq, xs = _quantisers(precision)[1](x)
        x_in = dequant_1x128(xq, xs)
    else:
        x_in = x
    d = x.shape[1]
    y_routed = np.zeros((T * K, d))
    y_shared = np.zeros((T, d))

    def one(e):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        we13, we2 = expert_weights(e)
        return e, lo, hi, expert_rows(x_in[sorted_token[lo:hi]], we13, we2, precision,
                                      weights_quantised=weights_quantised)

    todo = [e for e in range(n_experts + 1) if offsets[e + 1] > offsets[e]]
    results = _map_experts(one, todo, workers)
    for e, lo, hi, y in results:
        if e < n_experts:
            y_routed[lo:hi] = bf16_round(y) if precision != "exact" else y
        else:
            y_shared[:] = fp32_round(y) if precision != "exact" else y
    out = combine(y_routed, y_shared, pair_pos, gate)
    return out, {"offsets": offsets, "sorted_token": sorted_token, "pair_pos": pair_pos,
                 "y_routed": y_routed, "y_shared": y_shared}


def _map_experts(fn, experts, workers: int):
    """[fn(e) for e in experts], on `workers` threads when workers > 1 (each with a
    single-threaded BLAS, so the pool does not oversubscribe the cores).  Same arithmetic."""
    experts = list(experts)
    if workers <= 1:
        return [fn(e) for e in experts]
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, experts))


def _quantisers(precision: str):
    """(weight quantiser, activation quantiser) of an fp8 precision, each returning
    (E4M3 codes, scale values as float64)."""
    if precision == "fp8":
        return quant_128x128, quant_1x128

    def qw(w):
        q, c = quant_128x128_e8m0(w)
        return q, e8m0_decode(c)

    def qa(x):
        q, c = quant_1x128_e8m0(x)
        return q, e8m0_decode(c)
    return qw, qa


def expert_rows(rows, w13, w2, precision: str = "exact", return_h: bool = False, weights_quantised: bool = False):
    """One expert's FFN on already-gathered input rows (already dequantised on the fp8
    path), with the intermediate rounding of ``precision`` (see ``forward_sparse``).
    Returns y [m, d] before its own storage rounding (and h as stored, if asked)."""
    rows = np.asarray(rows, dtype=np.float64)
    if precision in ("fp8", "fp8_e8m0"):
        qw, qa = _quantisers(precision)
        w13d = np.asarray(w13, np.float64) if weights_quantised else dequant_128x128(*qw(w13))
        w2d = np.asarray(w2, np.float64) if weights_quantised else dequant_128x128(*qw(w2))
        h = swiglu_hidden(rows, w13d)
        hq, hs = qa(fp32_round(h))
        h_st = dequant_1x128(hq, hs)
        y = h_st @ w2d.T
    else:
        h = swiglu_hidden(rows, w13)
        h_st = bf16_round(h) if precision == "bf16" else h
        y = h_st @ np.asarray(w2, dtype=np.float64).T
    return (y, h_st) if return_h else y


def forward(x, w_router, bias, w13, w2, top_k, n_group=1, topk_group=1, precision="exact"):
    """Route on the (bf16) input in high precision, then run the sparse layer.
    w13: [N+1, 2I, d], w2: [N+1, d, I]; the shared expert is index N."""
    N = np.asarray(w_router).shape[0]
    r = route(x, w_router, bias, top_k, n_group, topk_group)
    out, extra = forward_sparse(x, r["idx"], r["gate"], N, lambda e: (w13[e], w2[e]), precision)
    return out, r, extra


# --------------------------------------------------------------------------------------
# Backward pass.  [TR] "FP8 混合精度訓練": the training step runs the layer's Fprop, Dgrad
# and Wgrad GEMMs; the gradients below are the chain rule of the forward definition above.
# The selection (top-K of z, and the bias inside z) is piecewise constant, so no gradient
# flows through it or to the bias; the gates carry the router's gradient.
# --------------------------------------------------------------------------------------


def backward(x, w_router, bias, w13, w2, top_k: int, d_out, n_group: int = 1, topk_group: int = 1,
             precision: str = "exact", workers: int = 1):
    """Gradients of L = sum(d_out * out) for the layer ``forward`` computes (float64).

    For every expert e and the rows routed to it (every token for the shared expert N):
      a = x W1^T, c = x W3^T, h = silu(a) c, y = h W2^T;
      dy = gate * d_out (routed) or d_out (shared); dgate = <d_out, y>;
      dW2 = dy^T h;  dh = dy W2;  da = dh c silu'(a), silu'(a) = sig(a) (1 + a (1 - sig(a)));
      dc = dh silu(a);  dW13 = [da | dc]^T x;  dx += da W1 + dc W3.
    Router, with the gates g_k = s_k / S over the selected affinities (S = sum of them):
      ds_k = (dgate_k - sum_j g_j dgate_j) / S;  du_k = ds_k s_k (1 - s_k);
      dx += sum_k du_k e_{idx_k};  dW_r[idx_k] += du_k x.
    precision "bf16" models the stored bfloat16 intermediates of the bf16 path: the forward's h
    and routed y, dy (the float32 product g * d_out, then bf16), [da | dc] and the routed rows'
    dx contributions are rounded to bf16 (RNE); everything else stays float64.
    precision "fp8" models the FP8 path ([TR] "FP8 混合精度訓練": Fprop, Dgrad and Wgrad in E4M3
    with 1x128 / 128x128 scaling): the forward as ``forward_sparse(..., "fp8")`` computes it
    (E4M3 x and weights, h stored as 1x128 E4M3, routed y bf16); Dgrad: dy and [da | dc] (bf16)
    quantised 1x128 along their reduction axis against the 128x128-quantised weights (the
    blocks of W^T are those of W, transposed); Wgrad: per expert, the operands transposed with
    the tokens as the reduction axis, zero-padded to a multiple of 128 from the expert's first
    row, dy^T and [da | dc]^T quantised 1x128 along the tokens, h^T (the stored E4M3 h as bf16)
    and x^T (the bf16 input) in 128x128 blocks; sums exact (float64).
    workers > 1 evaluates the experts concurrently (same arithmetic; their contributions are
    added in expert order).
    Returns dx [T, d], dw_router [N, d], dw13 [N+1, 2I, d], dw2 [N+1, d, I] and the
    intermediates dgate [T, K], du [T, K] and the routing dict."""
    assert precision in ("exact", "bf16", "fp8")
    fp8 = precision == "fp8"
    rnd = bf16_round if precision != "exact" else (lambda v: v)
    x = np.asarray(x, dtype=np.float64)
    wr = np.asarray(w_router, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    r = route(x, wr, bias, top_k, n_group, topk_group)
    idx, gate, s = r["idx"], r["gate"], r["s"]
    T, d = x.shape
    N = wr.shape[0]
    I = np.asarray(w13[0]).shape[0] // 2
    dx = np.zeros((T, d))
    dw13 = np.zeros((N + 1, 2 * I, d))
    dw2 = np.zeros((N + 1, d, I))
    dgate = np.zeros((T, top_k))
    x_in = dequant_1x128(*quant_1x128(x)) if fp8 else x

    def q_rows(m):     # 1x128 along the last axis, dequantised
        return dequant_1x128(*quant_1x128(m))

    def pad128(m):     # zero columns up to a multiple of 128
        return np.pad(m, ((0, 0), (0, (-m.shape[1]) % 128)))

    def one(e):
        """Expert e's contributions: (tok, slot, dgate values, dW2, dW13, dx rows) or None."""
        if e < N:
            tok, slot = np.nonzero(idx == e)   # each token picks distinct experts: tok is unique
        else:
            tok, slot = np.arange(T), None
        if len(tok) == 0:
            return None
        we13 = np.asarray(w13[e], dtype=np.float64)
        we2 = np.asarray(w2[e], dtype=np.float64)
        if fp8:
            we13 = dequant_128x128(*quant_128x128(we13))
            we2 = dequant_128x128(*quant_128x128(we2))
        xe = x_in[tok]
        a = xe @ we13[:I].T
        c = xe @ we13[I:].T
        sg = sigmoid(a)
        h = a * sg * c
        h = q_rows(fp32_round(h)) if fp8 else rnd(h)
        dg = None
        if e < N:
            dy = gate[tok, slot][:, None] * d_out[tok]
            dy = rnd(fp32_round(dy)) if precision != "exact" else dy
            dg = np.sum(d_out[tok] * rnd(h @ we2.T), axis=1)
        else:
            dy = d_out
        dh = (q_rows(dy) if fp8 else dy) @ we2
        da = rnd(dh * c * sg * (1.0 + a * (1.0 - sg)))
        dc = rnd(dh * a * sg)
        dac = np.concatenate([da, dc], axis=1)
        if fp8:
            dxe = q_rows(dac) @ we13
            dw2_e = q_rows(pad128(dy.T)) @ dequant_128x128(*quant_128x128(pad128(bf16_round(h).T))).T
            dw13_e = q_rows(pad128(dac.T)) @ dequant_128x128(*quant_128x128(pad128(x[tok].T))).T
        else:
            dw2_e = dy.T @ h
            dw13_e = dac.T @ xe
            dxe = dac @ we13
        return tok, slot, dg, dw2_e, dw13_e, rnd(dxe) if e < N else dxe

    results = _map_experts(one, range(N + 1), workers)
    for e, res in enumerate(results):
        if res is None:
            continue
        tok, slot, dg, dw2[e], dw13[e], dxe = res
        if dg is not None:
            dgate[tok, slot] = dg
        dx[tok] += dxe
    ssel = np.take_along_axis(s, idx, axis=1)
    S = ssel.sum(axis=1, keepdims=True)
    ds = (dgate - np.sum(gate * dgate, axis=1, keepdims=True)) / S
    du = ds * ssel * (1.0 - ssel)
    dwr = np.zeros((N, d))
    for k in range(top_k):
        dx += du[:, k:k + 1] * wr[idx[:, k]]
        np.add.at(dwr, idx[:, k], du[:, k:k + 1] * x)
    return {"dx": dx, "dw_router": dwr, "dw13": dw13, "dw2": dw2, "dgate": dgate, "du": du, "route": r}


def layer_flops(T: int, d: int, n_experts: int, top_k: int, inter: int, n_shared: int = 1) -> int:
    """Algorithmic FLOPs of one forward: router 2 T d N plus 6 d I per active expert-row."""
    return 2 * T * d * n_experts + 6 * d * inter * T * (top_k + n_shared)
