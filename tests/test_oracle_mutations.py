"""Plant plausible mistakes in the CPU oracle and check that its pins catch every one.

A pin set that lets a dropped term, a wrong sign, a swapped operand or a wrong rounding
rule through would not justify trusting the oracle; each mutation below must make at
least one pin fail.  The mutations are applied with monkeypatch, on the CPU only.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import oracle_pins as P


def _any_pin_fails():
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception:
            return pin.__name__
    return None


def _mut_gate_from_z(mp):
    real = O.route

    def route(x, w, b, k, n_group=1, topk_group=1):
        r = real(x, w, b, k, n_group, topk_group)
        zz = np.take_along_axis(r["z"], r["idx"], 1)
        r["gate"] = zz / zz.sum(1, keepdims=True)
        return r
    mp.setattr(O, "route", route)


def _mut_ascending(mp):
    real = O._rank_desc

    def rank(values, ids):
        o, v = real(values, ids)
        return o[::-1], v[::-1]
    mp.setattr(O, "_rank_desc", rank)


def _mut_tie_higher_index(mp):
    def rank(values, ids):
        key = np.where(np.isnan(values), -np.inf, values)
        order = sorted(range(len(ids)), key=lambda j: (-key[j], -ids[j]))
        return [int(ids[j]) for j in order], [float(key[j]) for j in order]
    mp.setattr(O, "_rank_desc", rank)


def _mut_silu_sign(mp):
    mp.setattr(O, "silu", lambda a: np.asarray(a, np.float64) / (1.0 + np.exp(np.asarray(a, np.float64))))


def _mut_swap_w1_w3(mp):
    def hidden(x_rows, w13):
        I = w13.shape[0] // 2
        w13 = np.asarray(w13, np.float64)
        return O.silu(x_rows @ w13[I:].T) * (x_rows @ w13[:I].T)
    mp.setattr(O, "swiglu_hidden", hidden)


def _mut_bias_sign(mp):
    real = O.bias_update
    mp.setattr(O, "bias_update", lambda b, c, T, k, g: real(b, c, T, k, -g))


def _mut_bias_mean_off(mp):
    real = O.bias_update
    mp.setattr(O, "bias_update", lambda b, c, T, k, g: real(b, c, T, k + 1, g))


def _mut_e4m3_ties_odd(mp):
    def enc(v):
        v = np.asarray(v, np.float64)
        sign = np.signbit(v)
        a = np.abs(v)
        hi = np.minimum(np.searchsorted(O._E4M3_POS, a, side="left"), 126)
        lo = np.maximum(hi - 1, 0)
        dh, dl = O._E4M3_POS[hi] - a, a - O._E4M3_POS[lo]
        code = np.where((dh < dl) | ((dh == dl) & (hi % 2 == 1)), hi, lo)
        code = np.where(a >= 448, 126, code)
        code = np.where(O._E4M3_POS[hi] == a, hi, code).astype(np.uint8)
        return np.where(sign, code | 0x80, code).astype(np.uint8)
    mp.setattr(O, "e4m3_encode", enc)


def _mut_fnuz_scale(mp):
    mp.setattr(O, "_tile_scale", lambda amax: np.where(amax == 0, np.float32(1), (amax.astype(np.float32) / np.float32(240))).astype(np.float32))


def _mut_bf16_truncate(mp):
    def trunc(a):
        a = np.asarray(a, np.float64)
        m, e = np.frexp(a)
        return np.ldexp(np.trunc(m * 256.0), e - 8)
    mp.setattr(O, "bf16_round", trunc)


def _mut_permute_token_desc(mp):
    real = O.permute

    def perm(idx, n, ns=1):
        idx = np.asarray(idx)
        off, st, pp = real(idx[::-1], n, ns)
        T = idx.shape[0]
        st = st.copy()
        st[:T * idx.shape[1]] = T - 1 - st[:T * idx.shape[1]]
        return off, st, pp[::-1]
    mp.setattr(O, "permute", perm)


def _mut_combine_no_shared(mp):
    real = O.combine
    mp.setattr(O, "combine", lambda y, sh, pp, g: real(y, None, pp, g))


def _mut_group_max_not_top2(mp):
    real = O.route

    def route(x, w, b, k, n_group=1, topk_group=1):
        if n_group == 1:
            return real(x, w, b, k)
        # use only the single best z of each group as the group score
        x = np.asarray(x, np.float64)
        s = O.sigmoid(x @ np.asarray(w, np.float64).T)
        z = s + np.asarray(b, np.float64)
        N = z.shape[1]
        gs = N // n_group
        r = real(x, w, b, k, n_group, topk_group)
        for t in range(x.shape[0]):
            sc = z[t].reshape(n_group, gs).max(1)
            kept = sorted(np.argsort(-sc, kind="stable")[:topk_group])
            allowed = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in kept])
            sel = allowed[np.argsort(-z[t, allowed], kind="stable")[:k]]
            r["idx"][t] = sel
            r["gate"][t] = s[t, sel] / s[t, sel].sum()
        return r
    mp.setattr(O, "route", route)


def _mut_sigmoid_softmax(mp):
    def sm(u):
        u = np.asarray(u, np.float64)
        e = np.exp(u - u.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    mp.setattr(O, "sigmoid", sm)


def _mut_quant_transposed_block_scale(mp):
    real = O.dequant_128x128

    def deq(q, s):
        if s.shape[0] == s.shape[1]:
            return real(q, s.T)
        n, k = q.shape
        v = O.e4m3_decode(q).reshape(n // 128, 128, k // 128, 128)
        s2 = s.reshape(-1)[::-1].reshape(s.shape)  # scales attached to the wrong blocks
        return (v * s2.astype(np.float64)[:, None, :, None]).reshape(n, k)
    mp.setattr(O, "dequant_128x128", deq)


def _mut_e8m0_floor(mp):
    """Round the exponent down instead of up (the tile max then saturates)."""
    def ex(amax):
        a = np.asarray(amax, np.float64)
        with np.errstate(divide="ignore"):
            k = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0) / 448.0)), 0.0)
        return np.clip(k, -127, 127).astype(np.int64)
    mp.setattr(O, "e8m0_exponent", ex)


def _mut_e8m0_bias_126(mp):
    mp.setattr(O, "E8M0_BIAS", 126)


def _mut_e8m0_scale_wrong_tile(mp):
    real = O.quant_1x128_e8m0

    def quant(x):
        q, c = real(x)
        return q, np.roll(c, 1, axis=1)  # each tile's code attached to its neighbour
    mp.setattr(O, "quant_1x128_e8m0", quant)


def _mut_backward(mp, what):
    real = O.backward

    def bwd(x, wr, b, w13, w2, K, d_out, n_group=1, topk_group=1):
        g = real(x, wr, b, w13, w2, K, d_out, n_group, topk_group)
        g = dict(g)
        if what == "no_norm_term":      # forget that the gates are normalised
            r = g["route"]
            ssel = np.take_along_axis(r["s"], r["idx"], axis=1)
            S = ssel.sum(axis=1, keepdims=True)
            extra = (np.sum(r["gate"] * g["dgate"], axis=1, keepdims=True) / S) * ssel * (1 - ssel)
            dx = g["dx"].copy()
            dwr = g["dw_router"].copy()
            for k in range(K):
                dx += extra[:, k:k + 1] * np.asarray(wr)[r["idx"][:, k]]
                np.add.at(dwr, r["idx"][:, k], extra[:, k:k + 1] * np.asarray(x))
            g["dx"], g["dw_router"] = dx, dwr
        elif what == "swap_w13_halves":
            I = g["dw13"].shape[1] // 2
            g["dw13"] = np.concatenate([g["dw13"][:, I:], g["dw13"][:, :I]], axis=1)
        elif what == "dw2_transposed_rows":
            g["dw2"] = g["dw2"][:, ::-1]
        return g
    mp.setattr(O, "backward", bwd)


def _mut_bwd_no_norm_term(mp):
    _mut_backward(mp, "no_norm_term")


def _mut_bwd_swap_w13_halves(mp):
    _mut_backward(mp, "swap_w13_halves")


def _mut_bwd_dw2_rows(mp):
    _mut_backward(mp, "dw2_transposed_rows")


def _mut_bwd_silu_grad(mp):
    real_sig = O.sigmoid
    calls = {"n": 0}
    real = O.backward

    def bwd(*a, **kw):
        # sigmoid is called once for the router, then once per expert: perturb the experts'
        def sig(u):
            calls["n"] += 1
            v = real_sig(u)
            return v if calls["n"] == 1 else v * 0.999 + 0.0005
        calls["n"] = 0
        mp.setattr(O, "sigmoid", sig)
        try:
            return real(*a, **kw)
        finally:
            mp.setattr(O, "sigmoid", real_sig)
    mp.setattr(O, "backward", bwd)


def _patch_source(mp, func_name, old, new):
    """Plant a mistake by editing one line of an oracle function's source: the edited
    function is compiled against a copy of the oracle module's globals and put in place of
    the original for this test only."""
    src = textwrap.dedent(inspect.getsource(getattr(O, func_name)))
    assert src.count(old) == 1, (func_name, old)
    ns = dict(O.__dict__)
    exec(compile(src.replace(old, new), O.__file__, "exec"), ns)
    mp.setattr(O, func_name, ns[func_name])


def _mut_fwd_bf16_no_h_rounding(mp):
    _patch_source(mp, "expert_rows", 'h_st = bf16_round(h) if precision == "bf16" else h', "h_st = h")


def _mut_fwd_fp8_no_h_quant(mp):
    _patch_source(mp, "expert_rows", "h_st = dequant_1x128(hq, hs)", "h_st = h")


def _mut_fwd_routed_y_unrounded(mp):
    _patch_source(mp, "forward_sparse", 'y_routed[lo:hi] = bf16_round(y) if precision != "exact" else y',
                  "y_routed[lo:hi] = y")


def _mut_fwd_shared_y_bf16(mp):
    _patch_source(mp, "forward_sparse", 'y_shared[:] = fp32_round(y) if precision != "exact" else y',
                  'y_shared[:] = bf16_round(y) if precision != "exact" else y')


def _mut_fwd_fp8_x_unquantised(mp):
    _patch_source(mp, "forward_sparse", "x_in = dequant_1x128(xq, xs)", "x_in = x")


def _mut_route_margin_x100(mp):
    _patch_source(mp, "route", "margin[t] = vals[top_k - 1] - vals[top_k]",
                  "margin[t] = 100 * (vals[top_k - 1] - vals[top_k])")


def _mut_route_group_margin_x100(mp):
    _patch_source(mp, "route", "gmargin[t] = gvals[topk_group - 1] - gvals[topk_group]",
                  "gmargin[t] = 100 * (gvals[topk_group - 1] - gvals[topk_group])")


def _mut_route_margin_vs_kth(mp):
    _patch_source(mp, "route", "margin[t] = vals[top_k - 1] - vals[top_k]",
                  "margin[t] = vals[0] - vals[top_k]")


def _mut_e4m3_half_ulp_doubled(mp):
    real = O.e4m3_half_ulp
    mp.setattr(O, "e4m3_half_ulp", lambda v: 2.0 * real(v))


def _mut_e4m3_half_ulp_normal_spacing_everywhere(mp):
    _patch_source(mp, "e4m3_half_ulp", "np.maximum(a, 2.0 ** -6)", "np.maximum(a, 2.0 ** -9)")


def _mut_bwd_no_dy_rounding(mp):
    _patch_source(mp, "backward", 'dy = rnd(fp32_round(dy)) if precision != "exact" else dy', "dy = dy")


def _mut_bwd_no_da_rounding(mp):
    _patch_source(mp, "backward", "da = rnd(dh * c * sg * (1.0 + a * (1.0 - sg)))",
                  "da = dh * c * sg * (1.0 + a * (1.0 - sg))")


def _mut_bwd_no_dc_rounding(mp):
    _patch_source(mp, "backward", "dc = rnd(dh * a * sg)", "dc = dh * a * sg")


def _mut_bwd_no_h_rounding(mp):
    _patch_source(mp, "backward", "h = q_rows(fp32_round(h)) if fp8 else rnd(h)",
                  "h = q_rows(fp32_round(h)) if fp8 else h")


def _mut_bwd_fp8_no_h_quant(mp):
    _patch_source(mp, "backward", "h = q_rows(fp32_round(h)) if fp8 else rnd(h)",
                  "h = fp32_round(h) if fp8 else rnd(h)")


def _mut_bwd_routed_dx_unrounded(mp):
    _patch_source(mp, "backward", "rnd(dxe) if e < N else dxe", "dxe")


def _mut_bwd_fp8_dgrad_dy_unquantised(mp):
    _patch_source(mp, "backward", "dh = (q_rows(dy) if fp8 else dy) @ we2", "dh = dy @ we2")


def _mut_bwd_fp8_dgrad_dac_unquantised(mp):
    _patch_source(mp, "backward", "dxe = q_rows(dac) @ we13", "dxe = dac @ we13")


def _mut_bwd_fp8_wgrad_dy_unquantised(mp):
    _patch_source(mp, "backward", "dw2_e = q_rows(pad128(dy.T))", "dw2_e = pad128(dy.T)")


def _mut_bwd_fp8_wgrad_h_unquantised(mp):
    _patch_source(mp, "backward", "dequant_128x128(*quant_128x128(pad128(bf16_round(h).T))).T",
                  "pad128(bf16_round(h).T).T")


def _mut_bwd_fp8_wgrad_x_unquantised(mp):
    _patch_source(mp, "backward", "dequant_128x128(*quant_128x128(pad128(x[tok].T))).T", "pad128(x[tok].T).T")


def _mut_bwd_fp8_wgrad_dac_unquantised(mp):
    _patch_source(mp, "backward", "dw13_e = q_rows(pad128(dac.T))", "dw13_e = pad128(dac.T)")


def _mut_bwd_fp8_wgrad_dy_wrong_axis(mp):
    _patch_source(mp, "backward", "dw2_e = q_rows(pad128(dy.T))", "dw2_e = pad128(q_rows(dy).T)")


def _mut_bwd_fp8_x_unquantised(mp):
    _patch_source(mp, "backward", "x_in = dequant_1x128(*quant_1x128(x)) if fp8 else x", "x_in = x")


def _mut_fp32_round_toward_zero(mp):
    def trunc32(a):
        a = np.asarray(a, dtype=np.float64)
        f = a.astype(np.float32)
        over = np.abs(f.astype(np.float64)) > np.abs(a)
        f = np.where(over, np.nextafter(f, np.float32(0)), f)
        return f.astype(np.float64)
    mp.setattr(O, "fp32_round", trunc32)


def _mut_quant_amax_signed(mp):
    _patch_source(mp, "quant_1x128", "amax = np.max(np.abs(t), axis=2)", "amax = np.max(t, axis=2)")


def _mut_quant128_amax_signed(mp):
    _patch_source(mp, "quant_128x128", "amax = np.max(np.abs(b), axis=(1, 3))", "amax = np.max(b, axis=(1, 3))")


def _mut_tile_scale_zero_tile(mp):
    _patch_source(mp, "_tile_scale", "return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)",
                  "return s.astype(np.float32)")


def _mut_dequant_divides(mp):
    _patch_source(mp, "dequant_1x128", "* s.astype(np.float64)[:, :, None]", "/ s.astype(np.float64)[:, :, None]")


def _mut_e4m3_overflow_to_nan(mp):
    _patch_source(mp, "e4m3_encode", "code = np.where((a >= E4M3_MAX) | (code > 126), 126, code)",
                  "code = np.where((a > E4M3_MAX) | (code > 126), 127, code)")


def _mut_e4m3_subnormal_boundary(mp):
    _patch_source(mp, "e4m3_encode", "e = np.where(a < 2.0 ** -6, -6, e - 1)", "e = np.where(a < 2.0 ** -7, -7, e - 1)")


def _mut_e8m0_decode_off_by_one(mp):
    _patch_source(mp, "e8m0_decode", "np.exp2((c - E8M0_BIAS).astype(np.float64))",
                  "np.exp2((c - E8M0_BIAS + 1).astype(np.float64))")


def _mut_sigmoid_of_minus(mp):
    _patch_source(mp, "sigmoid", "return 1.0 / (1.0 + np.exp(-u))", "return 1.0 / (1.0 + np.exp(u))")


def _mut_counts_top1_only(mp):
    _patch_source(mp, "expert_counts", "for e in np.asarray(idx).reshape(-1):", "for e in np.asarray(idx)[:, 0]:")


def _mut_combine_gates_reversed(mp):
    _patch_source(mp, "combine", "out += gate[:, k:k + 1] * y_routed[pair_pos[:, k]]",
                  "out += gate[:, K - 1 - k:K - k] * y_routed[pair_pos[:, k]]")


def _mut_bias_average_expert_moves(mp):
    _patch_source(mp, "bias_update", "return np.where(diff == 0, bias32, moved).astype(np.float32)",
                  "return moved.astype(np.float32)")


def _mut_route_one_group_too_many(mp):
    _patch_source(mp, "route", "kept = sorted(gorder[:topk_group])", "kept = sorted(gorder[:topk_group + 1])")


def _mut_group_score_top3(mp):
    _patch_source(mp, "route", "gscore[g] = zz[0] + zz[1]", "gscore[g] = zz[0] + zz[1] + zz[2]")


def _mut_swiglu_no_silu(mp):
    _patch_source(mp, "swiglu_hidden", "return silu(a) * c", "return a * c")


def _mut_permute_shared_reversed(mp):
    _patch_source(mp, "permute", "sorted_token[base:base + T] = np.arange(T)", "sorted_token[base:base + T] = np.arange(T)[::-1]")


def _mut_fwd_shared_uses_expert0(mp):
    _patch_source(mp, "forward_sparse", "we13, we2 = expert_weights(e)",
                  "we13, we2 = expert_weights(e if e < n_experts else 0)")


def _mut_fwd_fp8_weights_unquantised(mp):
    _patch_source(mp, "expert_rows", "w13d = np.asarray(w13, np.float64) if weights_quantised else dequant_128x128(*qw(w13))",
                  "w13d = np.asarray(w13, np.float64)")


def _mut_fwd_fp8_w2_unquantised(mp):
    _patch_source(mp, "expert_rows", "w2d = np.asarray(w2, np.float64) if weights_quantised else dequant_128x128(*qw(w2))",
                  "w2d = np.asarray(w2, np.float64)")


def _mut_fwd_fp8_h_quantised_from_fp64(mp):
    _patch_source(mp, "expert_rows", "hq, hs = qa(fp32_round(h))", "hq, hs = qa(h)")


def _mut_fwd_fp8_e8m0_uses_fp32_scales(mp):
    _patch_source(mp, "_quantisers", 'if precision == "fp8":', 'if precision in ("fp8", "fp8_e8m0"):')


def _mut_layer_flops_no_shared(mp):
    real = O.layer_flops
    mp.setattr(O, "layer_flops", lambda T, d, n, k, i, n_shared=1: real(T, d, n, k, i, 0))


MUTATIONS = [
    _mut_gate_from_z, _mut_ascending, _mut_tie_higher_index, _mut_silu_sign, _mut_swap_w1_w3,
    _mut_bias_sign, _mut_bias_mean_off, _mut_e4m3_ties_odd, _mut_fnuz_scale,
    _mut_bf16_truncate, _mut_permute_token_desc, _mut_combine_no_shared,
    _mut_group_max_not_top2, _mut_sigmoid_softmax, _mut_quant_transposed_block_scale,
    _mut_e8m0_floor, _mut_e8m0_bias_126, _mut_e8m0_scale_wrong_tile,
    _mut_bwd_no_norm_term, _mut_bwd_swap_w13_halves, _mut_bwd_dw2_rows, _mut_bwd_silu_grad,
    _mut_fwd_bf16_no_h_rounding, _mut_fwd_fp8_no_h_quant, _mut_fwd_routed_y_unrounded, _mut_fwd_shared_y_bf16,
    _mut_fwd_fp8_x_unquantised, _mut_route_margin_x100, _mut_route_group_margin_x100, _mut_route_margin_vs_kth,
    _mut_e4m3_half_ulp_doubled, _mut_e4m3_half_ulp_normal_spacing_everywhere, _mut_bwd_no_dy_rounding,
    _mut_bwd_no_da_rounding, _mut_bwd_no_dc_rounding, _mut_bwd_no_h_rounding, _mut_bwd_fp8_no_h_quant,
    _mut_bwd_routed_dx_unrounded, _mut_bwd_fp8_dgrad_dy_unquantised, _mut_bwd_fp8_dgrad_dac_unquantised,
    _mut_bwd_fp8_wgrad_dy_unquantised, _mut_bwd_fp8_wgrad_h_unquantised, _mut_bwd_fp8_wgrad_x_unquantised,
    _mut_bwd_fp8_wgrad_dac_unquantised, _mut_bwd_fp8_wgrad_dy_wrong_axis, _mut_bwd_fp8_x_unquantised,
    _mut_fp32_round_toward_zero, _mut_quant_amax_signed, _mut_quant128_amax_signed, _mut_tile_scale_zero_tile,
    _mut_dequant_divides, _mut_e4m3_overflow_to_nan, _mut_e4m3_subnormal_boundary, _mut_e8m0_decode_off_by_one,
    _mut_sigmoid_of_minus, _mut_counts_top1_only, _mut_combine_gates_reversed, _mut_bias_average_expert_moves,
    _mut_route_one_group_too_many, _mut_group_score_top3, _mut_swiglu_no_silu, _mut_permute_shared_reversed,
    _mut_fwd_shared_uses_expert0, _mut_fwd_fp8_weights_unquantised, _mut_fwd_fp8_w2_unquantised,
    _mut_fwd_fp8_h_quantised_from_fp64, _mut_fwd_fp8_e8m0_uses_fp32_scales, _mut_layer_flops_no_shared,
]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__[5:])
def test_mutation_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    caught = _any_pin_fails()
    assert caught is not None, f"no pin catches {mutation.__name__}"
