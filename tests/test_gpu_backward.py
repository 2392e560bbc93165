"""GPU parity of the backward pass (bf16 path) against the CPU oracle's ``backward``.

Each new kernel is checked on its own (the transpose and the dy rows bit-exact, the rest
against float64 within their rounding), then the whole layer backward in stages (every device
stage against float64 recomputed from the device's own upstream values) and end to end: dx,
dW_r, dW13, dW2 and du against the oracle's model of the bf16 path at max|err| / rms <= 1e-2.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_moe_layer_sigmoid_amd import inputs as I
from tests.gpu_common import FP8_DOT_REL, np64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BWD_TOL = 1e-2


def M():
    import sparse_moe_layer_sigmoid_amd as m
    return m


def test_segment_transpose_bitexact():
    """Segments of 0, 1, 63, 64, 65 and 200 rows, gathered rows, padded column blocks."""
    lens = np.array([0, 1, 63, 64, 65, 200])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pads = np.array([(n + 63) // 64 * 64 + (8 if n == 1 else 0) for n in lens])
    cols = np.concatenate([[0], np.cumsum(pads)]).astype(np.int32)
    rows, C = int(offs[-1]), 136
    src = I.gen_normal(71, (500, C), 1.0)
    gather = np.random.default_rng(5).integers(0, 500, rows).astype(np.int32)
    out = M()._lib.moe_segment_transpose(src.to(DEV), torch.from_numpy(offs).to(DEV), torch.from_numpy(cols).to(DEV),
                                         int(cols[-1]), src_rows=torch.from_numpy(gather).to(DEV))
    want = np.zeros((C, cols[-1]), dtype=np.float32)
    s = src.float().numpy()
    for g in range(len(lens)):
        for i in range(lens[g]):
            want[:, cols[g] + i] = s[gather[offs[g] + i]]
    assert np.array_equal(out.float().cpu().numpy(), want)


def test_segment_transpose_blocked():
    """Equal-width blocks [G][C][width]: segment g's rows land in its own zero-padded block."""
    lens = np.array([3, 0, 64, 40, 1])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    width = 64
    cols = np.arange(0, (len(lens) + 1) * width, width).astype(np.int32)
    C = 72
    src = I.gen_normal(74, (int(offs[-1]), C), 1.0)
    out = M()._lib.moe_segment_transpose(src.to(DEV), torch.from_numpy(offs).to(DEV), torch.from_numpy(cols).to(DEV),
                                         int(cols[-1]), width=width)
    want = np.zeros((len(lens), C, width), dtype=np.float32)
    s = src.float().numpy()
    for g in range(len(lens)):
        want[g, :, :lens[g]] = s[offs[g]:offs[g + 1]].T
    assert np.array_equal(out.float().cpu().numpy(), want)


def test_segment_transpose_unaligned_blocks():
    """Column blocks that start at arbitrary columns (the lanes' 8-column groups straddle them)."""
    lens = np.array([3, 0, 7, 20, 1, 9])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pads = lens + np.array([2, 1, 0, 5, 3, 4])
    cols = np.concatenate([[0], np.cumsum(pads)]).astype(np.int32)
    total = (int(cols[-1]) + 7) // 8 * 8
    cols[-1] = total
    C = 24
    src = I.gen_normal(77, (int(offs[-1]), C), 1.0)
    out = M()._lib.moe_segment_transpose(src.to(DEV), torch.from_numpy(offs).to(DEV), torch.from_numpy(cols).to(DEV),
                                         total)
    want = np.zeros((C, total), dtype=np.float32)
    s_ = src.float().numpy()
    for g in range(len(lens)):
        want[:, cols[g]:cols[g] + lens[g]] = s_[offs[g]:offs[g + 1]].T
    assert np.array_equal(out.float().cpu().numpy(), want)


@pytest.mark.parametrize("block", [False, True])
def test_segment_transpose_fp8_bitexact(block):
    """The fused transpose + E4M3 quantisation against the oracle's quantisers applied to the
    zero-padded transposed blocks: segments of 0, 1, 127, 128, 129 and 300 rows, gathered rows,
    an all-zero block, outliers."""
    lens = np.array([0, 1, 127, 128, 129, 300])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    width, C = 384, 256
    src = I.gen_normal(78, (900, C), 1.0).float().numpy()
    src[5, :] *= 1e-30   # tiny values
    src[17, 40] = 900.0  # an outlier
    src = torch.from_numpy(src).to(torch.bfloat16)
    gather = np.random.default_rng(6).integers(0, 900, int(offs[-1])).astype(np.int32)
    q, sc = M()._lib.moe_segment_transpose_fp8(src.to(DEV), torch.from_numpy(offs).to(DEV), width,
                                               src_rows=torch.from_numpy(gather).to(DEV), block_scales=block)
    s_ = src.float().numpy()
    blocks = np.zeros((len(lens), C, width), dtype=np.float32)
    for g in range(len(lens)):
        blocks[g, :, :lens[g]] = s_[gather[offs[g]:offs[g + 1]]].T
    if block:
        for g in range(len(lens)):
            wq, ws = O.quant_128x128(blocks[g])
            assert np.array_equal(q[g].cpu().numpy(), wq), g
            assert np.array_equal(sc[g].cpu().numpy(), ws), g
    else:
        wq, ws = O.quant_1x128(blocks.reshape(len(lens) * C, width))
        assert np.array_equal(q.cpu().numpy().reshape(len(lens) * C, width), wq)
        assert np.array_equal(sc.cpu().numpy(), ws)


def test_combine_backward_skipped_pair():
    """A pair the permutation skips (expert id out of range) contributes nothing: du = 0 there,
    the token's other gates are normalised over its valid affinities, no dy row is written."""
    T, K, N, d = 6, 3, 8, 64
    idx = torch.tensor([[1, 4, 6], [0, -1, 3], [2, 5, 7], [7, 9, 0], [3, 1, 2], [6, 5, 4]], dtype=torch.int32)
    offs, st_, pp = M()._lib.moe_permute(idx.to(DEV), N, 1)
    ppn = pp.cpu().numpy()
    assert ppn[1, 1] < 0 and ppn[3, 1] < 0
    rows = int(offs[-1].item())
    y = I.gen_normal(91, (T * K, d), 1.0)
    d_out = I.gen_normal(92, (T, d), 1.0)
    scores = torch.rand((T, N), generator=torch.Generator().manual_seed(3)) * 0.8 + 0.1
    gate = torch.rand((T, K), generator=torch.Generator().manual_seed(4))
    dy = torch.full((T * (K + 1), d), 7.0, dtype=torch.bfloat16, device=DEV)
    dy_, du, du_row = M()._lib.moe_combine_backward(d_out.to(DEV), y.to(DEV), idx.to(DEV), gate.to(DEV),
                                                    scores.to(DEV), pp, out={"dy": dy})
    du = du.cpu().numpy().astype(np.float64)
    yn, dn, sn, gn, ix = np64(y), np64(d_out), scores.double().numpy(), gate.double().numpy(), idx.numpy()
    for t_ in range(T):
        ok = ppn[t_] >= 0
        dg = np.array([np.dot(dn[t_], yn[ppn[t_, k]]) if ok[k] else 0.0 for k in range(K)])
        s = np.array([sn[t_, ix[t_, k]] if ok[k] else 0.0 for k in range(K)])
        g = np.where(ok, gn[t_], 0.0)
        want = np.where(ok, (dg - np.sum(g * dg)) / s.sum() * s * (1 - s), 0.0)
        assert np.allclose(du[t_], want, rtol=1e-4, atol=1e-6), (t_, du[t_], want)
    assert du[1, 1] == 0 and du[3, 1] == 0
    written = set(ppn[ppn >= 0].tolist()) | set(range(T * K, T * (K + 1)))
    untouched = [r for r in range(T * (K + 1)) if r not in written]
    assert torch.all(dy_[untouched] == 7.0)


def test_swiglu_backward():
    rows, inter = 77, 256
    ac = I.gen_normal(72, (rows, 2 * inter), 2.0, dtype=torch.float32)
    dh = I.gen_normal(73, (rows, inter), 1.0, dtype=torch.float32)
    dac = M()._lib.moe_swiglu_backward(ac.to(DEV), dh.to(DEV))
    a, c, g = ac[:, :inter].double().numpy(), ac[:, inter:].double().numpy(), dh.double().numpy()
    sg = O.sigmoid(a)
    want = np.concatenate([g * c * sg * (1 + a * (1 - sg)), g * a * sg], axis=1)
    got = np64(dac)
    # bf16 storage (2^-9 relative) plus the fast exp / reciprocal
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * np.sqrt(np.mean(want ** 2)))


def test_combine_and_swiglu_backward_fp8_outputs():
    """The E4M3 forms the two kernels write alongside their bf16 outputs: the oracle's 1x128
    quantiser applied to the device's own bf16 dy / [da | dc], bit for bit (including a skipped pair,
    whose rows stay unwritten, an all-zero d_out row and an outlier)."""
    T, K, N, d = 40, 4, 16, 384
    idx = torch.from_numpy(np.stack([np.random.default_rng(t).choice(N, K, replace=False) for t in range(T)])
                           .astype(np.int32))
    idx[5, 2] = -1  # skipped by the permutation
    offs, st_, pp = M()._lib.moe_permute(idx.to(DEV), N, 1)
    ppn = pp.cpu().numpy()
    y = I.gen_normal(95, (T * K, d), 1.0)
    dn = I.gen_normal(96, (T, d), 1.0).float().numpy()
    dn[7] = 0.0
    dn[9, 100] = 500.0
    d_out = torch.from_numpy(dn).to(torch.bfloat16)
    scores = torch.rand((T, N), generator=torch.Generator().manual_seed(5)) * 0.8 + 0.1
    gate = torch.rand((T, K), generator=torch.Generator().manual_seed(6))
    dy, du, du_row, dyq, dys = M()._lib.moe_combine_backward(d_out.to(DEV), y.to(DEV), idx.to(DEV), gate.to(DEV),
                                                             scores.to(DEV), pp, fp8=True)
    rows = sorted(set(ppn[ppn >= 0].tolist()) | set(range(T * K, T * (K + 1))))
    wq, ws = O.quant_1x128(dy[rows].float().cpu().numpy())
    assert np.array_equal(dyq[rows].cpu().numpy(), wq)
    assert np.array_equal(dys[rows].cpu().numpy(), ws)
    # the bf16 outputs are those of the plain call
    dy0, du0, _ = M()._lib.moe_combine_backward(d_out.to(DEV), y.to(DEV), idx.to(DEV), gate.to(DEV), scores.to(DEV), pp)
    assert torch.equal(dy0[rows], dy[rows]) and torch.equal(du0, du)

    r_, inter = 70, 256
    ac = I.gen_normal(97, (r_, 2 * inter), 2.0, dtype=torch.float32)
    dh = I.gen_normal(98, (r_, inter), 1.0, dtype=torch.float32)
    dh[3] = 0.0
    dac, dacq, dacs = M()._lib.moe_swiglu_backward(ac.to(DEV), dh.to(DEV), fp8=True)
    wq, ws = O.quant_1x128(dac.float().cpu().numpy())
    assert np.array_equal(dacq.cpu().numpy(), wq) and np.array_equal(dacs.cpu().numpy(), ws)
    assert torch.equal(M()._lib.moe_swiglu_backward(ac.to(DEV), dh.to(DEV)), dac)


def _layer(cfg):
    x = I.gen_x(cfg).to(torch.bfloat16)
    wr = I.gen_router(cfg).to(torch.bfloat16)
    bias = I.gen_bias(cfg)
    experts = [I.gen_expert(cfg, e) for e in range(cfg.groups)]
    W13 = torch.stack([e[0] for e in experts]).to(torch.bfloat16)
    W2 = torch.stack([e[1] for e in experts]).to(torch.bfloat16)
    return x, wr, bias, W13, W2


@pytest.mark.parametrize("cfg", [
    I.small(I.V3_BF16, name="bwd_small", T=300, d=256, n_experts=16, top_k=4, inter=128, w_std=0.05,
            router_std=0.05),
    I.small(I.V3_BF16, name="bwd_small_2", T=129, d=384, n_experts=32, top_k=8, inter=256, w_std=0.04,
            router_std=0.04),
], ids=lambda c: c.name)
def test_layer_backward(cfg):
    say(f"layer backward {cfg.name}")
    x, wr, bias, W13, W2 = _layer(cfg)
    layer = M().MoELayer(wr.to(DEV), W13.to(DEV), W2.to(DEV), bias.to(DEV), cfg.top_k)
    out, buf = layer.forward(x.to(DEV), out_dtype=torch.float32, train=True)
    d_out = I.gen_normal(cfg.seed + 900, (cfg.T, cfg.d), 1.0)
    g = layer.backward(d_out.to(DEV), buf, keep=True)
    torch.cuda.synchronize()
    x64, wr64, W13n, W2n, do64 = np64(x), np64(wr), np64(W13), np64(W2), np64(d_out)
    ref = O.backward(x64, wr64, bias.numpy(), W13n, W2n, cfg.top_k, do64)
    r = ref["route"]
    assert np.all(r["margin"] >= 1e-6), "a token sits in the tie window"
    assert np.array_equal(buf["topk_idx"].cpu().numpy(), r["idx"])
    # the pieces: dy rows bit-exact (RNE of the fp32 product), du against float64
    pp = buf["pair_pos"].cpu().numpy()
    dy = g["dy"].float().cpu().numpy()
    gate32 = buf["topk_gate"].cpu().numpy()
    do32 = d_out.float().numpy()
    for k in range(cfg.top_k):
        want = O.bf16_round((gate32[:, k:k + 1] * do32).astype(np.float32))
        assert np.array_equal(dy[pp[:, k]], want)
    assert np.array_equal(dy[cfg.T * cfg.top_k:], do32)
    # staged: every device stage against float64 recomputed from the device's own upstream
    # values (the forward's stored bf16 y and h, and each earlier stage's stored result)
    y = np64(buf["y"])
    h = np64(buf["h"])
    st_ = buf["sorted_token"].cpu().numpy()
    offs = buf["expert_offsets"].cpu().numpy()
    idx = buf["topk_idx"].cpu().numpy()
    s = buf["scores"].cpu().numpy().astype(np.float64)
    dyd = dy.astype(np.float64)
    dg = np.stack([np.sum(do32.astype(np.float64) * y[pp[:, k]], axis=1) for k in range(cfg.top_k)], axis=1)
    ssel = np.take_along_axis(s, idx, axis=1)
    gd = gate32.astype(np.float64)
    du_ref = (dg - np.sum(gd * dg, axis=1, keepdims=True)) / ssel.sum(1, keepdims=True) * ssel * (1 - ssel)
    du = g["du"].cpu().numpy().astype(np.float64)
    st_err = {"du": rel_err(du, du_ref)}
    assert np.array_equal(g["du_row"].cpu().numpy()[pp], g["du"].cpu().numpy())
    I_ = cfg.inter
    dac = np64(g["dac"])
    dac_ref = np.zeros_like(dac)
    dw2_ref = np.zeros((cfg.groups, cfg.d, I_))
    dw13_ref = np.zeros((cfg.groups, 2 * I_, cfg.d))
    dxr_ref = np.zeros((cfg.T * cfg.top_k, cfg.d))
    dxs_ref = np.zeros((cfg.T, cfg.d))
    for e in range(cfg.groups):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        xe = x64[st_[lo:hi]]
        a, c = xe @ W13n[e][:I_].T, xe @ W13n[e][I_:].T
        dh = dyd[lo:hi] @ W2n[e]
        sg = O.sigmoid(a)
        dac_ref[lo:hi] = np.concatenate([dh * c * sg * (1 + a * (1 - sg)), dh * a * sg], axis=1)
        dw2_ref[e] = dyd[lo:hi].T @ h[lo:hi]
        dw13_ref[e] = dac[lo:hi].T @ xe
        dxe = dac[lo:hi] @ W13n[e]
        if e < cfg.n_experts:
            dxr_ref[lo:hi] = dxe
        else:
            dxs_ref[:] = dxe
    # bf16-stored stages: each element within a bf16 half-step of the float64 value (half the
    # spacing 2^(floor(log2|v|) - 7)), plus fp32 rounding inside (the fast exp of silu, the GEMM
    # sums) on the tail's scale
    def bf16_bound(got, want, name):
        half = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 8)
        lim = half * 1.001 + 1e-4 * np.sqrt(np.mean(want ** 2))
        worst = float(np.max(np.abs(got - want) / lim))
        say(f"  {name}: max |err| / (bf16 half-step + 1e-4 rms) = {worst:.3f}")
        assert worst <= 1.0, name
    bf16_bound(dac, dac_ref, "dac")
    bf16_bound(np64(g["dx_routed"]), dxr_ref, "dx_routed")
    st_err["dx_shared"] = rel_err(np64(g["dx_shared"]), dxs_ref)
    dxr_dev = np64(g["dx_routed"])
    dx_ref = np64(g["dx_shared"]) + sum(du[:, k:k + 1] * wr64[idx[:, k]] + dxr_dev[pp[:, k]] for k in range(cfg.top_k))
    st_err["dx"] = rel_err(np64(g["dx"]), dx_ref)
    st_err["dw2"] = rel_err(np64(g["dw2"]), dw2_ref)
    st_err["dw13"] = rel_err(np64(g["dw13"]), dw13_ref)
    dwr_ref = np.zeros((cfg.n_experts, cfg.d))
    for k in range(cfg.top_k):
        np.add.at(dwr_ref, idx[:, k], du[:, k:k + 1] * x64)
    st_err["dw_router"] = rel_err(np64(g["dw_router"]), dwr_ref)
    say("  staged max|err| / rms: " + ", ".join(f"{k} {v:.2e}" for k, v in st_err.items()))
    # fp32 sums of exact products (du, dx, dW): far inside 1e-4 of the rms
    for k, v in st_err.items():
        assert v <= 1e-4, (k, v)
    # end to end against the oracle's model of the bf16 path (its stored intermediates rounded
    # as the device stores them): asserted at 1e-2; against the exact float64 gradients:
    # reported (the bf16 storage of h, y, dy, [da | dc] and the routed dx rows alone moves the
    # weight gradients by ~3e-2 of their rms at these sizes)
    model = O.backward(x64, wr64, bias.numpy(), W13n, W2n, cfg.top_k, do64, precision="bf16")
    errs, exact = {}, {}
    for name, got in (("dx", g["dx"]), ("dw_router", g["dw_router"]), ("dw13", g["dw13"]), ("dw2", g["dw2"]),
                      ("du", g["du"])):
        errs[name] = rel_err(np64(got), model[name])
        exact[name] = rel_err(np64(got), ref[name])
    say("  vs bf16 model max|err| / rms: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (tol {BWD_TOL})")
    say("  vs exact max|err| / rms: " + ", ".join(f"{k} {v:.2e}" for k, v in exact.items()))
    for k, v in errs.items():
        assert v <= BWD_TOL, (k, v)


def _bf16_bound(got, want, name, extra=0.0):
    half = np.exp2(np.floor(np.log2(np.maximum(np.abs(want) + extra, 1e-30))) - 8)
    lim = half * 1.001 + extra + 1e-4 * np.sqrt(np.mean(want ** 2))
    worst = float(np.max(np.abs(got - want) / lim))
    say(f"  {name}: max |err| / (bf16 half-step + 1e-4 rms) = {worst:.3f}")
    assert worst <= 1.0, name


@pytest.mark.parametrize("cfg", [
    I.small(I.V3_FP8, name="bwd_fp8_small", T=300, d=512, n_experts=32, top_k=4, inter=256, w_std=0.04,
            router_std=0.04, outlier_frac=7.2 / 512),
    I.small(I.V3_FP8, name="bwd_fp8_small_2", T=129, d=768, n_experts=16, top_k=8, inter=512, w_std=0.03,
            router_std=0.03),
], ids=lambda c: c.name)
def test_layer_backward_fp8(cfg):
    """The FP8 backward in stages: every quantisation bit-exact with the oracle's on the
    device's own bf16 operands, every E4M3 GEMM against float64 on the device's dequantised
    operands within the measured E4M3 dot-product bound (2^-10 of sum |a w|, pushed through
    the SwiGLU derivative for [da | dc]), bf16 stores within a half-step of that; end to end
    against the oracle's fp8 model at 3e-2 of each gradient's rms (rms, not max: E4M3 codes
    chosen near rounding midpoints differ between float32 and float64 sums, as in the forward,
    and one flipped code moves single elements by a visible fraction)."""
    say(f"layer backward fp8 {cfg.name}")
    x, wr, bias, W13, W2 = _layer(cfg)
    W13d, W2d = W13.to(DEV), W2.to(DEV)
    layer = M().MoELayer(wr.to(DEV), W13d, W2d, bias.to(DEV), cfg.top_k, fp8=True)
    out, buf = layer.forward(x.to(DEV), out_dtype=torch.float32, train=True)
    d_out = I.gen_normal(cfg.seed + 900, (cfg.T, cfg.d), 1.0)
    g = layer.backward(d_out.to(DEV), buf, keep=True)
    torch.cuda.synchronize()
    x64, wr64, do64 = np64(x), np64(wr), np64(d_out)
    I_, N, K, T = cfg.inter, cfg.n_experts, cfg.top_k, cfg.T
    offs = buf["expert_offsets"].cpu().numpy()
    st_ = buf["sorted_token"].cpu().numpy()
    pp = buf["pair_pos"].cpu().numpy()
    idx = buf["topk_idx"].cpu().numpy()
    dy = g["dy"].float().cpu().numpy()
    # quantisations, bit-exact on the device's own operands
    dyq, dys = O.quant_1x128(dy)
    assert np.array_equal(g["dyq"].cpu().numpy(), dyq) and np.array_equal(g["dys"].cpu().numpy(), dys)
    dac = np64(g["dac"])
    dacq, dacs = O.quant_1x128(dac)
    assert np.array_equal(g["dacq"].cpu().numpy(), dacq) and np.array_equal(g["dacs"].cpu().numpy(), dacs)
    # Dgrad stages against float64 from the device's quantised operands
    xd = O.dequant_1x128(buf["xq"].cpu().numpy(), buf["xs"].cpu().numpy())
    dyd = O.dequant_1x128(dyq, dys)
    dacd = O.dequant_1x128(dacq, dacs)
    dac_ref = np.zeros_like(dac)
    dac_tol = np.zeros_like(dac)
    dxr_ref = np.zeros((T * K, cfg.d))
    dxr_tol = np.zeros((T * K, cfg.d))
    dxs_ref = np.zeros((T, cfg.d))
    dxs_tol = np.zeros((T, cfg.d))
    for e in range(cfg.groups):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        w13 = O.dequant_128x128(layer.W13[e].cpu().numpy(), layer.W13_s[e].cpu().numpy())
        w2 = O.dequant_128x128(layer.W2[e].cpu().numpy(), layer.W2_s[e].cpu().numpy())
        xe = xd[st_[lo:hi]]
        a, c = xe @ w13[:I_].T, xe @ w13[I_:].T
        ea = FP8_DOT_REL * (np.abs(xe) @ np.abs(w13[:I_]).T)
        ec = FP8_DOT_REL * (np.abs(xe) @ np.abs(w13[I_:]).T)
        dh = dyd[lo:hi] @ w2
        edh = FP8_DOT_REL * (np.abs(dyd[lo:hi]) @ np.abs(w2))
        sg = O.sigmoid(a)
        ds = sg * (1 + a * (1 - sg))
        dac_ref[lo:hi] = np.concatenate([dh * c * ds, dh * a * sg], axis=1)
        # first-order propagation (|silu'| <= 1.1, |silu''| <= 0.6), doubled for the cross terms
        dac_tol[lo:hi] = 2 * np.concatenate([1.1 * np.abs(c) * edh + 1.1 * np.abs(dh) * ec + 0.6 * np.abs(dh * c) * ea,
                                             np.abs(a * sg) * edh + 1.1 * np.abs(dh) * ea], axis=1)
        dxe = dacd[lo:hi] @ w13
        etol = FP8_DOT_REL * (np.abs(dacd[lo:hi]) @ np.abs(w13))
        if e < N:
            dxr_ref[lo:hi], dxr_tol[lo:hi] = dxe, etol
        else:
            dxs_ref[:], dxs_tol[:] = dxe, etol
    _bf16_bound(dac, dac_ref, "dac", dac_tol)
    _bf16_bound(np64(g["dx_routed"]), dxr_ref, "dx_routed", dxr_tol)
    assert np.all(np.abs(np64(g["dx_shared"]) - dxs_ref) <= dxs_tol + 1e-6 * np.sqrt(np.mean(dxs_ref ** 2)))
    st_err = {}
    du = g["du"].cpu().numpy().astype(np.float64)
    dxr = np64(g["dx_routed"])
    dx_ref = np64(g["dx_shared"]) + sum(du[:, k:k + 1] * wr64[idx[:, k]] + dxr[pp[:, k]] for k in range(K))
    st_err["dx"] = rel_err(np64(g["dx"]), dx_ref)
    # Wgrad: the operands are the transposed, zero-padded rows, quantised as read; each GEMM
    # against float64 on its dequantised operands
    ops = g["wgrad_operands"]   # routed dW2, routed dW13, shared dW2, shared dW13
    h_dev = O.dequant_1x128(buf["h"].cpu().numpy(), buf["hs"].cpu().numpy())
    for which, (aq, as_, bq, bs) in enumerate(ops):
        aq, as_, bq, bs = (t_.cpu().numpy() for t_ in (aq, as_, bq, bs))
        A = O.dequant_1x128(aq, as_)
        ng = bq.shape[0]
        A = A.reshape(ng, -1, A.shape[1])
        dst = (g["dw2"] if which % 2 == 0 else g["dw13"])
        worst = 0.0
        for j in range(ng):
            B = O.dequant_128x128(bq[j], bs[j])
            e = j if which < 2 else N
            got = dst[e].cpu().numpy().astype(np.float64)
            want = A[j] @ B.T
            lim = FP8_DOT_REL * (np.abs(A[j]) @ np.abs(B).T) + 1e-30
            worst = max(worst, float(np.max(np.abs(got - want) / lim)))
        say(f"  Wgrad {('dW2', 'dW13')[which % 2]} ({'routed' if which < 2 else 'shared'}): max |err| / dot bound "
            f"= {worst:.3f}")
        assert worst <= 1.0
        # layout: the first routed expert's A operand is its rows transposed, 1x128 along tokens
        if which == 0:
            e = int(np.argmax(offs[1:N + 1] - offs[:N] > 0))
            lo, hi = int(offs[e]), int(offs[e + 1])
            kmax = aq.shape[1]
            want_q, want_s = O.quant_1x128(np.pad(dy[lo:hi].T, ((0, 0), (0, kmax - (hi - lo)))))
            assert np.array_equal(aq.reshape(ng, cfg.d, kmax)[e], want_q)
            hb = O.bf16_round(h_dev[lo:hi])
            wq, ws = O.quant_128x128(np.pad(hb.T, ((0, 0), (0, kmax - (hi - lo)))))
            assert np.array_equal(bq[e], wq) and np.array_equal(bs[e], ws)
    say("  staged max|err| / rms: " + ", ".join(f"{k} {v:.2e}" for k, v in st_err.items()))
    for k, v in st_err.items():
        assert v <= 1e-4, (k, v)
    ref = O.backward(x64, wr64, bias.numpy(), np64(W13), np64(W2), K, do64, precision="fp8")
    exact = O.backward(x64, wr64, bias.numpy(), np64(W13), np64(W2), K, do64)
    rep = []
    for name in ("dx", "dw_router", "dw13", "dw2"):
        got = np64(g[name])
        rms = np.sqrt(np.mean(ref[name] ** 2))
        rep.append(f"{name} {np.sqrt(np.mean((got - ref[name]) ** 2)) / rms:.2e} (exact "
                   f"{np.sqrt(np.mean((got - exact[name]) ** 2)) / np.sqrt(np.mean(exact[name] ** 2)):.2e})")
    say("  end to end, rms |err| / rms vs the oracle's fp8 model: " + ", ".join(rep))
    for name in ("dx", "dw_router", "dw13", "dw2"):
        got = np64(g[name])
        e = np.sqrt(np.mean((got - ref[name]) ** 2)) / np.sqrt(np.mean(ref[name] ** 2))
        assert e <= 3e-2, (name, e)


@pytest.mark.parametrize("cfg,fp8", [
    (I.small(I.V3_BF16, name="bwd_cache_bf16", T=300, d=256, n_experts=16, top_k=4, inter=128, w_std=0.05,
             router_std=0.05), False),
    (I.small(I.V3_FP8, name="bwd_cache_fp8", T=300, d=512, n_experts=32, top_k=4, inter=256, w_std=0.04,
             router_std=0.04), True),
], ids=["bf16", "fp8"])
def test_backward_cached_products_match_recompute(cfg, fp8):
    """The training forward (train=True) stores the gate/up products a | c beside h, and the
    backward takes them instead of running the gate/up GEMM again; without them in the buffers
    (a forward with keep=True only) it recomputes them.  Both ways give the same gradients bit for bit, and the stored a | c
    equal the recomputed ones."""
    say(f"backward cached vs recomputed a | c {cfg.name}")
    x, wr, bias, W13, W2 = _layer(cfg)
    layer = M().MoELayer(wr.to(DEV), W13.to(DEV), W2.to(DEV), bias.to(DEV), cfg.top_k, fp8=fp8)
    _, buf = layer.forward(x.to(DEV), out_dtype=torch.float32, train=True)
    assert buf["ac"] is not None and buf["ac"].shape == (cfg.T * (cfg.top_k + 1), 2 * cfg.inter)
    d_out = I.gen_normal(cfg.seed + 900, (cfg.T, cfg.d), 1.0).to(DEV)
    g1 = layer.backward(d_out, buf)
    ac = buf["ac"].clone()
    nobuf = dict(buf)
    del nobuf["ac"]
    g2 = layer.backward(d_out, nobuf)
    torch.cuda.synchronize()
    for k in ("dx", "dw_router", "dw13", "dw2"):
        assert torch.equal(g1[k], g2[k]), k
    # the recompute, as the backward runs it, against the stored products
    rows = cfg.T * (cfg.top_k + 1)
    again = torch.empty((rows, 2 * cfg.inter), dtype=torch.float32, device=DEV)
    if fp8:
        M().moe_grouped_gemm(buf["xq"], layer.W13, buf["expert_offsets"], 0, cfg.n_experts + 1, rows, again,
                             a_scale=buf["xs"], a_rows=buf["sorted_token"], w_scale=layer.W13_s)
    else:
        M().moe_grouped_gemm(buf["x"], layer.W13, buf["expert_offsets"], 0, cfg.n_experts + 1, rows, again,
                             a_rows=buf["sorted_token"])
    assert torch.equal(again, ac)
