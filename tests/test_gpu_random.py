"""Randomised shapes, seeded, against the oracle or float64.

moe_grouped_gemm: 64 draws of dtype (bf16 / E4M3), mode (f32 output, bf16 output with an f32
tail split, SwiGLU, ragged reduction), group count and sizes (empty groups included), K, N,
gathered or plain rows and a sub-range of the groups, each against a float64 product of the same
operands.  E4M3 operands are codes of small integers with power-of-two scales, so their sums are
exact in fp32 and those outputs must match bit for bit.

moe_route + moe_permute + moe_combine: 40 draws of T, d, the expert count, top-K and the group
limit: routing against the oracle's (sets exact outside the tie window, gates within 1e-6), the
permutation of the device's own routing bit-exact against the oracle's counting sort, and the
combine of random rows within the fp32 accumulation of the oracle's float64 sum.

moe_segment_transpose / moe_segment_transpose_fp8: 30 draws of segment counts and lengths, block
width, channel count and gathered rows."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from sparse_moe_layer_sigmoid_amd import inputs as I
from tests.gpu_common import check_route, np64, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def M():
    import sparse_moe_layer_sigmoid_amd as m
    return m


def _draw(seed):
    r = np.random.default_rng(7000 + seed)
    fp8 = bool(r.random() < 0.5)
    mode = ["f32", "tail", "swiglu", "ragged"][seed % 4]
    G = int(r.integers(1, 41))
    sizes = r.integers(0, 301, G)
    sizes[r.random(G) < 0.15] = 0
    gran = 128 if fp8 else 64
    K = gran * int(r.integers(1, 9))
    N = (256 if fp8 else 128) * int(r.integers(1, 3 if fp8 else 5))
    gather = bool(r.random() < 0.5)
    first = int(r.integers(0, G)) if r.random() < 0.3 else 0
    n_groups = G - first
    tail = int(r.integers(1, min(2, n_groups) + 1)) if mode == "tail" else 0
    return r, fp8, mode, G, sizes, gran, K, N, gather, first, n_groups, tail


@pytest.mark.parametrize("seed", range(64))
def test_gemm_random_shapes(seed):
    r, fp8, mode, G, sizes, gran, K, N, gather, first, n_groups, tail = _draw(seed)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows_all = int(offs[-1])
    base = int(offs[first])
    m_total = int(offs[first + n_groups]) - base
    say(f"random gemm seed {seed}: {'E4M3' if fp8 else 'bf16'} {mode} G={G} first={first} K={K} N={N} "
        f"rows={m_total} gather={gather}")
    T = int(r.integers(1, 400)) if gather else max(rows_all, 1)
    a_rows = r.integers(0, T, max(rows_all, 1)).astype(np.int32) if gather else None
    if fp8:
        A = I.gen_e4m3_codes(100 + seed, (T, K), small_int=True)
        W = I.gen_e4m3_codes(200 + seed, (G, N, K), small_int=True)
        As = torch.where(I.gen_scales(300 + seed, (T, K // 128), pow2=True) <= 2.0 ** -6, 2.0 ** -4, 2.0 ** -3).float()
        Ws = torch.where(I.gen_scales(400 + seed, (G, N // 128, K // 128), pow2=True) <= 2.0 ** -6, 2.0 ** -5,
                         2.0 ** -4).float()
        Ad = O.dequant_1x128(A.numpy(), As.numpy())
        Wd = np.stack([O.dequant_128x128(W[g].numpy(), Ws[g].numpy()) for g in range(G)])
        kw = dict(a_scale=As.to(DEV), w_scale=Ws.to(DEV))
    else:
        A = I.gen_normal(100 + seed, (T, K), 1.0)
        W = I.gen_normal(200 + seed, (G, N, K), 0.05)
        Ad, Wd = np64(A), np64(W)
        kw = {}
    o = torch.from_numpy(offs).to(DEV)
    if gather:
        kw["a_rows"] = torch.from_numpy(a_rows).to(DEV)
    kg = None
    if mode == "ragged":
        lens = r.integers(0, K + 1, G)
        kw["k_offsets"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(DEV)
        kg = np.minimum(K, np.maximum(gran, -(-lens // gran) * gran))
    swiglu = mode == "swiglu"
    oc = N // 2 if swiglu else N
    if mode in ("f32", "ragged"):
        out = torch.full((max(m_total, 1), oc), float("nan"), dtype=torch.float32, device=DEV)
    else:
        out = torch.full((max(m_total, 1), oc), float("nan"), dtype=torch.bfloat16, device=DEV)
    if tail:
        t_first = first + n_groups - tail
        t_rows = int(offs[first + n_groups]) - int(offs[t_first])
        out_tail = torch.full((max(t_rows, 1), N), float("nan"), dtype=torch.float32, device=DEV)
        kw.update(out_tail=out_tail, tail_groups=tail)
    M().moe_grouped_gemm(A.to(DEV), W.to(DEV), o, first, n_groups, m_total, out[:m_total], swiglu=swiglu, **kw)
    got = np64(out)
    got_tail = np64(out_tail) if tail else None
    for g in range(first, first + n_groups):
        lo, hi = int(offs[g]), int(offs[g + 1])
        if hi == lo:
            continue
        src = a_rows[lo:hi] if gather else np.arange(lo, hi)
        k = int(kg[g]) if kg is not None else K
        a, w = Ad[src, :k], Wd[g, :, :k]
        if swiglu:
            ref = O.swiglu_hidden(a, Wd[g])
        else:
            ref = a @ w.T
        in_tail = tail and g >= first + n_groups - tail
        if in_tail:
            dst = got_tail[lo - int(offs[first + n_groups - tail]):hi - int(offs[first + n_groups - tail])]
        else:
            dst = got[lo - base:hi - base]
        rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
        if mode in ("f32", "ragged") or in_tail:
            if fp8:
                assert np.array_equal(dst, ref), (seed, g)
            else:
                assert np.max(np.abs(dst - ref)) <= 1e-5 * max(rms, 1e-30), (seed, g)
        elif swiglu:  # silu in fp32 on the matrix cores' sums, then one bf16 rounding
            assert np.all(np.abs(dst - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-5 * rms), (seed, g)
        else:  # bf16 output: one rounding of the fp32 sum (exact for E4M3 operands)
            if fp8:
                assert np.array_equal(dst, O.bf16_round(ref.astype(np.float32)).astype(np.float64)), (seed, g)
            else:
                assert np.all(np.abs(dst - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6 * rms), (seed, g)


def _route_draw(seed):
    r = np.random.default_rng(9000 + seed)
    N = int(r.choice([8, 16, 32, 64, 128, 256]))
    ng, tg = 1, 1
    if r.random() < 0.5:
        cands = [g for g in (2, 4, 8, 16, 32, 64) if N % g == 0 and N // g >= 4]
        if cands:
            ng = int(r.choice(cands))
            tg = int(r.integers(1, ng + 1))
    K = int(r.integers(1, min(N, tg * (N // ng), 16) + 1))
    T = int(r.integers(0, 3000))
    d = 64 * int(r.integers(1, 17))
    return r, T, d, N, K, ng, tg


@pytest.mark.parametrize("seed", range(40))
def test_route_permute_combine_random(seed):
    r, T, d, N, K, ng, tg = _route_draw(seed)
    say(f"random route seed {seed}: T={T} d={d} N={N} K={K} groups={ng}/{tg}")
    x = I.gen_normal(500 + seed, (T, d), 1.0)
    wr = I.gen_normal(600 + seed, (N, d), 0.5 / np.sqrt(d))
    bias = torch.from_numpy(r.uniform(-0.02, 0.02, N).astype(np.float32))
    idx, gate, counts, scores = M().moe_route(x.to(DEV), wr.to(DEV), bias.to(DEV), K, ng, tg, want_scores=True)
    ro = O.route(np64(x), np64(wr), bias.numpy(), K, ng, tg)
    if T > 0:
        check_route(idx, gate, counts, scores, ro, N, K)
    else:
        assert not counts.cpu().numpy().any()
    # the permutation of the device's own routing, bit-exact
    offs, st, pp = M().moe_permute(idx, N, 1)
    want_offs, want_st, want_pp = O.permute(idx.cpu().numpy(), N, 1)
    assert np.array_equal(offs.cpu().numpy(), want_offs)
    assert np.array_equal(st.cpu().numpy(), want_st)
    assert np.array_equal(pp.cpu().numpy(), want_pp)
    # the combine of random routed rows (bf16) and shared rows (f32) with the device's gates
    if T > 0:
        y = I.gen_normal(700 + seed, (T * K, d), 1.0)
        ysh = I.gen_normal(800 + seed, (T, d), 1.0, dtype=torch.float32)
        out = M().moe_combine(y.to(DEV), ysh.to(DEV), pp, gate, torch.float32)
        ref = O.combine(np64(y), np64(ysh), pp.cpu().numpy(), gate.cpu().numpy().astype(np.float64))
        bound = (K + 1) * 2.0 ** -23 * (np.abs(np64(ysh)) + np.abs(np64(y))[pp.cpu().numpy()].sum(axis=1)) + 1e-30
        assert np.all(np.abs(np64(out) - ref) <= bound)


def _transpose_draw(seed):
    r = np.random.default_rng(11000 + seed)
    fp8 = bool(seed % 2)
    n_seg = int(r.integers(1, 21))
    lens = r.integers(0, 301, n_seg)
    lens[r.random(n_seg) < 0.15] = 0
    gran = 128 if fp8 else 64
    width = gran * int(r.integers(max(1, -(-int(lens.max()) // gran)), max(1, -(-int(lens.max()) // gran)) + 3))
    C = (128 if fp8 else 8) * int(r.integers(1, 5 if fp8 else 65))
    gather = bool(r.random() < 0.5)
    return r, fp8, lens, width, C, gather


@pytest.mark.parametrize("seed", range(30))
def test_segment_transpose_random(seed):
    """Random segments into equal-width blocks [n][C][width] (bf16: exact copies with zero padding;
    E4M3: the oracle's 1x128 or 128x128 quantisers applied to those padded bf16 blocks)."""
    r, fp8, lens, width, C, gather = _transpose_draw(seed)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n_seg, rows = len(lens), int(offs[-1])
    n_src = int(r.integers(1, 600)) if gather else max(rows, 1)
    say(f"random transpose seed {seed}: {'E4M3' if fp8 else 'bf16'} segments={n_seg} rows={rows} C={C} "
        f"width={width} gather={gather}")
    src = I.gen_normal(900 + seed, (n_src, C), 1.0)
    g_rows = r.integers(0, n_src, max(rows, 1)).astype(np.int32) if gather else None
    s_ = src.float().numpy()
    blocks = np.zeros((n_seg, C, width), dtype=np.float32)
    for g in range(n_seg):
        sel = g_rows[offs[g]:offs[g + 1]] if gather else np.arange(offs[g], offs[g + 1])
        blocks[g, :, :lens[g]] = s_[sel].T
    o = torch.from_numpy(offs).to(DEV)
    kw = dict(src_rows=torch.from_numpy(g_rows).to(DEV)) if gather else {}
    if fp8:
        block = bool(r.random() < 0.5)
        q, sc = M()._lib.moe_segment_transpose_fp8(src.to(DEV), o, width, block_scales=block, **kw)
        if block:
            for g in range(n_seg):
                wq, ws = O.quant_128x128(blocks[g])
                assert np.array_equal(q[g].cpu().numpy(), wq), g
                assert np.array_equal(sc[g].cpu().numpy(), ws), g
        else:
            wq, ws = O.quant_1x128(blocks.reshape(n_seg * C, width))
            assert np.array_equal(q.cpu().numpy().reshape(n_seg * C, width), wq)
            assert np.array_equal(sc.cpu().numpy(), ws)
    else:
        cols = np.arange(0, (n_seg + 1) * width, width).astype(np.int32)
        out = M()._lib.moe_segment_transpose(src.to(DEV), o, torch.from_numpy(cols).to(DEV), n_seg * width,
                                             width=width, **kw)
        assert np.array_equal(out.float().cpu().numpy(), blocks)


def _layer_draw(seed):
    r = np.random.default_rng(13000 + seed)
    N = int(r.choice([8, 16, 32, 64]))
    ng, tg = 1, 1
    if r.random() < 0.4:
        cands = [g for g in (2, 4, 8) if N % g == 0 and N // g >= 4]
        if cands:
            ng = int(r.choice(cands))
            tg = int(r.integers(1, ng + 1))
    K = int(r.integers(1, min(8, tg * (N // ng)) + 1))
    T = int(r.integers(1, 401))
    d = 128 * int(r.integers(1, 5))
    inter = 64 * int(r.integers(1, 5))
    return I.small(I.V3_BF16, name=f"rand_layer_{seed}", T=T, d=d, n_experts=N, top_k=K, inter=inter, n_group=ng,
                   topk_group=tg, w_std=0.05, router_std=0.05, seed=14000 + seed)


@pytest.mark.parametrize("seed", range(10))
def test_layer_bf16_random(seed):
    """Whole bf16 layers of random shape (T, d, expert count, top-K down to 1, group limit,
    width), stage by stage against float64 recomputed from the device's own upstream values:
    the routing against the oracle's; h = silu(a) c within one bf16 rounding of the float64 SwiGLU
    of x and W13; each routed row within one bf16 rounding, and the shared rows within fp32
    accumulation, of the float64 product of the device's h and W2; the output within the fp32
    accumulation of the combine of the device's rows.  The error against the oracle's bf16 model
    end to end is reported (with one expert per token a single bf16 rounding of a row near a
    midpoint can move an output element by 2^-7 of that row, beyond the 1e-2 bar of the K = 8
    layer)."""
    from tests.gpu_common import rel_err
    cfg = _layer_draw(seed)
    say(f"random layer seed {seed}: T={cfg.T} d={cfg.d} N={cfg.n_experts} K={cfg.top_k} I={cfg.inter} "
        f"groups={cfg.n_group}/{cfg.topk_group}")
    x = I.gen_x(cfg).to(torch.bfloat16)
    wr = I.gen_router(cfg).to(torch.bfloat16)
    bias = I.gen_bias(cfg)
    ex = [I.gen_expert(cfg, e) for e in range(cfg.groups)]
    W13 = torch.stack([a for a, _ in ex]).to(torch.bfloat16)
    W2 = torch.stack([b for _, b in ex]).to(torch.bfloat16)
    layer = M().MoELayer(wr.to(DEV), W13.to(DEV), W2.to(DEV), bias.to(DEV), cfg.top_k, cfg.n_group, cfg.topk_group)
    out32, buf = layer.forward(x.to(DEV), out_dtype=torch.float32, keep=True)
    x64 = np64(x)
    r = O.route(x64, np64(wr), bias.numpy(), cfg.top_k, cfg.n_group, cfg.topk_group)
    tie = check_route(buf["topk_idx"], buf["topk_gate"], buf["expert_counts"], None, r, cfg.n_experts, cfg.top_k)
    W13n, W2n = np64(W13), np64(W2)
    offs = buf["expert_offsets"].cpu().numpy()
    st = buf["sorted_token"].cpu().numpy()
    hd, yd, ysd = np64(buf["h"]), np64(buf["y"]), np64(buf["y_shared"])
    N, T = cfg.n_experts, cfg.T
    for e in range(N + 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        h64 = O.swiglu_hidden(x64[st[lo:hi]], W13n[e])
        hr = float(np.sqrt(np.mean(h64 ** 2)))
        assert np.all(np.abs(hd[lo:hi] - h64) <= np.abs(h64) * 2.0 ** -8 + 1e-5 * hr), (seed, e, "h")
        y64 = hd[lo:hi] @ W2n[e].T
        yrms = float(np.sqrt(np.mean(y64 ** 2)))
        if e < N:
            assert np.all(np.abs(yd[lo:hi] - y64) <= np.abs(y64) * 2.0 ** -8 + 1e-6 * yrms), (seed, e, "y")
        else:
            assert np.max(np.abs(ysd - y64)) <= 1e-5 * yrms, (seed, "shared y")
    pp = buf["pair_pos"].cpu().numpy()
    gate = buf["topk_gate"].cpu().numpy().astype(np.float64)
    comb = ysd + np.einsum("tk,tkd->td", gate, yd[pp])
    terms = np.abs(ysd) + np.einsum("tk,tkd->td", np.abs(gate), np.abs(yd[pp]))
    assert np.all(np.abs(np64(out32) - comb) <= (cfg.top_k + 1) * 2.0 ** -23 * terms + 1e-30), (seed, "combine")
    ref, _ = O.forward_sparse(x64, r["idx"], r["gate"], N, lambda e: (W13n[e], W2n[e]), "bf16")
    keep = ~tie
    say(f"  max|err|/rms vs the oracle's bf16 model {rel_err(np64(out32)[keep], ref[keep]):.2e}")
