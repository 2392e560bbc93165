"""MoELayer: sequences the C-ABI calls for one DeepSeekMoE layer forward on one GPU.

Holds the (device-resident) weights and allocates the per-batch buffers; every step runs
in libmoe's kernels:

    route -> permute -> [fp8: quantise x per 1x128] -> gate/up grouped GEMM + SwiGLU
          -> down grouped GEMM (routed experts to bf16 rows, the shared expert to fp32 rows)
          -> combine -> [bias update]

Layer definition: "DeepSeek-V3 Technical Report" (wiki summary), "DeepSeekMoE と補助損失
なしの負荷分散" (1 shared + N routed experts, top-K by sigmoid affinity + bias, gates from
the normalised original affinities, bias moved by gamma against the load) and
"FP8 混合精度訓練" (the FP8 variant).
"""
from __future__ import annotations

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, w_router, W13, W2, bias, top_k: int, n_group: int = 1, topk_group: int = 1,
                 fp8: bool = False, fp8_scales: str = "f32"):
        """w_router [N, d] bf16; W13 [N+1, 2I, d] bf16 (rows [0,I) gate, [I,2I) up; expert N is
        the shared one); W2 [N+1, d, I] bf16; bias [N] f32.  With fp8=True the weights are
        block-quantised once (128x128, E4M3) and the layer runs the FP8 path, with f32 tile
        scales (fp8_scales="f32") or power-of-two ones stored as E8M0 codes ("e8m0")."""
        if fp8_scales not in ("f32", "e8m0"):
            raise ValueError(f"fp8_scales must be 'f32' or 'e8m0', got {fp8_scales!r}")
        self.w_router = w_router
        self.bias = bias
        self.N = w_router.shape[0]
        self.d = w_router.shape[1]
        self.I = W13.shape[1] // 2
        self.top_k = top_k
        self.n_group = n_group
        self.topk_group = topk_group
        self.fp8 = fp8
        self.e8m0 = fp8 and fp8_scales == "e8m0"
        # the FP8 backward quantises W^T itself, from the bf16 weights (held by reference)
        self._src = (W13, W2) if fp8 else None
        if fp8:
            qw = L.fp8_quant_128x128_e8m0 if self.e8m0 else L.fp8_quant_128x128
            self.W13, self.W13_s = qw(W13)
            self.W2, self.W2_s = qw(W2)
        else:
            self.W13, self.W13_s = W13, None
            self.W2, self.W2_s = W2, None

    def forward(self, x, out_dtype=torch.bfloat16, update_bias: bool = False, gamma: float = 0.001,
                keep: bool = False, train: bool = False):
        """x [T, d] bf16 -> out [T, d] (bf16 or f32).  With keep=True returns (out, buffers), which
        the backward takes.  train=True (implies keep) is the training forward: the buffers then
        also hold the gate/up products a | c (f32, written by the gate/up GEMM beside h), which
        the backward takes instead of running the gate/up GEMM again."""
        if train:
            if self.e8m0:
                raise NotImplementedError("the backward pass runs on the bf16 and the f32-scale FP8 paths")
            keep = True
        T, d = x.shape
        N, K, I = self.N, self.top_k, self.I
        dev = x.device
        idx, gate, counts, scores = L.moe_route(x, self.w_router, self.bias, K, self.n_group, self.topk_group,
                                                want_scores=keep)
        offs, sorted_token, pair_pos = L.moe_permute(idx, N, 1)
        if keep:  # the backward sizes its weight-gradient operands from these: copied to the host now
            offs_host = torch.empty(offs.shape, dtype=offs.dtype, pin_memory=True)
            offs_host.copy_(offs, non_blocking=True)
            offs_ready = torch.cuda.Event()
            offs_ready.record()
        rows = T * (K + 1)
        ac = torch.empty((rows, 2 * I), dtype=torch.float32, device=dev) if train else None
        if self.fp8:
            xq, xs = (L.fp8_quant_1x128_e8m0 if self.e8m0 else L.fp8_quant_1x128)(x)
            h = torch.empty((rows, I), dtype=torch.uint8, device=dev)
            hs = torch.empty((rows, I // 128), dtype=xs.dtype, device=dev)
            L.moe_grouped_gemm(xq, self.W13, offs, 0, N + 1, rows, h, a_scale=xs, a_rows=sorted_token,
                               w_scale=self.W13_s, swiglu=True, out_scale=hs, out_preact=ac)
        else:
            xq = xs = hs = None
            h = torch.empty((rows, I), dtype=torch.bfloat16, device=dev)
            L.moe_grouped_gemm(x, self.W13, offs, 0, N + 1, rows, h, a_rows=sorted_token, swiglu=True,
                               out_preact=ac)
        y = torch.empty((T * K, d), dtype=torch.bfloat16, device=dev)
        ysh = torch.empty((T, d), dtype=torch.float32, device=dev)
        # one launch for all N + 1 down projections: routed rows to y (bf16), the shared
        # expert's rows (the last group) to ysh (f32)
        L.moe_grouped_gemm(h, self.W2, offs, 0, N + 1, rows, y, a_scale=hs, w_scale=self.W2_s, out_tail=ysh,
                           tail_groups=1)
        out = L.moe_combine(y, ysh, pair_pos, gate, out_dtype)
        if update_bias:
            L.moe_bias_update(self.bias, counts, T * K, gamma)
        if keep:
            return out, {"x": x, "scores": scores, "topk_idx": idx, "topk_gate": gate, "expert_counts": counts,
                         "expert_offsets": offs, "expert_offsets_host": (offs_host, offs_ready),
                         "sorted_token": sorted_token, "pair_pos": pair_pos,
                         "xq": xq, "xs": xs, "h": h, "hs": hs, "ac": ac, "y": y, "y_shared": ysh}
        return out

    # ------------------------------------------------------------------ backward (bf16 path)

    def _transposed_weights(self):
        """W13^T [N+1, d, 2I] and W2^T [N+1, I, d] for the Dgrad GEMMs, made once: bf16, or on
        the FP8 path E4M3 with 128x128 block scales (the blocks of W^T are those of W,
        transposed, so these are the forward's codes and scales in transposed order)."""
        if getattr(self, "_WT", None) is None:
            if self.e8m0:
                raise NotImplementedError("the backward pass runs on the bf16 and the f32-scale FP8 paths")
            W13, W2 = self._src if self.fp8 else (self.W13, self.W2)
            G, I2, d = W13.shape
            dev = W13.device
            one = lambda n: torch.tensor([0, n], dtype=torch.int32, device=dev)
            W13T = torch.empty((G, d, I2), dtype=torch.bfloat16, device=dev)
            W2T = torch.empty((G, I2 // 2, d), dtype=torch.bfloat16, device=dev)
            s13, s2 = one(I2), one(d)
            for g in range(G):
                L.moe_segment_transpose(W13[g], s13, s13, I2, dst=W13T[g])
                L.moe_segment_transpose(W2[g], s2, s2, d, dst=W2T[g])
            if self.fp8:
                W13T, W13T_s = L.fp8_quant_128x128(W13T)
                W2T, W2T_s = L.fp8_quant_128x128(W2T)
                self._WT = (W13T, W2T, W13T_s, W2T_s)
            else:
                self._WT = (W13T, W2T, None, None)
        return self._WT

    def backward(self, d_out, buf, grads=None, keep: bool = False):
        """Gradients of sum(d_out * out) for the forward that returned `buf` (keep=True):
        dict of dx [T, d], dw_router [N, d], dw13 [N+1, 2I, d], dw2 [N+1, d, I], all f32.
        `grads` may hold preallocated dw13 / dw2 tensors (overwritten) to reuse across steps;
        keep=True adds the intermediates (dy, du, dac, the input-gradient rows, FP8 operands).
        On the FP8 path ([TR] "FP8 混合精度訓練": Dgrad and Wgrad in E4M3) every GEMM operand is
        E4M3: dy and [da | dc] quantised 1x128 along their reduction axis against the 128x128
        weight blocks (Dgrad); for Wgrad the transposed dy and [da | dc] quantised 1x128 along
        the tokens and the transposed h (the stored E4M3 h, as bf16) and x in 128x128 blocks.

        Sequence: combine backward (dy, router logit gradients) -> Dgrad of the down projection
        (dh = dy W2) -> [a | c from the forward, or the gate/up GEMM again without SwiGLU when the
        buffers lack them] -> SwiGLU backward -> Dgrad of
        the gate/up projection (dx rows) -> two combines (router term + shared rows, then the
        routed rows) -> Wgrad per expert over transposed row segments -> router Wgrad."""
        W13T, W2T, W13T_s, W2T_s = self._transposed_weights()
        fp8 = self.fp8
        q1 = L.fp8_quant_1x128
        x = buf["x"]
        T, d = x.shape
        N, K, I = self.N, self.top_k, self.I
        G = N + 1
        rows = T * (K + 1)
        dev = x.device
        offs, st_, pp = buf["expert_offsets"], buf["sorted_token"], buf["pair_pos"]
        # the expert sizes size the weight-gradient operands: the forward copied the offsets to
        # pinned host memory right after the permutation, so this waits at most for that copy
        # and the whole pass is then queued without waiting
        offs_host, offs_ready = buf["expert_offsets_host"]
        offs_ready.synchronize()
        lens = offs_host[1:] - offs_host[:-1]
        d_out = d_out.to(torch.bfloat16).contiguous()
        cb = L.moe_combine_backward(d_out, buf["y"], buf["topk_idx"], buf["topk_gate"], buf["scores"], pp, fp8=fp8)
        dy, du, du_row = cb[:3]
        extra = {}
        dh = torch.empty((rows, I), dtype=torch.float32, device=dev)
        # a | c: cached by the forward's gate/up GEMM (the same fp32 values), else recomputed
        ac = buf.get("ac")
        recompute = ac is None
        if recompute:
            ac = torch.empty((rows, 2 * I), dtype=torch.float32, device=dev)
        dxr = torch.empty((T * K, d), dtype=torch.bfloat16, device=dev)
        dxs = torch.empty((T, d), dtype=torch.float32, device=dev)
        if fp8:
            dyq, dys = cb[3:]  # dy's 1x128 E4M3 form, written by the combine backward itself
            L.moe_grouped_gemm(dyq, W2T, offs, 0, G, rows, dh, a_scale=dys, w_scale=W2T_s)
            if recompute:
                L.moe_grouped_gemm(buf["xq"], self.W13, offs, 0, G, rows, ac, a_scale=buf["xs"], a_rows=st_,
                                   w_scale=self.W13_s)
            dac, dacq, dacs = L.moe_swiglu_backward(ac, dh, fp8=True)
            L.moe_grouped_gemm(dacq, W13T, offs, 0, G, rows, dxr, a_scale=dacs, w_scale=W13T_s, out_tail=dxs,
                               tail_groups=1)
            extra.update(dyq=dyq, dys=dys, dacq=dacq, dacs=dacs)
        else:
            L.moe_grouped_gemm(dy, W2T, offs, 0, G, rows, dh)
            if recompute:
                L.moe_grouped_gemm(x, self.W13, offs, 0, G, rows, ac, a_rows=st_)
            dac = L.moe_swiglu_backward(ac, dh)
            L.moe_grouped_gemm(dac, W13T, offs, 0, G, rows, dxr, out_tail=dxs, tail_groups=1)
        del ac, dh
        # dx = sum_k dxr[pair] + dxs + sum_k du_k e_{idx_k}: the router term and the shared rows
        # first (a combine over the router rows), then the routed rows
        part = L.moe_combine(self.w_router, dxs, buf["topk_idx"], du, torch.float32)
        dx = L.moe_combine(dxr, part, pp, torch.ones((T, K), dtype=torch.float32, device=dev), torch.float32)
        # Wgrad: each expert's rows are the reduction axis.  The routed experts' rows become
        # equal-width zero-padded blocks [N][C][kmax] (kmax = the largest routed segment,
        # rounded up to the K step), so one grouped GEMM covers all of them; the GEMM's ragged
        # reduction (k_offsets = the expert offsets) stops each expert at its own length
        # rounded up to the K step, and an empty expert reduces one zero step to a zero
        # gradient.  The shared expert (all T tokens) has its own launch.
        kq = 128 if fp8 else 64  # K granule of the GEMM
        kmax = max(kq, (int(lens[:N].max()) + kq - 1) // kq * kq)
        kp_s = (int(lens[N]) + kq - 1) // kq * kq
        seg_r, seg_s = offs[:N + 1], offs[N:N + 2]
        h = L.fp8_dequant_1x128(buf["h"], buf["hs"]) if fp8 else buf["h"]
        grads = grads or {}
        dw2 = grads.get("dw2")
        dw13 = grads.get("dw13")
        if dw2 is None:
            dw2 = torch.empty((G, d, I), dtype=torch.float32, device=dev)
        if dw13 is None:
            dw13 = torch.empty((G, 2 * I, d), dtype=torch.float32, device=dev)
        g_d = torch.arange(0, (N + 1) * d, d, dtype=torch.int32, device=dev)
        g_2i = torch.arange(0, (N + 1) * 2 * I, 2 * I, dtype=torch.int32, device=dev)

        def wgrad(a_src, b_src, seg, width, rows_b, n_groups, offsets, out):
            """out[g] = A_g^T B_g over segment g's rows: A = a_src rows, B = b_src rows (gathered
            through rows_b), both transposed into zero-padded blocks of `width` columns; on the FP8
            path quantised on the way (A 1x128 along the rows, B in 128x128 blocks)."""
            C = a_src.shape[1]
            if fp8:
                aq, as_ = L.moe_segment_transpose_fp8(a_src, seg, width)
                bq, bs = L.moe_segment_transpose_fp8(b_src, seg, width, src_rows=rows_b, block_scales=True)
                L.moe_grouped_gemm(aq.view(n_groups * C, width), bq, offsets, 0, n_groups, n_groups * C, out,
                                   a_scale=as_.view(n_groups * C, width // 128), w_scale=bs, k_offsets=seg)
                if keep:
                    extra.setdefault("wgrad_operands", []).append((aq.view(n_groups * C, width), as_, bq, bs))
            else:
                cols = torch.arange(0, (n_groups + 1) * width, width, dtype=torch.int32, device=dev)
                at = L.moe_segment_transpose(a_src, seg, cols, n_groups * width, width=width)
                bt = L.moe_segment_transpose(b_src, seg, cols, n_groups * width, src_rows=rows_b, width=width)
                L.moe_grouped_gemm(at.view(n_groups * C, width), bt, offsets, 0, n_groups, n_groups * C, out,
                                   k_offsets=seg)

        wgrad(dy, h, seg_r, kmax, None, N, g_d, dw2[:N].view(N * d, I))
        wgrad(dac, x, seg_r, kmax, st_, N, g_2i, dw13[:N].view(N * 2 * I, d))
        if kp_s > 0:
            wgrad(dy, h, seg_s, kp_s, None, 1, g_d[:2], dw2[N])
            wgrad(dac, x, seg_s, kp_s, st_, 1, g_2i[:2], dw13[N])
        else:
            dw2[N].zero_()
            dw13[N].zero_()
        dwr = L.moe_router_wgrad(x, st_, offs, du_row, N)
        res = {"dx": dx, "dw_router": dwr, "dw13": dw13, "dw2": dw2}
        if keep:
            res.update(du=du, du_row=du_row, dy=dy, dac=dac, dx_routed=dxr, dx_shared=dxs, **extra)
        return res
