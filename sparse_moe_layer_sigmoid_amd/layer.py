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
        if fp8:
            qw = L.fp8_quant_128x128_e8m0 if self.e8m0 else L.fp8_quant_128x128
            self.W13, self.W13_s = qw(W13)
            self.W2, self.W2_s = qw(W2)
        else:
            self.W13, self.W13_s = W13, None
            self.W2, self.W2_s = W2, None

    def forward(self, x, out_dtype=torch.bfloat16, update_bias: bool = False, gamma: float = 0.001,
                keep: bool = False):
        """x [T, d] bf16 -> out [T, d] (bf16 or f32).  With keep=True returns (out, buffers)."""
        T, d = x.shape
        N, K, I = self.N, self.top_k, self.I
        dev = x.device
        idx, gate, counts, _ = L.moe_route(x, self.w_router, self.bias, K, self.n_group, self.topk_group)
        offs, sorted_token, pair_pos = L.moe_permute(idx, N, 1)
        rows = T * (K + 1)
        if self.fp8:
            xq, xs = (L.fp8_quant_1x128_e8m0 if self.e8m0 else L.fp8_quant_1x128)(x)
            h = torch.empty((rows, I), dtype=torch.uint8, device=dev)
            hs = torch.empty((rows, I // 128), dtype=xs.dtype, device=dev)
            L.moe_grouped_gemm(xq, self.W13, offs, 0, N + 1, rows, h, a_scale=xs, a_rows=sorted_token,
                               w_scale=self.W13_s, swiglu=True, out_scale=hs)
        else:
            xq = xs = hs = None
            h = torch.empty((rows, I), dtype=torch.bfloat16, device=dev)
            L.moe_grouped_gemm(x, self.W13, offs, 0, N + 1, rows, h, a_rows=sorted_token, swiglu=True)
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
            return out, {"topk_idx": idx, "topk_gate": gate, "expert_counts": counts,
                         "expert_offsets": offs, "sorted_token": sorted_token, "pair_pos": pair_pos,
                         "xq": xq, "xs": xs, "h": h, "hs": hs, "y": y, "y_shared": ysh}
        return out
