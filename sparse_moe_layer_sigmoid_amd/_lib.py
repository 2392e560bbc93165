"""ctypes binding of libmoe.so: the C-ABI entry points under the same names.

Argument marshalling only (tensor -> pointer, shape -> int, output allocation, the current
HIP stream); every step of the layer runs in the library's HIP kernels.  There is no
fallback: if the library is not built, or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(7)
MOE_BF16, MOE_F32, MOE_FP8_E4M3 = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SWIGLU = 0, 1
MOE_SCALE_F32, MOE_SCALE_E8M0 = 0, 1

EXPORTS = (
    "moe_status_str", "moe_last_error", "moe_abi_version",
    "moe_route_workspace_size", "moe_route", "moe_route_noalloc",
    "moe_permute_workspace_size", "moe_permute",
    "fp8_quant_1x128", "fp8_quant_128x128", "fp8_quant_1x128_e8m0", "fp8_quant_128x128_e8m0", "fp8_dequant_1x128",
    "moe_grouped_gemm_workspace_size", "moe_grouped_gemm", "moe_combine", "moe_bias_update",
    "moe_combine_backward", "moe_swiglu_backward", "moe_segment_transpose", "moe_segment_transpose_fp8",
    "moe_router_wgrad",
)

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f = ctypes.c_float


class MoeGemmDesc(ctypes.Structure):
    _fields_ = [
        ("in_dtype", _i), ("a", _p), ("a_scale", _p), ("a_rows", _p), ("lda", _i64),
        ("w", _p), ("w_scale", _p), ("group_offsets", _p), ("first_group", _i),
        ("n_groups", _i), ("m_total", _i64), ("N", _i), ("K", _i), ("epilogue", _i),
        ("out", _p), ("out_dtype", _i), ("ldo", _i64), ("out_scale", _p),
        ("tail_groups", _i), ("out_tail", _p), ("ldo_tail", _i64), ("scale_fmt", _i), ("ldw", _i64),
        ("ws", _p), ("ws_bytes", _sz), ("k_offsets", _p), ("out_preact", _p), ("ldo_preact", _i64),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed: {status_str(status)}: {detail}")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_moe_layer_sigmoid_amd.build`"
                " (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [_i]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_abi_version.restype = _i
        L.moe_route_workspace_size.restype = _sz
        L.moe_route_workspace_size.argtypes = [_i, _i]
        L.moe_route.restype = _i
        L.moe_route.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]
        L.moe_route_noalloc.restype = _i
        L.moe_route_noalloc.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p]
        L.moe_permute_workspace_size.restype = _sz
        L.moe_permute_workspace_size.argtypes = [_i, _i]
        L.moe_permute.restype = _i
        L.moe_permute.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]
        L.fp8_quant_1x128.restype = _i
        L.fp8_quant_1x128.argtypes = [_p, _i, _i, _i64, _p, _p, _p]
        L.fp8_quant_128x128.restype = _i
        L.fp8_quant_128x128.argtypes = [_p, _i, _i, _i, _p, _p, _p]
        L.fp8_quant_1x128_e8m0.restype = _i
        L.fp8_quant_1x128_e8m0.argtypes = [_p, _i, _i, _i64, _p, _p, _p]
        L.fp8_quant_128x128_e8m0.restype = _i
        L.fp8_quant_128x128_e8m0.argtypes = [_p, _i, _i, _i, _p, _p, _p]
        L.fp8_dequant_1x128.restype = _i
        L.fp8_dequant_1x128.argtypes = [_p, _p, _i, _i, _p, _p]
        L.moe_grouped_gemm_workspace_size.restype = _sz
        L.moe_grouped_gemm_workspace_size.argtypes = []
        L.moe_grouped_gemm.restype = _i
        L.moe_grouped_gemm.argtypes = [ctypes.POINTER(MoeGemmDesc), _p]
        L.moe_combine.restype = _i
        L.moe_combine.argtypes = [_p, _p, _p, _p, _i, _i, _i, _p, _i, _p]
        L.moe_bias_update.restype = _i
        L.moe_bias_update.argtypes = [_p, _p, _i, _i64, _f, _p]
        L.moe_combine_backward.restype = _i
        L.moe_combine_backward.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p]
        L.moe_swiglu_backward.restype = _i
        L.moe_swiglu_backward.argtypes = [_p, _p, _i64, _i, _p, _p, _p, _p]
        L.moe_segment_transpose.restype = _i
        L.moe_segment_transpose.argtypes = [_p, _i64, _p, _p, _p, _i, _i, _i, _p, _i64, _i64, _p]
        L.moe_segment_transpose_fp8.restype = _i
        L.moe_segment_transpose_fp8.argtypes = [_p, _i64, _p, _p, _i, _i, _i, _i, _p, _p, _p]
        L.moe_router_wgrad.restype = _i
        L.moe_router_wgrad.argtypes = [_p, _p, _p, _p, _i, _i, _p, _p]
        _LIB = L
    return _LIB


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name: str, contiguous: bool = True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ----------------------------------------------------------------------------- entry points


def moe_route(x, w_router, bias, top_k: int, n_group: int = 1, topk_group: int = 1,
              want_scores: bool = False, out=None):
    """Returns (topk_idx [T,K] int32, topk_gate [T,K] f32, expert_counts [N] int32, scores|None)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    _dev(bias, torch.float32, "bias")
    T, d = x.shape
    N = w_router.shape[0]
    dev = x.device
    if out is None:
        out = {}
    idx = out.get("topk_idx") if "topk_idx" in out else torch.empty((T, top_k), dtype=torch.int32, device=dev)
    gate = out.get("topk_gate") if "topk_gate" in out else torch.empty((T, top_k), dtype=torch.float32, device=dev)
    counts = out.get("expert_counts") if "expert_counts" in out else torch.empty(N, dtype=torch.int32, device=dev)
    scores = torch.empty((T, N), dtype=torch.float32, device=dev) if want_scores else None
    wsb = lib().moe_route_workspace_size(T, N)
    ws = out.get("ws_route") if "ws_route" in out else torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    st = lib().moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, d, N, top_k, n_group, topk_group,
                         _ptr(idx), _ptr(gate), _ptr(counts), _ptr(scores), _ptr(ws), ws.numel(), _stream(x))
    _check("moe_route", st)
    return idx, gate, counts, scores


def moe_route_noalloc(x, w_router, bias, top_k: int, n_group: int = 1, topk_group: int = 1, out=None):
    """moe_route with the library's static scratch instead of a workspace (T <= 1024); the
    outputs are given in `out` (topk_idx, topk_gate, expert_counts, optional scores) or
    allocated here.  Returns (topk_idx, topk_gate, expert_counts, scores|None)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    _dev(bias, torch.float32, "bias")
    T, d = x.shape
    N = w_router.shape[0]
    dev = x.device
    out = out or {}
    idx = out["topk_idx"] if "topk_idx" in out else torch.empty((T, top_k), dtype=torch.int32, device=dev)
    gate = out["topk_gate"] if "topk_gate" in out else torch.empty((T, top_k), dtype=torch.float32, device=dev)
    counts = out["expert_counts"] if "expert_counts" in out else torch.empty(N, dtype=torch.int32, device=dev)
    scores = out.get("scores")
    st = lib().moe_route_noalloc(_ptr(x), _ptr(w_router), _ptr(bias), T, d, N, top_k, n_group, topk_group,
                                 _ptr(idx), _ptr(gate), _ptr(counts), _ptr(scores), _stream(x))
    _check("moe_route_noalloc", st)
    return idx, gate, counts, scores


def moe_permute(topk_idx, n_experts: int, n_shared: int = 1, out=None):
    """Returns (expert_offsets [N+n_shared+1], sorted_token [T*(K+n_shared)], pair_pos [T,K])."""
    _dev(topk_idx, torch.int32, "topk_idx")
    T, K = topk_idx.shape
    dev = topk_idx.device
    out = out or {}
    offs = out["expert_offsets"] if "expert_offsets" in out else torch.empty(n_experts + n_shared + 1, dtype=torch.int32, device=dev)
    st_ = out["sorted_token"] if "sorted_token" in out else torch.empty(T * (K + n_shared), dtype=torch.int32, device=dev)
    pp = out["pair_pos"] if "pair_pos" in out else torch.empty((T, K), dtype=torch.int32, device=dev)
    wsb = lib().moe_permute_workspace_size(T, n_experts)
    ws = out["ws_permute"] if "ws_permute" in out else torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    st = lib().moe_permute(_ptr(topk_idx), T, K, n_experts, n_shared, _ptr(offs), _ptr(st_), _ptr(pp),
                           _ptr(ws), ws.numel(), _stream(topk_idx))
    _check("moe_permute", st)
    return offs, st_, pp


def _quant_1x128(fn, sdtype, x, q, scale):
    _dev(x, torch.bfloat16, "x", contiguous=False)
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((rows, cols // 128), dtype=sdtype, device=x.device) if scale is None else scale
    st = getattr(lib(), fn)(_ptr(x), rows, cols, x.stride(0), _ptr(q), _ptr(scale), _stream(x))
    _check(fn, st)
    return q, scale


def _quant_128x128(fn, sdtype, w):
    _dev(w, torch.bfloat16, "w")
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    m, n, k = w3.shape
    q = torch.empty((m, n, k), dtype=torch.uint8, device=w.device)
    s = torch.empty((m, n // 128, k // 128), dtype=sdtype, device=w.device)
    st = getattr(lib(), fn)(_ptr(w3), m, n, k, _ptr(q), _ptr(s), _stream(w))
    _check(fn, st)
    return (q[0], s[0]) if squeeze else (q, s)


def fp8_quant_1x128(x, q=None, scale=None):
    """x [rows, cols] bf16 (row stride may exceed cols) -> (q uint8 [rows, cols], scale f32 [rows, cols/128])."""
    return _quant_1x128("fp8_quant_1x128", torch.float32, x, q, scale)


def fp8_quant_128x128(w):
    """w [n_mats, n, k] (or [n, k]) bf16 -> (q uint8 like w, scale f32 [n_mats, n/128, k/128])."""
    return _quant_128x128("fp8_quant_128x128", torch.float32, w)


def fp8_quant_1x128_e8m0(x, q=None, scale=None):
    """As fp8_quant_1x128 with power-of-two scales: scale = E8M0 codes, uint8 [rows, cols/128]."""
    return _quant_1x128("fp8_quant_1x128_e8m0", torch.uint8, x, q, scale)


def fp8_dequant_1x128(q, scale, out=None):
    """q uint8 [rows, cols] E4M3 + scale f32 [rows, cols/128] -> bf16 [rows, cols] (RNE of q * s)."""
    rows, cols = q.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=q.device)
    st = lib().fp8_dequant_1x128(_ptr(q), _ptr(scale), rows, cols, _ptr(out), _stream(q))
    _check("fp8_dequant_1x128", st)
    return out


def fp8_quant_128x128_e8m0(w):
    """As fp8_quant_128x128 with power-of-two scales: scale = E8M0 codes, uint8 [n_mats, n/128, k/128]."""
    return _quant_128x128("fp8_quant_128x128_e8m0", torch.uint8, w)


_DT = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32, torch.uint8: MOE_FP8_E4M3}

_GEMM_WS = {}


def gemm_workspace(device, stream=None) -> torch.Tensor:
    """The zero-filled moe_grouped_gemm workspace of one stream (made on first use and kept).
    Launches on one stream are ordered, so they may share it; every launch leaves it zeroed."""
    device = torch.device(device)
    stream = torch.cuda.current_stream(device) if stream is None else stream
    key = (device.index, stream.cuda_stream)
    ws = _GEMM_WS.get(key)
    if ws is None:
        ws = torch.zeros(lib().moe_grouped_gemm_workspace_size(), dtype=torch.uint8, device=device)
        torch.cuda.current_stream(device).synchronize()  # the zero fill precedes any use on `stream`
        _GEMM_WS[key] = ws
    return ws


def moe_grouped_gemm(a, w, group_offsets, first_group: int, n_groups: int, m_total: int, out,
                     a_scale=None, a_rows=None, w_scale=None, swiglu: bool = False, out_scale=None,
                     out_tail=None, tail_groups: int = 0, ws=None, k_offsets=None, out_preact=None):
    """out[r - off[first_group]] = epilogue(A[a_rows[r] or r] . W[g]^T) for each sorted row r
    of group g.  a: bf16 or uint8 (E4M3) [*, K]; w: same dtype [G, N, K]; out: bf16 / f32 /
    uint8 (E4M3, needs out_scale).  With tail_groups > 0 the last tail_groups groups write
    f32 rows to out_tail instead (row r -> r - off[first_group + n_groups - tail_groups]).
    FP8 scales are f32, or E8M0 codes when they are uint8 tensors (all of them alike).
    ws: the launch's workspace (default: the current stream's, see gemm_workspace).
    k_offsets: int32 offsets whose differences give each group's reduction length (ragged K,
    f32 output only; the K columns past a group's length rounded up to a K step are not read).
    out_preact: with swiglu, an f32 [rows, N] tensor that also receives the gate | up products."""
    fp8 = a.dtype == torch.uint8
    scales = [s for s in (a_scale, w_scale, out_scale) if s is not None]
    e8 = fp8 and any(s.dtype == torch.uint8 for s in scales)
    if e8 and any(s.dtype != torch.uint8 for s in scales):
        raise TypeError("FP8 scales must all be float32 or all uint8 (E8M0)")
    if w.dtype != a.dtype:
        raise TypeError("a and w must share a dtype")
    for t, nm in ((a, "a"), (w, "w"), (group_offsets, "group_offsets"), (out, "out")):
        if not t.is_cuda:
            raise TypeError(f"{nm} must be a GPU tensor")
    if k_offsets is not None:
        _dev(k_offsets, torch.int32, "k_offsets")
        if k_offsets.numel() < first_group + n_groups + 1:
            raise ValueError("k_offsets needs first_group + n_groups + 1 entries")
    if out_preact is not None:
        _dev(out_preact, torch.float32, "out_preact", contiguous=False)
        if out_preact.stride(-1) != 1:
            raise ValueError("rows of out_preact must be contiguous")
    if tail_groups:
        _dev(out_tail, torch.float32, "out_tail", contiguous=False)
        if out_tail.stride(-1) != 1:
            raise ValueError("rows of out_tail must be contiguous")
    G, N, K = w.shape
    if a.stride(-1) != 1 or out.stride(-1) != 1 or w.stride(-1) != 1 or (G > 1 and w.stride(0) != N * w.stride(1)):
        raise ValueError("rows of a/out/w must be contiguous and the W[g] packed (stride N * ldw)")
    ldw = w.stride(1)
    if ws is None:
        ws = gemm_workspace(a.device)
    _dev(ws, torch.uint8, "ws")
    desc = MoeGemmDesc(
        in_dtype=MOE_FP8_E4M3 if fp8 else MOE_BF16, a=a.data_ptr(),
        a_scale=a_scale.data_ptr() if a_scale is not None else None,
        a_rows=a_rows.data_ptr() if a_rows is not None else None, lda=a.stride(0),
        w=w.data_ptr(), w_scale=w_scale.data_ptr() if w_scale is not None else None,
        group_offsets=group_offsets.data_ptr(), first_group=first_group, n_groups=n_groups,
        m_total=m_total, N=N, K=K, epilogue=MOE_EPI_SWIGLU if swiglu else MOE_EPI_NONE,
        out=out.data_ptr(), out_dtype=_DT[out.dtype], ldo=out.stride(0),
        out_scale=out_scale.data_ptr() if out_scale is not None else None,
        tail_groups=tail_groups, out_tail=out_tail.data_ptr() if tail_groups else None,
        ldo_tail=out_tail.stride(0) if tail_groups else 0,
        scale_fmt=MOE_SCALE_E8M0 if e8 else MOE_SCALE_F32, ldw=0 if ldw == K else ldw,
        ws=ws.data_ptr(), ws_bytes=ws.numel(),
        k_offsets=k_offsets.data_ptr() if k_offsets is not None else None,
        out_preact=out_preact.data_ptr() if out_preact is not None else None,
        ldo_preact=out_preact.stride(0) if out_preact is not None else 0)
    st = lib().moe_grouped_gemm(ctypes.byref(desc), _stream(a))
    _check("moe_grouped_gemm", st)
    return out


def moe_combine(y_routed, y_shared, pair_pos, topk_gate, out_dtype=torch.bfloat16, out=None):
    _dev(y_routed, torch.bfloat16, "y_routed")
    _dev(pair_pos, torch.int32, "pair_pos")
    _dev(topk_gate, torch.float32, "topk_gate")
    if y_shared is not None:
        _dev(y_shared, torch.float32, "y_shared")
    T, K = pair_pos.shape
    d = y_routed.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=y_routed.device)
    st = lib().moe_combine(_ptr(y_routed), _ptr(y_shared), _ptr(pair_pos), _ptr(topk_gate), T, K, d,
                           _ptr(out), _DT[out.dtype], _stream(y_routed))
    _check("moe_combine", st)
    return out


def moe_bias_update(bias, expert_counts, total_assignments: int, gamma: float):
    _dev(bias, torch.float32, "bias")
    _dev(expert_counts, torch.int32, "expert_counts")
    st = lib().moe_bias_update(_ptr(bias), _ptr(expert_counts), bias.numel(), int(total_assignments),
                               float(gamma), _stream(bias))
    _check("moe_bias_update", st)
    return bias


# ----------------------------------------------------------------------------- backward


def moe_combine_backward(d_out, y_routed, topk_idx, topk_gate, scores, pair_pos, out=None, fp8: bool = False):
    """-> (dy bf16 [T*(K+1), d], du f32 [T, K], du_row f32 [T*K]); with fp8=True also
    (dy_q u8 [T*(K+1), d], dy_scale f32 [T*(K+1), d/128]), the 1x128 E4M3 form of dy."""
    _dev(d_out, torch.bfloat16, "d_out")
    _dev(y_routed, torch.bfloat16, "y_routed")
    _dev(scores, torch.float32, "scores")
    T, K = topk_idx.shape
    d = d_out.shape[1]
    dev = d_out.device
    out = out or {}
    dy = out.get("dy", None)
    if dy is None:
        dy = torch.empty((T * (K + 1), d), dtype=torch.bfloat16, device=dev)
    du = torch.empty((T, K), dtype=torch.float32, device=dev)
    du_row = torch.empty(T * K, dtype=torch.float32, device=dev)
    dyq = dys = None
    if fp8:
        dyq = torch.empty((T * (K + 1), d), dtype=torch.uint8, device=dev)
        dys = torch.empty((T * (K + 1), d // 128), dtype=torch.float32, device=dev)
    st = lib().moe_combine_backward(_ptr(d_out), _ptr(y_routed), _ptr(topk_idx), _ptr(topk_gate), _ptr(scores),
                                    _ptr(pair_pos), T, K, d, scores.shape[1], _ptr(dy), _ptr(du), _ptr(du_row),
                                    _ptr(dyq), _ptr(dys), _stream(d_out))
    _check("moe_combine_backward", st)
    return (dy, du, du_row, dyq, dys) if fp8 else (dy, du, du_row)


def moe_swiglu_backward(ac, dh, dac=None, fp8: bool = False):
    """ac f32 [rows, 2I] (a | c), dh f32 [rows, I] -> dac bf16 [rows, 2I] (da | dc); with fp8=True
    -> (dac, dac_q u8 [rows, 2I], dac_scale f32 [rows, 2I/128]), its 1x128 E4M3 form too."""
    _dev(ac, torch.float32, "ac")
    _dev(dh, torch.float32, "dh")
    rows, I = dh.shape
    if dac is None:
        dac = torch.empty((rows, 2 * I), dtype=torch.bfloat16, device=dh.device)
    dq = ds = None
    if fp8:
        dq = torch.empty((rows, 2 * I), dtype=torch.uint8, device=dh.device)
        ds = torch.empty((rows, 2 * I // 128), dtype=torch.float32, device=dh.device)
    st = lib().moe_swiglu_backward(_ptr(ac), _ptr(dh), rows, I, _ptr(dac), _ptr(dq), _ptr(ds), _stream(dh))
    _check("moe_swiglu_backward", st)
    return (dac, dq, ds) if fp8 else dac


def moe_segment_transpose(src, seg_offsets, dst_cols, total_cols: int, src_rows=None, dst=None, width: int = 0):
    """Row segments of src [*, C] (gathered through src_rows if given) -> zero-padded column
    blocks of dst [C, total_cols] bf16; with width > 0 (and dst_cols = g * width) separate
    blocks dst [G, C, width]."""
    _dev(src, torch.bfloat16, "src", contiguous=False)
    if src.stride(-1) != 1:
        raise ValueError("rows of src must be contiguous")
    C = src.shape[1]
    G = seg_offsets.numel() - 1
    if dst is None:
        shape = (G, C, width) if width else (C, total_cols)
        dst = torch.empty(shape, dtype=torch.bfloat16, device=src.device)
    ld = width if width else dst.stride(0)
    st = lib().moe_segment_transpose(_ptr(src), src.stride(0), _ptr(src_rows), _ptr(seg_offsets), _ptr(dst_cols), G,
                                     C, total_cols, _ptr(dst), ld, C * width if width else 0, _stream(src))
    _check("moe_segment_transpose", st)
    return dst


def moe_segment_transpose_fp8(src, seg_offsets, width: int, src_rows=None, block_scales: bool = False):
    """Row segments of src [*, C] (gathered through src_rows if given) -> E4M3 blocks q [G, C, width]
    (zero-padded past each segment) with 1x128 scales along each block row ([G * C, width / 128],
    block_scales=False) or one scale per 128x128 block ([G, C / 128, width / 128])."""
    _dev(src, torch.bfloat16, "src", contiguous=False)
    if src.stride(-1) != 1:
        raise ValueError("rows of src must be contiguous")
    C = src.shape[1]
    G = seg_offsets.numel() - 1
    q = torch.empty((G, C, width), dtype=torch.uint8, device=src.device)
    if block_scales:
        scale = torch.empty((G, C // 128, width // 128), dtype=torch.float32, device=src.device)
    else:
        scale = torch.empty((G * C, width // 128), dtype=torch.float32, device=src.device)
    st = lib().moe_segment_transpose_fp8(_ptr(src), src.stride(0), _ptr(src_rows), _ptr(seg_offsets), G, C, width,
                                         1 if block_scales else 0, _ptr(q), _ptr(scale), _stream(src))
    _check("moe_segment_transpose_fp8", st)
    return q, scale


def moe_router_wgrad(x, sorted_token, expert_offsets, du_row, n_experts: int, out=None):
    _dev(x, torch.bfloat16, "x")
    d = x.shape[1]
    if out is None:
        out = torch.empty((n_experts, d), dtype=torch.float32, device=x.device)
    st = lib().moe_router_wgrad(_ptr(x), _ptr(sorted_token), _ptr(expert_offsets), _ptr(du_row), n_experts, d,
                                _ptr(out), _stream(x))
    _check("moe_router_wgrad", st)
    return out
