"""The C ABI without a GPU: the library loads, exports every symbol moe.h declares, and
rejects bad arguments on the host before touching HIP (so these run anywhere the ROCm
runtime libraries are installed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from sparse_moe_layer_sigmoid_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return L


def test_header_declares_exactly_the_exports():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    declared = set(re.findall(r"\b(?:moe_status|size_t|int|const char\*)\s+(\w+)\s*\(", src))
    L = _lib()
    assert declared == set(L.EXPORTS)
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    L = _lib()
    assert L.lib().moe_abi_version() == 8
    assert L.status_str(0) == "MOE_OK" and L.status_str(5) == "MOE_ERR_WORKSPACE"


def _route(L, **kw):
    a = dict(x=16, w=16, bias=16, T=8, d=128, N=16, K=2, ng=1, tg=1, idx=16, gate=16, counts=16,
             scores=None, ws=16, wsb=1 << 20)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return L.lib().moe_route(p(a["x"]), p(a["w"]), p(a["bias"]), a["T"], a["d"], a["N"], a["K"], a["ng"],
                             a["tg"], p(a["idx"]), p(a["gate"]), p(a["counts"]), p(a["scores"]), p(a["ws"]),
                             a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(ws=None), 1), (dict(T=-1), 2), (dict(d=100), 2), (dict(N=300), 2),
    (dict(N=6), 2), (dict(K=0), 2), (dict(K=17), 2), (dict(ng=3), 2), (dict(ng=8, tg=9), 2),
    (dict(ng=8, tg=1, K=3), 2), (dict(ng=16, tg=2), 2), (dict(x=8), 4), (dict(wsb=4), 5),
])
def test_route_rejects(kw, code):
    L = _lib()
    assert _route(L, **kw) == code
    assert L.lib().moe_last_error().decode().startswith("moe_route")


def test_other_entry_points_reject():
    L = _lib()
    lib = L.lib()
    P = ctypes.c_void_p
    assert lib.moe_permute(None, 4, 2, 8, 1, P(16), P(16), P(16), P(16), 1 << 20, None) == 1
    assert lib.moe_permute(P(16), 4, 2, 8, 2, P(16), P(16), P(16), P(16), 1 << 20, None) == 2
    assert lib.moe_permute(P(16), 4, 9, 8, 1, P(16), P(16), P(16), P(16), 1 << 20, None) == 2
    assert lib.moe_permute(P(16), 4000, 2, 8, 1, P(16), P(16), P(16), P(16), 8, None) == 5
    assert lib.fp8_quant_1x128(P(16), 4, 100, 100, P(16), P(16), None) == 2
    assert lib.fp8_quant_1x128(P(16), 4, 128, 132, P(16), P(16), None) == 4
    assert lib.fp8_quant_128x128(P(16), 1, 128, 64, P(16), P(16), None) == 2
    assert lib.fp8_quant_1x128_e8m0(P(16), 4, 100, 100, P(16), P(16), None) == 2
    assert lib.fp8_quant_1x128_e8m0(None, 4, 128, 128, P(16), P(16), None) == 1
    assert lib.fp8_quant_128x128_e8m0(P(16), 1, 128, 64, P(16), P(16), None) == 2
    assert lib.fp8_quant_128x128_e8m0(P(8), 1, 128, 128, P(16), P(16), None) == 4
    assert lib.moe_combine(P(16), None, P(16), P(16), 4, 2, 12, P(16), 0, None) == 2
    assert lib.moe_combine(P(16), None, P(16), P(16), 4, 2, 16, P(16), 2, None) == 3
    assert lib.moe_bias_update(None, P(16), 8, 16, 0.001, None) == 1
    assert lib.moe_bias_update(P(16), P(16), 8, 16, float("nan"), None) == 2


def _gemm(L, **kw):
    d = dict(in_dtype=0, a=16, lda=256, w=16, group_offsets=16, first_group=0, n_groups=4, m_total=100,
             N=256, K=256, epilogue=0, out=16, out_dtype=1, ldo=256, ws=16, ws_bytes=256)
    d.update(kw)
    desc = L.MoeGemmDesc(**d)
    return L.lib().moe_grouped_gemm(ctypes.byref(desc), None)


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), 1), (dict(in_dtype=7), 3), (dict(epilogue=3), 3), (dict(out_dtype=9), 3),
    (dict(out_dtype=2), 3), (dict(epilogue=1, out_dtype=1), 3), (dict(n_groups=0), 2),
    (dict(K=96), 2), (dict(N=192), 2), (dict(epilogue=1, N=192, out_dtype=0), 2), (dict(in_dtype=2), 1),
    (dict(in_dtype=2, a_scale=16, w_scale=16, K=192), 2), (dict(lda=200), 4), (dict(ldo=100), 4),
    (dict(a=8), 4), (dict(m_total=-1), 2),
    (dict(tail_groups=5), 2), (dict(tail_groups=-1), 2), (dict(tail_groups=1, out_tail=16, ldo_tail=256), 3),
    (dict(tail_groups=1, out_dtype=0, ldo=256), 1), (dict(tail_groups=1, out_dtype=0, out_tail=8, ldo_tail=256), 4),
    (dict(tail_groups=1, out_dtype=0, out_tail=16, ldo_tail=100), 4),
    (dict(tail_groups=1, out_dtype=0, out_tail=16, ldo_tail=256, epilogue=1, N=512), 3),
    (dict(in_dtype=2, a_scale=16, w_scale=16, scale_fmt=5), 3),
    (dict(in_dtype=2, a_scale=16, w_scale=16, scale_fmt=1, K=256, lda=256), 2),
    (dict(ws=None), 5), (dict(ws_bytes=255), 5), (dict(ws=8), 5),
    (dict(k_offsets=16, out_dtype=0), 3), (dict(k_offsets=16, epilogue=1, N=512, out_dtype=0, ldo=256), 3),
    (dict(k_offsets=16, in_dtype=2, a_scale=16, w_scale=16, scale_fmt=1, K=512, lda=512), 3),
    (dict(out_preact=16, ldo_preact=256), 3),
    (dict(out_preact=8, ldo_preact=512, epilogue=1, N=512, out_dtype=0), 4),
    (dict(out_preact=16, ldo_preact=256, epilogue=1, N=512, out_dtype=0), 4),
    (dict(out_preact=16, ldo_preact=514, epilogue=1, N=512, out_dtype=0), 4),
    (dict(out_preact=16, ldo_preact=512, epilogue=1, N=512, out_dtype=2, in_dtype=2, a_scale=16, w_scale=16,
          out_scale=16, scale_fmt=1, K=512, lda=512), 3),
])
def test_gemm_rejects(kw, code):
    L = _lib()
    assert _gemm(L, **kw) == code, L.lib().moe_last_error()


def test_route_noalloc_rejects():
    """The allocation-free routing call checks its arguments like moe_route, and refuses T
    beyond its static scratch (1024 tokens) before anything else happens."""
    L = _lib()
    lib = L.lib()
    P = lambda n: ctypes.c_void_p(n)
    ok = dict(x=P(16), w=P(16), b=P(16), T=1024, d=7168, N=256, K=8, ng=1, tg=1, idx=P(16), gate=P(16), cnt=P(16))

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_route_noalloc(a["x"], a["w"], a["b"], a["T"], a["d"], a["N"], a["K"], a["ng"], a["tg"],
                                     a["idx"], a["gate"], a["cnt"], None, None)
    assert call(T=1025) == 2 and b"1024" in lib.moe_last_error()
    assert call(w=None) == 1 and call(d=100) == 2 and call(K=300) == 2 and call(x=P(8)) == 4
    assert lib.moe_last_error().decode().startswith("moe_route_noalloc")


def test_workspace_queries():
    L = _lib()
    lib = L.lib()
    assert lib.moe_route_workspace_size(4096, 256) > 0
    assert lib.moe_route_workspace_size(-1, 256) == 0
    assert lib.moe_permute_workspace_size(16384, 256) == 2 * 64 * 256 * 4
    assert lib.moe_grouped_gemm_workspace_size() == 256


def _rejects(lib, fn, args, code):
    st = getattr(lib, fn)(*args)
    assert st == code, (fn, args, st, lib.moe_last_error())
    assert lib.moe_last_error().decode().startswith(fn)


def test_backward_entry_points_reject():
    L = _lib()
    lib = L.lib()
    P = ctypes.c_void_p
    p = [P(16)] * 6
    # moe_combine_backward(d_out, y, idx, gate, scores, pair_pos, T, K, d, N, dy, du, du_row, dy_q, dy_scale,
    #                      stream)
    cb = lambda T=4, K=2, d=16, N=8, ptrs=None, dy=P(16), dq=None, ds=None: (
        *(ptrs or p), T, K, d, N, dy, P(16), P(16), dq, ds, None)
    _rejects(lib, "moe_combine_backward", cb(ptrs=[None] + p[1:]), 1)
    _rejects(lib, "moe_combine_backward", cb(T=-1), 2)
    _rejects(lib, "moe_combine_backward", cb(K=0), 2)
    _rejects(lib, "moe_combine_backward", cb(K=33, N=64), 2)
    _rejects(lib, "moe_combine_backward", cb(K=9, N=8), 2)
    _rejects(lib, "moe_combine_backward", cb(d=12), 2)
    _rejects(lib, "moe_combine_backward", cb(dy=P(8)), 4)
    _rejects(lib, "moe_combine_backward", cb(dq=P(16)), 1)                 # dy_q without dy_scale
    _rejects(lib, "moe_combine_backward", cb(d=64, dq=P(16), ds=P(16)), 2)  # E4M3 rows need d % 128 == 0
    _rejects(lib, "moe_combine_backward", cb(d=128, dq=P(4), ds=P(16)), 4)
    # moe_swiglu_backward(ac, dh, rows, inter, dac, dac_q, dac_scale, stream)
    _rejects(lib, "moe_swiglu_backward", (None, P(16), 4, 8, P(16), None, None, None), 1)
    _rejects(lib, "moe_swiglu_backward", (P(16), P(16), -1, 8, P(16), None, None, None), 2)
    _rejects(lib, "moe_swiglu_backward", (P(16), P(16), 4, 6, P(16), None, None, None), 2)
    _rejects(lib, "moe_swiglu_backward", (P(16), P(16), 4, 8, P(4), None, None, None), 4)
    _rejects(lib, "moe_swiglu_backward", (P(16), P(16), 4, 8, P(16), None, P(16), None), 1)
    _rejects(lib, "moe_swiglu_backward", (P(16), P(16), 4, 64, P(16), P(16), P(16), None), 2)
    _rejects(lib, "moe_swiglu_backward", (P(16), P(16), 4, 128, P(16), P(2), P(16), None), 4)
    # moe_segment_transpose(src, ld_src, src_rows, seg_offsets, dst_cols, n_seg, cols, total_cols, dst, ld_dst,
    #                       seg_stride, stream)
    st = lambda src=P(16), ld_src=64, n=2, cols=64, total=128, dst=P(16), ld_dst=128, ss=0: (
        src, ld_src, None, P(16), P(16), n, cols, total, dst, ld_dst, ss, None)
    _rejects(lib, "moe_segment_transpose", st(src=None), 1)
    _rejects(lib, "moe_segment_transpose", st(n=0), 2)
    _rejects(lib, "moe_segment_transpose", st(cols=60), 2)
    _rejects(lib, "moe_segment_transpose", st(total=100), 2)
    _rejects(lib, "moe_segment_transpose", st(ss=4), 4)
    _rejects(lib, "moe_segment_transpose", st(ld_src=32), 4)
    _rejects(lib, "moe_segment_transpose", st(ld_dst=64), 4)
    _rejects(lib, "moe_segment_transpose", st(dst=P(8)), 4)
    # moe_segment_transpose_fp8(src, ld_src, src_rows, seg_offsets, n_seg, cols, width, block_scales, q, scale,
    #                           stream)
    sf = lambda src=P(16), ld_src=128, n=2, cols=128, width=128, bs=0, q=P(16), sc=P(16): (
        src, ld_src, None, P(16), n, cols, width, bs, q, sc, None)
    _rejects(lib, "moe_segment_transpose_fp8", sf(q=None), 1)
    _rejects(lib, "moe_segment_transpose_fp8", sf(n=0), 2)
    _rejects(lib, "moe_segment_transpose_fp8", sf(cols=64), 2)
    _rejects(lib, "moe_segment_transpose_fp8", sf(width=192), 2)
    _rejects(lib, "moe_segment_transpose_fp8", sf(bs=2), 2)
    _rejects(lib, "moe_segment_transpose_fp8", sf(ld_src=64), 4)
    _rejects(lib, "moe_segment_transpose_fp8", sf(src=P(8)), 4)
    _rejects(lib, "moe_segment_transpose_fp8", sf(q=P(4)), 4)
    # moe_router_wgrad(x, sorted_token, expert_offsets, du_row, n_experts, d, dw_router, stream)
    _rejects(lib, "moe_router_wgrad", (P(16), P(16), None, P(16), 8, 16, P(16), None), 1)
    _rejects(lib, "moe_router_wgrad", (P(16), P(16), P(16), P(16), 0, 16, P(16), None), 2)
    _rejects(lib, "moe_router_wgrad", (P(16), P(16), P(16), P(16), 8, 12, P(16), None), 2)
    _rejects(lib, "moe_router_wgrad", (P(8), P(16), P(16), P(16), 8, 16, P(16), None), 4)
    # fp8_dequant_1x128(q, scale, rows, cols, out, stream)
    _rejects(lib, "fp8_dequant_1x128", (None, P(16), 4, 128, P(16), None), 1)
    _rejects(lib, "fp8_dequant_1x128", (P(16), P(16), 4, 100, P(16), None), 2)
    _rejects(lib, "fp8_dequant_1x128", (P(16), P(16), -1, 128, P(16), None), 2)
    _rejects(lib, "fp8_dequant_1x128", (P(4), P(16), 4, 128, P(16), None), 4)


@pytest.mark.parametrize("kw,code", [(dict(ldw=100), 4), (dict(ldw=260), 4)])
def test_gemm_rejects_weight_stride(kw, code):
    L = _lib()
    assert _gemm(L, **kw) == code, L.lib().moe_last_error()
    assert L.lib().moe_last_error().decode().startswith("moe_grouped_gemm")


def test_no_cpu_fallback(monkeypatch):
    """Without libmoe.so the binding raises instead of computing anything, and CPU tensors are
    refused before any library call: nothing on the product path runs on the host."""
    import torch

    from sparse_moe_layer_sigmoid_amd import _lib as L
    monkeypatch.setattr(L, "_LIB", None)
    monkeypatch.setattr(L, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libmoe.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        L.lib()
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="GPU tensor"):
        L.fp8_quant_1x128(x)
    with pytest.raises(TypeError, match="GPU tensor"):
        L.moe_combine(x, None, torch.zeros((2, 2), dtype=torch.int32), torch.zeros((2, 2)))


def test_package_does_not_import_the_oracle():
    """The library package and its layer never load the CPU oracle (test infrastructure only)."""
    import subprocess
    import sys
    code = ("import sys; import sparse_moe_layer_sigmoid_amd, sparse_moe_layer_sigmoid_amd.layer, "
            "sparse_moe_layer_sigmoid_amd._lib, sparse_moe_layer_sigmoid_amd.inputs; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr


def test_ceilings_library_exports_and_rejects():
    """The ceiling micro-benchmarks (measurement code, their own library): every probe is
    exported and refuses bad arguments on the host, before any launch."""
    path = os.path.join(ROOT, "sparse_moe_layer_sigmoid_amd", "libmoe_ceilings.so")
    if not os.path.exists(path):
        pytest.skip("libmoe_ceilings.so not built")
    lib = ctypes.CDLL(path)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
    lib.moe_ceil_hbm_read.argtypes = [P, S, P, S, I32, P]
    lib.moe_ceil_dma_read.argtypes = [P, I64, I32, P, S, I32, P]
    lib.moe_ceil_dma_resident.argtypes = [I32, P, I32, I32, I32, P, P, S, I32, P]
    lib.moe_ceil_dma_read_ring.argtypes = [I32, P, I64, I32, P, S, I32, P]
    lib.moe_ceil_lds_read.argtypes = [I32, I32, P, P, S, I32, P]
    lib.moe_ceil_mfma.argtypes = [I32, I32, P, P, S, I32, P]
    lib.moe_ceil_valu.argtypes = [I32, P, P, S, I32, P]
    big = 1 << 20
    assert lib.moe_ceil_hbm_read(16, 1000, 16, big, 4, None) == -1  # bytes not a multiple of 16
    assert lib.moe_ceil_hbm_read(16, 1024, 16, 100, 4, None) == -1  # sink too small
    assert lib.moe_ceil_dma_read(16, 300, 128, 16, big, 4, None) == -1  # rows not a multiple of 256
    assert lib.moe_ceil_dma_read(16, 256, 100, 16, big, 4, None) == -1  # row bytes not a multiple of 128
    assert lib.moe_ceil_dma_read_ring(6, 16, 256, 128, 16, big, 4, None) == -1  # slots
    assert lib.moe_ceil_dma_read_ring(1, 16, 256, 128, 16, big, 4, None) == -1  # slots
    assert lib.moe_ceil_dma_read_ring(3, 16, 300, 128, 16, big, 4, None) == -1  # rows not a multiple of 256
    assert lib.moe_ceil_dma_resident(2, 16, 1, 128, 3, 16, 16, big, 4, None) == -1  # mode
    assert lib.moe_ceil_dma_resident(0, 16, 1, 100, 3, 16, 16, big, 4, None) == -1  # row bytes not a multiple of 128
    assert lib.moe_ceil_dma_resident(0, 16, 1, 128, 4, 16, 16, big, 4, None) == -1  # steps not a multiple of 3
    assert lib.moe_ceil_dma_resident(0, 16, 0, 128, 3, 16, 16, big, 4, None) == -1  # no row block
    assert lib.moe_ceil_dma_resident(0, 16, 1, 128, 3, None, 16, big, 4, None) == -1  # cycles
    assert lib.moe_ceil_lds_read(4, 16, 16, 16, big, 4, None) == -1  # width
    assert lib.moe_ceil_lds_read(16, 20, 16, 16, big, 4, None) == -1  # iters not a multiple of 16
    assert lib.moe_ceil_mfma(3, 16, 16, 16, big, 4, None) == -1  # kind
    assert lib.moe_ceil_mfma(0, 16, None, 16, big, 4, None) == -1  # cycles
    assert lib.moe_ceil_valu(0, 16, 16, big, 4, None) == -1  # iters
