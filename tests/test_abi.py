"""C ABI checks that need no GPU: the library loads, exports every function that
include/fp8q.h declares, and rejects invalid arguments on the host before touching
the device (nothing is launched in these tests)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import fp8_block_scaled_weight_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")
A16 = 0x10000  # 16-byte-aligned fake address: never dereferenced, validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8q_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("fp8q_quant_weight_blk128", "fp8q_quant_act_g128", "fp8q_gemm_w8a8_blkscaled",
              "fp8q_grouped_gemm_w8a8", "fp8q_kv_quant"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = fq.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (fp8q_\w+)", out))
    assert set(_declared()) <= exported
    assert set(fq.EXPORTED) == set(_declared())


def test_version_and_status_strings():
    assert fq.abi_version() == 1
    for code, name in ((0, "FP8Q_OK"), (1, "FP8Q_ERR_NULL"), (2, "FP8Q_ERR_SHAPE"), (3, "FP8Q_ERR_STRIDE"),
                       (4, "FP8Q_ERR_ALIGN"), (5, "FP8Q_ERR_LAUNCH"), (6, "FP8Q_ERR_UNSUPPORTED"),
                       (7, "FP8Q_ERR_PRECONDITION")):
        assert fq.status_string(code) == name


def _act(**kw):
    a = dict(x=A16, m=4, k=256, ld_x=256, q=A16, ld_q=256, s=A16, ld_s=4, stream=None)
    a.update(kw)
    return fq.lib().fp8q_quant_act_g128(a["x"], a["m"], a["k"], a["ld_x"], a["q"], a["ld_q"], a["s"],
                                        a["ld_s"], a["stream"])


def test_act_quant_validation():
    assert _act(m=-1) == fq.FP8Q_ERR_SHAPE
    assert _act(k=100, ld_x=100, ld_q=100) == fq.FP8Q_ERR_SHAPE
    assert _act(x=None) == fq.FP8Q_ERR_NULL
    assert _act(s=None) == fq.FP8Q_ERR_NULL
    assert _act(ld_x=128) == fq.FP8Q_ERR_STRIDE
    assert _act(ld_s=3) == fq.FP8Q_ERR_STRIDE
    assert _act(x=A16 + 2) == fq.FP8Q_ERR_ALIGN
    assert _act(ld_q=264) == fq.FP8Q_ERR_ALIGN
    assert _act(ld_x=260) == fq.FP8Q_ERR_ALIGN
    assert "multiple of 128" in fq.last_error() or fq.last_error()


def _gemm(**kw):
    a = dict(a=A16, ld_a=256, a_s=A16, ld_as=8, b=A16, ld_b=256, b_s=A16, y=A16, ld_y=128, m=8, n=128, k=256)
    a.update(kw)
    return fq.lib().fp8q_gemm_w8a8_blkscaled(a["a"], a["ld_a"], a["a_s"], a["ld_as"], a["b"], a["ld_b"],
                                             a["b_s"], a["y"], a["ld_y"], a["m"], a["n"], a["k"], None)


def test_gemm_validation():
    assert _gemm(n=100) == fq.FP8Q_ERR_SHAPE
    assert _gemm(k=0) == fq.FP8Q_ERR_SHAPE
    assert _gemm(m=-3) == fq.FP8Q_ERR_SHAPE
    assert _gemm(b=None) == fq.FP8Q_ERR_NULL
    assert _gemm(ld_as=7) == fq.FP8Q_ERR_STRIDE
    assert _gemm(ld_y=64) == fq.FP8Q_ERR_STRIDE
    assert _gemm(ld_a=272, a=A16 + 8) == fq.FP8Q_ERR_ALIGN
    assert _gemm(ld_y=132) == fq.FP8Q_ERR_ALIGN
    # operands are addressed through 32-bit buffer ranges: at most 2 GiB each
    assert _gemm(m=(1 << 31) // 256 + 1, ld_as=(1 << 31) // 256 + 1) == fq.FP8Q_ERR_SHAPE
    big_n = (1 << 31) // 256 + 128
    assert _gemm(n=big_n, ld_y=big_n) == fq.FP8Q_ERR_SHAPE


# The token scales a_s are addressed as one [k/128][ld_as] fp32 range: a padded ld_as
# whose whole span 4 * ld_as * k/128 passes 2 GiB is rejected, though one row of it fits.
_LD_AS_WRAP = (1 << 31) // (4 * 64) + 16   # k = 8192: 64 scale rows of 4 * ld_as bytes


def test_gemm_rejects_a_token_scale_span_beyond_2gib():
    assert 4 * _LD_AS_WRAP < (1 << 31) < 4 * _LD_AS_WRAP * 64
    for f in (fq.lib().fp8q_gemm_w8a8_blkscaled, fq.lib().fp8q_gemm_w8a8_ue8m0):
        assert f(A16, 8192, A16, _LD_AS_WRAP, A16, 8192, A16, A16, 128, 8, 128, 8192, None) == fq.FP8Q_ERR_SHAPE
        assert "a_s" in fq.last_error()
        # the same call with a compact ld_as passes validation (no device here)
        assert f(A16, 8192, A16, 8, A16, 8192, A16, A16, 128, 8, 128, 8192, None) == fq.FP8Q_ERR_UNSUPPORTED
    for f in (fq.lib().fp8q_grouped_gemm_w8a8, fq.lib().fp8q_grouped_gemm_w8a8_ue8m0):
        assert f(A16, 8192, A16, _LD_AS_WRAP, A16, A16, A16, 4, 64, A16, 128, 128, 8192,
                 None) == fq.FP8Q_ERR_SHAPE
        assert f(A16, 8192, A16, 64, A16, A16, A16, 4, 64, A16, 128, 128, 8192, None) == fq.FP8Q_ERR_UNSUPPORTED
    L = fq.lib()
    assert L.fp8q_grouped_gemm_swiglu_quant(A16, 8192, A16, _LD_AS_WRAP, None, 0, A16, A16, A16, 4, 64, A16, 256,
                                            A16, 64, 256, 8192, None) == fq.FP8Q_ERR_SHAPE
    assert L.fp8q_grouped_gemm_swiglu_quant(A16, 8192, A16, 64, None, 0, A16, A16, A16, 4, 64, A16, 256,
                                            A16, 64, 256, 8192, None) == fq.FP8Q_ERR_UNSUPPORTED


def test_grouped_validation():
    L = fq.lib()
    f = L.fp8q_grouped_gemm_w8a8
    assert f(A16, 256, A16, 64, A16, A16, A16, 0, 64, A16, 128, 128, 256, None) == fq.FP8Q_ERR_SHAPE
    assert f(A16, 256, A16, 64, A16, A16, None, 4, 64, A16, 128, 128, 256, None) == fq.FP8Q_ERR_NULL
    assert f(A16, 256, A16, 32, A16, A16, A16, 4, 64, A16, 128, 128, 256, None) == fq.FP8Q_ERR_STRIDE
    assert f(A16, 256, A16, 64, A16, A16, A16, 4, 64, A16, 128, 192, 256, None) == fq.FP8Q_ERR_SHAPE


def test_weight_validation():
    L = fq.lib()
    d = (fq.WeightDesc * 2)()
    d[0] = fq.WeightDesc(A16, A16, A16, 256, 256, 256, 256)
    d[1] = fq.WeightDesc(A16, A16, A16, 128, 384, 384, 384)
    assert L.fp8q_quant_weight_blk128(d, 0, None) == fq.FP8Q_ERR_SHAPE
    assert L.fp8q_quant_weight_blk128(None, 1, None) == fq.FP8Q_ERR_NULL
    d[1] = fq.WeightDesc(A16, A16, A16, 100, 384, 384, 384)
    assert L.fp8q_quant_weight_blk128(d, 2, None) == fq.FP8Q_ERR_SHAPE
    d[1] = fq.WeightDesc(A16, None, A16, 128, 384, 384, 384)
    assert L.fp8q_quant_weight_blk128(d, 2, None) == fq.FP8Q_ERR_NULL
    d[1] = fq.WeightDesc(A16, A16, A16, 128, 384, 256, 384)
    assert L.fp8q_quant_weight_blk128(d, 2, None) == fq.FP8Q_ERR_STRIDE
    d[1] = fq.WeightDesc(A16, A16 + 4, A16, 128, 384, 384, 384)
    assert L.fp8q_quant_weight_blk128(d, 2, None) == fq.FP8Q_ERR_ALIGN


def test_kv_validation():
    L = fq.lib()

    def kv(**kw):
        a = dict(k=A16, ld_k=1024, v=A16, ld_v=1024, t=16, h=8, d=128, slots=A16, kc=A16, vc=A16, page=16,
                 pages=4, ks=A16, vs=A16, rng=448.0, flags=1)
        a.update(kw)
        return L.fp8q_kv_quant(a["k"], a["ld_k"], a["v"], a["ld_v"], a["t"], a["h"], a["d"], a["slots"],
                               a["kc"], a["vc"], a["page"], a["pages"], a["ks"], a["vs"], a["rng"],
                               a["flags"], None)

    assert kv(d=64) == fq.FP8Q_ERR_SHAPE
    assert kv(h=0) == fq.FP8Q_ERR_SHAPE
    assert kv(page=0) == fq.FP8Q_ERR_SHAPE
    assert kv(rng=0.0) == fq.FP8Q_ERR_SHAPE
    assert kv(rng=float("inf")) == fq.FP8Q_ERR_SHAPE
    assert kv(flags=2) == fq.FP8Q_ERR_SHAPE
    assert kv(ks=None) == fq.FP8Q_ERR_NULL
    assert kv(slots=None) == fq.FP8Q_ERR_NULL
    assert kv(ld_k=512) == fq.FP8Q_ERR_STRIDE
    assert kv(kc=A16 + 1) == fq.FP8Q_ERR_ALIGN


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_arguments_without_gpu_report_unsupported():
    assert _act() == fq.FP8Q_ERR_UNSUPPORTED
    assert _gemm() == fq.FP8Q_ERR_UNSUPPORTED
    assert "device" in fq.last_error()


def test_python_binding_refuses_host_tensors():
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    q = torch.zeros(4, 128, dtype=torch.uint8)
    s = torch.zeros(1, 4, dtype=torch.float32)
    with pytest.raises(ValueError):
        fq.fp8q_quant_act_g128(x, q, s, stream=0)


def test_ue8m0_entry_points_validate_like_the_fp32_ones():
    L = fq.lib()
    assert L.fp8q_quant_act_g128_ue8m0(A16, -1, 256, 256, A16, 256, A16, 4, None) == fq.FP8Q_ERR_SHAPE
    assert L.fp8q_quant_act_g128_ue8m0(None, 4, 256, 256, A16, 256, A16, 4, None) == fq.FP8Q_ERR_NULL
    assert L.fp8q_gemm_w8a8_ue8m0(A16, 256, A16, 64, A16, 256, A16, A16, 100, 64, 100, 256, None) == \
        fq.FP8Q_ERR_SHAPE
    assert L.fp8q_gemm_w8a8_ue8m0(A16, 256, A16, 7, A16, 256, A16, A16, 128, 64, 128, 256, None) == \
        fq.FP8Q_ERR_STRIDE
    assert L.fp8q_grouped_gemm_w8a8_ue8m0(A16, 256, A16, 64, A16, A16, A16, 0, 64, A16, 128, 128, 256, None) == \
        fq.FP8Q_ERR_SHAPE
    d = (fq.WeightDesc * 1)()
    d[0] = fq.WeightDesc(A16, A16, A16, 100, 256, 256, 256)
    assert L.fp8q_quant_weight_blk128_ue8m0(d, 1, None) == fq.FP8Q_ERR_SHAPE
    assert L.fp8q_quant_weight_blk128_ue8m0(d, 0, None) == fq.FP8Q_ERR_SHAPE


def test_moe_validation():
    L = fq.lib()

    def dispatch(**kw):
        a = dict(xq=A16, ld_xq=256, xs=A16, ld_xs=8, ids=A16, t=8, topk=2, e=4, k=256, aq=A16, ld_aq=256,
                 a_s=A16, ld_as=16, off=A16, row_of=A16)
        a.update(kw)
        return L.fp8q_moe_dispatch(a["xq"], a["ld_xq"], a["xs"], a["ld_xs"], a["ids"], a["t"], a["topk"], a["e"],
                                   a["k"], a["aq"], a["ld_aq"], a["a_s"], a["ld_as"], a["off"], a["row_of"], None)

    assert dispatch(topk=0) == fq.FP8Q_ERR_SHAPE
    assert dispatch(e=0) == fq.FP8Q_ERR_SHAPE
    assert dispatch(e=40000) == fq.FP8Q_ERR_SHAPE
    assert dispatch(k=200, ld_xq=200, ld_aq=200) == fq.FP8Q_ERR_SHAPE
    assert dispatch(t=1 << 30, topk=4) == fq.FP8Q_ERR_SHAPE
    assert dispatch(off=None) == fq.FP8Q_ERR_NULL
    assert dispatch(ids=None) == fq.FP8Q_ERR_NULL
    assert dispatch(ld_as=15) == fq.FP8Q_ERR_STRIDE
    assert dispatch(ld_xs=7) == fq.FP8Q_ERR_STRIDE
    assert dispatch(ids=A16 + 2) == fq.FP8Q_ERR_ALIGN
    assert dispatch(ld_aq=264) == fq.FP8Q_ERR_ALIGN

    def swiglu(**kw):
        a = dict(h=A16, m=4, n=256, ld_h=512, q=A16, ld_q=256, s=A16, ld_s=4)
        a.update(kw)
        return L.fp8q_swiglu_quant_g128(a["h"], a["m"], a["n"], a["ld_h"], a["q"], a["ld_q"], a["s"], a["ld_s"],
                                        None)

    assert swiglu(n=100) == fq.FP8Q_ERR_SHAPE
    assert swiglu(q=None) == fq.FP8Q_ERR_NULL
    assert swiglu(ld_h=256) == fq.FP8Q_ERR_STRIDE
    assert swiglu(ld_s=3) == fq.FP8Q_ERR_STRIDE
    assert swiglu(h=A16 + 8) == fq.FP8Q_ERR_ALIGN

    def combine(**kw):
        a = dict(y=A16, ld_y=256, row_of=A16, w=A16, t=4, topk=2, hidden=256, out=A16, ld_out=256)
        a.update(kw)
        return L.fp8q_moe_combine(a["y"], a["ld_y"], a["row_of"], a["w"], a["t"], a["topk"], a["hidden"],
                                  a["out"], a["ld_out"], None)

    assert combine(hidden=100) == fq.FP8Q_ERR_SHAPE
    assert combine(topk=0) == fq.FP8Q_ERR_SHAPE
    assert combine(w=None) == fq.FP8Q_ERR_NULL
    assert combine(ld_out=128) == fq.FP8Q_ERR_STRIDE
    assert combine(out=A16 + 4) == fq.FP8Q_ERR_ALIGN


def test_fused_swiglu_grouped_gemm_validation():
    L = fq.lib()

    def g(**kw):
        a = dict(a=A16, ld_a=256, a_s=A16, ld_as=64, tok=None, rows=0, b=A16, b_s=A16, off=A16, groups=4, m=64,
                 q=A16, ld_q=256, s=A16, ld_s=64, half=256, k=256)
        a.update(kw)
        return L.fp8q_grouped_gemm_swiglu_quant(a["a"], a["ld_a"], a["a_s"], a["ld_as"], a["tok"], a["rows"], a["b"],
                                                a["b_s"], a["off"], a["groups"], a["m"], a["q"], a["ld_q"], a["s"],
                                                a["ld_s"], a["half"], a["k"], None)

    assert g(groups=0) == fq.FP8Q_ERR_SHAPE
    assert g(half=100) == fq.FP8Q_ERR_SHAPE
    assert g(half=0) == fq.FP8Q_ERR_SHAPE
    assert g(k=200) == fq.FP8Q_ERR_SHAPE
    assert g(m=-1) == fq.FP8Q_ERR_SHAPE
    assert g(q=None) == fq.FP8Q_ERR_NULL
    assert g(off=None) == fq.FP8Q_ERR_NULL
    assert g(ld_q=128) == fq.FP8Q_ERR_STRIDE
    assert g(ld_s=63) == fq.FP8Q_ERR_STRIDE
    assert g(ld_as=32) == fq.FP8Q_ERR_STRIDE
    assert g(q=A16 + 8) == fq.FP8Q_ERR_ALIGN
    assert g(ld_q=264) == fq.FP8Q_ERR_ALIGN
    assert g(half=1 << 20, k=1 << 11, ld_q=1 << 20, ld_a=1 << 11) == fq.FP8Q_ERR_SHAPE  # weights beyond 2 GiB
    # rows read through row_token: token_rows bounds ld_as, and must be positive
    assert g(tok=A16, rows=0) == fq.FP8Q_ERR_SHAPE
    assert g(tok=A16, rows=100) == fq.FP8Q_ERR_STRIDE     # ld_as = 64 < 100 token rows
    assert g(tok=A16 + 2, rows=32) == fq.FP8Q_ERR_ALIGN
    # a valid call reaches the device check (none here)
    assert g() == fq.FP8Q_ERR_UNSUPPORTED
    assert g(tok=A16, rows=32) == fq.FP8Q_ERR_UNSUPPORTED


def test_moe_route_validation():
    L = fq.lib()

    def r(**kw):
        a = dict(ids=A16, t=16, topk=8, e=128, off=A16, row_of=A16, tok=A16)
        a.update(kw)
        return L.fp8q_moe_route(a["ids"], a["t"], a["topk"], a["e"], a["off"], a["row_of"], a["tok"], None)

    assert r(topk=0) == fq.FP8Q_ERR_SHAPE
    assert r(e=0) == fq.FP8Q_ERR_SHAPE
    assert r(t=-1) == fq.FP8Q_ERR_SHAPE
    assert r(off=None) == fq.FP8Q_ERR_NULL
    assert r(tok=None) == fq.FP8Q_ERR_NULL
    assert r(ids=A16 + 2) == fq.FP8Q_ERR_ALIGN
    assert r() == fq.FP8Q_ERR_UNSUPPORTED


def test_bf16act_gemm_validation():
    L = fq.lib()

    def g(**kw):
        a = dict(x=A16, ld_x=256, b=A16, ld_b=256, bs=A16, y=A16, ld_y=128, m=16, n=128, k=256)
        a.update(kw)
        return L.fp8q_gemm_w8a8_bf16act(a["x"], a["ld_x"], a["b"], a["ld_b"], a["bs"], a["y"], a["ld_y"], a["m"],
                                        a["n"], a["k"], None)

    assert g(m=65) == fq.FP8Q_ERR_SHAPE
    assert g(m=-1) == fq.FP8Q_ERR_SHAPE
    assert g(k=200, ld_x=200, ld_b=200) == fq.FP8Q_ERR_SHAPE
    assert g(x=None) == fq.FP8Q_ERR_NULL
    assert g(ld_x=128) == fq.FP8Q_ERR_STRIDE
    assert g(ld_x=260) == fq.FP8Q_ERR_ALIGN
    assert g(x=A16 + 2) == fq.FP8Q_ERR_ALIGN


def test_decode_attention_validation():
    L = fq.lib()

    def att(**kw):
        a = dict(q=A16, ld_q=1024, kc=A16, vc=A16, bt=A16, ld_bt=4, sl=A16, seqs=2, hq=8, hkv=2, d=128, ps=16,
                 pages=8, qs=A16, ks=A16, vs=A16, sm=0.088, rng=448.0, flags=1, out=A16, ld_out=1024)
        a.update(kw)
        return L.fp8q_paged_decode_attention(a["q"], a["ld_q"], a["kc"], a["vc"], a["bt"], a["ld_bt"], a["sl"],
                                             a["seqs"], a["hq"], a["hkv"], a["d"], a["ps"], a["pages"], a["qs"],
                                             a["ks"], a["vs"], a["sm"], a["rng"], a["flags"], a["out"], a["ld_out"],
                                             None)

    assert att(hq=6, hkv=4) == fq.FP8Q_ERR_SHAPE          # not a multiple
    assert att(hq=34, hkv=2) == fq.FP8Q_ERR_SHAPE         # group of 17
    assert att(d=64) == fq.FP8Q_ERR_SHAPE
    assert att(ps=0) == fq.FP8Q_ERR_SHAPE
    assert att(flags=2) == fq.FP8Q_ERR_SHAPE
    assert att(rng=0.0) == fq.FP8Q_ERR_SHAPE
    assert att(sm=float("nan")) == fq.FP8Q_ERR_SHAPE
    assert att(qs=None) == fq.FP8Q_ERR_NULL
    assert att(bt=None) == fq.FP8Q_ERR_NULL
    assert att(ld_q=512) == fq.FP8Q_ERR_STRIDE
    assert att(ld_bt=0) == fq.FP8Q_ERR_STRIDE
    assert att(kc=A16 + 8) == fq.FP8Q_ERR_ALIGN
    assert att(ld_out=1028) == fq.FP8Q_ERR_ALIGN
