"""The C library loads without a GPU, exports every symbol include/moe4.h
declares, and refuses bad arguments synchronously, before anything is
enqueued (so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

moe4 = pytest.importorskip("bit_mixture_experts_amd.moe4")
lib = moe4._lib

FAKE = 0x10000          # 256-byte aligned, never dereferenced: validation fails first
FAKE_MIS = 0x10004      # 4-byte aligned only


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "moe4.h")) as f:
        src = f.read()
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe4_\w+)\(", src, re.M))


def test_exports_every_declared_symbol():
    declared = _declared_symbols()
    assert declared == set(moe4.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _desc(**kw):
    d = moe4.Moe4Experts(format=moe4.MOE4_FMT_NF4, E=8, H=256, I=512,
                         gu_layout=moe4.MOE4_GU_HALVES, act=moe4.MOE4_ACT_SWIGLU,
                         act_alpha=1.702, act_limit=7.0, gu_q=FAKE, gu_s=FAKE, dn_q=FAKE,
                         dn_s=FAKE, lora_r=0, lora_scale=0.0, variant=0)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _fwd(d, rows=16, ws=FAKE, ws_bytes=1 << 30):
    return lib.moe4_expert_forward(ctypes.byref(d), FAKE, FAKE, rows, FAKE, None, None, ws,
                                   ws_bytes, None)


def test_quantize_refusals():
    assert lib.moe4_quantize_nf4(FAKE, 128, 32, FAKE, FAKE, None) == moe4.MOE4_EUNSUPPORTED
    assert lib.moe4_quantize_nf4(FAKE, 65, 64, FAKE, FAKE, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_quantize_nf4(None, 64, 64, FAKE, FAKE, None) == moe4.MOE4_EINVAL
    assert "w is NULL" in moe4.moe4_last_error()
    assert lib.moe4_quantize_nf4(FAKE_MIS, 64, 64, FAKE, FAKE, None) == moe4.MOE4_EALIGN
    assert lib.moe4_quantize_nf4(None, 0, 64, None, None, None) == moe4.MOE4_OK   # empty


def test_decode_route_combine_refusals():
    assert lib.moe4_decode_mxfp4(FAKE, FAKE, 4, 48, FAKE, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_decode_mxfp4(FAKE, FAKE, 4, 64, FAKE_MIS, None) == moe4.MOE4_EALIGN
    assert lib.moe4_convert_mxfp4_nf4(FAKE, FAKE, 4, 96, FAKE, FAKE, None) == moe4.MOE4_ESHAPE
    assert "multiple of 64" in moe4.moe4_last_error()
    assert lib.moe4_convert_mxfp4_nf4(FAKE, FAKE, -1, 64, FAKE, FAKE, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_convert_mxfp4_nf4(FAKE, FAKE, 4, 64, FAKE_MIS, FAKE, None) == moe4.MOE4_EALIGN
    assert lib.moe4_convert_mxfp4_nf4(None, FAKE, 4, 64, FAKE, FAKE, None) == moe4.MOE4_EINVAL
    assert lib.moe4_convert_mxfp4_nf4(None, None, 0, 64, None, None, None) == moe4.MOE4_OK
    assert lib.moe4_route(FAKE, 4, 8, 9, 1, FAKE, FAKE, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_route(FAKE, 4, 2000, 2, 1, FAKE, FAKE, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_route(FAKE, (1 << 28), 128, 8, 1, FAKE, FAKE, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_route(None, 4, 8, 2, 1, FAKE, FAKE, None) == moe4.MOE4_EINVAL
    assert lib.moe4_combine(FAKE, FAKE, None, 4, 2, 12, FAKE, 1, None) == moe4.MOE4_ESHAPE
    assert lib.moe4_combine(FAKE, None, None, 4, 2, 16, FAKE, 1, None) == moe4.MOE4_EINVAL
    assert lib.moe4_combine(FAKE, FAKE, None, 4, 2, 16, FAKE, 0, None) == moe4.MOE4_EINVAL
    assert "out_dtype unset" in moe4.moe4_last_error()


def test_double_quant_refusals():
    c = lib.moe4_compress_absmax
    assert c(FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE, 8192, None) == moe4.MOE4_ESHAPE
    assert c(FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None) == moe4.MOE4_EWORKSPACE
    assert c(FAKE, 100, None, FAKE, FAKE, FAKE, FAKE, 8192, None) == moe4.MOE4_EINVAL
    assert c(FAKE, 100, FAKE, FAKE_MIS + 1, FAKE, FAKE, FAKE, 8192, None) == moe4.MOE4_EALIGN
    assert c(None, 0, None, None, None, None, None, 0, None) == moe4.MOE4_OK
    x = lib.moe4_expand_absmax
    assert x(FAKE, FAKE, None, FAKE, 10, FAKE, None) == moe4.MOE4_EINVAL
    assert x(None, None, None, None, 0, None, None) == moe4.MOE4_OK
    # descriptor: the nested absmax fields are required with NF4_DQ, refused otherwise
    d = _desc(format=moe4.MOE4_FMT_NF4_DQ)
    assert _fwd(d) == moe4.MOE4_EINVAL and "gu_s2" in moe4.moe4_last_error()
    d = _desc(format=moe4.MOE4_FMT_NF4, dq_book=FAKE)
    assert _fwd(d) == moe4.MOE4_EINVAL and "double-quantised" in moe4.moe4_last_error()
    d = _desc(format=moe4.MOE4_FMT_NF4_DQ, gu_s2=FAKE, dn_s2=FAKE, gu_soff=FAKE, dn_soff=FAKE,
              dq_book=FAKE, H=96)
    assert _fwd(d) == moe4.MOE4_ESHAPE


def test_router_refusals():
    r = lib.moe4_router_logits
    assert r(FAKE, FAKE, None, 4, 64, 0, FAKE, None) == moe4.MOE4_ESHAPE
    assert r(FAKE, FAKE, None, 4, 60, 8, FAKE, None) == moe4.MOE4_ESHAPE
    assert "multiple of 8" in moe4.moe4_last_error()
    assert r(FAKE_MIS, FAKE, None, 4, 64, 8, FAKE, None) == moe4.MOE4_EALIGN
    assert r(FAKE, None, None, 4, 64, 8, FAKE, None) == moe4.MOE4_EINVAL
    assert r(None, None, None, 0, 64, 8, None, None) == moe4.MOE4_OK
    b = lib.moe4_route_backward
    args = [FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 4, 2, 8, 64, FAKE, FAKE, None]
    assert b(*args[:7], 4, 9, 8, 64, *args[11:]) == moe4.MOE4_ESHAPE          # k > E
    assert b(*args[:7], 4, 2, 8, 36, *args[11:]) == moe4.MOE4_ESHAPE         # H % 8
    assert b(FAKE, FAKE, None, 0, *args[4:]) == moe4.MOE4_EINVAL              # logits needed
    assert "renormalisation" in moe4.moe4_last_error()
    assert b(*args[:4], FAKE_MIS, *args[5:]) == moe4.MOE4_EALIGN              # dout
    assert b(*args[:11], None, FAKE, None) == moe4.MOE4_EINVAL                # dw
    assert b(None, None, None, 1, None, None, None, 0, 2, 8, 64, None, None, None) == moe4.MOE4_OK


def test_permute_refusals():
    # row_scale without x, undersized workspace for a large permutation
    assert lib.moe4_permute(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, None, FAKE, 0, None, None, 0,
                            None) == moe4.MOE4_EINVAL
    assert lib.moe4_permute(FAKE, 4096, 8, 128, FAKE, FAKE, FAKE, FAKE, None, 2048, FAKE, FAKE,
                            16, None) == moe4.MOE4_EWORKSPACE
    assert lib.moe4_permute(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, None, 12, FAKE, None, 0,
                            None) == moe4.MOE4_ESHAPE


def test_gather_rows_refusals():
    # k outside [1, 1024], H not a multiple of 8, a NULL slot map, misaligned rows;
    # nothing to gather (T = 0) is accepted with NULL buffers
    g = lib.moe4_gather_rows
    assert g(FAKE, 4, 0, 64, FAKE, None, FAKE, None) == moe4.MOE4_ESHAPE
    assert g(FAKE, 4, 2, 12, FAKE, None, FAKE, None) == moe4.MOE4_ESHAPE
    assert g(FAKE, -1, 2, 64, FAKE, None, FAKE, None) == moe4.MOE4_ESHAPE
    assert g(FAKE, 4, 2, 64, None, None, FAKE, None) == moe4.MOE4_EINVAL
    assert "slot_of_row" in moe4.moe4_last_error()
    assert g(FAKE_MIS, 4, 2, 64, FAKE, None, FAKE, None) == moe4.MOE4_EALIGN
    assert g(None, 0, 2, 64, None, None, None, None) == moe4.MOE4_OK


def test_forward_gather_refusals():
    fg = lib.moe4_expert_forward_gather
    d = _desc()
    ws = 1 << 30
    # adapters take x_perm; rows must be T*k; x within 2^29 bytes; alignment; nulls
    dl = _desc(lora_A=FAKE, lora_B=FAKE, lora_r=8, lora_scale=2.0)
    assert fg(ctypes.byref(dl), FAKE, 4, 2, FAKE, FAKE, 8, FAKE, None, FAKE, ws,
              None) == moe4.MOE4_EUNSUPPORTED
    assert fg(ctypes.byref(d), FAKE, 4, 2, FAKE, FAKE, 9, FAKE, None, FAKE, ws,
              None) == moe4.MOE4_ESHAPE
    assert fg(ctypes.byref(d), FAKE, 4, 0, FAKE, FAKE, 0, FAKE, None, FAKE, ws,
              None) == moe4.MOE4_ESHAPE
    assert fg(ctypes.byref(d), FAKE, 1 << 20, 1, FAKE, FAKE, 1 << 20, FAKE, None, FAKE, ws,
              None) == moe4.MOE4_ESHAPE
    assert "2^29" in moe4.moe4_last_error()
    assert fg(ctypes.byref(d), FAKE_MIS, 4, 2, FAKE, FAKE, 8, FAKE, None, FAKE, ws,
              None) == moe4.MOE4_EALIGN
    assert fg(ctypes.byref(d), FAKE, 4, 2, None, FAKE, 8, FAKE, None, FAKE, ws,
              None) == moe4.MOE4_EINVAL
    assert "slot_of_row is NULL" in moe4.moe4_last_error()
    assert fg(ctypes.byref(d), FAKE, 4, 2, FAKE, FAKE, 8, FAKE, None, FAKE, 16,
              None) == moe4.MOE4_EWORKSPACE


def test_route_permute_refusals():
    rp = lib.moe4_route_permute
    # E, k and T bounds; missing arrays; misaligned x; H not a multiple of 8;
    # undersized workspace for a large batch; T = 0 needs only offsets
    assert rp(FAKE, 4, 0, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, 0,
              None) == moe4.MOE4_ESHAPE
    assert rp(FAKE, 4, 8, 9, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, 0,
              None) == moe4.MOE4_ESHAPE
    assert rp(FAKE, -1, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, 0,
              None) == moe4.MOE4_ESHAPE
    assert rp(None, 4, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, None, 0,
              None) == moe4.MOE4_EINVAL
    assert "logits is NULL" in moe4.moe4_last_error()
    assert rp(FAKE, 4, 8, 2, 1, FAKE, FAKE, None, FAKE, FAKE, None, 0, None, None, 0,
              None) == moe4.MOE4_EINVAL
    assert rp(FAKE, 4, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE_MIS, 16, FAKE, None, 0,
              None) == moe4.MOE4_EALIGN
    assert rp(FAKE, 4, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 12, FAKE, None, 0,
              None) == moe4.MOE4_ESHAPE
    assert rp(FAKE, 4096, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2048, FAKE, FAKE, 16,
              None) == moe4.MOE4_EWORKSPACE
    assert rp(None, 0, 8, 2, 1, None, None, None, None, None, None, 0, None, None, 0,
              None) == moe4.MOE4_EINVAL   # offsets are still written


@pytest.mark.parametrize("field,value,code,msg", [
    ("format", 0, moe4.MOE4_EINVAL, "format unset"),
    ("format", 7, moe4.MOE4_EINVAL, "format unknown"),
    ("gu_layout", 0, moe4.MOE4_EINVAL, "gu_layout unset"),
    ("act", 0, moe4.MOE4_EINVAL, "act unset"),
    ("variant", 5, moe4.MOE4_EINVAL, "variant unknown"),
    ("E", 0, moe4.MOE4_ESHAPE, "E = 0"),
    ("E", 1025, moe4.MOE4_ESHAPE, "E = 1025"),
    ("H", 96, moe4.MOE4_ESHAPE, "not a multiple of 64"),
    ("I", 32, moe4.MOE4_ESHAPE, "not a multiple of 64"),
    ("I", 1 << 23, moe4.MOE4_ESHAPE, "under 2 GiB"),
    ("gu_q", None, moe4.MOE4_EINVAL, "gu_q is NULL"),
    ("dn_q", FAKE + 8, moe4.MOE4_EALIGN, "dn_q is not 16-byte aligned"),
    ("lora_A", FAKE, moe4.MOE4_EINVAL, "given together"),
])
def test_descriptor_refusals(field, value, code, msg):
    d = _desc(**{field: value})
    assert _fwd(d) == code
    assert msg in moe4.moe4_last_error()
    assert moe4.moe4_last_variant() == 0


def test_tile_offsets_refused():
    # one expert's packed matrix fits (I * H < 2^31) but a 320-row tile of
    # H fp32 values (the down GEMM's output rows) does not fit 32-bit byte
    # offsets with room for the out-of-range offset above it
    d = _desc(H=1 << 21, I=64)
    assert _fwd(d) == moe4.MOE4_ESHAPE
    assert "320-row fp32 tile" in moe4.moe4_last_error()
    d = _desc(H=64, I=1 << 20)   # K = 2I of the gate_up dgrad
    assert _fwd(d) == moe4.MOE4_ESHAPE
    d = _desc(H=1600 * 1024, I=64)   # near the limit passes validation
    assert 1280 * d.H < (1 << 31) - (1 << 24)
    assert lib.moe4_workspace_size(ctypes.byref(d), 4, 2) > 0


def test_mxfp4_alignment_and_clamp_parameters():
    d = _desc(format=moe4.MOE4_FMT_MXFP4, H=2880, I=2880, act=moe4.MOE4_ACT_SWIGLU_CLAMPED,
              act_limit=0.0)
    assert _fwd(d) == moe4.MOE4_EINVAL and "act_limit" in moe4.moe4_last_error()
    d = _desc(format=moe4.MOE4_FMT_MXFP4, H=80, I=64)
    assert _fwd(d) == moe4.MOE4_ESHAPE


def test_lora_rank_and_workspace():
    d = _desc(lora_A=FAKE, lora_B=FAKE, lora_r=65)
    assert _fwd(d) == moe4.MOE4_ESHAPE
    d = _desc(lora_A=FAKE, lora_B=FAKE, lora_r=8, lora_scale=2.0)
    need = lib.moe4_workspace_size(ctypes.byref(d), 64, 2)
    # forward: h [128, 512] bf16 + xa [128, 8] f32; backward: dGU [128, 1024] bf16 +
    # t [128, 8] f32 + the transposed adapter B [8 experts, 8, 1024] bf16 (all 256-aligned)
    assert need == max(128 * 512 * 2 + 128 * 8 * 4, 128 * 1024 * 2 + 128 * 8 * 4 + 8 * 8 * 1024 * 2)
    fwd_need = 128 * 512 * 2 + 128 * 8 * 4
    assert _fwd(d, rows=128, ws=FAKE, ws_bytes=fwd_need - 1) == moe4.MOE4_EWORKSPACE
    assert "131072" in moe4.moe4_last_error() or str(fwd_need) in moe4.moe4_last_error()
    assert _fwd(d, rows=128, ws=None, ws_bytes=0) == moe4.MOE4_EWORKSPACE
    assert _fwd(d, rows=128, ws=FAKE + 16, ws_bytes=need) == moe4.MOE4_EALIGN
    assert lib.moe4_workspace_size(ctypes.byref(_desc(format=0)), 4, 2) == 0


def test_backward_refusals():
    d = _desc()
    rc = lib.moe4_expert_backward(ctypes.byref(d), FAKE, FAKE, 16, FAKE, None, FAKE, FAKE,
                                  FAKE, None, FAKE, 1 << 30, None)
    assert rc == moe4.MOE4_EINVAL and "without LoRA" in moe4.moe4_last_error()
    d = _desc(lora_A=FAKE, lora_B=FAKE, lora_r=8)
    rc = lib.moe4_expert_backward(ctypes.byref(d), FAKE, FAKE, 16, FAKE, None, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == moe4.MOE4_EINVAL and "save_xa is NULL" in moe4.moe4_last_error()
