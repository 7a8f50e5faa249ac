"""Thin Python binding of libmoe4 (ctypes). Same names as the C interface in
include/moe4.h; the functions only marshal torch tensors into pointers, sizes
and the current HIP stream. Every step of the layer runs in the library's HIP
kernels; nothing here computes.

Importing this module loads libmoe4.so and fails loudly when it is missing.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE4_LIB_PATH names another build of the same library (the host-only ASan
# build that tests/test_abi_asan.py loads); by default the in-tree libmoe4.so
LIB_PATH = os.environ.get("MOE4_LIB_PATH") or os.path.join(_HERE, "libmoe4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; build it with `python -m bit_mixture_experts_amd.build` "
        "or __graft_entry__.build()")

_lib = ctypes.CDLL(LIB_PATH)

MOE4_OK, MOE4_EINVAL, MOE4_EUNSUPPORTED, MOE4_ESHAPE = 0, -1, -2, -3
MOE4_EALIGN, MOE4_EWORKSPACE, MOE4_EDEVICE = -4, -5, -6
MOE4_FMT_NF4, MOE4_FMT_MXFP4, MOE4_FMT_NF4_DQ = 1, 2, 3
MOE4_DQ_WS_BYTES = 8192
MOE4_GU_HALVES, MOE4_GU_INTERLEAVED = 1, 2
MOE4_ACT_SWIGLU, MOE4_ACT_SWIGLU_CLAMPED = 1, 2
MOE4_VARIANT_AUTO, MOE4_VARIANT_SKINNY, MOE4_VARIANT_TILED = 0, 1, 2
MOE4_DTYPE_BF16, MOE4_DTYPE_F32 = 1, 2
MOE4_NOALLOC_SCRATCH_BYTES = 16 << 20

# every symbol declared in include/moe4.h
EXPORTS = ("moe4_quantize_nf4", "moe4_compress_absmax", "moe4_expand_absmax",
           "moe4_decode_mxfp4", "moe4_convert_mxfp4_nf4",
           "moe4_router_logits", "moe4_route", "moe4_route_backward", "moe4_permute",
           "moe4_gather_rows", "moe4_route_permute", "moe4_expert_forward", "moe4_expert_forward_gather", "moe4_expert_forward_noalloc", "moe4_combine",
           "moe4_expert_backward",
           "moe4_workspace_size", "moe4_set_timing_events", "moe4_last_error",
           "moe4_last_variant")


class Moe4Experts(ctypes.Structure):
    """Mirror of the C struct moe4_experts."""
    _fields_ = [
        ("format", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32),
        ("I", ctypes.c_int32), ("gu_layout", ctypes.c_int32), ("act", ctypes.c_int32),
        ("act_alpha", ctypes.c_float), ("act_limit", ctypes.c_float),
        ("gu_q", ctypes.c_void_p), ("gu_s", ctypes.c_void_p),
        ("dn_q", ctypes.c_void_p), ("dn_s", ctypes.c_void_p),
        ("gu_bias", ctypes.c_void_p), ("dn_bias", ctypes.c_void_p),
        ("lora_A", ctypes.c_void_p), ("lora_B", ctypes.c_void_p),
        ("lora_r", ctypes.c_int32), ("lora_scale", ctypes.c_float),
        ("variant", ctypes.c_int32),
        ("gu_s2", ctypes.c_void_p), ("dn_s2", ctypes.c_void_p),
        ("gu_soff", ctypes.c_void_p), ("dn_soff", ctypes.c_void_p),
        ("dq_book", ctypes.c_void_p),
    ]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_P = ctypes.POINTER(Moe4Experts)
_SIGS = {
    "moe4_quantize_nf4": ([_vp, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "moe4_decode_mxfp4": ([_vp, _vp, _i64, _i64, _vp, _vp], ctypes.c_int),
    "moe4_compress_absmax": ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe4_expand_absmax": ([_vp, _vp, _vp, _vp, _i64, _vp, _vp], ctypes.c_int),
    "moe4_convert_mxfp4_nf4": ([_vp, _vp, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "moe4_route": ([_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "moe4_router_logits": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp], ctypes.c_int),
    "moe4_route_backward": ([_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp,
                             _vp, _vp], ctypes.c_int),
    "moe4_permute": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp],
                     ctypes.c_int),
    "moe4_gather_rows": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe4_route_permute": ([_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                            _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe4_expert_forward": ([_P, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe4_expert_forward_noalloc": ([_P, _vp, _vp, _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "moe4_expert_forward_gather": ([_P, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _sz, _vp],
                                   ctypes.c_int),
    "moe4_combine": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp], ctypes.c_int),
    "moe4_expert_backward": ([_P, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                             ctypes.c_int),
    "moe4_workspace_size": ([_P, _i32, _i32], ctypes.c_size_t),
    "moe4_set_timing_events": ([_vp, _i32], ctypes.c_int),
    "moe4_last_error": ([], ctypes.c_char_p),
    "moe4_last_variant": ([], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes, _f.restype = _args, _res


class Moe4Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"moe4 status {code}: {msg}")
        self.code = code


def moe4_last_error():
    return _lib.moe4_last_error().decode()


def moe4_last_variant():
    return _lib.moe4_last_variant()


def _check(rc):
    if rc != MOE4_OK:
        raise Moe4Error(rc, moe4_last_error())


def _ptr(t, dtypes=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


class Experts:
    """Owns references to one layer's stack tensors and the C descriptor."""

    def __init__(self, fmt, gu_q, gu_s, dn_q, dn_s, *, gu_layout, act, E, H, I,
                 gu_bias=None, dn_bias=None, lora_A=None, lora_B=None, lora_scale=0.0,
                 act_alpha=1.702, act_limit=7.0, variant=MOE4_VARIANT_AUTO,
                 gu_s2=None, dn_s2=None, gu_soff=None, dn_soff=None, dq_book=None):
        """fmt MOE4_FMT_NF4_DQ: gu_s / dn_s are the u8 absmax codes and
        gu_s2, dn_s2, gu_soff, dn_soff, dq_book the rest of the nested absmax
        (see moe4_compress_absmax)."""
        sdt = _F32 if fmt == MOE4_FMT_NF4 else _U8
        self.tensors = (gu_q, gu_s, dn_q, dn_s, gu_bias, dn_bias, lora_A, lora_B,
                        gu_s2, dn_s2, gu_soff, dn_soff, dq_book)
        self.desc = Moe4Experts(
            format=fmt, E=E, H=H, I=I, gu_layout=gu_layout, act=act,
            act_alpha=act_alpha, act_limit=act_limit,
            gu_q=_ptr(gu_q, _U8, "gu_q"), gu_s=_ptr(gu_s, sdt, "gu_s"),
            dn_q=_ptr(dn_q, _U8, "dn_q"), dn_s=_ptr(dn_s, sdt, "dn_s"),
            gu_bias=_ptr(gu_bias, _BF16, "gu_bias"), dn_bias=_ptr(dn_bias, _BF16, "dn_bias"),
            lora_A=_ptr(lora_A, _BF16, "lora_A"), lora_B=_ptr(lora_B, _BF16, "lora_B"),
            lora_r=0 if lora_A is None else int(lora_A.shape[1]),
            lora_scale=lora_scale, variant=variant,
            gu_s2=_ptr(gu_s2, _F32, "gu_s2"), dn_s2=_ptr(dn_s2, _F32, "dn_s2"),
            gu_soff=_ptr(gu_soff, _F32, "gu_soff"), dn_soff=_ptr(dn_soff, _F32, "dn_soff"),
            dq_book=_ptr(dq_book, _F32, "dq_book"))
        self.E, self.H, self.I = E, H, I
        self.lora_r = self.desc.lora_r

    def with_variant(self, variant):
        d = Moe4Experts()
        ctypes.pointer(d)[0] = self.desc
        d.variant = variant
        out = object.__new__(Experts)
        out.__dict__.update(self.__dict__)
        out.desc = d
        return out


def moe4_quantize_nf4(w, packed, absmax, blocksize=64, stream=None):
    _check(_lib.moe4_quantize_nf4(_ptr(w, _F32, "w"), w.numel(), blocksize,
                                  _ptr(packed, _U8, "packed"), _ptr(absmax, _F32, "absmax"),
                                  _stream(stream)))


def moe4_compress_absmax(absmax, book, code, absmax2, offset, ws, stream=None):
    """absmax f32 [n] -> code u8 [n], absmax2 f32 [ceil(n/256)], offset f32 [1];
    ws: at least MOE4_DQ_WS_BYTES bytes of device scratch."""
    n = absmax.numel()
    if code.numel() != n or absmax2.numel() != (n + 255) // 256 or offset.numel() != 1:
        raise ValueError("compress_absmax: output sizes do not match n")
    _check(_lib.moe4_compress_absmax(_ptr(absmax, _F32, "absmax"), n, _ptr(book, _F32, "book"),
                                     _ptr(code, _U8, "code"), _ptr(absmax2, _F32, "absmax2"),
                                     _ptr(offset, _F32, "offset"), _ptr(ws, None, "ws"),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def moe4_expand_absmax(code, absmax2, offset, book, out, stream=None):
    n = code.numel()
    if out.numel() != n or absmax2.numel() != (n + 255) // 256:
        raise ValueError("expand_absmax: sizes do not match")
    _check(_lib.moe4_expand_absmax(_ptr(code, _U8, "code"), _ptr(absmax2, _F32, "absmax2"),
                                   _ptr(offset, _F32, "offset"), _ptr(book, _F32, "book"), n,
                                   _ptr(out, _F32, "out"), _stream(stream)))


def moe4_decode_mxfp4(blocks, scales, out, stream=None):
    R = scales.numel() // scales.shape[-1] if scales.dim() else 0
    K = scales.shape[-1] * 32
    _check(_lib.moe4_decode_mxfp4(_ptr(blocks, _U8, "blocks"), _ptr(scales, _U8, "scales"),
                                  R, K, _ptr(out, _BF16, "out"), _stream(stream)))


def moe4_convert_mxfp4_nf4(blocks, scales, packed, absmax, stream=None):
    """blocks u8 [..., K/32, 16], scales u8 [..., K/32] -> packed u8 [..., K/2],
    absmax f32 [..., K/64]."""
    R = scales.numel() // scales.shape[-1] if scales.dim() else 0
    K = scales.shape[-1] * 32
    if packed.numel() != R * K // 2 or absmax.numel() != R * (K // 64):
        raise ValueError("packed / absmax do not match the MXFP4 stack's size")
    _check(_lib.moe4_convert_mxfp4_nf4(_ptr(blocks, _U8, "blocks"), _ptr(scales, _U8, "scales"),
                                       R, K, _ptr(packed, _U8, "packed"),
                                       _ptr(absmax, _F32, "absmax"), _stream(stream)))


def moe4_route(logits, k, topk_idx, topk_w, renormalize=True, stream=None):
    T, E = logits.shape
    _check(_lib.moe4_route(_ptr(logits, _F32, "logits"), T, E, k, int(bool(renormalize)),
                           _ptr(topk_idx, _I32, "topk_idx"), _ptr(topk_w, _F32, "topk_w"),
                           _stream(stream)))


def moe4_router_logits(x, wr, logits, bias=None, stream=None):
    """x bf16 [T, H], wr bf16 [E, H], bias f32 [E] or None -> logits f32 [T, E]."""
    T, H = x.shape
    E = wr.shape[0]
    if wr.shape[1] != H or tuple(logits.shape) != (T, E):
        raise ValueError("router_logits: x [T,H], wr [E,H] and logits [T,E] do not agree")
    _check(_lib.moe4_router_logits(_ptr(x, _BF16, "x"), _ptr(wr, _BF16, "wr"),
                                   _ptr(bias, _F32, "bias"), T, H, E,
                                   _ptr(logits, _F32, "logits"), _stream(stream)))


def moe4_route_backward(topk_idx, topk_w, dout, y_perm, row_of_slot, dw, dlogits,
                        logits=None, renormalize=True, stream=None):
    """dw f32 [T, k] and dlogits f32 [T, E] from the upstream gradient dout
    bf16 [T, H] and the slots' expert outputs y_perm f32 [T*k, H]."""
    T, k = topk_idx.shape
    E = dlogits.shape[1]
    H = dout.shape[1]
    _check(_lib.moe4_route_backward(_ptr(topk_idx, _I32, "topk_idx"), _ptr(topk_w, _F32, "topk_w"),
                                    _ptr(logits, _F32, "logits"), int(bool(renormalize)),
                                    _ptr(dout, _BF16, "dout"), _ptr(y_perm, _F32, "y_perm"),
                                    _ptr(row_of_slot, _I32, "row_of_slot"), T, k, E, H,
                                    _ptr(dw, _F32, "dw"), _ptr(dlogits, _F32, "dlogits"),
                                    _stream(stream)))


def moe4_permute(topk_idx, E, offsets, slot_of_row, row_of_slot, x=None, row_scale=None,
                 x_perm=None, ws=None, stream=None):
    T, k = topk_idx.shape
    H = 0 if x is None else x.shape[1]
    _check(_lib.moe4_permute(_ptr(topk_idx, _I32, "topk_idx"), T, k, E,
                             _ptr(offsets, _I32, "offsets"), _ptr(slot_of_row, _I32, "slot_of_row"),
                             _ptr(row_of_slot, _I32, "row_of_slot"), _ptr(x, _BF16, "x"),
                             _ptr(row_scale, _F32, "row_scale"), H,
                             _ptr(x_perm, _BF16, "x_perm"), _ptr(ws, None, "ws"),
                             0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)))


def moe4_gather_rows(x, k, slot_of_row, x_perm, row_scale=None, stream=None):
    """The row gather of moe4_permute on an existing permutation (slot_of_row)."""
    T, H = x.shape
    _check(_lib.moe4_gather_rows(_ptr(x, _BF16, "x"), T, k, H,
                                 _ptr(slot_of_row, _I32, "slot_of_row"),
                                 _ptr(row_scale, _F32, "row_scale"), _ptr(x_perm, _BF16, "x_perm"),
                                 _stream(stream)))


def moe4_route_permute(logits, k, topk_idx, topk_w, offsets, slot_of_row, row_of_slot, x=None,
                       x_perm=None, ws=None, renormalize=True, stream=None):
    """moe4_route then moe4_permute (no row_scale), one launch for small batches."""
    T, E = logits.shape
    H = 0 if x is None else x.shape[1]
    _check(_lib.moe4_route_permute(_ptr(logits, _F32, "logits"), T, E, k, int(bool(renormalize)),
                                   _ptr(topk_idx, _I32, "topk_idx"), _ptr(topk_w, _F32, "topk_w"),
                                   _ptr(offsets, _I32, "offsets"),
                                   _ptr(slot_of_row, _I32, "slot_of_row"),
                                   _ptr(row_of_slot, _I32, "row_of_slot"), _ptr(x, _BF16, "x"), H,
                                   _ptr(x_perm, _BF16, "x_perm"), _ptr(ws, None, "ws"),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream)))


def moe4_expert_forward_gather(ex, x, k, slot_of_row, offsets, y_perm, save_gu=None, ws=None,
                               stream=None):
    """moe4_expert_forward on rows gathered from x [T, H] by the GEMM itself."""
    T = x.shape[0]
    _check(_lib.moe4_expert_forward_gather(ctypes.byref(ex.desc), _ptr(x, _BF16, "x"), T, k,
                                           _ptr(slot_of_row, _I32, "slot_of_row"),
                                           _ptr(offsets, _I32, "offsets"), T * k,
                                           _ptr(y_perm, _F32, "y_perm"),
                                           _ptr(save_gu, _F32, "save_gu"), _ptr(ws, None, "ws"),
                                           0 if ws is None else ws.numel() * ws.element_size(),
                                           _stream(stream)))


def moe4_expert_forward(ex, x_perm, offsets, y_perm, save_gu=None, save_xa=None, ws=None,
                        stream=None):
    _check(_lib.moe4_expert_forward(ctypes.byref(ex.desc), _ptr(x_perm, _BF16, "x_perm"),
                                    _ptr(offsets, _I32, "offsets"), x_perm.shape[0],
                                    _ptr(y_perm, _F32, "y_perm"), _ptr(save_gu, _F32, "save_gu"),
                                    _ptr(save_xa, _F32, "save_xa"), _ptr(ws, None, "ws"),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))


def moe4_expert_forward_noalloc(ex, x_perm, offsets, y_perm, save_gu=None, save_xa=None,
                                stream=None):
    """moe4_expert_forward with the library's per-device scratch in place of a
    workspace (allocates nothing)."""
    _check(_lib.moe4_expert_forward_noalloc(
        ctypes.byref(ex.desc), _ptr(x_perm, _BF16, "x_perm"), _ptr(offsets, _I32, "offsets"),
        x_perm.shape[0], _ptr(y_perm, _F32, "y_perm"), _ptr(save_gu, _F32, "save_gu"),
        _ptr(save_xa, _F32, "save_xa"), _stream(stream)))


def moe4_combine(y_perm, row_of_slot, topk_w, out, k, stream=None):
    """out: bf16 [T, H] (rounded once) or float32 [T, H] (the fp32 sum)."""
    T, H = out.shape
    dt = MOE4_DTYPE_F32 if out.dtype == torch.float32 else MOE4_DTYPE_BF16
    _check(_lib.moe4_combine(_ptr(y_perm, _F32, "y_perm"), _ptr(row_of_slot, _I32, "row_of_slot"),
                             _ptr(topk_w, _F32, "topk_w"), T, k, H,
                             _ptr(out, _BF16 + _F32, "out"), dt, _stream(stream)))


def moe4_expert_backward(ex, x_perm, offsets, save_gu, save_xa, dy_perm, dx_perm, dA=None,
                         dB=None, ws=None, stream=None):
    _check(_lib.moe4_expert_backward(ctypes.byref(ex.desc), _ptr(x_perm, _BF16, "x_perm"),
                                     _ptr(offsets, _I32, "offsets"), dy_perm.shape[0],
                                     _ptr(save_gu, _F32, "save_gu"), _ptr(save_xa, _F32, "save_xa"),
                                     _ptr(dy_perm, _BF16, "dy_perm"), _ptr(dx_perm, _F32, "dx_perm"),
                                     _ptr(dA, _F32, "dA"), _ptr(dB, _F32, "dB"),
                                     _ptr(ws, None, "ws"),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))


def moe4_set_timing_events(events):
    """events: a ctypes array of hipEvent_t handles (len >= 4), or None to stop.
    The caller keeps the array alive while timing is on."""
    if events is None:
        _check(_lib.moe4_set_timing_events(None, 0))
    else:
        _check(_lib.moe4_set_timing_events(ctypes.cast(events, ctypes.c_void_p), len(events)))


def moe4_workspace_size(ex, T, k):
    n = _lib.moe4_workspace_size(ctypes.byref(ex.desc), T, k)
    if n == 0:
        raise Moe4Error(MOE4_EINVAL, moe4_last_error())
    return n
