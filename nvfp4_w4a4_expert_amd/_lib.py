"""ctypes binding of libnvfp4moe.so (include/nvfp4_moe.h).

Argument marshalling only: every function forwards to the C entry point of
the same name.  Device buffers are torch tensors on the GPU (their
``data_ptr()`` is passed); the stream is torch's current stream unless one
is given.  Errors come back as :class:`NVFP4Error`.

The library must have been built (``python -m nvfp4_w4a4_expert_amd.build``);
importing this module without it raises ImportError — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB_PATH

(OK, ERR_INVALID_ARG, ERR_BAD_SCALE, ERR_WORKSPACE, ERR_DEVICE, ERR_UNSUPPORTED,
 ERR_TOO_LARGE) = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20      # NVFP4_NOALLOC_SCRATCH_BYTES
SLOT_OK, SLOT_UNWRITTEN, SLOT_NAN, SLOT_INF, SLOT_NONPOSITIVE, SLOT_RECIP_OVERFLOW = range(6)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m nvfp4_w4a4_expert_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class MoEWeights(ctypes.Structure):
    _fields_ = [
        ("w13", _p), ("w13_sf", _p), ("w13_scale2", _p),
        ("w2", _p), ("w2_sf", _p), ("w2_scale2", _p),
        ("w13_input_scale", _p), ("w2_input_scale", _p),
        ("a1_gscale", _p), ("a2_gscale", _p),
        ("num_experts", _i32), ("hidden", _i32), ("inter", _i32),
    ]


class MoEDebug(ctypes.Structure):
    _fields_ = [
        ("topk_ids", _p), ("topk_weights", _p), ("expert_offsets", _p),
        ("src_pair", _p), ("inv_pair", _p), ("a1_codes", _p), ("a1_sf", _p),
        ("c1", _p), ("h", _p), ("a2_codes", _p), ("a2_sf", _p), ("c2", _p),
        ("stage_events", ctypes.POINTER(_p)),
    ]


MOE_STAGES = ("route", "permute", "quantize_a1", "gemm1_w13", "gemm2_w2", "combine")


_SIGS = {
    "nvfp4_status_string": (ctypes.c_char_p, [_i32]),
    "nvfp4_abi_version": (_i32, []),
    "nvfp4_validate_scales": (_i32, [_p, _p, _i32, _p, _p, _p]),
    "nvfp4_quantize_experts": (_i32, [_p, _i64, _i32, _p, _i32, _i32, _p, _i32, _p, _p, _p, _p]),
    "nvfp4_quantize_pairs": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _p, _i32, _p]),
    "nvfp4_quantize_experts_fp16": (_i32, [_p, _i64, _i32, _p, _i32, _i32, _p, _i32, _p, _p, _p, _p]),
    "nvfp4_route_topk": (_i32, [_p, _i32, _i32, _i32, _p, _p, _p]),
    "nvfp4_permute": (_i32, [_p, _i32, _i32, _i32, _p, _p, _p, _p]),
    "nvfp4_expert_absmax": (_i32, [_p, _i64, _i32, _p, _i32, _p, _i32, _i32, _p, _p]),
    "nvfp4_calibrate_input_scales": (_i32, [_p, _i64, _i32, _p, _i32, _p, _i32, _i32, _p, _p, _p]),
    "nvfp4_selftest_conversions": (_i32, [_p, _p]),
    "nvfp4_moe_pack_weights": (_i32, [_i32, _p, _p, _i32, _i32, _i32, _p, _p, _p]),
    "nvfp4_moe_workspace_size": (_i32, [_i32, _i32, ctypes.POINTER(MoEWeights), ctypes.POINTER(ctypes.c_size_t)]),
    "nvfp4_moe_forward": (_i32, [ctypes.POINTER(MoEWeights), _p, _p, _i32, _i32, _p, _p, _p,
                                 ctypes.c_size_t, ctypes.POINTER(MoEDebug), _p]),
    "nvfp4_quantize_experts_mx": (_i32, [_p, _i64, _i32, _p, _i32, _i32, _p, _i32, _p, _p, _p, _p]),
    "nvfp4_quantize_pairs_mx": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _p, _i32, _p]),
    "nvfp4_moe_pack_weights_mx": (_i32, [_i32, _p, _p, _i32, _i32, _i32, _p, _p, _p]),
    "nvfp4_moe_forward_mx": (_i32, [ctypes.POINTER(MoEWeights), _p, _p, _i32, _i32, _p, _p, _p,
                                    ctypes.c_size_t, ctypes.POINTER(MoEDebug), _p]),
    "nvfp4_moe_workspace_size_w4a16": (_i32, [_i32, _i32, ctypes.POINTER(MoEWeights),
                                              ctypes.POINTER(ctypes.c_size_t)]),
    "nvfp4_moe_forward_w4a16": (_i32, [ctypes.POINTER(MoEWeights), _p, _p, _i32, _i32, _p, _p,
                                       _p, ctypes.c_size_t, ctypes.POINTER(MoEDebug), _p]),
    "nvfp4_moe_forward_noalloc": (_i32, [ctypes.POINTER(MoEWeights), _p, _p, _i32, _i32, _p, _p,
                                         ctypes.POINTER(MoEDebug), _p]),
}

EXPORTED = tuple(_SIGS)

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return _lib.nvfp4_status_string(status).decode()


def abi_version() -> int:
    return int(_lib.nvfp4_abi_version())


def _check(status: int, where: str) -> None:
    if status != OK:
        raise NVFP4Error(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# --- host -------------------------------------------------------------------

def validate_scales(input_scale: np.ndarray, written: Optional[np.ndarray] = None):
    """Host arrays in; returns (status, gscale or None, slot_status, num_bad)."""
    x = np.ascontiguousarray(input_scale, dtype=np.float32)
    E = x.size
    wr = None if written is None else np.ascontiguousarray(written, dtype=np.uint8)
    gs = np.full(E, np.nan, dtype=np.float32)
    st = np.full(E, -1, dtype=np.int32)
    nb = ctypes.c_int32(-1)
    status = _lib.nvfp4_validate_scales(
        x.ctypes.data, None if wr is None else wr.ctypes.data, E, gs.ctypes.data,
        st.ctypes.data, ctypes.addressof(nb))
    return status, (gs if status == OK else None), st, nb.value


# --- device -----------------------------------------------------------------

def quantize_experts(x, ldx: int, K: int, src_row, num_src_rows: int, P: int, expert_offsets,
                     num_experts: int, gscale, codes, sf, stream=None):
    _check(_lib.nvfp4_quantize_experts(_ptr(x), ldx, K, _ptr(src_row), num_src_rows, P,
                                       _ptr(expert_offsets), num_experts, _ptr(gscale),
                                       _ptr(codes), _ptr(sf), _stream(stream)),
           "nvfp4_quantize_experts")


def quantize_experts_fp16(x, ldx: int, K: int, src_row, num_src_rows: int, P: int,
                          expert_offsets, num_experts: int, gscale, codes, sf, stream=None):
    _check(_lib.nvfp4_quantize_experts_fp16(_ptr(x), ldx, K, _ptr(src_row), num_src_rows, P,
                                            _ptr(expert_offsets), num_experts, _ptr(gscale),
                                            _ptr(codes), _ptr(sf), _stream(stream)),
           "nvfp4_quantize_experts_fp16")


def quantize_pairs(x, ldx: int, num_rows: int, K: int, topk: int, expert_idx, dst_row,
                   num_experts: int, gscale, codes, sf, num_dst_rows: int, stream=None):
    _check(_lib.nvfp4_quantize_pairs(_ptr(x), ldx, num_rows, K, topk, _ptr(expert_idx),
                                     _ptr(dst_row), num_experts, _ptr(gscale), _ptr(codes),
                                     _ptr(sf), num_dst_rows, _stream(stream)),
           "nvfp4_quantize_pairs")


def route_topk(logits, num_tokens: int, num_experts: int, k: int, ids, weights, stream=None):
    _check(_lib.nvfp4_route_topk(_ptr(logits), num_tokens, num_experts, k, _ptr(ids),
                                 _ptr(weights), _stream(stream)), "nvfp4_route_topk")


def permute(ids, num_tokens: int, k: int, num_experts: int, expert_offsets, src_pair, inv_pair,
            stream=None):
    _check(_lib.nvfp4_permute(_ptr(ids), num_tokens, k, num_experts, _ptr(expert_offsets),
                              _ptr(src_pair), _ptr(inv_pair), _stream(stream)), "nvfp4_permute")


def expert_absmax(x, ldx: int, K: int, src, src_div: int, expert_offsets, num_experts: int,
                  num_rows: int, amax_out, stream=None):
    _check(_lib.nvfp4_expert_absmax(_ptr(x), ldx, K, _ptr(src), src_div, _ptr(expert_offsets),
                                    num_experts, num_rows, _ptr(amax_out), _stream(stream)),
           "nvfp4_expert_absmax")


def calibrate_input_scales(x, ldx: int, K: int, src, src_div: int, expert_offsets,
                           num_experts: int, num_rows: int, input_scale_out, written_out,
                           stream=None):
    _check(_lib.nvfp4_calibrate_input_scales(_ptr(x), ldx, K, _ptr(src), src_div,
                                             _ptr(expert_offsets), num_experts, num_rows,
                                             _ptr(input_scale_out), _ptr(written_out),
                                             _stream(stream)),
           "nvfp4_calibrate_input_scales")


def selftest_conversions(mismatches, stream=None):
    _check(_lib.nvfp4_selftest_conversions(_ptr(mismatches), _stream(stream)),
           "nvfp4_selftest_conversions")


def moe_pack_weights(projection: int, codes, sf, num_experts: int, hidden: int, inter: int,
                     codes_out, sf_out, stream=None):
    _check(_lib.nvfp4_moe_pack_weights(projection, _ptr(codes), _ptr(sf), num_experts, hidden,
                                       inter, _ptr(codes_out), _ptr(sf_out), _stream(stream)),
           "nvfp4_moe_pack_weights")


def moe_workspace_size(num_tokens: int, k: int, weights: MoEWeights) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.nvfp4_moe_workspace_size(num_tokens, k, ctypes.byref(weights), ctypes.byref(n)),
           "nvfp4_moe_workspace_size")
    return int(n.value)


def moe_forward(weights: MoEWeights, x, router_logits, num_tokens: int, k: int, residual, out,
                workspace, workspace_bytes: int, debug: Optional[MoEDebug] = None, stream=None):
    _check(_lib.nvfp4_moe_forward(ctypes.byref(weights), _ptr(x), _ptr(router_logits),
                                  num_tokens, k, _ptr(residual), _ptr(out), _ptr(workspace),
                                  workspace_bytes, None if debug is None else ctypes.byref(debug),
                                  _stream(stream)), "nvfp4_moe_forward")


def moe_workspace_size_w4a16(num_tokens: int, k: int, weights: MoEWeights) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.nvfp4_moe_workspace_size_w4a16(num_tokens, k, ctypes.byref(weights),
                                               ctypes.byref(n)),
           "nvfp4_moe_workspace_size_w4a16")
    return int(n.value)


def moe_forward_w4a16(weights: MoEWeights, x, router_logits, num_tokens: int, k: int, residual,
                      out, workspace, workspace_bytes: int, debug: Optional[MoEDebug] = None,
                      stream=None):
    _check(_lib.nvfp4_moe_forward_w4a16(ctypes.byref(weights), _ptr(x), _ptr(router_logits),
                                        num_tokens, k, _ptr(residual), _ptr(out),
                                        _ptr(workspace), workspace_bytes,
                                        None if debug is None else ctypes.byref(debug),
                                        _stream(stream)), "nvfp4_moe_forward_w4a16")


def quantize_experts_mx(x, ldx: int, K: int, src_row, num_src_rows: int, P: int,
                        expert_offsets, num_experts: int, gscale, codes, sf, stream=None):
    _check(_lib.nvfp4_quantize_experts_mx(_ptr(x), ldx, K, _ptr(src_row), num_src_rows, P,
                                          _ptr(expert_offsets), num_experts, _ptr(gscale),
                                          _ptr(codes), _ptr(sf), _stream(stream)),
           "nvfp4_quantize_experts_mx")


def quantize_pairs_mx(x, ldx: int, num_rows: int, K: int, topk: int, expert_idx, dst_row,
                      num_experts: int, gscale, codes, sf, num_dst_rows: int, stream=None):
    _check(_lib.nvfp4_quantize_pairs_mx(_ptr(x), ldx, num_rows, K, topk, _ptr(expert_idx),
                                        _ptr(dst_row), num_experts, _ptr(gscale), _ptr(codes),
                                        _ptr(sf), num_dst_rows, _stream(stream)),
           "nvfp4_quantize_pairs_mx")


def moe_pack_weights_mx(projection: int, codes, sf, num_experts: int, hidden: int, inter: int,
                        codes_out, sf_out, stream=None):
    _check(_lib.nvfp4_moe_pack_weights_mx(projection, _ptr(codes), _ptr(sf), num_experts, hidden,
                                          inter, _ptr(codes_out), _ptr(sf_out), _stream(stream)),
           "nvfp4_moe_pack_weights_mx")


def moe_forward_mx(weights: MoEWeights, x, router_logits, num_tokens: int, k: int, residual, out,
                   workspace, workspace_bytes: int, debug: Optional[MoEDebug] = None,
                   stream=None):
    _check(_lib.nvfp4_moe_forward_mx(ctypes.byref(weights), _ptr(x), _ptr(router_logits),
                                     num_tokens, k, _ptr(residual), _ptr(out), _ptr(workspace),
                                     workspace_bytes, None if debug is None else ctypes.byref(debug),
                                     _stream(stream)), "nvfp4_moe_forward_mx")


def moe_forward_noalloc(weights: MoEWeights, x, router_logits, num_tokens: int, k: int, residual,
                        out, debug: Optional[MoEDebug] = None, stream=None):
    _check(_lib.nvfp4_moe_forward_noalloc(ctypes.byref(weights), _ptr(x), _ptr(router_logits),
                                          num_tokens, k, _ptr(residual), _ptr(out),
                                          None if debug is None else ctypes.byref(debug),
                                          _stream(stream)), "nvfp4_moe_forward_noalloc")
