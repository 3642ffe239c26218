"""One NVFP4 W4A4 routed-expert MoE layer on the GPU.

``NVFP4MoELayer`` holds one layer's checkpoint fields on the device and runs
``nvfp4_moe_forward``.  Construction performs the load-time scale check
(``nvfp4_validate_scales``) on the host before any reciprocal is kept: a
layer whose per-expert input scales are unwritten, NaN, infinite,
non-positive or too small to invert is rejected with :class:`BadScaleError`
and nothing is uploaded.

``quantize_expert_weights`` and ``calibrate_layer`` produce a layer from bf16
weights with the library's own kernels (static weight quantisation and
activation-scale calibration); they stand in for an offline exporter.
"""
from __future__ import annotations

import operator
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib

class BadScaleError(ValueError):
    """Per-expert activation scales failed the load-time check."""

    def __init__(self, projection: str, slot_status: np.ndarray):
        self.projection = projection
        self.slot_status = slot_status
        self.bad_slots = [int(e) for e in np.nonzero(slot_status != _lib.SLOT_OK)[0]]
        super().__init__(f"{projection}_input_scale: {len(self.bad_slots)} bad expert slot(s) "
                         f"{self.bad_slots}")


def _dev_u8(a, device):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def _dev_f32(a, device):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device`."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class NVFP4MoELayer:
    """Device-resident NVFP4 MoE layer (W4A4: activations quantised per expert).

    Weight tensors may be numpy arrays (uploaded) or device tensors, in the
    checkpoint layout: w13 [E, 2I, H/2] u8, w13_sf [E, 2I, H/16] u8,
    w13_scale2 [E] f32, w2 [E, H, I/2] u8, w2_sf [E, H, I/16] u8, w2_scale2
    [E] f32.  The input scales and `written` masks are host arrays; they are
    checked first.  Codes and block scales are then converted once into the
    kernel layout (nvfp4_moe_pack_weights); the inputs are left untouched.
    """

    def __init__(self, w13, w13_sf, w13_scale2, w2, w2_sf, w2_scale2,
                 w13_input_scale, w2_input_scale, written13=None, written2=None,
                 device="cuda"):
        s13 = np.ascontiguousarray(w13_input_scale, dtype=np.float32)
        s2 = np.ascontiguousarray(w2_input_scale, dtype=np.float32)
        st, gs1, slots, _ = _lib.validate_scales(s13, written13)
        if st != _lib.OK:
            raise BadScaleError("w13", slots)
        st, gs2, slots, _ = _lib.validate_scales(s2, written2)
        if st != _lib.OK:
            raise BadScaleError("w2", slots)
        self._load_weights(w13, w13_sf, w13_scale2, w2, w2_sf, w2_scale2, device)
        self.w13_input_scale = _dev_f32(s13, device)
        self.w2_input_scale = _dev_f32(s2, device)
        self.a1_gscale = _dev_f32(gs1, device)
        self.a2_gscale = _dev_f32(gs2, device)

    def _load_weights(self, w13, w13_sf, w13_scale2, w2, w2_sf, w2_scale2, device):
        up8 = (lambda a: a if isinstance(a, torch.Tensor) else _dev_u8(a, device))
        up32 = (lambda a: a if isinstance(a, torch.Tensor) else _dev_f32(a, device))
        w13, w13_sf, w2, w2_sf = up8(w13), up8(w13_sf), up8(w2), up8(w2_sf)
        self.E = int(w13.shape[0])
        self.I = int(w13.shape[1]) // 2
        self.H = int(w13.shape[2]) * 2
        # load-time layout conversion into the grouped GEMMs' kernel layout
        self.w13, self.w13_sf = torch.empty_like(w13), torch.empty_like(w13_sf)
        self.w2, self.w2_sf = torch.empty_like(w2), torch.empty_like(w2_sf)
        self._pack(0, w13, w13_sf, self.E, self.H, self.I, self.w13, self.w13_sf)
        self._pack(1, w2, w2_sf, self.E, self.H, self.I, self.w2, self.w2_sf)
        self.w13_scale2, self.w2_scale2 = up32(w13_scale2), up32(w2_scale2)
        self.device = device
        self._ws = None

    def weights(self) -> _lib.MoEWeights:
        def ptr(t):
            return 0 if t is None else t.data_ptr()
        return _lib.MoEWeights(
            self.w13.data_ptr(), self.w13_sf.data_ptr(), self.w13_scale2.data_ptr(),
            self.w2.data_ptr(), self.w2_sf.data_ptr(), self.w2_scale2.data_ptr(),
            ptr(self.w13_input_scale), ptr(self.w2_input_scale),
            ptr(self.a1_gscale), ptr(self.a2_gscale), self.E, self.H, self.I)

    _workspace_size = staticmethod(_lib.moe_workspace_size)
    _forward = staticmethod(_lib.moe_forward)
    _pack = staticmethod(_lib.moe_pack_weights)
    _sf_block = 16                  # elements per block scale
    _debug_names = ("topk_ids", "topk_weights", "expert_offsets", "src_pair", "inv_pair",
                    "a1_codes", "a1_sf", "c1", "h", "a2_codes", "a2_sf", "c2")

    def _torch_stream(self, stream):
        """The torch stream a call runs on (torch's current stream when None;
        an integer is a raw HIP stream handle on the layer's device)."""
        if stream is None:
            return torch.cuda.current_stream(self.w13.device)
        if isinstance(stream, int):
            return torch.cuda.ExternalStream(stream, device=self.w13.device)
        return stream

    def workspace(self, T: int, k: int, stream=None) -> torch.Tensor:
        """The workspace for a call on `stream`.  Each stream has its own
        buffer, allocated while that stream is current, so the caching
        allocator orders its reuse after the work queued on that stream; calls
        on different streams never share a buffer."""
        n = self._workspace_size(T, k, self.weights())
        s = self._torch_stream(stream)
        if self._ws is None:
            self._ws = {}
        ws = self._ws.get(s.cuda_stream)
        if ws is None or ws.numel() < n:
            with torch.cuda.stream(s):
                ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.w13.device)
            self._ws[s.cuda_stream] = ws
        return ws

    def _check_call(self, x, logits, k, residual, out):
        """Shapes, dtypes, layout and device of a forward's tensors: every
        pointer the library receives must cover the rows it reads or writes."""
        dev = self.w13.device

        def need(ok, msg):
            if not ok:
                raise ValueError(msg)

        def on_dev(t):
            return isinstance(t, torch.Tensor) and t.device == dev and t.is_contiguous()

        need(on_dev(x) and x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[1] == self.H,
             f"x must be a contiguous bf16 [T, {self.H}] tensor on {dev}")
        T = int(x.shape[0])
        need(on_dev(logits) and logits.dtype == torch.float32 and
             tuple(logits.shape) == (T, self.E),
             f"logits must be a contiguous fp32 [{T}, {self.E}] tensor on {dev}")
        try:
            k = operator.index(k)
        except TypeError:
            k = None
        need(k is not None and 1 <= k <= self.E, f"k must be an integer in [1, {self.E}]")
        for name, t in (("residual", residual), ("out", out)):
            if t is not None:
                need(on_dev(t) and t.dtype == torch.bfloat16 and t.shape == x.shape,
                     f"{name} must be a contiguous bf16 [{T}, {self.H}] tensor on {dev}")

    def forward(self, x: torch.Tensor, logits: torch.Tensor, k: int,
                residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                debug: bool = False, stream=None):
        """x bf16 [T, H], logits fp32 [T, E] -> out bf16 [T, H] (and a dict of
        intermediates when debug=True).  Raises ValueError for tensors of the
        wrong dtype, shape, layout or device.  The call is queued on `stream`
        (torch's current stream when None) and returns without waiting."""
        self._check_call(x, logits, k, residual, out)
        k = operator.index(k)
        T = int(x.shape[0])
        if out is None:
            out = torch.empty_like(x)
        ws = self.workspace(T, k, stream)
        w = self.weights()
        dbg = None
        bufs = None
        if debug:
            P, H, I, E = T * k, self.H, self.I, self.E
            dev = self.w13.device
            shapes = dict(
                topk_ids=((T, k), torch.int32), topk_weights=((T, k), torch.float32),
                expert_offsets=((E + 1,), torch.int32), src_pair=((P,), torch.int32),
                inv_pair=((P,), torch.int32), a1_codes=((P, H // 2), torch.uint8),
                a1_sf=((P, H // self._sf_block), torch.uint8), c1=((P, 2 * I), torch.float32),
                h=((P, I), torch.int16), a2_codes=((P, I // 2), torch.uint8),
                a2_sf=((P, I // self._sf_block), torch.uint8), c2=((P, H), torch.float32))
            with torch.cuda.stream(self._torch_stream(stream)):
                bufs = {name: torch.empty(shapes[name][0], dtype=shapes[name][1], device=dev)
                        for name in self._debug_names}
            dbg = _lib.MoEDebug(**{name: t.data_ptr() for name, t in bufs.items()})
        self._forward(w, x, logits, T, k, residual, out, ws, ws.numel(), dbg, stream)
        return (out, bufs) if debug else out


class NVFP4MXMoELayer(NVFP4MoELayer):
    """The W4A4 layer with UE8M0 (power-of-two) block scales per 32 elements
    (page 3, "NVFP4" section: the quantiser template's UE8M0_SF switch).
    Same arguments as NVFP4MoELayer, with w13_sf [E, 2I, H/32] and w2_sf
    [E, H, I/32] UE8M0 codes (quantize_expert_weights(..., mx=True)); both
    grouped GEMMs run on the scaled FP4 matrix instruction."""

    _forward = staticmethod(_lib.moe_forward_mx)
    _pack = staticmethod(_lib.moe_pack_weights_mx)
    _sf_block = 32


class NVFP4W4A16MoELayer(NVFP4MoELayer):
    """Weight-only (W4A16) execution of the same NVFP4 expert weights
    (page 3, "Kernel Backend": the Marlin backend runs W4A16 and consumes no
    activation input_scale).  Activations stay bf16; no activation scale is
    taken, checked or read, so a checkpoint whose input scales fail the
    load-time check still runs here.  Same weight arguments as NVFP4MoELayer.
    """

    def __init__(self, w13, w13_sf, w13_scale2, w2, w2_sf, w2_scale2, device="cuda"):
        self._load_weights(w13, w13_sf, w13_scale2, w2, w2_sf, w2_scale2, device)
        self.w13_input_scale = self.w2_input_scale = None
        self.a1_gscale = self.a2_gscale = None

    @classmethod
    def sharing(cls, layer: NVFP4MoELayer) -> "NVFP4W4A16MoELayer":
        """A weight-only view of an existing layer's packed weights (no copy)."""
        obj = cls.__new__(cls)
        for name in ("E", "H", "I", "w13", "w13_sf", "w13_scale2", "w2", "w2_sf", "w2_scale2",
                     "device"):
            setattr(obj, name, getattr(layer, name))
        obj.w13_input_scale = obj.w2_input_scale = None
        obj.a1_gscale = obj.a2_gscale = None
        obj._ws = None
        return obj

    _workspace_size = staticmethod(_lib.moe_workspace_size_w4a16)
    _forward = staticmethod(_lib.moe_forward_w4a16)
    _debug_names = ("topk_ids", "topk_weights", "expert_offsets", "src_pair", "inv_pair",
                    "c1", "h", "c2")


# --- producing a layer with the library's kernels ----------------------------

def quantize_expert_weights(w: torch.Tensor, stream=None, mx: bool = False):
    """Static NVFP4 quantisation of bf16 expert weights [E, N, K] on the GPU,
    with the library's kernels: weight_scale_2[e] = fl32(max|W[e]| / 2688)
    (the calibration pass over each expert's N rows), the load-time check and
    reciprocal of it (SFScaleVal), then the per-expert quantiser over the
    expert-grouped rows (UE8M0 scales per 32 elements when mx).
    Returns (codes, sf, scale2) tensors."""
    E, N, K = (int(s) for s in w.shape)
    dev = w.device
    flat = w.reshape(E * N, K)
    offsets = torch.arange(0, E * N + 1, N, dtype=torch.int32, device=dev)
    scale2 = torch.empty(E, dtype=torch.float32, device=dev)
    written = torch.empty(E, dtype=torch.uint8, device=dev)
    _lib.calibrate_input_scales(flat, K, K, None, 1, offsets, E, E * N, scale2, written, stream)
    st, gs, slots, _ = _lib.validate_scales(scale2.cpu().numpy(), written.cpu().numpy())
    if st != _lib.OK:
        raise BadScaleError("weight_scale_2", slots)
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((E, N, K // (32 if mx else 16)), dtype=torch.uint8, device=dev)
    quant = _lib.quantize_experts_mx if mx else _lib.quantize_experts
    quant(flat, K, K, None, E * N, E * N, offsets, E, torch.from_numpy(gs).to(dev), codes, sf,
          stream)
    return codes, sf, scale2


@dataclass
class Calibration:
    w13_input_scale: np.ndarray
    w2_input_scale: np.ndarray
    written13: np.ndarray
    written2: np.ndarray


def calibrate_layer(w13c, w13s, w13s2, w2c, w2s, w2s2, x_cal: torch.Tensor,
                    logits_cal: torch.Tensor, k: int, mx: bool = False) -> Calibration:
    """Per-expert activation scales from a calibration batch, with the
    library's calibration pass (nvfp4_calibrate_input_scales):
    w13_input_scale = fl32(amax|x| / 2688) over the rows routed to each
    expert; w2_input_scale = fl32(amax|h| / 2688) over the same rows, where h
    is the layer's own SiLU(gate)*up (which does not depend on the a2 scale).
    Experts without calibration rows stay unwritten (NaN, written 0).  mx:
    the weights are in the UE8M0 mode and h comes from that layer."""
    dev = x_cal.device
    Tc, H = (int(s) for s in x_cal.shape)
    E = int(w13c.shape[0])
    I = int(w13c.shape[1]) // 2
    P = Tc * k
    ids = torch.empty((Tc, k), dtype=torch.int32, device=dev)
    wts = torch.empty((Tc, k), dtype=torch.float32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    src = torch.empty(P, dtype=torch.int32, device=dev)
    inv = torch.empty(P, dtype=torch.int32, device=dev)
    _lib.route_topk(logits_cal, Tc, E, k, ids, wts)
    _lib.permute(ids, Tc, k, E, offsets, src, inv)
    s13_d = torch.empty(E, dtype=torch.float32, device=dev)
    written_d = torch.empty(E, dtype=torch.uint8, device=dev)
    _lib.calibrate_input_scales(x_cal, H, H, src, k, offsets, E, P, s13_d, written_d)
    s13 = s13_d.cpu().numpy()
    written = written_d.cpu().numpy()
    # h does not depend on a2_gscale: run the layer with placeholder unit
    # a2 scales, restricted to the written slots, and read h back.
    ones = np.ones(E, dtype=np.float32)
    s13_run = np.where(written == 1, s13, np.float32(1.0)).astype(np.float32)
    cls = NVFP4MXMoELayer if mx else NVFP4MoELayer
    layer = cls(w13c, w13s, w13s2, w2c, w2s, w2s2, s13_run, ones, device=dev)
    _, dbg = layer.forward(x_cal, logits_cal, k, debug=True)
    s2_d = torch.empty(E, dtype=torch.float32, device=dev)
    written2_d = torch.empty(E, dtype=torch.uint8, device=dev)
    _lib.calibrate_input_scales(dbg["h"], I, I, None, 1, dbg["expert_offsets"], E, P, s2_d,
                                written2_d)
    return Calibration(s13, s2_d.cpu().numpy(), written, written2_d.cpu().numpy())
