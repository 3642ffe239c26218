"""The C-ABI library loads on a machine without a GPU, exports every symbol
that include/nvfp4_moe.h declares, and its host-only paths work: the
load-time scale check (all rejection reasons, no output on failure) and
argument validation that returns before anything is enqueued.  No compute
call touches a device here."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import moe as OM

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_moe.h")


def _lib():
    from nvfp4_w4a4_expert_amd import _lib as L
    return L


def _declared_symbols():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"NVFP4_API\s+[\w\s\*]+?\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = _declared_symbols()
    for name in ["nvfp4_validate_scales", "nvfp4_quantize_experts", "nvfp4_moe_forward",
                 "nvfp4_moe_workspace_size", "nvfp4_route_topk", "nvfp4_permute",
                 "nvfp4_expert_absmax", "nvfp4_status_string", "nvfp4_abi_version",
                 "nvfp4_selftest_conversions", "nvfp4_moe_pack_weights",
                 "nvfp4_quantize_experts_fp16", "nvfp4_calibrate_input_scales",
                 "nvfp4_moe_forward_w4a16", "nvfp4_moe_workspace_size_w4a16",
                 "nvfp4_quantize_experts_mx", "nvfp4_moe_pack_weights_mx",
                 "nvfp4_moe_forward_mx", "nvfp4_moe_forward_noalloc",
                 "nvfp4_quantize_pairs", "nvfp4_quantize_pairs_mx"]:
        assert name in syms


def test_library_exports_every_declared_symbol():
    L = _lib()
    cdll = ctypes.CDLL(L.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(cdll, name), name
    assert set(_declared_symbols()) == set(L.EXPORTED)


def test_abi_version_and_status_strings():
    L = _lib()
    assert L.abi_version() == 6
    for s in range(7):
        assert L.status_string(s)
    assert "unknown" in L.status_string(99)


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def test_validator_matches_oracle_reasons():
    L = _lib()
    vals = np.array([0.5, np.nan, np.inf, -np.inf, 0.0, -0.0, -2.0, _f32(0x00000001),
                     _f32(0x00200000), _f32(0x00400000), 3e-3, 1.0, _f32(0x7FC00001),
                     _f32(0xFF800001)], dtype=np.float32)
    written = np.ones(vals.size, dtype=np.uint8)
    written[11] = 0
    st, gs, slots, nb = L.validate_scales(vals, written)
    ok, ogs, oslots = OM.validate_scales(vals, written)
    assert st == L.ERR_BAD_SCALE and gs is None and not ok
    assert slots.tolist() == oslots.tolist()
    assert nb == int(np.count_nonzero(oslots))


def test_validator_writes_nothing_on_failure():
    L = _lib()
    vals = np.array([1.0, np.nan], dtype=np.float32)
    out = np.full(2, 7.0, dtype=np.float32)
    status = L._lib.nvfp4_validate_scales(vals.ctypes.data, None, 2, out.ctypes.data, None, None)
    assert status == L.ERR_BAD_SCALE and out.tolist() == [7.0, 7.0]


def test_validator_success_is_fp32_reciprocal():
    L = _lib()
    rng = np.random.default_rng(0)
    vals = np.exp(rng.uniform(-80, 80, 1000)).astype(np.float32)
    vals = vals[np.isfinite(np.float32(1) / vals) & (vals > 0)]
    st, gs, slots, nb = L.validate_scales(vals)
    ok, ogs, _ = OM.validate_scales(vals)
    assert st == L.OK and ok and nb == 0
    assert np.array_equal(gs.view(np.uint32), ogs.view(np.uint32))


def test_validator_rejects_bad_args():
    L = _lib()
    assert L._lib.nvfp4_validate_scales(None, None, 4, None, None, None) == L.ERR_INVALID_ARG
    x = np.ones(1, dtype=np.float32)
    assert L._lib.nvfp4_validate_scales(x.ctypes.data, None, 0, None, None, None) == L.ERR_INVALID_ARG


def test_host_argument_checks_return_before_enqueue():
    L = _lib()
    f = L._lib
    # K not a multiple of 16 (both forms)
    assert f.nvfp4_quantize_pairs(16, 24, 1, 24, 1, None, None, 1, None, 16, 16, 1, None) \
        == L.ERR_INVALID_ARG
    assert f.nvfp4_quantize_experts(16, 24, 24, 16, 4, 1, 16, 1, None, 16, 16, None) \
        == L.ERR_INVALID_ARG
    # misaligned x
    assert f.nvfp4_quantize_pairs(8, 16, 1, 16, 1, None, None, 1, None, 16, 16, 1, None) \
        == L.ERR_INVALID_ARG
    assert f.nvfp4_quantize_experts(8, 16, 16, 16, 4, 1, 16, 1, None, 16, 16, None) \
        == L.ERR_INVALID_ARG
    # the gather form needs the expert offsets
    assert f.nvfp4_quantize_experts(16, 16, 16, 16, 4, 1, None, 1, None, 16, 16, None) \
        == L.ERR_INVALID_ARG
    # zero rows is a no-op that never touches the device
    assert f.nvfp4_quantize_pairs(None, 16, 0, 16, 1, None, None, 1, None, None, None, 0, None) \
        == L.OK
    assert f.nvfp4_quantize_experts(None, 16, 16, None, 0, 0, None, 1, None, None, None, None) \
        == L.OK
    # router: k > E, E too large
    assert f.nvfp4_route_topk(16, 4, 4, 5, 16, 16, None) == L.ERR_INVALID_ARG
    assert f.nvfp4_route_topk(16, 4, 2000, 8, 16, 16, None) == L.ERR_UNSUPPORTED
    assert f.nvfp4_route_topk(None, 0, 8, 2, None, None, None) == L.OK
    # forward: missing weights, zero tokens, missing workspace
    w = L.MoEWeights()
    assert f.nvfp4_moe_forward(ctypes.byref(w), None, None, 4, 2, None, None, None, 0, None, None) \
        == L.ERR_INVALID_ARG
    fake = 4096
    w = L.MoEWeights(*([fake] * 10), 4, 256, 128)
    assert f.nvfp4_moe_forward(ctypes.byref(w), None, None, 0, 2, None, None, None, 0, None, None) \
        == L.OK
    assert f.nvfp4_moe_forward(ctypes.byref(w), fake, fake, 4, 2, None, fake, None, 0, None, None) \
        == L.ERR_WORKSPACE
    w.hidden = 200   # not a multiple of 16
    assert f.nvfp4_moe_forward(ctypes.byref(w), fake, fake, 4, 2, None, fake, fake, 1 << 30, None,
                               None) == L.ERR_INVALID_ARG
    w.hidden = 256
    w.inter = 96     # multiple of 16 but not of the 64-column GEMM1 tile
    assert f.nvfp4_moe_forward(ctypes.byref(w), fake, fake, 4, 2, None, fake, fake, 1 << 30, None,
                               None) == L.ERR_UNSUPPORTED


def test_workspace_size_grows_with_tokens():
    L = _lib()
    w = L.MoEWeights(*([0] * 10), 128, 2816, 704)
    a = L.moe_workspace_size(16, 8, w)
    b = L.moe_workspace_size(4096, 8, w)
    assert 0 < a < b
    P = 4096 * 8
    assert b >= P * (2816 // 2 + 2816 // 16 + 704 // 2 + 704 // 16 + 2816 * 4 + 16)


def test_w4a16_host_checks_need_no_activation_scales():
    L = _lib()
    f = L._lib
    fake = 4096
    # weights present, all four activation-scale pointers NULL
    w = L.MoEWeights(*([fake] * 6), 0, 0, 0, 0, 4, 256, 128)
    # the W4A4 forward requires them, the weight-only forward does not
    assert f.nvfp4_moe_forward(ctypes.byref(w), fake, fake, 4, 2, None, fake, fake, 1 << 30,
                               None, None) == L.ERR_INVALID_ARG
    assert f.nvfp4_moe_forward_w4a16(ctypes.byref(w), fake, fake, 4, 2, None, fake, None, 0,
                                     None, None) == L.ERR_WORKSPACE
    assert f.nvfp4_moe_forward_w4a16(ctypes.byref(w), None, None, 0, 2, None, None, None, 0,
                                     None, None) == L.OK
    w13_missing = L.MoEWeights(0, *([fake] * 5), 0, 0, 0, 0, 4, 256, 128)
    assert f.nvfp4_moe_forward_w4a16(ctypes.byref(w13_missing), fake, fake, 4, 2, None, fake,
                                     fake, 1 << 30, None, None) == L.ERR_INVALID_ARG
    w.inter = 96
    assert f.nvfp4_moe_forward_w4a16(ctypes.byref(w), fake, fake, 4, 2, None, fake, fake,
                                     1 << 30, None, None) == L.ERR_UNSUPPORTED


def test_w4a16_workspace_holds_bf16_h_instead_of_codes():
    L = _lib()
    w = L.MoEWeights(*([0] * 10), 128, 2816, 704)
    P = 4096 * 8
    b = L.moe_workspace_size_w4a16(4096, 8, w)
    assert b >= P * (704 * 2 + 2816 * 4 + 16)
    assert b < L.moe_workspace_size(4096, 8, w) + P * 704 * 2
    assert b - P * (704 * 2 + 2816 * 4 + 16) < 8 * 256 + 129 * 4


def test_ue8m0_mode_host_checks():
    L = _lib()
    f = L._lib
    fake = 4096
    # hidden must be a multiple of 256 in the UE8M0 mode (w13 K step), 128 otherwise
    assert f.nvfp4_moe_pack_weights_mx(0, fake, fake, 8, 640, 320, 2 * fake, 2 * fake, None) \
        == L.ERR_UNSUPPORTED
    w = L.MoEWeights(*([fake] * 10), 8, 640, 320)
    assert f.nvfp4_moe_forward_mx(ctypes.byref(w), fake, fake, 4, 2, None, fake, fake, 1 << 30,
                                  None, None) == L.ERR_UNSUPPORTED
    # K not a multiple of 32 in the UE8M0 quantiser
    assert f.nvfp4_quantize_pairs_mx(16, 48, 1, 48, 1, None, None, 1, None, 16, 16, 1, None) \
        == L.ERR_INVALID_ARG
    assert f.nvfp4_quantize_experts_mx(16, 48, 48, 16, 4, 1, 16, 1, None, 16, 16, None) \
        == L.ERR_INVALID_ARG
    # the activation scales are required, as in the E4M3 mode
    w = L.MoEWeights(*([fake] * 6), 0, 0, 0, 0, 4, 256, 128)
    assert f.nvfp4_moe_forward_mx(ctypes.byref(w), fake, fake, 4, 2, None, fake, fake, 1 << 30,
                                  None, None) == L.ERR_INVALID_ARG


def test_bad_scales_are_rejected_before_upload():
    from nvfp4_w4a4_expert_amd import moe as M
    import synthetic as S
    w = S.WORKLOADS["tiny"]
    s = np.full(w.E, 1.0 / 2688, dtype=np.float32)
    s[2] = np.nan
    with pytest.raises(M.BadScaleError) as ei:
        # weight arguments are never touched: the check runs first
        M.NVFP4MoELayer(None, None, None, None, None, None, s, s.copy(), device="meta")
    assert ei.value.bad_slots == [2] and ei.value.projection == "w13"
    wr = np.ones(w.E, dtype=np.uint8)
    wr[1] = 0
    with pytest.raises(M.BadScaleError) as ei:
        M.NVFP4MoELayer(None, None, None, None, None, None, np.ones(w.E), np.ones(w.E),
                        written13=None, written2=wr, device="meta")
    assert ei.value.bad_slots == [1] and ei.value.projection == "w2"


def test_noalloc_forward_rejects_before_touching_the_device():
    """The allocation-free forward checks its arguments and the size of its
    fixed buffer on the host before any HIP call."""
    L = _lib()
    f = L._lib
    w = L.MoEWeights()
    assert f.nvfp4_moe_forward_noalloc(ctypes.byref(w), None, None, 4, 2, None, None, None,
                                       None) == L.ERR_INVALID_ARG
    assert f.nvfp4_moe_forward_noalloc(None, None, None, 4, 2, None, None, None,
                                       None) == L.ERR_INVALID_ARG
    fake = 4096
    w = L.MoEWeights(*([fake] * 10), 128, 2816, 704)
    need = L.moe_workspace_size(1024, 8, w)
    assert need > L.NOALLOC_SCRATCH_BYTES
    assert f.nvfp4_moe_forward_noalloc(ctypes.byref(w), fake, fake, 1024, 8, None, fake, None,
                                       None) == L.ERR_TOO_LARGE
    assert L.moe_workspace_size(512, 8, w) <= L.NOALLOC_SCRATCH_BYTES
    assert "fixed buffer" in L.status_string(L.ERR_TOO_LARGE)
