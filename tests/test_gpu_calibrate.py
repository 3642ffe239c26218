"""GPU parity of the calibration pass (nvfp4_calibrate_input_scales): the
per-expert scales fl32(amax / 2688) and the written mask, bit-exact against
the oracle's calibrator, and its coverage report feeding the load-time check
(page 3, "ROOT CAUSE": experts without calibration tokens)."""
import numpy as np
import pytest

import synthetic as S
from oracle import moe as OM

pytestmark = pytest.mark.gpu


def _calibrate(x_bits, logits, k):
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    T, E = logits.shape
    H = x_bits.shape[1]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    L.route_topk(torch.from_numpy(np.ascontiguousarray(logits)).cuda(), T, E, k, ids, wts)
    L.permute(ids, T, k, E, off, src, inv)
    scale = torch.full((E,), 7.0, dtype=torch.float32, device="cuda")
    written = torch.full((E,), 9, dtype=torch.uint8, device="cuda")
    L.calibrate_input_scales(M.bf16_tensor(x_bits), H, H, src, k, off, E, T * k, scale, written)
    torch.cuda.synchronize()
    return scale.cpu().numpy(), written.cpu().numpy()


def test_calibration_matches_oracle_full_coverage():
    w = S.WORKLOADS["decode"]
    xc, lc = S.calibration_batch(w)
    scale, written = _calibrate(xc, lc, w.k)
    rs, rw = OM.calibrate_input_scale(xc, lc, w.k, w.E)
    assert np.array_equal(written, rw) and written.all()
    assert np.array_equal(scale.view(np.uint32), rs.view(np.uint32))


def test_calibration_coverage_report_feeds_the_load_check():
    """A 512-token batch under the stack's Zipf router (8 experts masked)
    leaves experts without rows: they come back unwritten with NaN scales, and
    the load-time check rejects exactly those slots as unwritten."""
    from nvfp4_w4a4_expert_amd import _lib as L
    w = S.WORKLOADS["stack"]
    x = S.activations(w, layer=3, tokens=512)
    lg = S.router_logits(w, layer=3, tokens=512)
    scale, written = _calibrate(x, lg, w.k)
    rs, rw = OM.calibrate_input_scale(x, lg, w.k, w.E)
    assert np.array_equal(written, rw)
    missing = np.nonzero(rw == 0)[0]
    assert missing.size >= 8
    assert np.isnan(scale[missing]).all()
    ok = rw == 1
    assert np.array_equal(scale[ok].view(np.uint32), rs[ok].view(np.uint32))
    st, _, slots, nbad = L.validate_scales(scale, written)
    assert st == L.ERR_BAD_SCALE and nbad == missing.size
    assert np.array_equal(np.nonzero(slots != L.SLOT_OK)[0], missing)
    assert (slots[missing] == L.SLOT_UNWRITTEN).all()
