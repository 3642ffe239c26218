"""The 30-layer stack's load-time scale check, on the host: three seeded
corrupt expert slots are rejected by name before anything is uploaded or any
reciprocal is kept (the pages' missing-scale failure turned into a load
error).  Runs without a GPU."""
import numpy as np
import pytest

import synthetic as S


def test_stack_bad_scales_rejected_at_load():
    """The 30-layer stack's scale-validation case: three seeded corrupt slots
    (NaN, unwritten with a valid-looking stale value, unwritten with -inf
    bits) are named exactly and nothing is uploaded."""
    from nvfp4_w4a4_expert_amd import moe as M
    w = S.WORKLOADS["stack"]
    s13 = np.full(w.E, 1.0 / 2688, dtype=np.float32)
    s2 = np.full(w.E, 1.0 / 2688, dtype=np.float32)
    wr13 = np.ones(w.E, dtype=np.uint8)
    wr2 = np.ones(w.E, dtype=np.uint8)
    for proj, e, kind in S.bad_scale_slots(w):
        s, wr = (s13, wr13) if proj == "w13" else (s2, wr2)
        if kind == "nan":
            s[e] = np.nan
        elif kind == "unwritten_garbage":
            s[e] = np.float32(0.25)
            wr[e] = 0
        else:
            s[e] = -np.inf
            wr[e] = 0
    bad13 = sorted(e for p, e, _ in S.bad_scale_slots(w) if p == "w13")
    bad2 = sorted(e for p, e, _ in S.bad_scale_slots(w) if p == "w2")
    with pytest.raises(M.BadScaleError) as ei:
        M.NVFP4MoELayer(None, None, None, None, None, None, s13, s2, wr13, wr2, device="meta")
    assert ei.value.projection == "w13" and ei.value.bad_slots == bad13
    s13_ok = np.full(w.E, 1.0 / 2688, dtype=np.float32)
    with pytest.raises(M.BadScaleError) as ei:
        M.NVFP4MoELayer(None, None, None, None, None, None, s13_ok, s2, None, wr2, device="meta")
    assert ei.value.projection == "w2" and ei.value.bad_slots == bad2
