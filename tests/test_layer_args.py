"""NVFP4MoELayer.forward's argument checks (CPU).  The checks run before any
pointer reaches the library, so a layer object whose tensors live on the CPU
exercises them without a GPU: every malformed call raises ValueError."""
import pytest
import torch

from nvfp4_w4a4_expert_amd.moe import NVFP4MoELayer

E, H, T = 8, 64, 5


def _layer():
    lay = NVFP4MoELayer.__new__(NVFP4MoELayer)
    lay.E, lay.H, lay.I = E, H, 32
    lay.w13 = torch.zeros(E, 64, H // 2, dtype=torch.uint8)
    return lay


def _ok():
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    return dict(x=x, logits=torch.zeros(T, E, dtype=torch.float32), k=2,
                residual=torch.zeros_like(x), out=torch.zeros_like(x))


def test_well_formed_call_passes():
    a = _ok()
    _layer()._check_call(a["x"], a["logits"], a["k"], a["residual"], a["out"])
    _layer()._check_call(a["x"], a["logits"], E, None, None)


@pytest.mark.parametrize("field,value", [
    ("x", torch.zeros(T, H, dtype=torch.float32)),                 # dtype
    ("x", torch.zeros(T, H + 16, dtype=torch.bfloat16)),           # width
    ("x", torch.zeros(H, T, dtype=torch.bfloat16).t()),            # not contiguous
    ("x", torch.zeros(T * H, dtype=torch.bfloat16)),               # rank
    ("logits", torch.zeros(T, E, dtype=torch.bfloat16)),           # dtype
    ("logits", torch.zeros(T - 1, E, dtype=torch.float32)),        # rows
    ("logits", torch.zeros(T, E + 1, dtype=torch.float32)),        # experts
    ("logits", torch.zeros(E, T, dtype=torch.float32).t()),        # not contiguous
    ("residual", torch.zeros(T - 1, H, dtype=torch.bfloat16)),     # too few rows
    ("residual", torch.zeros(T, H, dtype=torch.float32)),          # dtype
    ("out", torch.zeros(T - 1, H, dtype=torch.bfloat16)),          # too few rows
    ("out", torch.zeros(2 * T, H, dtype=torch.bfloat16)[::2]),     # not contiguous
    ("k", 0), ("k", E + 1), ("k", 2.0), ("k", None),
])
def test_malformed_call_raises(field, value):
    a = _ok()
    a[field] = value
    with pytest.raises(ValueError):
        _layer()._check_call(a["x"], a["logits"], a["k"], a["residual"], a["out"])


def test_tensor_on_another_device_raises():
    a = _ok()
    lay = _layer()
    lay.w13 = torch.zeros(1, dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError):
        lay._check_call(a["x"], a["logits"], a["k"], None, None)
