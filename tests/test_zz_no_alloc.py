"""GPU test of nvfp4_moe_forward_noalloc, the forward that allocates nothing
(its workspace is the library's static per-device buffer): two calls in a
row through the C ABI, the second with a smaller batch, each compared with
nvfp4_moe_forward on a caller-allocated workspace.  The two run the same
kernels, so the outputs and every dumped intermediate must be bit-identical.
Also: a batch too large for the buffer is refused and leaves the output
untouched."""
import ctypes

import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu

E, H, I, K_TOP = 128, 2816, 704, 8


def _layer(torch):
    """An NVFP4 layer of the decode/prefill shape with seeded random codes and
    valid E4M3 block scales (no oracle needed: the reference here is the
    workspace forward)."""
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    rng = np.random.default_rng(2024)
    w13 = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w13s = rng.integers(0x28, 0x40, (E, 2 * I, H // 16), dtype=np.uint8)
    w2s = rng.integers(0x28, 0x40, (E, H, I // 16), dtype=np.uint8)
    s2a = np.full(E, 2.0 ** -9, dtype=np.float32)
    s2b = np.full(E, 2.0 ** -10, dtype=np.float32)
    in13 = (rng.uniform(1.0, 2.0, E) / 600).astype(np.float32)
    in2 = (rng.uniform(1.0, 2.0, E) / 2000).astype(np.float32)
    return M.NVFP4MoELayer(w13, w13s, s2a, w2, w2s, s2b, in13, in2, device="cuda")


def _inputs(torch, T, seed):
    from nvfp4_w4a4_expert_amd import moe as M
    rng = np.random.default_rng(seed)
    x = M.bf16_tensor(S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    res = M.bf16_tensor(S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    return x, res, lg


def _debug(torch, L, T):
    P = T * K_TOP
    bufs = dict(topk_ids=torch.empty((T, K_TOP), dtype=torch.int32, device="cuda"),
                expert_offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                a1_codes=torch.empty((P, H // 2), dtype=torch.uint8, device="cuda"),
                a2_codes=torch.empty((P, I // 2), dtype=torch.uint8, device="cuda"),
                c2=torch.empty((P, H), dtype=torch.float32, device="cuda"))
    return bufs, L.MoEDebug(**{k: v.data_ptr() for k, v in bufs.items()})


def test_noalloc_matches_workspace_forward_on_two_calls():
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    layer = _layer(torch)
    wst = layer.weights()
    # 576 tokens: the large-batch GEMM kernels and nearly the whole buffer;
    # then 40 tokens: the small-batch kernels on a buffer holding the first
    # call's data
    for T, seed in ((576, 1), (40, 2)):
        print(f"[noalloc] T={T}: workspace forward vs allocation-free forward", flush=True)
        x, res, lg = _inputs(torch, T, seed)
        nbytes = L.moe_workspace_size(T, K_TOP, wst)
        assert nbytes <= L.NOALLOC_SCRATCH_BYTES
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        out_ref = torch.empty_like(x)
        dref, dref_s = _debug(torch, L, T)
        L.moe_forward(wst, x, lg, T, K_TOP, res, out_ref, ws, nbytes, dref_s)
        out = torch.full_like(x, float("nan"))
        dgot, dgot_s = _debug(torch, L, T)
        L.moe_forward_noalloc(wst, x, lg, T, K_TOP, res, out, dgot_s)
        torch.cuda.synchronize()
        a = out_ref.view(torch.int16).cpu().numpy()
        b = out.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), f"T={T}: outputs differ"
        for name in dref:
            assert torch.equal(dref[name], dgot[name]), f"T={T}: {name} differs"
        of = out.float()
        assert torch.isfinite(of).all() and (of - res.float()).abs().max() > 0


def test_noalloc_refuses_a_batch_beyond_its_buffer():
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    layer = _layer(torch)
    wst = layer.weights()
    T = 1024
    assert L.moe_workspace_size(T, K_TOP, wst) > L.NOALLOC_SCRATCH_BYTES
    x, res, lg = _inputs(torch, T, 3)
    out = torch.zeros_like(x)
    with pytest.raises(L.NVFP4Error) as ei:
        L.moe_forward_noalloc(wst, x, lg, T, K_TOP, res, out)
    assert ei.value.status == L.ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).abs().max()) == 0
