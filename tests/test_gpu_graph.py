"""GPU test: the layer forward captured in a HIP graph (torch.cuda.CUDAGraph).

The forward launches kernels only (no memset, no allocation, no host
synchronisation), so a caller can capture it once and replay it.  Each
replay must reproduce, bit for bit, an eager forward on the inputs the
captured buffers hold at replay time.  Replays are interleaved with eager
forwards and synchronisations, and the inputs are rewritten in place
between replays, so a graph that replayed stale work or lost a node would
fail.  Covered: the workspace forward at both kernel sizes (16 tokens, the
small-batch GEMMs; 600 tokens, the large-batch ones) and the
allocation-free forward."""
import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu

E, H, I, K_TOP = 128, 2816, 704, 8


def _layer(torch):
    """A layer of the decode/prefill shape with seeded random codes and valid
    E4M3 block scales (the reference is the eager forward, not the oracle)."""
    from nvfp4_w4a4_expert_amd import moe as M
    rng = np.random.default_rng(77)
    w13 = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w2 = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w13s = rng.integers(0x28, 0x40, (E, 2 * I, H // 16), dtype=np.uint8)
    w2s = rng.integers(0x28, 0x40, (E, H, I // 16), dtype=np.uint8)
    s2a = np.full(E, 2.0 ** -9, dtype=np.float32)
    s2b = np.full(E, 2.0 ** -10, dtype=np.float32)
    in13 = (rng.uniform(1.0, 2.0, E) / 600).astype(np.float32)
    in2 = (rng.uniform(1.0, 2.0, E) / 2000).astype(np.float32)
    return M.NVFP4MoELayer(w13, w13s, s2a, w2, w2s, s2b, in13, in2, device="cuda")


def _fill_inputs(torch, x, lg, res, seed):
    """Write a fresh seeded batch into existing device buffers (in place)."""
    rng = np.random.default_rng(seed)
    T = x.shape[0]
    xb = S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    rb = S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x.view(torch.int16).copy_(torch.from_numpy(xb.view(np.int16)))
    res.view(torch.int16).copy_(torch.from_numpy(rb.view(np.int16)))
    lg.copy_(torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)))


def _bits(torch, t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("T,noalloc", [(16, False), (600, False), (16, True), (600, True)])
def test_graph_replays_match_eager(T, noalloc):
    import torch
    from nvfp4_w4a4_expert_amd import _lib as L
    layer = _layer(torch)
    wst = layer.weights()
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    res = torch.empty_like(x)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    nbytes = L.moe_workspace_size(T, K_TOP, wst)
    if noalloc:
        assert nbytes <= L.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    # an eager reference forward with its own workspace and output
    ws_ref = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out_ref = torch.empty_like(x)

    def fwd():
        if noalloc:
            L.moe_forward_noalloc(wst, x, lg, T, K_TOP, res, out, None)
        else:
            L.moe_forward(wst, x, lg, T, K_TOP, res, out, ws, nbytes)

    def reference():
        L.moe_forward(wst, x, lg, T, K_TOP, res, out_ref, ws_ref, nbytes)

    print(f"[graph] T={T} noalloc={noalloc}: eager warm-up, then capture", flush=True)
    _fill_inputs(torch, x, lg, res, seed=1)
    fwd()                                 # first call outside capture (one-time lookups)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        fwd()
    torch.cuda.synchronize()
    for rep, seed in enumerate((1, 2, 3, 2)):
        print(f"[graph] T={T} noalloc={noalloc}: replay {rep} on input seed {seed}", flush=True)
        _fill_inputs(torch, x, lg, res, seed)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(torch, out)
        reference()                       # eager work between replays
        torch.cuda.synchronize()
        want = _bits(torch, out_ref)
        assert np.array_equal(got, want), f"T={T} noalloc={noalloc}: replay {rep} differs from eager"
    del g
    torch.cuda.synchronize()
