"""GPU parity of the quantiser against the oracle quantiser, in both its
forms (nvfp4_quantize_experts over expert-grouped rows, nvfp4_quantize_pairs
fused with the regrouping): packed E2M1 codes and E4M3 scales bit-exact."""
import numpy as np
import pytest

import synthetic as S
from oracle import formats as OF
from oracle import moe as OM
from oracle import quant as OQ

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch


def _dev(a, dtype):
    torch = _torch()
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


def _gpu_quantize(x_bits, K, topk, expert_idx, dst_row, gscale, num_dst_rows):
    """nvfp4_quantize_pairs: token rows scattered to their destination rows."""
    torch = _torch()
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    R = x_bits.shape[0]
    E = 1 if gscale is None else len(gscale)
    codes = torch.full((num_dst_rows, K // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((num_dst_rows, K // 16), 0xCD, dtype=torch.uint8, device="cuda")
    L.quantize_pairs(M.bf16_tensor(x_bits), x_bits.shape[1], R, K, topk,
                     _dev(expert_idx, np.int32), _dev(dst_row, np.int32), E,
                     _dev(gscale, np.float32), codes, sf, num_dst_rows)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy()


def _gpu_quantize_gather(x_bits, K, src_row, offsets, gscale, P, fp16=False, num_src_rows=None):
    """nvfp4_quantize_experts(_fp16): grouped output rows gathered from x."""
    torch = _torch()
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    E = len(offsets) - 1
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
    codes = torch.full((P, K // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((P, K // 16), 0xCD, dtype=torch.uint8, device="cuda")
    fn = L.quantize_experts_fp16 if fp16 else L.quantize_experts
    n_src = x_bits.shape[0] if num_src_rows is None else num_src_rows
    fn(x, x_bits.shape[1], K, _dev(src_row, np.int32), n_src, P, _dev(offsets, np.int32), E,
       _dev(gscale, np.float32), codes, sf)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sf.cpu().numpy()


def _grouped(expert, E):
    """Rows grouped by expert (stable): source row of each grouped row, the
    expert offsets and each grouped row's expert."""
    order = np.argsort(expert, kind="stable")
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(np.bincount(expert, minlength=E))
    return order.astype(np.int32), offsets, np.asarray(expert)[order]


GS_SET = np.array([1.0, 1.0 / 3.0, 448.0 / 6.0, 2688.0, 1e-3, 3.0e38, 0.7071, 12345.678,
                   2.0 ** -20, 1.0 / 2688.0], dtype=np.float32)


def test_every_bf16_pattern_every_scale():
    """All 65,280 finite bf16 patterns (blocks of 16 in two arrangements) under
    ten SFScaleVal values covering both clamps, subnormal E4M3 scales and
    reciprocal overflow: codes and scales bit-exact."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(OF.bf16_to_f32(bits))
    bits = bits[finite]
    rng = np.random.default_rng(0)
    arr = [bits, bits[rng.permutation(bits.size)]]
    rows = []
    for a in arr:
        n = a.size // 256 * 256
        rows.append(a[:n].reshape(-1, 256))
    x = np.concatenate(rows)                          # [R, 256]
    R = x.shape[0]
    E = GS_SET.size
    expert = np.arange(R, dtype=np.int32) % E
    # the pairs form, one destination per row
    codes, sf = _gpu_quantize(x, 256, 1, expert, None, GS_SET, R)
    oc, osf = OQ.quantize_experts(x, expert, GS_SET)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)
    # the gather form over the rows grouped by expert
    src, offsets, rexp = _grouped(expert, E)
    codes, sf = _gpu_quantize_gather(x, 256, src, offsets, GS_SET, R)
    oc, osf = OQ.quantize_experts(x[src], rexp, GS_SET)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)


def test_every_fp16_pattern_every_scale():
    """All 63,488 finite fp16 patterns through the fp16 entry point under the
    ten SFScaleVal values: codes and scales bit-exact against the oracle's
    fp16 path."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(bits.view(np.float16))]
    rng = np.random.default_rng(5)
    arr = [bits, bits[rng.permutation(bits.size)]]
    x = np.concatenate([a[:a.size // 256 * 256].reshape(-1, 256) for a in arr])
    R = x.shape[0]
    expert = np.arange(R, dtype=np.int32) % GS_SET.size
    src, offsets, rexp = _grouped(expert, GS_SET.size)
    codes, sf = _gpu_quantize_gather(x, 256, src, offsets, GS_SET, R, fp16=True)
    oc, osf = OQ.quantize_experts(x[src], rexp, GS_SET, fp16=True)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)


def test_fp16_routed_rows_ragged():
    """fp16 rows of varied magnitude routed top-4 of 6 experts: the grouped
    rows gather token t = src_pair / k; a row width of 13 blocks."""
    rng = np.random.default_rng(6)
    T, K, k, E = 29, 208, 4, 6
    x = (rng.standard_normal((T, K)) * np.exp(rng.uniform(-6, 6, (T, 1)))).astype(np.float16)
    x_bits = x.view(np.uint16)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gs = np.exp(rng.uniform(-3, 6, E)).astype(np.float32)
    offsets, src, inv = OM.permute(ids, E)
    P = T * k
    codes, sf = _gpu_quantize_gather(x_bits, K, src // k, offsets, gs, P, fp16=True)
    oc, osf = OQ.quantize_experts(x_bits[src // k], OM.row_experts(offsets), gs, fp16=True)
    assert np.array_equal(codes, oc) and np.array_equal(sf, osf)


def test_gather_skips_rows_without_a_source_or_an_expert():
    """Output rows whose source row is negative or past the last source row,
    and rows outside [offsets[0], offsets[E]), are left untouched."""
    rng = np.random.default_rng(8)
    x = S.f32_to_bf16_bits(rng.standard_normal((6, 48)).astype(np.float32))
    src = np.array([0, -1, 5, 6, 2, 3, 1, 4], dtype=np.int32)      # -1 and 6 have no source
    offsets = np.array([1, 4, 7], dtype=np.int32)                 # rows 0 and 7 have no expert
    gs = np.array([0.5, 3.0], dtype=np.float32)
    codes, sf = _gpu_quantize_gather(x, 48, src, offsets, gs, 8)
    written = [2, 4, 5, 6]
    rexp = np.array([0, 1, 1, 1])
    oc, osf = OQ.quantize_experts(x[src[written]], rexp, gs)
    assert np.array_equal(codes[written], oc) and np.array_equal(sf[written], osf)
    for r in (0, 1, 3, 7):
        assert np.all(codes[r] == 0xAB) and np.all(sf[r] == 0xCD)


def test_topk_scatter_and_ragged_blocks():
    rng = np.random.default_rng(1)
    T, K, k, E = 37, 272, 3, 5
    x = S.f32_to_bf16_bits((rng.standard_normal((T, K)) * np.exp(rng.uniform(-4, 4, (T, 1)))).astype(np.float32))
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gs = np.exp(rng.uniform(-3, 6, E)).astype(np.float32)
    P = T * k
    dst = rng.permutation(P).astype(np.int32)
    codes, sf = _gpu_quantize(x, K, k, ids.reshape(-1), dst, gs, P)
    src_tok = np.empty(P, dtype=np.int64)
    src_tok[dst] = np.arange(P) // k
    row_exp = np.empty(P, dtype=np.int64)
    row_exp[dst] = ids.reshape(-1)
    oc, osf = OQ.quantize_experts(x[src_tok], row_exp, gs)
    assert np.array_equal(codes, oc) and np.array_equal(sf, osf)


def test_null_scale_means_unit_scale():
    rng = np.random.default_rng(2)
    x = S.f32_to_bf16_bits(rng.standard_normal((8, 64)).astype(np.float32) * 300)
    codes, sf = _gpu_quantize(x, 64, 1, None, None, None, 8)
    oc, osf = OQ.quantize_experts(x, np.zeros(8, dtype=np.int64), None)
    assert np.array_equal(codes, oc) and np.array_equal(sf, osf)
    codes, sf = _gpu_quantize_gather(x, 64, None, np.array([0, 3, 8], dtype=np.int32), None, 8)
    assert np.array_equal(codes, oc) and np.array_equal(sf, osf)


@pytest.mark.parametrize("K", [32, 64])
def test_out_of_range_destinations_are_skipped(K):
    """Pairs whose destination row or expert is out of range are skipped (K = 64
    runs the layer's specialised kernel, K = 32 the general one)."""
    rng = np.random.default_rng(3)
    x = S.f32_to_bf16_bits(rng.standard_normal((4, K)).astype(np.float32))
    dst = np.array([0, 7, -1, 2], dtype=np.int32)               # 7 and -1 out of range
    expert = np.array([0, 0, 0, 5], dtype=np.int32)             # 5 out of range
    codes, sf = _gpu_quantize(x, K, 1, expert, dst, np.ones(2, dtype=np.float32), 4)
    oc, osf = OQ.quantize_experts(x[[0]], np.array([0]), np.ones(1, dtype=np.float32))
    assert np.array_equal(codes[0], oc[0]) and np.array_equal(sf[0], osf[0])
    assert np.all(codes[1:] == 0xAB) and np.all(sf[1:] == 0xCD)


def test_quantizer_workload_full_size():
    """8192 tokens x 2816, top-8 of 128 experts (uniform router), 1% outlier
    channels x50, per-expert calibrated input scales: every code and scale
    bit-exact, and both saturation levels are exercised."""
    torch = _torch()
    w = S.WORKLOADS["quant"]
    x = S.activations(w)
    logits = S.router_logits(w)
    xc, lc = S.calibration_batch(w)
    s13, wr = OM.calibrate_input_scale(xc, lc, w.k, w.E)
    ok, gs, _ = OM.validate_scales(s13, wr)
    assert ok
    ids, _ = OM.route(logits, w.k)
    offsets, src, inv = OM.permute(ids, w.E)
    codes, sf = _gpu_quantize(x, w.H, w.k, ids.reshape(-1), inv, gs, w.P)
    oc, osf = OQ.quantize_experts(x[src // w.k], OM.row_experts(offsets), gs)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)
    codes, sf = _gpu_quantize_gather(x, w.H, src // w.k, offsets, gs, w.P)
    assert np.array_equal(sf, osf)
    assert np.array_equal(codes, oc)
    assert np.count_nonzero(osf == 0x7E) > 0
    assert np.count_nonzero((OF.unpack_nibbles(oc) & 7) == 7) > 0


def test_zero_rows_is_noop():
    torch = _torch()
    from nvfp4_w4a4_expert_amd import _lib as L
    codes = torch.full((1, 8), 7, dtype=torch.uint8, device="cuda")
    L.quantize_pairs(None, 16, 0, 16, 1, None, None, 1, None, codes, codes, 0)
    L.quantize_experts(None, 16, 16, None, 0, 0, None, 1, None, codes, codes)
    torch.cuda.synchronize()
    assert codes.cpu().numpy().tolist() == [[7] * 8]


def test_hardware_conversions_selftest():
    """The conversion instructions behind the codes, the block scales and the
    GEMM operands equal references built from the format definitions: E2M1
    encode on every non-NaN fp32 input, E2M1 -> fp16 on every byte, E4M3 ->
    fp16 on every non-NaN code, E4M3 block-scale encode on every non-negative
    fp32 input and +inf, E4M3 -> fp32 on every non-negative code."""
    torch = _torch()
    from nvfp4_w4a4_expert_amd import _lib as L
    cnt = torch.full((5,), 12345, dtype=torch.int64, device="cuda")
    L.selftest_conversions(cnt)
    torch.cuda.synchronize()
    assert cnt.cpu().tolist() == [0, 0, 0, 0, 0]


def _pack_reference(codes, sf, bk):
    """The kernel weight layout, stated directly: for expert e, 32-row block
    nb and K step ks, lane l's 16-byte pieces v hold row nb*32 + (l & 31),
    elements ks*bk + (l >> 5)*bk/2 + 32v + [0, 32); its scales hold the bk/32
    block scales of that row and K range."""
    E, N, Kh = codes.shape
    K = Kh * 2
    kvec, nks = bk // 64, K // bk
    out_c = np.empty(E * N * K // 2, dtype=np.uint8)
    out_s = np.empty(E * N * K // 16, dtype=np.uint8)
    lanes = np.arange(64)
    pc = ps = 0
    for e in range(E):
        for nb in range(N // 32):
            rows = nb * 32 + (lanes & 31)
            for ks in range(nks):
                for v in range(kvec):
                    k0 = ks * bk + (lanes >> 5) * (bk // 2) + 32 * v
                    for l in range(64):
                        out_c[pc:pc + 16] = codes[e, rows[l], k0[l] // 2:k0[l] // 2 + 16]
                        pc += 16
                b0 = (ks * bk + (lanes >> 5) * (bk // 2)) // 16
                for l in range(64):
                    out_s[ps:ps + bk // 32] = sf[e, rows[l], b0[l]:b0[l] + bk // 32]
                    ps += bk // 32
    return out_c, out_s


@pytest.mark.parametrize("projection", [0, 1])
def test_weight_packing_layout(projection):
    """nvfp4_moe_pack_weights is the stated byte permutation, bit for bit."""
    torch = _torch()
    from nvfp4_w4a4_expert_amd import _lib as L
    rng = np.random.default_rng(40 + projection)
    E, H, I = 3, 256, 128
    N, K = (2 * I, H) if projection == 0 else (H, I)
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, size=(E, N, K // 16), dtype=np.uint8)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(sf).cuda()
    oc, osf = torch.empty_like(dc), torch.empty_like(ds)
    L.moe_pack_weights(projection, dc, ds, E, H, I, oc, osf)
    torch.cuda.synchronize()
    rc, rs = _pack_reference(codes, sf, 128 if projection == 0 else 64)
    assert np.array_equal(oc.cpu().numpy().reshape(-1), rc)
    assert np.array_equal(osf.cpu().numpy().reshape(-1), rs)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("blocks,offset", [(21, 0), (20, 0), (20, 1), (43, 3)])
def test_scale_words_and_byte_fallback(mx, blocks, offset):
    """Scale bytes leave as 32-bit words when the row's scale count is a
    multiple of 4 (8 blocks of 16 in the UE8M0 mode) and the array is
    4-byte aligned, else one byte at a time: odd widths and a misaligned
    scale array, both modes, bit-exact against the oracle."""
    torch = _torch()
    from nvfp4_w4a4_expert_amd import _lib as L
    from nvfp4_w4a4_expert_amd import moe as M
    from oracle import mx as OX
    blk = 32 if mx else 16
    K = blk * blocks
    rng = np.random.default_rng(blocks * 10 + offset + (100 if mx else 0))
    T, E, k = 40, 6, 3
    x = S.f32_to_bf16_bits((rng.standard_normal((T, K)) * 10.0 ** rng.uniform(-3, 3, (T, 1)))
                           .astype(np.float32))
    ids, _ = OM.route(rng.standard_normal((T, E)).astype(np.float32), k)
    offsets, src, inv = OM.permute(ids, E)
    gs = (10.0 ** rng.uniform(-2, 2, E)).astype(np.float32)
    P = T * k
    codes = torch.full((P, K // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf_buf = torch.full((P * (K // blk) + 8,), 0xCD, dtype=torch.uint8, device="cuda")
    sf = sf_buf[offset:offset + P * (K // blk)]
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=t)).cuda()
    Q = OX if mx else OQ
    oc, osf = Q.quantize_experts(x[src // k], OM.row_experts(offsets), gs)
    for form in ("pairs", "gather"):
        codes.fill_(0xAB)
        sf_buf.fill_(0xCD)
        if form == "pairs":
            fn = L.quantize_pairs_mx if mx else L.quantize_pairs
            fn(M.bf16_tensor(x), K, T, K, k, dev(ids, np.int32), dev(inv, np.int32), E,
               dev(gs, np.float32), codes, sf, P)
        else:
            fn = L.quantize_experts_mx if mx else L.quantize_experts
            fn(M.bf16_tensor(x), K, K, dev(src // k, np.int32), T, P, dev(offsets, np.int32), E,
               dev(gs, np.float32), codes, sf)
        torch.cuda.synchronize()
        assert np.array_equal(sf.cpu().numpy().reshape(P, K // blk), osf), form
        assert np.array_equal(codes.cpu().numpy(), oc), form
        rest = sf_buf.cpu().numpy()
        assert np.all(rest[:offset] == 0xCD) and np.all(rest[offset + P * (K // blk):] == 0xCD)
