"""CPU oracle for the NVFP4 W4A4 routed-expert MoE block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports, links or runs
anything here, and this package imports nothing from the product.

It is a plain, slow, obviously-correct restatement of what the pages define,
written with NumPy (fp32 where the method's arithmetic is fp32, fp64 for the
GEMM references) and exact rationals for the brute-force encoders.

Sources (page 3, "Gemma 4 NVFP4 MoE 空输出", taking-lying-flat.github.io):
  * "NVFP4" section: the E2M1 code table, the round-to-nearest-even
    saturating encode, the two-level (E4M3 per 16 + FP32 global) scaling, the
    6 x 448 = 2688 combined range, the runtime-order figure of the
    activation quantiser, and the per-expert ``SFScale[expert_idx]`` lookup;
  * "ROOT CAUSE" section: reciprocal of unchecked per-expert input scales;
  * "矩阵融合" section: fused gate/up (w13), act(gate) x up, the MoE
    pipeline permute -> quant(a1) -> grouped w13 -> SiLU/mul + quant(a2) ->
    grouped w2 -> unpermute + routing-weight sum.

Modules:
  formats  E2M1 / E4M3 / bf16 bit-level codecs (scalar exact + vectorised)
  quant    the per-16 block quantiser (scalar exact + vectorised) and dequant
  moe      scale validation, router, permutation, fp64 GEMM references,
           SiLU*mul, combine, calibration and the whole layer
"""
