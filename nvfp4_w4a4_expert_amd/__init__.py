"""MI355X-native (gfx950) NVFP4 W4A4 routed-expert MoE block.

The compute lives in ``libnvfp4moe.so`` (hand-written HIP kernels behind the
C ABI in ``include/nvfp4_moe.h``); this package is its thin Python binding.
Submodules are imported lazily so that building the library does not require
it to exist:

    from nvfp4_w4a4_expert_amd import build      # compile the library
    from nvfp4_w4a4_expert_amd import _lib       # raw C entry points
    from nvfp4_w4a4_expert_amd import moe        # NVFP4MoELayer + weight prep
"""
__all__ = ["build", "_lib", "moe"]
