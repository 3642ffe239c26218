"""Oracle-side work of the 30-layer stack test (tests/test_gpu_stack.py), run
in worker processes: preparing a layer (the oracle draws, quantises and
calibrates it) and checking a layer's gathered GPU rows against the oracle.
Thirty layers of that is minutes of CPU work, so several layers are handled
at once beside the GPU chain.  Workers import only the oracle, the seeded
generators and the CPU-side checks, never the GPU library."""
import time

import numpy as np

import synthetic as S
from oracle import moe as OM

from gpu_helpers import check_gathered_subset

FIELDS = ("w13c", "w13s", "w13s2", "w2c", "w2s", "w2s2", "w13_input_scale", "w2_input_scale",
          "written13", "written2")


def init_worker(threads: int) -> None:
    """Cap the worker's BLAS and OpenMP pools at `threads`, so that several
    workers share the host's cores instead of each starting one thread per
    core."""
    from threadpoolctl import threadpool_limits
    globals()["_limits"] = threadpool_limits(limits=threads)
    globals()["_threads"] = threads


def prepare_stack_layer(layer_idx: int, threads: int = 0) -> dict:
    """The oracle's layer `layer_idx` of the stack workload (weights drawn,
    quantised and its activation scales calibrated by the oracle), as plain
    arrays."""
    t0 = time.perf_counter()
    threads = threads or globals().get("_threads", 2)
    w = S.WORKLOADS["stack"]
    w13, w2 = S.expert_weights(w, layer=layer_idx, threads=threads)
    xc, lc = S.calibration_batch(w, layer=layer_idx)
    layer = OM.prepare_layer(w13, w2, xc, lc, w.k, threads=threads)
    del w13, w2
    out = {name: np.asarray(getattr(layer, name)) for name in FIELDS}
    out["prep_seconds"] = time.perf_counter() - t0
    return out


def layer_from_fields(f: dict) -> OM.Layer:
    return OM.Layer(*(f[name] for name in FIELDS))


def check_stack_layer(fields: dict, x_sub, logits_sub, k, got, label) -> dict:
    """check_gathered_subset for one stack layer (residual = the layer's
    input, as in the chain)."""
    t0 = time.perf_counter()
    m = check_gathered_subset(layer_from_fields(fields), x_sub, logits_sub, k, x_sub, got, label)
    m["check_seconds"] = time.perf_counter() - t0
    return m
