"""CPU range check of the grouped GEMMs' global accesses (no GPU).

tests/host/gemm_ranges.cpp is built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer against nvfp4_w4a4_expert_amd/csrc/gemm_tiles.h,
the header through which the kernel forms its tile mapping and every global
address.  It walks each launch's tiles, wavefronts, lanes, staging chunks, K
steps and output elements, and checks that every access lies inside its
buffer and that the tiles cover each grouped row once.  The cases are the
per-expert row counts of every workload (routed by the oracle's router), the
tile-boundary counts of the GPU tile tests and a few extremes, in all three
operand modes (UE8M0 only where the hidden size allows it) and for both the
small- and large-batch kernels.

This guards the kind of fault a tile-mapping change can bring back: an
inactive wavefront that once formed a weight-block base before the start of
w13 (its first row computed as a negative offset), which faulted the GPU
only for some allocations."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synthetic as S
from oracle import moe as OM

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TILE_COUNTS = {                    # from the GPU tile-boundary tests (tiny layer, top-1)
    "odd": [97, 65, 33, 1],
    "even": [96, 64, 32, 129],
    "small": [33, 32, 31, 1],
}


def _workload_counts(name, layer=0, tokens=None):
    w = S.WORKLOADS[name]
    T = tokens or w.T
    ids, _ = OM.route(S.router_logits(w, layer=layer, tokens=T), w.k)
    return w, T, np.bincount(ids.reshape(-1), minlength=w.E)


def _cases():
    cases = []

    def add(label, E, H, I, k, T, counts):
        counts = [int(c) for c in counts]
        assert len(counts) == E and sum(counts) == T * k
        for mode in (0, 1, 2):
            if mode == 2 and H % 256:
                continue                      # the UE8M0 layer needs H % 256 == 0
            cases.append(f"{label} {mode} {E} {H} {I} {k} {T} " + " ".join(map(str, counts)))

    for name, layer, tokens in (("tiny", 0, None), ("decode", 0, None), ("prefill", 0, None),
                                ("stack", 0, None), ("stack", 29, None), ("maxsize", 0, 96),
                                ("maxsize", 0, None), ("shapes", 0, None)):
        w, T, counts = _workload_counts(name, layer, tokens)
        add(f"{name}-L{layer}-T{T}", w.E, w.H, w.I, w.k, T, counts)
    # the fused routing + quantisation parity shapes (hidden 1024, I 64)
    for E, k, T in ((64, 1, 5), (256, 32, 9), (512, 4, 33), (1024, 8, 3)):
        w = S.Workload(f"fused-E{E}-k{k}", 8, T=T, H=1024, E=E, I=64, k=k, router="normal",
                       calib_tokens=2048)
        ids, _ = OM.route(S.router_logits(w), k)
        add(w.name, E, 1024, 64, k, T, np.bincount(ids.reshape(-1), minlength=E))
    # the non-power-of-two expert count of the odd-expert parity tests
    for T in (2200, 40):
        w = S.Workload(f"odd-E200-T{T}", 9, T=T, H=1024, E=200, I=192, k=6, router="normal",
                       calib_tokens=2048)
        ids, _ = OM.route(S.router_logits(w), w.k)
        add(w.name, w.E, w.H, w.I, w.k, T, np.bincount(ids.reshape(-1), minlength=w.E))
    t = S.WORKLOADS["tiny"]
    for label, counts in TILE_COUNTS.items():
        add(f"tiles-{label}", t.E, t.H, t.I, 1, sum(counts), counts)
    # extremes: one expert takes everything; exactly at and one below the
    # large-batch switch (P = 32 E); a single expert; a single row
    add("one-expert", 4, 256, 128, 2, 300, [600, 0, 0, 0])
    add("switch-at", 4, 256, 128, 1, 128, [32, 32, 32, 32])
    add("switch-below", 4, 256, 128, 1, 127, [32, 32, 32, 31])
    add("single-expert", 1, 512, 192, 1, 77, [77])
    for T in (5, 300):                        # the single-expert GPU parity shapes
        add(f"single-expert-T{T}", 1, 256, 128, 1, T, [T])
    add("single-row", 8, 256, 64, 1, 1, [0, 0, 0, 0, 0, 0, 0, 1])
    add("wide-empty", 1024, 256, 128, 1, 3, [1] + [0] * 1021 + [1, 1])
    return cases


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_every_gemm_access_is_in_bounds(tmp_path):
    exe = str(tmp_path / "gemm_ranges")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I" + ROOT,
           os.path.join(ROOT, "tests", "host", "gemm_ranges.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    cases = _cases()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(cases) + "\n", capture_output=True, text=True,
                       timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:] + r.stderr[-3000:])
    assert f"gemm ranges ok ({len(cases)} cases)" in r.stdout
    assert r.stdout.count("in bounds") == 2 * len(cases)
