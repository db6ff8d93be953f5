"""The library against its conservative-sync twin (libqgemm_sync.so: the same
sources built with QGEMM_SYNC_TWIN=1, which drains every outstanding memory
and LDS operation and meets at a barrier at each stage boundary of the
LDS-staged kernels).  The twin multiplies in the same order, so every output
must be bit-identical -- INT8 and every floating-point path alike.  A wait the
fast build miscounts (a stage used before it landed, a slot refilled while
still being read, a scale word taken from the wrong round) makes the two
differ.  Shapes: every LDS-staged tile, K with whole and partial last rounds,
ragged M / N, random scale codes; repeated launches on the same buffers.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from block_scaled_precision_02_amd import inputs, build  # noqa: E402
import block_scaled_precision_02_amd as q  # noqa: E402

from tests import parity  # noqa: E402


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def twin():
    import os
    if not os.path.exists(build.LIB_SYNC):
        pytest.fail(f"{build.LIB_SYNC} is not built (python -m block_scaled_precision_02_amd.build)")
    return q.declare(ctypes.CDLL(build.LIB_SYNC))


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.force_tile(-1)
    yield
    q.force_tile(-1)


def _run_with(L, d, tile, monkeypatch):
    """One call through the given library copy (fast or twin), same tile."""
    monkeypatch.setattr(q, "_lib", L)
    q.force_tile(tile)
    try:
        out = parity.gpu_run(d)
        torch.cuda.synchronize()
        return parity.bits(out)
    finally:
        q.force_tile(-1)


CASES = [
    # (workload, M, N, K, tiles)
    ("i8_small", 300, 260, 1088, [0, 1, 2, 3, 4, 5, 6, 7]),       # 17 stages: a partial last round
    ("i8_small", 257, 513, 2048, [4, 5, 6, 7]),
    ("f8_ptpc", 200, 300, 448, [0, 1, 3, 4, 5, 6, 7]),
    ("mxfp8", 300, 520, 768, [0, 4, 5, 6, 7]),
    ("mxfp4", 260, 300, 1280, [0, 1, 4, 5, 6, 7]),
    ("f8_block", 280, 300, 640, [7, 10]),
    ("mx_a8w4", 200, 300, 640, [4, 5, 7]),
    ("mx_a4w8", 200, 300, 640, [4, 5, 7]),
    ("mxfp8", 200, 300, 704, [4, 5, 6, 7]),                       # K % 128 == 64
    ("mx_a8w4", 130, 260, 448, [4, 5, 7]),
    ("mx_a4w8", 130, 260, 448, [4, 5, 7]),
    ("mxfp4", 130, 260, 704, [4, 5, 7]),                          # e2m1 in 64-element stages
    ("mxfp8", 201, 289, 736, [4, 5, 6, 7]),                       # K % 64 == 32: a last half stage
    ("mx_a4w8", 130, 260, 480, [4, 5, 7]),
    ("mxfp4", 130, 260, 736, [4, 5, 7]),
    ("mxfp6", 200, 300, 640, [4, 7]),
    ("mxfp6_e3m2", 130, 260, 1024, [4, 7]),
]


@pytest.mark.parametrize("name,M,N,K,tiles", CASES, ids=[f"{c[0]}-{c[3]}" for c in CASES])
def test_fast_build_equals_sync_twin(twin, monkeypatch, name, M, N, K, tiles):
    d = inputs.make(name, M=M, N=N, K=K, bias=True)
    if d["kind"] in ("mx",):
        rng = np.random.default_rng(M + N + K)
        d["scale_a"] = rng.integers(112, 142, d["scale_a"].shape, dtype=np.uint8)
        d["scale_b"] = rng.integers(112, 142, d["scale_b"].shape, dtype=np.uint8)
    fast = q.lib()
    for tile in tiles:
        _say(f"[twin] {name} {M}x{N}x{K} tile {tile}")
        a = _run_with(fast, d, tile, monkeypatch)
        b = _run_with(twin, d, tile, monkeypatch)
        again = _run_with(fast, d, tile, monkeypatch)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"{name} tile {tile}: fast build != sync twin"
        assert np.array_equal(a, again), f"{name} tile {tile}: two launches differ"
    monkeypatch.setattr(q, "_lib", fast)
    ref, absdot, _ = parity.oracle_run(d)
    q.force_tile(tiles[0])
    parity.compare(d, parity.bits(parity.gpu_run(d)), ref, absdot, f"{name} vs oracle")
