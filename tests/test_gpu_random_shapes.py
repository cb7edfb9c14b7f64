"""GPU parity on seeded random shapes: the GEMV, the split-K GEMV at the
library's chosen split and the fused gate/up + SwiGLU GEMV, each against the
oracle's bound, over shapes drawn so that the launch planner takes many of
its paths (1 to 16 waves, every share size, x from LDS or from global memory,
one or several rounds per share, ragged N and ragged 8-row tiles); and the
prefill GEMM at its chosen split for 9 to 300 rows (every workgroup height),
with the atomic and with the two-stage combine, also against the product with
the fp16-rounded weights."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import oracle
from tests.gpu_common import Problem
from tests.test_gpu_gemm import check_rounded_weights
from tests.test_gpu_swiglu import SwigluProblem

pytestmark = pytest.mark.gpu


def _shapes(seed, count, max_macs):
    """(M, N, K) with K a multiple of 128 and M * N * K at most max_macs (N
    drawn after K, so long K comes with narrow N)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.integers(1, 9))
        G = int(rng.choice([1, 2, 3, 5, 7, 8, 12, 20, 28, 37, 40, 64, 96, 136, 148, 160]))
        K = 128 * G
        N = int(rng.integers(1, max(2, min(2600, max_macs // (M * K)))))
        out.append((M, N, K))
    return out


GEMV_SHAPES = _shapes(2026, 20, 24_000_000)
SWIGLU_SHAPES = _shapes(2027, 10, 12_000_000)
_rng = np.random.default_rng(2028)
GEMM_SHAPES = [(int(m), int(n), 128 * int(g)) for m, n, g in
               zip(_rng.integers(9, 301, 10), _rng.integers(1, 700, 10), _rng.choice([1, 3, 7, 28, 40, 96, 148], 10))]


@pytest.mark.parametrize("M,N,K", GEMV_SHAPES)
def test_random_gemv_and_chosen_split(M, N, K):
    print(f"[random] gemv M={M} N={N} K={K}", flush=True)
    p = Problem(M, N, K, seed=M * 7919 + N * 31 + K)
    ref, absref = p.reference()
    o = oracle.get()
    y = p.gemv()
    ok, worst = oracle.bound_report(y, ref, absref, o)
    assert ok, (M, N, K, worst)
    assert np.array_equal(y, p.gemv()), "run-to-run difference"
    splits = w.w4a16_splitk_choose(M, N, K)
    if splits > 1:
        print(f"[random] splitk {splits}", flush=True)
        ws = p.splitk_workspace(splits)
        ys = p.gemv_splitk(splits, ws)
        ok, worst = oracle.bound_report(ys, ref, absref, o)
        assert ok, (M, N, K, splits, worst)
        assert np.array_equal(ys, p.gemv_splitk(splits, ws)), "split-K run-to-run difference"
        assert p.workspace_is_zero(ws)


@pytest.mark.parametrize("M,F,K", SWIGLU_SHAPES)
def test_random_swiglu(M, F, K):
    print(f"[random] swiglu M={M} F={F} K={K}", flush=True)
    sp = SwigluProblem(M, F, K, seed=F * 13 + K)
    sp.check(sp.run())


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_random_gemm_chosen_split(M, N, K):
    splits = w.w4a16_gemm_splitk_choose(M, N, K)
    print(f"[random] gemm M={M} N={N} K={K} splits={splits}", flush=True)
    p = Problem(M, N, K, seed=M * 101 + N + K)
    ws = p.splitk_workspace(splits)
    y = p.gemm_splitk(splits, ws)
    p.check(y)
    check_rounded_weights(p, y)
    assert np.array_equal(y, p.gemm_splitk(splits, ws)), "run-to-run difference"
    if splits > 1:
        assert p.workspace_is_zero(ws)
    ps = w.w4a16_gemm_partials_choose(M, N, K)
    print(f"[random] gemm partials splits={ps}", flush=True)
    yp = p.gemm_partials(ps)
    p.check(yp)
    check_rounded_weights(p, yp)
