"""GPU check of w4a16_gemv_splitk_noalloc, the split-K GEMV whose accumulation
words live in the library's own per-GPU array (for callers that cannot
allocate): through the C ABI, its output must equal w4a16_gemv_splitk's (same
plan, same kernel, so bit for bit) and meet the oracle's bound, on two calls
in a row, the second with a smaller input; the array must be left usable."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import oracle
from tests.gpu_common import Problem, torch_dev

pytestmark = pytest.mark.gpu


def run_pair(p, splits):
    """(noalloc y, workspace y) for one problem and split count."""
    torch, dev = torch_dev()
    y_na, y_ws = p.new_y(), p.new_y()
    print(f"noalloc: M={p.M} N={p.N} K={p.K} splits={splits}", flush=True)
    w.w4a16_gemv_splitk_noalloc(p.M, p.N, p.K, splits, p.wq_d, p.sp_d, p.zp_d, p.x_d, y_na)
    ws = p.splitk_workspace(splits)
    w.w4a16_gemv_splitk(p.M, p.N, p.K, splits, p.wq_d, p.sp_d, p.zp_d, p.x_d, y_ws, ws)
    torch.cuda.synchronize()
    return y_na.cpu().numpy().view(np.uint16), y_ws.cpu().numpy().view(np.uint16)


def check(p, splits):
    y_na, y_ws = run_pair(p, splits)
    assert np.array_equal(y_na, y_ws), "noalloc differs from the workspace entry point"
    ref, absref = p.reference()
    ok, worst = oracle.bound_report(y_na, ref, absref, oracle.get())
    assert ok, worst


def test_noalloc_matches_workspace_entry_two_calls_shrinking():
    # first call: a 7B down-projection (K of 148 groups) at the library's
    # recommended split for a skinny shape; second: a smaller, ragged one
    big = Problem(2, 3584, 18944, seed=11)
    check(big, 8)
    small = Problem(1, 133, 4864, seed=12)
    check(small, 3)
    # and a third, larger again, to show the array was left zero
    check(Problem(3, 1000, 2048, seed=13), 5)


def test_noalloc_repeat_bit_identical_and_rejects_oversize():
    torch, dev = torch_dev()
    p = Problem(4, 512, 4096, seed=14)
    a, _ = run_pair(p, 4)
    b, _ = run_pair(p, 4)
    assert np.array_equal(a, b)
    cap = w.NOALLOC_SCRATCH_BYTES // 8
    y = torch.empty((1, 16), dtype=torch.int16, device=dev)
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_gemv_splitk_noalloc(1, cap + 16, 4096, 4, p.wq_d, p.sp_d, p.zp_d, p.x_d, y)
    assert e.value.status == w.W4A16_EUNSUPPORTED
