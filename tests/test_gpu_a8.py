"""GPU parity of the INT8-activation path (w4a16_act_quant_i8 then
w4a16_gemv_a8) through the C ABI against the oracle: the codes, scales and
code sums bit for bit (the rounding decision is taken in fp32 on both
sides), and y within the workload's bound around the oracle's integer-sum
product, 2e-3 * sum_g |term| + 1e-5. The fused variant (w4a16_gemv_a8_fused,
quantization inside the GEMV launch) must equal the two launches bit for
bit."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import oracle
import synthetic
from tests.gpu_common import Problem, torch_dev, upload

pytestmark = pytest.mark.gpu
GROUP = 128


def _say(*a):
    print("[a8]", *a, flush=True)


def _quantize_on_gpu(M, K, x_d):
    torch, dev = torch_dev()
    G = K // GROUP
    xq = torch.full((M, K), 99, dtype=torch.int8, device=dev)
    sx = torch.full((M, G), float("nan"), dtype=torch.float32, device=dev)
    xs = torch.full((M, G), -7, dtype=torch.int32, device=dev)
    w.w4a16_act_quant_i8(M, K, x_d, xq, sx, xs)
    torch.cuda.synchronize()
    return xq, sx, xs


def _gemv_a8(p, xq, sx, xs):
    torch, _ = torch_dev()
    y = p.new_y()
    w.w4a16_gemv_a8(p.M, p.N, p.K, p.wq_d, p.sp_d, p.zp_d, xq, sx, xs, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def _special_activations(M, K, seed):
    """Workload activations plus awkward groups: all zero, ties on an exact
    grid (scale 1), tiny values with fp16 subnormals, one large outlier."""
    x = synthetic.activations(M, K, seed=seed, tensor_id=5).view(np.float16).astype(np.float64)
    G = K // GROUP
    if G >= 2:
        x[0, 0:GROUP] = 0.0
        x[M - 1, GROUP:2 * GROUP] = np.tile([127.0, 2.5, -3.5, 0.5, -126.5, 1.5, -0.5, 60.0], 16)
    if G >= 3:
        x[0, 2 * GROUP:3 * GROUP] *= 2.0 ** -13
    x[M - 1, K - 1] = 300.0
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("M,K", [(1, 128), (1, 896), (3, 3584), (8, 18944), (5, 17408), (2, 5120), (8, 256)])
def test_act_quant_bit_exact(M, K):
    _say("quant", M, K)
    x = _special_activations(M, K, seed=M * 7 + K)
    xq, sx, xs = _quantize_on_gpu(M, K, upload(x))
    rq, rs, rsum = oracle.get().act_quant_i8(x)
    assert np.array_equal(xq.cpu().numpy(), rq)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xs.cpu().numpy(), rsum)


def _check_a8(p, y, xq_np, sx_np):
    ref, absref = oracle.get().gemv_a8(p.q, p.s, p.z, xq_np, sx_np)
    ok, worst = oracle.bound_report(y, ref, absref, oracle.get())
    assert ok, f"M={p.M} N={p.N} K={p.K}: worst |y-ref|/bound = {worst}"
    return worst


# Shapes: the 7B and 27B-class projections (full size), ragged N, one
# group, fewer groups than waves, and K whose codes at M = 8 take several
# rounds per wave.
SHAPES = [(1, 37888, 3584), (1, 3584, 18944), (8, 3584, 18944), (5, 17408, 5120), (2, 5120, 17408),
          (1, 896, 896), (4, 4864, 896), (3, 33, 256), (7, 1, 128), (6, 50, 1408), (8, 64, 7168),
          (4, 257, 18944), (5, 3584, 18944), (6, 130, 18944)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemv_a8_against_oracle(M, N, K):
    _say("gemv_a8", M, N, K)
    p = Problem(M, N, K, seed=M + N + K)
    xq, sx, xs = _quantize_on_gpu(M, K, p.x_d)
    xq_np, sx_np = xq.cpu().numpy(), sx.cpu().numpy()
    y = _gemv_a8(p, xq, sx, xs)
    _say(M, N, K, "worst", _check_a8(p, y, xq_np, sx_np))
    assert np.array_equal(y, _gemv_a8(p, xq, sx, xs)), "run-to-run difference"


@pytest.mark.parametrize("M,K", [(8, 3584), (8, 18944), (5, 18944)])
def test_gemv_a8_codes_from_oracle_and_batch_invariance(M, K):
    """The GEMV alone, fed the oracle's codes (not the GPU quantizer's), and
    each row of a multi-row call bit-identical to the same row alone (at
    K = 18944 the multi-row call takes 7-tile shares in two rounds, the
    single row one round of 10)."""
    N = 200
    p = Problem(M, N, K, seed=77)
    rq, rs, rsum = oracle.get().act_quant_i8(p.x)
    xq, sx, xs = upload(rq), upload(rs), upload(rsum)
    y = _gemv_a8(p, xq, sx, xs)
    _check_a8(p, y, rq, rs)
    for m in (0, 3, M - 1):
        one = Problem(1, N, K, q=p.q, s=p.s, z=p.z, x=p.x[m:m + 1])
        y1 = _gemv_a8(one, upload(rq[m:m + 1]), upload(rs[m:m + 1]), upload(rsum[m:m + 1]))
        assert np.array_equal(y1[0], y[m]), m


def test_gemv_a8_close_to_fp16_path():
    """End to end on the workload's shape: the INT8-activation y differs from
    the fp16-activation GEMV by about the activation rounding only (relative
    RMS below 2%)."""
    M, N, K = 2, 4608, 3584
    p = Problem(M, N, K, seed=5)
    xq, sx, xs = _quantize_on_gpu(M, K, p.x_d)
    ya8 = _gemv_a8(p, xq, sx, xs).view(np.float16).astype(np.float64)
    yfp = p.gemv().view(np.float16).astype(np.float64)
    assert np.sqrt(((ya8 - yfp) ** 2).mean()) < 0.02 * np.sqrt((yfp ** 2).mean())


@pytest.mark.parametrize("M,N,K", SHAPES + [(3, 3584, 18944), (8, 5120, 17408)])
def test_gemv_a8_fused_equals_two_launches(M, N, K):
    """One launch, fp16 x in: y bit-identical to act_quant_i8 + gemv_a8 (same
    codes from the same fp32 operations, same sums in the same order), on
    the workload's activations and on the awkward groups."""
    torch, dev = torch_dev()
    for special in (False, True):
        _say("fused", M, N, K, "special" if special else "")
        x = _special_activations(M, K, seed=M + K) if special else None
        p = Problem(M, N, K, seed=M + 2 * N + K, x=x)
        xq, sx, xs = _quantize_on_gpu(M, K, p.x_d)
        y2 = _gemv_a8(p, xq, sx, xs)
        y1 = p.new_y()
        w.w4a16_gemv_a8_fused(M, N, K, p.wq_d, p.sp_d, p.zp_d, p.x_d, y1)
        torch.cuda.synchronize()
        y1 = y1.cpu().numpy().view(np.uint16)
        assert np.array_equal(y1, y2), (M, N, K, special, int((y1 != y2).sum()))
