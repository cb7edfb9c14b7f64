"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar: dequant hook bit-exact; every GEMV output within
|y - ref| <= 2e-3 * sum_k |w x| + 1e-5 of the unrounded fp64 reference;
repeated calls bit-identical."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import oracle
import synthetic
from tests.gpu_common import Problem, torch_dev, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------- dequant to fp16

@pytest.mark.parametrize("N,K,scales_kind", [(896, 896, "workload"), (37, 384, "workload"),
                                             (4608, 3584, "workload"), (5, 18944, "workload"),
                                             (40, 1024, "any_bits")])
def test_dequant_f16_bit_exact(N, K, scales_kind):
    """fp16((q - z) * s) equals the oracle's fp64 product rounded to fp16 bit
    for bit, including overflow to inf and subnormal results when the scale
    bits are arbitrary (NaN scales excluded: any NaN payload is correct)."""
    _say("dequant f16", N, K, scales_kind)
    torch, dev = torch_dev()
    q, s, z = synthetic.weights(N, K, seed=N + K)
    if scales_kind == "any_bits":
        s = np.random.default_rng(7).integers(0, 0x7C00, s.shape).astype(np.uint16)
        s[::3] |= 0x8000
    wq, sp, zp = w.w4a16_pack(q, s, z)
    out = torch.empty((N, K), dtype=torch.int16, device=dev)
    w.w4a16_dequant_f16(N, K, upload(wq), upload(sp), upload(zp), out)
    torch.cuda.synchronize()
    o = oracle.get()
    want = o.f64_to_f16(o.dequant(q, s, z))
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------ dequant hook

@pytest.mark.parametrize("N,K", [(896, 896), (37, 384), (4608, 3584), (5, 18944)])
def test_dequant_hook_bit_exact(N, K):
    _say("dequant", N, K)
    torch, dev = torch_dev()
    q, s, z = synthetic.weights(N, K, seed=N + K, tensor_id=1)
    wq, sp, zp = w.w4a16_pack(q, s, z)
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device=dev)
    w.w4a16_dequant_f32(N, K, upload(wq), upload(sp), upload(zp), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.get().dequant(q, s, z)
    assert np.array_equal(want.astype(np.float32).astype(np.float64), want)  # exact in fp32
    assert np.array_equal(got, want.astype(np.float32))


# --------------------------------------------------------- the workloads

def test_single_896():
    _, N, K = synthetic.SINGLE_896
    p = Problem(1, N, K, seed=0)
    _say("single_896 worst", p.check(p.gemv()))


@pytest.mark.parametrize("name,N,K", synthetic.QWEN05B_LAYER)
def test_qwen05b_shapes(name, N, K):
    p = Problem(1, N, K, seed=1)
    _say(name, "worst", p.check(p.gemv()))


@pytest.mark.parametrize("name,N,K", synthetic.QWEN7B_LAYER + [synthetic.QWEN7B_LM_HEAD])
def test_qwen7b_shapes(name, N, K):
    p = Problem(1, N, K, seed=2)
    y = p.gemv()
    _say(name, "worst", p.check(y))
    assert np.array_equal(y, p.gemv()), "run-to-run difference"


@pytest.mark.parametrize("M", synthetic.VERIFY_M)
@pytest.mark.parametrize("name,N,K", synthetic.VERIFY27B)
def test_verify27b_shapes(name, N, K, M):
    """Full size, every output against the oracle, and (many workgroups per
    CU, x staged by direct LDS requests for 2 to 5 rows) four runs bit for
    bit equal, plain and with the library's split choice."""
    p = Problem(M, N, K, seed=3)
    y = p.gemv()
    _say(name, M, "worst", p.check(y))
    for _ in range(3):
        assert np.array_equal(y, p.gemv()), "run-to-run difference"
    splits = w.w4a16_splitk_choose(M, N, K)
    if splits > 1:
        ws = p.splitk_workspace(splits)
        ys = p.gemv_splitk(splits, ws)
        p.check(ys)
        for _ in range(3):
            assert np.array_equal(ys, p.gemv_splitk(splits, ws)), "run-to-run difference (split)"


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("M", range(1, 9))
@pytest.mark.parametrize("N,K", [(1, 128), (15, 256), (17, 1152), (133, 640), (16, 32768), (33, 65664)])
def test_ragged_and_small(M, N, K):
    p = Problem(M, N, K, seed=M * 100 + N)
    p.check(p.gemv())


def test_degenerate_q_equals_z_gives_exact_zero():
    N, K = 48, 1024
    G = K // 128
    z = synthetic.weights(N, K, seed=9)[2]
    q = np.repeat(z, 128, axis=1)
    s = synthetic.scales(N, G, seed=9)
    p = Problem(2, N, K, q=q, s=s, z=z, x=synthetic.activations(2, K, seed=9))
    y = p.gemv()
    assert not (y & 0x7FFF).any()
    p.check(y)


def test_extreme_values():
    """Largest |q - z| with the largest scale that keeps y finite, and fp16
    subnormal activations."""
    N, K = 32, 2048
    G = K // 128
    q = np.full((N, K), 15, np.uint8)
    q[1::2] = 0
    z = np.zeros((N, G), np.uint8)
    z[1::2] = 15
    s = np.full((N, G), np.float16(1.5).view(np.uint16), np.uint16)
    x = np.full((1, K), np.float16(1.0).view(np.uint16), np.uint16)
    x[0, ::3] = np.uint16(0x0001)  # smallest subnormal
    p = Problem(1, N, K, q=q, s=s, z=z, x=x)
    p.check(p.gemv())


# ------------------------------------------------------------- invariants

def test_power_of_two_scaling_is_exact():
    p = Problem(3, 4608, 3584, seed=5)
    y1 = p.gemv()
    x2 = (p.x.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    y2 = p.gemv(upload(x2))
    want = (y1.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(y2, want)


def test_row_permutation_permutes_output():
    N, K = 300, 1536
    q, s, z = synthetic.weights(N, K, seed=6)
    x = synthetic.activations(2, K, seed=6)
    y = Problem(2, N, K, q=q, s=s, z=z, x=x).gemv()
    perm = np.random.default_rng(6).permutation(N)
    yp = Problem(2, N, K, q=q[perm], s=s[perm], z=z[perm], x=x).gemv()
    assert np.array_equal(yp, y[:, perm])


def test_activation_rows_are_independent():
    """Permuting the rows of x permutes the rows of y bit for bit."""
    N, K = 512, 2048
    q, s, z = synthetic.weights(N, K, seed=7)
    x = synthetic.activations(4, K, seed=7)
    y4 = Problem(4, N, K, q=q, s=s, z=z, x=x).gemv()
    y4b = Problem(4, N, K, q=q, s=s, z=z, x=x[[2, 0, 3, 1]].copy()).gemv()
    assert np.array_equal(y4b, y4[[2, 0, 3, 1]])


@pytest.mark.parametrize("N,K", [(128, 896), (4608, 3584), (3584, 18944), (17408, 5120), (5120, 17408)])
def test_batch_invariance(N, K):
    """Row m of an M-row call is bit-identical to that row computed alone,
    for every M up to 8 (the verify pass of a speculative decoder must give
    the same row r whether it processes 1 row or 8)."""
    _say("batch invariance", N, K)
    q, s, z = synthetic.weights(N, K, seed=11)
    x = synthetic.activations(8, K, seed=11)
    alone = [Problem(1, N, K, q=q, s=s, z=z, x=x[m:m + 1].copy()).gemv() for m in range(8)]
    for M in range(2, 9):
        yM = Problem(M, N, K, q=q, s=s, z=z, x=x[:M].copy()).gemv()
        for m in range(M):
            assert np.array_equal(yM[m], alone[m][0]), (M, m)


# ---------------------------------------------------------------- split-K

@pytest.mark.parametrize("splits", [1, 2, 3, 7, 28])
@pytest.mark.parametrize("M,N,K", [(1, 3584, 3584), (5, 128, 896 * 4), (1, 896, 4864), (8, 200, 3584)])
def test_splitk(M, N, K, splits):
    """Split-K against the oracle; the workspace is back at zero after each
    call, so a second call on the same workspace gives the same bits (a word
    left behind would corrupt the next call's sums)."""
    if splits > K // 128:
        pytest.skip("more splits than groups")
    _say("splitk", M, N, K, splits)
    p = Problem(M, N, K, seed=splits)
    ws = p.splitk_workspace(splits)
    y = p.gemv_splitk(splits, ws)
    p.check(y)
    assert p.workspace_is_zero(ws)
    assert np.array_equal(y, p.gemv_splitk(splits, ws))


SKINNY = [("skinny_128x18944", 128, 18944), ("skinny_200x18944", 200, 18944), ("skinny_512x18944", 512, 18944),
          ("skinny_64x7168", 64, 7168)]


@pytest.mark.parametrize("name,N,K", synthetic.QWEN05B_LAYER + synthetic.QWEN7B_LAYER + synthetic.VERIFY27B + SKINNY)
def test_splitk_chosen_full_size(name, N, K):
    """The split count the library picks, at the full model shapes, M = 1
    and 5, against the oracle on every output."""
    for M in (1, 5):
        splits = w.w4a16_splitk_choose(M, N, K)
        assert 1 <= splits <= K // 128
        _say("splitk chosen", name, M, splits)
        p = Problem(M, N, K, seed=4)
        y = p.gemv_splitk(splits)
        _say(name, M, splits, "worst", p.check(y))


def test_splitk_overflowing_partials_match_plain():
    """A single huge product (largest |q - z|, scale and x) makes a split's
    partial far beyond the fixed-point range (2^29): it is clamped, and the
    output still overflows fp16 to the same +-inf the plain GEMV gives;
    ordinary rows of the same call stay within the bound."""
    N, K, splits = 48, 4096, 4
    _say("splitk overflow", N, K, splits)
    G = K // 128
    q = np.full((N, K), 8, np.uint8)
    z = np.full((N, G), 8, np.uint8)
    s = synthetic.scales(N, G, seed=13)
    q[5, 1000] = 15
    z[5, 1000 // 128] = 0      # row 5: (q - z) = 15 at k = 1000, otherwise 8 - 0 = 8 in that group
    s[5, 1000 // 128] = 0x7BFF  # largest finite fp16 scale
    x = synthetic.activations(1, K, seed=13)
    x[0, 1000] = 0x7BFF         # 65504
    p = Problem(1, N, K, q=q, s=s, z=z, x=x)
    plain = p.gemv()
    y = p.gemv_splitk(splits)
    assert (plain[0, 5] & 0x7FFF) == 0x7C00  # the plain path overflows to inf
    assert y[0, 5] == plain[0, 5]
    ref, absref = p.reference()
    rows = [n for n in range(N) if n != 5]
    ok, worst = oracle.bound_report(y[:, rows], ref[:, rows], absref[:, rows], oracle.get())
    assert ok, worst


def test_splitk_batch_invariance():
    """Split-K rows do not depend on how many activation rows come along."""
    N, K, splits = 3584, 18944, 4
    _say("splitk batch invariance", N, K, splits)
    q, s, z = synthetic.weights(N, K, seed=12)
    x = synthetic.activations(8, K, seed=12)
    alone = Problem(1, N, K, q=q, s=s, z=z, x=x[:1].copy()).gemv_splitk(splits)
    y8 = Problem(8, N, K, q=q, s=s, z=z, x=x.copy()).gemv_splitk(splits)
    assert np.array_equal(y8[0], alone[0])


# ------------------------------------------------------------ graph replay

def test_graph_replay_matches_eager():
    torch, dev = torch_dev()
    p = Problem(1, 3584, 3584, seed=8)
    eager = p.gemv()
    y = p.new_y()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        w.w4a16_gemv(1, p.N, p.K, p.wq_d, p.sp_d, p.zp_d, p.x_d, y, stream=stream)  # warm
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            w.w4a16_gemv(1, p.N, p.K, p.wq_d, p.sp_d, p.zp_d, p.x_d, y, stream=stream)
    for _ in range(3):
        y.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), eager)


def test_graph_replay_splitk():
    """A captured split-K call replays correctly many times: the zeroed words
    each replay leaves are what the next replay starts from."""
    torch, dev = torch_dev()
    p = Problem(1, 3584, 18944, seed=9)
    splits = 4
    ws = p.splitk_workspace(splits)
    eager = p.gemv_splitk(splits, ws)
    y = p.new_y()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        w.w4a16_gemv_splitk(1, p.N, p.K, splits, p.wq_d, p.sp_d, p.zp_d, p.x_d, y, ws, stream=stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            w.w4a16_gemv_splitk(1, p.N, p.K, splits, p.wq_d, p.sp_d, p.zp_d, p.x_d, y, ws, stream=stream)
    for _ in range(4):
        y.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), eager)
        assert p.workspace_is_zero(ws)
    p.check(eager)


# -------------------------------------------------- quantize -> pack -> GEMV

@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 3584, 3584), (5, 896, 4864)])
def test_quantized_weights_end_to_end(mode, M, N, K):
    """fp16 weights quantized by the library (w4a16_quantize), packed and
    multiplied on the GPU stay within the closed-form quantization error of
    the unquantized fp64 product: every weight moves at most s/2 (round to
    nearest), except that an asymmetric code at the top of the range can
    clamp from 16 to 15 when fp16 rounded s below (hi - lo)/15 and z rounded
    up: at most (0.5 + 15 * 2^-11) s there. So |y - W x| <= sum_g 0.51 s_g *
    sum_{k in g} |x_k|, plus the GEMV bound on the quantized product."""
    _say("quantized end to end", mode, M, N, K)
    rng = np.random.default_rng(60 + mode)
    w16 = rng.normal(0.0, 0.02, (N, K)).astype(np.float16).view(np.uint16)
    q, s, z = w.w4a16_quantize(w16, mode)
    p = Problem(M, N, K, q=q, s=s, z=z, x=synthetic.activations(M, K, seed=61))
    y = p.gemv()
    o = oracle.get()
    yd = o.f16_to_f64(y)
    xd = o.f16_to_f64(p.x)
    wd = o.f16_to_f64(w16)
    exact = xd @ wd.T  # unquantized product (numpy float64)
    ref, absref = p.reference()
    G = K // 128
    sd = o.f16_to_f64(s)  # [N][G]
    xabs_g = np.abs(xd).reshape(M, G, 128).sum(axis=2)  # [M][G]
    quant_err = 0.51 * xabs_g @ sd.T  # [M][N]
    allow = quant_err + oracle.BOUND_REL * absref + oracle.BOUND_ABS
    assert (np.abs(yd - exact) <= allow).all(), float((np.abs(yd - exact) / allow).max())


# --------------------------------------------------------- device errors

def test_misaligned_device_pointer_is_rejected():
    p = Problem(1, 64, 256, seed=1)
    L = w.lib()
    rc = L.w4a16_gemv(1, 64, 256, p.wq_d.data_ptr(), p.sp_d.data_ptr(), p.zp_d.data_ptr(),
                      p.x_d.data_ptr() + 2, p.new_y().data_ptr(), None)
    assert rc == w.W4A16_EINVAL


def test_read_probe_stores_nothing():
    """The read-ceiling probe reads its buffer and leaves the sink alone
    (the XOR of an all-zero buffer is 0, not the probe's one constant)."""
    torch, dev = torch_dev()
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    sink = torch.full((16,), 7, dtype=torch.uint8, device=dev)
    for grid in (1, 3, 1024):
        w.w4a16_read_probe(buf, grid, sink)
        w.w4a16_read_probe(buf[:4096 + 16], grid, sink)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 7).all()
