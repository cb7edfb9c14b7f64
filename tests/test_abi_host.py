"""Host-side checks of libw4a16.so (no GPU): exports, layout sizes, the packer
against the oracle's packing (bit-exact), unpack, and argument errors that are
decided before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import oracle
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "w4a16.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = w.lib()
    decl = declared_symbols()
    assert decl == sorted(w.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_layout_id_and_status_text():
    assert w.w4a16_layout_id() == 2
    w.w4a16_check_layout(2)
    for other in (0, 1, 3, -1):
        with pytest.raises(w.W4A16Error) as e:
            w.w4a16_check_layout(other)
        assert e.value.status == w.W4A16_ELAYOUT
    for code in (0, -1, -2, -3, -4):
        assert w.w4a16_strerror(code)
    assert w.w4a16_strerror(-99) == "unknown status"


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 896), (896, 896), (128, 4864), (37, 1152)])
def test_packed_sizes_match_oracle(orc, N, K):
    assert w.w4a16_packed_sizes(N, K) == orc.layout_sizes(N, K)


@pytest.mark.parametrize("N,K,seed", [(1, 128, 0), (15, 256, 1), (17, 896, 2), (40, 1152, 3),
                                      (896, 896, 0), (128, 4864, 5), (33, 18944, 6)])
def test_pack_matches_oracle_bytes(orc, N, K, seed):
    q, s, z = synthetic.weights(N, K, seed=seed)
    mine = w.w4a16_pack(q, s, z)
    ref = orc.pack(q, s, z)
    for a, b in zip(mine, ref):
        assert np.array_equal(a, b)
    q2, s2, z2 = w.w4a16_unpack(N, K, *mine)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(z, z2)


def test_pack_edge_patterns(orc):
    N, K = 19, 640
    G = K // 128
    for q, s, z in [
        (np.zeros((N, K), np.uint8), np.zeros((N, G), np.uint16), np.zeros((N, G), np.uint8)),
        (np.full((N, K), 15, np.uint8), np.full((N, G), 0xFFFF, np.uint16), np.full((N, G), 15, np.uint8)),
        ((np.arange(N * K) % 16).astype(np.uint8).reshape(N, K), np.arange(N * G, dtype=np.uint16).reshape(N, G),
         (np.arange(N * G) * 7 % 16).astype(np.uint8).reshape(N, G)),
    ]:
        for a, b in zip(w.w4a16_pack(q, s, z), orc.pack(q, s, z)):
            assert np.array_equal(a, b)


def _interleave_8(a_gate, a_up, fill=0):
    """16-row tiles of 8 gate rows and the 8 up rows of the same outputs
    (rows past F zero): tile j holds gate 8j .. 8j+7, then up 8j .. 8j+7."""
    F = a_gate.shape[0]
    tiles = (F + 7) // 8
    out = np.full((16 * tiles,) + a_gate.shape[1:], fill, a_gate.dtype)
    for f in range(F):
        out[16 * (f // 8) + f % 8] = a_gate[f]
        out[16 * (f // 8) + f % 8 + 8] = a_up[f]
    return out


@pytest.mark.parametrize("F,K", [(1, 128), (8, 256), (16, 256), (40, 896), (77, 640)])
def test_pack_gate_up_is_the_8_row_interleave(orc, F, K):
    """w4a16_pack_gate_up == the oracle's packing of the 8-row interleave."""
    qg, sg, zg = synthetic.weights(F, K, seed=F, tensor_id=1)
    qu, su, zu = synthetic.weights(F, K, seed=F, tensor_id=2)
    mine = w.w4a16_pack_gate_up(qg, sg, zg, qu, su, zu)
    ref = orc.pack(_interleave_8(qg, qu), _interleave_8(sg, su), _interleave_8(zg, zu))
    for a, b in zip(mine, ref):
        assert np.array_equal(a, b)
    L = w.lib()
    assert L.w4a16_pack_gate_up(F, K, None, sg.ctypes.data, zg.ctypes.data, qu.ctypes.data, su.ctypes.data,
                                zu.ctypes.data, *(m.ctypes.data for m in mine)) == w.W4A16_EINVAL
    assert L.w4a16_pack_gate_up(F, 200, *(a.ctypes.data for a in (qg, sg, zg, qu, su, zu)),
                                *(m.ctypes.data for m in mine)) == w.W4A16_EINVAL


@pytest.mark.parametrize("N,K,seed", [(1, 128, 0), (6, 512, 1), (64, 896, 2), (37, 4864, 3), (300, 1152, 4)])
@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_matches_oracle_bits(orc, N, K, seed, mode):
    """The library's quantizer equals the oracle's bit for bit: codes, fp16
    scales and zero points (both decide in fp64 with round half to even)."""
    from tests.oracle_pins import _quant_groups
    w16 = synthetic.activations(N, K, seed=seed, tensor_id=5)  # fp16 N(0,1) bits
    w16 = (w16.view(np.float16).astype(np.float64) * 0.02).astype(np.float16).view(np.uint16)
    if N >= 6 and K >= 512:
        w16[:6, :512] = _quant_groups(seed)
    for a, b in zip(w.w4a16_quantize(w16, mode), orc.quantize(w16, mode)):
        assert np.array_equal(a, b)


def test_quantize_ties_and_errors(orc):
    """Weights exactly half-way between two codes round to the even code in
    both quantizers; non-finite weights and bad modes are rejected."""
    c = 2.0 ** -4
    vals = np.zeros((1, 128))
    vals[0, 0] = 7 * c                               # absmax 7c: symmetric scale exactly c
    vals[0, 1:15] = (np.arange(-7, 7) + 0.5) * c     # the half-way points between codes
    w16 = vals.astype(np.float16).view(np.uint16)
    mine, ref = w.w4a16_quantize(w16, 0), orc.quantize(w16, 0)
    assert all(np.array_equal(a, b) for a, b in zip(mine, ref))
    assert orc.f16_to_f64(ref[1])[0, 0] == c
    assert (((ref[0][0, 1:15].astype(int) - 8) % 2) == 0).all()
    bad = w16.copy()
    bad[0, 3] = 0x7C00  # +inf
    with pytest.raises(w.W4A16Error):
        w.w4a16_quantize(bad, 0)
    with pytest.raises(w.W4A16Error):
        w.w4a16_quantize(w16, 2)


def test_pack_rejects_bad_values_and_shapes():
    L = w.lib()
    q = np.zeros((2, 128), np.uint8)
    s = np.zeros((2, 1), np.uint16)
    z = np.zeros((2, 1), np.uint8)
    wb, sb, zb = w.w4a16_packed_sizes(2, 128)
    out = [np.empty(n, np.uint8) for n in (wb, sb, zb)]
    args = lambda qq, zz: (2, 128, qq.ctypes.data, s.ctypes.data, zz.ctypes.data, *(o.ctypes.data for o in out))
    assert L.w4a16_pack(*args(q, z)) == w.W4A16_OK
    q_bad = q.copy(); q_bad[1, 77] = 16
    assert L.w4a16_pack(*args(q_bad, z)) == w.W4A16_EINVAL
    z_bad = z.copy(); z_bad[0, 0] = 200
    assert L.w4a16_pack(*args(q, z_bad)) == w.W4A16_EINVAL
    assert L.w4a16_pack(2, 100, q.ctypes.data, s.ctypes.data, z.ctypes.data, *(o.ctypes.data for o in out)) == w.W4A16_EINVAL
    assert L.w4a16_pack(2, 128, None, s.ctypes.data, z.ctypes.data, *(o.ctypes.data for o in out)) == w.W4A16_EINVAL
    assert L.w4a16_pack(0, 128, None, None, None, None, None, None) == w.W4A16_OK
    assert L.w4a16_packed_sizes(4, 129, None, None, None) == w.W4A16_EINVAL
    assert L.w4a16_packed_sizes(-1, 128, None, None, None) == w.W4A16_EINVAL


def test_device_entry_points_reject_before_launch():
    """Argument errors are returned without touching the GPU (none here)."""
    L = w.lib()
    fake = 1 << 20  # aligned, never dereferenced: every call below fails its checks first
    ptrs = [fake] * 5
    for M, N, K, want in [(1, 16, 100, w.W4A16_EINVAL), (1, 16, 0, w.W4A16_EINVAL), (-1, 16, 128, w.W4A16_EINVAL),
                          (1, -3, 128, w.W4A16_EINVAL), (9, 16, 128, w.W4A16_EUNSUPPORTED),
                          (0, 16, 128, w.W4A16_OK), (1, 0, 128, w.W4A16_OK)]:
        assert L.w4a16_gemv(M, N, K, *ptrs, None) == want, (M, N, K)
    # null and misaligned pointers
    assert L.w4a16_gemv(1, 16, 128, fake, fake, None, fake, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv(1, 16, 128, fake, fake, fake, fake + 2, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv(1, 16, 128, fake + 8, fake, fake, fake, fake, None) == w.W4A16_EINVAL
    # split-K: split count and workspace size
    ws = w.w4a16_splitk_workspace_bytes(2, 16, 3)
    assert ws == 8 * 2 * 16  # one uint64 word per output
    assert w.w4a16_splitk_workspace_bytes(1, 33, 2) == 272 and w.w4a16_splitk_workspace_bytes(1, 33, 9) == 272
    assert w.w4a16_splitk_workspace_bytes(-1, 16, 3) == 0
    assert w.w4a16_splitk_choose(1, 37888, 3584) == 1 and w.w4a16_splitk_choose(1, 3584, 7936) == 1
    assert w.w4a16_splitk_choose(1, 3584, 18944) == 1 and w.w4a16_splitk_choose(8, 5120, 17408) == 8
    assert w.w4a16_splitk_choose(1, 896, 4864) == 3 and w.w4a16_splitk_choose(5, 4608, 3584) == 1
    assert w.w4a16_splitk_choose(5, 17408, 5120) == 2 and w.w4a16_splitk_choose(1, 152064, 5120) == 1
    assert w.w4a16_splitk_choose(1, 37888, 3584) == 1 and w.w4a16_splitk_choose(8, 16384, 5120) == 2
    assert len({w.w4a16_splitk_choose(m, 5120, 17408) for m in range(1, 9)}) == 1  # never depends on M
    assert w.w4a16_splitk_choose(1, 128, 65536) == 16 and w.w4a16_splitk_choose(1, 8192, 131072) == 16
    assert w.w4a16_splitk_choose(1, 16, 200) == 0 and w.w4a16_splitk_choose(9, 16, 128) == 0
    for splits, wsb, want in [(0, ws, w.W4A16_EINVAL), (3, ws - 4, w.W4A16_EINVAL), (3, ws, None),
                              (8, 10 ** 9, w.W4A16_EINVAL)]:  # K = 768: at most 6 splits
        if want is None:
            continue
        assert L.w4a16_gemv_splitk(2, 16, 768, splits, *ptrs, fake, wsb, None) == want, splits
    assert L.w4a16_gemv_splitk(9, 16, 768, 2, *ptrs, fake, 10 ** 9, None) == w.W4A16_EUNSUPPORTED
    assert L.w4a16_gemv_splitk(1, 16, 128 * 40, 32, *ptrs, fake, 10 ** 9, None) == w.W4A16_EINVAL  # > 31 splits
    assert L.w4a16_gemv_splitk(2, 0, 768, 2, *ptrs, fake, 0, None) == w.W4A16_OK
    # split-K with the library's own accumulation array: the same checks, and
    # outputs beyond the array (8 bytes each) are refused before any GPU call
    cap = w.NOALLOC_SCRATCH_BYTES // 8
    for M, N, K, splits, want in [(1, 16, 200, 2, w.W4A16_EINVAL), (1, 16, 768, 0, w.W4A16_EINVAL),
                                  (1, 16, 768, 7, w.W4A16_EINVAL), (1, 16, 128 * 40, 32, w.W4A16_EINVAL),
                                  (9, 16, 768, 2, w.W4A16_EUNSUPPORTED), (-1, 16, 768, 2, w.W4A16_EINVAL),
                                  (0, 16, 768, 2, w.W4A16_OK), (2, 0, 768, 2, w.W4A16_OK),
                                  (1, cap + 1, 768, 2, w.W4A16_EUNSUPPORTED),
                                  (8, cap // 8 + 16, 768, 2, w.W4A16_EUNSUPPORTED)]:
        assert L.w4a16_gemv_splitk_noalloc(M, N, K, splits, *ptrs, None) == want, (M, N, K, splits)
    assert L.w4a16_gemv_splitk_noalloc(1, 16, 768, 2, fake, fake, fake, fake + 2, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv_splitk_noalloc(1, 16, 768, 2, fake, None, fake, fake, fake, None) == w.W4A16_EINVAL
    # fused SwiGLU
    assert L.w4a16_gemv_swiglu(1, 16, 200, *ptrs, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv_swiglu(9, 16, 128, *ptrs, None) == w.W4A16_EUNSUPPORTED
    assert L.w4a16_gemv_swiglu(1, 0, 128, *ptrs, None) == w.W4A16_OK
    assert L.w4a16_gemv_swiglu(1, 16, 128, fake, fake, fake, fake + 2, fake, None) == w.W4A16_EINVAL
    # GEMM for many rows
    assert L.w4a16_gemm(64, 16, 200, *ptrs, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm(-1, 16, 128, *ptrs, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm(0, 16, 128, *ptrs, None) == w.W4A16_OK
    assert L.w4a16_gemm(64, 16, 1 << 25, *ptrs, None) == w.W4A16_EUNSUPPORTED
    assert L.w4a16_gemm(64, 16, 128, fake, fake, fake, fake + 2, fake, None) == w.W4A16_EINVAL
    # read probe (measurement hook)
    assert L.w4a16_read_probe(fake, 100, 8, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_read_probe(fake, 1024, 0, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_read_probe(fake, 1024, 70000, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_read_probe(fake + 4, 1024, 8, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_read_probe(fake, 0, 8, fake, None) == w.W4A16_OK
    # GEMM with split K: split count, workspace, K limit, and the measured choice
    wsg = w.w4a16_splitk_workspace_bytes(64, 16, 3)
    for M, K, splits, wsb, want in [(64, 768, 0, wsg, w.W4A16_EINVAL), (64, 768, 7, wsg, w.W4A16_EINVAL),
                                    (64, 128 * 40, 32, 10 ** 9, w.W4A16_EINVAL), (64, 768, 3, wsg - 8, w.W4A16_EINVAL),
                                    (64, 200, 2, wsg, w.W4A16_EINVAL), (-1, 768, 2, wsg, w.W4A16_EINVAL),
                                    (0, 768, 3, 0, w.W4A16_OK), (64, 1 << 25, 2, 10 ** 12, w.W4A16_EUNSUPPORTED)]:
        assert L.w4a16_gemm_splitk(M, 16, K, splits, *ptrs, fake, wsb, None) == want, (M, K, splits, wsb)
    assert L.w4a16_gemm_splitk(64, 16, 768, 3, fake, fake, fake, fake + 2, fake, fake, wsg, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm_splitk(64, 16, 768, 3, *ptrs, None, wsg, None) == w.W4A16_EINVAL
    for M, N, K, want in [(16, 3584, 18944, 16), (17, 3584, 18944, 8), (64, 3584, 18944, 8),
                          (256, 3584, 18944, 4), (512, 3584, 18944, 2), (640, 3584, 18944, 3),
                          (768, 3584, 18944, 3), (1024, 3584, 18944, 1),
                          (16, 37888, 3584, 1), (16, 4608, 3584, 4), (64, 4608, 3584, 4), (96, 4608, 3584, 4),
                          (128, 4608, 3584, 1), (128, 3584, 3584, 4), (256, 3584, 3584, 1), (16, 200, 1024, 2),
                          (1, 16, 128, 1), (16, 16, 200, 0), (0, 16, 128, 0), (16, 16, 1 << 25, 0)]:
        assert w.w4a16_gemm_splitk_choose(M, N, K) == want, (M, N, K)
    # dequant to fp16
    assert L.w4a16_dequant_f16(16, 200, fake, fake, fake, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_dequant_f16(0, 128, None, None, None, None, None) == w.W4A16_OK
    assert L.w4a16_dequant_f16(16, 128, fake, fake, fake, fake + 4, None) == w.W4A16_EINVAL
    # INT8 activations: quantizer and GEMV
    assert L.w4a16_act_quant_i8(1, 200, fake, fake, fake, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_act_quant_i8(9, 128, fake, fake, fake, fake, None) == w.W4A16_EUNSUPPORTED
    assert L.w4a16_act_quant_i8(0, 128, None, None, None, None, None) == w.W4A16_OK
    assert L.w4a16_act_quant_i8(1, 128, fake, fake, fake + 4, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_act_quant_i8(1, 128, fake, None, fake, fake, None) == w.W4A16_EINVAL
    a8 = [fake] * 8
    assert L.w4a16_gemv_a8(1, 16, 200, *a8, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv_a8(9, 16, 128, *a8, None) == w.W4A16_EUNSUPPORTED
    assert L.w4a16_gemv_a8(1, 0, 128, *a8, None) == w.W4A16_OK
    assert L.w4a16_gemv_a8(1, 16, 128, fake, fake, fake, fake, fake, fake + 4, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv_a8(1, 16, 128, fake, fake, fake, fake, None, fake, fake, None) == w.W4A16_EINVAL
    # the same with the quantization fused (fp16 x)
    assert L.w4a16_gemv_a8_fused(1, 16, 200, *ptrs, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv_a8_fused(9, 16, 128, *ptrs, None) == w.W4A16_EUNSUPPORTED
    assert L.w4a16_gemv_a8_fused(0, 16, 128, *ptrs, None) == w.W4A16_OK
    assert L.w4a16_gemv_a8_fused(1, 16, 128, fake, fake, fake, fake + 2, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_gemv_a8_fused(1, 16, 128, fake, fake, None, fake, fake, None) == w.W4A16_EINVAL
    # dequant hook
    assert L.w4a16_dequant_f32(16, 200, fake, fake, fake, fake, None) == w.W4A16_EINVAL
    assert L.w4a16_dequant_f32(0, 128, None, None, None, None, None) == w.W4A16_OK
    assert L.w4a16_dequant_f32(16, 128, fake, fake, fake, fake + 4, None) == w.W4A16_EINVAL


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    """No fallback: a missing library is an ImportError, not a CPU path."""
    monkeypatch.setattr(w, "LIBRARY", os.path.join(tmp_path, "missing.so"))
    monkeypatch.setattr(w, "_lib", None)
    with pytest.raises(ImportError):
        w.lib()


def test_gemm_partials_sizes_choice_and_argument_checks():
    """w4a16_gemm_splitk_partials: the buffer size, the split choice and the
    argument checks that return before any launch (no GPU touched)."""
    L = w.lib()
    assert w.w4a16_gemm_partials_bytes(3, 5, 2) == 128  # 4 * 2 * 3 * 5 = 120, rounded up to 16
    assert w.w4a16_gemm_partials_bytes(64, 4608, 4) == 4 * 4 * 64 * 4608
    assert w.w4a16_gemm_partials_bytes(-1, 5, 2) == 0 and w.w4a16_gemm_partials_bytes(3, 5, 0) == 0
    for M, N, K in [(16, 4608, 3584), (128, 3584, 18944), (384, 4608, 3584), (64, 37888, 3584)]:
        s = w.w4a16_gemm_partials_choose(M, N, K)
        assert 1 <= s <= min(16, K // 128 // 4 if K // 128 >= 4 else 1)
    assert w.w4a16_gemm_partials_choose(64, 37888, 3584) == 1  # enough output tiles already
    assert w.w4a16_gemm_partials_choose(16, 64, 200) == 0       # K not a multiple of 128
    fake = 1 << 20
    ptrs = [fake] * 5
    need = w.w4a16_gemm_partials_bytes(64, 300, 4)
    assert L.w4a16_gemm_splitk_partials(64, 300, 1024, 4, *ptrs, fake, need - 16, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm_splitk_partials(64, 300, 1024, 4, *ptrs, None, need, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm_splitk_partials(64, 300, 1024, 4, *ptrs, fake + 8, need, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm_splitk_partials(64, 300, 1024, 9, *ptrs, fake, need, None) == w.W4A16_EINVAL  # > K/128
    assert L.w4a16_gemm_splitk_partials(64, 300, 1024, 0, *ptrs, fake, need, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm_splitk_partials(64, 300, 200, 2, *ptrs, fake, need, None) == w.W4A16_EINVAL
    assert L.w4a16_gemm_splitk_partials(0, 300, 1024, 4, *ptrs, None, 0, None) == w.W4A16_OK
