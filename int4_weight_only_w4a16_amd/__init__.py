"""Python binding of libw4a16.so (the MI355X W4A16 GEMV).

Argument marshalling only: every function forwards to the C entry point of the
same name declared in include/w4a16.h. Host functions take numpy arrays;
device functions take torch tensors (or raw integer device pointers), torch
being used only for device memory and streams. Nothing here computes: if the
HIP library is not built, importing the functions fails loudly.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libw4a16.so")

W4A16_OK = 0
W4A16_EINVAL = -1
W4A16_EUNSUPPORTED = -2
W4A16_ELAYOUT = -3
W4A16_EHIP = -4
GROUP = 128
MAX_M = 8

# Every symbol the header declares.
EXPORTS = ("w4a16_layout_id", "w4a16_check_layout", "w4a16_packed_sizes", "w4a16_pack", "w4a16_pack_gate_up", "w4a16_quantize",
           "w4a16_unpack",
           "w4a16_gemv", "w4a16_gemv_swiglu", "w4a16_splitk_workspace_bytes", "w4a16_splitk_choose",
           "w4a16_gemv_splitk", "w4a16_gemv_splitk_noalloc", "w4a16_act_quant_i8", "w4a16_gemv_a8", "w4a16_gemv_a8_fused", "w4a16_gemm", "w4a16_gemm_splitk_choose",
           "w4a16_gemm_splitk", "w4a16_gemm_partials_bytes", "w4a16_gemm_partials_choose", "w4a16_gemm_splitk_partials",
           "w4a16_dequant_f16",
           "w4a16_dequant_f32", "w4a16_read_probe", "w4a16_chain_plan", "w4a16_chain_run", "w4a16_strerror")


CHAIN_GEMV = 0
CHAIN_SWIGLU = 1
# Byte offset of the chain workspace's error word (0: the last run completed).
CHAIN_ERROR_OFFSET = 8


class ChainOp(ctypes.Structure):
    """struct w4a16_chain_op of the header."""
    _fields_ = [("kind", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int), ("splits", ctypes.c_int),
                ("x_src", ctypes.c_int), ("x_shift", ctypes.c_int), ("wq", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


class W4A16Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {w4a16_strerror(status)} (status {status})")


_lib = None
_i = ctypes.c_int
_p = ctypes.c_void_p
_sz = ctypes.c_size_t


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(f"libw4a16.so is not built ({LIBRARY}); run __graft_entry__.build()")
        # torch first: its HIP runtime then satisfies the library's
        # libamdhip64.so.7 dependency. Loaded the other way round, the process
        # holds two HIP (and HSA) runtimes, and one of them can fail to find
        # the device (hipFuncSetAttribute returned "no ROCm-capable device").
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIBRARY)
        L.w4a16_layout_id.restype = _i
        L.w4a16_layout_id.argtypes = []
        L.w4a16_check_layout.restype = _i
        L.w4a16_check_layout.argtypes = [_i]
        L.w4a16_packed_sizes.argtypes = [_i, _i, _p, _p, _p]
        L.w4a16_pack.argtypes = [_i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_pack_gate_up.argtypes = [_i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p]
        L.w4a16_unpack.argtypes = [_i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_quantize.argtypes = [_i, _i, _p, _i, _p, _p, _p]
        L.w4a16_gemv.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_gemv_swiglu.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_splitk_workspace_bytes.restype = _sz
        L.w4a16_splitk_workspace_bytes.argtypes = [_i, _i, _i]
        L.w4a16_splitk_choose.restype = _i
        L.w4a16_splitk_choose.argtypes = [_i, _i, _i]
        L.w4a16_gemv_splitk.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
        L.w4a16_gemv_splitk_noalloc.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_dequant_f32.argtypes = [_i, _i, _p, _p, _p, _p, _p]
        L.w4a16_read_probe.argtypes = [_p, _sz, _i, _p, _p]
        L.w4a16_dequant_f16.argtypes = [_i, _i, _p, _p, _p, _p, _p]
        L.w4a16_gemm.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_gemm_splitk_choose.restype = _i
        L.w4a16_gemm_splitk_choose.argtypes = [_i, _i, _i]
        L.w4a16_gemm_splitk.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
        L.w4a16_gemm_partials_bytes.restype = _sz
        L.w4a16_gemm_partials_bytes.argtypes = [_i, _i, _i]
        L.w4a16_gemm_partials_choose.restype = _i
        L.w4a16_gemm_partials_choose.argtypes = [_i, _i, _i]
        L.w4a16_gemm_splitk_partials.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]
        L.w4a16_act_quant_i8.argtypes = [_i, _i, _p, _p, _p, _p, _p]
        L.w4a16_gemv_a8.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]
        L.w4a16_gemv_a8_fused.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p]
        L.w4a16_chain_plan.argtypes = [_i, _i, ctypes.POINTER(ChainOp), _p, _sz, ctypes.POINTER(_sz),
                                       ctypes.POINTER(_sz)]
        L.w4a16_chain_run.argtypes = [_i, _p, _p, _sz, _p]
        L.w4a16_strerror.restype = ctypes.c_char_p
        L.w4a16_strerror.argtypes = [_i]
        _lib = L
    return _lib


def _ptr(t):
    """Device pointer of a torch tensor, or an int passed through (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != W4A16_OK:
        raise W4A16Error(status, where)


def w4a16_strerror(status):
    return lib().w4a16_strerror(int(status)).decode()


def w4a16_layout_id():
    return lib().w4a16_layout_id()


def w4a16_check_layout(layout_id):
    """Raises W4A16Error(W4A16_ELAYOUT) unless layout_id is this library's."""
    _check(lib().w4a16_check_layout(int(layout_id)), "w4a16_check_layout")


def w4a16_packed_sizes(N, K):
    a, b, c = _sz(), _sz(), _sz()
    _check(lib().w4a16_packed_sizes(N, K, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "w4a16_packed_sizes")
    return a.value, b.value, c.value


def w4a16_pack(q, s, z):
    """Host: q uint8 [N][K], s uint16 fp16 bits [N][K/128], z uint8 [N][K/128]
    -> (wq, s_packed, z_packed) uint8 numpy arrays in layout ID 2."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    N, K = q.shape
    if K % GROUP or s.shape != (N, K // GROUP) or z.shape != (N, K // GROUP):
        raise W4A16Error(W4A16_EINVAL, "w4a16_pack")
    wb, sb, zb = w4a16_packed_sizes(N, K)
    wq, sp, zp = np.empty(wb, np.uint8), np.empty(sb, np.uint8), np.empty(zb, np.uint8)
    _check(lib().w4a16_pack(N, K, q.ctypes.data, s.ctypes.data, z.ctypes.data,
                            wq.ctypes.data, sp.ctypes.data, zp.ctypes.data), "w4a16_pack")
    return wq, sp, zp


def w4a16_pack_gate_up(qg, sg, zg, qu, su, zu):
    """Host: gate and up in w4a16_pack's logical form (each F x K) -> the
    interleaved (wq, s_packed, z_packed) uint8 arrays w4a16_gemv_swiglu reads."""
    qg, qu = (np.ascontiguousarray(a, dtype=np.uint8) for a in (qg, qu))
    sg, su = (np.ascontiguousarray(a, dtype=np.uint16) for a in (sg, su))
    zg, zu = (np.ascontiguousarray(a, dtype=np.uint8) for a in (zg, zu))
    F, K = qg.shape
    G = K // GROUP if K % GROUP == 0 else -1
    if qu.shape != (F, K) or any(a.shape != (F, G) for a in (sg, su, zg, zu)):
        raise W4A16Error(W4A16_EINVAL, "w4a16_pack_gate_up")
    wb, sb, zb = w4a16_packed_sizes(16 * ((F + 7) // 8), K)  # 8 gate + 8 up rows per 16-row tile
    wq, sp, zp = np.empty(wb, np.uint8), np.empty(sb, np.uint8), np.empty(zb, np.uint8)
    _check(lib().w4a16_pack_gate_up(F, K, qg.ctypes.data, sg.ctypes.data, zg.ctypes.data, qu.ctypes.data,
                                    su.ctypes.data, zu.ctypes.data, wq.ctypes.data, sp.ctypes.data,
                                    zp.ctypes.data), "w4a16_pack_gate_up")
    return wq, sp, zp


def w4a16_quantize(w_f16_bits, mode):
    """Host: fp16 weights (uint16 bits or float16) [N][K] -> (q, s, z) in
    w4a16_pack's logical form; mode 0 symmetric absmax/7, 1 asymmetric."""
    w_f16_bits = np.ascontiguousarray(np.asarray(w_f16_bits).view(np.uint16))
    N, K = w_f16_bits.shape
    G = K // GROUP if K % GROUP == 0 else 0
    q, s, z = np.empty((N, K), np.uint8), np.empty((N, max(G, 1)), np.uint16), np.empty((N, max(G, 1)), np.uint8)
    _check(lib().w4a16_quantize(N, K, w_f16_bits.ctypes.data, int(mode), q.ctypes.data, s.ctypes.data,
                                z.ctypes.data), "w4a16_quantize")
    return q, s, z


def w4a16_unpack(N, K, wq, s_packed, z_packed):
    """Host inverse of w4a16_pack -> (q, s, z)."""
    wq, sp, zp = (np.ascontiguousarray(a, dtype=np.uint8) for a in (wq, s_packed, z_packed))
    wb, sb, zb = w4a16_packed_sizes(N, K)
    if wq.size < wb or sp.size < sb or zp.size < zb:
        raise W4A16Error(W4A16_EINVAL, "w4a16_unpack")
    G = K // GROUP
    q, s, z = np.empty((N, K), np.uint8), np.empty((N, G), np.uint16), np.empty((N, G), np.uint8)
    _check(lib().w4a16_unpack(N, K, wq.ctypes.data, sp.ctypes.data, zp.ctypes.data,
                              q.ctypes.data, s.ctypes.data, z.ctypes.data), "w4a16_unpack")
    return q, s, z


def w4a16_gemv(M, N, K, Wq, scales, zeros, x, y, stream=None):
    """Device: y[M][N] (fp16) = W x[M][K] (fp16) with W in layout ID 2."""
    _check(lib().w4a16_gemv(M, N, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                            _stream(stream)), "w4a16_gemv")


def w4a16_gemv_swiglu(M, F, K, Wq, scales, zeros, x, y, stream=None):
    """Device: y[M][F] (fp16) = silu(gate x) * (up x), W from w4a16_pack_gate_up."""
    _check(lib().w4a16_gemv_swiglu(M, F, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                                   _stream(stream)), "w4a16_gemv_swiglu")


def w4a16_splitk_workspace_bytes(M, N, splits):
    return lib().w4a16_splitk_workspace_bytes(M, N, splits)


def w4a16_splitk_choose(M, N, K):
    return lib().w4a16_splitk_choose(M, N, K)


def w4a16_gemv_splitk(M, N, K, splits, Wq, scales, zeros, x, y, workspace, ws_bytes=None, stream=None):
    """Device: split-K GEMV in one launch. workspace: zero-filled once before
    first use (one uint64 accumulation word per output; every call leaves it
    zero again)."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().w4a16_gemv_splitk(M, N, K, splits, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x),
                                   _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)),
           "w4a16_gemv_splitk")


NOALLOC_SCRATCH_BYTES = 2 << 20


def w4a16_gemv_splitk_noalloc(M, N, K, splits, Wq, scales, zeros, x, y, stream=None):
    """Device: w4a16_gemv_splitk with the library's own per-GPU accumulation
    array (no workspace argument, nothing allocated; calls on one GPU must
    not overlap in time)."""
    _check(lib().w4a16_gemv_splitk_noalloc(M, N, K, splits, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x),
                                           _ptr(y), _stream(stream)), "w4a16_gemv_splitk_noalloc")


def w4a16_act_quant_i8(M, K, x, xq, sx, xsum, stream=None):
    """Device: fp16 x[M][K] -> int8 codes xq[M][K], fp32 scales sx[M][K/128],
    int32 code sums xsum[M][K/128] (one symmetric scale per group of 128)."""
    _check(lib().w4a16_act_quant_i8(M, K, _ptr(x), _ptr(xq), _ptr(sx), _ptr(xsum), _stream(stream)),
           "w4a16_act_quant_i8")


def w4a16_gemv_a8(M, N, K, Wq, scales, zeros, xq, sx, xsum, y, stream=None):
    """Device: y[M][N] (fp16) from the int8 activation codes of
    w4a16_act_quant_i8 (integer sums per group, then both scales)."""
    _check(lib().w4a16_gemv_a8(M, N, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(xq), _ptr(sx), _ptr(xsum),
                               _ptr(y), _stream(stream)), "w4a16_gemv_a8")


def w4a16_gemv_a8_fused(M, N, K, Wq, scales, zeros, x, y, stream=None):
    """Device: w4a16_act_quant_i8 + w4a16_gemv_a8 in one launch (x fp16),
    bit-identical to the two launches."""
    _check(lib().w4a16_gemv_a8_fused(M, N, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                                     _stream(stream)), "w4a16_gemv_a8_fused")


def w4a16_gemm(M, N, K, Wq, scales, zeros, x, y, stream=None):
    """Device: y[M][N] (fp16) = x[M][K] W^T for many rows (prefill), MFMA."""
    _check(lib().w4a16_gemm(M, N, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y), _stream(stream)),
           "w4a16_gemm")


def w4a16_gemm_splitk_choose(M, N, K):
    return lib().w4a16_gemm_splitk_choose(M, N, K)


def w4a16_gemm_splitk(M, N, K, splits, Wq, scales, zeros, x, y, workspace, ws_bytes=None, stream=None):
    """Device: the GEMM with K split across workgroups, combined exactly
    through workspace (zero-filled once; every call leaves it zero)."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().w4a16_gemm_splitk(M, N, K, splits, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                                   _ptr(workspace), ws_bytes, _stream(stream)), "w4a16_gemm_splitk")


def w4a16_gemm_partials_bytes(M, N, splits):
    return lib().w4a16_gemm_partials_bytes(M, N, splits)


def w4a16_gemm_partials_choose(M, N, K):
    return lib().w4a16_gemm_partials_choose(M, N, K)


def w4a16_gemm_splitk_partials(M, N, K, splits, Wq, scales, zeros, x, y, partials, partials_bytes=None, stream=None):
    """Device: split-K GEMM combined in two stages (fp32 partials, then a
    final pass in split order). partials: device buffer of at least
    w4a16_gemm_partials_bytes(M, N, splits) bytes, no initial contents."""
    if partials_bytes is None:
        partials_bytes = partials.numel() * partials.element_size()
    _check(lib().w4a16_gemm_splitk_partials(M, N, K, splits, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(x), _ptr(y),
                                            _ptr(partials), partials_bytes, _stream(stream)),
           "w4a16_gemm_splitk_partials")


def w4a16_dequant_f16(N, K, Wq, scales, zeros, W_out, stream=None):
    """Device: W_out[N][K] fp16 = fp16((q - z) * s), rounded once to nearest even."""
    _check(lib().w4a16_dequant_f16(N, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(W_out),
                                   _stream(stream)), "w4a16_dequant_f16")


def w4a16_read_probe(buf, grid, sink, nbytes=None, stream=None):
    """Device: read the bytes of `buf` once (measurement hook for the
    plain-read ceiling); `sink` is a 16-byte device buffer."""
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    _check(lib().w4a16_read_probe(_ptr(buf), nbytes, grid, _ptr(sink), _stream(stream)), "w4a16_read_probe")


def w4a16_chain_plan(M, ops):
    """Host: plan of a chain of GEMVs. `ops` is a sequence of dicts with keys
    kind, N, K, splits, x_src, x_shift, wq, scales, zeros, x, y (device
    tensors or integer pointers; x may be None when x_src >= 0). Returns
    (plan bytes as a uint8 numpy array, workspace bytes)."""
    arr = (ChainOp * len(ops))()
    for i, o in enumerate(ops):
        arr[i] = ChainOp(int(o["kind"]), int(o["N"]), int(o["K"]), int(o.get("splits", 1)), int(o.get("x_src", -1)),
                         int(o.get("x_shift", 0)), _ptr(o["wq"]), _ptr(o["scales"]), _ptr(o["zeros"]),
                         _ptr(o.get("x")), _ptr(o["y"]))
    pb, wb = _sz(), _sz()
    _check(lib().w4a16_chain_plan(M, len(ops), arr, None, 0, ctypes.byref(pb), ctypes.byref(wb)), "w4a16_chain_plan")
    plan = np.zeros(pb.value, np.uint8)
    _check(lib().w4a16_chain_plan(M, len(ops), arr, plan.ctypes.data, pb.value, None, None), "w4a16_chain_plan")
    return plan, wb.value


def w4a16_chain_run(M, plan_dev, workspace, ws_bytes=None, stream=None):
    """Device: the whole chain in one launch. plan_dev: the plan copied to
    device memory; workspace: zero-filled once (its uint32 at byte 8 is the
    error word)."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().w4a16_chain_run(M, _ptr(plan_dev), _ptr(workspace), ws_bytes, _stream(stream)), "w4a16_chain_run")


def w4a16_dequant_f32(N, K, Wq, scales, zeros, W_out, stream=None):
    """Device test hook: W_out[N][K] fp32 = (q - z) * s."""
    _check(lib().w4a16_dequant_f32(N, K, _ptr(Wq), _ptr(scales), _ptr(zeros), _ptr(W_out),
                                   _stream(stream)), "w4a16_dequant_f32")
