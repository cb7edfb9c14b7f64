"""fp64 CPU oracle for the W4A16 GEMV -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may
import this package. The product library never imports, links or calls it,
and it shares no code with the HIP path.

The arithmetic lives in ``oracle_w4a16.c`` (plain C, OpenMP over output rows,
each sum sequential in ascending k, so results do not depend on the thread
count); this module only builds it with gcc and marshals numpy arrays.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_w4a16.c")
LIBRARY = os.path.join(_HERE, "liboracle_w4a16.so")
GROUP = 128

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(out_path=LIBRARY, plant=0):
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", f"-DOR_PLANT={int(plant)}",
           SOURCE, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path=LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path} (run oracle.build())")
        lib = ctypes.CDLL(path)
        self.lib = lib
        lib.or_f16_to_f64.restype = ctypes.c_double
        lib.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_f64_to_f16.restype = ctypes.c_uint16
        lib.or_f64_to_f16.argtypes = [ctypes.c_double]
        for name in ("or_f16_to_f64_array", "or_f64_to_f16_array"):
            getattr(lib, name).argtypes = [_p, _p, _i64]
            getattr(lib, name).restype = None
        lib.or_layout_sizes.argtypes = [_i64, _i64, _p]
        lib.or_pack.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p]
        lib.or_unpack.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p]
        lib.or_dequant.argtypes = [_i64, _i64, _p, _p, _p, _p]
        lib.or_gemv.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p]
        lib.or_gemv_packed.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p]
        lib.or_gemv_packed_rows.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _i64, _p, _p]
        lib.or_quantize.argtypes = [_i64, _i64, _p, ctypes.c_int, _p, _p, _p]
        lib.or_act_quant_i8.argtypes = [_i64, _i64, _p, _p, _p, _p]
        lib.or_gemv_a8.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _i64, _p, _p]
        self.plant = lib.or_plant()

    # -- fp16 codec -------------------------------------------------------
    def f16_to_f64(self, bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.or_f16_to_f64_array(bits.ctypes.data, out.ctypes.data, bits.size)
        return out

    def f64_to_f16(self, values):
        values = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(values.shape, dtype=np.uint16)
        self.lib.or_f64_to_f16_array(values.ctypes.data, out.ctypes.data, values.size)
        return out

    def num_threads(self):
        return self.lib.or_num_threads()

    # -- layout ID 2 --------------------------------------------------------
    def layout_sizes(self, N, K):
        out = np.zeros(3, dtype=np.int64)
        if self.lib.or_layout_sizes(N, K, out.ctypes.data):
            raise ValueError(f"invalid shape N={N} K={K}")
        return tuple(int(v) for v in out)

    def pack(self, q, s, z):
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint16)
        z = np.ascontiguousarray(z, dtype=np.uint8)
        N, K = q.shape
        wb, sb, zb = self.layout_sizes(N, K)
        wq = np.empty(wb, np.uint8)
        sp = np.empty(sb, np.uint8)
        zp = np.empty(zb, np.uint8)
        rc = self.lib.or_pack(N, K, q.ctypes.data, s.ctypes.data, z.ctypes.data,
                              wq.ctypes.data, sp.ctypes.data, zp.ctypes.data)
        if rc:
            raise ValueError("or_pack rejected its input")
        return wq, sp, zp

    def unpack(self, N, K, wq, sp, zp):
        G = K // GROUP
        q = np.empty((N, K), np.uint8)
        s = np.empty((N, G), np.uint16)
        z = np.empty((N, G), np.uint8)
        wq, sp, zp = (np.ascontiguousarray(a, dtype=np.uint8) for a in (wq, sp, zp))
        rc = self.lib.or_unpack(N, K, wq.ctypes.data, sp.ctypes.data, zp.ctypes.data,
                                q.ctypes.data, s.ctypes.data, z.ctypes.data)
        if rc:
            raise ValueError("or_unpack rejected its input")
        return q, s, z

    # -- arithmetic ---------------------------------------------------------
    def dequant(self, q, s, z):
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint16)
        z = np.ascontiguousarray(z, dtype=np.uint8)
        N, K = q.shape
        w = np.empty((N, K), np.float64)
        if self.lib.or_dequant(N, K, q.ctypes.data, s.ctypes.data, z.ctypes.data, w.ctypes.data):
            raise ValueError("or_dequant rejected its input")
        return w

    def quantize(self, w_f16_bits, mode):
        """fp16 bits [N][K] -> (q, s, z) by round-to-nearest; mode 0 symmetric
        (absmax / 7, z = 8), mode 1 asymmetric (min/max with 0, uint4 z)."""
        w_f16_bits = np.ascontiguousarray(w_f16_bits, dtype=np.uint16)
        N, K = w_f16_bits.shape
        G = K // GROUP
        q = np.empty((N, K), np.uint8)
        s = np.empty((N, G), np.uint16)
        z = np.empty((N, G), np.uint8)
        if self.lib.or_quantize(N, K, w_f16_bits.ctypes.data, int(mode), q.ctypes.data, s.ctypes.data,
                                z.ctypes.data):
            raise ValueError("or_quantize rejected its input")
        return q, s, z

    def gemv(self, q, s, z, x):
        """Returns (ref, absref), both float64 [M][N]."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint16)
        z = np.ascontiguousarray(z, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        N, K = q.shape
        M = x.shape[0]
        ref = np.empty((M, N), np.float64)
        absref = np.empty((M, N), np.float64)
        rc = self.lib.or_gemv(M, N, K, q.ctypes.data, s.ctypes.data, z.ctypes.data,
                              x.ctypes.data, ref.ctypes.data, absref.ctypes.data)
        if rc:
            raise ValueError("or_gemv rejected its input")
        return ref, absref

    def gemv_packed(self, M, N, K, wq, sp, zp, x, rows=None):
        """Product from layout-ID-2 buffers; with ``rows``, only those rows."""
        wq, sp, zp = (np.ascontiguousarray(a, dtype=np.uint8) for a in (wq, sp, zp))
        x = np.ascontiguousarray(x, dtype=np.uint16)
        if rows is None:
            ref = np.empty((M, N), np.float64)
            absref = np.empty((M, N), np.float64)
            rc = self.lib.or_gemv_packed(M, N, K, wq.ctypes.data, sp.ctypes.data, zp.ctypes.data,
                                         x.ctypes.data, ref.ctypes.data, absref.ctypes.data)
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            ref = np.empty((M, rows.size), np.float64)
            absref = np.empty((M, rows.size), np.float64)
            rc = self.lib.or_gemv_packed_rows(M, N, K, wq.ctypes.data, sp.ctypes.data,
                                              zp.ctypes.data, x.ctypes.data, rows.ctypes.data,
                                              rows.size, ref.ctypes.data, absref.ctypes.data)
        if rc:
            raise ValueError("or_gemv_packed rejected its input")
        return ref, absref

    # -- INT8 activations -----------------------------------------------------
    def act_quant_i8(self, x):
        """fp16 bits [M][K] -> (xq int8 [M][K], sx float32 [M][G], xsum int32
        [M][G]): symmetric codes per group of 128, decided in fp32."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        M, K = x.shape
        G = K // GROUP
        xq = np.empty((M, K), np.int8)
        sx = np.empty((M, G), np.float32)
        xsum = np.empty((M, G), np.int32)
        if self.lib.or_act_quant_i8(M, K, x.ctypes.data, xq.ctypes.data, sx.ctypes.data, xsum.ctypes.data):
            raise ValueError("or_act_quant_i8 rejected its input")
        return xq, sx, xsum

    def gemv_a8(self, q, s, z, xq, sx, rows=None):
        """Integer-sum product with int8 activations; returns (ref, absref)
        float64 [M][N], or [M][len(rows)] for the listed rows."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint16)
        z = np.ascontiguousarray(z, dtype=np.uint8)
        xq = np.ascontiguousarray(xq, dtype=np.int8)
        sx = np.ascontiguousarray(sx, dtype=np.float32)
        N, K = q.shape
        M = xq.shape[0]
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
        R = N if rows is None else rows.size
        ref = np.empty((M, R), np.float64)
        absref = np.empty((M, R), np.float64)
        rc = self.lib.or_gemv_a8(M, N, K, q.ctypes.data, s.ctypes.data, z.ctypes.data, xq.ctypes.data,
                                 sx.ctypes.data, None if rows is None else rows.ctypes.data, R,
                                 ref.ctypes.data, absref.ctypes.data)
        if rc:
            raise ValueError("or_gemv_a8 rejected its input")
        return ref, absref


# Acceptance bound of the workload definition: every output y (fp16, taken as
# a double) must satisfy |y - ref| <= REL * absref + ABS against the unrounded
# fp64 reference.
BOUND_REL = 2e-3
BOUND_ABS = 1e-5

# sup |d silu / dx| over the reals (attained near x = 2.40): silu' = s(1 + x(1 - s)),
# s the logistic function. Pinned numerically in the oracle pins.
SILU_LIPSCHITZ = 1.0999


def silu(v):
    """silu(v) = v / (1 + exp(-v)) in fp64 (the SwiGLU gate activation)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def gemv_swiglu(oracle, qg, sg, zg, qu, su, zu, x):
    """Fused gate/up + SwiGLU reference: y = silu(g) * u with g and u the
    fp64 GEMVs of the gate and up matrices (logical form), and a per-output
    acceptance bound derived from the GEMV bound:

    the kernel's g and u are fp32 sums within dg = REL*|Wg||x| + ABS and
    du = REL*|Wu||x| + ABS of the exact values (the GEMV bound, which also
    covers an fp16 rounding the fused path does not even make), so
        |silu(g~) u~ - silu(g) u| <= L dg (|u| + du) + |silu(g)| du,
    L = SILU_LIPSCHITZ; the fp32 epilogue and the final fp16 rounding add at
    most 2^-10 |y| more (plus ABS for underflow). Returns (ref, bound)."""
    g, ag = oracle.gemv(qg, sg, zg, x)
    u, au = oracle.gemv(qu, su, zu, x)
    return swiglu_bound(g, ag, u, au)


def swiglu_bound(g, ag, u, au):
    """SwiGLU reference and bound from the gate and up GEMVs' fp64 results
    (g, u) and their sums of |w x| (ag, au); see gemv_swiglu."""
    ref = silu(g) * u
    dg = BOUND_REL * ag + BOUND_ABS
    du = BOUND_REL * au + BOUND_ABS
    bound = SILU_LIPSCHITZ * dg * (np.abs(u) + du) + np.abs(silu(g)) * du + 2.0 ** -10 * np.abs(ref) + BOUND_ABS
    return ref, bound


def swiglu_report(y_f16_bits, ref, bound, oracle):
    """Returns (ok, worst) where worst = max |y-ref| / bound."""
    y = oracle.f16_to_f64(np.asarray(y_f16_bits, dtype=np.uint16))
    ratio = np.abs(y - ref) / bound
    ratio[np.isnan(ratio)] = np.inf
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= 1.0, worst


def bound_report(y_f16_bits, ref, absref, oracle):
    """Returns (ok, worst) where worst = max |y-ref| / (REL*absref + ABS)."""
    y = oracle.f16_to_f64(np.asarray(y_f16_bits, dtype=np.uint16))
    allow = BOUND_REL * absref + BOUND_ABS
    ratio = np.abs(y - ref) / allow
    ratio[np.isnan(ratio)] = np.inf
    worst = float(ratio.max()) if ratio.size else 0.0
    return worst <= 1.0, worst


_default = None


def get():
    """The default oracle, built on first use if the library is missing."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default
