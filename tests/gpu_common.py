"""Shared helpers of the GPU tests: upload packed inputs, run the C-ABI
entry points through the binding, compare with the oracle."""
import numpy as np

import int4_weight_only_w4a16_amd as w
import oracle
import synthetic


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def upload(a):
    torch, dev = torch_dev()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


class Problem:
    """Seeded logical inputs, their packed form on the device, and the oracle."""

    def __init__(self, M, N, K, seed=0, q=None, s=None, z=None, x=None):
        self.M, self.N, self.K = M, N, K
        if q is None:
            q, s, z = synthetic.weights(N, K, seed=seed, tensor_id=1)
        if x is None:
            x = synthetic.activations(M, K, seed=seed, tensor_id=2)
        self.q, self.s, self.z, self.x = q, s, z, x
        self.packed = w.w4a16_pack(q, s, z)
        self.wq_d, self.sp_d, self.zp_d = (upload(a) for a in self.packed)
        self.x_d = upload(x)
        self._ref = None

    def reference(self):
        if self._ref is None:
            self._ref = oracle.get().gemv(self.q, self.s, self.z, self.x)
        return self._ref

    def new_y(self):
        torch, dev = torch_dev()
        return torch.full((self.M, self.N), -1, dtype=torch.int16, device=dev)  # fp16 NaN pattern

    def gemv(self, x_d=None):
        torch, _ = torch_dev()
        y = self.new_y()
        w.w4a16_gemv(self.M, self.N, self.K, self.wq_d, self.sp_d, self.zp_d,
                     self.x_d if x_d is None else x_d, y)
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint16)

    def splitk_workspace(self, splits):
        """Zero-filled workspace of exactly the size the library asks for."""
        torch, dev = torch_dev()
        return torch.zeros(max(16, w.w4a16_splitk_workspace_bytes(self.M, self.N, splits)),
                           dtype=torch.uint8, device=dev)

    def gemv_splitk(self, splits, ws=None):
        torch, dev = torch_dev()
        y = self.new_y()
        if ws is None:
            ws = self.splitk_workspace(splits)
        w.w4a16_gemv_splitk(self.M, self.N, self.K, splits, self.wq_d, self.sp_d, self.zp_d, self.x_d, y, ws)
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint16)

    def gemm_splitk(self, splits, ws=None):
        torch, dev = torch_dev()
        y = self.new_y()
        if ws is None:
            ws = self.splitk_workspace(splits)
        w.w4a16_gemm_splitk(self.M, self.N, self.K, splits, self.wq_d, self.sp_d, self.zp_d, self.x_d, y, ws)
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint16)

    def gemm_partials(self, splits, part=None):
        """w4a16_gemm_splitk_partials; a fresh buffer is filled with NaN bits
        first (the call must write every partial before reading it)."""
        torch, dev = torch_dev()
        y = self.new_y()
        if part is None:
            part = torch.full((max(16, w.w4a16_gemm_partials_bytes(self.M, self.N, splits)),), 0xFF,
                              dtype=torch.uint8, device=dev)
        w.w4a16_gemm_splitk_partials(self.M, self.N, self.K, splits, self.wq_d, self.sp_d, self.zp_d, self.x_d, y,
                                     part)
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint16)

    def workspace_is_zero(self, ws):
        """Every split-K call leaves its accumulation words at zero."""
        return not ws.cpu().numpy().any()

    def check(self, y):
        ref, absref = self.reference()
        ok, worst = oracle.bound_report(y, ref, absref, oracle.get())
        assert ok, f"M={self.M} N={self.N} K={self.K}: worst |y-ref|/bound = {worst}"
        return worst
