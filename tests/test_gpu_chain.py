"""GPU parity of the GEMV chain (w4a16_chain_plan / w4a16_chain_run): a
sequence of GEMVs run in one persistent launch, each reading an earlier
GEMV's output.

Every output of every GEMV is checked against the oracle, the input of a
chained GEMV being the GPU's own fp16 output of its producer (first K
columns) times 2^-x_shift, rounded to fp16 on the host. Where the chain's
waves and shares equal a standalone entry point's (the 7B shapes), the
output must equal that entry point's on the same input, bit for bit. Runs
must be bit-identical, and the workspace's error word must stay 0."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import oracle
import synthetic
from tests.gpu_common import torch_dev, upload

pytestmark = pytest.mark.gpu


def rescale(y_bits, K, shift):
    """Host copy of the chain's input rule: first K columns, times 2^-shift
    (exact in fp32), rounded to fp16 (nearest even)."""
    y = np.ascontiguousarray(y_bits[:, :K]).view(np.float16).astype(np.float32)
    return (y * np.float32(2.0 ** -shift)).astype(np.float16).view(np.uint16)


class Chain:
    """Device buffers of a chain; logical weights kept when drawn on the host."""

    def __init__(self, M, spec, seed, device_weights=False):
        torch, dev = torch_dev()
        self.M, self.spec, self.ops, self.logical = M, spec, [], []
        for i, (kind, N, K, splits, x_src, x_shift) in enumerate(spec):
            rows = 16 * ((N + 7) // 8) if kind == w.CHAIN_SWIGLU else N
            if device_weights:
                wq, sc, zp = synthetic.device_packed_weights(rows, K, seed, 100 + i, dev)
                self.logical.append(None)
            else:
                if kind == w.CHAIN_SWIGLU:
                    g = synthetic.weights(N, K, seed=seed, tensor_id=2 * i + 100)
                    u = synthetic.weights(N, K, seed=seed, tensor_id=2 * i + 101)
                    packed = w.w4a16_pack_gate_up(*g, *u)
                    self.logical.append((g, u))
                else:
                    lw = synthetic.weights(N, K, seed=seed, tensor_id=2 * i + 100)
                    packed = w.w4a16_pack(*lw)
                    self.logical.append(lw)
                wq, sc, zp = (upload(a) for a in packed)
            x = upload(synthetic.activations(M, K, seed=seed, tensor_id=i)) if x_src < 0 else None
            y = torch.full((M, N), -1, dtype=torch.int16, device=dev)
            self.ops.append(dict(kind=kind, N=N, K=K, splits=splits, x_src=x_src, x_shift=x_shift,
                                 wq=wq, scales=sc, zeros=zp, x=x, y=y))
        plan, self.ws_bytes = w.w4a16_chain_plan(M, self.ops)
        self.plan = torch.from_numpy(plan).to(dev)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)

    def run(self):
        torch, _ = torch_dev()
        print(f"chain run: {len(self.ops)} GEMVs, M={self.M}", flush=True)
        w.w4a16_chain_run(self.M, self.plan, self.ws)
        torch.cuda.synchronize()
        err = int(self.ws[w.CHAIN_ERROR_OFFSET:w.CHAIN_ERROR_OFFSET + 4].cpu().numpy().view(np.uint32)[0])
        assert err == 0, f"chain error word {err}"
        return [o["y"].cpu().numpy().view(np.uint16).copy() for o in self.ops]

    def inputs(self, ys):
        """The input each GEMV read: external x, or its producer's output rescaled."""
        xs = []
        for i, o in enumerate(self.ops):
            if o["x_src"] < 0:
                xs.append(o["x"].cpu().numpy().view(np.uint16))
            else:
                xs.append(rescale(ys[o["x_src"]], o["K"], o["x_shift"]))
        return xs


def check_oracle(chain, ys, xs, only=None):
    orc = oracle.get()
    worst = 0.0
    for i, o in enumerate(chain.ops):
        if only is not None and i not in only:
            continue
        M, N, K = chain.M, o["N"], o["K"]
        if chain.logical[i] is not None:
            if o["kind"] == w.CHAIN_SWIGLU:
                (g, u) = chain.logical[i]
                ref, bound = oracle.gemv_swiglu(orc, *g, *u, xs[i])
                ok, r = oracle.swiglu_report(ys[i], ref, bound, orc)
            else:
                ref, absref = orc.gemv(*chain.logical[i], xs[i])
                ok, r = oracle.bound_report(ys[i], ref, absref, orc)
        else:
            host = [t.cpu().numpy() for t in (o["wq"], o["scales"], o["zeros"])]
            wq, sp, zp = host[0], host[1].view(np.uint8), host[2]
            if o["kind"] == w.CHAIN_SWIGLU:
                # packed rows: per 16-row tile, 8 gate rows then the 8 up rows of the same outputs
                NT = (N + 7) // 8
                r2, a2 = orc.gemv_packed(M, 16 * NT, K, wq, sp, zp, xs[i])
                blk = lambda a, h: a.reshape(M, NT, 2, 8)[:, :, h, :].reshape(M, 8 * NT)[:, :N]
                ref, bound = oracle.swiglu_bound(blk(r2, 0), blk(a2, 0), blk(r2, 1), blk(a2, 1))
                ok, r = oracle.swiglu_report(ys[i], ref, bound, orc)
            else:
                ref, absref = orc.gemv_packed(M, N, K, wq, sp, zp, xs[i])
                ok, r = oracle.bound_report(ys[i], ref, absref, orc)
        assert ok, (i, o["kind"], N, K, r)
        worst = max(worst, r)
    return worst


def standalone(o, x_bits, M):
    """The standalone entry point with the chain's waves and shares, on x."""
    torch, dev = torch_dev()
    x = upload(x_bits)
    y = torch.full((M, o["N"]), -1, dtype=torch.int16, device=dev)
    if o["kind"] == w.CHAIN_SWIGLU:
        w.w4a16_gemv_swiglu(M, o["N"], o["K"], o["wq"], o["scales"], o["zeros"], x, y)
    elif o["splits"] > 1:
        ws = torch.zeros(w.w4a16_splitk_workspace_bytes(M, o["N"], o["splits"]), dtype=torch.uint8, device=dev)
        w.w4a16_gemv_splitk(M, o["N"], o["K"], o["splits"], o["wq"], o["scales"], o["zeros"], x, y, ws)
    else:
        w.w4a16_gemv(M, o["N"], o["K"], o["wq"], o["scales"], o["zeros"], x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


MIXED = [(w.CHAIN_GEMV, 520, 1024, 1, -1, 0),     # external x, tile pairs, ragged last pair
         (w.CHAIN_GEMV, 300, 512, 2, 0, 3),       # split K, fed by GEMV 0
         (w.CHAIN_SWIGLU, 200, 256, 1, 1, 2),     # gate/up rows fed by the split GEMV (25 tiles: a clamped pair)
         (w.CHAIN_GEMV, 96, 128, 1, 2, 0),        # one group (empty shares), fed by the SwiGLU output
         (w.CHAIN_GEMV, 64, 7168, 1, -1, 0),      # 8 waves per tile
         (w.CHAIN_GEMV, 33, 4864, 4, -1, 0),      # split, ragged
         (w.CHAIN_GEMV, 1000, 512, 1, 0, 3),      # a second consumer of GEMV 0
         (w.CHAIN_GEMV, 7296, 256, 1, -1, 0),     # a wide producer
         (w.CHAIN_GEMV, 40, 7296, 1, 7, 2),       # 8 waves, shares in two rounds, fed by GEMV 7
         (w.CHAIN_SWIGLU, 36, 7296, 1, -1, 0),    # gate/up rows, 8 waves, shares in two rounds, ragged
         (w.CHAIN_GEMV, 200, 18944, 1, -1, 0)]    # three rounds


def test_chain_mixed_kinds_against_oracle_and_repeat():
    chain = Chain(1, MIXED, seed=21)
    ys = chain.run()
    check_oracle(chain, ys, chain.inputs(ys))
    again = chain.run()  # a new launch number: the tags of the first run are stale now
    for a, b in zip(ys, again):
        assert np.array_equal(a, b)


def layer_spec(layers, lm_head, down_splits=4):
    spec = []
    for layer in range(layers):
        base = len(spec)
        src = base - 1
        spec.append((w.CHAIN_GEMV, 4608, 3584, 1, src, 10 if src >= 0 else 0))  # qkv, from the previous down
        spec.append((w.CHAIN_GEMV, 3584, 3584, 1, base, 3))                    # o, from qkv (stands for attention)
        spec.append((w.CHAIN_SWIGLU, 18944, 3584, 1, base + 1, 3))             # gate/up + SwiGLU, from o
        spec.append((w.CHAIN_GEMV, 3584, 18944, down_splits, base + 2, 0))     # down, from the SwiGLU output
    if lm_head:
        spec.append((w.CHAIN_GEMV, 152064, 3584, 1, len(spec) - 1, 10))
    return spec


def test_chain_7b_layers_bit_identical_to_standalone():
    chain = Chain(1, layer_spec(2, lm_head=True), seed=22, device_weights=True)
    ys = chain.run()
    xs = chain.inputs(ys)
    for i, o in enumerate(chain.ops):
        ref = standalone(o, xs[i], 1)
        assert np.array_equal(ys[i], ref), (i, o["N"], o["K"])
    check_oracle(chain, ys, xs)


def test_chain_7b_layers_unsplit_down_in_rounds():
    """The down projection unsplit: 8 waves per tile, each taking its 18 or 19
    groups in three rounds. Every other GEMV still equals its standalone
    entry point; every GEMV is within the oracle's bound."""
    chain = Chain(1, layer_spec(2, lm_head=False, down_splits=1), seed=24, device_weights=True)
    ys = chain.run()
    xs = chain.inputs(ys)
    check_oracle(chain, ys, xs)
    for i, o in enumerate(chain.ops):
        if o["K"] != 18944:
            assert np.array_equal(ys[i], standalone(o, xs[i], 1)), i
    again = chain.run()
    for a, b in zip(ys, again):
        assert np.array_equal(a, b)


def test_chain_full_7b_step_oracle_sampled_and_repeat():
    chain = Chain(1, layer_spec(28, lm_head=True), seed=23, device_weights=True)
    ys = chain.run()
    xs = chain.inputs(ys)
    # the first layer, a middle one, the last one and the lm_head, against the oracle
    check_oracle(chain, ys, xs, only=set(range(4)) | set(range(56, 60)) | set(range(108, 113)))
    # every GEMV against the standalone entry point on the same input
    for i in range(0, len(chain.ops), 7):
        assert np.array_equal(ys[i], standalone(chain.ops[i], xs[i], 1)), i
    for _ in range(2):
        again = chain.run()
        for a, b in zip(ys, again):
            assert np.array_equal(a, b)


def test_chain_error_paths_from_the_host():
    """Failure handling, forced from the host with every workgroup leaving
    normally: a workspace smaller than the plan's is refused by the kernel
    (error word 2, outputs untouched); a nonzero error word is sticky (later
    runs return at once, outputs untouched) until the caller clears it."""
    torch, _ = torch_dev()
    chain = Chain(1, MIXED[:3], seed=25)
    off = w.CHAIN_ERROR_OFFSET
    err = lambda: int(chain.ws[off:off + 4].cpu().numpy().view(np.uint32)[0])
    # too small a workspace (the header fits): the kernel refuses the plan
    print("chain error path: short workspace", flush=True)
    w.w4a16_chain_run(1, chain.plan, chain.ws[:256])
    torch.cuda.synchronize()
    assert err() == 2
    assert all((o["y"].cpu().numpy() == -1).all() for o in chain.ops)  # nothing written
    # sticky: a run on the full workspace with the error word still set does nothing
    print("chain error path: sticky error word", flush=True)
    w.w4a16_chain_run(1, chain.plan, chain.ws)
    torch.cuda.synchronize()
    assert err() == 2
    assert all((o["y"].cpu().numpy() == -1).all() for o in chain.ops)
    # cleared by the caller: the chain runs and checks out
    chain.ws.zero_()
    torch.cuda.synchronize()
    ys = chain.run()
    check_oracle(chain, ys, chain.inputs(ys))
