"""Every device entry point captured together in one graph and replayed:
each replay, with the test's own eager work and synchronizations between
replays, must give the eager results bit for bit (the header promises that
device calls can be graph-captured: no allocation, no host synchronization,
no memset nodes)."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import synthetic
from tests.gpu_common import Problem, torch_dev, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[graphs]", *a, flush=True)


def test_all_entry_points_in_one_graph():
    torch, dev = torch_dev()
    _say("build inputs")
    # Plain and split-K GEMV (M = 3), INT8 activations (M = 2), GEMM (M = 70,
    # plain and split-K)
    # and dequantization share one 16-byte-aligned set of problems.
    pg = Problem(3, 1000, 4864, seed=31)
    splits = 4
    ws = pg.splitk_workspace(splits)
    pa = Problem(2, 777, 2048, seed=32)
    G = pa.K // 128
    pm = Problem(70, 300, 640, seed=33)
    ws_m = pm.splitk_workspace(3)
    gate = synthetic.weights(200, 1024, seed=34, tensor_id=1)
    up = synthetic.weights(200, 1024, seed=34, tensor_id=2)
    sw_packed = [upload(a) for a in w.w4a16_pack_gate_up(*gate, *up)]
    sw_x = upload(synthetic.activations(2, 1024, seed=35))

    outs = {
        "gemv": torch.empty((3, 1000), dtype=torch.int16, device=dev),
        "splitk": torch.empty((3, 1000), dtype=torch.int16, device=dev),
        "xq": torch.empty((2, pa.K), dtype=torch.int8, device=dev),
        "sx": torch.empty((2, G), dtype=torch.float32, device=dev),
        "xsum": torch.empty((2, G), dtype=torch.int32, device=dev),
        "a8": torch.empty((2, 777), dtype=torch.int16, device=dev),
        "a8_fused": torch.empty((2, 777), dtype=torch.int16, device=dev),
        "gemm": torch.empty((70, 300), dtype=torch.int16, device=dev),
        "gemm_splitk": torch.empty((70, 300), dtype=torch.int16, device=dev),
        "dequant": torch.empty((300, 640), dtype=torch.float16, device=dev),
        "swiglu": torch.empty((2, 200), dtype=torch.int16, device=dev),
    }

    def launch_all(stream):
        w.w4a16_gemv(3, 1000, 4864, pg.wq_d, pg.sp_d, pg.zp_d, pg.x_d, outs["gemv"], stream=stream)
        w.w4a16_gemv_splitk(3, 1000, 4864, splits, pg.wq_d, pg.sp_d, pg.zp_d, pg.x_d, outs["splitk"], ws,
                            stream=stream)
        w.w4a16_act_quant_i8(2, pa.K, pa.x_d, outs["xq"], outs["sx"], outs["xsum"], stream=stream)
        w.w4a16_gemv_a8(2, 777, pa.K, pa.wq_d, pa.sp_d, pa.zp_d, outs["xq"], outs["sx"], outs["xsum"],
                        outs["a8"], stream=stream)
        w.w4a16_gemv_a8_fused(2, 777, pa.K, pa.wq_d, pa.sp_d, pa.zp_d, pa.x_d, outs["a8_fused"], stream=stream)
        w.w4a16_gemm(70, 300, 640, pm.wq_d, pm.sp_d, pm.zp_d, pm.x_d, outs["gemm"], stream=stream)
        w.w4a16_gemm_splitk(70, 300, 640, 3, pm.wq_d, pm.sp_d, pm.zp_d, pm.x_d, outs["gemm_splitk"], ws_m,
                            stream=stream)
        w.w4a16_dequant_f16(300, 640, pm.wq_d, pm.sp_d, pm.zp_d, outs["dequant"], stream=stream)
        w.w4a16_gemv_swiglu(2, 200, 1024, *sw_packed, sw_x, outs["swiglu"], stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return {k: v.cpu().numpy().copy() for k, v in outs.items()}

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    _say("eager")
    with torch.cuda.stream(stream):
        launch_all(stream)
    eager = snapshot()
    _say("capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            launch_all(stream)
    for rep in range(3):
        for v in outs.values():
            if v.dtype == torch.float16:
                v.fill_(float("nan"))
            else:
                v.fill_(-1)
        # Eager work of the program's own between replays: a split-K call into
        # another output, through the same workspace, on the same stream.
        other = torch.empty((3, 1000), dtype=torch.int16, device=dev)
        with torch.cuda.stream(stream):
            w.w4a16_gemv_splitk(3, 1000, 4864, splits, pg.wq_d, pg.sp_d, pg.zp_d, pg.x_d, other, ws,
                                stream=stream)
        torch.cuda.synchronize()
        _say("replay", rep)
        g.replay()
        got = snapshot()
        for k in outs:
            assert np.array_equal(got[k].view(np.uint8), eager[k].view(np.uint8)), (rep, k)
        assert pg.workspace_is_zero(ws) and pm.workspace_is_zero(ws_m)
        assert np.array_equal(other.cpu().numpy(), eager["splitk"])
    # The eager results themselves are right (each path has its own parity
    # tests; these spot checks tie the graph to them).
    pg.check(eager["gemv"].view(np.uint16))
    pg.check(eager["splitk"].view(np.uint16))
    pm.check(eager["gemm_splitk"].view(np.uint16))
    assert np.array_equal(eager["a8_fused"], eager["a8"])
