"""CPU checks of the GEMV chain's plan (w4a16_chain_plan) and of the walk the
persistent kernel makes over it, without a GPU.

The plan is a byte image of descriptors. The test parses it and replays, in
numpy, the index arithmetic each wave of the kernel performs for every work
item: which row tile and groups a compute wave requests, where its x slice
comes from, and which outputs the item's epilogue writes. It checks that every
request stays inside its buffer, that the waves' shares cover every K range
exactly once, that every output is written exactly once, and that each item
depends only on items with smaller numbers (the progress argument of the
kernel). Device pointers are fake, aligned and never dereferenced."""
import numpy as np
import pytest

import int4_weight_only_w4a16_amd as w
import synthetic

HEADER = np.dtype([("magic", "<u4"), ("M", "<i4"), ("n_ops", "<i4"), ("total", "<i4"), ("plan_bytes", "<u8"),
                   ("ws_bytes", "<u8"), ("reserved", "<i4", 8)])
OPDEV = np.dtype([("wq", "<u8"), ("sw", "<u8"), ("zw", "<u8"), ("x_ext", "<u8"), ("y", "<u8"), ("yt_off", "<u8"),
                  ("xt_off", "<u8"), ("acc_off", "<u8"), ("N", "<i4"), ("K", "<i4"), ("G", "<i4"), ("kind", "<i4"),
                  ("splits", "<i4"), ("tp", "<i4"), ("wpt", "<i4"), ("row_tiles", "<i4"), ("per_split", "<i4"),
                  ("items", "<i4"), ("item_begin", "<i4"), ("x_shift", "<i4"), ("x_stride", "<i4"),
                  ("sentinel", "<i4"), ("x_src", "<i4"), ("split_q", "<i4"), ("rounds", "<i4"), ("pad", "<i4", 3)])
WAVES, SHARE, LANES = 8, 7, 64


class Fake:
    """Distinct aligned fake addresses, with the size of each buffer."""

    def __init__(self):
        self.next = 1 << 40
        self.sizes = {}

    def alloc(self, nbytes):
        a = self.next
        self.sizes[a] = nbytes
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return a


def make_ops(M, spec):
    """spec: list of (kind, N, K, splits, x_src, x_shift). Returns (ops, sizes)."""
    fake = Fake()
    ops = []
    for kind, N, K, splits, x_src, x_shift in spec:
        rows = 16 * ((N + 7) // 8) if kind == w.CHAIN_SWIGLU else N
        wb, sb, zb = w.w4a16_packed_sizes(rows, K)
        ops.append(dict(kind=kind, N=N, K=K, splits=splits, x_src=x_src, x_shift=x_shift,
                        wq=fake.alloc(wb), scales=fake.alloc(sb), zeros=fake.alloc(zb),
                        x=fake.alloc(2 * M * K) if x_src < 0 else None, y=fake.alloc(2 * M * N)))
    return ops, fake.sizes


def parse(plan):
    h = np.frombuffer(plan[:HEADER.itemsize].tobytes(), HEADER)[0]
    d = np.frombuffer(plan[HEADER.itemsize:].tobytes(), OPDEV)
    return h, d


def share_of(d, i, wave, rd=0):
    """The kernel's share_of(), element for element, for round rd."""
    per_split = int(d["per_split"])
    split, tg = i // per_split, i % per_split
    lt, wi = wave // int(d["wpt"]), wave % int(d["wpt"])
    tile = min(tg * int(d["tp"]) + lt, int(d["row_tiles"]) - 1)
    G, S, wpt = int(d["G"]), int(d["splits"]), int(d["wpt"])
    g_beg = 0 if S == 1 else split * G // S
    g_end = G if S == 1 else (split + 1) * G // S
    ng = g_end - g_beg
    beg = g_beg + wi * ng // wpt + rd * SHARE
    end = g_beg + (wi + 1) * ng // wpt
    return tile, beg, min(end - beg, SHARE)


def walk(plan, ops, sizes, M):
    """Replays the kernel's index arithmetic over every item and wave."""
    h, d = parse(plan)
    assert h["magic"] == 0x57344348 and h["M"] == M and h["n_ops"] == len(ops)
    assert d["items"].sum() == h["total"]
    assert (np.diff(d["item_begin"]) == d["items"][:-1]).all() and d["item_begin"][0] == 0
    ws_bytes = int(h["ws_bytes"])
    lanes = np.arange(LANES)
    rlane = lanes & 15
    covered = [np.zeros((int(e["row_tiles"]), int(e["G"])), np.int32) for e in d]
    written = [np.zeros((M, int(e["N"])), np.int32) for e in d]
    for j, e in enumerate(d):
        o = ops[j]
        G, N = int(e["G"]), int(e["N"])
        # a SwiGLU matrix: 8 outputs per 16-row tile (gate rows 0-7, up rows 8-15)
        matrix_rows = 16 * ((N + 7) // 8) if e["kind"] == w.CHAIN_SWIGLU else N
        assert int(e["row_tiles"]) == (matrix_rows + 15) // 16
        wb, sb, zb = w.w4a16_packed_sizes(matrix_rows, int(e["K"]))
        assert sizes[int(e["wq"])] == wb and sizes[int(e["sw"])] == sb and sizes[int(e["zw"])] == zb
        if e["x_src"] >= 0:
            p = int(e["x_src"])
            assert p < j and int(d[p]["N"]) >= int(e["K"]) and int(e["x_stride"]) == int(d[p]["N"])
            assert d[p]["yt_off"] == e["xt_off"] and e["xt_off"] >= 256
            assert e["xt_off"] + 4 * M * int(d[p]["N"]) <= ws_bytes
            assert e["sentinel"] == (M - 1) * int(d[p]["N"]) + int(d[p]["N"]) - 1
            # every item of the producer comes before every item of this GEMV
            assert d[p]["item_begin"] + d[p]["items"] <= e["item_begin"]
        if e["splits"] > 1:
            assert e["acc_off"] >= 256 and e["acc_off"] + 8 * M * N <= ws_bytes and e["acc_off"] % 256 == 0
        # staging of the whole input: 16-byte chunks of tagged words (4 per
        # chunk) or of external fp16 values (8 per chunk), all rows
        K = int(e["K"])
        if e["x_src"] >= 0:
            c = np.arange(M * K // 4)
            m, cw = c // (K // 4), c % (K // 4)
            word = m * int(e["x_stride"]) + cw * 4
            assert (word + 4 <= M * int(e["x_stride"])).all() and (cw * 4 + 4 <= K).all()
        else:
            c = np.arange(M * K // 8)
            m, cw = c // (K // 8), c % (K // 8)
            assert ((m * K + cw * 8) * 2 + 16 <= sizes[int(e["x_ext"])]).all()
        assert K <= 32768  # the LDS x buffer
        for i in range(int(e["items"])):
            for wave, rd in ((wv, r) for wv in range(WAVES) for r in range(int(e["rounds"]))):
                tile, beg, n = share_of(e, i, wave, rd)
                assert n <= SHARE, (j, i, wave, n)
                if n <= 0:
                    continue
                assert 0 <= tile < covered[j].shape[0]
                unclamped = (i % int(e["per_split"])) * int(e["tp"]) + wave // int(e["wpt"])
                if unclamped < int(e["row_tiles"]):
                    covered[j][tile, beg:beg + n] += 1  # a pair's missing second tile repeats the last, unstored
                q0 = tile * G
                gg = beg + np.minimum(np.arange(SHARE), n - 1)
                # weight, scale and zero requests against their buffers
                # (the resource starts at tile (tile, 0) and holds G tiles)
                assert ((q0 + gg) * 1024 + 1024 <= wb).all() and (gg * 1024 + lanes.max() * 16 + 16 <= G * 1024).all()
                assert ((q0 + gg) * 32 + (rlane.max() >> 1) * 4 + 4 <= sb).all()
                assert ((q0 + gg) * 8 + (rlane.max() >> 3) * 4 + 4 <= zb).all()
            # outputs of the item (its epilogue)
            split, tg = i // int(e["per_split"]), i % int(e["per_split"])
            per_tile = 8 if e["kind"] == w.CHAIN_SWIGLU else 16
            for lt in range(int(e["tp"])):
                t = tg * int(e["tp"]) + lt
                if t >= int(e["row_tiles"]):
                    continue
                n_idx = t * per_tile + np.arange(per_tile)
                n_idx = n_idx[n_idx < N]
                if split == int(e["splits"]) - 1:  # counted once per output
                    written[j][:, n_idx] += 1
        # the K range of every tile is covered exactly once over splits and waves
        assert (covered[j] == 1).all(), j
        assert (written[j] == 1).all(), j
    return h, d


@pytest.mark.parametrize("M", [1])
def test_mixed_chain_plan_walk(M):
    spec = [(w.CHAIN_GEMV, 520, 1024, 1, -1, 0),      # external x, pairs of tiles, ragged last pair
            (w.CHAIN_GEMV, 300, 512, 2, 0, 3),        # split K from a producer, ragged N
            (w.CHAIN_SWIGLU, 200, 256, 1, 1, 2),      # gate/up rows from the split GEMV's output, ragged
            (w.CHAIN_GEMV, 96, 128, 1, 2, 0),         # one group: empty shares
            (w.CHAIN_GEMV, 64, 7168, 1, -1, 0),       # 8 waves per tile
            (w.CHAIN_GEMV, 33, 4864, 4, -1, 0),       # split, 8 waves, ragged
            (w.CHAIN_GEMV, 40, 128 * 57, 1, -1, 0),   # 8 waves, two rounds (7 + 1 tiles at most)
            (w.CHAIN_SWIGLU, 36, 128 * 57, 1, -1, 0), # gate/up rows, 8 waves, two rounds, ragged
            (w.CHAIN_GEMV, 3584, 18944, 1, -1, 0)]    # unsplit down projection: three rounds
    ops, sizes = make_ops(M, spec)
    plan, ws = w.w4a16_chain_plan(M, ops)
    h, d = walk(plan, ops, sizes, M)
    assert list(d["wpt"]) == [4, 4, 4, 4, 8, 4, 8, 8, 8] and list(d["tp"]) == [2, 2, 2, 2, 1, 2, 1, 1, 1]
    assert list(d["rounds"]) == [1, 1, 1, 1, 1, 1, 2, 2, 3]
    assert ws == h["ws_bytes"]


def step_7b(M=1):
    spec = []
    for layer in range(synthetic.QWEN7B_LAYERS):
        base = len(spec)
        src = base - 1  # the previous layer's down projection (or the external input)
        spec.append((w.CHAIN_GEMV, 4608, 3584, 1, src, 10 if src >= 0 else 0))
        spec.append((w.CHAIN_GEMV, 3584, 3584, 1, base, 3))
        spec.append((w.CHAIN_SWIGLU, 18944, 3584, 1, base + 1, 3))
        spec.append((w.CHAIN_GEMV, 3584, 18944, 4, base + 2, 0))
    spec.append((w.CHAIN_GEMV, 152064, 3584, 1, len(spec) - 1, 10))
    return spec


def test_7b_step_plan_walk():
    M = 1
    ops, sizes = make_ops(M, step_7b(M))
    plan, ws = w.w4a16_chain_plan(M, ops)
    h, d = walk(plan, ops, sizes, M)
    assert h["n_ops"] == 113
    # 4 waves x 7 groups at K = 3584 (two tiles per item), 8 waves x 5 at 37-group splits
    assert set(d["wpt"][d["K"] == 3584]) == {4} and set(d["wpt"][d["K"] == 18944]) == {8}
    assert set(d["splits"][d["K"] == 18944]) == {4} and set(d["rounds"]) == {1}
    # the workspace holds the tagged handoff words and the split-K words
    assert ws == h["ws_bytes"] and ws < 8 << 20


def test_chain_plan_rejects():
    M = 1
    ops, _ = make_ops(M, [(w.CHAIN_GEMV, 64, 256, 1, -1, 0)])
    bad = dict(ops[0])
    for key, val, want in [("kind", 2, w.W4A16_EINVAL), ("K", 200, w.W4A16_EINVAL), ("splits", 3, w.W4A16_EINVAL),
                           ("x_src", 0, w.W4A16_EINVAL), ("N", 0, w.W4A16_EINVAL)]:
        o = dict(bad, **{key: val})
        with pytest.raises(w.W4A16Error) as e:
            w.w4a16_chain_plan(M, [o])
        assert e.value.status == want, key
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_chain_plan(M, [dict(bad, wq=bad["wq"] + 8)])
    assert e.value.status == w.W4A16_EINVAL
    # a producer narrower than the consumer's K; a shift out of range
    two, _ = make_ops(M, [(w.CHAIN_GEMV, 64, 256, 1, -1, 0), (w.CHAIN_GEMV, 64, 128, 1, 0, 0)])
    for o1, want in [(dict(two[1], K=256), w.W4A16_EINVAL), (dict(two[1], x_shift=25), w.W4A16_EINVAL)]:
        with pytest.raises(w.W4A16Error) as e:
            w.w4a16_chain_plan(M, [two[0], o1])
        assert e.value.status == want
    # SwiGLU takes no split; K beyond the LDS input buffer is unsupported
    sw, _ = make_ops(M, [(w.CHAIN_SWIGLU, 64, 5120, 1, -1, 0)])
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_chain_plan(M, [dict(sw[0], splits=2)])
    assert e.value.status == w.W4A16_EINVAL
    big, _ = make_ops(M, [(w.CHAIN_GEMV, 64, 32768 + 128, 1, -1, 0)])
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_chain_plan(M, big)
    assert e.value.status == w.W4A16_EUNSUPPORTED
    # run-time argument checks (no GPU touched)
    L = w.lib()
    assert L.w4a16_chain_run(1, None, 1 << 20, 4096, None) == w.W4A16_EINVAL
    assert L.w4a16_chain_run(1, 1 << 20, (1 << 20) + 8, 4096, None) == w.W4A16_EINVAL
    assert L.w4a16_chain_run(1, 1 << 20, 1 << 20, 100, None) == w.W4A16_EINVAL
    assert L.w4a16_chain_run(9, 1 << 20, 1 << 20, 4096, None) == w.W4A16_EUNSUPPORTED


class Walk:
    """The kernel's incremental walk (walk_enter / walk_advance, one round per
    advance), field for field."""

    def __init__(self, d, k):
        self.d, self.k, self.op = d, k, 0
        self.enter()

    def enter(self):
        d = self.d
        while self.k >= d[self.op]["item_begin"] + d[self.op]["items"]:
            self.op += 1
        e = d[self.op]
        self.end = int(e["item_begin"] + e["items"])
        self.rd, self.rounds = 0, int(e["rounds"])
        self.G, self.S, self.per_split = int(e["G"]), int(e["splits"]), int(e["per_split"])
        self.sq = int(e["split_q"])
        self.sr = self.G - self.sq * self.S
        i = self.k - int(e["item_begin"])
        self.split, self.tg = i // self.per_split, i % self.per_split
        self.g_beg = self.split * self.G // self.S
        nxt = (self.split + 1) * self.G
        self.g_end, self.r_end = nxt // self.S, nxt % self.S

    def advance(self, P, total):
        self.rd += 1
        if self.rd < self.rounds:
            return
        self.rd = 0
        self.k += P
        if self.k >= total:
            return
        if self.k >= self.end:
            self.enter()
            return
        self.tg += P
        while self.tg >= self.per_split:
            self.tg -= self.per_split
            self.split += 1
            self.g_beg = self.g_end
            self.g_end += self.sq
            self.r_end += self.sr
            if self.r_end >= self.S:
                self.g_end += 1
                self.r_end -= self.S


@pytest.mark.parametrize("P", [1, 7, 100, 256, 300])
def test_incremental_walk_matches_division(P):
    """Every workgroup's walk, advanced a round at a time and P items at a
    time, gives the GEMV, split, tile group, split range and round that
    direct division gives."""
    M = 1
    spec = [(w.CHAIN_GEMV, 520, 1024, 1, -1, 0), (w.CHAIN_GEMV, 300, 512, 2, 0, 3),
            (w.CHAIN_SWIGLU, 200, 256, 1, 1, 2), (w.CHAIN_GEMV, 96, 128, 1, 2, 0),
            (w.CHAIN_GEMV, 64, 7168, 1, -1, 0), (w.CHAIN_GEMV, 33, 4864, 4, -1, 0),
            (w.CHAIN_GEMV, 3584, 18944, 4, -1, 0), (w.CHAIN_GEMV, 2000, 3968, 31, -1, 0),
            (w.CHAIN_GEMV, 17, 1280, 7, -1, 0), (w.CHAIN_GEMV, 3584, 18944, 1, -1, 0),
            (w.CHAIN_SWIGLU, 48, 5120, 1, -1, 0)]
    ops, _ = make_ops(M, spec)
    plan, _ = w.w4a16_chain_plan(M, ops)
    h, d = parse(plan)
    total = int(h["total"])
    begins = np.asarray(d["item_begin"], dtype=np.int64)
    for wg in range(min(P, total)):
        wk = Walk(d, wg)
        while wk.k < total:
            j = int(np.searchsorted(begins, wk.k, side="right") - 1)
            e = d[j]
            i = wk.k - int(e["item_begin"])
            split, tg = i // int(e["per_split"]), i % int(e["per_split"])
            G, S = int(e["G"]), int(e["splits"])
            assert (wk.op, wk.split, wk.tg) == (j, split, tg)
            assert (wk.g_beg, wk.g_end) == (split * G // S, (split + 1) * G // S)
            for rd in range(int(e["rounds"])):  # every round of the item, in order
                assert (wk.k, wk.rd) == (int(e["item_begin"]) + i, rd)
                wk.advance(P, total)
