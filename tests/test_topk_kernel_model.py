"""A CPU model of the index arithmetic of the wide-row top-k kernels (topk_hist_kernel and
topk_final_kernel in csrc/topk.hip), run on the host only.

For every workgroup, wave and lane the model forms the addresses the kernels form — the
16-byte row loads from clamped positions and the separate tail, the histogram workspace slots,
the per-wave LDS candidate lists with their capacity guard, and the output positions of the
ordered compaction (list path and full-row fallback) — and asserts that each stays inside its
buffer, that the histogram pass counts every element of a row exactly once, and that the
positions written are exactly 0 .. min(k, n) - 1 holding the oracle's top-k.  Shapes: the GPU
tests' wide rows, the per-head (128 rows x 131072, k = 2622) and speculative-verify
(512 x 65536, k = 2048) selections, aligned and unaligned row strides, and data with heavy
ties (lists that overflow their LDS store and take the fallback).  The constants below are the
kernels' own."""
import numpy as np
import pytest

import oracle

THREADS_LARGE, WAVES_LARGE, WAVE = 1024, 16, 64
BINS, BIN_SHIFT = 4096, 20
LIST_PER_WAVE = 496
CAND_MAX = WAVES_LARGE * LIST_PER_WAVE
HIST_THREADS, HIST_UNROLL = 256, 4
FINAL_UNROLL = 8
CUS = 256


def order_keys(x):
    u = np.asarray(x, np.float32).copy().view(np.uint32)
    u[u == 0x80000000] = 0
    k = np.where((u & 0x80000000) != 0, ~u, u | 0x80000000).astype(np.uint32)
    k[np.isnan(np.asarray(x, np.float32))] = 0
    return k


def hist_chunks(rows):
    want = (4 * CUS + rows - 1) // max(rows, 1)
    return max(1, min(32, want))


def keys4_positions(i, n, aligned):
    """Element positions one keys4_load of group i reads (and whether the group owns them)."""
    if aligned:
        last = (n - 4) & ~3
        base = np.minimum(i, last)
        pos = base[..., None] + np.arange(4)
        own = i <= last
    else:
        pos = np.minimum(i[..., None] + np.arange(4), n - 1)
        own = np.ones_like(i, dtype=bool)
    return pos, own


def keys4_tail(n, aligned):
    return ((n - 4) & ~3) + 4 if aligned else n


def model_hist(n, rows, aligned):
    """topk_hist_kernel: every load in bounds; each element counted by exactly one (chunk,
    thread, load) or by the tail; the workspace slot range of the row."""
    C = hist_chunks(rows)
    chunk = (((n + C - 1) // C) + 1023) // 1024 * 1024
    counted = np.zeros(n, np.int64)
    tid = np.arange(HIST_THREADS)
    for c in range(C):
        beg = min(n, c * chunk)
        end = min(n, beg + chunk)
        i0 = beg + 4 * tid
        while True:
            live0 = i0 < end
            if not live0.any():
                break
            for u in range(HIST_UNROLL):
                i = i0 + u * 4 * HIST_THREADS
                pos, own = keys4_positions(i, n, aligned)
                assert pos.min() >= 0 and pos.max() <= n - 1
                for j in range(4):
                    take = live0 & own & (i + j < end)
                    np.add.at(counted, (i + j)[take], 1)
            i0 = i0 + 4 * HIST_THREADS * HIST_UNROLL
        t = keys4_tail(n, aligned) + tid
        tk = (tid < 3) & (t < n) & (t >= beg) & (t < end)
        assert (t[tk] <= n - 1).all()
        np.add.at(counted, t[tk], 1)
        # the chunk's histogram slots
        slot0 = c * BINS
        assert 0 <= slot0 and slot0 + BINS <= C * BINS
    assert (counted == 1).all(), "every element is counted exactly once"
    return C


def model_final(x, k, aligned):
    """topk_final_kernel on one row: returns the output positions written (index -> position)
    after asserting every access is in bounds."""
    n = x.shape[0]
    keys = order_keys(x)
    kk = min(k, n)
    if kk <= 0:
        return {}
    if kk == n:
        return {i: i for i in range(n)}
    hist = np.bincount(keys >> BIN_SHIFT, minlength=BINS)
    csum = np.cumsum(hist[::-1])                       # from the largest bin down
    b = int(np.searchsorted(csum, kk))                 # first top-down prefix reaching kk
    bstar = BINS - 1 - b
    above = int(csum[b - 1]) if b > 0 else 0
    overflow = hist[bstar] > CAND_MAX
    seg = (((n + WAVES_LARGE - 1) // WAVES_LARGE) + 255) // 256 * 256
    lists = []
    if not overflow:
        for w in range(WAVES_LARGE):
            sbeg = min(n, w * seg)
            send = min(n, sbeg + seg)
            taken = []
            nl = 0
            lane = np.arange(WAVE)
            for c0 in range(sbeg, send, 256 * FINAL_UNROLL):
                for u in range(FINAL_UNROLL):
                    i = c0 + 256 * u + 4 * lane
                    pos, own = keys4_positions(i, n, aligned)
                    assert pos.min() >= 0 and pos.max() <= n - 1, "row load out of bounds"
                    kv = keys[pos]
                    tk = own[:, None] & ((i[:, None] + np.arange(4)) < send) & \
                        ((kv >> BIN_SHIFT) >= bstar)
                    tot = int(tk.sum())
                    if tot:
                        if nl + tot <= LIST_PER_WAVE:
                            # lane-major, then j: positions nl .. nl + tot - 1
                            p = nl + np.arange(tot)
                            assert p.max() < LIST_PER_WAVE
                            taken.extend((i[:, None] + np.arange(4))[tk].tolist())
                        else:
                            overflow = True
                        nl += tot
            t = keys4_tail(n, aligned) + lane
            tkt = (lane < 3) & (t < n) & (t >= sbeg) & (t < send)
            if tkt.any():
                assert t[tkt].max() <= n - 1
                kvt = keys[t[tkt]]
                tkt2 = (kvt >> BIN_SHIFT) >= bstar
                tot = int(tkt2.sum())
                if tot:
                    if nl + tot <= LIST_PER_WAVE:
                        taken.extend(t[tkt][tkt2].tolist())
                    else:
                        overflow = True
                    nl += tot
            lists.append(taken)
    if not overflow:
        # the lists hold, per wave and in index order, every key at or above bin b*
        flat = [i for lst in lists for i in lst]
        assert flat == sorted(flat)
        assert set(flat) == set(np.nonzero((keys >> BIN_SHIFT) >= bstar)[0].tolist())
        order = flat
    else:
        order = list(range(n))                          # fallback: the whole row in order
    # threshold and ties as the radix search leaves them: the kk-th largest key, with `need`
    # of the keys equal to it kept (the first ones in index order)
    ks = np.sort(keys)[::-1]
    thr = ks[kk - 1]
    need = kk - int((keys > thr).sum())
    assert 1 <= need
    out = {}
    run_gt = run_eq = 0
    for i in order:
        kv = keys[i]
        if kv > thr:
            p = run_gt + min(run_eq, need)
            run_gt += 1
        elif kv == thr:
            p = run_gt + run_eq if run_eq < need else None
            run_eq += 1
        else:
            continue
        if p is not None:
            assert 0 <= p < kk, "output position out of bounds"
            out[i] = p
    assert above <= kk
    return out


def rows_of(kind, n, rows, seed):
    r = np.random.default_rng(seed)
    if kind == "normal":
        return r.standard_normal((rows, n)).astype(np.float32)
    if kind == "ties":
        return r.integers(-4, 5, size=(rows, n)).astype(np.float32)
    if kind == "allsame":
        return np.full((rows, n), 1.5, np.float32)
    x = r.integers(-2, 3, size=(rows, n)).astype(np.float32)
    x[r.random((rows, n)) < 0.2] = -0.0
    x[r.random((rows, n)) < 0.05] = np.inf
    x[r.random((rows, n)) < 0.05] = -np.inf
    x[r.random((rows, n)) < 0.05] = np.nan
    return x


SHAPES = [
    # rows, n, k values, rows modelled: the GPU tests' wide rows and the two workload shapes
    (300, 16390, (1, 700, 2622), 2),
    (260, 20480, (1, 700, 2622), 2),
    (2, 131072, (1, 700, 2622), 2),
    (3, 70001, (1, 23333, 70000), 1),
    (128, 131072, (2622,), 2),
    (512, 65536, (2048,), 2),
]


@pytest.mark.parametrize("rows,n,ks,nrows", SHAPES)
@pytest.mark.parametrize("aligned", [True, False])
def test_hist_kernel_index_math(rows, n, ks, nrows, aligned):
    C = model_hist(n, rows, aligned)
    assert C * BINS * 4 * rows > 0


@pytest.mark.parametrize("rows,n,ks,nrows", SHAPES)
@pytest.mark.parametrize("kind", ["normal", "ties", "allsame", "special"])
@pytest.mark.parametrize("aligned", [True, False])
def test_final_kernel_index_math(rows, n, ks, nrows, kind, aligned):
    if n >= 65536 and kind != "normal" and not aligned:
        pytest.skip("covered by the aligned case (the unaligned path differs only in the loads)")
    x = rows_of(kind, n, nrows, seed=n + nrows)
    for r in range(nrows):
        for k in ks:
            out = model_final(x[r], k, aligned)
            kk = min(k, n)
            assert sorted(out.values()) == list(range(kk))
            got = np.array(sorted(out, key=out.get), np.int64)
            assert got.tolist() == oracle.topk(x[r], k).tolist()
