"""Host-side bookkeeping of bench.py: the fetch lists the gather reference reads must be exactly
the rows the block attention reads (sinks, recent window and the selected blocks, each once);
the union sizes read only counted entries; a request for more than one GPU is refused."""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _expected(blocks, n_tokens, bs, n_sink, n_recent):
    rows = set(range(min(n_sink, n_tokens))) | set(range(max(n_tokens - n_recent, 0), n_tokens))
    for e in blocks:
        rows |= set(t for t in range(e * bs, e * bs + bs) if t < n_tokens)
    return rows


def test_block_fetch_lists_match_the_attended_rows():
    gen = torch.Generator().manual_seed(11)
    for (B, H, k, bs, N, ns, nr) in [(2, 3, 5, 64, 2048, 4, 512), (1, 2, 7, 16, 1000, 0, 37),
                                     (3, 1, 4, 64, 300, 8, 0), (1, 1, 3, 64, 256, 300, 300)]:
        nb = N // bs
        idx = torch.stack([torch.stack([torch.sort(torch.randperm(nb, generator=gen)[:k]).values
                                        for _ in range(H)]) for _ in range(B)]).unsqueeze(1).int()
        cnt = torch.randint(0, k + 1, (B, 1, H), generator=gen, dtype=torch.int32)
        lists = bench.block_fetch_lists(idx, cnt, N, bs, ns, nr)
        assert lists.dtype == torch.int32 and lists.shape[0] == B * H
        for g in range(B * H):
            b, h = g // H, g % H
            row = lists[g]
            live = row[row >= 0].tolist()
            assert len(live) == len(set(live)), "a row listed twice"
            assert set(live) == _expected(idx[b, 0, h, :int(cnt[b, 0, h])].tolist(), N, bs, ns, nr)
            assert all(0 <= t < N for t in live)
        total = int((lists >= 0).sum())
        full = torch.full_like(cnt, k)
        if bool((cnt == full).all()):
            assert total == bench.union_rows_block(idx, N, bs, ns, nr)


def test_union_rows_read_only_counted_entries_in_range():
    """union_rows_tokens counts each group's distinct rows over the first count entries of its
    selection rows only: entries past a row's count (never written by a selection call) and
    values outside [0, N) count for nothing, so uninitialised index memory cannot send the
    scatter out of bounds."""
    gen = torch.Generator().manual_seed(5)
    B, T, Hs, k, N, G = 2, 1, 8, 6, 40, 4
    idx = torch.randint(0, N, (B, T, Hs, k), generator=gen, dtype=torch.int32)
    cnt = torch.randint(0, k + 1, (B, T, Hs), generator=gen, dtype=torch.int32)
    garbage = idx.clone()
    live = torch.arange(k) < cnt.unsqueeze(-1)
    garbage[~live] = torch.randint(-(1 << 30), 1 << 30, (int((~live).sum()),), generator=gen,
                                   dtype=torch.int32)
    got = bench.union_rows_tokens(garbage, cnt, G, N).tolist()
    want = []
    for b in range(B):
        for h in range(Hs // G):
            rows = set()
            for j in range(h * G, (h + 1) * G):
                rows |= set(idx[b, 0, j, :int(cnt[b, 0, j])].tolist())
            want.append(len(rows))
    assert got == want
    # out-of-range values inside the counted part count for nothing either
    bad = idx.clone()
    bad[..., 0] = N + 3
    full = torch.full((B, T, Hs), k, dtype=torch.int32)
    got = bench.union_rows_tokens(bad, full, G, N).tolist()
    want = [len(set(bad[b, 0, h * G:(h + 1) * G, 1:].reshape(-1).tolist()))
            for b in range(B) for h in range(Hs // G)]
    assert got == want


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py --gpus N with N > 1 exits with status 2 and says why, before touching a GPU."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
