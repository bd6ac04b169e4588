"""The allocation-free attention entry point (sparse_decode_attn_noalloc, the library's fixed
scratch array as workspace) against the workspace entry point (sparse_decode_attn) and the
oracle, on two calls in a row, the second with a smaller input."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import steps as osteps
import sparse_top_kv_gqa_amd as spk

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _rand(shape, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).to(DEV)


def _sets(rows, n, k, seed):
    r = np.random.default_rng(seed)
    return np.stack([np.sort(r.choice(n, size=k, replace=False)) for _ in range(rows)]).astype(np.int32)


CASES = [
    # scope, B, Hq, Hkv, N, k, gran, n_sink, n_recent: per-head sets merged by the assembly
    # (fetch list, row masks and partials in the workspace), then a smaller one
    ("per_q_head", 4, 32, 8, 9000, 1500, 1, 0, 0),
    ("per_q_head", 2, 8, 2, 3001, 700, 1, 0, 0),
    # block ids with forced rows (list expanded in the partial kernel)
    ("per_kv_head", 4, 32, 8, 64 * 300 + 7, 24, 64, 4, 512),
    ("per_kv_head", 1, 8, 2, 64 * 50 + 3, 6, 64, 4, 64),
]


def _run(case, seed):
    scope, B, Hq, Hkv, N, k, gran, ns, nr = case
    G = Hq // Hkv
    d = 128
    q = _rand((B, 1, Hq, d), torch.bfloat16, seed)
    kc = _rand((B, Hkv, N, d), torch.bfloat16, seed + 1)
    vc = _rand((B, Hkv, N, d), torch.bfloat16, seed + 2)
    rows = B * Hq if scope == "per_q_head" else B * Hkv
    n_ids = N // gran
    sel = _sets(rows, n_ids, k, seed + 3)
    cnt = np.full(rows, k, np.int32)
    cnt[rows // 2] = k // 3                               # a ragged list
    selt = torch.tensor(sel, device=DEV)
    cntt = torch.tensor(cnt, device=DEV)
    need = spk.attn_workspace_size(scope, B, 1, Hq, Hkv, d, N, k, gran, ns, nr)
    say("noalloc", scope, B, Hq, Hkv, N, k, gran, "workspace", need)
    assert need <= spk.noalloc_max_bytes()
    out_a, lse_a = spk.sparse_decode_attn(q, kc, vc, selt, cntt, scope, N, gran=gran, n_sink=ns,
                                          n_recent=nr)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    spk.sparse_decode_attn_noalloc(q, kc, vc, selt, cntt, scope, N, out=out_b, lse=lse_b,
                                   gran=gran, n_sink=ns, n_recent=nr)
    torch.cuda.synchronize()
    # the same kernels over the same rows: bit for bit the workspace entry point's result
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), case
    # and the oracle's, to the parity bar, on two groups
    qh, kh, vh = host(q), host(kc), host(vc)
    scale = oracle.softmax_scale(d)
    for b, h in [(0, 0), (B - 1, Hkv - 1)]:
        for j in range(G):
            hq = h * G + j
            r = b * Hq + hq if scope == "per_q_head" else b * Hkv + h
            toks = oracle.selection_tokens(sel[r, :cnt[r]], gran, N, ns, nr)
            o_ref, l_ref, _ = oracle.attend(qh[b, 0, hq:hq + 1], kh[b, h][toks], vh[b, h][toks], scale)
            got = out_b[b, 0, hq].cpu().numpy()
            assert osteps.rel_err(got, o_ref[0]) <= osteps.ATTN_REGRESSION_BOUND
            assert osteps.elem_rel_err(got, o_ref[0]) <= osteps.TOL
            assert abs(float(lse_b[b, 0, hq]) - l_ref[0]) <= osteps.TOL * abs(l_ref[0]) + 1e-6


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3)])
def test_noalloc_two_calls_in_a_row_second_smaller(first, second):
    _run(CASES[first], 100 + first)
    _run(CASES[second], 200 + second)


def test_noalloc_refuses_a_workspace_beyond_its_scratch_array():
    """A call needing more than the fixed scratch array is refused before any launch; the
    device stays usable and the next call is correct."""
    B, Hq, Hkv, N, k, d = 64, 32, 8, 1 << 17, 4096, 128
    need = spk.attn_workspace_size("per_q_head", B, 1, Hq, Hkv, d, N, k)
    assert need > spk.noalloc_max_bytes()
    q = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16, device=DEV)
    sel = torch.zeros((B * Hq, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B * Hq,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)
    with pytest.raises(spk.SpkError) as err:
        spk.sparse_decode_attn_noalloc(q, kc, kc, sel, cnt, "per_q_head", N, out=out, lse=lse)
    assert err.value.status == 3 and "scratch" in str(err.value)
    del kc
    torch.cuda.synchronize()
    _run(CASES[1], 300)
