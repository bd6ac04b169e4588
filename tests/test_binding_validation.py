"""The binding's extent checks, on the host only.  The C ABI receives bare pointers, so the
Python binding must refuse every tensor whose dtype, shape or row layout does not match what
the kernels will index, before any library call.  Here "device" tensors are meta tensors (no
memory), the host pools are plain CPU tensors, and the library is a recorder: a valid call
reaches the launch, every mis-shaped one raises ValueError and launches nothing."""
import ctypes

import pytest
import torch

import sparse_top_kv_gqa_amd as spk

DEV = "meta"


class FakeLib:
    """Stands in for libspk.so: workspace queries report 0 bytes, every other call is recorded
    and returns SPK_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def fake(monkeypatch):
    f = FakeLib()
    monkeypatch.setattr(spk, "lib", lambda: f)
    monkeypatch.setattr(spk, "_is_dev", lambda t: t.device.type == "meta")
    monkeypatch.setattr(spk, "_is_pinned", lambda t: t.device.type == "cpu")
    monkeypatch.setattr(spk, "_stream", lambda stream=None: ctypes.c_void_p(0))
    return f


def launched(f, name):
    return [c for c in f.calls if c == name]


def d(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=DEV)


# ------------------------------------------------------------------------------ attention

B, T, Hq, Hkv, D, N, K = 2, 1, 8, 2, 128, 300, 40


def attn_args(**over):
    a = dict(q=d(B, T, Hq, D), k=d(B, Hkv, N, D), v=d(B, Hkv, N, D),
             sel_idx=d(B, T, Hkv, K, dtype=torch.int32), sel_count=d(B, T, Hkv, dtype=torch.int32),
             scope="per_kv_head", n_tokens=N)
    a.update(over)
    return a


def test_attention_valid_call_reaches_the_launch(fake):
    spk.sparse_decode_attn(**attn_args())
    assert launched(fake, "sparse_decode_attn") == ["sparse_decode_attn"]


def test_attention_valid_host_pools_and_logits(fake):
    loc = d(B, Hkv, N, dtype=torch.int32)
    kh = torch.empty((B, Hkv, 30, D), dtype=torch.bfloat16)
    lg = d(B, T, Hq, K, dtype=torch.float32)
    spk.sparse_decode_attn(**attn_args(k=d(B, Hkv, 64, D), v=d(B, Hkv, 64, D), k_host=kh,
                                       v_host=kh.clone(), loc=loc, logits=lg))
    # a loc view shared by the KV heads (stride 0) is a valid layout too
    spk.sparse_decode_attn(**attn_args(k_host=kh, v_host=kh.clone(),
                                       loc=d(B, N, dtype=torch.int32).unsqueeze(1).expand(B, Hkv, N)))
    assert len(launched(fake, "sparse_decode_attn")) == 2


BAD_ATTN = {
    "loc shorter than n_tokens": dict(loc=d(B, Hkv, N - 1, dtype=torch.int32),
                                      k_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16),
                                      v_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16)),
    "loc with the wrong KV heads": dict(loc=d(B, 1, N, dtype=torch.int32),
                                        k_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16),
                                        v_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16)),
    "loc with too few sequences": dict(loc=d(B - 1, Hkv, N, dtype=torch.int32),
                                       k_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16),
                                       v_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16)),
    "loc int64": dict(loc=d(B, Hkv, N, dtype=torch.int64),
                      k_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16),
                      v_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16)),
    "loc without host pools": dict(loc=d(B, Hkv, N, dtype=torch.int32)),
    "host pools without loc": dict(k_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16),
                                   v_host=torch.empty((B, Hkv, 8, D), dtype=torch.bfloat16)),
    "host pool with too few sequences": dict(
        loc=d(B, Hkv, N, dtype=torch.int32),
        k_host=torch.empty((B - 1, Hkv, 8, D), dtype=torch.bfloat16),
        v_host=torch.empty((B - 1, Hkv, 8, D), dtype=torch.bfloat16)),
    "host pool in device memory": dict(loc=d(B, Hkv, N, dtype=torch.int32), k_host=d(B, Hkv, 8, D),
                                       v_host=d(B, Hkv, 8, D)),
    "host pool of another dtype": dict(
        loc=d(B, Hkv, N, dtype=torch.int32),
        k_host=torch.empty((B, Hkv, 8, D), dtype=torch.float32),
        v_host=torch.empty((B, Hkv, 8, D), dtype=torch.float32)),
    "sel_idx with too few rows (per_q_head needs B*T*Hq)": dict(scope="per_q_head"),
    "sel_idx int64": dict(sel_idx=d(B, T, Hkv, K, dtype=torch.int64)),
    "sel_idx rows not contiguous": dict(sel_idx=d(B, T, Hkv, 2 * K, dtype=torch.int32)[..., :K]),
    "sel_count too short": dict(sel_count=d(B, T, Hkv - 1, dtype=torch.int32)),
    "sel_count float": dict(sel_count=d(B, T, Hkv, dtype=torch.float32)),
    "k batch smaller than B": dict(k=d(B - 1, Hkv, N, D), v=d(B - 1, Hkv, N, D)),
    "k shorter than n_tokens": dict(k=d(B, Hkv, N - 1, D), v=d(B, Hkv, N - 1, D)),
    "k head dim differs from q": dict(k=d(B, Hkv, N, 64), v=d(B, Hkv, N, 64)),
    "v of another dtype": dict(v=d(B, Hkv, N, D, dtype=torch.float32)),
    "k of an integer dtype": dict(k=d(B, Hkv, N, D, dtype=torch.int16),
                                  v=d(B, Hkv, N, D, dtype=torch.int16)),
    "Hq not a multiple of Hkv": dict(k=d(B, 3, N, D), v=d(B, 3, N, D)),
    "q not contiguous": dict(q=d(B, T, Hq, 2 * D)[..., :D]),
    "q on the host": dict(q=torch.empty((B, T, Hq, D), dtype=torch.bfloat16)),
    "out of the wrong shape": dict(out=d(B, T, Hq, 64, dtype=torch.float32)),
    "out bf16": dict(out=d(B, T, Hq, D)),
    "lse too short": dict(lse=d(B, T, Hq - 1, dtype=torch.float32)),
    "logits rows shorter than the fetch-list bound": dict(logits=d(B, T, Hq, K - 1, dtype=torch.float32)),
    "logits with too few rows": dict(logits=d(B, T, Hq - 1, K, dtype=torch.float32)),
    "workspace of another dtype": dict(ws=d(10 << 20, dtype=torch.float32)),
    "negative n_tokens": dict(n_tokens=-1),
}


@pytest.mark.parametrize("case", sorted(BAD_ATTN))
def test_attention_mis_shaped_inputs_raise_before_any_launch(fake, case):
    with pytest.raises(ValueError):
        spk.sparse_decode_attn(**attn_args(**BAD_ATTN[case]))
    assert launched(fake, "sparse_decode_attn") == []


def test_topk_attention_checks(fake):
    Hq1, nc = 8, 40
    good = dict(scores=d(B, 1, Hkv, nc, dtype=torch.float32), k=6, q=d(B, 1, Hq1, D),
                kc=d(B, Hkv, N, D), vc=d(B, Hkv, N, D), n_tokens=N, gran=4)
    spk.sparse_topk_decode_attn(**good)
    assert len(launched(fake, "sparse_topk_decode_attn")) == 1
    bad = [dict(scores=d(B, 1, Hkv - 1, nc, dtype=torch.float32)),
           dict(scores=d(B, 1, Hkv, nc)),
           dict(kc=d(B, Hkv, N - 1, D), vc=d(B, Hkv, N - 1, D)),
           dict(q=d(B, 2, Hq1, D)),
           dict(sel_idx=d(B, 1, Hkv, 5, dtype=torch.int32), sel_count=d(B, 1, Hkv, dtype=torch.int32)),
           dict(sel_idx=d(B, 1, Hkv, 6, dtype=torch.int32)),
           dict(out=d(B, 1, Hq1, D))]
    for b in bad:
        with pytest.raises(ValueError):
            spk.sparse_topk_decode_attn(**{**good, **b})
    assert len(launched(fake, "sparse_topk_decode_attn")) == 1


# ------------------------------------------------------------------------------ index, top-k

def test_index_score_checks(fake):
    q = d(B, 1, Hq, D)
    spk.sparse_index_score("token_per_head", q, d(B, Hkv, N, D), N)
    spk.sparse_index_score("block_pooled", d(B, 1, Hkv, D), d(B, Hkv, N // 64, D, dtype=torch.float32),
                           N, block_size=64)
    spk.sparse_index_score("block_raw", d(B, 1, Hkv, D), d(B, Hkv, N, D), N, block_size=64,
                           pooled_out=d(B, Hkv, N // 64, D, dtype=torch.float32))
    assert len(launched(fake, "sparse_index_score")) == 3
    bad = [("token_per_head", q, d(B, Hkv, N - 1, D), N, {}),                  # keys too short
           ("token_per_head", q, d(B - 1, Hkv, N, D), N, {}),                  # too few sequences
           ("token_per_head", q, d(B, Hkv, N, 64), N, {}),                     # head dim
           ("token_group_mean", q, d(B, Hkv, N, D), N,
            dict(scores=d(B, 1, Hkv, N - 1, dtype=torch.float32))),             # short score rows
           ("token_per_head", q, d(B, Hkv, N, D), N,
            dict(scores=d(B, 1, Hkv, N, dtype=torch.float32))),                 # Hq rows needed
           ("block_pooled", d(B, 1, Hkv, D), d(B, Hkv, N // 64, D, dtype=torch.float16), N,
            dict(block_size=64)),                                               # pooled keys fp16
           ("block_pooled", d(B, 1, Hkv, D), d(B, Hkv, N // 64 - 1, D, dtype=torch.float32), N,
            dict(block_size=64)),                                               # too few blocks
           ("block_pooled", d(B, 1, Hq, D), d(B, Hkv, N // 64, D, dtype=torch.float32), N,
            dict(block_size=64)),                                               # predictor heads
           ("block_raw", d(B, 1, Hkv, D), d(B, Hkv, N, D), N,
            dict(block_size=64, pooled_out=d(B, Hkv, N // 64 - 1, D, dtype=torch.float32))),
           ("token_per_head", q, d(B, Hkv, N, D), N, dict(pooled_out=d(B, Hkv, 4, D, dtype=torch.float32)))]
    for mode, qq, keys, n, kw in bad:
        with pytest.raises(ValueError):
            spk.sparse_index_score(mode, qq, keys, n, **kw)
    assert len(launched(fake, "sparse_index_score")) == 3


def test_topk_select_checks(fake):
    sc = d(3, 5, 100, dtype=torch.float32)
    spk.topk_select(sc, 7)
    spk.topk_select(d(3, 5, 128, dtype=torch.float32)[..., :100], 7)      # column slice: ld 128
    assert len(launched(fake, "topk_select")) == 2
    bad = [dict(scores=d(3, 5, 100)),                                        # bf16 scores
           dict(scores=sc, idx=d(3, 5, 6, dtype=torch.int32)),                 # idx rows too short
           dict(scores=sc, idx=d(3, 4, 7, dtype=torch.int32)),                 # too few idx rows
           dict(scores=sc, idx=d(3, 5, 14, dtype=torch.int32)[:, :, ::2]),     # strided idx
           dict(scores=sc, count=d(3, 4, dtype=torch.int32)),                  # short count
           dict(scores=sc, n=101),                                             # n past the row
           dict(scores=d(100, 3, dtype=torch.float32).t())]                    # transposed rows
    for b in bad:
        with pytest.raises(ValueError):
            spk.topk_select(k=7, **b)
    assert len(launched(fake, "topk_select")) == 2


def test_window_and_fused_index_checks(fake):
    spk.sparse_window_pool(d(B, Hkv, N, D), N, 32, 16)
    nw = spk.window_count(N, 32, 16)
    spk.sparse_index_score_windowed(d(B, 1, Hkv, D), d(B, Hkv, nw, D, dtype=torch.float32), N, 32,
                                    16, 64)
    spk.sparse_index_topk("block_pooled", d(B, 1, Hkv, D), d(B, Hkv, N // 64, D, dtype=torch.float32),
                          N, 2, block_size=64)
    with pytest.raises(ValueError):
        spk.sparse_window_pool(d(B, Hkv, N - 1, D), N, 32, 16)
    with pytest.raises(ValueError):
        spk.sparse_window_pool(d(B, Hkv, N, D), N, 32, 16, out=d(B, Hkv, nw - 1, D, dtype=torch.float32))
    with pytest.raises(ValueError):
        spk.sparse_index_score_windowed(d(B, 1, Hkv, D), d(B, Hkv, nw - 1, D, dtype=torch.float32),
                                        N, 32, 16, 64)
    with pytest.raises(ValueError):
        spk.sparse_index_topk("block_pooled", d(B, 1, Hkv, D),
                              d(B, Hkv, N // 64, D, dtype=torch.float32), N, 2, block_size=64,
                              idx=d(B, 1, Hkv, 1, dtype=torch.int32))
    assert fake.calls.count("sparse_window_pool") == 1
    assert fake.calls.count("sparse_index_score_windowed") == 1
    assert fake.calls.count("sparse_index_topk") == 1


# ------------------------------------------------------------------------------ importance, tiers

def test_importance_and_tier_checks(fake):
    L, Bs, n, ld = 3, 2, 500, 512
    s = d(Bs, ld, dtype=torch.float32)
    sel = d(Bs, ld, dtype=torch.int32)
    cnt = d(Bs, dtype=torch.int32)
    lg = d(L, Bs, 1, 4, ld, dtype=torch.float32)
    lse = d(L, Bs, 1, 4, dtype=torch.float32)
    spk.importance_accumulate(s, sel, cnt, lg, lse, n)
    spk.tier_classify(s, n, 4, 64)
    spk.tier_classify(s, n, 4, 64, evicted=d(Bs, ld, dtype=torch.uint8), tier=d(Bs, ld, dtype=torch.uint8),
                      sel_idx=sel, sel_count=cnt)
    bad_imp = [dict(s=d(Bs, n - 1, dtype=torch.float32)),
               dict(sel_idx=d(Bs + 1, ld, dtype=torch.int32)),
               dict(sel_count=d(Bs - 1, dtype=torch.int32)),
               dict(logits=d(L, Bs, 1, 4, ld - 1, dtype=torch.float32)),
               dict(logits=d(L, Bs + 1, 1, 4, ld, dtype=torch.float32)),
               dict(lse=d(L, Bs, 1, 3, dtype=torch.float32))]
    base = dict(s=s, sel_idx=sel, sel_count=cnt, logits=lg, lse=lse, n_tokens=n)
    for b in bad_imp:
        with pytest.raises(ValueError):
            spk.importance_accumulate(**{**base, **b})
    bad_tier = [dict(s=d(Bs, n - 1, dtype=torch.float32)),
                dict(evicted=d(Bs, n - 1, dtype=torch.uint8)),
                dict(evicted=d(Bs, n, dtype=torch.bool)),
                dict(tier=d(Bs - 1, n, dtype=torch.uint8)),
                dict(sel_idx=d(Bs, n - 1, dtype=torch.int32)),
                dict(sel_count=d(Bs + 1, dtype=torch.int32))]
    for b in bad_tier:
        with pytest.raises(ValueError):
            spk.tier_classify(**{**dict(s=s, n_tokens=n, n_sink=4, n_recent=64), **b})
    assert fake.calls.count("importance_accumulate") == 1
    assert fake.calls.count("tier_classify") == 2


def test_residency_checks(fake):
    Bs, n, cap = 2, 500, 128
    tier = d(Bs, n, dtype=torch.uint8)
    s = d(Bs, n, dtype=torch.float32)
    loc = d(Bs, n, dtype=torch.int32)
    ct, cs, cc = d(Bs, cap, dtype=torch.int32), d(Bs, cap, dtype=torch.int32), d(Bs, dtype=torch.int32)
    spk.residency_update(tier, s, n, cap, loc, ct, cs, cc)
    for b in [dict(loc=d(Bs, n - 1, dtype=torch.int32)), dict(s=d(Bs, n, dtype=torch.bfloat16)),
              dict(copy_tok=d(Bs, cap - 1, dtype=torch.int32)),
              dict(copy_count=d(Bs + 1, dtype=torch.int32))]:
        a = {**dict(tier=tier, s=s, n_tokens=n, capacity=cap, loc=loc, copy_tok=ct, copy_slot=cs,
                    copy_count=cc), **b}
        with pytest.raises(ValueError):
            spk.residency_update(**a)
    kh = torch.empty((Bs, 2, n, D), dtype=torch.bfloat16)
    kd = d(Bs, 2, cap, D)
    spk.residency_prefetch(kh, kh.clone(), kd, d(Bs, 2, cap, D), ct, cs, cc, cap)
    # device-memory source pools (rows produced on the GPU) are accepted too
    spk.residency_prefetch(d(Bs, 2, n, D), d(Bs, 2, n, D), kd, d(Bs, 2, cap, D), ct, cs, cc, cap)
    for b in [dict(k_host=torch.empty((Bs, 2, n, D), dtype=torch.float32),
                   v_host=torch.empty((Bs, 2, n, D), dtype=torch.float32)),
              dict(k_host=torch.empty((Bs - 1, 2, n, D), dtype=torch.bfloat16),
                   v_host=torch.empty((Bs - 1, 2, n, D), dtype=torch.bfloat16)),
              dict(v_hbm=d(Bs, 2, cap, 64)),
              dict(max_copies=cap + 1)]:
        a = {**dict(k_host=kh, v_host=kh.clone(), k_hbm=kd, v_hbm=d(Bs, 2, cap, D), copy_tok=ct,
                    copy_slot=cs, copy_count=cc, max_copies=cap), **b}
        with pytest.raises(ValueError):
            spk.residency_prefetch(**a)
    assert fake.calls.count("residency_update_tiers") == 1
    assert fake.calls.count("residency_prefetch") == 2
    spk.residency_append(loc, 400, n, cap, ct, cs, cc)
    for b in [dict(n_old=n + 1), dict(loc=d(Bs, n - 1, dtype=torch.int32)),
              dict(copy_tok=d(Bs, 50, dtype=torch.int32), copy_slot=d(Bs, 50, dtype=torch.int32)),
              dict(copy_count=d(Bs + 1, dtype=torch.int32)), dict(capacity=-1)]:
        with pytest.raises(ValueError):
            spk.residency_append(**{**dict(loc=loc, n_old=400, n_new=n, capacity=cap,
                                           copy_tok=ct, copy_slot=cs, copy_count=cc), **b})
    assert fake.calls.count("residency_append") == 1


def test_t2_checks(fake):
    Bs, Hk, n, cap = 2, 2, 500, 128
    src = d(Bs, Hk, n, D)
    codes = d(Bs, Hk, n, D, dtype=torch.int8)
    sc = d(Bs, Hk, n, dtype=torch.float32)
    spk.kv_quantize_int8(src, codes, sc)
    spk.kv_quantize_int8(src, codes, sc, 100, 200)
    for b in [dict(codes=d(Bs, Hk, n - 1, D, dtype=torch.int8)),
              dict(codes=d(Bs, Hk, n, D, dtype=torch.uint8)),
              dict(scales=d(Bs, Hk, n - 1, dtype=torch.float32)),
              dict(row_begin=10, row_end=5), dict(row_end=n + 1),
              dict(src=torch.empty((Bs, Hk, n, D), dtype=torch.bfloat16).transpose(2, 3))]:
        with pytest.raises(ValueError):
            spk.kv_quantize_int8(**{**dict(src=src, codes=codes, scales=sc), **b})
    k, v = d(Bs, Hk, cap + 64, D), d(Bs, Hk, cap + 64, D)
    ct, cs, cc = d(Bs, 64, dtype=torch.int32), d(Bs, 64, dtype=torch.int32), d(Bs, dtype=torch.int32)
    base = dict(codes_k=codes, codes_v=codes.clone(), scale_k=sc, scale_v=sc.clone(), k=k, v=v,
                stage_base=cap, copy_tok=ct, copy_slot=cs, copy_count=cc, max_copies=64)
    spk.t2_fetch(**base)
    for b in [dict(k=d(Bs, Hk, cap + 64, D, dtype=torch.float32)),
              dict(v=d(Bs, Hk, cap + 32, D)), dict(codes_v=d(Bs, Hk + 1, n, D, dtype=torch.int8)),
              dict(scale_k=d(Bs, Hk, n, dtype=torch.bfloat16)), dict(max_copies=65),
              dict(copy_count=d(Bs + 1, dtype=torch.int32)), dict(stage_base=-1)]:
        with pytest.raises(ValueError):
            spk.t2_fetch(**{**base, **b})
    tier, lr = d(Bs, n, dtype=torch.uint8), d(Bs, n, dtype=torch.int32)
    spk.t2_locations(tier, lr, lr.clone(), lr.clone(), n, cap)
    for b in [dict(tier=d(Bs, n, dtype=torch.int32)), dict(loc_t2=d(Bs, n - 1, dtype=torch.int32)),
              dict(loc_out=d(Bs + 1, n, dtype=torch.int32))]:
        with pytest.raises(ValueError):
            spk.t2_locations(**{**dict(tier=tier, loc_res=lr, loc_t2=lr.clone(), loc_out=lr.clone(),
                                       n_tokens=n, stage_base=cap), **b})
    assert fake.calls.count("kv_quantize_int8") == 2
    assert fake.calls.count("t2_fetch") == 1
    assert fake.calls.count("t2_locations") == 1


def test_empty_selection_rows_are_accepted(fake):
    """k = 0: rows of length zero have no meaningful stride and are accepted."""
    spk.sparse_decode_attn(**attn_args(sel_idx=d(B, T, Hkv, 0, dtype=torch.int32)))
    assert launched(fake, "sparse_decode_attn") == ["sparse_decode_attn"]
