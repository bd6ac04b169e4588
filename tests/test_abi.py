"""The C-ABI library loads, exports every entry point include/spk.h declares, and rejects bad
arguments before launching anything.  CPU only: no call here reaches a kernel."""
import ctypes
import os
import re

import pytest

import sparse_top_kv_gqa_amd as spk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spk.h")

# Fake, 16-byte-aligned device addresses: validation must fail before anything touches them.
A = ctypes.c_void_p(0x100000)
Bp = ctypes.c_void_p(0x200000)


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"SPK_API\s+[\w\s\*]+?\b(\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert set(names) == set(spk.EXPORTS), names
    L = spk.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.spk_version() == 1


def _err():
    return spk.lib().spk_last_error().decode()


def test_index_score_validation():
    L = spk.lib()
    # null q
    assert L.sparse_index_score(0, None, 1, A, 1, 128 * 64, 128 * 64, 128, 1, 1, 4, 1, 128, 64, 1,
                                Bp, 64, None, None) == 1
    assert "null" in _err()
    # Hq % Hkv != 0
    assert L.sparse_index_score(0, A, 1, A, 1, 128 * 64, 128 * 64, 128, 1, 1, 6, 4, 128, 64, 1,
                                Bp, 64, None, None) == 1
    # unsupported d
    assert L.sparse_index_score(0, A, 1, A, 1, 96 * 64, 96 * 64, 96, 1, 1, 4, 1, 96, 64, 1,
                                Bp, 64, None, None) == 2
    # unsupported dtype
    assert L.sparse_index_score(0, A, 7, A, 1, 128 * 64, 128 * 64, 128, 1, 1, 4, 1, 128, 64, 1,
                                Bp, 64, None, None) == 2
    # score leading dim too small
    assert L.sparse_index_score(0, A, 1, A, 1, 128 * 64, 128 * 64, 128, 1, 1, 4, 1, 128, 64, 1,
                                Bp, 63, None, None) == 1
    # pooled_out outside BLOCK_RAW
    assert L.sparse_index_score(2, A, 1, A, 0, 128 * 64, 128 * 64, 128, 1, 1, 1, 1, 128, 64, 16,
                                Bp, 64, Bp, None) == 1
    # too many score vectors per KV head (per head, T*G = 32)
    assert L.sparse_index_score(1, A, 1, A, 1, 128 * 64, 128 * 64, 128, 1, 8, 4, 1, 128, 64, 1,
                                Bp, 64, None, None) == 2


def test_topk_validation():
    L = spk.lib()
    assert L.topk_select(A, 100, 4, 100, -1, Bp, 10, None, None, 0, None) == 1
    assert L.topk_select(A, 100, 4, 100, 10, Bp, 9, None, None, 0, None) == 1      # idx_ld < k
    assert L.topk_select(A, 50, 4, 100, 10, Bp, 10, None, None, 0, None) == 1      # s_ld < n
    assert L.topk_select(None, 100, 4, 100, 10, Bp, 10, None, None, 0, None) == 1
    sz = ctypes.c_size_t(123)
    assert L.topk_select_workspace_size(4, 100, 10, ctypes.byref(sz)) == 0 and sz.value == 0
    # wide rows keep per-chunk histograms in the workspace
    assert L.topk_select_workspace_size(128, 131072, 2622, ctypes.byref(sz)) == 0 and sz.value > 0
    assert L.topk_select(A, 131072, 128, 131072, 2622, Bp, 2622, None, None, 0, None) == 3


def _attn(**kw):
    args = dict(q=A, q_dt=1, k=A, v=A, kv_dt=1, kv_sb=8 * 1024 * 128, kv_sh=1024 * 128, kv_sn=128,
                k_host=None, v_host=None, host_sb=0, host_sh=0, host_sn=0, host_slots=0, loc=None,
                loc_sb=0, loc_sh=0, hbm_slots=1024, sel_idx=Bp, sel_count=Bp, sel_ld=32, scope=1, gran=1, n_sink=0,
                n_recent=0, B=2, T=1, Hq=32, Hkv=8, d=128, n=1024, scale=0.1, out=Bp, lse=None,
                logits=None, logits_ld=0, ws=Bp, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return spk.lib().sparse_decode_attn(*args.values())


def test_attn_validation():
    assert _attn(Hq=30) == 1 and "Hq" in _err()
    assert _attn(d=80, kv_sn=80) == 2
    assert _attn(q=None) == 1
    assert _attn(loc=Bp) == 1 and "host" in _err()                 # loc without host pools
    assert _attn(ws_bytes=16) == 3                                   # workspace too small
    assert _attn(scope=9) == 1
    assert _attn(kv_sn=100) == 1                                     # stride not a multiple of 8
    assert _attn(q=ctypes.c_void_p(0x100004)) == 1                   # misaligned
    assert _attn(T=4, Hq=32, Hkv=4) == 2                             # 32 query vectors per group
    assert _attn(logits=Bp, logits_ld=8) == 1                        # logits_ld below the bound
    assert _attn(gran=0) == 1
    assert _attn(hbm_slots=1000) == 1 and "exceeds" in _err()       # cache shorter than n_tokens
    # 4 lists x 2^25 entries x granularity 2^7: more flattened rows than the assembly numbers
    assert _attn(scope=2, sel_ld=1 << 25, gran=1 << 7) == 2 and "2^31" in _err()
    # host pools must be pinned host memory known to HIP: a plain malloc'ed buffer is refused
    buf = ctypes.create_string_buffer(1 << 16)
    addr = (ctypes.addressof(buf) + 15) // 16 * 16
    assert _attn(loc=Bp, k_host=ctypes.c_void_p(addr), v_host=ctypes.c_void_p(addr), host_sb=128,
                 host_sh=128, host_sn=128, host_slots=4) == 1


def test_attn_workspace_query():
    n = spk.attn_workspace_size("per_kv_head", 8, 1, 32, 8, 128, 32768, 32, 64, 4, 512)
    assert n > 8 * 8 * 4 * 128 * 4          # at least one split of partial outputs per group
    assert spk.fetch_list_bound("per_kv_head", 1, 4, 32, 64, 4, 512, 32768) == 2564
    assert spk.fetch_list_bound("per_q_head", 1, 4, 2622, 1, 0, 0, 131072) == 10488


def test_importance_and_tier_validation():
    L = spk.lib()
    assert L.importance_accumulate(A, 100, 2, 100, Bp, Bp, 50, A, 50, A, 0, 4, None) == 1
    assert L.importance_accumulate(A, 100, 2, 100, Bp, Bp, 50, A, 50, A, 100, 100, None) == 2
    assert L.importance_accumulate(A, 100, 2, 100, Bp, Bp, 50, A, 40, A, 2, 4, None) == 1
    # t0 > t01; t01 > t012; t012 > 1000
    assert L.tier_classify(A, 100, 2, 100, 4, 8, 800, 700, 700, None, 0, Bp, 100, None, None, 0,
                           None, 0, None) == 1
    assert L.tier_classify(A, 100, 2, 100, 4, 8, 250, 750, 700, None, 0, Bp, 100, None, None, 0,
                           None, 0, None) == 1
    assert "t012_permille" in _err()
    assert L.tier_classify(A, 100, 2, 100, 4, 8, 250, 750, 1001, None, 0, Bp, 100, None, None, 0,
                           None, 0, None) == 1
    # sel_ld < n_tokens
    assert L.tier_classify(A, 100, 2, 100, 4, 8, 250, 750, 950, None, 0, Bp, 100, Bp, Bp, 50,
                           None, 0, None) == 1
    # sel_idx without sel_count
    assert L.tier_classify(A, 100, 2, 100, 4, 8, 250, 750, 750, None, 0, Bp, 100, Bp, None, 100,
                           None, 0, None) == 1


def test_residency_append_validation():
    L = spk.lib()
    # n_new < n_old; capacity above the limit; loc_ld < n_new; copy_ld too short
    assert L.residency_append(A, 100, 1, 50, 40, 16, A, A, 16, A, None) == 1
    assert L.residency_append(A, 100, 1, 50, 60, 131073, A, A, 16, A, None) == 2
    assert L.residency_append(A, 50, 1, 40, 60, 16, A, A, 16, A, None) == 1
    assert "loc_ld" in _err()
    assert L.residency_append(A, 100, 1, 40, 60, 16, A, A, 15, A, None) == 1
    assert "copy_ld" in _err()
    assert L.residency_append(A, 100, 0, 40, 60, 16, A, A, 16, A, None) == 0


def test_t2_validation():
    L = spk.lib()
    # residency classes outside a byte
    assert L.residency_update_tiers(A, 64, A, 64, 1, 64, 16, 0x100, A, 64, A, A, 16, A,
                                    None) == 1
    assert "tier_classes" in _err()
    # quantize: d = 96; row range reversed; src not memory HIP knows (host, not pinned)
    assert L.kv_quantize_int8(A, 1, 128, 128, 128, 1, 1, 96, 0, 8, A, 128, 128, 128, A, 8, 8,
                              None) == 2
    assert L.kv_quantize_int8(A, 1, 128, 128, 128, 1, 1, 128, 8, 4, A, 128, 128, 128, A, 8, 8,
                              None) == 1
    assert L.kv_quantize_int8(A, 1, 128, 128, 130, 1, 1, 128, 0, 8, A, 128, 128, 128, A, 8, 8,
                              None) == 1
    # nothing to do: no rows
    assert L.kv_quantize_int8(A, 1, 128, 128, 128, 1, 1, 128, 8, 8, A, 128, 128, 128, A, 8, 8,
                              None) == 0
    # fetch: fp32 pools; d = 96; negative stage_base
    assert L.t2_fetch(A, A, 128, 128, 128, A, A, 8, 8, 8, Bp, Bp, 0, 128, 128, 128, 8, 0, 1, 1,
                      128, A, A, 8, A, 8, None) == 2
    assert L.t2_fetch(A, A, 128, 128, 128, A, A, 8, 8, 8, Bp, Bp, 1, 128, 128, 128, 8, 0, 1, 1,
                      96, A, A, 8, A, 8, None) == 2
    assert L.t2_fetch(A, A, 128, 128, 128, A, A, 8, 8, 8, Bp, Bp, 1, 128, 128, 128, 8, -1, 1, 1,
                      128, A, A, 8, A, 8, None) == 1
    # locations: row stride below n_tokens; stage rows beyond int32
    assert L.t2_locations(A, 50, A, 100, A, 100, A, 100, 1, 100, 0, None) == 1
    assert L.t2_locations(A, 100, A, 100, A, 100, A, 100, 1, 100, 2 ** 31 - 50, None) == 1


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(spk, "_lib", None)
    monkeypatch.setattr(spk, "LIB_PATH", "/nonexistent/libspk.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        spk.lib()


def test_timing_hook_validation():
    L = spk.lib()
    assert L.spk_set_attn_timing_events(ctypes.c_void_p(1), None) == 1
    assert "both" in L.spk_last_error().decode()
    assert L.spk_set_attn_timing_events(None, None) == 0


def test_stream_read_host_validation():
    """The host streaming read refuses bad arguments before touching HIP: null buffer or sink,
    unaligned pointer or size, workgroups out of range; zero bytes is a no-op."""
    L = spk.lib()
    assert L.spk_stream_read_host(None, 1024, 8, A, None) == 1
    assert "null" in _err()
    assert L.spk_stream_read_host(A, 1024, 8, None, None) == 1
    assert L.spk_stream_read_host(ctypes.c_void_p(0x100004), 1024, 8, A, None) == 1
    assert L.spk_stream_read_host(A, 1000, 8, A, None) == 1
    assert L.spk_stream_read_host(A, 1024, 0, A, None) == 1
    assert L.spk_stream_read_host(A, 1024, (1 << 20) + 1, A, None) == 1
    assert "workgroups" in _err()
    assert L.spk_stream_read_host(A, 0, 8, A, None) == 0      # nothing to read: no query, no launch


def test_stream_read_validation():
    L = spk.lib()
    assert L.spk_stream_read(None, 1024, 8, A, None) == 1
    assert "null" in _err()
    assert L.spk_stream_read(A, 1024, 8, None, None) == 1
    assert L.spk_stream_read(ctypes.c_void_p(0x100004), 1024, 8, A, None) == 1
    assert "16" in _err()
    assert L.spk_stream_read(A, 1000, 8, A, None) == 1
    assert L.spk_stream_read(A, 1024, 0, A, None) == 1
    assert L.spk_stream_read(A, 1024, (1 << 20) + 1, A, None) == 1
    assert "workgroups" in _err()
    assert L.spk_stream_read(A, 0, 8, A, None) == 0      # nothing to read: no launch


def test_gather_read_validation():
    L = spk.lib()
    P = ctypes.c_void_p
    ok = dict(k=A, v=A, rb=256, sg=1 << 20, sn=256, n=4096, rows=A, ld=64, groups=8, wpg=4)

    def call(**kw):
        a = dict(ok, **kw)
        return L.spk_gather_read(a["k"], a["v"], a["rb"], a["sg"], a["sn"], a["n"], a["rows"],
                                 a["ld"], a["groups"], a["wpg"], A, None)
    assert call(k=None) == 1 and "null" in _err()
    assert call(rows=None) == 1
    assert call(rows=None, ld=0) == 0                   # no list, nothing to read
    for rb in (0, 16, 48, 96, 2048):
        assert call(rb=rb) == 1 and "row_bytes" in _err()
    assert call(v=P(0x100008)) == 1 and "16" in _err()
    assert call(sn=264) == 1 and call(sg=(1 << 20) + 8) == 1
    assert call(sn=128) == 1 and "strides" in _err()    # rows overlap
    assert call(n=-1) == 1 and call(ld=1 << 31) == 1 and call(groups=65536) == 1
    assert call(wpg=0) == 1 and "wg_per_group" in _err()
    assert call(wpg=65536) == 1
    assert call(groups=0) == 0 and call(ld=0) == 0 and call(n=0) == 0   # nothing to launch


def test_index_topk_validation():
    L = spk.lib()
    P = ctypes.c_void_p
    q = P(16)
    keys = P(32)
    idx = P(48)
    # BLOCK_RAW is not fused
    st = L.sparse_index_topk(3, q, 0, keys, 0, 64 * 128, 128, 128, 1, 1, 4, 1, 128, 4096, 64, 8,
                             None, 0, idx, 8, None, None)
    assert st == 2 and "BLOCK_RAW" in L.spk_last_error().decode()
    # too many candidates per row
    st = L.sparse_index_topk(0, q, 0, keys, 0, 1 << 24, 1 << 22, 128, 1, 1, 4, 1, 128, 9000, 1,
                             8, None, 0, idx, 8, None, None)
    assert st == 2
    # too many score vectors (per-head with G = 8)
    st = L.sparse_index_topk(1, q, 0, keys, 0, 1 << 20, 1 << 18, 128, 1, 1, 8, 1, 128, 1000, 1,
                             8, None, 0, idx, 8, None, None)
    assert st == 2
    # idx_ld smaller than min(k, candidates)
    st = L.sparse_index_topk(0, q, 0, keys, 0, 1 << 20, 1 << 18, 128, 1, 1, 4, 1, 128, 1000, 1,
                             8, None, 0, idx, 4, None, None)
    assert st == 1
    # null idx with k > 0
    st = L.sparse_index_topk(0, q, 0, keys, 0, 1 << 20, 1 << 18, 128, 1, 1, 4, 1, 128, 1000, 1,
                             8, None, 0, None, 8, None, None)
    assert st == 1
    assert spk.fused_index_topk_ok("block_pooled", 1, 4, 512)
    assert not spk.fused_index_topk_ok("token_per_head", 1, 8, 512)
    assert not spk.fused_index_topk_ok("token_group_mean", 1, 4, 131072)


def test_window_entries_validation():
    L = spk.lib()
    # sparse_window_pool: null keys; d = 96; w_cap smaller than the window count; stride 0
    assert L.sparse_window_pool(None, 1, 128 * 64, 128 * 64, 128, 1, 1, 128, 64, 32, 16, Bp, 3,
                                None) == 1
    assert L.sparse_window_pool(A, 1, 96 * 64, 96 * 64, 96, 1, 1, 96, 64, 32, 16, Bp, 3, None) == 2
    assert L.sparse_window_pool(A, 1, 128 * 64, 128 * 64, 128, 1, 1, 128, 64, 32, 16, Bp, 2,
                                None) == 1
    assert "w_cap" in _err()
    assert L.sparse_window_pool(A, 1, 128 * 64, 128 * 64, 128, 1, 1, 128, 64, 32, 0, Bp, 3,
                                None) == 1
    # sparse_index_score_windowed: T = 17; s_ld < blocks; a block over too many windows
    assert L.sparse_index_score_windowed(A, 1, Bp, 3, 1, 17, 1, 128, 64, 32, 16, 64, A, 1,
                                         None) == 1
    assert L.sparse_index_score_windowed(A, 1, Bp, 3, 1, 1, 1, 128, 128, 32, 16, 64, A, 2,
                                         None) == 1
    assert "w_cap" in _err()
    assert L.sparse_index_score_windowed(A, 1, Bp, 7, 1, 1, 1, 128, 128, 32, 16, 64, A, 1,
                                         None) == 1
    assert "s_ld" in _err()
    assert L.sparse_index_score_windowed(A, 1, Bp, 1 << 20, 1, 1, 1, 128, 1 << 16, 32, 1, 4096, A,
                                         64, None) == 2
    assert spk.window_count(64, 32, 16) == 3 and spk.window_count(31, 32, 16) == 0


def test_residency_validation():
    L = spk.lib()
    # residency_update: capacity above the limit; loc_ld < n_tokens; null loc
    assert L.residency_update(A, 200000, A, 200000, 1, 200000, 131073, A, 200000, A, A, 100, A,
                              None) == 2
    assert "131072" in _err()
    assert L.residency_update(A, 64, A, 64, 1, 64, 16, A, 32, A, A, 16, A, None) == 1
    assert "loc_ld" in _err()
    assert L.residency_update(A, 64, A, 64, 1, 64, 16, None, 64, A, A, 16, A, None) == 1
    # residency_prefetch: d = 96; strides not keeping 16-byte rows; pageable host pool
    assert L.residency_prefetch(A, A, 128, 128, 128, 8, Bp, Bp, 128, 128, 128, 8, 1, 1, 1, 96, A,
                                A, 8, A, 8, None) == 2
    assert L.residency_prefetch(A, A, 128, 128, 130, 8, Bp, Bp, 128, 128, 128, 8, 1, 1, 1, 128, A,
                                A, 8, A, 8, None) == 1
    host = ctypes.create_string_buffer(1 << 16)     # ordinary (pageable) memory
    hp = ctypes.c_void_p(ctypes.addressof(host))
    st = L.residency_prefetch(hp, hp, 128, 128, 128, 8, Bp, Bp, 128, 128, 128, 8, 1, 1, 1, 128, A,
                              A, 8, A, 8, None)
    assert st in (1, 4) and "k_host" in _err()


def _attn_noalloc(**kw):
    args = dict(q=A, q_dt=1, k=A, v=A, kv_dt=1, kv_sb=8 * 1024 * 128, kv_sh=1024 * 128, kv_sn=128,
                k_host=None, v_host=None, host_sb=0, host_sh=0, host_sn=0, host_slots=0, loc=None,
                loc_sb=0, loc_sh=0, hbm_slots=1024, sel_idx=Bp, sel_count=Bp, sel_ld=32, scope=1,
                gran=1, n_sink=0, n_recent=0, B=2, T=1, Hq=32, Hkv=8, d=128, n=1024, scale=0.1,
                out=Bp, lse=None, logits=None, logits_ld=0, stream=None)
    args.update(kw)
    return spk.lib().sparse_decode_attn_noalloc(*args.values())


def test_attn_noalloc_validation_and_size_limit():
    """The allocation-free variant validates like sparse_decode_attn and refuses, before any
    launch and with a clear error, a call whose workspace exceeds its fixed scratch array."""
    cap = spk.lib().sparse_decode_attn_noalloc_max_bytes()
    assert cap == 32 << 20
    assert _attn_noalloc(Hq=30) == 1 and "Hq" in _err()
    assert _attn_noalloc(q=None) == 1
    assert _attn_noalloc(loc=Bp) == 1 and "host" in _err()
    assert _attn_noalloc(d=80, kv_sn=80) == 2
    # 256 sequences x 8 KV heads x 4 lists of 4096 ids over 1M tokens: far beyond 32 MiB
    need = spk.attn_workspace_size("per_q_head", 256, 1, 32, 8, 128, 1 << 20, 4096)
    assert need > cap
    assert _attn_noalloc(B=256, scope=2, sel_ld=4096, n=1 << 20, hbm_slots=1 << 20,
                         kv_sb=8 * (1 << 20) * 128, kv_sh=(1 << 20) * 128) == 3
    assert "scratch" in _err() and str(need) in _err()
