"""A CPU model of the index arithmetic and key comparisons of the union top-k kernels
(csrc/topk_union.hip: union_range_kernel, union_gather_kernel, union_thr_kernel,
union_write_kernel), run on the host only.

The model forms what the kernels form — each sampled token of the range estimate, the segment
layout of the workspace (segment length, segment count, candidate slots packed with a token
offset into one 32-bit list entry), the sample ranks of the range's two ends — and asserts that
every index stays inside its buffer and every packed field inside its bits, for row lengths from
1 to the entry point's 2^22 and for the group counts of the GPU tests and workloads.  It also
checks the gather's float comparisons against the order-key comparisons they stand for, over
ordinary, tied and special values (signed zeros, infinities, NaN), with the range ends the
range kernel can produce.  The constants below are the kernels' own."""
import numpy as np
import pytest

MAX_SEG_LEN, MAX_SEGS = 1024, 4096
PIECES, PIECE_LEN = 256, 16
SAMPLE_MAX = PIECES * PIECE_LEN
SLOT_BITS = 22
CUS = 256


def sample_tokens(n):
    """union_range_kernel's sample_token(i, n) for i < min(n, 4096)."""
    m = min(n, SAMPLE_MAX)
    i = np.arange(m, dtype=np.int64)
    if n <= SAMPLE_MAX:
        return i
    return (i // PIECE_LEN) * n // PIECES + i % PIECE_LEN


def layout(groups, n):
    """make_layout's segment length, part count and segment count."""
    seg = MAX_SEG_LEN
    want = 2 * CUS
    ceil = lambda a, b: -(-a // b)
    while seg > 256 and groups * ceil(n, 4 * seg) < want:
        seg //= 2
    parts = ceil(max(n, 1), 4 * seg)
    return seg, parts, 4 * parts


def ranks(n, kk):
    """The sample ranks of hi and lo (None: no key above / every key in range)."""
    m = min(n, SAMPLE_MAX)
    if n <= SAMPLE_MAX:
        return kk, kk
    r = np.float32(kk) * np.float32(m) / np.float32(n)
    delta = np.float32(4.0) * np.sqrt(r, dtype=np.float32) + np.float32(2.0)
    qh, ql = int(np.floor(r - delta)), int(np.ceil(r + delta))
    return (qh if qh >= 1 else None), (ql if ql <= m else None)


def order_key(x):
    x = np.asarray(x, np.float32)
    u = x.copy().view(np.uint32)
    u[u == 0x80000000] = 0
    k = np.where((u & 0x80000000) != 0, ~u, u | 0x80000000).astype(np.uint32)
    k[np.isnan(x)] = 0
    return k


def key_float(k):
    k = np.asarray(k, np.uint32)
    u = np.where((k & 0x80000000) != 0, k & 0x7FFFFFFF, ~k).astype(np.uint32)
    return u.view(np.float32)


@pytest.mark.parametrize("n", [1, 2, 15, 100, 4095, 4096, 4097, 4111, 8191, 16385, 20000, 65536,
                               70001, 131072, 1 << 20, (1 << 22) - 3, 1 << 22])
def test_sample_tokens_in_row_and_distinct(n):
    t = sample_tokens(n)
    assert t.shape[0] == min(n, SAMPLE_MAX)
    assert t.min() >= 0 and t.max() < n
    assert np.all(np.diff(t) > 0)          # distinct and ascending: pieces never overlap


@pytest.mark.parametrize("groups", [1, 2, 4, 8, 32, 64, 128, 1024])
@pytest.mark.parametrize("n", [0, 1, 100, 1023, 1024, 1025, 4097, 16385, 20000, 65536, 70001,
                               131072, 1 << 21, 1 << 22])
def test_layout_slots_fit_their_fields(groups, n):
    seg, parts, nseg = layout(groups, n)
    assert seg in (256, 512, 1024) and seg <= MAX_SEG_LEN
    assert nseg <= MAX_SEGS                  # the threshold pass's LDS prefix holds nseg + 1
    assert nseg * seg >= n                   # the segments cover the row
    # a candidate slot (segment * seg + position < seg) packs below the token offset bits
    assert nseg * seg <= 1 << SLOT_BITS
    assert seg - 1 < 1 << (32 - SLOT_BITS)
    # the gather's grid: parts workgroups of 4 waves, one segment each, none left over
    assert parts * 4 == nseg


@pytest.mark.parametrize("n", [1, 100, 4096, 4097, 16385, 20000, 65536, 70001, 131072, 1 << 22])
def test_sample_ranks_inside_the_sample(n):
    m = min(n, SAMPLE_MAX)
    for kk in sorted({1, 2, 5, 32, 700, 2048, 2622, n // 3, n - 1, n}):
        if kk < 1 or kk > n:
            continue
        qh, ql = ranks(n, kk)
        assert qh is None or 1 <= qh <= m
        assert ql is None or 1 <= ql <= m
        if qh is not None and ql is not None:
            assert qh <= ql                  # lo <= hi: the range is never empty by rank
        if n <= SAMPLE_MAX:
            assert qh == ql == kk            # the whole row: the range is exact


def radix_threshold(keys, kk):
    """select_common.h's radix_threshold on uint32 keys: 8-bit digits from the top; stops
    ("whole") as soon as the chosen digit's bin holds exactly the keys still missing, and then
    returns a prefix that exactly the kk largest keys reach, else the kk-th largest key."""
    keys = np.asarray(keys, np.uint32)
    prefix, pmask, rem = 0, 0, kk
    for p in range(4):
        shift = 24 - 8 * p
        cand = keys[(keys & np.uint32(pmask)) == prefix]
        h = np.bincount((cand >> np.uint32(shift)) & np.uint32(255), minlength=256)
        incl = np.cumsum(h[::-1])                   # counts from digit 255 down
        j = int(np.argmax(incl >= rem))
        dsel = 255 - j
        above = int(incl[j] - h[dsel])
        rem -= above
        prefix |= dsel << shift
        pmask |= 0xFF << shift
        if h[dsel] == rem:
            return prefix, True
    return prefix, False


def range_end(sample_keys, q):
    """union_range_kernel's end of rank q: the bin of the q-th largest key by a 4096-bin
    histogram of the top 12 bits, the radix search over that bin's low 20 bits, and, when the
    search stopped on a prefix, the smallest sample key that reaches it."""
    k = np.asarray(sample_keys, np.uint32)
    bins = np.bincount(k >> np.uint32(20), minlength=4096)
    incl = np.cumsum(bins[::-1])
    j = int(np.argmax(incl >= q))
    bq = 4095 - j
    qin = q - int(incl[j] - bins[bq])
    inbin = k[(k >> np.uint32(20)) == bq]
    low, whole = radix_threshold((inbin << np.uint32(12)) & np.uint32(0xFFFFFFFF), qin)
    thr = (bq << 20) | (low >> 12)
    if whole:
        thr = int(k[k >= thr].min())
    return thr


def _values(kind, rng, size):
    if kind == "normal":
        return rng.standard_normal(size).astype(np.float32)
    if kind == "ties":
        return rng.integers(-3, 4, size).astype(np.float32)
    x = rng.integers(-2, 3, size).astype(np.float32)
    x[rng.random(size) < 0.2] = -0.0
    x[rng.random(size) < 0.05] = np.inf
    x[rng.random(size) < 0.05] = -np.inf
    x[rng.random(size) < 0.05] = np.nan
    return x


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
@pytest.mark.parametrize("m", [1, 2, 7, 300, 4096])
def test_range_ends_are_sample_keys(kind, m):
    """Every end the range kernel writes is the key of a sample score (a radix search that
    stops on a prefix is snapped to the smallest key reaching it), and it has the rank asked
    for: at least q sample keys are >= it, fewer than q are > it."""
    rng = np.random.default_rng(m)
    for trial in range(20):
        keys = order_key(_values(kind, rng, m))
        for q in sorted({1, 2, m // 3, m // 2, m - 1, m}):
            if q < 1 or q > m:              # the kernel asks for ranks 1 .. m only
                continue
            e = range_end(keys, q)
            assert e in set(keys.tolist()), (kind, m, q, hex(e))
            assert int((keys >= e).sum()) >= q > int((keys > e).sum())


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
def test_gather_float_compares_match_key_compares(kind):
    """union_gather_kernel classifies a score x against [lo, hi] as floats: above = x > f(hi),
    in range = not above and (lo == 0 or x >= f(lo)), f = key_float.  That equals the key
    classification key(x) > hi and lo <= key(x) <= hi for every range end the range kernel
    can produce — a key of a sample score (range_end, the kernel's own computation; order_key
    never yields the key of -0 or of a NaN other than 0), the sentinel 0xFFFFFFFF for hi and 0
    for lo — except hi = 0, NaN's key (a sample
    that is mostly NaN): then lo is 0 too and the float form puts every token in range and
    none above.  That is still a valid split for the threshold pass (nothing above, everything
    listed, so its whole-row fallback or its radix over the lists finds the exact top-k); it is
    asserted here as such."""
    rng = np.random.default_rng(7)
    x = _values(kind, rng, 4000)
    sample = order_key(np.concatenate([_values(kind, rng, 200), x[:200]]))
    made = [range_end(sample, q) for q in range(1, sample.shape[0] + 1, 3)]
    ends = np.unique(np.concatenate([np.array(made, np.uint32),
                                     np.array([0, 0xFFFFFFFF], np.uint32)]))
    kx = order_key(x)
    with np.errstate(invalid="ignore"):
        for hi in ends:
            for lo in ends[::7]:
                if lo > hi:
                    continue
                above_k = kx > hi
                inr_k = (kx >= lo) & (kx <= hi)
                above_f = x > key_float(hi)
                inr_f = ~above_f & ((lo == 0) | (x >= key_float(lo)))
                if hi == 0:
                    assert not above_f.any() and inr_f.all()
                    continue
                assert np.array_equal(above_k, above_f), (kind, hex(hi))
                assert np.array_equal(inr_k, inr_f), (kind, hex(lo), hex(hi))
