"""The CU masks of the partitioned streams (sparse_top_kv_gqa_amd/streams.py), on the host."""
import pytest

from sparse_top_kv_gqa_amd.streams import XCDS, cu_partition_streams, partition_masks


def _bits(words):
    return {32 * j + b for j, w in enumerate(words) for b in range(32) if w >> b & 1}


@pytest.mark.parametrize("part", [8, 16, 32, 48, 64, 80, 96, 128, 136, 200, 248])
def test_masks_split_the_device_and_reach_every_die(part):
    a, b = partition_masks(256, part)
    assert len(a) == len(b) == XCDS
    A, B = _bits(a), _bits(b)
    assert len(A) == part and not (A & B) and A | B == set(range(256))
    for words in (a, b):
        bits = _bits(words)
        # one die per 32-bit word: every word holds some CUs, the part the same number in each
        assert all(w != 0 for w in words)
        # die = CU number mod 8: every residue appears
        assert {i % XCDS for i in bits} == set(range(XCDS))
    assert all(bin(w).count("1") == part // XCDS for w in a)


@pytest.mark.parametrize("total, part", [(256, 0), (256, 256), (256, 12), (304, 64), (128, 64)])
def test_masks_refuse_what_they_cannot_split(total, part):
    with pytest.raises(ValueError):
        partition_masks(total, part)


def test_partitioned_streams_are_switched_off():
    with pytest.raises(NotImplementedError, match="switched off"):
        cu_partition_streams(64)
