"""CU-partitioned HIP streams: two streams whose kernels run on disjoint sets of compute units
(``hipExtStreamCreateWithCUMask``).  A kernel bound by PCIe reads keeps its workgroups resident
for as long as its host reads take; beside an HBM-bound kernel on the same CUs it takes that
kernel's workgroup slots and both slow down.  On disjoint CUs each keeps its own.

Stream plumbing only: no step of the path runs here.  The streams themselves are switched off
(``cu_partition_streams`` raises, with the reason); the mask arithmetic stays, tested on the host.

Mask layout.  A gfx950 device with 256 CUs has 8 accelerator complex dies (XCDs) of 32 CUs, and
the mask is 8 words of 32 bits.  The mask's documentation fixes the bit order (bit i of word j
is CU 32 j + i) but not how those CU numbers map onto the XCDs, and an XCD left with no CU in a
stream's mask could never run that stream's workgroups dispatched to it.  The masks built here
leave every XCD some CUs under either mapping, one die per word or die = CU number mod 8: every
word holds the same number of bits, laid out as a run (modulo 8, 16 or 32) whose start advances
from word to word so that every residue mod 8 appears.  The rest of the device gets the
complement, which has the same property.
"""
from __future__ import annotations

from typing import List, Tuple

XCDS = 8            # accelerator complex dies of a 256-CU gfx950 device
WORD_BITS = 32


def partition_masks(total_cus: int, part_cus: int) -> Tuple[List[int], List[int]]:
    """The CU masks (32-bit words) of a part of ``part_cus`` CUs and of the rest.

    Requires total_cus = XCDS * 32 (one word per die) and part_cus a multiple of XCDS with
    0 < part_cus < total_cus."""
    if total_cus != XCDS * WORD_BITS:
        raise ValueError(f"CU partition needs {XCDS * WORD_BITS} CUs, the device has {total_cus}")
    if part_cus <= 0 or part_cus >= total_cus or part_cus % XCDS:
        raise ValueError(f"part_cus must be a multiple of {XCDS} in (0, {total_cus}), "
                         f"got {part_cus}")
    n = part_cus // XCDS
    period = 8 if n <= 8 else 16 if n <= 16 else 32
    part = []
    for j in range(XCDS):
        word = 0
        for t in range(n):
            word |= 1 << ((n * j + t) % period)
        part.append(word)
    rest = [(~w) & 0xFFFFFFFF for w in part]
    return part, rest


SWITCHED_OFF = (
    "CU-partitioned streams are switched off: a process that created them, ran its steps and "
    "printed its results ended in a segmentation fault at exit, also with the mask given at its "
    "exact length and read back into an ample buffer; the cause is not found")


def cu_partition_streams(part_cus: int, device=None):
    """(rest, part): a stream on every CU but ``part_cus`` of them, and one on those.

    Switched off (raises): see SWITCHED_OFF.  The masks it would use are partition_masks'."""
    raise NotImplementedError(SWITCHED_OFF)
