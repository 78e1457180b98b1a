"""Oracle of the prompt page split (which split owns which logical page).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages deal Qwen prompt pages to the eight context-parallel ranks
block-cyclically (LongStraw review page, section 7 mind map,
"Qwen3.6-27B implementation": CP8 page ownership, block-cyclic) and insist that
a compact page be a real allocation of its own rather than a view into a
larger block (review page, section 2, item 2).  The block size is not given;
it is a parameter here.

Definitions (one split per emulated rank):
  * contiguous:   the n logical pages are cut into S consecutive ranges; with
                  n = a*S + b, the first b ranges hold a+1 pages, the others a;
  * block-cyclic: logical page p belongs to split (p // B) mod S;
  * explicit:     logical page p belongs to split owner[p].
Inside a split, pages are listed in increasing logical order.  The result is
CSR: ``order`` (logical page ids, split-major) and ``offsets [S+1]``.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

SPLIT_CONTIGUOUS = 0
SPLIT_BLOCK_CYCLIC = 1
SPLIT_EXPLICIT = 2


def split_pages(num_pages: int, num_splits: int, policy: int, block_pages: int = 1,
                owner: Optional[Sequence[int]] = None) -> Tuple[list, list]:
    owners = []
    if policy == SPLIT_CONTIGUOUS:
        a, b = divmod(num_pages, num_splits)
        for c in range(num_splits):
            owners += [c] * (a + (1 if c < b else 0))
    elif policy == SPLIT_BLOCK_CYCLIC:
        owners = [(p // block_pages) % num_splits for p in range(num_pages)]
    elif policy == SPLIT_EXPLICIT:
        owners = [int(x) for x in owner]
    else:
        raise ValueError("unknown policy")
    lists = [[] for _ in range(num_splits)]
    for p in range(num_pages):
        lists[owners[p]].append(p)
    order, offsets = [], [0]
    for c in range(num_splits):
        order += lists[c]
        offsets.append(len(order))
    return order, offsets
