"""On-demand page allocation and block tables (oracle; test infrastructure only).

The pages sketch the allocator without fixing its policy: a sequence's
cache is held in blocks of a fixed token count (16 unless configured
otherwise), which may sit anywhere in memory and are handed out one at a time
as the sequence grows, instead of one slab sized for the longest possible
sequence; a table per request translates logical block numbers into
physical ones
("Inference Engines" chapter 17, "The Breakthrough"; evaltude docs
"Transformer inference mechanics", "FlashAttention versus PagedAttention";
CS336 lecture 10 notes, "PagedAttention (vLLM)").

Concrete rules, the plainest reading that the pages support:

* The pool starts with a free list in a caller-given order (the random page
  placement of a workload is that order; identity if none is given).
* ``reserve(seq, n_tokens)`` grows ``seq`` to ceil(n_tokens / bs) blocks by
  taking pages from the front of the free list, in order; it never shrinks.
  If too few pages are free it fails and changes nothing.
* ``release(seq)`` returns the sequence's pages to the back of the free list,
  in block order, and forgets the sequence.
* A block-table row lists the sequence's pages in logical order, padded
  with -1.

Sharing of blocks between sequences (prefix sharing with copy-on-write,
described in the CS336 notes' "PagedAttention (vLLM)" section) is modelled by
``fork`` and ``reserve_for_write``: a fork gives the child the parent's pages
with each page's reference count raised; a write into a block whose page is
shared first replaces that block with a fresh page (the caller copies the
contents), dropping one reference from the old page.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np


class OutOfPages(Exception):
    pass


class PagePool:
    def __init__(self, num_pages: int, free_order: Optional[Iterable[int]] = None):
        order = list(range(num_pages)) if free_order is None else [int(p) for p in free_order]
        if sorted(order) != list(range(num_pages)):
            raise ValueError("free_order must be a permutation of 0..num_pages-1")
        self.num_pages = num_pages
        self.free = deque(order)
        self.seqs: Dict[int, List[int]] = {}
        self.refs = [0] * num_pages

    def num_free(self) -> int:
        return len(self.free)

    def blocks(self, seq_id: int) -> List[int]:
        return list(self.seqs.get(seq_id, []))

    def reserve(self, seq_id: int, n_tokens: int, block_size: int = 16) -> int:
        """Grow seq_id to hold n_tokens; returns how many pages were taken."""
        if n_tokens < 0 or block_size <= 0:
            raise ValueError("bad length or block size")
        pages = self.seqs.get(seq_id, [])
        need = -(-n_tokens // block_size) - len(pages)
        if need <= 0:
            self.seqs.setdefault(seq_id, pages)
            return 0
        if need > len(self.free):
            raise OutOfPages(f"need {need} pages, {len(self.free)} free")
        for _ in range(need):
            p = self.free.popleft()
            self.refs[p] = 1
            pages.append(p)
        self.seqs[seq_id] = pages
        return need

    def release(self, seq_id: int) -> None:
        if seq_id not in self.seqs:
            raise KeyError(seq_id)
        for p in self.seqs.pop(seq_id):
            self.refs[p] -= 1
            if self.refs[p] == 0:
                self.free.append(p)

    def fork(self, parent: int, child: int) -> None:
        """child shares every page of parent (reference counts go up by one)."""
        if parent not in self.seqs or child in self.seqs:
            raise KeyError((parent, child))
        pages = list(self.seqs[parent])
        for p in pages:
            self.refs[p] += 1
        self.seqs[child] = pages

    def reserve_for_write(self, seq_id: int, position: int,
                          block_size: int = 16) -> Optional[Tuple[int, int]]:
        """Make token `position` of seq_id writable.  Grows the sequence if the
        position is past its last block.  If the block holding the position is
        shared, it is replaced by a fresh page and (old_page, new_page) is
        returned so the caller can copy the contents; otherwise None."""
        self.reserve(seq_id, position + 1, block_size)
        pages = self.seqs[seq_id]
        blk = position // block_size
        old = pages[blk]
        if self.refs[old] == 1:
            return None
        if not self.free:
            raise OutOfPages("no page for copy-on-write")
        new = self.free.popleft()
        self.refs[new] = 1
        self.refs[old] -= 1
        pages[blk] = new
        return old, new

    def block_table(self, seq_ids: Iterable[int], max_blocks: int) -> np.ndarray:
        seq_ids = list(seq_ids)
        out = np.full((len(seq_ids), max_blocks), -1, dtype=np.int32)
        for i, s in enumerate(seq_ids):
            pages = self.seqs.get(s, [])
            if len(pages) > max_blocks:
                raise ValueError("sequence has more blocks than max_blocks")
            out[i, :len(pages)] = pages
        return out
