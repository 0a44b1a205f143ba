"""Host block allocation of a paged KV cache, written plainly (test infrastructure).

Follows the "PagedAttention principle" page, paged attention principle section:
memory is handed out in blocks of ``block_size`` token slots, so a request of n
tokens holds ceil(n / block_size) blocks and wastes less than one block; the
blocks need not be adjacent, a table keeps their order; the host knows each
request's blocks and hands the table to the kernels. A position's slot is the
Qwen3-0.6B engine walkthrough page's block * block_size + offset (section 2.6).

The pages fix no order in which free blocks are handed out (reading R12): here
the free list starts as 0, 1, ..., num_blocks - 1; a step takes blocks from its
front, sequence by sequence in the order listed, positions in increasing order;
releasing a sequence puts its blocks, in table order, back at the front.

Only the tests and the benchmark's CPU baseline use this module.
"""
from __future__ import annotations

import numpy as np


class NoSpace(Exception):
    """The step needs more blocks than are free; nothing was changed."""


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int):
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = list(range(num_blocks))
        self.tables: dict[int, list[int]] = {}   # sequence -> its blocks, position order
        self.lens: dict[int, int] = {}           # sequence -> tokens it holds

    def blocks_needed(self, n_tokens: int) -> int:
        """ceil(n / block_size): the page's allocation unit."""
        return -(-n_tokens // self.block_size)

    def slot(self, seq: int, pos: int) -> int:
        """Position pos of sequence seq lives in block table[pos // bs] at offset pos % bs."""
        return self.tables[seq][pos // self.block_size] * self.block_size + pos % self.block_size

    def step(self, seqs, num_new):
        """Grow sequence seqs[i] by num_new[i] tokens; return the step's metadata
        (slot of each new token, each sequence's table, new lengths, packed
        query offsets). Raises NoSpace (state unchanged) if blocks run out and
        ValueError for a malformed step."""
        seqs = [int(s) for s in seqs]
        num_new = [int(n) for n in num_new]
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence is listed twice")
        if any(n < 0 for n in num_new):
            raise ValueError("negative token count")
        need = 0
        for s, n in zip(seqs, num_new):
            have = len(self.tables.get(s, []))
            want = self.blocks_needed(self.lens.get(s, 0) + n)
            if want > self.max_blocks_per_seq:
                raise ValueError("sequence exceeds its table width")
            need += want - have
        if need > len(self.free):
            raise NoSpace(f"need {need} blocks, {len(self.free)} free")

        slots, tables, ctx, cu = [], [], [], [0]
        for s, n in zip(seqs, num_new):
            table = self.tables.setdefault(s, [])
            old = self.lens.get(s, 0)
            new = old + n
            while len(table) < self.blocks_needed(new):
                table.append(self.free.pop(0))
            self.lens[s] = new
            slots.extend(self.slot(s, p) for p in range(old, new))
            tables.append(list(table))
            ctx.append(new)
            cu.append(cu[-1] + n)
        return slots, tables, ctx, cu

    def release(self, seq: int) -> None:
        """Give back every block of seq; its length becomes 0."""
        self.free = self.tables.pop(seq, []) + self.free
        self.lens.pop(seq, None)

    def step_arrays(self, seqs, num_new, width: int, pad_seqs: int | None = None,
                    pad_tokens: int | None = None):
        """step() as the arrays the kernels take, padded with empty sequences
        (length 0, tables of -1) and skipped slots (-1)."""
        slots, tables, ctx, cu = self.step(seqs, num_new)
        B = len(seqs) if pad_seqs is None else pad_seqs
        T = len(slots) if pad_tokens is None else pad_tokens
        sm = np.full(T, -1, dtype=np.int64)
        sm[:len(slots)] = slots
        bt = np.full((B, width), -1, dtype=np.int32)
        for i, t in enumerate(tables):
            bt[i, :len(t)] = t
        cl = np.zeros(B, dtype=np.int32)
        cl[:len(ctx)] = ctx
        cs = np.full(B + 1, cu[-1], dtype=np.int32)
        cs[:len(cu)] = cu
        return sm, bt, cl, cs
