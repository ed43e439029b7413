"""Prefix-cache model (oracle; test infrastructure only).

What it models, from the pages: an engine can keep the KV cache of one request
and reuse it for a later request that starts with the same tokens; the reuse
runs from the first token up to the first token that differs, and nothing
after that point is reused even when later tokens agree again (ranksignal.fr
post 218, "Mettre en cache"; copy-on-write sharing of blocks between
sequences: "PagedAttention, décodage spéculatif, MoE et Blackwell", section 1).

This library's reading, which the C++ pool implements identically:
  * the unit of reuse is a whole 16-token block: block j of a prompt is reused
    only if tokens [0, 16 (j + 1)) all agree with a registered prompt, so a
    key is the whole token prefix up to the end of its block;
  * ``insert(seq, tokens)`` registers the full blocks of ``seq``'s first
    min(len(tokens), length) tokens that are not registered yet; each
    registered block gains one reference, held by the cache;
  * ``alloc_from(seq, tokens)`` starts ``seq`` sharing the longest registered
    run of leading blocks (one more reference each), with that many tokens;
  * every insert and alloc_from is one tick of a clock and marks the entries
    on its path as used at that tick;
  * ``evict(k)`` drops up to k entries, one at a time: always an entry that no
    other entry extends, the least recently used first, ties to the entry
    registered first; a block left with no reference goes to the back of the
    free list.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

from .allocator import BLOCK, InvalidError, PoolModel


class PrefixCacheModel:
    def __init__(self, pool: PoolModel):
        self.pool = pool
        # full token prefix (length a multiple of 16) -> [block, last use, registration order]
        self.entries: Dict[Tuple[int, ...], List[int]] = {}
        self.clock = 0
        self.registered = 0

    def __len__(self) -> int:
        return len(self.entries)

    def match(self, tokens: Sequence[int]) -> int:
        """Tokens (a multiple of 16) at the start of ``tokens`` held by registered blocks."""
        t = tuple(int(x) for x in tokens)
        m = 0
        # (at most one sequence's table of blocks)
        while m < self.pool.max_blocks and len(t) >= BLOCK * (m + 1) and t[: BLOCK * (m + 1)] in self.entries:
            m += 1
        return BLOCK * m

    def insert(self, seq: int, tokens: Sequence[int]) -> int:
        """Register the full blocks of ``seq`` named by ``tokens``; returns how
        many blocks were newly registered."""
        if not self.pool.live(seq):
            raise InvalidError("insert from a sequence that is not live")
        t = tuple(int(x) for x in tokens)
        nb = min(len(t), self.pool.length(seq)) // BLOCK
        table = self.pool.table(seq)
        self.clock += 1
        new = 0
        for j in range(nb):
            key = t[: BLOCK * (j + 1)]
            if key not in self.entries:
                b = table[j]
                self.entries[key] = [b, 0, self.registered]
                self.registered += 1
                self.pool.rc[b] += 1
                new += 1
            self.entries[key][1] = self.clock
        return new

    def alloc_from(self, seq: int, tokens: Sequence[int]) -> int:
        """Create ``seq`` holding the registered leading blocks of ``tokens``;
        returns its length (the matched tokens)."""
        self.pool.alloc(seq)  # checks the id; an empty sequence
        m = self.match(tokens)
        t = tuple(int(x) for x in tokens)
        self.clock += 1
        blocks = []
        for j in range(m // BLOCK):
            e = self.entries[t[: BLOCK * (j + 1)]]
            e[1] = self.clock
            blocks.append(e[0])
            self.pool.rc[e[0]] += 1
        self.pool.tables[seq] = blocks
        self.pool.lens[seq] = m
        return m

    def _is_leaf(self, key: Tuple[int, ...]) -> bool:
        n = len(key) + BLOCK
        return not any(len(k) == n and k[: len(key)] == key for k in self.entries)

    def evict(self, max_entries: int) -> int:
        if max_entries < 0:
            raise InvalidError("max_entries < 0")
        done = 0
        while done < max_entries and self.entries:
            leaves = [k for k in self.entries if self._is_leaf(k)]
            key = min(leaves, key=lambda k: (self.entries[k][1], self.entries[k][2]))
            b = self.entries.pop(key)[0]
            self.pool._release(b)
            done += 1
        return done
