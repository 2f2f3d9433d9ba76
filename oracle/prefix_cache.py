"""Reference model of the KV-page prefix cache (test infrastructure only).

What the cache must do, written as plainly as possible (Vosti deep-dive blog
(深入解析 Vosti), §3.2 engineering constraints, §5.4 exact prefix matching):
a registered page stands for one exact token prefix — every token from
position 0 through the end of the page — so lookups are keyed by that exact
tuple of tokens (no hashing at all: a hash collision cannot make two different
prefixes equal here); registered pages are immutable; only registered pages
with no reference and no registered child (leaves) are evicted, least recently
used first (ties by page id); free pages are handed out from a stack that
starts as 0, 1, 2, ...

The page-id bookkeeping (free stack, use clock) follows the library's
documented policy so that a differential test can compare page ids, not just
counts.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class PrefixCacheRef:
    def __init__(self, num_pages: int, page_size: int):
        self.P = page_size
        self.n = num_pages
        self.free: List[int] = list(range(num_pages - 1, -1, -1))  # popped from the end
        self.ref = [0] * num_pages
        self.prefix: Dict[int, Tuple[int, ...]] = {}   # registered page -> the exact prefix it completes
        self.page_of: Dict[Tuple[int, ...], int] = {}  # exact prefix -> registered page
        self.tick = [0] * num_pages
        self.clock = 0
        self.evictions = 0

    # -- helpers
    def _touch(self, p: int):
        self.clock += 1
        self.tick[p] = self.clock

    def _children(self, p: int) -> int:
        pre = self.prefix[p]
        return sum(1 for q, pr in self.prefix.items() if len(pr) == len(pre) + self.P and pr[:len(pre)] == pre)

    def _evictable(self) -> List[int]:
        return [p for p in self.prefix if self.ref[p] == 0 and self._children(p) == 0]

    # -- operations
    def match(self, tokens: Sequence[int], max_pages: int) -> List[int]:
        out = []
        k = 0
        while k < max_pages and (k + 1) * self.P <= len(tokens):
            p = self.page_of.get(tuple(tokens[:(k + 1) * self.P]))
            if p is None:
                break
            out.append(p)
            k += 1
        for p in out:
            self.ref[p] += 1
            self._touch(p)
        return out

    def alloc(self, n: int) -> Optional[List[int]]:
        # pages eviction could reclaim: registered pages with no referenced page in their subtree
        reclaimable = 0
        for p, pre in self.prefix.items():
            sub = [q for q, pr in self.prefix.items() if pr[:len(pre)] == pre]
            if all(self.ref[q] == 0 for q in sub):
                reclaimable += 1
        if len(self.free) + reclaimable < n:
            return None
        out = []
        for _ in range(n):
            if not self.free:
                victim = min(self._evictable(), key=lambda q: (self.tick[q], q))
                del self.page_of[self.prefix.pop(victim)]
                self.tick[victim] = 0
                self.free.append(victim)
                self.evictions += 1
            p = self.free.pop()
            self.ref[p] = 1
            self._touch(p)
            out.append(p)
        return out

    def register(self, page: int, parent: int, depth: int, tokens: Sequence[int]):
        """Returns (status, existing): status 0 registered, 1 duplicate, -1 page not
        private, -2 bad parent/depth."""
        if page in self.prefix or self.ref[page] != 1:
            return -1, -1
        if depth < 0 or (depth == 0) != (parent < 0):
            return -2, -1
        if parent >= 0 and (parent not in self.prefix or len(self.prefix[parent]) != depth * self.P):
            return -2, -1
        pre = (self.prefix[parent] if parent >= 0 else ()) + tuple(tokens)
        if pre in self.page_of:
            return 1, self.page_of[pre]
        self.prefix[page] = pre
        self.page_of[pre] = page
        self._touch(page)
        return 0, -1

    def release(self, pages: Sequence[int]) -> bool:
        need: Dict[int, int] = {}
        for p in pages:
            if p >= 0:
                need[p] = need.get(p, 0) + 1
        if any(c > self.ref[p] for p, c in need.items()):
            return False
        for p in pages:
            if p < 0:
                continue
            self.ref[p] -= 1
            if self.ref[p] == 0 and p not in self.prefix:
                self.tick[p] = 0
                self.free.append(p)
        return True

    def writable(self) -> List[int]:
        return [1 if (p not in self.prefix and self.ref[p] == 1) else 0 for p in range(self.n)]

    def stats(self) -> Tuple[int, int, int, int]:
        return (len(self.free), len(self.prefix), len(self._evictable()), self.evictions)
