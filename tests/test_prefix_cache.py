"""Prefix cache of KV pages (host C++ behind the C ABI), no GPU.

Hand-worked cases pin the reference model (oracle.PrefixCacheRef) to the
rules on the pages (Vosti deep-dive blog, §3.2 engineering constraints, §5.4):
exact prefix matching (tokens, depth, parent), immutable registered pages,
leaf-only eviction that never recycles a parent of a retained child.  The same
cases run on the library, with every hash colliding (hash_bits = 0) as well as
with the full hash, and a randomized differential test compares the library
with the reference operation by operation.
"""
import random

import numpy as np
import pytest

import deterministic_paged_attention_amd as bi
from deterministic_paged_attention_amd import BiError
from oracle import PrefixCacheRef

P = 4


class Both:
    """Runs every operation on the library and on the reference and checks they agree."""

    def __init__(self, n, hash_bits):
        self.lib = bi.PrefixCache(n, P, hash_bits)
        self.ref = PrefixCacheRef(n, P)

    def match(self, tokens, max_pages):
        a = self.lib.match(tokens, max_pages)
        b = self.ref.match(tokens, max_pages)
        assert a == b, (tokens, a, b)
        return a

    def alloc(self, n):
        b = self.ref.alloc(n)
        if b is None:
            before = self.lib.stats()
            with pytest.raises(BiError):
                self.lib.alloc(n)
            assert self.lib.stats() == before
            return None
        a = self.lib.alloc(n)
        assert a == b
        return a

    def register(self, page, parent, depth, tokens):
        st, ex = self.ref.register(page, parent, depth, tokens)
        if st < 0:
            with pytest.raises(BiError):
                self.lib.register(page, parent, depth, tokens)
            return st, ex
        assert self.lib.register(page, parent, depth, tokens) == ex
        return st, ex

    def release(self, pages):
        ok = self.ref.release(pages)
        if not ok:
            with pytest.raises(BiError):
                self.lib.release(pages)
        else:
            self.lib.release(pages)
        return ok

    def check(self):
        assert self.lib.stats() == self.ref.stats()
        assert list(self.lib.writable()) == self.ref.writable()


def _fill_chain(c, tokens):
    """Allocate and register one page per full page of tokens, as a request would."""
    pages = c.alloc(len(tokens) // P)
    parent = -1
    for d, p in enumerate(pages):
        st, _ = c.register(p, parent, d, tokens[d * P:(d + 1) * P])
        assert st == 0
        parent = p
    return pages


@pytest.mark.parametrize("hash_bits", [64, 0])
def test_exact_prefix_matching(hash_bits):
    c = Both(16, hash_bits)
    a = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12]
    pages = _fill_chain(c, a)
    assert c.match(a + [99], 3) == pages                          # whole chain
    assert c.match(a[:8] + [9, 10, 11, 0], 3) == pages[:2]        # third page differs in one token
    assert c.match([0] + a[1:], 3) == []                          # first page differs
    assert c.match(a, 2) == pages[:2]                             # capped by the caller
    assert c.match(a[:7], 3) == pages[:1]                         # only full pages count
    # same page tokens at another depth are not a match: [5..8] as a first page
    assert c.match(a[4:8] + a[8:12], 2) == []
    c.check()


@pytest.mark.parametrize("hash_bits", [64, 0])
def test_same_tokens_under_another_parent_are_another_page(hash_bits):
    c = Both(16, hash_bits)
    x = _fill_chain(c, [1, 1, 1, 1, 7, 7, 7, 7])
    y = _fill_chain(c, [2, 2, 2, 2, 7, 7, 7, 7])       # second page has x[1]'s tokens but another parent
    assert x[1] != y[1]
    assert c.match([2, 2, 2, 2, 7, 7, 7, 7], 2) == y
    assert c.match([1, 1, 1, 1, 7, 7, 7, 7], 2) == x
    c.check()


def test_duplicate_registration_keeps_the_page_private():
    c = Both(8, 64)
    first = _fill_chain(c, [3, 3, 3, 3])
    dup = c.alloc(1)
    st, ex = c.register(dup[0], -1, 0, [3, 3, 3, 3])
    assert (st, ex) == (1, first[0])
    assert c.lib.writable()[dup[0]] == 1 and c.lib.writable()[first[0]] == 0
    c.check()


def test_registered_and_shared_pages_are_not_writable_and_cannot_be_registered():
    c = Both(8, 64)
    pg = _fill_chain(c, [1, 2, 3, 4])
    assert c.lib.writable()[pg[0]] == 0
    assert c.register(pg[0], -1, 0, [1, 2, 3, 4])[0] == -1        # already registered
    other = c.alloc(1)
    shared = c.match([1, 2, 3, 4], 1)                            # a second holder of pg[0]
    assert shared == pg
    assert c.register(other[0], 5, 1, [0, 0, 0, 0])[0] == -2     # parent 5 is not registered
    assert c.register(other[0], -1, 1, [0, 0, 0, 0])[0] == -2    # depth 1 needs a parent
    assert c.register(other[0], pg[0], 2, [0, 0, 0, 0])[0] == -2  # parent sits at depth 0, not 1
    c.check()


def test_leaf_only_eviction_never_recycles_a_retained_childs_parent():
    c = Both(4, 64)
    chain = _fill_chain(c, [1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3])   # A <- B <- C, all held
    spare = c.alloc(1)
    assert c.alloc(1) is None                                        # pool exhausted, everything referenced
    c.release(chain[:2])                                             # A and B unreferenced, C still held
    assert c.ref.stats()[2] == 0                                     # ... but neither is a leaf: no eviction
    assert c.alloc(1) is None
    c.release(chain[2:])                                             # C released: C is the only leaf
    got = c.alloc(1)
    assert got == [chain[2]]                                         # the leaf goes first
    got2 = c.alloc(1)
    assert got2 == [chain[1]]                                        # then B, a leaf now
    assert c.match([1, 1, 1, 1, 2, 2, 2, 2], 2) == chain[:1]         # A is still cached
    c.release(spare + got + got2 + chain[:1])
    c.check()


def test_release_below_zero_is_refused_without_change():
    c = Both(4, 64)
    p = c.alloc(2)
    assert c.release([p[0], p[0]]) is False
    c.check()
    assert c.release(p) is True
    c.check()


@pytest.mark.parametrize("hash_bits,seed", [(64, 1), (3, 2), (0, 3), (64, 4)])
def test_random_operations_agree_with_reference(hash_bits, seed):
    """Random requests over a 3-letter alphabet (many shared and colliding
    prefixes) admitted, grown, registered and released on a 24-page pool."""
    rng = random.Random(seed)
    c = Both(24, hash_bits)
    live = {}    # request -> (tokens, pages, registered count)
    for step in range(400):
        op = rng.random()
        if op < 0.35 or not live:
            toks = [rng.randrange(3) for _ in range(rng.randrange(1, 5) * P + rng.randrange(P))]
            shared = c.match(toks, (len(toks) - 1) // P)
            need = -(-len(toks) // P) - len(shared)
            priv = c.alloc(need)
            if priv is None:
                c.release(shared)
                continue
            live[step] = (toks, shared + priv, len(shared))
        elif op < 0.7:
            rid = rng.choice(sorted(live))
            toks, pages, nreg = live[rid]
            full = len(toks) // P
            if nreg < full:   # register the next full page (its writes are done)
                parent = pages[nreg - 1] if nreg else -1
                st, ex = c.register(pages[nreg], parent, nreg, toks[nreg * P:(nreg + 1) * P])
                if st == 0:
                    live[rid] = (toks, pages, nreg + 1)
                else:           # an identical page exists: later pages cannot be registered under ours
                    live[rid] = (toks, pages, full)
        else:
            rid = rng.choice(sorted(live))
            toks, pages, _ = live.pop(rid)
            assert c.release(pages)
        if step % 20 == 0:
            c.check()
    for toks, pages, _ in live.values():
        assert c.release(pages)
    c.check()
    assert c.ref.stats()[0] + c.ref.stats()[1] == 24
    assert c.ref.evictions > 10          # the run did exercise eviction


def test_abi_rejects_bad_arguments():
    L = bi.lib
    import ctypes
    h = ctypes.c_void_p()
    assert L.bi_prefix_cache_create(0, 16, 64, ctypes.byref(h)) == 1
    assert L.bi_prefix_cache_create(8, 16, 65, ctypes.byref(h)) == 1
    c = bi.PrefixCache(8, 16)
    out = np.zeros(4, dtype=np.int32)
    assert L.bi_prefix_cache_alloc(c.handle, -1, out.ctypes.data) == 1
    assert L.bi_prefix_cache_alloc(c.handle, 9, out.ctypes.data) == 3       # more than the pool
    mask = np.zeros(7, dtype=np.uint8)
    assert L.bi_prefix_cache_writable(c.handle, mask.ctypes.data, 7) == 1   # mask must cover the pool
