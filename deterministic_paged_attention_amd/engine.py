"""A small continuous-batching engine over the decoder step and the prefix cache.

Each engine step (Vosti deep-dive blog (深入解析 Vosti), §3 engine model and
§3.2 engineering constraints):
  1. admission: a waiting request looks up its prompt in the prefix cache
     (exact matching of tokens, depth and parent) and starts from the pages
     found — cache reuse is resolved before anything of this step is written;
  2. scheduling: running requests in admission order each take a chunk of
     their prompt (prefill) or their last sampled token (decode), within a
     per-step token budget; their private pages are allocated as needed;
  3. the decoder step runs over all chunks at once (new K/V written to private
     pages only; the write plan can be checked against the cache's writable
     mask);
  4. greedy sampling (argmax) for every request whose chunk reached the end of
     its known history;
  5. pages filled by this step are registered in the prefix cache (immutable
     from then on); finished requests release their pages.

Scheduling decisions (batch composition, chunk sizes, page ids, eviction) are
free to differ between runs: the decoder's kernels make every logits row a
function of the request's token history only, which is what the per-request
view of Definition 2.1 (deep-dive §2) asks for.
"""
from __future__ import annotations

import dataclasses
import hashlib
from collections import deque
from typing import Dict, List, Optional

import numpy as np
import torch

from . import BiError, PrefixCache, bi_argmax, bi_check_write_plan


@dataclasses.dataclass
class Request:
    rid: int
    prompt: List[int]
    max_new: int
    history: List[int] = dataclasses.field(default_factory=list)
    pages: List[int] = dataclasses.field(default_factory=list)
    cached: int = 0            # positions whose K/V are in the cache
    registered: int = 0        # leading pages registered in (or taken from) the prefix cache
    can_register: bool = True
    reused_pages: int = 0
    tokens: List[int] = dataclasses.field(default_factory=list)        # sampled tokens
    logit_digests: List[str] = dataclasses.field(default_factory=list)  # sha256 of each sampled logits row

    def view(self):
        """Per-request view: the outputs of this request, in order."""
        return list(zip(self.tokens, self.logit_digests))


class _DecodeGraph:
    """A decode step (B sequences, one new token each) captured as one HIP
    graph over static input buffers; page tables up to `stride` entries and
    contexts up to stride * page_size tokens replay it with new contents."""

    def __init__(self, dec, kv, B: int, stride: int, page_size: int):
        dev = "cuda"
        self.B, self.stride = B, stride
        self.ids = torch.zeros(B, dtype=torch.int32, device=dev)
        self.pt = torch.full((B, stride), -1, dtype=torch.int32, device=dev)
        self.sl = torch.ones(B, dtype=torch.int32, device=dev)
        self.qsl = torch.arange(B + 1, dtype=torch.int32, device=dev)
        self.rows = torch.arange(B, dtype=torch.int32, device=dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.logits = dec.step(self.ids, kv, self.pt, self.sl, self.qsl, stride * page_size,
                                   logit_rows=self.rows)
            self.tokens = bi_argmax(self.logits)

    def run(self, ids, pt_host, sls):
        pad = np.full((self.B, self.stride), -1, dtype=np.int32)
        pad[:, :pt_host.shape[1]] = pt_host
        self.ids.copy_(torch.tensor(ids, dtype=torch.int32))
        self.pt.copy_(torch.from_numpy(pad))
        self.sl.copy_(torch.tensor(sls, dtype=torch.int32))
        self.graph.replay()
        return self.logits, self.tokens


class Engine:
    def __init__(self, decoder, num_pages: int, budget: int, check_writes: bool = True,
                 hash_bits: int = 64, graphs: bool = False, record_logits: bool = True):
        self.dec = decoder
        self.P = decoder.shape.page_size
        self.num_pages = num_pages
        self.cache = PrefixCache(num_pages, self.P, hash_bits)
        self.kv = decoder.new_caches(num_pages)
        self.budget = budget
        self.check_writes = check_writes
        self.graphs = graphs
        self.record_logits = record_logits
        self._graphs: Dict[tuple, _DecodeGraph] = {}
        self.waiting: deque = deque()
        self.running: List[Request] = []
        self.finished: Dict[int, Request] = {}
        self.steps = 0
        self.graph_replays = 0
        self.last_step_decode_only = False

    def add(self, rid: int, prompt: List[int], max_new: int):
        if not prompt or max_new < 1:
            raise ValueError("a request needs a prompt and at least one token to generate")
        self.waiting.append(Request(rid, list(prompt), max_new, history=list(prompt)))

    def _admit(self):
        while self.waiting:
            r = self.waiting.popleft()
            # the last prompt position is always computed (its logits give the first token)
            shared = self.cache.match(r.prompt, (len(r.prompt) - 1) // self.P)
            r.pages = list(shared)
            r.cached = len(shared) * self.P
            r.registered = len(shared)
            r.reused_pages = len(shared)
            self.running.append(r)

    def _ensure_pages(self, r: Request, end: int) -> bool:
        need = -(-end // self.P) - len(r.pages)
        if need <= 0:
            return True
        try:
            r.pages.extend(self.cache.alloc(need))
            return True
        except BiError:
            return False

    def step(self) -> bool:
        """One engine step; False when there is nothing left to do."""
        self._admit()
        if not self.running:
            return False
        batch = []
        left = self.budget
        for r in self.running:
            if left == 0:
                break
            n = min(left, len(r.history) - r.cached)
            if n <= 0 or not self._ensure_pages(r, r.cached + n):
                continue
            batch.append((r, n))
            left -= n
        if not batch:
            raise RuntimeError("no request can make progress (page pool too small)")
        dev = "cuda"
        ids, qsl, sls, rows = [], [0], [], []
        for r, n in batch:
            ids.extend(r.history[r.cached:r.cached + n])
            qsl.append(qsl[-1] + n)
            sls.append(r.cached + n)
            if r.cached + n == len(r.history):
                rows.append(qsl[-1] - 1)
        stride = max(len(r.pages) for r, _ in batch)
        pt = np.full((len(batch), stride), -1, dtype=np.int32)
        for i, (r, _) in enumerate(batch):
            pt[i, :len(r.pages)] = r.pages
        if self.check_writes:
            slots = [r.pages[p // self.P] * self.P + p % self.P for r, n in batch for p in range(r.cached, r.cached + n)]
            bi_check_write_plan(slots, self.cache.writable(), self.num_pages, self.P)
        decode_only = all(n == 1 for _, n in batch) and len(rows) == len(batch)
        self.last_step_decode_only = decode_only
        # Decode steps replay a captured graph once their shape bucket has been
        # seen (the first step of a bucket runs eagerly); everything else runs eagerly.
        bucket = (len(batch), -(-stride // 16) * 16)
        g = self._graphs.get(bucket) if (self.graphs and decode_only) else None
        if g is not None:
            logits, toks = g.run(ids, pt, sls)
            self.graph_replays += 1
        else:
            logits = self.dec.step(torch.tensor(ids, dtype=torch.int32, device=dev), self.kv,
                                   torch.from_numpy(pt).to(dev), torch.tensor(sls, dtype=torch.int32, device=dev),
                                   torch.tensor(qsl, dtype=torch.int32, device=dev), max(sls),
                                   logit_rows=torch.tensor(rows, dtype=torch.int32, device=dev) if rows else None)
            toks = bi_argmax(logits) if rows else None
            if self.graphs and decode_only:
                self._graphs[bucket] = _DecodeGraph(self.dec, self.kv, bucket[0], bucket[1], self.P)
        sampled = toks.cpu().tolist() if rows else []
        host_logits = logits.cpu().numpy() if (rows and self.record_logits) else None
        k = 0
        for r, n in batch:
            r.cached += n
            if r.cached == len(r.history):
                tok = int(sampled[k])
                r.tokens.append(tok)
                if host_logits is not None:
                    r.logit_digests.append(hashlib.sha256(host_logits[k].tobytes()).hexdigest())
                r.history.append(tok)
                k += 1
            self._register_full_pages(r)
        self.steps += 1
        for r in list(self.running):
            if len(r.tokens) >= r.max_new:
                self.cache.release(r.pages)
                r.pages = []
                self.running.remove(r)
                self.finished[r.rid] = r
        return True

    def _register_full_pages(self, r: Request):
        """Register the pages this request has filled (after the step that wrote them)."""
        while r.can_register and r.registered < r.cached // self.P:
            d = r.registered
            parent = r.pages[d - 1] if d > 0 else -1
            existing = self.cache.register(r.pages[d], parent, d, r.history[d * self.P:(d + 1) * self.P])
            if existing >= 0:
                # an identical page is already cached: ours stays private, and the
                # pages after it cannot hang under it
                r.can_register = False
                break
            r.registered += 1

    def run(self, max_steps: int = 100000, arrivals: Optional[Dict[int, List[tuple]]] = None):
        """Steps until every request has finished.  arrivals[s] lists
        (rid, prompt, max_new) added before step s."""
        arrivals = arrivals or {}
        s = 0
        while s < max_steps:
            for a in arrivals.get(s, []):
                self.add(*a)
            more = self.step() if (self.running or self.waiting) else False
            if not more and not any(k > s for k in arrivals):
                break
            s += 1
        return self.finished
