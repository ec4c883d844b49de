"""Plain Python model of a paged KV-cache block manager and its scheduler step.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library's C++ block
manager is checked against this model operation by operation.

What the pages fix ("KV cache, GQA, paging and continuous batching", sections
"PagedAttention: why fragmentation was eating most of the rest", "Prefix
caching: the biggest single lever most teams have" and "The scheduler, and
preemption"; "KV cache, continuous batching and paged attention", sections
"Paged attention" and "Prefix caching"):
  - the cache is a pool of fixed 16-token blocks; a sequence's block table
    maps its logical positions to physical blocks, allocated on demand as it
    grows, so at most its last block is partly filled;
  - sequences with a common prefix point at the same physical blocks, with
    copy-on-write when one of them writes into a shared block;
  - prefix caching reuses the blocks of an identical token prefix, a prefix
    match over whole blocks;
  - admission is bounded by free blocks (a request that does not fit waits),
    and when a running sequence cannot get a block the newest running
    sequence is preempted (its blocks freed, the request re-queued first, to
    be recomputed).

Where the pages are silent this model fixes one plain reading, and the C++
manager follows the same one:
  - free blocks form a FIFO queue, initially 0, 1, ..., num_blocks - 1;
    allocation takes the front, release appends to the back;
  - a full block written from a prompt is entered in the prefix cache under
    the chain key (key of the previous block, its 16 tokens); generated
    tokens' blocks are not cached;
  - a cached block whose last reference goes away is kept, evictable, in an
    LRU queue; allocation uses free blocks first, then evicts the oldest
    evictable block (dropping its cache entry); a cache hit on an evictable
    block takes it back;
  - a sequence's blocks are released last block first;
  - an operation that cannot get the blocks it needs changes nothing.
Chain keys are compared exactly (the whole key, not a hash), so there are
no false hits.
"""
from __future__ import annotations

from collections import OrderedDict, deque

BLOCK = 16


class NoBlocks(Exception):
    """Not enough free blocks: the operation changed nothing."""


class BlockManager:
    def __init__(self, num_blocks: int, prefix_cache: bool = True):
        self.num_blocks = num_blocks
        self.prefix_cache = prefix_cache
        self.free = deque(range(num_blocks))
        self.evictable = OrderedDict()      # block -> None, oldest first
        self.ref = [0] * num_blocks
        self.cache = {}                     # chain key -> block
        self.key_of = {}                    # block -> chain key
        self.tables = {}                    # seq -> list of blocks
        self.lens = {}                      # seq -> tokens

    # -- blocks -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:
            b, _ = self.evictable.popitem(last=False)
            del self.cache[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.evictable[b] = None
            else:
                self.free.append(b)

    # -- sequences ------------------------------------------------------------
    def add(self, seq, tokens) -> int:
        """Blocks for a prompt; returns how many of its tokens the prefix
        cache already held."""
        tokens = list(tokens)
        n = len(tokens)
        full = n // BLOCK
        keys, hits = [], []
        key = None
        for i in range(full):
            key = (key, tuple(tokens[i * BLOCK:(i + 1) * BLOCK]))
            keys.append(key)
        if self.prefix_cache:
            for k in keys:
                if k not in self.cache:
                    break
                hits.append(self.cache[k])
        need = -(-n // BLOCK) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if need > self.num_free() - revived:
            raise NoBlocks
        table = []
        for b in hits:
            if self.ref[b] == 0:
                del self.evictable[b]
            self.ref[b] += 1
            table.append(b)
        for i in range(len(hits), -(-n // BLOCK)):
            b = self._take()
            table.append(b)
            if self.prefix_cache and i < full and keys[i] not in self.cache:
                self.cache[keys[i]] = b
                self.key_of[b] = keys[i]
        self.tables[seq] = table
        self.lens[seq] = n
        return len(hits) * BLOCK

    def append(self, seq):
        """Room for one more token. Returns (src, dst) when the last block was
        shared and had to be copied first (copy-on-write), else None."""
        table, n = self.tables[seq], self.lens[seq]
        cow = None
        if n % BLOCK == 0:
            if self.num_free() < 1:
                raise NoBlocks
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            if self.num_free() < 1:
                raise NoBlocks
            src = table[-1]
            dst = self._take()
            self._drop(src)
            table[-1] = dst
            cow = (src, dst)
        self.lens[seq] = n + 1
        return cow

    def fork(self, parent, child) -> None:
        for b in self.tables[parent]:
            self.ref[b] += 1
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]

    def release(self, seq) -> None:
        for b in reversed(self.tables.pop(seq)):
            self._drop(b)
        del self.lens[seq]

    def slot(self, seq, pos: int) -> int:
        return self.tables[seq][pos // BLOCK] * BLOCK + pos % BLOCK


class Scheduler:
    """One step: admit waiting requests in order while their prompts fit,
    then give every running sequence room for its next token, oldest first;
    when a block is missing, preempt the newest running sequence (release its
    blocks, put its request, the prompt plus the tokens recorded so far,
    first in the waiting queue) and try again. A sequence that is itself the
    newest is preempted rather than another; the last running sequence is
    never preempted (the step reports it as stalled). After the step, the
    caller records each running sequence's new token with record()."""

    def __init__(self, bm: BlockManager):
        self.bm = bm
        self.waiting = deque()
        self.running = []           # oldest first
        self.tokens = {}

    def submit(self, seq, prompt) -> None:
        self.waiting.append(seq)
        self.tokens[seq] = list(prompt)

    def step(self):
        """Returns (running, preempted, cows, stalled)."""
        while self.waiting:
            s = self.waiting[0]
            try:
                self.bm.add(s, self.tokens[s])
            except NoBlocks:
                break
            self.waiting.popleft()
            self.running.append(s)
        preempted, cows, stalled = [], [], []
        i = 0
        while i < len(self.running):
            s = self.running[i]
            try:
                cow = self.bm.append(s)
            except NoBlocks:
                if len(self.running) == 1:
                    stalled.append(s)
                    i += 1
                    continue
                victim = self.running.pop()
                self.bm.release(victim)
                self.waiting.appendleft(victim)
                preempted.append(victim)
                continue
            if cow is not None:
                cows.append(cow)
            i += 1
        return [s for s in self.running if s not in stalled], preempted, cows, stalled

    def record(self, seq, token) -> None:
        self.tokens[seq].append(token)

    def finish(self, seq) -> None:
        self.running.remove(seq)
        self.bm.release(seq)
        del self.tokens[seq]
