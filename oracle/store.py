"""Chunk KV store: chunk keys and the store's hit / miss / eviction behaviour.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

From the pages:
* CacheBlend explainer, integration with vLLM: a hash table in CPU memory (about 16 MB per
  million chunks) finds where a chunk's KV cache is stored;
* the same page's RAG example keys a document by the first 16 hex digits (64 bits) of a
  SHA-256 digest of its content;
* KVBoost article, "dual hash keys": a content key from the chunk's tokens alone (the same
  text at another position gets the same key) and a prefix key from the chunk's tokens
  together with the hash values of every earlier chunk, both SHA-256;
* LMCache blog, sections 1 and the L1 experiment: eviction is least-recently-used, and a
  cyclic scan over a working set larger than the cache never hits.

Readings (the pages leave these open):
* tokens are hashed as little-endian int32; earlier keys as 8-byte big-endian integers and
  placed before the tokens; the key is the first 8 bytes of the digest read big-endian (the
  RAG example's 16 hex digits);
* the prefix key's "hash values of every earlier chunk" are those chunks' content keys;
* an entry is found only when its tokens (and earlier keys) are equal to the request's, not
  merely its key;
* a lookup that hits makes the entry the most recently used; inserting an entry that is
  already stored only refreshes it; a full store evicts its least recently used entry that
  no caller holds (pin), and refuses the insert when every entry is held.  The importance
  weighting of KVBoost's eviction is not modelled: the page does not say how importance and
  recency combine.
"""
from __future__ import annotations

import hashlib
from collections import OrderedDict
from typing import Optional, Sequence, Tuple

import numpy as np


def key_message(tokens: Sequence[int], prior: Sequence[int] = ()) -> bytes:
    """Bytes hashed for a chunk: earlier keys (8 bytes big-endian each), then the tokens."""
    head = b"".join(int(k).to_bytes(8, "big") for k in prior)
    return head + np.asarray(tokens, dtype="<i4").tobytes()


def chunk_key(tokens: Sequence[int], prior: Sequence[int] = ()) -> int:
    """64-bit key: the first 8 bytes of SHA-256(key_message), big-endian."""
    return int.from_bytes(hashlib.sha256(key_message(tokens, prior)).digest()[:8], "big")


def content_key(tokens: Sequence[int]) -> int:
    return chunk_key(tokens)


def prefix_keys(chunks: Sequence[Sequence[int]]) -> list:
    """Prefix key of every chunk of a prompt: its tokens with the content keys of all earlier
    chunks."""
    content = [content_key(c) for c in chunks]
    return [chunk_key(c, content[:i]) for i, c in enumerate(chunks)]


class StoreFull(Exception):
    """Every entry is held by a caller: nothing can be evicted."""


class ChunkStore:
    """LRU store of at most `capacity` chunks, identified by their full content.

    Entries are (tokens, prior keys) tuples; the order of the OrderedDict is recency (last =
    most recent); the value is how many callers hold the entry.
    """

    def __init__(self, capacity: int):
        assert capacity > 0
        self.capacity = capacity
        self.entries: "OrderedDict[Tuple[tuple, tuple], int]" = OrderedDict()
        self.hits = self.misses = self.evictions = 0

    @staticmethod
    def ident(tokens, prior=()) -> Tuple[tuple, tuple]:
        return tuple(int(t) for t in tokens), tuple(int(k) for k in prior)

    def lookup(self, tokens, prior=(), pin: bool = False) -> bool:
        e = self.ident(tokens, prior)
        if e not in self.entries:
            self.misses += 1
            return False
        self.hits += 1
        self.entries.move_to_end(e)
        if pin:
            self.entries[e] += 1
        return True

    def insert(self, tokens, prior=()) -> Optional[Tuple[tuple, tuple]]:
        """Store the chunk; returns the evicted entry, or None."""
        e = self.ident(tokens, prior)
        if e in self.entries:
            self.entries.move_to_end(e)
            return None
        victim = None
        if len(self.entries) >= self.capacity:
            victim = next((v for v, held in self.entries.items() if held == 0), None)
            if victim is None:
                raise StoreFull("every stored chunk is held")
            del self.entries[victim]
            self.evictions += 1
        self.entries[e] = 0
        return victim

    def release(self, tokens, prior=()) -> None:
        e = self.ident(tokens, prior)
        assert self.entries.get(e, 0) > 0, "release of an entry nobody holds"
        self.entries[e] -= 1

    def __contains__(self, item) -> bool:
        tokens, prior = item
        return self.ident(tokens, prior) in self.entries

    def __len__(self) -> int:
        return len(self.entries)
