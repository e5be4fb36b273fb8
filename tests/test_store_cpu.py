"""The library's chunk store and keys through the C ABI, on the CPU (pageable arena, no GPU):
SHA-256 against the FIPS 180-2 examples and hashlib, chunk keys and every hit / miss /
eviction against the oracle's store (oracle/store.py) on random operation sequences."""
import ctypes
import json
import os
import threading

import numpy as np
import pytest

from oracle import store as S
from rag_kv_cache_amd import _lib as L

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sha256_vectors.json")


def _desc(n_layers=2, n_kv=2, head_dim=4, dtype=L.CB_F32):
    return L.cb_model_desc(n_layers, 128, n_kv, n_kv, head_dim, 64, 16, 64, 10000.0, 1e-6, dtype)


@pytest.fixture
def make_store():
    made = []

    def mk(n_slots, max_tok=8, **kw):
        s = L.cb_store_create(_desc(**kw), max_tok, n_slots, False)
        made.append(s)
        return s
    yield mk
    for s in made:
        L.cb_store_destroy(s)


def test_sha256_fips_examples():
    with open(GOLD) as f:
        for v in json.load(f)["vectors"]:
            msg = v["message_ascii"].encode() * v["repeat"]
            assert L.cb_sha256(msg).hex() == v["digest"]


def test_sha256_block_boundaries_match_hashlib():
    import hashlib
    rng = np.random.default_rng(1)
    for n in list(range(0, 130)) + [191, 192, 193, 1000, 4095, 4096, 4097]:
        m = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert L.cb_sha256(m) == hashlib.sha256(m).digest(), n


def test_chunk_keys_match_oracle():
    rng = np.random.default_rng(2)
    for n in [0, 1, 2, 15, 16, 17, 63, 64, 65, 128, 512, 2048]:
        for n_prior in (0, 1, 3):
            t = rng.integers(-2**31, 2**31 - 1, n)
            p = rng.integers(0, 2**63, n_prior, dtype=np.uint64) * 2 + 1
            assert L.cb_chunk_key(t, p) == S.chunk_key(t.tolist(), [int(x) for x in p]), (n, n_prior)
    # prefix keys: content keys of every earlier chunk as prior
    chunks = [rng.integers(0, 150000, 128).tolist() for _ in range(4)]
    content = [L.cb_chunk_key(c) for c in chunks]
    lib = [L.cb_chunk_key(c, content[:i]) for i, c in enumerate(chunks)]
    assert lib == S.prefix_keys(chunks)


class _Mirror:
    """Drives the library store and the oracle store with the same operations."""

    def __init__(self, lib, cap):
        self.lib, self.ora = lib, S.ChunkStore(cap)
        self.slot_of = {}   # oracle identity -> library slot

    def lookup(self, t, p, pin):
        slot = L.cb_store_lookup(self.lib, t, p, pin)
        hit = self.ora.lookup(t, p, pin)
        assert (slot >= 0) == hit
        if hit:
            assert self.slot_of[S.ChunkStore.ident(t, p)] == slot
        return slot

    def insert(self, t, p, pin):
        try:
            victim = self.ora.insert(t, p)
            full = False
        except S.StoreFull:
            full = True
        if full:
            with pytest.raises(L.CbError) as e:
                L.cb_store_insert(self.lib, t, p, pin)
            assert e.value.status == L.CB_ESTATE
            return None
        ident = S.ChunkStore.ident(t, p)
        if pin:
            self.ora.entries[ident] += 1
        slot, new, ev = L.cb_store_insert(self.lib, t, p, pin)
        if victim is None:
            assert ev == -1
        else:
            assert ev == self.slot_of.pop(victim)
        assert new == (ident not in self.slot_of)
        if new:
            self.slot_of[ident] = slot
            L.cb_store_commit(self.lib, slot)
        assert self.slot_of[ident] == slot
        return slot

    def release(self, t, p):
        ident = S.ChunkStore.ident(t, p)
        self.ora.release(t, p)
        L.cb_store_release(self.lib, self.slot_of[ident])


@pytest.mark.parametrize("cap,vocab,seed", [(1, 3, 0), (3, 6, 1), (8, 14, 2), (16, 40, 3), (32, 50, 4)])
def test_store_matches_oracle_on_random_operations(make_store, cap, vocab, seed):
    rng = np.random.default_rng(seed)
    m = _Mirror(make_store(cap), cap)
    held = []
    for _ in range(3000):
        n = int(rng.integers(1, 4))
        t = [int(x) for x in rng.integers(0, vocab, 1)] * n      # few distinct chunks: repeats
        p = [int(rng.integers(1, 3))] if rng.random() < 0.2 else []
        op = rng.random()
        if op < 0.45:
            pin = rng.random() < 0.1
            if m.lookup(t, p, pin) >= 0 and pin:
                held.append((t, p))
        elif op < 0.9:
            pin = rng.random() < 0.05
            if m.insert(t, p, pin) is not None and pin:
                held.append((t, p))
        elif held:
            m.release(*held.pop(int(rng.integers(0, len(held)))))
    st = L.cb_store_get_stats(m.lib)
    assert (st.hits, st.misses, st.evictions) == (m.ora.hits, m.ora.misses, m.ora.evictions)
    assert st.entries == len(m.ora)


def test_cyclic_scan_trap_through_the_library(make_store):
    # the LMCache page's LRU trap: 10 documents cycled through a 4-entry store never hit
    s = make_store(4)
    for _ in range(3):
        for d in range(10):
            if L.cb_store_lookup(s, [d]) < 0:
                slot, _, _ = L.cb_store_insert(s, [d])
                L.cb_store_commit(s, slot)
    st = L.cb_store_get_stats(s)
    assert st.hits == 0 and st.misses == 30 and st.evictions == 26


def test_index_is_16_bytes_per_bucket_at_most_80_percent_full(make_store):
    s = make_store(1_000_000, max_tok=1, n_layers=1, n_kv=1, head_dim=1)
    st = L.cb_store_get_stats(s)
    assert st.index_bytes == 16 * (1_000_000 + 250_000 + 1)
    assert st.index_bytes / 2**20 <= 20.0  # about 16 MB per million chunks on the explainer
    assert st.capacity == 1_000_000 and st.slot_bytes == 8


def test_churn_keeps_every_live_key_reachable(make_store):
    cap = 20000
    s = make_store(cap, max_tok=2, n_layers=1, n_kv=1, head_dim=1)
    for i in range(3 * cap):                   # 2*cap evictions through backward-shift deletes
        slot, new, ev = L.cb_store_insert(s, [i, i ^ 0x5A5A])
        assert new and (ev == -1) == (i < cap)
        L.cb_store_commit(s, slot)
    for i in range(2 * cap, 3 * cap):
        assert L.cb_store_lookup(s, [i, i ^ 0x5A5A]) >= 0
    for i in range(0, 2 * cap, 97):
        assert L.cb_store_lookup(s, [i, i ^ 0x5A5A]) == -1
    st = L.cb_store_get_stats(s)
    assert st.evictions == 2 * cap and st.entries == cap


def test_uncommitted_entries_miss_and_insert_reports_new(make_store):
    s = make_store(4)
    slot, new, ev = L.cb_store_insert(s, [7, 8, 9])
    assert new and ev == -1 and slot == 0
    assert L.cb_store_lookup(s, [7, 8, 9]) == -1
    assert L.cb_store_insert(s, [7, 8, 9]) == (slot, False, -1)
    L.cb_store_commit(s, slot)
    assert L.cb_store_lookup(s, [7, 8, 9]) == slot
    assert L.cb_store_lookup(s, [7, 8]) == -1 and L.cb_store_lookup(s, [7, 8, 9], prior=[1]) == -1


def test_arena_layout(make_store):
    n_layers, n_kv, hd, max_tok = 3, 2, 4, 8
    s = make_store(3, max_tok=max_tok, n_layers=n_layers, n_kv=n_kv, head_dim=hd)
    row = n_kv * hd * 4
    slots = [L.cb_store_insert(s, [10 + i] * (i + 1))[0] for i in range(3)]
    addr = {}
    n_slots = 3
    for sl in slots:
        for l in range(n_layers):
            k, v, n = L.cb_store_layer(s, sl, l)
            assert n == sl + 1 and v - k == n_slots * max_tok * row
            addr[(sl, l)] = (k, v)
    # layer-major: per layer the K rows of every slot back to back, then their V rows, so that
    # consecutive slots' entries of one layer are adjacent (one copy for a run of them)
    base = addr[(0, 0)][0]
    for (sl, l), (k, v) in addr.items():
        assert k - base == (l * 2 * n_slots + sl) * max_tok * row
        if sl + 1 < n_slots:
            assert addr[(sl + 1, l)][0] - k == max_tok * row and addr[(sl + 1, l)][1] - v == max_tok * row
    # bytes written through one entry's pointers stay where they were put
    for (sl, l), (k, v) in addr.items():
        ctypes.memmove(k, bytes([sl * 16 + l * 2]) * (max_tok * row), max_tok * row)
        ctypes.memmove(v, bytes([sl * 16 + l * 2 + 1]) * (max_tok * row), max_tok * row)
    for (sl, l), (k, v) in addr.items():
        assert ctypes.string_at(k, max_tok * row) == bytes([sl * 16 + l * 2]) * (max_tok * row)
        assert ctypes.string_at(v, max_tok * row) == bytes([sl * 16 + l * 2 + 1]) * (max_tok * row)
    st = L.cb_store_get_stats(s)
    assert st.slot_bytes == n_layers * 2 * max_tok * row and st.arena_bytes == 3 * st.slot_bytes


def test_bf16_row_bytes(make_store):
    s = make_store(2, max_tok=4, n_layers=1, n_kv=2, head_dim=128, dtype=L.CB_BF16)
    assert L.cb_store_get_stats(s).slot_bytes == 2 * 4 * 2 * 128 * 2


def test_errors(make_store):
    s = make_store(2, max_tok=4)
    for bad in ([], [1, 2, 3, 4, 5]):
        with pytest.raises(L.CbError) as e:
            L.cb_store_insert(s, bad)
        assert e.value.status == L.CB_ESHAPE
    slot, _, _ = L.cb_store_insert(s, [1])
    with pytest.raises(L.CbError) as e:
        L.cb_store_release(s, slot)
    assert e.value.status == L.CB_ESTATE
    for bad_slot in (-1, 1, 2):
        with pytest.raises(L.CbError) as e:
            L.cb_store_layer(s, bad_slot, 0)
        assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError) as e:
        L.cb_store_layer(s, slot, 2)
    assert e.value.status == L.CB_EINVAL
    with pytest.raises(L.CbError):
        L.cb_store_create(_desc(), 0, 4, False)
    with pytest.raises(L.CbError):
        L.cb_store_create(_desc(), 4, 0, False)


def test_concurrent_callers(make_store):
    cap = 64
    s = make_store(cap)
    n_threads, n_ops = 4, 4000
    counts = [0] * n_threads

    def worker(w):
        rng = np.random.default_rng(100 + w)
        for _ in range(n_ops):
            t = [int(rng.integers(0, 200))]
            if L.cb_store_lookup(s, t) < 0:
                slot, new, _ = L.cb_store_insert(s, t)
                if new:
                    L.cb_store_commit(s, slot)
            counts[w] += 1

    th = [threading.Thread(target=worker, args=(w,)) for w in range(n_threads)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    st = L.cb_store_get_stats(s)
    assert st.hits + st.misses == sum(counts) == n_threads * n_ops
    assert st.entries == cap
    live = [d for d in range(200) if L.cb_store_lookup(s, [d]) >= 0]
    assert len(live) == cap
