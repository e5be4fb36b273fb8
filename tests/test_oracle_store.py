"""Pins of the chunk store oracle (oracle/store.py) to things other than itself: the SHA-256
examples of FIPS 180-2, hand-built messages whose bytes equal those examples (which fixes the
token and key encodings and their order), the LRU trap that the LMCache page measures, the
stack (inclusion) property of LRU, and a hand-worked eviction sequence."""
import json
import os

import numpy as np
import pytest

from oracle import store as S

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sha256_vectors.json")
MSG448 = b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq"


def _vectors():
    with open(GOLD) as f:
        return json.load(f)["vectors"]


def _tokens_le(b: bytes):
    """int32 tokens whose little-endian bytes are b (len(b) % 4 == 0)."""
    return np.frombuffer(b, dtype="<i4").astype(np.int64).tolist()


@pytest.mark.parametrize("v", _vectors(), ids=lambda v: f"{v['message_ascii'][:8]}x{v['repeat']}")
def test_sha256_fips_examples(v):
    import hashlib
    msg = v["message_ascii"].encode() * v["repeat"]
    assert hashlib.sha256(msg).hexdigest() == v["digest"]


def test_content_key_encoding_matches_fips_example():
    # 56 bytes = 14 tokens; the key is the first 8 digest bytes, big-endian
    toks = _tokens_le(MSG448)
    assert len(toks) == 14
    assert S.content_key(toks) == 0x248D6A61D20638B8
    assert S.key_message(toks) == MSG448


def test_empty_chunk_key():
    assert S.content_key([]) == 0xE3B0C44298FC1C14


def test_prior_keys_come_first_big_endian():
    prior = [int.from_bytes(MSG448[:8], "big")]
    toks = _tokens_le(MSG448[8:])
    assert S.chunk_key(toks, prior) == 0x248D6A61D20638B8
    two = [int.from_bytes(MSG448[:8], "big"), int.from_bytes(MSG448[8:16], "big")]
    assert S.chunk_key(_tokens_le(MSG448[16:]), two) == 0x248D6A61D20638B8


def test_negative_token_ids_are_twos_complement():
    # 'abcd' little-endian is 0x64636261; the byte pattern of -1 is ff ff ff ff
    assert S.key_message([-1]) == b"\xff\xff\xff\xff"
    assert S.key_message([0x64636261]) == b"abcd"


def test_content_key_is_position_free_prefix_key_is_not():
    rng = np.random.default_rng(7)
    a, b, c = (rng.integers(0, 150000, 128).tolist() for _ in range(3))
    p1 = S.prefix_keys([a, b, c])
    p2 = S.prefix_keys([b, a, c])
    assert S.content_key(c) == S.content_key(c)
    assert p1[2] != p2[2]                     # same chunk, other context
    assert p1[0] == S.content_key(a)          # nothing before the first chunk
    assert S.prefix_keys([a, b])[1] == p1[1]  # later chunks do not change earlier keys


def _scan(store, docs, passes):
    """Read every document in order, `passes` times, inserting on a miss; hits per pass."""
    out = []
    for _ in range(passes):
        h = 0
        for d in docs:
            if store.lookup(d):
                h += 1
            else:
                store.insert(d)
        out.append(h)
    return out


def test_cyclic_scan_over_a_larger_working_set_never_hits():
    # LMCache page, section 1: 10 documents of about 5,000 tokens against a 21,520-token KV
    # capacity, read twice in the same order: the second pass gets no hit under LRU.
    cap = 21520 // 5000
    docs = [[d] * 5 for d in range(10)]
    assert _scan(S.ChunkStore(cap), docs, 3) == [0, 0, 0]
    # one entry short of the working set is already enough to lose every hit
    assert _scan(S.ChunkStore(9), docs, 3) == [0, 0, 0]
    assert _scan(S.ChunkStore(10), docs, 3) == [0, 10, 10]


def test_lru_is_a_stack_algorithm():
    # LRU's inclusion property: on the same trace a larger store never hits less.
    rng = np.random.default_rng(3)
    p = 1.0 / np.arange(1, 61) ** 1.1            # Zipf-like popularity over 60 documents
    trace = rng.choice(60, size=3000, p=p / p.sum())
    hits = []
    for cap in range(1, 61):
        st = S.ChunkStore(cap)
        for d in trace:
            if not st.lookup([int(d)]):
                st.insert([int(d)])
        hits.append(st.hits)
    assert all(h0 <= h1 for h0, h1 in zip(hits, hits[1:]))
    assert hits[4] > 0                            # a small store still helps under skew
    assert hits[-1] == len(trace) - len(set(trace.tolist()))  # only first reads miss


def test_hand_worked_eviction_sequence():
    st = S.ChunkStore(2)
    assert st.insert([1]) is None and st.insert([2]) is None
    assert st.lookup([1])                          # 1 becomes most recent
    assert st.insert([3]) == ((2,), ())            # so 2 is the victim
    assert not st.lookup([2]) and st.lookup([1]) and st.lookup([3])
    assert st.insert([3]) is None and len(st) == 2  # already there: refresh only
    assert st.insert([4]) == ((1,), ())            # 3 was refreshed after 1
    assert (st.hits, st.misses, st.evictions) == (3, 1, 2)


def test_held_entries_are_not_evicted():
    st = S.ChunkStore(2)
    st.insert([1]), st.insert([2])
    assert st.lookup([1], pin=True)
    assert st.insert([3]) == ((2,), ())            # 1 is older but held
    assert st.lookup([3], pin=True)
    with pytest.raises(S.StoreFull):
        st.insert([4])
    st.release([1])
    assert st.insert([4]) == ((1,), ())


def test_prior_keys_are_part_of_the_identity():
    st = S.ChunkStore(4)
    st.insert([5, 6], prior=[11])
    assert not st.lookup([5, 6]) and not st.lookup([5, 6], prior=[12])
    assert st.lookup([5, 6], prior=[11])
