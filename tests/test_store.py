"""The pair store (hypic_store_*), host only: slot assignment and eviction
against a plain Python model of the stated policy on random traces, the
capacity refusal that changes nothing, eviction by key, and the content key
against the published FNV-1a 64 test vectors."""
import numpy as np
import pytest

import state_caching_segment_amd as hy


class Model:
    """The stated policy, written out plainly: hits keep their slot; a miss
    takes a free slot (lowest first, then most recently freed first), else
    evicts the entry acquired least often, ties by least recent acquisition,
    never one named earlier in the same call."""

    def __init__(self, n):
        self.n = n
        self.free = list(range(n - 1, -1, -1))   # stack: next at the end
        self.key_at = {}                          # slot -> key
        self.slot_of = {}                         # key -> slot
        self.freq, self.last = {}, {}
        self.tick = 0
        self.stats = dict(entries=0, hits=0, misses=0, evictions=0)

    def acquire(self, keys):
        if len(set(keys)) > self.n:
            return None
        named, slots, miss = set(), [None] * len(keys), [False] * len(keys)
        for i, k in enumerate(keys):              # hits first
            if k in self.slot_of:
                s = self.slot_of[k]
                if s not in named:
                    self.stats["hits"] += 1
                named.add(s)
                self.freq[s] += 1
                self.tick += 1
                self.last[s] = self.tick
                slots[i] = s
        for i, k in enumerate(keys):
            if slots[i] is not None:
                continue
            if k in self.slot_of:                 # repeat of a key that missed in this call
                s = self.slot_of[k]
                self.freq[s] += 1
                self.tick += 1
                self.last[s] = self.tick
                slots[i] = s
                continue
            if self.free:
                s = self.free.pop()
            else:
                cands = [s for s in self.key_at if s not in named]
                s = min(cands, key=lambda s: (self.freq[s], self.last[s], s))
                del self.slot_of[self.key_at[s]]
                self.stats["evictions"] += 1
            self.key_at[s] = k
            self.slot_of[k] = s
            self.freq[s] = 1
            self.tick += 1
            self.last[s] = self.tick
            named.add(s)
            slots[i], miss[i] = s, True
            self.stats["misses"] += 1
        self.stats["entries"] = len(self.slot_of)
        return slots, miss

    def evict(self, k):
        if k not in self.slot_of:
            return False
        s = self.slot_of.pop(k)
        del self.key_at[s], self.freq[s], self.last[s]
        self.free.append(s)
        self.stats["entries"] = len(self.slot_of)
        return True


@pytest.mark.parametrize("seed", range(6))
def test_store_follows_the_policy(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    st, m = hy.Store(n), Model(n)
    for _ in range(300):
        if rng.random() < 0.1:
            k = int(rng.integers(0, 15))
            assert st.evict(k) == m.evict(k)
            continue
        keys = rng.integers(0, 15, int(rng.integers(1, 5))).tolist()
        ref = m.acquire(keys)
        if ref is None:
            before = st.stats()
            with pytest.raises(hy.HypicError) as e:
                st.acquire(keys)
            assert e.value.status == -3 and st.stats() == before   # refused: nothing changed
            continue
        slots, miss = st.acquire(keys)
        assert slots.tolist() == ref[0] and miss.tolist() == ref[1], (keys, slots, miss, ref)
        assert st.stats() == m.stats
        assert len(set(slots.tolist())) == len(set(keys))           # distinct keys, distinct slots


def test_store_evicts_least_used_first():
    st = hy.Store(3)
    st.acquire([1, 2, 3])
    st.acquire([1, 1, 2])          # 1 used three times, 2 twice, 3 once
    slots, miss = st.acquire([4])  # 3 goes
    assert miss.tolist() == [True] and st.acquire([1, 2])[1].tolist() == [False, False]
    _, miss3 = st.acquire([3])
    assert miss3.tolist() == [True]
    assert st.stats()["evictions"] == 2


def test_store_arguments():
    with pytest.raises(hy.HypicError):
        hy.Store(0)
    st = hy.Store(2)
    assert st.acquire([])[0].size == 0
    with pytest.raises(hy.HypicError):
        st.acquire([1, 2, 3])
    assert st.stats()["entries"] == 0
    assert st.evict(99) is False


def test_content_key_fnv1a_test_vectors():
    # published FNV-1a 64-bit test vectors (Fowler, Noll, Vo)
    assert hy.hypic_content_key(b"") == 0xCBF29CE484222325
    assert hy.hypic_content_key(b"a") == 0xAF63DC4C8601EC8C
    assert hy.hypic_content_key(b"foobar") == 0x85944171F73967E8
    ids = np.arange(512, dtype=np.int32)
    assert hy.hypic_content_key(ids) == hy.hypic_content_key(ids.tobytes())
    assert hy.hypic_content_key(ids) != hy.hypic_content_key(ids[::-1].copy())
