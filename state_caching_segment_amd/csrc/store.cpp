// Pair store: the host-side index of a pool of cached pairs (HYPIC,
// codernav.top article, section on segment parallelism: segments are probed
// for cache hits, misses are inevitable because the corpus changes and
// rarely used documents are evicted; section "summary": multi-level caching
// of the pairs as future work).
//
// The pool itself is device memory the caller owns: slots 0 .. n_slots-1 of
// the T and S arrays hypic_segment_build writes and hypic_compose reads.  The
// store maps a segment's content key to its slot and decides which slot a
// miss takes: a free one, else the entry used least often (ties: least
// recently), never one named earlier in the same call.  It allocates host
// memory only.
#include <cstdint>
#include <cstring>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/hypic.h"

struct hypic_store {
    struct Slot {
        uint64_t key = 0;
        uint64_t freq = 0;   // acquisitions since it was filled
        uint64_t last = 0;   // tick of the last acquisition
        uint64_t pin = 0;    // call that last named it
        bool used = false;
    };
    std::vector<Slot> slots;
    std::unordered_map<uint64_t, int32_t> index;
    std::set<std::tuple<uint64_t, uint64_t, int32_t>> order;  // (freq, last, slot) of used slots
    std::vector<int32_t> free_list;                            // free slots, lowest index at the back
    uint64_t tick = 0, call = 0;
    int64_t hits = 0, misses = 0, evictions = 0;

    void touch(int32_t s) {
        Slot &e = slots[s];
        order.erase({e.freq, e.last, s});
        e.freq += 1;
        e.last = ++tick;
        e.pin = call;
        order.insert({e.freq, e.last, s});
    }
};

extern "C" {

hypic_store *hypic_store_create(int64_t n_slots) {
    if (n_slots < 1 || n_slots > 0x7fffffff) return nullptr;
    hypic_store *st = new (std::nothrow) hypic_store;
    if (!st) return nullptr;
    try {
        st->slots.resize((size_t)n_slots);
        st->free_list.reserve((size_t)n_slots);
        for (int64_t s = n_slots - 1; s >= 0; --s) st->free_list.push_back((int32_t)s);
        st->index.reserve((size_t)n_slots);
    } catch (...) {
        delete st;
        return nullptr;
    }
    return st;
}

void hypic_store_destroy(hypic_store *st) { delete st; }

int hypic_store_acquire(hypic_store *st, int32_t n, const uint64_t *keys, int32_t *slots_out, uint8_t *miss_out) {
    if (!st || n < 0) return HYPIC_E_INVALID;
    if (n == 0) return 0;
    if (!keys || !slots_out || !miss_out) return HYPIC_E_INVALID;
    // capacity first, so that a refused call changes nothing: the distinct
    // keys named here must fit in the pool together
    {
        std::unordered_map<uint64_t, char> seen;
        seen.reserve((size_t)n * 2);
        for (int32_t i = 0; i < n; ++i) seen.emplace(keys[i], 0);
        if ((int64_t)seen.size() > (int64_t)st->slots.size()) return HYPIC_E_WORKSPACE;
    }
    ++st->call;
    // hits first, so that they are pinned before any miss picks a victim
    for (int32_t i = 0; i < n; ++i) {
        auto it = st->index.find(keys[i]);
        miss_out[i] = 0;
        slots_out[i] = -1;
        if (it != st->index.end()) {
            slots_out[i] = it->second;
            if (st->slots[it->second].pin != st->call) ++st->hits;
            st->touch(it->second);
        }
    }
    int missed = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (slots_out[i] >= 0) continue;
        auto it = st->index.find(keys[i]);
        if (it != st->index.end()) {  // a repeat of a key that missed earlier in this call
            slots_out[i] = it->second;
            st->touch(it->second);
            continue;
        }
        int32_t s;
        if (!st->free_list.empty()) {
            s = st->free_list.back();
            st->free_list.pop_back();
        } else {
            // least used, least recent, not named in this call (one exists:
            // the distinct keys of this call fit in the pool)
            auto v = st->order.begin();
            while (st->slots[std::get<2>(*v)].pin == st->call) ++v;
            s = std::get<2>(*v);
            st->order.erase(v);
            st->index.erase(st->slots[s].key);
            ++st->evictions;
        }
        hypic_store::Slot &e = st->slots[s];
        e.key = keys[i];
        e.used = true;
        e.freq = 1;
        e.last = ++st->tick;
        e.pin = st->call;
        st->order.insert({e.freq, e.last, s});
        st->index[keys[i]] = s;
        slots_out[i] = s;
        miss_out[i] = 1;
        ++st->misses;
        ++missed;
    }
    return missed;
}

int hypic_store_evict(hypic_store *st, uint64_t key) {
    if (!st) return HYPIC_E_INVALID;
    auto it = st->index.find(key);
    if (it == st->index.end()) return 0;
    const int32_t s = it->second;
    hypic_store::Slot &e = st->slots[s];
    st->order.erase({e.freq, e.last, s});
    e = hypic_store::Slot{};
    st->index.erase(it);
    st->free_list.push_back(s);
    return 1;
}

int hypic_store_stats(const hypic_store *st, int64_t *out) {
    if (!st || !out) return HYPIC_E_INVALID;
    out[0] = (int64_t)st->index.size();
    out[1] = st->hits;
    out[2] = st->misses;
    out[3] = st->evictions;
    return HYPIC_OK;
}

uint64_t hypic_content_key(const void *data, size_t nbytes) {
    // FNV-1a, 64 bits
    const unsigned char *p = static_cast<const unsigned char *>(data);
    uint64_t h = 14695981039346656037ull;
    for (size_t i = 0; i < nbytes; ++i) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

}  // extern "C"
