// Host sanitizer driver for the pair store (test infrastructure): random
// acquire / evict traces under AddressSanitizer and UndefinedBehaviorSanitizer,
// checking after every call that distinct keys hold distinct slots, that a
// key's slot is stable while it stays, and that the counters add up.
#include <cstdint>
#include <cstdio>
#include <map>
#include <set>
#include <vector>

#include "../../include/hypic.h"

#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main() {
    uint64_t st = 0x9E3779B97F4A7C15ull;
    auto rnd = [&](uint64_t m) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st % m; };
    for (int n_slots = 1; n_slots <= 9; n_slots += 4) {
        hypic_store *s = hypic_store_create(n_slots);
        CHECK(s != nullptr);
        std::map<uint64_t, int32_t> held;  // key -> slot, as the store reported it
        int64_t calls_hits = 0, calls_misses = 0;
        for (int it = 0; it < 2000; ++it) {
            if (rnd(10) == 0) {
                uint64_t key = rnd(24);
                const int r = hypic_store_evict(s, key);
                CHECK(r == (held.count(key) ? 1 : 0));
                held.erase(key);
                continue;
            }
            const int n = (int)rnd(5);
            std::vector<uint64_t> keys(n);
            for (auto &k : keys) k = rnd(24);
            std::vector<int32_t> slots(n > 0 ? n : 1);
            std::vector<uint8_t> miss(n > 0 ? n : 1);
            const int r = hypic_store_acquire(s, n, keys.data(), slots.data(), miss.data());
            std::set<uint64_t> distinct(keys.begin(), keys.end());
            if ((int)distinct.size() > n_slots) {
                CHECK(r == HYPIC_E_WORKSPACE);
                continue;
            }
            CHECK(r >= 0);
            std::map<uint64_t, int32_t> now;
            for (int i = 0; i < n; ++i) {
                CHECK(slots[i] >= 0 && slots[i] < n_slots);
                if (now.count(keys[i])) CHECK(now[keys[i]] == slots[i]);
                now[keys[i]] = slots[i];
                if (!miss[i] && held.count(keys[i])) CHECK(held[keys[i]] == slots[i]);
            }
            std::set<int32_t> used;
            for (auto &kv : now) CHECK(used.insert(kv.second).second);
            // keys evicted to make room are gone from the host model too
            for (auto itk = held.begin(); itk != held.end();) {
                bool taken = false;
                for (auto &kv : now)
                    if (kv.second == itk->second && kv.first != itk->first) taken = true;
                if (taken) itk = held.erase(itk); else ++itk;
            }
            for (auto &kv : now) held[kv.first] = kv.second;
            int misses = 0;
            for (int i = 0; i < n; ++i) misses += miss[i];
            CHECK(r == misses);
            calls_misses += misses;
        }
        int64_t stats[4];
        CHECK(hypic_store_stats(s, stats) == HYPIC_OK);
        CHECK(stats[0] == (int64_t)held.size() && stats[2] == calls_misses);
        (void)calls_hits;
        hypic_store_destroy(s);
    }
    CHECK(hypic_store_create(0) == nullptr);
    CHECK(hypic_content_key("", 0) == 0xCBF29CE484222325ull);
    std::printf("store sanitizer driver: ok\n");
    return 0;
}
