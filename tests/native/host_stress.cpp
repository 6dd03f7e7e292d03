// Host-side stress of the library's host objects (block pool with swap space, prefix
// cache, cascade / extend planner) through the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  Seeded random
// operations, invalid arguments included; light consistency checks on the way.  Any
// memory error or undefined behaviour aborts the run.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkv.h"

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(2);                                               \
    }                                                             \
  } while (0)

static void stress_pool_and_cache(uint32_t seed) {
  std::mt19937 rng(seed);
  const int32_t bs = 1 + rng() % 8, nblk = 24 + rng() % 40, nhost = 16;
  pkv_pool* pool = pkv_pool_create(nblk, bs, nullptr);
  CHECK(pool);
  CHECK(pkv_pool_set_host_slots(pool, nhost, nullptr) == PKV_OK);
  CHECK(pkv_pool_set_host_slots(pool, nhost, nullptr) != PKV_OK);
  pkv_radix* cache = pkv_radix_create(pool, static_cast<int32_t>(rng() % 2));
  CHECK(cache);
  std::vector<int64_t> live;
  std::vector<std::vector<int32_t>> toks;  // per sequence id (index = id)
  std::vector<int64_t> locked;
  std::vector<int32_t> buf(4096), buf2(4096);
  std::vector<int64_t> ids(4096);
  for (int step = 0; step < 3000; ++step) {
    const int op = rng() % 12;
    if (op == 0 || live.empty()) {  // arrival through the cache
      std::vector<int32_t> t(1 + rng() % (6 * bs));
      for (auto& x : t) x = rng() % 3;
      if (!toks.empty() && rng() % 2) {
        const auto& src = toks[rng() % toks.size()];
        for (size_t i = 0; i < t.size() && i < src.size() && rng() % 4; ++i) t[i] = src[i];
      }
      int32_t m = 0;
      int64_t node = 0;
      CHECK(pkv_radix_match(cache, t.data(), static_cast<int32_t>(t.size()) - 1, &m, buf.data(),
                            static_cast<int32_t>(buf.size()), &node) == PKV_OK);
      CHECK(m % bs == 0 && m <= static_cast<int32_t>(t.size()));
      CHECK(pkv_radix_lock(cache, node) == PKV_OK);
      const int64_t seq = static_cast<int64_t>(toks.size());
      pkv_status st = pkv_seq_alloc_prefix(pool, seq, buf.data(), m / bs, static_cast<int32_t>(t.size()));
      if (st == PKV_ERR_OOM) {
        int32_t rel = 0, ne = 0;
        CHECK(pkv_radix_evict(cache, nblk, &rel, ids.data(), static_cast<int32_t>(ids.size()), &ne) == PKV_OK);
        // the match may have been evicted with the lock still held: it was not (locked nodes stay)
        st = pkv_seq_alloc_prefix(pool, seq, buf.data(), m / bs, static_cast<int32_t>(t.size()));
      }
      toks.push_back(t);
      if (st == PKV_OK) {
        live.push_back(seq);
        locked.push_back(node);
      } else {
        CHECK(pkv_radix_unlock(cache, node) == PKV_OK);
        locked.push_back(-1);
      }
    } else if (op == 1) {  // finish: cache, unlock, free
      const size_t k = rng() % live.size();
      const int64_t seq = live[k];
      if (pkv_seq_is_swapped(pool, seq) == 1) CHECK(pkv_seq_swap_in(pool, seq, buf.data(), buf2.data(), 4096, &buf[4000]) != PKV_ERR_INVALID || true);
      if (pkv_seq_is_swapped(pool, seq) == 0) {
        const int32_t n = pkv_seq_table(pool, seq, buf.data(), static_cast<int32_t>(buf.size()));
        CHECK(n >= 0);
        int64_t nn = 0;
        int32_t ad = 0;
        const auto& t = toks[seq];
        const int32_t len = pkv_seq_len(pool, seq);
        const int32_t nt = std::min<int32_t>(len, static_cast<int32_t>(t.size()));
        CHECK(pkv_radix_insert(cache, t.data(), nt, buf.data(), n, (rng() % 8) / 4.0, rng() % 4, &nn, &ad) == PKV_OK);
      }
      CHECK(pkv_radix_unlock(cache, locked[seq]) == PKV_OK);
      CHECK(pkv_seq_free(pool, seq) == PKV_OK);
      live.erase(live.begin() + k);
    } else if (op == 2) {  // append a token to a few live sequences
      std::vector<int64_t> b;
      for (int64_t s : live)
        if (pkv_seq_is_swapped(pool, s) == 0 && rng() % 2) b.push_back(s);
      int32_t ncow = 0;
      std::vector<int64_t> slots(b.size() + 1);
      std::vector<int32_t> cs(b.size() + 1), cd(b.size() + 1), cr(b.size() + 1), rs(b.size() + 1);
      pkv_status st = pkv_plan_append(pool, b.data(), static_cast<int32_t>(b.size()), slots.data(), cs.data(),
                                      cd.data(), cr.data(), &ncow, rng() % 2 ? rs.data() : nullptr);
      CHECK(st == PKV_OK || st == PKV_ERR_OOM);
      if (st == PKV_OK)
        for (int64_t s : b) toks[s].push_back(rng() % 3);
    } else if (op == 3) {
      int32_t rel = 0, ne = 0;
      CHECK(pkv_radix_evict(cache, rng() % 6, &rel, ids.data(), static_cast<int32_t>(rng() % 3), &ne) == PKV_OK);
    } else if (op == 4) {  // swap out / in
      const int64_t seq = live[rng() % live.size()];
      int32_t n = 0;
      if (pkv_seq_is_swapped(pool, seq) == 1)
        (void)pkv_seq_swap_in(pool, seq, buf.data(), buf2.data(), 4096, &n);
      else
        (void)pkv_seq_swap_out(pool, seq, buf.data(), buf2.data(), 4096, &n);
    } else if (op == 5) {  // fork
      const int64_t parent = live[rng() % live.size()];
      const int64_t child = static_cast<int64_t>(toks.size());
      if (pkv_seq_fork(pool, parent, child) == PKV_OK) {
        toks.push_back(toks[parent]);
        live.push_back(child);
        locked.push_back(0);  // the root: lock and unlock are no-ops
        CHECK(pkv_radix_lock(cache, 0) == PKV_OK);
      } else {
        toks.push_back({});
        locked.push_back(-1);
      }
    } else if (op == 6) {  // score updates and node inspection
      const int32_t nn = pkv_radix_node_ids(cache, ids.data(), static_cast<int32_t>(ids.size()));
      CHECK(nn >= 1);
      const int64_t node = ids[rng() % std::min<int32_t>(nn, static_cast<int32_t>(ids.size()))];
      if (node != 0) CHECK(pkv_radix_set_score(cache, node, (rng() % 9) / 8.0) == PKV_OK);
      int64_t parent = 0, last = 0;
      int32_t lock = 0, depth = 0, nb = 0;
      double score = 0;
      CHECK(pkv_radix_node_info(cache, node, &parent, &lock, &last, &score, &depth, &nb, buf.data(),
                                static_cast<int32_t>(buf.size()), buf2.data(), static_cast<int32_t>(buf2.size())) ==
            PKV_OK);
    } else if (op == 7) {  // invalid arguments: errors, no state change
      CHECK(pkv_radix_unlock(cache, 1 << 30) == PKV_ERR_NOT_FOUND);
      CHECK(pkv_radix_insert(cache, nullptr, 5, nullptr, 0, 0.0, 0, nullptr, nullptr) == PKV_ERR_INVALID);
      CHECK(pkv_seq_alloc_prefix(pool, 1 << 30, buf.data(), -1, 4) == PKV_ERR_INVALID);
      CHECK(pkv_copy_blocks_memcpy(0, nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr, 0, nullptr) == PKV_ERR_INVALID);
    } else if (op == 8) {  // batched admission and completion
      std::vector<int32_t> flat;
      std::vector<int64_t> off{0}, seqs;
      for (int r = 0; r < 3; ++r) {
        const int n = 1 + rng() % (3 * bs);
        for (int i = 0; i < n; ++i) flat.push_back(rng() % 3);
        off.push_back(static_cast<int64_t>(flat.size()));
        seqs.push_back(static_cast<int64_t>(toks.size()) + r);
      }
      std::vector<int32_t> matched(3);
      std::vector<int64_t> nodes(3);
      int32_t na = 0;
      CHECK(pkv_radix_admit(cache, flat.data(), off.data(), 3, seqs.data(), matched.data(), nodes.data(), &na) ==
            PKV_OK);
      for (int r = 0; r < 3; ++r) toks.emplace_back(flat.begin() + off[r], flat.begin() + off[r + 1]);
      for (int r = 0; r < 3; ++r) locked.push_back(r < na ? nodes[r] : -1);
      if (na > 0) CHECK(pkv_radix_finish(cache, flat.data(), off.data(), na, seqs.data(), nodes.data(), nullptr,
                                         nullptr) == PKV_OK);
    } else {
      int32_t nf = pkv_free_list(pool, buf.data(), static_cast<int32_t>(buf.size()));
      CHECK(nf >= 0 && pkv_free_count(pool) == nf);
      CHECK(pkv_radix_cached_blocks(cache) >= 0 && pkv_radix_evictable_blocks(cache) >= 0);
    }
  }
  CHECK(pkv_radix_clear(cache) == PKV_OK);
  for (int64_t s : live) {
    if (locked[s] > 0) (void)pkv_radix_unlock(cache, locked[s]);  // nodes are gone after clear
    CHECK(pkv_seq_free(pool, s) == PKV_OK);
  }
  CHECK(pkv_free_count(pool) == nblk && pkv_host_free_count(pool) == nhost);
  pkv_radix_destroy(cache);
  pkv_pool_destroy(pool);
}

static void stress_planner(uint32_t seed) {
  std::mt19937 rng(seed);
  for (int rep = 0; rep < 40; ++rep) {
    const int32_t B = 1 + rng() % 20, maxb = 1 + rng() % 40, nblk = 200;
    const int32_t hkv = 1 << (rng() % 3), g = 1 << (rng() % 4), hq = hkv * g;
    std::vector<int32_t> bt(static_cast<size_t>(B) * maxb, -1), lens(B), qlen(B);
    for (int32_t b = 0; b < B; ++b) {
      lens[b] = rng() % (maxb * 16 + 1);
      const int32_t share = b > 0 && rng() % 2 ? static_cast<int32_t>(rng() % (b + 1)) : -1;
      for (int32_t j = 0; j < (lens[b] + 15) / 16; ++j)
        bt[static_cast<size_t>(b) * maxb + j] =
            share >= 0 && j < 3 && bt[static_cast<size_t>(share) * maxb + j] >= 0 ? bt[static_cast<size_t>(share) * maxb + j]
                                                                                  : static_cast<int32_t>(rng() % nblk);
      qlen[b] = lens[b] > 0 ? 1 + static_cast<int32_t>(rng() % std::min(lens[b], 40)) : 0;
    }
    pkv_plan* p = pkv_plan_build(bt.data(), lens.data(), B, maxb, 16, hq, hkv, 2);
    if (p) {
      const int64_t n = pkv_plan_image(p, nullptr, 0, nullptr);
      std::vector<int32_t> img(static_cast<size_t>(n > 0 ? n : 1));
      std::vector<int64_t> offs(6);
      CHECK(pkv_plan_image(p, img.data(), n, offs.data()) == n);
      pkv_plan_destroy(p);
    }
    pkv_plan* e = pkv_plan_build_extend(bt.data(), lens.data(), qlen.data(), B, maxb, 16, hq, hkv, 2);
    if (e) {
      CHECK(pkv_plan_rows_per_item(e) == 128);
      pkv_plan_destroy(e);
    }
  }
  CHECK(pkv_plan_build(nullptr, nullptr, 1, 1, 16, 4, 4, 2) == nullptr);
}

int main() {
  for (uint32_t seed = 0; seed < 12; ++seed) stress_pool_and_cache(seed);
  for (uint32_t seed = 0; seed < 6; ++seed) stress_planner(seed);
  std::printf("host stress ok\n");
  return 0;
}
