// Host fuzz of the block manager, built with AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py.  Random new / fork / append / free
// sequences on pools of one-block and multi-block pages; after every step
// each live sequence must read back exactly its own token history through
// its table, from a simulated pool that receives the copy-on-write block
// copies and the appends the way a caller would issue them, and the pool
// accounting must add up.  Exit status 0 = every check held.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pagedattn.h"
#include "pagedattn_blocks.h"

#define CHECK(c)                                                               \
  do {                                                                         \
    if (!(c)) {                                                                \
      std::fprintf(stderr, "check failed %s:%d: %s (pool %d step %d)\n", __FILE__, __LINE__, #c, pool_id, step); \
      std::exit(1);                                                            \
    }                                                                          \
  } while (0)

static int pool_id = 0, step = 0;

int main(int argc, char** argv) {
  const int pools = argc > 1 ? std::atoi(argv[1]) : 200;
  const int steps = argc > 2 ? std::atoi(argv[2]) : 300;
  long long checked = 0, appends = 0, exhausted = 0, forks = 0, copies = 0, frees = 0;
  for (pool_id = 0; pool_id < pools; ++pool_id) {
    std::mt19937_64 rng(1000 + pool_id);
    auto pick = [&](long long n) { return (long long)(rng() % (unsigned long long)n); };
    const int bs = 16 << pick(3);                           // 16, 32, 64
    const int max_page = 1 << pick(5);                      // 1..16 blocks
    const int64_t NB = max_page * (2 + pick(40)) + pick(7); // not always a multiple of the page
    pa_block_manager* bm = nullptr;
    CHECK(pa_bm_create_paged(NB, bs, max_page, &bm) == PA_OK && bm);
    std::vector<int64_t> pool((size_t)NB * bs, -1);  // token id held by each slot
    std::map<int32_t, std::vector<int64_t>> hist;    // live sequence -> token ids by position
    int64_t next_token = 0;
    std::vector<int32_t> slots, src, dst;
    for (step = 0; step < steps; ++step) {
      const int op = (int)pick(10);
      if (hist.empty() || op == 0) {
        int32_t s = -1;
        const int lo = 1 << pick(5), hi = 1 << pick(5);
        const int mn = std::min(std::min(lo, hi), max_page), mx = std::min(std::max(lo, hi), max_page);
        CHECK(pa_bm_new_sequence_paged(bm, mn, mx, &s) == PA_OK && s >= 0);
        CHECK(hist.count(s) == 0);
        hist[s] = {};
      } else {
        auto it = hist.begin();
        std::advance(it, pick((long long)hist.size()));
        const int32_t s = it->first;
        if (op <= 2) {
          int32_t c = -1;
          CHECK(pa_bm_fork(bm, s, &c) == PA_OK && c >= 0 && hist.count(c) == 0);
          ++forks;
          hist[c] = it->second;
        } else if (op == 3) {
          CHECK(pa_bm_free_sequence(bm, s) == PA_OK);
          hist.erase(it);
          CHECK(pa_bm_free_sequence(bm, s) == PA_ERR_SEQ);
          ++frees;
        } else {
          const int ntok = 1 + (int)pick(op == 9 ? 700 : 40);
          slots.assign((size_t)ntok, -7);
          src.assign((size_t)max_page, -7);
          dst.assign((size_t)max_page, -7);
          int32_t ncopy = -1;
          int64_t free0, used0, waste0;
          CHECK(pa_bm_stats(bm, &free0, &used0, &waste0) == PA_OK);
          const int st = pa_bm_append(bm, s, ntok, slots.data(), src.data(), dst.data(), max_page, &ncopy);
          if (st == PA_ERR_NO_BLOCKS) {
            int64_t f, u, w;
            CHECK(pa_bm_stats(bm, &f, &u, &w) == PA_OK && f == free0 && u == used0 && w == waste0);
            ++exhausted;
          } else {
            CHECK(st == PA_OK && ncopy >= 0 && ncopy <= max_page);
            ++appends;
            copies += ncopy;
            for (int i = 0; i < ncopy; ++i) {  // kv_copy_blocks, then kv_append
              CHECK(src[i] >= 0 && src[i] < NB && dst[i] >= 0 && dst[i] < NB && src[i] != dst[i]);
              for (int o = 0; o < bs; ++o) pool[(size_t)dst[i] * bs + o] = pool[(size_t)src[i] * bs + o];
            }
            for (int i = 0; i < ntok; ++i) {
              CHECK(slots[i] >= 0 && (int64_t)slots[i] < NB * bs);
              pool[(size_t)slots[i]] = next_token;
              it->second.push_back(next_token++);
            }
          }
        }
      }
      // every live sequence reads back its own history; refcounts and stats add up
      std::vector<int32_t> owners((size_t)NB, 0);
      int64_t held_slots = 0, tokens = 0;
      std::vector<int32_t> row;
      for (auto& kv : hist) {
        int32_t nblk = -1;
        int64_t len = -1;
        CHECK(pa_bm_table(bm, kv.first, nullptr, 0, &nblk, &len) == PA_OK);
        CHECK(len == (int64_t)kv.second.size() && (int64_t)nblk * bs >= len);  // (whole pages: may hold more)
        row.assign((size_t)nblk + 1, -5);
        CHECK(pa_bm_table(bm, kv.first, row.data(), nblk, &nblk, &len) == PA_OK && row[(size_t)nblk] == -5);
        for (int64_t j = 0; j < len; ++j) {
          const int32_t b = row[(size_t)(j / bs)];
          CHECK(b >= 0 && b < NB);
          CHECK(pool[(size_t)b * bs + (size_t)(j % bs)] == kv.second[(size_t)j]);
          ++checked;
        }
        for (int32_t k = 0; k < nblk; ++k) owners[(size_t)row[(size_t)k]] += 1;
        tokens += len;
      }
      int64_t used = 0;
      for (int64_t b = 0; b < NB; ++b) {
        int32_t rc = -1;
        CHECK(pa_bm_block_refcount(bm, (int32_t)b, &rc) == PA_OK);
        // a page's blocks share one count; a block past a sequence's end may be
        // held by its page without being in its table
        CHECK(rc >= owners[(size_t)b]);
        used += rc > 0;
      }
      int64_t f, u, w;
      CHECK(pa_bm_stats(bm, &f, &u, &w) == PA_OK);
      CHECK(u == used && f + u == NB && w >= 0 && w <= u * bs);
      (void)held_slots;
      (void)tokens;
    }
    for (auto& kv : hist) CHECK(pa_bm_free_sequence(bm, kv.first) == PA_OK);
    int64_t f, u, w;
    CHECK(pa_bm_stats(bm, &f, &u, &w) == PA_OK && f == NB && u == 0 && w == 0);
    pa_bm_destroy(bm);
  }
  std::printf("block manager fuzz: %d pools; %lld appends (%lld block copies), %lld exhausted, %lld forks, "
              "%lld frees; %lld token reads checked\n", pools, appends, copies, exhausted, forks, frees, checked);
  return 0;
}
