// Host-side block manager of the paged KV cache: per-block reference counts,
// per-sequence block tables, fork by sharing, and copy-on-write of a shared,
// partially filled last page ("Ultimate Guide to PagedAttention": block
// table, on-demand allocation, memory sharing and copy-on-write).
//
// Pages are aligned runs of 2^k consecutive blocks, handed out by a buddy
// allocator (split on demand, merged with a free buddy on release); a
// sequence's pages are all of one size or double along the sequence, which
// is the power-of-two cache growth that "Paged Attention Meets
// FlexAttention" (abstract) reports for its memory curves.  Tables stay at
// block resolution, so the attention kernels see an ordinary pool of
// block_size-token blocks whatever the page sizes.  Bookkeeping only; the
// device work it implies (block copies, appends) is the caller's, through
// kv_copy_blocks and kv_append.
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "pagedattn.h"
#include "pagedattn_blocks.h"

struct pa_block_manager {
  struct Page {
    int32_t start;  // first block (a multiple of 2^order)
    int32_t order;  // 2^order blocks
  };
  struct Seq {
    std::vector<int32_t> blocks;  // logical block j -> physical block (every page, expanded)
    std::vector<Page> pages;
    int32_t min_order = 0, max_order = 0;  // page k has order min(min_order + k, max_order)
    int64_t len = 0;                       // tokens
    bool live = false;
  };
  int64_t num_blocks = 0;
  int32_t bs = 0;
  int32_t max_order = 0;                  // largest page: 2^max_order blocks
  std::vector<int32_t> refcount;          // per physical block (equal over a page)
  std::vector<int32_t> fill;              // tokens stored in a physical block (max over its owners)
  // Free pages: per order a stack of first blocks; free_pos[b] is the index
  // of the free page starting at block b in its order's stack (-1: none), so
  // a buddy leaves its stack in O(1) when it merges.
  std::vector<std::vector<int32_t>> free_pages;
  std::vector<int32_t> free_pos;
  std::vector<int8_t> free_ord;
  int64_t free_blocks = 0;

  void push_free(int32_t start, int32_t k) {
    free_pos[(size_t)start] = (int32_t)free_pages[(size_t)k].size();
    free_ord[(size_t)start] = (int8_t)k;
    free_pages[(size_t)k].push_back(start);
  }
  void drop_free(int32_t start) {
    std::vector<int32_t>& st = free_pages[(size_t)free_ord[(size_t)start]];
    const int32_t i = free_pos[(size_t)start];
    st[(size_t)i] = st.back();
    free_pos[(size_t)st[(size_t)i]] = i;
    st.pop_back();
    free_pos[(size_t)start] = -1;
  }
  std::vector<Seq> seqs;
  std::vector<int32_t> free_ids;
  mutable std::mutex mu;

  bool valid(int32_t s) const { return s >= 0 && (size_t)s < seqs.size() && seqs[s].live; }

  // A free page of 2^k blocks, splitting a larger one if needed; -1 if none.
  int32_t take_page(int32_t k) {
    int32_t j = k;
    while (j <= max_order && free_pages[(size_t)j].empty()) ++j;
    if (j > max_order) return -1;
    const int32_t start = free_pages[(size_t)j].back();
    drop_free(start);
    while (j > k) {  // keep the low half, free the high half
      --j;
      push_free(start + (1 << j), j);
    }
    for (int32_t b = start; b < start + (1 << k); ++b) {
      refcount[(size_t)b] = 1;
      fill[(size_t)b] = 0;
    }
    free_blocks -= (int64_t)1 << k;
    return start;
  }

  // Return a page whose blocks no sequence names any more, merging it with
  // its free buddy as long as there is one.
  void give_page(int32_t start, int32_t k) {
    for (int32_t b = start; b < start + (1 << k); ++b) {
      refcount[(size_t)b] = 0;
      fill[(size_t)b] = 0;
    }
    free_blocks += (int64_t)1 << k;
    while (k < max_order) {
      const int64_t buddy = (int64_t)start ^ ((int64_t)1 << k);
      if (buddy + ((int64_t)1 << k) > num_blocks) break;
      if (free_pos[(size_t)buddy] < 0 || free_ord[(size_t)buddy] != k) break;
      drop_free((int32_t)buddy);
      start = (int32_t)std::min<int64_t>(start, buddy);
      ++k;
    }
    push_free(start, k);
  }

  // Drop one owner of a page.
  void release_page(const Page& p) {
    bool last = false;
    for (int32_t b = p.start; b < p.start + (1 << p.order); ++b) last = (--refcount[(size_t)b] == 0);
    if (last) give_page(p.start, p.order);
  }

  int32_t new_id() {
    if (!free_ids.empty()) {
      const int32_t id = free_ids.back();
      free_ids.pop_back();
      return id;
    }
    seqs.emplace_back();
    return (int32_t)(seqs.size() - 1);
  }

};

namespace {

bool pow2_block(int32_t bs) { return bs >= 16 && bs <= 256 && (bs & (bs - 1)) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int32_t log2i(int64_t x) {
  int32_t k = 0;
  while (((int64_t)1 << k) < x) ++k;
  return k;
}
constexpr int32_t kMaxPageBlocks = 4096;

}  // namespace

extern "C" {

int pa_bm_create_paged(int64_t num_blocks, int32_t block_size, int32_t max_page_blocks, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (!pow2_block(block_size)) return PA_ERR_BLOCK_SIZE;
  // slots are int32 (kv_append's slot mapping): every slot of the pool must fit
  if (num_blocks < 0 || num_blocks * block_size > 0x7fffffffll) return PA_ERR_SIZE;
  if (!pow2(max_page_blocks) || max_page_blocks > kMaxPageBlocks) return PA_ERR_SIZE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_SIZE;
  bm->num_blocks = num_blocks;
  bm->bs = block_size;
  bm->max_order = log2i(max_page_blocks);
  bm->refcount.assign((size_t)num_blocks, 0);
  bm->fill.assign((size_t)num_blocks, 0);
  bm->free_pages.resize((size_t)bm->max_order + 1);
  bm->free_pos.assign((size_t)num_blocks, -1);
  bm->free_ord.assign((size_t)num_blocks, 0);
  // the pool as aligned free pages, each as large as alignment and size
  // allow; pushed from the top so that low block ids go out first
  std::vector<std::pair<int32_t, int32_t>> init;
  int64_t b = 0;
  while (b < num_blocks) {
    int32_t k = bm->max_order;
    while (k > 0 && ((b & (((int64_t)1 << k) - 1)) != 0 || b + ((int64_t)1 << k) > num_blocks)) --k;
    init.push_back({(int32_t)b, k});
    b += (int64_t)1 << k;
  }
  for (auto it = init.rbegin(); it != init.rend(); ++it) bm->push_free(it->first, it->second);
  bm->free_blocks = num_blocks;
  *out = bm;
  return PA_OK;
}

int pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out) {
  return pa_bm_create_paged(num_blocks, block_size, 1, out);
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_new_sequence_paged(pa_block_manager* bm, int32_t min_page_blocks, int32_t max_page_blocks, int32_t* seq) {
  if (!bm || !seq) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!pow2(min_page_blocks) || !pow2(max_page_blocks) || min_page_blocks > max_page_blocks ||
      log2i(max_page_blocks) > bm->max_order)
    return PA_ERR_SIZE;
  const int32_t id = bm->new_id();
  bm->seqs[id] = pa_block_manager::Seq();
  bm->seqs[id].min_order = log2i(min_page_blocks);
  bm->seqs[id].max_order = log2i(max_page_blocks);
  bm->seqs[id].live = true;
  *seq = id;
  return PA_OK;
}

int pa_bm_new_sequence(pa_block_manager* bm, int32_t* seq) { return pa_bm_new_sequence_paged(bm, 1, 1, seq); }

int pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child) {
  if (!bm || !child) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->valid(parent)) return PA_ERR_SEQ;
  const int32_t id = bm->new_id();
  bm->seqs[id] = bm->seqs[parent];  // (after new_id: seqs may have grown)
  for (int32_t blk : bm->seqs[id].blocks) ++bm->refcount[blk];
  *child = id;
  return PA_OK;
}

int pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  if (!bm) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->valid(seq)) return PA_ERR_SEQ;
  for (const pa_block_manager::Page& p : bm->seqs[seq].pages) bm->release_page(p);
  bm->seqs[seq] = pa_block_manager::Seq();
  bm->free_ids.push_back(seq);
  return PA_OK;
}

int pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t ntok, int32_t* slots_out, int32_t* copy_src,
                 int32_t* copy_dst, int32_t copy_cap, int32_t* ncopy) {
  if (!bm || !ncopy) return PA_ERR_NULL;
  if (ntok < 0 || copy_cap < 0) return PA_ERR_SIZE;
  if (ntok > 0 && !slots_out) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->valid(seq)) return PA_ERR_SEQ;
  pa_block_manager::Seq& s = bm->seqs[seq];
  *ncopy = 0;
  if (ntok == 0) return PA_OK;
  const int64_t bs = bm->bs;
  const int64_t cap_tokens = (int64_t)s.blocks.size() * bs;
  // A shared last page with room left: its owners would write into the same
  // free slots, so this sequence continues in a fresh page of the same size,
  // after copying the page's blocks that hold tokens.
  const bool cow = !s.pages.empty() && cap_tokens > s.len && bm->refcount[(size_t)s.pages.back().start] > 1;
  int32_t ncow = 0;
  if (cow) {
    const pa_block_manager::Page& last = s.pages.back();
    const int64_t page_first = cap_tokens - ((int64_t)bs << last.order);
    ncow = (int32_t)((s.len - page_first + bs - 1) / bs);
    if (copy_cap < ncow || !copy_src || !copy_dst) return PA_ERR_SIZE;
  }
  // every page this call takes, given back if the pool runs out midway
  std::vector<pa_block_manager::Page> taken;
  auto undo = [&]() {
    for (const pa_block_manager::Page& p : taken) bm->give_page(p.start, p.order);
    return PA_ERR_NO_BLOCKS;
  };
  int32_t cow_start = -1;
  if (cow) {
    cow_start = bm->take_page(s.pages.back().order);
    if (cow_start < 0) return PA_ERR_NO_BLOCKS;
    taken.push_back({cow_start, s.pages.back().order});
  }
  // new pages: page k of the sequence has order min(min_order + k, max_order);
  // a smaller page stands in when the pool has no page of that size left
  std::vector<pa_block_manager::Page> added;
  int64_t cap = cap_tokens;
  while (cap < s.len + ntok) {
    const int32_t want = std::min(s.min_order + (int32_t)(s.pages.size() + added.size()), s.max_order);
    int32_t k = want, start = -1;
    for (; k >= 0 && start < 0; --k) start = bm->take_page(k);
    if (start < 0) return undo();
    const int32_t order = k + 1;
    taken.push_back({start, order});
    added.push_back({start, order});
    cap += bs << order;
  }
  // commit
  if (cow) {
    pa_block_manager::Page& last = s.pages.back();
    const size_t first_blk = s.blocks.size() - ((size_t)1 << last.order);
    for (int32_t i = 0; i < ncow; ++i) {
      copy_src[i] = last.start + i;
      copy_dst[i] = cow_start + i;
      bm->fill[(size_t)(cow_start + i)] = bm->fill[(size_t)(last.start + i)];
    }
    for (int32_t i = 0; i < (1 << last.order); ++i) s.blocks[first_blk + (size_t)i] = cow_start + i;
    bm->release_page(last);
    last.start = cow_start;
    *ncopy = ncow;
  }
  for (const pa_block_manager::Page& p : added) {
    s.pages.push_back(p);
    for (int32_t i = 0; i < (1 << p.order); ++i) s.blocks.push_back(p.start + i);
  }
  for (int32_t i = 0; i < ntok; ++i) {
    const int64_t pos = s.len + i;
    const int32_t blk = s.blocks[(size_t)(pos / bs)];
    slots_out[i] = (int32_t)((int64_t)blk * bs + pos % bs);
    const int32_t f = (int32_t)(pos % bs) + 1;
    if (f > bm->fill[(size_t)blk]) bm->fill[(size_t)blk] = f;
  }
  s.len += ntok;
  return PA_OK;
}

int pa_bm_table(const pa_block_manager* bm, int32_t seq, int32_t* row, int32_t cap, int32_t* nblocks,
                int64_t* len) {
  if (!bm || !nblocks || !len) return PA_ERR_NULL;
  if (cap < 0) return PA_ERR_SIZE;
  if (cap > 0 && !row) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->valid(seq)) return PA_ERR_SEQ;
  const pa_block_manager::Seq& s = bm->seqs[seq];
  const size_t n = s.blocks.size();
  for (size_t j = 0; j < n && j < (size_t)cap; ++j) row[j] = s.blocks[j];
  *nblocks = (int32_t)n;
  *len = s.len;
  return PA_OK;
}

int pa_bm_stats(const pa_block_manager* bm, int64_t* free_blocks, int64_t* used_blocks, int64_t* waste_slots) {
  if (!bm || !free_blocks || !used_blocks || !waste_slots) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  int64_t used = 0, waste = 0;
  for (int64_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->refcount[(size_t)b] > 0) {
      ++used;
      waste += bm->bs - bm->fill[(size_t)b];
    }
  }
  *free_blocks = bm->free_blocks;
  *used_blocks = used;
  *waste_slots = waste;
  return PA_OK;
}

int pa_bm_pages(const pa_block_manager* bm, int32_t seq, int32_t* starts, int32_t* blocks, int32_t cap,
                int32_t* npages) {
  if (!bm || !npages) return PA_ERR_NULL;
  if (cap < 0) return PA_ERR_SIZE;
  if (cap > 0 && (!starts || !blocks)) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (!bm->valid(seq)) return PA_ERR_SEQ;
  const std::vector<pa_block_manager::Page>& p = bm->seqs[seq].pages;
  for (size_t i = 0; i < p.size() && i < (size_t)cap; ++i) {
    starts[i] = p[i].start;
    blocks[i] = 1 << p[i].order;
  }
  *npages = (int32_t)p.size();
  return PA_OK;
}

int pa_bm_block_refcount(const pa_block_manager* bm, int32_t block, int32_t* count) {
  if (!bm || !count) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  if (block < 0 || (int64_t)block >= bm->num_blocks) return PA_ERR_SIZE;
  *count = bm->refcount[(size_t)block];
  return PA_OK;
}

int pa_bm_prefix_levels(const pa_block_manager* bm, const int32_t* seqs, int32_t n, int32_t max_levels,
                        int32_t* group_starts, int32_t* prefix_starts, int32_t* prefix_ends, int32_t* num_groups,
                        int32_t* num_levels) {
  if (!bm || !num_levels) return PA_ERR_NULL;
  if (n < 0 || max_levels < 1 || max_levels > 8) return PA_ERR_SIZE;
  if (n > 0 && (!seqs || !group_starts || !prefix_starts || !prefix_ends || !num_groups)) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  *num_levels = 0;
  for (int32_t i = 0; i < n; ++i)
    if (!bm->valid(seqs[i])) return PA_ERR_SEQ;
  if (n == 0) return PA_OK;
  const int64_t bs = bm->bs;
  // shared[i]: tokens in the leading full blocks that sequences i and i+1 both name
  std::vector<int64_t> shared(n > 1 ? n - 1 : 0, 0);
  for (int32_t i = 0; i + 1 < n; ++i) {
    const pa_block_manager::Seq& a = bm->seqs[seqs[i]];
    const pa_block_manager::Seq& b = bm->seqs[seqs[i + 1]];
    const int64_t full = std::min(a.len, b.len) / bs;
    int64_t j = 0;
    while (j < full && a.blocks[(size_t)j] == b.blocks[(size_t)j]) ++j;
    shared[(size_t)i] = j * bs;
  }
  // groups of the current level: (first, last + 1, range end)
  struct Group {
    int32_t lo, hi;
    int64_t end;
  };
  std::vector<Group> cur{{0, n, 0}}, next;
  int32_t levels = 0;
  for (int32_t lvl = 0; lvl < max_levels; ++lvl) {
    next.clear();
    bool any = false;
    for (const Group& g : cur) {
      // maximal runs of neighbours sharing more than g.end
      int32_t a = g.lo;
      while (a < g.hi) {
        int32_t b = a + 1;
        int64_t end = INT64_MAX;
        while (b < g.hi && shared[(size_t)(b - 1)] > g.end) {
          end = std::min(end, shared[(size_t)(b - 1)]);
          ++b;
        }
        if (b - a < 2) end = g.end;  // alone: an empty range
        if (end > g.end) any = true;
        next.push_back({a, b, end});
        a = b;
      }
    }
    if (!any) break;
    int32_t* gs = group_starts + (size_t)lvl * (n + 1);
    int32_t* ps = prefix_starts + (size_t)lvl * n;
    int32_t* pe = prefix_ends + (size_t)lvl * n;
    // the range of a group starts where its members' previous range ended
    size_t k = 0;
    for (size_t i = 0; i < next.size(); ++i) {
      while (cur[k].hi <= next[i].lo) ++k;
      gs[i] = next[i].lo;
      ps[i] = (int32_t)cur[k].end;
      pe[i] = (int32_t)next[i].end;
    }
    gs[next.size()] = n;
    num_groups[lvl] = (int32_t)next.size();
    levels = lvl + 1;
    cur.swap(next);
  }
  *num_levels = levels;
  return PA_OK;
}

}  // extern "C"
