// Host-side block manager of the paged KV cache: a free list of physical
// blocks, per-block reference counts, per-sequence block tables, fork by
// sharing, and copy-on-write of a shared, partially filled last block
// ("Ultimate Guide to PagedAttention": block table, on-demand allocation,
// memory sharing and copy-on-write).  Bookkeeping only; the device work it
// implies (block copies, appends) is the caller's, through kv_copy_blocks and
// kv_append.
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "pagedattn.h"
#include "pagedattn_blocks.h"

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;  // logical block j -> physical block
    int64_t len = 0;              // tokens
    bool live = false;
  };
  int64_t num_blocks = 0;
  int32_t bs = 0;
  std::vector<int32_t> refcount;  // per physical block
  std::vector<int32_t> fill;      // tokens stored in a physical block (max over its owners)
  std::vector<int32_t> free_list; // stack of free physical blocks
  std::vector<Seq> seqs;
  std::vector<int32_t> free_ids;
  mutable std::mutex mu;

  bool valid(int32_t s) const { return s >= 0 && (size_t)s < seqs.size() && seqs[s].live; }

  int32_t new_id() {
    if (!free_ids.empty()) {
      const int32_t id = free_ids.back();
      free_ids.pop_back();
      return id;
    }
    seqs.emplace_back();
    return (int32_t)(seqs.size() - 1);
  }

  void release(int32_t blk) {
    if (--refcount[blk] == 0) {
      fill[blk] = 0;
      free_list.push_back(blk);
    }
  }
};

namespace {

bool pow2_block(int32_t bs) { return bs >= 16 && bs <= 256 && (bs & (bs - 1)) == 0; }

}  // namespace

extern "C" {

int pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 0 || num_blocks > 0x7fffffffll) return PA_ERR_SIZE;
  if (!pow2_block(block_size)) return PA_ERR_BLOCK_SIZE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_SIZE;
  bm->num_blocks = num_blocks;
  bm->bs = block_size;
  bm->refcount.assign((size_t)num_blocks, 0);
  bm->fill.assign((size_t)num_blocks, 0);
  bm->free_list.reserve((size_t)num_blocks);
  // hand out low block ids first
  for (int64_t b = num_blocks - 1; b >= 0; --b) bm->free_list.push_back((int32_t)b);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_new_sequence(pa_block_manager* bm, int32_t* seq) {
  if (!bm || !seq) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lk(bm->mu);
  const int32_t id = bm->new_id();
  bm->seqs[id] = pa_block_manager::Seq();
  bm->seqs[id].live = true;
  *seq = id;
  return PA_OK;
}

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
  for (int32_t blk : bm->seqs[seq].blocks) bm->release(blk);
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
  const int64_t in_last = s.len % bs;  // tokens already in the last block
  const bool cow = in_last != 0 && bm->refcount[s.blocks.back()] > 1;
  const int64_t new_blocks = (s.len + ntok + bs - 1) / bs - (int64_t)s.blocks.size();
  const int64_t need = new_blocks + (cow ? 1 : 0);
  if (need > (int64_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  if (cow && (copy_cap < 1 || !copy_src || !copy_dst)) return PA_ERR_SIZE;
  if (cow) {
    // the shared last block keeps its other owners; this sequence writes into a copy
    const int32_t old = s.blocks.back();
    const int32_t fresh = bm->free_list.back();
    bm->free_list.pop_back();
    bm->refcount[fresh] = 1;
    bm->fill[fresh] = (int32_t)in_last;
    bm->release(old);
    s.blocks.back() = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *ncopy = 1;
  }
  for (int64_t i = 0; i < new_blocks; ++i) {
    const int32_t blk = bm->free_list.back();
    bm->free_list.pop_back();
    bm->refcount[blk] = 1;
    bm->fill[blk] = 0;
    s.blocks.push_back(blk);
  }
  for (int32_t i = 0; i < ntok; ++i) {
    const int64_t pos = s.len + i;
    const int32_t blk = s.blocks[(size_t)(pos / bs)];
    slots_out[i] = (int32_t)((int64_t)blk * bs + pos % bs);
    const int32_t f = (int32_t)(pos % bs) + 1;
    if (f > bm->fill[blk]) bm->fill[blk] = f;
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
  *free_blocks = (int64_t)bm->free_list.size();
  *used_blocks = used;
  *waste_slots = waste;
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
