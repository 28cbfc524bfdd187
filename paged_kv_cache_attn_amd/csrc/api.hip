// C ABI entry points: host-side validation, split-KV sizing and launches.
// Every check happens before anything is enqueued; see include/pagedattn.h.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <initializer_list>
#include <mutex>

#include "pagedattn.h"
#include "pa_kernels.h"

namespace {

constexpr int kUnsplitLog2 = 30;
constexpr int kAutoSplitMax = 512;
constexpr int kAutoSplitMin = 64;
constexpr long long kAutoTargetUnits = 2048;  // ~8 wavefronts per compute unit
constexpr int kStreamWavesPerCU = 8;          // resident decode wavefronts per compute unit
constexpr int kStreamMaxSeqs = 4096;          // chunk prefix of all rows fits in 16 KB of LDS
constexpr int kWgMinSplitLog2 = 6;            // fixed partitions as work-groups from 64 keys up
constexpr int kSplitBalanced = -2;            // split_tokens code: the balanced split, always
constexpr int kSmallSplitLog2 = 9;            // default split of small batches: 512-key partitions
constexpr int kSmallMaxBlocksPerCU = 16;      // ... while that grid holds at most this many per unit
constexpr int kSmallMaxPartsLog2 = 5;         // ... longer pieces past 32 per row (one merge batch)
constexpr int kUnsplitMaxCtx = 256;           // rows this short are never split (no merge launch)
constexpr int kDefaultCUs = 256;              // MI355X, when no device is visible
constexpr int kPrefillMinSplitKeys = 512;     // split prefill: keys per range, at least

int ilog2(long long x) {
  int r = 0;
  while ((1ll << r) < x) ++r;
  return r;
}
bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }
// The product of non-negative factors exceeds limit (a negative factor
// counts as exceeding); computed in 128 bits, so it never overflows.
bool product_exceeds(std::initializer_list<long long> factors, long long limit) {
  unsigned __int128 p = 1;
  for (long long f : factors) {
    if (f < 0) return true;
    p *= (unsigned __int128)f;
    if (p > (unsigned __int128)limit) return true;
  }
  return false;
}

int check_dtype(int32_t dtype) { return (dtype == PA_F32 || dtype == PA_BF16) ? PA_OK : PA_ERR_DTYPE; }
int check_dim(int32_t d) { return (d == 64 || d == 128) ? PA_OK : PA_ERR_HEAD_DIM; }
int check_bs(int32_t bs) { return (is_pow2(bs) && bs >= 16 && bs <= 256) ? PA_OK : PA_ERR_BLOCK_SIZE; }
int check_heads(int32_t hq, int32_t hkv) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return PA_ERR_HEADS;
  return PA_OK;
}
int check_split(int32_t split) {
  if (split == 0 || split == -1 || split == kSplitBalanced) return PA_OK;
  return (is_pow2(split) && split >= 16 && split <= (1 << 29)) ? PA_OK : PA_ERR_SPLIT;
}
int check_mods(const pa_score_mods* m) {
  if (!m) return PA_OK;
  if (m->window < 0) return PA_ERR_MODS;
  if (!(m->softcap >= 0.f) || isinf(m->softcap)) return PA_ERR_MODS;
  if (const pa_block_mask* bm = m->block_mask) {
    if (!bm->bits) return PA_ERR_NULL;
    if (!is_pow2(bm->q_block) || !is_pow2(bm->kv_block) || bm->kv_block < 64 || bm->kv_block > (1 << 24) ||
        bm->rows_per_seq < 1 || bm->words_per_row < 1)
      return PA_ERR_MODS;
    if (reinterpret_cast<uintptr_t>(bm->bits) % 4 != 0) return PA_ERR_ALIGN;
  }
  return PA_OK;
}

pa::BlockMaskArgs block_mask_args(const pa_score_mods* m) {
  pa::BlockMaskArgs a{nullptr, 0, 0, 0, 0};
  if (m && m->block_mask) {
    const pa_block_mask* bm = m->block_mask;
    a.bits = bm->bits;
    a.q_log2 = ilog2(bm->q_block);
    a.kv_log2 = ilog2(bm->kv_block);
    a.rows = bm->rows_per_seq;
    a.words = bm->words_per_row;
  }
  return a;
}

// log2 of the partition length, kUnsplitLog2 for "never split".
int resolve_split_log2(int32_t B, int32_t Hkv, int32_t max_ctx, int32_t split) {
  if (split == -1) return kUnsplitLog2;
  if (split > 0) return ilog2(split);
  long long s = kAutoSplitMax;
  // (B * Hkv capped at the target: the comparison below is unchanged and the
  // product cannot overflow)
  const long long bh = std::min((long long)B * Hkv, kAutoTargetUnits);
  auto units = [&](long long sp) { return bh * (((long long)max_ctx + sp - 1) / sp); };
  while (s > kAutoSplitMin && units(s) < kAutoTargetUnits) s >>= 1;
  return ilog2(s);
}

int partitions(int32_t max_ctx, int split_log2) {
  if (split_log2 >= kUnsplitLog2 || max_ctx <= 0) return 1;
  const long long sp = 1ll << split_log2;
  return (int)((max_ctx + sp - 1) / sp);
}

int group_pad(int g) { return g <= 4 ? 4 : 8; }

// Compute units of the current device, queried once per device (concurrent
// first calls may both query; they store the same value).
int device_cus() {
  constexpr int kMaxDevices = 256;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return kDefaultCUs;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

struct Shape;
int wg_pays_off(int32_t B, int32_t Hkv, const Shape& s);

struct Shape {
  int g, GP, NG, P, split_log2;
  int W;   // > 0: balanced split over W wavefronts
  int wg;  // 1: fixed partitions as multi-wavefront work-groups
  int FW;  // > 0: fixed partitions walked by FW persistent wavefronts
};

// Fixed partitions of at least 64 keys run as 4-wavefront work-groups that
// merge in LDS when the whole grid is resident at once (two work-groups per
// compute unit): a small batch's partitions then stream four times faster.
// Larger grids keep one wavefront per partition: there a work-group holds four
// wavefront slots for each partition a short row leaves empty.
int wg_pays_off(int32_t B, int32_t Hkv, const Shape& s) {
  if (s.split_log2 < kWgMinSplitLog2) return 0;
  const long long blocks = (long long)B * Hkv * s.NG * s.P;
  return blocks <= 2ll * device_cus() ? 1 : 0;
}

// Decode grids of fixed partitions too large to be resident at once are
// walked by persistent wavefronts (8 per compute unit) over the partitions
// that exist, when the per-row prefix fits in LDS.
int fixed_waves_for(int32_t B, int32_t Hkv, const Shape& s) {
  if (s.wg || s.P <= 1 || B > kStreamMaxSeqs) return 0;
  const long long blocks = (long long)B * Hkv * s.NG * s.P;
  return (int)std::min(blocks, (long long)device_cus() * kStreamWavesPerCU);
}

// The default split of a batch too small for the balanced split to pay off:
// fixed 512-key partitions, while their grid holds at most 16 partitions per
// compute unit.  Measured on MI355X (cold calls, 32/8 heads, d128): 16.8
// against 18.7 us on 8 rows of 128..2048 keys, 20.5 against 21.1 us on 16
// rows of 1,280, 18.4 against 21.2 us on 8 rows of 2,048, 29.9 against 34.3
// us on 8 rows of 4,096; on the 64-row long batch (lengths 2k..32k) the
// balanced split is far faster (463 against 626 us), and its grid of 512-key
// partitions is 8x over the limit.  The host sees only max_context_len, so
// the rule counts every row at that length (kv-heads only, so that
// paged_attn_decode_split_tokens gives the same answer without num_heads).
bool small_batch_split(int32_t B, int32_t Hkv, int32_t max_ctx) {
  const long long parts = ((long long)max_ctx + (1 << kSmallSplitLog2) - 1) >> kSmallSplitLog2;
  return (long long)B * Hkv * parts <= (long long)kSmallMaxBlocksPerCU * device_cus();
}

// Partition length of the small-batch rule: 512 keys, lengthened (powers of
// two) until a row has at most 32 pieces, the states the merge reads in one
// round trip.  Single rows of 8,192 keys, 8 kv-heads: 16.7 us at 512 against
// 22.4 at 1024; of 32,768: 28.2 at 1024 against 30.7 at 512; of 65,536: 47.7
// at 2048 against 53.6 (cold).
int small_batch_split_log2(int32_t max_ctx) {
  return std::max(kSmallSplitLog2, ilog2(max_ctx) - kSmallMaxPartsLog2);
}

int decode_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_ctx, int32_t split, Shape& s) {
  s.g = Hq / Hkv;
  s.GP = group_pad(s.g);
  s.NG = (s.g - 1) / s.GP + 1;  // (g >= 1; no overflow for any int32 g)
  s.W = 0;
  s.wg = 0;
  s.FW = 0;
  if (split == 0 && max_ctx <= kUnsplitMaxCtx) {
    // every row fits a few chunks: one work-group per (row, head group)
    // finishes it faster than a split plus the merge launch would
    s.split_log2 = kUnsplitLog2;
    s.P = 1;
    s.wg = wg_pays_off(B, Hkv, s);
    return PA_OK;
  }
  if (split == 0 && small_batch_split(B, Hkv, max_ctx)) {
    s.split_log2 = small_batch_split_log2(max_ctx);
    s.P = partitions(max_ctx, s.split_log2);
    s.wg = wg_pays_off(B, Hkv, s);
    s.FW = fixed_waves_for(B, Hkv, s);
    return PA_OK;
  }
  if ((split == 0 || split == kSplitBalanced) && B <= kStreamMaxSeqs) {
    // balanced split: as many wavefronts as stay resident, but at least
    // pa::kStreamMinChunks chunks of work each for the largest possible batch
    const long long chunks = (long long)B * Hkv * s.NG * (((long long)max_ctx + 15) / 16 + 1);
    long long w = (long long)device_cus() * kStreamWavesPerCU;
    w = std::min(w, std::max(1ll, chunks / pa::kStreamMinChunks));
    s.W = (int)w;
    s.split_log2 = kUnsplitLog2;
    s.P = 1;
    return PA_OK;
  }
  s.split_log2 = resolve_split_log2(B, Hkv, max_ctx, split);
  s.P = partitions(max_ctx, s.split_log2);
  s.wg = wg_pays_off(B, Hkv, s);
  s.FW = fixed_waves_for(B, Hkv, s);
  return PA_OK;
}

size_t workspace_bytes_for(int32_t B, int32_t Hkv, int32_t D, const Shape& s) {
  if (s.W > 0) {
    const size_t items = (size_t)B * Hkv * s.NG;
    return ((size_t)s.W + items) * s.GP * (size_t)(D + 2) * sizeof(float) + items * 2 * sizeof(int32_t);
  }
  if (s.P <= 1) return 0;
  return (size_t)B * Hkv * s.NG * s.GP * (size_t)s.P * (size_t)(D + 2) * sizeof(float);
}

int common_decode_checks(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int64_t NB,
                         int32_t bt_stride, int32_t max_ctx, int32_t split, int32_t dtype,
                         const pa_score_mods* mods) {
  int st;
  if ((st = check_dtype(dtype))) return st;
  if (B < 0 || NB < 0 || max_ctx < 0) return PA_ERR_SIZE;
  if ((st = check_heads(Hq, Hkv))) return st;
  if ((st = check_dim(D))) return st;
  if ((st = check_bs(bs))) return st;
  if ((st = check_split(split))) return st;
  if ((st = check_mods(mods))) return st;
  if (B > 0 && bt_stride < 1) return PA_ERR_TABLE_STRIDE;
  return PA_OK;
}

void fill_row_args(pa::RowAttnArgs& a, void* out, const void* q, const void* kc, const void* vc,
                   const int32_t* bt, int32_t bt_stride, const int32_t* ctx, const int32_t* cu,
                   int32_t B, int32_t max_q, int32_t Hq, int32_t Hkv, int32_t bs, const Shape& s,
                   float scale, int32_t causal, const pa_score_mods* mods, void* ws, int32_t D) {
  a.out = out;
  a.q = q;
  a.k_cache = kc;
  a.v_cache = vc;
  a.block_tables = bt;
  a.context_lens = ctx;
  a.cu_q_lens = cu;
  a.bt_stride = bt_stride;
  a.max_q_len = max_q;
  a.num_seqs = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.g = s.g;
  a.NG = s.NG;
  a.bs_log2 = ilog2(bs);
  a.num_blocks = 0;  // set by the caller
  a.split_log2 = s.split_log2;
  a.P = s.P;
  a.stream_waves = s.W;
  a.wg_partitions = s.wg;
  a.fixed_waves = s.FW;
  a.causal = causal;
  a.window = mods ? mods->window : 0;
  a.scale = scale;
  a.softcap = mods ? mods->softcap : 0.f;
  a.alibi = mods ? mods->alibi_slopes : nullptr;
  a.prefix_lens = mods ? mods->prefix_lens : nullptr;
  a.doc_starts = mods ? mods->doc_starts : nullptr;
  a.bm = block_mask_args(mods);
  a.row_floor = nullptr;
  a.state_o = nullptr;
  a.state_lse = nullptr;
  float* w = static_cast<float*>(ws);
  const size_t units = s.W > 0 ? ((size_t)s.W + (size_t)B * Hkv * s.NG) * s.GP
                               : (size_t)B * max_q * Hkv * s.NG * s.GP * (size_t)s.P;
  a.ws_o = w;
  a.ws_ml = w ? w + units * D : nullptr;
  a.ws_meta = (w && s.W > 0) ? reinterpret_cast<int32_t*>(w + units * (D + 2)) : nullptr;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : (int)e; }

// Every tensor pointer given (NULL ones are checked elsewhere) is 16-byte aligned.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
  return true;
}

// ---- two-phase (shared-prefix) decode ----
constexpr int kCascadeMinTiles = 4;   // 64-key tiles per prefix key range, at least
constexpr int kCascadeMaxLevels = 8;  // prefix levels per call
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct CascadeLevel {
  int q_tiles, key_split, nsplit, range0;  // range0: index of the level's first key range
};

struct CascadeShape {
  CascadeLevel lv[kCascadeMaxLevels];
  int nranges;  // key ranges over all levels
  Shape dec;    // the suffix decode
  size_t off_part_lse, off_state_o, off_state_lse, off_key_start, off_dec, total;
};

// Prefix phase of one level: groups x kv-heads x query tiles work-groups per
// key range; enough ranges for two work-groups per compute unit, each range at
// least kCascadeMinTiles tiles.
void cascade_level(int32_t G, int32_t max_group, int32_t Hq, int32_t Hkv, int32_t max_range, CascadeLevel& l) {
  const int qt = pa::prefill_rows_per_tile(Hq / Hkv);
  l.q_tiles = (int)(((long long)max_group + qt - 1) / qt);
  const long long tiles = ((long long)max_range + 63) / 64;
  const long long base = std::max(1ll, (long long)G * Hkv * l.q_tiles);
  long long ns = (2ll * device_cus() + base - 1) / base;
  ns = std::max(1ll, std::min(ns, tiles / kCascadeMinTiles));
  const long long per = tiles > 0 ? (tiles + ns - 1) / ns : 1;
  l.key_split = (int)(per * 64);
  l.nsplit = (int)std::max(1ll, ((long long)max_range + l.key_split - 1) / l.key_split);
}

void cascade_shape(int32_t B, const pa_prefix_level* levels, int32_t L, int32_t Hq, int32_t Hkv, int32_t D,
                   int32_t max_ctx, CascadeShape& c) {
  c.nranges = 0;
  for (int i = 0; i < L; ++i) {
    cascade_level(levels[i].num_groups, levels[i].max_group_size, Hq, Hkv, levels[i].max_prefix_len, c.lv[i]);
    c.lv[i].range0 = c.nranges;
    c.nranges += c.lv[i].nsplit;
  }
  decode_shape(B, Hq, Hkv, max_ctx, 0, c.dec);
  const size_t rows = (size_t)B * Hq;
  size_t off = align_up((size_t)c.nranges * rows * D * sizeof(float));
  c.off_part_lse = off;
  off += align_up((size_t)c.nranges * rows * sizeof(float));
  c.off_state_o = off;
  off += align_up(rows * D * sizeof(float));
  c.off_state_lse = off;
  off += align_up(rows * sizeof(float));
  c.off_key_start = off;
  off += align_up((size_t)B * sizeof(int32_t));
  c.off_dec = off;
  off += align_up(workspace_bytes_for(B, Hkv, D, c.dec));
  c.total = off;
}

// Host-visible parts of the levels (the device arrays are checked for NULL
// by the call itself).
int check_cascade_levels(int32_t B, const pa_prefix_level* levels, int32_t L) {
  if (B == 0) return (L >= 0 && L <= kCascadeMaxLevels) ? PA_OK : PA_ERR_SIZE;
  if (!levels) return PA_ERR_NULL;
  if (L < 1 || L > kCascadeMaxLevels) return PA_ERR_SIZE;
  for (int i = 0; i < L; ++i) {
    const pa_prefix_level& v = levels[i];
    if (v.num_groups < 1 || v.max_group_size < 1 || v.max_prefix_len < 0) return PA_ERR_SIZE;
  }
  return PA_OK;
}

// The two-phase decode pays off once re-reading the shared keys per sequence
// costs more than its extra launches: measured on MI355X, a 16 x (1,024 +
// 256)-token batch (84 MB of logical K+V) ran 0.87x as fast two-phase as
// plain, and every batch of 335 MB or more (64 x (1,024 + 256) up to
// 64 x (16,384 + 1,024)) ran 1.2-4.8x faster.  The bound is host-side:
// num_seqs x max_context_len keys of K and V in every kv-head.
constexpr double kTwoPhaseMinLogicalBytes = 256.0 * (1 << 20);

bool two_phase_pays_off(int32_t B, int32_t Hkv, int32_t D, int32_t max_ctx) {
  return (double)B * max_ctx * Hkv * D * 2.0 * 2.0 >= kTwoPhaseMinLogicalBytes;
}

int cascade_impl(bool force_two_phase, void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                 int32_t num_seqs, const pa_prefix_level* levels, int32_t num_levels, int32_t num_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                 int32_t max_context_len, float scale, const pa_score_mods* mods, void* workspace,
                 size_t workspace_bytes, int32_t dtype, void* stream);

int decode_impl(bool do_partials, bool do_merge, void* out, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* block_tables, int32_t bt_stride,
                const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                int32_t bs, int64_t NB, int32_t max_ctx, float scale, int32_t split,
                const pa_score_mods* mods, void* workspace, size_t workspace_bytes, int32_t dtype,
                void* stream) {
  int st = common_decode_checks(B, Hq, Hkv, D, bs, NB, bt_stride, max_ctx, split, dtype, mods);
  if (st) return st;
  if (B == 0) return PA_OK;
  if (!out || !context_lens) return PA_ERR_NULL;
  if (do_partials && (!q || !k_cache || !v_cache || !block_tables)) return PA_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache, workspace})) return PA_ERR_ALIGN;
  Shape s;
  decode_shape(B, Hq, Hkv, max_ctx, split, s);
  const size_t need = workspace_bytes_for(B, Hkv, D, s);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const long long blocks = (long long)B * Hkv * s.NG * s.P;
  if (blocks > 0x7fffffffll || (long long)B * Hq > 0x7fffffffll) return PA_ERR_SIZE;
  pa::RowAttnArgs a;
  fill_row_args(a, out, q, k_cache, v_cache, block_tables, bt_stride, context_lens, nullptr, B, 1,
                Hq, Hkv, bs, s, scale, 1, mods, need > 0 ? workspace : nullptr, D);
  a.num_blocks = NB;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (do_partials) {
    if ((st = launch_status(pa::launch_row_partials(a, dtype, D, hs)))) return st;
  }
  if (do_merge && (s.P > 1 || s.W > 0)) {
    if ((st = launch_status(pa::launch_row_merge(a, dtype, D, hs)))) return st;
  }
  return PA_OK;
}

// ---- library-held decode scratch (paged_attn_decode_noalloc) ----
// One array per device, allocated with the code object when the library is
// loaded on that device and kept until the process ends.  Host code never
// uses the array's name as an address: its device address is looked up once
// per device with hipGetSymbolAddress and cached.
constexpr size_t kScratchBytes = (size_t)PA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (looked up on first use), or a
// positive hipError_t.
int scratch_for_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

int kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
              void* stream) {
  int st;
  if ((st = check_dtype(dtype))) return st;
  if (num_tokens < 0 || num_blocks < 0) return PA_ERR_SIZE;
  if (num_kv_heads <= 0) return PA_ERR_HEADS;
  if ((st = check_dim(head_dim))) return st;
  if ((st = check_bs(block_size))) return st;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16({k_new, v_new, k_cache, v_cache})) return PA_ERR_ALIGN;
  if ((long long)num_tokens * num_kv_heads > 0x7fffffffll) return PA_ERR_SIZE;
  pa::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slots = slot_mapping;
  a.num_blocks = num_blocks;
  a.T = num_tokens;
  a.Hkv = num_kv_heads;
  a.D = head_dim;
  a.bs_log2 = ilog2(block_size);
  return launch_status(pa::launch_kv_append(a, dtype, static_cast<hipStream_t>(stream)));
}

int32_t paged_attn_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t split_tokens) {
  if (check_split(split_tokens) || num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0) return 0;
  if (split_tokens == 0 && max_context_len <= kUnsplitMaxCtx) return -1;  // short rows: unsplit
  if (split_tokens == 0 && small_batch_split(num_seqs, num_kv_heads, max_context_len))
    return 1 << small_batch_split_log2(max_context_len);
  if ((split_tokens == 0 || split_tokens == kSplitBalanced) && num_seqs <= kStreamMaxSeqs)
    return 0;  // balanced split
  const int l2 = resolve_split_log2(num_seqs, num_kv_heads, max_context_len, split_tokens);
  return l2 >= kUnsplitLog2 ? -1 : (1 << l2);
}

int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks, const int32_t* dst_blocks,
                   int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, int32_t dtype, void* stream) {
  int st;
  if ((st = check_dtype(dtype))) return st;
  if (num_pairs < 0 || num_blocks < 0) return PA_ERR_SIZE;
  if (num_kv_heads <= 0) return PA_ERR_HEADS;
  if ((st = check_dim(head_dim))) return st;
  if ((st = check_bs(block_size))) return st;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks) return PA_ERR_NULL;
  if (!aligned16({k_cache, v_cache})) return PA_ERR_ALIGN;
  pa::CopyArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.src = src_blocks;
  a.dst = dst_blocks;
  a.pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.slab16 = (int32_t)((size_t)block_size * head_dim * (dtype == PA_BF16 ? 2 : 4) / 16);
  a.Hkv = num_kv_heads;
  if ((long long)num_pairs * num_kv_heads * 2 > 0x7fffffffll) return PA_ERR_SIZE;
  return launch_status(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t split_tokens) {
  if (num_seqs < 0 || max_context_len < 0 || check_heads(num_heads, num_kv_heads) ||
      check_dim(head_dim) || check_split(split_tokens))
    return 0;
  Shape s;
  decode_shape(num_seqs, num_heads, num_kv_heads, max_context_len, split_tokens, s);
  return workspace_bytes_for(num_seqs, num_kv_heads, head_dim, s);
}

int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int32_t max_context_len, float scale,
                      int32_t split_tokens, const pa_score_mods* mods, void* workspace,
                      size_t workspace_bytes, int32_t dtype, void* stream) {
  return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, block_table_stride,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_context_len, scale, split_tokens, mods, workspace,
                     workspace_bytes, dtype, stream);
}

int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, int32_t max_context_len, float scale,
                              int32_t split_tokens, const pa_score_mods* mods, int32_t dtype,
                              void* stream) {
  int st = common_decode_checks(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                block_table_stride, max_context_len, split_tokens, dtype, mods);
  if (st) return st;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PA_ERR_ALIGN;
  Shape s;
  decode_shape(num_seqs, num_heads, num_kv_heads, max_context_len, split_tokens, s);
  const size_t need = workspace_bytes_for(num_seqs, num_kv_heads, head_dim, s);
  if (need > kScratchBytes) return PA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && (st = scratch_for_current_device(&ws))) return st;
  // Every workspace byte the kernels read is written earlier in the same
  // call (per-item unit records, partials), so nothing is cleared here.
  return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, block_table_stride,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_context_len, scale, split_tokens, mods, ws, need > 0 ? kScratchBytes : 0,
                     dtype, stream);
}

int paged_attn_decode_partials(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               int32_t block_table_stride, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               int32_t max_context_len, float scale, int32_t split_tokens,
                               const pa_score_mods* mods, void* workspace,
                               size_t workspace_bytes, int32_t dtype, void* stream) {
  return decode_impl(true, false, out, q, k_cache, v_cache, block_tables, block_table_stride,
                     context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_context_len, scale, split_tokens, mods, workspace,
                     workspace_bytes, dtype, stream);
}

int paged_attn_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_context_len, int32_t split_tokens,
                            const pa_score_mods* mods, const void* workspace,
                            size_t workspace_bytes, int32_t dtype, void* stream) {
  return decode_impl(false, true, out, nullptr, nullptr, nullptr, nullptr, 1, context_lens,
                     num_seqs, num_heads, num_kv_heads, head_dim, 16, 0, max_context_len, 1.f,
                     split_tokens, mods, const_cast<void*>(workspace), workspace_bytes, dtype,
                     stream);
}

}  // extern "C"

namespace {

// Key ranges of a bf16 prefill whose grid of (sequence, kv-head, query tile)
// work-groups leaves compute units idle.  key_split: 0 library choice, -1
// never, > 0 keys per range (a multiple of 64).  The library splits only a
// grid smaller than the device (as a one-GPU share of a head split is) into
// ranges of at least 512 keys, up to about two work-groups per compute unit:
// shorter ranges cost more in merge traffic than they gain in parallelism.
// A block mask keeps the unsplit path.
struct PrefillSplit {
  int key_split = 0;  // 0: no split
  int nsplit = 1;
};

PrefillSplit prefill_split_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t q_tiles, int32_t max_ctx,
                                int32_t key_split, bool block_mask) {
  PrefillSplit p;
  if (key_split == -1 || max_ctx <= 0 || block_mask) return p;
  long long per = key_split;
  if (key_split == 0) {
    const long long blocks = (long long)num_seqs * num_kv_heads * q_tiles;
    const long long cus = device_cus();
    if (blocks <= 0 || blocks >= cus) return p;
    const long long n = std::min<long long>(2 * cus / blocks, max_ctx / kPrefillMinSplitKeys);
    if (n < 2) return p;
    per = ((max_ctx + n - 1) / n + 63) / 64 * 64;
  }
  const long long ns = (max_ctx + per - 1) / per;
  if (ns <= 1) return p;
  p.key_split = (int)per;
  p.nsplit = (int)ns;
  return p;
}

int check_prefill_split(int32_t key_split) {
  if (key_split == 0 || key_split == -1) return PA_OK;
  return (key_split >= 64 && key_split % 64 == 0) ? PA_OK : PA_ERR_SPLIT;
}

// Workspace of a split prefill: part_o [nsplit, total_q, Hq, D] then part_lse
// [nsplit, total_q, Hq] (256-byte aligned), fp32; 0 without a split, and
// SIZE_MAX when the sizes overflow.
size_t prefill_split_bytes(const PrefillSplit& p, int32_t total_q, int32_t num_heads, int32_t head_dim,
                           size_t* lse_offset) {
  if (p.nsplit <= 1 || total_q <= 0) return 0;
  const unsigned __int128 states = (unsigned __int128)p.nsplit * (unsigned)total_q * (unsigned)num_heads;
  const unsigned __int128 o_bytes = (states * (unsigned)head_dim * 4 + 255) / 256 * 256;
  const unsigned __int128 total = o_bytes + states * 4;
  if (total > (unsigned __int128)(SIZE_MAX / 2)) return SIZE_MAX;
  if (lse_offset) *lse_offset = (size_t)o_bytes;
  return (size_t)total;
}

int prefill_impl(void* out, const void* q, const int32_t* cu_q_lens, int32_t total_q, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, int32_t block_table_stride,
                 const int32_t* context_lens, int32_t num_seqs, int32_t max_q_len, int32_t num_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                 int32_t max_context_len, int32_t key_split, float scale, int32_t causal,
                 const pa_score_mods* mods, void* workspace, size_t workspace_bytes, int32_t dtype,
                 void* stream) {
  int st;
  if ((st = check_dtype(dtype))) return st;
  if (num_seqs < 0 || num_blocks < 0 || max_q_len < 0) return PA_ERR_SIZE;
  if ((st = check_heads(num_heads, num_kv_heads))) return st;
  if ((st = check_dim(head_dim))) return st;
  if ((st = check_bs(block_size))) return st;
  if (causal != 0 && causal != 1) return PA_ERR_FLAG;
  if ((st = check_mods(mods))) return st;
  if ((st = check_prefill_split(key_split))) return st;
  if (key_split != -1 && (total_q < 0 || max_context_len < 0)) return PA_ERR_SIZE;
  if (num_seqs > 0 && block_table_stride < 1) return PA_ERR_TABLE_STRIDE;
  if (num_seqs == 0 || max_q_len == 0 || (key_split != -1 && total_q == 0)) return PA_OK;
  if (!out || !q || !cu_q_lens || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PA_ERR_ALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int g = num_heads / num_kv_heads;
  if (dtype == PA_BF16 && 128 % g == 0) {
    pa::PrefillArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.cu_q_lens = cu_q_lens;
    a.alibi = mods ? mods->alibi_slopes : nullptr;
    a.prefix_lens = mods ? mods->prefix_lens : nullptr;
    a.doc_starts = mods ? mods->doc_starts : nullptr;
    a.bm = block_mask_args(mods);
    a.table_rows = nullptr;
    a.part_o = nullptr;
    a.part_lse = nullptr;
    a.row_key_start = nullptr;
    a.key_starts = nullptr;
    a.q_ctx = nullptr;
    a.num_cus = device_cus();
    a.chain = 0;
    a.key_split = 0;
    a.nsplit = 1;
    a.total_q = 0;
    a.bt_stride = block_table_stride;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.Hq = num_heads;
    a.Hkv = num_kv_heads;
    a.g = g;
    a.bs_log2 = ilog2(block_size);
    const int qt = pa::prefill_rows_per_tile(g);
    a.q_tiles = (max_q_len - 1) / qt + 1;  // (max_q_len >= 1 here)
    a.causal = causal;
    a.window = mods ? mods->window : 0;
    a.scale = scale;
    a.softcap = mods ? mods->softcap : 0.f;
    if (product_exceeds({num_seqs, num_kv_heads, a.q_tiles}, 0x7fffffffll)) return PA_ERR_SIZE;
    const long long grid = (long long)num_seqs * num_kv_heads * a.q_tiles;
    const PrefillSplit p = prefill_split_plan(num_seqs, num_kv_heads, a.q_tiles, max_context_len, key_split,
                                              a.bm.bits != nullptr);
    if (p.nsplit <= 1) return launch_status(pa::launch_prefill_mfma(a, head_dim, hs));
    size_t lse_off = 0;
    const size_t need = prefill_split_bytes(p, total_q, num_heads, head_dim, &lse_off);
    if (need == SIZE_MAX || grid * p.nsplit > 0x7fffffffll) return PA_ERR_SIZE;
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + lse_off);
    a.key_split = p.key_split;
    a.nsplit = p.nsplit;
    a.total_q = total_q;
    if ((st = launch_status(pa::launch_prefill_mfma(a, head_dim, hs)))) return st;
    return launch_status(pa::launch_prefill_split_merge(a, head_dim, hs));
  }
  // fp32 (and group sizes that do not divide 128): one query row per
  // wavefront over its whole admissible key range, no split.
  Shape s;
  s.g = g;
  s.GP = group_pad(g);
  s.NG = (g - 1) / s.GP + 1;
  s.split_log2 = kUnsplitLog2;
  s.P = 1;
  s.W = 0;
  s.wg = 0;
  s.FW = 0;
  if (product_exceeds({num_seqs, max_q_len, num_kv_heads, s.NG}, 0x7fffffffll)) return PA_ERR_SIZE;
  pa::RowAttnArgs a;
  fill_row_args(a, out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                cu_q_lens, num_seqs, max_q_len, num_heads, num_kv_heads, block_size, s, scale,
                causal, mods, nullptr, head_dim);
  a.num_blocks = num_blocks;
  return launch_status(pa::launch_row_partials(a, dtype, head_dim, hs));
}

}  // namespace

extern "C" {

int paged_attn_prefill(void* out, const void* q, const int32_t* cu_q_lens, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       int32_t block_table_stride, const int32_t* context_lens,
                       int32_t num_seqs, int32_t max_q_len, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, float scale, int32_t causal,
                       const pa_score_mods* mods, int32_t dtype, void* stream) {
  return prefill_impl(out, q, cu_q_lens, 0, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                      num_seqs, max_q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, 0, -1, scale,
                      causal, mods, nullptr, 0, dtype, stream);
}

size_t paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                                         int32_t key_split, int32_t dtype) {
  if (dtype != PA_BF16 || num_seqs <= 0 || total_q <= 0 || max_q_len <= 0 || max_context_len < 0 ||
      check_heads(num_heads, num_kv_heads) || check_dim(head_dim) || check_prefill_split(key_split))
    return 0;
  const int g = num_heads / num_kv_heads;
  if (128 % g != 0) return 0;
  const int q_tiles = (max_q_len - 1) / pa::prefill_rows_per_tile(g) + 1;
  if (product_exceeds({num_seqs, num_kv_heads, q_tiles}, 0x7fffffffll)) return 0;
  const PrefillSplit p = prefill_split_plan(num_seqs, num_kv_heads, q_tiles, max_context_len, key_split, false);
  const size_t n = prefill_split_bytes(p, total_q, num_heads, head_dim, nullptr);
  return n == SIZE_MAX ? 0 : n;
}

int paged_attn_prefill_split(void* out, const void* q, const int32_t* cu_q_lens, int32_t total_q,
                             const void* k_cache, const void* v_cache, const int32_t* block_tables,
                             int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_q_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int64_t num_blocks, int32_t max_context_len, int32_t key_split,
                             float scale, int32_t causal, const pa_score_mods* mods, void* workspace,
                             size_t workspace_bytes, int32_t dtype, void* stream) {
  return prefill_impl(out, q, cu_q_lens, total_q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                      num_seqs, max_q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_context_len, key_split, scale, causal, mods, workspace, workspace_bytes, dtype, stream);
}

size_t paged_attn_decode_cascade_workspace_size(int32_t num_seqs, const pa_prefix_level* levels,
                                                int32_t num_levels, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || max_context_len < 0 || check_heads(num_heads, num_kv_heads) || check_dim(head_dim) ||
      check_cascade_levels(num_seqs, levels, num_levels) || 128 % (num_heads / num_kv_heads) != 0)
    return 0;
  CascadeShape c;
  cascade_shape(num_seqs, levels, num_levels, num_heads, num_kv_heads, head_dim, max_context_len, c);
  return c.total;
}

int32_t paged_attn_decode_cascade_plan(int32_t num_seqs, const pa_prefix_level* levels, int32_t num_levels,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len) {
  if (num_seqs < 0 || max_context_len < 0 || check_heads(num_heads, num_kv_heads) || check_dim(head_dim) ||
      check_cascade_levels(num_seqs, levels, num_levels))
    return 0;
  return two_phase_pays_off(num_seqs, num_kv_heads, head_dim, max_context_len) ? 1 : 0;
}

int paged_attn_decode_cascade(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t num_seqs, const pa_prefix_level* levels,
                              int32_t num_levels, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, int32_t max_context_len, float scale,
                              const pa_score_mods* mods, void* workspace, size_t workspace_bytes, int32_t dtype,
                              void* stream) {
  return cascade_impl(false, out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs,
                      levels, num_levels, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_context_len, scale, mods, workspace, workspace_bytes, dtype, stream);
}

int paged_attn_decode_cascade_two_phase(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t block_table_stride,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        const pa_prefix_level* levels, int32_t num_levels, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int64_t num_blocks, int32_t max_context_len, float scale,
                                        const pa_score_mods* mods, void* workspace, size_t workspace_bytes,
                                        int32_t dtype, void* stream) {
  return cascade_impl(true, out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens, num_seqs,
                      levels, num_levels, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_context_len, scale, mods, workspace, workspace_bytes, dtype, stream);
}

}  // extern "C"

namespace {

int cascade_impl(bool force_two_phase, void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                 int32_t num_seqs, const pa_prefix_level* levels, int32_t num_levels, int32_t num_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                 int32_t max_context_len, float scale, const pa_score_mods* mods, void* workspace,
                 size_t workspace_bytes, int32_t dtype, void* stream) {
  int st = common_decode_checks(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                block_table_stride, max_context_len, 0, dtype, mods);
  if (st) return st;
  if (dtype != PA_BF16) return PA_ERR_DTYPE;
  if ((st = check_cascade_levels(num_seqs, levels, num_levels))) return st;
  const int g = num_heads / num_kv_heads;
  if (128 % g != 0) return PA_ERR_HEADS;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  for (int i = 0; i < num_levels; ++i)
    if (!levels[i].group_starts || !levels[i].prefix_ends) return PA_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PA_ERR_ALIGN;
  CascadeShape c;
  cascade_shape(num_seqs, levels, num_levels, num_heads, num_kv_heads, head_dim, max_context_len, c);
  if (!workspace || workspace_bytes < c.total || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return PA_ERR_WORKSPACE;
  const bool block_mask = mods && mods->block_mask;
  if (block_mask && force_two_phase) return PA_ERR_MODS;  // the shared parts take no block mask
  if (block_mask || !two_phase_pays_off(num_seqs, num_kv_heads, head_dim, max_context_len)) {
    // a batch this small is bound by launches, not by re-reading the shared
    // keys: the plain decode (one launch, or two) is faster; and a block mask
    // is taken by the plain decode only.  Its workspace is the region the
    // two-phase call keeps for its own-keys decode
    const size_t need = workspace_bytes_for(num_seqs, num_kv_heads, head_dim, c.dec);
    return decode_impl(true, true, out, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale,
                       0, mods, need > 0 ? static_cast<char*>(workspace) + c.off_dec : nullptr, need, dtype,
                       stream);
  }
  for (int i = 0; i < num_levels; ++i)
    if ((long long)levels[i].num_groups * num_kv_heads * c.lv[i].q_tiles * c.lv[i].nsplit > 0x7fffffffll)
      return PA_ERR_SIZE;
  if ((long long)num_seqs * num_heads > 0x7fffffffll) return PA_ERR_SIZE;
  char* ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_lse = reinterpret_cast<float*>(ws + c.off_part_lse);
  float* state_o = reinterpret_cast<float*>(ws + c.off_state_o);
  float* state_lse = reinterpret_cast<float*>(ws + c.off_state_lse);
  int32_t* key_start = reinterpret_cast<int32_t*>(ws + c.off_key_start);
  void* dec_ws = ws + c.off_dec;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const float softcap = mods ? mods->softcap : 0.f;
  const float* alibi = mods ? mods->alibi_slopes : nullptr;
  const int32_t window = mods ? mods->window : 0;
  const int32_t* doc_starts = mods ? mods->doc_starts : nullptr;
  const size_t plane = (size_t)num_seqs * num_heads;

  // 1) shared prefixes, level by level: the rows of a group are the query
  //    rows of one "sequence" whose keys are the group's range, read from the
  //    group's first member's table row, split into key ranges.  Each level
  //    leaves every row's range end as the next level's (and finally the
  //    suffix's) first key.
  for (int i = 0; i < num_levels; ++i) {
    const pa_prefix_level& v = levels[i];
    const CascadeLevel& l = c.lv[i];
    pa::PrefillArgs p;
    p.out = nullptr;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = v.prefix_ends;
    p.cu_q_lens = v.group_starts;
    p.alibi = alibi;
    p.prefix_lens = nullptr;  // (a decode row sees every earlier key anyway)
    p.doc_starts = doc_starts;
    p.bm = block_mask_args(nullptr);
    p.table_rows = v.group_starts;
    p.key_starts = v.prefix_starts;
    p.q_ctx = context_lens;
    p.num_cus = device_cus();
    p.part_o = part_o + (size_t)l.range0 * plane * head_dim;
    p.part_lse = part_lse + (size_t)l.range0 * plane;
    p.row_key_start = key_start;
    p.chain = i > 0;
    p.key_split = l.key_split;
    p.nsplit = l.nsplit;
    p.num_blocks = num_blocks;
    p.bt_stride = block_table_stride;
    p.num_seqs = v.num_groups;
    p.total_q = num_seqs;
    p.Hq = num_heads;
    p.Hkv = num_kv_heads;
    p.g = g;
    p.bs_log2 = ilog2(block_size);
    p.q_tiles = l.q_tiles;
    p.causal = 0;
    p.window = window;
    p.scale = scale;
    p.softcap = softcap;
    if ((st = launch_status(pa::launch_prefill_mfma(p, head_dim, hs)))) return st;
  }

  // 2) each sequence's own keys [last range end, n): the balanced decode with
  //    that end as a floor on every row's first admissible key (beside the
  //    caller's mods), leaving fp32 states
  pa::RowAttnArgs a;
  fill_row_args(a, nullptr, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                nullptr, num_seqs, 1, num_heads, num_kv_heads, block_size, c.dec, scale, 1, mods,
                workspace_bytes_for(num_seqs, num_kv_heads, head_dim, c.dec) > 0 ? dec_ws : nullptr,
                head_dim);
  a.row_floor = key_start;
  a.num_blocks = num_blocks;
  a.state_o = state_o;
  a.state_lse = state_lse;
  if ((st = launch_status(pa::launch_row_partials(a, dtype, head_dim, hs)))) return st;
  // (the balanced split's partials are merged by step 3 directly)
  if (c.dec.P > 1 && c.dec.W == 0) {
    if ((st = launch_status(pa::launch_row_merge(a, dtype, head_dim, hs)))) return st;
  }

  // 3) combine the key ranges' and the suffix's states into out
  pa::CascadeMergeArgs m;
  m.out = out;
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.state_o = state_o;
  m.state_lse = state_lse;
  m.ws_o = a.ws_o;
  m.ws_ml = a.ws_ml;
  m.ws_meta = c.dec.W > 0 ? a.ws_meta : nullptr;
  m.row_key_start = key_start;
  m.context_lens = context_lens;
  m.rows = num_seqs;
  m.Hq = num_heads;
  m.nsplit = c.nranges;
  m.Hkv = num_kv_heads;
  m.g = c.dec.g;
  m.NG = c.dec.NG;
  m.GP = c.dec.GP;
  return launch_status(pa::launch_cascade_merge(m, head_dim, hs));
}

}  // namespace

extern "C" {

const char* paged_attn_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SIZE: return "a count is negative or too large";
    case PA_ERR_HEADS: return "heads must be positive and num_heads a multiple of num_kv_heads";
    case PA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case PA_ERR_BLOCK_SIZE: return "block_size must be a power of two in [16, 256]";
    case PA_ERR_SPLIT:
      return "split_tokens must be 0, -1, -2 or a power of two >= 16 (key_split: 0, -1 or a multiple of 64)";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_DTYPE: return "dtype must be PA_F32 or PA_BF16";
    case PA_ERR_FLAG: return "causal must be 0 or 1";
    case PA_ERR_MODS: return "score mods: window and softcap must be finite and >= 0";
    case PA_ERR_TABLE_STRIDE: return "block_table_stride must be >= 1";
    case PA_ERR_NO_BLOCKS: return "block manager: no free block left in the pool";
    case PA_ERR_SEQ: return "block manager: unknown or freed sequence id";
    case PA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case PA_ERR_SCRATCH: return "the call needs more decode scratch than the library holds (16 MiB)";
    default: break;
  }
  if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
  return "unknown status";
}

}  // extern "C"
