// Paged (chunked) prefill on CDNA4 matrix cores, bf16 in / fp32 accumulate.
//
// A chunk of query rows per sequence attends to the sequence's paged context
// (the chunk's own keys are appended first).  The kernel gathers each key tile
// from the blocks the block table names, straight into LDS, and never builds a
// contiguous K/V copy (Joshi et al., "Paged Attention Meets FlexAttention",
// abstract: the fused kernel gathers scattered KV data; "Ultimate Guide to
// PagedAttention": block table).  Attention is exact, computed tile by tile
// with an online softmax (Dao et al., "FlashAttention", abstract).
//
// Work-group: 4 wavefronts, 128 query rows = QT = 128/g query positions x the
// g query heads of one kv-head, so every K/V tile read from HBM serves all g
// heads (GQA).  Two work-groups share a compute unit (<= 256 registers per
// lane, 64 KB of LDS each), so one's softmax overlaps the other's MFMAs.
// Per 64-key tile:
//   * the tile's K (64 x D) and V^T (D x 64) are fetched with direct-to-LDS
//     loads (global_load_lds_dwordx4) into one of two LDS buffers while the
//     previous tile is computed; each lane picks the global piece that must
//     land at its LDS slot, which is how the XOR swizzle is applied;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//     kept in registers); each lane then owns one query row's scores, so
//     softmax statistics are per-lane scalars;
//   * O^T += V^T P^T with the same MFMA (A = V^T rows from LDS -- V is
//     stored in dimension-major sub-slabs of 16 keys, so no transpose is
//     needed -- B = P^T straight from the S^T accumulators, rounded to bf16).
// The K rows of the S^T product are read in a permuted order inside each
// 16-key group (quarters 1 and 2 swapped) so that the accumulator registers
// a lane holds are exactly the 8 consecutive keys the next MFMA's B operand
// needs; no shuffles between the two products.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr uint32_t kBf16One2 = 0x3F803F80u;  // (1.0, 1.0) as a bf16 pair
constexpr int kTileKeys = 64;
constexpr int kRowsPerWG = 128;
constexpr int kThreads = 256;
constexpr int kWGsPerCU = 2;  // resident work-groups per compute unit (launch bounds)
// Score-mod instances: none (scale folded into the exponent), linear (scale
// and ALiBi bias), soft-capped (tanh cap, then the bias).  The soft cap is a
// compile-time choice: a run-time branch over both forms inside the
// pipelined step costs registers the step does not have.
constexpr int kModsNone = 0, kModsLinear = 1, kModsSoftcap = 2;

typedef __attribute__((address_space(3))) void* lds_ptr;
// Word 3 of a raw buffer resource (dword data, no swizzle) on this family.
constexpr int kBufferFlags = 0x00020000;

// 16 bytes per lane from base + voff + soff straight into LDS (lane i lands
// at dst + 16*i).  A buffer load rather than a global one: it counts only on
// the vector-memory counter, so waits for LDS reads issued while tile loads
// are in flight stay precise.  base and soff are wave-uniform.
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t voff, uint32_t soff, lds_ptr dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufferFlags), dst, 16, voff, soff, 0, 0);
}

// key slot (0..31) of a 32-key group -> key offset inside the group
__device__ __forceinline__ int key_of_slot(int u) {
  const int q = (u >> 2) & 3;
  const int qs = ((q & 1) << 1) | ((q >> 1) & 1);
  return (u & 16) | (qs << 2) | (u & 3);
}

// Offset (from k0 + 8*hl) of the key that accumulator element i of the
// S^T tile for key group kg holds: key_of_slot(8*(i/4) + 4*hl + i%4) + 32*kg
// with the hl term taken out.  A compile-time constant once unrolled.
__device__ __forceinline__ constexpr int key_off(int kg, int i) {
  return 32 * kg + 16 * ((i >> 3) & 1) + 4 * ((i >> 2) & 1) + (i & 3);
}

template <int P>
struct Par {
  static constexpr int value = P;
};

template <int KCH>
__device__ __forceinline__ int k_swz(int row, int c) { return c ^ (row & (KCH - 1) & 15); }
// The V^T tile is stored per tile-block j (the keys of one pool block, at
// most 64): [j][d][cpb chunks of 8 keys], cpb = min(bs, 64) / 8.  A row is
// cpb*16 bytes, so rows d and d + 16/cpb share banks: swizzle the chunk by
// d*cpb/16 to keep 16 consecutive rows on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int v_swz(int d, int cpb_log2) {
  return ((d << cpb_log2) >> 4) & ((1 << cpb_log2) - 1);
}

// KBL = log2(min(block_size, 64)): keys of one pool block inside a 64-key tile.
// kSplit: key-split mode (a.key_split > 0), a separate instance so that the
// plain prefill keeps its registers.
// kBM: the plain path with a block mask (the mods path takes one at run time).
template <int D, int kMods, int KBL, bool kSplit, bool kBM = false>
__global__ __launch_bounds__(kThreads, kWGsPerCU) void prefill_mfma_kernel(const PrefillArgs a, const int pair_tiles) {
  constexpr int KCH = D / 8;   // 16-byte chunks per K row
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;   // output 32-dim tiles
  constexpr int KPIECES = kTileKeys * KCH / kThreads;       // K pieces per thread per tile
  constexpr int VPIECES = D * (kTileKeys / 8) / kThreads;   // V^T pieces per thread per tile
  // Two K and two V tile buffers, each its own LDS object: the compiler can
  // then see that LDS reads of one buffer do not wait for the direct-to-LDS
  // loads in flight into the other.
  __shared__ u32x4 ktile0[kTileKeys * (D / 8)];  // [key][16-byte chunk], swizzled
  __shared__ u32x4 ktile1[kTileKeys * (D / 8)];
  __shared__ u32x4 vtile0[D * (kTileKeys / 8)];  // [tile-block][dim][8-key chunk], swizzled
  __shared__ u32x4 vtile1[D * (kTileKeys / 8)];
  auto kbuf = [&](auto P) -> u32x4* { if constexpr (decltype(P)::value == 0) return ktile0; else return ktile1; };
  auto vbuf = [&](auto P) -> u32x4* { if constexpr (decltype(P)::value == 0) return vtile0; else return vtile1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int hl = lane >> 5;      // half of the wave
  const int col = lane & 31;     // query row inside the wave's 32 rows

  const int QT = kRowsPerWG / a.g;
  const int BH = a.num_seqs * a.Hkv;
  constexpr bool ksplit = kSplit;
  const int split = ksplit ? blockIdx.x / (BH * a.q_tiles) : 0;  // key range
  const int flat = blockIdx.x - split * (BH * a.q_tiles);
  // Longest tiles first (causal rows further down see more keys).  When the
  // launcher finds the whole grid resident at once (pair_tiles), the second
  // half runs shortest first instead, so that work-groups i and i + half,
  // which tend to share a compute unit, hold tiles t and q_tiles - 1 - t.
  const int tslot = flat / BH;
  const int thalf = (a.q_tiles + 1) >> 1;
  const int qtile = (pair_tiles && tslot >= thalf) ? tslot - thalf : a.q_tiles - 1 - tslot;
  const int b = (flat % BH) / a.Hkv;
  const int kvh = flat % a.Hkv;

  // The sequence's lengths and the block-table entries of its first three
  // tiles, read together and waited for once: scalar loads return out of
  // order, so any use waits for all of them, and reading the entries only
  // after the work-group's key range is known would add a memory round trip.
  // Without a window, document starts or a key split every row's range starts
  // at key 0, and so does the first tile; an entry is used only then, and
  // only if its block lies within the sequence (see the prologue below).  The
  // index is clamped to the table row, so the read stays inside the table.
  const bool spec = !ksplit && a.window <= 0 && a.doc_starts == nullptr;
  const int n = a.context_lens[b];
  const int q0 = a.cu_q_lens[b];
  const int Lq = a.cu_q_lens[b + 1] - q0;
  int spec_blk[3];
  {
    const int32_t* row = a.block_tables + (size_t)b * a.bt_stride;
#pragma unroll
    for (int t = 0; t < 3; ++t)
      spec_blk[t] = __builtin_nontemporal_load(row + min((64 * t + 16 * wave) >> a.bs_log2, a.bt_stride - 1));
  }
  const int kstart = (ksplit && a.key_starts) ? a.key_starts[b] : 0;  // first key (key-split mode)
  asm volatile("" ::"s"(n), "s"(q0), "s"(Lq), "s"(kstart), "s"(spec_blk[0]), "s"(spec_blk[1]), "s"(spec_blk[2]));
  // (key-split mode: the sequences' rows must cover all total_q rows)
  PA_DEVICE_CHECK(!ksplit || ((b > 0 || q0 == 0) && (b + 1 < a.num_seqs || q0 + Lq == a.total_q) && Lq >= 0));
  const int q_start = qtile * QT;
  if (q_start >= Lq) return;
  PA_DEVICE_CHECK((ksplit || Lq <= n) && n >= 0 && (long long)n <= (long long)a.bt_stride << a.bs_log2);
  PA_DEVICE_CHECK(!ksplit || (kstart >= 0 && kstart <= n && (long long)(n - kstart) <= (long long)a.key_split * a.nsplit &&
                              Lq <= a.q_tiles * QT));

  // this lane's query row (column of S^T / O^T)
  const int r = wave * 32 + col;
  const int head_in = r / QT;
  const int qi = q_start + (r - head_in * QT);
  const bool row_ok = qi < Lq;
  // (key-split rows of decode rows sit at their own sequence's last position)
  const int pos = (ksplit && a.q_ctx) ? (row_ok ? a.q_ctx[q0 + qi] - 1 : 0) : n - Lq + qi;
  int row_hi = row_ok ? (a.causal ? min(n, pos + 1) : n) : 0;
  if (row_ok && a.causal && a.prefix_lens) row_hi = min(n, max(row_hi, a.prefix_lens[b]));
  int row_lo = (row_ok && a.window > 0) ? max(0, pos - a.window + 1) : 0;
  if (row_ok && a.doc_starts) row_lo = max(row_lo, a.doc_starts[q0 + qi]);
  if (ksplit) {
    // (64-bit: the last range may end past 2^31 keys)
    const long long range_lo = kstart + (long long)split * a.key_split;
    row_lo = (int)max((long long)row_lo, range_lo);
    row_hi = (int)min((long long)row_hi, range_lo + a.key_split);
    if (a.row_key_start && split == 0 && kvh == 0 && row_ok && head_in == 0 && hl == 0) {
      PA_DEVICE_CHECK(!a.chain || a.row_key_start[q0 + qi] == kstart);
      a.row_key_start[q0 + qi] = n;
    }
  }
  if (row_lo > row_hi) row_lo = row_hi;
  const int head = kvh * a.g + head_in;

  // Q^T operand (B of S^T): this lane's row, dims 16*ks + 8*hl .. +8 (read
  // here, so that it overlaps the work-group reduction below)
  bf16x8 qb[KSTEPS];
  {
    const char* qrow = static_cast<const char*>(a.q) + ((size_t)(q0 + (row_ok ? qi : 0)) * a.Hq + head) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 x = row_ok ? load16(qrow + (16 * ks + 8 * hl) * 2) : u32x4{0, 0, 0, 0};
      qb[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Key range of the whole work-group (uniform): keys [wg_lo, wg_hi) are
  // admissible for some row, keys [safe_lo, safe_hi) for every row.
  __shared__ int wg_bounds[4][4];
  int wg_lo, wg_hi, safe_lo, safe_hi;
  {
    int b0 = row_ok ? row_lo : 0x7fffffff, b1 = row_ok ? row_hi : 0;   // min lo, max hi
    int b2 = row_ok ? row_lo : 0, b3 = row_ok ? row_hi : 0x7fffffff;   // max lo, min hi
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      b0 = min(b0, __shfl_xor(b0, off, 64));
      b1 = max(b1, __shfl_xor(b1, off, 64));
      b2 = max(b2, __shfl_xor(b2, off, 64));
      b3 = min(b3, __shfl_xor(b3, off, 64));
    }
    if (lane == 0) {
      wg_bounds[wave][0] = b0;
      wg_bounds[wave][1] = b1;
      wg_bounds[wave][2] = b2;
      wg_bounds[wave][3] = b3;
    }
    __syncthreads();
    wg_lo = min(min(wg_bounds[0][0], wg_bounds[1][0]), min(wg_bounds[2][0], wg_bounds[3][0]));
    wg_hi = max(max(wg_bounds[0][1], wg_bounds[1][1]), max(wg_bounds[2][1], wg_bounds[3][1]));
    safe_lo = max(max(wg_bounds[0][2], wg_bounds[1][2]), max(wg_bounds[2][2], wg_bounds[3][2]));
    safe_hi = min(min(wg_bounds[0][3], wg_bounds[1][3]), min(wg_bounds[2][3], wg_bounds[3][3]));
    wg_lo = __builtin_amdgcn_readfirstlane(wg_lo);
    wg_hi = __builtin_amdgcn_readfirstlane(wg_hi);
    safe_lo = __builtin_amdgcn_readfirstlane(safe_lo);
    safe_hi = __builtin_amdgcn_readfirstlane(safe_hi);
  }

  const int32_t* table = a.block_tables + (size_t)((ksplit && a.table_rows) ? a.table_rows[b] : b) * a.bt_stride;
  const int bs = 1 << a.bs_log2;
  const size_t slab_bytes = (size_t)bs * D * 2;
  const char* kpool = static_cast<const char*>(a.k_cache) + (size_t)kvh * slab_bytes;
  const char* vpool = static_cast<const char*>(a.v_cache) + (size_t)kvh * slab_bytes;
  const size_t blk_stride = (size_t)a.Hkv * slab_bytes;
  const int last_blk = (n - 1) >> a.bs_log2;

  // Tile geometry: a 64-key tile covers nbt = 64/kb pool blocks of kb keys.
  constexpr int kb_log2 = KBL;
  constexpr int cpb_log2 = kb_log2 - 3;
  constexpr int cpb = 1 << cpb_log2;  // 8-key chunks per block row inside the tile
  constexpr int dcpb_log2 = cpb_log2 + (D == 128 ? 7 : 6);  // log2(D * cpb)

  // Direct-to-LDS loads of a tile.  Wave w fills K rows 16w..16w+15 and V^T
  // tile-block slots that hold keys of the same pool block (for bs = 16 the
  // tile-block is w itself), so one table entry per wave per tile -- the block
  // holding key k0 + 16w -- addresses all of its loads, and each instruction's
  // 64 lanes read one contiguous run.  Entries past the sequence's last block
  // are clamped to it (those keys are masked and their V entries zeroed).
  // Lane-dependent parts of the addresses are fixed for the whole loop.
  uint32_t k_off[KPIECES], v_off[VPIECES];
  int v_j[VPIECES];
#pragma unroll
  for (int it = 0; it < KPIECES; ++it) {
    const int rl = it * (64 / KCH) + lane / KCH;  // row - 16w
    const int c = (lane % KCH) ^ (rl & (KCH - 1) & 15);
    k_off[it] = (uint32_t)(rl * D + c * 8) * 2u;
  }
#pragma unroll
  for (int it = 0; it < VPIECES; ++it) {
    const int slot0 = (wave * VPIECES + it) * 64;
    v_j[it] = slot0 >> dcpb_log2;
    const int local = (slot0 & ((1 << dcpb_log2) - 1)) + lane;
    const int d = local >> cpb_log2;
    const int cc = (local & (cpb - 1)) ^ v_swz(d, cpb_log2);
    // keys 8cc..8cc+7 of the tile-block: sub-slab cc/2 (of 16 keys), row d, half cc%2
    v_off[it] = (uint32_t)(((cc >> 1) * D + d) * 16 + (cc & 1) * 8) * 2u;
  }
  auto issue_k = [&](int k0, auto buf, int blk) {
    const char* kb = kpool + (size_t)blk * blk_stride + (size_t)((k0 + 16 * wave) & (bs - 1)) * D * 2;
    char* lk = reinterpret_cast<char*>(kbuf(buf));
#pragma unroll
    for (int it = 0; it < KPIECES; ++it) {
      const int q = wave * KPIECES + it;
      buffer_load_lds16(kb, k_off[it], 0, (lds_ptr)(lk + q * 1024));
    }
  };
  auto issue_v = [&](int k0, auto buf, int blk) {
    const char* vb = vpool + (size_t)blk * blk_stride;
    char* lv = reinterpret_cast<char*>(vbuf(buf));
#pragma unroll
    for (int it = 0; it < VPIECES; ++it) {
      const int q = wave * VPIECES + it;
      // the tile-block's first key o sits at sub-slab o/16: o * D * 2 bytes in
      const uint32_t soff = (uint32_t)((k0 + (v_j[it] << kb_log2)) & (bs - 1)) * (uint32_t)(D * 2);
      buffer_load_lds16(vb, v_off[it], soff, (lds_ptr)(lv + q * 1024));
    }
  };

  const float scale_log2 = a.scale * kLog2e;
  float alibi_slope = 0.f;
  if constexpr (kMods) {
    if (a.alibi) alibi_slope = a.alibi[head];
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  const int k_begin = wg_lo & ~(kTileKeys - 1);
  const int ntiles_all = wg_hi > k_begin ? (wg_hi - k_begin + kTileKeys - 1) / kTileKeys : 0;
  // Block mask (mods instances only): the work-group visits only the key
  // tiles that some row's bitmap row admits, from a list built in LDS,
  // kBmListMax tiles of its range at a time.  Entry = the tile's first key,
  // | 1 when every row of the work-group admits the tile.
  constexpr int kBmListMax = (kMods || kBM) ? 2048 : 1;
  __shared__ int bm_list[kBmListMax];
  __shared__ int bm_count[4];
  const bool use_bm = (kMods || kBM) && a.bm.bits != nullptr;
  int ntiles = use_bm ? 0 : ntiles_all;
  auto tile_entry = [&](int t) { return __builtin_amdgcn_readfirstlane(bm_list[min(t, ntiles - 1)]); };
  auto tile_k0 = [&](int t) {
    if (use_bm) return tile_entry(t) & ~(kTileKeys - 1);
    return k_begin + min(t, ntiles - 1) * kTileKeys;
  };
  auto tile_full = [&](int k0) { return (k0 >= safe_lo) && (k0 + kTileKeys <= safe_hi); };
  auto tile_full_t = [&](int t) { return tile_full(tile_k0(t)) && (!use_bm || (tile_entry(t) & 1)); };
  // every row of the work-group admits tile t (always, without a block mask)
  auto tile_all_t = [&](int t) { return !use_bm || (tile_entry(t) & 1); };
  // A tile's raw list entry (first key | all-rows bit), for the step loop:
  // with a block mask it carries the entries of tiles t .. t+4 in scalar
  // registers and reads one more per step, a step before it is needed.
  auto raw_entry = [&](int t) { return tile_entry(t); };
  // this lane's bitmap row (valid rows only)
  const size_t bm_row = use_bm && row_ok ? ((size_t)b * a.bm.rows + (pos >> a.bm.q_log2)) * a.bm.words : 0;
  auto row_admits = [&](int k0) {
    const int kb = k0 >> a.bm.kv_log2;
    return ((a.bm.bits[bm_row + (kb >> 5)] >> (kb & 31)) & 1u) != 0;
  };
  // The list for tiles [seg * kBmListMax, ...) of the range: a tile goes in
  // when any of the work-group's bitmap rows admits its key block.
  auto bm_build = [&](int seg) {
    const int t0 = seg * kBmListMax;
    const int t1 = min(ntiles_all, t0 + kBmListMax);
    const int p_first = n - Lq + q_start;
    const int p_last = n - Lq + min(q_start + QT, Lq) - 1;
    const size_t r_lo = (size_t)b * a.bm.rows + (p_first >> a.bm.q_log2);
    const size_t r_hi = (size_t)b * a.bm.rows + (p_last >> a.bm.q_log2);
    __syncthreads();  // every wave is done with the previous segment's list
    int count = 0;
    for (int base = t0; base < t1; base += kThreads) {
      const int t = base + tid;
      const int k0 = k_begin + t * kTileKeys;
      bool any = false, all = true;
      if (t < t1) {
        const int kb = k0 >> a.bm.kv_log2;
        for (size_t r = r_lo; r <= r_hi; ++r) {
          const bool bit = ((a.bm.bits[r * a.bm.words + (kb >> 5)] >> (kb & 31)) & 1u) != 0;
          any |= bit;
          all &= bit;
        }
      }
      const uint64_t mask = __builtin_amdgcn_ballot_w64(any);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
      if (lane == 0) bm_count[wave] = __builtin_popcountll(mask);
      __syncthreads();
      int off = count;
      for (int w = 0; w < wave; ++w) off += bm_count[w];
      if (any) bm_list[off + below] = k0 | (all ? 1 : 0);
      count += bm_count[0] + bm_count[1] + bm_count[2] + bm_count[3];
      __syncthreads();  // the counts are read before the next round writes them
    }
    return count;
  };

  // S^T of one tile: 16 MFMAs, two independent accumulation chains.
  auto compute_s = [&](f32x16 (&S)[2], const u32x4* kt) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[kg][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        const int krow = 32 * kg + key_of_slot(col);
        const bf16x8 ka = __builtin_bit_cast(bf16x8, kt[krow * KCH + k_swz<KCH>(krow, 2 * ks + hl)]);
        S[kg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ks], S[kg], 0, 0, 0);
      }
    }
  };

  // Score mods (mods instances): a tile's raw scores to log2 units, s ->
  // (softcap(s * scale) + slope * (key - pos)) * log2(e), with softcap(x) =
  // c * tanh(x / c) written through exp2 and the hardware reciprocal
  // (tanh(y) = 1 - 2 / (e^{2y} + 1); an infinite e^{2y} gives 1).
  // Applied to S_{t+1} while the P.V MFMAs of tile t run, before its row
  // maxima and masks (a soft-capped -inf would be finite), so the rest of the
  // pipelined step is the plain path's with a unit exponent scale.
  const float mod_sc = a.scale * kLog2e;
  const float mod_cap_in = a.softcap > 0.f ? 2.f * kLog2e * a.scale / a.softcap : 0.f;
  const float mod_cap_out = a.softcap * kLog2e;
  const float mod_al = alibi_slope * kLog2e;
  auto transform = [&](f32x16 (&S)[2], const int k0) {
    const float base = mod_al * (float)(k0 + 8 * hl - pos);
    if constexpr (kMods == kModsSoftcap) {
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float ez = fast_exp2(S[kg][i] * mod_cap_in);
          const float th = fmaf(-2.f, __builtin_amdgcn_rcpf(ez + 1.f), 1.f);  // tanh(x / c)
          S[kg][i] = fmaf(mod_cap_out, th, fmaf(mod_al, (float)key_off(kg, i), base));
        }
    } else {
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          S[kg][i] = fmaf(S[kg][i], mod_sc, fmaf(mod_al, (float)key_off(kg, i), base));
    }
  };

  // O^T += V^T P^T: 16 MFMAs, DT independent accumulation chains.
  auto pv = [&](const u32x4* vt, const bf16x8 (&pb)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + col;
        const int c = 2 * s + hl;  // 8-key chunk of the tile
        const int j = c >> cpb_log2;
        const int cc = c & (cpb - 1);
        const bf16x8 va = __builtin_bit_cast(bf16x8, vt[(((j * D + d) << cpb_log2) | (cc ^ v_swz(d, cpb_log2)))]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s], oacc[dt], 0, 0, 0);
      }
    }
  };

  // V^T entries of keys >= n hold whatever the pool had: zero them (P is 0 there)
  auto fixup_v = [&](const int k0, auto buf) {
#pragma unroll
    for (int it = 0; it < VPIECES; ++it) {
      const int p = it * kThreads + tid;
      const int j = p >> dcpb_log2;
      const int local = p - (j << dcpb_log2);
      const int d = local >> cpb_log2;
      const int cc = (local & (cpb - 1)) ^ v_swz(d, cpb_log2);
      const int tok = k0 + (j << kb_log2) + 8 * cc;
      if (tok + 8 > n) {
        u32x4 x = vbuf(buf)[p];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int jj = tok + 2 * w;
          x[w] &= (jj < n ? 0xffffu : 0u) | (jj + 1 < n ? 0xffff0000u : 0u);
        }
        vbuf(buf)[p] = x;
      }
    }
  };

  auto wait_tiles = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct-to-LDS loads landed
    __syncthreads();                      // ... and every other wave's
    __asm__ volatile("" ::: "memory");
  };

  // Row maximum of a tile's raw scores (log2 units after the scale).
  auto row_max = [&](const f32x16 (&S)[2]) {
    float c = kNegInf;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int i = 0; i < 16; ++i) c = fmaxf(c, S[kg][i]);
    return fmaxf(c, shfl_xor32(c)) * (kMods ? 1.f : scale_log2);
  };
  // Keys outside this row's admissible range -> -inf (raw scores); a whole
  // tile for a row whose block-mask row does not admit it.
  auto mask_s = [&](f32x16 (&S)[2], const int k0, const bool all_rows) {
    const int kb = k0 + 8 * hl;
    const int lo = row_lo - kb, hi = row_hi - kb;
    const bool admits = all_rows || (row_ok && row_admits(k0));
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = key_off(kg, i);
        if (!admits || c < lo || c >= hi) S[kg][i] = kNegInf;
      }
  };
  // Lazy running-max update: the max moves only when a tile exceeds it by
  // kLazyRescale (log2 units); then O and l are rescaled.
  auto update_max = [&](const float cmax) {
    const float m_new = fmaxf(m_run, cmax);
    const bool need = m_new > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      if (need) m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
  };
  // Table entry of the block wave `wave` loads for tile t, read with a vector
  // load (all lanes, one address) so that waiting for it joins the wait for
  // the tile loads instead of the LDS counter.
  auto table_load_k = [&](int k0) {
    const int j = min((k0 + 16 * wave) >> a.bs_log2, last_blk);
    const int blk = __builtin_nontemporal_load(table + j);
    PA_DEVICE_CHECK(blk >= 0 && blk < a.num_blocks);
    return blk;
  };
  auto table_load = [&](int t) {
    const int j = min((tile_k0(t) + 16 * wave) >> a.bs_log2, last_blk);
    const int blk = __builtin_nontemporal_load(table + j);
    PA_DEVICE_CHECK(blk >= 0 && blk < a.num_blocks);
    return blk;
  };

  // Software pipeline over tiles (per wave).  Plain path, iteration t, one
  // basic block after the barrier: the loads of K_{t+2} and V_{t+1}, the
  // S_{t+1} MFMAs with the exp/convert of P_t, then the O += V_t P_t MFMAs
  // with the row maxima of S_{t+1}.  On entry S_t is masked and the running
  // max covers it.  LDS rings: K holds tiles t+1 (read) and t+2 (landing), V
  // holds tiles t (read) and t+1 (landing).  Block ids: b1 = tile t+1,
  // b2 = tile t+2 (scalars), bv = tile t+3 (vector load in flight).
  const int nseg = use_bm ? (ntiles_all + kBmListMax - 1) / kBmListMax : 1;
  for (int seg = 0; seg < nseg; ++seg) {
  if (use_bm) ntiles = bm_build(seg);
  f32x16 sA[2], sB[2];
  int b1 = 0, b2 = 0, bv = 0;
  int ent[5] = {0, 0, 0, 0, 0};  // raw entries of tiles t .. t+4 (step loop)
  if (ntiles > 0) {
    // the entries read at entry hold for tile t if the range starts at key 0,
    // the tile exists and its block for this wave is within the sequence
    auto first_entry = [&](int t) {
      if (spec && k_begin == 0 && t < ntiles && (!use_bm || tile_k0(t) == kTileKeys * t) &&
          ((64 * t + 16 * wave) >> a.bs_log2) <= last_blk) {
        PA_DEVICE_CHECK(spec_blk[t] >= 0 && spec_blk[t] < a.num_blocks);
        return spec_blk[t];
      }
      return table_load(t);
    };
    const int b0 = __builtin_amdgcn_readfirstlane(first_entry(0));
    b1 = __builtin_amdgcn_readfirstlane(first_entry(1));
    b2 = __builtin_amdgcn_readfirstlane(first_entry(2));
    issue_k(tile_k0(0), Par<0>{}, b0);
    issue_v(tile_k0(0), Par<0>{}, b0);
    if (ntiles > 1) issue_k(tile_k0(1), Par<1>{}, b1);
    bv = table_load(3);
    wait_tiles();
    compute_s(sA, ktile0);
    if constexpr (kMods) transform(sA, tile_k0(0));
    if (!tile_full_t(0)) mask_s(sA, tile_k0(0), tile_all_t(0));
    update_max(row_max(sA));
  }
  if (use_bm && ntiles > 0) {
#pragma unroll
    for (int i = 0; i < 5; ++i) ent[i] = raw_entry(i);
  }
  // P = t & 1 (compile time): K buffer 1-P is read, P receives tile t+2;
  // V buffer P is read, 1-P receives tile t+1.
  auto step = [&](auto P, f32x16 (&Scur)[2], f32x16 (&Snext)[2], const int t) {
    constexpr Par<1 - decltype(P)::value> Q{};
    // With a block mask, tiles t .. t+4 come from the carried entries and the
    // entry of tile t+5 is read from LDS now, for the next step; without
    // one, the tiles are consecutive from the range's first key.
    const int k0 = use_bm ? ent[0] & ~(kTileKeys - 1) : tile_k0(t);
    const int k1 = use_bm ? ent[1] & ~(kTileKeys - 1) : tile_k0(t + 1);
    const int k2 = use_bm ? ent[2] & ~(kTileKeys - 1) : tile_k0(t + 2);
    const int k4 = use_bm ? ent[4] & ~(kTileKeys - 1) : tile_k0(t + 4);
    const bool all1 = !use_bm || (ent[1] & 1) != 0;
    const bool full1 = tile_full(k1) && all1;
    const int e5 = use_bm ? raw_entry(t + 5) : 0;
    wait_tiles();  // K_{t+1}, V_t and the table entry bv landed; all waves are past iteration t-1
    const int b3 = __builtin_amdgcn_readfirstlane(bv);
    if (k0 + kTileKeys > n) {
      fixup_v(k0, P);
      __syncthreads();
    }
    bf16x8 pb[4];
    {
      // Loads of K_{t+2} and V_{t+1}, unconditional so that they join this
      // block: past the last tile they reload it into buffers nobody reads
      // any more.  S_{t+1} (on the last tile from a stale K buffer, never
      // used) and P_t.  Without mods s * scale * log2(e) is folded into the
      // exp argument (scale > 0 there); with mods S_t is already in log2
      // units.  The row sum adds the bf16-rounded weights that enter P.V (a
      // dot2 of each packed pair with (1, 1)), so the weights sum to one and
      // a row whose weight sits on one key returns that key's V row.
      issue_k(k2, P, b2);
      issue_v(k1, Q, b1);
      b1 = b2;
      b2 = b3;
      bv = table_load_k(k4);
      compute_s(Snext, kbuf(Q));
      const float nm = (m_run == kNegInf) ? 0.f : -m_run;
      float psum = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(fmaf(Scur[s >> 1][8 * (s & 1) + 2 * j], kMods ? 1.f : scale_log2, nm));
          const float p1 = fast_exp2(fmaf(Scur[s >> 1][8 * (s & 1) + 2 * j + 1], kMods ? 1.f : scale_log2, nm));
          w[j] = cvt_bf16x2(p0, p1);
          psum = dot2_bf16(w[j], kBf16One2, psum);
        }
        pb[s] = __builtin_bit_cast(bf16x8, w);
      }
      l_run += psum;
      pv(vbuf(P), pb);
      if constexpr (kMods) transform(Snext, k1);
      float cmax = row_max(Snext);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads ahead
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (S)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU (P)
        if (i < KPIECES + VPIECES + 1)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (tile loads, table)
      }
#pragma unroll
      for (int i = 0; i < 4 * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA (PV)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, kMods ? 6 : 3, 0);  // VALU (mods, row max)
      }
      if (t + 1 < ntiles) {  // (S_{t+1} of the last tile is stale: no update)
        if (!full1) {  // rare: maxima over admissible keys only
          mask_s(Snext, k1, all1);
          cmax = row_max(Snext);
        }
        update_max(cmax);
      }
    }
    ent[0] = ent[1];
    ent[1] = ent[2];
    ent[2] = ent[3];
    ent[3] = ent[4];
    ent[4] = e5;
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(Par<0>{}, sA, sB, t);
    if (t + 1 < ntiles) step(Par<1>{}, sB, sA, t + 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no direct-to-LDS load outlives the loop
  }  // segments of the block-mask tile list

  // ---- normalise and store: lane holds row `r`, dims 32dt + 8(i/4) + 4hl + i%4 ----
  const float l_tot = l_run + shfl_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (ksplit) {
    if (!row_ok) return;
    // this key range's state: normalised output and log-sum-exp, fp32
    const size_t prow = ((size_t)split * a.total_q + q0 + qi) * a.Hq + head;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * hl;
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = oacc[dt][4 * g4 + i] * inv;
        *reinterpret_cast<f32x4*>(po + d) = w;
      }
    }
    if (hl == 0) a.part_lse[prow] = state_lse2(m_run, l_tot);
  } else {
    // The rows go through LDS (the K tile buffers, free now: every wave has
    // waited for its own tile loads above) so that each store instruction
    // writes whole rows: a lane's accumulators hold 8-byte pieces of one row,
    // and stores of such pieces, one row per lane, cost more than the
    // transpose.  Rows r < 64 sit in ktile0, the rest in ktile1, their 16-byte
    // chunks swizzled as the K tiles are, so that writes down a column spread
    // over the banks.
    // The stores are non-temporal: nothing here reads the output again.
    __syncthreads();  // every wave is done reading the tiles
    char* srow = reinterpret_cast<char*>(r < 64 ? ktile0 : ktile1) + (size_t)(r & 63) * (D * 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        uint2 w;
        w.x = cvt_bf16x2(oacc[dt][4 * g4 + 0] * inv, oacc[dt][4 * g4 + 1] * inv);
        w.y = cvt_bf16x2(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(srow + k_swz<KCH>(r, 4 * dt + g4) * 16 + hl * 8) = w;
      }
    }
    __syncthreads();
    // 16-byte chunk e of the work-group's output, ordered (query position,
    // head, chunk): the g heads of one position are one contiguous run
    // (g * QT = 128: the matrix-core path takes only such groups)
    const int g = a.g;
#pragma unroll
    for (int k = 0; k < kRowsPerWG * KCH / kThreads; ++k) {
      const int e = k * kThreads + tid;
      const int c = e % KCH;
      const int hi = (e / KCH) % g;
      const int ql = e / (KCH * g);
      const int rr = hi * QT + ql;
      if (q_start + ql < Lq) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(rr < 64 ? ktile0 : ktile1) +
                                                        (size_t)(rr & 63) * (D * 2) + k_swz<KCH>(rr, c) * 16);
        char* dst = static_cast<char*>(a.out) + ((size_t)(q0 + q_start + ql) * a.Hq + kvh * g + hi) * D * 2 + c * 16;
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dst));
      }
    }
  }
}

// Key-split prefill, last step: one wavefront per (row, query head) combines
// the row's nsplit range states, each a normalised output o_s with its
// log-sum-exp lse_s (log2 units), as sum_s 2^(lse_s - M) o_s / sum_s
// 2^(lse_s - M), M = max_s lse_s, in range order; a row no range admits any
// key of gets zeros (every lse_s is -inf).  Four wavefronts per work-group.
template <int D>
__global__ __launch_bounds__(256) void prefill_split_merge_kernel(const PrefillArgs a) {
  constexpr int R = D / 64;  // dimensions per lane
  constexpr int U = 4;       // states whose loads are in flight together
  const int lane = threadIdx.x & 63;
  const size_t plane = (size_t)a.total_q * a.Hq;
  const size_t rh = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row * Hq + head
  if (rh >= plane) return;
  float M = kNegInf;
  for (int s = lane; s < a.nsplit; s += 64) M = fmaxf(M, a.part_lse[(size_t)s * plane + rh]);
  M = wave_max(M);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
    for (int s0 = 0; s0 < a.nsplit; s0 += U) {
      float w[U], x[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = min(s0 + u, a.nsplit - 1);
        const float lse = a.part_lse[(size_t)s * plane + rh];
        w[u] = (s0 + u < a.nsplit) ? fast_exp2(lse - M) : 0.f;
        const float* o = a.part_o + ((size_t)s * plane + rh) * D;
#pragma unroll
        for (int r = 0; r < R; ++r) x[u][r] = o[lane + 64 * r];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        L += w[u];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = fmaf(w[u], x[u][r], acc[r]);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + rh * D;
#pragma unroll
  for (int r = 0; r < R; ++r) orow[lane + 64 * r] = (uint16_t)f32_to_bf16_bits(acc[r] * inv);
}

}  // namespace

int prefill_rows_per_tile(int g) { return kRowsPerWG / g; }

hipError_t launch_prefill_split_merge(const PrefillArgs& a, int D, hipStream_t s) {
  const long long pairs = (long long)a.total_q * a.Hq;
  if (pairs <= 0 || a.nsplit <= 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
  if (D == 64)
    hipLaunchKernelGGL((prefill_split_merge_kernel<64>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((prefill_split_merge_kernel<128>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int D, hipStream_t s) {
  const long long blocks = (long long)a.num_seqs * a.Hkv * a.q_tiles * (a.key_split > 0 ? a.nsplit : 1);
  if (blocks <= 0) return hipSuccess;
  // the fast path folds a positive scale into the exponent; a block mask
  // takes the fast path's block-mask instance, or the mods path with mods
  const int mods = a.softcap > 0.f ? kModsSoftcap
                   : (a.alibi != nullptr || !(a.scale > 0.f)) ? kModsLinear : kModsNone;
  const bool bm = a.bm.bits != nullptr;
  const int kbl = a.bs_log2 < 6 ? a.bs_log2 : 6;
  const bool split = a.key_split > 0;
  const dim3 grid((unsigned)blocks), block(kThreads);
  const int pair = !split && blocks <= (long long)kWGsPerCU * a.num_cus;
#define PA_PREFILL_LAUNCH(DD, MM, KK)                                                                 \
  do {                                                                                                \
    if (split)                                                                                        \
      hipLaunchKernelGGL((prefill_mfma_kernel<DD, MM, KK, true>), grid, block, 0, s, a, pair);         \
    else if (!(MM) && bm)                                                                             \
      hipLaunchKernelGGL((prefill_mfma_kernel<DD, kModsNone, KK, false, true>), grid, block, 0, s, a, pair); \
    else                                                                                              \
      hipLaunchKernelGGL((prefill_mfma_kernel<DD, MM, KK, false>), grid, block, 0, s, a, pair);        \
  } while (0)
#define PA_PREFILL_KBL(DD, MM)                    \
  switch (kbl) {                                  \
    case 4: PA_PREFILL_LAUNCH(DD, MM, 4); break;  \
    case 5: PA_PREFILL_LAUNCH(DD, MM, 5); break;  \
    default: PA_PREFILL_LAUNCH(DD, MM, 6); break; \
  }
  if (D == 64) {
    if (mods == kModsSoftcap) { PA_PREFILL_KBL(64, kModsSoftcap) }
    else if (mods == kModsLinear) { PA_PREFILL_KBL(64, kModsLinear) }
    else { PA_PREFILL_KBL(64, kModsNone) }
  } else {
    if (mods == kModsSoftcap) { PA_PREFILL_KBL(128, kModsSoftcap) }
    else if (mods == kModsLinear) { PA_PREFILL_KBL(128, kModsLinear) }
    else { PA_PREFILL_KBL(128, kModsNone) }
  }
#undef PA_PREFILL_KBL
#undef PA_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace pa
