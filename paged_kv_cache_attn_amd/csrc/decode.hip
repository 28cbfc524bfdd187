// Paged attention for query rows that each attend to (a range of) their own
// sequence's paged context: decode (one row per sequence) and the fp32 path
// of prefill (one row per query position).  gfx950 / CDNA4, wave64.
//
// Method: attention reads the K/V blocks of a sequence where they lie in the
// shared pool, found through the block table, with no contiguous copy
// (Joshi et al., "Paged Attention Meets FlexAttention", abstract; "Ultimate
// Guide to PagedAttention", block table), computing exact softmax attention
// with a running (online) softmax over tiles of keys (Dao et al.,
// "FlashAttention", abstract: tiling between HBM and on-chip memory).
//
// Work decomposition (one wavefront = one work-group):
//   (row slot, head group, partition) -- a head group is the GP <= 8 query
//   heads of one kv-head, so each K/V byte is read once for all of them;
//   a partition is 2^split_log2 consecutive keys (split-KV).
// Per 16-token chunk (always inside one block, since block sizes are powers
// of two >= 16):
//   * q.k on VALU: GP lanes share a token, each holding 1/GP of head_dim for
//     all GP heads; bf16 uses v_dot2_f32_bf16.  A reduce-scatter across the
//     GP lanes (DPP row_ror:8, permlane16_swap, permlane32_swap) leaves each
//     lane with one head's full score, with no select instructions: q rows
//     are loaded in a lane-dependent order that makes every step an add.
//   * online softmax in the log2 domain; the running max is raised lazily
//     (only when a new score exceeds it by more than 2^8), so rescaling of
//     the accumulators is rare after the first chunk.
//   * P.V with lanes over head_dim: V is stored in dimension-major sub-slabs
//     of 16 tokens, so one dword holds two consecutive tokens of one
//     dimension -- exactly the bf16 pair v_dot2 wants against a (p_j, p_j+1)
//     pair read from LDS -- and a chunk's V is one contiguous run whatever
//     the page size.
#include "pa_device.h"
#include "pa_kernels.h"



namespace pa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units

template <typename E, int D, int GP>
struct Cfg {
  static constexpr int ES = E::kBytes;
  static constexpr bool kBf16 = (ES == 2);
  static constexpr int kRowBytes = D * ES;        // one K row
  static constexpr int kPieces = kRowBytes / 16;  // 16-byte pieces per K row
  static constexpr int TPI = 64 / GP;             // tokens per pass
  static constexpr int NPASS = 16 / TPI;          // passes per 16-token chunk
  static constexpr int PPL = kPieces / GP;        // pieces per lane per token
  // P.V: lane = (dimension row vr = lane/2, token half vh = lane%2); a V row
  // of one 16-token chunk is 16*ES bytes, so the two halves of a wave's 32
  // rows are one contiguous run when the block holds exactly the chunk.
  static constexpr int RPL = D / 32;              // V rows (dims) per lane
  static constexpr int VPR = 8 * ES / 16;         // 16-byte loads per (row, 8 tokens)
  static_assert(PPL >= 1 && RPL >= 1, "unsupported shape");
};

template <typename E, int D, int GP>
struct Chunk {
  using C = Cfg<E, D, GP>;
  u32x4 k[C::NPASS][C::PPL];
  u32x4 v[C::RPL][C::VPR];
};

// Which head (0..GP-1 within the group) lane group e holds after the reduce.
template <int GP>
__device__ __forceinline__ int final_head(int e) {
  if constexpr (GP == 8) {
    return ((e & 1) << 2) | (e & 2) | ((e >> 2) & 1);
  } else {
    return ((e & 1) << 1) | ((e >> 1) & 1);
  }
}

// Head loaded into q slot s by lane group e (makes every reduce step an add).
template <int GP>
__device__ __forceinline__ int slot_head(int s, int e) {
  if constexpr (GP == 8) return (e & 1) ? (s ^ 4) : s;
  return s;
}

template <int GP>
__device__ __forceinline__ float reduce_scatter(const float (&acc)[GP]) {
  if constexpr (GP == 8) {
    float r4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r4[k] = acc[k] + dpp<kDppRowRor8>(acc[k + 4]);
    float r2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) r2[k] = swap_add16(r4[k], r4[k + 2]);
    return swap_add32(r2[0], r2[1]);
  } else {
    float r2[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) r2[k] = swap_add16(acc[k], acc[k + 2]);
    return swap_add32(r2[0], r2[1]);
  }
}

// max / sum over the TPI consecutive lanes that hold one head
template <int TPI, bool kMax>
__device__ __forceinline__ float group_reduce(float x) {
  auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
  x = op(x, dpp<kDppQuadXor1>(x));
  x = op(x, dpp<kDppQuadXor2>(x));
  x = op(x, dpp<kDppRowHalfMirror>(x));
  if constexpr (TPI == 16) x = op(x, dpp<kDppRowMirror>(x));
  return x;
}

struct RowRange {
  int qrow;   // query / output row
  int pos;    // logical position of the query
  int lo;     // first admissible key
  int hi;     // one past the last admissible key
  int start;  // lo rounded down to a chunk
  int nparts; // partitions the row uses (>= 1)
};

__device__ __forceinline__ bool row_range(const RowAttnArgs& a, int slot, RowRange& r) {
  const int b = slot / a.max_q_len;
  const int i = slot - b * a.max_q_len;
  const int n = a.context_lens[b];
  int Lq = 1, q0 = b;
  if (a.cu_q_lens) {
    q0 = a.cu_q_lens[b];
    Lq = a.cu_q_lens[b + 1] - q0;
  }
  if (i >= Lq) return false;
  // (a decode row may have no key at all; prefill rows sit inside the context;
  // a merge-only launch has no block table, so no table extent to check)
  PA_DEVICE_CHECK(n >= 0 && (!a.block_tables || (long long)n <= (long long)a.bt_stride << a.bs_log2) &&
                  (!a.cu_q_lens || Lq <= n));
  r.qrow = q0 + i;
  r.pos = n - Lq + i;
  r.hi = a.causal ? min(n, r.pos + 1) : n;
  if (a.causal && a.prefix_lens) r.hi = min(n, max(r.hi, a.prefix_lens[b]));
  r.lo = a.window > 0 ? max(0, r.pos - a.window + 1) : 0;
  if (a.doc_starts) r.lo = max(r.lo, a.doc_starts[r.qrow]);
  if (a.row_floor) r.lo = max(r.lo, a.row_floor[r.qrow]);
  if (r.hi < 0) r.hi = 0;
  if (r.lo > r.hi) r.lo = r.hi;
  r.start = r.lo & ~15;
  const int span = r.hi - r.start;
  r.nparts = span > 0 ? ((span + (1 << a.split_log2) - 1) >> a.split_log2) : 1;
  // a context longer than the host's max_context_len breaks the caller
  // contract; clamping keeps every workspace access inside the buffer
  r.nparts = min(r.nparts, a.P);
  return true;
}

// Instances of the row kernels (template argument kMods): no score mods; the
// soft-cap / ALiBi score mods (unconditional chunk loads, like the plain
// path); those mods plus a block mask (chunks a row's bitmap does not admit
// are skipped, so loads are conditional and the pipeline waits follow them).
constexpr int kModsNone = 0, kModsScore = 1, kModsBlockMask = 2;

// Attention of one row slot over keys [c_begin, c_end) (a segment of its
// admissible range), for the GP query heads of head group hg.  Writes the
// normalised output when the segment is the whole range (`whole`), else the
// unnormalised partial (o, m, l) at workspace unit `unit`; with kToLds the
// unnormalised state goes to this wavefront's LDS slots instead (o as
// [GP][D] in lds_o, (m, l) per head in lds_ml) for a work-group merge.
template <typename E, int D, int GP, int kMods, bool kToLds = false>
__device__ __forceinline__ void attend_segment(const RowAttnArgs& a, const RowRange& rr, const int slot,
                                               const int hg, const int c_begin, const int c_end,
                                               const bool whole, const size_t unit, uint32_t* p_lds,
                                               float* stat_lds, float* lds_o = nullptr,
                                               float* lds_ml = nullptr) {
  using C = Cfg<E, D, GP>;
  constexpr int TPI = C::TPI;
  const int lane = threadIdx.x & 63;
  const int kvh = hg / a.NG;
  const int head0 = kvh * a.g + (hg - kvh * a.NG) * GP;  // first global head of the group
  const int nvalid = min(GP, a.g - (hg - kvh * a.NG) * GP);

  const int t = lane % TPI;
  const int e = lane / TPI;
  const int my_head = final_head<GP>(e);
  const int vh = lane & 1;   // token half for P.V
  const int vr = lane >> 1;  // first V row for P.V

  // ---- q slice of every head in the group (lane-dependent head order) ----
  u32x4 qv[GP][C::PPL];
  {
    const char* qbase = static_cast<const char*>(a.q) + (size_t)rr.qrow * a.Hq * D * C::ES;
#pragma unroll
    for (int s = 0; s < GP; ++s) {
      const int h = slot_head<GP>(s, e);
#pragma unroll
      for (int i = 0; i < C::PPL; ++i) {
        if (h < nvalid) {
          qv[s][i] = load16(qbase + ((size_t)(head0 + h) * D) * C::ES + (e + GP * i) * 16);
        } else {
          qv[s][i] = u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  const float scale_log2 = a.scale * kLog2e;
  float alibi_slope = 0.f;
  if constexpr (kMods) {
    if (a.alibi && my_head < nvalid) alibi_slope = a.alibi[head0 + my_head];
  }

  float m_run = kNegInf;  // log2 domain, for head my_head
  float l_run = 0.f;      // partial sum over this lane's tokens
  float o[GP][C::RPL];  // rows d = vr + 32 r, over this lane's token half
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int r = 0; r < C::RPL; ++r) o[h][r] = 0.f;

  const int b = slot / a.max_q_len;
  const int n = a.context_lens[b];
  const int32_t* table = a.block_tables + (size_t)b * a.bt_stride;
  const int bs = 1 << a.bs_log2;
  const size_t kslab_bytes = (size_t)bs * D * C::ES;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);

  auto load_chunk = [&](Chunk<E, D, GP>& ch, int tok0) {
    const int blk = load_ro_i32(table, tok0 >> a.bs_log2);
    PA_DEVICE_CHECK(blk >= 0 && blk < a.num_blocks);
    const int off = tok0 & (bs - 1);
    const size_t slab = ((size_t)blk * a.Hkv + kvh) * kslab_bytes;
    const char* ks = kpool + slab + (size_t)off * C::kRowBytes;
    const char* vs = vpool + slab + (size_t)(off >> 4) * (D * 16 * C::ES);  // the chunk's V sub-slab
#pragma unroll
    for (int ps = 0; ps < C::NPASS; ++ps)
#pragma unroll
      for (int i = 0; i < C::PPL; ++i)
        ch.k[ps][i] = load16_stream(ks + (ps * TPI + t) * C::kRowBytes + (e + GP * i) * 16);
#pragma unroll
    for (int r = 0; r < C::RPL; ++r)
#pragma unroll
      for (int w = 0; w < C::VPR; ++w)
        ch.v[r][w] = load16_stream(vs + ((size_t)(vr + 32 * r) * 16 + vh * 8) * C::ES + w * 16);
  };

  // one 16-token chunk: scores, online softmax, P.V.  A chunk that starts at
  // or past c_end is entirely masked and leaves the state unchanged.
  auto process = [&](Chunk<E, D, GP>& cur, const int tok0) {

    // ---- scores for this lane's tokens, head my_head ----
    float s[C::NPASS];
#pragma unroll
    for (int ps = 0; ps < C::NPASS; ++ps) {
      float acc[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < C::PPL; ++i) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (C::kBf16) {
              x = dot2_bf16(qv[h][i][w], cur.k[ps][i][w], x);
            } else {
              x = fmaf(__uint_as_float(qv[h][i][w]), __uint_as_float(cur.k[ps][i][w]), x);
            }
          }
        }
        acc[h] = x;
      }
      const float dotv = reduce_scatter<GP>(acc);
      const int tok = tok0 + ps * TPI + t;
      float sc;
      if constexpr (kMods) {
        float x = dotv * a.scale;
        if (a.softcap > 0.f) {
          const float z = x / a.softcap;
          const float ez = fast_exp2(2.f * kLog2e * z);
          x = a.softcap * (1.f - 2.f / (ez + 1.f));
        }
        x += alibi_slope * (float)(tok - rr.pos);
        sc = x * kLog2e;
      } else {
        sc = dotv * scale_log2;
      }
      const bool ok = (tok >= rr.lo) && (tok < c_end);
      s[ps] = ok ? sc : kNegInf;
    }

    // ---- online softmax (lazy max) ----
    float cmax = s[0];
#pragma unroll
    for (int ps = 1; ps < C::NPASS; ++ps) cmax = fmaxf(cmax, s[ps]);
    cmax = group_reduce<TPI, true>(cmax);
    const float m_new = fmaxf(m_run, cmax);
    const bool need = m_new > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      if (need) m_run = m_new;
      l_run *= alpha;
      if (t == 0) stat_lds[my_head] = alpha;
      __builtin_amdgcn_wave_barrier();
      float al[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) al[h] = stat_lds[h];
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int r = 0; r < C::RPL; ++r) o[h][r] *= al[h];
      __builtin_amdgcn_wave_barrier();
    }
    const float msafe = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
    for (int ps = 0; ps < C::NPASS; ++ps) {
      const float pv = fast_exp2(s[ps] - msafe);
      const int j = ps * TPI + t;
      if constexpr (C::kBf16) {
        const uint32_t bits = f32_to_bf16_bits(pv);
        l_run += __uint_as_float(bits << 16);
        reinterpret_cast<uint16_t*>(p_lds)[((j >> 1) * GP + my_head) * 2 + (j & 1)] = (uint16_t)bits;
      } else {
        l_run += pv;
        reinterpret_cast<float*>(p_lds)[j * GP + my_head] = pv;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- keys past the sequence end may hold anything: zero their V ----
    if (tok0 + 16 > n) {
#pragma unroll
      for (int r = 0; r < C::RPL; ++r)
#pragma unroll
        for (int w = 0; w < C::VPR; ++w)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if constexpr (C::kBf16) {
              const int j0 = tok0 + vh * 8 + w * 8 + c * 2;
              uint32_t m = (j0 < n ? 0xffffu : 0u) | (j0 + 1 < n ? 0xffff0000u : 0u);
              cur.v[r][w][c] &= m;
            } else {
              const int j0 = tok0 + vh * 8 + w * 4 + c;
              if (j0 >= n) cur.v[r][w][c] = 0u;
            }
          }
    }

    // ---- o += P.V ----
    if constexpr (C::kBf16) {
#pragma unroll
      for (int jl = 0; jl < 4; ++jl) {
        const int jp = vh * 4 + jl;  // token pair inside the chunk
        uint32_t pp[GP];
#pragma unroll
        for (int h4 = 0; h4 < GP / 4; ++h4) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(&p_lds[jp * GP + h4 * 4]);
          pp[h4 * 4 + 0] = x[0];
          pp[h4 * 4 + 1] = x[1];
          pp[h4 * 4 + 2] = x[2];
          pp[h4 * 4 + 3] = x[3];
        }
#pragma unroll
        for (int r = 0; r < C::RPL; ++r) {
          const uint32_t v2 = cur.v[r][0][jl];
#pragma unroll
          for (int h = 0; h < GP; ++h) o[h][r] = dot2_bf16(pp[h], v2, o[h][r]);
        }
      }
    } else {
#pragma unroll
      for (int jl = 0; jl < 8; ++jl) {
        const int j = vh * 8 + jl;
        float pj[GP];
#pragma unroll
        for (int h4 = 0; h4 < GP / 4; ++h4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&reinterpret_cast<const float*>(p_lds)[j * GP + h4 * 4]);
          pj[h4 * 4 + 0] = x[0];
          pj[h4 * 4 + 1] = x[1];
          pj[h4 * 4 + 2] = x[2];
          pj[h4 * 4 + 3] = x[3];
        }
#pragma unroll
        for (int r = 0; r < C::RPL; ++r) {
          const float vj = __uint_as_float(cur.v[r][jl >> 2][jl & 3]);
#pragma unroll
          for (int h = 0; h < GP; ++h) o[h][r] = fmaf(pj[h], vj, o[h][r]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Block mask (kMods == kModsBlockMask instances only): a chunk whose key
  // block the row's bitmap row does not admit is neither loaded nor computed.
  // A chunk lies inside one key block (blocks are whole multiples of 64 keys).
  const uint32_t* bm_row = nullptr;
  if constexpr (kMods == kModsBlockMask) {
    bm_row = a.bm.bits + ((size_t)b * a.bm.rows + (rr.pos >> a.bm.q_log2)) * a.bm.words;
  }
  auto chunk_ok = [&](int tok0) -> bool {
    if constexpr (kMods != kModsBlockMask) {
      return true;
    } else {
      if (tok0 >= c_end) return false;  // (past the segment: nothing to compute, no word to read)
      const int kb = tok0 >> a.bm.kv_log2;
      return ((bm_row[kb >> 5] >> (kb & 31)) & 1u) != 0;
    }
  };

  // Software pipeline over two register buffers: while one chunk is computed
  // the next two are in flight.  Every load is unconditional (addresses past
  // the partition are clamped to its last chunk, which is fetched again) and
  // the loop is unrolled by two, so every path keeps the same loads in flight
  // and each vmcnt wait covers exactly the chunk about to be used (a block
  // mask makes loads conditional; the waits then follow the compiler's count).
  if (c_begin < c_end) {
    const int last_chunk = c_begin + ((c_end - c_begin - 1) & ~15);
    Chunk<E, D, GP> buf0, buf1;
    if (chunk_ok(c_begin)) load_chunk(buf0, c_begin);
    if (chunk_ok(min(c_begin + 16, last_chunk))) load_chunk(buf1, min(c_begin + 16, last_chunk));
    for (int tok0 = c_begin; tok0 < c_end; tok0 += 32) {
      if (chunk_ok(tok0)) process(buf0, tok0);
      if (chunk_ok(min(tok0 + 32, last_chunk))) load_chunk(buf0, min(tok0 + 32, last_chunk));
      if (chunk_ok(tok0 + 16)) process(buf1, tok0 + 16);
      if (chunk_ok(min(tok0 + 48, last_chunk))) load_chunk(buf1, min(tok0 + 48, last_chunk));
    }
  }

  // ---- finish: add the two token halves; per-head (m, l) to every lane ----
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int r = 0; r < C::RPL; ++r) o[h][r] += dpp<kDppQuadXor1>(o[h][r]);
  const float l_tot = group_reduce<TPI, false>(l_run);
  if (t == 0) {
    stat_lds[2 * my_head] = m_run;
    stat_lds[2 * my_head + 1] = l_tot;
  }
  __builtin_amdgcn_wave_barrier();
  if constexpr (kToLds) {
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int r = 0; r < C::RPL; ++r)
        if ((r & 1) == vh) lds_o[h * D + vr + 32 * r] = o[h][r];
    if (lane < 2 * GP) lds_ml[lane] = stat_lds[lane];
    return;
  }
  float mh[GP], lh[GP];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    mh[h] = stat_lds[2 * h];
    lh[h] = stat_lds[2 * h + 1];
  }

  if (whole && a.state_o) {
    // two-phase decode: the row's state (normalised output, log-sum-exp), fp32
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h >= nvalid) continue;
      const float inv = lh[h] > 0.f ? 1.f / lh[h] : 0.f;
      const size_t srow = (size_t)rr.qrow * a.Hq + head0 + h;
#pragma unroll
      for (int r = 0; r < C::RPL; ++r)
        if ((r & 1) == vh) a.state_o[srow * D + vr + 32 * r] = o[h][r] * inv;
      if (lane == 0) a.state_lse[srow] = state_lse2(mh[h], lh[h]);
    }
  } else if (whole) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      if (h >= nvalid) continue;
      const float inv = lh[h] > 0.f ? 1.f / lh[h] : 0.f;
      char* orow = static_cast<char*>(a.out) + ((size_t)rr.qrow * a.Hq + head0 + h) * D * C::ES;
#pragma unroll
      for (int r = 0; r < C::RPL; ++r) {
        if ((r & 1) != vh) continue;  // each half writes every other row
        const int d = vr + 32 * r;
        const float val = o[h][r] * inv;
        if constexpr (C::kBf16) {
          reinterpret_cast<uint16_t*>(orow)[d] = (uint16_t)f32_to_bf16_bits(val);
        } else {
          reinterpret_cast<float*>(orow)[d] = val;
        }
      }
    }
  } else {
    float* wo = a.ws_o + unit * GP * D;
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int r = 0; r < C::RPL; ++r)
        if ((r & 1) == vh) wo[h * D + vr + 32 * r] = o[h][r];
    if (lane < GP) {
      a.ws_ml[unit * GP * 2 + 2 * lane] = mh[lane];
      a.ws_ml[unit * GP * 2 + 2 * lane + 1] = lh[lane];
    }
  }
}

// Fixed partitions: one wavefront per (row slot, head group, partition of
// 2^split_log2 keys).  Also the unsplit path (P == 1) used by fp32 prefill.
template <typename E, int D, int GP, int kMods>
__global__ __launch_bounds__(64) void row_partials_kernel(const RowAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t p_lds[16 * GP];  // bf16 pairs or f32
  __shared__ __attribute__((aligned(16))) float stat_lds[2 * GP];
  const int HG = a.Hkv * a.NG;
  const int flat = blockIdx.x;
  const int p = flat % a.P;
  const int hg = (flat / a.P) % HG;
  const int slot = flat / (a.P * HG);
  RowRange rr;
  if (!row_range(a, slot, rr)) return;
  if (p >= rr.nparts) return;
  const int c_begin = rr.start + (p << a.split_log2);
  const int c_end = min(rr.hi, c_begin + (1 << a.split_log2));
  attend_segment<E, D, GP, kMods>(a, rr, slot, hg, c_begin, c_end, rr.nparts == 1,
                                  ((size_t)slot * HG + hg) * a.P + p, p_lds, stat_lds);
}

// Fixed partitions with NW wavefronts per work-group: the partition's chunks
// are dealt out in NW contiguous runs, one per wavefront, and the work-group
// merges the NW states (log-sum-exp weights, wavefront order) in LDS before it
// writes the partition's output or partial, in the layout row_partials_kernel
// writes.  A partition then streams NW times faster: the launch for grids that
// fit the device at once (small batches), where each partition's own latency
// is the call's.
template <typename E, int D, int GP, int kMods, int NW>
__global__ __launch_bounds__(64 * NW) void row_partials_wg_kernel(const RowAttnArgs a) {
  using C = Cfg<E, D, GP>;
  __shared__ __attribute__((aligned(16))) uint32_t p_lds[NW][16 * GP];
  __shared__ __attribute__((aligned(16))) float stat_lds[NW][2 * GP];
  __shared__ __attribute__((aligned(16))) float st_o[NW][GP * D];
  __shared__ float st_ml[NW][2 * GP];
  const int HG = a.Hkv * a.NG;
  const int flat = blockIdx.x;
  const int p = flat % a.P;
  const int hg = (flat / a.P) % HG;
  const int slot = flat / (a.P * HG);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (uniform: scalar table loads)
  RowRange rr;
  if (!row_range(a, slot, rr)) return;
  if (p >= rr.nparts) return;
  const int c_begin = rr.start + (p << a.split_log2);
  const int c_end = min(rr.hi, c_begin + (1 << a.split_log2));
  const int nch = c_end > c_begin ? (c_end - c_begin + 15) >> 4 : 0;
  const int per = (nch + NW - 1) / NW;
  const int w_begin = min(c_end, c_begin + 16 * per * wave);
  const int w_end = min(c_end, c_begin + 16 * per * (wave + 1));
  attend_segment<E, D, GP, kMods, true>(a, rr, slot, hg, w_begin, w_end, false, 0, p_lds[wave],
                                        stat_lds[wave], st_o[wave], st_ml[wave]);
  __syncthreads();

  const bool whole = rr.nparts == 1;
  const size_t unit = ((size_t)slot * HG + hg) * a.P + p;
  const int kvh = hg / a.NG;
  const int head0 = kvh * a.g + (hg - kvh * a.NG) * GP;
  const int nvalid = min(GP, a.g - (hg - kvh * a.NG) * GP);
  for (int el = threadIdx.x; el < GP * D; el += 64 * NW) {
    const int h = el / D;
    const int d = el - h * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, st_ml[w][2 * h]);
    float O = 0.f, L = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = fast_exp2(st_ml[w][2 * h] - M);
        L = fmaf(wt, st_ml[w][2 * h + 1], L);
        O = fmaf(wt, st_o[w][h * D + d], O);
      }
    }
    if (!whole) {
      a.ws_o[unit * GP * D + el] = O;
      if (d == 0) {
        a.ws_ml[unit * GP * 2 + 2 * h] = M;
        a.ws_ml[unit * GP * 2 + 2 * h + 1] = L;
      }
      continue;
    }
    if (h >= nvalid) continue;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t srow = (size_t)rr.qrow * a.Hq + head0 + h;
    if (a.state_o) {
      // two-phase decode: the row's state (normalised output, log-sum-exp), fp32
      a.state_o[srow * D + d] = O * inv;
      if (d == 0) a.state_lse[srow] = state_lse2(M, L);
    } else if constexpr (C::kBf16) {
      static_cast<uint16_t*>(a.out)[srow * D + d] = (uint16_t)f32_to_bf16_bits(O * inv);
    } else {
      static_cast<float*>(a.out)[srow * D + d] = O * inv;
    }
  }
}

// 16-token chunks a decode row's admissible range spans (>= 1, so that an
// empty context still gets a (fully masked) chunk and a zero output).
__device__ __forceinline__ int decode_chunks(const RowAttnArgs& a, int b) {
  RowRange rr;
  row_range(a, b, rr);  // decode: slot b is sequence b's only row
  const int c = (rr.hi - rr.start + 15) >> 4;
  return c > 1 ? c : 1;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_scan(int x) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if ((int)(threadIdx.x & 63) >= d) x += y;
  }
  return x;
}

// Exclusive chunk prefix of every decode row into pre[0..B] (LDS).
__device__ __forceinline__ void chunk_prefix(const RowAttnArgs& a, int* pre) {
  const int lane = threadIdx.x;
  int carry = 0;
  if (lane == 0) pre[0] = 0;
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int b = base + lane;
    const int c = b < a.num_seqs ? decode_chunks(a, b) : 0;
    const int incl = wave_scan(c);
    if (b < a.num_seqs) pre[b + 1] = carry + incl;
    carry += __shfl(incl, 63, 64);
  }
  __builtin_amdgcn_wave_barrier();
}

// Exclusive prefix of every decode row's partition count into pre[0..B] (LDS).
__device__ __forceinline__ void partition_prefix(const RowAttnArgs& a, int* pre) {
  const int lane = threadIdx.x;
  int carry = 0;
  if (lane == 0) pre[0] = 0;
  for (int base = 0; base < a.num_seqs; base += 64) {
    const int b = base + lane;
    int c = 0;
    if (b < a.num_seqs) {
      RowRange rr;
      row_range(a, b, rr);  // decode: slot b is sequence b's only row
      c = rr.nparts;
    }
    const int incl = wave_scan(c);
    if (b < a.num_seqs) pre[b + 1] = carry + incl;
    carry += __shfl(incl, 63, 64);
  }
  __builtin_amdgcn_wave_barrier();
}

// Fixed partitions of a large decode grid, walked by persistent wavefronts:
// the (row, head group, partition) items that exist -- those inside each
// row's range -- are numbered end to end and wavefront w takes items w, w +
// W, w + 2W, ...  Each item is computed exactly as row_partials_kernel
// computes it and lands at the same workspace unit, but no wavefront is
// launched for the partitions a short row leaves empty (two thirds of the
// grid on the long-context batch at 512-key partitions).
template <typename E, int D, int GP, int kMods>
__global__ __launch_bounds__(64) void decode_fixed_persistent_kernel(const RowAttnArgs a) {
  extern __shared__ int pre[];  // [num_seqs + 1]
  __shared__ __attribute__((aligned(16))) uint32_t p_lds[16 * GP];
  __shared__ __attribute__((aligned(16))) float stat_lds[2 * GP];
  const int HG = a.Hkv * a.NG;
  partition_prefix(a, pre);
  // (wave-uniform through readfirstlane, as in the balanced split)
  const long long total = (long long)__builtin_amdgcn_readfirstlane(pre[a.num_seqs]) * HG;
  for (long long g = blockIdx.x; g < total; g += gridDim.x) {
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)__builtin_amdgcn_readfirstlane(pre[mid]) * HG <= g) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int pb = __builtin_amdgcn_readfirstlane(pre[b]);
    const int np = __builtin_amdgcn_readfirstlane(pre[b + 1]) - pb;
    const int r = (int)(g - (long long)pb * HG);
    const int hg = r / np;
    const int p = r - hg * np;
    RowRange rr;
    row_range(a, b, rr);
    const int c_begin = rr.start + (p << a.split_log2);
    const int c_end = min(rr.hi, c_begin + (1 << a.split_log2));
    attend_segment<E, D, GP, kMods>(a, rr, b, hg, c_begin, c_end, rr.nparts == 1,
                                    ((size_t)b * HG + hg) * a.P + p, p_lds, stat_lds);
  }
}

// Balanced decode ("stream" split): the items (row, head group) are laid end
// to end as one sequence of 16-token chunks and wavefront w takes chunks
// [w*S, (w+1)*S), S = ceil(total / waves), crossing item boundaries as it
// goes.  Every wavefront does the same amount of work, so there is no tail of
// long partitions, and no wavefront is launched just to find it has nothing
// to do.  A wavefront that covers an item entirely writes its output; pieces
// of items split between wavefronts leave partials at unit w + item (unique:
// the wavefronts touching an item, and the items a wavefront touches, are
// both contiguous) for the merge kernel.
template <typename E, int D, int GP, int kMods>
__global__ __launch_bounds__(64) void decode_stream_kernel(const RowAttnArgs a) {
  extern __shared__ int pre[];  // [num_seqs + 1]
  __shared__ __attribute__((aligned(16))) uint32_t p_lds[16 * GP];
  __shared__ __attribute__((aligned(16))) float stat_lds[2 * GP];
  const int HG = a.Hkv * a.NG;
  chunk_prefix(a, pre);
  // (prefix values are read through readfirstlane: everything derived from
  // them -- row, head group, key range -- is then wave-uniform, so the block
  // table is read with scalar loads whose waits never hold back the K/V
  // loads in flight)
  const long long total = (long long)__builtin_amdgcn_readfirstlane(pre[a.num_seqs]) * HG;
  const long long W = gridDim.x;
  // (at least kStreamMinChunks per wavefront, counted on the actual lengths:
  // the host sized the grid from max_context_len; surplus wavefronts exit)
  const long long S = max((total + W - 1) / W, (long long)kStreamMinChunks);
  long long g = (long long)blockIdx.x * S;
  const long long g_end = min(total, g + S);
  if (g >= g_end) return;
  // row containing chunk g: largest b with pre[b] * HG <= g
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)__builtin_amdgcn_readfirstlane(pre[mid]) * HG <= g) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  while (g < g_end) {
    const int pb = __builtin_amdgcn_readfirstlane(pre[b]);
    const int nc = __builtin_amdgcn_readfirstlane(pre[b + 1]) - pb;
    const long long row0 = (long long)pb * HG;
    const int hg = (int)((g - row0) / nc);
    const long long item0 = row0 + (long long)hg * nc;  // first chunk of item (b, hg)
    const int c0 = (int)(g - item0);
    const int c1 = (int)min((long long)nc, g_end - item0);
    RowRange rr;
    row_range(a, b, rr);
    const int c_begin = rr.start + 16 * c0;
    const int c_end = min(rr.hi, rr.start + 16 * c1);
    const bool whole = (c0 == 0) && (c1 == nc);
    const size_t item = (size_t)b * HG + hg;
    if (c0 == 0 && threadIdx.x == 0) {
      // where the merge finds this item's partials: units w0 + item .. w1 + item
      const long long w1 = (item0 + nc - 1) / S;
      a.ws_meta[2 * item] = (int)(blockIdx.x + item);
      a.ws_meta[2 * item + 1] = (int)(w1 - blockIdx.x + 1);
    }
    attend_segment<E, D, GP, kMods>(a, rr, b, hg, c_begin, c_end, whole, blockIdx.x + item, p_lds,
                                    stat_lds);
    g = item0 + c1;
    if (hg + 1 == HG) ++b;
  }
}

// Combine np consecutive partials (units unit0 .. unit0+np-1, head slot hs)
// into output row qrow, head h: log-sum-exp weights, ascending unit order.
template <int U>
struct MergeBatch {
  static constexpr int value = U;
};

template <typename E, int D, int GP>
__device__ __forceinline__ void merge_units(const RowAttnArgs& a, const size_t unit0, const int np,
                                            const int hs, const int qrow, const int h) {
  constexpr int ES = E::kBytes;
  constexpr int R = D / 64;
  const int lane = threadIdx.x;
  const float* ml = a.ws_ml + unit0 * GP * 2 + 2 * hs;  // unit u at ml[u * 2 * GP]
  const float* op = a.ws_o + (unit0 * GP + hs) * D;     // unit u at op[u * GP * D]
  // Batches of U partials, each one memory round trip: lane j reads the (m, l)
  // of partial p0 + j while every lane reads its dimensions of all U output
  // rows; the batch's maximum and weights follow from those registers (the
  // weights broadcast by readlane).  A later batch with a larger maximum
  // rescales what is summed so far.  Summation in ascending partial order.
  // Batches of 8 for at most 8 partials (no loads of padding), else of 32.
  float M = kNegInf, L = 0.f;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  auto batches = [&](auto UC) {
    constexpr int U = decltype(UC)::value;  // partials whose loads are in flight together
    for (int p0 = 0; p0 < np; p0 += U) {
      const int n = min(U, np - p0);
      float mv = kNegInf, lv = 0.f;
      if (lane < n) {
        mv = ml[(size_t)(p0 + lane) * 2 * GP];
        lv = ml[(size_t)(p0 + lane) * 2 * GP + 1];
      }
      float x[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + min(u, n - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) x[u][r] = op[(size_t)p * GP * D + lane + 64 * r];
      }
      const float Mn = fmaxf(M, wave_max(mv));
      if (Mn == kNegInf) continue;  // no key in any partial so far
      if (M != kNegInf && Mn > M) {
        const float alpha = fast_exp2(M - Mn);
        L *= alpha;
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] *= alpha;
      }
      M = Mn;
      const float wv = lane < n ? fast_exp2(mv - M) : 0.f;  // (an empty partial: 0)
      L += wave_sum(wv * lv);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), u));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = fmaf(w, x[u][r], acc[r]);
      }
    }
  };
  if (np <= 8) {
    batches(MergeBatch<8>{});
  } else {
    batches(MergeBatch<32>{});
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (a.state_o) {
    // two-phase decode: the row's state (normalised output, log-sum-exp), fp32
    const size_t srow = (size_t)qrow * a.Hq + h;
#pragma unroll
    for (int r = 0; r < R; ++r) a.state_o[srow * D + lane + 64 * r] = acc[r] * inv;
    if (lane == 0) a.state_lse[srow] = state_lse2(M, L);
    return;
  }
  char* orow = static_cast<char*>(a.out) + ((size_t)qrow * a.Hq + h) * D * ES;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int d = lane + 64 * r;
    if constexpr (ES == 2) {
      reinterpret_cast<uint16_t*>(orow)[d] = (uint16_t)f32_to_bf16_bits(acc[r] * inv);
    } else {
      reinterpret_cast<float*>(orow)[d] = acc[r] * inv;
    }
  }
}

// Merge for the balanced split: one wavefront per (decode row, query head);
// the item's partial units were recorded by the wavefront that started it.
template <typename E, int D, int GP>
__global__ __launch_bounds__(64) void decode_stream_merge_kernel(const RowAttnArgs a) {
  const int h = blockIdx.x % a.Hq;
  const int b = blockIdx.x / a.Hq;
  const int kvh = h / a.g;
  const int hin = h - kvh * a.g;
  const size_t item = (size_t)b * a.Hkv * a.NG + kvh * a.NG + hin / GP;
  const int unit0 = a.ws_meta[2 * item];
  const int np = a.ws_meta[2 * item + 1];
  if (np <= 1) return;  // written whole by the stream kernel
  merge_units<E, D, GP>(a, (size_t)unit0, np, hin % GP, b, h);
}

constexpr int kMergeSpecParts = 8;  // fixed-partition merges this small read every state up front

// Merge for fixed partitions: one wavefront per (row slot, query head).
template <typename E, int D, int GP>
__global__ __launch_bounds__(64) void row_merge_kernel(const RowAttnArgs a) {
  const int h = blockIdx.x % a.Hq;
  const int slot = blockIdx.x / a.Hq;
  const int kvh = h / a.g;
  const int hin = h - kvh * a.g;
  const int hg = kvh * a.NG + hin / GP;
  const int HG = a.Hkv * a.NG;
  const size_t unit0 = ((size_t)slot * HG + hg) * a.P;
  if (a.P <= kMergeSpecParts && !a.cu_q_lens) {
    // Few partitions per row: every partition's state is read beside the
    // row's length instead of after it (one dependent round trip less); the
    // states past the row's partition count are in the workspace but unused.
    constexpr int R = D / 64;
    const int lane = threadIdx.x;
    const int hs = hin % GP;
    const float* ml = a.ws_ml + unit0 * GP * 2 + 2 * hs;
    const float* op = a.ws_o + (unit0 * GP + hs) * D;
    float m[kMergeSpecParts], l[kMergeSpecParts], x[kMergeSpecParts][R];
#pragma unroll
    for (int p = 0; p < kMergeSpecParts; ++p) {
      m[p] = kNegInf;
      l[p] = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) x[p][r] = 0.f;
      if (p < a.P) {
        m[p] = ml[(size_t)p * 2 * GP];
        l[p] = ml[(size_t)p * 2 * GP + 1];
#pragma unroll
        for (int r = 0; r < R; ++r) x[p][r] = op[(size_t)p * GP * D + lane + 64 * r];
      }
    }
    RowRange rr;
    if (!row_range(a, slot, rr)) return;
    const int np = rr.nparts;
    if (np <= 1) return;
    float M = kNegInf;
#pragma unroll
    for (int p = 0; p < kMergeSpecParts; ++p)
      if (p < np) M = fmaxf(M, m[p]);
    float acc[R], L = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int p = 0; p < kMergeSpecParts; ++p) {
        if (p >= np) continue;
        const float w = fast_exp2(m[p] - M);
        L = fmaf(w, l[p], L);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = fmaf(w, x[p][r], acc[r]);
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (a.state_o) {
      // two-phase decode: the row's state (normalised output, log-sum-exp), fp32
      const size_t srow = (size_t)rr.qrow * a.Hq + h;
#pragma unroll
      for (int r = 0; r < R; ++r) a.state_o[srow * D + lane + 64 * r] = acc[r] * inv;
      if (lane == 0) a.state_lse[srow] = state_lse2(M, L);
      return;
    }
    char* orow = static_cast<char*>(a.out) + ((size_t)rr.qrow * a.Hq + h) * D * E::kBytes;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int d = lane + 64 * r;
      if constexpr (E::kBytes == 2) {
        reinterpret_cast<uint16_t*>(orow)[d] = (uint16_t)f32_to_bf16_bits(acc[r] * inv);
      } else {
        reinterpret_cast<float*>(orow)[d] = acc[r] * inv;
      }
    }
    return;
  }
  RowRange rr;
  if (!row_range(a, slot, rr)) return;
  if (rr.nparts <= 1) return;
  merge_units<E, D, GP>(a, unit0, rr.nparts, hin % GP, rr.qrow, h);
}

// Two-phase decode, last step: one wavefront per (row, query head) combines
// the prefix states of every key range with the suffix: its whole state, or
// the balanced decode's partials of it.  Every state is (m, l, o) with o
// summed relative to 2^m: a normalised state with log-sum-exp lse is
// (lse, 1, o).  Weights are 2^(m_i - max m); a row with no key gets zeros.
template <int D, int GP>
__global__ __launch_bounds__(64) void cascade_merge_kernel(const CascadeMergeArgs a) {
  constexpr int R = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.Hq;
  const int b = blockIdx.x / a.Hq;
  const size_t rh = blockIdx.x;  // row * Hq + head
  const size_t plane = (size_t)a.rows * a.Hq;
  PA_DEVICE_CHECK(a.row_key_start[b] <= a.context_lens[b]);
  // suffix: whole state, or np decode partials from unit unit0
  int unit0 = 0, np = 0;
  if (a.ws_meta) {
    const int kvh = h / a.g;
    const int hin = h - kvh * a.g;
    const size_t item = (size_t)b * a.Hkv * a.NG + kvh * a.NG + hin / GP;
    unit0 = a.ws_meta[2 * item];
    np = a.ws_meta[2 * item + 1];
    if (np <= 1) np = 0;
    unit0 = unit0 * GP + hin % GP;  // (unit, head slot) index
  }
  const int ns = a.nsplit + (np > 0 ? np : 1);
  auto m_of = [&](int i) {
    if (i < a.nsplit) return a.part_lse[(size_t)i * plane + rh];
    if (np == 0) return a.state_lse[rh];
    return a.ws_ml[(size_t)(unit0 + (i - a.nsplit) * GP) * 2];
  };
  auto l_of = [&](int i) {
    return (i < a.nsplit || np == 0) ? 1.f : a.ws_ml[(size_t)(unit0 + (i - a.nsplit) * GP) * 2 + 1];
  };
  auto o_of = [&](int i) {
    if (i < a.nsplit) return a.part_o + ((size_t)i * plane + rh) * D;
    if (np == 0) return a.state_o + rh * D;
    return a.ws_o + (size_t)(unit0 + (i - a.nsplit) * GP) * D;
  };
  // Batches of states as in merge_units: lane j holds the (m, l) of state
  // i0 + j, every lane loads its dimensions of all the batch's outputs, one
  // memory round trip per batch; ascending state order.
  float M = kNegInf, L = 0.f;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  auto batches = [&](auto UC) {
    constexpr int U = decltype(UC)::value;  // states whose loads are in flight together
    for (int i0 = 0; i0 < ns; i0 += U) {
      const int n = min(U, ns - i0);
      float mv = kNegInf, lv = 0.f;
      if (lane < n) {
        mv = m_of(i0 + lane);
        lv = l_of(i0 + lane);
      }
      float x[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* op = o_of(i0 + min(u, n - 1));
#pragma unroll
        for (int r = 0; r < R; ++r) x[u][r] = op[lane + 64 * r];
      }
      const float Mn = fmaxf(M, wave_max(mv));
      if (Mn == kNegInf) continue;  // no key in any state so far
      if (M != kNegInf && Mn > M) {
        const float alpha = fast_exp2(M - Mn);
        L *= alpha;
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] *= alpha;
      }
      M = Mn;
      const float wv = lane < n ? fast_exp2(mv - M) : 0.f;  // (an empty state: 0)
      L += wave_sum(wv * lv);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), u));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = fmaf(w, x[u][r], acc[r]);
      }
    }
  };
  if (ns <= 8) {
    batches(MergeBatch<8>{});
  } else {
    batches(MergeBatch<32>{});
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + rh * D;
#pragma unroll
  for (int r = 0; r < R; ++r) orow[lane + 64 * r] = (uint16_t)f32_to_bf16_bits(acc[r] * inv);
}

constexpr int kWgWaves = 4;  // wavefronts per fixed-partition work-group

template <typename E, int D, int GP, int M>
hipError_t launch_partials_m(const RowAttnArgs& a, hipStream_t s) {
  if (a.stream_waves > 0) {
    const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
    hipLaunchKernelGGL((decode_stream_kernel<E, D, GP, M>), dim3(a.stream_waves), dim3(64), lds, s, a);
    return hipGetLastError();
  }
  const long long blocks = (long long)a.num_seqs * a.max_q_len * a.Hkv * a.NG * a.P;
  if (blocks <= 0) return hipSuccess;
  if (a.wg_partitions) {
    hipLaunchKernelGGL((row_partials_wg_kernel<E, D, GP, M, kWgWaves>), dim3((unsigned)blocks),
                       dim3(64 * kWgWaves), 0, s, a);
  } else if (a.fixed_waves > 0) {
    const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
    hipLaunchKernelGGL((decode_fixed_persistent_kernel<E, D, GP, M>), dim3(a.fixed_waves), dim3(64), lds, s, a);
  } else {
    hipLaunchKernelGGL((row_partials_kernel<E, D, GP, M>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

template <typename E, int D, int GP>
hipError_t launch_partials_t(const RowAttnArgs& a, int mods, hipStream_t s) {
  if (mods == kModsBlockMask) return launch_partials_m<E, D, GP, kModsBlockMask>(a, s);
  if (mods == kModsScore) return launch_partials_m<E, D, GP, kModsScore>(a, s);
  return launch_partials_m<E, D, GP, kModsNone>(a, s);
}

template <typename E, int D, int GP>
hipError_t launch_merge_t(const RowAttnArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.num_seqs * a.max_q_len * a.Hq;
  if (blocks <= 0) return hipSuccess;
  if (a.stream_waves > 0) {
    hipLaunchKernelGGL((decode_stream_merge_kernel<E, D, GP>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  } else {
    hipLaunchKernelGGL((row_merge_kernel<E, D, GP>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

template <typename E, int D>
hipError_t dispatch_gp(const RowAttnArgs& a, bool merge, int mods, hipStream_t s) {
  const int GP = a.g <= 4 ? 4 : 8;
  if (GP == 4) return merge ? launch_merge_t<E, D, 4>(a, s) : launch_partials_t<E, D, 4>(a, mods, s);
  return merge ? launch_merge_t<E, D, 8>(a, s) : launch_partials_t<E, D, 8>(a, mods, s);
}

template <typename E>
hipError_t dispatch_d(const RowAttnArgs& a, int D, bool merge, int mods, hipStream_t s) {
  if (D == 64) return dispatch_gp<E, 64>(a, merge, mods, s);
  return dispatch_gp<E, 128>(a, merge, mods, s);
}

int mods_instance(const RowAttnArgs& a) {
  if (a.bm.bits) return kModsBlockMask;
  return (a.softcap > 0.f || a.alibi != nullptr) ? kModsScore : kModsNone;
}

}  // namespace

hipError_t launch_row_partials(const RowAttnArgs& a, int dtype, int D, hipStream_t s) {
  return dtype == 1 ? dispatch_d<BF16>(a, D, false, mods_instance(a), s)
                    : dispatch_d<F32>(a, D, false, mods_instance(a), s);
}

hipError_t launch_row_merge(const RowAttnArgs& a, int dtype, int D, hipStream_t s) {
  return dtype == 1 ? dispatch_d<BF16>(a, D, true, kModsNone, s) : dispatch_d<F32>(a, D, true, kModsNone, s);
}

hipError_t launch_cascade_merge(const CascadeMergeArgs& a, int D, hipStream_t s) {
  const long long blocks = (long long)a.rows * a.Hq;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(64);
  if (D == 64) {
    if (a.GP == 4) hipLaunchKernelGGL((cascade_merge_kernel<64, 4>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((cascade_merge_kernel<64, 8>), grid, block, 0, s, a);
  } else {
    if (a.GP == 4) hipLaunchKernelGGL((cascade_merge_kernel<128, 4>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((cascade_merge_kernel<128, 8>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
