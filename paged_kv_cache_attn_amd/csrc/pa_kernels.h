// Launch-side view of the gfx950 kernels (argument blocks and launchers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Debug builds (PA_DEBUG_CHECKS) check the device-side caller contracts the
// host cannot see (block ids in range, lengths within the table) and trap on
// a violation; release builds compile the checks away.
#ifdef PA_DEBUG_CHECKS
#define PA_DEVICE_CHECK(cond) \
  do {                         \
    if (!(cond)) __builtin_trap(); \
  } while (0)
#else
#define PA_DEVICE_CHECK(cond) \
  do {                         \
  } while (0)
#endif

namespace pa {

// Everything one decode-style launch needs.  A "row slot" is (sequence b,
// query index i < max_q_len); decode has max_q_len == 1.
struct RowAttnArgs {
  void* out;                 // [rows, Hq, D]
  const void* q;             // [rows, Hq, D]
  const void* k_cache;       // [NB, Hkv, bs, D]
  const void* v_cache;       // [NB, Hkv, D, bs]
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;  // nullptr: one row per sequence, row index b
  float* ws_o;               // [row_slots, head_groups, P, GP, D]
  float* ws_ml;              // [row_slots, head_groups, P, GP, 2]
  int32_t* ws_meta;          // balanced split: per item (first partial unit, count)
  const float* alibi;        // [Hq] or nullptr
  const int32_t* prefix_lens;  // [num_seqs] or nullptr (prefix-LM, with causal)
  const int32_t* doc_starts;   // [rows] or nullptr (first admissible key per row)
  int64_t num_blocks;        // pool size (debug checks only)
  int32_t bt_stride;
  int32_t max_q_len;
  int32_t num_seqs;
  int32_t Hq, Hkv, g, NG;    // g = Hq/Hkv; NG = head groups per kv-head
  int32_t bs_log2;
  int32_t split_log2;        // partition length in tokens (log2); 30 = unsplit
  int32_t P;                 // partitions per row slot in the workspace / grid
  int32_t stream_waves;      // > 0: balanced decode split over this many wavefronts
  int32_t causal;
  int32_t window;
  float scale;               // softmax scale
  float softcap;             // 0: none
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int64_t num_blocks;        // pool size (debug checks only)
  int32_t T, Hkv, D, bs_log2;
};

struct PrefillArgs {
  void* out;                 // [total_q, Hq, D] bf16
  const void* q;             // [total_q, Hq, D] bf16
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
  const float* alibi;
  const int32_t* prefix_lens;  // [num_seqs] or nullptr
  const int32_t* doc_starts;   // [total_q] or nullptr
  int64_t num_blocks;          // pool size (debug checks only)
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t Hq, Hkv, g;
  int32_t bs_log2;
  int32_t q_tiles;           // query tiles per (sequence, kv-head) in the grid
  int32_t causal;
  int32_t window;
  float scale;
  float softcap;
};

struct CopyArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* src;        // [pairs] physical blocks
  const int32_t* dst;        // [pairs]
  int64_t num_blocks;        // pool size (debug checks only)
  int32_t pairs;
  int32_t slab16;            // 16-byte units in one (block, kv-head) slab
  int32_t Hkv;
};

hipError_t launch_kv_append(const AppendArgs& a, int dtype, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s);
hipError_t launch_row_partials(const RowAttnArgs& a, int dtype, int D, hipStream_t s);
hipError_t launch_row_merge(const RowAttnArgs& a, int dtype, int D, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, int D, hipStream_t s);
int prefill_rows_per_tile(int g);

}  // namespace pa
