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

// Block mask on the device: row b * rows + (position >> q_log2) of bits
// [*, words] admits key j when bit (j >> kv_log2) is set (LSB first).
struct BlockMaskArgs {
  const uint32_t* bits;
  int32_t q_log2, kv_log2, rows, words;
};

// Everything one decode-style launch needs.  A "row slot" is (sequence b,
// query index i < max_q_len); decode has max_q_len == 1.
// 16-token chunks a wavefront of the balanced decode split takes at least.
constexpr int kStreamMinChunks = 8;

struct RowAttnArgs {
  void* out;                 // [rows, Hq, D]
  const void* q;             // [rows, Hq, D]
  const void* k_cache;       // [NB, Hkv, bs, D]
  const void* v_cache;       // [NB, Hkv, bs/16, D, 16]
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;  // nullptr: one row per sequence, row index b
  float* ws_o;               // [row_slots, head_groups, P, GP, D]
  float* ws_ml;              // [row_slots, head_groups, P, GP, 2]
  int32_t* ws_meta;          // balanced split: per item (first partial unit, count)
  const float* alibi;        // [Hq] or nullptr
  const int32_t* prefix_lens;  // [num_seqs] or nullptr (prefix-LM, with causal)
  const int32_t* doc_starts;   // [rows] or nullptr (first admissible key per row)
  const int32_t* row_floor;    // [rows] or nullptr: a second first-admissible-key bound
  BlockMaskArgs bm;            // bm.bits == nullptr: no block mask
  // nullptr: final rows go to out.  Else (two-phase decode) each row's
  // normalised output goes to state_o [rows, Hq, D] and its log-sum-exp
  // (log2 units of the scaled scores) to state_lse [rows, Hq], in fp32.
  float* state_o;
  float* state_lse;
  int64_t num_blocks;        // pool size (debug checks only)
  int32_t bt_stride;
  int32_t max_q_len;
  int32_t num_seqs;
  int32_t Hq, Hkv, g, NG;    // g = Hq/Hkv; NG = head groups per kv-head
  int32_t bs_log2;
  int32_t split_log2;        // partition length in tokens (log2); 30 = unsplit
  int32_t P;                 // partitions per row slot in the workspace / grid
  int32_t stream_waves;      // > 0: balanced decode split over this many wavefronts
  int32_t wg_partitions;     // 1: each fixed partition is one multi-wavefront work-group
  int32_t fixed_waves;       // > 0: fixed partitions walked by this many persistent wavefronts
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
  BlockMaskArgs bm;            // bm.bits == nullptr: no block mask
  // Key-split mode (key_split > 0): the grid also runs over nsplit key ranges
  // of key_split keys; the work-group of range s writes each row's output
  // over keys [s*key_split, (s+1)*key_split) (every other mask still applies)
  // normalised to part_o [nsplit, total_q, Hq, D] and its log-sum-exp (log2
  // units) to part_lse [nsplit, total_q, Hq], fp32; an empty range gives 0 and
  // -inf.  Used by the two-phase decode (shared parts) and by the prefill of
  // grids that leave compute units idle (then merged by
  // launch_prefill_split_merge).  With key_starts, sequence b's keys are
  // [key_starts[b], context_lens[b]) and range s is counted from
  // key_starts[b].  Sequence b reads table row table_rows[b] (nullptr: row
  // b), and the work-groups of range 0 and kv-head 0 store context_lens[b]
  // into row_key_start[row] for each of its rows (nullptr: not stored); with
  // chain set, the value found there must be key_starts[b] (checked in debug
  // builds).
  const int32_t* table_rows;
  const int32_t* key_starts;
  // key-split mode: nullptr, or per row the context length of the decode row
  // it is (the row sits at position q_ctx[row] - 1, for window and ALiBi)
  const int32_t* q_ctx;
  int32_t chain;
  float* part_o;
  float* part_lse;
  int32_t* row_key_start;
  int32_t key_split;
  int32_t nsplit;
  int64_t num_blocks;          // pool size (debug checks only)
  int32_t bt_stride;
  int32_t num_seqs;
  int32_t total_q;
  int32_t Hq, Hkv, g;
  int32_t bs_log2;
  int32_t q_tiles;           // query tiles per (sequence, kv-head) in the grid
  int32_t num_cus;           // compute units of the device (0: unknown)
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

// Two-phase decode, last step: for each (row b, query head h), the nsplit
// prefix states part_o/part_lse [nsplit, rows, Hq, (D)] and the suffix's
// state are combined with log-sum-exp weights into out [rows, Hq, D] (bf16).
// The suffix state is state_o/state_lse [rows, Hq, (D)] (fp32, log2-unit
// log-sum-exps) -- or, when ws_meta is set (balanced decode split) and the
// row's item was split, the decode's partials (ws_o, ws_ml at the units
// ws_meta names), merged here instead of by the decode's own merge.
struct CascadeMergeArgs {
  void* out;
  const float* part_o;
  const float* part_lse;
  const float* state_o;
  const float* state_lse;
  const float* ws_o;
  const float* ws_ml;
  const int32_t* ws_meta;
  const int32_t* row_key_start;  // debug checks only
  const int32_t* context_lens;   // debug checks only
  int32_t rows, Hq, nsplit;
  int32_t Hkv, g, NG, GP;        // decode item geometry (head groups of GP heads)
};

hipError_t launch_kv_append(const AppendArgs& a, int dtype, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t s);
hipError_t launch_row_partials(const RowAttnArgs& a, int dtype, int D, hipStream_t s);
hipError_t launch_row_merge(const RowAttnArgs& a, int dtype, int D, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, int D, hipStream_t s);
hipError_t launch_prefill_split_merge(const PrefillArgs& a, int D, hipStream_t s);
hipError_t launch_cascade_merge(const CascadeMergeArgs& a, int D, hipStream_t s);
int prefill_rows_per_tile(int g);

}  // namespace pa
