// Internal declarations shared by the host C++ and HIP sources of libpagedkv.
#pragma once

#include <cstdint>
#include <cstdio>
#include <cstdarg>

#include "pagedkv.h"

struct pa_pool {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_heads;
  int32_t head_dim;
  pa_dtype kv_dtype;
  void* k_cache;
  void* v_cache;
  void* k_scale;   // fp16 [num_blocks][num_heads], int8 and int4 pools only
  void* v_scale;
  int32_t err_slot;  // index of the pool's device error word
  int32_t* err;      // device address of that word (on `device`)
  int32_t device;    // device current at pa_alloc_pool
};

namespace pa {

// Rows a decode wave loads as one unit: a 16-row slice of a (block, head)
// tile. Blocks of 32 or 64 tokens are 2 or 4 such slices, contiguous.
constexpr int kTileRows = 16;

inline bool block_size_supported(int32_t block_size) {
  return block_size == 16 || block_size == 32 || block_size == 64;
}

// log2(block_size) for a supported block size.
inline int block_shift(int32_t block_size) {
  return block_size == 16 ? 4 : block_size == 32 ? 5 : 6;
}

// Records the message of a failing call for pa_last_error() and returns st.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Bytes of one row of head_dim values (int4: two values per byte).
inline int64_t row_bytes(pa_dtype t, int32_t head_dim) {
  return t == PA_F32 ? 4 * int64_t(head_dim) : t == PA_F16 ? 2 * int64_t(head_dim)
                                             : t == PA_I8 ? int64_t(head_dim) : int64_t(head_dim) / 2;
}

// Pools that store codes with one fp16 scale per (block, head).
inline bool is_quantised(pa_dtype t) { return t == PA_I8 || t == PA_I4; }

inline bool geometry_supported(int32_t block_size, int32_t head_dim) {
  return block_size_supported(block_size) && (head_dim == 64 || head_dim == 128);
}

// Kernel launchers (decode.hip, cache_ops.hip). Arguments are validated by the
// C-ABI layer before these are called. Each returns hipSuccess or the launch
// error as an int.
struct DecodeArgs {
  const void* q;
  pa_dtype q_dtype;
  void* out;
  const void* k;          // pool base, or contiguous [S][H][T][D] base
  const void* v;
  const void* k_scale;    // int8 pools only
  const void* v_scale;
  pa_dtype kv_dtype;
  const int32_t* tables;  // nullptr => contiguous layout
  int32_t max_blocks;     // table row stride
  int32_t block_size;     // tokens per block (16 for the contiguous layout)
  int64_t max_tokens;     // contiguous layout: tokens per (seq, head) row
  const int32_t* ctx;
  const int32_t* order;   // optional schedule (permutation of the batch), may be null
  int32_t schedule;       // PA_SCHED_*: how ordered (rank, head) items map to XCDs
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t num_blocks;     // pool size, for range checks
  int32_t max_ctx;
  float sm_scale;
  int32_t partition_tokens;  // 0 => single pass
  int32_t num_partitions;    // ceil(max_ctx / partition_tokens), 1 for single pass
  float* ws_m;
  float* ws_l;
  float* ws_o;
  // Fused write (pa_write_decode): nullptr slots = none.
  const void* k_new;
  const void* v_new;
  pa_dtype new_dtype;
  const int64_t* slots;
  // Mixed-precision pages (pa_decode_mixed): nullptr hot_blocks = none. The
  // pool above (k, v, scales) is then the int8 cold pool.
  const void* hot_k;
  const void* hot_v;
  const int32_t* hot_blocks;
  int32_t num_hot;
  int32_t* err;           // device error word the kernels flag
};

int launch_decode(const DecodeArgs& a, void* stream);
// Several new tokens per sequence (pa_prefill): fp16 pool, q and out.
struct PrefillArgs {
  const pa_pool* pool;
  const void* q;
  void* out;
  const int32_t* query_start;  // [num_seqs + 1]
  int32_t num_rows;            // rows of q and out
  const int32_t* tables;
  int32_t max_blocks;
  const int32_t* ctx;
  const int32_t* order;        // [num_seqs] dispatch order, or nullptr
  int32_t num_seqs;
  int32_t max_query_len;
  int32_t max_ctx;
  float sm_scale;
};
// Workgroups of one pa_prefill launch.
int64_t prefill_groups(int32_t num_seqs, int32_t num_heads, int32_t max_query_len);
int launch_prefill(const PrefillArgs& a, void* stream);
int launch_write_kv(const pa_pool* p, const void* k_new, const void* v_new, pa_dtype src,
                    const int64_t* slots, int32_t n, void* stream);
int launch_copy_blocks(const pa_pool* p, const int32_t* pairs, int32_t n, void* stream);
int launch_demote_blocks(const pa_pool* hot, const pa_pool* cold, const int32_t* pairs, int32_t n, void* stream);
// Device views of a host pool (pinned host memory) for launch_swap_blocks.
struct SwapHost {
  void* k;
  void* v;
  void* k_scale;   // int8 pools only
  void* v_scale;
  int32_t num_blocks;
};
int launch_swap_blocks(const pa_pool* p, const SwapHost& h, const int32_t* pairs, int32_t n, bool out_dir,
                       void* stream);
int launch_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);
int launch_stream_read(const void* src, int64_t bytes, void* sink, void* stream);
int launch_stage_copy(void* dst, const void* src_device_view, int64_t bytes, void* stream);
// Device error words (api.hip): one per live pool plus word 0 for calls tied
// to no pool. kErrorWords bounds the pools alive at once.
constexpr int kErrorWords = 4096;
// Takes a free word on the current device and clears it. Returns a hipError_t
// as int: hipErrorOutOfMemory if every word is taken.
int acquire_error_word(int32_t* slot, int32_t** word, int32_t* device);
void release_error_word(int32_t slot);
// Device address of word 0 on the current device (nullptr if the lookup
// fails; kernels then skip flagging).
int32_t* shared_error_word();
// Atomically reads and clears word `slot` on the current device (after the
// stream's earlier work), returning a hipError_t as int.
int read_and_clear_error_word(int32_t slot, void* stream, int32_t* value);

}  // namespace pa
