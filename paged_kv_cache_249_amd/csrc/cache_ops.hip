// Cache-side kernels for gfx950: writing new K/V rows into their slots,
// copy-on-write block copies, swapping blocks to pinned host memory and back,
// demoting fp16 blocks to int8 or int4, the copy of a pinned staging buffer,
// and plain streaming copy and read kernels (measurement baselines).
//
// write_kv (reshape-and-cache): row i of the new K/V goes to slot
// slots[i] = block * B + offset for a block size B of 16, 32 or 64, the
// lookup of "PagedAttention — 把 KV cache 当虚拟内存页来管理", 实践案例 /
// 案例 2. Writing new tokens into pages is also the only data movement of
// the sliding window ("KV Cache与长上下文管理", the section
// on the second problem paging solves: the new token is written into the page
// the oldest data occupied).
//
// int8 pools quantise on write with one fp16 scale per (block, head), for K
// and V separately (FP16 -> INT8 compression is listed in "KV Cache与长上下文管理",
// section 二.3, without a scheme; the group rule below is this library's and
// is stated in pagedkv.h). int4 pools (INT4, the next entry of the same list)
// use the same rule with codes in [-7, 7], two per byte. One wave handles
// one run of adjacent slot entries that hit the same block (at most B rows),
// for one head and one tensor.
//
// copy_blocks: whole-block copies, the copy-on-write unit of "PagedAttention
// — 把 KV cache 当虚拟内存页来管理", 实践案例 / 案例 3.
//
// swap_blocks: whole blocks between the device pool and a pool in pinned host
// memory, page by page ("KV Cache与长上下文管理", the fourth point on what paging
// makes possible), read or written by the kernel directly over the host link.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float ld_f(const T* p) {
  return float(*p);
}

// ---------------------------------------------------------------------------
// Float pools: one thread per 16 destination bytes.
template <typename DST, typename SRC, int D>
__global__ __launch_bounds__(kThreads) void write_kv_kernel(const SRC* __restrict__ k_new,
                                                            const SRC* __restrict__ v_new,
                                                            DST* __restrict__ k_pool,
                                                            DST* __restrict__ v_pool,
                                                            const int64_t* __restrict__ slots, int n,
                                                            int H, int num_blocks, int bshift, int32_t* err) {
  constexpr int kEPT = 16 / int(sizeof(DST));   // elements per thread
  constexpr int kCPR = D / kEPT;                // threads per (row, head)
  const int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t total = int64_t(n) * H * kCPR;
  if (idx >= total) return;
  const int64_t row = idx / kCPR;   // (i, h)
  const int chunk = int(idx % kCPR);
  const int64_t i = row / H;
  const int h = int(row % H);
  const int64_t slot = slots[i];
  if (slot < 0) return;
  const int64_t blk = slot >> bshift;
  const int off = int(slot & ((int64_t(1) << bshift) - 1));
  if (blk >= num_blocks) {
    flag_error(err, PA_DEV_BAD_SLOT);
    return;
  }
  const SRC* src = (blockIdx.y == 0 ? k_new : v_new) + row * D + chunk * kEPT;
  DST* dst = (blockIdx.y == 0 ? k_pool : v_pool) + (((blk * H + h) << bshift) + off) * D + chunk * kEPT;
  DST vals[kEPT];
#pragma unroll
  for (int e = 0; e < kEPT; ++e) vals[e] = DST(ld_f(src + e));
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(vals);
}

// ---------------------------------------------------------------------------
// Quantised pools write a block's rows of one call as one group, by one wave
// per run of adjacent rows hitting that block. A second, non-adjacent run into
// the same block would be written by another wave at the same time, so it is
// flagged (PA_DEV_BAD_RUN) instead: the wave of the later run leader i (head
// 0, K tensor only) looks for the block among the rows before i. Reads are 8
// wave-wide loads of 512 bytes in flight per step.
__device__ bool earlier_run_hits(const int64_t* __restrict__ slots, int64_t i, int64_t blk, int bshift) {
  constexpr int kUnroll = 8;
  const int lane = threadIdx.x & (kWave - 1);
  bool hit = false;
  int64_t j = lane;
  for (; j + (kUnroll - 1) * kWave < i; j += kUnroll * kWave) {
    int64_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = slots[j + u * kWave];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) hit |= v[u] >= 0 && (v[u] >> bshift) == blk;
  }
  for (; j < i; j += kWave) {
    const int64_t v = slots[j];
    hit |= v >= 0 && (v >> bshift) == blk;
  }
  return __ballot(hit) != 0;
}

// ---------------------------------------------------------------------------
// int8 pools: one wave per (run leader i, head h, tensor).
template <typename SRC, int D>
__global__ __launch_bounds__(kThreads) void write_kv_i8_kernel(
    const SRC* __restrict__ k_new, const SRC* __restrict__ v_new, int8_t* __restrict__ k_pool,
    int8_t* __restrict__ v_pool, _Float16* __restrict__ k_scale, _Float16* __restrict__ v_scale,
    const int64_t* __restrict__ slots, int n, int H, int num_blocks, int bshift, int32_t* err) {
  constexpr int kDPL = D / kWave;   // dims per lane
  const int bs = 1 << bshift;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = int64_t(blockIdx.x) * (kThreads / kWave) + wave_uniform(threadIdx.x / kWave);
  if (wid >= int64_t(n) * H) return;
  const int64_t i = wid / H;
  const int h = int(wid % H);
  const int64_t slot = slots[i];
  if (slot < 0) return;
  const int64_t blk = slot >> bshift;
  if (blk >= num_blocks) {
    if (lane == 0) flag_error(err, PA_DEV_BAD_SLOT);
    return;
  }
  if (i > 0) {
    const int64_t prev = slots[i - 1];
    if (prev >= 0 && (prev >> bshift) == blk) return;   // not the first row of its run
  }
  const bool is_v = blockIdx.y != 0;
  const SRC* src = is_v ? v_new : k_new;
  int8_t* pool = is_v ? v_pool : k_pool;
  _Float16* scale = is_v ? v_scale : k_scale;

  // The run: rows i .. i+R-1 hitting block blk.
  uint64_t mask = 0;
  int R = 0;
  bool dup = false;
  while (R < bs && i + R < n) {
    const int64_t sl = slots[i + R];
    if (sl < 0 || (sl >> bshift) != blk) break;
    const uint64_t bit = uint64_t(1) << int(sl & (bs - 1));
    dup |= (mask & bit) != 0;
    mask |= bit;
    ++R;
  }
  if (i + R < n && R == bs) {
    const int64_t sl = slots[i + R];
    dup |= sl >= 0 && (sl >> bshift) == blk;
  }
  if (h == 0 && !is_v && i > 1) dup |= earlier_run_hits(slots, i - 1, blk, bshift);
  if (dup && lane == 0) flag_error(err, PA_DEV_BAD_RUN);

  float a = 0.f;
  for (int r = 0; r < R; ++r) {
    const SRC* x = src + ((i + r) * H + h) * D + lane * kDPL;
#pragma unroll
    for (int e = 0; e < kDPL; ++e) a = fmaxf(a, fabsf(ld_f(x + e)));
  }
  a = wave_max(a);
  const float s_new = float(_Float16(a / 127.0f));
  const int64_t sidx = blk * H + h;
  const float s_old = (mask & 1u) ? 0.f : float(scale[sidx]);
  const float s = fmaxf(s_old, s_new);
  int8_t* tile = pool + (sidx << bshift) * D;

  if (s_old > 0.f && s > s_old) {
    for (int o = 0; o < bs; ++o) {
      if (mask & (uint64_t(1) << o)) continue;
#pragma unroll
      for (int e = 0; e < kDPL; ++e) {
        int8_t* c = tile + o * D + lane * kDPL + e;
        const float qf = __builtin_rintf((float(*c) * s_old) / s);
        *c = int8_t(fminf(fmaxf(qf, -127.f), 127.f));
      }
    }
  }
  for (int r = 0; r < R; ++r) {
    const int o = int(slots[i + r] & (bs - 1));
    const SRC* x = src + ((i + r) * H + h) * D + lane * kDPL;
#pragma unroll
    for (int e = 0; e < kDPL; ++e) {
      float qf = 0.f;
      if (s > 0.f) qf = fminf(fmaxf(__builtin_rintf(ld_f(x + e) / s), -127.f), 127.f);
      tile[o * D + lane * kDPL + e] = int8_t(qf);
    }
  }
  if (lane == 0) scale[sidx] = _Float16(s);
}

// ---------------------------------------------------------------------------
// int4 pools: the int8 group rule with codes in [-7, 7]; a row is D / 2
// bytes, byte j holding code[2j] + 8 in its low nibble and code[2j+1] + 8 in
// its high one, so lane l owns byte l of every row (dims 2l and 2l+1; at
// D = 64 the upper half of the wave holds no byte). One wave per (run leader
// i, head h, tensor), as for int8.
template <typename SRC, int D>
__global__ __launch_bounds__(kThreads) void write_kv_i4_kernel(
    const SRC* __restrict__ k_new, const SRC* __restrict__ v_new, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, _Float16* __restrict__ k_scale, _Float16* __restrict__ v_scale,
    const int64_t* __restrict__ slots, int n, int H, int num_blocks, int bshift, int32_t* err) {
  constexpr int kRowBytes = D / 2;
  static_assert(kRowBytes <= kWave, "one byte per lane");
  const int bs = 1 << bshift;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = int64_t(blockIdx.x) * (kThreads / kWave) + wave_uniform(threadIdx.x / kWave);
  if (wid >= int64_t(n) * H) return;
  const int64_t i = wid / H;
  const int h = int(wid % H);
  const int64_t slot = slots[i];
  if (slot < 0) return;
  const int64_t blk = slot >> bshift;
  if (blk >= num_blocks) {
    if (lane == 0) flag_error(err, PA_DEV_BAD_SLOT);
    return;
  }
  if (i > 0) {
    const int64_t prev = slots[i - 1];
    if (prev >= 0 && (prev >> bshift) == blk) return;   // not the first row of its run
  }
  const bool is_v = blockIdx.y != 0;
  const SRC* src = is_v ? v_new : k_new;
  uint8_t* pool = is_v ? v_pool : k_pool;
  _Float16* scale = is_v ? v_scale : k_scale;

  // The run: rows i .. i+R-1 hitting block blk.
  uint64_t mask = 0;
  int R = 0;
  bool dup = false;
  while (R < bs && i + R < n) {
    const int64_t sl = slots[i + R];
    if (sl < 0 || (sl >> bshift) != blk) break;
    const uint64_t bit = uint64_t(1) << int(sl & (bs - 1));
    dup |= (mask & bit) != 0;
    mask |= bit;
    ++R;
  }
  if (i + R < n && R == bs) {
    const int64_t sl = slots[i + R];
    dup |= sl >= 0 && (sl >> bshift) == blk;
  }
  if (h == 0 && !is_v && i > 1) dup |= earlier_run_hits(slots, i - 1, blk, bshift);
  if (dup && lane == 0) flag_error(err, PA_DEV_BAD_RUN);

  const bool mine = lane < kRowBytes;   // this lane owns a byte of each row
  float a = 0.f;
  if (mine) {
    for (int r = 0; r < R; ++r) {
      const SRC* x = src + ((i + r) * H + h) * D + 2 * lane;
      a = fmaxf(a, fmaxf(fabsf(ld_f(x)), fabsf(ld_f(x + 1))));
    }
  }
  a = wave_max(a);
  const float s_new = float(_Float16(a / 7.0f));
  const int64_t sidx = blk * H + h;
  const float s_old = (mask & 1u) ? 0.f : float(scale[sidx]);
  const float s = fmaxf(s_old, s_new);
  uint8_t* tile = pool + (sidx << bshift) * kRowBytes;
  auto code = [](float qf) { return uint32_t(int(fminf(fmaxf(qf, -7.f), 7.f)) + 8); };

  if (s_old > 0.f && s > s_old && mine) {
    for (int o = 0; o < bs; ++o) {
      if (mask & (uint64_t(1) << o)) continue;
      uint8_t* c = tile + o * kRowBytes + lane;
      const uint32_t b = *c;
      const float lo = __builtin_rintf((float(int(b & 15u) - 8) * s_old) / s);
      const float hi = __builtin_rintf((float(int(b >> 4) - 8) * s_old) / s);
      *c = uint8_t(code(lo) | (code(hi) << 4));
    }
  }
  for (int r = 0; r < R && mine; ++r) {
    const int o = int(slots[i + r] & (bs - 1));
    const SRC* x = src + ((i + r) * H + h) * D + 2 * lane;
    float lo = 0.f, hi = 0.f;
    if (s > 0.f) {
      lo = __builtin_rintf(ld_f(x) / s);
      hi = __builtin_rintf(ld_f(x + 1) / s);
    }
    tile[o * kRowBytes + lane] = uint8_t(code(lo) | (code(hi) << 4));
  }
  if (lane == 0) scale[sidx] = _Float16(s);
}

// ---------------------------------------------------------------------------
// Demotion of full fp16 hot blocks into int8 cold blocks (mixed-precision
// pages): one wave per (pair, head, tensor). The (block, head) tile of 16
// fp16 rows is 16 * D contiguous values; lane l quantises the kPer values
// starting at l * kPer. The arithmetic is write_kv_i8_kernel's for a group
// that writes the whole block (so the earlier scale plays no part).
template <int D>
__global__ __launch_bounds__(kThreads) void demote_kernel(const int32_t* __restrict__ pairs, int n,
                                                          const _Float16* __restrict__ hot_k,
                                                          const _Float16* __restrict__ hot_v,
                                                          int8_t* __restrict__ cold_k, int8_t* __restrict__ cold_v,
                                                          _Float16* __restrict__ k_scale,
                                                          _Float16* __restrict__ v_scale, int H, int num_hot,
                                                          int num_cold, int32_t* err) {
  constexpr int kRows = 16;
  constexpr int kPer = kRows * D / kWave;   // values per lane: 32 (D = 128) or 16 (D = 64)
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = int64_t(blockIdx.x) * (kThreads / kWave) + wave_uniform(threadIdx.x / kWave);
  if (wid >= int64_t(n) * H) return;
  const int pair = int(wid / H);
  const int h = int(wid % H);
  const bool is_v = blockIdx.y != 0;
  const int src = pairs[2 * pair];
  const int dst = pairs[2 * pair + 1];
  if (unsigned(src) >= unsigned(num_hot) || unsigned(dst) >= unsigned(num_cold)) {
    if (lane == 0 && h == 0 && !is_v) flag_error(err, PA_DEV_BAD_PAIR);
    return;
  }
  const _Float16* x = (is_v ? hot_v : hot_k) + (int64_t(src) * H + h) * kRows * D + lane * kPer;
  _Float16 vals[kPer];
#pragma unroll
  for (int j = 0; j < kPer / 8; ++j)
    *reinterpret_cast<uint4*>(vals + 8 * j) = reinterpret_cast<const uint4*>(x)[j];
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) a = fmaxf(a, fabsf(float(vals[e])));
  a = wave_max(a);
  const float s = float(_Float16(a / 127.0f));
  int8_t codes[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    float qf = 0.f;
    if (s > 0.f) qf = fminf(fmaxf(__builtin_rintf(float(vals[e]) / s), -127.f), 127.f);
    codes[e] = int8_t(qf);
  }
  int8_t* y = (is_v ? cold_v : cold_k) + (int64_t(dst) * H + h) * kRows * D + lane * kPer;
#pragma unroll
  for (int j = 0; j < kPer / 16; ++j)
    reinterpret_cast<uint4*>(y)[j] = *reinterpret_cast<const uint4*>(codes + 16 * j);
  if (lane == 0) (is_v ? v_scale : k_scale)[int64_t(dst) * H + h] = _Float16(s);
}

// The same demotion into int4 cold blocks: lane l quantises the kPer values
// of the tile starting at l * kPer into kPer / 2 bytes (32 values into 16
// bytes at D = 128, 16 into 8 at D = 64).
template <int D>
__global__ __launch_bounds__(kThreads) void demote_i4_kernel(const int32_t* __restrict__ pairs, int n,
                                                             const _Float16* __restrict__ hot_k,
                                                             const _Float16* __restrict__ hot_v,
                                                             uint8_t* __restrict__ cold_k,
                                                             uint8_t* __restrict__ cold_v,
                                                             _Float16* __restrict__ k_scale,
                                                             _Float16* __restrict__ v_scale, int H, int num_hot,
                                                             int num_cold, int32_t* err) {
  constexpr int kRows = 16;
  constexpr int kPer = kRows * D / kWave;   // values per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = int64_t(blockIdx.x) * (kThreads / kWave) + wave_uniform(threadIdx.x / kWave);
  if (wid >= int64_t(n) * H) return;
  const int pair = int(wid / H);
  const int h = int(wid % H);
  const bool is_v = blockIdx.y != 0;
  const int src = pairs[2 * pair];
  const int dst = pairs[2 * pair + 1];
  if (unsigned(src) >= unsigned(num_hot) || unsigned(dst) >= unsigned(num_cold)) {
    if (lane == 0 && h == 0 && !is_v) flag_error(err, PA_DEV_BAD_PAIR);
    return;
  }
  const _Float16* x = (is_v ? hot_v : hot_k) + (int64_t(src) * H + h) * kRows * D + lane * kPer;
  _Float16 vals[kPer];
#pragma unroll
  for (int j = 0; j < kPer / 8; ++j)
    *reinterpret_cast<uint4*>(vals + 8 * j) = reinterpret_cast<const uint4*>(x)[j];
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) a = fmaxf(a, fabsf(float(vals[e])));
  a = wave_max(a);
  const float s = float(_Float16(a / 7.0f));
  uint8_t bytes[kPer / 2];
#pragma unroll
  for (int e = 0; e < kPer / 2; ++e) {
    float lo = 0.f, hi = 0.f;
    if (s > 0.f) {
      lo = fminf(fmaxf(__builtin_rintf(float(vals[2 * e]) / s), -7.f), 7.f);
      hi = fminf(fmaxf(__builtin_rintf(float(vals[2 * e + 1]) / s), -7.f), 7.f);
    }
    bytes[e] = uint8_t(uint32_t(int(lo) + 8) | (uint32_t(int(hi) + 8) << 4));
  }
  uint8_t* y = (is_v ? cold_v : cold_k) + (int64_t(dst) * H + h) * kRows * (D / 2) + lane * (kPer / 2);
  if constexpr (kPer / 2 == 16)
    *reinterpret_cast<uint4*>(y) = *reinterpret_cast<const uint4*>(bytes);
  else
    *reinterpret_cast<uint2*>(y) = *reinterpret_cast<const uint2*>(bytes);
  if (lane == 0) (is_v ? v_scale : k_scale)[int64_t(dst) * H + h] = _Float16(s);
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const int32_t* __restrict__ pairs, int n,
                                                               char* __restrict__ k, char* __restrict__ v,
                                                               int64_t block_bytes, _Float16* ks,
                                                               _Float16* vs, int H, int num_blocks,
                                                               int32_t* err) {
  const int pair = blockIdx.y;
  const int src = pairs[2 * pair];
  const int dst = pairs[2 * pair + 1];
  if (unsigned(src) >= unsigned(num_blocks) || unsigned(dst) >= unsigned(num_blocks)) {
    if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) flag_error(err, PA_DEV_BAD_PAIR);
    return;
  }
  char* base = blockIdx.z == 0 ? k : v;
  const int64_t off = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 16;
  if (off < block_bytes) {
    const uint4 val = *reinterpret_cast<const uint4*>(base + int64_t(src) * block_bytes + off);
    *reinterpret_cast<uint4*>(base + int64_t(dst) * block_bytes + off) = val;
  }
  if (ks && blockIdx.x == 0) {
    _Float16* sc = blockIdx.z == 0 ? ks : vs;
    for (int hh = threadIdx.x; hh < H; hh += kThreads) sc[int64_t(dst) * H + hh] = sc[int64_t(src) * H + hh];
  }
}

// One workgroup per 4 KiB of one block of one tensor. A thread moves two
// 8-byte words 512 bytes apart, so each load and store instruction of a wave
// covers 512 contiguous bytes on both sides. Host memory is accessed with
// system-scope loads and stores: no GPU cache serves a stale copy of it or
// holds back a write to it.
constexpr int kSwapWordsPerGroup = 2 * kThreads;   // 8-byte words per workgroup

__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    const int32_t* __restrict__ pairs, uint64_t* dev_k, uint64_t* dev_v, uint64_t* host_k, uint64_t* host_v,
    int64_t block_words, uint16_t* dev_ks, uint16_t* dev_vs, uint16_t* host_ks, uint16_t* host_vs, int H,
    int num_blocks, int num_host_blocks, int out_dir, int32_t* err) {
  const int pair = blockIdx.y;
  const int a = pairs[2 * pair];
  const int b = pairs[2 * pair + 1];
  const int dblk = out_dir ? a : b;
  const int hblk = out_dir ? b : a;
  if (unsigned(dblk) >= unsigned(num_blocks) || unsigned(hblk) >= unsigned(num_host_blocks)) {
    if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) flag_error(err, PA_DEV_BAD_PAIR);
    return;
  }
  uint64_t* dev = (blockIdx.z == 0 ? dev_k : dev_v) + int64_t(dblk) * block_words;
  uint64_t* host = (blockIdx.z == 0 ? host_k : host_v) + int64_t(hblk) * block_words;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w0 = int64_t(blockIdx.x) * kSwapWordsPerGroup + (threadIdx.x / kWave) * (2 * kWave) + lane;
  const int64_t w1 = w0 + kWave;
  // Blocks are whole 512-byte wave spans (the smallest row is 32 bytes and a
  // block holds a multiple of 16 rows), so a wave's first word can be in range
  // while its second is not: each word has its own guard.
  const bool in0 = w0 < block_words, in1 = w1 < block_words;
  if (out_dir) {
    uint64_t x0 = 0, x1 = 0;
    if (in0) x0 = dev[w0];
    if (in1) x1 = dev[w1];
    if (in0) __hip_atomic_store(host + w0, x0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (in1) __hip_atomic_store(host + w1, x1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  } else {
    uint64_t x0 = 0, x1 = 0;
    if (in0) x0 = __hip_atomic_load(host + w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (in1) x1 = __hip_atomic_load(host + w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (in0) dev[w0] = x0;
    if (in1) dev[w1] = x1;
  }
  if (dev_ks && blockIdx.x == 0) {
    uint16_t* ds = (blockIdx.z == 0 ? dev_ks : dev_vs) + int64_t(dblk) * H;
    uint16_t* hs = (blockIdx.z == 0 ? host_ks : host_vs) + int64_t(hblk) * H;
    for (int hh = threadIdx.x; hh < H; hh += kThreads) {
      if (out_dir)
        __hip_atomic_store(hs + hh, ds[hh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else
        ds[hh] = __hip_atomic_load(hs + hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(uint4* __restrict__ dst,
                                                               const uint4* __restrict__ src,
                                                               int64_t n16) {
  constexpr int kUnroll = 4;
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = r[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// Copies n16 16-byte words from pinned host memory (read directly over the
// host link) to device memory, on the compute queue. The reads are
// system-scope atomic loads, so no cache can serve a stale copy of a staging
// buffer the host has rewritten since an earlier step.
__global__ __launch_bounds__(kThreads) void stage_copy_kernel(uint4* __restrict__ dst,
                                                              const uint64_t* __restrict__ src, int64_t n16) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) {
    const uint64_t lo = __hip_atomic_load(src + 2 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const uint64_t hi = __hip_atomic_load(src + 2 * i + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    dst[i] = make_uint4(uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32));
  }
}

// Reads a buffer chunk by chunk: workgroup b reads bytes [b * kReadChunk,
// +kReadChunk) through a buffer resource (the hardware returns zeros past the
// end of the buffer), four 16-byte non-temporal loads per lane in flight (the
// cache policy of the decode kernel's K/V tiles), and folds them into a
// checksum; the store that keeps the loads alive fires only for one checksum
// value in 2^32.
constexpr int kReadChunk = 65536;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, int64_t bytes,
                                                               uint32_t* __restrict__ sink) {
  constexpr int kUnroll = 4;
  constexpr int kStep = kThreads * 16;
  const int64_t base = int64_t(blockIdx.x) * kReadChunk;
  const int64_t left = bytes - base;
  const int n = int(left < kReadChunk ? left : kReadChunk);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src + base), 0, n, 0x00020000);
  uint32_t acc = 0;
  for (int off = threadIdx.x * 16; off < kReadChunk; off += kStep * kUnroll) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      r[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + u * kStep, 0, 2));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023] = acc;
}

template <typename DST, typename SRC>
int launch_write_float(const pa_pool* p, const void* k_new, const void* v_new, const int64_t* slots,
                       int32_t n, hipStream_t st) {
  const int cpr = p->head_dim / (16 / int(sizeof(DST)));
  const int64_t total = int64_t(n) * p->num_heads * cpr;
  const dim3 grid(unsigned((total + kThreads - 1) / kThreads), 2);
  if (p->head_dim == 64)
    hipLaunchKernelGGL((write_kv_kernel<DST, SRC, 64>), grid, dim3(kThreads), 0, st,
                       static_cast<const SRC*>(k_new), static_cast<const SRC*>(v_new),
                       static_cast<DST*>(p->k_cache), static_cast<DST*>(p->v_cache), slots, n,
                       p->num_heads, p->num_blocks, block_shift(p->block_size), p->err);
  else
    hipLaunchKernelGGL((write_kv_kernel<DST, SRC, 128>), grid, dim3(kThreads), 0, st,
                       static_cast<const SRC*>(k_new), static_cast<const SRC*>(v_new),
                       static_cast<DST*>(p->k_cache), static_cast<DST*>(p->v_cache), slots, n,
                       p->num_heads, p->num_blocks, block_shift(p->block_size), p->err);
  return int(hipGetLastError());
}

template <typename SRC>
int launch_write_i8(const pa_pool* p, const void* k_new, const void* v_new, const int64_t* slots,
                    int32_t n, hipStream_t st) {
  const int64_t waves = int64_t(n) * p->num_heads;
  const dim3 grid(unsigned((waves + (kThreads / kWave) - 1) / (kThreads / kWave)), 2);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st, static_cast<const SRC*>(k_new),
                       static_cast<const SRC*>(v_new), static_cast<int8_t*>(p->k_cache),
                       static_cast<int8_t*>(p->v_cache), static_cast<_Float16*>(p->k_scale),
                       static_cast<_Float16*>(p->v_scale), slots, n, p->num_heads, p->num_blocks,
                       block_shift(p->block_size), p->err);
  };
  if (p->head_dim == 64)
    args(write_kv_i8_kernel<SRC, 64>);
  else
    args(write_kv_i8_kernel<SRC, 128>);
  return int(hipGetLastError());
}

template <typename SRC>
int launch_write_i4(const pa_pool* p, const void* k_new, const void* v_new, const int64_t* slots,
                    int32_t n, hipStream_t st) {
  const int64_t waves = int64_t(n) * p->num_heads;
  const dim3 grid(unsigned((waves + (kThreads / kWave) - 1) / (kThreads / kWave)), 2);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st, static_cast<const SRC*>(k_new),
                       static_cast<const SRC*>(v_new), static_cast<uint8_t*>(p->k_cache),
                       static_cast<uint8_t*>(p->v_cache), static_cast<_Float16*>(p->k_scale),
                       static_cast<_Float16*>(p->v_scale), slots, n, p->num_heads, p->num_blocks,
                       block_shift(p->block_size), p->err);
  };
  if (p->head_dim == 64)
    args(write_kv_i4_kernel<SRC, 64>);
  else
    args(write_kv_i4_kernel<SRC, 128>);
  return int(hipGetLastError());
}

}  // namespace

int launch_write_kv(const pa_pool* p, const void* k_new, const void* v_new, pa_dtype src,
                    const int64_t* slots, int32_t n, void* stream) {
  if (n == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (p->kv_dtype) {
    case PA_F32:
      return src == PA_F32 ? launch_write_float<float, float>(p, k_new, v_new, slots, n, st)
                           : launch_write_float<float, _Float16>(p, k_new, v_new, slots, n, st);
    case PA_F16:
      return src == PA_F32 ? launch_write_float<_Float16, float>(p, k_new, v_new, slots, n, st)
                           : launch_write_float<_Float16, _Float16>(p, k_new, v_new, slots, n, st);
    case PA_I8:
      return src == PA_F32 ? launch_write_i8<float>(p, k_new, v_new, slots, n, st)
                           : launch_write_i8<_Float16>(p, k_new, v_new, slots, n, st);
    case PA_I4:
      return src == PA_F32 ? launch_write_i4<float>(p, k_new, v_new, slots, n, st)
                           : launch_write_i4<_Float16>(p, k_new, v_new, slots, n, st);
  }
  return int(hipErrorInvalidValue);
}

int launch_demote_blocks(const pa_pool* hot, const pa_pool* cold, const int32_t* pairs, int32_t n, void* stream) {
  if (n == 0) return 0;
  const int64_t waves = int64_t(n) * hot->num_heads;
  const dim3 grid(unsigned((waves + (kThreads / kWave) - 1) / (kThreads / kWave)), 2);
  if (cold->kv_dtype == PA_I4) {
    auto go4 = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), pairs, n,
                         static_cast<const _Float16*>(hot->k_cache), static_cast<const _Float16*>(hot->v_cache),
                         static_cast<uint8_t*>(cold->k_cache), static_cast<uint8_t*>(cold->v_cache),
                         static_cast<_Float16*>(cold->k_scale), static_cast<_Float16*>(cold->v_scale),
                         hot->num_heads, hot->num_blocks, cold->num_blocks, cold->err);
    };
    if (hot->head_dim == 64)
      go4(demote_i4_kernel<64>);
    else
      go4(demote_i4_kernel<128>);
    return int(hipGetLastError());
  }
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), pairs, n,
                       static_cast<const _Float16*>(hot->k_cache), static_cast<const _Float16*>(hot->v_cache),
                       static_cast<int8_t*>(cold->k_cache), static_cast<int8_t*>(cold->v_cache),
                       static_cast<_Float16*>(cold->k_scale), static_cast<_Float16*>(cold->v_scale),
                       hot->num_heads, hot->num_blocks, cold->num_blocks, cold->err);
  };
  if (hot->head_dim == 64)
    go(demote_kernel<64>);
  else
    go(demote_kernel<128>);
  return int(hipGetLastError());
}

int launch_copy_blocks(const pa_pool* p, const int32_t* pairs, int32_t n, void* stream) {
  if (n == 0) return 0;
  const int64_t block_bytes = int64_t(p->num_heads) * p->block_size * row_bytes(p->kv_dtype, p->head_dim);
  const dim3 grid(unsigned((block_bytes / 16 + kThreads - 1) / kThreads), unsigned(n), 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), pairs,
                     n, static_cast<char*>(p->k_cache), static_cast<char*>(p->v_cache), block_bytes,
                     static_cast<_Float16*>(p->k_scale), static_cast<_Float16*>(p->v_scale),
                     p->num_heads, p->num_blocks, p->err);
  return int(hipGetLastError());
}

int launch_swap_blocks(const pa_pool* p, const SwapHost& h, const int32_t* pairs, int32_t n, bool out_dir,
                       void* stream) {
  if (n == 0) return 0;
  const int64_t block_bytes = int64_t(p->num_heads) * p->block_size * row_bytes(p->kv_dtype, p->head_dim);
  const int64_t words = block_bytes / 8;   // a multiple of 64: whole 512-byte wave spans
  const dim3 grid(unsigned((words + kSwapWordsPerGroup - 1) / kSwapWordsPerGroup), unsigned(n), 2);
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), pairs,
                     static_cast<uint64_t*>(p->k_cache), static_cast<uint64_t*>(p->v_cache),
                     static_cast<uint64_t*>(h.k), static_cast<uint64_t*>(h.v), words,
                     static_cast<uint16_t*>(p->k_scale), static_cast<uint16_t*>(p->v_scale),
                     static_cast<uint16_t*>(h.k_scale), static_cast<uint16_t*>(h.v_scale), p->num_heads,
                     p->num_blocks, h.num_blocks, out_dir ? 1 : 0, p->err);
  return int(hipGetLastError());
}

int launch_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  int64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n16);
  return int(hipGetLastError());
}

int launch_stage_copy(void* dst, const void* src_device_view, int64_t bytes, void* stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  int64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(stage_copy_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                     static_cast<const uint64_t*>(src_device_view), n16);
  return int(hipGetLastError());
}

int launch_stream_read(const void* src, int64_t bytes, void* sink, void* stream) {
  if (bytes == 0) return 0;
  const int64_t chunks = (bytes + kReadChunk - 1) / kReadChunk;
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(chunks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(src), bytes,
                     static_cast<uint32_t*>(sink));
  return int(hipGetLastError());
}

}  // namespace pa
