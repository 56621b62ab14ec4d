// Paged decode attention for gfx950.
//
// Computes, for every sequence s and head h, softmax(q . k_t * scale) v over
// the sequence's first ctx[s] tokens ("One Deep Concept #01 — PagedAttention:
// From Operating System Virtual Memory to Large Language Model Memory
// Systems", §2 Background), where token t lives in physical block
// table[s][t / B] at offset t % B ("PagedAttention — 把 KV cache 当虚拟内存页来
// 管理", 实践案例 / 案例 2, with B = 16; the same pages list 32 and 64 as the
// other common block sizes). Decode reads a lot and computes little (same
// note, 学到什么), so the kernel is built around HBM streaming, not matrix cores.
//
// Units. One (block, head) tile is B rows of head_dim elements, contiguous in
// the pool. The kernel walks every tile as B / 16 units of 16 rows, so one
// code path serves all block sizes; unit u of a sequence lives in table entry
// u / (B / 16), slice u % (B / 16) of that tile.
//
// Work decomposition. A partition is a run of whole blocks; in single-pass
// mode it covers the whole context. A workgroup (4 waves) takes one
// (sequence, head) and one or more consecutive partitions of it; its waves
// own whole units (unit j goes to wave j % 4), so the 4 waves read adjacent
// units, and each keeps its own online-softmax state: the hot loop has no
// barriers. Short split partitions with few per sequence go a wave each
// instead (a workgroup covers 4 of them).
//
// Tile mapping. A wave reads one 16-row unit with NLD 16-byte loads per lane;
// load i of lane l covers bytes [i*1024 + 16*l, +16) of the unit, so every
// load instruction moves 1 KiB contiguous. In bytes-per-row terms, the 16
// rows split into groups of TPI = 64 / CPT rows per load, CPT lanes per row
// (CPT = row bytes / 16). Lane l therefore always sees the same CPT-th slice
// of head_dim (its "column", l % CPT) of rows i*TPI + l / CPT.
//
// Per unit, per lane: the partial dot of its slice with q for each of its NLD
// rows, summed over the CPT lanes of the row with DPP row operations (no LDS);
// then an fp32 online-softmax update on the lane's own rows in base 2
// (logits pre-multiplied by log2 e), and acc[e] += p * v for its slice. Lanes
// of different row groups are independent softmax streams until a partition
// ends for the wave: its streams then meet across lanes (log-sum-exp
// identity) and the wave parks the partition's partial in LDS; the last wave
// of the workgroup to finish (an LDS counter, no barrier) merges the parked
// partials of every partition and writes them.
//
// Masking: only the last unit of a sequence can be partial. Rows at t >= ctx
// get logit -inf and their raw K/V registers are zeroed before use, so stale
// or NaN data in unused slots never reaches the result. A table entry outside
// the pool flags the device error word and its block is treated as empty.
//
// Split-K. A partition writes m (largest logit, natural units), l (sum of
// exp(logit - m)) and o (its normalised output, fp32) into the workspace; the
// reduce kernel merges partitions as out = sum w_p o_p / sum w_p with
// w_p = exp(m_p - M) l_p. Sequences with one partition are written directly.
//
// Mixed-precision pages. With an fp16 hot pool, the table holds the int8 (or
// int4) cold blocks and the last unit of every sequence comes from its hot
// block: the wave that owns that unit reads its fp16 rows together with its
// first tile, in the cold pool's lane layout (each lane 16 values of a row),
// and folds them into the same softmax stream.
//
// XCD-aware order. Workgroup ids are dealt to the 8 XCDs round-robin; groups
// of 4 consecutive work items are steered onto one XCD, while the deal stays
// interleaved at that granularity for load balance. Without a dispatch order,
// work item w enumerates (partition, head, sequence) with the sequence
// fastest. With one (e.g. longest first) the items of each partition follow
// the order's ranks, in one of two schedules: PA_SCHED_HEADS runs all heads
// of a sequence together (an XCD takes 4 adjacent heads, 4 adjacent tiles of
// each block: the faster layout when nothing is shared), PA_SCHED_SHARED
// takes ranks in groups of 4 and runs a group head by head (an XCD takes one
// head of 4 adjacent ranks, so samples that share blocks read them through
// one L2 at about the same time).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Waves per workgroup: each owns every kWaves-th unit of the workgroup's range.
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
constexpr int kWaves = PA_DECODE_WAVES;
constexpr int kThreads = kWaves * kWave;
constexpr int kXcds = 8;
constexpr int kXcdGroup = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "no logit yet" so exp2(m - m_new) stays defined
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3 for raw dword access on gfx9-family parts

// Cache policy of the K/V tile loads (buffer instruction aux bits; 2 = nt,
// non-temporal): KV rows are read once per step, so they are streamed —
// unless blocks are shared by several sequences of the batch (the shared
// schedule): then the loads are temporal (aux 0), so that the other readers
// of a block find it in L2 (shared-prefix batch: 88 -> 77 us; on a batch
// without sharing, temporal loads cost 12%).
#ifndef PA_DECODE_LOAD_AUX
#define PA_DECODE_LOAD_AUX 2
#endif
constexpr int kLoadAuxShared = 0;
// Tiles each wave keeps in flight beyond the one it works on: 1 = register
// double buffering (~110 VGPRs, 4 waves per SIMD); 0 = one tile per wave and
// more waves per SIMD (~60 VGPRs).
#ifndef PA_DECODE_PREFETCH
#define PA_DECODE_PREFETCH 1
#endif
// Split launches with partitions of at most this many tokens give each wave
// a partition of its own.
#ifndef PA_DECODE_WAVE_PART_MAX
#define PA_DECODE_WAVE_PART_MAX 512
#endif
constexpr int kWavePartMaxTokens = PA_DECODE_WAVE_PART_MAX;
// Split launches with many partitions per sequence: a workgroup streams
// several consecutive partitions, about kGroupTokens tokens, as long as the
// launch keeps at least kMinGroups workgroups.
#ifndef PA_DECODE_GROUP_TOKENS
#define PA_DECODE_GROUP_TOKENS 8192
#endif
#ifndef PA_DECODE_MIN_GROUPS
#define PA_DECODE_MIN_GROUPS 2048
#endif
constexpr int kGroupTokens = PA_DECODE_GROUP_TOKENS;
constexpr int kMinGroups = PA_DECODE_MIN_GROUPS;
// At most this many partitions per workgroup: their per-wave partials wait in
// LDS, kWaves * (D + 2) floats each (33 KB at D = 128).
constexpr int kMaxGroupParts = 16;

// Minimum waves per SIMD the register allocator must leave room for.
#ifndef PA_DECODE_MIN_WAVES
#define PA_DECODE_MIN_WAVES (PA_DECODE_PREFETCH ? 4 : 8)
#endif

// int4 pools: a tag type for bytes that hold two codes (each nibble code + 8,
// even dim in the low nibble).
struct Int4 {};
template <typename KV>
struct KvBits {
  static constexpr int value = 8 * int(sizeof(KV));
};
template <>
struct KvBits<Int4> {
  static constexpr int value = 4;
};
template <typename KV>
constexpr bool kQuantKV = std::is_same<KV, int8_t>::value || std::is_same<KV, Int4>::value;

// A lane loads 16-byte chunks (int4: 8-byte chunks, 16 values, so that q and
// the accumulators of a lane stay at 16 values each and the lane layout is
// int8's at the same head_dim).
template <typename KV, int D>
struct Geo {
  static constexpr int kChunkBytes = std::is_same<KV, Int4>::value ? 8 : 16;
  using Chunk = typename std::conditional<kChunkBytes == 8, uint2, uint4>::type;
  static constexpr int kRowBytes = D * KvBits<KV>::value / 8;
  static constexpr int kCPT = kRowBytes / kChunkBytes;   // lanes per row
  static constexpr int kTPI = kWave / kCPT;        // rows per wave-wide load
  static constexpr int kNLD = kTileRows / kTPI;    // loads per lane per unit
  static constexpr int kEPC = kChunkBytes * 8 / KvBits<KV>::value;  // elements per lane per row
  static constexpr int kLoadBytes = kWave * kChunkBytes;     // one wave-wide load
  static constexpr int kTileBytes = kTileRows * kRowBytes;   // one 16-row unit
  static_assert(kCPT >= 4 && kCPT <= 32, "unsupported row size");
};

struct Params {
  const void* q;
  void* out;
  const char* k;
  const char* v;
  const _Float16* k_scale;
  const _Float16* v_scale;
  const int32_t* tables;
  int64_t max_tokens;       // contiguous layout row length
  const int32_t* ctx;
  const int32_t* order;     // optional schedule: the r-th sequence dispatched is order[r]
  int32_t sched;            // PA_SCHED_HEADS or PA_SCHED_SHARED (with order)
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_blocks;
  int32_t max_ctx;
  int32_t partition_units;  // 16-row units per partition
  int32_t parts_per_group;  // shared partitions: how many one workgroup streams
  int32_t unit_shift;       // log2(block_size / 16)
  int32_t num_partitions;
  float scale_log2;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t* err;
  // Fused write (float pools): row s of k_new / v_new is sequence s's newest
  // token, stored at slots[s]; null slots = no write.
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
  int32_t new_is_f32;
  // Mixed-precision pages: fp16 hot pool and each sequence's hot block.
  const char* hot_k;
  const char* hot_v;
  const int32_t* hot_blocks;
  int32_t num_hot;
};

// Bijection from dispatch order g to work item w: inside every chunk of
// kXcds * kXcdGroup ids, the ids that land on XCD x (g % kXcds == x) take the
// kXcdGroup consecutive work items x*kXcdGroup ... ; a ragged tail maps to itself.
__device__ __forceinline__ int xcd_remap(int g, int total) {
  constexpr int kChunk = kXcds * kXcdGroup;
  const int full = (total / kChunk) * kChunk;
  if (g >= full) return g;
  const int base = g - g % kChunk;
  const int r = g % kChunk;
  return base + (r % kXcds) * kXcdGroup + r / kXcds;
}

// q slice of one lane, in the form its dot product wants.
template <typename KV, typename QT, int EPC>
struct QSlice {
  float f[EPC];
  __device__ void load(const QT* src) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) f[e] = float(src[e]);
  }
};

template <>
struct QSlice<_Float16, _Float16, 8> {
  uint32_t w[4];
  __device__ void load(const _Float16* src) {
    const uint4 r = *reinterpret_cast<const uint4*>(src);
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
  }
};

// Codes as fp16 without a conversion instruction per value. A byte b placed
// under the exponent byte 0x64 reads as the fp16 value 1024 + b (ulp 1); int8
// codes, flipped to b = c + 128, become 1152 + c. An int4 nibble n placed in
// the high nibble of a byte under 0x54 reads as 64 + n (ulp 1/16 times 16),
// so a code c = n - 8 becomes 72 + c. One v_perm_b32 builds two such fp16
// values from two code bytes; the dot with q then runs on v_dot2c_f32_f16
// (exact fp16 products, fp32 sums) and the V sum on v_fma_mix_f32 (fp32
// weight times fp16 value, fp32 sum). The constant offsets are taken off once
// per row of logits (offset * sum of q) and once per hand-over of the
// weighted V sum (offset * sum of the weights applied).
constexpr uint32_t kPermLo = 0x04010400u;   // bytes b0, b1 of the second operand under the first's byte 0
constexpr uint32_t kPermHi = 0x04030402u;   // bytes b2, b3
constexpr float kInt8Offset = 1152.f;       // 1024 + 128
constexpr float kInt4Offset = 72.f;         // 64 + 8

__device__ __forceinline__ uint32_t i8_pair(uint32_t flipped, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, flipped, sel);
}
__device__ __forceinline__ uint32_t i4_pair(uint32_t high_nibbles, uint32_t sel) {
  return __builtin_amdgcn_perm(0x54545454u, high_nibbles, sel);
}

// int8 pools with fp16 q: q as fp16 pairs in natural order (the order
// i8_pair gives the codes of a word), and as floats for the fp16 hot rows of
// mixed pages (dead, and dropped, in the other kernels).
template <>
struct QSlice<int8_t, _Float16, 16> {
  uint32_t w[8];
  float f[16];
  __device__ void load(const _Float16* src) {
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 b = reinterpret_cast<const uint4*>(src)[1];
    const uint32_t n[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      w[m] = n[m];
      f[2 * m] = lo_f16(n[m]);
      f[2 * m + 1] = hi_f16(n[m]);
    }
  }
};

// int4 pools with fp16 q. Word j of an 8-byte chunk holds dims 8j .. 8j+7,
// the even ones in the low nibbles; i4_pair gives (8j, 8j+2), (8j+4, 8j+6)
// from the even nibbles and (8j+1, 8j+3), (8j+5, 8j+7) from the odd ones, so
// q is kept in pairs of that order.
template <>
struct QSlice<Int4, _Float16, 16> {
  uint32_t w[8];
  float f[16];
  __device__ void load(const _Float16* src) {
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 b = reinterpret_cast<const uint4*>(src)[1];
    const uint32_t n[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};   // n[m] = (q[2m], q[2m+1])
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[4 * j + 0] = __builtin_amdgcn_perm(n[4 * j + 1], n[4 * j], 0x05040100u);      // q[8j], q[8j+2]
      w[4 * j + 1] = __builtin_amdgcn_perm(n[4 * j + 3], n[4 * j + 2], 0x05040100u);  // q[8j+4], q[8j+6]
      w[4 * j + 2] = __builtin_amdgcn_perm(n[4 * j + 1], n[4 * j], 0x07060302u);      // q[8j+1], q[8j+3]
      w[4 * j + 3] = __builtin_amdgcn_perm(n[4 * j + 3], n[4 * j + 2], 0x07060302u);  // q[8j+5], q[8j+7]
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      f[2 * m] = lo_f16(n[m]);
      f[2 * m + 1] = hi_f16(n[m]);
    }
  }
};

// Offset carried by the logits of a path (0: none).
template <typename KV, typename QT>
constexpr float kKOffset = std::is_same<QT, _Float16>::value
                               ? (std::is_same<KV, int8_t>::value ? kInt8Offset
                                  : std::is_same<KV, Int4>::value ? kInt4Offset : 0.f)
                               : (std::is_same<KV, Int4>::value ? 8.f : 0.f);
// Offset carried by the values of a path's V sum (0: none).
template <typename KV>
constexpr float kVOffset = std::is_same<KV, int8_t>::value ? kInt8Offset
                           : std::is_same<KV, Int4>::value ? kInt4Offset : 0.f;

template <typename KV, typename QT, int EPC>
__device__ __forceinline__ float dot16(const uint4& r, const QSlice<KV, QT, EPC>& q) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  float s = 0.f;
  if constexpr (std::is_same<KV, float>::value) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(__builtin_bit_cast(float, w[j]), q.f[j], s);
  } else if constexpr (std::is_same<KV, _Float16>::value) {
    if constexpr (std::is_same<QT, _Float16>::value) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_fdot2(as_h2(w[j]), as_h2(q.w[j]), s, false);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = fmaf(lo_f16(w[j]), q.f[2 * j], s);
        s = fmaf(hi_f16(w[j]), q.f[2 * j + 1], s);
      }
    }
  } else if constexpr (std::is_same<QT, _Float16>::value) {
    // int8 codes with fp16 q: sum of q (1152 + c).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = w[j] ^ 0x80808080u;
      s = __builtin_amdgcn_fdot2(as_h2(i8_pair(x, kPermLo)), as_h2(q.w[2 * j]), s, false);
      s = __builtin_amdgcn_fdot2(as_h2(i8_pair(x, kPermHi)), as_h2(q.w[2 * j + 1]), s, false);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s = fmaf(i8_at<0>(w[j]), q.f[4 * j + 0], s);
      s = fmaf(i8_at<1>(w[j]), q.f[4 * j + 1], s);
      s = fmaf(i8_at<2>(w[j]), q.f[4 * j + 2], s);
      s = fmaf(i8_at<3>(w[j]), q.f[4 * j + 3], s);
    }
  }
  return s;
}

template <typename KV, int EPC>
__device__ __forceinline__ void axpy16(float p, const uint4& r, float (&acc)[EPC]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if constexpr (std::is_same<KV, float>::value) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(p, __builtin_bit_cast(float, w[j]), acc[j]);
  } else if constexpr (std::is_same<KV, _Float16>::value) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = fmaf(p, lo_f16(w[j]), acc[2 * j]);
      acc[2 * j + 1] = fmaf(p, hi_f16(w[j]), acc[2 * j + 1]);
    }
  } else {
    // int8 codes: acc += p (1152 + c).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = w[j] ^ 0x80808080u;
      const h2_t lo = as_h2(i8_pair(x, kPermLo));
      const h2_t hi = as_h2(i8_pair(x, kPermHi));
      acc[4 * j + 0] = fmaf(p, float(lo.x), acc[4 * j + 0]);
      acc[4 * j + 1] = fmaf(p, float(lo.y), acc[4 * j + 1]);
      acc[4 * j + 2] = fmaf(p, float(hi.x), acc[4 * j + 2]);
      acc[4 * j + 3] = fmaf(p, float(hi.y), acc[4 * j + 3]);
    }
  }
}

// int4 chunks: 8 bytes, 16 unsigned nibbles n = code + 8. The low nibbles of
// word j are dims 8j, 8j+2, 8j+4, 8j+6, the high ones 8j+1, .... With fp16 q
// both products go through i4_pair (above). With fp32 q the logits take each
// byte of a masked word to float in one instruction (v_cvt_f32_ubyte0..3);
// the masked words pass through an empty asm statement so that the compiler,
// which knows they hold nibbles, does not fold each conversion into a
// bit-field extract plus a conversion.
__device__ __forceinline__ void nibble_words(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = w & 0x0F0F0F0Fu;
  hi = (w >> 4) & 0x0F0F0F0Fu;
  asm("" : "+v"(lo), "+v"(hi));
}
template <typename KV, typename QT, int EPC>
__device__ __forceinline__ float dot16(const uint2& r, const QSlice<KV, QT, EPC>& q) {
  static_assert(std::is_same<KV, Int4>::value && EPC == 16, "8-byte chunks are int4");
  const uint32_t w[2] = {r.x, r.y};
  float s = 0.f;
  if constexpr (std::is_same<QT, _Float16>::value) {
    // Sum of q (72 + c): even dims' nibbles moved up into the high nibble.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t ev = (w[j] << 4) & 0xF0F0F0F0u;
      const uint32_t od = w[j] & 0xF0F0F0F0u;
      s = __builtin_amdgcn_fdot2(as_h2(i4_pair(ev, kPermLo)), as_h2(q.w[4 * j + 0]), s, false);
      s = __builtin_amdgcn_fdot2(as_h2(i4_pair(ev, kPermHi)), as_h2(q.w[4 * j + 1]), s, false);
      s = __builtin_amdgcn_fdot2(as_h2(i4_pair(od, kPermLo)), as_h2(q.w[4 * j + 2]), s, false);
      s = __builtin_amdgcn_fdot2(as_h2(i4_pair(od, kPermHi)), as_h2(q.w[4 * j + 3]), s, false);
    }
  } else {
    // fp32 q: sum of q n with n = c + 8.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t lo, hi;
      nibble_words(w[j], lo, hi);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        s = fmaf(float((lo >> (8 * b)) & 0xFFu), q.f[8 * j + 2 * b], s);
        s = fmaf(float((hi >> (8 * b)) & 0xFFu), q.f[8 * j + 2 * b + 1], s);
      }
    }
  }
  return s;
}

// acc += p (72 + c) over the 16 codes of an 8-byte int4 chunk.
template <typename KV, int EPC>
__device__ __forceinline__ void axpy16(float p, const uint2& r, float (&acc)[EPC]) {
  static_assert(std::is_same<KV, Int4>::value && EPC == 16, "8-byte chunks are int4");
  const uint32_t w[2] = {r.x, r.y};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t ev = (w[j] << 4) & 0xF0F0F0F0u;
    const uint32_t od = w[j] & 0xF0F0F0F0u;
    const h2_t e01 = as_h2(i4_pair(ev, kPermLo)), e23 = as_h2(i4_pair(ev, kPermHi));
    const h2_t o01 = as_h2(i4_pair(od, kPermLo)), o23 = as_h2(i4_pair(od, kPermHi));
    acc[8 * j + 0] = fmaf(p, float(e01.x), acc[8 * j + 0]);
    acc[8 * j + 2] = fmaf(p, float(e01.y), acc[8 * j + 2]);
    acc[8 * j + 4] = fmaf(p, float(e23.x), acc[8 * j + 4]);
    acc[8 * j + 6] = fmaf(p, float(e23.y), acc[8 * j + 6]);
    acc[8 * j + 1] = fmaf(p, float(o01.x), acc[8 * j + 1]);
    acc[8 * j + 3] = fmaf(p, float(o01.y), acc[8 * j + 3]);
    acc[8 * j + 5] = fmaf(p, float(o23.x), acc[8 * j + 5]);
    acc[8 * j + 7] = fmaf(p, float(o23.y), acc[8 * j + 7]);
  }
}

// W consecutive 32-bit words from a 16-byte aligned address (8-byte aligned
// when W == 2), with the widest loads that fit.
template <typename T, int W>
__device__ __forceinline__ void load_words(const T* src, uint32_t (&w)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
      const uint4 r = reinterpret_cast<const uint4*>(src)[j];
      w[4 * j] = r.x;
      w[4 * j + 1] = r.y;
      w[4 * j + 2] = r.z;
      w[4 * j + 3] = r.w;
    }
  } else {
    static_assert(W == 2, "chunk shape");
    const uint2 r = *reinterpret_cast<const uint2*>(src);
    w[0] = r.x;
    w[1] = r.y;
  }
}

// Element e of a chunk of T values packed in 32-bit words, as float (exact).
template <typename T, int W>
__device__ __forceinline__ float word_elem(const uint32_t (&w)[W], int e) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(float, w[e]);
  } else {
    return e % 2 ? hi_f16(w[e / 2]) : lo_f16(w[e / 2]);
  }
}

template <typename QT>
__device__ __forceinline__ QT to_out(float x) {
  return QT(x);   // fp32 -> fp16 conversion rounds to nearest even
}

// NEW: element type of the fused-write source rows (void = no fused write).
// kMixed: an int8 or int4 cold pool (KV) through the table plus an fp16 hot
// block per sequence.
// kWavePart: each wave owns one whole partition (a workgroup covers kWaves
// consecutive partitions of one (sequence, head)). Otherwise the kWaves waves
// share each partition, taking every kWaves-th unit, and a workgroup streams
// p.parts_per_group consecutive partitions; a wave parks its share of a
// partition's (m, l, o) when its last unit of the partition is done, with the
// next partition's loads already in flight.
// kCached: temporal tile loads (blocks shared within the batch).
template <typename KV, typename QT, int D, bool kPaged, typename NEW, bool kMixed = false, bool kWavePart = false,
          bool kCached = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PA_DECODE_MIN_WAVES)))
void decode_kernel(Params p, const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_ctx,
                   const int64_t* __restrict__ new_slots) {
  // tables / seq_ctx / new_slots are p.tables / p.ctx / p.slots, passed as
  // restrict arguments so the compiler knows the kernel's stores (pool,
  // output) never alias them and keeps reading them through the scalar cache.
  using G = Geo<KV, D>;
  constexpr int CPT = G::kCPT, TPI = G::kTPI, NLD = G::kNLD, EPC = G::kEPC;
  using Chunk = typename G::Chunk;
  constexpr bool kInt8 = std::is_same<KV, int8_t>::value;
  constexpr bool kInt4 = std::is_same<KV, Int4>::value;
  constexpr bool kQuant = kQuantKV<KV>;

  const int parts_per_group = kWavePart ? kWaves : p.parts_per_group;
  const int groups = (p.num_partitions + parts_per_group - 1) / parts_per_group;
  const int total = p.num_seqs * p.num_heads * groups;
  const int w = xcd_remap(int(blockIdx.x), total);
  int s, h;
  const int pgroup = w / (p.num_seqs * p.num_heads);
  if (p.order) {
    const int r = w % (p.num_seqs * p.num_heads);
    int rank;
    if (p.sched == PA_SCHED_HEADS) {
      // Ranks one after the other, all heads of a rank together.
      rank = r / p.num_heads;
      h = r - rank * p.num_heads;
    } else {
      // Ranks in groups of kXcdGroup, a group's items head by head, so the
      // group's sequences with one head form kXcdGroup consecutive items.
      const int g = r / (kXcdGroup * p.num_heads);
      const int gs = min(kXcdGroup, p.num_seqs - g * kXcdGroup);
      const int q_in = r - g * kXcdGroup * p.num_heads;
      h = q_in / gs;
      rank = g * kXcdGroup + q_in % gs;
    }
    s = p.order[rank];
    if (unsigned(s) >= unsigned(p.num_seqs)) {
      if (threadIdx.x == 0) flag_error(p.err, PA_DEV_BAD_CONTEXT);
      return;
    }
  } else {
    s = w % p.num_seqs;
    h = (w / p.num_seqs) % p.num_heads;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_uniform(threadIdx.x / kWave);
  // The wave's partition (shared partitions: the workgroup's first one).
  const int part = kWavePart ? pgroup * kWaves + wave : pgroup * parts_per_group;
  const int grp = lane / CPT;
  const int col = lane % CPT;
  const int64_t sh = int64_t(s) * p.num_heads + h;
  const int ushift = p.unit_shift;
  const int bshift = ushift + 4;                                  // log2(block size)
  const int64_t head_stride = int64_t(G::kTileBytes) << ushift;   // one (block, head) tile
  const int64_t block_stride = int64_t(p.num_heads) * head_stride;
  const int unit_begin = part * p.partition_units;
  // This wave's units are first, first + ustride, first + 2 ustride, ...:
  // every kWaves-th unit of the shared partition, or all of its own one.
  constexpr int ustride = kWavePart ? 1 : kWaves;
  const int first = unit_begin + (kWavePart ? 0 : wave);
  const int32_t* trow = kPaged ? tables + int64_t(s) * p.max_blocks : nullptr;

  // Shared partitions: the waves that are done are counted in LDS, and the
  // last one merges the workgroup's partials. The count is zeroed before any
  // load is issued, so this barrier waits for nothing but the other waves'
  // start.
  __shared__ int s_done;
  if constexpr (!kWavePart) {
    if (threadIdx.x == 0) s_done = 0;
    __syncthreads();
  }

  // Loads that do not depend on the context length go out together with it:
  // the table entries of the wave's first two units (inside the row; unused
  // if past the context) and its q slice. The first unit then waits for one
  // round trip.
  int ctx = seq_ctx[s];
  int e0 = 0, e1 = 0;
  if constexpr (kPaged) {
    e0 = (first >> ushift) < p.max_blocks ? trow[first >> ushift] : 0;
    e1 = ((first + ustride) >> ushift) < p.max_blocks ? trow[(first + ustride) >> ushift] : 0;
  }
  QSlice<KV, QT, EPC> qs;
  qs.load(reinterpret_cast<const QT*>(p.q) + sh * D + col * EPC);
  // Fused write (float pools): the new row's slot and this lane's chunk of
  // the row, fetched speculatively with the rest (used only by the wave that
  // owns the sequence's last block).
  constexpr bool kFusable = kPaged && !kQuant && !std::is_same<NEW, void>::value;
  using NewT = typename std::conditional<std::is_same<NEW, void>::value, float, NEW>::type;
  constexpr int kNewWords = EPC * int(sizeof(NewT)) / 4;        // 32-bit words per lane chunk
  int64_t new_slot = -1;
  uint32_t rk[kNewWords], rv[kNewWords];                       // raw chunk, converted later
  if constexpr (kFusable) {
    new_slot = new_slots[s];
    const NewT* ksrc = static_cast<const NewT*>(p.k_new) + sh * D + col * EPC;
    const NewT* vsrc = static_cast<const NewT*>(p.v_new) + sh * D + col * EPC;
    load_words(ksrc, rk);
    load_words(vsrc, rv);
  }

  static_assert(!kMixed || (kQuant && kPaged && std::is_same<NEW, void>::value),
                "mixed pages: int8 or int4 cold pool");
  int hot_blk = 0;
  if constexpr (kMixed) hot_blk = p.hot_blocks[s];
  const bool bad_ctx = ctx < 0 || ctx > p.max_ctx;
  if (bad_ctx) ctx = ctx < 0 ? 0 : p.max_ctx;
  const int nunits = (ctx + kTileRows - 1) / kTileRows;
  const int seq_parts = nunits == 0 ? 1 : (nunits + p.partition_units - 1) / p.partition_units;
  if (part >= seq_parts) return;
  // Units read through the table (mixed pages: all but the last, hot one).
  const int table_units = kMixed ? max(nunits - 1, 0) : nunits;
  const int unit_end = min(unit_begin + (kWavePart ? 1 : parts_per_group) * p.partition_units, table_units);
  const int iters = first < unit_end ? (unit_end - first + ustride - 1) / ustride : 0;

  // Table entry of the wave's k-th unit. Reads are wave-uniform and the loop
  // stores nothing to global memory, so they go through the scalar cache and
  // are counted apart from the vector loads: each is issued half an iteration
  // before it is used.
  auto entry = [&](int k) -> int {
    if constexpr (kPaged) {
      return trow[(first + ustride * k) >> ushift];
    } else {
      return 0;
    }
  };
  // Byte offset of unit b of head h (its table entry is phys); *ok is false
  // for an entry outside the pool (the unit is then read from block 0 and
  // masked).
  auto tile_offset = [&](int b, int phys, bool* ok) -> int64_t {
    if constexpr (kPaged) {
      *ok = unsigned(phys) < unsigned(p.num_blocks);
      return (*ok ? int64_t(phys) : 0) * block_stride + int64_t(h) * head_stride +
             int64_t(b & ((1 << ushift) - 1)) * G::kTileBytes;
    } else {
      *ok = true;
      return (sh * p.max_tokens + int64_t(b) * kTileRows) * G::kRowBytes;
    }
  };
  // A unit is read through a buffer resource built per unit (uniform base in
  // SGPRs, loop-invariant lane offset): no 64-bit vector address arithmetic in
  // the loop, and the hardware clamps any access outside the unit to zero.
  auto load_tile = [&](const char* base, int64_t off, Chunk (&r)[NLD]) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), 0, G::kTileBytes, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      if constexpr (G::kChunkBytes == 16)
        r[i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + i * G::kLoadBytes, 0,
                                                         kCached ? kLoadAuxShared : PA_DECODE_LOAD_AUX));
      else
        r[i] = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, lane * 8 + i * G::kLoadBytes, 0,
                                                        kCached ? kLoadAuxShared : PA_DECODE_LOAD_AUX));
  };
  struct TileRef {
    int b;
    int phys;
    bool ok;
    float kscale, vscale;
  };
  // Issue the loads of the wave's k-th unit (table entry phys) into (kr, vr).
  auto fetch = [&](int k, int phys, Chunk (&kr)[NLD], Chunk (&vr)[NLD]) -> TileRef {
    TileRef t;
    t.b = first + k * ustride;
    t.phys = phys;
    const int64_t off = tile_offset(t.b, phys, &t.ok);
    load_tile(p.k, off, kr);
    load_tile(p.v, off, vr);
    if constexpr (kQuant) {
      // A masked unit (entry outside the pool) weighs nothing, whatever
      // block 0's scale holds. (Loaded unconditionally, then selected: a
      // conditional load would become a branch around it.)
      const int64_t si = int64_t(t.ok ? phys : 0) * p.num_heads + h;
      const float ks = float(p.k_scale[si]);
      const float vs = float(p.v_scale[si]);
      t.kscale = t.ok ? ks : 0.f;
      t.vscale = t.ok ? vs : 0.f;
    } else {
      t.kscale = 1.f;
      t.vscale = 1.f;
    }
    return t;
  };

  float m = kNegBig, l = 0.f;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  // Quantised pools: the loop works on codes plus a constant offset (see
  // kKOffset / kVOffset). A logit is then sum q (c + off_k) - off_k sum q
  // (q_bias = off_k sum q over the row, set before the first unit), and
  // every value of the lane's rows carries off_v, so the lane also keeps
  // vbias = sum of the weights it has applied (rescaled with acc) and takes
  // off_v vbias off acc when it hands over.
  constexpr float kKOff = kKOffset<KV, QT>;
  constexpr float kVOff = kVOffset<KV>;
  float q_bias = 0.f, vbias = 0.f;
  auto prepare_q = [&]() {
    if constexpr (kKOff != 0.f) {
      float qsum = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) qsum += qs.f[e];
      q_bias = kKOff * group_sum<CPT>(qsum);
    }
  };
  // A bad table entry is only recorded here and flagged after the loop: a
  // store inside the loop would stop the compiler from fetching table entries
  // and scales through the scalar cache.
  bool bad_entry = false;

  // Fused write of the sequence's new token: the owning wave's lanes that
  // hold row new_row of the last unit patch the new row into the unit's
  // registers when that unit comes (if its physical block is the slot's),
  // and store the row after the loop.
  int new_row = -1;
  bool patched = false, bad_slot = false;
  int64_t new_dst = 0;
  uint4 nk = make_uint4(0u, 0u, 0u, 0u), nv = nk;
  const int64_t in_block = (int64_t(1) << bshift) - 1;   // offset mask inside a block
  if constexpr (kFusable) {
    if (new_slots != nullptr && new_slot >= 0) {
      const bool owner = unit_end == nunits && nunits > 0 && nunits - 1 >= first &&
                         (nunits - 1 - first) % ustride == 0;
      if (nunits == 0 || (new_slot & in_block) != ((ctx - 1) & in_block)) {
        bad_slot = part == 0 && wave == 0;       // reported once per (sequence, head)
      } else if (owner) {
        new_row = (ctx - 1) % kTileRows;
      }
    }
  }
  // The new row in the pool's element type (issued after the first tile's
  // loads so their latencies overlap).
  auto convert_new_row = [&]() {
    if constexpr (kFusable) {
      if (new_row >= 0) {
        KV kv_k[EPC], kv_v[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          kv_k[e] = KV(word_elem<NewT>(rk, e));
          kv_v[e] = KV(word_elem<NewT>(rv, e));
        }
        nk = *reinterpret_cast<const uint4*>(kv_k);
        nv = *reinterpret_cast<const uint4*>(kv_v);
      }
    }
  };

  // Hand over the wave's partial result for partition pidx and restart its
  // stream. The wave's TPI row-group streams meet first, across lanes (the
  // lanes of one column, CPT apart), by the log-sum-exp identity. A wave that
  // owns its partition then writes (m, l, o) — or the output when the
  // sequence has one partition. Waves that share partitions park the partial
  // in their own LDS slot; the workgroup's partitions are merged once, after
  // the loop.
  float* s_o = nullptr;       // [parts_per_group][kWaves][D] unnormalised o
  float* s_m = nullptr;       // [parts_per_group][kWaves] running max (base 2)
  float* s_l = nullptr;       // [parts_per_group][kWaves] softmax denominators
  if constexpr (!kWavePart) {
    extern __shared__ __align__(16) float lds_partials[];
    s_o = lds_partials;
    s_m = s_o + parts_per_group * kWaves * D;
    s_l = s_m + parts_per_group * kWaves;
  }
  auto emit = [&](int pidx, int d, float M, float L, float O) {
    const float res = L > 0.f ? O / L : 0.f;
    if (seq_parts == 1) {
      reinterpret_cast<QT*>(p.out)[sh * D + d] = to_out<QT>(res);
    } else {
      const int64_t slot = sh * p.num_partitions + pidx;
      p.ws_o[slot * D + d] = res;
      if (d == 0) {
        p.ws_m[slot] = M * kLn2;
        p.ws_l[slot] = L;
      }
    }
  };
  auto flush = [&](int pidx) {
    float fm = m, fl = l, fa[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) fa[e] = kVOff != 0.f ? acc[e] - kVOff * vbias : acc[e];
#pragma unroll
    for (int mask = CPT; mask < kWave; mask <<= 1) {
      const float m2 = __shfl_xor(fm, mask);
      const float l2 = __shfl_xor(fl, mask);
      const float mn = fmaxf(fm, m2);
      const float a = __builtin_amdgcn_exp2f(fm - mn);
      const float b = __builtin_amdgcn_exp2f(m2 - mn);
      fl = fl * a + l2 * b;
#pragma unroll
      for (int e = 0; e < EPC; ++e) fa[e] = fa[e] * a + __shfl_xor(fa[e], mask) * b;
      fm = mn;
    }
    if (grp == 0) {
      if constexpr (kWavePart) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) emit(pidx, col * EPC + e, fm, fl, fa[e]);
      } else {
        const int slot = (pidx - part) * kWaves + wave;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s_o[slot * D + col * EPC + e] = fa[e];
        if (col == 0) {
          s_m[slot] = fm;
          s_l[slot] = fl;
        }
      }
    }
    m = kNegBig;
    l = 0.f;
    vbias = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  };
  // The unit that starts the workgroup's next partition (shared partitions).
  // Partitions are a multiple of kWaves units whenever a workgroup streams
  // more than one, so every wave holds units of each full partition and hands
  // over every partition once: at its last unit of the partition, or after
  // the loop for the last one (an empty stream if it holds none of it).
  int next_flush = unit_begin + p.partition_units;

  // Online-softmax update with one unit.
  auto process = [&](const TileRef& t, Chunk (&kr)[NLD], Chunk (&vr)[NLD]) {
    bad_entry |= !t.ok;
    const int t0 = t.b * kTileRows;
    if constexpr (kFusable) {
      if (new_row >= 0 && t.b == nunits - 1) {
        if (t.ok && int64_t(t.phys) == (new_slot >> bshift)) {
          patched = true;
          new_dst = int64_t(t.phys) * block_stride + int64_t(h) * head_stride +
                    (new_slot & in_block) * G::kRowBytes + col * 16;
#pragma unroll
          for (int i = 0; i < NLD; ++i) {
            if (i == new_row / TPI && grp == new_row % TPI) {
              kr[i] = nk;
              vr[i] = nv;
            }
          }
        } else {
          bad_slot = true;
        }
      }
    }
    float sc[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (kKOff != 0.f)
        sc[i] = (group_sum<CPT>(dot16(kr[i], qs)) - q_bias) * (t.kscale * p.scale_log2);
      else
        sc[i] = group_sum<CPT>(dot16(kr[i], qs)) * (t.kscale * p.scale_log2);
    }
    if (t0 + kTileRows > ctx || !t.ok) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        if (!t.ok || t0 + i * TPI + grp >= ctx) {
          sc[i] = -INFINITY;
          vr[i] = Chunk{};
        }
      }
    }
    float bmax = sc[0];
#pragma unroll
    for (int i = 1; i < NLD; ++i) bmax = fmaxf(bmax, sc[i]);
    const float mn = fmaxf(m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
    if constexpr (kVOff != 0.f) vbias *= alpha;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const float pi = __builtin_amdgcn_exp2f(sc[i] - mn);
      l += pi;
      axpy16<KV, EPC>(pi * t.vscale, vr[i], acc);
      if constexpr (kVOff != 0.f) vbias += pi * t.vscale;
    }
    m = mn;
    if constexpr (!kWavePart && !kMixed) {
      if (t.b + ustride >= next_flush && next_flush < unit_end) {   // the wave's last unit of a partition
        flush(next_flush / p.partition_units - 1);
        next_flush += p.partition_units;
      }
    }
  };

  // Mixed pages: the hot unit (the sequence's last, fp16, from its hot
  // block), by the wave that owns it. Its loads go out before the wave's
  // first tile's, and it is folded in while that tile is in flight, so the
  // hot block costs no round trip of its own.
  constexpr int kHW = kMixed ? EPC * 2 / 16 : 1;   // 16-byte words of fp16 per lane and row
  const int hu = nunits - 1;
  const bool hot_mine = kMixed && nunits > 0 && hu >= first && hu < unit_begin + p.partition_units &&
                        (hu - first) % ustride == 0;
  uint4 hk[NLD][kHW], hv[NLD][kHW];
  bool hot_ok = false;
  auto hot_load = [&]() {
    if constexpr (kMixed) {
      hot_ok = unsigned(hot_blk) < unsigned(p.num_hot);
      bad_entry |= !hot_ok;
      const int64_t tile = (int64_t(hot_ok ? hot_blk : 0) * p.num_heads + h) * kTileRows * D * 2;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int64_t off = tile + int64_t(i * TPI + grp) * D * 2 + col * EPC * 2;
#pragma unroll
        for (int j = 0; j < kHW; ++j) {
          hk[i][j] = *reinterpret_cast<const uint4*>(p.hot_k + off + 16 * j);
          hv[i][j] = *reinterpret_cast<const uint4*>(p.hot_v + off + 16 * j);
        }
      }
    }
  };
  auto hot_process = [&]() {
    if constexpr (kMixed) {
      const int t0 = hu * kTileRows;
      float sc[NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < kHW; ++j) {
          const uint32_t w[4] = {hk[i][j].x, hk[i][j].y, hk[i][j].z, hk[i][j].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            d = fmaf(lo_f16(w[c]), qs.f[8 * j + 2 * c], d);
            d = fmaf(hi_f16(w[c]), qs.f[8 * j + 2 * c + 1], d);
          }
        }
        sc[i] = group_sum<CPT>(d) * p.scale_log2;
        if (!hot_ok || t0 + i * TPI + grp >= ctx) {
          sc[i] = -INFINITY;
#pragma unroll
          for (int j = 0; j < kHW; ++j) hv[i][j] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      float bmax = sc[0];
#pragma unroll
      for (int i = 1; i < NLD; ++i) bmax = fmaxf(bmax, sc[i]);
      const float mn = fmaxf(m, bmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      if constexpr (kVOff != 0.f) vbias *= alpha;   // hot rows are fp16: they add no offset
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] *= alpha;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const float pi = __builtin_amdgcn_exp2f(sc[i] - mn);
        l += pi;
#pragma unroll
        for (int j = 0; j < kHW; ++j) {
          const uint32_t w[4] = {hv[i][j].x, hv[i][j].y, hv[i][j].z, hv[i][j].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[8 * j + 2 * c] = fmaf(pi, lo_f16(w[c]), acc[8 * j + 2 * c]);
            acc[8 * j + 2 * c + 1] = fmaf(pi, hi_f16(w[c]), acc[8 * j + 2 * c + 1]);
          }
        }
      }
      m = mn;
    }
  };

  // Two register buffers in turn. Inside the loop the next tile's loads are
  // always issued before the current tile is used, so every wait leaves one
  // tile in flight; the last one or two tiles are peeled off so that no load
  // is issued that nothing consumes.
  // Double buffering holds 4 * NLD 16-byte registers of tiles per lane; with
  // 8 loads per unit (fp32 rows of 128) that would spill, and 8 loads per
  // lane already keep enough bytes in flight, so those run single-buffered.
  constexpr bool kDouble = PA_DECODE_PREFETCH != 0 && NLD <= 4;
  // Work that goes out with the wave's first unit: the hot block of mixed
  // pages is loaded just before it and folded in while it is in flight.
  auto before_first = [&]() {
    if constexpr (kMixed) {
      if (hot_mine) hot_load();
    }
  };
  auto after_first = [&]() {
    prepare_q();
    if constexpr (kMixed) {
      if (hot_mine) hot_process();
    }
    convert_new_row();
  };
  if (!kDouble) {
    prepare_q();
    convert_new_row();
    int e = e0;
    for (int k = 0; k < iters; ++k) {
      const int e_next = k + 1 < iters ? (k == 0 ? e1 : entry(k + 1)) : 0;   // consumed next iteration
      Chunk ka[NLD], va[NLD];
      const TileRef ta = fetch(k, e, ka, va);
      process(ta, ka, va);
      e = e_next;
    }
  } else if (iters > 0) {
    Chunk ka[NLD], va[NLD], kb[NLD], vb[NLD];
    const int last = iters - 1;
    int e_next = last >= 1 ? e1 : e0;
    before_first();
    TileRef ta = fetch(0, e0, ka, va);
    after_first();
    int k = 0;
    for (; k + 2 < iters; k += 2) {
      const int e1 = e_next;
      const int e2 = entry(k + 2);
      const TileRef tb = fetch(k + 1, e1, kb, vb);
      process(ta, ka, va);
      e_next = entry(min(k + 3, last));
      ta = fetch(k + 2, e2, ka, va);
      process(tb, kb, vb);
    }
    if (k + 1 < iters) {
      const TileRef tb = fetch(k + 1, e_next, kb, vb);
      process(ta, ka, va);
      process(tb, kb, vb);
    } else {
      process(ta, ka, va);
    }
  }

  // Mixed pages: the hot unit of a wave that had no tile to overlap it with.
  if constexpr (kMixed) {
    if (hot_mine && !(kDouble && iters > 0)) {
      hot_load();
      hot_process();
    }
  }

  if (patched && grp == new_row % TPI) {
    *reinterpret_cast<uint4*>(const_cast<char*>(p.k) + new_dst) = nk;
    *reinterpret_cast<uint4*>(const_cast<char*>(p.v) + new_dst) = nv;
  }
  if (bad_slot && lane == 0) flag_error(p.err, PA_DEV_BAD_SLOT);
  if (bad_entry && lane == 0) flag_error(p.err, PA_DEV_BAD_TABLE_ENTRY);
  if (bad_ctx && threadIdx.x == 0 && part == 0) flag_error(p.err, PA_DEV_BAD_CONTEXT);

  // The last (or only) partition: the one holding the last unit read through
  // the table, else the first (an empty context, or mixed pages whose
  // partition holds just the hot unit).
  const int last = unit_end > unit_begin ? (unit_end - 1) / p.partition_units : part;
  flush(last);
  if constexpr (!kWavePart) {
    // The last wave to park its partials merges every partition of the
    // workgroup; the others end here. (With a workgroup barrier instead, every
    // wave would wait for the slowest: over a long stream the waves drift
    // apart, and waiting waves hold their slots.)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    int prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(&s_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__shfl(prev, 0) != kWaves - 1) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    typedef float f4v __attribute__((ext_vector_type(4)));
    constexpr int kQ = D / 4;
    const int nparts = last - part + 1;
    const int64_t slot0 = sh * p.num_partitions + part;
    // (m, l) of partition `lane`, stored as whole runs of the workspace.
    if (seq_parts != 1 && lane < nparts) {
      const float* mm = s_m + lane * kWaves;
      const float* ll = s_l + lane * kWaves;
      float M = mm[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mm[w]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) L = fmaf(__builtin_amdgcn_exp2f(mm[w] - M), ll[w], L);
      p.ws_m[slot0 + lane] = M * kLn2;
      p.ws_l[slot0 + lane] = L;
    }
    // o: a lane merges 4 adjacent dims at a time (16-byte LDS reads and
    // stores), so the merging wave, which holds the workgroup's slot, issues
    // few instructions.
    const f4v* o4 = reinterpret_cast<const f4v*>(s_o);
    for (int i = lane; i < nparts * kQ; i += kWave) {
      const int idx = i / kQ, c = i % kQ;
      const float* mm = s_m + idx * kWaves;
      const float* ll = s_l + idx * kWaves;
      float M = mm[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mm[w]);
      float L = 0.f;
      f4v O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wgt = __builtin_amdgcn_exp2f(mm[w] - M);
        L = fmaf(wgt, ll[w], L);
        O += wgt * o4[(idx * kWaves + w) * kQ + c];
      }
      const f4v res = L > 0.f ? O / L : f4v{0.f, 0.f, 0.f, 0.f};
      if (seq_parts == 1) {
        QT* o = reinterpret_cast<QT*>(p.out) + sh * D + 4 * c;
        o[0] = to_out<QT>(res.x);
        o[1] = to_out<QT>(res.y);
        o[2] = to_out<QT>(res.z);
        o[3] = to_out<QT>(res.w);
      } else {
        // Written once and read once by the reduce: kept out of the caches
        // that the tile stream runs through (plain stores cost the stream 3%).
        __builtin_nontemporal_store(res, reinterpret_cast<f4v*>(p.ws_o) + (slot0 + idx) * kQ + c);
      }
    }
  }
}

// Merge the partitions of every (sequence, head) that has more than one.
// One workgroup per (sequence, head): thread t reads 4 adjacent dims (16
// bytes) of every kLanes-th partition, kLanes = 256 / (D / 4) partitions at a
// time with 4 loads each in flight, and the partial sums meet in LDS.
#ifndef PA_REDUCE_THREADS
#define PA_REDUCE_THREADS 256
#endif
#ifndef PA_REDUCE_UNROLL
#define PA_REDUCE_UNROLL 4
#endif
constexpr int kReduceThreads = PA_REDUCE_THREADS;

template <typename QT, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(Params p) {
  constexpr int kQuads = D / 4;                       // threads per partition row
  constexpr int kLanes = kReduceThreads / kQuads;     // partitions read at a time
  constexpr int kUnroll = PA_REDUCE_UNROLL;
  const int sh = blockIdx.x;
  const int s = sh / p.num_heads;
  int ctx = p.ctx[s];
  ctx = ctx < 0 ? 0 : (ctx > p.max_ctx ? p.max_ctx : ctx);
  const int nunits = (ctx + kTileRows - 1) / kTileRows;
  const int parts = nunits == 0 ? 1 : (nunits + p.partition_units - 1) / p.partition_units;
  if (parts <= 1) return;
  const float* m = p.ws_m + int64_t(sh) * p.num_partitions;
  const float* l = p.ws_l + int64_t(sh) * p.num_partitions;
  const float4* o = reinterpret_cast<const float4*>(p.ws_o + int64_t(sh) * p.num_partitions * D);

  __shared__ float s_max[kReduceThreads / kWave];
  __shared__ float s_l[kLanes];
  __shared__ float4 s_o[kLanes][kQuads];
  float M = kNegBig;
  for (int i = threadIdx.x; i < parts; i += kReduceThreads) M = fmaxf(M, m[i]);
  M = wave_max(M);
  if ((threadIdx.x & (kWave - 1)) == 0) s_max[threadIdx.x / kWave] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kReduceThreads / kWave; ++i) M = fmaxf(M, s_max[i]);

  const int dq = threadIdx.x % kQuads;
  const int lane_p = threadIdx.x / kQuads;
  float L = 0.f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](int i, const float4& x) {
    const float wgt = __builtin_amdgcn_exp2f((m[i] - M) * kLog2e) * l[i];
    L += wgt;
    O.x = fmaf(wgt, x.x, O.x);
    O.y = fmaf(wgt, x.y, O.y);
    O.z = fmaf(wgt, x.z, O.z);
    O.w = fmaf(wgt, x.w, O.w);
  };
  int i = lane_p;
  for (; i + (kUnroll - 1) * kLanes < parts; i += kUnroll * kLanes) {
    float4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = o[int64_t(i + u * kLanes) * kQuads + dq];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) add(i + u * kLanes, x[u]);
  }
  for (; i < parts; i += kLanes) add(i, o[int64_t(i) * kQuads + dq]);
  s_o[lane_p][dq] = O;
  if (dq == 0) s_l[lane_p] = L;
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float Lt = 0.f, Ot = 0.f;
#pragma unroll
    for (int j = 0; j < kLanes; ++j) {
      Lt += s_l[j];
      const float4 v = s_o[j][d / 4];
      Ot += (d % 4 == 0) ? v.x : (d % 4 == 1) ? v.y : (d % 4 == 2) ? v.z : v.w;
    }
    // Every partition masked (flagged bad table entries): zeros, as the
    // single pass writes.
    reinterpret_cast<QT*>(p.out)[int64_t(sh) * D + d] = to_out<QT>(Lt > 0.f ? Ot / Lt : 0.f);
  }
}

template <typename KV, typename QT, int D, bool kPaged, typename NEW, bool kMixed, bool kWP>
void launch_one(const Params& p, int grid, size_t lds, hipStream_t st) {
  if constexpr (kPaged) {
    if (p.sched == PA_SCHED_SHARED) {
      hipLaunchKernelGGL((decode_kernel<KV, QT, D, kPaged, NEW, kMixed, kWP, true>), dim3(grid), dim3(kThreads), lds,
                         st, p, p.tables, p.ctx, p.slots);
      return;
    }
  }
  hipLaunchKernelGGL((decode_kernel<KV, QT, D, kPaged, NEW, kMixed, kWP, false>), dim3(grid), dim3(kThreads), lds, st,
                     p, p.tables, p.ctx, p.slots);
}

template <typename KV, typename QT, int D, bool kPaged, bool kWP>
void launch_kernels(const Params& p, int grid, hipStream_t st) {
  // Shared partitions park per-wave partials in LDS until the workgroup merges them.
  const size_t lds = kWP ? 0 : size_t(p.parts_per_group) * kWaves * (D + 2) * sizeof(float);
  if constexpr (kPaged && std::is_same<KV, int8_t>::value) {
    if (p.hot_blocks != nullptr)
      launch_one<KV, QT, D, kPaged, void, true, kWP>(p, grid, lds, st);
    else
      launch_one<KV, QT, D, kPaged, void, false, kWP>(p, grid, lds, st);
  } else if constexpr (kPaged && std::is_same<KV, Int4>::value) {
    if (p.hot_blocks != nullptr)
      launch_one<KV, QT, D, kPaged, void, true, kWP>(p, grid, lds, st);
    else
      launch_one<KV, QT, D, kPaged, void, false, kWP>(p, grid, lds, st);
  } else if constexpr (kPaged) {
    if (p.slots != nullptr) {
      if (p.new_is_f32)
        launch_one<KV, QT, D, kPaged, float, false, kWP>(p, grid, lds, st);
      else
        launch_one<KV, QT, D, kPaged, _Float16, false, kWP>(p, grid, lds, st);
    } else {
      launch_one<KV, QT, D, kPaged, void, false, kWP>(p, grid, lds, st);
    }
  } else {
    launch_one<KV, QT, D, kPaged, void, false, kWP>(p, grid, lds, st);
  }
}

template <typename KV, typename QT, int D, bool kPaged>
int launch_typed(const Params& p, int sh_count, hipStream_t st) {
  // Many partitions per sequence: a workgroup streams several (start-up paid
  // once, loads kept in flight across partition ends, and the kWaves waves
  // read adjacent units, which HBM serves faster than kWaves distant runs).
  // Otherwise short split partitions go a wave each (start-up and merge paid
  // per wave, no barrier), longer ones a workgroup each.
  const int P = p.num_partitions;
  const int ptok = p.partition_units * kTileRows;
  int ppg = 1;
  if (P > 1 && p.hot_blocks == nullptr && p.partition_units % kWaves == 0)
    ppg = max(1, min(min(kGroupTokens / ptok, kMaxGroupParts), int(int64_t(sh_count) * P / kMinGroups)));
  if (ppg > 1) {
    Params q = p;
    q.parts_per_group = ppg;
    launch_kernels<KV, QT, D, kPaged, false>(q, sh_count * ((P + ppg - 1) / ppg), st);
  } else if (P > 1 && ptok <= kWavePartMaxTokens) {
    launch_kernels<KV, QT, D, kPaged, true>(p, sh_count * ((P + kWaves - 1) / kWaves), st);
  } else {
    launch_kernels<KV, QT, D, kPaged, false>(p, sh_count * P, st);
  }
  if (p.num_partitions > 1)
    hipLaunchKernelGGL((reduce_kernel<QT, D>), dim3(sh_count), dim3(kReduceThreads), 0, st, p);
  return int(hipGetLastError());
}

template <typename KV, typename QT, bool kPaged>
int launch_d(const Params& p, int D, int sh_count, hipStream_t st) {
  return D == 64 ? launch_typed<KV, QT, 64, kPaged>(p, sh_count, st)
                 : launch_typed<KV, QT, 128, kPaged>(p, sh_count, st);
}

template <typename KV, bool kPaged>
int launch_q(const Params& p, pa_dtype qd, int D, int sh_count, hipStream_t st) {
  return qd == PA_F32 ? launch_d<KV, float, kPaged>(p, D, sh_count, st)
                      : launch_d<KV, _Float16, kPaged>(p, D, sh_count, st);
}

}  // namespace

int launch_decode(const DecodeArgs& a, void* stream) {
  Params p;
  p.q = a.q;
  p.out = a.out;
  p.k = static_cast<const char*>(a.k);
  p.v = static_cast<const char*>(a.v);
  p.k_scale = static_cast<const _Float16*>(a.k_scale);
  p.v_scale = static_cast<const _Float16*>(a.v_scale);
  p.tables = a.tables;
  p.max_tokens = a.max_tokens;
  p.ctx = a.ctx;
  p.order = a.order;
  p.sched = a.schedule;
  p.max_blocks = a.max_blocks;
  p.num_seqs = a.num_seqs;
  p.num_heads = a.num_heads;
  p.num_blocks = a.num_blocks;
  p.max_ctx = a.max_ctx;
  // Single pass: one partition large enough for any context.
  p.partition_units = a.partition_tokens > 0 ? a.partition_tokens / kTileRows
                                              : (a.max_ctx + kTileRows - 1) / kTileRows + 1;
  p.unit_shift = block_shift(a.block_size) - 4;
  p.parts_per_group = 1;
  p.num_partitions = a.num_partitions;
  p.scale_log2 = a.sm_scale * kLog2e;
  p.ws_m = a.ws_m;
  p.ws_l = a.ws_l;
  p.ws_o = a.ws_o;
  p.err = a.err;
  p.k_new = a.k_new;
  p.v_new = a.v_new;
  p.slots = a.slots;
  p.new_is_f32 = a.new_dtype == PA_F32 ? 1 : 0;
  p.hot_k = static_cast<const char*>(a.hot_k);
  p.hot_v = static_cast<const char*>(a.hot_v);
  p.hot_blocks = a.hot_blocks;
  p.num_hot = a.num_hot;
  const int sh_count = a.num_seqs * a.num_heads;
  if (sh_count == 0) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool paged = a.tables != nullptr;
  switch (a.kv_dtype) {
    case PA_F32:
      return paged ? launch_q<float, true>(p, a.q_dtype, a.head_dim, sh_count, st)
                   : launch_q<float, false>(p, a.q_dtype, a.head_dim, sh_count, st);
    case PA_F16:
      return paged ? launch_q<_Float16, true>(p, a.q_dtype, a.head_dim, sh_count, st)
                   : launch_q<_Float16, false>(p, a.q_dtype, a.head_dim, sh_count, st);
    case PA_I8:
      return launch_q<int8_t, true>(p, a.q_dtype, a.head_dim, sh_count, st);
    case PA_I4:
      return launch_q<Int4, true>(p, a.q_dtype, a.head_dim, sh_count, st);
  }
  return int(hipErrorInvalidValue);
}

}  // namespace pa
