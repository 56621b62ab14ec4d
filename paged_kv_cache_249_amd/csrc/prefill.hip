// Several new tokens of each sequence attending at once over paged KV (fp16,
// int8 or int4 pools).
//
// The attention formula of "One Deep Concept #01" (§2 Background) takes a
// matrix of queries. When the last n tokens of a sequence are processed
// together (their K and V already written into the pool), the token at
// position p attends to tokens 0..p: each gets exactly its own decode over the
// context up to itself ("PagedAttention的终极用途", part 一: a generated token
// attends to every earlier token and itself). K and V are read through the
// block table as in decode ("PagedAttention — 把 KV cache 当虚拟内存页来管理",
// 实践案例 / 案例 2).
//
// Unlike decode, every K and V row here meets up to 128 queries, so the two
// products are dense and run on the matrix cores (v_mfma_f32_16x16x32_f16,
// fp32 accumulation). A workgroup of 4 waves owns 128 query rows of one
// (sequence, head); a wave holds two 16-row query tiles. The context is
// walked 32 tokens per step; the workgroup stages each step's K and V rows in
// LDS (fp16 pools straight from memory into three buffers, two steps ahead;
// int8 and int4 pools through registers, where codes become fp16), one
// barrier per step. Per step and query tile:
//   S^T[t][q] = K[t] . Q[q]          two 16x16 tiles, k = head_dim in steps of 32
//   online softmax per query column  (exp2 domain, fp32, lazy reference max)
//   O[q][d] += P[q][t] V[t][d]       one 16x16x32 product per 16 output columns
// S^T's accumulator layout (lane = query column, 4 tokens per lane and lane
// group) is exactly the A-operand layout P needs for the second product, so P
// never leaves the registers. V reaches the second product through gfx950's
// transposing LDS reads (ds_read_b64_tr_b16), which hand each lane one
// dimension of four consecutive rows: output column j of tile c is dimension
// 16c + j.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kPfWaves = 4;          // waves per workgroup
constexpr int kPfTiles = 2;          // 16-row query tiles per wave
constexpr int kPfRows = 16 * kPfTiles;   // query rows per wave
constexpr int kPfWgRows = kPfWaves * kPfRows;
constexpr int kPfStep = 32;          // tokens per step: the k extent of one 16x16x32 product
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;        // log2 headroom before the reference max moves
constexpr int kTabCap = 2048;       // table entries a workgroup can keep in LDS
constexpr int kPfWindow = 4;        // groups whose row tiles an XCD interleaves

struct PrefillParams {
  const _Float16* q;             // [num_rows][H][D]
  _Float16* out;                 // [num_rows][H][D]
  const void* k;                 // pool [num_blocks][H][B][D]: fp16, int8 codes, or int4 code pairs
  const void* v;
  const _Float16* k_scale;       // int8 and int4 pools: fp16 [num_blocks][H]
  const _Float16* v_scale;
  const int32_t* query_start;    // [S + 1]
  const int32_t* tables;         // [S][max_blocks]
  const int32_t* ctx;            // [S]
  const int32_t* order;          // [S] dispatch order (a permutation), or nullptr
  int32_t num_seqs;
  int32_t num_rows;
  int32_t max_blocks;
  int32_t num_heads;
  int32_t num_blocks;
  int32_t max_ctx;
  int32_t max_query;
  int32_t row_tiles;             // workgroups per (sequence, head): ceil(max_query / 128)
  float scale_log2;              // sm_scale * log2(e)
  int32_t* err;
};

// Four int8 codes (one 32-bit word) times an fp16 scale, as four fp16
// values (two words). Each code c becomes the half 1024 + (c + 128) by
// placing the byte c ^ 0x80 under the exponent byte 0x64 (exact: halves in
// [1024, 2048) step by 1); subtracting 1152 gives c exactly, and one
// multiply rounds c * s to nearest even, as fp32 c * s rounded to fp16 would.
__device__ __forceinline__ void dequant4(uint32_t w, f16x2 s2, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const f16x2 off = f16x2{_Float16(1152.f), _Float16(1152.f)};
  const f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(u, 0x64646464u, 0x00050004u));
  const f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(u, 0x64646464u, 0x00070006u));
  lo = __builtin_bit_cast(uint32_t, f16x2((a - off) * s2));
  hi = __builtin_bit_cast(uint32_t, f16x2((b - off) * s2));
}

// Eight int4 codes (one 32-bit word: byte j holds dim 2j in its low nibble
// and dim 2j+1 in its high one, each as code + 8) times an fp16 scale, as
// eight fp16 values in dim order (four words). Each nibble n goes under the
// exponent byte 0x64 (the half 1024 + n, exact); subtracting 1032 gives the
// code exactly and one multiply rounds code * s to nearest even.
__device__ __forceinline__ void dequant8_i4(uint32_t w, f16x2 s2, uint32_t (&out)[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const f16x2 off = f16x2{_Float16(1032.f), _Float16(1032.f)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // Bytes: lo[j], 0, hi[j], 0 (selector 0x0C yields zero), then the exponent bytes.
    const uint32_t t = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + 0x00010001u * uint32_t(j)) | 0x64006400u;
    out[j] = __builtin_bit_cast(uint32_t, f16x2((__builtin_bit_cast(f16x2, t) - off) * s2));
  }
}

// Max over the four lanes of a column (lanes l, l^16, l^32, l^48). With both
// operands the same value, permlane16_swap returns rows (0,0,2,2) and
// (1,1,3,3) of it, and permlane32_swap the lower and the upper 32 lanes each
// twice, so two swaps and two maxima reduce across the rows without LDS.
__device__ __forceinline__ float col_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Pool element types the kernel reads.
enum : int { kKvF16 = 0, kKvI8 = 1, kKvI4 = 2 };

// LDS layout of a step's K and V rows: rows of D halves, unpadded, with the
// 16-byte chunks of row r stored at chunk index c ^ swz(r). The swizzle was
// chosen by measuring the kernel's access patterns on gfx950 (K operand
// reads: 16 rows x one chunk per lane group; staging: whole rows): with it
// the K reads run at the LDS's throughput, while rows padded by 16 bytes
// took 1.7x that (4 bank-conflict cycles per LDS cycle) and unpadded rows
// 6.7x. V's transposing reads (8 bytes of each of 4 rows per lane group)
// cost about 2.4x a 16-byte read per byte under every swizzle measured.
template <int D>
__device__ __forceinline__ int lds_swizzle(int row) {
  if constexpr (D == 128) return (row & 3) * 4 + ((row >> 2) & 3);
  else return (row & 3) * 2 + ((row >> 2) & 1);
}
// Half offset of 16-byte chunk c of row r.
template <int D>
__device__ __forceinline__ int lds_at(int row, int c) {
  return row * D + ((c ^ lds_swizzle<D>(row)) << 3);
}

template <int D, int BS, bool kTabLds, int kKV>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_kernel(PrefillParams p) {
  constexpr bool kI8 = kKV == kKvI8;
  constexpr bool kI4 = kKV == kKvI4;
  constexpr bool kQuant = kI8 || kI4;
  constexpr int kNT = D / 16;      // output tiles; column j of tile c is dim 16c + j
  constexpr int kKS = D / 32;      // k steps of the QK product
  constexpr int kGD = D / 4;       // dims a lane group covers in the QK product
  // Steps' K and V rows (32 tokens each), shared by the workgroup's waves.
  // fp16 pools: three buffers of each, filled straight from memory (the
  // products read one while the next two steps land in the others);
  // quantised pools: two, filled through registers (the products read one
  // while the next step is stored into the other). Separate arrays, so that
  // the compiler can tell a load into one buffer from reads of another.
  constexpr bool kDirect = !kQuant;
  __shared__ __align__(16) _Float16 lk0[kPfStep * D], lk1[kPfStep * D], lk2[kDirect ? kPfStep * D : 8];
  __shared__ __align__(16) _Float16 lv0[kPfStep * D], lv1[kPfStep * D], lv2[kDirect ? kPfStep * D : 8];
  // The workgroup's table row (when the launch's contexts fit): entries are
  // then LDS broadcasts, so the only vector loads in flight are K and V rows
  // and waiting for a table entry never drains them.
  __shared__ int32_t ltab[kTabLds ? kTabCap : 1];

  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;       // MFMA row/column index of this lane
  const int grp = lane >> 4;       // MFMA lane group (k slice / output row quad)

  // Workgroup -> (sequence, head, row tile). Workgroups are dealt to the 8
  // XCDs round robin (block b runs on XCD b % 8, as its (b / 8)-th). Groups
  // (the row tiles of one (sequence, head)) are dealt round robin over the
  // XCDs in dispatch order, all tiles of a group on one XCD so they share its
  // L2: XCD x takes groups x, x + 8, ... — every XCD gets its share of long
  // and short sequences whatever the order. Heavier row tiles (the last rows
  // attend to the most tokens) go first.
  const int T = p.row_tiles;
  const int groups = int(gridDim.x) / T;
  int g, k;
  if ((groups & 7) == 0) {
    // Within an XCD, windows of kPfWindow groups (about what its CUs hold
    // at once, so their K/V share the L2 as before): a window's tiles go
    // heaviest first across its groups, so the last tiles dealt are light
    // ones and the XCD's CUs run out of work together.
    const int x = int(blockIdx.x) & 7, j = int(blockIdx.x) >> 3;
    const int per_xcd = groups >> 3;
    const int win = j / (kPfWindow * T);
    const int wg = min(kPfWindow, per_xcd - win * kPfWindow);   // groups in this window
    const int r = j - win * kPfWindow * T;
    g = x + 8 * (win * kPfWindow + r % wg);
    k = r / wg;
  } else {
    g = int(blockIdx.x) / T;
    k = int(blockIdx.x) % T;
  }
  const int tile = T - 1 - k;
  const int h = g % p.num_heads;
  const int rank = g / p.num_heads;
  const int s = p.order ? p.order[rank] : rank;      // sequences in the caller's dispatch order
  if (unsigned(s) >= unsigned(p.num_seqs)) {
    if (tile == 0 && h == 0 && threadIdx.x == 0) flag_error(p.err, PA_DEV_BAD_CONTEXT);
    return;
  }

  // Everything up to the loop depends on (s, tile) only, so a workgroup
  // leaves as a whole or not at all (the loop has barriers).
  const int qa = p.query_start[s];
  const int n = p.query_start[s + 1] - qa;
  const int wg_r0 = tile * kPfWgRows;                   // first chunk row of the workgroup
  if (wg_r0 >= n) {
    if (n < 0 && tile == 0 && tid == 0 && h == 0) flag_error(p.err, PA_DEV_BAD_CONTEXT);
    return;
  }
  const int ctx = p.ctx[s];
  if (qa < 0 || qa + n > p.num_rows || n > ctx || ctx > p.max_ctx || n > p.max_query) {
    if (tid == 0) flag_error(p.err, PA_DEV_BAD_CONTEXT);
    return;
  }
  const int base_pos = ctx - n;                         // position of chunk row 0
  const int wg_t_end = base_pos + min(wg_r0 + kPfWgRows, n);   // tokens the workgroup reads
  const int r0 = wg_r0 + wave * kPfRows;                // first chunk row of this wave
  const bool active = r0 < n;
  const int last = active ? min(r0 + kPfRows, n) - 1 : r0;      // last valid row of this wave
  const int t_end = active ? base_pos + last + 1 : 0;   // tokens this wave attends: [0, t_end)
  // Query tile qt of the wave holds rows r0 + 16 qt .. + 15; lane column col
  // is row min(r0 + 16 qt + col, last) (rows past the chunk repeat its last
  // row and are never stored); my_pos is that row's position.
  int my_pos[kPfTiles];
#pragma unroll
  for (int qt = 0; qt < kPfTiles; ++qt) my_pos[qt] = base_pos + min(r0 + 16 * qt + col, last);

  // Q as the B operand of S^T = K Q^T: this lane's row, dims grp*kGD + 8*kk .. +7.
  f16x8 qv[kPfTiles][kKS];
#pragma unroll
  for (int qt = 0; qt < kPfTiles; ++qt) {
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) qv[qt][kk] = f16x8{};
    if (active) {
      const int row = my_pos[qt] - base_pos;
      const _Float16* qrow = p.q + (int64_t(qa + row) * p.num_heads + h) * D + grp * kGD;
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) qv[qt][kk] = *reinterpret_cast<const f16x8*>(qrow + 8 * kk);
    }
  }

  const int32_t* trow = p.tables + int64_t(s) * p.max_blocks;
  const int64_t head_off = int64_t(h) * BS * D;
  const int64_t block_elems = int64_t(p.num_heads) * BS * D;

  // A 16-row half of a step lies in one block (B is 16, 32 or 64 and steps
  // start at multiples of 32), so its table entry is one value for the
  // workgroup. No table entry at or past the workgroup's last token is read.
  int tab[2] = {0, 0};               // table entries of the two halves of the next step to load
  if constexpr (kTabLds) {
    // Entries are checked here, once: a bad one is flagged and read as block
    // 0 (the rows it should have named are then unspecified, never out of
    // bounds), so the loop below needs no checks.
    const int nblk = (wg_t_end + BS - 1) / BS;   // <= kTabCap: the host checked the launch's max_ctx
    for (int i = tid; i < nblk; i += kPfWaves * 64) {
      int b = trow[i];
      if (unsigned(b) >= unsigned(p.num_blocks)) {
        flag_error(p.err, PA_DEV_BAD_TABLE_ENTRY);
        b = 0;
      }
      ltab[i] = b;
    }
    __syncthreads();
  }
  auto fetch_table = [&](int t0, int (&dst)[2]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int t = t0 + 16 * half;
      if constexpr (kTabLds) dst[half] = t < wg_t_end ? ltab[t / BS] : 0;
      else dst[half] = t < wg_t_end ? trow[t / BS] : 0;
    }
  };

  f32x4 o[kPfTiles][kNT];
  // Weight sums of rows 4*grp + r (P times a ones operand: every column of
  // this tile holds its row's sum), rescaled together with o.
  f32x4 osum[kPfTiles];
  // Reference max (log2 units) of this lane's query column. Weights are
  // exp2(logit - m); m moves (and o, osum are rescaled) only when a logit
  // exceeds it by more than kLazy, so weights stay below 2^kLazy and most
  // steps skip the rescale. Any reference gives the same quotient o / osum.
  float m[kPfTiles];
  float thr[kPfTiles];   // raw q.k above which a logit exceeds m + kLazy
#pragma unroll
  for (int qt = 0; qt < kPfTiles; ++qt) {
    thr[qt] = -INFINITY;
#pragma unroll
    for (int c = 0; c < kNT; ++c) o[qt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    osum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[qt] = -INFINITY;
  }
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = _Float16(1.f);
  const float c2 = p.scale_log2;

  // Products of one step over the rows in LDS buffer ck / cv.
  auto compute = [&](int t0, const _Float16* ck, const _Float16* cv) {
    if (t0 < t_end) {                // wave-uniform: this wave still has rows to serve
      // S^T tiles: lane holds S^T[t = 16j + 4*grp + r][q = col] of query tile
      // qt, r = 0..3 (raw q.k). Each K operand serves both query tiles.
      f32x4 sc[kPfTiles][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int qt = 0; qt < kPfTiles; ++qt) sc[qt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKS; ++kk) {
          const f16x8 kv = *reinterpret_cast<const f16x8*>(ck + lds_at<D>(16 * j + col, grp * (kGD / 8) + kk));
#pragma unroll
          for (int qt = 0; qt < kPfTiles; ++qt)
            sc[qt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kv, qv[qt][kk], sc[qt][j], 0, 0, 0);
        }
      }
      // V as the B operand of the second product: column col of output tile c
      // is dim 16c + col, k = this lane's 8 tokens t = 16*(e/4) + 4*grp + e%4
      // (the order of P's A operand). Transposing LDS reads deliver it: in each
      // 16-lane group, lane s fetches dims 16c + 4(s%4) .. +3 of row
      // 16j + 4*grp + s/4 and receives dim 16c + s of the group's four rows.
      f16x8 vb[kNT];
#pragma unroll
      for (int c = 0; c < kNT; ++c) {
        f16x4 t[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int dim = 16 * c + 4 * (col & 3);
          t[j] = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(
                                               cv + lds_at<D>(16 * j + 4 * grp + (col >> 2), dim >> 3) + (dim & 7))));
        }
        vb[c] = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7);
      }

      // Softmax of both query tiles. The tests below are taken once per step
      // for both tiles, so the common path (no mask, no move of the
      // reference max) is one straight run of code in which the weights of
      // one tile are computed while the other's products are in flight.
      float x[kPfTiles][8];
#pragma unroll
      for (int qt = 0; qt < kPfTiles; ++qt)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[qt][e] = sc[qt][e >> 2][e & 3];
      // Only steps reaching past the wave's first position need the causal
      // mask (it also hides the zero rows past the workgroup's last token).
      if (t0 + kPfStep - 1 > base_pos + r0) {
#pragma unroll
        for (int qt = 0; qt < kPfTiles; ++qt)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = t0 + 16 * (e >> 2) + grp * 4 + (e & 3);
            if (t > my_pos[qt]) x[qt][e] = -INFINITY;
          }
      }
      float mx[kPfTiles];
      bool up = false;
#pragma unroll
      for (int qt = 0; qt < kPfTiles; ++qt) {
        mx[qt] = x[qt][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx[qt] = fmaxf(mx[qt], x[qt][e]);
        up = up || mx[qt] > thr[qt];
      }
      // A logit of a column past m + kLazy shows in this lane's own maximum
      // already (thr = (m + kLazy) / c2, c2 > 0): the column-wide maximum is
      // needed only to move m. Moving m when no logit passed the threshold
      // is harmless (any reference gives the same quotient o / osum, and
      // weights stay at most 2^kLazy). Token 0 is visible to every query in
      // the first step, so every m is finite after it and the first step
      // always moves it (from m = -inf, thr = -inf).
      if (__any(up)) {
#pragma unroll
        for (int qt = 0; qt < kPfTiles; ++qt) {
          const float m_new = fmaxf(m[qt], col_max(mx[qt]) * c2);
          const float alpha = __builtin_amdgcn_exp2f(m[qt] - m_new);
          m[qt] = m_new;
          thr[qt] = (m_new + kLazy) / c2;
          // O rows are 4*grp + r: their factors live in the lanes whose column is that row.
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, grp * 4 + r, 64);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            osum[qt][r] *= ar[r];
#pragma unroll
            for (int c = 0; c < kNT; ++c) o[qt][c][r] *= ar[r];
          }
        }
      }
      f16x8 pa[kPfTiles];
#pragma unroll
      for (int qt = 0; qt < kPfTiles; ++qt) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pa[qt][e] = _Float16(__builtin_amdgcn_exp2f(__builtin_fmaf(x[qt][e], c2, -m[qt])));
        osum[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[qt], ones, osum[qt], 0, 0, 0);
      }
      // P (A operand: row = this lane's query column, k = the lane's 8 tokens) times V.
#pragma unroll
      for (int qt = 0; qt < kPfTiles; ++qt) {
#pragma unroll
        for (int c = 0; c < kNT; ++c)
          o[qt][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[qt], vb[c], o[qt][c], 0, 0, 0);
      }
      // Issue order of this run of code: the first tile's weights (VALU),
      // then its matrix products one at a time, each followed by two VALU
      // instructions of the second tile's weights, then the second tile's
      // products. The matrix cores work while the second tile's exponentials
      // are computed. (Masks: 0x2 VALU, 0x8 MFMA.)
      __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 9, 0);
    }
  };

  if constexpr (kDirect) {
    // fp16: each step's rows go from the pool straight into LDS
    // (buffer_load_dwordx4 ... lds): a wave instruction fills 1 KB of LDS,
    // lane L the 16 bytes at 16 L, i.e. kRpi whole rows; each lane loads the
    // logical chunk that belongs at its LDS position under the swizzle. Rows
    // at or past the workgroup's last token (and rows of a bad table entry)
    // take an offset past the buffer resource, which covers one 16-row slice
    // of a (block, head) tile, and land as zeros. Loads run two steps ahead:
    // when step t is computed, steps t+1 and t+2 are on their way, and the
    // wait before each barrier leaves exactly the newest step's loads in
    // flight (loads complete in order). No register holds staged rows.
    constexpr int kLaneChunks = D / 8;                  // 16-byte chunks per row
    constexpr int kRpi = 64 / kLaneChunks;              // rows per wave instruction
    constexpr int kIpw = kPfStep / kRpi / kPfWaves;     // instructions per wave, step and tensor
    static_assert(kIpw * kRpi * kPfWaves == kPfStep && 16 % kRpi == 0, "step rows must split into waves");
    constexpr int kSliceBytes = 16 * D * 2;             // one 16-row slice of a (block, head) tile
    constexpr int kRsrcWord3 = 0x00020000;
    // s_waitcnt: vmcnt <= 2 kIpw (the newest step's K and V loads), lgkmcnt
    // 0 (this wave's LDS reads of the step done), expcnt unconstrained.
    constexpr int kStepWait = (2 * kIpw) | (7 << 4);
    const int drow = lane / kLaneChunks;                // row within a wave instruction
    const int dchunk = lane % kLaneChunks;              // physical chunk this lane fills
    // The buffer resource and the LDS address of an instruction are wave
    // uniform (scalar registers); the wave index and the table entries (read
    // from LDS, the same address in every lane) are declared so.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int t0, const int (&blk)[2], _Float16* dk, _Float16* dv) {
#pragma unroll
      for (int i = 0; i < kIpw; ++i) {
        const int g = wv * kIpw + i;                    // rows g kRpi .. of the step
        const int r = g * kRpi + drow;
        const int half = (g * kRpi) >> 4;
        int b = __builtin_amdgcn_readfirstlane(blk[half]);   // one entry for the whole instruction
        bool ok = t0 + r < wg_t_end;
        if (unsigned(b) >= unsigned(p.num_blocks)) {    // only possible when entries are read as we go
          if (ok) flag_error(p.err, PA_DEV_BAD_TABLE_ENTRY);
          b = 0;
          ok = false;
        }
        // Token-head row index of the slice: 32 bits (the host refuses pools
        // of more rows; a pool that fits in HBM has fewer, a row being at
        // least 128 bytes). Read back as a scalar so that the resource is
        // built in scalar registers.
        const uint64_t slice = __builtin_amdgcn_readfirstlane(
            (uint32_t(b) * uint32_t(p.num_heads) + uint32_t(h)) * uint32_t(BS) + uint32_t((t0 + 16 * half) % BS));
        const int voff = ok ? (r & 15) * D * 2 + ((dchunk ^ lds_swizzle<D>(r)) << 4) : kSliceBytes;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<_Float16*>(static_cast<const _Float16*>(p.k)) + slice * D, 0, kSliceBytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<_Float16*>(static_cast<const _Float16*>(p.v)) + slice * D, 0, kSliceBytes, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dk + g * kRpi * D), 16,
                                                 voff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dv + g * kRpi * D), 16,
                                                 voff, 0, 0, 0);
      }
    };
    {
      int blk[2];
      fetch_table(0, blk);
      issue(0, blk, lk0, lv0);
      fetch_table(kPfStep, blk);
      issue(kPfStep, blk, lk1, lv1);
      fetch_table(2 * kPfStep, tab);
    }
    __builtin_amdgcn_s_waitcnt(kStepWait);
    __builtin_amdgcn_s_barrier();
    // Step at t0 from buffer (ck, cv); the step two ahead into (nk, nv), which
    // every wave left before the last barrier.
    auto dstep = [&](int t0, const _Float16* ck, const _Float16* cv, _Float16* nk, _Float16* nv) {
      int nt[2];
      fetch_table(t0 + 3 * kPfStep, nt);
      issue(t0 + 2 * kPfStep, tab, nk, nv);
      tab[0] = nt[0];
      tab[1] = nt[1];
      compute(t0, ck, cv);
      __builtin_amdgcn_s_waitcnt(kStepWait);          // next step landed; this step's reads done
      __builtin_amdgcn_s_barrier();
    };
    for (int t0 = 0; t0 < wg_t_end;) {
      dstep(t0, lk0, lv0, lk2, lv2);
      t0 += kPfStep;
      if (t0 >= wg_t_end) break;
      dstep(t0, lk1, lv1, lk0, lv0);
      t0 += kPfStep;
      if (t0 >= wg_t_end) break;
      dstep(t0, lk2, lv2, lk1, lv1);
      t0 += kPfStep;
    }
    // No load into LDS may still be in flight when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(0);
  } else {
    // int8 and int4 pools: thread tid stages one chunk of the step's K and V
    // rows (row tid / 8, its D/8 codes from (tid % 8) D/8 on) through
    // registers and scales it into fp16 on the way to LDS.
    constexpr int kChunkVals = D / 8;
    static_assert(kPfStep * 8 == kPfWaves * 64, "one chunk per thread covers a step");
    // One chunk of codes: int8 16 bytes (D 128) or 8; int4 8 (D 128) or 4.
    using Raw = typename std::conditional<
        kI4, typename std::conditional<D == 64, uint32_t, uint2>::type,
        typename std::conditional<D == 64, uint2, uint4>::type>::type;
    const int srow = tid / 8;                           // step row this thread stages
    const int schunk = (tid % 8) * (kChunkVals / 8);   // first 16-byte LDS chunk it fills
    // A chunk as the thread holds it, with the scales of the block it came from.
    struct Stage {
      Raw k, v;
      f16x2 ks, vs;
    };
    // Every call issues the same loads whatever the step (rows past the
    // workgroup's last token, or a whole step past it, read the pool's first
    // row instead), so the loads in flight are counted the same on every path
    // and waiting for one stage never drains the next.
    auto load_step = [&](int t0, const int (&blk)[2], Stage& st) {
      const int tt = t0 + srow;
      const int b = blk[srow >> 4];
      bool ok = tt < wg_t_end;
      if constexpr (!kTabLds) {
        if (ok && unsigned(b) >= unsigned(p.num_blocks)) {
          flag_error(p.err, PA_DEV_BAD_TABLE_ENTRY);
          ok = false;
        }
      }
      const int64_t off =   // in codes
          ok ? int64_t(b) * block_elems + head_off + int64_t(tt % BS) * D + (tid % 8) * kChunkVals
             : int64_t(0);
      const int64_t byte = kI4 ? off / 2 : off;      // int4: two codes per byte
      st.k = *reinterpret_cast<const Raw*>(static_cast<const uint8_t*>(p.k) + byte);
      st.v = *reinterpret_cast<const Raw*>(static_cast<const uint8_t*>(p.v) + byte);
      const int64_t si = ok ? int64_t(b) * p.num_heads + h : int64_t(0);
      const _Float16 ks = p.k_scale[si], vs = p.v_scale[si];
      st.ks = f16x2{ks, ks};
      st.vs = f16x2{vs, vs};
    };
    // Rows at or past the workgroup's last token are stored as zeros: no
    // unused slot of a last block (or other row read in its place) reaches
    // the products.
    auto store_step = [&](int buf, int t0, const Stage& st) {
      // Workgroup-uniform outer test: only the last step has such rows.
      const bool zero = t0 + kPfStep > wg_t_end && t0 + srow >= wg_t_end;
      constexpr int kW = int(sizeof(Raw)) / 4;      // code words per chunk
      constexpr int kOut = kI4 ? 4 * kW : 2 * kW;    // fp16 pair words they become
      uint32_t kw[kOut], vw[kOut];
      const uint32_t* kr = reinterpret_cast<const uint32_t*>(&st.k);
      const uint32_t* vr = reinterpret_cast<const uint32_t*>(&st.v);
#pragma unroll
      for (int i = 0; i < kW; ++i) {
        if constexpr (kI4) {
          uint32_t a[4], b[4];
          dequant8_i4(kr[i], st.ks, a);
          dequant8_i4(vr[i], st.vs, b);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kw[4 * i + e] = a[e];
            vw[4 * i + e] = b[e];
          }
        } else {
          dequant4(kr[i], st.ks, kw[2 * i], kw[2 * i + 1]);
          dequant4(vr[i], st.vs, vw[2 * i], vw[2 * i + 1]);
        }
      }
#pragma unroll
      for (int i = 0; i < kOut / 4; ++i) {
        uint4 kx = uint4{kw[4 * i], kw[4 * i + 1], kw[4 * i + 2], kw[4 * i + 3]};
        uint4 vx = uint4{vw[4 * i], vw[4 * i + 1], vw[4 * i + 2], vw[4 * i + 3]};
        if (zero) {
          kx = uint4{0u, 0u, 0u, 0u};
          vx = uint4{0u, 0u, 0u, 0u};
        }
        *reinterpret_cast<uint4*>(&(buf ? lk1 : lk0)[lds_at<D>(srow, schunk + i)]) = kx;
        *reinterpret_cast<uint4*>(&(buf ? lv1 : lv0)[lds_at<D>(srow, schunk + i)]) = vx;
      }
    };

    // Two register stages: while a step is computed, the next one's rows wait
    // in registers for the other LDS buffer and the one after is in flight
    // from memory (a first touch from HBM can outlast one step's products).
    // Table entries are read one step further ahead still.
    Stage sA, sB;
    {
      int blk[2];
      fetch_table(0, blk);
      load_step(0, blk, sA);
      fetch_table(kPfStep, blk);
      load_step(kPfStep, blk, sB);
      fetch_table(2 * kPfStep, tab);
      store_step(0, 0, sA);
    }
    __syncthreads();
    // nx: the next step's rows (stored after the products); fr: free, it
    // receives the step after it.
    auto step = [&](int t0, int buf, Stage& nx, Stage& fr) {
      int nt[2];
      fetch_table(t0 + 3 * kPfStep, nt);
      load_step(t0 + 2 * kPfStep, tab, fr);
      tab[0] = nt[0];
      tab[1] = nt[1];
      compute(t0, buf ? lk1 : lk0, buf ? lv1 : lv0);
      // The other buffer: every wave left it before the last barrier.
      if (t0 + kPfStep < wg_t_end) store_step(buf ^ 1, t0 + kPfStep, nx);
      __syncthreads();                 // next step's rows stored; this step's reads done
    };
    for (int t0 = 0; t0 < wg_t_end;) {
      step(t0, 0, sB, sA);
      t0 += kPfStep;
      if (t0 >= wg_t_end) break;
      step(t0, 1, sA, sB);
      t0 += kPfStep;
    }
  }
  if (!active) return;

  // osum[r] >= 1: the largest weight applied is at least exp2(0).
#pragma unroll
  for (int qt = 0; qt < kPfTiles; ++qt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ir = 1.f / osum[qt][r];
      const int row = r0 + 16 * qt + grp * 4 + r;
      if (row < n) {
        _Float16* orow = p.out + (int64_t(qa + row) * p.num_heads + h) * D + col;
#pragma unroll
        for (int c = 0; c < kNT; ++c) orow[16 * c] = _Float16(o[qt][c][r] * ir);
      }
    }
  }
}

template <int D, int BS, int kKV>
int launch_prefill_d(const PrefillParams& p, int64_t groups, hipStream_t st) {
  // Every workgroup's table row fits in LDS when the launch's longest context does.
  if ((int64_t(p.max_ctx) + BS - 1) / BS <= kTabCap)
    hipLaunchKernelGGL((prefill_kernel<D, BS, true, kKV>), dim3(unsigned(groups)), dim3(kPfWaves * 64), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BS, false, kKV>), dim3(unsigned(groups)), dim3(kPfWaves * 64), 0, st, p);
  return int(hipGetLastError());
}

template <int D, int kKV>
int launch_prefill_bs(const PrefillParams& p, int block_size, int64_t groups, hipStream_t st) {
  switch (block_size) {
    case 16: return launch_prefill_d<D, 16, kKV>(p, groups, st);
    case 32: return launch_prefill_d<D, 32, kKV>(p, groups, st);
    default: return launch_prefill_d<D, 64, kKV>(p, groups, st);
  }
}

template <int D>
int launch_prefill_kv(const PrefillParams& p, pa_dtype kv, int block_size, int64_t groups, hipStream_t st) {
  switch (kv) {
    case PA_I8: return launch_prefill_bs<D, kKvI8>(p, block_size, groups, st);
    case PA_I4: return launch_prefill_bs<D, kKvI4>(p, block_size, groups, st);
    default: return launch_prefill_bs<D, kKvF16>(p, block_size, groups, st);
  }
}

}  // namespace

int64_t prefill_groups(int32_t num_seqs, int32_t num_heads, int32_t max_query_len) {
  const int64_t tiles = (int64_t(max_query_len) + kPfWgRows - 1) / kPfWgRows;
  return int64_t(num_seqs) * num_heads * tiles;
}

int launch_prefill(const PrefillArgs& a, void* stream) {
  const int64_t groups = prefill_groups(a.num_seqs, a.pool->num_heads, a.max_query_len);
  if (groups == 0) return 0;
  PrefillParams p{};
  p.q = static_cast<const _Float16*>(a.q);
  p.out = static_cast<_Float16*>(a.out);
  p.k = a.pool->k_cache;
  p.v = a.pool->v_cache;
  p.k_scale = static_cast<const _Float16*>(a.pool->k_scale);
  p.v_scale = static_cast<const _Float16*>(a.pool->v_scale);
  p.query_start = a.query_start;
  p.tables = a.tables;
  p.ctx = a.ctx;
  p.order = a.order;
  p.num_seqs = a.num_seqs;
  p.num_rows = a.num_rows;
  p.max_blocks = a.max_blocks;
  p.num_heads = a.pool->num_heads;
  p.num_blocks = a.pool->num_blocks;
  p.max_ctx = a.max_ctx;
  p.max_query = a.max_query_len;
  p.row_tiles = int32_t((int64_t(a.max_query_len) + kPfWgRows - 1) / kPfWgRows);
  p.scale_log2 = a.sm_scale * kLog2e;
  p.err = a.pool->err;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.pool->head_dim == 64) return launch_prefill_kv<64>(p, a.pool->kv_dtype, a.pool->block_size, groups, st);
  return launch_prefill_kv<128>(p, a.pool->kv_dtype, a.pool->block_size, groups, st);
}

}  // namespace pa
