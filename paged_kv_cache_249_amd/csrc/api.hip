// C ABI of libpagedkv: argument validation, the error model, the pool
// descriptor and the device error words. The attention kernels live in
// decode.hip and prefill.hip, the cache kernels (write, copy, swap, demote)
// in cache_ops.hip; the host block managers in block_manager.cpp and
// mixed_manager.cpp.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <string>

#include "pa_internal.h"

namespace pa {

// Device error words. Word 0 takes the flags of calls tied to no pool
// (pa_decode_contiguous); every live pool owns one of the others, handed out
// by pa_alloc_pool and returned by pa_free_pool, so the flags of two pools
// never mix and reading one pool's word leaves the others alone. Each GPU
// holds its own copy of both arrays; host code reaches them through the
// addresses that hipGetSymbolAddress gives on each device.
__device__ int32_t g_error_words[kErrorWords];
// Where pa_check_errors' read-and-clear kernel leaves the old value of a word.
__device__ int32_t g_error_readout[kErrorWords];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceWords {
  int32_t* words = nullptr;
  int32_t* readout = nullptr;
};

std::mutex g_err_mutex;               // guards the tables below and readouts
DeviceWords g_dev_words[kMaxDevices];
std::deque<int32_t> g_free_words;     // FIFO: a freed word is reused last
bool g_words_init = false;

// Device addresses of the error arrays on device dev (looked up once per
// device, with that device current). Caller holds g_err_mutex.
hipError_t words_of(int dev, DeviceWords* out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceWords& w = g_dev_words[dev];
  if (!w.words) {
    void* a = nullptr;
    void* b = nullptr;
    hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(g_error_words));
    if (e != hipSuccess) return e;
    e = hipGetSymbolAddress(&b, HIP_SYMBOL(g_error_readout));
    if (e != hipSuccess) return e;
    w.words = static_cast<int32_t*>(a);
    w.readout = static_cast<int32_t*>(b);
  }
  *out = w;
  return hipSuccess;
}

// One thread swaps the word with 0 and keeps the old value: no flag set by a
// kernel between the read and the clear can be lost.
__global__ void read_clear_kernel(int32_t* word, int32_t* readout) { *readout = atomicExch(word, 0); }

}  // namespace

int acquire_error_word(int32_t* slot, int32_t** word, int32_t* device) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  std::lock_guard<std::mutex> lock(g_err_mutex);
  DeviceWords w;
  e = words_of(dev, &w);
  if (e != hipSuccess) return int(e);
  if (!g_words_init) {
    for (int32_t i = 1; i < kErrorWords; ++i) g_free_words.push_back(i);
    g_words_init = true;
  }
  if (g_free_words.empty()) return int(hipErrorOutOfMemory);
  const int32_t i = g_free_words.front();
  // A word starts clear whatever an earlier pool left in it (synchronous copy).
  const int32_t zero = 0;
  e = hipMemcpy(w.words + i, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return int(e);
  g_free_words.pop_front();
  *slot = i;
  *word = w.words + i;
  *device = dev;
  return 0;
}

void release_error_word(int32_t slot) {
  if (slot <= 0 || slot >= kErrorWords) return;
  std::lock_guard<std::mutex> lock(g_err_mutex);
  g_free_words.push_back(slot);
}

int32_t* shared_error_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_err_mutex);
  DeviceWords w;
  if (words_of(dev, &w) != hipSuccess) return nullptr;
  return w.words;
}

int read_and_clear_error_word(int32_t slot, void* stream, int32_t* value) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  std::lock_guard<std::mutex> lock(g_err_mutex);
  DeviceWords w;
  e = words_of(dev, &w);
  if (e != hipSuccess) return int(e);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(read_clear_kernel, dim3(1), dim3(1), 0, st, w.words + slot, w.readout + slot);
  e = hipGetLastError();
  int32_t host = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&host, w.readout + slot, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return int(e);
  if (value) *value = host;
  return 0;
}

// Split-K workspace of pa_decode_noalloc: a file-scope device array, so that
// callers that cannot allocate (graph capture, tight serving loops) still get
// split-K decode. Each GPU holds its own copy for the life of the process.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the host-side name of the array is not a
// device address).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kMaxDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

}  // namespace pa

using pa::fail;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status check_geometry(const char* fn, int32_t num_blocks, int32_t block_size, int32_t num_heads,
                         int32_t head_dim, pa_dtype kv_dtype) {
  if (num_blocks <= 0 || num_heads <= 0 || block_size <= 0 || head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: sizes must be positive (blocks=%d bs=%d heads=%d dim=%d)", fn,
                num_blocks, block_size, num_heads, head_dim);
  if (!pa::geometry_supported(block_size, head_dim))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size=%d head_dim=%d (supported: 16/32/64 and 64/128)", fn,
                block_size, head_dim);
  if (kv_dtype != PA_F32 && kv_dtype != PA_F16 && kv_dtype != PA_I8 && kv_dtype != PA_I4)
    return fail(PA_ERR_UNSUPPORTED, "%s: kv dtype %d", fn, int(kv_dtype));
  return PA_OK;
}

pa_status hip_status(const char* fn, int e) {
  if (e == 0) return PA_OK;
  return fail(PA_ERR_HIP, "%s: HIP error %d (%s)", fn, e, hipGetErrorString(hipError_t(e)));
}

}  // namespace

extern "C" {

pa_status pa_pool_bytes(int32_t num_blocks, int32_t block_size, int32_t num_heads, int32_t head_dim,
                        pa_dtype kv_dtype, int64_t* kv_bytes, int64_t* scale_bytes) {
  if (!kv_bytes || !scale_bytes) return fail(PA_ERR_INVALID_ARG, "pa_pool_bytes: NULL output");
  pa_status st = check_geometry("pa_pool_bytes", num_blocks, block_size, num_heads, head_dim, kv_dtype);
  if (st != PA_OK) return st;
  *kv_bytes = int64_t(num_blocks) * num_heads * block_size * pa::row_bytes(kv_dtype, head_dim);
  *scale_bytes = pa::is_quantised(kv_dtype) ? int64_t(num_blocks) * num_heads * 2 : 0;
  return PA_OK;
}

pa_status pa_alloc_pool(int32_t num_blocks, int32_t block_size, int32_t num_heads, int32_t head_dim,
                        pa_dtype kv_dtype, void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                        pa_pool** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "pa_alloc_pool: out is NULL");
  *out = nullptr;
  pa_status st = check_geometry("pa_alloc_pool", num_blocks, block_size, num_heads, head_dim, kv_dtype);
  if (st != PA_OK) return st;
  if (!k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "pa_alloc_pool: NULL cache buffer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "pa_alloc_pool: cache buffers must be 16-byte aligned");
  if (pa::is_quantised(kv_dtype)) {
    if (!k_scale || !v_scale) return fail(PA_ERR_INVALID_ARG, "pa_alloc_pool: int8/int4 pool needs scales");
  } else if (k_scale || v_scale) {
    return fail(PA_ERR_INVALID_ARG, "pa_alloc_pool: scales given for a float pool");
  }
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return fail(PA_ERR_INVALID_ARG, "pa_alloc_pool: out of host memory");
  *p = pa_pool{num_blocks, block_size, num_heads, head_dim, kv_dtype, k_cache, v_cache, k_scale, v_scale,
               0, nullptr, 0};
  const hipError_t e = hipError_t(pa::acquire_error_word(&p->err_slot, &p->err, &p->device));
  if (e == hipErrorNoDevice) {
    // No GPU in this process: the descriptor still serves host-side
    // validation; any call that reaches a launch fails with PA_ERR_HIP.
    p->err_slot = 0;
    p->err = nullptr;
    p->device = -1;
  } else if (e != hipSuccess) {
    delete p;
    if (e == hipErrorOutOfMemory)
      return fail(PA_ERR_OUT_OF_RANGE, "pa_alloc_pool: more than %d pools alive", pa::kErrorWords - 1);
    return fail(PA_ERR_HIP, "pa_alloc_pool: error word: HIP error %d (%s)", int(e), hipGetErrorString(e));
  }
  *out = p;
  return PA_OK;
}

pa_status pa_free_pool(pa_pool* pool) {
  if (pool) pa::release_error_word(pool->err_slot);
  delete pool;
  return PA_OK;
}

pa_status pa_write_kv(pa_pool* pool, const void* k_new, const void* v_new, pa_dtype src_dtype,
                      const int64_t* slot_mapping, int32_t n, pa_stream stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pa_write_kv: pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "pa_write_kv: n=%d", n);
  if (n == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "pa_write_kv: NULL buffer");
  if (src_dtype != PA_F32 && src_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: source dtype %d (F32 or F16)", int(src_dtype));
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_INVALID_ARG, "pa_write_kv: new rows must be 16-byte aligned");
  return hip_status("pa_write_kv", pa::launch_write_kv(pool, k_new, v_new, src_dtype, slot_mapping, n, stream));
}

pa_status pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int32_t n, pa_stream stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pool is NULL");
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: n=%d", n);
  if (n == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pairs is NULL");
  if (n > 65535) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: n=%d > 65535 pairs per call", n);
  return hip_status("pa_copy_blocks", pa::launch_copy_blocks(pool, pairs, n, stream));
}

// Device view of pinned host memory, or nullptr (with *e set) if it has none.
// A failed lookup is cleared from the runtime's last-error slot so that it
// is not reported again by the next launch check.
static void* host_view(void* host, hipError_t* e) {
  void* view = nullptr;
  *e = hipHostGetDevicePointer(&view, host, 0);
  if (*e != hipSuccess || !view) {
    (void)hipGetLastError();
    return nullptr;
  }
  return view;
}

pa_status pa_swap_blocks(pa_pool* pool, void* host_k, void* host_v, void* host_k_scale, void* host_v_scale,
                         int32_t num_host_blocks, const int32_t* pairs, int32_t n, int32_t direction,
                         pa_stream stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: pool is NULL");
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: direction %d", direction);
  if (n < 0 || num_host_blocks < 0) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: negative size");
  if (n == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: pairs is NULL");
  if (n > 65535) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: n=%d > 65535 pairs per call", n);
  if (!host_k || !host_v || !aligned16(host_k) || !aligned16(host_v))
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: host K/V must be non-NULL and 16-byte aligned");
  const bool quant = pa::is_quantised(pool->kv_dtype);
  if (quant != (host_k_scale != nullptr && host_v_scale != nullptr) || (!quant && (host_k_scale || host_v_scale)))
    return fail(PA_ERR_INVALID_ARG,
                "pa_swap_blocks: host scales are required for int8 and int4 pools and only for them");
  pa::SwapHost h{};
  hipError_t e = hipSuccess;
  h.num_blocks = num_host_blocks;
  void* in[4] = {host_k, host_v, host_k_scale, host_v_scale};
  void** view[4] = {&h.k, &h.v, &h.k_scale, &h.v_scale};
  for (int i = 0; i < 4; ++i) {
    if (!in[i]) continue;
    *view[i] = host_view(in[i], &e);
    if (!*view[i])
      return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: host buffer %d is not pinned host memory (%s)", i,
                  hipGetErrorString(e));
  }
  if (!aligned16(h.k) || !aligned16(h.v))
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: device view of the host pool is unaligned");
  return hip_status("pa_swap_blocks", pa::launch_swap_blocks(pool, h, pairs, n, direction == PA_SWAP_OUT, stream));
}

static int64_t num_partitions(int32_t max_ctx, int32_t partition_tokens) {
  if (partition_tokens <= 0) return 1;
  const int64_t p = (int64_t(max_ctx) + partition_tokens - 1) / partition_tokens;
  return p < 1 ? 1 : p;
}

// m and l hold n = S * H * P floats each, padded to a multiple of 4 so that
// o starts 16-byte aligned.
static int64_t padded4(int64_t n) { return (n + 3) / 4 * 4; }

static int64_t workspace_bytes_for(int64_t S, int64_t H, int64_t D, int64_t P) {
  if (P <= 1) return 0;
  const int64_t n = S * H * P;
  return (2 * padded4(n) + n * D) * 4;
}

pa_status pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t max_context_len,
                                    int32_t partition_tokens, int64_t* bytes) {
  if (!pool || !bytes) return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_bytes: NULL argument");
  if (num_seqs < 0 || max_context_len < 0 || partition_tokens < 0 || partition_tokens % pool->block_size)
    return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_bytes: bad sizes (partition_tokens=%d, block_size=%d)",
                partition_tokens, pool->block_size);
  *bytes = workspace_bytes_for(num_seqs, pool->num_heads, pool->head_dim,
                               num_partitions(max_context_len, partition_tokens));
  return PA_OK;
}

static pa_status decode_common(const char* fn, pa::DecodeArgs& a, void* workspace, int64_t ws_bytes,
                               pa_stream stream) {
  if (!a.q || !a.out || !a.ctx) return fail(PA_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  if (a.q_dtype != PA_F32 && a.q_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "%s: q dtype %d (F32 or F16)", fn, int(a.q_dtype));
  if (a.num_seqs < 0 || a.max_ctx < 0) return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (a.schedule != PA_SCHED_HEADS && a.schedule != PA_SCHED_SHARED)
    return fail(PA_ERR_INVALID_ARG, "%s: schedule %d", fn, a.schedule);
  if (a.partition_tokens < 0 || a.partition_tokens % a.block_size)
    return fail(PA_ERR_INVALID_ARG, "%s: partition_tokens=%d (0 or a multiple of the block size %d)", fn,
                a.partition_tokens, a.block_size);
  if (a.q_dtype == PA_F16 && !aligned16(a.q))
    return fail(PA_ERR_INVALID_ARG, "%s: fp16 q must be 16-byte aligned", fn);
  if (!(a.sm_scale > 0.f) || std::isinf(a.sm_scale)) a.sm_scale = 1.0f / std::sqrt(float(a.head_dim));
  const int64_t P = num_partitions(a.max_ctx, a.partition_tokens);
  const int64_t grid = int64_t(a.num_seqs) * a.num_heads * P;
  if (grid > int64_t(0x7fffffff)) return fail(PA_ERR_INVALID_ARG, "%s: grid of %lld workgroups too large", fn, (long long)grid);
  a.num_partitions = int32_t(P);
  a.ws_m = a.ws_l = a.ws_o = nullptr;
  const int64_t need = workspace_bytes_for(a.num_seqs, a.num_heads, a.head_dim, P);
  if (need > 0) {
    if (!workspace || ws_bytes < need)
      return fail(PA_ERR_INVALID_ARG, "%s: workspace of %lld bytes needed, %lld given", fn, (long long)need,
                  (long long)ws_bytes);
    if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
    const int64_t n = int64_t(a.num_seqs) * a.num_heads * P;
    a.ws_m = static_cast<float*>(workspace);
    a.ws_l = a.ws_m + padded4(n);
    a.ws_o = a.ws_l + padded4(n);
  }
  if (a.num_seqs == 0) return PA_OK;
  return hip_status(fn, pa::launch_decode(a, stream));
}

pa_status pa_decode(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                    float sm_scale, int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                    pa_stream stream) {
  return pa_decode_ordered(pool, q, q_dtype, out, block_tables, max_blocks, context_lens, nullptr, PA_SCHED_HEADS,
                           num_seqs, max_context_len, sm_scale, partition_tokens, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, float sm_scale,
                            int32_t partition_tokens, pa_stream stream) {
  const char* fn = "pa_decode_noalloc";
  if (!pool) return fail(PA_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (num_seqs < 0 || max_context_len < 0 || partition_tokens < 0 || partition_tokens % pool->block_size)
    return fail(PA_ERR_INVALID_ARG, "%s: bad sizes (partition_tokens=%d, block_size=%d)", fn, partition_tokens,
                pool->block_size);
  const int64_t need = workspace_bytes_for(num_seqs, pool->num_heads, pool->head_dim,
                                           num_partitions(max_context_len, partition_tokens));
  if (need > pa::kScratchBytes)
    return fail(PA_ERR_OUT_OF_RANGE, "%s: split-K needs %lld bytes of workspace, more than the %lld of the "
                "library's static scratch (fewer sequences, shorter contexts or longer partitions)", fn,
                (long long)need, (long long)pa::kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int e = pa::scratch_address(&ws);
    if (e != 0) return hip_status(fn, e);
  }
  if (!block_tables) return fail(PA_ERR_INVALID_ARG, "%s: block_tables is NULL", fn);
  if (max_blocks < 0 || int64_t(max_blocks) * pool->block_size < int64_t(max_context_len))
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks=%d cannot hold max_context_len=%d", fn, max_blocks,
                max_context_len);
  pa::DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.out = out;
  a.k = pool->k_cache;
  a.v = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.kv_dtype = pool->kv_dtype;
  a.tables = block_tables;
  a.max_blocks = max_blocks;
  a.block_size = pool->block_size;
  a.max_tokens = 0;
  a.err = pool->err;
  a.ctx = context_lens;
  a.order = nullptr;
  a.schedule = PA_SCHED_HEADS;
  a.num_seqs = num_seqs;
  a.num_heads = pool->num_heads;
  a.head_dim = pool->head_dim;
  a.num_blocks = pool->num_blocks;
  a.max_ctx = max_context_len;
  a.sm_scale = sm_scale;
  a.partition_tokens = partition_tokens;
  return decode_common(fn, a, ws, need, stream);
}

pa_status pa_decode_ordered(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                            const int32_t* seq_order, int32_t schedule, int32_t num_seqs, int32_t max_context_len,
                            float sm_scale,
                            int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                            pa_stream stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pa_decode: pool is NULL");
  if (!block_tables) return fail(PA_ERR_INVALID_ARG, "pa_decode: block_tables is NULL");
  if (max_context_len < 0 || max_blocks < 0 ||
      int64_t(max_blocks) * pool->block_size < int64_t(max_context_len))
    return fail(PA_ERR_INVALID_ARG, "pa_decode: max_blocks=%d cannot hold max_context_len=%d", max_blocks,
                max_context_len);
  pa::DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.out = out;
  a.k = pool->k_cache;
  a.v = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.kv_dtype = pool->kv_dtype;
  a.tables = block_tables;
  a.max_blocks = max_blocks;
  a.block_size = pool->block_size;
  a.max_tokens = 0;
  a.err = pool->err;
  a.ctx = context_lens;
  a.order = seq_order;
  a.schedule = schedule;
  a.num_seqs = num_seqs;
  a.num_heads = pool->num_heads;
  a.head_dim = pool->head_dim;
  a.num_blocks = pool->num_blocks;
  a.max_ctx = max_context_len;
  a.sm_scale = sm_scale;
  a.partition_tokens = partition_tokens;
  return decode_common("pa_decode", a, workspace, workspace_bytes, stream);
}

pa_status pa_prefill(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out, const int32_t* query_start,
                     int32_t num_rows, const int32_t* block_tables, int32_t max_blocks,
                     const int32_t* context_lens, int32_t num_seqs, int32_t max_query_len,
                     int32_t max_context_len, float sm_scale, pa_stream stream) {
  return pa_prefill_ordered(pool, q, q_dtype, out, query_start, num_rows, block_tables, max_blocks, context_lens,
                            nullptr, num_seqs, max_query_len, max_context_len, sm_scale, stream);
}

pa_status pa_prefill_ordered(pa_pool* pool, const void* q, pa_dtype q_dtype, void* out,
                             const int32_t* query_start, int32_t num_rows, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, const int32_t* seq_order,
                             int32_t num_seqs, int32_t max_query_len, int32_t max_context_len, float sm_scale,
                             pa_stream stream) {
  const char* fn = "pa_prefill";
  if (!pool) return fail(PA_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (pool->kv_dtype != PA_F16 && pool->kv_dtype != PA_I8 && pool->kv_dtype != PA_I4)
    return fail(PA_ERR_UNSUPPORTED, "%s: pool dtype %d (F16, I8 or I4 only)", fn, int(pool->kv_dtype));
  if (q_dtype != PA_F16) return fail(PA_ERR_UNSUPPORTED, "%s: q dtype %d (F16 only)", fn, int(q_dtype));
  if (num_seqs < 0 || num_rows < 0 || max_query_len < 0 || max_context_len < 0 || max_blocks < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (int64_t(max_blocks) * pool->block_size < int64_t(max_context_len))
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks=%d cannot hold max_context_len=%d", fn, max_blocks,
                max_context_len);
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!q || !out || !query_start || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  if (!aligned16(q) || !aligned16(out)) return fail(PA_ERR_INVALID_ARG, "%s: q and out must be 16-byte aligned", fn);
  if (pa::prefill_groups(num_seqs, pool->num_heads, max_query_len) > int64_t(0x7fffffff))
    return fail(PA_ERR_INVALID_ARG, "%s: grid too large", fn);
  // The kernel indexes pool rows (one token of one head) with 32 bits.
  if (int64_t(pool->num_blocks) * pool->num_heads * pool->block_size > int64_t(0xffffffff))
    return fail(PA_ERR_UNSUPPORTED, "%s: pool of more than 2^32 token-head rows", fn);
  pa::PrefillArgs a{};
  a.pool = pool;
  a.q = q;
  a.out = out;
  a.query_start = query_start;
  a.num_rows = num_rows;
  a.tables = block_tables;
  a.max_blocks = max_blocks;
  a.ctx = context_lens;
  a.order = seq_order;
  a.num_seqs = num_seqs;
  a.max_query_len = max_query_len;
  a.max_ctx = max_context_len;
  a.sm_scale = (sm_scale > 0.f && !std::isinf(sm_scale)) ? sm_scale : 1.0f / std::sqrt(float(pool->head_dim));
  return hip_status(fn, pa::launch_prefill(a, stream));
}

pa_status pa_write_decode(pa_pool* pool, const void* k_new, const void* v_new, pa_dtype src_dtype,
                          const int64_t* slot_mapping, const void* q, pa_dtype q_dtype, void* out,
                          const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                          const int32_t* seq_order, int32_t schedule, int32_t num_seqs, int32_t max_context_len,
                          float sm_scale,
                          int32_t partition_tokens, void* workspace, int64_t workspace_bytes,
                          pa_stream stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "pa_write_decode: pool is NULL");
  if (pa::is_quantised(pool->kv_dtype))
    return fail(PA_ERR_UNSUPPORTED, "pa_write_decode: int8 and int4 pools quantise per block; use pa_write_kv");
  if (src_dtype != PA_F32 && src_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "pa_write_decode: source dtype %d (F32 or F16)", int(src_dtype));
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return fail(PA_ERR_INVALID_ARG, "pa_write_decode: NULL new rows or slots");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_INVALID_ARG, "pa_write_decode: new rows must be 16-byte aligned");
  if (!block_tables) return fail(PA_ERR_INVALID_ARG, "pa_write_decode: block_tables is NULL");
  if (max_context_len < 0 || max_blocks < 0 || int64_t(max_blocks) * pool->block_size < int64_t(max_context_len))
    return fail(PA_ERR_INVALID_ARG, "pa_write_decode: max_blocks=%d cannot hold max_context_len=%d", max_blocks,
                max_context_len);
  pa::DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.out = out;
  a.k = pool->k_cache;
  a.v = pool->v_cache;
  a.kv_dtype = pool->kv_dtype;
  a.tables = block_tables;
  a.max_blocks = max_blocks;
  a.block_size = pool->block_size;
  a.ctx = context_lens;
  a.order = seq_order;
  a.schedule = schedule;
  a.num_seqs = num_seqs;
  a.num_heads = pool->num_heads;
  a.head_dim = pool->head_dim;
  a.num_blocks = pool->num_blocks;
  a.max_ctx = max_context_len;
  a.sm_scale = sm_scale;
  a.partition_tokens = partition_tokens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_dtype = src_dtype;
  a.slots = slot_mapping;
  a.err = pool->err;
  return decode_common("pa_write_decode", a, workspace, workspace_bytes, stream);
}

// The two pools of mixed-precision pages: int8 or int4 cold, fp16 hot,
// 16-token blocks, equal heads and head_dim.
static pa_status check_mixed_pools(const char* fn, const pa_pool* cold, const pa_pool* hot) {
  if (!cold || !hot) return fail(PA_ERR_INVALID_ARG, "%s: pool is NULL", fn);
  if (!pa::is_quantised(cold->kv_dtype) || hot->kv_dtype != PA_F16 || cold->block_size != 16 ||
      hot->block_size != 16 || cold->num_heads != hot->num_heads || cold->head_dim != hot->head_dim)
    return fail(PA_ERR_INVALID_ARG, "%s: needs an int8 or int4 cold pool and an fp16 hot pool of 16-token "
                "blocks with equal heads and head_dim", fn);
  return PA_OK;
}

pa_status pa_demote_blocks(pa_pool* hot_pool, pa_pool* cold_pool, const int32_t* pairs, int32_t n,
                           pa_stream stream) {
  pa_status st = check_mixed_pools("pa_demote_blocks", cold_pool, hot_pool);
  if (st != PA_OK) return st;
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "pa_demote_blocks: n=%d", n);
  if (n == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID_ARG, "pa_demote_blocks: pairs is NULL");
  if (n > 65535) return fail(PA_ERR_INVALID_ARG, "pa_demote_blocks: n=%d > 65535 pairs per call", n);
  return hip_status("pa_demote_blocks", pa::launch_demote_blocks(hot_pool, cold_pool, pairs, n, stream));
}

pa_status pa_decode_mixed(pa_pool* cold_pool, pa_pool* hot_pool, const void* q, pa_dtype q_dtype, void* out,
                          const int32_t* cold_tables, int32_t max_blocks, const int32_t* hot_blocks,
                          const int32_t* context_lens, const int32_t* seq_order, int32_t schedule,
                          int32_t num_seqs,
                          int32_t max_context_len, float sm_scale, int32_t partition_tokens, void* workspace,
                          int64_t workspace_bytes, pa_stream stream) {
  pa_status st = check_mixed_pools("pa_decode_mixed", cold_pool, hot_pool);
  if (st != PA_OK) return st;
  if (!cold_tables || !hot_blocks) return fail(PA_ERR_INVALID_ARG, "pa_decode_mixed: tables are NULL");
  if (max_context_len < 0 || max_blocks < 0 || int64_t(max_blocks) * 16 + 16 < int64_t(max_context_len))
    return fail(PA_ERR_INVALID_ARG, "pa_decode_mixed: max_blocks=%d cannot hold max_context_len=%d", max_blocks,
                max_context_len);
  pa::DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.out = out;
  a.k = cold_pool->k_cache;
  a.v = cold_pool->v_cache;
  a.k_scale = cold_pool->k_scale;
  a.v_scale = cold_pool->v_scale;
  a.kv_dtype = cold_pool->kv_dtype;
  a.tables = cold_tables;
  a.max_blocks = max_blocks;
  a.block_size = 16;
  a.ctx = context_lens;
  a.order = seq_order;
  a.schedule = schedule;
  a.num_seqs = num_seqs;
  a.num_heads = cold_pool->num_heads;
  a.head_dim = cold_pool->head_dim;
  a.num_blocks = cold_pool->num_blocks;
  a.max_ctx = max_context_len;
  a.sm_scale = sm_scale;
  a.partition_tokens = partition_tokens;
  a.hot_k = hot_pool->k_cache;
  a.hot_v = hot_pool->v_cache;
  a.hot_blocks = hot_blocks;
  a.num_hot = hot_pool->num_blocks;
  a.err = cold_pool->err;
  return decode_common("pa_decode_mixed", a, workspace, workspace_bytes, stream);
}

pa_status pa_decode_contiguous(const void* k, const void* v, pa_dtype kv_dtype, int32_t num_heads,
                               int32_t head_dim, int32_t max_tokens, const void* q, pa_dtype q_dtype,
                               void* out, const int32_t* context_lens, const int32_t* seq_order,
                               int32_t num_seqs, float sm_scale, int32_t partition_tokens, void* workspace,
                               int64_t workspace_bytes, pa_stream stream) {
  if (!k || !v) return fail(PA_ERR_INVALID_ARG, "pa_decode_contiguous: NULL cache");
  if (kv_dtype != PA_F32 && kv_dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_contiguous: float KV only");
  if (num_heads <= 0 || max_tokens < 0 || max_tokens % pa::kTileRows)
    return fail(PA_ERR_INVALID_ARG, "pa_decode_contiguous: heads=%d max_tokens=%d (a multiple of 16)",
                num_heads, max_tokens);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_decode_contiguous: head_dim %d", head_dim);
  if (!aligned16(k) || !aligned16(v)) return fail(PA_ERR_INVALID_ARG, "pa_decode_contiguous: unaligned cache");
  pa::DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.out = out;
  a.k = k;
  a.v = v;
  a.kv_dtype = kv_dtype;
  a.tables = nullptr;
  a.block_size = pa::kTileRows;
  a.max_tokens = max_tokens;
  a.ctx = context_lens;
  a.order = seq_order;
  a.schedule = PA_SCHED_HEADS;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.num_blocks = 0;
  a.max_ctx = max_tokens;
  a.err = pa::shared_error_word();
  a.sm_scale = sm_scale;
  a.partition_tokens = partition_tokens;
  return decode_common("pa_decode_contiguous", a, workspace, workspace_bytes, stream);
}

pa_status pa_check_errors(const pa_pool* pool, pa_stream stream, int32_t* device_error) {
  if (pool) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != pool->device)
      return fail(PA_ERR_INVALID_ARG, "pa_check_errors: the pool lives on device %d, device %d is current",
                  pool->device, dev);
  }
  return hip_status("pa_check_errors", pa::read_and_clear_error_word(pool ? pool->err_slot : 0, stream,
                                                                      device_error));
}

pa_status pa_stream_copy(void* dst, const void* src, int64_t bytes, pa_stream stream) {
  if (!dst || !src || bytes < 0 || bytes % 16 || !aligned16(dst) || !aligned16(src))
    return fail(PA_ERR_INVALID_ARG, "pa_stream_copy: bad arguments");
  return hip_status("pa_stream_copy", pa::launch_stream_copy(dst, src, bytes, stream));
}

pa_status pa_stage_copy(void* dst, const void* host_src, int64_t bytes, pa_stream stream) {
  if (!dst || !host_src || bytes < 0 || bytes % 16 || !aligned16(dst) || !aligned16(host_src))
    return fail(PA_ERR_INVALID_ARG, "pa_stage_copy: bad arguments");
  if (bytes == 0) return PA_OK;
  hipError_t e = hipSuccess;
  void* view = host_view(const_cast<void*>(host_src), &e);
  if (!view)
    return fail(PA_ERR_INVALID_ARG, "pa_stage_copy: source is not pinned host memory (%s)", hipGetErrorString(e));
  if (!aligned16(view)) return fail(PA_ERR_INVALID_ARG, "pa_stage_copy: device view of the source is unaligned");
  return hip_status("pa_stage_copy", pa::launch_stage_copy(dst, view, bytes, stream));
}

pa_status pa_host_view(void* host, void** device_view) {
  if (!host || !device_view) return fail(PA_ERR_INVALID_ARG, "pa_host_view: NULL argument");
  hipError_t e = hipSuccess;
  *device_view = host_view(host, &e);
  if (!*device_view)
    return fail(PA_ERR_INVALID_ARG, "pa_host_view: not pinned host memory (%s)", hipGetErrorString(e));
  return PA_OK;
}

pa_status pa_stream_read(const void* src, int64_t bytes, void* sink, pa_stream stream) {
  if (!src || !sink || bytes < 0 || bytes % 16 || !aligned16(src))
    return fail(PA_ERR_INVALID_ARG, "pa_stream_read: bad arguments");
  return hip_status("pa_stream_read", pa::launch_stream_read(src, bytes, sink, stream));
}

}  // extern "C"
