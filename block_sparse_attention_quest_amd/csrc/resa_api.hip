// C ABI of libresa.so: argument validation, workspace sizing and launch order.
// All checks run on the host before anything is launched; nothing here reads
// device memory or synchronises with the device, except in checked builds
// (RESA_DEBUG_CHECKS), where each call waits for its stream and reads the word
// the kernels' precondition checks set.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "resa_internal.h"

namespace {

thread_local char g_err[512] = "";

resa_status fail(resa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

resa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RESA_OK;
  return fail(RESA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// Element arrays are read with vector loads of up to 16 bytes, integer arrays
// with 4-byte loads.
resa_status check_aligned16(const char* what, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !aligned(p, 16)) return fail(RESA_ERR_INVALID, "%s must be 16-byte aligned", what);
  return RESA_OK;
}

resa_status check_cache(const resa_cache* c, resa::CacheView* v) {
  if (!c) return fail(RESA_ERR_INVALID, "cache is NULL");
  if (c->dtype != RESA_FP32 && c->dtype != RESA_BF16) return fail(RESA_ERR_INVALID, "dtype %d", c->dtype);
  if (c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 || c->head_dim < 1)
    return fail(RESA_ERR_INVALID, "batch, head counts and head_dim must be positive");
  if (c->num_q_heads % c->num_kv_heads != 0)
    return fail(RESA_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d", c->num_q_heads,
                c->num_kv_heads);
  const int G = c->num_q_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(RESA_ERR_UNSUPPORTED, "group size %d (built: 1, 2, 4, 8)", G);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(RESA_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", c->head_dim);
  if (c->block_size != resa::kBlock) return fail(RESA_ERR_INVALID, "block_size must be 16, got %d", c->block_size);
  if (c->num_pages < 1 || c->max_blocks_per_seq < 1 || c->max_seq_len < 1)
    return fail(RESA_ERR_INVALID, "num_pages, max_blocks_per_seq and max_seq_len must be positive");
  if ((long)c->max_seq_len > (long)c->max_blocks_per_seq * resa::kBlock)
    return fail(RESA_ERR_INVALID, "max_seq_len %d exceeds max_blocks_per_seq * 16", c->max_seq_len);
  if (c->max_blocks_per_seq > resa::kTopnThreads * resa::kTopnMaxPerThread)
    return fail(RESA_ERR_UNSUPPORTED, "max_blocks_per_seq %d exceeds %d", c->max_blocks_per_seq,
                resa::kTopnThreads * resa::kTopnMaxPerThread);
  if ((long)c->num_kv_heads * c->head_dim > 4096)
    return fail(RESA_ERR_UNSUPPORTED, "num_kv_heads * head_dim exceeds 4096");
  if (!c->k_pages || !c->v_pages || !c->desc || !c->block_table || !c->seq_lens)
    return fail(RESA_ERR_INVALID, "cache has a NULL pointer");
  if (!aligned(c->k_pages, 16) || !aligned(c->v_pages, 16) || !aligned(c->desc, 16))
    return fail(RESA_ERR_INVALID, "k_pages, v_pages and desc must be 16-byte aligned");
  if (!aligned(c->block_table, 4) || !aligned(c->seq_lens, 4))
    return fail(RESA_ERR_INVALID, "block_table and seq_lens must be 4-byte aligned");
  v->dtype = c->dtype;
  v->B = c->batch;
  v->Hq = c->num_q_heads;
  v->Hkv = c->num_kv_heads;
  v->D = c->head_dim;
  v->G = G;
  v->num_pages = c->num_pages;
  v->maxb = c->max_blocks_per_seq;
  v->max_seq_len = c->max_seq_len;
  v->k = c->k_pages;
  v->v = c->v_pages;
  v->kw = c->k_pages;
  v->vw = c->v_pages;
  v->desc = c->desc;
  v->bt = c->block_table;
  v->seq_lens = c->seq_lens;
  v->dbg = nullptr;
  return RESA_OK;
}

resa_status check_params(const resa_select_params* p) {
  if (!p) return fail(RESA_ERR_INVALID, "params is NULL");
  if (p->n_min < 1) return fail(RESA_ERR_INVALID, "n_min must be >= 1");
  if (p->n_local < 0) return fail(RESA_ERR_INVALID, "n_local must be >= 0");
  if (!(p->r > 0.0 && p->r <= 1.0)) return fail(RESA_ERR_INVALID, "r must be in (0, 1]");
  return RESA_OK;
}

constexpr int kMaxDevices = 64;

// The device address of a __device__ array on the current device `dev`,
// looked up once per device (each GPU holds its own copy of the array).
resa_status symbol_on_device(const void* sym, const char* name, std::atomic<void*>* cache, int dev, void** out) {
  static std::mutex mu;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = cache[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, sym);
      if (e != hipSuccess) return fail(RESA_ERR_HIP, "hipGetSymbolAddress(%s): %s", name, hipGetErrorString(e));
      if (!p) return fail(RESA_ERR_HIP, "hipGetSymbolAddress(%s) returned NULL", name);
      cache[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RESA_OK;
}

resa_status current_device(int* dev) {
  const hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (*dev < 0 || *dev >= kMaxDevices) return fail(RESA_ERR_UNSUPPORTED, "device %d (at most %d devices)", *dev, kMaxDevices);
  return RESA_OK;
}

// Scratch of resa_sparse_decode_noalloc: the decode's split partials live in
// this array instead of a caller workspace. Each GPU the library runs on holds
// its own copy until the process ends; host code never uses the array's name as
// an address, only the device pointer hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

#ifdef RESA_DEBUG_CHECKS
// Checked builds: the word the kernels' precondition checks set (one per
// device). Every launching call attaches it to the cache view, then waits for
// its stream and turns a set bit into RESA_ERR_INVALID. Calls that overlap on
// one device share the word, so a failed check may be reported by another of
// them; checked builds are for testing, one stream at a time.
static __device__ int debug_word[1];
std::atomic<void*> g_debug_ptr[kMaxDevices];

resa_status debug_attach(resa::CacheView* v) {
  int dev = -1;
  resa_status st = current_device(&dev);
  if (st != RESA_OK) return st;
  void* p = nullptr;
  if ((st = symbol_on_device(HIP_SYMBOL(debug_word), "debug_word", g_debug_ptr, dev, &p)) != RESA_OK) return st;
  v->dbg = static_cast<int*>(p);
  return RESA_OK;
}

resa_status debug_collect(resa_status st, hipStream_t s, const resa::CacheView& v) {
  if (st != RESA_OK) return st;
  // under graph capture nothing runs yet and the stream cannot be waited on:
  // a check that fails on a replay is reported by the next uncaptured call
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return hip_status(e, "hipStreamIsCapturing (checked build)");
  if (cap != hipStreamCaptureStatusNone) return RESA_OK;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "hipStreamSynchronize (checked build)");
  int word = 0;
  if ((e = hipMemcpy(&word, v.dbg, sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_status(e, "reading the check word");
  if (!word) return RESA_OK;
  const int zero = 0;
  if ((e = hipMemcpy(v.dbg, &zero, sizeof(int), hipMemcpyHostToDevice)) != hipSuccess)
    return hip_status(e, "clearing the check word");
  return fail(RESA_ERR_INVALID, "device-side precondition check failed:%s%s%s%s%s",
              word & resa::kChkSeqLen ? " seq_lens[b] outside 0 .. max_seq_len;" : "",
              word & resa::kChkPage ? " a held block's block_table entry outside 0 .. num_pages - 1;" : "",
              word & resa::kChkEmpty ? " an empty sequence where a token is needed;" : "",
              word & resa::kChkSelection ? " count above n_cap or a selected block outside the sequence;" : "",
              word & resa::kChkRectF ? " f above seq_lens[b];" : "");
}
#define RESA_DEBUG_ATTACH(v)                              \
  do {                                                    \
    const resa_status ast = debug_attach(&(v));           \
    if (ast != RESA_OK) return ast;                       \
  } while (0)
#define RESA_DEBUG_COLLECT(expr, stream, v) debug_collect((expr), (stream), (v))
#else
#define RESA_DEBUG_ATTACH(v) \
  do {                       \
  } while (0)
#define RESA_DEBUG_COLLECT(expr, stream, v) (expr)
#endif

int n_for(int M, const resa_select_params* p) {
  int n = (int)ceil((double)M * p->r);
  if (n < p->n_min) n = p->n_min;
  return n < M ? n : M;
}

}  // namespace

extern "C" {

int32_t resa_n_cap(const resa_cache* cache, const resa_select_params* params) {
  resa::CacheView v;
  if (check_cache(cache, &v) != RESA_OK || check_params(params) != RESA_OK) return -1;
  return n_for((v.max_seq_len + resa::kBlock - 1) / resa::kBlock, params);
}

size_t resa_select_workspace_size(const resa_cache* cache) {
  resa::CacheView v;
  if (check_cache(cache, &v) != RESA_OK) return 0;
  return resa::select_ws_bytes(v);
}

size_t resa_decode_workspace_size(const resa_cache* cache, int32_t n_cap) {
  resa::CacheView v;
  if (check_cache(cache, &v) != RESA_OK || n_cap < 1) return 0;
  return resa::decode_ws_bytes(v, n_cap);
}

size_t resa_rectify_workspace_size(const resa_cache* cache, int32_t f) {
  resa::CacheView v;
  if (check_cache(cache, &v) != RESA_OK || f < 1 || f > resa::kMaxRectF) return 0;
  return resa::rectify_ws_bytes(v, f);
}

resa_status resa_update_descriptors(const resa_cache* cache, const void* k_new, const void* v_new,
                                    int32_t n_new, void* stream) {
  resa::CacheView v;
  resa_status st = check_cache(cache, &v);
  if (st != RESA_OK) return st;
  if (n_new < 0) return fail(RESA_ERR_INVALID, "n_new must be >= 0");
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(RESA_ERR_INVALID, "k_new and v_new must both be set or both be NULL");
  if (n_new == 0 && k_new) return fail(RESA_ERR_INVALID, "a rebuild (n_new == 0) takes no new tokens");
  if (n_new > v.max_seq_len) return fail(RESA_ERR_INVALID, "n_new %d exceeds max_seq_len %d", n_new, v.max_seq_len);
  if ((st = check_aligned16("k_new and v_new", {k_new, v_new})) != RESA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RESA_DEBUG_ATTACH(v);
  const hipError_t e = n_new == 0 ? resa::launch_rebuild(v, s) : resa::launch_update_tail(v, k_new, v_new, n_new, s);
  return RESA_DEBUG_COLLECT(hip_status(e, "resa_update_descriptors"), s, v);
}

resa_status resa_select_blocks(const resa_cache* cache, const void* q, const resa_select_params* params,
                               int32_t* idx, int32_t* count, int32_t n_cap, void* ws, size_t ws_bytes,
                               void* stream) {
  resa::CacheView v;
  resa_status st = check_cache(cache, &v);
  if (st != RESA_OK) return st;
  if ((st = check_params(params)) != RESA_OK) return st;
  if (!q || !idx || !count) return fail(RESA_ERR_INVALID, "q, idx and count must not be NULL");
  if ((st = check_aligned16("q and ws", {q, ws})) != RESA_OK) return st;
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(RESA_ERR_INVALID, "idx and count must be 4-byte aligned");
  const int need_cap = n_for((v.max_seq_len + resa::kBlock - 1) / resa::kBlock, params);
  if (n_cap < need_cap) return fail(RESA_ERR_INVALID, "n_cap %d is below resa_n_cap() = %d", n_cap, need_cap);
  const size_t need = resa::select_ws_bytes(v);
  if (!ws || ws_bytes < need) return fail(RESA_ERR_WORKSPACE, "select workspace %zu < %zu bytes", ws_bytes, need);
  RESA_DEBUG_ATTACH(v);
  return RESA_DEBUG_COLLECT(
      hip_status(resa::launch_select(v, q, *params, idx, count, n_cap, ws, static_cast<hipStream_t>(stream)),
                 "resa_select_blocks"),
      static_cast<hipStream_t>(stream), v);
}

resa_status resa_append_select(const resa_cache* cache, const void* k_new, const void* v_new, const void* q,
                               const resa_select_params* params, int32_t* idx, int32_t* count, int32_t n_cap,
                               void* ws, size_t ws_bytes, void* stream) {
  resa::CacheView v;
  resa_status st = check_cache(cache, &v);
  if (st != RESA_OK) return st;
  if ((st = check_params(params)) != RESA_OK) return st;
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(RESA_ERR_INVALID, "k_new and v_new must both be set or both be NULL");
  if (!q || !idx || !count) return fail(RESA_ERR_INVALID, "q, idx and count must not be NULL");
  if ((st = check_aligned16("q, k_new, v_new and ws", {q, k_new, v_new, ws})) != RESA_OK) return st;
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(RESA_ERR_INVALID, "idx and count must be 4-byte aligned");
  const int need_cap = n_for((v.max_seq_len + resa::kBlock - 1) / resa::kBlock, params);
  if (n_cap < need_cap) return fail(RESA_ERR_INVALID, "n_cap %d is below resa_n_cap() = %d", n_cap, need_cap);
  const size_t need = resa::select_ws_bytes(v);
  if (!ws || ws_bytes < need) return fail(RESA_ERR_WORKSPACE, "select workspace %zu < %zu bytes", ws_bytes, need);
  RESA_DEBUG_ATTACH(v);
  return RESA_DEBUG_COLLECT(hip_status(resa::launch_append_select(v, k_new, v_new, q, *params, idx, count, n_cap, ws,
                                                                  static_cast<hipStream_t>(stream)),
                                       "resa_append_select"),
                            static_cast<hipStream_t>(stream), v);
}

resa_status resa_sparse_decode(const resa_cache* cache, const void* q, const int32_t* idx,
                               const int32_t* count, int32_t n_cap, float scale, void* out, void* ws,
                               size_t ws_bytes, void* stream) {
  resa::CacheView v;
  resa_status st = check_cache(cache, &v);
  if (st != RESA_OK) return st;
  if (!q || !idx || !count || !out) return fail(RESA_ERR_INVALID, "q, idx, count and out must not be NULL");
  if ((st = check_aligned16("q, out and ws", {q, out, ws})) != RESA_OK) return st;
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(RESA_ERR_INVALID, "idx and count must be 4-byte aligned");
  if (n_cap < 1 || n_cap > v.maxb) return fail(RESA_ERR_INVALID, "n_cap %d outside 1 .. max_blocks_per_seq", n_cap);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RESA_ERR_INVALID, "scale must be positive and finite");
  const size_t need = resa::decode_ws_bytes(v, n_cap);
  if (!ws || ws_bytes < need) return fail(RESA_ERR_WORKSPACE, "decode workspace %zu < %zu bytes", ws_bytes, need);
  RESA_DEBUG_ATTACH(v);
  return RESA_DEBUG_COLLECT(
      hip_status(resa::launch_decode(v, q, idx, count, n_cap, scale, out, ws, static_cast<hipStream_t>(stream)),
                 "resa_sparse_decode"),
      static_cast<hipStream_t>(stream), v);
}

resa_status resa_sparse_decode_noalloc(const resa_cache* cache, const void* q, const int32_t* idx,
                                       const int32_t* count, int32_t n_cap, float scale, void* out,
                                       void* stream) {
  resa::CacheView v;
  resa_status st = check_cache(cache, &v);
  if (st != RESA_OK) return st;
  if (!q || !idx || !count || !out) return fail(RESA_ERR_INVALID, "q, idx, count and out must not be NULL");
  if ((st = check_aligned16("q and out", {q, out})) != RESA_OK) return st;
  if (!aligned(idx, 4) || !aligned(count, 4)) return fail(RESA_ERR_INVALID, "idx and count must be 4-byte aligned");
  if (n_cap < 1 || n_cap > v.maxb) return fail(RESA_ERR_INVALID, "n_cap %d outside 1 .. max_blocks_per_seq", n_cap);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RESA_ERR_INVALID, "scale must be positive and finite");
  const size_t need = resa::decode_ws_bytes(v, n_cap);
  if (need > kNoAllocScratchBytes)
    return fail(RESA_ERR_UNSUPPORTED, "the decode needs %zu bytes of scratch; resa_sparse_decode_noalloc holds %zu",
                need, kNoAllocScratchBytes);
  int dev = -1;
  if ((st = current_device(&dev)) != RESA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s) {
    hipDevice_t sdev = -1;
    const hipError_t e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(RESA_ERR_INVALID, "stream belongs to device %d but device %d is current", int(sdev), dev);
  }
  void* ws = nullptr;
  if ((st = symbol_on_device(HIP_SYMBOL(scratch), "scratch", g_scratch_ptr, dev, &ws)) != RESA_OK) return st;
  RESA_DEBUG_ATTACH(v);
  return RESA_DEBUG_COLLECT(
      hip_status(resa::launch_decode(v, q, idx, count, n_cap, scale, out, ws, s), "resa_sparse_decode_noalloc"), s, v);
}

resa_status resa_rectify(const resa_cache* cache, const void* q, const void* k_new, const void* v_new,
                         int32_t f, float scale, void* out, void* ws, size_t ws_bytes, void* stream) {
  resa::CacheView v;
  resa_status st = check_cache(cache, &v);
  if (st != RESA_OK) return st;
  if (!q || !k_new || !v_new || !out) return fail(RESA_ERR_INVALID, "q, k_new, v_new and out must not be NULL");
  if ((st = check_aligned16("q, k_new, v_new, out and ws", {q, k_new, v_new, out, ws})) != RESA_OK) return st;
  if (f < 1 || f > resa::kMaxRectF) return fail(RESA_ERR_UNSUPPORTED, "f %d outside 1 .. %d", f, resa::kMaxRectF);
  if (f > v.max_seq_len) return fail(RESA_ERR_INVALID, "f %d exceeds max_seq_len %d", f, v.max_seq_len);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(RESA_ERR_INVALID, "scale must be positive and finite");
  const size_t need = resa::rectify_ws_bytes(v, f);
  if (!ws || ws_bytes < need) return fail(RESA_ERR_WORKSPACE, "rectify workspace %zu < %zu bytes", ws_bytes, need);
  // the write and refresh come first: rectified rows attend to the rectified
  // K/V of earlier rows
  RESA_DEBUG_ATTACH(v);
  return RESA_DEBUG_COLLECT(
      hip_status(resa::launch_rectify(v, q, k_new, v_new, f, scale, out, ws, static_cast<hipStream_t>(stream)),
                 "resa_rectify"),
      static_cast<hipStream_t>(stream), v);
}

const char* resa_last_error(void) { return g_err; }

}  // extern "C"
