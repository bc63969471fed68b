// Internal declarations shared by the libresa translation units: device helpers,
// kernel argument blocks and the launchers the C ABI layer calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "resa.h"

namespace resa {

constexpr int kBlock = 16;              // tokens per page = selection block
constexpr int kTopnThreads = 1024;      // one workgroup per (sequence, KV head)
constexpr int kTopnMaxPerThread = 32;   // => at most 32768 blocks per sequence
constexpr int kRectTileKeys = 32;       // keys per MFMA key tile
constexpr int kMaxRectF = 1024;
constexpr size_t kLastLevelCacheBytes = size_t(256) << 20;  // MI355X Infinity Cache
constexpr int kCachePolicyNT = 2;  // cache-policy operand of the direct-to-LDS load: non-temporal

// Workgroups are dealt to the 8 XCDs (each with its own L2) in turn by linear
// id. With a grid of NX workgroups per (sequence, KV head) pair, laid out
// (x, KV head, sequence), this remap runs every workgroup of pair gi on XCD
// gi % 8. Kernels launched over a (KV head, sequence, ...) grid run pair gi
// there too (the top-n before the decode, the merge after it), so what one
// writes the next finds in that XCD's L2. Applied when the KV heads are a
// multiple of 8: every XCD then holds one-eighth of the heads of every
// sequence, whatever the length mix. Returns the (x, KV head, sequence) the
// workgroup takes.
__device__ __forceinline__ int3 xcd_pair_remap(int x, int g, int b, int NX, int Hkv) {
  if ((Hkv & 7) != 0) return make_int3(x, g, b);
  const int i = x + NX * (g + Hkv * b);
  const int k = i >> 3, gi = (i & 7) + 8 * (k / NX);
  return make_int3(k % NX, gi % Hkv, gi / Hkv);
}

// Row stride (in keys) of the selection workspace: max_blocks_per_seq rounded
// up to even, so every row starts on 16 bytes.
__host__ __device__ constexpr int key_stride(int maxb) { return (maxb + 1) & ~1; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// DPP lane moves (CDNA encodings).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // reverse within each group of 8 lanes
constexpr int kDppRowMirror = 0x140;    // reverse within each row of 16 lanes
constexpr int kDppRowShr1 = 0x111;      // row_shr:1 (row_shr:n is 0x110 + n)
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the whole next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3

// Operand types of the direct global-to-LDS load builtin.
typedef __attribute__((address_space(1))) const void* global_ptr_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until at most N vector-memory instructions of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt(((N >> 4) & 3) << 14 | (0xF << 8) | (7 << 4) | (N & 15));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the
// same bits (each step adds a commutative pair).
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f32<kDppHalfMirror>(x);
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  return x;
}

__device__ __forceinline__ double shfl_xor_f64(double x, int m) {
  return __shfl_xor(x, m, 64);
}

// ---------------------------------------------------------------------------
// Launchers (one per kernel family; each returns hipGetLastError()).
// ---------------------------------------------------------------------------
struct CacheView {
  int dtype, B, Hq, Hkv, D, G, num_pages, maxb, max_seq_len;
  const void* k;
  const void* v;
  void* kw;   // writable aliases of k / v pages
  void* vw;
  void* desc;
  const int32_t* bt;
  const int32_t* seq_lens;
  int* dbg;   // checked builds: the device word the precondition checks set (NULL otherwise)
};

// ---------------------------------------------------------------------------
// Device-side precondition checks (built with RESA_DEBUG_CHECKS only). A
// kernel that finds a caller precondition broken sets its bit in the device
// word (c.dbg) and clamps the offending value into range, so that every access
// stays in bounds and every workgroup still reaches its barriers (the results
// are then meaningless); the entry point synchronises its stream and returns
// RESA_ERR_INVALID. Release builds compile every check away.
// ---------------------------------------------------------------------------
enum DebugCheck {
  kChkSeqLen = 1,     // seq_lens[b] outside 0 .. max_seq_len
  kChkPage = 2,       // a held block's block_table entry outside 0 .. num_pages - 1
  kChkEmpty = 4,      // seq_lens[b] < 1 where selection or decoding needs a token
  kChkSelection = 8,  // count[b] > n_cap, or a selected block outside 0 .. M_b - 1
  kChkRectF = 16,     // f > seq_lens[b] in a rectification
};
#ifdef RESA_DEBUG_CHECKS
#define RESA_CHECK(dbg, cond, bit, fix)          \
  do {                                           \
    if (!(cond)) {                               \
      atomicOr((dbg), int(bit));                 \
      fix;                                       \
    }                                            \
  } while (0)
#else
#define RESA_CHECK(dbg, cond, bit, fix) \
  do {                                  \
  } while (0)
#endif

// A sequence length read for a kernel, checked against the cache capacity.
__device__ __forceinline__ int checked_len(const CacheView& c, int b) {
  int L = c.seq_lens[b];
  RESA_CHECK(c.dbg, L >= 0 && L <= c.max_seq_len, kChkSeqLen, L = min(max(L, 0), c.max_seq_len));
  return L;
}
// A block-table entry of a held block, checked against the page pool.
__device__ __forceinline__ int checked_page(const CacheView& c, int b, int j) {
  int page = c.bt[size_t(b) * c.maxb + j];
  RESA_CHECK(c.dbg, page >= 0 && page < c.num_pages, kChkPage, page = 0);
  return page;
}

hipError_t launch_update_tail(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                              hipStream_t s);
hipError_t launch_rebuild(const CacheView& c, hipStream_t s);

size_t select_ws_bytes(const CacheView& c);
hipError_t launch_select(const CacheView& c, const void* q, const resa_select_params& p, int32_t* idx,
                         int32_t* count, int n_cap, void* ws, hipStream_t s);
hipError_t launch_append_select(const CacheView& c, const void* k_new, const void* v_new, const void* q,
                                const resa_select_params& p, int32_t* idx, int32_t* count, int n_cap, void* ws,
                                hipStream_t s);

struct DecodePlan {
  int bps;     // selected blocks per split
  int splits;  // splits per (sequence, KV head)
};
DecodePlan plan_decode(const CacheView& c, int n_cap);
size_t decode_ws_bytes(const CacheView& c, int n_cap);
hipError_t launch_decode(const CacheView& c, const void* q, const int32_t* idx, const int32_t* count,
                         int n_cap, float scale, void* out, void* ws, hipStream_t s);

struct RectPlan {
  int rows;     // G * f query rows per KV head
  int tile_rows;  // rows per row tile: 128 (4 waves) or 256 (8 waves)
  int rtiles;   // row tiles per (sequence, KV head)
  int rows_pad; // partial slots per item: the rows of one tile, rounded up to 32
  int target;   // workgroups aimed for (one round over the chip)
  int slots;    // workgroups launched: the most any plan within the capacities uses
  int cap;      // upper bound on work items
};
RectPlan plan_rectify(const CacheView& c, int f);
size_t rectify_ws_bytes(const CacheView& c, int f);
// The whole rectification: write the f rows and refresh their blocks, then the
// causal rows (the first launch also builds the bf16 path's work plan).
hipError_t launch_rectify(const CacheView& c, const void* q, const void* k_new, const void* v_new, int f,
                          float scale, void* out, void* ws, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace resa
