// Block descriptors: per block of 16 tokens and per KV head, the channel-wise
// min and max of the keys over the block's valid tokens (the Quest-style block
// statistics of the Pith review of "Rectified Sparse Attention", section "What
// carries the argument"). Exact: min/max never round, so the stored values are
// keys from the cache.
//
// One wave per (sequence, block, KV head). A token row of head_dim elements is
// read by the 64 lanes in one coalesced access (lane owns head_dim/64 channels),
// so a block costs 16 row reads of 128-512 bytes and one 2-row descriptor write.
// The same kernel performs the append: tokens in the refreshed range come from
// k_new/v_new, are stored into their page (K token-major, V channel-major), and
// enter the min/max directly.
#include "resa_internal.h"

namespace resa {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ static float load(const void* p, size_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void store(void* p, size_t i, float x) { static_cast<float*>(p)[i] = x; }
};
template <>
struct Elem<uint16_t> {  // bf16 bits
  __device__ static float load(const void* p, size_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  // Only ever stores values that came from bf16, so the conversion is exact.
  __device__ static void store(void* p, size_t i, float x) {
    static_cast<uint16_t*>(p)[i] = uint16_t(__float_as_uint(x) >> 16);
  }
};

// blockIdx: x = block slot within the refreshed range, y = KV head, z = sequence.
// n_new == 0: rebuild (slot = logical block index, nothing written).
template <typename T, int D>
__global__ __launch_bounds__(64) void k_refresh_blocks(CacheView c, const void* __restrict__ k_new,
                                                       const void* __restrict__ v_new, int n_new) {
  constexpr int CPL = D / 64;  // channels per lane
  const int b = blockIdx.z, g = blockIdx.y, lane = threadIdx.x;
  const int L = c.seq_lens[b];
  const int lo = n_new > 0 ? max(0, L - n_new) : 0;
  const int j = lo / kBlock + blockIdx.x;
  if (j * kBlock >= L) return;
  const int page = c.bt[size_t(b) * c.maxb + j];
  const int valid = min(kBlock, L - j * kBlock);
  const size_t row0 = (size_t(page) * c.Hkv + g) * kBlock;  // token-row index of slot 0

  float mn[CPL], mx[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  // All 16 rows are read with unconditional loads (slots past the end re-read
  // slot 0 and are ignored) so they are in flight together; fresh rows come
  // from k_new and are stored into the page.
  float kv[kBlock][CPL];
#pragma unroll
  for (int t = 0; t < kBlock; ++t)
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      kv[t][e] = Elem<T>::load(c.k, (row0 + (t < valid ? t : 0)) * D + lane + 64 * e);
  const int first_new = n_new > 0 && k_new != nullptr ? lo - j * kBlock : kBlock;  // slot of the first fresh row
#pragma unroll
  for (int t = 0; t < kBlock; ++t) {
    if (t >= valid) continue;
    if (t >= first_new) {
      const size_t src_row = (size_t(b) * n_new + (j * kBlock + t - (L - n_new))) * c.Hkv + g;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const int ch = lane + 64 * e;
        kv[t][e] = Elem<T>::load(k_new, src_row * D + ch);
        Elem<T>::store(c.kw, (row0 + t) * D + ch, kv[t][e]);
        // V tiles are channel-major: [page][head][channel][slot]
        Elem<T>::store(c.vw, (row0 * D + size_t(ch) * kBlock) + t, Elem<T>::load(v_new, src_row * D + ch));
      }
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      mn[e] = fminf(mn[e], kv[t][e]);
      mx[e] = fmaxf(mx[e], kv[t][e]);
    }
  }
  const size_t d0 = (size_t(page) * c.Hkv + g) * 2 * D;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const int ch = lane + 64 * e;
    Elem<T>::store(c.desc, d0 + ch, mn[e]);
    Elem<T>::store(c.desc, d0 + D + ch, mx[e]);
  }
}

template <typename T, int D>
hipError_t launch_refresh_t(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                            hipStream_t s) {
  const int slots = n_new > 0 ? (n_new + kBlock - 1) / kBlock + 1 : c.maxb;
  dim3 grid(slots, c.Hkv, c.B);
  hipLaunchKernelGGL((k_refresh_blocks<T, D>), grid, dim3(64), 0, s, c, k_new, v_new, n_new);
  return hipGetLastError();
}

hipError_t launch_refresh(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                          hipStream_t s) {
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_refresh_t<uint16_t, 128>(c, k_new, v_new, n_new, s)
                      : launch_refresh_t<uint16_t, 64>(c, k_new, v_new, n_new, s);
  return c.D == 128 ? launch_refresh_t<float, 128>(c, k_new, v_new, n_new, s)
                    : launch_refresh_t<float, 64>(c, k_new, v_new, n_new, s);
}

}  // namespace

hipError_t launch_update_tail(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                              hipStream_t s) {
  return launch_refresh(c, k_new, v_new, n_new, s);
}

hipError_t launch_rebuild(const CacheView& c, hipStream_t s) {
  return launch_refresh(c, nullptr, nullptr, 0, s);
}

}  // namespace resa
