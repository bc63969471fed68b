// Block descriptor refresh as a device routine, shared by the descriptor
// kernel and the selection kernel's fused append: per block of 16 tokens and
// per KV head, the channel-wise min and max of the keys over the block's valid
// tokens (the Quest-style block statistics of the Pith review of "Rectified
// Sparse Attention", section "What carries the argument"). Exact: min/max never
// round, so the stored values are keys from the cache.
#pragma once

#include "resa_internal.h"

namespace resa {

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

// One wave (64 lanes) refreshes block j of sequence b, KV head g, whose
// sequence holds L tokens. Rows of the range [L - n_new, L) come from k_new /
// v_new ([B][n_new][Hkv][D]) when those are given, are stored into the page
// first (K token-major, V channel-major) and enter the min/max directly. A
// token row is read by the 64 lanes in one coalesced access (a lane owns D/64
// channels); all 16 rows are loaded unconditionally (slots past the end re-read
// slot 0 and are ignored) so they are in flight together.
template <typename T, int D>
__device__ __forceinline__ void refresh_block(const CacheView& c, const void* __restrict__ k_new,
                                              const void* __restrict__ v_new, int n_new, int b, int g, int j,
                                              int L, int lane) {
  constexpr int CPL = D / 64;  // channels per lane
  const int lo = n_new > 0 ? max(0, L - n_new) : 0;
  const int page = c.bt[size_t(b) * c.maxb + j];
  const int valid = min(kBlock, L - j * kBlock);
  const size_t row0 = (size_t(page) * c.Hkv + g) * kBlock;  // token-row index of slot 0

  float mn[CPL], mx[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
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

}  // namespace resa
