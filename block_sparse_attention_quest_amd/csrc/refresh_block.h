// Block descriptor refresh as a device routine, shared by the descriptor
// kernel and the selection kernel's fused append: per block of 16 tokens and
// per KV head, the channel-wise min and max of the keys over the block's valid
// tokens (the Quest-style block statistics of the Pith review of "Rectified
// Sparse Attention", section "What carries the argument"). Exact: min/max never
// round, so the stored values are keys from the cache.
#pragma once

#include "resa_internal.h"

namespace resa {

// A lane's CPL consecutive elements of a row, as one vector access (the row
// offset i is a multiple of CPL).
template <typename T, int CPL>
struct Elem;
template <int CPL>
struct Elem<float, CPL> {
  typedef float vec __attribute__((ext_vector_type(CPL)));
  __device__ static void load(const void* p, size_t i, float* x) {
    const vec v = *reinterpret_cast<const vec*>(static_cast<const float*>(p) + i);
#pragma unroll
    for (int e = 0; e < CPL; ++e) x[e] = v[e];
  }
  __device__ static void store(void* p, size_t i, const float* x) {
    vec v;
#pragma unroll
    for (int e = 0; e < CPL; ++e) v[e] = x[e];
    *reinterpret_cast<vec*>(static_cast<float*>(p) + i) = v;
  }
  __device__ static void store1(void* p, size_t i, float x) { static_cast<float*>(p)[i] = x; }
};
template <int CPL>
struct Elem<uint16_t, CPL> {  // bf16 bits
  typedef uint16_t vec __attribute__((ext_vector_type(CPL)));
  __device__ static void load(const void* p, size_t i, float* x) {
    const vec v = *reinterpret_cast<const vec*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int e = 0; e < CPL; ++e) x[e] = bf16_to_f32(v[e]);
  }
  // Only ever stores values that came from bf16, so the conversion is exact.
  __device__ static void store(void* p, size_t i, const float* x) {
    vec v;
#pragma unroll
    for (int e = 0; e < CPL; ++e) v[e] = uint16_t(__float_as_uint(x[e]) >> 16);
    *reinterpret_cast<vec*>(static_cast<uint16_t*>(p) + i) = v;
  }
  __device__ static void store1(void* p, size_t i, float x) {
    static_cast<uint16_t*>(p)[i] = uint16_t(__float_as_uint(x) >> 16);
  }
};

// One wave (64 lanes) refreshes block j of sequence b, KV head g, whose
// sequence holds L tokens. Rows of the range [L - n_new, L) come from k_new /
// v_new ([B][n_new][Hkv][D]) when those are given, are stored into the page
// (K token-major, V channel-major) and enter the min/max directly; only older
// rows are read from the page. A lane owns D/64 consecutive channels, so a
// token row is one coalesced access of the wave. Every row load of the block
// is issued before any is used: slots past the end read slot 0's source again
// (a repeat leaves min and max unchanged), and the V rows are consumed by an
// empty asm statement ahead of the stores so that the compiler cannot move
// each row's load next to its conditional store.
// NEW = false builds the variant that never takes rows from k_new (the caller
// passes none), which keeps the per-row V registers out of it.
template <typename T, int D, bool NEW = true>
__device__ __forceinline__ void refresh_block(const CacheView& c, const void* __restrict__ k_new,
                                              const void* __restrict__ v_new, int n_new, int b, int g, int j,
                                              int L, int lane) {
  constexpr int CPL = D / 64;  // channels per lane
  typedef Elem<T, CPL> E;
  const int c0 = lane * CPL;
  const bool has_new = NEW && n_new > 0 && k_new != nullptr;
  const int lo = n_new > 0 ? max(0, L - n_new) : 0;
  const int page = checked_page(c, b, j);
  const int valid = min(kBlock, L - j * kBlock);
  const size_t row0 = (size_t(page) * c.Hkv + g) * kBlock;  // token-row index of slot 0
  const int first_new = has_new ? lo - j * kBlock : kBlock;  // slot of the first fresh row
  // new-token row of slot t (clamped into the sequence's rows of k_new)
  auto new_row = [&](int t) {
    const int i = min(max(j * kBlock + t - (L - n_new), 0), n_new - 1);
    return (size_t(b) * n_new + i) * c.Hkv + g;
  };

  float kv[kBlock][CPL], vv[kBlock][CPL];
#pragma unroll
  for (int t = 0; t < kBlock; ++t) {
    const int tt = t < valid ? t : 0;
    if (tt >= first_new)
      E::load(k_new, new_row(tt) * D + c0, kv[t]);
    else
      E::load(c.k, (row0 + tt) * D + c0, kv[t]);
  }
  if (has_new) {
#pragma unroll
    for (int t = 0; t < kBlock; ++t) E::load(v_new, new_row(t) * D + c0, vv[t]);
#pragma unroll
    for (int t = 0; t < kBlock; ++t)
#pragma unroll
      for (int e = 0; e < CPL; ++e) asm volatile("" ::"v"(vv[t][e]));
  }
  float mn[CPL], mx[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    mn[e] = kv[0][e];
    mx[e] = kv[0][e];
  }
#pragma unroll
  for (int t = 1; t < kBlock; ++t)
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      mn[e] = fminf(mn[e], kv[t][e]);
      mx[e] = fmaxf(mx[e], kv[t][e]);
    }
  if (has_new) {
#pragma unroll
    for (int t = 0; t < kBlock; ++t) {
      if (t < first_new || t >= valid) continue;
      E::store(c.kw, (row0 + t) * D + c0, kv[t]);
      // V tiles are channel-major: [page][head][channel][slot]
#pragma unroll
      for (int e = 0; e < CPL; ++e) E::store1(c.vw, row0 * D + size_t(c0 + e) * kBlock + t, vv[t][e]);
    }
  }
  const size_t d0 = (size_t(page) * c.Hkv + g) * 2 * D;
  E::store(c.desc, d0 + c0, mn);
  E::store(c.desc, d0 + D + c0, mx);
}

}  // namespace resa
