// Block-sparse decoding over the selected blocks (Eq. 2 of the paper as the Pith
// review's referee report, minor comment 3, restates it: a key is attended iff
// its 16-token block is selected), split over the key axis in the manner of
// Flash-Decoding (reference [6] of the Pith reference list), then merged exactly.
//
// k_decode_split: one wave per (sequence, KV head, split). The wave streams one
// selected block (16 tokens x head_dim of K and of V, 4 KiB each at d=128 bf16)
// per iteration and serves all G query heads of the group from it, so each
// selected byte is fetched once per group. Lane layout: lane = 8 * tp + cg; the
// lane holds tokens tp and tp + 8 and channels cg*8 + 64*k + [0, 8), so every
// 16-byte load instruction of the wave covers 8 full 128-byte lines. q.k uses
// v_dot2 on packed bf16 pairs (fp32 accumulate), then a 3-step DPP sum over the
// 8 lanes sharing the tokens. Each group of 8 lanes keeps its own online-softmax
// state (running max m, sum l, unnormalised accumulator) over its tokens, so no
// cross-lane max is needed per block; m is only moved up when a new logit
// exceeds it by more than 2^8 (the result is unchanged: numerator and
// denominator share every rescale). At the end the 8 states are merged with
// log-sum-exp weights and written to the workspace as (m, l, acc[d]) in fp32.
//
// k_decode_combine: one wave per (sequence, query head) merges the live splits.
#include "resa_internal.h"

namespace resa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units

template <typename T, int D>
struct TokenRow;  // one lane's D/8 channels of one token row

template <int D>
struct TokenRow<uint16_t, D> {
  static constexpr int NCH = D / 64;  // 16-byte chunks per lane
  uint4 u[NCH];
  __device__ void load(const uint16_t* row, int cg) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) u[k] = *reinterpret_cast<const uint4*>(row + cg * 8 + 64 * k);
  }
  __device__ void zero() {
#pragma unroll
    for (int k = 0; k < NCH; ++k) u[k] = make_uint4(0, 0, 0, 0);
  }
  __device__ float get(int i) const {  // channel i of the lane's 8*NCH
    const uint4 w = u[i / 8];
    const uint32_t x = (i % 8) < 2 ? w.x : (i % 8) < 4 ? w.y : (i % 8) < 6 ? w.z : w.w;
    return (i & 1) ? bf16_hi(x) : bf16_lo(x);
  }
};

template <int D>
struct TokenRow<float, D> {
  static constexpr int NCH = D / 64;
  float4 u[NCH][2];
  __device__ void load(const float* row, int cg) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const float4* p = reinterpret_cast<const float4*>(row + cg * 8 + 64 * k);
      u[k][0] = p[0];
      u[k][1] = p[1];
    }
  }
  __device__ void zero() {
#pragma unroll
    for (int k = 0; k < NCH; ++k) u[k][0] = u[k][1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ float get(int i) const {
    const float4 w = u[i / 8][(i % 8) / 4];
    const int r = i % 4;
    return r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w;
  }
};

// The query of one head, restricted to the lane's channels.
template <typename T, int D>
struct QRow;
template <int D>
struct QRow<uint16_t, D> {
  static constexpr int NCH = D / 64;
  uint32_t w[NCH * 4];
  __device__ void load(const uint16_t* row, int cg) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + cg * 8 + 64 * k);
      w[4 * k + 0] = u.x; w[4 * k + 1] = u.y; w[4 * k + 2] = u.z; w[4 * k + 3] = u.w;
    }
  }
  __device__ float dot(const TokenRow<uint16_t, D>& kr) const {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const uint32_t kk[4] = {kr.u[k].x, kr.u[k].y, kr.u[k].z, kr.u[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[4 * k + i]),
                                            __builtin_bit_cast(bf16x2_t, kk[i]), s, false);
    }
    return s;
  }
};
template <int D>
struct QRow<float, D> {
  static constexpr int NC = D / 8;
  float w[NC];
  __device__ void load(const float* row, int cg) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const float4* p = reinterpret_cast<const float4*>(row + cg * 8 + 64 * k);
      const float4 a = p[0], b = p[1];
      w[8 * k + 0] = a.x; w[8 * k + 1] = a.y; w[8 * k + 2] = a.z; w[8 * k + 3] = a.w;
      w[8 * k + 4] = b.x; w[8 * k + 5] = b.y; w[8 * k + 6] = b.z; w[8 * k + 7] = b.w;
    }
  }
  __device__ float dot(const TokenRow<float, D>& kr) const {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) s = fmaf(w[i], kr.get(i), s);
    return s;
  }
};

struct DecodeArgs {
  CacheView c;
  const void* q;
  const int32_t* idx;
  const int32_t* count;
  int n_cap, bps, splits;
  float scale_log2;
  float* part_ml;   // [B][Hq][splits][2]
  float* part_acc;  // [B][Hq][splits][D]
};

// grid: x = split, y = KV head, z = sequence; 64 threads.
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void k_decode_split(DecodeArgs a) {
  constexpr int NC = D / 8;  // channels per lane
  const CacheView& c = a.c;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, tp = lane >> 3, cg = lane & 7;
  const int n = a.count[b];
  const int first = s * a.bps;
  const int nblk = min(a.bps, n - first);
  if (nblk <= 0) return;
  const int L = c.seq_lens[b];

  QRow<T, D> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(static_cast<const T*>(a.q) + (size_t(b) * c.Hq + size_t(g) * G + h) * D, cg);

  int my_blk = 0, my_page = 0;
  if (lane < nblk) {
    my_blk = a.idx[(size_t(b) * c.Hkv + g) * a.n_cap + first + lane];
    my_page = c.bt[size_t(b) * c.maxb + my_blk];
  }

  float m[G], l[G], acc[G][NC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -__builtin_inff();
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[h][i] = 0.f;
  }

  const T* kbase = static_cast<const T*>(c.k);
  const T* vbase = static_cast<const T*>(c.v);
  auto row_ptr = [&](const T* base, int page, int t) {
    return base + ((size_t(page) * c.Hkv + g) * kBlock + t) * D;
  };

  TokenRow<T, D> k0, k1, v0, v1, nk0, nk1, nv0, nv1;
  {
    const int page = __builtin_amdgcn_readlane(my_page, 0);
    k0.load(row_ptr(kbase, page, tp), cg);
    k1.load(row_ptr(kbase, page, tp + 8), cg);
    v0.load(row_ptr(vbase, page, tp), cg);
    v1.load(row_ptr(vbase, page, tp + 8), cg);
  }
  for (int it = 0; it < nblk; ++it) {
    const int blk = __builtin_amdgcn_readlane(my_blk, it);
    if (it + 1 < nblk) {  // prefetch the next block
      const int np = __builtin_amdgcn_readlane(my_page, it + 1);
      nk0.load(row_ptr(kbase, np, tp), cg);
      nk1.load(row_ptr(kbase, np, tp + 8), cg);
      nv0.load(row_ptr(vbase, np, tp), cg);
      nv1.load(row_ptr(vbase, np, tp + 8), cg);
    }
    const int valid = min(kBlock, L - blk * kBlock);
    const bool ok0 = tp < valid, ok1 = tp + 8 < valid;
    if (!ok0) { k0.zero(); v0.zero(); }
    if (!ok1) { k1.zero(); v1.zero(); }

    float x0[G], x1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      x0[h] = sum8(qr[h].dot(k0)) * a.scale_log2;
      x1[h] = sum8(qr[h].dot(k1)) * a.scale_log2;
      if (!ok0) x0[h] = -__builtin_inff();
      if (!ok1) x1[h] = -__builtin_inff();
    }
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) need |= fmaxf(x0[h], x1[h]) > m[h] + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float cand = fmaxf(x0[h], x1[h]);
        if (cand > m[h] + kLazyRescale) {
          const float alpha = m[h] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m[h] - cand);
          l[h] *= alpha;
#pragma unroll
          for (int i = 0; i < NC; ++i) acc[h][i] *= alpha;
          m[h] = cand;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p0 = ok0 ? __builtin_amdgcn_exp2f(x0[h] - m[h]) : 0.f;
      const float p1 = ok1 ? __builtin_amdgcn_exp2f(x1[h] - m[h]) : 0.f;
      l[h] += p0 + p1;
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[h][i] = fmaf(p0, v0.get(i), fmaf(p1, v1.get(i), acc[h][i]));
    }
    if (it + 1 < nblk) {
      k0 = nk0; k1 = nk1; v0 = nv0; v1 = nv1;
    }
  }

  // merge the 8 token-pair states (lanes differing in bits 3..5)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mm = m[h];
    mm = fmaxf(mm, __shfl_xor(mm, 8, 64));
    mm = fmaxf(mm, __shfl_xor(mm, 16, 64));
    mm = fmaxf(mm, __shfl_xor(mm, 32, 64));
    const float alpha = m[h] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m[h] - mm);
    float ll = l[h] * alpha;
    ll += __shfl_xor(ll, 8, 64);
    ll += __shfl_xor(ll, 16, 64);
    ll += __shfl_xor(ll, 32, 64);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      float v = acc[h][i] * alpha;
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[h][i] = v;
    }
    const size_t slot = (size_t(b) * c.Hq + size_t(g) * G + h) * a.splits + s;
    if (tp == h % 8) {
      float* dst = a.part_acc + slot * D;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        float4* p = reinterpret_cast<float4*>(dst + cg * 8 + 64 * k);
        p[0] = make_float4(acc[h][8 * k + 0], acc[h][8 * k + 1], acc[h][8 * k + 2], acc[h][8 * k + 3]);
        p[1] = make_float4(acc[h][8 * k + 4], acc[h][8 * k + 5], acc[h][8 * k + 6], acc[h][8 * k + 7]);
      }
      if (cg == 0) {
        a.part_ml[slot * 2 + 0] = mm;
        a.part_ml[slot * 2 + 1] = ll;
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t i, float x) {
  if constexpr (sizeof(T) == 2) static_cast<uint16_t*>(out)[i] = f32_to_bf16(x);
  else static_cast<float*>(out)[i] = x;
}

// grid: x = query head, y = sequence; 64 threads.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_decode_combine(const float* __restrict__ part_ml,
                                                       const float* __restrict__ part_acc,
                                                       const int32_t* __restrict__ count, int Hq,
                                                       int bps, int splits, void* __restrict__ out) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int live = (count[b] + bps - 1) / bps;
  const size_t slot0 = (size_t(b) * Hq + h) * splits;
  float mx = -__builtin_inff();
  for (int s = lane; s < live; s += 64) mx = fmaxf(mx, part_ml[(slot0 + s) * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float num[D / 64], den = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) num[e] = 0.f;
  for (int s = 0; s < live; ++s) {
    const float ms = part_ml[(slot0 + s) * 2];
    const float w = ms == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
    den = fmaf(w, part_ml[(slot0 + s) * 2 + 1], den);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) num[e] = fmaf(w, part_acc[(slot0 + s) * D + lane + 64 * e], num[e]);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < D / 64; ++e)
    store_out<T>(out, (size_t(b) * Hq + h) * D + lane + 64 * e, num[e] * inv);
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, void* out, hipStream_t st) {
  const CacheView& c = a.c;
  dim3 g1(a.splits, c.Hkv, c.B);
  hipLaunchKernelGGL((k_decode_split<T, D, G>), g1, dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(c.Hq, c.B);
  hipLaunchKernelGGL((k_decode_combine<T, D>), g2, dim3(64), 0, st, a.part_ml, a.part_acc, a.count, c.Hq,
                     a.bps, a.splits, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_g(const DecodeArgs& a, void* out, hipStream_t st) {
  switch (a.c.G) {
    case 1: return launch_decode_t<T, D, 1>(a, out, st);
    case 2: return launch_decode_t<T, D, 2>(a, out, st);
    case 4: return launch_decode_t<T, D, 4>(a, out, st);
    default: return launch_decode_t<T, D, 8>(a, out, st);
  }
}

}  // namespace

DecodePlan plan_decode(const CacheView& c, int n_cap) {
  // Aim for ~2048 single-wave workgroups (8 per CU) so the gathered loads of
  // all CUs overlap; a split holds 4..64 blocks (one block id per lane).
  const long work = long(c.B) * c.Hkv * n_cap;
  int bps = int((work + 2047) / 2048);
  bps = bps < 4 ? 4 : (bps > 64 ? 64 : bps);
  DecodePlan p;
  p.bps = bps;
  p.splits = (n_cap + bps - 1) / bps;
  return p;
}

size_t decode_ws_bytes(const CacheView& c, int n_cap) {
  const DecodePlan p = plan_decode(c, n_cap);
  const size_t slots = size_t(c.B) * c.Hq * p.splits;
  return align_up(slots * 2 * sizeof(float), 256) + slots * c.D * sizeof(float);
}

hipError_t launch_decode(const CacheView& c, const void* q, const int32_t* idx, const int32_t* count,
                         int n_cap, float scale, void* out, void* ws, hipStream_t st) {
  const DecodePlan p = plan_decode(c, n_cap);
  const size_t slots = size_t(c.B) * c.Hq * p.splits;
  DecodeArgs a;
  a.c = c;
  a.q = q;
  a.idx = idx;
  a.count = count;
  a.n_cap = n_cap;
  a.bps = p.bps;
  a.splits = p.splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.part_ml = static_cast<float*>(ws);
  a.part_acc = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(slots * 2 * sizeof(float), 256));
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_decode_g<uint16_t, 128>(a, out, st) : launch_decode_g<uint16_t, 64>(a, out, st);
  return c.D == 128 ? launch_decode_g<float, 128>(a, out, st) : launch_decode_g<float, 64>(a, out, st);
}

}  // namespace resa
