// Dense rectification attention (Pith review of "Rectified Sparse Attention",
// "What carries the argument" and "The reading"): after the f newest positions
// of every sequence have been overwritten with their re-encoded K/V (done by the
// descriptor kernel on the same stream), row i of every query head attends
// causally over the whole cache, positions 0 .. L - f + i.
//
// bf16 path (k_rect_mfma): per KV head the G * f query rows form one dense
// contraction against every key, so it runs on the matrix cores
// (v_mfma_f32_32x32x16_bf16). One workgroup of 4 waves takes one (sequence, KV
// head, key chunk); the K/V of the chunk are fetched once per group from HBM
// into LDS in tiles of 32 keys and shared by all G * f rows (so HBM traffic is
// the cache once per event, not once per head). Each wave owns 32-row tiles of
// queries, kept in registers. Scores are computed transposed, S^T = K Q^T, so a
// lane holds 16 keys of one query row: the softmax row max needs one cross-lane
// step, and the probabilities feed the second product O^T = V^T P^T as its B
// operand with no data movement (the key order inside a 16-key step is the same
// permutation on both operands). V pages are channel-major in HBM, so the V^T
// tile for the A operand is copied into LDS with plain 16-byte stores. Partial (m, l, O) per row and chunk go to the workspace; a combine
// kernel merges the chunks with log-sum-exp weights.
//
// fp32 path (k_rect_valu): one wave per (sequence, row, head), plain VALU.
#include "resa_internal.h"

namespace resa {
namespace {

struct RectArgs {
  CacheView c;
  const void* q;  // [B][f][Hq][D]
  int f, rows, rows_pad, chunk, splits;
  float scale_log2;
  float* part_ml;   // [B][Hkv][splits][rows_pad][2]
  float* part_acc;  // [B][Hkv][splits][rows_pad][D]
};

template <int D>
struct RectSmem {
  static constexpr int KS = D + 8;               // K row stride (elements)
  static constexpr int VS = kRectTileKeys + 8;   // V^T row stride (elements)
  uint16_t k[kRectTileKeys * KS];
  uint16_t vt[D * VS];
};

// grid: x = key chunk, y = KV head, z = sequence; 256 threads.
template <int D, int TPW>
__global__ __launch_bounds__(256) void k_rect_mfma(RectArgs a) {
  constexpr int KSTEPS = D / 16;   // 16-deep k-steps of the score product
  constexpr int DT = D / 32;       // 32-wide output column tiles
  constexpr int EPT = D / 8;       // elements per thread of a tile row load
  __shared__ RectSmem<D> sm;
  const CacheView& c = a.c;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = c.seq_lens[b];
  const int key_lo = s * a.chunk;
  if (key_lo >= L) return;
  const int key_hi = min(L, key_lo + a.chunk);
  const int G = c.G;
  const int col = lane & 31, half = lane >> 5;

  // query rows of this lane (one per owned row tile), as MFMA B operands
  bf16x8_t qreg[TPW][KSTEPS];
  int limit[TPW];  // last key position the row may see (-1: padding row)
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int r = (wave + 4 * u) * 32 + col;
    const bool live = r < a.rows;
    const int i = r / G, h = r % G;
    limit[u] = live ? L - a.f + i : -1;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((size_t(b) * a.f + i) * c.Hq + size_t(g) * G + h) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (live) w = *reinterpret_cast<const uint4*>(qrow + ks * 16 + 8 * half);
      qreg[u][ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  f32x16_t o[TPW][DT];
  float m[TPW], lsum[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    m[u] = -__builtin_inff();
    lsum[u] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u][t][r] = 0.f;
  }

  const uint16_t* kb = static_cast<const uint16_t*>(c.k);
  const uint16_t* vb = static_cast<const uint16_t*>(c.v);
  // K: thread -> (key lk, columns lc .. lc + EPT) of the token-major K rows.
  // V: the page tiles are channel-major (d x 16 tokens); thread -> 16-byte
  // pieces u = tid + 256 e: page pg of the tile, channel ch, 8 tokens at 8 vh.
  const int lk = tid / 8;
  const int lc = (tid % 8) * EPT;
  uint4 kreg[EPT / 8], vreg[EPT / 8];
  // Keys past the chunk end are read from the chunk's first key (always valid)
  // and zeroed, so uninitialised slots never reach the products.
  auto load_tile = [&](int base) {
    {
      const int key = base + lk;
      const bool ok = key < key_hi;
      const int kk = ok ? key : key_lo;
      const int page = c.bt[size_t(b) * c.maxb + (kk >> 4)];
      const size_t off = ((size_t(page) * c.Hkv + g) * kBlock + (kk & 15)) * D + lc;
      const uint32_t keep = ok ? 0xffffffffu : 0u;
#pragma unroll
      for (int e = 0; e < EPT / 8; ++e) {
        const uint4 kv = *reinterpret_cast<const uint4*>(kb + off + 8 * e);
        kreg[e] = make_uint4(kv.x & keep, kv.y & keep, kv.z & keep, kv.w & keep);
      }
    }
#pragma unroll
    for (int e = 0; e < EPT / 8; ++e) {
      const int u = tid + 256 * e;
      const int pg = u / (2 * D), ch = (u % (2 * D)) / 2, vh = u % 2;
      const int t0 = base + pg * 16 + vh * 8;  // key of the first of the 8 tokens
      const int kk = t0 < key_hi ? t0 : key_lo;
      const int page = c.bt[size_t(b) * c.maxb + (kk >> 4)];
      const size_t off = ((size_t(page) * c.Hkv + g) * D + ch) * kBlock + (t0 < key_hi ? vh * 8 : 0);
      uint4 vv = *reinterpret_cast<const uint4*>(vb + off);
      const int nvalid = key_hi - t0;  // tokens of the 8 that exist
      if (nvalid < 8) {
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
        uint32_t o[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          o[x] = w[x] & ((2 * x < nvalid ? 0x0000ffffu : 0u) | (2 * x + 1 < nvalid ? 0xffff0000u : 0u));
        vv = make_uint4(o[0], o[1], o[2], o[3]);
      }
      vreg[e] = vv;
    }
  };

  load_tile(key_lo);
  for (int base = key_lo; base < key_hi; base += kRectTileKeys) {
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int e = 0; e < EPT / 8; ++e) {
      *reinterpret_cast<uint4*>(&sm.k[lk * RectSmem<D>::KS + lc + 8 * e]) = kreg[e];
      const int u = tid + 256 * e;
      const int pg = u / (2 * D), ch = (u % (2 * D)) / 2, vh = u % 2;
      *reinterpret_cast<uint4*>(&sm.vt[ch * RectSmem<D>::VS + pg * 16 + vh * 8]) = vreg[e];
    }
    __syncthreads();
    if (base + kRectTileKeys < key_hi) load_tile(base + kRectTileKeys);

#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if ((wave + 4 * u) * 32 >= a.rows) continue;  // wave-uniform
      f32x16_t sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8_t ak =
            *reinterpret_cast<const bf16x8_t*>(&sm.k[col * RectSmem<D>::KS + ks * 16 + 8 * half]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[u][ks], sacc, 0, 0, 0);
      }
      // lane holds keys 8*(r/4) + 4*half + r%4 of query row `col`
      float x[16];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = base + 8 * (r / 4) + 4 * half + (r % 4);
        x[r] = (key < key_hi && key <= limit[u]) ? sacc[r] * a.scale_log2 : -__builtin_inff();
        tmax = fmaxf(tmax, x[r]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m[u], tmax);
      const float alpha = mnew == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m[u] - mnew);
      float p[16];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = x[r] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(x[r] - mnew);
        psum += p[r];
      }
      lsum[u] = lsum[u] * alpha + psum;
      m[u] = mnew;
      bf16x8_t pb[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint32_t w[4];
#pragma unroll
        for (int x2 = 0; x2 < 4; ++x2)
          w[x2] = uint32_t(f32_to_bf16(p[8 * k2 + 2 * x2])) | (uint32_t(f32_to_bf16(p[8 * k2 + 2 * x2 + 1])) << 16);
        pb[k2] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        o[u][t] *= alpha;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const uint16_t* vrow = &sm.vt[(t * 32 + col) * RectSmem<D>::VS + k2 * 16 + 4 * half];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[u][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[k2], o[u][t], 0, 0, 0);
        }
      }
    }
  }

  // write partials: lane holds O^T[dcol][row col] for dcol = 32t + 8(r/4) + 4 half + r%4
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int rt = wave + 4 * u;
    if (rt * 32 >= a.rows) continue;
    const int r = rt * 32 + col;
    const float ltot = lsum[u] + __shfl_xor(lsum[u], 32, 64);
    const size_t slot = ((size_t(b) * c.Hkv + g) * a.splits + s) * a.rows_pad + r;
    if (half == 0) {
      a.part_ml[slot * 2 + 0] = m[u];
      a.part_ml[slot * 2 + 1] = ltot;
    }
    float* dst = a.part_acc + slot * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(dst + t * 32 + 8 * q4 + 4 * half) =
            make_float4(o[u][t][4 * q4 + 0], o[u][t][4 * q4 + 1], o[u][t][4 * q4 + 2], o[u][t][4 * q4 + 3]);
  }
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t i, float x) {
  if constexpr (sizeof(T) == 2) static_cast<uint16_t*>(out)[i] = f32_to_bf16(x);
  else static_cast<float*>(out)[i] = x;
}

template <typename T>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Merge the key chunks of every query row. grid: x = row group of 4, y = KV
// head, z = sequence; 256 threads, one wave per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_rect_combine(RectArgs a, void* __restrict__ out) {
  const CacheView& c = a.c;
  const int b = blockIdx.z, g = blockIdx.y, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  const int L = c.seq_lens[b];
  const int live = (L + a.chunk - 1) / a.chunk;
  const size_t base = (size_t(b) * c.Hkv + g) * a.splits;
  float mx = -__builtin_inff();
  for (int s = lane; s < live; s += 64) mx = fmaxf(mx, a.part_ml[((base + s) * a.rows_pad + r) * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float num[D / 64], den = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) num[e] = 0.f;
  for (int s = 0; s < live; ++s) {
    const size_t slot = (base + s) * a.rows_pad + r;
    const float ms = a.part_ml[slot * 2];
    const float w = ms == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
    den = fmaf(w, a.part_ml[slot * 2 + 1], den);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) num[e] = fmaf(w, a.part_acc[slot * D + lane + 64 * e], num[e]);
  }
  const int i = r / c.G, h = r % c.G;
  const float inv = 1.f / den;
  const size_t o0 = ((size_t(b) * a.f + i) * c.Hq + size_t(g) * c.G + h) * D;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) store_out<T>(out, o0 + lane + 64 * e, num[e] * inv);
}

// Plain VALU causal attention for the fp32 cache: one wave per (row, head).
// grid: x = query head, y = row i, z = sequence; 64 threads.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_rect_valu(RectArgs a, void* __restrict__ out) {
  const CacheView& c = a.c;
  const int h = blockIdx.x, i = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int g = h / c.G;
  const int L = c.seq_lens[b];
  const int P = L - a.f + i;  // last visible position
  __shared__ float qs[D];
  __shared__ float ps[64];
  const size_t qo = ((size_t(b) * a.f + i) * c.Hq + h) * D;
  for (int ch = lane; ch < D; ch += 64) qs[ch] = load_elem<T>(a.q, qo + ch);
  __syncthreads();
  float m = -__builtin_inff(), l = 0.f, acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  for (int t0 = 0; t0 <= P; t0 += 64) {
    const int t = t0 + lane;
    float x = -__builtin_inff();
    if (t <= P) {
      const int page = c.bt[size_t(b) * c.maxb + (t >> 4)];
      const size_t row = ((size_t(page) * c.Hkv + g) * kBlock + (t & 15)) * D;
      float sdot = 0.f;
      for (int ch = 0; ch < D; ++ch) sdot = fmaf(qs[ch], load_elem<T>(c.k, row + ch), sdot);
      x = sdot * a.scale_log2;
    }
    float tmax = x;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
    const float mnew = fmaxf(m, tmax);
    const float alpha = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
    const float p = t <= P ? __builtin_amdgcn_exp2f(x - mnew) : 0.f;
    float psum = p;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) psum += __shfl_xor(psum, o, 64);
    l = l * alpha + psum;
    m = mnew;
    __syncthreads();
    ps[lane] = p;
    __syncthreads();
    const int nt = min(64, P + 1 - t0);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] *= alpha;
    for (int k = 0; k < nt; ++k) {
      const int tt = t0 + k;
      const int page = c.bt[size_t(b) * c.maxb + (tt >> 4)];
      const size_t vt = (size_t(page) * c.Hkv + g) * D * kBlock + (tt & 15);  // channel-major V tile
#pragma unroll
      for (int e = 0; e < D / 64; ++e)
        acc[e] = fmaf(ps[k], load_elem<T>(c.v, vt + size_t(lane + 64 * e) * kBlock), acc[e]);
    }
  }
  const size_t oo = ((size_t(b) * a.f + i) * c.Hq + h) * D;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) store_out<T>(out, oo + lane + 64 * e, acc[e] / l);
}

template <int D>
hipError_t launch_mfma(const RectArgs& a, void* out, hipStream_t st) {
  const CacheView& c = a.c;
  dim3 grid(a.splits, c.Hkv, c.B);
  const int tiles = a.rows_pad / 32;
  if (tiles <= 4)
    hipLaunchKernelGGL((k_rect_mfma<D, 1>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_rect_mfma<D, 2>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((a.rows + 3) / 4, c.Hkv, c.B);
  hipLaunchKernelGGL((k_rect_combine<uint16_t, D>), g2, dim3(256), 0, st, a, out);
  return hipGetLastError();
}

}  // namespace

RectPlan plan_rectify(const CacheView& c, int f) {
  RectPlan p;
  p.rows = c.G * f;
  p.rows_pad = (p.rows + 31) / 32 * 32;
  // ~1536 workgroups over the longest sequence; chunks are whole key tiles.
  const long keys = long(c.B) * c.Hkv * c.max_seq_len;
  long chunk = (keys + 1535) / 1536;
  chunk = (chunk + 255) / 256 * 256;
  if (chunk < 256) chunk = 256;
  if (chunk > 16384) chunk = 16384;
  p.chunk = int(chunk);
  p.splits = (c.max_seq_len + p.chunk - 1) / p.chunk;
  return p;
}

size_t rectify_ws_bytes(const CacheView& c, int f) {
  const RectPlan p = plan_rectify(c, f);
  const size_t slots = size_t(c.B) * c.Hkv * p.splits * p.rows_pad;
  return align_up(slots * 2 * sizeof(float), 256) + slots * c.D * sizeof(float);
}

hipError_t launch_rectify_attention(const CacheView& c, const void* q, int f, float scale, void* out,
                                    void* ws, hipStream_t st) {
  const RectPlan p = plan_rectify(c, f);
  RectArgs a;
  a.c = c;
  a.q = q;
  a.f = f;
  a.rows = p.rows;
  a.rows_pad = p.rows_pad;
  a.chunk = p.chunk;
  a.splits = p.splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  const size_t slots = size_t(c.B) * c.Hkv * p.splits * p.rows_pad;
  char* scratch = static_cast<char*>(ws);
  a.part_ml = reinterpret_cast<float*>(scratch);
  a.part_acc = reinterpret_cast<float*>(scratch + align_up(slots * 2 * sizeof(float), 256));
  if (c.dtype == RESA_BF16) return c.D == 128 ? launch_mfma<128>(a, out, st) : launch_mfma<64>(a, out, st);
  dim3 grid(c.Hq, f, c.B);
  if (c.D == 128)
    hipLaunchKernelGGL((k_rect_valu<float, 128>), grid, dim3(64), 0, st, a, out);
  else
    hipLaunchKernelGGL((k_rect_valu<float, 64>), grid, dim3(64), 0, st, a, out);
  return hipGetLastError();
}

}  // namespace resa
