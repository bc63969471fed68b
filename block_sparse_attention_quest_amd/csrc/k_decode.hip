// Block-sparse decoding over the selected blocks (Eq. 2 of the paper as the Pith
// review's referee report, minor comment 3, restates it: a key is attended iff
// its 16-token block is selected), split over the key axis in the manner of
// Flash-Decoding (reference [6] of the Pith reference list), then merged exactly.
//
// k_decode, grid (split, KV head, sequence), 4 waves. A split is a run of the
// group's selected blocks; wave w takes every 4th of them. Per block the wave
// reads the K tile (16 tokens x d, token-major) and the V tile (stored
// channel-major, d x 16 tokens) of one page, 4 KiB each at d = 128 bf16, and
// serves all G query heads of the group from them, so each selected byte is
// fetched once per group. Two blocks ahead are in flight while one is
// processed (three rotating register sets, so no copy ever waits on a load).
//   q.k: lane = 8 * tp + cg holds tokens tp and tp + 8 and channels
//   cg*8 + 64*k + [0, 8) of K (every 16-byte load covers whole 128-byte lines);
//   bf16 pairs go through v_dot2 with fp32 accumulation, then a 3-step DPP sum
//   over the 8 lanes that share the tokens.
//   softmax: one running max per head for the whole wave, moved only when a
//   logit exceeds it by more than 2^8 (numerator and denominator share every
//   rescale, so the result is unchanged); each of the 2G (token, head) pairs of
//   a token pair is exponentiated by one lane and published through LDS.
//   p.V: lane owns head_dim/64 channels; its V rows are 16 contiguous tokens,
//   so with bf16 the probabilities are rounded to bf16 and multiplied in token
//   pairs with v_dot2 (fp32 accumulation; the softmax denominator sums the
//   same rounded values).
// The 4 wave states are merged through LDS into one split partial (m, l,
// acc[d]) in fp32; k_decode_combine then merges a group's splits with
// log-sum-exp weights (a separate kernel, so the hand-off needs no
// device-scope fence).
#include "resa_internal.h"

namespace resa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;

// One lane's channels of one K token row.
template <typename T, int D>
struct KRow;
template <int D>
struct KRow<uint16_t, D> {
  static constexpr int NCH = D / 64;
  uint4 u[NCH];
  __device__ void load(const uint16_t* row, int cg) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) u[k] = *reinterpret_cast<const uint4*>(row + cg * 8 + 64 * k);
  }
};
template <int D>
struct KRow<float, D> {
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
  __device__ float get(int i) const {
    const float4 w = u[i / 8][(i % 8) / 4];
    const int r = i % 4;
    return r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w;
  }
};

// The query of one head restricted to the lane's K channels.
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
  __device__ float dot(const KRow<uint16_t, D>& kr) const {
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
  __device__ float dot(const KRow<float, D>& kr) const {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) s = fmaf(w[i], kr.get(i), s);
    return s;
  }
};

// One lane's V rows (channel-major page tile): CPL channels x 16 tokens.
template <typename T, int CPL>
struct VRows;
template <int CPL>
struct VRows<uint16_t, CPL> {
  uint4 u[CPL][2];  // 16 bf16 tokens per channel
  __device__ void load(const uint16_t* tile, int lane) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const uint4* p = reinterpret_cast<const uint4*>(tile + (lane * CPL + cc) * 16);
      u[cc][0] = p[0];
      u[cc][1] = p[1];
    }
  }
  __device__ float get(int cc, int t) const {
    const uint4 w = u[cc][t / 8];
    const int r = (t % 8) / 2;
    const uint32_t x = r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w;
    return (t & 1) ? bf16_hi(x) : bf16_lo(x);
  }
  __device__ static uint32_t keep2(uint32_t x, int t0, int valid) {
    return x & ((t0 < valid ? 0x0000ffffu : 0u) | (t0 + 1 < valid ? 0xffff0000u : 0u));
  }
  __device__ void mask_tokens(int valid) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4& w = u[cc][i];
        w.x = keep2(w.x, 8 * i + 0, valid);
        w.y = keep2(w.y, 8 * i + 2, valid);
        w.z = keep2(w.z, 8 * i + 4, valid);
        w.w = keep2(w.w, 8 * i + 6, valid);
      }
  }
};
template <int CPL>
struct VRows<float, CPL> {
  float4 u[CPL][4];
  __device__ void load(const float* tile, int lane) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const float4* p = reinterpret_cast<const float4*>(tile + (lane * CPL + cc) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) u[cc][i] = p[i];
    }
  }
  __device__ float get(int cc, int t) const {
    const float4 w = u[cc][t / 4];
    const int r = t % 4;
    return r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w;
  }
  __device__ void mask_tokens(int valid) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4& w = u[cc][i];
        w.x = 4 * i + 0 < valid ? w.x : 0.f;
        w.y = 4 * i + 1 < valid ? w.y : 0.f;
        w.z = 4 * i + 2 < valid ? w.z : 0.f;
        w.w = 4 * i + 3 < valid ? w.w : 0.f;
      }
  }
};

struct DecodeArgs {
  CacheView c;
  const void* q;
  const int32_t* idx;
  const int32_t* count;
  int n_cap, bps, splits;
  float scale_log2;
  float* part_ml;      // [B*Hkv][splits][G][2]
  float* part_acc;     // [B*Hkv][splits][G][D]
};

template <typename T>
__device__ __forceinline__ void store_out(void* out, size_t i, float x) {
  if constexpr (sizeof(T) == 2) static_cast<uint16_t*>(out)[i] = f32_to_bf16(x);
  else static_cast<float*>(out)[i] = x;
}

template <int G, int D>
struct DecSmem {
  float p[kDecWaves][16][G];       // fp32 cache: probabilities of the current block
  uint16_t pb[kDecWaves][G][16];   // bf16 cache: the same, rounded, token pairs adjacent
  float m[kDecWaves][G];
  float l[kDecWaves][G];
  float acc[kDecWaves][G][D];
};

// The K rows (tokens tp, tp + 8) and V rows of one block for one lane.
template <typename T, int D>
struct BlockRegs {
  KRow<T, D> k0, k1;
  VRows<T, D / 64> v;
  __device__ void load(const T* kt, const T* vt, int tp, int cg, int lane) {
    k0.load(kt + tp * D, cg);
    k1.load(kt + (tp + 8) * D, cg);
    v.load(vt, lane);
  }
};

// grid: x = split, y = KV head, z = sequence; 256 threads.
template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeArgs a) {
  constexpr int CPL = D / 64;                      // V channels per lane
  constexpr int PAIRS = 2 * G;                     // (token, head) pairs per token pair
  constexpr int PPL = PAIRS > 8 ? PAIRS / 8 : 1;   // pairs per lane
  constexpr bool BF16 = sizeof(T) == 2;
  __shared__ DecSmem<G, D> sm;
  const CacheView& c = a.c;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tp = lane >> 3, cg = lane & 7;
  const size_t gi = size_t(b) * c.Hkv + g;
  const int first = s * a.bps;

  // Block ids and page ids of this wave's blocks (first + wave + 4 i), read
  // before the count is known: indices are clamped into the idx row, the block
  // table row and the page pool, so every load is in bounds; blocks past the
  // count are never used.
  int my_blk = 0, my_page = 0;
  if (lane * kDecWaves < a.bps) {
    const int pos = min(first + wave + kDecWaves * lane, a.n_cap - 1);
    my_blk = min(max(a.idx[gi * a.n_cap + pos], 0), c.maxb - 1);
    my_page = min(max(c.bt[size_t(b) * c.maxb + my_blk], 0), c.num_pages - 1);
  }
  const int n = a.count[b];
  const int L = c.seq_lens[b];
  QRow<T, D> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(static_cast<const T*>(a.q) + (size_t(b) * c.Hq + size_t(g) * G + h) * D, cg);

  const T* kbase = static_cast<const T*>(c.k);
  const T* vbase = static_cast<const T*>(c.v);
  auto tile = [&](const T* base, int page) { return base + (size_t(page) * c.Hkv + g) * kBlock * D; };
  BlockRegs<T, D> A, B, C;
  {
    const int p0 = __builtin_amdgcn_readlane(my_page, 0);
    const int p1 = __builtin_amdgcn_readlane(my_page, 1);
    A.load(tile(kbase, p0), tile(vbase, p0), tp, cg, lane);
    B.load(tile(kbase, p1), tile(vbase, p1), tp, cg, lane);
  }
  const int nblk = min(a.bps, n - first);
  if (nblk <= 0) return;
  const int nw = nblk > wave ? (nblk - wave + kDecWaves - 1) / kDecWaves : 0;

  float m[G], lpart[PPL], acc[G][CPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -__builtin_inff();
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) acc[h][cc] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < PPL; ++u) lpart[u] = 0.f;

  // One block: q.k, online softmax, p.V. `spare` receives block it + 2.
  auto step = [&](int it, BlockRegs<T, D>& cur, BlockRegs<T, D>& spare) {
    if (it + 2 < nw) {
      const int np = __builtin_amdgcn_readlane(my_page, it + 2);
      spare.load(tile(kbase, np), tile(vbase, np), tp, cg, lane);
    }
    const int blk = __builtin_amdgcn_readlane(my_blk, it);
    const int valid = min(kBlock, L - blk * kBlock);
    const bool ok0 = tp < valid, ok1 = tp + 8 < valid;
    float x0[G], x1[G];
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      x0[h] = ok0 ? sum8(qr[h].dot(cur.k0)) * a.scale_log2 : -__builtin_inff();
      x1[h] = ok1 ? sum8(qr[h].dot(cur.k1)) * a.scale_log2 : -__builtin_inff();
      need |= fmaxf(x0[h], x1[h]) > m[h] + kLazyRescale;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float bm = fmaxf(x0[h], x1[h]);
        bm = fmaxf(bm, __shfl_xor(bm, 8, 64));
        bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        if (bm > m[h] + kLazyRescale) {  // wave-uniform
          const float alpha = m[h] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m[h] - bm);
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) acc[h][cc] *= alpha;
#pragma unroll
          for (int u = 0; u < PPL; ++u)
            if ((cg + 8 * u) % G == h) lpart[u] *= alpha;
          m[h] = bm;
        }
      }
    }
    // publish p for the (token, head) pairs this lane owns
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int pr = cg + 8 * u;
      if (pr < PAIRS) {
        const int h = pr % G;
        const bool second = pr >= G;
        float x = x0[0], mh = m[0];
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          if (hh == h) {
            x = second ? x1[hh] : x0[hh];
            mh = m[hh];
          }
        const float pf = x == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(x - mh);
        const int t = second ? tp + 8 : tp;
        if constexpr (BF16) {
          const uint16_t pbits = f32_to_bf16(pf);  // the value p.V uses; l sums the same value
          lpart[u] += bf16_to_f32(pbits);
          sm.pb[wave][h][t] = pbits;
        } else {
          lpart[u] += pf;
          sm.p[wave][t][h] = pf;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid < kBlock) cur.v.mask_tokens(valid);  // slots past the sequence end may hold anything
    if constexpr (BF16) {
      // p.V as bf16 pair dot products: a V row word holds tokens (2i, 2i + 1)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4* pp = reinterpret_cast<const uint4*>(&sm.pb[wave][h][0]);
        const uint4 p03 = pp[0], p47 = pp[1];
        const uint32_t pw[8] = {p03.x, p03.y, p03.z, p03.w, p47.x, p47.y, p47.z, p47.w};
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          const uint32_t vw[8] = {cur.v.u[cc][0].x, cur.v.u[cc][0].y, cur.v.u[cc][0].z, cur.v.u[cc][0].w,
                                  cur.v.u[cc][1].x, cur.v.u[cc][1].y, cur.v.u[cc][1].z, cur.v.u[cc][1].w};
          float sacc = acc[h][cc];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            sacc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]),
                                                   __builtin_bit_cast(bf16x2_t, vw[i]), sacc, false);
          acc[h][cc] = sacc;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kBlock; ++t) {
        float pt[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pt[h] = sm.p[wave][t][h];
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          const float vv = cur.v.get(cc, t);
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][cc] = fmaf(pt[h], vv, acc[h][cc]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // three rotating buffers: block it in one, it + 1 in the next, it + 2 loading
  for (int it = 0; it < nw; it += 3) {
    step(it, A, C);
    if (it + 1 >= nw) break;
    step(it + 1, B, A);
    if (it + 2 >= nw) break;
    step(it + 2, C, B);
  }

  // wave state -> LDS
  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = 0.f;
#pragma unroll
  for (int u = 0; u < PPL; ++u) {
    const int pr = cg + 8 * u;
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (pr < PAIRS && pr % G == h) lsum[h] += lpart[u];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lsum[h] += __shfl_xor(lsum[h], o, 64);
    if (lane == 0) {
      sm.m[wave][h] = nw > 0 ? m[h] : -__builtin_inff();
      sm.l[wave][h] = nw > 0 ? lsum[h] : 0.f;
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) sm.acc[wave][h][lane * CPL + cc] = acc[h][cc];
  }
  __syncthreads();
  // merge the waves into this split's partial: thread -> (head, channels)
  const size_t part = gi * a.splits + s;
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int h = i / D, ch = i % D;
    float mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, sm.m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = sm.m[w][h];
      const float e = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - mx);
      num = fmaf(e, sm.acc[w][h][ch], num);
      den = fmaf(e, sm.l[w][h], den);
    }
    a.part_acc[(part * G + h) * D + ch] = num;
    if (ch == 0) {
      a.part_ml[(part * G + h) * 2 + 0] = mx;
      a.part_ml[(part * G + h) * 2 + 1] = den;
    }
  }
}

// grid: x = KV head, y = sequence; 256 threads: merge a group's splits. Each
// thread owns (head, channel) outputs; the partials of up to 16 splits are
// requested in one batch before any is used, merged with log-sum-exp weights.
constexpr int kMaxSplits = 512;  // plan_decode keeps splits at or below this
constexpr int kCombThreads = 256;

// Sum (SUM) or maximum over the workgroup; every thread gets the result.
template <bool SUM>
__device__ __forceinline__ float block_reduce(float x, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o, 64);
    x = SUM ? x + y : fmaxf(x, y);
  }
  if (lane == 0) red[wave] = x;
  __syncthreads();
  x = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) x = SUM ? x + red[w] : fmaxf(x, red[w]);
  __syncthreads();
  return x;
}

// Merge the splits of one query head: grid (KV head, sequence, head of the
// group), 256 threads. The splits' maxima and log-sum-exp weights come first
// (threads over splits), then thread (part, channel) accumulates every
// (256 / D)-th split's partial of its channel with all loads independent, and
// the parts are summed in LDS.
template <typename T, int D, int G>
__global__ __launch_bounds__(kCombThreads) void k_decode_combine(DecodeArgs a, void* __restrict__ out) {
  constexpr int PARTS = kCombThreads / D;
  __shared__ float w[kMaxSplits];
  __shared__ float red[kCombThreads / 64];
  __shared__ float part_num[PARTS][D];
  const CacheView& c = a.c;
  const int g = blockIdx.x, b = blockIdx.y, h = blockIdx.z, tid = threadIdx.x;
  const size_t gi = size_t(b) * c.Hkv + g;
  const int live = (a.count[b] + a.bps - 1) / a.bps;
  const float* ml = a.part_ml + (gi * a.splits * G + h) * 2;  // split sp at ml[sp * G * 2]
  float mx = -__builtin_inff();
  for (int sp = tid; sp < live; sp += kCombThreads) mx = fmaxf(mx, ml[sp * G * 2]);
  mx = block_reduce<false>(mx, red);
  float den = 0.f;
  for (int sp = tid; sp < live; sp += kCombThreads) {
    const float m = ml[sp * G * 2];
    const float e = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mx);
    w[sp] = e;
    den = fmaf(e, ml[sp * G * 2 + 1], den);
  }
  den = block_reduce<true>(den, red);  // its barriers also publish w
  const int ch = tid % D, part = tid / D;
  const float* acc = a.part_acc + (gi * a.splits * G + h) * D + ch;  // split sp at acc[sp * G * D]
  float num = 0.f;
#pragma unroll 16
  for (int sp = part; sp < live; sp += PARTS) num = fmaf(w[sp], acc[size_t(sp) * G * D], num);
  part_num[part][ch] = num;
  __syncthreads();
  if (part == 0) {
    float t = part_num[0][ch];
#pragma unroll
    for (int q = 1; q < PARTS; ++q) t += part_num[q][ch];
    store_out<T>(out, (size_t(b) * c.Hq + size_t(g) * G + h) * D + ch, t / den);
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, void* out, hipStream_t st) {
  const CacheView& c = a.c;
  dim3 grid(a.splits, c.Hkv, c.B);
  hipLaunchKernelGGL((k_decode<T, D, G>), grid, dim3(kDecThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(c.Hkv, c.B, G);
  hipLaunchKernelGGL((k_decode_combine<T, D, G>), g2, dim3(kCombThreads), 0, st, a, out);
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
  // About 512 workgroups of 4 waves (2 per CU) over the largest selection; a
  // split holds at most 256 blocks (64 per wave, one block id per lane).
  const long work = long(c.B) * c.Hkv * n_cap;
  int bps = int((work + 511) / 512);
  bps = bps < 4 ? 4 : (bps > 256 ? 256 : bps);
  DecodePlan p;
  p.bps = bps;
  p.splits = (n_cap + bps - 1) / bps;  // <= 512 (kMaxSplits): bps >= ceil(work / 512) >= n_cap / 512
  return p;
}

size_t decode_ws_bytes(const CacheView& c, int n_cap) {
  const DecodePlan p = plan_decode(c, n_cap);
  const size_t parts = size_t(c.B) * c.Hkv * p.splits * c.G;
  return align_up(parts * 2 * sizeof(float), 256) + parts * c.D * sizeof(float);
}

hipError_t launch_decode(const CacheView& c, const void* q, const int32_t* idx, const int32_t* count,
                         int n_cap, float scale, void* out, void* ws, hipStream_t st) {
  const DecodePlan p = plan_decode(c, n_cap);
  const size_t parts = size_t(c.B) * c.Hkv * p.splits * c.G;
  char* w = static_cast<char*>(ws);
  DecodeArgs a;
  a.c = c;
  a.q = q;
  a.idx = idx;
  a.count = count;
  a.n_cap = n_cap;
  a.bps = p.bps;
  a.splits = p.splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.part_ml = reinterpret_cast<float*>(w);
  a.part_acc = reinterpret_cast<float*>(w + align_up(parts * 2 * sizeof(float), 256));
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_decode_g<uint16_t, 128>(a, out, st) : launch_decode_g<uint16_t, 64>(a, out, st);
  return c.D == 128 ? launch_decode_g<float, 128>(a, out, st) : launch_decode_g<float, 64>(a, out, st);
}

}  // namespace resa
