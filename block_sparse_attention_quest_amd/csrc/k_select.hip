// GBSA block selection (Pith review of "Rectified Sparse Attention", "What
// carries the argument"; count rule Eq. 5 from its referee report, major
// comment 1, with an explicit active ratio r).
//
// k_score, grid (block chunk, KV head, sequence): every workgroup scores
// kScoreChunk blocks of one (sequence, KV head) group. The group's G query
// heads are pooled into their mean q_bar (float64, summed in head order), and
// block j gets the Quest upper bound
//   s_j = sum_c max(q_bar_c kmin_jc, q_bar_c kmax_jc),
// evaluated as q_bar_c * (q_bar_c >= 0 ? kmax_jc : kmin_jc): the two are equal
// because kmin <= kmax, rounding is monotone and these float64 products of
// bf16/fp32 keys are exact. A block's descriptor record for one head is
// 2 x head_dim contiguous elements; head_dim/8 lanes read it with 16-byte loads
// (all of a lane's loads are issued before any is used), and the lanes' float64
// partials are summed with DPP moves inside a row. Scores go to the workspace.
//
// k_topn, grid (KV head, sequence), 1024 threads: n = min(M, max(n_min,
// ceil(M r))) in IEEE double; the min(n_local, n) newest blocks are always
// taken; the other places go to the highest scores, ties to the lower index.
// The candidates' order-preserving 64-bit keys stay in registers (each thread
// issues exactly as many score loads as the longest sequence needs). The
// threshold is found exactly by radix selection with 12-bit digits starting
// below the common prefix of the candidates' key range (usually one pass)
// until the candidates that share the threshold's prefix number at most 64;
// one wave then ranks those exactly (key descending, index ascending). Chosen blocks are marked in an LDS
// bitmap and compacted in index order, so the output is sorted ascending.
//
// The two kernels hand over through the workspace at the kernel boundary: a
// cross-workgroup hand-off inside one kernel would need device-scope fences,
// which write back and invalidate a whole L2 on this multi-die part.
#include "refresh_block.h"

namespace resa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreChunk = 64;  // blocks scored per workgroup
constexpr int kTopnWaves = kTopnThreads / 64;
constexpr int kBitmapWords = kTopnThreads * kTopnMaxPerThread / 32;  // 1024
constexpr int kRankGroup = 64;

template <typename T>
struct Chunk8;  // 8 consecutive channels of a descriptor row
template <>
struct Chunk8<uint16_t> {
  uint4 u;
  __device__ void load(const void* base, size_t off) {
    u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  __device__ float get(int e) const {
    const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Chunk8<float> {
  float4 a, b;
  __device__ void load(const void* base, size_t off) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    a = p[0];
    b = p[1];
  }
  __device__ float get(int e) const {
    const float4 w = e < 4 ? a : b;
    const int r = e & 3;
    return r == 0 ? w.x : r == 1 ? w.y : r == 2 ? w.z : w.w;
  }
};

// Eq. 5's block count with the explicit ratio, in IEEE double.
__device__ __forceinline__ int select_count(int M, const resa_select_params& p) {
  return min(M, max(p.n_min, int(ceil(double(M) * p.r))));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = uint64_t(__double_as_longlong(x));
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(u)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(u >> 32)), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo)));
}

// Sum over aligned groups of N lanes (N = 8 or 16, inside one DPP row). Lane 0
// of each group always adds in the same order, so its result is deterministic.
template <int N>
__device__ __forceinline__ double row_sum_f64(double x) {
  if constexpr (N == 16) x += dpp_f64<0x128>(x);  // row_ror:8 pairs lanes i and i^8
  x += dpp_f64<kDppHalfMirror>(x);                 // then an 8-lane butterfly
  x += dpp_f64<kDppQuadXor1>(x);
  x += dpp_f64<kDppQuadXor2>(x);
  return x;
}

// grid: x = chunk of kScoreChunk blocks, y = KV head, z = sequence. Only the
// candidates, blocks below M - min(n_local, n), are scored (the forced newest
// blocks need no score). With append set, the last x index is not a chunk: its
// first wave writes the step's new token (k_new / v_new, [B][1][Hkv][D]) at
// position L - 1 and refreshes that block's descriptor, which no scoring
// workgroup reads because with n_local >= 1 it is always forced.
template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void k_score(CacheView c, const void* __restrict__ q,
                                                         resa_select_params p, double* __restrict__ scores,
                                                         bool append, const void* __restrict__ k_new,
                                                         const void* __restrict__ v_new) {
  constexpr int LPB = D / 8;     // lanes per block record (8 channels each)
  constexpr int BPW = 64 / LPB;  // blocks per wave per row of loads
  constexpr int ROWS = kScoreChunk / (4 * BPW);
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = c.seq_lens[b];
  const int M = (L + kBlock - 1) / kBlock;
  if (append && chunk == int(gridDim.x) - 1) {
    if (wave == 0 && L > 0) refresh_block<T, D>(c, k_new, v_new, 1, b, g, (L - 1) / kBlock, L, lane);
    return;
  }
  const int Mo = M - min(p.n_local, select_count(M, p));
  if (chunk * kScoreChunk >= Mo) return;
  const size_t gi = size_t(b) * c.Hkv + g;
  const int sub = lane % LPB, slot = lane / LPB, c0 = sub * 8;

  // The group's G query rows (this lane's 8 channels) first, then all page
  // ids, then all descriptor loads, every one issued unconditionally (blocks
  // past the candidates re-read block 0) so they are in flight together.
  Chunk8<T> qh[8];
  const size_t qbase = (size_t(b) * c.Hq + size_t(g) * c.G) * D + c0;
#pragma unroll
  for (int h = 0; h < 8; ++h)
    if (h < c.G) qh[h].load(q, qbase + size_t(h) * D);
  int jr[ROWS], page[ROWS];
  Chunk8<T> lo[ROWS], hi[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    jr[r] = chunk * kScoreChunk + (r * 4 + wave) * BPW + slot;
    page[r] = c.bt[size_t(b) * c.maxb + (jr[r] < Mo ? jr[r] : 0)];
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const size_t rec = (size_t(page[r]) * c.Hkv + g) * 2 * D;
    lo[r].load(c.desc, rec + c0);
    hi[r].load(c.desc, rec + D + c0);
  }
  // pooled query: heads summed in order in float64, then divided by G (G is a
  // power of two, so multiplying by 1/G is the same exact operation)
  double qb[8];
  const double inv_g = 1.0 / double(c.G);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    double acc = double(qh[0].get(e));
#pragma unroll
    for (int h = 1; h < 8; ++h)
      if (h < c.G) acc += double(qh[h].get(e));
    qb[e] = acc * inv_g;
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    double part = 0.0;
    if (jr[r] < Mo) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part += qb[e] * double(qb[e] >= 0.0 ? hi[r].get(e) : lo[r].get(e));
    }
    part = row_sum_f64<LPB>(part);
    if (sub == 0 && jr[r] < Mo) scores[gi * c.maxb + jr[r]] = part;
  }
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(x)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(x >> 32)), CTRL, 0xF, 0xF, false);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

// Maximum (MAX) or minimum over each row of 16 lanes, every lane of the row
// gets it (four DPP steps).
template <bool MAX>
__device__ __forceinline__ uint64_t row_reduce_u64(uint64_t x) {
  auto pick = [](uint64_t a, uint64_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = pick(x, dpp_u64<kDppQuadXor1>(x));
  x = pick(x, dpp_u64<kDppQuadXor2>(x));
  x = pick(x, dpp_u64<kDppHalfMirror>(x));
  return pick(x, dpp_u64<kDppRowMirror>(x));
}

// The same over the 64 lanes of a wave: the rows, then two lane swaps across
// rows.
template <bool MAX>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t x) {
  auto pick = [](uint64_t a, uint64_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = row_reduce_u64<MAX>(x);
  x = pick(x, uint64_t(__shfl_xor((unsigned long long)x, 16, 64)));
  x = pick(x, uint64_t(__shfl_xor((unsigned long long)x, 32, 64)));
  return x;
}

__device__ __forceinline__ uint64_t order_key(double s) {
  if (s == 0.0) s = 0.0;  // -0 and +0 are equal scores
  const uint64_t u = uint64_t(__double_as_longlong(s));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kTopnBits = 12;
constexpr int kTopnBins = 1 << kTopnBits;  // 4 bins per thread

struct TopnSmem {
  int hist[kTopnBins];
  uint32_t sel[kBitmapWords];
  uint32_t tie[kBitmapWords];
  uint64_t red_max[kTopnWaves], red_min[kTopnWaves];
  int scan[kTopnWaves];
  uint64_t gk[kRankGroup];
  int gj[kRankGroup];
  int gcount;
  int digit, k_rem, gsize;
};

// Exclusive scan over the 1024 threads; `total` gets the sum.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTopnWaves; ++w) {
    const int t = tmp[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// grid: x = KV head, y = sequence; 1024 threads. EMAX >= ceil(M / 1024) keys
// per thread, so every thread issues exactly EMAX score loads.
template <int EMAX>
__global__ __launch_bounds__(kTopnThreads) void k_topn(const double* __restrict__ scores,
                                                       const int32_t* __restrict__ seq_lens, int maxb,
                                                       int Hkv, resa_select_params p, int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ count, int n_cap) {
  __shared__ TopnSmem sm;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int L = seq_lens[b];
  const int M = (L + kBlock - 1) / kBlock;
  const int n = select_count(M, p);
  if (g == 0 && tid == 0) count[b] = n;
  const int keep = min(p.n_local, n);
  const int quota = n - keep;
  const int Mo = M - keep;  // candidates: blocks 0 .. Mo-1
  const size_t gi = size_t(b) * Hkv + g;
  const double* row = scores + gi * maxb;

  // keys of the candidates, block j = e * 1024 + tid (loads issued together;
  // out-of-range slots re-read block 0 and are ignored)
  uint64_t key[EMAX];
  {
    double sc[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int j = e * kTopnThreads + tid;
      sc[e] = row[j < Mo ? j : 0];
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e) key[e] = order_key(sc[e]);
  }
  for (int i = tid; i < kTopnBins; i += kTopnThreads) sm.hist[i] = 0;
  if (tid == 0) sm.gcount = 0;

  // mode: 0 none of the candidates, 1 every member of the prefix group,
  // 2 the lowest indices of the (exactly tied) prefix group, 3 ranked group
  int mode = 0;
  uint64_t prefix = 0, mask = 0;
  int k = quota;
  if (quota > 0) {
    uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e * kTopnThreads + tid < Mo) {
        kmax = key[e] > kmax ? key[e] : kmax;
        kmin = key[e] < kmin ? key[e] : kmin;
      }
    }
    kmax = wave_reduce_u64<true>(kmax);
    kmin = wave_reduce_u64<false>(kmin);
    if (lane == 0) {
      sm.red_max[wave] = kmax;
      sm.red_min[wave] = kmin;
    }
    __syncthreads();
    // lanes 0 .. 15 of every wave take one wave's result each, then reduce them
    // inside the row of 16
    kmax = sm.red_max[lane & (kTopnWaves - 1)];
    kmin = sm.red_min[lane & (kTopnWaves - 1)];
    kmax = row_reduce_u64<true>(kmax);
    kmin = row_reduce_u64<false>(kmin);
    const int plen = kmax == kmin ? 64 : __clzll((long long)(kmax ^ kmin));
    mask = plen == 0 ? 0ull : (~0ull << (64 - plen));
    prefix = kmax & mask;
    int gsize = Mo;  // every candidate lies in [kmin, kmax], so shares the prefix
    int bits_left = 64 - plen;
    bool first = true;
    while (gsize > kRankGroup && gsize != k && bits_left > 0) {
      const int nb = bits_left < kTopnBits ? bits_left : kTopnBits;
      const int shift = bits_left - nb;
      const int nbins = 1 << nb;
      const bool first_pass = first;
      if (!first) {
        for (int i = tid; i < kTopnBins; i += kTopnThreads) sm.hist[i] = 0;
        __syncthreads();
      }
      first = false;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        // the first pass takes every candidate: all share the range's prefix
        if (e * kTopnThreads + tid < Mo && (first_pass || (key[e] & mask) == prefix))
          atomicAdd(&sm.hist[int(key[e] >> shift) & (nbins - 1)], 1);
      }
      __syncthreads();
      // thread t owns the 4 digits nbins-1-4t .. nbins-4-4t (from the top)
      int h[4], mine = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = nbins - 1 - (4 * tid + u);
        h[u] = d >= 0 ? sm.hist[d] : 0;
        mine += h[u];
      }
      int total;
      int above = wg_exclusive_scan(mine, sm.scan, total);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (above < k && above + h[u] >= k) {
          sm.digit = nbins - 1 - (4 * tid + u);
          sm.k_rem = k - above;
          sm.gsize = h[u];
        }
        above += h[u];
      }
      __syncthreads();
      prefix |= uint64_t(sm.digit) << shift;
      mask |= uint64_t(nbins - 1) << shift;
      k = sm.k_rem;
      gsize = sm.gsize;
      bits_left -= nb;
    }
    mode = gsize == k ? 1 : (bits_left == 0 ? 2 : 3);
  }
  // mark the chosen blocks: a wave's 64 consecutive blocks are two bitmap
  // words, stored whole by its first lane from ballots (each word has exactly
  // one writer, so no clearing or atomics are needed); in mode 3 the members
  // of the threshold's prefix group are gathered for ranking on the way
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int j = e * kTopnThreads + tid;
    bool s = false, t = false;
    if (j < Mo) {
      const uint64_t km = key[e] & mask;
      const bool above = km > prefix, at = km == prefix;
      s = mode != 0 && (above || (at && mode == 1));
      t = at && mode == 2;
      if (at && mode == 3) {
        const int slot = atomicAdd(&sm.gcount, 1);
        sm.gk[slot] = key[e];
        sm.gj[slot] = j;
      }
    } else if (j < M) {
      s = true;
    }
    const uint64_t bs = __builtin_amdgcn_ballot_w64(s);
    const int w0 = (e * kTopnThreads + wave * 64) >> 5;
    if (lane == 0) {
      sm.sel[w0] = uint32_t(bs);
      sm.sel[w0 + 1] = uint32_t(bs >> 32);
    }
    if (mode == 2) {  // the tie words are read in mode 2 only
      const uint64_t bt = __builtin_amdgcn_ballot_w64(t);
      if (lane == 0) {
        sm.tie[w0] = uint32_t(bt);
        sm.tie[w0 + 1] = uint32_t(bt >> 32);
      }
    }
  }
  __syncthreads();
  if (mode == 3 && tid < 64) {  // wave 0 ranks the gathered group, one candidate per lane
    const int gs = sm.gcount;
    const uint64_t kt = tid < gs ? sm.gk[tid] : 0;
    const int jt = tid < gs ? sm.gj[tid] : 0;
    const uint32_t klo = uint32_t(kt), khi = uint32_t(kt >> 32);
    int rank = 0;
    for (int u = 0; u < gs; ++u) {  // candidate u broadcast from its lane
      const uint64_t ku = (uint64_t(uint32_t(__builtin_amdgcn_readlane(khi, u))) << 32) |
                          uint32_t(__builtin_amdgcn_readlane(klo, u));
      const int ju = __builtin_amdgcn_readlane(jt, u);
      rank += (ku > kt || (ku == kt && ju < jt)) ? 1 : 0;
    }
    if (tid < gs && rank < k) atomicOr(&sm.sel[jt >> 5], 1u << (jt & 31));
  }
  __syncthreads();
  // exactly tied threshold group: the k lowest indices
  const int W = (M + 31) / 32;
  uint32_t word = tid < W ? sm.sel[tid] : 0u;
  if (mode == 2) {
    const uint32_t tw = tid < W ? sm.tie[tid] : 0u;
    int total;
    int before = wg_exclusive_scan(__builtin_popcount(tw), sm.scan, total);
    uint32_t f = tw;
    while (f) {
      const uint32_t bit = f & (~f + 1u);
      if (before++ < k) word |= bit;
      f &= f - 1u;
    }
  }
  int total;
  int pos = wg_exclusive_scan(__builtin_popcount(word), sm.scan, total);
  int32_t* out = idx + gi * n_cap;
  while (word && pos < n) {  // exactly n bits are set; the bound keeps every store in the row
    const int e = __builtin_ctz(word);
    word &= word - 1u;
    out[pos++] = tid * 32 + e;
  }
}

hipError_t launch_topn(const CacheView& c, const resa_select_params& p, int32_t* idx, int32_t* count,
                       int n_cap, const double* scores, hipStream_t s) {
  const int mmax = (c.max_seq_len + kBlock - 1) / kBlock;
  const int e = (mmax + kTopnThreads - 1) / kTopnThreads;
  dim3 grid(c.Hkv, c.B);
#define RESA_TOPN(E) hipLaunchKernelGGL(k_topn<E>, grid, dim3(kTopnThreads), 0, s, scores, c.seq_lens, c.maxb, \
                                        c.Hkv, p, idx, count, n_cap)
  // every thread handles EMAX keys: exact up to 18 (256K context), then
  // coarser steps
  switch (e) {
    case 0: case 1: case 2: RESA_TOPN(2); break;
    case 3: case 4: RESA_TOPN(4); break;
    case 5: case 6: RESA_TOPN(6); break;
    case 7: case 8: RESA_TOPN(8); break;
    case 9: RESA_TOPN(9); break;
    case 10: RESA_TOPN(10); break;
    case 11: case 12: RESA_TOPN(12); break;
    case 13: case 14: RESA_TOPN(14); break;
    case 15: case 16: RESA_TOPN(16); break;
    case 17: RESA_TOPN(17); break;
    case 18: RESA_TOPN(18); break;
    case 19: case 20: RESA_TOPN(20); break;
    case 21: case 22: case 23: case 24: RESA_TOPN(24); break;
    default: RESA_TOPN(32); break;
  }
#undef RESA_TOPN
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_select_t(const CacheView& c, const void* q, const resa_select_params& p, int32_t* idx,
                           int32_t* count, int n_cap, double* scores, bool append, const void* k_new,
                           const void* v_new, hipStream_t s) {
  dim3 g1((c.maxb + kScoreChunk - 1) / kScoreChunk + (append ? 1 : 0), c.Hkv, c.B);
  hipLaunchKernelGGL((k_score<T, D>), g1, dim3(kScoreThreads), 0, s, c, q, p, scores, append, k_new, v_new);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topn(c, p, idx, count, n_cap, scores, s);
}

}  // namespace

size_t select_ws_bytes(const CacheView& c) { return size_t(c.B) * c.Hkv * c.maxb * sizeof(double); }

namespace {
hipError_t select_dispatch(const CacheView& c, const void* q, const resa_select_params& p, int32_t* idx,
                           int32_t* count, int n_cap, void* ws, bool append, const void* k_new,
                           const void* v_new, hipStream_t s) {
  double* scores = static_cast<double*>(ws);
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_select_t<uint16_t, 128>(c, q, p, idx, count, n_cap, scores, append, k_new, v_new, s)
                      : launch_select_t<uint16_t, 64>(c, q, p, idx, count, n_cap, scores, append, k_new, v_new, s);
  return c.D == 128 ? launch_select_t<float, 128>(c, q, p, idx, count, n_cap, scores, append, k_new, v_new, s)
                    : launch_select_t<float, 64>(c, q, p, idx, count, n_cap, scores, append, k_new, v_new, s);
}
}  // namespace

hipError_t launch_select(const CacheView& c, const void* q, const resa_select_params& p, int32_t* idx,
                         int32_t* count, int n_cap, void* ws, hipStream_t s) {
  return select_dispatch(c, q, p, idx, count, n_cap, ws, false, nullptr, nullptr, s);
}

// One decode step's append (n_new = 1) and selection. With n_local >= 1 the
// newest block is forced, never scored, so its refresh rides in the scoring
// launch; otherwise the refresh must finish before scoring and runs first.
hipError_t launch_append_select(const CacheView& c, const void* k_new, const void* v_new, const void* q,
                                const resa_select_params& p, int32_t* idx, int32_t* count, int n_cap, void* ws,
                                hipStream_t s) {
  if (p.n_local >= 1) return select_dispatch(c, q, p, idx, count, n_cap, ws, true, k_new, v_new, s);
  const hipError_t e = launch_update_tail(c, k_new, v_new, 1, s);
  if (e != hipSuccess) return e;
  return launch_select(c, q, p, idx, count, n_cap, ws, s);
}

}  // namespace resa
