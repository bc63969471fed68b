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
// partials are summed with DPP moves inside a row. Each score goes to the
// workspace as its order-preserving 64-bit key (unsigned order of keys is the
// numeric order of scores, -0 and +0 equal), in rows of an even stride.
//
// k_topn, grid (KV head, sequence), 1024 threads: n = min(M, max(n_min,
// ceil(M r))) in IEEE double; the min(n_local, n) newest blocks are always
// taken; the other places go to the highest scores, ties to the lower index.
// The candidates' keys stay in registers (each thread issues exactly as many
// loads as the longest sequence needs, before the sequence length arrives).
// The threshold is found exactly by radix selection with 12-bit digits
// starting below the common prefix of the candidates' key range (usually one
// pass) until the candidates that share the threshold's prefix number at most
// 64. Chosen blocks are marked in an LDS bitmap from ballots; the members of
// that last group are listed per wave and ranked exactly (key descending,
// index ascending) by one wave, a member per lane. The bitmap
// is compacted in index order, so the output is sorted ascending. Prefix sums
// and reductions run on DPP lane moves; values every lane shares are moved to
// scalar registers so that the per-mode branches are scalar.
//
// The two kernels hand over through the workspace at the kernel boundary: a
// cross-workgroup hand-off inside one kernel would need device-scope fences,
// which write back and invalidate a whole L2 on this multi-die part.
#include <type_traits>

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

// Order-preserving key of a score: unsigned comparison of keys is numeric
// comparison of scores, with -0 and +0 equal.
__device__ __forceinline__ uint64_t order_key(double s) {
  if (s == 0.0) s = 0.0;
  const uint64_t u = uint64_t(__double_as_longlong(s));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
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
                                                         resa_select_params p, uint64_t* __restrict__ keys,
                                                         bool append, const void* __restrict__ k_new,
                                                         const void* __restrict__ v_new) {
  constexpr int LPB = D / 8;     // lanes per block record (8 channels each)
  constexpr int BPW = 64 / LPB;  // blocks per wave per row of loads
  constexpr int ROWS = kScoreChunk / (4 * BPW);
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = checked_len(c, b);
  RESA_CHECK(c.dbg, L >= 1, kChkEmpty, (void)0);
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
    page[r] = checked_page(c, b, jr[r] < Mo ? jr[r] : 0);
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
    if (sub == 0 && jr[r] < Mo) keys[gi * key_stride(c.maxb) + jr[r]] = order_key(part);
  }
}

// Maximum (MAX) or minimum of x over each row of 16 lanes; every lane of the
// row gets it (four DPP steps).
template <bool MAX>
__device__ __forceinline__ uint32_t row_reduce_u32(uint32_t x) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = pick(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), kDppQuadXor1, 0xF, 0xF, false)));
  x = pick(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), kDppQuadXor2, 0xF, 0xF, false)));
  x = pick(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), kDppHalfMirror, 0xF, 0xF, false)));
  return pick(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), kDppRowMirror, 0xF, 0xF, false)));
}

// The same over the 64 lanes of a wave: the rows, then their four results
// read out into scalars.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = row_reduce_u32<MAX>(x);
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return pick(pick(a, b), pick(c, d));
}

// Inclusive prefix sum inside each row of 16 lanes (DPP row shifts by 1, 2, 4
// and 8; a lane with no source lane adds 0).
__device__ __forceinline__ int row_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1 + 1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1 + 3, 0xF, 0xF, false);
  return x + __builtin_amdgcn_update_dpp(0, x, kDppRowShr1 + 7, 0xF, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: the rows, then the last
// lane of row 0 added into rows 1 and 3 (of row 2 into row 3), then that of
// row 1 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = row_incl_scan(x);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);
  return x + __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);
}

// A value every lane of the wave holds, moved to a scalar register so that
// branches on it are scalar branches.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return uint32_t(__builtin_amdgcn_readfirstlane(int(x))); }

// Exclusive prefix sum of v over the 1024 threads; `total` gets the sum. One
// barrier. `tmp` (one int per wave) must not be in use by another scan that
// some wave may still be reading.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(int(threadIdx.x >> 6));
  const int x = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  const int w = row_incl_scan(lane < kTopnWaves ? tmp[lane] : 0);  // lanes 0 .. 15: waves 0 .. lane
  total = __builtin_amdgcn_readlane(w, kTopnWaves - 1);
  const int before = wave == 0 ? 0 : __builtin_amdgcn_readlane(w, wave - 1);
  return before + x - v;
}

constexpr int kTopnBits = 12;
constexpr int kTopnBins = 1 << kTopnBits;  // 4 bins per thread

// Selection state in LDS. The histogram is dead once the threshold is known,
// so the bitmaps and the ranked group's lists reuse its space.
struct TopnAfter {
  uint32_t sel[kBitmapWords];
  uint32_t tie[kBitmapWords];
  uint64_t gk[kTopnWaves][kRankGroup];  // ranked group: each wave's members in its own order
  int gj[kTopnWaves][kRankGroup];
  uint64_t ck[kRankGroup];  // the ranked group laid end to end
  int cj[kRankGroup];
};
struct alignas(16) TopnShared {
  union {
    int hist[kTopnBins];
    TopnAfter a;
  } u;
  uint32_t red[4][kTopnWaves];  // per wave: max, min of the keys' high words, then of the low words
  int scan_a[kTopnWaves], scan_b[kTopnWaves];
  int gcount[kTopnWaves];
  int digit, k_rem, gsize;
};

// Keys in registers: EMAX per thread, block j = e * 1024 + tid, all loads
// issued together (slots past the row re-read entry 0 and are ignored). The
// per-block steps are unrolled over the EMAX registers.
template <int EMAX>
struct RegKeys {
  uint64_t k[EMAX];
  __device__ void load(const uint64_t* row, int len) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int j = e * kTopnThreads + int(threadIdx.x);
      k[e] = row[j < len ? j : 0];
    }
  }
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) f(e * kTopnThreads + int(threadIdx.x), k[e]);
  }
};

// Selection of one (sequence, KV head) row. keys.each(f) calls f(j, key) for
// every block j < M (and past it, up to the register count), with the same
// j - lane across a wave; out is the row of idx.
template <class Keys>
__device__ __forceinline__ void topn_row(const Keys& keys, TopnShared& sm, int M, int n, int keep,
                                         int32_t* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(int(tid >> 6));
  const int quota = n - keep;
  const int Mo = M - keep;  // candidates: blocks 0 .. Mo-1

  // mode: 0 none of the candidates, 1 every member of the prefix group,
  // 2 the lowest indices of the (exactly tied) prefix group, 3 ranked group
  int mode = 0;
  uint64_t prefix = 0, mask = 0;
  int k = quota;
  if (quota > 0) {
    reinterpret_cast<int4*>(sm.u.hist)[tid] = int4{0, 0, 0, 0};  // kTopnBins = 4 x 1024
    // the candidates' key range, high words first; the low words only when
    // every high word is the same
    uint32_t hmax = 0, hmin = ~0u;
    keys.each([&](int j, uint64_t key) {
      if (j < Mo) {
        const uint32_t h = uint32_t(key >> 32);
        hmax = h > hmax ? h : hmax;
        hmin = h < hmin ? h : hmin;
      }
    });
    hmax = wave_reduce_u32<true>(hmax);
    hmin = wave_reduce_u32<false>(hmin);
    if (lane == 0) {
      sm.red[0][wave] = hmax;
      sm.red[1][wave] = hmin;
    }
    __syncthreads();
    // lanes 0 .. 15 of every row take one wave's result each, then reduce them
    // inside the row of 16
    hmax = uniform(row_reduce_u32<true>(sm.red[0][lane & (kTopnWaves - 1)]));
    hmin = uniform(row_reduce_u32<false>(sm.red[1][lane & (kTopnWaves - 1)]));
    int plen;
    if (hmax != hmin) {
      plen = __clz(hmax ^ hmin);
      prefix = uint64_t(hmax) << 32;
    } else {
      uint32_t lmax = 0, lmin = ~0u;
      keys.each([&](int j, uint64_t key) {
        if (j < Mo) {
          const uint32_t l = uint32_t(key);
          lmax = l > lmax ? l : lmax;
          lmin = l < lmin ? l : lmin;
        }
      });
      lmax = wave_reduce_u32<true>(lmax);
      lmin = wave_reduce_u32<false>(lmin);
      if (lane == 0) {
        sm.red[2][wave] = lmax;
        sm.red[3][wave] = lmin;
      }
      __syncthreads();
      lmax = uniform(row_reduce_u32<true>(sm.red[2][lane & (kTopnWaves - 1)]));
      lmin = uniform(row_reduce_u32<false>(sm.red[3][lane & (kTopnWaves - 1)]));
      plen = 32 + (lmax == lmin ? 32 : __clz(lmax ^ lmin));
      prefix = (uint64_t(hmax) << 32) | lmax;
    }
    mask = plen == 0 ? 0ull : (~0ull << (64 - plen));
    prefix &= mask;
    int gsize = Mo;  // every candidate lies in the range, so shares its prefix
    int bits_left = 64 - plen;
    bool first = true;
    while (gsize > kRankGroup && gsize != k && bits_left > 0) {
      const int nb = bits_left < kTopnBits ? bits_left : kTopnBits;
      const int shift = bits_left - nb;
      const int nbins = 1 << nb;
      const bool first_pass = first;
      if (!first) {
        reinterpret_cast<int4*>(sm.u.hist)[tid] = int4{0, 0, 0, 0};
        __syncthreads();
      }
      first = false;
      // the first pass takes every candidate: all share the range's prefix
      keys.each([&](int j, uint64_t key) {
        if (j < Mo && (first_pass || (key & mask) == prefix))
          atomicAdd(&sm.u.hist[int(key >> shift) & (nbins - 1)], 1);
      });
      __syncthreads();
      // thread t owns the 4 digits nbins-1-4t .. nbins-4-4t (from the top)
      int h[4], mine = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = nbins - 1 - (4 * tid + u);
        h[u] = d >= 0 ? sm.u.hist[d] : 0;
        mine += h[u];
      }
      int total;
      int above = wg_exclusive_scan(mine, sm.scan_a, total);
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
      prefix |= uint64_t(uniform(sm.digit)) << shift;
      mask |= uint64_t(nbins - 1) << shift;
      k = uniform(sm.k_rem);
      gsize = uniform(sm.gsize);
      bits_left -= nb;
    }
    mode = gsize == k ? 1 : (bits_left == 0 ? 2 : 3);
  }
  // mark the chosen blocks: a wave's 64 consecutive blocks are two bitmap
  // words, stored whole by its first lane from ballots (each word has exactly
  // one writer, so no clearing or atomics are needed); in mode 3 every wave
  // lists its members of the threshold's prefix group (at most 64 in all)
  int wcount = 0;  // wave-uniform
  // (key & mask) > prefix  <=>  key > prefix | ~mask;  (key & mask) >= prefix  <=>  key >= prefix
  const uint64_t top = prefix | ~mask;
  // one loop per mode, so that every test in it is a per-lane comparison
  auto mark = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    keys.each([&](int j, uint64_t key) {
      const bool cand = j < Mo, forced = !cand && j < M;
      bool s = forced, at = false;
      if constexpr (MODE == 1) s = (cand && key >= prefix) || forced;
      if constexpr (MODE >= 2) {
        const bool gt = key > top;
        s = (cand && gt) || forced;
        at = cand && !gt && key >= prefix;
      }
      const uint64_t bs = __builtin_amdgcn_ballot_w64(s);
      const int w0 = (j - lane) >> 5;
      if (lane == 0) {
        sm.u.a.sel[w0] = uint32_t(bs);
        sm.u.a.sel[w0 + 1] = uint32_t(bs >> 32);
      }
      if constexpr (MODE == 2) {  // the tie words are read in mode 2 only
        const uint64_t bt = __builtin_amdgcn_ballot_w64(at);
        if (lane == 0) {
          sm.u.a.tie[w0] = uint32_t(bt);
          sm.u.a.tie[w0 + 1] = uint32_t(bt >> 32);
        }
      }
      if constexpr (MODE == 3) {
        const uint64_t bt = __builtin_amdgcn_ballot_w64(at);
        if (bt) {
          if (at) {
            const int slot = wcount + int(__builtin_amdgcn_mbcnt_hi(uint32_t(bt >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo(uint32_t(bt), 0u)));
            sm.u.a.gk[wave][slot] = key;
            sm.u.a.gj[wave][slot] = j;
          }
          wcount += __builtin_popcountll(bt);
        }
      }
    });
  };
  switch (mode) {
    case 0: mark(std::integral_constant<int, 0>{}); break;
    case 1: mark(std::integral_constant<int, 1>{}); break;
    case 2: mark(std::integral_constant<int, 2>{}); break;
    default: mark(std::integral_constant<int, 3>{}); break;
  }
  if (mode == 3 && lane == 0) sm.gcount[wave] = wcount;
  __syncthreads();
  if (mode == 3 && wave == 0) {
    // ranked group (key descending, index ascending; a few dozen blocks at
    // most): member i in lane i (the waves' lists laid end to end), then every
    // member counts the members that come before it
    const int incl = row_incl_scan(lane < kTopnWaves ? sm.gcount[lane] : 0);
    const int gs = __builtin_amdgcn_readlane(incl, kTopnWaves - 1);
    int owner = 0, base = 0;
#pragma unroll
    for (int w = 0; w < kTopnWaves - 1; ++w) {
      const int iw = __builtin_amdgcn_readlane(incl, w);
      if (iw <= lane) {
        owner = w + 1;
        base = iw;
      }
    }
    uint64_t kt = 0;
    int jt = 0;
    if (lane < gs) {
      kt = sm.u.a.gk[owner][lane - base];
      jt = sm.u.a.gj[owner][lane - base];
    }
    // the group goes to LDS once, then every member is read back as a
    // broadcast (one address for the whole wave), several in flight at once;
    // the same wave writes and reads, so program order makes the writes visible
    sm.u.a.ck[lane] = kt;
    sm.u.a.cj[lane] = jt;
    int rank = 0;
#pragma unroll 8
    for (int u = 0; u < gs; ++u) {
      const uint64_t ku = sm.u.a.ck[u];
      const int ju = sm.u.a.cj[u];
      rank += int(ku > kt) | (int(ku == kt) & int(ju < jt));  // no short circuit: both loads issue
    }
    if (lane < gs && rank < k) atomicOr(&sm.u.a.sel[jt >> 5], 1u << (jt & 31));
  }
  if (mode == 3) __syncthreads();
  // exactly tied threshold group: the k lowest indices
  const int W = (M + 31) / 32;
  uint32_t word = tid < W ? sm.u.a.sel[tid] : 0u;
  if (mode == 2) {
    const uint32_t tw = tid < W ? sm.u.a.tie[tid] : 0u;
    int total;
    int before = wg_exclusive_scan(__builtin_popcount(tw), sm.scan_a, total);
    uint32_t f = tw;
    while (f) {
      const uint32_t bit = f & (~f + 1u);
      if (before++ < k) word |= bit;
      f &= f - 1u;
    }
  }
  int total;
  int pos = wg_exclusive_scan(__builtin_popcount(word), sm.scan_b, total);
  while (word && pos < n) {  // exactly n bits are set; the bound keeps every store in the row
    const int e = __builtin_ctz(word);
    word &= word - 1u;
    out[pos++] = tid * 32 + e;
  }
}

// grid: x = KV head, y = sequence; 1024 threads. EMAX >= ceil(M / 1024) keys
// per thread, held in registers.
template <int EMAX>
__global__ __launch_bounds__(kTopnThreads) void k_topn(const uint64_t* __restrict__ keys, int stride,
                                                       const int32_t* __restrict__ seq_lens, int Hkv,
                                                       resa_select_params p, int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ count, int n_cap, int max_len,
                                                       int* dbg) {
  __shared__ TopnShared sm;
  const int g = blockIdx.x, b = blockIdx.y;
  const size_t gi = size_t(b) * Hkv + g;
  RegKeys<EMAX> rk;
  rk.load(keys + gi * stride, stride);  // issued before the sequence length arrives
  int L = seq_lens[b];
  RESA_CHECK(dbg, L >= 0 && L <= max_len, kChkSeqLen, L = min(max(L, 0), max_len));
  const int M = (L + kBlock - 1) / kBlock;
  const int n = select_count(M, p);
  if (g == 0 && threadIdx.x == 0) count[b] = n;
  topn_row(rk, sm, M, n, min(p.n_local, n), idx + gi * n_cap);
}

hipError_t launch_topn(const CacheView& c, const resa_select_params& p, int32_t* idx, int32_t* count,
                       int n_cap, const uint64_t* keys, hipStream_t s) {
  const int mmax = (c.max_seq_len + kBlock - 1) / kBlock;
  const int stride = key_stride(c.maxb);
  dim3 grid(c.Hkv, c.B);
  const int e = (mmax + kTopnThreads - 1) / kTopnThreads;
#define RESA_TOPN(E) hipLaunchKernelGGL(k_topn<E>, grid, dim3(kTopnThreads), 0, s, keys, stride, c.seq_lens, \
                                        c.Hkv, p, idx, count, n_cap, c.max_seq_len, c.dbg)
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
                           int32_t* count, int n_cap, uint64_t* keys, bool append, const void* k_new,
                           const void* v_new, hipStream_t s) {
  dim3 g1((c.maxb + kScoreChunk - 1) / kScoreChunk + (append ? 1 : 0), c.Hkv, c.B);
  hipLaunchKernelGGL((k_score<T, D>), g1, dim3(kScoreThreads), 0, s, c, q, p, keys, append, k_new, v_new);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topn(c, p, idx, count, n_cap, keys, s);
}

}  // namespace

// The keys' rows, 16-byte aligned (one extra piece of slack for aligning the
// caller's pointer).
size_t select_ws_bytes(const CacheView& c) { return size_t(c.B) * c.Hkv * key_stride(c.maxb) * sizeof(uint64_t) + 16; }

namespace {
hipError_t select_dispatch(const CacheView& c, const void* q, const resa_select_params& p, int32_t* idx,
                           int32_t* count, int n_cap, void* ws, bool append, const void* k_new,
                           const void* v_new, hipStream_t s) {
  uint64_t* keys = reinterpret_cast<uint64_t*>((reinterpret_cast<uintptr_t>(ws) + 15) & ~uintptr_t(15));
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_select_t<uint16_t, 128>(c, q, p, idx, count, n_cap, keys, append, k_new, v_new, s)
                      : launch_select_t<uint16_t, 64>(c, q, p, idx, count, n_cap, keys, append, k_new, v_new, s);
  return c.D == 128 ? launch_select_t<float, 128>(c, q, p, idx, count, n_cap, keys, append, k_new, v_new, s)
                    : launch_select_t<float, 64>(c, q, p, idx, count, n_cap, keys, append, k_new, v_new, s);
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
