// Block-sparse decoding over the selected blocks (Eq. 2 of the paper as the Pith
// review's referee report, minor comment 3, restates it: a key is attended iff
// its 16-token block is selected), split over the key axis in the manner of
// Flash-Decoding (reference [6] of the Pith reference list), then merged exactly.
//
// grid (split, KV head, sequence), 4 waves. A split is a run of the group's
// selected blocks; wave w takes every 4th of them. Per block the wave reads the
// K tile (16 tokens x d, token-major) and the V tile (stored channel-major,
// d x 16 tokens) of one page, 4 KiB each at d = 128 bf16, and serves all G
// query heads of the group from them, so each selected byte is fetched once per
// group. The next blocks are in flight while one is processed (rotating
// register sets, so no copy ever waits on a load). The softmax keeps one running
// max per head, moved only when a logit exceeds it by more than 2^8 (numerator
// and denominator share every rescale, so the result is unchanged). The 4 wave
// states are merged through LDS into one split partial (m, l, acc[d]) in fp32;
// k_decode_combine then merges a group's splits with log-sum-exp weights (a
// separate kernel, so the hand-off needs no device-scope fence).
//
// k_decode_mfma (bf16 cache) runs both products on the matrix cores; k_decode
// (fp32 cache) on the VALU.
#include <type_traits>

#include "resa_internal.h"

namespace resa {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecBuffers = 3;   // blocks per wave in registers: one in use, the rest loading

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Loads of the gathered K/V pages. They are non-temporal: a step's selection
// is read once and the next step's differs, while the block descriptors, which
// every step's scoring reads again, fit in the last-level cache only if these
// pages do not displace them (measured: selection 36.3 -> 30.9 us and this
// call 42.9 -> 39.7 us per step at 128K context, batch 4).
__device__ __forceinline__ uint4 load_kv16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ uint2 load_kv8(const void* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(static_cast<const u32x2_t*>(p)));
}

// One lane's channels of one K token row.
template <typename T, int D>
struct KRow;
template <int D>
struct KRow<float, D> {
  static constexpr int NCH = D / 64;
  float4 u[NCH][2];
  __device__ void load(const float* row, int cg) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const float* p = row + cg * 8 + 64 * k;
      u[k][0] = __builtin_bit_cast(float4, load_kv16(p));
      u[k][1] = __builtin_bit_cast(float4, load_kv16(p + 4));
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
struct VRows<float, CPL> {
  float4 u[CPL][4];
  __device__ void load(const float* tile, int lane) {
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const float* p = tile + (lane * CPL + cc) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) u[cc][i] = __builtin_bit_cast(float4, load_kv16(p + 4 * i));
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

// The wave states of a split, merged into its partial.
template <int G, int D>
struct DecMerge {
  float m[kDecWaves][G];
  float l[kDecWaves][G];
  float acc[kDecWaves][G][D];
};
template <int G, int D>
struct DecSmem : DecMerge<G, D> {
  float p[kDecWaves][16][G];       // probabilities of the current block
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

// fp32 cache, VALU. grid: x = split, y = KV head, z = sequence; 256 threads.
//   q.k: lane = 8 * tp + cg holds tokens tp and tp + 8 and channels
//   cg*8 + 64*k + [0, 8) of K; fp32 FMAs, then a 3-step DPP sum over the 8 lanes
//   that share the tokens.
//   softmax: each of the 2G (token, head) pairs of a token pair is
//   exponentiated by one lane and published through LDS.
//   p.V: lane owns head_dim/64 channels; its V rows are 16 contiguous tokens.
template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeArgs a) {
  static_assert(sizeof(T) == 4, "the bf16 cache decodes on the matrix cores");
  constexpr int CPL = D / 64;                      // V channels per lane
  constexpr int PAIRS = 2 * G;                     // (token, head) pairs per token pair
  constexpr int PPL = PAIRS > 8 ? PAIRS / 8 : 1;   // pairs per lane
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
#ifdef RESA_DEBUG_CHECKS
  int raw_blk = 0, raw_page = 0;
#endif
  if (lane * kDecWaves < a.bps) {
    const int pos = min(first + wave + kDecWaves * lane, a.n_cap - 1);
    my_blk = min(max(a.idx[gi * a.n_cap + pos], 0), c.maxb - 1);
    my_page = min(max(c.bt[size_t(b) * c.maxb + my_blk], 0), c.num_pages - 1);
#ifdef RESA_DEBUG_CHECKS
    raw_blk = a.idx[gi * a.n_cap + pos];
    raw_page = c.bt[size_t(b) * c.maxb + my_blk];
#endif
  }
  const int n = a.count[b];
  const int L = c.seq_lens[b];
#ifdef RESA_DEBUG_CHECKS
  {  // the indices above are clamped into their arrays whatever they hold; here they are only checked
    const int M = (L + kBlock - 1) / kBlock;
    RESA_CHECK(c.dbg, L >= 0 && L <= c.max_seq_len, kChkSeqLen, (void)0);
    RESA_CHECK(c.dbg, L >= 1, kChkEmpty, (void)0);
    RESA_CHECK(c.dbg, n >= 0 && n <= a.n_cap, kChkSelection, (void)0);
    if (lane * kDecWaves < a.bps && first + wave + kDecWaves * lane < min(n, a.n_cap)) {
      RESA_CHECK(c.dbg, raw_blk >= 0 && raw_blk < M, kChkSelection, (void)0);
      RESA_CHECK(c.dbg, raw_page >= 0 && raw_page < c.num_pages, kChkPage, (void)0);
    }
  }
#endif
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
        lpart[u] += pf;
        sm.p[wave][t][h] = pf;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid < kBlock) cur.v.mask_tokens(valid);  // slots past the sequence end may hold anything
    {
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

// bf16 cache: the same split and wave structure with both products on the
// matrix cores. Per block a wave computes S^T = K Q^T with D/32 MFMAs
// 16x16x32 (A: the K tile, lane l holding token l % 16 and channels
// 32 ks + 8 (l / 16) + [0, 8); B: the group's queries in the same channel order,
// lane l holding head l % 16, zero for l % 16 >= G). The result leaves lane l
// with head l % 16 and tokens 4 (l / 16) + [0, 4), so after the online
// softmax the probabilities go straight into O^T += V^T P^T with no data
// movement: D/16 MFMAs 16x16x32 whose A operands are the lane's 8-byte piece
// of the channel-major V tile (lane l: channel 16 dt + l % 16, tokens
// 4 (l / 16) + [0, 4)) written twice, and whose B operand is that lane's
// probabilities as the bf16 pair hi + lo (hi = bf16(p), lo = bf16(p - hi)):
// k = 8 (l / 16) + [0, 4) takes hi, k = 8 (l / 16) + [4, 8) lo, so one
// instruction adds V^T P_hi^T + V^T P_lo^T, and p carries about 16
// significant bits instead of 8 (a row whose weight sits on a few keys would
// otherwise carry up to 2^-9 of p's rounding times the spread of its values).
// The denominator sums the same hi + lo values. A lane keeps the running max,
// denominator and O^T column of one head: no cross-lane sums, one max over the
// four lane groups per block.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct MfmaBlock {
  uint4 k[D / 32];  // S^T A operand pieces
  uint2 v[D / 16];  // O^T A operand pieces
  __device__ void load(const uint16_t* kt, const uint16_t* vt, int lane) {
    const int t = lane & 15, j = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) k[ks] = load_kv16(kt + t * D + 32 * ks + 8 * j);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) v[dt] = load_kv8(vt + (16 * dt + t) * kBlock + 4 * j);
  }
};

// grid: x = split, y = KV head, z = sequence (dealt to XCDs by xcd_pair_remap);
// 256 threads.
template <int D, int G, int NB>
__global__ __launch_bounds__(kDecThreads) void k_decode_mfma(DecodeArgs a) {
  constexpr int KS = D / 32, DT = D / 16;
  __shared__ DecMerge<G, D> sm;
  const CacheView& c = a.c;
  const int3 w = xcd_pair_remap(blockIdx.x, blockIdx.y, blockIdx.z, a.splits, c.Hkv);
  const int s = w.x, g = w.y, b = w.z;  // split, KV head, sequence
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane & 15, j = lane >> 4;  // head column, token group
  const size_t gi = size_t(b) * c.Hkv + g;
  const int first = s * a.bps;

  // block and page ids of this wave's blocks (first + wave + 4 i), clamped
  // into their rows so every load is in bounds; as in the VALU kernel
  int my_blk = 0, my_page = 0;
#ifdef RESA_DEBUG_CHECKS
  int raw_blk = 0, raw_page = 0;
#endif
  if (lane * kDecWaves < a.bps) {
    const int pos = min(first + wave + kDecWaves * lane, a.n_cap - 1);
    my_blk = min(max(a.idx[gi * a.n_cap + pos], 0), c.maxb - 1);
    my_page = min(max(c.bt[size_t(b) * c.maxb + my_blk], 0), c.num_pages - 1);
#ifdef RESA_DEBUG_CHECKS
    raw_blk = a.idx[gi * a.n_cap + pos];
    raw_page = c.bt[size_t(b) * c.maxb + my_blk];
#endif
  }
  const int n = a.count[b];
  const int L = c.seq_lens[b];
#ifdef RESA_DEBUG_CHECKS
  {  // the indices above are clamped into their arrays whatever they hold; here they are only checked
    const int M = (L + kBlock - 1) / kBlock;
    RESA_CHECK(c.dbg, L >= 0 && L <= c.max_seq_len, kChkSeqLen, (void)0);
    RESA_CHECK(c.dbg, L >= 1, kChkEmpty, (void)0);
    RESA_CHECK(c.dbg, n >= 0 && n <= a.n_cap, kChkSelection, (void)0);
    if (lane * kDecWaves < a.bps && first + wave + kDecWaves * lane < min(n, a.n_cap)) {
      RESA_CHECK(c.dbg, raw_blk >= 0 && raw_blk < M, kChkSelection, (void)0);
      RESA_CHECK(c.dbg, raw_page >= 0 && raw_page < c.num_pages, kChkPage, (void)0);
    }
  }
#endif
  uint4 qk[KS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (size_t(b) * c.Hq + size_t(g) * G + (h < G ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * j);
      qk[ks] = h < G ? x : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const uint16_t* kbase = static_cast<const uint16_t*>(c.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(c.v);
  auto tile = [&](const uint16_t* base, int page) { return base + (size_t(page) * c.Hkv + g) * kBlock * D; };
  // NB rotating buffers: block it in one, blocks it + 1 .. it + NB - 1 loading
  MfmaBlock<D> buf[NB];
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    const int pu = __builtin_amdgcn_readlane(my_page, u);
    buf[u].load(tile(kbase, pu), tile(vbase, pu), lane);
  }
  const int nblk = min(a.bps, n - first);
  if (nblk <= 0) return;
  const int nw = nblk > wave ? (nblk - wave + kDecWaves - 1) / kDecWaves : 0;

  float m = -__builtin_inff(), lsum = 0.f;
  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t ones = 0x3F803F80u;  // bf16 pair (1, 1)

  auto step = [&](int it, MfmaBlock<D>& cur, MfmaBlock<D>& spare) {
    if (it + NB - 1 < nw) {
      const int np = __builtin_amdgcn_readlane(my_page, it + NB - 1);
      spare.load(tile(kbase, np), tile(vbase, np), lane);
    }
    const int blk = __builtin_amdgcn_readlane(my_blk, it);
    const int valid = min(kBlock, L - blk * kBlock);
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[ks]),
                                                    __builtin_bit_cast(bf16x8_t, qk[ks]), sc, 0, 0, 0);
    if (valid < kBlock) {  // wave-uniform: slots past the sequence end may hold anything
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * j + r >= valid) sc[r] = -__builtin_inff();
      const uint32_t m0 = (4 * j + 0 < valid ? 0x0000ffffu : 0u) | (4 * j + 1 < valid ? 0xffff0000u : 0u);
      const uint32_t m1 = (4 * j + 2 < valid ? 0x0000ffffu : 0u) | (4 * j + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        cur.v[dt].x &= m0;
        cur.v[dt].y &= m1;
      }
    }
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.scale_log2;
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    // the running max moves only on a jump of more than 2^8; numerator and
    // denominator share every rescale
    if (__builtin_amdgcn_ballot_w64(bm > m + kLazyRescale)) {
      if (bm > m + kLazyRescale) {
        const float alpha = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - bm);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        lsum *= alpha;
        m = bm;
      }
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      p[r] = sc[r] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2, -m));
    // p as the bf16 pair hi + lo (hi = bf16(p), lo = bf16(p - hi): about 16
    // significant bits), so a row whose weight sits on a few keys keeps its
    // accuracy; the denominator sums the same hi + lo values
    const f32x2_t p01 = {p[0], p[1]}, p23 = {p[2], p[3]};
    const uint32_t w01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2_t));
    const uint32_t w23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2_t));
    const f32x2_t l01 = {p[0] - bf16_lo(w01), p[1] - bf16_hi(w01)}, l23 = {p[2] - bf16_lo(w23), p[3] - bf16_hi(w23)};
    const uint32_t x01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(l01, bf16x2_t));
    const uint32_t x23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(l23, bf16x2_t));
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w01), __builtin_bit_cast(bf16x2_t, ones), lsum,
                                           false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w23), __builtin_bit_cast(bf16x2_t, ones), lsum,
                                           false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x01), __builtin_bit_cast(bf16x2_t, ones), lsum,
                                           false);
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x23), __builtin_bit_cast(bf16x2_t, ones), lsum,
                                           false);
    // One 16x16x32 MFMA per channel tile takes both halves: lane (h, j)
    // supplies k = 8 j + [0, 8) as (hi of tokens 4 j .. 4 j + 3, lo of the same
    // tokens) in B, and the A operand repeats its V piece of those four tokens,
    // so O^T += V^T P_hi^T + V^T P_lo^T in one instruction.
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, make_uint4(w01, w23, x01, x23));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 vp = cur.v[dt];
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, make_uint4(vp.x, vp.y, vp.x, vp.y)),
                                                      pb, o[dt], 0, 0, 0);
    }
  };

  for (int it0 = 0; it0 < nw; it0 += NB) {
    bool done = false;
    static_for<0, NB>([&](auto U) {
      constexpr int u = U.value;
      if (!done) {
        if (it0 + u >= nw) {
          done = true;
        } else {
          step(it0 + u, buf[u], buf[(u + NB - 1) % NB]);
        }
      }
    });
  }

  // wave state -> LDS: lane (h, j) holds O^T rows 16 dt + 4 j + r of head h
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (h < G) {
    if (j == 0) {
      sm.m[wave][h] = nw > 0 ? m : -__builtin_inff();
      sm.l[wave][h] = nw > 0 ? lsum : 0.f;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.acc[wave][h][16 * dt + 4 * j + r] = o[dt][r];
  }
  __syncthreads();
  const size_t part = gi * a.splits + s;
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int hh = i / D, ch = i % D;
    float mx = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, sm.m[w][hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = sm.m[w][hh];
      const float e = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - mx);
      num = fmaf(e, sm.acc[w][hh][ch], num);
      den = fmaf(e, sm.l[w][hh], den);
    }
    a.part_acc[(part * G + hh) * D + ch] = num;
    if (ch == 0) {
      a.part_ml[(part * G + hh) * 2 + 0] = mx;
      a.part_ml[(part * G + hh) * 2 + 1] = den;
    }
  }
}

// grid: x = KV head, y = sequence; 256 threads: merge a group's splits. Each
// thread owns (head, channel) outputs; the partials of up to 16 splits are
// requested in one batch before any is used, merged with log-sum-exp weights.
constexpr int kCombThreads = 256;

// Merge the splits of one query head: grid (KV head, sequence, head of the
// group), 256 threads. Thread (part, channel) folds every (256 / D)-th split
// of its channel into a running (max, numerator, denominator), requesting the
// splits' (m, l) and partials in batches of 16 before any is used, so a batch
// costs one round trip; the parts are then merged through LDS with the same
// log-sum-exp weights.
template <typename T, int D, int G>
__global__ __launch_bounds__(kCombThreads) void k_decode_combine(DecodeArgs a, void* __restrict__ out) {
  constexpr int PARTS = kCombThreads / D;
  constexpr int BATCH = 16;
  __shared__ float pm[PARTS][D], pnum[PARTS][D], pden[PARTS][D];
  const CacheView& c = a.c;
  const int g = blockIdx.x, b = blockIdx.y, h = blockIdx.z, tid = threadIdx.x;
  const size_t gi = size_t(b) * c.Hkv + g;
  // a count above n_cap (a caller's mistake) would name splits past the
  // partials of this group
  const int live = (min(a.count[b], a.n_cap) + a.bps - 1) / a.bps;
  const int ch = tid % D, part = tid / D;  // part is wave-uniform
  const float* ml = a.part_ml + (gi * a.splits * G + h) * 2;         // split sp at ml[sp * G * 2]
  const float* acc = a.part_acc + (gi * a.splits * G + h) * D + ch;  // split sp at acc[sp * G * D]
  float mx = -__builtin_inff(), num = 0.f, den = 0.f;
  for (int sp0 = part; sp0 < live; sp0 += PARTS * BATCH) {
    float mv[BATCH], lv[BATCH], av[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int sp = sp0 + u * PARTS;
      const int sc = sp < live ? sp : part;  // past the live splits: re-read this part's first
      mv[u] = ml[size_t(sc) * G * 2];
      lv[u] = ml[size_t(sc) * G * 2 + 1];
      av[u] = acc[size_t(sc) * G * D];
    }
    // the batch's maximum first, one rescale, then independent weights
    float bm = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (sp0 + u * PARTS >= live) mv[u] = -__builtin_inff();
      bm = fmaxf(bm, mv[u]);
    }
    if (bm > mx) {  // wave-uniform
      const float sc = mx == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mx - bm);
      num *= sc;
      den *= sc;
      mx = bm;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float e = mv[u] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mv[u] - mx);
      num = fmaf(e, av[u], num);
      den = fmaf(e, lv[u], den);
    }
  }
  pm[part][ch] = mx;
  pnum[part][ch] = num;
  pden[part][ch] = den;
  __syncthreads();
  if (part == 0) {
    float m = pm[0][ch];
#pragma unroll
    for (int q = 1; q < PARTS; ++q) m = fmaxf(m, pm[q][ch]);
    float t = 0.f, d = 0.f;
#pragma unroll
    for (int q = 0; q < PARTS; ++q) {
      const float e = pm[q][ch] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(pm[q][ch] - m);
      t = fmaf(e, pnum[q][ch], t);
      d = fmaf(e, pden[q][ch], d);
    }
    store_out<T>(out, (size_t(b) * c.Hq + size_t(g) * G + h) * D + ch, t / d);
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a, void* out, hipStream_t st) {
  const CacheView& c = a.c;
  dim3 grid(a.splits, c.Hkv, c.B);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((k_decode_mfma<D, G, kDecBuffers>), grid, dim3(kDecThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode<float, D, G>), grid, dim3(kDecThreads), 0, st, a);
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
  p.splits = (n_cap + bps - 1) / bps;  // <= 512: bps >= ceil(work / 512) >= n_cap / 512
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
