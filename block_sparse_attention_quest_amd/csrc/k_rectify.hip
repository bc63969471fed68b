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
#include <type_traits>

#include "resa_internal.h"

namespace resa {
namespace {

struct RectArgs {
  CacheView c;
  const void* q;  // [B][f][Hq][D]
  int f, rows, rows_pad, target, cap;
  float scale_log2;
  int4* items;      // [cap] work items: (sequence, KV head, first key, end key)
  int2* groups;     // [B * Hkv] (first item, item count) of every (sequence, KV head)
  int* nitems;      // [1]
  float* part_ml;   // [cap][rows_pad][2]
  float* part_acc;  // [cap][rows_pad][D]
};

// Work plan of one rectification, built on the device from seq_lens: every
// (sequence, KV head) is cut into key ranges of one common length (a multiple
// of the key tile), chosen so that all items together make about `target`
// workgroups, i.e. one full round over the chip whatever the mix of lengths.
// Items of one (sequence, KV head) are consecutive. 1 workgroup.
__global__ __launch_bounds__(256) void k_rect_plan(RectArgs a) {
  const CacheView& c = a.c;
  __shared__ int chunk_s;
  if (threadIdx.x == 0) {
    long total = 0;
    for (int b = 0; b < c.B; ++b) total += c.seq_lens[b];
    total *= c.Hkv;
    long chunk = (total + a.target - 1) / a.target;
    chunk = (chunk + kRectTileKeys - 1) / kRectTileKeys * kRectTileKeys;
    if (chunk < 256) chunk = 256;
    if (chunk > 16384) chunk = 16384;
    int base = 0;
    for (int b = 0; b < c.B; ++b) {
      const int nb = (c.seq_lens[b] + int(chunk) - 1) / int(chunk);
      for (int g = 0; g < c.Hkv; ++g) {
        a.groups[b * c.Hkv + g] = make_int2(base, nb);
        base += nb;
      }
    }
    a.nitems[0] = base;
    chunk_s = int(chunk);
  }
  __syncthreads();
  const int chunk = chunk_s;
  for (int bg = threadIdx.x; bg < c.B * c.Hkv; bg += blockDim.x) {
    const int b = bg / c.Hkv, g = bg % c.Hkv;
    const int2 gr = a.groups[bg];
    const int L = c.seq_lens[b];
    for (int sp = 0; sp < gr.y; ++sp)
      a.items[gr.x + sp] = make_int4(b, g, sp * chunk, min(L, (sp + 1) * chunk));
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const void* global_ptr_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A 16-byte zero piece: the source of every tile piece that lies past the end of
// the keys, so that such LDS slots hold zeros rather than whatever the cache
// slot holds.
__device__ uint4 kZeroPiece[1];

// Wait until at most N vector-memory instructions of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt(((N >> 4) & 3) << 14 | (0xF << 8) | (7 << 4) | (N & 15));
}

constexpr int kMaxChunkPages = 1024;  // keys per split <= 16384

// Tile stages live in separate LDS arrays, one per stage, and the tile loop is
// unrolled by the stage count, so every access names one array at compile time.
// The compiler can then tell that reading one stage does not depend on the
// direct-to-LDS loads still in flight into the others.
//   K stage: [32 keys][D/8 pieces of 8 channels]; piece c of key r sits at
//            position c ^ (r % (D/8)) of its row (XOR swizzle: the 32 rows read
//            at one column by an MFMA operand load hit distinct banks).
//   V stage: [4 groups of 8 keys][D channels] pieces; piece (q, ch) holds channel
//            ch of keys 8q .. 8q + 7 (V page tiles are channel-major in HBM).
#define RESA_STAGE_DECL(i) __shared__ uint4 sk##i[PIECES], sv##i[PIECES]
template <int S>
__device__ __forceinline__ uint4* pick(uint4* a0, uint4* a1, uint4* a2, uint4* a3, uint4* a4, uint4* a5,
                                       uint4* a6, uint4* a7) {
  if constexpr (S == 0) return a0;
  else if constexpr (S == 1) return a1;
  else if constexpr (S == 2) return a2;
  else if constexpr (S == 3) return a3;
  else if constexpr (S == 4) return a4;
  else if constexpr (S == 5) return a5;
  else if constexpr (S == 6) return a6;
  else return a7;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// grid: x = work item (see k_rect_plan); NWV waves. Wave w owns query rows
// 32w .. 32w + 31 (a wave past G * f rows only loads). NS tile stages.
template <int D, int NWV, int NS>
__global__ __launch_bounds__(64 * NWV, 2) void k_rect_mfma(RectArgs a) {
  constexpr int NT = 64 * NWV;
  constexpr int KSTEPS = D / 16;   // 16-deep k-steps of the score product
  constexpr int DT = D / 32;       // 32-wide output column tiles
  constexpr int CPR = D / 8;       // pieces per K row
  constexpr int PIECES = kRectTileKeys * D / 8;  // per tile, K and V each
  constexpr int INSTR = 2 * PIECES / 64;         // wave-wide loads per tile
  constexpr int LPT = INSTR / NWV;               // loads per thread per tile
  static_assert(INSTR % NWV == 0, "tile loads must split evenly over the waves");
  static_assert(NS >= 2 && NS <= 8, "2 .. 8 stages");
  constexpr float kLazy = 8.0f;    // log2 units
  RESA_STAGE_DECL(0); RESA_STAGE_DECL(1); RESA_STAGE_DECL(2); RESA_STAGE_DECL(3);
  RESA_STAGE_DECL(4); RESA_STAGE_DECL(5); RESA_STAGE_DECL(6); RESA_STAGE_DECL(7);
  __shared__ int pages[kMaxChunkPages];
  const CacheView& c = a.c;
  const int item = blockIdx.x;
  if (item >= a.nitems[0]) return;
  const int4 it = a.items[item];
  const int b = it.x, g = it.y, key_lo = it.z, key_hi = it.w;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = c.seq_lens[b];
  const int ntiles = (key_hi - key_lo + kRectTileKeys - 1) / kRectTileKeys;
  const int G = c.G;
  const int col = lane & 31, half = lane >> 5;
  const bool has_rows = wave * 32 < a.rows;  // wave-uniform
  const int first_masked = L - a.f;          // keys from here on are seen by some rows only

  // page ids of the chunk
  const int page0 = key_lo >> 4;
  const int npages = (key_hi - 1) / kBlock - page0 + 1;
  for (int i = tid; i < npages; i += NT) pages[i] = c.bt[size_t(b) * c.maxb + page0 + i];

  // this lane's query row as MFMA B operands (S^T = K Q^T)
  bf16x8_t qreg[KSTEPS];
  int limit;  // last key position the row may see (-1: padding row)
  {
    const int r = wave * 32 + col;
    const bool live = r < a.rows;
    const int i = r / G, h = r % G;
    limit = live ? L - a.f + i : -1;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((size_t(b) * a.f + (live ? i : 0)) * c.Hq + size_t(g) * G + (live ? h : 0)) * D;
    // a padding row reads row 0: all of its keys are masked and it writes nothing
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16 + 8 * half));
  }
  wait_vmcnt<0>();  // query rows and page ids are in before any tile load is issued
  __syncthreads();  // page ids visible

  const uint16_t* kb = static_cast<const uint16_t*>(c.k);
  const uint16_t* vb = static_cast<const uint16_t*>(c.v);
  // Issue the LPT direct-to-LDS loads of tile ti into the given stage arrays.
  auto issue_tile = [&](int ti, uint4* kst, uint4* vst) {
    const int base = key_lo + ti * kRectTileKeys;
#pragma unroll
    for (int li = 0; li < LPT; ++li) {
      const int ins = li * NWV + wave;  // wave-uniform
      const void* src;
      uint4* dst;
      if (ins < INSTR / 2) {  // K pieces
        const int pidx = ins * 64 + lane;
        const int key = pidx / CPR, cpos = pidx % CPR;
        const int cl = cpos ^ (key % CPR);
        const int kg = base + key;
        src = kg < key_hi ? static_cast<const void*>(
                                kb + ((size_t(pages[(kg >> 4) - page0]) * c.Hkv + g) * kBlock + (kg & 15)) * D + cl * 8)
                          : static_cast<const void*>(kZeroPiece);
        dst = kst + ins * 64;
      } else {  // V pieces
        const int pidx = (ins - INSTR / 2) * 64 + lane;
        const int q = pidx / D, ch = pidx % D;
        const int t0 = base + 8 * q;
        src = t0 < key_hi ? static_cast<const void*>(
                                vb + ((size_t(pages[(t0 >> 4) - page0]) * c.Hkv + g) * D + ch) * kBlock + (t0 & 15))
                          : static_cast<const void*>(kZeroPiece);
        dst = vst + (ins - INSTR / 2) * 64;
      }
      __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)dst, 16, 0, 0);
    }
  };

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m = -__builtin_inff(), lsum = 0.f;

  auto compute = [&](int ti, const uint4* kst, const uint4* vst) {
    const int base = key_lo + ti * kRectTileKeys;
    f32x16_t sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    bf16x8_t ak[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      ak[ks] = __builtin_bit_cast(bf16x8_t, kst[col * CPR + ((2 * ks + half) ^ (col % CPR))]);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], qreg[ks], sacc, 0, 0, 0);
    // lane holds keys base + 8 (r/4) + 4 half + r%4 of query row `col`
    float x[16];
    if (base + kRectTileKeys > first_masked || base + kRectTileKeys > key_hi) {  // wave-uniform
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = base + 8 * (r / 4) + 4 * half + (r % 4);
        x[r] = (key < key_hi && key <= limit) ? sacc[r] * a.scale_log2 : -__builtin_inff();
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = limit >= 0 ? sacc[r] * a.scale_log2 : -__builtin_inff();
    }
    float tmax = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, x[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // the running max moves only when a logit exceeds it by more than 2^8;
    // numerator and denominator share every rescale
    if (__builtin_amdgcn_ballot_w64(tmax > m + kLazy)) {
      const float mnew = fmaxf(m, tmax);
      const float alpha = m == -__builtin_inff() ? (mnew == -__builtin_inff() ? 1.f : 0.f)
                                                 : __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
      m = mnew;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = x[r] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(x[r] - m);
      lsum += p[r];
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      uint32_t w[4];
#pragma unroll
      for (int x2 = 0; x2 < 4; ++x2) {
        const f32x2_t pr = {p[8 * k2 + 2 * x2], p[8 * k2 + 2 * x2 + 1]};
        w[x2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
      }
      pb[k2] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        // keys 16 k2 + 4 half + [0, 4) from group 2 k2, + 8 from group 2 k2 + 1
        const uint2 lo = reinterpret_cast<const uint2*>(&vst[(2 * k2) * D + t * 32 + col])[half];
        const uint2 hi = reinterpret_cast<const uint2*>(&vst[(2 * k2 + 1) * D + t * 32 + col])[half];
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[k2], o[t], 0, 0, 0);
      }
    }
  };

  // Pipeline: NS - 1 tiles are in flight. At step t the wave waits for its own
  // loads of tile t, a barrier makes everyone's visible, tile t + NS - 1 is
  // requested into the stage tile t - 1 used (every wave finished computing it
  // before this barrier), and tile t is computed.
  static_for<0, NS - 1>([&](auto S) {
    if (S.value < ntiles)
      issue_tile(S.value, pick<S.value>(sk0, sk1, sk2, sk3, sk4, sk5, sk6, sk7),
                 pick<S.value>(sv0, sv1, sv2, sv3, sv4, sv5, sv6, sv7));
  });
  for (int t0 = 0; t0 < ntiles; t0 += NS) {
    static_for<0, NS>([&](auto S) {
      const int t = t0 + S.value;
      if (t >= ntiles) return;
      constexpr int SN = (S.value + NS - 1) % NS;  // stage of tile t + NS - 1
      uint4* kcur = pick<S.value>(sk0, sk1, sk2, sk3, sk4, sk5, sk6, sk7);
      uint4* vcur = pick<S.value>(sv0, sv1, sv2, sv3, sv4, sv5, sv6, sv7);
      const int ahead = min(NS - 2, ntiles - 1 - t);  // tiles after t already requested
      if (ahead >= NS - 2) wait_vmcnt<(NS - 2) * LPT>();
      else if (ahead <= 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<LPT>();
      else if (ahead == 2) wait_vmcnt<2 * LPT>();
      else if (ahead == 3) wait_vmcnt<3 * LPT>();
      else if (ahead == 4) wait_vmcnt<4 * LPT>();
      else wait_vmcnt<0>();
      // Every wave has its own loads of tile t complete; the bare barrier (no
      // fence) then makes the whole tile visible without draining the loads of
      // later tiles that are still in flight. The memory clobber keeps the
      // compiler from moving LDS accesses across it.
      asm volatile("s_barrier" ::: "memory");
      if (t == ntiles - 1 && (key_hi & 7) != 0) {
        // the last V group holds keys past the end: zero them
        const int q = ((key_hi - key_lo) - t * kRectTileKeys) / 8;
        const int from = key_hi & 7;
        for (int ch = tid; ch < D; ch += NT) {
          uint16_t* e = reinterpret_cast<uint16_t*>(&vcur[q * D + ch]);
          for (int x2 = from; x2 < 8; ++x2) e[x2] = 0;
        }
        __syncthreads();
      }
      if (t + NS - 1 < ntiles)
        issue_tile(t + NS - 1, pick<SN>(sk0, sk1, sk2, sk3, sk4, sk5, sk6, sk7),
                   pick<SN>(sv0, sv1, sv2, sv3, sv4, sv5, sv6, sv7));
      if (has_rows) compute(t, kcur, vcur);
    });
  }

  // partials: lane holds O^T[dcol][row col] for dcol = 32t + 8(r/4) + 4 half + r%4
  if (!has_rows) return;
  const int r = wave * 32 + col;
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const size_t slot = size_t(item) * a.rows_pad + r;
  if (half == 0) {
    a.part_ml[slot * 2 + 0] = m;
    a.part_ml[slot * 2 + 1] = ltot;
  }
  float* dst = a.part_acc + slot * D;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(dst + t * 32 + 8 * q4 + 4 * half) =
          make_float4(o[t][4 * q4 + 0], o[t][4 * q4 + 1], o[t][4 * q4 + 2], o[t][4 * q4 + 3]);
}
#undef RESA_STAGE_DECL

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
  const int2 gr = a.groups[size_t(b) * c.Hkv + g];
  const int live = gr.y;
  float mx = -__builtin_inff();
  for (int sp = lane; sp < live; sp += 64) mx = fmaxf(mx, a.part_ml[((size_t(gr.x) + sp) * a.rows_pad + r) * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float num[D / 64], den = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) num[e] = 0.f;
  for (int sp = 0; sp < live; ++sp) {
    const size_t slot = (size_t(gr.x) + sp) * a.rows_pad + r;
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

template <int D, int NWV, int NS>
hipError_t launch_mfma_t(const RectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_rect_mfma<D, NWV, NS>), dim3(a.cap), dim3(64 * NWV), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const RectArgs& a, void* out, hipStream_t st) {
  const CacheView& c = a.c;
  hipLaunchKernelGGL(k_rect_plan, dim3(1), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = a.rows_pad <= 128 ? launch_mfma_t<D, 4, 4>(a, st) : launch_mfma_t<D, 8, 8>(a, st);
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
  // one round of workgroups: two per CU with 4 waves (128 rows), one with 8
  p.target = p.rows_pad <= 128 ? 512 : 256;
  // items <= total / chunk + one per (sequence, KV head) while the chunk is not
  // clamped; a clamped chunk (16384 keys) gives at most ceil(L / 16384) each
  const int groups = c.B * c.Hkv;
  const int clamped = groups * ((c.max_seq_len + 16383) / 16384);
  p.cap = p.target + groups > clamped ? p.target + groups : clamped;
  return p;
}

static size_t plan_bytes(const CacheView& c, const RectPlan& p) {
  return align_up(size_t(p.cap) * sizeof(int4), 256) + align_up(size_t(c.B) * c.Hkv * sizeof(int2), 256) + 256;
}

size_t rectify_ws_bytes(const CacheView& c, int f) {
  const RectPlan p = plan_rectify(c, f);
  const size_t slots = size_t(p.cap) * p.rows_pad;
  return plan_bytes(c, p) + align_up(slots * 2 * sizeof(float), 256) + slots * c.D * sizeof(float);
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
  a.target = p.target;
  a.cap = p.cap;
  a.scale_log2 = scale * 1.4426950408889634f;
  char* w = static_cast<char*>(ws);
  a.items = reinterpret_cast<int4*>(w);
  w += align_up(size_t(p.cap) * sizeof(int4), 256);
  a.groups = reinterpret_cast<int2*>(w);
  w += align_up(size_t(c.B) * c.Hkv * sizeof(int2), 256);
  a.nitems = reinterpret_cast<int*>(w);
  w += 256;
  const size_t slots = size_t(p.cap) * p.rows_pad;
  a.part_ml = reinterpret_cast<float*>(w);
  a.part_acc = reinterpret_cast<float*>(w + align_up(slots * 2 * sizeof(float), 256));
  if (c.dtype == RESA_BF16) return c.D == 128 ? launch_mfma<128>(a, out, st) : launch_mfma<64>(a, out, st);
  dim3 grid(c.Hq, f, c.B);
  if (c.D == 128)
    hipLaunchKernelGGL((k_rect_valu<float, 128>), grid, dim3(64), 0, st, a, out);
  else
    hipLaunchKernelGGL((k_rect_valu<float, 64>), grid, dim3(64), 0, st, a, out);
  return hipGetLastError();
}

}  // namespace resa
