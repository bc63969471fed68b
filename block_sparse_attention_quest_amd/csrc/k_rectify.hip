// Dense rectification attention (Pith review of "Rectified Sparse Attention",
// "What carries the argument" and "The reading"): after the f newest positions
// of every sequence have been overwritten with their re-encoded K/V and their
// blocks' descriptors refreshed (the first launch of the call), row i of every
// query head attends causally over the whole cache, positions 0 .. L - f + i.
//
// bf16 path (k_rect_mfma): per KV head the G * f query rows form one dense
// contraction against every key, so it runs on the matrix cores
// (v_mfma_f32_32x32x16_bf16). The rows are cut into row tiles of 128 or 256
// (one wave per 32 rows); a row tile needs the keys up to the last position its
// last row sees. The key ranges of all (sequence, KV head, row tile) segments,
// laid end to end in tiles of 32 keys, are cut into one equal range per
// workgroup (the work plan, built by one workgroup of the first launch,
// k_rect_prep, beside the write and refresh), so a mixed-length batch still fills
// the chip evenly; a range that crosses from one segment into the next becomes
// two work items with a partial each. For an item the K/V tiles stream from HBM
// into LDS once and serve all G * f rows (HBM traffic is the cache once per
// event, not once per head); when the K/V the call may read exceeds the
// last-level cache, the tile loads are non-temporal. Each wave owns a 32-row tile of queries, kept in
// registers. Scores are computed transposed, S^T = K Q^T, so a lane holds 16
// keys of one query row and the probabilities feed O^T = V^T P^T as its B
// operand with no data movement. The rows of a K tile are stored in LDS in an
// order (bits 2 and 3 of the key index swapped) that makes the 8 keys a lane
// holds per 16-key step consecutive, so the V^T operand is a single 16-byte
// piece of the channel-major V page. Scores of tile t + 1 are issued to the
// matrix cores before the softmax of tile t, which then overlaps them. Partial
// (m, l, O) per row and item go to the workspace; a combine kernel merges the
// items of every (sequence, KV head) with log-sum-exp weights.
//
// fp32 path (k_rect_valu): one wave per (sequence, row, head), plain VALU.
#include <type_traits>

#include "refresh_block.h"

namespace resa {
namespace {

constexpr int kMaxItemTiles = 1024;  // tiles per workgroup range (32768 keys)

struct RectArgs {
  CacheView c;
  const void* q;  // [B][f][Hq][D]
  int f, rows, rows_pad;
  int tile_rows;  // rows per row tile (32 per wave of the launch)
  int rtiles;     // row tiles per (sequence, KV head)
  int target;     // workgroups aimed for: one round over the chip
  int slots;      // workgroups launched (>= what any plan uses)
  float scale_log2;
  int4* items;    // [slots + B * Hkv * rtiles] (sequence, KV head | row tile << 16, first key, end key)
  int2* groups;   // [B * Hkv * rtiles] (first item, item count) of every segment
  int* wg_first;  // [slots + 1] first item of every workgroup; the rest are nitems
  long long* ptile;  // [B] key tiles of the sequences before each one
  float* part_ml;   // [items][rows_pad][2]
  float* part_acc;  // [items][rows_pad][D]
};

__device__ __forceinline__ long long ceil_div_ll(long long x, long long y) { return (x + y - 1) / y; }

// Exclusive prefix sum over the workgroup (wave shuffles, then one pass over
// the wave totals); *total gets the sum of all values.
template <int NT>
__device__ long long block_exclusive_scan(long long v, long long* sh, long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  long long before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const long long t = sh[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Work plan of one rectification, built on the device from seq_lens.
// Segment s = (sequence b, KV head g, row tile rt) covers the key tiles up to
// the last position its last row sees, T_(b,rt) = ceil((L_b - f + i_last + 1) /
// 32) (the same for every g); segments in order (b, g, rt) make one line of
// TT tiles, split into P equal workgroup ranges at lo(w) = floor(w TT / P).
// P is the fewest whole rounds
// of the target count that keep every range within kMaxItemTiles (so all
// workgroups of a round finish together), and at most TT. Items are the pieces of the
// line cut at segment starts and range starts, in line order; the item that
// starts a range is that workgroup's first. Boundaries inside segment [a, e)
// are lo(w) for w in [ceil((a+1) P / TT), ceil(e P / TT) - 1]. Threads take
// contiguous runs of sequences, then of segments; consecutive boundaries are
// stepped without division (lo(w) = w q + floor(w r / P), TT = q P + r).
// NT threads of one workgroup build the plan.
// IN_LDS (batches up to kPlanLdsSeqs): lengths and tile prefixes stay in LDS,
// so the segment passes make no further global round trip; otherwise they are
// read back from the workspace and seq_lens.
constexpr int kPlanLdsSeqs = 1024;

template <int NT, bool IN_LDS>
__device__ __forceinline__ void rect_plan(const RectArgs& a) {
  const CacheView& c = a.c;
  __shared__ long long sh[NT / 64];
  __shared__ int s_len[IN_LDS ? kPlanLdsSeqs : 1];
  __shared__ long long s_pt[IN_LDS ? kPlanLdsSeqs : 1];
  const int tid = threadIdx.x;
  const long long Hkv = c.Hkv;
  const int RT = a.rtiles;
  // end key (exclusive) of row tile rt of a sequence of length L
  auto key_end = [&](int L, int rt) {
    const int r_last = min(a.rows, (rt + 1) * a.tile_rows) - 1;
    return max(1, L - a.f + r_last / c.G + 1);
  };
  auto rt_tiles = [&](int L, int rt) { return (long long)(key_end(L, rt) + kRectTileKeys - 1) / kRectTileKeys; };
  auto tiles_of = [&](int L) {  // all row tiles of one (sequence, KV head)
    long long t = 0;
    for (int rt = 0; rt < RT; ++rt) t += rt_tiles(L, rt);
    return t;
  };

  const int per_b = (c.B + NT - 1) / NT;
  const int b0 = min(c.B, tid * per_b), b1 = min(c.B, b0 + per_b);
  // a length read for the plan: checked builds clamp it into f .. max_seq_len,
  // so that the plan stays within the launch's workgroups and work items
  auto plan_len = [&](int b) {
    int L = checked_len(c, b);
    RESA_CHECK(c.dbg, L >= a.f, kChkRectF, L = max(L, a.f));
    return L;
  };
  long long tloc = 0;
  for (int b = b0; b < b1; ++b) {
    const int L = plan_len(b);
    if (IN_LDS) s_len[b] = L;
    tloc += tiles_of(L);
  }
  long long tsum;
  long long pt = block_exclusive_scan<NT>(tloc, sh, &tsum);
  for (int b = b0; b < b1; ++b) {
    if (IN_LDS)
      s_pt[b] = pt;
    else
      a.ptile[b] = pt;
    pt += tiles_of(IN_LDS ? s_len[b] : plan_len(b));
  }
  auto len_of = [&](int b) {
    if constexpr (IN_LDS) return s_len[b];
    else return plan_len(b);
  };
  auto ptile_of = [&](int b) {
    if constexpr (IN_LDS) return s_pt[b];
    else return a.ptile[b];
  };
  const long long TT = tsum * Hkv;
  // whole rounds of `target` workgroups, as few as keep ranges <= kMaxItemTiles
  long long P = a.target * ceil_div_ll(TT, (long long)a.target * kMaxItemTiles);
  if (P > TT) P = TT;
  const long long q = TT / P, r = TT % P;
  __syncthreads();  // lengths and prefixes visible to the workgroup

  const int S = c.B * c.Hkv * RT;
  const int per_s = (S + NT - 1) / NT;
  const int s0 = min(S, tid * per_s), s1 = min(S, s0 + per_s);
  // segment s: first tile, end tile, and the range starts strictly inside
  auto segment = [&](int s, long long& as, long long& es, long long& wl, long long& wh) {
    const int b = s / (c.Hkv * RT), g = (s / RT) % c.Hkv, rt = s % RT;
    const int L = len_of(b);
    long long before = 0;  // key tiles of the sequence's earlier row tiles
    for (int x = 0; x < rt; ++x) before += rt_tiles(L, x);
    as = ptile_of(b) * Hkv + g * tiles_of(L) + before;
    es = as + rt_tiles(L, rt);
    wl = ceil_div_ll((as + 1) * P, TT);
    wh = ceil_div_ll(es * P, TT) - 1;
  };
  long long cloc = 0;
  for (int s = s0; s < s1; ++s) {
    long long as, es, wl, wh;
    segment(s, as, es, wl, wh);
    cloc += 1 + (wh >= wl ? wh - wl + 1 : 0);
  }
  long long nitems;
  long long fi = block_exclusive_scan<NT>(cloc, sh, &nitems);
  for (int s = s0; s < s1; ++s) {
    long long as, es, wl, wh;
    segment(s, as, es, wl, wh);
    const int b = s / (c.Hkv * RT), g = (s / RT) % c.Hkv, rt = s % RT;
    const int kend = key_end(len_of(b), rt);
    const int cnt = 1 + int(wh >= wl ? wh - wl + 1 : 0);
    a.groups[s] = make_int2(int(fi), cnt);
    // the range that holds tile as starts exactly there: this item is its first
    const long long wprev = wl - 1;
    if (wprev * q + (wprev * r) / P == as) a.wg_first[wprev] = int(fi);
    long long lo_next = wl * q + (wl * r) / P, rem = (wl * r) % P;  // lo(wl)
    long long st = as;
    for (int j = 0; j < cnt; ++j) {
      const long long en = j == cnt - 1 ? es : lo_next;
      a.items[fi + j] = make_int4(b, g | (rt << 16), int((st - as) * kRectTileKeys),
                                  int(min((long long)kend, (en - as) * kRectTileKeys)));
      if (j > 0) a.wg_first[wl + j - 1] = int(fi + j);
      st = en;
      lo_next += q;
      rem += r;
      if (rem >= P) {
        lo_next += 1;
        rem -= P;
      }
    }
    fi += cnt;
  }
  for (long long w = P + tid; w <= a.slots; w += NT) a.wg_first[w] = int(nitems);
}

// The first launch of a bf16 rectification: the write of the f rectified rows
// and the refresh of their blocks' descriptors (one wave per (block slot, KV
// head, sequence), as resa_update_descriptors does), with the work plan built
// by one more workgroup, the first of an extra x column (the plan reads only
// the lengths, so the two are independent). grid (slots + 1, Hkv, B), 64
// threads.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_rect_prep(RectArgs a, const void* __restrict__ k_new,
                                                  const void* __restrict__ v_new) {
  if (blockIdx.x == gridDim.x - 1) {
    if (blockIdx.y == 0 && blockIdx.z == 0) {
      if (a.c.B <= kPlanLdsSeqs)
        rect_plan<64, true>(a);
      else
        rect_plan<64, false>(a);
    }
    return;
  }
  const CacheView& c = a.c;
  const int b = blockIdx.z, g = blockIdx.y, lane = threadIdx.x;
  int L = checked_len(c, b);
  RESA_CHECK(c.dbg, L >= a.f, kChkRectF, L = max(L, a.f));
  const int j = max(0, L - a.f) / kBlock + blockIdx.x;
  if (j * kBlock >= L) return;
  refresh_block<T, D>(c, k_new, v_new, a.f, b, g, j, L, lane);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Wait until this wave's LDS accesses are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((3 << 14) | (7 << 4) | 15); }

// Tile stages live in separate LDS arrays, one per stage, and the tile loop is
// unrolled by the stage count, so every access names one array at compile time.
// The compiler can then tell that reading one stage does not depend on the
// direct-to-LDS loads still in flight into the others.
// A stage array holds the K tile, then the V tile:
//   K tile: [32 rows][D/8 pieces of 8 channels]. Row i holds key pi(i), pi
//            swapping bits 2 and 3 of the index; piece c of a row sits at
//            position c ^ (i % (D/8)) (XOR swizzle: the 32 rows read at one
//            column by an MFMA operand load hit distinct banks).
//   V tile: [4 groups of 8 keys][D channels] pieces; piece (q, ch) holds channel
//            ch of keys 8q .. 8q + 7 (V page tiles are channel-major in HBM).
#define RESA_STAGE_DECL(i) __shared__ uint4 st##i[2 * PIECES]
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

// grid: x = workgroup range of the plan (slots); NWV waves. In an item of row
// tile rt, wave w owns query rows 32 (NWV rt + w) .. + 31 (a wave past the G * f
// rows only loads). NS tile stages. CPOL is the cache policy of the K/V tile
// loads (0, or kCachePolicyNT to stream them past the caches).
template <int D, int NWV, int NS, int CPOL>
__global__ __launch_bounds__(64 * NWV, 2) void k_rect_mfma(RectArgs a) {
  constexpr int NT = 64 * NWV;
  constexpr int KSTEPS = D / 16;   // 16-deep k-steps of the score product
  constexpr int DT = D / 32;       // 32-wide output column tiles
  constexpr int CPR = D / 8;       // pieces per K row
  constexpr int PIECES = kRectTileKeys * D / 8;  // per tile, K and V each
  constexpr int INSTR = 2 * PIECES / 64;         // wave-wide loads per tile
  constexpr int LPT = INSTR / NWV;               // loads per thread per tile
  constexpr int PAGE_BYTES = kBlock * D * 2;     // one KV head's K (or V) of a page
  static_assert(INSTR % NWV == 0 && (INSTR / NWV) % 2 == 0 || INSTR / NWV == 1,
                "tile loads must split evenly over the waves");
  static_assert(NS >= 4 && NS <= 8 && NS % 2 == 0, "4, 6 or 8 stages");
  constexpr float kLazy = 8.0f;    // log2 units
  RESA_STAGE_DECL(0); RESA_STAGE_DECL(1); RESA_STAGE_DECL(2); RESA_STAGE_DECL(3);
  RESA_STAGE_DECL(4); RESA_STAGE_DECL(5); RESA_STAGE_DECL(6); RESA_STAGE_DECL(7);
  __shared__ int2 tile_pages[kMaxItemTiles + 2 * NS];  // the two pages of each tile
  const CacheView& c = a.c;
  // the wave index is wave-uniform: from a scalar register, the per-wave
  // load constants below and the tile-load addresses stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int G = c.G;
  const int item_begin = a.wg_first[blockIdx.x], item_end = a.wg_first[blockIdx.x + 1];

  // Per-thread constants of the tile loads. Load li of a tile is one
  // wave-wide instruction; with two or more per thread the first half fill
  // the K stage and the rest the V stage, with one per thread the first half
  // of the waves take K.
  int ld_off[LPT];   // byte offset inside the page's K or V tile
  int ld_ph[LPT];    // which of the tile's two pages (wave-uniform)
  int ld_dst[LPT];   // first piece of the instruction in its stage array (wave-uniform)
  bool ld_k[LPT];    // wave-uniform; compile-time when LPT >= 2
#pragma unroll
  for (int li = 0; li < LPT; ++li) {
    int ins;
    if constexpr (LPT >= 2) {
      ld_k[li] = li < LPT / 2;
      ins = (li % (LPT / 2)) * NWV + wave;
    } else {
      ld_k[li] = wave < NWV / 2;
      ins = wave % (NWV / 2);
    }
    const int pidx = ins * 64 + lane;
    if (ld_k[li]) {
      const int i = pidx / CPR, cp = (pidx % CPR) ^ (i % CPR);
      const int kt = (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
      ld_off[li] = ((kt & 15) * D + cp * 8) * 2;
      ld_ph[li] = __builtin_amdgcn_readfirstlane(kt >> 4);  // a wave's rows share bit 4
    } else {
      const int q = pidx / D, ch = pidx % D;
      ld_off[li] = (ch * kBlock + 8 * (q & 1)) * 2;
      ld_ph[li] = __builtin_amdgcn_readfirstlane(q >> 1);  // a wave's pieces share q
    }
    ld_dst[li] = ins * 64;
  }
  const uint32_t ones = 0x3F803F80u;  // bf16 pair (1, 1)
  // LDS byte offsets of this lane's operand pieces inside a stage: K piece of
  // k-step ks, and the first V piece (the others are fixed strides from it)
  uint32_t koff_base[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) koff_base[ks] = (col * CPR + ((2 * ks + half) ^ (col % CPR))) * 16;
  const uint32_t voff_base = (half * D + col) * 16;

  for (int item = item_begin; item < item_end; ++item) {
    const int4 it = a.items[item];
    const int b = it.x, g = it.y & 0xffff, key_lo = it.z, key_hi = it.w;
    const int row0 = (it.y >> 16) * 32 * NWV;       // first row of the item's row tile
    const bool has_rows = row0 + wave * 32 < a.rows;  // wave-uniform
    int L = checked_len(c, b);
    RESA_CHECK(c.dbg, L >= a.f, kChkRectF, L = max(L, a.f));
    const int ntiles = (key_hi - key_lo + kRectTileKeys - 1) / kRectTileKeys;
    const int first_masked = L - a.f;  // keys from here on are seen by some rows only

    __syncthreads();  // the previous item is done with the page list and the stages
    // page ids of the item's tiles (two per tile) and of the tiles requested
    // past the end (the last page repeated)
    const int page0 = key_lo / kBlock, last = (key_hi - 1) / kBlock;
    // the pipeline reads the page ids of tiles up to one step past its last request
    const int nreq = (ntiles + NS - 1) / NS * NS + NS;
    for (int i = tid; i < nreq; i += NT)
      tile_pages[i] = make_int2(checked_page(c, b, min(page0 + 2 * i, last)),
                                checked_page(c, b, min(page0 + 2 * i + 1, last)));

    // this lane's query row as MFMA B operands (S^T = K Q^T)
    bf16x8_t qreg[KSTEPS];
    int limit;  // last key position the row may see (-1: padding row)
    {
      const int r = row0 + wave * 32 + col;
      const bool live = r < a.rows;
      const int i = r / G, h = r % G;
      limit = live ? L - a.f + i : -1;
      const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                             ((size_t(b) * a.f + (live ? i : 0)) * c.Hq + size_t(g) * G + (live ? h : 0)) * D;
      // a padding row reads row 0: it writes nothing that is read back
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        qreg[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16 + 8 * half));
    }
    wait_vmcnt<0>();  // query rows and page ids are in before any tile load is issued
    __syncthreads();  // page ids visible

    const char* kbase = static_cast<const char*>(c.k) + size_t(g) * PAGE_BYTES;
    const char* vbase = static_cast<const char*>(c.v) + size_t(g) * PAGE_BYTES;
    // a page's stride, Hkv K (or V) tiles; Hkv * D <= 4096 keeps it within 32
    // bits (at most 128 KiB), so a page's byte offset is one 32 x 32 -> 64-bit
    // scalar product of the (non-negative) page id and the stride
    const uint32_t pstride = uint32_t(c.Hkv) * PAGE_BYTES;
    // The two page ids of tile ti. In the loop they are read one step before
    // the tile's loads are issued, so that no step waits on an LDS round trip
    // before its loads go out.
    auto read_pages = [&](int ti) { return tile_pages[ti]; };
    // Issue the LPT direct-to-LDS loads of a tile (page ids pg) into the given
    // stage arrays. Every lane of a wave-wide load reads the same page, so the
    // page's address is scalar work and only the lane's 32-bit offset inside
    // it is a vector operand.
    auto issue_pages = [&](int2 pg, uint4* kst, uint4* vst) {
      const uint64_t o0 = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(pg.x))) * pstride;
      const uint64_t o1 = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(pg.y))) * pstride;
#pragma unroll
      for (int li = 0; li < LPT; ++li) {
        const bool isk = LPT >= 2 ? li < LPT / 2 : ld_k[li];
        const char* pbase = (isk ? kbase : vbase) + (ld_ph[li] ? o1 : o0);
        asm("" : "+s"(pbase));  // kept whole in scalar registers
        const char* src = pbase + uint32_t(ld_off[li]);
        uint4* dst = (isk ? kst : vst) + ld_dst[li];
        __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)dst, 16, 0, CPOL);
      }
    };

    f32x16_t o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float m = -__builtin_inff(), lsum = 0.f;
    // kept beside m, changed only by a rescale: the exponent offset -m (0
    // while m = -inf: such a row has seen only masked logits) and the raw
    // logit above which the running max moves, (m + kLazy) / scale_log2
    // (scale > 0)
    float nm = 0.f, thr = -__builtin_inff();

    // S^T tile of one stage: lane holds keys 16 (r / 8) + 8 half + r % 8 of
    // query row `col` (tile-relative key order after the row permutation).
    // The lane offsets pass through an empty asm at the top of every pass of
    // the pipelined loop, so the compiler adds them to each stage's base where
    // they are read instead of keeping a precomputed address per stage and
    // k-step live across the loop.
    auto score_operands = [&](bf16x8_t (&ak)[KSTEPS], const uint4* kst) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        ak[ks] = __builtin_bit_cast(bf16x8_t,
                                    *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(kst) + koff_base[ks]));
    };
    auto score = [&](f32x16_t& acc, const uint4* kst) {
      bf16x8_t ak[KSTEPS];
      score_operands(ak, kst);
      f32x16_t z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], qreg[0], z, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < KSTEPS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], qreg[ks], acc, 0, 0, 0);
    };

    auto rescale = [&](float tmax) {
      const float mnew = fmaxf(m, tmax);
      // m == -inf: nothing accumulated yet, o and lsum are zero
      const float alpha = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
      m = mnew;
      nm = m == -__builtin_inff() ? 0.f : -m;
      thr = (m + kLazy) / a.scale_log2;
    };

    // the logits are finite or -inf (masked), never NaN: the NaN-propagating
    // maximum needs no quieting of its operands
    auto half_max = [&](float x) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };

    // One pipeline step's work: the softmax of tile t (scores in sacc), the
    // score products of tile t + 1 (into snext, from K stage kst; past the end
    // a requested but unused tile), and the O^T update of tile t (V stage vst).
    // The exponentials and packing of tile t are interleaved one MFMA at a time
    // with the next tile's products, so the matrix cores and the VALU work
    // together within the wave.
    auto step_compute = [&](int t, f32x16_t& sacc, f32x16_t& snext, const uint4* kst, const uint4* vst) {
      bf16x8_t ak[KSTEPS];
      score_operands(ak, kst);
      const int base = key_lo + t * kRectTileKeys;
      // wave-uniform: the tile reaches the causal diagonal or the end
      const bool edge = base + kRectTileKeys > first_masked || base + kRectTileKeys > key_hi;
      if (edge) {
        int k0 = 8 * half;
        asm volatile("" : "+v"(k0));
        // highest key this lane's row may see, relative to the lane's first key
        const int vis = min(key_hi - 1, limit) - (base + k0);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 16 * (r / 8) + (r % 8) <= vis ? sacc[r] : -__builtin_inff();
      }
      float mx = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sacc[r]);
      const float hmax = half_max(mx);
      // the running max moves only when a logit exceeds it by more than 2^8;
      // numerator and denominator share every rescale
      if (__builtin_amdgcn_ballot_w64(hmax > thr)) rescale(hmax * a.scale_log2);
      f32x16_t z;
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = 0.f;
      snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[0], qreg[0], z, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < KSTEPS; ++ks)
        snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], qreg[ks], snext, 0, 0, 0);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], a.scale_log2, nm));
      bf16x8_t pb[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        uint32_t w[4];
#pragma unroll
        for (int x2 = 0; x2 < 4; ++x2) {
          const f32x2_t pr = {p[8 * k2 + 2 * x2], p[8 * k2 + 2 * x2 + 1]};
          w[x2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
          // the denominator sums the same rounded probabilities the product uses
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[x2]),
                                                 __builtin_bit_cast(bf16x2_t, ones), lsum, false);
        }
        pb[k2] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
      // interleave: each score product with a share of the softmax arithmetic
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 48 / KSTEPS, 0);    // then VALU
      }
      // Rows near the diagonal may see only a few keys, where one probability's
      // bf16 rounding is not averaged out; there p also goes in as the bf16
      // pair hi + lo (hi = bf16(p), lo = bf16(p - hi)), about 16 bits of p.
      bf16x8_t pl[2];
      if (edge) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          uint32_t w[4];
          const uint4 hw = __builtin_bit_cast(uint4, pb[k2]);
          const uint32_t hv[4] = {hw.x, hw.y, hw.z, hw.w};
#pragma unroll
          for (int x2 = 0; x2 < 4; ++x2) {
            const f32x2_t lr = {p[8 * k2 + 2 * x2] - __uint_as_float(hv[x2] << 16),
                                p[8 * k2 + 2 * x2 + 1] - __uint_as_float(hv[x2] & 0xffff0000u)};
            w[x2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lr, bf16x2_t));
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[x2]),
                                                   __builtin_bit_cast(bf16x2_t, ones), lsum, false);
          }
          pl[k2] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
      const uint4* vl = vst + (half * D + col);
#pragma unroll
      for (int tt = 0; tt < DT; ++tt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          // keys 16 k2 + 8 half + [0, 8): one piece of channel 32 tt + col
          const uint4 vv = vl[2 * k2 * D + tt * 32];
          o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pb[k2], o[tt], 0, 0, 0);
        }
      if (edge) {
#pragma unroll
        for (int tt = 0; tt < DT; ++tt)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const uint4 vv = vl[2 * k2 * D + tt * 32];
            o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pl[k2], o[tt], 0, 0, 0);
          }
      }
    };

    // Pipeline: NS - 1 tiles are requested ahead. At step t the wave waits for
    // its own loads of tile t + 1, a barrier makes everyone's visible, tile
    // t + NS - 1 is requested into the stage tile t - 1 used (every wave
    // finished tile t - 1 before this barrier), the scores of tile t + 1 go to
    // the matrix cores and tile t (scored one step earlier) is consumed. Every
    // step requests a tile, past the end one of the repeated last page (its
    // contents are never used), so each wait is a fixed count and the
    // compiler's own tracking of the loads sees every stage complete before it
    // is read, without adding waits of its own.
    f32x16_t s0, s1;
    static_for<0, NS - 1>([&](auto S) {
      issue_pages(read_pages(S.value), pick<S.value>(st0, st1, st2, st3, st4, st5, st6, st7),
                  pick<S.value>(st0, st1, st2, st3, st4, st5, st6, st7) + PIECES);
    });
    wait_vmcnt<(NS - 2) * LPT>();
    asm volatile("s_barrier" ::: "memory");
    if (has_rows) score(s0, st0);
    int2 pg_next = read_pages(NS - 1);
    for (int t0 = 0; t0 < ntiles; t0 += NS) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" : "+v"(koff_base[ks]));
      static_for<0, NS>([&](auto S) {
        const int t = t0 + S.value;
        constexpr int SN = (S.value + 1) % NS;       // stage of tile t + 1
        constexpr int SR = (S.value + NS - 1) % NS;  // stage of tile t + NS - 1
        // tiles t + 2 .. t + NS - 2 may stay in flight
        wait_vmcnt<(NS - 3) * LPT>();
        // Every wave has its own loads of tile t + 1 complete; the bare barrier
        // (no fence) then makes the whole tile visible without draining the
        // loads of later tiles that are still in flight. The memory clobber
        // keeps the compiler from moving LDS accesses across it.
        asm volatile("s_barrier" ::: "memory");
        const int kk = key_hi - (key_lo + t * kRectTileKeys);  // keys of tile t
        if (kk > 0 && kk < kRectTileKeys) {  // workgroup-uniform: the last tile is partial
          // its V slots past the end may hold anything (p is 0 there, but
          // 0 * NaN is not): zero them
          uint4* vz = pick<S.value>(st0, st1, st2, st3, st4, st5, st6, st7) + PIECES;
          for (int idx = tid; idx < 4 * D; idx += NT) {
            const int from = kk - 8 * (idx / D);  // valid keys in this piece
            if (from < 8) {
              uint16_t* e = reinterpret_cast<uint16_t*>(&vz[idx]);
              for (int x2 = from < 0 ? 0 : from; x2 < 8; ++x2) e[x2] = 0;
            }
          }
          wait_lgkm0();
          asm volatile("s_barrier" ::: "memory");
        }
        issue_pages(pg_next, pick<SR>(st0, st1, st2, st3, st4, st5, st6, st7),
                    pick<SR>(st0, st1, st2, st3, st4, st5, st6, st7) + PIECES);
        pg_next = read_pages(t + NS);  // the next step's tile
        if (has_rows && t < ntiles) {
          if constexpr (S.value % 2 == 0)
            step_compute(t, s0, s1, pick<SN>(st0, st1, st2, st3, st4, st5, st6, st7),
                         pick<S.value>(st0, st1, st2, st3, st4, st5, st6, st7) + PIECES);
          else
            step_compute(t, s1, s0, pick<SN>(st0, st1, st2, st3, st4, st5, st6, st7),
                         pick<S.value>(st0, st1, st2, st3, st4, st5, st6, st7) + PIECES);
        }
      });
    }
    wait_vmcnt<0>();  // the loads past the end land before the stages are reused

    // partials: lane holds O^T[dcol][row col] for dcol = 32t + 8(r/4) + 4 half + r%4
    if (has_rows) {
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
  }
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
// head, z = sequence; 256 threads, one wave per row (row R lies in row tile
// R / tile_rows). BATCH > 1: the build for plans whose segments hold many items
// each (few segments, so few waves: the batch's registers cost no occupancy
// that matters); BATCH = 1 keeps the registers, and the occupancy, of a batch
// with many segments.
template <typename T, int D, int BATCH>
__global__ __launch_bounds__(256) void k_rect_combine(RectArgs a, void* __restrict__ out) {
  const CacheView& c = a.c;
  const int b = blockIdx.z, g = blockIdx.y, lane = threadIdx.x & 63;
  const int R = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (R >= a.rows) return;
  const int r = R % a.tile_rows;  // the row's slot in its tile's partials
  const int2 gr = a.groups[(size_t(b) * c.Hkv + g) * a.rtiles + R / a.tile_rows];
  const int live = gr.y;
  float mx = -__builtin_inff();
  for (int sp = lane; sp < live; sp += 64) mx = fmaxf(mx, a.part_ml[((size_t(gr.x) + sp) * a.rows_pad + r) * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float num[D / 64], den = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) num[e] = 0.f;
  // With BATCH > 1 a row with more than 4 items requests its partials in
  // batches before any is used, one round trip per batch instead of one per
  // item (past the last item: the last one again, unused); otherwise items go
  // one by one.
  auto merge = [&](auto batch_c) {
    constexpr int NB = decltype(batch_c)::value;
    for (int sp0 = 0; sp0 < live; sp0 += NB) {
      float ms[NB], ls[NB], av[NB][D / 64];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const size_t slot = (size_t(gr.x) + min(sp0 + u, live - 1)) * a.rows_pad + r;
        ms[u] = a.part_ml[slot * 2];
        ls[u] = a.part_ml[slot * 2 + 1];
#pragma unroll
        for (int e = 0; e < D / 64; ++e) av[u][e] = a.part_acc[slot * D + lane + 64 * e];
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (sp0 + u >= live) break;  // wave-uniform
        const float w = ms[u] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms[u] - mx);
        den = fmaf(w, ls[u], den);
#pragma unroll
        for (int e = 0; e < D / 64; ++e) num[e] = fmaf(w, av[u][e], num[e]);
      }
    }
  };
  if (BATCH > 1 && live > 4)
    merge(std::integral_constant<int, BATCH>{});
  else
    merge(std::integral_constant<int, 1>{});
  const int i = R / c.G, h = R % c.G;
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
  int L = checked_len(c, b);
  RESA_CHECK(c.dbg, L >= a.f, kChkRectF, L = max(L, a.f));
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
      const int page = checked_page(c, b, t >> 4);
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
      const int page = checked_page(c, b, tt >> 4);
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
hipError_t launch_mfma_t(const RectArgs& a, bool stream, hipStream_t st) {
  if (stream)
    hipLaunchKernelGGL((k_rect_mfma<D, NWV, NS, kCachePolicyNT>), dim3(a.slots), dim3(64 * NWV), 0, st, a);
  else
    hipLaunchKernelGGL((k_rect_mfma<D, NWV, NS, 0>), dim3(a.slots), dim3(64 * NWV), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const RectArgs& a, const void* k_new, const void* v_new, void* out, hipStream_t st) {
  const CacheView& c = a.c;
  const int slots = (a.f + kBlock - 1) / kBlock + 1;  // blocks a range of f positions can touch
  hipLaunchKernelGGL((k_rect_prep<uint16_t, D>), dim3(slots + 1, c.Hkv, c.B), dim3(64), 0, st, a, k_new, v_new);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The K/V a call may read: when it is larger than the last-level cache, no
  // later call can find it there, so the tiles stream past the caches and leave
  // them to the block descriptors (the periodic rectification of long contexts:
  // 414 -> 395 us at 128K, batch 4); when it fits, the next call over the same
  // prefix (the next prefill chunk) reads it from there (streaming it cost the
  // 32K chunked prefill 9%).
  const size_t kv_bytes = size_t(c.B) * c.Hkv * c.max_seq_len * 2 * D * sizeof(uint16_t);
  const bool stream = kv_bytes > kLastLevelCacheBytes;
  e = a.tile_rows == 128 ? launch_mfma_t<D, 4, 4>(a, stream, st) : launch_mfma_t<D, 8, 8>(a, stream, st);
  if (e != hipSuccess) return e;
  // Segments with many items each (a prefill chunk: few segments over a round of
  // workgroups) take the batched merge: 12.8 -> 9.5 us per call for the 32K
  // prefill in chunks of 64; the mixed batch (about 2 items per segment, 8192
  // merge workgroups) keeps the lean one (28.3 us batched against 20.0).
  dim3 g2((a.rows + 3) / 4, c.Hkv, c.B);
  const long long segments = (long long)c.B * c.Hkv * a.rtiles;
  if (a.slots >= 24 * segments)
    hipLaunchKernelGGL((k_rect_combine<uint16_t, D, 16>), g2, dim3(256), 0, st, a, out);
  else
    hipLaunchKernelGGL((k_rect_combine<uint16_t, D, 1>), g2, dim3(256), 0, st, a, out);
  return hipGetLastError();
}

}  // namespace

RectPlan plan_rectify(const CacheView& c, int f) {
  RectPlan p;
  p.rows = c.G * f;
  // up to 128 rows: one tile of 4 waves; more: tiles of 256 rows (8 waves)
  p.tile_rows = p.rows <= 128 ? 128 : 256;
  p.rtiles = (p.rows + p.tile_rows - 1) / p.tile_rows;
  p.rows_pad = p.rtiles == 1 ? (p.rows + 31) / 32 * 32 : p.tile_rows;
  // one round of workgroups: two per CU with 4 waves, one with 8
  p.target = p.tile_rows == 128 ? 512 : 256;
  // the plan adds whole rounds of workgroups while a range would exceed
  // kMaxItemTiles tiles; the launch covers the largest cache the capacities allow
  const long long segments = (long long)c.B * c.Hkv * p.rtiles;
  const long long tt_max = segments * ((c.max_seq_len + kRectTileKeys - 1) / kRectTileKeys);
  const long long rounds = (tt_max + (long long)p.target * kMaxItemTiles - 1) / ((long long)p.target * kMaxItemTiles);
  p.slots = int(p.target * (rounds > 0 ? rounds : 1));
  p.cap = p.slots + int(segments);  // items: one per range plus one per segment
  return p;
}

static size_t plan_bytes(const CacheView& c, const RectPlan& p) {
  return align_up(size_t(p.cap) * sizeof(int4), 256) + align_up(size_t(c.B) * c.Hkv * p.rtiles * sizeof(int2), 256) +
         align_up(size_t(p.slots + 1) * sizeof(int), 256) + align_up(size_t(c.B) * sizeof(long long), 256);
}

size_t rectify_ws_bytes(const CacheView& c, int f) {
  const RectPlan p = plan_rectify(c, f);
  const size_t slots = size_t(p.cap) * p.rows_pad;
  return plan_bytes(c, p) + align_up(slots * 2 * sizeof(float), 256) + slots * c.D * sizeof(float);
}

hipError_t launch_rectify(const CacheView& c, const void* q, const void* k_new, const void* v_new, int f,
                          float scale, void* out, void* ws, hipStream_t st) {
  const RectPlan p = plan_rectify(c, f);
  RectArgs a;
  a.c = c;
  a.q = q;
  a.f = f;
  a.rows = p.rows;
  a.rows_pad = p.rows_pad;
  a.tile_rows = p.tile_rows;
  a.rtiles = p.rtiles;
  a.target = p.target;
  a.slots = p.slots;
  a.scale_log2 = scale * 1.4426950408889634f;
  char* w = static_cast<char*>(ws);
  a.items = reinterpret_cast<int4*>(w);
  w += align_up(size_t(p.cap) * sizeof(int4), 256);
  a.groups = reinterpret_cast<int2*>(w);
  w += align_up(size_t(c.B) * c.Hkv * p.rtiles * sizeof(int2), 256);
  a.wg_first = reinterpret_cast<int*>(w);
  w += align_up(size_t(p.slots + 1) * sizeof(int), 256);
  a.ptile = reinterpret_cast<long long*>(w);
  w += align_up(size_t(c.B) * sizeof(long long), 256);
  const size_t slots = size_t(p.cap) * p.rows_pad;
  a.part_ml = reinterpret_cast<float*>(w);
  a.part_acc = reinterpret_cast<float*>(w + align_up(slots * 2 * sizeof(float), 256));
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_mfma<128>(a, k_new, v_new, out, st) : launch_mfma<64>(a, k_new, v_new, out, st);
  // fp32: the write and refresh, then the plain rows
  const hipError_t e = launch_update_tail(c, k_new, v_new, f, st);
  if (e != hipSuccess) return e;
  dim3 grid(c.Hq, f, c.B);
  if (c.D == 128)
    hipLaunchKernelGGL((k_rect_valu<float, 128>), grid, dim3(64), 0, st, a, out);
  else
    hipLaunchKernelGGL((k_rect_valu<float, 64>), grid, dim3(64), 0, st, a, out);
  return hipGetLastError();
}

}  // namespace resa
