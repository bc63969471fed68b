// Block descriptors: per block of 16 tokens and per KV head, the channel-wise
// min and max of the keys over the block's valid tokens (the Quest-style block
// statistics of the Pith review of "Rectified Sparse Attention", section "What
// carries the argument"). Exact: min/max never round, so the stored values are
// keys from the cache.
//
// One wave per (sequence, block, KV head). A token row of head_dim elements is
// read by the 64 lanes in one coalesced access (lane owns head_dim/64 channels),
// so a block costs 16 row reads of 128-512 bytes and one 2-row descriptor write.
// The same kernel performs the append: tokens in the refreshed range come from
// k_new/v_new, are stored into their page (K token-major, V channel-major), and
// enter the min/max directly.
#include "refresh_block.h"

namespace resa {
namespace {

// blockIdx: x = block slot within the refreshed range, y = KV head, z = sequence.
// n_new == 0: rebuild (slot = logical block index, nothing written). NEW: rows
// come from k_new / v_new (false when the caller passes none).
template <typename T, int D, bool NEW>
__global__ __launch_bounds__(64) void k_refresh_blocks(CacheView c, const void* __restrict__ k_new,
                                                       const void* __restrict__ v_new, int n_new) {
  const int b = blockIdx.z, g = blockIdx.y, lane = threadIdx.x;
  const int L = checked_len(c, b);
  const int lo = n_new > 0 ? max(0, L - n_new) : 0;
  const int j = lo / kBlock + blockIdx.x;
  if (j * kBlock >= L) return;
  refresh_block<T, D, NEW>(c, k_new, v_new, n_new, b, g, j, L, lane);
}

template <typename T, int D>
hipError_t launch_refresh_t(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                            hipStream_t s) {
  const int slots = n_new > 0 ? (n_new + kBlock - 1) / kBlock + 1 : c.maxb;
  dim3 grid(slots, c.Hkv, c.B);
  if (n_new > 0 && k_new != nullptr)
    hipLaunchKernelGGL((k_refresh_blocks<T, D, true>), grid, dim3(64), 0, s, c, k_new, v_new, n_new);
  else
    hipLaunchKernelGGL((k_refresh_blocks<T, D, false>), grid, dim3(64), 0, s, c, k_new, v_new, n_new);
  return hipGetLastError();
}

hipError_t launch_refresh(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                          hipStream_t s) {
  if (c.dtype == RESA_BF16)
    return c.D == 128 ? launch_refresh_t<uint16_t, 128>(c, k_new, v_new, n_new, s)
                      : launch_refresh_t<uint16_t, 64>(c, k_new, v_new, n_new, s);
  return c.D == 128 ? launch_refresh_t<float, 128>(c, k_new, v_new, n_new, s)
                    : launch_refresh_t<float, 64>(c, k_new, v_new, n_new, s);
}

}  // namespace

hipError_t launch_update_tail(const CacheView& c, const void* k_new, const void* v_new, int n_new,
                              hipStream_t s) {
  return launch_refresh(c, k_new, v_new, n_new, s);
}

hipError_t launch_rebuild(const CacheView& c, hipStream_t s) {
  return launch_refresh(c, nullptr, nullptr, 0, s);
}

}  // namespace resa
