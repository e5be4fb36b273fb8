// Gradual-filtering selection: keep the k context rows of largest deviation (ties to the
// lower index), output ascending, then append every query row.
//
// One workgroup of 1024 threads (16 wavefronts).  The k-th largest key is found exactly by
// an MSB-first radix select over order-preserving uint32 images of the fp32 scores (four
// 8-bit digits, LDS histograms with integer atomics, so the counts are exact; the digit is
// located by a suffix scan of the histogram across one wavefront).  Rows are
// then compacted in index order with wavefront ballots + popcounts and a 16-entry LDS
// prefix: rows above the threshold are all kept, rows equal to it are kept lowest index
// first until k is reached.
#include "cb_common.h"
#include "cb_kernels.h"

namespace cb {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((u >> 31) ? 0xffffffffu : 0x80000000u);
}

// Exclusive prefix count of `flag` over the workgroup (index order = thread order) and the
// total.  Uses `scratch` (TK_WAVES entries); contains two barriers.
__device__ __forceinline__ uint32_t block_scan(bool flag, uint32_t* scratch, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const uint32_t below = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) scratch[wave] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    const uint32_t c = scratch[w];
    before += (w < wave) ? c : 0u;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + below;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const float* dev, const int32_t* sel, int n_cand,
                                                          int n_query, int k, int32_t* new_sel,
                                                          int32_t* new_local) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_rem;
  __shared__ uint32_t scan_a[TK_WAVES], scan_b[TK_WAVES];
  const int tid = threadIdx.x;

  if (k >= n_cand) {
    for (int i = tid; i < n_cand; i += TK_THREADS) {
      new_sel[i] = sel[i];
      new_local[i] = i;
    }
  } else if (k > 0) {
    uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n_cand; i += TK_THREADS) {
        const uint32_t u = order_key(dev[i]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {  // digit of the remaining-th largest among the matching keys: the one bin b
        // with above(b) < remaining <= above(b) + hist[b], above(b) = count in bins > b; lane l
        // holds bins 4l .. 4l+3, a suffix scan over the lanes gives above() of its top bin
        const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2], h3 = hist[4 * tid + 3];
        const uint32_t own = h0 + h1 + h2 + h3;
        uint32_t incl = own;  // sum over lanes >= tid
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t t = __shfl_down(incl, d);
          if (tid + d < 64) incl += t;
        }
        const uint32_t a3 = incl - own, a2 = a3 + h3, a1 = a2 + h2, a0 = a1 + h1;
        if (a3 < remaining && remaining <= a3 + h3) { s_digit = 4 * tid + 3; s_rem = remaining - a3; }
        if (a2 < remaining && remaining <= a2 + h2) { s_digit = 4 * tid + 2; s_rem = remaining - a2; }
        if (a1 < remaining && remaining <= a1 + h1) { s_digit = 4 * tid + 1; s_rem = remaining - a1; }
        if (a0 < remaining && remaining <= a0 + h0) { s_digit = 4 * tid; s_rem = remaining - a0; }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      mask |= 255u << shift;
      remaining = s_rem;
      __syncthreads();
    }
    const uint32_t thr = prefix;  // image of the k-th largest score
    uint32_t base_eq = 0, base_take = 0;
    for (int c0 = 0; c0 < n_cand; c0 += TK_THREADS) {
      const int i = c0 + tid;
      const bool valid = i < n_cand;
      const uint32_t u = valid ? order_key(dev[i]) : 0u;
      const bool eq = valid && u == thr;
      uint32_t tot_eq, tot_take;
      const uint32_t eq_rank = base_eq + block_scan(eq, scan_a, &tot_eq);
      const bool take = valid && (u > thr || (eq && eq_rank < remaining));
      const uint32_t at = base_take + block_scan(take, scan_b, &tot_take);
      if (take) {
        new_sel[at] = sel[i];
        new_local[at] = i;
      }
      base_eq += tot_eq;
      base_take += tot_take;
    }
  }
  for (int q = tid; q < n_query; q += TK_THREADS) {
    new_sel[k + q] = sel[n_cand + q];
    new_local[k + q] = n_cand + q;
  }
}

}  // namespace

hipError_t topk_select(const float* dev, const int32_t* sel, int n_cand, int n_query, int k, int32_t* new_sel,
                       int32_t* new_local, hipStream_t s) {
  if (n_cand + n_query <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(TK_THREADS), 0, s, dev, sel, n_cand, n_query, k, new_sel,
                     new_local);
  return hipGetLastError();
}

}  // namespace cb
