// Expert co-activation histogram (Cobalt page, English abstract: pairs of
// experts activated together by a single token).
//
// gfx950 mapping: each workgroup owns a private upper-triangular E x E
// counter matrix in LDS (E(E-1)/2 32-bit cells: 127.5 KiB at E = 256, which
// fits the 160 KiB of LDS of a gfx950 CU), counts its tokens' unordered
// pairs with LDS atomics, then flushes every non-zero cell into both
// mirrored entries of the global matrix with global atomics. Integer
// atomics commute, so the result is exact and independent of timing.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int tri_row_start(int a, int E) {
  // cells (a, b), b > a, of rows 0..a-1 come first
  return a * (E - 1) - (a * (a - 1)) / 2;
}

__global__ __launch_bounds__(1024) void coact_lds_kernel(const int32_t* __restrict__ topk_idx,
                                                         int T, int E, int k, int tok_per_wg,
                                                         int32_t* __restrict__ coact) {
  extern __shared__ uint32_t tri[];
  const int ncell = E * (E - 1) / 2;
  for (int i = threadIdx.x; i < ncell; i += blockDim.x) tri[i] = 0u;
  __syncthreads();

  const int t0 = blockIdx.x * tok_per_wg;
  const int t1 = min(T, t0 + tok_per_wg);
  for (int t = t0 + (int)threadIdx.x; t < t1; t += blockDim.x) {
    int e[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) e[j] = j < k ? topk_idx[(size_t)t * k + j] : -1;
#pragma unroll
    for (int i = 0; i < kMaxK; ++i) {
#pragma unroll
      for (int j = i + 1; j < kMaxK; ++j) {
        if (j < k) {
          int a = min(e[i], e[j]), b = max(e[i], e[j]);
          if (a >= 0 && b < E && a != b) atomicAdd(&tri[tri_row_start(a, E) + b - a - 1], 1u);
        }
      }
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int nwave = blockDim.x / kWave;
  for (int a = threadIdx.x / kWave; a < E - 1; a += nwave) {
    const int base = tri_row_start(a, E) - a - 1;
    for (int b = a + 1 + lane; b < E; b += kWave) {
      const uint32_t c = tri[base + b];
      if (c) {
        atomicAdd(&coact[(size_t)a * E + b], (int32_t)c);
        atomicAdd(&coact[(size_t)b * E + a], (int32_t)c);
      }
    }
  }
}

// Fallback when the triangle does not fit in LDS: global atomics per pair.
__global__ __launch_bounds__(256) void coact_global_kernel(const int32_t* __restrict__ topk_idx,
                                                           int T, int E, int k,
                                                           int32_t* __restrict__ coact) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  for (int i = 0; i < k; ++i)
    for (int j = 0; j < k; ++j) {
      const int a = topk_idx[(size_t)t * k + i], b = topk_idx[(size_t)t * k + j];
      if (i != j && a >= 0 && a < E && b >= 0 && b < E && a != b)
        atomicAdd(&coact[(size_t)a * E + b], 1);
    }
}

int max_lds_per_block() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return 0;
  return v;
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT moe_status moe_coact_hist(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                     int32_t* coact, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0 || k == 1) return MOE_OK;
  if (!topk_idx || !coact) return MOE_ERR_ARG;
  const size_t lds = sizeof(uint32_t) * (size_t)E * (E - 1) / 2;
  static int lds_limit = -1;
  if (lds_limit < 0) lds_limit = max_lds_per_block();
  if (lds <= (size_t)lds_limit) {
    // about 32k pair updates per workgroup, at most one workgroup per CU
    const int64_t pairs = (int64_t)T * k * (k - 1) / 2;
    int nwg = (int)std::min<int64_t>(256, std::max<int64_t>(1, ceil_div(pairs, 32768)));
    const int tok_per_wg = (int)ceil_div(T, nwg);
    nwg = (int)ceil_div(T, tok_per_wg);
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)coact_lds_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(coact_lds_kernel, dim3(nwg), dim3(1024), lds, stream, topk_idx, T, E, k,
                       tok_per_wg, coact);
  } else {
    hipLaunchKernelGGL(coact_global_kernel, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0,
                       stream, topk_idx, T, E, k, coact);
  }
  return launch_status();
}
