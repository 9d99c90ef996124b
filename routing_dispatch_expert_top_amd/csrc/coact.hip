// Expert co-activation histogram (Cobalt page, English abstract: pairs of
// experts activated together by a single token).
//
// Two gfx950 mappings; integer atomics commute, so both give the exact
// count, independent of timing.
//  row owner (small E*T*k): workgroup (a, chunk) scans its chunk of the
//    routing result and, for each token that chose expert a, bumps LDS
//    counters of row a; it then adds the row's non-zero cells to the global
//    matrix. Every CU streams the (L2-resident) routing result, no workgroup
//    flushes more than E cells, and global atomics on one cell come only
//    from the chunks of one row.
//  triangle (large E*T*k): each workgroup owns a private upper-triangular
//    E x E counter matrix in LDS (E(E-1)/2 32-bit cells: 127.5 KiB at
//    E = 256, which fits the 160 KiB of LDS of a gfx950 CU), counts its
//    tokens' unordered pairs with LDS atomics, then flushes every non-zero
//    cell into both mirrored entries of the global matrix.
#include "moe_internal.h"

#include <atomic>

namespace moe {
namespace {

__device__ __forceinline__ int tri_row_start(int a, int E) {
  // cells (a, b), b > a, of rows 0..a-1 come first
  return a * (E - 1) - (a * (a - 1)) / 2;
}

// Workgroup (a, chunk) scans the flat entries [f0, f1) of the routing result
// with coalesced loads (16 bytes per lane when VEC) and queues, in LDS, the
// positions of entries equal to a; then every queued hit re-reads its token
// row (all k loads in flight at once) and bumps the counters of the token's
// other experts. Hits are rare (about T*k/E per row in all), so both passes
// cost one or two memory round trips. A token holding a h times adds h to
// each of its other experts, as its ordered index pairs do.
constexpr int kHitQueue = 2048;

template <bool VEC>
__global__ __launch_bounds__(256) void coact_rows_kernel(const int32_t* __restrict__ topk_idx,
                                                        int T, int E, int k, int per_wg,
                                                        int32_t* __restrict__ coact) {
  __shared__ uint32_t row[kMaxE];
  __shared__ int32_t queue[kHitQueue];
  __shared__ int32_t nq;
  const int a = blockIdx.x;
  for (int b = threadIdx.x; b < E; b += blockDim.x) row[b] = 0u;
  if (threadIdx.x == 0) nq = 0;
  __syncthreads();
  auto hit = [&](int p) {
    const int32_t* r = topk_idx + (size_t)(p / k) * k;
    int e[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) e[j] = j < k ? r[j] : -1;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (e[j] >= 0 && e[j] < E && e[j] != a) atomicAdd(&row[e[j]], 1u);
  };
  auto enqueue = [&](int p) {
    const int i = atomicAdd(&nq, 1);
    if (i < kHitQueue) queue[i] = p;
    else hit(p);  // overflow: only with many repeats of a in one chunk
  };
  const int n = T * k;
  const int f0 = blockIdx.y * per_wg;
  const int f1 = min(n, f0 + per_wg);
  if (VEC) {
    // f0 and per_wg are multiples of 4 and topk_idx is 16-byte aligned
    constexpr int U = 4;
    for (int f = f0 + 4 * (int)threadIdx.x; f < f1; f += 4 * U * (int)blockDim.x) {
      int4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = f + 4 * u * (int)blockDim.x;
        v[u] = g + 3 < f1 ? *reinterpret_cast<const int4*>(topk_idx + g)
                          : make_int4(g < f1 ? topk_idx[g] : -1, g + 1 < f1 ? topk_idx[g + 1] : -1,
                                      g + 2 < f1 ? topk_idx[g + 2] : -1, -1);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = f + 4 * u * (int)blockDim.x;
        if (v[u].x == a) enqueue(g);
        if (v[u].y == a) enqueue(g + 1);
        if (v[u].z == a) enqueue(g + 2);
        if (v[u].w == a) enqueue(g + 3);
      }
    }
  } else {
    for (int f = f0 + (int)threadIdx.x; f < f1; f += blockDim.x)
      if (topk_idx[f] == a) enqueue(f);
  }
  __syncthreads();
  const int nh = min(nq, kHitQueue);
  for (int i = threadIdx.x; i < nh; i += blockDim.x) hit(queue[i]);
  __syncthreads();
  for (int b = threadIdx.x; b < E; b += blockDim.x) {
    const uint32_t c = row[b];
    if (c) atomicAdd(&coact[(size_t)a * E + b], (int32_t)c);
  }
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

// Largest E*T*k for the row-owner kernel: its reads of the routing result
// grow as E*T*k (4 bytes each, from L2), the triangle kernel's work as T*k*k.
constexpr int64_t kRowOwnerMaxWork = int64_t(1) << 26;

// LDS bytes a workgroup may use on the current device, cached per device
// (the relaxed atomics make concurrent first calls from several host threads
// safe: each stores the same value).
constexpr int kMaxDevices = 64;
std::atomic<int> g_lds_limit[kMaxDevices];  // 0: not read yet

int max_lds_per_block() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_lds_limit[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return 0;
  if (dev >= 0 && dev < kMaxDevices && v > 0) g_lds_limit[dev].store(v, std::memory_order_relaxed);
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
  if ((int64_t)E * T * k <= kRowOwnerMaxWork) {
    // about 2048 workgroups, at least 2048 entries each
    const int n = T * k;
    const int chunks = (int)std::max<int64_t>(
        1, std::min<int64_t>(ceil_div(2048, E), ceil_div(n, 2048)));
    const int per_wg = (int)ceil_div(ceil_div(n, chunks), 4) * 4;
    const dim3 grid(E, (unsigned)ceil_div(n, per_wg));
    if ((uintptr_t)topk_idx % 16 == 0)
      hipLaunchKernelGGL(coact_rows_kernel<true>, grid, dim3(256), 0, stream, topk_idx, T, E, k,
                         per_wg, coact);
    else
      hipLaunchKernelGGL(coact_rows_kernel<false>, grid, dim3(256), 0, stream, topk_idx, T, E, k,
                         per_wg, coact);
    return launch_status();
  }
  const size_t lds = sizeof(uint32_t) * (size_t)E * (E - 1) / 2;
  if (lds <= (size_t)max_lds_per_block()) {
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
