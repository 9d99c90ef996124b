// Debug validation of the routing inputs of the hot path.
//
// The routing, co-activation and layout kernels stay in bounds for any
// values, but values outside their domain give results the pages do not
// define: a NaN router logit has no place in the descending order of
// logits, an expert id outside [0,E) or repeated within one token is not a
// choice of k distinct experts out of E (Zyphra correlated expert placement
// page, English abstract: each token goes to k of the E experts), and a rank
// outside [0,G) is not a placement of the experts on the G ranks. This
// kernel reads every value once and ORs a flag per kind of fault into a
// device word, which the caller reads after synchronising; nothing traps.
//
// gfx950 mapping: a grid-stride pass, one element per lane; each wave ORs
// its lanes' flags together with a ballot per flag, and one lane per wave
// issues a single atomicOr when any flag is set.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void wave_flag(uint32_t f, uint32_t* err) {
  uint32_t all = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (__ballot((f >> b) & 1u)) all |= 1u << b;
  if (all && (threadIdx.x & (kWave - 1)) == 0) atomicOr(err, all);
}

__global__ __launch_bounds__(256) void validate_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ topk_idx,
                                                       int T, int E, int k,
                                                       const int32_t* __restrict__ place, int G,
                                                       uint32_t* __restrict__ err) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // logits: NaN is the only value outside the domain (-inf is a mask)
  if (logits) {
    const int64_t n = (int64_t)T * E;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x; b < n; b += stride) {
      const int64_t i = b + threadIdx.x;
      const float v = i < n ? logits[i] : 0.f;
      wave_flag(v != v ? MOE_BAD_LOGIT : 0u, err);
    }
  }
  // one lane per token: its k choices in range and pairwise distinct
  if (topk_idx) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x; b < T; b += stride) {
      const int64_t t = b + threadIdx.x;
      uint32_t f = 0;
      if (t < T) {
        const int32_t* r = topk_idx + t * k;
        for (int j = 0; j < k; ++j) {
          const int e = r[j];
          if (e < 0 || e >= E) f |= MOE_BAD_EXPERT;
          for (int i = 0; i < j; ++i)
            if (r[i] == e) f |= MOE_BAD_REPEAT;
        }
      }
      wave_flag(f, err);
    }
  }
  if (place) {
    for (int64_t e = i0; e < E; e += stride) {
      const int g = place[e];
      if (g < 0 || g >= G) atomicOr(err, (uint32_t)MOE_BAD_RANK);
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT moe_status moe_validate_routing(const float* logits, const int32_t* topk_idx,
                                           int32_t T, int32_t E, int32_t k, const int32_t* place,
                                           int32_t G, uint32_t* err, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || G < 1 || !err) return MOE_ERR_ARG;
  if (k > kMaxK || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  const int64_t work = std::max<int64_t>({(int64_t)T * E, (int64_t)T, (int64_t)E});
  const unsigned grid = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(work, 256)));
  hipLaunchKernelGGL(validate_kernel, dim3(grid), dim3(256), 0, stream, T > 0 ? logits : nullptr,
                     T > 0 ? topk_idx : nullptr, T, E, k, place, G, err);
  return launch_status();
}
