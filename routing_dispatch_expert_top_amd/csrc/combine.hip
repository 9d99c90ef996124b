// Gate-weighted combine back into token order (Zyphra correlated expert
// placement page, English abstract: after the experts, the results are
// combined). out[t] = sum_j gates[t,j] * y[slot_of[t*k+j]], fp32 accumulation
// in j order, stored in the activation type.
//
// gfx950 mapping: one wavefront per token gathers its k expert rows with
// 16-byte loads per lane (a row is contiguous, so each load instruction is a
// fully used 1 KiB segment), issuing all k loads of a chunk before
// accumulating, and writes the output row once.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ gates, int T,
                                                      int k, int row_vecs,
                                                      uint4* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  int slot[kMaxK];
  float g[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    slot[j] = j < k ? slot_of[(size_t)t * k + j] : 0;
    g[j] = j < k ? gates[(size_t)t * k + j] : 0.f;
  }
  for (int c = lane; c < row_vecs; c += kWave) {
    uint4 v[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k) v[j] = y[(size_t)slot[j] * row_vecs + c];
    if (BF16) {
      float acc[8] = {};
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
          const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(g[j], bf16lo(w[q]), acc[2 * q]);
            acc[2 * q + 1] = fmaf(g[j], bf16hi(w[q]), acc[2 * q + 1]);
          }
        }
      }
      out[(size_t)t * row_vecs + c] =
          make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      float acc[4] = {};
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
          acc[0] = fmaf(g[j], __uint_as_float(v[j].x), acc[0]);
          acc[1] = fmaf(g[j], __uint_as_float(v[j].y), acc[1]);
          acc[2] = fmaf(g[j], __uint_as_float(v[j].z), acc[2]);
          acc[3] = fmaf(g[j], __uint_as_float(v[j].w), acc[3]);
        }
      }
      out[(size_t)t * row_vecs + c] = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                                 __float_as_uint(acc[2]), __float_as_uint(acc[3]));
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT moe_status moe_combine(const void* y, const int32_t* slot_of, const float* gates,
                                  int32_t T, int32_t k, int32_t d, moe_dtype dt, void* out,
                                  hipStream_t stream) {
  if (T < 0 || k < 1 || d < 1 || !valid_dtype(dt)) return MOE_ERR_ARG;
  if (k > kMaxK || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !slot_of || !gates || !out) return MOE_ERR_ARG;
  if (((size_t)d * dtype_bytes(dt)) % 16 != 0 || (uintptr_t)y % 16 || (uintptr_t)out % 16)
    return MOE_ERR_UNSUPPORTED;
  const int row_vecs = (int)((size_t)d * dtype_bytes(dt) / 16);
  const dim3 grid((unsigned)ceil_div(T, 4));
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(y), slot_of, gates, T, k, row_vecs,
                       static_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(y), slot_of, gates, T, k, row_vecs,
                       static_cast<uint4*>(out));
  return launch_status();
}
