// Internal helpers shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/moe.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {

constexpr int kMaxK = 16;
constexpr int kMaxE = 256;
constexpr int kMaxG = 32;
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes, a native vector

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
// two bf16 packed in a 32-bit word: low half first
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// Two floats to two bf16 (RNE) in one word, low half first: one
// v_cvt_pk_bf16_f32 (converting each on its own costs two conversions, a
// shift and an or).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

inline bool valid_dtype(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }
inline int dtype_bytes(moe_dtype dt) { return dt == MOE_F32 ? 4 : 2; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Weight-gradient mode of the forward's persistent bf16 grouped GEMM
// (ffn.hip): out[e][m][n] = sum over the slots s of expert e of a[s][m]
// bt[n][kseg[e] + s - expert_off[e]]; a is [slots][M0] (M contiguous), bt is
// N0 x ldk (bf16, K contiguous, each expert's segment padded with zeros to a
// multiple of 64), fp32 output split at row msplit.
// Data-gradient mode (ffn.hip): c[s] = a[s] W[e] for the slots s of expert
// e, W[e] = [K][N0] bf16 (rows k < ksplit from w0's panel e of ksplit x N0,
// the rest from w1's); with uv, the epilogue applies the SwiGLU backward and
// c holds [du | dv] rows of 2 N0, else c is [rows][N0].
bool dgrad_offsets_fit(int64_t rows, int64_t k);
void launch_dgrad_bf16(const uint16_t* a, int64_t rows, const int32_t* expert_off, int E, int K,
                       const uint16_t* w0, const uint16_t* w1, int ksplit, int N0,
                       const uint16_t* uv, uint16_t* c, hipStream_t stream);
bool wgrad_offsets_fit(int64_t m0, int64_t n0, int64_t ldk);
// eorder [8 * ceil(E/8)]: expert at each position of the tile walk (-1: none);
// XCD x takes positions [x ceil(E/8), (x+1) ceil(E/8)). A persistent launch:
// queue (16 words) must be zero when it starts and is left zero.
moe_status launch_wgrad_bf16(const uint16_t* a, const uint16_t* bt, const int32_t* expert_off,
                             const int32_t* kseg, const int32_t* eorder, int E, int M0, int N0,
                             int ldk, int msplit, float* o0, float* o1, uint32_t* queue,
                             hipStream_t stream);

}  // namespace moe
