// Gate-weighted combine back into token order (Zyphra correlated expert
// placement page, English abstract: after the experts, the results are
// combined). out[t] = sum_j gates[t,j] * y[slot_of[t*k+j]], fp32 accumulation
// in j order, stored in the activation type; a choice with a negative slot
// (dropped by the replica-aware layout) contributes nothing.
//
// gfx950 mapping: one wavefront per token. The token's k slots and gates are
// wave-uniform and come in through scalar loads (SGPRs); each lane then
// gathers 16-byte chunks of the k expert rows (a row is contiguous, so each
// load instruction is a fully used 1 KiB segment), with two chunks per lane
// in flight per row, and writes the output row once, 8 KiB at a time after
// the reads that produce it; each token starts at a different 1 KiB block of
// its rows. k is a template parameter for the
// common values so the row loads fully unroll.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool BF16>
__device__ __forceinline__ void accum(float (&acc)[8], const u32x4& v, float g) {
  if (BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(g, bf16lo(v[q]), acc[2 * q]);
      acc[2 * q + 1] = fmaf(g, bf16hi(v[q]), acc[2 * q + 1]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(g, __uint_as_float(v[q]), acc[q]);
  }
}

template <bool BF16>
__device__ __forceinline__ u32x4 pack(const float (&acc)[8]) {
  if (BF16)
    return u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  return u32x4{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
               __float_as_uint(acc[3])};
}

// KK > 0: k == KK at compile time; KK == 0: runtime k <= kMaxK.
// WHOLE: the row is a whole number of 1 KiB blocks (no per-lane tail test).
// HOLD: the row is at most kHoldBlocks blocks, and its output is held in
// registers until all of it is computed.
constexpr int kHoldBlocks = 8;
template <bool BF16, int KK, bool WHOLE, bool HOLD>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4* __restrict__ y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ gates, int T,
                                                      int k_rt, int row_vecs,
                                                      u32x4* __restrict__ out) {
  constexpr int KM = KK > 0 ? KK : kMaxK;
  const int k = KK > 0 ? KK : k_rt;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * (blockDim.x / kWave) + wave;  // wave-uniform
  if (t >= T) return;
  // A negative slot is a dropped choice (no copy of its expert was
  // assigned): it reads nothing and adds nothing.
  const u32x4* rows[KM];
  float g[KM];
  bool live[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    live[j] = false;
    if (j < k) {
      const int s = slot_of[(size_t)t * k + j];
      live[j] = s >= 0;
      rows[j] = y + (size_t)(live[j] ? s : 0) * row_vecs;
      g[j] = gates ? gates[(size_t)t * k + j] : 1.0f;
    }
  }
  u32x4* o = out + (size_t)t * row_vecs;
  // The row is walked in 1 KiB blocks (64 lanes x 16 bytes), two blocks per
  // step so two loads per expert row are in flight. Token t starts at block
  // t mod nblk and wraps around: waves working at the same moment then read
  // different offsets of their 8 KiB-strided rows instead of all hitting the
  // same HBM channels (a fixed start measured ~6% slower).
  const int nblk = (row_vecs + kWave - 1) / kWave;
  const int sb = t % nblk;
  auto blk = [&](int b) {  // the row block visited at step b
    const int p = b + sb;
    return p >= nblk ? p - nblk : p;
  };
  // CHK: some choice of this token is dropped (rare); the common path has no
  // per-choice test in its loop
  auto walk = [&](auto chk_c) {
    constexpr bool CHK = decltype(chk_c)::value;
    // blocks b and b + 1 (if b + 1 < nblk) of the walk, packed
    auto pair = [&](int b, u32x4& r0, u32x4& r1) {
      const int c0 = blk(b) * kWave + lane;
      const int c1 = b + 1 < nblk ? blk(b + 1) * kWave + lane : row_vecs;
      const bool ok0 = WHOLE || c0 < row_vecs, ok1 = (WHOLE && b + 1 < nblk) || c1 < row_vecs;
      u32x4 v0[KM], v1[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < k && (!CHK || live[j])) {
          v0[j] = ok0 ? __builtin_nontemporal_load(rows[j] + c0) : u32x4{0, 0, 0, 0};
          v1[j] = ok1 ? __builtin_nontemporal_load(rows[j] + c1) : u32x4{0, 0, 0, 0};
        }
      float a0[8] = {}, a1[8] = {};
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j < k && (!CHK || live[j])) {
          accum<BF16>(a0, v0[j], g[j]);
          accum<BF16>(a1, v1[j], g[j]);
        }
      r0 = pack<BF16>(a0);
      r1 = pack<BF16>(a1);
    };
    auto ok = [&](int c) { return WHOLE || c < row_vecs; };
    if constexpr (HOLD) {
      // The whole output row stays in registers and is written after the
      // last read, as one run of non-temporal stores: stores mixed into the
      // read stream, one or two after every step, cost HBM read/write
      // turnarounds (-6% on a 4096-wide bf16 row).
      u32x4 ob[kHoldBlocks];
#pragma unroll
      for (int b = 0; b < kHoldBlocks; b += 2) {
        if (b >= nblk) break;  // uniform
        pair(b, ob[b], ob[b + 1]);
        // One step's loads live at a time: its sums are complete (operands
        // of the empty asm) before the next step's loads, which the
        // compiler would otherwise hoist for the whole row (256 registers,
        // one wave per SIMD).
        asm volatile("" : "+v"(ob[b]), "+v"(ob[b + 1])::"memory");
      }
#pragma unroll
      for (int b = 0; b < kHoldBlocks; ++b) {
        if (b >= nblk) break;  // uniform
        const int c = blk(b) * kWave + lane;
        if (ok(c)) __builtin_nontemporal_store(ob[b], o + c);
      }
    } else {
      for (int b = 0; b < nblk; b += 2) {
        u32x4 r0, r1;
        pair(b, r0, r1);
        const int c0 = blk(b) * kWave + lane;
        if (ok(c0)) o[c0] = r0;
        if (b + 1 < nblk) {
          const int c1 = blk(b + 1) * kWave + lane;
          if (ok(c1)) o[c1] = r1;
        }
      }
    }
  };
  bool all_live = true;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) all_live = all_live && live[j];
  if (all_live) walk(std::false_type{});
  else walk(std::true_type{});
}

template <bool BF16, bool WHOLE, bool HOLD>
void launch_combine(const void* y, const int32_t* slot_of, const float* gates, int T, int k,
                    int row_vecs, void* out, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  const u32x4* yy = static_cast<const u32x4*>(y);
  u32x4* oo = static_cast<u32x4*>(out);
#define MOE_COMBINE_CASE(KV)                                                                    \
  case KV:                                                                                      \
    hipLaunchKernelGGL((combine_kernel<BF16, KV, WHOLE, HOLD>), grid, block, 0, stream, yy,     \
                       slot_of, gates, T, k, row_vecs, oo);                                     \
    return;
  switch (k) {
    MOE_COMBINE_CASE(1)
    MOE_COMBINE_CASE(2)
    MOE_COMBINE_CASE(4)
    MOE_COMBINE_CASE(6)
    MOE_COMBINE_CASE(8)
    default:
      hipLaunchKernelGGL((combine_kernel<BF16, 0, WHOLE, HOLD>), grid, block, 0, stream, yy,
                         slot_of, gates, T, k, row_vecs, oo);
  }
#undef MOE_COMBINE_CASE
}

template <bool BF16>
void launch_combine(const void* y, const int32_t* slot_of, const float* gates, int T, int k,
                    int row_vecs, void* out, hipStream_t stream) {
  const bool whole = row_vecs % kWave == 0;
  const bool hold = row_vecs <= kHoldBlocks * kWave;
  if (whole && hold) launch_combine<BF16, true, true>(y, slot_of, gates, T, k, row_vecs, out, stream);
  else if (whole) launch_combine<BF16, true, false>(y, slot_of, gates, T, k, row_vecs, out, stream);
  else if (hold) launch_combine<BF16, false, true>(y, slot_of, gates, T, k, row_vecs, out, stream);
  else launch_combine<BF16, false, false>(y, slot_of, gates, T, k, row_vecs, out, stream);
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
  if (!y || !slot_of || !out) return MOE_ERR_ARG;  // gates NULL: every gate is 1
  if (((size_t)d * dtype_bytes(dt)) % 16 != 0 || (uintptr_t)y % 16 || (uintptr_t)out % 16)
    return MOE_ERR_UNSUPPORTED;
  const int row_vecs = (int)((size_t)d * dtype_bytes(dt) / 16);
  if (dt == MOE_BF16) launch_combine<true>(y, slot_of, gates, T, k, row_vecs, out, stream);
  else launch_combine<false>(y, slot_of, gates, T, k, row_vecs, out, stream);
  return launch_status();
}
