// Top-k routing with softmax gates: one sub-wave of L lanes per token.
//
// Each token is sent to k of its E experts (Zyphra correlated expert
// placement page, English abstract). The choice is the k largest logits,
// ties to the lower expert index, listed by descending logit; the gates are
// the softmax of the k chosen logits. The group-limited variant keeps only
// the topk_groups contiguous expert groups with the largest maximum logit.
//
// gfx950 mapping: L = next power of two >= ceil(E/4) lanes per token (at
// most a 64-lane wavefront), each lane holding 4 consecutive logits, so one
// 16-byte load per lane reads the row. A (logit, index) pair is packed into
// one 64-bit key whose unsigned order is the routing order; the k rounds of
// selection are k sub-wave max-reductions over that key (DPP moves within 16
// lanes, cross-lane shuffles beyond; no LDS, no atomics: the result is exact
// and deterministic). When each group of the group-limited variant is a
// power-of-two run of whole lanes, its maximum is a reduction over its own
// lanes; other group sizes take one reduction over the token per group.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxGroups = 32;

// Unsigned key whose order is the float order; -0 is folded onto +0.
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Larger key = earlier in the routing order. Key 0 marks "not available";
// every real key is larger (its low word is >= 2^32 - 256).
__device__ __forceinline__ uint64_t make_key(float f, int e) {
  return ((uint64_t)ord_f32(f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// One max step against the lane the DPP control CTRL names (within a row of
// 16 lanes), on both 32-bit halves of the key.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t x) {
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)phi << 32) | plo;
  return o > x ? o : x;
}

// Max over each aligned group of L lanes, left in every lane of the group.
// Inside a 16-lane row the partners come from DPP (quad permutes for the
// lanes 1 and 2 away, then the half-row and row mirrors, which pair each lane
// with one in the other half of its 8- or 16-lane group): a few cycles each
// instead of an LDS-crossbar round trip. Wider groups take one permute per
// doubling.
template <int L>
__device__ __forceinline__ uint64_t subwave_max(uint64_t x) {
  if (L >= 2) x = dpp_max_step<0xB1>(x);   // quad_perm [1,0,3,2]
  if (L >= 4) x = dpp_max_step<0x4E>(x);   // quad_perm [2,3,0,1]
  if (L >= 8) x = dpp_max_step<0x141>(x);  // row_half_mirror
  if (L >= 16) x = dpp_max_step<0x140>(x); // row_mirror
#pragma unroll
  for (int off = 16; off < L; off <<= 1) {
    const uint64_t o = __shfl_xor(x, off, L);
    x = o > x ? o : x;
  }
  return x;
}

// Max over aligned groups of `lanes` lanes (a power of two, uniform).
__device__ __forceinline__ uint64_t lane_group_max(uint64_t x, int lanes) {
  if (lanes >= 2) x = dpp_max_step<0xB1>(x);
  if (lanes >= 4) x = dpp_max_step<0x4E>(x);
  if (lanes >= 8) x = dpp_max_step<0x141>(x);
  if (lanes >= 16) x = dpp_max_step<0x140>(x);
  for (int off = 16; off < lanes; off <<= 1) {
    const uint64_t o = __shfl_xor(x, off, kWave);
    x = o > x ? o : x;
  }
  return x;
}

template <int L>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int n_groups, int topk_groups,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ gates, bool vec4) {
  constexpr int kTokPerWave = kWave / L;
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane & (L - 1);
  const int wave = threadIdx.x / kWave;
  const int t = (blockIdx.x * (blockDim.x / kWave) + wave) * kTokPerWave + lane / L;
  const bool active = t < T;
  const int e0 = sub * 4;

  float val[4];
  if (active && vec4 && e0 < E) {
    float4 q = *reinterpret_cast<const float4*>(logits + (size_t)t * E + e0);
    val[0] = q.x; val[1] = q.y; val[2] = q.z; val[3] = q.w;
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      val[v] = (active && e0 + v < E) ? logits[(size_t)t * E + e0 + v] : 0.f;
  }
  uint64_t key[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) key[v] = (active && e0 + v < E) ? make_key(val[v], e0 + v) : 0ull;

  // group key = largest expert key of the group: its order is the order of
  // the group maxima, ties going to the lower group (its experts have the
  // lower indices)
  const int gsz = n_groups > 1 ? E / n_groups : E;
  const int lpg = gsz >> 2;  // lanes per group when groups are whole lanes
  if (n_groups > 1 && (gsz & 3) == 0 && (lpg & (lpg - 1)) == 0) {
    // A lane's 4 logits lie in one group and group m is the aligned lanes
    // [m lpg, (m+1) lpg) of the token, so the group key is a reduction over
    // those lanes alone; the group's rank is read from the groups' first
    // lanes.
    uint64_t gk = key[0];
#pragma unroll
    for (int v = 1; v < 4; ++v) gk = key[v] > gk ? key[v] : gk;
    gk = lane_group_max(gk, lpg);
    const int base = lane & ~(L - 1);  // the token's first lane
    int rank = 0;
    for (int m = 0; m < n_groups; ++m) {
      const uint64_t o = __shfl(gk, base + m * lpg, kWave);
      rank += o > gk ? 1 : 0;
    }
    if (rank >= topk_groups) {
#pragma unroll
      for (int v = 0; v < 4; ++v) key[v] = 0;
    }
  } else if (n_groups > 1) {
    uint64_t gmax[kMaxGroups];
#pragma unroll
    for (int m = 0; m < kMaxGroups; ++m) {
      if (m < n_groups) {
        uint64_t mx = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (key[v] && (e0 + v) / gsz == m && key[v] > mx) mx = key[v];
        gmax[m] = subwave_max<L>(mx);
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (!key[v]) continue;
      const int mine = (e0 + v) / gsz;
      uint64_t gk = 0;
#pragma unroll
      for (int m = 0; m < kMaxGroups; ++m)
        if (m == mine) gk = gmax[m];
      int rank = 0;
#pragma unroll
      for (int m = 0; m < kMaxGroups; ++m)
        if (m < n_groups && gmax[m] > gk) ++rank;
      if (rank >= topk_groups) key[v] = 0;
    }
  }

  // k rounds: take the best remaining key of the token
  uint64_t sel[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      uint64_t best = key[0];
#pragma unroll
      for (int v = 1; v < 4; ++v) best = key[v] > best ? key[v] : best;
      best = subwave_max<L>(best);
      sel[j] = best;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (key[v] == best) key[v] = 0;
    }
  }
  if (!active) return;

  // softmax over the chosen logits, shifted by the largest (the first)
  const float l0 = unord_f32((uint32_t)(sel[0] >> 32));
  float p[kMaxK];
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      p[j] = expf(unord_f32((uint32_t)(sel[j] >> 32)) - l0);
      den += p[j];
    }
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k && (j & (L - 1)) == sub) {
      topk_idx[(size_t)t * k + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)sel[j]);
      gates[(size_t)t * k + j] = p[j] * inv;
    }
  }
}

template <int L>
void launch_route(const float* logits, int T, int E, int k, int ng, int tg, int32_t* idx,
                  float* gates, bool vec4, hipStream_t s) {
  constexpr int kThreads = 256;
  const int tok_per_block = (kThreads / kWave) * (kWave / L);
  const int grid = (int)ceil_div(T, tok_per_block);
  hipLaunchKernelGGL(route_kernel<L>, dim3(grid), dim3(kThreads), 0, s, logits, T, E, k, ng, tg,
                     idx, gates, vec4);
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                                int32_t n_groups, int32_t topk_groups, int32_t* topk_idx,
                                float* gates, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_groups < 1 || topk_groups < 1 ||
      topk_groups > n_groups || E % n_groups != 0 ||
      (int64_t)topk_groups * (E / n_groups) < k)
    return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || n_groups > kMaxGroups || (int64_t)T * k >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !gates) return MOE_ERR_ARG;
  const bool vec4 = (E % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  int L = 1;
  while (L * 4 < E) L *= 2;
  switch (L) {
    case 1: launch_route<1>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
    case 2: launch_route<2>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
    case 4: launch_route<4>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
    case 8: launch_route<8>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
    case 16: launch_route<16>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
    case 32: launch_route<32>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
    default: launch_route<64>(logits, T, E, k, n_groups, topk_groups, topk_idx, gates, vec4, stream); break;
  }
  return launch_status();
}
