// Tile scheduling, LDS swizzle and activation helpers shared by the grouped
// GEMM kernels of the forward and backward expert networks (gfx950 only).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding)
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 0x3) << 14))
// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned
#define MOE_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14))

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// An accumulator element read into a VGPR where it is used: as an asm
// statement the read keeps its place, so the compiler neither copies every
// accumulator to VGPRs at the start of an epilogue nor moves them between
// AGPRs (which a pin of each fragment before its use costs).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

constexpr int kXcd = 8;  // MI355X: workgroups go round-robin over 8 XCDs
// Tile queue of the persistent grouped GEMMs: 8 XCD counters, the finish
// count, padding. Zero when a launch starts; the launch leaves it zero.
constexpr int kQueueWords = 16;

// Per-workgroup tile schedule: prefix of M-tiles per expert in LDS.
struct Sched {
  int mt_off[kMaxE + 1];
  int wave_tot[16];
};

// Exclusive prefix (over experts) of ceil(M_e / BM); all threads participate.
__device__ void build_schedule(Sched& sc, const int32_t* __restrict__ expert_off, int E, int BM) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwave = blockDim.x / kWave;
  // blockDim.x >= 256 >= E: one expert per thread
  const int e = threadIdx.x;
  int v = 0;
  if (e < E) {
    const int m = expert_off[e + 1] - expert_off[e];
    v = m > 0 ? (m + BM - 1) / BM : 0;
  }
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sc.wave_tot[wave] = incl;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += sc.wave_tot[w];
  if (e < E) sc.mt_off[e] = pre + incl - v;
  if (e == E - 1) sc.mt_off[E] = pre + incl;
  (void)nwave;
  __syncthreads();
}

// Logical tile index for this block, or -1. Consecutive logical tiles share
// an XCD: block i runs on XCD i % 8, and XCD x takes tiles [x*q, (x+1)*q).
__device__ __forceinline__ int xcd_logical_tile(int total) {
  const int i = blockIdx.x;
  const int q = (total + kXcd - 1) / kXcd;
  const int slot = i / kXcd;
  const int logical = (i % kXcd) * q + slot;
  if (slot >= q || logical >= total) return -1;
  return logical;
}

// Tile order inside an expert: blocks of kMBlock m-tiles; within a block,
// n-tiles outer and m-tiles inner. Consecutive tiles (which start close
// together on one XCD) share a weight panel, and an activation tile comes
// back kMBlock tiles later, while its slices are still in the XCD's L2. With
// m-tiles innermost over a whole expert, a large expert's activation tiles
// would come back only after all of its m-tiles, long evicted.
constexpr int kMBlock = 4;

// tile -> (expert, n-tile, m-tile)
__device__ __forceinline__ void decode_tile(const Sched& sc, int E, int NT, int tile, int& e,
                                            int& nt, int& mt) {
  int lo = 0, hi = E - 1;  // last e with mt_off[e] * NT <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sc.mt_off[mid] * NT <= tile) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  const int rem = tile - sc.mt_off[e] * NT;
  const int mte = sc.mt_off[e + 1] - sc.mt_off[e];
  const int b = rem / (kMBlock * NT);        // m-block
  const int bm = min(kMBlock, mte - b * kMBlock);  // m-tiles in this block
  const int within = rem - b * kMBlock * NT;
  nt = within / bm;
  mt = b * kMBlock + within % bm;
}

struct TileSel {
  int wave_tot[16];
  int sel[5];  // expert, its first m-tile, its m-tile count, its segment start and end
};

// This workgroup's tile of a grouped launch over ceil(M_e / BM) m-tiles per
// expert and NT n-tiles, in the order of decode_tile and the XCD grouping of
// xcd_logical_tile; false if the workgroup has none (uniform). Thread e
// scans expert e's m-tiles and, holding its own prefix and segment bounds,
// claims the tile if it falls in that expert's range, so the tile is known
// after one LDS round instead of a search over the prefix and a reload of
// the segment bounds. All threads take part (blockDim.x >= E).
__device__ __forceinline__ bool select_tile(TileSel& ts, const int32_t* __restrict__ expert_off,
                                            int E, int BM, int NT, int& e, int& nt, int& mt,
                                            int& seg0, int& seg1) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwave = blockDim.x / kWave;
  const int t = threadIdx.x;
  int v = 0, o0 = 0, o1 = 0;
  if (t < E) {
    o0 = expert_off[t];
    o1 = expert_off[t + 1];
    v = (o1 - o0 + BM - 1) / BM;
  }
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) ts.wave_tot[wave] = incl;
  __syncthreads();
  int pre = 0, all = 0;
  for (int w = 0; w < nwave; ++w) {
    const int x = ts.wave_tot[w];
    if (w < wave) pre += x;
    all += x;
  }
  const int tile = xcd_logical_tile(all * NT);
  if (tile < 0) return false;  // uniform over the workgroup
  const int first = pre + incl - v;  // this expert's first m-tile
  if (t < E && v > 0 && first * NT <= tile && tile < (first + v) * NT) {
    ts.sel[0] = t;
    ts.sel[1] = first;
    ts.sel[2] = v;
    ts.sel[3] = o0;
    ts.sel[4] = o1;
  }
  __syncthreads();
  e = ts.sel[0];
  const int mte = ts.sel[2];
  seg0 = ts.sel[3];
  seg1 = ts.sel[4];
  const int rem = tile - ts.sel[1] * NT;
  const int b = rem / (kMBlock * NT);
  const int bm = min(kMBlock, mte - b * kMBlock);
  const int within = rem - b * kMBlock * NT;
  nt = within / bm;
  mt = b * kMBlock + within % bm;
  return true;
}

// silu(u) * v = u * v / (1 + e^-u), with the hardware exp2 and reciprocal
// (about 1 ulp each: far below the bf16 rounding of h and the fp32 tolerance).
// Six VALU operations instead of the ~20 of a full-precision exp and an IEEE
// division; e^-u overflowing to inf gives -0 for large negative u, as the
// exact value rounds to.
__device__ __forceinline__ float silu_mul(float u, float v) {
  const float e = __builtin_amdgcn_exp2f(-u * 1.44269504088896341f);
  return u * v * __builtin_amdgcn_rcpf(1.0f + e);
}

// LDS slot of chunk c of row r when a K slice has CH 16-byte chunks per row
// (CH = 8: 128-byte rows, CH = 4: 64-byte rows). 256 bytes of LDS cover all
// banks; the fragment reads take 16 consecutive rows at one logical chunk,
// and XOR-ing the chunk with the row's index among the rows sharing a bank
// phase gives those 16 rows 16 distinct 16-byte bank groups.
template <int CH>
__device__ __forceinline__ int swz_ch(int r, int c) {
  constexpr int kRowsPer256 = 16 / CH;
  return r * CH + (c ^ ((r / kRowsPer256) & (CH - 1)));
}

// Upper bound of sum_e ceil(M_e / BM) for sum_e M_e = rows over E experts.
inline int64_t mtile_upper(int64_t rows, int E, int BM) {
  return std::min<int64_t>(rows, (rows + (int64_t)E * (BM - 1)) / BM);
}
inline unsigned grid_for(int64_t tiles) {
  return (unsigned)(ceil_div(std::max<int64_t>(tiles, 1), kXcd) * kXcd);
}

}  // namespace
}  // namespace moe
