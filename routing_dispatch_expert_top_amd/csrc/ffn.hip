// Grouped SwiGLU expert FFN over variable-length expert segments.
//
// The pages only say the MoE layer holds E expert networks that each token
// visits k of (Zyphra correlated expert placement page, English abstract);
// the expert form used here is a bias-free SwiGLU MLP:
//     h = silu(W_gate a) * (W_up a),   y = W_down h.
// Two launches: gate/up (with the SwiGLU epilogue fused, writing h) and
// down (writing y). Rows are slots in expert-grouped order; expert e owns
// slots expert_off[e] .. expert_off[e+1]-1, and the gate/up launch gathers
// its A rows from the dispatched rows through perm_row.
//
// bf16 path (gfx950): v_mfma_f32_32x32x16_bf16, fp32 accumulation. A
// workgroup computes a BM x BN tile (BN counts B rows: for gate/up, half
// gate rows and half up rows of the same F columns, so the epilogue has u
// and v of an element in the same lane). The K loop stages 64-wide K slices
// of A and B through double-buffered LDS (16-byte chunks, XOR-swizzled by
// row so the MFMA fragment reads spread over the banks), prefetching the
// next slice into registers while the MFMAs run on the current one.
// The tile list is derived on the device from expert_off (each workgroup
// scans it in LDS), so no host round trip is needed; blocks are remapped so
// that consecutive tiles of one (expert, N-tile) land on the same XCD and
// share its L2 copy of the weight tile.
//
// fp32 path: a plain LDS-tiled FMA kernel with the same schedule.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kXcd = 8;  // MI355X: workgroups go round-robin over 8 XCDs

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

// tile -> (expert, n-tile, m-tile); m-tiles innermost
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
  nt = rem / mte;
  mt = rem % mte;
}

__device__ __forceinline__ float silu_mul(float u, float v) { return u / (1.0f + expf(-u)) * v; }

// ---------------------------------------------------------------- bf16 MFMA

template <int BM, int BN, int WM, int WN, bool SWIGLU>
struct TileCfg {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kBK = 64;                  // K per LDS stage
  static constexpr int kChunks = kBK / 8;         // 16-byte chunks per row
  static constexpr int kWaveRows = BM / WM;
  static constexpr int kWaveCols = BN / WN;       // B rows per wave
  static constexpr int TM = kWaveRows / 32;
  static constexpr int TN = kWaveCols / 32;
  static constexpr int kOutCols = SWIGLU ? BN / 2 : BN;
  static constexpr int kALoads = BM * kChunks / kThreads;
  static constexpr int kBLoads = BN * kChunks / kThreads;
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "tile shape");
  static_assert(!SWIGLU || TN % 2 == 0, "gate/up pairs");
  static_assert((BM * kChunks) % kThreads == 0 && (BN * kChunks) % kThreads == 0, "loads");
};

template <int BM, int BN, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(WM* WN* kWave) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm_row,
    const int32_t* __restrict__ expert_off, int E, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, int K, int N0, uint16_t* __restrict__ C) {
  using Cfg = TileCfg<BM, BN, WM, WN, SWIGLU>;
  constexpr int CH = Cfg::kChunks;
  __shared__ u32x4 As[2][BM * CH];
  __shared__ u32x4 Bs[2][BN * CH];
  __shared__ Sched sc;

  build_schedule(sc, expert_off, E, BM);
  const int NT = (N0 + Cfg::kOutCols - 1) / Cfg::kOutCols;
  const int tile = xcd_logical_tile(sc.mt_off[E] * NT);
  if (tile < 0) return;
  int e, nt, mt;
  decode_tile(sc, E, NT, tile, e, nt, mt);
  const int seg0 = expert_off[e], seg1 = expert_off[e + 1];
  const int m0 = seg0 + mt * BM;
  const int c0 = nt * Cfg::kOutCols;  // first output column of the tile

  const int tid = threadIdx.x;
  // global source rows of this thread's A and B chunks (fixed over K)
  const u32x4* aptr[Cfg::kALoads];
  const u32x4* bptr[Cfg::kBLoads];
  const size_t kvec = (size_t)K / 8;  // 16-byte chunks per K row
#pragma unroll
  for (int i = 0; i < Cfg::kALoads; ++i) {
    const int q = tid + i * Cfg::kThreads;
    const int r = q / CH, c = q % CH;
    const int s = min(m0 + r, seg1 - 1);
    const int src = perm_row ? perm_row[s] : s;
    aptr[i] = reinterpret_cast<const u32x4*>(A) + (size_t)src * kvec + c;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kBLoads; ++i) {
    const int q = tid + i * Cfg::kThreads;
    const int r = q / CH, c = q % CH;
    const uint16_t* base;
    int n;
    if (SWIGLU) {
      base = r < BN / 2 ? B0 : B1;
      n = c0 + (r < BN / 2 ? r : r - BN / 2);
    } else {
      base = B0;
      n = c0 + r;
    }
    n = min(n, N0 - 1);
    bptr[i] = reinterpret_cast<const u32x4*>(base) + ((size_t)e * N0 + n) * kvec + c;
  }

  // LDS slot (16-byte units) of each staged chunk: row r, chunk c -> r*8 + (c ^ (r & 7))
  int a_lds[Cfg::kALoads], b_lds[Cfg::kBLoads];
#pragma unroll
  for (int i = 0; i < Cfg::kALoads; ++i) {
    const int q = tid + i * Cfg::kThreads;
    const int r = q / CH, c = q % CH;
    a_lds[i] = r * CH + (c ^ (r & 7));
  }
#pragma unroll
  for (int i = 0; i < Cfg::kBLoads; ++i) {
    const int q = tid + i * Cfg::kThreads;
    const int r = q / CH, c = q % CH;
    b_lds[i] = r * CH + (c ^ (r & 7));
  }

  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * Cfg::kWaveRows;
  const int li = lane & 31, lk = lane >> 5;
  // LDS slots of the MFMA fragments for k-step 0 (k-step ks adds 2*ks to the
  // chunk, i.e. XORs 2*ks into the swizzled chunk index)
  int fa_row[Cfg::TM], fb_row[Cfg::TN];
#pragma unroll
  for (int tm = 0; tm < Cfg::TM; ++tm) fa_row[tm] = arow0 + tm * 32 + li;
#pragma unroll
  for (int tn = 0; tn < Cfg::TN; ++tn) {
    int br;
    if (SWIGLU) {
      constexpr int half = Cfg::TN / 2;
      br = (tn < half ? 0 : BN / 2) + wn * (Cfg::kWaveCols / 2) + (tn % half) * 32;
    } else {
      br = wn * Cfg::kWaveCols + tn * 32;
    }
    fb_row[tn] = br + li;
  }

  f32x16 acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / Cfg::kBK;
  u32x4 ra[Cfg::kALoads], rb[Cfg::kBLoads];
#pragma unroll
  for (int i = 0; i < Cfg::kALoads; ++i) ra[i] = aptr[i][0];
#pragma unroll
  for (int i = 0; i < Cfg::kBLoads; ++i) rb[i] = bptr[i][0];
#pragma unroll
  for (int i = 0; i < Cfg::kALoads; ++i) As[0][a_lds[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < Cfg::kBLoads; ++i) Bs[0][b_lds[i]] = rb[i];
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      const size_t off = (size_t)(kt + 1) * CH;
#pragma unroll
      for (int i = 0; i < Cfg::kALoads; ++i) ra[i] = aptr[i][off];
#pragma unroll
      for (int i = 0; i < Cfg::kBLoads; ++i) rb[i] = bptr[i][off];
    }
    const u32x4* as = As[cur];
    const u32x4* bs = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < Cfg::kBK / 16; ++ks) {
      const int ch = ks * 2 + lk;
      bf16x8 fa[Cfg::TM], fb[Cfg::TN];
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
        fa[tm] = __builtin_bit_cast(bf16x8, as[fa_row[tm] * CH + (ch ^ (fa_row[tm] & 7))]);
#pragma unroll
      for (int tn = 0; tn < Cfg::TN; ++tn)
        fb[tn] = __builtin_bit_cast(bf16x8, bs[fb_row[tn] * CH + (ch ^ (fb_row[tn] & 7))]);
#pragma unroll
      for (int tm = 0; tm < Cfg::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[tm], fb[tn], acc[tm][tn], 0, 0, 0);
    }
    if (more) {
      u32x4* asn = As[cur ^ 1];
      u32x4* bsn = Bs[cur ^ 1];
#pragma unroll
      for (int i = 0; i < Cfg::kALoads; ++i) asn[a_lds[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < Cfg::kBLoads; ++i) bsn[b_lds[i]] = rb[i];
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows (r&3) + 4*(lane>>5) + 8*(r>>2)
#pragma unroll
  for (int tm = 0; tm < Cfg::TM; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + arow0 + tm * 32 + (r & 3) + 4 * lk + 8 * (r >> 2);
      if (row >= seg1) continue;
      if (SWIGLU) {
        constexpr int half = Cfg::TN / 2;
#pragma unroll
        for (int tg = 0; tg < half; ++tg) {
          const int col = c0 + wn * (Cfg::kWaveCols / 2) + tg * 32 + li;
          if (col < N0)
            C[(size_t)row * N0 + col] = f32_to_bf16(silu_mul(acc[tm][tg][r], acc[tm][tg + half][r]));
        }
      } else {
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn) {
          const int col = c0 + wn * Cfg::kWaveCols + tn * 32 + li;
          if (col < N0) C[(size_t)row * N0 + col] = f32_to_bf16(acc[tm][tn][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 SIMT

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ perm_row,
                                                       const int32_t* __restrict__ expert_off,
                                                       int E, const float* __restrict__ B0,
                                                       const float* __restrict__ B1, int K,
                                                       int N0, float* __restrict__ C) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int kOutCols = SWIGLU ? BN / 2 : BN;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ Sched sc;
  build_schedule(sc, expert_off, E, BM);
  const int NT = (N0 + kOutCols - 1) / kOutCols;
  const int tile = xcd_logical_tile(sc.mt_off[E] * NT);
  if (tile < 0) return;
  int e, nt, mt;
  decode_tile(sc, E, NT, tile, e, nt, mt);
  const int seg0 = expert_off[e], seg1 = expert_off[e + 1];
  const int m0 = seg0 + mt * BM;
  const int c0 = nt * kOutCols;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;

  // loads: 64 rows x 16 k per operand, 4 floats per thread
  const int lr = tid / 4, lk = (tid % 4) * 4;
  const int s = min(m0 + lr, seg1 - 1);
  const float* arow = A + (size_t)(perm_row ? perm_row[s] : s) * K;
  const float* bsrc;
  {
    int n;
    const float* base;
    if (SWIGLU) {
      base = lr < BN / 2 ? B0 : B1;
      n = c0 + (lr < BN / 2 ? lr : lr - BN / 2);
    } else {
      base = B0;
      n = c0 + lr;
    }
    n = min(n, N0 - 1);
    bsrc = base + ((size_t)e * N0 + n) * K;
  }
  // this thread's 4 B rows inside the tile
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bcol[j] = SWIGLU ? ((j < 2 ? 0 : BN / 2) + tx * 2 + (j & 1)) : tx * 4 + j;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    const float4 av = *reinterpret_cast<const float4*>(arow + k0 + lk);
    const float4 bv = *reinterpret_cast<const float4*>(bsrc + k0 + lk);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][bcol[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= seg1) continue;
    if (SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = c0 + tx * 2 + j;
        if (col < N0) C[(size_t)row * N0 + col] = silu_mul(acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = c0 + tx * 4 + j;
        if (col < N0) C[(size_t)row * N0 + col] = acc[i][j];
      }
    }
  }
}

// ---------------------------------------------------------------- launch

// Upper bound of sum_e ceil(M_e / BM) for sum_e M_e = rows over E experts.
inline int64_t mtile_upper(int64_t rows, int E, int BM) {
  return std::min<int64_t>(rows, (rows + (int64_t)E * (BM - 1)) / BM);
}
inline unsigned grid_for(int64_t tiles) {
  return (unsigned)(ceil_div(std::max<int64_t>(tiles, 1), kXcd) * kXcd);
}

// gate/up: BM x BN = 128 x 128 B rows (64 F columns), 2 x 2 wavefronts
constexpr int kUpBM = 128, kUpBN = 128, kUpWM = 2, kUpWN = 2;
// down: 128 x 128, 2 x 2 wavefronts
constexpr int kDnBM = 128, kDnBN = 128, kDnWM = 2, kDnWN = 2;

moe_status check_ffn(int32_t T, int32_t E, int32_t k, int32_t d, int32_t F, moe_dtype dt) {
  if (T < 0 || E < 1 || k < 1 || k > E || d < 1 || F < 1 || !valid_dtype(dt)) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || (int64_t)T * k >= (1ll << 31) || d % 64 || F % 64)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT moe_status moe_expert_gate_up(const void* x_disp, const int32_t* perm_row,
                                         const int32_t* expert_off, int32_t T, int32_t E,
                                         int32_t k, int32_t d, int32_t F, const void* w_gate,
                                         const void* w_up, moe_dtype dt, void* h,
                                         hipStream_t stream) {
  moe_status st = check_ffn(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_disp || !perm_row || !expert_off || !w_gate || !w_up || !h) return MOE_ERR_ARG;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    constexpr int kOut = kUpBN / 2;
    const int64_t tiles = mtile_upper(rows, E, kUpBM) * ceil_div(F, kOut);
    hipLaunchKernelGGL((gemm_bf16_kernel<kUpBM, kUpBN, kUpWM, kUpWN, true>), dim3(grid_for(tiles)),
                       dim3(kUpWM * kUpWN * kWave), 0, stream, static_cast<const uint16_t*>(x_disp),
                       perm_row, expert_off, E, static_cast<const uint16_t*>(w_gate),
                       static_cast<const uint16_t*>(w_up), d, F, static_cast<uint16_t*>(h));
  } else {
    const int64_t tiles = mtile_upper(rows, E, 64) * ceil_div(F, 32);
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid_for(tiles)), dim3(256), 0, stream,
                       static_cast<const float*>(x_disp), perm_row, expert_off, E,
                       static_cast<const float*>(w_gate), static_cast<const float*>(w_up), d, F,
                       static_cast<float*>(h));
  }
  return launch_status();
}

MOE_EXPORT moe_status moe_expert_down(const void* h, const int32_t* expert_off, int32_t T,
                                      int32_t E, int32_t k, int32_t d, int32_t F,
                                      const void* w_down, moe_dtype dt, void* y,
                                      hipStream_t stream) {
  moe_status st = check_ffn(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!h || !expert_off || !w_down || !y) return MOE_ERR_ARG;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    const int64_t tiles = mtile_upper(rows, E, kDnBM) * ceil_div(d, kDnBN);
    hipLaunchKernelGGL((gemm_bf16_kernel<kDnBM, kDnBN, kDnWM, kDnWN, false>),
                       dim3(grid_for(tiles)), dim3(kDnWM * kDnWN * kWave), 0, stream,
                       static_cast<const uint16_t*>(h), nullptr, expert_off, E,
                       static_cast<const uint16_t*>(w_down), nullptr, F, d,
                       static_cast<uint16_t*>(y));
  } else {
    const int64_t tiles = mtile_upper(rows, E, 64) * ceil_div(d, 64);
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid_for(tiles)), dim3(256), 0, stream,
                       static_cast<const float*>(h), nullptr, expert_off, E,
                       static_cast<const float*>(w_down), nullptr, F, d, static_cast<float*>(y));
  }
  return launch_status();
}

MOE_EXPORT moe_status moe_grouped_ffn(const void* x_disp, const int32_t* perm_row,
                                      const int32_t* expert_off, int32_t T, int32_t E, int32_t k,
                                      int32_t d, int32_t F, const void* w_gate, const void* w_up,
                                      const void* w_down, moe_dtype dt, void* h, void* y,
                                      hipStream_t stream) {
  moe_status st = moe_expert_gate_up(x_disp, perm_row, expert_off, T, E, k, d, F, w_gate, w_up,
                                     dt, h, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down(h, expert_off, T, E, k, d, F, w_down, dt, y, stream);
}
