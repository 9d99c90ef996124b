// Backward pass of the MoE layer: the exact gradient of the forward for a
// loss whose gradient at the layer output is dout.
//
// The pages train these layers: expert parallelism runs its all-to-all in
// the forward and the backward pass (Zyphra correlated expert placement
// page, English abstract). The backward steps, in order:
//   combine   dy[slot(t,j)] = g_tj dout[t],  dgates[t,j] = <dout[t], y_tj>
//   down      dh = dy W_down[e] (then SwiGLU backward with the saved u, v:
//             du = dh v silu'(u), dv = dh silu(u)),  dW_down[e] = dy^T h
//   gate/up   da = du W_gate[e] + dv W_up[e],  dW_gate[e] = du^T a,
//             dW_up[e] = dv^T a
//   dispatch  dx[t] = sum_j da[slot(t,j)]
//   routing   dlogits[t, idx[t,j]] = g_j (dg_j - sum_i g_i dg_i), else 0
//
// gfx950 mapping of the two GEMM shapes (bf16), both on the forward's DMA
// grouped GEMMs (ffn.hip):
//   data gradients (one-tile kernel): rows = an expert's slots; the weight
//     panel is read as [K][N] (output dimension contiguous): its slices are
//     DMA-loaded raw and the MFMA fragments come from gfx950's transposing
//     LDS reads; the down data gradient applies the SwiGLU backward in its
//     epilogue;
//   weight gradients (persistent kernel): the reduction runs over an
//     expert's slots; the first operand (dy, or [du dv]) is read as it lies
//     through the same transposing LDS reads, the second (h, or the
//     gathered a) is first transposed into K-contiguous rows with each
//     expert's slot range zero-padded to whole 64-wide K slices
//     (transpose_pad_kernel, through LDS); each expert's K segment is walked
//     and the result written in fp32. Each expert call runs its weight
//     gradient first, so the data gradient the next call reads is written
//     last.
// fp32 runs every GEMM on the fp32 matrix cores (gemm_bwd_f32_kernel).
#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- combine backward

// One wavefront per token: dout[t] is read once; for each choice the lane
// chunk of y's row feeds the dot product (fp32) and the scaled dout chunk is
// written to dy's row. dgates comes out of a wave reduction per choice.
// KK > 0: k == KK at compile time (the common values), so the token's slots
// and gates are read once into registers and every choice's y chunk is
// loaded before any is used; KK == 0: runtime k <= kMaxK.
// HOLD: the row is at most kBwdHoldBlocks 1 KiB blocks; dout's row is held
// in registers, every y block is read first, and the dy rows are written
// afterwards, each as one contiguous run.
constexpr int kBwdHoldBlocks = 8;
template <bool BF16, int KK, bool HOLD>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const u32x4* __restrict__ dout, const u32x4* __restrict__ y,
    const int32_t* __restrict__ slot_of, const float* __restrict__ gates, int T, int k_rt,
    int row_vecs, u32x4* __restrict__ dy, float* __restrict__ dgates) {
  constexpr int KM = KK > 0 ? KK : kMaxK;
  const int k = KK > 0 ? KK : k_rt;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * (blockDim.x / kWave) + wave;
  if (t >= T) return;
  // A negative slot is a dropped choice: no y row is read, no dy row is
  // written, and its gate gradient is 0.
  float dot[KM];
  int sl[KM];
  float gt[KM];
  bool live[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    dot[j] = 0.f;
    sl[j] = j < k ? slot_of[(size_t)t * k + j] : 0;
    live[j] = j < k && sl[j] >= 0;
    gt[j] = j < k ? gates[(size_t)t * k + j] : 0.f;
  }
  const u32x4* o = dout + (size_t)t * row_vecs;
  // Token t walks its rows' 1 KiB blocks from block t mod nblk, wrapping
  // around, so waves working at the same moment read different offsets of
  // their strided rows rather than the same HBM channels; two blocks per
  // step, all of their loads issued before any is used.
  const int nblk = (row_vecs + kWave - 1) / kWave;
  const int sb = t % nblk;
  auto widen = [&](const u32x4& ov, float (&of)[8]) {
    if (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        of[2 * q] = bf16lo(ov[q]);
        of[2 * q + 1] = bf16hi(ov[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) of[q] = __uint_as_float(ov[q]);
    }
  };
  // the dot products' share of one block (fp32, in element order)
  auto dots = [&](auto chk_c, const u32x4& ov, const u32x4 (&yv)[KM]) {
    constexpr bool CHK = decltype(chk_c)::value;
    float of[8];
    widen(ov, of);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k || (CHK && !live[j])) continue;
      if (BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          dot[j] = fmaf(of[2 * q], bf16lo(yv[j][q]), dot[j]);
          dot[j] = fmaf(of[2 * q + 1], bf16hi(yv[j][q]), dot[j]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) dot[j] = fmaf(of[q], __uint_as_float(yv[j][q]), dot[j]);
      }
    }
  };
  // g times one dout block, in the activation type
  auto scaled = [&](const u32x4& ov, float g) {
    float of[8];
    widen(ov, of);
    u32x4 w;
    if (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(g * of[2 * q], g * of[2 * q + 1]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = __float_as_uint(g * of[q]);
    }
    return w;
  };
  auto block = [&](auto chk_c, int c, const u32x4& ov, const u32x4 (&yv)[KM]) {
    constexpr bool CHK = decltype(chk_c)::value;
    dots(chk_c, ov, yv);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k || (CHK && !live[j])) continue;
      dy[(size_t)sl[j] * row_vecs + c] = scaled(ov, gt[j]);
    }
  };
  auto blk = [&](int b) {  // the row block visited at step b
    const int p = b + sb;
    return p >= nblk ? p - nblk : p;
  };
  // CHK: some choice of this token is dropped (rare); the common path has no
  // per-choice test in its loop
  auto walk = [&](auto chk_c) {
    constexpr bool CHK = decltype(chk_c)::value;
    if constexpr (HOLD) {
      // Reads and writes apart: y blocks interleaved with dy stores cost HBM
      // read/write turnarounds, and dy does not depend on y.
      u32x4 ov[kBwdHoldBlocks];
#pragma unroll
      for (int b = 0; b < kBwdHoldBlocks; ++b) {
        if (b >= nblk) break;  // uniform
        const int c = blk(b) * kWave + lane;
        ov[b] = c < row_vecs ? __builtin_nontemporal_load(o + c) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int b = 0; b < kBwdHoldBlocks; b += 2) {
        if (b >= nblk) break;  // uniform
        const int c0 = blk(b) * kWave + lane;
        const int c1 = b + 1 < nblk ? blk(b + 1) * kWave + lane : row_vecs;
        const bool ok0 = c0 < row_vecs, ok1 = c1 < row_vecs;
        u32x4 yv0[KM], yv1[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k && (!CHK || live[j])) {
            yv0[j] = ok0 ? __builtin_nontemporal_load(y + (size_t)sl[j] * row_vecs + c0) : ov[b];
            yv1[j] = ok1 ? __builtin_nontemporal_load(y + (size_t)sl[j] * row_vecs + c1)
                         : ov[b + 1];
          }
        if (ok0) dots(chk_c, ov[b], yv0);
        if (ok1) dots(chk_c, ov[b + 1], yv1);
        // One step's loads live at a time: its sums are complete (operands
        // of the empty asm statements) before the next step's loads.
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k) asm volatile("" : "+v"(dot[j]));
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j >= k || (CHK && !live[j])) continue;
        u32x4* const dr = dy + (size_t)sl[j] * row_vecs;
#pragma unroll
        for (int b = 0; b < kBwdHoldBlocks; ++b) {
          if (b >= nblk) break;  // uniform
          const int c = blk(b) * kWave + lane;
          if (c < row_vecs) dr[c] = scaled(ov[b], gt[j]);
        }
      }
    } else {
      for (int b = 0; b < nblk; b += 2) {
        const int c0 = blk(b) * kWave + lane;
        const int c1 = b + 1 < nblk ? blk(b + 1) * kWave + lane : row_vecs;
        const bool ok0 = c0 < row_vecs, ok1 = c1 < row_vecs;  // the last block may be partial
        u32x4 ov0 = {0, 0, 0, 0}, ov1 = {0, 0, 0, 0};
        u32x4 yv0[KM], yv1[KM];
        if (ok0) ov0 = __builtin_nontemporal_load(o + c0);
        if (ok1) ov1 = __builtin_nontemporal_load(o + c1);
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k && (!CHK || live[j])) {
            yv0[j] = ok0 ? __builtin_nontemporal_load(y + (size_t)sl[j] * row_vecs + c0) : ov0;
            yv1[j] = ok1 ? __builtin_nontemporal_load(y + (size_t)sl[j] * row_vecs + c1) : ov1;
          }
        if (ok0) block(chk_c, c0, ov0, yv0);
        if (ok1) block(chk_c, c1, ov1, yv1);
      }
    }
  };
  bool all_live = true;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) all_live = all_live && live[j];
  if (all_live) walk(std::false_type{});
  else walk(std::true_type{});
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j >= k) continue;
    float v = dot[j];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    if (lane == 0) dgates[(size_t)t * k + j] = v;
  }
}

// ---------------------------------------------------------------- routing backward

// One wavefront per token: lanes j < k hold the gates and their gradients;
// the inner product sum_i g_i dg_i is a wave sum; every lane then writes its
// share of the token's E logit gradients (0 for experts not chosen).
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* __restrict__ gates,
                                                        const float* __restrict__ dgates,
                                                        const int32_t* __restrict__ topk_idx,
                                                        int T, int E, int k,
                                                        float* __restrict__ dlogits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * (blockDim.x / kWave) + wave;
  if (t >= T) return;
  float g = 0.f, dg = 0.f;
  int e = -1;
  if (lane < k) {
    g = gates[(size_t)t * k + lane];
    dg = dgates[(size_t)t * k + lane];
    e = topk_idx[(size_t)t * k + lane];
  }
  float inner = g * dg;
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) inner += __shfl_xor(inner, off, kWave);
  const float mine = g * (dg - inner);
  // every lane gets the k (expert, gradient) pairs while all lanes are active
  int ej[kMaxK];
  float vj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    ej[j] = __shfl(e, j, kWave);
    vj[j] = __shfl(mine, j, kWave);
  }
  for (int c = lane; c < E; c += kWave) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < k && ej[j] == c) v = vj[j];
    dlogits[(size_t)t * E + c] = v;
  }
}

// ---------------------------------------------------------------- padded transposes

// kseg[e] = sum over e' < e of ceil(M_e' / 64) * 64 (each expert's slot count
// rounded up to whole 64-wide K slices), kseg[E] = the padded total.
// eorder[8 * cap] (cap = ceil(E / 8)): the experts in the order the
// weight-gradient GEMM walks them. Its tiles go to the 8 XCDs in 8
// contiguous ranges of cap experts each, and a tile's work grows with its
// expert's slot count, so the experts are dealt longest first (ties: lower
// expert) to the ranges in turn: rank r to range r mod 8, position r / 8;
// unused positions hold -1. What imbalance is left, the launch evens out by
// claiming across XCDs at its end. (A serial least-loaded greedy over the
// ranks balanced a little better but took about 25 us of one wavefront.)
// It also clears the weight-gradient launch's tile queue.
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t* __restrict__ expert_off,
                                                          int E, int32_t* __restrict__ kseg,
                                                          int32_t* __restrict__ eorder,
                                                          uint32_t* __restrict__ queue) {
  if (threadIdx.x < kQueueWords) queue[threadIdx.x] = 0u;
  __shared__ Sched sc;
  build_schedule(sc, expert_off, E, 64);
  const int e = threadIdx.x, cap = (E + 7) / 8;
  for (int i = threadIdx.x; i <= E; i += blockDim.x) kseg[i] = sc.mt_off[i] * 64;
  if (e < E) {  // rank by padded length, longest first (ties: lower expert)
    const int my = sc.mt_off[e + 1] - sc.mt_off[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int len = sc.mt_off[f + 1] - sc.mt_off[f];
      rank += len > my || (len == my && f < e);
    }
    eorder[(rank % 8) * cap + rank / 8] = e;  // longest first, dealt to the ranges in turn
  }
  for (int r = E + (int)threadIdx.x; r < 8 * cap; r += blockDim.x) eorder[(r % 8) * cap + r / 8] = -1;
}

// dst [W][ldk] (bf16): dst[w][kseg[e] + j] = src[row(s)][w] for slot s =
// expert_off[e] + j of expert e (row(s) = gather[s] if given), and 0 in the
// padding columns up to kseg[e+1]. Workgroup = one 64-wide K tile (inside
// one expert's padded segment) x kTrW tiles of 64 columns of src: 16-byte
// row loads into LDS, transposed reads, 16-byte row stores. The segment
// search and the gathered row indices of the K tile serve all kTrW column
// tiles (one column tile per workgroup spent most of its time on them).
constexpr int kTrW = 4;
__global__ __launch_bounds__(256) void transpose_pad_kernel(
    const uint16_t* __restrict__ src, int ld_src, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ kseg, int E, int W,
    int ldk, uint16_t* __restrict__ dst) {
  const int col0 = blockIdx.x * 64;
  if (col0 >= kseg[E]) return;  // past every segment: never read
  int lo = 0, hi = E - 1;       // last e with kseg[e] <= col0 (a non-empty segment)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kseg[mid] <= col0) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int seg0 = expert_off[e], n_e = expert_off[e + 1] - seg0, j0 = col0 - kseg[e];
  __shared__ uint16_t tile[64][64 + 8];  // [k][w], rows 144 bytes apart
  const int tid = threadIdx.x;
  int src_row[2];  // source row of this thread's two K rows (-1: padding)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid + 256 * h) >> 3;
    const int s = seg0 + j0 + r;
    src_row[h] = j0 + r < n_e ? (gather ? gather[s] : s) : -1;
  }
  for (int wt = 0; wt < kTrW; ++wt) {
    const int w0 = (blockIdx.y * kTrW + wt) * 64;
    if (w0 >= W) break;  // uniform
    if (wt > 0) __syncthreads();  // the previous column tile has been read out
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + 256 * h, r = q >> 3, c = q & 7;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (src_row[h] >= 0)
        v = *reinterpret_cast<const u32x4*>(src + (size_t)src_row[h] * ld_src + w0 + c * 8);
      *reinterpret_cast<u32x4*>(&tile[r][c * 8]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = tid + 256 * h, wr = q >> 3, kc = q & 7;
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = (uint32_t)tile[kc * 8 + 2 * i][wr] | ((uint32_t)tile[kc * 8 + 2 * i + 1][wr] << 16);
      *reinterpret_cast<u32x4*>(dst + (size_t)(w0 + wr) * ldk + col0 + kc * 8) = v;
    }
  }
}

// Padded K length of the transposed operands for S slots over E experts.
inline int64_t padded_k(int64_t S, int E) { return ceil_div(S + 63 * (int64_t)E, 64) * 64; }

// Workspace of the weight-gradient path: kseg, the expert order, the tile
// queue, then the transposed second operand.
struct WgradWorkspace {
  size_t kseg, eorder, queue, bt, total;
};
inline WgradWorkspace wgrad_workspace(int64_t S, int E, int64_t rows_b) {
  const int64_t ldk = padded_k(S, E);
  WgradWorkspace w;
  w.kseg = 0;
  w.eorder = ceil_div((E + 1) * 4, 256) * 256;
  w.queue = w.eorder + ceil_div(8 * ceil_div(E, 8) * 4, 256) * 256;
  w.bt = w.queue + 256;
  w.total = w.bt + ceil_div(rows_b * ldk * 2, 256) * 256;
  return w;
}

// The bf16 expert GEMMs of the backward load through 32-bit offsets: the
// activation-side operands (rows x K) and the expert-padded transposes.
bool bwd_bf16_fits(int64_t S, int E, int64_t k_dgrad, int64_t m0, int64_t n0) {
  const int64_t ldk = padded_k(S, E);
  return dgrad_offsets_fit(S, k_dgrad) && wgrad_offsets_fit(m0, n0, ldk) &&
         ldk < (int64_t(1) << 31);
}

// bf16 weight gradients through the forward's persistent GEMM: transpose b
// into expert-padded K-contiguous rows (zero past each expert's slots), then
// out[e] = a_e^T bt_e^T per expert segment, a read as it lies ([slots][M0]).
moe_status wgrad_bf16(const uint16_t* a, int M0, const uint16_t* b, int ldb,
                      const int32_t* b_gather, int N0, const int32_t* expert_off, int E, int64_t S,
                      int msplit, float* o0, float* o1, void* workspace, hipStream_t stream) {
  const int64_t ldk = padded_k(S, E);
  const WgradWorkspace ws = wgrad_workspace(S, E, N0);
  char* w = static_cast<char*>(workspace);
  int32_t* kseg = reinterpret_cast<int32_t*>(w + ws.kseg);
  int32_t* eorder = reinterpret_cast<int32_t*>(w + ws.eorder);
  uint32_t* queue = reinterpret_cast<uint32_t*>(w + ws.queue);
  uint16_t* bt = reinterpret_cast<uint16_t*>(w + ws.bt);
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, stream, expert_off, E, kseg,
                     eorder, queue);
  const unsigned kt = (unsigned)(ldk / 64);
  hipLaunchKernelGGL(transpose_pad_kernel, dim3(kt, (unsigned)ceil_div(N0 / 64, kTrW)), dim3(256), 0,
                     stream, b, ldb, b_gather, expert_off, kseg, E, N0, (int)ldk, bt);
  return launch_wgrad_bf16(a, bt, expert_off, kseg, eorder, E, M0, N0, (int)ldk, msplit, o0, o1,
                           queue, stream);
}

// ---------------------------------------------------------------- fp32 GEMM descriptors

enum BwdMode : int {
  kDgradSwiglu = 0,  // dh = dy W_down[e]; epilogue: SwiGLU backward -> du, dv
  kDgradPlain = 1,   // da = [du dv] [W_gate[e]; W_up[e]]
  kWgrad = 2,        // dW[e] = A_e^T B_e over the expert's slots
};

struct BwdArgs {
  const int32_t* expert_off;
  int E;
  // data gradients: C[s][n] = sum_k A[s][k] W[e][k][n], k < ksplit from W0
  // (row k), else from W1 (row k - ksplit); W panels are K x N0, estride
  // elements apart
  const uint16_t* A;
  int lda, K, N0, ksplit;
  const uint16_t* W0;
  const uint16_t* W1;
  size_t estride;
  uint16_t* C;     // plain: [S][ldc]
  int ldc;
  const uint16_t* uv;  // swiglu: saved [S][2F] (u then v), output duv [S][2F]
  uint16_t* duv;
  int F;
  // weight gradients: Out[e][m][n] = sum_s At[s][m] Bt[row(s)][n], rows m <
  // msplit to O0 (msplit x N0 per expert), the others to O1; row(s) =
  // b_gather[s] if given
  const uint16_t* At;
  int ldat, M0;
  const uint16_t* Bt;
  const int32_t* b_gather;
  int ldbt, msplit;
  float* O0;
  float* O1;
};

__device__ __forceinline__ void silu_parts(float u, float& silu, float& dsilu) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * 1.44269504088896341f));
  silu = u * sg;
  dsilu = sg * (1.0f + u * (1.0f - sg));
}

// ---------------------------------------------------------------- fp32 MFMA GEMM

// The same three GEMMs in fp32 on the fp32 matrix cores: 64 x 64 tiles,
// 16-deep K slices staged in LDS K-major through the mode's index map, and
// 4 wavefronts as 2 x 2, each accumulating a 32 x 32 block with
// v_mfma_f32_32x32x2_f32 (lane l feeds row l % 32 at k = 2i + l / 32).
template <int MODE>
__global__ __launch_bounds__(256) void gemm_bwd_f32_kernel(BwdArgs p, const float* A,
                                                           const float* W0, const float* W1,
                                                           float* C, const float* uv, float* duv,
                                                           const float* At, const float* Bt) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ __align__(16) float As[BK][BM + 4];
  __shared__ __align__(16) float Bs[BK][BN + 4];
  __shared__ Sched sc;
  int e, mt, nt, seg0, seg1, m0, c0, Kt;
  if (MODE != kWgrad) {
    build_schedule(sc, p.expert_off, p.E, BM);
    const int NT = (p.N0 + BN - 1) / BN;
    const int tile = xcd_logical_tile(sc.mt_off[p.E] * NT);
    if (tile < 0) return;
    decode_tile(sc, p.E, NT, tile, e, nt, mt);
    seg0 = p.expert_off[e];
    seg1 = p.expert_off[e + 1];
    m0 = seg0 + mt * BM;
    c0 = nt * BN;
    Kt = p.K;
  } else {
    const int MT = (p.M0 + BM - 1) / BM, NT = (p.N0 + BN - 1) / BN;
    const int tile = xcd_logical_tile(p.E * MT * NT);
    if (tile < 0) return;
    e = tile / (MT * NT);
    const int rem = tile - e * MT * NT;
    mt = rem / NT;
    nt = rem % NT;
    seg0 = p.expert_off[e];
    seg1 = p.expert_off[e + 1];
    m0 = mt * BM;
    c0 = nt * BN;
    Kt = seg1 - seg0;
  }
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int kh = lane >> 5;
  const int ar = (wave >> 1) * 32 + (lane & 31), bc = (wave & 1) * 32 + (lane & 31);
  f32x16 acc = {};
  // Each thread loads one 16-byte piece of each operand per slice. Data
  // gradients: A rows [S][K] (row tid / 4, k 4 (tid % 4) ..) and the weight
  // panel [K][N0] (k row tid / 16, n 4 (tid % 16) ..); weight gradients: At
  // [S][M0] and Bt [S][N0] (slot k0 + tid / 16, m or n 4 (tid % 16) ..). M0,
  // N0 and K are multiples of 64, so every piece is in bounds and aligned.
  // The next slice's pieces are loaded before the current one's MFMAs.
  const int r4 = tid >> 2, k4 = (tid & 3) * 4;  // data gradients: A piece
  const int kr = tid >> 4, c4 = (tid & 15) * 4;  // the other pieces
  const float* arow = nullptr;
  if (MODE != kWgrad) arow = A + (size_t)min(m0 + r4, seg1 - 1) * p.lda;
  auto load = [&](int k0, float4& av, float4& bv) {
    const int k = k0 + kr;
    if (MODE != kWgrad) {
      av = *reinterpret_cast<const float4*>(arow + k0 + k4);
      const float* w = k < p.ksplit ? W0 + (size_t)e * p.estride + (size_t)k * p.N0
                                    : W1 + (size_t)e * p.estride + (size_t)(k - p.ksplit) * p.N0;
      bv = *reinterpret_cast<const float4*>(w + c0 + c4);
    } else if (k < Kt) {
      const int s = seg0 + k;
      av = *reinterpret_cast<const float4*>(At + (size_t)s * p.ldat + m0 + c4);
      bv = *reinterpret_cast<const float4*>(Bt + (size_t)(p.b_gather ? p.b_gather[s] : s) * p.ldbt +
                                            c0 + c4);
    } else {
      av = bv = float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  float4 av, bv;
  if (Kt > 0) load(0, av, bv);
  for (int k0 = 0; k0 < Kt; k0 += BK) {
    if (MODE != kWgrad) {
      As[k4 + 0][r4] = av.x;
      As[k4 + 1][r4] = av.y;
      As[k4 + 2][r4] = av.z;
      As[k4 + 3][r4] = av.w;
    } else {
      *reinterpret_cast<float4*>(&As[kr][c4]) = av;
    }
    *reinterpret_cast<float4*>(&Bs[kr][c4]) = bv;
    __syncthreads();
    if (k0 + BK < Kt) load(k0 + BK, av, bv);
#pragma unroll
    for (int i = 0; i < BK / 2; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[2 * i + kh][ar], Bs[2 * i + kh][bc], acc, 0, 0,
                                                 0);
    __syncthreads();
  }
  // Register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4 and
  // column l % 32 of the wave's 32 x 32 block.
  const int col = c0 + bc;
  if (col >= p.N0) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + (wave >> 1) * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    if (MODE != kWgrad ? row >= seg1 : row >= p.M0) continue;
    if (MODE == kDgradPlain) {
      C[(size_t)row * p.ldc + col] = acc[r];
    } else if (MODE == kDgradSwiglu) {
      const size_t o = (size_t)row * (2 * p.F) + col;
      const float u = uv[o], v = uv[o + p.F];
      float sl, ds;
      silu_parts(u, sl, ds);
      duv[o] = acc[r] * v * ds;
      duv[o + p.F] = acc[r] * sl;
    } else {
      float* out = row < p.msplit
                       ? p.O0 + ((size_t)e * p.msplit + row) * p.N0
                       : p.O1 + ((size_t)e * (p.M0 - p.msplit) + (row - p.msplit)) * p.N0;
      out[col] = acc[r];
    }
  }
}

// ---------------------------------------------------------------- launch

template <int MODE>
void launch_gemm_f32_bwd(const BwdArgs& p, int64_t rows, hipStream_t stream) {
  const int64_t tiles = MODE == kWgrad ? (int64_t)p.E * ceil_div(p.M0, 64) * ceil_div(p.N0, 64)
                                       : mtile_upper(rows, p.E, 64) * ceil_div(p.N0, 64);
  hipLaunchKernelGGL(gemm_bwd_f32_kernel<MODE>, dim3(grid_for(tiles)), dim3(256), 0, stream, p,
                     reinterpret_cast<const float*>(p.A), reinterpret_cast<const float*>(p.W0),
                     reinterpret_cast<const float*>(p.W1), reinterpret_cast<float*>(p.C),
                     reinterpret_cast<const float*>(p.uv), reinterpret_cast<float*>(p.duv),
                     reinterpret_cast<const float*>(p.At), reinterpret_cast<const float*>(p.Bt));
}

moe_status check_bwd(int32_t T, int32_t E, int32_t k, int32_t d, int32_t F, moe_dtype dt) {
  if (T < 0 || E < 1 || k < 1 || k > E || d < 1 || F < 1 || !valid_dtype(dt)) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || (int64_t)T * k >= (1ll << 31) || d % 64 || F % 64)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if ((uintptr_t)q % 16) return true;
  return false;
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT moe_status moe_combine_bwd(const void* dout, const void* y, const int32_t* slot_of,
                                      const float* gates, int32_t T, int32_t k, int32_t d,
                                      moe_dtype dt, void* dy, float* dgates, hipStream_t stream) {
  if (T < 0 || k < 1 || d < 1 || !valid_dtype(dt)) return MOE_ERR_ARG;
  if (k > kMaxK || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dout || !y || !slot_of || !gates || !dy || !dgates) return MOE_ERR_ARG;
  if (((size_t)d * dtype_bytes(dt)) % 16 || misaligned({dout, y, dy})) return MOE_ERR_UNSUPPORTED;
  const int row_vecs = (int)((size_t)d * dtype_bytes(dt) / 16);
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  auto launch = [&](auto bf16_c, auto kk_c) {
    constexpr bool B = decltype(bf16_c)::value;
    constexpr int KV = decltype(kk_c)::value;
    if (row_vecs <= kBwdHoldBlocks * kWave)
      hipLaunchKernelGGL((combine_bwd_kernel<B, KV, true>), grid, block, 0, stream,
                         static_cast<const u32x4*>(dout), static_cast<const u32x4*>(y), slot_of,
                         gates, T, k, row_vecs, static_cast<u32x4*>(dy), dgates);
    else
      hipLaunchKernelGGL((combine_bwd_kernel<B, KV, false>), grid, block, 0, stream,
                         static_cast<const u32x4*>(dout), static_cast<const u32x4*>(y), slot_of,
                         gates, T, k, row_vecs, static_cast<u32x4*>(dy), dgates);
  };
  auto by_k = [&](auto bf16_c) {
    switch (k) {
      case 1: launch(bf16_c, std::integral_constant<int, 1>{}); break;
      case 2: launch(bf16_c, std::integral_constant<int, 2>{}); break;
      case 4: launch(bf16_c, std::integral_constant<int, 4>{}); break;
      case 6: launch(bf16_c, std::integral_constant<int, 6>{}); break;
      case 8: launch(bf16_c, std::integral_constant<int, 8>{}); break;
      default: launch(bf16_c, std::integral_constant<int, 0>{}); break;
    }
  };
  if (dt == MOE_BF16) by_k(std::true_type{});
  else by_k(std::false_type{});
  return launch_status();
}

MOE_EXPORT size_t moe_expert_bwd_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t d,
                                                 int32_t F) {
  if (T < 0 || E < 1 || k < 1 || d < 1 || F < 1) return 0;
  const int64_t S = (int64_t)T * k;
  const size_t a = wgrad_workspace(S, E, F).total;  // down: h^T
  const size_t b = wgrad_workspace(S, E, d).total;  // gate/up: gathered a^T
  return std::max(a, b);
}

MOE_EXPORT moe_status moe_expert_down_bwd(const void* dy, const void* h, const void* uv,
                                          const int32_t* expert_off, int32_t T, int32_t E,
                                          int32_t k, int32_t d, int32_t F, const void* w_down,
                                          moe_dtype dt, void* duv, float* dw_down,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  moe_status st = check_bwd(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (!expert_off || !w_down || !dw_down || (T > 0 && (!dy || !h || !uv || !duv)))
    return MOE_ERR_ARG;
  if (misaligned({dy, h, uv, w_down, duv, dw_down})) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    if (!workspace || workspace_bytes < moe_expert_bwd_workspace_bytes(T, E, k, d, F) ||
        (uintptr_t)workspace % 16)
      return MOE_ERR_WORKSPACE;
    if (!bwd_bf16_fits(rows, E, d, d, F)) return MOE_ERR_UNSUPPORTED;
    // dW_down[e] = dy^T h over the expert's slots (first: the data gradient's
    // output, du dv, is what the next call reads, so it is written last)
    st = wgrad_bf16(static_cast<const uint16_t*>(dy), d, static_cast<const uint16_t*>(h), F,
                    nullptr, F, expert_off, E, rows, d, dw_down, dw_down, workspace, stream);
    if (st != MOE_OK) return st;
    // dh = dy W_down[e] (W_down[e] = d x F = K x N0), SwiGLU backward in the epilogue
    if (rows > 0)
      launch_dgrad_bf16(static_cast<const uint16_t*>(dy), rows, expert_off, E, d,
                        static_cast<const uint16_t*>(w_down), static_cast<const uint16_t*>(w_down),
                        d, F, static_cast<const uint16_t*>(uv), static_cast<uint16_t*>(duv), stream);
    return launch_status();
  }
  BwdArgs p = {};
  p.expert_off = expert_off;
  p.E = E;
  p.A = static_cast<const uint16_t*>(dy);
  p.lda = d;
  p.K = d;
  p.N0 = F;
  p.ksplit = d;
  p.W0 = p.W1 = static_cast<const uint16_t*>(w_down);
  p.estride = (size_t)d * F;
  p.uv = static_cast<const uint16_t*>(uv);
  p.duv = static_cast<uint16_t*>(duv);
  p.F = F;
  if (rows > 0) launch_gemm_f32_bwd<kDgradSwiglu>(p, rows, stream);
  BwdArgs q = {};
  q.expert_off = expert_off;
  q.E = E;
  q.At = static_cast<const uint16_t*>(dy);
  q.ldat = d;
  q.M0 = d;
  q.Bt = static_cast<const uint16_t*>(h);
  q.ldbt = F;
  q.N0 = F;
  q.msplit = d;
  q.O0 = q.O1 = dw_down;
  launch_gemm_f32_bwd<kWgrad>(q, rows, stream);
  return launch_status();
}

MOE_EXPORT moe_status moe_expert_gate_up_bwd(const void* duv, const void* x_disp,
                                             const int32_t* perm_row, const int32_t* expert_off,
                                             int32_t T, int32_t E, int32_t k, int32_t d,
                                             int32_t F, const void* w_gate, const void* w_up,
                                             moe_dtype dt, void* da, float* dw_gate,
                                             float* dw_up, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_bwd(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (!expert_off || !w_gate || !w_up || !dw_gate || !dw_up ||
      (T > 0 && (!duv || !x_disp || !perm_row || !da)))
    return MOE_ERR_ARG;
  if (misaligned({duv, x_disp, w_gate, w_up, da, dw_gate, dw_up})) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    if (!workspace || workspace_bytes < moe_expert_bwd_workspace_bytes(T, E, k, d, F) ||
        (uintptr_t)workspace % 16)
      return MOE_ERR_WORKSPACE;
    if (!bwd_bf16_fits(rows, E, 2 * F, 2 * F, d)) return MOE_ERR_UNSUPPORTED;
    // [dW_gate; dW_up][e] = [du dv]^T a over the expert's slots, a = x_disp[perm_row[s]]
    // (first: da, which the dispatch backward reads next, is written last)
    st = wgrad_bf16(static_cast<const uint16_t*>(duv), 2 * F, static_cast<const uint16_t*>(x_disp),
                    d, perm_row, d, expert_off, E, rows, F, dw_gate, dw_up, workspace, stream);
    if (st != MOE_OK) return st;
    // da = du W_gate[e] + dv W_up[e]: K = 2F (rows of W_gate[e], then of W_up[e]), N0 = d
    if (rows > 0)
      launch_dgrad_bf16(static_cast<const uint16_t*>(duv), rows, expert_off, E, 2 * F,
                        static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
                        F, d, nullptr, static_cast<uint16_t*>(da), stream);
    return launch_status();
  }
  BwdArgs p = {};
  p.expert_off = expert_off;
  p.E = E;
  p.A = static_cast<const uint16_t*>(duv);
  p.lda = 2 * F;
  p.K = 2 * F;
  p.N0 = d;
  p.ksplit = F;
  p.W0 = static_cast<const uint16_t*>(w_gate);
  p.W1 = static_cast<const uint16_t*>(w_up);
  p.estride = (size_t)F * d;
  p.C = static_cast<uint16_t*>(da);
  p.ldc = d;
  if (rows > 0) launch_gemm_f32_bwd<kDgradPlain>(p, rows, stream);
  BwdArgs q = {};
  q.expert_off = expert_off;
  q.E = E;
  q.At = static_cast<const uint16_t*>(duv);
  q.ldat = 2 * F;
  q.M0 = 2 * F;
  q.Bt = static_cast<const uint16_t*>(x_disp);
  q.b_gather = perm_row;
  q.ldbt = d;
  q.N0 = d;
  q.msplit = F;
  q.O0 = dw_gate;
  q.O1 = dw_up;
  launch_gemm_f32_bwd<kWgrad>(q, rows, stream);
  return launch_status();
}

MOE_EXPORT moe_status moe_dispatch_bwd(const void* da, const int32_t* slot_of, int32_t T,
                                       int32_t k, int32_t d, moe_dtype dt, void* dx,
                                       hipStream_t stream) {
  // dx[t] = sum_j da[slot(t, j)]: the combine with every gate equal to one
  return moe_combine(da, slot_of, nullptr, T, k, d, dt, dx, stream);
}

MOE_EXPORT moe_status moe_route_bwd(const float* gates, const float* dgates,
                                    const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                    float* dlogits, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if (k > kMaxK || E > 1024 || (int64_t)T * E >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!gates || !dgates || !topk_idx || !dlogits) return MOE_ERR_ARG;
  hipLaunchKernelGGL(route_bwd_kernel, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0, stream,
                     gates, dgates, topk_idx, T, E, k, dlogits);
  return launch_status();
}
