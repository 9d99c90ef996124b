// Dispatch layout: once-per-rank rows and the expert-grouped slot order.
//
// Zyphra correlated expert placement page, English abstract: experts sit on
// GPUs according to a placement, and the dispatcher sends each token to each
// GPU once. Here the G expert-parallel ranks are a map: the layout built is
// exactly the send plan of such a dispatcher, and the dispatched rows are
// the bytes it would send.
//
// Orders (fixed so that results are reproducible bit for bit):
//  rows  : rank by rank, tokens ascending within a rank;
//  slots : experts ascending, tokens ascending within an expert.
//
// gfx950 mapping. Tokens are cut into blocks of 256 (one per lane of a
// 256-thread workgroup). A block sets one bit per (key, token) in LDS
// bitmaps (key = expert or rank, 8 words of 32 tokens each) with atomicOr,
// which commutes, so the bitmaps do not depend on timing. The stable rank of
// a token among the block's tokens with the same key is the popcount of the
// bits before it. Two launches:
//   count : per-block key counts, the bitmaps and their per-word prefix
//           counts (to the workspace), and rank_mask; the last block to
//           finish turns the counts into per-block bases and the
//           expert_off / rank_off prefixes (no host round trip: R stays on
//           the device);
//   token : one wavefront per token finds its rows and slots from the
//           bases and bitmaps (a lane per rank and per chosen expert),
//           writes disp_token, perm_row and slot_of, then reads the token's
//           row once and writes it to each of its rows (16 bytes per lane).
#include "moe_internal.h"

#include <atomic>

namespace moe {
namespace {

constexpr int kBlockTok = 256;
constexpr int kWords = kBlockTok / 32;

struct BlockMasks {
  uint32_t emask[kMaxE * kWords];
  uint32_t rmask[kMaxG * kWords];
  int32_t place[kMaxE];
  int32_t idx[kBlockTok * kMaxK];  // the block's routing choices
};

// Builds the block's bitmaps; returns the token's rank mask (0 if t >= T).
// A choice's rank is place[expert], or rank_of[t * k + j] when rank_of is
// given (replica-aware assignment). The block's choices are first staged in
// LDS, all loads issued before the LDS is cleared, so the loop over a
// token's choices waits for no memory. The loads are 16 bytes wide when
// topk_idx is 16-byte aligned (a block's chunk starts 1024 k bytes in),
// 4 bytes otherwise.
__device__ uint32_t build_masks(BlockMasks& sm, const int32_t* __restrict__ topk_idx, int T,
                                int E, int k, const int32_t* __restrict__ place,
                                const int32_t* __restrict__ rank_of, int G) {
  const int tb = blockIdx.x * kBlockTok;
  const int n = min(kBlockTok, T - tb) * k;
  {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(topk_idx + (size_t)tb * k);
    const int nv = (reinterpret_cast<uintptr_t>(topk_idx) & 15) ? 0 : n / 4;
    u32x4 v[4];
    int pl = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { const int i = threadIdx.x + j * kBlockTok; if (i < nv) v[j] = s4[i]; }
    if (!rank_of && (int)threadIdx.x < E) pl = place[threadIdx.x];
    for (int i = threadIdx.x; i < E * kWords; i += blockDim.x) sm.emask[i] = 0u;
    for (int i = threadIdx.x; i < G * kWords; i += blockDim.x) sm.rmask[i] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) { const int i = threadIdx.x + j * kBlockTok; if (i < nv) reinterpret_cast<u32x4*>(sm.idx)[i] = v[j]; }
    for (int i = 4 * nv + threadIdx.x; i < n; i += kBlockTok) sm.idx[i] = topk_idx[(size_t)tb * k + i];
    if (!rank_of && (int)threadIdx.x < E) sm.place[threadIdx.x] = pl;
  }
  __syncthreads();
  const int t = tb + threadIdx.x;
  const int w = threadIdx.x >> 5;
  const uint32_t bit = 1u << (threadIdx.x & 31);
  uint32_t m = 0u;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = sm.idx[threadIdx.x * k + j];
      if (e < 0 || e >= E) continue;
      const int g = rank_of ? rank_of[(size_t)t * k + j] : sm.place[e];
      if (g < 0 || g >= G) continue;
      atomicOr(&sm.emask[e * kWords + w], bit);
      m |= 1u << g;
    }
    for (uint32_t mm = m; mm; mm &= mm - 1) atomicOr(&sm.rmask[(__ffs(mm) - 1) * kWords + w], bit);
  }
  __syncthreads();
  return m;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive scan of n <= 256 values held in LDS by one wavefront (4 per lane).
__device__ void wave_excl_scan_256(const int32_t* in, int32_t* out, int n, int32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = lane * 4 + i;
    v[i] = q < n ? in[q] : 0;
    s += v[i];
  }
  const int incl = wave_incl_scan(s);
  int run = incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = lane * 4 + i;
    if (q < n) out[q] = run;
    run += v[i];
  }
  if (lane == kWave - 1) *total = incl;
}

// Per-key totals over the blocks, the two exclusive scans, then per-block
// bases, by one workgroup (the last count block to finish). A thread owns a
// key and walks the blocks in chunks of kScanChunk whose loads are all
// issued before any is used, so the walk costs nblk / kScanChunk memory
// round trips instead of nblk. The counts are read with device-coherent
// loads: other workgroups wrote them.
constexpr int kScanChunk = 8;

__device__ __forceinline__ int load_cnt(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct ScanSmem {
  int32_t tot[kMaxE + kMaxG];
  int32_t off[kMaxE + kMaxG];
};

// Up to kScanFast blocks with one key per thread: every count of the
// thread's key is loaded in one round (all loads issued before any is used)
// and kept in registers for the bases, instead of two walks in chunks.
constexpr int kScanFast = 32;

__device__ void scan_blocks(ScanSmem& sm, int32_t* __restrict__ cnt, int nblk, int E, int G,
                            int32_t* __restrict__ expert_off, int32_t* __restrict__ rank_off) {
  const int Q = E + G;
  if (nblk <= kScanFast && Q <= (int)blockDim.x) {  // uniform
    const int q = threadIdx.x;
    int c[kScanFast];
#pragma unroll
    for (int i = 0; i < kScanFast; ++i)
      c[i] = q < Q && i < nblk ? load_cnt(&cnt[(size_t)i * Q + q]) : 0;
    int s = 0;
#pragma unroll
    for (int i = 0; i < kScanFast; ++i) s += c[i];
    if (q < Q) sm.tot[q] = s;
    __syncthreads();
    const int wave = threadIdx.x / kWave;
    if (wave == 0) wave_excl_scan_256(sm.tot, sm.off, E, &expert_off[E]);
    if (wave == 1) wave_excl_scan_256(sm.tot + E, sm.off + E, G, &rank_off[G]);
    __syncthreads();
    if (q < Q) {
      int run = sm.off[q];
      if (q < E) expert_off[q] = run;
      else rank_off[q - E] = run;
#pragma unroll
      for (int i = 0; i < kScanFast; ++i) {
        if (i < nblk) cnt[(size_t)i * Q + q] = run;
        run += c[i];
      }
    }
    return;
  }
  for (int q = threadIdx.x; q < Q; q += blockDim.x) {
    int s = 0;
    for (int b0 = 0; b0 < nblk; b0 += kScanChunk) {
      int c[kScanChunk];
#pragma unroll
      for (int i = 0; i < kScanChunk; ++i)
        c[i] = b0 + i < nblk ? load_cnt(&cnt[(size_t)(b0 + i) * Q + q]) : 0;
#pragma unroll
      for (int i = 0; i < kScanChunk; ++i) s += c[i];
    }
    sm.tot[q] = s;
  }
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  if (wave == 0) wave_excl_scan_256(sm.tot, sm.off, E, &expert_off[E]);
  if (wave == 1) wave_excl_scan_256(sm.tot + E, sm.off + E, G, &rank_off[G]);
  __syncthreads();
  for (int q = threadIdx.x; q < Q; q += blockDim.x) {
    int run = sm.off[q];
    if (q < E) expert_off[q] = run;
    else rank_off[q - E] = run;
    for (int b0 = 0; b0 < nblk; b0 += kScanChunk) {
      int c[kScanChunk];
#pragma unroll
      for (int i = 0; i < kScanChunk; ++i)
        c[i] = b0 + i < nblk ? load_cnt(&cnt[(size_t)(b0 + i) * Q + q]) : 0;
#pragma unroll
      for (int i = 0; i < kScanChunk; ++i) {
        if (b0 + i < nblk) cnt[(size_t)(b0 + i) * Q + q] = run;
        run += c[i];
      }
    }
  }
}

// An empty batch: no count blocks, so one workgroup writes the zero offsets.
__global__ __launch_bounds__(256) void layout_empty_kernel(int E, int G,
                                                           int32_t* __restrict__ expert_off,
                                                           int32_t* __restrict__ rank_off) {
  for (int q = threadIdx.x; q <= E; q += blockDim.x) expert_off[q] = 0;
  for (int q = threadIdx.x; q <= G; q += blockDim.x) rank_off[q] = 0;
}

// Per block and key q (experts 0..E-1, then ranks): cnt[b][q] = tokens of
// block b with key q; wmask[b][q][w] = the key's bitmap word w and
// wpre[b][q][w] = popcount of words 0..w-1 (a token's rank within the block
// is wpre + popcount of the bits before it in its word).
// The last block to finish (a counter in the workspace, which that block
// sets back to zero) then turns the counts into per-block bases and the
// expert / rank offsets, so the layout needs no separate scan launch.
__global__ __launch_bounds__(kBlockTok) void layout_count_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int k, const int32_t* __restrict__ place,
    const int32_t* __restrict__ rank_of, int G, uint32_t* __restrict__ rank_mask,
    int32_t* __restrict__ cnt, uint32_t* __restrict__ wmask, int32_t* __restrict__ wpre,
    uint32_t* __restrict__ done, int32_t* __restrict__ expert_off,
    int32_t* __restrict__ rank_off) {
  __shared__ BlockMasks sm;
  __shared__ ScanSmem ssm;
  __shared__ int last;
  const uint32_t m = build_masks(sm, topk_idx, T, E, k, place, rank_of, G);
  const int t = blockIdx.x * kBlockTok + threadIdx.x;
  if (t < T) rank_mask[t] = m;
  const int Q = E + G;
  uint32_t* wm = wmask + (size_t)blockIdx.x * Q * kWords;
  int32_t* wp = wpre + (size_t)blockIdx.x * Q * kWords;
  for (int q = threadIdx.x; q < Q; q += blockDim.x) {
    const uint32_t* mk = q < E ? &sm.emask[q * kWords] : &sm.rmask[(q - E) * kWords];
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) {
      wm[q * kWords + w] = mk[w];
      wp[q * kWords + w] = c;
      c += __popc(mk[w]);
    }
    // device-scope store: written through to where other XCDs' device-scope
    // loads read it (a release fence would instead write back this XCD's
    // whole L2, which costs more than the scan saves)
    __hip_atomic_store(&cnt[(size_t)blockIdx.x * Q + q], c, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // every count of this block has been written through (the stores are
  // complete) before the block is counted as finished
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           gridDim.x - 1;
  __syncthreads();
  if (!last) return;  // uniform
  scan_blocks(ssm, cnt, gridDim.x, E, G, expert_off, rank_off);
  if (threadIdx.x == 0)  // zero again for the next call
    __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wavefront per token. Lane i < n handles the token's i-th rank (in
// ascending rank order): row = base + wpre + popcount of the bits before the
// token. Lane j < k handles choice j: its slot likewise from the expert's
// bitmap, and the row of its expert's rank comes from the rank lane by a
// lane shuffle. If x is given, the token's row is read once (eight 1 KiB
// blocks per step, the whole 8 KiB row at d = 4096 bf16; the first step is
// issued with the first index loads) and written to each of its rows.
__global__ __launch_bounds__(256) void dispatch_token_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int k, const int32_t* __restrict__ place,
    const int32_t* __restrict__ rank_of, int G, const uint32_t* __restrict__ rank_mask,
    const int32_t* __restrict__ base,
    const uint32_t* __restrict__ wmask, const int32_t* __restrict__ wpre,
    int32_t* __restrict__ disp_token, int32_t* __restrict__ perm_row,
    int32_t* __restrict__ slot_of, const u32x4* __restrict__ x, int row_vecs,
    u32x4* __restrict__ x_disp) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t = blockIdx.x * (blockDim.x / kWave) + wave;  // wave-uniform
  if (t >= T) return;
  const int Q = E + G;
  const int b = t / kBlockTok, tl = t % kBlockTok, w = tl >> 5;
  const uint32_t below = (1u << (tl & 31)) - 1u;
  const int32_t* bb = base + (size_t)b * Q;
  const uint32_t* wm = wmask + (size_t)b * Q * kWords;
  const int32_t* wp = wpre + (size_t)b * Q * kWords;
  const uint32_t m = rank_mask[t];
  const int e_lane = lane < k ? topk_idx[(size_t)t * k + lane] : -1;
  // The token's row is loaded here, right behind the first index loads and
  // before the dependent ones, so its HBM latency overlaps the row and slot
  // computation instead of following it.
  constexpr int U = 8;
  const u32x4* src = x ? x + (size_t)t * row_vecs : x;
  u32x4 v0[U];
  if (x) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = u * kWave + lane;
      if (c < row_vecs) v0[u] = __builtin_nontemporal_load(src + c);
    }
  }
  const int n = __popc(m);
  // rank lanes
  int row = 0;
  if (lane < n) {
    uint32_t mm = m;
    for (int i = 0; i < lane; ++i) mm &= mm - 1;  // drop the lane lowest ranks
    const int q = E + __ffs(mm) - 1;
    row = bb[q] + wp[q * kWords + w] + __popc(wm[q * kWords + w] & below);
    disp_token[row] = t;
  }
  // choice lanes
  int g = -1, s = 0;
  if (lane < k) {
    const int e = e_lane;
    if (e >= 0 && e < E) {
      const int pe = rank_of ? rank_of[(size_t)t * k + lane] : place[e];
      if (pe >= 0 && pe < G) {
        g = pe;
        s = bb[e] + wp[e * kWords + w] + __popc(wm[e * kWords + w] & below);
      }
    }
  }
  const int src_lane = g >= 0 ? __popc(m & ((1u << g) - 1u)) : 0;
  const int grow = __shfl(row, src_lane, kWave);
  if (g >= 0) perm_row[s] = grow;
  if (lane < k) slot_of[(size_t)t * k + lane] = g >= 0 ? s : -1;  // -1: dropped choice
  if (!x) return;
  // One register set for the row: later chunks (rows longer than 8 KiB)
  // reload into it, so the kernel keeps more wavefronts in flight.
  for (int c0 = 0; c0 < row_vecs; c0 += kWave * U) {
    if (c0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < row_vecs) v0[u] = __builtin_nontemporal_load(src + c);
      }
    }
    for (int i = 0; i < n; ++i) {
      u32x4* dst = x_disp + (size_t)__builtin_amdgcn_readlane(row, i) * row_vecs;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < row_vecs) dst[c] = v0[u];
      }
    }
  }
}

// Replica-aware assignment (Cobalt page, English abstract: route each token
// to fewer remote nodes given where the expert replicas are). A greedy
// cover per token: while choices remain, take the node holding a copy of the
// most remaining choices (ties: the token's home node, then the lower node)
// and give it every remaining choice it can serve; inside that node, while
// its choices remain, take the rank holding the most of them (ties: the home
// rank, then the lower rank) and give it all it holds. Home rank = t * G / T
// (tokens sharded in order over the ranks). A choice whose expert is out of
// range or has no copy gets rank -1.
//
// gfx950 mapping: one lane per (token, choice). A token owns a group of P
// consecutive lanes (P = power of two >= k, at most 16), so a wavefront holds
// 64 / P tokens and the counts of the greedy are popcounts of one wave ballot
// masked to the group. Every decision depends only on the group's ballots,
// so the lanes of a group always take the same branch.
__global__ __launch_bounds__(256) void replica_assign_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int k, int log_p,
    const uint32_t* __restrict__ rep_mask, int G, int rpn, int32_t* __restrict__ rank_of,
    uint32_t* __restrict__ node_mask) {
  const int lane = threadIdx.x & (kWave - 1);
  const int P = 1 << log_p;
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(gt >> log_p);
  const int j = lane & (P - 1);
  const uint64_t grp = (P == kWave ? ~0ull : ((1ull << P) - 1ull)) << (lane & ~(P - 1));
  const bool mine = t < T && j < k;
  uint32_t cm = 0;
  if (mine) {
    const int e = topk_idx[(size_t)t * k + j];
    if (e >= 0 && e < E) cm = rep_mask[e] & (G == 32 ? 0xFFFFFFFFu : ((1u << G) - 1u));
  }
  const int home = t < T ? (int)((int64_t)t * G / T) : 0;
  const int hnode = home / rpn, nodes = G / rpn;
  const uint32_t node0 = rpn == 32 ? 0xFFFFFFFFu : ((1u << rpn) - 1u);
  uint64_t left = __ballot(cm != 0u) & grp;
  int32_t rk = -1;
  uint32_t nm = 0;
  while (left) {
    const bool in_left = (left >> lane) & 1ull;
    int best = 0, bc = -1;
    uint64_t bj = 0;
    for (int n = 0; n < nodes; ++n) {
      const uint64_t jm = __ballot(in_left && (cm & (node0 << (n * rpn))) != 0u) & grp;
      const int c = __popcll(jm);
      if (c > bc || (c == bc && n == hnode && best != hnode)) {
        best = n;
        bc = c;
        bj = jm;
      }
    }
    left &= ~bj;
    nm |= 1u << best;
    while (bj) {
      const bool in_node = (bj >> lane) & 1ull;
      int br = 0, brc = -1;
      uint64_t brj = 0;
      for (int r = best * rpn; r < (best + 1) * rpn; ++r) {
        const uint64_t jm = __ballot(in_node && ((cm >> r) & 1u)) & grp;
        const int c = __popcll(jm);
        if (c > brc || (c == brc && r == home && br != home)) {
          br = r;
          brc = c;
          brj = jm;
        }
      }
      if ((brj >> lane) & 1ull) rk = br;
      bj &= ~brj;
    }
  }
  if (mine) rank_of[(size_t)t * k + j] = rk;
  if (t < T && j == 0) node_mask[t] = nm;
}

// Token shuffling destinations (Zyphra correlated expert placement page,
// English abstract: under sequence parallelism each token moves, during the
// reduce-scatter after attention, to the GPU predicted to hold its
// next-layer experts). Token t goes to the rank g with the largest score
// sum_j aff[want[t, j]][g] over its valid experts (ties: its home rank
// t * G / T, then the lowest rank).
//
// gfx950 mapping: one lane per (token, rank). A token owns P consecutive
// lanes (P = power of two >= G), so a wavefront scores 64 / P tokens; each
// lane gathers its rank's column entry of the token's k table rows (the
// table is E * G * 4 bytes and stays in cache), the group maximum is an xor
// butterfly over P lanes, and a ballot of the lanes at the maximum applies
// the tie rules. Block 0 also writes the identity map rank -> rank that the
// layout kernels use as the placement of the "experts" 0..G-1.
__global__ __launch_bounds__(256) void token_dest_kernel(
    const int32_t* __restrict__ want, int T, int E, int k, const int32_t* __restrict__ aff, int G,
    int log_p, int32_t* __restrict__ dest, int32_t* __restrict__ ident) {
  if (blockIdx.x == 0 && threadIdx.x < (unsigned)G) ident[threadIdx.x] = threadIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int P = 1 << log_p;
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int t = (int)(gt >> log_p);
  const int g = lane & (P - 1);
  const int base = lane & ~(P - 1);
  int64_t sc = INT64_MIN;
  if (t < T && g < G) {
    sc = 0;
    for (int j = 0; j < k; ++j) {
      const int e = want[(size_t)t * k + j];
      if (e >= 0 && e < E) sc += aff[(size_t)e * G + g];
    }
  }
  int64_t mx = sc;
  for (int off = 1; off < P; off <<= 1) {
    const int64_t o = __shfl_xor((long long)mx, off, kWave);
    mx = o > mx ? o : mx;
  }
  const uint64_t grp = (P == kWave ? ~0ull : ((1ull << P) - 1ull)) << base;
  const uint64_t top = __ballot(t < T && g < G && sc == mx) & grp;
  if (t < T && g == 0) {
    const int home = (int)((int64_t)t * G / T);
    dest[t] = ((top >> (base + home)) & 1ull) ? home : __ffsll((unsigned long long)top) - 1 - base;
  }
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace: the finished-block counter (first 256 bytes; zero before the
// first call, and every call leaves it zero), then per-block key counts
// (turned into bases), the key bitmaps and their word prefixes.
struct Workspace {
  size_t done_bytes, cnt_bytes, mask_bytes, total;
};
inline Workspace workspace_layout(int32_t T, int32_t E, int32_t k, int32_t G) {
  (void)k;
  Workspace w;
  const size_t nblk = (size_t)ceil_div(T, kBlockTok);
  w.done_bytes = kAlign;
  w.cnt_bytes = align_up(nblk * (size_t)(E + G) * sizeof(int32_t));
  w.mask_bytes = align_up(nblk * (size_t)(E + G) * kWords * sizeof(uint32_t));
  w.total = w.done_bytes + w.cnt_bytes + 2 * w.mask_bytes;
  return w;
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT size_t moe_dispatch_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t G) {
  if (T < 0 || E < 1 || k < 1 || G < 1) return 0;
  return workspace_layout(T, E, k, G).total;
}

namespace moe {
namespace {

moe_status layout_impl(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                       const int32_t* place, const int32_t* rank_of, int32_t G, const void* x,
                       int32_t d, moe_dtype dt, uint32_t* rank_mask, int32_t* rank_off,
                       int32_t* disp_token, int32_t* expert_off, int32_t* perm_row,
                       int32_t* slot_of, void* x_disp, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (T > 0 && (!topk_idx || !rank_mask || !disp_token || !perm_row || !slot_of))
    return MOE_ERR_ARG;
  if (!rank_off || !expert_off) return MOE_ERR_ARG;
  if (x) {
    if (!valid_dtype(dt) || d < 1 || (T > 0 && !x_disp)) return MOE_ERR_ARG;
    if (((size_t)d * dtype_bytes(dt)) % 16 != 0 || (uintptr_t)x % 16 || (uintptr_t)x_disp % 16)
      return MOE_ERR_UNSUPPORTED;
  }
  const Workspace ws = workspace_layout(T, E, k, G);
  if (!workspace || workspace_bytes < ws.total) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)workspace % 16) return MOE_ERR_WORKSPACE;
  char* wsp = static_cast<char*>(workspace);
  uint32_t* done = reinterpret_cast<uint32_t*>(wsp);
  int32_t* cnt = reinterpret_cast<int32_t*>(wsp + ws.done_bytes);
  uint32_t* wmask = reinterpret_cast<uint32_t*>(wsp + ws.done_bytes + ws.cnt_bytes);
  int32_t* wpre = reinterpret_cast<int32_t*>(wsp + ws.done_bytes + ws.cnt_bytes + ws.mask_bytes);
  const int nblk = (int)ceil_div(T, kBlockTok);

  if (nblk > 0)
    hipLaunchKernelGGL(layout_count_kernel, dim3(nblk), dim3(kBlockTok), 0, stream, topk_idx, T,
                       E, k, place, rank_of, G, rank_mask, cnt, wmask, wpre, done, expert_off,
                       rank_off);
  else
    hipLaunchKernelGGL(layout_empty_kernel, dim3(1), dim3(256), 0, stream, E, G, expert_off,
                       rank_off);
  if (nblk > 0) {
    const int row_vecs = x ? (int)((size_t)d * dtype_bytes(dt) / 16) : 0;
    hipLaunchKernelGGL(dispatch_token_kernel, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0,
                       stream, topk_idx, T, E, k, place, rank_of, G, rank_mask, cnt, wmask, wpre,
                       disp_token, perm_row, slot_of, static_cast<const u32x4*>(x), row_vecs,
                       static_cast<u32x4*>(x_disp));
  }
  return launch_status();
}

}  // namespace
}  // namespace moe

MOE_EXPORT moe_status moe_dispatch_layout(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                          const int32_t* place, int32_t G, const void* x, int32_t d,
                                          moe_dtype dt, uint32_t* rank_mask, int32_t* rank_off,
                                          int32_t* disp_token, int32_t* expert_off,
                                          int32_t* perm_row, int32_t* slot_of, void* x_disp,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || G < 1) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || G > kMaxG || (int64_t)T * k >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  if (!place) return MOE_ERR_ARG;
  return layout_impl(topk_idx, T, E, k, place, nullptr, G, x, d, dt, rank_mask, rank_off,
                     disp_token, expert_off, perm_row, slot_of, x_disp, workspace,
                     workspace_bytes, stream);
}

namespace moe {
namespace {

// Scratch of moe_dispatch_layout_noalloc: the layout workspace (the
// finished-block counter, per-block key counts, bitmaps and their word
// prefixes) in a file-scope device array, so that call allocates nothing.
// Each device holds its own copy at its own address until the process ends;
// host code uses the address hipGetSymbolAddress returns on that device,
// never the array's name (a host-side stand-in). The counter must start at
// zero: the array does (static storage is zero-filled when the code object
// loads), and every call sets it back to zero; everything else is written
// before it is read.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static_assert(kNoAllocScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "header and library agree");
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per
// device), or nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);  // racing threads store the same value
  return p;
}

}  // namespace
}  // namespace moe

MOE_EXPORT moe_status moe_dispatch_layout_noalloc(const int32_t* topk_idx, int32_t T, int32_t E,
                                                  int32_t k, const int32_t* place, int32_t G,
                                                  const void* x, int32_t d, moe_dtype dt,
                                                  uint32_t* rank_mask, int32_t* rank_off,
                                                  int32_t* disp_token, int32_t* expert_off,
                                                  int32_t* perm_row, int32_t* slot_of,
                                                  void* x_disp, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || G < 1) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || G > kMaxG || (int64_t)T * k >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  if (!place) return MOE_ERR_ARG;
  if (workspace_layout(T, E, k, G).total > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_DEVICE;
  return layout_impl(topk_idx, T, E, k, place, nullptr, G, x, d, dt, rank_mask, rank_off,
                     disp_token, expert_off, perm_row, slot_of, x_disp, ws, kNoAllocScratchBytes,
                     stream);
}

MOE_EXPORT moe_status moe_replica_layout(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                         const uint32_t* rep_mask, int32_t G,
                                         int32_t ranks_per_node, const void* x, int32_t d,
                                         moe_dtype dt, int32_t* rank_of, uint32_t* node_mask,
                                         uint32_t* rank_mask, int32_t* rank_off,
                                         int32_t* disp_token, int32_t* expert_off,
                                         int32_t* perm_row, int32_t* slot_of, void* x_disp,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || G < 1 || ranks_per_node < 1) return MOE_ERR_ARG;
  if (G % ranks_per_node != 0) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || G > kMaxG || (int64_t)T * k >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  if (!rep_mask || (T > 0 && (!rank_of || !node_mask))) return MOE_ERR_ARG;
  if (T > 0) {
    int log_p = 0;
    while ((1 << log_p) < k) ++log_p;  // k <= kMaxK = 16, so a group fits a wave
    const int64_t lanes = (int64_t)T << log_p;
    hipLaunchKernelGGL(replica_assign_kernel, dim3((unsigned)ceil_div(lanes, 256)), dim3(256), 0,
                       stream, topk_idx, T, E, k, log_p, rep_mask, G, ranks_per_node, rank_of,
                       node_mask);
  }
  return layout_impl(topk_idx, T, E, k, nullptr, rank_of, G, x, d, dt, rank_mask, rank_off,
                     disp_token, expert_off, perm_row, slot_of, x_disp, workspace,
                     workspace_bytes, stream);
}

namespace moe {
namespace {

struct ShuffleWorkspace {
  size_t ident, rank_mask, expert_off, perm_row, layout, total;
};
inline ShuffleWorkspace shuffle_workspace(int32_t T, int32_t G) {
  ShuffleWorkspace w;
  w.ident = 0;
  w.rank_mask = w.ident + align_up((size_t)G * sizeof(int32_t));
  w.expert_off = w.rank_mask + align_up((size_t)T * sizeof(uint32_t));
  w.perm_row = w.expert_off + align_up((size_t)(G + 1) * sizeof(int32_t));
  w.layout = w.perm_row + align_up((size_t)T * sizeof(int32_t));
  w.total = w.layout + workspace_layout(T, G, 1, G).total;
  return w;
}

}  // namespace
}  // namespace moe

MOE_EXPORT size_t moe_shuffle_workspace_bytes(int32_t T, int32_t G) {
  if (T < 0 || G < 1 || G > kMaxG) return 0;
  return shuffle_workspace(T, G).total;
}

MOE_EXPORT moe_status moe_token_shuffle(const int32_t* want_idx, int32_t T, int32_t E, int32_t k,
                                        const int32_t* aff, int32_t G, const void* x, int32_t d,
                                        moe_dtype dt, int32_t* dest, int32_t* rank_off,
                                        int32_t* perm, int32_t* pos, void* x_shuf,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || G < 1) return MOE_ERR_ARG;
  if (k > kMaxK || G > kMaxG || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (!aff || !rank_off || (T > 0 && (!want_idx || !dest || !perm || !pos))) return MOE_ERR_ARG;
  if (x) {  // checked here so that nothing is enqueued on an argument error
    if (!valid_dtype(dt) || d < 1 || (T > 0 && !x_shuf)) return MOE_ERR_ARG;
    if (((size_t)d * dtype_bytes(dt)) % 16 != 0 || (uintptr_t)x % 16 || (uintptr_t)x_shuf % 16)
      return MOE_ERR_UNSUPPORTED;
  }
  const ShuffleWorkspace ws = shuffle_workspace(T, G);
  if (!workspace || workspace_bytes < ws.total) return MOE_ERR_WORKSPACE;
  char* wsp = static_cast<char*>(workspace);
  int32_t* ident = reinterpret_cast<int32_t*>(wsp + ws.ident);
  int log_p = 0;
  while ((1 << log_p) < G) ++log_p;  // G <= 32: a token's lanes fit in a wave
  const int64_t lanes = (int64_t)(T > 0 ? T : 1) << log_p;
  hipLaunchKernelGGL(token_dest_kernel, dim3((unsigned)ceil_div(lanes, 256)), dim3(256), 0, stream,
                     want_idx, T, E, k, aff, G, log_p, dest, ident);
  // The shuffled order is the once-per-rank layout of a batch in which token
  // t has the single choice dest[t] and "expert" g sits on rank g: its rows
  // are the tokens grouped by rank (perm), its slots give each token's
  // position in that order (pos), and its dispatched rows are x[perm].
  return layout_impl(dest, T, G, 1, ident, nullptr, G, x, d, dt,
                     reinterpret_cast<uint32_t*>(wsp + ws.rank_mask), rank_off, perm,
                     reinterpret_cast<int32_t*>(wsp + ws.expert_off),
                     reinterpret_cast<int32_t*>(wsp + ws.perm_row), pos, x_shuf, wsp + ws.layout,
                     workspace_bytes - ws.layout, stream);
}
