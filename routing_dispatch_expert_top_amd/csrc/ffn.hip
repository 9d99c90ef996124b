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
// and v of an element in the same lane). The K loop streams K slices of A
// and B into a ring of LDS stages with direct-to-LDS loads (16-byte chunks,
// XOR-swizzled so the MFMA fragment reads are free of bank conflicts) while
// the MFMAs consume an earlier slice.
// The tile list is derived on the device from expert_off, so no host round
// trip is needed. The forward launches are persistent: one workgroup per CU
// walks its XCD's share of the tile list in order, claiming tiles from a
// per-XCD counter in the caller's workspace, so that the tiles running at
// once on an XCD are neighbours that share weight panels and activation
// tiles in its L2 (at the end, workgroups of an XCD that is done take the
// other XCDs' remaining tiles). The same kernel, in a weight-gradient mode, computes the
// backward's weight gradients; a one-tile-per-workgroup kernel computes its
// data gradients.
//
// fp32 path: the fp32 matrix cores (v_mfma_f32_32x32x2_f32), 64 x 64 tiles
// staged K-major in LDS.
#include "moe_internal.h"
#include "gemm_common.h"

#include <atomic>

namespace moe {
namespace {

// ---------------------------------------------------------------- bf16 MFMA

template <int BM, int BN, int WM, int WN, bool SWIGLU>
struct TileCfg {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kWaveRows = BM / WM;
  static constexpr int kWaveCols = BN / WN;       // B rows per wave
  static constexpr int TM = kWaveRows / 32;
  static constexpr int TN = kWaveCols / 32;
  static constexpr int kOutCols = SWIGLU ? BN / 2 : BN;
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "tile shape");
  static_assert(!SWIGLU || TN % 2 == 0, "gate/up pairs");
};

// ---------------------------------------------------------------- bf16 MFMA kernel
//
// K slices travel HBM/L2 -> LDS with
// gfx950's 16-byte direct-to-LDS loads (global_load_lds_dwordx4: each lane's
// 16 bytes land at wave base + 16 * lane), so no registers stage them and
// later slices are in flight while the MFMAs consume one. One DMA
// instruction fills 8 LDS rows of 128 bytes; a lane picks the global chunk
// whose swizzled slot is its own, so the LDS image is the XOR-swizzled one
// the fragment reads expect. Waits are explicit (vmcnt = DMA instructions
// still allowed in flight) and the workgroup barrier carries no memory fence,
// so the compiler does not drain every outstanding load at each K step.

typedef __attribute__((address_space(3))) void lds_void_t;


// Two 16-byte direct-to-LDS loads per lane. Global address of load j =
// base + voff_j + (OFF + 1024 j) (base in SGPRs, voff_j a 32-bit per-lane
// byte offset); its LDS destination = M0 + (OFF + 1024 j) + 16 * lane: the
// immediate offset moves both addresses (checked on the device), so one M0
// value serves a wave's run of consecutive 1 KiB LDS blocks. Issued as
// inline asm so the compiler does not add its own "wait for every LDS DMA"
// before later LDS reads; completion is tracked by the explicit vmcnt waits
// of the K loop (VMEM ops count in issue order, so the compiler's own waits
// for earlier loads stay correct). M0 is restored so the compiler's view of
// it holds.
template <int OFF>
__device__ __forceinline__ void dma_pair(uint32_t voff0, uint32_t voff1, const void* base,
                                         uint32_t m0) {
  static_assert(OFF >= 0 && OFF + 1024 < 4096, "immediate offset range");
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3 offset:%5\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:%6\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff0), "v"(voff1), "s"(base), "s"(m0), "i"(OFF), "i"(OFF + 1024)
      : "memory");
}

// Per-lane DMA offsets are biased by this much (and the SGPR bases lowered
// by it), so offset - (immediate of the load) never goes below zero.
constexpr uint32_t kDmaBias = 3072;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// Ring stages: NSA stages of A rows and NSB stages of B rows (weights). The
// weights get the deeper ring: they are the larger stream from HBM and
// their misses cost the most. With NSA = 2 and NSB = 3 at 256 x 256 x 64 the
// ring is exactly the 160 KiB of LDS of a gfx950 CU, so the tile schedule is
// built inside the ring before the first DMA lands there.
// The one-tile kernel computes the backward's data gradients: C[s] = A[s]
// W[e] for the slots s of expert e, where the weight panel is read as
// [K][N0] (N contiguous; expert e's panel = ksplit x N0 elements of B0 for
// k < ksplit, of B1 for k >= ksplit).
// Its slices are DMA-loaded raw (two 512-byte K rows per 1 KiB block, the
// 16-byte chunk index XOR-ed with 2 (row & 3)) and each B fragment is two
// ds_read_b64_tr_b16: inside a group of 16 lanes, lane j receives element
// j mod 4 of the 8 bytes addressed by lane 4 m + j / 4 as its value m, so
// lanes that address K row k0 + s / 4, columns n0 + 4 (s mod 4) give lane j
// the 4 K values of column n0 + j (checked on the device).
// SWB (SwiGLU backward epilogue): C = [du | dv] rows of 2 N0, from the tile
// (dh) and the saved [u | v] rows in UV.
template <int BM, int BN, int BK, int WM, int WN, int NSA, int NSB, bool SWB = false>
__global__ __launch_bounds__(WM* WN* kWave) void dgrad_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm_row,
    const int32_t* __restrict__ expert_off, int E, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, int K, int N0, uint16_t* __restrict__ C,
    uint16_t* __restrict__ UV, int ksplit = 0) {
  static_assert(BK == 64, "two 512-byte K rows per 1 KiB DMA block");
  using Cfg = TileCfg<BM, BN, WM, WN, false>;
  constexpr int NW = WM * WN;
  constexpr int CH = BK / 8;           // 16-byte chunks per row of a K slice
  constexpr int RPI = 512 / BK;        // rows filled by one 1 KiB DMA instruction
  constexpr int A_INS = BM / RPI / NW;  // DMA instructions per wave per slice
  constexpr int B_INS = BN / RPI / NW;
  constexpr int LPS = A_INS + B_INS;
  static_assert(BK == 32 || BK == 64, "K slice");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "DMA row split");
  static_assert(NSA >= 2 && NSB >= NSA, "ring depths: weights get at least as many stages");
  constexpr int kRing = (NSA * BM + NSB * BN) * CH;  // 16-byte units
  __shared__ u32x4 ring[kRing];
  u32x4 (*As)[BM * CH] = reinterpret_cast<u32x4 (*)[BM * CH]>(ring);
  u32x4 (*Bs)[BN * CH] = reinterpret_cast<u32x4 (*)[BN * CH]>(ring + NSA * BM * CH);
  static_assert(BM * Cfg::kOutCols * 2 <= kRing * 16, "output tile fits the ring");
  static_assert(sizeof(TileSel) <= kRing * 16, "tile selection fits the ring");

  int e = 0, nt = 0, mt = 0, seg0 = 0, send = 0;
  {
    TileSel& ts = *reinterpret_cast<TileSel*>(ring);
    const int NT = (N0 + Cfg::kOutCols - 1) / Cfg::kOutCols;
    if (!select_tile(ts, expert_off, E, BM, NT, e, nt, mt, seg0, send)) return;  // uniform
    __syncthreads();  // every wave has its tile before the first DMA overwrites the selection
  }
  // An expert's rows are split evenly, in whole 32-row bands, over its
  // ceil(rows / BM) m-tiles rather than as full tiles and a short last one:
  // the m-tiles of one weight panel then cost the same, start together and
  // stay in step, so each weight slice is fetched into the XCD's L2 once for
  // all of them (a short tile runs ahead and fetches the panel again).
  const int me = send - seg0, nmt = (me + BM - 1) / BM;
  const int rows_per = min(BM, ((me + nmt - 1) / nmt + 31) & ~31);
  const int m0 = seg0 + mt * rows_per;
  const int seg1 = min(send, m0 + rows_per);  // end of this tile's rows
  const int c0 = nt * Cfg::kOutCols;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  // lane -> (row, physical chunk) of its DMA slot; it fetches the logical
  // chunk stored there (the swizzle is an involution). DMA instruction i of
  // a wave fills the 1 KiB block of rows [RPI * (wave * INS + i), + RPI) of
  // its operand (INS = A_INS or B_INS), so a wave's blocks are contiguous
  // and groups of 4 share one M0 value (immediate offsets 0..3072).
  static_assert(A_INS % 2 == 0 && B_INS % 2 == 0 && (LPS / (BK / 16)) % 2 == 0, "DMA pairs");
  const uint32_t krow = (uint32_t)K * 2;  // bytes per operand row
  uint32_t aoff[A_INS], boff[B_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int r = RPI * (wave * A_INS + i) + lane / CH;
    const int c = swz_ch<CH>(r, lane % CH) - r * CH;
    const int s = min(m0 + r, seg1 - 1);
    const int src = perm_row ? perm_row[s] : s;
    aoff[i] = (uint32_t)src * krow + (uint32_t)c * 16 + kDmaBias - 1024u * (i & 3);
  }
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    // block i of the wave = K rows 2 (wave B_INS + i) + {0, 1} of the slice
    const int r = 2 * (wave * B_INS + i) + lane / 32;
    const int c = (lane % 32) ^ (2 * (r & 3));  // logical chunk in this physical slot
    const int n = min(c0 + c * 8, N0 - 8);
    boff[i] = (uint32_t)(r * N0 + n) * 2u + kDmaBias - 1024u * (i & 3);
  }
  const char* a_base = reinterpret_cast<const char*>(A) - kDmaBias;
  // DMA instructions i, i+1 (i even) of slice kt: i < A_INS fills A rows,
  // the rest B rows
  auto dma_ins2 = [&](int i, int kt) {
    const bool is_a = i < A_INS;
    const int ii = is_a ? i : i - A_INS;
    const int ins = is_a ? A_INS : B_INS;
    const u32x4* stage = is_a ? As[kt % NSA] : Bs[kt % NSB];
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        lds_addr(stage + RPI * (wave * ins + (ii & ~3)) * CH));
    const char* base;
    if (!is_a) {
      const int k0 = kt * BK;
      const bool hi = k0 >= ksplit;  // uniform over the slice
      base = reinterpret_cast<const char*>(hi ? B1 : B0) +
             ((size_t)e * ksplit * N0 + (size_t)(hi ? k0 - ksplit : k0) * N0) * 2 - kDmaBias;
    } else {
      base = a_base + (size_t)kt * (BK * 2);
    }
    const uint32_t v0 = is_a ? aoff[ii] : boff[ii];
    const uint32_t v1 = is_a ? aoff[ii + 1] : boff[ii + 1];
    if ((ii & 3) == 0) dma_pair<0>(v0, v1, base, m0v);
    else dma_pair<2048>(v0, v1, base, m0v);
  };

  const int wm = wave / WN, wn = wave % WN;
  // The tile's 32-row MFMA bands are dealt to the WM wave rows in turn
  // (band tm * WM + wm is this wave's tm-th), so in a tile that ends inside
  // an expert's segment the live bands split evenly over the wave rows and
  // the slowest wave, which sets every slice's barrier, carries about half
  // of them rather than all of its contiguous half of the tile.
  auto band_row = [&](int tm) { return (tm * WM + wm) * 32; };  // first tile row of band tm
  const int li = lane & 31, lk = lane >> 5;
  int fa_row[Cfg::TM];
#pragma unroll
  for (int tm = 0; tm < Cfg::TM; ++tm) fa_row[tm] = band_row(tm) + li;
  // byte offset in a B stage of this lane's first transposed read of
  // fragment tn at k-step 0 (k-step ks adds 16 K rows = 8192 bytes, the
  // second read 4 K rows = 2048 bytes)
  uint32_t fbt_off[Cfg::TN];
  {
    const int g = lane >> 4, sl = lane & 15;
    const int kb = 8 * (g >> 1) + sl / 4;
#pragma unroll
    for (int tn = 0; tn < Cfg::TN; ++tn) {
      const int col = wn * Cfg::kWaveCols + tn * 32 + 16 * (g & 1) + 4 * (sl % 4);
      fbt_off[tn] = (uint32_t)(kb * 512 + (((col >> 3) ^ (2 * (kb & 3))) << 4) + (col & 7) * 2);
    }
  }
  auto read_bt = [&](const u32x4* bs, int tn, int ks) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const char* b = reinterpret_cast<const char*>(bs) + fbt_off[tn] + ks * 8192;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(const lds_void_t*)(b));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(const lds_void_t*)(b + 2048));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[Cfg::TM][Cfg::TN];
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
  // Issue order (vmcnt counts in issue order): prologue A(0), .., A(NSA-2),
  // B(0), .., B(NSB-2); then the DMA issued during slice kt is A(kt+NSA-1)
  // followed by B(kt+NSB-1), into the stages slice kt-1 used. When slice kt
  // is needed, what was issued after the later of A(kt) and B(kt) may still
  // be in flight.
#pragma unroll
  for (int p = 0; p < NSA - 1; ++p)
    if (p < KT) {
#pragma unroll
      for (int i = 0; i < A_INS; i += 2) dma_ins2(i, p);
    }
#pragma unroll
  for (int p = 0; p < NSB - 1; ++p)
    if (p < KT) {
#pragma unroll
      for (int i = A_INS; i < LPS; i += 2) dma_ins2(i, p);
    }
  constexpr int KS = BK / 16;  // MFMA k-steps per slice
  static_assert(KS % 2 == 0, "fragment double buffer parity");
  // Fragments are double-buffered (set (ks & 1) holds k-step ks). The last
  // k-step of a slice is read before the barrier and multiplied after it,
  // so its MFMAs keep the matrix pipe busy while the barrier releases, the
  // next DMA is issued and the next slice's first fragments are read. No
  // wave reads a slice's LDS stages after that barrier, so they can be
  // refilled right after it.
  // 32-row MFMA bands of this wave holding at least one real slot: bands
  // wholly past the expert's last slot issue neither fragment reads nor
  // MFMAs. The K loop is instantiated per count (dispatched once per tile),
  // so the steady-state code has no per-band branches.
  const int nb_live = max(0, min(BM / 32, (seg1 - m0 + 31) / 32));  // the tile's live bands
  const int tm_live = min(Cfg::TM, nb_live > wm ? (nb_live - wm + WM - 1) / WM : 0);
  bf16x8 fa[2][Cfg::TM], fb[2][Cfg::TN];
  auto k_loop = [&](auto live_c) {
    constexpr int LIVE = decltype(live_c)::value;
    constexpr int NM = LIVE * Cfg::TN;  // MFMAs per k-step
    constexpr int NR = LIVE + Cfg::TN;  // fragment reads per k-step
    static_assert(NM >= NR || LIVE <= 1, "reads fit between the MFMAs");
    // One k-step: the NM MFMAs on fragment set `set`, with the NR fragment
    // reads of k-step ks_next into the other set (if rd) and the DMA
    // instructions [lo, hi) of the slices issued during slice kt placed
    // between them, one read and at most one or two DMAs after each MFMA.
    // The DMA asm statements keep their place in the instruction stream, so
    // the matrix pipe is fed while the loads issue instead of draining
    // behind a burst of them.
    auto kstep = [&](auto chk_c, int set, bool rd, const u32x4* as, const u32x4* bs, int ks_next,
                     int kt, int lo, int hi) {
      constexpr bool CHK = decltype(chk_c)::value;  // false: every target slice exists
      const int ch = ks_next * 2 + lk;
      const int nd = hi - lo;
      auto read_frag = [&](int j) {
        if (j < LIVE)
          fa[set ^ 1][j] = __builtin_bit_cast(bf16x8, as[swz_ch<CH>(fa_row[j], ch)]);
        else
          fb[set ^ 1][j - LIVE] = read_bt(bs, j - LIVE, ks_next);
      };
      auto dma_at = [&](int j) {  // DMA pairs that go right after MFMA j
        const int np = nd / 2;
#pragma unroll
        for (int q = 0; q < LPS / 2; ++q) {
          if (q >= np) break;
          if ((NM > 0 ? q * NM / np : 0) != j) continue;
          const int i = lo + 2 * q;
          const int nx = i < A_INS ? kt + NSA - 1 : kt + NSB - 1;
          if (!CHK || nx < KT) dma_ins2(i, nx);
        }
      };
      if (NM == 0) {
        dma_at(0);
        return;
      }
      // nothing crosses a k-step boundary: the MFMAs of this k-step use
      // fragments read during the previous one, so none of them waits on the
      // reads issued here (left free, the scheduler hoists the next k-step's
      // MFMAs right behind their reads and the wave stalls on lgkmcnt)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        const int tm = j / Cfg::TN, tn = j % Cfg::TN;
        // B fragment as the first operand: the result is the transposed
        // tile (rows = output columns, columns = slots), so each lane ends
        // with 4 consecutive output columns of one slot per register quad
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][tn], fa[set][tm], acc[tm][tn], 0, 0, 0);
        if (rd && j < NR) read_frag(j);
        if (rd && NM < NR && j == NM - 1)
#pragma unroll
          for (int r = NM; r < NR; ++r) read_frag(r);
        dma_at(j);
      }
      if (rd) {
        // one fragment read after each MFMA, then the remaining MFMAs (or reads)
        // (a transposed-weight B fragment is two LDS reads)
        constexpr int NP = NM < NR ? NM : NR;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (i >= LIVE) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
          else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // DS read
        }
        constexpr int REM_B = NR - (NP > LIVE ? NP : LIVE);
        constexpr int REM_DS = (NR - NP) + (REM_B > 0 ? REM_B : 0);
        if (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
        if (REM_DS > 0) __builtin_amdgcn_sched_group_barrier(0x100, REM_DS, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto read_first = [&](const u32x4* as, const u32x4* bs) {  // k-step 0 of a slice into set 0
      if (LIVE == 0) return;
      const int ch = lk;
#pragma unroll
      for (int tm = 0; tm < LIVE; ++tm)
        fa[0][tm] = __builtin_bit_cast(bf16x8, as[swz_ch<CH>(fa_row[tm], ch)]);
#pragma unroll
      for (int tn = 0; tn < Cfg::TN; ++tn)
        fb[0][tn] = read_bt(bs, tn, 0);
    };
    auto slice_ready = [&](int kt) {  // slice kt landed; every wave is done with slice kt-1
      MOE_WAIT_LGKM0();  // fragment reads of slice kt-1 complete before its stages are refilled
      // steady state: the NSA-2 slices of DMA issued after the one holding
      // A(kt), and before them, if NSB > NSA, that slice's B(kt+NSB-NSA) (when
      // NSB = NSA it is B(kt) itself, which must have landed), all of them
      // issued (their last target B(kt+NSB-2) exists); after the prologue:
      // B(1) .. B(NSB-2); otherwise nothing may stay in flight
      constexpr int kSteady = (NSB > NSA ? B_INS : 0) + (NSA - 2) * (A_INS + B_INS);
      constexpr int kFirst = (NSB - 2) * B_INS;
      static_assert(kSteady < 64 && kFirst < 64, "vmcnt range");
      if (kt == 0 && NSB - 2 < KT) MOE_WAIT_VMCNT(kFirst);
      else if (kt > 0 && kt >= NSA - 1 && kt + NSB - 2 < KT) MOE_WAIT_VMCNT(kSteady);
      else MOE_WAIT_VMCNT(0);
      wg_barrier();
    };
    // The DMA issued during slice kt (A(kt+NSA-1), then B(kt+NSB-1)) is spread
    // evenly over KS k-steps: the last k-step of slice kt-1 (multiplied after
    // the barrier that frees the stages) and the first KS-1 k-steps of slice
    // kt; the last k-step is left for the loads to land.
    auto dlo = [](int q) { return q * LPS / KS; };
    auto middle_steps = [&](auto chk_c, int kt) {  // k-steps 0..KS-2 of slice kt; leaves set 1 = k-step KS-1
      const u32x4* as = As[kt % NSA];
      const u32x4* bs = Bs[kt % NSB];
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks)
        kstep(chk_c, ks & 1, true, as, bs, ks + 1, kt, dlo(ks + 1), dlo(ks + 2));
    };
    auto step = [&](auto chk_c, int kt) {  // slice kt's first steps, the barrier, its last step
      middle_steps(chk_c, kt);
      slice_ready(kt + 1);
      // last k-step of slice kt (set 1) while reading k-step 0 of slice kt+1
      // into set 0 and issuing the first DMA share of slice kt+1
      kstep(chk_c, 1, true, As[(kt + 1) % NSA], Bs[(kt + 1) % NSB], 0, kt + 1, 0, dlo(1));
    };
    constexpr std::false_type kNoCheck{};
    constexpr std::true_type kCheck{};

    slice_ready(0);
    read_first(As[0], Bs[0]);
    {
      // the DMA share of "k-step KS-1 of slice -1": nothing to multiply yet
#pragma unroll
      for (int i = 0; i < LPS; i += 2)
        if (i < dlo(1)) {
          const int nx = i < A_INS ? NSA - 1 : NSB - 1;
          if (nx < KT) dma_ins2(i, nx);
        }
    }
    // steady state: while kt + kLead < KT every slice the DMA of step kt
    // targets exists (A(kt+NSA) in the share issued with its last k-step,
    // which holds A instructions only, and B(kt+NSB-1)), so the loop body has
    // no branch; the last slices check, and the last one is peeled off
    static_assert(LPS / KS <= A_INS, "the first DMA share of a slice is A rows only");
    constexpr int kLead = NSA > NSB - 1 ? NSA : NSB - 1;
    int kt = 0;
    for (; kt + kLead < KT; ++kt) step(kNoCheck, kt);
    for (; kt + 1 < KT; ++kt) step(kCheck, kt);
    middle_steps(kCheck, KT - 1);
    kstep(kCheck, 1, false, As[0], Bs[0], 0, KT, 0, 0);
  };
  static_assert(Cfg::TM <= 4, "band-count dispatch");
  switch (tm_live) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, (Cfg::TM >= 1 ? 1 : 0)>{}); break;
    case 2: k_loop(std::integral_constant<int, (Cfg::TM >= 2 ? 2 : 0)>{}); break;
    case 3: k_loop(std::integral_constant<int, (Cfg::TM >= 3 ? 3 : 0)>{}); break;
    default: k_loop(std::integral_constant<int, Cfg::TM>{}); break;
  }

  // Epilogue. Each lane owns slot row (lane & 31) of each 32-row band and,
  // per register quad q, output columns 8q + 4*(lane>>5) + 0..3 of a 32-wide
  // column tile: 4 consecutive values = one 8-byte bf16 piece.
  //  plain (da): the pieces go into a row-major tile in the (now free) LDS
  //           ring with 16-byte chunks XOR-swizzled by row, and the workgroup
  //           writes the rows out, 16 bytes per lane (fully coalesced;
  //           scattered 8-byte stores cost more).
  //  SwiGLU backward: the fp32 tile through the ring in two halves of BM/2
  //           rows (a whole tile does not fit).
  if (SWB) {
    // SwiGLU backward: dh (the tile) with the saved u, v of the same columns
    // gives du = dh v silu'(u) and dv = dh silu(u), stored as [du | dv] rows.
    // The fp32 tile goes through the freed ring in two halves of BM/2 rows
    // (16-byte chunks XOR-swizzled by row), and the workgroup then walks
    // whole rows: 16-byte u, v loads and du, dv stores, 8 columns per thread
    // (direct 8-byte accesses from the MFMA layout touch 32 rows each).
    constexpr int OC = Cfg::kOutCols;   // dh columns per tile
    constexpr int CH4 = OC / 4;         // 16-byte fp32 chunks per staged row
    constexpr int HR = BM / 2;          // rows per half
    static_assert(HR * OC * 4 <= kRing * 16, "half tile fits the ring");
    static_assert(WM == 2 && Cfg::TM == 4, "bands 2h, 2h+1 of each wave row are half h");
    constexpr int CPR = OC / 8;                  // 8-column pieces per row
    constexpr int RSTEP = Cfg::kThreads / CPR;   // rows per pass
    constexpr int NB = 4;                        // rows whose loads are in flight together
    static_assert(Cfg::kThreads % CPR == 0 && HR % (RSTEP * NB) == 0, "row passes");
    float* st = reinterpret_cast<float*>(ring);
    auto st_off = [&](int row, int ch) { return row * OC + ((ch ^ (row & (CH4 - 1))) << 2); };
    const int rows_here = min(BM, seg1 - m0);
    const int pc = tid % CPR, pr = tid / CPR;
    const int col = c0 + pc * 8;
    const int colc = min(col, N0 - 8);  // loads stay in the u part of the row
    MOE_WAIT_LGKM0();  // every wave's last fragment reads are done: the ring is free
    wg_barrier();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh) __syncthreads();  // the first half has been read out
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int tm = 2 * hh + b;
        const int row = band_row(tm) - hh * HR + li;
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int ch = (wn * Cfg::kWaveCols + tn * 32 + 8 * qd + 4 * lk) >> 2;
            const f32x16& a = acc[tm][tn];
            *reinterpret_cast<f32x4*>(st + st_off(row, ch)) =
                f32x4{a[4 * qd + 0], a[4 * qd + 1], a[4 * qd + 2], a[4 * qd + 3]};
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int p0 = 0; p0 < HR / RSTEP; p0 += NB) {
        u32x4 uu[NB], vv[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int r = hh * HR + pr + (p0 + q) * RSTEP;  // tile row
          const size_t o = (size_t)min(m0 + r, seg1 - 1) * (2 * N0) + colc;
          uu[q] = *reinterpret_cast<const u32x4*>(UV + o);
          vv[q] = *reinterpret_cast<const u32x4*>(UV + o + N0);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const int rh = pr + (p0 + q) * RSTEP;  // row in the half
          const int r = hh * HR + rh;
          if (r >= rows_here || col >= N0) continue;
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(st + st_off(rh, 2 * pc));
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(st + st_off(rh, 2 * pc + 1));
          const float dh[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          uint32_t du2[4], dv2[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float du[2], dv[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float u = h2 ? bf16hi(uu[q][i]) : bf16lo(uu[q][i]);
              const float v = h2 ? bf16hi(vv[q][i]) : bf16lo(vv[q][i]);
              const float g = dh[2 * i + h2];
              const float sg =
                  __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u * 1.44269504088896341f));
              du[h2] = g * v * (sg * (1.0f + u * (1.0f - sg)));
              dv[h2] = g * (u * sg);
            }
            du2[i] = pack_bf16x2(du[0], du[1]);
            dv2[i] = pack_bf16x2(dv[0], dv[1]);
          }
          const size_t o = (size_t)(m0 + r) * (2 * N0) + col;
          *reinterpret_cast<u32x4*>(C + o) = u32x4{du2[0], du2[1], du2[2], du2[3]};
          *reinterpret_cast<u32x4*>(C + o + N0) = u32x4{dv2[0], dv2[1], dv2[2], dv2[3]};
        }
      }
    }
  } else {
    // The output tile (da) is staged row-major in the freed ring, 16-byte
    // chunks XOR-swizzled by row, and written out in whole rows, 16 bytes per
    // lane.
    constexpr int OC = Cfg::kOutCols;  // output columns per tile
    constexpr int CPR = OC / 8;        // 16-byte chunks per output row
    static_assert(CPR >= 8 && (CPR & (CPR - 1)) == 0, "output row chunks: a power of two");
    MOE_WAIT_LGKM0();  // every wave's last fragment reads are done: the ring is free
    wg_barrier();
    char* ot = reinterpret_cast<char*>(ring);
    auto ot_addr = [&](int row, int col) {  // byte address of (row, col) in the tile
      return row * (OC * 2) + (((col >> 3) ^ (row & (CPR - 1))) << 4) + ((col & 7) << 1);
    };
#pragma unroll
    for (int tm = 0; tm < Cfg::TM; ++tm) {
      const int row = band_row(tm) + li;
#pragma unroll
      for (int tn = 0; tn < Cfg::TN; ++tn) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int col = wn * Cfg::kWaveCols + tn * 32 + 8 * qd + 4 * lk;
          const f32x16& a = acc[tm][tn];
          uint2 pk;
          pk.x = pack_bf16x2(a[4 * qd + 0], a[4 * qd + 1]);
          pk.y = pack_bf16x2(a[4 * qd + 2], a[4 * qd + 3]);
          *reinterpret_cast<uint2*>(ot + ot_addr(row, col)) = pk;
        }
      }
    }
    __syncthreads();
    // Thread tid writes 16-byte chunk tid % CPR of rows tid / CPR + RSTEP p,
    // p = 0 .. BM / RSTEP - 1. Unrolled in batches of 8 rows: 8 LDS reads in
    // flight, then their 8 stores (a rolled loop waits out the LDS latency
    // before every store). Rows past the tile's last slot read the ring
    // (in range) and store nothing.
    const int rows_here = min(BM, seg1 - m0);
    constexpr int RSTEP = Cfg::kThreads / CPR;
    constexpr int NPASS = BM / RSTEP;
    static_assert(Cfg::kThreads % CPR == 0 && BM % RSTEP == 0 && NPASS % 8 == 0, "write-back passes");
    const int c = tid % CPR, r0 = tid / CPR;
    const int col = c0 + c * 8;
    uint16_t* gout = C + (size_t)(m0 + r0) * N0 + col;
#pragma unroll
    for (int p0 = 0; p0 < NPASS; p0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = *reinterpret_cast<const u32x4*>(ot + ot_addr(r0 + (p0 + j) * RSTEP, c * 8));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r0 + (p0 + j) * RSTEP < rows_here && col < N0)
          *reinterpret_cast<u32x4*>(gout + (size_t)(p0 + j) * RSTEP * N0) = v[j];
    }
  }
}

// ---------------------------------------------------------------- persistent forward GEMM
//
// The forward gate/up and down launches as a persistent grid: one workgroup
// per CU (the ring fills a CU's LDS), each walking tiles until its XCD's
// share is done. What a one-tile workgroup pays per tile (start, tile
// selection, the activation-row gather's index loads, the first slices'
// load latency, the output stores' drain) then overlaps the previous tile:
//  - the tile list is decoded from a per-wave register copy of the expert
//    schedule (lane l holds experts 4l .. 4l+3), built once;
//  - tile i+1's activation-row indices are loaded while tile i multiplies;
//  - tile i+1's first A slice and first two B slices are issued at the start
//    of tile i's epilogue, into the ring stages tile i's last slices did not
//    use, while its output is staged through the other two and stored;
//  - the stores drain while tile i+1 multiplies.
// Tiles are handed out in order, per XCD: XCD x owns logical tiles
// [x q, (x+1) q) (the order of decode_tile, q = ceil(tiles / 8)); its
// workgroups take local tiles s and s + S first (S workgroups per XCD, slot
// s), then claim the next one from the XCD's counter (and, in launches of
// at least 8 tiles per workgroup, from the other XCDs' counters once their
// own is exhausted). Tiles running at one
// moment on an XCD therefore stay a window of neighbouring tiles that share
// weight panels and activation tiles in that XCD's L2 (a static walk lets
// workgroups drift apart and lose that sharing). A claim is made two tiles
// ahead (in tile i's epilogue, for tile i+2) and handed to the workgroup's
// other waves through the freed staging area, because the ring leaves no LDS
// free.
// The queue (8 counters and a finished-workgroup count) must be zero when a
// launch starts; the last workgroup to finish sets it back to zero.
// WG (weight-gradient mode, for the backward): Out[e][m][n] = sum over
// the slots s of expert e, [expert_off[e], expert_off[e+1]), of A[s][m]
// B0[n][kpad[e] + s - expert_off[e]]: A is [slots][M0] as it lies (M
// contiguous), B0 the expert-padded transpose, N0 K-contiguous rows of
// length K whose segment [kpad[e], kpad[e+1]) is zero past the expert's
// slots; in fp32, rows m < msplit to O0 (msplit x N0 per expert) and the
// others to O1. perm_row holds the expert walk: position p is expert perm_row[p] (-1:
// none), 8 ceil(E/8) positions of ceil(M0/256) x ceil(N0/256) tiles each,
// n-tiles inner; XCD x owns positions [x ceil(E/8), (x+1) ceil(E/8)). An
// expert with an empty segment gets zeros. A tile's K loop length is its
// expert's. The 256 KiB fp32 output goes through the two ring stages the
// next tile's prologue leaves free, 64 rows a pass, and is stored in whole
// 1 KiB rows (from the accumulator layout each store instruction would
// touch 32 rows with 32 bytes each, and the CU's write path, not HBM, set
// the pace).

template <bool SWIGLU, bool WG = false, bool KEEP = false>
__global__ __launch_bounds__(256) void ffn_persistent_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm_row,
    const int32_t* __restrict__ expert_off, int E, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, int K, int N0, uint16_t* __restrict__ C,
    uint32_t* __restrict__ queue, int M0 = 0, int msplit = 0, float* __restrict__ O0 = nullptr,
    float* __restrict__ O1 = nullptr, const int32_t* __restrict__ kpad = nullptr,
    uint16_t* __restrict__ UV = nullptr) {
  static_assert(!(WG && SWIGLU), "weight-gradient mode has a plain epilogue");
  static_assert(!KEEP || SWIGLU, "u and v are kept by the gate/up launch");
  constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 2, NSA = 2, NSB = 3;
  using Cfg = TileCfg<BM, BN, WM, WN, SWIGLU>;
  constexpr int NW = WM * WN;
  constexpr int CH = BK / 8;
  constexpr int RPI = 512 / BK;
  constexpr int A_INS = BM / RPI / NW;
  constexpr int B_INS = BN / RPI / NW;
  constexpr int LPS = A_INS + B_INS;
  constexpr int kStageA = BM * CH, kStageB = BN * CH;  // 16-byte units
  // output stores per thread and staging pass (a pass is 32 KiB x 2 of rows)
  constexpr int kStPass = 2 * 32768 / 16 / (WM * WN * kWave);
  constexpr int kMaxPendSt = (SWIGLU ? (KEEP ? 3 : 1) : 2) * kStPass;
  __shared__ u32x4 ring[NSA * kStageA + NSB * kStageB];
  auto stA = [&](int s) { return ring + (s % NSA) * kStageA; };
  auto stB = [&](int s) { return ring + NSA * kStageA + (s % NSB) * kStageB; };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int NT = (N0 + Cfg::kOutCols - 1) / Cfg::kOutCols;
  int KT = WG ? 0 : K / BK;  // weight gradients: the current tile's expert segment
  const uint32_t krow = (uint32_t)K * 2;

  // ---- expert schedule in registers: lane l holds the m-tile prefix of
  // experts 4l .. 4l+3 (two values per lane); the decode finds the lane by
  // a ballot and the expert inside it from scalar loads of expert_off
  // Weight gradients: positions p = 0 .. 8 ceil(E/8) - 1 of the expert walk
  // (expert perm_row[p], -1: none) times MT x NT tiles each, n-tiles inner;
  // expert_off holds the padded K offsets of the experts' segments.
  const int MT = WG ? (M0 + BM - 1) / BM : 1;
  int lane_mt = 0;
  if (!WG) {
    int prev = expert_off[min(4 * lane, E)];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      const int hi = expert_off[min(e + 1, E)];
      lane_mt += e < E ? (hi - prev + BM - 1) / BM : 0;
      prev = hi;
    }
  }
  int incl = lane_mt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  const int excl = incl - lane_mt;
  const int total = WG ? 8 * ((E + 7) / 8) * MT * NT : __builtin_amdgcn_readlane(incl, kWave - 1) * NT;

  const int xcd = blockIdx.x % kXcd;
  const int S = gridDim.x / kXcd;  // workgroups per XCD (the grid is a multiple of 8)
  const int q = (total + kXcd - 1) / kXcd;
  const int qx = min(q, total - xcd * q);  // tiles of this XCD (may be <= 0)

  // local tile j of this XCD -> expert, n-tile, m-tile, segment (all uniform)
  struct Tile {
    int e, nt, mt, seg0, seg1;
    int kb, kt;  // weight gradients: first padded K column of B, K slices
  };
  auto decode = [&](int j) {
    const int n = j;  // global tile index
    if (WG) {
      const int pos = n / (MT * NT), rem = n - pos * MT * NT;
      Tile t{perm_row[pos], rem % NT, rem / NT, 0, 0, 0, 0};
      if (t.e >= 0) {
        t.seg0 = expert_off[t.e];  // the expert's slots (A rows)
        t.seg1 = expert_off[t.e + 1];
        t.kb = kpad[t.e];  // and its padded columns of B
        t.kt = (kpad[t.e + 1] - t.kb) / BK;
      }
      return t;
    }
    const uint64_t bal = __ballot(incl * NT > n);
    const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)bal) - 1);
    int first = __builtin_amdgcn_readlane(excl, L);
    Tile t{0, 0, 0, 0, 0, 0, 0};
    int lo = expert_off[min(4 * L, E)];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int e = 4 * L + qq;
      const int hi = expert_off[min(e + 1, E)];
      const int m = e < E ? (hi - lo + BM - 1) / BM : 0;
      if (m > 0 && first * NT <= n && n < (first + m) * NT) {
        t.e = e;
        const int rem = n - first * NT;
        const int b = rem / (kMBlock * NT);
        const int bm = min(kMBlock, m - b * kMBlock);
        const int within = rem - b * kMBlock * NT;
        t.nt = within / bm;
        t.mt = b * kMBlock + within % bm;
        t.seg0 = lo;
        t.seg1 = hi;
      }
      first += m;
      lo = hi;
    }
    return t;
  };

  // Lane-dependent values of the tile set-up and the epilogue are derived
  // from this copy of the thread id, which the compiler cannot see through:
  // it recomputes them where they are used instead of hoisting them out of
  // the tile loop and keeping them live across the K loop.
  auto opaque_tid = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  };
  // the same for uniform values (e.g. the row strides of the output stores)
  auto opaque_s = [&](int v) {
    asm volatile("" : "+s"(v));
    return v;
  };

  // ---- per-tile geometry
  // An expert's rows are split evenly, in whole 32-row bands, over its
  // ceil(rows / BM) m-tiles, so the m-tiles of one weight panel cost the
  // same and stay in step.
  auto tile_rows = [&](const Tile& t, int& m0, int& m1) {
    if (WG) {  // rows of A (the weight gradient's rows)
      m0 = t.mt * BM;
      m1 = min(M0, m0 + BM);
      return;
    }
    const int me = t.seg1 - t.seg0, nmt = (me + BM - 1) / BM;
    const int rows_per = min(BM, ((me + nmt - 1) / nmt + 31) & ~31);
    m0 = t.seg0 + t.mt * rows_per;
    m1 = min(t.seg1, m0 + rows_per);
  };
  // A wave's DMA slots fetch tile rows 64 wave .. 64 wave + 63 (slot i of
  // lane l: row 64 wave + 8 i + l / 8). Each lane loads the perm_row entry
  // of row 64 wave + l (gate/up gathers its rows; down reads h in slot
  // order), and set_aoff hands the entries to the slots by lane shuffles.
  auto load_rows = [&](int m0, int m1) {
    const int ln = opaque_tid() & (kWave - 1);
    const int sl = min(m0 + 64 * wave + ln, m1 - 1);
    return SWIGLU ? perm_row[sl] : sl;
  };
  uint32_t aoff[A_INS], boff[B_INS];
  auto set_aoff = [&](int src_row) {
    const int ln = opaque_tid() & (kWave - 1);
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = RPI * (wave * A_INS + i) + ln / CH;
      const int c = swz_ch<CH>(r, ln % CH) - r * CH;
      const int src = __shfl(src_row, RPI * i + ln / CH, kWave);
      aoff[i] = (uint32_t)src * krow + (uint32_t)c * 16 + kDmaBias - 1024u * (i & 3);
    }
  };
  // Weight gradients: A is read as it lies, [slot][M0] (M contiguous), one
  // K slice = 64 slot rows of the tile's 256 columns. DMA instruction i of
  // the wave fills K rows 2 (wave A_INS + i) + {0, 1} of the stage, 512
  // bytes each, lane l the physical 16-byte chunk l % 32 of row l / 32 with
  // the logical chunk (l % 32) ^ 2 (row & 3) in it (as the data gradients'
  // transposed weights); columns past M0 read the last 8 again.
  auto set_aoff_raw = [&](int m0) {
    const int ln = opaque_tid() & (kWave - 1);
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = 2 * (wave * A_INS + i) + ln / 32;
      const int c = (ln % 32) ^ (2 * (r & 3));
      const int m = min(m0 + c * 8, M0 - 8);
      aoff[i] = (uint32_t)(r * M0 + m) * 2u + kDmaBias - 1024u * (i & 3);
    }
  };
  const bool b_up = SWIGLU && wave * B_INS * RPI >= BN / 2;  // wave-uniform
  auto set_boff = [&](int c0) {
    const int ln = opaque_tid() & (kWave - 1);
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int r = RPI * (wave * B_INS + i) + ln / CH;
      const int c = swz_ch<CH>(r, ln % CH) - r * CH;
      const int n = min(c0 + (b_up ? r - BN / 2 : r), N0 - 1);
      boff[i] = (uint32_t)n * krow + (uint32_t)c * 16 + kDmaBias - 1024u * (i & 3);
    }
  };
  const char* a_base = reinterpret_cast<const char*>(A) - kDmaBias;
  auto b_base_of = [&](int e) {
    return reinterpret_cast<const char*>(b_up ? B1 : B0) + (size_t)e * N0 * krow - kDmaBias;
  };
  // Weight gradients: A from the expert's first slot row, B from its first
  // padded column. In the last slice of an expert whose slot count is not a
  // multiple of 64, rows past its last slot read that last slot's row again
  // (B is zero there, and no other expert's rows enter its gradient).
  int a_clamp_kt = -1, a_clamp_r = 0;  // that slice, and the last valid row in it
  auto wg_bases = [&](const Tile& t, const char*& bb) {
    a_base = reinterpret_cast<const char*>(A) + (size_t)t.seg0 * M0 * 2 - kDmaBias;
    bb = reinterpret_cast<const char*>(B0) + (size_t)t.kb * 2 - kDmaBias;
    const int len = t.seg1 - t.seg0;
    a_clamp_kt = (t.e >= 0 && len % BK) ? t.kt - 1 : -1;
    a_clamp_r = len - 1 - (t.kt - 1) * BK;
  };
  auto wg_kt = [&](const Tile& t) { return t.e >= 0 ? t.kt : 0; };
  // DMA instructions i, i+1 (i even) of K slice kt into ring slot gs
  // (slots count slices across tiles: slice kt of a tile starting at slot g
  // goes to stA(g + kt), stB(g + kt))
  auto dma2 = [&](int i, int kt, int gs, const char* b_base) {
    const bool is_a = i < A_INS;
    const int ii = is_a ? i : i - A_INS;
    const int ins = is_a ? A_INS : B_INS;
    const u32x4* stage = is_a ? stA(gs) : stB(gs);
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        lds_addr(stage + RPI * (wave * ins + (ii & ~3)) * CH));
    const char* base = (is_a ? a_base : b_base) + (size_t)kt * (BK * 2);
    uint32_t v0 = is_a ? aoff[ii] : boff[ii];
    uint32_t v1 = is_a ? aoff[ii + 1] : boff[ii + 1];
    if (WG && is_a) {
      base = a_base + (size_t)kt * BK * M0 * 2;  // slice kt = slot rows 64 kt ..
      if (kt == a_clamp_kt) {  // uniform
        const int r = 2 * (wave * A_INS + ii) + (lane >> 5);
        v0 -= (uint32_t)(max(0, r - a_clamp_r) * M0 * 2);
        v1 -= (uint32_t)(max(0, r + 2 - a_clamp_r) * M0 * 2);
      }
    }
    if ((ii & 3) == 0) dma_pair<0>(v0, v1, base, m0v);
    else dma_pair<2048>(v0, v1, base, m0v);
  };
  // first A slice and first NSB-1 B slices of a tile starting at slot g
  // Weight gradients: A(0), B(0), B(1) of a tile starting at slot g (its
  // A(1) and B(2) stages stage the previous tile's output meanwhile).
  auto prologue_wg = [&](int g, const char* b_base, int kt_n) {
    if (kt_n > 0) {
#pragma unroll
      for (int i = 0; i < A_INS; i += 2) dma2(i, 0, g, b_base);
#pragma unroll
      for (int p = 0; p < NSB - 1; ++p)
        if (p < kt_n) {
#pragma unroll
          for (int i = A_INS; i < LPS; i += 2) dma2(i, p, g + p, b_base);
        }
    }
  };
  auto prologue = [&](int g, const char* b_base) {
#pragma unroll
    for (int p = 0; p < NSA - 1; ++p)
      if (p < KT) {
#pragma unroll
        for (int i = 0; i < A_INS; i += 2) dma2(i, p, g + p, b_base);
      }
#pragma unroll
    for (int p = 0; p < NSB - 1; ++p)
      if (p < KT) {
#pragma unroll
        for (int i = A_INS; i < LPS; i += 2) dma2(i, p, g + p, b_base);
      }
  };

  const int wm = wave / WN, wn = wave % WN;
  auto band_row = [&](int tm) { return (tm * WM + wm) * 32; };
  const int li = lane & 31, lk = lane >> 5;
  // Fragment addresses. Fragment rows are r = 32 b + li (b: a 32-row band),
  // so the swizzle term (r / 2) & 7 = (li / 2) & 7 is the same for every
  // fragment of a lane: the LDS index of (row r, chunk c) splits into a
  // per-lane part li CH + (c ^ xo), one value per k-step, a wave-uniform part
  // and a compile-time band offset that the LDS read takes as an immediate.
  // (Left to itself the compiler keeps one address per fragment and k-step
  // live, which crowds out the tile loop's own registers.)
  const int xo = (li >> 1) & 7;
  const int a_uni = wm * 32 * CH;  // band_row(tm) CH = a_uni + tm WM 32 CH
  auto b_row0 = [&](int tn) {        // first B row of fragment tn
    if (SWIGLU) {
      constexpr int half = Cfg::TN / 2;
      return (tn < half ? 0 : BN / 2) + wn * (Cfg::kWaveCols / 2) + (tn % half) * 32;
    }
    return wn * Cfg::kWaveCols + tn * 32;
  };
  auto lane_off = [&](int ks) { return li * CH + ((2 * ks + lk) ^ xo); };
  // Weight gradients: an A fragment from a raw [K][M] stage is two
  // ds_read_b64_tr_b16 (K rows 16 ks + 8 (lane / 32) + 0..3 and + 4..7 of
  // column band_row(tm) + lane % 32, as the data gradients' B fragments).
  // fat0: this lane's byte offset of the first read of band 0 at k-step 0;
  // band tm adds 128 tm bytes (the chunk XOR leaves the band bits alone),
  // k-step ks 8192 ks, the second read 2048.
  uint32_t fat0 = 0;
  if (WG) {
    const int g4 = lane >> 4, sl = lane & 15, kr = 8 * (g4 >> 1) + sl / 4;
    const int col = wm * 32 + 16 * (g4 & 1) + 4 * (sl % 4);
    fat0 = (uint32_t)(kr * 512 + (((col >> 3) ^ (2 * (kr & 3))) << 4) + (col & 7) * 2);
  }
  auto read_at = [&](const u32x4* as, int tm, int ks) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const char* b = reinterpret_cast<const char*>(as) + fat0 + tm * 128 + ks * 8192;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_void_t*)(b));
    const v4i16 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_void_t*)(b + 2048));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  // ---- the walk
  // Tiles are global indices (-1: none). Slot s starts with its XCD's local
  // tiles s and s + S, then claims.
  auto own = [&](int l) { return l < qx ? xcd * q + l : -1; };
  // The global tile of claim c on this XCD's counter. Launches of at least
  // 8 tiles per workgroup: once the XCD's own tiles are all taken,
  // thread 0 claims from the other XCDs' counters in turn (the XCDs run at
  // different speeds, so equal shares end apart: up to 13% on a skewed
  // load); every counter value is still taken by exactly one claim. With
  // fewer tiles a stolen tile's lost L2 sharing and the serial claims cost
  // more than the tail they save.
  const bool steal = q >= 8 * S;
  auto next_global = [&](int c) {
    int gt = own(2 * S + c);
    for (int i = 1; i < kXcd && gt < 0 && steal; ++i) {
      const int x2 = (xcd + i) & (kXcd - 1);
      const int q2 = min(q, total - x2 * q);
      if (2 * S >= q2) continue;  // nothing that is claimed there
      const int c2 = (int)atomicAdd(&queue[x2], 1u);
      if (2 * S + c2 < q2) gt = x2 * q + 2 * S + c2;
    }
    return gt;
  };
  int cur_j = own(blockIdx.x / kXcd);
  int nxt_j = own(blockIdx.x / kXcd + S);
  Tile cur{}, nxt{};
  int cm0 = 0, cm1 = 0, nm0 = 0, nm1 = 0;
  int nsrc = 0;
  int g = 0;  // ring slot of the current tile's slice 0
  const char* b_base = nullptr;
  if (cur_j >= 0) {
    cur = decode(cur_j);
    tile_rows(cur, cm0, cm1);
    set_boff(cur.nt * Cfg::kOutCols);
    if (WG) {
      set_aoff_raw(cm0);
      wg_bases(cur, b_base);
      KT = wg_kt(cur);
      prologue_wg(0, b_base, KT);
    } else {
      set_aoff(load_rows(cm0, cm1));
      b_base = b_base_of(cur.e);
      prologue(0, b_base);
    }
  }
  int pend_st = 0;  // store instructions of the previous epilogue (per thread, uniform)
  while (cur_j >= 0) {
    const bool has_next = nxt_j >= 0;  // uniform
    int claim = 0;
    if (has_next) {
      nxt = decode(nxt_j);
      tile_rows(nxt, nm0, nm1);
      if (!WG) nsrc = load_rows(nm0, nm1);  // consumed in this tile's epilogue
      // claim tile i+2 now; its value is read in the epilogue, after the K
      // loop has waited for every load (so reading it costs no extra wait)
      if (tid == 0) claim = (int)atomicAdd(&queue[xcd], 1u);
    }
    const int c0 = cur.nt * Cfg::kOutCols;

    f32x16 acc[Cfg::TM][Cfg::TN];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int jn = 0; jn < Cfg::TN; ++jn)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jn][r] = 0.f;

    const int nb_live = max(0, min(BM / 32, (cm1 - cm0 + 31) / 32));
    const int tm_live = min(Cfg::TM, nb_live > wm ? (nb_live - wm + WM - 1) / WM : 0);
    bf16x8 fa[2][Cfg::TM], fb[2][Cfg::TN];
    auto k_loop = [&](auto live_c) {
      constexpr int LIVE = decltype(live_c)::value;
      constexpr int NM = LIVE * Cfg::TN;
      constexpr int NR = LIVE + Cfg::TN;
      static_assert(NM >= NR || LIVE <= 1, "reads fit between the MFMAs");
      auto kstep = [&](auto chk_c, int set, bool rd, const u32x4* as, const u32x4* bs,
                       int ks_next, int kt, int lo, int hi) {
        constexpr bool CHK = decltype(chk_c)::value;
        const int nd = hi - lo;
        const int lo_ = lane_off(ks_next);
        const u32x4* asl = as + a_uni + lo_;
        const u32x4* bsl = bs + lo_;
        auto read_frag = [&](int jr) {
          if (jr < LIVE && WG)
            fa[set ^ 1][jr] = read_at(as, jr, ks_next);
          else if (jr < LIVE)
            fa[set ^ 1][jr] = __builtin_bit_cast(bf16x8, asl[jr * WM * 32 * CH]);
          else
            fb[set ^ 1][jr - LIVE] = __builtin_bit_cast(bf16x8, bsl[b_row0(jr - LIVE) * CH]);
        };
        auto dma_at = [&](int jm) {
          const int np = nd / 2;
#pragma unroll
          for (int qd = 0; qd < LPS / 2; ++qd) {
            if (qd >= np) break;
            if ((NM > 0 ? qd * NM / np : 0) != jm) continue;
            const int i = lo + 2 * qd;
            const int nx = i < A_INS ? kt + NSA - 1 : kt + NSB - 1;
            // weight gradients: slice 0's share (A(1), B(2)) came with the prologue
            if (!CHK || nx < KT) dma2(i, nx, g + nx, b_base);
          }
        };
        if (NM == 0) {
          dma_at(0);
          return;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jm = 0; jm < NM; ++jm) {
          const int tm = jm / Cfg::TN, tn = jm % Cfg::TN;
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][tn], fa[set][tm],
                                                                 acc[tm][tn], 0, 0, 0);
          if (rd && jm < NR) read_frag(jm);
          if (rd && NM < NR && jm == NM - 1)
#pragma unroll
            for (int r = NM; r < NR; ++r) read_frag(r);
          dma_at(jm);
        }
        if (rd) {
          constexpr int NP = NM < NR ? NM : NR;
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (WG && i < LIVE) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two tr reads
            else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
          if (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      auto read_first = [&](const u32x4* as, const u32x4* bs) {
        if (LIVE == 0) return;
        const int lo_ = lane_off(0);
#pragma unroll
        for (int tm = 0; tm < LIVE; ++tm)
          fa[0][tm] = WG ? read_at(as, tm, 0)
                         : __builtin_bit_cast(bf16x8, as[a_uni + lo_ + tm * WM * 32 * CH]);
#pragma unroll
        for (int tn = 0; tn < Cfg::TN; ++tn)
          fb[0][tn] = __builtin_bit_cast(bf16x8, bs[lo_ + b_row0(tn) * CH]);
      };
      constexpr int KS = BK / 16;
      auto slice_ready = [&](int kt) {
        MOE_WAIT_LGKM0();
        // As in the one-tile kernel. At a tile's slice 0 the issue order
        // after B(0) is: B(1), the previous epilogue's pend_st stores
        // (exactly that many: every thread issues all of them), the next
        // tile's row-index load and the claim; so B(0) has landed once at
        // most kFirst + pend_st remain, and the stores keep draining.
        constexpr int kSteady = (NSB > NSA ? B_INS : 0) + (NSA - 2) * (A_INS + B_INS);
        constexpr int kFirst = (NSB - 2) * B_INS;
        static_assert(kSteady < 64 && kFirst + kMaxPendSt < 64, "vmcnt range");
        if (WG) {
          // Issue order at a tile's start: A(0), B(0), B(1) (if it exists),
          // the previous tile's pend_st stores, the claim. A full tile's
          // stores (kWgSt) alone outnumber the 63 a wait can leave in flight,
          // so waiting for 63 covers A(0) and B(0); otherwise only the loads
          // are counted. From slice 1 on, as in the forward.
          constexpr int kWgSt = Cfg::TM * Cfg::TN * 4;
          static_assert(kWgSt >= 63, "weight-gradient waits");
          if (kt == 0) {
            if (pend_st >= kWgSt) MOE_WAIT_VMCNT(63);
            else if (KT > 1) MOE_WAIT_VMCNT(B_INS);
            else MOE_WAIT_VMCNT(0);
          } else if (kt >= NSA - 1 && kt + NSB - 2 < KT) {
            MOE_WAIT_VMCNT(kSteady);
          } else {
            MOE_WAIT_VMCNT(0);
          }
          wg_barrier();
          return;
        }
        if (kt == 0 && NSB - 2 < KT) {
          if (pend_st == 3 * kStPass) MOE_WAIT_VMCNT(kFirst + 3 * kStPass);
          else if (pend_st == 2 * kStPass) MOE_WAIT_VMCNT(kFirst + 2 * kStPass);
          else if (pend_st == kStPass) MOE_WAIT_VMCNT(kFirst + kStPass);
          else MOE_WAIT_VMCNT(kFirst);
        } else if (kt > 0 && kt >= NSA - 1 && kt + NSB - 2 < KT) {
          MOE_WAIT_VMCNT(kSteady);
        } else {
          MOE_WAIT_VMCNT(0);
        }
        wg_barrier();
      };
      auto dlo = [](int qd) { return qd * LPS / KS; };
      auto middle_steps = [&](auto chk_c, int kt) {
        const u32x4* as = stA(g + kt);
        const u32x4* bs = stB(g + kt);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks)
          kstep(chk_c, ks & 1, true, as, bs, ks + 1, kt, dlo(ks + 1), dlo(ks + 2));
      };
      auto step = [&](auto chk_c, int kt) {
        middle_steps(chk_c, kt);
        slice_ready(kt + 1);
        kstep(chk_c, 1, true, stA(g + kt + 1), stB(g + kt + 1), 0, kt + 1, 0, dlo(1));
      };
      constexpr std::false_type kNoCheck{};
      constexpr std::true_type kCheck{};
      slice_ready(0);
      read_first(stA(g), stB(g));
#pragma unroll
      for (int i = 0; i < LPS; i += 2)
        if (i < dlo(1)) {
          const int nx = i < A_INS ? NSA - 1 : NSB - 1;
          if (nx < KT) dma2(i, nx, g + nx, b_base);
        }
      static_assert(LPS / KS <= A_INS, "the first DMA share of a slice is A rows only");
      constexpr int kLead = NSA > NSB - 1 ? NSA : NSB - 1;
      int kt = 0;
      for (; kt + kLead < KT; ++kt) step(kNoCheck, kt);
      for (; kt + 1 < KT; ++kt) step(kCheck, kt);
      middle_steps(kCheck, KT - 1);
      kstep(kCheck, 1, false, stA(g), stB(g), 0, KT, 0, 0);
    };
    static_assert(Cfg::TM <= 4, "band-count dispatch");
    if (WG && KT == 0) {
      // an expert without slots (zero gradients) or an unused position
    } else switch (tm_live) {
      case 0: k_loop(std::integral_constant<int, 0>{}); break;
      case 1: k_loop(std::integral_constant<int, 1>{}); break;
      case 2: k_loop(std::integral_constant<int, 2>{}); break;
      case 3: k_loop(std::integral_constant<int, 3>{}); break;
      default: k_loop(std::integral_constant<int, Cfg::TM>{}); break;
    }

    // ---- epilogue of the current tile, prologue of the next
    MOE_WAIT_LGKM0();  // every wave's last fragment reads are done: the ring is free
    wg_barrier();
    // The last slice waited for every load of the wave (the row indices and
    // the claim included) and nothing was issued since, so this costs
    // nothing; it tells the compiler so, and the claim moves to an SGPR
    // (otherwise the compiler waits for it where it is used, after the next
    // tile's first loads and this tile's stores have been issued).
    MOE_WAIT_VMCNT(0);
    const int claim_s = __builtin_amdgcn_readfirstlane(claim);
    const int gl = g + KT - 1;  // ring slot of the last slice: its stages stage the output
    g += KT;
    if constexpr (WG) {
      char* const rb = reinterpret_cast<char*>(ring);
      int claimed = 0, kt_n = 0;
      if (has_next) {
        // hand the claim (tile i+2) to every wave before the ring is refilled
        if (tid == 0) *reinterpret_cast<int*>(rb) = next_global(claim_s);
        wg_barrier();
        claimed = *reinterpret_cast<const int*>(rb);
        MOE_WAIT_LGKM0();
        wg_barrier();
        set_aoff_raw(nm0);
        set_boff(nxt.nt * Cfg::kOutCols);
        wg_bases(nxt, b_base);
        kt_n = wg_kt(nxt);
        prologue_wg(g, b_base, kt_n);
      }
      // fp32 gradient rows through the two ring stages the prologue left
      // free (32 rows each), four passes of 64 tile rows: each wave writes
      // its band's 16-byte pieces (chunk index XOR-ed with the row), then
      // every wave stores whole 1 KiB rows, one per instruction, as
      // non-temporal stores: nothing reads the gradients back, and whole
      // lines need no merging in the L2.
      pend_st = 0;
      if (cur.e >= 0) {
        const int etid = opaque_tid();
        const int eli = etid & 31, elk = (etid >> 5) & 1;
        const int ln = etid & 63;
        const int n0e = opaque_s(N0);
        u32x4* const rg0 = stA(g + 1);
        u32x4* const rg1 = stB(g + 2);
#pragma unroll
        for (int ps = 0; ps < Cfg::TM; ++ps) {
          if (cm0 + 64 * ps >= cm1) break;  // uniform
          if (ps) wg_barrier();  // the previous pass has been read out
          u32x4* wr = (wm ? rg1 : rg0) + eli * 64;
#pragma unroll
          for (int tn = 0; tn < Cfg::TN; ++tn) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              f32x4 v;
#pragma unroll
              for (int e4 = 0; e4 < 4; ++e4) v[e4] = acc_read(acc[ps][tn][4 * qd + e4]);
              const int ch = wn * 32 + tn * 8 + 2 * qd + elk;
              wr[ch ^ eli] = __builtin_bit_cast(u32x4, v);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          MOE_WAIT_LGKM0();
          wg_barrier();
          const bool colok = 4 * ln < n0e - c0;
#pragma unroll
          for (int i0 = 0; i0 < 16; i0 += 8) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int r = wave + 4 * (i0 + i);
              v[i] = (r < 32 ? rg0 : rg1)[(r & 31) * 64 + (ln ^ (r & 31))];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int row = cm0 + 64 * ps + wave + 4 * (i0 + i);
              float* orow = row < msplit ? O0 + ((size_t)cur.e * msplit + row) * n0e
                                         : O1 + ((size_t)cur.e * (M0 - msplit) + (row - msplit)) * n0e;
              if (colok) __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4*>(orow + c0 + 4 * ln));
            }
          }
          pend_st += 16;
        }
      }
      if (!has_next) break;  // uniform
      cur = nxt;
      cm0 = nm0;
      cm1 = nm1;
      KT = kt_n;
      cur_j = nxt_j;
      nxt_j = __builtin_amdgcn_readfirstlane(claimed);
      continue;
    }
    if (has_next) {
      // every DMA of this tile has landed (its last slice waited for all),
      // so the row indices loaded during the K loop are in too
      set_aoff(nsrc);
      set_boff(nxt.nt * Cfg::kOutCols);
      b_base = b_base_of(nxt.e);
    }
    // The next tile's prologue (its first A slice and first NSB-1 B slices,
    // kProCalls DMA pairs, in the order of prologue()) is issued spread over
    // the first staging pass, one or two pairs per fragment group, so the
    // wave's VALU and LDS work of the staging runs while the memory pipeline
    // takes the DMA instructions (issued in one run, they held the wave for
    // about as long as the TA needs for them). All of it precedes the
    // output stores, as the next tile's first wait assumes.
    constexpr int kProA = (NSA - 1) * (A_INS / 2), kProCalls = kProA + (NSB - 1) * (B_INS / 2);
    auto pro_call = [&](int c) {
      if (c < kProA) {
        const int p = c / (A_INS / 2), i = 2 * (c % (A_INS / 2));
        if (p < KT) dma2(i, p, g + p, b_base);
      } else {
        const int cc = c - kProA;
        const int p = cc / (B_INS / 2), i = A_INS + 2 * (cc % (B_INS / 2));
        if (p < KT) dma2(i, p, g + p, b_base);
      }
    };
    constexpr int kGroups = SWIGLU ? Cfg::TM * (Cfg::TN / 2) : (Cfg::TM / 2) * Cfg::TN;
    static_assert(SWIGLU || Cfg::TM % 2 == 0, "two staging passes for down");
    auto pro_part = [&](int gi) {  // gi: fragment group of the first staging pass
      if (!has_next) return;       // uniform
#pragma unroll
      for (int c = gi * kProCalls / kGroups; c < (gi + 1) * kProCalls / kGroups; ++c) pro_call(c);
    };
    // Output staging: rows go through the two stages of the last slice,
    // region 0 = its A stage, region 1 = its B stage (32 KiB each), 16-byte
    // chunks XOR-swizzled by row; then whole rows are stored, 16 bytes per
    // lane. gate/up (h, 128 columns, 256 B a row): rows 0-127 and 128-255.
    // down (y, 256 columns, 512 B a row): two passes of 128 rows, 64 rows
    // per region. gate/up keeping u and v: three passes of the whole tile,
    // h, then u, then v (the u | v rows of UV, 2 N0 wide).
    // byte offsets of the two regions in the ring (integers, so every access
    // below stays an LDS access the compiler can see)
    const int rgn0 = (gl % NSA) * kStageA * 16;
    const int rgn1 = (NSA * kStageA + (gl % NSB) * kStageB) * 16;
    char* const ring_b = reinterpret_cast<char*>(ring);
    constexpr int OC = Cfg::kOutCols;
    constexpr int CPR = OC / 8;                  // 16-byte chunks per row
    constexpr int RPR = 32768 / (OC * 2);         // rows per region
    constexpr int PASSES = SWIGLU ? (KEEP ? 3 : 1) : 2;
    constexpr int PR = SWIGLU ? BM : BM / PASSES;  // rows per pass
    static_assert(PR == 2 * RPR, "a pass fills both regions");
    auto ot_addr = [&](int row, int col) {  // row within the pass
      return ring_b + (row < RPR ? rgn0 : rgn1) + (row % RPR) * (OC * 2) +
             (((col >> 3) ^ (row & (CPR - 1))) << 4) + ((col & 7) << 1);
    };
    const int rows_here = cm1 - cm0;
    const int etid = opaque_tid();
    const int eli = etid & 31, elk = (etid >> 5) & 1;
    constexpr int RSTEP = Cfg::kThreads / CPR;
    constexpr int NPASS = PR / RSTEP;
    static_assert(Cfg::kThreads % CPR == 0 && PR % RSTEP == 0 && NPASS % 8 == 0, "passes");
    // Every thread issues all of its stores (a fixed count, which the next
    // tile's first wait relies on): a row past the tile's last one stores
    // the last row again and a column chunk past N0 the last chunk again,
    // the same bytes to the same addresses. A pass with no row of the tile
    // (down, at most 128 rows) is skipped as a whole.
    const int oc = etid % CPR, r0 = etid / CPR;
    const int occ = min(oc, (N0 - c0) / 8 - 1);
    const int col = c0 + occ * 8;
    pend_st = 0;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      if (!SWIGLU && ps && rows_here <= ps * PR) break;  // uniform
      if (ps) wg_barrier();  // the previous pass has been read out
      constexpr int TMP = SWIGLU ? Cfg::TM : Cfg::TM / PASSES;  // bands of this wave in one pass
#pragma unroll
      for (int b = 0; b < TMP; ++b) {
        const int tm = SWIGLU ? b : ps * TMP + b;
        const int row = band_row(tm) - (SWIGLU ? 0 : ps * PR) + eli;
        if (SWIGLU) {
          constexpr int half = Cfg::TN / 2;
#pragma unroll
          for (int tg = 0; tg < half; ++tg) {
            if (ps == 0) pro_part(b * half + tg);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              const int cc = wn * (Cfg::kWaveCols / 2) + tg * 32 + 8 * qd + 4 * elk;
              float u[4], v[4];
#pragma unroll
              for (int e4 = 0; e4 < 4; ++e4) {
                if (ps != 2) u[e4] = acc_read(acc[tm][tg][4 * qd + e4]);
                if (ps != 1) v[e4] = acc_read(acc[tm][tg + half][4 * qd + e4]);
              }
              uint2 pk;
              if (ps == 0) {  // h = silu(u) v
                pk.x = pack_bf16x2(silu_mul(u[0], v[0]), silu_mul(u[1], v[1]));
                pk.y = pack_bf16x2(silu_mul(u[2], v[2]), silu_mul(u[3], v[3]));
              } else {  // u, then v
                const float* w4 = ps == 1 ? u : v;
                pk.x = pack_bf16x2(w4[0], w4[1]);
                pk.y = pack_bf16x2(w4[2], w4[3]);
              }
              *reinterpret_cast<uint2*>(ot_addr(row, cc)) = pk;
            }
            // one fragment pair at a time: the compiler would otherwise read
            // every accumulator of the pass into VGPRs first
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int tn = 0; tn < Cfg::TN; ++tn) {
            if (ps == 0) pro_part(b * Cfg::TN + tn);
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              const int cc = wn * Cfg::kWaveCols + tn * 32 + 8 * qd + 4 * elk;
              float a[4];
#pragma unroll
              for (int e4 = 0; e4 < 4; ++e4) a[e4] = acc_read(acc[tm][tn][4 * qd + e4]);
              uint2 pk;
              pk.x = pack_bf16x2(a[0], a[1]);
              pk.y = pack_bf16x2(a[2], a[3]);
              *reinterpret_cast<uint2*>(ot_addr(row, cc)) = pk;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __syncthreads();
      const int n0e = opaque_s(N0);
      const int last = rows_here - 1 - (SWIGLU ? 0 : ps * PR);  // last row of the tile in this pass
      // h and y: rows of N0; u, v: the halves of UV's rows of 2 N0
      const int ostride = (KEEP && ps > 0) ? 2 * n0e : n0e;
      uint16_t* gout = (KEEP && ps > 0)
                           ? UV + (size_t)cm0 * ostride + (ps == 2 ? n0e : 0) + col
                           : C + (size_t)(cm0 + (SWIGLU ? 0 : ps * PR)) * n0e + col;
#pragma unroll
      for (int p0 = 0; p0 < NPASS; p0 += 8) {
        u32x4 v[8];
        int rr[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          rr[jj] = min(r0 + (p0 + jj) * RSTEP, last);
          v[jj] = *reinterpret_cast<const u32x4*>(ot_addr(rr[jj], occ * 8));
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          *reinterpret_cast<u32x4*>(gout + (size_t)rr[jj] * ostride) = v[jj];
      }
      pend_st += NPASS;
      MOE_WAIT_LGKM0();
    }
    if (!has_next) break;  // uniform
    // hand the claim (tile i+2) to every wave through region 0, then move on
    wg_barrier();  // every staged row has been read
    if (tid == 0) *reinterpret_cast<int*>(ring_b + rgn0) = next_global(claim_s);
    wg_barrier();
    const int claimed = *reinterpret_cast<const int*>(ring_b + rgn0);  // read before the next
    // tile's slice 0 barrier, after which its A(1) DMA may overwrite region 0
    cur = nxt;
    cm0 = nm0;
    cm1 = nm1;
    cur_j = nxt_j;
    nxt_j = __builtin_amdgcn_readfirstlane(claimed);
  }
  // The last workgroup to finish leaves the queue zeroed for the next
  // launch. Every workgroup's claims have returned (their values were used)
  // before it counts itself finished, so no claim can follow the reset; no
  // fence is needed (one would write back the XCD's whole L2).
  if (tid == 0) {
    if (__hip_atomic_fetch_add(&queue[kXcd], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        gridDim.x - 1) {
#pragma unroll
      for (int i = 0; i <= kXcd; ++i)
        __hip_atomic_store(&queue[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------- fp32 MFMA

// fp32 expert launches on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).
// A tile is 64 slots x 64 output columns; its 4 wavefronts are 2 x 2, each
// owning 32 slots x 32 columns: for gate/up one 32 x 32 block of u and one
// of v (the same columns of W_gate and W_up, so u and v of an element sit
// in the same lane and register), for down one block of y. K runs in 32-wide
// slices staged in LDS K-major (A as [k][slot], B as [k][weight row]), so
// the operand a lane feeds each MFMA (row lane % 32, k = 2i + lane / 32) is
// one 4-byte LDS read and a wave's read covers consecutive words. d and F
// are multiples of 64, so K is a whole number of slices.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ perm_row,
                                                       const int32_t* __restrict__ expert_off,
                                                       int E, const float* __restrict__ B0,
                                                       const float* __restrict__ B1, int K,
                                                       int N0, float* __restrict__ C,
                                                       float* __restrict__ UV) {
  constexpr int BM = 64, OC = 64, BK = 32;
  constexpr int BR = SWIGLU ? 2 * OC : OC;  // weight rows per tile
  // LDS row pitch in words: odd, so the 4 consecutive k a thread writes for
  // one row, and the rows of neighbouring threads, fall in distinct banks
  constexpr int PA = BM + 1, PB = BR + 1;
  __shared__ float As[BK * PA];
  __shared__ float Bs[BK * PB];
  __shared__ Sched sc;
  build_schedule(sc, expert_off, E, BM);
  const int NT = (N0 + OC - 1) / OC;
  const int tile = xcd_logical_tile(sc.mt_off[E] * NT);
  if (tile < 0) return;
  int e, nt, mt;
  decode_tile(sc, E, NT, tile, e, nt, mt);
  const int seg0 = expert_off[e], seg1 = expert_off[e + 1];
  const int m0 = seg0 + mt * BM;
  const int c0 = nt * OC;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;

  // Loads: 8 threads per row, each 4 consecutive k (one 16-byte load) of a
  // 32-wide slice; A rows in 2 passes of 32, weight rows in BR / 32.
  const int lr = tid >> 3, lk = (tid & 7) * 4;
  const float* arow[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int s = min(m0 + lr + 32 * p, seg1 - 1);  // rows past the segment: clamped, not stored
    arow[p] = A + (size_t)(perm_row ? perm_row[s] : s) * K;
  }
  constexpr int BP = BR / 32;
  const float* brow[BP];
#pragma unroll
  for (int p = 0; p < BP; ++p) {
    const int r = lr + 32 * p;  // tile row: [0, OC) gate (or down) rows, [OC, 2 OC) up rows
    const float* base = (SWIGLU && r >= OC) ? B1 : B0;
    const int n = min(c0 + (r % OC), N0 - 1);
    brow[p] = base + ((size_t)e * N0 + n) * K;
  }

  f32x16 acc0 = {}, acc1 = {};
  const int ar = wm * 32 + (lane & 31), kh = lane >> 5;
  const int br0 = wn * 32 + (lane & 31), br1 = br0 + OC;
  // The next slice's pieces are loaded before the current one's MFMAs.
  float4 av[2], bv[BP];
  auto load = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) av[p] = *reinterpret_cast<const float4*>(arow[p] + k0 + lk);
#pragma unroll
    for (int p = 0; p < BP; ++p) bv[p] = *reinterpret_cast<const float4*>(brow[p] + k0 + lk);
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = lr + 32 * p;
      As[(lk + 0) * PA + r] = av[p].x;
      As[(lk + 1) * PA + r] = av[p].y;
      As[(lk + 2) * PA + r] = av[p].z;
      As[(lk + 3) * PA + r] = av[p].w;
    }
#pragma unroll
    for (int p = 0; p < BP; ++p) {
      const int r = lr + 32 * p;
      Bs[(lk + 0) * PB + r] = bv[p].x;
      Bs[(lk + 1) * PB + r] = bv[p].y;
      Bs[(lk + 2) * PB + r] = bv[p].z;
      Bs[(lk + 3) * PB + r] = bv[p].w;
    }
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int i = 0; i < BK / 2; ++i) {
      const int kk = 2 * i + kh;
      const float a = As[kk * PA + ar];
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Bs[kk * PB + br0], acc0, 0, 0, 0);
      if (SWIGLU) acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Bs[kk * PB + br1], acc1, 0, 0, 0);
    }
    __syncthreads();  // every wave is done reading the slice
  }
  // Register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4 and
  // column l % 32 of the wave's 32 x 32 block.
  const int col = c0 + wn * 32 + (lane & 31);
  if (col >= N0) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    if (row >= seg1) continue;
    if (SWIGLU) {
      C[(size_t)row * N0 + col] = silu_mul(acc0[r], acc1[r]);
      if (UV) {
        UV[(size_t)row * (2 * N0) + col] = acc0[r];
        UV[(size_t)row * (2 * N0) + N0 + col] = acc1[r];
      }
    } else {
      C[(size_t)row * N0 + col] = acc0[r];
    }
  }
}

// ---------------------------------------------------------------- launch

// Tile shape of both launches: 256 x 256 (for gate/up, 128 gate + 128 up B
// rows = 128 F columns), 64-wide K slices, 4 wavefronts as 2 x 2 (128 x 128
// each, accumulators in AGPRs, one wave per SIMD), 2 LDS stages of A rows and
// 3 of weight rows (the whole 160 KiB of LDS). 256 x 256 is the smallest tile
// whose LDS fill rate (BM*BN/(BM+BN) = 128 flop per byte) lets the L2 keep up
// with the MFMA peak; 128 x 128 wave tiles read a third fewer fragment bytes
// from LDS per MFMA than 64 x 128 ones, which matters on a power-limited chip
// (8 waves of 64 x 128 are ~1-3% slower here).
constexpr int kBM = 256, kBN = 256, kBK = 64, kWM = 2, kWN = 2, kNSA = 2, kNSB = 3;
// Workspace of the persistent forward launches: the tile queue.
constexpr size_t kExpertWorkspaceBytes = 256;
static_assert(kQueueWords * 4 <= kExpertWorkspaceBytes, "queue fits the workspace");

// The bf16 kernel addresses its operands with 32-bit per-lane byte offsets:
// from the activation matrix (rows x K) and from one expert's weight panel
// (N0 x K), both plus kDmaBias, must stay below 4 GiB.
inline bool dma_offsets_fit(int64_t a_rows, int64_t n0, int64_t k) {
  const int64_t lim = (int64_t(1) << 32) - kDmaBias - 16;
  return a_rows * k * 2 <= lim && n0 * k * 2 <= lim;
}

// Compute units of the current device (cached per device); the persistent
// launches run one workgroup per CU.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kMaxDevices && v > 0) g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Persistent forward launch over at most `tiles_ub` tiles: S workgroups per
// XCD, S = CUs / 8 (one per CU), fewer when there are fewer tiles.
template <bool SWIGLU, bool KEEP = false>
moe_status launch_persistent(const uint16_t* a, const int32_t* perm_row, const int32_t* expert_off,
                             int E, const uint16_t* b0, const uint16_t* b1, int K, int N0,
                             uint16_t* c, uint32_t* queue, int64_t tiles_ub, hipStream_t stream,
                             uint16_t* uv = nullptr) {
  const int cus = cu_count();
  if (cus <= 0) return MOE_ERR_DEVICE;
  const int64_t per_xcd = ceil_div(std::max<int64_t>(tiles_ub, 1), kXcd);
  const int S = (int)std::max<int64_t>(1, std::min<int64_t>(cus / kXcd, per_xcd));
  hipLaunchKernelGGL((ffn_persistent_kernel<SWIGLU, false, KEEP>), dim3(kXcd * S), dim3(256), 0,
                     stream, a, perm_row, expert_off, E, b0, b1, K, N0, c, queue, 0, 0, nullptr,
                     nullptr, nullptr, uv);
  return launch_status();
}

moe_status check_ffn(int32_t T, int32_t E, int32_t k, int32_t d, int32_t F, moe_dtype dt) {
  if (T < 0 || E < 1 || k < 1 || k > E || d < 1 || F < 1 || !valid_dtype(dt)) return MOE_ERR_ARG;
  if (E > kMaxE || k > kMaxK || (int64_t)T * k >= (1ll << 31) || d % 64 || F % 64)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

namespace moe {

bool wgrad_offsets_fit(int64_t m0, int64_t n0, int64_t ldk) { return dma_offsets_fit(m0, n0, ldk); }

bool dgrad_offsets_fit(int64_t rows, int64_t k) { return dma_offsets_fit(rows, 1, k); }

void launch_dgrad_bf16(const uint16_t* a, int64_t rows, const int32_t* expert_off, int E, int K,
                       const uint16_t* w0, const uint16_t* w1, int ksplit, int N0,
                       const uint16_t* uv, uint16_t* c, hipStream_t stream) {
  const int64_t tiles = mtile_upper(rows, E, kBM) * ceil_div(N0, kBN);
  if (uv)
    hipLaunchKernelGGL((dgrad_bf16_kernel<kBM, kBN, kBK, kWM, kWN, kNSA, kNSB, true>),
                       dim3(grid_for(tiles)), dim3(kWM * kWN * kWave), 0, stream, a, nullptr,
                       expert_off, E, w0, w1, K, N0, c, const_cast<uint16_t*>(uv), ksplit);
  else
    hipLaunchKernelGGL((dgrad_bf16_kernel<kBM, kBN, kBK, kWM, kWN, kNSA, kNSB, false>),
                       dim3(grid_for(tiles)), dim3(kWM * kWN * kWave), 0, stream, a, nullptr,
                       expert_off, E, w0, w1, K, N0, c, nullptr, ksplit);
}

moe_status launch_wgrad_bf16(const uint16_t* a, const uint16_t* bt, const int32_t* expert_off,
                             const int32_t* kseg, const int32_t* eorder, int E, int M0, int N0,
                             int ldk, int msplit, float* o0, float* o1, uint32_t* queue,
                             hipStream_t stream) {
  const int64_t tiles = 8 * ceil_div(E, 8) * ceil_div(M0, kBM) * ceil_div(N0, kBN);
  const int cus = cu_count();
  if (cus <= 0) return MOE_ERR_DEVICE;
  const int S = (int)std::max<int64_t>(1, std::min<int64_t>(cus / kXcd, tiles / kXcd));
  hipLaunchKernelGGL((ffn_persistent_kernel<false, true>), dim3(kXcd * S), dim3(256), 0, stream,
                     a, eorder, expert_off, E, bt, nullptr, ldk, N0, nullptr, queue, M0, msplit, o0,
                     o1, kseg);
  return launch_status();
}

}  // namespace moe

using namespace moe;

MOE_EXPORT size_t moe_expert_workspace_bytes(void) { return kExpertWorkspaceBytes; }

MOE_EXPORT moe_status moe_expert_gate_up(const void* x_disp, const int32_t* perm_row,
                                         const int32_t* expert_off, int32_t T, int32_t E,
                                         int32_t k, int32_t d, int32_t F, const void* w_gate,
                                         const void* w_up, moe_dtype dt, void* h, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_ffn(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_disp || !perm_row || !expert_off || !w_gate || !w_up || !h) return MOE_ERR_ARG;
  if (!workspace || workspace_bytes < kExpertWorkspaceBytes || (uintptr_t)workspace % 16)
    return MOE_ERR_WORKSPACE;
  if (((uintptr_t)x_disp | (uintptr_t)w_gate | (uintptr_t)w_up | (uintptr_t)h) % 16)
    return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    if (!dma_offsets_fit(rows, F, d)) return MOE_ERR_UNSUPPORTED;
    const int64_t tiles = mtile_upper(rows, E, kBM) * ceil_div(F, kBN / 2);
    return launch_persistent<true>(static_cast<const uint16_t*>(x_disp), perm_row, expert_off, E,
                                   static_cast<const uint16_t*>(w_gate),
                                   static_cast<const uint16_t*>(w_up), d, F,
                                   static_cast<uint16_t*>(h), static_cast<uint32_t*>(workspace),
                                   tiles, stream);
  }
  const int64_t tiles = mtile_upper(rows, E, 64) * ceil_div(F, 64);
  hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid_for(tiles)), dim3(256), 0, stream,
                     static_cast<const float*>(x_disp), perm_row, expert_off, E,
                     static_cast<const float*>(w_gate), static_cast<const float*>(w_up), d, F,
                     static_cast<float*>(h), nullptr);
  return launch_status();
}

MOE_EXPORT moe_status moe_expert_gate_up_save(const void* x_disp, const int32_t* perm_row,
                                              const int32_t* expert_off, int32_t T, int32_t E,
                                              int32_t k, int32_t d, int32_t F,
                                              const void* w_gate, const void* w_up, moe_dtype dt,
                                              void* h, void* uv, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_ffn(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_disp || !perm_row || !expert_off || !w_gate || !w_up || !h || !uv) return MOE_ERR_ARG;
  if (!workspace || workspace_bytes < kExpertWorkspaceBytes || (uintptr_t)workspace % 16)
    return MOE_ERR_WORKSPACE;
  if (((uintptr_t)x_disp | (uintptr_t)w_gate | (uintptr_t)w_up | (uintptr_t)h | (uintptr_t)uv) % 16)
    return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    if (!dma_offsets_fit(rows, F, d)) return MOE_ERR_UNSUPPORTED;
    const int64_t tiles = mtile_upper(rows, E, kBM) * ceil_div(F, kBN / 2);
    return launch_persistent<true, true>(static_cast<const uint16_t*>(x_disp), perm_row,
                                         expert_off, E, static_cast<const uint16_t*>(w_gate),
                                         static_cast<const uint16_t*>(w_up), d, F,
                                         static_cast<uint16_t*>(h),
                                         static_cast<uint32_t*>(workspace), tiles, stream,
                                         static_cast<uint16_t*>(uv));
  } else {
    const int64_t tiles = mtile_upper(rows, E, 64) * ceil_div(F, 64);
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid_for(tiles)), dim3(256), 0, stream,
                       static_cast<const float*>(x_disp), perm_row, expert_off, E,
                       static_cast<const float*>(w_gate), static_cast<const float*>(w_up), d, F,
                       static_cast<float*>(h), static_cast<float*>(uv));
  }
  return launch_status();
}

MOE_EXPORT moe_status moe_expert_down(const void* h, const int32_t* expert_off, int32_t T,
                                      int32_t E, int32_t k, int32_t d, int32_t F,
                                      const void* w_down, moe_dtype dt, void* y, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_ffn(T, E, k, d, F, dt);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!h || !expert_off || !w_down || !y) return MOE_ERR_ARG;
  if (!workspace || workspace_bytes < kExpertWorkspaceBytes || (uintptr_t)workspace % 16)
    return MOE_ERR_WORKSPACE;
  if (((uintptr_t)h | (uintptr_t)w_down | (uintptr_t)y) % 16) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (dt == MOE_BF16) {
    if (!dma_offsets_fit(rows, d, F)) return MOE_ERR_UNSUPPORTED;
    const int64_t tiles = mtile_upper(rows, E, kBM) * ceil_div(d, kBN);
    return launch_persistent<false>(static_cast<const uint16_t*>(h), nullptr, expert_off, E,
                                    static_cast<const uint16_t*>(w_down), nullptr, F, d,
                                    static_cast<uint16_t*>(y), static_cast<uint32_t*>(workspace),
                                    tiles, stream);
  }
  const int64_t tiles = mtile_upper(rows, E, 64) * ceil_div(d, 64);
  hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid_for(tiles)), dim3(256), 0, stream,
                     static_cast<const float*>(h), nullptr, expert_off, E,
                     static_cast<const float*>(w_down), nullptr, F, d, static_cast<float*>(y),
                     nullptr);
  return launch_status();
}

MOE_EXPORT moe_status moe_grouped_ffn(const void* x_disp, const int32_t* perm_row,
                                      const int32_t* expert_off, int32_t T, int32_t E, int32_t k,
                                      int32_t d, int32_t F, const void* w_gate, const void* w_up,
                                      const void* w_down, moe_dtype dt, void* h, void* y,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  moe_status st = moe_expert_gate_up(x_disp, perm_row, expert_off, T, E, k, d, F, w_gate, w_up,
                                     dt, h, workspace, workspace_bytes, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down(h, expert_off, T, E, k, d, F, w_down, dt, y, workspace, workspace_bytes,
                         stream);
}
