// Building blocks of the bf16 expert GEMM kernels (gfx950): the block -> tile
// mapping, the compile-time tile shapes, the LDS swizzles, the global -> LDS
// transfers of a tile's K steps, the MFMA fragment reads and the epilogue
// that stores a finished tile.  Internal to libmoe.
#pragma once

#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace moe {
namespace {

struct TileCoords {
  int group;   // expert index relative to group_base (routed) or 0
  int row0;
  int nrows;
  int ntile;   // N-tile within the group
  int ngroup;  // N-group (shared experts laid along N)
  int kpart;   // part of a split K (static tiling)
  bool valid;
};

// Block -> (expert, N-tile, M-tile).  The logical tile order runs expert by
// expert, N-tile by N-tile, with the expert's M-tiles fastest, so a window of
// consecutive logical tiles is a compact (all M-tiles) x (a few N-tiles) block
// of one expert: its weight tiles and its token rows are each fetched once
// into L2 and shared.  Hardware deals workgroups to the 8 XCDs round-robin
// (block p -> XCD p % 8); each XCD takes a contiguous eighth of the logical
// tiles that actually exist (their count is read from the device tile list),
// so the XCDs stay balanced whatever the routing.
template <int TBM>
__device__ __forceinline__ TileCoords tile_coords(const GroupedGemm& p, int ntn,
                                                  int /*nblocks*/) {
  TileCoords tc{0, 0, 0, 0, 0, 0, false};
  const int ntn_all = ntn * p.ngroups_n;
  const int mtiles = p.tiles ? *p.ntiles : (p.static_rows + TBM - 1) / TBM;
  const int x = blockIdx.x & 7;
  const int i = blockIdx.x >> 3;
  int L;
  if (p.kcut_slots > 0) {
    // Two K parts cut unevenly (kcut_steps): each XCD takes a contiguous
    // eighth of the tiles and runs all their part-0 units before any part-1
    // unit, so the longer parts go first and the M-tiles of one weight tile
    // still start each part together.
    const int ntiles = mtiles * ntn_all;
    const int tx = (ntiles + 7) >> 3;
    if (i >= 2 * tx) return tc;
    tc.kpart = i >= tx ? 1 : 0;
    L = x * tx + i - tc.kpart * tx;
    if (L >= ntiles) return tc;
  } else {
    const int ks = p.ksplit;
    const int total = mtiles * ntn_all * ks;
    const int per = (total + 7) >> 3;
    if (i >= per) return tc;
    const int LK = x * per + i;
    if (LK >= total) return tc;
    tc.kpart = LK % ks;   // K parts of one tile are adjacent: they share A rows
    L = LK / ks;
  }
  int m, n_all;
  if (p.tiles) {
    // expert e owns logical tiles [tstart[e] * ntn_all, tstart[e+1] * ntn_all)
    int lo = 0, hi = p.n_experts;            // find e with tstart[e]*ntn_all <= L
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tstart[mid] * ntn_all <= L) lo = mid; else hi = mid;
    }
    const int t0 = p.tstart[lo];
    const int mt = p.tstart[lo + 1] - t0;
    const int local = L - t0 * ntn_all;
    n_all = local / mt;
    m = t0 + local % mt;
    const Tile t = p.tiles[m];
    tc.group = t.group;
    tc.row0 = t.row0;
    tc.nrows = t.nrows;
  } else {
    n_all = L / mtiles;
    m = L % mtiles;
    tc.row0 = m * TBM;
    tc.nrows = min(TBM, p.static_rows - tc.row0);
  }
  tc.ngroup = n_all / ntn;
  tc.ntile = n_all % ntn;
  tc.valid = tc.nrows > 0;
  return tc;
}

// The K step where part 0 ends when a plain GEMM's two K parts are cut
// unevenly for `slots` resident workgroups (part-0 units dispatched first).
// With ntiles = k slots + rem: part 0 takes (k+1)/(k+2) of K when rem
// (k+2) <= slots, so the slots that ran a long part 0 and then a short part
// 1 finish with those that ran two long parts; 2/3 when there are fewer
// tiles than slots but more than half as many; otherwise half.  (Modelled as
// rounds of equal tiles: 592 tiles on 512 slots take 1.33 tile lengths
// instead of 1.5 with equal halves.)
__device__ __forceinline__ int kcut_steps(int nk, int ntiles, int slots) {
  const int k = ntiles / slots;
  const int rem = ntiles - k * slots;
  int num = 1, den = 2;
  if (k >= 1 && rem * (k + 2) <= slots) {
    num = k + 1;
    den = k + 2;
  } else if (k == 0 && 2 * ntiles > slots) {
    num = 2;
    den = 3;
  }
  const int cut = (nk * num + den / 2) / den;
  return min(max(cut, 1), nk - 1);
}

// ===========================================================================
// bf16 MFMA kernel, gfx950 data path
//
// Global -> LDS with global_load_lds_dwordx4 (the load unit writes LDS
// directly: no staging registers, no LDS write instructions) into an
// NS-deep ring of stages, so NS-1 K steps of loads are in flight while one is
// computed.  The weight tile keeps the orientation it has in memory:
//   - Row-major weights (N contiguous): the B stage holds K rows, and the
//     MFMA B fragments are read with ds_read_b64_tr_b16, which transposes
//     16-bit elements across each 16-lane group: source lane 4q+r supplies
//     columns 4r..4r+3 of row k_q, and result lane i receives column i of
//     rows k_0..k_3.  Two such reads give a lane the 8 consecutive k values
//     of one column that v_mfma_f32_16x16x32_bf16 takes.
//   - Packed weights (each 32-row block stored column by column, K
//     contiguous): the B stage holds BN column rows laid out like the A
//     stage, and a B fragment is one ds_read_b128, as an A fragment is.
//     Measured in a micro-benchmark of this tile's loop (reads, MFMAs, the
//     LDS transfers and a barrier per K step): 15% faster than the
//     transposing reads, with a third fewer LDS read instructions.
//
// LDS layouts (no padding; XOR swizzles keep every read conflict-free):
//   A stage: BM rows x 2*BK bytes; 16-byte chunk c of row m is stored at
//            a_chunk(m, c) (an XOR of c with bits 1-2 of m).
//   B stage, row-major weights: BK rows x 2*BN bytes; 32-byte segment s
//            (16 columns) of row k sits at segment s ^ ((k & 3) | ((k >> 1) & 4)).
//   B stage, packed weights: BN rows (one per tile column) x 2*BK bytes,
//            chunk c of column row n at a_chunk(n, c), as in the A stage.
//
// The shape is a compile-time configuration: M-tile BM, B-tile width BN
// (SwiGLU: BN/2 columns each of W1 and W3), K step BK, wavefronts NW (WM
// along M), NS stages.  Configurations with at most 80 KB of LDS run two
// workgroups per CU, so one workgroup's barrier, tile set-up and epilogue
// overlap the other's MFMAs.
// ===========================================================================
namespace dma {

template <int BM_, int BN_, int BK_, int NW_, int WM_, int NS_>
struct Shape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NW = NW_, WM = WM_, NS = NS_;
  static constexpr int WN = NW / WM;
  static constexpr int WROWS = BM / WM;
  static constexpr int WCOLS = BN / WN;
  static constexpr int MI = WROWS / 16;              // MFMA tiles per wavefront
  static constexpr int NJ = WCOLS / 16;
  static constexpr int HALVES = BK / 32;             // 32-deep MFMA steps per stage
  static constexpr int A_ROW = 2 * BK;               // bytes per A row
  static constexpr int CA = BK / 8;                  // 16-byte chunks per A row
  static constexpr int B_ROW = 2 * BN;               // bytes per B row
  static constexpr int A_STAGE = BM * A_ROW;
  static constexpr int B_STAGE = BK * B_ROW;
  static constexpr int STAGE = A_STAGE + B_STAGE;
  static constexpr int A_ROWS_PER_LOAD = 1024 / A_ROW;   // one 64-lane x 16 B load
  static constexpr int B_ROWS_PER_LOAD = 1024 / B_ROW;
  static constexpr int A_LOADS = A_STAGE / 1024 / NW;    // per thread per stage
  static constexpr int B_LOADS = B_STAGE / 1024 / NW;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int LDS = NS * STAGE;
  static constexpr int BLOCKS_PER_CU = LDS <= 80 * 1024 ? 2 : 1;
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && NJ % 2 == 0 && MI >= 1, "shape");
  static_assert(A_STAGE % (1024 * NW) == 0 && B_STAGE % (1024 * NW) == 0, "loads");
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(BN / 16 <= 16 && BN >= 128, "B segments");
  static_assert(3 * LOADS < 64, "vmcnt");
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Stored position of 16-byte chunk c of A row m.  The A fragment read
// (ds_read_b128: lane l takes row l % 16, chunk l / 16 of a 32-deep half)
// runs in four LDS cycles of 16 lanes over 16 bank groups of 16 bytes.
// Measured with the bank-conflict counter, lanes share a cycle when they
// agree in lane bit 5 and in the parity of lane bits 2-4 (not simply 16
// consecutive lanes).  With 4 chunks per row (BK = 32): c ^ ((m >> 1) & 2);
// with 8 (BK = 64): c ^ (m & 6).  Either way the 16 lanes of a cycle hit 16
// different bank groups in both halves.
template <int CA>
__device__ __forceinline__ int a_chunk(int m, int c) {
  if constexpr (CA == 8) return c ^ (m & 6);
  return c ^ ((m >> 1) & 2);
}
__device__ __forceinline__ int b_swz(int k) { return (k & 3) | ((k >> 1) & 4); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most `later` stages of LOADS transfers each are in flight.
template <int LOADS>
__device__ __forceinline__ void wait_stages(int later) {
  if (later >= 2) wait_vmcnt<2 * LOADS>();
  else if (later == 1) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
}

// s_waitcnt: at most N vector-memory operations and no LDS operation of this
// wavefront still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
// ... until at most `later` (0..3) stages of LOADS transfers each remain.
template <int LOADS>
__device__ __forceinline__ void wait_stages_lgkm0(int later) {
  if (later >= 3) wait_vmcnt_lgkm0<3 * LOADS>();
  else if (later == 2) wait_vmcnt_lgkm0<2 * LOADS>();
  else if (later == 1) wait_vmcnt_lgkm0<LOADS>();
  else wait_vmcnt_lgkm0<0>();
}

// First B-tile column of MFMA tile j of wavefront column wn.
template <class S, bool SWIGLU>
__device__ __forceinline__ int bcol_of(int j, int wn) {
  if constexpr (SWIGLU) {
    constexpr int H = S::NJ / 2;   // first half: W1 columns, second half: W3
    return (j < H) ? (wn * (S::WCOLS / 2) + j * 16)
                   : (S::BN / 2 + wn * (S::WCOLS / 2) + (j - H) * 16);
  }
  return wn * S::WCOLS + j * 16;
}

// First tile row of MFMA row fragment i (16 rows) of wavefront row wm.  The
// fragments are dealt to the WM wavefront rows in turn, so the rows of a
// short tile (an expert's last) spread evenly over the wavefronts, and with
// them over the SIMDs, when the fragments past the tile's end are skipped.
template <class S>
__device__ __forceinline__ int frag_row(int wm, int i) {
  return (i * S::WM + wm) * 16;
}

// f(integral_constant<int, n>) for a run-time n in 0..N.
template <int N, class F>
__device__ __forceinline__ void with_count(int n, F& f) {
  if constexpr (N == 0) {
    f(std::integral_constant<int, 0>{});
  } else {
    if (n >= N) f(std::integral_constant<int, N>{});
    else with_count<N - 1>(n, f);
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// One 16-byte-per-lane global -> LDS transfer: lane i's 16 bytes from src land
// at LDS byte address lds + 16 i.  Written as asm so that the compiler, which
// cannot tell these LDS writes apart from the LDS reads of other stages, does
// not wait for them before every LDS read; the kernel waits on vmcnt itself.
// The instruction has no result register.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}


// Global sources of one wavefront's share of a tile's K steps, in the LDS
// layout above.
//   A: load i of this wavefront fills rows (wave*A_LOADS + i)*A_ROWS_PER_LOAD
//   onward; lane -> row + lane/CA, stored chunk lane%CA.  Rows past the
//   tile's end repeat its first row (their results are not stored).  In the
//   K-blocked layout (a_block_rows = R > 0) element (row, k) sits at
//   ((k / 32) * R + row) * 32 + k % 32, so one K step of a tile's rows is a
//   contiguous run of memory.
//   B, row-major weights (BT false): load i fills rows (wave*B_LOADS +
//   i)*B_ROWS_PER_LOAD onward; lane -> row + lane/(BN/8), stored 16-byte
//   chunk q = lane%(BN/8), which is half (q&1) of stored segment q/2.
//   B, packed weights (BT true): load i fills column rows (wave*B_LOADS +
//   i)*A_ROWS_PER_LOAD onward; lane -> column row + lane/CA, stored chunk
//   lane%CA, as for A.  In a packed block element (k, n) sits at
//   (n % Wb) * 32 + k % 32, so one K step of a tile's columns is a
//   contiguous run of each block it touches.
//   Columns past N read column 0 (their outputs are never stored).  Either
//   way the step advances by K-step x ldb.
template <bool SWIGLU, class S, bool BT>
struct TileSources {
  const uint16_t* asrc[S::A_LOADS];
  const uint16_t* bsrc[S::B_LOADS];
  int64_t a_kstride;   // elements per unit of k along A (K-blocked: R)
  int64_t ldb;

  __device__ __forceinline__ void init(const GroupedGemm& p, const TileCoords& tc, int wave,
                                       int lane, int n0, int64_t boff) {
    const uint16_t* A = static_cast<const uint16_t*>(p.A);
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) {
      const int r = (wave * S::A_LOADS + i) * S::A_ROWS_PER_LOAD + lane / S::CA;
      const int rr = tc.row0 + (r < tc.nrows ? r : 0);
      const int sc = a_chunk<S::CA>(r, lane % S::CA) * 8;   // source column in the step
      if (p.a_block_rows > 0) {
        asrc[i] = A + ((sc >> 5) * p.a_block_rows + rr) * 32 + (sc & 31);
      } else {
        const int64_t src = p.perm ? static_cast<int64_t>(p.perm[rr] / p.topk) : rr;
        asrc[i] = A + src * p.lda + sc;
      }
    }
    a_kstride = p.a_block_rows > 0 ? p.a_block_rows : 1;
    ldb = p.ldb;
    constexpr int BN = S::BN;
    if constexpr (BT) {
      // packed blocks of w columns, each column's 32 k values contiguous
      const int w = p.b_block_cols;
#pragma unroll
      for (int i = 0; i < S::B_LOADS; ++i) {
        const int n = (wave * S::B_LOADS + i) * S::A_ROWS_PER_LOAD + lane / S::CA;
        const int kk = a_chunk<S::CA>(n, lane % S::CA) * 8;   // k within the step
        const uint16_t* base;
        int col;
        if constexpr (SWIGLU) {
          base = static_cast<const uint16_t*>(n < BN / 2 ? p.B : p.B3);
          col = n0 + (n & (BN / 2 - 1));
        } else {
          base = static_cast<const uint16_t*>(p.B);
          col = n0 + n;
        }
        if (col >= p.N) col = 0;
        const int64_t bo = static_cast<int64_t>(kk >> 5) * 32 * p.ldb +
                           static_cast<int64_t>(col / w) * 32 * w + (col % w) * 32 + (kk & 31);
        bsrc[i] = base + boff + bo;
      }
      return;
    }
    constexpr int BCH = BN / 8;                 // 16-byte chunks per B row
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i) {
      const int kr = (wave * S::B_LOADS + i) * S::B_ROWS_PER_LOAD + lane / BCH;
      const int q = lane % BCH;
      const int seg = (q >> 1) ^ b_swz(kr);
      const int n = seg * 16 + (q & 1) * 8;
      const uint16_t* base;
      int col;
      if constexpr (SWIGLU) {
        base = static_cast<const uint16_t*>(n < BN / 2 ? p.B : p.B3);
        col = n0 + (n & (BN / 2 - 1));
      } else {
        base = static_cast<const uint16_t*>(p.B);
        col = n0 + n;
      }
      if (col >= p.N) col = 0;
      int64_t bo;
      if (p.b_block_cols) {
        // packed: row kr of the step lies in block row kr / 32 (BK = 64 spans
        // two), column col in block col / W
        const int w = p.b_block_cols;
        bo = static_cast<int64_t>(kr >> 5) * 32 * p.ldb + ((col / w) * 32 + (kr & 31)) * w + col % w;
      } else {
        bo = static_cast<int64_t>(kr) * p.ldb + col;
      }
      bsrc[i] = base + boff + bo;
    }
  }

  // Transfer idx (A loads first, then B loads) of this wavefront's share of
  // the K step starting at k0, into the stage at LDS byte address sb.
  template <int IDX>
  __device__ __forceinline__ void issue_one(uint32_t sb, int k0, int wave_u) const {
    if constexpr (IDX < S::A_LOADS) {
      dma16(asrc[IDX] + k0 * a_kstride, sb + (wave_u * S::A_LOADS + IDX) * 1024);
    } else if constexpr (IDX < S::LOADS) {
      constexpr int i = IDX - S::A_LOADS;
      dma16(bsrc[i] + static_cast<int64_t>(k0) * ldb, sb + S::A_STAGE + (wave_u * S::B_LOADS + i) * 1024);
    }
  }
  // This wavefront's transfers of the K step starting at element k0 into the
  // stage at LDS byte address sb (wave_u: the wave index, wave-uniform).
  __device__ __forceinline__ void issue(uint32_t sb, int k0, int wave_u) const {
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i)
      dma16(asrc[i] + k0 * a_kstride, sb + (wave_u * S::A_LOADS + i) * 1024);
    const int64_t kb = static_cast<int64_t>(k0) * ldb;
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i)
      dma16(bsrc[i] + kb, sb + S::A_STAGE + (wave_u * S::B_LOADS + i) * 1024);
  }
};

// MFMA fragments from a stage (sb: its first byte).  A: row fragment i of
// wavefront row wm, 32-deep half h (ds_read_b128: lane -> row i16, k block
// g).  B: column fragment j of wavefront column wn, 8 consecutive k of one
// column per lane (row-major weights: two transposing reads; packed: one
// ds_read_b128).
template <class S>
__device__ __forceinline__ bf16x8 frag_a(const char* sb, int wm, int h, int i, int lane) {
  const int g = lane >> 4, i16 = lane & 15;
  const int m = frag_row<S>(wm, i) + i16;
  return *reinterpret_cast<const bf16x8*>(sb + m * S::A_ROW + a_chunk<S::CA>(m, h * 4 + g) * 16);
}
template <class S, bool SWIGLU, bool BT>
__device__ __forceinline__ bf16x8 frag_b(const char* sb, int wn, int h, int j, int lane) {
  const int g = lane >> 4, i16 = lane & 15;
  if constexpr (BT) {
    // column row n of the packed-weight stage: lane -> column i16, k block g
    const int n = bcol_of<S, SWIGLU>(j, wn) + i16;
    return *reinterpret_cast<const bf16x8*>(sb + S::A_STAGE + n * S::A_ROW +
                                            a_chunk<S::CA>(n, h * 4 + g) * 16);
  }
  const int tq = i16 >> 2, tr = i16 & 3;
  const int k_lo = h * 32 + g * 8 + tq;   // rows of the two transposing reads
  const int k_hi = k_lo + 4;
  const int sg = bcol_of<S, SWIGLU>(j, wn) >> 4;
  const char* blo = sb + S::A_STAGE + k_lo * S::B_ROW + ((sg ^ b_swz(k_lo)) * 32) + tr * 8;
  const char* bhi = sb + S::A_STAGE + k_hi * S::B_ROW + ((sg ^ b_swz(k_hi)) * 32) + tr * 8;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)blo);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)bhi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Stores this wavefront's finished accumulators.  MFMA 16x16 output: lane
// holds rows 4*(lane/16) + r, column lane % 16.  SwiGLU: h = silu(u) * v
// rounded once to bf16, u and v in accumulators j and j + NJ/2, into H
// (row-major or K-blocked).  Plain: fp32 rows of K part kpart.
template <bool SWIGLU, class S>
__device__ __forceinline__ void store_tile(const GroupedGemm& p, const TileCoords& tc,
                                           f32x4 (&acc)[S::MI][S::NJ], int wm, int wn,
                                           int lane, int n0) {
  constexpr int MI = S::MI, NJ = S::NJ;
  const int64_t cgo = static_cast<int64_t>(tc.ngroup) * p.c_group_col;
  if constexpr (SWIGLU) {
    uint16_t* H = static_cast<uint16_t*>(p.C);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = frag_row<S>(wm, i) + (lane >> 4) * 4 + r;
        if (rl >= tc.nrows) continue;
        const int64_t row = tc.row0 + rl;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int col = n0 + wn * (S::WCOLS / 2) + j * 16 + (lane & 15);
          if (col < p.N) {
            const uint16_t h = f32_to_bf16(silu_f32(acc[i][j][r]) * acc[i][j + NJ / 2][r]);
            const int64_t c = cgo + col;
            if (p.c_block_rows > 0)
              H[((c >> 5) * p.c_block_rows + row) * 32 + (c & 31)] = h;
            else
              H[row * p.ldc + c] = h;
          }
        }
      }
    }
  } else {
    float* Y = static_cast<float*>(p.C) + tc.kpart * p.c_split;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = frag_row<S>(wm, i) + (lane >> 4) * 4 + r;
        if (rl >= tc.nrows) continue;
        float* yrow = Y + static_cast<int64_t>(tc.row0 + rl) * p.ldc + cgo;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = n0 + wn * S::WCOLS + j * 16 + (lane & 15);
          if (col < p.N) yrow[col] = acc[i][j][r];
        }
      }
    }
  }
}

// Grid of a grouped GEMM: every logical (M-tile, N-tile, N-group, K part),
// rounded up to whole groups of 8 (one per XCD).
template <typename Kern>
hipError_t launch_grid(Kern kern, const GroupedGemm& g, int ntn, hipStream_t s, int waves = 4) {
  const int64_t tiles = static_cast<int64_t>(g.max_mtiles) * ntn * g.ngroups_n;
  if (tiles <= 0) return hipSuccess;
  // unevenly cut parts: two blocks per tile of each XCD's eighth
  const int nblocks = g.kcut_slots > 0 ? static_cast<int>(16 * ((tiles + 7) / 8))
                                       : static_cast<int>((tiles * g.ksplit + 7) / 8 * 8);
  kern<<<nblocks, 64 * waves, 0, s>>>(g, ntn, nblocks);
  return hipGetLastError();
}

}  // namespace dma
}  // namespace
}  // namespace moe
