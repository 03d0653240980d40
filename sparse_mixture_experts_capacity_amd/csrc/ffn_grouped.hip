// Grouped expert GEMMs for libmoe (gfx950).
//
// The expert FFN is the layer's only dense contraction: per expert e with
// kept rows X_e, H_e = silu(X_e W1[e]) * (X_e W3[e]) and Y_e = H_e W2[e]
// ([Mixtral explainer] "Mixtral 8x7B and MoE explained" (allinfo.ai.kr),
// "Plain explanation" para 2: the feed-forward widens each token to the
// hidden size and back; para 4: experts that were not chosen are not
// computed at all).  One launch runs every (M-tile, N-tile) of every expert;
// M-tiles come from a device-side tile list, so the host never reads the
// routing back.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with fp32 accumulators in VGPRs.  Both
// operands go from global memory straight into LDS with global_load_lds_dwordx4
// (no staging registers, no LDS store instructions) through a ring of NS
// K-steps, NS - 1 of them in flight while the current one is multiplied.
// Token rows are gathered through the dispatch permutation as 16-byte chunks.
// Weights stay in LDS as stored, [K][N] with N contiguous; the B fragments
// (8 consecutive k of one column per lane) are read with ds_read_b64_tr_b16,
// which transposes 4 x 4 blocks of 16-bit values across each 16-lane group.
// Both tiles use XOR swizzles instead of padding so the DMA rows stay dense
// and the fragment reads are free of bank conflicts.  The weights may be
// row-major or packed in 32-row blocks (then a tile's K step reads whole
// contiguous runs); only the source addresses differ.  Tile shapes (the
// list near the end of the dma namespace):
//   32 x 256 or 32 x 128, K step 64, 4 wavefronts, 4 stages: short batches
//     (decode), where the weights stream once and K may be split over
//     several workgroups;
//   128 x 256, K step 32, 8 wavefronts, 3 stages, 72 KB: two workgroups per
//     CU, for experts with hundreds to ~1500 rows (prefill);
//   256 x 256, K step 32, 8 wavefronts, 4 stages, 128 KB: one workgroup per
//     CU, for a few hundred rows per expert or for thousands.
// On an expert's last, short M-tile the 16-row fragments past its end are
// neither read nor multiplied.
//
// SwiGLU epilogue: a tile's 256 B columns are 128 W1 columns followed by the
// same 128 W3 columns, and each wavefront owns matching halves, so u and v of
// one output element sit in the same lane and register: h = silu(u) * v is
// rounded once to bf16.
//
// The XCD-aware block order keeps consecutive logical tiles on one XCD; the
// logical order runs M-tiles fastest, so the M-tiles sharing a weight tile
// run together on one XCD and read it from HBM once.
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
  const int ks = p.ksplit;
  const int total = mtiles * ntn_all * ks;
  const int per = (total + 7) >> 3;
  const int x = blockIdx.x & 7;
  const int i = blockIdx.x >> 3;
  if (i >= per) return tc;
  const int LK = x * per + i;
  if (LK >= total) return tc;
  tc.kpart = LK % ks;   // K parts of one tile are adjacent: they share A rows
  const int L = LK / ks;
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

// ===========================================================================
// bf16 MFMA kernel, gfx950 data path
//
// Global -> LDS with global_load_lds_dwordx4 (the load unit writes LDS
// directly: no staging registers, no LDS write instructions) into an
// NS-deep ring of stages, so NS-1 K steps of loads are in flight while one is
// computed.  The weight tile stays N-contiguous in LDS, exactly as it sits in
// memory, and the MFMA B fragments are read with ds_read_b64_tr_b16, which
// transposes 16-bit elements across each 16-lane group: source lane 4q+r
// supplies columns 4r..4r+3 of row k_q, and result lane i receives column i
// of rows k_0..k_3.  Two such reads give a lane the 8 consecutive k values of
// one column that v_mfma_f32_16x16x32_bf16 takes.
//
// LDS layouts (no padding; XOR swizzles keep every read conflict-free):
//   A stage: BM rows x 2*BK bytes; 16-byte chunk c of row m is stored at
//            a_chunk(m, c) (an XOR of c with low bits of m).
//   B stage: BK rows x 2*BN bytes; 32-byte segment s (16 columns) of row k
//            sits at segment s ^ ((k & 3) | ((k >> 1) & 4)).
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

// Stored position of 16-byte chunk c of A row m.  With 8 chunks per row
// (BK = 64): c ^ (m & 7) ^ ((m >> 3) & 1); with 4 (BK = 32):
// c ^ (m & 3) ^ ((m >> 2) & 3).  Either way 16 consecutive rows read at one
// chunk hit 16 different 16-byte bank groups.
template <int CA>
__device__ __forceinline__ int a_chunk(int m, int c) {
  if constexpr (CA == 8) return c ^ (m & 7) ^ ((m >> 3) & 1);
  return c ^ (m & 3) ^ ((m >> 2) & 3);
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

template <bool SWIGLU, class S>
// The second launch bound is the minimum wavefronts per SIMD: BLOCKS_PER_CU
// workgroups of NW wavefronts over 4 SIMDs, which caps the registers.
__global__ __launch_bounds__(64 * S::NW, S::BLOCKS_PER_CU * S::NW / 4) void grouped_bf16_dma_kernel(
    GroupedGemm p, int ntn, int nblocks) {
  constexpr int BM = S::BM, BN = S::BN, BK = S::BK, NS = S::NS, MI = S::MI, NJ = S::NJ;
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];

  const TileCoords tc = tile_coords<BM>(p, ntn, nblocks);
  if (!tc.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / S::WN;
  const int wn = wave % S::WN;
  const int e = p.group_base + tc.group + tc.ngroup;
  const int64_t boff = static_cast<int64_t>(e) * p.b_stride;
  constexpr int NOUT = SWIGLU ? BN / 2 : BN;
  const int n0 = tc.ntile * NOUT;

  // ---- DMA sources ---------------------------------------------------------
  // A: load i of this wavefront fills rows (wave*A_LOADS + i)*A_ROWS_PER_LOAD
  // onward; lane -> row + lane/CA, stored chunk lane%CA.  Rows past the
  // tile's end repeat its first row (their results are not stored).  In the
  // K-blocked layout (a_block_rows = R > 0) element (row, k) sits at
  // ((k / 32) * R + row) * 32 + k % 32, so one K step of a tile's rows is a
  // contiguous run of memory.
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const uint16_t* asrc[S::A_LOADS];
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
  // element offset of K step k0 along A (a multiple of 32)
  const int64_t a_kstride = p.a_block_rows > 0 ? p.a_block_rows : 1;
  // B: load i fills rows (wave*B_LOADS + i)*B_ROWS_PER_LOAD onward; lane ->
  // row + lane/(BN/8), stored 16-byte chunk q = lane%(BN/8), which is half
  // (q&1) of stored segment q/2.  Columns past N read column 0 (their
  // outputs are never stored).  With packed weights a step's rows of one
  // tile are whole 32-row blocks: one contiguous run per block instead of a
  // short piece of every row.  Either way the step advances by K-step x ldb.
  constexpr int BCH = BN / 8;                 // 16-byte chunks per B row
  const uint16_t* bsrc[S::B_LOADS];
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

  // LDS byte address of this wavefront's destinations in stage 0
  // (wave-uniform: M0 takes it).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  // This block's share of K: part kpart of ksplit near-equal runs of BK steps.
  const int nk_all = p.K / BK;
  const int kb0 = static_cast<int>(static_cast<int64_t>(tc.kpart) * nk_all / p.ksplit);
  const int kb1 = static_cast<int>(static_cast<int64_t>(tc.kpart + 1) * nk_all / p.ksplit);
  const int kbase = kb0 * BK;
  // step: K step to load; stage: its ring slot (step % NS).
  auto issue = [&](int step, int stage) __attribute__((always_inline)) {
    const uint32_t sb = lds0 + stage * S::STAGE;
    const int k0 = kbase + step * BK;
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i)
      dma16(asrc[i] + k0 * a_kstride, sb + (wave_u * S::A_LOADS + i) * 1024);
    const int64_t kb = static_cast<int64_t>(k0) * p.ldb;
#pragma unroll
    for (int i = 0; i < S::B_LOADS; ++i)
      dma16(bsrc[i] + kb, sb + S::A_STAGE + (wave_u * S::B_LOADS + i) * 1024);
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragment addressing (bytes within a stage).
  const int g = lane >> 4;         // k block of 8 within a 32-k MFMA step
  const int i16 = lane & 15;
  const int tq = i16 >> 2, tr = i16 & 3;

  // One 32-deep half of a stage for this wavefront: MI A fragments
  // (ds_read_b128) and NJ B fragments (two transposing reads each).
  struct Frags {
    bf16x8 a[MI];
    bf16x8 b[NJ];
  };
  auto rd_a = [&](int stage, int h, int i) __attribute__((always_inline)) -> bf16x8 {
    const char* sb = smem + stage * S::STAGE;
    const int m = frag_row<S>(wm, i) + i16;
    return *reinterpret_cast<const bf16x8*>(sb + m * S::A_ROW + a_chunk<S::CA>(m, h * 4 + g) * 16);
  };
  auto rd_b = [&](int stage, int h, int j) __attribute__((always_inline)) -> bf16x8 {
    const char* sb = smem + stage * S::STAGE;
    const int k_lo = h * 32 + g * 8 + tq;   // rows of the two transposing reads
    const int k_hi = k_lo + 4;
    const int sg = bcol_of<S, SWIGLU>(j, wn) >> 4;
    const char* blo = sb + S::A_STAGE + k_lo * S::B_ROW + ((sg ^ b_swz(k_lo)) * 32) + tr * 8;
    const char* bhi = sb + S::A_STAGE + k_hi * S::B_ROW + ((sg ^ b_swz(k_hi)) * 32) + tr * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)blo);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)bhi);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // MV: row fragments of this wavefront that hold tile rows (a constant of
  // the specialised pipeline below); the others are neither read nor
  // multiplied.
  auto load_frags = [&](Frags& f, int stage, int h, auto mv_c) __attribute__((always_inline)) {
    constexpr int MV = decltype(mv_c)::value;
#pragma unroll
    for (int i = 0; i < MV; ++i) f.a[i] = rd_a(stage, h, i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b[j] = rd_b(stage, h, j);
  };
  // The MFMAs of the fragments in f, column by column.  When `more`, the
  // fragments of the next 32-deep half (ring slot nstage, half nh) are read
  // into the same registers as they fall free: each B fragment after its
  // column, the A fragments during the last column.  So the next half's
  // reads overlap this half's MFMAs and no extra registers are held.
  auto mfma_reload = [&](Frags& f, int nstage, int nh, bool more, auto mv_c)
                         __attribute__((always_inline)) {
    constexpr int MV = decltype(mv_c)::value;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j < NJ - 1) {
#pragma unroll
        for (int i = 0; i < MV; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (more) f.b[j] = rd_b(nstage, nh, j);
        __builtin_amdgcn_sched_barrier(0);
      } else {
#pragma unroll
        for (int i = 0; i < MV; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (more) f.a[i] = rd_a(nstage, nh, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (more) f.b[j] = rd_b(nstage, nh, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- pipeline --------------------------------------------------------------
  // NS ring slots of K steps.  The wavefront always holds in registers the
  // fragments of the 32-deep half it multiplies next, read while the previous
  // half's MFMAs ran.  Before the last half of step ks, once this thread's
  // transfers of step ks+1 have landed and its reads of step ks are done, a
  // barrier makes step ks+1 readable by all (its fragments are read during
  // that half) and frees step ks's slot, which is refilled with step ks+NS.
  // The pipeline is specialised on MV, the number of this wavefront's row
  // fragments that hold tile rows: on an expert's last, short M-tile the
  // fragments past the end are neither read nor multiplied, and a wavefront
  // with none keeps loading and meeting the barriers only.
  const int nk = kb1 - kb0;
  const int nfr = min((tc.nrows + 15) >> 4, BM / 16);   // >= 1
  const int mv = min(MI, (nfr - __builtin_amdgcn_readfirstlane(wm) + S::WM - 1) / S::WM);
  auto run = [&](auto mv_c) __attribute__((always_inline)) {
    constexpr int MV = decltype(mv_c)::value;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      if (st < nk) issue(st, st);
    Frags f;
    if (nk > 0) {
      wait_stages_lgkm0<S::LOADS>(min(NS - 1, nk - 1));
      // A bare barrier: __syncthreads() adds a release fence that would wait
      // for every transfer in flight, the later stages' included.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MV > 0) load_frags(f, 0, 0, mv_c);
      __builtin_amdgcn_sched_barrier(0);
    }
    // One K step held in ring slot `stage` (a constant in the unrolled loop
    // below, so every LDS address of the step is a fixed offset).  HAS_NEXT:
    // a step ks+1 follows (every step but the last), so its stage is waited
    // for, the slot of step ks is refilled, and its fragments are read ahead.
    auto step_body = [&](int ks, int stage, auto has_next_c) __attribute__((always_inline)) {
      constexpr bool HAS_NEXT = decltype(has_next_c)::value;
      const int next_slot = stage == NS - 1 ? 0 : stage + 1;
#pragma unroll
      for (int h = 0; h < S::HALVES; ++h) {
        if (HAS_NEXT && h == S::HALVES - 1) {
          wait_stages_lgkm0<S::LOADS>(min(NS - 2, nk - ks - 2));
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if (ks + NS < nk) issue(ks + NS, stage);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MV > 0) {
          if (h + 1 < S::HALVES) mfma_reload(f, stage, h + 1, true, mv_c);
          else mfma_reload(f, next_slot, 0, HAS_NEXT, mv_c);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    int ks = 0;
    // steps 0 .. nk-2 (each followed by another), NS at a time, then the last
    for (; ks + NS <= nk - 1; ks += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) step_body(ks + u, u, yes{});
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (ks + u < nk - 1) step_body(ks + u, u, yes{});
    if (nk > 0) step_body(nk - 1, (nk - 1) % NS, no{});
  };
  with_count<MI>(mv, run);

  // ---- epilogue -----------------------------------------------------------
  // MFMA 16x16 output: lane holds rows 4*(lane/16) + r, column lane % 16.
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

// Shapes in use (the M-tile the host chooses picks one):
//   0: 32-row M-tiles for short batches; 4-stage ring, one workgroup per CU;
//      with narrow_n, 128-wide B tiles (80 KB, two workgroups per CU): twice
//      the tiles, so the weights of several hit experts stream from more CUs.
//   1: 128 x 256 x 32, 8 wavefronts, 3 stages (72 KB): two workgroups per CU
//      (4 wavefronts per SIMD); best when experts have many rows.
//   2: 256 x 256 x 32, 8 wavefronts (4 x 2) of 64 x 128, 4 stages (128 KB):
//      one workgroup per CU.  For a few hundred rows per expert (fine-grained
//      experts, where the weights' HBM traffic is the bound): one M-tile per
//      expert reads each weight tile once, and on an expert's short tile the
//      16-row fragments past its end are skipped.
using ShapeShort = Shape<32, 256, 64, 4, 1, 4>;
using ShapeShortN = Shape<32, 128, 64, 4, 1, 4>;
using ShapeLongA = Shape<128, 256, 32, 8, 2, 3>;
using ShapeWide = Shape<256, 256, 32, 8, 4, 4>;

}  // namespace dma

// ===========================================================================
// fp32 kernel (the fp32 layer): 64 x 64 output tiles, K step 16, each thread
// a 4 x 4 block (of u and v for SwiGLU).  Plain FMA in fp32.
// ===========================================================================
constexpr int FBM = kF32BM;  // 64
constexpr int FBN = 64;
constexpr int FBK = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_f32_kernel(GroupedGemm p, int ntn,
                                                          int nblocks) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN];
  __shared__ float B3s[SWIGLU ? FBK : 1][SWIGLU ? FBN : 1];
  const TileCoords tc = tile_coords<FBM>(p, ntn, nblocks);
  if (!tc.valid) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int e = p.group_base + tc.group + tc.ngroup;
  const int64_t boff = static_cast<int64_t>(e) * p.b_stride;
  const int n0 = tc.ntile * FBN;
  const float* A = static_cast<const float*>(p.A);
  const float* B = static_cast<const float*>(p.B) + boff;
  const float* B3 = SWIGLU ? static_cast<const float*>(p.B3) + boff : nullptr;

  // A loader: thread loads rows (tid/16) + 16 i, column tid%16 of the K step.
  int64_t arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 4) + 16 * i;
    const int rr = tc.row0 + (r < tc.nrows ? r : 0);
    arow[i] = (p.perm ? static_cast<int64_t>(p.perm[rr] / p.topk) : rr) * p.lda;
  }
  float acc[4][4], acc3[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc3[i][j] = 0.f;

  for (int k0 = 0; k0 < p.K; k0 += FBK) {
    const int kk = tid & 15;
    const bool kin = k0 + kk < p.K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      As[kk][r] = kin ? A[arow[i] + k0 + kk] : 0.f;
    }
    // B loader: 16 x 64 = 1024 values, 4 per thread.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int kr = idx >> 6, c = idx & 63;
      const bool in = (k0 + kr < p.K) && (n0 + c < p.N);
      const int64_t off = static_cast<int64_t>(k0 + kr) * p.ldb + n0 + c;
      Bs[kr][c] = in ? B[off] : 0.f;
      if constexpr (SWIGLU) B3s[kr][c] = in ? B3[off] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk2 = 0; kk2 < FBK; ++kk2) {
      float a[4], b[4], b3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk2][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = Bs[kk2][tx * 4 + j];
        if constexpr (SWIGLU) b3[j] = B3s[kk2][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if constexpr (SWIGLU) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }
  const int64_t cgo = static_cast<int64_t>(tc.ngroup) * p.c_group_col;
  float* C = static_cast<float*>(p.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = ty * 4 + i;
    if (rl >= tc.nrows) continue;
    float* crow = C + static_cast<int64_t>(tc.row0 + rl) * p.ldc + cgo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < p.N)
        if constexpr (SWIGLU) {
          crow[col] = silu_f32_accurate(acc[i][j]) * acc3[i][j];
        } else {
          crow[col] = acc[i][j];
        }
    }
  }
}

// Token rows of the kept assignments, in slot order and K-blocked:
// Xb[((k / 32) * R + s) * 32 + k % 32] = x[perm[s] / topk][k] for slots
// s < offsets[E].  Each thread moves 16 bytes; consecutive threads write
// consecutive memory.
__global__ __launch_bounds__(256) void gather_blocked_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ perm, int topk,
    const int32_t* __restrict__ nrows_dev, int64_t R, int d, uint16_t* __restrict__ Xb) {
  const int64_t n = R * (d / 8);
  const int64_t total = *nrows_dev;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t kb = t / (R * 4);
    const int64_t rem = t - kb * R * 4;
    const int64_t sl = rem >> 2;
    const int c = static_cast<int>(rem & 3);
    if (sl >= total) continue;
    const int64_t tok = perm[sl] / topk;
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + tok * ldx + kb * 32 + c * 8);
    *reinterpret_cast<u32x4*>(Xb + (kb * R + sl) * 32 + c * 8) = v;
  }
}

// Packed weights: output element o (8 at a time, consecutive threads on
// consecutive 16 bytes) of expert e is element (k, n) of its row-major
// [K, N] matrix, or 0 past column N.
__global__ __launch_bounds__(256) void pack_blocks_kernel(const uint16_t* __restrict__ src,
                                                          int64_t nexp, int K, int N, int W,
                                                          int Npad, uint16_t* __restrict__ dst) {
  const int64_t per = static_cast<int64_t>(K) * Npad;
  const int64_t n8 = nexp * per / 8;
  const int nbw = Npad / W;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n8;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t o = t * 8;
    const int64_t e = o / per;
    const int64_t rem = o - e * per;
    const int64_t blk = rem / (32 * W);
    const int within = static_cast<int>(rem - blk * 32 * W);
    const int k = static_cast<int>(blk / nbw) * 32 + within / W;
    const int n = static_cast<int>(blk % nbw) * W + within % W;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N) v = *reinterpret_cast<const u32x4*>(src + (e * K + k) * static_cast<int64_t>(N) + n);
    *reinterpret_cast<u32x4*>(dst + o) = v;
  }
}

template <typename Kern>
hipError_t launch_grid(Kern kern, const GroupedGemm& g, int ntn, hipStream_t s, int waves = 4) {
  const int64_t logical = static_cast<int64_t>(g.max_mtiles) * ntn * g.ngroups_n * g.ksplit;
  if (logical <= 0) return hipSuccess;
  const int nblocks = static_cast<int>((logical + 7) / 8 * 8);
  kern<<<nblocks, 64 * waves, 0, s>>>(g, ntn, nblocks);
  return hipGetLastError();
}

}  // namespace

template <bool SWIGLU, class S>
hipError_t launch_bf16_shape(const GroupedGemm& g, hipStream_t s) {
  const int cols = SWIGLU ? S::BN / 2 : S::BN;
  return launch_grid(dma::grouped_bf16_dma_kernel<SWIGLU, S>, g, (g.N + cols - 1) / cols, s, S::NW);
}
template <bool SWIGLU>
hipError_t launch_bf16(const GroupedGemm& g, hipStream_t s) {
  if (g.bm == kGroupedBMShort) {
    if (g.narrow_n) return launch_bf16_shape<SWIGLU, dma::ShapeShortN>(g, s);
    return launch_bf16_shape<SWIGLU, dma::ShapeShort>(g, s);
  }
  if (g.bm == kGroupedBMWide) return launch_bf16_shape<SWIGLU, dma::ShapeWide>(g, s);
  return launch_bf16_shape<SWIGLU, dma::ShapeLongA>(g, s);
}
hipError_t launch_pack_blocks(const void* src, int64_t nexp, int K, int N, int W, void* dst,
                              hipStream_t s) {
  const int Npad = (N + W - 1) / W * W;
  const int64_t n8 = nexp * K * static_cast<int64_t>(Npad) / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 256 * 64);
  pack_blocks_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(
      static_cast<const uint16_t*>(src), nexp, K, N, W, Npad, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}
hipError_t launch_gather_blocked(const void* x, int64_t ldx, const int32_t* perm, int topk,
                                 const int32_t* nrows_dev, int64_t R, int d, void* Xb,
                                 hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const int64_t n = R * (d / 8);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 32);
  gather_blocked_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(
      static_cast<const uint16_t*>(x), ldx, perm, topk, nrows_dev, R, d,
      static_cast<uint16_t*>(Xb));
  return hipGetLastError();
}
hipError_t launch_grouped_swiglu_bf16(const GroupedGemm& g, hipStream_t s) {
  return launch_bf16<true>(g, s);
}
hipError_t launch_grouped_plain_bf16(const GroupedGemm& g, hipStream_t s) {
  return launch_bf16<false>(g, s);
}
hipError_t launch_grouped_swiglu_f32(const GroupedGemm& g, hipStream_t s) {
  return launch_grid(grouped_f32_kernel<true>, g, (g.N + FBN - 1) / FBN, s);
}
hipError_t launch_grouped_plain_f32(const GroupedGemm& g, hipStream_t s) {
  return launch_grid(grouped_f32_kernel<false>, g, (g.N + FBN - 1) / FBN, s);
}

}  // namespace moe
