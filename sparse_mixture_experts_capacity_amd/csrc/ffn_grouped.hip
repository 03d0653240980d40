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
#include "ffn_dma.h"

namespace moe {
namespace {
namespace dma {

template <bool SWIGLU, class S, bool BT>
// BT: packed weights (B stage in column rows, see TileSources).
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
  TileSources<SWIGLU, S, BT> src;
  src.init(p, tc, wave, lane, n0, boff);

  // LDS byte address of this wavefront's destinations in stage 0
  // (wave-uniform: M0 takes it).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  // This block's share of K: part kpart of ksplit near-equal runs of BK
  // steps, or of two parts cut at kcut_steps.
  const int nk_all = p.K / BK;
  int kb0 = static_cast<int>(static_cast<int64_t>(tc.kpart) * nk_all / p.ksplit);
  int kb1 = static_cast<int>(static_cast<int64_t>(tc.kpart + 1) * nk_all / p.ksplit);
  if (p.kcut_slots > 0) {
    const int cut = kcut_steps(nk_all, *p.ntiles * ntn * p.ngroups_n, p.kcut_slots);
    kb0 = tc.kpart ? cut : 0;
    kb1 = tc.kpart ? nk_all : cut;
  }
  const int kbase = kb0 * BK;
  // step: K step to load; stage: its ring slot (step % NS).
  auto issue = [&](int step, int stage) __attribute__((always_inline)) {
    src.issue(lds0 + stage * S::STAGE, kbase + step * BK, wave_u);
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 32-deep half of a stage for this wavefront: MI A fragments
  // (ds_read_b128) and NJ B fragments (two transposing reads each).
  struct Frags {
    bf16x8 a[MI];
    bf16x8 b[NJ];
  };
  auto rd_a = [&](int stage, int h, int i) __attribute__((always_inline)) -> bf16x8 {
    return frag_a<S>(smem + stage * S::STAGE, wm, h, i, lane);
  };
  auto rd_b = [&](int stage, int h, int j) __attribute__((always_inline)) -> bf16x8 {
    return frag_b<S, SWIGLU, BT>(smem + stage * S::STAGE, wn, h, j, lane);
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
  // With one workgroup per CU (kSpread) a step's transfers are not issued
  // in one burst after the barrier but spread over the MFMA columns: with
  // `dma`, transfer j of the later K step (stage address dsb, first element
  // dk0) follows column j's MFMAs, and the rest follow the last column.
  // (Measured: the skew layer's 256 x 256 GEMM1 4% faster, DeepSeek's 1.5%;
  // with two workgroups per CU the other one fills the gap and the burst is
  // as fast.)
  constexpr bool kSpread = S::BLOCKS_PER_CU == 1;
  auto dma_at = [&](auto idx_c, bool dma, uint32_t dsb, int dk0) __attribute__((always_inline)) {
    constexpr int IDX = decltype(idx_c)::value;
    if (dma) src.template issue_one<IDX>(dsb, dk0, wave_u);
  };
  auto mfma_reload = [&](Frags& f, int nstage, int nh, bool more, auto mv_c, bool dma,
                         uint32_t dsb, int dk0) __attribute__((always_inline)) {
    constexpr int MV = decltype(mv_c)::value;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j < NJ - 1) {
#pragma unroll
        for (int i = 0; i < MV; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (more) f.b[j] = rd_b(nstage, nh, j);
        if (j == 0) dma_at(std::integral_constant<int, 0>{}, dma, dsb, dk0);
        if (j == 1) dma_at(std::integral_constant<int, 1>{}, dma, dsb, dk0);
        if (j == 2) dma_at(std::integral_constant<int, 2>{}, dma, dsb, dk0);
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
        // the transfers not issued after an earlier column
        if (NJ - 1 <= 0) dma_at(std::integral_constant<int, 0>{}, dma, dsb, dk0);
        if (NJ - 1 <= 1) dma_at(std::integral_constant<int, 1>{}, dma, dsb, dk0);
        if (NJ - 1 <= 2) dma_at(std::integral_constant<int, 2>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 3>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 4>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 5>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 6>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 7>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 8>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 9>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 10>{}, dma, dsb, dk0);
        dma_at(std::integral_constant<int, 11>{}, dma, dsb, dk0);
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
        // the transfers of step ks + NS into the freed slot: all at once, or
        // (kSpread) one after each MFMA column of the half that follows
        bool dma = false;
        if (HAS_NEXT && h == S::HALVES - 1) {
          wait_stages_lgkm0<S::LOADS>(min(NS - 2, nk - ks - 2));
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          const bool more_k = ks + NS < nk;
          if (kSpread && MV > 0) dma = more_k;
          else if (more_k) issue(ks + NS, stage);
          __builtin_amdgcn_sched_barrier(0);
        }
        const uint32_t dsb = lds0 + stage * S::STAGE;
        const int dk0 = kbase + (ks + NS) * BK;
        if constexpr (MV > 0) {
          if (h + 1 < S::HALVES) mfma_reload(f, stage, h + 1, true, mv_c, dma, dsb, dk0);
          else mfma_reload(f, next_slot, 0, HAS_NEXT, mv_c, dma, dsb, dk0);
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
  store_tile<SWIGLU, S>(p, tc, acc, wm, wn, lane, n0);
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
//      16-row fragments past its end are skipped.  Also for thousands of rows
//      per expert.  With packed weights the same M-tile is run by 16
//      wavefronts (4 x 4) of 64 x 64 over 3 stages (96 KB): with the packed
//      B path the 8-wavefront form spills registers at 4 stages, and the
//      16-wavefront form measured 0.2-0.3% faster than it at 3.
using ShapeShort = Shape<32, 256, 64, 4, 1, 4>;
using ShapeShortN = Shape<32, 128, 64, 4, 1, 4>;
using ShapeLongA = Shape<128, 256, 32, 8, 2, 3>;
using ShapeWide = Shape<256, 256, 32, 8, 4, 4>;
using ShapeWidePacked = Shape<256, 256, 32, 16, 4, 3>;

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

// Packed weights: output elements o..o+7 (consecutive threads on consecutive
// 16 bytes) of expert e are elements (k..k+7, n) of its row-major [K, N]
// matrix, or 0 past column N: each 32 x W block is stored column by column.
// A one-off copy, so the 8 reads along a column are plain 2-byte loads.
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
    const int k = static_cast<int>(blk / nbw) * 32 + (within & 31);
    const int n = static_cast<int>(blk % nbw) * W + (within >> 5);
    uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (n < N) {
      const uint16_t* col = src + (e * K + k) * static_cast<int64_t>(N) + n;
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = col[static_cast<int64_t>(q) * N];
    }
    u32x4 w4;
#pragma unroll
    for (int q = 0; q < 4; ++q) w4[q] = static_cast<uint32_t>(v[2 * q]) | (static_cast<uint32_t>(v[2 * q + 1]) << 16);
    *reinterpret_cast<u32x4*>(dst + o) = w4;
  }
}

}  // namespace

template <bool SWIGLU, class S, bool BT>
hipError_t launch_bf16_shape(const GroupedGemm& g, hipStream_t s) {
  const int cols = SWIGLU ? S::BN / 2 : S::BN;
  return dma::launch_grid(dma::grouped_bf16_dma_kernel<SWIGLU, S, BT>, g, (g.N + cols - 1) / cols, s,
                          S::NW);
}
template <bool SWIGLU, bool BT>
hipError_t launch_bf16_layout(const GroupedGemm& g, hipStream_t s) {
  if (g.bm == kGroupedBMShort) {
    if (g.narrow_n) return launch_bf16_shape<SWIGLU, dma::ShapeShortN, BT>(g, s);
    return launch_bf16_shape<SWIGLU, dma::ShapeShort, BT>(g, s);
  }
  if (g.bm == kGroupedBMWide) {
    if constexpr (BT) return launch_bf16_shape<SWIGLU, dma::ShapeWidePacked, BT>(g, s);
    else return launch_bf16_shape<SWIGLU, dma::ShapeWide, BT>(g, s);
  }
  return launch_bf16_shape<SWIGLU, dma::ShapeLongA, BT>(g, s);
}
template <bool SWIGLU>
hipError_t launch_bf16(const GroupedGemm& g, hipStream_t s) {
  if (g.b_block_cols > 0) return launch_bf16_layout<SWIGLU, true>(g, s);
  return launch_bf16_layout<SWIGLU, false>(g, s);
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
  return dma::launch_grid(grouped_f32_kernel<true>, g, (g.N + FBN - 1) / FBN, s);
}
hipError_t launch_grouped_plain_f32(const GroupedGemm& g, hipStream_t s) {
  return dma::launch_grid(grouped_f32_kernel<false>, g, (g.N + FBN - 1) / FBN, s);
}

}  // namespace moe
