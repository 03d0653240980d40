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
// bf16 path: v_mfma_f32_16x16x32_bf16 on 128 x 256 workgroup tiles, K step 64,
// 4 wavefronts (2 x 2), each a 64 x 128 sub-tile (4 x 8 MFMA tiles, fp32
// accumulators).  Weights are stored [K, N] with N contiguous, while the MFMA
// B operand wants 8 consecutive k per lane; each thread therefore loads an
// 8 (k) x 8 (n) block with 16-byte loads and transposes it in registers before
// writing k-contiguous rows to LDS.  Token rows are gathered through the
// dispatch permutation as 16-byte chunks.  LDS is double buffered and the
// next K step is prefetched into registers while the MFMAs run.
//
// SwiGLU epilogue: a tile's 256 B columns are 128 W1 columns followed by the
// same 128 W3 columns, and each wavefront owns matching halves, so u and v of
// one output element sit in the same lane and register: h = silu(u) * v is
// rounded once to bf16.
//
// The XCD-aware block order keeps consecutive logical tiles on one XCD; the
// logical order runs M-tiles fastest, so the M-tiles sharing a weight tile
// run together on one XCD and read it from HBM once.
#include "kernels.h"

namespace moe {
namespace {

struct TileCoords {
  int group;   // expert index relative to group_base (routed) or 0
  int row0;
  int nrows;
  int ntile;   // N-tile within the group
  int ngroup;  // N-group (shared experts laid along N)
  bool valid;
};

template <int TBM>
__device__ __forceinline__ TileCoords tile_coords(const GroupedGemm& p, int ntn,
                                                  int nblocks) {
  TileCoords tc{0, 0, 0, 0, 0, false};
  const int L = xcd_local_block(blockIdx.x, nblocks);
  const int mt = L % p.max_mtiles;
  const int nt_all = L / p.max_mtiles;
  if (nt_all >= ntn * p.ngroups_n) return tc;
  tc.ngroup = nt_all / ntn;
  tc.ntile = nt_all % ntn;
  if (p.tiles) {
    if (mt >= *p.ntiles) return tc;
    const Tile t = p.tiles[mt];
    tc.group = t.group;
    tc.row0 = t.row0;
    tc.nrows = t.nrows;
  } else {
    tc.row0 = mt * TBM;
    if (tc.row0 >= p.static_rows) return tc;
    tc.nrows = min(TBM, p.static_rows - tc.row0);
  }
  tc.valid = tc.nrows > 0;
  return tc;
}

// ===========================================================================
// bf16 MFMA kernel
// ===========================================================================
constexpr int BM = kGroupedBM;  // 128
constexpr int BN = 256;         // B-tile columns (SwiGLU: 128 W1 + 128 W3)
constexpr int BK = 64;
constexpr int LDK = BK + 8;     // padded LDS row (144 bytes, conflict-free)

// 8 (k) x 8 (n) bf16 block transpose: in[r] holds row r (n = 0..7, two per
// dword), out[c] holds column c (k = 0..7, two per dword).
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* r = reinterpret_cast<const uint32_t*>(in);
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = r[(2 * q) * 4 + (c >> 1)];
      const uint32_t b = r[(2 * q + 1) * 4 + (c >> 1)];
      o[c * 4 + q] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u))
                             : ((a & 0xffffu) | (b << 16));
    }
  }
}

template <bool SWIGLU>
__global__ __launch_bounds__(256, 1) void grouped_bf16_kernel(GroupedGemm p, int ntn,
                                                              int nblocks) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

  const TileCoords tc = tile_coords<BM>(p, ntn, nblocks);
  if (!tc.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int e = p.group_base + tc.group + tc.ngroup;
  const int64_t boff = static_cast<int64_t>(e) * p.b_stride;
  constexpr int NOUT = SWIGLU ? BN / 2 : BN;   // output columns per tile
  const int n0 = tc.ntile * NOUT;

  // ---- A loader: 4 chunks of 8 bf16 per thread (rows tid/8 + 32 i) --------
  const uint16_t* A = static_cast<const uint16_t*>(p.A);
  const int akc = tid & 7;
  const uint16_t* aptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int rr = tc.row0 + (r < tc.nrows ? r : 0);
    const int64_t src = p.perm ? static_cast<int64_t>(p.perm[rr] / p.topk) : rr;
    aptr[i] = A + src * p.lda + akc * 8;
  }
  // ---- B loader: one 8 x 8 block per thread --------------------------------
  const int kb = tid & 7;    // k rows kb*8 .. kb*8+7
  const int nb = tid >> 3;   // B-tile columns nb*8 .. nb*8+7
  const uint16_t* bsrc;
  int bcol;
  if constexpr (SWIGLU) {
    bsrc = static_cast<const uint16_t*>(nb < 16 ? p.B : p.B3);
    bcol = n0 + (nb & 15) * 8;
  } else {
    bsrc = static_cast<const uint16_t*>(p.B);
    bcol = n0 + nb * 8;
  }
  const bool bvalid = bcol < p.N;
  const uint16_t* bptr = bsrc + boff + static_cast<int64_t>(kb * 8) * p.ldb + (bvalid ? bcol : 0);

  uint4 ra[4];
  uint4 rb[8];
  auto load_regs = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(aptr[i] + k0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (bvalid)
        rb[r] = *reinterpret_cast<const uint4*>(bptr + static_cast<int64_t>(k0 + r) * p.ldb);
      else
        rb[r] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(&As[buf][r * LDK + akc * 8]) = ra[i];
    }
    uint4 col[8];
    transpose8x8(rb, col);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<uint4*>(&Bs[buf][(nb * 8 + c) * LDK + kb * 8]) = col[c];
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B-tile column of MFMA tile j owned by this wavefront.
  auto bcol_of = [&](int j) -> int {
    if constexpr (SWIGLU) return (j < 4) ? (wn * 64 + j * 16) : (128 + wn * 64 + (j - 4) * 16);
    return wn * 128 + j * 16;
  };

  const int nk = p.K / BK;
  load_regs(0);
  store_lds(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) load_regs((ks + 1) * BK);
    const uint16_t* as = As[cur];
    const uint16_t* bs = Bs[cur];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int koff = s * 32 + (lane >> 4) * 8;
      bf16x8 af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&as[(wm * 64 + i * 16 + (lane & 15)) * LDK + koff]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 bf =
            *reinterpret_cast<const bf16x8*>(&bs[(bcol_of(j) + (lane & 15)) * LDK + koff]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf, acc[i][j], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue -----------------------------------------------------------
  // MFMA 16x16 output: lane holds rows 4*(lane/16) + r, column lane % 16.
  const int64_t cgo = static_cast<int64_t>(tc.ngroup) * p.c_group_col;
  if constexpr (SWIGLU) {
    uint16_t* H = static_cast<uint16_t*>(p.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (rl >= tc.nrows) continue;
        uint16_t* hrow = H + static_cast<int64_t>(tc.row0 + rl) * p.ldc + cgo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + (lane & 15);
          if (col < p.N) {
            const float u = acc[i][j][r];
            const float v = acc[i][j + 4][r];
            hrow[col] = f32_to_bf16(silu_f32(u) * v);
          }
        }
      }
    }
  } else {
    float* Y = static_cast<float*>(p.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (rl >= tc.nrows) continue;
        float* yrow = Y + static_cast<int64_t>(tc.row0 + rl) * p.ldc + cgo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = n0 + wn * 128 + j * 16 + (lane & 15);
          if (col < p.N) yrow[col] = acc[i][j][r];
        }
      }
    }
  }
}

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
        if constexpr (SWIGLU) crow[col] = silu_f32_accurate(acc[i][j]) * acc3[i][j];
        else crow[col] = acc[i][j];
    }
  }
}

template <typename Kern>
hipError_t launch_grid(Kern kern, const GroupedGemm& g, int ntn, hipStream_t s) {
  const int64_t logical = static_cast<int64_t>(g.max_mtiles) * ntn * g.ngroups_n;
  if (logical <= 0) return hipSuccess;
  const int nblocks = static_cast<int>((logical + 7) / 8 * 8);
  kern<<<nblocks, 256, 0, s>>>(g, ntn, nblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_swiglu_bf16(const GroupedGemm& g, hipStream_t s) {
  return launch_grid(grouped_bf16_kernel<true>, g, (g.N + BN / 2 - 1) / (BN / 2), s);
}
hipError_t launch_grouped_plain_bf16(const GroupedGemm& g, hipStream_t s) {
  return launch_grid(grouped_bf16_kernel<false>, g, (g.N + BN - 1) / BN, s);
}
hipError_t launch_grouped_swiglu_f32(const GroupedGemm& g, hipStream_t s) {
  return launch_grid(grouped_f32_kernel<true>, g, (g.N + FBN - 1) / FBN, s);
}
hipError_t launch_grouped_plain_f32(const GroupedGemm& g, hipStream_t s) {
  return launch_grid(grouped_f32_kernel<false>, g, (g.N + FBN - 1) / FBN, s);
}

}  // namespace moe
