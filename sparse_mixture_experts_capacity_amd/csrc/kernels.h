// Launchers of the libmoe HIP kernels, called by the host layer
// (moe_api.cpp).  Internal; the public interface is include/moe.h.
#pragma once

#include "common.h"

namespace moe {

// ---- routing.hip ----------------------------------------------------------
hipError_t launch_router(const void* x, const void* Wg, const float* bias,
                         float* logits, int64_t T, int d, int E, bool bf16,
                         hipStream_t s);
// Router scores of a short bf16 batch as nparts K parts of d / nparts
// columns each (lpart[p][t][e], parts T * E apart), for the top-k pass to
// add in part order.  E = 8 or 16, T * E <= 64, d / nparts a multiple of 4;
// x and Wg 16-byte aligned.
inline bool router_parts_fit(int64_t T, int E, int d) {
  return (E == 8 || E == 16) && T >= 1 && T * E <= 64 && d > 0 && d % 4 == 0;
}
hipError_t launch_router_parts(const void* x, const void* Wg, int T, int d, int E, int nparts,
                               float* lpart, hipStream_t s);
// Router scores of a bf16 batch with 8 <= E <= 64 experts (E % 8 == 0) as
// nparts K parts (lpart[p][t][e], parts T * E apart) on the matrix cores,
// for the top-k pass to add in part order.  d a multiple of 64 * nparts; the
// part's transposed W_gate rows must fit the workgroup's 64 KB of LDS; x and
// Wg 16-byte aligned.
inline size_t router_narrow_lds(int E, int KP) {
  return static_cast<size_t>(16) * ((E + 15) / 16) * (KP + 8) * 2;
}
inline bool router_narrow_fit(int64_t T, int E, int d, int nparts) {
  return E >= 8 && E <= 64 && E % 8 == 0 && T >= 1 && T <= (int64_t(1) << 30) &&
         nparts >= 1 && d > 0 && d % (64 * nparts) == 0 &&
         router_narrow_lds(E, d / nparts) <= 64 * 1024;
}
hipError_t launch_router_narrow(const void* x, const void* Wg, int64_t T, int d, int E,
                                int nparts, float* lpart, hipStream_t s);
int topk_group_size(int E);
// Router scores are read as the sum of `nsplit` partial arrays (split_stride
// apart) plus the optional bias, in a fixed order; when logits_out is given
// the summed scores are also stored there.
hipError_t launch_topk_gate(const float* lpart, int nsplit, int64_t split_stride,
                            const float* bias, float* logits_out, int64_t T, int E,
                            int k, int gating, int renorm, int32_t* topk_idx,
                            float* topk_w, float* Ppart, float* Hpart,
                            int nblocks, int tokens_per_block, hipStream_t s);
// Overflow sent to spare experts: the full router scores [T, E] fp32 (as the
// top-k pass saw them) and three int32 [T*k] scratch arrays.
struct Reroute {
  const float* logits;
  int k;
  int32_t* ovf;
  int32_t* xdest;
  int32_t* xrel;
};
// rr == nullptr: assignments beyond capacity C are dropped.
hipError_t launch_dispatch(const int32_t* topk_idx, int64_t TK, int E, int C,
                           int32_t* lrank, int32_t* blkcnt, int32_t* counts,
                           int32_t* kcount, int32_t* offsets, int32_t* slot,
                           int32_t* perm, int bm, Tile* tiles, int32_t* ntiles,
                           int32_t* tstart, const Reroute* rr, hipStream_t s);
// Short batches: top-k, gates and the whole dispatch in one workgroup
// (T <= kSmallT, T * k <= kSmallTK); results equal launch_topk_gate with one
// block followed by launch_dispatch.
constexpr int kSmallT = 128;
constexpr int kSmallTK = 2048;
hipError_t launch_route_small(const float* lpart, int nsplit, int64_t split_stride,
                              const float* bias, float* logits_out, int T, int E, int k,
                              int gating, int renorm, int32_t* topk_idx, float* topk_w,
                              float* Ppart, float* Hpart, int C, int32_t* counts,
                              int32_t* kcount, int32_t* offsets, int32_t* slot,
                              int32_t* perm, int bm, Tile* tiles, int32_t* ntiles,
                              int32_t* tstart, hipStream_t s);
hipError_t launch_stats(const float* Ppart, const float* Hpart, int nblk,
                        const int32_t* counts, const int32_t* kcount, int64_t T,
                        int k, int E, double* out, hipStream_t s);

// ---- grouped expert GEMMs (ffn_grouped.hip) --------------------------------
// One launch covers every M-tile of every group.  Rows of a tile are either
// gathered (A row = perm[row] / topk: token rows of routed assignments) or
// taken as is (slot rows, or token rows for shared experts).
struct GroupedGemm {
  const void* A;            // bf16 or fp32 rows
  int64_t lda;
  const int32_t* perm;      // non-null: gather A rows through perm / topk
  int topk;
  const void* B;            // W1 (SwiGLU) or W2 base
  const void* B3;           // W3 base (SwiGLU only)
  int64_t b_stride;         // elements between consecutive experts
  int group_base;           // expert index of group 0
  int ldb;                  // row stride of B: its N (packed: N padded to the block)
  int K;                    // contraction length
  int N;                    // output columns per group
  int ngroups_n;            // groups laid side by side along N (shared GEMM1)
  void* C;                  // output rows
  int64_t ldc;
  int64_t c_group_col;      // output column offset per N-group
  const Tile* tiles;        // device tile list, or null for static tiling
  const int32_t* ntiles;    // number of tiles in the list
  const int32_t* tstart;    // [E+1] first tile of each expert in the list
  int n_experts;
  int static_rows;          // rows when tiles == null
  int max_mtiles;           // upper bound of M-tiles
  int bm;                   // M-tile rows (bf16: 32, 128 or 256; fp32: 64); tiles match it
  int narrow_n;             // bm 32: 128-wide B tiles instead of 256
  int ksplit;               // K is split in this many parts (plain fp32 output only);
  int64_t c_split;          // part p writes C + p * c_split (fp32 partial sums)
  // K-blocked layouts (bf16 kernels): element (row, k) of a matrix with R
  // rows at ((k / 32) * R + row) * 32 + k % 32.  0 = row-major.
  int64_t a_block_rows;     // A (then perm and lda are not used)
  int64_t c_block_rows;     // SwiGLU output H
  // Packed B (bf16 kernels): 0 = row-major with row stride ldb; otherwise the
  // block width W (128 or 256): element (k, n) of an expert's matrix at
  // ((k / 32) * (ldb / W) + n / W) * 32 * W + (n % W) * 32 + k % 32, with ldb
  // the padded N (a multiple of W) and b_stride = K * ldb.
  int b_block_cols;
  // > 0 (plain GEMM, ksplit 2, device tile list): the two K parts are cut at
  // the step that suits this many resident workgroups for the tiles that
  // exist, and each XCD runs its tiles' part-0 units first; 0 = equal parts.
  int kcut_slots;
};
// Packed copy of nexp row-major [K, N] bf16 matrices in the layout above
// (block width W, padded width Npad = N rounded up to W; pad columns zero).
// K % 32 == 0.
hipError_t launch_pack_blocks(const void* src, int64_t nexp, int K, int N, int W, void* dst,
                              hipStream_t s);
// Xb = kept token rows x[perm[s] / topk] for slots s < *nrows_dev, K-blocked
// with R rows.
hipError_t launch_gather_blocked(const void* x, int64_t ldx, const int32_t* perm, int topk,
                                 const int32_t* nrows_dev, int64_t R, int d, void* Xb,
                                 hipStream_t s);
constexpr int kGroupedBM = 128;   // M-tile of the bf16 MFMA kernels, long batches
constexpr int kGroupedBMShort = 32;  // M-tile for short batches (few rows per expert)
constexpr int kGroupedBMWide = 256;  // M-tile for a few hundred, or thousands of, rows per expert
constexpr int kF32BM = 64;        // M-tile of the fp32 kernels
hipError_t launch_grouped_swiglu_bf16(const GroupedGemm& g, hipStream_t s);
hipError_t launch_grouped_plain_bf16(const GroupedGemm& g, hipStream_t s);
hipError_t launch_grouped_swiglu_f32(const GroupedGemm& g, hipStream_t s);
hipError_t launch_grouped_plain_f32(const GroupedGemm& g, hipStream_t s);

// ---- backward.hip ------------------------------------------------------------
// Router backward from the routing state a forward call left behind.
struct RouterBackward {
  const void* x;            // [T, d] layer dtype
  const void* Wg;           // [d, E] layer dtype
  const void* dout;         // [T, d] layer dtype
  const void* Y;            // expert output rows, ysplit K parts ystride apart
  int ysplit;
  int64_t ystride;
  int64_t rows;             // rows of each part (slots at or past it are not read)
  bool vec4;                // d % 4 == 0 and dout aligned to 4 elements
  const int32_t* slot;      // [T*k]
  const int32_t* idx;       // [T*k]
  const float* w;           // [T*k] gates
  const float* logits;      // [T, E] summed router scores
  const int32_t* counts;    // [E] assignments per expert before capacity
  int64_t T;
  int k, E, d;
  bool bf16;
  int chosen_softmax;       // gates are a softmax over the k chosen scores
  float aux_scale;          // aux_coef * E / T
  float ent_scale;          // entropy_coef / T
  float inv_tk;             // 1 / (T k)
  float* dlogits;           // [T, E] out
  float* dW;                // [d, E] out or null
  float* dbias;             // [E] out or null
  float* dx;                // [T, d] out or null
  float* part;              // vector path: [nchunk, d, E] and [nchunk, E];
                            // MFMA path: [wsplit, E, d], then [d, E] and [E]
  float* bpart;
  int nchunk;
  int64_t tokens_per_chunk;
  // bf16 layers: both router products on the MFMA GEMM
  bool mfma;
  int Kp;                   // E rounded up to 64
  int64_t Tp;               // T rounded up to 64
  int64_t T64;              // T rounded down to 64 (the GEMM's share of dW)
  int wsplit;               // K parts of the dW GEMM
  uint16_t* dlb;            // [T, Kp]
  uint16_t* dlT;            // [E, Tp]
  uint16_t* Wt;             // [Kp, d]
};
// dlogits; the bf16 operands of the MFMA products; dW_gate and dbias (when
// requested); the router's share of dx.
hipError_t launch_gate_backward(const RouterBackward& b, hipStream_t s);
hipError_t launch_router_pack(const RouterBackward& b, hipStream_t s);
hipError_t launch_router_wgrad(const RouterBackward& b, hipStream_t s);
hipError_t launch_router_dx(const RouterBackward& b, hipStream_t s);

// ---- combine.hip -------------------------------------------------------------
// out[t] = sum_j [slot >= 0] w[t,j] * sum_p Y[p][slot] + sum_p Ys[p][t]
// Y rows and their K parts are fp32; out is bf16 (RNE) or fp32.
hipError_t launch_combine(const float* Y, int ysplit, int64_t ysplit_stride,
                          const int32_t* slot, const float* topk_w,
                          const float* Ys, int ys_split, int64_t ys_stride,
                          int64_t T, int k, int d, void* out, bool bf16out,
                          hipStream_t s);

}  // namespace moe
