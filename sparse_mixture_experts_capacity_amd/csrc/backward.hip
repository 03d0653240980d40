// Router backward for libmoe (gfx950): gradients of
//   L = sum(dout * out) + aux_coef * aux
// with respect to the router scores, W_gate, the score bias and the router's
// share of x, from the routing state and expert output rows a forward call
// left in the workspace.
//
// Pages: [Routing guide] "MoE routing, fully explained" (allinfo.ai.kr),
// "Plain explanation" para 2 (the router learns through its softmax over the
// experts) and para 4 (the auxiliary load-balancing product E sum f_i P_i).
// The selection, the capacity decisions and the counts f_i are piecewise
// constant and carry no gradient.
//
// Every sum runs in a fixed order (no atomics): results are bitwise
// reproducible.
#include "kernels.h"

#include <math.h>

namespace moe {

// Four consecutive elements of a row as fp32 (column group c4).
__device__ __forceinline__ f32x4 load4(const float* p, int c4) {
  return reinterpret_cast<const f32x4*>(p)[c4];
}
__device__ __forceinline__ f32x4 load4(const uint16_t* p, int c4) {
  const uint2 v = reinterpret_cast<const uint2*>(p)[c4];
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int off = kWave / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// ---------------------------------------------------------------------------
// Gate backward, one wavefront per token t:
//   dw_j = dout[t] . y_j for each assignment some expert ran (y_j: the sum of
//          the down projection's K parts at the assignment's slot), else 0;
//   s    = sum_j w_j dw_j;
//   chosen-softmax gates (top-k then softmax, or renormalised):
//          dl[c_j] = w_j (dw_j - s), 0 for the other experts;
//   softmax over all experts read at the chosen ones:
//          dl[i] = p_i (G_i - s) with G_i = dw_j for i = c_j, else 0;
//   plus aux_scale p_i (f_i - sum_m f_m p_m), aux_scale = aux_coef E / T,
//   f_i = counts_i / (T k);
//   plus ent_scale (-p_i (ln p_i + H_t)), ent_scale = entropy_coef / T, the
//   gradient of the mean router entropy, H_t = -sum_i p_i ln p_i.
// p is the full softmax of the stored scores (NaN as -infinity), formed as
// the forward forms it.  Lane i holds experts i, i + 64, i + 128, i + 192.
// ---------------------------------------------------------------------------
template <typename TOut>
__global__ __launch_bounds__(256) void gate_backward_kernel(
    const TOut* __restrict__ dout, const void* __restrict__ Yv, int ysplit,
    int64_t ystride,
    int64_t rows, bool vec4, const int32_t* __restrict__ slot, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const float* __restrict__ logits,
    const int32_t* __restrict__ counts, int64_t T, int k, int E, int d, int chosen_softmax,
    float aux_scale, float ent_scale, float inv_tk, float* __restrict__ dlogits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  constexpr int V = kMaxExperts / kWave;
  float G[V], Wc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) G[v] = Wc[v] = 0.f;
  const TOut* g = dout + t * d;
  float s = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t a = t * k + j;
    const int sl = slot[a];
    float dwj = 0.f;
    if (sl >= 0 && sl < rows) {   // slots outside the row buffer are never read
      const float* y = static_cast<const float*>(Yv) + static_cast<int64_t>(sl) * d;
      float acc = 0.f;
      if (vec4) {
        // 4 columns per lane per step: 16-byte row loads, 8- or 16-byte dout loads
        const f32x4* y4 = reinterpret_cast<const f32x4*>(y);
        const int64_t ys4 = ystride / 4;
#pragma unroll 4
        for (int c4 = lane; c4 < d / 4; c4 += kWave) {
          f32x4 yv = y4[c4];
          for (int q = 1; q < ysplit; ++q) yv += y4[q * ys4 + c4];
          const f32x4 gv = load4(g, c4);
          acc += gv.x * yv.x + gv.y * yv.y + gv.z * yv.z + gv.w * yv.w;
        }
      } else {
#pragma unroll 4
        for (int c = lane; c < d; c += kWave) {
          float yv = y[c];
          for (int q = 1; q < ysplit; ++q) yv += y[q * ystride + c];
          acc += load_elem(g, c) * yv;
        }
      }
      dwj = wave_sum(acc);
    }
    const float wj = w[a];
    s += wj * dwj;
    const int cj = idx[a];
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (lane + v * kWave == cj) {
        G[v] = dwj;
        Wc[v] = wj;
      }
  }
  // full softmax of the token's scores
  float l[V];
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int i = lane + v * kWave;
    float x = -INFINITY;
    if (i < E) {
      x = logits[t * E + i];
      if (x != x) x = -INFINITY;
    }
    l[v] = x;
    m = fmaxf(m, x);
  }
  m = wave_max(m);
  float ex[V];
  float z = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    ex[v] = (l[v] > -INFINITY) ? expf(l[v] - m) : 0.f;
    z += ex[v];
  }
  z = wave_sum(z);
  const float inv_z = 1.0f / z;
  float fp = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int i = lane + v * kWave;
    if (i < E) fp += counts[i] * inv_tk * (ex[v] * inv_z);
  }
  fp = wave_sum(fp);
  // H_t = ln z - sum_i p_i (l_i - m); ln p_i = (l_i - m) - ln z
  const float lnz = logf(z);
  float plm = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float p = ex[v] * inv_z;
    if (p > 0.f) plm += p * (l[v] - m);
  }
  const float H = lnz - wave_sum(plm);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int i = lane + v * kWave;
    if (i >= E) continue;
    const float p = ex[v] * inv_z;
    float dl = chosen_softmax ? Wc[v] * (G[v] - s) : p * (G[v] - s);
    if (aux_scale != 0.f) dl += aux_scale * p * (counts[i] * inv_tk - fp);
    if (ent_scale != 0.f && p > 0.f) dl -= ent_scale * p * ((l[v] - m - lnz) + H);
    dlogits[t * E + i] = dl;
  }
}

// ---------------------------------------------------------------------------
// dW_gate partial sums: part[chunk][c][e] = sum over the chunk's tokens of
// x[t, c] dl[t, e], and bpart[chunk][e] = sum of dl[t, e].  A workgroup
// covers 64 columns c and 32 experts; lane c of wavefront q keeps experts
// e0 + 8q .. e0 + 8q + 7.  The scores a wavefront reads are the same for all
// its lanes.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void router_wgrad_kernel(
    const TIn* __restrict__ x, const float* __restrict__ dl, int64_t T, int d, int E,
    int64_t tfirst, int64_t tokens_per_chunk, float* __restrict__ part,
    float* __restrict__ bpart) {
  const int cl = threadIdx.x & (kWave - 1);
  const int q = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
  const int c = blockIdx.x * kWave + cl;
  const int e0 = blockIdx.y * 32 + q * 8;
  const int64_t chunk = blockIdx.z;
  const int64_t t0 = tfirst + chunk * tokens_per_chunk;
  const int64_t t1 = min(T, t0 + tokens_per_chunk);
  float acc[8], bs[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = bs[u] = 0.f;
  if (e0 < E) {
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
      const float xv = c < d ? load_elem(x, t * d + c) : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float g = (e0 + u < E) ? dl[t * E + e0 + u] : 0.f;
        acc[u] += xv * g;
        bs[u] += g;
      }
    }
  }
  if (c < d) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (e0 + u < E) part[(chunk * d + c) * E + e0 + u] = acc[u];
  }
  if (blockIdx.x == 0 && cl == 0) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (e0 + u < E) bpart[chunk * E + e0 + u] = bs[u];
  }
}

// dW_gate[i] = sum of the chunks' partial sums in chunk order, i < d*E;
// dbias[e] likewise.
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ bpart, int nchunk, int64_t n,
    int E, float* __restrict__ dW, float* __restrict__ dbias) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (dW && i < n) {
    float s = 0.f;
    for (int q = 0; q < nchunk; ++q) s += part[q * n + i];
    dW[i] = s;
  }
  if (dbias && i < E) {
    float s = 0.f;
    for (int q = 0; q < nchunk; ++q) s += bpart[q * E + i];
    dbias[i] = s;
  }
}

// ---------------------------------------------------------------------------
// The router's share of dx: dx[t, c] = sum_e dl[t, e] W_gate[c, e].  A
// workgroup covers 256 columns and kDxTokens tokens; their scores sit in LDS
// and every thread reads the same entry at a time (a broadcast); thread c
// reads its own row of W_gate, 8 experts at a time.
// ---------------------------------------------------------------------------
constexpr int kDxTokens = 32;
template <typename TIn>
__global__ __launch_bounds__(256) void router_dx_kernel(
    const float* __restrict__ dl, const TIn* __restrict__ Wg, int64_t T, int d, int E,
    float* __restrict__ dx) {
  __shared__ float sdl[kDxTokens * kMaxExperts];
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kDxTokens;
  const int nt = static_cast<int>(min<int64_t>(kDxTokens, T - t0));
  for (int i = threadIdx.x; i < kDxTokens * E; i += blockDim.x) {
    const int r = i / E;
    sdl[i] = r < nt ? dl[(t0 + r) * E + (i - r * E)] : 0.f;
  }
  __syncthreads();
  if (c >= d) return;
  float acc[kDxTokens];
#pragma unroll
  for (int r = 0; r < kDxTokens; ++r) acc[r] = 0.f;
  const TIn* wrow = Wg + static_cast<int64_t>(c) * E;
  for (int e0 = 0; e0 < E; e0 += 8) {
    float wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) wv[u] = (e0 + u < E) ? load_elem(wrow, e0 + u) : 0.f;
#pragma unroll
    for (int r = 0; r < kDxTokens; ++r)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (e0 + u < E) acc[r] += sdl[r * E + e0 + u] * wv[u];
  }
  for (int r = 0; r < nt; ++r) dx[(t0 + r) * d + c] = acc[r];
}

// ---------------------------------------------------------------------------
// bf16 layers run both router products on the MFMA GEMM.  Operands:
//   dlb [T, Kp]  bf16 dlogits, columns E .. Kp-1 zero   (dx = dlb Wt)
//   dlT [E, Tp]  bf16 dlogits transposed, columns T .. Tp-1 zero
//                                                     (dW^T = dlT x)
//   Wt  [Kp, d]  bf16 W_gate transposed, rows E .. Kp-1 zero
// with Kp and Tp multiples of 64.  Rounding the score gradients to bf16
// moves each product by at most 2^-9 of the sum of its terms' magnitudes.
// 32 x 32 tiles through LDS keep both the reads and the transposed writes
// coalesced.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_dlogits_kernel(
    const float* __restrict__ dl, int64_t T, int E, int Kp, int64_t Tp,
    uint16_t* __restrict__ dlb, uint16_t* __restrict__ dlT) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int e0 = blockIdx.y * 32;
  for (int r = ty; r < 32; r += 8) {
    const int64_t t = t0 + r;
    const int e = e0 + tx;
    const float v = (t < T && e < E) ? dl[t * E + e] : 0.f;
    tile[r][tx] = v;
    if (t < T && e < Kp) dlb[t * Kp + e] = f32_to_bf16(v);
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r;
    const int64_t t = t0 + tx;
    if (e < E && t < Tp) dlT[static_cast<int64_t>(e) * Tp + t] = f32_to_bf16(tile[tx][r]);
  }
}

__global__ __launch_bounds__(256) void transpose_gate_kernel(
    const uint16_t* __restrict__ Wg, int d, int E, int Kp, uint16_t* __restrict__ Wt) {
  __shared__ uint16_t tile[32][34];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int c0 = blockIdx.x * 32;
  const int e0 = blockIdx.y * 32;
  for (int r = ty; r < 32; r += 8) {
    const int c = c0 + r, e = e0 + tx;
    tile[r][tx] = (c < d && e < E) ? Wg[static_cast<int64_t>(c) * E + e] : 0;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, c = c0 + tx;
    if (e < Kp && c < d) Wt[static_cast<int64_t>(e) * d + c] = tile[tx][r];
  }
}

// dW_gate[c, e] = sum of the GEMM's K parts of dW^T[e, c] in part order, plus
// the vector kernel's sum over the tokens past the last whole 64 (tail[c, e]).
// Threads run over (e, c) with c fastest, so the parts are read coalesced.
__global__ __launch_bounds__(256) void router_wgrad_finish_kernel(
    const float* __restrict__ partT, int nparts, const float* __restrict__ tail, int d, int E,
    float* __restrict__ dW) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = static_cast<int64_t>(d) * E;
  if (i >= n) return;
  const int e = static_cast<int>(i / d), c = static_cast<int>(i - static_cast<int64_t>(e) * d);
  float s = 0.f;
  for (int q = 0; q < nparts; ++q) s += partT[static_cast<int64_t>(q) * n + i];
  const int64_t o = static_cast<int64_t>(c) * E + e;
  if (tail) s += tail[o];
  dW[o] = s;
}

// dbias[e] = sum over t of dl[t, e]: one workgroup per expert, a strided
// per-thread sum and a fixed tree over the workgroup.
__global__ __launch_bounds__(256) void column_sum_kernel(const float* __restrict__ dl,
                                                         int64_t T, int E,
                                                         float* __restrict__ out) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += blockDim.x) s += dl[t * E + e];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = red[0];
}

hipError_t launch_gate_backward(const RouterBackward& b, hipStream_t s) {
  const int wpb = 4;   // tokens (wavefronts) per workgroup
  const unsigned blocks = static_cast<unsigned>((b.T + wpb - 1) / wpb);
  if (b.bf16)
    gate_backward_kernel<uint16_t><<<blocks, wpb * kWave, 0, s>>>(
        static_cast<const uint16_t*>(b.dout), b.Y, b.ysplit, b.ystride, b.rows, b.vec4, b.slot, b.idx, b.w,
        b.logits, b.counts, b.T, b.k, b.E, b.d, b.chosen_softmax, b.aux_scale, b.ent_scale, b.inv_tk,
        b.dlogits);
  else
    gate_backward_kernel<float><<<blocks, wpb * kWave, 0, s>>>(
        static_cast<const float*>(b.dout), b.Y, b.ysplit, b.ystride, b.rows, b.vec4, b.slot, b.idx, b.w,
        b.logits, b.counts, b.T, b.k, b.E, b.d, b.chosen_softmax, b.aux_scale, b.ent_scale, b.inv_tk,
        b.dlogits);
  return hipGetLastError();
}

hipError_t launch_router_pack(const RouterBackward& b, hipStream_t s) {
  if (!b.mfma) return hipSuccess;
  const dim3 g1(static_cast<unsigned>((b.Tp + 31) / 32), (b.Kp + 31) / 32);
  pack_dlogits_kernel<<<g1, 256, 0, s>>>(b.dlogits, b.T, b.E, b.Kp, b.Tp, b.dlb, b.dlT);
  if (b.dx) {
    const dim3 g2((b.d + 31) / 32, (b.Kp + 31) / 32);
    transpose_gate_kernel<<<g2, 256, 0, s>>>(static_cast<const uint16_t*>(b.Wg), b.d, b.E,
                                              b.Kp, b.Wt);
  }
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const RouterBackward& b, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(b.d) * b.E;
  if (!b.mfma) {
    const dim3 grid((b.d + kWave - 1) / kWave, (b.E + 31) / 32, b.nchunk);
    if (b.bf16)
      router_wgrad_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(b.x),
                                                         b.dlogits, b.T, b.d, b.E, 0,
                                                         b.tokens_per_chunk, b.part, b.bpart);
    else
      router_wgrad_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(b.x),
                                                      b.dlogits, b.T, b.d, b.E, 0,
                                                      b.tokens_per_chunk, b.part, b.bpart);
    const int64_t cover = n > b.E ? n : b.E;
    router_wgrad_reduce_kernel<<<static_cast<unsigned>((cover + 255) / 256), 256, 0, s>>>(
        b.part, b.bpart, b.nchunk, n, b.E, b.dW, b.dbias);
    return hipGetLastError();
  }
  if (b.dbias) column_sum_kernel<<<b.E, 256, 0, s>>>(b.dlogits, b.T, b.E, b.dbias);
  if (!b.dW) return hipGetLastError();
  // dW^T = dlT x over the first T64 tokens, K split into wsplit parts
  if (b.T64 > 0) {
    GroupedGemm g{};
    g.A = b.dlT; g.lda = b.Tp; g.perm = nullptr; g.topk = 1;
    g.B = b.x; g.B3 = nullptr; g.b_stride = 0; g.group_base = 0; g.ldb = b.d;
    g.K = static_cast<int>(b.T64); g.N = b.d; g.ngroups_n = 1;
    g.C = b.part; g.ldc = b.d; g.c_group_col = 0;
    g.tiles = nullptr; g.ntiles = nullptr; g.tstart = nullptr; g.n_experts = 1;
    g.static_rows = b.E; g.bm = b.E <= 64 ? kGroupedBMShort : kGroupedBM;
    g.max_mtiles = (b.E + g.bm - 1) / g.bm;
    g.narrow_n = 0; g.ksplit = b.wsplit; g.c_split = n;
    g.a_block_rows = 0; g.c_block_rows = 0;
    hipError_t e = launch_grouped_plain_bf16(g, s);
    if (e != hipSuccess) return e;
  }
  // the tokens past the last whole 64 on the vector kernel, one chunk
  float* tail = nullptr;
  if (b.T64 < b.T) {
    tail = b.part + static_cast<int64_t>(b.wsplit) * n;
    const dim3 grid((b.d + kWave - 1) / kWave, (b.E + 31) / 32, 1);
    router_wgrad_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(b.x),
                                                       b.dlogits, b.T, b.d, b.E, b.T64,
                                                       b.T - b.T64, tail, tail + n);
  }
  router_wgrad_finish_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      b.part, b.T64 > 0 ? b.wsplit : 0, tail, b.d, b.E, b.dW);
  return hipGetLastError();
}

hipError_t launch_router_dx(const RouterBackward& b, hipStream_t s) {
  if (b.mfma) {
    GroupedGemm g{};
    g.A = b.dlb; g.lda = b.Kp; g.perm = nullptr; g.topk = 1;
    g.B = b.Wt; g.B3 = nullptr; g.b_stride = 0; g.group_base = 0; g.ldb = b.d;
    g.K = b.Kp; g.N = b.d; g.ngroups_n = 1;
    g.C = b.dx; g.ldc = b.d; g.c_group_col = 0;
    g.tiles = nullptr; g.ntiles = nullptr; g.tstart = nullptr; g.n_experts = 1;
    g.static_rows = static_cast<int>(b.T); g.bm = b.T <= 64 ? kGroupedBMShort : kGroupedBM;
    g.max_mtiles = static_cast<int>((b.T + g.bm - 1) / g.bm);
    g.narrow_n = 0; g.ksplit = 1; g.c_split = 0;
    g.a_block_rows = 0; g.c_block_rows = 0;
    return launch_grouped_plain_bf16(g, s);
  }
  const dim3 grid((b.d + 255) / 256, static_cast<unsigned>((b.T + kDxTokens - 1) / kDxTokens));
  if (b.bf16)
    router_dx_kernel<uint16_t><<<grid, 256, 0, s>>>(
        b.dlogits, static_cast<const uint16_t*>(b.Wg), b.T, b.d, b.E, b.dx);
  else
    router_dx_kernel<float><<<grid, 256, 0, s>>>(b.dlogits, static_cast<const float*>(b.Wg),
                                                 b.T, b.d, b.E, b.dx);
  return hipGetLastError();
}

}  // namespace moe
