// Router scores, top-k gating, capacity-limited dispatch and routing
// statistics for libmoe (gfx950).
//
// Pages: [Mixtral explainer] "Mixtral 8x7B and MoE explained"
// (allinfo.ai.kr), "Plain explanation" para 3 (router logits, top-2,
// softmax over the two); [Routing guide] "MoE routing, fully explained"
// (allinfo.ai.kr), "Plain explanation" paras 2-5 (distribution over all
// experts, top-k, capacity, dropping the overflow, aux load-balancing
// product), "Key insights" item 3 (counts, overflow, entropy).
//
// Everything here is deterministic: no floating-point atomics, and integer
// ranks come from wavefront ballots processed in a fixed order.
#include "kernels.h"

#include <float.h>
#include <limits.h>

namespace moe {

// ---------------------------------------------------------------------------
// Router scores, few experts (E <= 16): one wavefront per token; each lane
// walks a strided slice of d and keeps E partial sums, then a fixed butterfly
// sums across the wavefront.  bf16 x bf16 products are exact in fp32.
// ---------------------------------------------------------------------------
template <typename TIn, int EC>
__global__ __launch_bounds__(256) void router_small_e_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ Wg,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t T,
    int d, int E) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float acc[EC];
#pragma unroll
  for (int e = 0; e < EC; ++e) acc[e] = 0.f;
  const TIn* xr = x + t * d;
  for (int c = lane; c < d; c += kWave) {
    const float xv = load_elem(xr, c);
    const TIn* wr = Wg + static_cast<int64_t>(c) * E;
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E) acc[e] = fmaf(xv, load_elem(wr, e), acc[e]);
  }
#pragma unroll
  for (int e = 0; e < EC; ++e) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[e] += __shfl_xor(acc[e], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < EC; ++e)
      if (e < E) logits[t * E + e] = acc[e] + (bias ? bias[e] : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Router scores, many experts: a workgroup owns 16 tokens; thread e owns
// expert e (and e+256 ...); token rows are staged in LDS 256 columns at a
// time and W_gate rows are read coalesced across experts.
// ---------------------------------------------------------------------------
constexpr int kRouterTB = 16;
template <typename TIn>
__global__ __launch_bounds__(256) void router_large_e_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ Wg,
    const float* __restrict__ bias, float* __restrict__ logits, int64_t T,
    int d, int E) {
  __shared__ float xs[kRouterTB][256];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTB;
  const int e = tid;
  float acc[kRouterTB];
#pragma unroll
  for (int i = 0; i < kRouterTB; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < d; c0 += 256) {
    const int cn = min(256, d - c0);
    for (int i = 0; i < kRouterTB; ++i) {
      const int64_t t = t0 + i;
      xs[i][tid] = (t < T && tid < cn) ? load_elem(x + t * d, c0 + tid) : 0.f;
    }
    __syncthreads();
    if (e < E) {
      for (int cc = 0; cc < cn; ++cc) {
        const float w = load_elem(Wg, static_cast<int64_t>(c0 + cc) * E + e);
#pragma unroll
        for (int i = 0; i < kRouterTB; ++i) acc[i] = fmaf(xs[i][cc], w, acc[i]);
      }
    }
    __syncthreads();
  }
  if (e < E) {
    const float b = bias ? bias[e] : 0.f;
    for (int i = 0; i < kRouterTB; ++i) {
      const int64_t t = t0 + i;
      if (t < T) logits[t * E + e] = acc[i] + b;
    }
  }
}

template <typename TIn>
hipError_t launch_router_t(const TIn* x, const TIn* Wg, const float* bias,
                           float* logits, int64_t T, int d, int E,
                           hipStream_t s) {
  if (E <= 8) {
    router_small_e_kernel<TIn, 8><<<(T + 3) / 4, 256, 0, s>>>(x, Wg, bias, logits, T, d, E);
  } else if (E <= 16) {
    router_small_e_kernel<TIn, 16><<<(T + 3) / 4, 256, 0, s>>>(x, Wg, bias, logits, T, d, E);
  } else {
    router_large_e_kernel<TIn><<<(T + kRouterTB - 1) / kRouterTB, 256, 0, s>>>(
        x, Wg, bias, logits, T, d, E);
  }
  return hipGetLastError();
}

hipError_t launch_router(const void* x, const void* Wg, const float* bias,
                         float* logits, int64_t T, int d, int E, bool bf16,
                         hipStream_t s) {
  if (bf16)
    return launch_router_t(static_cast<const uint16_t*>(x),
                           static_cast<const uint16_t*>(Wg), bias, logits, T,
                           d, E, s);
  return launch_router_t(static_cast<const float*>(x),
                         static_cast<const float*>(Wg), bias, logits, T, d, E,
                         s);
}

// ---------------------------------------------------------------------------
// Router scores of a short bf16 batch in K parts ([Mixtral explainer]
// "Plain explanation" para 3: one score per expert from the token's vector):
// part p of score (t, e) is sum over its column range of x[t][c] Wg[c][e],
// and the top-k pass adds the parts in part order.  One wavefront per part.
// Lane l takes columns 4l .. 4l+3 of each 256-column run of the part and
// keeps NV = TM * NE register sums, one per (token, expert) for T <= TM
// tokens (the rows from T on read as zero).  The wavefront then sums them by
// recursive halving: at lane bit b (b = 5, 4, ...), a lane keeps the half of
// its current sums that its bit selects and adds the partner's copy of that
// half, so after log2 NV exchanges lane l holds sum index l >> (6 - log2 NV)
// over 2^log2 NV lanes; an xor butterfly over the lower lane bits completes
// it.  NV - 1 + (6 - log2 NV) exchanges in all, in a fixed order.
// ---------------------------------------------------------------------------
template <int NE, int TM>
__global__ __launch_bounds__(64) void router_parts_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg, int T, int d, int cols,
    float* __restrict__ lpart) {
  constexpr int NV = TM * NE;
  constexpr int LV = NV == 8 ? 3 : NV == 16 ? 4 : NV == 32 ? 5 : 6;
  static_assert((1 << LV) == NV, "NV must be 8, 16, 32 or 64");
  const int lane = threadIdx.x;
  const int c_begin = blockIdx.x * cols;
  const int c_end = c_begin + cols;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = 0.f;
  for (int c0 = c_begin + 4 * lane; c0 < c_end; c0 += 4 * kWave) {
    uint4 wv[4][NE / 8];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < NE / 8; ++h)
        wv[q][h] = *reinterpret_cast<const uint4*>(Wg + static_cast<int64_t>(c0 + q) * NE + 8 * h);
    uint2 xv[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
      xv[t] = t < T ? *reinterpret_cast<const uint2*>(x + static_cast<int64_t>(t) * d + c0)
                    : make_uint2(0u, 0u);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float w[NE];
#pragma unroll
      for (int h = 0; h < NE / 8; ++h) {
        const uint32_t u[4] = {wv[q][h].x, wv[q][h].y, wv[q][h].z, wv[q][h].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          w[8 * h + 2 * r] = __uint_as_float(u[r] << 16);
          w[8 * h + 2 * r + 1] = __uint_as_float(u[r] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const uint32_t xw = q < 2 ? xv[t].x : xv[t].y;
        const float xq = __uint_as_float((q & 1) ? (xw & 0xffff0000u) : (xw << 16));
#pragma unroll
        for (int e = 0; e < NE; ++e) v[t * NE + e] = fmaf(xq, w[e], v[t * NE + e]);
      }
    }
  }
  // recursive halving over lane bits 5 .. 6 - LV
#pragma unroll
  for (int st = 0; st < LV; ++st) {
    const int off = kWave >> (st + 1);
    const int half = NV >> (st + 1);
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = upper ? v[i + half] : v[i];
      const float send = upper ? v[i] : v[i + half];
      v[i] = keep + __shfl_xor(send, off);
    }
  }
  float r = v[0];
#pragma unroll
  for (int off = (kWave >> LV) >> 1; off >= 1; off >>= 1) r += __shfl_xor(r, off);
  constexpr int kLow = kWave >> LV;   // lanes sharing one sum index
  const int idx = lane / kLow;
  if (lane % kLow == 0 && idx < T * NE)
    lpart[static_cast<int64_t>(blockIdx.x) * T * NE + idx] = r;
}

hipError_t launch_router_parts(const void* x, const void* Wg, int T, int d, int E, int nparts,
                               float* lpart, hipStream_t s) {
  if (!router_parts_fit(T, E, d) || nparts < 1 || d % nparts || (d / nparts) % 4)
    return hipErrorInvalidValue;
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* wb = static_cast<const uint16_t*>(Wg);
  const int cols = d / nparts;
#define MOE_PARTS_LAUNCH(NE, TM) \
  router_parts_kernel<NE, TM><<<nparts, kWave, 0, s>>>(xb, wb, T, d, cols, lpart)
  if (E == 8) {
    if (T <= 1) MOE_PARTS_LAUNCH(8, 1);
    else if (T <= 2) MOE_PARTS_LAUNCH(8, 2);
    else if (T <= 4) MOE_PARTS_LAUNCH(8, 4);
    else MOE_PARTS_LAUNCH(8, 8);
  } else {
    if (T <= 1) MOE_PARTS_LAUNCH(16, 1);
    else if (T <= 2) MOE_PARTS_LAUNCH(16, 2);
    else MOE_PARTS_LAUNCH(16, 4);
  }
#undef MOE_PARTS_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router scores of a bf16 batch with few experts (E a multiple of 8, at most
// 64) in K parts, on the matrix cores ([Mixtral explainer] "Plain
// explanation" para 3: one score per expert from the token's vector).  Part
// p of score (t, e) is the sum over columns [p KP, (p+1) KP) of x[t][c]
// Wg[c][e], and the top-k pass adds the parts in part order.  A workgroup
// takes one part and 64 tokens.  It stages the part's W_gate rows in LDS
// transposed: one row of KP values per expert, 16 NJ rows with those past E
// zero, each row padded by 16 bytes so that the 16 rows one read touches
// fall in different bank groups.  Each of its four wavefronts multiplies 16
// tokens with v_mfma_f32_16x16x32_bf16 (lane l: token l % 16, k block
// l / 16), reading the token fragments straight from memory in chunks of
// kNarrowSteps K steps (16 bytes per lane each): the first chunk is loaded
// while the weights are staged, and each next one while the current one is
// multiplied.  The tiled expert GEMM would give the scores a 256-wide weight
// tile; here the weight operand is E columns rounded up to 16.
// ---------------------------------------------------------------------------
constexpr int kNarrowSteps = 8;
template <int NJ>
__global__ __launch_bounds__(256) void router_narrow_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wg, int T, int d, int E,
    int KP, float* __restrict__ lpart) {
  extern __shared__ __attribute__((aligned(16))) uint16_t wt[];   // [16 NJ][KP + 8]
  const int RS = KP + 8;
  const int part = blockIdx.y;
  const int64_t k0 = static_cast<int64_t>(part) * KP;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int i16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 64 + wave * 16;
  const bool active = t0 < T;   // wave-uniform
  // rows past T repeat row T - 1 (their sums are not stored)
  const int trow = min(t0 + i16, T - 1);
  const uint16_t* xr = x + static_cast<int64_t>(trow) * d + k0 + g * 8;
  const int nsteps = KP / 32;
  // K steps s0 .. s0+7 of this lane's token fragment; steps past the part
  // repeat its last step (loaded, never multiplied), so every load is
  // unconditional and the waits before the MFMAs count exactly.
  auto load_chunk = [&](bf16x8 (&a)[kNarrowSteps], int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kNarrowSteps; ++c)
      a[c] = *reinterpret_cast<const bf16x8*>(xr + min(s0 + c, nsteps - 1) * 32);
  };
  // The first chunk's token fragments are in flight while the weights are
  // staged (also in wavefronts past T, whose rows all repeat row T - 1:
  // unconditional, so nothing waits on them before the staging).
  bf16x8 a[kNarrowSteps];
  load_chunk(a, 0);
  // W_gate rows k0 .. k0+KP: thread -> row kk, 16 bytes (8 experts) at a time
  const int eg = E >> 3;
  for (int kk = threadIdx.x; kk < KP; kk += blockDim.x) {
    const uint16_t* wrow = Wg + (k0 + kk) * E;
    for (int q = 0; q < eg; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(wrow + q * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wt[(q * 8 + 2 * j) * RS + kk] = static_cast<uint16_t>(v[j] & 0xffffu);
        wt[(q * 8 + 2 * j + 1) * RS + kk] = static_cast<uint16_t>(v[j] >> 16);
      }
    }
  }
  for (int r = E; r < 16 * NJ; ++r)
    for (int kk = threadIdx.x; kk < KP; kk += blockDim.x) wt[r * RS + kk] = 0;
  __syncthreads();
  if (!active) return;   // no barrier follows

  const uint16_t* wr = wt + i16 * RS + g * 8;
  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsteps; s0 += kNarrowSteps) {
    // the next chunk's loads go out before this chunk is multiplied
    bf16x8 an[kNarrowSteps];
    const bool more = s0 + kNarrowSteps < nsteps;
    if (more) load_chunk(an, s0 + kNarrowSteps);
#pragma unroll
    for (int c = 0; c < kNarrowSteps; ++c) {
      if (s0 + c < nsteps) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(wr + j * 16 * RS + (s0 + c) * 32);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], b, acc[j], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < kNarrowSteps; ++c) a[c] = an[c];
    }
  }
  // lane l holds tokens t0 + 4 (l / 16) + r, expert 16 j + l % 16
  float* out = lpart + static_cast<int64_t>(part) * T * E;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * 16 + i16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + g * 4 + r;
      if (t < T && e < E) out[static_cast<int64_t>(t) * E + e] = acc[j][r];
    }
  }
}

hipError_t launch_router_narrow(const void* x, const void* Wg, int64_t T, int d, int E,
                                int nparts, float* lpart, hipStream_t s) {
  if (!router_narrow_fit(T, E, d, nparts)) return hipErrorInvalidValue;
  const auto* xb = static_cast<const uint16_t*>(x);
  const auto* wb = static_cast<const uint16_t*>(Wg);
  const int KP = d / nparts;
  const int NJ = (E + 15) / 16;
  const size_t lds = router_narrow_lds(E, KP);
  const dim3 grid(static_cast<unsigned>((T + 63) / 64), static_cast<unsigned>(nparts));
  const int Ti = static_cast<int>(T);
  if (NJ == 1) router_narrow_kernel<1><<<grid, 256, lds, s>>>(xb, wb, Ti, d, E, KP, lpart);
  else if (NJ == 2) router_narrow_kernel<2><<<grid, 256, lds, s>>>(xb, wb, Ti, d, E, KP, lpart);
  else if (NJ == 3) router_narrow_kernel<3><<<grid, 256, lds, s>>>(xb, wb, Ti, d, E, KP, lpart);
  else router_narrow_kernel<4><<<grid, 256, lds, s>>>(xb, wb, Ti, d, E, KP, lpart);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k + gates + softmax statistics.  A group of G lanes (G a power of two,
// G >= E/4) handles one token; lane g of the group holds the scores of
// experts g, g+G, g+2G, g+3G.  k rounds of a group-wide argmax by butterfly
// exchange pick the experts best first; order is (score descending, index
// ascending) under IEEE comparison, so -0 and +0 tie and the lower index
// wins.  Each group also accumulates the full softmax p[t, :] and the
// per-token entropy for the load-balance statistics; the workgroup then sums
// its groups in a fixed order into one partial row per workgroup.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return (a > b) || (a == b && ia < ib);
}

// Top-k selection and gates of token t by a group of G lanes (lane gl of the
// group): the router score of expert i is the sum of the nsplit partial
// arrays (split_stride apart) plus bias[i]; lane gl holds experts gl + v*G.
// Lane 0 writes the chosen experts (best first) and their gates; every lane
// adds its experts' full-softmax probabilities to pacc and lane 0 the
// token's router entropy to hacc.  When sidx is given, lane 0 also stores the
// chosen experts there.
template <int V>
__device__ __forceinline__ void topk_token(
    int64_t t, const float* __restrict__ lpart, int nsplit, int64_t split_stride,
    const float* __restrict__ bias, float* __restrict__ logits_out, int E, int k, int G,
    int gl, int gating, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int* sidx, float (&pacc)[V], float& hacc) {
  float val[V];
  bool taken[V];
  // The K parts of the lane's V scores, summed in the fixed order q = 0, 1,
  // ...; kParts parts of every score are loaded before the first add, so
  // V * kParts = 8 loads are in flight together.
  constexpr int kParts = 8 / V > 2 ? 8 / V : 2;
  float lsum[V];
#pragma unroll
  for (int v = 0; v < V; ++v) lsum[v] = 0.f;
  for (int q0 = 0; q0 < nsplit; q0 += kParts) {
    float part[V][kParts];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int i = gl + v * G;
#pragma unroll
      for (int u = 0; u < kParts; ++u)
        part[v][u] = (i < E && q0 + u < nsplit)
                         ? lpart[static_cast<int64_t>(q0 + u) * split_stride + t * E + i]
                         : 0.f;
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
      for (int u = 0; u < kParts; ++u) {
        if (q0 + u < nsplit) lsum[v] = (q0 + u == 0) ? part[v][u] : lsum[v] + part[v][u];
      }
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int i = gl + v * G;
    float l = -INFINITY;
    if (i < E) {
      l = lsum[v];
      if (bias) l += bias[i];
      if (logits_out) logits_out[t * E + i] = l;
      // A NaN score ranks as -infinity: never ahead of a number, ties by
      // index, so a valid expert index is always chosen.
      if (l != l) l = -INFINITY;
    }
    val[v] = l;
    taken[v] = !(i < E);
  }
  float m = 0.f;
  float esum = 0.f;  // sum of e^(l_j - m) over the chosen experts (lane 0)
  for (int j = 0; j < k; ++j) {
    // sentinel loses to every real expert, -infinity scores included
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int i = gl + v * G;
      if (!taken[v] && better(val[v], i, bv, bi)) { bv = val[v]; bi = i; }
    }
    for (int off = G >> 1; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, G);
      const int oi = __shfl_xor(bi, off, G);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (j == 0) m = bv;
    if ((bi % G) == gl) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (gl + v * G == bi) taken[v] = true;
    }
    if (gl == 0 && topk_idx) topk_idx[t * k + j] = bi;
    if (gl == 0 && sidx) sidx[t * k + j] = bi;
    if (gl == 0 && topk_w) {
      // un-normalised gate e^(l_j - m); scaled below once Z is known
      const float ej = bv > -INFINITY ? expf(bv - m) : 0.f;
      topk_w[t * k + j] = ej;
      esum += ej;
    }
  }
  // Full softmax over all E experts, shifted by the top score m.
  float ex[V];
  float z = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    ex[v] = (gl + v * G < E && val[v] > -INFINITY) ? expf(val[v] - m) : 0.f;
    z += ex[v];
  }
  for (int off = G >> 1; off >= 1; off >>= 1) z += __shfl_xor(z, off, G);
  const float inv_z = 1.0f / z;
  float plogp = 0.f;  // sum_i p_i (l_i - m)
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const float p = ex[v] * inv_z;
    pacc[v] += p;
    if (p > 0.f) plogp += p * (val[v] - m);
  }
  for (int off = G >> 1; off >= 1; off >>= 1) plogp += __shfl_xor(plogp, off, G);
  if (gl == 0) hacc += logf(z) - plogp;

  // Gate weights: Mixtral order w_j = e_j / sum_j' e_j; DeepSeek order
  // w_j = e_j / Z (the full softmax at the chosen expert), or e_j / sum e
  // when renormalised.  Lane 0 rescales the values it wrote above.
  if (gl == 0 && topk_w) {
    const float scale = (gating == 0 || renorm) ? 1.0f / esum : inv_z;
    for (int j = 0; j < k; ++j) topk_w[t * k + j] *= scale;
  }
}

template <int V>
__global__ __launch_bounds__(256) void topk_gate_kernel(
    const float* __restrict__ lpart, int nsplit, int64_t split_stride,
    const float* __restrict__ bias, float* __restrict__ logits_out, int64_t T,
    int E, int k, int G, int gating, int renorm, int tokens_per_block,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ Ppart, float* __restrict__ Hpart) {
  __shared__ float pbuf[256 * 4];   // [groups][E], groups*E <= 256*V <= 1024
  __shared__ float hbuf[256];
  const int tid = threadIdx.x;
  const int gl = tid % G;
  const int grp = tid / G;
  const int ngroups = blockDim.x / G;
  float pacc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) pacc[v] = 0.f;
  float hacc = 0.f;

  const int64_t tb = static_cast<int64_t>(blockIdx.x) * tokens_per_block;
  const int64_t te = min(T, tb + tokens_per_block);
  for (int64_t t = tb + grp; t < te; t += ngroups)
    topk_token<V>(t, lpart, nsplit, split_stride, bias, logits_out, E, k, G, gl, gating,
                  renorm, topk_idx, topk_w, nullptr, pacc, hacc);
  // Workgroup reduction of the softmax statistics in a fixed order.
  if (Ppart) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int i = gl + v * G;
      if (i < E) pbuf[grp * E + i] = pacc[v];
    }
    if (gl == 0) hbuf[grp] = hacc;
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
      float s = 0.f;
      for (int g = 0; g < ngroups; ++g) s += pbuf[g * E + e];
      Ppart[static_cast<int64_t>(blockIdx.x) * E + e] = s;
    }
    if (tid == 0) {
      float s = 0.f;
      for (int g = 0; g < ngroups; ++g) s += hbuf[g];
      Hpart[blockIdx.x] = s;
    }
  }
}

int topk_group_size(int E) {
  int G = 1;
  while (G * 4 < E) G <<= 1;
  // at least E/4 lanes per token, at most a wavefront
  while (G < 64 && G < E) G <<= 1;
  return G > 64 ? 64 : G;
}

hipError_t launch_topk_gate(const float* lpart, int nsplit, int64_t split_stride,
                            const float* bias, float* logits_out, int64_t T, int E,
                            int k, int gating, int renorm, int32_t* topk_idx,
                            float* topk_w, float* Ppart, float* Hpart,
                            int nblocks, int tokens_per_block, hipStream_t s) {
  const int G = topk_group_size(E);
  const int V = (E + G - 1) / G;
#define MOE_TOPK_ARGS                                                                \
  lpart, nsplit, split_stride, bias, logits_out, T, E, k, G, gating, renorm,        \
      tokens_per_block, topk_idx, topk_w, Ppart, Hpart
  if (V <= 1)
    topk_gate_kernel<1><<<nblocks, 256, 0, s>>>(MOE_TOPK_ARGS);
  else if (V <= 2)
    topk_gate_kernel<2><<<nblocks, 256, 0, s>>>(MOE_TOPK_ARGS);
  else
    topk_gate_kernel<4><<<nblocks, 256, 0, s>>>(MOE_TOPK_ARGS);
#undef MOE_TOPK_ARGS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dispatch, pass 1: stable rank of each assignment inside its chunk of
// kDispatchChunk assignments.  Each of the workgroup's kRankWaves wavefronts
// walks a quarter of the chunk 64 assignments at a time; lanes with the same
// expert are found with 8 ballots (one per bit of the expert id) and ranked
// by popcount of the lower lanes; the wavefront's LDS counters carry the
// rank across its steps.  The quarters are then joined in order: a rank is
// offset by the counts of the same expert in the earlier quarters.  Writes
// the chunk's per-expert totals.  (One wavefront over the whole chunk took
// four times the serial steps.)
// ---------------------------------------------------------------------------
constexpr int kRankWaves = 4;
static_assert(kDispatchChunk % (kRankWaves * kWave) == 0, "rank chunk");
__global__ __launch_bounds__(kRankWaves * kWave) void dispatch_rank_kernel(
    const int32_t* __restrict__ topk_idx, int64_t TK, int E,
    int32_t* __restrict__ lrank, int32_t* __restrict__ blkcnt) {
  __shared__ int cnt[kRankWaves][kMaxExperts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kRankWaves * E; i += blockDim.x) cnt[i / E][i % E] = 0;
  __syncthreads();
  constexpr int kQuarter = kDispatchChunk / kRankWaves;
  constexpr int kSteps = kQuarter / kWave;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kDispatchChunk + wave * kQuarter;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // All of the lane's expert ids are loaded before the first is ranked, so
  // the loads are in flight together rather than one per step.
  int ids[kSteps];
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int64_t a = base + it * kWave + lane;
    ids[it] = a < TK ? topk_idx[a] : -1;
  }
  int* c = cnt[wave];
  int rk[kSteps];
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int ein = ids[it];
    const bool valid = ein >= 0 && ein < E;   // ids outside [0, E) are ignored
    const int e = valid ? ein : 0;
    uint64_t match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const int before = valid ? c[e] : 0;
    __builtin_amdgcn_wave_barrier();
    const bool leader = valid && (__ffsll(static_cast<unsigned long long>(match)) - 1 == lane);
    if (leader) c[e] = before + __popcll(match);
    __builtin_amdgcn_wave_barrier();
    rk[it] = before + __popcll(match & lt);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int64_t a = base + it * kWave + lane;
    const int ein = ids[it];
    if (ein >= 0 && ein < E) {
      int off = 0;
      for (int w = 0; w < wave; ++w) off += cnt[w][ein];
      lrank[a] = rk[it] + off;
    }
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) total += cnt[w][e];
    blkcnt[static_cast<int64_t>(blockIdx.x) * E + e] = total;
  }
}

// ---------------------------------------------------------------------------
// Slot offsets (exclusive prefix sum of the kept counts kc, in LDS) and the
// M-tile list of the grouped expert GEMMs: tiles of at most `bm` rows, expert
// by expert, with tstart[e] the first tile of expert e and tstart[E] their
// number.  Called by every thread of one workgroup (blockDim.x >= 64); off and
// toff are LDS arrays of E + 1 entries.
// ---------------------------------------------------------------------------
__device__ void slot_offsets_and_tiles(const int* kc, int E, int bm, int* off, int* toff,
                                       int32_t* __restrict__ offsets, Tile* __restrict__ tiles,
                                       int32_t* __restrict__ ntiles,
                                       int32_t* __restrict__ tstart) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    // Wavefront 0: lane l sums experts [l*per, (l+1)*per), a shuffle scan
    // gives each lane the rows and tiles of the experts before its run, and
    // the lane then writes its run's exclusive offsets.
    const int per = (E + kWave - 1) / kWave;
    const int i0 = tid * per;
    int rows = 0, ntl = 0;
    for (int u = 0; u < per; ++u) {
      const int i = i0 + u;
      if (i < E) {
        rows += kc[i];
        if (bm > 0) ntl += (kc[i] + bm - 1) / bm;
      }
    }
    int rows_in = rows, ntl_in = ntl;   // inclusive scans over the lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int r = __shfl_up(rows_in, o);
      const int t = __shfl_up(ntl_in, o);
      if (tid >= o) {
        rows_in += r;
        ntl_in += t;
      }
    }
    int so = rows_in - rows, ts = ntl_in - ntl;
    for (int u = 0; u < per; ++u) {
      const int i = i0 + u;
      if (i < E) {
        off[i] = so;
        toff[i] = ts;
        so += kc[i];
        if (bm > 0) ts += (kc[i] + bm - 1) / bm;
      }
    }
    if (tid == kWave - 1) {
      off[E] = rows_in;
      toff[E] = ntl_in;
      if (ntiles) *ntiles = ntl_in;
    }
  }
  __syncthreads();
  for (int i = tid; i <= E; i += blockDim.x) {
    offsets[i] = off[i];
    if (tstart) tstart[i] = toff[i];
  }
  if (tiles && bm > 0) {
    for (int e = tid; e < E; e += blockDim.x) {
      int n = 0;
      for (int r = 0; r < kc[e]; r += bm, ++n)
        tiles[toff[e] + n] = Tile{e, off[e] + r, min(bm, kc[e] - r), 0};
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch, pass 2 (one workgroup): per expert, turn chunk totals into
// exclusive chunk bases (in place) and the total count; apply the capacity;
// prefix-sum the kept counts into slot offsets; build the M-tile list of the
// grouped expert GEMMs (tiles of at most `bm` rows, expert by expert) and the
// index of each expert's first tile (tstart[E] = number of tiles).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dispatch_scan_kernel(
    int32_t* __restrict__ blkcnt, int nblk, int E, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ kcount,
    int32_t* __restrict__ offsets, int bm, Tile* __restrict__ tiles,
    int32_t* __restrict__ ntiles, int32_t* __restrict__ tstart) {
  __shared__ int kc[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int toff[kMaxExperts + 1];
  const int e = threadIdx.x;
  if (e < E) {
    // 16 chunk totals are read before any is overwritten with its base, so
    // their loads overlap.
    constexpr int kBatch = 16;
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        c[u] = b0 + u < nblk ? blkcnt[static_cast<int64_t>(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (b0 + u < nblk) {
          blkcnt[static_cast<int64_t>(b0 + u) * E + e] = run;
          run += c[u];
        }
      }
    }
    counts[e] = run;
    kc[e] = min(run, C);
    kcount[e] = kc[e];
  }
  __syncthreads();
  slot_offsets_and_tiles(kc, E, bm, off, toff, offsets, tiles, ntiles, tstart);
}

// ---------------------------------------------------------------------------
// Dispatch, pass 2b (one workgroup of 1024 threads), only when overflow is
// sent to spare experts ([Routing guide] "Plain explanation" para 3).  After
// pass 2 every expert holds its first min(count, C) assignments.  The
// overflow assignments (rank >= C) are then handled one after another in flat
// order a = t*k + j: each goes to the highest-scoring expert of token t (ties:
// lower index; NaN as -infinity) that t did not choose, that t's earlier
// assignments were not sent to, and that still has a free slot, behind the
// rows already there, or is dropped when none has.
//   A. all threads list the overflow assignments in flat order (ovf);
//   B. in chunks of up to kRerouteRows assignments: all threads copy the
//      chunk's score rows into LDS, writing NaN where an expert is not
//      available (full, one of the token's own choices, or a spare expert
//      one of its assignments of an earlier chunk was sent to); then
//      wavefront 0 takes the chunk 64 assignments at a time, lane i the
//      i-th, in rounds: each pending lane takes the r-th best available
//      expert of its row, r being the number of its token's rows on earlier
//      pending lanes (a token's rows are adjacent and see the same available
//      experts, so they pick distinct ones), and the lanes are accepted in
//      order up to the first one whose expert the lanes before it filled.
//      An accepted expert becomes NaN in the later rows of the same token,
//      a full expert in every row of the chunk.  The first pending lane is
//      always accepted, so a batch takes at most 64 rounds;
//   C. kcount becomes the final rows per expert; offsets and tiles as pass 2.
// xdest[a] / xrel[a] (overflow assignments only) receive the new expert (or
// -1) and the row inside its range.
// ---------------------------------------------------------------------------
constexpr int kRerouteThreads = 1024;
constexpr int kRerouteLds = kWave * (kMaxExperts + 1);   // floats of staged scores
constexpr int kRerouteRows = 1792;   // rows staged at most: kRerouteLds / 9, floor to 64
// QN: best experts a row keeps from one scan (k rounded up to 2, 4, 6 or 8:
// a token has at most k - 1 rows ahead of any of its rows).
template <int QN>
__global__ __launch_bounds__(kRerouteThreads) void dispatch_reroute_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ blkbase, const float* __restrict__ logits, int64_t TK,
    int k, int E, int C, int32_t* __restrict__ kcount, int32_t* __restrict__ offsets,
    int bm, Tile* __restrict__ tiles, int32_t* __restrict__ ntiles,
    int32_t* __restrict__ tstart, int32_t* __restrict__ ovf, int32_t* __restrict__ xdest,
    int32_t* __restrict__ xrel) {
  __shared__ float srow[kRerouteLds];
  __shared__ int sa[kRerouteRows];
  __shared__ int fill[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int toff[kMaxExperts + 1];
  constexpr int U = 16;   // assignments per thread per pass of A
  __shared__ int wsum[U][kRerouteThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nwaves = blockDim.x / kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = tid; e < E; e += blockDim.x) fill[e] = kcount[e];

  // A. overflow assignments in flat order, U per thread per pass (their
  // loads in flight together)
  int64_t n = 0;
  for (int64_t base = 0; base < TK; base += U * blockDim.x) {
    bool over[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t a = base + u * blockDim.x + tid;
      over[u] = false;
      if (a < TK) {
        const int e = topk_idx[a];
        if (e >= 0 && e < E)
          over[u] = blkbase[(a / kDispatchChunk) * E + e] + lrank[a] >= C;
      }
      const uint64_t b = __ballot(over[u]);
      if (lane == 0) wsum[u][wave] = __popcll(b);
    }
    __syncthreads();
    int64_t before = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t a = base + u * blockDim.x + tid;
      int64_t mine = before, total = 0;
      for (int w = 0; w < nwaves; ++w) {
        const int c = wsum[u][w];
        if (w < wave) mine += c;
        total += c;
      }
      const uint64_t b = __ballot(over[u]);
      if (over[u]) ovf[n + mine + __popcll(b & lt)] = static_cast<int32_t>(a);
      before += total;
    }
    n += before;
    __syncthreads();
  }

  // B. the greedy pass
  const int E8 = (E + 7) & ~7;     // scanned columns; those >= E are never available
  const int stride = E8 + 1;       // odd: the 64 lanes' rows fall in distinct LDS banks
  const int R = min(kRerouteRows, kRerouteLds / stride / kWave * kWave);
  const float kNaN = __builtin_nanf("");
  int64_t room = 0;   // free slots left over all experts (wavefront 0)
  if (wave == 0) {
    for (int e = lane; e < E; e += kWave) room += C - fill[e];
    for (int sh = kWave / 2; sh >= 1; sh >>= 1) room += __shfl_xor(room, sh);
  }
  for (int64_t cbase = 0; cbase < n; cbase += R) {
    const int rows = static_cast<int>(min<int64_t>(R, n - cbase));
    // the tokens' scores (NaN read as -infinity), NaN where the expert is
    // full; element-wise over all threads
    for (int i = tid; i < rows * E8; i += blockDim.x) {
      const int r = i / E8;
      const int c = i - r * E8;
      const int a = ovf[cbase + r];
      if (c == 0) sa[r] = a;
      float v = kNaN;
      if (c < E && fill[c] < C) {
        v = logits[static_cast<int64_t>(a / k) * E + c];
        v = (v != v) ? -INFINITY : v;
      }
      srow[r * stride + c] = v;
    }
    __syncthreads();
    // NaN at the token's own choices, and at the spare experts its overflow
    // assignments of earlier chunks (before the chunk's first row, a0) were
    // sent to; the chunk's own rows are excluded as they are placed
    const int a0 = sa[0];
    for (int i = tid; i < rows * k; i += blockDim.x) {
      const int r = i / k;
      const int a = sa[r];
      const int aj = a - a % k + (i - r * k);
      const int c = topk_idx[aj];
      if (c >= 0 && c < E) {
        srow[r * stride + c] = kNaN;
        if (aj < a0 && blkbase[(aj / kDispatchChunk) * E + c] + lrank[aj] >= C) {
          const int x = xdest[aj];
          if (x >= 0 && x < E) srow[r * stride + x] = kNaN;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int ebits = E > 1 ? 32 - __clz(E - 1) : 0;   // bits of an expert index
      const int qmax = min(k, kWave);   // a token's rows lie within k lanes
      for (int b0 = 0; b0 < rows; b0 += kWave) {
        const bool have = b0 + lane < rows;
        const int a = have ? sa[b0 + lane] : 0;
        const int tok = have ? a / k : -1;
        const float* row = srow + (b0 + lane) * stride;
        bool pending = have;
        // The row's best available experts at its last scan, best first
        // (ncand of them; `more`: the scan found others beyond QN).
        // Availability only shrinks, so entries are re-checked, not rescanned.
        int cand[QN];
#pragma unroll
        for (int i = 0; i < QN; ++i) cand[i] = -1;
        int ncand = 0;
        bool more = false, known = false;
        // Every round accepts at least the first pending lane (rank 0, an
        // available expert or none), so 64 rounds suffice; the bound only
        // guards against a hang.
        for (int round = 0; round <= kWave && __ballot(pending); ++round) {
          // rows of the same token on earlier pending lanes: this row takes
          // the token's rank-th best available expert (all of a token's
          // pending rows see the same available experts)
          int rank = 0;
          for (int q = 1; q < qmax; ++q) {
            const int src = lane >= q ? lane - q : lane;
            const int tq = __shfl(tok, src);
            const int pq = __shfl(pending ? 1 : 0, src);
            if (lane >= q && pq && tq == tok) ++rank;
          }
          int pick = -1, nvalid = 0;
          if (pending && known) {
#pragma unroll
            for (int i = 0; i < QN; ++i) {
              if (i < ncand) {
                const int c = cand[i];
                const float v = row[c];
                if (fill[c] < C && v == v) {
                  if (nvalid == rank) pick = c;
                  ++nvalid;
                }
              }
            }
          }
          const bool scan = pending && (!known || (pick < 0 && more));
          if (__ballot(scan)) {
            if (scan) {
              ncand = 0;
              more = false;
              if (room > 0) {
                // strict > over ascending indices keeps the lower index on
                // ties; NaN (unavailable) is skipped; -infinity ranks after
                // every number, by index
                float cv[QN];
                int ci[QN];
#pragma unroll
                for (int i = 0; i < QN; ++i) {
                  cv[i] = 0.f;
                  ci[i] = -1;
                }
                int navail = 0;
                for (int c0 = 0; c0 < E8; c0 += 8) {
                  float v8[8];
#pragma unroll
                  for (int u = 0; u < 8; ++u) v8[u] = row[c0 + u];
#pragma unroll
                  for (int u = 0; u < 8; ++u) {
                    const float v = v8[u];
                    if (v == v) {
                      ++navail;
                      bool bt[QN];
#pragma unroll
                      for (int i = 0; i < QN; ++i) bt[i] = ci[i] < 0 || v > cv[i];
#pragma unroll
                      for (int i = QN - 1; i >= 1; --i) {
                        if (bt[i - 1]) {
                          cv[i] = cv[i - 1];
                          ci[i] = ci[i - 1];
                        } else if (bt[i]) {
                          cv[i] = v;
                          ci[i] = c0 + u;
                        }
                      }
                      if (bt[0]) {
                        cv[0] = v;
                        ci[0] = c0 + u;
                      }
                    }
                  }
                }
                ncand = min(navail, QN);
                more = navail > QN;
#pragma unroll
                for (int i = 0; i < QN; ++i) cand[i] = ci[i];
              }
              known = true;
              pick = -1;
#pragma unroll
              for (int i = 0; i < QN; ++i)
                if (i == rank && i < ncand) pick = cand[i];
            }
          }
          // no pick: dropped when the token has no expert left for this row;
          // with candidates beyond the cached ones, the row waits for the
          // token's earlier rows (`again`: accepted no further this round)
          const bool again = pending && pick < 0 && more;
          const int cur = pending ? pick : -1;
          // lanes before this one (in this round) that picked the same expert
          const bool valid = cur >= 0;
          const int e = valid ? cur : 0;
          uint64_t match = __ballot(valid);
          for (int bit = 0; bit < ebits; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t m = __ballot(on);
            match &= on ? m : ~m;
          }
          const int fb = valid ? fill[e] : 0;
          const int ahead = __popcll(match & lt);
          const uint64_t clash = __ballot((valid && fb + ahead >= C) || again);
          const int first = clash ? __ffsll(static_cast<unsigned long long>(clash)) - 1 : kWave;
          const bool accept = pending && lane < first;
          if (accept) {
            xdest[a] = cur;
            xrel[a] = valid ? fb + ahead : -1;
          }
          const uint64_t took = __ballot(accept && valid);
          const uint64_t mine = match & took;
          const bool leader = accept && valid &&
                              __ffsll(static_cast<unsigned long long>(mine)) - 1 == lane;
          const int nfill = fb + __popcll(mine);
          __builtin_amdgcn_wave_barrier();
          if (leader) fill[e] = nfill;
          room -= __popcll(took);
          pending = pending && !accept;
          // the expert an accepted row took is no longer available to the
          // token's later rows: NaN in their staged scores
          if (accept && valid) {
            for (int q = 1; q < k; ++q) {
              const int r2 = b0 + lane + q;
              if (r2 >= rows || sa[r2] / k != tok) break;
              srow[r2 * stride + e] = kNaN;
            }
          }
          // experts this round filled up: unavailable in every row of the chunk
          uint64_t filled = __ballot(leader && nfill >= C);
          while (filled) {
            const int l = __ffsll(static_cast<unsigned long long>(filled)) - 1;
            filled &= filled - 1;
            const int cf = __shfl(e, l);
            for (int r = lane; r < rows; r += kWave) srow[r * stride + cf] = kNaN;
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
    __syncthreads();
  }

  // C. final rows per expert, offsets, tiles
  for (int e = tid; e < E; e += blockDim.x) kcount[e] = fill[e];
  slot_offsets_and_tiles(fill, E, bm, off, toff, offsets, tiles, ntiles, tstart);
}

// ---------------------------------------------------------------------------
// Dispatch, pass 3: final rank = chunk base + rank in chunk; kept iff
// rank < C; slot = offsets[e] + rank; perm[slot] = a.  Unused perm entries
// (from offsets[E] on) are set to -1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ lrank,
    const int32_t* __restrict__ blkbase, const int32_t* __restrict__ offsets,
    int64_t TK, int E, int C, int32_t* __restrict__ slot,
    int32_t* __restrict__ perm, const int32_t* __restrict__ xdest,
    const int32_t* __restrict__ xrel) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (a >= TK) return;
  const int e = topk_idx[a];
  const int total = offsets[E];
  if (a >= total) perm[a] = -1;
  if (e < 0 || e >= E) {  // not produced by the top-k pass; never dispatched
    slot[a] = -1;
    return;
  }
  const int64_t chunk = a / kDispatchChunk;
  const int rank = blkbase[chunk * E + e] + lrank[a];
  if (rank < C) {
    const int s = offsets[e] + rank;
    slot[a] = s;
    perm[s] = static_cast<int32_t>(a);
  } else if (xdest && xdest[a] >= 0) {   // rerouted to a spare expert
    const int s = offsets[xdest[a]] + xrel[a];
    slot[a] = s;
    perm[s] = static_cast<int32_t>(a);
  } else {
    slot[a] = -1;
  }
}

hipError_t launch_dispatch(const int32_t* topk_idx, int64_t TK, int E, int C,
                           int32_t* lrank, int32_t* blkcnt, int32_t* counts,
                           int32_t* kcount, int32_t* offsets, int32_t* slot,
                           int32_t* perm, int bm, Tile* tiles, int32_t* ntiles,
                           int32_t* tstart, const Reroute* rr, hipStream_t s) {
  const int nblk = static_cast<int>((TK + kDispatchChunk - 1) / kDispatchChunk);
  dispatch_rank_kernel<<<nblk, kRankWaves * kWave, 0, s>>>(topk_idx, TK, E, lrank, blkcnt);
  dispatch_scan_kernel<<<1, 256, 0, s>>>(blkcnt, nblk, E, C, counts, kcount,
                                         offsets, bm, tiles, ntiles, tstart);
  if (rr) {
#define MOE_REROUTE(QN)                                                                   \
  dispatch_reroute_kernel<QN><<<1, kRerouteThreads, 0, s>>>(                               \
      topk_idx, lrank, blkcnt, rr->logits, TK, rr->k, E, C, kcount, offsets, bm, tiles, ntiles, \
      tstart, rr->ovf, rr->xdest, rr->xrel)
    if (rr->k <= 2) MOE_REROUTE(2);
    else if (rr->k <= 4) MOE_REROUTE(4);
    else if (rr->k <= 6) MOE_REROUTE(6);
    else MOE_REROUTE(8);
#undef MOE_REROUTE
  }
  dispatch_scatter_kernel<<<(TK + 255) / 256, 256, 0, s>>>(
      topk_idx, lrank, blkcnt, offsets, TK, E, C, slot, perm, rr ? rr->xdest : nullptr,
      rr ? rr->xrel : nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Short batches (T <= kSmallT, T*k <= kSmallTK): top-k gating and the whole
// dispatch in one workgroup of 1024 threads, with the same results as the
// top-k pass and the three dispatch passes above.
//   1. top-k and gates per token (topk_token), chosen experts kept in LDS,
//      softmax statistics reduced into Ppart[0..E) and Hpart[0];
//   2. each of the 16 wavefronts ranks a contiguous chunk of the T*k
//      assignments (ballot matching as in pass 1, per-wavefront counters);
//   3. per expert, chunk bases in chunk order, counts, capacity; offsets and
//      the M-tile list as in pass 2;
//   4. slot / perm as in pass 3.
// ---------------------------------------------------------------------------
constexpr int kSmallWaves = 16;
template <int V>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ lpart, int nsplit, int64_t split_stride,
    const float* __restrict__ bias, float* __restrict__ logits_out, int T, int E, int k,
    int G, int gating, int renorm, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ Ppart, float* __restrict__ Hpart, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ kcount,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ perm,
    int bm, Tile* __restrict__ tiles, int32_t* __restrict__ ntiles,
    int32_t* __restrict__ tstart) {
  __shared__ int sidx[kSmallTK];
  __shared__ int srank[kSmallTK];
  __shared__ int ccnt[kSmallWaves][kMaxExperts];
  __shared__ float pbuf[1024 * 4];   // [groups][E], groups*E <= 1024*V
  __shared__ float hbuf[1024];
  __shared__ int kc[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int toff[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int TK = T * k;

  // 1. top-k and gates
  {
    const int gl = tid % G;
    const int grp = tid / G;
    const int ngroups = blockDim.x / G;
    float pacc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) pacc[v] = 0.f;
    float hacc = 0.f;
    for (int t = grp; t < T; t += ngroups)
      topk_token<V>(t, lpart, nsplit, split_stride, bias, logits_out, E, k, G, gl, gating,
                    renorm, topk_idx, topk_w, sidx, pacc, hacc);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int i = gl + v * G;
      if (i < E) pbuf[grp * E + i] = pacc[v];
    }
    if (gl == 0) hbuf[grp] = hacc;
    for (int i = tid; i < kSmallWaves * E; i += blockDim.x) ccnt[i / E][i % E] = 0;
    __syncthreads();
    // groups from T on took no token and hold zeros: the sums stop before them
    const int gused = min(ngroups, T);
    for (int e = tid; e < E; e += blockDim.x) {
      float sp = 0.f;
      for (int g = 0; g < gused; ++g) sp += pbuf[g * E + e];
      Ppart[e] = sp;
    }
    if (tid == 0) {
      float sh = 0.f;
      for (int g = 0; g < gused; ++g) sh += hbuf[g];
      Hpart[0] = sh;
    }
  }

  // 2. stable ranks within each wavefront's chunk of assignments
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int chunk = ((TK + kSmallWaves - 1) / kSmallWaves + kWave - 1) / kWave * kWave;
  {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int* cnt = ccnt[wave];
    for (int it = 0; it < chunk; it += kWave) {
      const int a = wave * chunk + it + lane;
      const int ein = a < TK ? sidx[a] : -1;
      const bool valid = ein >= 0 && ein < E;
      const int e = valid ? ein : 0;
      uint64_t match = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        match &= bit ? m : ~m;
      }
      const int before = valid ? cnt[e] : 0;
      __builtin_amdgcn_wave_barrier();
      const bool leader = valid && (__ffsll(static_cast<unsigned long long>(match)) - 1 == lane);
      if (leader) cnt[e] = before + __popcll(match);
      __builtin_amdgcn_wave_barrier();
      if (valid) srank[a] = before + __popcll(match & lt);
    }
  }
  __syncthreads();

  // 3. chunk bases, counts, capacity, offsets, M-tiles
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < kSmallWaves; ++w) {
      const int c = ccnt[w][e];
      ccnt[w][e] = run;
      run += c;
    }
    counts[e] = run;
    kc[e] = min(run, C);
    kcount[e] = kc[e];
  }
  __syncthreads();
  slot_offsets_and_tiles(kc, E, bm, off, toff, offsets, tiles, ntiles, tstart);

  // 4. slots and the permutation (unused entries -1)
  const int total = off[E];
  for (int a = tid; a < TK; a += blockDim.x) {
    if (a >= total) perm[a] = -1;
    const int e = sidx[a];
    if (e < 0 || e >= E) {
      slot[a] = -1;
      continue;
    }
    const int rank = ccnt[a / chunk][e] + srank[a];
    if (rank < C) {
      const int sl = off[e] + rank;
      slot[a] = sl;
      perm[sl] = a;
    } else {
      slot[a] = -1;
    }
  }
}

hipError_t launch_route_small(const float* lpart, int nsplit, int64_t split_stride,
                              const float* bias, float* logits_out, int T, int E, int k,
                              int gating, int renorm, int32_t* topk_idx, float* topk_w,
                              float* Ppart, float* Hpart, int C, int32_t* counts,
                              int32_t* kcount, int32_t* offsets, int32_t* slot,
                              int32_t* perm, int bm, Tile* tiles, int32_t* ntiles,
                              int32_t* tstart, hipStream_t s) {
  if (T <= 0 || T > kSmallT || T * k > kSmallTK) return hipErrorInvalidValue;
  const int G = topk_group_size(E);
  const int V = (E + G - 1) / G;
#define MOE_SMALL_ARGS                                                                 \
  lpart, nsplit, split_stride, bias, logits_out, T, E, k, G, gating, renorm, topk_idx, \
      topk_w, Ppart, Hpart, C, counts, kcount, offsets, slot, perm, bm, tiles, ntiles, tstart
  if (V <= 1)
    route_small_kernel<1><<<1, 1024, 0, s>>>(MOE_SMALL_ARGS);
  else if (V <= 2)
    route_small_kernel<2><<<1, 1024, 0, s>>>(MOE_SMALL_ARGS);
  else
    route_small_kernel<4><<<1, 1024, 0, s>>>(MOE_SMALL_ARGS);
#undef MOE_SMALL_ARGS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Statistics (one workgroup): sums the softmax partial rows in a fixed
// order and forms, in double precision,
//   f_i = counts_i / (T k), P_i = mean_t p[t, i], aux = E sum f_i P_i,
//   aux over kept counts, overflow = dropped / (T k),
//   H_load = -sum f_i ln f_i, H_tok = mean_t H_t.
// out[0..5] = aux, aux_kept, overflow, H_load, H_tok, dropped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stats_kernel(
    const float* __restrict__ Ppart, const float* __restrict__ Hpart, int nblk,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kcount,
    int64_t T, int k, int E, double* __restrict__ out) {
  __shared__ double red[5][256];
  const int tid = threadIdx.x;
  const double n = static_cast<double>(T) * k;
  // Thread e: P_e from the partial rows, 8 interleaved running sums (their
  // loads in flight together) added in a fixed order; then its expert's
  // terms of aux, aux over kept counts, the load entropy and the drops.
  double terms[4] = {0.0, 0.0, 0.0, 0.0};
  if (tid < E) {
    double s8[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        s8[u] += static_cast<double>(Ppart[static_cast<int64_t>(b + u) * E + tid]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (b + u < nblk) s8[u] += static_cast<double>(Ppart[static_cast<int64_t>(b + u) * E + tid]);
    double sum = 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += s8[u];
    const double P = sum / static_cast<double>(T);
    const double f = counts ? counts[tid] / n : 0.0;
    const double fk = kcount ? kcount[tid] / n : 0.0;
    terms[0] = f * P;
    terms[1] = fk * P;
    terms[2] = f > 0.0 ? -f * log(f) : 0.0;
    terms[3] = (counts && kcount) ? static_cast<double>(counts[tid] - kcount[tid]) : 0.0;
  }
  // the per-token entropy partials, strided over the workgroup
  double h = 0.0;
  for (int b = tid; b < nblk; b += blockDim.x) h += static_cast<double>(Hpart[b]);
#pragma unroll
  for (int q = 0; q < 4; ++q) red[q][tid] = terms[q];
  red[4][tid] = h;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {   // fixed tree
    if (tid < w)
#pragma unroll
      for (int q = 0; q < 5; ++q) red[q][tid] += red[q][tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    out[0] = E * red[0][0];
    out[1] = E * red[1][0];
    out[2] = red[3][0] / n;
    out[3] = red[2][0];
    out[4] = red[4][0] / static_cast<double>(T);
    out[5] = red[3][0];
  }
}

hipError_t launch_stats(const float* Ppart, const float* Hpart, int nblk,
                        const int32_t* counts, const int32_t* kcount, int64_t T,
                        int k, int E, double* out, hipStream_t s) {
  stats_kernel<<<1, 256, 0, s>>>(Ppart, Hpart, nblk, counts, kcount, T, k, E, out);
  return hipGetLastError();
}

}  // namespace moe
