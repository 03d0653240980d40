// Gate-weighted combine for libmoe (gfx950).
//
// out[t] = sum over j with slot[t,j] >= 0 of w[t,j] * Y[slot[t,j]]
//          + (shared-expert sum for token t)
// [MoE wiki] "Mixture of experts" (wikiprompt.org), "How it works": the chosen
// experts' outputs are combined, weighted by the router's confidence;
// [Routing guide] "MoE routing, fully explained" (allinfo.ai.kr), "Plain
// explanation" para 4: shared experts see every token; para 3: a dropped
// assignment is simply not computed, so it adds nothing (the surviving gates
// are not rescaled).
//
// Y rows are fp32 and may be split into `ysplit` partial sums over K
// (weight-streaming path); the partials are added in a fixed order, so
// results are bitwise reproducible.  One workgroup per token, columns strided
// over threads so each Y row is read with coalesced 16-byte loads.  With one
// part, the loads of all k rows of a column group are issued before the
// first is used (the kernel is bound by memory latency, not by arithmetic),
// and the sum is taken in j order.  The output is stored rounded to bf16
// (RNE) or as the fp32 sum itself; both kernels form the same fp32 sum, so a
// bf16 output is exactly the rounding of the fp32 one.
#include "kernels.h"

namespace moe {
namespace {

// NB: K parts loaded together (in flight at once), then added in part order.
template <bool BF16OUT, int NB>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ Y, int ysplit, int64_t ysplit_stride,
    const int32_t* __restrict__ slot, const float* __restrict__ topk_w,
    const float* __restrict__ Ys, int ys_split, int64_t ys_stride, int64_t T,
    int k, int d, void* __restrict__ out) {
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  const bool vec = (d & 3) == 0;
  const int ncols = vec ? d / 4 : d;
  // blockIdx.y picks a chunk of blockDim.x columns (float4 units when d % 4 == 0)
  for (int c = blockIdx.y * blockDim.x + threadIdx.x; c < ncols; c += gridDim.y * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int s = slot[t * k + j];
      if (s < 0) continue;
      const float w = topk_w[t * k + j];
      float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
      // the parts are loaded NB at a time (their loads in flight together)
      // and added in part order
      for (int p0 = 0; p0 < ysplit; p0 += NB) {
        float4 v[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (p0 + u < ysplit) {
            const float* row = Y + (p0 + u) * ysplit_stride + static_cast<int64_t>(s) * d;
            if (vec) v[u] = reinterpret_cast<const float4*>(row)[c];
            else v[u].x = row[c];
          }
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (p0 + u < ysplit) {
            y.x += v[u].x; y.y += v[u].y; y.z += v[u].z; y.w += v[u].w;
          }
        }
      }
      acc.x = fmaf(w, y.x, acc.x);
      acc.y = fmaf(w, y.y, acc.y);
      acc.z = fmaf(w, y.z, acc.z);
      acc.w = fmaf(w, y.w, acc.w);
    }
    if (Ys) {
      for (int p = 0; p < ys_split; ++p) {
        const float* row = Ys + p * ys_stride + t * d;
        if (vec) {
          const float4 v = reinterpret_cast<const float4*>(row)[c];
          acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        } else {
          acc.x += row[c];
        }
      }
    }
    if (BF16OUT) {
      uint16_t* o = static_cast<uint16_t*>(out) + t * d;
      if (vec) {
        const uint32_t lo = f32_to_bf16(acc.x) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
        const uint32_t hi = f32_to_bf16(acc.z) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
        reinterpret_cast<uint2*>(o)[c] = make_uint2(lo, hi);
      } else {
        o[c] = f32_to_bf16(acc.x);
      }
    } else {
      float* o = static_cast<float*>(out) + t * d;
      if (vec) reinterpret_cast<float4*>(o)[c] = acc;
      else o[c] = acc.x;
    }
  }
}

// One K part, d % 8 == 0: each thread takes 8 columns (two 16-byte loads per
// row).  Up to 8 rows' loads are in flight at once; the weighted sum runs in
// j order with the same operations as combine_kernel, so the two give the
// same bits.
template <bool BF16OUT>
__global__ __launch_bounds__(512) void combine_rows_kernel(
    const float* __restrict__ Y, const int32_t* __restrict__ slot,
    const float* __restrict__ topk_w, const float* __restrict__ Ys, int ys_split,
    int64_t ys_stride, int64_t T, int k, int d, void* __restrict__ out) {
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  const int ncols = d / 8;
  const int32_t* st = slot + t * k;
  const float* wt = topk_w + t * k;
  for (int c = blockIdx.y * blockDim.x + threadIdx.x; c < ncols; c += gridDim.y * blockDim.x) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      float4 v[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v[u][0] = v[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j0 + u < k) {
          const int s = st[j0 + u];
          if (s >= 0) {
            const float4* row = reinterpret_cast<const float4*>(Y + static_cast<int64_t>(s) * d);
            v[u][0] = row[2 * c];
            v[u][1] = row[2 * c + 1];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < k && st[j0 + u] >= 0) {
          const float w = wt[j0 + u];
          const float y[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w,
                              v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, 0.f + y[e], acc[e]);
        }
      }
    }
    if (Ys) {
      for (int p = 0; p < ys_split; ++p) {
        const float4* row = reinterpret_cast<const float4*>(Ys + p * ys_stride + t * d);
        const float4 a = row[2 * c], b = row[2 * c + 1];
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
      }
    }
    if (BF16OUT) {
      uint4 o;
      o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
      o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
      o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
      o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + t * d)[c] = o;
    } else {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + t * d);
      o[2 * c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      o[2 * c + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* Y, int ysplit, int64_t ysplit_stride,
                          const int32_t* slot, const float* topk_w,
                          const float* Ys, int ys_split, int64_t ys_stride,
                          int64_t T, int k, int d, void* out, bool bf16out,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (ysplit == 1 && (d & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    // 8 columns per thread; at most 512 threads per token, as few passes as
    // possible with the threads evenly loaded.  Short batches: 64-thread
    // workgroups over 64 column groups each.
    const int n8 = d / 8;
    int tpb, chunks;
    if (T < 64) {
      tpb = 64;
      chunks = (n8 + 63) / 64;
    } else {
      const int passes = (n8 + 511) / 512;
      tpb = ((n8 + passes - 1) / passes + 63) / 64 * 64;
      chunks = 1;
    }
    const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(chunks));
    if (bf16out)
      combine_rows_kernel<true><<<grid, tpb, 0, s>>>(Y, slot, topk_w, Ys, ys_split, ys_stride,
                                                    T, k, d, out);
    else
      combine_rows_kernel<false><<<grid, tpb, 0, s>>>(Y, slot, topk_w, Ys, ys_split, ys_stride,
                                                     T, k, d, out);
    return hipGetLastError();
  }
  // enough workgroups to cover the GPU even for a handful of tokens: short
  // batches take 64-thread workgroups, each over 64 column groups
  const int ncols = (d & 3) == 0 ? d / 4 : d;
  const int tpb = T < 64 ? 64 : 256;
  int chunks = (ncols + tpb - 1) / tpb;
  if (T >= 256) chunks = 1;
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(chunks));
  // parts loaded together: as many as there are, up to 16 (registers)
#define MOE_COMBINE_NB(O, NB)                                                          \
  combine_kernel<O, NB><<<grid, tpb, 0, s>>>(Y, ysplit, ysplit_stride, slot, topk_w, Ys, \
                                             ys_split, ys_stride, T, k, d, out)
#define MOE_COMBINE(O)                  \
  if (ysplit <= 2) MOE_COMBINE_NB(O, 2); \
  else if (ysplit <= 8) MOE_COMBINE_NB(O, 8); \
  else MOE_COMBINE_NB(O, 16)
  if (bf16out) { MOE_COMBINE(true); }
  else { MOE_COMBINE(false); }
#undef MOE_COMBINE
#undef MOE_COMBINE_NB
  return hipGetLastError();
}

}  // namespace moe
