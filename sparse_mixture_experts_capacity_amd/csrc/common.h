// Internal helpers shared by the libmoe HIP kernels (gfx950 / CDNA4).
// Not part of the public interface (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kMaxExperts = 256;
constexpr int kDispatchChunk = 1024;  // assignments ranked by one workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte staging

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the top half of the
// fp32 bits).  Narrowing rounds to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element loaders for the two storage types.
__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, int64_t i, float v) {
  p[i] = f32_to_bf16(v);
}

// silu(u) = u * sigmoid(u) = u / (1 + e^-u).  For very negative u, e^-u
// overflows to +inf and the quotient is -0, the correct limit.
__device__ __forceinline__ float silu_f32(float u) { return u / (1.0f + __expf(-u)); }
__device__ __forceinline__ float silu_f32_accurate(float u) { return u / (1.0f + expf(-u)); }

// Logical block index with consecutive indices placed on the same XCD.
// Hardware deals workgroups round-robin over the 8 XCDs of an MI355X; the
// grid size must be a multiple of 8.
__device__ __forceinline__ int xcd_local_block(int p, int nblocks) {
  return (p & 7) * (nblocks >> 3) + (p >> 3);
}

// Tile descriptor of one M-tile of a grouped GEMM: rows row0 .. row0+nrows-1
// (in slot space) of group (expert) `group`.
struct Tile {
  int32_t group;
  int32_t row0;
  int32_t nrows;
  int32_t pad;
};

}  // namespace moe
