// kda_epilogue.hip -- the operator's output epilogue on gfx950: head-wise
// RMSNorm times a sigmoid output gate.
//
// Pages cited (by title and section):
//   [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
//        §6 layer diagram (KDA -> RMSNorm -> sigmoid output gate -> output
//        projection) and §6.3 (the output is normalised per head, then
//        multiplied by a sigmoid gate computed from the input).
//
// Per (token, head) row of d_v outputs:
//   y_j = o_j / sqrt(mean_i o_i^2 + eps) * w_j * sigmoid(z_j)
// eps and the per-channel weight w (shared by the heads) are not fixed by the
// pages; they are arguments.  A row is one 16-byte access per lane for a
// group of DV / (16 / sizeof(T)) lanes; the mean square is reduced across the
// group with lane shuffles, so a row is read once and written once: the
// kernel is a pure HBM stream (6 bytes per element at bf16 plus w).  Each
// wave issues the loads of four row groups before any of their math, to keep
// enough bytes in flight per CU.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef unsigned int u32x4e_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2e_t __attribute__((ext_vector_type(2)));
constexpr int kEpiThreads = 64;
constexpr int kEpiUnroll = 4;       // row groups per wave with loads in flight together
// one-wave workgroups, as many as the rows need up to 16384 (one pass each
// for 262144 rows of 128; beyond that a grid-stride loop): measured ~7 %
// faster than 2048 workgroups of four waves making two passes
constexpr int kEpiMaxBlocks = 16384;

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int E = 4;  // elements per 16 bytes
  static __device__ __forceinline__ void unpack(u32x4e_t v, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(v[e]);
  }
  static __device__ __forceinline__ u32x4e_t pack(const float* x) {
    return u32x4e_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                    __float_as_uint(x[3])};
  }
};
template <> struct Vec<__hip_bfloat16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(u32x4e_t v, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(v[e] << 16);
      x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4e_t pack(const float* x) {
    u32x4e_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2e_t p = {(__bf16)x[2 * e], (__bf16)x[2 * e + 1]};
      v[e] = __builtin_bit_cast(unsigned int, p);
    }
    return v;
  }
};

template <typename T, int DV>
__global__ __launch_bounds__(kEpiThreads) void gate_norm_kernel(
    const T* __restrict__ o, const T* __restrict__ z, const float* __restrict__ w, float eps,
    T* y, int64_t rows) {
  using V = Vec<T>;
  constexpr int E = V::E, LPR = DV / E, RPW = 64 / LPR;  // lanes per row, rows per wave
  constexpr int U = kEpiUnroll;                          // row groups in flight per wave
  constexpr int RPB = (kEpiThreads / 64) * RPW * U;      // rows per workgroup pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  float wv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) wv[e] = w ? w[li * E + e] : 1.f;
  for (int64_t r0 = (int64_t)blockIdx.x * RPB; r0 < rows; r0 += (int64_t)gridDim.x * RPB) {
    // all U row groups' loads first (clamped, so every lane loads), then math
    u32x4e_t ov[U], zv[U];
    int64_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + (wave * U + u) * RPW + sub;
      off[u] = (r < rows ? r : rows - 1) * DV + li * E;
      ov[u] = *reinterpret_cast<const u32x4e_t*>(o + off[u]);
      zv[u] = *reinterpret_cast<const u32x4e_t*>(z + off[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + (wave * U + u) * RPW + sub;
      float x[E], g[E];
      V::unpack(ov[u], x);
      V::unpack(zv[u], g);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss += x[e] * x[e];
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = rsqrtf(ss * (1.f / DV) + eps);
#pragma unroll
      for (int e = 0; e < E; ++e)
        x[e] = x[e] * inv * wv[e] * __builtin_amdgcn_rcpf(1.f + __expf(-g[e]));
      // y is not read here again: stored non-temporally (measured ~2 % faster;
      // non-temporal loads of o and z measured slower)
      if (r < rows) __builtin_nontemporal_store(V::pack(x), reinterpret_cast<u32x4e_t*>(y + off[u]));
    }
  }
}

template <typename T, int DV>
hipError_t launch_typed(int64_t rows, const void* o, const void* z, const float* w, float eps,
                        void* y, hipStream_t stream) {
  constexpr int RPB = (kEpiThreads / 64) * (64 / (DV / Vec<T>::E)) * kEpiUnroll;
  const int64_t want = (rows + RPB - 1) / RPB;
  const unsigned blocks = (unsigned)(want < kEpiMaxBlocks ? want : kEpiMaxBlocks);
  hipLaunchKernelGGL((gate_norm_kernel<T, DV>), dim3(blocks), dim3(kEpiThreads), 0, stream,
                     static_cast<const T*>(o), static_cast<const T*>(z), w, eps,
                     static_cast<T*>(y), rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_norm(int64_t rows, int dv, int dtype, const void* o, const void* z,
                            const float* w, float eps, void* y, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const bool bf = dtype == KDA_DTYPE_BF16;
  if (dv == 128)
    return bf ? launch_typed<__hip_bfloat16, 128>(rows, o, z, w, eps, y, stream)
              : launch_typed<float, 128>(rows, o, z, w, eps, y, stream);
  return bf ? launch_typed<__hip_bfloat16, 64>(rows, o, z, w, eps, y, stream)
            : launch_typed<float, 64>(rows, o, z, w, eps, y, stream);
}

}  // namespace kda
