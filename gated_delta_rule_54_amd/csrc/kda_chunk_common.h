// kda_chunk_common.h -- device helpers shared by the chunkwise forward
// (kda_chunk.hip) and backward (kda_chunk_bwd.hip) kernels: element
// conversions, the MFMA operand conventions and operand-order layouts, and
// the chunk geometry of dense and varlen batches.  Each translation unit gets
// its own internal copy (anonymous namespace).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <stdint.h>

namespace kda {
namespace {

constexpr int kC = 64;            // chunk length
constexpr int kThreads = 256;     // 4 waves
constexpr float kNormEps = 1e-6f;
constexpr float kFastDecayBound = -80.f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __hip_bfloat16 bf16;

// ---------------------------------------------------------------------------
// Element helpers.  bf16 values are handled as raw 16-bit patterns (no
// class-typed objects in LDS or unions); rounding is round-to-nearest-even.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint16_t bf_bits(float x) {
  return __bfloat16_as_ushort(__float2bfloat16(x));
}
__device__ __forceinline__ float bf_val(uint32_t b) { return __uint_as_float(b << 16); }
// Two values to a bf16 pair (v_cvt_pk_bf16_f32, round-to-nearest-even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// One fp32 value stored as an element of the MFMA type (bf16: rounded to
// nearest even, as the packed conversion of the operand fragments rounds).
__device__ __forceinline__ void st_elem(bf16* p, float x) {
  *reinterpret_cast<uint16_t*>(p) = bf_bits(x);
}
__device__ __forceinline__ void st_elem(float* p, float x) { *p = x; }

__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const bf16* p) {
  return bf_val(*reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ void st_f(float* p, float x) { *p = x; }
__device__ __forceinline__ void st_f(bf16* p, float x) {
  *reinterpret_cast<uint16_t*>(p) = bf_bits(x);
}

// Store 4 consecutive elements (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
// Load 4 consecutive elements as floats.
__device__ __forceinline__ f32x4_t ld4(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  return f32x4_t{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ f32x4_t ld4(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4_t{bf_val(u.x & 0xffffu), bf_val(u.x >> 16), bf_val(u.y & 0xffffu),
                 bf_val(u.y >> 16)};
}
// Four consecutive elements kept as raw bits until use (a prefetch must not
// convert at load time: that would wait for the load).
template <typename T> struct Raw4;
template <> struct Raw4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ f32x4_t get() const { return f32x4_t{v.x, v.y, v.z, v.w}; }
};
template <> struct Raw4<bf16> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ f32x4_t get() const {
    return f32x4_t{bf_val(v.x & 0xffffu), bf_val(v.x >> 16), bf_val(v.y & 0xffffu),
                   bf_val(v.y >> 16)};
  }
};
// Two consecutive elements kept as raw bits until use.
template <typename T> struct Raw2;
// Buffer-resource forms (load(rsrc, off)): off is the byte offset of the pair;
// a pair past the resource's bound reads as zero.  aux 2 = non-temporal.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <> struct Raw2<float> {
  float2 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
  __device__ __forceinline__ float2 get() const { return v; }
  __device__ __forceinline__ void set(float a, float b) { v = make_float2(a, b); }
};
template <> struct Raw2<bf16> {
  uint32_t v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ float2 get() const { return make_float2(bf_val(v & 0xffffu), bf_val(v >> 16)); }
  // two values rounded to bf16 (nearest even) in place of the loaded pair
  __device__ __forceinline__ void set(float a, float b) { v = pack_bf16x2(a, b); }
};
// Two consecutive elements as raw bits through a non-temporal load: for
// inputs read once, so that they do not displace data that is read again
// soon (the chunk records the state pass reads right after) in the caches.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <typename T> struct RawNt2;
template <> struct RawNt2<float> {
  f32x2_t v;
  __device__ __forceinline__ void load(const float* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(p));
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
  }
  __device__ __forceinline__ float2 get() const { return make_float2(v[0], v[1]); }
  __device__ __forceinline__ void set(float a, float b) { v = f32x2_t{a, b}; }
};
template <> struct RawNt2<bf16> {
  uint32_t v;
  __device__ __forceinline__ void load(const bf16* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    v = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2);
  }
  __device__ __forceinline__ float2 get() const { return make_float2(bf_val(v & 0xffffu), bf_val(v >> 16)); }
  __device__ __forceinline__ void set(float a, float b) { v = pack_bf16x2(a, b); }
};
// Load N consecutive elements (16-byte aligned, N a multiple of 8) as floats.
template <int N>
__device__ __forceinline__ void ld_seg(const float* p, float* out) {
#pragma unroll
  for (int j = 0; j < N; j += 4) {
    const float4 v = *reinterpret_cast<const float4*>(p + j);
    out[j] = v.x; out[j + 1] = v.y; out[j + 2] = v.z; out[j + 3] = v.w;
  }
}
template <int N>
__device__ __forceinline__ void ld_seg(const bf16* p, float* out) {
#pragma unroll
  for (int j = 0; j < N; j += 8) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + j);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      out[j + 2 * t] = bf_val(v[t] & 0xffffu);
      out[j + 2 * t + 1] = bf_val(v[t] >> 16);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA 16x16 tiles.  Lane l of a wave supplies, for operand A (M x K), row
// l%16 and KPL consecutive k starting at KPL*(l/16); operand B (K x N) the
// same with column l%16.  The accumulator holds rows 4*(l/16)+j, j = 0..3, of
// column l%16.  Both operands are therefore read from buffers whose rows are
// the tile's non-K index with k contiguous.
template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32, KPL = 8;
  using frag = bf16x8_t;
  static __device__ __forceinline__ frag load(const bf16* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const u32x4_t*>(p));
  }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 4, KPL = 1;
  using frag = float;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4_t mma(frag a, frag b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Word 3 of the raw buffer resources used here (untyped 32-bit data).
constexpr int kRsrcWord3 = 0x00020000;
// A byte offset (1 GiB) past a resource's bound reads zeros without touching
// memory.  Where the zeros are relied on (the state pass's record resource)
// the bound is at most one segment's records, 160 MiB; where they are not
// (lanes whose value is unused) a larger bound only costs a read.
constexpr uint32_t kPastBound = 0x40000000u;

// One operand fragment (a lane's KPL elements) through a buffer resource:
// off is the lane's byte offset, soff a scalar byte offset.
template <typename T> struct BufFrag;
template <> struct BufFrag<bf16> {
  static __device__ __forceinline__ bf16x8_t load(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                  uint32_t soff) {
    return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
  }
};
template <> struct BufFrag<float> {
  static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
  }
};

// LDS-direct load: 16 bytes per lane from the buffer into LDS at lds + 16 *
// lane (one 1 KiB block per wave and instruction).
__device__ __forceinline__ void dma_load16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}
// s_waitcnt operand that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt is 6 bits: low 4 at [3:0], high 2 at
// [15:14]) and leaves expcnt and lgkmcnt alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier for the state passes.  __syncthreads() carries a workgroup
// release fence, which in a producer wave must also wait for every
// LDS-direct load in flight (they write LDS) and would drain its prefetch;
// here each wave waits only for its own LDS reads and writes (lgkmcnt), the
// hardware barrier follows, and the empty asm statements keep the compiler
// from moving LDS accesses across it.  A producer wave waits for the loads
// the compute waves are about to read with an explicit vmcnt before the
// barrier (see the state passes).
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left as they are
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Fragment of rows [row0, row0+16) and k-step ks of a row-major buffer.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_at(const T* base, int ld, int row0, int ks,
                                                         int lane) {
  return Mma<T>::load(base + (int64_t)(row0 + (lane & 15)) * ld + ks * Mma<T>::KSTEP +
                      Mma<T>::KPL * (lane >> 4));
}

// The summed index k of a product may be permuted freely as long as both
// operands use the same permutation.  Operands that K2 loads use the one
// below inside each k-step: position kpos(k) holds index k.  It is chosen so
// that the four consecutive accumulator rows 4*(l/16)+j a lane holds form
// one contiguous piece of an operand fragment when the accumulator's rows
// are the k index -- the intra-chunk kernel then stores its products
// directly in operand order, and K2 loads each fragment as 64 lanes x KPL
// contiguous elements.
//   bf16 (k-step 32): position 8g+e holds k = 4g+e (e < 4), 16+4g+(e-4) (e >= 4)
//   fp32 (k-step 4, blocks of 16): position 4s+g holds k = 4g+s
template <typename T> __device__ __forceinline__ int kpos(int k);
template <> __device__ __forceinline__ int kpos<bf16>(int k) {
  const int cc = k & 31;
  return (k & ~31) + ((cc & 15) >> 2) * 8 + (cc >> 4) * 4 + (cc & 3);
}
template <> __device__ __forceinline__ int kpos<float>(int k) {
  const int cc = k & 15;
  return (k & ~15) + (cc & 3) * 4 + (cc >> 2);
}
// Operand-order ("fragment-native") matrix with rows m and nks k-steps:
// 16-row tile, then k-step, then the 64 lanes' KPL elements.  Element (m, k):
template <typename T>
__device__ __forceinline__ int fnat(int m, int k, int nks) {
  using M = Mma<T>;
  const int p = kpos<T>(k);
  const int q = p % M::KSTEP;
  return (((m >> 4) * nks + p / M::KSTEP) * 64 + (m & 15) + 16 * (q / M::KPL)) * M::KPL +
         q % M::KPL;
}
// Record of one (head, chunk slot): the operands the state pass reads,
// written by the intra-chunk kernel (or, for the backward's states-only pass,
// by the backward's per-chunk preparation).
template <typename T, int D>
struct Rec {
  // element offsets inside a record (in units of T), then gamma (fp32).
  // QG, KT, WN and P are fragment-native (see fnat) with the k index named;
  // U is stored as 16x16 accumulator tiles [n/16][r/16][lane][4].  A state
  // pass without output reads only KT, WN, UT and e^gamma.
  static constexpr int64_t QG = 0;                 // rows r, k = channel: q^ o e^G
  static constexpr int64_t KT = QG + kC * D;       // rows channel, k = r: k^ o e^(gamma-G)
  static constexpr int64_t WN = KT + D * kC;       // rows r, k = channel: -Wk
  static constexpr int64_t UT = WN + kC * D;       // U (rows r, columns n) as tiles
  static constexpr int64_t P = UT + D * kC;        // rows r, k = i: P (zero for i > r)
  static constexpr int64_t END = P + kC * kC;
  static constexpr int64_t BYTES_T = END * (int64_t)sizeof(T);
  static constexpr int64_t BYTES = ((BYTES_T + D * 4 + 255) / 256) * 256;  // + e^gamma
};

// Stores of k-runs of row m into a fragment-native matrix (k0 % 4 == 0 for
// runs of 4, k0 % 8 == 0 for runs of 8, k0 even for pairs).  For bf16 a run
// of 4 is one 8-byte piece; fp32 scatters.
__device__ __forceinline__ void st_fnat4(bf16* base, int nks, int m, int k0, float a, float b,
                                         float c, float d) {
  *reinterpret_cast<uint2*>(base + fnat<bf16>(m, k0, nks)) =
      make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st_fnat4(float* base, int nks, int m, int k0, float a, float b,
                                         float c, float d) {
  base[fnat<float>(m, k0, nks)] = a;
  base[fnat<float>(m, k0 + 1, nks)] = b;
  base[fnat<float>(m, k0 + 2, nks)] = c;
  base[fnat<float>(m, k0 + 3, nks)] = d;
}
template <typename T>
__device__ __forceinline__ void st_fnat8(T* base, int nks, int m, int k0, const float* x) {
  st_fnat4(base, nks, m, k0, x[0], x[1], x[2], x[3]);
  st_fnat4(base, nks, m, k0 + 4, x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void st_fnat2(bf16* base, int nks, int m, int k0, float a, float b) {
  *reinterpret_cast<uint32_t*>(base + fnat<bf16>(m, k0, nks)) = pack_bf16x2(a, b);
}
__device__ __forceinline__ void st_fnat2(float* base, int nks, int m, int k0, float a, float b) {
  base[fnat<float>(m, k0, nks)] = a;
  base[fnat<float>(m, k0 + 1, nks)] = b;
}
// Four consecutive k (k0 % 4 == 0) into an LDS row whose columns follow kpos.
__device__ __forceinline__ void st_perm4(bf16* row, int k0, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(row + kpos<bf16>(k0)) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void st_perm4(float* row, int k0, float a, float b, float c, float d) {
  row[kpos<float>(k0)] = a;
  row[kpos<float>(k0 + 1)] = b;
  row[kpos<float>(k0 + 2)] = c;
  row[kpos<float>(k0 + 3)] = d;
}

// 16x16 fp32 tile product through MFMA: acc += A[ra.., ka..] * B[kb.., cb..],
// A and B fp32 in LDS (row-major, leading dim lda / ldb), K = 16.
__device__ __forceinline__ f32x4_t mm16_f32(const float* A, int lda, const float* B, int ldb,
                                            f32x4_t acc, int lane) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const float a = A[(lane & 15) * lda + ks * 4 + (lane >> 4)];
    const float b = B[(ks * 4 + (lane >> 4)) * ldb + (lane & 15)];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
  return acc;
}
// Store a 16x16 accumulator tile (rows 4*(l/16)+j, column l%16) into LDS.
__device__ __forceinline__ void st_tile_f32(float* C, int ldc, f32x4_t v, float sgn, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) C[(4 * (lane >> 4) + j) * ldc + (lane & 15)] = sgn * v[j];
}

// Unit lower triangular inverse T = (I + A)^-1 of a 64 x 64 strictly lower
// A, both fp32 in LDS with leading dimension kTriLd; uses 1024 floats of
// LDS scratch and at least 4 waves, and must be reached by every thread of
// the workgroup (it contains __syncthreads).  With scratch == nullptr the
// intermediate products are kept in T's blocks above the 16 x 16 diagonal
// blocks instead, which are then left undefined (T is lower triangular;
// the caller reads only its lower triangle).  The 16 x 16 diagonal blocks are
// inverted by forward substitution (wave 0, one lane per block column), then
// the blocks below the diagonal follow from T_ij = -T_ii (sum_k A_ik T_kj):
// first within each 32 x 32 half, then the lower-left 32 x 32 quarter.
constexpr int kTriLd = 64 + 4;
__device__ __forceinline__ void tri_inv64(const float* sA, float* sT, float* scratch, int wave,
                                          int lane) {
  constexpr int LD = kTriLd;
  if (wave == 0) {
    // diagonal 16x16 blocks by forward substitution; lane = (block, column)
    const int b = lane >> 4, col = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == col) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= sA[(b * 16 + r) * LD + b * 16 + i] * x[i];
      x[r] = acc;
      sT[(b * 16 + r) * LD + b * 16 + col] = acc;
    }
  }
  __syncthreads();
  // level 1: T_10 = -T_11 A_10 T_00 (wave 0), T_32 = -T_33 A_32 T_22 (wave 1)
  if (wave < 2) {
    const int b0 = wave * 32;  // the 32x32 diagonal block
    // in place: the block above T_10, rows b0.., columns b0+16..
    float* xs = scratch ? scratch + wave * 256 : sT + b0 * LD + b0 + 16;
    const int ldx = scratch ? 16 : LD;
    f32x4_t x = mm16_f32(sA + (b0 + 16) * LD + b0, LD, sT + b0 * LD + b0, LD,
                         f32x4_t{0.f, 0.f, 0.f, 0.f}, lane);
    st_tile_f32(xs, ldx, x, 1.f, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4_t y = mm16_f32(sT + (b0 + 16) * LD + b0 + 16, LD, xs, ldx,
                         f32x4_t{0.f, 0.f, 0.f, 0.f}, lane);
    st_tile_f32(sT + (b0 + 16) * LD + b0, LD, y, -1.f, lane);
  }
  __syncthreads();
  // level 2: T[32:64, 0:32] = -T_low A[32:64, 0:32] T_high; waves 0..3 own
  // one 16x16 output tile each (rows 32 + 16*(w/2), cols 16*(w%2)); every
  // wave takes part in the barrier between the two products
  {
    const bool active = wave < 4;
    const int tr = 32 + 16 * ((wave & 3) >> 1), tc = 16 * (wave & 1);
    // 32x32 X; in place: T's upper-right quarter, rows 0..31, columns 32..63
    float* xs = scratch ? scratch : sT + 32;
    const int ldx = scratch ? 32 : LD;
    if (active) {
      f32x4_t x = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // X = A[tr.., 0:32] T_high[0:32, tc..]: T_high is lower triangular, so
      // only k-blocks >= tc/16 contribute
      for (int kb = tc / 16; kb < 2; ++kb)
        x = mm16_f32(sA + tr * LD + kb * 16, LD, sT + (kb * 16) * LD + tc, LD, x, lane);
      st_tile_f32(xs + (tr - 32) * ldx + tc, ldx, x, 1.f, lane);
    }
    __syncthreads();
    if (active) {
      // Y = T_low[tr.., 32:64] X[0:32, tc..]: T_low lower triangular, k-blocks <= tr
      f32x4_t y = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int kb = 0; kb <= (tr - 32) / 16; ++kb)
        y = mm16_f32(sT + tr * LD + 32 + kb * 16, LD, xs + (kb * 16) * ldx + tc, ldx, y, lane);
      st_tile_f32(sT + tr * LD + tc, LD, y, -1.f, lane);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Per-chunk states handed from the forward pass and the reverse pass to the
// backward's per-chunk kernel are stored slice-blocked: [D/16][D][16], i.e.
// the 16-column slices one state-pass workgroup owns are contiguous (each
// step writes whole lines), rows c inside a slice, columns n last.
template <int D>
__device__ __forceinline__ int sblk(int c, int n) {
  return ((n >> 4) * D + c) * 16 + (n & 15);
}

// ---------------------------------------------------------------------------
// Where a chunk slot lives in the token stream.  Slots number the chunks of
// all sequences back to back: dense sequence b owns slots [b*spq, (b+1)*spq)
// with spq = ceil(T/64); varlen sequence n owns [chunk_off[n], chunk_off[n+1]).
struct ChunkGeom {
  const int32_t* cu;          // varlen: sanitised cu_seqlens (device); dense: nullptr
  const int32_t* chunk_off;   // varlen: [N+1] chunk offsets (device)
  int64_t T;                  // dense: tokens per sequence
  int64_t spq;                // dense: chunk slots per sequence
  int32_t N;
};

struct ChunkLoc { int64_t tok0; int len; int seq; };

// Slot range, first token and token count of sequence `seq`.
struct SeqSpan { int64_t c0, c1, tok0, ntok; };
__device__ __forceinline__ SeqSpan seq_span(const ChunkGeom& gm, int seq) {
  if (gm.cu == nullptr)
    return SeqSpan{(int64_t)seq * gm.spq, (int64_t)(seq + 1) * gm.spq, (int64_t)seq * gm.T, gm.T};
  return SeqSpan{gm.chunk_off[seq], gm.chunk_off[seq + 1], gm.cu[seq],
                 (int64_t)gm.cu[seq + 1] - gm.cu[seq]};
}

__device__ __forceinline__ bool locate(const ChunkGeom& gm, int64_t slot, ChunkLoc& L) {
  int n;
  if (gm.cu == nullptr) {
    if (gm.spq == 0) return false;
    n = (int)(slot / gm.spq);
    if (n >= gm.N) return false;
  } else {
    if (slot >= gm.chunk_off[gm.N]) return false;
    int lo = 0, hi = gm.N;  // find n with chunk_off[n] <= slot < chunk_off[n+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (gm.chunk_off[mid] <= slot) lo = mid; else hi = mid;
    }
    n = lo;
  }
  const SeqSpan sp = seq_span(gm, n);
  const int64_t off = (slot - sp.c0) * kC;
  L.seq = n;
  L.tok0 = sp.tok0 + off;
  L.len = (int)min<int64_t>(kC, sp.ntok - off);
  return L.len > 0;
}

// Varlen chunk map, one workgroup.  The caller's cu_seqlens are not trusted:
// each entry is clamped to [0, T] and made non-decreasing (a running max), so
// no later kernel can address a token outside [0, T).  For valid input the
// sanitised offsets equal cu_seqlens.  Then chunk_off[n] = sum_(m<n)
// ceil(len_m / 64), the first chunk slot of sequence n.
__global__ __launch_bounds__(kThreads) void kda_chunk_map(const int32_t* __restrict__ cu, int N,
                                                          int64_t T, int32_t* __restrict__ cu_s,
                                                          int32_t* __restrict__ chunk_off) {
  __shared__ int32_t s_scan[kThreads];
  __shared__ int32_t s_carry_max, s_carry_sum;
  const int tid = threadIdx.x;
  if (tid == 0) { s_carry_max = 0; s_carry_sum = 0; }
  __syncthreads();
  // pass 1: sanitised offsets (inclusive max-scan of clamped values)
  for (int n0 = 0; n0 <= N; n0 += kThreads) {
    const int n = n0 + tid;
    int32_t x = 0;
    if (n <= N) x = (int32_t)min<int64_t>(max<int64_t>((int64_t)cu[n], 0), T);
    s_scan[tid] = x;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int32_t other = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] = max(s_scan[tid], other);
      __syncthreads();
    }
    if (n <= N) cu_s[n] = max(s_scan[tid], s_carry_max);
    __syncthreads();
    if (tid == 0) s_carry_max = max(s_carry_max, s_scan[kThreads - 1]);
    __syncthreads();
  }
  // pass 2: chunk offsets (exclusive sum-scan of per-sequence chunk counts)
  for (int n0 = 0; n0 < N; n0 += kThreads) {
    const int n = n0 + tid;
    int32_t c = 0;
    if (n < N) c = (cu_s[n + 1] - cu_s[n] + kC - 1) / kC;
    s_scan[tid] = c;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int32_t add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    if (n < N) chunk_off[n + 1] = s_carry_sum + s_scan[tid];
    __syncthreads();
    if (tid == 0) s_carry_sum += s_scan[kThreads - 1];
    __syncthreads();
  }
  if (tid == 0) chunk_off[0] = 0;
}

}  // namespace
}  // namespace kda
