// kda_chunk_bwd.hip -- chunkwise KDA backward (input gradients) for gfx950.
//
// Pages cited (by title and section):
//   [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
//
// [XT §5] has training run the same chunkwise form as prefill but gives no
// gradient algorithm; what follows is the vector-Jacobian product of the
// chunk form written out in kda_chunk.hip (same notation, one chunk of n <= 64
// rows, entering state S, leaving state S', scale folded into dO' = scale dO):
//
//   Kp = K^ o e^G   Km = K^ o e^-G   Qp = Q^ o e^G   K~ = K^ o e^(gamma-G)
//   A  = Diag(beta) tril_-1(Kp Km^T)   T = (I + A)^-1   P = tril(Qp Km^T)
//   W  = T Diag(beta) (V - Kp S)        O = scale (Qp S + P W)
//   S' = Diag(e^gamma) S + K~^T W
//
// Given dO and dS' = dL/dS', with dW = P^T dO' + K~ dS' (what reaches W) and
// L = T^T dW (the adjoint of the triangular solve (I + A) W = beta (V - Kp S)):
//   dV     = Diag(beta) L
//   dbeta  = rowsum(L o (V - Kp S)) + rowsum(dA o Kp Km^T),  dA = -tril_-1(L W^T)
//   dQp    = dO' S^T + dP Km,                                dP = tril(dO' W^T)
//   dKp    = -Diag(beta) L S^T + dB Km,                      dB = Diag(beta) dA
//   dKm    = dB^T Kp + dP^T Qp
//   dK~    = W dS'^T
//   dgamma = colsum(dK~ o K~) + e^gamma o rowsum(S o dS')
//   dS     = Diag(e^gamma) dS' + Qp^T dO' - Kp^T Diag(beta) L
//          = M dS' + Z^T dO',   M = Diag(e^gamma) - Wk^T K~,  Z = Qp - P Wk,
//                               Wk = T Diag(beta) Kp
// and through the gates and the norm (per element, then per row / column):
//   dk^ = dKp o e^G + dKm o e^-G + dK~ o e^(gamma-G)      dq^ = dQp o e^G
//   dG  = k^ o (dKp o e^G - dKm o e^-G - dK~ o e^(gamma-G)) + q^ o dq^
//         (+ dgamma on the chunk's last row: gamma = G_63, rows past the
//          sequence's end carry g = 0)
//   dg_r = sum_(s>=r) dG_s      (the in-chunk prefix sum, reversed)
//   dk  = r_k (dk^ - (k^ . dk^) k^),  r_k = (|k|^2 + eps)^(-1/2)   (q alike)
// Gated DeltaNet mode (one gate per token and head) sums dg over channels.
//
// Launches, all on the caller's stream:
//   1. the forward (kda_chunk.hip) with o off and every chunk's entering
//      state S written to the workspace;
//   2. kda_bwd_prep, one workgroup per (chunk, head): M and Z^T in operand
//      order for the reverse pass;
//   3. kda_bwd_state_pass, one workgroup per (sequence, head, 16 columns of
//      d_v), sequential over the sequence's chunks from the last: dS' of every
//      chunk to the workspace, dS of the first to d_init_state;
//   4. kda_bwd_intra, one workgroup per (chunk, head): every gradient above.
// The per-chunk kernels recompute the chunk's operands (norms, G, A, T, P)
// rather than store them.
//
// Operand layouts.  A workgroup of D/16 waves gives wave w the 16 columns
// [16w, 16w+16) of every chunk x d matrix, all 64 rows, in MFMA accumulator
// layout (lane: column l%16, rows 16t + 4(l/16) + j).  A product whose summed
// index is the chunk row can take such an accumulator straight as an operand
// (see acc_frag) when the other operand is read with the same row order
// (the kpos permutation of kda_chunk_common.h); everything else is staged in
// LDS in the MFMA type.
//
// Domain: the split exponentials e^G, e^-G need every chunk's per-channel
// decay gamma >= -80 (the forward's fast-path bound); beyond it the backward's
// results are unspecified (no fault, no hang).  fp32 operands at d = 128 do
// not fit one workgroup's LDS and are not supported.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <algorithm>

#include "kda_internal.h"
#include "kda_chunk_common.h"

namespace kda {
namespace {

// ---------------------------------------------------------------------------
// Operand fragments beyond frag_at (k contiguous along rows):
//   frag_cm       element (m, k) = X[k * ld + m]        (k strided)
//   frag_rm_perm  element (m, k) = X[m * ld + k], k in kpos order
//   frag_cm_perm  element (m, k) = X[k * ld + m], k in kpos order
//   acc_frag      operand whose k index is the row index of four stacked
//                 16-row accumulator tiles, in kpos order (no data movement)
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_cm(const T* X, int ld, int m0, int ks,
                                                         int lane);
template <>
__device__ __forceinline__ bf16x8_t frag_cm<bf16>(const bf16* X, int ld, int m0, int ks,
                                                  int lane) {
  const uint16_t* p =
      reinterpret_cast<const uint16_t*>(X) + (ks * 32 + 8 * (lane >> 4)) * ld + m0 + (lane & 15);
  u32x4_t u;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    u[t] = (uint32_t)p[(2 * t) * ld] | ((uint32_t)p[(2 * t + 1) * ld] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}
template <>
__device__ __forceinline__ float frag_cm<float>(const float* X, int ld, int m0, int ks, int lane) {
  return X[(ks * 4 + (lane >> 4)) * ld + m0 + (lane & 15)];
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_rm_perm(const T* X, int ld, int m0, int ks,
                                                              int lane);
template <>
__device__ __forceinline__ bf16x8_t frag_rm_perm<bf16>(const bf16* X, int ld, int m0, int ks,
                                                       int lane) {
  const bf16* row = X + (m0 + (lane & 15)) * ld + ks * 32 + 4 * (lane >> 4);
  const uint2 a = *reinterpret_cast<const uint2*>(row);
  const uint2 b = *reinterpret_cast<const uint2*>(row + 16);
  return __builtin_bit_cast(bf16x8_t, (u32x4_t{a.x, a.y, b.x, b.y}));
}
template <>
__device__ __forceinline__ float frag_rm_perm<float>(const float* X, int ld, int m0, int ks,
                                                     int lane) {
  return X[(m0 + (lane & 15)) * ld + 16 * (ks >> 2) + 4 * (lane >> 4) + (ks & 3)];
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_cm_perm(const T* X, int ld, int m0, int ks,
                                                              int lane);
template <>
__device__ __forceinline__ bf16x8_t frag_cm_perm<bf16>(const bf16* X, int ld, int m0, int ks,
                                                       int lane) {
  const uint16_t* p =
      reinterpret_cast<const uint16_t*>(X) + (ks * 32 + 4 * (lane >> 4)) * ld + m0 + (lane & 15);
  u32x4_t u;
  u[0] = (uint32_t)p[0] | ((uint32_t)p[ld] << 16);
  u[1] = (uint32_t)p[2 * ld] | ((uint32_t)p[3 * ld] << 16);
  u[2] = (uint32_t)p[16 * ld] | ((uint32_t)p[17 * ld] << 16);
  u[3] = (uint32_t)p[18 * ld] | ((uint32_t)p[19 * ld] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}
template <>
__device__ __forceinline__ float frag_cm_perm<float>(const float* X, int ld, int m0, int ks,
                                                     int lane) {
  return X[(16 * (ks >> 2) + 4 * (lane >> 4) + (ks & 3)) * ld + m0 + (lane & 15)];
}

// Eight (bf16) or one (fp32) fp32 values to an operand fragment.
__device__ __forceinline__ bf16x8_t to_frag(const float* x, bf16) {
  const u32x4_t u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ float to_frag(const float* x, float) { return x[0]; }

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag acc_frag(const f32x4_t* tiles, int ks) {
  if constexpr (sizeof(T) == 2) {
    const float x[8] = {tiles[2 * ks][0],     tiles[2 * ks][1],     tiles[2 * ks][2],
                        tiles[2 * ks][3],     tiles[2 * ks + 1][0], tiles[2 * ks + 1][1],
                        tiles[2 * ks + 1][2], tiles[2 * ks + 1][3]};
    return to_frag(x, T{});
  } else {
    return tiles[ks >> 2][ks & 3];
  }
}

// The operand fragment of row m at k-step ks (k = column, contiguous) of a
// slice-blocked D x D state stored in the MFMA type (sblk; KPL <= 8 columns
// never cross a 16-column slice): one 16-byte load (bf16) or one element.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag grow_frag(const T* X, int m, int ks, int lane) {
  using M = Mma<T>;
  const T* p = X + sblk<D>(m, ks * M::KSTEP + M::KPL * (lane >> 4));
  if constexpr (M::KPL == 8) {
    return __builtin_bit_cast(typename M::frag, *reinterpret_cast<const u32x4_t*>(p));
  } else {
    return p[0];
  }
}
// Element e of a fragment as fp32.
__device__ __forceinline__ float frag_val(bf16x8_t f, int e) {
  const u32x4_t u = __builtin_bit_cast(u32x4_t, f);
  return (e & 1) ? __uint_as_float(u[e >> 1] & 0xffff0000u) : __uint_as_float(u[e >> 1] << 16);
}
__device__ __forceinline__ float frag_val(float f, int) { return f; }
// KPL raw elements (ld_raw bits) to an operand fragment.
__device__ __forceinline__ bf16x8_t raw_frag(const uint32_t* x, bf16) {
  const u32x4_t u = {x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16),
                     x[6] | (x[7] << 16)};
  return __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ float raw_frag(const uint32_t* x, float) { return __uint_as_float(x[0]); }

// One element as raw bits (a load whose value is converted only at use does
// not make the wave wait where it is issued), and its value.
__device__ __forceinline__ uint32_t ld_raw(const bf16* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}
__device__ __forceinline__ uint32_t ld_raw(const float* p) { return __float_as_uint(*p); }
__device__ __forceinline__ uint32_t ld_raw_nt(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ uint32_t ld_raw_nt(const float* p) {
  return __float_as_uint(__builtin_nontemporal_load(p));
}
template <typename T>
__device__ __forceinline__ float raw_val(uint32_t b) {
  if constexpr (sizeof(T) == 2) return bf_val(b);
  else return __uint_as_float(b);
}

// Gradient outputs are written once and read by nobody here: non-temporal
// stores, so they do not push out of the caches the chunk's S, dS', k, q and
// g that the workgroup reads again.
__device__ __forceinline__ void st_nt(bf16* p, float x) {
  __builtin_nontemporal_store(bf_bits(x), reinterpret_cast<uint16_t*>(p));
}
__device__ __forceinline__ void st_nt(float* p, float x) { __builtin_nontemporal_store(x, p); }

// Sum over the 16 lanes of a lane group (the 16 columns of an accumulator).
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------------------
// LDS of the per-chunk backward kernels (bytes).  kda_bwd_intra (COMPACT =
// false) keeps every operand for the whole kernel; kda_bwd_prep (COMPACT)
// needs Kp, Km, Qp only until A and P are formed, so the fp32 A and T of the
// inverse, and then K~, reuse their region, and two workgroups fit a CU.
template <typename T, int D, bool COMPACT = false>
struct BwdLds {
  static constexpr int NW = D / 16, NT = 64 * NW;  // waves (one per 16 columns), threads
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int LDX = D + PAD, LDC = kC + PAD;  // leading dims: C x D, C x C
  static constexpr int XB = kC * LDX * (int)sizeof(T);
  static constexpr int CB = kC * LDC * (int)sizeof(T);
  static constexpr int FB = kC * kTriLd * 4;  // fp32 A or T of the inverse
  static constexpr int UB = 2 * (XB > FB ? XB : FB);
  static_assert(CB >= 4096, "the inverse's scratch lives in the dB buffer");
  // full layout: Kp, Km, Qp, K~ (later L); union {A, T fp32} then {W, dO'};
  // T, P (later dP), dB; small fp32 arrays
  // compact layout: {Kp, Km, Qp} then {A, T, scratch} then {K~}; T, P; small
  static constexpr int R0 = (3 * XB > 2 * FB + 4096) ? 3 * XB : 2 * FB + 4096;
  static constexpr int KP = 0, KM = XB, QP = 2 * XB;
  static constexpr int KT = COMPACT ? 0 : 3 * XB;
  static constexpr int U = COMPACT ? 0 : 4 * XB;
  static constexpr int TB = COMPACT ? R0 : U + UB;
  static constexpr int PB = TB + CB;
  static constexpr int DB = COMPACT ? -1 : PB + CB;
  static constexpr int SCR = COMPACT ? 2 * FB : DB;
  static constexpr int SM = COMPACT ? PB + CB : DB + CB;
  // small: beta, rk, rq, x0, x1, x2 [kC] and red [2][NW][kC]
  static constexpr int BYTES = SM + (6 * kC + 2 * NW * kC) * 4;
  static_assert(BYTES <= 160 * 1024, "per-chunk backward LDS exceeds a CU");
};

template <typename T, int D, bool COMPACT = false>
struct BwdSmem {
  using L = BwdLds<T, D, COMPACT>;
  T *kp, *km, *qp, *kt, *tb, *pb, *db, *wb, *dob;
  float *sA, *sT, *scratch, *beta, *rk, *rq, *x0, *x1, *x2, *red;
  __device__ explicit BwdSmem(char* s) {
    kp = reinterpret_cast<T*>(s + L::KP);
    km = reinterpret_cast<T*>(s + L::KM);
    qp = reinterpret_cast<T*>(s + L::QP);
    kt = reinterpret_cast<T*>(s + L::KT);
    sA = reinterpret_cast<float*>(s + L::U);
    sT = sA + kC * kTriLd;
    wb = reinterpret_cast<T*>(s + L::U);
    dob = reinterpret_cast<T*>(s + L::U + L::XB);
    tb = reinterpret_cast<T*>(s + L::TB);
    pb = reinterpret_cast<T*>(s + L::PB);
    db = COMPACT ? nullptr : reinterpret_cast<T*>(s + L::DB);
    scratch = reinterpret_cast<float*>(s + L::SCR);
    beta = reinterpret_cast<float*>(s + L::SM);
    rk = beta + kC;
    rq = rk + kC;
    x0 = rq + kC;
    x1 = x0 + kC;
    x2 = x1 + kC;
    red = x2 + kC;
  }
};

// Registers the prologue leaves to its kernel, in accumulator layout (wave w:
// column c = 16w + l%16, rows 16t + 4(l/16) + j).
struct BwdRegs {
  float G[4][4];   // in-chunk prefix sum of g
  float kh[4][4];  // k^ (0 past the chunk's end)
  float qh[4][4];  // q^
  float gam;       // gamma of this lane's column
};

// Raw k, q, g of this lane's column and rows (zero past the chunk's end).
// NTL: read non-temporally (the caller reads them once).
template <typename T, int D, bool GS, bool NTL = false>
__device__ __forceinline__ void load_cols(const T* __restrict__ q, const T* __restrict__ k,
                                          const float* __restrict__ g, const ChunkLoc& loc, int H,
                                          int h, int c, int grp, BwdRegs& R, float (&gr)[4][4]) {
  // uniform bases (the chunk's first row) and 32-bit per-lane offsets
  const int64_t row0 = loc.tok0 * H + h;
  const T* kb = k + row0 * D;
  const T* qb = q + row0 * D;
  const float* gb = GS ? g + row0 : g + row0 * D;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      const int off = min(r, loc.len - 1) * H * D + c;
      const bool ok = r < loc.len;
      const float* gp = GS ? gb + min(r, loc.len - 1) * H : gb + off;
      if constexpr (NTL) {
        R.kh[t][j] = ok ? raw_val<T>(ld_raw_nt(kb + off)) : 0.f;
        R.qh[t][j] = ok ? raw_val<T>(ld_raw_nt(qb + off)) : 0.f;
        gr[t][j] = ok ? __builtin_nontemporal_load(gp) : 0.f;
      } else {
        R.kh[t][j] = ok ? ld_f(kb + off) : 0.f;
        R.qh[t][j] = ok ? ld_f(qb + off) : 0.f;
        gr[t][j] = ok ? *gp : 0.f;
      }
    }
}

// Prologue loads: the chunk's k, q and g rows in coalesced 16-byte pieces
// through buffer resources bounded at the chunk's last valid row (rows past
// it read as zero), the q/k row norms reduced across the lanes that hold each
// row, and the raw rows staged in LDS for reads in the column layout: k at
// byte 0, g (fp32) at XB, q at 3 XB -- space no layout uses before the gated
// operands are written.  NTL: read non-temporally (read once).
template <typename T, int D, bool GS, bool NTL>
__device__ __forceinline__ void stage_rows(const T* q, const T* k, const float* g,
                                           const ChunkLoc& loc, int H, int h, int qk_l2norm,
                                           char* stage, float* rk, float* rq) {
  using L = BwdLds<T, D>;
  constexpr int NT = L::NT, LDX = L::LDX, LDG = D + 4;
  constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int PR = D / VE, NPK = kC * PR / NT;    // k, q: pieces per row, per thread
  constexpr int PRG = D / 4, NPG = kC * PRG / NT;   // g: the same
  static_assert(kC * PR % NT == 0 && kC * PRG % NT == 0 && PR <= 64 && 64 % PR == 0,
                "pieces must tile the threads, a row's pieces within one wave");
  static_assert(64 * LDG * 4 <= 2 * L::XB, "staged g must fit two regions");
  constexpr int aux = NTL ? 2 : 0;
  const int tid = threadIdx.x;
  const int rs = H * D;
  const int64_t row0 = loc.tok0 * H + h;
  const int span = (loc.len - 1) * rs + D;
  auto rsrc = [](const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
  };
  const __amdgpu_buffer_rsrc_t rkr = rsrc(k + row0 * D, span * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t rqr = rsrc(q + row0 * D, span * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t rgr =
      rsrc(GS ? g + row0 : g + row0 * D, GS ? ((loc.len - 1) * H + 1) * 4 : span * 4);
  u32x4_t kv[NPK], qv[NPK], gv[NPG];
  float gs = 0.f;
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int p = i * NT + tid, row = p / PR, cp = p % PR;
    kv[i] = __builtin_amdgcn_raw_buffer_load_b128(rkr, (uint32_t)((row * rs + cp * VE) * (int)sizeof(T)), 0, aux);
  }
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int p = i * NT + tid, row = p / PR, cp = p % PR;
    qv[i] = __builtin_amdgcn_raw_buffer_load_b128(rqr, (uint32_t)((row * rs + cp * VE) * (int)sizeof(T)), 0, aux);
  }
  if constexpr (GS) {
    gs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       rgr, (uint32_t)((tid % kC) * H * 4), 0, aux));
  } else {
#pragma unroll
    for (int i = 0; i < NPG; ++i) {
      const int p = i * NT + tid, row = p / PRG, cp = p % PRG;
      gv[i] = __builtin_amdgcn_raw_buffer_load_b128(rgr, (uint32_t)((row * rs + cp * 4) * 4), 0, aux);
    }
  }
  T* sk = reinterpret_cast<T*>(stage);
  float* sg = reinterpret_cast<float*>(stage + L::XB);
  T* sq = reinterpret_cast<T*>(stage + 3 * L::XB);
#pragma unroll
  for (int i = 0; i < NPK; ++i) {
    const int p = i * NT + tid, row = p / PR, cp = p % PR;
    float a = 0.f, b = 0.f;  // this piece's part of |k_row|^2, |q_row|^2
    // (plain fp32 arithmetic: the packed bf16 dot-product instruction gave
    // wrong sums in this kernel, so it is not used)
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float k0 = bf_val(kv[i][e] & 0xffffu), k1 = bf_val(kv[i][e] >> 16);
        const float q0 = bf_val(qv[i][e] & 0xffffu), q1 = bf_val(qv[i][e] >> 16);
        a += k0 * k0 + k1 * k1;
        b += q0 * q0 + q1 * q1;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __uint_as_float(kv[i][e]), y = __uint_as_float(qv[i][e]);
        a += x * x;
        b += y * y;
      }
    }
#pragma unroll
    for (int o = PR / 2; o >= 1; o >>= 1) {
      a += __shfl_xor(a, o);
      b += __shfl_xor(b, o);
    }
    if (cp == 0) {
      rk[row] = qk_l2norm ? rsqrtf(a + kNormEps) : 1.f;
      rq[row] = qk_l2norm ? rsqrtf(b + kNormEps) : 1.f;
    }
    *reinterpret_cast<u32x4_t*>(sk + row * LDX + cp * VE) = kv[i];
    *reinterpret_cast<u32x4_t*>(sq + row * LDX + cp * VE) = qv[i];
  }
  if constexpr (GS) {
    if (tid < kC) sg[tid * LDG] = gs;  // the row's one gate, in column 0
  } else {
#pragma unroll
    for (int i = 0; i < NPG; ++i) {
      const int p = i * NT + tid, row = p / PRG, cp = p % PRG;
      *reinterpret_cast<u32x4_t*>(sg + row * LDG + cp * 4) = gv[i];
    }
  }
}

// G = prefix sum of gr down the 64 rows of this lane's column -- within the
// lane's 4 rows, then across the 4 lane groups, then across the tiles -- and
// gamma = G of the last row.
__device__ __forceinline__ void prefix_G(const float (&gr)[4][4], int lane, BwdRegs& R) {
  const int grp = lane >> 4;
  float carry = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float loc4[4];
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) { run += gr[t][j]; loc4[j] = run; }
    float x = run;
    float y = __shfl_up(x, 16);
    if (grp >= 1) x += y;
    y = __shfl_up(x, 32);
    if (grp >= 2) x += y;
    const float excl = x - run;
    const float total = __shfl(x, 48 + (lane & 15));
#pragma unroll
    for (int j = 0; j < 4; ++j) R.G[t][j] = carry + excl + loc4[j];
    carry += total;
  }
  R.gam = carry;
}

// Prologue shared by the per-chunk backward kernels: loads, q/k norms, G,
// the gated operands in LDS (K~ left to the caller in the compact layout), A
// and P, T = (I + A)^-1 (times Diag(beta) when TBETA) in the MFMA type.  Bm receives this wave's tiles of Kp Km^T
// (tile p = wave + NW * tt: rows 16(p/4), columns 16(p%4)).
template <typename T, int D, bool GS, bool TBETA, bool COMPACT, bool NTL = false>
__device__ __forceinline__ void bwd_prologue(const T* __restrict__ q, const T* __restrict__ k,
                                             const float* __restrict__ g,
                                             const float* __restrict__ beta, const ChunkLoc& loc,
                                             int H, int h, int qk_l2norm,
                                             BwdSmem<T, D, COMPACT>& sm, BwdRegs& R,
                                             f32x4_t* Bm) {
  using L = BwdLds<T, D, COMPACT>;
  using M = Mma<T>;
  constexpr int NW = L::NW, NT = L::NT, LDX = L::LDX, LDC = L::LDC, NTW = 16 / NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
  const int c = 16 * wave + (lane & 15);
  float gr[4][4];
  {
    char* stage = reinterpret_cast<char*>(sm.kp);  // the layout's first byte
    stage_rows<T, D, GS, NTL>(q, k, g, loc, H, h, qk_l2norm, stage, sm.rk, sm.rq);
    if (tid < kC) sm.beta[tid] = tid < loc.len ? beta[(loc.tok0 + tid) * H + h] : 0.f;
    __syncthreads();
    const T* sk = reinterpret_cast<const T*>(stage);
    const float* sg = reinterpret_cast<const float*>(stage + L::XB);
    const T* sq = reinterpret_cast<const T*>(stage + 3 * L::XB);
    constexpr int LDG = D + 4;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * t + 4 * grp + j;
        R.kh[t][j] = ld_f(sk + r * LDX + c);
        R.qh[t][j] = ld_f(sq + r * LDX + c);
        gr[t][j] = GS ? sg[r * LDG] : sg[r * LDG + c];
      }
  }
  prefix_G(gr, lane, R);
  __syncthreads();
  // gated operands
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      R.kh[t][j] *= sm.rk[r];
      R.qh[t][j] *= sm.rq[r];
      const float G = R.G[t][j];
      const float eg = __expf(G), en = __expf(-G), et = __expf(R.gam - G);
      st_f(sm.kp + r * LDX + c, R.kh[t][j] * eg);
      st_f(sm.km + r * LDX + c, R.kh[t][j] * en);
      st_f(sm.qp + r * LDX + c, R.qh[t][j] * eg);
      if constexpr (!COMPACT) st_f(sm.kt + r * LDX + c, R.kh[t][j] * et);
    }
  __syncthreads();
  // A = Diag(beta) tril_-1(Kp Km^T) (fp32) and P = tril(Qp Km^T)
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt) {
    const int p = wave + NW * tt, rb = p >> 2, ib = p & 3;
    f32x4_t ab = {0.f, 0.f, 0.f, 0.f}, ap = ab;
#pragma unroll
    for (int ks = 0; ks < D / M::KSTEP; ++ks) {
      const auto bk = frag_at<T>(sm.km, LDX, 16 * ib, ks, lane);
      ab = M::mma(frag_at<T>(sm.kp, LDX, 16 * rb, ks, lane), bk, ab);
      ap = M::mma(frag_at<T>(sm.qp, LDX, 16 * rb, ks, lane), bk, ap);
    }
    Bm[tt] = ab;
    const int i = 16 * ib + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) st_f(sm.pb + (16 * rb + 4 * grp + j) * LDC + i, i <= 16 * rb + 4 * grp + j ? ap[j] : 0.f);
  }
  // A from the kept Bm tiles; in the compact layout A overlays Kp and Km, so
  // every wave must be done reading them first
  if constexpr (COMPACT) __syncthreads();
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt) {
    const int p = wave + NW * tt, rb = p >> 2, ib = p & 3;
    const int i = 16 * ib + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * rb + 4 * grp + j;
      sm.sA[r * kTriLd + i] = i < r ? sm.beta[r] * Bm[tt][j] : 0.f;
    }
  }
  __syncthreads();
  tri_inv64(sm.sA, sm.sT, sm.scratch, wave, lane);
  for (int e = tid; e < kC * kC; e += NT) {
    const int r = e >> 6, i = e & 63;
    const float t = i <= r ? sm.sT[r * kTriLd + i] : 0.f;
    st_f(sm.tb + r * LDC + i, TBETA ? t * sm.beta[i] : t);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Reverse-pass record of one (head, chunk slot): M and scale Z^T in operand
// order (see fnat), rows = key channel c, k = c' (M) or chunk row r (Z^T).
template <typename T, int D>
struct BRec {
  static constexpr int64_t MF = 0;
  static constexpr int64_t ZF = MF + (int64_t)D * D;
  static constexpr int64_t END = ZF + (int64_t)D * kC;
  static constexpr int64_t BYTES = (END * (int64_t)sizeof(T) + 255) / 256 * 256;
};

template <typename T, int D, bool GS>
__global__ __launch_bounds__((BwdLds<T, D>::NT), 1)
__attribute__((amdgpu_waves_per_eu(4))) void kda_bwd_prep(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, ChunkGeom gm, int H, int64_t nslot, int64_t slot_base,
    int qk_l2norm, float scale, char* __restrict__ brec) {
  using L = BwdLds<T, D, true>;
  using M = Mma<T>;
  using RC = BRec<T, D>;
  constexpr int NW = L::NW, LDX = L::LDX, LDC = L::LDC, NTW = 16 / NW;
  constexpr int KC = kC / M::KSTEP, KD = D / M::KSTEP;
  extern __shared__ __align__(16) char smem[];
  const int h = blockIdx.x;
  const int64_t slot = slot_base + blockIdx.y;
  ChunkLoc loc;
  if (!locate(gm, slot, loc)) return;
  BwdSmem<T, D, true> sm(smem);
  BwdRegs R;
  f32x4_t Bm[NTW];
  bwd_prologue<T, D, GS, true, true, true>(q, k, g, beta, loc, H, h, qk_l2norm, sm, R, Bm);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, grp = lane >> 4;
  const int c = 16 * wave + (lane & 15);
  // K~ into the region the inverse has finished with
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      st_f(sm.kt + (16 * t + 4 * grp + j) * LDX + c, R.kh[t][j] * __expf(R.gam - R.G[t][j]));
  __syncthreads();
  T* rec = reinterpret_cast<T*>(brec + ((int64_t)h * nslot + slot) * RC::BYTES);

  // Wk = T Diag(beta) Kp for this wave's columns, B = Kp from registers
  f32x4_t kpa[4], wk[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) kpa[t][j] = R.kh[t][j] * __expf(R.G[t][j]);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wk[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      wk[t] = M::mma(frag_rm_perm<T>(sm.tb, LDC, 16 * t, ks, lane), acc_frag<T>(kpa, ks), wk[t]);
  }
  // Z = Qp - P Wk, stored as scale Z^T (rows c, k = r; the reverse pass then
  // takes dO as it is): each lane's 4 rows are 4 consecutive k
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4_t pw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      pw = M::mma(frag_rm_perm<T>(sm.pb, LDC, 16 * t, ks, lane), acc_frag<T>(wk, ks), pw);
    float z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = scale * (R.qh[t][j] * __expf(R.G[t][j]) - pw[j]);
    st_fnat4(rec + RC::ZF, KC, c, 16 * t + 4 * grp, z[0], z[1], z[2], z[3]);
  }
  // M^T tiles (rows c', column c) = Diag(e^gamma) - K~^T Wk, stored as M
  // (rows c, k = c')
  const float egam = __expf(R.gam);
#pragma unroll
  for (int cb = 0; cb < NW; ++cb) {
    f32x4_t mt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      mt = M::mma(frag_cm_perm<T>(sm.kt, LDX, 16 * cb, ks, lane), acc_frag<T>(wk, ks), mt);
    float m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c2 = 16 * cb + 4 * grp + j;
      m[j] = (c2 == c ? egam : 0.f) - mt[j];
    }
    st_fnat4(rec + RC::MF, KD, c, 16 * cb + 4 * grp, m[0], m[1], m[2], m[3]);
  }
}

// ---------------------------------------------------------------------------
// Reverse state pass: dS = M dS' + (scale Z)^T dO chunk by chunk from the last, one
// workgroup per (sequence, head, 16 columns of d_v).  Wave w owns rows
// [16 CBW w, 16 CBW (w+1)) of dS in accumulators; dS' crosses LDS once per
// chunk (double-buffered, so one barrier per chunk).  Each chunk's dS' (the
// gradient of the state leaving it) goes to dstates for kda_bwd_intra.
constexpr int kBwdSliceW = 16;
constexpr int kBwdPassThreads = 256;

template <typename T, int D>
struct BwdPassFrags {
  using M = Mma<T>;
  static constexpr int CBW = D / 64, KD = D / M::KSTEP, KC = kC / M::KSTEP;
  // dO slice of the chunk (64 rows x 16 columns): 16 bytes per lane, VE
  // elements of one row; NO lanes hold the slice, the rest read nothing
  static constexpr int VE = 16 / (int)sizeof(T), LPR = kBwdSliceW / VE, NO = kC * LPR;
  static_assert(NO <= kBwdPassThreads, "the dO slice must fit one load per lane");
  typename M::frag mf[CBW][KD], zf[CBW][KC];
  u32x4_t dov;  // raw dO bits of row tid / LPR, columns VE (tid % LPR) ..
};

template <typename T, int D>
__global__ __launch_bounds__(kBwdPassThreads, 1) void kda_bwd_state_pass(
    const char* __restrict__ brec, int64_t nslot, ChunkGeom gm, int H, int NH, int nslice,
    const T* __restrict__ d_o, const float* __restrict__ dfinal, T* __restrict__ dstates,
    float* __restrict__ dinit) {
  using M = Mma<T>;
  using RC = BRec<T, D>;
  using F = BwdPassFrags<T, D>;
  constexpr int CBW = F::CBW, KD = F::KD, KC = F::KC, LDS_S = D + 8;
  constexpr int VE = F::VE, LPR = F::LPR, NO = F::NO;
  // per chunk, double-buffered: dS' in the MFMA type (the exchange), dO^T
  // (columns n, rows r), and dS' untransposed for the store to dstates
  constexpr int LDO = kC + 16 / (int)sizeof(T), LDF = kBwdSliceW + 16 / (int)sizeof(T);
  __shared__ __align__(16) T sD[2][kBwdSliceW * LDS_S];
  __shared__ __align__(16) T sO[2][kBwdSliceW * LDO];
  __shared__ __align__(16) T sF[2][D * LDF];
  const int id = blockIdx.x;
  const int nh = (id & 7) + 8 * (id / (8 * nslice));
  const int slice = (id >> 3) % nslice;
  if (nh >= NH) return;
  const int seq = nh / H, h = nh % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, grp = lane >> 4;
  const int n0 = slice * kBwdSliceW, n = n0 + (lane & 15);
  const int64_t sidx = (int64_t)nh * D * D;
  const SeqSpan sp = seq_span(gm, seq);
  if (sp.c0 == sp.c1) {  // empty sequence: d_init = d_final
    if (dinit == nullptr) return;
    for (int e = threadIdx.x; e < D * kBwdSliceW; e += kBwdPassThreads) {
      const int64_t idx = sidx + (int64_t)(e / kBwdSliceW) * D + n0 + e % kBwdSliceW;
      dinit[idx] = dfinal ? dfinal[idx] : 0.f;
    }
    return;
  }
  f32x4_t dS[CBW];
#pragma unroll
  for (int i = 0; i < CBW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = (wave * CBW + i) * 16 + 4 * grp + j;
      dS[i][j] = dfinal ? dfinal[sidx + (int64_t)c * D + n] : 0.f;
    }
  const int nch = (int)(sp.c1 - sp.c0);
  const int len_last = (int)(sp.ntok - (int64_t)(nch - 1) * kC);

  // Record fragments through a buffer resource rebased at each chunk's
  // record (scalar), a per-lane offset computed once, and the fragment's
  // offset as a scalar constant: no per-load address math.
  constexpr uint32_t FBY = 64 * M::KPL * sizeof(T);  // bytes of one fragment
  const uint32_t lo_m = (uint32_t)((wave * CBW * KD * 64 + lane) * M::KPL * sizeof(T));
  const uint32_t lo_z = (uint32_t)((wave * CBW * KC * 64 + lane) * M::KPL * sizeof(T));
  auto rec_of = [&](int ci) {
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(brec + ((int64_t)h * nslot + sp.c0 + ci) * RC::BYTES), (short)0, (int)RC::BYTES,
        kRsrcWord3);
  };
  auto load_m = [&](F& f, __amdgpu_buffer_rsrc_t r, int i) {
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
      f.mf[i][ks] = BufFrag<T>::load(r, lo_m, (uint32_t)(RC::MF * sizeof(T)) + (i * KD + ks) * FBY);
  };
  auto load_z = [&](F& f, __amdgpu_buffer_rsrc_t r, int ci) {
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int ks = 0; ks < KC; ++ks)
        f.zf[i][ks] = BufFrag<T>::load(r, lo_z, (uint32_t)(RC::ZF * sizeof(T)) + (i * KC + ks) * FBY);
    // The chunk's dO slice as raw bits, one 16-byte piece per lane: the
    // buffer's bound ends after the chunk's last valid row, so rows past a
    // sequence's end read as zero, and lanes beyond the slice read past the
    // bound (zero, no memory access) -- every load is unconditional.
    const int len = ci == nch - 1 ? len_last : kC;
    const T* ob = d_o + ((sp.tok0 + (int64_t)ci * kC) * H + h) * D + n0;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ob, (short)0, (int)(((len - 1) * H * D + kBwdSliceW) * sizeof(T)), kRsrcWord3);
    const int tid = threadIdx.x;
    const uint32_t off = tid < NO ? (uint32_t)(((tid / LPR) * H * D + VE * (tid % LPR)) * sizeof(T))
                                  : kPastBound;
    f.dov = __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0);
  };
  auto load = [&](F& f, int ci) {
    const __amdgpu_buffer_rsrc_t r = rec_of(ci);
#pragma unroll
    for (int i = 0; i < CBW; ++i) load_m(f, r, i);
    load_z(f, r, ci);
  };
  // One chunk step: consumes the fragments in f and fills fn with those of
  // chunk cn, the loads spread over the step (a wave issuing a whole record
  // at once stalls behind the CU's vector memory queue).  dS on entry is dS'
  // of chunk ci (the gradient of the state leaving it): it crosses LDS in
  // the MFMA type, transposed for the product and as is for dstates
  // (kda_bwd_intra reads it only as an operand of that type and in one fp32
  // row sum), whose slice block is then stored in 16-byte pieces.  The dO
  // slice crosses LDS transposed, so each lane's fragment is two runs of rows.
  auto step = [&](const F& f, F& fn, int ci, int cn, int buf) {
    T* sb = sD[buf];
    T* sf = sF[buf];
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      const int c4 = (wave * CBW + i) * 16 + 4 * grp;
      st_perm4(sb + (lane & 15) * LDS_S, c4, dS[i][0], dS[i][1], dS[i][2], dS[i][3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_elem(sf + (c4 + j) * LDF + (lane & 15), dS[i][j]);
    }
    if (threadIdx.x < NO) {
      const int r = threadIdx.x / LPR, cb = VE * (threadIdx.x % LPR);
      T* so = sO[buf] + cb * LDO + r;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          reinterpret_cast<uint16_t*>(so)[(2 * e) * LDO] = (uint16_t)(f.dov[e] & 0xffffu);
          reinterpret_cast<uint16_t*>(so)[(2 * e + 1) * LDO] = (uint16_t)(f.dov[e] >> 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) so[e * LDO] = __uint_as_float(f.dov[e]);
      }
    }
    __syncthreads();
    typename M::frag bfr[KD], dof[KC];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) bfr[ks] = frag_at<T>(sb, LDS_S, 0, ks, lane);
    const T* sor = sO[buf] + (lane & 15) * LDO;
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) {
      if constexpr (M::KPL == 8) {  // kpos order: rows 32ks + 4grp.., then 32ks + 16 + 4grp..
        const uint2 a = *reinterpret_cast<const uint2*>(sor + ks * 32 + 4 * grp);
        const uint2 b = *reinterpret_cast<const uint2*>(sor + ks * 32 + 16 + 4 * grp);
        dof[ks] = __builtin_bit_cast(typename M::frag, u32x4_t{a.x, a.y, b.x, b.y});
      } else {
        dof[ks] = M::load(sor + 16 * (ks >> 2) + 4 * grp + (ks & 3));
      }
    }
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) acc = M::mma(f.zf[i][ks], dof[ks], acc);
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) acc = M::mma(f.mf[i][ks], bfr[ks], acc);
      dS[i] = acc;
    }
    __builtin_amdgcn_sched_barrier(0);
    const __amdgpu_buffer_rsrc_t rn = rec_of(cn);
    load_m(fn, rn, 0);
    __builtin_amdgcn_sched_barrier(0);
    // dS' of chunk ci: this slice's contiguous D x 16 block (sblk), in
    // 16-byte pieces (2 per row in bf16, 4 in fp32)
    T* dst = dstates + ((sp.c0 + ci) * H + h) * (int64_t)D * D + sblk<D>(0, n0);
    {
      constexpr int VEF = 16 / (int)sizeof(T), PPR = kBwdSliceW / VEF, NPC = D * PPR;
#pragma unroll
      for (int pr = 0; pr < (NPC + kBwdPassThreads - 1) / kBwdPassThreads; ++pr) {
        const int pc = pr * kBwdPassThreads + threadIdx.x, row = pc / PPR, cv = VEF * (pc % PPR);
        if (NPC % kBwdPassThreads == 0 || pc < NPC)
          *reinterpret_cast<u32x4_t*>(dst + row * 16 + cv) =
              *reinterpret_cast<const u32x4_t*>(sf + row * LDF + cv);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < CBW; ++i) load_m(fn, rn, i);
    load_z(fn, rn, cn);
    // No second barrier: the next chunk writes the other buffers, and these
    // are rewritten only after the next chunk's barrier, which every wave
    // reaches after its reads of them.
  };
  // Three register sets: each chunk's record is prefetched two chunks ahead
  // (clamped at the first chunk, so every load is unconditional), and the
  // loop body is three whole steps so each set stays in fixed registers.
  // Steps alternate the two LDS buffers.
  F fa, fb, fc;
  load(fa, nch - 1);
  load(fb, max(nch - 2, 0));
  int s = 0;
  for (; s + 3 <= nch; s += 3) {
    const int ci = nch - 1 - s;
    step(fa, fc, ci, max(ci - 2, 0), s & 1);
    step(fb, fa, ci - 1, max(ci - 3, 0), (s + 1) & 1);
    step(fc, fb, ci - 2, max(ci - 4, 0), s & 1);
  }
  if (s < nch) step(fa, fc, nch - 1 - s, 0, s & 1);
  if (s + 1 < nch) step(fb, fa, nch - 2 - s, 0, (s + 1) & 1);
  if (dinit != nullptr) {
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = (wave * CBW + i) * 16 + 4 * grp + j;
        dinit[sidx + (int64_t)c * D + n] = dS[i][j];
      }
  }
}

// ---------------------------------------------------------------------------
// Every gradient of one (chunk, head), given the entering state S and the
// gradient dS' of the leaving state.
template <typename T, int D, bool GS>
__global__ __launch_bounds__((BwdLds<T, D>::NT), 1) void kda_bwd_intra(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const T* __restrict__ d_o,
    const T* __restrict__ states, const T* __restrict__ dstates, ChunkGeom gm, int H,
    int64_t slot_base, int qk_l2norm, float scale, T* __restrict__ dq, T* __restrict__ dk,
    T* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta) {
  using L = BwdLds<T, D>;
  using M = Mma<T>;
  constexpr int NW = L::NW, LDX = L::LDX, LDC = L::LDC, NTW = 16 / NW;
  constexpr int KC = kC / M::KSTEP, KD = D / M::KSTEP, KPL = M::KPL;
  extern __shared__ __align__(16) char smem[];
  const int h = blockIdx.x;
  const int64_t slot = slot_base + blockIdx.y;
  ChunkLoc loc;
  if (!locate(gm, slot, loc)) return;
  BwdSmem<T, D> sm(smem);
  f32x4_t Bm[NTW];
  {
    BwdRegs R0;  // recomputed at the end rather than kept live (registers)
    bwd_prologue<T, D, GS, false, false>(q, k, g, beta, loc, H, h, qk_l2norm, sm, R0, Bm);
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
  const int c = 16 * wave + (lane & 15);  // this lane's column (d_k or d_v)
  const T* S = states + (slot * H + h) * (int64_t)D * D;
  const T* dS = dstates + (slot * H + h) * (int64_t)D * D;
  // per-token tensors: uniform bases at the chunk's first row, 32-bit offsets
  const int64_t row0 = loc.tok0 * H + h;
  const T* vb = v + row0 * D;
  const T* ob = d_o + row0 * D;
  T* dqb = dq + row0 * D;
  T* dkb = dk + row0 * D;
  T* dvb = dv + row0 * D;
  float* dgb = GS ? dg + row0 : dg + row0 * D;
  float* dbb = dbeta + row0;
  auto tok = [&](int r) { return r * H; };  // row offset, in rows of D elements

  // ---- value side: columns n = c --------------------------------------------
  // Every global read of this phase is issued at once, as raw bits converted
  // at use, so the phase waits for memory once: the S and dS' columns of the
  // two B operands (k = c), and the chunk's v and dO rows.  v and dO come in
  // coalesced 16-byte pieces through buffer resources bounded at the chunk's
  // last valid row (rows past it read as zero) and are staged where W and dO'
  // go (the inverse's region, dead now): each lane then reads its own column
  // and later overwrites exactly those positions, so no barrier separates
  // the reads from the W and dO' writes.
  uint32_t sraw[KD][KPL], draw[KD][KPL];
  {
    constexpr int NT = L::NT;
    constexpr int VE = 16 / (int)sizeof(T), PR = D / VE, NPK = kC * PR / NT;
    const int rs = H * D, span = (loc.len - 1) * rs + D;
    const __amdgpu_buffer_rsrc_t rvr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(vb), (short)0, span * (int)sizeof(T), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ror = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(ob), (short)0, span * (int)sizeof(T), kRsrcWord3);
    u32x4_t vv[NPK], ov[NPK];
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int p = i * NT + tid, row = p / PR, cp = p % PR;
      const uint32_t off = (uint32_t)((row * rs + cp * VE) * (int)sizeof(T));
      vv[i] = __builtin_amdgcn_raw_buffer_load_b128(rvr, off, 0, 2);
      ov[i] = __builtin_amdgcn_raw_buffer_load_b128(ror, off, 0, 2);
    }
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int cc = ks * M::KSTEP + KPL * grp + e;
        sraw[ks][e] = ld_raw(S + sblk<D>(cc, c));
        draw[ks][e] = ld_raw(dS + sblk<D>(cc, c));
      }
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int p = i * NT + tid, row = p / PR, cp = p % PR;
      *reinterpret_cast<u32x4_t*>(sm.wb + row * LDX + cp * VE) = vv[i];
      *reinterpret_cast<u32x4_t*>(sm.dob + row * LDX + cp * VE) = ov[i];
    }
  }
  __syncthreads();
  // Kp S, then R = Diag(beta)(V - Kp S) and W = T R
  f32x4_t vmk[4], acc[4], w[4];
  {
    typename M::frag sb[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) sb[ks] = raw_frag(sraw[ks], T{});
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_sched_barrier(0);  // one tile at a time (registers)
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) a = M::mma(frag_at<T>(sm.kp, LDX, 16 * t, ks, lane), sb[ks], a);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * t + 4 * grp + j;
        const float vv = ld_f(sm.wb + r * LDX + c);  // zero past the chunk's end
        vmk[t][j] = vv - a[j];
        acc[t][j] = sm.beta[r] * vmk[t][j];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    __builtin_amdgcn_sched_barrier(0);  // one tile at a time (registers)
    w[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      w[t] = M::mma(frag_rm_perm<T>(sm.tb, LDC, 16 * t, ks, lane), acc_frag<T>(acc, ks), w[t]);
  }
  // dO' (kept for P^T dO') ; W and dO' into LDS
  f32x4_t dov[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      dov[t][j] = scale * ld_f(sm.dob + r * LDX + c);  // zero past the chunk's end
      st_f(sm.wb + r * LDX + c, w[t][j]);
      st_f(sm.dob + r * LDX + c, dov[t][j]);
    }
  // dW = P^T dO' + K~ dS'
  {
    typename M::frag dsb[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) dsb[ks] = raw_frag(draw[ks], T{});
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_sched_barrier(0);  // one tile at a time (registers)
      f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KC; ++ks)
        a = M::mma(frag_cm_perm<T>(sm.pb, LDC, 16 * t, ks, lane), acc_frag<T>(dov, ks), a);
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) a = M::mma(frag_at<T>(sm.kt, LDX, 16 * t, ks, lane), dsb[ks], a);
      acc[t] = a;
    }
  }
  // L = T^T dW; dV = Diag(beta) L; dbeta, first part: rowsum(L o (V - Kp S))
  f32x4_t lam[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    __builtin_amdgcn_sched_barrier(0);  // one tile at a time (registers)
    lam[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      lam[t] = M::mma(frag_cm_perm<T>(sm.tb, LDC, 16 * t, ks, lane), acc_frag<T>(acc, ks), lam[t]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      if (r < loc.len) st_nt(dvb + tok(r) * D + c, sm.beta[r] * lam[t][j]);
      const float part = sum16(lam[t][j] * vmk[t][j]);
      if ((lane & 15) == 0) sm.red[wave * kC + r] = part;
    }
  }
  __syncthreads();  // every read of K~ is done: its region becomes L
  T* lb = sm.kt;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) st_f(lb + (16 * t + 4 * grp + j) * LDX + c, lam[t][j]);
  __syncthreads();

  // ---- chunk x chunk: dP = tril(dO' W^T), dA = -tril_-1(L W^T), dB ------------
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt) {
    const int p = wave + NW * tt, rb = p >> 2, ib = p & 3;
    f32x4_t ap = {0.f, 0.f, 0.f, 0.f}, aa = ap;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const auto bw = frag_at<T>(sm.wb, LDX, 16 * ib, ks, lane);
      ap = M::mma(frag_at<T>(sm.dob, LDX, 16 * rb, ks, lane), bw, ap);
      aa = M::mma(frag_at<T>(lb, LDX, 16 * rb, ks, lane), bw, aa);
    }
    const int i = 16 * ib + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * rb + 4 * grp + j;
      const float da = i < r ? -aa[j] : 0.f;
      st_f(sm.pb + r * LDC + i, i <= r ? ap[j] : 0.f);
      st_f(sm.db + r * LDC + i, sm.beta[r] * da);
      const float part = sum16(da * Bm[tt][j]);
      if ((lane & 15) == 0) sm.red[(NW + ib) * kC + r] = part;  // one tile per (ib, r)
    }
  }
  __syncthreads();
  if (tid < kC) {
    float b = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) b += sm.red[w2 * kC + tid];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) b += sm.red[(NW + ib) * kC + tid];
    sm.x0[tid] = b;
  }

  __syncthreads();  // red is free again (x0 was formed from it)

  // ---- key side: columns c, then the gates ----------------------------------
  // (the scheduler fences between phases keep each phase's loads in it:
  // hoisted early, they would hold registers across the phases before)
  __builtin_amdgcn_sched_barrier(0);
  // G, k^, q^ again (the chunk's k, q, g are still in the cache)
  BwdRegs R;
  {
    float gr[4][4];
    load_cols<T, D, GS>(q, k, g, loc, H, h, c, grp, R, gr);
    prefix_G(gr, lane, R);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * t + 4 * grp + j;
        R.kh[t][j] *= sm.rk[r];
        R.qh[t][j] *= sm.rq[r];
      }
  }
  // Two passes, each with its own B operands, the gate factors applied per
  // tile so that one tile's accumulators are live at a time:
  //   1. dQp = dO' S^T + dP Km,  dKp = dB Km - Diag(beta) L S^T
  //   2. dKm = dB^T Kp + dP^T Qp,  dK~ = W dS'^T,  rowsum(S o dS')
  // (q^ is read again for the norm's projection at the end rather than kept)
  float dkh[4][4], dqh[4][4], dG[4][4];  // dkh holds dKp o e^G after pass 1
  __builtin_amdgcn_sched_barrier(0);
  {
    typename M::frag st[KD], kmc[KC];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) st[ks] = grow_frag<T, D>(S, c, ks, lane);
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) kmc[ks] = frag_cm<T>(sm.km, LDX, 16 * wave, ks, lane);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_sched_barrier(0);  // one tile at a time (registers)
      f32x4_t a = {0.f, 0.f, 0.f, 0.f}, x = a, b = a;
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        a = M::mma(frag_at<T>(sm.dob, LDX, 16 * t, ks, lane), st[ks], a);  // dO' S^T
        x = M::mma(frag_at<T>(lb, LDX, 16 * t, ks, lane), st[ks], x);      // L S^T
      }
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        a = M::mma(frag_at<T>(sm.pb, LDC, 16 * t, ks, lane), kmc[ks], a);  // dP Km
        b = M::mma(frag_at<T>(sm.db, LDC, 16 * t, ks, lane), kmc[ks], b);  // dB Km
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float eg = __expf(R.G[t][j]);
        dqh[t][j] = a[j] * eg;
        dkh[t][j] = (b[j] - sm.beta[16 * t + 4 * grp + j] * x[j]) * eg;
        dG[t][j] = R.qh[t][j] * dqh[t][j];  // q^ is not needed again until the end
        const float qd = sum16(R.qh[t][j] * dqh[t][j]);  // row dot q^ . dq^, this wave's part
        if ((lane & 15) == 0) sm.red[(NW + wave) * kC + 16 * t + 4 * grp + j] = qd;
      }
    }
  }
  float rs = 0.f, dgam = 0.f;  // rowsum(S o dS') of row c
  __builtin_amdgcn_sched_barrier(0);
  {
    typename M::frag dst[KD], kpc[KC], qpc[KC];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const typename M::frag xs = grow_frag<T, D>(S, c, ks, lane);
      dst[ks] = grow_frag<T, D>(dS, c, ks, lane);
#pragma unroll
      for (int e = 0; e < KPL; ++e) rs += frag_val(xs, e) * frag_val(dst[ks], e);
    }
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) {
      kpc[ks] = frag_cm<T>(sm.kp, LDX, 16 * wave, ks, lane);
      qpc[ks] = frag_cm<T>(sm.qp, LDX, 16 * wave, ks, lane);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_sched_barrier(0);  // one tile at a time (registers)
      f32x4_t m = {0.f, 0.f, 0.f, 0.f}, kt = m;
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        kt = M::mma(frag_at<T>(sm.wb, LDX, 16 * t, ks, lane), dst[ks], kt);  // W dS'^T
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        m = M::mma(frag_cm<T>(sm.db, LDC, 16 * t, ks, lane), kpc[ks], m);  // dB^T Kp
        m = M::mma(frag_cm<T>(sm.pb, LDC, 16 * t, ks, lane), qpc[ks], m);  // dP^T Qp
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float G = R.G[t][j];
        const float a = dkh[t][j], bm = m[j] * __expf(-G), e = kt[j] * __expf(R.gam - G);
        dkh[t][j] = a + bm + e;
        dG[t][j] += R.kh[t][j] * (a - bm - e);
        dgam += R.kh[t][j] * e;
      }
    }
  }
  rs += __shfl_xor(rs, 16);
  rs += __shfl_xor(rs, 32);
  dgam += __shfl_xor(dgam, 16);
  dgam += __shfl_xor(dgam, 32);
  dgam += __expf(R.gam) * rs;
  if (grp == 3) dG[3][3] += dgam;  // gamma = G of row 63
  // dg_r = sum_(s >= r) dG_s: within the lane's 4 rows, across the lane
  // groups, then across the tiles from the last
  float dgo[4][4];
  {
    float carry = 0.f;
#pragma unroll
    for (int t = 3; t >= 0; --t) {
      float suf[4];
      float run = 0.f;
#pragma unroll
      for (int j = 3; j >= 0; --j) { run += dG[t][j]; suf[j] = run; }
      float x = run;
      float y = __shfl_down(x, 16);
      if (grp <= 2) x += y;
      y = __shfl_down(x, 32);
      if (grp <= 1) x += y;
      const float excl = x - run;
      const float total = __shfl(x, lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) dgo[t][j] = carry + excl + suf[j];
      carry += total;
    }
  }
  // row dots k^ . dk^ (q^ . dq^ was taken in pass 1) over all columns
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = sum16(R.kh[t][j] * dkh[t][j]);
      if ((lane & 15) == 0) sm.red[wave * kC + 16 * t + 4 * grp + j] = a;
    }
  __syncthreads();
  if (tid < kC) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      a += sm.red[w2 * kC + tid];
      b += sm.red[(NW + w2) * kC + tid];
    }
    sm.x1[tid] = a;
    sm.x2[tid] = b;
    if (tid < loc.len) st_nt(dbb + tok(tid), sm.x0[tid]);
  }
  __syncthreads();
  // dk, dq (and dg) leave through LDS: each lane writes its column of the
  // row-major tiles (the layout's first bytes, free since the barrier
  // above), and the tiles go out in 16-byte non-temporal pieces through
  // buffer resources bounded at the chunk's last valid row, whole lines at
  // a time (rows past the end are dropped by the bound).
  char* ostage = reinterpret_cast<char*>(sm.kp);
  T* sdk = reinterpret_cast<T*>(ostage);
  T* sdq = reinterpret_cast<T*>(ostage + L::XB);
  float* sdg = reinterpret_cast<float*>(ostage + 2 * L::XB);
  constexpr int LDG = D + 4;
  static_assert(2 * L::XB + kC * LDG * 4 <= 4 * L::XB, "staged gradients must fit");
  const T* qrow = q + row0 * D;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      float gk = dkh[t][j], gq = dqh[t][j];
      if (qk_l2norm) {
        const float qn = r < loc.len ? ld_f(qrow + tok(r) * D + c) * sm.rq[r] : 0.f;
        gk = sm.rk[r] * (gk - sm.x1[r] * R.kh[t][j]);
        gq = sm.rq[r] * (gq - sm.x2[r] * qn);
      }
      st_f(sdk + r * LDX + c, gk);
      st_f(sdq + r * LDX + c, gq);
      if constexpr (!GS) sdg[r * LDG + c] = dgo[t][j];
    }
  __syncthreads();
  {
    constexpr int NT = L::NT;
    constexpr int VE = 16 / (int)sizeof(T), PR = D / VE, NPK = kC * PR / NT;
    constexpr int PRG = D / 4, NPG = kC * PRG / NT;
    constexpr int kNt = 2;  // non-temporal: nothing here reads the gradients again
    const int rs = H * D, span = (loc.len - 1) * rs + D;
    auto rsrc = [](void* base, int bytes) {
      return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, kRsrcWord3);
    };
    const __amdgpu_buffer_rsrc_t rdk = rsrc(dkb, span * (int)sizeof(T));
    const __amdgpu_buffer_rsrc_t rdq = rsrc(dqb, span * (int)sizeof(T));
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int p = i * NT + tid, row = p / PR, cp = p % PR;
      const uint32_t off = (uint32_t)((row * rs + cp * VE) * (int)sizeof(T));
      __builtin_amdgcn_raw_buffer_store_b128(
          *reinterpret_cast<const u32x4_t*>(sdk + row * LDX + cp * VE), rdk, off, 0, kNt);
      __builtin_amdgcn_raw_buffer_store_b128(
          *reinterpret_cast<const u32x4_t*>(sdq + row * LDX + cp * VE), rdq, off, 0, kNt);
    }
    if constexpr (!GS) {
      const __amdgpu_buffer_rsrc_t rdg = rsrc(dgb, span * 4);
#pragma unroll
      for (int i = 0; i < NPG; ++i) {
        const int p = i * NT + tid, row = p / PRG, cp = p % PRG;
        __builtin_amdgcn_raw_buffer_store_b128(
            *reinterpret_cast<const u32x4_t*>(sdg + row * LDG + cp * 4), rdg,
            (uint32_t)((row * rs + cp * 4) * 4), 0, kNt);
      }
    }
  }
  if constexpr (GS) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = sum16(dgo[t][j]);
        if ((lane & 15) == 0) sm.red[wave * kC + 16 * t + 4 * grp + j] = a;
      }
    __syncthreads();
    if (tid < loc.len) {
      float a = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) a += sm.red[w2 * kC + tid];
      st_nt(dgb + tok(tid), a);
    }
  }
}

// ---------------------------------------------------------------------------
// Workspace: [forward workspace | S per slot | dS' per slot | M, Z^T records |
// chunk map].  Slots are sized for the larger of the dense and varlen bounds.
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

struct BwdPlan {
  int64_t slots, fwd, states, recs, map, total;
};

BwdPlan bwd_plan(const kda_desc_t& d) {
  BwdPlan p{};
  p.slots = std::max(chunk_slot_bound(d, true), chunk_slot_bound(d, false));
  kda_desc_t df = d;
  df.ckpt_every = 0;
  p.fwd = align256((int64_t)chunk_workspace_bytes(df));
  // S and dS' in the MFMA type (the element type of q/k/v)
  p.states = align256(p.slots * d.heads * (int64_t)d.dk * d.dv *
                      (d.dtype == KDA_DTYPE_BF16 ? 2 : 4));
  const int64_t rb = d.dtype == KDA_DTYPE_BF16
                         ? (d.dk == 128 ? BRec<bf16, 128>::BYTES : BRec<bf16, 64>::BYTES)
                         : (d.dk == 128 ? BRec<float, 128>::BYTES : BRec<float, 64>::BYTES);
  p.recs = p.slots * d.heads * rb;
  p.map = 2 * align256(((int64_t)d.num_seqs + 1) * 4);
  p.total = p.fwd + 2 * p.states + p.recs + p.map;
  return p;
}

template <typename T, int D>
hipError_t run_bwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* init_state, const int32_t* cu,
                   const void* d_o, const float* d_final, void* dq, void* dk, void* dv,
                   float* dg, float* dbeta, float* d_init, char* ws, hipStream_t stream) {
  using L = BwdLds<T, D>;
  const BwdPlan p = bwd_plan(d);
  const bool varlen = cu != nullptr;
  const int H = d.heads, NH = d.num_seqs * d.heads;
  T* states = reinterpret_cast<T*>(ws + p.fwd);
  T* dstates = reinterpret_cast<T*>(ws + p.fwd + p.states);
  char* recs = ws + p.fwd + 2 * p.states;
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + p.fwd + 2 * p.states + p.recs);
  int32_t* cu_s = chunk_off + (p.map / 2) / 4;
  const int64_t nslot = chunk_slot_bound(d, varlen);

  kda_desc_t df = d;
  df.ckpt_every = 0;
  hipError_t e = launch_chunk_fwd(df, q, k, v, g, beta, init_state, cu, nullptr, nullptr,
                                  nullptr, states, ws, stream);
  if (e != hipSuccess) return e;
  ChunkGeom gm{nullptr, nullptr, d.seqlen, (d.seqlen + kC - 1) / kC, d.num_seqs};
  if (varlen) {
    hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(kThreads), 0, stream, cu, d.num_seqs,
                       d.seqlen, cu_s, chunk_off);
    gm = ChunkGeom{cu_s, chunk_off, d.seqlen, 0, d.num_seqs};
  }
  using LP = BwdLds<T, D, true>;
  static bool attr_set = false;
  if (!attr_set) {
    for (const void* fn : {(const void*)kda_bwd_prep<T, D, false>,
                           (const void*)kda_bwd_prep<T, D, true>}) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LP::BYTES);
      if (e != hipSuccess) return e;
    }
    for (const void* fn : {(const void*)kda_bwd_intra<T, D, false>,
                           (const void*)kda_bwd_intra<T, D, true>}) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  // chunk slots go in the grid's y dimension, at most kMaxGridY per launch
  constexpr int64_t kMaxGridY = 32768;
  auto prep = d.gate_per_head ? kda_bwd_prep<T, D, true> : kda_bwd_prep<T, D, false>;
  for (int64_t sb = 0; sb < nslot; sb += kMaxGridY) {
    const unsigned ny = (unsigned)std::min<int64_t>(kMaxGridY, nslot - sb);
    hipLaunchKernelGGL(prep, dim3(H, ny), dim3(LP::NT), LP::BYTES, stream, (const T*)q,
                       (const T*)k, g, beta, gm, H, nslot, sb, d.qk_l2norm, d.scale, recs);
  }
  const int nslice = D / kBwdSliceW;
  const int nhpad = (NH + 7) / 8 * 8;
  hipLaunchKernelGGL((kda_bwd_state_pass<T, D>), dim3(nhpad * nslice), dim3(kBwdPassThreads), 0,
                     stream, recs, nslot, gm, H, NH, nslice, (const T*)d_o, d_final, dstates,
                     d_init);
  auto intra = d.gate_per_head ? kda_bwd_intra<T, D, true> : kda_bwd_intra<T, D, false>;
  for (int64_t sb = 0; sb < nslot; sb += kMaxGridY) {
    const unsigned ny = (unsigned)std::min<int64_t>(kMaxGridY, nslot - sb);
    hipLaunchKernelGGL(intra, dim3(H, ny), dim3(L::NT), L::BYTES, stream, (const T*)q,
                       (const T*)k, (const T*)v, g, beta, (const T*)d_o, states, dstates, gm, H,
                       sb, d.qk_l2norm, d.scale, (T*)dq, (T*)dk, (T*)dv, dg, dbeta);
  }
  return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_workspace_bytes(const kda_desc_t& d) { return (size_t)bwd_plan(d).total; }

hipError_t launch_chunk_bwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, const void* d_o, const float* d_final,
                            void* dq, void* dk, void* dv, float* dg, float* dbeta,
                            float* d_init, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  if (d.dtype == KDA_DTYPE_BF16) {
    if (d.dk == 128)
      return run_bwd<bf16, 128>(d, q, k, v, g, beta, init_state, cu_seqlens, d_o, d_final, dq,
                                dk, dv, dg, dbeta, d_init, ws, stream);
    return run_bwd<bf16, 64>(d, q, k, v, g, beta, init_state, cu_seqlens, d_o, d_final, dq, dk,
                             dv, dg, dbeta, d_init, ws, stream);
  }
  if (d.dk == 64)
    return run_bwd<float, 64>(d, q, k, v, g, beta, init_state, cu_seqlens, d_o, d_final, dq, dk,
                              dv, dg, dbeta, d_init, ws, stream);
  return hipErrorInvalidValue;  // fp32 at d = 128: rejected by the caller
}

}  // namespace kda
