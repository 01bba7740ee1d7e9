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
//   1. the forward's states, per segment of chunk slots (kda_chunk.hip's
//      launch_chunk_states): kda_bwd_prep, one workgroup per (chunk, head),
//      forms the chunk's norms, G, A, P, T and writes the forward state
//      pass's record (K~, -Wk, U, e^gamma), the reverse pass's record (M and
//      Z^T in operand order) and T; the forward's state pass (without output)
//      then writes every chunk's entering state S to the workspace;
//   2. kda_bwd_state_pass, one workgroup per (sequence, head, 16 columns of
//      d_v), sequential over the sequence's chunks from the last: dS' of every
//      chunk to the workspace, dS of the first to d_init_state;
//   3. kda_bwd_intra, one workgroup per (chunk, head): every gradient above;
//   4. kda_bwd_exact, a persistent grid: the gradients of the chunks prep
//      flagged as beyond the mid reference's exponent range (none, usually).
// The intra-chunk kernel recomputes the chunk's operands (norms, G, A, P)
// rather than store them; T it loads.
//
// Operand layouts.  A workgroup of D/16 waves gives wave w the 16 columns
// [16w, 16w+16) of every chunk x d matrix, all 64 rows, in MFMA accumulator
// layout (lane: column l%16, rows 16t + 4(l/16) + j).  A product whose summed
// index is the chunk row can take such an accumulator straight as an operand
// (see acc_frag) when the other operand is read with the same row order
// (the kpos permutation of kda_chunk_common.h); everything else is staged in
// LDS in the MFMA type.
//
// Exponents: the chunk-local products take e^(G_r - G_i) split as
// e^(G_r - m) e^(m - G_i) around a per-channel reference m, as the forward
// does: the chunk start while every channel's chunk decay gamma >= -80, else
// G of row 31 while each half of the chunk decays by at most 80 (gamma down to
// about -160; see BwdMode).  For a chunk beyond that, kda_bwd_prep forms A
// and P exactly (so the forward states after it and its reverse-pass record
// hold) and flags it, kda_bwd_intra leaves its gradients to kda_bwd_exact,
// which forms every gate factor from its own exponent difference, and the
// caller's range flag (when given) is set.  fp32 operands at d = 128 do not
// fit one workgroup's LDS and are not supported.
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
// The bf16 column fragments come from LDS transpose reads
// (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces named by lanes i / 4 + 4e, e = 0..3.  So if
// lane j names row k0 + j / 4, columns m0 + 4 (j % 4) .. +3 of a row-major X,
// lane i receives X[k0 .. k0+3][m0 + i]: four consecutive k of its own
// column m, half an operand fragment (layout measured on gfx950).
typedef short tr16_v4 __attribute__((__vector_size__(4 * sizeof(short))));
__device__ __forceinline__ uint2 ld_tr16(const bf16* p) {
  const tr16_v4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) tr16_v4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(uint2, v);
}
// k0: the first of the fragment's two runs of four k; the second starts
// `gap` rows further.
__device__ __forceinline__ bf16x8_t frag_tr(const bf16* X, int ld, int m0, int k0, int gap,
                                            int lane) {
  const int j = lane & 15;
  const bf16* p = X + (k0 + (j >> 2)) * ld + m0 + 4 * (j & 3);
  const uint2 a = ld_tr16(p), b = ld_tr16(p + gap * ld);
  return __builtin_bit_cast(bf16x8_t, (u32x4_t{a.x, a.y, b.x, b.y}));
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_cm(const T* X, int ld, int m0, int ks,
                                                         int lane);
template <>
__device__ __forceinline__ bf16x8_t frag_cm<bf16>(const bf16* X, int ld, int m0, int ks,
                                                  int lane) {
  return frag_tr(X, ld, m0, ks * 32 + 8 * (lane >> 4), 4, lane);
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
  // positions 0..3: k = 32 ks + 4 g + 0..3; 4..7: k = 32 ks + 16 + 4 g + 0..3
  return frag_tr(X, ld, m0, ks * 32 + 4 * (lane >> 4), 16, lane);
}
template <>
__device__ __forceinline__ float frag_cm_perm<float>(const float* X, int ld, int m0, int ks,
                                                     int lane) {
  return X[(16 * (ks >> 2) + 4 * (lane >> 4) + (ks & 3)) * ld + m0 + (lane & 15)];
}

// One 16-byte piece of the MFMA type from fp32 values (8 bf16 rounded to
// nearest even, or 4 fp32).
__device__ __forceinline__ u32x4_t pack16(const float* x, bf16) {
  return u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
}
__device__ __forceinline__ u32x4_t pack16(const float* x, float) {
  return u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                 __float_as_uint(x[3])};
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
// st_fnat4 with non-temporal stores: the reverse pass's records are read once,
// after the forward pass, and allocated in the last-level cache they would
// push out the state pass's records that the forward reads next.
__device__ __forceinline__ void st_fnat4_nt(bf16* base, int nks, int m, int k0, float a, float b,
                                            float c, float d) {
  __builtin_nontemporal_store(u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)},
                              reinterpret_cast<u32x2_t*>(base + fnat<bf16>(m, k0, nks)));
}
__device__ __forceinline__ void st_fnat4_nt(float* base, int nks, int m, int k0, float a, float b,
                                            float c, float d) {
  __builtin_nontemporal_store(a, base + fnat<float>(m, k0, nks));
  __builtin_nontemporal_store(b, base + fnat<float>(m, k0 + 1, nks));
  __builtin_nontemporal_store(c, base + fnat<float>(m, k0 + 2, nks));
  __builtin_nontemporal_store(d, base + fnat<float>(m, k0 + 3, nks));
}

// A copy of x the compiler cannot see through: lane indices renewed from it
// at a phase boundary make the phase form its own address arithmetic there,
// rather than keep an earlier phase's addresses live in registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Sum over the 16 lanes of a lane group (the 16 columns of an accumulator),
// every lane of the group receiving it.  The lane group is a DPP row: swap
// neighbours, then pairs (quad permutations), then the quads of each half-row
// (half-row mirror), then the halves (row mirror) -- four VALU steps with no
// LDS traffic.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// The sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16), every lane of
// a group receiving it.
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "DPP row groups only");
  if constexpr (N >= 2) x += dpp_f<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) x += dpp_f<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_f<0x140>(x); // row_mirror
  return x;
}
__device__ __forceinline__ float sum16(float x) { return sum_lanes<16>(x); }

// Exchanges between the four 16-lane groups (rows) of a wave, on the VALU:
// permlane16_swap(x, x) returns rows (x0, x0, x2, x2) and (x1, x1, x3, x3),
// permlane32_swap(x, x) returns (x0, x1, x0, x1) and (x2, x3, x2, x3)
// (measured on gfx950), so each lane reaches the same lane of row g ^ 1 or
// g ^ 2 in one instruction.
__device__ __forceinline__ float row_xor1(float x, int grp) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((grp & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float row_xor2(float x, int grp) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((grp & 2) ? r[0] : r[1]);
}
// Row 3's value of this lane's column, in every row.
__device__ __forceinline__ float row3_bcast(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const auto b = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
  return __uint_as_float(b[1]);
}
// Prefix (rows 0..g) and suffix (rows g..3) sums over the rows of each
// column, and the column's total.
__device__ __forceinline__ float rows_prefix(float x, int grp, float& total) {
  const float pair = x + row_xor1(x, grp);
  const float other = row_xor2(pair, grp);
  total = pair + other;
  return ((grp & 1) ? pair : x) + ((grp & 2) ? other : 0.f);
}
__device__ __forceinline__ float rows_suffix(float x, int grp, float& total) {
  const float pair = x + row_xor1(x, grp);
  const float other = row_xor2(pair, grp);
  total = pair + other;
  return ((grp & 1) ? x : pair) + ((grp & 2) ? 0.f : other);
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
  static constexpr int SMALL = (6 * kC + 2 * NW * kC) * 4;
  // full layout, where it fits: the fp32 tiles of Kp Km^T (for dbeta), kept
  // from the prologue to the chunk x chunk products in LDS rather than in
  // registers
  static constexpr int LDB = kC + 4;
  static constexpr int BM = SM + SMALL;
  static constexpr bool BM_LDS = !COMPACT && BM + kC * LDB * 4 <= 160 * 1024;
  static constexpr int BYTES = BM_LDS ? BM + kC * LDB * 4 : SM + SMALL;
  static_assert(BYTES <= 160 * 1024, "per-chunk backward LDS exceeds a CU");
};

template <typename T, int D, bool COMPACT = false>
struct BwdSmem {
  using L = BwdLds<T, D, COMPACT>;
  T *kp, *km, *qp, *kt, *tb, *pb, *db, *wb, *dob;
  float *sA, *sT, *scratch, *beta, *rk, *rq, *x0, *x1, *x2, *red, *bm;
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
    bm = L::BM_LDS ? reinterpret_cast<float*>(s + L::BM) : nullptr;
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

// Exponent reference of the chunk-local products (A, P, dP Km, dB Km,
// dB^T Kp + dP^T Qp), chosen per chunk as in the forward: the chunk start
// while every channel's gamma >= -80 (Kp = K^ o e^G, Km = K^ o e^-G), else
// m = G of row 31 per channel while each half of the chunk decays by at most
// 80 (the products then take K^ o e^(G-m), K^ o e^(m-G), Q^ o e^(G-m), whose
// factors stay within [e^-80, e^80] wherever they matter, and the per-element
// gate factors become e^(G-m) and e^(m-G)).  Beyond that the chunk's
// gradients come from kda_bwd_exact.
enum BwdMode { kBwdFast = 0, kBwdMid = 1, kBwdBeyond = 2 };
// G of row 31 of this lane's column (the lanes of lane group 3 hold it)
__device__ __forceinline__ float g_row31(const BwdRegs& R, int lane) {
  (void)lane;
  return row3_bcast(R.G[1][3]);
}
__device__ __forceinline__ int bwd_mode(const BwdRegs& R, int lane) {
  if (__syncthreads_or(R.gam < kFastDecayBound) == 0) return kBwdFast;
  const float m = g_row31(R, lane);
  return __syncthreads_or(m < kFastDecayBound || R.gam - m < kFastDecayBound) ? kBwdBeyond
                                                                               : kBwdMid;
}

// Raw k, q, g of this lane's column and rows, as loaded (the loads are
// issued here and waited for where cols_from_raw uses them, so a caller can
// put other work between the two); rows past the chunk's end read its last
// row and are zeroed by cols_from_raw.
struct ColsRaw {
  uint32_t k[4][4], q[4][4];
  float g[4][4];
};
template <typename T, int D, bool GS>
__device__ __forceinline__ void load_cols_raw(const T* __restrict__ q, const T* __restrict__ k,
                                              const float* __restrict__ g, const ChunkLoc& loc,
                                              int H, int h, int c, int grp, ColsRaw& X) {
  // uniform bases (the chunk's first row) and 32-bit per-lane offsets
  const int64_t row0 = loc.tok0 * H + h;
  const T* kb = k + row0 * D;
  const T* qb = q + row0 * D;
  const float* gb = GS ? g + row0 : g + row0 * D;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = min(16 * t + 4 * grp + j, loc.len - 1);
      const int off = r * H * D + c;
      X.k[t][j] = ld_raw(kb + off);
      X.q[t][j] = ld_raw(qb + off);
      X.g[t][j] = GS ? gb[r * H] : gb[off];
    }
}
// k, q (in R) and g (in gr) from the raw loads, zero past the chunk's end.
template <typename T>
__device__ __forceinline__ void cols_from_raw(const ColsRaw& X, const ChunkLoc& loc, int grp,
                                              BwdRegs& R, float (&gr)[4][4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = 16 * t + 4 * grp + j < loc.len;
      R.kh[t][j] = ok ? raw_val<T>(X.k[t][j]) : 0.f;
      R.qh[t][j] = ok ? raw_val<T>(X.q[t][j]) : 0.f;
      gr[t][j] = ok ? X.g[t][j] : 0.f;
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
    a = sum_lanes<PR>(a);  // every thread is active here
    b = sum_lanes<PR>(b);
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
    float total;
    const float excl = rows_prefix(run, grp, total) - run;
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
// INV: form T here (else the caller puts T in tb before its next barrier);
// tout (or nullptr): where T itself (without Diag(beta)) also goes, 64 x 64
// row-major in the MFMA type.
// A and P of a chunk beyond the mid reference's range, exactly: every entry
// from its own exponent differences, A_ri = beta_r sum_c k^_rc k^_ic
// e^(G_rc - G_ic) (i < r) and P_ri = sum_c q^_rc k^_ic e^(G_rc - G_ic) (i <= r),
// so that T, the forward states and the reverse pass's record (Z = Qp - P Wk)
// hold for any gate.  Channels come 16 at a time, k^ and G channel-major in
// `stage`, q^ in `sqs`; thread (row r = lane, columns i = wave + NW e) adds
// their terms to its entries of A and P in LDS (the first block starts them,
// the last scales A by beta_r and clears the entries above the diagonals).
// LDS operands only, so it adds few registers to the common path.
template <int NW>
__device__ __forceinline__ void exact_AP_block(const float* stage, const float* sqs,
                                               const float* beta, float* sA, float* sP, int lane,
                                               int wave, bool first, bool last) {
  constexpr int EPT = kC / NW;
  const float* sk = stage;
  const float* sg = stage + 16 * kC;
#pragma unroll 1
  for (int e = 0; e < EPT; ++e) {
    const int i = wave + NW * e;  // the same for the whole wave: broadcast reads
    float a = first ? 0.f : sA[lane * kTriLd + i];
    float p = first ? 0.f : sP[lane * kTriLd + i];
#pragma unroll 4
    for (int cc = 0; cc < 16; ++cc) {
      const float d = i < lane ? sg[cc * kC + lane] - sg[cc * kC + i] : 0.f;
      const float x = sk[cc * kC + i] * __expf(d);
      a += sk[cc * kC + lane] * x;
      p += sqs[cc * kC + lane] * x;
    }
    sA[lane * kTriLd + i] = last ? (i < lane ? beta[lane] * a : 0.f) : a;
    sP[lane * kTriLd + i] = last ? (i <= lane ? p : 0.f) : p;
  }
}

// EXA: a chunk beyond the mid reference's range forms A and P exactly
// (exact_AP_block), staged in T's and P's LDS, with P accumulated in fp32
// T's space, before T is written; otherwise such a chunk's A, T and P are not
// meaningful (the intra-chunk kernel leaves its gradients to the exact
// kernel).
template <typename T, int D, bool GS, bool TBETA, bool COMPACT, bool NTL = false, bool INV = true,
          bool EXA = false>
__device__ __forceinline__ int bwd_prologue(const T* __restrict__ q, const T* __restrict__ k,
                                            const float* __restrict__ g,
                                            const float* __restrict__ beta, const ChunkLoc& loc,
                                            int H, int h, int qk_l2norm,
                                            BwdSmem<T, D, COMPACT>& sm, BwdRegs& R,
                                            f32x4_t* Bm, T* __restrict__ tout = nullptr) {
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
  const int mode = bwd_mode(R, lane);  // (its barriers also end the staged reads)
  const float mr = mode == kBwdFast ? 0.f : g_row31(R, lane);
  // gated operands: Kp, Km, Qp relative to the mode's reference
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      R.kh[t][j] *= sm.rk[r];
      R.qh[t][j] *= sm.rq[r];
      const float G = R.G[t][j];
      const float eg = __expf(G - mr), en = __expf(mr - G), et = __expf(R.gam - G);
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
  if constexpr (!INV) {
    __syncthreads();
    return mode;
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
  if constexpr (EXA) {
    static_assert(2 * 16 * kC * 4 <= L::CB, "exact A's stage must fit T's buffer");
    static_assert(16 * kC * 4 <= L::CB, "exact P's q stage must fit P's buffer");
    if (mode == kBwdBeyond) {  // T's and P's buffers and fp32 T are free until the inverse
      float* xs = reinterpret_cast<float*>(sm.tb);
      float* xq = reinterpret_cast<float*>(sm.pb);
#pragma unroll 1
      for (int b = 0; b < NW; ++b) {
        if (wave == b) {  // this wave's 16 channels, channel-major
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 16 * t + 4 * grp + j;
              xs[(lane & 15) * kC + r] = R.kh[t][j];
              xs[16 * kC + (lane & 15) * kC + r] = R.G[t][j];
              xq[(lane & 15) * kC + r] = R.qh[t][j];
            }
        }
        __syncthreads();
        exact_AP_block<NW>(xs, xq, sm.beta, sm.sA, sm.sT, lane, wave, b == 0, b == NW - 1);
        __syncthreads();
      }
      for (int e = tid; e < kC * kC; e += NT) {
        const int r = e >> 6, i = e & 63;
        st_f(sm.pb + r * LDC + i, sm.sT[r * kTriLd + i]);
      }
      __syncthreads();
    }
  }
  tri_inv64(sm.sA, sm.sT, sm.scratch, wave, lane);
  for (int e = tid; e < kC * kC; e += NT) {
    const int r = e >> 6, i = e & 63;
    const float t = i <= r ? sm.sT[r * kTriLd + i] : 0.f;
    st_f(sm.tb + r * LDC + i, TBETA ? t * sm.beta[i] : t);
  }
  if (tout != nullptr) {
    // 16-byte pieces of T's rows, rounded as the tb copy above
    constexpr int VE = 16 / (int)sizeof(T), PR = kC / VE;
    for (int p = tid; p < kC * PR; p += NT) {
      const int r = p / PR, i0 = VE * (p % PR);
      float x[VE];
#pragma unroll
      for (int u = 0; u < VE; ++u) x[u] = i0 + u <= r ? sm.sT[r * kTriLd + i0 + u] : 0.f;
      __builtin_nontemporal_store(pack16(x, T{}), reinterpret_cast<u32x4_t*>(tout + r * kC + i0));
    }
  }
  __syncthreads();
  return mode;
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

// kda_bwd_prep, one workgroup per (chunk, head) of one segment of chunk slots:
// the chunk's norms, G, A, P, T = (I + A)^-1, then
//  * the reverse pass's record (M and scale Z^T) and T (for the intra-chunk
//    kernel), indexed by the batch's slot;
//  * the state pass's record (K~, -Wk, U = T Diag(beta) V, e^gamma), indexed
//    by the slot within the segment (frec, fnrec slots per head): the
//    backward's forward pass runs the state pass on these instead of the
//    intra-chunk kernel's.
// A chunk beyond the mid reference's range forms A and P exactly, so its
// state-pass record, T and its reverse-pass record hold; xflag[slot H + h]
// tells kda_bwd_exact whether the chunk is one (1) or not (0), and one lane
// stores 1 into *range_flag (when given) for such a chunk.
template <typename T, int D, bool GS>
__global__ __launch_bounds__((BwdLds<T, D>::NT), 1)
__attribute__((amdgpu_waves_per_eu(4))) void kda_bwd_prep(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, ChunkGeom gm, int H,
    int64_t nslot, int64_t slot_base, int qk_l2norm, float scale, char* __restrict__ brec,
    T* __restrict__ tinv, char* __restrict__ frec, int64_t fnrec, uint32_t* __restrict__ xflag,
    uint32_t* range_flag) {
  using L = BwdLds<T, D, true>;
  using M = Mma<T>;
  using RC = BRec<T, D>;
  using RF = Rec<T, D>;
  constexpr int NW = L::NW, NT = L::NT, LDX = L::LDX, LDC = L::LDC, NTW = 16 / NW;
  constexpr int KC = kC / M::KSTEP, KD = D / M::KSTEP;
  extern __shared__ __align__(16) char smem[];
  const int h = blockIdx.x;
  const int64_t slot = slot_base + blockIdx.y;
  ChunkLoc loc;
  if (!locate(gm, slot, loc)) return;
  BwdSmem<T, D, true> sm(smem);
  BwdRegs R;
  f32x4_t Bm[NTW];
  const int mode = bwd_prologue<T, D, GS, true, true, true, true, true>(
      q, k, g, beta, loc, H, h, qk_l2norm, sm, R, Bm, tinv + (slot * H + h) * (int64_t)(kC * kC));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4;
  const int c = 16 * wave + (lane & 15);
  // v's rows in 16-byte pieces through a resource bounded at the chunk's last
  // valid row (rows past it read as zero), non-temporal as k, q, g; staged in
  // LDS after M, for U
  constexpr int VE = 16 / (int)sizeof(T), PR = D / VE, NPV = kC * PR / NT;
  static_assert(kC * PR % NT == 0, "v's pieces must tile the threads");
  u32x4_t vp[NPV];
  {
    const int rs = H * D;
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(v + (loc.tok0 * H + h) * D), (short)0,
        ((loc.len - 1) * rs + D) * (int)sizeof(T), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int p = i * NT + tid, row = p / PR, cp = p % PR;
      vp[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rv, (uint32_t)((row * rs + cp * VE) * (int)sizeof(T)), 0, 2);
    }
  }
  if (tid == 0) {
    xflag[slot * H + h] = mode == kBwdBeyond ? 1u : 0u;
    if (mode == kBwdBeyond && range_flag != nullptr) *range_flag = 1u;
  }
  char* fr = frec + ((int64_t)h * fnrec + blockIdx.y) * RF::BYTES;
  T* wKT = reinterpret_cast<T*>(fr) + RF::KT;
  T* wWN = reinterpret_cast<T*>(fr) + RF::WN;
  T* wUT = reinterpret_cast<T*>(fr) + RF::UT;
  float* wEG = reinterpret_cast<float*>(fr + RF::BYTES_T);
  // K~ into the region the inverse has finished with, and into the record;
  // Kp = K^ o e^G, and Qp = Q^ o e^G in place of Q^ (G is dead after this)
  f32x4_t kpa[4], wk[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float kt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float eg = __expf(R.G[t][j]);
      kt[j] = R.kh[t][j] * __expf(R.gam - R.G[t][j]);
      kpa[t][j] = R.kh[t][j] * eg;
      R.qh[t][j] *= eg;
      st_f(sm.kt + (16 * t + 4 * grp + j) * LDX + c, kt[j]);
    }
    st_fnat4(wKT, KC, c, 16 * t + 4 * grp, kt[0], kt[1], kt[2], kt[3]);
  }
  const float egam = __expf(R.gam);
  if (grp == 0) wEG[c] = egam;
  __syncthreads();
  T* rec = reinterpret_cast<T*>(brec + ((int64_t)h * nslot + slot) * RC::BYTES);

  // Wk = T Diag(beta) Kp for this wave's columns, B = Kp from registers; the
  // record's -Wk from the transposed product (rows r, four channels a lane)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wk[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t wt = wk[t];
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) {
      wk[t] = M::mma(frag_rm_perm<T>(sm.tb, LDC, 16 * t, ks, lane), acc_frag<T>(kpa, ks), wk[t]);
      wt = M::mma(acc_frag<T>(kpa, ks), frag_rm_perm<T>(sm.tb, LDC, 16 * t, ks, lane), wt);
    }
    st_fnat4(wWN, KD, 16 * t + (lane & 15), 16 * wave + 4 * grp, -wt[0], -wt[1], -wt[2], -wt[3]);
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
    for (int j = 0; j < 4; ++j) z[j] = scale * (R.qh[t][j] - pw[j]);
    st_fnat4_nt(rec + RC::ZF, KC, c, 16 * t + 4 * grp, z[0], z[1], z[2], z[3]);
  }
  // M^T tiles (rows c', column c) = Diag(e^gamma) - K~^T Wk, stored as M
  // (rows c, k = c')
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
    st_fnat4_nt(rec + RC::MF, KD, c, 16 * cb + 4 * grp, m[0], m[1], m[2], m[3]);
  }
  // U = T Diag(beta) V: V row-major in the region after K~'s (the inverse's,
  // free since the prologue), read as column fragments
  T* sv = reinterpret_cast<T*>(smem + L::XB);
  static_assert(2 * L::XB <= L::R0, "V must fit region 0 beside K~");
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    const int p = i * NT + tid, row = p / PR, cp = p % PR;
    *reinterpret_cast<u32x4_t*>(sv + row * LDX + cp * VE) = vp[i];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4_t u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
      u = M::mma(frag_rm_perm<T>(sm.tb, LDC, 16 * t, ks, lane),
                 frag_cm_perm<T>(sv, LDX, 16 * wave, ks, lane), u);
    // rows 16 t + 4 (lane / 16) + j, column c: tile (c / 16, t)
    st4(wUT + ((wave * (kC / 16) + t) * 64 + lane) * 4, u[0], u[1], u[2], u[3]);
  }
}

// ---------------------------------------------------------------------------
// Reverse state pass: dS = M dS' + (scale Z)^T dO chunk by chunk from the last, one
// workgroup per (sequence, head, 16 columns of d_v).  Compute wave w owns rows
// [16 CBW w, 16 CBW (w+1)) of dS in accumulators; dS' crosses LDS once per
// chunk (double-buffered, so one barrier per chunk).  Each chunk's dS' (the
// gradient of the state leaving it) goes to dstates for kda_bwd_intra.  M,
// two thirds of a chunk's record, comes into a ring of three LDS buffers by
// LDS-direct loads of two producer waves, two chunks ahead; scale Z^T and
// the dO slice stay on the compute waves' VGPR path, so the two paths feed
// the CU together.
constexpr int kBwdSliceW = 16;
constexpr int kBwdPassCompute = 256;  // compute threads (four waves)
constexpr int kBwdProducers = 2;
constexpr int kBwdPassThreads = kBwdPassCompute + 64 * kBwdProducers;

template <typename T, int D>
struct BwdPassFrags {
  using M = Mma<T>;
  static constexpr int CBW = D / 64, KD = D / M::KSTEP, KC = kC / M::KSTEP;
  // dO slice of the chunk (64 rows x 16 columns): 16 bytes per lane, VE
  // elements of one row; NO lanes hold the slice, the rest read nothing
  static constexpr int VE = 16 / (int)sizeof(T), LPR = kBwdSliceW / VE, NO = kC * LPR;
  static_assert(NO <= kBwdPassCompute, "the dO slice must fit one load per lane");
  typename M::frag zf[CBW][KC];
  u32x4_t dov;  // raw dO bits of row tid / LPR, columns VE (tid % LPR) ..
};

// LDS of the reverse pass (bytes): the M ring, then the exchange buffers.
template <typename T, int D>
struct BwdPassLds {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int LDS_S = D + 8;                                    // dS' exchange row
  static constexpr int LDO = kC + 16 / ES, LDF = kBwdSliceW + 16 / ES;  // dO^T, dS' store rows
  static constexpr int MB = D * D * ES;                                  // M of one chunk
  static constexpr int NBUF = 3;  // two chunks ahead (the step loop assumes 3)
  static constexpr int SD = NBUF * MB;
  static constexpr int SO = SD + 2 * kBwdSliceW * LDS_S * ES;
  static constexpr int SF = SO + 2 * kBwdSliceW * LDO * ES;
  static constexpr int BYTES = SF + 2 * D * LDF * ES;
  static constexpr int PER_PRODUCER = MB / 1024 / kBwdProducers;  // 1 KiB loads per chunk
  static_assert(MB % (1024 * kBwdProducers) == 0, "M splits into whole 1 KiB loads per producer");
  static_assert(BYTES <= 160 * 1024, "reverse-pass LDS exceeds a CU");
};

template <typename T, int D>
__global__ __launch_bounds__(kBwdPassThreads, 1) void kda_bwd_state_pass(
    const char* __restrict__ brec, int64_t nslot, ChunkGeom gm, int H, int NH, int nslice,
    const T* __restrict__ d_o, const float* __restrict__ dfinal, T* __restrict__ dstates,
    float* __restrict__ dinit) {
  using M = Mma<T>;
  using RC = BRec<T, D>;
  using F = BwdPassFrags<T, D>;
  using PL = BwdPassLds<T, D>;
  constexpr int CBW = F::CBW, KD = F::KD, KC = F::KC, LDS_S = PL::LDS_S;
  constexpr int VE = F::VE, LPR = F::LPR, NO = F::NO;
  // per chunk, double-buffered: dS' in the MFMA type (the exchange), dO^T
  // (columns n, rows r), and dS' untransposed for the store to dstates
  constexpr int LDO = PL::LDO, LDF = PL::LDF;
  extern __shared__ __align__(16) char smem[];
  char* mring = smem;
  T (*sD)[kBwdSliceW * LDS_S] = reinterpret_cast<T (*)[kBwdSliceW * LDS_S]>(smem + PL::SD);
  T (*sO)[kBwdSliceW * LDO] = reinterpret_cast<T (*)[kBwdSliceW * LDO]>(smem + PL::SO);
  T (*sF)[D * LDF] = reinterpret_cast<T (*)[D * LDF]>(smem + PL::SF);
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
  const int nch = (int)(sp.c1 - sp.c0);
  const int len_last = (int)(sp.ntok - (int64_t)(nch - 1) * kC);
  auto rec_of = [&](int ci) {
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(brec + ((int64_t)h * nslot + sp.c0 + ci) * RC::BYTES), (short)0, (int)RC::BYTES,
        kRsrcWord3);
  };
  if (wave >= kBwdPassCompute / 64) {
    // Producer waves: LDS-direct loads of the M block of the chunk of step st
    // (steps run from the last chunk; clamped at the first, so the tail's
    // loads stay inside the sequence) into ring buffer st % 3, two steps
    // ahead.  A producer issues nothing else, so its vmcnt counts exactly
    // these loads: before step st's barrier it waits until only step
    // st + 1's are in flight, and after it -- by which the compute waves have
    // finished reading step st - 1's buffer -- it refills that buffer.
    const int pw = wave - kBwdPassCompute / 64;
    auto produce = [&](int st) {
      const __amdgpu_buffer_rsrc_t rr = rec_of(max(nch - 1 - st, 0));
      char* b = mring + (st % PL::NBUF) * PL::MB;
#pragma unroll
      for (int t = 0; t < PL::PER_PRODUCER; ++t) {
        const int f = pw + t * kBwdProducers;  // 1 KiB block of M
        dma_load16(rr, b + f * 1024, (uint32_t)(RC::MF * sizeof(T) + f * 1024 + lane * 16), 0);
      }
    };
    produce(0);
    produce(1);
    for (int st = 0; st < nch; ++st) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PL::PER_PRODUCER));
      lds_barrier();
      produce(st + 2);
    }
    __builtin_amdgcn_s_waitcnt(0);
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

  // Record fragments through a buffer resource rebased at each chunk's
  // record (scalar), a per-lane offset computed once, and the fragment's
  // offset as a scalar constant: no per-load address math.
  constexpr uint32_t FBY = 64 * M::KPL * sizeof(T);  // bytes of one fragment
  const uint32_t lo_z = (uint32_t)((wave * CBW * KC * 64 + lane) * M::KPL * sizeof(T));
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
  auto load = [&](F& f, int ci) { load_z(f, rec_of(ci), ci); };
  // One chunk step: consumes the fragments in f and fills fn with those of
  // chunk cn, the loads spread over the step (a wave issuing a whole record
  // at once stalls behind the CU's vector memory queue).  dS on entry is dS'
  // of chunk ci (the gradient of the state leaving it): it crosses LDS in
  // the MFMA type, transposed for the product and as is for dstates
  // (kda_bwd_intra reads it only as an operand of that type and in one fp32
  // row sum), whose slice block is then stored in 16-byte pieces.  The dO
  // slice crosses LDS transposed, so each lane's fragment is two runs of rows.
  auto step = [&](const F& f, F& fn, int ci, int cn, int buf, int rb) {
    T* sb = sD[buf];
    T* sf = sF[buf];
    const T* mr = reinterpret_cast<const T*>(mring + rb * PL::MB);  // this chunk's M
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      const int c4 = (wave * CBW + i) * 16 + 4 * grp;
      st_perm4(sb + (lane & 15) * LDS_S, c4, dS[i][0], dS[i][1], dS[i][2], dS[i][3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) st_elem(sf + (c4 + j) * LDF + (lane & 15), dS[i][j]);
    }
    if (threadIdx.x < NO) {
      const int r = threadIdx.x / LPR, cb = VE * (threadIdx.x % LPR);
      if constexpr (sizeof(T) == 2) {
        // as loaded: the slice row-major, [64 rows][16], one 16-byte piece
        *reinterpret_cast<u32x4_t*>(sO[buf] + r * kBwdSliceW + cb) = f.dov;
      } else {
        T* so = sO[buf] + cb * LDO + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) so[e * LDO] = __uint_as_float(f.dov[e]);
      }
    }
    lds_barrier();
    // this wave's M fragments first (read from the ring once, ahead of the
    // products), then the exchanged dS' and dO operands
    typename M::frag mfr[CBW][KD];
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
        mfr[i][ks] = M::load(mr + (((wave * CBW + i) * KD + ks) * 64 + lane) * M::KPL);
    typename M::frag bfr[KD], dof[KC];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) bfr[ks] = frag_at<T>(sb, LDS_S, 0, ks, lane);
#pragma unroll
    for (int ks = 0; ks < KC; ++ks) {
      if constexpr (M::KPL == 8) {
        // kpos order (rows 32ks + 4grp.., then 32ks + 16 + 4grp..) of column
        // n: transpose reads of the row-major slice
        dof[ks] = frag_cm_perm<T>(sO[buf], kBwdSliceW, 0, ks, lane);
      } else {
        dof[ks] = M::load(sO[buf] + (lane & 15) * LDO + 16 * (ks >> 2) + 4 * grp + (ks & 3));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // (keeps the reads ahead of the products)
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) acc = M::mma(f.zf[i][ks], dof[ks], acc);
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) acc = M::mma(mfr[i][ks], bfr[ks], acc);
      dS[i] = acc;
    }
    __builtin_amdgcn_sched_barrier(0);
    const __amdgpu_buffer_rsrc_t rn = rec_of(cn);
    // dS' of chunk ci: this slice's contiguous D x 16 block (sblk), in
    // 16-byte pieces (2 per row in bf16, 4 in fp32)
    T* dst = dstates + ((sp.c0 + ci) * H + h) * (int64_t)D * D + sblk<D>(0, n0);
    {
      constexpr int VEF = 16 / (int)sizeof(T), PPR = kBwdSliceW / VEF, NPC = D * PPR;
#pragma unroll
      for (int pr = 0; pr < (NPC + kBwdPassCompute - 1) / kBwdPassCompute; ++pr) {
        const int pc = pr * kBwdPassCompute + threadIdx.x, row = pc / PPR, cv = VEF * (pc % PPR);
        if (NPC % kBwdPassCompute == 0 || pc < NPC)
          *reinterpret_cast<u32x4_t*>(dst + row * 16 + cv) =
              *reinterpret_cast<const u32x4_t*>(sf + row * LDF + cv);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
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
    step(fa, fc, ci, max(ci - 2, 0), s & 1, 0);
    step(fb, fa, ci - 1, max(ci - 3, 0), (s + 1) & 1, 1);
    step(fc, fb, ci - 2, max(ci - 4, 0), s & 1, 2);
  }
  // (s is a multiple of 3 here: steps s and s + 1 use ring buffers 0 and 1)
  if (s < nch) step(fa, fc, nch - 1 - s, 0, s & 1, 0);
  if (s + 1 < nch) step(fb, fa, nch - 2 - s, 0, (s + 1) & 1, 1);
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
    float* __restrict__ dg, float* __restrict__ dbeta, const T* __restrict__ tinv) {
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
  int mode;
  f32x4_t Bm[L::BM_LDS ? 1 : NTW];  // (unused when the tiles live in LDS)
  // T = (I + A)^-1 as kda_bwd_prep formed it (the same operations on the same
  // inputs, so the same values as forming it here), in 16-byte pieces loaded
  // before the prologue's own loads and put in tb after the prologue
  constexpr int TVE = 16 / (int)sizeof(T), TPR = kC / TVE, TNP = kC * TPR / L::NT;
  static_assert(kC * TPR % L::NT == 0, "T's pieces must tile the threads");
  u32x4_t tpc[TNP];
  {
    const T* tb0 = tinv + (slot * H + h) * (int64_t)(kC * kC);
#pragma unroll
    for (int u = 0; u < TNP; ++u) {
      const int p = u * L::NT + threadIdx.x;
      tpc[u] = *reinterpret_cast<const u32x4_t*>(tb0 + (p / TPR) * kC + TVE * (p % TPR));
    }
  }
  {
    BwdRegs R0;  // recomputed at the end rather than kept live (registers)
    f32x4_t Bp[NTW];
    mode = bwd_prologue<T, D, GS, false, false, false, false>(q, k, g, beta, loc, H, h,
                                                               qk_l2norm, sm, R0, Bp);
#pragma unroll
    for (int u = 0; u < TNP; ++u) {
      const int p = u * L::NT + threadIdx.x;
      *reinterpret_cast<u32x4_t*>(sm.tb + (p / TPR) * L::LDC + TVE * (p % TPR)) = tpc[u];
    }
    if constexpr (!L::BM_LDS) {
#pragma unroll
      for (int tt = 0; tt < NTW; ++tt) Bm[tt] = Bp[tt];
    } else {
      const int lane0 = threadIdx.x & 63, w0 = threadIdx.x >> 6;
#pragma unroll
      for (int tt = 0; tt < NTW; ++tt) {
        const int p = w0 + NW * tt, i = 16 * (p & 3) + (lane0 & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sm.bm[(16 * (p >> 2) + 4 * (lane0 >> 4) + j) * L::LDB + i] = Bp[tt][j];
      }
    }
    if (mode == kBwdMid) {
      // W needs the true Kp = K^ o e^G (it multiplies S): this lane's column
      const int lane0 = threadIdx.x & 63, c0 = 16 * (threadIdx.x >> 6) + (lane0 & 15);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st_f(sm.kp + (16 * t + 4 * (lane0 >> 4) + j) * LDX + c0,
               R0.kh[t][j] * __expf(R0.G[t][j]));
    }
  }
  const int tid = threadIdx.x, wave = tid >> 6;
  int lane = tid & 63, grp = lane >> 4;
  int c = 16 * wave + (lane & 15);  // this lane's column (d_k or d_v)
  auto renew = [&]() {
    lane = opaque(tid) & 63;
    grp = lane >> 4;
    c = 16 * wave + (lane & 15);
  };
  if (mode == kBwdBeyond) {
    // a half of the chunk decays by more than 80 in some channel: its
    // gradients come from kda_bwd_exact, launched after this kernel, which
    // overwrites these placeholders
    const float nan = __builtin_nanf("");
    const int64_t r0 = loc.tok0 * H + h;
    for (int e = tid; e < loc.len * D; e += L::NT) {
      const int64_t o = (r0 + (int64_t)(e / D) * H) * D + e % D;
      st_f(dq + o, nan);
      st_f(dk + o, nan);
      st_f(dv + o, nan);
      if (!GS) dg[o] = nan;
    }
    for (int r = tid; r < loc.len; r += L::NT) {
      dbeta[r0 + (int64_t)r * H] = nan;
      if (GS) dg[r0 + (int64_t)r * H] = nan;
    }
    return;
  }
  renew();
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
  uint32_t sraw[KD][KPL];
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
  uint32_t draw[KD][KPL];
  f32x4_t vmk[4], acc[4], w[4];
  {
    typename M::frag sb[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) sb[ks] = raw_frag(sraw[ks], T{});
    // the dS' columns (k = c) once S's raw registers are free: their latency
    // overlaps the Kp S and T R products
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
#pragma unroll
      for (int e = 0; e < KPL; ++e)
        draw[ks][e] = ld_raw(dS + sblk<D>(ks * M::KSTEP + KPL * grp + e, c));
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
  renew();
  // the key side's k, q, g columns, loaded while this phase runs (the chunk's
  // rows are still in the cache; the registers are free here)
  ColsRaw cols;
  load_cols_raw<T, D, GS>(q, k, g, loc, H, h, c, grp, cols);
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
      // dP strictly below the diagonal; the diagonal stays in fp32 (x1):
      // see the key side
      st_f(sm.pb + r * LDC + i, i < r ? ap[j] : 0.f);
      if (i == r) sm.x1[r] = ap[j];
      st_f(sm.db + r * LDC + i, sm.beta[r] * da);
      // (a select, not a product with the zero mask: with the mid reference the
      // masked tiles above the diagonal may hold inf)
      float bmv;
      if constexpr (L::BM_LDS) bmv = sm.bm[r * L::LDB + i];
      else bmv = Bm[tt][j];
      const float part = sum16(i < r ? da * bmv : 0.f);
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
  // G, k^, q^ again, from the loads issued before the chunk x chunk products
  renew();
  BwdRegs R;
  {
    float gr[4][4];
    cols_from_raw<T>(cols, loc, grp, R, gr);
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
  const bool mid = mode == kBwdMid;
  const float mr = mid ? g_row31(R, lane) : 0.f, em = mid ? __expf(mr) : 1.f;
  // Two passes, each with its own B operands, the gate factors applied per
  // tile so that one tile's accumulators are live at a time:
  //   1. dQp = dO' S^T + dP Km,  dKp = dB Km - Diag(beta) L S^T
  //   2. dKm = dB^T Kp + dP^T Qp,  dK~ = W dS'^T,  rowsum(S o dS')
  // dq^ is complete after pass 1: it goes to LDS at once, into this wave's
  // own columns of Km (read by no other wave, and by this one only into the
  // kmc registers before it), which is where the output stage stages dq;
  // q^ stays in registers for the norm's projection there.
  float dkh[4][4], dG[4][4];  // dkh holds dKp o e^G (+ P's diagonal) after pass 1
  T* sdqh = sm.km;
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
      // dq^ = (dO' S^T) o e^G + (dP Km) o e^(G-m) = (e^m dO' S^T + dP Km) o e^(G-m)
      // with m the reference (e^m = 1 on the fast path); dk^ alike
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] *= em;
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        a = M::mma(frag_at<T>(sm.pb, LDC, 16 * t, ks, lane), kmc[ks], a);  // dP Km
        b = M::mma(frag_at<T>(sm.db, LDC, 16 * t, ks, lane), kmc[ks], b);  // dB Km
      }
      // P's diagonal (dP_rr) enters dq^ as dP_rr k^_r and dk^ as dP_rr q^_r,
      // and the two cancel in dG exactly.  It is kept out of the MFMA
      // products (bf16 operands) and added here in fp32, so dG never forms
      // that cancellation from rounded operands (with fast-forgetting gates
      // the rest of dG is small beside it).
      float ddv[4];
      __asm__ volatile("" ::: "memory");  // this tile's diagonal values only
#pragma unroll
      for (int j = 0; j < 4; ++j) ddv[j] = sm.x1[16 * t + 4 * grp + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * t + 4 * grp + j;
        const float eg = __expf(R.G[t][j] - mr), dd = ddv[j];
        const float dqs = a[j] * eg;  // dq^ without the diagonal term
        const float dqh = dqs + dd * R.kh[t][j];
        st_f(sdqh + r * LDX + c, dqh);
        dkh[t][j] = (b[j] - sm.beta[r] * x[j] * em) * eg + dd * R.qh[t][j];
        // (pass 2 adds k^ dkh to dG: its diagonal term is taken off here)
        dG[t][j] = R.qh[t][j] * dqs - R.kh[t][j] * (dd * R.qh[t][j]);
        const float qd = sum16(R.qh[t][j] * dqh);  // row dot q^ . dq^, this wave's part
        if ((lane & 15) == 0) sm.red[(NW + wave) * kC + r] = qd;
      }
    }
  }
  float rs = 0.f, dgam = 0.f;  // rowsum(S o dS') of row c
  __builtin_amdgcn_sched_barrier(0);
  renew();
  {
    typename M::frag dst[KD], kpc[KC], qpc[KC];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const typename M::frag xs = grow_frag<T, D>(S, c, ks, lane);
      dst[ks] = grow_frag<T, D>(dS, c, ks, lane);
#pragma unroll
      for (int e = 0; e < KPL; ++e) rs += frag_val(xs, e) * frag_val(dst[ks], e);
    }
    if (mid) {
      // Kp relative to the reference again (W, the only product of the true
      // Kp, is done); each wave reads back only its own columns, which its
      // own lanes write: wave-local ordering suffices
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st_f(sm.kp + (16 * t + 4 * grp + j) * LDX + c, R.kh[t][j] * __expf(R.G[t][j] - mr));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
        const float a = dkh[t][j], bm = m[j] * __expf(mr - G), e = kt[j] * __expf(R.gam - G);
        dkh[t][j] = a + bm + e;
        dG[t][j] += R.kh[t][j] * (a - bm - e);
        dgam += R.kh[t][j] * e;
      }
    }
  }
  rs += row_xor1(rs, grp);
  rs += row_xor2(rs, grp);
  dgam += row_xor1(dgam, grp);
  dgam += row_xor2(dgam, grp);
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
      float total;
      const float excl = rows_suffix(run, grp, total) - run;
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
  renew();
  char* ostage = reinterpret_cast<char*>(sm.kp);
  T* sdk = reinterpret_cast<T*>(ostage);
  T* sdq = reinterpret_cast<T*>(ostage + L::XB);  // = sdqh, dq^ already there
  float* sdg = reinterpret_cast<float*>(ostage + 2 * L::XB);
  constexpr int LDG = D + 4;
  static_assert(2 * L::XB + kC * LDG * 4 <= 4 * L::XB, "staged gradients must fit");
  static_assert(L::KM == L::KP + L::XB, "dq^ is staged where the output stage reads dq");
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * t + 4 * grp + j;
      float gk = dkh[t][j];
      if (qk_l2norm) {
        gk = sm.rk[r] * (gk - sm.x1[r] * R.kh[t][j]);
        const float gq = ld_f(sdq + r * LDX + c);
        st_f(sdq + r * LDX + c, sm.rq[r] * (gq - sm.x2[r] * R.qh[t][j]));
      }
      st_f(sdk + r * LDX + c, gk);
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
// kda_bwd_exact: the gradients of the chunks beyond the mid reference's
// exponent range (xflag set by kda_bwd_prep), in plain fp32 arithmetic with
// every gate factor formed from its own exponent difference, so no factor
// exceeds 1 for any gate ([XT §4] names the chunk form's e^(-G) division as
// its precision concern).  The same closed forms as the file header, each
// e^(G_r - G_i) product summed entry by entry:
//   (Kp Km^T)_ri = sum_c k^_rc k^_ic e^(G_rc - G_ic)   P_ri = sum_c q^_rc k^_ic e^(...)
//   dq^_rc = e^G_rc (dO' S^T)_rc + sum_(i<=r) dP_ri k^_ic e^(G_rc - G_ic)
//   dKp o e^G  = -beta_r e^G_rc (L S^T)_rc + sum_(i<r) dB_ri k^_ic e^(G_rc - G_ic)
//   dKm o e^-G = sum_(s>r) dB_sr k^_sc e^(G_sc - G_rc) + sum_(s>=r) dP_sr q^_sc e^(G_sc - G_rc)
//   dK~ o e^(gamma-G) = e^(gamma_c - G_rc) (W dS'^T)_rc
// S, dS' and T are the stored copies the other kernels read (S, dS'
// slice-blocked, T row-major, in the MFMA type).  A persistent grid walks
// every (slot, head) and skips the unflagged ones (one word each).  k^, q^,
// G, dA and dP live in LDS; the chunk's other intermediates (fp32, among
// them transposed copies of S and dS') in this workgroup's part of `scr`
// (ExScr<D>, L2-resident).  Each thread owns a 4 x 4 tile of every product
// (16-byte loads of the operand that is contiguous along the tile's columns,
// four broadcast loads of the other), and of the per-element terms, whose
// sums over the chunk rows carry a factor e^(G_rc - G_ic) per (r, i, c).
// No MFMA and one chunk per workgroup: only for chunks the fast kernels
// cannot represent.
constexpr int kExactThreads = 256;
constexpr int kExactMaxGroups = 256;  // one per CU (132 KB of LDS each)
template <int D>
struct ExScr {
  static constexpr int64_t CD = (int64_t)kC * D, CC = (int64_t)kC * kC;
  // [kC][D]: Kp = K^ o e^G, K~ = K^ o e^(gamma-G), X = V - Kp S (V first),
  // W, dO', dW (then dG), L, dO' S^T (then dq^), L S^T (then dk^terms),
  // W dS'^T (then dK~ o K~ / K^)
  static constexpr int64_t KP = 0, KT = KP + CD, X = KT + CD, W = X + CD, OP = W + CD;
  static constexpr int64_t DW = OP + CD, LM = DW + CD, DOS = LM + CD, LS = DOS + CD;
  static constexpr int64_t WDS = LS + CD;
  // [kC][kC]: Kp Km^T, P, T
  static constexpr int64_t KPM = WDS + CD, PM = KPM + CC, TM = PM + CC;
  // [D][D]: S and dS' transposed ([n][c])
  static constexpr int64_t ST = TM + CC, DST = ST + (int64_t)D * D;
  static constexpr int64_t END = DST + (int64_t)D * D;
  static constexpr int64_t BYTES = (END * 4 + 255) / 256 * 256;
  // LDS: k^, q^, G [kC][D]; dA, dP [kC][kC]; beta, rk, rq, two dot products [kC]; gamma [D]
  static constexpr int LDS = (3 * kC * D + 2 * kC * kC + 5 * kC + D) * 4;
};

__device__ __forceinline__ void ex_ld4(const float* p, float (&x)[4]) {
  const float4 t = *reinterpret_cast<const float4*>(p);
  x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
}
__device__ __forceinline__ void ex_ld4(const bf16* p, float (&x)[4]) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  x[0] = bf_val(t.x & 0xffffu); x[1] = bf_val(t.x >> 16);
  x[2] = bf_val(t.y & 0xffffu); x[3] = bf_val(t.y >> 16);
}
__device__ __forceinline__ void ex_st4(float* p, const float (&x)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
// acc[i][j] += sum_(kk in [k0, k1)) a(kk)[i] b(kk)[j]
template <typename FA, typename FB>
__device__ __forceinline__ void ex_mm(float (&acc)[4][4], int k0, int k1, FA fa, FB fb) {
#pragma unroll 2
  for (int kk = k0; kk < k1; ++kk) {
    float a[4], b[4];
    fa(kk, a);
    fb(kk, b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
  }
}

template <typename T, int D, bool GS>
__global__ __launch_bounds__(kExactThreads) void kda_bwd_exact(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const T* __restrict__ d_o,
    const T* __restrict__ states, const T* __restrict__ dstates, const T* __restrict__ tinv,
    const uint32_t* __restrict__ xflag, ChunkGeom gm, int H, int64_t nslot, int qk_l2norm,
    float scale, float* __restrict__ scr, T* __restrict__ dq, T* __restrict__ dk,
    T* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta) {
  using X = ExScr<D>;
  constexpr int NT = kExactThreads;
  constexpr int TD = kC / 4 * (D / 4), TC = kC / 4 * (kC / 4);  // 4 x 4 tiles of C x D, C x C
  extern __shared__ __align__(16) char smem[];
  float* sk = reinterpret_cast<float*>(smem);
  float* sq = sk + kC * D;
  float* sg = sq + kC * D;
  float* lda = sg + kC * D;
  float* ldp = lda + kC * kC;
  float* sb = ldp + kC * kC;
  float* rk = sb + kC;
  float* rq = rk + kC;
  float* dotq = rq + kC;
  float* dotk = dotq + kC;
  float* gam = dotk + kC;
  float* w = scr + blockIdx.x * (X::BYTES / 4);
  float *kp = w + X::KP, *kt = w + X::KT, *xm = w + X::X, *wm = w + X::W, *op = w + X::OP;
  float *dw = w + X::DW, *lm = w + X::LM, *dos = w + X::DOS, *ls = w + X::LS, *wds = w + X::WDS;
  float *kpm = w + X::KPM, *pm = w + X::PM, *tm = w + X::TM, *st = w + X::ST, *dst = w + X::DST;
  const int tid = threadIdx.x;
  // Items (slot, head) = slot H + h.  Each pass looks at NT items at once,
  // thread t at item base + t gridDim.x (its flag, after locating the slot),
  // and lists the flagged ones in LDS; then the workgroup takes them one by
  // one.  (Walking the items one flag load at a time cost ~25 us per call
  // with nothing flagged.)
  __shared__ int s_list[NT];
  __shared__ int s_cnt;
  const int64_t nitem = nslot * H;
  for (int64_t base = blockIdx.x; base < nitem; base += (int64_t)gridDim.x * NT) {
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    {
      const int64_t it = base + (int64_t)tid * gridDim.x;
      ChunkLoc l0;
      if (it < nitem && locate(gm, it / H, l0) && xflag[it] != 0u) s_list[atomicAdd(&s_cnt, 1)] = tid;
    }
    __syncthreads();
    const int nflag = s_cnt;
    for (int jf = 0; jf < nflag; ++jf) {
      const int64_t item = base + (int64_t)s_list[jf] * gridDim.x;
      const int64_t slot = item / H;
      const int h = (int)(item % H);
      ChunkLoc loc;
      locate(gm, slot, loc);
      const int len = loc.len;
      const int64_t row0 = loc.tok0 * H + h;
      const T* S = states + (slot * H + h) * (int64_t)D * D;
      const T* dS = dstates + (slot * H + h) * (int64_t)D * D;
      const T* tb = tinv + (slot * H + h) * (int64_t)(kC * kC);
      // raw rows (zero past the chunk's end), beta, V and dO' = scale dO, T,
      // S and dS' transposed
      for (int e = tid; e < kC * D; e += NT) {
        const int r = e / D, c = e % D;
        const bool ok = r < len;
        const int64_t o = (row0 + (int64_t)r * H) * D + c;
        sk[e] = ok ? ld_f(k + o) : 0.f;
        sq[e] = ok ? ld_f(q + o) : 0.f;
        sg[e] = ok ? (GS ? g[row0 + (int64_t)r * H] : g[o]) : 0.f;
        xm[e] = ok ? ld_f(v + o) : 0.f;
        op[e] = ok ? scale * ld_f(d_o + o) : 0.f;
      }
      if (tid < kC) sb[tid] = tid < len ? beta[row0 + (int64_t)tid * H] : 0.f;
      for (int e = tid; e < kC * kC; e += NT) tm[e] = (e % kC) <= (e / kC) ? ld_f(tb + e) : 0.f;
      for (int e = tid; e < D * D; e += NT) {  // e = n D + c
        const int n = e / D, c = e % D;
        st[e] = ld_f(S + sblk<D>(c, n));
        dst[e] = ld_f(dS + sblk<D>(c, n));
      }
      __syncthreads();
      if (tid < kC) {
        float a = 0.f, b = 0.f;
#pragma unroll 4
        for (int c = 0; c < D; ++c) {
          a += sk[tid * D + c] * sk[tid * D + c];
          b += sq[tid * D + c] * sq[tid * D + c];
        }
        rk[tid] = qk_l2norm ? rsqrtf(a + kNormEps) : 1.f;
        rq[tid] = qk_l2norm ? rsqrtf(b + kNormEps) : 1.f;
      } else if (tid < kC + D) {  // in-chunk cumulative gate of channel c
        const int c = tid - kC;
        float run = 0.f;
        for (int r = 0; r < kC; ++r) {
          run += sg[r * D + c];
          sg[r * D + c] = run;
        }
        gam[c] = run;
      }
      __syncthreads();
      // k^, q^; Kp = K^ o e^G, K~ = K^ o e^(gamma-G) (every exponent <= 0)
      for (int e = tid; e < kC * D; e += NT) {
        const int r = e / D, c = e % D;
        const float kh = sk[e] * rk[r];
        sk[e] = kh;
        sq[e] *= rq[r];
        kp[e] = kh * __expf(sg[e]);
        kt[e] = kh * __expf(gam[c] - sg[e]);
      }
      __syncthreads();
      // X = V - Kp S; Kp Km^T and P, each entry from its own exponents
      for (int t = tid; t < TD; t += NT) {
        const int r0 = 4 * (t / (D / 4)), n0 = 4 * (t % (D / 4));
        float acc[4][4] = {};
        ex_mm(acc, 0, D, [&](int c, float (&a)[4]) {
          for (int i = 0; i < 4; ++i) a[i] = kp[(r0 + i) * D + c];
        }, [&](int c, float (&b)[4]) { ex_ld4(S + sblk<D>(c, n0), b); });
        for (int i = 0; i < 4; ++i) {
          float x[4];
          ex_ld4(xm + (r0 + i) * D + n0, x);
          for (int j = 0; j < 4; ++j) x[j] -= acc[i][j];
          ex_st4(xm + (r0 + i) * D + n0, x);
        }
      }
      for (int t = tid; t < TC; t += NT) {
        const int r0 = 4 * (t / (kC / 4)), i0 = 4 * (t % (kC / 4));
        float a[4][4] = {}, pp[4][4] = {};
        if (i0 <= r0 + 3) {
#pragma unroll 2
          for (int c = 0; c < D; ++c) {
            float kr[4], qr[4], gr[4], ki[4], gi[4];
            for (int u = 0; u < 4; ++u) {
              kr[u] = sk[(r0 + u) * D + c];
              qr[u] = sq[(r0 + u) * D + c];
              gr[u] = sg[(r0 + u) * D + c];
              ki[u] = sk[(i0 + u) * D + c];
              gi[u] = sg[(i0 + u) * D + c];
            }
            for (int u = 0; u < 4; ++u)
              for (int j = 0; j < 4; ++j) {
                const float x = i0 + j <= r0 + u ? ki[j] * __expf(gr[u] - gi[j]) : 0.f;
                a[u][j] += kr[u] * x;
                pp[u][j] += qr[u] * x;
              }
          }
        }
        for (int u = 0; u < 4; ++u)
          for (int j = 0; j < 4; ++j) {
            const int r = r0 + u, i = i0 + j;
            kpm[r * kC + i] = i < r ? a[u][j] : 0.f;
            pm[r * kC + i] = i <= r ? pp[u][j] : 0.f;
          }
      }
      __syncthreads();
      // W = T Diag(beta) X
      for (int t = tid; t < TD; t += NT) {
        const int r0 = 4 * (t / (D / 4)), n0 = 4 * (t % (D / 4));
        float acc[4][4] = {};
        ex_mm(acc, 0, r0 + 4, [&](int i, float (&a)[4]) {
          for (int u = 0; u < 4; ++u) a[u] = tm[(r0 + u) * kC + i] * sb[i];
        }, [&](int i, float (&b)[4]) { ex_ld4(xm + i * D + n0, b); });
        for (int i = 0; i < 4; ++i) ex_st4(wm + (r0 + i) * D + n0, acc[i]);
      }
      __syncthreads();
      // dW = P^T dO' + K~ dS'
      for (int t = tid; t < TD; t += NT) {
        const int r0 = 4 * (t / (D / 4)), n0 = 4 * (t % (D / 4));
        float acc[4][4] = {};
        ex_mm(acc, r0, kC, [&](int s2, float (&a)[4]) { ex_ld4(pm + s2 * kC + r0, a); },
              [&](int s2, float (&b)[4]) { ex_ld4(op + s2 * D + n0, b); });
        ex_mm(acc, 0, D, [&](int c, float (&a)[4]) {
          for (int u = 0; u < 4; ++u) a[u] = kt[(r0 + u) * D + c];
        }, [&](int c, float (&b)[4]) { ex_ld4(dS + sblk<D>(c, n0), b); });
        for (int i = 0; i < 4; ++i) ex_st4(dw + (r0 + i) * D + n0, acc[i]);
      }
      __syncthreads();
      // L = T^T dW
      for (int t = tid; t < TD; t += NT) {
        const int r0 = 4 * (t / (D / 4)), n0 = 4 * (t % (D / 4));
        float acc[4][4] = {};
        ex_mm(acc, r0, kC, [&](int s2, float (&a)[4]) { ex_ld4(tm + s2 * kC + r0, a); },
              [&](int s2, float (&b)[4]) { ex_ld4(dw + s2 * D + n0, b); });
        for (int i = 0; i < 4; ++i) ex_st4(lm + (r0 + i) * D + n0, acc[i]);
      }
      __syncthreads();
      // dV = Diag(beta) L; dA = -tril_-1(L W^T), dP = tril(dO' W^T) (LDS);
      // dO' S^T, L S^T, W dS'^T
      for (int e = tid; e < kC * D; e += NT) {
        const int r = e / D, n = e % D;
        if (r < len) st_f(dv + (row0 + (int64_t)r * H) * D + n, sb[r] * lm[e]);
      }
      for (int t = tid; t < TC; t += NT) {
        const int r0 = 4 * (t / (kC / 4)), i0 = 4 * (t % (kC / 4));
        float a[4][4] = {}, pp[4][4] = {};
        if (i0 <= r0 + 3) {
#pragma unroll 1
          for (int n = 0; n < D; n += 4) {
            float lr[4][4], orow[4][4], wi[4][4];
            for (int u = 0; u < 4; ++u) {
              ex_ld4(lm + (r0 + u) * D + n, lr[u]);
              ex_ld4(op + (r0 + u) * D + n, orow[u]);
              ex_ld4(wm + (i0 + u) * D + n, wi[u]);
            }
            for (int u = 0; u < 4; ++u)
              for (int j = 0; j < 4; ++j)
                for (int e = 0; e < 4; ++e) {
                  a[u][j] += lr[u][e] * wi[j][e];
                  pp[u][j] += orow[u][e] * wi[j][e];
                }
          }
        }
        for (int u = 0; u < 4; ++u)
          for (int j = 0; j < 4; ++j) {
            const int r = r0 + u, i = i0 + j;
            lda[r * kC + i] = i < r ? -a[u][j] : 0.f;
            ldp[r * kC + i] = i <= r ? pp[u][j] : 0.f;
          }
      }
      for (int t = tid; t < TD; t += NT) {
        const int r0 = 4 * (t / (D / 4)), c0 = 4 * (t % (D / 4));
        float a1[4][4] = {}, a2[4][4] = {}, a3[4][4] = {};
#pragma unroll 1
        for (int n = 0; n < D; ++n) {
          float o4[4], l4[4], w4[4], s4[4], d4[4];
          for (int u = 0; u < 4; ++u) {
            o4[u] = op[(r0 + u) * D + n];
            l4[u] = lm[(r0 + u) * D + n];
            w4[u] = wm[(r0 + u) * D + n];
          }
          ex_ld4(st + n * D + c0, s4);
          ex_ld4(dst + n * D + c0, d4);
          for (int u = 0; u < 4; ++u)
            for (int j = 0; j < 4; ++j) {
              a1[u][j] += o4[u] * s4[j];
              a2[u][j] += l4[u] * s4[j];
              a3[u][j] += w4[u] * d4[j];
            }
        }
        for (int u = 0; u < 4; ++u) {
          ex_st4(dos + (r0 + u) * D + c0, a1[u]);
          ex_st4(ls + (r0 + u) * D + c0, a2[u]);
          ex_st4(wds + (r0 + u) * D + c0, a3[u]);
        }
      }
      __syncthreads();
      // dbeta = rowsum(L o X) + rowsum(dA o Kp Km^T)
      if (tid < len) {
        const int r = tid;
        float a = 0.f;
#pragma unroll 4
        for (int n = 0; n < D; ++n) a += lm[r * D + n] * xm[r * D + n];
        for (int i = 0; i < r; ++i) a += lda[r * kC + i] * kpm[r * kC + i];
        dbeta[row0 + (int64_t)r * H] = a;
      }
      // per element: dq^ (into dos), dk^ (into ls), dK~ o K~ / k^ (into wds)
      // and dG (into dw)
      for (int t = tid; t < TD; t += NT) {
        const int r0 = 4 * (t / (D / 4)), c0 = 4 * (t % (D / 4));
        float gr[4][4], dqv[4][4], tp[4][4], tmv[4][4];
        for (int u = 0; u < 4; ++u) {
          ex_ld4(sg + (r0 + u) * D + c0, gr[u]);
          float a1[4], a2[4];
          ex_ld4(dos + (r0 + u) * D + c0, a1);
          ex_ld4(ls + (r0 + u) * D + c0, a2);
          for (int j = 0; j < 4; ++j) {
            const float eg = __expf(gr[u][j]);
            dqv[u][j] = eg * a1[j];
            tp[u][j] = -sb[r0 + u] * eg * a2[j];
            tmv[u][j] = 0.f;
          }
        }
#pragma unroll 1
        for (int i = 0; i < kC; ++i) {
          float ki[4], qi[4], gi[4], pc[4], ac[4];
          ex_ld4(sk + i * D + c0, ki);
          ex_ld4(sq + i * D + c0, qi);
          ex_ld4(sg + i * D + c0, gi);
          ex_ld4(ldp + i * kC + r0, pc);  // dP_(i, r0..r0+3)
          ex_ld4(lda + i * kC + r0, ac);  // dA_(i, r0..r0+3)
          const float bi = sb[i];
          for (int u = 0; u < 4; ++u) {
            const int r = r0 + u;
            const float pr = ldp[r * kC + i], br = sb[r] * lda[r * kC + i];
            for (int j = 0; j < 4; ++j) {
              // i <= r: e^(G_rc - G_ic) <= 1; i >= r: e^(G_ic - G_rc) <= 1
              const float x = i <= r ? __expf(gr[u][j] - gi[j]) : 0.f;
              const float y = i >= r ? __expf(gi[j] - gr[u][j]) : 0.f;
              dqv[u][j] += pr * ki[j] * x;
              tp[u][j] += br * ki[j] * x;
              tmv[u][j] += (pc[u] * qi[j] + bi * ac[u] * ki[j]) * y;
            }
          }
        }
        for (int u = 0; u < 4; ++u) {
          float w4[4], kr[4], qr[4], o1[4], o2[4], o3[4], o4[4];
          ex_ld4(wds + (r0 + u) * D + c0, w4);
          ex_ld4(sk + (r0 + u) * D + c0, kr);
          ex_ld4(sq + (r0 + u) * D + c0, qr);
          for (int j = 0; j < 4; ++j) {
            const float ttv = __expf(gam[c0 + j] - gr[u][j]) * w4[j];
            o1[j] = dqv[u][j];
            o2[j] = tp[u][j] + tmv[u][j] + ttv;
            o3[j] = kr[j] * ttv;  // dK~ o K~, summed over rows for dgamma
            o4[j] = kr[j] * (tp[u][j] - tmv[u][j] - ttv) + qr[j] * dqv[u][j];
          }
          ex_st4(dos + (r0 + u) * D + c0, o1);
          ex_st4(ls + (r0 + u) * D + c0, o2);
          ex_st4(wds + (r0 + u) * D + c0, o3);
          ex_st4(dw + (r0 + u) * D + c0, o4);
        }
      }
      __syncthreads();
      // dgamma = colsum(dK~ o K~) + e^gamma o rowsum(S o dS'), on the last row;
      // then the in-chunk prefix sum reversed; the norms' row dot products
      if (tid < D) {
        const int c = tid;
        float a = 0.f, b = 0.f;
        for (int r = 0; r < kC; ++r) a += wds[r * D + c];
#pragma unroll 4
        for (int n = 0; n < D; ++n) b += st[n * D + c] * dst[n * D + c];
        float run = a + __expf(gam[c]) * b;
        for (int r = kC - 1; r >= 0; --r) {
          run += dw[r * D + c];
          dw[r * D + c] = run;
        }
      } else if (tid < D + kC) {
        const int r = tid - D;
        float a = 0.f, b = 0.f;
#pragma unroll 4
        for (int c = 0; c < D; ++c) {
          a += sq[r * D + c] * dos[r * D + c];
          b += sk[r * D + c] * ls[r * D + c];
        }
        dotq[r] = a;
        dotk[r] = b;
      }
      __syncthreads();
      // outputs: dg, and dq, dk through the norm (dx = r (dx^ - (x^ . dx^) x^))
      for (int e = tid; e < kC * D; e += NT) {
        const int r = e / D, c = e % D;
        if (r >= len) continue;
        const int64_t o = (row0 + (int64_t)r * H) * D + c;
        const float vq = qk_l2norm ? rq[r] * (dos[e] - dotq[r] * sq[e]) : dos[e];
        const float vk = qk_l2norm ? rk[r] * (ls[e] - dotk[r] * sk[e]) : ls[e];
        st_f(dq + o, vq);
        st_f(dk + o, vk);
        if (!GS) dg[o] = dw[e];
      }
      if (GS && tid < len) {
        float a = 0.f;
        for (int c = 0; c < D; ++c) a += dw[tid * D + c];
        dg[row0 + (int64_t)tid * H] = a;
      }
      __syncthreads();  // LDS and scratch are reused by the next item
    }
    __syncthreads();  // s_cnt and s_list are rewritten by the next pass
  }
}

// ---------------------------------------------------------------------------
// Workspace: [forward workspace | S per slot | dS' per slot | M, Z^T records |
// T per (slot, head) | chunk map | exact-path flag per (slot, head) | exact
// kernel's scratch].  Slots are sized for the larger of the dense and varlen
// bounds.
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

struct BwdPlan {
  int64_t slots, fwd, states, recs, tinv, map, xflag, xgroups, xscr, total;
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
  p.tinv = align256(p.slots * d.heads * (int64_t)kC * kC * (d.dtype == KDA_DTYPE_BF16 ? 2 : 4));
  p.map = 2 * align256(((int64_t)d.num_seqs + 1) * 4);
  p.xflag = align256(p.slots * d.heads * 4);
  p.xgroups = std::max<int64_t>(1, std::min<int64_t>(kExactMaxGroups, p.slots * d.heads));
  p.xscr = p.xgroups * (d.dk == 128 ? ExScr<128>::BYTES : ExScr<64>::BYTES);
  p.total = p.fwd + 2 * p.states + p.recs + p.tinv + p.map + p.xflag + p.xscr;
  return p;
}

// The backward's record stage for the forward's state pass (see
// launch_chunk_states): kda_bwd_prep over one segment of chunk slots.
template <typename T>
struct PrepStage {
  const T *q, *k, *v;
  const float *g, *beta;
  ChunkGeom gm;
  int H;
  int64_t nslot;
  int qk_l2norm;
  float scale;
  char* brec;
  T* tinv;
  bool gate_per_head;
  uint32_t* xflag;
  uint32_t* range_flag;
};

template <typename T, int D>
hipError_t prep_stage(void* ctx, int64_t s0, int64_t s1, char* recs, hipStream_t stream) {
  const PrepStage<T>& c = *static_cast<const PrepStage<T>*>(ctx);
  using LP = BwdLds<T, D, true>;
  auto prep = c.gate_per_head ? kda_bwd_prep<T, D, true> : kda_bwd_prep<T, D, false>;
  hipLaunchKernelGGL(prep, dim3(c.H, (unsigned)(s1 - s0)), dim3(LP::NT), LP::BYTES, stream, c.q,
                     c.k, c.v, c.g, c.beta, c.gm, c.H, c.nslot, s0, c.qk_l2norm, c.scale, c.brec,
                     c.tinv, recs, s1 - s0, c.xflag, c.range_flag);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_bwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* init_state, const int32_t* cu,
                   const void* d_o, const float* d_final, void* dq, void* dk, void* dv,
                   float* dg, float* dbeta, float* d_init, uint32_t* range_flag, char* ws,
                   hipStream_t stream) {
  using L = BwdLds<T, D>;
  const BwdPlan p = bwd_plan(d);
  const bool varlen = cu != nullptr;
  const int H = d.heads, NH = d.num_seqs * d.heads;
  T* states = reinterpret_cast<T*>(ws + p.fwd);
  T* dstates = reinterpret_cast<T*>(ws + p.fwd + p.states);
  char* recs = ws + p.fwd + 2 * p.states;
  T* tinv = reinterpret_cast<T*>(ws + p.fwd + 2 * p.states + p.recs);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + p.fwd + 2 * p.states + p.recs + p.tinv);
  int32_t* cu_s = chunk_off + (p.map / 2) / 4;
  char* xbase = ws + p.fwd + 2 * p.states + p.recs + p.tinv + p.map;
  uint32_t* xflag = reinterpret_cast<uint32_t*>(xbase);
  float* xscr = reinterpret_cast<float*>(xbase + p.xflag);
  const int64_t nslot = chunk_slot_bound(d, varlen);

  ChunkGeom gm{nullptr, nullptr, d.seqlen, (d.seqlen + kC - 1) / kC, d.num_seqs};
  if (varlen) {
    hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(kThreads), 0, stream, cu, d.num_seqs,
                       d.seqlen, cu_s, chunk_off);
    gm = ChunkGeom{cu_s, chunk_off, d.seqlen, 0, d.num_seqs};
  }
  using LP = BwdLds<T, D, true>;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t e = once_per_device(attr_done, [&]() {
    for (const void* fn : {(const void*)kda_bwd_prep<T, D, false>,
                           (const void*)kda_bwd_prep<T, D, true>}) {
      hipError_t ea = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LP::BYTES);
      if (ea != hipSuccess) return ea;
    }
    for (const void* fn : {(const void*)kda_bwd_intra<T, D, false>,
                           (const void*)kda_bwd_intra<T, D, true>}) {
      hipError_t ea = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
      if (ea != hipSuccess) return ea;
    }
    for (const void* fn : {(const void*)kda_bwd_exact<T, D, false>,
                           (const void*)kda_bwd_exact<T, D, true>}) {
      hipError_t ea = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          ExScr<D>::LDS);
      if (ea != hipSuccess) return ea;
    }
    return hipFuncSetAttribute((const void*)kda_bwd_state_pass<T, D>,
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               BwdPassLds<T, D>::BYTES);
  });
  if (e != hipSuccess) return e;
  // the forward pass: per segment of chunk slots, kda_bwd_prep writes the
  // state pass's records (and the reverse pass's records and T of those
  // slots), then the state pass writes the state entering every chunk
  PrepStage<T> ps{(const T*)q, (const T*)k, (const T*)v, g, beta, gm, H, nslot,
                  d.qk_l2norm, d.scale, recs, tinv, d.gate_per_head != 0, xflag, range_flag};
  kda_desc_t df = d;
  df.ckpt_every = 0;
  e = launch_chunk_states(df, init_state, cu, states, ws, prep_stage<T, D>, &ps, stream);
  if (e != hipSuccess) return e;
  // chunk slots go in the grid's y dimension, at most kMaxGridY per launch
  constexpr int64_t kMaxGridY = 32768;
  const int nslice = D / kBwdSliceW;
  const int nhpad = (NH + 7) / 8 * 8;
  constexpr int kPassLds = BwdPassLds<T, D>::BYTES;
  hipLaunchKernelGGL((kda_bwd_state_pass<T, D>), dim3(nhpad * nslice), dim3(kBwdPassThreads),
                     kPassLds, stream, recs, nslot, gm, H, NH, nslice, (const T*)d_o, d_final,
                     dstates, d_init);
  auto intra = d.gate_per_head ? kda_bwd_intra<T, D, true> : kda_bwd_intra<T, D, false>;
  for (int64_t sb = 0; sb < nslot; sb += kMaxGridY) {
    const unsigned ny = (unsigned)std::min<int64_t>(kMaxGridY, nslot - sb);
    hipLaunchKernelGGL(intra, dim3(H, ny), dim3(L::NT), L::BYTES, stream, (const T*)q,
                       (const T*)k, (const T*)v, g, beta, (const T*)d_o, states, dstates, gm, H,
                       sb, d.qk_l2norm, d.scale, (T*)dq, (T*)dk, (T*)dv, dg, dbeta, tinv);
  }
  // the chunks beyond the mid reference's range (prep's flags), exactly
  auto exact = d.gate_per_head ? kda_bwd_exact<T, D, true> : kda_bwd_exact<T, D, false>;
  const unsigned ngx = (unsigned)std::max<int64_t>(1, std::min<int64_t>(p.xgroups, nslot * H));
  hipLaunchKernelGGL(exact, dim3(ngx), dim3(kExactThreads), ExScr<D>::LDS, stream, (const T*)q,
                     (const T*)k, (const T*)v, g, beta, (const T*)d_o, states, dstates, tinv,
                     xflag, gm, H, nslot, d.qk_l2norm, d.scale, xscr, (T*)dq, (T*)dk, (T*)dv,
                     dg, dbeta);
  return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_workspace_bytes(const kda_desc_t& d) { return (size_t)bwd_plan(d).total; }

hipError_t launch_chunk_bwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, const void* d_o, const float* d_final,
                            void* dq, void* dk, void* dv, float* dg, float* dbeta,
                            float* d_init, uint32_t* range_flag, void* workspace,
                            hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  if (d.dtype == KDA_DTYPE_BF16) {
    if (d.dk == 128)
      return run_bwd<bf16, 128>(d, q, k, v, g, beta, init_state, cu_seqlens, d_o, d_final, dq,
                                dk, dv, dg, dbeta, d_init, range_flag, ws, stream);
    return run_bwd<bf16, 64>(d, q, k, v, g, beta, init_state, cu_seqlens, d_o, d_final, dq, dk,
                             dv, dg, dbeta, d_init, range_flag, ws, stream);
  }
  if (d.dk == 64)
    return run_bwd<float, 64>(d, q, k, v, g, beta, init_state, cu_seqlens, d_o, d_final, dq, dk,
                              dv, dg, dbeta, d_init, range_flag, ws, stream);
  return hipErrorInvalidValue;  // fp32 at d = 128: rejected by the caller
}

}  // namespace kda
