// kda_chunk.hip -- chunkwise KDA prefill for gfx950 (MI355X).
//
// Pages cited (by title and section):
//   [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
//   [XD] xiudou.site, "Kimi Delta Attention：把遗忘门做到每个通道"
//
// Method.  [XT §5] splits the sequence into chunks of C = 64 tokens: work
// inside a chunk is parallel, chunks are chained through the d x d state,
// and the UT transform turns a chunk's rank-1 transitions into dense
// products.  [XT §4] notes that the shared key of (I - beta k k^T) Diag(alpha)
// is what keeps this cheap.  Written out for one chunk of n <= 64 rows with
// entering state S (d_k x d_v, rows = key channels):
//
//   G_r   = sum_(s<=r) g_s            cumulative log-gate, per channel
//   A_ri  = beta_r sum_c k_rc k_ic e^(G_rc - G_ic)          (i < r)
//   T     = (I + A)^-1                unit lower triangular
//   U     = T Diag(beta) V            Wk = T Diag(beta) (K o e^G)
//   W     = U - Wk S                  the chunk's "pseudo-values"
//   P_ri  = sum_c q_rc k_ic e^(G_rc - G_ic)                  (i <= r)
//   O     = (Q o e^G) S + P W         inter-chunk + intra-chunk read-out
//   S'    = Diag(e^gamma) S + (K o e^(gamma - G))^T W,   gamma = G_n
//
// This follows by induction from the per-token update
// S_t = Diag(a_t) S_(t-1) + k_t u_t^T, u_t = beta_t (v_t - (Diag(a_t) S_(t-1))^T k_t)
// [XT §3]: S_r = Diag(e^G_r) S + sum_(i<=r) Diag(e^(G_r - G_i)) k_i u_i^T, and
// stacking the u_r gives (I + A) U_rows = Diag(beta)(V - (K o e^G) S).  It is
// exact; only rounding separates it from the token-by-token recurrence.
//
// Kernels.
//   K1 (kda_intra_chunk): one workgroup per (chunk, head), fully parallel.
//     q/k L2 norm, the in-chunk prefix sum of g, A and P on MFMA, the
//     triangular inverse T in fp32, then U and Wk on MFMA.  Writes the
//     operands K2 consumes to the workspace.
//   K2 (kda_state_pass): one workgroup per (sequence, head, d_v slice),
//     sequential over that sequence's chunks.  The fp32 state slice lives in
//     MFMA accumulators for the whole sequence; per chunk it forms W, the
//     output and the next state with three MFMA chains.  On the bf16 path two
//     producer waves bring the chain's record fragments into LDS by
//     LDS-direct loads beside the four compute waves.
//   The d_v columns of the state never mix, so splitting d_v across
//   workgroups lets one head's chain use several CUs; the slices of one head
//   are placed on one XCD so their shared operand reads hit the same L2.
//
// Exponent handling.  g <= 0 makes G non-increasing inside a chunk.  A and P
// factor e^(G_r - G_i) = e^(G_r - m) * e^(m - G_i) around a per-channel
// reference m.  The fast path takes m = 0 (the chunk start): e^G <= 1 and
// e^-G <= e^80 when every channel's chunk decay gamma >= -80, so nothing
// overflows fp32/bf16 (both have an 8-bit exponent) and each product keeps
// the operands' relative precision.  [XT §4] names the precision loss of this
// division as a design concern.  A chunk beyond that bound takes m = G at row
// 31 (the mid reference, in the same code): every factor that matters then
// stays within [e^-80, e^80] as long as each half of the chunk decays by at
// most 80 (gamma down to about -160), and A and P are the same MFMA products
// of other operand values.  Beyond even that, each 16-row block pair of A
// and P takes its own reference (k1_blocked_ap, still on MFMA: the last row
// of the column block when the blocks differ, so both factors are <= 1 for
// any gate; row 7 of a diagonal block, while each 8-row half of it decays by
// at most 80), and past that an exact path forms each e^(G_r - G_i) <= 1
// from its own difference (k1_exact_ap; slow, but never overflows).
//
// Precision.  MFMA operands are the input dtype (bf16 or fp32); MFMA
// accumulation, the state, T, G and gamma are fp32.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>

#include "kda_internal.h"
#include "kda_chunk_common.h"

namespace kda {
namespace {

// One segment's records (all heads) are kept within kSegRecordBudget bytes,
// so that they are still in the last-level cache (256 MB on MI355X) when the
// state pass reads them right after the intra-chunk kernel wrote them.
constexpr int64_t kSegRecordBudget = 160ll << 20;
constexpr int64_t kSegSlotsMax = 1024;  // chunk slots per K1/K2 launch pair, at most

// The state pass addresses one head's records of a segment through a buffer
// resource with 32-bit offsets and relies on reads at kPastBound returning
// zeros: a segment's records per head must stay below that offset.
static_assert(kSegSlotsMax * Rec<float, 128>::BYTES < (int64_t)kPastBound,
              "one head's segment records must stay below the past-the-bound offset");

// ---------------------------------------------------------------------------
// K1: intra-chunk transform.  LDS holds three equal regions, reused by phase:
//   region 0: K o e^G (row-major) [exact path: raw k]  -> V^T          (U phase)
//   region 1: Q o e^G (row-major) [exact path: raw q]  -> A (fp32)    -> (K o e^G)^T
//   region 2: scan partials -> K o e^-G (row-major) / exact-path staging
//             -> T (fp32) -> T Diag(beta)
// (K o e^G)^T is computed with the other operands but held in registers
// until A is dead.  Three regions (~52 KiB at d = 128) let three workgroups
// share a CU, where four allowed two.
// Thread layout "channel pair" (tid = cp + (D/2) part): two adjacent channels
// of RPP consecutive rows.  The D/2 threads of a part hold whole rows (one
// wave at d = 128, half a wave at d = 64), so the q/k row norms are reduced
// across lanes without a second read of q and k.  A channel-pair thread holds
// its rows contiguously, so the transposed LDS tiles ((K o e^G)^T, V^T) are
// written 8 rows at a time.  The operand-order record blocks of Q o e^G and
// K~ are gathered from LDS on the bf16 fast path (whole 1 KiB blocks per
// wave) and stored per thread otherwise.
// K1 workgroup size: 512 threads for bf16 at d = 128 (more waves in flight to
// hide the input loads, and half the rows and registers per thread); fp32
// operands keep 256 threads (their registers are full).
template <typename T, int D>
constexpr int k1_threads() { return (sizeof(T) == 2 && D == 128) ? 512 : 256; }

template <typename T, int D>
struct K1Lds {
  static constexpr int LDR = D + 16 / (int)sizeof(T);  // row-major leading dim (16-byte pad)
  // Transposed tiles (rows = channel or chunk row, 64 wide): 68 elements,
  // so bf16 rows are only 8-byte aligned and are accessed 8 bytes at a time.
  static constexpr int LDT = kC + 4;
  static constexpr int LDA = kC + 4;       // fp32 64x64 leading dim (16-byte rows)
  static constexpr int RM = kC * LDR * (int)sizeof(T);
  static constexpr int TR = D * LDT * (int)sizeof(T);
  static constexpr int MX = RM > TR ? RM : TR;
  static constexpr int FP = kC * LDA * 4;                     // fp32 A / T tile
  static constexpr int REG = ((MX > FP ? MX : FP) + 255) / 256 * 256;
  static constexpr int NCP = D / 2;                        // channel pairs
  static constexpr int NPART = k1_threads<T, D>() / NCP;   // row parts
  static constexpr int RPP = kC / NPART;                   // rows per part (8 or 16)
  static_assert(RPP % 8 == 0, "transposed stores take 8 rows at a time");
  static_assert(3 * 16 * (kC + 4) * 4 <= REG, "exact-path staging must fit a region");
  static_assert(NPART * D * 4 <= REG, "the scan partials must fit a region");
  // + per row: 1/|k|, 1/|q|, beta; per channel: e^(gamma-m).  (Not one
  // float more: at 512 more bytes three workgroups no longer share a CU --
  // measured, the intra-chunk kernel then takes ~17 us more per call.)
  static constexpr int BYTES = 3 * REG + (3 * kC + D) * 4;
  // Under the mid reference e^m per channel is parked in the 16-byte row pads
  // of region 2 (row-major there until T is written), rows kC/2 .. kC/2 +
  // D/4 - 1, four channels a row; the Wk phase takes it from the row-norm
  // arrays (1/|k|, 1/|q|: 2 kC floats, dead after the operands).
  static_assert((LDR - D) * (int)sizeof(T) == 16 && kC / 2 + D / 4 <= kC,
                "four floats of pad per row, D/4 rows");
  static_assert(D <= 2 * kC, "e^m fits the row-norm arrays");
  static __device__ __forceinline__ float* em_pad(T* r2, int c) {
    return reinterpret_cast<float*>(r2 + (kC / 2 + c / 4) * LDR + D) + (c & 3);
  }
};

constexpr float kLog2eF = 1.44269504088896341f;  // log2(e), rounded to fp32

// Pack 8 values to the MFMA type and store 16 bytes (bf16) / 32 bytes (fp32).
__device__ __forceinline__ void st8(bf16* p, const float* x) {
  u32x4_t u;
#pragma unroll
  for (int t = 0; t < 4; ++t) u[t] = pack_bf16x2(x[2 * t], x[2 * t + 1]);
  *reinterpret_cast<u32x4_t*>(p) = u;
}
__device__ __forceinline__ void st8(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
// Eight values of one transposed-tile row segment, packed to the MFMA type
// when computed and stored later (8-byte aligned for bf16).
template <typename T> struct Tr8;
template <> struct Tr8<bf16> {
  uint32_t u[4];
  __device__ __forceinline__ void set2(int t, float a, float b) { u[t] = pack_bf16x2(a, b); }
  __device__ __forceinline__ void set(const float* x) {
#pragma unroll
    for (int t = 0; t < 4; ++t) set2(t, x[2 * t], x[2 * t + 1]);
  }
  __device__ __forceinline__ void store(bf16* p) const {
    reinterpret_cast<uint2*>(p)[0] = make_uint2(u[0], u[1]);
    reinterpret_cast<uint2*>(p)[1] = make_uint2(u[2], u[3]);
  }
};
template <> struct Tr8<float> {
  float x[8];
  __device__ __forceinline__ void set2(int t, float a, float b) { x[2 * t] = a; x[2 * t + 1] = b; }
  __device__ __forceinline__ void set(const float* v) {
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = v[t];
  }
  __device__ __forceinline__ void store(float* p) const { st8(p, x); }
};
template <typename T>
__device__ __forceinline__ void st8t(T* p, const float* x) {
  Tr8<T> h;
  h.set(x);
  h.store(p);
}
// MFMA fragment of a transposed tile (rows 8-byte aligned for bf16).
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag frag_t(const T* base, int ld, int row0, int ks,
                                                        int lane) {
  const T* p = base + (row0 + (lane & 15)) * ld + ks * Mma<T>::KSTEP + Mma<T>::KPL * (lane >> 4);
  if constexpr (sizeof(T) == 2) {
    const uint2 a = reinterpret_cast<const uint2*>(p)[0], b = reinterpret_cast<const uint2*>(p)[1];
    return __builtin_bit_cast(typename Mma<T>::frag, u32x4_t{a.x, a.y, b.x, b.y});
  } else {
    return Mma<T>::load(p);
  }
}
// Two adjacent elements: load as floats / store from floats.
__device__ __forceinline__ float2 ld2(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ float2 ld2(const bf16* p) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(bf_val(u & 0xffffu), bf_val(u >> 16));
}
__device__ __forceinline__ void st2(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void st2(bf16* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}

// Waves per SIMD the kernel is built for: three workgroups per CU (LDS
// allows it) except fp32 at d = 128, whose registers fill a CU alone.
template <typename T, int D, bool CONV = false>
constexpr int k1_waves_per_simd() {
  return (sizeof(T) == 4 && D == 128) ? 1 : (CONV ? 2 : 3) * k1_threads<T, D>() / 256;
}

// One operand fragment from KPL floats (bf16: rounded to nearest even).
template <typename T> __device__ __forceinline__ typename Mma<T>::frag frag_of(const float* x);
template <> __device__ __forceinline__ bf16x8_t frag_of<bf16>(const float* x) {
  return __builtin_bit_cast(bf16x8_t, (u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                               pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])}));
}
template <> __device__ __forceinline__ float frag_of<float>(const float* x) { return x[0]; }

// A and P of a chunk beyond the mid reference's range on MFMA, block pair by
// block pair with a reference per pair (see k1_exact_ap, which checks that
// the reference rows keep every kept factor in range).  G is staged 32
// channels at a time; each wave forms its pairs' operand fragments from k^,
// q^ (LDS) and the staged G in registers, the same 10 pairs per wave as the
// common path, and writes A and P as the common path does.
template <typename T, int D, int RPP>
__device__ __forceinline__ void k1_blocked_ap(const T* khat, const T* qhat, float* stage,
                                              float* sA, const float* s_beta, T* wP,
                                              const float2 (&G)[RPP], float offx, float offy) {
  using L = K1Lds<T, D>;
  using M = Mma<T>;
  constexpr int NCP = L::NCP, NT = k1_threads<T, D>(), NW = NT / 64;
  constexpr int NPAIR = 10, PMAX = (NPAIR + NW - 1) / NW, SG = 32 + 4, KPL = M::KPL;
  static_assert(kC * SG * 4 <= L::REG, "the G stage must fit a region");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cp = tid % NCP, part = tid / NCP, c0 = 2 * cp, r0p = part * RPP;
  auto pair_I = [](int p) { return p < 4 ? 0 : p < 7 ? 1 : p < 9 ? 2 : 3; };
  auto pair_R = [](int p) { return p < 4 ? p : p < 7 ? p - 3 : p < 9 ? p - 5 : 3; };
  f32x4_t accA[PMAX], accP[PMAX];
#pragma unroll
  for (int t = 0; t < PMAX; ++t) {
    accA[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accP[t] = accA[t];
  }
  for (int cb = 0; cb < D / 32; ++cb) {
    if (c0 / 32 == cb) {
#pragma unroll
      for (int j = 0; j < RPP; ++j) {
        stage[(r0p + j) * SG + c0 % 32] = G[j].x + offx;
        stage[(r0p + j) * SG + c0 % 32 + 1] = G[j].y + offy;
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < PMAX; ++t) {
      const int p = wave + t * NW;
      if (p >= NPAIR) continue;
      const int I = pair_I(p), R = pair_R(p);
      const int ri = 16 * I + (lane & 15), rr = 16 * R + (lane & 15);
      const int mrow = I == R ? 16 * I + 7 : 16 * I + 15;
#pragma unroll 1
      for (int ks = 0; ks < 32 / M::KSTEP; ++ks) {
        const int cl = ks * M::KSTEP + KPL * (lane >> 4);  // channel within the block
        const int cg = 32 * cb + cl;
        float m[KPL], x[KPL], y[KPL];
#pragma unroll
        for (int e = 0; e < KPL; ++e) m[e] = stage[mrow * SG + cl + e];
#pragma unroll
        for (int e = 0; e < KPL; ++e)
          x[e] = ld_f(khat + ri * L::LDR + cg + e) * __expf(m[e] - stage[ri * SG + cl + e]);
        const auto fa = frag_of<T>(x);
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const float f = __expf(stage[rr * SG + cl + e] - m[e]);
          x[e] = ld_f(khat + rr * L::LDR + cg + e) * f;
          y[e] = ld_f(qhat + rr * L::LDR + cg + e) * f;
        }
        accA[t] = M::mma(fa, frag_of<T>(x), accA[t]);
        accP[t] = M::mma(fa, frag_of<T>(y), accP[t]);
      }
    }
    __syncthreads();
  }
  // sA aliases qhat: every read of it ended at the barrier above
#pragma unroll
  for (int t = 0; t < PMAX; ++t) {
    const int p = wave + t * NW;
    if (p >= NPAIR) continue;
    const int I = pair_I(p), R = pair_R(p);
    const int r = R * 16 + (lane & 15);
    const int i0 = I * 16 + 4 * (lane >> 4);
    const float br = s_beta[r];
    float a4[4], p4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // above the diagonal the products may overflow: not kept
      a4[j] = (i0 + j < r) ? br * accA[t][j] : 0.f;
      p4[j] = (i0 + j <= r) ? accP[t][j] : 0.f;
    }
    *reinterpret_cast<float4*>(sA + r * L::LDA + i0) = make_float4(a4[0], a4[1], a4[2], a4[3]);
    st_fnat4(wP, kC / M::KSTEP, r, i0, p4[0], p4[1], p4[2], p4[3]);
  }
}

// Exact-decay path of A and P: each entry from its own exponent difference
// (<= 0), with G, k^ and q^ staged in blocks of 16 channels, channel-major
// (a row of 64 chunk rows per channel).  k^ and q^ are the row-major LDS
// tiles khat and qhat; G is formed again from g (as the kernel forms it: the
// prefix sum over the thread's rows, plus the part offset), once, before the
// blocks.  Thread t < 136 owns the 4 x 4 tile t of the lower triangle
// (row block rb, column block ib <= rb, t = rb (rb + 1) / 2 + ib) and reads
// its four rows and four columns of a channel as 16-byte pieces.  Out of
// line: few chunks take it, and inlined it would set the register budget of
// the common path.  Every thread of the workgroup calls it.
template <typename T, int D, bool GS>
__device__ __forceinline__ void k1_exact_ap(
    const T* khat, const T* qhat, float* stage, float* sA, const float* s_beta, T* wP,
    const float* gb, int64_t rowstride, int H, int len, float offx, float offy) {
  using L = K1Lds<T, D>;
  using M = Mma<T>;
  constexpr int NCP = L::NCP, RPP = L::RPP, NT = k1_threads<T, D>();
  constexpr int NTILE = (kC / 4) * (kC / 4 + 1) / 2;  // 4 x 4 tiles of the lower triangle
  static_assert(NTILE <= NT, "one lower-triangle tile per thread");
  const int tid = threadIdx.x, cp = tid % NCP, part = tid / NCP;
  const int c0 = 2 * cp, r0p = part * RPP;
  // channel-major rows of 64 chunk rows, 16-byte aligned
  constexpr int SR = kC + 4;
  float* stG = stage;
  float* stK = stG + 16 * SR;
  float* stQ = stK + 16 * SR;
  // this thread's G (channels c0, c0 + 1, rows r0p ..), all loads issued at once
  float2 G[RPP];
#pragma unroll
  for (int j = 0; j < RPP; ++j) {
    const int rr = min(r0p + j, len - 1);
    const float2 gj = GS ? make_float2(gb[rr * H], gb[rr * H]) : ld2(gb + rr * rowstride + c0);
    G[j] = r0p + j < len ? gj : make_float2(0.f, 0.f);
  }
#pragma unroll
  for (int j = 1; j < RPP; ++j) { G[j].x += G[j - 1].x; G[j].y += G[j - 1].y; }
  // Blocked form, on MFMA, when each 8-row half of every 16-row block decays
  // by at most 80 per channel: block pair (R, I) of A and P is
  // (K_I o e^(m - G_I)) (K_R o e^(G_R - m))^T (and Q_R for P) with m = G of
  // row 16 I + 15 when R > I (both factors <= 1 for any gate) and of row
  // 16 I + 7 when R = I (factors within [e^-80, e^80] wherever the result is
  // kept).  The halves' decays are sums of this thread's own g: rows 16 I ..
  // 16 I + 7 and 16 I + 8 .. 16 I + 15 each lie inside one thread's rows.
  bool wide = false;
#pragma unroll
  for (int j = 0; j < RPP; ++j) {
    const int b = r0p + j;
    if ((b & 7) == 7) {
      const int a = (b & 15) == 7 ? b - 7 : b - 8;  // the span's first row, or the row before it
      const float2 ga = a - r0p >= 0 ? G[a - r0p] : make_float2(0.f, 0.f);
      wide |= G[j].x - ga.x < kFastDecayBound || G[j].y - ga.y < kFastDecayBound;
    }
  }
  if (__syncthreads_or(wide) == 0) {
    k1_blocked_ap<T, D>(khat, qhat, stage, sA, s_beta, wP, G, offx, offy);
    return;
  }
  // this thread's tile
  int rb = 0;
  while ((rb + 1) * (rb + 2) / 2 <= tid) ++rb;
  const int ib = tid - rb * (rb + 1) / 2;
  const bool owner = tid < NTILE, diag = rb == ib;
  float ea[4][4], ep[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) { ea[u][j] = 0.f; ep[u][j] = 0.f; }
  for (int cb = 0; cb < D / 16; ++cb) {
    if (c0 / 16 == cb) {
      const int cc = c0 % 16;
#pragma unroll
      for (int j = 0; j < RPP; ++j) {
        const int r = r0p + j;
        stG[cc * SR + r] = G[j].x + offx;
        stG[(cc + 1) * SR + r] = G[j].y + offy;
        const float2 kh = ld2(khat + r * L::LDR + c0), qh = ld2(qhat + r * L::LDR + c0);
        stK[cc * SR + r] = kh.x; stK[(cc + 1) * SR + r] = kh.y;
        stQ[cc * SR + r] = qh.x; stQ[(cc + 1) * SR + r] = qh.y;
      }
    }
    __syncthreads();
    if (owner) {
#pragma unroll 2
      for (int c = 0; c < 16; ++c) {
        const float4 gr = *reinterpret_cast<const float4*>(stG + c * SR + 4 * rb);
        const float4 gi = *reinterpret_cast<const float4*>(stG + c * SR + 4 * ib);
        const float4 kr = *reinterpret_cast<const float4*>(stK + c * SR + 4 * rb);
        const float4 ki = *reinterpret_cast<const float4*>(stK + c * SR + 4 * ib);
        const float4 qr = *reinterpret_cast<const float4*>(stQ + c * SR + 4 * rb);
        const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, giv[4] = {gi.x, gi.y, gi.z, gi.w};
        const float krv[4] = {kr.x, kr.y, kr.z, kr.w}, kiv[4] = {ki.x, ki.y, ki.z, ki.w};
        const float qrv[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // above the diagonal G_r - G_i >= 0 may overflow: not formed
            const float x = (!diag || j <= u) ? kiv[j] * __expf(grv[u] - giv[j]) : 0.f;
            ea[u][j] += krv[u] * x;
            ep[u][j] += qrv[u] * x;
          }
      }
    }
    __syncthreads();
  }
  // sA aliases qhat: every read of it ended at the barrier above
  if (owner) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * rb + u, i = 4 * ib + j;
        if (i <= r) {
          sA[r * L::LDA + i] = i < r ? s_beta[r] * ea[u][j] : 0.f;
          st_f(wP + fnat<T>(r, i, kC / M::KSTEP), ep[u][j]);
        }
      }
  }
  // the exact path writes no upper-triangle entries of the diagonal blocks
  for (int e = tid; e < kC * kC; e += NT) {
    const int r = e >> 6, i = e & 63;
    if (i > r && (i >> 4) == (r >> 4)) st_f(wP + fnat<T>(r, i, kC / M::KSTEP), 0.f);
  }
}

// A and P of a chunk beyond the mid reference's range (some half of the chunk
// decays by more than 80 in some channel), from raw k^ (region 0) and q^
// (region 1): k1_exact_ap, with region 2 free for its staging.  One call site
// out of line, so that its registers do not weigh on the common path.  Every
// thread of the workgroup calls it.
template <typename T, int D, bool GS>
__device__ __attribute__((noinline)) void k1_slow_ap(T* r0, T* r1, T* r2, const float* s_beta,
                                                     T* wP, const float* gb, int64_t rowstride,
                                                     int H, int len, float offx, float offy) {
  k1_exact_ap<T, D, GS>(r0, r1, reinterpret_cast<float*>(r2), reinterpret_cast<float*>(r1),
                        s_beta, wP, gb, rowstride, H, len, offx, offy);
}

// The ShortConv + Swish prologue (width 4) fused into K1's loads: per tensor
// (q, k, v) its [C, 4] fp32 weights (C = H D), its [C] fp32 bias or null, and
// the [N, C, 3] fp32 inputs carried in before each sequence (oldest first),
// or null for zeros.
struct ConvIn {
  const float* w[3];
  const float* bias[3];
  const float* state[3];
};

// ShortConv + Swish of the thread's RPP rows of channels c0, c0+1, in the
// separate prologue kernel's order and arithmetic (so the results are the
// same bits): a = bias + w3 x_t + w0 x_(t-3) + w1 x_(t-2) + w2 x_(t-1),
// y = a rcp(1 + e^-a); each loaded pair is replaced by its y in the element
// type (as that kernel stores y).  win holds the three inputs before the
// thread's first row; rows from nvalid on (past the chunk's end) give 0.
template <int RPP, typename Raw>
__device__ __forceinline__ void conv_swish(Raw (&x)[RPP], float2 (&win)[3], const float4 (&w)[2],
                                           const float (&b)[2], int nvalid) {
#pragma unroll
  for (int j = 0; j < RPP; ++j) {
    const float2 xt = x[j].get();
    float a0 = b[0] + w[0].w * xt.x;
    a0 += w[0].x * win[0].x;
    a0 += w[0].y * win[1].x;
    a0 += w[0].z * win[2].x;
    float a1 = b[1] + w[1].w * xt.y;
    a1 += w[1].x * win[0].y;
    a1 += w[1].y * win[1].y;
    a1 += w[1].z * win[2].y;
    float y0 = a0 * __builtin_amdgcn_rcpf(1.f + __expf(-a0));
    float y1 = a1 * __builtin_amdgcn_rcpf(1.f + __expf(-a1));
    if (j >= nvalid) {
      y0 = 0.f;
      y1 = 0.f;
    }
    win[0] = win[1];
    win[1] = win[2];
    win[2] = xt;
    x[j].set(y0, y1);
  }
}

// The three input rows before the thread's first (row r0p), channels c0,
// c0+1, of one fused-prologue tensor: from the rows before the chunk (same
// sequence) when the chunk is not its sequence's first, else, for the rows
// before the chunk, from the carried state or zero.  `base` is the chunk's
// first row of this head; the halo loads go through a resource over the
// chunk's rows plus the three before it (three rows of a sequence's first
// chunk lie before the sequence: there the resource starts at the chunk and
// the rows before it, past its bound, read as zero).
template <typename T, typename Raw>
__device__ __forceinline__ void conv_halo_load(Raw (&hal)[3], const T* base, bool first, int span,
                                               int rs, int r0p, int c0) {
  const int back = first ? 0 : 3;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(base - back * rs), (short)0, (span + back * rs) * (int)sizeof(T), kRsrcWord3);
#pragma unroll
  for (int p = 0; p < 3; ++p)
    hal[p].load(r, (uint32_t)(((r0p - 3 + p + back) * rs + c0) * (int)sizeof(T)));
}
template <typename Raw>
__device__ __forceinline__ void conv_window(float2 (&win)[3], const Raw (&hal)[3], bool from_state,
                                            const float* state, int64_t sidx) {
#pragma unroll
  for (int p = 0; p < 3; ++p) win[p] = hal[p].get();
  if (from_state && state != nullptr) {
#pragma unroll
    for (int p = 0; p < 3; ++p) win[p] = make_float2(state[sidx + p], state[sidx + 3 + p]);
  }
}
__device__ __forceinline__ void conv_weights(float4 (&w)[2], float (&b)[2], const float* wt,
                                             const float* bias, int64_t ch) {
  w[0] = *reinterpret_cast<const float4*>(wt + ch * 4);
  w[1] = *reinterpret_cast<const float4*>(wt + (ch + 1) * 4);
  b[0] = bias ? bias[ch] : 0.f;
  b[1] = bias ? bias[ch + 1] : 0.f;
}

// GS: one gate per (token, head), broadcast over the key channels (Gated
// DeltaNet) instead of one per channel.  CONV: q, k, v are the prologue's
// inputs, convolved on load (ConvIn).
template <typename T, int D, bool GS, bool CONV = false>
__global__ __launch_bounds__((k1_threads<T, D>()), (k1_waves_per_simd<T, D, CONV>())) void kda_intra_chunk(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, ChunkGeom gm, int H,
    int64_t slot_base, int64_t nrec, int qk_l2norm, char* __restrict__ ws, ConvIn cv) {
  using L = K1Lds<T, D>;
  using M = Mma<T>;
  using R = Rec<T, D>;
  constexpr int NCP = L::NCP, NPART = L::NPART, RPP = L::RPP;
  constexpr int NT = k1_threads<T, D>(), NW = NT / 64;  // threads, waves
  extern __shared__ __align__(16) char smem[];
  T* r0 = reinterpret_cast<T*>(smem);
  T* r1 = reinterpret_cast<T*>(smem + L::REG);
  T* r2 = reinterpret_cast<T*>(smem + 2 * L::REG);
  float* s_rk = reinterpret_cast<float*>(smem + 3 * L::REG);
  float* s_rq = s_rk + kC;
  float* s_beta = s_rq + kC;
  float* s_eg = s_beta + kC;  // e^(gamma-m) per channel (K~'s factor)
  float* s_em = s_rk;         // e^m per channel for the Wk phase (mid reference)

  // heads vary fastest across workgroups: concurrently resident workgroups
  // then read whole token rows (all heads) of neighbouring tokens
  const int h = blockIdx.x;
  const int64_t slot = slot_base + blockIdx.y;
  ChunkLoc loc;
  if (!locate(gm, slot, loc)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t rowstride = (int64_t)H * D;  // elements between consecutive tokens
  const T* qb = q + (loc.tok0 * H + h) * D;
  const T* kb = k + (loc.tok0 * H + h) * D;
  const T* vb = v + (loc.tok0 * H + h) * D;
  const float* gb = GS ? g + loc.tok0 * H + h : g + (loc.tok0 * H + h) * D;
  char* rec = ws + ((int64_t)h * nrec + (slot - slot_base)) * R::BYTES;
  T* wQG = reinterpret_cast<T*>(rec) + R::QG;
  T* wKT = reinterpret_cast<T*>(rec) + R::KT;
  T* wWN = reinterpret_cast<T*>(rec) + R::WN;
  T* wUT = reinterpret_cast<T*>(rec) + R::UT;
  T* wP = reinterpret_cast<T*>(rec) + R::P;
  float* wEG = reinterpret_cast<float*>(rec + R::BYTES_T);

  // ---- global loads --------------------------------------------------------
  // Every load is unconditional and keeps its raw bits until all loads are in
  // flight: a load under a branch, or converted on arrival, makes the wave
  // wait for it before issuing the next one.  Each input is read through a
  // buffer resource over this chunk's rows, bounded at the end of its last
  // valid row: rows past the chunk's end read as zero (as the method wants
  // them), and a load's address is one 32-bit offset.
  // channel-pair layout: channels c0, c0+1 of rows r0p .. r0p+RPP-1
  const int cp = tid % NCP, part = tid / NCP;
  const int c0 = 2 * cp, r0p = part * RPP;
  // Loads are issued tensor by tensor in the order they are consumed (g for
  // the scan, then k and q for the norms; v, needed only after A and P, is
  // loaded after the operands): the wait counter is in-order, so each use
  // then waits only for the loads it needs.  g and v are loaded
  // non-temporally: the chunk records this kernel writes are what the state
  // pass reads next, and these inputs streaming past would otherwise push
  // them out of the last-level cache (measured: the state pass 67 -> 60 us
  // per segment).
  const int rs = H * D;  // elements between consecutive tokens
  const int span = (loc.len - 1) * rs + D;  // elements from the first to the last valid
  auto rsrc = [](const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
  };
  const __amdgpu_buffer_rsrc_t rq = rsrc(qb, span * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t rk = rsrc(kb, span * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t rv = rsrc(vb, span * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t rg = rsrc(gb, GS ? ((loc.len - 1) * H + 1) * 4 : span * 4);
  const uint32_t offT = (uint32_t)((r0p * rs + c0) * (int)sizeof(T));   // row r0p, channel c0
  const uint32_t rowT = (uint32_t)(rs * (int)sizeof(T));                // bytes per token
  RawNt2<float> graw[RPP];
  float gsc[RPP];  // GS: the row's one gate
  Raw2<T> kraw[RPP], qraw[RPP];
  RawNt2<T> vraw[RPP];
#pragma unroll
  for (int j = 0; j < RPP; ++j) {
    if constexpr (GS)
      gsc[j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)((r0p + j) * H * 4), 0, 2));
    else
      graw[j].load(rg, (uint32_t)((r0p * rs + c0) * 4) + (uint32_t)j * (uint32_t)(rs * 4));
  }
#pragma unroll
  for (int j = 0; j < RPP; ++j) kraw[j].load(rk, offT + (uint32_t)j * rowT);
#pragma unroll
  for (int j = 0; j < RPP; ++j) qraw[j].load(rq, offT + (uint32_t)j * rowT);
  // CONV: the chunk is its sequence's first when it starts the sequence
  const bool first = CONV && seq_span(gm, loc.seq).tok0 == loc.tok0;
  const int64_t sidx = ((int64_t)loc.seq * rs + h * D + c0) * 3;  // carried state, channel c0
  Raw2<T> khal[3], qhal[3];
  if constexpr (CONV) {
    conv_halo_load(khal, kb, first, span, rs, r0p, c0);
    conv_halo_load(qhal, qb, first, span, rs, r0p, c0);
  }
  if (tid < kC) s_beta[tid] = tid < loc.len ? beta[(loc.tok0 + tid) * H + h] : 0.f;
  if constexpr (CONV) {
    float4 w[2];
    float b[2];
    float2 win[3];
    conv_weights(w, b, cv.w[1], cv.bias[1], (int64_t)h * D + c0);
    conv_window(win, khal, first && r0p == 0, cv.state[1], sidx);
    conv_swish<RPP>(kraw, win, w, b, loc.len - r0p);
    conv_weights(w, b, cv.w[0], cv.bias[0], (int64_t)h * D + c0);
    conv_window(win, qhal, first && r0p == 0, cv.state[0], sidx);
    conv_swish<RPP>(qraw, win, w, b, loc.len - r0p);
  }
  float2 G[RPP];
#pragma unroll
  for (int j = 0; j < RPP; ++j) G[j] = GS ? make_float2(gsc[j], gsc[j]) : graw[j].get();
  // Row norms: the 2 RPP squared partial sums (q rows, then k rows) of the
  // D/2 lanes of a part, reduced by a butterfly that halves the values each
  // lane keeps at every step (reduce-scatter) and then sums the last one
  // over the remaining lanes; lane bits name the value a lane ends with.
  {
    constexpr int V = 2 * RPP;
    static_assert(V <= NCP, "one value per lane after the reduce-scatter");
    float x[V];
#pragma unroll
    for (int j = 0; j < RPP; ++j) {
      // rows past the chunk's end read as zero (their norms are never used)
      const float2 qj = qraw[j].get(), kj = kraw[j].get();
      x[j] = qj.x * qj.x + qj.y * qj.y;
      x[RPP + j] = kj.x * kj.x + kj.y * kj.y;
    }
    int idx = 0;
#pragma unroll
    for (int s = 0; (NCP >> (s + 1)) >= 1; ++s) {
      const int o = NCP >> (s + 1);
      const int cnt = (V >> s) >= 2 ? (V >> s) : 1;
      if (cnt > 1) {
        const int half = cnt / 2;
        const bool up = (lane & o) != 0;
#pragma unroll
        for (int t = 0; t < half; ++t) {
          const float send = up ? x[t] : x[half + t];
          const float keep = up ? x[half + t] : x[t];
          x[t] = keep + __shfl_xor(send, o);
        }
        if (up) idx += half;
      } else {
        x[0] += __shfl_xor(x[0], o);
      }
    }
    constexpr int LOWMASK = NCP / V - 1;
    if ((lane & LOWMASK) == 0) {
      const float rn = qk_l2norm ? rsqrtf(x[0] + kNormEps) : 1.f;
      if (idx < RPP) s_rq[r0p + idx] = rn; else s_rk[r0p + idx - RPP] = rn;
    }
  }
  // ---- in-chunk prefix sum of g ---------------------------------------------
  float* scan = reinterpret_cast<float*>(r2);  // part totals; region 2 is free until the operands
#pragma unroll
  for (int j = 1; j < RPP; ++j) { G[j].x += G[j - 1].x; G[j].y += G[j - 1].y; }
  scan[part * D + c0] = G[RPP - 1].x;
  scan[part * D + c0 + 1] = G[RPP - 1].y;
  __syncthreads();
  float2 off = make_float2(0.f, 0.f), gamma = make_float2(0.f, 0.f);
#pragma unroll
  for (int p = 0; p < NPART; ++p) {
    const float2 t = make_float2(scan[p * D + c0], scan[p * D + c0 + 1]);
    if (p < part) { off.x += t.x; off.y += t.y; }
    gamma.x += t.x; gamma.y += t.y;
  }
#pragma unroll
  for (int j = 0; j < RPP; ++j) { G[j].x += off.x; G[j].y += off.y; }
  // Exponent modes (a workgroup vote): the fast path's reference m = 0
  // while every channel's gamma >= -80; else the mid reference m = G of row
  // 31 while each half of the chunk decays by at most 80 in every channel --
  // the same products on MFMA, from K o e^(G-m), Q o e^(G-m), K o e^(m-G),
  // whose factors stay within [e^-80, e^80] wherever a product's result is
  // kept; beyond that, k1_slow_ap's exact path (raw k^, q^ staged, records
  // written per thread).
  const bool beyond =
      __syncthreads_or(gamma.x < kFastDecayBound || gamma.y < kFastDecayBound) != 0;
  float2 mref = make_float2(0.f, 0.f);  // G of row 31, from the part totals
  bool mid = false;
  if (beyond) {
#pragma unroll
    for (int p = 0; p < (kC / 2) / RPP; ++p) {
      mref.x += scan[p * D + c0];
      mref.y += scan[p * D + c0 + 1];
    }
    mid = __syncthreads_or(mref.x < kFastDecayBound || mref.y < kFastDecayBound ||
                           gamma.x - mref.x < kFastDecayBound ||
                           gamma.y - mref.y < kFastDecayBound) == 0;
    if (mid) {  // G relative to the reference: G - m
#pragma unroll
      for (int j = 0; j < RPP; ++j) { G[j].x -= mref.x; G[j].y -= mref.y; }
    } else {
      mref = make_float2(0.f, 0.f);
    }
  }
  const bool exact = beyond && !mid;

  // ---- operands ---------------------------------------------------------------
  // e^gamma for the record; K~'s factor e^(gamma-m); e^m rescales the mid
  // reference's relative Q o e^(G-m) and Wk to their true values (1 off it)
  const float2 eg_gamma = make_float2(__expf(gamma.x), __expf(gamma.y));
  const float2 eg_kt =
      mid ? make_float2(__expf(gamma.x - mref.x), __expf(gamma.y - mref.y)) : eg_gamma;
  // bf16 records off the exact path take Q o e^G and K~ from LDS below, in
  // whole operand fragments; otherwise every thread stores its own values
  constexpr bool kStaged = sizeof(T) == 2;
  const bool direct = !kStaged || exact;
  float2 em = make_float2(1.f, 1.f);
  if (mid) em = make_float2(__expf(mref.x), __expf(mref.y));
  if (part == 0) {
    wEG[c0] = eg_gamma.x; wEG[c0 + 1] = eg_gamma.y;
    s_eg[c0] = eg_kt.x; s_eg[c0 + 1] = eg_kt.y;
    if (mid) { *L::em_pad(r2, c0) = em.x; *L::em_pad(r2, c0 + 1) = em.y; }
  }
  // (K o e^(G-m))^T, 8 rows of channels c0 and c0+1 per entry, stored after
  // the inverse.  Rows are taken in pairs, so that each pair goes straight
  // into the held tile and K~ leaves as pairs (few values live at a time).
  Tr8<T> kgh[RPP / 8][2];
#pragma unroll
  for (int j = 0; j < RPP; j += 2) {
    float kgx[2], kgy[2], ktx[2] = {0.f, 0.f}, kty[2] = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = j + e, r = r0p + jj;
      const float rk = s_rk[r], rq = s_rq[r];
      const float2 kk = kraw[jj].get(), qq = qraw[jj].get();  // zero past the end
      const float khx = kk.x * rk, khy = kk.y * rk;
      const float qhx = qq.x * rq, qhy = qq.y * rq;
      // e^(+-(G-m)) as 2^(+-(G-m) log2 e): one scaling for both signs (the
      // same operations as __expf, so the same values)
      const float gsx = G[jj].x * kLog2eF, gsy = G[jj].y * kLog2eF;
      const float egx = __builtin_amdgcn_exp2f(gsx), egy = __builtin_amdgcn_exp2f(gsy);
      if (direct) {  // the true Q o e^G (bf16 only on the exact path, where m = 0)
        if constexpr (kStaged)
          st_fnat2(wQG, D / M::KSTEP, r, c0, qhx * egx, qhy * egy);
        else
          st_fnat2(wQG, D / M::KSTEP, r, c0, qhx * egx * em.x, qhy * egy * em.y);
      }
      kgx[e] = khx * egx;
      kgy[e] = khy * egy;
      if (!exact) {
        const float enx = __builtin_amdgcn_exp2f(-gsx), eny = __builtin_amdgcn_exp2f(-gsy);
        st2(r0 + r * L::LDR + c0, khx * egx, khy * egy);     // K o e^(G-m)
        st2(r1 + r * L::LDR + c0, qhx * egx, qhy * egy);     // Q o e^(G-m)
        st2(r2 + r * L::LDR + c0, khx * enx, khy * eny);     // K o e^(m-G)
        if constexpr (!kStaged) {
          ktx[e] = khx * (eg_kt.x * enx);
          kty[e] = khy * (eg_kt.y * eny);
        }
      } else {
        st2(r0 + r * L::LDR + c0, khx, khy);                 // k^ (staged later)
        st2(r1 + r * L::LDR + c0, qhx, qhy);                 // q^
        ktx[e] = khx * __expf(gamma.x - G[jj].x);
        kty[e] = khy * __expf(gamma.y - G[jj].y);
      }
    }
    kgh[j / 8][0].set2((j & 7) / 2, kgx[0], kgx[1]);
    kgh[j / 8][1].set2((j & 7) / 2, kgy[0], kgy[1]);
    if (direct) {  // K o e^(gamma-G), rows c, k = chunk rows r0p+j, r0p+j+1
      st_fnat2(wKT, kC / M::KSTEP, c0, r0p + j, ktx[0], ktx[1]);
      st_fnat2(wKT, kC / M::KSTEP, c0 + 1, r0p + j, kty[0], kty[1]);
    }
  }
  __syncthreads();
  if (mid && tid < D) s_em[tid] = *L::em_pad(r2, tid);  // the row norms are dead
  // v is needed only after A and P: loading it here keeps its registers free
  // through the operands, and the staged writes and A, P cover its latency
  // (the exact path loads it after its own A and P).  Its row offsets are
  // formed again: they equal the first loads' and would otherwise be held
  // in registers until now.
  RawNt2<T> vhal[3];
  auto load_v = [&]() {
    uint32_t ov = offT;
    __asm__ volatile("" : "+v"(ov));
#pragma unroll
    for (int j = 0; j < RPP; ++j) vraw[j].load(rv, ov + (uint32_t)j * rowT);
    if constexpr (CONV) conv_halo_load(vhal, vb, first, span, rs, r0p, c0);
  };
  if (!exact) load_v();

  // Staged record writes (bf16, off the exact path): Q o e^(G-m) is region 1
  // and K o e^(m-G) region 2, so every lane slot of the operand-order blocks
  // is gathered from LDS and each wave writes whole 1 KiB blocks.  K~ =
  // e^(gamma-m) (K o e^(m-G)) per channel, and under the mid reference
  // Q o e^G = e^m (Q o e^(G-m)): a second bf16 rounding of the LDS values.
  if constexpr (kStaged) {
    if (!exact) {
      constexpr int QB = (kC / 16) * (D / 32), KB = (D / 16) * (kC / 32);  // blocks
      for (int sidx = tid; sidx < (QB + KB) * 64; sidx += NT) {
        const int b = sidx >> 6, L = sidx & 63, g = L >> 4;
        float v[8];
        if (b < QB) {  // Q o e^G: rows r, k = channel
          const int r = (b / (D / 32)) * 16 + (L & 15), cb = (b % (D / 32)) * 32 + 4 * g;
          const T* row = r1 + r * L::LDR;
          if (!mid) {  // bf16 already: copied as raw bits
            const uint2 lo = *reinterpret_cast<const uint2*>(row + cb);
            const uint2 hi = *reinterpret_cast<const uint2*>(row + cb + 16);
            *reinterpret_cast<u32x4_t*>(wQG + (b * 64 + L) * 8) = u32x4_t{lo.x, lo.y, hi.x, hi.y};
          } else {
            const float4 e0 = *reinterpret_cast<const float4*>(L::em_pad(r2, cb));
            const float4 e1 = *reinterpret_cast<const float4*>(L::em_pad(r2, cb + 16));
            const float ea[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = ea[e] * ld_f(row + cb + e);
              v[4 + e] = ea[4 + e] * ld_f(row + cb + 16 + e);
            }
            st8(wQG + (b * 64 + L) * 8, v);
          }
        } else {       // K~: rows c, k = chunk row i
          const int bk = b - QB;
          const int c = (bk / (kC / 32)) * 16 + (L & 15), ib = (bk % (kC / 32)) * 32 + 4 * g;
          const float eg = s_eg[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = eg * ld_f(r2 + (ib + e) * L::LDR + c);
            v[4 + e] = eg * ld_f(r2 + (ib + 16 + e) * L::LDR + c);
          }
          st8(wKT + (bk * 64 + L) * 8, v);
        }
      }
    }
  }

  // ---- A (strict lower, x beta_r) and P (lower) ------------------------------
  // Tiles are computed transposed (A^T, P^T) so each lane's 4 accumulator
  // rows are 4 consecutive columns of A / P: one vector store each.  The 10
  // block pairs (I <= R) are dealt to the waves round-robin (pair w, w+NW,
  // ...), as are the 6 all-zero blocks of P above the diagonal.
  constexpr int NPAIR = 10, PMAX = (NPAIR + NW - 1) / NW;
  auto pair_I = [](int p) { return p < 4 ? 0 : p < 7 ? 1 : p < 9 ? 2 : 3; };
  auto pair_R = [](int p) { return p < 4 ? p : p < 7 ? p - 3 : p < 9 ? p - 5 : 3; };
  f32x4_t accA[PMAX], accP[PMAX];
  if (!exact) {
#pragma unroll
    for (int t = 0; t < PMAX; ++t) {
      accA[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accP[t] = accA[t];
      const int p = wave + t * NW;
      if (p >= NPAIR) continue;
      const int I = pair_I(p), Rb = pair_R(p);
#pragma unroll
      for (int ks = 0; ks < D / M::KSTEP; ++ks) {
        const auto a = frag_at<T>(r2, L::LDR, I * 16, ks, lane);    // K o e^-G, rows I
        const auto bk = frag_at<T>(r0, L::LDR, Rb * 16, ks, lane);  // K o e^G, rows R
        const auto bq = frag_at<T>(r1, L::LDR, Rb * 16, ks, lane);  // Q o e^G, rows R
        accA[t] = M::mma(a, bk, accA[t]);
        accP[t] = M::mma(a, bq, accP[t]);
      }
    }
  } else {
    k1_slow_ap<T, D, GS>(r0, r1, r2, s_beta, wP, gb, rowstride, H, loc.len, off.x, off.y);
    load_v();
  }
  if (!exact) {
    __syncthreads();  // all reads of regions 0..2 done; region 1 becomes A
    float* sA = reinterpret_cast<float*>(r1);
#pragma unroll
    for (int t = 0; t < PMAX; ++t) {
      const int p = wave + t * NW;
      if (p >= NPAIR) continue;
      const int I = pair_I(p), Rb = pair_R(p);
      const int r = Rb * 16 + (lane & 15);
      const int i0 = I * 16 + 4 * (lane >> 4);
      const float br = s_beta[r];
      float a4[4], p4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a4[j] = (i0 + j < r) ? br * accA[t][j] : 0.f;
        p4[j] = (i0 + j <= r) ? accP[t][j] : 0.f;
      }
      *reinterpret_cast<float4*>(sA + r * L::LDA + i0) = make_float4(a4[0], a4[1], a4[2], a4[3]);
      st_fnat4(wP, kC / M::KSTEP, r, i0, p4[0], p4[1], p4[2], p4[3]);
    }
  }
  {
    // zero blocks of P above the diagonal, (R, I) = (0,1) (0,2) (0,3) (1,2)
    // (1,3) (2,3): only those inside a k-step the state pass reads for rows
    // R (its lowest 16-row block <= R; the others it reads as zeros)
    const int zR[6] = {0, 0, 0, 1, 1, 2}, zI[6] = {1, 2, 3, 2, 3, 3};
    for (int z = wave; z < 6; z += NW) {
      if ((zI[z] * 16 / M::KSTEP) * M::KSTEP / 16 > zR[z]) continue;
      const int r = zR[z] * 16 + (lane & 15), i0 = zI[z] * 16 + 4 * (lane >> 4);
      st_fnat4(wP, kC / M::KSTEP, r, i0, 0.f, 0.f, 0.f, 0.f);
    }
  }

  if constexpr (CONV) {
    float4 w[2];
    float b[2];
    float2 win[3];
    conv_weights(w, b, cv.w[2], cv.bias[2], (int64_t)h * D + c0);
    conv_window(win, vhal, first && r0p == 0, cv.state[2], sidx);
    conv_swish<RPP>(vraw, win, w, b, loc.len - r0p);
  }
  // V^T into region 0 (its row-major content is dead now), 8 rows per store
#pragma unroll
  for (int j0 = 0; j0 < RPP; j0 += 8) {
    float vx[8], vy[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 vt = vraw[j0 + t].get();  // zero past the chunk's end
      vx[t] = vt.x;
      vy[t] = vt.y;
    }
    st8t(r0 + c0 * L::LDT + r0p + j0, vx);
    st8t(r0 + (c0 + 1) * L::LDT + r0p + j0, vy);
  }
  __syncthreads();

  // ---- T = (I + A)^-1 in fp32 --------------------------------------------------
  const float* sA = reinterpret_cast<const float*>(r1);
  float* sT = reinterpret_cast<float*>(r2);
  static_assert(L::LDA == kTriLd, "A and T use the inverse's leading dimension");
  tri_inv64(sA, sT, nullptr, wave, lane);  // its scratch: T's upper blocks
  // T Diag(beta) in the MFMA type, lower triangle only, over T in region 2:
  // thread = (row, group of TW columns).  A is dead: (K o e^G)^T goes to
  // region 1 meanwhile.
  T* sTb = r2;
  {
    constexpr int TG = NT / kC, TW = kC / TG;  // threads per row, columns each
    const int r = tid / TG, i0 = (tid % TG) * TW;
    float vals[TW];
#pragma unroll
    for (int t = 0; t < TW; t += 4) {
      const float4 tv = *reinterpret_cast<const float4*>(sT + r * L::LDA + i0 + t);
      const float4 bv = *reinterpret_cast<const float4*>(s_beta + i0 + t);
      vals[t] = (i0 + t <= r) ? tv.x * bv.x : 0.f;
      vals[t + 1] = (i0 + t + 1 <= r) ? tv.y * bv.y : 0.f;
      vals[t + 2] = (i0 + t + 2 <= r) ? tv.z * bv.z : 0.f;
      vals[t + 3] = (i0 + t + 3 <= r) ? tv.w * bv.w : 0.f;
    }
#pragma unroll
    for (int b = 0; b < RPP / 8; ++b) {
      kgh[b][0].store(r1 + c0 * L::LDT + r0p + 8 * b);
      kgh[b][1].store(r1 + (c0 + 1) * L::LDT + r0p + 8 * b);
    }
    __syncthreads();  // every read of T done
#pragma unroll
    for (int t = 0; t < TW; t += 8) st8t(sTb + r * L::LDT + i0 + t, vals + t);
  }
  __syncthreads();

  // ---- U = T Diag(beta) V and Wk^T = (K o e^G)^T (T Diag(beta))^T --------------
  // (from (K o e^(G-m))^T, then times e^m per channel)
  {
    // wave w: the 16 rows rb = w % 4 of T, and column blocks nb of its
    // share (with 8 waves, waves 4..7 take the second half of the blocks)
    const int rb = wave & 3;
    constexpr int NBW = (D / 16) / (NW / 4);
    const int nb0 = (wave >> 2) * NBW;
    typename M::frag tb[kC / M::KSTEP];
#pragma unroll
    for (int ks = 0; ks < kC / M::KSTEP; ++ks) tb[ks] = frag_t<T>(sTb, L::LDT, rb * 16, ks, lane);
#pragma unroll
    for (int nb = nb0; nb < nb0 + NBW; ++nb) {
      f32x4_t u = {0.f, 0.f, 0.f, 0.f}, wk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kC / M::KSTEP; ++ks) {
        u = M::mma(tb[ks], frag_t<T>(r0, L::LDT, nb * 16, ks, lane), u);    // B = V^T rows
        wk = M::mma(frag_t<T>(r1, L::LDT, nb * 16, ks, lane), tb[ks], wk);   // A = KG^T rows
      }
      // u: rows r = rb*16 + 4*(lane/16) + j, column n = nb*16 + lane%16 -> tile (nb, rb)
      st4(wUT + ((nb * (kC / 16) + rb) * 64 + lane) * 4, u[0], u[1], u[2], u[3]);
      // wk: rows c = nb*16 + 4*(lane/16) + j of Wk^T, column r = rb*16 + lane%16
      const int c4 = nb * 16 + 4 * (lane >> 4), r = rb * 16 + (lane & 15);
      if (mid) {  // from K o e^(G-m): times e^m per channel
        const float4 e4 = *reinterpret_cast<const float4*>(s_em + c4);
        wk[0] *= e4.x; wk[1] *= e4.y; wk[2] *= e4.z; wk[3] *= e4.w;
      }
      st_fnat4(wWN, D / M::KSTEP, r, c4, -wk[0], -wk[1], -wk[2], -wk[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// K2: sequential state pass over one sequence's chunks for one d_v slice.
//
// Per chunk, wave w owns output rows [16w, 16w+16) (W and O) and state rows
// [16*CBW*w, 16*CBW*(w+1)) (S).  The fragments a wave needs from the chunk's
// record -- its rows of -Wk, Q o e^G and P, its rows of K~, its U tiles and
// e^gamma -- are private to the wave and go straight from memory into
// registers (the record is stored in operand order, so each fragment is one
// contiguous 1 KiB wave load); only S and W, which every wave reads in full,
// pass through LDS.  Fragments are prefetched two chunks ahead into three
// register sets (see the loop at the end of the kernel).
// Buffer-resource loads: one resource per head's records, a per-lane 32-bit
// offset computed once, the slot's record offset in a scalar register and the
// fragment's constant offset in the instruction -- no per-load address math.
// Four consecutive elements, raw bits.
template <typename T> struct BufRaw4;
template <> struct BufRaw4<bf16> {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
  }
  __device__ __forceinline__ f32x4_t get() const {
    return f32x4_t{bf_val(v[0] & 0xffffu), bf_val(v[0] >> 16), bf_val(v[1] & 0xffffu),
                   bf_val(v[1] >> 16)};
  }
};
template <> struct BufRaw4<float> {
  u32x4_t v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
    v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  }
  __device__ __forceinline__ f32x4_t get() const { return __builtin_bit_cast(f32x4_t, v); }
};
// Four consecutive elements from floats, as one buffer store.
// o is written once and read by nobody here: non-temporal (the buffer
// instruction's cache-policy operand, bit 1) keeps the chunk records in the
// caches instead.
constexpr int kNtStore = 2;
template <typename T> struct BufStore4;
template <> struct BufStore4<bf16> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float a,
                                               float b, float c, float d) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kNtStore);
  }
};
template <> struct BufStore4<float> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float a,
                                               float b, float c, float d) {
    const u32x4_t v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c),
                       __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNtStore);
  }
};

// Per-wave fragments of one chunk's record (see kda_state_pass).
//
// On the bf16 path the chain's own operands (-Wk and K~ fragments) come by
// LDS-direct loads: a buffer load with the LDS bit writes each lane's 16
// bytes straight into LDS (at the wave's M0 base + 16 x lane), bypassing the
// VGPRs.  Measured on MI355X, a CU takes in ~100 B/ns of L2 or last-level
// cache data this way against ~60 B/ns through VGPR loads, and the state
// pass is bound by that intake.  Each fragment is one contiguous 1 KiB block
// of the record (operand order), so one LDS-direct load moves one fragment
// into one 1 KiB LDS block, and the wave that uses it reads its 16 bytes
// back with one ds_read_b128 (no bank conflicts).  The loads are issued by
// producer waves that do nothing else (see kda_state_pass); the compute
// waves' fragments of U, e^gamma, Q o e^G and P stay on the VGPR path, so
// the two paths feed the CU together.  fp32 operands (4 bytes per lane and
// k-step, twice the bytes) keep every fragment on the VGPR path.
template <typename T> constexpr bool k2_dma() { return sizeof(T) == 2; }
constexpr int kK2Producers = 2;  // producer waves of a bf16 state-pass workgroup
template <typename T> constexpr int k2_threads() {
  return k2_dma<T>() ? kThreads + 64 * kK2Producers : kThreads;
}

template <typename T, int D, int WS, bool OUT>
struct K2Frags {
  using M = Mma<T>;
  using R = Rec<T, D>;
  static constexpr int NB = WS / 16, CBW = D / 64, KD = D / M::KSTEP, KC = kC / M::KSTEP;
  static constexpr uint32_t ES = sizeof(T), FB = M::KPL * ES;  // bytes of a lane's fragment
  static constexpr bool DMA = k2_dma<T>();
  // LDS-direct fragments per wave and chunk: -Wk (KD), then K~ (CBW x KC)
  static constexpr int NDMA = KD + CBW * KC;
  static constexpr int WAVE_LDS = DMA ? NDMA * 64 * (int)FB : 0;  // bytes per wave and buffer
  static_assert(!DMA || (4 * NDMA) % kK2Producers == 0, "fragments split evenly over producers");
  static constexpr int VW = DMA ? 1 : KD, VC = DMA ? 1 : CBW, VK = DMA ? 1 : KC;
  typename M::frag wn[VW], qg[KD], p[KC], kt[VC][VK];
  BufRaw4<T> ut[NB];
  BufRaw4<float> eg[CBW];

  // lane offsets (bytes within a record), computed once per workgroup
  struct Offs { uint32_t wn, qg, p, kt, ut, eg, pz; };
  static __device__ __forceinline__ Offs offsets(int wave, int lane, int n0) {
    Offs o;
    o.wn = (uint32_t)(R::WN * ES) + ((wave * KD) * 64 + lane) * FB;
    o.qg = (uint32_t)(R::QG * ES) + ((wave * KD) * 64 + lane) * FB;
    o.p = (uint32_t)(R::P * ES) + ((wave * KC) * 64 + lane) * FB;
    o.kt = (uint32_t)(R::KT * ES) + ((wave * CBW * KC) * 64 + lane) * FB;
    o.ut = (uint32_t)(R::UT * ES) + (((n0 / 16) * (kC / 16) + wave) * 64 + lane) * 4 * ES;
    o.eg = (uint32_t)R::BYTES_T + (wave * CBW * 16 + 4 * (lane >> 4)) * 4;
    o.pz = (uint32_t)wave;
    return o;
  }
  // -Wk fragment ks and K~ fragment (i, ks) of this wave, from its block of
  // an LDS record buffer (DMA path) or from registers
  __device__ __forceinline__ typename M::frag wn_at(const char* wl, int ks, int lane) const {
    if constexpr (DMA)
      return M::load(reinterpret_cast<const T*>(wl + ks * 64 * FB) + lane * M::KPL);
    else
      return wn[ks];
  }
  __device__ __forceinline__ typename M::frag kt_at(const char* wl, int i, int ks, int lane) const {
    if constexpr (DMA)
      return M::load(reinterpret_cast<const T*>(wl + (KD + i * KC + ks) * 64 * FB) + lane * M::KPL);
    else
      return kt[i][ks];
  }
  // The loads come in four groups so that a step can spread them between
  // its phases: a CU's vector memory path takes ~1 KiB per 16 cycles, and
  // a wave that issues a whole record at once stalls behind it.  On the DMA
  // path -Wk and K~ are not loaded here (the producer waves bring them).
  template <int PART>
  __device__ __forceinline__ void load_part(__amdgpu_buffer_rsrc_t r, uint32_t soff, const Offs& o) {
    // in the order a step consumes them: U and -Wk (W), Q o e^G (O), e^gamma
    // and K~ (state update), P (O)
    if constexpr (PART == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ut[nb].load(r, o.ut + nb * (kC / 16) * 64 * 4 * ES, soff);
      if constexpr (!DMA) {
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) wn[ks] = BufFrag<T>::load(r, o.wn + ks * 64 * FB, soff);
      }
    } else if constexpr (PART == 1) {
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) qg[ks] = BufFrag<T>::load(r, o.qg + ks * 64 * FB, soff);
    } else if constexpr (PART == 2) {
#pragma unroll
      for (int i = 0; i < CBW; ++i) eg[i].load(r, o.eg + i * 64, soff);
      if constexpr (!DMA) {
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
          for (int ks = 0; ks < KC; ++ks)
            kt[i][ks] = BufFrag<T>::load(r, o.kt + (i * KC + ks) * 64 * FB, soff);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        // a k-step whose lowest 16-row block lies past this wave's rows is
        // zero (P is lower triangular): read past the bound instead (zeros,
        // no memory access, the same instruction count in every wave)
        const bool zero = (ks * M::KSTEP) / 16 > (int)o.pz;
        p[ks] = BufFrag<T>::load(r, zero ? kPastBound : o.p + ks * 64 * FB, soff);
      }
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t soff, const Offs& o) {
    load_part<0>(r, soff, o);
    if constexpr (OUT) load_part<1>(r, soff, o);
    load_part<2>(r, soff, o);
    if constexpr (OUT) load_part<3>(r, soff, o);
  }
  // Producer side: LDS-direct loads of one chunk's -Wk and K~ fragments for
  // all four compute waves into record buffer `buf` ([wave][fragment][lane]
  // [16 bytes]); producer wave pw of kK2Producers takes every
  // kK2Producers-th fragment.  Returns nothing; each call issues PER_PRODUCER
  // loads.
  static constexpr int PER_PRODUCER = 4 * NDMA / kK2Producers;
  static __device__ __forceinline__ void produce(__amdgpu_buffer_rsrc_t r, uint32_t soff,
                                                 char* buf, int pw, int lane) {
#pragma unroll
    for (int t = 0; t < PER_PRODUCER; ++t) {
      const int f = pw + t * kK2Producers;    // fragment of the workgroup's record share
      const int cw = f / NDMA, fi = f % NDMA;  // compute wave, its fragment index
      const uint32_t voff =
          fi < KD ? (uint32_t)(R::WN * ES) + ((cw * KD + fi) * 64 + lane) * FB
                  : (uint32_t)(R::KT * ES) + ((cw * CBW * KC + (fi - KD)) * 64 + lane) * FB;
      dma_load16(r, buf + (cw * NDMA + fi) * 64 * FB, voff, soff);
    }
  }
};

// OUT = false (the forward states inside the backward, over records that
// kda_bwd_prep writes): no output, so neither Q o e^G nor P is loaded and O
// is not formed.
template <typename T, int D, int WS, bool OUT>
__global__ __launch_bounds__(k2_threads<T>(), 1) void kda_state_pass(
    const char* __restrict__ ws, ChunkGeom gm, int H, int64_t s0, int64_t s1, int seg,
    int nseg, int64_t seg_slots, int nslice, int NH, const float* __restrict__ init, float* __restrict__ carry,
    float* __restrict__ fin, float* __restrict__ ckpt, int64_t ckpt_every, int64_t nckpt,
    T* __restrict__ states, float scale, T* __restrict__ o) {
  using M = Mma<T>;
  using R = Rec<T, D>;
  using F = K2Frags<T, D, WS, OUT>;
  constexpr int NB = F::NB, CBW = F::CBW, KD = F::KD, KC = F::KC;
  constexpr int LDS_S = D + 8, LDS_W = kC + 8;
  __shared__ __align__(16) char lds_raw[(WS * LDS_S + WS * LDS_W) * sizeof(T)];
  T* sSt = reinterpret_cast<T*>(lds_raw);                // S^T slice [n][c]
  T* sWt = sSt + WS * LDS_S;                             // W^T slice [n][i]
  constexpr int LDF = WS + 16 / (int)sizeof(T);
  __shared__ __align__(16) T sSf[D * LDF];               // S slice [c][n] (states)
  // LDS record buffers for the LDS-direct fragments of chunks j, j + 1 and
  // j + 2 (bf16 path), each [compute wave][fragment][lane][16 bytes]
  constexpr int RBB = F::DMA ? (kThreads / 64) * F::WAVE_LDS : 16;
  __shared__ __align__(16) char rb0[RBB];
  __shared__ __align__(16) char rb1[RBB];
  __shared__ __align__(16) char rb2[RBB];

  // XCD-aware placement: workgroups of one (sequence, head) share id mod 8.
  const int id = blockIdx.x;
  const int nh = (id & 7) + 8 * (id / (8 * nslice));
  const int slice = (id >> 3) % nslice;
  if (nh >= NH) return;
  const int seq = nh / H, h = nh % H;
  const int n0 = slice * WS;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // This sequence's chunks inside the segment's slot range [s0, s1).  The
  // state enters from init_state at the sequence's first chunk, otherwise from
  // the carry buffer the previous segment left; it leaves to final_state after
  // the last chunk, otherwise to the carry buffer.
  const SeqSpan sp = seq_span(gm, seq);
  const int64_t nrec = s1 - s0;
  if (sp.c0 == sp.c1) {  // empty sequence: final = init, once
    if (seg != (int)min<int64_t>(sp.c0 / seg_slots, nseg - 1) || fin == nullptr) return;
    const int64_t base = (int64_t)nh * D * D;
    for (int e = threadIdx.x; e < D * WS; e += blockDim.x) {
      const int64_t idx = base + (int64_t)(e / WS) * D + n0 + e % WS;
      fin[idx] = init ? init[idx] : 0.f;
    }
    return;
  }
  const int64_t slot0 = max(sp.c0, s0), slot1 = min(sp.c1, s1);
  if (slot0 >= slot1) return;
  const float* src = slot0 == sp.c0 ? init : carry;
  float* dst = slot1 == sp.c1 ? fin : carry;

  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ws + (int64_t)h * nrec * R::BYTES), (short)0, (int)(nrec * R::BYTES), kRsrcWord3);
  auto soff = [](int j) { return (uint32_t)j * (uint32_t)R::BYTES; };
  // The loop runs over 32-bit record indices j in [j0, j1) relative to the
  // segment (64-bit scalar compares would need vector temporaries, whose
  // reuse makes the compiler drain the prefetched loads).
  const int j0 = (int)(slot0 - s0), j1 = (int)(slot1 - s0);

  // Producer waves (bf16 path): LDS-direct loads of each chunk's -Wk and K~
  // fragments into three record buffers, two chunks ahead.  A producer
  // issues nothing but these loads, so its vmcnt counts exactly them: before
  // a step's first barrier it waits until only the next chunk's loads are in
  // flight (this chunk's have landed in LDS), and after that barrier -- by
  // which every compute wave has finished reading the chunk before this
  // one -- it refills that chunk's buffer with chunk j + 2.  It takes part in
  // both barriers of every step, as the compute waves do, and ends with no
  // load in flight.  The compute waves issue no LDS-direct load, so the
  // compiler's wait tracking never makes them wait for one.
  if constexpr (F::DMA) {
    if (wave >= 4) {
      const int pw = wave - 4;
      F::produce(rsrc, soff(j0), rb0, pw, lane);
      F::produce(rsrc, soff(min(j0 + 1, j1 - 1)), rb1, pw, lane);
      int b2 = 2;  // buffer of chunk j + 2
      for (int j = j0; j < j1; ++j) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(F::PER_PRODUCER));
        lds_barrier();
        F::produce(rsrc, soff(min(j + 2, j1 - 1)), b2 == 0 ? rb0 : b2 == 1 ? rb1 : rb2, pw, lane);
        b2 = b2 == 2 ? 0 : b2 + 1;
        lds_barrier();
      }
      __builtin_amdgcn_s_waitcnt(0);
      return;
    }
  }

  // state accumulators: wave owns rows (cb = wave*CBW + i) x all NB column blocks
  f32x4_t S[CBW][NB];
  const int64_t sbase = (int64_t)nh * D * D;
#pragma unroll
  for (int i = 0; i < CBW; ++i)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = (wave * CBW + i) * 16 + 4 * (lane >> 4) + j;
        const int n = n0 + nb * 16 + (lane & 15);
        S[i][nb][j] = src ? src[sbase + (int64_t)c * D + n] : 0.f;
      }

  const typename F::Offs offs = F::offsets(wave, lane, n0);
  const int cdelta = (int)(s0 - sp.c0);             // chunk index = j + cdelta
  const int ci_last = (int)((sp.ntok - 1) / kC);    // the sequence's last chunk
  const int len_last = (int)(sp.ntok - (int64_t)ci_last * kC);
  const int r_out = wave * 16 + (lane & 15);  // this lane's output row in a chunk
  const int64_t ostride = (int64_t)kC * H * D;  // elements from one chunk's rows to the next's
  // Checkpoints fall after every ck_chunks whole chunks of the sequence;
  // ck_left counts the chunks up to and including the next one.
  const int ck_chunks = ckpt != nullptr ? (int)(ckpt_every / kC) : 1;
  int ck_left = ck_chunks - (j0 + cdelta) % ck_chunks;

  // Output of a chunk is stored during the next step (so the store never
  // waits for the MFMA pipe): O holds the pending chunk's O^T, o_pend its
  // first row for this lane's column block, len_pend its valid rows.  The
  // store is a buffer store whose bound ends after row len_pend - 1, so rows
  // past a sequence's end are dropped by the hardware, without a branch.
  // Without o (the forward pass run inside the backward) every store is
  // dropped the same way.
  f32x4_t O[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) O[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  T* o_pend = o ? o + ((sp.tok0 + (int64_t)(j0 + cdelta) * kC) * H + h) * D + n0 : nullptr;
  int len_pend = 0;
  const uint32_t o_voff = (uint32_t)((r_out * H * D + 4 * (lane >> 4)) * sizeof(T));
  auto store_o = [&]() {
    const int nbytes =
        (o_pend != nullptr && len_pend > 0) ? ((len_pend - 1) * H * D + WS) * (int)sizeof(T) : 0;
    // (a bound of 0 on a real address when there is no o: every store dropped)
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        o_pend ? (void*)o_pend : (void*)ws, (short)0, nbytes, kRsrcWord3);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      BufStore4<T>::store(ro, o_voff + nb * 16 * sizeof(T), scale * O[nb][0], scale * O[nb][1],
                          scale * O[nb][2], scale * O[nb][3]);
  };

  // For the backward: the state entering chunk slot s0 + j, [slot][H] of
  // slice-blocked D x D in the MFMA type (sblk: this workgroup's slice is one
  // contiguous D x 16 block; the backward uses S only as a product operand,
  // rounded to that type the same way, and in one fp32 row sum).  Step j
  // passes S through LDS beside the transposed MFMA copy, and after the
  // barrier the block is stored in 16-byte pieces
  // -- after the step's first prefetch loads (the wait counter is in order,
  // so a store issued before them would hold up every wait for them).
  // Only the pass without o (inside the backward) writes states.
  const bool want_states = !OUT && states != nullptr;
  auto store_state = [&](int j) {
    static_assert(WS == 16, "states are stored in 16-column slices");
    T* sd = states + ((s0 + j) * H + h) * (int64_t)D * D + sblk<D>(0, n0);
    constexpr int VE = 16 / (int)sizeof(T), PPR = WS / VE;  // 16-byte pieces per row
#pragma unroll
    for (int pr = 0; pr < (D * PPR + kThreads - 1) / kThreads; ++pr) {
      const int pc = pr * kThreads + threadIdx.x, row = pc / PPR, cv = VE * (pc % PPR);
      if (D * PPR % kThreads == 0 || pc < D * PPR)
        *reinterpret_cast<u32x4_t*>(sd + row * 16 + cv) =
            *reinterpret_cast<const u32x4_t*>(sSf + row * LDF + cv);
    }
  };
  // One chunk step: consumes the fragments in f and fills fn with those of
  // record jn (clamped to the last record), the loads spread over the step.
  auto step = [&](const F& f, F& fn, const char* lcur, int j, int jn) {
    const uint32_t son = soff(min(jn, j1 - 1));
    const char* wl = lcur + wave * F::WAVE_LDS;   // this wave's -Wk, K~ of chunk j (DMA path)
    const int ci = j + cdelta;  // chunk index within the sequence
    const int len = ci == ci_last ? len_last : kC;

    // (a) S -> LDS as S^T in the MFMA type
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c4 = (wave * CBW + i) * 16 + 4 * (lane >> 4);
        const int n = nb * 16 + (lane & 15);
        st_perm4(sSt + n * LDS_S, c4, S[i][nb][0], S[i][nb][1], S[i][nb][2], S[i][nb][3]);
        if (want_states) {
#pragma unroll
          for (int e = 0; e < 4; ++e) st_elem(sSf + (c4 + e) * LDF + n, S[i][nb][e]);
        }
      }
    lds_barrier();
    // -Wk fragments: in the chunk's LDS record buffer once the producers have
    // passed the barrier above
    typename M::frag wnf[KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) wnf[ks] = f.wn_at(wl, ks, lane);

    // (b) W = U + (-Wk) S for this wave's 16 rows -- the chain's critical
    // path -- is issued first; then the previous chunk's output store and
    // O^T = S^T (Q o e^G)^T, which overlap the W -> LDS hand-off.
    typename M::frag sfr[NB][KD];
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sfr[nb][ks] = frag_at<T>(sSt, LDS_S, nb * 16, ks, lane);
    f32x4_t W[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) W[nb] = f.ut[nb].get();
#pragma unroll
    for (int ks = 0; ks < KD; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) W[nb] = M::mma(wnf[ks], sfr[nb][ks], W[nb]);
    __builtin_amdgcn_sched_barrier(0);
    fn.template load_part<0>(rsrc, son, offs);
    // sSf is written again only after this step's second barrier
    if (want_states) store_state(j);
    if constexpr (OUT) {
      store_o();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) O[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KD; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb] = M::mma(sfr[nb][ks], f.qg[ks], O[nb]);
      __builtin_amdgcn_sched_barrier(0);
      fn.template load_part<1>(rsrc, son, offs);
    }
    __builtin_amdgcn_sched_barrier(0);

    // (c) W -> LDS as W^T
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = nb * 16 + (lane & 15);
      st_perm4(sWt + n * LDS_W, wave * 16 + 4 * (lane >> 4), W[nb][0], W[nb][1], W[nb][2], W[nb][3]);
    }
    // K~ fragments (own LDS-direct loads)
    typename M::frag ktf[CBW][KC];
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) ktf[i][ks] = f.kt_at(wl, i, ks, lane);
    lds_barrier();

    // (d) S = Diag(e^gamma) S + K~^T W first (critical path), then O^T += W^T P^T
    typename M::frag wf[NB][KC];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) wf[nb][ks] = frag_at<T>(sWt, LDS_W, nb * 16, ks, lane);
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4_t eg = f.eg[i].get();
#pragma unroll
        for (int j = 0; j < 4; ++j) S[i][nb][j] *= eg[j];
#pragma unroll
        for (int ks = 0; ks < KC; ++ks) S[i][nb] = M::mma(ktf[i][ks], wf[nb][ks], S[i][nb]);
      }
    __builtin_amdgcn_sched_barrier(0);
    fn.template load_part<2>(rsrc, son, offs);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (OUT) {
#pragma unroll
      for (int ks = 0; ks < KC; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb] = M::mma(wf[nb][ks], f.p[ks], O[nb]);
      __builtin_amdgcn_sched_barrier(0);
      fn.template load_part<3>(rsrc, son, offs);
      __builtin_amdgcn_sched_barrier(0);
    }

    // (e) checkpoint after every ckpt_every tokens (dense, chunk-aligned)
    if (ckpt != nullptr && --ck_left == 0) {
      ck_left = ck_chunks;
      if (len == kC) {
        const int64_t jslot = (ci + 1) / ck_chunks - 1;
        float* cdst = ckpt + (((int64_t)seq * nckpt + jslot) * H + h) * (int64_t)D * D;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int c = (wave * CBW + i) * 16 + 4 * (lane >> 4) + j;
              cdst[(int64_t)c * D + n0 + nb * 16 + (lane & 15)] = S[i][nb][j];
            }
      }
    }
    // this chunk's output is now pending
    o_pend = (j == j0 || o_pend == nullptr) ? o_pend : o_pend + ostride;
    len_pend = len;
    // No barrier here: the next chunk's sSt writes follow this chunk's
    // second barrier (after every wave read sSt), and its sWt writes follow
    // the next chunk's first barrier (after every wave read sWt).
  };


  // Fragments are prefetched two chunks ahead in three register sets; the
  // loop body is three whole steps, so each set stays in fixed registers,
  // and the one or two steps left over run after it.  Every prefetch is
  // unconditional (past the end it re-reads the last record) and the loop
  // has no early exit, so the in-order wait counter only ever waits for the
  // set being consumed.
  // Register set fa and LDS buffer rb0 hold chunk j, fb / rb1 chunk j + 1,
  // fc / rb2 chunk j + 2 (the LDS-direct fragments follow the same rotation).
  F fa, fb, fc;
  fa.load(rsrc, soff(j0), offs);
  __asm__ volatile("" ::: "memory");  // issue the first set's loads first
  fb.load(rsrc, soff(min(j0 + 1, j1 - 1)), offs);
  int j = j0;
  for (; j + 3 <= j1; j += 3) {
    step(fa, fc, rb0, j, j + 2);
    step(fb, fa, rb1, j + 1, j + 3);
    step(fc, fb, rb2, j + 2, j + 4);
  }
  if (j < j1) step(fa, fc, rb0, j, j + 2);
  if (j + 1 < j1) step(fb, fa, rb1, j + 1, j + 3);
  if constexpr (OUT) store_o();

  if (dst != nullptr) {
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = (wave * CBW + i) * 16 + 4 * (lane >> 4) + j;
          dst[sbase + (int64_t)c * D + n0 + nb * 16 + (lane & 15)] = S[i][nb][j];
        }
  }
}

// ---------------------------------------------------------------------------
// Host side: workspace plan and launches.
//
// Chunk slots are processed in segments of at most seg_slots() slots: K1 fills
// the segment's records, then K2 advances every sequence through its chunks
// inside the segment.  The workspace therefore holds one segment's records
// (bounded for any T), the fp32 states carried between segments, and the
// varlen chunk map.
struct Plan {
  int64_t slot_bound;   // upper bound on chunk slots (dense exact, varlen bound)
  int64_t seg_slots;    // slots per segment
  int64_t rec_bytes;
  int64_t rec_total;    // bytes of one segment's records
  int64_t carry_bytes;  // fp32 states carried between segments
  int64_t map_bytes;    // varlen: sanitised cu_seqlens + chunk offsets
};

int64_t rec_bytes_for(const kda_desc_t& d) {
  if (d.dtype == KDA_DTYPE_BF16)
    return d.dk == 128 ? Rec<bf16, 128>::BYTES : Rec<bf16, 64>::BYTES;
  return d.dk == 128 ? Rec<float, 128>::BYTES : Rec<float, 64>::BYTES;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Segment length in chunk slots: the record budget over the records of one
// slot (all heads), a multiple of 8 in [8, kSegSlotsMax].  KDA_SEG_SLOTS
// (read once) overrides it for tuning.  It fixes the workspace size, so it
// depends only on the descriptor.
int64_t seg_slots(const kda_desc_t& d) {
  static const int64_t env = [] {
    const char* e = getenv("KDA_SEG_SLOTS");
    const long long x = e ? atoll(e) : 0;
    return x > 0 ? std::max<int64_t>(8, std::min<int64_t>(kSegSlotsMax, x)) & ~(int64_t)7
                 : (int64_t)0;
  }();
  if (env) return env;
  const int64_t per_slot = (int64_t)d.heads * rec_bytes_for(d);
  const int64_t s = (kSegRecordBudget / per_slot) & ~(int64_t)7;
  return std::max<int64_t>(8, std::min<int64_t>(kSegSlotsMax, s));
}

// Workspace plan for segments of at most ss chunk slots.
Plan make_plan(const kda_desc_t& d, bool varlen, int64_t ss) {
  Plan p{};
  const int64_t T = d.seqlen;
  p.slot_bound = varlen ? (T + (int64_t)(kC - 1) * d.num_seqs) / kC
                        : (int64_t)d.batch * ((T + kC - 1) / kC);
  p.seg_slots = std::min<int64_t>(p.slot_bound, ss);
  p.rec_bytes = rec_bytes_for(d);
  p.rec_total = p.seg_slots * d.heads * p.rec_bytes;
  p.carry_bytes = p.slot_bound > ss ? (int64_t)d.num_seqs * d.heads * d.dk * d.dv * 4 : 0;
  p.map_bytes = varlen ? 2 * align256(((int64_t)d.num_seqs + 1) * 4) : 0;
  return p;
}
Plan make_plan(const kda_desc_t& d, bool varlen) { return make_plan(d, varlen, seg_slots(d)); }

// Workspace bytes for segments of at most ss slots: the larger of the dense
// and varlen layouts (whether cu_seqlens will be passed is not known here;
// they differ only in the slot bound and the map).
int64_t workspace_for(const kda_desc_t& d, int64_t ss) {
  const Plan pv = make_plan(d, true, ss), pd = make_plan(d, false, ss);
  const int64_t a = pv.rec_total + pv.carry_bytes + pv.map_bytes;
  const int64_t b = pd.rec_total + pd.carry_bytes + pd.map_bytes;
  return a > b ? a : b;
}

template <typename T, int D>
hipError_t run_typed(const kda_desc_t& d, const void* q, const void* k, const void* v,
                     const float* g, const float* beta, const float* init_state,
                     const int32_t* cu, void* o, float* final_state, float* ckpt,
                     void* states, char* ws, int64_t SS, chunk_record_stage_fn stage,
                     void* stage_ctx, const ConvIn* conv, hipStream_t stream) {
  const bool varlen = cu != nullptr;
  const Plan p = make_plan(d, varlen, SS);
  const int H = d.heads, NH = d.num_seqs * d.heads;
  char* recs = ws;
  float* carry = p.carry_bytes ? reinterpret_cast<float*>(ws + p.rec_total) : nullptr;
  int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + p.rec_total + p.carry_bytes);
  int32_t* cu_s = chunk_off + (p.map_bytes / 2) / 4;  // sanitised cu_seqlens
  // d_v columns per K2 workgroup: the smallest MFMA tile width.  A
  // workgroup loads the same per-chunk operands whatever its width, so
  // narrower slices spread the per-step math over more CUs at no extra
  // per-CU traffic (one (sequence, head) chain then occupies D/16 CUs).
  constexpr int WS = 16;
  const int nslice = D / WS;
  const int nhpad = (NH + 7) / 8 * 8;
  const int k1_lds = K1Lds<T, D>::BYTES;
  // the per-chunk states are written only by the pass without o, and only
  // that pass takes its records from a caller's stage
  if (o != nullptr && (states != nullptr || stage != nullptr)) return hipErrorInvalidValue;
  // K1's dynamic LDS limit, once per device
  static std::atomic<uint64_t> attr_done{0};
  hipError_t ea = once_per_device(attr_done, [&]() {
    for (const void* fn : {(const void*)kda_intra_chunk<T, D, false>,
                           (const void*)kda_intra_chunk<T, D, true>,
                           (const void*)kda_intra_chunk<T, D, false, true>,
                           (const void*)kda_intra_chunk<T, D, true, true>}) {
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, k1_lds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
  if (ea != hipSuccess) return ea;
  const int64_t nck = d.ckpt_every > 0 ? d.seqlen / d.ckpt_every : 0;
  ChunkGeom gm{nullptr, nullptr, d.seqlen, (d.seqlen + kC - 1) / kC, d.num_seqs};
  if (varlen) {
    hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(kThreads), 0, stream, cu, d.num_seqs,
                       d.seqlen, cu_s, chunk_off);
    gm = ChunkGeom{cu_s, chunk_off, d.seqlen, 0, d.num_seqs};
  }
  const int64_t nseg = p.slot_bound == 0 ? 1 : (p.slot_bound + SS - 1) / SS;
  for (int64_t s = 0; s < nseg; ++s) {
    const int64_t s0 = s * SS, s1 = std::min<int64_t>(p.slot_bound, s0 + SS);
    if (s1 > s0 && stage != nullptr) {
      const hipError_t es = stage(stage_ctx, s0, s1, recs, stream);
      if (es != hipSuccess) return es;
    } else if (s1 > s0) {
      if (o == nullptr) return hipErrorInvalidValue;  // a states-only pass takes a stage
      auto k1 = conv != nullptr
                    ? (d.gate_per_head ? kda_intra_chunk<T, D, true, true>
                                       : kda_intra_chunk<T, D, false, true>)
                    : (d.gate_per_head ? kda_intra_chunk<T, D, true> : kda_intra_chunk<T, D, false>);
      hipLaunchKernelGGL(k1, dim3(H, (unsigned)(s1 - s0)), dim3(k1_threads<T, D>()), k1_lds,
                         stream, (const T*)q, (const T*)k, (const T*)v, g, beta, gm, H, s0,
                         s1 - s0, d.qk_l2norm, recs, conv != nullptr ? *conv : ConvIn{});
    }
    auto k2 = o ? kda_state_pass<T, D, WS, true> : kda_state_pass<T, D, WS, false>;
    hipLaunchKernelGGL(k2, dim3(nhpad * nslice), dim3(k2_threads<T>()), 0,
                       stream, recs, gm, H, s0, s1, (int)s, (int)nseg, SS, nslice, NH, init_state,
                       carry, final_state, ckpt, d.ckpt_every, nck, (T*)states, d.scale, (T*)o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t chunk_workspace_bytes(const kda_desc_t& d) { return (size_t)workspace_for(d, seg_slots(d)); }

int64_t chunk_slot_bound(const kda_desc_t& d, bool varlen) {
  return make_plan(d, varlen).slot_bound;
}

namespace {
hipError_t launch_with(const kda_desc_t& d, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* init_state,
                       const int32_t* cu_seqlens, void* o, float* final_state, float* state_ckpt,
                       void* chunk_states, char* ws, int64_t ss, hipStream_t stream,
                       chunk_record_stage_fn stage = nullptr, void* stage_ctx = nullptr,
                       const ConvIn* conv = nullptr) {
  const bool bf = d.dtype == KDA_DTYPE_BF16;
  if (d.dk == 128)
    return bf ? run_typed<bf16, 128>(d, q, k, v, g, beta, init_state, cu_seqlens, o,
                                     final_state, state_ckpt, chunk_states, ws, ss, stage,
                                     stage_ctx, conv, stream)
              : run_typed<float, 128>(d, q, k, v, g, beta, init_state, cu_seqlens, o,
                                      final_state, state_ckpt, chunk_states, ws, ss, stage,
                                      stage_ctx, conv, stream);
  return bf ? run_typed<bf16, 64>(d, q, k, v, g, beta, init_state, cu_seqlens, o, final_state,
                                  state_ckpt, chunk_states, ws, ss, stage, stage_ctx, conv,
                                  stream)
            : run_typed<float, 64>(d, q, k, v, g, beta, init_state, cu_seqlens, o,
                                   final_state, state_ckpt, chunk_states, ws, ss, stage,
                                   stage_ctx, conv, stream);
}
}  // namespace

hipError_t launch_chunk_fwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, void* o, float* final_state,
                            float* state_ckpt, void* chunk_states, void* workspace,
                            hipStream_t stream) {
  return launch_with(d, q, k, v, g, beta, init_state, cu_seqlens, o, final_state, state_ckpt,
                     chunk_states, static_cast<char*>(workspace), seg_slots(d), stream);
}

hipError_t launch_chunk_states(const kda_desc_t& d, const float* init_state,
                               const int32_t* cu_seqlens, void* chunk_states, void* workspace,
                               chunk_record_stage_fn stage, void* stage_ctx,
                               hipStream_t stream) {
  if (stage == nullptr || chunk_states == nullptr) return hipErrorInvalidValue;
  return launch_with(d, nullptr, nullptr, nullptr, nullptr, nullptr, init_state, cu_seqlens,
                     nullptr, nullptr, nullptr, chunk_states, static_cast<char*>(workspace),
                     seg_slots(d), stream, stage, stage_ctx);
}

hipError_t launch_chunk_fwd_conv(const kda_desc_t& d, const void* const x[3],
                                 const float* const w[3], const float* const bias[3],
                                 const float* const state_in[3], float* const state_out[3],
                                 const float* g, const float* beta, const float* init_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state,
                                 float* state_ckpt, void* workspace, hipStream_t stream) {
  const ConvIn conv{{w[0], w[1], w[2]}, {bias[0], bias[1], bias[2]},
                    {state_in[0], state_in[1], state_in[2]}};
  hipError_t e = launch_with(d, x[0], x[1], x[2], g, beta, init_state, cu_seqlens, o, final_state,
                             state_ckpt, nullptr, static_cast<char*>(workspace), seg_slots(d),
                             stream, nullptr, nullptr, &conv);
  if (e != hipSuccess) return e;
  // the carried-out inputs, after every read of the carried-in ones (they
  // may be the same arrays)
  return launch_conv_state_out(d.seqlen, d.num_seqs, d.heads * d.dk, d.dtype, x, state_in,
                               state_out, cu_seqlens, stream);
}

// ---------------------------------------------------------------------------
// The prefill without a caller workspace: the scratch is a fixed device array
// of the library (one copy per device, held until the process ends), and the
// chunk records use segments small enough to fit it.  Host code never uses
// the array's name as an address: each device's address comes from
// hipGetSymbolAddress, once per device, with that device current.
namespace {
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_for_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return hipSuccess;
}
}  // namespace

int64_t noalloc_seg_slots(const kda_desc_t& d) {
  // the segment length the normal path uses, or the largest multiple of 8
  // below it whose workspace fits the array (records shrink with the segment;
  // the carried states and the varlen map do not)
  for (int64_t ss = seg_slots(d); ss >= 8; ss -= 8)
    if (workspace_for(d, ss) <= (int64_t)kNoAllocScratchBytes) return ss;
  return workspace_for(d, 8) <= (int64_t)kNoAllocScratchBytes ? 8 : 0;
}

int64_t noalloc_min_bytes(const kda_desc_t& d) { return workspace_for(d, 8); }

hipError_t launch_chunk_fwd_noalloc(const kda_desc_t& d, const void* q, const void* k,
                                    const void* v, const float* g, const float* beta,
                                    const float* init_state, const int32_t* cu_seqlens, void* o,
                                    float* final_state, float* state_ckpt, hipStream_t stream) {
  const int64_t ss = noalloc_seg_slots(d);
  if (ss == 0) return hipErrorInvalidValue;  // the caller checks the size first
  char* ws = nullptr;
  hipError_t e = scratch_for_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_with(d, q, k, v, g, beta, init_state, cu_seqlens, o, final_state, state_ckpt,
                     nullptr, ws, ss, stream);
}

}  // namespace kda
