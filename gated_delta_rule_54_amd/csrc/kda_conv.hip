// kda_conv.hip -- the ShortConv + Swish prologue on gfx950.
//
// Pages cited (by title and section):
//   [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
//        §6 layer diagram (the q, k, v projections pass ShortConv -> Swish
//        before the operator) and §6.1.
//   [XD] xiudou.site, "Kimi Delta Attention：把遗忘门做到每个通道"
//        the preprocessing list: a small-window causal convolution mixing
//        each position with the few tokens just before it, then Swish.
//
// Per sequence n, channel c, token t (W taps, one filter per channel):
//   y_t[c] = swish(bias[c] + sum_{i<W} w[c][i] * x~[t - (W-1) + i][c])
// x~ is the sequence's input preceded by its carried state (the W-1 inputs
// before it, oldest first) or by zeros; the last W-1 entries of x~ are
// carried out.  Swish(a) = a * sigmoid(a).
//
// A thread owns kTB consecutive tokens of one 16-byte channel group and keeps
// the previous W-1 inputs of its channels in registers, so x is read once
// (plus W-1 halo rows per block, cache-served) and y written once: an HBM
// stream of 2 x element size per element.  Sequence starts inside a block
// (varlen packing) re-seed the window from the carried state; the thread
// that processes a sequence's last token writes its carried-out state.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <algorithm>

#include "kda_internal.h"

namespace kda {
namespace {

typedef unsigned int u32x4c_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2c_t __attribute__((ext_vector_type(2)));
constexpr int kConvThreads = 64;  // small workgroups spread the few long-lived ones evenly
constexpr int kTB = (int)kConvInPlaceMaxTokens;  // tokens per thread
constexpr int kGroup = 4;                          // token rows loaded together

template <typename T> struct CVec;
template <> struct CVec<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void unpack(u32x4c_t v, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(v[e]);
  }
  static __device__ __forceinline__ u32x4c_t pack(const float* x) {
    return u32x4c_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                    __float_as_uint(x[3])};
  }
};
template <> struct CVec<__hip_bfloat16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(u32x4c_t v, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(v[e] << 16);
      x[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ u32x4c_t pack(const float* x) {
    u32x4c_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2c_t p = {(__bf16)x[2 * e], (__bf16)x[2 * e + 1]};
      v[e] = __builtin_bit_cast(unsigned int, p);
    }
    return v;
  }
};

// Sequence of a packed token: the n with cu[n] <= t < cu[n+1] (the last such
// n, so empty sequences are skipped).
__device__ __forceinline__ int seq_of(const int32_t* cu, int N, int64_t t) {
  int lo = 0, hi = N;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// One workgroup per (token block, 64 channel groups): the token block is
// blockIdx.y, uniform over the workgroup, so each row's address is a scalar
// base plus the lane's channel offset -- no per-element address arithmetic
// -- and the 32-token loop is unrolled whole, so the window of the previous
// W-1 inputs lives in renamed registers instead of being shifted.  (The same thread -> memory mapping copies at ~6 TB/s without
// arithmetic; the kernel had been bound by its address, window and branch
// instructions on top of the convolution itself.)
template <typename T, int W>
__global__ __launch_bounds__(kConvThreads) void short_conv_kernel(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const float* state_in, const int32_t* __restrict__ cu, T* __restrict__ y, float* state_out,
    int64_t T_, int N, int C, int64_t nblocks_tok, int64_t tb_base) {
  using V = CVec<T>;
  constexpr int E = V::E, HW = W - 1;
  const int CG = C / E;  // channel groups per token row
  const int cg = blockIdx.x * kConvThreads + threadIdx.x;
  if (cg >= CG) return;
  const int64_t tb = tb_base + blockIdx.y;  // token block, or past them: a sequence
  if (tb >= nblocks_tok) {
    // rows past the token blocks (launched only with state_out): empty
    // sequences carry their state out unchanged (or zeros)
    const int n = (int)(tb - nblocks_tok);
    const int64_t len = cu ? (int64_t)cu[n + 1] - cu[n] : T_;
    if (len > 0) return;
    for (int k = 0; k < E * HW; ++k) {
      const int64_t idx = ((int64_t)n * C + cg * E) * HW + k;
      state_out[idx] = state_in ? state_in[idx] : 0.f;
    }
    return;
  }
  // dense: sequence b = tb / blocks_per_seq; varlen: packed tokens
  int64_t tok0, tok1;      // this block's rows
  int n;
  int64_t s_start, s_end;  // current sequence's rows [s_start, s_end)
  if (cu == nullptr) {
    const int64_t bps = (T_ + kTB - 1) / kTB;
    n = (int)(tb / bps);
    const int64_t seq_base = (int64_t)n * T_;
    tok0 = seq_base + (tb % bps) * kTB;
    tok1 = min(tok0 + kTB, seq_base + T_);
    s_start = seq_base;
    s_end = seq_base + T_;
  } else {
    tok0 = tb * kTB;
    tok1 = min(tok0 + kTB, T_);
    n = seq_of(cu, N, tok0);
    // clamped so that offsets not checked on the host cannot move a read
    // outside [0, T): valid offsets are unchanged
    s_start = min((int64_t)max(cu[n], 0), tok0);
    s_end = max(min((int64_t)cu[n + 1], T_), tok0 + 1);
  }
  const int c0 = cg * E;
  // this thread's E filters are E*W consecutive floats of w
  float wv[E][W], bv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bv[e] = bias ? bias[c0 + e] : 0.f;
    if constexpr (W == 4) {
      const float4 f = *reinterpret_cast<const float4*>(w + (c0 + e) * 4);
      wv[e][0] = f.x; wv[e][1] = f.y; wv[e][2] = f.z; wv[e][W - 1] = f.w;
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) wv[e][i] = w[(c0 + e) * W + i];
    }
  }
  // window: win[e][j] = x~ at row (t - HW + j) for the token t about to be
  // processed, j = 0..HW-1 (oldest first)
  float win[E][HW > 0 ? HW : 1];
  auto seed = [&](int64_t t) {  // window for token t of the current sequence
#pragma unroll
    for (int j = 0; j < HW; ++j) {
      const int64_t r = t - HW + j;
      if (r >= s_start) {
        float xv[E];
        V::unpack(*reinterpret_cast<const u32x4c_t*>(x + r * C + c0), xv);
#pragma unroll
        for (int e = 0; e < E; ++e) win[e][j] = xv[e];
      } else {
        const int64_t k = HW - (s_start - r);  // index into the carried state
#pragma unroll
        for (int e = 0; e < E; ++e)
          win[e][j] = state_in ? state_in[((int64_t)n * C + c0 + e) * HW + k] : 0.f;
      }
    }
  };
  seed(tok0);
  // one token: y_t from x_t and the window, then the window moves on
  auto token = [&](const u32x4c_t& xraw, float* out) {
    float xv[E];
    V::unpack(xraw, xv);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = bv[e] + wv[e][W - 1] * xv[e];
#pragma unroll
      for (int j = 0; j < HW; ++j) acc += wv[e][j] * win[e][j];
      // swish: a * sigmoid(a), the reciprocal in one hardware instruction
      out[e] = acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc));
      if constexpr (HW > 0) {
#pragma unroll
        for (int j = 0; j + 1 < HW; ++j) win[e][j] = win[e][j + 1];
        win[e][HW - 1] = xv[e];
      }
    }
  };
  auto carry_out = [&]() {
    if (state_out == nullptr) return;
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int j = 0; j < HW; ++j) state_out[((int64_t)n * C + c0 + e) * HW + j] = win[e][j];
  };
  if (tok1 - tok0 == kTB && s_end >= tok1) {
    // a whole block inside one sequence (every block of a dense batch): each
    // row through a pointer uniform over the workgroup (a scalar base) and
    // the lane's channel offset, and the loop unrolled whole so the window
    // stays in renamed registers.  (Global, not buffer, stores: a buffer
    // store with a register soffset is not given the wait state that a VALU
    // write of its data registers right after it needs, and its first data
    // dword was seen to take the new value.)
#pragma unroll
    for (int g0 = 0; g0 < kTB; g0 += kGroup) {
      u32x4c_t xr[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k)
        xr[k] = *reinterpret_cast<const u32x4c_t*>(x + (tok0 + g0 + k) * C + c0);
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        float out[E];
        token(xr[k], out);
        *reinterpret_cast<u32x4c_t*>(y + (tok0 + g0 + k) * C + c0) = V::pack(out);
      }
    }
    if (tok1 == s_end) carry_out();
    return;
  }
  // A block that ends early or holds a sequence start (varlen): tokens in
  // groups of kGroup, the group's rows loaded first (clamped to the block, so
  // every load is unconditional), then processed in order.
  for (int64_t tg = tok0; tg < tok1; tg += kGroup) {
    u32x4c_t xr[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int64_t tt = min(tg + k, tok1 - 1);
      xr[k] = *reinterpret_cast<const u32x4c_t*>(x + tt * C + c0);
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int64_t t = tg + k;
      if (t >= tok1) break;
      if (t == s_end) {  // a new (non-empty) sequence starts at this row
        n = seq_of(cu, N, t);
        s_start = min((int64_t)max(cu[n], 0), t);
        s_end = max(min((int64_t)cu[n + 1], T_), t + 1);
        seed(t);
      }
      float out[E];
      token(xr[k], out);
      *reinterpret_cast<u32x4c_t*>(y + t * C + c0) = V::pack(out);
      if (t + 1 == s_end) carry_out();
    }
  }
}

template <typename T, int W>
hipError_t launch_w(const kda_conv_args& a, hipStream_t stream) {
  const int CG = a.channels / CVec<T>::E;
  const int64_t nblocks_tok = a.cu ? (a.seqlen + kTB - 1) / kTB
                                   : (int64_t)a.batch * ((a.seqlen + kTB - 1) / kTB);
  const unsigned gx = (unsigned)((CG + kConvThreads - 1) / kConvThreads);
  // token blocks, then one row per sequence for the empty sequences' states,
  // in the grid's y dimension, at most kMaxY rows per launch
  const int64_t rows = nblocks_tok + (a.state_out != nullptr ? a.num_seqs : 0);
  constexpr int64_t kMaxY = 32768;
  for (int64_t b0 = 0; b0 < rows; b0 += kMaxY) {
    const unsigned gy = (unsigned)std::min<int64_t>(kMaxY, rows - b0);
    hipLaunchKernelGGL((short_conv_kernel<T, W>), dim3(gx, gy), dim3(kConvThreads), 0, stream,
                       static_cast<const T*>(a.x), a.w, a.bias, a.state_in, a.cu,
                       static_cast<T*>(a.y), a.state_out, a.seqlen, a.num_seqs, a.channels,
                       nblocks_tok, b0);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const kda_conv_args& a, hipStream_t stream) {
  switch (a.width) {
    case 1: return launch_w<T, 1>(a, stream);
    case 2: return launch_w<T, 2>(a, stream);
    case 3: return launch_w<T, 3>(a, stream);
    default: return launch_w<T, 4>(a, stream);
  }
}

// The inputs each sequence carries out when the prologue is fused into the
// operator (kda_chunk_fwd_conv, width 4): state_out[n, c, i] = x~[len_n + i],
// i < 3, where x~ is sequence n's input preceded by state_in[n, c, :] (or
// zeros) -- what the prologue kernel's carried window ends with.  One thread
// per (sequence, channel), grid y = the tensor (q, k, v; one launch for the
// three); its reads come before its writes, so state_out may be state_in.
struct ConvStateOut {
  const void* x[3];
  const float* state_in[3];
  float* state_out[3];
};

template <typename T>
__global__ void conv_state_out_kernel(ConvStateOut a, const int32_t* __restrict__ cu, int64_t T_,
                                      int N, int C) {
  const int t = blockIdx.y;
  float* state_out = a.state_out[t];
  if (state_out == nullptr) return;
  const T* __restrict__ x = static_cast<const T*>(a.x[t]);
  const float* state_in = a.state_in[t];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * C) return;
  const int n = (int)(i / C), c = (int)(i % C);
  int64_t tok0 = (int64_t)n * T_, len = T_;
  if (cu != nullptr) {
    // clamped as in the prologue kernel: offsets not checked on the host
    // cannot move a read outside [0, T)
    tok0 = min(max((int64_t)cu[n], (int64_t)0), T_);
    len = max(min((int64_t)cu[n + 1], T_) - tok0, (int64_t)0);
  }
  float s[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int64_t u = len + j;  // index into x~ (its first three entries carried in)
    s[j] = u < 3 ? (state_in ? state_in[i * 3 + u] : 0.f)
                 : static_cast<float>(x[(tok0 + u - 3) * C + c]);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) state_out[i * 3 + j] = s[j];
}

}  // namespace

hipError_t launch_conv_state_out(int64_t seqlen, int32_t num_seqs, int32_t channels,
                                 int32_t dtype, const void* const x[3],
                                 const float* const state_in[3], float* const state_out[3],
                                 const int32_t* cu, hipStream_t stream) {
  const int64_t n = (int64_t)num_seqs * channels;
  if (n == 0 || (!state_out[0] && !state_out[1] && !state_out[2])) return hipSuccess;
  const ConvStateOut a{{x[0], x[1], x[2]},
                       {state_in[0], state_in[1], state_in[2]},
                       {state_out[0], state_out[1], state_out[2]}};
  const dim3 grid((unsigned)((n + 255) / 256), 3);
  if (dtype == KDA_DTYPE_BF16)
    hipLaunchKernelGGL(conv_state_out_kernel<__hip_bfloat16>, grid, dim3(256), 0, stream, a, cu,
                       seqlen, num_seqs, channels);
  else
    hipLaunchKernelGGL(conv_state_out_kernel<float>, grid, dim3(256), 0, stream, a, cu, seqlen,
                       num_seqs, channels);
  return hipGetLastError();
}

hipError_t launch_short_conv(const kda_conv_args& a, hipStream_t stream) {
  return a.dtype == KDA_DTYPE_BF16 ? launch_t<__hip_bfloat16>(a, stream)
                                   : launch_t<float>(a, stream);
}

}  // namespace kda
