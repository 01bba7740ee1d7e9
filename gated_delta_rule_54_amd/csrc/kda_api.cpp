// kda_api.cpp -- the C ABI declared in include/kda.h: descriptor validation,
// workspace sizing, status strings and dispatch to the HIP launchers.
//
// Validation is host-only and never synchronises the device; on error nothing
// is launched.  The library allocates no device memory.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "kda_internal.h"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string t_last_error;

kda_status_t fail(kda_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return st;
}

kda_status_t ok() {
  t_last_error.clear();
  return KDA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

// Checks shared by both entry points: dims, dtype, chunk, scale.
kda_status_t check_common(const kda_desc_t* d) {
  if (!d) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->gate_per_head != 0 && d->gate_per_head != 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "gate_per_head must be 0 or 1");
  if (d->heads < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "heads must be >= 1 (got %d)", d->heads);
  if (d->dtype != KDA_DTYPE_F32 && d->dtype != KDA_DTYPE_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
  if (d->dk < 1 || d->dv < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "dk and dv must be positive (got %d, %d)", d->dk, d->dv);
  if (d->dk != d->dv || (d->dk != 64 && d->dk != 128))
    return fail(KDA_ERR_UNSUPPORTED, "supported head dims: dk = dv = 64 or 128 (got %d, %d)",
                d->dk, d->dv);
  if (!std::isfinite(d->scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (d->qk_l2norm != 0 && d->qk_l2norm != 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "qk_l2norm must be 0 or 1");
  return KDA_OK;
}

kda_status_t check_chunk_desc(const kda_desc_t* d) {
  kda_status_t st = check_common(d);
  if (st != KDA_OK) return st;
  if (d->chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", d->chunk);
  if (d->batch < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", d->batch);
  if (d->num_seqs < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1 (got %d)", d->num_seqs);
  if (d->seqlen < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "seqlen must be >= 0");
  if (d->seqlen > (int64_t(1) << 40))
    return fail(KDA_ERR_UNSUPPORTED, "seqlen %lld exceeds 2^40", (long long)d->seqlen);
  if (d->ckpt_every < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "ckpt_every must be >= 0");
  if (d->ckpt_every > 0) {
    if (d->ckpt_every % d->chunk != 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "ckpt_every (%lld) must be a multiple of chunk",
                  (long long)d->ckpt_every);
    if (d->seqlen % d->ckpt_every != 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "ckpt_every (%lld) must divide seqlen (%lld)",
                  (long long)d->ckpt_every, (long long)d->seqlen);
  }
  return KDA_OK;
}

}  // namespace

KDA_EXPORT const char* kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_STATUS_UNKNOWN";
}

KDA_EXPORT const char* kda_last_error(void) { return t_last_error.c_str(); }

KDA_EXPORT int kda_abi_version(void) { return KDA_ABI_VERSION; }

KDA_EXPORT size_t kda_chunk_fwd_workspace_bytes(const kda_desc_t* desc) {
  if (check_chunk_desc(desc) != KDA_OK) return 0;
  return kda::chunk_workspace_bytes(*desc);
}

namespace {
// Validation shared by kda_chunk_fwd and kda_chunk_fwd_noalloc (everything
// but the workspace).
kda_status_t check_chunk_fwd_args(const kda_desc_t* desc, const void* q, const void* k,
                                  const void* v, const float* g, const float* beta,
                                  const float* init_state, const int32_t* cu_seqlens, void* o,
                                  float* final_state, float* state_ckpt) {
  kda_status_t st = check_chunk_desc(desc);
  if (st != KDA_OK) return st;
  const kda_desc_t& d = *desc;
  if (cu_seqlens) {
    if (d.batch != 1)
      return fail(KDA_ERR_INVALID_ARGUMENT, "varlen (cu_seqlens != NULL) needs batch == 1");
    if (d.ckpt_every > 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "state checkpoints need the dense layout");
    if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)
      return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  } else if (d.num_seqs != d.batch) {
    return fail(KDA_ERR_INVALID_ARGUMENT, "dense layout needs num_seqs == batch (%d vs %d)",
                d.num_seqs, d.batch);
  }
  if ((d.ckpt_every > 0) != (state_ckpt != nullptr))
    return fail(KDA_ERR_INVALID_ARGUMENT,
                "state_ckpt must be given exactly when ckpt_every > 0");
  // q, k, v, g, o rows are moved with vector accesses (16-byte aligned rows);
  // everything else, and per-head gates, with 4-byte scalar accesses.
  const bool has_tokens = d.seqlen > 0;
  const void* need[] = {q, k, v, g, beta, o};
  const char* names[] = {"q", "k", "v", "g", "beta", "o"};
  const uintptr_t align[] = {16, 16, 16, uintptr_t(d.gate_per_head ? 4 : 16), 4, 16};
  for (int i = 0; i < 6; ++i) {
    if (has_tokens && !need[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (need[i] && !aligned(need[i], align[i]))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i],
                  (int)align[i]);
  }
  const void* opt[] = {init_state, final_state, state_ckpt};
  const char* onames[] = {"init_state", "final_state", "state_ckpt"};
  for (int i = 0; i < 3; ++i)
    if (opt[i] && !aligned(opt[i], 4))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", onames[i]);
  if (o && (o == q || o == k || o == v || o == (const void*)g || o == (const void*)beta))
    return fail(KDA_ERR_INVALID_ARGUMENT, "o must not alias an input");
  return KDA_OK;
}
}  // namespace

KDA_EXPORT kda_status_t kda_chunk_fwd(const kda_desc_t* desc, const void* q, const void* k,
                                      const void* v, const float* g, const float* beta,
                                      const float* init_state, const int32_t* cu_seqlens,
                                      void* o, float* final_state, float* state_ckpt,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  kda_status_t st = check_chunk_fwd_args(desc, q, k, v, g, beta, init_state, cu_seqlens, o,
                                         final_state, state_ckpt);
  if (st != KDA_OK) return st;
  const kda_desc_t& d = *desc;
  if (workspace && !aligned(workspace, 16))
    return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
  const size_t need_ws = kda::chunk_workspace_bytes(d);
  if (need_ws > 0 && (!workspace || workspace_bytes < need_ws))
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu%s", need_ws,
                workspace_bytes, workspace ? "" : " (NULL)");
  hipError_t e = kda::launch_chunk_fwd(d, q, k, v, g, beta, init_state, cu_seqlens, o,
                                       final_state, state_ckpt, nullptr, workspace, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_chunk_fwd launch: %s", hipGetErrorString(e));
  return ok();
}

KDA_EXPORT kda_status_t kda_chunk_fwd_conv(const kda_desc_t* desc, const void* xq,
                                           const void* xk, const void* xv,
                                           const float* const* conv_w,
                                           const float* const* conv_bias,
                                           const float* const* conv_state_in,
                                           float* const* conv_state_out, const float* g,
                                           const float* beta, const float* init_state,
                                           const int32_t* cu_seqlens, void* o,
                                           float* final_state, float* state_ckpt,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  kda_status_t st = check_chunk_fwd_args(desc, xq, xk, xv, g, beta, init_state, cu_seqlens, o,
                                         final_state, state_ckpt);
  if (st != KDA_OK) return st;
  const kda_desc_t& d = *desc;
  static const char* names[3] = {"q", "k", "v"};
  const float* w[3] = {nullptr, nullptr, nullptr};
  const float* bias[3] = {nullptr, nullptr, nullptr};
  const float* sin[3] = {nullptr, nullptr, nullptr};
  float* sout[3] = {nullptr, nullptr, nullptr};
  if (!conv_w) return fail(KDA_ERR_INVALID_ARGUMENT, "conv_w is NULL");
  const size_t state_bytes = (size_t)d.num_seqs * d.heads * d.dk * 3 * sizeof(float);
  for (int t = 0; t < 3; ++t) {
    w[t] = conv_w[t];
    bias[t] = conv_bias ? conv_bias[t] : nullptr;
    sin[t] = conv_state_in ? conv_state_in[t] : nullptr;
    sout[t] = conv_state_out ? conv_state_out[t] : nullptr;
    if (!w[t]) return fail(KDA_ERR_INVALID_ARGUMENT, "conv_w[%d] (%s) is NULL", t, names[t]);
    if (!aligned(w[t], 16))
      return fail(KDA_ERR_INVALID_ARGUMENT, "conv_w[%d] (%s) is not 16-byte aligned", t, names[t]);
    const void* al[3] = {bias[t], sin[t], sout[t]};
    const char* an[3] = {"conv_bias", "conv_state_in", "conv_state_out"};
    for (int i = 0; i < 3; ++i)
      if (al[i] && !aligned(al[i], 4))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s[%d] (%s) is not 4-byte aligned", an[i], t,
                    names[t]);
    if (sin[t] && sout[t] && (const void*)sout[t] != (const void*)sin[t]) {
      const char* a = reinterpret_cast<const char*>(sin[t]);
      const char* b = reinterpret_cast<const char*>(sout[t]);
      if (a < b + state_bytes && b < a + state_bytes)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "conv_state_out[%d] (%s) overlaps conv_state_in[%d] without being it", t,
                    names[t], t);
    }
  }
  if (workspace && !aligned(workspace, 16))
    return fail(KDA_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
  const size_t need_ws = kda::chunk_workspace_bytes(d);
  if (need_ws > 0 && (!workspace || workspace_bytes < need_ws))
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu%s", need_ws,
                workspace_bytes, workspace ? "" : " (NULL)");
  const void* x[3] = {xq, xk, xv};
  hipError_t e = kda::launch_chunk_fwd_conv(d, x, w, bias, sin, sout, g, beta, init_state,
                                            cu_seqlens, o, final_state, state_ckpt, workspace,
                                            stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_chunk_fwd_conv launch: %s", hipGetErrorString(e));
  return ok();
}

KDA_EXPORT kda_status_t kda_chunk_fwd_noalloc(const kda_desc_t* desc, const void* q,
                                              const void* k, const void* v, const float* g,
                                              const float* beta, const float* init_state,
                                              const int32_t* cu_seqlens, void* o,
                                              float* final_state, float* state_ckpt,
                                              hipStream_t stream) {
  kda_status_t st = check_chunk_fwd_args(desc, q, k, v, g, beta, init_state, cu_seqlens, o,
                                         final_state, state_ckpt);
  if (st != KDA_OK) return st;
  const kda_desc_t& d = *desc;
  if (kda::noalloc_seg_slots(d) == 0)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                "kda_chunk_fwd_noalloc holds %zu bytes of scratch per device; this descriptor "
                "needs at least %lld (%d sequences x %d heads of carried states plus one "
                "8-chunk segment of records): use kda_chunk_fwd with a workspace",
                (size_t)KDA_NOALLOC_SCRATCH_BYTES, (long long)kda::noalloc_min_bytes(d),
                d.num_seqs, d.heads);
  hipError_t e = kda::launch_chunk_fwd_noalloc(d, q, k, v, g, beta, init_state, cu_seqlens, o,
                                               final_state, state_ckpt, stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_chunk_fwd_noalloc launch: %s", hipGetErrorString(e));
  return ok();
}

namespace {
// Backward support: the forward's shapes, except fp32 operands at d = 128.
kda_status_t check_bwd_desc(const kda_desc_t* d) {
  kda_status_t st = check_chunk_desc(d);
  if (st != KDA_OK) return st;
  if (d->dtype == KDA_DTYPE_F32 && d->dk == 128)
    return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_bwd: fp32 operands need dk = dv = 64");
  return KDA_OK;
}
}  // namespace

KDA_EXPORT size_t kda_chunk_bwd_workspace_bytes(const kda_desc_t* desc) {
  if (check_bwd_desc(desc) != KDA_OK) return 0;
  return kda::chunk_bwd_workspace_bytes(*desc);
}

KDA_EXPORT kda_status_t kda_chunk_bwd(const kda_desc_t* desc, const void* q, const void* k,
                                      const void* v, const float* g, const float* beta,
                                      const float* init_state, const int32_t* cu_seqlens,
                                      const void* d_o, const float* d_final_state, void* dq,
                                      void* dk, void* dv, float* dg, float* dbeta,
                                      float* d_init_state, uint32_t* range_flag,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  kda_status_t st = check_bwd_desc(desc);
  if (st != KDA_OK) return st;
  const kda_desc_t& d = *desc;
  if (cu_seqlens) {
    if (d.batch != 1)
      return fail(KDA_ERR_INVALID_ARGUMENT, "varlen (cu_seqlens != NULL) needs batch == 1");
    if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)
      return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  } else if (d.num_seqs != d.batch) {
    return fail(KDA_ERR_INVALID_ARGUMENT, "dense layout needs num_seqs == batch (%d vs %d)",
                d.num_seqs, d.batch);
  }
  const bool has_tokens = d.seqlen > 0;
  const void* need[] = {q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta};
  const char* names[] = {"q", "k", "v", "g", "beta", "d_o", "dq", "dk", "dv", "dg", "dbeta"};
  const uintptr_t align[] = {16, 16, 16, uintptr_t(d.gate_per_head ? 4 : 16), 4, 16,
                             16, 16, 16, 4, 4};
  for (int i = 0; i < 11; ++i) {
    if (has_tokens && !need[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (need[i] && !aligned(need[i], align[i]))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i],
                  (int)align[i]);
  }
  const void* opt[] = {init_state, d_final_state, d_init_state, range_flag, workspace};
  const char* onames[] = {"init_state", "d_final_state", "d_init_state", "range_flag",
                          "workspace"};
  const uintptr_t oalign[] = {4, 4, 4, 4, 16};
  for (int i = 0; i < 5; ++i)
    if (opt[i] && !aligned(opt[i], oalign[i]))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", onames[i],
                  (int)oalign[i]);
  // outputs never alias an input
  const void* ins[] = {q, k, v, g, beta, init_state, d_o, d_final_state};
  const void* outs[] = {dq, dk, dv, dg, dbeta, d_init_state};
  for (const void* o : outs)
    for (const void* in : ins)
      if (o && o == in) return fail(KDA_ERR_INVALID_ARGUMENT, "gradients must not alias inputs");
  if (range_flag)
    for (const void* o : outs)
      if (o == range_flag)
        return fail(KDA_ERR_INVALID_ARGUMENT, "range_flag must not alias a gradient");
  const size_t need_ws = kda::chunk_bwd_workspace_bytes(d);
  if (!workspace || workspace_bytes < need_ws)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu%s", need_ws,
                workspace_bytes, workspace ? "" : " (NULL)");
  hipError_t e = kda::launch_chunk_bwd(d, q, k, v, g, beta, init_state, cu_seqlens, d_o,
                                       d_final_state, dq, dk, dv, dg, dbeta, d_init_state,
                                       range_flag, workspace, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_chunk_bwd launch: %s", hipGetErrorString(e));
  return ok();
}

KDA_EXPORT kda_status_t kda_decode_step(const kda_desc_t* desc, const void* q, const void* k,
                                        const void* v, const float* g, const float* beta,
                                        float* state, void* o, hipStream_t stream) {
  kda_status_t st = check_common(desc);
  if (st != KDA_OK) return st;
  const kda_desc_t& d = *desc;
  if (d.num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if ((int64_t)d.num_seqs * d.heads > 0x7fffffffLL)
    return fail(KDA_ERR_UNSUPPORTED, "num_seqs * heads exceeds 2^31 - 1");
  if (d.num_seqs == 0) return ok();
  // The state is moved with 16-byte vector accesses, the rest element-wise.
  const uintptr_t el = d.dtype == KDA_DTYPE_BF16 ? 2 : 4;
  const void* need[] = {q, k, v, g, beta, state, o};
  const char* names[] = {"q", "k", "v", "g", "beta", "state", "o"};
  const uintptr_t align[] = {el, el, el, 4, 4, 16, el};
  for (int i = 0; i < 7; ++i) {
    if (!need[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned(need[i], align[i]))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i],
                  (int)align[i]);
  }
  if (o == q || o == k || o == v || o == (const void*)g || o == (const void*)beta ||
      o == (const void*)state)
    return fail(KDA_ERR_INVALID_ARGUMENT, "o must not alias an input or the state");
  hipError_t e = kda::launch_decode(d, q, k, v, g, beta, state, o, stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_decode_step launch: %s", hipGetErrorString(e));
  return ok();
}

KDA_EXPORT kda_status_t kda_output_gate_norm(int64_t rows, int32_t dv, int32_t dtype,
                                             const void* o, const void* z, const float* w,
                                             float eps, void* y, hipStream_t stream) {
  if (rows < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
  if (dv != 64 && dv != 128) return fail(KDA_ERR_UNSUPPORTED, "dv must be 64 or 128 (got %d)", dv);
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (rows == 0) return ok();
  const void* need[] = {o, z, y};
  const char* names[] = {"o", "z", "y"};
  for (int i = 0; i < 3; ++i) {
    if (!need[i]) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(need[i]))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (w && !aligned(w, 4)) return fail(KDA_ERR_INVALID_ARGUMENT, "w is not 4-byte aligned");
  const uintptr_t bytes = (uintptr_t)rows * dv * (dtype == KDA_DTYPE_BF16 ? 2 : 4);
  auto overlap = [&](const void* a, const void* b) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + bytes && pb < pa + bytes;
  };
  if (overlap(y, z)) return fail(KDA_ERR_INVALID_ARGUMENT, "y must not overlap z");
  if (y != o && overlap(y, o))
    return fail(KDA_ERR_INVALID_ARGUMENT, "y must equal o or not overlap it");
  hipError_t e = kda::launch_gate_norm(rows, dv, dtype, o, z, w, eps, y, stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_output_gate_norm launch: %s", hipGetErrorString(e));
  return ok();
}

KDA_EXPORT kda_status_t kda_short_conv_swish(int32_t batch, int64_t seqlen, int32_t num_seqs,
                                             int32_t channels, int32_t width, int32_t dtype,
                                             const void* x, const float* w, const float* bias,
                                             const float* state_in, const int32_t* cu_seqlens,
                                             void* y, float* state_out, hipStream_t stream) {
  if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
  if (width < 1 || width > 4)
    return fail(KDA_ERR_UNSUPPORTED, "width must be 1 ... 4 (got %d)", width);
  const int el = dtype == KDA_DTYPE_BF16 ? 2 : 4;
  if (channels < 1 || channels % (16 / el) != 0)
    return fail(KDA_ERR_UNSUPPORTED, "channels must be a positive multiple of %d (got %d)",
                16 / el, channels);
  if ((int64_t)channels * el > KDA_CONV_MAX_ROW_BYTES)
    return fail(KDA_ERR_UNSUPPORTED, "channels must be at most %d at this dtype (got %d)",
                (int)(KDA_CONV_MAX_ROW_BYTES / el), channels);
  if (batch < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", batch);
  if (seqlen < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "seqlen must be >= 0");
  if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (cu_seqlens) {
    if (batch != 1)
      return fail(KDA_ERR_INVALID_ARGUMENT, "varlen (cu_seqlens != NULL) needs batch == 1");
    if (!aligned(cu_seqlens, 4))
      return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  } else if (num_seqs != batch) {
    return fail(KDA_ERR_INVALID_ARGUMENT, "dense layout needs num_seqs == batch (%d vs %d)",
                num_seqs, batch);
  }
  if ((double)batch * (double)seqlen * channels > 9.0e18)
    return fail(KDA_ERR_UNSUPPORTED, "tensor too large");
  if (!w) return fail(KDA_ERR_INVALID_ARGUMENT, "w is NULL");
  if (width == 4 && !aligned16(w))
    return fail(KDA_ERR_INVALID_ARGUMENT, "w must be 16-byte aligned for width 4");
  const void* p4[] = {w, bias, state_in, state_out};
  const char* n4[] = {"w", "bias", "state_in", "state_out"};
  for (int i = 0; i < 4; ++i)
    if (p4[i] && !aligned(p4[i], 4))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", n4[i]);
  const bool has_tokens = seqlen > 0;
  if (has_tokens) {
    if (!x || !y) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", x ? "y" : "x");
    if (!aligned16(x) || !aligned16(y))
      return fail(KDA_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned");
    const uintptr_t bytes = (uintptr_t)batch * (uintptr_t)seqlen * channels * el;
    const uintptr_t px = reinterpret_cast<uintptr_t>(x), py = reinterpret_cast<uintptr_t>(y);
    if (px < py + bytes && py < px + bytes)
      return fail(KDA_ERR_INVALID_ARGUMENT, "y must not overlap x");
  }
  if (state_in && state_out && width > 1) {
    const uintptr_t sb = (uintptr_t)num_seqs * channels * (width - 1) * 4;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(state_in);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(state_out);
    const bool same = pa == pb;
    const bool in_place_ok = cu_seqlens == nullptr && seqlen <= kda::kConvInPlaceMaxTokens;
    if (same ? !in_place_ok : (pa < pb + sb && pb < pa + sb))
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "state_out may equal state_in only in the dense layout with seqlen <= %d, "
                  "and must not otherwise overlap it",
                  (int)kda::kConvInPlaceMaxTokens);
  }
  if (num_seqs == 0 || (channels == 0)) return ok();
  const kda::kda_conv_args a{batch, seqlen, num_seqs, channels, width, dtype, x, w, bias,
                             state_in, cu_seqlens, y, width > 1 ? state_out : nullptr};
  hipError_t e = kda::launch_short_conv(a, stream);
  if (e != hipSuccess)
    return fail(KDA_ERR_HIP, "kda_short_conv_swish launch: %s", hipGetErrorString(e));
  return ok();
}
