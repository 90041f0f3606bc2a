// fa_api.cpp -- the C ABI declared in include/fa.h: host-side argument checks,
// workspace sizing and dispatch to the kernel launchers.  Nothing here touches
// the GPU before every argument has been checked.
#include "../../include/fa.h"

#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fa_kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// A required buffer: non-NULL and 16-byte aligned.
bool present(const void* p) { return p != nullptr && aligned16(p); }

constexpr int kMaxLen = 1 << 29;  // longest query or key sequence (keeps i + offset +- window in int)

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// The raw value of an enum argument.  A C caller may pass any int; reading an
// out-of-range value through the C++ enum type is undefined, so every enum the
// ABI receives is read as an int first and only then compared.
static_assert(sizeof(fa_dtype_t) == sizeof(int) && sizeof(fa_status_t) == sizeof(int), "enums are ints");
template <typename E>
int raw(const E& e) {
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

thread_local hipEvent_t* g_events = nullptr;
thread_local int g_nevents = 0;

// Checks an extended problem; on FA_OK fills the kernel-side description and
// the number of query rows and key rows (over all heads).
fa_status_t check(const fa_params_t* p, fa::Problem* pb, long long* qrows, long long* krows) {
  if (p == nullptr) return FA_ERR_INVALID_ARG;
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 0 || p->Sq < 0 || p->Skv < 0 || p->D < 0) return FA_ERR_INVALID_ARG;
  const int dt = raw(p->dtype);
  if (dt != FA_F32 && dt != FA_F16 && dt != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!isfinite(p->scale)) return FA_ERR_INVALID_ARG;
  if (p->alibi_slopes != nullptr && !aligned4(p->alibi_slopes)) return FA_ERR_INVALID_ARG;
  const bool packed = p->cu_seqlens_q != nullptr || p->cu_seqlens_k != nullptr;
  if (packed) {
    if (p->cu_seqlens_q == nullptr || p->cu_seqlens_k == nullptr) return FA_ERR_INVALID_ARG;
    if (!aligned4(p->cu_seqlens_q) || !aligned4(p->cu_seqlens_k)) return FA_ERR_INVALID_ARG;
    if (p->total_q < 0 || p->total_k < 0) return FA_ERR_INVALID_ARG;
    *qrows = (long long)p->Hq * p->total_q;
    *krows = (long long)p->Hkv * p->total_k;
  } else {
    *qrows = (long long)p->B * p->Hq * p->Sq;
    *krows = (long long)p->B * p->Hkv * p->Skv;
  }
  if (*qrows == 0 && *krows == 0) {
    if (p->Hkv > 0 && p->Hq > 0 && p->Hq % p->Hkv != 0) return FA_ERR_INVALID_ARG;
  } else {
    if (p->B == 0 || p->Hq == 0 || p->Hkv == 0 || p->Hq % p->Hkv != 0) return FA_ERR_INVALID_ARG;
    if (p->D != 64 && p->D != 128) return FA_ERR_UNSUPPORTED;
    if (!(p->scale > 0.f)) return FA_ERR_UNSUPPORTED;
    // the kernels index rows and workgroups with 32-bit ints
    if (p->Sq > kMaxLen || p->Skv > kMaxLen) return FA_ERR_UNSUPPORTED;
    if ((long long)(p->Sq / 128 + 1) * p->B * p->Hq > INT_MAX ||
        (long long)(p->Skv / 128 + 1) * p->B * p->Hkv > INT_MAX)
      return FA_ERR_UNSUPPORTED;
  }
  // a window of Skv or more keys hides nothing (i + offset - window < 0 for
  // every query), so it is the same problem without a window
  const int window = (p->window < 0 || p->window >= p->Skv) ? -1 : p->window;
  *pb = fa::Problem{p->B,       p->Hq,  p->Hkv, p->Sq, p->Skv, p->causal ? 1 : 0, window,
                    packed ? p->cu_seqlens_q : nullptr, packed ? p->cu_seqlens_k : nullptr,
                    packed ? p->total_q : 0, packed ? p->total_k : 0, p->alibi_slopes};
  return FA_OK;
}

// The backward's buffers: those of a side with rows must be present.
bool bwd_buffers_ok(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                    const void* dq, const void* dk, const void* dv, long long qrows, long long krows) {
  if (qrows > 0 && (!present(q) || !present(o) || !present(lse) || !present(dO) || !present(dq))) return false;
  if (krows > 0 && (!present(k) || !present(v) || !present(dk) || !present(dv))) return false;
  return true;
}

// Split-KV plan: nsplit key ranges of `chunk` keys (whole split-kernel tiles).
// With no request, enough ranges to give the GPU about kSplitTarget
// workgroups, keeping at least two tiles per range: one round of one
// workgroup per CU (the split kernel's LDS holds one).  Measured on 16
// sequences x 8 KV heads x 8192 keys: 2 ranges (256 workgroups) 6 % faster
// than 4 (512), and 8 slower still.
constexpr long long kSplitTarget = fa::kCUs;
struct SplitPlan {
  int nsplit, chunk;
};
SplitPlan plan_split(const fa_params_t* p, int requested) {
  const int bc = fa::split_tile_keys(p->dtype);
  const int ntile = p->Skv > 0 ? (p->Skv + bc - 1) / bc : 1;
  int ns = requested;
  if (ns <= 0) {
    const long long units = (long long)p->B * p->Hkv;
    const long long want = units > 0 ? (kSplitTarget + units - 1) / units : 1;
    ns = (int)(want < ntile / 2 ? want : ntile / 2);
    if (ns < 1) ns = 1;
  }
  if (ns > ntile) ns = ntile;
  const int per = (ntile + ns - 1) / ns;  // tiles per range
  return SplitPlan{(ntile + per - 1) / per, per * bc};
}

long long split_work_floats(const fa_params_t* p, const SplitPlan& sp, long long qrows) {
  return (long long)sp.nsplit * qrows * (p->D + 1);
}

fa_params_t dense(int B, int Hq, int Hkv, int S, int D, float scale, int causal, fa_dtype_t dtype) {
  fa_params_t p{};
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = S;
  p.Skv = S;
  p.D = D;
  p.scale = scale;
  p.causal = causal;
  p.window = -1;
  memcpy(&p.dtype, &dtype, sizeof p.dtype);  // checked later as a raw value
  return p;
}

}  // namespace

extern "C" {

void fa_profile_events(hipEvent_t* events, int n) {
  g_events = (events != nullptr && n > 0) ? events : nullptr;
  g_nevents = g_events ? n : 0;
}

const char* fa_status_string(fa_status_t s) {
  switch (raw(s)) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, const fa_params_t* p,
                      hipStream_t stream) {
  fa::Problem pb;
  long long qrows = 0, krows = 0;
  fa_status_t st = check(p, &pb, &qrows, &krows);
  if (st != FA_OK || qrows == 0) return st;
  if (!present(q) || !present(o) || (lse && !aligned16(lse))) return FA_ERR_INVALID_ARG;
  if (krows > 0 && (!present(k) || !present(v))) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, pb, p->D, p->scale, (int)p->dtype, g_events, g_nevents};
  return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_ex_workspace_bytes(const fa_params_t* p) {
  fa::Problem pb;
  long long qrows = 0, krows = 0;
  if (check(p, &pb, &qrows, &krows) != FA_OK) return 0;
  return qrows > 0 ? round256((size_t)qrows * sizeof(float)) : 0;
}

fa_status_t fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                      void* dq, void* dk, void* dv, const fa_params_t* p, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  fa::Problem pb;
  long long qrows = 0, krows = 0;
  fa_status_t st = check(p, &pb, &qrows, &krows);
  if (st != FA_OK || (qrows == 0 && krows == 0)) return st;
  if (!bwd_buffers_ok(q, k, v, o, lse, dO, dq, dk, dv, qrows, krows)) return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_ex_workspace_bytes(p);
  if (need > 0 && (!workspace || !aligned16(workspace))) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, static_cast<float*>(workspace), pb, p->D, p->scale,
                (int)p->dtype, g_events, g_nevents};
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_splitkv_workspace_bytes(const fa_params_t* p, int num_splits) {
  fa::Problem pb;
  long long qrows = 0, krows = 0;
  if (check(p, &pb, &qrows, &krows) != FA_OK || qrows == 0) return 0;
  if ((long long)(p->Hq / p->Hkv) * p->Sq > 32 || p->alibi_slopes != nullptr) return 0;
  return round256((size_t)split_work_floats(p, plan_split(p, num_splits), qrows) * sizeof(float));
}

fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, const fa_params_t* p,
                           int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::Problem pb;
  long long qrows = 0, krows = 0;
  fa_status_t st = check(p, &pb, &qrows, &krows);
  if (st != FA_OK || qrows == 0) return st;
  // the query rows of one KV group form one 32-column matrix block
  if ((long long)(p->Hq / p->Hkv) * p->Sq > 32) return FA_ERR_UNSUPPORTED;
  if (p->alibi_slopes != nullptr) return FA_ERR_UNSUPPORTED;  // no position bias in the split kernels
  if (!present(q) || !present(o) || (lse && !aligned16(lse))) return FA_ERR_INVALID_ARG;
  if (krows > 0 && (!present(k) || !present(v))) return FA_ERR_INVALID_ARG;
  if (!present(workspace)) return FA_ERR_INVALID_ARG;
  const SplitPlan sp = plan_split(p, num_splits);
  if (workspace_bytes < (size_t)split_work_floats(p, sp, qrows) * sizeof(float)) return FA_ERR_WORKSPACE;
  fa::SplitArgs a{q,        k,        v,         o,     lse,   static_cast<float*>(workspace),
                  pb,       p->D,     p->scale,  (int)p->dtype, sp.nsplit, sp.chunk,
                  qrows,    g_events, g_nevents};
  return fa::launch_splitkv(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int S,
                   int D, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  const fa_params_t p = dense(B, Hq, Hkv, S, D, scale, causal, dtype);
  return fa_fwd_ex(q, k, v, o, lse, &p, stream);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
  const fa_params_t p = dense(B, Hq, Hkv, S, D, 1.0f, 1, FA_BF16);
  return fa_bwd_ex_workspace_bytes(&p);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                   fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fa_params_t p = dense(B, Hq, Hkv, S, D, scale, causal, dtype);
  return fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, &p, workspace, workspace_bytes, stream);
}

fa_status_t fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D,
                           float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  const fa_params_t p = dense(B, Hq, Hkv, S, D, scale, causal, dtype);
  fa::Problem pb;
  long long qrows = 0, krows = 0;
  fa_status_t st = check(&p, &pb, &qrows, &krows);
  if (st != FA_OK || (qrows == 0 && krows == 0)) return st;
  if (!bwd_buffers_ok(q, k, v, o, lse, dO, dq, dk, dv, qrows, krows)) return FA_ERR_INVALID_ARG;
  if (qrows > FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_WORKSPACE;
  static_assert(FA_BWD_NOALLOC_MAX_ROWS == fa::kNoAllocRows, "one size for the static array");
  // the array's address is per device: the stream must run on the current one
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
  if (cur != sdev) return FA_ERR_INVALID_ARG;
  float* rowdot = nullptr;
  if (fa::noalloc_rowdot(&rowdot) != hipSuccess) return FA_ERR_HIP;
  fa::BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, rowdot, pb, D, scale, (int)dtype, g_events, g_nevents};
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
