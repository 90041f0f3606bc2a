// fa_api.cpp -- the C ABI declared in include/fa.h: host-side argument checks,
// workspace sizing and dispatch to the kernel launchers.  Nothing here touches
// the GPU before every argument has been checked.
#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_kernels.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape / scalar checks of fa_fwd and fa_bwd.  Returns FA_OK and sets
// *empty when there is nothing to compute.
fa_status_t check_problem(int B, int Hq, int Hkv, int S, int D, float scale, fa_dtype_t dtype, bool* empty) {
  *empty = false;
  if (B < 0 || Hq < 0 || Hkv < 0 || S < 0 || D < 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if ((long long)B * Hq * S == 0) {
    if (Hkv > 0 && Hq > 0 && Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    *empty = true;
    return FA_OK;
  }
  if (Hkv == 0 || Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

thread_local hipEvent_t* g_events = nullptr;
thread_local int g_nevents = 0;

}  // namespace

extern "C" {

void fa_profile_events(hipEvent_t* events, int n) {
  g_events = (events != nullptr && n > 0) ? events : nullptr;
  g_nevents = g_events ? n : 0;
}

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int S,
                   int D, float scale, int causal, fa_dtype_t dtype, hipStream_t stream) {
  bool empty = false;
  fa_status_t st = check_problem(B, Hq, Hkv, S, D, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, S, D, scale, causal ? 1 : 0, (int)dtype, g_events, g_nevents};
  return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
  bool empty = false;
  if (check_problem(B, Hq, Hkv, S, D, 1.0f, FA_BF16, &empty) != FA_OK || empty) return 0;
  return round256((size_t)B * Hq * S * sizeof(float));
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int S, int D, float scale, int causal,
                   fa_dtype_t dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  fa_status_t st = check_problem(B, Hq, Hkv, S, D, scale, dtype, &empty);
  if (st != FA_OK || empty) return st;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, Hq, Hkv, S, D)) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, static_cast<float*>(workspace),
                B, Hq, Hkv, S, D, scale, causal ? 1 : 0, (int)dtype, g_events, g_nevents};
  return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
