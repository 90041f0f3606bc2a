// fa_seq.hpp -- device-side view of a Problem: where a sequence's rows live,
// which work item a workgroup takes, which keys a query sees.  Included by the
// kernels only.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_problem.hpp"

namespace fa {

// One (batch, query head, KV head) sequence.  Rows of its queries are
// q_row0 .. q_row0 + sq - 1 of the [rows][D] view of q (and of o, dq, lse, the
// row-dot workspace); its keys are kv_row0 .. kv_row0 + skv - 1 of k (v, dk, dv).
struct Seq {
  size_t q_row0, kv_row0;
  int sq, skv, off;
};

// Packed offsets are clamped into [0, T] and lengths to the stated maxima, so
// malformed offsets can make results wrong but never move an access out of
// the buffers the caller described.
__device__ inline Seq seq_of(const Problem& p, int b, int hq, int hkv) {
  Seq s;
  if (p.cu_q != nullptr) {
    const int q0 = min(max(p.cu_q[b], 0), p.Tq);
    const int q1 = min(max(p.cu_q[b + 1], q0), p.Tq);
    const int k0 = min(max(p.cu_k[b], 0), p.Tk);
    const int k1 = min(max(p.cu_k[b + 1], k0), p.Tk);
    s.sq = min(q1 - q0, p.Sq);
    s.skv = min(k1 - k0, p.Skv);
    s.q_row0 = (size_t)hq * p.Tq + q0;
    s.kv_row0 = (size_t)hkv * p.Tk + k0;
  } else {
    s.sq = p.Sq;
    s.skv = p.Skv;
    s.q_row0 = ((size_t)b * p.Hq + hq) * p.Sq;
    s.kv_row0 = ((size_t)b * p.Hkv + hkv) * p.Skv;
  }
  s.off = s.skv - s.sq;
  return s;
}

// Distance in rows between the first query rows of heads hq and hq + 1 of
// one sequence (the query layouts' head stride).
__device__ inline size_t q_head_stride(const Problem& p) { return p.cu_q != nullptr ? (size_t)p.Tq : (size_t)p.Sq; }

// Work item of a kernel over query tiles: KV group major, then query tile
// (heaviest first when causal), then the group's query heads.  The G heads
// that read the same K/V rows run side by side and share them in L2.
struct QTile {
  int b, hq, qt;
};
template <bool CAUSAL>
__device__ inline QTile qtile_of(int work, int nqt, const Problem& p) {
  const int G = p.Hq / p.Hkv;
  const int rest = work / G;
  const int t = rest % nqt;
  const int bk = rest / nqt;
  const int b = bk / p.Hkv;
  return {b, (bk - b * p.Hkv) * G + (work - rest * G), CAUSAL ? nqt - 1 - t : t};
}

// Visibility of key j to query i (both relative to their sequence); the mask
// kinds are compile-time so the common causal-only path carries no window.
template <bool CAUSAL, bool WINDOW>
__device__ inline bool key_visible(const Problem& p, const Seq& s, int i, int j) {
  return j < s.skv && (!CAUSAL || j <= i + s.off) && (!WINDOW || j >= i + s.off - p.window);
}

}  // namespace fa
