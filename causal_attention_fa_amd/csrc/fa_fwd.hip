// fa_fwd.hip -- forward pass: O = softmax(mask(scale * Q K^T)) V and L = logsumexp,
// by online softmax over KV tiles (gfx950, wave64, 32x32 MFMA).
//
// Method: "Phase 14: Flash Attention 2 for SM120 — Design Document", section
// "FA2 算法" (Q tile outer, loaded once; KV tiles inner; running max / sum with
// rescale by exp(m - m_new)); section "Causal Mask" (tiles wholly after the
// diagonal are skipped, the rest masked per element); section "GQA 支持"
// (KV head = query head / group size, indexed in the kernel).  L = m + log l is
// the forward's saved state ("Phase T14: 融合 Flash-Attention Kernel — Design
// Document", section "什么是 flash-attention" and decision ②).
//
// Work decomposition (MI355X-specific, not the pages'):
//   * one workgroup = NW waves = one tile of 32*NW query rows of one (b, head);
//   * each wave owns 32 query rows.  It computes S^T = K Q^T so that one query
//     row sits in one lane pair: the softmax max is a register max plus one
//     cross-half exchange, the rescale factor is a per-lane scalar, and the
//     probabilities P^T come out of the accumulators already laid out as the B
//     operand of O^T += V^T P^T (no LDS round trip for P);
//   * Q stays in registers (B operand of S^T) for the whole kernel;
//   * K and V tiles are staged row-major (XOR-swizzled) in LDS, double
//     buffered: the next tile's direct global->LDS loads are issued before the
//     current tile's math; V^T fragments come from gfx950's LDS transpose read;
//   * softmax in base 2: p = exp2(s * scale*log2e - m), m tracked in that unit,
//     and the accumulator is rescaled only when a row's max grows by > 2^4;
//   * the row sum l is one more MFMA per step (all-ones A operand), so it sums
//     exactly the rounded P that multiplies V;
//   * causal: workgroups are launched heaviest (last query tiles) first, a wave
//     skips KV tiles that lie wholly after its rows, and the element mask is
//     applied on diagonal tiles only;
//   * each XCD takes a contiguous run of heads, so the query heads of a KV
//     group stream that group's K/V through one L2.
#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Lazy rescale threshold (log2 units): the running reference m only moves
// when some row's maximum grows by more than this, so p <= 2^kRescaleLog2.
// The row sum l is taken from the same dtype-rounded P that multiplies V, so
// O = sum(P~ V) / sum(P~) stays a consistent weighted average: with that, a
// threshold of 2^4 keeps the bf16 error of eager rescaling (measured on the
// long-context workload), while 2^8 with an unrounded l does not.
constexpr float kRescaleLog2 = 4.f;

template <typename T, int HD, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (sizeof(T) == 2 ? 2 : 1)) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, int Hq, int Hkv, int S, float c, int nqt) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  using Tile = RowTile<T, BC, HD>;
  constexpr int kBuf = 2 * Tile::kElems;  // K tile, then V tile
  __shared__ __attribute__((aligned(16))) T lds[2 * kBuf];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h = lane >> 5;
  // work item: (b*Hq + hq) major, query tiles heaviest first within a head;
  // one XCD takes a contiguous run of heads (a KV group for GQA)
  const int work = xcd_slice(blockIdx.x, gridDim.x);
  const int bh = work / nqt;
  const int qt = CAUSAL ? (nqt - 1 - (work - bh * nqt)) : (work - bh * nqt);
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hkv = hq / (Hq / Hkv);
  const T* Qh = Q + (size_t)bh * S * HD;
  const T* Kh = K + ((size_t)b * Hkv + hkv) * S * HD;
  const T* Vh = V + ((size_t)b * Hkv + hkv) * S * HD;
  const int i0 = qt * BR;
  const int qw0 = i0 + 32 * w;
  const int myq = qw0 + r;

  // rows past the end read row S-1: their results are never stored
  vec8<T> qf[HD / 16];
  const T* qrow = Qh + (size_t)min(myq, S - 1) * HD + 8 * h;
#pragma unroll
  for (int t = 0; t < HD / 16; ++t) qf[t] = load8<T>(qrow + 16 * t);

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d) oacc[d] = f32x16{};
  // Row sums on the matrix cores: an all-ones A operand turns O^T += V^T P^T
  // into lacc += 1 P^T, whose every register holds sum_kv P~[kv][q] for the
  // lane's query q (the full sum, both lane halves included).
  f32x16 lacc = f32x16{};
  vec8<T> ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = to_elem<T>(1.f);
  float m = -INFINITY;

  const int kv_end = CAUSAL ? min(S, i0 + BR) : S;
  const int ntiles = (kv_end + BC - 1) / BC;

  TileLoader<T, BC, HD, NT> kld, vld;
  kld.init(tid);
  vld.init(tid);
  kld.issue(Kh, 0, S, lds, tid);
  vld.issue(Vh, 0, S, lds + Tile::kElems, tid);
  kld.land(tid);
  vld.land(tid);
  __syncthreads();

  for (int jt = 0; jt < ntiles; ++jt) {
    const int j0 = jt * BC;
    const bool more = jt + 1 < ntiles;
    if (more) {  // the other buffer was last read before the previous barrier
      T* nb = lds + ((jt + 1) & 1) * kBuf;
      kld.issue(Kh, j0 + BC, S, nb, tid);
      vld.issue(Vh, j0 + BC, S, nb + Tile::kElems, tid);
    }
    const T* Ks = lds + (jt & 1) * kBuf;
    const T* Vs = Ks + Tile::kElems;
    const bool active = !CAUSAL || j0 <= qw0 + 31;
    if (active) {
      // S^T (BC x 32) = K_tile Q_w^T
      f32x16 s[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < HD / 16; ++t) s[kb] = mma<T>(Tile::frag(Ks, 32 * kb + r, 16 * t, h), qf[t], s[kb]);
      }
      // keys after the query (causal) or past the end (last tile) get -inf
      const bool edge = CAUSAL ? (j0 + BC - 1 > qw0) : (j0 + BC > S);
      if (edge) {
        const int lim = CAUSAL ? myq : S - 1;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kv = j0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
            s[kb][i] = kv > lim ? -INFINITY : s[kb][i];
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = wave_xor32_max(mx) * c;
      // Move the reference only when a row's max outgrows it by 2^8 (any lane:
      // the branch is wave-uniform).  O = acc / l is exact for any reference.
      if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        lacc *= alpha;
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) oacc[d] *= alpha;
        m = m_new;
      }
      const float ref = (m == -INFINITY) ? 0.f : m;  // a row with no key yet keeps p = 0
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -ref));
      // O^T (HD x 32) += V_tile^T P^T ; l += 1^T P^T
#pragma unroll
      for (int kt = 0; kt < BC / 16; ++kt) {
        const vec8<T> pf = acc_to_frag<T>(s[kt >> 1], 8 * (kt & 1));
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) oacc[d] = mma<T>(Tile::tr_frag(Vs, kt, 32 * d, lane), pf, oacc[d]);
        lacc = mma<T>(ones, pf, lacc);
      }
    }
    if (more) {
      kld.land(tid);
      vld.land(tid);
    }
    __syncthreads();
  }

  const float l = lacc[0];
  if (myq < S) {
    const float inv = 1.f / l;
    T* Or = O + (size_t)bh * S * HD + (size_t)myq * HD;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<T>(Or + 32 * d + 8 * g + 4 * h, oacc[d][4 * g] * inv, oacc[d][4 * g + 1] * inv,
                  oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv);
    if (LSE != nullptr && h == 0) LSE[(size_t)bh * S + myq] = (m + log2f(l)) * kLn2;
  }
}

template <typename T, int HD, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  constexpr int NW = 4, BC = 64, BR = 32 * NW;
  const int nqt = (a.S + BR - 1) / BR;
  dim3 grid(nqt * a.B * a.Hq), block(NW * 64);
  mark(a.ev, a.nev, 0, st);
  hipLaunchKernelGGL((fwd_kernel<T, HD, BC, NW, CAUSAL>), grid, block, 0, st, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.o, a.lse, a.Hq, a.Hkv, a.S, a.scale * kLog2e, nqt);
  mark(a.ev, a.nev, 1, st);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t st) {
  if (a.D == 64) return a.causal ? launch_fwd_t<T, 64, true>(a, st) : launch_fwd_t<T, 64, false>(a, st);
  return a.causal ? launch_fwd_t<T, 128, true>(a, st) : launch_fwd_t<T, 128, false>(a, st);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 0: return launch_fwd_d<float>(a, st);
    case 1: return launch_fwd_d<_Float16>(a, st);
    default: return launch_fwd_d<__bf16>(a, st);
  }
}

}  // namespace fa
