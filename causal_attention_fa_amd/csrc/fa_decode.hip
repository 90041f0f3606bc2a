// fa_decode.hip -- split-KV forward for decode-shaped problems: few query rows
// per KV head (G * Sq <= 32), many keys.
//
// Method: the dedicated decode kernel that "Phase 14: Flash Attention 2 for
// SM120 — Design Document" (section 已知局限与后续优化方向) asks for, reducing
// in parallel along the KV dimension, with the split-KV merge that
// "FlashAttention 与 SDPA Backend" lists among a real kernel's choices.  Each
// split runs the online softmax of the forward over its own keys and leaves a
// normalised partial result (O_s, L_s); the merge is the logsumexp identity
//   L = log sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s.
//
// MI355X layout:
//   * split_kernel: a workgroup owns (b, KV head, key split).  The G query
//     heads of the KV group and their Sq positions form the 32 columns of one
//     MFMA block, so K and V are read once per KV group (decode is HBM-bound
//     and GQA's sharing is the whole saving).  K/V tiles of 32*NW keys are
//     filled by direct global->LDS loads, double buffered; wave w takes keys
//     32w..32w+31 of every tile with its own running (m, l, O^T), and the
//     waves are combined through LDS once at the end;
//   * merge_kernel: one wave per query row reads the splits' (L_s, O_s) and
//     writes O in the input dtype and L.
// No atomics: the result is deterministic for a given split count.
#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_seq.hpp"

namespace fa {

template <typename T>
struct SplitCfg {
  static constexpr int kDtype = sizeof(T) == 4 ? 0 : 2;  // fp32, or a 16-bit type
  static constexpr int NW = split_waves(kDtype);
  static constexpr int BC = split_tile_keys(kDtype);
};

template <typename T, int HD, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(SplitCfg<T>::NW * 64, 1) void split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, float* __restrict__ Opart,
    float* __restrict__ Lpart, Problem pb, float c, int nsplit, int chunk, long long qrows) {
  constexpr int NW = SplitCfg<T>::NW;
  constexpr int BC = SplitCfg<T>::BC;
  constexpr int NT = NW * 64;
  using Tile = RowTile<T, BC, HD>;
  constexpr int kBuf = 2 * Tile::kElems;  // K tile, then V tile
  constexpr int kRedStride = HD + 4;     // fp32 row stride of the combine buffer
  static_assert(NW * 32 * kRedStride * 4 + 2 * NW * 32 * 4 <= 2 * kBuf * (int)sizeof(T), "combine fits in tiles");
  __shared__ __attribute__((aligned(16))) T lds[2 * kBuf];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform
  const int lane = tid & 63, r = lane & 31, h = lane >> 5;
  const int split = blockIdx.x % nsplit;
  const int bg = blockIdx.x / nsplit;
  const int b = bg / pb.Hkv, hkv = bg - b * pb.Hkv;
  const int G = pb.Hq / pb.Hkv;
  const Seq sv = seq_of(pb, b, hkv * G, hkv);
  const int R = G * sv.sq;  // query rows of the group (<= 32, checked on the host)
  if (R == 0) return;
  // lane r carries row (g, i) = (r / sq, r % sq); rows past R repeat row R-1
  const int rr = min(r, R - 1);
  const int g = rr / sv.sq, qi = rr - g * sv.sq;
  const size_t qrow = seq_of(pb, b, hkv * G + g, hkv).q_row0 + qi;
  const T* Kh = K + sv.kv_row0 * HD;
  const T* Vh = V + sv.kv_row0 * HD;
  const int off = sv.off;

  vec8<T> qf[HD / 16];
#pragma unroll
  for (int t = 0; t < HD / 16; ++t) qf[t] = load8<T>(Q + qrow * HD + 8 * h + 16 * t);

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d) oacc[d] = f32x16{};
  float lsum = 0.f, m = -INFINITY;

  // this split's keys, narrowed to those some row of the group can see
  int lo = split * chunk;
  int hi = min(sv.skv, lo + chunk);
  if (CAUSAL) hi = min(hi, sv.sq - 1 + off + 1);
  if (WINDOW) lo = max(lo, off - pb.window);
  const int ntiles = hi > lo ? (hi - lo + BC - 1) / BC : 0;

  LoopLoader<T, BC, HD, NT> kld, vld;
  kld.init(tid);
  vld.init(tid);
  if (ntiles > 0) {
    kld.issue(Kh, lo, sv.skv, lds, tid);
    vld.issue(Vh, lo, sv.skv, lds + Tile::kElems, tid);
    kld.land(tid);
    vld.land(tid);
  }
  __syncthreads();
  // Everything issued so far has landed; a wait the compiler sees tells it
  // so, and it then places no waits for these loads inside the loop, where
  // they would also wait for the loop's own assembly loads.
  __builtin_amdgcn_s_waitcnt(0);

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = lo + it * BC;
    const bool more = it + 1 < ntiles;
    if (more) {  // the other buffer was last read before the previous barrier
      T* nb = lds + ((it + 1) & 1) * kBuf;
      kld.issue(Kh, j0 + BC, sv.skv, nb, tid);
      vld.issue(Vh, j0 + BC, sv.skv, nb + Tile::kElems, tid);
    }
    const T* Ks = lds + (it & 1) * kBuf;
    const T* Vs = Ks + Tile::kElems;
    const int kw0 = j0 + 32 * w;  // this wave's first key
    if (kw0 < hi) {
      // S^T (32 keys x 32 rows) = K_w Q^T
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < HD / 16; ++t) s = mma<T>(Tile::frag(Ks, 32 * w + r, 16 * t, h), qf[t], s);
      // keys past the split, the sequence or a row's mask get -inf; padding
      // rows (r >= R) repeat row R-1 and are never stored
      const bool edge = kw0 + 31 >= hi || (CAUSAL && kw0 + 31 > off) ||
                        (WINDOW && kw0 < sv.sq - 1 + off - pb.window);
      if (edge) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kv = kw0 + 8 * (i >> 2) + 4 * h + (i & 3);
          s[i] = (kv < hi && key_visible<CAUSAL, WINDOW>(pb, sv, qi, kv)) ? s[i] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = wave_xor32_max(mx) * c;
      if (mx > m) {  // per lane: no wave-wide rescale branch needed at 16 scores per row
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mx);
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) oacc[d] *= alpha;
        m = mx;
      }
      const float ref = (m == -INFINITY) ? 0.f : m;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -ref));
      // O^T (HD x 32) += V_w^T P^T ; l += the lane's P
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const vec8<T> pf = acc_to_frag<T>(s, 8 * kk);
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) oacc[d] = mma<T>(Tile::tr_frag(Vs, 2 * w + kk, 32 * d, lane), pf, oacc[d]);
        lsum = frag_sum(pf, lsum);
      }
    }
    if (more) {
      kld.land(tid);
      vld.land(tid);
    }
    __syncthreads();
  }

  // combine the NW waves through LDS (the tile buffers are free after the
  // loop's last barrier): red[w][row][d] = O_w, then per-row (m_w, l_w)
  float* red = reinterpret_cast<float*>(lds);
  float* red_m = red + NW * 32 * kRedStride;
  float* red_l = red_m + NW * 32;
  {
    float* mine = red + (w * 32 + r) * kRedStride;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(mine + 32 * d + 8 * g4 + 4 * h) =
            f32x4{oacc[d][4 * g4], oacc[d][4 * g4 + 1], oacc[d][4 * g4 + 2], oacc[d][4 * g4 + 3]};
    const float l = wave_xor32_sum(lsum);
    if (h == 0) {
      red_m[w * 32 + r] = m;
      red_l[w * 32 + r] = l;
    }
  }
  __syncthreads();
  // each thread finishes 4 consecutive columns of one row per pass
  constexpr int kQuads = 32 * HD / 4;
  for (int u = tid; u < kQuads; u += NT) {
    const int row = u / (HD / 4);
    const int col = (u % (HD / 4)) * 4;
    if (row >= R) continue;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, red_m[v * 32 + row]);
    float l = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float mv = red_m[v * 32 + row];
      const float a = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
      l += a * red_l[v * 32 + row];
      o += a * *reinterpret_cast<const f32x4*>(red + (v * 32 + row) * kRedStride + col);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int gg = row / sv.sq, ii = row - gg * sv.sq;
    const size_t orow = seq_of(pb, b, hkv * G + gg, hkv).q_row0 + ii;
    *reinterpret_cast<f32x4*>(Opart + ((size_t)split * qrows + orow) * HD + col) = o * inv;
    if (col == 0) Lpart[(size_t)split * qrows + orow] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
  }
}

// One wave per query row: O = sum_s exp(L_s - L) O_s, L = log sum_s exp(L_s).
template <typename T, int HD>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                                                    T* __restrict__ O, float* __restrict__ LSE, int nsplit,
                                                    long long qrows) {
  constexpr int kPer = HD / 64;  // columns per lane
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= qrows) return;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, Lpart[(size_t)s * qrows + row]);
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float z = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float Ls = Lpart[(size_t)s * qrows + row];
      const float a = __expf(Ls - M);  // 0 for an empty split (L_s = -inf)
      z += a;
      const float* src = Opart + ((size_t)s * qrows + row) * HD + lane * kPer;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(a, src[e], acc[e]);
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  T* dst = O + row * HD + lane * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e) dst[e] = to_elem<T>(acc[e] * inv);
  if (LSE != nullptr && lane == 0) LSE[row] = z > 0.f ? M + __logf(z) : -INFINITY;
}

template <typename T, int HD, bool CAUSAL, bool WINDOW>
static hipError_t launch_split_t(const SplitArgs& a, hipStream_t st) {
  const Problem& pb = a.pb;
  float* Opart = a.work;
  float* Lpart = a.work + (size_t)a.nsplit * a.qrows * HD;
  dim3 grid((unsigned)(a.nsplit * pb.B * pb.Hkv));
  mark(a.ev, a.nev, 0, st);
  if (grid.x > 0)
    hipLaunchKernelGGL((split_kernel<T, HD, CAUSAL, WINDOW>), grid, dim3(SplitCfg<T>::NW * 64), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, Opart, Lpart, pb, a.scale * kLog2e, a.nsplit,
                       a.chunk, a.qrows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark(a.ev, a.nev, 1, st);
  hipLaunchKernelGGL((merge_kernel<T, HD>), dim3((unsigned)((a.qrows + 3) / 4)), dim3(256), 0, st,
                     (const float*)Opart, (const float*)Lpart, (T*)a.o, a.lse, a.nsplit, a.qrows);
  mark(a.ev, a.nev, 2, st);
  return hipGetLastError();
}

template <typename T, int HD>
static hipError_t launch_split_m(const SplitArgs& a, hipStream_t st) {
  if (a.pb.window >= 0)
    return a.pb.causal ? launch_split_t<T, HD, true, true>(a, st) : launch_split_t<T, HD, false, true>(a, st);
  return a.pb.causal ? launch_split_t<T, HD, true, false>(a, st) : launch_split_t<T, HD, false, false>(a, st);
}

template <typename T>
static hipError_t launch_split_d(const SplitArgs& a, hipStream_t st) {
  return a.D == 64 ? launch_split_m<T, 64>(a, st) : launch_split_m<T, 128>(a, st);
}


hipError_t launch_splitkv(const SplitArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 0: return launch_split_d<float>(a, st);
    case 1: return launch_split_d<_Float16>(a, st);
    default: return launch_split_d<__bf16>(a, st);
  }
}

}  // namespace fa
