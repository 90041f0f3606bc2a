// fa_bwd.hip -- backward pass of softmax attention, recomputing P from Q, K and L.
//
// Method: "Phase T14: 融合 Flash-Attention Kernel — Design Document", section
// "什么是 flash-attention" (recompute s = scale Q K^T, p = exp(s - L),
// dp = dO V^T, ds = p (dp - D) scale, then dQ += ds K, dK += ds^T Q,
// dV += p^T dO) and decision ③ (D[i] = sum_d dO[i,d] O[i,d] replaces the
// softmax Jacobian).  GQA head mapping from "Phase 14: Flash Attention 2 for
// SM120 — Design Document", section "GQA 支持"; dK and dV of a KV head are the
// sums over the query heads of its group.
//
// Three kernels on the caller's stream:
//   rowdot_kernel  D = rowsum(dO * O) in fp32 (HBM-bound, one pass).
//   dkdv_kernel    KV-tile outer: a workgroup owns 32*NW keys of one (b, KV
//                  head) and keeps their dK, dV accumulators in registers while
//                  it walks every query head of the group and every query tile
//                  that can see those keys.  No atomics: each dK / dV row has
//                  exactly one owner.
//   dq_kernel      query-tile outer, shaped like the forward: a workgroup owns
//                  32*NW query rows, keeps Q, dO, L and D of its rows in
//                  registers and walks the KV tiles.  dQ rows have one owner,
//                  so dQ needs no fp32 atomics either.
// The split recomputes S and dP in both kernels (7 products per (q, k) pair
// instead of 5) in exchange for no atomic traffic and deterministic outputs.
// An optional linear position bias (ALiBi) enters the exponent of P in a
// compile-time variant of both gradient kernels; the gradient formulas are
// unchanged, since the bias does not depend on Q, K or V.
//
// Layout choices (MI355X-specific):
//   dkdv: S = Q K^T and dP = dO V^T are formed with the wave's keys as MFMA
//   columns, so P and dS come out of the accumulators as the B operands of
//   dV^T += dO^T P and dK^T += Q^T dS.  Q and dO tiles are staged row-major
//   (XOR-swizzled, direct global->LDS loads) in LDS (A operands of S and dP);
//   the A operands of the gradient products,
//   dO^T and Q^T, come from gfx950's LDS transpose read of the same tiles.  L
//   and D of the tile's rows are staged in LDS too.  Each transpose read is
//   issued one product ahead; this fits two waves per SIMD because the
//   per-lane read offsets are computed once and kept in registers.  Small
//   grids take one of two variants: two wave groups sharing a workgroup's keys
//   (up to three workgroups per CU at D = 128, two at D = 64), or one wave per
//   SIMD with the S and dP fragments read two steps ahead (D = 64 up to three
//   per CU, and the bias kernels, which two groups do not fit).
//   dq: S^T = K Q^T and dP^T = V dO^T put one query row per lane pair (like
//   the forward), and dS^T is the B operand of dQ^T += K^T dS^T, whose K^T
//   operand is a transpose read of the row-major K tile.
#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_seq.hpp"

#include <mutex>
#include <type_traits>

namespace fa {

// ------------------------------------------------------------------ static scratch
// The row dot products of fa_bwd_noalloc.  Each GPU holds its own copy at its
// own address; host code reaches it only through the address that
// hipGetSymbolAddress returns with that GPU current (the array's name on the
// host is a host-side stand-in, not a device address).
static __device__ __align__(256) float scratch[kNoAllocRows];

hipError_t noalloc_rowdot(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

// ------------------------------------------------------------------ D = rowsum(dO * O)
template <typename T, int HD>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                     float* __restrict__ Dd, long long rows) {
  constexpr int kEpv = Elem<T>::kEpv;
  constexpr int kLanesPerRow = HD / kEpv;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int col = (threadIdx.x % kLanesPerRow) * kEpv;
  float acc = 0.f;
  if (row < rows) {
    Unit<T> a = load_unit<T>(O + row * HD + col);
    Unit<T> b = load_unit<T>(dO + row * HD + col);
    const T* ea = reinterpret_cast<const T*>(&a.bits);
    const T* eb = reinterpret_cast<const T*>(&b.bits);
#pragma unroll
    for (int e = 0; e < kEpv; ++e) acc = fmaf((float)ea[e], (float)eb[e], acc);
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && threadIdx.x % kLanesPerRow == 0) Dd[row] = acc;
}

// ------------------------------------------------------------------ dK, dV
// NG = 2: two groups of NW waves share the workgroup's keys (wave w and wave
// w + NW own the same 32 keys) and take alternate (query head, query tile)
// iterations of the walk, each through its own pair of LDS buffers; at the
// end the second group's dK, dV partial sums are added to the first's through
// LDS, in a fixed order.  This doubles the waves a small grid runs with (the
// keys of a problem give one wave per 32 keys and KV head, which at S = 4096
// and 8 KV heads is one wave per SIMD).
template <typename T, int HD, int BQ, int NW, int NG, bool CAUSAL, bool WINDOW, bool ALIBI, bool AHEAD>
__global__ __launch_bounds__(NG * NW * 64, 1) void dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dd, T* __restrict__ dK, T* __restrict__ dV,
    Problem pb, float c, float scale, int nkt) {
  constexpr int BKV = 32 * NW;
  constexpr int NT = NW * 64;  // threads of one group
  using Tile = RowTile<T, BQ, HD>;
  constexpr int kOffQ = 0;
  constexpr int kOffD = Tile::kElems;
  constexpr int kElems = 2 * Tile::kElems;
  using VTile = RowTile<T, BKV, HD>;
  static_assert(NG == 1 || NG == 2, "one or two wave groups");
  __shared__ __attribute__((aligned(16))) T lds[NG * 2 * kElems];   // [group][buf] Q, dO tiles
  __shared__ __attribute__((aligned(16))) T lds_v[VTile::kElems];  // this workgroup's V rows
  __shared__ __attribute__((aligned(16))) float lds_ld[NG][2][2][BQ];  // [group][buf][L*log2e, -D][row]

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform
  const int w = NG == 1 ? wv : wv % NW;                     // the wave's 32 keys
  const int grp = NG == 1 ? 0 : wv / NW;                    // its group
  const int gtid = NG == 1 ? tid : tid % NT;                // thread index within the group
  const int lane = tid & 63, r = lane & 31, h = lane >> 5;
  // work item: (b*Hkv + hkv) major, key tiles in order within a group (small
  // key tiles see the most queries: launched first); one XCD takes a
  // contiguous run, so the group's Q and dO stream through one L2
  const int work = xcd_slice(blockIdx.x, gridDim.x);
  const int bg = work / nkt;
  const int kvt = work - bg * nkt;
  const int b = bg / pb.Hkv, hkv = bg - b * pb.Hkv;
  const int G = pb.Hq / pb.Hkv;
  const Seq sv0 = seq_of(pb, b, hkv * G, hkv);  // key side is the same for the whole group
  const int kv0 = kvt * BKV;
  if (kv0 >= sv0.skv) return;  // a shorter sequence of a packed batch: no keys here
  const int kw0 = kv0 + 32 * w;
  const int mykv = kw0 + r;
  const int off = sv0.off;
  const T* Kh = K + sv0.kv_row0 * HD;
  const T* Vh = V + sv0.kv_row0 * HD;

  // keys past the end read key skv-1: their dK, dV are never stored.  K stays
  // in registers (B operand of S); V, the B operand of dP, is read from LDS
  // each tile, which keeps the kernel within 256 VGPRs (two waves per SIMD)
  vec8<T> kf[HD / 16];
  {
    const size_t o = (size_t)min(mykv, sv0.skv - 1) * HD + 8 * h;
#pragma unroll
    for (int t = 0; t < HD / 16; ++t) kf[t] = load8<T>(Kh + o + 16 * t);
  }
  {
    TileLoader<T, BKV, HD, NG * NT> vld;
    vld.init(tid);
    vld.issue(Vh, kv0, sv0.skv, lds_v, tid);
    vld.land(tid);  // published by the first barrier below
  }
  f32x16 dk[HD / 32], dv[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }
  // byte offsets of the lane's Q / dO fragment reads (16-bit tiles), computed
  // once and kept in registers so a read's tile and step parts are its
  // immediate (the compiler otherwise recomputed the swizzled addresses every
  // tile): fro: row r, columns 16t + 8h of a 32-row block; tro: the two
  // transposed reads for dK / dV columns 32d.  With two groups the group's
  // buffer pair is part of them, so the buffer of a step is a compile-time
  // constant.  The registers this frees let the gradient products read their
  // transposed fragments one product ahead at two waves per SIMD.
  // (The one-group 4-wave bias kernel at D = 128 keeps computing its
  // addresses, with its buffer chosen at run time: held offsets or the
  // unrolled loop take it past 256 registers, which halves its waves per SIMD.)
  constexpr bool kPin = sizeof(T) == 2 && !(ALIBI && NG == 1 && NW == 4 && !AHEAD && HD == 128);
  uint32_t fro[HD / 16], tro[HD / 32][2];
  if constexpr (kPin) {
    const uint32_t gb = NG == 1 ? 0u : (uint32_t)(grp * 2 * kElems * (int)sizeof(T));
#pragma unroll
    for (int t = 0; t < HD / 16; ++t) fro[t] = gb + (uint32_t)(Tile::at(r, 16 * t + 8 * h) * (int)sizeof(T));
    const int x = 4 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
    for (int d = 0; d < HD / 32; ++d) {
      const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tro[d][0] = gb + (uint32_t)(Tile::at(x, col) * (int)sizeof(T));
      tro[d][1] = gb + (uint32_t)(Tile::at(x + 8, col) * (int)sizeof(T));
    }
  }

  // query rows that can see one of the keys [kv0, kv0 + BKV): [qlo, qhi)
  const int qlo = CAUSAL ? max(0, kv0 - off) : 0;
  const int qhi = WINDOW ? min(sv0.sq, kv0 + BKV - 1 - off + pb.window + 1) : sv0.sq;
  const int first = qlo / BQ;
  const int nqt = qhi > qlo ? (qhi + BQ - 1) / BQ : first;
  const int per_head = nqt - first;
  const int total = G * per_head;

  LoopLoader<T, BQ, HD, NT> qld, dold;
  qld.init(gtid);
  dold.init(gtid);
  float ld_l = 0.f, ld_d = 0.f;
  // (query head, query tile) of an iteration, advanced without divisions.
  // Query tiles are walked from the last one down, and for each tile the
  // group's query heads one after another: every workgroup of a KV group
  // starts on the same tile and they all visit the tiles in the same order
  // (a workgroup of later keys stops earlier), so the tiles in use at any time
  // stay few and hit in the XCD's L2.
  const int hq0 = hkv * G;
  auto advance = [&](int& hq, int& qt) {
    if (++hq == hq0 + G) {
      hq = hq0;
      --qt;
    }
  };
  // a group takes iterations grp, grp + NG, grp + 2 NG, ... of the walk
  int cur_hq = hq0, cur_qt = nqt - 1;  // the tile in the group's LDS buffer `step & 1`
  if (grp == 1) advance(cur_hq, cur_qt);
  int nxt_hq = cur_hq, nxt_qt = cur_qt;  // the tile being prefetched
  const int mine = NG == 1 ? total : total > grp ? (total - grp + NG - 1) / NG : 0;  // this group's iterations
  const int steps = NG == 1 ? total : (total + NG - 1) / NG;                       // every group's loop count
  // a head's first query row, from the group's first head (no offset loads)
  const size_t hstride = q_head_stride(pb);
  // L and D of the tile's rows: every lane loads one (lanes past BQ repeat a
  // row), outside any branch and scaled only at commit, so nothing waits for
  // them (or, behind them, for the tile's loads) before the tile is needed
  auto issue = [&](int hq, int i0, int buf) {
    const size_t q_row0 = sv0.q_row0 + (size_t)(hq - hkv * G) * hstride;
    const size_t row = q_row0 + min(i0 + (tid & (BQ - 1)), sv0.sq - 1);
    ld_l = LSE[row];
    ld_d = Dd[row];
    T* base = lds + (grp * 2 + buf) * kElems;
    qld.issue(Q + q_row0 * HD, i0, sv0.sq, base + kOffQ, gtid);
    dold.issue(dO + q_row0 * HD, i0, sv0.sq, base + kOffD, gtid);
  };
  auto commit = [&](int buf) {
    qld.land(gtid);
    dold.land(gtid);
    if (gtid < BQ) {
      lds_ld[grp][buf][0][gtid] = ld_l * kLog2e;
      lds_ld[grp][buf][1][gtid] = -ld_d;
    }
  };

  if (mine > 0) {
    issue(cur_hq, cur_qt * BQ, 0);
    commit(0);
  }
  __syncthreads();
  // unrolled by two: every LDS address names its buffer at compile time
  // (except in the kernel that keeps computing its addresses, see kPin)
  auto body = [&](const int it, auto bufc) __attribute__((always_inline)) {
    const int buf = bufc;
    const int i0 = cur_qt * BQ;
    const bool more = it + 1 < mine;
    if (more) {  // the other buffer was last read before the previous barrier
#pragma unroll
      for (int k = 0; k < NG; ++k) advance(nxt_hq, nxt_qt);
      issue(nxt_hq, nxt_qt * BQ, buf ^ 1);
    }
    const T* Qs = lds + (grp * 2 + buf) * kElems + kOffQ;
    const T* dOs = lds + (grp * 2 + buf) * kElems + kOffD;
    if constexpr (kPin) {
#pragma unroll
      for (int t = 0; t < HD / 16; ++t) asm volatile("" : "+v"(fro[t]));
#pragma unroll
      for (int d = 0; d < HD / 32; ++d) asm volatile("" : "+v"(tro[d][0]), "+v"(tro[d][1]));
    }
    auto at_b = [](const T* base, uint32_t b) __attribute__((always_inline)) {
      return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + b);
    };
    // the step's buffer pair of group 0 (the group's offset is in fro and tro)
    const T* Qb = lds + buf * kElems + kOffQ;
    const T* dOb = lds + buf * kElems + kOffD;
    // does a query of the tile see one of this wave's keys?  (a group with
    // one iteration fewer sits out the last step)
    const bool active = it < mine && (!CAUSAL || i0 + BQ - 1 + off >= kw0) &&
                        (!WINDOW || i0 + off - pb.window <= kw0 + 31);
    if (active) {
      // linear position bias of the tile's head, in log2 units
      const float sl2 = ALIBI ? pb.alibi[cur_hq] * kLog2e : 0.f;
      // S, dP - D (BQ x 32): rows = queries of the tile, columns = this wave's
      // keys; the dP products start from -D of their rows, so dS = P (dP - D)
      // needs one multiply per element
      f32x16 s[BQ / 32], dp[BQ / 32];
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        f32x16 nd;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&lds_ld[grp][buf][1][32 * qb + 8 * g4 + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) nd[4 * g4 + e] = x[e];
        }
        if constexpr (sizeof(T) == 2) {
          // the Q, dO and V fragments of step t + LA are read before the
          // products of step t, in registers of their own, and a fence after
          // every step keeps the S and dP products alternating; the read-ahead
          // variant (one wave per SIMD) has the registers for two steps, the
          // bias kernel that computes its addresses (kPin) for none
          constexpr int NS = HD / 16;
          constexpr int LA = AHEAD ? 2 : kPin ? 1 : 0;
          vec8<T> qq[NS], oq[NS], vq[NS];
          auto rd = [&](int t) __attribute__((always_inline)) {
            if constexpr (kPin) {
              qq[t] = load8<T>(at_b(Qb + 32 * qb * Tile::kStride, fro[t]));
              oq[t] = load8<T>(at_b(dOb + 32 * qb * Tile::kStride, fro[t]));
            } else {
              qq[t] = Tile::frag(Qs, 32 * qb + r, 16 * t, h);
              oq[t] = Tile::frag(dOs, 32 * qb + r, 16 * t, h);
            }
            vq[t] = VTile::frag(lds_v, 32 * w + r, 16 * t, h);
          };
          if constexpr (LA > 0) rd(0);
          if constexpr (LA == 2) rd(1);
#pragma unroll
          for (int t = 0; t < NS; ++t) {
            if constexpr (LA == 0) rd(t);
            if (LA > 0 && t + LA < NS) rd(t + LA);
            s[qb] = mma<T>(qq[t], kf[t], t == 0 ? f32x16{} : s[qb]);
            dp[qb] = mma<T>(oq[t], vq[t], t == 0 ? nd : dp[qb]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < HD / 16; ++t) {
            s[qb] = mma<T>(Tile::frag(Qs, 32 * qb + r, 16 * t, h), kf[t], t == 0 ? f32x16{} : s[qb]);
            dp[qb] = mma<T>(Tile::frag(dOs, 32 * qb + r, 16 * t, h), VTile::frag(lds_v, 32 * w + r, 16 * t, h),
                            t == 0 ? nd : dp[qb]);
          }
        }
      }
      // invisible (query, key) pairs and queries past the end get p = 0 (keys
      // past the end only feed dK / dV columns that are never stored)
      const bool edge = (CAUSAL && i0 + off < kw0 + 31) ||
                        (WINDOW && i0 + BQ - 1 + off - pb.window > kw0) || (i0 + BQ > sv0.sq);
      if constexpr (CAUSAL && !WINDOW && !ALIBI) {
        // masked pairs get P = dS = 0 in a branch of their own: with the mask
        // inside the loop the compiler computed it (and selected) every tile
#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int qrow = 32 * qb + 8 * g4 + 4 * h;  // first of 4 consecutive query rows
            const f32x4 lv = *reinterpret_cast<const f32x4*>(&lds_ld[grp][buf][0][qrow]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * g4 + e;
              const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][i], c, -lv[e]));
              s[qb][i] = p;
              dp[qb][i] = p * dp[qb][i];
            }
          }
        if (edge) {
#pragma unroll
          for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int q = i0 + 32 * qb + 8 * (i >> 2) + 4 * h + (i & 3);
              const bool vis = q < sv0.sq && mykv <= q + off;
              s[qb][i] = vis ? s[qb][i] : 0.f;
              dp[qb][i] = vis ? dp[qb][i] : 0.f;
            }
        }
      } else {
        // (the split form above needs more registers with these masks)
        // query i0 + 32qb + 8g4 + 4h + e is |i0 + off - mykv + ...| keys from this key
        const float dl = (float)(i0 + off - mykv + 4 * h);
#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int qrow = 32 * qb + 8 * g4 + 4 * h;
            const f32x4 lv = *reinterpret_cast<const f32x4*>(&lds_ld[grp][buf][0][qrow]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * g4 + e;
              float e0 = -lv[e];
              if constexpr (ALIBI) e0 = fmaf(-sl2, fabsf(dl + (float)(32 * qb + 8 * g4 + e)), e0);
              float p = __builtin_amdgcn_exp2f(fmaf(s[qb][i], c, e0));
              if (edge) {
                const int q = i0 + qrow + e;
                const bool vis = q < sv0.sq && (!CAUSAL || mykv <= q + off) &&
                                 (!WINDOW || mykv >= q + off - pb.window);
                p = vis ? p : 0.f;
              }
              s[qb][i] = p;
              dp[qb][i] = p * dp[qb][i];
            }
          }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the tile's queries)
#pragma unroll
      for (int kt = 0; kt < BQ / 16; ++kt) {
        const vec8<T> pf = acc_to_frag<T>(s[kt >> 1], 8 * (kt & 1));
        const vec8<T> sf = acc_to_frag<T>(dp[kt >> 1], 8 * (kt & 1));
#pragma unroll
        for (int d = 0; d < HD / 32; ++d) {
          if constexpr (kPin) {
            auto trp = [&](const T* tile) __attribute__((always_inline)) {
              const T* tb = tile + 16 * kt * Tile::kStride;
              const vec4<T> a4 = lds_tr4<T>(at_b(tb, tro[d][0])), b4 = lds_tr4<T>(at_b(tb, tro[d][1]));
              return vec8<T>{a4[0], a4[1], a4[2], a4[3], b4[0], b4[1], b4[2], b4[3]};
            };
            dv[d] = mma<T>(trp(dOb), pf, dv[d]);
            dk[d] = mma<T>(trp(Qb), sf, dk[d]);
          } else {
            dv[d] = mma<T>(Tile::tr_frag(dOs, kt, 32 * d, lane), pf, dv[d]);
            dk[d] = mma<T>(Tile::tr_frag(Qs, kt, 32 * d, lane), sf, dk[d]);
          }
        }
      }
      if constexpr ((AHEAD || NW == 8 || NG == 2 || HD == 64) && sizeof(T) == 2) {
        // the transposed fragments of product n + 1 are read before product n
        // (the one-group 4-wave form at D = 128, used with the bias, would need
        // more than 256 registers for it)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
#pragma unroll
        for (int n = 0; n < 2 * (BQ / 16) * (HD / 32) - 1; ++n) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix products
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    if (more) commit(buf ^ 1);
#pragma unroll
    for (int k = 0; k < NG; ++k) advance(cur_hq, cur_qt);
    __syncthreads();
  };
  if constexpr (kPin || sizeof(T) == 4) {
    for (int it = 0; it < steps; it += 2) {
      body(it, std::integral_constant<int, 0>{});
      if (it + 1 < steps) body(it + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int it = 0; it < steps; ++it) body(it, it & 1);
  }

  if constexpr (NG == 2) {
    // dK, dV of the two groups: the second group's partial sums go through
    // the (now free) tile buffers, one accumulator set at a time, and the
    // first group adds them to its own
    static_assert(NW * (HD / 32) * 16 * 64 * 4 <= (int)sizeof(lds), "a group's accumulators fit the tile buffers");
    f32x4* xf = reinterpret_cast<f32x4*>(lds);
    auto fold = [&](f32x16(&acc)[HD / 32]) __attribute__((always_inline)) {
      if (grp == 1) {
#pragma unroll
        for (int d = 0; d < HD / 32; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            xf[((w * (HD / 32) + d) * 4 + g) * 64 + lane] =
                f32x4{acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]};
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int d = 0; d < HD / 32; ++d)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 x = xf[((w * (HD / 32) + d) * 4 + g) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[d][4 * g + e] += x[e];
          }
      }
      __syncthreads();
    };
    fold(dk);
    fold(dv);
    if (grp != 0) return;
  }

  if constexpr (sizeof(T) == 2 && !WINDOW && !ALIBI) {
    // dK and dV rows leave through LDS, the wave's share of the V rows (read
    // for the last time before the loop's last barrier): whole rows per store
    // instruction.  The window and bias kernels store straight from the
    // accumulators: they have no registers to spare for it.
    static_assert(NW * 32 * HD <= VTile::kElems, "a wave's rows fit its share of the V rows");
    T* stg = lds_v + w * 32 * HD;
    store_block_rows<T, HD>(dk, scale, stg, dK + (sv0.kv_row0 + kw0) * HD, sv0.skv - kw0, lane);
    store_block_rows<T, HD>(dv, 1.f, stg, dV + (sv0.kv_row0 + kw0) * HD, sv0.skv - kw0, lane);
  } else if (mykv < sv0.skv) {
    T* dKr = dK + (sv0.kv_row0 + mykv) * HD;
    T* dVr = dV + (sv0.kv_row0 + mykv) * HD;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * h;
        store4<T>(dKr + col, dk[d][4 * g] * scale, dk[d][4 * g + 1] * scale, dk[d][4 * g + 2] * scale,
                  dk[d][4 * g + 3] * scale);
        store4<T>(dVr + col, dv[d][4 * g], dv[d][4 * g + 1], dv[d][4 * g + 2], dv[d][4 * g + 3]);
      }
  }
}

// ------------------------------------------------------------------ dQ
// NG = 2: two groups of NW waves share the workgroup's query rows (waves w and
// w + NW own the same 32 rows) and take alternate KV tiles, each in its own
// pair of LDS buffers; at the end the second group's dQ partial sums are added
// to the first's through LDS, in a fixed order (small grids: twice the waves).
template <typename T, int HD, int BC, int NW, int NG, bool CAUSAL, bool WINDOW, bool ALIBI>
__global__ __launch_bounds__(NG * NW * 64, 1) void dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dd, T* __restrict__ dQ, Problem pb, float c,
    float scale, int nqt) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;  // threads of one group
  static_assert(NG == 1 || NG == 2, "one or two wave groups");
  using Tile = RowTile<T, BC, HD>;
  constexpr int kOffK = 0;
  constexpr int kOffV = Tile::kElems;
  constexpr int kElems = 2 * Tile::kElems;
  __shared__ __attribute__((aligned(16))) T lds[NG * 2 * kElems];  // [group][buf] K, V tiles

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform
  const int w = NG == 1 ? wv : wv & (NW - 1);               // the wave's 32 rows
  const int grp = NG == 1 ? 0 : wv / NW;                    // its group
  const int gtid = NG == 1 ? tid : tid & (NT - 1);          // thread within the group
  const int lane = tid & 63, r = lane & 31, h = lane >> 5;
  const QTile wt = qtile_of<CAUSAL>(xcd_slice(blockIdx.x, gridDim.x), nqt, pb);
  const int b = wt.b, hq = wt.hq, qt = wt.qt;
  const Seq sv = seq_of(pb, b, hq, hq / (pb.Hq / pb.Hkv));
  const int i0 = qt * BR;
  if (i0 >= sv.sq) return;
  const T* Kh = K + sv.kv_row0 * HD;
  const T* Vh = V + sv.kv_row0 * HD;
  const int qw0 = i0 + 32 * w;
  const int myq = qw0 + r;
  const int off = sv.off;

  // query rows past the end read row sq-1: their dQ is never stored
  vec8<T> qf[HD / 16], df[HD / 16];
  const size_t qrow = sv.q_row0 + min(myq, sv.sq - 1);
  {
    const size_t o = qrow * HD + 8 * h;
#pragma unroll
    for (int t = 0; t < HD / 16; ++t) {
      qf[t] = load8<T>(Q + o + 16 * t);
      df[t] = load8<T>(dO + o + 16 * t);
    }
  }
  const float lq = LSE[qrow] * kLog2e;
  // linear position bias of the head, in log2 units
  const float sl2 = ALIBI ? pb.alibi[hq] * kLog2e : 0.f;
  f32x16 ndq;  // -D of the lane's row in every slot: the start of its dP^T products
#pragma unroll
  for (int i = 0; i < 16; ++i) ndq[i] = -Dd[qrow];
  f32x16 acc[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d) acc[d] = f32x16{};
  // byte offsets within a K tile of the lane's two transposed reads for each
  // 32-column block of dQ (16-bit tiles): computed once and kept in registers,
  // so the tile and key-block parts of an address are the read's immediate
  uint32_t tro[HD / 32][2];
  if constexpr (sizeof(T) == 2) {
    const int x = 4 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
    for (int d = 0; d < HD / 32; ++d) {
      const int col = 32 * d + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      tro[d][0] = (uint32_t)(Tile::at(x, col) * (int)sizeof(T));
      tro[d][1] = (uint32_t)(Tile::at(x + 8, col) * (int)sizeof(T));
    }
  }

  const int last = min(i0 + BR, sv.sq) - 1;
  const int hi = CAUSAL ? min(sv.skv, last + off + 1) : sv.skv;
  const int lo = WINDOW ? max(0, i0 + off - pb.window) : 0;
  const int jt0 = lo / BC;
  const int ntiles = hi > lo ? (hi + BC - 1) / BC - jt0 : 0;

  LoopLoader<T, BC, HD, NT> kld, vld;
  kld.init(gtid);
  vld.init(gtid);
  // a group takes tiles grp, grp + NG, ... of the range, in its own buffers
  // (buffer bb of the group; formed from the array itself, which keeps the
  // one-group kernel's LDS addressing as it was)
  auto gbuf = [&](int bb) __attribute__((always_inline)) -> T* {
    if constexpr (NG == 1)
      return lds + bb * kElems;
    else
      return lds + (grp * 2 + bb) * kElems;
  };
  const int mine = NG == 1 ? ntiles : ntiles > grp ? (ntiles - grp + NG - 1) / NG : 0;  // this group's tiles
  const int steps = NG == 1 ? ntiles : (ntiles + NG - 1) / NG;                         // every group's loop count
  if (mine > 0) {
    kld.issue(Kh, (jt0 + grp) * BC, sv.skv, gbuf(0) + kOffK, gtid);
    vld.issue(Vh, (jt0 + grp) * BC, sv.skv, gbuf(0) + kOffV, gtid);
    kld.land(gtid);
    vld.land(gtid);
  }
  __syncthreads();
  // Everything issued so far has landed; a wait the compiler sees tells it
  // so, and it then places no waits for these loads inside the loop, where
  // they would also wait for the loop's own assembly loads.
  __builtin_amdgcn_s_waitcnt(0);

  // unrolled by two: every LDS address names its buffer at compile time
  auto tile = [&](const int li, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int j0 = (jt0 + li * NG + grp) * BC;
    const bool more = li + 1 < mine;
    if (more) {  // the other buffer was last read before the previous barrier
      T* nb = gbuf(buf ^ 1);
      kld.issue(Kh, j0 + NG * BC, sv.skv, nb + kOffK, gtid);
      vld.issue(Vh, j0 + NG * BC, sv.skv, nb + kOffV, gtid);
    }
    const T* Ks = gbuf(buf) + kOffK;
    const T* Vs = gbuf(buf) + kOffV;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int d = 0; d < HD / 32; ++d) asm volatile("" : "+v"(tro[d][0]), "+v"(tro[d][1]));
    }
    // (a group with one tile fewer sits out the last step)
    const bool active = (NG == 1 || li < mine) && (!CAUSAL || j0 <= qw0 + 31 + off) &&
                        (!WINDOW || j0 + BC - 1 >= qw0 + off - pb.window);
    if (active) {
      const bool edge = (CAUSAL && j0 + BC - 1 > qw0 + off) ||
                        (WINDOW && j0 < qw0 + 31 + off - pb.window) || (j0 + BC > sv.skv);
      // one 32-key block at a time: its S^T, dP^T and dS^T are dead before the
      // next block's are formed, which halves the accumulator registers
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        // dP^T starts from -D of the lane's row, so dS = P (dP - D) is one
        // multiply per element
        f32x16 s, dp;
        if constexpr (sizeof(T) == 2) {
          // the K and V fragments of step t+2 are read before the products of
          // step t, in registers of their own, and a fence after every step
          // keeps the S and dP products alternating (with a scheduling hint
          // alone the compiler ran the whole S chain first, each product
          // waiting for the fragment read just before it)
          constexpr int NS = HD / 16;
          vec8<T> kq[NS], vq[NS];
          kq[0] = Tile::frag(Ks, 32 * kb + r, 0, h);
          vq[0] = Tile::frag(Vs, 32 * kb + r, 0, h);
          kq[1] = Tile::frag(Ks, 32 * kb + r, 16, h);
          vq[1] = Tile::frag(Vs, 32 * kb + r, 16, h);
#pragma unroll
          for (int t = 0; t < NS; ++t) {
            if (t + 2 < NS) {
              kq[t + 2] = Tile::frag(Ks, 32 * kb + r, 16 * (t + 2), h);
              vq[t + 2] = Tile::frag(Vs, 32 * kb + r, 16 * (t + 2), h);
            }
            s = mma<T>(kq[t], qf[t], t == 0 ? f32x16{} : s);
            dp = mma<T>(vq[t], df[t], t == 0 ? ndq : dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < HD / 16; ++t) {
            s = mma<T>(Tile::frag(Ks, 32 * kb + r, 16 * t, h), qf[t], t == 0 ? f32x16{} : s);
            dp = mma<T>(Tile::frag(Vs, 32 * kb + r, 16 * t, h), df[t], t == 0 ? ndq : dp);
          }
        }
        // P and dS; the masked form is a branch of its own (a mask inside the
        // loop is computed, and selected, for every tile)
        // key j0 + 32kb + 4h + e of register i (e = 8(i/4) + i%4) is |dl - e|
        // keys from this query's diagonal
        const float dl = (float)(myq + off - j0 - 32 * kb - 4 * h);
        auto elementwise = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float e0 = -lq;
            if constexpr (ALIBI) e0 = fmaf(-sl2, fabsf(dl - (float)(8 * (i >> 2) + (i & 3))), e0);
            float p = __builtin_amdgcn_exp2f(fmaf(s[i], c, e0));
            if constexpr (decltype(masked)::value) {
              const int kv = j0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
              p = key_visible<CAUSAL, WINDOW>(pb, sv, myq, kv) ? p : 0.f;
            }
            dp[i] = p * dp[i];
          }
        };
        if (edge)
          elementwise(std::true_type{});
        else
          elementwise(std::false_type{});
        // dQ^T (HD x 32) += K_block^T dS^T
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const vec8<T> sf = acc_to_frag<T>(dp, 8 * kk);
#pragma unroll
          for (int d = 0; d < HD / 32; ++d) {
            if constexpr (sizeof(T) == 2) {
              const char* tb = reinterpret_cast<const char*>(Ks + 16 * (2 * kb + kk) * Tile::kStride);
              const vec4<T> lo4 = lds_tr4<T>(reinterpret_cast<const T*>(tb + tro[d][0]));
              const vec4<T> hi4 = lds_tr4<T>(reinterpret_cast<const T*>(tb + tro[d][1]));
              const vec8<T> kf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
              acc[d] = mma<T>(kf, sf, acc[d]);
            } else {
              acc[d] = mma<T>(Tile::tr_frag(Ks, 2 * kb + kk, 32 * d, lane), sf, acc[d]);
            }
          }
        }
        if constexpr (sizeof(T) == 2) {
          // the transposed K fragments of product n + 1 are read before product n
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
#pragma unroll
          for (int n = 0; n < 2 * (HD / 32) - 1; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix products
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (more) {
      kld.land(tid);
      vld.land(tid);
    }
    __syncthreads();
  };
  for (int li = 0; li < steps; li += 2) {
    tile(li, std::integral_constant<int, 0>{});
    if (li + 1 < steps) tile(li + 1, std::integral_constant<int, 1>{});
  }

  if constexpr (NG == 2) {
    // the second group's dQ partial sums through the (now free) tile buffers
    static_assert(NW * (HD / 32) * 16 * 64 * 4 <= (int)sizeof(lds), "a group's accumulators fit the tile buffers");
    f32x4* xf = reinterpret_cast<f32x4*>(lds);
    if (grp == 1) {
#pragma unroll
      for (int d = 0; d < HD / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xf[((w * (HD / 32) + d) * 4 + g) * 64 + lane] =
              f32x4{acc[d][4 * g], acc[d][4 * g + 1], acc[d][4 * g + 2], acc[d][4 * g + 3]};
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = xf[((w * (HD / 32) + d) * 4 + g) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[d][4 * g + e] += x[e];
      }
  }

  if constexpr (sizeof(T) == 2 && !WINDOW && !ALIBI) {
    // dQ rows leave through LDS (free after the loop's last barrier; with two
    // groups, past the partial sums): whole rows per store instruction.  The
    // window and bias kernels store straight from the accumulators.
    constexpr int kStg = NG == 1 ? 0 : NW * (HD / 32) * 4 * 64 * 16 / (int)sizeof(T);
    static_assert(kStg + NW * 32 * HD <= (int)(sizeof(lds) / sizeof(T)), "the dQ rows fit the tile buffers");
    store_block_rows<T, HD>(acc, scale, lds + kStg + w * 32 * HD, dQ + (sv.q_row0 + qw0) * HD, sv.sq - qw0, lane);
  } else if (myq < sv.sq) {
    T* dQr = dQ + (sv.q_row0 + myq) * HD;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<T>(dQr + 32 * d + 8 * g + 4 * h, acc[d][4 * g] * scale, acc[d][4 * g + 1] * scale,
                  acc[d][4 * g + 2] * scale, acc[d][4 * g + 3] * scale);
  }
}

// ------------------------------------------------------------------ launch
template <typename T, int HD, int NW, int NG, bool CAUSAL, bool WINDOW, bool ALIBI>
static void launch_dq_nw(const BwdArgs& a, hipStream_t st, float c) {
  constexpr int BC = 64;
  const Problem& pb = a.pb;
  const int nqt = (pb.Sq + 32 * NW - 1) / (32 * NW);
  dim3 grid(nqt * pb.B * pb.Hq);
  if (grid.x > 0)
    hipLaunchKernelGGL((dq_kernel<T, HD, BC, NW, NG, CAUSAL, WINDOW, ALIBI>), grid, dim3(NG * NW * 64), 0, st, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, (const T*)a.dO, a.lse, (const float*)a.rowdot, (T*)a.dq, pb, c,
                       a.scale, nqt);
}

template <typename T, int HD, int BQ, int NW, int NG, bool CAUSAL, bool WINDOW, bool ALIBI, bool AHEAD>
static void launch_dkdv(const BwdArgs& a, hipStream_t st, dim3 grid, float c, int nkt) {
  hipLaunchKernelGGL((dkdv_kernel<T, HD, BQ, NW, NG, CAUSAL, WINDOW, ALIBI, AHEAD>), grid, dim3(NG * NW * 64), 0, st,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dO, a.lse, (const float*)a.rowdot,
                     (T*)a.dk, (T*)a.dv, a.pb, c, a.scale, nkt);
}

template <typename T, int HD, bool CAUSAL, bool WINDOW, bool ALIBI>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const Problem& pb = a.pb;
  const long long rows = pb.cu_q != nullptr ? (long long)pb.Hq * pb.Tq : (long long)pb.B * pb.Hq * pb.Sq;
  if (rows > 0) {
    constexpr int kRowsPerBlock = 256 / (HD / Elem<T>::kEpv);
    dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    mark(a.ev, a.nev, 0, st);
    hipLaunchKernelGGL((rowdot_kernel<T, HD>), grid, dim3(256), 0, st, (const T*)a.o, (const T*)a.dO, a.rowdot,
                       rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float c = a.scale * kLog2e;
  {
    constexpr int NW = 4, BQ = (HD == 128 || sizeof(T) == 4) ? 32 : 64;
    const int nkt = (pb.Skv + 32 * NW - 1) / (32 * NW);
    dim3 grid(nkt * pb.B * pb.Hkv);
    mark(a.ev, a.nev, 1, st);
    // Grids counted in 4-wave workgroups of 128 keys (measured on the backward):
    //   two wave groups per workgroup up to three per CU at D = 128 (against
    //     the next choice: +16 % at S = 6144, +11 % at 8192, +15 % at 10240,
    //     +7 % at 12288 with 32/8 heads, a tie at 16384) and up to two at
    //     D = 64 (+14 % at two, mixed at three); ALiBi's extra registers do
    //     not fit it;
    //   then up to three: the read-ahead variant, one wave per SIMD (+13 % at
    //     one workgroup per CU, +2 % at three against the plain kernel; at
    //     four it loses 9 %).
    // Larger 16-bit D = 128 grids: 8-wave workgroups of 256 keys (one per CU),
    // so that each Q / dO tile a workgroup loads serves twice the keys and the
    // L2 reads of those tiles halve (+1.1 % on the long-context backward).
    if (grid.x > 0) {
      bool done = false;
      if constexpr (sizeof(T) == 2) {
        if constexpr (!ALIBI) {
          if ((long long)grid.x <= (HD == 128 ? 3 : 2) * kCUs) {
            launch_dkdv<T, HD, BQ, NW, 2, CAUSAL, WINDOW, ALIBI, false>(a, st, grid, c, nkt);
            done = true;
          }
        }
        if (!done && (long long)grid.x <= 3 * kCUs) {
          launch_dkdv<T, HD, BQ, NW, 1, CAUSAL, WINDOW, ALIBI, true>(a, st, grid, c, nkt);
          done = true;
        }
      }
      if (!done) {
        if constexpr (sizeof(T) == 2 && HD == 128 && !ALIBI) {
          const int nkt8 = (pb.Skv + 255) / 256;
          launch_dkdv<T, HD, BQ, 8, 1, CAUSAL, WINDOW, ALIBI, false>(a, st, dim3(nkt8 * pb.B * pb.Hkv), c, nkt8);
        } else {
          launch_dkdv<T, HD, BQ, NW, 1, CAUSAL, WINDOW, ALIBI, false>(a, st, grid, c, nkt);
        }
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark(a.ev, a.nev, 2, st);
  // dQ: 8-wave workgroups when there are enough of them (as the forward)
  bool wide = false;
  if constexpr (sizeof(T) == 2) {  // fp32 keeps 4-wave workgroups (no 8-wave instances)
    wide = (long long)((pb.Sq + 255) / 256) * pb.B * pb.Hq >= kWideGrid;
    if (wide) launch_dq_nw<T, HD, 8, 1, CAUSAL, WINDOW, ALIBI>(a, st, c);
  }
  if (!wide) {
    // 16-bit grids of one 4-wave workgroup per CU or fewer: two wave groups
    // per workgroup split the KV tiles (two waves per SIMD instead of one;
    // ALiBi's extra registers do not fit it)
    bool split = false;
    if constexpr (sizeof(T) == 2 && !ALIBI) {
      split = (long long)((pb.Sq + 127) / 128) * pb.B * pb.Hq <= kCUs;
      if (split) launch_dq_nw<T, HD, 4, 2, CAUSAL, WINDOW, ALIBI>(a, st, c);
    }
    if (!split) launch_dq_nw<T, HD, 4, 1, CAUSAL, WINDOW, ALIBI>(a, st, c);
  }
  mark(a.ev, a.nev, 3, st);
  return hipGetLastError();
}

template <typename T, int HD, bool ALIBI>
static hipError_t launch_bwd_m(const BwdArgs& a, hipStream_t st) {
  if (a.pb.window >= 0)
    return a.pb.causal ? launch_bwd_t<T, HD, true, true, ALIBI>(a, st) : launch_bwd_t<T, HD, false, true, ALIBI>(a, st);
  return a.pb.causal ? launch_bwd_t<T, HD, true, false, ALIBI>(a, st) : launch_bwd_t<T, HD, false, false, ALIBI>(a, st);
}

template <typename T, int HD>
static hipError_t launch_bwd_b(const BwdArgs& a, hipStream_t st) {
  return a.pb.alibi != nullptr ? launch_bwd_m<T, HD, true>(a, st) : launch_bwd_m<T, HD, false>(a, st);
}

template <typename T>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  return a.D == 64 ? launch_bwd_b<T, 64>(a, st) : launch_bwd_b<T, 128>(a, st);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 0: return launch_bwd_d<float>(a, st);
    case 1: return launch_bwd_d<_Float16>(a, st);
    default: return launch_bwd_d<__bf16>(a, st);
  }
}

}  // namespace fa
