// fa_fwd.hip -- forward pass: O = softmax(mask(scale * Q K^T)) V and L = logsumexp,
// by online softmax over KV tiles (gfx950, wave64, 32x32 MFMA).
//
// Method: "Phase 14: Flash Attention 2 for SM120 — Design Document", section
// "FA2 算法" (Q tile outer, loaded once; KV tiles inner; running max / sum with
// rescale by exp(m - m_new)); section "Causal Mask" (tiles wholly after the
// diagonal are skipped, the rest masked per element); section "GQA 支持"
// (KV head = query head / group size, indexed in the kernel), where a longer
// key sequence is aligned bottom-right (kv_offset = kv_len - q_len).  L = m + log l is
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
//     buffered: the next stage's direct global->LDS loads are issued before
//     the current stage's math; V^T fragments come from gfx950's LDS
//     transpose read.  A stage (and tile) is 128 keys for 8-wave
//     workgroups, which have the CU's LDS to themselves, and 64 keys
//     otherwise; the waves synchronise once per stage, and in 8-wave
//     workgroups only waves 0-3 issue the loads (the other wave of each SIMD
//     keeps computing while a loading wave waits for the memory pipeline);
//   * softmax in base 2: p = exp2(s * scale*log2e - m), m tracked in that unit,
//     and the accumulator is rescaled only when a row's max grows by > 2^4;
//   * the row sum l is taken over exactly the rounded P that multiplies V
//     (packed dot products with (1, 1) on the vector ALU);
//   * an optional linear position bias (ALiBi) is added to the scaled scores of
//     each tile before its row max, in a compile-time variant of the kernel;
//   * causal: workgroups are launched heaviest (last query tiles) first, a wave
//     skips KV tiles that lie wholly after its rows (or, with a window, wholly
//     before them), and the element mask is applied on edge tiles only;
//   * packed variable-length batches: a workgroup past its sequence's end
//     returns at once; every sequence has its own key offset;
//   * work items run KV group by KV group, and within a group query tile by
//     query tile with the group's heads side by side; each XCD takes a
//     contiguous run of them, so the heads that stream the same K/V rows do
//     so at the same time through one L2.
#include "fa_common.hpp"
#include "fa_kernels.hpp"
#include "fa_seq.hpp"

namespace fa {

// Lazy rescale threshold (log2 units): the running reference m only moves
// when some row's maximum grows by more than this, so p <= 2^kRescaleLog2.
// The row sum l is taken from the same dtype-rounded P that multiplies V, so
// O = sum(P~ V) / sum(P~) stays a consistent weighted average: with that, a
// threshold of 2^4 keeps the bf16 error of eager rescaling (measured on the
// long-context workload), while 2^8 with an unrounded l does not.
constexpr float kRescaleLog2 = 4.f;

// NG = 2: two groups of NW waves share the workgroup's query rows (waves w and
// w + NW own the same 32 rows) and take alternate KV stages, each with its own
// online-softmax state and its own pair of LDS buffers; at the end the second
// group's (m, l, O) is merged into the first's by the logsumexp identity,
// through LDS, in a fixed order.  This doubles the waves of a small grid
// (32 query rows per wave give one wave per SIMD at 8 heads of 4096 rows).
template <typename T, int HD, int BC, int BS, int NW, int NG, bool CAUSAL, bool WINDOW, bool ALIBI>
__global__ __launch_bounds__(NG * NW * 64, (sizeof(T) == 2 ? 2 : 1)) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ O,
    float* __restrict__ LSE, Problem pb, float c, int nqt) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;  // threads of one group
  static_assert(NG == 1 || (NG == 2 && NW == 4), "two groups of four waves");
  using Tile = RowTile<T, BC, HD>;   // the unit of the products: BC keys
  using Stage = RowTile<T, BS, HD>;  // the unit of the loads and barriers: BS keys
  constexpr int kSub = BS / BC;
  static_assert(BS % BC == 0 && BC % 16 == 0, "a stage is whole tiles; the swizzle repeats every 16 rows");
  // Two buffers laid out as K stage 0, K stage 1, V stage 0, V stage 1, and
  // the stage loop unrolled by two: a lane's K (or V) fragments of either
  // buffer are one register each plus a constant offset below 64 KiB.
  constexpr int kVOff = 2 * Stage::kElems;
  __shared__ __attribute__((aligned(16))) T lds[NG * 2 * kVOff];  // [group] K0, K1, V0, V1

  const int tid = threadIdx.x;
  const int w = NG == 1 ? tid >> 6 : (tid >> 6) & (NW - 1), lane = tid & 63, r = lane & 31, h = lane >> 5;
  const int grp = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / NW;  // the wave's group
  const int gtid = NG == 1 ? tid : tid & (NT - 1);                                                  // thread within it
  // work item: KV group major, then query tile (heaviest first), then the
  // group's heads; one XCD takes a contiguous run of work items
  const QTile wt = qtile_of<CAUSAL>(xcd_slice(blockIdx.x, gridDim.x), nqt, pb);
  const int b = wt.b, hq = wt.hq, qt = wt.qt;
  const Seq sv = seq_of(pb, b, hq, hq / (pb.Hq / pb.Hkv));
  const int i0 = qt * BR;
  if (i0 >= sv.sq) return;  // a shorter sequence of a packed batch: no rows here
  const T* Qh = Q + sv.q_row0 * HD;
  const T* Kh = K + sv.kv_row0 * HD;
  const T* Vh = V + sv.kv_row0 * HD;
  const int qw0 = i0 + 32 * w;
  const int myq = qw0 + r;
  const int off = sv.off;
  // linear position bias: the head's slope in log2 units (c s - a |i + off - j|
  // is then the score the softmax takes, already scaled)
  const float sl2 = ALIBI ? pb.alibi[hq] * kLog2e : 0.f;
  const float cs = ALIBI ? 1.f : c;

  // rows past the end read row sq-1: their results are never stored
  vec8<T> qf[HD / 16];
  const T* qrow = Qh + (size_t)min(myq, sv.sq - 1) * HD + 8 * h;
#pragma unroll
  for (int t = 0; t < HD / 16; ++t) qf[t] = load8<T>(qrow + 16 * t);

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int d = 0; d < HD / 32; ++d) oacc[d] = f32x16{};
  // Row sum of the rounded P that multiplies V.  16-bit: on the matrix core,
  // one 16x16x32 product per 16 keys with a constant 0/1 operand: read as
  // that product's B operand, a lane pair's P fragment gives output row 0
  // the keys of query n and row 1 those of query n + 16 (n = lane % 16), so
  // lanes 0-15 accumulate every row's sum in rsum[0] and rsum[1].  (Summed
  // instead with packed dot products on the vector ALU, the 16-bit pairs wait
  // for the matrix core while its products run.)  fp32: each lane sums its
  // half of the keys on the vector ALU and the halves are added at the end.
  constexpr bool kRowSumMfma = sizeof(T) == 2;
  float lsum = 0.f;
  f32x4 rsum = {0.f, 0.f, 0.f, 0.f};
  vec8<T> sel;
  {
    const int n = lane & 15, j = (lane >> 4) & 1;
    const T v = (T)(((n == 0 && j == 0) || (n == 1 && j == 1)) ? 1.f : 0.f);
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = v;
  }
  float m = -INFINITY;

  // keys the workgroup's rows can see: [lo, hi)
  const int last = min(i0 + BR, sv.sq) - 1;
  const int hi = CAUSAL ? min(sv.skv, last + off + 1) : sv.skv;
  const int lo = WINDOW ? max(0, i0 + off - pb.window) : 0;
  const int jt0 = lo / BS;
  const int nstages = hi > lo ? (hi + BS - 1) / BS - jt0 : 0;

  // In 8-wave workgroups only waves 0-3 issue the K/V loads: a wave that
  // issues loads waits until the memory pipeline has taken them, and the
  // other wave of its SIMD keeps the matrix core busy meanwhile.
  constexpr int NTL = NW == 8 ? NT / 2 : NT;
  const bool loader = (__builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1)) < NTL / 64;
  LoopLoader<T, BS, HD, NTL> kld, vld;
  kld.init(gtid);
  vld.init(gtid);
  // a group takes stages grp, grp + NG, ... of the tile's range, in its own buffers
  T* const gl = lds + grp * 2 * kVOff;
  const int mine = NG == 1 ? nstages : nstages > grp ? (nstages - grp + NG - 1) / NG : 0;  // this group's stages
  const int steps = NG == 1 ? nstages : (nstages + NG - 1) / NG;                          // every group's loop count
  if (mine > 0 && loader) {
    kld.issue(Kh, (jt0 + grp) * BS, sv.skv, gl, gtid);
    vld.issue(Vh, (jt0 + grp) * BS, sv.skv, gl + kVOff, gtid);
    kld.land(gtid);
    vld.land(gtid);
  }
  __syncthreads();
  // Q has landed too (the loads above waited for it): a wait the compiler
  // sees says so, and it then places no waits for Q inside the loop, where
  // they would also wait for the loop's own assembly loads.
  __builtin_amdgcn_s_waitcnt(0);

  // The V stages' offset, opaque to the compiler: it then forms each lane's V
  // addresses once and reaches every V tile by a constant offset (a constant
  // of 64 KiB or more it folds into every address instead).
  int voff = kVOff;
  asm("" : "+s"(voff));
  // one KV stage: compute on `cur` while the next stage streams into `nxt`
  // (the K stages; each V stage sits kVOff further on).
  // The waves synchronise once per stage; within it each wave runs through
  // the stage's tiles at its own pace.
  auto stage = [&](const int li, const T* cur, T* nxt) __attribute__((always_inline)) {
    const int s0 = (jt0 + li * NG + grp) * BS;
    const bool more = li + 1 < mine;
    if (more && loader) {  // the other buffer was last read before the previous barrier
      kld.issue(Kh, s0 + NG * BS, sv.skv, nxt, gtid);
      vld.issue(Vh, s0 + NG * BS, sv.skv, nxt + kVOff, gtid);
    }
    // (a group with one stage fewer sits out the last step)
#pragma unroll
    for (int sub = 0; sub < kSub && (NG == 1 || li < mine); ++sub) {
      const int j0 = s0 + sub * BC;
      const T* Ks = cur + sub * Tile::kElems;
      const T* Vs = cur + voff + sub * Tile::kElems;
      // does any of this wave's rows see a key of the tile?
      const bool active = j0 < hi && (!CAUSAL || j0 <= qw0 + 31 + off) &&
                          (!WINDOW || j0 + BC - 1 >= qw0 + off - pb.window);
      if (active) {
        // S^T (BC x 32) = K_tile Q_w^T; the key blocks' accumulation chains are
        // interleaved so each pair of LDS reads feeds two independent products,
        // and each step's reads are issued one step ahead of its products
        f32x16 s[BC / 32];
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < HD / 16; ++t)
#pragma unroll
          for (int kb = 0; kb < BC / 32; ++kb) s[kb] = mma<T>(Tile::frag(Ks, 32 * kb + r, 16 * t, h), qf[t], s[kb]);
        if constexpr (sizeof(T) == 2) {
          // order: the fragments of step t+1 are read before the products of
          // step t (one 16-byte LDS read and one product per fragment)
          __builtin_amdgcn_sched_group_barrier(0x100, BC / 32, 0);  // LDS reads
#pragma unroll
          for (int t = 0; t < HD / 16 - 1; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x100, BC / 32, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, BC / 32, 0);  // matrix products
          }
          __builtin_amdgcn_sched_group_barrier(0x008, BC / 32, 0);
        }
        // invisible keys (causal / window / past the end) get -inf
        const bool edge = (CAUSAL && j0 + BC - 1 > qw0 + off) ||
                          (WINDOW && j0 < qw0 + 31 + off - pb.window) || (j0 + BC > sv.skv);
        if (edge) {
          // key j0 + 4h + e (e a constant per register) is visible to row myq
          // when e < e_end, e <= e_diag (causal) and e >= e_win (window): the
          // rule of key_visible with the lane's terms taken out once
          const int base = j0 + 4 * h;
          const int e_end = sv.skv - base, e_diag = myq + off - base, e_win = myq + off - pb.window - base;
#pragma unroll
          for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int e = 32 * kb + 8 * (i >> 2) + (i & 3);
              const bool vis = e < e_end && (!CAUSAL || e <= e_diag) && (!WINDOW || e >= e_win);
              s[kb][i] = vis ? s[kb][i] : -INFINITY;
            }
        }
        if constexpr (ALIBI) {
          // key j0 + 32kb + 4h + e of register i (e = 8(i/4) + i%4) is
          // |myq + off - j| keys from the lane's diagonal
          const float dl = (float)(myq + off - j0 - 4 * h);
#pragma unroll
          for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              s[kb][i] = fmaf(s[kb][i], c, -sl2 * fabsf(dl - (float)(32 * kb + 8 * (i >> 2) + (i & 3))));
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = wave_xor32_max(mx) * cs;
        // Move the reference only when a row's max outgrows it by 2^4 (any lane:
        // the branch is wave-uniform).  O = acc / l is exact for any reference.
        if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleLog2) != 0) {
          const float m_new = fmaxf(m, mx);
          // a row that has seen no key keeps m = -inf and alpha = 1
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
          lsum *= alpha;
          if constexpr (kRowSumMfma) {
            // rsum[1] of lane n holds query n + 16's sum: its factor is lane n + 16's
            const float a16 = __shfl_xor(alpha, 16);
            rsum[0] *= alpha;
            rsum[1] *= a16;
          }
#pragma unroll
          for (int d = 0; d < HD / 32; ++d) oacc[d] *= alpha;
          m = m_new;
        }
        const float ref = (m == -INFINITY) ? 0.f : m;  // a row with no key yet keeps p = 0
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], cs, -ref));
        // O^T (HD x 32) += V_tile^T P^T ; l += sum of the lane's P
#pragma unroll
        for (int kt = 0; kt < BC / 16; ++kt) {
          const vec8<T> pf = acc_to_frag<T>(s[kt >> 1], 8 * (kt & 1));
#pragma unroll
          for (int d = 0; d < HD / 32; ++d) oacc[d] = mma<T>(Tile::tr_frag(Vs, kt, 32 * d, lane), pf, oacc[d]);
          if constexpr (kRowSumMfma)
            rsum = row_sum_mma<T>(sel, pf, rsum);
          else
            lsum = frag_sum(pf, lsum);
        }
        if constexpr (kRowSumMfma) {
          // the transposed V reads of 16-key step kt+1 before the four PV
          // products and the row-sum product of step kt (left to itself, the
          // compiler put a stage's row-sum products at its end, one dependent
          // chain, holding every P fragment of the stage until then)
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (HD / 32), 0);  // LDS reads
#pragma unroll
          for (int kt = 0; kt < BC / 16 - 1; ++kt) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * (HD / 32), 0);
            __builtin_amdgcn_sched_group_barrier(0x008, HD / 32 + 1, 0);  // matrix products
          }
          __builtin_amdgcn_sched_group_barrier(0x008, HD / 32 + 1, 0);
        }
      }
    }
    if (more && loader) {
      kld.land(gtid);
      vld.land(gtid);
    }
    __syncthreads();
  };
  for (int li = 0; li < steps; li += 2) {
    stage(li, gl, gl + Stage::kElems);
    if (li + 1 < steps) stage(li + 1, gl + Stage::kElems, gl);
  }

  if constexpr (kRowSumMfma) {
    // every lane of a row pair takes its query's whole sum (the merge below is
    // linear in it)
    const int src = r & 15;
    const float s0 = __shfl(rsum[0], src), s1 = __shfl(rsum[1], src);
    lsum = r < 16 ? s0 : s1;
  }
  if constexpr (NG == 2) {
    // the second group's reference, lane sum and accumulators, through the
    // (now free) stage buffers; the first group rescales both to the larger
    // reference and adds them
    static_assert(NW * (HD / 32 + 1) * 16 * 64 * 4 <= (int)sizeof(lds), "a group's state fits the stage buffers");
    f32x4* xf = reinterpret_cast<f32x4*>(lds);
    const int base = w * (HD / 32 * 4 + 1) * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int d = 0; d < HD / 32; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xf[base + (d * 4 + g) * 64] = f32x4{oacc[d][4 * g], oacc[d][4 * g + 1], oacc[d][4 * g + 2], oacc[d][4 * g + 3]};
      xf[base + HD / 32 * 4 * 64] = f32x4{m, lsum, 0.f, 0.f};
    }
    __syncthreads();
    if (grp == 1) return;
    const f32x4 ml = xf[base + HD / 32 * 4 * 64];
    const float mm = fmaxf(m, ml[0]);
    // a group that saw no key of these rows has m = -inf and weight 0
    const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mm);
    const float a1 = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - mm);
    lsum = lsum * a0 + ml[1] * a1;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = xf[base + (d * 4 + g) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[d][4 * g + e] = oacc[d][4 * g + e] * a0 + x[e] * a1;
      }
    m = mm;
  }

  const float l = kRowSumMfma ? lsum : wave_xor32_sum(lsum);
  // a row that saw no key has an empty softmax: O = 0, L = -inf
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if constexpr (sizeof(T) == 2 && !WINDOW && !ALIBI) {
    // O rows leave through LDS, free once every wave has passed the last
    // stage's barrier (with two groups: past the merge state).  The window and
    // bias kernels store straight from the accumulators: they have no
    // registers to spare for it.
    constexpr int kStg = NG == 1 ? 0 : NW * (HD / 32 * 4 + 1) * 64 * 16 / (int)sizeof(T);
    static_assert(kStg + NW * 32 * HD <= (int)(sizeof(lds) / sizeof(T)), "the output rows fit the stage buffers");
    store_block_rows<T, HD>(oacc, inv, lds + kStg + w * 32 * HD, O + (sv.q_row0 + qw0) * HD, sv.sq - qw0, lane);
    if (LSE != nullptr && h == 0 && myq < sv.sq) LSE[sv.q_row0 + myq] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  } else if (myq < sv.sq) {
    T* Or = O + (sv.q_row0 + myq) * HD;
#pragma unroll
    for (int d = 0; d < HD / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<T>(Or + 32 * d + 8 * g + 4 * h, oacc[d][4 * g] * inv, oacc[d][4 * g + 1] * inv,
                  oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv);
    if (LSE != nullptr && h == 0) LSE[sv.q_row0 + myq] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <typename T, int HD, int NW, int NG, bool CAUSAL, bool WINDOW, bool ALIBI>
static void launch_fwd_nw(const FwdArgs& a, hipStream_t st) {
  // 8-wave workgroups (one per CU) load, synchronise and compute per 128 keys,
  // in two buffers of up to 64 KiB; 4-wave ones (two per CU) per 64 keys.  A
  // 128-key tile takes one row max, exchange and rescale test per 128 keys.
  // At D = 64, where the softmax outweighs the products, two-group workgroups
  // (one per CU) take 128-key tiles too: measured +10 % on the fp16
  // [1, 8, 4096, 64] forward, while one-group 4-wave workgroups lose 2-3 %
  // with them.
  constexpr int BS = (sizeof(T) == 2 && (NW == 8 || (HD == 64 && NG == 2))) ? 128 : 64, BC = BS, BR = 32 * NW;
  const int nqt = (a.pb.Sq + BR - 1) / BR;
  dim3 grid(nqt * a.pb.B * a.pb.Hq), block(NG * NW * 64);
  if (grid.x > 0)
    hipLaunchKernelGGL((fwd_kernel<T, HD, BC, BS, NW, NG, CAUSAL, WINDOW, ALIBI>), grid, block, 0, st, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, (T*)a.o, a.lse, a.pb, a.scale * kLog2e, nqt);
}

template <typename T, int HD, bool CAUSAL, bool WINDOW, bool ALIBI>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  mark(a.ev, a.nev, 0, st);
  // 16-bit: workgroups of 8 waves (256 query rows; one fits a CU at a time)
  // share each K/V tile among twice the waves.  Measured: at D = 128 they are
  // faster from one workgroup per CU up when the queries fill their rows
  // (S = 4096 to 16384, and B = 4 at S = 2048); otherwise (D = 64, short
  // query blocks) only when they fill the GPU several times over.
  bool wide = false;
  if constexpr (sizeof(T) == 2) {  // fp32 keeps 4-wave workgroups (no 8-wave instances)
    const long long n8 = (long long)((a.pb.Sq + 255) / 256) * a.pb.B * a.pb.Hq;
    wide = n8 >= ((HD == 128 && a.pb.Sq >= 256) ? kCUs : kWideGrid);
    if (wide) launch_fwd_nw<T, HD, 8, 1, CAUSAL, WINDOW, ALIBI>(a, st);
  }
  if (!wide) {
    // 16-bit grids of one 4-wave workgroup per CU or fewer: two wave groups per
    // workgroup split each tile's KV stages (two waves per SIMD instead of one)
    bool split = false;
    if constexpr (sizeof(T) == 2) {
      const long long n4 = (long long)((a.pb.Sq + 127) / 128) * a.pb.B * a.pb.Hq;
      split = n4 <= kCUs;
      if (split) launch_fwd_nw<T, HD, 4, 2, CAUSAL, WINDOW, ALIBI>(a, st);
    }
    if (!split) launch_fwd_nw<T, HD, 4, 1, CAUSAL, WINDOW, ALIBI>(a, st);
  }
  mark(a.ev, a.nev, 1, st);
  return hipGetLastError();
}

template <typename T, int HD, bool ALIBI>
static hipError_t launch_fwd_m(const FwdArgs& a, hipStream_t st) {
  if (a.pb.window >= 0)
    return a.pb.causal ? launch_fwd_t<T, HD, true, true, ALIBI>(a, st) : launch_fwd_t<T, HD, false, true, ALIBI>(a, st);
  return a.pb.causal ? launch_fwd_t<T, HD, true, false, ALIBI>(a, st) : launch_fwd_t<T, HD, false, false, ALIBI>(a, st);
}

template <typename T, int HD>
static hipError_t launch_fwd_b(const FwdArgs& a, hipStream_t st) {
  return a.pb.alibi != nullptr ? launch_fwd_m<T, HD, true>(a, st) : launch_fwd_m<T, HD, false>(a, st);
}

template <typename T>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t st) {
  return a.D == 64 ? launch_fwd_b<T, 64>(a, st) : launch_fwd_b<T, 128>(a, st);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case 0: return launch_fwd_d<float>(a, st);
    case 1: return launch_fwd_d<_Float16>(a, st);
    default: return launch_fwd_d<__bf16>(a, st);
  }
}

}  // namespace fa
