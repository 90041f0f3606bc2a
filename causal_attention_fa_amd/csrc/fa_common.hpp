// fa_common.hpp -- device building blocks shared by the attention kernels (gfx950).
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA family, wave64):
//   * A operand (M x K) and B operand (K x N): lane l carries row / column l % 32;
//     within one 16-wide step of the contraction index, lane half h = l / 32
//     carries contraction indices 16*t + 8*h + j in slots j = 0..7.  Only the
//     pairing of A and B slots matters for the sum, so any layout of the
//     contraction index works as long as both operands use the same one.
//   * Accumulator (32 x 32, f32x16): register i of lane l holds
//     row 8*(i/4) + 4*h + (i%4), column l % 32.
// So a wave owns 32 "columns" (one per lane pair l, l+32) and every per-column
// statistic (softmax max / sum of one query row, say) lives in one lane pair.
//
// Element types: bf16 and fp16 use the 32x32x16 MFMAs (8 values per lane per
// step); fp32 uses eight 32x32x2 fp32 MFMAs per step (slot j of both halves
// forms one 2-deep product), so fp32 inputs are multiplied in true fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
using vec8 = T __attribute__((ext_vector_type(8)));
template <typename T>
using vec4 = T __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ element traits
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static constexpr int kEpv = 8;  // elements per 16-byte vector
  __device__ static inline f32x16 mma(vec8<__bf16> a, vec8<__bf16> b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Elem<_Float16> {
  static constexpr int kEpv = 8;
  __device__ static inline f32x16 mma(vec8<_Float16> a, vec8<_Float16> b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Elem<float> {
  static constexpr int kEpv = 4;
  __device__ static inline f32x16 mma(vec8<float> a, vec8<float> b, f32x16 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
};

template <typename T>
__device__ inline f32x16 mma(vec8<T> a, vec8<T> b, f32x16 c) {
  return Elem<T>::mma(a, b, c);
}

// ------------------------------------------------------------------ vector moves
// 16-byte unit: kEpv elements.
template <typename T>
struct Unit {
  u32x4 bits;
};

template <typename T>
__device__ inline Unit<T> load_unit(const T* p) {
  return Unit<T>{*reinterpret_cast<const u32x4*>(p)};
}
template <typename T>
__device__ inline Unit<T> zero_unit() {
  return Unit<T>{u32x4{0u, 0u, 0u, 0u}};
}

// 8 consecutive elements starting at p (16-byte aligned).
template <typename T>
__device__ inline vec8<T> load8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const vec8<T>*>(p);
  } else {
    f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    return vec8<T>{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Two runs of 4 consecutive elements (p0[0..3], p1[0..3]) as one fragment.
template <typename T>
__device__ inline vec8<T> load4x2(const T* p0, const T* p1) {
  vec4<T> a = *reinterpret_cast<const vec4<T>*>(p0);
  vec4<T> b = *reinterpret_cast<const vec4<T>*>(p1);
  return vec8<T>{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename T>
__device__ inline vec8<T> zero8() {
  return vec8<T>{};
}

// fp32 -> T, round to nearest even.
template <typename T>
__device__ inline T to_elem(float x) {
  return static_cast<T>(x);
}

// Slots j = 0..7 of a B fragment taken from accumulator registers base..base+7.
template <typename T>
__device__ inline vec8<T> acc_to_frag(const f32x16& acc, int base) {
  vec8<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = to_elem<T>(acc[base + j]);
  return f;
}

__device__ inline float wave_xor32_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ inline float wave_xor32_sum(float x) { return x + __shfl_xor(x, 32); }

// ------------------------------------------------------------------ LDS tiles
// Row tile: ROWS x HD elements, row stride HD + 16 bytes of padding so that the
// 32 rows read by one A-fragment load fall in different banks.
template <typename T, int ROWS, int HD>
struct RowTile {
  static constexpr int kStride = HD + 16 / (int)sizeof(T);
  static constexpr int kElems = ROWS * kStride;
  // A fragment: rows `row`, contraction (column) indices c0 + 8h + j.
  __device__ static inline vec8<T> frag(const T* base, int row, int c0, int h) {
    return load8<T>(base + row * kStride + c0 + 8 * h);
  }
  __device__ static inline void put_unit(T* base, int row, int col, Unit<T> u) {
    *reinterpret_cast<u32x4*>(base + row * kStride + col) = u.bits;
  }
};

// Transposed tile: holds X^T for an X of COLS rows and HD columns, i.e. HD rows
// of COLS elements (+4 elements of padding).  An A fragment of X^T for
// contraction step kt reads, at row d, the runs [16kt + 4h, +4) and
// [16kt + 8 + 4h, +4): exactly the indices that accumulator registers
// 8*(kt%2) .. 8*(kt%2)+7 of a 32x32 tile hold for lane half h.
template <typename T, int HD, int COLS>
struct TrTile {
  static constexpr int kStride = COLS + 4;
  static constexpr int kElems = HD * kStride;
  __device__ static inline vec8<T> frag(const T* base, int d, int kt, int h) {
    const T* p = base + d * kStride + 16 * kt + 4 * h;
    return load4x2<T>(p, p + 8);
  }
};

// ------------------------------------------------------------------ global -> LDS staging
// A tile of ROWS rows x HD columns of a row-major [S][HD] matrix, rows at or
// beyond `nvalid` read as zero.  Work unit: 4 rows x kEpv columns (four 16-byte
// loads per unit).  The same registers can be written to a RowTile, a TrTile,
// or both.
template <typename T, int ROWS, int HD, int NT>
struct Stager {
  static constexpr int kEpv = Elem<T>::kEpv;
  static constexpr int kUnitsPerRowGroup = HD / kEpv;
  static constexpr int kUnits = (ROWS / 4) * kUnitsPerRowGroup;
  static constexpr int kPerThread = (kUnits + NT - 1) / NT;
  static_assert(ROWS % 4 == 0, "rows in groups of 4");
  Unit<T> u[kPerThread][4];

  __device__ inline void load(const T* __restrict__ g, int row0, int nvalid, int tid) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int unit = tid + p * NT;
      if (kUnits % NT == 0 || unit < kUnits) {
        const int rg = unit / kUnitsPerRowGroup;
        const int col = (unit % kUnitsPerRowGroup) * kEpv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = row0 + 4 * rg + rr;
          u[p][rr] = row < nvalid ? load_unit<T>(g + (size_t)row * HD + col) : zero_unit<T>();
        }
      }
    }
  }

  __device__ inline void store_rows(T* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int unit = tid + p * NT;
      if (kUnits % NT == 0 || unit < kUnits) {
        const int rg = unit / kUnitsPerRowGroup;
        const int col = (unit % kUnitsPerRowGroup) * kEpv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) RowTile<T, ROWS, HD>::put_unit(lds, 4 * rg + rr, col, u[p][rr]);
      }
    }
  }

  // Transposed store: column c of the unit becomes LDS row (col + c), and the
  // unit's 4 rows become 4 consecutive elements of that row.
  __device__ inline void store_transposed(T* lds, int tid) const {
    constexpr int kStride = TrTile<T, HD, ROWS>::kStride;
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int unit = tid + p * NT;
      if (kUnits % NT == 0 || unit < kUnits) {
        const int rg = unit / kUnitsPerRowGroup;
        const int col = (unit % kUnitsPerRowGroup) * kEpv;
        if constexpr (sizeof(T) == 2) {
          // 16-bit elements: element c of row rr is half (c & 1) of word c/2.
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int w = c >> 1;
            const int sh = (c & 1) * 16;
            const uint32_t e0 = (u[p][0].bits[w] >> sh) & 0xFFFFu;
            const uint32_t e1 = (u[p][1].bits[w] >> sh) & 0xFFFFu;
            const uint32_t e2 = (u[p][2].bits[w] >> sh) & 0xFFFFu;
            const uint32_t e3 = (u[p][3].bits[w] >> sh) & 0xFFFFu;
            u32x2 packed{e0 | (e1 << 16), e2 | (e3 << 16)};
            *reinterpret_cast<u32x2*>(lds + (col + c) * kStride + 4 * rg) = packed;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x4 packed{u[p][0].bits[c], u[p][1].bits[c], u[p][2].bits[c], u[p][3].bits[c]};
            *reinterpret_cast<u32x4*>(lds + (col + c) * kStride + 4 * rg) = packed;
          }
        }
      }
    }
  }
};

// Stores 4 consecutive output elements (fp32 values) at p.
template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  vec4<T> v{to_elem<T>(a), to_elem<T>(b), to_elem<T>(c), to_elem<T>(d)};
  *reinterpret_cast<vec4<T>*>(p) = v;
}

}  // namespace fa
