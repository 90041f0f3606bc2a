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

#include <type_traits>

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

// acc + the sum of a fragment's 8 elements, in fp32.  16-bit types use the
// packed dot product with (1, 1), so the sum is over exactly the rounded
// values the matrix product consumes.
__device__ inline float frag_sum(const vec8<__bf16>& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), one, acc, false);
}
__device__ inline float frag_sum(const vec8<_Float16>& f, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(f, f, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(f, f, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(f, f, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2(__builtin_shufflevector(f, f, 6, 7), one, acc, false);
}
__device__ inline float frag_sum(const vec8<float>& f, float acc) {
  return acc + (((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7])));
}

// acc += sel * p as a 16x16x32 product (16-bit operands, fp32 accumulation):
// the row sums of fwd_kernel's rounded P, with its constant 0/1 selector.
template <typename T>
__device__ inline f32x4 row_sum_mma(const vec8<T>& sel, const vec8<T>& p, f32x4 acc) {
  if constexpr (std::is_same<T, __bf16>::value)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p, acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(sel, p, acc, 0, 0, 0);
}

// Workgroup order for MI355X's 8 XCDs.  The dispatcher hands consecutive
// workgroup ids to the XCDs round-robin (id % 8), and each XCD has its own L2.
// Returns the work item a workgroup should take so that XCD x processes the
// contiguous slice [x*N/8, (x+1)*N/8) of a work list ordered by reuse (all
// tiles of one head or KV group together), in list order.  A bijection on
// [0, N); the last N % 8 ids keep their own index.
__device__ inline int xcd_slice(int id, int n) {
  const int per = n >> 3;
  if (id >= (per << 3)) return id;
  return (id & 7) * per + (id >> 3);
}

// Combine a value with the one in lane l ^ 32: gfx950's permlane32 swap
// exchanges the two wave halves in registers (no LDS round trip).
__device__ inline float2 wave_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wave_xor32_max(float x) {
  const float2 p = wave_halves(x);
  return fmaxf(p.x, p.y);
}
__device__ inline float wave_xor32_sum(float x) {
  const float2 p = wave_halves(x);
  return p.x + p.y;
}

// ------------------------------------------------------------------ LDS tiles
// Row tile: ROWS x HD elements, row-major.
//
// 16-bit elements: rows are packed (stride HD) and the 16-byte chunks of each
// row are XOR-swizzled, physical chunk = chunk ^ swz(row).  With 64 banks of
// 4 bytes, 16-byte accesses served 16 lanes at a time and 8-byte (and
// transpose) accesses 32 lanes at a time, this makes every access pattern the
// kernels use conflict-free: a row fragment (16 consecutive rows, one chunk),
// a transpose read (4 consecutive rows, an aligned quad of chunks) and a
// staging store (whole rows).  A plain 16-byte row padding leaves the
// transpose reads 4-way conflicted.
//   256-byte rows (16 chunks): swz = 4 (row & 3) + ((row >> 2) & 3)
//   128-byte rows ( 8 chunks): swz = 4 ((row >> 1) & 1) + ((row >> 2) & 3)
// fp32 elements: rows padded by 16 bytes, no swizzle.
template <typename T, int ROWS, int HD>
struct RowTile {
  static constexpr bool kSwizzle = sizeof(T) == 2;
  static constexpr int kChunks = HD * (int)sizeof(T) / 16;
  static constexpr int kEpc = 16 / (int)sizeof(T);  // elements per chunk
  static constexpr int kStride = kSwizzle ? HD : HD + kEpc;
  static constexpr int kElems = ROWS * kStride;
  static_assert(!kSwizzle || kChunks == 16 || kChunks == 8, "swizzle defined for 128/256-byte rows");

  __device__ static inline int swz(int row) {
    if constexpr (kChunks == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
  // element offset of (row, col); col's chunk is swizzled, its offset within
  // the chunk is kept
  __device__ static inline int at(int row, int col) {
    if constexpr (kSwizzle) {
      const int ch = col / kEpc;
      return row * kStride + ((ch ^ swz(row)) * kEpc) + (col % kEpc);
    } else {
      return row * kStride + col;
    }
  }
  // A or B fragment with the tile's rows as the fragment rows / columns and the
  // tile's columns as contraction index: row `row`, columns c0 + 8h + j.
  __device__ static inline vec8<T> frag(const T* base, int row, int c0, int h) {
    return load8<T>(base + at(row, c0 + 8 * h));
  }
  __device__ static inline void put_unit(T* base, int row, int col, Unit<T> u) {
    *reinterpret_cast<u32x4*>(base + at(row, col)) = u.bits;
  }
  // Transposed fragment: the tile's rows are the contraction index and its
  // columns the fragment rows.  Lane l = 32h + r receives, for contraction step
  // kt, X[16kt + 8(j/4) + 4h + (j%4)][col0 + r] in slot j -- the indices that
  // accumulator registers 8(kt%2)..8(kt%2)+7 of a 32x32 tile hold for lane
  // half h, so it pairs with acc_to_frag().
  __device__ static inline vec8<T> tr_frag(const T* base, int kt, int col0, int lane);
};

// 16-bit elements: gfx950's LDS transpose read.  Within each group of 16
// lanes, lane j supplies the address of X[R0 + j/4][C0 + 4(j%4)] (4 elements)
// and lane i receives X[R0 + k][C0 + i], k = 0..3.  Two reads (rows R0 and
// R0 + 8) make one 8-slot fragment.
typedef short s16x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ inline vec4<T> lds_tr4(const T* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(vec4<T>, v);
}

template <typename T, int ROWS, int HD>
__device__ inline vec8<T> RowTile<T, ROWS, HD>::tr_frag(const T* base, int kt, int col0, int lane) {
  if constexpr (sizeof(T) == 2) {
    // the swizzle reads row bits 0..3 only: the lane's place within a group of
    // 16 rows is the same for every kt, which then is a constant offset
    const int x = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const T* g = base + 16 * kt * kStride;
    vec4<T> a = lds_tr4<T>(g + at(x, col));
    vec4<T> b = lds_tr4<T>(g + at(x + 8, col));
    return vec8<T>{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    // fp32: eight scalar reads (only the small fp32 workloads take this path)
    const int h = lane >> 5, r = lane & 31;
    vec8<T> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = base[at(16 * kt + 4 * h + 8 * (j >> 2) + (j & 3), col0 + r)];
    return f;
  }
}

// ------------------------------------------------------------------ global -> LDS staging
// A tile of ROWS rows x HD columns of a row-major [S][HD] matrix.  Rows at or
// beyond `nvalid` are loaded from row nvalid - 1 instead (every kernel masks
// those rows' scores or never stores their results), so loads need no
// branches.  Each thread moves whole 16-byte units through registers: load()
// issues the global loads, store_rows() writes them to a RowTile.
template <typename T, int ROWS, int HD, int NT>
struct Stager {
  static constexpr int kEpv = Elem<T>::kEpv;
  static constexpr int kUnitsPerRow = HD / kEpv;
  static constexpr int kUnits = ROWS * kUnitsPerRow;
  static constexpr int kPerThread = (kUnits + NT - 1) / NT;
  Unit<T> u[kPerThread];

  __device__ inline void load(const T* __restrict__ g, int row0, int nvalid, int tid) {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int unit = tid + p * NT;
      if (kUnits % NT == 0 || unit < kUnits) {
        const int row = min(row0 + unit / kUnitsPerRow, nvalid - 1);
        const int col = (unit % kUnitsPerRow) * kEpv;
        u[p] = load_unit<T>(g + (size_t)row * HD + col);
      }
    }
  }

  __device__ inline void store_rows(T* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < kPerThread; ++p) {
      const int unit = tid + p * NT;
      if (kUnits % NT == 0 || unit < kUnits)
        RowTile<T, ROWS, HD>::put_unit(lds, unit / kUnitsPerRow, (unit % kUnitsPerRow) * kEpv, u[p]);
    }
  }
};

// ------------------------------------------------------------------ tile loader
// Moves a ROWS x HD tile of a row-major [S][HD] matrix into a RowTile.  Rows
// at or beyond `nvalid` read row nvalid - 1 (every kernel masks or discards
// them).  Interface: issue() starts the transfer into an LDS tile, land()
// completes it; the tile may be read after land() and a workgroup barrier.
//
// 16-bit elements use gfx950's direct global -> LDS loads (16 bytes per lane,
// no VGPR staging): instruction p of wave w writes LDS bytes
// [(p*NW + w)*1024, +1024) of the tile, lane l the 16 bytes at +16 l, so each
// lane loads the logical chunk that the swizzle places at its physical slot
// (a permutation within one row: the loads stay coalesced).  The data is in
// LDS once the wave's vector-memory counter drains, which the barrier's
// release fence waits for; land() has nothing to do.
// fp32 elements go through registers (Stager) into the padded tile.
template <typename T, int ROWS, int HD, int NT, bool DIRECT = (sizeof(T) == 2)>
struct TileLoader {
  Stager<T, ROWS, HD, NT> st;
  T* dst = nullptr;
  __device__ inline void init(int) {}
  __device__ inline void issue(const T* __restrict__ g, int row0, int nvalid, T* lds, int tid) {
    st.load(g, row0, nvalid, tid);
    dst = lds;
  }
  __device__ inline void land(int tid) { st.store_rows(dst, tid); }
};

template <typename T, int ROWS, int HD, int NT>
struct TileLoader<T, ROWS, HD, NT, true> {
  using Tile = RowTile<T, ROWS, HD>;
  static constexpr int kNW = NT / 64;
  static constexpr int kRowBytes = HD * 2;
  static constexpr int kInstr = ROWS * kRowBytes / (kNW * 1024);
  static constexpr int kRowsPerInstr = kNW * 1024 / kRowBytes;  // tile rows one instruction of all waves covers
  static_assert(ROWS * kRowBytes % (kNW * 1024) == 0, "tile must be whole 1 KiB wave slices");
  // The swizzle reads row bits 0..3 only, so with a multiple of 16 rows per
  // instruction a lane loads the same (swizzled) column in every instruction
  // and only its row advances: one 32-bit offset per lane serves them all,
  // and the per-instruction step is uniform.
  static_assert(kRowsPerInstr % 16 == 0, "per-instruction row step must keep the swizzle");
  uint32_t col;  // byte offset of this lane's logical 16-byte chunk within its row
  int row;       // tile row this lane loads in instruction 0
  int wslot;     // wave index (uniform)

  __device__ inline void init(int tid) {
    wslot = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int byte = wslot * 1024 + 16 * (tid & 63);
    row = byte / kRowBytes;
    const int pch = (byte % kRowBytes) / 16;
    col = (uint32_t)((pch ^ Tile::swz(row)) * 16);
  }
  __device__ inline void issue(const T* __restrict__ g, int row0, int nvalid, T* lds, int) {
    if (row0 + ROWS <= nvalid) {
      // uniform base (scalar registers) + one per-lane 32-bit offset
      const char* gb = reinterpret_cast<const char*>(g + (size_t)row0 * HD);
      const uint32_t off = (uint32_t)(row * kRowBytes) + col;
#pragma unroll
      for (int p = 0; p < kInstr; ++p)
        __builtin_amdgcn_global_load_lds((const void*)(gb + (size_t)p * kRowsPerInstr * kRowBytes + off),
                                         (__attribute__((address_space(3))) void*)(lds + (p * kNW + wslot) * 512),
                                         16, 0, 0);
    } else {
#pragma unroll
      for (int p = 0; p < kInstr; ++p) {
        const int r = min(row0 + row + p * kRowsPerInstr, nvalid - 1);
        __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(g) + (size_t)r * kRowBytes + col),
                                         (__attribute__((address_space(3))) void*)(lds + (p * kNW + wslot) * 512),
                                         16, 0, 0);
      }
    }
  }
  __device__ inline void land(int) {}
};

// The direct loads of TileLoader written as inline assembly, for tiles
// streamed inside a loop.  Seen by the compiler, direct loads cost twice:
//   * it makes an LDS read wait for every direct load still in flight unless
//     it can prove the two do not overlap, which it cannot when a kernel
//     picks its double buffer at run time (or reads other LDS tiles besides);
//   * with a direct load in a loop it no longer counts LDS reads one by one:
//     every wait for a fragment waits for all reads in flight, which undoes
//     reading fragments ahead of their products.
// It does not see these loads at all, so neither happens.  land() waits for
// them explicitly (vector memory completes in order, so a wait the compiler
// places for any load issued after them covers them too); the caller's
// barrier then publishes the tile.  The flip side: a wait the compiler places
// for a load issued before the loop (say, a fragment kept in registers)
// counts as if these loads did not exist, so it would also wait for them.
// Kernels therefore make every earlier load land before the loop with a wait
// the compiler sees (__builtin_amdgcn_s_waitcnt(0)).
template <typename T, int ROWS, int HD, int NT>
struct AsmTileLoader : TileLoader<T, ROWS, HD, NT, true> {
  using Base = TileLoader<T, ROWS, HD, NT, true>;
  using Base::col;
  using Base::row;
  using Base::wslot;
  static constexpr int kNW = Base::kNW, kInstr = Base::kInstr, kRowBytes = Base::kRowBytes;
  static constexpr int kRowsPerInstr = Base::kRowsPerInstr;

  // LDS byte address of this wave's 1 KiB slice of instruction p (uniform),
  // handed to each load in M0 through the "{m0}" operand, so the compiler
  // itself sets M0 and knows its value.
  //
  // Each load starts with 5 wait states (s_nop 4).  A vector memory
  // instruction that reads an SGPR written by a VALU instruction (the
  // compiler reloads spilled scalars with v_readlane) needs 5 of them, and
  // one that reads M0 after a scalar write of it needs 1.  The compiler
  // inserts these for its own memory instructions but cannot see that the
  // assembly is one, so the assembly provides them itself; without them the
  // load can take a stale base address.
  __device__ static inline uint32_t slice(T* lds, int p, int w) {
    const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) T*)lds);
    return __builtin_amdgcn_readfirstlane(base + (uint32_t)((p * kNW + w) * 1024));
  }
  __device__ inline void issue(const T* g, int row0, int nvalid, T* lds, int) {
    if (row0 + ROWS <= nvalid) {
      const char* gb = reinterpret_cast<const char*>(g + (size_t)row0 * HD);
      const uint32_t off = (uint32_t)(row * kRowBytes) + col;
#pragma unroll
      for (int p = 0; p < kInstr; ++p) {
        const char* src = gb + (size_t)p * kRowsPerInstr * kRowBytes;
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                     :
                     : "v"(off), "s"(src), "{m0}"(slice(lds, p, wslot))
                     : "memory");
      }
    } else {
#pragma unroll
      for (int p = 0; p < kInstr; ++p) {
        const int r = min(row0 + row + p * kRowsPerInstr, nvalid - 1);
        const char* src = reinterpret_cast<const char*>(g) + (size_t)r * kRowBytes + col;
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src), "{m0}"(slice(lds, p, wslot))
                     : "memory");
      }
    }
  }
  __device__ inline void land(int) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
};

// Loader for tiles streamed inside a loop: the assembly form for 16-bit
// elements, register staging for fp32.
template <typename T, int ROWS, int HD, int NT>
using LoopLoader = typename std::conditional<sizeof(T) == 2, AsmTileLoader<T, ROWS, HD, NT>,
                                             TileLoader<T, ROWS, HD, NT>>::type;

// Stores 4 consecutive output elements (fp32 values) at p.
template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  vec4<T> v{to_elem<T>(a), to_elem<T>(b), to_elem<T>(c), to_elem<T>(d)};
  *reinterpret_cast<vec4<T>*>(p) = v;
}

// Writes a wave's 32 x HD output block, held as 32x32 accumulators (lane
// 32h + r: row r, columns 32d + 8g + 4h .. + 3 in acc[d][4g .. 4g + 3]), times
// the lane's factor `mul`, to rows out[0 .. valid) (row stride HD) through a
// private LDS region of 32 * HD elements.  Stored straight from the
// accumulators, every store instruction would write 8 bytes in each of 32
// rows; through LDS each writes whole rows, 16 bytes per lane.  The region is
// laid out as a swizzled row tile, so the 32 rows of one column group fall in
// different banks.  16-bit types only; the wave must be the region's only user.
template <typename T, int HD>
__device__ inline void store_block_rows(const f32x16 (&acc)[HD / 32], float mul, T* stg, T* out, int valid,
                                        int lane) {
  static_assert(sizeof(T) == 2, "16-bit outputs");
  using Blk = RowTile<T, 32, HD>;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int d = 0; d < HD / 32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4<T>(stg + Blk::at(r, 32 * d + 8 * g + 4 * h), acc[d][4 * g] * mul, acc[d][4 * g + 1] * mul,
                acc[d][4 * g + 2] * mul, acc[d][4 * g + 3] * mul);
  // the wave reads back what its other lanes wrote: its LDS accesses complete
  // in program order, and the fences keep the compiler from moving them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kLanesPerRow = HD * (int)sizeof(T) / 16;
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
  const int pr = lane / kLanesPerRow, pc = (lane % kLanesPerRow) * 8;
#pragma unroll
  for (int i = 0; i < 32 / kRowsPerPass; ++i) {
    const int row = pr + kRowsPerPass * i;
    const vec8<T> x = load8<T>(stg + Blk::at(row, pc));
    if (row < valid) *reinterpret_cast<vec8<T>*>(out + (size_t)row * HD + pc) = x;
  }
}

}  // namespace fa
