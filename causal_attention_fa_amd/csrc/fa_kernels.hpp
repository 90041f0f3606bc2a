// fa_kernels.hpp -- internal launcher interface between the C ABI (fa_api.cpp)
// and the kernel files.  Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_problem.hpp"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Problem pb;
  int D;
  float scale;
  int dtype;  // 0 fp32, 1 fp16, 2 bf16 (fa_dtype_t)
  hipEvent_t* ev;  // optional timing events (fa_profile_events), nev of them
  int nev;
};

// Grids of at least this many 8-wave workgroups (8 per CU) run the dQ
// kernel (and the forward at D = 64) with 8 waves per workgroup; smaller ones
// use 4.
constexpr long long kWideGrid = 2048;
// compute units of an MI355X
constexpr long long kCUs = 256;

// Records ev[i] on the stream when instrumentation asked for it.
inline void mark(hipEvent_t* ev, int nev, int i, hipStream_t st) {
  if (ev != nullptr && i < nev) (void)hipEventRecord(ev[i], st);
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* rowdot;  // workspace: D[i] = sum_d dO[i,d] * O[i,d], one fp32 per query row
  Problem pb;
  int D;
  float scale;
  int dtype;
  hipEvent_t* ev;
  int nev;
};

// Split-KV forward: nsplit key ranges of `chunk` keys each (a multiple of
// split_tile_keys(dtype)); `work` holds nsplit * qrows * (D + 1) fp32 values
// (partial O rows, then partial L).
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* work;
  Problem pb;
  int D;
  float scale;
  int dtype;
  int nsplit;
  int chunk;
  long long qrows;
  hipEvent_t* ev;
  int nev;
};

// Device address, on the current device, of the static row-dot array behind
// fa_bwd_noalloc (kNoAllocRows fp32 values): looked up on the first request on
// each device and kept.
constexpr long long kNoAllocRows = 1LL << 22;
hipError_t noalloc_rowdot(float** ptr);

// Waves of a split-KV workgroup: 16-bit tiles of 128 keys over 4 waves; fp32
// tiles are twice the bytes (and padded), so 64 keys over 2 waves keep K and
// V double buffered in LDS.  Each wave takes 32 keys of a tile.
constexpr int split_waves(int dtype) { return dtype == 0 ? 2 : 4; }
// keys per split-kernel tile (the unit of a key range)
constexpr int split_tile_keys(int dtype) { return 32 * split_waves(dtype); }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_splitkv(const SplitArgs& a, hipStream_t stream);

}  // namespace fa
