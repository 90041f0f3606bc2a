// fa_problem.hpp -- the attention problem as the kernels see it: dense batches
// ([B][H][S][D]) or packed variable-length batches ([H][T][D] with cumulative
// sequence offsets), queries and keys of different lengths, an optional left
// window, an optional linear position bias.  Plain data, shared by the host
// code and the kernels; the device-side helpers are in fa_seq.hpp.
#pragma once

namespace fa {

struct Problem {
  int B, Hq, Hkv;
  int Sq, Skv;        // dense: the lengths; packed: upper bounds of the per-sequence lengths
  int causal;         // key j visible to query i iff j <= i + (skv - sq)
  int window;         // < 0: none; else also j >= i + (skv - sq) - window
  const int* cu_q;    // packed: B + 1 cumulative query offsets (device); nullptr: dense
  const int* cu_k;
  int Tq, Tk;         // packed: rows per head slab of q/o/dq and of k/v/dk/dv
  const float* alibi; // linear position bias: one slope per query head (device), or nullptr
};

}  // namespace fa
