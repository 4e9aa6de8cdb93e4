// echo_internal.h -- types shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace echo {

constexpr int kMaxRanks = 16;

// element-type tags (same values as the ECHO_* constants of the public header)
constexpr int kInBF16 = 0, kInF16 = 1;
constexpr int kOutBF16 = 0, kOutF32 = 1;
constexpr int kStateF32 = 0, kStateBF16 = 1;

// Upper bound on blocks of the state-reset fill; larger arrays stride.
constexpr uint64_t kZeroGridCap = 1u << 20;

// Payload pointers of every segment, passed by value as kernel arguments.
struct SegTable {
  void* codes[kMaxRanks];
  uint32_t* params[kMaxRanks];
};

// Feedback gain and the two moving averages' keep/take weights.
struct Coef {
  float eta;
  float bS, aS;  // short memory: S = bS*S + aS*r
  float bL, aL;  // long memory:  L = bL*L + aL*r
};

struct LaunchArgs {
  int bits, group, in_dtype, out_dtype, state_dtype;
  int P, rank;
  uint64_t n;         // elements of the message
  uint64_t seg_len;   // elements per segment: ceil(ceil(n/P)/group)*group
  const void* x;
  void* state;   // interleaved short/long memories: state[2j] = S_j, state[2j+1] = L_j
  SegTable segs;
  void* out_codes;
  uint32_t* out_params;
  void* out;
  Coef coef;
};

// Each returns the first launch error (hipSuccess when every launch went out).
hipError_t run_quant_feedback(const LaunchArgs& a, hipStream_t st);
hipError_t run_owner_reduce_requant(const LaunchArgs& a, hipStream_t st);
hipError_t run_dequant_gather(const LaunchArgs& a, hipStream_t st);
hipError_t run_zero(void* p, uint64_t bytes, hipStream_t st);

}  // namespace echo
