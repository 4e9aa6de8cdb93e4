// echo_kernels.hip -- gfx950 kernels of one rank's share of an Echo all-reduce.
//
// Pages cited:
//   [JP-W] "テンソル並列の通信を4bitに圧縮する「Echo」" (Japanese explainer),
//          section "なぜ4bit通信は難しかったのか".
//   [JP-1] same page, section "Echoの仕組み①".
//   [JP-2] same page, section "Echoの仕組み②".
//   [JP-F] same page, section "よくある質問".
//
// The whole path streams HBM: per element it reads the 16-bit input and the
// two state words, writes the state back and moves sub-byte payloads.  There
// is no dense contraction, so no MFMA; what matters is full-width coalesced
// loads/stores and keeping every group's min/max reduction inside registers.
//
// Thread mapping shared by the entry pass and the owner pass: one group of
// 128 elements per half-wave (32 lanes), 4 consecutive elements per lane.
// A wave-wide dwordx4 state access is then 1 KiB contiguous, the 16-bit
// input a contiguous 512 B dwordx2, and the group min/max a 5-step
// butterfly of DPP moves plus one ds_swizzle, all within the half-wave.
//
// Arithmetic is IEEE binary32 with no contraction (the library is built with
// -ffp-contract=off); the only fused multiply-add is the dequantizer's
// explicit fmaf.  16-bit conversions use the hardware's round-to-nearest-even
// converts.  With a fixed summation order the results are a unique function
// of the inputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "echo_internal.h"

namespace echo {

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <int IN_T>
__device__ __forceinline__ float in_to_f32(uint32_t h) {
  return IN_T == kInF16 ? f16_to_f32(h) : bf16_to_f32(h);
}

// DPP lane moves inside a row of 16 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// lane i <-> i ^ 16 inside each 32-lane half (ds_swizzle bit-mask mode:
// and 0x1f, or 0, xor 0x10).
__device__ __forceinline__ float swz_xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// Min and max over the 32 lanes of a half-wave; every lane gets the result.
__device__ __forceinline__ void halfwave_minmax(float& mn, float& mx) {
  mn = fminf(mn, dpp<kDppXor1>(mn));
  mx = fmaxf(mx, dpp<kDppXor1>(mx));
  mn = fminf(mn, dpp<kDppXor2>(mn));
  mx = fmaxf(mx, dpp<kDppXor2>(mx));
  mn = fminf(mn, dpp<kDppHalfMirror>(mn));
  mx = fmaxf(mx, dpp<kDppHalfMirror>(mx));
  mn = fminf(mn, dpp<kDppMirror>(mn));
  mx = fmaxf(mx, dpp<kDppMirror>(mx));
  mn = fminf(mn, swz_xor16(mn));
  mx = fmaxf(mx, swz_xor16(mx));
}

// Group parameters of the zero-point-aware asymmetric quantizer ([JP-1]):
// zero = fp16(min) (range-clamped, never -0), step = fp16((max-zero)/qmax)
// (clamped to [0, 65504]; a non-positive step quantizes everything to 0).
struct QParams {
  float zf, sf, inv;
  uint32_t word;  // scale bits | zero bits << 16
};

template <int BITS>
__device__ __forceinline__ QParams group_params(float mn, float mx) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  const float zc = fminf(fmaxf(mn, -65504.0f), 65504.0f);
  uint32_t zb = f32_to_f16(zc);
  zb = (zb == 0x8000u) ? 0u : zb;
  const float zf = f16_to_f32(zb);
  float s = (mx - zf) / qmax;
  s = (s > 0.0f) ? fminf(s, 65504.0f) : 0.0f;
  const uint32_t sb = f32_to_f16(s);
  const float sf = f16_to_f32(sb);
  const float inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;
  return QParams{zf, sf, inv, sb | (zb << 16)};
}

template <int BITS>
__device__ __forceinline__ uint32_t encode(float v, const QParams& q) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  const float t = (v - q.zf) * q.inv;
  const float r = fminf(fmaxf(rintf(t), 0.0f), qmax);
  return (uint32_t)r;
}

__device__ __forceinline__ float decode(uint32_t code, float sf, float zf) {
  return fmaf((float)code, sf, zf);
}

// 4 consecutive 16-bit inputs
template <int IN_T>
__device__ __forceinline__ void load_in4(const uint16_t* __restrict__ p, float (&v)[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = in_to_f32<IN_T>(w.x & 0xffffu);
  v[1] = in_to_f32<IN_T>(w.x >> 16);
  v[2] = in_to_f32<IN_T>(w.y & 0xffffu);
  v[3] = in_to_f32<IN_T>(w.y >> 16);
}

// 4 consecutive state values
template <int ST_T>
__device__ __forceinline__ void load_state4(const void* base, uint64_t e, float (&v)[4]) {
  if constexpr (ST_T == kStateF32) {
    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + e);
    v[0] = bf16_to_f32(w.x & 0xffffu);
    v[1] = bf16_to_f32(w.x >> 16);
    v[2] = bf16_to_f32(w.y & 0xffffu);
    v[3] = bf16_to_f32(w.y >> 16);
  }
}

template <int ST_T>
__device__ __forceinline__ void store_state4(void* base, uint64_t e, const float (&v)[4]) {
  if constexpr (ST_T == kStateF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + e) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 w;
    w.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    w.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + e) = w;
  }
}

// Codes of 4 consecutive elements starting at segment index k (k % 4 == 0).
template <int BITS>
__device__ __forceinline__ void store_codes4(uint8_t* __restrict__ codes, uint64_t k,
                                             const uint32_t (&q)[4]) {
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint16_t*>(codes + k / 2) =
        (uint16_t)(q[0] | (q[1] << 4) | (q[2] << 8) | (q[3] << 12));
  } else {
    *reinterpret_cast<uint32_t*>(codes + k) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t load_codes4(const uint8_t* __restrict__ codes, uint64_t k) {
  if constexpr (BITS == 4) return *reinterpret_cast<const uint16_t*>(codes + k / 2);
  else return *reinterpret_cast<const uint32_t*>(codes + k);
}

template <int BITS>
__device__ __forceinline__ uint32_t code_at(uint32_t word, int i) {
  return BITS == 4 ? (word >> (4 * i)) & 0xfu : (word >> (8 * i)) & 0xffu;
}

// One step of both moving averages ([JP-2]); products rounded, then added.
__device__ __forceinline__ void ema(float& s, float& l, float r, const Coef& c) {
  const float s_keep = c.bS * s, s_new = c.aS * r;
  const float l_keep = c.bL * l, l_new = c.aL * r;
  s = s_keep + s_new;
  l = l_keep + l_new;
}

// Feedback-added input ([JP-2]): v = x + eta * (S + L).
__device__ __forceinline__ float feedback(float x, float s, float l, float eta) {
  const float u = s + l;
  const float f = eta * u;
  return x + f;
}

constexpr int kThreads = 256;
constexpr int kHalfWaves = kThreads / 32;

// ------------------------------------------------------------------ K1
// Entry pass of `rank` ([JP-1]: only the segments this rank does not own are
// quantized; [JP-2]: feedback-add, residual and state update fused here).
// grid.y = P-1 non-owned segments, grid.x strides over the segment's groups.
template <int BITS, int IN_T, int ST_T>
__global__ __launch_bounds__(kThreads) void k_quant_feedback(
    const uint16_t* __restrict__ x, void* __restrict__ S, void* __restrict__ L, SegTable out,
    int rank, uint32_t groups, uint64_t seg_len, Coef c) {
  const int slot = blockIdx.y;
  const int p = slot + (slot >= rank ? 1 : 0);
  const uint64_t base = (uint64_t)p * seg_len;
  uint8_t* __restrict__ codes = static_cast<uint8_t*>(out.codes[p]);
  uint32_t* __restrict__ params = out.params[p];
  const uint32_t hw = threadIdx.x >> 5, lane = threadIdx.x & 31;
  for (uint32_t g = blockIdx.x * kHalfWaves + hw; g < groups; g += gridDim.x * kHalfWaves) {
    const uint64_t k = (uint64_t)g * kGroup + lane * 4;  // index within the segment
    const uint64_t e = base + k;
    float xv[4], s[4], l[4], v[4];
    load_in4<IN_T>(x + e, xv);
    load_state4<ST_T>(S, e, s);
    load_state4<ST_T>(L, e, l);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = feedback(xv[i], s[i], l[i], c.eta);
    float mn = fminf(fminf(v[0], v[1]), fminf(v[2], v[3]));
    float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    halfwave_minmax(mn, mx);
    const QParams qp = group_params<BITS>(mn, mx);
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = encode<BITS>(v[i], qp);
      const float r = v[i] - decode(q[i], qp.sf, qp.zf);
      ema(s[i], l[i], r, c);
    }
    store_state4<ST_T>(S, e, s);
    store_state4<ST_T>(L, e, l);
    store_codes4<BITS>(codes, k, q);
    if (lane == 0) params[g] = qp.word;
  }
}

// ------------------------------------------------------------------ K2
// Owner pass over segment `rank` ([JP-1]: sum in fp32 in rank order with the
// owner's own unquantized term, requantize; [JP-W] the round trip; [JP-2]
// the owner's residual against the output value, state update fused).
template <int BITS, int IN_T, int ST_T, int OUT_T>
__global__ __launch_bounds__(kThreads) void k_owner_reduce_requant(
    const uint16_t* __restrict__ x, void* __restrict__ S, void* __restrict__ L, SegTable in,
    int P, int rank, uint32_t groups, uint64_t seg_len, uint8_t* __restrict__ out_codes,
    uint32_t* __restrict__ out_params, Coef c) {
  const uint64_t base = (uint64_t)rank * seg_len;
  const uint32_t hw = threadIdx.x >> 5, lane = threadIdx.x & 31;
  for (uint32_t g = blockIdx.x * kHalfWaves + hw; g < groups; g += gridDim.x * kHalfWaves) {
    const uint64_t k = (uint64_t)g * kGroup + lane * 4;
    const uint64_t e = base + k;
    // incoming payload words first, so that all loads are in flight together
    uint32_t cw[kMaxRanks], pw[kMaxRanks];
#pragma unroll
    for (int p = 0; p < kMaxRanks; ++p) {
      if (p < P && p != rank) {
        cw[p] = load_codes4<BITS>(static_cast<const uint8_t*>(in.codes[p]), k);
        pw[p] = in.params[p][g];
      }
    }
    float xv[4], s[4], l[4], own[4];
    load_in4<IN_T>(x + e, xv);
    load_state4<ST_T>(S, e, s);
    load_state4<ST_T>(L, e, l);
#pragma unroll
    for (int i = 0; i < 4; ++i) own[i] = feedback(xv[i], s[i], l[i], c.eta);
    float acc[4];
#pragma unroll
    for (int p = 0; p < kMaxRanks; ++p) {
      if (p < P) {
        float t[4];
        if (p == rank) {
#pragma unroll
          for (int i = 0; i < 4; ++i) t[i] = own[i];
        } else {
          const float sf = f16_to_f32(pw[p] & 0xffffu), zf = f16_to_f32(pw[p] >> 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) t[i] = decode(code_at<BITS>(cw[p], i), sf, zf);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = (p == 0) ? t[i] : acc[i] + t[i];
      }
    }
    float mn = fminf(fminf(acc[0], acc[1]), fminf(acc[2], acc[3]));
    float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    halfwave_minmax(mn, mx);
    const QParams qp = group_params<BITS>(mn, mx);
    uint32_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = encode<BITS>(acc[i], qp);
      const float d = decode(q[i], qp.sf, qp.zf);
      const float o = (OUT_T == kOutBF16) ? bf16_to_f32(f32_to_bf16(d)) : d;
      ema(s[i], l[i], acc[i] - o, c);
    }
    store_state4<ST_T>(S, e, s);
    store_state4<ST_T>(L, e, l);
    store_codes4<BITS>(out_codes, k, q);
    if (lane == 0) out_params[g] = qp.word;
  }
}

// ------------------------------------------------------------------ K3
// Dequantize the P owners' payloads into the output ([JP-1]).
// bf16 output: 8 elements per lane (one 16-byte store), 16 lanes per group;
// fp32 output: 4 elements per lane (one 16-byte store), 32 lanes per group.
template <int BITS, int OUT_T>
__global__ __launch_bounds__(kThreads) void k_dequant_gather(SegTable in, uint32_t groups,
                                                             uint64_t seg_len, void* __restrict__ out) {
  constexpr int EPL = (OUT_T == kOutBF16) ? 8 : 4;
  constexpr int LPG = kGroup / EPL;
  constexpr int GPB = kThreads / LPG;
  const int p = blockIdx.y;
  const uint8_t* __restrict__ codes = static_cast<const uint8_t*>(in.codes[p]);
  const uint32_t* __restrict__ params = in.params[p];
  const uint64_t base = (uint64_t)p * seg_len;
  const uint32_t gl = threadIdx.x / LPG, lane = threadIdx.x % LPG;
  for (uint32_t g = blockIdx.x * GPB + gl; g < groups; g += gridDim.x * GPB) {
    const uint64_t k = (uint64_t)g * kGroup + lane * EPL;
    const uint32_t pw = params[g];
    const float sf = f16_to_f32(pw & 0xffffu), zf = f16_to_f32(pw >> 16);
    float d[EPL];
    if constexpr (BITS == 4 && EPL == 8) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + k / 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = decode((w >> (4 * i)) & 0xfu, sf, zf);
    } else if constexpr (BITS == 4) {
      const uint32_t w = *reinterpret_cast<const uint16_t*>(codes + k / 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = decode((w >> (4 * i)) & 0xfu, sf, zf);
    } else if constexpr (EPL == 8) {
      const uint2 w = *reinterpret_cast<const uint2*>(codes + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        d[i] = decode((w.x >> (8 * i)) & 0xffu, sf, zf);
        d[4 + i] = decode((w.y >> (8 * i)) & 0xffu, sf, zf);
      }
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = decode((w >> (8 * i)) & 0xffu, sf, zf);
    }
    if constexpr (OUT_T == kOutBF16) {
      uint4 o;
      o.x = f32_to_bf16(d[0]) | (f32_to_bf16(d[1]) << 16);
      o.y = f32_to_bf16(d[2]) | (f32_to_bf16(d[3]) << 16);
      o.z = f32_to_bf16(d[4]) | (f32_to_bf16(d[5]) << 16);
      o.w = f32_to_bf16(d[6]) | (f32_to_bf16(d[7]) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + base + k) = o;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + base + k) =
          make_float4(d[0], d[1], d[2], d[3]);
    }
  }
}

// ------------------------------------------------------------------ reset
// Zero `bytes` bytes (a multiple of 2) at a 16-byte aligned address.
__global__ __launch_bounds__(kThreads) void k_zero(uint8_t* __restrict__ a, uint64_t bytes) {
  const uint64_t n16 = bytes / 16;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(a)[i] = make_uint4(0, 0, 0, 0);
  const uint64_t tail = bytes - n16 * 16;  // < 16, even
  if (blockIdx.x == 0 && threadIdx.x < tail / 2)
    reinterpret_cast<uint16_t*>(a + n16 * 16)[threadIdx.x] = 0;
}

// ------------------------------------------------------------------ launchers
namespace {

// Blocks along x: enough for one group per half-wave, capped so very large
// segments stride (each block then handles several groups).
unsigned blocks_for(uint64_t groups, uint64_t groups_per_block, unsigned ny) {
  const uint64_t want = (groups + groups_per_block - 1) / groups_per_block;
  const uint64_t cap = (kGridCap + ny - 1) / ny;
  const uint64_t b = want < cap ? want : cap;
  return (unsigned)(b == 0 ? 1 : b);
}

}  // namespace

template <int BITS, int IN_T, int ST_T>
static void launch_k1(const LaunchArgs& a, hipStream_t st) {
  const uint64_t groups = a.seg_len / kGroup;
  const unsigned ny = (unsigned)(a.P - 1);
  dim3 grid(blocks_for(groups, kHalfWaves, ny), ny);
  hipLaunchKernelGGL((k_quant_feedback<BITS, IN_T, ST_T>), grid, dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(a.x), a.S, a.L, a.segs, a.rank,
                     (uint32_t)groups, a.seg_len, a.coef);
}

template <int BITS, int IN_T, int ST_T, int OUT_T>
static void launch_k2(const LaunchArgs& a, hipStream_t st) {
  const uint64_t groups = a.seg_len / kGroup;
  dim3 grid(blocks_for(groups, kHalfWaves, 1));
  hipLaunchKernelGGL((k_owner_reduce_requant<BITS, IN_T, ST_T, OUT_T>), grid, dim3(kThreads), 0,
                     st, static_cast<const uint16_t*>(a.x), a.S, a.L, a.segs, a.P, a.rank,
                     (uint32_t)groups, a.seg_len, static_cast<uint8_t*>(a.out_codes),
                     a.out_params, a.coef);
}

template <int BITS, int OUT_T>
static void launch_k3(const LaunchArgs& a, hipStream_t st) {
  const uint64_t groups = a.seg_len / kGroup;
  constexpr int gpb = kThreads / (kGroup / ((OUT_T == kOutBF16) ? 8 : 4));
  const unsigned ny = (unsigned)a.P;
  dim3 grid(blocks_for(groups, gpb, ny), ny);
  hipLaunchKernelGGL((k_dequant_gather<BITS, OUT_T>), grid, dim3(kThreads), 0, st, a.segs,
                     (uint32_t)groups, a.seg_len, a.out);
}

// Runtime -> template dispatch.
void run_quant_feedback(const LaunchArgs& a, hipStream_t st) {
#define ECHO_K1(B, I, S) \
  if (a.bits == B && a.in_dtype == I && a.state_dtype == S) return launch_k1<B, I, S>(a, st);
  ECHO_K1(4, kInBF16, kStateF32) ECHO_K1(4, kInBF16, kStateBF16)
  ECHO_K1(4, kInF16, kStateF32)  ECHO_K1(4, kInF16, kStateBF16)
  ECHO_K1(8, kInBF16, kStateF32) ECHO_K1(8, kInBF16, kStateBF16)
  ECHO_K1(8, kInF16, kStateF32)  ECHO_K1(8, kInF16, kStateBF16)
#undef ECHO_K1
}

void run_owner_reduce_requant(const LaunchArgs& a, hipStream_t st) {
#define ECHO_K2(B, I, S, O)                                                             \
  if (a.bits == B && a.in_dtype == I && a.state_dtype == S && a.out_dtype == O) \
    return launch_k2<B, I, S, O>(a, st);
#define ECHO_K2_IO(B, I) \
  ECHO_K2(B, I, kStateF32, kOutBF16) ECHO_K2(B, I, kStateF32, kOutF32) \
  ECHO_K2(B, I, kStateBF16, kOutBF16) ECHO_K2(B, I, kStateBF16, kOutF32)
  ECHO_K2_IO(4, kInBF16) ECHO_K2_IO(4, kInF16) ECHO_K2_IO(8, kInBF16) ECHO_K2_IO(8, kInF16)
#undef ECHO_K2_IO
#undef ECHO_K2
}

void run_dequant_gather(const LaunchArgs& a, hipStream_t st) {
  if (a.bits == 4 && a.out_dtype == kOutBF16) return launch_k3<4, kOutBF16>(a, st);
  if (a.bits == 4 && a.out_dtype == kOutF32) return launch_k3<4, kOutF32>(a, st);
  if (a.bits == 8 && a.out_dtype == kOutBF16) return launch_k3<8, kOutBF16>(a, st);
  if (a.bits == 8 && a.out_dtype == kOutF32) return launch_k3<8, kOutF32>(a, st);
}

void run_zero(void* p, uint64_t bytes, hipStream_t st) {
  const uint64_t n16 = bytes / 16;
  uint64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > kGridCap) blocks = kGridCap;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                     static_cast<uint8_t*>(p), bytes);
}

}  // namespace echo
