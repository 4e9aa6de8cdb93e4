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
// Error-state layout: one array per rank holding the two memories of each
// element side by side, state[2j] = S_j (short), state[2j+1] = L_j (long).
// One dwordx4 then carries both memories of 2 elements (fp32 state) or 4
// elements (bf16 state), so the state is a single contiguous stream; on
// gfx950 this streams markedly faster than two separate S and L arrays.
//
// Thread mapping of the entry and owner passes: EPL consecutive elements per
// lane (2 for fp32 state, 4 for bf16 state), so a group of G elements (32,
// 64 or 128) is an aligned run of G/EPL lanes -- one whole wave for G = 128
// with fp32 state -- and every wave-wide load or store of the state is 1 KiB
// contiguous.  The group min/max is a butterfly of DPP moves and, for runs of
// 32 or more lanes, a ds_swizzle; a whole-wave group then combines its two
// halves with a readlane of lanes 0 and 32.  Streamed arrays use nontemporal
// loads and stores, except the owner pass's payload loads, where L2 should
// serve the second half of a line to the neighbouring wave.  (Plain code
// stores look faster for a kernel repeated alone, but they leave dirty lines
// in the memory-side cache that the next kernel pays to write back.)
// Launches are one-shot, one group per lane run, with enough blocks to cover
// a segment: short-lived waves stream best here.  The owner pass numbers its
// blocks XCD-contiguously.
//
// A message whose length is not a multiple of P*G has one partial group (in
// its last non-empty segment); the main entry and owner kernels handle whole
// groups only and that group runs in a one-block tail kernel with element-wise
// guarded accesses, so the streaming kernels carry no guarded path.  The
// dequantize pass guards its last lane per element.
//
// Dequantize pass: 8 elements per lane for bf16 output, 4 for fp32 (one
// 16-byte store either way), two chunks per lane one wave-width apart.
//
// Arithmetic is IEEE binary32 with no contraction (the library is built with
// -ffp-contract=off); the only fused multiply-add is the dequantizer's
// explicit fmaf.  16-bit conversions use the hardware's round-to-nearest-even
// converts.  With a fixed summation order the results are a unique function
// of the inputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Combine the two already-reduced 32-lane halves of a wave (wave-uniform).
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Plain or nontemporal access to streamed arrays.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
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

// EPL consecutive 16-bit inputs (EPL = 2 or 4)
template <int IN_T, int EPL, bool NT>
__device__ __forceinline__ void load_in(const uint16_t* __restrict__ p, float* v) {
  if constexpr (EPL == 2) {
    const uint32_t w = ld<NT>(reinterpret_cast<const uint32_t*>(p));
    v[0] = in_to_f32<IN_T>(w & 0xffffu);
    v[1] = in_to_f32<IN_T>(w >> 16);
  } else {
    const u32x2 w = ld<NT>(reinterpret_cast<const u32x2*>(p));
    v[0] = in_to_f32<IN_T>(w.x & 0xffffu);
    v[1] = in_to_f32<IN_T>(w.x >> 16);
    v[2] = in_to_f32<IN_T>(w.y & 0xffffu);
    v[3] = in_to_f32<IN_T>(w.y >> 16);
  }
}

// Both memories of EPL consecutive elements: one 16-byte access.
// fp32 state: EPL = 2, {S0, L0, S1, L1}; bf16 state: EPL = 4, word i = S_i | L_i << 16.
template <int ST_T>
struct StateIO {
  static constexpr int kEPL = (ST_T == kStateF32) ? 2 : 4;
  template <bool NT>
  static __device__ __forceinline__ void load(const void* base, uint64_t e, float* s, float* l) {
    if constexpr (ST_T == kStateF32) {
      const f32x4 w = ld<NT>(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + 2 * e));
      s[0] = w.x; l[0] = w.y; s[1] = w.z; l[1] = w.w;
    } else {
      const u32x4 w = ld<NT>(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + 2 * e));
      const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = bf16_to_f32(a[i] & 0xffffu);
        l[i] = bf16_to_f32(a[i] >> 16);
      }
    }
  }
  template <bool NT>
  static __device__ __forceinline__ void store(void* base, uint64_t e, const float* s, const float* l) {
    if constexpr (ST_T == kStateF32) {
      f32x4 w = {s[0], l[0], s[1], l[1]};
      st<NT>(reinterpret_cast<f32x4*>(static_cast<float*>(base) + 2 * e), w);
    } else {
      u32x4 w;
      w.x = f32_to_bf16(s[0]) | (f32_to_bf16(l[0]) << 16);
      w.y = f32_to_bf16(s[1]) | (f32_to_bf16(l[1]) << 16);
      w.z = f32_to_bf16(s[2]) | (f32_to_bf16(l[2]) << 16);
      w.w = f32_to_bf16(s[3]) | (f32_to_bf16(l[3]) << 16);
      st<NT>(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + 2 * e), w);
    }
  }
};

// Codes of EPL consecutive elements starting at segment index k (k % EPL == 0):
// EPL*BITS bits, i.e. 1, 2 or 4 bytes.
template <int BITS, int EPL>
struct CodeIO {
  static constexpr int kBits = BITS * EPL;
  using word = typename std::conditional<kBits == 8, uint8_t,
               typename std::conditional<kBits == 16, uint16_t, uint32_t>::type>::type;
  template <bool NT>
  static __device__ __forceinline__ void store(uint8_t* __restrict__ codes, uint64_t k, const uint32_t* q) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) w |= q[i] << (BITS * i);
    st<NT>(reinterpret_cast<word*>(codes + k * BITS / 8), (word)w);
  }
  template <bool NT>
  static __device__ __forceinline__ uint32_t load(const uint8_t* __restrict__ codes, uint64_t k) {
    return ld<NT>(reinterpret_cast<const word*>(codes + k * BITS / 8));
  }
};

// Element-wise forms for the one partial group of a ragged message: only the
// lane's first nv elements exist (nv = 0 .. EPL); nothing past them is read
// or written.  An INT4 byte holding one valid element gets a 0 high nibble.
template <int IN_T, int EPL>
__device__ __forceinline__ void load_in_part(const uint16_t* __restrict__ p, float* v, int nv) {
#pragma unroll
  for (int i = 0; i < EPL; ++i) v[i] = i < nv ? in_to_f32<IN_T>(p[i]) : 0.0f;
}

template <int ST_T>
__device__ __forceinline__ void load_state_part(const void* base, uint64_t e, float* s, float* l,
                                                int nv) {
#pragma unroll
  for (int i = 0; i < StateIO<ST_T>::kEPL; ++i) {
    s[i] = l[i] = 0.0f;
    if (i < nv) {
      if constexpr (ST_T == kStateF32) {
        const float* q = static_cast<const float*>(base) + 2 * (e + i);
        s[i] = q[0];
        l[i] = q[1];
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + 2 * (e + i));
        s[i] = bf16_to_f32(w & 0xffffu);
        l[i] = bf16_to_f32(w >> 16);
      }
    }
  }
}

template <int ST_T>
__device__ __forceinline__ void store_state_part(void* base, uint64_t e, const float* s,
                                                 const float* l, int nv) {
#pragma unroll
  for (int i = 0; i < StateIO<ST_T>::kEPL; ++i) {
    if (i < nv) {
      if constexpr (ST_T == kStateF32) {
        float* q = static_cast<float*>(base) + 2 * (e + i);
        q[0] = s[i];
        q[1] = l[i];
      } else {
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + 2 * (e + i)) =
            f32_to_bf16(s[i]) | (f32_to_bf16(l[i]) << 16);
      }
    }
  }
}

template <int BITS, int EPL>
__device__ __forceinline__ void store_codes_part(uint8_t* __restrict__ codes, uint64_t k,
                                                 const uint32_t* q, int nv) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i < nv) codes[k + i] = (uint8_t)q[i];
  } else {
#pragma unroll
    for (int b = 0; b < EPL / 2; ++b)
      if (2 * b < nv) codes[k / 2 + b] = (uint8_t)(q[2 * b] | ((2 * b + 1 < nv ? q[2 * b + 1] : 0u) << 4));
  }
}

// Full groups per segment: `all` in segments before `last` (the last
// non-empty one), `in_last` in it, none after it.
struct FullGroups {
  uint32_t all, last, in_last;
  __device__ __forceinline__ uint32_t of(uint32_t p) const {
    return p < last ? all : (p == last ? in_last : 0u);
  }
};

// Elements of segment p of a message of n elements cut into segments of
// seg_len: seg_len everywhere but the last non-empty segment, 0 after it.
__device__ __forceinline__ uint64_t segment_count(uint64_t n, uint64_t seg_len, uint32_t p) {
  const uint64_t start = (uint64_t)p * seg_len;
  if (start >= n) return 0;
  return (n - start) < seg_len ? (n - start) : seg_len;
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
constexpr uint32_t kXcds = 8;   // MI355X: 8 accelerator dies, each with its own L2

// Blocks are dealt to the XCDs round-robin in launch order.  Renumber them so
// that each XCD works through one contiguous range of the grid: data that
// neighbouring blocks share at sub-line granularity (the 4-byte group
// parameters, 32 groups per 128-byte line) then stays in one L2.
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t b, uint32_t nb) {
  const uint32_t q = nb / kXcds, r = nb % kXcds;
  const uint32_t x = b % kXcds, i = b / kXcds;
  return x * q + (x < r ? x : r) + i;
}

// Mapping of one group of G elements onto lanes for a state type (see the
// file header): kLanes = G / EPL consecutive lanes, aligned runs.
template <int ST_T, int G>
struct GroupMap {
  static constexpr int kEPL = StateIO<ST_T>::kEPL;       // elements per lane
  static constexpr int kLanes = G / kEPL;                 // lanes per group: 8 .. 64
  static constexpr int kGroupsPerBlock = kThreads / kLanes;
  static_assert(kLanes == 8 || kLanes == 16 || kLanes == 32 || kLanes == 64, "lanes per group");
};

// Min and max over each aligned run of LANES lanes; every lane of a run gets
// its run's result.
template <int LANES>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
  mn = fminf(mn, dpp<kDppXor1>(mn));
  mx = fmaxf(mx, dpp<kDppXor1>(mx));
  mn = fminf(mn, dpp<kDppXor2>(mn));
  mx = fmaxf(mx, dpp<kDppXor2>(mx));
  mn = fminf(mn, dpp<kDppHalfMirror>(mn));
  mx = fmaxf(mx, dpp<kDppHalfMirror>(mx));
  if constexpr (LANES >= 16) {
    mn = fminf(mn, dpp<kDppMirror>(mn));
    mx = fmaxf(mx, dpp<kDppMirror>(mx));
  }
  if constexpr (LANES >= 32) {
    mn = fminf(mn, swz_xor16(mn));
    mx = fmaxf(mx, swz_xor16(mx));
  }
  if constexpr (LANES == 64) {
    mn = fminf(lane_value(mn, 0), lane_value(mn, 32));
    mx = fmaxf(lane_value(mx, 0), lane_value(mx, 32));
  }
}

// ------------------------------------------------------------------ K1
// Entry pass of `rank` ([JP-1]: only the segments this rank does not own are
// quantized; [JP-2]: feedback-add, residual and state update fused here).
// One group of G elements per run of G/EPL lanes.  FULL: every element of
// the group exists; otherwise the lane holds nv of its EPL elements.
template <int BITS, int IN_T, int ST_T, int G, bool NT, bool FULL>
__device__ __forceinline__ void entry_group(const uint16_t* __restrict__ x, void* __restrict__ state,
                                            uint8_t* __restrict__ codes, uint32_t* __restrict__ params,
                                            uint32_t g, uint32_t lane, uint64_t base, int nv,
                                            const Coef& c) {
  using M = GroupMap<ST_T, G>;
  constexpr int E = M::kEPL;
  const uint64_t k = (uint64_t)g * G + lane * E;   // index within the segment
  const uint64_t e = base + k;
  float xv[E], s[E], l[E], v[E];
  if constexpr (FULL) {
    load_in<IN_T, E, NT>(x + e, xv);
    StateIO<ST_T>::template load<NT>(state, e, s, l);
  } else {
    load_in_part<IN_T, E>(x + e, xv, nv);
    load_state_part<ST_T>(state, e, s, l, nv);
  }
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    v[i] = feedback(xv[i], s[i], l[i], c.eta);
    if (FULL || i < nv) {
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
  }
  group_minmax<M::kLanes>(mn, mx);
  const QParams qp = group_params<BITS>(mn, mx);
  uint32_t q[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    q[i] = (FULL || i < nv) ? encode<BITS>(v[i], qp) : 0u;
    ema(s[i], l[i], v[i] - decode(q[i], qp.sf, qp.zf), c);
  }
  if constexpr (FULL) {
    StateIO<ST_T>::template store<NT>(state, e, s, l);
    CodeIO<BITS, E>::template store<NT>(codes, k, q);
  } else {
    store_state_part<ST_T>(state, e, s, l, nv);
    store_codes_part<BITS, E>(codes, k, q, nv);
  }
  if (lane == 0) params[g] = qp.word;
}

// grid.y = P-1 non-owned segments, grid.x covers a full segment's groups.
// Full groups only; the partial group of a ragged message goes to
// k_quant_feedback_tail, so this kernel carries no guarded path.
template <int BITS, int IN_T, int ST_T, int G, bool NT, bool XCD>
__global__ __launch_bounds__(kThreads) void k_quant_feedback(
    const uint16_t* __restrict__ x, void* __restrict__ state, SegTable out, int rank,
    FullGroups fg, uint64_t seg_len, uint32_t bx0, Coef c) {
  using M = GroupMap<ST_T, G>;
  uint32_t bx = blockIdx.x, slot = blockIdx.y;
  if constexpr (XCD) {
    const uint32_t L = xcd_contiguous_block(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
    slot = L / gridDim.x;
    bx = L - slot * gridDim.x;
  }
  bx += bx0;
  const uint32_t p = slot + ((int)slot >= rank ? 1u : 0u);
  const uint32_t lane = threadIdx.x % M::kLanes;
  const uint32_t g = bx * M::kGroupsPerBlock + threadIdx.x / M::kLanes;
  if (g >= fg.of(p)) return;   // whole groups only: the lanes of a group leave together
  entry_group<BITS, IN_T, ST_T, G, NT, true>(x, state, static_cast<uint8_t*>(out.codes[p]),
                                             out.params[p], g, lane, (uint64_t)p * seg_len,
                                             M::kEPL, c);
}

// The one partial group (`valid` < G elements) of segment p: one block of
// G/EPL lanes.
template <int BITS, int IN_T, int ST_T, int G>
__global__ void k_quant_feedback_tail(const uint16_t* __restrict__ x, void* __restrict__ state,
                                      uint8_t* __restrict__ codes, uint32_t* __restrict__ params,
                                      uint64_t base, uint32_t g, uint32_t valid, Coef c) {
  using M = GroupMap<ST_T, G>;
  const int nv = (int)valid - (int)threadIdx.x * M::kEPL;
  entry_group<BITS, IN_T, ST_T, G, false, false>(x, state, codes, params, g, threadIdx.x, base,
                                                 nv < 0 ? 0 : nv > M::kEPL ? M::kEPL : nv, c);
}

// ------------------------------------------------------------------ K2
// Owner pass over segment `rank` ([JP-1]: sum in fp32 in rank order with the
// owner's own unquantized term, requantize; [JP-W] the round trip; [JP-2]
// the owner's residual against the output value, state update fused).
template <int BITS, int IN_T, int ST_T, int OUT_T, int G, int NP, bool NT, bool NTP, bool FULL>
__device__ __forceinline__ void owner_group(const uint16_t* __restrict__ x, void* __restrict__ state,
                                            const SegTable& in, int P, int rank,
                                            uint8_t* __restrict__ out_codes,
                                            uint32_t* __restrict__ out_params, uint32_t g,
                                            uint32_t lane, uint64_t base, int nv, const Coef& c) {
  using M = GroupMap<ST_T, G>;
  constexpr int E = M::kEPL;
  const uint64_t k = (uint64_t)g * G + lane * E;
  const uint64_t e = base + k;
  // Incoming payload words first, so that all loads are in flight together.
  // NP >= P slots are loaded without a branch: the launcher points the
  // owner's own slot and the slots from P on at another rank's payload, and
  // those words are ignored.  (Loads under a per-slot branch made the
  // compiler wait for the first one before issuing the rest.)  A payload is
  // sized for a full segment: the word of a partial group exists, its bytes
  // past the group's end are ignored.
  uint32_t cw[NP], pw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    cw[p] = CodeIO<BITS, E>::template load<NTP>(static_cast<const uint8_t*>(in.codes[p]), k);
    pw[p] = in.params[p][g];
  }
  float xv[E], s[E], l[E], acc[E];
  if constexpr (FULL) {
    load_in<IN_T, E, NT>(x + e, xv);
    StateIO<ST_T>::template load<NT>(state, e, s, l);
  } else {
    load_in_part<IN_T, E>(x + e, xv, nv);
    load_state_part<ST_T>(state, e, s, l, nv);
  }
  // Keep every payload load here, ahead of the per-slot branches below:
  // without this use the compiler sinks a slot's load into its branch, and
  // the wave then waits for it before issuing the next.
#pragma unroll
  for (int p = 0; p < NP; ++p) asm volatile("" ::"v"(cw[p]), "v"(pw[p]));
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p < P) {
      if (p == rank) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float t = feedback(xv[i], s[i], l[i], c.eta);
          acc[i] = (p == 0) ? t : acc[i] + t;
        }
      } else {
        const float sf = f16_to_f32(pw[p] & 0xffffu), zf = f16_to_f32(pw[p] >> 16);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float t = decode(code_at<BITS>(cw[p], i), sf, zf);
          acc[i] = (p == 0) ? t : acc[i] + t;
        }
      }
    }
  }
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (FULL || i < nv) {
      mn = fminf(mn, acc[i]);
      mx = fmaxf(mx, acc[i]);
    }
  }
  group_minmax<M::kLanes>(mn, mx);
  const QParams qp = group_params<BITS>(mn, mx);
  uint32_t q[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    q[i] = (FULL || i < nv) ? encode<BITS>(acc[i], qp) : 0u;
    const float d = decode(q[i], qp.sf, qp.zf);
    const float o = (OUT_T == kOutBF16) ? bf16_to_f32(f32_to_bf16(d)) : d;
    ema(s[i], l[i], acc[i] - o, c);
  }
  if constexpr (FULL) {
    StateIO<ST_T>::template store<NT>(state, e, s, l);
    CodeIO<BITS, E>::template store<NT>(out_codes, k, q);
  } else {
    store_state_part<ST_T>(state, e, s, l, nv);
    store_codes_part<BITS, E>(out_codes, k, q, nv);
  }
  if (lane == 0) out_params[g] = qp.word;
}

// Full groups only (see k_quant_feedback); the partial group goes to
// k_owner_reduce_requant_tail.
template <int BITS, int IN_T, int ST_T, int OUT_T, int G, int NP, bool NT, bool NTP, bool XCD>
__global__ __launch_bounds__(kThreads) void k_owner_reduce_requant(
    const uint16_t* __restrict__ x, void* __restrict__ state, SegTable in, int P, int rank,
    FullGroups fg, uint64_t seg_len, uint32_t bx0, uint8_t* __restrict__ out_codes,
    uint32_t* __restrict__ out_params, Coef c) {
  using M = GroupMap<ST_T, G>;
  const uint32_t lane = threadIdx.x % M::kLanes;
  const uint32_t bx = (XCD ? xcd_contiguous_block(blockIdx.x, gridDim.x) : blockIdx.x) + bx0;
  const uint32_t g = bx * M::kGroupsPerBlock + threadIdx.x / M::kLanes;
  if (g >= fg.of((uint32_t)rank)) return;
  owner_group<BITS, IN_T, ST_T, OUT_T, G, NP, NT, NTP, true>(x, state, in, P, rank, out_codes,
                                                             out_params, g, lane,
                                                             (uint64_t)rank * seg_len, M::kEPL, c);
}

template <int BITS, int IN_T, int ST_T, int OUT_T, int G>
__global__ void k_owner_reduce_requant_tail(const uint16_t* __restrict__ x, void* __restrict__ state,
                                            SegTable in, int P, int rank,
                                            uint8_t* __restrict__ out_codes,
                                            uint32_t* __restrict__ out_params, uint64_t base,
                                            uint32_t g, uint32_t valid, Coef c) {
  using M = GroupMap<ST_T, G>;
  const int nv = (int)valid - (int)threadIdx.x * M::kEPL;
  owner_group<BITS, IN_T, ST_T, OUT_T, G, kMaxRanks, false, false, false>(
      x, state, in, P, rank, out_codes, out_params, g, threadIdx.x, base,
      nv < 0 ? 0 : nv > M::kEPL ? M::kEPL : nv, c);
}

// ------------------------------------------------------------------ K3
// Dequantize the P owners' payloads into the output ([JP-1]).
// EPL elements per lane and chunk (8 for bf16 output, 4 for fp32: one 16-byte
// store either way), G/EPL lanes per group, so a wave covers 64*EPL/G groups
// per chunk; each lane does CH chunks, one wave-width (64*EPL elements)
// apart, so every store instruction is 1 KiB contiguous.
template <int OUT_T, int G>
struct GatherMap {
  static constexpr int kEPL = (OUT_T == kOutBF16) ? 8 : 4;
  static constexpr int kLanes = G / kEPL;
  static constexpr int kGroupsPerWave = 64 / kLanes;
};

// The EPL codes of one lane and chunk: 4 bytes (INT4, bf16 out: 8 codes),
// 2 bytes (INT4, fp32 out), 8 bytes (INT8, bf16 out) or 4 bytes (INT8, fp32).
template <int BITS, int EPL, bool NT>
__device__ __forceinline__ u32x2 gather_codes(const uint8_t* __restrict__ codes, uint64_t k) {
  u32x2 w = {0u, 0u};
  if constexpr (BITS == 4 && EPL == 8) w.x = ld<NT>(reinterpret_cast<const uint32_t*>(codes + k / 2));
  else if constexpr (BITS == 4) w.x = ld<NT>(reinterpret_cast<const uint16_t*>(codes + k / 2));
  else if constexpr (EPL == 8) w = ld<NT>(reinterpret_cast<const u32x2*>(codes + k));
  else w.x = ld<NT>(reinterpret_cast<const uint32_t*>(codes + k));
  return w;
}

// Dequantize and store the EPL elements a lane holds for one chunk.
template <int BITS, int OUT_T, int EPL, bool NT>
__device__ __forceinline__ void gather_store(void* __restrict__ out, uint64_t e, u32x2 cw, uint32_t pw) {
  const float sf = f16_to_f32(pw & 0xffffu), zf = f16_to_f32(pw >> 16);
  float d[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const uint32_t w = (BITS * i < 32) ? cw.x : cw.y;
    d[i] = decode((w >> ((BITS * i) % 32)) & ((1u << BITS) - 1u), sf, zf);
  }
  if constexpr (OUT_T == kOutBF16) {
    u32x4 o;
    o.x = f32_to_bf16(d[0]) | (f32_to_bf16(d[1]) << 16);
    o.y = f32_to_bf16(d[2]) | (f32_to_bf16(d[3]) << 16);
    o.z = f32_to_bf16(d[4]) | (f32_to_bf16(d[5]) << 16);
    o.w = f32_to_bf16(d[6]) | (f32_to_bf16(d[7]) << 16);
    st<NT>(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e), o);
  } else {
    f32x4 o = {d[0], d[1], d[2], d[3]};
    st<NT>(reinterpret_cast<f32x4*>(static_cast<float*>(out) + e), o);
  }
}

template <int OUT_T, int G, int CH>
constexpr uint32_t gather_groups_per_block() {
  return (kThreads / 64) * GatherMap<OUT_T, G>::kGroupsPerWave * CH;
}

// Whole tiles of gather_groups_per_block() whole groups only: straight-line
// code, every chunk's loads issued before the first store (a wave waits for
// memory once).  The rest of each segment -- fewer than a tile of groups,
// and the partial group of a ragged message -- goes to k_dequant_gather_tail.
template <int BITS, int OUT_T, int G, int CH, bool NT, bool NTP>
__global__ __launch_bounds__(kThreads) void k_dequant_gather(SegTable in, FullGroups fg,
                                                             uint64_t seg_len, uint32_t bx0,
                                                             void* __restrict__ out) {
  using M = GatherMap<OUT_T, G>;
  constexpr int EPL = M::kEPL;
  constexpr uint32_t kTile = gather_groups_per_block<OUT_T, G, CH>();
  const uint32_t p = blockIdx.y;
  const uint32_t bx = blockIdx.x + bx0;
  if (bx >= fg.of(p) / kTile) return;   // whole block
  const uint8_t* __restrict__ codes = static_cast<const uint8_t*>(in.codes[p]);
  const uint32_t* __restrict__ params = in.params[p];
  const uint64_t base = (uint64_t)p * seg_len;
  const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const uint32_t g0 = (bx * (kThreads / 64) + wave) * M::kGroupsPerWave * CH;
  const uint32_t in_group = (lane % M::kLanes) * EPL;
  u32x2 cw[CH];
  uint32_t pw[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const uint32_t g = g0 + ch * M::kGroupsPerWave + lane / M::kLanes;
    cw[ch] = gather_codes<BITS, EPL, NTP>(codes, (uint64_t)g * G + in_group);
    pw[ch] = params[g];
  }
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const uint32_t g = g0 + ch * M::kGroupsPerWave + lane / M::kLanes;
    gather_store<BITS, OUT_T, EPL, NT>(out, base + (uint64_t)g * G + in_group, cw[ch], pw[ch]);
  }
}

// One block per segment: the groups after its last whole tile, up to the
// segment's end (the last non-empty segment may end in a partial group;
// nothing past element n-1 is written).
template <int BITS, int OUT_T, int G, int CH>
__global__ __launch_bounds__(kThreads) void k_dequant_gather_tail(SegTable in, FullGroups fg,
                                                                  uint64_t n, uint64_t seg_len,
                                                                  void* __restrict__ out) {
  using M = GatherMap<OUT_T, G>;
  constexpr int EPL = M::kEPL;
  constexpr uint32_t kTile = gather_groups_per_block<OUT_T, G, CH>();
  const uint32_t p = blockIdx.y;
  const uint64_t len = segment_count(n, seg_len, p);
  if (len == 0) return;   // an empty segment's payload is not read
  const uint8_t* __restrict__ codes = static_cast<const uint8_t*>(in.codes[p]);
  const uint32_t* __restrict__ params = in.params[p];
  const uint64_t base = (uint64_t)p * seg_len;
  const uint32_t first = fg.of(p) / kTile * kTile;
  const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const uint32_t in_group = (lane % M::kLanes) * EPL;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const uint32_t g = first + (wave * CH + ch) * M::kGroupsPerWave + lane / M::kLanes;
    const uint64_t k = (uint64_t)g * G + in_group;
    if (k >= len) break;   // lanes are independent here
    const u32x2 cw = gather_codes<BITS, EPL, false>(codes, k);   // the payload holds seg_len codes
    const uint32_t pw = params[g];
    if (k + EPL <= len) {
      gather_store<BITS, OUT_T, EPL, false>(out, base + k, cw, pw);
      continue;
    }
    // the last lane of a ragged message: element-wise stores
    const float sf = f16_to_f32(pw & 0xffffu), zf = f16_to_f32(pw >> 16);
    const int nv = (int)(len - k);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (i < nv) {
        const uint32_t w = (BITS * i < 32) ? cw.x : cw.y;
        const float d = decode((w >> ((BITS * i) % 32)) & ((1u << BITS) - 1u), sf, zf);
        if constexpr (OUT_T == kOutBF16)
          static_cast<uint16_t*>(out)[base + k + i] = (uint16_t)f32_to_bf16(d);
        else
          static_cast<float*>(out)[base + k + i] = d;
      }
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

// The partial group of a ragged message, if any: segment p, group g, and its
// number of elements (valid = 0: every group is full).
struct Tail {
  uint32_t p, g, valid;
};
Tail tail_of(uint64_t n, uint64_t seg_len, int group) {
  const uint64_t p = (n - 1) / seg_len;                 // last non-empty segment
  const uint64_t len = n - p * seg_len;
  return Tail{(uint32_t)p, (uint32_t)(len / group), (uint32_t)(len % group)};
}

FullGroups full_groups(uint64_t n, uint64_t seg_len, int group) {
  const Tail t = tail_of(n, seg_len, group);
  return FullGroups{(uint32_t)(seg_len / group), t.p, t.g};
}

// Blocks along x: enough for every group, one group per lane run.
uint64_t blocks_for(uint64_t groups, uint64_t groups_per_block) {
  const uint64_t b = (groups + groups_per_block - 1) / groups_per_block;
  return b == 0 ? 1 : b;
}

// A dispatch holds at most 2^32 - 1 work-items along x, so a grid of more
// blocks than this goes out as several launches, each told the index of its
// first block.  Only segments beyond about 2^33 elements need more than one.
constexpr uint64_t kMaxBlocksX = 0xffffffffull / kThreads;

// Launch blocks [0, blocks) along x as chunks of at most kMaxBlocksX; f(first,
// count) makes one launch and returns its status.
template <typename F>
hipError_t in_chunks(uint64_t blocks, F&& f) {
  hipError_t e = hipSuccess;
  for (uint64_t b0 = 0; b0 < blocks && e == hipSuccess; b0 += kMaxBlocksX)
    e = f((uint32_t)b0, (unsigned)(blocks - b0 < kMaxBlocksX ? blocks - b0 : kMaxBlocksX));
  return e;
}

}  // namespace

// Launch `kernel` with its own status: hipLaunchKernel returns the launch's
// error, so no pending error of the caller's is read or cleared.  The
// arguments convert to the kernel's parameter types.
template <typename T>
struct Same {
  using type = T;
};
template <typename... Params>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t st,
                  typename Same<Params>::type... args) {
  void* ptrs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, st);
}

template <int BITS, int IN_T, int ST_T, int G, bool NT, bool XCD>
hipError_t launch_k1(const LaunchArgs& a, hipStream_t st) {
  const uint64_t groups = a.seg_len / G;
  const unsigned ny = (unsigned)(a.P - 1);
  hipError_t e = in_chunks(blocks_for(groups, GroupMap<ST_T, G>::kGroupsPerBlock),
                           [&](uint32_t b0, unsigned nb) {
    return launch(k_quant_feedback<BITS, IN_T, ST_T, G, NT, XCD>, dim3(nb, ny), dim3(kThreads), st,
                  static_cast<const uint16_t*>(a.x), a.state, a.segs, a.rank,
                  full_groups(a.n, a.seg_len, G), a.seg_len, b0, a.coef);
  });
  const Tail t = tail_of(a.n, a.seg_len, G);
  if (e == hipSuccess && t.valid && (int)t.p != a.rank)
    e = launch(k_quant_feedback_tail<BITS, IN_T, ST_T, G>, dim3(1), dim3(GroupMap<ST_T, G>::kLanes),
               st, static_cast<const uint16_t*>(a.x), a.state,
               static_cast<uint8_t*>(a.segs.codes[t.p]), a.segs.params[t.p],
               (uint64_t)t.p * a.seg_len, t.g, t.valid, a.coef);
  return e;
}

// The incoming table as the owner pass reads it: the owner's own slot, which
// the caller leaves unset, and every slot from P on point at another rank's
// payload (the owner's outgoing one when P = 1), so that the kernel can load
// a fixed number of slots without branches.
SegTable owner_table(const LaunchArgs& a) {
  SegTable t = a.segs;
  const int other = (a.rank + 1) % a.P;
  void* codes = a.P > 1 ? a.segs.codes[other] : a.out_codes;
  uint32_t* params = a.P > 1 ? a.segs.params[other] : a.out_params;
  for (int p = 0; p < kMaxRanks; ++p) {
    if (p == a.rank || p >= a.P) {
      t.codes[p] = codes;
      t.params[p] = params;
    }
  }
  return t;
}

template <int BITS, int IN_T, int ST_T, int OUT_T, int G, int NP, bool NT, bool NTP, bool XCD>
hipError_t launch_k2(const LaunchArgs& a, hipStream_t st) {
  const uint64_t groups = a.seg_len / G;
  const SegTable in = owner_table(a);
  hipError_t e = in_chunks(blocks_for(groups, GroupMap<ST_T, G>::kGroupsPerBlock),
                           [&](uint32_t b0, unsigned nb) {
    return launch(k_owner_reduce_requant<BITS, IN_T, ST_T, OUT_T, G, NP, NT, NTP, XCD>, dim3(nb),
                  dim3(kThreads), st, static_cast<const uint16_t*>(a.x), a.state, in, a.P, a.rank,
                  full_groups(a.n, a.seg_len, G), a.seg_len, b0,
                  static_cast<uint8_t*>(a.out_codes), a.out_params, a.coef);
  });
  const Tail t = tail_of(a.n, a.seg_len, G);
  if (e == hipSuccess && t.valid && (int)t.p == a.rank)
    e = launch(k_owner_reduce_requant_tail<BITS, IN_T, ST_T, OUT_T, G>, dim3(1),
               dim3(GroupMap<ST_T, G>::kLanes), st, static_cast<const uint16_t*>(a.x), a.state, in,
               a.P, a.rank, static_cast<uint8_t*>(a.out_codes), a.out_params,
               (uint64_t)t.p * a.seg_len, t.g, t.valid, a.coef);
  return e;
}

template <int BITS, int OUT_T, int G, int CH, bool NT, bool NTP>
hipError_t launch_k3(const LaunchArgs& a, hipStream_t st) {
  constexpr uint32_t tile = gather_groups_per_block<OUT_T, G, CH>();
  const FullGroups fg = full_groups(a.n, a.seg_len, G);
  const Tail t = tail_of(a.n, a.seg_len, G);
  hipError_t e = hipSuccess;
  if (fg.all / tile > 0)
    e = in_chunks(fg.all / tile, [&](uint32_t b0, unsigned nb) {
      return launch(k_dequant_gather<BITS, OUT_T, G, CH, NT, NTP>, dim3(nb, a.P), dim3(kThreads), st,
                    a.segs, fg, a.seg_len, b0, a.out);
    });
  if (e == hipSuccess && (fg.all % tile || fg.in_last % tile || t.valid))
    e = launch(k_dequant_gather_tail<BITS, OUT_T, G, CH>, dim3(1, a.P), dim3(kThreads), st, a.segs,
               fg, a.n, a.seg_len, a.out);
  return e;
}

// Nontemporal loads and stores for every streamed array, except the owner
// pass's incoming payloads: the two halves of a 128-byte code line belong to
// neighbouring waves of one block, and a nontemporal first read makes the
// second fetch the line again.
constexpr bool kNT = true;
constexpr bool kNTOwnerPayload = false;
// XCD-contiguous block order: the owner pass reads P-1 parameter arrays at 4
// bytes per group and gains from it; the entry pass measured slightly slower.
constexpr bool kXcdOrderEntry = false, kXcdOrderOwner = true;
// Chunks per lane of the gather pass.
constexpr int kGatherChunks = 2;

// Runtime -> template dispatch: each call hands f one std::integral_constant.
template <int V>
using IC = std::integral_constant<int, V>;

template <typename F>
void with_bits(int v, F&& f) { if (v == 4) f(IC<4>{}); else f(IC<8>{}); }
template <typename F>
void with_group(int v, F&& f) {
  if (v == 32) f(IC<32>{});
  else if (v == 64) f(IC<64>{});
  else f(IC<128>{});
}
template <typename F>
void with_in(int v, F&& f) { if (v == kInF16) f(IC<kInF16>{}); else f(IC<kInBF16>{}); }
template <typename F>
void with_state(int v, F&& f) { if (v == kStateBF16) f(IC<kStateBF16>{}); else f(IC<kStateF32>{}); }
template <typename F>
void with_out(int v, F&& f) { if (v == kOutF32) f(IC<kOutF32>{}); else f(IC<kOutBF16>{}); }
// Payload slots the owner pass loads: P rounded up to a power of two (>= 2).
template <typename F>
void with_slots(int P, F&& f) {
  if (P <= 2) f(IC<2>{});
  else if (P <= 4) f(IC<4>{});
  else if (P <= 8) f(IC<8>{});
  else f(IC<kMaxRanks>{});
}

hipError_t run_quant_feedback(const LaunchArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  with_group(a.group, [&](auto G) { with_bits(a.bits, [&](auto B) { with_in(a.in_dtype, [&](auto I) {
    with_state(a.state_dtype, [&](auto S) {
      e = launch_k1<B(), I(), S(), G(), kNT, kXcdOrderEntry>(a, st);
    }); }); }); });
  return e;
}

hipError_t run_owner_reduce_requant(const LaunchArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  with_group(a.group, [&](auto G) { with_bits(a.bits, [&](auto B) { with_in(a.in_dtype, [&](auto I) {
    with_state(a.state_dtype, [&](auto S) { with_out(a.out_dtype, [&](auto O) {
      with_slots(a.P, [&](auto NP) {
        e = launch_k2<B(), I(), S(), O(), G(), NP(), kNT, kNTOwnerPayload, kXcdOrderOwner>(a, st);
      }); }); }); }); }); });
  return e;
}

hipError_t run_dequant_gather(const LaunchArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  with_group(a.group, [&](auto G) { with_bits(a.bits, [&](auto B) { with_out(a.out_dtype, [&](auto O) {
    e = launch_k3<B(), O(), G(), kGatherChunks, kNT, kNT>(a, st);
  }); }); });
  return e;
}

hipError_t run_zero(void* p, uint64_t bytes, hipStream_t st) {
  const uint64_t n16 = bytes / 16;
  uint64_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > kZeroGridCap) blocks = kZeroGridCap;
  if (blocks == 0) blocks = 1;
  return launch(k_zero, dim3((unsigned)blocks), dim3(kThreads), st, static_cast<uint8_t*>(p), bytes);
}

}  // namespace echo
