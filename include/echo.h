/*
 * echo.h -- C ABI of the Echo low-bit all-reduce hot path on one AMD
 * Instinct gfx950 GPU: one rank's share of one all-reduce call.
 *
 * Echo (arXiv 2610.14277) rebuilds a tensor-parallel all-reduce as
 * all-to-all + high-precision sum at the segment owner + all-gather, moves
 * the data as 4-bit (or 8-bit) integers with half-precision group
 * parameters, and feeds the error each call injects back into later calls
 * through two moving averages.  This library holds the per-GPU compute of
 * one call; moving the payloads between GPUs is the caller's job.
 *
 * Pages cited below:
 *   [EA]   "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for
 *          LLM Training and Inference" -- arXiv abstract.
 *   [JP-W] "テンソル並列の通信を4bitに圧縮する「Echo」" (Japanese explainer),
 *          section "なぜ4bit通信は難しかったのか".
 *   [JP-1] same page, section "Echoの仕組み①" (high-precision sum, low-bit
 *          transport, zero-point-aware asymmetric quantization).
 *   [JP-2] same page, section "Echoの仕組み②" (dual-time-constant feedback
 *          fused into the entry pass).
 *   [JP-F] same page, section "よくある質問" (4-bit integers + half-precision
 *          parameters).
 *
 * Layout (every call):
 *   - A message of n >= 1 elements per rank is split into P contiguous
 *     segments of whole groups: seg_len = echo_segment_len(n, P, group) =
 *     ceil(ceil(n/P) / group) * group, and rank p owns segment p =
 *     [p*seg_len, min((p+1)*seg_len, n)).  When n is a multiple of P*group
 *     every segment holds n/P elements; otherwise the last non-empty segment
 *     ends in a partial group (quantized over its valid elements) and the
 *     segments after it are empty.
 *   - Groups of `group` consecutive elements of a segment (128 by default;
 *     32 and 64 are also accepted) share one scale and one zero point, both
 *     IEEE binary16; params[g] = scale | zero << 16.
 *   - Codes: bits = 4 -> two per byte, the even element in the low nibble
 *     (an odd-length segment leaves its last high nibble 0); bits = 8 -> one
 *     per byte.  Codes and params of a segment are two separate arrays
 *     ("payload", echo_seg), always sized for seg_len elements:
 *     echo_codes_bytes(seg_len, bits) and echo_params_bytes(seg_len, group).
 *   - Dequantized value = fma(code, scale, zero) in fp32.
 *   - Error state: one array per rank of 2n elements of the config's
 *     state type (fp32 or bf16) holding the short memory S and the long
 *     memory L of each element side by side: state[2j] = S_j,
 *     state[2j+1] = L_j.  It is updated in place and persists between
 *     calls (checkpointing it = copying it).
 *
 * Conventions:
 *   - All buffer pointers are device pointers, 16-byte aligned; the caller
 *     owns every buffer.  echo_config and echo_seg arrays are host memory
 *     read during the call only.  The library allocates nothing and keeps
 *     no state between calls; calls on different streams touching disjoint
 *     buffers may run concurrently.
 *   - All calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and never synchronize.
 *   - Payload buffers must not overlap x, the state, the output or each other.
 *   - Every call validates all arguments before touching the GPU and
 *     returns ECHO_OK or a negative error code.  ECHO_ERR_ARG, ECHO_ERR_SHAPE
 *     and ECHO_ERR_ALIGN are returned before anything is launched.  A call
 *     may make more than one launch (the one partial group of a ragged
 *     message runs in a launch of its own, and a segment of more than about
 *     2^33 elements is split over several); ECHO_ERR_HIP can therefore come
 *     after some launches of the call went out, and the state and payloads
 *     it writes may then be partly updated: reset (or restore) the state
 *     before the next call.  No exception crosses this interface.
 */
#ifndef ECHO_H
#define ECHO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define ECHO_OK          0
#define ECHO_ERR_ARG    -1   /* null pointer, unsupported or out-of-range parameter */
#define ECHO_ERR_SHAPE  -2   /* n <= 0, or a segment of more than 2^31 groups
                                (every n > 2^48 is one) */
#define ECHO_ERR_ALIGN  -3   /* a buffer pointer is not 16-byte aligned */
#define ECHO_ERR_HIP    -4   /* the HIP runtime reported an error at a launch (earlier
                                launches of the same call may have gone out) */

/* element types */
#define ECHO_IN_BF16     0   /* 16-bit input message: bfloat16 */
#define ECHO_IN_F16      1   /*                       IEEE binary16 */
#define ECHO_OUT_BF16    0   /* all-reduce output: bfloat16 (round to nearest even) */
#define ECHO_OUT_F32     1   /*                    fp32 */
#define ECHO_STATE_F32   0   /* error state S, L: fp32 */
#define ECHO_STATE_BF16  1   /*                   bfloat16 (round to nearest even) */

#define ECHO_MAX_RANKS  16
#define ECHO_GROUP      128  /* default group size; 32 and 64 are also accepted */

typedef struct echo_config {
    int32_t bits;        /* 4 or 8: code width ([JP-F]; 8-bit for early sites) */
    int32_t group;       /* elements per scale/zero pair: 32, 64 or 128 */
    int32_t in_dtype;    /* ECHO_IN_*    */
    int32_t out_dtype;   /* ECHO_OUT_*   */
    int32_t state_dtype; /* ECHO_STATE_* */
    float   eta;         /* feedback gain; finite */
    float   beta_short;  /* decay of the short memory, in [0, 1) */
    float   beta_long;   /* decay of the long memory, in [0, 1) */
    float   mix_long;    /* share of each residual given to the long memory, in [0, 1] */
} echo_config;

/* One segment's payload: codes (seg_len * bits/8 bytes) and params (seg_len/group words). */
typedef struct echo_seg {
    void*     codes;
    uint32_t* params;
} echo_seg;

/*
 * echo_state_reset -- empty both memories: S_j = L_j = +0 for j < n.
 *   state: device array of echo_state_bytes(n, cfg->state_dtype) bytes.
 *   The feedback of [JP-2] carries error into later calls; a chain of calls
 *   starts from an empty state.  Implemented as a fill kernel (no memset
 *   node), so it may be captured in a HIP graph.
 *   Errors: ECHO_ERR_ARG (null cfg/pointer, n <= 0 or n > 2^48, bad state type),
 *   ECHO_ERR_ALIGN, ECHO_ERR_HIP.
 */
int echo_state_reset(const echo_config* cfg, void* state, int64_t n, void* stream);

/*
 * echo_quantize_feedback -- entry pass of rank `rank` ([JP-1], [JP-2]).
 *   For every element j of every segment p != rank:
 *     v = x[j] + eta * (S_j + L_j)                   (fp32, unfused)
 *   each group of v is quantized to `bits` with an fp16 zero point
 *   (the group minimum) and fp16 step ((max - zero) / (2^bits - 1)), codes
 *   round half to even; the payload goes to out[p].  With r = v - dequant:
 *     S_j = beta_short * S_j + (1-beta_short)(1-mix_long) * r
 *     L_j = beta_long  * L_j + (1-beta_long) * mix_long   * r
 *   (each product rounded to fp32, then the sum; the two weights are
 *   computed in double from the float parameters and rounded once).
 *   The owned segment is not read or written (its feedback is applied by
 *   echo_owner_reduce_requant); P = 1 launches nothing.
 *   x: device, n 16-bit elements (in_dtype).  state: device, n (S, L) pairs.
 *   out: host array of P echo_seg; out[rank] is ignored, every other entry
 *   must point at a payload sized for seg_len elements (nothing is written
 *   for an empty segment).
 *   Errors: ECHO_ERR_ARG, ECHO_ERR_SHAPE, ECHO_ERR_ALIGN, ECHO_ERR_HIP.
 */
int echo_quantize_feedback(const echo_config* cfg, int P, int rank, int64_t n,
                           const void* x, void* state,
                           const echo_seg* out, void* stream);

/*
 * echo_owner_reduce_requant -- owner pass of rank `rank` over its segment
 * ([JP-1]: the owner sums in high precision and requantizes; [JP-W]).
 *   For every element j of segment `rank`:
 *     v_own = x[j] + eta * (S_j + L_j)
 *     acc   = sum over p = 0..P-1 in that order of
 *             (p == rank ? v_own : dequant of in[p]'s code for j)    (fp32)
 *   acc is requantized per group into *out (same quantizer as above);
 *   o = the output value of j (bf16-rounded dequant for ECHO_OUT_BF16,
 *   the fp32 dequant for ECHO_OUT_F32); r = acc - o; S_j and L_j are
 *   updated with r as above.  Segments p != rank of x and state are not
 *   read or written.
 *   in: host array of P echo_seg (payloads the other ranks sent for this
 *   segment); in[rank] is ignored.  out: host pointer to one echo_seg.
 *   Errors: ECHO_ERR_ARG, ECHO_ERR_SHAPE, ECHO_ERR_ALIGN, ECHO_ERR_HIP.
 */
int echo_owner_reduce_requant(const echo_config* cfg, int P, int rank, int64_t n,
                              const void* x, void* state,
                              const echo_seg* in, const echo_seg* out, void* stream);

/*
 * echo_dequant_gather -- turn the P owners' requantized payloads into the
 * all-reduce output ([JP-1]: the owner's requantized sum goes to every GPU).
 *   out[p*seg_len + k] = dequant of in[p]'s code k, as out_dtype (bf16
 *   round to nearest even, or fp32), for every p < P and every k below the
 *   element count of segment p (seg_len, fewer in the last non-empty
 *   segment, none after it); nothing past out[n-1] is written.
 *   in: host array of P echo_seg, every entry a valid payload (an empty
 *   segment's payload is not read).  out: device, n elements.
 *   Errors: ECHO_ERR_ARG, ECHO_ERR_SHAPE, ECHO_ERR_ALIGN, ECHO_ERR_HIP.
 */
int echo_dequant_gather(const echo_config* cfg, int P, int64_t n,
                        const echo_seg* in, void* out, void* stream);

/* Sizes (0 for invalid input): the segment length of an n-element message
 * over P ranks, the payload of a segment of seg_len elements, and the error
 * state of an n-element message. */
int64_t echo_segment_len(int64_t n, int P, int group);
size_t echo_codes_bytes(int64_t seg_len, int bits);
size_t echo_params_bytes(int64_t seg_len, int group);
size_t echo_state_bytes(int64_t n, int state_dtype);

/* Static description of an error code. */
const char* echo_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* ECHO_H */
