/*
 * echo_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU model of one rank's share of an Echo all-reduce
 * call.  It exists to check the GPU library: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.  Everything is one element at a time, in the order the method
 * describes, with no blocking, fusion or reordering.
 *
 * Pages this file follows (cited by tag below):
 *   [EA]   "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for
 *          LLM Training and Inference" -- the arXiv abstract on that page.
 *   [EKP]  same page, "Key Points".
 *   [JP-W] "テンソル並列の通信を4bitに圧縮する「Echo」" (Japanese explainer),
 *          section "なぜ4bit通信は難しかったのか" (why 4-bit was hard).
 *   [JP-1] same page, section "Echoの仕組み①" (sum in high precision,
 *          carry in low precision).
 *   [JP-2] same page, section "Echoの仕組み②" (dual-time-constant feedback).
 *   [JP-T] same page, section "理論保証" (the bound).
 *   [JP-F] same page, section "よくある質問" (4-bit integers + half-precision
 *          parameters; ~3.8x ceiling).
 *
 * Arithmetic: IEEE binary32 throughout (the pages fix the sum at "high
 * precision" and the payload at 4-bit integers with half-precision
 * parameters; the codes are decided in binary32 as the GPU decides them).
 * Build with -ffp-contract=off so that no a*b+c is fused; the only fused
 * multiply-add is the explicit fmaf() of the dequantizer.  Round to nearest
 * even everywhere (rintf under the default rounding mode; the binary16 and
 * bfloat16 conversions below are written from the IEEE-754 definitions).
 *
 * Readings of points the pages leave open (all recorded with reasons in the
 * design notes of this repository):
 *   - quantizer: per group of G elements, zero = fp16(min), scale =
 *     fp16((max - zero) / qmax), code = clamp(rint((v - zero) * (1/scale)),
 *     0, qmax), dequant = fma(code, scale, zero); a scale that is not
 *     positive after rounding gives all codes 0 and dequant = zero;
 *     zero and scale are clamped to the finite fp16 range, -0 -> +0.
 *   - ownership: P contiguous segments of seg_len = ceil(ceil(n/P)/G)*G
 *     elements (whole groups), rank p owns segment p = [p*seg_len,
 *     min((p+1)*seg_len, n)); only the last non-empty segment can end in a
 *     partial group, and trailing segments may be empty.  Groups are
 *     numbered within a segment in element order.  A partial group is
 *     quantized over its valid elements; an INT4 segment of odd length
 *     leaves the last byte's high nibble 0.
 *   - payload: INT4 codes two per byte, even element in the low nibble;
 *     INT8 one per byte; params[group] = scale_bits | zero_bits << 16.
 *   - owner sum: fp32, ranks in order 0..P-1, the owner's own term is its
 *     unquantized feedback-added value.
 *   - residual: non-owned v - dequant; owned acc - o, where o is the value
 *     the output will hold (bf16-rounded when the output is bf16).
 *   - state: per element, per rank, two fp32 moving averages S (short
 *     memory, decay bS) and L (long memory, decay bL); each residual is
 *     split with shares (1 - lam) and lam; the feedback added to the next
 *     call's input is eta * (S + L).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define EO_OK 0
#define EO_ERR_ARG -1
#define EO_ERR_SHAPE -2

#define EO_IN_BF16 0
#define EO_IN_F16 1
#define EO_OUT_BF16 0
#define EO_OUT_F32 1
#define EO_STATE_F32 0
#define EO_STATE_BF16 1

/* ------------------------------------------------------------------ */
/* binary32 <-> binary16 / bfloat16, from the IEEE-754 definitions      */
/* ------------------------------------------------------------------ */

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round the non-negative integer `m` right by `sh` bits, ties to even. */
static uint32_t shift_rne(uint32_t m, int sh)
{
    if (sh <= 0) return m;
    if (sh >= 32) return 0;
    uint32_t kept = m >> sh;
    uint32_t rest = m - (kept << sh);
    uint32_t half = 1u << (sh - 1);
    if (rest > half || (rest == half && (kept & 1u))) kept += 1u;
    return kept;
}

/* binary32 -> binary16, round to nearest even; overflow -> infinity. */
uint16_t eo_f32_to_f16(float f)
{
    uint32_t u = bits_of(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e32 = (u >> 23) & 0xffu;
    uint32_t m32 = u & 0x7fffffu;
    if (e32 == 0xffu) { /* infinity or NaN */
        if (m32 == 0) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | 0x7e00u | (m32 >> 13));
    }
    if (e32 == 0) return sign; /* binary32 zero or subnormal: far below 2^-25 */
    int e = (int)e32 - 127;           /* |f| = sig * 2^(e-23), sig has 24 bits */
    uint32_t sig = m32 | 0x800000u;
    if (e >= -14) {
        /* binary16 normal range: 11-bit significand, drop 13 bits. */
        uint32_t s11 = shift_rne(sig, 13);     /* may carry to 2^11 */
        int he = e + 15;
        if (s11 == 0x800u) { s11 = 0x400u; he += 1; }
        if (he >= 31) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | ((uint32_t)he << 10) | (s11 & 0x3ffu));
    }
    /* binary16 subnormal range: value in units of 2^-24 is sig * 2^(e+1). */
    int sh = -(e + 1);                 /* e <= -15 -> sh >= 14 */
    uint32_t units = shift_rne(sig, sh);   /* 0 .. 0x400 (0x400 = min normal) */
    return (uint16_t)(sign | units);
}

float eo_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1fu;
    uint32_t m = (uint32_t)h & 0x3ffu;
    if (e == 0x1fu) return float_of(sign | 0x7f800000u | (m << 13));
    if (e == 0) {
        float mag = ldexpf((float)m, -24);   /* exact */
        return sign ? -mag : mag;
    }
    return float_of(sign | ((e + 112u) << 23) | (m << 13));
}

/* binary32 -> bfloat16 (8-bit exponent, 8-bit significand), RNE. */
uint16_t eo_f32_to_bf16(float f)
{
    uint32_t u = bits_of(f);
    uint32_t e32 = (u >> 23) & 0xffu;
    uint32_t m32 = u & 0x7fffffu;
    if (e32 == 0xffu && m32 != 0) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
    uint32_t mag = u & 0x7fffffffu;
    uint32_t r = shift_rne(mag, 16);   /* carry into the exponent is correct, */
    return (uint16_t)(((u >> 16) & 0x8000u) | r);   /* and reaches inf at the top */
}

float eo_bf16_to_f32(uint16_t b) { return float_of((uint32_t)b << 16); }

/* bulk forms, for exhaustive checks */
void eo_f32_to_f16_array(const float* in, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = eo_f32_to_f16(in[i]); }
void eo_f16_to_f32_array(const uint16_t* in, float* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = eo_f16_to_f32(in[i]); }
void eo_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = eo_f32_to_bf16(in[i]); }

/* ------------------------------------------------------------------ */
/* The quantizer Q over one group ([JP-1] zero-point-aware asymmetric;  */
/* [JP-F] 4-bit integers carried with half-precision parameters).       */
/* ------------------------------------------------------------------ */

/* Quantize v[0..g) with 2^bits levels.  Writes one code per element to
 * q[] (unpacked), the fp16 bit patterns of scale and zero, and the
 * dequantized values deq[] (may be NULL). */
void eo_quantize_group(const float* v, int g, int bits, uint8_t* q,
                       uint16_t* scale_bits, uint16_t* zero_bits, float* deq)
{
    const float qmax = (float)((1 << bits) - 1);
    float mn = v[0], mx = v[0];
    for (int i = 1; i < g; ++i) {
        if (v[i] < mn) mn = v[i];
        if (v[i] > mx) mx = v[i];
    }
    /* zero point: the group minimum, as a finite fp16 value, never -0 */
    float zc = mn;
    if (zc < -65504.0f) zc = -65504.0f;
    if (zc > 65504.0f) zc = 65504.0f;
    uint16_t zh = eo_f32_to_f16(zc);
    if (zh == 0x8000u) zh = 0;
    float zf = eo_f16_to_f32(zh);
    /* step: span above the zero point over the number of steps */
    float s = (mx - zf) / qmax;
    if (!(s > 0.0f)) s = 0.0f;
    if (s > 65504.0f) s = 65504.0f;
    uint16_t sh = eo_f32_to_f16(s);
    float sf = eo_f16_to_f32(sh);
    float inv = (sf > 0.0f) ? 1.0f / sf : 0.0f;
    for (int i = 0; i < g; ++i) {
        float t = (v[i] - zf) * inv;
        float r = rintf(t);
        if (r < 0.0f) r = 0.0f;
        if (r > qmax) r = qmax;
        q[i] = (uint8_t)r;
        if (deq) deq[i] = fmaf((float)q[i], sf, zf);
    }
    *scale_bits = sh;
    *zero_bits = zh;
}

/* dequantize one code with its group's parameters */
static float eo_dequant(uint32_t code, uint32_t param)
{
    float sf = eo_f16_to_f32((uint16_t)(param & 0xffffu));
    float zf = eo_f16_to_f32((uint16_t)(param >> 16));
    return fmaf((float)code, sf, zf);
}

/* ------------------------------------------------------------------ */
/* payload layout helpers                                               */
/* ------------------------------------------------------------------ */

static uint32_t eo_get_code(const uint8_t* codes, int bits, int64_t i)
{
    if (bits == 8) return codes[i];
    uint8_t b = codes[i / 2];
    return (i % 2 == 0) ? (uint32_t)(b & 0x0fu) : (uint32_t)(b >> 4);
}

static void eo_put_code(uint8_t* codes, int bits, int64_t i, uint32_t q)
{
    if (bits == 8) { codes[i] = (uint8_t)q; return; }
    uint8_t* b = &codes[i / 2];
    if (i % 2 == 0) *b = (uint8_t)((*b & 0xf0u) | (q & 0x0fu));
    else            *b = (uint8_t)((*b & 0x0fu) | ((q & 0x0fu) << 4));
}

/* ------------------------------------------------------------------ */
/* element access for inputs and state                                  */
/* ------------------------------------------------------------------ */

static float eo_load_in(const void* x, int in_dtype, int64_t j)
{
    uint16_t h = ((const uint16_t*)x)[j];
    return in_dtype == EO_IN_F16 ? eo_f16_to_f32(h) : eo_bf16_to_f32(h);
}

static float eo_load_state(const void* s, int state_dtype, int64_t j)
{
    if (state_dtype == EO_STATE_BF16) return eo_bf16_to_f32(((const uint16_t*)s)[j]);
    return ((const float*)s)[j];
}

static void eo_store_state(void* s, int state_dtype, int64_t j, float val)
{
    if (state_dtype == EO_STATE_BF16) ((uint16_t*)s)[j] = eo_f32_to_bf16(val);
    else ((float*)s)[j] = val;
}

/* The two moving-average weights, computed once in double from the float
 * parameters and rounded once to float: a residual r enters the short
 * memory with weight (1-bS)(1-lam) and the long memory with (1-bL)lam. */
static void eo_weights(float bS, float bL, float lam, float* aS, float* aL)
{
    *aS = (float)((1.0 - (double)bS) * (1.0 - (double)lam));
    *aL = (float)((1.0 - (double)bL) * (double)lam);
}

/* Feedback-added input ([JP-2]: the stored error is added back into the
 * next call's input with gain eta): v = x + eta * (S + L). */
static float eo_feedback_input(float xf, float S, float L, float eta)
{
    float u = S + L;
    float f = eta * u;
    return xf + f;
}

/* One step of both moving averages with residual r ([JP-2]). */
static void eo_ema_update(void* S, void* L, int state_dtype, int64_t j, float r,
                          float bS, float aS, float bL, float aL)
{
    float s0 = eo_load_state(S, state_dtype, j);
    float l0 = eo_load_state(L, state_dtype, j);
    float s_keep = bS * s0, s_new = aS * r;
    float l_keep = bL * l0, l_new = aL * r;
    eo_store_state(S, state_dtype, j, s_keep + s_new);
    eo_store_state(L, state_dtype, j, l_keep + l_new);
}

/* Segment length (whole groups) and the element count of segment p. */
int64_t eo_segment_len(int64_t n, int P, int group)
{
    int64_t per = (n + P - 1) / P;
    return (per + group - 1) / group * group;
}

static int64_t eo_segment_count(int64_t n, int64_t seg_len, int p)
{
    int64_t start = (int64_t)p * seg_len;
    if (start >= n) return 0;
    return (n - start) < seg_len ? (n - start) : seg_len;
}

static int eo_check_common(int bits, int group, int P, int64_t n)
{
    if (bits != 4 && bits != 8) return EO_ERR_ARG;
    if (group < 1 || group > 256 || P < 1 || P > 64 || n <= 0) return EO_ERR_ARG;
    if (bits == 4 && group % 2 != 0) return EO_ERR_ARG;   /* groups start on byte boundaries */
    return EO_OK;
}

/* INT4: clear the code bytes of one group before its nibbles are written. */
static void eo_clear_codes(uint8_t* codes, int bits, int64_t first, int glen)
{
    if (bits == 8) return;
    for (int64_t b = first / 2; b < (first + glen + 1) / 2; ++b) codes[b] = 0;
}

/* ------------------------------------------------------------------ */
/* Entry pass of rank `rank` ([JP-1]: each GPU quantizes only the       */
/* segments it does not own; [JP-2]: the compensation is fused into     */
/* the entry pass).                                                     */
/* ------------------------------------------------------------------ */

/* For every segment p != rank and every group in it: v = x + eta(S+L),
 * quantize into payload p (codes[p], params[p]), residual r = v - deq,
 * S and L updated in place.  qpass (optional, length n) is incremented
 * once for every element that passes through the quantizer. */
int eo_quantize_feedback(int bits, int group, int in_dtype, int state_dtype,
                         float eta, float bS, float bL, float lam,
                         int P, int rank, int64_t n,
                         const void* x, void* S, void* L,
                         uint8_t* const* codes, uint32_t* const* params,
                         uint32_t* qpass)
{
    int rc = eo_check_common(bits, group, P, n);
    if (rc) return rc;
    if (rank < 0 || rank >= P) return EO_ERR_ARG;
    float aS, aL;
    eo_weights(bS, bL, lam, &aS, &aL);
    const int64_t seg = eo_segment_len(n, P, group);
    float v[256], deq[256];
    uint8_t q[256];
    for (int p = 0; p < P; ++p) {
        if (p == rank) continue;   /* the owned segment is never quantized here */
        const int64_t len = eo_segment_count(n, seg, p);
        for (int64_t gi = 0; gi * group < len; ++gi) {
            const int64_t base = (int64_t)p * seg + gi * group;
            const int glen = (int)((len - gi * group) < group ? (len - gi * group) : group);
            for (int i = 0; i < glen; ++i) {
                int64_t j = base + i;
                v[i] = eo_feedback_input(eo_load_in(x, in_dtype, j),
                                         eo_load_state(S, state_dtype, j),
                                         eo_load_state(L, state_dtype, j), eta);
            }
            uint16_t sh, zh;
            eo_quantize_group(v, glen, bits, q, &sh, &zh, deq);
            params[p][gi] = (uint32_t)sh | ((uint32_t)zh << 16);
            eo_clear_codes(codes[p], bits, gi * group, glen);
            for (int i = 0; i < glen; ++i) {
                int64_t j = base + i;
                eo_put_code(codes[p], bits, gi * group + i, q[i]);
                float r = v[i] - deq[i];
                eo_ema_update(S, L, state_dtype, j, r, bS, aS, bL, aL);
                if (qpass) qpass[j] += 1u;
            }
        }
    }
    return EO_OK;
}

/* ------------------------------------------------------------------ */
/* Owner pass of rank `rank` over its own segment ([JP-1]: the owner    */
/* sums in high precision, requantizes the sum and sends it to all;     */
/* [JP-W]: quantize -> send -> decode -> add -> requantize).            */
/* qpass (optional, length n) counts quantizer passes per element;      */
/* acc_out (optional, one float per element of the segment) receives    */
/* the fp32 sum before requantization.                                  */
/* ------------------------------------------------------------------ */

int eo_owner_reduce_requant(int bits, int group, int in_dtype, int state_dtype,
                            int out_dtype, float eta, float bS, float bL, float lam,
                            int P, int rank, int64_t n,
                            const void* x, void* S, void* L,
                            const uint8_t* const* in_codes,
                            const uint32_t* const* in_params,
                            uint8_t* out_codes, uint32_t* out_params,
                            uint32_t* qpass, float* acc_out)
{
    int rc = eo_check_common(bits, group, P, n);
    if (rc) return rc;
    if (rank < 0 || rank >= P) return EO_ERR_ARG;
    float aS, aL;
    eo_weights(bS, bL, lam, &aS, &aL);
    const int64_t seg = eo_segment_len(n, P, group);
    const int64_t len = eo_segment_count(n, seg, rank);
    float acc[256], deq[256];
    uint8_t q[256];
    for (int64_t gi = 0; gi * group < len; ++gi) {
        const int64_t base = (int64_t)rank * seg + gi * group;
        const int glen = (int)((len - gi * group) < group ? (len - gi * group) : group);
        for (int i = 0; i < glen; ++i) {
            const int64_t j = base + i;
            const int64_t k = gi * group + i;   /* index within the segment */
            float v_own = eo_feedback_input(eo_load_in(x, in_dtype, j),
                                            eo_load_state(S, state_dtype, j),
                                            eo_load_state(L, state_dtype, j), eta);
            float a = 0.0f;
            for (int p = 0; p < P; ++p) {
                float term = (p == rank)
                    ? v_own
                    : eo_dequant(eo_get_code(in_codes[p], bits, k), in_params[p][gi]);
                a = (p == 0) ? term : a + term;
            }
            acc[i] = a;
            if (acc_out) acc_out[k] = a;   /* the fp32 sum, for tests that check it */
        }
        uint16_t sh, zh;
        eo_quantize_group(acc, glen, bits, q, &sh, &zh, deq);
        out_params[gi] = (uint32_t)sh | ((uint32_t)zh << 16);
        eo_clear_codes(out_codes, bits, gi * group, glen);
        for (int i = 0; i < glen; ++i) {
            const int64_t j = base + i;
            eo_put_code(out_codes, bits, gi * group + i, q[i]);
            float o = (out_dtype == EO_OUT_BF16) ? eo_bf16_to_f32(eo_f32_to_bf16(deq[i]))
                                                 : deq[i];
            float r = acc[i] - o;
            eo_ema_update(S, L, state_dtype, j, r, bS, aS, bL, aL);
            if (qpass) qpass[j] += 1u;
        }
    }
    return EO_OK;
}

/* ------------------------------------------------------------------ */
/* Dequantize the gathered payloads into the output ([JP-1]: the owners */
/* distribute their requantized sums to every GPU).                     */
/* ------------------------------------------------------------------ */

int eo_dequant_gather(int bits, int group, int out_dtype, int P, int64_t n,
                      const uint8_t* const* codes, const uint32_t* const* params,
                      void* out)
{
    int rc = eo_check_common(bits, group, P, n);
    if (rc) return rc;
    const int64_t seg = eo_segment_len(n, P, group);
    for (int p = 0; p < P; ++p) {
        const int64_t len = eo_segment_count(n, seg, p);
        for (int64_t k = 0; k < len; ++k) {
            float d = eo_dequant(eo_get_code(codes[p], bits, k), params[p][k / group]);
            int64_t j = (int64_t)p * seg + k;
            if (out_dtype == EO_OUT_BF16) ((uint16_t*)out)[j] = eo_f32_to_bf16(d);
            else ((float*)out)[j] = d;
        }
    }
    return EO_OK;
}

/* Error state at the start of a chain of calls: both memories empty. */
int eo_state_reset(void* S, void* L, int state_dtype, int64_t n)
{
    if (n <= 0) return EO_ERR_ARG;
    for (int64_t j = 0; j < n; ++j) {
        eo_store_state(S, state_dtype, j, 0.0f);
        eo_store_state(L, state_dtype, j, 0.0f);
    }
    return EO_OK;
}
