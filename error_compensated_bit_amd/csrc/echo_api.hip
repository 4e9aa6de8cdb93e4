// echo_api.hip -- the C ABI declared in include/echo.h: argument validation,
// kernel-argument marshalling and launch.  Every check runs before the first
// HIP call, so invalid arguments are reported without touching a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "echo.h"
#include "echo_internal.h"

using echo::LaunchArgs;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_config(const echo_config* c) {
  if (!c) return ECHO_ERR_ARG;
  if (c->bits != 4 && c->bits != 8) return ECHO_ERR_ARG;
  if (c->group != 32 && c->group != 64 && c->group != 128) return ECHO_ERR_ARG;
  if (c->in_dtype != ECHO_IN_BF16 && c->in_dtype != ECHO_IN_F16) return ECHO_ERR_ARG;
  if (c->out_dtype != ECHO_OUT_BF16 && c->out_dtype != ECHO_OUT_F32) return ECHO_ERR_ARG;
  if (c->state_dtype != ECHO_STATE_F32 && c->state_dtype != ECHO_STATE_BF16) return ECHO_ERR_ARG;
  if (!isfinite(c->eta)) return ECHO_ERR_ARG;
  if (!(c->beta_short >= 0.0f && c->beta_short < 1.0f)) return ECHO_ERR_ARG;
  if (!(c->beta_long >= 0.0f && c->beta_long < 1.0f)) return ECHO_ERR_ARG;
  if (!(c->mix_long >= 0.0f && c->mix_long <= 1.0f)) return ECHO_ERR_ARG;
  return ECHO_OK;
}

// Segments of whole groups: ceil(n/P) rounded up to a multiple of the group.
int64_t segment_len(int64_t n, int P, int group) {
  const int64_t per = (n + P - 1) / P;
  return (per + group - 1) / group * group;
}

// Longest message segment_len() is evaluated for: far beyond any valid shape
// (16 ranks * 128 * 2^31 groups = 2^42), and small enough that its rounding
// cannot overflow.
constexpr int64_t kMaxLen = (int64_t)1 << 48;

// P ranks, message of n >= 1 elements; a segment may hold at most 2^31 groups
// (the kernels' 32-bit group index then cannot wrap).
int check_shape(int P, int64_t n, int group) {
  if (P < 1 || P > ECHO_MAX_RANKS) return ECHO_ERR_ARG;
  if (n <= 0 || n > kMaxLen) return ECHO_ERR_SHAPE;
  if (segment_len(n, P, group) / group > ((int64_t)1 << 31)) return ECHO_ERR_SHAPE;
  return ECHO_OK;
}

int check_buf(const void* p) {
  if (!p) return ECHO_ERR_ARG;
  return aligned16(p) ? ECHO_OK : ECHO_ERR_ALIGN;
}

int check_seg(const echo_seg* s) {
  if (!s) return ECHO_ERR_ARG;
  int rc = check_buf(s->codes);
  if (rc) return rc;
  return check_buf(s->params);
}

// Moving-average weights, computed in double from the float parameters and
// rounded once: a residual r enters S with (1-bS)(1-mix) and L with (1-bL)mix.
echo::Coef make_coef(const echo_config* c) {
  echo::Coef k;
  k.eta = c->eta;
  k.bS = c->beta_short;
  k.bL = c->beta_long;
  k.aS = (float)((1.0 - (double)c->beta_short) * (1.0 - (double)c->mix_long));
  k.aL = (float)((1.0 - (double)c->beta_long) * (double)c->mix_long);
  return k;
}

LaunchArgs base_args(const echo_config* c, int P, int rank, int64_t n) {
  LaunchArgs a;
  memset(&a, 0, sizeof a);
  a.bits = c->bits;
  a.group = c->group;
  a.in_dtype = c->in_dtype;
  a.out_dtype = c->out_dtype;
  a.state_dtype = c->state_dtype;
  a.P = P;
  a.rank = rank;
  a.n = (uint64_t)n;
  a.seg_len = (uint64_t)segment_len(n, P, c->group);
  a.coef = make_coef(c);
  return a;
}

int launched(hipError_t e) { return e == hipSuccess ? ECHO_OK : ECHO_ERR_HIP; }

}  // namespace

extern "C" {

int echo_state_reset(const echo_config* cfg, void* state, int64_t n, void* stream) {
  if (!cfg) return ECHO_ERR_ARG;
  if (cfg->state_dtype != ECHO_STATE_F32 && cfg->state_dtype != ECHO_STATE_BF16) return ECHO_ERR_ARG;
  if (n <= 0 || n > kMaxLen) return ECHO_ERR_ARG;
  int rc;
  if ((rc = check_buf(state))) return rc;
  return launched(echo::run_zero(state, echo_state_bytes(n, cfg->state_dtype),
                                 static_cast<hipStream_t>(stream)));
}

int echo_quantize_feedback(const echo_config* cfg, int P, int rank, int64_t n, const void* x,
                           void* state, const echo_seg* out, void* stream) {
  int rc;
  if ((rc = check_config(cfg)) || (rc = check_shape(P, n, cfg->group))) return rc;
  if (rank < 0 || rank >= P) return ECHO_ERR_ARG;
  if ((rc = check_buf(x)) || (rc = check_buf(state))) return rc;
  if (!out) return ECHO_ERR_ARG;
  LaunchArgs a = base_args(cfg, P, rank, n);
  for (int p = 0; p < P; ++p) {
    if (p == rank) continue;
    if ((rc = check_seg(&out[p]))) return rc;
    a.segs.codes[p] = out[p].codes;
    a.segs.params[p] = out[p].params;
  }
  if (P == 1) return ECHO_OK;  // nothing is sent when a rank owns the whole message
  a.x = x;
  a.state = state;
  return launched(echo::run_quant_feedback(a, static_cast<hipStream_t>(stream)));
}

int echo_owner_reduce_requant(const echo_config* cfg, int P, int rank, int64_t n, const void* x,
                              void* state, const echo_seg* in, const echo_seg* out,
                              void* stream) {
  int rc;
  if ((rc = check_config(cfg)) || (rc = check_shape(P, n, cfg->group))) return rc;
  if (rank < 0 || rank >= P) return ECHO_ERR_ARG;
  if ((rc = check_buf(x)) || (rc = check_buf(state))) return rc;
  if (!in && P > 1) return ECHO_ERR_ARG;
  if ((rc = check_seg(out))) return rc;
  LaunchArgs a = base_args(cfg, P, rank, n);
  for (int p = 0; p < P; ++p) {
    if (p == rank) continue;
    if ((rc = check_seg(&in[p]))) return rc;
    a.segs.codes[p] = in[p].codes;
    a.segs.params[p] = in[p].params;
  }
  a.x = x;
  a.state = state;
  a.out_codes = out->codes;
  a.out_params = out->params;
  return launched(echo::run_owner_reduce_requant(a, static_cast<hipStream_t>(stream)));
}

int echo_dequant_gather(const echo_config* cfg, int P, int64_t n, const echo_seg* in, void* out,
                        void* stream) {
  int rc;
  if ((rc = check_config(cfg)) || (rc = check_shape(P, n, cfg->group))) return rc;
  if (!in) return ECHO_ERR_ARG;
  if ((rc = check_buf(out))) return rc;
  LaunchArgs a = base_args(cfg, P, 0, n);
  for (int p = 0; p < P; ++p) {
    if ((rc = check_seg(&in[p]))) return rc;
    a.segs.codes[p] = in[p].codes;
    a.segs.params[p] = in[p].params;
  }
  a.out = out;
  return launched(echo::run_dequant_gather(a, static_cast<hipStream_t>(stream)));
}

size_t echo_codes_bytes(int64_t seg_len, int bits) {
  if (seg_len <= 0 || seg_len > kMaxLen || (bits != 4 && bits != 8)) return 0;
  if (bits == 4 && seg_len % 2) return 0;
  return (size_t)seg_len * (size_t)bits / 8;
}

int64_t echo_segment_len(int64_t n, int P, int group) {
  if (n <= 0 || n > kMaxLen || P < 1 || P > ECHO_MAX_RANKS ||
      (group != 32 && group != 64 && group != 128))
    return 0;
  return segment_len(n, P, group);
}

size_t echo_state_bytes(int64_t n, int state_dtype) {
  if (n <= 0 || n > kMaxLen) return 0;
  if (state_dtype == ECHO_STATE_F32) return (size_t)n * 8;
  if (state_dtype == ECHO_STATE_BF16) return (size_t)n * 4;
  return 0;
}

size_t echo_params_bytes(int64_t seg_len, int group) {
  if (seg_len <= 0 || group <= 0 || seg_len % group) return 0;
  return (size_t)(seg_len / group) * sizeof(uint32_t);
}

const char* echo_error_string(int code) {
  switch (code) {
    case ECHO_OK: return "ok";
    case ECHO_ERR_ARG: return "invalid argument";
    case ECHO_ERR_SHAPE: return "message length is not positive or a segment exceeds 2^31 groups";
    case ECHO_ERR_ALIGN: return "buffer not 16-byte aligned";
    case ECHO_ERR_HIP: return "HIP launch error";
    default: return "unknown error";
  }
}

}  // extern "C"
