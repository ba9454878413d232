// Status strings, last-error storage, region counts and argument checks.
// Pure host C++: no HIP call is made here, so everything in this file works
// on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "pop_internal.h"

namespace pop {

static thread_local char g_err[512];

pop_status fail(pop_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

int& debug_nesting() {
  static thread_local int depth = 0;
  return depth;
}

// Round half away from zero (C's round()).
static int64_t round_half_away(double v) { return (int64_t)round(v); }

static double clamp01(double v) { return v < 0.0 ? 0.0 : (v > 1.0 ? 1.0 : v); }

// POP notes, "Key design 1": thresholds at the quantiles r - delta and
// r + delta (delta = gamma), taken as order statistics at the cut ranks
// round(p * d_ff).  "Key design 2": |R| plus the selected candidates equals
// the live count round((1 - r) * d_ff).
pop_counts counts(int32_t d_ff, double r, double gamma) {
  pop_counts c;
  const double n = (double)d_ff;
  const double p_lo = clamp01(r - gamma);
  const double p_hi = clamp01(r + gamma);
  c.d_ff = d_ff;
  c.c_low = (int32_t)round_half_away(p_lo * n);
  c.c_high = (int32_t)round_half_away(p_hi * n);
  c.n_live = (int32_t)round_half_away((1.0 - r) * n);
  int32_t c_mid = d_ff - c.n_live;
  if (c_mid < c.c_low) c_mid = c.c_low;
  if (c_mid > c.c_high) c_mid = c.c_high;
  c.n_P = c.c_low;
  c.n_C = c.c_high - c.c_low;
  c.n_R = d_ff - c.c_high;
  c.k = c.c_high - c_mid;
  return c;
}

int32_t live_count(int32_t d_ff, double r) { return (int32_t)round_half_away((1.0 - r) * (double)d_ff); }

int32_t topk_count(int32_t d_ff, double r, int32_t n_R, int32_t n_C) {
  int32_t k = live_count(d_ff, r) - n_R;
  if (k < 0) k = 0;
  if (k > n_C) k = n_C;
  return k;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

int elem_bytes(pop_dtype dt) { return dt == POP_BF16 ? 2 : 4; }

pop_status check_dtype_width(pop_dtype dt, int64_t d) {
  if (dt != POP_F32 && dt != POP_BF16) return fail(POP_ERR_UNSUPPORTED_DTYPE, "dtype %d is not POP_F32 or POP_BF16", (int)dt);
  if (d <= 0 || d > POP_MAX_D) return fail(POP_ERR_BAD_SHAPE, "d=%lld outside [1, %d]", (long long)d, POP_MAX_D);
  const int vec = dt == POP_BF16 ? 8 : 4;
  if (d % vec != 0) return fail(POP_ERR_BAD_SHAPE, "d=%lld is not a multiple of %d for this dtype", (long long)d, vec);
  return POP_OK;
}

pop_status check_rate(double r, double gamma) {
  if (!(r >= 0.0 && r < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
  if (!(gamma >= 0.0 && gamma < 1.0)) return fail(POP_ERR_INVALID_ARGUMENT, "gamma=%g outside [0, 1)", gamma);
  return POP_OK;
}

}  // namespace pop

extern "C" {

const char* pop_status_string(pop_status s) {
  switch (s) {
    case POP_OK: return "POP_OK";
    case POP_ERR_INVALID_ARGUMENT: return "POP_ERR_INVALID_ARGUMENT";
    case POP_ERR_UNSUPPORTED_DTYPE: return "POP_ERR_UNSUPPORTED_DTYPE";
    case POP_ERR_BAD_SHAPE: return "POP_ERR_BAD_SHAPE";
    case POP_ERR_MISALIGNED: return "POP_ERR_MISALIGNED";
    case POP_ERR_WORKSPACE_TOO_SMALL: return "POP_ERR_WORKSPACE_TOO_SMALL";
    case POP_ERR_HIP: return "POP_ERR_HIP";
  }
  return "POP_ERR_UNKNOWN";
}

const char* pop_last_error(void) { return pop::g_err; }

pop_status pop_partition_counts(int32_t d_ff, double r, double gamma, pop_counts* out) {
  pop::clear_error();
  if (out == nullptr) return pop::fail(POP_ERR_INVALID_ARGUMENT, "out is NULL");
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return pop::fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  pop_status s = pop::check_rate(r, gamma);
  if (s != POP_OK) return s;
  *out = pop::counts(d_ff, r, gamma);
  return POP_OK;
}

pop_status pop_decode_topk_count(int32_t d_ff, double r, int32_t n_R, int32_t n_C, int32_t* k) {
  pop::clear_error();
  if (k == nullptr) return pop::fail(POP_ERR_INVALID_ARGUMENT, "k is NULL");
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return pop::fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (!(r >= 0.0 && r < 1.0)) return pop::fail(POP_ERR_INVALID_ARGUMENT, "r=%g outside [0, 1)", r);
  if (n_R < 0 || n_C < 0 || (int64_t)n_R + n_C > d_ff)
    return pop::fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d inconsistent with d_ff=%d", n_R, n_C, d_ff);
  *k = pop::topk_count(d_ff, r, n_R, n_C);
  return POP_OK;
}

pop_status pop_check_lists(const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, const int32_t* P,
                           int32_t n_P, int32_t d_ff) {
  pop::clear_error();
  if (d_ff < 1 || d_ff > POP_MAX_D_FF) return pop::fail(POP_ERR_BAD_SHAPE, "d_ff=%d outside [1, %d]", d_ff, POP_MAX_D_FF);
  if (n_R < 0 || n_C < 0 || n_P < 0 || (int64_t)n_R + n_C + n_P > d_ff)
    return pop::fail(POP_ERR_INVALID_ARGUMENT, "n_R=%d, n_C=%d, n_P=%d inconsistent with d_ff=%d", n_R, n_C, n_P,
                     d_ff);
  const int32_t* lists[3] = {R, C, P};
  const int32_t ns[3] = {n_R, n_C, n_P};
  const char* names[3] = {"R", "C", "P"};
  std::vector<signed char> owner((size_t)d_ff, (signed char)-1);  // the list holding each channel
  for (int l = 0; l < 3; ++l) {
    if (ns[l] > 0 && lists[l] == nullptr) return pop::fail(POP_ERR_INVALID_ARGUMENT, "%s is NULL with %d entries", names[l], ns[l]);
    for (int32_t i = 0; i < ns[l]; ++i) {
      const int32_t c = lists[l][i];
      if (c < 0 || c >= d_ff)
        return pop::fail(POP_ERR_INVALID_ARGUMENT, "%s[%d] = %d outside [0, %d)", names[l], i, c, d_ff);
      if (i > 0 && c <= lists[l][i - 1])
        return pop::fail(POP_ERR_INVALID_ARGUMENT, "%s[%d] = %d does not follow %s[%d] = %d in ascending order",
                         names[l], i, c, names[l], i - 1, lists[l][i - 1]);
      if (owner[(size_t)c] >= 0)
        return pop::fail(POP_ERR_INVALID_ARGUMENT, "channel %d is in %s and %s (%s[%d])", c, names[owner[(size_t)c]],
                         names[l], names[l], i);
      owner[(size_t)c] = (signed char)l;
    }
  }
  return POP_OK;
}

}  // extern "C"
