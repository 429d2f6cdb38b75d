// Host planner of libdla (see dla_plan.h).  No HIP here: this file also
// builds with g++ alone for CPU tests under the address and UB sanitizers.
#include "dla_plan.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

namespace dla {

static thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("DLA_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

// One line per plan: sizes, patterns and the derived layout (DLA_LOG=1).
static void log_plan(const Plan& p) {
  char pats[kMaxP * 24] = "";
  size_t n = 0;
  for (int i = 0; i < p.P && n < sizeof(pats); ++i)
    n += snprintf(pats + n, sizeof(pats) - n, "%s(%d,%d)%s", i ? "," : "", p.w[i], p.r[i],
                  p.span[i] ? "*" : "");
  fprintf(stderr,
          "[dla] plan: B=%lld N=%lld H=%lld %s %s patterns %s primary=%d merge=%d finalize=%d "
          "pairs=%lld ws_fwd=%zu ws_bwd=%zu%s\n",
          (long long)p.B, (long long)p.N, (long long)p.H, p.dtype == DLA_BF16 ? "bf16" : "fp32",
          p.causal ? "causal" : "non-causal", pats, p.prim, (int)p.need_combine, (int)p.need_finalize,
          (long long)p.pairs, p.ws_fwd, p.ws_bwd, p.shard ? " (shard; * spans devices)" : "");
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int make_plan(const dla_desc* desc, const dla_shape* shape, Plan* plan, const dla_shard* shard) {
  if (!desc || !shape || !plan) return fail(DLA_E_INVALID, "null descriptor or shape");
  Plan& p = *plan;
  memset(&p, 0, sizeof(p));
  if (desc->num_patterns < 1 || desc->num_patterns > kMaxP)
    return fail(DLA_E_INVALID, "num_patterns=%d outside 1..%d", desc->num_patterns, kMaxP);
  if (!desc->patterns) return fail(DLA_E_INVALID, "null pattern array");
  if (desc->causal != 0 && desc->causal != 1)
    return fail(DLA_E_INVALID, "causal=%d is not 0 or 1", desc->causal);
  if (!isfinite(desc->scale) || !(desc->scale > 0.0f))
    return fail(DLA_E_INVALID, "scale must be finite and > 0");
  if (shape->dtype != DLA_F32 && shape->dtype != DLA_BF16)
    return fail(DLA_E_UNSUPPORTED, "dtype=%d is neither DLA_F32 nor DLA_BF16", shape->dtype);
  if (shape->D != kD) return fail(DLA_E_UNSUPPORTED, "head dim D=%lld, only 64 is supported",
                                  (long long)shape->D);
  if (shape->B < 0 || shape->H < 0 || shape->N < 1)
    return fail(DLA_E_INVALID, "bad sizes B=%lld N=%lld H=%lld", (long long)shape->B,
                (long long)shape->N, (long long)shape->H);
  if (shape->N > (int64_t)INT32_MAX || shape->H > 65535)
    return fail(DLA_E_UNSUPPORTED, "N must be < 2^31 and H <= 65535");
  if (shape->stride_b <= 0 || shape->stride_n <= 0 || shape->stride_h <= 0)
    return fail(DLA_E_INVALID, "strides must be positive");
  if (shape->stride_b % 8 || shape->stride_n % 8 || shape->stride_h % 8)
    return fail(DLA_E_INVALID, "strides must be multiples of 8 elements (16-byte rows)");

  p.B = shape->B;
  p.N = shape->N;
  p.H = shape->H;
  p.dtype = shape->dtype;
  p.esize = shape->dtype == DLA_F32 ? 4 : 2;
  p.sb = shape->stride_b;
  p.sn = shape->stride_n;
  p.sh = shape->stride_h;
  p.P = desc->num_patterns;
  p.causal = desc->causal;
  p.scale = desc->scale;
  p.empty = (p.B == 0 || p.H == 0);

  int64_t total = p.N, start = 0;
  if (shard) {
    total = shard->total_rows;
    start = shard->shard_start;
    if (total < p.N || total % p.N)
      return fail(DLA_E_INVALID, "total_rows=%lld is not a positive multiple of N=%lld",
                  (long long)total, (long long)p.N);
    if (start < 0 || start >= total || start % p.N)
      return fail(DLA_E_INVALID, "shard_start=%lld is not a multiple of N=%lld below total_rows",
                  (long long)start, (long long)p.N);
    if (p.dtype != DLA_BF16) return fail(DLA_E_UNSUPPORTED, "sequence shards are implemented for bf16");
  }
  p.shard = shard != nullptr;

  for (int i = 0; i < p.P; ++i) {
    const int w = desc->patterns[i].w, r = desc->patterns[i].r;
    if (w < 1 || r < 1) return fail(DLA_E_INVALID, "pattern %d: w=%d r=%d must be >= 1", i, w, r);
    if (w % r) return fail(DLA_E_UNSUPPORTED, "pattern %d: r=%d does not divide w=%d", i, r, w);
    // A whole sequence may end inside a segment (its last segment is cut
    // short); a sequence split over shards needs whole segments.
    if (shard && w > total)
      return fail(DLA_E_UNSUPPORTED, "pattern %d: w=%d exceeds the sequence of %lld rows", i, w,
                  (long long)total);
    if (shard && total % w)
      return fail(DLA_E_UNSUPPORTED, "pattern %d: w=%d does not divide the sequence of %lld rows",
                  i, w, (long long)total);
    const bool spans = shard && w > p.N;
    if (shard && !spans && p.N % w)
      return fail(DLA_E_UNSUPPORTED, "pattern %d: w=%d does not divide the shard length N=%lld", i,
                  w, (long long)p.N);
    if (spans && (w % p.N || p.N % r || (p.N / r) % 64))
      return fail(DLA_E_UNSUPPORTED,
                  "pattern %d: a segment (w=%d) spanning shards of N=%lld rows needs N | w, r | N "
                  "and 64 | N/r (r=%d)", i, w, (long long)p.N, r);
    // The backward streams 64 dilated rows per tile through one 32-bit
    // buffer offset range.
    if ((int64_t)64 * r * shape->stride_n * (shape->dtype == DLA_F32 ? 4 : 2) + 128 > INT32_MAX)
      return fail(DLA_E_UNSUPPORTED, "pattern %d: 64 dilated rows span more than 2 GiB", i);
    p.w[i] = w;
    p.r[i] = r;
    p.span[i] = spans;
    p.Lk[i] = w / r;
    p.L[i] = spans ? (int)(p.N / r) : w / r;
    p.qoff[i] = spans ? (int)((start % w) / r) : 0;
    p.nseg[i] = spans ? 1 : (p.N + w - 1) / w;
    p.nsp[i] = (p.N + r - 1) / r;
  }

  // The pattern that keeps the most rows (smallest r, first on ties) writes
  // o/lse directly; the others leave partial results for the merge pass.
  p.prim = 0;
  for (int i = 1; i < p.P; ++i)
    if (p.r[i] < p.r[p.prim]) p.prim = i;
  p.need_combine = !(p.P == 1 && p.r[0] == 1);

  size_t off = 0;
  for (int i = 0; i < p.P; ++i) {
    p.part_o_off[i] = p.part_lse_off[i] = (size_t)-1;
    if (i == p.prim) continue;
    const size_t rows = (size_t)p.B * p.H * p.nsp[i];
    p.part_o_off[i] = off;
    off = align_up(off + rows * kD * p.esize, 256);
    p.part_lse_off[i] = off;
    off = align_up(off + rows * sizeof(float), 256);
  }
  p.ws_fwd = off;

  p.span_mask = 0;
  int lk_max = 0;
  for (int i = 0; i < p.P; ++i)
    if (p.span[i]) {
      p.span_mask |= 1u << i;
      lk_max = std::max(lk_max, p.Lk[i]);
    }
  const size_t rows_all = (size_t)p.B * p.N * p.H;
  off = 0;
  p.ld_off = off;
  off = align_up(off + rows_all * 2 * sizeof(float), 256);
  p.need_finalize = p.P > 1 || p.span_mask != 0;
  for (int i = 0; i < p.P; ++i)
    for (int t = 0; t < 3; ++t) {
      p.part_g_off[i][t] = (size_t)-1;
      if (!p.need_finalize) continue;
      const size_t rows = (size_t)p.B * p.H * p.nsp[i];
      p.part_g_off[i][t] = off;
      off = align_up(off + rows * kD * sizeof(float), 256);
    }
  for (int t = 0; t < 7; ++t) p.seg_off[t] = (size_t)-1;
  if (p.span_mask) {
    const size_t seg_rows = (size_t)p.B * p.H * lk_max;
    const size_t bytes[7] = {seg_rows * kD * 2, seg_rows * kD * 2, seg_rows * 8, seg_rows * kD * 2,
                             seg_rows * kD * 2, seg_rows * kD * 4, seg_rows * kD * 4};
    for (int t = 0; t < 7; ++t) {
      p.seg_off[t] = off;
      off = align_up(off + bytes[t], 256);
    }
  }
  p.ws_bwd = off;

  // Useful (query, key) pairs; a count beyond int64 is refused.
  int64_t pairs = 0;
  bool ovf = false;
  for (int i = 0; i < p.P; ++i) {
    const int64_t L = p.L[i];
    int64_t per = 0, seg_pairs = 0;
    if (p.span[i]) {
      // local queries qoff .. qoff+L-1 of a segment with Lk keys
      if (p.causal) {
        int64_t head = 0;
        ovf |= __builtin_mul_overflow(L, (int64_t)p.qoff[i], &head);
        per = L * (L + 1) / 2;
        ovf |= __builtin_add_overflow(per, head, &per);
      } else {
        ovf |= __builtin_mul_overflow(L, (int64_t)p.Lk[i], &per);
      }
    } else {
      ovf |= __builtin_mul_overflow(L, p.causal ? L + 1 : L, &per);
      if (p.causal) per /= 2;
    }
    // per (batch, head): whole segments, then a cut-short last one whose
    // row count depends on the head offset
    const int64_t whole = p.span[i] ? 1 : p.N / p.w[i];
    ovf |= __builtin_mul_overflow(whole, per, &seg_pairs);
    ovf |= __builtin_mul_overflow(seg_pairs, p.H, &seg_pairs);
    const int64_t left = p.N - whole * p.w[i];
    if (!p.span[i] && left > 0)
      for (int64_t h = 0; h < p.H; ++h) {
        const int64_t off = h % p.r[i];
        const int64_t Ls = left > off ? (left - 1 - off) / p.r[i] + 1 : 0;
        ovf |= __builtin_add_overflow(seg_pairs, p.causal ? Ls * (Ls + 1) / 2 : Ls * Ls, &seg_pairs);
      }
    ovf |= __builtin_add_overflow(pairs, seg_pairs, &pairs);
  }
  ovf |= __builtin_mul_overflow(pairs, p.B, &pairs);
  if (ovf) return fail(DLA_E_UNSUPPORTED, "the number of attention pairs exceeds 2^63");
  p.pairs = pairs;
  if (log_enabled()) log_plan(p);
  return DLA_OK;
}

// Streamed bytes per group of the schedule: the rows that the units of a
// group re-stream (two tensors of L rows per segment-head) should stay in
// the 256 MB last-level cache while the group runs.  At 1M tokens this took
// the forward from 9.30 to 8.52 ms and at 2 x 32K tokens the backward from
// 1.85 to 1.79 ms; 96 MB measured the same and 48 MB slower.
constexpr double kGroupBytes = 192.0 * (1 << 20);

uint32_t class_step(const Plan& p) {
  int ones = 0;
  int64_t rmin = 0;
  for (int i = 0; i < p.P; ++i) {
    const int r = p.r[i];
    if (r & (r - 1)) return 1;                              // not a power of two
    if (r == 1) {
      if (++ones > 1 || ((p.span_mask >> i) & 1u)) return 1;
    } else if (rmin == 0 || r < rmin) {
      rmin = r;
    }
  }
  return ones == 1 && rmin > 0 ? (uint32_t)rmin : 1u;
}

void make_schedule(const Plan& p, int tile_rows, Schedule* s) {
  memset(s, 0, sizeof(*s));
  const double budget = kGroupBytes;
  double bytes = 0;
  for (int i = 0; i < p.P; ++i) bytes += (double)p.B * p.H * p.nseg[i] * p.L[i] * kD * p.esize * 2;
  int64_t groups = std::max<int64_t>(1, (int64_t)ceil(bytes / budget));
  int64_t most = 0;
  for (int i = 0; i < p.P; ++i) most = std::max<int64_t>(most, p.B * p.H * p.nseg[i]);
  groups = std::max<int64_t>(1, std::min<int64_t>(groups, most));
  s->groups = groups;
  int ntile[kMaxP];
  for (int i = 0; i < p.P; ++i) {
    ntile[i] = (p.L[i] + tile_rows - 1) / tile_rows;
    s->order[i] = i;
    s->count[i] = p.B * p.H * p.nseg[i];
    s->chunk[i] = (s->count[i] + groups - 1) / groups;
  }
  std::stable_sort(s->order, s->order + p.P,
                   [&](int a, int b) { return ntile[a] > ntile[b]; });
  s->cum[0] = 0;
  for (int i = 0; i < p.P; ++i) s->cum[i + 1] = s->cum[i] + s->chunk[s->order[i]];
  int64_t start = 0;
  int nb = 0;
  for (int i = 0; i < p.P; ++i) {
    const int hi = ntile[s->order[i]];
    const int lo = (i + 1 < p.P) ? ntile[s->order[i + 1]] : 0;
    if (hi == lo) continue;
    s->band_hi[nb] = hi;
    s->band_npat[nb] = i + 1;
    s->band_start[nb] = start;
    start += (int64_t)(hi - lo) * s->cum[i + 1];
    ++nb;
  }
  s->band_start[nb] = start;
  s->nband = nb;
  s->upg = start;
  s->total = start * groups;
  if (log_enabled())
    fprintf(stderr, "[dla] schedule: %d-row units, %lld units in %lld group(s) of %lld, %d band(s)\n",
            tile_rows, (long long)s->total, (long long)groups, (long long)s->upg, nb);
}

}  // namespace dla

extern "C" {

int dla_plan_check(const dla_desc* desc, const dla_shape* shape, size_t* ws_fwd_bytes,
                   size_t* ws_bwd_bytes) {
  dla::Plan p;
  const int rc = dla::make_plan(desc, shape, &p);
  if (rc != DLA_OK) return rc;
  if (ws_fwd_bytes) *ws_fwd_bytes = p.ws_fwd;
  if (ws_bwd_bytes) *ws_bwd_bytes = p.ws_bwd;
  return DLA_OK;
}

int dla_plan_check_shard(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                         size_t* ws_fwd_bytes, size_t* ws_bwd_bytes) {
  if (!shard) return dla::fail(DLA_E_INVALID, "null shard");
  dla::Plan p;
  const int rc = dla::make_plan(desc, shape, &p, shard);
  if (rc != DLA_OK) return rc;
  if (ws_fwd_bytes) *ws_fwd_bytes = p.ws_fwd;
  if (ws_bwd_bytes) *ws_bwd_bytes = p.ws_bwd;
  return DLA_OK;
}

int dla_pair_count_shard(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                         int64_t* pairs) {
  if (!shard) return dla::fail(DLA_E_INVALID, "null shard");
  dla::Plan p;
  const int rc = dla::make_plan(desc, shape, &p, shard);
  if (rc != DLA_OK) return rc;
  if (!pairs) return dla::fail(DLA_E_INVALID, "null output pointer");
  *pairs = p.pairs;
  return DLA_OK;
}

int dla_pair_count_varlen(const dla_desc* desc, const dla_shape* shape, const int32_t* lengths,
                          int64_t* pairs) {
  dla::Plan p;
  int rc = dla::make_plan(desc, shape, &p);
  if (rc != DLA_OK) return rc;
  if (!pairs) return dla::fail(DLA_E_INVALID, "null output pointer");
  if (!lengths && shape->B > 0) return dla::fail(DLA_E_INVALID, "null lengths");
  int64_t total = 0;
  for (int64_t b = 0; b < shape->B; ++b) {
    const int64_t n = lengths[b] < 0 ? 0 : (lengths[b] > shape->N ? shape->N : lengths[b]);
    if (n == 0) continue;
    dla_shape one = *shape;
    one.B = 1;
    one.N = n;
    if ((rc = dla::make_plan(desc, &one, &p)) != DLA_OK) return rc;
    if (__builtin_add_overflow(total, p.pairs, &total))
      return dla::fail(DLA_E_UNSUPPORTED, "the number of attention pairs exceeds 2^63");
  }
  *pairs = total;
  return DLA_OK;
}

int dla_pair_count(const dla_desc* desc, const dla_shape* shape, int64_t* pairs) {
  dla::Plan p;
  const int rc = dla::make_plan(desc, shape, &p);
  if (rc != DLA_OK) return rc;
  if (!pairs) return dla::fail(DLA_E_INVALID, "null output pointer");
  *pairs = p.pairs;
  return DLA_OK;
}

const char* dla_strerror(int code) {
  switch (code) {
    case DLA_OK: return "success";
    case DLA_E_INVALID: return "invalid argument";
    case DLA_E_UNSUPPORTED: return "unsupported configuration";
    case DLA_E_WORKSPACE: return "workspace too small";
    case DLA_E_HIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

const char* dla_last_error(void) { return dla::g_err; }

}  // extern "C"
