// C ABI entry points of the backward pass (see include/dla.h).
//
// Launch sequence on the caller's stream: one preprocessing pass (D =
// rowsum(dO*O) next to the combined LSE; zero gradients for rows no pattern
// keeps), one attention pass over all patterns (rows kept by one pattern are
// written directly; rows kept by several leave fp32 partials), and, with
// several patterns, a finalize pass that sums the partials.  Every gradient
// is rounded exactly once.
//
// A sequence shard adds, per pattern whose segments span devices, one pass
// over that segment: the shard's query rows (a window of the segment)
// against the gathered keys, written as fp32 partials, the dK/dV of the
// whole segment going out in the exchange layout.  The rows those patterns
// keep get dK/dV from dla_shard_finish, after the caller's exchange.
#include <stdint.h>

#include "dla_kernels.h"

using namespace dla;

static int check_ptr(const void* p, const char* name) {
  if (!p) return fail(DLA_E_INVALID, "%s is null", name);
  if ((uintptr_t)p & 15u) return fail(DLA_E_INVALID, "%s is not 16-byte aligned", name);
  return DLA_OK;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(DLA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// lcm of the rates when the residue-class launch fits (R divides N and rows
// per class >= 32), else 0 (the per-row launch).
static void residue_classes(const Plan& pl, uint32_t* R_out, uint32_t* rpc_out) {
  int64_t R = 1;
  for (int i = 0; i < pl.P; ++i) {
    int64_t g = R, x = pl.r[i];
    while (x) { const int64_t t = g % x; g = x; x = t; }
    R = R / g * pl.r[i];
    if (R > pl.N) break;
  }
  const int64_t rpc = R <= pl.N ? pl.N / R : 0;
  *R_out = 0;
  *rpc_out = 0;
  if (rpc >= 32 && R <= 65535 && pl.B * pl.H <= 65535 && R * rpc == pl.N) {
    *R_out = (uint32_t)R;
    *rpc_out = (uint32_t)rpc;
  }
}

static hipError_t run_prep(const Plan& pl, const void* o, const float* lse, const void* dout,
                           float2* ld, void* dq, void* dk, void* dv, hipStream_t st,
                           const int32_t* lengths = nullptr) {
  BwdPrepArgs pa{};
  pa.lengths = lengths;
  pa.o = o;
  pa.dout = dout;
  pa.lse = lse;
  pa.ld = ld;
  pa.dq = dq;
  pa.dk = dk;
  pa.dv = dv;
  pa.sb = pl.sb;
  pa.sn = pl.sn;
  pa.sh = pl.sh;
  pa.B = pl.B;
  pa.N = pl.N;
  pa.H = pl.H;
  pa.P = pl.P;
  for (int i = 0; i < pl.P; ++i) pa.r_all[i] = pl.r[i];
  pa.zero_uncovered = pl.r[pl.prim] != 1;
  return launch_bwd_prep(pa, pl.dtype, st);
}

// The attention pass of the patterns that do not span shards (all of them
// for a whole sequence).  Every pattern's rate enters the epilogue's count
// of the patterns keeping a row.
static int run_attention(const Plan& pl, const void* q, const void* k, const void* v,
                         const void* dout, const float2* ld, char* wsb, void* dq, void* dk,
                         void* dv, hipStream_t st, const int32_t* lengths = nullptr) {
  AttnBwdArgs a{};
  a.lengths = lengths;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.ld = ld;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.sb = pl.sb;
  a.sn = pl.sn;
  a.sh = pl.sh;
  a.B = pl.B;
  a.N = pl.N;
  a.H = pl.H;
  a.causal = pl.causal;
  a.scale = pl.scale;
  a.scale_log2 = pl.scale * 1.4426950408889634f;
  a.P = pl.P;
  Plan local = pl;  // the schedules skip spanning patterns (their segments run separately)
  for (int i = 0; i < pl.P; ++i) {
    a.w[i] = pl.w[i];
    a.r[i] = pl.r[i];
    a.L[i] = pl.L[i];
    a.nseg[i] = pl.nseg[i];
    a.nsp[i] = pl.nsp[i];
    for (int g = 0; g < 3; ++g)
      a.part[i][g] = pl.need_finalize ? (float*)(wsb + pl.part_g_off[i][g]) : nullptr;
    if (pl.span[i]) local.nseg[i] = 0;
  }
  make_schedule(local, kBwdUnitRows, &a.sched_kv);
  make_schedule(local, kBwdUnitRows, &a.sched_q);
  if (a.sched_kv.total + a.sched_q.total > 0x7FFFFFFF)
    return fail(DLA_E_UNSUPPORTED, "too many work units for one launch");
  hipError_t e = launch_attn_bwd_bf16(a, st);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return DLA_OK;
}

static int run_finalize(const Plan& pl, char* wsb, void* dq, void* dk, void* dv, hipStream_t st,
                        const int32_t* lengths = nullptr) {
  BwdFinalizeArgs f{};
  f.lengths = lengths;
  for (int i = 0; i < pl.P; ++i) {
    for (int g = 0; g < 3; ++g) f.part[i][g] = (const float*)(wsb + pl.part_g_off[i][g]);
    f.r[i] = pl.r[i];
    f.nsp[i] = pl.nsp[i];
    f.shift[i] = (pl.r[i] & (pl.r[i] - 1)) == 0 ? __builtin_ctz((unsigned)pl.r[i]) : -1;
  }
  f.grad[0] = dq;
  f.grad[1] = dk;
  f.grad[2] = dv;
  f.sb = pl.sb;
  f.sn = pl.sn;
  f.sh = pl.sh;
  f.B = pl.B;
  f.N = pl.N;
  f.H = pl.H;
  f.P = pl.P;
  f.nblk = (uint32_t)((pl.N + 31) / 32);
  f.span_mask = pl.span_mask;
  residue_classes(pl, &f.R, &f.rows_per_class);
  f.cls_step = f.R ? class_step(pl) : 1u;  // classes kept by two or more patterns
  hipError_t e = launch_bwd_finalize(f, st);
  if (e != hipSuccess) return hip_fail(e, "backward finalize launch");
  return DLA_OK;
}

static int backward_impl(const Plan& pl, const int32_t* lengths, const void* q, const void* k,
                         const void* v, const void* o, const float* lse, const void* dout,
                         void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (pl.empty) return DLA_OK;  // nothing is read or written; pointers may be null
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")))
    return rc;
  if (ws_bytes < pl.ws_bwd)
    return fail(DLA_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu", pl.ws_bwd, ws_bytes);
  if ((rc = check_ptr(ws, "workspace"))) return rc;
  if (pl.dtype != DLA_BF16)
    return fail(DLA_E_UNSUPPORTED, "the backward pass is implemented for bf16 tensors");
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float2* ld = (float2*)(wsb + pl.ld_off);
  hipError_t e = run_prep(pl, o, lse, dout, ld, dq, dk, dv, st, lengths);
  if (e != hipSuccess) return hip_fail(e, "backward preprocessing launch");
  if ((rc = run_attention(pl, q, k, v, dout, ld, wsb, dq, dk, dv, st, lengths))) return rc;
  if (pl.need_finalize && (rc = run_finalize(pl, wsb, dq, dk, dv, st, lengths))) return rc;
  return DLA_OK;
}

extern "C" int dla_backward(const dla_desc* desc, const dla_shape* shape, const void* q,
                            const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* stream) {
  clear_error();
  Plan pl;
  int rc = make_plan(desc, shape, &pl);
  if (rc) return rc;
  return backward_impl(pl, nullptr, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream);
}

extern "C" int dla_backward_varlen(const dla_desc* desc, const dla_shape* shape,
                                   const int32_t* lengths, const void* q, const void* k,
                                   const void* v, const void* o, const float* lse,
                                   const void* dout, void* dq, void* dk, void* dv, void* ws,
                                   size_t ws_bytes, void* stream) {
  clear_error();
  Plan pl;
  int rc = make_plan(desc, shape, &pl);
  if (rc) return rc;
  if (!pl.empty && (!lengths || ((uintptr_t)lengths & 3u)))
    return fail(DLA_E_INVALID, "lengths is null or not 4-byte aligned");
  return backward_impl(pl, lengths, q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, stream);
}

// One spanning pattern p of a shard: its segment contiguous per (batch,
// head) in the workspace, the shard's queries as the window [qoff, qoff+cr).
static int run_spanning(const Plan& pl, int p, const void* q, const void* dout, const float2* ld,
                        const void* ext_k, const void* ext_v, void* ext_dk, void* ext_dv, char* wsb,
                        void* dq, void* dk, void* dv, hipStream_t st) {
  const int64_t Lk = pl.Lk[p], cr = pl.N / pl.r[p], C = Lk / cr, qoff = pl.qoff[p];
  void* seg[7];
  for (int t = 0; t < 7; ++t) seg[t] = wsb + pl.seg_off[t];
  hipError_t e;
  // The shard's rows of the segment: q and dO at rows qoff.., (LSE2, D) too.
  ShardGatherArgs g{};
  g.sb = pl.sb;
  g.sn = pl.sn;
  g.sh = pl.sh;
  g.B = pl.B;
  g.H = pl.H;
  g.r = pl.r[p];
  g.cr = cr;
  g.out_rows = Lk;
  g.out_row0 = qoff;
  g.x = q;
  g.out = seg[0];
  if ((e = launch_shard_gather(g, st)) != hipSuccess) return hip_fail(e, "shard gather launch");
  g.x = dout;
  g.out = seg[1];
  if ((e = launch_shard_gather(g, st)) != hipSuccess) return hip_fail(e, "shard gather launch");
  ShardLdArgs l{};
  l.ld = ld;
  l.out = (float2*)seg[2];
  l.B = pl.B;
  l.H = pl.H;
  l.N = pl.N;
  l.r = pl.r[p];
  l.cr = cr;
  l.out_rows = Lk;
  l.out_row0 = qoff;
  if ((e = launch_shard_ld(l, st)) != hipSuccess) return hip_fail(e, "shard gather launch");
  // The gathered keys and values, contiguous per (batch, head).
  ShardRelayoutArgs rl{};
  rl.C = C;
  rl.B = pl.B;
  rl.H = pl.H;
  rl.cr = cr;
  rl.pieces = 8;
  rl.to_ext = 0;
  rl.src = ext_k;
  rl.dst = seg[3];
  if ((e = launch_shard_relayout(rl, st)) != hipSuccess) return hip_fail(e, "shard relayout launch");
  rl.src = ext_v;
  rl.dst = seg[4];
  if ((e = launch_shard_relayout(rl, st)) != hipSuccess) return hip_fail(e, "shard relayout launch");

  // The segment as one single-pattern problem (w = Lk, r = 1, [B, H, Lk, D]).
  AttnBwdArgs a{};
  a.q = seg[0];
  a.dout = seg[1];
  a.ld = (const float2*)seg[2];
  a.k = seg[3];
  a.v = seg[4];
  a.dq = dq;  // not written: every result of a window is a partial
  a.dk = dk;
  a.dv = dv;
  a.sn = kD;
  a.sh = Lk * kD;
  a.sb = pl.H * Lk * kD;
  a.B = pl.B;
  a.N = Lk;
  a.H = pl.H;
  a.causal = pl.causal;
  a.scale = pl.scale;
  a.scale_log2 = pl.scale * 1.4426950408889634f;
  a.P = 1;
  a.w[0] = (int)Lk;
  a.r[0] = 1;
  a.L[0] = (int)Lk;
  a.nseg[0] = 1;
  a.nsp[0] = Lk;
  // dQ rows qoff.. land in pattern p's partial rows 0.. ([B,H,cr,D]).
  a.part[0][0] = (float*)(wsb + pl.part_g_off[p][0]) - qoff * kD;
  a.part[0][1] = (float*)seg[5];
  a.part[0][2] = (float*)seg[6];
  a.qlo = (int)qoff;
  a.qhi = (int)(qoff + cr);
  a.nsp_q = cr;
  Plan sp{};
  sp.B = pl.B;
  sp.H = pl.H;
  sp.P = 1;
  sp.nseg[0] = 1;
  sp.L[0] = (int)Lk;
  make_schedule(sp, kBwdUnitRows, &a.sched_kv);
  sp.L[0] = (int)cr;
  make_schedule(sp, kBwdUnitRows, &a.sched_q);
  if ((e = launch_attn_bwd_bf16(a, st)) != hipSuccess) return hip_fail(e, "backward launch");

  // This shard's dK, dV contributions to the whole segment, exchange layout.
  rl.pieces = 16;
  rl.to_ext = 1;
  rl.src = seg[5];
  rl.dst = ext_dk;
  if ((e = launch_shard_relayout(rl, st)) != hipSuccess) return hip_fail(e, "shard relayout launch");
  rl.src = seg[6];
  rl.dst = ext_dv;
  if ((e = launch_shard_relayout(rl, st)) != hipSuccess) return hip_fail(e, "shard relayout launch");
  return DLA_OK;
}

static int check_span_bwd(const Plan& pl) {
  for (int i = 0; i < pl.P; ++i)
    if (pl.span[i] && (pl.N / pl.r[i]) % kBwdUnitRows)
      return fail(DLA_E_UNSUPPORTED,
                  "pattern %d spans shards: the backward needs N / r to be a multiple of %d", i,
                  kBwdUnitRows);
  return DLA_OK;
}

extern "C" int dla_backward_shard(const dla_desc* desc, const dla_shape* shape,
                                  const dla_shard* shard, const void* q, const void* k,
                                  const void* v, const void* o, const float* lse,
                                  const void* dout, const void* const* ext_k,
                                  const void* const* ext_v, void* dq, void* dk, void* dv,
                                  void* const* ext_dk, void* const* ext_dv, void* ws,
                                  size_t ws_bytes, void* stream) {
  clear_error();
  if (!shard) return fail(DLA_E_INVALID, "null shard");
  Plan pl;
  int rc = make_plan(desc, shape, &pl, shard);
  if (rc) return rc;
  if ((rc = check_span_bwd(pl))) return rc;
  if (pl.empty) return DLA_OK;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv")))
    return rc;
  if (pl.span_mask) {
    if (!ext_k || !ext_v || !ext_dk || !ext_dv)
      return fail(DLA_E_INVALID, "patterns span shards: ext_k, ext_v, ext_dk and ext_dv are needed");
    for (int i = 0; i < pl.P; ++i)
      if (pl.span[i] &&
          ((rc = check_ptr(ext_k[i], "ext_k[pattern]")) || (rc = check_ptr(ext_v[i], "ext_v[pattern]")) ||
           (rc = check_ptr(ext_dk[i], "ext_dk[pattern]")) || (rc = check_ptr(ext_dv[i], "ext_dv[pattern]"))))
        return rc;
  }
  if (ws_bytes < pl.ws_bwd)
    return fail(DLA_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu", pl.ws_bwd, ws_bytes);
  if ((rc = check_ptr(ws, "workspace"))) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float2* ld = (float2*)(wsb + pl.ld_off);
  hipError_t e = run_prep(pl, o, lse, dout, ld, dq, dk, dv, st);
  if (e != hipSuccess) return hip_fail(e, "backward preprocessing launch");
  if ((rc = run_attention(pl, q, k, v, dout, ld, wsb, dq, dk, dv, st))) return rc;
  for (int i = 0; i < pl.P; ++i)
    if (pl.span[i] &&
        (rc = run_spanning(pl, i, q, dout, ld, ext_k[i], ext_v[i], ext_dk[i], ext_dv[i], wsb, dq, dk, dv, st)))
      return rc;
  if (pl.need_finalize && (rc = run_finalize(pl, wsb, dq, dk, dv, st))) return rc;
  return DLA_OK;
}

extern "C" int dla_shard_finish(const dla_desc* desc, const dla_shape* shape,
                                const dla_shard* shard, const float* const* red_dk,
                                const float* const* red_dv, void* dk, void* dv, void* ws,
                                size_t ws_bytes, void* stream) {
  clear_error();
  if (!shard) return fail(DLA_E_INVALID, "null shard");
  Plan pl;
  int rc = make_plan(desc, shape, &pl, shard);
  if (rc) return rc;
  if ((rc = check_span_bwd(pl))) return rc;
  if (pl.empty || !pl.span_mask) return DLA_OK;
  if ((rc = check_ptr(dk, "dk")) || (rc = check_ptr(dv, "dv"))) return rc;
  if (!red_dk || !red_dv) return fail(DLA_E_INVALID, "red_dk and red_dv are needed");
  for (int i = 0; i < pl.P; ++i)
    if (pl.span[i] &&
        ((rc = check_ptr(red_dk[i], "red_dk[pattern]")) || (rc = check_ptr(red_dv[i], "red_dv[pattern]"))))
      return rc;
  if (ws_bytes < pl.ws_bwd)
    return fail(DLA_E_WORKSPACE, "backward workspace needs %zu bytes, got %zu", pl.ws_bwd, ws_bytes);
  if ((rc = check_ptr(ws, "workspace"))) return rc;
  char* wsb = (char*)ws;
  ShardFinishArgs f{};
  for (int i = 0; i < pl.P; ++i) {
    for (int g = 0; g < 3; ++g) f.part[i][g] = (const float*)(wsb + pl.part_g_off[i][g]);
    if (pl.span[i]) {
      f.red_k[i] = red_dk[i];
      f.red_v[i] = red_dv[i];
    }
    f.r[i] = pl.r[i];
    f.nsp[i] = pl.nsp[i];
  }
  f.dk = dk;
  f.dv = dv;
  f.sb = pl.sb;
  f.sn = pl.sn;
  f.sh = pl.sh;
  f.B = pl.B;
  f.N = pl.N;
  f.H = pl.H;
  f.P = pl.P;
  f.span_mask = pl.span_mask;
  f.nblk = (uint32_t)((pl.N + 31) / 32);
  hipError_t e = launch_shard_finish(f, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "shard finish launch");
  return DLA_OK;
}
