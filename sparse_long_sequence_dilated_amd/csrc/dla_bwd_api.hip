// C ABI entry point of the backward pass (see include/dla.h).
//
// Launch sequence on the caller's stream: one preprocessing pass (D =
// rowsum(dO*O) next to the combined LSE; zero gradients for rows no pattern
// keeps), one attention pass over all patterns (rows kept by one pattern are
// written directly; rows kept by several leave fp32 partials), and, with
// several patterns, a finalize pass that sums the partials.  Every gradient
// is rounded exactly once.
#include <stdint.h>

#include "dla_kernels.h"

using namespace dla;

static int check_ptr(const void* p, const char* name) {
  if (!p) return fail(DLA_E_INVALID, "%s is null", name);
  if ((uintptr_t)p & 15u) return fail(DLA_E_INVALID, "%s is not 16-byte aligned", name);
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

  BwdPrepArgs pa{};
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
  hipError_t e = launch_bwd_prep(pa, pl.dtype, st);
  if (e != hipSuccess) return fail(DLA_E_HIP, "backward preprocessing launch: %s", hipGetErrorString(e));

  AttnBwdArgs a{};
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
  for (int i = 0; i < pl.P; ++i) {
    a.w[i] = pl.w[i];
    a.r[i] = pl.r[i];
    a.L[i] = pl.L[i];
    a.nseg[i] = pl.nseg[i];
    a.nsp[i] = pl.N / pl.r[i];
    for (int g = 0; g < 3; ++g)
      a.part[i][g] = pl.need_finalize ? (float*)(wsb + pl.part_g_off[i][g]) : nullptr;
  }
  make_schedule(pl, kBwdUnitRows, &a.sched_kv);
  make_schedule(pl, kBwdUnitRows, &a.sched_q);
  if (a.sched_kv.total + a.sched_q.total > 0x7FFFFFFF)
    return fail(DLA_E_UNSUPPORTED, "too many work units for one launch");
  e = launch_attn_bwd_bf16(a, st);
  if (e != hipSuccess) return fail(DLA_E_HIP, "backward launch: %s", hipGetErrorString(e));

  if (pl.need_finalize) {
    BwdFinalizeArgs f{};
    for (int i = 0; i < pl.P; ++i) {
      for (int g = 0; g < 3; ++g) f.part[i][g] = a.part[i][g];
      f.r[i] = pl.r[i];
      f.nsp[i] = pl.N / pl.r[i];
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
    // R = lcm of the rates divides N (every r divides its w, which divides N).
    int64_t R = 1;
    for (int i = 0; i < pl.P; ++i) {
      int64_t g = R, x = pl.r[i];
      while (x) { const int64_t t = g % x; g = x; x = t; }
      R = R / g * pl.r[i];
      if (R > pl.N) break;
    }
    const int64_t rpc = R <= pl.N ? pl.N / R : 0;
    f.R = 0;
    if (rpc >= 32 && R <= 65535 && pl.B * pl.H <= 65535 && R * rpc == pl.N) {
      f.R = (uint32_t)R;
      f.rows_per_class = (uint32_t)rpc;
    }
    e = launch_bwd_finalize(f, st);
    if (e != hipSuccess) return fail(DLA_E_HIP, "backward finalize launch: %s", hipGetErrorString(e));
  }
  return DLA_OK;
}
