// C ABI entry points of libdla that enqueue GPU work (see include/dla.h).
// Every check runs on the host before the first launch; a failing call
// enqueues nothing.
#include <stdint.h>

#include <mutex>

#include "dla_kernels.h"

namespace dla {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int check_ptr(const void* p, const char* name) {
  if (!p) return fail(DLA_E_INVALID, "%s is null", name);
  if (!aligned16(p)) return fail(DLA_E_INVALID, "%s is not 16-byte aligned", name);
  return DLA_OK;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(DLA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

static void fill_fwd_args(const Plan& pl, AttnFwdArgs* a) {
  a->sb = pl.sb;
  a->sn = pl.sn;
  a->sh = pl.sh;
  a->B = pl.B;
  a->N = pl.N;
  a->H = pl.H;
  a->P = pl.P;
  a->prim = pl.prim;
  a->causal = pl.causal;
  a->scale = pl.scale;
  a->scale_log2 = pl.scale * 1.4426950408889634f;
  for (int i = 0; i < pl.P; ++i) {
    a->w[i] = pl.w[i];
    a->r[i] = pl.r[i];
    a->L[i] = pl.L[i];
    a->nseg[i] = pl.nseg[i];
    a->nsp[i] = pl.nsp[i];
    a->Lk[i] = pl.Lk[i];
    a->qoff[i] = pl.qoff[i];
  }
}

// Attention pass and merge for a validated plan (whole sequence or shard).
static int forward_impl(const Plan& pl, const void* q, const void* k, const void* v,
                        const void* const* ext_k, const void* const* ext_v, void* o, float* lse,
                        void* ws, size_t ws_bytes, void* stream, const int32_t* lengths = nullptr,
                        const float* k_scale = nullptr, const float* v_scale = nullptr) {
  int rc;
  if (pl.empty) return DLA_OK;  // nothing is read or written; pointers may be null
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse")))
    return rc;
  if (ws_bytes < pl.ws_fwd)
    return fail(DLA_E_WORKSPACE, "forward workspace needs %zu bytes, got %zu", pl.ws_fwd, ws_bytes);
  if (pl.ws_fwd && (rc = check_ptr(ws, "workspace"))) return rc;

  AttnFwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.lengths = lengths;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  fill_fwd_args(pl, &a);
  for (int i = 0; i < pl.P; ++i) {
    if (!pl.span[i]) continue;
    if (!ext_k || !ext_v) return fail(DLA_E_INVALID, "pattern %d spans shards: ext_k/ext_v are null", i);
    if ((rc = check_ptr(ext_k[i], "ext_k[pattern]")) || (rc = check_ptr(ext_v[i], "ext_v[pattern]")))
      return rc;
    a.ext_k[i] = ext_k[i];
    a.ext_v[i] = ext_v[i];
  }
  for (int i = 0; i < pl.P; ++i) {
    if (i == pl.prim) continue;
    a.part_o[i] = (char*)ws + pl.part_o_off[i];
    a.part_lse[i] = (float*)((char*)ws + pl.part_lse_off[i]);
  }
  make_schedule(pl, pl.dtype == DLA_BF16 ? 256 : 64, &a.sched);
  if (a.sched.total > 0x7FFFFFFF) return fail(DLA_E_UNSUPPORTED, "too many work units for one launch");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = pl.dtype == DLA_BF16 ? launch_attn_fwd_bf16(a, st) : launch_attn_fwd_f32(a, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (pl.need_combine || lengths) {
    CombineArgs cb{};
    cb.o = o;
    cb.lse = lse;
    cb.lengths = lengths;
    for (int i = 0; i < pl.P; ++i) {
      cb.part_o[i] = a.part_o[i];
      cb.part_lse[i] = a.part_lse[i];
      cb.r[i] = pl.r[i];
      cb.nsp[i] = pl.nsp[i];
    }
    cb.sb = pl.sb;
    cb.sn = pl.sn;
    cb.sh = pl.sh;
    cb.B = pl.B;
    cb.N = pl.N;
    cb.H = pl.H;
    cb.P = pl.P;
    cb.prim = pl.prim;
    for (int i = 0; i < pl.P; ++i) {
      const int r = pl.r[i];
      cb.shift[i] = (r & (r - 1)) ? -1 : __builtin_ctz((unsigned)r);
    }
    const int64_t nblk = (pl.N + 31) / 32;
    if (nblk * pl.B > 0x7FFFFFFF)
      return fail(DLA_E_UNSUPPORTED, "B * N / 32 exceeds the launch grid");
    cb.nblk = (uint32_t)nblk;
    // R = lcm of the rates; the residue-class launch needs R | N.
    int64_t R = 1;
    for (int i = 0; i < pl.P; ++i) {
      int64_t g = R, x = pl.r[i];
      while (x) { const int64_t t = g % x; g = x; x = t; }
      R = R / g * pl.r[i];
      if (R > pl.N) break;
    }
    const int64_t rpc = R <= pl.N ? pl.N / R : 0;
    cb.R = 0;
    cb.cls_step = 1;
    if (rpc >= 32 && R <= 65535 && pl.B * pl.H <= 65535 && R * (int64_t)rpc == pl.N) {
      cb.R = (uint32_t)R;
      cb.rows_per_class = (uint32_t)rpc;
      // Only the classes that another pattern than the primary keeps.
      if (pl.r[pl.prim] == 1) cb.cls_step = class_step(pl);
    }
    if (pl.need_combine) {
      e = launch_combine(cb, pl.dtype, st);
      if (e != hipSuccess) return hip_fail(e, "combine launch");
    }
    e = launch_pad_rows(cb, pl.dtype, st);  // rows past a batch's length
    if (e != hipSuccess) return hip_fail(e, "padding launch");
  }
  return DLA_OK;
}

}  // namespace dla

using namespace dla;

extern "C" int dla_forward(const dla_desc* desc, const dla_shape* shape, const void* q,
                           const void* k, const void* v, void* o, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
  clear_error();
  Plan pl;
  int rc = make_plan(desc, shape, &pl);
  if (rc) return rc;
  return forward_impl(pl, q, k, v, nullptr, nullptr, o, lse, ws, ws_bytes, stream);
}

// ---- The forward for callers that cannot allocate --------------------------
//
// A file-scope device array stands in for the caller's workspace.  Each GPU
// holds its own copy (at its own address) from the moment the library's code
// is loaded on it until the process ends.  Host code never passes the
// array's name to a kernel or a copy: in host code that name is only a
// stand-in; the device address comes from hipGetSymbolAddress, taken once
// per device with that device current and kept in `g_scratch_ptr`.
namespace dla {
constexpr size_t kScratchBytes = DLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace dla

static __device__ __align__(256) unsigned char scratch[dla::kScratchBytes];

namespace dla {
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DLA_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(DLA_E_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DLA_OK;
}
}  // namespace
}  // namespace dla

extern "C" int dla_forward_noalloc(const dla_desc* desc, const dla_shape* shape, const void* q,
                                   const void* k, const void* v, void* o, float* lse,
                                   void* stream) {
  clear_error();
  Plan pl;
  int rc = make_plan(desc, shape, &pl);
  if (rc) return rc;
  if (pl.ws_fwd > kScratchBytes)
    return fail(DLA_E_WORKSPACE,
                "dla_forward_noalloc: this problem needs %zu bytes of workspace, more than the %zu "
                "bytes of the library's static scratch; call dla_forward with a workspace",
                pl.ws_fwd, kScratchBytes);
  if (pl.empty) return DLA_OK;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  // The partial results are written before they are read (every row a
  // pattern keeps is written by its attention pass; the merge reads only
  // those rows), so nothing in the scratch needs clearing between calls.
  return forward_impl(pl, q, k, v, nullptr, nullptr, o, lse, ws, kScratchBytes, stream);
}

extern "C" int dla_forward_varlen(const dla_desc* desc, const dla_shape* shape,
                                  const int32_t* lengths, const void* q, const void* k,
                                  const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  clear_error();
  Plan pl;
  int rc = make_plan(desc, shape, &pl);
  if (rc) return rc;
  if (!pl.empty && (!lengths || ((uintptr_t)lengths & 3u)))
    return fail(DLA_E_INVALID, "lengths is null or not 4-byte aligned");
  return forward_impl(pl, q, k, v, nullptr, nullptr, o, lse, ws, ws_bytes, stream, lengths);
}

static int check_f32(const void* p, const char* name) {
  if (!p) return fail(DLA_E_INVALID, "%s is null", name);
  if ((uintptr_t)p & 3u) return fail(DLA_E_INVALID, "%s is not 4-byte aligned", name);
  return DLA_OK;
}

extern "C" int dla_forward_fp8kv(const dla_desc* desc, const dla_shape* shape, const void* q,
                                 const uint8_t* k8, const uint8_t* v8, const float* k_scale,
                                 const float* v_scale, void* o, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  clear_error();
  Plan pl;
  int rc = make_plan(desc, shape, &pl);
  if (rc) return rc;
  if (pl.dtype != DLA_BF16) return fail(DLA_E_UNSUPPORTED, "8-bit keys and values need bf16 q and o");
  if (pl.empty) return DLA_OK;
  if ((rc = check_f32(k_scale, "k_scale")) || (rc = check_f32(v_scale, "v_scale"))) return rc;
  return forward_impl(pl, q, k8, v8, nullptr, nullptr, o, lse, ws, ws_bytes, stream, nullptr, k_scale,
                      v_scale);
}

extern "C" int dla_quantize_fp8(const dla_shape* shape, const void* x, uint8_t* x8, float* scale,
                                void* stream) {
  clear_error();
  if (!shape) return fail(DLA_E_INVALID, "null shape");
  if (shape->dtype != DLA_BF16) return fail(DLA_E_UNSUPPORTED, "quantization reads bf16");
  if (shape->D != kD) return fail(DLA_E_UNSUPPORTED, "head dimension must be %d", kD);
  if (shape->B < 0 || shape->N < 0 || shape->H < 0) return fail(DLA_E_INVALID, "negative size");
  if (shape->stride_b <= 0 || shape->stride_n <= 0 || shape->stride_h <= 0)
    return fail(DLA_E_INVALID, "strides must be positive");
  if (shape->stride_b % 8 || shape->stride_n % 8 || shape->stride_h % 8)
    return fail(DLA_E_INVALID, "strides must be multiples of 8 elements");
  if (shape->B * shape->H > 65535) return fail(DLA_E_UNSUPPORTED, "B * H exceeds 65535");
  if (shape->B * shape->H == 0) return DLA_OK;
  int rc;
  if ((rc = check_f32(scale, "scale"))) return rc;
  if (shape->N > 0 && ((rc = check_ptr(x, "x")) || (rc = check_ptr(x8, "x8")))) return rc;
  QuantArgs a{};
  a.x = x;
  a.x8 = x8;
  a.scale = scale;
  a.sb = shape->stride_b;
  a.sn = shape->stride_n;
  a.sh = shape->stride_h;
  a.B = shape->B;
  a.N = shape->N;
  a.H = shape->H;
  hipError_t e = launch_quantize_fp8(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantization launch");
  return DLA_OK;
}

extern "C" int dla_forward_shard(const dla_desc* desc, const dla_shape* shape,
                                 const dla_shard* shard, const void* q, const void* k,
                                 const void* v, const void* const* ext_k,
                                 const void* const* ext_v, void* o, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  clear_error();
  if (!shard) return fail(DLA_E_INVALID, "null shard");
  Plan pl;
  int rc = make_plan(desc, shape, &pl, shard);
  if (rc) return rc;
  return forward_impl(pl, q, k, v, ext_k, ext_v, o, lse, ws, ws_bytes, stream);
}

extern "C" int dla_shard_gather(const dla_desc* desc, const dla_shape* shape,
                                const dla_shard* shard, int32_t pattern, const void* x, void* out,
                                void* stream) {
  clear_error();
  if (!shard) return fail(DLA_E_INVALID, "null shard");
  Plan pl;
  int rc = make_plan(desc, shape, &pl, shard);
  if (rc) return rc;
  if (pattern < 0 || pattern >= pl.P)
    return fail(DLA_E_INVALID, "pattern index %d outside 0..%d", pattern, pl.P - 1);
  if (!pl.span[pattern])
    return fail(DLA_E_INVALID, "pattern %d does not span shards (w <= N)", pattern);
  if (pl.empty) return DLA_OK;
  if ((rc = check_ptr(x, "x")) || (rc = check_ptr(out, "out"))) return rc;
  ShardGatherArgs a{};
  a.x = x;
  a.out = out;
  a.sb = pl.sb;
  a.sn = pl.sn;
  a.sh = pl.sh;
  a.B = pl.B;
  a.H = pl.H;
  a.r = pl.r[pattern];
  a.cr = pl.N / pl.r[pattern];
  a.out_rows = a.cr;
  a.out_row0 = 0;
  hipError_t e = launch_shard_gather(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "shard gather launch");
  return DLA_OK;
}

extern "C" int dla_row_map(const dla_desc* desc, int64_t N, int32_t H, int32_t pattern,
                           int32_t* out, void* stream) {
  clear_error();
  dla_shape sh{};
  sh.B = 1;
  sh.N = N;
  sh.H = H;
  sh.D = kD;
  sh.dtype = DLA_BF16;
  sh.stride_h = kD;
  sh.stride_n = (H > 0 ? H : 1) * kD;
  sh.stride_b = N * sh.stride_n;
  Plan pl;
  int rc = make_plan(desc, &sh, &pl);
  if (rc) return rc;
  if (pattern < 0 || pattern >= pl.P)
    return fail(DLA_E_INVALID, "pattern index %d outside 0..%d", pattern, pl.P - 1);
  if (!out) return fail(DLA_E_INVALID, "out is null");
  if ((uintptr_t)out & 3u) return fail(DLA_E_INVALID, "out is not 4-byte aligned");
  if (H == 0) return DLA_OK;
  RowMapArgs a{};
  a.out = out;
  a.N = N;
  a.H = H;
  a.w = pl.w[pattern];
  a.r = pl.r[pattern];
  a.L = pl.L[pattern];
  hipError_t e = launch_row_map(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "row map launch");
  return DLA_OK;
}
