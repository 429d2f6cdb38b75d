// A LongNet attention layer around the operator: Q = X W_q, K = X W_k,
// V = X W_v (W_qkv = [W_q | W_k | W_v]), dilated attention A = DA(Q, K, V),
// and Y = A W_o, with random weights at the pages' model settings (the
// gptget.net LongNet summary, section 实验设计: 768-dimensional model, 12
// heads).  The projections are plain GEMMs and go to hipBLASLt; the attention
// runs through dla_forward / dla_backward.  q, k, v (and their gradients)
// live in one [3, B, N, H, D] buffer, each contiguous like the attention
// output, so that all eight attention tensors share one layout.
//
// Row-major C[M, N] = op(A)[M, K] op(B)[K, N] is the column-major product
// C^T = op(B)^T op(A)^T, which is how the calls below are issued.
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <tuple>

#include "dla_device.h"

using namespace dla;

namespace {

int check(const void* p, const char* name) {
  if (!p) return fail(DLA_E_INVALID, "%s is null", name);
  if ((uintptr_t)p & 15u) return fail(DLA_E_INVALID, "%s is not 16-byte aligned", name);
  return DLA_OK;
}

#define DLA_BLAS(call)                                                                  \
  do {                                                                                  \
    const hipblasStatus_t s_ = (call);                                                  \
    if (s_ != HIPBLAS_STATUS_SUCCESS) {                                                 \
      rc = fail(DLA_E_HIP, "hipBLASLt %s failed with status %d", #call, (int)s_);        \
      goto done;                                                                        \
    }                                                                                   \
  } while (0)

// A strided batch of products: `count` problems, operand i at A + i sa,
// B + i sb, C + i sc (strides in elements).
struct Batch {
  int count = 1;
  int64_t sa = 0, sb = 0, sc = 0;
};

// The handle behind dla_blas_create: hipBLASLt's handle plus, per product
// shape, the matmul and layout descriptors and the algorithm its heuristic
// chose, made on the first call with that shape and reused afterwards.
struct GemmKey {
  bool ta, tb;
  int64_t M, N, K, lda, ldb, ldc;
  int ctype;
  int count;
  int64_t sa, sb, sc;
  uint64_t ws;
  bool operator<(const GemmKey& o) const {
    return std::tie(ta, tb, M, N, K, lda, ldb, ldc, ctype, count, sa, sb, sc, ws) <
           std::tie(o.ta, o.tb, o.M, o.N, o.K, o.lda, o.ldb, o.ldc, o.ctype, o.count, o.sa, o.sb, o.sc, o.ws);
  }
};
struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};
void destroy_plan(GemmPlan& g) {
  if (g.lc) hipblasLtMatrixLayoutDestroy(g.lc);
  if (g.lb) hipblasLtMatrixLayoutDestroy(g.lb);
  if (g.la) hipblasLtMatrixLayoutDestroy(g.la);
  if (g.desc) hipblasLtMatmulDescDestroy(g.desc);
  g = GemmPlan{};
}
struct Blas {
  hipblasLtHandle_t h = nullptr;
  std::mutex mu;                      // guards `plans` (calls may come from several threads)
  std::map<GemmKey, GemmPlan> plans;
};

// Descriptors and algorithm of one product shape; DLA_OK or an error code.
// Row-major C[M, N] is issued as the column-major C^T = op(B)^T op(A)^T.
int make_gemm_plan(hipblasLtHandle_t h, const GemmKey& k, GemmPlan* out) {
  int rc = DLA_OK;
  GemmPlan g;
  hipblasLtMatmulPreference_t pref = nullptr;
  hipblasLtMatmulHeuristicResult_t heur{};
  int found = 0;
  const hipblasOperation_t op1 = k.tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipblasOperation_t op2 = k.ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const hipDataType ctype = (hipDataType)k.ctype;
  const uint64_t wsb = k.ws;
  DLA_BLAS(hipblasLtMatmulDescCreate(&g.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  DLA_BLAS(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op1, sizeof(op1)));
  DLA_BLAS(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op2, sizeof(op2)));
  DLA_BLAS(hipblasLtMatrixLayoutCreate(&g.la, HIP_R_16BF, k.tb ? k.K : k.N, k.tb ? k.N : k.K, k.ldb));
  DLA_BLAS(hipblasLtMatrixLayoutCreate(&g.lb, HIP_R_16BF, k.ta ? k.M : k.K, k.ta ? k.K : k.M, k.lda));
  DLA_BLAS(hipblasLtMatrixLayoutCreate(&g.lc, ctype, k.N, k.M, k.ldc));
  if (k.count > 1) {
    const hipblasLtMatrixLayout_t lay[3] = {g.la, g.lb, g.lc};
    const int64_t stride[3] = {k.sb, k.sa, k.sc};
    for (int i = 0; i < 3; ++i) {
      DLA_BLAS(hipblasLtMatrixLayoutSetAttribute(lay[i], HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &k.count,
                                                 sizeof(k.count)));
      DLA_BLAS(hipblasLtMatrixLayoutSetAttribute(lay[i], HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET,
                                                 &stride[i], sizeof(stride[i])));
    }
  }
  DLA_BLAS(hipblasLtMatmulPreferenceCreate(&pref));
  DLA_BLAS(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                 &wsb, sizeof(wsb)));
  DLA_BLAS(hipblasLtMatmulAlgoGetHeuristic(h, g.desc, g.la, g.lb, g.lc, g.lc, pref, 1, &heur, &found));
  if (found < 1) {
    rc = fail(DLA_E_UNSUPPORTED, "hipBLASLt has no algorithm for a %lldx%lldx%lld product",
              (long long)k.M, (long long)k.N, (long long)k.K);
    goto done;
  }
  g.algo = heur.algo;
done:
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (rc == DLA_OK) *out = g;
  else destroy_plan(g);
  return rc;
}

// Row-major C = op(A) op(B) + beta C, A and B bf16, C bf16 or fp32, fp32
// accumulation.  A is [M, K] (or [K, M] with ta), B is [K, N] (or [N, K]),
// C is [M, N]; lda, ldb, ldc are their row-major leading dimensions.
int gemm_rm(Blas* bl, hipStream_t st, void* ws, size_t ws_bytes, bool ta, bool tb,
            int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
            int64_t ldb, void* C, int64_t ldc, hipDataType ctype, float beta,
            const Batch& bt = Batch{}) {
  int rc = DLA_OK;
  const GemmKey key{ta, tb, M, N, K, lda, ldb, ldc, (int)ctype, bt.count,
                    bt.count > 1 ? bt.sa : 0, bt.count > 1 ? bt.sb : 0, bt.count > 1 ? bt.sc : 0,
                    (uint64_t)ws_bytes};
  GemmPlan g;
  {
    std::lock_guard<std::mutex> lk(bl->mu);
    auto it = bl->plans.find(key);
    if (it == bl->plans.end()) {
      if ((rc = make_gemm_plan(bl->h, key, &g))) return rc;
      bl->plans.emplace(key, g);
    } else {
      g = it->second;
    }
  }
  const float alpha = 1.f;
  // column-major operands: first = B (as op(B)^T), second = A (as op(A)^T)
  DLA_BLAS(hipblasLtMatmul(bl->h, g.desc, &alpha, B, g.la, A, g.lb, &beta, C, g.lc, C, g.lc, &g.algo, ws,
                           ws_bytes, st));
done:
  return rc;
}
#undef DLA_BLAS

constexpr size_t kGemmWs = (size_t)32 << 20;  // hipBLASLt workspace in the caller's buffer

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* src, __bf16* dst, int64_t n) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (int64_t)gridDim.x * 256 * 8) {
    const float4 a = *(const float4*)(src + i), b = *(const float4*)(src + i + 4);
    *(uint4*)(dst + i) = uint4{pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w)};
  }
}

// n a multiple of 8 (M * E with E = 64 H)
hipError_t launch_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n / 8 + 255) / 256, 65536);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, (__bf16*)dst, n);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Weight gradients W^T-shaped [E, E] = X^T dP reduce over all M = B N rows.
// One product of that shape has only (E / tile)^2 output tiles, too few to
// fill the chip, so the rows are cut into `splits` chunks: a strided batch of
// products writes one fp32 partial per chunk, and one pass sums them.
int weight_splits(int64_t M) {
  int s = 1;
  while (s < 16 && M % (2 * s) == 0 && M / (2 * s) >= 2048) s *= 2;
  return s;
}

// out[j] (row stride ldo[j]) = sum over s of part[j][s], for j < 4 gradients of [E, E].
struct SplitSumArgs {
  const float* part;  // [4, splits, E, E]
  float* out[4];
  int64_t ldo[4];
  int splits;
  int E;
};

__global__ __launch_bounds__(256) void split_sum_kernel(SplitSumArgs a) {
  const int j = blockIdx.y;
  const int64_t ee = (int64_t)a.E * a.E;
  const float* base = a.part + (int64_t)j * a.splits * ee;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < ee; i += (int64_t)gridDim.x * 256 * 4) {
    float4 acc = *(const float4*)(base + i);
    for (int s = 1; s < a.splits; ++s) {
      const float4 t = *(const float4*)(base + s * ee + i);
      acc.x += t.x;
      acc.y += t.y;
      acc.z += t.z;
      acc.w += t.w;
    }
    const int64_t row = i / a.E, col = i % a.E;  // E % 4 == 0: a float4 stays in one row
    *(float4*)(a.out[j] + row * a.ldo[j] + col) = acc;
  }
}

// q, k, v, the attention output and the gradients: contiguous [B, N, H, D].
dla_shape head_shape(int64_t B, int64_t N, int64_t H) {
  dla_shape s{};
  s.B = B;
  s.N = N;
  s.H = H;
  s.D = kD;
  s.dtype = DLA_BF16;
  s.stride_h = kD;
  s.stride_n = H * kD;
  s.stride_b = N * H * kD;
  return s;
}

// Layer workspace: forward = attention workspace + GEMM workspace; backward
// = dA [M, E] bf16 + dQKV [3, M, E] bf16 + dX [M, E] fp32 + weight-gradient
// partials [4, splits, E, E] fp32 + attention backward workspace + GEMM
// workspace.
int layer_plan(const dla_desc* desc, int64_t B, int64_t N, int64_t H, size_t* fwd, size_t* bwd) {
  if (B < 1 || N < 1 || H < 1) return fail(DLA_E_INVALID, "B, N and H must be positive");
  dla_shape s = head_shape(B, N, H);
  size_t af = 0, ab = 0;
  const int rc = dla_plan_check(desc, &s, &af, &ab);
  if (rc) return rc;
  const size_t M = (size_t)B * N, E = (size_t)H * kD;
  if (fwd) *fwd = align256(af) + kGemmWs;
  const size_t parts = (size_t)4 * weight_splits((int64_t)M) * E * E * 4;
  if (bwd)
    *bwd = align256(M * E * 2) + align256(M * 3 * E * 2) + align256(M * E * 4) + align256(parts) + align256(ab) +
           kGemmWs;
  return DLA_OK;
}

}  // namespace

extern "C" int dla_blas_create(void** handle) {
  clear_error();
  if (!handle) return fail(DLA_E_INVALID, "null handle pointer");
  hipblasLtHandle_t h = nullptr;
  const hipblasStatus_t s = hipblasLtCreate(&h);
  if (s != HIPBLAS_STATUS_SUCCESS) return fail(DLA_E_HIP, "hipblasLtCreate failed with status %d", (int)s);
  Blas* bl = new (std::nothrow) Blas;
  if (!bl) {
    hipblasLtDestroy(h);
    return fail(DLA_E_HIP, "out of host memory");
  }
  bl->h = h;
  *handle = bl;
  return DLA_OK;
}

extern "C" int dla_blas_destroy(void* handle) {
  clear_error();
  if (!handle) return DLA_OK;
  Blas* bl = (Blas*)handle;
  for (auto& kv : bl->plans) destroy_plan(kv.second);
  hipblasLtDestroy(bl->h);
  delete bl;
  return DLA_OK;
}

extern "C" int dla_layer_plan_check(const dla_desc* desc, int64_t B, int64_t N, int64_t H,
                                    size_t* ws_fwd_bytes, size_t* ws_bwd_bytes) {
  clear_error();
  return layer_plan(desc, B, N, H, ws_fwd_bytes, ws_bwd_bytes);
}

extern "C" int dla_layer_forward(const dla_desc* desc, int64_t B, int64_t N, int64_t H,
                                 const void* x, const void* w_qkv, const void* w_o, void* qkv,
                                 void* attn, float* lse, void* y, void* blas, void* ws,
                                 size_t ws_bytes, void* stream) {
  clear_error();
  size_t need = 0;
  int rc = layer_plan(desc, B, N, H, &need, nullptr);
  if (rc) return rc;
  if ((rc = check(x, "x")) || (rc = check(w_qkv, "w_qkv")) || (rc = check(w_o, "w_o")) ||
      (rc = check(qkv, "qkv")) || (rc = check(attn, "attn")) || (rc = check(lse, "lse")) ||
      (rc = check(y, "y")) || (rc = check(ws, "workspace")))
    return rc;
  if (!blas) return fail(DLA_E_INVALID, "blas handle is null");
  if (ws_bytes < need) return fail(DLA_E_WORKSPACE, "layer workspace needs %zu bytes, got %zu", need, ws_bytes);
  Blas* h = (Blas*)blas;
  hipStream_t st = (hipStream_t)stream;
  const int64_t M = B * N, E = H * kD;
  char* gws = (char*)ws + (need - kGemmWs);
  // Q, K, V = X W_q, X W_k, X W_v (column blocks of W_qkv)
  char* qb = (char*)qkv;
  for (int j = 0; j < 3; ++j)
    if ((rc = gemm_rm(h, st, gws, kGemmWs, false, false, M, E, E, x, E, (const __bf16*)w_qkv + j * E,
                      3 * E, qb + (size_t)j * M * E * 2, E, HIP_R_16BF, 0.f)))
      return rc;
  // A = DA(Q, K, V)
  const dla_shape s = head_shape(B, N, H);
  if ((rc = dla_forward(desc, &s, qb, qb + (size_t)M * E * 2, qb + (size_t)2 * M * E * 2, attn, lse, ws,
                        need - kGemmWs, stream)))
    return rc;
  // Y = A W_o
  return gemm_rm(h, st, gws, kGemmWs, false, false, M, E, E, attn, E, w_o, E, y, E, HIP_R_16BF, 0.f);
}

extern "C" int dla_layer_backward(const dla_desc* desc, int64_t B, int64_t N, int64_t H,
                                  const void* x, const void* w_qkv, const void* w_o,
                                  const void* qkv, const void* attn, const float* lse,
                                  const void* dy, void* dx, float* dw_qkv, float* dw_o, void* blas,
                                  void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  size_t need = 0;
  int rc = layer_plan(desc, B, N, H, nullptr, &need);
  if (rc) return rc;
  if ((rc = check(x, "x")) || (rc = check(w_qkv, "w_qkv")) || (rc = check(w_o, "w_o")) ||
      (rc = check(qkv, "qkv")) || (rc = check(attn, "attn")) || (rc = check(lse, "lse")) ||
      (rc = check(dy, "dy")) || (rc = check(dx, "dx")) || (rc = check(dw_qkv, "dw_qkv")) ||
      (rc = check(dw_o, "dw_o")) || (rc = check(ws, "workspace")))
    return rc;
  if (!blas) return fail(DLA_E_INVALID, "blas handle is null");
  if (ws_bytes < need) return fail(DLA_E_WORKSPACE, "layer workspace needs %zu bytes, got %zu", need, ws_bytes);
  Blas* h = (Blas*)blas;
  hipStream_t st = (hipStream_t)stream;
  const int64_t M = B * N, E = H * kD;
  char* da = (char*)ws;                                         // dA [M, E] bf16
  char* dqkv = da + align256((size_t)M * E * 2);                // dQ, dK, dV [3, M, E] bf16
  char* dxf = dqkv + align256((size_t)M * 3 * E * 2);           // dX [M, E] fp32
  const int S = weight_splits(M);
  float* part = (float*)(dxf + align256((size_t)M * E * 4));    // [4, S, E, E] fp32
  char* aws = (char*)part + align256((size_t)4 * S * E * E * 4);  // attention backward workspace
  const size_t aws_bytes = need - kGemmWs - (size_t)(aws - (char*)ws);
  char* gws = (char*)ws + (need - kGemmWs);
  // dA = dY W_o^T; partials of dW_o = A^T dY (chunk s: rows s M / S ...)
  const int64_t mk = M / S;
  const Batch wb{S, mk * E, mk * E, E * E};
  if ((rc = gemm_rm(h, st, gws, kGemmWs, false, true, M, E, E, dy, E, w_o, E, da, E, HIP_R_16BF, 0.f)))
    return rc;
  if ((rc = gemm_rm(h, st, gws, kGemmWs, true, false, E, E, mk, attn, E, dy, E, part + 3 * S * E * E, E,
                    HIP_R_32F, 0.f, wb)))
    return rc;
  // dQ, dK, dV
  const dla_shape s = head_shape(B, N, H);
  const char* qb = (const char*)qkv;
  const size_t t = (size_t)M * E * 2;
  if ((rc = dla_backward(desc, &s, qb, qb + t, qb + 2 * t, attn, lse, da, dqkv, dqkv + t, dqkv + 2 * t,
                         aws, aws_bytes, stream)))
    return rc;
  // dX = sum_j dP_j W_j^T in fp32, rounded once; dW_qkv column blocks = X^T dP_j
  for (int j = 0; j < 3; ++j)
    if ((rc = gemm_rm(h, st, gws, kGemmWs, false, true, M, E, E, dqkv + j * t, E,
                      (const __bf16*)w_qkv + j * E, 3 * E, dxf, E, HIP_R_32F, j ? 1.f : 0.f)))
      return rc;
  hipError_t e = launch_f32_to_bf16((const float*)dxf, dx, M * E, st);
  if (e != hipSuccess) return fail(DLA_E_HIP, "conversion launch: %s", hipGetErrorString(e));
  for (int j = 0; j < 3; ++j)
    if ((rc = gemm_rm(h, st, gws, kGemmWs, true, false, E, E, mk, x, E, dqkv + j * t, E, part + j * S * E * E,
                      E, HIP_R_32F, 0.f, wb)))
      return rc;
  // dW_qkv column blocks and dW_o: sums of the partials
  SplitSumArgs sa{};
  sa.part = part;
  for (int j = 0; j < 3; ++j) {
    sa.out[j] = dw_qkv + j * E;
    sa.ldo[j] = 3 * E;
  }
  sa.out[3] = dw_o;
  sa.ldo[3] = E;
  sa.splits = S;
  sa.E = (int)E;
  const int64_t blocks = std::min<int64_t>((E * E / 4 + 255) / 256, 1024);
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)blocks, 4), dim3(256), 0, st, sa);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(DLA_E_HIP, "split sum launch: %s", hipGetErrorString(e));
  return DLA_OK;
}
