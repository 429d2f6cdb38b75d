// Dilated attention forward in fp32 (no reduced-precision step anywhere).
//
// Same decomposition as the bf16 kernel (units of sparse query rows of one
// pattern/batch/head/segment, rows gathered with the strided address
// generator; the gptget.net LongNet summary, section 方法论), computed on the
// fp32 vector ALUs: four lanes share one query row, each owning 16 of the 64
// head dimensions; scores are reduced across the four lanes.  K and V tiles of
// 32 rows are staged in LDS.
#include "dla_device.h"

namespace dla {

constexpr int kF32BM = 64;
constexpr int kF32BN = 32;

__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const AttnFwdArgs a) {
  __shared__ float ks[kF32BN][kD + 4];
  __shared__ float vs[kF32BN][kD + 4];
  const int tid = threadIdx.x;
  int p, b, h, tile;
  int64_t seg;
  if (!decode_unit(a.sched, blockIdx.x, (int)a.H, a.nseg, p, b, h, seg, tile)) return;
  const int w = a.w[p], r = a.r[p], L_full = a.L[p];
  // fewer in a cut-short last segment (of the sequence or of this batch's)
  const int L = seg_rows(batch_len(a.lengths, b, a.N), seg, w, r, h, L_full);
  if (tile * kF32BM >= L) return;                      // nothing of this segment left
  const int64_t base_row = seg_base_row(seg, w, r, h);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int64_t rstride = (int64_t)r * a.sn;
  const float* Qh = (const float*)a.q + head_off + base_row * a.sn;
  const float* Kh = (const float*)a.k + head_off + base_row * a.sn;
  const float* Vh = (const float*)a.v + head_off + base_row * a.sn;

  const int q0 = tile * kF32BM;
  const int qi = tid >> 2, pp = tid & 3;
  const int row = q0 + qi;
  const bool valid = row < L;
  const float c = a.scale_log2;

  float qv[16], acc[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 t = valid ? *(const float4*)(Qh + (int64_t)row * rstride + 16 * pp + 4 * i)
                     : float4{0.f, 0.f, 0.f, 0.f};
    qv[4 * i] = t.x; qv[4 * i + 1] = t.y; qv[4 * i + 2] = t.z; qv[4 * i + 3] = t.w;
  }
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = a.causal ? min(L, q0 + kF32BM) : L;
  for (int k0 = 0; k0 < kend; k0 += kF32BN) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int kr = idx >> 4, c4 = idx & 15;
      const int key = k0 + kr;
      float4 kx = float4{0.f, 0.f, 0.f, 0.f}, vx = float4{0.f, 0.f, 0.f, 0.f};
      if (key < L) {
        kx = *(const float4*)(Kh + (int64_t)key * rstride + 4 * c4);
        vx = *(const float4*)(Vh + (int64_t)key * rstride + 4 * c4);
      }
      *(float4*)&ks[kr][4 * c4] = kx;
      *(float4*)&vs[kr][4 * c4] = vx;
    }
    __syncthreads();
    float sc[kF32BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < 16; ++d) s = __builtin_fmaf(qv[d], ks[j][16 * pp + d], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      const int key = k0 + j;
      if (key >= L || (a.causal && key > row)) s = -INFINITY;
      sc[j] = s;
      mx = fmaxf(mx, s);
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      const float pv = exp2f(__builtin_fmaf(sc[j], c, -m_use));
      l_run += pv;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] = __builtin_fmaf(pv, vs[j][16 * pp + d], acc[d]);
    }
    __syncthreads();
  }

  if (!valid) return;
  const float inv = 1.f / l_run;
  const float lse = (m_run + log2f(l_run)) * kLn2;
  const int64_t bh = (int64_t)b * a.H + h;
  float* dst;
  float* lse_dst;
  if (p == a.prim) {
    const int64_t n = base_row + (int64_t)row * r;
    dst = (float*)a.o + head_off + n * a.sn;
    lse_dst = a.lse + bh * a.N + n;
  } else {
    const int64_t nsparse = a.nsp[p];
    const int64_t m = seg * L_full + row;
    dst = (float*)a.part_o[p] + (bh * nsparse + m) * kD;
    lse_dst = a.part_lse[p] + bh * nsparse + m;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(float4*)(dst + 16 * pp + 4 * i) = float4{acc[4 * i] * inv, acc[4 * i + 1] * inv,
                                               acc[4 * i + 2] * inv, acc[4 * i + 3] * inv};
  if (pp == 0) *lse_dst = lse;
}

hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a, hipStream_t stream) {
  if (a.sched.total == 0) return hipSuccess;
  TimedLaunch tl("attn_fwd_f32", stream);
  hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)a.sched.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
