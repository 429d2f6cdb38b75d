// Dilated attention forward in fp32 on the fp32 matrix cores (gfx950).
//
// Same decomposition as the bf16 kernel (units of sparse query rows of one
// pattern/batch/head/segment, rows gathered with the strided address
// generator; the gptget.net LongNet summary, section 方法论).  Nothing is
// rounded below fp32: v_mfma_f32_16x16x4_f32 takes fp32 operands and
// accumulates in fp32, and the softmax runs in fp32 on the vector ALUs.  The
// fp32 matrix rate equals the packed-vector fp32 rate and is twice what
// plain (unpacked) vector FMAs reach, and it leaves the vector ALUs free for
// the softmax, which is a small fraction of the work here (the matrix cores
// take 16x more cycles per product than with bf16 operands).
//
// A workgroup takes 64 sparse query rows: 4 waves x 16.  Each wave computes
// S^T = K Q^T for 16 keys x its 16 queries per MFMA chain (the head dimension
// contracted 4 at a time: step t pairs dimension 16g + t with lane group
// g = lane / 16), so a lane holds one query's scores for 4 keys of every
// 16-key block, then O^T += V^T P^T with P^T taken straight from that
// accumulator layout (step s contracts keys 4g + s of the block).
// K tiles sit in LDS key-major and V tiles d-major (transposed on their way
// in), both padded so that the 16-byte operand reads of 16 lanes hit
// distinct banks.  Tiles of 32 keys, double-buffered: the next tile's global
// loads are in registers while the current one is computed.
#include "dla_device.h"

namespace dla {

constexpr int kF32BM = 64;        // query rows per workgroup (4 waves x 16)
constexpr int kF32BN = 32;        // keys per LDS tile (two 16-key blocks)
constexpr int kF32KPad = kD + 4;  // floats per key row of the K tile
constexpr int kF32VPad = kF32BN + 4;  // floats per head-dimension row of the V^T tile

struct __align__(16) F32Stage {
  float k[kF32BN * kF32KPad];     // K[key][d]
  float vt[kD * kF32VPad];        // V^T[d][key]
};

__device__ __forceinline__ f32x4 mfma16(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const AttnFwdArgs a) {
  __shared__ F32Stage st[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
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
  const int qrow = q0 + 16 * wave + li;      // this lane's query (as B operand and in S^T)
  const float c = a.scale_log2;

  // Q^T operand: lane (query li, group g) holds Q[qrow][16g .. 16g+15].
  float qv[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 t = qrow < L ? *(const float4*)(Qh + (int64_t)qrow * rstride + 16 * g + 4 * i)
                              : float4{0.f, 0.f, 0.f, 0.f};
    qv[4 * i] = t.x; qv[4 * i + 1] = t.y; qv[4 * i + 2] = t.z; qv[4 * i + 3] = t.w;
  }

  // Tile loads: 32 keys x 16 float4 per tensor, two of each per thread.
  // Rows past the segment end load zeros (their scores are masked, and a
  // zero value row keeps 0 * V finite).
  const int kend = a.causal ? min(L, q0 + kF32BM) : L;
  const int ntile = (kend + kF32BN - 1) / kF32BN;
  float4 kx[2], vx[2];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int key = t * kF32BN + (idx >> 4), c4 = idx & 15;
      if (key < L) {
        kx[i] = *(const float4*)(Kh + (int64_t)key * rstride + 4 * c4);
        vx[i] = *(const float4*)(Vh + (int64_t)key * rstride + 4 * c4);
      } else {
        kx[i] = float4{0.f, 0.f, 0.f, 0.f};
        vx[i] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_tile = [&](F32Stage& s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int kr = idx >> 4, c4 = idx & 15;
      *(float4*)&s.k[kr * kF32KPad + 4 * c4] = kx[i];
      s.vt[(4 * c4 + 0) * kF32VPad + kr] = vx[i].x;
      s.vt[(4 * c4 + 1) * kF32VPad + kr] = vx[i].y;
      s.vt[(4 * c4 + 2) * kF32VPad + kr] = vx[i].z;
      s.vt[(4 * c4 + 3) * kF32VPad + kr] = vx[i].w;
    }
  };

  f32x4 oacc[4];                    // O^T[16 db + 4g + v][query li]
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;          // running maximum of this lane's query (log2 domain)
  float l_run = 0.f;                // this lane's part of the row sum (its 8 keys per tile)

  load_tile(0);
  store_tile(st[0]);
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const F32Stage& cur = st[t & 1];
    if (t + 1 < ntile) load_tile(t + 1);

    // S^T of the tile's two 16-key blocks: two independent chains of 16.
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
    const float* k0row = &cur.k[li * kF32KPad + 16 * g];
    const float* k1row = &cur.k[(16 + li) * kF32KPad + 16 * g];
#pragma unroll
    for (int cq = 0; cq < 4; ++cq) {
      const float4 ka = *(const float4*)(k0row + 4 * cq);
      const float4 kb = *(const float4*)(k1row + 4 * cq);
      s0 = mfma16(ka.x, qv[4 * cq + 0], s0);
      s1 = mfma16(kb.x, qv[4 * cq + 0], s1);
      s0 = mfma16(ka.y, qv[4 * cq + 1], s0);
      s1 = mfma16(kb.y, qv[4 * cq + 1], s1);
      s0 = mfma16(ka.z, qv[4 * cq + 2], s0);
      s1 = mfma16(kb.z, qv[4 * cq + 2], s1);
      s0 = mfma16(ka.w, qv[4 * cq + 3], s0);
      s1 = mfma16(kb.w, qv[4 * cq + 3], s1);
    }

    // Mask and online softmax: element v of block bb is key t*32 + 16bb + 4g + v.
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    const int kbase = t * kF32BN + 4 * g;
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kbase + 16 * (e >> 2) + (e & 3);
      if (key >= L || (a.causal && key > qrow)) sv[e] = -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) oacc[db][v] *= alpha;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = exp2f(__builtin_fmaf(sv[e], c, -m_use));
      l_run += pv[e];
    }

    // O^T += V^T P^T: per 16-key block and 16-dim block, four steps (keys 4g + s).
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const float4 va = *(const float4*)&cur.vt[(16 * db + li) * kF32VPad + 16 * bb + 4 * g];
        oacc[db] = mfma16(va.x, pv[4 * bb + 0], oacc[db]);
        oacc[db] = mfma16(va.y, pv[4 * bb + 1], oacc[db]);
        oacc[db] = mfma16(va.z, pv[4 * bb + 2], oacc[db]);
        oacc[db] = mfma16(va.w, pv[4 * bb + 3], oacc[db]);
      }

    if (t + 1 < ntile) store_tile(st[(t + 1) & 1]);
    __syncthreads();
  }

  // Row sum over the four lane groups that share the query.
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  if (qrow >= L) return;
  const float inv = 1.f / lt;
  const float lse = (m_run + log2f(lt)) * kLn2;
  const int64_t bh = (int64_t)b * a.H + h;
  float* dst;
  float* lse_dst;
  if (p == a.prim) {
    const int64_t n = base_row + (int64_t)qrow * r;
    dst = (float*)a.o + head_off + n * a.sn;
    lse_dst = a.lse + bh * a.N + n;
  } else {
    const int64_t nsparse = a.nsp[p];
    const int64_t m = seg * L_full + qrow;
    dst = (float*)a.part_o[p] + (bh * nsparse + m) * kD;
    lse_dst = a.part_lse[p] + bh * nsparse + m;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
    *(float4*)(dst + 16 * db + 4 * g) = float4{oacc[db][0] * inv, oacc[db][1] * inv,
                                               oacc[db][2] * inv, oacc[db][3] * inv};
  if (g == 0) *lse_dst = lse;
}

hipError_t launch_attn_fwd_f32(const AttnFwdArgs& a, hipStream_t stream) {
  if (a.sched.total == 0) return hipSuccess;
  TimedLaunch tl("attn_fwd_f32", stream);
  hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)a.sched.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dla
