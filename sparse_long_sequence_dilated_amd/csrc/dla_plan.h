// Host planner of libdla: validation, workspace layout and the work-unit
// schedule shared by all launches.  Pure C++ (no HIP), so it is built and
// tested on the CPU as well.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dla.h"

namespace dla {

constexpr int kMaxP = DLA_MAX_PATTERNS;
constexpr int kD = DLA_HEAD_DIM;

// Longest-first decode of a flat work-unit index into (pattern, batch, head,
// segment, tile).  A unit is one tile of rows of one sparsified segment.
// Under a causal mask the work of a tile grows with its index, so units are
// ordered by tile index, highest first, with all patterns interleaved at each
// tile level; inside a level the order is pattern, batch, head, segment.
struct Schedule {
  int nband;                    // bands of tile levels with the same active patterns
  int order[kMaxP];             // patterns sorted by tile count, descending
  int64_t cum[kMaxP + 1];       // prefix sums of B*H*nseg over `order`
  int band_hi[kMaxP];           // band covers tile levels [band_lo, band_hi), high first
  int band_npat[kMaxP];         // patterns active in the band (a prefix of `order`)
  int64_t band_start[kMaxP + 1];
  int64_t total;                // number of units
  // The (batch, head, segment) units of every pattern are split into
  // `groups` equal runs, scheduled one after another (each longest first):
  // group j holds segment-heads j*chunk[p] .. (j+1)*chunk[p]-1 of pattern p,
  // so that a group's keys and values stay cache-resident while its units
  // re-stream them.  Units past a pattern's last segment-head are empty.
  int64_t groups;
  int64_t upg;                  // units per group
  int64_t chunk[kMaxP];         // segment-heads of each pattern per group
  int64_t count[kMaxP];         // segment-heads of each pattern: B * H * nseg
};

struct Plan {
  int64_t B, N, H;
  int dtype;                    // dla_dtype
  int esize;                    // bytes per element of q/k/v/o
  int64_t sb, sn, sh;           // element strides of [B, N, H, D] tensors
  int P;
  int causal;
  float scale;
  int w[kMaxP], r[kMaxP], L[kMaxP];
  int64_t nseg[kMaxP];          // ceil(N / w): a last segment may be cut short
  int64_t nsp[kMaxP];           // ceil(N / r): sparse rows per (batch, head)
  // Sequence shard (dla_forward_shard): a pattern whose segments are longer
  // than the shard spans devices; the shard holds L = N/r of its Lk = w/r
  // sparse rows, starting at sparse row qoff of one segment (nseg = 1).
  bool shard;
  bool span[kMaxP];
  int Lk[kMaxP];                // key rows per segment (== L unless spanning)
  int qoff[kMaxP];              // segment row of local sparse row 0 (0 unless spanning)
  int prim;                     // pattern whose result goes straight to o/lse
  bool need_combine;            // a merge pass is needed after the attention pass
  bool empty;                   // B == 0 or H == 0: nothing to do
  // forward workspace: per-pattern partial O_p [B,H,N/r,D] and LSE_p [B,H,N/r]
  size_t part_o_off[kMaxP];
  size_t part_lse_off[kMaxP];
  size_t ws_fwd;
  // backward workspace: (-LSE * log2 e, -D), D = rowsum(dO*O), [B,H,N] float pairs;
  // with several patterns, per pattern the fp32 partial dQ, dK, dV [B,H,N/r,D]
  // in sparse order (only rows that another pattern also keeps are written)
  size_t ld_off;
  size_t part_g_off[kMaxP][3];
  bool need_finalize;           // some rows are kept by several patterns
  size_t ws_bwd;
  // shard backward (after the partials, which persist until the finish
  // pass): one spanning segment at a time, contiguous per (batch, head):
  // q, dO, k, v [B,H,Lk,D] bf16, (LSE2, D) [B,H,Lk] float2, dK, dV [B,H,Lk,D]
  // fp32, sized for the longest spanning segment.
  uint32_t span_mask;
  size_t seg_off[7];            // q, do, ld, k, v, dk, dv
  int64_t pairs;
};

// Validate and fill `plan` (for one shard of a longer sequence when `shard`
// is not null).  Returns DLA_OK or an error code; the message is recorded for
// dla_last_error().
int make_plan(const dla_desc* desc, const dla_shape* shape, Plan* plan,
              const dla_shard* shard = nullptr);

// Fill `s` for tiles of `tile_rows` sparse rows per unit.
void make_schedule(const Plan& plan, int tile_rows, Schedule* s);

// Residue classes rho (mod the lcm of the rates) that the merge passes must
// visit for head h.  When exactly one pattern has r = 1 (and its segments
// stay on this device) and every rate is a power of two, a row that any
// other pattern keeps has rho = h mod r_min, r_min being the smallest other
// rate (it divides the others); rows of the other classes are kept by the
// r = 1 pattern alone and need no merge.  Returns r_min then, else 1 (every
// class).
uint32_t class_step(const Plan& plan);

// True when the environment has DLA_LOG=1 (read once): the planner then
// writes one line per plan and per schedule to stderr.
bool log_enabled();

// Record a formatted message for dla_last_error() and return `code`.
int fail(int code, const char* fmt, ...);
void clear_error();

}  // namespace dla
