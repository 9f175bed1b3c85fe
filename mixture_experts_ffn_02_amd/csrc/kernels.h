// Host-side launch interface of the HIP kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Compute units of the current device (queried once, 256 if the query fails).
int cu_count();

// ------------------------------------------------------------------ router
struct RouteLaunch {
  const void* x;         // [T, d] fp32 or bf16 bits
  int dtype;             // 0 fp32, 1 bf16
  int64_t T;
  int d, E, k, score, renorm;
  const float* w_router;  // [E, d]
  const float* bias;      // [E] or null
  int32_t* idx;           // [T, k]
  float* w;               // [T, k]
  int32_t* hist;          // [n_blocks, E] or null
  int32_t* rank;          // [T, k] or null (needs hist)
  float* logits;          // [T, E] scratch for the small-batch split path, or null (always fused)
  int bias_on_logits;     // nonzero: selection value = logit + bias (else score + bias)
  const float* noise;     // [T, E] added to the selection value, or null
  double* mpart;          // [n_blocks, E + 1] metric partials (score sums, sum of lse^2), or null
};
// Tokens per router block (its rows of the block histograms) for a launch
// with a logits buffer over T tokens of d features.
int route_tokens_per_block(int E, int64_t T, int d);
size_t route_lds_bytes(int E, int k);
hipError_t launch_route(const RouteLaunch& a, hipStream_t s);
// The fp32 logits alone ([T, E] into a.logits), the same fma chains as the router.
hipError_t launch_logits(const RouteLaunch& a, hipStream_t s);
// out[6] = z-loss, aux loss, cv, entropy (bits), max/mean load, unused share,
// from the partials of launch_route (nb blocks) and the expert counts.
hipError_t launch_router_metrics(const double* mpart, int nb, const int32_t* counts, int64_t T, int E, int k,
                                 double* out, hipStream_t s);
// One step of the balance controller on bias [E] from counts [E].
hipError_t launch_bias_update(const int32_t* counts, int E, float rate, float* bias, hipStream_t s);

// --------------------------------------------------------------- dispatch
// Per-block expert histograms and ranks from expert ids (no routing).
int hist_tokens_per_block();
hipError_t launch_hist_rank(const int32_t* idx, int64_t T, int k, int E, int32_t* hist, int32_t* rank,
                            hipStream_t s);
// counts[e] = sum over blocks of hist[b, e].
hipError_t launch_counts(const int32_t* hist, int nb, int E, int32_t* counts, hipStream_t s);
// counts, offsets [E+1], per-block bases [nb, E], and the tile list of a
// grouped GEMM with row tile bm: tiles[i] = (group, m-tile), n_tiles[0] = count.
// extra > 0 appends group E of `extra` rows (offsets then has E + 2 entries).
hipError_t launch_scan(const int32_t* hist, int nb, int E, int32_t* counts, int32_t* offsets, int32_t* base, int bm,
                       int32_t* n_tiles, int2* tiles, hipStream_t s, int64_t extra = 0);
// Tile list from device offsets [G+1].
hipError_t launch_tiles_from_offsets(const int32_t* offsets, int G, int bm, int32_t* n_tiles, int2* tiles,
                                     hipStream_t s);
// row_of [T, k], tok_of_row [T*k] and optionally x_perm rows; with `extra`
// also tok_of_row[T*k + t] = t (the rows of an appended all-token group).
hipError_t launch_scatter(const int32_t* idx, const int32_t* rank, const int32_t* base, int64_t T, int k, int E,
                          int tokens_per_block, int32_t* row_of, int32_t* tok_of_row, const void* x, void* x_perm,
                          int row_bytes, hipStream_t s, bool extra = false);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// ------------------------------------------------------------------- GEMM
constexpr int kXcd = 8;     // XCDs (L2 domains); workgroup i runs on XCD i % kXcd
constexpr int kGroupM = 8;  // default row tiles per raster group

struct GemmLaunch {
  int dtype;               // 0 fp32, 1 bf16 (operands; accumulation fp32)
  bool gateup;             // true: out = silu(A B0^T) * (A B1^T) in dtype; false: out = A B0^T in fp32
  bool b_stream = false;   // weight rows read once (few rows per group): non-temporal DMA
  int bn_cap = 0;          // forward products with 64-row tiles: widest column tile at most this (0: widest)
  bool raster_by_group = false;  // grouped eight-wave gate/up: raster groups stay inside each group's row tiles
  const void* a;           // rows of K elements
  const int32_t* a_rows;   // null, or the source row of a for every grouped row (gather)
  int64_t a_row_count;     // rows of a (gather indices are clamped into range)
  int n_groups;            // G (tile entries naming another group are skipped)
  const void* b0;          // [G, N, K]
  const void* b1;          // [G, N, K] (gateup)
  int extra_group = -1;    // group whose weights are bx0 / bx1 instead of rows of b0 / b1 (-1: none)
  const void* bx0 = nullptr;  // [N, K]
  const void* bx1 = nullptr;  // [N, K] (gateup)
  void* out;               // [rows, N]
  int N, K;
  // bf16 plain product only: b0 / b1 / bx0 / bx1 hold [K, N] (N contiguous)
  // per group instead of [N, K]; K rows below bt_ksplit (a multiple of 64)
  // come from b0 / bx0, the others from b1 / bx1 (0: all from b0 / bx0)
  bool bt = false;
  int bt_ksplit = 0;
  // grouped mode: tile list from launch_scan / launch_tiles_from_offsets
  const int32_t* offsets;  // [G+1] or null for one dense group of `rows` rows
  const int2* tiles;
  const int32_t* n_tiles;
  int64_t max_m_tiles;     // grid bound on m-tiles
  int group_m;             // row tiles per raster group (0: default)
  int64_t rows;            // dense mode: number of rows
  // gate/up only: also store the fp32 pre-activations g and u ([rows, N]),
  // which the backward pass needs
  float* out_g = nullptr;
  float* out_u = nullptr;
  // K-grouped mode (weight gradients): entry v of the tile list is chunk v,
  // vgroups[v] = (group e, first K column, end K column, slot), reducing over
  // those K columns (multiples of the K stage) of A (m_rows rows) and B (N
  // rows), both panelled with K capacity K and panels of BM (A) and BN (B)
  // rows (see panel_offset). Its output is [m_rows, N] (rows >= m_valid are
  // not stored): for slot -1 the gradient of group e (kg_out_row), else
  // partial buffer `part` + slot*m_rows*N. No row gather, no weight stacking.
  // koffs marks the mode (the group segments the chunks were cut from).
  const int32_t* koffs = nullptr;
  const int4* vgroups = nullptr;
  float* part = nullptr;
  const int32_t* xcd_bounds = nullptr;  // [kXcd + 1] ranges of the raster order per XCD (launch_kg_setup)
  int m_rows = 0, m_valid = 0, m0 = 0;
  void* out1 = nullptr;
  void* xout0 = nullptr;
  void* xout1 = nullptr;
};

// K-grouped output row mm (of m_rows) of group grp: rows below m0 go to out +
// grp*m0*N, the others to out1 + grp*(m_rows-m0)*N (m0 = 0: all to out, grp*
// m_rows*N); the extra group writes to xout0 / xout1 instead. fp32.
__host__ __device__ inline float* kg_out_row(const GemmLaunch& g, int grp, int mm) {
  const bool second = g.m0 > 0 && mm >= g.m0;
  const int rows0 = g.m0 > 0 ? g.m0 : g.m_rows;
  float* base;
  if (grp == g.extra_group)
    base = static_cast<float*>(second ? g.xout1 : g.xout0);
  else if (second)
    base = static_cast<float*>(g.out1) + (size_t)grp * (g.m_rows - g.m0) * g.N;
  else
    base = static_cast<float*>(g.out) + (size_t)grp * rows0 * g.N;
  return base + (size_t)(second ? mm - g.m0 : mm) * g.N;
}
// Row tile (64, 128 or 256) for `rows` rows in `groups` groups, n output
// columns of the gate/up product and its K = d_in; the tile list of a grouped
// launch must be built with the same value.
int gemm_bm(int dtype, int64_t rows, int64_t groups, int n, int d_in);
// Row tile of the forward gate/up and down products (gemm_bm, or 256 where
// the eight-wave kernel runs both and the groups are long enough).
int gemm_bm_fwd(int dtype, int64_t rows, int64_t groups, int n, int d_in);
// Column-tile caps (GemmLaunch::bn_cap) of the forward gate/up and down
// products with the row tile of gemm_bm_fwd; d_out = N of the down product.
struct GemmCaps {
  int gateup, down;
};
GemmCaps gemm_bn_caps(int dtype, int64_t rows, int64_t groups, int n, int d_in, int d_out);
// Smallest row tile of a grouped launch: tile lists hold at most
// rows / kMinTileRows + groups entries.
constexpr int kMinTileRows = 64;
hipError_t launch_gemm(const GemmLaunch& g, int bm, hipStream_t s);
// bf16 forward products (gate/up with SwiGLU, or down) on 256 x 256 tiles of
// eight waves (gemm8.hip): K % 64 == 0, N % 128 (gate/up) or N % 256 (down);
// grouped launches take tile lists built with a row tile of 256.
hipError_t launch_gemm8(const GemmLaunch& g, hipStream_t s);
// Forward products with row tile bm: launch_gemm8 where bm is 256 and the
// shape fits it, else launch_gemm.
bool gemm8_fits(const GemmLaunch& g, int bm);
hipError_t launch_gemm_fwd(const GemmLaunch& g, int bm, hipStream_t s);

// --------------------------------------------------------------- backward
hipError_t launch_to_bf16(int64_t n, const float* in, uint16_t* out, hipStream_t s);
// Per token: d_w[t,j] = <h_r, dhu_r> for its routed rows r = row_of[t,j];
// dgu[r] = [dG | dU] of dH = w dhu (w = 1 on the shared row T*k + t);
// wrow[r] = w.
hipError_t launch_swiglu_bwd(int dtype, int64_t T, int k, int f, const float* dhu, const float* g, const float* u,
                             const void* h, const float* w, const int32_t* row_of, bool shared, void* dgu, float* dtw,
                             float* wrow, hipStream_t s);
// dx[t] = sum_j dxp[row_of[t, j]] (+ dxp[T*k + t], shared) (+ dxr[t]), and,
// when dl is given, + sum_{e<E} dl[t, e] w_router[e] (the router term
// computed in place, fp32, experts ascending; for few experts).
hipError_t launch_gather_bwd(int64_t T, int d, int k, const float* dxp, const int32_t* row_of, bool shared,
                             const float* dxr, const float* dl, int ep, int E, const float* w_router, float* dx,
                             hipStream_t s);
// Panelled operand of a K-grouped GEMM: rows in panels of P rows (one GEMM
// tile), each panel K-blocked with K capacity kcap, so that a tile walks one
// contiguous stretch of memory. Element (r, col), in elements, with kb = 128
// bytes / element size (one K stage):
__host__ __device__ inline int64_t panel_offset(int64_t r, int64_t col, int P, int64_t kcap, int kb) {
  return (r / P) * P * kcap + (col / kb) * P * kb + (r % P) * kb + col % kb;
}
// out[b][c][col0 + r] = in[b][r][c] (r < R), 0 for R <= r < Rpad; dtype 0 fp32, 1 bf16.
// panel > 0: out (one batch) is instead the panelled matrix with C rows,
// panels of `panel` rows and K capacity Rpad (ldo, col0 unused).
hipError_t launch_transpose(int dtype_in, int dtype_out, const void* in, void* out, int64_t batch, int64_t R,
                            int64_t Rpad, int C, int64_t ldo, int64_t col0, hipStream_t s, int panel = 0);
// Grouped rows (through row_map when given; times scale[row] when given)
// into per-group zero-padded K segments (columns koffs[e] ..) of a panelled
// matrix with C rows, panels of `panel` rows (a multiple of 64 dividing C)
// and K capacity max_cols; in has dtype_in (fp32 into bf16 allowed).
hipError_t launch_transpose_groups(int dtype_in, int dtype, const void* in, const int32_t* row_map,
                                   const float* scale, const int32_t* offsets, const int32_t* koffs, int G, int C,
                                   int panel, int64_t max_cols, void* out, hipStream_t s);
// out[e][c] = sum over segments s (in order) of part[s][e][c], e < rows_out
hipError_t launch_sum_segments(const float* part, int nseg, int64_t seg_stride, int64_t n, float* out, hipStream_t s);
// K segments, chunks and tile list of a K-grouped launch: koffs[e] = sum over
// groups before e of their row counts rounded up to kp (no offsets: kp each);
// groups longer than cap stages (ke K elements each; cap <= 0: no cut) are cut
// into chunks, vgroups[v] as GemmLaunch describes; red / n_red list the cut
// groups for launch_kg_reduce; tiles = every (chunk, m-tile), mt m-tiles a
// chunk. With xcd_bounds: the ranges of the launch's raster order (ntn column
// tiles, kGroupM row tiles a raster group) that give each XCD an equal share
// of K stages. Sizes: vgroups and red hold G + (total stages) / cap entries.
hipError_t launch_kg_setup(int G, const int32_t* offsets, int kp, int mt, int32_t* koffs, int2* tiles,
                           int32_t* n_tiles, int4* vgroups, int cap, int4* red, int32_t* n_red, hipStream_t s,
                           int ntn = 0, int ke = 1, int32_t* xcd_bounds = nullptr);
// Adds the partial sums of every cut group (red, n_red[0] of at most max_red)
// to its gradient in slot order.
hipError_t launch_kg_reduce(const GemmLaunch& g, const int4* red, const int32_t* n_red, int max_red, hipStream_t s);
// Work-conserving chunk length (K stages) for a K-grouped launch of row tile
// bm with mt x ntn tiles per group and at most `stages` K stages in all.
int gemm_kg_cap(int bm, int64_t stages, int mt, int ntn);
hipError_t launch_router_bwd(int64_t T, int E, int ep, int k, const float* logits, const int32_t* idx,
                             const float* dtw, const int32_t* counts, int score, int renorm, float z_coef,
                             float aux_coef, float* dl, hipStream_t s);
// Row tile and column tile of a K-grouped launch with m_rows output rows and
// n columns: the panel heights of its A and B operands.
int gemm_kg_bm(int dtype, int m_rows, int n, int groups);
int gemm_kg_bn(int bm, int n);

// ---------------------------------------------------------------- combine
hipError_t launch_combine(int64_t T, int d, int k, const float* y_perm, const int32_t* row_of, const float* w,
                          const float* y_shared, float* y, hipStream_t s);

}  // namespace moe
