// Backward pass of the MoE FFN layer: the element-wise and data-movement
// kernels around the grouped GEMMs (which gemm.hip runs).
//
// The layer's forward (moe-200m-qwen3-100b README, "Architecture diagram" and
// "SigmoidRouter"; SpecForge PR #930, "What this adds") is
//   y_t = sum_j w_tj E_{e_tj}(x_t) (+ S(x_t)),  E(x) = W_down (silu(W_gate x) * W_up x),
// with w from the unbiased scores of the chosen experts. Given dy, the
// backward runs (row r = slot (t, j), or the shared row of t, weight 1)
//   down^T    : dHu_r = dy_t W_down      (grouped GEMM gathering rows of dy)
//   combine^T : d_w[t,j] = <h_r, dHu_r>  (which equals <dy_t, y_r>), dH_r = w dHu_r
//   SwiGLU^T  : dG = dH u silu'(g), dU = dH silu(g)
//   gate/up^T : dXp = dG W_gate + dU W_up (grouped GEMM, one K = 2 d_ff)
//   gather^T  : dx_t = sum_j dXp[row_of[t,j]] (+ shared row) (+ router term)
//   weights   : dW = (per-group transposed activations) products (K-grouped GEMMs)
//   router    : d logits from d_w through the weight rule (+ z-loss, aux loss)
// Every reduction runs in a fixed order; nothing uses atomics.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
  return f32_to_bf16(v);
}
template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return bf16_to_f32(v);
}

// Four consecutive elements as fp32, and back. load4s: the same as a
// streaming (non-temporal) load, for data this kernel is the last to read.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p);
template <typename T>
__device__ __forceinline__ f32x4 load4s(const T* p);
template <>
__device__ __forceinline__ f32x4 load4s<float>(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
template <>
__device__ __forceinline__ f32x4 load4s<uint16_t>(const uint16_t* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return f32x4{bf16_to_f32((uint16_t)(v.x & 0xFFFF)), bf16_to_f32((uint16_t)(v.x >> 16)),
               bf16_to_f32((uint16_t)(v.y & 0xFFFF)), bf16_to_f32((uint16_t)(v.y >> 16))};
}
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4{bf16_to_f32((uint16_t)(v.x & 0xFFFF)), bf16_to_f32((uint16_t)(v.x >> 16)),
               bf16_to_f32((uint16_t)(v.y & 0xFFFF)), bf16_to_f32((uint16_t)(v.y >> 16))};
}
template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 v) {
  uint2 o;
  o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = o;
}

// dy in the operand type (bf16 layers): the down^T GEMM gathers its rows.
__global__ __launch_bounds__(256) void k_to_bf16(int64_t n4, const float* __restrict__ in, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  store4<uint16_t>(out + 4 * i, reinterpret_cast<const f32x4*>(in)[i]);
}

// One block per token t, its k routed rows (slot j: row row_of[t,j], weight
// w[t,j]) and its shared-expert row (T*k + t, weight 1). The down^T GEMM gave
// the unweighted dHu_r = dy_t W_down (the layer's expert output for the row
// being y_r = h_r W_down^T). Per row:
//   d_w[t,j] = <h_r, dHu_r>  (= <dy_t, y_r>; fixed-order block reduction)
//   dH = w dHu;  dG = dH u s (1 + g (1 - s)),  dU = dH g s,  s = sigmoid(g)
// stored side by side, dgu[r] = [dG_r | dU_r]; wrow[r] = w (the row's weight,
// for the weight gradient of W_down).
template <typename DT>
__global__ __launch_bounds__(256) void k_swiglu_bwd(int64_t T, int k, int f, const float* __restrict__ dhu,
                                                    const float* __restrict__ gp, const float* __restrict__ up,
                                                    const DT* __restrict__ hp, const float* __restrict__ w,
                                                    const int32_t* __restrict__ row_of, int shared,
                                                    DT* __restrict__ dgu, float* __restrict__ dtw,
                                                    float* __restrict__ wrow) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nj = k + (shared ? 1 : 0);
  for (int j = 0; j < nj; ++j) {
    const int64_t r = j < k ? (int64_t)row_of[t * k + j] : T * k + t;
    const float wt = j < k ? w[t * k + j] : 1.0f;
    float dot = 0.0f;
    for (int c = tid * 4; c < f; c += 1024) {
      const int64_t i = r * f + c;
      const f32x4 dv = load4s<float>(dhu + i);  // read once
      const f32x4 gv = load4s<float>(gp + i);
      const f32x4 uv = load4s<float>(up + i);
      const f32x4 hv = load4<DT>(hp + i);
      f32x4 dg, du;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dot = __builtin_fmaf(hv[q], dv[q], dot);
        const float h = wt * dv[q], g = gv[q], u = uv[q];
        const float s = 1.0f / (1.0f + __expf(-g));
        dg[q] = h * u * s * (1.0f + g * (1.0f - s));
        du[q] = h * g * s;
      }
      store4<DT>(dgu + r * 2 * f + c, dg);
      store4<DT>(dgu + r * 2 * f + f + c, du);
    }
    if (j < k) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
      if (lane == 0) red[wave] = dot;
      __syncthreads();
      if (tid == 0 && dtw) dtw[t * k + j] = (red[0] + red[1]) + (red[2] + red[3]);
      __syncthreads();
    }
    if (tid == 0) wrow[r] = wt;
  }
}

// dx_t = sum_j dXp[row_of[t, j]] (slots in order) (+ dXp[T*k + t], the
// shared expert) (+ dxr_t, the router term).
template <bool ROUTER>
__global__ __launch_bounds__(256) void k_gather_bwd(int64_t T, int d, int k, const float* __restrict__ dxp,
                                                    const int32_t* __restrict__ row_of, int shared,
                                                    const float* __restrict__ dxr, const float* __restrict__ dl, int ep,
                                                    int E, const float* __restrict__ wr, float* __restrict__ dx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of dx
  const int nq = d / 4;
  if (i >= T * nq) return;
  const int64_t t = i / nq;
  const int c = (int)(i % nq) * 4;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // rows read once: streaming loads
  for (int j = 0; j < k; ++j)
    acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dxp + (int64_t)row_of[t * k + j] * d + c));
  if (shared) acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dxp + (T * k + t) * d + c));
  if (dxr) acc += *reinterpret_cast<const f32x4*>(dxr + t * d + c);
  if constexpr (ROUTER) {
    f32x4 r = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* dlr = dl + t * ep;
    for (int e = 0; e < E; ++e) {
      const float a = dlr[e];
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(wr + (size_t)e * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) r[q] = __builtin_fmaf(a, w4[q], r[q]);
    }
    acc += r;
  }
  *reinterpret_cast<f32x4*>(dx + t * d + c) = acc;
}

// Batched transpose through 64 x 64 LDS tiles (C and Rpad multiples of 64):
//   out[b][c][col0 + r] = in[b][r][c] for r < R, c < C; 0 for R <= r < Rpad.
// in rows have C elements (batch stride R*C); out rows have ldo elements
// (batch stride C*ldo). BLOCKED: out is instead the panelled matrix with C
// rows, panels of `panel` rows and K capacity Rpad. 16-byte loads and stores.
template <typename TI, typename TO, bool BLOCKED>
__global__ __launch_bounds__(256) void k_transpose(const TI* __restrict__ in, TO* __restrict__ out, int64_t R,
                                                   int64_t Rpad, int C, int64_t ldo, int64_t col0, int panel) {
  constexpr int KB = 128 / (int)sizeof(TO);
  constexpr int VI = 16 / (int)sizeof(TI), LI = 64 / VI, VO = 16 / (int)sizeof(TO), LO = 64 / VO;
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int64_t b = blockIdx.z;
  const TI* ib = in + b * R * C;
  TO* ob = out + b * (int64_t)C * ldo;
  for (int i = tid; i < 64 * LI; i += 256) {
    const int q = i / LI, c = (i % LI) * VI;
    const int64_t r = r0 + q;
#pragma unroll
    for (int v = 0; v < VI; v += 4) {
      const f32x4 x = r < R ? load4<TI>(ib + r * C + c0 + c + v) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < 4; ++u) tile[q][c + v + u] = x[u];
    }
  }
  __syncthreads();
  for (int i = tid; i < 64 * LO; i += 256) {
    const int c = i / LO, q = (i % LO) * VO;  // out row c0 + c, columns r0 + q ..
    TO* dst = BLOCKED ? out + panel_offset(c0 + c, r0 + q, panel, Rpad, KB) : ob + (int64_t)(c0 + c) * ldo + col0 + r0 + q;
#pragma unroll
    for (int v = 0; v < VO; v += 4)
      store4<TO>(dst + v, f32x4{tile[q + v][c], tile[q + v + 1][c], tile[q + v + 2][c], tile[q + v + 3][c]});
  }
}

// Rows of grouped activations into per-group zero-padded K segments of a
// panelled matrix with C rows (panels of `panel` rows, K capacity kcap):
// column koffs[e] + i holds row offsets[e] + i (through row_map when given)
// for i < count_e, zeros up to koffs[e+1]. A block owns one K stage of
// columns (kb = 128 bytes / element size) x 64 features, which lie in one
// panel: the group of each column is looked up once, rows are read as 64
// contiguous features and written as one contiguous 64 x kb block.
// With scale, the value of grouped row i is multiplied by scale[i].
template <typename TI, typename T>
__global__ __launch_bounds__(256) void k_transpose_groups(const TI* __restrict__ in, const int32_t* __restrict__ row_map,
                                                          const float* __restrict__ scale,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ koffs, int G, int C, int panel,
                                                          int64_t kcap, T* __restrict__ out) {
  constexpr int KB = 128 / (int)sizeof(T);
  __shared__ int64_t src[KB];
  __shared__ float sc[KB];
  __shared__ float tile[KB][65];
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * KB;
  const int c0 = blockIdx.y * 64;
  const int64_t qend = koffs[G];
  if (q0 >= qend) return;  // uniform across the block
  if (tid < KB) {
    const int64_t col = q0 + tid;
    int64_t sr = -1;
    float sv = 0.0f;
    if (col < qend) {
      int lo = 0, hi = G - 1;  // last group with koffs[e] <= col
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (koffs[mid] <= col) lo = mid; else hi = mid - 1;
      }
      const int64_t i = col - koffs[lo];
      if (i < offsets[lo + 1] - offsets[lo]) {
        sr = offsets[lo] + i;
        sv = scale ? scale[sr] : 1.0f;
        if (row_map) sr = row_map[sr];
      }
    }
    src[tid] = sr;
    sc[tid] = sv;
  }
  __syncthreads();
  // 16-byte loads: VI features each, 64 / VI per row
  constexpr int VI = 16 / (int)sizeof(TI), LI = 64 / VI;
  for (int i = tid; i < KB * LI; i += 256) {
    const int q = i / LI, c = (i % LI) * VI;
    const int64_t sr = src[q];
    if (sr >= 0) {
      const float a = sc[q];
#pragma unroll
      for (int v = 0; v < VI; v += 4) {
        const f32x4 x = load4<TI>(in + sr * C + c0 + c + v);
#pragma unroll
        for (int u = 0; u < 4; ++u) tile[q][c + v + u] = a * x[u];
      }
    } else {
#pragma unroll
      for (int v = 0; v < VI; ++v) tile[q][c + v] = 0.0f;
    }
  }
  __syncthreads();
  // 16-byte stores: VO columns each, KB / VO per row
  constexpr int VO = 16 / (int)sizeof(T), LO = KB / VO;
  T* ob = out + panel_offset(c0, q0, panel, kcap, KB);  // row c0 + c at ob + c * KB
  for (int i = tid; i < 64 * LO; i += 256) {
    const int c = i / LO, q = (i % LO) * VO;
#pragma unroll
    for (int v = 0; v < VO; v += 4)
      store4<T>(ob + c * KB + q + v, f32x4{tile[q + v][c], tile[q + v + 1][c], tile[q + v + 2][c], tile[q + v + 3][c]});
  }
}

// out[i] = sum over segments s, in order, of part[s * seg_stride + i]
__global__ __launch_bounds__(256) void k_sum_segments(const float* __restrict__ part, int nseg, int64_t seg_stride,
                                                      int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = 0.0f;
  for (int s = 0; s < nseg; ++s) acc += part[s * seg_stride + i];
  out[i] = acc;
}

// Exclusive prefix sum of x over the 1024 threads of a block (lane shuffles
// inside each wave, then the 16 wave totals); *total gets the sum. tmp: 16
// LDS slots.
__device__ int64_t block_scan_1024(int64_t x, int64_t* tmp, int64_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int64_t s = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(s, off);
    if (lane >= off) s += y;
  }
  if (lane == 63) tmp[w] = s;
  __syncthreads();
  if (w == 0) {
    int64_t t = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int64_t y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < 16) tmp[lane] = t;
  }
  __syncthreads();
  const int64_t before = w > 0 ? tmp[w - 1] : 0;
  *total = tmp[15];
  __syncthreads();  // tmp free for the next call
  return before + s - x;
}

constexpr int kKgMaxG = 2048;       // groups of a K-grouped launch, at most
constexpr int kKgMaxV = 4096;       // chunks (virtual groups) of a K-grouped launch, at most
constexpr int kKgMaxRaster = 4096;  // raster groups for the XCD balance (more: equal tile counts)
constexpr int kKgTileCost = 4;      // per-tile prologue and epilogue, in K stages

// K segments of the weight-gradient GEMMs, one block: koffs[e] = sum over
// groups before e of their row counts rounded up to kp (with no offsets: one
// segment of kp columns).
// Chunks: a group of s stages (ke K elements each) longer than cap stages
// (cap > 0) is cut into ceil(s / cap) chunks of near-equal stage counts, so
// that no tile (skewed routing, the shared expert's T rows) runs far longer
// than the average; vg[v] = (group, first K column, end K column, slot) per
// chunk, slot -1 for a group's first chunk (which writes the gradient
// itself) and a partial-buffer slot for the others; red[i] = (group, first
// slot, slot count) for every cut group, n_red[0] of them, for the ordered
// reduction that follows the GEMM. The tile list holds every (chunk, m-tile),
// empty groups included (their gradient is zero).
// A tile's work is its chunk's K stages plus kKgTileCost. With xb, the
// raster order (as the GEMM walks it: raster groups of kGroupM row tiles x
// ntn column tiles, row tile fastest) is cut into kXcd ranges of about equal
// work, at whole columns of a raster group.
__global__ __launch_bounds__(1024) void k_kg_setup(int G, const int32_t* __restrict__ offsets, int kp, int mt,
                                                   int32_t* __restrict__ koffs, int2* __restrict__ tiles,
                                                   int32_t* __restrict__ n_tiles, int ntn, int ke,
                                                   int32_t* __restrict__ xb, int cap, int4* __restrict__ vg,
                                                   int4* __restrict__ red, int32_t* __restrict__ n_red) {
  __shared__ int32_t ko[kKgMaxG + 1];
  __shared__ int32_t vst[kKgMaxV];          // K stages of each chunk
  __shared__ int64_t rc[kKgMaxRaster + 1];  // prefix work of the raster groups
  __shared__ int64_t tmp[16];
  __shared__ int32_t nv_s;
  const int tid = threadIdx.x;
  int64_t carry = 0;
  for (int e0 = 0; e0 < G; e0 += 1024) {  // uniform loop
    const int e = e0 + tid;
    const int64_t v = e < G ? (offsets ? (int64_t)(offsets[e + 1] - offsets[e] + kp - 1) / kp * kp : kp) : 0;
    int64_t tot;
    const int64_t ex = block_scan_1024(v, tmp, &tot);
    if (e < G) {
      ko[e] = (int32_t)(carry + ex);
      koffs[e] = (int32_t)(carry + ex);
    }
    carry += tot;
  }
  if (tid == 0) {
    ko[G] = (int32_t)carry;
    koffs[G] = (int32_t)carry;
  }
  __syncthreads();
  // chunks of every group
  int64_t vcarry = 0, scarry = 0, rcarry = 0;
  for (int e0 = 0; e0 < G; e0 += 1024) {  // uniform loop
    const int e = e0 + tid;
    const int st = e < G ? (ko[e + 1] - ko[e]) / ke : 0;
    const int nch = e < G ? ((cap > 0 && st > cap) ? (st + cap - 1) / cap : 1) : 0;
    int64_t tv, ts, tr;
    const int64_t vb = vcarry + block_scan_1024(nch, tmp, &tv);
    const int64_t sb = scarry + block_scan_1024(nch > 1 ? nch - 1 : 0, tmp, &ts);
    const int64_t rb = rcarry + block_scan_1024(nch > 1 ? 1 : 0, tmp, &tr);
    if (e < G) {
      const int q = (st + nch - 1) / nch;  // stages per chunk
      for (int c = 0; c < nch; ++c) {
        const int s0 = c * q < st ? c * q : st, s1 = (c + 1) * q < st ? (c + 1) * q : st;
        const int64_t vi = vb + c;
        vg[vi] = make_int4(e, ko[e] + s0 * ke, ko[e] + s1 * ke, c == 0 ? -1 : (int)(sb + c - 1));
        if (vi < kKgMaxV) vst[vi] = s1 - s0;
      }
      if (nch > 1) red[rb] = make_int4(e, (int)sb, nch - 1, 0);
    }
    vcarry += tv;
    scarry += ts;
    rcarry += tr;
  }
  if (tid == 0) {
    nv_s = (int32_t)vcarry;
    n_red[0] = (int32_t)rcarry;
    n_tiles[0] = (int32_t)vcarry * mt;
  }
  __syncthreads();
  const int nv = nv_s;
  for (int i = tid; i < nv * mt; i += 1024) tiles[i] = make_int2(i / mt, i % mt);
  if (!xb) return;  // uniform
  const int64_t m_tiles = (int64_t)nv * mt, total = m_tiles * ntn;
  const int64_t nrg = (m_tiles + kGroupM - 1) / kGroupM;
  if (nrg > kKgMaxRaster || nv > kKgMaxV) {  // uniform: equal tile counts
    const int64_t c = (total + kXcd - 1) / kXcd;
    if (tid <= kXcd) xb[tid] = (int32_t)(c * tid < total ? c * tid : total);
    return;
  }
  // work of one column of raster group r (its row tiles), per thread
  auto col_work = [&](int64_t r) {
    int64_t w = 0;
    const int64_t m1 = (r + 1) * kGroupM < m_tiles ? (r + 1) * kGroupM : m_tiles;
    for (int64_t m = r * kGroupM; m < m1; ++m) w += vst[m / mt] + kKgTileCost;
    return w;
  };
  // prefix sums: each thread a contiguous run of raster groups, then the runs
  const int per = (int)((nrg + 1023) / 1024);
  int64_t acc = 0;
  for (int j = 0; j < per; ++j) {
    const int64_t r = (int64_t)tid * per + j;
    if (r < nrg) acc += col_work(r) * ntn;
  }
  {
    int64_t tot;
    int64_t run = block_scan_1024(acc, tmp, &tot);
    for (int j = 0; j < per; ++j) {
      const int64_t r = (int64_t)tid * per + j;
      if (r < nrg) {
        rc[r] = run;
        run += col_work(r) * ntn;
      }
    }
    if (tid == 1023) rc[nrg] = run;
  }
  __syncthreads();
  if (tid <= kXcd) {
    const int64_t all = rc[nrg];
    int64_t L;
    if (tid == 0) L = 0;
    else if (tid == kXcd || all == 0) L = tid == kXcd ? total : total * tid / kXcd;
    else {
      const int64_t target = all * tid / kXcd;
      int64_t lo = 0, hi = nrg - 1;  // last raster group starting at or before target
      while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (rc[mid] <= target) lo = mid; else hi = mid - 1;
      }
      const int64_t cw = col_work(lo);
      int64_t cols = cw > 0 ? (target - rc[lo] + cw / 2) / cw : 0;
      cols = cols > ntn ? ntn : cols;
      const int64_t gm = (lo + 1) * kGroupM < m_tiles ? kGroupM : m_tiles - lo * kGroupM;
      L = lo * (int64_t)kGroupM * ntn + cols * gm;
    }
    xb[tid] = (int32_t)L;
  }
}

// After a chunked K-grouped GEMM: the gradient of every cut group gets its
// partial sums added, in slot order, to what its first chunk wrote. One
// thread per 4 columns of one row; blockIdx.y picks the cut group.
__global__ __launch_bounds__(256) void k_kg_reduce(GemmLaunch g, const int4* __restrict__ red,
                                                   const int32_t* __restrict__ n_red) {
  // blocks of row y of the grid stride over the 4-column pieces of cut
  // groups y, y + gridDim.y, ... (the grid is sized by the pieces of one
  // group and a few groups at a time, not by the bound on cut groups)
  const int nr = n_red[0];
  const int64_t n4 = (int64_t)g.m_valid * g.N / 4;
  for (int ri = blockIdx.y; ri < nr; ri += gridDim.y) {
    const int4 r = red[ri];
    for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n4; p += (int64_t)gridDim.x * 256) {
      const int64_t i = p * 4;
      const int mm = (int)(i / g.N), col = (int)(i % g.N);
      float* dst = kg_out_row(g, r.x, mm) + col;
      f32x4 acc = *reinterpret_cast<const f32x4*>(dst);
      for (int q = 0; q < r.z; ++q)
        acc += *reinterpret_cast<const f32x4*>(g.part + ((size_t)(r.y + q) * g.m_rows + mm) * g.N + col);
      *reinterpret_cast<f32x4*>(dst) = acc;
    }
  }
}

// Router logit gradients in fp32, one wave per token and a lane per expert
// (experts lane + 64 q): from the combine-weight gradients through the
// forward's weight rule, plus the z-loss (2 lse softmax / T) and aux-loss
// (E/T f_e dscore_e) terms with the caller's coefficients; written to
// dl [T, ep] (zero past E). Sums over experts are wave reductions in a fixed
// shuffle order, sums over slots run in slot order, so the result is the
// same bits on every call.
template <int QN>
__global__ __launch_bounds__(256) void k_router_bwd(int64_t T, int E, int ep, int k, const float* __restrict__ logits,
                                                    const int32_t* __restrict__ idx, const float* __restrict__ dtw,
                                                    const int32_t* __restrict__ counts, int score, int renorm,
                                                    float z_coef, float aux_coef, float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* l = logits + t * E;
  const int32_t* id = idx + t * k;
  const float* g = dtw + t * k;
  auto wave_sum = [](float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
  };
  float v[QN], o[QN];
  float m = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? l[e] : -__builtin_inff();
    m = v[q] > m ? v[q] : m;
    o[q] = 0.0f;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(m, off, 64);
    m = y > m ? y : m;
  }
  float p[QN];  // softmax over all experts
  float zl = 0.0f;
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    p[q] = lane + 64 * q < E ? expf(v[q] - m) : 0.0f;
    zl += p[q];
  }
  const float z = wave_sum(zl);
  const float lse = m + logf(z);
#pragma unroll
  for (int q = 0; q < QN; ++q) p[q] = p[q] / z;
  // add `term` to the logit gradient of expert e (its owner lane)
  auto add_to = [&](int e, float term) {
#pragma unroll
    for (int q = 0; q < QN; ++q)
      if (e == lane + 64 * q) o[q] += term;
  };
  if (score == 0 && renorm) {
    float mk = l[id[0]];
    for (int j = 1; j < k; ++j) mk = l[id[j]] > mk ? l[id[j]] : mk;
    float zk = 0.0f, dot = 0.0f;
    for (int j = 0; j < k; ++j) zk += expf(l[id[j]] - mk);
    for (int j = 0; j < k; ++j) dot += expf(l[id[j]] - mk) / zk * g[j];
    for (int j = 0; j < k; ++j) add_to(id[j], expf(l[id[j]] - mk) / zk * (g[j] - dot));
  } else if (score == 0) {
    float dot = 0.0f;
    for (int j = 0; j < k; ++j) dot += expf(l[id[j]] - m) / z * g[j];
#pragma unroll
    for (int q = 0; q < QN; ++q) o[q] -= p[q] * dot;
    for (int j = 0; j < k; ++j) add_to(id[j], expf(l[id[j]] - m) / z * g[j]);
  } else if (renorm) {
    float S = 0.0f, dot = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float sj = 1.0f / (1.0f + expf(-l[id[j]]));
      S += sj;
      dot += g[j] * sj;
    }
    const float D = S + 1e-9f;
    for (int j = 0; j < k; ++j) {
      const float sj = 1.0f / (1.0f + expf(-l[id[j]]));
      add_to(id[j], (g[j] / D - dot / (D * D)) * sj * (1.0f - sj));
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const float sj = 1.0f / (1.0f + expf(-l[id[j]]));
      add_to(id[j], g[j] * sj * (1.0f - sj));
    }
  }
  if (z_coef != 0.0f) {
#pragma unroll
    for (int q = 0; q < QN; ++q) o[q] += z_coef * 2.0f * lse * p[q] / (float)T;
  }
  if (aux_coef != 0.0f) {
    const float scale = aux_coef * (float)E / (float)T;
    float fl = 0.0f;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int e = lane + 64 * q;
      if (score == 0 && e < E) fl += (float)counts[e] / (float)T * p[q];
    }
    const float fp = score == 0 ? wave_sum(fl) : 0.0f;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int e = lane + 64 * q;
      if (e >= E) continue;
      const float f = (float)counts[e] / (float)T;
      if (score == 1) {
        const float sv = 1.0f / (1.0f + expf(-v[q]));
        o[q] += scale * f * sv * (1.0f - sv);
      } else {
        o[q] += scale * p[q] * (f - fp);
      }
    }
  }
  float* orow = dl + t * ep;
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int e = lane + 64 * q;
    if (e < ep) orow[e] = e < E ? o[q] : 0.0f;
  }
}

}  // namespace

hipError_t launch_to_bf16(int64_t n, const float* in, uint16_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_to_bf16, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, n / 4, in, out);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, int64_t T, int k, int f, const float* dhu, const float* g, const float* u,
                             const void* h, const float* w, const int32_t* row_of, bool shared, void* dgu, float* dtw,
                             float* wrow, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (f % 4) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(k_swiglu_bwd<uint16_t>, dim3((unsigned)T), dim3(256), 0, s, T, k, f, dhu, g, u,
                       (const uint16_t*)h, w, row_of, (int)shared, (uint16_t*)dgu, dtw, wrow);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<float>, dim3((unsigned)T), dim3(256), 0, s, T, k, f, dhu, g, u, (const float*)h,
                       w, row_of, (int)shared, (float*)dgu, dtw, wrow);
  return hipGetLastError();
}

hipError_t launch_gather_bwd(int64_t T, int d, int k, const float* dxp, const int32_t* row_of, bool shared,
                             const float* dxr, const float* dl, int ep, int E, const float* w_router, float* dx,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)((T * (d / 4) + 255) / 256));
  if (dl)
    hipLaunchKernelGGL(k_gather_bwd<true>, grid, dim3(256), 0, s, T, d, k, dxp, row_of, (int)shared, dxr, dl, ep, E,
                       w_router, dx);
  else
    hipLaunchKernelGGL(k_gather_bwd<false>, grid, dim3(256), 0, s, T, d, k, dxp, row_of, (int)shared, dxr, dl, ep,
                       E, w_router, dx);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype_in, int dtype_out, const void* in, void* out, int64_t batch, int64_t R,
                            int64_t Rpad, int C, int64_t ldo, int64_t col0, hipStream_t s, int panel) {
  if (batch <= 0 || Rpad <= 0 || C <= 0) return hipSuccess;
  const bool blocked = panel > 0;
  const int kb = dtype_out == 1 ? 64 : 32;
  if (blocked && (batch != 1 || C % panel || Rpad % kb)) return hipErrorInvalidValue;
  if (C % 64 || Rpad % 64 || Rpad < R || (!blocked && (ldo % 8 || col0 % 8 || col0 + Rpad > ldo)))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(Rpad / 64), (unsigned)(C / 64), (unsigned)batch);
#define MOE_TRANSPOSE(TI, TO)                                                                                        \
  do {                                                                                                               \
    if (blocked)                                                                                                     \
      hipLaunchKernelGGL((k_transpose<TI, TO, true>), grid, dim3(256), 0, s, (const TI*)in, (TO*)out, R, Rpad, C,    \
                         ldo, col0, panel);                                                                                 \
    else                                                                                                             \
      hipLaunchKernelGGL((k_transpose<TI, TO, false>), grid, dim3(256), 0, s, (const TI*)in, (TO*)out, R, Rpad, C,   \
                         ldo, col0, panel);                                                                                 \
  } while (0)
  if (dtype_in == 1 && dtype_out == 1)
    MOE_TRANSPOSE(uint16_t, uint16_t);
  else if (dtype_in == 1)
    MOE_TRANSPOSE(uint16_t, float);
  else if (dtype_out == 1)
    MOE_TRANSPOSE(float, uint16_t);
  else
    MOE_TRANSPOSE(float, float);
#undef MOE_TRANSPOSE
  return hipGetLastError();
}

hipError_t launch_transpose_groups(int dtype_in, int dtype, const void* in, const int32_t* row_map,
                                   const float* scale, const int32_t* offsets, const int32_t* koffs, int G, int C,
                                   int panel, int64_t max_cols, void* out, hipStream_t s) {
  if (max_cols <= 0 || C <= 0) return hipSuccess;
  const int kb = dtype == 1 ? 64 : 32;
  if (panel <= 0 || panel % 64 || C % panel || max_cols % kb || C % 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((max_cols + kb - 1) / kb), (unsigned)((C + 63) / 64));
  if (dtype == 1 && dtype_in == 1)
    hipLaunchKernelGGL((k_transpose_groups<uint16_t, uint16_t>), grid, dim3(256), 0, s, (const uint16_t*)in, row_map,
                       scale, offsets, koffs, G, C, panel, max_cols, (uint16_t*)out);
  else if (dtype == 1)
    hipLaunchKernelGGL((k_transpose_groups<float, uint16_t>), grid, dim3(256), 0, s, (const float*)in, row_map,
                       scale, offsets, koffs, G, C, panel, max_cols, (uint16_t*)out);
  else if (dtype_in == 0)
    hipLaunchKernelGGL((k_transpose_groups<float, float>), grid, dim3(256), 0, s, (const float*)in, row_map, scale,
                       offsets, koffs, G, C, panel, max_cols, (float*)out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_sum_segments(const float* part, int nseg, int64_t seg_stride, int64_t n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sum_segments, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, nseg, seg_stride, n,
                     out);
  return hipGetLastError();
}

hipError_t launch_kg_setup(int G, const int32_t* offsets, int kp, int mt, int32_t* koffs, int2* tiles,
                           int32_t* n_tiles, int4* vgroups, int cap, int4* red, int32_t* n_red, hipStream_t s, int ntn,
                           int ke, int32_t* xcd_bounds) {
  if (G < 1 || G > kKgMaxG || mt < 1 || ke < 1 || !vgroups || !red || !n_red) return hipErrorInvalidValue;
  if (xcd_bounds && ntn < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kg_setup, dim3(1), dim3(1024), 0, s, G, offsets, kp, mt, koffs, tiles, n_tiles, ntn, ke,
                     xcd_bounds, cap, vgroups, red, n_red);
  return hipGetLastError();
}

hipError_t launch_kg_reduce(const GemmLaunch& g, const int4* red, const int32_t* n_red, int max_red, hipStream_t s) {
  if (max_red <= 0 || g.m_valid <= 0 || g.N % 4) return hipSuccess;
  const int64_t n4 = (int64_t)g.m_valid * g.N / 4;
  const int gy = max_red < 16 ? max_red : 16;
  const int64_t cap = (int64_t)cu_count() * 32 / gy;  // blocks per group row: enough to stream its pieces
  const int64_t blocks = (n4 + 255) / 256 < cap ? (n4 + 255) / 256 : (cap > 0 ? cap : 1);
  hipLaunchKernelGGL(k_kg_reduce, dim3((unsigned)blocks, (unsigned)gy), dim3(256), 0, s, g, red, n_red);
  return hipGetLastError();
}

hipError_t launch_router_bwd(int64_t T, int E, int ep, int k, const float* logits, const int32_t* idx,
                             const float* dtw, const int32_t* counts, int score, int renorm, float z_coef,
                             float aux_coef, float* dl, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E < 1 || ep < E || ep > 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + 3) / 4));
#define ROUTER_BWD(QN_)                                                                                            \
  hipLaunchKernelGGL(k_router_bwd<QN_>, grid, dim3(256), 0, s, T, E, ep, k, logits, idx, dtw, counts, score, renorm, \
                     z_coef, aux_coef, dl)
  if (ep <= 64) ROUTER_BWD(1);
  else if (ep <= 128) ROUTER_BWD(2);
  else if (ep <= 256) ROUTER_BWD(4);
  else if (ep <= 512) ROUTER_BWD(8);
  else ROUTER_BWD(16);
#undef ROUTER_BWD
  return hipGetLastError();
}

}  // namespace moe
