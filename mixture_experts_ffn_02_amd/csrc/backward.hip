// Backward pass of the MoE FFN layer: the element-wise and data-movement
// kernels around the grouped GEMMs (which gemm.hip runs).
//
// The layer's forward (moe-200m-qwen3-100b README, "Architecture diagram" and
// "SigmoidRouter"; SpecForge PR #930, "What this adds") is
//   y_t = sum_j w_tj E_{e_tj}(x_t) (+ S(x_t)),  E(x) = W_down (silu(W_gate x) * W_up x),
// with w from the unbiased scores of the chosen experts. Given dy, the
// backward runs
//   combine^T : d_w[t,j] = <dy_t, Y[row]>, dY[row] = w[t,j] dy_t (shared row: dy_t)
//   down^T    : dH = dY W_down           (grouped GEMM)
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

// One wave per token: for each slot, d_w = <dy_t, Y[row]> (lanes over
// features, then a fixed xor-shuffle tree) and dY[row] = w dy_t in the
// operand type; with a shared expert, dY[T*k + t] = dy_t.
template <typename DT>
__global__ __launch_bounds__(256) void k_combine_bwd(int64_t T, int d, int k, const float* __restrict__ dy,
                                                     const float* __restrict__ yperm, const int32_t* __restrict__ row_of,
                                                     const float* __restrict__ w, float* __restrict__ dtw,
                                                     DT* __restrict__ dyp, int shared) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* dyt = dy + t * d;
  for (int j = 0; j < k; ++j) {
    const int64_t r = row_of[t * k + j];
    const float wt = w[t * k + j];
    float s = 0.0f;
    for (int c = lane * 4; c < d; c += 256) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(dyt + c);
      const f32x4 b = *reinterpret_cast<const f32x4*>(yperm + r * d + c);
      s = __builtin_fmaf(a[0], b[0], s);
      s = __builtin_fmaf(a[1], b[1], s);
      s = __builtin_fmaf(a[2], b[2], s);
      s = __builtin_fmaf(a[3], b[3], s);
#pragma unroll
      for (int q = 0; q < 4; ++q) dyp[r * d + c + q] = from_f32<DT>(wt * a[q]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0 && dtw) dtw[t * k + j] = s;
  }
  if (shared) {
    const int64_t r = T * k + t;
    for (int c = lane; c < d; c += 64) dyp[r * d + c] = from_f32<DT>(dyt[c]);
  }
}

// dG = dH u s (1 + g (1 - s)), dU = dH g s with s = sigmoid(g), stored side
// by side: dgu[r] = [dG_r | dU_r] (2 f values).
template <typename DT>
__global__ __launch_bounds__(256) void k_swiglu_bwd(int64_t rows, int f, const float* __restrict__ dh,
                                                    const float* __restrict__ gp, const float* __restrict__ up,
                                                    DT* __restrict__ dgu) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * f) return;
  const int64_t r = i / f;
  const int c = (int)(i % f);
  const float g = gp[i], u = up[i], h = dh[i];
  const float s = 1.0f / (1.0f + __expf(-g));
  dgu[r * 2 * f + c] = from_f32<DT>(h * u * s * (1.0f + g * (1.0f - s)));
  dgu[r * 2 * f + f + c] = from_f32<DT>(h * g * s);
}

// dx_t = sum_j dXp[row_of[t, j]] (slots in order) (+ dXp[T*k + t], the
// shared expert) (+ dxr_t, the router term).
__global__ __launch_bounds__(256) void k_gather_bwd(int64_t T, int d, int k, const float* __restrict__ dxp,
                                                    const int32_t* __restrict__ row_of, int shared,
                                                    const float* __restrict__ dxr, float* __restrict__ dx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of dx
  const int nq = d / 4;
  if (i >= T * nq) return;
  const int64_t t = i / nq;
  const int c = (int)(i % nq) * 4;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < k; ++j) acc += *reinterpret_cast<const f32x4*>(dxp + (int64_t)row_of[t * k + j] * d + c);
  if (shared) acc += *reinterpret_cast<const f32x4*>(dxp + (T * k + t) * d + c);
  if (dxr) acc += *reinterpret_cast<const f32x4*>(dxr + t * d + c);
  *reinterpret_cast<f32x4*>(dx + t * d + c) = acc;
}

// Batched transpose through 32 x 32 LDS tiles:
//   out[b][c][col0 + r] = in[b][r][c] for r < R, c < C; 0 for R <= r < Rpad.
// in rows have C elements (batch stride R*C); out rows have ldo elements
// (batch stride C*ldo).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_transpose(const TI* __restrict__ in, TO* __restrict__ out, int64_t R,
                                                   int64_t Rpad, int C, int64_t ldo, int64_t col0) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int64_t r0 = (int64_t)blockIdx.x * 32;
  const int c0 = blockIdx.y * 32;
  const int64_t b = blockIdx.z;
  const TI* ib = in + b * R * C;
  TO* ob = out + b * (int64_t)C * ldo;
  for (int q = ty; q < 32; q += 8) {
    const int64_t r = r0 + q;
    const int c = c0 + tx;
    tile[q][tx] = (r < R && c < C) ? to_f32<TI>(ib[r * C + c]) : 0.0f;
  }
  __syncthreads();
  for (int q = ty; q < 32; q += 8) {
    const int c = c0 + q;
    const int64_t r = r0 + tx;
    if (c < C && r < Rpad) ob[(int64_t)c * ldo + col0 + r] = from_f32<TO>(tile[tx][q]);
  }
}

// Rows of grouped activations into per-group K segments of a transposed
// matrix: out[c][koffs[e] + i] = in[src(offsets[e] + i)][c] for i < count_e,
// 0 for count_e <= i < koffs[e+1] - koffs[e]; src is row_map[] when given.
// The grid covers columns 0 .. koffs[G] in blocks of 32.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_groups(const T* __restrict__ in, const int32_t* __restrict__ row_map,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ koffs, int G, int C,
                                                          int64_t ldo, T* __restrict__ out) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t q0 = (int64_t)blockIdx.x * 32;
  const int c0 = blockIdx.y * 32;
  const int64_t qend = koffs[G];
  if (q0 >= qend) return;  // uniform across the block
  for (int q = ty; q < 32; q += 8) {
    const int64_t col = q0 + q;
    float v = 0.0f;
    if (col < qend) {
      int lo = 0, hi = G - 1;  // group with koffs[e] <= col < koffs[e+1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (koffs[mid] <= col) lo = mid; else hi = mid - 1;
      }
      const int64_t i = col - koffs[lo];
      if (i < offsets[lo + 1] - offsets[lo]) {
        int64_t src = offsets[lo] + i;
        if (row_map) src = row_map[src];
        if (c0 + tx < C) v = to_f32<T>(in[src * C + c0 + tx]);
      }
    }
    tile[q][tx] = v;
  }
  __syncthreads();
  for (int q = ty; q < 32; q += 8) {
    const int64_t col = q0 + tx;
    if (col < qend && c0 + q < C) out[(int64_t)(c0 + q) * ldo + col] = from_f32<T>(tile[tx][q]);
  }
}

// K segments of the weight-gradient GEMMs, one block: koffs[e] = sum over
// groups before e of their row counts rounded up to kp (with no offsets: one
// segment of kp columns); the tile list holds every (group, m-tile), empty
// groups included (their gradient is zero).
__global__ __launch_bounds__(1024) void k_kg_setup(int G, const int32_t* __restrict__ offsets, int kp, int mt,
                                                   int32_t* __restrict__ koffs, int2* __restrict__ tiles,
                                                   int32_t* __restrict__ n_tiles) {
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < G; ++e) {
      koffs[e] = run;
      run += offsets ? (offsets[e + 1] - offsets[e] + kp - 1) / kp * kp : kp;
    }
    koffs[G] = run;
    n_tiles[0] = G * mt;
  }
  for (int i = threadIdx.x; i < G * mt; i += 1024) tiles[i] = make_int2(i / mt, i % mt);
}

// Router logit gradients, one thread per token, in fp32: from the
// combine-weight gradients through the forward's weight rule, plus the
// z-loss (2 lse softmax / T) and aux-loss (E/T f_e dscore_e) terms with the
// caller's coefficients; written to dl [T, ep] (zero past E).
__global__ __launch_bounds__(256) void k_router_bwd(int64_t T, int E, int ep, int k, const float* __restrict__ logits,
                                                    const int32_t* __restrict__ idx, const float* __restrict__ dtw,
                                                    const int32_t* __restrict__ counts, int score, int renorm,
                                                    float z_coef, float aux_coef, float* __restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* l = logits + t * E;
  float* o = dl + t * ep;
  const int32_t* id = idx + t * k;
  const float* g = dtw + t * k;
  float m = l[0];
  for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
  float z = 0.0f;
  for (int e = 0; e < E; ++e) z += expf(l[e] - m);
  const float lse = m + logf(z);
  for (int e = 0; e < ep; ++e) o[e] = 0.0f;
  if (score == 0 && renorm) {
    float mk = l[id[0]];
    for (int j = 1; j < k; ++j) mk = l[id[j]] > mk ? l[id[j]] : mk;
    float zk = 0.0f, dot = 0.0f;
    for (int j = 0; j < k; ++j) zk += expf(l[id[j]] - mk);
    for (int j = 0; j < k; ++j) dot += expf(l[id[j]] - mk) / zk * g[j];
    for (int j = 0; j < k; ++j) o[id[j]] += expf(l[id[j]] - mk) / zk * (g[j] - dot);
  } else if (score == 0) {
    float dot = 0.0f;
    for (int j = 0; j < k; ++j) dot += expf(l[id[j]] - m) / z * g[j];
    for (int e = 0; e < E; ++e) o[e] -= expf(l[e] - m) / z * dot;
    for (int j = 0; j < k; ++j) o[id[j]] += expf(l[id[j]] - m) / z * g[j];
  } else if (renorm) {
    float S = 0.0f, dot = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float s = 1.0f / (1.0f + expf(-l[id[j]]));
      S += s;
      dot += g[j] * s;
    }
    const float D = S + 1e-9f;
    for (int j = 0; j < k; ++j) {
      const float s = 1.0f / (1.0f + expf(-l[id[j]]));
      o[id[j]] += (g[j] / D - dot / (D * D)) * s * (1.0f - s);
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const float s = 1.0f / (1.0f + expf(-l[id[j]]));
      o[id[j]] += g[j] * s * (1.0f - s);
    }
  }
  if (z_coef != 0.0f)
    for (int e = 0; e < E; ++e) o[e] += z_coef * 2.0f * lse * expf(l[e] - m) / z / (float)T;
  if (aux_coef != 0.0f) {
    const float scale = aux_coef * (float)E / (float)T;
    float fp = 0.0f;
    if (score == 0)
      for (int e = 0; e < E; ++e) fp += (float)counts[e] / (float)T * expf(l[e] - m) / z;
    for (int e = 0; e < E; ++e) {
      const float f = (float)counts[e] / (float)T;
      if (score == 1) {
        const float s = 1.0f / (1.0f + expf(-l[e]));
        o[e] += scale * f * s * (1.0f - s);
      } else {
        o[e] += scale * expf(l[e] - m) / z * (f - fp);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine_bwd(int dtype, int64_t T, int d, int k, const float* dy, const float* yperm,
                              const int32_t* row_of, const float* w, float* dtw, void* dyp, bool shared,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4));
  if (dtype == 1)
    hipLaunchKernelGGL(k_combine_bwd<uint16_t>, grid, dim3(256), 0, s, T, d, k, dy, yperm, row_of, w, dtw,
                       (uint16_t*)dyp, (int)shared);
  else
    hipLaunchKernelGGL(k_combine_bwd<float>, grid, dim3(256), 0, s, T, d, k, dy, yperm, row_of, w, dtw, (float*)dyp,
                       (int)shared);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, int64_t rows, int f, const float* dh, const float* g, const float* u,
                             void* dgu, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows * f + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(k_swiglu_bwd<uint16_t>, grid, dim3(256), 0, s, rows, f, dh, g, u, (uint16_t*)dgu);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<float>, grid, dim3(256), 0, s, rows, f, dh, g, u, (float*)dgu);
  return hipGetLastError();
}

hipError_t launch_gather_bwd(int64_t T, int d, int k, const float* dxp, const int32_t* row_of, bool shared,
                             const float* dxr, float* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_bwd, dim3((unsigned)((T * (d / 4) + 255) / 256)), dim3(256), 0, s, T, d, k, dxp, row_of,
                     (int)shared, dxr, dx);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype_in, int dtype_out, const void* in, void* out, int64_t batch, int64_t R,
                            int64_t Rpad, int C, int64_t ldo, int64_t col0, hipStream_t s) {
  if (batch <= 0 || Rpad <= 0 || C <= 0) return hipSuccess;
  const dim3 grid((unsigned)((Rpad + 31) / 32), (unsigned)((C + 31) / 32), (unsigned)batch);
  if (dtype_in == 1 && dtype_out == 1)
    hipLaunchKernelGGL((k_transpose<uint16_t, uint16_t>), grid, dim3(256), 0, s, (const uint16_t*)in, (uint16_t*)out,
                       R, Rpad, C, ldo, col0);
  else if (dtype_in == 1)
    hipLaunchKernelGGL((k_transpose<uint16_t, float>), grid, dim3(256), 0, s, (const uint16_t*)in, (float*)out, R,
                       Rpad, C, ldo, col0);
  else if (dtype_out == 1)
    hipLaunchKernelGGL((k_transpose<float, uint16_t>), grid, dim3(256), 0, s, (const float*)in, (uint16_t*)out, R,
                       Rpad, C, ldo, col0);
  else
    hipLaunchKernelGGL((k_transpose<float, float>), grid, dim3(256), 0, s, (const float*)in, (float*)out, R, Rpad, C,
                       ldo, col0);
  return hipGetLastError();
}

hipError_t launch_transpose_groups(int dtype, const void* in, const int32_t* row_map, const int32_t* offsets,
                                   const int32_t* koffs, int G, int C, int64_t max_cols, int64_t ldo, void* out,
                                   hipStream_t s) {
  if (max_cols <= 0 || C <= 0) return hipSuccess;
  const dim3 grid((unsigned)((max_cols + 31) / 32), (unsigned)((C + 31) / 32));
  if (dtype == 1)
    hipLaunchKernelGGL(k_transpose_groups<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)in, row_map, offsets,
                       koffs, G, C, ldo, (uint16_t*)out);
  else
    hipLaunchKernelGGL(k_transpose_groups<float>, grid, dim3(256), 0, s, (const float*)in, row_map, offsets, koffs,
                       G, C, ldo, (float*)out);
  return hipGetLastError();
}

hipError_t launch_kg_setup(int G, const int32_t* offsets, int kp, int mt, int32_t* koffs, int2* tiles,
                           int32_t* n_tiles, hipStream_t s) {
  hipLaunchKernelGGL(k_kg_setup, dim3(1), dim3(1024), 0, s, G, offsets, kp, mt, koffs, tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_router_bwd(int64_t T, int E, int ep, int k, const float* logits, const int32_t* idx,
                             const float* dtw, const int32_t* counts, int score, int renorm, float z_coef,
                             float aux_coef, float* dl, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_bwd, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, T, E, ep, k, logits, idx, dtw,
                     counts, score, renorm, z_coef, aux_coef, dl);
  return hipGetLastError();
}

}  // namespace moe
