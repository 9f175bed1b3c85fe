// Weighted combine back to token order (moe-200m-qwen3-100b README,
// "Architecture diagram": routed experts and the always-on shared expert feed
// one weighted sum).
//   y[t] = sum_{j<k} w[t,j] * Y[row_of[t,j]]  (+ S[t], weight 1, added last)
// A gather: one wave per token reads its k expert rows and writes its output
// row in fp32, slots in order, each lane keeping a group of up to eight row
// loads in flight (with more than eight slots the row is written after each
// group and read back for the next, which leaves every sum unchanged). The
// token's row ids and weights are wave-uniform. No atomics, so the result is
// the same bits on every run. When the tokens are too few to give every CU work, the
// row is also split into column ranges over grid.y (each element's sum is
// unchanged).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <int KG>
__global__ __launch_bounds__(256) void k_combine(int64_t T, int d, int k, const float* __restrict__ y_perm,
                                                 const int32_t* __restrict__ row_of, const float* __restrict__ w,
                                                 const float* __restrict__ y_shared, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  // the token is wave-uniform: its row ids and weights are read with scalar
  // loads, and every slot test below is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int n4 = d >> 2;
  const int span = (n4 + gridDim.y - 1) / gridDim.y;  // float4 columns of this block
  const int c0 = blockIdx.y * span, c1 = c0 + span < n4 ? c0 + span : n4;
  const int64_t n_rows = T * k;
  const f32x4* Y = reinterpret_cast<const f32x4*>(y_perm);
  for (int j0 = 0; j0 < k; j0 += KG) {
    // slots j0 .. j0 + KG - 1: base of each row (a slot past k or an invalid
    // row id reads row 0 and contributes nothing)
    const f32x4* src[KG];
    float wj[KG];
    bool use[KG];
#pragma unroll
    for (int q = 0; q < KG; ++q) {
      const int j = j0 + q < k ? j0 + q : k - 1;  // every load in range
      const int r = __builtin_amdgcn_readfirstlane(row_of[t * k + j]);
      use[q] = j0 + q < k && r >= 0 && r < n_rows;
      wj[q] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, w[t * k + j])));
      src[q] = Y + (size_t)(use[q] ? r : 0) * n4;
    }
    for (int c = c0 + lane; c < c1; c += 64) {
      float* out = y + ((size_t)t * n4 + c) * 4;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j0 > 0) acc = *reinterpret_cast<const f32x4*>(out);  // the earlier slot groups' sum
      f32x4 v[KG];
#pragma unroll
      for (int q = 0; q < KG; ++q) v[q] = __builtin_nontemporal_load(src[q] + c);  // read once: streaming
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        if (!use[q]) continue;  // invalid row ids contribute nothing
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wj[q], v[q][e], acc[e]);
      }
      if (y_shared && j0 + KG >= k) {
        const f32x4 sv = reinterpret_cast<const f32x4*>(y_shared)[(size_t)t * n4 + c];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += sv[q];
      }
      *reinterpret_cast<f32x4*>(out) = acc;
    }
  }
}

}  // namespace

hipError_t launch_combine(int64_t T, int d, int k, const float* y_perm, const int32_t* row_of, const float* w,
                          const float* y_shared, float* y, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (k > 32 || (d & 3)) return hipErrorInvalidValue;
  // column ranges of at least 64 float4 (one per lane), enough of them for
  // about two blocks per CU
  const int64_t bx = (T + 3) / 4;
  const int64_t want = (2 * (int64_t)cu_count() + bx - 1) / bx;
  const int64_t most = ((d >> 2) + 63) / 64;
  const unsigned by = (unsigned)(want < most ? want : most);
  const dim3 grid((unsigned)bx, by > 0 ? by : 1u);
  // slot groups of 1, 2, 4 or 8 loads in flight per lane
  if (k >= 8)
    hipLaunchKernelGGL(k_combine<8>, grid, dim3(256), 0, s, T, d, k, y_perm, row_of, w, y_shared, y);
  else if (k >= 4)
    hipLaunchKernelGGL(k_combine<4>, grid, dim3(256), 0, s, T, d, k, y_perm, row_of, w, y_shared, y);
  else if (k >= 2)
    hipLaunchKernelGGL(k_combine<2>, grid, dim3(256), 0, s, T, d, k, y_perm, row_of, w, y_shared, y);
  else
    hipLaunchKernelGGL(k_combine<1>, grid, dim3(256), 0, s, T, d, k, y_perm, row_of, w, y_shared, y);
  return hipGetLastError();
}

}  // namespace moe
