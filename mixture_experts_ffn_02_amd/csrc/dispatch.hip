// Dispatch into expert-contiguous order: per-expert counts, exclusive scan,
// per-block bases, the grouped-GEMM tile list, and the row scatter.
//
// Tokens per expert are the column sums of the per-block histograms that the
// router (or k_hist_rank) wrote ("SigmoidRouter": one-hot counts summed over
// tokens, moe-200m-qwen3-100b README). Rows of one expert are ordered by
// token id: row_of[t, j] = offsets[e] + (tokens before t's block that chose e)
// + (tokens before t inside its block that chose e). Everything here is
// integer arithmetic without atomics, so the order is reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;

// Exclusive prefix sum over v[0..n) in LDS (n <= kScanThreads): an inclusive
// scan inside each wave with lane shuffles, then the scan of the wave totals
// by wave 0; tmp holds at least kScanThreads / 64 ints. Returns the total.
__device__ int block_exclusive_scan(int* v, int* tmp, int n) {
  constexpr int kWaves = kScanThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int x = tid < n ? v[tid] : 0;
  int s = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(s, off);
    if (lane >= off) s += y;
  }
  if (lane == 63) tmp[w] = s;
  __syncthreads();
  if (w == 0) {
    int t = lane < kWaves ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < kWaves) tmp[lane] = t;
  }
  __syncthreads();
  const int before = w > 0 ? tmp[w - 1] : 0;
  const int total = tmp[kWaves - 1];
  if (tid < n) v[tid] = before + s - x;
  __syncthreads();
  return total;
}

// counts[e] = sum over blocks of hist[b, e]: one block; thread (g, e) sums
// rows g, g + R, ... of column e (R = 1024 / E rounded to a power of two),
// so that the loads of many rows are in flight at once.
__global__ __launch_bounds__(kScanThreads) void k_counts(const int32_t* __restrict__ hist, int nb, int E,
                                                         int32_t* __restrict__ counts) {
  __shared__ int part[kScanThreads];
  const int tid = threadIdx.x;
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int R = kScanThreads / ep;
  const int g = tid / ep, e = tid % ep;
  int c = 0;
  if (e < E)
    for (int b = g; b < nb; b += R) c += hist[(size_t)b * E + e];
  part[tid] = c;
  __syncthreads();
  if (tid < E) {
    int t = 0;
    for (int gg = 0; gg < R; ++gg) t += part[gg * ep + tid];
    counts[tid] = t;
  }
}

// One block. Thread (g, e) owns expert e over block range g. `extra` > 0
// appends one more group of that many rows after the E experts (offsets then
// has E + 2 entries and the tile list ends with its tiles).
__global__ __launch_bounds__(kScanThreads) void k_scan(const int32_t* __restrict__ hist, int nb, int E,
                                                       int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ base, int bm,
                                                       int32_t* __restrict__ n_tiles, int2* __restrict__ tiles,
                                                       int extra) {
  __shared__ int part[kScanThreads];
  __shared__ int cnt[kScanThreads];
  __shared__ int toff[kScanThreads];
  __shared__ int tmp[kScanThreads / 64];
  const int tid = threadIdx.x;
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int R = kScanThreads / ep;
  const int g = tid / ep, e = tid % ep;
  const int chunk = (nb + R - 1) / R;
  const int b0 = g * chunk, b1 = min(nb, b0 + chunk);
  int s = 0;
  if (e < E) {
    // the loads of a thread's blocks are independent: batch them (16, then 8)
    int b = b0;
    for (; b + 16 <= b1; b += 16) {
      int v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = hist[(size_t)(b + q) * E + e];
#pragma unroll
      for (int q = 0; q < 16; ++q) s += v[q];
    }
    for (; b + 8 <= b1; b += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = hist[(size_t)(b + q) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) s += v[q];
    }
    for (; b < b1; ++b) s += hist[(size_t)b * E + e];
  }
  part[tid] = s;
  __syncthreads();
  // per expert: inclusive prefix over the block ranges, log2(R) steps
  for (int off = 1; off < R; off <<= 1) {
    const int y = g >= off ? part[tid - off * ep] : 0;
    __syncthreads();
    part[tid] += y;
    __syncthreads();
  }
  if (g == R - 1 && e < E) cnt[e] = part[tid];
  __syncthreads();
  if (tid < E) {
    counts[tid] = cnt[tid];
    toff[tid] = (cnt[tid] + bm - 1) / bm;
  }
  __syncthreads();
  const int total = block_exclusive_scan(cnt, tmp, E);  // cnt -> offsets
  const int total_tiles = block_exclusive_scan(toff, tmp, E);
  const int extra_tiles = (extra + bm - 1) / bm;
  if (tid < E) offsets[tid] = cnt[tid];
  if (tid == 0) {
    offsets[E] = total;
    if (extra > 0) offsets[E + 1] = total + extra;
    n_tiles[0] = total_tiles + extra_tiles;
  }
  if (e < E) {
    int run = cnt[e] + part[tid] - s;  // rows of expert e before block b0
    int b = b0;
    for (; b + 16 <= b1; b += 16) {
      int v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) v[q] = hist[(size_t)(b + q) * E + e];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        base[(size_t)(b + q) * E + e] = run;
        run += v[q];
      }
    }
    for (; b + 8 <= b1; b += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = hist[(size_t)(b + q) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        base[(size_t)(b + q) * E + e] = run;
        run += v[q];
      }
    }
    for (; b < b1; ++b) {
      base[(size_t)b * E + e] = run;
      run += hist[(size_t)b * E + e];
    }
  }
  if (tid < E) {
    const int nt = (tid + 1 < E ? toff[tid + 1] : total_tiles) - toff[tid];
    for (int i = 0; i < nt; ++i) tiles[toff[tid] + i] = make_int2(tid, i);
  }
  for (int i = tid; i < extra_tiles; i += kScanThreads) tiles[total_tiles + i] = make_int2(E, i);
}

__global__ __launch_bounds__(kScanThreads) void k_tiles_from_offsets(const int32_t* __restrict__ offsets, int G,
                                                                     int bm, int32_t* __restrict__ n_tiles,
                                                                     int2* __restrict__ tiles) {
  __shared__ int toff[kScanThreads];
  __shared__ int tmp[kScanThreads / 64];
  const int tid = threadIdx.x;
  // groups are processed in slices of kScanThreads
  int carry = 0;
  for (int g0 = 0; g0 < G; g0 += kScanThreads) {
    const int n = min(kScanThreads, G - g0);
    const int gid = g0 + tid;
    int nt = 0;
    if (tid < n) {
      const int rows = offsets[gid + 1] - offsets[gid];
      nt = rows > 0 ? (rows + bm - 1) / bm : 0;
      toff[tid] = nt;
    }
    __syncthreads();
    const int tot = block_exclusive_scan(toff, tmp, n);
    if (tid < n)
      for (int i = 0; i < nt; ++i) tiles[carry + toff[tid] + i] = make_int2(gid, i);
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) n_tiles[0] = carry;
}

// One wave per token: rows of its k slots, the inverse map, and optionally
// the copy of x[t] into its k rows of x_perm. The row is read from HBM once,
// into registers (16 KB of it per pass, 16 bytes per lane per load, all in
// flight together), and each pass is then stored to the k rows with
// non-temporal stores (x_perm is written once and not read back here).
// Measured against a loop that re-read the row for every slot: 3.5 -> 5.2
// TB/s at the DeepSeek-style layer (2.43 -> 1.61 ms), 3.4 -> 4.9 TB/s at the
// Qwen3-like one; the non-temporal stores give 5-14% of that over plain ones.
constexpr int kPermPass = 16;  // 16-byte chunks per lane per pass
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, const int32_t* __restrict__ rank,
                                                 const int32_t* __restrict__ base, int64_t T, int k, int E, int tpb,
                                                 int32_t* __restrict__ row_of, int32_t* __restrict__ tok_of_row,
                                                 const unsigned char* __restrict__ x, unsigned char* __restrict__ x_perm,
                                                 int row_bytes, int extra) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t n_rows = T * k;
  if (extra && lane == 63) tok_of_row[n_rows + t] = (int32_t)t;  // the extra group: every token once
  int my_row = -1;
  if (lane < k) {
    const int e = idx[t * k + lane];
    if (e >= 0 && e < E) my_row = base[(t / tpb) * E + e] + rank[t * k + lane];
    if (my_row >= n_rows) my_row = -1;  // only reachable with invalid ids; never write out of range
    row_of[t * k + lane] = my_row;
    if (my_row >= 0) tok_of_row[my_row] = (int32_t)t;
  }
  if (!x_perm) return;
  const int nchunk = row_bytes >> 4;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * row_bytes);
  for (int c0 = 0; c0 < nchunk; c0 += 64 * kPermPass) {
    u32x4 v[kPermPass];
#pragma unroll
    for (int i = 0; i < kPermPass; ++i) {
      const int c = c0 + 64 * i + lane;
      if (c < nchunk) v[i] = src[c];
    }
    for (int j = 0; j < k; ++j) {
      const int r = __shfl(my_row, j);  // every lane of the wave is active here
      if (r < 0) continue;
      u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (size_t)r * row_bytes);
#pragma unroll
      for (int i = 0; i < kPermPass; ++i) {
        const int c = c0 + 64 * i + lane;
        if (c < nchunk) __builtin_nontemporal_store(v[i], dst + c);
      }
    }
  }
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_counts(const int32_t* hist, int nb, int E, int32_t* counts, hipStream_t s) {
  if (E > kScanThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_counts, dim3(1), dim3(kScanThreads), 0, s, hist, nb, E, counts);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* hist, int nb, int E, int32_t* counts, int32_t* offsets, int32_t* base, int bm,
                       int32_t* n_tiles, int2* tiles, hipStream_t s, int64_t extra) {
  if (E > kScanThreads || extra < 0 || extra > 0x3FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, hist, nb, E, counts, offsets, base, bm, n_tiles,
                     tiles, (int)extra);
  return hipGetLastError();
}

hipError_t launch_tiles_from_offsets(const int32_t* offsets, int G, int bm, int32_t* n_tiles, int2* tiles,
                                     hipStream_t s) {
  hipLaunchKernelGGL(k_tiles_from_offsets, dim3(1), dim3(kScanThreads), 0, s, offsets, G, bm, n_tiles, tiles);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, const int32_t* rank, const int32_t* base, int64_t T, int k, int E,
                          int tokens_per_block, int32_t* row_of, int32_t* tok_of_row, const void* x, void* x_perm,
                          int row_bytes, hipStream_t s, bool extra) {
  if (T <= 0) return hipSuccess;
  const int64_t nb = (T + 3) / 4;
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)nb), dim3(256), 0, s, idx, rank, base, T, k, E, tokens_per_block,
                     row_of, tok_of_row, (const unsigned char*)x, (unsigned char*)x_perm, row_bytes, (int)extra);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace moe
