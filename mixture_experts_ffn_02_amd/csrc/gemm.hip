// Grouped GEMMs of the SwiGLU experts on MFMA (gfx950).
//
// Each expert is a SwiGLU FFN (moe-200m-qwen3-100b README, "Architecture
// diagram": routed and shared SwiGLU experts) with weights stacked
// [E, out, in] (SpecForge PR #930, "Why FSDP is enough here"); rows are
// grouped by expert so that the work scales with routed tokens, not with the
// number of experts (same section). Two kernels of one template:
//   gate/up : H[r, n] = silu(sum_k A[r,k] Wg[e,n,k]) * (sum_k A[r,k] Wu[e,n,k]),
//             stored in the operand dtype (bf16 rounding to nearest even);
//   down    : Y[r, n] = sum_k H[r,k] Wd[e,n,k], stored in fp32.
// Both operands are K-contiguous ([rows, K] and [N, K]), which is the layout
// the MFMA operands want: every lane reads 16 contiguous bytes of one row.
//
// Tiling: a block of 256 threads (4 waves, 2 x 2) computes BM = 128 rows x BN
// output columns (gate/up: 64 columns of H, i.e. 64 gate + 64 up weight rows;
// down: 128 columns). K advances in stages of 128 bytes per row (64 bf16 or
// 32 fp32), double-buffered in LDS; global loads of stage s+1 are in flight
// while stage s feeds the MFMAs. LDS rows are 128 bytes with the 16-byte
// chunks XOR-swizzled by (row & 7) so that the 16 lanes reading one MFMA
// fragment column hit distinct banks.
// MFMA: bf16 v_mfma_f32_16x16x32_bf16 (one per 32-wide K step), fp32
// v_mfma_f32_16x16x4_f32 (four per 16-wide K step); accumulation in fp32.
// Row tiles come from a device-side tile list (group, m-tile) written by the
// dispatch, so no group size ever travels to the host; blocks beyond the
// list's length exit at once.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRowBytes = 128;
constexpr int kChunks = kRowBytes / 16;

template <typename DT, bool GATEUP, int BN_>
struct GemmShape {
  static constexpr int BM = 128;
  static constexpr int BN = BN_;
  static constexpr int NB = GATEUP ? 2 * BN : BN;  // weight rows staged per block
  static constexpr int WN = 2;                     // waves along N (2 along M)
  static constexpr int TM = BM / 2;
  static constexpr int TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int NG = GATEUP ? 2 : 1;        // accumulator sets (gate, up)
  static constexpr int KE = kRowBytes / (int)sizeof(DT);
  static constexpr int A_CH = BM * kChunks / 256;
  static constexpr int B_CH = NB * kChunks / 256;
  static constexpr int LDS = 2 * (BM + NB) * kRowBytes;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

template <typename DT>
__device__ __forceinline__ void mfma_step(f32x4& acc, const u32x4& a, const u32x4& b);

template <>
__device__ __forceinline__ void mfma_step<uint16_t>(f32x4& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(f32x4& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[q]), __uint_as_float(b[q]), acc, 0, 0, 0);
}

template <typename DT>
__device__ __forceinline__ DT to_out(float v);
template <>
__device__ __forceinline__ uint16_t to_out<uint16_t>(float v) {
  return f32_to_bf16(v);
}
template <>
__device__ __forceinline__ float to_out<float>(float v) {
  return v;
}

template <typename DT, bool GATEUP, int BN>
__global__ __launch_bounds__(256) void k_gemm(GemmLaunch g) {
  using S = GemmShape<DT, GATEUP, BN>;
  __shared__ __align__(16) unsigned char lds[S::LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WN, wn = wave % S::WN;
  const int n_tiles_n = g.N / S::BN;
  const int64_t tile_m = (int64_t)blockIdx.x / n_tiles_n;
  const int tile_n = (int)((int64_t)blockIdx.x % n_tiles_n);

  int grp;
  int64_t row0;
  int rows;
  if (g.offsets) {
    if (tile_m >= g.n_tiles[0]) return;
    const int2 t = g.tiles[tile_m];
    if (t.x < 0 || t.x >= g.n_groups || t.y < 0) return;
    grp = t.x;
    row0 = (int64_t)g.offsets[grp] + (int64_t)t.y * S::BM;
    const int64_t left = (int64_t)g.offsets[grp + 1] - row0;
    rows = (int)(left < S::BM ? left : S::BM);
  } else {
    grp = 0;
    row0 = tile_m * S::BM;
    const int64_t left = g.rows - row0;
    rows = (int)(left < S::BM ? left : S::BM);
  }
  if (rows <= 0) return;
  const int n0 = tile_n * S::BN;
  const size_t kbytes = (size_t)g.K * sizeof(DT);
  const unsigned char* A = reinterpret_cast<const unsigned char*>(g.a);
  const unsigned char* B0 = reinterpret_cast<const unsigned char*>(g.b0) + (size_t)grp * g.N * kbytes;
  const unsigned char* B1 = GATEUP ? reinterpret_cast<const unsigned char*>(g.b1) + (size_t)grp * g.N * kbytes : B0;

  // Global sources of this thread's 16-byte chunks and their LDS slots.
  const unsigned char* a_src[S::A_CH];
  int a_dst[S::A_CH];
  bool a_ok[S::A_CH];
#pragma unroll
  for (int i = 0; i < S::A_CH; ++i) {
    const int q = tid + i * 256, r = q >> 3, c = q & 7;
    a_ok[i] = r < rows;
    int64_t src_row = row0 + (a_ok[i] ? r : 0);
    if (g.a_rows) {
      src_row = g.a_rows[src_row];
      src_row = src_row < 0 ? 0 : (src_row >= g.a_row_count ? g.a_row_count - 1 : src_row);
    }
    a_src[i] = A + (size_t)src_row * kbytes + c * 16;
    a_dst[i] = swz(r, c);
  }
  const unsigned char* b_src[S::B_CH];
  int b_dst[S::B_CH];
#pragma unroll
  for (int i = 0; i < S::B_CH; ++i) {
    const int q = tid + i * 256, r = q >> 3, c = q & 7;
    const unsigned char* base = (GATEUP && r >= S::BN) ? B1 + (size_t)(n0 + r - S::BN) * kbytes
                                                       : B0 + (size_t)(n0 + r) * kbytes;
    b_src[i] = base + c * 16;
    b_dst[i] = swz(S::BM + r, c);
  }

  u32x4 ra[S::A_CH], rb[S::B_CH];
  auto gload = [&](int kt) {
    const size_t off = (size_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < S::A_CH; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4*>(a_src[i] + off) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < S::B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + off);
  };
  auto lstore = [&](int buf) {
    unsigned char* base = lds + buf * (S::BM + S::NB) * kRowBytes;
#pragma unroll
    for (int i = 0; i < S::A_CH; ++i) *reinterpret_cast<u32x4*>(base + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < S::B_CH; ++i) *reinterpret_cast<u32x4*>(base + b_dst[i]) = rb[i];
  };

  f32x4 acc[S::NG][S::FM][S::FN];
#pragma unroll
  for (int h = 0; h < S::NG; ++h)
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
      for (int j = 0; j < S::FN; ++j) acc[h][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / S::KE;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    const unsigned char* base = lds + (kt & 1) * (S::BM + S::NB) * kRowBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ch = s * 4 + (lane >> 4);
      u32x4 af[S::FM];
#pragma unroll
      for (int i = 0; i < S::FM; ++i) {
        const int r = wm * S::TM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const u32x4*>(base + swz(r, ch));
      }
#pragma unroll
      for (int h = 0; h < S::NG; ++h) {
        u32x4 bfr[S::FN];
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
          const int r = S::BM + h * S::BN + wn * S::TN + j * 16 + (lane & 15);
          bfr[j] = *reinterpret_cast<const u32x4*>(base + swz(r, ch));
        }
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
          for (int j = 0; j < S::FN; ++j) mfma_step<DT>(acc[h][i][j], af[i], bfr[j]);
      }
    }
    if (kt + 1 < nk) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue. Lane l holds, for each 16 x 16 tile, rows 4*(l/16) + 0..3 of
  // column l % 16.
#pragma unroll
  for (int i = 0; i < S::FM; ++i) {
#pragma unroll
    for (int j = 0; j < S::FN; ++j) {
      const int n = n0 + wn * S::TN + j * 16 + (lane & 15);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = wm * S::TM + i * 16 + (lane >> 4) * 4 + rr;
        if (m >= rows) continue;
        const size_t o = (size_t)(row0 + m) * g.N + n;
        if constexpr (GATEUP) {
          const float gv = acc[0][i][j][rr], uv = acc[1][i][j][rr];
          const float hv = gv / (1.0f + __expf(-gv)) * uv;
          reinterpret_cast<DT*>(g.out)[o] = to_out<DT>(hv);
        } else {
          reinterpret_cast<float*>(g.out)[o] = acc[0][i][j][rr];
        }
      }
    }
  }
}

template <typename DT, bool GATEUP, int BN>
hipError_t launch_t(const GemmLaunch& g, hipStream_t s) {
  using S = GemmShape<DT, GATEUP, BN>;
  if (g.N % S::BN || g.K % S::KE) return hipErrorInvalidValue;
  const int64_t m_tiles = g.offsets ? g.max_m_tiles : (g.rows + S::BM - 1) / S::BM;
  const int64_t blocks = m_tiles * (g.N / S::BN);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm<DT, GATEUP, BN>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int gemm_bm(int, bool) { return 128; }

// gate/up: 64 columns of H per block; down: 128 output columns, or 64 when
// the width is an odd multiple of 64.
hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s) {
  const bool wide = g.N % 128 == 0;
  if (g.dtype == 1) {
    if (g.gateup) return launch_t<uint16_t, true, 64>(g, s);
    return wide ? launch_t<uint16_t, false, 128>(g, s) : launch_t<uint16_t, false, 64>(g, s);
  }
  if (g.gateup) return launch_t<float, true, 64>(g, s);
  return wide ? launch_t<float, false, 128>(g, s) : launch_t<float, false, 64>(g, s);
}

}  // namespace moe
