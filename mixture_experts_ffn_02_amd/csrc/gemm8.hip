// Grouped GEMMs of the SwiGLU experts with 256 x 256 tiles on eight waves
// (gfx950), for layers with many rows per expert or a long K.
//
// What is computed is the same as k_gemm in gemm.hip (SwiGLU experts,
// moe-200m-qwen3-100b README, "Architecture diagram"; experts stacked
// [E, out, in], SpecForge PR #930, "Why FSDP is enough here"):
//   gate/up : H[r, n] = silu(sum_k A[r,k] Wg[e,n,k]) * (sum_k A[r,k] Wu[e,n,k]),
//             stored in bf16 (rounded to nearest even);
//   down    : Y[r, n] = sum_k H[r,k] Wd[e,n,k], stored in fp32.
// bf16 operands, fp32 accumulation, both operands K-contiguous.
//
// Why a second kernel. With one wave per SIMD (k_gemm's 4-wave 256-row
// tiles), the wave that issues the global -> LDS copies and waits at the
// stage barrier is also the only one that can issue MFMAs, so every such
// stall idles the matrix core; measured, the copy and MFMA times of a stage
// add up instead of overlapping. Here two waves share each SIMD:
//   * 8 waves (waves w and w + 4 share a SIMD); wave w owns rows
//     128 (w / 4) .. +127 of the tile and, for gate/up, 32 columns of H
//     (gate rows 32 (w % 4).. and up rows 128 + 32 (w % 4)..), for down 64
//     output columns. Each wave holds 8 accumulator tiles of 32 x 32 (128
//     registers), so two waves fit a SIMD's register file.
//   * K advances in stages of 64 elements (128 bytes per row), four MFMA K
//     steps of 16. A wave reads the fragments of K step s + 1 from LDS while
//     its MFMAs of step s run (two fragment sets, interleaved one by one).
//     Both waves of a SIMD stream fragments at once: measured, one wave per
//     SIMD reads LDS at about 25 bytes per clock, two at about 44, and a
//     wave needs 6 KB per 8 MFMAs (256 cycles).
//   * A stage is two 32 KB halves (A rows, weight rows) in a ring of five
//     half-stage LDS buffers (160 KB). At the one barrier per stage (every
//     wave has read stage t and its copies of stage t + 1 have landed) each
//     wave copies its eighth of the weight half of stage t + 2 and of the A
//     half of stage t + 3: the A rows, gathered token rows that mostly miss
//     L2, are requested two stages ahead, the weight rows (shared by the
//     tiles that run together on one XCD) one stage ahead.
//   * Copies use global_load_lds_dwordx4 (lane i of a wave writes bytes
//     16i..16i+15 of a 1 KB run of LDS rows); the 16-byte chunks of an LDS
//     row are XOR-swizzled (applied on the global side) so that the
//     fragment reads of 16 consecutive rows hit distinct banks.
//   * Persistent grid, one block per CU, tiles split into 8 contiguous
//     ranges, one per XCD (block b runs on XCD b % 8), each walked in raster
//     groups of GM row tiles x all column tiles so the blocks resident on an
//     XCD share weight and A stages in its L2. Row tiles come from the
//     device-side tile list of the dispatch (group, m-tile).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 256;              // rows of a tile
constexpr int kBR = 256;              // weight rows staged per tile
constexpr int kSB = 128;              // bytes of one row in one stage
constexpr int kKE = 64;               // K elements (bf16) per stage
constexpr int kHalf = kBM * kSB;      // bytes of one operand's half-stage (32 KB)
constexpr int kNH = 5;                // half-stage buffers
constexpr int kRuns = kHalf / 1024 / 8;  // 1 KB copies per wave per half-stage (4)
constexpr int kScratch = 32 * (32 * 4 + 16);  // epilogue scratch per wave

typedef float f32x16 __attribute__((ext_vector_type(16)));

// XOR key of LDS row `row` (128-byte rows, 8 chunks): the 16 lanes of one
// ds_read_b128 phase read one logical chunk of 16 consecutive rows; rows r
// and r + 8 differ in bit 0 of the key, so the 16 reads land in 16 distinct
// 16-byte bank groups of a 256-byte window.
__device__ __forceinline__ int key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kSB + ((chunk ^ key(row)) << 4); }

// The stage barrier: at most n of this wave's 1 KB copies still in flight
// (n a block-uniform multiple of kRuns) and its LDS reads done, then s_barrier, in
// one asm block with a memory clobber so that no LDS access moves across.
__device__ __forceinline__ void stage_barrier(int n) {
  static_assert(kRuns == 4, "vmcnt immediates below assume 4 copies per half-stage");
  if (n >= 3 * kRuns)
    asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n >= 2 * kRuns)
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n >= kRuns)
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// One K step: 8 MFMAs with the 6 fragment reads of the next step (and VM
// copy issues) placed between them.
template <int RD, int VM>
__device__ __forceinline__ void interleave8() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (i < VM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM read (copy)
    if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
  }
}

// STREAM: weight copies non-temporal (each weight tile read about once).
template <bool GATEUP, bool GROUPED, bool STREAM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm8(GemmLaunch g) {
  __shared__ __align__(16) unsigned char lds[kNH * kHalf];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int wm = wave >> 2, wn = wave & 3;  // rows half, column slice
  const int n_tiles_n = GATEUP ? g.N / 128 : g.N / 256;
  const int64_t m_tiles = GROUPED ? (int64_t)g.n_tiles[0] : (g.rows + kBM - 1) / kBM;
  const int64_t total = m_tiles * n_tiles_n;
  const int per_xcd = gridDim.x / kXcd;
  const int xcd = blockIdx.x % kXcd, slot = blockIdx.x / kXcd;
  const int64_t span = (total + kXcd - 1) / kXcd;
  const int64_t L0 = xcd * span;
  const int64_t L1 = L0 + span < total ? L0 + span : total;
  const size_t kbytes = (size_t)g.K * 2;
  const int nk = g.K / kKE;
  const int group_m = g.group_m > 0 ? g.group_m : kGroupM;
  // Copy lanes: copy run R (= 8 i + wave, i < 4) of a half-stage writes LDS
  // rows 8R .. 8R + 7; lane l writes row 8R + l / 8, physical chunk l % 8,
  // which holds logical chunk (l % 8) ^ key(row) = (l % 8) ^ (l / 8) ^ (wave & 1).
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow ^ (wave & 1);
  // Fragment lane offsets: every fragment row is lane % 32 plus a multiple
  // of 32, so the reads of K step s4 (0..3) share one offset.
  uint32_t loff[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) loff[s4] = (uint32_t)swz(lane & 31, 2 * s4 + (lane >> 5));
  const int wrow0 = GATEUP ? wn * 32 : wn * 64;  // weight row of tile j = 0
  constexpr int kWStep = GATEUP ? 128 * kSB : 32 * kSB;  // tile j = 1 is this many bytes further
  unsigned char* const scratch = lds + wave * kScratch;

  for (int64_t L = L0 + slot; L < L1; L += per_xcd) {
    const int64_t gsz = (int64_t)group_m * n_tiles_n;
    const int64_t first_m = (L / gsz) * group_m;
    const int64_t gm = (m_tiles - first_m) < group_m ? (m_tiles - first_m) : group_m;
    const int64_t within = L % gsz;
    const int64_t tile_m = first_m + within % gm;
    const int tile_n = (int)(within / gm);

    int e = 0;
    int64_t row0;
    int rows;
    bool skip = false;
    if constexpr (GROUPED) {
      const int2 t = g.tiles[tile_m];
      skip = t.x < 0 || t.x >= g.n_groups || t.y < 0;
      e = skip ? 0 : t.x;
      row0 = (int64_t)g.offsets[e] + (int64_t)t.y * kBM;
      const int64_t left = (int64_t)g.offsets[e + 1] - row0;
      rows = (int)(left < kBM ? left : kBM);
    } else {
      row0 = tile_m * kBM;
      const int64_t left = g.rows - row0;
      rows = (int)(left < kBM ? left : kBM);
    }
    if (skip || rows <= 0) continue;  // uniform across the block
    const bool xg = e == g.extra_group;
    const unsigned char* A = reinterpret_cast<const unsigned char*>(g.a);
    const unsigned char* B0 = xg ? reinterpret_cast<const unsigned char*>(g.bx0)
                                 : reinterpret_cast<const unsigned char*>(g.b0) + (size_t)e * g.N * kbytes;
    const unsigned char* B1 = !GATEUP ? B0
                              : xg    ? reinterpret_cast<const unsigned char*>(g.bx1)
                                      : reinterpret_cast<const unsigned char*>(g.b1) + (size_t)e * g.N * kbytes;
    // gate/up: weight rows 0..127 of a stage are gate rows n0.., 128..255 up
    // rows n0..; down: 256 weight rows n0..
    const int n0 = GATEUP ? tile_n * 128 : tile_n * 256;

    // Source rows of this lane's A copies: run 8 i + wave covers tile rows
    // 64 i + 8 wave .. +7. Rows past the tile's end read a valid row; their
    // results are never stored. Weight run 8 i + wave covers weight rows
    // 64 i + 8 wave .. (gate/up: runs with i >= 2 are up rows 64 (i - 2)..),
    // a block-uniform base plus one lane offset.
    int32_t a_row[kRuns];
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      int r = 64 * i + 8 * wave + lrow;
      r = r < rows ? r : rows - 1;
      int64_t src = row0 + r;
      if (g.a_rows) {
        src = g.a_rows[src];
        src = src < 0 ? 0 : (src >= g.a_row_count ? g.a_row_count - 1 : src);
      }
      a_row[i] = (int32_t)src;
    }
    const uint32_t b_lane = (uint32_t)((8 * wave + lrow) * kbytes) + lchunk * 16;
    // Copy of half-stage h (even: A rows of stage h / 2, odd: weight rows)
    // into buffer h % 5.
    auto issue = [&](int h) {
      unsigned char* dst = lds + (h % kNH) * kHalf + wave * 1024;
      const size_t koff = (size_t)(h >> 1) * kSB;
      if ((h & 1) == 0) {
#pragma unroll
        for (int i = 0; i < kRuns; ++i)
          lds_dma16(A + (size_t)(uint32_t)a_row[i] * kbytes + koff + lchunk * 16, dst + i * 8192);
        return;
      }
      auto wbase = [&](int i) {
        return (GATEUP && i >= 2) ? B1 + (size_t)(n0 + 64 * (i - 2)) * kbytes + koff + b_lane
                                  : B0 + (size_t)(n0 + 64 * i) * kbytes + koff + b_lane;
      };
#pragma unroll
      for (int i = 0; i < kRuns; ++i) lds_dma16<STREAM>(wbase(i), dst + i * 8192);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.0f;

    // Fragments of one K step: A tiles i (rows 128 wm + 32 i + lane % 32)
    // and weight tiles j (rows wrow0 + lane % 32, and kWStep further).
    struct Frag {
      u32x4 a[4], b[2];
    };
    auto load_frag = [&](Frag& f, uint32_t abuf, uint32_t bbuf, int s4) {
      const unsigned char* ab = lds + abuf + wm * 128 * kSB + loff[s4];
      const unsigned char* bb = lds + bbuf + wrow0 * kSB + loff[s4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const u32x4*>(ab + i * 32 * kSB);
      f.b[0] = *reinterpret_cast<const u32x4*>(bb);
      f.b[1] = *reinterpret_cast<const u32x4*>(bb + kWStep);
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                              __builtin_bit_cast(bf16x8, f.b[j]), acc[i][j], 0, 0, 0);
    };

    // Prologue: half-stages 0..4 (stages 0 and 1, the A half of stage 2).
    const int nh = 2 * nk;
    const int pro = nh < kNH ? nh : kNH;
    for (int h = 0; h < pro; ++h) issue(h);
    stage_barrier((pro - 2) * kRuns);  // stage 0 landed; the later halves may be in flight
    Frag P, Q;
    uint32_t abuf = 0, bbuf = kHalf;  // ring offsets of stage t's halves ((2t) % 5, (2t + 1) % 5)
    // One stage: K steps 0..2 with the next step's fragment reads between
    // the MFMAs; the stage barrier (this wave's copies of stage t + 1 have
    // landed, the A half of stage t + 2 issued after them may still be in
    // flight, and every wave has read stage t); then, stage t's buffers
    // being free, the copies of the weight half of stage t + 2 and the A
    // half of stage t + 3, the reads of step 0 of stage t + 1 and the MFMAs
    // of step 3. FULL: all of those exist (t + 3 < nk), so the last step is
    // one basic block the scheduler can interleave.
    auto stage = [&](int t, auto full) {
      load_frag(Q, abuf, bbuf, 1);
      mma(P);
      interleave8<6, 0>();
      __builtin_amdgcn_sched_barrier(0);
      load_frag(P, abuf, bbuf, 2);
      mma(Q);
      interleave8<6, 0>();
      __builtin_amdgcn_sched_barrier(0);
      load_frag(Q, abuf, bbuf, 3);
      mma(P);
      interleave8<6, 0>();
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t na = abuf + 2 * kHalf >= kNH * kHalf ? abuf + 2 * kHalf - kNH * kHalf : abuf + 2 * kHalf;
      const uint32_t nb = bbuf + 2 * kHalf >= kNH * kHalf ? bbuf + 2 * kHalf - kNH * kHalf : bbuf + 2 * kHalf;
      if constexpr (decltype(full)::value) {
        stage_barrier(kRuns);
        __builtin_amdgcn_sched_barrier(0);
        issue(2 * t + 5);
        issue(2 * t + 6);
        load_frag(P, na, nb, 0);
        mma(Q);
        interleave8<6, 8>();
      } else {
        stage_barrier(2 * t + 4 < nh ? kRuns : 0);
        __builtin_amdgcn_sched_barrier(0);
        if (2 * t + 5 < nh) issue(2 * t + 5);
        if (2 * t + 6 < nh) issue(2 * t + 6);
        if (t + 1 < nk) load_frag(P, na, nb, 0);
        mma(Q);
      }
      __builtin_amdgcn_sched_barrier(0);
      abuf = na;
      bbuf = nb;
    };
    load_frag(P, abuf, bbuf, 0);
    int t = 0;
    for (; t + 3 < nk; ++t) stage(t, std::true_type{});
    for (; t < nk; ++t) stage(t, std::false_type{});
    barrier();  // every wave is done with the stage buffers

    // Epilogue of this wave's 4 x 2 accumulator tiles (gate/up: 4 tiles of
    // H, SwiGLU applied; down: 8 fp32 tiles). A 32 x 32 tile goes through
    // the wave's scratch (row-major, padded rows) and leaves as 16-byte row
    // chunks. Element x of a tile sits in row 8(x/4) + 4(l/32) + x%4, column
    // l % 32 of lane l.
    auto put_tile = [&](auto zero, const f32x16& v, int i, int col0) {
      using T = decltype(zero);
      constexpr int EB = (int)sizeof(T), P2 = 32 * EB + 16, CH = 32 * EB / 16;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int r = 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
        T o;
        if constexpr (sizeof(T) == 2)
          o = f32_to_bf16(v[x]);
        else
          o = v[x];
        *reinterpret_cast<T*>(scratch + r * P2 + (lane & 31) * EB) = o;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // tile base (block-uniform) plus a 32-bit offset: m < 256 rows
      unsigned char* obase = reinterpret_cast<unsigned char*>(g.out) + (size_t)row0 * g.N * EB;
#pragma unroll
      for (int q0 = 0; q0 < 32 * CH; q0 += 64) {
        const int qq = q0 + lane, r = qq / CH, c16 = qq % CH;
        const u32x4 val = *reinterpret_cast<const u32x4*>(scratch + r * P2 + c16 * 16);
        const int m = wm * 128 + i * 32 + r;
        if (m < rows) *reinterpret_cast<u32x4*>(obase + (uint32_t)((m * g.N + col0 + c16 * (16 / EB)) * EB)) = val;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (GATEUP) {
        f32x16 hv;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float gv = acc[i][0][x], uv = acc[i][1][x];
          hv[x] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        }
        put_tile(uint16_t{}, hv, i, n0 + wn * 32);
      } else {
        put_tile(float{}, acc[i][0], i, n0 + wn * 64);
        put_tile(float{}, acc[i][1], i, n0 + wn * 64 + 32);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    barrier();  // scratch reads done before the next tile's copies
  }
}

}  // namespace

// 256 x 256 eight-wave tiles for bf16 forward products; the caller checks
// dtype, K % 64 and N (gate/up: % 128, down: % 256).
hipError_t launch_gemm8(const GemmLaunch& g, hipStream_t s) {
  if (g.dtype != 1 || g.K % kKE || (g.gateup ? g.N % 128 : g.N % 256) || g.bt || g.koffs || g.out_g)
    return hipErrorInvalidValue;
  int64_t blocks = cu_count();
  blocks = (blocks + kXcd - 1) / kXcd * kXcd;
  if (!g.offsets) {
    const int64_t tiles = (g.rows + kBM - 1) / kBM * (g.gateup ? g.N / 128 : g.N / 256);
    if (tiles <= 0) return hipSuccess;
    const int64_t need = (tiles + kXcd - 1) / kXcd * kXcd;
    blocks = need < blocks ? need : blocks;
  }
  const dim3 grid((unsigned)blocks), block(512);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, g); };
  if (g.gateup) {
    if (g.offsets) {
      if (g.b_stream) go(k_gemm8<true, true, true>); else go(k_gemm8<true, true, false>);
    } else {
      if (g.b_stream) go(k_gemm8<true, false, true>); else go(k_gemm8<true, false, false>);
    }
  } else {
    if (g.offsets) {
      if (g.b_stream) go(k_gemm8<false, true, true>); else go(k_gemm8<false, true, false>);
    } else {
      if (g.b_stream) go(k_gemm8<false, false, true>); else go(k_gemm8<false, false, false>);
    }
  }
  return hipGetLastError();
}

// Forward products with row tile bm: the eight-wave kernel where bm is 256
// and the shape fits it, else k_gemm. MOE_GEMM8=0 at build time keeps
// k_gemm everywhere (for comparisons).
#ifndef MOE_GEMM8
#define MOE_GEMM8 1
#endif
bool gemm8_fits(const GemmLaunch& g, int bm) {
  return MOE_GEMM8 && bm == 256 && g.dtype == 1 && g.K % kKE == 0 && (g.gateup ? g.N % 128 == 0 : g.N % 256 == 0) &&
         !g.bt && !g.koffs && !g.out_g;
}

hipError_t launch_gemm_fwd(const GemmLaunch& g, int bm, hipStream_t s) {
  return gemm8_fits(g, bm) ? launch_gemm8(g, s) : launch_gemm(g, bm, s);
}

}  // namespace moe
