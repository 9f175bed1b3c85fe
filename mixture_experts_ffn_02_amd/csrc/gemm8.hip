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
//   * A stage is two 32 KB halves (weight rows, A rows) in a ring of five
//     half-stage LDS buffers (160 KB). One barrier per stage: every wave has
//     read stage t, and its copies of stage t + 1 have landed. Stage t's
//     buffers are then free, and each wave spreads its eighth of the copies
//     of the A half of stage t + 2 and of the weight half of stage t + 3 over
//     the next four K steps, two 1 KB copies per step (issued all at once
//     after the barrier, they stalled both waves of every SIMD together).
//     The weight rows are requested two stages ahead, the A rows (gathered
//     token rows) one stage ahead (measured 0.2-5% faster per launch than
//     the other way round).
//   * The copy stream runs on across the block's tiles: the last two stages
//     of a tile copy the next tile's first stages, and the epilogue stores
//     straight from the accumulators (buffer stores through a resource that
//     spans the tile's rows, whose range check drops the rows past the
//     tile's end), so no LDS is needed between tiles and the matrix cores
//     never wait for a new tile's first stage.
//   * Copies write 1 KB runs of LDS rows (lane i of a wave writes bytes
//     16i..16i+15); the 16-byte chunks of an LDS row are XOR-swizzled
//     (applied on the global side) so that the fragment reads of 16
//     consecutive rows hit distinct banks (measured: no bank conflicts).
//     Down products copy with buffer_load_dwordx4 ... lds, gate/up with
//     global_load_lds_dwordx4. While a global (FLAT) copy into LDS is in
//     flight the compiler cannot order LDS reads in the lgkm counter and
//     makes every fragment wait lgkmcnt(0); with buffer copies each MFMA
//     waits for its own two fragments only (reads issued weights first),
//     which took 2-4% off the down launches. For gate/up the buffer copies
//     were no faster and fetched about 50% more bytes past L2 (105 vs 70 GB
//     per launch at the DeepSeek-style layer), so those stay global.
//   * Persistent grid, one block per CU, tiles split into 8 contiguous
//     ranges, one per XCD (block b runs on XCD b % 8, measured), each walked
//     in raster groups of GM row tiles x all column tiles so the blocks
//     resident on an XCD share weight and A stages in its L2 (about 72% of
//     the copies' requests hit L2 on the DeepSeek-style routed gate/up).
//     Row tiles come from the device-side tile list of the dispatch (group,
//     m-tile).
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
// Every wave issues an eighth of each half-stage's copies (measured: leaving
// the copies to the second wave of each SIMD alone was 6% slower).
constexpr int kRuns = kHalf / 1024 / 8;  // 1 KB copies per wave per half-stage (4)
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Word 3 of a raw buffer resource (32-bit data format; offsets in bytes,
// range-checked against the resource's size).
constexpr uint32_t kRsrcWord3 = 0x00020000;
// A block-uniform pointer, said to be so: a buffer resource built from a
// value the compiler holds in vector registers becomes a loop over lanes.
__device__ __forceinline__ const unsigned char* uni(const unsigned char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  return reinterpret_cast<const unsigned char*>(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                                                (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v));
}

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
  if (n >= 24)
    asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n >= 12)
    asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n >= 8)
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (n >= 4)
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
    // a global -> LDS copy: the scheduler classes it with LDS writes (0x200)
    if (i < VM) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
  }
}

// One output tile of a launch: group e (grouped) or 0, rows row0 ..
// row0 + rows - 1 of A and of the output, output columns from n0.
struct Tile8 {
  int64_t row0;
  int e, rows, n0;
};

// STREAM: weight copies non-temporal (each weight tile read about once).
// BYGROUP: raster groups inside each group's row tiles (see tile_at).
template <bool GATEUP, bool GROUPED, bool STREAM, bool BYGROUP = false>
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
  const int nk = g.K / kKE;  // >= 3 (launch_gemm8 checks)
  const int nh = 2 * nk;     // half-stages of a tile
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
  // copy run R = 8 i + wave covers rows 8R .. 8R + 7 of a half-stage
  constexpr int kSlots = 8;
  const uint32_t b_lane = (uint32_t)((8 * wave + lrow) * kbytes) + lchunk * 16;

  // The block's tiles, in raster order: 8 contiguous ranges of the order,
  // one per XCD, each walked in groups of group_m row tiles x all column
  // tiles; a tile of the device-side list naming no group, or with no rows,
  // is skipped. BYGROUP cuts the raster groups inside each group's (expert's)
  // row tiles instead of across the whole list, so that no raster group
  // mixes two experts' weight panels: group e's row tiles are list entries
  // T_e .. T_e + r_e - 1 and its tiles raster positions T_e n_tiles_n ..
  // (T_e + r_e) n_tiles_n - 1, walked in ceil(r_e / group_m) chunks of
  // equal size.
  auto tile_at = [&](int64_t L, Tile8& t) -> bool {
    int64_t tile_m;
    int tile_n;
    if constexpr (GROUPED && BYGROUP) {
      const int64_t m0 = L / n_tiles_n;
      const int2 h = g.tiles[m0];
      if (h.x < 0 || h.x >= g.n_groups || h.y < 0) return false;
      const int64_t te = m0 - h.y;
      const int64_t re = ((int64_t)g.offsets[h.x + 1] - g.offsets[h.x] + kBM - 1) / kBM;
      const int64_t nc = (re + group_m - 1) / group_m;
      const int64_t cs = (re + nc - 1) / nc;
      const int64_t within = L - te * n_tiles_n;
      const int64_t c = within / (cs * n_tiles_n);
      const int64_t gm = (re - c * cs) < cs ? (re - c * cs) : cs;
      const int64_t w2 = within - c * cs * n_tiles_n;
      tile_m = te + c * cs + w2 % gm;
      tile_n = (int)(w2 / gm);
    } else {
      const int64_t gsz = (int64_t)group_m * n_tiles_n;
      const int64_t first_m = (L / gsz) * group_m;
      const int64_t gm = (m_tiles - first_m) < group_m ? (m_tiles - first_m) : group_m;
      const int64_t within = L % gsz;
      tile_m = first_m + within % gm;
      tile_n = (int)(within / gm);
    }
    t.n0 = GATEUP ? tile_n * 128 : tile_n * 256;
    if constexpr (GROUPED) {
      const int2 tl = g.tiles[tile_m];
      if (tl.x < 0 || tl.x >= g.n_groups || tl.y < 0) return false;
      t.e = tl.x;
      t.row0 = (int64_t)g.offsets[t.e] + (int64_t)tl.y * kBM;
      const int64_t left = (int64_t)g.offsets[t.e + 1] - t.row0;
      t.rows = (int)(left < kBM ? left : kBM);
    } else {
      t.e = 0;
      t.row0 = tile_m * kBM;
      const int64_t left = g.rows - t.row0;
      t.rows = (int)(left < kBM ? left : kBM);
    }
    // the tile is block-uniform: say so, so that its values stay scalar
    t.e = __builtin_amdgcn_readfirstlane(t.e);
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.row0 = ((int64_t)__builtin_amdgcn_readfirstlane((int)(t.row0 >> 32)) << 32) |
             (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)t.row0);
    return t.rows > 0;
  };
  int64_t L = L0 + slot;
  auto next_tile = [&](Tile8& t) -> bool {  // the next tile of this block from L on
    for (; L < L1; L += per_xcd)
      if (tile_at(L, t)) {
        L += per_xcd;
        return true;
      }
    return false;
  };
  // Per tile, for the copies (block-uniform bases and size; down builds
  // buffer resources from them): the row of abase that each of this lane's
  // A runs reads (run 8 i + wave covers tile rows 64 i + 8 wave .. +7; rows
  // past the tile's end read a valid row, or nothing, and their results are
  // never stored)
  // and the weight bases (gate/up: runs with i >= 2 are up rows). Gathered
  // rows index all of A, contiguous ones the tile's own rows.
  struct Src {
    uint32_t a_row[kRuns];
    const unsigned char* abase;
    uint32_t a_bytes;
    const unsigned char* b0;
    const unsigned char* b1;
  };
  const unsigned char* const A = reinterpret_cast<const unsigned char*>(g.a);
  auto make_src = [&](const Tile8& t, Src& sr) __attribute__((always_inline)) {
    if (g.a_rows) {
      sr.abase = A;
      sr.a_bytes = (uint32_t)(g.a_row_count * (int64_t)kbytes);
    } else {
      sr.abase = A + (size_t)t.row0 * kbytes;
      sr.a_bytes = (uint32_t)((int64_t)t.rows * kbytes);
    }
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      int r = 8 * (kSlots * i + wave) + lrow;
      // rows past the tile's end copy its last row, except in down products
      // of contiguous rows: there they stay past the end of the copy's buffer
      // range, so the hardware drops them (nothing fetched; the copy is still
      // issued and counted by the stage waits)
      if (GATEUP || g.a_rows) r = r < t.rows ? r : t.rows - 1;
      int64_t src = r;
      if (g.a_rows) {
        src = g.a_rows[t.row0 + r];
        src = src < 0 ? 0 : (src >= g.a_row_count ? g.a_row_count - 1 : src);
      }
      sr.a_row[i] = (uint32_t)src;
    }
    // block-uniform bases; the lane offset b_lane is added at the copy
    const bool xg = t.e == g.extra_group;
    sr.b0 = (xg ? reinterpret_cast<const unsigned char*>(g.bx0)
                : reinterpret_cast<const unsigned char*>(g.b0) + (size_t)t.e * g.N * kbytes) +
            (size_t)t.n0 * kbytes;
    sr.b1 = GATEUP ? (xg ? reinterpret_cast<const unsigned char*>(g.bx1)
                         : reinterpret_cast<const unsigned char*>(g.b1) + (size_t)t.e * g.N * kbytes) +
                         (size_t)t.n0 * kbytes
                   : sr.b0;
  };
  const uint32_t w_bytes = (uint32_t)(kBR * kbytes);  // a down tile's weight rows
  // Copy runs I0 .. I0 + NR - 1 of half-stage h of the tile described by sr
  // (even h: weight rows of stage h / 2, odd: A rows) into ring buffer `buf`.
  auto issue_runs = [&](const Src& sr, int h, int buf, auto i0c, auto nc) __attribute__((always_inline)) {
    constexpr int I0 = decltype(i0c)::value, NR = decltype(nc)::value;
    unsigned char* dst = lds + buf * kHalf + wave * 1024;
    const uint32_t koff = (uint32_t)(h >> 1) * kSB;
    if constexpr (GATEUP) {  // global copies (gate/up: buffer copies fetched 50% more past L2)
      if ((h & 1) == 1) {
#pragma unroll
        for (int i = I0; i < I0 + NR; ++i)
          lds_dma16(sr.abase + (size_t)sr.a_row[i] * kbytes + koff + lchunk * 16, dst + i * kSlots * 1024);
        return;
      }
      // weight run i starts at weight row 8 kSlots i; the second half of
      // the runs are up rows
#pragma unroll
      for (int i = I0; i < I0 + NR; ++i) {
        const unsigned char* src = i >= kRuns / 2
                                       ? sr.b1 + (size_t)(8 * kSlots * (i - kRuns / 2)) * kbytes + koff + b_lane
                                       : sr.b0 + (size_t)(8 * kSlots * i) * kbytes + koff + b_lane;
        lds_dma16<STREAM>(src, dst + i * kSlots * 1024);
      }
      return;
    }
    // down: buffer copies (32-bit offsets: a gathered A under 4 GiB, which
    // the launch checks)
    if ((h & 1) == 1) {
      const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
          (void*)uni(sr.abase), 0, (uint32_t)__builtin_amdgcn_readfirstlane((int)sr.a_bytes), kRsrcWord3);
#pragma unroll
      for (int i = I0; i < I0 + NR; ++i) {
        // (a local: passing the array element drops the kernel's host stub)
        const uint32_t vo = sr.a_row[i] * (uint32_t)kbytes + lchunk * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(dst + i * kSlots * 1024),
                                                 16, vo, koff, 0, 0);
      }
      return;
    }
    // weight run i starts at weight row 8 kSlots i
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)uni(sr.b0), 0, w_bytes, kRsrcWord3);
#pragma unroll
    for (int i = I0; i < I0 + NR; ++i) {
      const uint32_t row = (uint32_t)(8 * kSlots * i) * (uint32_t)kbytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(dst + i * kSlots * 1024),
                                               16, b_lane, koff + row, 0, STREAM ? 2 : 0);
    }
  };
  using R0 = std::integral_constant<int, 0>;
  using R2 = std::integral_constant<int, kRuns / 2>;   // half of a half-stage's runs
  using R4 = std::integral_constant<int, kRuns>;

  Tile8 cur, nxt;
  if (!next_tile(cur)) return;
  Src sc, sn;
  make_src(cur, sc);
  bool has_next = next_tile(nxt);
  if (has_next) make_src(nxt, sn);

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
  auto load_frag = [&](Frag& f, int abuf, int bbuf, int s4) __attribute__((always_inline)) {
    const unsigned char* ab = lds + abuf * kHalf + wm * 128 * kSB + loff[s4];
    const unsigned char* bb = lds + bbuf * kHalf + wrow0 * kSB + loff[s4];
    f.b[0] = *reinterpret_cast<const u32x4*>(bb);
    f.b[1] = *reinterpret_cast<const u32x4*>(bb + kWStep);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const u32x4*>(ab + i * 32 * kSB);
  };
  auto mma = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                            __builtin_bit_cast(bf16x8, f.b[j]), acc[i][j], 0, 0, 0);
  };

  // Epilogue of a finished tile straight from the accumulators (no LDS, so
  // it overlaps the next tile's copies): element x of a 32 x 32 tile sits in
  // row 8(x/4) + 4(l/32) + x%4, column l % 32 of lane l, so each store
  // writes 32 consecutive columns of two rows. gate/up: H = silu(g) u in
  // bf16; down: fp32. Buffer stores through a resource that spans exactly
  // the tile's rows, so the hardware range check drops the rows past the
  // tile's end, and every address is one 32-bit lane offset plus a constant.
  auto epilogue = [&](const Tile8& t) __attribute__((always_inline)) {
    constexpr int EB = GATEUP ? 2 : 4;
    unsigned char* const obase = reinterpret_cast<unsigned char*>(g.out) + (size_t)t.row0 * g.N * EB;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(obase, 0, t.rows * g.N * EB, kRsrcWord3);
    const int col = (GATEUP ? t.n0 + wn * 32 : t.n0 + wn * 64) + (lane & 31);
    const int lane_off = ((wm * 128 + 4 * (lane >> 5)) * g.N + col) * EB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int off = lane_off + (i * 32 + 8 * (x >> 2) + (x & 3)) * g.N * EB;
        if constexpr (GATEUP) {
          const float gv = acc[i][0][x], uv = acc[i][1][x];
          const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(h), rs, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][0][x]), rs, off, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][1][x]), rs, off + 32 * 4, 0, 0);
        }
      }
    }
  };

  // The copy stream. Half-stage q of the block counts the half-stages of all
  // its tiles in order (q = tile's first q + h); it lives in ring buffer
  // q % 5. Over the four K steps that follow the barrier of stage t (whose
  // buffers it frees) each wave issues its eighth of half-stage 2t + 5 (the
  // A half of stage t + 2; runs 0-1, then 2-3) and 2t + 6 (the weight half
  // of stage t + 3; runs 0-1, 2-3): in stage t that is half-stage 2t + 3 runs
  // 2-3 in step 0, 2t + 4 in steps 1-2, 2t + 5 runs 0-1 in step 3.
  // Half-stages past the tile's end belong to the next tile: with nk >= 3
  // they occur only in stages nk - 2 (2t + 4, 2t + 5) and nk - 1 (all). The
  // block's very first tile copies half-stages 0 .. 4 up front.
  int qbase = 0;  // ring position of the current tile's half-stage 0
  enum { kNone = 0, kCur = 1, kNext = 2 };
  // copy of half-stage h (current tile's numbering) for slot owner w
  auto issue_q = [&](int w, int h, auto i0c, auto nc) __attribute__((always_inline)) {
    if (w == kCur)
      issue_runs(sc, h, (qbase + h) % kNH, i0c, nc);
    else if (w == kNext)
      issue_runs(sn, h - nh, (qbase + h) % kNH, i0c, nc);
  };
  for (int h = 0; h < kNH; ++h) issue_runs(sc, h, h, R0{}, R4{});
  stage_barrier(kRuns * (kNH - 2));  // stage 0 landed; three halves may be in flight
  Frag P, Q;
  load_frag(P, (qbase + 1) % kNH, qbase % kNH, 0);
  // Stage t. STEADY: every copy belongs to the current tile and the next
  // stage exists (one basic block per K step, so the scheduler interleaves
  // the copies, reads and MFMAs). Otherwise the copy slots w0 (step 0),
  // w12 (steps 1-2), w3 (step 3) name the tile each copy belongs to (or
  // none); `more`: the stage after it exists (its first fragments are read
  // in step 3); `inflight`: the weight half of stage t + 2 exists, so the
  // barrier lets its copies stay in flight.
  // Down products: each K step's MFMAs and interleaved reads and copies run
  // at wave priority 1, the barrier waits and the epilogue at 0 (measured:
  // 2-3% off the down launches of the three large layers; no gain for
  // gate/up, whose epilogue is small).
  auto raise_prio = [&]() __attribute__((always_inline)) {
    if constexpr (!GATEUP) __builtin_amdgcn_s_setprio(1);
  };
  auto lower_prio = [&]() __attribute__((always_inline)) {
    if constexpr (!GATEUP) __builtin_amdgcn_s_setprio(0);
  };
  auto stage = [&](int t, auto steady, int w0, int w12, int w3, bool more, bool inflight)
      __attribute__((always_inline)) {
    constexpr bool S = decltype(steady)::value;
    const int bbuf = (qbase + 2 * t) % kNH, abuf = (qbase + 2 * t + 1) % kNH;
    const int na = (abuf + 2) % kNH, nb = (bbuf + 2) % kNH;
    load_frag(Q, abuf, bbuf, 1);
    if (S) issue_runs(sc, 2 * t + 3, (qbase + 2 * t + 3) % kNH, R2{}, R2{});
    else issue_q(w0, 2 * t + 3, R2{}, R2{});
    raise_prio();
    mma(P);
    interleave8<6, kRuns / 2>();
    __builtin_amdgcn_sched_barrier(0);
    lower_prio();
    load_frag(P, abuf, bbuf, 2);
    if (S) issue_runs(sc, 2 * t + 4, (qbase + 2 * t + 4) % kNH, R0{}, R2{});
    else issue_q(w12, 2 * t + 4, R0{}, R2{});
    raise_prio();
    mma(Q);
    interleave8<6, kRuns / 2>();
    __builtin_amdgcn_sched_barrier(0);
    lower_prio();
    load_frag(Q, abuf, bbuf, 3);
    if (S) issue_runs(sc, 2 * t + 4, (qbase + 2 * t + 4) % kNH, R2{}, R2{});
    else issue_q(w12, 2 * t + 4, R2{}, R2{});
    raise_prio();
    mma(P);
    interleave8<6, kRuns / 2>();
    __builtin_amdgcn_sched_barrier(0);
    lower_prio();
    // stage barrier: this wave's copies of stage t + 1 have landed (the
    // weight half of stage t + 2, issued after them, may still be in flight) and
    // every wave has read stage t
    stage_barrier(S || inflight ? kRuns : 0);
    __builtin_amdgcn_sched_barrier(0);
    if (S) issue_runs(sc, 2 * t + 5, (qbase + 2 * t + 5) % kNH, R0{}, R2{});
    else issue_q(w3, 2 * t + 5, R0{}, R2{});
    if (S || more) load_frag(P, na, nb, 0);
    raise_prio();
    mma(Q);
    interleave8<6, kRuns / 2>();
    __builtin_amdgcn_sched_barrier(0);
    lower_prio();
  };
  using Steady = std::true_type;
  using Generic = std::false_type;
  bool first = true;
  while (true) {
    int t = 0;
    if (first) {  // half-stages 3 and 4 were copied up front
      stage(0, Generic{}, kNone, kNone, kCur, true, true);
      t = 1;
    }
    for (; t < nk - 2; ++t) stage(t, Steady{}, 0, 0, 0, true, true);
    const int wn_ = has_next ? kNext : kNone;
    stage(nk - 2, Generic{}, kCur, wn_, wn_, true, has_next);
    stage(nk - 1, Generic{}, wn_, wn_, wn_, has_next, has_next);
    epilogue(cur);
    if (!has_next) break;
    // the next tile becomes current; its first stages are already in flight
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[i][j][x] = 0.0f;
    qbase = (qbase + nh) % kNH;
    cur = nxt;
    sc = sn;
    has_next = next_tile(nxt);
    if (has_next) make_src(nxt, sn);
    first = false;
  }
}

}  // namespace

// The down product's buffer copies address gathered rows by 32-bit offsets
// into all of A (the forward's down products read their rows in place).
static bool gather_fits(const GemmLaunch& g) {
  return g.gateup || !g.a_rows || g.a_row_count * 2 * (int64_t)g.K < ((int64_t)1 << 32);
}

// 256 x 256 eight-wave tiles for bf16 forward products; the caller checks
// dtype, K % 64, N (gate/up: % 128, down: % 256) and, for down, a gathered A
// under 4 GiB.
hipError_t launch_gemm8(const GemmLaunch& g, hipStream_t s) {
  if (g.dtype != 1 || g.K % kKE || g.K < 3 * kKE || (g.gateup ? g.N % 128 : g.N % 256) || g.bt || g.koffs || g.out_g ||
      !gather_fits(g))
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
  auto go = [&](auto kern) __attribute__((always_inline)) { hipLaunchKernelGGL(kern, grid, block, 0, s, g); };
  if (g.gateup) {
    if (g.offsets) {
      if (g.raster_by_group && !g.b_stream) go(k_gemm8<true, true, false, true>);
      else if (g.b_stream) go(k_gemm8<true, true, true>); else go(k_gemm8<true, true, false>);
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
  return MOE_GEMM8 && bm == 256 && g.dtype == 1 && g.K % kKE == 0 && g.K >= 3 * kKE &&
         (g.gateup ? g.N % 128 == 0 : g.N % 256 == 0) &&
         !g.bt && !g.koffs && !g.out_g && gather_fits(g);
}

hipError_t launch_gemm_fwd(const GemmLaunch& g, int bm, hipStream_t s) {
  return gemm8_fits(g, bm) ? launch_gemm8(g, s) : launch_gemm(g, bm, s);
}

}  // namespace moe
