// Grouped GEMMs of the SwiGLU experts on MFMA (gfx950).
//
// Each expert is a SwiGLU FFN (moe-200m-qwen3-100b README, "Architecture
// diagram": routed and shared SwiGLU experts) with weights stacked
// [E, out, in] (SpecForge PR #930, "Why FSDP is enough here"); rows are
// grouped by expert so that the work scales with routed tokens, not with the
// number of experts (same section). Two kernels of one template:
//   gate/up : H[r, n] = silu(sum_k A[r,k] Wg[e,n,k]) * (sum_k A[r,k] Wu[e,n,k]),
//             stored in the operand dtype (bf16: rounded to nearest even);
//   down    : Y[r, n] = sum_k H[r,k] Wd[e,n,k], stored in fp32.
// Both operands are K-contiguous ([rows, K] and [N, K]): every MFMA lane reads
// 16 contiguous bytes of one row.
//
// Work decomposition
//   * A block of 256 threads (4 waves as 2 x 2) owns an output tile of BM rows
//     x BN columns; for gate/up the staged weight tile holds BN gate rows and
//     BN up rows, and each wave keeps gate and up accumulators of the same
//     (row, column) so the SwiGLU epilogue needs no exchange.
//   * K advances in stages of SB bytes per row (64 or 128). A stage is copied
//     from global memory straight into LDS (global_load_lds_dwordx4: lane i
//     of a wave writes bytes 16i..16i+15 of a 1 KB run); NBUF stage buffers
//     rotate, so a stage is requested NBUF-1 stages before it is needed.
//   * The 16-byte chunks of an LDS row are XOR-swizzled so that the 8 lanes
//     of one ds_read_b128 phase (8 consecutive rows, same logical chunk) hit
//     8 distinct bank groups. The swizzle is applied on the global side (each
//     lane fetches the chunk that belongs at its LDS position).
//   * The grid is persistent: one or two blocks per CU loop over output tiles.
//     Tiles are split into 8 contiguous ranges, one per XCD (blocks are
//     dispatched to XCDs round-robin, so block b runs on XCD b % 8), and each
//     range is walked in groups of GM row tiles x all column tiles, so the
//     blocks resident on one XCD share weight and activation tiles in that
//     XCD's L2. Row tiles come from the device-side tile list that the
//     dispatch wrote (group, m-tile); no group size travels to the host.
//   * MFMA 32 x 32 tiles: bf16 v_mfma_f32_32x32x16_bf16, fp32
//     v_mfma_f32_32x32x2_f32 (four per 16-byte chunk); accumulation in fp32.
//     A stage is SB/32 MFMA K steps; the fragments of the next K step are
//     read from LDS while the MFMAs of the current one run, and the one
//     barrier of a stage sits before its last step.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Tile configuration. SB: bytes of one row in one LDS stage (64 or 128);
// NBUF: LDS stage buffers.
template <typename DT, bool GATEUP, int BM_, int BN_, int SB_, int NBUF_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, SB = SB_, NBUF = NBUF_;
  static constexpr int NB = GATEUP ? 2 * BN : BN;  // weight rows staged per stage
  static constexpr int TM = BM / 2, TN = BN / 2;   // per wave
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32 x 32 MFMA tiles per wave
  static constexpr int NG = GATEUP ? 2 : 1;
  static constexpr int KE = SB / (int)sizeof(DT);  // K elements per stage
  static constexpr int SPS = SB / 32;              // MFMA K steps (32 bytes each) per stage
  static constexpr int CPR = SB / 16;              // 16-byte chunks per LDS row
  static constexpr int RPR = 1024 / SB;            // rows per 1 KB DMA run
  static constexpr int ROWS = BM + NB;
  static constexpr int STAGE = ROWS * SB;
  static constexpr int LPS = ROWS / (4 * RPR);     // DMA runs per wave per stage
  static constexpr int A_LOADS = BM / (4 * RPR);
  static constexpr int OCC = STAGE * NBUF > 80 * 1024 ? 1 : 2;  // blocks per CU
  static_assert(SB == 64 || SB == 128, "stage row bytes");
  static_assert(BM % (4 * RPR) == 0 && NB % (4 * RPR) == 0 && BN % (4 * RPR) == 0, "DMA runs");
  static_assert(TN % 32 == 0 && TM % 32 == 0, "tile shape");
  static_assert(NBUF >= 2 && NBUF <= 5 && STAGE * NBUF <= 160 * 1024, "LDS");
  static_assert((NBUF - 2) * LPS < 64, "vmcnt range");
  // XOR key of LDS row `row`. A ds_read_b128 of a fragment reads one logical
  // chunk of 16 consecutive rows per 16-lane phase; the key makes those 16
  // reads hit 16 distinct 16-byte bank groups of a 256-byte bank window (and
  // any 8 consecutive rows 8 distinct groups of a 128-byte window).
  //   SB = 128: bank group (row * 8 + p) % 16, p = chunk ^ key
  //   SB = 64 : bank group (row * 4 + p) % 16
  __device__ static int key(int row) {
    if constexpr (SB == 128)
      return (row & 7) ^ ((row >> 3) & 1);
    else
      return ((row >> 1) & 3) ^ ((row >> 3) & 1);
  }
  __device__ static int swz(int row, int chunk) { return row * SB + ((chunk ^ key(row)) << 4); }
};

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// XOR key of K row kr of a transposed-weight stage (rows of 2*BN bytes): a
// transposing read takes, per 16-lane group, 8 bytes from each of 4
// consecutive rows and 4 consecutive 16-byte chunks' halves; keys 0/4/8/12
// (rows of at least 16 chunks) or 0/0/4/4 (8-chunk rows, whose odd rows sit
// 128 bytes further in the bank window) put two groups' 32 reads in 32
// distinct bank pairs.
template <int BN>
__device__ __forceinline__ int tkey(int kr) {
  if constexpr (BN >= 128)
    return 4 * (kr & 3);
  else
    return 4 * ((kr >> 1) & 1);
}

// One 32 x 32 MFMA tile over the 16 bytes of K that each lane holds: lane l
// provides row l % 32 of A (and column l % 32 of B) for K group l / 32.
template <typename DT>
__device__ __forceinline__ void mfma_step(f32x16& acc, const u32x4& a, const u32x4& b);

template <>
__device__ __forceinline__ void mfma_step<uint16_t>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[q]), __uint_as_float(b[q]), acc, 0, 0, 0);
}

// Scheduling shape of one K step: MFMAs alternating with LDS reads (RD) and
// DMA issues (VM), as long as either lasts, then the remaining MFMAs.
template <int MF, int RD, int VM>
__device__ __forceinline__ void interleave() {
  constexpr int OTHER = RD + VM;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (i < VM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM read (DMA)
    if (i < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
  }
  static_assert(OTHER >= 0, "");
}

// Output element type: gate/up stores the activation in the operand type,
// down stores fp32.
template <typename DT, bool GATEUP>
struct Out {
  using T = float;
};
template <typename DT>
struct Out<DT, true> {
  using T = DT;
};

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


// GROUPED: rows come from the tile list over group offsets (routed experts);
// otherwise one dense group of g.rows rows (the shared expert).
// BWD: the backward-pass variants: gate/up that also stores the fp32
// pre-activations (GATEUP), the K-grouped weight gradients (otherwise); the
// forward kernels compile without them.
// BT (bf16, plain product): the weights are stored [K, N] per group (N
// contiguous), as the backward products dy W_down and [dG | dU] [W_gate ;
// W_up] find them; a stage holds KE rows of BN columns, and the fragment reads
// transpose them with ds_read_b64_tr_b16, so the weights need no transposed
// copy.
template <typename DT, bool GATEUP, bool GROUPED, int BM, int BN, int SB, int NBUF, bool BWD, bool BT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Cfg<DT, GATEUP, BM, BN, SB, NBUF>::OCC)))
void k_gemm(GemmLaunch g) {
  static_assert(!BT || (!GATEUP && !BWD && sizeof(DT) == 2 && SB == 128 && BN >= 64), "transposed-weight variant");
  using C = Cfg<DT, GATEUP, BM, BN, SB, NBUF>;
  __shared__ __align__(16) unsigned char lds[NBUF * C::STAGE];
  __attribute__((address_space(3))) unsigned char* const lds_as3 = (__attribute__((address_space(3))) unsigned char*)lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tiles_n = g.N / BN;
  const int64_t m_tiles = GROUPED ? (int64_t)g.n_tiles[0] : (g.rows + BM - 1) / BM;
  const int64_t total = m_tiles * n_tiles_n;
  const int per_xcd = gridDim.x / kXcd;
  const int xcd = blockIdx.x % kXcd, slot = blockIdx.x / kXcd;
  constexpr bool kg = BWD && !GATEUP && GROUPED;  // K-grouped (weight-gradient) mode
  // This XCD's range of the raster order: equal shares of the tiles, or in
  // K-grouped mode the ranges of equal work that launch_kg_setup computed
  const int64_t chunk = (total + kXcd - 1) / kXcd;
  int64_t L0 = xcd * chunk;
  int64_t L1 = L0 + chunk < total ? L0 + chunk : total;
  if (kg && g.xcd_bounds) {
    L0 = g.xcd_bounds[xcd];
    L1 = g.xcd_bounds[xcd + 1];
  }
  // Row stride of the operands: a row of K elements, or in K-grouped mode one
  // SB-byte piece (those operands are panelled: K stage s of the BM rows of
  // an A tile is one block of BM * SB bytes, the panel of the tile holds its
  // stages one after another, K capacity g.K; B likewise with BN rows)
  const size_t kbytes = kg ? (size_t)SB : (size_t)g.K * sizeof(DT);
  const int nk_all = g.K / C::KE;
  const int group_m = g.group_m > 0 ? g.group_m : kGroupM;
  // Position of this lane in a 1 KB DMA run: row lane / CPR of the run, LDS
  // chunk lane % CPR, which holds logical chunk (lane % CPR) ^ key(row).
  const int lrow = lane / C::CPR;
  // Every run this wave copies starts at an LDS row congruent to wave * RPR
  // modulo 32 (runs of 4 * RPR rows per wave set), which is all the key reads.
  const int lchunk = (lane % C::CPR) ^ C::key(wave * C::RPR + lrow);

  for (int64_t L = L0 + slot; L < L1; L += per_xcd) {
    // grouped raster: GM row tiles x every column tile
    const int64_t gsz = (int64_t)group_m * n_tiles_n;
    const int64_t first_m = (L / gsz) * group_m;
    const int64_t gm = (m_tiles - first_m) < group_m ? (m_tiles - first_m) : group_m;
    const int64_t within = L % gsz;
    const int64_t tile_m = first_m + within % gm;
    const int tile_n = (int)(within / gm);

    int grp = 0;
    int64_t row0;
    int rows;
    bool skip = false;
    int4 chunk_k = make_int4(0, 0, 0, -1);  // K-grouped: (group, first K column, end K column, slot)
    if constexpr (GROUPED) {
      const int2 t = g.tiles[tile_m];
      skip = t.x < 0 || t.x >= g.n_groups || t.y < 0;
      grp = skip ? 0 : t.x;
      if (kg) {
        chunk_k = g.vgroups[grp];
        grp = chunk_k.x;
        row0 = (int64_t)t.y * BM;
        const int64_t left = (int64_t)g.m_valid - row0;
        rows = (int)(left < BM ? left : BM);
      } else {
        row0 = (int64_t)g.offsets[grp] + (int64_t)t.y * BM;
        const int64_t left = (int64_t)g.offsets[grp + 1] - row0;
        rows = (int)(left < BM ? left : BM);
      }
    } else {
      row0 = tile_m * BM;
      const int64_t left = g.rows - row0;
      rows = (int)(left < BM ? left : BM);
    }
    if (skip || rows <= 0) continue;  // uniform across the block
    const int n0 = tile_n * BN;
    // K-grouped: the tile's panels of A and B
    const unsigned char* A = reinterpret_cast<const unsigned char*>(g.a) +
                             (kg ? (size_t)row0 * g.K * sizeof(DT) : (size_t)0);
    const bool xg = grp == g.extra_group;
    // K range of this tile: the whole K, or the chunk's columns (K-grouped)
    const int nk = kg ? (chunk_k.z - chunk_k.y) / C::KE : nk_all;
    const int64_t st0 = kg ? (int64_t)chunk_k.y / C::KE : 0;  // first K stage of the chunk
    const unsigned char* B0 = kg ? reinterpret_cast<const unsigned char*>(g.b0) + (size_t)n0 * g.K * sizeof(DT)
                              : xg ? reinterpret_cast<const unsigned char*>(g.bx0)
                                   : reinterpret_cast<const unsigned char*>(g.b0) + (size_t)grp * g.N * kbytes;
    const unsigned char* B1 = !GATEUP ? B0
                              : xg    ? reinterpret_cast<const unsigned char*>(g.bx1)
                                      : reinterpret_cast<const unsigned char*>(g.b1) + (size_t)grp * g.N * kbytes;
    // BT: this group's [K, N] weights, K rows below bt_ksplit from b0 (bx0),
    // the rest from b1 (bx1)
    const size_t ldb = (size_t)g.N * 2;
    const int64_t kfirst = g.bt_ksplit > 0 ? g.bt_ksplit : g.K;
    const unsigned char* T0 = xg ? reinterpret_cast<const unsigned char*>(g.bx0)
                                 : reinterpret_cast<const unsigned char*>(g.b0) + (size_t)grp * kfirst * ldb;
    const unsigned char* T1 = xg ? reinterpret_cast<const unsigned char*>(g.bx1)
                                 : reinterpret_cast<const unsigned char*>(g.b1) + (size_t)grp * (g.K - kfirst) * ldb;

    // Source row of each A run of this lane. Rows past the tile's end read a
    // valid row; their results are never stored. Weight rows are addressed
    // from one block-uniform base plus a per-lane offset.
    int32_t a_row[C::A_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      int r = (i * 4 + wave) * C::RPR + lrow;
      r = r < rows ? r : rows - 1;
      int64_t src_row = kg ? r : row0 + r;
      if (g.a_rows) {
        src_row = g.a_rows[src_row];
        src_row = src_row < 0 ? 0 : (src_row >= g.a_row_count ? g.a_row_count - 1 : src_row);
      }
      a_row[i] = (int32_t)src_row;
    }
    const unsigned char* bbase0 = kg ? B0 : B0 + (size_t)n0 * kbytes;
    const unsigned char* bbase1 = kg ? B1 : B1 + (size_t)n0 * kbytes;
    const uint32_t lane_off = (uint32_t)((wave * C::RPR + lrow) * kbytes) + lchunk * 16;
    auto issue = [&](int kt) {
      unsigned char* sb = lds + (kt % NBUF) * C::STAGE + wave * C::RPR * SB;
      const size_t off_a = kg ? (size_t)(st0 + kt) * BM * SB : (size_t)kt * SB;
      const size_t off_b = kg ? (size_t)(st0 + kt) * BN * SB : (size_t)kt * SB;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i)
        lds_dma16(A + (size_t)(uint32_t)a_row[i] * kbytes + off_a + lchunk * 16, sb + i * 4 * C::RPR * SB);
      if constexpr (BT) {
        // KE rows of 2*BN bytes; 1 KB run r of the region holds bytes
        // r*1024 .. of it, lane l's 16 bytes at physical chunk pc of row kr,
        // which takes logical chunk pc ^ tkey(kr)
        const int k0 = kt * C::KE;
        const bool second = g.bt_ksplit > 0 && k0 >= g.bt_ksplit;
        const unsigned char* tb = second ? T1 + (size_t)(k0 - g.bt_ksplit) * ldb : T0 + (size_t)k0 * ldb;
        tb += (size_t)n0 * 2;
#pragma unroll
        for (int i = C::A_LOADS; i < C::LPS; ++i) {
          const int byte = ((i - C::A_LOADS) * 4 + wave) * 1024 + lane * 16;
          const int kr = byte / (2 * BN), pc = (byte % (2 * BN)) >> 4;
          const unsigned char* src = tb + (size_t)kr * ldb + ((pc ^ tkey<BN>(kr)) << 4);
          if (g.b_stream)
            lds_dma16<true>(src, sb + i * 4 * C::RPR * SB);
          else
            lds_dma16(src, sb + i * 4 * C::RPR * SB);
        }
        return;
      }
#pragma unroll
      for (int i = C::A_LOADS; i < C::LPS; ++i) {
        const int rb0 = (i - C::A_LOADS) * 4 * C::RPR;
        const unsigned char* src = (GATEUP && rb0 >= BN) ? bbase1 + (size_t)(rb0 - BN) * kbytes
                                                         : bbase0 + (size_t)rb0 * kbytes;
        if (g.b_stream)
          lds_dma16<true>(src + lane_off + off_b, sb + i * 4 * C::RPR * SB);
        else
          lds_dma16(src + lane_off + off_b, sb + i * 4 * C::RPR * SB);
      }
    };

    f32x16 acc[C::NG][C::FM][C::FN];
#pragma unroll
    for (int h = 0; h < C::NG; ++h)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[h][i][j][e] = 0.0f;

    // Fragments of one K step (s = 0 or 1 of a stage): FM A tiles and
    // NG x FN weight tiles; lane l reads row l % 32, logical chunk 2s + l/32.
    struct Frag {
      u32x4 a[C::FM];
      u32x4 b[C::NG][C::FN];
    };
    auto load_frag = [&](Frag& f, int kt, int s) {
      const unsigned char* base = lds + (kt % NBUF) * C::STAGE;
      const int ch = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        f.a[i] = *reinterpret_cast<const u32x4*>(base + C::swz(wm * C::TM + i * 32 + (lane & 31), ch));
      if constexpr (BT) {
        // lane l: column l % 32 of the 32-column tile, K rows 16s + 8(l/32)
        // + 0..7 as two transposing reads of 4 rows; within each 16-lane
        // group, lane L addresses row L/4 of the 4 and columns 4(L%4) .. +3
        const int grp16 = lane >> 4, L = lane & 15;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int n = wn * C::TN + j * 32 + 16 * (grp16 & 1) + 4 * (L & 3);
          const int c = n >> 3, half = (n >> 2) & 1;
          u32x2 q[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int kr = 16 * s + 8 * (grp16 >> 1) + 4 * t + (L >> 2);
            const int off = BM * SB + kr * (2 * BN) + ((c ^ tkey<BN>(kr)) << 4) + half * 8;
            q[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (__attribute__((address_space(3))) v4i16*)(lds_as3 + (base - lds) + off)));
          }
          f.b[0][j] = u32x4{q[0][0], q[0][1], q[1][0], q[1][1]};
        }
        return;
      }
#pragma unroll
      for (int h = 0; h < C::NG; ++h)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          f.b[h][j] =
              *reinterpret_cast<const u32x4*>(base + C::swz(BM + h * BN + wn * C::TN + j * 32 + (lane & 31), ch));
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
      for (int h = 0; h < C::NG; ++h)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) mfma_step<DT>(acc[h][i][j], f.a[i], f.b[h][j]);
    };
    // Wait until stage kt+1 has landed while `ahead` later stages stay in
    // flight, and until this wave's fragment reads are done.
    auto wait_stage = [&](int ahead) {
      if (ahead >= 3 && NBUF >= 5)
        wait_vm_lgkm0<(NBUF >= 5 ? 3 : 0) * C::LPS>();
      else if (ahead >= 2 && NBUF >= 4)
        wait_vm_lgkm0<(NBUF >= 4 ? 2 : 0) * C::LPS>();
      else if (ahead >= 1 && NBUF >= 3)
        wait_vm_lgkm0<(NBUF >= 3 ? 1 : 0) * C::LPS>();
      else
        wait_vm_lgkm0<0>();
    };

    // Pipeline: NBUF LDS stages, two fragment sets P and Q alternating over
    // the SPS K steps of a stage (SPS is even, so step 0 always uses P).
    // Step s < SPS-1: MFMAs of step s with the LDS reads of step s+1 (into the
    // other set) interleaved one by one, so the reads complete under the
    // MFMAs instead of in front of them.
    // Last step: wait for stage kt+1 and for this wave's reads, barrier (every
    // wave is done with stage kt, so its buffer takes stage kt + NBUF); then
    // the MFMAs of the last step with that stage's DMA issues and the reads of
    // step 0 of stage kt+1 (into P) interleaved.
    Frag P, Q;
#pragma unroll
    for (int q = 0; q < NBUF; ++q)
      if (q < nk) issue(q);
    {
      const int ahead = (nk < NBUF ? nk : NBUF) - 1;  // stages issued after stage 0
      if (ahead >= 4)
        wait_vm<(NBUF >= 5 ? 4 : 0) * C::LPS>();
      else if (ahead == 3)
        wait_vm<(NBUF >= 4 ? 3 : 0) * C::LPS>();
      else if (ahead == 2)
        wait_vm<(NBUF >= 3 ? 2 : 0) * C::LPS>();
      else if (ahead == 1)
        wait_vm<C::LPS>();
      else
        wait_vm<0>();
    }
    __syncthreads();
    load_frag(P, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int s = 0; s < C::SPS; ++s) {
        Frag& cur = (s & 1) ? Q : P;
        Frag& nxt = (s & 1) ? P : Q;
        if (s + 1 < C::SPS) {
          load_frag(nxt, kt, s + 1);
          mma(cur);
          interleave<C::NG * C::FM * C::FN, C::FM + (BT ? 2 : 1) * C::NG * C::FN, 0>();
        } else {
          // stages in flight beyond kt+1: kt+2 .. min(kt+NBUF-1, nk-1)
          const int last = (kt + NBUF - 1 < nk - 1) ? kt + NBUF - 1 : nk - 1;
          wait_stage(last - (kt + 1));
          __syncthreads();
          __builtin_amdgcn_sched_barrier(0);
          if (kt + NBUF < nk) issue(kt + NBUF);
          if (kt + 1 < nk) load_frag(nxt, kt + 1, 0);
          mma(cur);
          interleave<C::NG * C::FM * C::FN, C::FM + (BT ? 2 : 1) * C::NG * C::FN, C::LPS>();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // every wave is done with the stage buffers

    // Epilogue, one 32 x 32 accumulator tile at a time. Element e of a tile
    // sits in row 8*(e/4) + 4*(l/32) + e%4 and column l % 32 of lane l; the
    // wave writes the tile (converted to the output type) to its own LDS
    // scratch, row-major with padded rows, and reads it back as 16-byte row
    // chunks, so that each store covers contiguous columns. `row_ptr(m)` is
    // the output row of tile row m; rows at or past `rows` are not stored.
    {
      static_assert(4 * 32 * (32 * 4 + 16) <= NBUF * C::STAGE, "epilogue scratch");
      unsigned char* scr = lds + wave * 32 * (32 * 4 + 16);
      auto put_tile = [&](auto zero, const f32x16& v, int i, int j, auto row_ptr) {
        using T = decltype(zero);
        constexpr int EB = (int)sizeof(T), P = 32 * EB + 16, CH = 32 * EB / 16;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          T o;
          if constexpr (sizeof(T) == 2)
            o = f32_to_bf16(v[e]);
          else
            o = v[e];
          *reinterpret_cast<T*>(scr + r * P + (lane & 31) * EB) = o;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int q0 = 0; q0 < 32 * CH; q0 += 64) {
          const int q = q0 + lane, r = q / CH, c16 = q % CH;
          const u32x4 val = *reinterpret_cast<const u32x4*>(scr + r * P + c16 * 16);
          const int m = wm * C::TM + i * 32 + r;
          const int n = n0 + wn * C::TN + j * 32 + c16 * (16 / EB);
          if (m < rows) {
            if constexpr (kg)  // weight gradients and partials: streaming stores (measured faster)
              __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(row_ptr(m) + (size_t)n * EB));
            else
              *reinterpret_cast<u32x4*>(row_ptr(m) + (size_t)n * EB) = val;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
      using OT = typename Out<DT, GATEUP>::T;
      auto plain_row = [&](void* base, int eb) {
        return [=](int m) { return reinterpret_cast<unsigned char*>(base) + (size_t)(row0 + m) * g.N * eb; };
      };
      // K-grouped output rows: row row0 + m of group grp's m_rows, or of the
      // chunk's partial-buffer slot
      auto kg_row = [&](int m) {
        const int mm = (int)row0 + m;
        float* p = chunk_k.w >= 0 ? g.part + ((size_t)chunk_k.w * g.m_rows + mm) * g.N : kg_out_row(g, grp, mm);
        return reinterpret_cast<unsigned char*>(p);
      };
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          if constexpr (GATEUP) {
            f32x16 hv;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float gv = acc[0][i][j][e], uv = acc[1][i][j][e];
              hv[e] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
            }
            put_tile(OT{}, hv, i, j, plain_row(g.out, (int)sizeof(OT)));
            if (BWD && g.out_g) {
              put_tile(float{}, acc[0][i][j], i, j, plain_row(g.out_g, 4));
              put_tile(float{}, acc[1][i][j], i, j, plain_row(g.out_u, 4));
            }
          } else {
            if (kg)
              put_tile(float{}, acc[0][i][j], i, j, kg_row);
            else
              put_tile(float{}, acc[0][i][j], i, j, plain_row(g.out, 4));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __syncthreads();  // scratch reads done before the next tile's DMA
  }
}

template <typename DT, bool GATEUP, int BM, int BN, int SB, int NBUF, bool BWD = false, bool BT = false>
hipError_t launch_t(const GemmLaunch& g, hipStream_t s) {
  using C = Cfg<DT, GATEUP, BM, BN, SB, NBUF>;
  if (g.N % BN || (!g.koffs && g.K % C::KE)) return hipErrorInvalidValue;
  int64_t blocks = (int64_t)cu_count() * C::OCC;
  blocks = (blocks + kXcd - 1) / kXcd * kXcd;
  if (!g.offsets) {
    // dense: no more blocks than tiles (rounded up to whole XCD groups)
    const int64_t tiles = (g.rows + BM - 1) / BM * (g.N / BN);
    if (tiles <= 0) return hipSuccess;
    const int64_t need = (tiles + kXcd - 1) / kXcd * kXcd;
    blocks = need < blocks ? need : blocks;
  }
  if (g.offsets)
    hipLaunchKernelGGL((k_gemm<DT, GATEUP, true, BM, BN, SB, NBUF, BWD, BT>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm<DT, GATEUP, false, BM, BN, SB, NBUF, BWD, BT>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}


// Rows per busy group up to which a grouped product counts as a batch of a
// few tokens (gemm_bm, gemm_bn_caps).
constexpr int64_t kFewRows = 32;

// Row tile of a grouped GEMM: 256 rows when groups are long enough to fill
// such tiles and there are enough of them to give every CU several (the
// persistent grid has one 256-row block per CU), else 128 (less padding in
// short groups, four times as many tiles).
int gemm_bm(int dtype, int64_t rows, int64_t groups, int n, int d_in) {
  if (dtype != 1 || groups <= 0) return 128;
  const int64_t avg = rows / groups;
  // Few rows per group (small batches, many experts): the weights dominate
  // the traffic, and 64-row tiles with wider weight tiles stage fewer
  // padding rows per weight byte, as long as their tiles still give every
  // block slot of the persistent grid one (else more, narrower tiles win;
  // at most `rows` groups hold rows). Measured up to 128 rows per group:
  // 3-6% faster than 128-row tiles at 72-112 rows of 256 experts with
  // d_in 7168, 3% at 96-128 rows of 128 experts with d_in 2048.
  const int64_t busy = groups < rows ? groups : rows;
  const int64_t tiles64 = busy * (n % 128 == 0 ? n / 128 : n / 64);
  if (avg <= 128 && tiles64 >= 2 * (int64_t)cu_count()) return 64;
  // A handful of rows per busy group (batches of a few tokens): every row
  // tile is mostly padding, and its padding rows cost copies like weight
  // rows do, so the shortest tile wins; gemm_bn_caps then narrows the weight
  // tiles so that the few groups still spread over every CU.
  if (rows <= kFewRows * busy) return 64;
  // 256-row tiles read each weight panel once per group: they pay for their
  // padding with many rows per group, or with a long K, where a 128-row
  // pair re-reads multi-MB panels that do not stay in L2 (d_in 7168: 3% at
  // 144 rows per group, 1% at 288; d_in 2048 at 256 rows: 7% slower)
  const int64_t tiles256 = (rows / 256) * (n / 128);
  const bool long_k = d_in >= 4096;
  return ((avg >= 768 || long_k) && tiles256 >= 4 * (int64_t)cu_count()) ? 256 : 128;
}

// Row tile of the forward products: gemm_bm, except where the eight-wave
// 256 x 256 kernel (gemm8.hip) runs both products (gate/up N % 128, down N =
// d_in % 256): its 256-row tiles then win from 65 rows per group on average
// as long as the row tiles give every CU two column strips (step times,
// Qwen3-like layer at 2,048 / 4,096 / 8,192 tokens: 0.492 -> 0.416, 0.701 ->
// 0.622, 1.18 -> 0.98 ms; DeepSeek-style at 2,048 / 3,072: 5.86 -> 5.73,
// 7.11 -> 6.27 ms; iso-width at 512 / 1,024: 0.79 -> 0.67, 1.09 -> 0.84 ms;
// the large layers' full batches already took these tiles), and with a K of
// 2048 or more and many experts 128-row tiles beat 64-row ones above 48 rows
// per group (DeepSeek-style at 1,536 tokens 5.61 -> 5.05 ms, Qwen3-like at
// 1,024 0.396 -> 0.339 ms; the iso-width layer's 16 experts at 64 rows each
// were 10% slower with them).
int gemm_bm_fwd(int dtype, int64_t rows, int64_t groups, int n, int d_in) {
  const int bm = gemm_bm(dtype, rows, groups, n, d_in);
  if (dtype != 1 || groups <= 0 || bm == 256) return bm;
  const int64_t busy = groups < rows ? groups : rows;
  if (rows <= kFewRows * busy) return bm;  // a few tokens
  const int64_t avg = rows / groups;
  const bool fits8 = n % 128 == 0 && d_in % 256 == 0 && n >= 3 * 64 && d_in >= 3 * 64;
  const int64_t row_tiles = rows / 256 > busy ? rows / 256 : busy;
  if (fits8 && avg > 64 && row_tiles * (n / 128) >= 2 * (int64_t)cu_count()) return 256;
  if (bm == 64 && avg > 48 && d_in >= 2048 && groups >= 64) return 128;
  return bm;
}

// Column-tile caps: none (0) unless gemm_bm took 64-row tiles for a handful
// of rows per busy group where the widest tiles would not give every block
// slot one; then gate/up and down each take the widest tile whose count over
// the busy groups still spreads over every CU (measured against 128-row
// tiles at 1-3 tokens of the DeepSeek-style layer: step 0.236 -> 0.215,
// 0.393 -> 0.334, 0.466 -> 0.415 ms; 1 token of the Qwen3-like layer 0.079
// -> 0.065 ms).
GemmCaps gemm_bn_caps(int dtype, int64_t rows, int64_t groups, int n, int d_in, int d_out) {
  GemmCaps c{0, 0};
  if (dtype != 1 || groups <= 0 || gemm_bm_fwd(dtype, rows, groups, n, d_in) != 64) return c;
  const int64_t busy = groups < rows ? groups : rows;
  if (rows / groups <= 128 && busy * (n % 128 == 0 ? n / 128 : n / 64) >= 2 * (int64_t)cu_count()) return c;
  // the widest tile whose count reaches `want`, else the narrowest: gate/up
  // one tile per CU (measured at 2 tokens of the DeepSeek-style layer: 288
  // tiles of 128 columns 186 us, 576 of 64 columns 191 us), down, whose K is
  // the short d_ff, one and a half (1 token of the DeepSeek-style layer: 504
  // tiles of 128 columns 43 us, 1008 of 64 columns 45 us; 2 tokens of the
  // Qwen3-like layer: 256 tiles of 128 columns 16.5 us, 512 of 64 12.2 us)
  auto cap = [&](int n_out, int widest, int64_t want) {
    for (int bn = widest; bn > 64; bn /= 2)
      if (n_out % bn == 0 && busy * (n_out / bn) >= want) return bn;
    return 64;
  };
  c.gateup = cap(n, 128, cu_count());
  c.down = cap(d_out, 256, 3 * (int64_t)cu_count() / 2);
  return c;
}

// Row tile of a K-grouped (weight-gradient) GEMM: bf16 takes 256 x 256 tiles
// when m_rows and n divide and there are several such tiles per CU (each
// tile then runs a group's whole K), else the largest of 128 and 64 that
// divides m_rows.
int gemm_kg_bm(int dtype, int m_rows, int n, int groups) {
  if (dtype == 1 && m_rows % 256 == 0 && n % 256 == 0 &&
      (int64_t)groups * (m_rows / 256) * (n / 256) >= 4 * (int64_t)cu_count())
    return 256;
  return m_rows % 128 == 0 ? 128 : 64;
}

// Column tile of a K-grouped launch: 256 with 256-row tiles, else the wider
// of 128 and 64 that divides n.
int gemm_kg_bn(int bm, int n) { return bm == 256 ? 256 : (n % 128 == 0 ? 128 : 64); }

// Chunk length: the average K stages per persistent block (one block per CU
// for 256-row tiles, two otherwise), at least 16, so that a long group's
// tiles do not outlast the rest of the launch.
int gemm_kg_cap(int bm, int64_t stages, int mt, int ntn) {
  const int64_t slots = (int64_t)cu_count() * (bm == 256 ? 1 : 2);
  const int64_t avg = (stages * mt * ntn + slots - 1) / slots;
  return (int)(avg < 16 ? 16 : (avg > (1 << 30) ? (1 << 30) : avg));
}

// gate/up: BN columns of H (gate and up rows staged together); down: BN output
// columns. The widest tile that divides N. K-grouped launches (weight
// gradients) take the row tile bm from gemm_kg_bm.
hipError_t launch_gemm(const GemmLaunch& g, int bm, hipStream_t s) {
  if (g.koffs) {
    if (g.gateup || g.N % 64 || (bm != 64 && bm != 128 && bm != 256) || g.m_rows % bm) return hipErrorInvalidValue;
    if (bm == 256 && (g.dtype != 1 || g.N % 256)) return hipErrorInvalidValue;
    const bool wide = gemm_kg_bn(bm, g.N) == 128, tall = bm == 128;
    if (bm == 256) return launch_t<uint16_t, false, 256, 256, 128, 2, true>(g, s);
    if (g.dtype == 1) {
      if (tall)
        return wide ? launch_t<uint16_t, false, 128, 128, 128, 2, true>(g, s)
                    : launch_t<uint16_t, false, 128, 64, 128, 2, true>(g, s);
      return wide ? launch_t<uint16_t, false, 64, 128, 128, 2, true>(g, s)
                  : launch_t<uint16_t, false, 64, 64, 128, 2, true>(g, s);
    }
    if (tall)
      return wide ? launch_t<float, false, 128, 128, 128, 2, true>(g, s) : launch_t<float, false, 128, 64, 128, 2, true>(g, s);
    return wide ? launch_t<float, false, 64, 128, 128, 2, true>(g, s) : launch_t<float, false, 64, 64, 128, 2, true>(g, s);
  }
  if (bm == 64 && (g.dtype != 1 || g.koffs)) return hipErrorInvalidValue;
  if (g.bt) {  // weights stored [K, N]
    if (g.dtype != 1 || g.gateup || g.out_g || g.bt_ksplit < 0 || g.bt_ksplit % 64 || g.bt_ksplit >= g.K ||
        (g.extra_group >= 0 && !g.bx0) || (g.bt_ksplit > 0 && (!g.b1 || (g.extra_group >= 0 && !g.bx1))))
      return hipErrorInvalidValue;
    if (bm == 64) {
      if (g.N % 256 == 0) return launch_t<uint16_t, false, 64, 256, 128, 2, false, true>(g, s);
      if (g.N % 128 == 0) return launch_t<uint16_t, false, 64, 128, 128, 2, false, true>(g, s);
      return launch_t<uint16_t, false, 64, 64, 128, 2, false, true>(g, s);
    }
    if (bm == 256) {
      if (g.N % 256 == 0) return launch_t<uint16_t, false, 256, 256, 128, 2, false, true>(g, s);
      if (g.N % 128 == 0) return launch_t<uint16_t, false, 256, 128, 128, 2, false, true>(g, s);
      return launch_t<uint16_t, false, 256, 64, 128, 2, false, true>(g, s);
    }
    if (g.N % 128 == 0) return launch_t<uint16_t, false, 128, 128, 128, 2, false, true>(g, s);
    return launch_t<uint16_t, false, 128, 64, 128, 2, false, true>(g, s);
  }
  if (g.out_g) {  // gate/up that also stores the pre-activations (backward recompute)
    if (!g.gateup) return hipErrorInvalidValue;
    if (g.dtype == 1) {
      if (bm == 64)
        return g.N % 128 == 0 ? launch_t<uint16_t, true, 64, 128, 128, 2, true>(g, s)
                              : launch_t<uint16_t, true, 64, 64, 128, 2, true>(g, s);
      if (bm == 256 && g.N % 128 == 0) return launch_t<uint16_t, true, 256, 128, 128, 2, true>(g, s);
      if (bm == 256) return launch_t<uint16_t, true, 256, 64, 128, 2, true>(g, s);
      return launch_t<uint16_t, true, 128, 64, 128, 2, true>(g, s);
    }
    return launch_t<float, true, 128, 64, 128, 2, true>(g, s);
  }
  if (g.dtype == 1) {
    if (bm == 64) {
      // bn_cap set (a handful of rows per group): the narrowest tiles take a
      // third stage buffer, so that each block keeps two weight stages in
      // flight (measured at 1-2 tokens: DeepSeek-style gate/up 111 -> 104
      // and 227 -> 186 us, Qwen3-like 1-token step 75 -> 65 us; with 64 x 128
      // down tiles it was 3 us slower)
      const int cap = g.bn_cap > 0 ? g.bn_cap : 256;
      const bool deep = g.bn_cap > 0;
      if (g.gateup) {
        if (g.N % 128 == 0 && cap >= 128) return launch_t<uint16_t, true, 64, 128, 128, 2>(g, s);
        return deep ? launch_t<uint16_t, true, 64, 64, 128, 3>(g, s) : launch_t<uint16_t, true, 64, 64, 128, 2>(g, s);
      }
      if (g.N % 256 == 0 && cap >= 256) return launch_t<uint16_t, false, 64, 256, 128, 2>(g, s);
      if (g.N % 128 == 0 && cap >= 128) return launch_t<uint16_t, false, 64, 128, 128, 2>(g, s);
      return deep ? launch_t<uint16_t, false, 64, 64, 128, 3>(g, s) : launch_t<uint16_t, false, 64, 64, 128, 2>(g, s);
    }
    if (g.gateup) {
      if (bm == 256 && g.N % 128 == 0) return launch_t<uint16_t, true, 256, 128, 128, 2>(g, s);
      if (bm == 256) return launch_t<uint16_t, true, 256, 64, 128, 2>(g, s);
      return launch_t<uint16_t, true, 128, 64, 128, 2>(g, s);
    }
    if (bm == 256) {
      if (g.N % 256 == 0) return launch_t<uint16_t, false, 256, 256, 128, 2>(g, s);
      if (g.N % 128 == 0) return launch_t<uint16_t, false, 256, 128, 128, 2>(g, s);
      return launch_t<uint16_t, false, 256, 64, 128, 2>(g, s);
    }
    if (g.N % 128 == 0) return launch_t<uint16_t, false, 128, 128, 128, 2>(g, s);
    return launch_t<uint16_t, false, 128, 64, 128, 2>(g, s);
  }
  if (g.gateup) return launch_t<float, true, 128, 64, 128, 2>(g, s);
  if (g.N % 128 == 0) return launch_t<float, false, 128, 128, 128, 2>(g, s);
  return launch_t<float, false, 128, 64, 128, 2>(g, s);
}

}  // namespace moe
