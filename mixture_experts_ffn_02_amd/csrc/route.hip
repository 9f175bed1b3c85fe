// Router kernel: fp32 gate product, scores, wavefront top-k, combine weights,
// and the per-block expert histogram and ranks used by the dispatch.
//
// The layer's router runs in fp32 whatever the activation dtype
// (moe-200m-qwen3-100b README, "Per-layer numerics"; "SigmoidRouter":
// logits, sigmoid, bias for selection only, topk, weight gather and
// renormalisation; SpecForge PR #930, "What this adds": softmax over all
// experts with renormalised top-k weights).
//
// This file is compiled with -ffp-contract=off, IEEE division and fp32
// denormals kept, so that every value that decides an expert id is a fixed
// sequence of IEEE operations:
//   * logits: one fma chain per (token, expert), features ascending, from +0;
//   * exp: canonical_exp below (Cody-Waite reduction, Taylor degree 7);
//   * softmax normaliser: summed over experts in ascending order.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// exp(a) in fp32 from +, -, *, / and fma only.
//  n = rint(a * log2 e); r = a - n*ln2 with ln2 = hi + lo (hi = ln2 rounded to
//  fp32, lo = the fp32 rounding of the remainder), one fma each (Cody & Waite
//  1980); exp(r) = Taylor series to r^7 in Horner form; scale by 2^n built
//  from its exponent bits, in two steps when 2^n is not a normal fp32 so that
//  only the last multiply rounds.
__device__ __forceinline__ float canonical_exp(float a) {
  if (a != a) return a;
  if (a > 88.72283935546875f) return __builtin_inff();
  if (a < -103.972084045410f) return 0.0f;
  const float n = __builtin_rintf(a * 1.44269504088896340736f);
  float r = __builtin_fmaf(-n, 0.693147182464599609375f, a);
  r = __builtin_fmaf(-n, -1.9046542121259336e-09f, r);
  float p = 1.0f / 5040.0f;
  p = __builtin_fmaf(p, r, 1.0f / 720.0f);
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const int ni = (int)n;
  if (ni > 127) return (p * 2.0f) * __uint_as_float((uint32_t)(ni - 1 + 127) << 23);
  if (ni < -126)
    return (p * __uint_as_float((uint32_t)(ni + 64 + 127) << 23)) * __uint_as_float((uint32_t)(127 - 64) << 23);
  return p * __uint_as_float((uint32_t)(ni + 127) << 23);
}

__device__ __forceinline__ float sigmoid_canon(float l) { return 1.0f / (1.0f + canonical_exp(-l)); }

// Orderable 64-bit key: larger value first, then lower expert id.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  v = v + 0.0f;  // -0 -> +0, so that the two zeros tie
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N - 1 (unrolled,
// with every i a compile-time constant).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// acc += (w of lane L of this lane's 16-lane row) * x: v_fmac_f32 with a DPP
// row_newbcast operand. w must not be written by a VALU instruction right
// before (the DPP read hazard): here it always comes from a memory load.
template <int L>
__device__ __forceinline__ void fmac_bcast(float& acc, float w, float x) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(w), "v"(x), "n"(L));
}

// Launch shape per padded expert count EP (power of two, 8..1024):
//   ME experts x MT tokens per thread, EG expert groups x TG token groups
//   = 256 threads, TT = TG*MT tokens per block, at most KC features per LDS
//   stage (a stage holds KC features when KC divides d, else 64; d is a
//   multiple of 64).
template <int EP>
struct RouteShape;
#define ROUTE_SHAPE(EP_, ME_, MT_, KC_)                        \
  template <>                                                  \
  struct RouteShape<EP_> {                                     \
    static constexpr int ME = ME_, MT = MT_, KC = KC_;         \
    static constexpr int EG = EP_ / ME_, TG = 256 / (EP_ / ME_); \
    static constexpr int TT = (256 / (EP_ / ME_)) * MT_;       \
  };
// Few tokens per block (16-128) so that even the smaller layers spread over
// every CU. With few experts the block is 16 or 32 tokens and a stage is up
// to 128 features: the loop over d then has few stages, each of which waits
// for its loads once (16 experts: one chain per thread and 16-token blocks,
// two blocks per CU at 8192 tokens, measured faster than 32-token blocks;
// 128 experts: two tokens per thread, 32-token blocks, measured faster than
// one or four). At 256 experts the stage is 16 features so that two blocks
// fit in one CU's LDS.
ROUTE_SHAPE(8, 1, 1, 128)
ROUTE_SHAPE(16, 1, 1, 128)
ROUTE_SHAPE(32, 4, 1, 128)
ROUTE_SHAPE(64, 8, 1, 64)
ROUTE_SHAPE(128, 8, 2, 32)
ROUTE_SHAPE(256, 8, 8, 16)
ROUTE_SHAPE(512, 16, 4, 16)
ROUTE_SHAPE(1024, 16, 4, 8)
#undef ROUTE_SHAPE

// Tokens per block of the selection that reads stored logits (split path):
// there is no gate product to share, so small blocks spread over the chip.
constexpr int kSelTT = 16;

// Gate product with the router weights broadcast from registers (up to 32
// experts, many tokens): a block holds 64 tokens, lane l of each wave owns
// token l, and wave w the experts w*EP/4 .. (w+1)*EP/4 - 1 (ME = EP/4
// chains per lane). Token rows are staged in fp32 through LDS (kDppKC
// features per stage); the router weights go straight from memory into
// registers, each 16-lane row of a wave holding the wave's ME experts x
// 16/ME runs of 4 features, and every fma reads its weight from the lane
// that holds it with a DPP row_share operand (d a multiple of kDppKC). Per fma a lane reads 1 byte of
// LDS (a token's 4 features serve 4 x ME fmas) where the LDS-staged shapes
// read 4-8.
constexpr int kDppTT = 64;
constexpr int kDppKC = 128;
constexpr int kDppPitch = kDppKC + 4;  // floats; 16 lanes' rows fall 16 bytes apart in the banks

template <int EP, bool FROM_LOGITS = false, bool DPP = false>
struct RouteLds {
  using S = RouteShape<EP>;
  static constexpr int TT = FROM_LOGITS ? kSelTT : (DPP ? kDppTT : S::TT);
  // One token per thread (MT = 1): stage rows are token- and expert-major,
  // padded by 4 floats, so that a lane reads 4 features with one 16-byte
  // load. Otherwise feature-major ([feature][token] and [feature][expert]).
  static constexpr bool kRows = S::MT == 1;
  static constexpr int kPitch = kRows ? S::KC + 4 : S::KC;
  static constexpr int kStage = FROM_LOGITS ? 0 : (DPP ? 2 * kDppPitch * kDppTT : 2 * kPitch * (S::TT + EP));  // floats
  static constexpr int kLogits = TT * (EP + 1);                               // floats
  static constexpr int kUnion = kStage > kLogits ? kStage : kLogits;
  static constexpr int kWords = (TT + 63) / 64;
  static size_t bytes(int k) {
    return sizeof(float) * kUnion + sizeof(uint64_t) * EP * kWords + sizeof(int) * TT * k +
           sizeof(float) * (EP + 2 * TT);
  }
};

template <typename XT>
struct XLoad;
template <>
struct XLoad<uint16_t> {
  static constexpr int V = 8;  // elements per 16-byte load
  __device__ static void widen(const u32x4& r, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(r[i] << 16);
      o[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct XLoad<float> {
  static constexpr int V = 4;
  __device__ static void widen(const u32x4& r, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(r[i]);
  }
};

// Ranks of a block's (token, slot) pairs within their expert, and the block's
// expert histogram, from the chosen ids in LDS (sel[tt*k + j]). Bit tt of
// masks[e*W + tt/64] marks that token tt of the block chose e; the rank of
// (tt, e) is the number of marked tokens before tt. Integer OR is order-free,
// so the result is deterministic.
__device__ void block_hist_rank(const int* sel, int tt_count, int k, int E, int W, uint64_t* masks,
                                int32_t* hist_row, int32_t* rank_out) {
  for (int q = threadIdx.x; q < tt_count * k; q += blockDim.x) {
    const int tt = q / k, e = sel[q];
    atomicOr((unsigned long long*)&masks[e * W + (tt >> 6)], 1ull << (tt & 63));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int h = 0;
    for (int w = 0; w < W; ++w) h += __popcll(masks[e * W + w]);
    hist_row[e] = h;
  }
  if (!rank_out) return;
  for (int q = threadIdx.x; q < tt_count * k; q += blockDim.x) {
    const int tt = q / k, e = sel[q];
    int r = 0;
    for (int w = 0; w < (tt >> 6); ++w) r += __popcll(masks[e * W + w]);
    r += __popcll(masks[e * W + (tt >> 6)] & ((1ull << (tt & 63)) - 1ull));
    rank_out[q] = r;
  }
}

// FROM_LOGITS: the logits were computed by k_logits into p.logits [T, E];
// otherwise the gate product runs here, fused with the selection.
template <int EP, typename XT, bool FROM_LOGITS, bool DPP = false>
__global__ __launch_bounds__(256) void k_route(RouteLaunch p) {
  using S = RouteShape<EP>;
  using L = RouteLds<EP, FROM_LOGITS, DPP>;
  constexpr int ME = S::ME, MT = S::MT, KC = S::KC, EG = S::EG, TG = S::TG, TT = L::TT;
  // features per register group of the gate-product loop (fewer when a
  // thread holds many chains, to bound the registers)
  constexpr int U = (ME * MT <= 4) ? 8 : ((ME * MT <= 16) ? 4 : 2);
  static_assert(!RouteLds<EP>::kRows || U % 4 == 0, "row layout reads 4 features at a time");
  constexpr int V = XLoad<XT>::V;
  constexpr int W = L::kWords;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  float* uni = reinterpret_cast<float*>(lds_raw);
  uint64_t* masks = reinterpret_cast<uint64_t*>(uni + L::kUnion);
  int* sel = reinterpret_cast<int*>(masks + EP * W);
  float* bias_s = reinterpret_cast<float*>(sel + TT * p.k);
  float* tok_m = bias_s + EP;
  float* tok_z = tok_m + TT;

  const int tid = threadIdx.x;
  const int E = p.E, k = p.k, d = p.d;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int tt_count = (int)((p.T - t0) < TT ? (p.T - t0) : TT);
  const XT* __restrict__ x = reinterpret_cast<const XT*>(p.x);
  const float* __restrict__ wr = p.w_router;

  for (int e = tid; e < EP; e += 256) bias_s[e] = (p.bias && e < E) ? p.bias[e] : 0.0f;
  for (int q = tid; q < EP * W; q += 256) masks[q] = 0ull;

  float* lg = uni;
  if constexpr (FROM_LOGITS) {
    // logits of this block's tokens, rows of E contiguous floats
    for (int q = tid; q < TT * EP; q += 256) {
      const int tt = q / EP, e = q % EP;
      lg[tt * (EP + 1) + e] = (tt < tt_count && e < E) ? p.logits[(t0 + tt) * E + e] : 0.0f;
    }
    __syncthreads();
  } else if constexpr (DPP) {
    static_assert(EP >= 8 && EP <= 32, "register-broadcast gate product: 8 to 32 experts");
    constexpr int MD = EP / 4;         // chains per lane
    constexpr int QN = 16 / MD;        // 4-feature runs per expert in a 16-lane row
    constexpr int FC = 4 * QN;         // features per weight chunk
    constexpr int V = XLoad<XT>::V;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int kc = kDppKC;  // d is a multiple (launch_route_ep checks)
    const int nstage = d / kc;
    // weights: lane l loads expert wave*MD + (l%16)/QN, features 4((l%16)%QN) .. +3 of each chunk
    // (experts past E read expert E-1: their logits are never used)
    const int we = wave * MD + (lane & 15) / QN, wq = (lane & 15) % QN;
    const float* wrow = wr + (size_t)(we < E ? we : E - 1) * d + 4 * wq;
    constexpr int XL = kDppTT * kc / V / 256;  // 16-byte x loads per thread per stage
    constexpr int xch = kc / V;                // 16-byte loads per token row and stage
    u32x4 xr[XL];
    // rows past the batch read its last token (their logits are never used),
    // so that every load is unconditional
    auto load_x = [&](int s) {
#pragma unroll
      for (int i = 0; i < XL; ++i) {
        const int q = tid + i * 256, c = q % xch;
        int tt = q / xch;
        tt = tt < tt_count ? tt : tt_count - 1;
        xr[i] = *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + tt) * d + s * kc + c * V);
      }
    };
    auto store_x = [&](int buf) {
      float* xs = uni + buf * kDppPitch * kDppTT;
#pragma unroll
      for (int i = 0; i < XL; ++i) {
        const int q = tid + i * 256, tt = q / xch, c = q % xch;
        float f[V];
        XLoad<XT>::widen(xr[i], f);
#pragma unroll
        for (int v = 0; v < V; v += 4)
          *reinterpret_cast<f32x4*>(xs + tt * kDppPitch + c * V + v) = f32x4{f[v], f[v + 1], f[v + 2], f[v + 3]};
      }
    };
    float acc[MD];
#pragma unroll
    for (int j = 0; j < MD; ++j) acc[j] = 0.0f;
    // the weights of a stage, loaded a stage ahead into one of two register
    // sets (stages unrolled by two, so that the sets are named statically)
    constexpr int CH = kc / FC;
    f32x4 wa[CH], wb[CH];
    auto load_w = [&](f32x4 (&w)[CH], int s) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CH; ++c) w[c] = *reinterpret_cast<const f32x4*>(wrow + s * kc + c * FC);
    };
    // features s*kc + c*FC + 4q + r, ascending: run q of every expert sits
    // in lane e*QN + q of the lane's 16-lane row. One v_fmac_f32 per
    // (expert, feature), its weight broadcast by DPP from that lane (the
    // compiler does not fold a DPP move into fmac itself).
    auto compute = [&](const f32x4 (&w)[CH], int s) __attribute__((always_inline)) {
      const float* xrow = uni + (s & 1) * kDppPitch * kDppTT + lane * kDppPitch;
      static_for<CH>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        static_for<QN>([&](auto qc) {
          constexpr int q = decltype(qc)::value;
          const f32x4 xv = *reinterpret_cast<const f32x4*>(xrow + c * FC + 4 * q);
          static_for<4>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            static_for<MD>([&](auto ec) {
              constexpr int e = decltype(ec)::value;
              fmac_bcast<e * QN + q>(acc[e], w[c][r], xv[r]);
            });
          });
        });
      });
    };
    load_x(0);
    load_w(wa, 0);
    store_x(0);
    __syncthreads();
    // The next stage's loads are unconditional (the last stage loads itself
    // again, into the buffer no one reads): a guarded load makes the
    // compiler's wait for the current weights count only the loads on the
    // path without it, which waits for the prefetch too.
    for (int s = 0; s < nstage; s += 2) {
      const int s1 = s + 1 < nstage ? s + 1 : s;
      load_x(s1);
      load_w(wb, s1);
      compute(wa, s);
      store_x((s + 1) & 1);
      __syncthreads();
      if (s + 1 >= nstage) break;
      const int s2 = s + 2 < nstage ? s + 2 : s + 1;
      load_x(s2);
      load_w(wa, s2);
      compute(wb, s + 1);
      store_x(s & 1);
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < MD; ++j) lg[lane * (EP + 1) + wave * MD + j] = acc[j];
    __syncthreads();
  } else {
  // ---- gate product: logits[tt][e] = fma chain over features ascending
  const int tg = tid % TG, eg = tid / TG;
  float acc[MT][ME];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) acc[i][j] = 0.0f;

  // features per stage: KC when it divides d, else 64 (d is a multiple of 64)
  const int kc = (KC <= 64 || d % KC == 0) ? KC : 64;
  const int xsh = __builtin_ctz((unsigned)(kc / V));  // log2 of 16-byte x loads per row and stage
  const int wsh = __builtin_ctz((unsigned)(kc / 4));
  const int XCH = TT * kc / V;                 // 16-byte x loads per stage
  constexpr int XPT = (TT * KC / V + 255) / 256;
  const int WCH = EP * kc / 4;                 // 16-byte router-weight loads per stage
  constexpr int WPT = (EP * KC / 4 + 255) / 256;
  u32x4 xr[XPT], wreg[WPT];
  const int nstage = d / kc;

  auto load_stage = [&](int s) {
    const int k0 = s * kc;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int q = tid + i * 256;
      xr[i] = u32x4{0u, 0u, 0u, 0u};
      if (q < XCH) {
        const int tt = q >> xsh, c = q & ((1 << xsh) - 1);
        if (tt < tt_count)
          xr[i] = *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + tt) * d + k0 + c * V);
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int q = tid + i * 256;
      wreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (q < WCH) {
        const int e = q >> wsh, c = q & ((1 << wsh) - 1);
        if (e < E) wreg[i] = *reinterpret_cast<const u32x4*>(wr + (size_t)e * d + k0 + c * 4);
      }
    }
  };
  constexpr bool ROWS = L::kRows;
  constexpr int PK = L::kPitch;
  auto store_stage = [&](int buf) {
    float* xs = uni + buf * PK * (TT + EP);
    float* ws = xs + PK * TT;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int q = tid + i * 256;
      if (q < XCH) {
        const int tt = q >> xsh, c = q & ((1 << xsh) - 1);
        float f[V];
        XLoad<XT>::widen(xr[i], f);
        if constexpr (ROWS) {
#pragma unroll
          for (int v = 0; v < V; v += 4)
            *reinterpret_cast<f32x4*>(xs + tt * PK + c * V + v) = f32x4{f[v], f[v + 1], f[v + 2], f[v + 3]};
        } else {
#pragma unroll
          for (int v = 0; v < V; ++v) xs[(c * V + v) * TT + tt] = f[v];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int q = tid + i * 256;
      if (q < WCH) {
        const int e = q >> wsh, c = q & ((1 << wsh) - 1);
        if constexpr (ROWS) {
          *reinterpret_cast<u32x4*>(ws + e * PK + c * 4) = wreg[i];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) ws[(c * 4 + v) * EP + e] = __uint_as_float(wreg[i][v]);
        }
      }
    }
  };

  auto compute_stage = [&](int s) {
    const float* xs = uni + (s & 1) * PK * (TT + EP);
    const float* ws = xs + PK * TT;
    // Features in groups of U: the LDS reads of group g+1 are in flight while
    // the fmas of group g run (every chain still adds its features in
    // ascending order). kc is a multiple of 8, so of U.
    float a[2][U][MT], b[2][U][ME];
    auto read_group = [&](int h, int k0) {
      if constexpr (ROWS) {
#pragma unroll
        for (int u = 0; u < U; u += 4) {
          const f32x4 av = *reinterpret_cast<const f32x4*>(xs + tg * PK + k0 + u);
#pragma unroll
          for (int q = 0; q < 4; ++q) a[h][u + q][0] = av[q];
#pragma unroll
          for (int j = 0; j < ME; ++j) {
            const f32x4 bv = *reinterpret_cast<const f32x4*>(ws + (eg * ME + j) * PK + k0 + u);
#pragma unroll
            for (int q = 0; q < 4; ++q) b[h][u + q][j] = bv[q];
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int i = 0; i < MT; ++i) a[h][u][i] = xs[(k0 + u) * TT + tg * MT + i];
#pragma unroll
          for (int j = 0; j < ME; ++j) b[h][u][j] = ws[(k0 + u) * EP + eg * ME + j];
        }
      }
    };
    auto fma_group = [&](int h) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < ME; ++j) acc[i][j] = __builtin_fmaf(a[h][u][i], b[h][u][j], acc[i][j]);
    };
    read_group(0, 0);
#pragma unroll 1
    for (int k0 = 0; k0 < kc; k0 += 2 * U) {
      if (k0 + U < kc) read_group(1, k0 + U);
      fma_group(0);
      if (k0 + U >= kc) break;
      if (k0 + 2 * U < kc) read_group(0, k0 + 2 * U);
      fma_group(1);
    }
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    if (s + 1 < nstage) load_stage(s + 1);
    compute_stage(s);
    if (s + 1 < nstage) store_stage((s + 1) & 1);
    __syncthreads();
  }

  // ---- logits to LDS: lg[tt * (EP+1) + e]
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) lg[(tg * MT + i) * (EP + 1) + eg * ME + j] = acc[i][j];
  __syncthreads();
  }

  // softmax normaliser per token: max, then the sum of exp over experts
  // ascending. A wave per token: lanes take the exps of experts lane + 64 q,
  // and the sum runs serially over lanes (readlane), so it adds the terms in
  // the same order as a single loop over e would.
  auto normalisers = [&]() {
    constexpr int QN = (EP + 63) / 64;
    const int lane = tid & 63;
    for (int tt = tid >> 6; tt < tt_count; tt += 4) {
      const float* l = lg + tt * (EP + 1);
      float v[QN];
      float m = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const int e = lane + 64 * q;
        v[q] = e < E ? l[e] : -__builtin_inff();
        m = v[q] > m ? v[q] : m;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(m, off, 64);
        m = o > m ? o : m;
      }
      float z = 0.0f;
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        const float ex = lane + 64 * q < E ? canonical_exp(v[q] - m) : 0.0f;
        const int n = E - 64 * q < 64 ? E - 64 * q : 64;
        for (int i = 0; i < n; ++i) z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), i));
      }
      if (lane == 0) {
        tok_m[tt] = m;
        tok_z[tt] = z;
      }
    }
    __syncthreads();
  };
  const bool need_z = (p.score == 0) && ((p.bias != nullptr && !p.bias_on_logits) || !p.renorm);
  if (need_z) normalisers();

  // ---- top-k: a group of G lanes per token, VPL values per lane
  {
    constexpr int G = EP < 64 ? EP : 64;
    constexpr int VPL = EP / G;
    constexpr int TPW = 64 / G;
    const int lane = tid & 63, wave = tid >> 6;
    const int gi = lane / G, li = lane % G;
    const bool has_bias = p.bias != nullptr;
    const bool logit_bias = p.bias_on_logits != 0;
    const bool sigmoid = p.score == 1;
    const float* __restrict__ noise = p.noise;
    for (int base = 0; base < tt_count; base += 4 * TPW) {
      if (base + wave * TPW >= tt_count) break;  // this wave's tokens are all padding
      const int tt = base + wave * TPW + gi;
      const float* l = lg + tt * (EP + 1);
      uint64_t key[VPL];
#pragma unroll
      for (int q = 0; q < VPL; ++q) {
        const int e = li + G * q;
        key[q] = 0ull;
        if (e < E && tt < tt_count) {
          float v = l[e];
          if (has_bias) {
            if (logit_bias)
              v = v + bias_s[e];
            else
              v = sigmoid ? sigmoid_canon(v) + bias_s[e] : canonical_exp(v - tok_m[tt]) / tok_z[tt] + bias_s[e];
          }
          if (noise && tt < tt_count) v = v + noise[(t0 + tt) * E + e];
          key[q] = topk_key(v, e);
        }
      }
      for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int q = 1; q < VPL; ++q) best = key[q] > best ? key[q] : best;
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) {
          const uint64_t o = __shfl_xor(best, off, G);
          best = o > best ? o : best;
        }
        const int ew = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
#pragma unroll
        for (int q = 0; q < VPL; ++q)
          if (li + G * q == ew) key[q] = 0ull;
        if (li == 0 && tt < tt_count) sel[tt * k + j] = ew;
      }
    }
  }
  __syncthreads();

  // ---- combine weights, one thread per token, slots in order
  for (int tt = tid; tt < tt_count; tt += 256) {
    const float* l = lg + tt * (EP + 1);
    const int* s = sel + tt * k;
    const int64_t t = t0 + tt;
    if (p.score == 0) {
      if (p.renorm) {
        float mk = l[s[0]];
        for (int j = 1; j < k; ++j) mk = l[s[j]] > mk ? l[s[j]] : mk;
        float sum = 0.0f;
        for (int j = 0; j < k; ++j) sum += canonical_exp(l[s[j]] - mk);
        for (int j = 0; j < k; ++j) {
          p.idx[t * k + j] = s[j];
          p.w[t * k + j] = canonical_exp(l[s[j]] - mk) / sum;
        }
      } else {
        for (int j = 0; j < k; ++j) {
          p.idx[t * k + j] = s[j];
          p.w[t * k + j] = canonical_exp(l[s[j]] - tok_m[tt]) / tok_z[tt];
        }
      }
    } else {
      float sum = 0.0f;
      if (p.renorm)
        for (int j = 0; j < k; ++j) sum += sigmoid_canon(l[s[j]]);
      for (int j = 0; j < k; ++j) {
        const float sj = sigmoid_canon(l[s[j]]);
        p.idx[t * k + j] = s[j];
        p.w[t * k + j] = p.renorm ? sj / (sum + 1e-9f) : sj;
      }
    }
  }

  // ---- metric partials of this block: per-expert sums of the unbiased
  // scores over its tokens (ascending token order) and the sum of lse^2
  if (p.mpart) {
    __syncthreads();
    if (!need_z) normalisers();
    double* row = p.mpart + (size_t)blockIdx.x * (E + 1);
    for (int e = tid; e < E; e += 256) {
      double acc = 0.0;
      for (int tt = 0; tt < tt_count; ++tt) {
        const float l = lg[tt * (EP + 1) + e];
        acc += (double)(p.score == 1 ? sigmoid_canon(l) : canonical_exp(l - tok_m[tt]) / tok_z[tt]);
      }
      row[e] = acc;
    }
    if (tid == 255) {
      double acc = 0.0;
      for (int tt = 0; tt < tt_count; ++tt) {
        const double lse = (double)tok_m[tt] + (double)logf(tok_z[tt]);
        acc += lse * lse;
      }
      row[E] = acc;
    }
  }

  if (p.hist) {
    block_hist_rank(sel, tt_count, k, E, W, masks, p.hist + (size_t)blockIdx.x * E,
                    p.rank ? p.rank + t0 * k : nullptr);
  }
}

// Router losses and health metrics from the per-block partials and the
// counts (one block of 1024 threads; every sum runs in a fixed order, so the
// result is bitwise repeatable):
//   P_e = (sum over blocks of the score sums) / T
//   z-loss = (sum of lse^2) / T; aux = E sum_e (c_e / T) P_e;
//   cv = unbiased std(c) / max(mean(c), 1); entropy = -sum p log2 p over
//   p = max(P, 1e-9) normalised; max/mean load; share of experts with c = 0.
__global__ __launch_bounds__(1024) void k_router_metrics(const double* __restrict__ mpart, int nb,
                                                         const int32_t* __restrict__ counts, int64_t T, int E, int k,
                                                         double* __restrict__ out) {
  __shared__ double part[16][64];
  __shared__ double P[1025];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // column sums: lane = column within a chunk of 64, wave = row phase
  for (int c0 = 0; c0 <= E; c0 += 64) {
    const int c = c0 + lane;
    double s = 0.0;
    if (c <= E)
      for (int b = wave; b < nb; b += 16) s += mpart[(size_t)b * (E + 1) + c];
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && c <= E) {
      double t = 0.0;
      for (int w = 0; w < 16; ++w) t += part[w][lane];
      P[c] = t;
    }
    __syncthreads();
  }
  if (wave != 0) return;
  const double Td = (double)T;
  const double mean = (double)(T * k) / (double)E;
  double aux = 0.0, var = 0.0, mx = 0.0, unused = 0.0, psum = 0.0;
  for (int e = lane; e < E; e += 64) {
    const double pe = P[e] / Td, c = (double)counts[e];
    aux += (c / Td) * pe;
    var += (c - mean) * (c - mean);
    mx = c > mx ? c : mx;
    unused += c == 0.0 ? 1.0 : 0.0;
    psum += pe > 1e-9 ? pe : 1e-9;
  }
  for (int off = 32; off > 0; off >>= 1) {
    aux += __shfl_xor(aux, off);
    var += __shfl_xor(var, off);
    const double o = __shfl_xor(mx, off);
    mx = o > mx ? o : mx;
    unused += __shfl_xor(unused, off);
    psum += __shfl_xor(psum, off);
  }
  double ent = 0.0;
  for (int e = lane; e < E; e += 64) {
    const double pe = P[e] / Td;
    const double q = (pe > 1e-9 ? pe : 1e-9) / psum;
    ent -= q * log(q);
  }
  for (int off = 32; off > 0; off >>= 1) ent += __shfl_xor(ent, off);
  if (lane == 0) {
    out[0] = P[E] / Td;
    out[1] = (double)E * aux;
    out[2] = E > 1 ? sqrt(var / (double)(E - 1)) / (mean > 1.0 ? mean : 1.0) : 0.0;
    out[3] = ent / log(2.0);
    out[4] = mean > 0.0 ? mx / mean : 0.0;
    out[5] = unused / (double)E;
  }
}

// One step of the aux-loss-free balance controller (README,
// "SigmoidRouter", step_bias_update), in fp32 in the order of that code:
// p = c / max(sum c, 1); err = 1/E - p, plus 0.5 where p < 0.1/E;
// bias += err * rate; bias clamped to [-10, 10]. The sum of counts is exact
// integer arithmetic; 1/E and 0.1/E are formed in fp64 and rounded once.
__global__ __launch_bounds__(256) void k_bias_update(const int32_t* __restrict__ counts, int E, float rate,
                                                     float* __restrict__ bias) {
  __shared__ long long part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long s = 0;
  for (int e = tid; e < E; e += 256) s += counts[e];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  const long long sum = part[0] + part[1] + part[2] + part[3];
  float total = (float)sum;
  if (total < 1.0f) total = 1.0f;
  const float target = (float)(1.0 / (double)E);
  const float starved = (float)(0.1 * (1.0 / (double)E));
  for (int e = tid; e < E; e += 256) {
    const float pe = (float)counts[e] / total;
    float err = target - pe;
    if (pe < starved) err = err + 0.5f;
    float b = bias[e] + err * rate;
    b = b < -10.0f ? -10.0f : b;
    b = b > 10.0f ? 10.0f : b;
    bias[e] = b;
  }
}

// Gate product alone: logits[t, e] into p.logits, one fma chain per logit
// over features ascending (the same chains as the fused router). Used where
// whole-row router blocks would leave CUs idle, and by the backward pass.
//
// A block owns TT tokens x TE experts; a thread MT x ME chains. Stages of
// 64 features stream into a ring of NS LDS buffers by global->LDS DMA, NS-1
// stages ahead of the fmas, so that with few tokens (short of work per
// chain) the loads in flight still hide the latency. Stage layout:
// router-weight rows (16-byte chunks, chunk c of row e at position
// c ^ ((e / ME) & 15), so that the 16 rows read together sit in distinct
// banks), then the token rows; every thread issues the same number of DMAs
// (spare ones fetch a valid address into the slack at the end). bf16 token
// rows are widened once per stage into an fp32 copy (rows padded by 16 bytes)
// rather than by every chain that reads them.
constexpr int kLogKC = 64;  // d is a multiple of this
template <int TT_, int TE_, int MT_, int ME_, int NS_, int KC_ = kLogKC, int NT_ = 256>
struct LogitShape {
  static constexpr int TT = TT_, TE = TE_, MT = MT_, ME = ME_, NS = NS_, KC = KC_, NT = NT_;
  static constexpr int TGN = TT / MT, EGN = TE / ME;
  static_assert(TGN * EGN == NT && NT % 64 == 0 && NT <= 256, "threads of the block");
  static_assert(NS >= 2 && NS <= 8, "ring depth");
  static_assert(EGN <= 64 && 64 % EGN == 0, "a wave spans whole token groups");
  static_assert(TE * KC / 4 >= NT, "the first DMA of every thread is a weight chunk");
  static constexpr int XP = KC + 4;  // fp32 token-row pitch (floats)
  template <typename XT>
  static constexpr int wch() { return TE * KC / 4; }
  template <typename XT>
  static constexpr int xch() { return TT * KC * (int)sizeof(XT) / 16; }
  template <typename XT>
  static constexpr int loads() { return (wch<XT>() + xch<XT>() + NT - 1) / NT; }  // DMAs per thread per stage
  template <typename XT>
  static constexpr int stage_bytes() { return loads<XT>() * NT * 16; }
  template <typename XT>
  static constexpr int widened_bytes() { return sizeof(XT) == 2 ? TT * XP * 4 : 0; }
  template <typename XT>
  static constexpr int lds_bytes() { return NS * stage_bytes<XT>() + widened_bytes<XT>(); }
};
// few tokens: one chain per thread, 16 x 16 blocks, stages of 128 features
// five deep in the ring (64 features eight deep where d is not a multiple of
// 128)
using LogitNarrow = LogitShape<16, 16, 1, 1, 5, 128>;
using LogitNarrow64 = LogitShape<16, 16, 1, 1, 8>;
// a handful of tokens: one wave per block, 4 tokens x 16 experts, stages of
// 256 features four deep (128 five deep where d is not a multiple of 256):
// long stages spread the per-stage waits and barriers over more fmas
using LogitTiny = LogitShape<4, 16, 1, 1, 4, 256, 64>;
using LogitTiny128 = LogitShape<4, 16, 1, 1, 5, 128, 64>;
// more: 2 x 4 chains, 32 x 64 blocks; many: 4 x 4 chains, 64 x 64 blocks
// (two blocks per CU fit in LDS with bf16 tokens)
using LogitMid = LogitShape<32, 64, 2, 4, 3>;
using LogitWide = LogitShape<64, 64, 4, 4, 2>;
// at most 16 experts: 4 x 1 chains, 64 x 16 blocks
using LogitFewE = LogitShape<64, 16, 4, 1, 3>;

template <typename LS, typename XT>
__global__ __launch_bounds__(LS::NT) void k_logits(RouteLaunch p) {
  constexpr int NT = LS::NT;
  constexpr int TT = LS::TT, TE = LS::TE, MT = LS::MT, ME = LS::ME, NS = LS::NS, EGN = LS::EGN;
  constexpr int KC = LS::KC, CPR = KC / 4;  // 16-byte weight chunks per row and stage
  constexpr int XB = (int)sizeof(XT);
  constexpr int WCH = LS::template wch<XT>(), XCH = LS::template xch<XT>();
  constexpr int L = LS::template loads<XT>();
  constexpr int SBYTES = LS::template stage_bytes<XT>();
  constexpr int XCPR = KC * XB / 16;  // 16-byte token chunks per row and stage
  constexpr int XP = LS::XP;
  __shared__ __align__(16) unsigned char lds_raw[LS::template lds_bytes<XT>()];
  float* xw = reinterpret_cast<float*>(lds_raw + NS * SBYTES);  // widened bf16 token rows [TT][XP]
  const int tid = threadIdx.x, wave = tid >> 6;
  const int eg = tid % EGN, tg = tid / EGN;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int e0 = blockIdx.y * TE;
  const int d = p.d, E = p.E;
  const int64_t T = p.T;
  const unsigned char* __restrict__ xb = reinterpret_cast<const unsigned char*>(p.x);
  const unsigned char* __restrict__ wb = reinterpret_cast<const unsigned char*>(p.w_router);

  // global source of this thread's DMA i (feature offset added per stage)
  const unsigned char* src[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int q = i * NT + tid;
    if (q < WCH) {
      const int e = q / CPR, c = (q % CPR) ^ ((e / ME) & 15);
      const int er = e0 + e < E ? e0 + e : E - 1;
      src[i] = wb + ((size_t)er * d + c * 4) * 4;
    } else if (q < WCH + XCH) {
      const int tt = (q - WCH) / XCPR, c = (q - WCH) % XCPR;
      const int64_t tr = t0 + tt < T ? t0 + tt : T - 1;
      src[i] = xb + ((size_t)tr * d) * XB + c * 16;
    } else {
      src[i] = src[0];  // spare: a copy of this thread's first weight chunk, into the slack
    }
  }
  auto issue = [&](int st) {
    unsigned char* base = lds_raw + (st % NS) * SBYTES + wave * 1024;
    const size_t wk = (size_t)st * KC * 4, xk = (size_t)st * KC * XB;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = i * NT + tid;
      const size_t off = (q < WCH || q >= WCH + XCH) ? wk : xk;
      lds_dma16(src[i] + off, base + i * NT * 16);
    }
  };

  float acc[MT][ME];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) acc[i][j] = 0.0f;
  // a wave whose tokens are all past T skips the fmas (it still loads); the
  // test is on a scalar so that the branch is uniform
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool active = t0 + (int64_t)(wave_s * 64 / EGN) * MT < T;

  const int nst = d / KC;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nst) issue(st);
  for (int st = 0; st < nst; ++st) {
    // stage st landed (later stages may still be in flight), and this wave's
    // LDS reads of the previous stage are done
    const int ahead = nst - 1 - st < NS - 2 ? nst - 1 - st : NS - 2;
    if (NS >= 8 && ahead >= 6) wait_vm_lgkm0<(NS >= 8 ? 6 : 0) * L>();
    else if (NS >= 7 && ahead == 5) wait_vm_lgkm0<(NS >= 7 ? 5 : 0) * L>();
    else if (NS >= 6 && ahead == 4) wait_vm_lgkm0<(NS >= 6 ? 4 : 0) * L>();
    else if (NS >= 5 && ahead == 3) wait_vm_lgkm0<(NS >= 5 ? 3 : 0) * L>();
    else if (NS >= 4 && ahead == 2) wait_vm_lgkm0<(NS >= 4 ? 2 : 0) * L>();
    else if (NS >= 3 && ahead == 1) wait_vm_lgkm0<L>();
    else wait_vm_lgkm0<0>();
    // A bare s_barrier: __syncthreads would also wait for the DMAs still in
    // flight. The memory clobber keeps the LDS reads below it.
    asm volatile("s_barrier" ::: "memory");
    const unsigned char* sb = lds_raw + (st % NS) * SBYTES;
    const float* xs;  // fp32 token rows of this stage, pitch xp floats
    int xp;
    if constexpr (XB == 2) {
      // widen: 8 features (16 bytes) per item; the previous stage's reads of
      // xw finished before the barrier above
      for (int q = tid; q < TT * KC / 8; q += NT) {
        const int tt = q / (KC / 8), c = q % (KC / 8);
        const u32x4 v = *reinterpret_cast<const u32x4*>(sb + WCH * 16 + tt * KC * 2 + c * 16);
        float* o = xw + tt * XP + c * 8;
        *reinterpret_cast<f32x4*>(o) = f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                                             __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xFFFF0000u),
                                                 __uint_as_float(v[3] << 16), __uint_as_float(v[3] & 0xFFFF0000u)};
      }
      wait_vm_lgkm0<63>();  // this wave's LDS writes done (DMAs may stay in flight)
      asm volatile("s_barrier" ::: "memory");
      xs = xw;
      xp = XP;
    } else {
      xs = reinterpret_cast<const float*>(sb + WCH * 16);
      xp = KC;
    }
    if (st + NS - 1 < nst) issue(st + NS - 1);  // into the buffer of stage st-1
    if (active) {
      // chunks in groups of CG, the LDS reads of group g+1 issued before the
      // fmas of group g (the chains still take the features in order)
      constexpr int CG = (MT + ME) <= 2 ? 8 : 2;
      f32x4 a[2][CG][MT], b[2][CG][ME];
      auto read = [&](int h, int c0) {
#pragma unroll
        for (int cc = 0; cc < CG; ++cc) {
          const int c = c0 + cc;
#pragma unroll
          for (int i = 0; i < MT; ++i) a[h][cc][i] = *reinterpret_cast<const f32x4*>(xs + (tg * MT + i) * xp + c * 4);
#pragma unroll
          for (int j = 0; j < ME; ++j) {
            const int e = eg * ME + j;
            b[h][cc][j] = *reinterpret_cast<const f32x4*>(sb + (e * CPR + (c ^ ((e / ME) & 15))) * 16);
          }
        }
      };
      read(0, 0);
#pragma unroll
      for (int g = 0; g < CPR / CG; ++g) {
        if (g + 1 < CPR / CG) read((g + 1) & 1, (g + 1) * CG);
#pragma unroll
        for (int cc = 0; cc < CG; ++cc)
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
              for (int j = 0; j < ME; ++j)
                acc[i][j] = __builtin_fmaf(a[g & 1][cc][i][u], b[g & 1][cc][j][u], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t t = t0 + tg * MT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < ME; ++j) {
      const int e = e0 + eg * ME + j;
      if (e < E) p.logits[t * E + e] = acc[i][j];
    }
  }
}

// Expert histogram and ranks of blocks of 256 tokens, from expert ids.
constexpr int kHistTT = 256;
__global__ __launch_bounds__(256) void k_hist_rank(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                   int32_t* __restrict__ hist, int32_t* __restrict__ rank) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  constexpr int W = kHistTT / 64;
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds_raw);
  int* sel = reinterpret_cast<int*>(masks + (size_t)E * W);
  const int64_t t0 = (int64_t)blockIdx.x * kHistTT;
  const int tt_count = (int)((T - t0) < kHistTT ? (T - t0) : kHistTT);
  for (int q = threadIdx.x; q < E * W; q += 256) masks[q] = 0ull;
  for (int q = threadIdx.x; q < tt_count * k; q += 256) sel[q] = idx[t0 * k + q];
  __syncthreads();
  block_hist_rank(sel, tt_count, k, E, W, masks, hist + (size_t)blockIdx.x * E, rank + t0 * k);
}

template <typename K>
hipError_t launch_k(K kern, dim3 grid, size_t lds, hipStream_t s, const RouteLaunch& a, int threads = 256) {
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(threads), lds, s, a);
  return hipGetLastError();
}

// Logits kernel shape for a batch: at most 16 experts, 64 x 16 blocks;
// otherwise one chain per thread (one-wave 4 x 16 blocks up to 64 tokens,
// then 16 x 16 blocks while 32 x 64 blocks would not give every CU one), 32 x
// 64 blocks while 64 x 64 ones would not give every CU two, else 64 x 64.
template <typename LS, typename XT>
hipError_t launch_logits_shape(const RouteLaunch& a, hipStream_t s) {
  const dim3 g((unsigned)((a.T + LS::TT - 1) / LS::TT), (unsigned)((a.E + LS::TE - 1) / LS::TE));
  return launch_k(k_logits<LS, XT>, g, 0, s, a, LS::NT);
}
template <typename XT>
hipError_t launch_logits_t(const RouteLaunch& a, hipStream_t s) {
  const int64_t cu = cu_count(), et = (a.E + 63) / 64;
  if (a.E <= 16) return launch_logits_shape<LogitFewE, XT>(a, s);
  if (a.T <= 64 && a.d % 128 == 0)
    return a.d % 256 == 0 ? launch_logits_shape<LogitTiny, XT>(a, s) : launch_logits_shape<LogitTiny128, XT>(a, s);
  if ((a.T + 31) / 32 * et < cu)
    return a.d % 128 == 0 ? launch_logits_shape<LogitNarrow, XT>(a, s) : launch_logits_shape<LogitNarrow64, XT>(a, s);
  if ((a.T + 63) / 64 * et < 2 * cu) return launch_logits_shape<LogitMid, XT>(a, s);
  return launch_logits_shape<LogitWide, XT>(a, s);
}

// Split path when the experts are many and whole-row blocks would not give
// every CU two (four for shapes with at most 16 chains per thread, whose
// fused gate product measured slower than the logits kernel's: 128 experts
// at 512 blocks): logits first (grid over tokens and experts), then the
// selection from them in blocks of kSelTT tokens.
template <int EP>
bool route_split_ep(int E, int64_t T) {
  using S = RouteShape<EP>;
  const int64_t nb = (T + S::TT - 1) / S::TT;
  const int64_t per_cu = S::ME * S::MT >= 32 ? 2 : 4;
  return E >= 64 && nb < per_cu * (int64_t)cu_count();
}

// The register-broadcast gate product: up to 32 experts and enough tokens
// for two 64-token blocks per CU.
#ifndef MOE_DPP_MIN_BLOCKS_PER_CU
#define MOE_DPP_MIN_BLOCKS_PER_CU 2
#endif
template <int EP>
bool route_dpp_ep(int64_t T, int d) {
  return EP <= 32 && d % kDppKC == 0 && (T + kDppTT - 1) / kDppTT >= (int64_t)MOE_DPP_MIN_BLOCKS_PER_CU * cu_count();
}

template <int EP>
hipError_t launch_route_ep(const RouteLaunch& a, hipStream_t s) {
  using S = RouteShape<EP>;
  if constexpr (EP <= 32) {
    if (route_dpp_ep<EP>(a.T, a.d)) {
      const size_t lds_d = RouteLds<EP, false, true>::bytes(a.k);
      const dim3 g((unsigned)((a.T + kDppTT - 1) / kDppTT));
      return a.dtype == 1 ? launch_k(k_route<EP, uint16_t, false, true>, g, lds_d, s, a)
                          : launch_k(k_route<EP, float, false, true>, g, lds_d, s, a);
    }
  }
  const size_t lds = RouteLds<EP>::bytes(a.k);
  const int64_t nb = (a.T + S::TT - 1) / S::TT;
  const size_t lds_sel = RouteLds<EP, true>::bytes(a.k);
  const int64_t nb_sel = (a.T + kSelTT - 1) / kSelTT;
  if (a.d % 64) return hipErrorInvalidValue;  // stages of 64 features (or a multiple)
  const bool split = a.logits != nullptr && route_split_ep<EP>(a.E, a.T);
  if (split) {
    hipError_t e = a.dtype == 1 ? launch_logits_t<uint16_t>(a, s) : launch_logits_t<float>(a, s);
    if (e != hipSuccess) return e;
    return a.dtype == 1 ? launch_k(k_route<EP, uint16_t, true>, dim3((unsigned)nb_sel), lds_sel, s, a)
                        : launch_k(k_route<EP, float, true>, dim3((unsigned)nb_sel), lds_sel, s, a);
  }
  return a.dtype == 1 ? launch_k(k_route<EP, uint16_t, false>, dim3((unsigned)nb), lds, s, a)
                      : launch_k(k_route<EP, float, false>, dim3((unsigned)nb), lds, s, a);
}

int padded_experts(int E) {
  int ep = 8;
  while (ep < E) ep *= 2;
  return ep;
}

}  // namespace

int route_tokens_per_block(int E, int64_t T, int d) {
  switch (padded_experts(E)) {
    case 8: return route_dpp_ep<8>(T, d) ? kDppTT : RouteShape<8>::TT;
    case 16: return route_dpp_ep<16>(T, d) ? kDppTT : RouteShape<16>::TT;
    case 32: return route_dpp_ep<32>(T, d) ? kDppTT : RouteShape<32>::TT;
    case 64: return route_split_ep<64>(E, T) ? kSelTT : RouteShape<64>::TT;
    case 128: return route_split_ep<128>(E, T) ? kSelTT : RouteShape<128>::TT;
    case 256: return route_split_ep<256>(E, T) ? kSelTT : RouteShape<256>::TT;
    case 512: return route_split_ep<512>(E, T) ? kSelTT : RouteShape<512>::TT;
    default: return route_split_ep<1024>(E, T) ? kSelTT : RouteShape<1024>::TT;
  }
}

size_t route_lds_bytes(int E, int k) {
  switch (padded_experts(E)) {
    case 8: return RouteLds<8>::bytes(k);
    case 16: return RouteLds<16>::bytes(k);
    case 32: return RouteLds<32>::bytes(k);
    case 64: return RouteLds<64>::bytes(k);
    case 128: return RouteLds<128>::bytes(k);
    case 256: return RouteLds<256>::bytes(k);
    case 512: return RouteLds<512>::bytes(k);
    default: return RouteLds<1024>::bytes(k);
  }
}

hipError_t launch_route(const RouteLaunch& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  switch (padded_experts(a.E)) {
    case 8: return launch_route_ep<8>(a, s);
    case 16: return launch_route_ep<16>(a, s);
    case 32: return launch_route_ep<32>(a, s);
    case 64: return launch_route_ep<64>(a, s);
    case 128: return launch_route_ep<128>(a, s);
    case 256: return launch_route_ep<256>(a, s);
    case 512: return launch_route_ep<512>(a, s);
    case 1024: return launch_route_ep<1024>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_router_metrics(const double* mpart, int nb, const int32_t* counts, int64_t T, int E, int k,
                                 double* out, hipStream_t s) {
  if (T <= 0 || E > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_router_metrics, dim3(1), dim3(1024), 0, s, mpart, nb, counts, T, E, k, out);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int E, float rate, float* bias, hipStream_t s) {
  if (E <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bias_update, dim3(1), dim3(256), 0, s, counts, E, rate, bias);
  return hipGetLastError();
}

hipError_t launch_logits(const RouteLaunch& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.d % kLogKC || !a.logits || a.E <= 0) return hipErrorInvalidValue;
  return a.dtype == 1 ? launch_logits_t<uint16_t>(a, s) : launch_logits_t<float>(a, s);
}

int hist_tokens_per_block() { return kHistTT; }

hipError_t launch_hist_rank(const int32_t* idx, int64_t T, int k, int E, int32_t* hist, int32_t* rank,
                            hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t nb = (T + kHistTT - 1) / kHistTT;
  const size_t lds = sizeof(uint64_t) * (size_t)E * (kHistTT / 64) + sizeof(int) * kHistTT * k;
  hipError_t e = hipFuncSetAttribute((const void*)k_hist_rank, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hist_rank, dim3((unsigned)nb), dim3(256), lds, s, idx, T, k, E, hist, rank);
  return hipGetLastError();
}

}  // namespace moe
