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

template <int EP>
struct RouteLds {
  using S = RouteShape<EP>;
  // One token per thread (MT = 1): stage rows are token- and expert-major,
  // padded by 4 floats, so that a lane reads 4 features with one 16-byte
  // load. Otherwise feature-major ([feature][token] and [feature][expert]).
  static constexpr bool kRows = S::MT == 1;
  static constexpr int kPitch = kRows ? S::KC + 4 : S::KC;
  static constexpr int kStage = 2 * kPitch * (S::TT + EP);  // floats
  static constexpr int kLogits = S::TT * (EP + 1);          // floats
  static constexpr int kUnion = kStage > kLogits ? kStage : kLogits;
  static constexpr int kWords = (S::TT + 63) / 64;
  static size_t bytes(int k) {
    return sizeof(float) * kUnion + sizeof(uint64_t) * EP * kWords + sizeof(int) * S::TT * k +
           sizeof(float) * (EP + 2 * S::TT);
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
template <int EP, typename XT, bool FROM_LOGITS>
__global__ __launch_bounds__(256) void k_route(RouteLaunch p) {
  using S = RouteShape<EP>;
  using L = RouteLds<EP>;
  constexpr int ME = S::ME, MT = S::MT, KC = S::KC, EG = S::EG, TG = S::TG, TT = S::TT;
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

  // softmax normaliser per token: max, then sum of exp over experts ascending
  auto normalisers = [&]() {
    for (int tt = tid; tt < TT; tt += 256) {
      const float* l = lg + tt * (EP + 1);
      float m = l[0];
      for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
      float z = 0.0f;
      for (int e = 0; e < E; ++e) z += canonical_exp(l[e] - m);
      tok_m[tt] = m;
      tok_z[tt] = z;
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
    for (int base = 0; base < TT; base += 4 * TPW) {
      const int tt = base + wave * TPW + gi;
      const float* l = lg + tt * (EP + 1);
      uint64_t key[VPL];
#pragma unroll
      for (int q = 0; q < VPL; ++q) {
        const int e = li + G * q;
        key[q] = 0ull;
        if (e < E) {
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

// Gate product alone, for batches too small to fill the GPU with whole-row
// router blocks: a block owns 16 tokens x 64 experts (thread: 1 token x 4
// experts), so the grid also spans the experts. Each logit is still one fma
// chain over features ascending, identical to the fused kernel's.
constexpr int kLogTT = 16, kLogTE = 64, kLogKC = 32;
template <typename XT>
__global__ __launch_bounds__(256) void k_logits(RouteLaunch p) {
  constexpr int V = XLoad<XT>::V;
  __shared__ __align__(16) float xs[2][kLogKC][kLogTT];
  __shared__ __align__(16) float ws[2][kLogKC][kLogTE];
  const int tid = threadIdx.x;
  const int tg = tid % kLogTT, eg = tid / kLogTT;  // 16 x 16
  const int64_t t0 = (int64_t)blockIdx.x * kLogTT;
  const int e0 = blockIdx.y * kLogTE;
  const int d = p.d, E = p.E;
  const XT* __restrict__ x = reinterpret_cast<const XT*>(p.x);
  constexpr int XCH = kLogTT * kLogKC / V;  // 16-byte x loads per stage
  constexpr int WCH = kLogTE * kLogKC / 4;  // 512
  u32x4 xr = u32x4{0u, 0u, 0u, 0u}, wreg[WCH / 256];
  auto load = [&](int st) {
    const int k0 = st * kLogKC;
    if (tid < XCH) {
      const int tt = tid / (kLogKC / V), c = tid % (kLogKC / V);
      xr = u32x4{0u, 0u, 0u, 0u};
      if (t0 + tt < p.T) xr = *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + tt) * d + k0 + c * V);
    }
#pragma unroll
    for (int i = 0; i < WCH / 256; ++i) {
      const int q = tid + i * 256, e = q / (kLogKC / 4), c = q % (kLogKC / 4);
      wreg[i] = u32x4{0u, 0u, 0u, 0u};
      if (e0 + e < E) wreg[i] = *reinterpret_cast<const u32x4*>(p.w_router + (size_t)(e0 + e) * d + k0 + c * 4);
    }
  };
  auto store = [&](int buf) {
    if (tid < XCH) {
      const int tt = tid / (kLogKC / V), c = tid % (kLogKC / V);
      float f[V];
      XLoad<XT>::widen(xr, f);
#pragma unroll
      for (int v = 0; v < V; ++v) xs[buf][c * V + v][tt] = f[v];
    }
#pragma unroll
    for (int i = 0; i < WCH / 256; ++i) {
      const int q = tid + i * 256, e = q / (kLogKC / 4), c = q % (kLogKC / 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) ws[buf][c * 4 + v][e] = __uint_as_float(wreg[i][v]);
    }
  };
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int nst = d / kLogKC;
  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) load(st + 1);
    const int b = st & 1;
#pragma unroll 8
    for (int kk = 0; kk < kLogKC; ++kk) {
      const float a = xs[b][kk][tg];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(a, ws[b][kk][eg * 4 + j], acc[j]);
    }
    if (st + 1 < nst) store((st + 1) & 1);
    __syncthreads();
  }
  if (t0 + tg < p.T) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e0 + eg * 4 + j < E) p.logits[(t0 + tg) * E + e0 + eg * 4 + j] = acc[j];
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
hipError_t launch_k(K kern, dim3 grid, size_t lds, hipStream_t s, const RouteLaunch& a) {
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

int cu_count_route() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    n = (hipGetDevice(&dev) == hipSuccess &&
         hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            ? v
            : 256;
  }
  return n;
}

template <int EP>
hipError_t launch_route_ep(const RouteLaunch& a, hipStream_t s) {
  using S = RouteShape<EP>;
  const size_t lds = RouteLds<EP>::bytes(a.k);
  const int64_t nb = (a.T + S::TT - 1) / S::TT;
  if (a.d % 64 || a.d % kLogKC) return hipErrorInvalidValue;  // stages of min(KC, 64) features
  // Split path when whole-row blocks would leave CUs idle and the experts are
  // many: logits first (grid over tokens and experts), then the selection.
  const bool split = a.logits != nullptr && a.E >= 64 && 4 * nb < cu_count_route();
  if (split) {
    const dim3 g((unsigned)((a.T + kLogTT - 1) / kLogTT), (unsigned)((a.E + kLogTE - 1) / kLogTE));
    hipError_t e = a.dtype == 1 ? launch_k(k_logits<uint16_t>, g, 0, s, a) : launch_k(k_logits<float>, g, 0, s, a);
    if (e != hipSuccess) return e;
    return a.dtype == 1 ? launch_k(k_route<EP, uint16_t, true>, dim3((unsigned)nb), lds, s, a)
                        : launch_k(k_route<EP, float, true>, dim3((unsigned)nb), lds, s, a);
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

int route_tokens_per_block(int E) {
  switch (padded_experts(E)) {
    case 8: return RouteShape<8>::TT;
    case 16: return RouteShape<16>::TT;
    case 32: return RouteShape<32>::TT;
    case 64: return RouteShape<64>::TT;
    case 128: return RouteShape<128>::TT;
    case 256: return RouteShape<256>::TT;
    case 512: return RouteShape<512>::TT;
    default: return RouteShape<1024>::TT;
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
  if (a.d % kLogKC || !a.logits) return hipErrorInvalidValue;
  const dim3 g((unsigned)((a.T + kLogTT - 1) / kLogTT), (unsigned)((a.E + kLogTE - 1) / kLogTE));
  return a.dtype == 1 ? launch_k(k_logits<uint16_t>, g, 0, s, a) : launch_k(k_logits<float>, g, 0, s, a);
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
