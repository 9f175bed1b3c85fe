// C ABI of libmoe.so: argument validation, workspace layout and the launch
// sequence of the MoE FFN layer forward pass. Declarations and the contract
// of every entry point are in include/moe.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Checks of a layer description that do not depend on T.
moe_status check_layer(const moe_layer* L, bool need_experts) {
  if (!L) return MOE_ERR_INVALID;
  if (L->dtype != MOE_F32 && L->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (L->score != MOE_SOFTMAX && L->score != MOE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (L->d_model <= 0 || L->d_ff <= 0 || L->n_experts <= 0 || L->d_ff_shared < 0) return MOE_ERR_INVALID;
  if (L->top_k < 1 || L->top_k > L->n_experts) return MOE_ERR_INVALID;
  if (L->d_model % 64 || L->d_ff % 64 || L->d_ff_shared % 64) return MOE_ERR_UNSUPPORTED;
  if (L->n_experts > 1024 || L->top_k > 32) return MOE_ERR_UNSUPPORTED;
  if (!L->w_router || !aligned16(L->w_router)) return MOE_ERR_INVALID;
  // The shared expert is stated by all three weights and a width, or by none.
  const int n_shared = (L->ws_gate != nullptr) + (L->ws_up != nullptr) + (L->ws_down != nullptr);
  if (n_shared != 0 && n_shared != 3) return MOE_ERR_INVALID;
  if ((n_shared == 3) != (L->d_ff_shared > 0)) return MOE_ERR_INVALID;
  if (n_shared == 3 && (!aligned16(L->ws_gate) || !aligned16(L->ws_up) || !aligned16(L->ws_down)))
    return MOE_ERR_INVALID;
  if (need_experts) {
    if (!L->w_gate || !L->w_up || !L->w_down) return MOE_ERR_INVALID;
    if (!aligned16(L->w_gate) || !aligned16(L->w_up) || !aligned16(L->w_down)) return MOE_ERR_INVALID;
  }
  return MOE_OK;
}

// The shared expert joins the routed grouped GEMMs as one more group (all T
// tokens, weight 1) when it has the routed width and is small (T * d_ff up to
// 2^25): its own launches would leave the GPU partly idle, one gate/up and
// one down launch over every expert do not. A large shared expert keeps two
// dense launches, whose tiles (and weight traffic) spread over all XCDs; as
// the last group of the tile list its tiles would fall to one XCD.
#ifndef MOE_STREAM_TILES
#define MOE_STREAM_TILES 1
#endif
// Weight rows are streamed (non-temporal DMA) when the groups average at
// most this many row tiles: each weight tile is then read about once, and
// keeping it in L2 only evicts data that is read again.
bool stream_weights(int64_t rows, int64_t groups, int bm) {
  return groups > 0 && rows <= groups * (int64_t)bm * MOE_STREAM_TILES;
}

// The routed gate/up launch of the eight-wave kernel walks its raster groups
// inside each expert's row tiles when there are many experts averaging four
// or more 256-row tiles, or two or more with a K of at least 4096 (multi-MB
// weight panels): a raster group of 8 row tiles across the list then mixes
// several experts' weight panels in most of its rounds. Measured on the
// DeepSeek-style layer (8.5 row tiles per expert) 28.2 -> 27.7 ms, and at
// 16,384 tokens (2.2 per expert) 9.60 -> 9.32 ms; the Qwen3-like layer (K
// 2048) within noise at 4 row tiles per expert and 1.3% slower at 3; down
// launches 2% slower that way, so down keeps the plain order; the iso-width
// layer's 16 experts of 32 row tiles keep it too (0.6% slower).
bool raster_by_group(int64_t rows, int64_t groups, int d_in) {
  if (groups < 64) return false;
  return rows >= groups * 4 * (int64_t)256 || (d_in >= 4096 && rows >= groups * 2 * (int64_t)256);
}

// The backward adds the router's input gradient dl W_router inside the final
// gather (E fmas per element) up to this many experts, else by a GEMM.
constexpr int kRouterInGatherMaxE = 16;

bool shared_as_group(const moe_layer* L, int64_t T) {
  return L->d_ff_shared > 0 && L->d_ff_shared == L->d_ff && T * (int64_t)L->d_ff_shared <= (int64_t)1 << 25;
}

struct Layout {
  size_t hist, base, rank, counts, offsets, n_tiles, tiles, row_of, tok_of_row, idx, w, logits, mpart, h, yperm, hs,
      ys, total;
  int64_t nb;         // histogram rows (blocks)
  int64_t gemm_rows;  // rows of the grouped GEMMs: T*k routed (+ T shared when it is a group)
  int64_t max_tiles;  // bound on grouped GEMM row tiles
};

// One layout serves moe_forward, moe_route, moe_permute and moe_combine.
Layout make_layout(const moe_layer* L, int64_t T) {
  Layout o{};
  const int64_t E = L->n_experts, k = L->top_k, d = L->d_model, f = L->d_ff, fs = L->d_ff_shared;
  const int64_t rows = T * k;
  const int eb = elem_bytes(L->dtype);
  const int64_t tpb_r = route_tokens_per_block((int)E, T, (int)L->d_model), tpb_h = hist_tokens_per_block();
  const int64_t tpb = tpb_r < tpb_h ? tpb_r : tpb_h;
  o.nb = (T + tpb - 1) / tpb;
  const bool merged = shared_as_group(L, T);
  o.gemm_rows = rows + (merged ? T : 0);
  o.max_tiles = (o.gemm_rows + kMinTileRows - 1) / kMinTileRows + E + 1;  // bound for the smallest row tile
  size_t p = 0;
  auto take = [&](size_t bytes) {
    const size_t at = p;
    p = align_up(p + bytes);
    return at;
  };
  o.hist = take(sizeof(int32_t) * (size_t)(o.nb * E));
  o.base = take(sizeof(int32_t) * (size_t)(o.nb * E));
  o.rank = take(sizeof(int32_t) * (size_t)rows);
  o.counts = take(sizeof(int32_t) * (size_t)E);
  o.offsets = take(sizeof(int32_t) * (size_t)(E + 2));
  o.n_tiles = take(sizeof(int32_t));
  o.tiles = take(sizeof(int2) * (size_t)o.max_tiles);
  o.row_of = take(sizeof(int32_t) * (size_t)rows);
  o.tok_of_row = take(sizeof(int32_t) * (size_t)o.gemm_rows);
  o.idx = take(sizeof(int32_t) * (size_t)rows);
  o.w = take(sizeof(float) * (size_t)rows);
  o.logits = take(sizeof(float) * (size_t)(T * E));
  o.mpart = take(sizeof(double) * (size_t)(o.nb * (E + 1)));
  o.h = take((size_t)eb * (size_t)(o.gemm_rows * f));
  o.yperm = take(sizeof(float) * (size_t)(o.gemm_rows * d));
  o.hs = take((size_t)eb * (size_t)(merged ? 0 : T * fs));
  o.ys = take(sizeof(float) * (size_t)(fs > 0 && !merged ? T * d : 0));
  o.total = p;
  return o;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(reinterpret_cast<unsigned char*>(ws) + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                                \
  do {                                               \
    const hipError_t moe_e_ = (expr);                \
    if (moe_e_ != hipSuccess) return MOE_ERR_HIP;    \
  } while (0)

}  // namespace

struct moe_timing {
  hipEvent_t ev[MOE_N_PHASES + 1];
  uint32_t mask;  // phases timed; boundary i is recorded when phase i or phase i-1 is
};

namespace {

void mark(moe_timing* t, int i, hipStream_t s) {
  if (t && (((t->mask << 1) >> i) & 3u)) (void)hipEventRecord(t->ev[i], s);  // phase i or i-1 timed
}

moe_status check_T(int64_t T, int k) {
  if (T < 0) return MOE_ERR_INVALID;
  if (T * (int64_t)k > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;  // row ids are int32
  return MOE_OK;
}

// Options: noise must be 16-byte aligned device data; metrics need tokens.
moe_status check_opts(const moe_route_opts* o, int64_t T) {
  if (!o) return MOE_OK;
  if (o->sel_noise && !aligned16(o->sel_noise)) return MOE_ERR_INVALID;
  if (o->metrics && (T <= 0 || ((uintptr_t)o->metrics & 7u))) return MOE_ERR_INVALID;
  return MOE_OK;
}

RouteLaunch route_launch(const moe_layer* L, const void* x, int64_t T, const moe_route_opts* o, int32_t* idx,
                         float* w, int32_t* hist, int32_t* rank, void* ws, const Layout& lo) {
  RouteLaunch r{x, L->dtype, T, L->d_model, L->n_experts, L->top_k, L->score, L->renorm, L->w_router, L->sel_bias,
                idx, w, hist, rank, at<float>(ws, lo.logits)};
  r.bias_on_logits = L->bias_on_logits;
  r.noise = o ? o->sel_noise : nullptr;
  r.mpart = (o && o->metrics) ? at<double>(ws, lo.mpart) : nullptr;
  return r;
}

moe_status forward_impl(const moe_layer* L, const void* x, int64_t T, const moe_route_opts* opts, float* y,
                        int32_t* idx, float* w, int32_t* counts, void* ws, size_t ws_bytes, hipStream_t s,
                        moe_timing* tm) {
  moe_status st = check_layer(L, true);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->top_k)) != MOE_OK) return st;
  if ((st = check_opts(opts, T)) != MOE_OK) return st;
  if (T > 0 && (!x || !y || !aligned16(x) || !aligned16(y))) return MOE_ERR_INVALID;
  if ((idx && !aligned16(idx)) || (w && !aligned16(w))) return MOE_ERR_INVALID;
  const Layout lo = make_layout(L, T);
  if (T > 0 && (!ws || ws_bytes < lo.total || !aligned16(ws))) return MOE_ERR_WORKSPACE;
  (void)hipGetLastError();
  if (T == 0) {
    for (int i = 0; i <= MOE_N_PHASES; ++i) mark(tm, i, s);
    if (counts) MOE_TRY(launch_fill_i32(counts, L->n_experts, 0, s));
    return MOE_OK;
  }
  const int E = L->n_experts, k = L->top_k, d = L->d_model;
  int32_t* idx_p = idx ? idx : at<int32_t>(ws, lo.idx);
  float* w_p = w ? w : at<float>(ws, lo.w);
  int32_t* counts_p = counts ? counts : at<int32_t>(ws, lo.counts);
  int32_t* hist = at<int32_t>(ws, lo.hist);
  int32_t* rank = at<int32_t>(ws, lo.rank);
  int32_t* base = at<int32_t>(ws, lo.base);
  int32_t* offsets = at<int32_t>(ws, lo.offsets);
  int32_t* n_tiles = at<int32_t>(ws, lo.n_tiles);
  int2* tiles = at<int2>(ws, lo.tiles);
  int32_t* row_of = at<int32_t>(ws, lo.row_of);
  int32_t* tok_of_row = at<int32_t>(ws, lo.tok_of_row);
  const bool merged = shared_as_group(L, T);
  if (merged && T * (int64_t)(k + 1) > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;  // row ids are int32
  const int n_groups = E + (merged ? 1 : 0);
  const int bm = gemm_bm_fwd(L->dtype, lo.gemm_rows, n_groups, L->d_ff, L->d_model);
  const GemmCaps caps = gemm_bn_caps(L->dtype, lo.gemm_rows, n_groups, L->d_ff, L->d_model, L->d_model);
  const int tpb = route_tokens_per_block(E, T, L->d_model);
  const int64_t nb_route = (T + tpb - 1) / tpb;

  mark(tm, MOE_PHASE_ROUTE, s);
  const RouteLaunch r = route_launch(L, x, T, opts, idx_p, w_p, hist, rank, ws, lo);
  MOE_TRY(launch_route(r, s));
  mark(tm, MOE_PHASE_SCAN, s);
  MOE_TRY(launch_scan(hist, (int)nb_route, E, counts_p, offsets, base, bm, n_tiles, tiles, s, merged ? T : 0));
  if (r.mpart) MOE_TRY(launch_router_metrics(r.mpart, (int)nb_route, counts_p, T, E, k, opts->metrics, s));
  mark(tm, MOE_PHASE_SCATTER, s);
  MOE_TRY(launch_scatter(idx_p, rank, base, T, k, E, tpb, row_of, tok_of_row, nullptr, nullptr, 0, s, merged));

  mark(tm, MOE_PHASE_GATEUP, s);
  GemmLaunch gu{};
  gu.dtype = L->dtype;
  gu.gateup = true;
  gu.a = x;
  gu.a_rows = tok_of_row;
  gu.a_row_count = T;
  gu.n_groups = n_groups;
  gu.b0 = L->w_gate;
  gu.b1 = L->w_up;
  if (merged) {
    gu.extra_group = E;
    gu.bx0 = L->ws_gate;
    gu.bx1 = L->ws_up;
  }
  gu.out = at<void>(ws, lo.h);
  gu.N = L->d_ff;
  gu.K = d;
  gu.offsets = offsets;
  gu.tiles = tiles;
  gu.n_tiles = n_tiles;
  gu.max_m_tiles = lo.max_tiles;
  gu.b_stream = stream_weights(lo.gemm_rows, n_groups, bm);
  gu.bn_cap = caps.gateup;
  gu.raster_by_group = raster_by_group(lo.gemm_rows, n_groups, L->d_model);
  MOE_TRY(launch_gemm_fwd(gu, bm, s));
  mark(tm, MOE_PHASE_DOWN, s);
  GemmLaunch dn = gu;
  dn.gateup = false;
  dn.bn_cap = caps.down;
  dn.raster_by_group = false;
  dn.a = at<void>(ws, lo.h);
  dn.a_rows = nullptr;
  dn.b0 = L->w_down;
  dn.b1 = nullptr;
  dn.bx0 = L->ws_down;
  dn.bx1 = nullptr;
  dn.out = at<void>(ws, lo.yperm);
  dn.N = d;
  dn.K = L->d_ff;
  MOE_TRY(launch_gemm_fwd(dn, bm, s));

  // shared expert: rows T*k .. T*k+T-1 of the grouped output, or its own GEMMs
  const float* shared_out = merged ? at<float>(ws, lo.yperm) + (size_t)T * k * d : nullptr;
  const int bm_s = gemm_bm_fwd(L->dtype, T, 1, L->d_ff_shared, L->d_model);
  const GemmCaps caps_s = gemm_bn_caps(L->dtype, T, 1, L->d_ff_shared, L->d_model, L->d_model);
  mark(tm, MOE_PHASE_SHARED_GATEUP, s);
  if (L->d_ff_shared > 0 && !merged) {
    GemmLaunch sg{};
    sg.dtype = L->dtype;
    sg.gateup = true;
    sg.a = x;
    sg.b0 = L->ws_gate;
    sg.b1 = L->ws_up;
    sg.out = at<void>(ws, lo.hs);
    sg.N = L->d_ff_shared;
    sg.K = d;
    sg.rows = T;
    sg.b_stream = stream_weights(T, 1, bm_s);
    sg.bn_cap = caps_s.gateup;
    MOE_TRY(launch_gemm_fwd(sg, bm_s, s));
  }
  mark(tm, MOE_PHASE_SHARED_DOWN, s);
  if (L->d_ff_shared > 0 && !merged) {
    GemmLaunch sd{};
    sd.dtype = L->dtype;
    sd.gateup = false;
    sd.a = at<void>(ws, lo.hs);
    sd.b0 = L->ws_down;
    sd.out = at<void>(ws, lo.ys);
    sd.N = d;
    sd.K = L->d_ff_shared;
    sd.rows = T;
    sd.b_stream = stream_weights(T, 1, bm_s);
    sd.bn_cap = caps_s.down;
    MOE_TRY(launch_gemm_fwd(sd, bm_s, s));
    shared_out = at<float>(ws, lo.ys);
  }
  mark(tm, MOE_PHASE_COMBINE, s);
  MOE_TRY(launch_combine(T, d, k, at<float>(ws, lo.yperm), row_of, w_p, shared_out, y, s));
  mark(tm, MOE_N_PHASES, s);
  return MOE_OK;
}

// ---------------------------------------------------------------- backward

constexpr int kKPad = 64;  // K-segment granularity of the weight-gradient GEMMs (a K stage)

// Rows per group up to which the bf16 backward products read the weights as
// stored ([K, N], transposing LDS reads) rather than from transposed copies:
// the transposes cost ~2x the weight bytes of HBM traffic, the transposing
// reads a few percent of MFMA time, so few rows per weight byte favour them.
// Measured: DeepSeek-style layer at 144 rows per group 18% faster backward,
// Qwen3-like at 1024 rows 1.5%; iso-width at 8192 rows 3.6% slower.
constexpr int64_t kBtMaxRows = 2048;

struct BwdLayout {
  size_t hist, base, rank, counts, offsets, n_tiles, tiles, row_of, tok_of_row;
  size_t h, g, u, dyb, wrow, dh, dgu, dxp, wdt, wgut;
  size_t koffs, kg_tiles, kg_n, xt, dyt, ht, dgut;
  size_t logits, dtw, dl, dlt, xtr, wrt, dxr, rkoffs, rtiles, rn, rpart, xb, vg, red, nred, part;
  size_t total;
  int64_t nb, rows, gemm_rows, max_tiles, kp, tp, kg_tiles_max, rseg;
  int G, ep, nseg;
  // bf16 with at most kBtMaxRows rows per group on average: the backward
  // products read the weights as stored instead of transposed copies
  bool bt;
  // weight-gradient launches: row / column tiles, m-tiles per chunk, chunk
  // length (K stages) and the bound on chunks (virtual groups)
  int bm_d, bm_gu, bn_d, bn_gu, mt_d, mt_gu, cap_d, cap_gu, vmax;
};

BwdLayout make_bwd_layout(const moe_layer* L, int64_t T) {
  BwdLayout o{};
  const int64_t E = L->n_experts, k = L->top_k, d = L->d_model, f = L->d_ff;
  const bool shared = L->d_ff_shared > 0;
  const int eb = elem_bytes(L->dtype);
  o.G = (int)E + (shared ? 1 : 0);
  o.rows = T * k;
  o.gemm_rows = o.rows + (shared ? T : 0);
  o.bt = L->dtype == 1 && o.gemm_rows <= kBtMaxRows * (int64_t)o.G;
  const int64_t tpb = hist_tokens_per_block();
  o.nb = (T + tpb - 1) / tpb;
  o.max_tiles = (o.gemm_rows + kMinTileRows - 1) / kMinTileRows + o.G;
  o.kp = (o.gemm_rows + (int64_t)kKPad * o.G + kKPad - 1) / kKPad * kKPad;  // bound on the padded K columns
  o.ep = (int)((E + 127) / 128 * 128);
  // The router weight gradient dl^T x has few output tiles: it is split into
  // nseg K segments of rseg tokens (about 512 tiles in all), summed in order.
  {
    const int64_t tpad = (T + kKPad - 1) / kKPad * kKPad;
    const int64_t tiles = (o.ep / gemm_kg_bm(0, o.ep, d, 1)) * (d % 128 == 0 ? d / 128 : d / 64);
    const int64_t want = (512 + tiles - 1) / tiles;
    int64_t seg = (tpad + want - 1) / want;
    seg = (seg + kKPad - 1) / kKPad * kKPad;
    seg = seg < 256 ? 256 : seg;
    seg = seg > tpad ? tpad : seg;
    o.rseg = seg;
    o.nseg = (int)((tpad + seg - 1) / seg);
    o.tp = o.nseg * seg;
  }
  // Weight-gradient launches: groups longer than a chunk are cut (at most
  // stages / cap extra chunks, each with a partial buffer of m_rows x N fp32).
  const int dt = L->dtype;
  const int64_t stages = o.kp / (dt == MOE_BF16 ? 64 : 32);
  o.bm_d = gemm_kg_bm(dt, (int)d, (int)f, o.G);
  o.bm_gu = gemm_kg_bm(dt, (int)(2 * f), (int)d, o.G);
  o.bn_d = gemm_kg_bn(o.bm_d, (int)f);
  o.bn_gu = gemm_kg_bn(o.bm_gu, (int)d);
  o.mt_d = (int)(d / o.bm_d);
  o.mt_gu = (int)(2 * f / o.bm_gu);
  o.cap_d = gemm_kg_cap(o.bm_d, stages, o.mt_d, (int)(f / o.bn_d));
  o.cap_gu = gemm_kg_cap(o.bm_gu, stages, o.mt_gu, (int)(d / o.bn_gu));
  const int64_t extra_d = stages / o.cap_d, extra_gu = stages / o.cap_gu;
  const int64_t vmax = o.G + (extra_d > extra_gu ? extra_d : extra_gu);
  o.vmax = (int)(vmax > o.nseg ? vmax : o.nseg);
  const int64_t mt = o.mt_d > o.mt_gu ? o.mt_d : o.mt_gu;
  o.kg_tiles_max = (int64_t)o.vmax * mt;
  const int64_t part_floats = (extra_d * d * f > extra_gu * 2 * f * d) ? extra_d * d * f : extra_gu * 2 * f * d;
  size_t p = 0;
  auto take = [&](size_t bytes) {
    const size_t at = p;
    p = align_up(p + bytes);
    return at;
  };
  const size_t R = (size_t)o.gemm_rows;
  o.hist = take(4 * (size_t)(o.nb * E));
  o.base = take(4 * (size_t)(o.nb * E));
  o.rank = take(4 * (size_t)o.rows);
  o.counts = take(4 * (size_t)E);
  o.offsets = take(4 * (size_t)(E + 2));
  o.n_tiles = take(4);
  o.tiles = take(sizeof(int2) * (size_t)o.max_tiles);
  o.row_of = take(4 * (size_t)o.rows);
  o.tok_of_row = take(4 * R);
  o.h = take((size_t)eb * R * f);
  o.g = take(4 * R * f);
  o.u = take(4 * R * f);
  o.dyb = L->dtype == 1 ? take(2 * (size_t)(T * d)) : 0;
  o.wrow = take(4 * R);
  o.dh = take(4 * R * f);
  o.dgu = take((size_t)eb * R * 2 * f);
  o.dxp = take(4 * R * d);
  // transposed weights, unless the GEMMs read [K, N] weights as stored
  o.wdt = take(o.bt ? 0 : (size_t)eb * o.G * f * d);
  o.wgut = take(o.bt ? 0 : (size_t)eb * o.G * d * 2 * f);
  o.koffs = take(4 * (size_t)(o.G + 1));
  o.kg_tiles = take(sizeof(int2) * (size_t)o.kg_tiles_max);
  o.kg_n = take(4);
  o.xt = take((size_t)eb * d * o.kp);
  o.dyt = take((size_t)eb * d * o.kp);
  o.ht = take((size_t)eb * f * o.kp);
  o.dgut = take((size_t)eb * 2 * f * o.kp);
  o.logits = take(4 * (size_t)(T * E));
  o.dtw = take(4 * (size_t)o.rows);
  o.dl = take(4 * (size_t)T * o.ep);
  o.dlt = take(4 * (size_t)o.ep * o.tp);
  o.xtr = take(4 * (size_t)d * o.tp);
  o.wrt = take(4 * (size_t)d * o.ep);
  o.dxr = take(4 * (size_t)(T * d));
  o.rkoffs = take(4 * (size_t)(o.nseg + 1));
  o.rtiles = take(sizeof(int2) * (size_t)o.nseg * (o.ep / 64));
  o.rn = take(4);
  o.rpart = o.nseg > 1 ? take(4 * (size_t)o.nseg * o.ep * d) : 0;
  o.xb = take(4 * (kXcd + 1));
  o.vg = take(sizeof(int4) * (size_t)o.vmax);
  o.red = take(sizeof(int4) * (size_t)(o.G > o.nseg ? o.G : o.nseg));
  o.nred = take(4);
  o.part = part_floats > 0 ? take(4 * (size_t)part_floats) : 0;
  o.total = p;
  return o;
}

moe_status check_backward(const moe_layer* L, int64_t T) {
  moe_status st = check_layer(L, true);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->top_k)) != MOE_OK) return st;
  // the shared expert runs as one more group of the grouped GEMMs
  if (L->d_ff_shared > 0 && L->d_ff_shared != L->d_ff) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)(L->top_k + 1) > 0x3FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_backward_workspace_size(const moe_layer* L, int64_t T, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID;
  moe_status st = check_backward(L, T);
  if (st != MOE_OK) return st;
  *bytes = make_bwd_layout(L, T).total;
  return MOE_OK;
}

moe_status moe_backward(const moe_layer* L, const void* x, int64_t T, const int32_t* topk_idx, const float* topk_w,
                        const float* dy, float z_loss_coef, float aux_loss_coef, const moe_grads* gr, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status st = check_backward(L, T);
  if (st != MOE_OK) return st;
  if (!gr || !gr->dx || !gr->dw_router || !gr->dw_gate || !gr->dw_up || !gr->dw_down) return MOE_ERR_INVALID;
  const bool shared = L->d_ff_shared > 0;
  if (shared != (gr->dws_gate && gr->dws_up && gr->dws_down)) return MOE_ERR_INVALID;
  if (T > 0 && (!x || !topk_idx || !topk_w || !dy || !aligned16(x) || !aligned16(dy) || !aligned16(gr->dx)))
    return MOE_ERR_INVALID;
  // gradients are written (and chunk sums added) 16 bytes at a time
  if (!aligned16(gr->dw_router) || !aligned16(gr->dw_gate) || !aligned16(gr->dw_up) || !aligned16(gr->dw_down) ||
      (shared && (!aligned16(gr->dws_gate) || !aligned16(gr->dws_up) || !aligned16(gr->dws_down))))
    return MOE_ERR_INVALID;
  const BwdLayout lo = make_bwd_layout(L, T);
  if (T > 0 && (!ws || ws_bytes < lo.total || !aligned16(ws))) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_ERR_INVALID;  // the gradients of an empty batch are not defined here
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const int E = L->n_experts, k = L->top_k, d = L->d_model, f = L->d_ff, dt = L->dtype, G = lo.G;
  const int eb = elem_bytes(dt);
  int32_t* hist = at<int32_t>(ws, lo.hist);
  int32_t* rank = at<int32_t>(ws, lo.rank);
  int32_t* base = at<int32_t>(ws, lo.base);
  int32_t* counts = at<int32_t>(ws, lo.counts);
  int32_t* offsets = at<int32_t>(ws, lo.offsets);
  int32_t* n_tiles = at<int32_t>(ws, lo.n_tiles);
  int2* tiles = at<int2>(ws, lo.tiles);
  int32_t* row_of = at<int32_t>(ws, lo.row_of);
  int32_t* tok_of_row = at<int32_t>(ws, lo.tok_of_row);
  float* dtw = gr->d_topk_w ? gr->d_topk_w : at<float>(ws, lo.dtw);

  // 1. dispatch of the given routing (shared expert as group E)
  const int tpb = hist_tokens_per_block();
  const int bm = gemm_bm(dt, lo.gemm_rows, G, f, L->d_model);
  MOE_TRY(launch_hist_rank(topk_idx, T, k, E, hist, rank, s));
  MOE_TRY(launch_scan(hist, (int)lo.nb, E, counts, offsets, base, bm, n_tiles, tiles, s, shared ? T : 0));
  MOE_TRY(launch_scatter(topk_idx, rank, base, T, k, E, tpb, row_of, tok_of_row, nullptr, nullptr, 0, s, shared));

  // 2. forward recompute: H and the pre-activations G, U
  GemmLaunch gu{};
  gu.dtype = dt;
  gu.gateup = true;
  gu.a = x;
  gu.a_rows = tok_of_row;
  gu.a_row_count = T;
  gu.n_groups = G;
  gu.b0 = L->w_gate;
  gu.b1 = L->w_up;
  if (shared) {
    gu.extra_group = E;
    gu.bx0 = L->ws_gate;
    gu.bx1 = L->ws_up;
  }
  gu.out = at<void>(ws, lo.h);
  gu.out_g = at<float>(ws, lo.g);
  gu.out_u = at<float>(ws, lo.u);
  gu.N = f;
  gu.K = d;
  gu.offsets = offsets;
  gu.tiles = tiles;
  gu.n_tiles = n_tiles;
  gu.max_m_tiles = lo.max_tiles;
  gu.b_stream = stream_weights(lo.gemm_rows, G, bm);
  MOE_TRY(launch_gemm(gu, bm, s));

  // 3. dy in the operand type
  const void* dya = dy;
  if (dt == 1) {
    MOE_TRY(launch_to_bf16((int64_t)T * d, dy, at<uint16_t>(ws, lo.dyb), s));
    dya = at<void>(ws, lo.dyb);
  }

  // 4. weights transposed once per call (the GEMM wants K-contiguous rows),
  //    or with few rows per expert read as stored, [K, N] per expert
  unsigned char* wdt = at<unsigned char>(ws, lo.wdt);
  unsigned char* wgut = at<unsigned char>(ws, lo.wgut);
  const bool bt = lo.bt;
  if (!bt) {
  MOE_TRY(launch_transpose(dt, dt, L->w_down, wdt, E, d, d, f, d, 0, s));                 // [E, d, f] -> [E, f, d]
  MOE_TRY(launch_transpose(dt, dt, L->w_gate, wgut, E, f, f, d, 2 * f, 0, s));           // [E, f, d] -> [E, d, 0:f]
  MOE_TRY(launch_transpose(dt, dt, L->w_up, wgut, E, f, f, d, 2 * f, f, s));             //           -> [E, d, f:2f]
  }
  if (shared && !bt) {
    MOE_TRY(launch_transpose(dt, dt, L->ws_down, wdt + (size_t)E * f * d * eb, 1, d, d, f, d, 0, s));
    MOE_TRY(launch_transpose(dt, dt, L->ws_gate, wgut + (size_t)E * d * 2 * f * eb, 1, f, f, d, 2 * f, 0, s));
    MOE_TRY(launch_transpose(dt, dt, L->ws_up, wgut + (size_t)E * d * 2 * f * eb, 1, f, f, d, 2 * f, f, s));
  }

  // 5. down^T: dHu = dy W_down (grouped, rows gathered from dy, unweighted),
  //    then combine^T and SwiGLU^T per token: d_w = <h, dHu>, dH = w dHu
  GemmLaunch g1{};
  g1.dtype = dt;
  g1.gateup = false;
  g1.a = dya;
  g1.a_rows = tok_of_row;
  g1.a_row_count = T;
  g1.n_groups = G;
  g1.b0 = wdt;
  if (bt) {  // W_down[e] is [d, f]: K = d rows of N = f; the shared expert's as group E
    g1.bt = true;
    g1.b0 = L->w_down;
    if (shared) {
      g1.extra_group = E;
      g1.bx0 = L->ws_down;
    }
  }
  g1.out = at<void>(ws, lo.dh);
  g1.N = f;
  g1.K = d;
  g1.offsets = offsets;
  g1.tiles = tiles;
  g1.n_tiles = n_tiles;
  g1.max_m_tiles = lo.max_tiles;
  g1.b_stream = stream_weights(lo.gemm_rows, G, bm);
  MOE_TRY(launch_gemm(g1, bm, s));
  float* wrow = at<float>(ws, lo.wrow);
  MOE_TRY(launch_swiglu_bwd(dt, T, k, f, at<float>(ws, lo.dh), at<float>(ws, lo.g), at<float>(ws, lo.u),
                            at<void>(ws, lo.h), topk_w, row_of, shared, at<void>(ws, lo.dgu), dtw, wrow, s));

  // 6. gate/up^T: dXp = [dG | dU] [W_gate^T ; W_up^T]^T (grouped, K = 2 f)
  GemmLaunch g2 = g1;
  g2.a = at<void>(ws, lo.dgu);
  g2.a_rows = nullptr;
  g2.b0 = wgut;
  if (bt) {  // K = 2f rows: W_gate[e] ([f, d]) then W_up[e]
    g2.b0 = L->w_gate;
    g2.b1 = L->w_up;
    g2.bt_ksplit = f;
    if (shared) {
      g2.bx0 = L->ws_gate;
      g2.bx1 = L->ws_up;
    }
  }
  g2.out = at<void>(ws, lo.dxp);
  g2.N = d;
  g2.K = 2 * f;
  MOE_TRY(launch_gemm(g2, bm, s));

  // 7. router: logits, logit gradients, dW_router = dl^T x, dx_router = dl W_router
  RouteLaunch rl{x, dt, T, d, E, k, L->score, L->renorm, L->w_router, nullptr, nullptr, nullptr, nullptr, nullptr,
                 at<float>(ws, lo.logits)};
  MOE_TRY(launch_logits(rl, s));
  float* dl = at<float>(ws, lo.dl);
  MOE_TRY(launch_router_bwd(T, E, lo.ep, k, at<float>(ws, lo.logits), topk_idx, dtw, counts, L->score, L->renorm,
                            z_loss_coef, aux_loss_coef, dl, s));
  float* dlt = at<float>(ws, lo.dlt);
  float* xtr = at<float>(ws, lo.xtr);
  float* wrt = at<float>(ws, lo.wrt);
  // panelled transposes (panels of one GEMM tile), zero columns from T to tp
  const int rbm = gemm_kg_bm(0, lo.ep, d, 1), rbn = gemm_kg_bn(rbm, d);
  MOE_TRY(launch_transpose(0, 0, dl, dlt, 1, T, lo.tp, lo.ep, 0, 0, s, rbm));    // [T, ep] -> [ep, tp]
  MOE_TRY(launch_transpose(dt, 0, x, xtr, 1, T, lo.tp, d, 0, 0, s, rbn));        // [T, d] -> [d, tp] fp32
  // dx_router = dl W_router: a GEMM for many experts; with few, the gather
  // below adds it in place
  const bool router_in_gather = E <= kRouterInGatherMaxE;
  if (!router_in_gather)
    MOE_TRY(launch_transpose(0, 0, L->w_router, wrt, 1, E, lo.ep, d, lo.ep, 0, s)); // [E, d] -> [d, ep]
  int32_t* rkoffs = at<int32_t>(ws, lo.rkoffs);
  // nseg K segments of rseg tokens each
  int4* vg = at<int4>(ws, lo.vg);
  int4* red = at<int4>(ws, lo.red);
  int32_t* nred = at<int32_t>(ws, lo.nred);
  MOE_TRY(launch_kg_setup(lo.nseg, nullptr, (int)lo.rseg, lo.ep / rbm, rkoffs, at<int2>(ws, lo.rtiles),
                          at<int32_t>(ws, lo.rn), vg, 0, red, nred, s, d / rbn, 32, at<int32_t>(ws, lo.xb)));
  GemmLaunch rw{};
  rw.dtype = 0;
  rw.gateup = false;
  rw.a = dlt;
  rw.b0 = xtr;
  rw.out = lo.nseg > 1 ? at<void>(ws, lo.rpart) : gr->dw_router;
  rw.N = d;
  rw.K = (int)lo.tp;  // K capacity of the panels
  rw.n_groups = lo.nseg;
  rw.offsets = rkoffs;  // unused in K-grouped mode except as the "grouped" marker
  rw.tiles = at<int2>(ws, lo.rtiles);
  rw.n_tiles = at<int32_t>(ws, lo.rn);
  rw.max_m_tiles = (int64_t)lo.nseg * (lo.ep / rbm);
  rw.koffs = rkoffs;
  rw.xcd_bounds = at<int32_t>(ws, lo.xb);
  rw.vgroups = vg;
  rw.m_rows = lo.ep;
  rw.m_valid = E;
  MOE_TRY(launch_gemm(rw, rbm, s));
  if (lo.nseg > 1)
    MOE_TRY(launch_sum_segments(at<float>(ws, lo.rpart), lo.nseg, (int64_t)lo.ep * d, (int64_t)E * d, gr->dw_router,
                                s));
  if (!router_in_gather) {
    GemmLaunch rx{};
    rx.dtype = 0;
    rx.gateup = false;
    rx.a = dl;
    rx.b0 = wrt;
    rx.out = at<void>(ws, lo.dxr);
    rx.N = d;
    rx.K = lo.ep;
    rx.rows = T;
    MOE_TRY(launch_gemm(rx, 128, s));
  }

  // 8. gather^T: dx
  if (router_in_gather)
    MOE_TRY(launch_gather_bwd(T, d, k, at<float>(ws, lo.dxp), row_of, shared, nullptr, dl, lo.ep, E, L->w_router,
                              gr->dx, s));
  else
    MOE_TRY(launch_gather_bwd(T, d, k, at<float>(ws, lo.dxp), row_of, shared, at<float>(ws, lo.dxr), nullptr, 0, 0,
                              nullptr, gr->dx, s));

  // 9. weight gradients: per-group K segments of transposed activations
  int32_t* koffs = at<int32_t>(ws, lo.koffs);
  const int bm_d = lo.bm_d, bm_gu = lo.bm_gu, bn_d = lo.bn_d, bn_gu = lo.bn_gu, mt_d = lo.mt_d, mt_gu = lo.mt_gu;
  unsigned char* xt = at<unsigned char>(ws, lo.xt);
  unsigned char* dyt = at<unsigned char>(ws, lo.dyt);
  unsigned char* ht = at<unsigned char>(ws, lo.ht);
  unsigned char* dgut = at<unsigned char>(ws, lo.dgut);
  const int ke = dt == 1 ? 64 : 32;  // K elements of one stage
  int32_t* xb = at<int32_t>(ws, lo.xb);
  // chunks of at most cap_d stages (the long groups' partial sums are added in order after the GEMM)
  MOE_TRY(launch_kg_setup(G, offsets, kKPad, mt_d, koffs, at<int2>(ws, lo.kg_tiles), at<int32_t>(ws, lo.kg_n), vg,
                          lo.cap_d, red, nred, s, f / bn_d, ke, xb));
  // per-group zero-padded K segments, panelled for the GEMM that reads them
  // (panels of its row or column tile, K capacity kp >= koffs[G])
  // dY rows are w dy_t, formed here from the fp32 dy (one rounding)
  MOE_TRY(launch_transpose_groups(dt, dt, x, tok_of_row, nullptr, offsets, koffs, G, d, bn_gu, lo.kp, xt, s));
  MOE_TRY(launch_transpose_groups(0, dt, dy, tok_of_row, wrow, offsets, koffs, G, d, bm_d, lo.kp, dyt, s));
  MOE_TRY(launch_transpose_groups(dt, dt, at<void>(ws, lo.h), nullptr, nullptr, offsets, koffs, G, f, bn_d, lo.kp, ht,
                                  s));
  MOE_TRY(launch_transpose_groups(dt, dt, at<void>(ws, lo.dgu), nullptr, nullptr, offsets, koffs, G, 2 * f, bm_gu,
                                  lo.kp, dgut, s));
  GemmLaunch wd{};  // dW_down[e] [d, f] = dY_e^T H_e
  wd.dtype = dt;
  wd.gateup = false;
  wd.a = dyt;
  wd.b0 = ht;
  wd.out = gr->dw_down;
  wd.N = f;
  wd.K = (int)lo.kp;  // K capacity of the panels
  wd.n_groups = lo.vmax;  // chunks
  wd.extra_group = shared ? E : -1;
  wd.xout0 = gr->dws_down;
  wd.offsets = offsets;
  wd.tiles = at<int2>(ws, lo.kg_tiles);
  wd.n_tiles = at<int32_t>(ws, lo.kg_n);
  wd.max_m_tiles = lo.kg_tiles_max;
  wd.koffs = koffs;
  wd.vgroups = vg;
  wd.part = lo.part ? at<float>(ws, lo.part) : nullptr;
  wd.xcd_bounds = xb;
  wd.m_rows = d;
  wd.m_valid = d;
  MOE_TRY(launch_gemm(wd, bm_d, s));
  MOE_TRY(launch_kg_reduce(wd, red, nred, lo.part ? G : 0, s));
  // dW_gate[e], dW_up[e] [f, d] = [dG_e | dU_e]^T X_e: one launch of 2f rows
  MOE_TRY(launch_kg_setup(G, offsets, kKPad, mt_gu, koffs, at<int2>(ws, lo.kg_tiles), at<int32_t>(ws, lo.kg_n), vg,
                          lo.cap_gu, red, nred, s, d / bn_gu, ke, xb));
  GemmLaunch wg = wd;
  wg.a = dgut;
  wg.b0 = xt;
  wg.out = gr->dw_gate;
  wg.out1 = gr->dw_up;
  wg.xout0 = gr->dws_gate;
  wg.xout1 = gr->dws_up;
  wg.N = d;
  wg.m_rows = 2 * f;
  wg.m_valid = 2 * f;
  wg.m0 = f;
  MOE_TRY(launch_gemm(wg, bm_gu, s));
  MOE_TRY(launch_kg_reduce(wg, red, nred, lo.part ? G : 0, s));
  return MOE_OK;
}


const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or option not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch or runtime error";
  }
  return "unknown moe_status";
}

moe_status moe_workspace_size(const moe_layer* L, int64_t T, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID;
  moe_status st = check_layer(L, false);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->top_k)) != MOE_OK) return st;
  *bytes = make_layout(L, T).total;
  return MOE_OK;
}

moe_status moe_route(const moe_layer* L, const void* x, int64_t T, int32_t* topk_idx, float* topk_w,
                     int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  return moe_route_ex(L, x, T, nullptr, topk_idx, topk_w, counts, ws, ws_bytes, stream);
}

moe_status moe_route_ex(const moe_layer* L, const void* x, int64_t T, const moe_route_opts* opts,
                        int32_t* topk_idx, float* topk_w, int32_t* counts, void* ws, size_t ws_bytes,
                        void* stream) {
  moe_status st = check_layer(L, false);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->top_k)) != MOE_OK) return st;
  if ((st = check_opts(opts, T)) != MOE_OK) return st;
  if (T > 0 && (!x || !topk_idx || !topk_w || !aligned16(x))) return MOE_ERR_INVALID;
  const Layout lo = make_layout(L, T);
  if (T > 0 && (!ws || ws_bytes < lo.total || !aligned16(ws))) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (T == 0) {
    if (counts) MOE_TRY(launch_fill_i32(counts, L->n_experts, 0, s));
    return MOE_OK;
  }
  // metrics need the counts: kept in the workspace when the caller wants none
  const bool metrics = opts && opts->metrics;
  int32_t* counts_p = counts ? counts : (metrics ? at<int32_t>(ws, lo.counts) : nullptr);
  int32_t* hist = counts_p ? at<int32_t>(ws, lo.hist) : nullptr;
  const RouteLaunch r = route_launch(L, x, T, opts, topk_idx, topk_w, hist, nullptr, ws, lo);
  MOE_TRY(launch_route(r, s));
  const int tpb = route_tokens_per_block(L->n_experts, T, L->d_model);
  const int nb = (int)((T + tpb - 1) / tpb);
  if (counts_p) MOE_TRY(launch_counts(hist, nb, L->n_experts, counts_p, s));
  if (metrics) MOE_TRY(launch_router_metrics(r.mpart, nb, counts_p, T, L->n_experts, L->top_k, opts->metrics, s));
  return MOE_OK;
}

moe_status moe_bias_update(int32_t n_experts, const int32_t* counts, float rate, float* bias, void* stream) {
  if (n_experts < 1 || !counts || !bias) return MOE_ERR_INVALID;
  if (n_experts > 1024) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  MOE_TRY(launch_bias_update(counts, n_experts, rate, bias, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_permute(const moe_layer* L, const void* x, int64_t T, const int32_t* topk_idx, void* x_perm,
                       int32_t* offsets, int32_t* row_of, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_layer(L, false);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->top_k)) != MOE_OK) return st;
  if (!offsets) return MOE_ERR_INVALID;
  if (T > 0 && (!topk_idx || !row_of)) return MOE_ERR_INVALID;
  if (T > 0 && x_perm && (!x || !aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID;
  const Layout lo = make_layout(L, T);
  if (!ws || ws_bytes < lo.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const int E = L->n_experts, k = L->top_k;
  if (T == 0) {
    MOE_TRY(launch_fill_i32(offsets, E + 1, 0, s));
    return MOE_OK;
  }
  const int tpb = hist_tokens_per_block();
  const int64_t nb = (T + tpb - 1) / tpb;
  int32_t* hist = at<int32_t>(ws, lo.hist);
  int32_t* rank = at<int32_t>(ws, lo.rank);
  int32_t* base = at<int32_t>(ws, lo.base);
  MOE_TRY(launch_hist_rank(topk_idx, T, k, E, hist, rank, s));
  MOE_TRY(launch_scan(hist, (int)nb, E, at<int32_t>(ws, lo.counts), offsets, base, 128,
                      at<int32_t>(ws, lo.n_tiles), at<int2>(ws, lo.tiles), s));
  MOE_TRY(launch_scatter(topk_idx, rank, base, T, k, E, tpb, row_of, at<int32_t>(ws, lo.tok_of_row), x, x_perm,
                         L->d_model * elem_bytes(L->dtype), s));
  return MOE_OK;
}

moe_status moe_grouped_swiglu_workspace_size(int32_t dtype, int32_t n_groups, int32_t d_in, int32_t d_ff,
                                             int64_t rows, size_t* bytes) {
  if (!bytes || n_groups < 1 || d_in <= 0 || d_ff <= 0 || rows < 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d_in % 64 || d_ff % 64) return MOE_ERR_UNSUPPORTED;
  if (rows > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
  const int64_t max_tiles = (rows + kMinTileRows - 1) / kMinTileRows + n_groups;
  size_t p = align_up(sizeof(int32_t));
  p += align_up(sizeof(int2) * (size_t)max_tiles);
  p += align_up((size_t)elem_bytes(dtype) * (size_t)rows * (size_t)d_ff);
  *bytes = p;
  return MOE_OK;
}

moe_status moe_grouped_swiglu(int32_t dtype, int32_t n_groups, int32_t d_in, int32_t d_ff, int64_t rows,
                              const void* a, const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, float* out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  moe_status st = moe_grouped_swiglu_workspace_size(dtype, n_groups, d_in, d_ff, rows, &need);
  if (st != MOE_OK) return st;
  if (!offsets || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down)) return MOE_ERR_INVALID;
  if (rows > 0 && (!a || !out || !aligned16(a) || !aligned16(out))) return MOE_ERR_INVALID;
  if (rows == 0) return MOE_OK;
  if (!ws || ws_bytes < need || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const int bm = gemm_bm_fwd(dtype, rows, n_groups, d_ff, d_in);
  const GemmCaps caps = gemm_bn_caps(dtype, rows, n_groups, d_ff, d_in, d_in);
  const int64_t max_tiles = (rows + kMinTileRows - 1) / kMinTileRows + n_groups;
  int32_t* n_tiles = at<int32_t>(ws, 0);
  int2* tiles = at<int2>(ws, align_up(sizeof(int32_t)));
  void* h = at<void>(ws, align_up(sizeof(int32_t)) + align_up(sizeof(int2) * (size_t)max_tiles));
  MOE_TRY(launch_tiles_from_offsets(offsets, n_groups, bm, n_tiles, tiles, s));
  GemmLaunch gu{};
  gu.dtype = dtype;
  gu.gateup = true;
  gu.a = a;
  gu.b0 = w_gate;
  gu.b1 = w_up;
  gu.out = h;
  gu.N = d_ff;
  gu.K = d_in;
  gu.offsets = offsets;
  gu.tiles = tiles;
  gu.n_tiles = n_tiles;
  gu.max_m_tiles = max_tiles;
  gu.n_groups = n_groups;
  gu.b_stream = stream_weights(rows, n_groups, bm);
  gu.bn_cap = caps.gateup;
  gu.raster_by_group = raster_by_group(rows, n_groups, d_in);
  MOE_TRY(launch_gemm_fwd(gu, bm, s));
  GemmLaunch dn = gu;
  dn.gateup = false;
  dn.bn_cap = caps.down;
  dn.raster_by_group = false;
  dn.a = h;
  dn.b0 = w_down;
  dn.b1 = nullptr;
  dn.out = out;
  dn.N = d_in;
  dn.K = d_ff;
  MOE_TRY(launch_gemm_fwd(dn, bm, s));
  return MOE_OK;
}

moe_status moe_combine(const moe_layer* L, int64_t T, const float* y_perm, const int32_t* row_of,
                       const float* topk_w, const float* y_shared, float* y, void* stream) {
  moe_status st = check_layer(L, false);
  if (st != MOE_OK) return st;
  if ((st = check_T(T, L->top_k)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!y_perm || !row_of || !topk_w || !y) return MOE_ERR_INVALID;
  if (!aligned16(y_perm) || !aligned16(y) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID;
  (void)hipGetLastError();
  MOE_TRY(launch_combine(T, L->d_model, L->top_k, y_perm, row_of, topk_w, y_shared, y, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_layer* L, const void* x, int64_t T, float* y, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(L, x, T, nullptr, y, topk_idx, topk_w, counts, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

// Scratch of moe_forward_noalloc: one array per GPU, held until the process
// ends. In host code `scratch` names a host-side stand-in, not device
// memory: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// used for every launch.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (null on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

moe_status moe_forward_noalloc(const moe_layer* L, const void* x, int64_t T, float* y, int32_t* topk_idx,
                               float* topk_w, int32_t* counts, void* stream) {
  size_t need = 0;
  moe_status st = moe_workspace_size(L, T, &need);
  if (st != MOE_OK) return st;
  if (need > MOE_NOALLOC_BYTES) return MOE_ERR_WORKSPACE;
  if (T == 0) return forward_impl(L, x, T, nullptr, y, topk_idx, topk_w, counts, nullptr, 0, (hipStream_t)stream,
                                  nullptr);
  // forward_impl reads no workspace byte it has not written in the same
  // call, so what earlier calls left in the array needs no clearing
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_HIP;
  return forward_impl(L, x, T, nullptr, y, topk_idx, topk_w, counts, ws, MOE_NOALLOC_BYTES, (hipStream_t)stream,
                      nullptr);
}

moe_status moe_forward_ex(const moe_layer* L, const void* x, int64_t T, const moe_route_opts* opts, float* y,
                          int32_t* topk_idx, float* topk_w, int32_t* counts, void* ws, size_t ws_bytes, void* stream,
                          moe_timing* timing) {
  return forward_impl(L, x, T, opts, y, topk_idx, topk_w, counts, ws, ws_bytes, (hipStream_t)stream, timing);
}

moe_status moe_timing_create(moe_timing** out) {
  if (!out) return MOE_ERR_INVALID;
  moe_timing* t = new (std::nothrow) moe_timing;
  if (!t) return MOE_ERR_HIP;
  for (int i = 0; i <= MOE_N_PHASES; ++i) {
    // timing-only events: no system-scope fence (no cache writeback and
    // invalidation between the phases they separate)
    if (hipEventCreateWithFlags(&t->ev[i], hipEventDisableSystemFence) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(t->ev[j]);
      delete t;
      return MOE_ERR_HIP;
    }
  }
  t->mask = (1u << MOE_N_PHASES) - 1u;
  *out = t;
  return MOE_OK;
}

moe_status moe_timing_select(moe_timing* t, uint32_t phase_mask) {
  if (!t || phase_mask == 0 || (phase_mask >> MOE_N_PHASES)) return MOE_ERR_INVALID;
  t->mask = phase_mask;
  return MOE_OK;
}

moe_status moe_timing_destroy(moe_timing* t) {
  if (!t) return MOE_ERR_INVALID;
  for (int i = 0; i <= MOE_N_PHASES; ++i) (void)hipEventDestroy(t->ev[i]);
  delete t;
  return MOE_OK;
}

moe_status moe_timing_read(moe_timing* t, float* phase_ms) {
  if (!t || !phase_ms) return MOE_ERR_INVALID;
  int last = 0;  // the latest boundary recorded
  for (int i = 0; i <= MOE_N_PHASES; ++i)
    if (((t->mask << 1) >> i) & 3u) last = i;
  if (hipEventSynchronize(t->ev[last]) != hipSuccess) return MOE_ERR_HIP;
  for (int i = 0; i < MOE_N_PHASES; ++i) {
    float ms = -1.0f;
    if (((t->mask >> i) & 1u) && hipEventElapsedTime(&ms, t->ev[i], t->ev[i + 1]) != hipSuccess) return MOE_ERR_HIP;
    phase_ms[i] = ms;
  }
  return MOE_OK;
}

}  // extern "C"
