// Host side of the C ABI declared in include/moe.h: validation, workspace
// layout, launch sequencing and hipGraph capture of decode-sized calls.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "../../include/moe.h"
#include "costmodel_params.h"
#include "layer.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                    \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// Tile configurations the library has kernels for: 0 = streaming, 1..3 =
// tiled with row blocks of cfg_rows(cfg).  bf16 stops at 64-row blocks (a
// 128-row bf16 token tile would not leave registers for the accumulators).
constexpr int kNumCfgs = 4;
int num_cfgs(int) { return kNumCfgs; }

int fmt_of(const moe_layer_desc& d) {
  if (d.w_format == MOE_W_BF16 && d.a_format == MOE_A_BF16) return F_BF16;
  if (d.w_format == MOE_W_FP8_CHANNEL && d.a_format == MOE_A_FP8_TOKEN) return F_FP8_CH;
  if (d.w_format == MOE_W_FP8_BLOCK128 && d.a_format == MOE_A_FP8_G128) return F_FP8_BLK;
  if (d.w_format == MOE_W_MXFP4 && d.a_format == MOE_A_MXFP8_G32) return F_MX;
  return -1;
}

int wbits_of(int fmt) { return fmt == F_BF16 ? 16 : fmt == F_MX ? 4 : 8; }
int xbits_of(int fmt) { return fmt == F_BF16 ? 16 : 8; }

int validate_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_EINVAL, "desc is NULL");
  if (d->hidden <= 0 || d->inter <= 0) return fail(MOE_EINVAL, "hidden/inter must be positive");
  if (d->hidden % 128 || d->inter % 128)
    return fail(MOE_EUNSUPPORTED, "hidden (%d) and inter (%d) must be multiples of 128", d->hidden,
                d->inter);
  if (d->hidden > 16384 || d->inter > 16384)
    return fail(MOE_EUNSUPPORTED, "hidden and inter are limited to 16384");
  if (d->num_experts < 1 || d->num_experts > 256)
    return fail(MOE_EINVAL, "num_experts must be in [1, 256], got %d", d->num_experts);
  int kmax = d->num_experts < 16 ? d->num_experts : 16;
  if (d->top_k < 1 || d->top_k > kmax)
    return fail(MOE_EINVAL, "top_k must be in [1, %d], got %d", kmax, d->top_k);
  if (d->shared_experts != 0 && d->shared_experts != 1)
    return fail(MOE_EUNSUPPORTED, "shared_experts must be 0 or 1");
  if (d->shared_experts && d->shared_inter != d->inter)
    return fail(MOE_EUNSUPPORTED, "the shared expert must have the routed intermediate size");
  if (d->score_fn < MOE_SCORE_SOFTMAX || d->score_fn > MOE_SCORE_PROBS)
    return fail(MOE_EINVAL, "unknown score_fn %d", d->score_fn);
  if (d->renormalize != 1) return fail(MOE_EUNSUPPORTED, "only renormalize = 1 is supported");
  if (fmt_of(*d) < 0)
    return fail(MOE_EUNSUPPORTED, "unsupported weight/activation format pair (%d, %d)", d->w_format,
                d->a_format);
  if (d->activation < MOE_ACT_SWIGLU || d->activation > MOE_ACT_RELU2)
    return fail(MOE_EINVAL, "unknown activation %d", d->activation);
  if (!(d->act_limit == d->act_limit)) return fail(MOE_EINVAL, "act_limit is NaN");
  if (d->max_tokens < 1) return fail(MOE_EINVAL, "max_tokens must be >= 1");
  if ((long)d->max_tokens * d->top_k > (1L << 20))
    return fail(MOE_EUNSUPPORTED, "max_tokens * top_k must not exceed 1048576");
  return MOE_OK;
}

struct Layout {
  size_t ids, w, counts, indptr, gather, inv, active, tiles, meta, chunk;
  size_t xq, xs, h, hq, hs, out_slot, dstate, cmth, total;
  long S, S_tot, G, max_tiles, nchunks;
  // single-launch decode layer state: barrier words, then per-parity row
  // maxima and (token, channel-block) arrival counters
  long amax_stride, cnt_stride;
  size_t dstate_bytes;
};

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

Layout make_layout(const moe_layer_desc& d) {
  Layout L{};
  long T = d.max_tokens, k = d.top_k, E = d.num_experts, H = d.hidden, I = d.inter;
  L.G = E + d.shared_experts;
  L.S = T * k;
  L.S_tot = L.S + (d.shared_experts ? T : 0);
  L.max_tiles = L.S_tot / 16 + L.G + 1;
  L.nchunks = (T + 1024 / k - 1) / (1024 / k);   // whole-token chunks of <= 1024 slots
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.ids = take(4 * L.S);
  L.w = take(4 * L.S);
  L.counts = take(4 * L.G);
  L.indptr = take(4 * (L.G + 1));
  L.gather = take(4 * L.S_tot);
  L.inv = take(4 * L.S);
  L.active = take(4 * L.G);
  L.tiles = take(8 * L.max_tiles);
  L.meta = take(4 * META_WORDS);
  L.chunk = take(4 * L.nchunks * E);
  L.xq = take((size_t)T * H);
  L.xs = take((size_t)T * (H / 32) * 4);
  L.h = take((size_t)L.S_tot * I * 4);
  L.hq = take((size_t)L.S_tot * I);
  L.hs = take((size_t)L.S_tot * (I / 32) * 4);
  L.out_slot = take((size_t)L.S_tot * H * 4);
  L.amax_stride = (long)DECODE_STREAM_TOKENS * (k + d.shared_experts);
  L.cnt_stride = (long)DECODE_STREAM_TOKENS * (H / 16);
  L.dstate_bytes = 256 + 4 * 2 * (size_t)(L.amax_stride + L.cnt_stride);
  L.dstate = take(L.dstate_bytes);
  L.cmth = take(sizeof kCostModelTheta);   // the cost model's parameters, read by dispatch
  L.total = off;
  return L;
}

// One instantiated decode graph per (token count, stream).  The pointers it
// was captured with are kept: a call with other buffers re-captures and
// updates the instance in place (hipGraphExecUpdate), so the number of
// instances never grows with the buffers a caller rotates through.
struct GraphKey {
  int T;
  const void* st;
  bool operator<(const GraphKey& o) const { return std::tie(T, st) < std::tie(o.T, o.st); }
};
struct GraphPtrs {
  const void *x, *scores, *y;
  const void* wp[12];
  bool operator==(const GraphPtrs& o) const {
    return x == o.x && scores == o.scores && y == o.y && memcmp(wp, o.wp, sizeof wp) == 0;
  }
};
struct GraphEntry {
  hipGraphExec_t exec;
  GraphPtrs ptrs;
};

}  // namespace

struct moe_ws {
  moe_layer_desc d;
  Layout L;
  char* base;
  int fmt;
  int force_cfg = -1;
  int graphs = 1;
  int fused_decode = 0;    // single-launch decode layer: opt-in (slower on gfx950, see the header)
  int config_model = 1;    // fitted cost model picks the configuration (0: the histogram rule)
  int decode_grid = -1;   // resident workgroups of the decode layer (computed once)
  int device = 0;
  std::map<GraphKey, GraphEntry> execs;
  hipEvent_t stage_ev[14][2] = {};   // 0-6 forward stages, 7-13 backward stages
  bool any_stage_events() const {
    for (int i = 0; i < 7; ++i)
      if (stage_ev[i][0] || stage_ev[i][1]) return true;
    return false;
  }
  template <class T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(base + off);
  }
};

namespace {

int device_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

// ---------------------------------------------------------------------------
// Host side of the fitted configuration cost model.  Before the histogram
// exists the host only knows the batch, so it evaluates the model on the two
// routings that bound what the histogram can be (T*k rows spread evenly
// over the experts, and packed into k experts of T rows; a shared expert
// adds a group of T rows).  Over the
// sets of kernel launches it takes the one whose best configuration's
// predicted time, averaged over those routings with kRoutingPrior's weights,
// plus kLaunchUs for every launch beyond the first, is least (the first such
// set on a tie), and passes the
// configurations those launches serve to the dispatch kernel, which picks,
// on the real histogram, the least predicted time among them.
// grouped_gemm_amd/costmodel.py (candidate_mask) computes the same set.
// a kernel family launched for both projections that the device may not
// choose: a launch that returns at once still holds the stream ~4.7 us
constexpr double kLaunchUs = 9.0;
// weights of the two bounding routings (even, packed): routers trained with
// load balancing keep histograms near even
constexpr double kRoutingPrior[2] = {0.8, 0.2};

void add_groups(HistStats& h, long c, long m) {
  if (c <= 0 || m <= 0) return;
  h.mx = c > h.mx ? (int)c : h.mx;
  h.active += (int)m;
  h.rows += (int)(c * m);
  h.s16 += (int)(m * ((c + 15) / 16));
  h.s32 += (int)(m * ((c + 31) / 32));
  h.s64 += (int)(m * ((c + 63) / 64));
  h.s128 += (int)(m * ((c + 127) / 128));
}


// The configurations each kernel launch serves (bit c): the streaming
// kernel; bf16 one launch per tiled configuration; FP8 one for 32/64-row
// blocks and one for 128-row blocks; MXFP4 one for every tiled one.
int launch_families(int fmt, int* fam) {
  fam[0] = 1;
  if (fmt == F_MX) {
    fam[1] = 14;
    return 2;
  }
  fam[1] = 6;
  fam[2] = 8;
  return 3;
}

CostModel cost_model(const moe_ws* ws, int T) {
  CostModel m{};
  m.th = ws->at<double>(ws->L.cmth);
  if (!ws->config_model || ws->force_cfg >= 0 || T < 0) return m;   // off: the rule
  const double* th = &kCostModelTheta[0][0];
  const moe_layer_desc& d = ws->d;
  const long E = d.num_experts, k = d.top_k, q = (long)T * k / E, r = (long)T * k % E;
  const int nc = num_cfgs(ws->fmt), cus = device_cus();
  HistStats h[2] = {};
  add_groups(h[0], q + 1, r);                    // even: the first r experts one row more
  add_groups(h[0], q, E - r);
  add_groups(h[1], T, k);                        // packed
  for (auto& x : h)
    if (d.shared_experts) add_groups(x, T, 1);
  double t[2][kNumCfgs];
  for (int i = 0; i < 2; ++i)
    for (int c = 0; c < nc; ++c) t[i][c] = cost_model_time(th, h[i], c, ws->fmt, d.hidden, d.inter, T, cus);
  int fam[4];
  const int nf = launch_families(ws->fmt, fam);
  int best = 0;
  double best_cost = 0.0;
  for (int sel = 1; sel < (1 << nf); ++sel) {
    // every configuration a launched kernel serves is a candidate
    int mask = 0, nl = 0;
    for (int i = 0; i < nf; ++i)
      if ((sel >> i) & 1) {
        mask |= fam[i];
        ++nl;
      }
    mask &= (1 << nc) - 1;
    if (!mask) continue;
    double cost = 0.0;
    for (int i = 0; i < 2; ++i) {
      double mn = 0.0;
      bool any = false;
      for (int c = 0; c < nc; ++c)
        if ((mask >> c) & 1 && (!any || t[i][c] < mn)) {
          mn = t[i][c];
          any = true;
        }
      cost += kRoutingPrior[i] * mn;
    }
    cost += kLaunchUs * (nl - 1);
    if (best == 0 || cost < best_cost) {
      best = mask;
      best_cost = cost;
    }
  }
  m.on = 1;
  m.mask = best;
  return m;
}

DispatchArgs dispatch_args(const moe_ws* ws, int T) {
  DispatchArgs a{};
  const moe_layer_desc& d = ws->d;
  a.T = T;
  a.E = d.num_experts;
  a.k = d.top_k;
  a.score_fn = d.score_fn;
  a.shared = d.shared_experts;
  a.ids = ws->at<int32_t>(ws->L.ids);
  a.w = ws->at<float>(ws->L.w);
  a.counts = ws->at<int32_t>(ws->L.counts);
  a.indptr = ws->at<int32_t>(ws->L.indptr);
  a.gather = ws->at<int32_t>(ws->L.gather);
  a.inv = ws->at<int32_t>(ws->L.inv);
  a.active = ws->at<int32_t>(ws->L.active);
  a.tiles = ws->at<int32_t>(ws->L.tiles);
  a.meta = ws->at<int32_t>(ws->L.meta);
  a.chunk = ws->at<int32_t>(ws->L.chunk);
  a.force_cfg = ws->force_cfg;
  a.H = d.hidden;
  a.I = d.inter;
  a.wbits = wbits_of(ws->fmt);
  a.xbits = xbits_of(ws->fmt);
  a.num_cfgs = num_cfgs(ws->fmt);
  a.cus = device_cus();
  a.fmt = ws->fmt;
  a.cm = cost_model(ws, T);
  if (a.cm.on && !(a.cm.mask & (a.cm.mask - 1))) {
    // one candidate: the dispatch kernel takes it without evaluating the model
    a.force_cfg = __builtin_ctz(a.cm.mask);
    a.cm.on = 0;
  }
  return a;
}

// The clamp of the bounded activations (the desc's, else 10 for bounded
// SwiGLU and 7 for SwiGLU-OAI).
float act_limit(const moe_layer_desc& d) {
  if (d.act_limit > 0.0f) return d.act_limit;
  return d.activation == MOE_ACT_SWIGLU_BOUNDED ? 10.0f : (d.activation == MOE_ACT_SWIGLU_OAI ? 7.0f : 0.0f);
}

GemmArgs gemm_args(const moe_ws* ws) {
  GemmArgs g{};
  g.E = ws->d.num_experts;
  g.act = ws->d.activation;
  g.act_limit = act_limit(ws->d);
  g.counts = ws->at<int32_t>(ws->L.counts);
  g.indptr = ws->at<int32_t>(ws->L.indptr);
  g.active = ws->at<int32_t>(ws->L.active);
  g.tiles = ws->at<int32_t>(ws->L.tiles);
  g.meta = ws->at<int32_t>(ws->L.meta);
  g.cfg_self = -1;
  g.max_group_rows = 1 << 30;
  return g;
}

// Which kernel families the device's choice can land on, from bounds the
// host knows without reading the histogram: rows_tot rows spread over at
// most min(G, rows_tot) groups.  The device rule picks the streaming kernel
// for batches of at most DECODE_STREAM_TOKENS tokens, and otherwise exactly
// when a 32-row tiled grid would have fewer items than half the CUs, with
// items = (sum over groups of ceil(rows/32)) * (I/128), and that sum lies in
// [ceil(rows_tot/32), floor((rows_tot + 31 * groups) / 32)] (each group
// adds at most 31/32 of a tile to its exact share).  A forced configuration
// is known outright.
// With the cost model on, the candidates are the model's mask (the device
// picks within it).
struct Candidates {
  bool stream, small, big;   // streaming kernel; tiled configurations 1-2; configuration 3
  int mask;                  // configurations whose kernels are launched (bit c)
};
Candidates from_flags(bool stream, bool small, bool big) {
  return {stream, small, big, (stream ? 1 : 0) | (small ? 6 : 0) | (big ? 8 : 0)};
}
Candidates from_mask(int mask) { return {(mask & 1) != 0, (mask & 6) != 0, (mask & 8) != 0, mask}; }
Candidates forced(int cfg) { return from_mask(1 << cfg); }
Candidates candidates(const moe_ws* ws, long rows_tot, int T) {
  if (ws->force_cfg >= 0) return forced(ws->force_cfg);
  const CostModel m = cost_model(ws, T);
  if (m.on) return from_mask(m.mask);
  // the device rule streams every batch of at most DECODE_STREAM_TOKENS tokens
  if (T <= DECODE_STREAM_TOKENS || num_cfgs(ws->fmt) <= 1) return from_flags(true, false, false);
  const long cus = device_cus(), cb = ws->d.inter / 128;
  const long G = ws->L.G;
  const long groups = rows_tot < G ? rows_tot : G;
  const long lo = (rows_tot + 31) / 32, hi = (rows_tot + 31 * groups) / 32;
  const bool tiled = 2 * hi * cb >= cus;
  // configuration 3 needs a group above 64 rows, at least 64 rows per
  // active group and CFG3_MIN_ROWS rows; it is certain when every group
  // count bound forces it (mean over all groups above 64, enough items)
  const bool big = tiled && num_cfgs(ws->fmt) > 3 && rows_tot >= CFG3_MIN_ROWS && rows_tot > 64;
  const bool big_certain = big && 2 * lo * cb >= cus && rows_tot > 64 * G;
  return from_flags(2 * lo * cb < cus, tiled && !big_certain, big);
}

// Run a projection with the kernel families the configuration can land on;
// a launch whose family the device did not choose returns at once.
// `tiled_out` and `tiled_scale` redirect the fused gate/up output of the
// tiled kernels, which requantise the intermediate in their epilogue for the
// 1x128 and MX formats.
hipError_t run_gemm_c(const moe_ws* ws, bool gateup, GemmArgs g, void* tiled_out, void* tiled_scale,
                      const Candidates& cand, hipStream_t st) {
  if (cand.stream) {
    g.cfg_self = 0;
    // a streaming launch the device may not choose gets a capped grid whose
    // workgroups stride the work items: when it returns at once it starts
    // a few thousand workgroups instead of one per (group, 16 channels)
    if (cand.mask != 1) g.grid_cap = device_cus() * 8;
    hipError_t e = launch_gemm_stream(ws->fmt, gateup, g, st);
    g.grid_cap = 0;
    if (e != hipSuccess) return e;
  }
  if (!cand.small && !cand.big) return hipSuccess;
  if (tiled_out) {
    g.out = tiled_out;
    g.out_scale = tiled_scale;
  }
  g.cfg_self = ws->force_cfg > 0 ? ws->force_cfg : -1;   // any tiled configuration
  // MXFP4 runs every tiled configuration in one kernel (four-wave blocks
  // throughout), so it takes one launch whichever of them the device picks
  if (ws->fmt == F_MX) return launch_gemm_pipe(ws->fmt, gateup, 0, g, st);
  if (cand.small) {
    hipError_t e = launch_gemm_pipe(ws->fmt, gateup, 0, g, st);
    if (e != hipSuccess) return e;
  }
  if (cand.big) return launch_gemm_pipe(ws->fmt, gateup, 1, g, st);
  return hipSuccess;
}

hipError_t run_gemm(const moe_ws* ws, bool gateup, GemmArgs g, void* tiled_out, void* tiled_scale,
                    long rows_tot, int T, hipStream_t st) {
  return run_gemm_c(ws, gateup, g, tiled_out, tiled_scale, candidates(ws, rows_tot, T), st);
}

// Whether the single-launch decode layer serves a call of T tokens: small
// batches, the streaming configuration (or the device's choice), K of both
// projections a multiple of four 128-wide steps, and a grid that fits.
bool use_fused_decode(moe_ws* ws, int T) {
  const moe_layer_desc& d = ws->d;
  if (!ws->fused_decode || T > DECODE_STREAM_TOKENS) return false;
  if (ws->force_cfg > 0) return false;
  if (d.hidden % 512 || d.inter % 512) return false;
  if (ws->decode_grid < 0) ws->decode_grid = decode_layer_grid(ws->fmt, d.activation, device_cus());
  return ws->decode_grid > 0;
}

int enqueue_fused_decode(moe_ws* ws, const moe_weights* w, const uint16_t* x, const float* scores,
                         int T, uint16_t* y, hipStream_t st) {
  const moe_layer_desc& d = ws->d;
  const Layout& L = ws->L;
  const bool relu2 = d.activation == MOE_ACT_RELU2;
  DecodeArgs a{};
  a.scores = scores;
  a.x = x;
  a.y = y;
  a.T = T;
  a.E = d.num_experts;
  a.k = d.top_k;
  a.score_fn = d.score_fn;
  a.shared = d.shared_experts;
  a.H = d.hidden;
  a.I = d.inter;
  a.wg = (const uint8_t*)(relu2 ? w->w_up : w->w_gate);
  a.wu = (const uint8_t*)w->w_up;
  a.wd = (const uint8_t*)w->w_down;
  a.sg = relu2 ? w->s_up : w->s_gate;
  a.su = w->s_up;
  a.sd = w->s_down;
  a.shg = (const uint8_t*)(relu2 ? w->sh_up : w->sh_gate);
  a.shu = (const uint8_t*)w->sh_up;
  a.shd = (const uint8_t*)w->sh_down;
  a.ssg = relu2 ? w->ss_up : w->ss_gate;
  a.ssu = w->ss_up;
  a.ssd = w->ss_down;
  a.act = d.activation;
  a.act_limit = act_limit(d);
  a.ids = ws->at<int32_t>(L.ids);
  a.w = ws->at<float>(L.w);
  a.counts = ws->at<int32_t>(L.counts);
  a.indptr = ws->at<int32_t>(L.indptr);
  a.gather = ws->at<int32_t>(L.gather);
  a.inv = ws->at<int32_t>(L.inv);
  a.meta = ws->at<int32_t>(L.meta);
  a.h = ws->at<float>(L.h);
  a.out_slot = ws->at<uint16_t>(L.out_slot);
  a.bar = ws->at<int32_t>(L.dstate);
  a.amax = (uint32_t*)(ws->at<char>(L.dstate) + 256);
  a.cnt = (int32_t*)(a.amax + 2 * L.amax_stride);
  a.amax_stride = (int)L.amax_stride;
  a.cnt_stride = (int)L.cnt_stride;
  a.spin_limit = 1L << 21;
  auto mark = [&](int stage, int which) -> hipError_t {
    hipEvent_t e = ws->stage_ev[stage][which];
    return e ? hipEventRecord(e, st) : hipSuccess;
  };
  HIP_TRY(mark(6, 0), "event record");
  HIP_TRY(launch_decode_layer(ws->fmt, a, ws->decode_grid, st), "decode layer launch");
  HIP_TRY(mark(6, 1), "event record");
  return MOE_OK;
}

int enqueue_layer(moe_ws* ws, const moe_weights* w, const uint16_t* x, const float* scores, int T,
                  uint16_t* y, hipStream_t st) {
  if (use_fused_decode(ws, T)) return enqueue_fused_decode(ws, w, x, scores, T, y, st);
  const moe_layer_desc& d = ws->d;
  const Layout& L = ws->L;
  const int S = T * d.top_k, S_tot = S + (d.shared_experts ? T : 0);
  const int G = (int)L.G;
  auto mark = [&](int stage, int which) -> hipError_t {
    hipEvent_t e = ws->stage_ev[stage][which];
    return e ? hipEventRecord(e, st) : hipSuccess;
  };
  DispatchArgs da = dispatch_args(ws, T);
  da.scores = scores;
  const bool quant = ws->fmt != F_BF16;
  // the input quantisation rides on the routing launch's spare waves (its
  // stage events stay empty)
  if (quant)
    da.fq = QuantArgs{x, 1, T, d.hidden, nullptr, ws->at<uint8_t>(L.xq), ws->at<void>(L.xs),
                      d.a_format};
  HIP_TRY(mark(0, 0), "event record");
  HIP_TRY(launch_dispatch(da, st), "dispatch launch");
  HIP_TRY(mark(0, 1), "event record");
  HIP_TRY(mark(1, 0), "event record");
  HIP_TRY(mark(1, 1), "event record");
  int max_groups = d.num_experts < S ? d.num_experts : S;
  max_groups += d.shared_experts;
  if (max_groups > G) max_groups = G;
  GemmArgs g1 = gemm_args(ws);
  // ReLU^2 has no gate projection: the up weights serve as both operands
  const bool relu2 = d.activation == MOE_ACT_RELU2;
  g1.w0 = (const uint8_t*)(relu2 ? w->w_up : w->w_gate);
  g1.w1 = (const uint8_t*)w->w_up;
  g1.w0s = relu2 ? w->s_up : w->s_gate;
  g1.w1s = w->s_up;
  g1.sh_w0 = (const uint8_t*)(relu2 ? w->sh_up : w->sh_gate);
  g1.sh_w1 = (const uint8_t*)w->sh_up;
  g1.sh_w0s = relu2 ? w->ss_up : w->ss_gate;
  g1.sh_w1s = w->ss_up;
  g1.N = d.inter;
  g1.K = d.hidden;
  g1.a = quant ? ws->at<uint8_t>(L.xq) : (const uint8_t*)x;
  g1.a_scale = quant ? ws->at<void>(L.xs) : nullptr;
  g1.gather = ws->at<int32_t>(L.gather);
  g1.gather_div = d.top_k;
  g1.out = ws->at<void>(L.h);
  g1.max_groups = max_groups;
  g1.max_rows = S_tot;
  g1.max_group_rows = T;   // a token takes at most one slot per group
  // the tiled kernels requantise 1x128 and MX intermediates themselves
  const bool fused_requant = ws->fmt == F_FP8_BLK || ws->fmt == F_MX;
  HIP_TRY(mark(2, 0), "event record");
  HIP_TRY(run_gemm(ws, true, g1, fused_requant ? ws->at<void>(L.hq) : nullptr,
                   fused_requant ? ws->at<void>(L.hs) : nullptr, S_tot, T, st),
          "gate/up grouped GEMM launch");
  HIP_TRY(mark(2, 1), "event record");
  // with the fused requantisation only the streaming configuration leaves
  // fp32 h behind; skip the launch when that configuration cannot occur
  if (quant && (!fused_requant || candidates(ws, S_tot, T).stream)) {
    QuantArgs q{ws->at<void>(L.h), 0, S_tot, d.inter, nullptr, ws->at<uint8_t>(L.hq),
                ws->at<void>(L.hs), d.a_format};
    if (fused_requant) {   // only the streaming configuration left fp32 h behind
      q.meta = ws->at<int32_t>(L.meta);
      q.only_cfg = 0;
    }
    HIP_TRY(mark(3, 0), "event record");
    HIP_TRY(launch_quant(q, st), "intermediate quantisation launch");
    HIP_TRY(mark(3, 1), "event record");
  }
  GemmArgs g2 = gemm_args(ws);
  g2.w0 = (const uint8_t*)w->w_down;
  g2.w0s = w->s_down;
  g2.sh_w0 = (const uint8_t*)w->sh_down;
  g2.sh_w0s = w->ss_down;
  g2.N = d.hidden;
  g2.K = d.inter;
  g2.a = quant ? ws->at<uint8_t>(L.hq) : ws->at<uint8_t>(L.h);
  g2.a_scale = quant ? ws->at<void>(L.hs) : nullptr;
  g2.gather = nullptr;
  g2.gather_div = 1;
  g2.out = ws->at<void>(L.out_slot);
  g2.max_groups = max_groups;
  g2.max_rows = S_tot;
  g2.max_group_rows = T;
  g2.row_w = ws->at<float>(L.w);          // weight of slot = w[gather[slot]]
  g2.row_w_idx = ws->at<int32_t>(L.gather);
  g2.row_w_n = S;
  HIP_TRY(mark(4, 0), "event record");
  HIP_TRY(run_gemm(ws, false, g2, nullptr, nullptr, S_tot, T, st), "down grouped GEMM launch");
  HIP_TRY(mark(4, 1), "event record");
  CombineArgs c{ws->at<void>(L.out_slot), ws->at<float>(L.w), ws->at<int32_t>(L.inv), T,
                d.top_k, d.hidden, d.shared_experts, y, 1};
  HIP_TRY(mark(5, 0), "event record");
  HIP_TRY(launch_combine(c, st), "combine launch");
  HIP_TRY(mark(5, 1), "event record");
  return MOE_OK;
}

int check_weights(const moe_ws* ws, const moe_weights* w) {
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  // the two-weight ReLU^2 form reads no gate weights
  const bool gate = ws->d.activation != MOE_ACT_RELU2;
  if ((gate && !w->w_gate) || !w->w_up || !w->w_down)
    return fail(MOE_EINVAL, "null routed weight pointer");
  if (ws->fmt != F_BF16 && ((gate && !w->s_gate) || !w->s_up || !w->s_down))
    return fail(MOE_EINVAL, "null weight scale pointer");
  if (ws->d.shared_experts) {
    if ((gate && !w->sh_gate) || !w->sh_up || !w->sh_down)
      return fail(MOE_EINVAL, "null shared-expert weight pointer");
    if (ws->fmt != F_BF16 && ((gate && !w->ss_gate) || !w->ss_up || !w->ss_down))
      return fail(MOE_EINVAL, "null shared-expert scale pointer");
  }
  return MOE_OK;
}

// ------------------------------------------------- no-allocation dispatch
// Scratch of moe_dispatch_noalloc in device memory the library owns for the
// life of the process (one copy per GPU, each at its own address): the meta
// words, the active-group list, the block table and the per-chunk expert
// histograms of the largest dispatch the entry point accepts (1,048,576
// slots, 256 experts).  The host never uses the array's name as an address;
// it takes each device's address from hipGetSymbolAddress once.
constexpr int NA_MAX_SLOTS = 1 << 20;
constexpr int NA_MAX_E = 256;
constexpr int NA_MAX_TILES = NA_MAX_SLOTS / 16 + NA_MAX_E + 1;
constexpr int NA_MAX_CHUNKS = 1100;   // ceil(T / floor(1024 / k)) <= 1035 for T*k <= 2^20
constexpr size_t NA_META = 0, NA_ACTIVE = 64, NA_TILES = NA_ACTIVE + NA_MAX_E,
                 NA_CHUNK = NA_TILES + 2 * (size_t)NA_MAX_TILES,
                 NA_WORDS = NA_CHUNK + (size_t)NA_MAX_CHUNKS * NA_MAX_E;
static __device__ __align__(256) int32_t scratch[NA_WORDS];

constexpr int NA_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[NA_MAX_DEVICES] = {};

// The calling device's copy of the scratch array (resolved once per device,
// with that device current).
int scratch_for_current_device(int32_t** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "get device");
  if (dev < 0 || dev >= NA_MAX_DEVICES) return fail(MOE_EUNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch symbol address");
    g_scratch_ptr[dev] = (int32_t*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dispatch_noalloc(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                         int32_t* m_indptr, int32_t* gather, int32_t* inv, void* stream) {
  if (E < 1 || E > NA_MAX_E) return fail(MOE_EINVAL, "E must be in [1, %d]", NA_MAX_E);
  const int kmax = E < 16 ? E : 16;
  if (k < 1 || k > kmax) return fail(MOE_EINVAL, "k must be in [1, %d]", kmax);
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if ((long)T * k > NA_MAX_SLOTS)
    return fail(MOE_ECAPACITY, "T*k = %ld exceeds the %d slots of the static scratch", (long)T * k,
                NA_MAX_SLOTS);
  if (!counts || !m_indptr || (T > 0 && (!topk_ids || !gather || !inv)))
    return fail(MOE_EINVAL, "null pointer");
  const long TC = 1024 / k, nch = (T + TC - 1) / TC;
  if (nch > NA_MAX_CHUNKS) return fail(MOE_ECAPACITY, "%ld chunks exceed the static scratch", nch);
  int32_t* scr = nullptr;
  int rc = scratch_for_current_device(&scr);
  if (rc) return rc;
  DispatchArgs a{};
  a.T = T;
  a.E = E;
  a.k = k;
  a.shared = 0;
  a.ids_in = topk_ids;
  a.counts = counts;
  a.indptr = m_indptr;
  a.gather = gather;
  a.inv = inv;
  a.meta = scr + NA_META;
  a.active = scr + NA_ACTIVE;
  a.tiles = scr + NA_TILES;
  a.chunk = scr + NA_CHUNK;
  a.force_cfg = 0;     // no layer shape: the table is built for the streaming height
  a.H = a.I = 128;
  a.wbits = a.xbits = 8;
  a.num_cfgs = 1;
  a.cus = device_cus();
  HIP_TRY(launch_dispatch(a, (hipStream_t)stream), "dispatch launch");
  return MOE_OK;
}

// ---------------------------------------------------------------- backward
namespace {

struct BwdScratch {
  size_t G, U, R, Hb, DGU, DA, WdT, WguT, WDY, tok, chunks, nch, pbase, multi, order, partial,
      total;
  int piece;       // rows per weight-gradient work chunk
  int max_chunks;  // bound on the chunks
};

// Weight-gradient work chunks: each expert's rows in pieces of at most
// `piece` rows; one piece keeps piece / 32 steps of every output block in
// one workgroup.  The chunks are dispatched longest first, so a piece no
// longer than one workgroup slot's average share of all the steps (S / 32
// steps times the 128 x 128 blocks per expert, over two workgroups on each
// of 256 CUs) bounds the tail; splitting less saves the partial buffers and
// their reduction.  At least 1024 rows, a multiple of 32.
int bwd_piece(const moe_layer_desc& d) {
  const long S = (long)d.max_tokens * d.top_k;
  const long tiles = (long)(d.hidden / 128) * (d.inter / 128);
  const long share = S * tiles / 512;
  const long piece = share < 1024 ? 1024 : (share + 31) / 32 * 32;
  return piece < (1 << 30) ? (int)piece : (1 << 30);
}

BwdScratch bwd_scratch(const moe_layer_desc& d) {
  const size_t S = (size_t)d.max_tokens * d.top_k, I = d.inter, H = d.hidden, E = d.num_experts;
  BwdScratch b{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  b.G = take(S * I * 4);
  b.U = take(S * I * 4);
  b.R = take(S * I * 4);
  b.Hb = take(S * I * 2);
  b.DGU = take(S * 2 * I * 2);
  b.DA = take(S * H * 4);
  // transposed weights, only where the input-gradient GEMM cannot read the
  // stored ones K-major (its 256-channel items need N % 256 == 0)
  b.WdT = I % 256 ? take(E * I * H * 2) : 0;         // W_down transposed: [E, I, H]
  b.WguT = H % 256 ? take(E * H * 2 * I * 2) : 0;    // W_gate | W_up transposed: [E, H, 2 I]
  b.WDY = take(S * H * 2);            // w dy_t per slot [S, H]
  b.tok = take(4 * (S + 64));         // token of each slot, 64 entries of slack
  b.piece = bwd_piece(d);
  const size_t extra = b.piece < (1 << 30) ? (S + b.piece - 1) / b.piece : 0;
  b.max_chunks = (int)(E + extra);
  b.chunks = take(4 * (4 + 4 * (size_t)b.max_chunks));
  b.nch = take(4 * E);
  b.pbase = take(4 * E);
  b.multi = take(4 * (E + 1));
  b.order = take(4 * (size_t)b.max_chunks);
  b.partial = take(extra * H * I * 4);
  b.total = off;
  return b;
}

int bwd_check_desc(const moe_layer_desc& d) {
  if (d.w_format != MOE_W_BF16 || d.a_format != MOE_A_BF16)
    return fail(MOE_EUNSUPPORTED, "the backward takes bf16 weights and activations");
  if (d.shared_experts) return fail(MOE_EUNSUPPORTED, "the backward has no shared expert");
  if (d.activation == MOE_ACT_REGLU) return fail(MOE_EUNSUPPORTED, "no backward for ReGLU");
  if (d.hidden % 128 || d.inter % 128)
    return fail(MOE_EUNSUPPORTED, "the backward needs hidden and inter multiples of 128");
  return MOE_OK;
}

}  // namespace

int moe_backward_scratch_size(const moe_layer_desc* desc, size_t* bytes) {
  if (!desc || !bytes) return fail(MOE_EINVAL, "null pointer");
  int rc = bwd_check_desc(*desc);
  if (rc) return rc;
  *bytes = bwd_scratch(*desc).total;
  return MOE_OK;
}

int moe_expert_backward(moe_ws* ws, const moe_weights* w, const void* x, const int32_t* topk_ids,
                        const float* topk_w, int T, const void* dy, void* dx, float* d_w_gate,
                        float* d_w_up, float* d_w_down, float* d_topk_w, void* scratch,
                        size_t scratch_bytes, void* stream) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  const moe_layer_desc& d = ws->d;
  int rc = bwd_check_desc(d);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T > d.max_tokens) return fail(MOE_ECAPACITY, "T=%d exceeds max_tokens=%d", T, d.max_tokens);
  if (T == 0) return MOE_OK;
  const bool relu2 = d.activation == MOE_ACT_RELU2;
  if (!w || !w->w_up || !w->w_down || (!relu2 && !w->w_gate))
    return fail(MOE_EINVAL, "null weight pointer");
  if (!x || !topk_ids || !topk_w || !dy || !dx || !d_w_up || !d_w_down || !d_topk_w ||
      (!relu2 && !d_w_gate) || !scratch)
    return fail(MOE_EINVAL, "null pointer");
  const BwdScratch b = bwd_scratch(d);
  if (scratch_bytes < b.total)
    return fail(MOE_ECAPACITY, "scratch holds %zu bytes, the backward needs %zu", scratch_bytes,
                b.total);
  hipStream_t st = (hipStream_t)stream;
  auto mark = [&](int stage, int which) -> hipError_t {
    hipEvent_t e = ws->stage_ev[stage][which];
    return e ? hipEventRecord(e, st) : hipSuccess;
  };
  char* sc = (char*)scratch;
  const int E = d.num_experts, k = d.top_k, H = d.hidden, I = d.inter, S = T * k;
  // dispatch of the given routing, block table for 128-row blocks (the
  // pipelined grouped GEMM's eight-wave configuration)
  DispatchArgs a = dispatch_args(ws, T);
  a.scores = nullptr;
  a.ids_in = topk_ids;
  a.shared = 0;
  a.force_cfg = 3;
  a.cm.on = 0;
  a.fq = QuantArgs{};
  HIP_TRY(launch_dispatch(a, st), "dispatch launch");
  const int32_t* gather = ws->at<int32_t>(ws->L.gather);
  const int32_t* inv = ws->at<int32_t>(ws->L.inv);
  const int32_t* counts = ws->at<int32_t>(ws->L.counts);
  const int32_t* indptr = ws->at<int32_t>(ws->L.indptr);
  const int32_t* tiles = ws->at<int32_t>(ws->L.tiles);
  const int32_t* meta = ws->at<int32_t>(ws->L.meta);
  float* G = (float*)(sc + b.G);
  float* U = (float*)(sc + b.U);
  float* R = (float*)(sc + b.R);
  uint16_t* Hb = (uint16_t*)(sc + b.Hb);
  uint16_t* DGU = (uint16_t*)(sc + b.DGU);
  float* DA = (float*)(sc + b.DA);
  uint16_t* WdT = (uint16_t*)(sc + b.WdT);
  uint16_t* WguT = (uint16_t*)(sc + b.WguT);
  uint16_t* WDY = (uint16_t*)(sc + b.WDY);
  int32_t* tok = (int32_t*)(sc + b.tok);
  // The input gradients contract the stored weights along their N axis:
  // the pipelined grouped GEMM reads them K-major as stored (w_kn) when the
  // output width is a multiple of 256; otherwise the active experts'
  // weights are first transposed to the forward's [N, K] layout.
  const bool kn_r = I % 256 == 0, kn_da = H % 256 == 0;
  HIP_TRY(mark(7, 0), "event record");
  BwdTranspose tr{};
  tr.counts = counts;
  tr.gather_div = 1;
  tr.in = (const uint16_t*)w->w_down;   // [H, I] per expert -> [I, H]
  tr.in_ld = I;
  tr.in_zstride = (long)H * I;
  tr.out = WdT;
  tr.out_ld = H;
  tr.out_zstride = (long)I * H;
  tr.R = H;
  tr.C = I;
  if (!kn_r) HIP_TRY(launch_bwd_transpose(tr, E, st), "weight transpose launch");
  tr.in_ld = H;                         // [I, H] per expert -> [H, 2 I] halves
  tr.in_zstride = (long)I * H;
  tr.out = WguT;
  tr.out_ld = 2 * I;
  tr.out_zstride = (long)H * 2 * I;
  tr.R = I;
  tr.C = H;
  // ReLU^2 has no gate: its dg is zero, and W_up fills both halves so that
  // the gate half holds finite values
  tr.in = (const uint16_t*)(relu2 ? w->w_up : w->w_gate);
  tr.out_col0 = 0;
  if (!kn_da) HIP_TRY(launch_bwd_transpose(tr, E, st), "weight transpose launch");
  tr.in = (const uint16_t*)w->w_up;
  tr.out_col0 = I;
  if (!kn_da) HIP_TRY(launch_bwd_transpose(tr, E, st), "weight transpose launch");
  // g and u recomputed by the pipelined bf16 grouped GEMM (128-row blocks,
  // plain op: fp32 rows)
  GemmArgs g = gemm_args(ws);
  g.E = E;
  g.N = I;
  g.K = H;
  g.a = (const uint8_t*)x;
  g.gather = gather;
  g.gather_div = k;
  g.max_groups = E < S ? E : S;
  g.max_rows = S;
  g.max_group_rows = T;
  g.cfg_self = 3;
  if (!relu2) {
    g.w0 = (const uint8_t*)w->w_gate;
    g.out = G;
    HIP_TRY(launch_gemm_pipe(F_BF16, false, 1, g, st), "gate recompute launch");
  }
  g.w0 = (const uint8_t*)w->w_up;
  g.out = U;
  HIP_TRY(launch_gemm_pipe(F_BF16, false, 1, g, st), "up recompute launch");
  HIP_TRY(mark(7, 1), "event record");
  // r = W_down^T dy: rows of dy gathered by token against W_down [H, I]
  // read K-major (or its transpose [I, H])
  HIP_TRY(mark(8, 0), "event record");
  g.a = (const uint8_t*)dy;
  g.w0 = kn_r ? (const uint8_t*)w->w_down : (const uint8_t*)WdT;
  g.w_kn = kn_r;
  g.w_k0 = H;
  g.out = R;
  HIP_TRY(launch_gemm_pipe(F_BF16, false, 1, g, st), "down input-gradient launch");
  HIP_TRY(mark(8, 1), "event record");
  BwdSlot sl{};
  sl.G = relu2 ? nullptr : G;
  sl.U = U;
  sl.R = R;
  sl.topk_w = topk_w;
  sl.gather = gather;
  sl.indptr = indptr;
  sl.E = E;
  sl.k = k;
  sl.I = I;
  sl.act = d.activation;
  sl.limit = act_limit(d);
  sl.Hb = Hb;
  sl.DGU = DGU;
  sl.dw = d_topk_w;
  sl.dy = (const uint16_t*)dy;
  sl.H = H;
  sl.WDY = WDY;
  sl.tok = tok;
  HIP_TRY(mark(9, 0), "event record");
  HIP_TRY(launch_bwd_slot(sl, S, st), "activation backward launch");
  HIP_TRY(mark(9, 1), "event record");
  // da = [dg | du] [W_gate^T ; W_up^T] (K = 2 I; for ReLU^2 dg is zero)
  HIP_TRY(mark(10, 0), "event record");
  g.a = (const uint8_t*)DGU;
  g.gather = nullptr;
  g.gather_div = 1;
  if (kn_da) {            // K rows 0 .. I - 1 from W_gate [I, H], the rest from W_up
    g.w0 = (const uint8_t*)(relu2 ? w->w_up : w->w_gate);
    g.w1 = (const uint8_t*)w->w_up;
  } else {
    g.w0 = (const uint8_t*)WguT;
    g.w1 = nullptr;
  }
  g.w_kn = kn_da;
  g.w_k0 = I;
  g.N = H;
  g.K = 2 * I;
  g.out = DA;
  HIP_TRY(launch_gemm_pipe(F_BF16, false, 1, g, st), "gate/up input-gradient launch");
  HIP_TRY(mark(10, 1), "event record");
  BwdDx bx{DA, inv, T, k, H, (uint16_t*)dx};
  HIP_TRY(mark(11, 0), "event record");
  HIP_TRY(launch_bwd_dx(bx, st), "input-gradient combine launch");
  HIP_TRY(mark(11, 1), "event record");
  // weight gradients over each expert's slots, from the slot rows as stored
  HIP_TRY(mark(12, 0), "event record");
  int32_t* chunks = (int32_t*)(sc + b.chunks);
  int32_t* nch = (int32_t*)(sc + b.nch);
  int32_t* pbase = (int32_t*)(sc + b.pbase);
  int32_t* multi = (int32_t*)(sc + b.multi);
  int32_t* order = (int32_t*)(sc + b.order);
  HIP_TRY(launch_bwd_chunks(indptr, E, b.piece, chunks, nch, pbase, multi, order, st),
          "chunk table launch");
  BwdWgrad wg{};
  wg.chunks = chunks;
  wg.nch = nch;
  wg.pbase = pbase;
  wg.multi = multi;
  wg.order = order;
  wg.partial = (float*)(sc + b.partial);
  wg.a = WDY;                           // dW_down[e] = sum (w dy_t) h^T
  wg.lda = H;
  wg.b = Hb;
  wg.ldb = I;
  wg.b_tok = nullptr;
  wg.M = H;
  wg.N = I;
  wg.out = d_w_down;
  HIP_TRY(launch_bwd_wgrad(wg, E, b.max_chunks, st), "down weight-gradient launch");
  HIP_TRY(mark(12, 1), "event record");
  HIP_TRY(mark(13, 0), "event record");
  wg.b = (const uint16_t*)x;            // dW_gate[e] = sum dg x_t^T, dW_up[e] = sum du x_t^T
  wg.ldb = H;
  wg.b_tok = tok;
  wg.a = DGU;
  wg.lda = 2 * I;
  wg.M = I;
  wg.N = H;
  if (!relu2) {
    wg.out = d_w_gate;
      HIP_TRY(launch_bwd_wgrad(wg, E, b.max_chunks, st), "gate weight-gradient launch");
  }
  wg.a = DGU + I;
  wg.out = d_w_up;
  HIP_TRY(launch_bwd_wgrad(wg, E, b.max_chunks, st), "up weight-gradient launch");
  HIP_TRY(mark(13, 1), "event record");
  return MOE_OK;
}

int moe_router_backward(const float* scores, const int32_t* topk_ids, const float* topk_w,
                        const float* d_topk_w, int T, int E, int k, int score_fn, float* d_scores,
                        void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (E < 1) return fail(MOE_EINVAL, "E must be >= 1");
  const int kmax = E < 16 ? E : 16;
  if (k < 1 || k > kmax) return fail(MOE_EINVAL, "k must be in [1, %d]", kmax);
  if (score_fn < 0 || score_fn > 2) return fail(MOE_EINVAL, "unknown score_fn");
  if (T == 0) return MOE_OK;
  if (!scores || !topk_ids || !topk_w || !d_topk_w || !d_scores) return fail(MOE_EINVAL, "null pointer");
  RouterBwd r{scores, topk_ids, topk_w, d_topk_w, T, E, k, score_fn, d_scores};
  HIP_TRY(launch_router_bwd(r, (hipStream_t)stream), "router backward launch");
  return MOE_OK;
}

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or format";
    case MOE_ECAPACITY: return "exceeds workspace capacity";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_workspace_size(const moe_layer_desc* desc, size_t* bytes) {
  int rc = validate_desc(desc);
  if (rc) return rc;
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = make_layout(*desc).total;
  return MOE_OK;
}

int moe_workspace_create(const moe_layer_desc* desc, void* dev_buf, size_t bytes, moe_ws** out) {
  int rc = validate_desc(desc);
  if (rc) return rc;
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!dev_buf) return fail(MOE_EINVAL, "dev_buf is NULL");
  if ((uintptr_t)dev_buf & 255) return fail(MOE_EINVAL, "dev_buf must be 256-byte aligned");
  Layout L = make_layout(*desc);
  if (bytes < L.total)
    return fail(MOE_ECAPACITY, "workspace needs %zu bytes, got %zu", L.total, bytes);
  moe_ws* ws = new moe_ws();
  ws->d = *desc;
  ws->L = L;
  ws->base = (char*)dev_buf;
  ws->fmt = fmt_of(*desc);
  if (hipGetDevice(&ws->device) != hipSuccess) ws->device = 0;
  // the decode layer's barrier words and counters start cleared (they are
  // kept cleared by the kernel from then on)
  hipError_t e = hipMemset(ws->at<char>(L.dstate), 0, L.dstate_bytes);
  if (e != hipSuccess) {
    delete ws;
    return hip_fail(e, "clear the decode-layer state");
  }
  e = hipMemcpy(ws->at<char>(L.cmth), kCostModelTheta, sizeof kCostModelTheta, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    delete ws;
    return hip_fail(e, "copy the cost model's parameters");
  }
  *out = ws;
  return MOE_OK;
}

int moe_workspace_destroy(moe_ws* ws) {
  if (!ws) return MOE_OK;
  for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second.exec);
  delete ws;
  return MOE_OK;
}

int moe_route_topk(const float* scores, int T, int E, int k, int score_fn, int renorm, int32_t* ids,
                   float* w, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (E < 1 || E > 256) return fail(MOE_EINVAL, "E must be in [1, 256]");
  int kmax = E < 16 ? E : 16;
  if (k < 1 || k > kmax) return fail(MOE_EINVAL, "k must be in [1, %d]", kmax);
  if (score_fn < 0 || score_fn > 2) return fail(MOE_EINVAL, "unknown score_fn");
  if (renorm != 1) return fail(MOE_EUNSUPPORTED, "only renorm = 1 is supported");
  if (T == 0) return MOE_OK;
  if (!scores || !ids || !w) return fail(MOE_EINVAL, "null pointer");
  HIP_TRY(launch_route(scores, T, E, k, score_fn, ids, w, QuantArgs{}, (hipStream_t)stream),
          "route launch");
  return MOE_OK;
}

int moe_dispatch(moe_ws* ws, const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                 int32_t* m_indptr, int32_t* gather, int32_t* inv, void* stream) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (E != ws->d.num_experts || k != ws->d.top_k)
    return fail(MOE_EINVAL, "E/k must match the workspace (%d/%d)", ws->d.num_experts, ws->d.top_k);
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T > ws->d.max_tokens) return fail(MOE_ECAPACITY, "T=%d exceeds max_tokens", T);
  if (!counts || !m_indptr || (T > 0 && (!topk_ids || !gather || !inv)))
    return fail(MOE_EINVAL, "null pointer");
  DispatchArgs a = dispatch_args(ws, T);
  a.shared = 0;
  a.ids_in = topk_ids;
  a.counts = counts;
  a.indptr = m_indptr;
  a.gather = gather;
  a.inv = inv;
  HIP_TRY(launch_dispatch(a, (hipStream_t)stream), "dispatch launch");
  return MOE_OK;
}

int moe_grouped_gemm(moe_ws* ws, int op, const void* a, const void* a_scale,
                     const int32_t* a_gather, int gather_div, const int32_t* m_indptr, int E, int N,
                     int K, const void* b0, const void* b0_scale, const void* b1,
                     const void* b1_scale, void* out, void* out_scale, void* stream) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (op != MOE_OP_PLAIN && op != MOE_OP_GATEUP_ACT) return fail(MOE_EINVAL, "unknown op");
  if (E < 1 || E > ws->d.num_experts + ws->d.shared_experts)
    return fail(MOE_EINVAL, "E must be in [1, %d]", ws->d.num_experts + ws->d.shared_experts);
  if (N <= 0 || K <= 0 || N % 128 || K % 128)
    return fail(MOE_EUNSUPPORTED, "N and K must be positive multiples of 128");
  if (N > 16384 || K > 16384) return fail(MOE_EUNSUPPORTED, "N and K are limited to 16384");
  const bool gateup = op == MOE_OP_GATEUP_ACT;
  const bool quant = ws->fmt != F_BF16;
  // ReLU^2 has no gate projection: B1 (up) serves as both operands
  if (gateup && ws->d.activation == MOE_ACT_RELU2) {
    b0 = b1;
    b0_scale = b1_scale;
  }
  if (!a || !m_indptr || !b0 || !out || (gateup && !b1)) return fail(MOE_EINVAL, "null pointer");
  if (quant && (!a_scale || !b0_scale || (gateup && (!b1_scale || !out_scale))))
    return fail(MOE_EINVAL, "null scale pointer");
  if (a_gather && gather_div < 1) return fail(MOE_EINVAL, "gather_div must be >= 1");
  const long cap = ws->L.S_tot;
  if (gateup && (long)N > ws->d.inter && quant)
    return fail(MOE_ECAPACITY, "N exceeds the workspace's intermediate staging width");
  hipStream_t st = (hipStream_t)stream;
  // the group table and the tile configuration come from m_indptr on the
  // device, as in the layer (largest group in place of the token count)
  DispatchArgs da = dispatch_args(ws, -1);
  da.E = E;
  da.shared = 0;
  da.I = N;
  HIP_TRY(launch_indptr_table(m_indptr, (int)cap, da, st), "group table launch");
  GemmArgs g = gemm_args(ws);
  g.E = E;   // every group is a routed group here
  g.w0 = (const uint8_t*)b0;
  g.w1 = (const uint8_t*)b1;
  g.w0s = b0_scale;
  g.w1s = b1_scale;
  g.N = N;
  g.K = K;
  g.a = (const uint8_t*)a;
  g.a_scale = a_scale;
  g.gather = a_gather;
  g.gather_div = a_gather ? gather_div : 1;
  g.max_groups = E;
  g.max_rows = (int)cap;
  g.max_group_rows = (int)cap;
  g.cfg_self = -1;
  // the host does not know the histogram: every kernel family the device
  // may choose is launched, and those it did not choose return at once
  Candidates cand = from_flags(true, num_cfgs(ws->fmt) > 1, num_cfgs(ws->fmt) > 3 && cap >= CFG3_MIN_ROWS);
  if (ws->force_cfg >= 0) cand = forced(ws->force_cfg);
  if (gateup && quant) {
    // fp32 staging, requantised by a separate pass, except where the tiled
    // 1x128 and MX epilogues requantise in place
    const bool fused_requant = ws->fmt == F_FP8_BLK || ws->fmt == F_MX;
    g.out = ws->at<void>(ws->L.h);
    HIP_TRY(run_gemm_c(ws, true, g, fused_requant ? out : nullptr, fused_requant ? out_scale : nullptr,
                       cand, st),
            "grouped GEMM launch");
    if (!fused_requant || cand.stream) {
      // the grid covers the capacity; rows at or beyond m_indptr[E] (read
      // on the device) return at once, so only the R rows of `out` are
      // written
      QuantArgs q{ws->at<void>(ws->L.h), 0, (int)cap, N, m_indptr + E, (uint8_t*)out, out_scale,
                  ws->d.a_format};
      if (fused_requant) {   // only the streaming configuration left fp32 h behind
        q.meta = ws->at<int32_t>(ws->L.meta);
        q.only_cfg = 0;
      }
      HIP_TRY(launch_quant(q, st), "intermediate quantisation launch");
    }
  } else {
    g.out = out;
    HIP_TRY(run_gemm_c(ws, gateup, g, nullptr, nullptr, cand, st), "grouped GEMM launch");
  }
  return MOE_OK;
}

int moe_quantize_act(moe_ws* ws, const uint16_t* x, int T, uint8_t* q, void* scale, void* stream) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (ws->fmt == F_BF16) return fail(MOE_EUNSUPPORTED, "bf16 activations are not quantised");
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return MOE_OK;
  if (!x || !q || !scale) return fail(MOE_EINVAL, "null pointer");
  QuantArgs qa{x, 1, T, ws->d.hidden, nullptr, q, scale, ws->d.a_format};
  HIP_TRY(launch_quant_rows(qa, (hipStream_t)stream), "quantisation launch");
  return MOE_OK;
}

int moe_combine(moe_ws* ws, const float* out_slot, const float* topk_w, const int32_t* inv, int T,
                uint16_t* y, void* stream) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T > ws->d.max_tokens) return fail(MOE_ECAPACITY, "T=%d exceeds max_tokens", T);
  if (T == 0) return MOE_OK;
  if (!out_slot || !topk_w || !inv || !y) return fail(MOE_EINVAL, "null pointer");
  CombineArgs c{out_slot, topk_w, inv, T, ws->d.top_k, ws->d.hidden, ws->d.shared_experts, y, 0};
  HIP_TRY(launch_combine(c, (hipStream_t)stream), "combine launch");
  return MOE_OK;
}

int moe_layer_forward(moe_ws* ws, const moe_weights* w, const uint16_t* x, const float* scores,
                      int T, uint16_t* y, void* stream) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T > ws->d.max_tokens) return fail(MOE_ECAPACITY, "T=%d exceeds max_tokens=%d", T, ws->d.max_tokens);
  if (T == 0) return MOE_OK;
  if (!x || !scores || !y) return fail(MOE_EINVAL, "null pointer");
  int rc = check_weights(ws, w);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  // inside a caller's stream capture the launches become part of the
  // caller's graph; otherwise decode-sized calls replay a graph of their own
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (st != nullptr) HIP_TRY(hipStreamIsCapturing(st, &cap), "capture query");
  const bool use_graph = ws->graphs && st != nullptr && T <= 128 && !ws->any_stage_events() &&
                         cap == hipStreamCaptureStatusNone;
  if (!use_graph) return enqueue_layer(ws, w, x, scores, T, y, st);
  const GraphKey key{T, st};
  GraphPtrs ptrs{x, scores, y, {w->w_gate, w->w_up, w->w_down, w->s_gate, w->s_up, w->s_down,
                                w->sh_gate, w->sh_up, w->sh_down, w->ss_gate, w->ss_up, w->ss_down}};
  auto it = ws->execs.find(key);
  if (it == ws->execs.end() || !(it->second.ptrs == ptrs)) {
    hipGraph_t graph;
    HIP_TRY(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal), "begin capture");
    rc = enqueue_layer(ws, w, x, scores, T, y, st);
    hipError_t e = hipStreamEndCapture(st, &graph);
    if (rc) {
      if (e == hipSuccess) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return hip_fail(e, "end capture");
    if (it != ws->execs.end()) {
      // same launch sequence, other buffers: update the instance in place
      hipGraphExecUpdateResult res = hipGraphExecUpdateError;
      hipGraphNode_t err_node = nullptr;
      e = hipGraphExecUpdate(it->second.exec, graph, &err_node, &res);
      if (e == hipSuccess && res == hipGraphExecUpdateSuccess) {
        (void)hipGraphDestroy(graph);
        it->second.ptrs = ptrs;
        HIP_TRY(hipGraphLaunch(it->second.exec, st), "graph launch");
        return MOE_OK;
      }
      (void)hipGetLastError();
      (void)hipGraphExecDestroy(it->second.exec);
      ws->execs.erase(it);
    }
    hipGraphExec_t exec;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "graph instantiate");
    it = ws->execs.emplace(key, GraphEntry{exec, ptrs}).first;
  }
  HIP_TRY(hipGraphLaunch(it->second.exec, st), "graph launch");
  return MOE_OK;
}

int moe_workspace_routing(const moe_ws* ws, const int32_t** ids, const float** w,
                          const int32_t** counts, const int32_t** indptr, const int32_t** gather,
                          const int32_t** inv) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (ids) *ids = ws->at<int32_t>(ws->L.ids);
  if (w) *w = ws->at<float>(ws->L.w);
  if (counts) *counts = ws->at<int32_t>(ws->L.counts);
  if (indptr) *indptr = ws->at<int32_t>(ws->L.indptr);
  if (gather) *gather = ws->at<int32_t>(ws->L.gather);
  if (inv) *inv = ws->at<int32_t>(ws->L.inv);
  return MOE_OK;
}

int moe_workspace_force_config(moe_ws* ws, int cfg) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (cfg < -1 || cfg >= num_cfgs(ws->fmt))
    return fail(MOE_EINVAL, "cfg must be in [-1, %d)", num_cfgs(ws->fmt));
  ws->force_cfg = cfg;
  for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second.exec);
  ws->execs.clear();
  return MOE_OK;
}

int moe_workspace_last_config(const moe_ws* ws, int* cfg, void* stream) {
  if (!ws || !cfg) return fail(MOE_EINVAL, "null pointer");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "stream synchronise");
  HIP_TRY(hipMemcpy(cfg, ws->at<int32_t>(ws->L.meta) + META_CFG, 4, hipMemcpyDeviceToHost),
          "read configuration");
  return MOE_OK;
}

int moe_workspace_tiles(const moe_ws* ws, const int32_t** tiles, const int32_t** meta) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (tiles) *tiles = ws->at<int32_t>(ws->L.tiles);
  if (meta) *meta = ws->at<int32_t>(ws->L.meta);
  return MOE_OK;
}

int moe_workspace_check(const moe_ws* ws, int* device_status, void* stream) {
  if (!ws || !device_status) return fail(MOE_EINVAL, "null pointer");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream), "stream synchronise");
  int32_t err = 0;
  HIP_TRY(hipMemcpy(&err, ws->at<int32_t>(ws->L.meta) + META_ERROR, 4, hipMemcpyDeviceToHost),
          "read device status");
  *device_status = err == 0 ? MOE_OK : (err == 2 ? MOE_EHIP : MOE_EINVAL);
  if (err == 2)
    fail(MOE_EHIP, "the single-launch decode layer could not make its whole grid resident and "
                   "stopped at its barrier; the output is incomplete and the workspace must be "
                   "created again");
  else if (err)
    fail(MOE_EINVAL, "the device rejected the last m_indptr (not non-decreasing from 0, or more "
                     "rows than the workspace holds); no rows were computed");
  return MOE_OK;
}

int moe_workspace_graph_count(const moe_ws* ws, int* host_n) {
  if (!ws || !host_n) return fail(MOE_EINVAL, "null pointer");
  *host_n = (int)ws->execs.size();
  return MOE_OK;
}

int moe_config_rows(int cfg) { return (cfg >= 0 && cfg < kNumCfgs) ? cfg_rows(cfg) : -1; }

int moe_workspace_set_graphs(moe_ws* ws, int enable) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  ws->graphs = enable ? 1 : 0;
  if (!enable) {
    for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second.exec);
    ws->execs.clear();
  }
  return MOE_OK;
}

int moe_workspace_set_fused_decode(moe_ws* ws, int enable) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  ws->fused_decode = enable ? 1 : 0;
  for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second.exec);
  ws->execs.clear();
  return MOE_OK;
}

int moe_workspace_set_config_model(moe_ws* ws, int enable) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  ws->config_model = enable ? 1 : 0;
  for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second.exec);
  ws->execs.clear();
  return MOE_OK;
}

int moe_workspace_candidates(const moe_ws* ws, int T, int* host_mask) {
  if (!ws || !host_mask) return fail(MOE_EINVAL, "null pointer");
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  *host_mask = candidates(ws, (long)T * ws->d.top_k + (ws->d.shared_experts ? T : 0), T).mask;
  return MOE_OK;
}

int moe_config_model_params(double* host_theta20) {
  if (!host_theta20) return fail(MOE_EINVAL, "null pointer");
  memcpy(host_theta20, kCostModelTheta, sizeof kCostModelTheta);
  return MOE_OK;
}

int moe_workspace_set_stage_events(moe_ws* ws, int stage, void* ev_begin, void* ev_end) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (stage < 0 || stage > 13) return fail(MOE_EINVAL, "stage must be in [0, 13]");
  ws->stage_ev[stage][0] = (hipEvent_t)ev_begin;
  ws->stage_ev[stage][1] = (hipEvent_t)ev_end;
  return MOE_OK;
}

}  // extern "C"
