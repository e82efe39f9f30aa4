// Host side of the C ABI declared in include/moe.h: validation, workspace
// layout, launch sequencing and hipGraph capture of decode-sized calls.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <tuple>

#include "../../include/moe.h"
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
int num_cfgs(int fmt) { return fmt == F_BF16 ? 3 : kNumCfgs; }

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
  size_t xq, xs, h, hq, hs, out_slot, total;
  long S, S_tot, G, max_tiles, nchunks;
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
  L.total = off;
  return L;
}

struct GraphKey {
  int T;
  const void *x, *scores, *y, *st;
  const void* wp[12];
  bool operator<(const GraphKey& o) const {
    return std::tie(T, x, scores, y, st) < std::tie(o.T, o.x, o.scores, o.y, o.st) ||
           (std::tie(T, x, scores, y, st) == std::tie(o.T, o.x, o.scores, o.y, o.st) &&
            memcmp(wp, o.wp, sizeof wp) < 0);
  }
};

}  // namespace

struct moe_ws {
  moe_layer_desc d;
  Layout L;
  char* base;
  int fmt;
  int force_cfg = -1;
  int graphs = 1;
  int device = 0;
  std::map<GraphKey, hipGraphExec_t> execs;
  hipEvent_t stage_ev[6][2] = {};
  bool any_stage_events() const {
    for (auto& p : stage_ev)
      if (p[0] || p[1]) return true;
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
struct Candidates {
  bool stream, small, big;   // streaming kernel; tiled configurations 1-2; configuration 3
};
Candidates candidates(const moe_ws* ws, long rows_tot, int T) {
  if (ws->force_cfg >= 0)
    return {ws->force_cfg == 0, ws->force_cfg == 1 || ws->force_cfg == 2, ws->force_cfg == 3};
  // the device rule streams every batch of at most DECODE_STREAM_TOKENS tokens
  if (T <= DECODE_STREAM_TOKENS || num_cfgs(ws->fmt) <= 1) return {true, false, false};
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
  return {2 * lo * cb < cus, tiled && !big_certain, big};
}

// Run a projection with the kernel families the configuration can land on;
// a launch whose family the device did not choose returns at once.
// `tiled_out` and `tiled_scale` redirect the fused gate/up output of the
// tiled kernels, which requantise the intermediate in their epilogue for the
// 1x128 and MX formats.
hipError_t run_gemm(const moe_ws* ws, bool gateup, GemmArgs g, void* tiled_out, void* tiled_scale,
                    long rows_tot, int T, hipStream_t st) {
  const Candidates cand = candidates(ws, rows_tot, T);
  if (cand.stream) {
    g.cfg_self = 0;
    hipError_t e = launch_gemm_stream(ws->fmt, gateup, g, st);
    if (e != hipSuccess) return e;
  }
  if (!cand.small && !cand.big) return hipSuccess;
  if (tiled_out) {
    g.out = tiled_out;
    g.out_scale = tiled_scale;
  }
  if (ws->fmt != F_BF16) {
    g.cfg_self = ws->force_cfg > 0 ? ws->force_cfg : -1;   // any tiled configuration
    if (cand.small) {
      hipError_t e = launch_gemm_pipe(ws->fmt, gateup, 0, g, st);
      if (e != hipSuccess) return e;
    }
    if (cand.big) return launch_gemm_pipe(ws->fmt, gateup, 1, g, st);
    return hipSuccess;
  }
  for (int c = 1; c < num_cfgs(ws->fmt); ++c) {
    g.cfg_self = c;
    hipError_t e = launch_gemm_tiled(ws->fmt, gateup, c, g, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int enqueue_layer(moe_ws* ws, const moe_weights* w, const uint16_t* x, const float* scores, int T,
                  uint16_t* y, hipStream_t st) {
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

}  // namespace

extern "C" {

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
  *out = ws;
  return MOE_OK;
}

int moe_workspace_destroy(moe_ws* ws) {
  if (!ws) return MOE_OK;
  for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second);
  delete ws;
  return MOE_OK;
}

int moe_route_topk(const float* scores, int T, int E, int k, int score_fn, int32_t* ids, float* w,
                   void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (E < 1 || E > 256) return fail(MOE_EINVAL, "E must be in [1, 256]");
  int kmax = E < 16 ? E : 16;
  if (k < 1 || k > kmax) return fail(MOE_EINVAL, "k must be in [1, %d]", kmax);
  if (score_fn < 0 || score_fn > 2) return fail(MOE_EINVAL, "unknown score_fn");
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
  DispatchArgs da = dispatch_args(ws, 0);
  da.E = E;
  da.shared = 0;
  da.force_cfg = 0;
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
  if (gateup && quant) {
    g.out = ws->at<void>(ws->L.h);
    HIP_TRY(launch_gemm_stream(ws->fmt, true, g, st), "grouped GEMM launch");
    // the grid covers the capacity; rows at or beyond m_indptr[E] (read on
    // the device) return at once, so only the R rows of `out` are written
    QuantArgs q{ws->at<void>(ws->L.h), 0, (int)cap, N, m_indptr + E, (uint8_t*)out, out_scale,
                ws->d.a_format};
    HIP_TRY(launch_quant(q, st), "intermediate quantisation launch");
  } else {
    g.out = out;
    HIP_TRY(launch_gemm_stream(ws->fmt, gateup, g, st), "grouped GEMM launch");
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
  GraphKey key{};
  key.T = T;
  key.x = x;
  key.scores = scores;
  key.y = y;
  key.st = st;
  const void* wp[12] = {w->w_gate, w->w_up, w->w_down, w->s_gate, w->s_up, w->s_down,
                        w->sh_gate, w->sh_up, w->sh_down, w->ss_gate, w->ss_up, w->ss_down};
  memcpy(key.wp, wp, sizeof wp);
  auto it = ws->execs.find(key);
  if (it == ws->execs.end()) {
    hipGraph_t graph;
    HIP_TRY(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal), "begin capture");
    rc = enqueue_layer(ws, w, x, scores, T, y, st);
    hipError_t e = hipStreamEndCapture(st, &graph);
    if (rc) {
      if (e == hipSuccess) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return hip_fail(e, "end capture");
    hipGraphExec_t exec;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "graph instantiate");
    it = ws->execs.emplace(key, exec).first;
  }
  HIP_TRY(hipGraphLaunch(it->second, st), "graph launch");
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
  for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second);
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

int moe_config_rows(int cfg) { return (cfg >= 0 && cfg < kNumCfgs) ? cfg_rows(cfg) : -1; }

int moe_workspace_set_graphs(moe_ws* ws, int enable) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  ws->graphs = enable ? 1 : 0;
  if (!enable) {
    for (auto& kv : ws->execs) (void)hipGraphExecDestroy(kv.second);
    ws->execs.clear();
  }
  return MOE_OK;
}

int moe_workspace_set_stage_events(moe_ws* ws, int stage, void* ev_begin, void* ev_end) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (stage < 0 || stage > 5) return fail(MOE_EINVAL, "stage must be in [0, 5]");
  ws->stage_ev[stage][0] = (hipEvent_t)ev_begin;
  ws->stage_ev[stage][1] = (hipEvent_t)ev_end;
  return MOE_OK;
}

}  // extern "C"
