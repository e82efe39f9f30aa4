// Internal declarations shared by the kernels and the host library.
#pragma once
#include "common.h"

#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_SCORE_PROBS 2

// meta[] words written by the dispatch step
#define META_NACTIVE 0   // active row groups (experts with rows, plus the shared group)
#define META_NTILES 1    // entries of the block table
#define META_CFG 2       // chosen configuration
#define META_MAXCNT 3    // largest group
#define META_ROWS 4      // total rows (slots), shared group included
#define META_BM 5        // row-block height of the table
#define META_ERROR 6     // nonzero: the device rejected the group offsets
#define META_WORDS 16

// Slots up to which one 1024-thread block does the whole dispatch (it also
// routes, when the batch routes in one or two passes); larger batches take
// the two-launch chunked path.
#define SMALL_DISPATCH_SLOTS 2048
// Slots up to which one wave does the whole dispatch (at most 64 groups)
#define TINY_DISPATCH_SLOTS 1024
// Router scores (floats) the one-wave path stages in LDS before routing
#define TINY_SCORE_LDS 4096
// Expert counts up to which one thread routes a token (above: a 16-lane row)
#define SMALL_E_THREAD_ROUTE 32

// Tile configurations: 0 streams weights (decode-sized groups); the others
// are LDS-tiled with the given row-block height.
#define NUM_CFGS_MAX 4

__host__ __device__ inline int cfg_rows(int cfg) {
  switch (cfg) {
    case 0: return 64;
    case 1: return 32;
    case 2: return 64;
    case 3: return 128;
    default: return 64;
  }
}

struct QuantArgs {
  const void* in;         // rows [R, n], bf16 (in_bf16) or fp32
  int in_bf16;
  int R, n;
  const int32_t* nrows;   // optional device row count (NULL: R)
  uint8_t* q;             // [R, n] e4m3
  void* scale;            // fp32 [R] / fp32 [R, n/128] / uint8 [R, n/32]
  int a_format;
  const int32_t* meta;    // optional: run only if meta[META_CFG] == only_cfg
  int only_cfg;
};

// Histogram statistics the configuration choice reads: largest group,
// active groups, rows, and the row blocks of 16, 32, 64 and 128 rows the
// groups need (sums of ceil(rows / b)).
struct HistStats {
  int mx, active, rows, s16, s32, s64, s128;
};

// The fitted tile-configuration cost model (RaMP abstract: a four-parameter
// wave cost model over the runtime expert histogram, depending only on the
// kernels' grid geometry).  Predicted time of configuration cfg for a layer
// of shape (H, I) in weight format fmt (0 bf16, 1/2 fp8, 3 MXFP4) and T
// tokens: th[row][0] + th[row][1] * (weight bytes streamed / HBM peak)
//        + th[row][2] * (padded MFMA work / MFMA peak) + th[row][3] * waves,
// row = cfg (row 4: streaming above DECODE_STREAM_TOKENS tokens).  The
// features mirror grouped_gemm_amd/costmodel.py, which fits th.
struct CostModel {
  const double* th;       // th[5][4], row-major (device memory in DispatchArgs)
  int on;                 // 0: the histogram rule instead
  int mask;               // configurations the device may choose (bit c)
};

__host__ __device__ inline double cost_model_time(const double* th, const HistStats& h, int cfg,
                                                  int fmt, int H, int I, int T, int cus) {
  // no fused multiply-adds: host and device then predict the same times
#pragma clang fp contract(off)
  const double wbytes = fmt == 0 ? 2.0 : (fmt == 3 ? 0.5 : 1.0);
  const double peak = fmt == 0 ? 2.5e9 : 5.0e9;          // MFMA flop per us
  const double hbm = 8.0e6;                              // HBM bytes per us
  const double mlp = 3.0 * H * I * wbytes, flop_row = 6.0 * H * I;
  double wb, padded, waves;
  int row = cfg;
  if (cfg == 0) {
    const bool dec = T >= 0 ? T <= 16 : h.mx <= 16;
    row = dec ? 0 : 4;
    wb = (dec ? h.s16 : h.s64) * mlp;
    padded = 16.0 * h.s16;
    waves = (double)h.active * (I / 16 + H / 16) / (cus * 8.0);
  } else {
    const int bm = cfg == 1 ? 32 : (cfg == 2 ? 64 : 128);
    const int tiles = cfg == 1 ? h.s32 : (cfg == 2 ? h.s64 : h.s128);
    int cb_gu, cb_dn;
    if (cfg == 3) {
      cb_gu = I / 128;
      cb_dn = H % 256 == 0 ? H / 256 : H / 128;
    } else {
      cb_gu = I / (fmt == 1 ? 64 : 128);
      cb_dn = H / 128;
    }
    wb = h.active * mlp;
    padded = (double)tiles * bm;
    waves = (double)(((long)tiles * cb_gu + cus - 1) / cus + ((long)tiles * cb_dn + cus - 1) / cus);
  }
  const double* t = th + 4 * row;
  return t[0] + t[1] * (wb / hbm) + t[2] * (padded * flop_row / peak) + t[3] * waves;
}

struct DispatchArgs {
  const float* scores;    // [T,E] or NULL when ids are given
  const int32_t* ids_in;  // [T,k] when scores == NULL
  int32_t* ids;           // [T,k] routing output (when scores != NULL)
  float* w;               // [T,k]
  int T, E, k, score_fn, shared;
  int32_t* counts;        // [G]
  int32_t* indptr;        // [G+1]
  int32_t* gather;        // [S + shared*T]
  int32_t* inv;           // [S]
  int32_t* active;        // [G]
  int32_t* tiles;         // [2 * max tiles]
  int32_t* meta;          // [META_WORDS]
  int32_t* chunk;         // [chunks * E], chunks = ceil(T / floor(1024 / k))
  int force_cfg;          // -1: choose from the histogram
  int H, I, wbits, xbits; // for the cost model
  int num_cfgs;           // configurations the library has kernels for
  int cus;                // compute units of the device (configuration rule)
  QuantArgs fq;           // activation rows the routing launch quantises on
                          // its spare waves (fq.R = 0: none)
  int fmt;                // weight format (Fmt), for the cost model
  CostModel cm;           // fitted configuration cost model (cm.on = 0: the rule)
};

// Grouped GEMM over expert-major row groups.
// Batches of at most this many tokens take the streaming configuration (every
// group then holds at most this many rows: one 16-row token tile).
constexpr int DECODE_STREAM_TOKENS = 16;

struct GemmArgs {
  const uint8_t* w0;      // routed weights [E, N, K] (gate or down)
  const uint8_t* w1;      // routed up weights (gate/up op)
  const void* w0s;        // weight scales per format
  const void* w1s;
  const uint8_t* sh_w0;   // shared expert (group E), or NULL
  const uint8_t* sh_w1;
  const void* sh_w0s;
  const void* sh_w1s;
  int E;                  // routed groups; group E is the shared expert
  int N, K;
  const uint8_t* a;       // activation rows (bf16 or e4m3 codes)
  const void* a_scale;    // per format
  const int32_t* gather;  // NULL: row = slot; else row = gather[slot] / gather_div
  int gather_div;
  const int32_t* counts;
  const int32_t* indptr;
  const int32_t* active;
  const int32_t* tiles;
  const int32_t* meta;
  int cfg_self;           // this launch runs only if meta[META_CFG] == cfg_self (or -1)
  void* out;              // gate/up: bf16 h, fp32 h staging or e4m3 h; down: fp32 [rows, N]
  void* out_scale;        // gate/up with in-kernel requantisation: h scales
  int max_groups;         // grid bound on active groups
  int max_rows;           // grid bound on rows (all groups)
  int max_group_rows;     // bound on the rows of any one group
  // down projection of the layer: when row_w is set, row `slot` is scaled by
  // its routing weight row_w[row_w_idx[slot]] (1 for slot >= row_w_n, the
  // shared expert) and stored as bf16; otherwise stored as fp32
  const float* row_w;
  const int32_t* row_w_idx;
  int row_w_n;
  // gate/up op: expert activation (ACT_*) and its clamp
  int act;
  float act_limit;
  int grid_cap;           // streaming kernel: most workgroups (0: one per work item)
  // bf16 plain op only: w_kn = 1 takes the weights K-major as stored for
  // the forward's other side: w0 [E, w_k0, N] supplies K rows 0 .. w_k0 - 1
  // and w1 [E, K - w_k0, N] the rest (w_k0 == K: w0 alone)
  int w_kn, w_k0;
};

// Store four consecutive down-projection outputs of one row.
DEVI void store_down(const GemmArgs& p, int slot, int n0, f32x4 v) {
  if (p.row_w) {
    const float w = slot < p.row_w_n ? p.row_w[p.row_w_idx[slot]] : 1.0f;
    v = v * w;
    uint32_t lo = pack_bf16x2(v[0], v[1]);
    uint32_t hi = pack_bf16x2(v[2], v[3]);
    *(uint2*)((uint16_t*)p.out + (size_t)slot * p.N + n0) = make_uint2(lo, hi);
  } else {
    *(f32x4*)((float*)p.out + (size_t)slot * p.N + n0) = v;
  }
}


struct CombineArgs {
  const void* out_slot;   // [S + shared*T, H]: fp32 unweighted, or bf16 pre-weighted
  const float* w;         // [T,k]
  const int32_t* inv;     // [T*k]
  int T, k, H, shared;
  uint16_t* y;            // [T,H] bf16
  int weighted_bf16;      // out_slot rows are bf16 and already carry w[t,j]
};

// The single-launch decode layer (batches of at most DECODE_STREAM_TOKENS
// tokens).  ids .. meta receive the routing results for the caller (written
// by workgroup 0); h, out_slot, amax and cnt are its scratch; bar holds the
// grid barrier's arrival count and generation.
struct DecodeArgs {
  const float* scores;    // [T, E]
  const uint16_t* x;      // [T, H] bf16
  uint16_t* y;            // [T, H] bf16
  int T, E, k, score_fn, shared, H, I;
  const uint8_t *wg, *wu, *wd;      // routed weights [E, N, K] (format codes)
  const void *sg, *su, *sd;         // their scales
  const uint8_t *shg, *shu, *shd;   // shared expert [1, N, K] or NULL
  const void *ssg, *ssu, *ssd;
  int act;
  float act_limit;
  int32_t* ids;           // [T, k]
  float* w;               // [T, k]
  int32_t* counts;        // [G]
  int32_t* indptr;        // [G + 1]
  int32_t* gather;        // [S_tot]
  int32_t* inv;           // [S]
  int32_t* meta;          // [META_WORDS]
  float* h;               // [S_tot, I] fp32 intermediate (bf16 for the bf16 format)
  uint16_t* out_slot;     // [S_tot, H] weighted bf16 slot rows
  uint32_t* amax;         // [2][amax_stride] per-row maxima of |h|, by launch parity
  int32_t* cnt;           // [2][cnt_stride] arrivals per (token, 16-channel block), by parity
  int32_t* bar;           // [2] grid barrier: arrival count, generation
  int amax_stride, cnt_stride;
  long spin_limit;        // bound on the barrier's wait (polls)
};
// Workgroups of the decode layer's persistent grid that are resident at
// once on `cus` compute units (0: the kernel cannot run).
int decode_layer_grid(int fmt, int act, int cus);
hipError_t launch_decode_layer(int fmt, const DecodeArgs& a, int grid, hipStream_t st);

hipError_t launch_route(const float* scores, int T, int E, int k, int score_fn, int32_t* ids,
                        float* w, const QuantArgs& fq, hipStream_t st);
hipError_t launch_dispatch(const DispatchArgs& d, hipStream_t st);
size_t dispatch_small_lds(int S, int G);
hipError_t launch_quant(const QuantArgs& q, hipStream_t st);
// bf16 activation rows, one wave per row (the routing launches' quantiser)
hipError_t launch_quant_rows(const QuantArgs& q, hipStream_t st);
hipError_t launch_combine(const CombineArgs& c, hipStream_t st);
hipError_t launch_indptr_table(const int32_t* user_indptr, int cap, const DispatchArgs& d,
                               hipStream_t st);
// Streaming (decode) grouped GEMM; fmt = Fmt, gateup = fused SwiGLU op.
hipError_t launch_gemm_stream(int fmt, bool gateup, const GemmArgs& g, hipStream_t st);
// Pipelined grouped GEMM (FP8 and MX formats).  Family 0 covers the tiled
// configurations 1 and 2 (row blocks of 32/64, four waves), family 1
// configuration 3 (128-row blocks, eight waves); g.cfg_self = -1 runs
// whichever of the family's configurations the device chose, a value >= 1
// only that one.
hipError_t launch_gemm_pipe(int fmt, bool gateup, int family, const GemmArgs& g, hipStream_t st);
// Rows from which the 128-row configuration may be chosen.
#define CFG3_MIN_ROWS 4096

// ---------------------------------------------------------------- backward
// Tiled transpose (64 x 64 blocks): out[z][c][out_col0 + r] =
// bf16(scale(r) * in[z][row(r)][c]) for r < R, c < C (C a multiple of 64),
// row(r) = gather ? gather[r] / gather_div : r, scale(r) = scale[gather[r]]
// or 1; rows r in [R, 64 ceil(R / 64)) are written as zeros; matrices z
// with counts[z] == 0 are skipped.
struct BwdTranspose {
  const uint16_t* in;
  long in_ld, in_zstride;
  uint16_t* out;
  long out_ld, out_zstride;
  int out_col0;
  int R, C;
  const int32_t* gather;
  int gather_div;
  const float* scale;
  const int32_t* counts;
};
// Weight-gradient GEMM: out[e][m, n] = sum over s in [indptr[e],
// indptr[e+1]) of a[s * lda + m] * b[row_b(s) * ldb + n], row_b(s) =
// b_tok[s] when b_tok is set, else s; out fp32 [E, M, N] (zeros for experts
// without rows).  M, N multiples of 128; lda, ldb multiples of 8; a and b
// 16-byte aligned; b_tok readable 64 entries past the last slot.
// Work comes from a chunk table (launch_bwd_chunks): each expert's rows in
// pieces; an expert's first piece writes out[e], the others partial
// buffers that a second pass adds to out[e] in piece order.  The grid
// takes the chunks in `order`, longest first.
struct BwdWgrad {
  const uint16_t* a;       // [slots, lda]
  long lda;
  const uint16_t* b;       // [rows, ldb]
  long ldb;
  const int32_t* b_tok;    // [slots + 64] b's row of each slot, or NULL
  const int32_t* chunks;   // [0]: count; from [4]: (expert, row0, row1, partial) per chunk
  const int32_t* nch;      // [E] pieces per expert
  const int32_t* pbase;    // [E] first partial index per expert
  const int32_t* multi;    // [0]: count; from [1]: the experts in more than one piece
  const int32_t* order;    // chunk indices, longest chunk first
  int M, N;
  float* out;
  float* partial;          // [partials, M, N]
};
// Per-slot pass of the backward (see backward.hip).
struct BwdSlot {
  const float* G;          // [rows, I] gate pre-activations (NULL for ReLU^2)
  const float* U;          // [rows, I]
  const float* R;          // [rows, I] Wd^T dy
  const float* topk_w;     // [T, k]
  const int32_t* gather;   // slot -> t * k + j
  const int32_t* indptr;   // [E + 1]
  int E, k, I, act;
  float limit;
  uint16_t* Hb;            // [rows, I] bf16 h
  uint16_t* DGU;           // [rows, 2 I] bf16: dg, then du
  float* dw;               // [T, k]
  const uint16_t* dy;      // [T, H] bf16
  int H;
  uint16_t* WDY;           // [rows, H] bf16 w dy_t
  int32_t* tok;            // [rows] t of each slot
};
struct BwdDx {
  const float* DA;         // [rows, H]
  const int32_t* inv;      // [T * k]
  int T, k, H;
  uint16_t* dx;            // [T, H] bf16
};
struct RouterBwd {
  const float* scores;     // [T, E]
  const int32_t* ids;      // [T, k]
  const float* w;          // [T, k]
  const float* dw;         // [T, k]
  int T, E, k, score_fn;
  float* ds;               // [T, E]
};
hipError_t launch_bwd_transpose(const BwdTranspose& a, int nz, hipStream_t st);
hipError_t launch_bwd_chunks(const int32_t* indptr, int E, int piece, int32_t* chunks,
                             int32_t* nch, int32_t* pbase, int32_t* multi, int32_t* order,
                             hipStream_t st);
// max_chunks: the grid's bound on chunks (E when every expert is one piece)
hipError_t launch_bwd_wgrad(const BwdWgrad& a, int E, int max_chunks, hipStream_t st);
hipError_t launch_bwd_slot(const BwdSlot& a, int max_rows, hipStream_t st);
hipError_t launch_bwd_dx(const BwdDx& a, hipStream_t st);
hipError_t launch_router_bwd(const RouterBwd& a, hipStream_t st);
