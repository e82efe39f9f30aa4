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
};

// Store four consecutive down-projection outputs of one row.
DEVI void store_down(const GemmArgs& p, int slot, int n0, f32x4 v) {
  if (p.row_w) {
    const float w = slot < p.row_w_n ? p.row_w[p.row_w_idx[slot]] : 1.0f;
    v = v * w;
    uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
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
hipError_t launch_gemm_tiled(int fmt, bool gateup, int cfg, const GemmArgs& g, hipStream_t st);
// Pipelined grouped GEMM (FP8 and MX formats).  Family 0 covers the tiled
// configurations 1 and 2 (row blocks of 32/64, four waves), family 1
// configuration 3 (128-row blocks, eight waves); g.cfg_self = -1 runs
// whichever of the family's configurations the device chose, a value >= 1
// only that one.
hipError_t launch_gemm_pipe(int fmt, bool gateup, int family, const GemmArgs& g, hipStream_t st);
// Rows from which the 128-row configuration may be chosen.
#define CFG3_MIN_ROWS 4096
