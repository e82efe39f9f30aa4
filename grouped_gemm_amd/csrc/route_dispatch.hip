// Top-k routing, deterministic expert-major dispatch, the block table and
// the on-device tile-configuration choice.
//
// Routing follows the Alpha-MoE news page ("How the megakernel works":
// routing and gating are stages of the layer) and the LightMoE README ("MoE
// inference": int32 ids distinct per token, fp32 weights).  Dispatch follows
// the LightMoE README (API table: deterministic expert-major dispatch;
// "Grouped GEMM": m_indptr of E+1 entries, zero-row experts valid; "MoE
// training": gather indices and inverse slots).  The block table is the
// block-id -> (expert, row offset) map of the pure-Triton MoE commentary
// (second paragraph).  The configuration is chosen from the runtime expert
// histogram as in the RaMP abstract.
//
// Determinism: integer counts are order-independent sums; every slot
// position comes from a stable rank (count of earlier equal ids), computed
// with wave ballots and per-wave prefix sums, never from atomic arrival order.
#include "layer.h"
#include "quant_row.h"
#include "route.h"

// One thread routes one token (small expert counts, E <= 32): k passes over
// the E scores, each taking the largest remaining key (score, then lowest
// index) -- exactly the order route_row16 produces.  Compact rolled loops,
// for scores staged in LDS; the choices go to ids_lds, from which a second
// pass forms the renormalised weights (no read-back of global memory).
DEVI void route_token_thread(const float* row, int E, int k, int score_fn, int32_t* ids_out,
                             float* w_out, int32_t* ids_lds) {
  uint32_t taken = 0;
  float top = 0.f, sum = 0.f;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    uint32_t bk = 0;
    for (int e = 0; e < E; ++e) {
      if ((taken >> e) & 1u) continue;
      const uint32_t key = score_key(row[e]);
      if (best < 0 || key > bk) {
        best = e;
        bk = key;
      }
    }
    taken |= 1u << best;
    ids_lds[j] = best;
    const float l = row[best];
    if (j == 0) top = l;
    sum += score_fn == MOE_SCORE_SOFTMAX ? expf(l - top)
           : score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-l)) : l;
  }
  for (int j = 0; j < k; ++j) {
    const int id = ids_lds[j];
    const float l = row[id];
    const float x = score_fn == MOE_SCORE_SOFTMAX ? expf(l - top)
                    : score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-l)) : l;
    ids_out[j] = id;
    w_out[j] = x / sum;
  }
}

// The same selection with the token's scores held in registers (all loads
// issued at once), for scores read from global memory.  The pass loop stays
// rolled (short code); the selection runs twice -- once for the weights'
// sum, once to write ids and renormalised weights -- rather than reading
// the unnormalised weights back from global memory.
DEVI void route_token_regs(const float* row, int E, int k, int score_fn, int32_t* ids_out,
                           float* w_out, int32_t* ids_lds) {
  float v[SMALL_E_THREAD_ROUTE];
#pragma unroll
  for (int e = 0; e < SMALL_E_THREAD_ROUTE; ++e) v[e] = e < E ? row[e] : 0.f;
  uint32_t key[SMALL_E_THREAD_ROUTE];
#pragma unroll
  for (int e = 0; e < SMALL_E_THREAD_ROUTE; ++e) key[e] = score_key(v[e]);
  float top = 0.f, sum = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    uint32_t taken = 0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      uint32_t bk = 0;
      float bv = 0.f;
#pragma unroll
      for (int e = 0; e < SMALL_E_THREAD_ROUTE; ++e) {
        const bool ok = e < E && !((taken >> e) & 1u) && (best < 0 || key[e] > bk);
        best = ok ? e : best;
        bk = ok ? key[e] : bk;
        bv = ok ? v[e] : bv;
      }
      taken |= 1u << best;
      if (j == 0) top = bv;
      const float x = score_fn == MOE_SCORE_SOFTMAX ? expf(bv - top)
                      : score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-bv)) : bv;
      if (pass == 0) {
        sum += x;
      } else {
        ids_out[j] = best;
        w_out[j] = x / sum;
        if (ids_lds) ids_lds[j] = best;
      }
    }
  }
}


template <int QF>
__global__ void __launch_bounds__(256) k_route_thread(const float* __restrict__ scores, int T, int E,
                                                      int k, int score_fn, int32_t* __restrict__ ids,
                                                      float* __restrict__ w, QuantArgs fq) {
  const int rb = (T + 255) / 256;
  if ((int)blockIdx.x >= rb) {
    quant_rows_waves<QF>(fq, ((int)blockIdx.x - rb) * 4 + (threadIdx.x >> 6), ((int)gridDim.x - rb) * 4,
                     threadIdx.x & 63);
    return;
  }
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  route_token_regs(scores + (size_t)t * E, E, k, score_fn, ids + (size_t)t * k, w + (size_t)t * k,
                     nullptr);
}

// Sixteen tokens per 256-thread block, one DPP row each.
template <int QF>
__global__ void __launch_bounds__(256) k_route16(const float* __restrict__ scores, int T, int E,
                                                 int k, int score_fn, int32_t* __restrict__ ids,
                                                 float* __restrict__ w, QuantArgs fq) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = (T + 15) / 16;
  if ((int)blockIdx.x >= rb) {
    quant_rows_waves<QF>(fq, ((int)blockIdx.x - rb) * 4 + wave, ((int)gridDim.x - rb) * 4, lane);
    return;
  }
  const int t = (int)blockIdx.x * 16 + (int)(threadIdx.x >> 4);
  const bool tv = t < T;
  const size_t tt = tv ? (size_t)t : 0;
  route_row16(scores + tt * E, tv, E, k, score_fn, threadIdx.x & 15, ids + tt * k, w + tt * k,
              nullptr);
}

// ------------------------------------------------------------------ ranks
// For lanes holding key e (valid, 0 <= e < 2^nbits), the number of lower
// lanes with the same key, the number of lanes with that key, and whether
// this lane is the highest one of its key.  The lanes holding my key are the
// intersection over the key bits b of ballot(bit b set) or its complement.
DEVI void wave_match(int e, bool valid, int lane, int nbits, int& rank, int& cnt, bool& last) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    m &= bit ? bb : ~bb;
  }
  rank = __popcll(m & ((1ull << lane) - 1ull));
  cnt = __popcll(m);
  last = (m >> lane) == 1ull;
}

DEVI int key_bits(int n) { return n <= 1 ? 0 : 32 - __clz(n - 1); }

// Stable ranks of up to 1024 keys held one per thread of a 1024-thread
// block (thread order = slot order).  wcnt is LDS [16][G] and must be zero
// on entry; it is zero again on exit.  Returns each valid thread's rank
// among lower threads with the same key; if `totals` is given, adds each
// key's count in this round to totals[key].
DEVI int block_stable_rank(int e, bool valid, int32_t* wcnt, int G, int32_t* totals) {
  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int rank, cnt;
  bool last;
  wave_match(e, valid, lane, key_bits(G), rank, cnt, last);
  if (valid && last) wcnt[wave * G + e] = cnt;
  __syncthreads();
  int pre = 0;
  if (valid)
    for (int w = 0; w < wave; ++w) pre += wcnt[w * G + e];
  __syncthreads();
  for (int g = tid; g < G; g += blockDim.x) {
    int s = 0;
    for (int w = 0; w < 16; ++w) {
      s += wcnt[w * G + g];
      wcnt[w * G + g] = 0;
    }
    if (totals) totals[g] += s;
  }
  __syncthreads();
  return pre + rank;
}

// Exclusive prefix sum of a[0..n) (n <= 1024) in LDS, in place, by all
// threads of a 1024-thread block: one element per thread (conflict-free LDS
// access), shuffle scans inside each wave, the 16 wave totals scanned by
// wave 0.  wsum is LDS [16]; *total (LDS) receives the sum.  Every thread
// must call it; a[] and *total are ready when it returns.
DEVI void block_exclusive_scan(int32_t* a, int n, int32_t* wsum, int32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = tid < n ? a[tid] : 0;
  const int inc = wave_incl_scan<false>(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? wsum[lane] : 0;
    const int winc = wave_incl_scan<false>(w);
    if (lane < 16) wsum[lane] = winc - w;
    if (lane == 15) *total = winc;
  }
  __syncthreads();
  if (tid < n) a[tid] = inc - v + wsum[wave];
  __syncthreads();
}

// ---------------------------------------------------------------- config choice
// Configuration from the runtime expert histogram (RaMP abstract: the best
// kernel configuration depends on the routing distribution, not on the batch
// size alone).  Statistics of the histogram: the active groups A, the largest
// group m, the mean group r = rows / A.  The rule, in order:
//  0. a batch of at most 16 tokens (every group then holds at most 16 rows)
//     -> cfg 0: the single-tile streaming kernel measured as fast as or
//     faster than 32-row tiles there (Mixtral-shaped T=8/16: 3-5% faster);
//  1. the work items a 32-row tiled grid would have (row blocks times output
//     channel blocks of the first projection) cannot fill half the CUs ->
//     cfg 0, the streaming kernel, which splits K across waves instead (with
//     rule 0 in place, larger batches leave it candidate only for layers
//     this small, so its launch rarely runs for nothing);
//  2. every group fits one 32-row block -> cfg 1 (each weight byte read
//     once, least MFMA padding);
//  3. every group fits one 64-row block -> cfg 2;
//  4. groups average 64 rows or more -> cfg 3 (128-row blocks, the
//     highest MFMA intensity per staged byte); otherwise cfg 2.
// The rule reproduces the fastest measured configuration on the benchmarked
// layer shapes; a fitted cost model over these statistics can replace it.
DEVI int config_rule(int mx, int active, int rows, int tiles32, int I, int num_cfgs, int cus, int T) {
  // T < 0 (a caller-supplied grouping, no token count): the largest group
  // bounds the rows of every group instead
  if (num_cfgs <= 1 || (T >= 0 ? T : mx) <= DECODE_STREAM_TOKENS) return 0;
  const long items32 = (long)tiles32 * (I / 128);
  if (2 * items32 < cus) return 0;
  if (mx <= 32) return 1;
  if (mx <= 64 || num_cfgs < 4) return num_cfgs < 3 ? 1 : 2;
  return (active > 0 && rows >= 64 * active && rows >= CFG3_MIN_ROWS) ? 3 : 2;
}

// The configuration of a histogram: the fitted cost model's least
// predicted time among the configurations the host launched kernels for
// (d.cm.mask; the lowest configuration on a tie), else the rule.  The loop
// over configurations is unrolled, so each evaluation reads the statistics
// at fixed fields (a per-lane configuration index would make the compiler
// index them through scratch memory).
DEVI int pick_config(const DispatchArgs& d, const HistStats& h) {
  // one candidate (the host launched one kernel family): nothing to weigh
  if (d.cm.on && d.cm.mask && !(d.cm.mask & (d.cm.mask - 1)) && d.cm.mask < (1 << d.num_cfgs))
    return __builtin_ctz((unsigned)d.cm.mask);
  if (d.cm.on && d.cm.mask) {
    int best = -1;
    double bt = 0.0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < d.num_cfgs && ((d.cm.mask >> c) & 1)) {
        const double t = cost_model_time(d.cm.th, h, c, d.fmt, d.H, d.I, d.T, d.cus);
        if (best < 0 || t < bt) {
          best = c;
          bt = t;
        }
      }
    }
    if (best >= 0) return best;
  }
  return config_rule(h.mx, h.active, h.rows, h.s32, d.I, d.num_cfgs, d.cus, d.T);
}

// Wave-wide histogram statistics from each lane's partial ones.
DEVI HistStats wave_stats(HistStats h) {
  h.mx = wave_total<true>(h.mx);
  h.active = wave_total<false>(h.active);
  h.rows = wave_total<false>(h.rows);
  h.s16 = wave_total<false>(h.s16);
  h.s32 = wave_total<false>(h.s32);
  h.s64 = wave_total<false>(h.s64);
  h.s128 = wave_total<false>(h.s128);
  return h;
}

DEVI void add_group(HistStats& h, int c) {
  h.mx = c > h.mx ? c : h.mx;
  h.active += c > 0;
  h.rows += c;
  h.s16 += (c + 15) >> 4;
  h.s32 += (c + 31) >> 5;
  h.s64 += (c + 63) >> 6;
  h.s128 += (c + 127) >> 7;
}

// The histogram statistics by one wave over the counts in LDS, then the
// configuration.
DEVI int choose_config(const DispatchArgs& d, const int32_t* cnt, int G, int lane, int* max_out) {
  HistStats h{};
  for (int g = lane; g < G; g += 64) add_group(h, cnt[g]);
  h = wave_stats(h);
  *max_out = h.mx;
  return pick_config(d, h);
}

// Shared tail of both dispatch paths.  cnt (LDS, G entries) holds the
// group counts; writes counts, m_indptr, the active-group list, the chosen
// configuration, its block table and meta.  All threads of a 1024-thread
// block must call it.
DEVI void finalize_dispatch(const DispatchArgs& d, int32_t* cnt, int32_t* scan_buf,
                            int32_t* flag_buf, int32_t* tiles_buf, int G, int S_total) {
  const int tid = threadIdx.x;
  __shared__ int32_t s_total, s_active, s_cfg, s_max, s_ntiles;
  __shared__ int32_t wsum[16];
  for (int g = tid; g < G; g += blockDim.x) {
    scan_buf[g] = cnt[g];
    flag_buf[g] = cnt[g] > 0 ? 1 : 0;
    d.counts[g] = cnt[g];
  }
  __syncthreads();
  if (tid < 64) {
    // one wave derives the configuration from the histogram
    int mx = 0;
    int cfg = choose_config(d, cnt, G, tid, &mx);
    if (d.force_cfg >= 0) cfg = d.force_cfg;
    if (tid == 0) {
      s_max = mx;
      s_cfg = cfg;
    }
  }
  block_exclusive_scan(scan_buf, G, wsum, &s_total);   // group offsets
  block_exclusive_scan(flag_buf, G, wsum, &s_active);  // positions in the active list
  for (int g = tid; g < G; g += blockDim.x)
    if (cnt[g] > 0) d.active[flag_buf[g]] = g;
  for (int g = tid; g <= G; g += blockDim.x) d.indptr[g] = (g < G) ? scan_buf[g] : s_total;
  // block table for the chosen row-block height: one entry per thread, its
  // group found by binary search over the groups' first table entries
  const int bm = cfg_rows(s_cfg);
  for (int g = tid; g < G; g += blockDim.x) tiles_buf[g] = (cnt[g] + bm - 1) / bm;
  __syncthreads();
  block_exclusive_scan(tiles_buf, G, wsum, &s_ntiles);
  for (int i = tid; i < s_ntiles; i += blockDim.x) {
    // the last group whose first entry is <= i owns entry i (groups without
    // rows share their first entry with the next group)
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tiles_buf[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    d.tiles[2 * i] = lo;
    d.tiles[2 * i + 1] = (i - tiles_buf[lo]) * bm;
  }
  if (tid == 0) {
    d.meta[META_NACTIVE] = s_active;
    d.meta[META_NTILES] = s_ntiles;
    d.meta[META_CFG] = s_cfg;
    d.meta[META_MAXCNT] = s_max;
    d.meta[META_ROWS] = S_total;
    d.meta[META_BM] = bm;
    d.meta[META_ERROR] = 0;
  }
}

// ---------------------------------------------------------------- small path
// Routing of tokens [t0, t0 + nt) by a 1024-thread block, ids also to
// ids_l[(t - t0) * k + j]: one thread per token for small expert counts,
// else one 16-lane row per token (64 tokens per pass).
DEVI void block_route(const DispatchArgs& d, int t0, int nt, int32_t* ids_l) {
  const int tid = threadIdx.x, k = d.k, E = d.E;
  if (E <= SMALL_E_THREAD_ROUTE) {
    for (int t = tid; t < nt; t += blockDim.x)
      route_token_regs(d.scores + (size_t)(t0 + t) * E, E, k, d.score_fn,
                       d.ids + (size_t)(t0 + t) * k, d.w + (size_t)(t0 + t) * k, ids_l + t * k);
  } else {
    for (int tb = 0; tb < nt; tb += 64) {
      // a wave whose four rows all lie past the batch skips the routine (its
      // cross-lane steps stay inside 16-lane rows), so at small batches the
      // idle waves do not compete with the working row for the SIMDs
      if (tb + 4 * (tid >> 6) >= nt) continue;
      const int t = tb + (tid >> 4);
      const bool tv = t < nt;
      const int tt = tv ? t : 0;
      route_row16(d.scores + (size_t)(t0 + tt) * E, tv, E, k, d.score_fn, tid & 15,
                  d.ids + (size_t)(t0 + tt) * k, d.w + (size_t)(t0 + tt) * k, ids_l + tt * k);
    }
  }
}

// One 1024-thread block: (optionally) routing, then counts, scan, stable
// scatter, active list, configuration and block table, for batches that
// route in one or two passes.  Blocks past the first quantise the
// activation rows.
template <int QF>
__global__ void __launch_bounds__(1024) k_dispatch_small(DispatchArgs d) {
  extern __shared__ int32_t smem[];
  const int G = d.E + d.shared;
  const int S = d.T * d.k;
  int32_t* ids_l = smem;                       // [S]
  int32_t* cnt = ids_l + S;                    // [G]
  int32_t* run = cnt + G;                      // [G] running offsets
  int32_t* wcnt = run + G;                     // [16*G]
  int32_t* scan_buf = wcnt + 16 * G;           // [G]
  int32_t* flag_buf = scan_buf + G;            // [G]
  int32_t* tiles_buf = flag_buf + G;           // [G]
  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x != 0) {   // blocks past the first quantise the activation rows
    quant_rows_waves<QF>(d.fq, ((int)blockIdx.x - 1) * 16 + wave, ((int)gridDim.x - 1) * 16, lane);
    return;
  }
  if (d.scores) {
    block_route(d, 0, d.T, ids_l);
  } else {
    for (int p = tid; p < S; p += blockDim.x) ids_l[p] = d.ids_in[p];
  }
  for (int g = tid; g < G; g += blockDim.x) {
    cnt[g] = 0;
    run[g] = 0;
  }
  for (int i = tid; i < 16 * G; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  for (int p = tid; p < S; p += blockDim.x) {
    const int e = ids_l[p];
    if ((unsigned)e < (unsigned)d.E) atomicAdd(&cnt[e], 1);   // an id out of range is dropped
  }
  __syncthreads();
  if (tid == 0 && d.shared) cnt[d.E] = d.T;
  __syncthreads();
  finalize_dispatch(d, cnt, scan_buf, flag_buf, tiles_buf, G, S + (d.shared ? d.T : 0));
  __syncthreads();
  // Stable scatter, 1024 slots per round.  scan_buf[g] is the next free
  // slot of group g; `run` collects this round's per-group totals.
  for (int base = 0; base < S; base += 1024) {
    int p = base + tid;
    int e = p < S ? ids_l[p] : 0;
    const bool valid = p < S && (unsigned)e < (unsigned)d.E;
    if (p < S && !valid) d.inv[p] = -1;
    e = valid ? e : 0;
    int r = block_stable_rank(e, valid, wcnt, G, run);
    if (valid) {
      int slot = scan_buf[e] + r;
      d.gather[slot] = p;
      d.inv[p] = slot;
    }
    __syncthreads();
    for (int g = tid; g < G; g += blockDim.x) {
      scan_buf[g] += run[g];
      run[g] = 0;
    }
    __syncthreads();
  }
  if (d.shared)
    for (int t = tid; t < d.T; t += blockDim.x) d.gather[S + t] = t * d.k;
}

// ---------------------------------------------------------------- tiny path
// LDS ordering inside one wave: its LDS operations complete in order, so
// waiting for them (and keeping the compiler from moving memory operations
// across) publishes every lane's writes to the other lanes.
DEVI void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One wave does everything for decode-sized batches (S <= 1024 slots, at
// most 64 groups): thread-per-token routing on scores staged in LDS,
// stable ranks over 64-slot chunks from ballots (group g's running count
// lives in lane g), the group scan, the active list, the configuration and
// its block table -- with no workgroup barrier.  The other waves of the
// grid quantise the activation rows meanwhile.
template <int QF>
__global__ void __launch_bounds__(256) k_dispatch_tiny(DispatchArgs d) {
  __shared__ int32_t ids_l[TINY_DISPATCH_SLOTS];
  __shared__ int32_t rk_l[TINY_DISPATCH_SLOTS];
  __shared__ float sc_l[TINY_SCORE_LDS];
  const int lane = threadIdx.x & 63;
  if (blockIdx.x != 0 || threadIdx.x >= 64) {
    quant_rows_waves<QF>(d.fq, (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6) - 1, (int)gridDim.x * 4 - 1,
                     lane);
    return;
  }
  const int G = d.E + d.shared;
  const int S = d.T * d.k;
  if (d.scores) {
    const int n = d.T * d.E;
    const float* src = d.scores;
    if (n <= TINY_SCORE_LDS) {
      // sixteen loads in flight per lane and pass (indices clamped into
      // the array, so no load waits behind a branch)
      for (int i = lane; i < n; i += 1024) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = d.scores[min(i + 64 * u, n - 1)];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (i + 64 * u < n) sc_l[i + 64 * u] = v[u];
      }
      wave_lds_sync();
      src = sc_l;
    }
    for (int t = lane; t < d.T; t += 64)
      route_token_thread(src + (size_t)t * d.E, d.E, d.k, d.score_fn, d.ids + (size_t)t * d.k,
                         d.w + (size_t)t * d.k, ids_l + t * d.k);
  } else {
    for (int p = lane; p < S; p += 64) ids_l[p] = d.ids_in[p];
  }
  wave_lds_sync();
  // Stable ranks, chunk by chunk in slot order.  Ids are below 64, so the
  // lanes holding id x are the intersection over the six id bits b of
  // ballot(bit b set) or its complement: M(x).  A lane's rank in its chunk
  // is the number of lower lanes in M(id); lane g adds |M(g)| to its
  // running count of group g.
  const uint64_t below = (1ull << lane) - 1ull;
  int run = 0;                               // lane g: rows of group g so far
  const int nch = (S + 63) / 64;
  for (int c = 0; c < nch; ++c) {
    const int p = c * 64 + lane;
    const int e0 = p < S ? ids_l[p] : 0;
    const bool valid = p < S && (unsigned)e0 < (unsigned)d.E;   // an id out of range is dropped
    const int e = valid ? e0 : 0;
    const uint64_t vm = __ballot(valid);
    uint64_t me = vm, mg = vm;                // lanes with my id / with id == lane
#pragma unroll
    for (int bt = 0; bt < 6; ++bt) {
      const uint64_t bb = __ballot(valid && ((e >> bt) & 1));
      me &= ((e >> bt) & 1) ? bb : ~bb;
      mg &= ((lane >> bt) & 1) ? bb : ~bb;
    }
    const int base = __shfl(run, e, 64);
    if (valid) rk_l[p] = base + __popcll(me & below);
    run += __popcll(mg);
  }
  const int cnt = lane < d.E ? run : (lane < G ? d.T : 0);   // group E is the shared expert
  // exclusive scan of the counts
  const int inc = wave_incl_scan<false>(cnt);
  const int excl = inc - cnt;
  const int total = __builtin_amdgcn_readlane(inc, 63);
  if (lane < G) {
    d.counts[lane] = cnt;
    d.indptr[lane] = excl;
  }
  if (lane == 0) d.indptr[G] = total;
  // active list
  const uint64_t act = __ballot(lane < G && cnt > 0);
  if (lane < G && cnt > 0) d.active[__popcll(act & below)] = lane;
  // configuration from the histogram statistics (lane g holds group g)
  HistStats hs{};
  add_group(hs, cnt);
  const int mx = wave_total<true>(cnt);
  const int cfg = d.force_cfg >= 0 ? d.force_cfg : pick_config(d, wave_stats(hs));
  // block table for the chosen row-block height
  const int bm = cfg_rows(cfg);
  const int nt = lane < G ? (cnt + bm - 1) / bm : 0;
  const int tinc = wave_incl_scan<false>(nt);
  for (int r = 0, b = tinc - nt; r < nt; ++r) {
    d.tiles[2 * (b + r)] = lane;
    d.tiles[2 * (b + r) + 1] = r * bm;
  }
  const int ntiles = __builtin_amdgcn_readlane(tinc, 63);
  if (lane == 0) {
    d.meta[META_NACTIVE] = __popcll(act);
    d.meta[META_NTILES] = ntiles;
    d.meta[META_CFG] = cfg;
    d.meta[META_MAXCNT] = mx;
    d.meta[META_ROWS] = total;
    d.meta[META_BM] = bm;
    d.meta[META_ERROR] = 0;
  }
  // gather / inverse slots (a lane reads back only its own rank entries)
  for (int c = 0; c < nch; ++c) {
    const int p = c * 64 + lane;
    const int e0 = p < S ? ids_l[p] : 0;
    const bool valid = p < S && (unsigned)e0 < (unsigned)d.E;
    const int e = valid ? e0 : 0;
    const int slot = __shfl(excl, e, 64) + (valid ? rk_l[p] : 0);
    if (valid) {
      d.gather[slot] = p;
      d.inv[p] = slot;
    } else if (p < S) {
      d.inv[p] = -1;
    }
  }
  if (d.shared)
    for (int t = lane; t < d.T; t += 64) d.gather[S + t] = t * d.k;
}

// ---------------------------------------------------------------- chunked path
// Two launches for large batches.  Chunk c holds the tokens
// [c*TC, c*TC + TC), TC = floor(1024 / k): whole tokens, at most 1024 slots.
DEVI int chunk_tokens(int k) { return 1024 / k; }

// Pass 1, block c: route the chunk's tokens (or read their ids), rank each
// slot among the chunk's slots of the same expert (slot order, so stable)
// and write the chunk's expert histogram.  The rank is parked in inv[];
// pass 2 replaces it by the slot.  Blocks past the chunks quantise the
// activation rows.
template <int QF>
__global__ void __launch_bounds__(1024) k_dispatch_chunk(DispatchArgs d) {
  extern __shared__ int32_t smem[];
  int32_t* ids_l = smem;             // [1024]
  int32_t* wcnt = smem + 1024;       // [16][E]
  const int E = d.E, k = d.k, TC = chunk_tokens(k);
  const int nch = (d.T + TC - 1) / TC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if ((int)blockIdx.x >= nch) {
    quant_rows_waves<QF>(d.fq, ((int)blockIdx.x - nch) * 16 + wave, ((int)gridDim.x - nch) * 16, lane);
    return;
  }
  const int c = blockIdx.x, t0 = c * TC, nt = min(TC, d.T - t0), ns = nt * k, p0 = t0 * k;
  for (int i = tid; i < 16 * E; i += blockDim.x) wcnt[i] = 0;
  if (d.scores) block_route(d, t0, nt, ids_l);
  else
    for (int i = tid; i < ns; i += blockDim.x) ids_l[i] = d.ids_in[p0 + i];
  __syncthreads();
  const int e0 = tid < ns ? ids_l[tid] : 0;
  const bool valid = tid < ns && (unsigned)e0 < (unsigned)E;   // an id out of range is dropped
  const int e = valid ? e0 : 0;
  int rank, cnt;
  bool last;
  wave_match(e, valid, lane, key_bits(E), rank, cnt, last);
  if (valid && last) wcnt[wave * E + e] = cnt;
  __syncthreads();
  if (valid) {
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wcnt[w * E + e];
    d.inv[p0 + tid] = pre + rank;
  }
  for (int g = tid; g < E; g += blockDim.x) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) s += wcnt[w * E + g];
    d.chunk[(size_t)c * E + g] = s;
  }
}

// Pass 2.  Block c < nch: from the chunk histograms, each group's total and
// its rows in the chunks before c (P = 1024/E threads per group split the
// chunks); the exclusive scan of the totals gives the group starts, and the
// chunk's slots land at start + earlier rows + rank.  Block nch writes
// counts, m_indptr, the active list, the configuration and its block table
// (and the shared group's gather entries), so no placing block waits for
// it.  ids_in holds the routed ids.
__global__ void __launch_bounds__(1024) k_dispatch_place(DispatchArgs d) {
  extern __shared__ int32_t smem[];
  const int E = d.E, G = E + d.shared, k = d.k, TC = chunk_tokens(k);
  const int S = d.T * k, nch = (d.T + TC - 1) / TC;
  int32_t* cnt = smem;                 // [G]
  int32_t* pre_l = cnt + G;            // [G]
  int32_t* scan_buf = pre_l + G;       // [G]
  int32_t* flag_buf = scan_buf + G;    // [G]
  int32_t* tiles_buf = flag_buf + G;   // [G]
  int32_t* part = tiles_buf + G;       // [2][1024]
  const int c = blockIdx.x, tid = threadIdx.x;
  const bool table = c == nch;
  // this thread's slot: its id and rank load first, in flight meanwhile
  const int t0 = c * TC, ns = table ? 0 : min(TC, d.T - t0) * k, p = t0 * k + tid;
  const bool mine = tid < ns;
  const int e = mine ? d.ids_in[p] : -1;
  const int rank = mine ? d.inv[p] : 0;
  const int P = 1024 / E, g = tid % E, q = tid / E;
  int tot = 0, pre = 0;
  if (q < P) {
    for (int c0 = q; c0 < nch; c0 += 16 * P) {   // sixteen loads in flight
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int cc = c0 + u * P;
        v[u] = d.chunk[(size_t)min(cc, nch - 1) * E + g];
        v[u] = cc < nch ? v[u] : 0;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        tot += v[u];
        pre += c0 + u * P < c ? v[u] : 0;
      }
    }
  }
  part[tid] = tot;
  part[1024 + tid] = pre;
  __syncthreads();
  if (tid < E) {
    int a = 0, b = 0;
    for (int qq = 0; qq < P; ++qq) {
      a += part[qq * E + tid];
      b += part[1024 + qq * E + tid];
    }
    cnt[tid] = a;
    pre_l[tid] = b;
  }
  if (tid == 0 && d.shared) cnt[E] = d.T;
  __syncthreads();
  if (table) {
    finalize_dispatch(d, cnt, scan_buf, flag_buf, tiles_buf, G, S + (d.shared ? d.T : 0));
    if (d.shared)
      for (int t = tid; t < d.T; t += blockDim.x) d.gather[S + t] = t * k;
    return;
  }
  for (int i = tid; i < G; i += blockDim.x) scan_buf[i] = cnt[i];
  __syncthreads();
  __shared__ int32_t wsum_p[16], total_p;
  block_exclusive_scan(scan_buf, G, wsum_p, &total_p);
  if (mine) {
    if ((unsigned)e < (unsigned)E) {
      const int slot = scan_buf[e] + pre_l[e] + rank;
      d.gather[slot] = p;
      d.inv[p] = slot;
    } else {
      d.inv[p] = -1;
    }
  }
}

// ---------------------------------------------------------------- decode path
// Batches of at most DECODE_STREAM_TOKENS tokens, any expert count: one
// 256-thread block routes every token (one 16-lane row each), counts the
// groups in LDS, scans the counts with one wave (five groups per lane),
// places each slot by counting the earlier slots of its group (at most 255)
// and writes the tables (with ids distinct per token a group holds at most
// 16 rows, one block-table entry whatever the configuration).  Blocks past
// the first quantise the activation rows.
template <int QF>
__global__ void __launch_bounds__(256) k_dispatch_decode(DispatchArgs d) {
  __shared__ int32_t ids_l[DECODE_STREAM_TOKENS * 16];
  __shared__ int32_t cnt_l[320];
  __shared__ int32_t ind_l[321];
  __shared__ int32_t act_l[320];
  __shared__ int32_t tof_l[321];
  __shared__ int32_t nact_l, mx_l, cfg_l, ntiles_l;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x != 0) {
    quant_rows_waves<QF>(d.fq, ((int)blockIdx.x - 1) * 4 + wave, ((int)gridDim.x - 1) * 4, lane);
    return;
  }
  const int T = d.T, E = d.E, k = d.k, S = T * k;
  const int G = E + d.shared;
  if (d.scores) {
    const int t = wave * 4 + (lane >> 4);
    const bool tv = t < T;
    route_row16(d.scores + (size_t)(tv ? t : 0) * E, tv, E, k, d.score_fn, lane & 15,
                d.ids + (size_t)(tv ? t : 0) * k, d.w + (size_t)(tv ? t : 0) * k,
                ids_l + (tv ? t : 0) * k);
  } else {
    for (int p = tid; p < S; p += 256) ids_l[p] = d.ids_in[p];
  }
  for (int g = tid; g < 320; g += 256) cnt_l[g] = 0;
  __syncthreads();
  for (int p = tid; p < S; p += 256) {
    const int e = ids_l[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt_l[e], 1);   // an id out of range is dropped
  }
  __syncthreads();
  if (tid == 0 && d.shared) cnt_l[E] = T;
  __syncthreads();
  if (wave == 0) {
    int c[5], f[5], cs = 0, fs = 0;
    HistStats hs{};
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      c[i] = cnt_l[lane * 5 + i];   // zero past G
      f[i] = c[i] > 0;
      cs += c[i];
      fs += f[i];
      add_group(hs, c[i]);
    }
    int ce = wave_incl_scan<false>(cs) - cs, fe = wave_incl_scan<false>(fs) - fs;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int gg = lane * 5 + i;
      if (gg < G) {
        ind_l[gg] = ce;
        if (f[i]) act_l[fe] = gg;
      }
      ce += c[i];
      fe += f[i];
    }
    const int tot = wave_total<false>(cs), nact = wave_total<false>(fs);
    const int mx = wave_total<true>(hs.mx);
    const int cfg = d.force_cfg >= 0 ? d.force_cfg : pick_config(d, wave_stats(hs));
    if (lane == 0) {
      ind_l[G] = tot;
      nact_l = nact;
      mx_l = mx;
      cfg_l = cfg;
    }
  }
  __syncthreads();
  // stable placement: slot order is expert, then flat index t*k+j
  for (int p = tid; p < S; p += 256) {
    const int e = ids_l[p];
    if ((unsigned)e < (unsigned)E) {
      int r = 0;
      for (int q = 0; q < p; ++q) r += ids_l[q] == e;
      const int slot = ind_l[e] + r;
      d.gather[slot] = p;
      d.inv[p] = slot;
    } else {
      d.inv[p] = -1;
    }
  }
  if (d.shared)
    for (int t = tid; t < T; t += 256) d.gather[S + t] = t * k;
  const int nact = nact_l, bm = cfg_rows(cfg_l);
  for (int g = tid; g < G; g += 256) d.counts[g] = cnt_l[g];
  for (int g = tid; g <= G; g += 256) d.indptr[g] = ind_l[g];
  for (int i = tid; i < nact; i += 256) d.active[i] = act_l[i];
  // block table: ceil(rows / bm) entries per group, groups ascending
  if (wave == 0) {
    int nt[5], ns = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      nt[i] = (cnt_l[lane * 5 + i] + bm - 1) / bm;
      ns += nt[i];
    }
    int o = wave_incl_scan<false>(ns) - ns;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      tof_l[lane * 5 + i] = o;
      o += nt[i];
    }
    const int tot = wave_total<false>(ns);
    if (lane == 0) ntiles_l = tot;
  }
  __syncthreads();
  for (int g = tid; g < G; g += 256) {
    const int n = (cnt_l[g] + bm - 1) / bm, o = tof_l[g];
    for (int r = 0; r < n; ++r) {
      d.tiles[2 * (o + r)] = g;
      d.tiles[2 * (o + r) + 1] = r * bm;
    }
  }
  if (tid == 0) {
    d.meta[META_NACTIVE] = nact;
    d.meta[META_NTILES] = ntiles_l;
    d.meta[META_CFG] = cfg_l;
    d.meta[META_MAXCNT] = mx_l;
    d.meta[META_ROWS] = S + (d.shared ? T : 0);
    d.meta[META_BM] = cfg_rows(cfg_l);
    d.meta[META_ERROR] = 0;
  }
}

// ---------------------------------------------------------------- host launchers
size_t dispatch_small_lds(int S, int G) {
  return sizeof(int32_t) * ((size_t)S + 2 * G + 16 * G + 3 * G);
}

// The one-block path routes in at most two passes (thread per token for
// small expert counts, else 64 tokens per pass) and scatters at most two
// rounds of 1024 slots.
static bool small_path(const DispatchArgs& d) {
  const int S = d.T * d.k;
  return S <= SMALL_DISPATCH_SLOTS && (d.E <= SMALL_E_THREAD_ROUTE || d.T <= 128);
}

// Blocks (of `wpb` waves) to add to a launch so its spare waves quantise
// fq.R rows: about one wave per row, at most a few blocks per CU.
static int quant_blocks(const QuantArgs& fq, int wpb, int spare_waves) {
  if (fq.R <= 0) return 0;
  const int need = fq.R - spare_waves;
  if (need <= 0) return spare_waves > 0 ? 0 : 1;
  const int b = (need + wpb - 1) / wpb;
  return b < 2048 ? b : 2048;
}

hipError_t launch_route(const float* scores, int T, int E, int k, int score_fn, int32_t* ids,
                        float* w, const QuantArgs& fq, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (E <= SMALL_E_THREAD_ROUTE) {
    const int rb = (T + 255) / 256;
    LAUNCH_QF(quant_format(fq), k_route_thread, dim3(rb + quant_blocks(fq, 4, 0)), dim3(256), 0, st,
              scores, T, E, k, score_fn, ids, w, fq);
  } else {
    const int rb = (T + 15) / 16;
    LAUNCH_QF(quant_format(fq), k_route16, dim3(rb + quant_blocks(fq, 4, 0)), dim3(256), 0, st,
              scores, T, E, k, score_fn, ids, w, fq);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& d, hipStream_t st) {
  const int G = d.E + d.shared;
  const int S = d.T * d.k;
  if (d.T >= 1 && d.T <= DECODE_STREAM_TOKENS && G <= 320) {
    const int grid = 1 + (d.fq.R > 0 ? (d.fq.R + 3) / 4 : 0);
    LAUNCH_QF(quant_format(d.fq), k_dispatch_decode, dim3(grid), dim3(256), 0, st, d);
    return hipGetLastError();
  }
  if (S <= TINY_DISPATCH_SLOTS && G <= 64 && (!d.scores || d.E <= SMALL_E_THREAD_ROUTE)) {
    const int grid = 1 + quant_blocks(d.fq, 4, 3);
    LAUNCH_QF(quant_format(d.fq), k_dispatch_tiny, dim3(grid), dim3(256), 0, st, d);
    return hipGetLastError();
  }
  if (small_path(d)) {
    const int grid = 1 + quant_blocks(d.fq, 16, 0);
    LAUNCH_QF(quant_format(d.fq), k_dispatch_small, dim3(grid), dim3(1024), dispatch_small_lds(S, G),
              st, d);
    return hipGetLastError();
  }
  // chunked path: routing (with the input quantisation on spare blocks) as
  // a grid of its own over every CU -- concentrated on the chunk blocks it
  // would be bound by their vector ALUs -- then ranks and histograms per
  // chunk, then placement
  DispatchArgs d1 = d;
  if (d.scores) {
    hipError_t e = launch_route(d.scores, d.T, d.E, d.k, d.score_fn, d.ids, d.w, d.fq, st);
    if (e != hipSuccess) return e;
    d1.scores = nullptr;
    d1.ids_in = d.ids;
    d1.fq.R = 0;
  }
  const int TC = 1024 / d.k, nch = (d.T + TC - 1) / TC;
  LAUNCH_QF(quant_format(d1.fq), k_dispatch_chunk, dim3(nch + quant_blocks(d1.fq, 16, 0)), dim3(1024),
            sizeof(int32_t) * (1024 + 16 * d.E), st, d1);
  DispatchArgs d2 = d1;
  d2.fq.R = 0;
  hipLaunchKernelGGL(k_dispatch_place, dim3(nch + 1), dim3(1024), sizeof(int32_t) * (5 * G + 2048),
                     st, d2);
  return hipGetLastError();
}

// Block table, counts and active list from a caller-supplied m_indptr (the
// standalone grouped GEMM).  Rejects (runs nothing) when m_indptr is not
// non-decreasing from 0 or exceeds `cap` rows.
__global__ void __launch_bounds__(1024) k_indptr_table(const int32_t* __restrict__ user_indptr,
                                                       int cap, DispatchArgs d) {
  extern __shared__ int32_t smem[];
  const int G = d.E;
  int32_t* cnt = smem;
  int32_t* scan_buf = cnt + G;
  int32_t* flag_buf = scan_buf + G;
  int32_t* tiles_buf = flag_buf + G;
  __shared__ int bad;
  int tid = threadIdx.x;
  if (tid == 0) bad = (user_indptr[0] != 0 || user_indptr[G] > cap) ? 1 : 0;
  __syncthreads();
  for (int g = tid; g < G; g += blockDim.x) {
    int c = user_indptr[g + 1] - user_indptr[g];
    if (c < 0) atomicOr(&bad, 1);
    cnt[g] = c;
  }
  __syncthreads();
  if (bad) {
    for (int g = tid; g < G; g += blockDim.x) cnt[g] = 0;
    __syncthreads();
  }
  finalize_dispatch(d, cnt, scan_buf, flag_buf, tiles_buf, G, bad ? 0 : user_indptr[G]);
  if (tid == 0 && bad) d.meta[META_ERROR] = 1;
}

hipError_t launch_indptr_table(const int32_t* user_indptr, int cap, const DispatchArgs& d,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_indptr_table, dim3(1), dim3(1024), sizeof(int32_t) * 4 * d.E, st,
                     user_indptr, cap, d);
  return hipGetLastError();
}
