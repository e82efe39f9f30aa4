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

// Order-preserving map of an fp32 score to uint32 (+0 and -0 compare equal).
DEVI uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

DEVI uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// One wave routes one token.  Each lane keeps up to four candidate experts
// (e = lane + 64*i) as 64-bit keys (score key, 0xFFFF - e): the maximum key
// is the highest score with the lowest index among equals.
DEVI void route_one_token(const float* row, int E, int k, int score_fn, int lane, int32_t* ids_out,
                          float* w_out, int32_t* ids_lds) {
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)score_key(row[e]) << 32) | (uint32_t)(0xFFFF - e)) : 0ull;
  }
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      uint64_t other = shfl_xor_u64(best, o);
      best = other > best ? other : best;
    }
    int be = 0xFFFF - (int)(best & 0xFFFFu);
    if (lane == (be & 63)) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i == (be >> 6)) key[i] = 0ull;
    }
    if (lane == j) my_id = be;
  }
  // gate weights over the chosen k, renormalised
  float l = (lane < k) ? row[my_id] : 0.f;
  float top = __shfl(l, 0, 64);
  float v = 0.f;
  if (lane < k) {
    if (score_fn == MOE_SCORE_SOFTMAX)
      v = expf(l - top);
    else if (score_fn == MOE_SCORE_SIGMOID)
      v = 1.0f / (1.0f + expf(-l));
    else
      v = l;
  }
  float sum = wave_sum(v);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = v / sum;
    if (ids_lds) ids_lds[lane] = my_id;
  }
}

// One thread routes one token (small expert counts, E <= 32): k passes over
// the E scores, each taking the largest remaining key (score, then lowest
// index) -- exactly the order route_one_token produces.  Compact rolled
// loops, for scores staged in LDS.
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
    ids_out[j] = best;
    if (ids_lds) ids_lds[j] = best;
    const float l = row[best];
    if (j == 0) top = l;
    const float x = score_fn == MOE_SCORE_SOFTMAX ? expf(l - top)
                    : score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-l)) : l;
    w_out[j] = x;
    sum += x;
  }
  for (int j = 0; j < k; ++j) w_out[j] = w_out[j] / sum;
}

// The same selection with the token's scores held in registers (all loads
// issued at once), for scores read from global memory.
DEVI void route_token_regs(const float* row, int E, int k, int score_fn, int32_t* ids_out,
                           float* w_out, int32_t* ids_lds) {
  float v[SMALL_E_THREAD_ROUTE];
#pragma unroll
  for (int e = 0; e < SMALL_E_THREAD_ROUTE; ++e) v[e] = e < E ? row[e] : 0.f;
  uint32_t key[SMALL_E_THREAD_ROUTE];
#pragma unroll
  for (int e = 0; e < SMALL_E_THREAD_ROUTE; ++e) key[e] = score_key(v[e]);
  uint32_t taken = 0;
  float top = 0.f, sum = 0.f;
  // the pass loop stays rolled (short code); unnormalised weights go to
  // w_out and are divided by their sum once all k are known
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
    ids_out[j] = best;
    if (ids_lds) ids_lds[j] = best;
    if (j == 0) top = bv;
    const float x = score_fn == MOE_SCORE_SOFTMAX ? expf(bv - top)
                    : score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-bv)) : bv;
    w_out[j] = x;
    sum += x;
  }
  for (int j = 0; j < k; ++j) w_out[j] = w_out[j] / sum;
}

__global__ void __launch_bounds__(256) k_route_thread(const float* __restrict__ scores, int T, int E,
                                                      int k, int score_fn, int32_t* __restrict__ ids,
                                                      float* __restrict__ w, QuantArgs fq) {
  const int rb = (T + 255) / 256;
  if ((int)blockIdx.x >= rb) {
    quant_rows_waves(fq, ((int)blockIdx.x - rb) * 4 + (threadIdx.x >> 6), ((int)gridDim.x - rb) * 4,
                     threadIdx.x & 63);
    return;
  }
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  route_token_regs(scores + (size_t)t * E, E, k, score_fn, ids + (size_t)t * k, w + (size_t)t * k,
                     nullptr);
}

__global__ void __launch_bounds__(256) k_route(const float* __restrict__ scores, int T, int E, int k,
                                               int score_fn, int32_t* __restrict__ ids,
                                               float* __restrict__ w, QuantArgs fq) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = (T + 3) / 4;
  if ((int)blockIdx.x >= rb) {
    quant_rows_waves(fq, ((int)blockIdx.x - rb) * 4 + wave, ((int)gridDim.x - rb) * 4, lane);
    return;
  }
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  route_one_token(scores + (size_t)t * E, E, k, score_fn, lane, ids + (size_t)t * k,
                  w + (size_t)t * k, nullptr);
}

// ------------------------------------------------------------------ ranks
// For lanes holding key e (valid), the number of lower lanes with the same
// key, the number of lanes with that key, and whether this lane is the
// highest one of its key.
DEVI void wave_match(int e, bool valid, int lane, int& rank, int& cnt, bool& last) {
  uint64_t todo = __ballot(valid);
  rank = 0;
  cnt = 0;
  last = false;
  while (todo) {
    int leader = __ffsll((unsigned long long)todo) - 1;
    int le = __shfl(e, leader, 64);
    bool mine = valid && e == le;
    uint64_t m = __ballot(mine);
    if (mine) {
      rank = __popcll(m & ((1ull << lane) - 1ull));
      cnt = __popcll(m);
      last = lane == (63 - __clzll(m));
    }
    todo &= ~m;
  }
}

// Stable ranks of up to 1024 keys held one per thread of a 1024-thread
// block (thread order = slot order).  wcnt is LDS [16][G] and must be zero
// on entry; it is zero again on exit.  Returns each valid thread's rank
// among lower threads with the same key; if `totals` is given, adds each
// key's count in this round to totals[key].
DEVI int block_stable_rank(int e, bool valid, int32_t* wcnt, int G, int32_t* totals) {
  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int rank, cnt;
  bool last;
  wave_match(e, valid, lane, rank, cnt, last);
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

// Exclusive prefix sum of n <= 1024 ints in LDS, in place, by one wave
// (wave 0); returns nothing, result visible after the caller's barrier.
DEVI void wave0_exclusive_scan(int32_t* a, int n, int32_t* total) {
  int tid = threadIdx.x;
  if (tid >= 64) return;
  constexpr int PER = 16;
  int base = tid * PER;
  int loc[PER];
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    loc[i] = (base + i < n) ? a[base + i] : 0;
    s += loc[i];
  }
  int inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(inc, o, 64);
    if (tid >= o) inc += v;
  }
  int run = inc - s;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (base + i < n) a[base + i] = run;
    run += loc[i];
  }
  if (tid == 63 && total) *total = inc;
}

// ---------------------------------------------------------------- config choice
// Configuration from the runtime expert histogram (RaMP abstract: the best
// kernel configuration depends on the routing distribution, not on the batch
// size alone).  Statistics of the histogram: the active groups A, the largest
// group m, the mean group r = rows / A.  The rule, in order:
//  1. the work items a 32-row tiled grid would have (row blocks times output
//     channel blocks of the first projection) cannot fill the CUs -> cfg 0,
//     the streaming kernel, which splits K across waves instead;
//  2. every group fits one 32-row block -> cfg 1 (each weight byte read
//     once, least MFMA padding);
//  3. every group fits one 64-row block -> cfg 2;
//  4. groups average 64 rows or more -> cfg 3 (128-row blocks, the
//     highest MFMA intensity per staged byte); otherwise cfg 2.
// The rule reproduces the fastest measured configuration on the benchmarked
// layer shapes; a fitted cost model over these statistics can replace it.
DEVI int config_rule(int mx, int active, int rows, int tiles32, int I, int num_cfgs, int cus) {
  if (num_cfgs <= 1) return 0;
  const long items32 = (long)tiles32 * (I / 128);
  if (items32 < cus) return 0;
  if (mx <= 32) return 1;
  if (mx <= 64 || num_cfgs < 4) return num_cfgs < 3 ? 1 : 2;
  return (active > 0 && rows >= 64 * active && rows >= CFG3_MIN_ROWS) ? 3 : 2;
}

// The histogram statistics by one wave over the counts in LDS, then the rule.
DEVI int choose_config(const int32_t* cnt, int G, int I, int num_cfgs, int cus, int lane,
                      int* max_out) {
  int mx = 0, active = 0, rows = 0, tiles32 = 0;
  for (int g = lane; g < G; g += 64) {
    const int c = cnt[g];
    mx = c > mx ? c : mx;
    active += c > 0;
    rows += c;
    tiles32 += (c + 31) / 32;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int v = __shfl_xor(mx, o, 64);
    mx = v > mx ? v : mx;
    active += __shfl_xor(active, o, 64);
    rows += __shfl_xor(rows, o, 64);
    tiles32 += __shfl_xor(tiles32, o, 64);
  }
  *max_out = mx;
  return config_rule(mx, active, rows, tiles32, I, num_cfgs, cus);
}

// Shared tail of both dispatch paths.  cnt (LDS, G entries) holds the
// group counts; writes counts, m_indptr, the active-group list, the chosen
// configuration, its block table and meta.  All threads of a 1024-thread
// block must call it.
DEVI void finalize_dispatch(const DispatchArgs& d, int32_t* cnt, int32_t* scan_buf,
                            int32_t* flag_buf, int32_t* tiles_buf, int G, int S_total) {
  int tid = threadIdx.x;
  __shared__ int32_t s_total, s_active, s_cfg, s_max, s_ntiles;
  for (int g = tid; g < G; g += blockDim.x) {
    scan_buf[g] = cnt[g];
    flag_buf[g] = cnt[g] > 0 ? 1 : 0;
    d.counts[g] = cnt[g];
  }
  __syncthreads();
  wave0_exclusive_scan(scan_buf, G, &s_total);
  __syncthreads();
  if (tid >= 64 && tid < 128) {
    // a second wave scans the active flags concurrently
    int l = tid - 64;
    constexpr int PER = 16;
    int base = l * PER, loc[PER], s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      loc[i] = (base + i < G) ? flag_buf[base + i] : 0;
      s += loc[i];
    }
    int inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(inc, o, 64);
      if (l >= o) inc += v;
    }
    int run = inc - s;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (base + i < G && loc[i]) d.active[run] = base + i;
      run += loc[i];
    }
    if (l == 63) s_active = inc;
  }
  if (tid >= 128 && tid < 192) {
    // one wave derives the configuration from the histogram
    int l = tid - 128, mx = 0;
    int cfg = choose_config(cnt, G, d.I, d.num_cfgs, d.cus, l, &mx);
    if (d.force_cfg >= 0) cfg = d.force_cfg;
    if (l == 0) {
      s_max = mx;
      s_cfg = cfg;
    }
  }
  __syncthreads();
  for (int g = tid; g <= G; g += blockDim.x) d.indptr[g] = (g < G) ? scan_buf[g] : s_total;
  // block table for the chosen row-block height
  int bm = cfg_rows(s_cfg);
  for (int g = tid; g < G; g += blockDim.x) tiles_buf[g] = (cnt[g] + bm - 1) / bm;
  __syncthreads();
  wave0_exclusive_scan(tiles_buf, G, &s_ntiles);
  __syncthreads();
  for (int g = tid; g < G; g += blockDim.x) {
    int n = (cnt[g] + bm - 1) / bm, base = tiles_buf[g];
    for (int r = 0; r < n; ++r) {
      d.tiles[2 * (base + r)] = g;
      d.tiles[2 * (base + r) + 1] = r * bm;
    }
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
// One 1024-thread block: (optionally) routing, then counts, scan, stable
// scatter, active list, configuration and block table.  For S = T*k <= 8192.
// Blocks past the first quantise the activation rows.
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
  float* sc_l = (float*)(tiles_buf + G);       // [T*E] router scores (routing fused)
  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x != 0) {   // blocks past the first quantise the activation rows
    quant_rows_waves(d.fq, ((int)blockIdx.x - 1) * 16 + wave, ((int)gridDim.x - 1) * 16, lane);
    return;
  }

  if (d.scores) {
    // all scores into LDS with coalesced loads, then one wave per token
    const int n = d.T * d.E;
    for (int i = tid; i < n; i += blockDim.x) sc_l[i] = d.scores[i];
    __syncthreads();
    if (d.E <= SMALL_E_THREAD_ROUTE) {
      for (int t = tid; t < d.T; t += blockDim.x)
        route_token_thread(sc_l + t * d.E, d.E, d.k, d.score_fn, d.ids + (size_t)t * d.k,
                           d.w + (size_t)t * d.k, ids_l + t * d.k);
    } else {
      for (int t = wave; t < d.T; t += 16)
        route_one_token(sc_l + t * d.E, d.E, d.k, d.score_fn, lane, d.ids + (size_t)t * d.k,
                        d.w + (size_t)t * d.k, ids_l + t * d.k);
    }
  } else {
    for (int p = tid; p < S; p += blockDim.x) ids_l[p] = d.ids_in[p];
  }
  for (int g = tid; g < G; g += blockDim.x) {
    cnt[g] = 0;
    run[g] = 0;
  }
  for (int i = tid; i < 16 * G; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  for (int p = tid; p < S; p += blockDim.x) atomicAdd(&cnt[ids_l[p]], 1);
  __syncthreads();
  if (tid == 0 && d.shared) cnt[d.E] = d.T;
  __syncthreads();
  finalize_dispatch(d, cnt, scan_buf, flag_buf, tiles_buf, G, S + (d.shared ? d.T : 0));
  __syncthreads();
  // Stable scatter, 1024 slots per round.  scan_buf[g] is the next free
  // slot of group g; `run` collects this round's per-group totals.
  for (int base = 0; base < S; base += 1024) {
    int p = base + tid;
    bool valid = p < S;
    int e = valid ? ids_l[p] : 0;
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
__global__ void __launch_bounds__(256) k_dispatch_tiny(DispatchArgs d) {
  __shared__ int32_t ids_l[TINY_DISPATCH_SLOTS];
  __shared__ int32_t rk_l[TINY_DISPATCH_SLOTS];
  __shared__ float sc_l[TINY_SCORE_LDS];
  const int lane = threadIdx.x & 63;
  if (blockIdx.x != 0 || threadIdx.x >= 64) {
    quant_rows_waves(d.fq, (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6) - 1, (int)gridDim.x * 4 - 1,
                     lane);
    return;
  }
  const int G = d.E + d.shared;
  const int S = d.T * d.k;
  if (d.scores) {
    const int n = d.T * d.E;
    const float* src = d.scores;
    if (n <= TINY_SCORE_LDS) {
      // four loads in flight per lane and pass
      for (int i = lane; i < n; i += 256) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = i + 64 * u < n ? d.scores[i + 64 * u] : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
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
    const bool valid = p < S;
    const int e = valid ? ids_l[p] : 0;
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
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  const int excl = inc - cnt;
  const int total = __shfl(inc, 63, 64);
  if (lane < G) {
    d.counts[lane] = cnt;
    d.indptr[lane] = excl;
  }
  if (lane == 0) d.indptr[G] = total;
  // active list
  const uint64_t act = __ballot(lane < G && cnt > 0);
  if (lane < G && cnt > 0) d.active[__popcll(act & below)] = lane;
  // configuration from the histogram statistics (lane g holds group g)
  int mx = cnt, t32 = (cnt + 31) / 32;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int v = __shfl_xor(mx, o, 64);
    mx = v > mx ? v : mx;
    t32 += __shfl_xor(t32, o, 64);
  }
  int cfg = config_rule(mx, __popcll(act), total, t32, d.I, d.num_cfgs, d.cus);
  if (d.force_cfg >= 0) cfg = d.force_cfg;
  // block table for the chosen row-block height
  const int bm = cfg_rows(cfg);
  const int nt = lane < G ? (cnt + bm - 1) / bm : 0;
  int tinc = nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(tinc, o, 64);
    if (lane >= o) tinc += v;
  }
  for (int r = 0, b = tinc - nt; r < nt; ++r) {
    d.tiles[2 * (b + r)] = lane;
    d.tiles[2 * (b + r) + 1] = r * bm;
  }
  const int ntiles = __shfl(tinc, 63, 64);   // every lane takes part in the shuffle
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
    const bool valid = p < S;
    const int e = valid ? ids_l[p] : 0;
    const int slot = __shfl(excl, e, 64) + (valid ? rk_l[p] : 0);
    if (valid) {
      d.gather[slot] = p;
      d.inv[p] = slot;
    }
  }
  if (d.shared)
    for (int t = lane; t < d.T; t += 64) d.gather[S + t] = t * d.k;
}

// ---------------------------------------------------------------- large path
// 1) per-chunk histograms (1024 slots per chunk)
__global__ void __launch_bounds__(1024) k_dispatch_hist(DispatchArgs d) {
  extern __shared__ int32_t smem[];
  int32_t* cnt = smem;   // [E]
  int S = d.T * d.k, c = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < d.E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  int p = c * 1024 + tid;
  if (p < S) atomicAdd(&cnt[d.ids_in[p]], 1);
  __syncthreads();
  for (int e = tid; e < d.E; e += blockDim.x) d.chunk[(size_t)c * d.E + e] = cnt[e];
}

// 2) one block: chunk bases, group counts, scan, active list, config, table.
// The per-chunk counts are staged through LDS in coalesced passes of CG
// chunks, so no thread walks a chain of dependent global loads.
__global__ void __launch_bounds__(1024) k_dispatch_scan(DispatchArgs d) {
  extern __shared__ int32_t smem[];
  const int G = d.E + d.shared;
  int32_t* cnt = smem;
  int32_t* scan_buf = cnt + G;
  int32_t* flag_buf = scan_buf + G;
  int32_t* tiles_buf = flag_buf + G;
  int32_t* stage = tiles_buf + G;                 // [CG][E]
  const int CG = SCAN_STAGE_INTS / d.E;
  int S = d.T * d.k, nchunks = (S + 1023) / 1024, tid = threadIdx.x;
  int run = 0;
  for (int c0 = 0; c0 < nchunks; c0 += CG) {
    const int n = min(CG, nchunks - c0);
    for (int i = tid; i < n * d.E; i += blockDim.x) stage[i] = d.chunk[(size_t)c0 * d.E + i];
    __syncthreads();
    if (tid < d.E) {
      for (int c = 0; c < n; ++c) {
        const int v = stage[c * d.E + tid];
        d.chunk[(size_t)(c0 + c) * d.E + tid] = run;
        run += v;
      }
    }
    __syncthreads();
  }
  if (tid < d.E) cnt[tid] = run;
  if (tid == 0 && d.shared) cnt[d.E] = d.T;
  __syncthreads();
  finalize_dispatch(d, cnt, scan_buf, flag_buf, tiles_buf, G, S + (d.shared ? d.T : 0));
  if (d.shared)
    for (int t = tid; t < d.T; t += blockDim.x) d.gather[S + t] = t * d.k;
}

// 3) stable scatter of each chunk
__global__ void __launch_bounds__(1024) k_dispatch_scatter(DispatchArgs d) {
  extern __shared__ int32_t smem[];
  const int G = d.E;
  int32_t* wcnt = smem;  // [16*E]
  int S = d.T * d.k, c = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < 16 * G; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  int p = c * 1024 + tid;
  bool valid = p < S;
  int e = valid ? d.ids_in[p] : 0;
  int r = block_stable_rank(e, valid, wcnt, G, nullptr);
  if (valid) {
    int slot = d.indptr[e] + d.chunk[(size_t)c * d.E + e] + r;
    d.gather[slot] = p;
    d.inv[p] = slot;
  }
}

// ---------------------------------------------------------------- host launchers
size_t dispatch_small_lds(int T, int k, int G, int E, bool route) {
  return sizeof(int32_t) * ((size_t)T * k + 2 * G + 16 * G + 3 * G + (route ? (size_t)T * E : 0));
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
    hipLaunchKernelGGL(k_route_thread, dim3(rb + quant_blocks(fq, 4, 0)), dim3(256), 0, st, scores,
                       T, E, k, score_fn, ids, w, fq);
  } else {
    const int rb = (T + 3) / 4;
    hipLaunchKernelGGL(k_route, dim3(rb + quant_blocks(fq, 4, 0)), dim3(256), 0, st, scores, T, E, k,
                       score_fn, ids, w, fq);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& d, hipStream_t st) {
  const int G = d.E + d.shared;
  const int S = d.T * d.k;
  if (S <= TINY_DISPATCH_SLOTS && G <= 64 && (!d.scores || d.E <= SMALL_E_THREAD_ROUTE)) {
    const int grid = 1 + quant_blocks(d.fq, 4, 3);
    hipLaunchKernelGGL(k_dispatch_tiny, dim3(grid), dim3(256), 0, st, d);
    return hipGetLastError();
  }
  if (S <= SMALL_DISPATCH_SLOTS) {
    // routing is fused into the block when the scores fit in its LDS
    if (d.scores && dispatch_small_lds(d.T, d.k, G, d.E, true) > DISPATCH_LDS_MAX) {
      hipError_t e = launch_route(d.scores, d.T, d.E, d.k, d.score_fn, d.ids, d.w, d.fq, st);
      if (e != hipSuccess) return e;
      DispatchArgs d2 = d;
      d2.scores = nullptr;
      d2.ids_in = d.ids;
      d2.fq.R = 0;
      hipLaunchKernelGGL(k_dispatch_small, dim3(1), dim3(1024),
                         dispatch_small_lds(d.T, d.k, G, d.E, false), st, d2);
      return hipGetLastError();
    }
    const int grid = 1 + quant_blocks(d.fq, 16, 0);
    hipLaunchKernelGGL(k_dispatch_small, dim3(grid), dim3(1024),
                       dispatch_small_lds(d.T, d.k, G, d.E, d.scores != nullptr), st, d);
    return hipGetLastError();
  }
  // large path: routing (if requested, with the input quantisation) runs as
  // its own grid first
  DispatchArgs d2 = d;
  d2.fq.R = 0;
  if (d.scores) {
    hipError_t e = launch_route(d.scores, d.T, d.E, d.k, d.score_fn, d.ids, d.w, d.fq, st);
    if (e != hipSuccess) return e;
    d2.scores = nullptr;
    d2.ids_in = d.ids;
  } else if (d.fq.R > 0) {
    hipError_t e = launch_quant(d.fq, st);
    if (e != hipSuccess) return e;
  }
  int nchunks = (S + 1023) / 1024;
  hipLaunchKernelGGL(k_dispatch_hist, dim3(nchunks), dim3(1024), sizeof(int32_t) * d.E, st, d2);
  hipLaunchKernelGGL(k_dispatch_scan, dim3(1), dim3(1024),
                     sizeof(int32_t) * (4 * G + SCAN_STAGE_INTS), st, d2);
  hipLaunchKernelGGL(k_dispatch_scatter, dim3(nchunks), dim3(1024), sizeof(int32_t) * 16 * d.E, st,
                     d2);
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
