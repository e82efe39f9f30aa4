// The whole MoE layer in one launch for decode batches (at most 16 tokens):
// routing, dispatch, input quantisation, the fused gate/up grouped GEMM with
// its activation, the intermediate's requantisation, the down grouped GEMM
// and the weighted combine (Alpha-MoE news page, "How the megakernel works":
// the layer's stages in one persistent kernel, so the small stages cost no
// launches of their own).
//
// Every workgroup first routes the batch itself (a few hundred scores at
// most) and keeps the dispatch tables in LDS, so no workgroup waits for
// another before streaming weights.  The activations are quantised while
// they are loaded as MFMA operands, with the quantiser's own arithmetic (the
// codes equal those of the separate pass bit for bit).  One grid barrier
// separates the projections: the per-token scale of the intermediate needs
// the maximum over all its channels, which the gate/up workgroups reduce by
// device-wide atomic maxima.  The combine runs in the down phase: the last
// workgroup to store a (token, 16-channel block) of slot rows sums them in
// the fixed order j = 0..k-1, then the shared expert.
//
// The persistent grid holds only as many workgroups as can be resident at
// once, and the barrier's wait is bounded: a launch that could not make all
// workgroups resident sets the device status word and returns instead of
// waiting for ever.
#include "layer.h"
#include "quant_row.h"
#include "route.h"
#include "onthefly.h"

namespace {

constexpr int DL_THREADS = 256;            // four waves per workgroup
constexpr int DL_MAX_SLOTS = DECODE_STREAM_TOKENS * 16;
constexpr int DL_MAX_GROUPS = 257;

// Arrival at the grid barrier of this launch.  Every thread's earlier global
// stores are released before its workgroup arrives, and every thread
// acquires after the barrier.  The arrival count returns to 0 with each
// completed barrier, and the generation word counts completed barriers.
DEVI bool grid_barrier(int32_t* bar, int nblocks, long spin_limit) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  __shared__ int ok_l;
  if (threadIdx.x == 0) {
    const int gen = __hip_atomic_load(bar + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    const int old = __hip_atomic_fetch_add(bar, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    if (old == nblocks - 1) {
      __hip_atomic_store(bar, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(bar + 1, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      long n = 0;
      while (__hip_atomic_load(bar + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(2);
        if (++n > spin_limit) {
          ok = 0;
          break;
        }
      }
    }
    ok_l = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok_l != 0;
}



// One projection item: 16 output channels (weight rows n0 .. n0+15 of group
// g) for the group's rows (at most 16).  The four waves split K; wave 0
// holds the fixed-order sum.  GATEUP: both matrices, activation in the
// epilogue, h stored (fp32, or bf16 for the bf16 format) with the per-row
// maxima reduced for per-token scales; otherwise the weighted bf16 slot row.
template <int F, bool GATEUP, int ACT>
struct DecodeItem {
  static constexpr int WB = FmtBits<F>::W;
  static DEVI void run(const DecodeArgs& a, int g, int nb, int m0, int M, const int32_t* gat_l,
                       const float* w_l, float rowscale, f32x4 (*red)[2][64], uint32_t* amax_p,
                       int lane, int wave) {
    const int r16 = lane & 15, lg = lane >> 4;
    const bool sh = g >= a.E;
    const int N = GATEUP ? a.I : a.H, K = GATEUP ? a.H : a.I;
    const long wrow = row_bytes<WB>(K);
    const int n_ld = nb * 16 + r16;
    const uint8_t* wb0 = GATEUP ? (sh ? a.shg : a.wg) : (sh ? a.shd : a.wd);
    const uint8_t* wb1 = GATEUP ? (sh ? a.shu : a.wu) : nullptr;
    const void* s0 = GATEUP ? (sh ? a.ssg : a.sg) : (sh ? a.ssd : a.sd);
    const void* s1 = GATEUP ? (sh ? a.ssu : a.su) : nullptr;
    const size_t ge = sh ? 0 : (size_t)g;
    const uint8_t* W0 = wb0 + ge * N * wrow + (size_t)n_ld * wrow;
    const uint8_t* W1 = GATEUP ? wb1 + ge * N * wrow + (size_t)n_ld * wrow : nullptr;
    size_t s_off = 0;
    if (F == F_FP8_CH) s_off = ge * N * 4;
    if (F == F_FP8_BLK) s_off = ge * (N / 128) * (K / 128) * 4;
    if (F == F_MX) s_off = ge * N * (K / 32);
    s0 = (const uint8_t*)s0 + s_off;
    if (GATEUP) s1 = (const uint8_t*)s1 + s_off;
    constexpr bool GATE = !(GATEUP && ACT == ACT_RELU2);

    const bool tv = r16 < M;
    const int slot = m0 + (tv ? r16 : 0);
    const int flat = gat_l[slot];
    const int tok = slot < a.T * a.k ? flat / a.k : slot - a.T * a.k;
    // operand row: the token's bf16 x (gate/up) or the slot's intermediate (down)
    const void* brow = GATEUP ? (const void*)(a.x + (size_t)tok * a.H)
                              : (F == F_BF16 ? (const void*)((const uint16_t*)a.h + (size_t)slot * a.I)
                                             : (const void*)(a.h + (size_t)slot * a.I));
    constexpr bool BIN16 = GATEUP || F == F_BF16;   // operand rows stored as bf16

    const int Kw = K / 4, kbeg = wave * Kw, kend = kbeg + Kw;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int ks0 = kbeg; ks0 < kend; ks0 += 256) {
      Frag<WB> a0[2], a1[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ks = ks0 + 128 * u;
        if (ks < kend) {
          if (GATE) a0[u].load(W0, ks, lg);
          else a0[u].zero();
          if (GATEUP) a1[u].load(W1, ks, lg);
        } else {
          a0[u].zero();
          if (GATEUP) a1[u].zero();
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ks = ks0 + 128 * u;
        if (ks >= kend) break;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if constexpr (F == F_BF16) {
          Frag<16> b;
          if (tv) b.load((const uint8_t*)brow, ks, lg);
          else b.zero();
          if constexpr (GATE) acc0 = mma_step(a0[u], b, acc0);
          if (GATEUP) acc1 = mma_step(a1[u], b, acc1);
        } else {
          float v[32];
          if (tv) load_step32<BIN16>(brow, ks, lg, v);
          else
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = 0.f;
          if constexpr (F == F_FP8_CH) {
            const i32x8 b = tv ? codes_fp8(v, rowscale) : zero8();
            if constexpr (GATE) acc0 = mfma_f8(a0[u].v, b, acc0);
            if (GATEUP) acc1 = mfma_f8(a1[u].v, b, acc1);
          } else if constexpr (F == F_FP8_BLK) {
            // the 1x128 group is this step: its maximum over the four lane groups
            float m = amax32(v);
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            const float sq = qr_scale(m);
            const float sx = tv ? sq : 0.f;
            const i32x8 b = tv ? codes_fp8(v, sq) : zero8();
            // the 128x128 weight block of these 16 rows and this K step
            const size_t wblk = (size_t)(nb * 16 / 128) * (K / 128) + (ks >> 7);
            if constexpr (GATE) {
              const f32x4 d0 = mfma_f8(a0[u].v, b, z);
              acc0 += d0 * (sx * ((const float*)s0)[wblk]);
            }
            if (GATEUP) {
              const f32x4 d1 = mfma_f8(a1[u].v, b, z);
              acc1 += d1 * (sx * ((const float*)s1)[wblk]);
            }
          } else {   // F_MX
            int sb;
            const i32x8 b = codes_mx(v, lane, sb);
            const int kq = (ks >> 5) + lg;
            if (!tv) sb = 127;
            if constexpr (GATE) {
              const int sa0 = ((const uint8_t*)s0)[(size_t)n_ld * (K / 32) + kq];
              acc0 = mfma_f4f8_scaled(a0[u].v, tv ? b : zero8(), acc0, sa0, sb);
            }
            if (GATEUP) {
              const int sa1 = ((const uint8_t*)s1)[(size_t)n_ld * (K / 32) + kq];
              acc1 = mfma_f4f8_scaled(a1[u].v, tv ? b : zero8(), acc1, sa1, sb);
            }
          }
        }
      }
    }
    // fixed-order reduction of the K quarters: wave 0 adds waves 1, 2, 3
    if (wave > 0) {
      red[wave - 1][0][lane] = acc0;
      if (GATEUP) red[wave - 1][1][lane] = acc1;
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < 4; ++w) {
        acc0 += red[w - 1][0][lane];
        if (GATEUP) acc1 += red[w - 1][1][lane];
      }
      if (tv) {
        const int n0 = nb * 16 + 4 * lg;   // four output channels of this lane
        f32x4 v0 = acc0, v1 = acc1;
        if constexpr (F == F_FP8_CH) {
          const f32x4 ws0 = *(const f32x4*)((const float*)s0 + n0);
          v0 = v0 * rowscale * ws0;
          if (GATEUP) {
            const f32x4 ws1 = *(const f32x4*)((const float*)s1 + n0);
            v1 = v1 * rowscale * ws1;
          }
        }
        if constexpr (GATEUP) {
          f32x4 h;
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = gated_act<ACT>(a.act_limit, v0[i], v1[i]);
          if constexpr (F == F_BF16) {
            const uint32_t lo = pack_bf16x2(h[0], h[1]);
            const uint32_t hi = pack_bf16x2(h[2], h[3]);
            *(uint2*)((uint16_t*)a.h + (size_t)slot * a.I + n0) = make_uint2(lo, hi);
          } else {
            *(f32x4*)(a.h + (size_t)slot * a.I + n0) = h;
          }
          if constexpr (F == F_FP8_CH) {
            // this item's share of the row maximum (non-negative floats
            // order as their bit patterns)
            float m = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (lg == 0)
              __hip_atomic_fetch_max(amax_p + slot, __float_as_uint(m), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          const float w = slot < a.T * a.k ? w_l[flat] : 1.0f;
          const f32x4 vw = v0 * w;
          const uint32_t lo = pack_bf16x2(vw[0], vw[1]);
          const uint32_t hi = pack_bf16x2(vw[2], vw[3]);
          *(uint2*)(a.out_slot + (size_t)slot * a.H + n0) = make_uint2(lo, hi);
        }
      }
    }
    __syncthreads();   // red is reused by the next item
  }
};

}  // namespace

template <int F, int ACT>
__global__ void __launch_bounds__(DL_THREADS) k_decode_layer(DecodeArgs a) {
  __shared__ int32_t ids_l[DL_MAX_SLOTS];
  __shared__ float w_l[DL_MAX_SLOTS];
  __shared__ int32_t cnt_l[DL_MAX_GROUPS];
  __shared__ int32_t ind_l[DL_MAX_GROUPS + 1];
  __shared__ int32_t act_l[DL_MAX_GROUPS];
  __shared__ int32_t gat_l[DL_MAX_SLOTS + DECODE_STREAM_TOKENS];
  __shared__ int32_t inv_l[DL_MAX_SLOTS];
  __shared__ float xsc_l[4][16];
  __shared__ f32x4 red[3][2][64];
  __shared__ int32_t nact_l, gen_l;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, E = a.E, k = a.k, S = T * k;
  const int G = E + a.shared, S_tot = S + (a.shared ? T : 0);

  // ---------------------------------------------------------------- routing
  if (tid == 0) gen_l = __hip_atomic_load(a.bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  {
    const int t = wave * 4 + (lane >> 4);   // one 16-lane row per token
    const bool tv = t < T;
    route_row16(a.scores + (size_t)(tv ? t : 0) * E, tv, E, k, a.score_fn, lane & 15,
                ids_l + (tv ? t : 0) * k, w_l + (tv ? t : 0) * k, nullptr);
  }
  for (int g = tid; g < G; g += DL_THREADS) cnt_l[g] = 0;
  __syncthreads();
  for (int p = tid; p < S; p += DL_THREADS) atomicAdd(&cnt_l[ids_l[p]], 1);
  __syncthreads();
  if (tid == 0 && a.shared) cnt_l[E] = T;
  __syncthreads();
  if (wave == 0) {
    // offsets and the active list: five groups per lane, one wave scan each
    int c[5], f[5], cs = 0, fs = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int gg = lane * 5 + i;
      c[i] = gg < G ? cnt_l[gg] : 0;
      f[i] = c[i] > 0;
      cs += c[i];
      fs += f[i];
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
    if (lane == 0) {
      ind_l[G] = tot;
      nact_l = nact;
    }
  }
  __syncthreads();
  // stable placement: slot order is expert, then flat index t*k+j
  for (int p = tid; p < S; p += DL_THREADS) {
    const int e = ids_l[p];
    int r = 0;
    for (int q = 0; q < p; ++q) r += ids_l[q] == e;
    const int slot = ind_l[e] + r;
    gat_l[slot] = p;
    inv_l[p] = slot;
  }
  if (a.shared)
    for (int t = tid; t < T; t += DL_THREADS) gat_l[S + t] = t * k;
  __syncthreads();
  const int nact = nact_l, par = gen_l & 1;
  uint32_t* amax_p = a.amax + (size_t)par * a.amax_stride;
  int32_t* cnt_p = a.cnt + (size_t)par * a.cnt_stride;
  if (blockIdx.x == 0) {
    // the routing results for the caller, and the other parity's words
    // cleared for the next launch
    for (int p = tid; p < S; p += DL_THREADS) {
      a.ids[p] = ids_l[p];
      a.w[p] = w_l[p];
      a.inv[p] = inv_l[p];
    }
    for (int s = tid; s < S_tot; s += DL_THREADS) a.gather[s] = gat_l[s];
    for (int g = tid; g < G; g += DL_THREADS) {
      a.counts[g] = cnt_l[g];
      a.indptr[g] = ind_l[g];
    }
    if (tid == 0) {
      a.indptr[G] = ind_l[G];
      a.meta[META_NACTIVE] = nact;
      a.meta[META_NTILES] = 0;
      a.meta[META_CFG] = 0;
      a.meta[META_ROWS] = S_tot;
      a.meta[META_BM] = 0;
      a.meta[META_ERROR] = 0;
    }
    uint32_t* amax_n = a.amax + (size_t)(par ^ 1) * a.amax_stride;
    int32_t* cnt_n = a.cnt + (size_t)(par ^ 1) * a.cnt_stride;
    for (int i = tid; i < a.amax_stride; i += DL_THREADS) amax_n[i] = 0;
    for (int i = tid; i < a.cnt_stride; i += DL_THREADS) cnt_n[i] = 0;
  }

  // ---------------------------------------------------------------- gate/up
  const int r16 = lane & 15;
  {
    const int nbI = a.I / 16, nI = nact * nbI;
    for (int item = blockIdx.x; item < nI; item += gridDim.x) {
      const int gi = item / nbI, nb = item - gi * nbI;
      const int g = act_l[gi], m0 = ind_l[g], M = cnt_l[g];
      float rowscale = 0.f;
      if constexpr (F == F_FP8_CH) {
        // per-token scale of the row: maximum over the four K quarters
        const bool tv = r16 < M;
        const int slot = m0 + (tv ? r16 : 0);
        const int tok = slot < S ? gat_l[slot] / k : slot - S;
        const int Kw = a.H / 4, kbeg = wave * Kw;
        float m = 0.f;
        if (tv)
          for (int ks = kbeg; ks < kbeg + Kw; ks += 128) {
            float v[32];
            load_step32<true>(a.x + (size_t)tok * a.H, ks, lane >> 4, v);
            m = fmaxf(m, amax32(v));
          }
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (lane < 16) xsc_l[wave][lane] = m;
        __syncthreads();
        const float mm = fmaxf(fmaxf(xsc_l[0][r16], xsc_l[1][r16]), fmaxf(xsc_l[2][r16], xsc_l[3][r16]));
        rowscale = qr_scale(mm);
        __syncthreads();
      }
      DecodeItem<F, true, ACT>::run(a, g, nb, m0, M, gat_l, w_l, rowscale, red, amax_p, lane, wave);
    }
  }

  if (!grid_barrier(a.bar, gridDim.x, a.spin_limit)) {
    if (tid == 0) a.meta[META_ERROR] = 2;
    return;
  }

  // ---------------------------------------------------------------- down + combine
  {
    const int nbH = a.H / 16, nH = nact * nbH;
    const int kt = k + (a.shared ? 1 : 0);
    for (int item = blockIdx.x; item < nH; item += gridDim.x) {
      const int gi = item / nbH, nb = item - gi * nbH;
      const int g = act_l[gi], m0 = ind_l[g], M = cnt_l[g];
      float rowscale = 0.f;
      if constexpr (F == F_FP8_CH) {
        const int slot = m0 + (r16 < M ? r16 : 0);
        rowscale = qr_scale(__uint_as_float(__hip_atomic_load(amax_p + slot, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_AGENT)));
      }
      DecodeItem<F, false, ACT>::run(a, g, nb, m0, M, gat_l, w_l, rowscale, red, amax_p, lane, wave);
      // the last workgroup to store a token's rows of this channel block sums
      // them (j ascending, then the shared expert) into y
      if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane < M) {
          const int slot = m0 + lane;
          const int tok = slot < S ? gat_l[slot] / k : slot - S;
          const int old = __hip_atomic_fetch_add(cnt_p + (size_t)tok * nbH + nb, 1, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
          if (old == kt - 1) {
            float acc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
            for (int j = 0; j < kt; ++j) {
              const int s2 = j < k ? inv_l[tok * k + j] : S + tok;
              const uint4* src = (const uint4*)(a.out_slot + (size_t)s2 * a.H + nb * 16);
              const uint4 q0 = src[0], q1 = src[1];
              const uint32_t wv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                acc[2 * i] += __uint_as_float(wv[i] << 16);
                acc[2 * i + 1] += __uint_as_float(wv[i] & 0xFFFF0000u);
              }
            }
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
              o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
            uint4* dst = (uint4*)(a.y + (size_t)tok * a.H + nb * 16);
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
          }
        }
      }
    }
  }
}

namespace {

template <int F, int ACT>
hipError_t launch_dl(const DecodeArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_layer<F, ACT>), dim3(grid), dim3(DL_THREADS), 0, st, a);
  return hipGetLastError();
}

template <int F>
hipError_t launch_dl_f(const DecodeArgs& a, int grid, hipStream_t st) {
  return with_act(a.act, [&](auto c) { return launch_dl<F, decltype(c)::value>(a, grid, st); });
}

template <int F, int ACT>
int resident_blocks() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)k_decode_layer<F, ACT>, DL_THREADS, 0) !=
      hipSuccess)
    return 0;
  return n;
}

}  // namespace

int decode_layer_grid(int fmt, int act, int cus) {
  int per = 0;
  auto pick = [&](auto fc) {
    constexpr int F = decltype(fc)::value;
    per = with_act(act, [&](auto c) { return resident_blocks<F, decltype(c)::value>(); });
  };
  switch (fmt) {
    case F_BF16: pick(std::integral_constant<int, F_BF16>{}); break;
    case F_FP8_CH: pick(std::integral_constant<int, F_FP8_CH>{}); break;
    case F_FP8_BLK: pick(std::integral_constant<int, F_FP8_BLK>{}); break;
    case F_MX: pick(std::integral_constant<int, F_MX>{}); break;
    default: return 0;
  }
  if (per <= 0) return 0;
  // every workgroup must be resident at once (the grid barrier); four per
  // compute unit keep sixteen waves streaming weights on each
  if (per > 4) per = 4;
  return per * cus;
}

hipError_t launch_decode_layer(int fmt, const DecodeArgs& a, int grid, hipStream_t st) {
  switch (fmt) {
    case F_BF16: return launch_dl_f<F_BF16>(a, grid, st);
    case F_FP8_CH: return launch_dl_f<F_FP8_CH>(a, grid, st);
    case F_FP8_BLK: return launch_dl_f<F_FP8_BLK>(a, grid, st);
    case F_MX: return launch_dl_f<F_MX>(a, grid, st);
  }
  return hipErrorInvalidValue;
}
