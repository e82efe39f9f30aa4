// Streaming grouped GEMM for decode-sized expert groups.
//
// When each expert holds few rows the projections are bound by reading the
// expert weights once from HBM.  Here every weight byte is loaded straight
// into MFMA operand registers (no LDS round trip), sixteen output channels
// per workgroup, with the contraction split across the workgroup's waves
// and reduced through LDS in a fixed order.  The token rows of the group
// (at most 16*MT per pass) are the MFMA B operand and come from L2.
//
// Gate/up op: both projections share the token fragments of each K step
// (pure-Triton MoE commentary, second paragraph: gate and up share the
// input tile), and SiLU(gate)*up is formed on the accumulators.
// Group g < E is routed expert g; group E is the shared expert.
#include "layer.h"

template <int F>
struct WScale {
  // per-K-step weight scale for 16 rows starting at n0 (block format)
  static DEVI float blk(const void* s, int N, int K, int n0, int kb) {
    return ((const float*)s)[(size_t)(n0 / 128) * (K / 128) + kb];
  }
};

// ACT: the gate/up epilogue's activation (ACT_*).  MT: 16-row token tiles
// per pass; U: K steps whose loads are issued together.  Groups of at most
// 16 rows (decode) run MT = 1, U = 2: the registers of the unused tiles and
// of deep load batches would cut the waves per SIMD, and at decode sizes
// more waves in flight move more bytes (Mixtral-shaped T=1 layer 97 ->
// 84 us) than deeper batches per wave.
template <int F, bool GATEUP, int WAVES, int MT, int ACT, int U, bool LOOP>
__global__ void __launch_bounds__(WAVES * 64) k_gemm_stream(GemmArgs p) {
  constexpr int WB = FmtBits<F>::W, XB = FmtBits<F>::X;
  constexpr int NW = GATEUP ? 2 : 1;
  // ReLU^2 has no gate projection: its loads and products are skipped
  constexpr bool GATE = !(GATEUP && ACT == ACT_RELU2);
  const int nblk = p.N >> 4;
  // one work item (active group gi, channel block nb) per pass: one
  // workgroup per item, or (LOOP) a capped grid whose workgroups stride the
  // items, so that a launch the device did not choose starts few
  // workgroups.  The first item is located before the configuration check,
  // so the argument loads it needs overlap the check's.
  unsigned item = blockIdx.x;
  int gi = (int)(item / (unsigned)nblk), nb = (int)item - gi * nblk;
  if (p.cfg_self >= 0 && p.meta[META_CFG] != p.cfg_self) return;
  const int nact = p.meta[META_NACTIVE];
  __shared__ f32x4 red[WAVES > 1 ? WAVES - 1 : 1][MT][NW][64];
  while (gi < nact) {
    const int g = p.active[gi];
    const int m0 = p.indptr[g], M = p.counts[g];
    const int lane = threadIdx.x & 63;
    // The wave index must be a scalar (SGPR) value: every branch that guards
    // an MFMA below depends on it, and MFMA ignores the EXEC mask, so those
    // branches have to be uniform scalar branches, never EXEC-masked ones.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, lg = lane >> 4;
    const int K = p.K, N = p.N;
    const long wrow = row_bytes<WB>(K), xrow = row_bytes<XB>(K);
    const bool sh = g >= p.E;
    const int n_ld = nb * 16 + r16;   // weight row this lane feeds to the MFMA
    const uint8_t* W0 = (sh ? p.sh_w0 : p.w0 + (size_t)g * N * wrow) + (size_t)n_ld * wrow;
    const uint8_t* W1 = GATEUP ? (sh ? p.sh_w1 : p.w1 + (size_t)g * N * wrow) + (size_t)n_ld * wrow
                               : nullptr;
    const void* S0 = sh ? p.sh_w0s : p.w0s;
    const void* S1 = sh ? p.sh_w1s : p.w1s;
    // per-expert offset of the scale tensors
    size_t s_off = 0;
    if (!sh) {
      if (F == F_FP8_CH) s_off = (size_t)g * N * 4;
      if (F == F_FP8_BLK) s_off = (size_t)g * (N / 128) * (K / 128) * 4;
      if (F == F_MX) s_off = (size_t)g * N * (K / 32);
    }
    S0 = (const uint8_t*)S0 + s_off;
    if (GATEUP) S1 = (const uint8_t*)S1 + s_off;

    const int Kw = K / WAVES;
    const int kbeg = wave * Kw, kend = kbeg + Kw;

    for (int c0 = 0; c0 < M; c0 += 16 * MT) {
      const int nsub = min(MT, (M - c0 + 15) >> 4);
      f32x4 acc[MT][NW];
      const uint8_t* xr[MT];
      int tok[MT];
      bool tv[MT];
  #pragma unroll
      for (int t = 0; t < MT; ++t) {
  #pragma unroll
        for (int j = 0; j < NW; ++j) acc[t][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        int r = c0 + 16 * t + r16;
        tv[t] = r < M;
        int slot = m0 + (tv[t] ? r : 0);
        int row = p.gather ? p.gather[slot] / p.gather_div : slot;
        tok[t] = row;
        xr[t] = p.a + (size_t)row * xrow;
      }
      for (int ks0 = kbeg; ks0 < kend; ks0 += 128 * U) {
        Frag<WB> a0[U], a1[U];
  #pragma unroll
        for (int u = 0; u < U; ++u) {
          int ks = ks0 + 128 * u;
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
        for (int t = 0; t < MT; ++t) {
          if (t >= nsub) break;
          Frag<XB> b[U];
  #pragma unroll
          for (int u = 0; u < U; ++u) {
            int ks = ks0 + 128 * u;
            if (ks < kend && tv[t]) b[u].load(xr[t], ks, lg);
            else b[u].zero();
          }
  #pragma unroll
          for (int u = 0; u < U; ++u) {
            int ks = ks0 + 128 * u;
            if (ks >= kend) break;
            if constexpr (F == F_FP8_BLK) {
              const int kb = ks >> 7;
              float sx = tv[t] ? ((const float*)p.a_scale)[(size_t)tok[t] * (K / 128) + kb] : 0.f;
              f32x4 z = {0.f, 0.f, 0.f, 0.f};
              if constexpr (GATE) {
                f32x4 d0 = mfma_f8(a0[u].v, b[u].v, z);
                float s0 = sx * WScale<F>::blk(S0, N, K, nb * 16, kb);
                acc[t][0] += d0 * s0;
              }
              if (GATEUP) {
                f32x4 d1 = mfma_f8(a1[u].v, b[u].v, z);
                float s1 = sx * WScale<F>::blk(S1, N, K, nb * 16, kb);
                acc[t][NW - 1] += d1 * s1;
              }
            } else if constexpr (F == F_MX) {
              const int kq = (ks >> 5) + lg;
              int sb = tv[t] ? ((const uint8_t*)p.a_scale)[(size_t)tok[t] * (K / 32) + kq] : 127;
              if constexpr (GATE) {
                int sa0 = ((const uint8_t*)S0)[(size_t)n_ld * (K / 32) + kq];
                acc[t][0] = mfma_f4f8_scaled(a0[u].v, b[u].v, acc[t][0], sa0, sb);
              }
              if (GATEUP) {
                int sa1 = ((const uint8_t*)S1)[(size_t)n_ld * (K / 32) + kq];
                acc[t][NW - 1] = mfma_f4f8_scaled(a1[u].v, b[u].v, acc[t][NW - 1], sa1, sb);
              }
            } else {
              if constexpr (GATE) acc[t][0] = mma_step(a0[u], b[u], acc[t][0]);
              if (GATEUP) acc[t][NW - 1] = mma_step(a1[u], b[u], acc[t][NW - 1]);
            }
          }
        }
      }
      // fixed-order reduction of the K partitions: wave 0 adds waves 1..W-1
      if (WAVES > 1) {
        if (wave > 0) {
  #pragma unroll
          for (int t = 0; t < MT; ++t)
  #pragma unroll
            for (int j = 0; j < NW; ++j)
              if (t < nsub) red[wave - 1][t][j][lane] = acc[t][j];
        }
        __syncthreads();
        if (wave == 0) {
          for (int w = 1; w < WAVES; ++w)
  #pragma unroll
            for (int t = 0; t < MT; ++t)
  #pragma unroll
              for (int j = 0; j < NW; ++j)
                if (t < nsub) acc[t][j] += red[w - 1][t][j][lane];
        }
      }
      if (wave == 0) {
  #pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t >= nsub || !tv[t]) continue;
          const int slot = m0 + c0 + 16 * t + r16;
          const int n0 = nb * 16 + 4 * lg;   // four output channels of this lane
          f32x4 v0 = acc[t][0], v1 = acc[t][NW - 1];
          if constexpr (F == F_FP8_CH) {
            float sx = ((const float*)p.a_scale)[tok[t]];
            f32x4 w0 = *(const f32x4*)((const float*)S0 + n0);
            v0 = v0 * sx * w0;
            if (GATEUP) {
              f32x4 w1 = *(const f32x4*)((const float*)S1 + n0);
              v1 = v1 * sx * w1;
            }
          }
          if (GATEUP) {
            f32x4 h;
  #pragma unroll
            for (int i = 0; i < 4; ++i)
              h[i] = gated_act<ACT>(p.act_limit, v0[i], v1[i]);
            if (F == F_BF16) {
              uint32_t lo = pack_bf16x2(h[0], h[1]);
              uint32_t hi = pack_bf16x2(h[2], h[3]);
              *(uint2*)((uint16_t*)p.out + (size_t)slot * N + n0) = make_uint2(lo, hi);
            } else {
              *(f32x4*)((float*)p.out + (size_t)slot * N + n0) = h;
            }
          } else {
            store_down(p, slot, n0, v0);
          }
        }
      }
      if (WAVES > 1) __syncthreads();
    }
    if (!LOOP) break;
    item += gridDim.x;
    gi = (int)(item / (unsigned)nblk);
    nb = (int)item - gi * nblk;
  }
}

template <int F, bool GATEUP, int ACT>
static hipError_t stream_waves_x(const GemmArgs& g, hipStream_t st) {
  const int steps = g.K / 128;
  const long items = (long)g.max_groups * (g.N / 16);
  dim3 grid((unsigned)(g.grid_cap > 0 && items > g.grid_cap ? g.grid_cap : items));
  if (grid.x == 0) return hipSuccess;
  const bool dec = g.max_group_rows <= DECODE_STREAM_TOKENS && steps % 4 == 0;
  if (grid.x < items) {
    if (dec)
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 4, 1, ACT, 2, true>), grid, dim3(256), 0, st, g);
    else if (steps % 4 == 0)
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 4, 4, ACT, 4, true>), grid, dim3(256), 0, st, g);
    else if (steps % 2 == 0)
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 2, 4, ACT, 4, true>), grid, dim3(128), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 1, 4, ACT, 4, true>), grid, dim3(64), 0, st, g);
  } else {
    if (dec)
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 4, 1, ACT, 2, false>), grid, dim3(256), 0, st, g);
    else if (steps % 4 == 0)
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 4, 4, ACT, 4, false>), grid, dim3(256), 0, st, g);
    else if (steps % 2 == 0)
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 2, 4, ACT, 4, false>), grid, dim3(128), 0, st, g);
    else
      hipLaunchKernelGGL((k_gemm_stream<F, GATEUP, 1, 4, ACT, 4, false>), grid, dim3(64), 0, st, g);
  }
  return hipGetLastError();
}

template <int F, bool GATEUP>
static hipError_t stream_waves(const GemmArgs& g, hipStream_t st) {
  if constexpr (GATEUP) {
    return with_act(g.act, [&](auto a) { return stream_waves_x<F, true, decltype(a)::value>(g, st); });
  } else {
    return stream_waves_x<F, false, ACT_SWIGLU>(g, st);
  }
}

hipError_t launch_gemm_stream(int fmt, bool gateup, const GemmArgs& g, hipStream_t st) {
  switch (fmt) {
    case F_BF16: return gateup ? stream_waves<F_BF16, true>(g, st) : stream_waves<F_BF16, false>(g, st);
    case F_FP8_CH: return gateup ? stream_waves<F_FP8_CH, true>(g, st) : stream_waves<F_FP8_CH, false>(g, st);
    case F_FP8_BLK: return gateup ? stream_waves<F_FP8_BLK, true>(g, st) : stream_waves<F_FP8_BLK, false>(g, st);
    case F_MX: return gateup ? stream_waves<F_MX, true>(g, st) : stream_waves<F_MX, false>(g, st);
  }
  return hipErrorInvalidValue;
}
