// Tiled grouped GEMM for expert groups with many rows.
//
// One work item = (row block of one expert group from the block table, block
// of output channels).  The block table maps a flat work index to (expert,
// row offset) so that every group, whatever its size, is covered by one
// launch without padding rows to a common size (pure-Triton MoE commentary,
// second paragraph).  A persistent grid walks the items.
//
// Data movement per K step of 128 elements:
//  * the BM token rows of the block (gathered through the dispatch
//    permutation for the first projection) are staged in LDS once per
//    workgroup, double-buffered, and read by all four waves as MFMA B
//    fragments; rows are padded by 16 bytes so the fragment reads are free of
//    bank conflicts;
//  * each wave owns RTW 16-row tiles of every weight matrix (gate and up for
//    the fused op) and loads them straight from HBM into MFMA A operand
//    registers, one K step ahead of the MFMAs (register double buffer).
// Gate/up op: SwiGLU on the accumulators, then the intermediate is written
// in the activation format: bf16; fp32 staging for per-token scales (their
// amax spans every channel block); FP8 with a 1x128 scale computed across the
// four waves through LDS; MXFP8 with an e8m0 scale per 32 channels (within
// one wave).  Block-scaled FP8 applies the 128x128 weight scale times the
// 1x128 token scale to each K step's MFMA result before accumulating.
#include "layer.h"

namespace {

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;

template <int F>
struct TileFmt {
  static constexpr int XB = FmtBits<F>::X, WB = FmtBits<F>::W;
  static constexpr int XSTEP = 128 * XB / 8;          // token bytes per K step
  static constexpr int XPITCH = XSTEP + 16;            // padded LDS row pitch
};

template <int F, int BM>
struct Lds {
  static constexpr int TOK = BM * TileFmt<F>::XPITCH;   // one token buffer
  static constexpr int SCL = (F == F_FP8_BLK) ? BM * 4 : (F == F_MX ? BM * 4 : 0);
  static constexpr int BUF = TOK + SCL;
  static constexpr int TOTAL = 2 * BUF + 4 * BM * 4;    // + cross-wave amax [4][BM]
};

}  // namespace

// ACT: the gate/up epilogue's activation (ACT_*).
template <int F, bool GATEUP, int BM, int RTW, int ACT>
__global__ void __launch_bounds__(THREADS) k_gemm_tiled(GemmArgs p) {
  using TF = TileFmt<F>;
  constexpr int XB = TF::XB, WB = TF::WB;
  constexpr int XSTEP = TF::XSTEP, XPITCH = TF::XPITCH;
  constexpr int TT = BM / 16;                 // token tiles
  constexpr int NM = GATEUP ? 2 : 1;          // weight matrices
  constexpr int NBR = WAVES * RTW * 16;       // output channels per item
  constexpr int CHUNKS = BM * XSTEP / 16;     // 16-byte token chunks per K step
  constexpr int CPT = (CHUNKS + THREADS - 1) / THREADS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[Lds<F, BM>::TOTAL];

  if (p.cfg_self >= 0 && p.meta[META_CFG] != p.cfg_self) return;
  const int ntiles = p.meta[META_NTILES];
  const int N = p.N, K = p.K;
  const int nblk = N / NBR;
  const int n_items = ntiles * nblk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, lg = lane >> 4;
  const long wrow = row_bytes<WB>(K), xrow = row_bytes<XB>(K);
  const int nsteps = K / 128;
  float* amax_l = (float*)(lds + 2 * Lds<F, BM>::BUF);

  const ItemRange ir = xcd_items(n_items);
  for (int item = ir.begin; item < ir.end; item += ir.step) {
    const int tile = item / nblk, nb = item - tile * nblk;
    const int g = p.tiles[2 * tile], r0 = p.tiles[2 * tile + 1];
    const int m0 = p.indptr[g] + r0;
    const int M = min(BM, p.counts[g] - r0);
    const bool sh = g >= p.E;
    const int nw0 = nb * NBR + wave * RTW * 16;   // first channel of this wave
    // weight row pointers of this lane (row r16 of each row tile)
    const uint8_t* wbase[NM];
    {
      const uint8_t* b0 = sh ? p.sh_w0 : p.w0 + (size_t)g * N * wrow;
      wbase[0] = b0 + (size_t)(nw0 + r16) * wrow;
      if (GATEUP) {
        const uint8_t* b1 = sh ? p.sh_w1 : p.w1 + (size_t)g * N * wrow;
        wbase[NM - 1] = b1 + (size_t)(nw0 + r16) * wrow;
      }
    }
    const void* S[NM];
    {
      size_t s_off = 0;
      if (!sh) {
        if (F == F_FP8_CH) s_off = (size_t)g * N * 4;
        if (F == F_FP8_BLK) s_off = (size_t)g * (N / 128) * (K / 128) * 4;
        if (F == F_MX) s_off = (size_t)g * N * (K / 32);
      }
      S[0] = (const uint8_t*)(sh ? p.sh_w0s : p.w0s) + s_off;
      if (GATEUP) S[NM - 1] = (const uint8_t*)(sh ? p.sh_w1s : p.w1s) + s_off;
    }
    // token source rows for this thread's staging chunks
    const uint8_t* src[CPT];
    int srow[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      int ch = tid + c * THREADS;
      int row = ch / (XSTEP / 16);
      srow[c] = -1;
      src[c] = nullptr;
      if (ch < CHUNKS && row < M) {
        int slot = m0 + row;
        int r = p.gather ? p.gather[slot] / p.gather_div : slot;
        srow[c] = r;
        src[c] = p.a + (size_t)r * xrow + (ch % (XSTEP / 16)) * 16;
      }
    }
    // scale rows for this thread (threads < BM stage one token's scales)
    int sc_row = -1;
    if ((F == F_FP8_BLK || F == F_MX) && tid < BM && tid < M) {
      int slot = m0 + tid;
      sc_row = p.gather ? p.gather[slot] / p.gather_div : slot;
    }

    auto stage_load = [&](int s, i32x4 (&reg)[CPT], uint32_t& sreg) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        if (srow[c] >= 0) reg[c] = *(const i32x4*)(src[c] + (size_t)s * XSTEP);
        else reg[c] = (i32x4){0, 0, 0, 0};
      }
      if constexpr (F == F_FP8_BLK) {
        sreg = sc_row >= 0 ? __float_as_uint(((const float*)p.a_scale)[(size_t)sc_row * (K / 128) + s])
                           : 0u;
      } else if constexpr (F == F_MX) {
        sreg = sc_row >= 0 ? *(const uint32_t*)((const uint8_t*)p.a_scale + (size_t)sc_row * (K / 32) + 4 * s)
                           : 0x7F7F7F7Fu;
      }
    };
    auto stage_store = [&](int buf, const i32x4 (&reg)[CPT], uint32_t sreg) {
      uint8_t* tb = lds + buf * Lds<F, BM>::BUF;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        int ch = tid + c * THREADS;
        if (ch < CHUNKS) {
          int row = ch / (XSTEP / 16), col = ch % (XSTEP / 16);
          *(i32x4*)(tb + row * XPITCH + col * 16) = reg[c];
        }
      }
      if constexpr (F == F_FP8_BLK || F == F_MX) {
        if (tid < BM) ((uint32_t*)(tb + Lds<F, BM>::TOK))[tid] = sreg;
      }
    };
    auto wload = [&](int s, Frag<WB> (&wf)[NM][RTW]) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) wf[m][rt].load(wbase[m] + (size_t)rt * 16 * wrow, s * 128, lg);
    };

    f32x4 acc[NM][RTW][TT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[m][rt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    i32x4 treg[CPT];
    uint32_t sreg = 0;
    Frag<WB> wfa[NM][RTW], wfb[NM][RTW];
    stage_load(0, treg, sreg);
    wload(0, wfa);
    stage_store(0, treg, sreg);
    __syncthreads();

    // One K step: prefetch step s+1 (tokens into registers, weights into
    // the other register buffer), run the MFMAs of step s from LDS buffer
    // s&1, then publish the prefetched tokens into the other LDS buffer.
    auto kstep = [&](int s, Frag<WB> (&wcur)[NM][RTW], Frag<WB> (&wnext)[NM][RTW]) {
      const int cur = s & 1;
      const bool more = s + 1 < nsteps;
      if (more) {
        stage_load(s + 1, treg, sreg);
        wload(s + 1, wnext);
      }
      const uint8_t* tb = lds + cur * Lds<F, BM>::BUF;
      float wsc[NM];
      if constexpr (F == F_FP8_BLK) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
          wsc[m] = ((const float*)S[m])[(size_t)(nw0 / 128) * (K / 128) + s];
      }
      int wmx[NM][RTW];
      if constexpr (F == F_MX) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt)
            wmx[m][rt] = ((const uint8_t*)S[m])[(size_t)(nw0 + rt * 16 + r16) * (K / 32) + 4 * s + lg];
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        Frag<XB> b;
        const uint8_t* trow = tb + (t * 16 + r16) * XPITCH;
        if constexpr (XB == 8) {
          const i32x4 lo = *(const i32x4*)(trow + 16 * lg);
          const i32x4 hi = *(const i32x4*)(trow + 64 + 16 * lg);
          b.v = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) b.v[q] = *(const bf16x8*)(trow + 2 * (32 * q + 8 * lg));
        }
        if constexpr (F == F_FP8_BLK) {
          const float sx = ((const float*)(tb + Lds<F, BM>::TOK))[t * 16 + r16];
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const float sc = sx * wsc[m];
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
              f32x4 d = mfma_f8(wcur[m][rt].v, b.v, (f32x4){0.f, 0.f, 0.f, 0.f});
              acc[m][rt][t] += d * sc;
            }
          }
        } else if constexpr (F == F_MX) {
          const int sb = (tb + Lds<F, BM>::TOK)[(t * 16 + r16) * 4 + lg];
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
              acc[m][rt][t] = mfma_f4f8_scaled(wcur[m][rt].v, b.v, acc[m][rt][t], wmx[m][rt], sb);
        } else {
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) acc[m][rt][t] = mma_step(wcur[m][rt], b, acc[m][rt][t]);
        }
      }
      if (more) stage_store(cur ^ 1, treg, sreg);
      __syncthreads();
    };
    for (int s = 0; s < nsteps; s += 2) {
      kstep(s, wfa, wfb);
      if (s + 1 < nsteps) kstep(s + 1, wfb, wfa);
    }

    // ------------------------------------------------------------ epilogue
    // lane holds channels nw0 + rt*16 + 4*lg + i for token row t*16 + r16
    int tok[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      int r = t * 16 + r16;
      int slot = m0 + (r < M ? r : 0);
      tok[t] = p.gather ? p.gather[slot] / p.gather_div : slot;
    }
    if constexpr (F == F_FP8_CH) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sx = ((const float*)p.a_scale)[tok[t]];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) {
            f32x4 wsv = *(const f32x4*)((const float*)S[m] + nw0 + rt * 16 + 4 * lg);
            acc[m][rt][t] = acc[m][rt][t] * sx * wsv;
          }
      }
    }
    if constexpr (!GATEUP) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int r = t * 16 + r16;
        if (r >= M) continue;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) store_down(p, m0 + r, nw0 + rt * 16 + 4 * lg, acc[0][rt][t]);
      }
    } else {
      // h = act(gate, up), in place in acc[0]
      if constexpr (ACT == ACT_SWIGLU) {
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[0][rt][t][i] = silu(acc[0][rt][t][i]) * acc[1][rt][t][i];
      } else {
        const float L = p.act_limit;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[0][rt][t][i] = gated_act<ACT>(L, acc[0][rt][t][i], acc[1][rt][t][i]);
      }
      if constexpr (F == F_BF16) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = t * 16 + r16;
          if (r >= M) continue;
          uint16_t* orow = (uint16_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) {
            f32x4 h = acc[0][rt][t];
            uint32_t lo = pack_bf16x2(h[0], h[1]);
            uint32_t hi = pack_bf16x2(h[2], h[3]);
            *(uint2*)(orow + nw0 + rt * 16 + 4 * lg) = make_uint2(lo, hi);
          }
        }
      } else if constexpr (F == F_FP8_CH) {
        // per-token scales span every channel block: stage fp32 for the
        // requantisation pass
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = t * 16 + r16;
          if (r >= M) continue;
          float* orow = (float*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) *(f32x4*)(orow + nw0 + rt * 16 + 4 * lg) = acc[0][rt][t];
        }
      } else if constexpr (F == F_FP8_BLK) {
        // 1x128 groups: the item's 128 channels (NBR == 128) across 4 waves
        static_assert(!GATEUP || F != F_FP8_BLK || NBR == 128, "block-scaled gate/up needs 128 channels");
        float pm[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          float m = 0.f;
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[0][rt][t][i]));
          m = fmaxf(m, __shfl_xor(m, 16, 64));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          pm[t] = m;
        }
        if (lg == 0) {
#pragma unroll
          for (int t = 0; t < TT; ++t) amax_l[wave * BM + t * 16 + r16] = pm[t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = t * 16 + r16;
          float a = fmaxf(fmaxf(amax_l[r], amax_l[BM + r]), fmaxf(amax_l[2 * BM + r], amax_l[3 * BM + r]));
          float sc = a > 0.f ? a / 448.0f : 1.0f;
          if (r < M) {
            uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
              f32x4 h = acc[0][rt][t];
              *(uint32_t*)(orow + nw0 + rt * 16 + 4 * lg) = cvt4_e4m3(h[0] / sc, h[1] / sc, h[2] / sc, h[3] / sc);
            }
            if (wave == 0 && lg == 0)
              ((float*)p.out_scale)[(size_t)(m0 + r) * (N / 128) + nb] = sc;
          }
        }
        __syncthreads();
      } else {   // F_MX: 32-channel groups = two row tiles of one wave
        static_assert(F != F_MX || RTW % 2 == 0, "MX gate/up needs pairs of row tiles");
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = t * 16 + r16;
#pragma unroll
          for (int gp = 0; gp < RTW / 2; ++gp) {
            float m = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[0][2 * gp + q][t][i]));
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            int ex = m > 0.f ? ilog2_floor(m) - 8 : -127;
            ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
            const float inv = __builtin_ldexpf(1.0f, -ex);
            if (r < M) {
              uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                f32x4 h = acc[0][2 * gp + q][t];
                *(uint32_t*)(orow + nw0 + (2 * gp + q) * 16 + 4 * lg) =
                    cvt4_e4m3(h[0] * inv, h[1] * inv, h[2] * inv, h[3] * inv);
              }
              if (lg == 0)
                ((uint8_t*)p.out_scale)[(size_t)(m0 + r) * (N / 32) + (nw0 + 32 * gp) / 32] =
                    (uint8_t)(ex + 127);
            }
          }
        }
      }
    }
    __syncthreads();   // LDS buffers are reused by the next item
  }
}

// ------------------------------------------------------------------ launch
namespace {

int g_cu_count = 0;

int cu_count() {
  if (!g_cu_count) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_cu_count = n;
    else
      g_cu_count = 256;
  }
  return g_cu_count;
}

template <int F, bool GATEUP, int BM, int RTW>
hipError_t launch_one(const GemmArgs& g, hipStream_t st) {
  constexpr int NBR = WAVES * RTW * 16;
  if (g.N % NBR) return hipErrorInvalidValue;
  // upper bound on work items: the largest possible block table
  long max_tiles = (long)g.max_rows / BM + g.max_groups;
  long items = max_tiles * (g.N / NBR);
  long grid = (long)cu_count() * 2;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  if constexpr (GATEUP) {
    with_act(g.act, [&](auto a) {
      hipLaunchKernelGGL((k_gemm_tiled<F, true, BM, RTW, decltype(a)::value>), dim3((unsigned)grid),
                         dim3(THREADS), 0, st, g);
      return 0;
    });
  } else {
    hipLaunchKernelGGL((k_gemm_tiled<F, false, BM, RTW, ACT_SWIGLU>), dim3((unsigned)grid), dim3(THREADS), 0, st, g);
  }
  return hipGetLastError();
}

template <int F, bool GATEUP>
hipError_t launch_bm(int bm, const GemmArgs& g, hipStream_t st) {
  if constexpr (F != F_BF16) {
    return hipErrorInvalidValue;   // FP8 and MX formats use launch_gemm_pipe
  } else {
    switch (bm) {
      case 32: return launch_one<F, GATEUP, 32, 2>(g, st);
      case 64: return launch_one<F, GATEUP, 64, 2>(g, st);
    }
    return hipErrorInvalidValue;   // bf16 stops at 64-row blocks
  }
}

}  // namespace

hipError_t launch_gemm_tiled(int fmt, bool gateup, int cfg, const GemmArgs& g, hipStream_t st) {
  const int bm = cfg_rows(cfg);
  switch (fmt) {
    case F_BF16: return gateup ? launch_bm<F_BF16, true>(bm, g, st) : launch_bm<F_BF16, false>(bm, g, st);
    case F_FP8_CH: return gateup ? launch_bm<F_FP8_CH, true>(bm, g, st) : launch_bm<F_FP8_CH, false>(bm, g, st);
    case F_FP8_BLK: return gateup ? launch_bm<F_FP8_BLK, true>(bm, g, st) : launch_bm<F_FP8_BLK, false>(bm, g, st);
    case F_MX: return gateup ? launch_bm<F_MX, true>(bm, g, st) : launch_bm<F_MX, false>(bm, g, st);
  }
  return hipErrorInvalidValue;
}
