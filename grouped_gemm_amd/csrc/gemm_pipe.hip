// Pipelined grouped GEMM for large expert groups (prefill batches).
//
// Work item = (128-row block of one expert group from the block table, block
// of output channels), walked by a persistent grid (pure-Triton MoE
// commentary, second paragraph: block-id -> (expert, row offset) map, one
// launch, no padding between groups).
//
// Per K step of 128 elements a workgroup stages, in a ring of NSTAGE LDS
// buffers, the 128 token rows of its block and the 256 weight rows of its
// channel block.  Both are copied by asynchronous global->LDS loads
// (global_load_lds_dwordx4), so loads of the next NSTAGE-1 steps are in
// flight while the MFMAs of the current step run and no registers are held
// by them.  Rows land in LDS with their 16-byte chunks XOR-swizzled by the
// row index, which makes the MFMA fragment reads (16 rows, same chunk)
// bank-conflict free without padding.
//
// The four waves form a 2x2 grid: a wave owns 64 tokens and 128 weight rows
// (64 gate + 64 up rows for the fused op, so each lane holds matching gate
// and up values; 128 output channels for the down projection).
#include "layer.h"

namespace {

constexpr int PTHREADS = 256;
constexpr int PBM = 128;       // token rows per item
constexpr int PNR = 256;       // weight rows per item

typedef __attribute__((address_space(3))) void lds_void;

DEVI void lds_dma16(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}
DEVI void lds_dma4(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 4, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are pending.
DEVI void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every outstanding vector-memory operation, including the
// asynchronous stage loads that must stay in flight.  Callers wait for what
// they need (wait_vm, lgkmcnt) before it.
DEVI void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int F>
struct PipeFmt {
  static constexpr int WB = FmtBits<F>::W;            // 8 or 4
  static constexpr int WROWB = 128 * WB / 8;           // weight bytes per row per step
  static constexpr int TOKB = PBM * 128;               // token bytes per stage
  static constexpr int WTB = PNR * WROWB;              // weight bytes per stage
  static constexpr bool ASC = F == F_FP8_BLK || F == F_MX;   // activation scales per step
  static constexpr int ASB = ASC ? 4 * 256 : 0;        // 256 dword slots (4 waves x 64)
  static constexpr int WSB = F == F_MX ? 4 * PNR : 0;  // e8m0 weight scales, dword per row
  static constexpr int STAGE = TOKB + WTB + ASB + WSB;
  // per-wave DMA instructions per stage (vmcnt units)
  static constexpr int NTOK = TOKB / 1024 / 4;
  static constexpr int NWT = WTB / 1024 / 4;
  static constexpr int LOADS = NTOK + NWT + (ASC ? 1 : 0) + (F == F_MX ? 1 : 0);
};

// byte offset of (row, 16-byte chunk) in a swizzled [rows][128 B] block
DEVI int swz128(int row, int chunk) { return row * 128 + 16 * (chunk ^ (row & 7)); }
// byte offset of (row, chunk) in a swizzled [rows][64 B] block
DEVI int swz64(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 1) & 3)); }

}  // namespace

template <int F, bool GATEUP, int NSTAGE>
__global__ void __launch_bounds__(PTHREADS) k_gemm_pipe(GemmArgs p) {
  using PF = PipeFmt<F>;
  constexpr int WB = PF::WB;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int RT = GATEUP ? 4 : 8;           // 16-row weight tiles per matrix per wave
  constexpr int TT = 4;                        // 16-token tiles per wave
  constexpr int NBC = GATEUP ? 128 : 256;      // output channels per item
  constexpr int WSC_MAX = 128;                 // K steps covered by the scale table
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * PF::STAGE + 2 * PBM * 4 + 2 * 2 * WSC_MAX * 4];

  if (p.cfg_self >= 0 && p.meta[META_CFG] != p.cfg_self) return;
  const int ntiles = p.meta[META_NTILES];
  const int N = p.N, K = p.K;
  const int nblk = N / NBC;
  const int n_items = ntiles * nblk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, lg = lane >> 4;
  const long wrow = row_bytes<WB>(K), xrow = K;   // token rows are e4m3 here
  const int nsteps = K / 128;
  float* amax_l = (float*)(lds + NSTAGE * PF::STAGE);
  float* wsc_l = amax_l + 2 * PBM;            // [matrix][block of this item][K step]

  const ItemRange ir = xcd_items(n_items);
  for (int item = ir.begin; item < ir.end; item += ir.step) {
    const int tile = item / nblk, nb = item - tile * nblk;
    const int g = p.tiles[2 * tile], r0 = p.tiles[2 * tile + 1];
    const int m0 = p.indptr[g] + r0;
    const int M = min(PBM, p.counts[g] - r0);
    const bool sh = g >= p.E;
    const uint8_t* W0 = sh ? p.sh_w0 : p.w0 + (size_t)g * N * wrow;
    const uint8_t* W1 = GATEUP ? (sh ? p.sh_w1 : p.w1 + (size_t)g * N * wrow) : nullptr;
    size_t s_off = 0;
    if (!sh) {
      if (F == F_FP8_CH) s_off = (size_t)g * N * 4;
      if (F == F_FP8_BLK) s_off = (size_t)g * (N / 128) * (K / 128) * 4;
      if (F == F_MX) s_off = (size_t)g * N * (K / 32);
    }
    const uint8_t* S0 = (const uint8_t*)(sh ? p.sh_w0s : p.w0s) + s_off;
    const uint8_t* S1 = GATEUP ? (const uint8_t*)(sh ? p.sh_w1s : p.w1s) + s_off : nullptr;

    // --- source addresses of this lane's DMA slots (fixed for the item)
    // tokens: instruction i of this wave fills LDS token rows (wave*NTOK+i)*8 .. +8
    const uint8_t* tsrc[PF::NTOK];
#pragma unroll
    for (int i = 0; i < PF::NTOK; ++i) {
      const int row = (wave * PF::NTOK + i) * 8 + (lane >> 3);
      const int slot = m0 + (row < M ? row : 0);
      const int r = p.gather ? p.gather[slot] / p.gather_div : slot;
      const int chunk = (lane & 7) ^ (row & 7);
      tsrc[i] = p.a + (size_t)r * xrow + 16 * chunk;
    }
    // weights: LDS weight row R -> global row
    const uint8_t* wsrc[PF::NWT];
#pragma unroll
    for (int j = 0; j < PF::NWT; ++j) {
      int R, chunk;
      if constexpr (WB == 8) {
        R = (wave * PF::NWT + j) * 8 + (lane >> 3);
        chunk = (lane & 7) ^ (R & 7);
      } else {
        R = (wave * PF::NWT + j) * 16 + (lane >> 2);
        chunk = (lane & 3) ^ ((R >> 1) & 3);
      }
      const uint8_t* base;
      int grow;
      if (GATEUP) {
        base = R < 128 ? W0 : W1;
        grow = nb * 128 + (R & 127);
      } else {
        base = W0;
        grow = nb * 256 + R;
      }
      wsrc[j] = base + (size_t)grow * wrow + 16 * chunk;
    }
    // activation scales: lane covers token row wave*64 + lane (rows >= BM unused)
    const uint8_t* asrc = nullptr;
    if constexpr (PF::ASC) {
      const int row = wave * 64 + lane;
      const int slot = m0 + (row < M ? row : 0);
      const int r = p.gather ? p.gather[slot] / p.gather_div : slot;
      if (F == F_FP8_BLK) asrc = (const uint8_t*)p.a_scale + ((size_t)r * (K / 128)) * 4;
      else asrc = (const uint8_t*)p.a_scale + (size_t)r * (K / 32);
    }
    // MX weight scales: lane covers weight row wave*64 + lane
    const uint8_t* wssrc = nullptr;
    if constexpr (F == F_MX) {
      const int R = wave * 64 + lane;
      const uint8_t* sb = GATEUP ? (R < 128 ? S0 : S1) : S0;
      const int grow = GATEUP ? nb * 128 + (R & 127) : nb * 256 + R;
      wssrc = sb + (size_t)grow * (K / 32);
    }

    auto issue = [&](int s) {
      uint8_t* st = lds + (s % NSTAGE) * PF::STAGE;
#pragma unroll
      for (int i = 0; i < PF::NTOK; ++i) lds_dma16(tsrc[i] + (size_t)s * 128, st + (wave * PF::NTOK + i) * 1024);
#pragma unroll
      for (int j = 0; j < PF::NWT; ++j)
        lds_dma16(wsrc[j] + (size_t)s * PF::WROWB, st + PF::TOKB + (wave * PF::NWT + j) * 1024);
      if constexpr (F == F_FP8_BLK) lds_dma4(asrc + 4 * s, st + PF::TOKB + PF::WTB + wave * 256);
      if constexpr (F == F_MX) {
        lds_dma4(asrc + 4 * s, st + PF::TOKB + PF::WTB + wave * 256);
        lds_dma4(wssrc + 4 * s, st + PF::TOKB + PF::WTB + PF::ASB + wave * 256);
      }
    };

    f32x4 acc[NM][RT][TT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[m][rt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if constexpr (F == F_FP8_BLK) {
      // the item's 128x128 weight block scales for every K step, into LDS
      // (gate/up: blocks nb of both matrices; down: blocks 2nb and 2nb+1)
      for (int i = tid; i < 2 * nsteps; i += PTHREADS) {
        const int which = i / nsteps, ks = i - which * nsteps;
        float v;
        if (GATEUP) v = ((const float*)(which == 0 ? S0 : S1))[(size_t)nb * (K / 128) + ks];
        else v = ((const float*)S0)[(size_t)(2 * nb + which) * (K / 128) + ks];
        wsc_l[which * WSC_MAX + ks] = v;
      }
      __syncthreads();
    }

    // prologue: NSTAGE-1 steps in flight
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nsteps) issue(s);

    for (int s = 0; s < nsteps; ++s) {
      const int ahead = min(NSTAGE - 2, nsteps - 1 - s);   // later stages still loading
      wait_vm(ahead * PF::LOADS);
      raw_barrier();
      if (s + NSTAGE - 1 < nsteps) issue(s + NSTAGE - 1);
      const uint8_t* st = lds + (s % NSTAGE) * PF::STAGE;
      // token fragments of this wave (64 tokens)
      i32x8 bfr[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int row = wm * 64 + t * 16 + r16;
        const i32x4 lo = *(const i32x4*)(st + swz128(row, lg));
        const i32x4 hi = *(const i32x4*)(st + swz128(row, lg + 4));
        bfr[t] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      float sx[TT];
      int sbx[TT];
      if constexpr (F == F_FP8_BLK) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
          sx[t] = ((const float*)(st + PF::TOKB + PF::WTB))[wm * 64 + t * 16 + r16];
      }
      if constexpr (F == F_MX) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
          sbx[t] = (st + PF::TOKB + PF::WTB)[(wm * 64 + t * 16 + r16) * 4 + lg];
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        float wsc = 1.f;
        if constexpr (F == F_FP8_BLK) wsc = wsc_l[(GATEUP ? m : wn) * WSC_MAX + s];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // LDS weight row of this lane for tile rt
          const int R = GATEUP ? (m * 128 + wn * 64 + rt * 16 + r16) : (wn * 128 + rt * 16 + r16);
          i32x8 afr;
          int sw = 0;
          if constexpr (WB == 8) {
            const i32x4 lo = *(const i32x4*)(st + PF::TOKB + swz128(R, lg));
            const i32x4 hi = *(const i32x4*)(st + PF::TOKB + swz128(R, lg + 4));
            afr = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            const i32x4 q = *(const i32x4*)(st + PF::TOKB + swz64(R, lg));
            afr = (i32x8){q[0], q[1], q[2], q[3], 0, 0, 0, 0};
            sw = (st + PF::TOKB + PF::WTB + PF::ASB)[R * 4 + lg];
          }
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            if constexpr (F == F_FP8_BLK) {
              f32x4 d = mfma_f8(afr, bfr[t], (f32x4){0.f, 0.f, 0.f, 0.f});
              acc[m][rt][t] += d * (sx[t] * wsc);
            } else if constexpr (F == F_MX) {
              acc[m][rt][t] = mfma_f4f8_scaled(afr, bfr[t], acc[m][rt][t], sw, sbx[t]);
            } else {
              acc[m][rt][t] = mfma_f8(afr, bfr[t], acc[m][rt][t]);
            }
          }
        }
      }
    }
    __syncthreads();   // every wave is done with the ring before it is refilled

    // ------------------------------------------------------------ epilogue
    // lane: channel c0 + rt*16 + 4*lg + i, token row wm*64 + t*16 + r16
    const int c0 = GATEUP ? nb * 128 + wn * 64 : nb * 256 + wn * 128;
    int tok[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int r = wm * 64 + t * 16 + r16;
      const int slot = m0 + (r < M ? r : 0);
      tok[t] = p.gather ? p.gather[slot] / p.gather_div : slot;
    }
    if constexpr (F == F_FP8_CH) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sxt = ((const float*)p.a_scale)[tok[t]];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f32x4 wsv = *(const f32x4*)((const float*)(m == 0 ? S0 : S1) + c0 + rt * 16 + 4 * lg);
            acc[m][rt][t] = acc[m][rt][t] * sxt * wsv;
          }
      }
    }
    if constexpr (!GATEUP) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int r = wm * 64 + t * 16 + r16;
        if (r >= M) continue;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) store_down(p, m0 + r, c0 + rt * 16 + 4 * lg, acc[0][rt][t]);
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[0][rt][t][i] = silu(acc[0][rt][t][i]) * acc[1][rt][t][i];
      if constexpr (F == F_FP8_CH) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = wm * 64 + t * 16 + r16;
          if (r >= M) continue;
          float* orow = (float*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) *(f32x4*)(orow + c0 + rt * 16 + 4 * lg) = acc[0][rt][t];
        }
      } else if constexpr (F == F_FP8_BLK) {
        // 1x128 group = this item's 128 channels = the two waves wn = 0, 1
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          float mx = 0.f;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[0][rt][t][i]));
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          if (lg == 0) amax_l[wn * PBM + wm * 64 + t * 16 + r16] = mx;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = wm * 64 + t * 16 + r16;
          const float a = fmaxf(amax_l[r], amax_l[PBM + r]);
          const float sc = a > 0.f ? a / 448.0f : 1.0f;
          if (r < M) {
            uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const f32x4 h = acc[0][rt][t];
              *(uint32_t*)(orow + c0 + rt * 16 + 4 * lg) =
                  cvt4_e4m3(h[0] / sc, h[1] / sc, h[2] / sc, h[3] / sc);
            }
            if (wn == 0 && lg == 0) ((float*)p.out_scale)[(size_t)(m0 + r) * (N / 128) + nb] = sc;
          }
        }
        __syncthreads();
      } else {   // F_MX: 32-channel groups = row-tile pairs of this wave
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = wm * 64 + t * 16 + r16;
#pragma unroll
          for (int gp = 0; gp < RT / 2; ++gp) {
            float mx = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[0][2 * gp + q][t][i]));
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            int ex = mx > 0.f ? ilog2_floor(mx) - 8 : -127;
            ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
            const float inv = __builtin_ldexpf(1.0f, -ex);
            if (r < M) {
              uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                const f32x4 h = acc[0][2 * gp + q][t];
                *(uint32_t*)(orow + c0 + (2 * gp + q) * 16 + 4 * lg) =
                    cvt4_e4m3(h[0] * inv, h[1] * inv, h[2] * inv, h[3] * inv);
              }
              if (lg == 0) ((uint8_t*)p.out_scale)[(size_t)(m0 + r) * (N / 32) + (c0 + 32 * gp) / 32] = (uint8_t)(ex + 127);
            }
          }
        }
      }
    }
  }
}

namespace {

int pipe_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <int F, bool GATEUP>
hipError_t launch_pipe_t(const GemmArgs& g, hipStream_t st) {
  constexpr int NBC = GATEUP ? 128 : 256;
  if (g.N % NBC || g.K % 128 || g.K > 128 * 128) return hipErrorInvalidValue;
  long max_tiles = (long)g.max_rows / PBM + g.max_groups;
  long items = max_tiles * (g.N / NBC);
  long grid = pipe_cus();
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_gemm_pipe<F, GATEUP, 3>), dim3((unsigned)grid), dim3(PTHREADS), 0, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_pipe(int fmt, bool gateup, const GemmArgs& g, hipStream_t st) {
  switch (fmt) {
    case F_FP8_CH: return gateup ? launch_pipe_t<F_FP8_CH, true>(g, st) : launch_pipe_t<F_FP8_CH, false>(g, st);
    case F_FP8_BLK: return gateup ? launch_pipe_t<F_FP8_BLK, true>(g, st) : launch_pipe_t<F_FP8_BLK, false>(g, st);
    case F_MX: return gateup ? launch_pipe_t<F_MX, true>(g, st) : launch_pipe_t<F_MX, false>(g, st);
  }
  return hipErrorInvalidValue;
}
