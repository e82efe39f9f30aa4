// Pipelined grouped GEMM for large expert groups (prefill batches).
//
// Work item = (128-row block of one expert group from the block table, block
// of output channels), walked by a persistent grid (pure-Triton MoE
// commentary, second paragraph: block-id -> (expert, row offset) map, one
// launch, no padding between groups).
//
// Per K step of 128 elements a workgroup stages, in a ring of NSTAGE LDS
// buffers, the BM token rows of its block and the NR weight rows of its
// channel block (gate rows then up rows for the fused op).  Both are copied by asynchronous global->LDS loads
// (global_load_lds_dwordx4), so loads of the next NSTAGE-1 steps are in
// flight while the MFMAs of the current step run and no registers are held
// by them.  Rows land in LDS with their 16-byte chunks XOR-swizzled by the
// row index, which makes the MFMA fragment reads (16 rows, same chunk)
// bank-conflict free without padding.
//
// The four waves form a WM x WN grid over (tokens, channels): a wave owns
// BM/WM tokens and NBC/WN output channels (the matching gate and up rows for
// the fused op, so each lane holds gate and up values of the same channel).
// Large blocks (BM = 128, NR = 256) serve prefill; BM = 32/64 with deep rings
// serve decode, where the kernel is a stream of weight bytes with several
// K steps of every workgroup in flight.
#include "layer.h"

namespace {

constexpr int LDS_RING_BUDGET = 150 * 1024;   // bytes of LDS for the stage ring

typedef __attribute__((address_space(3))) void lds_void;

DEVI void lds_dma16(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}
DEVI void lds_dma4(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 4, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are pending
// (n is wave-uniform; the counter field holds 0..63).
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
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
    case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 33: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
    case 34: asm volatile("s_waitcnt vmcnt(34)" ::: "memory"); break;
    case 35: asm volatile("s_waitcnt vmcnt(35)" ::: "memory"); break;
    case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
    case 37: asm volatile("s_waitcnt vmcnt(37)" ::: "memory"); break;
    case 38: asm volatile("s_waitcnt vmcnt(38)" ::: "memory"); break;
    case 39: asm volatile("s_waitcnt vmcnt(39)" ::: "memory"); break;
    case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 41: asm volatile("s_waitcnt vmcnt(41)" ::: "memory"); break;
    case 42: asm volatile("s_waitcnt vmcnt(42)" ::: "memory"); break;
    case 43: asm volatile("s_waitcnt vmcnt(43)" ::: "memory"); break;
    case 44: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
    case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
    case 46: asm volatile("s_waitcnt vmcnt(46)" ::: "memory"); break;
    case 47: asm volatile("s_waitcnt vmcnt(47)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    case 49: asm volatile("s_waitcnt vmcnt(49)" ::: "memory"); break;
    case 50: asm volatile("s_waitcnt vmcnt(50)" ::: "memory"); break;
    case 51: asm volatile("s_waitcnt vmcnt(51)" ::: "memory"); break;
    case 52: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
    case 53: asm volatile("s_waitcnt vmcnt(53)" ::: "memory"); break;
    case 54: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
    case 55: asm volatile("s_waitcnt vmcnt(55)" ::: "memory"); break;
    case 56: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
    case 57: asm volatile("s_waitcnt vmcnt(57)" ::: "memory"); break;
    case 58: asm volatile("s_waitcnt vmcnt(58)" ::: "memory"); break;
    case 59: asm volatile("s_waitcnt vmcnt(59)" ::: "memory"); break;
    case 60: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
    case 61: asm volatile("s_waitcnt vmcnt(61)" ::: "memory"); break;
    case 62: asm volatile("s_waitcnt vmcnt(62)" ::: "memory"); break;
    case 63: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// The same with a compile-time count (no dispatch on the value).
template <int N>
DEVI void wait_vm_c() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for a*L + b*M outstanding operations, a = A, A-1, ..., 0 tried in
// that order (the first is the steady state), b in {0, 1}.
template <int L, int M, int A>
DEVI void wait_vm_ab(int a, bool b) {
  if constexpr (A >= 0) {
    if (a == A) {
      if (b) wait_vm_c<A * L + M>();
      else wait_vm_c<A * L>();
    } else {
      wait_vm_ab<L, M, A - 1>(a, b);
    }
  } else {
    wait_vm_c<0>();
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

// K-major weight fragments: for each of RT LDS addresses the transpose
// reads of K rows +0, +4 (2048 bytes on), +32 and +36.  One asm block that
// waits for its own reads before it ends, so every output is written when
// it returns (the builtin form makes the compiler wait for every
// asynchronous global->LDS load in flight before each read, as it cannot
// tell them from the stage read here, which the ring's waits and barrier
// already cover).
typedef int i32x2 __attribute__((ext_vector_type(2)));
template <int RT> struct KnFrags { i32x2 v[4 * RT]; };
template <int RT> DEVI KnFrags<RT> read_kn_frags(const uint32_t (&ad)[RT]);
template <> DEVI KnFrags<4> read_kn_frags<4>(const uint32_t (&ad)[4]) {
  KnFrags<4> f;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n"
      "ds_read_b64_tr_b16 %2, %16 offset:16384\n"
      "ds_read_b64_tr_b16 %3, %16 offset:18432\n"
      "ds_read_b64_tr_b16 %4, %17\n"
      "ds_read_b64_tr_b16 %5, %17 offset:2048\n"
      "ds_read_b64_tr_b16 %6, %17 offset:16384\n"
      "ds_read_b64_tr_b16 %7, %17 offset:18432\n"
      "ds_read_b64_tr_b16 %8, %18\n"
      "ds_read_b64_tr_b16 %9, %18 offset:2048\n"
      "ds_read_b64_tr_b16 %10, %18 offset:16384\n"
      "ds_read_b64_tr_b16 %11, %18 offset:18432\n"
      "ds_read_b64_tr_b16 %12, %19\n"
      "ds_read_b64_tr_b16 %13, %19 offset:2048\n"
      "ds_read_b64_tr_b16 %14, %19 offset:16384\n"
      "ds_read_b64_tr_b16 %15, %19 offset:18432\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.v[0]), "=&v"(f.v[1]), "=&v"(f.v[2]), "=&v"(f.v[3]), "=&v"(f.v[4]),
        "=&v"(f.v[5]), "=&v"(f.v[6]), "=&v"(f.v[7]), "=&v"(f.v[8]), "=&v"(f.v[9]),
        "=&v"(f.v[10]), "=&v"(f.v[11]), "=&v"(f.v[12]), "=&v"(f.v[13]), "=&v"(f.v[14]),
        "=&v"(f.v[15])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
  return f;
}

template <int F, bool GATEUP, int BM, int NR, int WM, int NW>
struct PipeCfg {
  static constexpr int WN = NW / WM;
  static constexpr int WB = FmtBits<F>::W;             // 8 or 4
  // a K step is 128 bytes of a row: 128 elements of the 8- and 4-bit
  // formats (64 bytes of e2m1 weights), 64 of bf16
  static constexpr int KE = F == F_BF16 ? 64 : 128;    // K elements per step
  static constexpr int WROWB = KE * WB / 8;            // weight bytes per row per step
  static constexpr int TOKB = BM * 128;                // token bytes per stage
  static constexpr int WTB = NR * WROWB;               // weight bytes per stage
  static constexpr bool ASC = F == F_FP8_BLK || F == F_MX;   // per-step scale slots
  static constexpr int ASB = ASC ? NW * 256 : 0;       // 64 dwords per wave
  static constexpr int WSB = F == F_MX ? NW * 256 : 0; // e8m0 weight scales, dword per row
  static constexpr int STAGE = TOKB + WTB + ASB + WSB;
  static constexpr int NSTAGE_FIT = LDS_RING_BUDGET / STAGE;
  static constexpr int NSTAGE = NSTAGE_FIT > 8 ? 8 : NSTAGE_FIT;
  static constexpr int NBC = GATEUP ? NR / 2 : NR;     // output channels per item
  static constexpr int NM_ = GATEUP ? 2 : 1;           // weight matrices
  static constexpr int TT = BM / WM / 16;              // 16-token tiles per wave
  static constexpr int RT = NBC / WN / 16;             // 16-row tiles per matrix per wave
  static constexpr int RB = BM > 64 ? BM : 64;         // rows per row-metadata buffer
  // per-wave DMA instructions per stage (vmcnt units), and per item start
  static constexpr int NTOK = TOKB / (NW * 1024);
  static constexpr int NWT = WTB / (NW * 1024);
  static constexpr int LOADS = NTOK + NWT + (ASC ? 1 : 0) + (F == F_MX ? 1 : 0);
  static constexpr int NMETA = 4;
  static_assert(NSTAGE >= 2, "stage ring does not fit");
  static_assert(TT >= 1 && RT >= 1 && NTOK >= 1 && NWT >= 1, "tile shape");
  static_assert(!(GATEUP && F == F_FP8_BLK) || NBC == 128, "1x128 requantisation needs 128 channels");
  static_assert(!(GATEUP && F == F_MX) || RT % 2 == 0, "MX requantisation needs 32-channel groups");
  static_assert(F != F_FP8_BLK || BM <= (NW - 1) * 64, "the last wave's scale slot carries weight scales");
  static_assert(TOKB % (NW * 1024) == 0 && WTB % (NW * 1024) == 0, "whole DMA instructions per wave");
  static_assert(F != F_MX || !GATEUP || NR == 256, "MX gate/up scale rows: one matrix per wave pair");
  static_assert((NSTAGE - 2) * (LOADS + NMETA) <= 63, "vmcnt range");
  static_assert(NM_ * NBC <= NW * 64 && NBC % 64 == 0, "channel scales: one per lane of the waves");
  static_assert(RT % 2 == 0 || BM < 128 || (GATEUP && F != F_FP8_BLK), "regrouped stores pair 16-channel tiles");
};

// Regrouping of two 16-channel MFMA output tiles (a: channels 0..15, b:
// channels 16..31 of a 32-channel half; the lanes of 16-lane row g hold one
// dword of channels 4g..4g+3 of each) into the layout where row g holds
// channels 8g..8g+7 as two dwords (.x: 8g..8g+3, .y: 8g+4..8g+7).  Rows 0/1
// take a's dwords of rows 0,1 / 2,3, rows 2/3 take b's.  Two gfx950 lane
// swaps: the 32-lane swap exchanges a's rows 2,3 with b's rows 0,1, then
// the 16-lane swap exchanges odd rows of the first result with even rows of
// the second.  Every lane of the wave takes part.
DEVI uint2 regroup32(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  const auto q = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
  return make_uint2(q[0], q[1]);
}

// Maximum over the four 16-lane rows (lanes l, l^16, l^32, l^48), in every
// lane: a lane swap with itself pairs lane l with l^32, then with l^16.
DEVI float max_over_rows(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// byte offset of (row, 16-byte chunk) in a swizzled [rows][128 B] block
DEVI int swz128(int row, int chunk) { return row * 128 + 16 * (chunk ^ (row & 7)); }
// byte offset of (row, chunk) in a swizzled [rows][64 B] block
DEVI int swz64(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 1) & 3)); }

}  // namespace

// LDS bytes one tile shape needs: stage ring, cross-wave amax, item
// metadata (double-buffered row indices, activation scales, routing weights
// and per-channel weight scales) and a sink for the metadata loads of waves
// that carry none.
template <int F, bool GATEUP, int BM, int NR, int WM, int NW>
constexpr int pipe_lds_bytes() {
  using PC = PipeCfg<F, GATEUP, BM, NR, WM, NW>;
  return PC::NSTAGE * PC::STAGE + PC::WN * BM * 4 + 3 * 2 * PC::RB * 4 + 2 * 256 * 4 + NW * 256;
}

// One persistent workgroup walks its items (row block x channel block) as a
// single stream of K steps: the ring runs on across item boundaries, so the
// first stages of the next item load while the current item finishes and
// writes its outputs.  Per item, the rows' metadata (gather indices, then
// per-row activation scales and routing weights) is also brought into LDS by
// asynchronous loads issued ahead of the item's first stage.
//
// All DMA sources are a wave-uniform base (advanced per step in scalar
// registers) plus a fixed 32-bit per-lane offset.
// ACT: the gate/up epilogue's activation (ACT_*; the down projection
// ignores it).
// WT: bf16 plain op with K-major weights (GemmArgs::w_kn): a stage's weight
// tile is 64 K rows of the item's 256 channels (512 bytes each, 32-byte
// blocks XOR-swizzled by row), and the weight fragments come from LDS
// transpose reads (ds_read_b64_tr_b16: within each 16-lane group, lane i
// receives element i % 4 of the 8-byte pieces addressed by lanes i / 4 + 4 k;
// lane j addressing K row kb + j / 4 at channels 4 (j % 4) .. + 3 of a
// 16-channel block, lane i gets K rows kb .. kb + 3 of channel i).
template <int F, bool GATEUP, int BM, int NR, int WM, int NW, int ACT, bool WT = false>
DEVI void pipe_body(const GemmArgs& p, uint8_t* lds) {
  using PC = PipeCfg<F, GATEUP, BM, NR, WM, NW>;
  static_assert(!WT || (F == F_BF16 && !GATEUP && NR == 256 && PC::NWT * NW * 2 == 64),
                "K-major weights: bf16 plain op, 256-channel items, 64 K rows per stage");
  constexpr int WB = PC::WB, WN = PC::WN, NSTAGE = PC::NSTAGE;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int RT = PC::RT, TT = PC::TT, NBC = PC::NBC, RB = PC::RB;
  constexpr int NTOK = PC::NTOK, NWT = PC::NWT, LOADS = PC::LOADS, NMETA = PC::NMETA;
  constexpr int MW = (BM + 63) / 64;             // waves whose lanes carry item rows

  const int N = p.N, K = p.K;
  const int nblk = N / NBC;
  const int n_items = ldu(p.meta + META_NTILES) * nblk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves w and w + NW/2 share a SIMD; with two row halves (WM = 2) they
  // hold different halves, so a block whose rows end in the first half
  // leaves each SIMD one wave of MFMA work
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, lg = lane >> 4;
  // token rows: e4m3 codes, or bf16
  const uint32_t wrow = (uint32_t)row_bytes<WB>(K), xrow = (uint32_t)row_bytes<FmtBits<F>::X>(K);
  const int ns = K / PC::KE;
  // activation-scale bytes per token row
  const uint32_t srow = F == F_FP8_BLK ? (uint32_t)(K / 128) * 4 : (uint32_t)(K / 32);

  float* amax_l = (float*)(lds + NSTAGE * PC::STAGE);   // [WN][BM]
  int32_t* idx_l = (int32_t*)(amax_l + WN * BM);         // [2][RB] row index source values
  float* as_l = (float*)(idx_l + 2 * RB);                // [2][RB] per-row activation scale (FP8 per channel)
  float* rw_l = as_l + 2 * RB;                           // [2][RB] routing weight of the row's slot
  float* cs_l = rw_l + 2 * RB;                           // [2][256] channel scales (FP8 per channel)
  uint8_t* sink_l = (uint8_t*)(cs_l + 2 * 256);          // [NW][256]

  const ItemRange ir = xcd_items(n_items);
  if (ir.begin >= ir.end) return;
  const int nit = (ir.end - ir.begin + ir.step - 1) / ir.step;
  const int nq = nit * ns;                               // K steps of this workgroup
  const int D = min(NSTAGE - 1, ns);                     // stages loaded ahead

  // array whose values select the rows of an item: the activation gather, or
  // (down projection) the slot -> routing-weight index
  const int32_t* rowsrc = p.gather ? p.gather : (p.row_w ? p.row_w_idx : nullptr);

  struct It {
    int g, m0, M, cbase;
    bool sh;
  };
  auto info = [&](int j) {
    const int item = ir.begin + j * ir.step;
    const int tile = item / nblk, nb = item - tile * nblk;
    It r;
    r.g = ldu(p.tiles + 2 * tile);
    const int r0 = ldu(p.tiles + 2 * tile + 1);
    r.m0 = ldu(p.indptr + r.g) + r0;
    r.M = min(BM, ldu(p.counts + r.g) - r0);
    r.sh = r.g >= p.E;
    r.cbase = nb * NBC;
    return r;
  };

  // ---- per-lane DMA offsets that are the same for every item.  The weight
  // rows of one wave belong to one matrix (gate or up) and its DMA
  // instructions differ by a whole number of row groups, so one lane offset
  // serves all of them; the rest is a wave-uniform base.
  constexpr int RPI = PC::WROWB == 128 ? 8 : 16;         // weight rows per DMA instruction
  static_assert(!GATEUP || NBC % (NWT * RPI) == 0, "a wave's weight rows lie in one matrix");
  const int wr0 = wave * NWT * RPI;                      // first weight row of this wave
  const bool wup = GATEUP && wr0 >= NBC;                 // wave loads up rows
  uint32_t woff;
  if constexpr (PC::WROWB == 128) woff = (uint32_t)(lane >> 3) * wrow + 16 * ((lane & 7) ^ ((lane >> 3) & 7));
  else woff = (uint32_t)(lane >> 2) * wrow + 16 * ((lane & 3) ^ ((lane >> 3) & 3));
  const size_t wrel = (size_t)(wup ? wr0 - NBC : wr0) * wrow;   // wave's rows in its matrix
  // K-major weights: this wave loads K rows 8 wave + 2 jj + lane / 32 of a
  // step (jj < NWT), 16-byte piece lane % 32 of the row's 512 bytes; the
  // piece at LDS position q (32-byte block q / 2) holds source block
  // (q / 2) ^ swz(row), swz(row) = (row & 3) | ((row >> 3) & 1) << 2, whose
  // row & 3 follows the parity of jj
  const uint32_t krow = (uint32_t)N * 2;                 // bytes per K row
  uint32_t woff_kn[2] = {0, 0};
  if constexpr (WT) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int r = 2 * par + (lane >> 5);
      const int sw = (r & 3) | ((wave & 1) << 2);
      const int q = lane & 31;
      woff_kn[par] = (uint32_t)(lane >> 5) * krow + 16 * (2 * ((q >> 1) ^ sw) + (q & 1));
    }
  }
  const int ks_w1 = WT ? p.w_k0 / PC::KE : 1 << 30;      // first step from w1
  const uint8_t* ib_w1 = nullptr;                        // K-major: the item's w1 base
  uint32_t wsoff = 0;        // MX: e8m0 scale row of this lane's weight row
  if constexpr (F == F_MX) {
    const int R0 = wave * 64 + lane;
    const int R = R0 < NR ? R0 : 0;
    wsoff = (uint32_t)(GATEUP && R >= NBC ? R - NBC : R) * (uint32_t)(K / 32);
  }

  // ---- issue-side state: bases advanced by one K step per issued stage
  const uint8_t* ib_tok = nullptr;         // token rows (uniform)
  const uint8_t* ib_w = nullptr;           // this wave's weight rows
  const uint8_t* ib_a = nullptr;           // activation scales
  const uint8_t* ib_ws = nullptr;          // weight scales (BLK: lane-selected block; MX: wave's matrix)
  uint32_t toff[NTOK];
  uint32_t aoff = 0;
  const uint8_t* ib_sc = nullptr;          // FP8 1x128: this lane's per-step scale source
  int m_even = 0, m_odd = 0;               // rows of the last begun items, by parity

  const int mrow = wave * 64 + lane;       // metadata row of this lane
  const bool mwave = wave < MW;

  // row-index values of item jn -> idx_l[jn&1] (sink when absent)
  auto meta_rows = [&](int jn) {
    const int32_t* src = p.meta;
    uint8_t* dst = sink_l + wave * 256;
    if (jn < nit && rowsrc && mwave) {
      const It n = info(jn);
      src = rowsrc + n.m0 + min(mrow, n.M - 1);
      dst = (uint8_t*)(idx_l + (jn & 1) * RB + wave * 64);
    }
    lds_dma4(src, dst);
  };

  // build the issue-side state of item j (its row indices are in idx_l) and
  // issue its per-item metadata: per-row activation scale (per-channel FP8),
  // routing weight of the down projection's weighted store, and the
  // per-channel weight scales
  auto begin_item = [&](int j) {
    const It it = info(j);
    if (j & 1) m_odd = it.M;
    else m_even = it.M;
    const int32_t* ix = idx_l + (j & 1) * RB;
    const bool gat = p.gather != nullptr;
    ib_tok = gat ? p.a : p.a + (size_t)it.m0 * xrow;
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
      const int row = (wave * NTOK + i) * 8 + (lane >> 3);
      const int rr = min(row, it.M - 1);
      const uint32_t r = gat ? (uint32_t)(ix[rr] / p.gather_div) : (uint32_t)rr;
      toff[i] = r * xrow + 16 * ((lane & 7) ^ (row & 7));
    }
    const int rr = min(mrow, it.M - 1);
    const uint32_t rm = gat ? (uint32_t)(ix[rr] / p.gather_div) : (uint32_t)rr;
    if constexpr (PC::ASC) {
      ib_a = gat ? (const uint8_t*)p.a_scale : (const uint8_t*)p.a_scale + (size_t)it.m0 * srow;
      aoff = rm * srow;
    }
    if constexpr (WT) {
      const size_t c0 = (size_t)it.cbase * 2 + (size_t)wave * 8 * krow;
      ib_w = (ks_w1 == 0 ? p.w1 : p.w0 + (size_t)it.g * p.w_k0 * krow) + c0;
      ib_w1 = p.w1 ? p.w1 + (size_t)it.g * (K - p.w_k0) * krow + c0 : ib_w;
    } else {
      const size_t wexp = (size_t)it.g * N * wrow;
      const uint8_t* wm0 = wup ? (it.sh ? p.sh_w1 : p.w1 + wexp) : (it.sh ? p.sh_w0 : p.w0 + wexp);
      ib_w = wm0 + (size_t)it.cbase * wrow + wrel;
    }
    if constexpr (F == F_FP8_BLK) {
      // lane 0: block of the gate (down: first 128 rows), lane 1: up (down:
      // the second 128 rows when the item has them)
      const size_t so = it.sh ? 0 : (size_t)it.g * (N / 128) * (K / 128) * 4;
      const size_t blk = (size_t)(it.cbase / 128) * (K / 128) * 4;
      const uint8_t* s0 = (const uint8_t*)(it.sh ? p.sh_w0s : p.w0s) + so + blk;
      const uint8_t* s1;
      if (GATEUP) s1 = (const uint8_t*)(it.sh ? p.sh_w1s : p.w1s) + so + blk;
      else s1 = NR > 128 ? s0 + (size_t)(K / 128) * 4 : s0;
      ib_ws = (lane & 1) ? s1 : s0;
      ib_sc = wave == NW - 1 ? ib_ws : ib_a + aoff;
    }
    if constexpr (F == F_MX) {
      const size_t so = it.sh ? 0 : (size_t)it.g * N * (K / 32);
      const size_t ro = (size_t)it.cbase * (K / 32);
      const bool up = GATEUP && wave * 64 >= NBC;
      ib_ws = (const uint8_t*)(up ? (it.sh ? p.sh_w1s : p.w1s) : (it.sh ? p.sh_w0s : p.w0s)) + so + ro;
    }
    const void* as_src = p.meta;
    uint8_t* as_dst = sink_l + wave * 256;
    const void* rw_src = p.meta;
    uint8_t* rw_dst = sink_l + wave * 256;
    if (mwave) {
      if (F == F_FP8_CH) {
        as_src = gat ? (const float*)p.a_scale + rm : (const float*)p.a_scale + it.m0 + rr;
        as_dst = (uint8_t*)(as_l + (j & 1) * RB + wave * 64);
      }
      if (p.row_w) {
        const int slot = it.m0 + rr;
        rw_src = slot < p.row_w_n ? p.row_w + ix[rr] : p.row_w;
        rw_dst = (uint8_t*)(rw_l + (j & 1) * RB + wave * 64);
      }
    }
    lds_dma4(as_src, as_dst);
    lds_dma4(rw_src, rw_dst);
    const void* cs_src = p.meta;
    uint8_t* cs_dst = sink_l + wave * 256;
    if (F == F_FP8_CH && wave * 64 < NM * NBC) {
      const int m = wave * 64 / NBC;          // the matrix is uniform per wave (NBC % 64 == 0)
      const size_t so = it.sh ? 0 : (size_t)it.g * N;
      const void* sbase;
      if (m == 0) sbase = it.sh ? p.sh_w0s : p.w0s;
      else sbase = it.sh ? p.sh_w1s : p.w1s;
      cs_src = (const float*)sbase + so + it.cbase + (wave * 64 - m * NBC) + lane;
      cs_dst = (uint8_t*)(cs_l + (j & 1) * 256 + wave * 64);
    }
    lds_dma4(cs_src, cs_dst);
  };

  // One stage into ring slot `slot` is NP DMA instructions per wave (token
  // rows, weight rows, then the step's scales); part k issues the k-th.
  // The main loop spreads the parts between its MFMA groups, so the
  // address unit streams the next stage while the matrix cores work;
  // advance() then moves the bases by one K step.
  constexpr int NSC = F == F_FP8_BLK ? 1 : (F == F_MX ? 2 : 0);
  constexpr int NP = NTOK + NWT + NSC;
  constexpr bool SPREAD = F != F_MX;   // parts spread over the MFMA groups
  auto issue_part = [&](int slot, int k) {
    uint8_t* st = lds + slot * PC::STAGE;
    if (k < NTOK) {
      lds_dma16(ib_tok + toff[k], st + (wave * NTOK + k) * 1024);
    } else if (k < NTOK + NWT) {
      const int jj = k - NTOK;
      // the offset is re-materialised as a 32-bit value, so the loads take
      // the scalar base + 32-bit lane offset form
      if constexpr (WT) {
        uint32_t wo = woff_kn[jj & 1];
        asm volatile("" : "+v"(wo));
        lds_dma16(ib_w + (size_t)jj * 2 * krow + wo, st + PC::TOKB + (wave * NWT + jj) * 1024);
      } else {
        uint32_t wo = woff;
        asm volatile("" : "+v"(wo));
        lds_dma16(ib_w + (size_t)jj * RPI * wrow + wo, st + PC::TOKB + (wave * NWT + jj) * 1024);
      }
    } else if constexpr (F == F_FP8_BLK) {
      // activation scales of the step's rows; the last wave, the step's
      // weight block scales (lanes 0 and 1)
      lds_dma4(ib_sc, st + PC::TOKB + PC::WTB + wave * 256);
    } else if constexpr (F == F_MX) {
      if (k == NTOK + NWT)
        lds_dma4(ib_a + aoff, st + PC::TOKB + PC::WTB + wave * 256);
      else
        lds_dma4(ib_ws + wsoff, st + PC::TOKB + PC::WTB + PC::ASB + wave * 256);
    }
  };
  // next_step: the step of the stage issued next (K-major weights switch
  // to w1 at step ks_w1)
  auto advance = [&](int next_step) {
    ib_tok += 128;
    if constexpr (WT) ib_w = next_step == ks_w1 ? ib_w1 : ib_w + (size_t)PC::KE * krow;
    else ib_w += PC::WROWB;
    ib_a += 4;
    ib_ws += 4;
    ib_sc += 4;
  };
  auto issue = [&](int slot) {
#pragma unroll
    for (int k = 0; k < NP; ++k) issue_part(slot, k);
  };

  // ---- start: row indices of the first item, then the first D stages.
  // The bases point at the stage to issue next: begin_item sets them to an
  // item's first step, advance() moves them on after a stage whose item
  // has more steps (after an item's last stage they stay where they are, so
  // the loads past the last item read valid addresses again).
  meta_rows(0);
  wait_vm(0);
  raw_barrier();
  begin_item(0);
  meta_rows(1);
  for (int q = 0; q < D; ++q) {
    issue(q);
    if (q + 1 < ns) advance(q + 1);
  }

  f32x4 acc[NM][RT][TT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[m][rt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int trow0 = wm * (BM / WM);                      // first token row of the wave
  const int wrow0 = wn * (NBC / WN);                     // first weight row (per matrix)
  // compute position (item j, step s, ring slot cs); issue position (item
  // ji, step si, ring slot is_) runs D stages ahead, at most one item ahead
  int j = 0, s = 0, cs = 0;
  int ji = D == ns ? 1 : 0, si = D == ns ? 0 : D, is_ = D % NSTAGE;
  for (int q = 0; q < nq; ++q) {
    // Wait for stage q; stages q+1 .. q+ahead may stay in flight.  The
    // count is the number of stage loads issued after stage q, n.  Loads
    // complete in order, so while stage q is incomplete all n later loads
    // are outstanding too and the counter stays above n: the wait is exact
    // for loads.  The epilogues' output stores share the counter and may
    // complete in any order; counted nowhere, they can only keep the
    // counter higher (a longer wait), never let it pass early.  Metadata
    // loads issued with an item start among the stages ahead are not
    // counted either (the wait then also covers a few loads of the next
    // stage, once per item).
    // Every step issues one stage, also past the last item (then it loads
    // the last issued stage's addresses again into the slot no remaining
    // step reads), so D - 1 stages always follow stage q.
    if (D == NSTAGE - 1) wait_vm_c<(NSTAGE - 2) * LOADS>();
    else wait_vm_ab<LOADS, 0, NSTAGE - 3>(D - 1, false);
    raw_barrier();
    // the stage this step issues (into the slot every wave has finished
    // reading: the barrier above), spread over the MFMA groups below
    const bool iss = ji < nit;
    const int islot = is_;
    if (iss) {
      if (si == 0) {
        begin_item(ji);
        meta_rows(ji + 1);
      }
      is_ = is_ + 1 == NSTAGE ? 0 : is_ + 1;
      if (++si == ns) {
        si = 0;
        ++ji;
      }
    }
    // MX weights (half the bytes per row) measure faster issued at once
    if constexpr (!SPREAD) {
#pragma unroll
      for (int k = 0; k < NP; ++k) issue_part(islot, k);
    }
    const uint8_t* st = lds + cs * PC::STAGE;
    cs = cs + 1 == NSTAGE ? 0 : cs + 1;
    // The step's work for the wave's first NT 16-row token tiles (the
    // others lie past the item's last row and are skipped; the stage is
    // issued the same way in every variant).  Every fragment is read from
    // LDS up front, so the reads overlap each other and the MFMAs wait only
    // for their own operands (the step's scales first, then the token
    // fragments, then the weight fragments in MFMA group order).
    auto compute = [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;
      constexpr int NC = NM * RT;
      constexpr int PPC = (NP + NC - 1) / NC;   // DMA parts per MFMA group
      if constexpr (NT == 0) {
        if constexpr (SPREAD) {
#pragma unroll
          for (int k = 0; k < NP; ++k) issue_part(islot, k);
        }
        return;
      } else {
      float sa_raw[NT], sw_raw[NM];
      if constexpr (F == F_FP8_BLK) {
        const float* scl = (const float*)(st + PC::TOKB + PC::WTB);
#pragma unroll
        for (int m = 0; m < NM; ++m) sw_raw[m] = scl[(NW - 1) * 64 + (GATEUP ? m : (wrow0 / 128))];
#pragma unroll
        for (int t = 0; t < NT; ++t) sa_raw[t] = scl[trow0 + t * 16 + r16];
      }
      i32x8 bfr[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int row = trow0 + t * 16 + r16;
        const i32x4 lo = *(const i32x4*)(st + swz128(row, lg));
        const i32x4 hi = *(const i32x4*)(st + swz128(row, lg + 4));
        bfr[t] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      i32x8 afr[NM][RT];
      int sw[NM][RT];
      if constexpr (WT) {
        // K rows 8 lg + r16 / 4 (+4, +32, +36) of channel block
        // (wrow0 + 16 rt) / 16, 8-byte part r16 % 4: K elements 8 lg .. + 7
        // and 32 + 8 lg .. + 7 of channel wrow0 + 16 rt + r16, the token
        // fragments' K order
        const int r0 = 8 * lg + (r16 >> 2);
        const int sw0 = (r0 & 3) | (((r0 >> 3) & 1) << 2);   // the same for r0 + 4, + 32, + 36
        const uint32_t wl = (uint32_t)(uintptr_t)(lds_void*)(st + PC::TOKB) + r0 * 512 + 8 * (r16 & 3);
        uint32_t ad[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) ad[rt] = wl + 32 * (((wrow0 >> 4) + rt) ^ sw0);
        const KnFrags<RT> f = read_kn_frags<RT>(ad);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          sw[0][rt] = 0;
          const i32x2 a = f.v[4 * rt], b = f.v[4 * rt + 1], c = f.v[4 * rt + 2], d = f.v[4 * rt + 3];
          afr[0][rt] = (i32x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        }
      } else
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int R = m * NBC + wrow0 + rt * 16 + r16;     // LDS weight row of this lane
          sw[m][rt] = 0;
          if constexpr (PC::WROWB == 128) {
            const i32x4 lo = *(const i32x4*)(st + PC::TOKB + swz128(R, lg));
            const i32x4 hi = *(const i32x4*)(st + PC::TOKB + swz128(R, lg + 4));
            afr[m][rt] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            const i32x4 qv = *(const i32x4*)(st + PC::TOKB + swz64(R, lg));
            afr[m][rt] = (i32x8){qv[0], qv[1], qv[2], qv[3], 0, 0, 0, 0};
            sw[m][rt] = (st + PC::TOKB + PC::WTB + PC::ASB)[R * 4 + lg];
          }
        }
      if constexpr (F == F_FP8_BLK) {
        // 128x128 block scaling: each K step is one scale block, so every
        // product is formed unscaled and then added with its row's
        // (activation scale x weight block scale).  Products of one weight
        // row tile go to one of two register sets, and the scaling of one
        // set runs while the MFMAs of the other are in flight (the scale
        // products are formed after the first MFMA groups, so those wait
        // only for their fragments).
        float sc[NM][NT];
        f32x4 d[2][NT];
        // a wave issuing its MFMA groups goes first, so the other wave of
        // the SIMD fills the gaps with its LDS reads and scaling
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c <= NC; ++c) {
          if (c < NC) {
#pragma unroll
            for (int k = c * PPC; k < (c + 1) * PPC && k < NP; ++k) issue_part(islot, k);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NT; ++t)
              d[c & 1][t] = mfma_f8(afr[c / RT][c % RT], bfr[t], (f32x4){0.f, 0.f, 0.f, 0.f});
            __builtin_amdgcn_sched_barrier(0);
          }
          if (c == 1) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int t = 0; t < NT; ++t) sc[m][t] = sa_raw[t] * sw_raw[m];
          }
          if (c > 0) {
            const int pc = c - 1, pm = pc / RT, prt = pc % RT;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[pm][prt][t] += d[pc & 1][t] * sc[pm][t];
          }
        }
        __builtin_amdgcn_s_setprio(0);
      } else {
        int sbx[NT];
        if constexpr (F == F_MX) {
#pragma unroll
          for (int t = 0; t < NT; ++t) sbx[t] = (st + PC::TOKB + PC::WTB)[(trow0 + t * 16 + r16) * 4 + lg];
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int c = m * RT + rt;
            if (SPREAD) {
#pragma unroll
              for (int k = c * PPC; k < (c + 1) * PPC && k < NP; ++k) issue_part(islot, k);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if constexpr (F == F_MX)
                acc[m][rt][t] = mfma_f4f8_scaled(afr[m][rt], bfr[t], acc[m][rt][t], sw[m][rt], sbx[t]);
              else if constexpr (F == F_BF16)
                acc[m][rt][t] = mfma_bf16_pair(afr[m][rt], bfr[t], acc[m][rt][t]);
              else
                acc[m][rt][t] = mfma_f8(afr[m][rt], bfr[t], acc[m][rt][t]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      }
    };
    // Blocks split into two row halves: a wave whose half holds no row of
    // the item (rows are padded to 128 per block, and most of the padding
    // sits in the blocks of experts with few tokens) only issues its
    // stage loads.  (Finer variants, per 16-row tile, cost register copies
    // of the accumulators at every step.)
    if constexpr (WM > 1) {
      if (((j & 1) ? m_odd : m_even) <= trow0) compute(std::integral_constant<int, 0>{});
      else compute(std::integral_constant<int, TT>{});
    } else {
      compute(std::integral_constant<int, TT>{});
    }
    if (iss && si != 0) advance(si);
    if (++s < ns) continue;

    // ------------------------------------------------------------ epilogue
    // lane: channel c0 + rt*16 + 4*lg + i, token row trow0 + t*16 + r16
    const It cur = info(j);
    const int m0 = cur.m0, M = cur.M;
    const int c0 = cur.cbase + wrow0;
    const float* asj = as_l + (j & 1) * RB;
    const float* rwj = rw_l + (j & 1) * RB;
    if constexpr (F == F_FP8_CH) {
      const float* csj = cs_l + (j & 1) * 256;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sxt = asj[trow0 + t * 16 + r16];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f32x4 wsv = *(const f32x4*)(csj + m * NBC + wrow0 + rt * 16 + 4 * lg);
            acc[m][rt][t] = acc[m][rt][t] * sxt * wsv;
          }
      }
    }
    // Prefill tiles regroup their outputs for wider stores (decode tiles,
    // whose rows are few, measured faster with the direct stores).
    constexpr bool REGROUP = BM >= 128;
    if constexpr (!GATEUP) {
      if (REGROUP && p.row_w) {
        // Weighted bf16 slot rows.  The MFMA layout gives a lane 4 channels
        // of each 16-channel tile (16 rows x 32 B per store); two lane swaps
        // per dword regroup them so lane lg holds channels 8lg..8lg+7 of
        // each 32-channel half, and each 16-byte store covers 16 rows x 64 B.
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = trow0 + t * 16 + r16;
          const int slot = m0 + r;
          const float w = (r < M && slot < p.row_w_n) ? rwj[r] : 1.0f;
          uint32_t pk[RT][2];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f32x4 vw = acc[0][rt][t] * w;
            pk[rt][0] = pack_bf16x2(vw[0], vw[1]);
            pk[rt][1] = pack_bf16x2(vw[2], vw[3]);
          }
#pragma unroll
          for (int h = 0; h < RT / 2; ++h) {
            uint32_t o[4];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              const uint2 q = regroup32(pk[2 * h][x], pk[2 * h + 1][x]);
              o[x] = q.x;
              o[2 + x] = q.y;
            }
            if (r < M)
              *(uint4*)((uint16_t*)p.out + (size_t)slot * N + c0 + 32 * h + 8 * lg) =
                  make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      } else {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int r = trow0 + t * 16 + r16;
        if (r >= M) continue;
        const int slot = m0 + r;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const f32x4 v = acc[0][rt][t];
          const int n0 = c0 + rt * 16 + 4 * lg;
          if (p.row_w) {
            const float w = slot < p.row_w_n ? rwj[r] : 1.0f;
            const f32x4 vw = v * w;
            const uint32_t lo = pack_bf16x2(vw[0], vw[1]);
            const uint32_t hi = pack_bf16x2(vw[2], vw[3]);
            *(uint2*)((uint16_t*)p.out + (size_t)slot * N + n0) = make_uint2(lo, hi);
          } else {
            *(f32x4*)((float*)p.out + (size_t)slot * N + n0) = v;
          }
        }
      }
      }
    } else {
      if constexpr (ACT == ACT_SWIGLU) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[0][rt][t][i] = silu(acc[0][rt][t][i]) * acc[1][rt][t][i];
      } else {
        const float L = p.act_limit;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[0][rt][t][i] = gated_act<ACT>(L, acc[0][rt][t][i], acc[1][rt][t][i]);
      }
      if constexpr (F == F_BF16) {
        // bf16 intermediate rows, regrouped as in the down projection's
        // store (16 rows x 64 B per 16-byte store)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = trow0 + t * 16 + r16;
          uint32_t pk[RT][2];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            pk[rt][0] = pack_bf16x2(acc[0][rt][t][0], acc[0][rt][t][1]);
            pk[rt][1] = pack_bf16x2(acc[0][rt][t][2], acc[0][rt][t][3]);
          }
#pragma unroll
          for (int h = 0; h < RT / 2; ++h) {
            uint32_t o[4];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              const uint2 q = regroup32(pk[2 * h][x], pk[2 * h + 1][x]);
              o[x] = q.x;
              o[2 + x] = q.y;
            }
            if (r < M)
              *(uint4*)((uint16_t*)p.out + (size_t)(m0 + r) * N + c0 + 32 * h + 8 * lg) =
                  make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      } else if constexpr (F == F_FP8_CH) {
  #pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = trow0 + t * 16 + r16;
          if (r >= M) continue;
          float* orow = (float*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) *(f32x4*)(orow + c0 + rt * 16 + 4 * lg) = acc[0][rt][t];
        }
      } else if constexpr (F == F_FP8_BLK && REGROUP) {
        // 1x128 group = the item's 128 channels, spread over the WN waves
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          float mx = 0.f;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[0][rt][t][i]));
          mx = max_over_rows(mx);
          if (lg == 0) amax_l[wn * BM + trow0 + t * 16 + r16] = mx;
        }
        // LDS-only exchange: the stage loads in flight must not be waited for
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        raw_barrier();
        const int nb = cur.cbase / 128;
        // codes regrouped as in the down projection's store: lane lg writes
        // channels 8lg..8lg+7 of each 32-channel half (16 rows x 32 B per
        // store instead of 16 rows x 16 B)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = trow0 + t * 16 + r16;
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) a = fmaxf(a, amax_l[w * BM + r]);
          const float sc = a > 0.f ? a / 448.0f : 1.0f;
          const float isc = 1.0f / sc;
          uint32_t cd[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const f32x4 h = acc[0][rt][t];
            cd[rt] = cvt4_e4m3(h[0] * isc, h[1] * isc, h[2] * isc, h[3] * isc);
          }
          uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
          for (int hh = 0; hh < RT / 2; ++hh) {
            const uint2 q = regroup32(cd[2 * hh], cd[2 * hh + 1]);
            if (r < M) *(uint2*)(orow + c0 + 32 * hh + 8 * lg) = q;
          }
          if (r < M && wn == 0 && lg == 0) ((float*)p.out_scale)[(size_t)(m0 + r) * (N / 128) + nb] = sc;
        }
      } else if constexpr (F == F_FP8_BLK) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          float mx = 0.f;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[0][rt][t][i]));
          mx = max_over_rows(mx);
          if (lg == 0) amax_l[wn * BM + trow0 + t * 16 + r16] = mx;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        raw_barrier();
        const int nb = cur.cbase / 128;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = trow0 + t * 16 + r16;
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) a = fmaxf(a, amax_l[w * BM + r]);
          const float sc = a > 0.f ? a / 448.0f : 1.0f;
          const float isc = 1.0f / sc;
          if (r < M) {
            uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const f32x4 h = acc[0][rt][t];
              *(uint32_t*)(orow + c0 + rt * 16 + 4 * lg) =
                  cvt4_e4m3(h[0] * isc, h[1] * isc, h[2] * isc, h[3] * isc);
            }
            if (wn == 0 && lg == 0) ((float*)p.out_scale)[(size_t)(m0 + r) * (N / 128) + nb] = sc;
          }
        }
      } else {   // F_MX: 32-channel groups = row-tile pairs of this wave
  #pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int r = trow0 + t * 16 + r16;
#pragma unroll
          for (int gp = 0; gp < RT / 2; ++gp) {
            float mx = 0.f;
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[0][2 * gp + qq][t][i]));
            mx = max_over_rows(mx);
            int ex = mx > 0.f ? ilog2_floor(mx) - 8 : -127;
            ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
            const float inv = __builtin_ldexpf(1.0f, -ex);
            if (r < M) {
              uint8_t* orow = (uint8_t*)p.out + (size_t)(m0 + r) * N;
#pragma unroll
              for (int qq = 0; qq < 2; ++qq) {
                const f32x4 h = acc[0][2 * gp + qq][t];
                *(uint32_t*)(orow + c0 + (2 * gp + qq) * 16 + 4 * lg) =
                    cvt4_e4m3(h[0] * inv, h[1] * inv, h[2] * inv, h[3] * inv);
              }
              if (lg == 0) ((uint8_t*)p.out_scale)[(size_t)(m0 + r) * (N / 32) + (c0 + 32 * gp) / 32] = (uint8_t)(ex + 127);
            }
          }
        }
      }
    }
    s = 0;
    ++j;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[m][rt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  // the stages issued past the last item land before the workgroup's LDS is
  // released
  wait_vm_c<0>();
}

// Tile shape of each row-block height (per format and op):
//   32/64 rows (decode-sized groups), four waves as 1x4: gate/up items of
//            128 channels (256 weight rows), or 64 channels for per-channel
//            FP8 (it requantises in a separate pass, so the 1x128 group
//            constraint does not apply); down items of 128 channels;
//   128 rows (prefill), waves per Pipe8Waves: gate/up items of 128
//            channels, down items of 256 channels when H allows, else 128.
// Wave layout of the 128-row blocks: eight waves as 2x4 (two per SIMD) for
// the FP8 formats, whose per-step scaling and LDS waits one wave hides
// behind the other's MFMAs; four waves as 1x4 for MXFP4 (the hardware
// applies its scales, and 128-row wave tiles read fewer fragments per
// MFMA: measured ~3% faster, while FP8 128x128 blocks ran ~30% slower).
template <int F>
struct Pipe8Waves {
  static constexpr int WM = F == F_MX ? 1 : 2;
  static constexpr int NW = F == F_MX ? 4 : 8;
};

template <int F, bool GATEUP>
struct PipeShapes {
  static constexpr int NR_SMALL = (GATEUP && F != F_FP8_CH) ? 256 : 128;
  // MXFP4's 128-row blocks also run four waves, so one kernel holds all
  // three tiled configurations (no launch that returns at once)
  static constexpr bool ONE_KERNEL = Pipe8Waves<F>::NW == 4;
  static constexpr int LDS4 = [] {
    const int a = pipe_lds_bytes<F, GATEUP, 32, NR_SMALL, 1, 4>();
    const int b = pipe_lds_bytes<F, GATEUP, 64, NR_SMALL, 1, 4>();
    int m = a > b ? a : b;
    if constexpr (ONE_KERNEL) {
      const int c = pipe_lds_bytes<F, GATEUP, 128, 256, 1, 4>();
      int d = 0;
      if constexpr (!GATEUP) d = pipe_lds_bytes<F, GATEUP, 128, 128, 1, 4>();
      m = m > c ? m : c;
      m = m > d ? m : d;
    }
    return m;
  }();
  static constexpr int LDS8 = [] {
    constexpr int WM = Pipe8Waves<F>::WM, NW = Pipe8Waves<F>::NW;
    const int c = pipe_lds_bytes<F, GATEUP, 128, 256, WM, NW>();
    int d = 0;
    if constexpr (!GATEUP) d = pipe_lds_bytes<F, GATEUP, 128, 128, WM, NW>();
    return c > d ? c : d;
  }();
};

// The device's configuration choice (meta) selects the tile shape: this
// kernel serves configurations 1 and 2 (and 3 when its blocks also run four
// waves) and returns at once for the others.
template <int F, bool GATEUP, int ACT>
__global__ void __launch_bounds__(256) k_gemm_pipe(GemmArgs p) {
  using SH = PipeShapes<F, GATEUP>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SH::LDS4];
  const int cfg = p.meta[META_CFG];
  if (p.cfg_self >= 0 && cfg != p.cfg_self) return;
  if (cfg == 1) pipe_body<F, GATEUP, 32, SH::NR_SMALL, 1, 4, ACT>(p, lds);
  else if (cfg == 2) pipe_body<F, GATEUP, 64, SH::NR_SMALL, 1, 4, ACT>(p, lds);
  else if constexpr (SH::ONE_KERNEL) {
    if (cfg == 3) {
      if (GATEUP || p.N % 256 == 0) pipe_body<F, GATEUP, 128, 256, 1, 4, ACT>(p, lds);
      else if constexpr (!GATEUP) pipe_body<F, GATEUP, 128, 128, 1, 4, ACT>(p, lds);
    }
  }
}

// Configuration 3 (128-row blocks).
// WT: K-major bf16 weights (GemmArgs::w_kn), N a multiple of 256.
template <int F, bool GATEUP, int ACT, bool WT = false>
__global__ void __launch_bounds__(Pipe8Waves<F>::NW * 64) k_gemm_pipe8(GemmArgs p) {
  using SH = PipeShapes<F, GATEUP>;
  constexpr int WM = Pipe8Waves<F>::WM, NW = Pipe8Waves<F>::NW;
  if constexpr (SH::ONE_KERNEL) {
    return;   // configuration 3 runs inside k_gemm_pipe
  } else {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[SH::LDS8];
    const int cfg = p.meta[META_CFG];
    if (cfg != 3 || (p.cfg_self >= 0 && cfg != p.cfg_self)) return;
    if constexpr (WT) pipe_body<F, GATEUP, 128, 256, WM, NW, ACT, true>(p, lds);
    else if (GATEUP || p.N % 256 == 0) pipe_body<F, GATEUP, 128, 256, WM, NW, ACT>(p, lds);
    else if constexpr (!GATEUP) pipe_body<F, GATEUP, 128, 128, WM, NW, ACT>(p, lds);
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
hipError_t launch_pipe_t(int family, const GemmArgs& g, hipStream_t st) {
  if (g.N % (GATEUP ? 64 : 128) || g.K % 128) return hipErrorInvalidValue;
  if (GATEUP && F != F_FP8_CH && g.N % 128) return hipErrorInvalidValue;
  // persistent grid: one workgroup per CU (the stage ring fills the LDS),
  // a multiple of the 8 XCDs
  const unsigned grid = (unsigned)pipe_cus();
  const dim3 b8(Pipe8Waves<F>::NW * 64);
  // one kernel holds every tiled configuration for this format: family 1
  // (configuration 3) is the same launch as family 0
  if (PipeShapes<F, GATEUP>::ONE_KERNEL) family = 0;
  if constexpr (GATEUP) {
    return with_act(g.act, [&](auto a) {
      constexpr int ACT = decltype(a)::value;
      if (family == 0) hipLaunchKernelGGL((k_gemm_pipe<F, true, ACT>), dim3(grid), dim3(256), 0, st, g);
      else hipLaunchKernelGGL((k_gemm_pipe8<F, true, ACT>), dim3(grid), b8, 0, st, g);
      return hipGetLastError();
    });
  } else {
    if constexpr (F == F_BF16) {
      if (g.w_kn) {   // K-major weights: configuration 3 only, 256-channel items
        if (family != 1 || g.cfg_self != 3 || g.N % 256 || g.w_k0 <= 0 || g.w_k0 > g.K ||
            g.w_k0 % 64 || (g.w_k0 < g.K && !g.w1) || g.sh_w0)
          return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_gemm_pipe8<F, false, ACT_SWIGLU, true>), dim3(grid), b8, 0, st, g);
        return hipGetLastError();
      }
    }
    if (family == 0) hipLaunchKernelGGL((k_gemm_pipe<F, false, ACT_SWIGLU>), dim3(grid), dim3(256), 0, st, g);
    else hipLaunchKernelGGL((k_gemm_pipe8<F, false, ACT_SWIGLU>), dim3(grid), b8, 0, st, g);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_gemm_pipe(int fmt, bool gateup, int family, const GemmArgs& g, hipStream_t st) {
  switch (fmt) {
    case F_FP8_CH:
      return gateup ? launch_pipe_t<F_FP8_CH, true>(family, g, st) : launch_pipe_t<F_FP8_CH, false>(family, g, st);
    case F_FP8_BLK:
      return gateup ? launch_pipe_t<F_FP8_BLK, true>(family, g, st) : launch_pipe_t<F_FP8_BLK, false>(family, g, st);
    case F_MX:
      return gateup ? launch_pipe_t<F_MX, true>(family, g, st) : launch_pipe_t<F_MX, false>(family, g, st);
    case F_BF16:
      return gateup ? launch_pipe_t<F_BF16, true>(family, g, st) : launch_pipe_t<F_BF16, false>(family, g, st);
  }
  return hipErrorInvalidValue;
}
