// Backward of the routed expert layer in bf16 (LightMoE README, "MoE
// training" and "Highlights": deterministic dispatch, combine, input-,
// weight- and router-gradient kernels).  Per slot (t, j) of expert e, with
// the forward g = Wg x_t, u = Wu x_t, h = act(g, u), o = Wd h and
// y_t = sum_j w[t, j] o:
//   r  = Wd^T dy_t                    (input-gradient GEMM)
//   dw = <r, h>,  dg = w r dact/dg,  du = w r dact/du   (per-slot pass)
//   da = Wg^T dg + Wu^T du            (input-gradient GEMM, K = 2 I)
//   dx_t = sum_j da, j ascending      (dispatch backward)
//   dWd[e] = sum_slots (w dy_t) h^T, dWg[e] = sum dg x^T, dWu[e] = sum du x^T
//                                     (weight-gradient GEMMs over each group's rows)
// Every sum has a fixed order (no atomics), so the gradients are
// bit-for-bit reproducible.
//
// Layout.  A 16x16x32 bf16 MFMA takes, per lane, 8 consecutive elements of
// the contraction (K) dimension: lane l feeds row (or column) l % 16 with K
// elements [8 (l/16), 8 (l/16) + 8); the result lane l holds rows
// 4 (l/16) .. +3 of column l % 16.  The forward's tiled grouped GEMM wants
// its weights [N, K] with K contiguous; the input gradients contract the
// stored weights along their other axis, so the active experts' weights are
// transposed once per call (k_bwd_transpose) and the forward kernel runs
// the input gradients, and the gate/up recomputation, unchanged.  The
// weight gradients contract over a group's rows, so their operands (w dy,
// h, dg | du, gathered x) are written feature-major (slots contiguous) by
// the same transpose, and k_bwd_wgrad loads MFMA fragments straight from
// memory.
#include "layer.h"

namespace {

constexpr int BT = 256;            // threads per workgroup (four waves)

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

DEVI bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

DEVI float sigm(float z) { return 1.0f / (1.0f + __expf(-z)); }

// The forward activation in fp32, as the forward epilogues compute it.
DEVI float act_f(int act, float L, float g, float u) {
  switch (act) {
    case ACT_SWIGLU_BOUNDED: {
      const float gc = fminf(g, L), uc = fminf(fmaxf(u, -L), L);
      return gc * sigm(gc) * uc;
    }
    case ACT_SWIGLU_OAI: {
      const float gc = fminf(g, L), uc = fminf(fmaxf(u, -L), L);
      return gc * sigm(1.702f * gc) * (uc + 1.0f);
    }
    case ACT_GEGLU:
      return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f)) * u;
    case ACT_RELU2:
      return u > 0.0f ? u * u : 0.0f;
    default:
      return g * sigm(g) * u;
  }
}

// Partial derivatives of the activation with respect to g and u.  At a
// clamp boundary the branch the forward takes: min(g, L) passes g only for
// g < L, clamp(u, -L, L) passes u for -L <= u <= L.
DEVI void act_grad(int act, float L, float g, float u, float* dg, float* du) {
  switch (act) {
    case ACT_SWIGLU_BOUNDED: {
      const bool gin = g < L, uin = u >= -L && u <= L;
      const float gc = gin ? g : L, uc = fminf(fmaxf(u, -L), L), s = sigm(gc);
      *dg = gin ? s * (1.0f + gc * (1.0f - s)) * uc : 0.0f;
      *du = uin ? gc * s : 0.0f;
      return;
    }
    case ACT_SWIGLU_OAI: {
      const bool gin = g < L, uin = u >= -L && u <= L;
      const float gc = gin ? g : L, uc = fminf(fmaxf(u, -L), L), s = sigm(1.702f * gc);
      *dg = gin ? (s + 1.702f * gc * s * (1.0f - s)) * (uc + 1.0f) : 0.0f;
      *du = uin ? gc * s : 0.0f;
      return;
    }
    case ACT_GEGLU: {
      const float Phi = 0.5f * (1.0f + erff(g * 0.70710678118654752f));
      const float phi = __expf(-0.5f * g * g) * 0.39894228040143268f;   // 1 / sqrt(2 pi)
      *dg = (Phi + g * phi) * u;
      *du = g * Phi;
      return;
    }
    case ACT_RELU2:
      *dg = 0.0f;
      *du = u > 0.0f ? 2.0f * u : 0.0f;
      return;
    default: {
      const float s = sigm(g);
      *dg = s * (1.0f + g * (1.0f - s)) * u;
      *du = g * s;
      return;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Tiled transpose of 64 x 64 blocks through LDS:
//   out[z][c][out_col0 + r] = bf16(scale(r) * in[z][row(r)][c]),  r < R, c < C,
// row(r) = gather ? gather[r] / gather_div : r; scale(r) = scale[gather[r]]
// (or 1).  Rows r in [R, 64 * ceil(R / 64)) are written as zeros, so a
// whole padded row of out is defined.  Matrices z with counts[z] == 0 are
// skipped.  Used for the weights (their [N, K] storage read along N) and
// for the per-slot operands of the weight gradients (slot-major to
// feature-major, so that the slot dimension is contiguous).
__global__ void __launch_bounds__(BT) k_bwd_transpose(BwdTranspose p) {
  __shared__ uint16_t t[64][64 + 2];
  const int z = blockIdx.z;
  if (p.counts && p.counts[z] == 0) return;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const uint16_t* in = p.in + (size_t)z * p.in_zstride;
  // load: 64 rows x 64 columns, two 8-column chunks per thread
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + q * BT, rr = i >> 3, cc = (i & 7) * 8;
    const int r = r0 + rr;
    u16x8 v = (u16x8){0, 0, 0, 0, 0, 0, 0, 0};
    if (r < p.R) {
      const long row = p.gather ? p.gather[r] / p.gather_div : r;
      v = *(const u16x8*)(in + row * p.in_ld + c0 + cc);
      if (p.scale) {
        const float sc = p.scale[p.gather[r]];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16(sc * bf16_to_f32(v[e]));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t[rr][cc + e] = v[e];
  }
  __syncthreads();
  // store: 64 output rows (columns c) x 64 r, eight r per 16-byte chunk
  uint16_t* out = p.out + (size_t)z * p.out_zstride;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + q * BT, cc = i >> 3, rr = (i & 7) * 8;
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[rr + e][cc];
    *(u16x8*)(out + (size_t)(c0 + cc) * p.out_ld + p.out_col0 + r0 + rr) = v;
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM over each group's slots:
//   out[e][m, n] = sum over s in [row0, row1) of a[s, m] * b[row_b(s), n]
// with the operands as the per-slot pass and the inputs store them: a
// [slots, lda] bf16, b [rows, ldb] bf16, row_b(s) = b_tok[s] (the token of
// slot s, for x) or s.  Work item = (chunk, 128 x 64 WN output block), one
// per workgroup; blockIdx.z walks the chunks longest first (a permutation
// from launch_bwd_chunks), so that the in-order dispatch of workgroups
// starts the long items early and the short ones fill the tail.  2 x WN
// waves, each 64 x 64 (WN = 4 where N allows: 256 columns per item read
// three quarters of the operand bytes per MFMA that 128 columns do).  Per
// step of 32 slots the workgroup copies the 32 slot rows of its columns of
// a and of b into a ring of LDS stages with asynchronous global->LDS loads,
// so the next steps' loads are in flight while this step's MFMAs run.  The
// MFMA wants 8 consecutive slots per lane for one column: LDS transpose
// reads (ds_read_b64_tr_b16) give them straight from the slot rows.  Within
// each 16-lane group, lane i of such a read receives element i % 4 of the
// 8-byte pieces addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and
// i / 4 + 12; with lane j addressing slot row kb + j / 4 at columns
// 4 (j % 4) .. + 3 of a 16-column block, lane i ends with slots kb .. kb + 3
// of column i.  The 32-byte blocks of a row are XOR-swizzled by the row so
// that the eight rows a half-wave reads sit in distinct banks.  Slots
// outside the range are masked on the a side after the LDS read (their
// rows are loaded from a valid row of the range).
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x2 __attribute__((ext_vector_type(2)));

// ring geometry per WN: a stage holds a (32 slots x 256 B) then b (32 slots
// x 128 WN bytes); 2 workgroups per CU
template <int WN> struct WgCfg {
  static constexpr int NWV = 2 * WN;                 // waves
  static constexpr int BROW = 128 * WN;              // b bytes per slot row
  static constexpr int STAGE = 8192 + 32 * BROW;
  static constexpr int NS = WN == 2 ? 4 : 3;         // stages
  static constexpr int IA = 8 / NWV;                 // a loads per wave per stage (4 rows each)
  static constexpr int RPB = 1024 / BROW;            // b rows per load
  static constexpr int IB = 32 / RPB / NWV;          // b loads per wave per stage
  static constexpr int LOADS = IA + IB;
  static_assert(IA * NWV * 4 == 32 && IB * NWV * RPB == 32, "whole loads per wave");
};

DEVI void dma16(const void* src, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_block, 16, 0, 0);
}
// 32-byte block swizzle of slot row r (distinct over rows 0-3 and 8-11)
DEVI int blk_swz(int r) { return (r & 3) | (((r >> 3) & 1) << 2); }
// The step's 16 transpose reads: for each of the 4 a addresses the rows at
// it and 4 rows (1024 bytes) further, for each of the 4 b addresses the
// rows at it and 4 rows (BOFF bytes) further.  One asm block that waits for
// its own reads before it ends, so every output is written when the block
// returns.  (The builtin form makes the compiler wait for every
// asynchronous global->LDS load in flight before each read, as it cannot
// tell them apart; the ring's own waits and barrier already cover the
// stage read here.)
struct Frags { i32x2 v[16]; };
#define WG_TR_READS(BOFF)                                                                     \
  asm volatile(                                                                               \
      "ds_read_b64_tr_b16 %0, %16\n"                                                          \
      "ds_read_b64_tr_b16 %1, %16 offset:1024\n"                                              \
      "ds_read_b64_tr_b16 %2, %17\n"                                                          \
      "ds_read_b64_tr_b16 %3, %17 offset:1024\n"                                              \
      "ds_read_b64_tr_b16 %4, %18\n"                                                          \
      "ds_read_b64_tr_b16 %5, %18 offset:1024\n"                                              \
      "ds_read_b64_tr_b16 %6, %19\n"                                                          \
      "ds_read_b64_tr_b16 %7, %19 offset:1024\n"                                              \
      "ds_read_b64_tr_b16 %8, %20\n"                                                          \
      "ds_read_b64_tr_b16 %9, %20 offset:" #BOFF "\n"                                         \
      "ds_read_b64_tr_b16 %10, %21\n"                                                         \
      "ds_read_b64_tr_b16 %11, %21 offset:" #BOFF "\n"                                        \
      "ds_read_b64_tr_b16 %12, %22\n"                                                         \
      "ds_read_b64_tr_b16 %13, %22 offset:" #BOFF "\n"                                        \
      "ds_read_b64_tr_b16 %14, %23\n"                                                         \
      "ds_read_b64_tr_b16 %15, %23 offset:" #BOFF "\n"                                        \
      "s_waitcnt lgkmcnt(0)"                                                                  \
      : "=&v"(f.v[0]), "=&v"(f.v[1]), "=&v"(f.v[2]), "=&v"(f.v[3]), "=&v"(f.v[4]),            \
        "=&v"(f.v[5]), "=&v"(f.v[6]), "=&v"(f.v[7]), "=&v"(f.v[8]), "=&v"(f.v[9]),            \
        "=&v"(f.v[10]), "=&v"(f.v[11]), "=&v"(f.v[12]), "=&v"(f.v[13]), "=&v"(f.v[14]),       \
        "=&v"(f.v[15])                                                                        \
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),   \
        "v"(ad[7])                                                                            \
      : "memory")
template <int WN> DEVI Frags read_tr16(const uint32_t (&ad)[8]) {
  Frags f;
  if constexpr (WN == 2) WG_TR_READS(1024);
  else WG_TR_READS(2048);
  return f;
}
#undef WG_TR_READS
DEVI u16x8 join_frag(i32x2 lo, i32x2 hi) {
  const i32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(u16x8, v);
}
// wait until at most n of this wave's asynchronous loads are pending
DEVI void wait_vm_steps(int n) {
  switch (n) {
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}
// workgroup barrier without __syncthreads()'s fence, which would also wait
// for the ring's loads in flight (each wave waits for its own first)
DEVI void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Eight consecutive token indices from index i through the scalar cache
// (the table comes from an earlier launch; the pointer goes through an
// integer so that the compiler keeps the constant address space).  A
// lane-dependent pick among them must stay a chain of register selects:
// folded into an indexed read, it becomes a private array that the
// compiler places in LDS, whose writes then wait for every asynchronous
// load in flight.
struct Tok8 { int t0, t1, t2, t3, t4, t5, t6, t7; };
DEVI Tok8 tok8(const int32_t* tok, int i) {
  typedef const __attribute__((address_space(4))) int cint;
  const cint* t = (const cint*)(uintptr_t)(tok + i);
  return Tok8{__builtin_amdgcn_readfirstlane(t[0]), __builtin_amdgcn_readfirstlane(t[1]),
              __builtin_amdgcn_readfirstlane(t[2]), __builtin_amdgcn_readfirstlane(t[3]),
              __builtin_amdgcn_readfirstlane(t[4]), __builtin_amdgcn_readfirstlane(t[5]),
              __builtin_amdgcn_readfirstlane(t[6]), __builtin_amdgcn_readfirstlane(t[7])};
}
// value k of a Tok8 (k a compile-time constant after unrolling)
DEVI int tok_at(const Tok8& t, int k) {
  switch (k) {
    case 0: return t.t0;
    case 1: return t.t1;
    case 2: return t.t2;
    case 3: return t.t3;
    case 4: return t.t4;
    case 5: return t.t5;
    case 6: return t.t6;
    default: return t.t7;
  }
}

}  // namespace

template <int WN>
__global__ void __launch_bounds__(128 * WN) k_bwd_wgrad(BwdWgrad p) {
  using C = WgCfg<WN>;
  constexpr int NS = C::NS, STAGE = C::STAGE, BROW = C::BROW, IA = C::IA, IB = C::IB, RPB = C::RPB;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * STAGE];
  // work chunk: a group's whole row range, or one piece of it (split K)
  if ((int)blockIdx.z >= p.chunks[0]) return;
  const int z = p.order[blockIdx.z];
  const int4 ch = ((const int4*)(p.chunks + 4))[z];   // expert, first row, end row, partial
  const int e = ch.x, s0 = ch.y, s1 = ch.z;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 64 * WN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, l16 = lane & 15;
  const int sb = s0 & ~31;                 // first 32-aligned step
  const int steps = s1 > s0 ? (s1 - sb + 31) / 32 : 0;
  // DMA: per stage this wave loads a slot rows 4 (IA wave + ia) + lane / 16
  // and b slot rows RPB (IB wave + ib) + lane / (64 / RPB), 16 bytes each;
  // a lane's LDS place is 16-byte piece q of its row, holding source piece
  // 2 ((q / 2) ^ swz(row)) + q % 2 of the row's columns
  auto src_piece = [&](int row, int q) { return 2 * ((q >> 1) ^ blk_swz(row)) + (q & 1); };
  uint32_t aoff[IA], boff[IB];
  int arow[IA], brow[IB];
#pragma unroll
  for (int ia = 0; ia < IA; ++ia) {
    arow[ia] = 4 * (IA * wave + ia) + (lane >> 4);
    aoff[ia] = 16 * src_piece(arow[ia], lane & 15);
  }
#pragma unroll
  for (int ib = 0; ib < IB; ++ib) {
    brow[ib] = RPB * (IB * wave + ib) + lane / (64 / RPB);
    boff[ib] = 16 * src_piece(brow[ib], lane % (64 / RPB));
  }
  const uint8_t* a_col = (const uint8_t*)(p.a + m0);
  const uint8_t* b_col = (const uint8_t*)(p.b + n0);
  const int tbase = RPB * IB * wave;       // this wave's first b row in a stage
  Tok8 tk{};
  if (p.b_tok && steps > 0) tk = tok8(p.b_tok, sb + tbase);
  auto issue = [&](int st) {
    uint8_t* stg = ring + (st % NS) * STAGE;
    const int sr = sb + st * 32;           // the stage's first slot row
#pragma unroll
    for (int ia = 0; ia < IA; ++ia) {
      const int s = sr + arow[ia];
      const int r = s < s1 ? s : s1 - 1;
      dma16(a_col + (size_t)r * p.lda * 2 + aoff[ia], stg + (IA * wave + ia) * 1024);
    }
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
      const int s = sr + brow[ib];
      const bool in = s < s1;
      int r = in ? s : s1 - 1;
      if (p.b_tok) {
        // row brow[ib] - tbase of the wave's rows: index RPB ib + sub,
        // sub = lane / (64 / RPB) (a select over registers, not an indexed
        // array, which would go to scratch)
        // (each candidate passes through an empty asm as a register value,
        // so the selects cannot be folded into one indexed load)
        const int sub = lane / (64 / RPB);
        int tv = tok_at(tk, RPB * ib);
        asm("" : "+s"(tv));
#pragma unroll
        for (int c = 1; c < RPB; ++c) {
          int vc = tok_at(tk, RPB * ib + c);
          asm("" : "+s"(vc));
          tv = sub == c ? vc : tv;
        }
        r = in ? tv : 0;
      }
      dma16(b_col + (size_t)r * p.ldb * 2 + boff[ib], stg + 8192 + (IB * wave + ib) * 1024);
    }
    // the next stage's token indices (only read after the next barrier)
    if (p.b_tok && st + 1 < steps) tk = tok8(p.b_tok, sr + 32 + tbase);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // fragment reads: lane reads slot rows 8 g + l16 / 4 (+ 4) of the
  // fragment's 32-byte block, 8-byte part l16 % 4
  const int r0 = 8 * g + (l16 >> 2);
  const int hsw = blk_swz(r0);             // the same for r0 + 4
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_void*)ring;
  const uint32_t fa_off = ring_lds + r0 * 256 + 8 * (l16 & 3);
  const uint32_t fb_off = ring_lds + 8192 + r0 * BROW + 8 * (l16 & 3);
  for (int q = 0; q < NS - 1 && q < steps; ++q) issue(q);
  for (int st = 0; st < steps; ++st) {
    const int later = steps - 1 - st < NS - 2 ? steps - 1 - st : NS - 2;
    wait_vm_steps(C::LOADS * later);   // this step's stage has landed (this wave's part)
    raw_barrier();                     // ... and every wave's; the previous stage is free
    if (st + NS - 1 < steps) issue(st + NS - 1);
    const uint32_t so = (st % NS) * STAGE;
    uint32_t ad[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = fa_off + so + 32 * ((4 * wm + i) ^ hsw);
#pragma unroll
    for (int j = 0; j < 4; ++j) ad[4 + j] = fb_off + so + 32 * ((4 * wn + j) ^ hsw);
    const Frags fr = read_tr16<WN>(ad);
    u16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = join_frag(fr.v[2 * i], fr.v[2 * i + 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = join_frag(fr.v[8 + 2 * j], fr.v[9 + 2 * j]);
    const int c = sb + st * 32 + 8 * g;      // this lane's 8 slots
    if (c < s0 || c + 8 > s1) {             // a chunk at the range's ends
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c + k < s0 || c + k >= s1) fa[i][k] = 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j]);
  }
  // Lane: rows m0 + wm 64 + 16 i + 4 g + r of column n0 + wn 64 + 16 j + l16.
  // Each store covers 64 contiguous bytes of four rows (measured faster than
  // one 16-byte store per lane with the operands swapped).
  float* out = ch.w < 0 ? p.out + (size_t)e * p.M * p.N : p.partial + (size_t)ch.w * p.M * p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + g * 4 + r;
      float* o = out + (size_t)m * p.N + n0 + wn * 64 + l16;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j * 16] = acc[i][j][r];
    }
}

// Work chunks of the weight-gradient GEMM, from the group offsets: each
// expert's rows in pieces of at most `piece` rows (one piece, possibly
// empty, for an expert without rows).  Entry i: (expert, first row, end row,
// partial index), partial index -1 for an expert's first piece (written to
// the output) and consecutive indices for the rest; per expert its piece
// count and first partial index; and a permutation of the chunks by
// decreasing length in steps of 32 rows (lengths from 63 steps up share a
// bucket; the order within a bucket is arbitrary and does not affect any
// result).  One 256-thread block, a thread per expert, exclusive scans of
// the piece and partial counts in LDS (E <= 256).
__global__ void __launch_bounds__(256) k_bwd_chunks(const int32_t* indptr, int E, int piece,
                                                    int32_t* chunks, int32_t* nch, int32_t* pbase,
                                                    int32_t* multi, int32_t* order) {
  __shared__ int sp[256], sq[256], sm[256], hist[64];
  const int e = threadIdx.x;
  int s0 = 0, s1 = 0, pieces = 0;
  if (e < E) {
    s0 = indptr[e];
    s1 = indptr[e + 1];
    pieces = s1 > s0 ? (s1 - s0 + piece - 1) / piece : 1;
  }
  sp[e] = pieces;
  sq[e] = pieces > 0 ? pieces - 1 : 0;
  sm[e] = pieces > 1;
  if (e < 64) hist[e] = 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {      // inclusive scans
    const int a = e >= o ? sp[e - o] : 0, b = e >= o ? sq[e - o] : 0, c = e >= o ? sm[e - o] : 0;
    __syncthreads();
    sp[e] += a;
    sq[e] += b;
    sm[e] += c;
    __syncthreads();
  }
  if (pieces > 1) multi[sm[e]] = e;         // experts split in pieces, from multi[1]
  if (e == 255) multi[0] = sm[255];
  // bucket 63 - min(steps, 63) of a piece: longest first
  auto bucket = [&](int c) {
    const int a = s0 + c * piece, b = a + piece < s1 ? a + piece : s1;
    const int steps = b > a ? (b - (a & ~31) + 31) >> 5 : 0;
    return 63 - (steps < 63 ? steps : 63);
  };
  for (int c = 0; c < pieces; ++c) atomicAdd(&hist[bucket(c)], 1);
  const int first = sp[e] - pieces;
  if (e < E) {
    const int pfirst = sq[e] - (pieces - 1);
    nch[e] = pieces;
    pbase[e] = pfirst;
    int4* tab = (int4*)(chunks + 4);
    for (int c = 0; c < pieces; ++c) {
      const int a = s0 + c * piece, b = a + piece < s1 ? a + piece : s1;
      tab[first + c] = make_int4(e, a, b > a ? b : a, c == 0 ? -1 : pfirst + c - 1);
    }
  }
  if (e == 255) chunks[0] = sp[255];
  __syncthreads();
  if (e == 0) {                              // bucket starts
    int acc = 0;
    for (int k = 0; k < 64; ++k) {
      const int n = hist[k];
      hist[k] = acc;
      acc += n;
    }
  }
  __syncthreads();
  for (int c = 0; c < pieces; ++c) order[atomicAdd(&hist[bucket(c)], 1)] = first + c;
}

// out[e] += partial pieces 1.. of expert e, in piece order (a fixed order,
// so the sum is reproducible), for the experts the chunk table lists as
// split.  Four elements per thread.
__global__ void __launch_bounds__(BT) k_bwd_wgrad_reduce(BwdWgrad p) {
  const size_t MN = (size_t)p.M * p.N;
  const size_t i = ((size_t)blockIdx.x * BT + threadIdx.x) * 4;
  if (i >= MN) return;
  const int nm = p.multi[0];
  for (int q = 0; q < nm; ++q) {
    const int e = p.multi[1 + q], n = p.nch[e];
    f32x4* o = (f32x4*)(p.out + e * MN + i);
    f32x4 a = *o;
    for (int c = 0; c < n - 1; ++c) a += *(const f32x4*)(p.partial + (size_t)(p.pbase[e] + c) * MN + i);
    *o = a;
  }
}

// ---------------------------------------------------------------------------
// Per-slot pass: h = bf16(act(g, u)), dw = <r, h> (fixed-order block
// reduction), dg = bf16(w r dact/dg) and du = bf16(w r dact/du) side by
// side in one row of 2 I; and the weight gradients' slot rows
// wdy = bf16(w dy_t) and tok = t.  One workgroup per slot.
__global__ void __launch_bounds__(BT) k_bwd_slot(BwdSlot p) {
  __shared__ float red[BT];
  const int s = blockIdx.x;
  if (s >= p.indptr[p.E]) return;
  const int tid = threadIdx.x;
  const int pos = p.gather[s];                 // t * k + j
  const float w = p.topk_w[pos];
  const int tkn = pos / p.k;
  if (tid == 0) p.tok[s] = tkn;
  for (int c = tid * 8; c < p.H; c += BT * 8) {
    const u16x8 v = *(const u16x8*)(p.dy + (size_t)tkn * p.H + c);
    uint4 o;
    o.x = pack_bf16x2(w * bf16_to_f32(v[0]), w * bf16_to_f32(v[1]));
    o.y = pack_bf16x2(w * bf16_to_f32(v[2]), w * bf16_to_f32(v[3]));
    o.z = pack_bf16x2(w * bf16_to_f32(v[4]), w * bf16_to_f32(v[5]));
    o.w = pack_bf16x2(w * bf16_to_f32(v[6]), w * bf16_to_f32(v[7]));
    *(uint4*)(p.WDY + (size_t)s * p.H + c) = o;
  }
  const int I = p.I;
  float part = 0.0f;
  for (int n = tid; n < I; n += BT) {
    const size_t o = (size_t)s * I + n;
    const float g = p.G ? p.G[o] : 0.0f, u = p.U[o], r = p.R[o];
    const uint16_t hb = f32_to_bf16(act_f(p.act, p.limit, g, u));
    p.Hb[o] = hb;
    part += r * bf16_to_f32(hb);
    float pg, pu;
    act_grad(p.act, p.limit, g, u, &pg, &pu);
    const float dh = w * r;
    p.DGU[(size_t)s * 2 * I + n] = f32_to_bf16(dh * pg);
    p.DGU[(size_t)s * 2 * I + I + n] = f32_to_bf16(dh * pu);
  }
  red[tid] = part;
  __syncthreads();
  for (int o = BT / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) p.dw[pos] = red[0];
}

// dx_t = bf16(sum_j da[inv[t k + j]]), j ascending.  Four channels per thread.
__global__ void __launch_bounds__(BT) k_bwd_dx(BwdDx p) {
  const long i = (long)blockIdx.x * BT + threadIdx.x;
  const int H4 = p.H / 4;
  if (i >= (long)p.T * H4) return;
  const int t = (int)(i / H4), c = (int)(i - (long)t * H4) * 4;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < p.k; ++j) {
    const int slot = p.inv[t * p.k + j];
    a += *(const f32x4*)(p.DA + (size_t)slot * p.H + c);
  }
  uint2 v;
  v.x = pack_bf16x2(a[0], a[1]);
  v.y = pack_bf16x2(a[2], a[3]);
  *(uint2*)(p.dx + (size_t)t * p.H + c) = v;
}

// Router backward: one wave per token; lane e (strided) writes d_scores[t, e]:
// with m = sum_j w_j dw_j, a selected expert gets
//   softmax  w_i (dw_i - m);  sigmoid  s_i (1 - s_i) (dw_i - m) / sum_sel s;
//   probs    (dw_i - m) / sum_sel p;
// every other expert 0.
__global__ void __launch_bounds__(64) k_router_bwd(RouterBwd p) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int k = p.k, E = p.E;
  const int32_t* ids = p.ids + (size_t)t * k;
  const float* w = p.w + (size_t)t * k;
  const float* dw = p.dw + (size_t)t * k;
  const float* sc = p.scores + (size_t)t * E;
  float m = 0.0f, den = 0.0f;
  for (int j = 0; j < k; ++j) {
    m += w[j] * dw[j];
    const float l = sc[ids[j]];
    den += p.score_fn == 1 ? sigm(l) : l;
  }
  for (int e = lane; e < E; e += 64) {
    float v = 0.0f;
    for (int j = 0; j < k; ++j)
      if (ids[j] == e) {
        const float d = dw[j] - m, l = sc[e];
        if (p.score_fn == 0) v = w[j] * d;
        else if (p.score_fn == 1) v = sigm(l) * (1.0f - sigm(l)) * d / den;
        else v = d / den;
      }
    p.ds[(size_t)t * E + e] = v;
  }
}

// ---------------------------------------------------------------- host launchers
hipError_t launch_bwd_transpose(const BwdTranspose& a, int nz, hipStream_t st) {
  if (a.C % 64 || a.R <= 0 || nz <= 0) return a.R == 0 ? hipSuccess : hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bwd_transpose, dim3(a.C / 64, (a.R + 63) / 64, nz), dim3(BT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_chunks(const int32_t* indptr, int E, int piece, int32_t* chunks,
                             int32_t* nch, int32_t* pbase, int32_t* multi, int32_t* order,
                             hipStream_t st) {
  if (E <= 0 || piece <= 0) return hipErrorInvalidValue;
  if (E > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bwd_chunks, dim3(1), dim3(256), 0, st, indptr, E, piece, chunks, nch, pbase,
                     multi, order);
  return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const BwdWgrad& a, int E, int max_chunks, hipStream_t st) {
  if (a.M % 128 || a.N % 128 || E <= 0 || max_chunks <= 0 || a.lda % 8 || a.ldb % 8 ||
      (uintptr_t)a.a % 16 || (uintptr_t)a.b % 16)
    return hipErrorInvalidValue;
  if (a.N % 256 == 0)   // 128 x 256 items, eight waves
    hipLaunchKernelGGL(k_bwd_wgrad<4>, dim3(a.N / 256, a.M / 128, max_chunks), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(k_bwd_wgrad<2>, dim3(a.N / 128, a.M / 128, max_chunks), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_chunks == E) return e;   // one piece per expert: nothing to add
  const size_t MN = (size_t)a.M * a.N;
  hipLaunchKernelGGL(k_bwd_wgrad_reduce, dim3((unsigned)((MN / 4 + BT - 1) / BT)), dim3(BT), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_slot(const BwdSlot& a, int max_rows, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_slot, dim3(max_rows), dim3(BT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdDx& a, hipStream_t st) {
  if (a.H % 4) return hipErrorInvalidValue;
  const long n = (long)a.T * (a.H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_dx, dim3((unsigned)((n + BT - 1) / BT)), dim3(BT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwd& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_bwd, dim3(a.T), dim3(64), 0, st, a);
  return hipGetLastError();
}
