// Backward of the routed expert layer in bf16 (LightMoE README, "MoE
// training" and "Highlights": deterministic dispatch, combine, input-,
// weight- and router-gradient kernels).  Per slot (t, j) of expert e, with
// the forward g = Wg x_t, u = Wu x_t, h = act(g, u), o = Wd h and
// y_t = sum_j w[t, j] o:
//   r  = Wd^T dy_t                    (grouped GEMM, B not transposed)
//   dw = <r, h>,  dg = w r dact/dg,  du = w r dact/du   (per-slot pass)
//   da = Wg^T dg + Wu^T du            (grouped GEMM, B not transposed)
//   dx_t = sum_j da, j ascending      (dispatch backward)
//   dWd[e] = sum_slots (w dy_t) h^T, dWg[e] = sum dg x^T, dWu[e] = sum du x^T
//                                     (weight-gradient GEMMs over each group's rows)
// g and u are recomputed by the forward's tiled bf16 grouped GEMM.  Every
// sum has a fixed order (no atomics), so the gradients are bit-for-bit
// reproducible.
//
// MFMA operand layout (16x16x32 bf16): lane l feeds row (or column) l % 16
// with K elements [8 (l/16), 8 (l/16) + 8); the result lane l holds rows
// 4 (l/16) .. +3 of column l % 16.  The two new GEMM shapes need some
// operand with K strided in memory (B row-major [K, N] for the input
// gradients; both operands for the weight gradients, whose K runs over a
// group's rows): those tiles are transposed on their way into LDS, so
// every fragment read is one 16-byte LDS read.
#include "layer.h"

namespace {

constexpr int BT = 256;            // threads per workgroup (four waves)
constexpr int KS = 32;             // K elements per step (one MFMA deep)
constexpr int PK = KS + 8;         // LDS pitch of a transposed row, bf16 elements

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
// Input-gradient GEMM over expert row groups, B not transposed:
//   out[slot, n] = sum_src sum_k A_src[row(slot), k] * B_src[e][k, n]
// B_src[e] is [K, N] row-major (the stored [N_fwd, K_fwd] weight read along
// its first axis).  Work item = (row block of 64 rows from the block table,
// 128 output columns); four waves as 2 x 2, each 32 rows x 64 columns.
template <int NSRC>
__global__ void __launch_bounds__(BT) k_bwd_nn(BwdNN p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[64 * PK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * PK];   // [n][k]
  const int tile = blockIdx.y;
  if (tile >= p.meta[META_NTILES]) return;
  const int grp = p.tiles[2 * tile], r0 = p.tiles[2 * tile + 1];
  const int cnt = p.counts[grp], base = p.indptr[grp];
  const int n0 = blockIdx.x * 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;   // wave's 32-row and 64-column block
  const int K = p.K, N = p.N;
  // staging assignment: A: one 16-byte chunk (8 k) of one row per thread;
  // B: two 8-column chunks of one k row per thread
  const int ar = tid >> 2, ak = (tid & 3) * 8;
  const int rrow = r0 + ar;
  const bool av = rrow < cnt;
  const int slot = base + (av ? rrow : 0);
  const long arow = p.a_gather ? p.a_gather[slot] / p.gather_div : slot;
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int steps = NSRC * (K / KS);
  u16x8 ra, rb[2];
  auto gload = [&](int st) {
    const int src = st / (K / KS), k0 = (st - src * (K / KS)) * KS;
    const uint16_t* A = src ? p.a1 : p.a0;
    const uint16_t* B = (src ? p.b1 : p.b0) + (size_t)grp * K * N;
    ra = av ? *(const u16x8*)(A + arow * K + k0 + ak) : (u16x8){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = tid + c * BT;             // 512 chunks: 32 k rows x 16 chunks
      const int kr = q >> 4, nc = (q & 15) * 8;
      rb[c] = *(const u16x8*)(B + (size_t)(k0 + kr) * N + n0 + nc);
    }
  };
  gload(0);
  for (int st = 0; st < steps; ++st) {
    __syncthreads();   // the previous step's fragment reads are done
    *(u16x8*)(As + ar * PK + ak) = ra;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = tid + c * BT, kr = q >> 4, nc = (q & 15) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) Bs[(nc + i) * PK + kr] = rb[c][i];
    }
    __syncthreads();
    if (st + 1 < steps) gload(st + 1);   // in flight while this step computes
    const int g8 = (lane >> 4) * 8, l16 = lane & 15;
    bf16x8 fa[2], fb[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = as_bf16x8(*(const u16x8*)(As + (wr * 32 + i * 16 + l16) * PK + g8));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = as_bf16x8(*(const u16x8*)(Bs + (wc * 64 + j * 16 + l16) * PK + g8));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
  }
  // lane holds rows 4 (lane/16) .. +3 of column lane % 16 of each 16x16 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = r0 + wr * 32 + i * 16 + (lane >> 4) * 4 + r;
      if (rr >= cnt) continue;
      float* o = p.out + (size_t)(base + rr) * N + n0 + wc * 64 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j * 16] = acc[i][j][r];
    }
}

// ---------------------------------------------------------------------------
// Weight-gradient GEMM over expert row groups:
//   out[e][m, n] = sum over rows s of group e of A[s, m] * B[brow(s), n]
// A [rows, M] and B [*, N] bf16 row-major (brow = b_gather[s] / div, or s).
// Work item = (expert, 128 x 128 output block); four waves as 2 x 2, each
// 64 x 64.  K runs over the group's rows in ascending order, 32 per step;
// experts without rows write zeros.
__global__ void __launch_bounds__(BT) k_bwd_tn(BwdTN p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[128 * PK];   // [m][s]
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * PK];   // [n][s]
  const int e = blockIdx.z, m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, N = p.N;
  const int base = p.indptr[e], cnt = p.indptr[e + 1] - base;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // staging: 32 rows x 128 columns per operand = 512 chunks of 8 columns,
  // two per thread
  u16x8 ra[2], rb[2];
  auto gload = [&](int s0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = tid + c * BT, sr = q >> 4, cc = (q & 15) * 8;
      const int s = s0 + sr;
      if (s < cnt) {
        const long arow = base + s;
        const long brow = p.b_gather ? p.b_gather[base + s] / p.gather_div : base + s;
        ra[c] = *(const u16x8*)(p.a + arow * M + m0 + cc);
        rb[c] = *(const u16x8*)(p.b + brow * N + n0 + cc);
      } else {
        ra[c] = (u16x8){0, 0, 0, 0, 0, 0, 0, 0};
        rb[c] = ra[c];
      }
    }
  };
  const int steps = (cnt + KS - 1) / KS;
  if (steps > 0) gload(0);
  for (int st = 0; st < steps; ++st) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int q = tid + c * BT, sr = q >> 4, cc = (q & 15) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        As[(cc + i) * PK + sr] = ra[c][i];
        Bs[(cc + i) * PK + sr] = rb[c][i];
      }
    }
    __syncthreads();
    if (st + 1 < steps) gload((st + 1) * KS);
    const int g8 = (lane >> 4) * 8, l16 = lane & 15;
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = as_bf16x8(*(const u16x8*)(As + (wm * 64 + i * 16 + l16) * PK + g8));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = as_bf16x8(*(const u16x8*)(Bs + (wn * 64 + j * 16 + l16) * PK + g8));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
  }
  float* out = p.out + (size_t)e * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
      float* o = out + (size_t)m * N + n0 + wn * 64 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j * 16] = acc[i][j][r];
    }
}

// ---------------------------------------------------------------------------
// Per-slot pass: h = bf16(act(g, u)), dw = <r, h> (fixed-order block
// reduction), dg = bf16(w r dact/dg), du = bf16(w r dact/du), and the
// weighted upstream row w dy_t in bf16.  One workgroup per slot.
__global__ void __launch_bounds__(BT) k_bwd_slot(BwdSlot p) {
  __shared__ float red[BT];
  const int s = blockIdx.x;
  if (s >= p.indptr[p.E]) return;
  const int tid = threadIdx.x;
  const int pos = p.gather[s];                 // t * k + j
  const int t = pos / p.k;
  const float w = p.topk_w[pos];
  const int I = p.I, H = p.H;
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
    p.DG[o] = f32_to_bf16(dh * pg);
    p.DU[o] = f32_to_bf16(dh * pu);
  }
  for (int c = tid; c < H; c += BT)
    p.DO[(size_t)s * H + c] = f32_to_bf16(w * bf16_to_f32(p.dy[(size_t)t * H + c]));
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
  v.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  v.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
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
hipError_t launch_bwd_nn(const BwdNN& a, int nsrc, int max_tiles, hipStream_t st) {
  if (a.N % 128 || a.K % KS || max_tiles <= 0) return hipErrorInvalidValue;
  dim3 grid(a.N / 128, max_tiles);
  if (nsrc == 2) hipLaunchKernelGGL(k_bwd_nn<2>, grid, dim3(BT), 0, st, a);
  else hipLaunchKernelGGL(k_bwd_nn<1>, grid, dim3(BT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_tn(const BwdTN& a, int E, hipStream_t st) {
  if (a.M % 128 || a.N % 128 || E <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bwd_tn, dim3(a.N / 128, a.M / 128, E), dim3(BT), 0, st, a);
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
