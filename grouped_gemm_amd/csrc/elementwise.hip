// Dynamic activation quantisation and the weighted top-k combine.
//
// Quantisation (LightMoE README, "MoE inference": BF16 input quantisation
// before the gate/up projection and requantisation of the intermediate;
// Alpha-MoE news page, "The MoE bottleneck": FP8 W8A8).  Per group of a
// row: a = max|v|; FP8 groups use the fp32 scale s = a/448 (1 when a = 0)
// and q = e4m3_rne(clamp(v/s, +-448)) with the correctly rounded fp32 quotient; MX groups (OCP MX
// v1.0) use X = 2^(floor(log2 a) - 8) stored as e8m0, and q = e4m3_rne_sat(v/X).
//
// Combine (LightMoE README, "MoE inference": routing-weight application and
// deterministic combine): y[t] = sum over j ascending of w[t,j] times the
// slot output of (t, j), plus the shared expert's row, rounded to bf16 once.
#include "layer.h"
#include "quant_row.h"

#include <type_traits>

template <int AF>
struct QGroup {
  static constexpr int CHUNKS = AF == MOE_A_FP8_G128 ? 16 : AF == MOE_A_MXFP8_G32 ? 4 : 0;
};

// A block of NT threads quantises one row at a time and strides over the
// rows (the grid is bounded, so a launch whose rows are absent or that the
// chosen configuration skips costs a few blocks); thread owns 8-element
// chunks c = tid + NT*j.  Per-token scales take 1024-thread blocks: the whole
// row is one block's, and more threads per row divide its quotient work.
template <int AF, bool IN_BF16, int MAXJ, int NT>
__global__ void __launch_bounds__(NT) k_quant(QuantArgs qa) {
  if (qa.meta && qa.meta[META_CFG] != qa.only_cfg) return;
  const int nrows = qa.nrows ? min(*qa.nrows, qa.R) : qa.R;
  const int n = qa.n, nch = n / 8;
  const int tid = threadIdx.x;
  for (int row = blockIdx.x; row < nrows; row += gridDim.x) {
  // all chunk loads of the row first (indices clamped into the row), so
  // they are in flight together
  QrChunk<IN_BF16> raw[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = tid + NT * j;
    raw[j] = qr_fetch<IN_BF16>(qa.in, row, n, c < nch ? c : nch - 1);
  }
  float v[MAXJ][8];
  float gmax[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    qr_unpack<IN_BF16>(raw[j], v[j]);
    gmax[j] = tid + NT * j < nch ? qr_amax8(v[j]) : 0.f;
  }
  if (AF == MOE_A_FP8_TOKEN) {
    __shared__ float red[NT / 64];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) m = fmaxf(m, gmax[j]);
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, red[w]);
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) gmax[j] = m;
  } else {
    constexpr int CH = QGroup<AF>::CHUNKS;   // consecutive lanes sharing a group
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
#pragma unroll
      for (int o = 1; o < CH; o <<= 1) gmax[j] = fmaxf(gmax[j], __shfl_xor(gmax[j], o, 64));
  }
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    int c = tid + NT * j;
    if (c >= nch) continue;
    float a = gmax[j];
    uint32_t lo, hi;
    if (AF == MOE_A_MXFP8_G32) {
      int ex = a > 0.f ? ilog2_floor(a) - 8 : -127;
      ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
      float inv = __builtin_ldexpf(1.0f, -ex);   // exact power of two
      lo = cvt4_e4m3(v[j][0] * inv, v[j][1] * inv, v[j][2] * inv, v[j][3] * inv);
      hi = cvt4_e4m3(v[j][4] * inv, v[j][5] * inv, v[j][6] * inv, v[j][7] * inv);
      if ((c & 3) == 0) ((uint8_t*)qa.scale)[(size_t)row * (n / 32) + c / 4] = (uint8_t)(ex + 127);
    } else {
      float s = qr_scale(a);
      const uint2 qc = qr_codes_div(v[j], s);
      lo = qc.x;
      hi = qc.y;
      if (AF == MOE_A_FP8_TOKEN) {
        if (c == 0) ((float*)qa.scale)[row] = s;
      } else if ((c & 15) == 0) {
        ((float*)qa.scale)[(size_t)row * (n / 128) + c / 16] = s;
      }
    }
    *(uint2*)(qa.q + (size_t)row * n + 8 * c) = make_uint2(lo, hi);
  }
  if (AF == MOE_A_FP8_TOKEN) __syncthreads();   // red[] is reused by the next row
  }
}

// bounded persistent grid: a few blocks per compute unit
static int elementwise_grid(int rows) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return rows < 8 * cus ? rows : 8 * cus;
}

template <int AF, bool IN_BF16>
static hipError_t quant_dispatch_j(const QuantArgs& q, hipStream_t st) {
  constexpr int NT = AF == MOE_A_FP8_TOKEN ? 1024 : 256;
  int nch = q.n / 8, j = (nch + NT - 1) / NT;
  // a launch that runs only for one configuration (its rows are then few)
  // keeps a small grid, so skipping it costs little
  int blocks = elementwise_grid(q.R);
  if (q.meta && blocks > 64) blocks = 64;
  dim3 grid(blocks), block(NT);
  if (j <= 1) hipLaunchKernelGGL((k_quant<AF, IN_BF16, 1, NT>), grid, block, 0, st, q);
  else if (j <= 2) hipLaunchKernelGGL((k_quant<AF, IN_BF16, 2, NT>), grid, block, 0, st, q);
  else if (j <= 4) hipLaunchKernelGGL((k_quant<AF, IN_BF16, 4, NT>), grid, block, 0, st, q);
  else if (j <= 8) hipLaunchKernelGGL((k_quant<AF, IN_BF16, 8, NT>), grid, block, 0, st, q);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs& q, hipStream_t st) {
  if (q.R == 0) return hipSuccess;
  switch (q.a_format) {
    case MOE_A_FP8_TOKEN:
      return q.in_bf16 ? quant_dispatch_j<MOE_A_FP8_TOKEN, true>(q, st)
                       : quant_dispatch_j<MOE_A_FP8_TOKEN, false>(q, st);
    case MOE_A_FP8_G128:
      return q.in_bf16 ? quant_dispatch_j<MOE_A_FP8_G128, true>(q, st)
                       : quant_dispatch_j<MOE_A_FP8_G128, false>(q, st);
    case MOE_A_MXFP8_G32:
      return q.in_bf16 ? quant_dispatch_j<MOE_A_MXFP8_G32, true>(q, st)
                       : quant_dispatch_j<MOE_A_MXFP8_G32, false>(q, st);
    default:
      return hipErrorInvalidValue;
  }
}

// bf16 rows, one wave per row: the same device code the routing launches
// run on their spare waves
template <int QF>
__global__ void __launch_bounds__(256) k_quant_rows(QuantArgs q) {
  quant_rows_waves<QF>(q, (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), (int)gridDim.x * 4,
                       threadIdx.x & 63);
}

hipError_t launch_quant_rows(const QuantArgs& q, hipStream_t st) {
  if (q.R == 0) return hipSuccess;
  if (!q.in_bf16) return hipErrorInvalidValue;
  const int blocks = (q.R + 3) / 4;
  LAUNCH_QF(quant_format(q), k_quant_rows, dim3(blocks < 2048 ? blocks : 2048), dim3(256), 0, st, q);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// One 256-thread block per token; thread owns 8-column chunks.  Slot rows
// are either fp32 (weights applied here) or bf16 already scaled by their
// routing weight in the down projection's epilogue; either way the k rows
// (then the shared expert's) are added in a fixed order in fp32 and the sum
// is rounded to bf16 once.
// Blocks stride over the tokens.  The k slot rows of a chunk are loaded in
// groups of CK, all loads of a group issued before any is used (slots past
// k re-read the first row and are not added); rows are added in ascending
// j, then the shared expert's.  WB: bf16 slot rows carrying their weights.
// One item = one token's channel range of 256 eight-channel chunks (one
// pass of the block), so a small batch still spreads over many blocks; the
// item's slots and weights are read before its rows, and every row of the
// item (the k routed rows, then the shared expert's) is fetched before any
// is added.
template <int CK, bool WB, bool SH>
__global__ void __launch_bounds__(256) k_combine(CombineArgs c) {
  const int H = c.H, nch = H / 8, k = c.k;
  const int S = c.T * k;
  const int nsplit = (nch + 255) / 256;
  for (int item = blockIdx.x; item < c.T * nsplit; item += gridDim.x) {
    const int t = item / nsplit;
    const int ch = (item - t * nsplit) * 256 + threadIdx.x;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += CK) {
      int slot[CK];
      float wj[CK];
#pragma unroll
      for (int u = 0; u < CK; ++u) {
        const int j = j0 + u < k ? j0 + u : j0;
        slot[u] = ldu(c.inv + (size_t)t * k + j);
        wj[u] = WB ? 1.0f : ldu(c.w + (size_t)t * k + j);
      }
      if (ch >= nch) continue;
      QrChunk<WB> raw[SH ? CK + 1 : CK];
      // a negative slot (an id the dispatch dropped) has no row: it adds
      // nothing and its row is not read
#pragma unroll
      for (int u = 0; u < CK; ++u) raw[u] = qr_fetch<WB>(c.out_slot, (size_t)(slot[u] < 0 ? 0 : slot[u]), H, ch);
      const bool sh = SH && j0 + CK >= k;   // the last pass also takes the shared row
      if constexpr (SH) {
        if (sh) raw[CK] = qr_fetch<WB>(c.out_slot, (size_t)(S + t), H, ch);
      }
#pragma unroll
      for (int u = 0; u < CK; ++u) {
        if (j0 + u < k && slot[u] >= 0) {
          float v[8];
          qr_unpack<WB>(raw[u], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += wj[u] * v[i];
        }
      }
      if constexpr (SH) {
        if (!sh) continue;
        float v[8];
        qr_unpack<WB>(raw[CK], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
    }
    if (ch >= nch) continue;
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(uint4*)(c.y + (size_t)t * H + 8 * ch) = make_uint4(p[0], p[1], p[2], p[3]);
  }
}

hipError_t launch_combine(const CombineArgs& c, hipStream_t st) {
  if (c.T == 0) return hipSuccess;
  const int nsplit = (c.H / 8 + 255) / 256;
  const dim3 grid(elementwise_grid(c.T * nsplit)), block(256);
  // the shared expert's row is a template choice, so layers without one
  // carry no code or registers for it
  auto go = [&](auto wb, auto sh) {
    constexpr bool WB = decltype(wb)::value, SH = decltype(sh)::value;
    if (c.k <= 2) hipLaunchKernelGGL((k_combine<2, WB, SH>), grid, block, 0, st, c);
    else if (c.k <= 4) hipLaunchKernelGGL((k_combine<4, WB, SH>), grid, block, 0, st, c);
    else hipLaunchKernelGGL((k_combine<8, WB, SH>), grid, block, 0, st, c);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (c.weighted_bf16) {
    if (c.shared) go(T_{}, T_{});
    else go(T_{}, F_{});
  } else {
    if (c.shared) go(F_{}, T_{});
    else go(F_{}, F_{});
  }
  return hipGetLastError();
}
