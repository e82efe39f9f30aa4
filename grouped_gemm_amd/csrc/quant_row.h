// One wave quantises one activation row (dynamic FP8 scales), so the work
// can ride along in any launch that has spare waves: the routing and
// dispatch kernels quantise x while they route (the input quantisation of
// the LightMoE README, "MoE inference", has no dependency on the routing).
//
// Rule (same as the block-per-row kernel): per group a = max|v|; FP8 groups
// use s = a/448 in fp32 (1 when a = 0) and q = e4m3_rne(clamp(v/s)) with the
// correctly rounded fp32 quotient; MX groups (OCP MX v1.0) X = 2^(floor(log2 a) - 8) as e8m0
// and q = e4m3_rne_sat(v/X).  Lane l owns the 8-element chunks l + 64*j, so
// a 1x128 group is 16 consecutive lanes and an MX group 4.
#pragma once
#include "layer.h"

template <bool IN_BF16>
DEVI void qr_load8(const void* in, size_t row, int n, int c, float (&v)[8]) {
  if (IN_BF16) {
    const uint4 raw = *(const uint4*)((const uint16_t*)in + row * n + 8 * c);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(w4[i] & 0xFFFF));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(w4[i] >> 16));
    }
  } else {
    const float* src = (const float*)in + row * n + 8 * c;
    const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

DEVI float qr_amax8(const float (&v)[8]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// a / s rounded to nearest, from r = RN(1/s) and one residual step:
// q0 = RN(a*r) is within an ulp of a/s, the residual e = a - q0*s is exact
// and RN(q0 + e*r) = RN(a/s) (Markstein's theorem on FMA-based division),
// provided no intermediate underflows or overflows -- which holds for
// s in [2^-60, 2^60] and |a| >= 2^-60.  e = 0 means q0 is exact (this also
// keeps the sign of a zero a).
DEVI float qr_div_fast(float a, float s, float r) {
  const float q0 = a * r;
  const float e = __builtin_fmaf(-q0, s, a);
  return e == 0.f ? q0 : __builtin_fmaf(e, r, q0);
}

// the IEEE quotients of a chunk (outside the residual step's domain; kept
// out of line so the common path stays short)
__device__ __attribute__((noinline)) uint2 qr_codes_ieee(float4 a, float4 b, float s) {
  return make_uint2(cvt4_e4m3(a.x / s, a.y / s, a.z / s, a.w / s),
                    cvt4_e4m3(b.x / s, b.y / s, b.z / s, b.w / s));
}

// codes of one chunk with the FP8 scale s: v/s rounded to nearest (the
// IEEE quotient), by the residual step where its domain holds, else by the
// division itself
DEVI uint2 qr_codes_div(const float (&v)[8], float s) {
  bool fast = s >= 0x1p-60f && s <= 0x1p60f;
#pragma unroll
  for (int i = 0; i < 8; ++i) fast = fast && (fabsf(v[i]) >= 0x1p-60f || v[i] == 0.f);
  if (!fast)
    return qr_codes_ieee(make_float4(v[0], v[1], v[2], v[3]), make_float4(v[4], v[5], v[6], v[7]), s);
  const float r = 1.0f / s;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = qr_div_fast(v[i], s, r);
  return make_uint2(cvt4_e4m3(o[0], o[1], o[2], o[3]), cvt4_e4m3(o[4], o[5], o[6], o[7]));
}

// Per-token scale: the whole row shares one amax.  Rows of up to 4096
// elements stay in registers; longer rows are read twice.
template <bool IN_BF16>
DEVI void quant_row_wave_token(const QuantArgs& q, int row, int lane) {
  const int n = q.n, nch = n / 8;
  uint8_t* qrow = q.q + (size_t)row * n;
  if (nch <= 8 * 64) {
    float v[8][8];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) {
        qr_load8<IN_BF16>(q.in, row, n, c, v[j]);
        m = fmaxf(m, qr_amax8(v[j]));
      }
    }
    m = wave_max(m);
    const float s = m > 0.f ? m / 448.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) *(uint2*)(qrow + 8 * c) = qr_codes_div(v[j], s);
    }
    if (lane == 0) ((float*)q.scale)[row] = s;
    return;
  }
  float m = 0.f;
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    qr_load8<IN_BF16>(q.in, row, n, c, v);
    m = fmaxf(m, qr_amax8(v));
  }
  m = wave_max(m);
  const float s = m > 0.f ? m / 448.0f : 1.0f;
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    qr_load8<IN_BF16>(q.in, row, n, c, v);
    *(uint2*)(qrow + 8 * c) = qr_codes_div(v, s);
  }
  if (lane == 0) ((float*)q.scale)[row] = s;
}

// Group scales (1x128 or MX-32): every 64-chunk pass is independent;
// groups never straddle a pass because 64 is a multiple of 16.  Four passes
// have their loads in flight together; the group maximum is a DPP row (16
// lanes) or quad (4 lanes) reduction.
template <int AF, bool IN_BF16>
DEVI void quant_row_wave_group(const QuantArgs& q, int row, int lane) {
  constexpr int QP = 4;
  const int n = q.n, nch = n / 8;
  uint8_t* qrow = q.q + (size_t)row * n;
  for (int c0 = 0; c0 < nch; c0 += 64 * QP) {
    float v[QP][8];
    float m[QP];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int c = c0 + 64 * u + lane;
      m[u] = 0.f;
      if (c < nch) {
        qr_load8<IN_BF16>(q.in, row, n, c, v[u]);
        m[u] = qr_amax8(v[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      // non-negative floats order as their bit patterns
      const uint32_t mb = __float_as_uint(m[u]);
      m[u] = __uint_as_float(AF == MOE_A_FP8_G128 ? row16_max(mb) : quad_max(mb));
    }
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int c = c0 + 64 * u + lane;
      if (c >= nch) continue;
      if (AF == MOE_A_MXFP8_G32) {
        int ex = m[u] > 0.f ? ilog2_floor(m[u]) - 8 : -127;
        ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
        const float inv = __builtin_ldexpf(1.0f, -ex);   // exact power of two
        *(uint2*)(qrow + 8 * c) = make_uint2(
            cvt4_e4m3(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv),
            cvt4_e4m3(v[u][4] * inv, v[u][5] * inv, v[u][6] * inv, v[u][7] * inv));
        if ((c & 3) == 0) ((uint8_t*)q.scale)[(size_t)row * (n / 32) + c / 4] = (uint8_t)(ex + 127);
      } else {
        const float s = m[u] > 0.f ? m[u] / 448.0f : 1.0f;
        *(uint2*)(qrow + 8 * c) = qr_codes_div(v[u], s);
        if ((c & 15) == 0) ((float*)q.scale)[(size_t)row * (n / 128) + c / 16] = s;
      }
    }
  }
}

// Rows wave_id, wave_id + n_waves, ... of a bf16 activation matrix, in
// activation format AF (0: nothing to do).  The format is a template
// argument so a launch carries the code of one format only.
template <int AF>
DEVI void quant_rows_waves(const QuantArgs& q, int wave_id, int n_waves, int lane) {
  if constexpr (AF == MOE_A_FP8_TOKEN || AF == MOE_A_FP8_G128 || AF == MOE_A_MXFP8_G32) {
    for (int row = wave_id; row < q.R; row += n_waves) {
      if constexpr (AF == MOE_A_FP8_TOKEN) quant_row_wave_token<true>(q, row, lane);
      else quant_row_wave_group<AF, true>(q, row, lane);
    }
  }
}

// Format of the rows a launch's spare waves quantise (0: none).
inline int quant_format(const QuantArgs& q) { return q.R > 0 ? q.a_format : 0; }

// hipLaunchKernelGGL of K<format> for the runtime format qf.
#define LAUNCH_QF(qf, K, grid, block, lds, st, ...)                                          \
  do {                                                                                      \
    switch (qf) {                                                                           \
      case MOE_A_FP8_TOKEN:                                                                 \
        hipLaunchKernelGGL(K<MOE_A_FP8_TOKEN>, grid, block, lds, st, __VA_ARGS__);          \
        break;                                                                              \
      case MOE_A_FP8_G128:                                                                  \
        hipLaunchKernelGGL(K<MOE_A_FP8_G128>, grid, block, lds, st, __VA_ARGS__);           \
        break;                                                                              \
      case MOE_A_MXFP8_G32:                                                                 \
        hipLaunchKernelGGL(K<MOE_A_MXFP8_G32>, grid, block, lds, st, __VA_ARGS__);          \
        break;                                                                              \
      default:                                                                              \
        hipLaunchKernelGGL(K<0>, grid, block, lds, st, __VA_ARGS__);                        \
        break;                                                                              \
    }                                                                                       \
  } while (0)
