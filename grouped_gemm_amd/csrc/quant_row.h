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

// Raw bytes of one 8-element chunk (bf16: 16 B, fp32: 32 B).  Callers
// fetch all chunks of a pass first (indices clamped into the row, so no
// load sits behind a branch) and unpack afterwards, keeping the loads in
// flight together.
template <bool IN_BF16>
struct QrChunk {
  uint4 w[IN_BF16 ? 1 : 2];
};

template <bool IN_BF16>
DEVI QrChunk<IN_BF16> qr_fetch(const void* in, size_t row, int n, int c) {
  QrChunk<IN_BF16> r;
  if constexpr (IN_BF16) {
    r.w[0] = *(const uint4*)((const uint16_t*)in + row * n + 8 * c);
  } else {
    const uint4* p = (const uint4*)((const float*)in + row * n + 8 * c);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
  return r;
}

template <bool IN_BF16>
DEVI void qr_unpack(const QrChunk<IN_BF16>& r, float (&v)[8]) {
  if constexpr (IN_BF16) {
    const uint32_t w4[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w4[i] << 16);
      v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(r.w[0].x); v[1] = __uint_as_float(r.w[0].y);
    v[2] = __uint_as_float(r.w[0].z); v[3] = __uint_as_float(r.w[0].w);
    v[4] = __uint_as_float(r.w[1].x); v[5] = __uint_as_float(r.w[1].y);
    v[6] = __uint_as_float(r.w[1].z); v[7] = __uint_as_float(r.w[1].w);
  }
}

DEVI float qr_amax8(const float (&v)[8]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// FP8 scale of a group maximum m > 0: s = RN(m / 448), by one residual
// step from the constant RN(1/448) (Markstein's theorem on FMA-based
// division: q0 = RN(m*y) is within an ulp of m/448, the residual
// e = m - 448*q0 is exact and RN(q0 + e*y) = RN(m/448) while nothing
// underflows or overflows, which holds for m in [2^-40, 2^68]).
DEVI float qr_scale448(float m) {
  constexpr float y = 1.0f / 448.0f;
  const float q0 = m * y;
  const float e = __builtin_fmaf(-q0, 448.0f, m);
  return __builtin_fmaf(e, y, q0);
}

// The codes of one chunk need e4m3_rne(RN(v/s)).  For s in [2^-49, 2^60]
// the same residual step from r = RN(1/s) gives RN(v/s) exactly for every
// |v| >= 2^-60 (and v = 0, whose sign copysign restores); for smaller
// nonzero |v| the quotient is below 2^-11, which rounds to an e4m3 zero of
// v's sign whichever way its last bits fall.  Groups outside that range of
// s divide.
DEVI bool qr_fast_scale(float s) { return s >= 0x1p-49f && s <= 0x1p60f; }

DEVI uint2 qr_codes_fast(const float (&v)[8], float s) {
  const float r = 1.0f / s;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q0 = v[i] * r;
    const float e = __builtin_fmaf(-q0, s, v[i]);
    o[i] = __builtin_copysignf(__builtin_fmaf(e, r, q0), v[i]);
  }
  return make_uint2(cvt4_e4m3(o[0], o[1], o[2], o[3]), cvt4_e4m3(o[4], o[5], o[6], o[7]));
}

// the IEEE quotients of a chunk (out of line: rare)
__device__ __attribute__((noinline)) uint2 qr_codes_ieee(float4 a, float4 b, float s) {
  return make_uint2(cvt4_e4m3(a.x / s, a.y / s, a.z / s, a.w / s),
                    cvt4_e4m3(b.x / s, b.y / s, b.z / s, b.w / s));
}

__device__ __attribute__((noinline)) float qr_div448_ieee(float m) { return m / 448.0f; }

// scale of group maximum m (1 when m = 0)
DEVI float qr_scale(float m) {
  if (m <= 0.f) return 1.0f;
  if (m >= 0x1p-40f && m <= 0x1p68f) return qr_scale448(m);
  return qr_div448_ieee(m);
}

// codes of one chunk with the FP8 scale s: e4m3_rne(clamp(v/s))
DEVI uint2 qr_codes_div(const float (&v)[8], float s) {
  if (qr_fast_scale(s)) return qr_codes_fast(v, s);
  return qr_codes_ieee(make_float4(v[0], v[1], v[2], v[3]), make_float4(v[4], v[5], v[6], v[7]), s);
}

// Per-token scale: the whole row shares one amax.  Rows of up to 4096
// elements stay in registers; longer rows are read twice.
template <bool IN_BF16>
DEVI void quant_row_wave_token(const QuantArgs& q, int row, int lane) {
  const int n = q.n, nch = n / 8;
  uint8_t* qrow = q.q + (size_t)row * n;
  if (nch <= 8 * 64) {
    QrChunk<IN_BF16> raw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = lane + 64 * j;
      raw[j] = qr_fetch<IN_BF16>(q.in, row, n, c < nch ? c : nch - 1);
    }
    float v[8][8];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qr_unpack<IN_BF16>(raw[j], v[j]);
      if (lane + 64 * j < nch) m = fmaxf(m, qr_amax8(v[j]));
    }
    m = wave_max(m);
    const float s = qr_scale(m);
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
    qr_unpack<IN_BF16>(qr_fetch<IN_BF16>(q.in, row, n, c), v);
    m = fmaxf(m, qr_amax8(v));
  }
  m = wave_max(m);
  const float s = qr_scale(m);
  for (int c = lane; c < nch; c += 64) {
    float v[8];
    qr_unpack<IN_BF16>(qr_fetch<IN_BF16>(q.in, row, n, c), v);
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
    QrChunk<IN_BF16> raw[QP];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int c = c0 + 64 * u + lane;
      raw[u] = qr_fetch<IN_BF16>(q.in, row, n, c < nch ? c : nch - 1);
    }
    float v[QP][8];
    float m[QP];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      qr_unpack<IN_BF16>(raw[u], v[u]);
      m[u] = c0 + 64 * u + lane < nch ? qr_amax8(v[u]) : 0.f;
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
        const float s = qr_scale(m[u]);
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
