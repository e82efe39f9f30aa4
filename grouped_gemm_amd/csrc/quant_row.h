// One wave quantises one activation row (dynamic FP8 scales), so the work
// can ride along in any launch that has spare waves: the routing and
// dispatch kernels quantise x while they route (the input quantisation of
// the LightMoE README, "MoE inference", has no dependency on the routing).
//
// Rule (same as the block-per-row kernel): per group a = max|v|; FP8 groups
// use s = a/448 in fp32 (1 when a = 0) and q = e4m3_rne(clamp(v/s)) with
// IEEE division; MX groups (OCP MX v1.0) X = 2^(floor(log2 a) - 8) as e8m0
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

// codes of one chunk with the FP8 scale s (IEEE division, as the rule says)
DEVI uint2 qr_codes_div(const float (&v)[8], float s) {
  return make_uint2(cvt4_e4m3(v[0] / s, v[1] / s, v[2] / s, v[3] / s),
                    cvt4_e4m3(v[4] / s, v[5] / s, v[6] / s, v[7] / s));
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

// Group scales (1x128 or MX-32): every 64-chunk pass is independent; groups
// never straddle a pass because 64 is a multiple of 16.
template <int AF, bool IN_BF16>
DEVI void quant_row_wave_group(const QuantArgs& q, int row, int lane) {
  constexpr int CH = AF == MOE_A_FP8_G128 ? 16 : 4;   // lanes per group
  const int n = q.n, nch = n / 8;
  uint8_t* qrow = q.q + (size_t)row * n;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    float v[8];
    float m = 0.f;
    if (c < nch) {
      qr_load8<IN_BF16>(q.in, row, n, c, v);
      m = qr_amax8(v);
    }
#pragma unroll
    for (int o = 1; o < CH; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (c >= nch) continue;
    if (AF == MOE_A_MXFP8_G32) {
      int ex = m > 0.f ? ilog2_floor(m) - 8 : -127;
      ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
      const float inv = __builtin_ldexpf(1.0f, -ex);   // exact power of two
      *(uint2*)(qrow + 8 * c) =
          make_uint2(cvt4_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                     cvt4_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv));
      if ((c & 3) == 0) ((uint8_t*)q.scale)[(size_t)row * (n / 32) + c / 4] = (uint8_t)(ex + 127);
    } else {
      const float s = m > 0.f ? m / 448.0f : 1.0f;
      *(uint2*)(qrow + 8 * c) = qr_codes_div(v, s);
      if ((c & 15) == 0) ((float*)q.scale)[(size_t)row * (n / 128) + c / 16] = s;
    }
  }
}

template <bool IN_BF16>
DEVI void quant_row_wave(const QuantArgs& q, int row, int lane) {
  switch (q.a_format) {
    case MOE_A_FP8_TOKEN: quant_row_wave_token<IN_BF16>(q, row, lane); break;
    case MOE_A_FP8_G128: quant_row_wave_group<MOE_A_FP8_G128, IN_BF16>(q, row, lane); break;
    case MOE_A_MXFP8_G32: quant_row_wave_group<MOE_A_MXFP8_G32, IN_BF16>(q, row, lane); break;
    default: break;
  }
}

// Rows wave_id, wave_id + n_waves, ... of a bf16 activation matrix.
DEVI void quant_rows_waves(const QuantArgs& q, int wave_id, int n_waves, int lane) {
  for (int row = wave_id; row < q.R; row += n_waves) quant_row_wave<true>(q, row, lane);
}
