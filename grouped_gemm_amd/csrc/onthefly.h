// Quantisation of MFMA operands while they are loaded: a lane's 32 values of
// one 128-wide K step (bf16 activations or fp32 intermediate rows) turned
// into e4m3 codes under the quantiser's own rule (per-token and 1x128 FP8
// groups, MX-32), so the codes equal those of the separate quantisation
// pass bit for bit.
#pragma once
#include "layer.h"
#include "quant_row.h"

// The 32 values a lane feeds to one 128-wide K step of a 16x16x128 MFMA (K
// [16g, 16g+16) and [64+16g, 64+16g+16) of its row, g = lane / 16).
template <bool BF16_IN>
DEVI void load_step32(const void* row, int ks, int lg, float (&v)[32]) {
  if constexpr (BF16_IN) {
    const uint16_t* r = (const uint16_t*)row;
    uint4 q[4];
    q[0] = *(const uint4*)(r + ks + 16 * lg);
    q[1] = *(const uint4*)(r + ks + 16 * lg + 8);
    q[2] = *(const uint4*)(r + ks + 64 + 16 * lg);
    q[3] = *(const uint4*)(r + ks + 64 + 16 * lg + 8);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  } else {
    const float* r = (const float*)row;
    float4 q[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      q[2 * c] = *(const float4*)(r + ks + (c < 2 ? 0 : 64) + 16 * lg + 8 * (c & 1));
      q[2 * c + 1] = *(const float4*)(r + ks + (c < 2 ? 0 : 64) + 16 * lg + 8 * (c & 1) + 4);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[4 * c] = q[c].x;
      v[4 * c + 1] = q[c].y;
      v[4 * c + 2] = q[c].z;
      v[4 * c + 3] = q[c].w;
    }
  }
}

DEVI float amax32(const float (&v)[32]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// e4m3 codes of the 32 values with the FP8 scale s (the quantiser's rule:
// e4m3_rne(clamp(RN(v / s)))), packed as the lane's MFMA operand.
DEVI i32x8 codes_fp8(const float (&v)[32], float s) {
  uint2 c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = v[8 * q + i];
    c[q] = qr_codes_div(w, s);
  }
  return (i32x8){(int)c[0].x, (int)c[0].y, (int)c[1].x, (int)c[1].y,
                 (int)c[2].x, (int)c[2].y, (int)c[3].x, (int)c[3].y};
}

// MX-32 codes of the 32 values and the e8m0 scale the MFMA takes for this
// lane's K block.  The lo half (K [16g, 16g+16)) belongs to 32-group g/2,
// the hi half to group 2 + g/2, each shared with the lane 16 away; the
// operand scale of lane group g is that of group g.
DEVI i32x8 codes_mx(const float (&v)[32], int lane, int& sb) {
  const int lg = lane >> 4, r16 = lane & 15;
  float mlo = 0.f, mhi = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mlo = fmaxf(mlo, fabsf(v[i]));
    mhi = fmaxf(mhi, fabsf(v[16 + i]));
  }
  mlo = fmaxf(mlo, __shfl_xor(mlo, 16, 64));
  mhi = fmaxf(mhi, __shfl_xor(mhi, 16, 64));
  int elo = mlo > 0.f ? ilog2_floor(mlo) - 8 : -127;
  int ehi = mhi > 0.f ? ilog2_floor(mhi) - 8 : -127;
  elo = elo < -127 ? -127 : (elo > 127 ? 127 : elo);
  ehi = ehi < -127 ? -127 : (ehi > 127 ? 127 : ehi);
  const float ilo = __builtin_ldexpf(1.0f, -elo), ihi = __builtin_ldexpf(1.0f, -ehi);
  uint32_t d[8];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d[q] = cvt4_e4m3(v[4 * q] * ilo, v[4 * q + 1] * ilo, v[4 * q + 2] * ilo, v[4 * q + 3] * ilo);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d[4 + q] = cvt4_e4m3(v[16 + 4 * q] * ihi, v[16 + 4 * q + 1] * ihi, v[16 + 4 * q + 2] * ihi,
                         v[16 + 4 * q + 3] * ihi);
  // group g: 0 -> own lo; 1 -> lo of lane group 2; 2 -> own hi (lane group 0); 3 -> hi of lane group 2
  const int lo2 = __shfl(elo, r16 + 32, 64), hi0 = __shfl(ehi, r16, 64), hi2 = __shfl(ehi, r16 + 32, 64);
  const int e = lg == 0 ? elo : (lg == 1 ? lo2 : (lg == 2 ? hi0 : hi2));
  sb = e + 127;
  return (i32x8){(int)d[0], (int)d[1], (int)d[2], (int)d[3], (int)d[4], (int)d[5], (int)d[6], (int)d[7]};
}

DEVI i32x8 zero8() { return (i32x8){0, 0, 0, 0, 0, 0, 0, 0}; }
