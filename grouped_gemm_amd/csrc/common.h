// Device-side building blocks shared by the gfx950 kernels of the MoE layer.
//
// MFMA conventions used throughout (measured on gfx950):
//  * v_mfma_*_16x16x128_f8f6f4: operand "A" supplies 16 rows, operand "B" 16
//    columns, both over 128 K elements.  For 8-bit elements, lane l (row
//    l%16, lane group g = l/16) holds K elements [16g, 16g+16) in its first
//    four registers and [64+16g, 64+16g+16) in the next four.  For 4-bit
//    elements lane group g holds K [32g, 32g+32), the even element in the low
//    nibble.  The scale operand of lane l covers row l%16 and the 32-wide K
//    block l/16.
//  * the fp32 result: lane l holds D[4*(l/16) + i][l%16], i = 0..3.
//  * v_mfma_f32_16x16x32_bf16: lane group g holds K [8g, 8g+8) of its row.
// In every kernel here operand A is the expert weight (rows = output
// channels) and operand B the token rows, so a lane ends up with four
// consecutive output channels of one token.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Format enumerations (mirrored in the public header).
#define MOE_W_BF16 0
#define MOE_W_FP8_CHANNEL 1
#define MOE_W_FP8_BLOCK128 2
#define MOE_W_MXFP4 3
#define MOE_A_BF16 0
#define MOE_A_FP8_TOKEN 1
#define MOE_A_FP8_G128 2
#define MOE_A_MXFP8_G32 3

// Weight/activation format pairs supported by the kernels.
enum Fmt { F_BF16 = 0, F_FP8_CH = 1, F_FP8_BLK = 2, F_MX = 3 };

#define DEVI __device__ __forceinline__

// ---------------------------------------------------------------- scalars
DEVI float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (finite inputs).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even: one
// gfx950 pair conversion.
DEVI uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
DEVI uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, 0.0f); }

// Two fp32 -> two OCP e4m3 codes (RNE).  The hardware conversion is exact
// round-to-nearest-even inside the finite range; inputs are clamped to
// +-448 first because out-of-range inputs may produce the NaN code.
DEVI uint32_t cvt2_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

DEVI uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// z * sigmoid(z); the reciprocal is the hardware one (1 ulp), far inside the
// rounding of the bf16 / e4m3 values the result is stored as.
DEVI float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Expert activations of a gate value g and an up value u (LightMoE README,
// "Compatibility": SwiGLU, bounded SwiGLU, SwiGLU-OAI, GeGLU, ReGLU and the
// two-weight ReLU^2, whose kernels receive the up projection as both
// operands).  L clamps the bounded forms.  Kernels take the activation as a
// template argument, so each instantiation inlines exactly one formula.
enum { ACT_SWIGLU = 0, ACT_SWIGLU_BOUNDED, ACT_SWIGLU_OAI, ACT_GEGLU, ACT_REGLU, ACT_RELU2 };
template <int ACT>
DEVI float gated_act(float L, float g, float u) {
  if constexpr (ACT == ACT_SWIGLU_BOUNDED) {
    return silu(fminf(g, L)) * fminf(fmaxf(u, -L), L);
  } else if constexpr (ACT == ACT_SWIGLU_OAI) {
    const float gc = fminf(g, L);
    return gc * __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * gc)) * (fminf(fmaxf(u, -L), L) + 1.0f);
  } else if constexpr (ACT == ACT_GEGLU) {
    return 0.5f * g * (1.0f + erff(g * 0.70710678118654752f)) * u;
  } else if constexpr (ACT == ACT_REGLU) {
    return fmaxf(g, 0.0f) * u;
  } else if constexpr (ACT == ACT_RELU2) {
    const float r = fmaxf(u, 0.0f);
    return r * r;
  } else {
    return silu(g) * u;
  }
}

// Calls f(std::integral_constant<int, ACT>{}) for the runtime activation id
// (SwiGLU for ids outside the table, which the API rejects earlier).
template <class Fn>
inline auto with_act(int act, Fn&& f) {
  switch (act) {
    case ACT_SWIGLU_BOUNDED: return f(std::integral_constant<int, ACT_SWIGLU_BOUNDED>{});
    case ACT_SWIGLU_OAI: return f(std::integral_constant<int, ACT_SWIGLU_OAI>{});
    case ACT_GEGLU: return f(std::integral_constant<int, ACT_GEGLU>{});
    case ACT_REGLU: return f(std::integral_constant<int, ACT_REGLU>{});
    case ACT_RELU2: return f(std::integral_constant<int, ACT_RELU2>{});
    default: return f(std::integral_constant<int, ACT_SWIGLU>{});
  }
}


// floor(log2(a)) for a finite a > 0 (exact, from the exponent field).
DEVI int ilog2_floor(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF);
  if (e == 0) {                       // subnormal: 2^-149 * mantissa
    uint32_t m = u & 0x7FFFFF;
    return -149 + (31 - __builtin_clz(m));
  }
  return e - 127;
}

// ---------------------------------------------------------------- wave reductions
DEVI float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
DEVI float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reductions over a row of 16 lanes by DPP moves (no LDS round trip): xor 1
// and xor 2 inside quads, then the half-row and row mirrors, after which
// every lane of the row holds the row's result.
template <int CTRL>
DEVI uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
DEVI uint32_t row16_max(uint32_t v) {
  uint32_t o = dpp_mov<0xB1>(v);
  v = o > v ? o : v;
  o = dpp_mov<0x4E>(v);
  v = o > v ? o : v;
  o = dpp_mov<0x141>(v);
  v = o > v ? o : v;
  o = dpp_mov<0x140>(v);
  return o > v ? o : v;
}
// max over the 4 lanes of a quad
DEVI uint32_t quad_max(uint32_t v) {
  uint32_t o = dpp_mov<0xB1>(v);
  v = o > v ? o : v;
  o = dpp_mov<0x4E>(v);
  return o > v ? o : v;
}
DEVI uint32_t row16_min(uint32_t v) {
  uint32_t o = dpp_mov<0xB1>(v);
  v = o < v ? o : v;
  o = dpp_mov<0x4E>(v);
  v = o < v ? o : v;
  o = dpp_mov<0x141>(v);
  v = o < v ? o : v;
  o = dpp_mov<0x140>(v);
  return o < v ? o : v;
}
// (each pairing adds the same two partial sums, so all lanes agree bitwise)
DEVI float row16_sum(float v) {
  v += __uint_as_float(dpp_mov<0xB1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<0x4E>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<0x141>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<0x140>(__float_as_uint(v)));
  return v;
}

// Inclusive prefix over the 64 lanes of a wave by DPP (GFX9 row shifts and
// row broadcasts; no LDS-crossbar round trip per step): shifts by 1, 2, 4
// and 8 inside each 16-lane row (lanes shifted in from before the row read
// 0), then lane 15 is added into row 1, lane 47 into row 3, and lane 31 into
// rows 2 and 3.  The operation is + or max over non-negative ints (0 is the
// identity of both).  Every lane of the wave must be active.
template <bool MAX>
DEVI int wave_incl_scan(int v) {
  auto op = [](int a, int b) { return MAX ? (a > b ? a : b) : a + b; };
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false));   // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false));   // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false));   // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false));   // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return v;
}
// The wave's sum or maximum (lane 63 of the inclusive scan), as a scalar.
template <bool MAX>
DEVI int wave_total(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan<MAX>(v), 63);
}

// ---------------------------------------------------------------- MFMA
DEVI f32x4 mfma_f8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// A = e2m1 (format 4), B = e4m3 (format 0), per-lane e8m0 scales.
DEVI f32x4 mfma_f4f8_scaled(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}
DEVI f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Two bf16 16x16x32 products over a 128-byte row chunk read as two 16-byte
// halves per lane (dwords 0..3: K elements 8g..8g+7, dwords 4..7: 32+8g..;
// g = lane / 16), the same lane layout as one 16x16x128 FP8 product's.
DEVI f32x4 mfma_bf16_pair(const i32x8& a, const i32x8& b, f32x4 c) {
  const i32x4 alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
  const i32x4 blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
  c = mfma_bf16(__builtin_bit_cast(bf16x8, alo), __builtin_bit_cast(bf16x8, blo), c);
  return mfma_bf16(__builtin_bit_cast(bf16x8, ahi), __builtin_bit_cast(bf16x8, bhi), c);
}

// ---------------------------------------------------------------- fragments
// One K step = 128 elements.  Per-lane operand bytes per step: fp8 32,
// fp4 16, bf16 64 (four 16x16x32 sub-steps).
template <int ELEM_BITS>
struct Frag;

template <>
struct Frag<8> {
  i32x8 v;
  DEVI void load(const uint8_t* row, int k0, int g) {
    const i32x4 lo = *(const i32x4*)(row + k0 + 16 * g);
    const i32x4 hi = *(const i32x4*)(row + k0 + 64 + 16 * g);
    v = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  DEVI void zero() { v = (i32x8){0, 0, 0, 0, 0, 0, 0, 0}; }
};

template <>
struct Frag<4> {
  i32x8 v;
  DEVI void load(const uint8_t* row, int k0, int g) {   // row = packed bytes
    const i32x4 q = *(const i32x4*)(row + (k0 >> 1) + 16 * g);
    v = (i32x8){q[0], q[1], q[2], q[3], 0, 0, 0, 0};
  }
  DEVI void zero() { v = (i32x8){0, 0, 0, 0, 0, 0, 0, 0}; }
};

template <>
struct Frag<16> {
  bf16x8 v[4];
  DEVI void load(const uint8_t* row, int k0, int g) {   // row = bf16 bytes
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = *(const bf16x8*)(row + 2 * (k0 + 32 * s + 8 * g));
  }
  DEVI void zero() {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      for (int i = 0; i < 8; ++i) v[s][i] = (__bf16)0.0f;
  }
};

// Bits per element of the weight (A) and activation (B) operands.
template <int F> struct FmtBits;
template <> struct FmtBits<F_BF16> { static constexpr int W = 16, X = 16; };
template <> struct FmtBits<F_FP8_CH> { static constexpr int W = 8, X = 8; };
template <> struct FmtBits<F_FP8_BLK> { static constexpr int W = 8, X = 8; };
template <> struct FmtBits<F_MX> { static constexpr int W = 4, X = 8; };

// Load from a wave-uniform address through the scalar data cache.  Only for
// arrays that the running kernel never writes (routing tables, scales).
template <class T> DEVI T ldu(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Bytes of one operand row of K elements.
template <int BITS> DEVI constexpr long row_bytes(int K) { return (long)K * BITS / 8; }

// acc += A*B for one K step, for the unscaled formats.
DEVI f32x4 mma_step(const Frag<8>& a, const Frag<8>& b, f32x4 c) { return mfma_f8(a.v, b.v, c); }
DEVI f32x4 mma_step(const Frag<16>& a, const Frag<16>& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = mfma_bf16(a.v[s], b.v[s], c);
  return c;
}

// ---------------------------------------------------------------- XCD-aware work split
// Workgroups of a launch are dealt to the 8 XCDs of the chip in turn
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  A
// persistent grid therefore gives every XCD one contiguous range of the
// (expert-major) work items, walked by that XCD's workgroups, so the items
// that share an expert's weights and a row block's tokens meet in one L2.
struct ItemRange {
  int begin, end, step;
};
DEVI ItemRange xcd_items(int n_items) {
  constexpr int NX = 8;
  const int grid = gridDim.x;
  if (grid % NX) return {(int)blockIdx.x, n_items, grid};
  const int x = blockIdx.x % NX, j = blockIdx.x / NX, per = grid / NX;
  const int chunk = (n_items + NX - 1) / NX;
  const int b = x * chunk;
  const int e = b + chunk < n_items ? b + chunk : n_items;
  return {b + j, e, per};
}
