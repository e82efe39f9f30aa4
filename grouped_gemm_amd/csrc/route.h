// Top-k selection of one token by a 16-lane row (shared by the routing
// and dispatch kernels and the single-launch decode layer).
//
// Routing follows the Alpha-MoE news page ("How the megakernel works":
// routing and gating are stages of the layer) and the LightMoE README ("MoE
// inference": int32 ids distinct per token, fp32 weights): the k largest
// scores, ties to the lower expert index, weights renormalised over the k.
#pragma once
#include "layer.h"

// Order-preserving map of an fp32 score to uint32 (+0 and -0 compare equal).
DEVI uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

DEVI uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Inverse of score_key (a -0 score comes back as +0, which weighs the same).
DEVI float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// One row of 16 lanes routes one token (E <= 256): lane l of the row holds
// the keys of experts e = 4l + j + 64q (j, q < 4).  Pass j takes the row
// maximum of the keys, then the lowest expert index holding it (the key
// order: score, then lowest index), and the owning lane drops that key.
// Lane j < k keeps the j-th choice; the weights are renormalised over the
// k.  Every lane of the row must run this (rows with tv = false compute on
// zero keys and write nothing).
DEVI void route_row16(const float* row, bool tv, int E, int k, int score_fn, int l16,
                      int32_t* ids_out, float* w_out, int32_t* ids_lds) {
  uint32_t key[16];
  if (((E & 3) | ((uintptr_t)row & 15)) == 0) {   // 16-byte aligned rows: four experts per load
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e0 = 4 * l16 + 64 * q;
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      const bool ok = tv && e0 < E;
      if (ok) f = *(const float4*)(row + e0);
      key[4 * q + 0] = ok ? score_key(f.x) : 0u;
      key[4 * q + 1] = ok ? score_key(f.y) : 0u;
      key[4 * q + 2] = ok ? score_key(f.z) : 0u;
      key[4 * q + 3] = ok ? score_key(f.w) : 0u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = 4 * l16 + (i & 3) + 64 * (i >> 2);
      key[i] = (tv && e < E) ? score_key(row[e]) : 0u;
    }
  }
  // finite scores have keys >= 0x00800000, so 0 marks an absent or taken expert
  uint32_t my_id = 0, my_key = 0, top_key = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = key[i] > m ? key[i] : m;
    m = row16_max(m);
    uint32_t be = 0xFFFFu;
#pragma unroll
    for (int i = 15; i >= 0; --i)   // indices grow with i: the lowest match wins
      be = key[i] == m ? (uint32_t)(4 * l16 + (i & 3) + 64 * (i >> 2)) : be;
    be = row16_min(be);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      key[i] = (uint32_t)(4 * l16 + (i & 3) + 64 * (i >> 2)) == be ? 0u : key[i];
    top_key = j == 0 ? m : top_key;
    my_id = l16 == j ? be : my_id;
    my_key = l16 == j ? m : my_key;
  }
  const float lv = key_score(my_key), top = key_score(top_key);
  float v = score_fn == MOE_SCORE_SOFTMAX ? expf(lv - top)
            : score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-lv)) : lv;
  v = l16 < k ? v : 0.f;
  const float sum = row16_sum(v);
  if (tv && l16 < k) {
    ids_out[l16] = (int32_t)my_id;
    w_out[l16] = v / sum;
    if (ids_lds) ids_lds[l16] = (int32_t)my_id;
  }
}

