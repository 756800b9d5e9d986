// Softmax-mass bookkeeping shared by the recall diagnostics: logits of 32
// keys x 32 queries come from v_mfma_f32_32x32x16_bf16 (S^T = K Q^T, A = key
// rows, B = query rows, both gathered straight from global memory), and each
// lane keeps, for its query, a running maximum m, the total mass and the
// mass on kept keys, in log2 units.
//
// Accumulator layout of a 32x32 MFMA block: lane (li, g) = (lane % 32,
// lane / 32) holds column li (the query) and rows key_of(r, g), r < 16 (the
// keys), so the two lane groups of one query see disjoint halves of the keys
// and are merged once at the end.
#pragma once

#include "rf_internal.h"

#include <math.h>

namespace rf_mass {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

__device__ constexpr int key_of(int r, int g) { return 8 * (r / 4) + 4 * g + (r % 4); }

// MFMA operand fragments of one token row (bf16, d = D): chunk m holds
// elements 16m + 8g .. 16m + 8g + 7.
template <int D>
__device__ inline void load_row(const __bf16* row, int g, bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
    f[m] = *reinterpret_cast<const bf16x8*>(row + 16 * m + 8 * g);
}

// Logits block S^T[key][query] = sum_c k[key][c] q[query][c] (unscaled).
template <int D>
__device__ inline f32x16 logits(const bf16x8 (&k)[D / 16], const bf16x8 (&q)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[m], q[m], s, 0, 0, 0);
  return s;
}

struct Mass {
  float m = -INFINITY, tot = 0.f, kmass = 0.f;

  // Adds the 16 logits of this lane: bit r of `valid` marks a real key,
  // bit r of `keep` a key inside the mask.
  __device__ inline void absorb(const f32x16& s, uint32_t valid, uint32_t keep,
                                float scale_log2) {
    float l[16];
    float cm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      l[r] = ((valid >> r) & 1u) ? s[r] * scale_log2 : -INFINITY;
      cm = fmaxf(cm, l[r]);
    }
    if (cm > m) {
      const float f = m == -INFINITY ? 0.f : exp2f(m - cm);
      tot *= f;
      kmass *= f;
      m = cm;
    }
    if (m == -INFINITY) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = exp2f(l[r] - m);
      tot += e;
      kmass += ((keep >> r) & 1u) ? e : 0.f;
    }
  }

  // Combines the two lane groups of each query (lane and lane ^ 32).
  __device__ inline void merge_halves() {
    const float m2 = __shfl_xor(m, 32), t2 = __shfl_xor(tot, 32), k2 = __shfl_xor(kmass, 32);
    merge(m2, t2, k2);
  }

  __device__ inline void merge(float m2, float t2, float k2) {
    const float mt = fmaxf(m, m2);
    const float fa = m == -INFINITY ? 0.f : exp2f(m - mt);
    const float fb = m2 == -INFINITY ? 0.f : exp2f(m2 - mt);
    tot = tot * fa + t2 * fb;
    kmass = kmass * fa + k2 * fb;
    m = mt;
  }
};

}  // namespace rf_mass
