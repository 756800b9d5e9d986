// Attention-recall diagnostic: the share of each sampled query's dense
// softmax mass that falls inside the key tiles its row keeps (RainFusion
// review page, "What carries the argument": the masked recall R', mass
// surviving a mask over the mass with no mask).
//
// One workgroup per (sample, b*H + h), one thread per query slot of the
// sampled tile.  The row's kept tiles become a bitmap in LDS; keys are
// streamed in chunks of 32 rows through LDS (every thread reads the same key
// row, an LDS broadcast), and each thread keeps, in log2 units, a running
// maximum m, the total mass T and the kept mass K, rescaled together once per
// chunk.  fp32 throughout; a diagnostic, not on the hot path.
#include "rf_internal.h"

#include <math.h>

namespace {

constexpr int kChunk = 32;              // key rows staged per step (one validity word)
constexpr int kMaxBitmapWords = 8192;   // 262144 tiles

template <int E>
__device__ inline float ld(const uint8_t* p, int64_t i) {
  if constexpr (E == 2) {
    const uint32_t u = uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16;
    return __uint_as_float(u);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <int E, int D, int BS>
__global__ __launch_bounds__(BS) void recall_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ kp,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ samples,
    int32_t n_sample, float* __restrict__ out,
    const uint32_t* __restrict__ tile_bits, int64_t Lt, int32_t nb,
    int32_t n_tt, int32_t row_len_video, int64_t nnz, float scale_log2) {
  extern __shared__ uint32_t kept_bits[];      // [(n_tiles + 31) / 32]
  __shared__ float kc[kChunk][D];
  const int32_t s = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int t = threadIdx.x;
  const int32_t n_tiles = nb + n_tt;
  float* dst = out + (bh * n_sample + s) * BS;
  const int32_t qt = samples[s];
  if (qt < 0 || qt >= n_tiles) {               // uniform over the workgroup
    dst[t] = NAN;
    return;
  }
  // Kept-tile bitmap of the sampled row.
  const int words = (n_tiles + 31) / 32;
  for (int w = t; w < words; w += BS) kept_bits[w] = 0u;
  __syncthreads();
  const int32_t row_len = qt < nb ? row_len_video : n_tiles;
  const int64_t row0 = qt < nb ? int64_t(qt) * row_len_video
                               : int64_t(nb) * row_len_video + int64_t(qt - nb) * n_tiles;
  const int32_t* row = kept + bh * nnz + row0;
  for (int j = t; j < row_len; j += BS) {
    const int32_t kt = row[j];
    if (kt >= 0 && kt < n_tiles) atomicOr(&kept_bits[kt / 32], 1u << (kt % 32));
  }
  __syncthreads();

  float q[D];
  const int64_t qrow = int64_t(qt) * BS + t;
  const uint8_t* qsrc = qp + ((bh * Lt + qrow) * D) * E;
#pragma unroll
  for (int c = 0; c < D; ++c) q[c] = ld<E>(qsrc, c);
  const bool qvalid = (tile_bits[qt * 4 + t / 32] >> (t % 32)) & 1u;

  float m = -INFINITY, tot = 0.f, kmass = 0.f;
  const uint8_t* kh = kp + (bh * Lt * D) * E;
  for (int32_t kt = 0; kt < n_tiles; ++kt) {
    const bool is_kept = (kept_bits[kt / 32] >> (kt % 32)) & 1u;
    for (int c0 = 0; c0 < BS; c0 += kChunk) {
      const uint32_t vbits = tile_bits[kt * 4 + c0 / 32] >> (c0 % 32);
      if (vbits == 0u) continue;                // uniform: no valid key in the chunk
      __syncthreads();
      for (int i = t; i < kChunk * D; i += BS) {
        const int r = i / D, c = i % D;
        kc[r][c] = ld<E>(kh, (int64_t(kt) * BS + c0 + r) * D + c);
      }
      __syncthreads();
      float lg[kChunk];
      float cm = -INFINITY;
#pragma unroll 4
      for (int r = 0; r < kChunk; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc = fmaf(q[c], kc[r][c], acc);
        lg[r] = ((vbits >> r) & 1u) ? acc * scale_log2 : -INFINITY;
        cm = fmaxf(cm, lg[r]);
      }
      if (cm > m) {
        const float a = m == -INFINITY ? 0.f : exp2f(m - cm);
        tot *= a;
        kmass *= a;
        m = cm;
      }
      float ct = 0.f;
#pragma unroll 4
      for (int r = 0; r < kChunk; ++r) ct += exp2f(lg[r] - m);
      tot += ct;
      if (is_kept) kmass += ct;
    }
  }
  dst[t] = qvalid ? kmass / tot : NAN;
}

template <int E, int D, int BS>
void launch(const rf_plan* p, const void* qp, const void* kp, const int32_t* kept,
            const int32_t* samples, int32_t n_sample, float* out, int BH,
            const rf_keep& kc, float scale, hipStream_t st) {
  const int words = (p->sz.n_tiles + 31) / 32;
  hipLaunchKernelGGL((recall_kernel<E, D, BS>), dim3(n_sample, BH), dim3(BS),
                     words * sizeof(uint32_t), st, static_cast<const uint8_t*>(qp),
                     static_cast<const uint8_t*>(kp), kept, samples, n_sample, out,
                     p->tile_bits, p->sz.Lt, p->sz.nb, p->sz.n_text_tiles,
                     kc.row_len_video, kc.nnz_per_head, scale * 1.4426950408889634f);
}

}  // namespace

extern "C" rf_status rf_attention_recall(const rf_plan* plan, const void* qp,
                                         const void* kp, const int32_t* kept_idx,
                                         int32_t sparsity_pct,
                                         const int32_t* sample_tiles,
                                         int32_t n_sample, int32_t B, int32_t H,
                                         int32_t d, float scale, rf_dtype dtype,
                                         float* recall, hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, "rf_attention_recall");
  if (st != RF_OK) return st;
  if (!rf::aligned16(qp) || !rf::aligned16(kp) || !rf::aligned16(kept_idx) ||
      sample_tiles == nullptr || (reinterpret_cast<uintptr_t>(sample_tiles) & 3u) ||
      !rf::aligned16(recall))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_attention_recall: null or misaligned buffer");
  if (n_sample < 1 || n_sample > 65535)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_attention_recall: n_sample must be in [1, 65535]");
  if (!(scale > 0.f) || !(scale < 1e30f))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_attention_recall: scale must be positive and finite");
  if ((plan->sz.n_tiles + 31) / 32 > kMaxBitmapWords)
    return rf::fail(RF_ERR_UNSUPPORTED, "rf_attention_recall: more than %d tiles",
                    kMaxBitmapWords * 32);
  rf_keep kc;
  st = rf_keep_count(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  const int BH = B * H;
  const int bs = plan->sz.bs;
  const bool bf = dtype == RF_BF16;
  if (bf && d == 128 && bs == 128) launch<2, 128, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else if (bf && d == 128 && bs == 64) launch<2, 128, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else if (bf && d == 64 && bs == 128) launch<2, 64, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else if (bf && d == 64 && bs == 64) launch<2, 64, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else if (!bf && d == 128 && bs == 128) launch<4, 128, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else if (!bf && d == 128 && bs == 64) launch<4, 128, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else if (!bf && d == 64 && bs == 128) launch<4, 64, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  else launch<4, 64, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, recall, BH, kc, scale, stream);
  return rf::check_launch("rf_attention_recall");
}
