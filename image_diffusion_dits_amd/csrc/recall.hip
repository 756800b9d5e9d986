// Attention-recall diagnostic: the share of each sampled query's dense
// softmax mass that falls inside the key tiles its row keeps (RainFusion
// review page, "What carries the argument": the masked recall R', mass
// surviving a mask over the mass with no mask).
//
// One workgroup per (sample, b*H + h); the row's kept tiles become a bitmap
// in LDS.  Each lane keeps, in log2 units, a running maximum m, the total
// mass T and the kept mass K, rescaled together per block of keys.
//   bf16: four waves split the sequence's 32-key blocks; each wave holds all
//         query slots of the sampled tile as MFMA operands and takes the
//         logits of 32 keys x 32 queries per v_mfma_f32_32x32x16_bf16 chain;
//         the waves' partial sums are merged through LDS at the end.
//   fp32: one thread per query slot, fp32 FMA over key rows staged 32 at a
//         time through LDS (every thread reads the same row).
#include "rf_internal.h"
#include "mass.h"

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
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, qt, nb, row_len_video, n_tiles);
  const int32_t row_len = rr.len;
  const int32_t* row = kept + bh * nnz + rr.offset;
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
#pragma unroll
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
#pragma unroll
      for (int r = 0; r < kChunk; ++r) ct += exp2f(lg[r] - m);
      tot += ct;
      if (is_kept) kmass += ct;
    }
  }
  dst[t] = qvalid ? kmass / tot : NAN;
}

constexpr int kMfmaWaves = 4;

template <int D, int BS>
__global__ __launch_bounds__(kMfmaWaves * 64) void recall_mfma_kernel(
    const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ samples,
    int32_t n_sample, float* __restrict__ out,
    const uint32_t* __restrict__ tile_bits, int64_t Lt, int32_t nb,
    int32_t n_tt, int32_t row_len_video, int64_t nnz, float scale_log2) {
  using namespace rf_mass;
  constexpr int NQ = BS / 32;                  // 32-query blocks of the tile
  constexpr int kThreads = kMfmaWaves * 64;
  extern __shared__ uint32_t kept_bits[];      // [(n_tiles + 31) / 32]
  __shared__ float part[kMfmaWaves][3][NQ][32];
  const int32_t s = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int t = threadIdx.x, w = t / 64, lane = t % 64, li = lane % 32, g = lane / 32;
  const int32_t n_tiles = nb + n_tt;
  float* dst = out + (bh * n_sample + s) * BS;
  const int32_t qt = samples[s];
  if (qt < 0 || qt >= n_tiles) {               // uniform over the workgroup
    if (t < BS) dst[t] = NAN;
    return;
  }
  const int words = (n_tiles + 31) / 32;
  for (int x = t; x < words; x += kThreads) kept_bits[x] = 0u;
  __syncthreads();
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, qt, nb, row_len_video, n_tiles);
  const int32_t* row = kept + bh * nnz + rr.offset;
  for (int j = t; j < rr.len; j += kThreads) {
    const int32_t kt = row[j];
    if (kt >= 0 && kt < n_tiles) atomicOr(&kept_bits[kt / 32], 1u << (kt % 32));
  }
  __syncthreads();

  const __bf16* qh = qp + bh * Lt * D;
  const __bf16* kh = kp + bh * Lt * D;
  bf16x8 qf[NQ][D / 16];
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb)
    load_row<D>(qh + (int64_t(qt) * BS + qb * 32 + li) * D, g, qf[qb]);
  Mass acc[NQ];
  // Key blocks j = tile * NQ + block; wave w takes j = w, w + 4, ...
  const int32_t nblk = n_tiles * NQ;
  bf16x8 kf[D / 16], kn[D / 16];
  if (w < nblk) load_row<D>(kh + (int64_t(w) * 32 + li) * D, g, kf);
  for (int32_t j = w; j < nblk; j += kMfmaWaves) {
    if (j + kMfmaWaves < nblk)
      load_row<D>(kh + (int64_t(j + kMfmaWaves) * 32 + li) * D, g, kn);
    const int32_t kt = j / NQ;
    const uint32_t vword = tile_bits[kt * 4 + j % NQ];
    uint32_t valid = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) valid |= ((vword >> key_of(r, g)) & 1u) << r;
    const uint32_t keep = ((kept_bits[kt / 32] >> (kt % 32)) & 1u) ? 0xFFFFu : 0u;
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) acc[qb].absorb(logits<D>(kf, qf[qb]), valid, keep, scale_log2);
#pragma unroll
    for (int m = 0; m < D / 16; ++m) kf[m] = kn[m];
  }
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    acc[qb].merge_halves();
    if (g == 0) {
      part[w][0][qb][li] = acc[qb].m;
      part[w][1][qb][li] = acc[qb].tot;
      part[w][2][qb][li] = acc[qb].kmass;
    }
  }
  __syncthreads();
  if (t < BS) {
    const int qb = t / 32, q = t % 32;
    Mass total;
#pragma unroll
    for (int x = 0; x < kMfmaWaves; ++x)
      total.merge(part[x][0][qb][q], part[x][1][qb][q], part[x][2][qb][q]);
    const bool qvalid = (tile_bits[qt * 4 + t / 32] >> (t % 32)) & 1u;
    dst[t] = qvalid ? total.kmass / total.tot : NAN;
  }
}

template <int E, int D, int BS>
void launch(const rf_plan* p, const void* qp, const void* kp, const int32_t* kept,
            const int32_t* samples, int32_t n_sample, float* out, int BH,
            int32_t row_len_video, int64_t nnz, float scale, hipStream_t st) {
  const int words = (p->sz.n_tiles + 31) / 32;
  if constexpr (E == 2) {
    hipLaunchKernelGGL((recall_mfma_kernel<D, BS>), dim3(n_sample, BH), dim3(kMfmaWaves * 64),
                       words * sizeof(uint32_t), st, static_cast<const __bf16*>(qp),
                       static_cast<const __bf16*>(kp), kept, samples, n_sample, out,
                       p->tile_bits, p->sz.Lt, p->sz.nb, p->sz.n_text_tiles,
                       row_len_video, nnz, scale * 1.4426950408889634f);
  } else {
    hipLaunchKernelGGL((recall_kernel<E, D, BS>), dim3(n_sample, BH), dim3(BS),
                       words * sizeof(uint32_t), st, static_cast<const uint8_t*>(qp),
                       static_cast<const uint8_t*>(kp), kept, samples, n_sample, out,
                       p->tile_bits, p->sz.Lt, p->sz.nb, p->sz.n_text_tiles,
                       row_len_video, nnz, scale * 1.4426950408889634f);
  }
}

rf_status recall(const rf_plan* plan, const void* qp, const void* kp,
                 const int32_t* kept_idx, int32_t row_len_video, int64_t nnz,
                 const int32_t* sample_tiles, int32_t n_sample, int32_t B,
                 int32_t H, int32_t d, float scale, rf_dtype dtype,
                 float* out, hipStream_t stream, const char* fn) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, fn);
  if (st != RF_OK) return st;
  if (!rf::aligned16(qp) || !rf::aligned16(kp) || !rf::aligned16(kept_idx) ||
      sample_tiles == nullptr || (reinterpret_cast<uintptr_t>(sample_tiles) & 3u) ||
      !rf::aligned16(out))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  if (n_sample < 1 || n_sample > 65535)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: n_sample must be in [1, 65535]", fn);
  if (!(scale > 0.f) || !(scale < 1e30f))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if ((plan->sz.n_tiles + 31) / 32 > kMaxBitmapWords)
    return rf::fail(RF_ERR_UNSUPPORTED, "%s: more than %d tiles", fn, kMaxBitmapWords * 32);
  const int BH = B * H;
  const int bs = plan->sz.bs;
  const bool bf = dtype == RF_BF16;
  const int32_t rl = row_len_video;
  if (bf && d == 128 && bs == 128) launch<2, 128, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else if (bf && d == 128 && bs == 64) launch<2, 128, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else if (bf && d == 64 && bs == 128) launch<2, 64, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else if (bf && d == 64 && bs == 64) launch<2, 64, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else if (!bf && d == 128 && bs == 128) launch<4, 128, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else if (!bf && d == 128 && bs == 64) launch<4, 128, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else if (!bf && d == 64 && bs == 128) launch<4, 64, 128>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  else launch<4, 64, 64>(plan, qp, kp, kept_idx, sample_tiles, n_sample, out, BH, rl, nnz, scale, stream);
  return rf::check_launch(fn);
}

}  // namespace

extern "C" rf_status rf_attention_recall(const rf_plan* plan, const void* qp,
                                         const void* kp, const int32_t* kept_idx,
                                         int32_t sparsity_pct,
                                         const int32_t* sample_tiles,
                                         int32_t n_sample, int32_t B, int32_t H,
                                         int32_t d, float scale, rf_dtype dtype,
                                         float* recall_out, hipStream_t stream) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_attention_recall: null plan");
  rf_keep kc;
  rf_status st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  return recall(plan, qp, kp, kept_idx, kc.row_len_video, kc.nnz_per_head, sample_tiles,
                n_sample, B, H, d, scale, dtype, recall_out, stream, "rf_attention_recall");
}

extern "C" rf_status rf_attention_recall_rows(const rf_plan* plan, const void* qp,
                                              const void* kp, const int32_t* kept_rows,
                                              int32_t row_width,
                                              const int32_t* sample_tiles,
                                              int32_t n_sample, int32_t B, int32_t H,
                                              int32_t d, float scale, rf_dtype dtype,
                                              float* recall_out, hipStream_t stream) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_attention_recall_rows: null plan");
  if (row_width < 1 || row_width > plan->sz.n_tiles)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_attention_recall_rows: row_width %d outside [1, %d]",
                    row_width, plan->sz.n_tiles);
  return recall(plan, qp, kp, kept_rows, -row_width, int64_t(plan->sz.n_tiles) * row_width,
                sample_tiles, n_sample, B, H, d, scale, dtype, recall_out, stream,
                "rf_attention_recall_rows");
}
