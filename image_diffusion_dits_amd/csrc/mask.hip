// Online sparse-mask prediction from the block representative tokens
// (RainFusion2.0 page, Abstract key insights (1) mean tokens for sparse mask
// prediction and (3) first-frame sink; TL;DR).
//
// For query block i of head (b, h): logits l_ij = qbar_i . kbar_j / sqrt(d)
// over the video key blocks, keep the sink blocks plus the k_eff - n_sink
// highest non-sink logits (ties to the lower block index), then every text
// tile.  The row softmax is monotone, so ranking by the raw fp32 dot product
// is ranking by the softmax score.
//
// One workgroup serves R query rows of one head:
//   1. the R x nb dot products, kept in LDS.  Up to 1024 blocks per row:
//      R = 16 (three workgroups per CU for the selection below to spread
//      over) and the dots come from fp32 MFMA (v_mfma_f32_16x16x4_f32), each
//      wave taking every fourth group of 16 keys with the query rows held in
//      registers.  Beyond that: R = 4 and every thread
//      owns key blocks and accumulates R dots with fp32 FMA (query rows read
//      by LDS broadcast);
//   2. each wave selects for its rows: an exact k-th-largest search over the
//      order-preserving integer image of the fp32 dots (32 bisection steps of
//      wave-wide ballots), then an ascending ballot/prefix-count compaction
//      that also breaks ties by index.  No atomics: the result is bitwise
//      deterministic.
#include "rf_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ inline uint32_t order_key(float f) {
  if (f == 0.f) f = 0.f;  // -0 and +0 rank equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int popc64(uint64_t m) { return __popcll(m); }

// One wave selects one row: the k_sel largest keys among the non-sink
// blocks (ties to the lower index), plus every sink, written ascending,
// then the text tiles.  Lane l holds blocks l + 64 m (m < MMAX) in
// registers as order-preserving keys, 0 for sinks and out-of-range blocks
// (0 is below the key of every float, so they are never counted).
//   tau: the largest t with #{key >= t} >= k_sel, found bit by bit from the
//        top (wave ballots count); once #{key >= t} == k_sel exactly, the
//        kept set is {key >= t} and the search stops.
//   keep key > tau, and of the keys == tau the lowest-indexed
//   k_sel - #{key > tau}; the ascending compaction is a ballot prefix count.
// The sink bits of lane l's blocks l + 64 m (bit m of a 64-bit mask, as
// MMAX reaches 64), the same for every row: loaded once per wave, all loads
// in flight together.
template <int MMAX>
__device__ __attribute__((always_inline)) uint64_t sink_bits(const uint8_t* __restrict__ is_sink,
                                                             int nb, int lane) {
  static_assert(MMAX <= 64, "one mask bit per register chunk");
  uint64_t sinkm = 0;
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    const int j = lane + 64 * m;
    const uint32_t sk = is_sink[min(j, nb - 1)];
    sinkm |= uint64_t(j < nb && sk != 0) << m;
  }
  return sinkm;
}

template <int MMAX>
__device__ __attribute__((always_inline)) void select_row(const float* __restrict__ row,
                                                          uint64_t sinkm, int nb, int k_sel,
                                                          int k_eff, int n_tt,
                                                          int32_t* __restrict__ out, int lane) {
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t key[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    const int j = lane + 64 * m;
    const uint32_t k = order_key(row[min(j, nb - 1)]);
    key[m] = (j < nb && !((sinkm >> m) & 1ull)) ? k : 0u;
  }
  uint32_t tau = 0;
  if (k_sel > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = tau | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int m = 0; m < MMAX; ++m) cnt += popc64(__ballot(key[m] >= t));
      if (cnt >= k_sel) {
        tau = t;
        if (cnt == k_sel) break;
      }
    }
  }
  int n_gt = 0;
  if (k_sel > 0) {
#pragma unroll
    for (int m = 0; m < MMAX; ++m) n_gt += popc64(__ballot(key[m] > tau));
  }
  const int n_eq_take = k_sel - n_gt;
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    const int j = lane + 64 * m;
    const bool sink = (sinkm >> m) & 1ull;
    const bool eq = k_sel > 0 && key[m] != 0 && key[m] == tau;
    bool keep = sink || (k_sel > 0 && key[m] > tau);
    const uint64_t eqm = __ballot(eq);
    if (eq && eq_seen + popc64(eqm & lt_mask) < n_eq_take) keep = true;
    eq_seen += popc64(eqm);
    const uint64_t km = __ballot(keep);
    const int at = pos + popc64(km & lt_mask);
    if (keep && at < k_eff) out[at] = j;
    pos += popc64(km);
  }
  for (int t = lane; t < n_tt; t += 64) out[k_eff + t] = nb + t;
}

template <int D, int R, int MMAX>
__global__ __launch_bounds__(kThreads) void predict_mask_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar,
    const uint8_t* __restrict__ is_sink, int32_t* __restrict__ kept,
    float* __restrict__ logits, int32_t nb, int32_t n_sink, int32_t k_eff,
    int32_t n_tt, int32_t row_len, int64_t nnz, float scale) {
  extern __shared__ float smem[];
  float* qs = smem;            // [R][D]
  float* sc = smem + R * D;    // [R][nb]
  const int64_t bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const float* qh = qbar + bh * nb * D;
  const float* kh = kbar + bh * nb * D;
  for (int t = threadIdx.x; t < R * D; t += kThreads) {
    const int r = t / D;
    qs[t] = (i0 + r < nb) ? qh[int64_t(i0 + r) * D + t % D] : 0.f;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += kThreads) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    const float4* kr = reinterpret_cast<const float4*>(kh + int64_t(j) * D);
#pragma unroll 4
    for (int c = 0; c < D / 4; ++c) {
      const float4 kv = kr[c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4 qv = reinterpret_cast<const float4*>(qs + r * D)[c];
        acc[r] = fmaf(kv.x, qv.x, acc[r]);
        acc[r] = fmaf(kv.y, qv.y, acc[r]);
        acc[r] = fmaf(kv.z, qv.z, acc[r]);
        acc[r] = fmaf(kv.w, qv.w, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sc[r * nb + j] = acc[r];
      if (logits != nullptr && i0 + r < nb)
        logits[(bh * nb + i0 + r) * nb + j] = acc[r] * scale;
    }
  }
  __syncthreads();

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int k_sel = k_eff - n_sink;
  const uint64_t sinkm = sink_bits<MMAX>(is_sink, nb, lane);
  for (int r = wave; r < R; r += kWaves) {
    const int i = i0 + r;
    if (i >= nb) break;
    select_row<MMAX>(sc + r * nb, sinkm, nb, k_sel, k_eff, n_tt,
                     kept + bh * nnz + int64_t(i) * row_len, lane);
  }
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Dots on MFMA for R = 16 query rows and 16 key blocks at a time
// (v_mfma_f32_16x16x4_f32).  Lane (li, q) = (lane % 16, lane / 16) supplies
// A[i = li][k] = qbar[i0 + li][k] and B[k][j = li] = kbar[j0 + li][k] for
// the k = 16c + 4q + e (c < D/16, e < 4) it loads as float4; the product
// sums over all k whatever their order, and accumulator register r holds
// row 4q + r, column li.
template <int D, int MMAX>
__global__ __launch_bounds__(kThreads) void predict_mask_mfma_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar,
    const uint8_t* __restrict__ is_sink, int32_t* __restrict__ kept,
    float* __restrict__ logits, int32_t nb, int32_t n_sink, int32_t k_eff,
    int32_t n_tt, int32_t row_len, int64_t nnz, float scale) {
  constexpr int R = 16;
  extern __shared__ float sc[];          // [R][nb]
  const int64_t bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int li = lane % 16, q = lane / 16;
  const float* qh = qbar + bh * nb * D;
  const float* kh = kbar + bh * nb * D;
  float4 qf[D / 16];
  {
    const float4* qr = reinterpret_cast<const float4*>(qh + int64_t(min(i0 + li, nb - 1)) * D);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qf[c] = qr[4 * c + q];
  }
  const int nkb = (nb + 15) / 16;
  // The next block's key rows are loaded while this block's MFMAs run.
  auto load_keys = [&](int kb, float4 (&kf)[D / 16]) {
    const float4* kr =
        reinterpret_cast<const float4*>(kh + int64_t(min(kb * 16 + li, nb - 1)) * D);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) kf[c] = kr[4 * c + q];
  };
  float4 kn[D / 16];
  if (wave < nkb) load_keys(wave, kn);
  for (int kb = wave; kb < nkb; kb += kWaves) {
    const int j = kb * 16 + li;
    float4 kf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) kf[c] = kn[c];
    if (kb + kWaves < nkb) load_keys(kb + kWaves, kn);
    f32x4v acc = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[c].x, kf[c].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[c].y, kf[c].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[c].z, kf[c].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[c].w, kf[c].w, acc, 0, 0, 0);
    }
    if (j < nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * q + r;
        sc[i * nb + j] = acc[r];
        if (logits != nullptr && i0 + i < nb)
          logits[(bh * nb + i0 + i) * nb + j] = acc[r] * scale;
      }
    }
  }
  __syncthreads();
  const int k_sel = k_eff - n_sink;
  const uint64_t sinkm = sink_bits<MMAX>(is_sink, nb, lane);
  for (int r = wave; r < R; r += kWaves) {
    const int i = i0 + r;
    if (i >= nb) break;
    select_row<MMAX>(sc + r * nb, sinkm, nb, k_sel, k_eff, n_tt,
                     kept + bh * nnz + int64_t(i) * row_len, lane);
  }
}

// Text query tiles attend to every tile.
__global__ void text_rows_kernel(int32_t* __restrict__ kept, int32_t nb,
                                 int32_t n_tiles, int32_t row_len_video,
                                 int64_t nnz) {
  const int64_t bh = blockIdx.y;
  int32_t* out = kept + bh * nnz + int64_t(nb) * row_len_video +
                 int64_t(blockIdx.x) * n_tiles;
  for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) out[t] = t;
}

// Dense copy of the kept sets, one workgroup per (query tile, head): the
// row is cleared, then each kept entry sets its byte.
__global__ void dense_mask_kernel(const int32_t* __restrict__ kept,
                                  uint8_t* __restrict__ mask, int32_t nb,
                                  int32_t n_tiles, int32_t row_len_video,
                                  int64_t nnz) {
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x;
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, tile, nb, row_len_video, n_tiles);
  const int32_t* row = kept + bh * nnz + rr.offset;
  uint8_t* dst = mask + (bh * n_tiles + tile) * int64_t(n_tiles);
  for (int t = threadIdx.x; t < n_tiles; t += blockDim.x) dst[t] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < rr.len; j += blockDim.x) {
    const int32_t t = row[j];
    if (t >= 0 && t < n_tiles) dst[t] = 1;
  }
}

template <int D, int MMAX>
void launch_mfma(const rf_plan* p, const float* qbar, const float* kbar,
                 int32_t* kept, float* logits, int BH, const rf_keep& kc,
                 hipStream_t st) {
  const int nb = p->sz.nb;
  const size_t lds = sizeof(float) * 16 * size_t(nb);
  dim3 grid((nb + 15) / 16, BH);
  hipLaunchKernelGGL((predict_mask_mfma_kernel<D, MMAX>), grid, dim3(kThreads), lds, st,
                     qbar, kbar, p->is_sink, kept, logits, nb, p->sz.n_sink,
                     kc.k_eff, p->sz.n_text_tiles, kc.row_len_video,
                     kc.nnz_per_head, 1.0f / sqrtf(float(D)));
}

template <int D>
void launch_mfma_any(const rf_plan* p, const float* qbar, const float* kbar,
                     int32_t* kept, float* logits, int BH, const rf_keep& kc,
                     hipStream_t st) {
  const int chunks = (p->sz.nb + 63) / 64;
  if (chunks <= 4) launch_mfma<D, 4>(p, qbar, kbar, kept, logits, BH, kc, st);
  else if (chunks <= 8) launch_mfma<D, 8>(p, qbar, kbar, kept, logits, BH, kc, st);
  else if (chunks <= 12) launch_mfma<D, 12>(p, qbar, kbar, kept, logits, BH, kc, st);
  else launch_mfma<D, 16>(p, qbar, kbar, kept, logits, BH, kc, st);
}

template <int D, int R, int MMAX>
void launch(const rf_plan* p, const float* qbar, const float* kbar,
            int32_t* kept, float* logits, int BH, const rf_keep& kc,
            hipStream_t st) {
  const int nb = p->sz.nb;
  const size_t lds = sizeof(float) * (size_t(R) * D + size_t(R) * nb);
  dim3 grid((nb + R - 1) / R, BH);
  hipLaunchKernelGGL((predict_mask_kernel<D, R, MMAX>), grid, dim3(kThreads), lds, st,
                     qbar, kbar, p->is_sink, kept, logits, nb, p->sz.n_sink,
                     kc.k_eff, p->sz.n_text_tiles, kc.row_len_video,
                     kc.nnz_per_head, 1.0f / sqrtf(float(D)));
}

template <int D, int MMAX>
hipError_t allow_mfma_lds() {
  // The largest row this instantiation serves: nb <= 64 MMAX (and <= 1024).
  const int nb = 64 * MMAX < 1024 ? 64 * MMAX : 1024;
  return hipFuncSetAttribute(
      reinterpret_cast<const void*>(&predict_mask_mfma_kernel<D, MMAX>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(sizeof(float) * 16 * nb));
}

template <int D, int R, int MMAX>
hipError_t allow_lds() {
  return hipFuncSetAttribute(
      reinterpret_cast<const void*>(&predict_mask_kernel<D, R, MMAX>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      int(sizeof(float) * (size_t(R) * D + size_t(R) * 4096)));
}

}  // namespace

// Raises the dynamic-LDS limit of every mask kernel to the most it can ask
// for, once per plan (at creation, on the plan's device) instead of on every
// rf_predict_mask call.
rf_status rf::prepare_mask_kernels() {
  const hipError_t errs[] = {
      allow_mfma_lds<128, 4>(), allow_mfma_lds<128, 8>(), allow_mfma_lds<128, 12>(),
      allow_mfma_lds<128, 16>(), allow_mfma_lds<64, 4>(), allow_mfma_lds<64, 8>(),
      allow_mfma_lds<64, 12>(), allow_mfma_lds<64, 16>(), allow_lds<128, 4, 64>(),
      allow_lds<64, 4, 64>()};
  for (hipError_t e : errs)
    if (e != hipSuccess)
      return rf::fail(RF_ERR_HIP, "mask kernel LDS limit: %s", hipGetErrorString(e));
  return RF_OK;
}

extern "C" rf_status rf_predict_mask(const rf_plan* plan, const float* qbar,
                                     const float* kbar, int32_t B, int32_t H,
                                     int32_t d, int32_t sparsity_pct,
                                     int32_t* kept_idx, uint8_t* mask_or_null,
                                     float* logits_or_null, hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, RF_F32, "rf_predict_mask");
  if (st != RF_OK) return st;
  if (!rf::aligned16(qbar) || !rf::aligned16(kbar) || !rf::aligned16(kept_idx))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_predict_mask: null or misaligned buffer");
  if (logits_or_null != nullptr && !rf::aligned16(logits_or_null))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_predict_mask: misaligned logits");
  rf_keep kc;
  st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  const int nb = plan->sz.nb;
  // Dots of R rows x nb blocks must fit in LDS next to the R query rows.
  const size_t budget = 128 * 1024;
  const int BH = B * H;
  // Rows per workgroup R: their dots must fit in LDS next to the R query
  // rows.  MMAX: register chunks per lane for the selection (nb <= 64 MMAX).
  if (nb <= 1024) {
    if (d == 128) launch_mfma_any<128>(plan, qbar, kbar, kept_idx, logits_or_null, BH, kc, stream);
    else launch_mfma_any<64>(plan, qbar, kbar, kept_idx, logits_or_null, BH, kc, stream);
  } else if (nb <= 4096 && sizeof(float) * 4 * (size_t(nb) + d) <= budget) {
    if (d == 128) launch<128, 4, 64>(plan, qbar, kbar, kept_idx, logits_or_null, BH, kc, stream);
    else launch<64, 4, 64>(plan, qbar, kbar, kept_idx, logits_or_null, BH, kc, stream);
  } else {
    return rf::fail(RF_ERR_UNSUPPORTED, "rf_predict_mask: %d blocks per row "
                    "exceed the supported maximum of 4096", nb);
  }
  if (plan->sz.n_text_tiles > 0) {
    dim3 grid(plan->sz.n_text_tiles, BH);
    hipLaunchKernelGGL(text_rows_kernel, grid, dim3(256), 0, stream, kept_idx,
                       nb, plan->sz.n_tiles, kc.row_len_video, kc.nnz_per_head);
  }
  if (mask_or_null != nullptr) {
    dim3 grid(plan->sz.n_tiles, BH);
    hipLaunchKernelGGL(dense_mask_kernel, grid, dim3(256), 0, stream, kept_idx,
                       mask_or_null, nb, plan->sz.n_tiles, kc.row_len_video,
                       kc.nnz_per_head);
  }
  return rf::check_launch("rf_predict_mask");
}
