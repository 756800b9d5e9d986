// Head-pattern masks and the online pattern classifier of RainFusion v1
// ("RainFusion: Adaptive Video Generation Acceleration via Multi-Dimensional
// Visual Redundancy", review page: "What carries the argument", "Core claim"
// and the free-parameter list), expressed on the tiles of the block-sparse
// attention so that they feed the same kernel as the RainFusion2.0 mask.
//
//   spatial   video tile i keeps video tile j when |i - j| <= band, tiles in
//             frame-major order (the block index);
//   temporal  |r(i) - r(j)| <= band, r the tile's position in spatial-major
//             order (tiles sorted by (h, w, t) of their first token);
//   textural  j = i (mod tau): the checkerboard that keeps one residue class.
// Text tiles are appended to every video row; text query rows keep all tiles.
//
// The classifier (ARM) takes every stride-th raster token of frame 0 (local
// sample) or of the whole video (global sample) as both queries and keys,
// and measures per sampled query the share of its softmax mass over the
// sampled keys that the candidate mask keeps.  A head is temporal when the
// mean local recall under the temporal mask reaches alpha, else spatial when
// the mean global recall under the spatial mask does, else textural.
#include "rf_internal.h"
#include "mass.h"

#include <math.h>

namespace {

constexpr int kRowThreads = 256;
constexpr int kArmThreads = 64;
constexpr int kChunk = 32;

__device__ inline bool keeps(int32_t pattern, int32_t i, int32_t j, int32_t ri,
                             int32_t rj, int32_t band, int32_t tau) {
  if (pattern == RF_SPATIAL) return abs(i - j) <= band;
  if (pattern == RF_TEMPORAL) return abs(ri - rj) <= band;
  return i % tau == j % tau;
}

// One workgroup per (query tile, b*H + h): evaluates the head's pattern over
// the video key tiles 256 at a time and compacts the kept ids in ascending
// order (wave ballots plus per-wave counts in LDS), then appends the text
// tiles and pads the row with -1.
__global__ __launch_bounds__(kRowThreads) void pattern_rows_kernel(
    const int32_t* __restrict__ head_pattern, const int32_t* __restrict__ rank,
    int32_t nb, int32_t n_tt, int32_t band, int32_t tau, int32_t width,
    int32_t* __restrict__ rows) {
  constexpr int kWaves = kRowThreads / 64;
  __shared__ int32_t wave_count[kWaves];
  const int32_t i = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int t = threadIdx.x, wave = t / 64, lane = t % 64;
  const int32_t n_tiles = nb + n_tt;
  int32_t* out = rows + (bh * n_tiles + i) * int64_t(width);
  const int32_t p = head_pattern[bh];
  if (i >= nb || p < RF_SPATIAL || p > RF_TEXTURAL) {
    // Text query row: every tile.  Unknown pattern: an empty row.
    const bool all = i >= nb;
    for (int32_t j = t; j < width; j += kRowThreads) out[j] = (all && j < n_tiles) ? j : -1;
    return;
  }
  const int32_t ri = rank[i];
  int32_t base = 0;
  for (int32_t j0 = 0; j0 < nb; j0 += kRowThreads) {
    const int32_t j = j0 + t;
    const bool k = j < nb && keeps(p, i, j, ri, rank[min(j, nb - 1)], band, tau);
    const uint64_t bal = __ballot(k);
    const int before = __popcll(bal & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wave_count[wave] = __popcll(bal);
    __syncthreads();
    int32_t off = base, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      off += w < wave ? wave_count[w] : 0;
      total += wave_count[w];
    }
    if (k) out[off + before] = j;
    base += total;
    __syncthreads();
  }
  for (int32_t x = t; x < width - base; x += kRowThreads)
    out[base + x] = x < n_tt ? nb + x : -1;
}

template <int E>
__device__ inline float ld(const uint8_t* p, int64_t i) {
  if constexpr (E == 2) {
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

// fp32 operands: one thread per sampled query, 64 per workgroup; the sampled
// keys are staged 32 at a time through LDS (each thread reads the same key
// row).  In log2 units each thread keeps a running maximum, the total mass
// and the mass on keys the mask keeps, rescaled together once per chunk.
template <int E, int D>
__global__ __launch_bounds__(kArmThreads) void arm_recall_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ kp,
    const int32_t* __restrict__ tok_slot, const int32_t* __restrict__ rank,
    int64_t stride, int32_t n_s, int32_t bs, int64_t Lt, int32_t pattern,
    int32_t band, int32_t tau, float scale_log2, float* __restrict__ out) {
  __shared__ float kc[kChunk][D];
  __shared__ int32_t kslot[kChunk], ktile[kChunk], krank[kChunk];
  const int t = threadIdx.x;
  const int32_t a = blockIdx.x * kArmThreads + t;
  const int64_t bh = blockIdx.y;
  const bool active = a < n_s;
  const int32_t qslot = tok_slot[int64_t(active ? a : 0) * stride];
  const int32_t qt = qslot / bs;
  const int32_t rq = rank[qt];
  float q[D];
  const uint8_t* qsrc = qp + ((bh * Lt + qslot) * D) * E;
#pragma unroll
  for (int c = 0; c < D; ++c) q[c] = ld<E>(qsrc, c);
  const uint8_t* kh = kp + (bh * Lt * D) * E;

  float m = -INFINITY, tot = 0.f, kmass = 0.f;
  for (int32_t b0 = 0; b0 < n_s; b0 += kChunk) {
    const int nk = min(kChunk, n_s - b0);
    __syncthreads();
    if (t < kChunk) {
      const int32_t s = tok_slot[int64_t(b0 + min(t, nk - 1)) * stride];
      kslot[t] = s;
      ktile[t] = s / bs;
      krank[t] = rank[s / bs];
    }
    __syncthreads();
    for (int x = t; x < kChunk * D; x += kArmThreads) {
      const int r = x / D, c = x % D;
      kc[r][c] = ld<E>(kh, int64_t(kslot[r]) * D + c);
    }
    __syncthreads();
    // Sub-blocks of 8 keys keep the logits in registers.
    for (int r0 = 0; r0 < kChunk; r0 += 8) {
      float lg[8];
      float cm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc = fmaf(q[c], kc[r0 + r][c], acc);
        lg[r] = r0 + r < nk ? acc * scale_log2 : -INFINITY;
        cm = fmaxf(cm, lg[r]);
      }
      if (cm > m) {
        const float f = m == -INFINITY ? 0.f : exp2f(m - cm);
        tot *= f;
        kmass *= f;
        m = cm;
      }
      if (m == -INFINITY) continue;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e = exp2f(lg[r] - m);
        tot += e;
        if (keeps(pattern, qt, ktile[r0 + r], rq, krank[r0 + r], band, tau)) kmass += e;
      }
    }
  }
  if (active) out[bh * n_s + a] = kmass / tot;
}

// bf16 operands: each wave takes 32 sampled queries against every block of
// 32 sampled keys; the logits come from one v_mfma_f32_32x32x16_bf16 chain
// per block, the query and key rows gathered straight from global memory
// through the plan's token -> slot table.  A key's mask coordinate (its tile,
// or its tile's spatial-major rank for the temporal pattern) is loaded by
// the lane that loads the key and passed to the lanes that need it.
constexpr int kArmWaves = 4;

__device__ inline int32_t coord(int32_t pattern, int32_t tile, const int32_t* rank) {
  return pattern == RF_TEMPORAL ? rank[tile] : tile;
}

template <int D>
__global__ __launch_bounds__(kArmWaves * 64) void arm_mfma_kernel(
    const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
    const int32_t* __restrict__ tok_slot, const int32_t* __restrict__ rank,
    int64_t stride, int32_t n_s, int32_t bs, int64_t Lt, int32_t pattern,
    int32_t band, int32_t tau, float scale_log2, float* __restrict__ out) {
  using namespace rf_mass;
  const int t = threadIdx.x, w = t / 64, lane = t % 64, li = lane % 32, g = lane / 32;
  const int64_t bh = blockIdx.y;
  const int32_t a = (blockIdx.x * kArmWaves + w) * 32 + li;   // this lane's query
  const __bf16* qh = qp + bh * Lt * D;
  const __bf16* kh = kp + bh * Lt * D;
  const int32_t qslot = tok_slot[int64_t(min(a, n_s - 1)) * stride];
  const int32_t cq = coord(pattern, qslot / bs, rank);
  bf16x8 qf[D / 16];
  load_row<D>(qh + int64_t(qslot) * D, g, qf);
  Mass acc;
  for (int32_t b0 = 0; b0 < n_s; b0 += 32) {
    const int32_t kslot = tok_slot[int64_t(min(b0 + li, n_s - 1)) * stride];
    const int32_t ck = coord(pattern, kslot / bs, rank);
    bf16x8 kf[D / 16];
    load_row<D>(kh + int64_t(kslot) * D, g, kf);
    uint32_t valid = 0u, keep = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = key_of(r, g);
      const int32_t c = __shfl(ck, kk);
      const bool kept = pattern == RF_TEXTURAL ? (cq % tau == c % tau) : (abs(cq - c) <= band);
      valid |= uint32_t(b0 + kk < n_s) << r;
      keep |= uint32_t(kept) << r;
    }
    acc.absorb(logits<D>(kf, qf), valid, keep, scale_log2);
  }
  acc.merge_halves();
  if (g == 0 && a < n_s) out[bh * n_s + a] = acc.kmass / acc.tot;
}

// One workgroup per head: mean of both recall samples (fixed-order tree
// reduction) and the decision temporal -> spatial -> textural.
__global__ __launch_bounds__(256) void arm_classify_kernel(
    const float* __restrict__ loc, int32_t nl, const float* __restrict__ glo,
    int32_t ng, float alpha, int32_t* __restrict__ head_pattern,
    float* __restrict__ mean) {
  __shared__ float red[2][256];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  float sl = 0.f, sg = 0.f;
  for (int32_t i = t; i < nl; i += 256) sl += loc[bh * nl + i];
  for (int32_t i = t; i < ng; i += 256) sg += glo[bh * ng + i];
  red[0][t] = sl;
  red[1][t] = sg;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) {
      red[0][t] += red[0][t + s];
      red[1][t] += red[1][t + s];
    }
    __syncthreads();
  }
  if (t == 0) {
    const float bR = red[0][0] / float(nl), eR = red[1][0] / float(ng);
    head_pattern[bh] = bR >= alpha ? RF_TEMPORAL : (eR >= alpha ? RF_SPATIAL : RF_TEXTURAL);
    if (mean != nullptr) {
      mean[2 * bh] = bR;
      mean[2 * bh + 1] = eR;
    }
  }
}

rf_status check_plan(const rf_plan* plan, int32_t B, int32_t H, const char* fn) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "%s: null plan", fn);
  if (B < 1 || H < 1 || int64_t(B) * H > 65535)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: B=%d H=%d out of range", fn, B, H);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: current device %d is not the plan's device %d",
                    fn, dev, plan->device);
  return RF_OK;
}

template <int E, int D>
void launch_arm(const rf_plan* p, const void* qp, const void* kp, int64_t stride,
                int32_t n_s, int BH, int32_t pattern, int32_t band, int32_t tau,
                float scale, float* out, hipStream_t st) {
  if constexpr (E == 2) {
    const dim3 grid((n_s + kArmWaves * 32 - 1) / (kArmWaves * 32), BH);
    hipLaunchKernelGGL((arm_mfma_kernel<D>), grid, dim3(kArmWaves * 64), 0, st,
                       static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp),
                       p->tok_slot, p->tile_rank, stride, n_s, p->sz.bs, p->sz.Lt,
                       pattern, band, tau, scale * 1.4426950408889634f, out);
  } else {
    const dim3 grid((n_s + kArmThreads - 1) / kArmThreads, BH);
    hipLaunchKernelGGL((arm_recall_kernel<E, D>), grid, dim3(kArmThreads), 0, st,
                       static_cast<const uint8_t*>(qp), static_cast<const uint8_t*>(kp),
                       p->tok_slot, p->tile_rank, stride, n_s, p->sz.bs, p->sz.Lt,
                       pattern, band, tau, scale * 1.4426950408889634f, out);
  }
}

}  // namespace

extern "C" rf_status rf_pattern_mask(const rf_plan* plan, const int32_t* head_pattern,
                                     int32_t B, int32_t H, int32_t band, int32_t tau,
                                     int32_t* kept_rows, int32_t row_width,
                                     hipStream_t stream) {
  const char* fn = "rf_pattern_mask";
  rf_status st = check_plan(plan, B, H, fn);
  if (st != RF_OK) return st;
  if (head_pattern == nullptr || (reinterpret_cast<uintptr_t>(head_pattern) & 3u) ||
      !rf::aligned16(kept_rows))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  int32_t need = 0;
  st = rf_pattern_row_width(&plan->lay, band, tau, &need);
  if (st != RF_OK) return st;
  if (row_width < need || row_width > plan->sz.n_tiles)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: row_width %d outside [%d, %d]", fn,
                    row_width, need, plan->sz.n_tiles);
  hipLaunchKernelGGL(pattern_rows_kernel, dim3(plan->sz.n_tiles, B * H), dim3(kRowThreads),
                     0, stream, head_pattern, plan->tile_rank, plan->sz.nb,
                     plan->sz.n_text_tiles, band, tau, row_width, kept_rows);
  return rf::check_launch(fn);
}

extern "C" rf_status rf_arm_recall(const rf_plan* plan, const void* qp, const void* kp,
                                   int32_t local, int32_t stride, int32_t pattern,
                                   int32_t band, int32_t tau, int32_t B, int32_t H,
                                   int32_t d, float scale, rf_dtype dtype,
                                   float* recall, hipStream_t stream) {
  const char* fn = "rf_arm_recall";
  rf_status st = rf::check_call(plan, B, H, d, dtype, fn);
  if (st != RF_OK) return st;
  if (!rf::aligned16(qp) || !rf::aligned16(kp) || recall == nullptr ||
      (reinterpret_cast<uintptr_t>(recall) & 3u))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  if (pattern < RF_SPATIAL || pattern > RF_TEXTURAL)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: unknown pattern %d", fn, pattern);
  if (band < 0 || tau < 1)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: band %d must be >= 0 and tau %d >= 1", fn,
                    band, tau);
  if (!(scale > 0.f) || !(scale < 1e30f))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  int32_t n_s = 0;
  st = rf_arm_sample_count(&plan->lay, local, stride, &n_s);
  if (st != RF_OK) return st;
  const int BH = B * H;
  const bool bf = dtype == RF_BF16;
  if (bf && d == 128) launch_arm<2, 128>(plan, qp, kp, stride, n_s, BH, pattern, band, tau, scale, recall, stream);
  else if (bf) launch_arm<2, 64>(plan, qp, kp, stride, n_s, BH, pattern, band, tau, scale, recall, stream);
  else if (d == 128) launch_arm<4, 128>(plan, qp, kp, stride, n_s, BH, pattern, band, tau, scale, recall, stream);
  else launch_arm<4, 64>(plan, qp, kp, stride, n_s, BH, pattern, band, tau, scale, recall, stream);
  return rf::check_launch(fn);
}

extern "C" rf_status rf_arm_classify(const float* local_recall, int32_t n_local,
                                     const float* global_recall, int32_t n_global,
                                     int32_t BH, float alpha, int32_t* head_pattern,
                                     float* mean_or_null, hipStream_t stream) {
  const char* fn = "rf_arm_classify";
  if (local_recall == nullptr || global_recall == nullptr || head_pattern == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null buffer", fn);
  if (n_local < 1 || n_global < 1 || BH < 1 || BH > 65535)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: n_local=%d n_global=%d BH=%d out of range", fn,
                    n_local, n_global, BH);
  if (!(alpha == alpha))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: alpha is NaN", fn);
  hipLaunchKernelGGL(arm_classify_kernel, dim3(BH), dim3(256), 0, stream, local_recall,
                     n_local, global_recall, n_global, alpha, head_pattern, mean_or_null);
  return rf::check_launch(fn);
}
