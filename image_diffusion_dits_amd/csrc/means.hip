// Block-mean pooling: the representative token of each video block is the
// mean of its valid slots (RainFusion2.0 page, Abstract key insight (1),
// "block-wise mean values as representative tokens"; TL;DR "blockwise
// representative tokens").  Pad slots are skipped by the plan's per-tile
// validity mask, whatever values they hold.
//
// HBM-bound: one workgroup reads one block (bs rows) once.  Threads own a
// 16-byte column chunk and a set of rows; partial sums are combined in LDS
// in a fixed order, so results are deterministic.
#include "rf_internal.h"

namespace {

constexpr int kThreads = 256;

template <int E, int D, int BS>
__global__ __launch_bounds__(kThreads) void block_means_kernel(
    const uint8_t* __restrict__ qp, const uint8_t* __restrict__ kp,
    float* __restrict__ qbar, float* __restrict__ kbar,
    const uint32_t* __restrict__ tile_bits,
    const int32_t* __restrict__ tile_count, int64_t Lt, int32_t nb) {
  constexpr int VE = 16 / E;          // elements per 16-byte chunk
  constexpr int CPR = D / VE;         // chunks per row
  constexpr int RG = kThreads / CPR;  // row groups
  static_assert(RG >= 1 && BS % RG == 0, "layout");
  __shared__ float part[RG][D];
  const int blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const uint8_t* src = (blockIdx.z == 0 ? qp : kp) +
                       ((bh * Lt + int64_t(blk) * BS) * D) * E;
  float* dst = (blockIdx.z == 0 ? qbar : kbar) + (bh * nb + blk) * D;
  const int k = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  const uint32_t* bits = tile_bits + blk * 4;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = rg; s < BS; s += RG) {
    if ((bits[s >> 5] >> (s & 31)) & 1u) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t(s) * D) * E + k * 16);
      if constexpr (E == 2) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(w[e] << 16);
          acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
        }
      } else {
        acc[0] += __uint_as_float(v.x);
        acc[1] += __uint_as_float(v.y);
        acc[2] += __uint_as_float(v.z);
        acc[3] += __uint_as_float(v.w);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) part[rg][k * VE + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) sum += part[r][threadIdx.x];
    dst[threadIdx.x] = sum / float(tile_count[blk]);
  }
}

template <int E, int D, int BS>
void launch(const rf_plan* p, const void* qp, const void* kp, float* qbar,
            float* kbar, int BH, hipStream_t st) {
  dim3 grid(p->sz.nb, BH, 2);
  hipLaunchKernelGGL((block_means_kernel<E, D, BS>), grid, dim3(kThreads), 0,
                     st, static_cast<const uint8_t*>(qp),
                     static_cast<const uint8_t*>(kp), qbar, kbar, p->tile_bits,
                     p->tile_count, p->sz.Lt, p->sz.nb);
}

}  // namespace

extern "C" rf_status rf_block_means(const rf_plan* plan, const void* qp,
                                    const void* kp, float* qbar, float* kbar,
                                    int32_t B, int32_t H, int32_t d,
                                    rf_dtype dtype, hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, "rf_block_means");
  if (st != RF_OK) return st;
  if (!rf::aligned16(qp) || !rf::aligned16(kp) || !rf::aligned16(qbar) ||
      !rf::aligned16(kbar))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_block_means: null or misaligned buffer");
  const int BH = B * H;
  const int bs = plan->sz.bs;
  const bool bf = dtype == RF_BF16;
  if (bf && d == 128 && bs == 128) launch<2, 128, 128>(plan, qp, kp, qbar, kbar, BH, stream);
  else if (bf && d == 128 && bs == 64) launch<2, 128, 64>(plan, qp, kp, qbar, kbar, BH, stream);
  else if (bf && d == 64 && bs == 128) launch<2, 64, 128>(plan, qp, kp, qbar, kbar, BH, stream);
  else if (bf && d == 64 && bs == 64) launch<2, 64, 64>(plan, qp, kp, qbar, kbar, BH, stream);
  else if (!bf && d == 128 && bs == 128) launch<4, 128, 128>(plan, qp, kp, qbar, kbar, BH, stream);
  else if (!bf && d == 128 && bs == 64) launch<4, 128, 64>(plan, qp, kp, qbar, kbar, BH, stream);
  else if (!bf && d == 64 && bs == 128) launch<4, 64, 128>(plan, qp, kp, qbar, kbar, BH, stream);
  else launch<4, 64, 64>(plan, qp, kp, qbar, kbar, BH, stream);
  return rf::check_launch("rf_block_means");
}
