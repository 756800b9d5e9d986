// 3D window permutation and its inverse (RainFusion2.0 page, Abstract key
// insight (2) "spatiotemporal-aware token permutation"; TL;DR "3D window
// permutation"; Figure 3 shows the artifacts it removes at 80% sparsity).
//
// Pure data movement, bound by HBM bandwidth.  Every thread moves 16-byte
// chunks; the gather side reads whole window rows (ww tokens contiguous in
// raster order), the write side is fully contiguous.  The slot -> token map
// comes from the plan, so the kernels hold no index arithmetic of their own.
#include "rf_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunksPerThread = 4;

// 16-byte store that does not allocate in the caches: the permuted and
// unpermuted tensors are written once and read back by another kernel much
// later (non-temporal stores took the row kernels 4-8% faster).
__device__ inline void store_nt(void* p, const uint4& v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// xp[bh][s][:] = x[bh][slot_src[s]][:] (zeros for pad), s < Lt.  Grid: x over the
// chunks of one (b, h), y over b*H + h.
__global__ __launch_bounds__(kThreads) void permute_rows_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ xp,
    const int32_t* __restrict__ slot_src, int32_t cpr, int64_t L, int64_t Lt) {
  const int64_t bh = blockIdx.y;
  const int32_t per_head = int32_t(Lt) * cpr;
  const uint4* src = x + bh * L * cpr;
  uint4* dst = xp + bh * Lt * cpr;
  const int32_t base = blockIdx.x * (kThreads * kChunksPerThread) + threadIdx.x;
  uint4 v[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int32_t c = base + u * kThreads;
    v[u] = make_uint4(0, 0, 0, 0);
    if (c < per_head) {
      const int32_t s = c / cpr;
      const int32_t tok = slot_src[s];
      if (tok >= 0) v[u] = src[int64_t(tok) * cpr + (c - s * cpr)];
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int32_t c = base + u * kThreads;
    if (c < per_head) store_nt(dst + c, v[u]);
  }
}

// x[bh][n][:] = xp[bh][tok_slot[n]][:].
__global__ __launch_bounds__(kThreads) void unpermute_rows_kernel(
    const uint4* __restrict__ xp, uint4* __restrict__ x,
    const int32_t* __restrict__ tok_slot, int32_t cpr, int64_t L, int64_t Lt) {
  const int64_t bh = blockIdx.y;
  const int32_t per_head = int32_t(L) * cpr;
  const uint4* src = xp + bh * Lt * cpr;
  uint4* dst = x + bh * L * cpr;
  const int32_t base = blockIdx.x * (kThreads * kChunksPerThread) + threadIdx.x;
  uint4 v[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int32_t c = base + u * kThreads;
    if (c < per_head) {
      const int32_t n = c / cpr;
      v[u] = src[int64_t(tok_slot[n]) * cpr + (c - n * cpr)];
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int32_t c = base + u * kThreads;
    if (c < per_head) store_nt(dst + c, v[u]);
  }
}

// Tile-transposed permutation: xt[bh][tile][f][s] = x[bh][slot_src[tile*BS+s]][f].
// One workgroup per (tile, b*H + h).  The tile's BS rows are gathered into
// LDS, then each thread transposes one VE x VE sub-block (VE = elements per
// 16-byte chunk) in registers and writes VE output chunks.  Consecutive
// lanes take consecutive slot chunks of the same features, so each run of
// BS*E/16 lanes writes whole output rows; in LDS, chunk k of row s sits at
// chunk k ^ ((s / VE) % CPR), which keeps both the row-wise stores and the
// column-wise loads free of bank conflicts.  E = element bytes, D = head dim.
template <int E, int D, int BS>
__global__ __launch_bounds__(kThreads) void permute_tiles_t_kernel(
    const uint8_t* __restrict__ x, uint8_t* __restrict__ xt,
    const int32_t* __restrict__ slot_src, int64_t L, int32_t n_tiles) {
  constexpr int VE = 16 / E;            // elements per chunk
  constexpr int CPR = D / VE;           // chunks per token row
  constexpr int ROW = D * E;            // LDS row (bytes), swizzled chunks
  constexpr int SCN = BS / VE;          // slot chunks per output row
  __shared__ __align__(16) uint8_t lds[BS * ROW];
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x;
  const uint8_t* src = x + bh * L * (D * E);
  // All of the thread's row chunks are loaded before any is stored, so the
  // gathers of a workgroup are in flight together.
  constexpr int NC = BS * CPR / kThreads;
  static_assert(BS * CPR % kThreads == 0, "chunk split");
  uint4 v[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int s = c / CPR, k = c % CPR;
    const int32_t tok = slot_src[int64_t(tile) * BS + s];
    v[u] = make_uint4(0, 0, 0, 0);
    if (tok >= 0)
      v[u] = *reinterpret_cast<const uint4*>(src + int64_t(tok) * (D * E) + k * 16);
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int s = c / CPR, k = c % CPR;
    *reinterpret_cast<uint4*>(lds + s * ROW + (k ^ ((s / VE) % CPR)) * 16) = v[u];
  }
  __syncthreads();
  // Sub-block (fc, sc): features fc*VE.., slots sc*VE..
  constexpr int NSUB = CPR * (BS / VE);
  uint8_t* dst = xt + (bh * n_tiles + tile) * int64_t(D) * BS * E;
  for (int b = threadIdx.x; b < NSUB; b += kThreads) {
    const int sc = b % SCN, fc = b / SCN;
    uint4 rows[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e)
      rows[e] = *reinterpret_cast<const uint4*>(lds + (sc * VE + e) * ROW +
                                                 (fc ^ (sc % CPR)) * 16);
#pragma unroll
    for (int f = 0; f < VE; ++f) {
      uint4 out;
      if constexpr (E == 2) {
        uint16_t t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          t[e] = reinterpret_cast<const uint16_t*>(&rows[e])[f];
        out = *reinterpret_cast<const uint4*>(t);
      } else {
        uint32_t t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          t[e] = reinterpret_cast<const uint32_t*>(&rows[e])[f];
        out = *reinterpret_cast<const uint4*>(t);
      }
      store_nt(dst + (int64_t(fc * VE + f) * BS + sc * VE) * E, out);
    }
  }
}

// Permutation fused with block-mean pooling: one workgroup per
// (tile, b*H + h) gathers the tile's BS rows, writes them contiguously and,
// for video blocks, accumulates each feature over the valid slots (fp32,
// fixed order) and writes the mean.  The pooling then costs no extra HBM
// pass.  Text tiles are only copied.
template <int E, int D, int BS>
__global__ __launch_bounds__(kThreads) void permute_means_kernel(
    const uint8_t* __restrict__ x, uint8_t* __restrict__ xp,
    float* __restrict__ xbar, const int32_t* __restrict__ slot_src,
    const int32_t* __restrict__ tile_count, int64_t L, int64_t Lt,
    int32_t nb) {
  constexpr int VE = 16 / E;            // elements per 16-byte chunk
  constexpr int CPR = D / VE;           // chunks per row
  constexpr int RG = kThreads / CPR;    // row groups
  static_assert(RG >= 1 && BS % RG == 0, "layout");
  __shared__ float part[RG][D];
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x;
  const uint8_t* src = x + bh * L * (D * E);
  // xp == nullptr: the means only (no permuted rows are written).
  uint8_t* dst = xp != nullptr ? xp + (bh * Lt + int64_t(tile) * BS) * (D * E) : nullptr;
  const int k = threadIdx.x % CPR, rg = threadIdx.x / CPR;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  uint4 v[BS / RG];
#pragma unroll
  for (int i = 0; i < BS / RG; ++i) {
    const int s = rg + i * RG;
    const int32_t tok = slot_src[int64_t(tile) * BS + s];
    v[i] = make_uint4(0, 0, 0, 0);
    if (tok >= 0)
      v[i] = *reinterpret_cast<const uint4*>(src + int64_t(tok) * (D * E) + k * 16);
  }
#pragma unroll
  for (int i = 0; i < BS / RG; ++i) {
    const int s = rg + i * RG;
    if (xp != nullptr) store_nt(dst + int64_t(s) * (D * E) + k * 16, v[i]);
    // Pad slots hold zeros here, so summing every slot sums the valid ones.
    if constexpr (E == 2) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      acc[0] += __uint_as_float(v[i].x);
      acc[1] += __uint_as_float(v[i].y);
      acc[2] += __uint_as_float(v[i].z);
      acc[3] += __uint_as_float(v[i].w);
    }
  }
  if (tile >= nb) return;                       // text: copy only (uniform)
#pragma unroll
  for (int e = 0; e < VE; ++e) part[rg][k * VE + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) sum += part[r][threadIdx.x];
    xbar[(bh * nb + tile) * D + threadIdx.x] = sum / float(tile_count[tile]);
  }
}

template <int E, int D, int BS>
void launch_means(const rf_plan* p, const void* x, void* xp, float* xbar,
                  int BH, hipStream_t st) {
  // Without permuted rows the text tiles have nothing to do.
  dim3 grid(xp != nullptr ? p->sz.n_tiles : p->sz.nb, BH);
  hipLaunchKernelGGL((permute_means_kernel<E, D, BS>), grid, dim3(kThreads), 0, st,
                     static_cast<const uint8_t*>(x), static_cast<uint8_t*>(xp),
                     xbar, p->slot_src, p->tile_count, p->sz.L, p->sz.Lt,
                     p->sz.nb);
}

template <int E, int D, int BS>
void launch_tiles_t(const rf_plan* p, const void* x, void* xt, int BH,
                    hipStream_t st) {
  dim3 grid(p->sz.n_tiles, BH);
  hipLaunchKernelGGL((permute_tiles_t_kernel<E, D, BS>), grid, dim3(kThreads),
                     0, st, static_cast<const uint8_t*>(x),
                     static_cast<uint8_t*>(xt), p->slot_src, p->sz.L, p->sz.n_tiles);
}

}  // namespace

extern "C" {

rf_status rf_permute(const rf_plan* plan, const void* x, void* xp, int32_t B,
                     int32_t H, int32_t d, rf_dtype dtype, rf_order order,
                     hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, "rf_permute");
  if (st != RF_OK) return st;
  if (!rf::aligned16(x) || !rf::aligned16(xp))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_permute: null or misaligned buffer");
  if (order != RF_ROWS && order != RF_TILES_T)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_permute: unknown order %d", int(order));
  const int E = rf::esize(dtype);
  const int cpr = d * E / 16;
  const int BH = B * H;
  if (order == RF_ROWS) {
    const int64_t per_head = plan->sz.Lt * cpr;
    dim3 grid((per_head + kThreads * kChunksPerThread - 1) /
                  (kThreads * kChunksPerThread), BH);
    hipLaunchKernelGGL(permute_rows_kernel, grid, dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(x), static_cast<uint4*>(xp),
                       plan->slot_src, cpr, plan->sz.L, plan->sz.Lt);
  } else {
    const int bs = plan->sz.bs;
    if (E == 2 && d == 128 && bs == 128) launch_tiles_t<2, 128, 128>(plan, x, xp, BH, stream);
    else if (E == 2 && d == 128 && bs == 64) launch_tiles_t<2, 128, 64>(plan, x, xp, BH, stream);
    else if (E == 2 && d == 64 && bs == 128) launch_tiles_t<2, 64, 128>(plan, x, xp, BH, stream);
    else if (E == 2 && d == 64 && bs == 64) launch_tiles_t<2, 64, 64>(plan, x, xp, BH, stream);
    else if (E == 4 && d == 128 && bs == 128) launch_tiles_t<4, 128, 128>(plan, x, xp, BH, stream);
    else if (E == 4 && d == 128 && bs == 64) launch_tiles_t<4, 128, 64>(plan, x, xp, BH, stream);
    else if (E == 4 && d == 64 && bs == 128) launch_tiles_t<4, 64, 128>(plan, x, xp, BH, stream);
    else launch_tiles_t<4, 64, 64>(plan, x, xp, BH, stream);
  }
  return rf::check_launch("rf_permute");
}

rf_status rf_permute_means(const rf_plan* plan, const void* x, void* xp,
                           float* xbar, int32_t B, int32_t H, int32_t d,
                           rf_dtype dtype, hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, "rf_permute_means");
  if (st != RF_OK) return st;
  if (!rf::aligned16(x) || (xp != nullptr && !rf::aligned16(xp)) || !rf::aligned16(xbar))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_permute_means: null or misaligned buffer");
  const int BH = B * H;
  const int bs = plan->sz.bs;
  const bool bf = dtype == RF_BF16;
  if (bf && d == 128 && bs == 128) launch_means<2, 128, 128>(plan, x, xp, xbar, BH, stream);
  else if (bf && d == 128 && bs == 64) launch_means<2, 128, 64>(plan, x, xp, xbar, BH, stream);
  else if (bf && d == 64 && bs == 128) launch_means<2, 64, 128>(plan, x, xp, xbar, BH, stream);
  else if (bf && d == 64 && bs == 64) launch_means<2, 64, 64>(plan, x, xp, xbar, BH, stream);
  else if (!bf && d == 128 && bs == 128) launch_means<4, 128, 128>(plan, x, xp, xbar, BH, stream);
  else if (!bf && d == 128 && bs == 64) launch_means<4, 128, 64>(plan, x, xp, xbar, BH, stream);
  else if (!bf && d == 64 && bs == 128) launch_means<4, 64, 128>(plan, x, xp, xbar, BH, stream);
  else launch_means<4, 64, 64>(plan, x, xp, xbar, BH, stream);
  return rf::check_launch("rf_permute_means");
}

rf_status rf_unpermute(const rf_plan* plan, const void* xp, void* x,
                       int32_t B, int32_t H, int32_t d, rf_dtype dtype,
                       hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, "rf_unpermute");
  if (st != RF_OK) return st;
  if (!rf::aligned16(x) || !rf::aligned16(xp))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_unpermute: null or misaligned buffer");
  const int cpr = d * rf::esize(dtype) / 16;
  const int64_t per_head = plan->sz.L * cpr;
  dim3 grid((per_head + kThreads * kChunksPerThread - 1) /
                (kThreads * kChunksPerThread), B * H);
  hipLaunchKernelGGL(unpermute_rows_kernel, grid, dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(xp), static_cast<uint4*>(x),
                     plan->tok_slot, cpr, plan->sz.L, plan->sz.Lt);
  return rf::check_launch("rf_unpermute");
}

}  // extern "C"
