// FP8 (OCP e4m3) operands for the block-sparse attention: the quantization
// step of the FP8 variant (RainFusion2.0 page, TL;DR: integration with
// quantization named as future work).
//
// Each group of values gets one power-of-two scale 2^e, e the smallest
// integer with amax <= 448 * 2^e (e = 0 for an all-zero group), and codes
// e4m3(x * 2^-e) by v_cvt_pk_fp8_f32 (round to nearest, ties to even).  The
// product x * 2^-e is exact (v_ldexp_f32), so the codes depend only on x and
// e.  Groups:
//   RF_ROWS     one scale per (b, h, tile) over its bs x d values (Q, K): the
//               two scales of a tile pair fold into the logit multiplier;
//   RF_TILES_T  one scale per (b, h, feature) over all slots (V): the scale
//               is constant along the keys the PV product sums over, so it
//               is applied once to the output.
// rf_quantize_fp8 converts permuted bf16 tensors; rf_permute_fp8 permutes
// raster bf16 tensors straight into codes (and, for Q and K, the block means
// of the bf16 values), so the bf16 permuted copies are never written.  Both
// give the same codes and scales.
#include "rf_internal.h"

#include <math.h>

namespace {

constexpr int kThreads = 256;

__device__ inline float bf16_to_f32(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

// Smallest e with amax <= 448 * 2^e: with amax = m 2^k, m in [0.5, 1) and
// 448 = 0.875 * 2^9, e = k - 9 when m <= 0.875, else k - 8.
__device__ inline int pow2_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float m = frexpf(amax, &k);
  return m <= 0.875f ? k - 9 : k - 8;
}

__device__ inline uint32_t pack4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return uint32_t(v);
}

// One workgroup per (tile, b*H + h) of an RF_ROWS tensor: the tile's bs*d
// values are loaded once into registers (N per thread, 8 per 16-byte load),
// reduced to their amax across the workgroup, scaled and converted.
template <int N>
__global__ __launch_bounds__(kThreads) void quant_tiles_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ x8, float* __restrict__ scale,
    int64_t tile_elems, int32_t n_tiles) {
  __shared__ float wmax[kThreads / 64];
  const int32_t tile = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int t = threadIdx.x;
  const int64_t base = (bh * n_tiles + tile) * tile_elems;
  typedef uint16_t u16x8 __attribute__((__vector_size__(16)));
  float v[N];
#pragma unroll
  for (int c = 0; c < N / 8; ++c) {
    const u16x8 w = *reinterpret_cast<const u16x8*>(x + base + (int64_t(c) * kThreads + t) * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * c + e] = bf16_to_f32(w[e]);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (t % 64 == 0) wmax[t / 64] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = pow2_exponent(m);
  if (t == 0) scale[bh * n_tiles + tile] = ldexpf(1.f, e);
  typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
#pragma unroll
  for (int c = 0; c < N / 8; ++c) {
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = ldexpf(v[8 * c + k], -e);
    const u32x2 out = {pack4(s[0], s[1], s[2], s[3]), pack4(s[4], s[5], s[6], s[7])};
    *reinterpret_cast<u32x2*>(x8 + base + (int64_t(c) * kThreads + t) * 8) = out;
  }
}

// Per-feature amax of an RF_TILES_T tensor ([tile][d][bs]), accumulated
// with atomicMax on the bit patterns (non-negative floats order like their
// bits) into `amax` [BH][d], which starts at zero.  Grid (BH, chunks of
// tiles); thread t reads one half of feature row t / 2 of each tile.
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void feature_amax_kernel(
    const uint16_t* __restrict__ x, uint32_t* __restrict__ amax, int32_t n_tiles,
    int32_t tiles_per_chunk) {
  static_assert(D * BS / kThreads % 8 == 0 && kThreads % D == 0, "split");
  constexpr int kPerRow = kThreads / D;          // threads per feature row
  constexpr int kN = BS / kPerRow;               // values per thread and tile
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const int dd = t / kPerRow, part = t % kPerRow;
  const int32_t t0 = blockIdx.y * tiles_per_chunk;
  const int32_t t1 = min(n_tiles, t0 + tiles_per_chunk);
  typedef uint16_t u16x8 __attribute__((__vector_size__(16)));
  float m = 0.f;
  for (int32_t tile = t0; tile < t1; ++tile) {
    const uint16_t* row = x + ((bh * n_tiles + tile) * D + dd) * BS + part * kN;
#pragma unroll
    for (int c = 0; c < kN / 8; ++c) {
      const u16x8 w = *reinterpret_cast<const u16x8*>(row + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(bf16_to_f32(w[e])));
    }
  }
#pragma unroll
  for (int off = kPerRow / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (part == 0 && m > 0.f) atomicMax(&amax[bh * D + dd], __float_as_uint(m));
}

__global__ void zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// One workgroup per (tile, b*H + h) of an RF_TILES_T tensor: thread t
// converts one half of feature row t / 2 with that feature's scale.
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void quant_features_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
    const uint32_t* __restrict__ amax, int32_t n_tiles) {
  constexpr int kPerRow = kThreads / D;
  constexpr int kN = BS / kPerRow;
  const int32_t tile = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int t = threadIdx.x;
  const int dd = t / kPerRow, part = t % kPerRow;
  const int e = pow2_exponent(__uint_as_float(amax[bh * D + dd]));
  const int64_t off = ((bh * n_tiles + tile) * D + dd) * BS + part * kN;
  typedef uint16_t u16x8 __attribute__((__vector_size__(16)));
  typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
#pragma unroll
  for (int c = 0; c < kN / 8; ++c) {
    const u16x8 w = *reinterpret_cast<const u16x8*>(x + off + 8 * c);
    float s[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) s[k] = ldexpf(bf16_to_f32(w[k]), -e);
    const u32x2 out = {pack4(s[0], s[1], s[2], s[3]), pack4(s[4], s[5], s[6], s[7])};
    *reinterpret_cast<u32x2*>(x8 + off + 8 * c) = out;
  }
}

// amax bits -> scale 2^e, in place, once every tile has been converted.
__global__ void feature_scale_kernel(uint32_t* __restrict__ amax_scale, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n)
    amax_scale[i] = __float_as_uint(ldexpf(1.f, pow2_exponent(__uint_as_float(amax_scale[i]))));
}

template <int D, int BS>
void launch_features(const rf_plan* p, const void* xp, void* x8, float* scale, int BH,
                     hipStream_t st) {
  const int32_t nt = p->sz.n_tiles;
  const int64_t n = int64_t(BH) * D;
  uint32_t* am = reinterpret_cast<uint32_t*>(scale);
  hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, am, n);
  const int32_t chunk = 16;
  hipLaunchKernelGGL((feature_amax_kernel<D, BS>), dim3(BH, (nt + chunk - 1) / chunk),
                     dim3(kThreads), 0, st, static_cast<const uint16_t*>(xp), am, nt, chunk);
  hipLaunchKernelGGL((quant_features_kernel<D, BS>), dim3(nt, BH), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(xp), static_cast<uint8_t*>(x8), am, nt);
  hipLaunchKernelGGL(feature_scale_kernel, dim3((n + 255) / 256), dim3(256), 0, st, am, n);
}

// Permutation fused with the per-tile quantization (and optionally the block
// means): one workgroup per (tile, b*H + h) gathers the tile's rows into
// registers exactly as the bf16 permute-and-pool kernel does, so the means
// are the same bits, then converts them with the tile's scale.
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void permute_quant_rows_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ x8, float* __restrict__ scale,
    float* __restrict__ xbar, const int32_t* __restrict__ slot_src,
    const int32_t* __restrict__ tile_count, int64_t L, int64_t Lt, int32_t nb,
    int32_t n_tiles) {
  constexpr int VE = 8;                 // bf16 per 16-byte chunk
  constexpr int CPR = D / VE;           // chunks per row
  constexpr int RG = kThreads / CPR;    // row groups
  static_assert(RG >= 1 && BS % RG == 0, "layout");
  __shared__ float part[RG][D];
  __shared__ float wmax[kThreads / 64];
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x;
  const int t = threadIdx.x;
  const uint16_t* src = x + bh * L * D;
  const int k = t % CPR, rg = t / CPR;
  uint4 v[BS / RG];
#pragma unroll
  for (int i = 0; i < BS / RG; ++i) {
    const int s = rg + i * RG;
    const int32_t tok = slot_src[int64_t(tile) * BS + s];
    v[i] = make_uint4(0, 0, 0, 0);
    if (tok >= 0) v[i] = *reinterpret_cast<const uint4*>(src + int64_t(tok) * D + k * VE);
  }
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < BS / RG; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
      acc[2 * e] += lo;
      acc[2 * e + 1] += hi;
      m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (t % 64 == 0) wmax[t / 64] = m;
  if (xbar != nullptr && tile < nb) {
#pragma unroll
    for (int e = 0; e < VE; ++e) part[rg][k * VE + e] = acc[e];
  }
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int ex = pow2_exponent(m);
  if (t == 0) scale[bh * n_tiles + tile] = ldexpf(1.f, ex);
  uint8_t* dst = x8 + (bh * Lt + int64_t(tile) * BS) * D;
  typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
#pragma unroll
  for (int i = 0; i < BS / RG; ++i) {
    const int s = rg + i * RG;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = ldexpf(__uint_as_float(w[e] << 16), -ex);
      f[2 * e + 1] = ldexpf(__uint_as_float(w[e] & 0xffff0000u), -ex);
    }
    const u32x2 out = {pack4(f[0], f[1], f[2], f[3]), pack4(f[4], f[5], f[6], f[7])};
    // Written once, read by the attention kernel later: no cache allocation.
    __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(dst + int64_t(s) * D + k * VE));
  }
  if (xbar != nullptr && tile < nb && t < D) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) sum += part[r][t];
    xbar[(bh * nb + tile) * D + t] = sum / float(tile_count[tile]);
  }
}

// Per-feature amax of a raster tensor [BH][L][D] (the permuted tensor holds
// the same values plus zeros), accumulated like feature_amax_kernel.  Grid
// (BH, chunks of rows); thread t reads 8 features of rows t / (D/8) + ...
template <int D>
__global__ __launch_bounds__(kThreads) void raster_amax_kernel(
    const uint16_t* __restrict__ x, uint32_t* __restrict__ amax, int64_t L,
    int32_t rows_per_chunk) {
  constexpr int CPR = D / 8;
  constexpr int RG = kThreads / CPR;
  __shared__ float part[RG][D];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x, k = t % CPR, rg = t / CPR;
  const int64_t r0 = int64_t(blockIdx.y) * rows_per_chunk;
  const int64_t r1 = min(L, r0 + rows_per_chunk);
  typedef uint16_t u16x8 __attribute__((__vector_size__(16)));
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Four rows per thread in flight at a time.
  for (int64_t r = r0 + rg; r < r1; r += 4 * RG) {
    u16x8 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t rr = min(r + u * RG, r1 - 1);
      w[u] = *reinterpret_cast<const u16x8*>(x + (bh * L + rr) * D + k * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(bf16_to_f32(w[u][e])));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][k * 8 + e] = m[e];
  __syncthreads();
  if (t < D) {
    float mm = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) mm = fmaxf(mm, part[r][t]);
    if (mm > 0.f) atomicMax(&amax[bh * D + t], __float_as_uint(mm));
  }
}

// Tile-transposed permutation fused with the per-feature quantization: the
// tile's rows are gathered into LDS (as in the bf16 kernel), then each thread
// writes the codes of 8 slots of one feature with that feature's scale.
template <int D, int BS>
__global__ __launch_bounds__(kThreads) void permute_quant_tiles_t_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
    const uint32_t* __restrict__ amax, const int32_t* __restrict__ slot_src, int64_t L,
    int32_t n_tiles) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int ROW = D * 2;            // LDS row (bytes): chunk k of row s at k ^ ((s / 8) % CPR)
  constexpr int SCN = BS / 8;           // 8-slot pieces per output row
  constexpr int NC = BS * CPR / kThreads;
  static_assert(BS * CPR % kThreads == 0, "chunk split");
  __shared__ __align__(16) uint8_t lds[BS * ROW];
  const int64_t bh = blockIdx.y;
  const int32_t tile = blockIdx.x;
  const uint16_t* src = x + bh * L * D;
  uint4 v[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int s = c / CPR, k = c % CPR;
    const int32_t tok = slot_src[int64_t(tile) * BS + s];
    v[u] = make_uint4(0, 0, 0, 0);
    if (tok >= 0) v[u] = *reinterpret_cast<const uint4*>(src + int64_t(tok) * D + k * 8);
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = threadIdx.x + u * kThreads;
    const int s = c / CPR, k = c % CPR;
    *reinterpret_cast<uint4*>(lds + s * ROW + (k ^ ((s / 8) % CPR)) * 16) = v[u];
  }
  __syncthreads();
  // Sub-block (fc, sc): features fc*8 .. +8, slots sc*8 .. +8.  Consecutive
  // lanes take consecutive sc, so SCN lanes write one whole output row; the
  // swizzle keeps the LDS stores and loads free of bank conflicts.
  constexpr int NSUB = CPR * SCN;
  uint8_t* dst = x8 + (bh * n_tiles + tile) * int64_t(D) * BS;
  typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
  for (int b = threadIdx.x; b < NSUB; b += kThreads) {
    const int sc = b % SCN, fc = b / SCN;
    uint4 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      rows[e] = *reinterpret_cast<const uint4*>(lds + (sc * 8 + e) * ROW + (fc ^ (sc % CPR)) * 16);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int ex = pow2_exponent(__uint_as_float(amax[bh * D + fc * 8 + f]));
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        y[e] = ldexpf(bf16_to_f32(reinterpret_cast<const uint16_t*>(&rows[e])[f]), -ex);
      const u32x2 out = {pack4(y[0], y[1], y[2], y[3]), pack4(y[4], y[5], y[6], y[7])};
      __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(dst + int64_t(fc * 8 + f) * BS + sc * 8));
    }
  }
}

template <int D, int BS>
void launch_permute_fp8(const rf_plan* p, const void* x, rf_order order, void* x8,
                        float* scale, float* xbar, int BH, hipStream_t st) {
  const int32_t nt = p->sz.n_tiles;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  uint8_t* y = static_cast<uint8_t*>(x8);
  if (order == RF_ROWS) {
    hipLaunchKernelGGL((permute_quant_rows_kernel<D, BS>), dim3(nt, BH), dim3(kThreads), 0, st,
                       xs, y, scale, xbar, p->slot_src, p->tile_count, p->sz.L, p->sz.Lt,
                       p->sz.nb, nt);
    return;
  }
  const int64_t n = int64_t(BH) * D;
  uint32_t* am = reinterpret_cast<uint32_t*>(scale);
  hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st, am, n);
  const int32_t rows = 512;
  hipLaunchKernelGGL((raster_amax_kernel<D>), dim3(BH, (p->sz.L + rows - 1) / rows),
                     dim3(kThreads), 0, st, xs, am, p->sz.L, rows);
  hipLaunchKernelGGL((permute_quant_tiles_t_kernel<D, BS>), dim3(nt, BH), dim3(kThreads), 0, st,
                     xs, y, am, p->slot_src, p->sz.L, nt);
  hipLaunchKernelGGL(feature_scale_kernel, dim3((n + 255) / 256), dim3(256), 0, st, am, n);
}

}  // namespace

extern "C" rf_status rf_permute_fp8(const rf_plan* plan, const void* x, rf_order order,
                                    void* x8, float* scale, float* xbar_or_null, int32_t B,
                                    int32_t H, int32_t d, rf_dtype dtype, hipStream_t stream) {
  const char* fn = "rf_permute_fp8";
  rf_status st = rf::check_call(plan, B, H, d, dtype, fn);
  if (st != RF_OK) return st;
  if (dtype != RF_BF16)
    return rf::fail(RF_ERR_UNSUPPORTED, "%s: the FP8 variant quantizes bf16 tensors", fn);
  if (!rf::aligned16(x) || !rf::aligned16(x8) || scale == nullptr ||
      (reinterpret_cast<uintptr_t>(scale) & 3u) ||
      (xbar_or_null != nullptr && !rf::aligned16(xbar_or_null)))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  if (order != RF_ROWS && order != RF_TILES_T)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: unknown order %d", fn, int(order));
  if (order == RF_TILES_T && xbar_or_null != nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: block means come with RF_ROWS only", fn);
  const int BH = B * H;
  const int bs = plan->sz.bs;
  if (d == 128 && bs == 128) launch_permute_fp8<128, 128>(plan, x, order, x8, scale, xbar_or_null, BH, stream);
  else if (d == 128) launch_permute_fp8<128, 64>(plan, x, order, x8, scale, xbar_or_null, BH, stream);
  else if (bs == 128) launch_permute_fp8<64, 128>(plan, x, order, x8, scale, xbar_or_null, BH, stream);
  else launch_permute_fp8<64, 64>(plan, x, order, x8, scale, xbar_or_null, BH, stream);
  return rf::check_launch(fn);
}

extern "C" rf_status rf_quantize_fp8(const rf_plan* plan, const void* xp, rf_order order,
                                     void* x8, float* scale, int32_t B, int32_t H, int32_t d,
                                     rf_dtype dtype, hipStream_t stream) {
  const char* fn = "rf_quantize_fp8";
  rf_status st = rf::check_call(plan, B, H, d, dtype, fn);
  if (st != RF_OK) return st;
  if (dtype != RF_BF16)
    return rf::fail(RF_ERR_UNSUPPORTED, "%s: the FP8 variant quantizes bf16 tensors", fn);
  if (!rf::aligned16(xp) || !rf::aligned16(x8) || scale == nullptr ||
      (reinterpret_cast<uintptr_t>(scale) & 3u))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  const int BH = B * H;
  const int bs = plan->sz.bs;
  if (order == RF_ROWS) {
    const int64_t te = int64_t(bs) * d;
    const int n = int(te / kThreads);            // 64, 32 or 16 values per thread
    const dim3 grid(plan->sz.n_tiles, BH);
    const uint16_t* x = static_cast<const uint16_t*>(xp);
    uint8_t* y = static_cast<uint8_t*>(x8);
    if (n == 64) hipLaunchKernelGGL((quant_tiles_kernel<64>), grid, dim3(kThreads), 0, stream, x, y, scale, te, plan->sz.n_tiles);
    else if (n == 32) hipLaunchKernelGGL((quant_tiles_kernel<32>), grid, dim3(kThreads), 0, stream, x, y, scale, te, plan->sz.n_tiles);
    else hipLaunchKernelGGL((quant_tiles_kernel<16>), grid, dim3(kThreads), 0, stream, x, y, scale, te, plan->sz.n_tiles);
  } else if (order == RF_TILES_T) {
    if (d == 128 && bs == 128) launch_features<128, 128>(plan, xp, x8, scale, BH, stream);
    else if (d == 128) launch_features<128, 64>(plan, xp, x8, scale, BH, stream);
    else if (bs == 128) launch_features<64, 128>(plan, xp, x8, scale, BH, stream);
    else launch_features<64, 64>(plan, xp, x8, scale, BH, stream);
  } else {
    return rf::fail(RF_ERR_INVALID_ARG, "%s: unknown order %d", fn, int(order));
  }
  return rf::check_launch(fn);
}
