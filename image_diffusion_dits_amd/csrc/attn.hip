// Block-sparse flash-attention forward over the kept tiles (RainFusion2.0
// page, Abstract: skip computation for insignificant tokens, block-wise
// sparse attention; RainFusion review page, Assumptions: softmax attention,
// Eq. (1)).
//
// bf16 path (gfx950 MFMA).  One workgroup per (b, h, query tile) with one
// wave per 32 queries.  Per kept key tile:
//   S^T = K Q^T       v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                     B = the wave's Q held in registers for the whole row;
//   online softmax    in fp32 registers; in the S^T accumulator layout each
//                     lane owns one query column, so row max / row sum need
//                     one exchange with lane ^ 32;
//   O^T += V^T P^T    A = V^T rows from LDS (the V operand arrives tile-
//                     transposed from the permutation, so no transpose is
//                     done here), B = P^T taken straight from the S^T
//                     accumulators converted to bf16;
// and O^T's accumulator layout again gives each lane one query column, so
// the softmax rescale is a per-lane scalar.  K and V^T tiles are staged in
// padded LDS rows (conflict-free 16-byte / 8-byte reads), the next tile's
// global loads are issued before the current tile's math.  Pad keys get
// -inf from the plan's per-tile validity masks; pad query rows are written
// as zeros.  Workgroups are renumbered so that each XCD (one L2) works on a
// contiguous range of query tiles of one head; the heavy text query tiles
// (which keep every tile) start first.
//
// fp32 path: one thread per query row, fp32 FMA and expf, the same tile
// walk; used where fp32 accuracy is required.
#include "rf_internal.h"

namespace {

typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kXcds = 8;

struct TileJob {
  int64_t bh;
  int32_t tile;
};

// Workgroup id -> (b*H + h, query tile).  Text query tiles of all heads come
// first; video tiles are dealt so that ids landing on the same XCD (id mod 8)
// cover a contiguous run of (head, tile).
__device__ inline TileJob job_of(int32_t pid, int32_t BH, int32_t nb,
                                 int32_t n_tt) {
  const int32_t n_text_jobs = BH * n_tt;
  if (pid < n_text_jobs) return {pid / n_tt, nb + pid % n_tt};
  const int32_t p = pid - n_text_jobs;
  const int32_t total = BH * nb;
  const int32_t q = total / kXcds, r = total % kXcds;
  const int32_t x = p % kXcds, idx = p / kXcds;
  const int32_t logical = (x < r) ? x * (q + 1) + idx : r * (q + 1) + (x - r) * q + idx;
  return {logical / nb, logical % nb};
}

__device__ inline int64_t row_offset(int32_t tile, int32_t nb,
                                     int32_t row_len_video, int32_t n_tiles) {
  return tile < nb ? int64_t(tile) * row_len_video
                   : int64_t(nb) * row_len_video + int64_t(tile - nb) * n_tiles;
}

// ---------------------------------------------------------------- bf16 MFMA

template <int D, int BS>
struct Bf16Cfg {
  static constexpr int kWaves = BS / 32;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKStride = D + 8;    // K row in LDS (bf16)
  static constexpr int kVStride = BS + 4;   // V^T row in LDS (bf16)
  static constexpr int kKChunks = BS * D / 8;  // 16-byte chunks per tile
  static constexpr int kPerThread = kKChunks / kThreads;
};

template <int D, int BS>
__global__ __launch_bounds__((BS / 32) * 64) void attn_bf16_kernel(
    const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ kept,
    __bf16* __restrict__ op, const uint32_t* __restrict__ tile_bits,
    const int32_t* __restrict__ tile_count, int64_t Lp, int32_t BH,
    int32_t nb, int32_t n_tt, int32_t row_len_video, int64_t nnz,
    float scale_log2) {
  using C = Bf16Cfg<D, BS>;
  __shared__ __align__(16) __bf16 ks[BS * C::kKStride];
  __shared__ __align__(16) __bf16 vs[D * C::kVStride];
  const int32_t n_tiles = nb + n_tt;
  const TileJob job = job_of(blockIdx.x, BH, nb, n_tt);
  const int64_t bh = job.bh;
  const int32_t qtile = job.tile;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int li = lane % 32, g = lane / 32;

  const __bf16* kh = kp + bh * Lp * D;
  const __bf16* vh = vt + bh * int64_t(n_tiles) * D * BS;
  const int32_t* row = kept + bh * nnz + row_offset(qtile, nb, row_len_video, n_tiles);
  const int32_t row_len = qtile < nb ? row_len_video : n_tiles;

  // Q operand (B of S^T = K Q^T): lane (li, g) holds q[li][16m + 8g .. +8].
  const int64_t qrow = int64_t(qtile) * BS + wave * 32 + li;
  bf16x8 qf[D / 16];
  {
    const __bf16* qsrc = qp + (bh * Lp + qrow) * D + 8 * g;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      if (qrow < Lp) qf[m] = *reinterpret_cast<const bf16x8*>(qsrc + 16 * m);
      else qf[m] = bf16x8{};
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  uint4 pk[C::kPerThread], pv[C::kPerThread];
  auto fetch = [&](int32_t kt) {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int c = threadIdx.x + u * C::kThreads;
      const int r = c / (D / 8), cc = c % (D / 8);
      const int64_t slot = int64_t(kt) * BS + r;
      pk[u] = slot < Lp ? *reinterpret_cast<const uint4*>(kh + slot * D + cc * 8)
                        : make_uint4(0, 0, 0, 0);
      const int vr = c / (BS / 8), vc = c % (BS / 8);
      pv[u] = *reinterpret_cast<const uint4*>(vh + (int64_t(kt) * D + vr) * BS + vc * 8);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < C::kPerThread; ++u) {
      const int c = threadIdx.x + u * C::kThreads;
      const int r = c / (D / 8), cc = c % (D / 8);
      *reinterpret_cast<uint4*>(ks + r * C::kKStride + cc * 8) = pk[u];
      const int vr = c / (BS / 8), vc = c % (BS / 8);
      uint2* vd = reinterpret_cast<uint2*>(vs + vr * C::kVStride + vc * 8);
      vd[0] = make_uint2(pv[u].x, pv[u].y);
      vd[1] = make_uint2(pv[u].z, pv[u].w);
    }
  };
  auto valid_tile = [&](int32_t kt) { return kt >= 0 && kt < n_tiles; };

  int it = 0;
  while (it < row_len && !valid_tile(row[it])) ++it;
  if (it < row_len) fetch(row[it]);
  while (it < row_len) {
    const int32_t kt = row[it];
    int nxt = it + 1;
    while (nxt < row_len && !valid_tile(row[nxt])) ++nxt;
    __syncthreads();
    stash();
    __syncthreads();
    if (nxt < row_len) fetch(row[nxt]);

    // S^T blocks: s[kb] covers keys kb*32 .. +32 (rows) x the wave's 32
    // queries (columns).  Lane (li, g), element r: key 8(r/4) + 4g + r%4.
    f32x16 s[BS / 32];
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) {
      s[kb] = f32x16{};
      const __bf16* ka = ks + (kb * 32 + li) * C::kKStride + 8 * g;
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(ka + 16 * m), qf[m], s[kb], 0, 0, 0);
    }
    const bool full = tile_count[kt] == BS;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) {
      const uint32_t bits = full ? 0xffffffffu : tile_bits[kt * 4 + kb];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r / 4) + 4 * g + (r % 4);
        float x = s[kb][r] * scale_log2;
        if (!((bits >> key) & 1u)) x = -INFINITY;
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[BS / 32][2];
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(s[kb][8 * h + e] - m_new);
          psum += p[e];
        }
        pb[kb][h] = __builtin_convertvector(p, bf16x8);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

    // O^T[db] += V^T[db rows, keys] P^T.  For MFMA (kb, h) the k slots of
    // lane group g, element e are keys kb*32 + 16h + 8(e/4) + 4g + e%4,
    // matching the S^T accumulator registers 8h .. 8h+7.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const __bf16* va = vs + (db * 32 + li) * C::kVStride + 4 * g;
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(va + kb * 32 + 16 * h);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(va + kb * 32 + 16 * h + 8);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][h], o[db], 0, 0, 0);
        }
      }
    }
    it = nxt;
  }

  // Lane (li, g) holds O^T[dd = db*32 + 8a + 4g + b][query li].
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow >= Lp) return;
  const int qs = wave * 32 + li;
  const bool qvalid = (tile_bits[qtile * 4 + qs / 32] >> (qs % 32)) & 1u;
  const float inv = (qvalid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  __bf16* dst = op + (bh * Lp + qrow) * D + 4 * g;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float4 v4 = make_float4(o[db][4 * a] * inv, o[db][4 * a + 1] * inv,
                              o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv);
      typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
      const f32x4 f = {v4.x, v4.y, v4.z, v4.w};
      *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * a) = __builtin_convertvector(f, bf16x4);
    }
  }
}

// ---------------------------------------------------------------- fp32

template <int D, int BS>
__global__ __launch_bounds__(BS) void attn_f32_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp,
    const float* __restrict__ vt, const int32_t* __restrict__ kept,
    float* __restrict__ op, const uint32_t* __restrict__ tile_bits,
    const int32_t* __restrict__ tile_count, int64_t Lp, int32_t BH,
    int32_t nb, int32_t n_tt, int32_t row_len_video, int64_t nnz,
    float scale) {
  // Keys are staged 32 at a time: K rows and V^T columns of one chunk.
  __shared__ __align__(16) float ks[32][D];
  __shared__ __align__(16) float vs[D][32];
  const int32_t n_tiles = nb + n_tt;
  const TileJob job = job_of(blockIdx.x, BH, nb, n_tt);
  const int64_t bh = job.bh;
  const int32_t qtile = job.tile;
  const int t = threadIdx.x;
  const int64_t qrow = int64_t(qtile) * BS + t;
  const float* kh = kp + bh * Lp * D;
  const float* vh = vt + bh * int64_t(n_tiles) * D * BS;
  const int32_t* row = kept + bh * nnz + row_offset(qtile, nb, row_len_video, n_tiles);
  const int32_t row_len = qtile < nb ? row_len_video : n_tiles;

  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qrow < Lp ? qp[(bh * Lp + qrow) * D + c] : 0.f;
    o[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int it = 0; it < row_len; ++it) {
    const int32_t kt = row[it];
    if (kt < 0 || kt >= n_tiles) continue;
    const bool full = tile_count[kt] == BS;
    for (int kc = 0; kc < BS / 32; ++kc) {
      __syncthreads();
      for (int c = t; c < 32 * D; c += BS) {
        const int r = c / D, cc = c % D;
        const int64_t slot = int64_t(kt) * BS + kc * 32 + r;
        ks[r][cc] = slot < Lp ? kh[slot * D + cc] : 0.f;
        const int vr = c / 32, vc = c % 32;
        vs[vr][vc] = vh[(int64_t(kt) * D + vr) * BS + kc * 32 + vc];
      }
      __syncthreads();
      const uint32_t bits = full ? 0xffffffffu : tile_bits[kt * 4 + kc];
      float s[32];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc = fmaf(q[c], ks[j][c], acc);
        acc = ((bits >> j) & 1u) ? acc * scale : -INFINITY;
        s[j] = acc;
        mx = fmaxf(mx, acc);
      }
      const float m_new = fmaxf(m_run, mx);
      if (m_new == -INFINITY) continue;  // chunk of pad keys only
      const float alpha = expf(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        s[j] = expf(s[j] - m_new);
        psum += s[j];
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        float acc = o[c] * alpha;
#pragma unroll
        for (int j = 0; j < 32; ++j) acc = fmaf(s[j], vs[c][j], acc);
        o[c] = acc;
      }
    }
  }
  if (qrow >= Lp) return;
  const bool qvalid = (tile_bits[qtile * 4 + t / 32] >> (t % 32)) & 1u;
  const float inv = (qvalid && l_run > 0.f) ? 1.f / l_run : 0.f;
  float* dst = op + (bh * Lp + qrow) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) dst[c] = o[c] * inv;
}

template <int D, int BS>
void launch_bf16(const rf_plan* p, const void* qp, const void* kp,
                 const void* vt, const int32_t* kept, void* op, int BH,
                 const rf_keep& kc, float scale, hipStream_t st) {
  const int nb = p->sz.nb, n_tt = p->sz.n_text_tiles;
  dim3 grid(BH * (nb + n_tt));
  hipLaunchKernelGGL((attn_bf16_kernel<D, BS>), grid,
                     dim3(Bf16Cfg<D, BS>::kThreads), 0, st,
                     static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp),
                     static_cast<const __bf16*>(vt), kept, static_cast<__bf16*>(op),
                     p->tile_bits, p->tile_count, p->sz.Lp, BH, nb, n_tt,
                     kc.row_len_video, kc.nnz_per_head,
                     scale * 1.4426950408889634f);
}

template <int D, int BS>
void launch_f32(const rf_plan* p, const void* qp, const void* kp,
                const void* vt, const int32_t* kept, void* op, int BH,
                const rf_keep& kc, float scale, hipStream_t st) {
  const int nb = p->sz.nb, n_tt = p->sz.n_text_tiles;
  dim3 grid(BH * (nb + n_tt));
  hipLaunchKernelGGL((attn_f32_kernel<D, BS>), grid, dim3(BS), 0, st,
                     static_cast<const float*>(qp), static_cast<const float*>(kp),
                     static_cast<const float*>(vt), kept, static_cast<float*>(op),
                     p->tile_bits, p->tile_count, p->sz.Lp, BH, nb, n_tt,
                     kc.row_len_video, kc.nnz_per_head, scale);
}

}  // namespace

extern "C" rf_status rf_sparse_attn(const rf_plan* plan, const void* qp,
                                    const void* kp, const void* vt,
                                    const int32_t* kept_idx,
                                    int32_t sparsity_pct, void* op, int32_t B,
                                    int32_t H, int32_t d, float scale,
                                    rf_dtype dtype, hipStream_t stream) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, "rf_sparse_attn");
  if (st != RF_OK) return st;
  if (!rf::aligned16(qp) || !rf::aligned16(kp) || !rf::aligned16(vt) ||
      !rf::aligned16(kept_idx) || !rf::aligned16(op))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn: null or misaligned buffer");
  if (!(scale > 0.f) || !(scale < 1e30f))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn: scale must be positive and finite");
  rf_keep kc;
  st = rf_keep_count(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  const int BH = B * H;
  if (int64_t(BH) * plan->sz.n_tiles >= (int64_t(1) << 31))
    return rf::fail(RF_ERR_UNSUPPORTED, "rf_sparse_attn: too many tiles");
  const int bs = plan->sz.bs;
  if (dtype == RF_BF16) {
    if (d == 128 && bs == 128) launch_bf16<128, 128>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
    else if (d == 128 && bs == 64) launch_bf16<128, 64>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
    else if (d == 64 && bs == 128) launch_bf16<64, 128>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
    else launch_bf16<64, 64>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
  } else {
    if (d == 128 && bs == 128) launch_f32<128, 128>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
    else if (d == 128 && bs == 64) launch_f32<128, 64>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
    else if (d == 64 && bs == 128) launch_f32<64, 128>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
    else launch_f32<64, 64>(plan, qp, kp, vt, kept_idx, op, BH, kc, scale, stream);
  }
  return rf::check_launch("rf_sparse_attn");
}
