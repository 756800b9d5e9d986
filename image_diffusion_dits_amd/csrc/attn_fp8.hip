// FP8 variant of the block-sparse attention forward (RainFusion2.0 page,
// TL;DR: integration with quantization named as future work): QK^T and PV on
// OCP e4m3 operands with v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation and
// softmax, bf16 output.  Operands come from rf_quantize_fp8: Q and K with one
// power-of-two scale per tile, V^T tiles with one per feature.
//
// The structure is the bf16 ping-pong kernel's (two groups of four waves per
// 128-slot query tile, one phase apart: MFMA phase PV(i-1) then S(i), VALU
// phase softmax(i)).  What changes with 8-bit operands:
//   * tiles are 16 KB, so each group double-buffers K and V^T (128 KB of
//     LDS) and starts the copies of K(i+1) and V^T(i) at the end of its MFMA
//     phase of tile i, into the slots that phase did not read: the issue
//     stalls of the copies fall in the wait at the barrier rather than in
//     the softmax;
//   * one MFMA reduces 64 features (or keys): 8 MFMAs for S and 8 for PV per
//     tile and wave, each fed 32 bytes per lane (two 16-byte LDS reads);
//   * P^T must reach the PV MFMA straight from the S^T accumulators.  Lane
//     group g of S block kb holds MFMA rows 8a + 4g + b, so K rows are
//     copied into LDS permuted: LDS row 32 kb + x holds key
//       pi(kb, x) = 64 (kb/2) + 32 ((x/4) % 2) + 16 (kb % 2) + 4 (x/8) + x % 4,
//     and register r of block kb in lane group g is key
//       64 (kb/2) + 32 g + 16 (kb % 2) + r.
//     The 32 weights of blocks 2s and 2s + 1 in lane group g are then keys
//     64 s + 32 g .. +32 in order, which is exactly the 32-byte V^T run the
//     same lane group reads for k-step s;
//   * the row sum of the e4m3 weights comes from two more MFMAs whose A
//     operand is 1 for valid and 0 for pad keys, so the normalisation uses
//     the weights the PV product used, the vector ALU does not convert them
//     back, and pad keys of partial tiles need no mask on the usual path;
//   * logits are dot(q8, k8) * scale * 2^(eq + ek) (the key tile's scale
//     enters the exp2 multiplier), and the feature scales of V multiply the
//     output once at the end.
// Weights are exp2(l - m + 4) <= 2^8 under a lazy rescale with threshold 4,
// inside the e4m3 range (448), with weights down to 2^-10 of the row maximum
// still normal e4m3 numbers.
#include "rf_internal.h"
#include "tile_common.h"

namespace {

using namespace rf_tile;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int BS = 128;
constexpr int kGroupWaves = 4;
constexpr int kThreads = 2 * kGroupWaves * 64;
constexpr int kRowBytes = 128;                  // K row (D fp8) and V^T row (BS fp8)
constexpr int kTileBytes = BS * D;              // 16 KB
constexpr int kCopies = kTileBytes / 16 / (kGroupWaves * 64);   // 4 per thread
static_assert(kCopies == 4, "copy split");
// Softmax weights: rescale threshold and exponent shift (log2 units); their
// sum bounds every weight by 2^8, within e4m3's largest finite value.
// A smaller threshold allows a larger shift (finer small weights) but makes
// rescales more frequent: 8/0 -> 4/4 costs about 1.5% of the kernel's time at
// 720p / 80% sparsity and cuts the error of the weight sum about tenfold on
// wide logit distributions.
constexpr float kRescale = 4.f;
constexpr float kShift = 4.f;
static_assert(kRescale + kShift <= 8.f, "weights must stay within e4m3");

__device__ inline f32x16 mma(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four e4m3 codes in one word.  The first conversion writes the low half and
// keeps the high half of its `old` operand, which the second overwrites, so
// `old` is any register (here a's): no zeroing move is needed.
__device__ inline int pack4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

__global__ __launch_bounds__(kThreads, 2) void attn_fp8_pp_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const int32_t* __restrict__ kept, __bf16* __restrict__ op, float* __restrict__ lse,
    const int32_t* __restrict__ out_row, int64_t out_rows,
    const uint32_t* __restrict__ tile_bits, const int32_t* __restrict__ tile_count,
    int64_t Lt, int32_t BH, int32_t nb, int32_t n_tt, int32_t row_len_video, int64_t nnz,
    float scale_log2) {
  constexpr int kWaitVm0 = 0x0F70;     // s_waitcnt vmcnt(0)
  // Two K and two V^T tiles per group (K(i) in K slot i % 2, V^T(i) in V
  // slot i % 2); reused for the merge.
  __shared__ __align__(16) uint8_t lds[8 * kTileBytes];
  __shared__ float m_buf[kGroupWaves * 64], l_buf[kGroupWaves * 64];

  const int32_t n_tiles = nb + n_tt;
  const TileJob job = job_of(blockIdx.x, BH, nb, n_tt);
  const int64_t bh = job.bh;
  const int32_t qtile = job.tile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int grp = wave / kGroupWaves;
  const int qw = wave % kGroupWaves;
  const int lane = threadIdx.x % 64;
  const int li = lane % 32, g = lane / 32;
  uint8_t* const kslot = lds + (4 * grp) * kTileBytes;       // + (i % 2) * kTileBytes
  uint8_t* const vslot = lds + (4 * grp + 2) * kTileBytes;

  const char* kh = reinterpret_cast<const char*>(k8 + bh * Lt * D);
  const char* vh = reinterpret_cast<const char*>(v8 + bh * int64_t(n_tiles) * D * BS);
  const float* ksc = k_scale + bh * n_tiles;
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, qtile, nb, row_len_video, n_tiles);
  const __attribute__((address_space(4))) int32_t* row =
      (const __attribute__((address_space(4))) int32_t*)(kept + bh * nnz + rr.offset);
  const int32_t row_len = rr.len;
  // Phase pairs of the walk; on an odd row group 1 has one step fewer and
  // does no work in the missing one (it still takes part in the barriers).
  const int32_t n_grp = (row_len + 1) / 2;
  const int32_t n_own = (row_len + 1 - grp) / 2;
  // Kept tile of this group's step i, or -1 for an id out of range (walked
  // as a fully masked tile).  Past the end of the row the last entry is
  // read; such steps are never walked, and their tiles are read only where
  // a step's existence is tested anyway.
  auto tile_of = [&](int32_t i) -> int32_t {
    const int32_t kt = row[max(min(2 * i + grp, row_len - 1), 0)];
    return uint32_t(kt) < uint32_t(n_tiles) ? kt : -1;
  };

  // Q operand (B of S^T = K Q^T): lane (li, g) holds q[li][64m + 32g .. +32].
  const int64_t qrow = int64_t(qtile) * BS + qw * 32 + li;
  i32x8 qf[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
    qf[m] = *reinterpret_cast<const i32x8*>(q8 + (bh * Lt + qrow) * D + 64 * m + 32 * g);
  const float c_q = scale_log2 * q_scale[bh * n_tiles + qtile];

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  f32x16 lsum = {};                     // every register: the row sum
  float m_run = -INFINITY;
  f32x16 s[BS / 32];
  i32x8 pb[2];
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // e4m3 1.0

  // Copies.  V^T rows land in order; K rows land permuted by pi: copy u fills
  // LDS rows 32u .. 32u + 31 (block kb = u), whose keys are those of copy 0
  // shifted by 64 (u/2) + 16 (u%2).  The swizzle of row 32u + x equals that
  // of row x.
  const int qlin = qw * 64 + lane;
  const int xr = qlin / 8, pc = qlin % 8;
  const int key0 = 32 * ((xr / 4) % 2) + 4 * (xr / 8) + xr % 4;
  const uint32_t koff = uint32_t(key0 * kRowBytes + (pc ^ swz_rows<kRowBytes>(xr)) * 16);
  const uint32_t ksoff[kCopies] = {0u, 16u * kRowBytes, 64u * kRowBytes, 80u * kRowBytes};
  const uint32_t voff = dma_offset<kRowBytes, kRowBytes, kGroupWaves>(qw, lane);
  // One buffer resource per head for each of K and V^T; a tile's offset
  // goes to the copies' scalar offset.
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(kh), 0, n_tiles * kTileBytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(vh), 0, n_tiles * kTileBytes, kBufferWord3);
  auto copy_k = [&](int32_t kt, int par) {
    dma_tile_perm_at<kCopies, kGroupWaves>(krsrc, max(kt, 0) * kTileBytes,
                                           kslot + par * kTileBytes, koff, qw, ksoff);
  };
  auto copy_v = [&](int32_t kt, int par) {
    dma_tile_at<kCopies, kGroupWaves>(vrsrc, max(kt, 0) * kTileBytes, vslot + par * kTileBytes,
                                      voff, qw);
  };
  const int rswz = swz_rows<kRowBytes>(li);     // rows 32 kb + li and 32 db + li
  // 32 bytes of row r at 16-byte chunks c0 and c0 + 1 (c0 = 4 step + 2g): the
  // row offset and the two swizzled chunk offsets 16 ((2g + e) ^ swz) are
  // passed through an empty asm at each phase, so the addresses of the
  // current slots are derived there instead of held for both parities.
  auto operand = [&](const uint8_t* rowp, int step, int x0, int x1) -> i32x8 {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(rowp + ((64 * step) ^ x0));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(rowp + ((64 * step) ^ x1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  constexpr int kAhead = 4;                     // MFMAs whose operands are read ahead
  auto pipeline_reads = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);    // DS reads
#pragma unroll
    for (int j = 0; j < 8 - kAhead; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);           // DS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };

  // Row-sum operand of the previous tile: e4m3 1.0 for every valid key, 0 for
  // pad keys (whose weights need not be zero, see the VALU phase).  Byte e of
  // k-step st in lane group g is key 64 st + 32 g + e: bit e of validity word
  // 2 st + g, which the VALU phase leaves in vw[st] (all ones for a full
  // tile), spread four bits per dword by a multiply.
  uint32_t vw[2] = {~0u, ~0u};
  bool vw_full = true;
  auto row_sum_operand = [&](int st) -> i32x8 {
    if (vw_full) return ones;
    i32x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t nib = (vw[st] >> (4 * e)) & 0xfu;
      a[e] = int(((nib * 0x00204081u) & 0x01010101u) * 0x38u);
    }
    return a;
  };

  // Per-tile scalars of this group's walk, carried in SGPRs: the kept tiles
  // of steps i and i + 1, the validity words and the K scale of step i.
  // Each VALU phase loads those of the next step early on (uniform scalar
  // loads: a per-lane vector load would wait, in order, for every tile copy
  // issued before it), so that no phase starts waiting on scalar memory.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const __attribute__((address_space(4))) u32x4* tbits4 =
      (const __attribute__((address_space(4))) u32x4*)tile_bits;
  const __attribute__((address_space(4))) float* kscale =
      (const __attribute__((address_space(4))) float*)ksc;
  int32_t kt_cur = tile_of(0), kt_nxt = tile_of(1);
  u32x4 bits_cur = tbits4[max(kt_cur, 0)];
  float ks_cur = kscale[max(kt_cur, 0)];
  // Validity word w + g of the current tile (0 for a masked tile).
  auto tile_word = [&](const u32x4& b, int w) -> uint32_t {
    const uint32_t w0 = w == 0 ? b.x : b.z, w1 = w == 0 ? b.y : b.w;
    return g ? w1 : w0;
  };

  // The wave in its MFMA phase takes issue priority over the softmax wave on
  // its SIMD.  Otherwise the older wave wins each issue cycle whatever it
  // runs: in the phase where group 1 issues MFMAs beside group 0's softmax,
  // its MFMAs waited for issue slots and that phase took about 700 cycles
  // more than the other (per step, 720p video).
  // MFMA phase of step i: PV of step i - 1 if pv, scores of step i if sc.
  auto mfma_phase = [&](int32_t i, bool pv, bool sc) {
    __builtin_amdgcn_s_setprio(3);
    int lrow = li * kRowBytes, x0 = ((2 * g) ^ rswz) * 16, x1 = ((2 * g + 1) ^ rswz) * 16;
    asm volatile("" : "+v"(lrow), "+v"(x0), "+v"(x1));
    if (pv) {
      // O^T[db] += V^T[db rows, keys 64s .. +64] P^T(i-1), k-steps s = 0, 1.
      const uint8_t* const vs = vslot + ((i - 1) & 1) * kTileBytes + lrow;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = mma(operand(vs + db * 32 * kRowBytes, st, x0, x1), pb[st], o[db]);
      pipeline_reads();
      lsum = mma(row_sum_operand(0), pb[0], lsum);
      lsum = mma(row_sum_operand(1), pb[1], lsum);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (sc) {
      const uint8_t* const ks = kslot + (i & 1) * kTileBytes + lrow;
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int m = 0; m < 2; ++m)
          s[kb] = mma(operand(ks + kb * 32 * kRowBytes, m, x0, x1), qf[m], s[kb]);
      }
      pipeline_reads();
      // The copies of K(i+1) and V^T(i) go to the slots not read in this
      // phase (they were last read in the group's previous MFMA phase), after
      // this phase's LDS reads: their issue stalls fall in the wait at the
      // barrier, and the group's VALU phase waits for them at its end.
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < n_own) {
        poison_tile<kCopies, kGroupWaves>(kslot + ((i + 1) & 1) * kTileBytes, qw, lane);
        copy_k(kt_nxt, (i + 1) & 1);
      }
      poison_tile<kCopies, kGroupWaves>(vslot + (i & 1) * kTileBytes, qw, lane);
      copy_v(kt_cur, i & 1);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto valu_phase = [&](int32_t i) {
    const int32_t kt = kt_cur;
    // The next step's scalars (in flight during the softmax).
    const int32_t kt_n2 = tile_of(i + 2);
    const u32x4 bits_n = tbits4[max(kt_nxt, 0)];
    const float ks_n = kscale[max(kt_nxt, 0)];
    const u32x4 bits = kt >= 0 ? bits_cur : u32x4{0u, 0u, 0u, 0u};
    const float c = c_q * (kt >= 0 ? ks_cur : 1.f);
    vw_full = (bits.x & bits.y & bits.z & bits.w) == 0xFFFFFFFFu;
#pragma unroll
    for (int st = 0; st < 2; ++st) vw[st] = tile_word(bits, 2 * st);
    // Row max over the tile's raw dot products (the scale is positive).
    auto row_max = [&]() {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[kb][r]);
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(m),
                                                       __float_as_uint(m), false, false);
      return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));   // with lane ^ 32
    };
    float mx = row_max();
    // Pad keys have all-zero K rows, so their scores are exactly 0, and
    // all-zero V^T columns, so their weights add nothing to O; the row sum
    // counts valid keys only.  When every query's tile maximum is positive it
    // comes from a valid key, and a pad weight 2^(0 - m + kShift) stays below
    // 2^(kRescale + kShift) = 2^8 (see below), so the pads need no mask.
    // Otherwise (and for a masked tile, kt < 0, whose copies hold tile 0)
    // they are set to -inf.
    if (!vw_full && (kt < 0 || __ballot(!(mx > 0.f)) != 0)) {
      // Register r of block kb in lane group g is key 64(kb/2) + 32g +
      // 16(kb%2) + r: validity word 2(kb/2) + g, bit 16(kb%2) + r.
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb) {
        const uint32_t pad =
            ~(tile_word(bits, 2 * (kb / 2)) >> (16 * (kb % 2)));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t m = uint32_t(int32_t(pad << (31 - r)) >> 31);
          s[kb][r] = __uint_as_float((m & 0xff800000u) | (~m & __float_as_uint(s[kb][r])));
        }
      }
      mx = row_max();
    }
    // Weights are 2^(logit - m + kShift), m the running maximum, which only
    // moves (rescaling O and l) when some query's tile maximum exceeds it by
    // more than kRescale: every weight then stays within 2^8 (e4m3 holds up
    // to 448), and the shift puts weights down to 2^-10 of the maximum in the
    // normal e4m3 range instead of leaving them to the subnormal steps.
    const float mt = mx * c;
    if (__ballot(mt > m_run + kRescale) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      lsum[0] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : kShift - m_run;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kb = 2 * st + e / 4, r0 = 4 * (e % 4);
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + j], c, neg_m));
        pb[st][e] = pack4(p[0], p[1], p[2], p[3]);
      }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the copies have landed
    // The next step's scalars have arrived too (forced here, before the
    // barrier, so that no scalar load is in flight during the MFMA phase,
    // where it would coarsen the LDS waits).
    asm volatile("" ::"s"(kt_n2), "s"(bits_n.x), "s"(bits_n.y), "s"(bits_n.z),
                 "s"(bits_n.w), "s"(ks_n));
    kt_cur = kt_nxt;
    kt_nxt = kt_n2;
    bits_cur = bits_n;
    ks_cur = ks_n;
  };

  if (n_own > 0) {
    poison_tile<kCopies, kGroupWaves>(kslot, qw, lane);
    copy_k(kt_cur, 0);
  }
  // Every scalar the loop reads is resident before it starts (a scalar load
  // pending at the loop entry would coarsen the LDS waits of every phase).
  asm volatile("" ::"s"(kt_nxt), "s"(bits_cur.x), "s"(bits_cur.y), "s"(bits_cur.z),
               "s"(bits_cur.w), "s"(ks_cur), "s"(scale_log2), "s"(c_q), "s"(n_grp), "s"(n_own),
               "s"(row_len));
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_barrier();
  // Phase pairs i = 0 .. n_grp: MFMA(i) takes the PV of step i - 1 and the
  // scores of step i where those steps are the group's own (i - 1 < n_own,
  // i < n_own; n_own is n_grp for group 0), and VALU(i) runs for i < n_own.
  if (grp == 0) {
    for (int32_t i = 0; i <= n_grp; ++i) {
      mfma_phase(i, i >= 1, i < n_grp);
      __builtin_amdgcn_s_barrier();
      if (i < n_grp) valu_phase(i);
      __builtin_amdgcn_s_barrier();
    }
  } else {
    for (int32_t i = 0; i <= n_grp; ++i) {
      const bool own_prev = i >= 1 && i - 1 < n_own;
      if (own_prev) valu_phase(i - 1);
      __builtin_amdgcn_s_barrier();
      mfma_phase(i, own_prev, i < n_own);
      __builtin_amdgcn_s_barrier();
    }
  }

  // Merge: group 1 publishes O (register quads), m and l; group 0 combines,
  // applies the feature scales of V and stores.
  float4* ob = reinterpret_cast<float4*>(lds);
  constexpr int kQuads = D / 32 * 4;
  const float l_run = lsum[0];
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        ob[((qw * kQuads + db * 4 + a) * 64) + lane] =
            make_float4(o[db][4 * a], o[db][4 * a + 1], o[db][4 * a + 2], o[db][4 * a + 3]);
    m_buf[qw * 64 + lane] = m_run;
    l_buf[qw * 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp == 1) return;
  const float m_b = m_buf[qw * 64 + lane], l_b = l_buf[qw * 64 + lane];
  const float m_t = fmaxf(m_run, m_b);
  const float fa = m_t == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_t);
  const float fb = m_t == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_b - m_t);
  const float l_tot = l_run * fa + l_b * fb;   // both lane groups hold the full sum
  const int qs = qw * 32 + li;
  const bool qvalid = (tile_bits[qtile * 4 + qs / 32] >> (qs % 32)) & 1u;
  const float inv = (qvalid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const float ca = fa * inv, cb = fb * inv;
  // Output row of this query slot: the slot itself, or (raster output) its
  // raster token, -1 for a pad slot, which then has no output row.
  const int64_t orow = out_row != nullptr ? int64_t(out_row[qrow]) : qrow;
  if (orow < 0) return;
  if (lse != nullptr && g == 0) lse[bh * out_rows + orow] = lse_of(m_t - kShift, l_tot, qvalid);
  // Lane (li, g) holds O^T[dd = db*32 + 8a + 4g + b][query li].
  __bf16* dst = op + (bh * out_rows + orow) * D + 4 * g;
  const float* vsc = v_scale + bh * D + 4 * g;
  typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
  typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 x = ob[((qw * kQuads + db * 4 + a) * 64) + lane];
      const float4 w = *reinterpret_cast<const float4*>(vsc + db * 32 + 8 * a);
      const f32x4 f = {(o[db][4 * a] * ca + x.x * cb) * w.x,
                       (o[db][4 * a + 1] * ca + x.y * cb) * w.y,
                       (o[db][4 * a + 2] * ca + x.z * cb) * w.z,
                       (o[db][4 * a + 3] * ca + x.w * cb) * w.w};
      *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * a) = __builtin_convertvector(f, bf16x4);
    }
  }
}

rf_status attn_fp8(const rf_plan* plan, const void* q8, const float* q_scale, const void* k8,
                   const float* k_scale, const void* v8, const float* v_scale,
                   const int32_t* kept, int32_t row_len_video, int64_t nnz, void* op,
                   float* lse, int32_t B, int32_t H, int32_t d, float scale, hipStream_t stream,
                   const char* fn, bool raster = false) {
  rf_status st = rf::check_call(plan, B, H, d, RF_BF16, fn);
  if (st != RF_OK) return st;
  if (d != D || plan->sz.bs != BS)
    return rf::fail(RF_ERR_UNSUPPORTED, "%s: the FP8 kernel needs d = %d and bs = %d", fn, D, BS);
  if (!rf::aligned16(q8) || !rf::aligned16(k8) || !rf::aligned16(v8) ||
      !rf::aligned16(kept) || !rf::aligned16(op) || !rf::aligned16(v_scale) ||
      q_scale == nullptr || k_scale == nullptr ||
      (reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  if (reinterpret_cast<uintptr_t>(lse) & 3u)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: misaligned lse", fn);
  if (!(scale > 0.f) || !(scale < 1e30f))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  const int BH = B * H;
  if (int64_t(BH) * plan->sz.n_tiles >= (int64_t(1) << 31))
    return rf::fail(RF_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  const int nb = plan->sz.nb, n_tt = plan->sz.n_text_tiles;
  hipLaunchKernelGGL(attn_fp8_pp_kernel, dim3(BH * (nb + n_tt)), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(q8), q_scale, static_cast<const uint8_t*>(k8),
                     k_scale, static_cast<const uint8_t*>(v8), v_scale, kept,
                     static_cast<__bf16*>(op), lse, raster ? plan->slot_src : nullptr,
                     raster ? plan->sz.L : plan->sz.Lt, plan->tile_bits, plan->tile_count,
                     plan->sz.Lt, BH, nb, n_tt, row_len_video, nnz,
                     scale * 1.4426950408889634f);
  return rf::check_launch(fn);
}

}  // namespace

extern "C" rf_status rf_sparse_attn_fp8(const rf_plan* plan, const void* q8,
                                        const float* q_scale, const void* k8,
                                        const float* k_scale, const void* v8,
                                        const float* v_scale, const int32_t* kept_idx,
                                        int32_t sparsity_pct, void* op, float* lse_or_null,
                                        int32_t B, int32_t H, int32_t d, float scale,
                                        hipStream_t stream) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_fp8: null plan");
  rf_keep kc;
  rf_status st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  return attn_fp8(plan, q8, q_scale, k8, k_scale, v8, v_scale, kept_idx, kc.row_len_video,
                  kc.nnz_per_head, op, lse_or_null, B, H, d, scale, stream,
                  "rf_sparse_attn_fp8");
}

extern "C" rf_status rf_sparse_attn_fp8_raster(const rf_plan* plan, const void* q8,
                                               const float* q_scale, const void* k8,
                                               const float* k_scale, const void* v8,
                                               const float* v_scale, const int32_t* kept_idx,
                                               int32_t sparsity_pct, void* o, float* lse_or_null,
                                               int32_t B, int32_t H, int32_t d, float scale,
                                               hipStream_t stream) {
  if (plan == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_fp8_raster: null plan");
  if (o != nullptr && (o == q8 || o == k8 || o == v8))
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_fp8_raster: o must not overlap the operands");
  rf_keep kc;
  rf_status st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  return attn_fp8(plan, q8, q_scale, k8, k_scale, v8, v_scale, kept_idx, kc.row_len_video,
                  kc.nnz_per_head, o, lse_or_null, B, H, d, scale, stream,
                  "rf_sparse_attn_fp8_raster", true);
}

extern "C" rf_status rf_sparse_attn_fp8_rows(const rf_plan* plan, const void* q8,
                                             const float* q_scale, const void* k8,
                                             const float* k_scale, const void* v8,
                                             const float* v_scale, const int32_t* kept_rows,
                                             int32_t row_width, void* op,
                                             float* lse_or_null, int32_t B, int32_t H,
                                             int32_t d, float scale, hipStream_t stream) {
  if (plan == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_fp8_rows: null plan");
  if (row_width < 1 || row_width > plan->sz.n_tiles)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_fp8_rows: row_width %d outside [1, %d]",
                    row_width, plan->sz.n_tiles);
  return attn_fp8(plan, q8, q_scale, k8, k_scale, v8, v_scale, kept_rows, -row_width,
                  int64_t(plan->sz.n_tiles) * row_width, op, lse_or_null, B, H, d, scale,
                  stream,
                  "rf_sparse_attn_fp8_rows");
}
