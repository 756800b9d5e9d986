// Block-sparse flash-attention forward over the kept tiles (RainFusion2.0
// page, Abstract: skip computation for insignificant tokens, block-wise
// sparse attention; RainFusion review page, Assumptions: softmax attention,
// Eq. (1)).
//
// bf16 path (gfx950 MFMA), one wave per 32 queries.  Per kept key tile:
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
// the softmax rescale is a per-lane scalar.  K and V^T tiles are copied into
// XOR-swizzled LDS rows by LDS DMA (conflict-free 16-byte reads).  Pad keys
// get -inf from the plan's per-tile validity masks; pad query rows are
// written as zeros.  Workgroups are renumbered so that each XCD (one L2)
// works on a contiguous range of query tiles of one head; the heavy text
// query tiles (which keep every tile) start first.
//
// For 128-slot tiles the ping-pong kernel runs two groups of four waves per
// query tile, one phase apart, so that MFMA and softmax work of the two
// waves on each SIMD overlap (attn_bf16_pp_kernel); 64-slot tiles use one
// group of waves that alternates the phases itself (attn_bf16_kernel).
//
// fp32 path: one thread per query row, fp32 FMA and expf, the same tile
// walk; used where fp32 accuracy is required.
#include "rf_internal.h"
#include "tile_common.h"

#include <type_traits>

namespace {

using namespace rf_tile;

typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));

// Rows of the query operand, the output and the LSE.  slot_src == nullptr:
// permuted tensors [BH][Lt][d] ([BH][Lt] for the LSE), query slot q at row q.
// Otherwise raster tensors [BH][rows][d]: slot q reads and writes raster row
// slot_src[q], and pad slots (slot_src < 0) read zeros and write nothing.
struct RowIo {
  const int32_t* slot_src;
  int64_t rows;
};

__device__ inline int64_t io_row(const RowIo& io, int64_t slot) {
  return io.slot_src != nullptr ? int64_t(io.slot_src[slot]) : slot;
}

// ---------------------------------------------------------------- bf16 MFMA

typedef const __attribute__((address_space(1))) void global_cvoid;

template <int D, int BS>
struct Bf16Cfg {
  static constexpr int kWaves = BS / 32;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKRowBytes = D * 2;     // one K row (bf16)
  static constexpr int kVRowBytes = BS * 2;    // one V^T row (bf16)
  static constexpr int kKChunks = BS * D / 8;  // 16-byte chunks per K tile
  static constexpr int kVChunks = D * BS / 8;  // 16-byte chunks per V^T tile
  static constexpr int kKLoads = kKChunks / kThreads;  // per thread
  static constexpr int kVLoads = kVChunks / kThreads;
  static_assert(kKChunks % kThreads == 0 && kVChunks % kThreads == 0, "tile");
};

// XOR swizzle of the 16-byte chunks of an LDS row.  Rows of 256 bytes span
// all 64 banks, so chunk p of row r is stored at p ^ (r % 16); rows of 128
// bytes pair up per bank sweep, so at p ^ ((r / 2) % 8).  Either way the 16
// lanes of one ds_read_b128 phase, which read one chunk column of 16
// consecutive rows, land on 16 distinct bank groups.
template <int ROW_BYTES>
__device__ inline int swz(int row) {
  if constexpr (ROW_BYTES >= 256) return row % 16;
  else return (row / 2) % 8;
}

// sigma swaps bits 2 and 3 of a row index inside a 32-row MFMA block.
__device__ inline int sigma(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Lane offset (bytes) of a wave's global -> LDS copies of one tile whose
// LDS rows are ROW_BYTES long: copy u of wave w moves 16-byte chunk
// u*THREADS + w*64 + lane of the tile.  When the rows advanced per copy are
// a multiple of 16 the swizzle of the copied row, and so the offset, is the
// same for every copy; otherwise it alternates between two values.
template <int ROW_BYTES, int THREADS>
struct CopyPlan {
  static constexpr int kCpr = ROW_BYTES / 16;          // chunks per row
  static constexpr int kRowsPerCopy = THREADS / kCpr;  // rows per copy step
  static constexpr int kVariants = (kRowsPerCopy % 16 == 0) ? 1 : 2;
  // Global byte offset, inside the tile, of the chunk this lane copies in
  // copy u (u < kVariants gives the per-lane part; add u*kRowsPerCopy rows).
  __device__ static uint32_t lane_offset(int wave, int lane, int u) {
    const int pch = u * THREADS + wave * 64 + lane;
    const int r = pch / kCpr, pc = pch % kCpr;
    const int gc = pc ^ swz<ROW_BYTES>(r);
    return uint32_t(((r - u * kRowsPerCopy) * ROW_BYTES) + gc * 16);
  }
};

template <int D, int BS>
__global__ __launch_bounds__((BS / 32) * 64, 2) void attn_bf16_kernel(
    const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ kept,
    __bf16* __restrict__ op, float* __restrict__ lse, RowIo io,
    const uint32_t* __restrict__ tile_bits,
    const int32_t* __restrict__ tile_count, int64_t Lt, int32_t BH,
    int32_t nb, int32_t n_tt, int32_t row_len_video, int64_t nnz,
    float scale_log2) {
  using C = Bf16Cfg<D, BS>;
  using KCopy = CopyPlan<C::kKRowBytes, C::kThreads>;
  using VCopy = CopyPlan<C::kVRowBytes, C::kThreads>;
  __shared__ __align__(16) __bf16 ks[BS * D];   // K tile, swizzled rows
  __shared__ __align__(16) __bf16 vs[D * BS];   // V^T tile, swizzled rows
  const int32_t n_tiles = nb + n_tt;
  const TileJob job = job_of(blockIdx.x, BH, nb, n_tt);
  const int64_t bh = job.bh;
  const int32_t qtile = job.tile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int li = lane % 32, g = lane / 32;

  const char* kh = reinterpret_cast<const char*>(kp + bh * Lt * D);
  const char* vh = reinterpret_cast<const char*>(vt + bh * int64_t(n_tiles) * D * BS);
  // The kept row is read through the constant address space: uniform
  // scalar loads that do not wait on the tile copies in flight.
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, qtile, nb, row_len_video, n_tiles);
  const __attribute__((address_space(4))) int32_t* row =
      (const __attribute__((address_space(4))) int32_t*)(kept + bh * nnz + rr.offset);
  const int32_t row_len = rr.len;

  // Q operand (B of S^T = K Q^T): lane (li, g) holds q[li][16m + 8g .. +8].
  const int64_t qrow = int64_t(qtile) * BS + wave * 32 + li;
  const int64_t iorow = io_row(io, qrow);
  bf16x8 qf[D / 16];
  {
    const __bf16* qsrc = qp + (bh * io.rows + max(iorow, int64_t(0))) * D + 8 * g;
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
      qf[m] = iorow >= 0 ? *reinterpret_cast<const bf16x8*>(qsrc + 16 * m) : bf16x8{};
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Global -> LDS copies (global_load_lds_dwordx4: lane l of a wave
  // instruction lands at LDS base + 16 l, so the LDS position is fixed and
  // the swizzle is applied to the source chunk).  Addresses are a uniform
  // tile base plus one 32-bit lane offset per variant.
  uint32_t koff[KCopy::kVariants], voff[VCopy::kVariants];
#pragma unroll
  for (int u = 0; u < KCopy::kVariants; ++u) koff[u] = KCopy::lane_offset(wave, lane, u);
#pragma unroll
  for (int u = 0; u < VCopy::kVariants; ++u) voff[u] = VCopy::lane_offset(wave, lane, u);
  auto load_k = [&](int32_t kt) {
    poison_tile<C::kKLoads, C::kWaves>(ks, wave, lane);
    const char* base = kh + int64_t(kt) * BS * C::kKRowBytes;
#pragma unroll
    for (int u = 0; u < C::kKLoads; ++u) {
      const char* src = base + u * KCopy::kRowsPerCopy * C::kKRowBytes;
      __builtin_amdgcn_global_load_lds(
          (global_cvoid*)(src + koff[u % KCopy::kVariants]),
          (lds_void*)(ks + (u * C::kWaves + wave) * 512), 16, 0, 0);
    }
  };
  auto load_v = [&](int32_t kt) {
    poison_tile<C::kVLoads, C::kWaves>(vs, wave, lane);
    const char* base = vh + int64_t(kt) * D * C::kVRowBytes;
#pragma unroll
    for (int u = 0; u < C::kVLoads; ++u) {
      const char* src = base + u * VCopy::kRowsPerCopy * C::kVRowBytes;
      __builtin_amdgcn_global_load_lds(
          (global_cvoid*)(src + voff[u % VCopy::kVariants]),
          (lds_void*)(vs + (u * C::kWaves + wave) * 512), 16, 0, 0);
    }
  };

  // LDS element offsets of this lane's operand chunks.
  //   K (A of S^T): row kb*32 + sigma(li), chunk 2m + g.
  //   V^T (A of O^T): row db*32 + li, chunk 4kb + 2h + g.
  const int krow0 = sigma(li);
  const int kswz = swz<C::kKRowBytes>(krow0);  // kb*32 does not change it
  const int vswz = swz<C::kVRowBytes>(li);     // nor does db*32

  // Schedule per kept tile t (one LDS buffer each for K and V^T):
  //   S(t) = K(t) Q^T                      LDS reads, no copy in flight
  //   barrier; copy K(t+1)
  //   softmax(t) -> P(t)                   VALU, overlaps the K copy
  //   wait copies; barrier
  //   O^T += V^T(t) P^T(t)                 LDS reads, no copy in flight
  //   barrier; copy V(t+1); wait; barrier
  // Keeping copies out of the LDS-read phases keeps the compiler's LDS waits
  // precise (with a copy pending they degrade to full drains); the V copy
  // latency is covered by the other workgroup on the CU.  Waits use the
  // s_waitcnt builtin so the compiler knows the copies have landed; the
  // barriers are plain s_barrier.
  constexpr int kWaitVm0 = 0x0F70;     // s_waitcnt vmcnt(0)
  constexpr int kWaitLgkm0 = 0xC07F;   // s_waitcnt lgkmcnt(0)
  auto next_valid = [&](int i) {
    while (i < row_len && (row[i] < 0 || row[i] >= n_tiles)) ++i;  // own bounds check
    return i;
  };
  int it = next_valid(0);
  if (it < row_len) {
    load_k(row[it]);
    load_v(row[it]);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_barrier();
  while (it < row_len) {
    const int32_t kt = row[it];
    const int nxt = next_valid(it + 1);
    const int32_t kt_next = nxt < row_len ? row[nxt] : 0;
    // Per-tile metadata is loaded here and forced complete before the LDS
    // reads start: scalar loads in flight would also degrade the LDS waits.
    const int32_t tcount = tile_count[kt];
    uint32_t tbits[BS / 32];
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) tbits[kb] = tile_bits[kt * 4 + kb];
    if constexpr (BS == 128)
      asm volatile("" ::"s"(kt_next), "s"(tcount), "s"(tbits[0]), "s"(tbits[1]),
                   "s"(tbits[2]), "s"(tbits[3]) : "memory");
    else
      asm volatile("" ::"s"(kt_next), "s"(tcount), "s"(tbits[0]), "s"(tbits[1])
                   : "memory");

    // S^T blocks: s[kb] covers keys kb*32 .. +32 (rows) x the wave's 32
    // queries (columns).  MFMA row x of block kb is fed K row kb*32 +
    // sigma(x), so accumulator register r = 4a + b of lane group g holds key
    //   kb*32 + 16(a/2) + 8g + 4(a%2) + b,
    // which makes the 8 keys behind registers 8h .. 8h+7 contiguous
    // (kb*32 + 16h + 8g .. +8): the P V product then reads V^T with one
    // 16-byte LDS access per operand.
    f32x16 s[BS / 32];
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) {
      s[kb] = f32x16{};
      const __bf16* ka = ks + (kb * 32 + krow0) * D;
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(ka + ((2 * m + g) ^ kswz) * 8), qf[m],
            s[kb], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    if (nxt < row_len) load_k(kt_next);

    // Row max over the tile (raw dot products; the scale is positive).
    float mx = -INFINITY;
    if (tcount == BS) {
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    } else {
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb) {
        // Keys of lane group g sit at bit 8g + (16(a/2) + 4(a%2) + b).
        const uint32_t bits = tbits[kb] >> (8 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int a = r / 4, b = r % 4;
          const float x = ((bits >> (16 * (a / 2) + 4 * (a % 2) + b)) & 1u)
                              ? s[kb][r] : -INFINITY;
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the running max only moves (and O, l are rescaled)
    // when some query's tile max exceeds it by more than 8 in log2 units;
    // otherwise exponents stay below 2^8 relative to the stale max, which
    // fp32 accumulation and bf16 P absorb.  The final 1/l uses the same
    // reference, so the result is unchanged.
    const float mt = mx * scale_log2;
    if (__ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
    const float neg_m = -m_run;
    float psum[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pb[BS / 32][2];
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * h + e], scale_log2, neg_m));
          psum[e % 4] += p[e];
        }
        pb[kb][h] = __builtin_convertvector(p, bf16x8);
      }
    }
    l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_barrier();

    // O^T[db] += V^T[db rows, keys] P^T; MFMA (kb, h) takes keys
    // kb*32 + 16h + 8g .. +8 in lane group g (see sigma above).
#pragma unroll
    for (int kb = 0; kb < BS / 32; ++kb) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const __bf16* va = vs + (db * 32 + li) * BS;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(va + ((4 * kb + 2 * h + g) ^ vswz) * 8),
              pb[kb][h], o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    if (nxt < row_len) {
      load_v(kt_next);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
    }
    it = nxt;
  }

  // Lane (li, g) holds O^T[dd = db*32 + 8a + 4g + b][query li].
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int qs = wave * 32 + li;
  const bool qvalid = (tile_bits[qtile * 4 + qs / 32] >> (qs % 32)) & 1u;
  const float inv = (qvalid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (iorow < 0) return;                      // pad slot of a raster output
  if (lse != nullptr && g == 0) lse[bh * io.rows + iorow] = lse_of(m_run, l_tot, qvalid);
  __bf16* dst = op + (bh * io.rows + iorow) * D + 4 * g;
  typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 f = {o[db][4 * a] * inv, o[db][4 * a + 1] * inv,
                       o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv};
      *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * a) = __builtin_convertvector(f, bf16x4);
    }
  }
}

// ------------------------------- bf16 MFMA, ping-pong over two wave groups

// One workgroup of eight waves per query tile of 128 slots, one workgroup per
// CU.  Waves w and w + 4 share a SIMD; both hold the same 32 queries.  Group
// 0 (waves 0-3) walks the even entries of the kept row, group 1 the odd
// ones, each with its own K and V^T tile in LDS and its own softmax state.
// Work alternates between two phases separated by workgroup barriers:
//   MFMA phase of tile i:  O^T += V^T(i-1) P^T(i-1), then S(i) = K(i) Q^T
//   VALU phase of tile i:  copies of K(i+1) and V^T(i); softmax(i) -> P(i)
// and the groups are one phase apart, so on every SIMD one wave issues
// MFMAs while the other runs its softmax: the matrix core and the vector
// ALU work at the same time by construction.  The copies of a group land
// during its own VALU phase.  At the end group 1 hands its O, m and l to
// group 0 through LDS and group 0 merges and stores.
template <int D>
struct PpCfg {
  static constexpr int BS = 128;
  static constexpr int kGroupWaves = 4;                 // one per SIMD
  static constexpr int kThreads = 2 * kGroupWaves * 64;
  static constexpr int kKRowBytes = D * 2;              // K row (LDS and global)
  static constexpr int kVRowBytes = BS * 2;             // V^T row (LDS and global)
  static constexpr int kTileBytes = BS * D * 2;         // K or V^T tile
  static constexpr int kTileElems = BS * D;
  static constexpr int kCopies = kTileBytes / 16 / (kGroupWaves * 64);   // per thread
  static_assert(kCopies * 16 * kGroupWaves * 64 == kTileBytes, "copy split");
};

template <int D>
__global__ __launch_bounds__(512, 2) void attn_bf16_pp_kernel(
    const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
    const __bf16* __restrict__ vt, const int32_t* __restrict__ kept,
    __bf16* __restrict__ op, float* __restrict__ lse, RowIo io,
    const uint32_t* __restrict__ tile_bits,
    const int32_t* __restrict__ tile_count, int64_t Lt, int32_t BH,
    int32_t nb, int32_t n_tt, int32_t row_len_video, int64_t nnz,
    float scale_log2) {
  using C = PpCfg<D>;
  constexpr int BS = C::BS;
  constexpr int kWaitVm0 = 0x0F70;     // s_waitcnt vmcnt(0)
  // K and V^T tiles of group 0, then of group 1; reused for the merge.
  __shared__ __align__(16) __bf16 lds[4 * C::kTileElems];

  const int32_t n_tiles = nb + n_tt;
  const TileJob job = job_of(blockIdx.x, BH, nb, n_tt);
  const int64_t bh = job.bh;
  const int32_t qtile = job.tile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int grp = wave / C::kGroupWaves;
  const int qw = wave % C::kGroupWaves;
  const int lane = threadIdx.x % 64;
  const int li = lane % 32, g = lane / 32;
  __bf16* const ks = lds + (2 * grp) * C::kTileElems;
  __bf16* const vsg = lds + (2 * grp + 1) * C::kTileElems;

  const char* kh = reinterpret_cast<const char*>(kp + bh * Lt * D);
  const char* vh = reinterpret_cast<const char*>(vt + bh * int64_t(n_tiles) * D * BS);
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, qtile, nb, row_len_video, n_tiles);
  const __attribute__((address_space(4))) int32_t* row =
      (const __attribute__((address_space(4))) int32_t*)(kept + bh * nnz + rr.offset);
  const int32_t row_len = rr.len;
  // Phase pairs of the walk: group 0 takes the even entries, group 1 the
  // odd ones, so on an odd row group 1 has one step fewer; it still takes
  // part in every barrier but does no work in its missing step.
  const int32_t n_grp = (row_len + 1) / 2;
  const int32_t n_own = (row_len + 1 - grp) / 2;
  // Kept tile of this group's step i, or -1 for an id out of range, which is
  // walked as a fully masked tile (whose copies read tile 0).  Past the end
  // of the row the last entry is read; such steps are never walked, and
  // their tiles are read only where a step's existence is tested anyway.
  auto tile_of = [&](int32_t i) -> int32_t {
    const int32_t kt = row[max(min(2 * i + grp, row_len - 1), 0)];
    return uint32_t(kt) < uint32_t(n_tiles) ? kt : -1;
  };

  // Q operand (B of S^T = K Q^T): lane (li, g) holds q[li][16m + 8g .. +8].
  const int64_t qrow = int64_t(qtile) * BS + qw * 32 + li;
  bf16x8 qf[D / 16];
  {
    const int64_t iorow = io_row(io, qrow);
    const __bf16* qsrc = qp + (bh * io.rows + max(iorow, int64_t(0))) * D + 8 * g;
#pragma unroll
    for (int m = 0; m < D / 16; ++m)
      qf[m] = iorow >= 0 ? *reinterpret_cast<const bf16x8*>(qsrc + 16 * m) : bf16x8{};
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 s[BS / 32];
  bf16x8 pb[BS / 32][2];

  // Each wave copies a contiguous quarter of every K and V^T tile.
  using KCopy = ContigTileCopy<C::kKRowBytes, C::kCopies>;
  using VCopy = ContigTileCopy<C::kVRowBytes, C::kCopies>;
  uint32_t klo[KCopy::P], vlo[VCopy::P];
  KCopy::lane_offsets(lane, klo);
  VCopy::lane_offsets(lane, vlo);
  // One buffer resource per head for each of K and V^T; a tile's offset
  // goes to the copies' scalar offset.
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(kh), 0, n_tiles * C::kTileBytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(vh), 0, n_tiles * C::kTileBytes, kBufferWord3);
  auto copy_k = [&](int32_t kt) {
    const KCopy ck(krsrc, max(kt, 0) * C::kTileBytes, ks, klo, qw);
    static_for<C::kCopies>([&](auto u) { ck.template issue<decltype(u)::value>(); });
  };

  // LDS element offsets of this lane's operand chunks.
  //   K (A of S^T): row kb*32 + sigma(li), chunk 2m + g.
  //   V^T (A of O^T): row db*32 + li, chunk 4kb + 2h + g.
  const int krow0 = sigma(li);
  const int kswz = swz_rows<C::kKRowBytes>(krow0);  // kb*32 does not change it
  const int vswz = swz_rows<C::kVRowBytes>(li);     // nor does db*32

  // Instruction order of one block of 32 operand reads and 32 MFMAs: the
  // reads run kAhead MFMAs ahead of their use, so LDS latency is covered
  // inside the wave (the other wave on the SIMD is in its VALU phase).
  constexpr int kAhead = 8;
  constexpr int kBlockMfma = BS / 32 * D / 16;   // 32 for D = 128
  auto pipeline_reads = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);        // DS reads
#pragma unroll
    for (int j = 0; j < kBlockMfma - kAhead; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };

  // MFMA phase of step i: PV of step i - 1 if pv, scores of step i if sc.
  // The wave in its MFMA phase takes issue priority over the softmax wave on
  // its SIMD, so that the matrix core is fed first when both have an
  // instruction ready.
  auto mfma_phase = [&](bool pv, bool sc) {
    __builtin_amdgcn_s_setprio(3);
    // The lane parts of the operand addresses pass through an empty asm at
    // each phase, so the swizzled addresses are derived here (a few VALU
    // instructions beside the MFMAs) instead of all being held in registers
    // across the softmax.  Chunk c of a row sits at chunk c ^ swz(row); for
    // even c0, (c0 + g) ^ swz = c0 ^ (g ^ swz).
    int vlane = li * C::kVRowBytes, vx = (g ^ vswz) * 16;
    int klane = krow0 * C::kKRowBytes, kx = (g ^ kswz) * 16;
    asm volatile("" : "+v"(vlane), "+v"(vx), "+v"(klane), "+v"(kx));
    const char* const vs = reinterpret_cast<const char*>(vsg) + vlane;
    const char* const kq = reinterpret_cast<const char*>(ks) + klane;
    if (pv) {
      // O^T[db] += V^T[db rows, keys] P^T(i-1); MFMA (kb, h) takes keys
      // kb*32 + 16h + 8g .. +8 in lane group g.
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const char* va = vs + db * 32 * C::kVRowBytes;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *reinterpret_cast<const bf16x8*>(va + (((4 * kb + 2 * h) * 16) ^ vx)),
                pb[kb][h], o[db], 0, 0, 0);
        }
      }
      pipeline_reads();
    }
    // P(i-1) dies with the PV above before the scores of tile i are born.
    __builtin_amdgcn_sched_barrier(0);
    if (sc) {
      // S^T blocks: s[kb] covers keys kb*32 .. +32 x the wave's 32 queries.
      // MFMA row x of block kb is fed K row kb*32 + sigma(x), so
      // accumulator register r = 4a + b of lane group g holds key
      //   kb*32 + 16(a/2) + 8g + 4(a%2) + b,
      // and the 8 keys behind registers 8h .. 8h+7 are contiguous
      // (kb*32 + 16h + 8g .. +8): the P^T operand of the next PV.
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb) {
        s[kb] = f32x16{};
        const char* ka = kq + kb * 32 * C::kKRowBytes;
#pragma unroll
        for (int m = 0; m < D / 16; ++m)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(ka + ((2 * m * 16) ^ kx)), qf[m],
              s[kb], 0, 0, 0);
      }
      pipeline_reads();
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Per-tile scalars of this group's walk, carried in SGPRs: the kept tiles
  // of steps i and i + 1 and the validity words of step i.  Each VALU phase
  // loads those of the next step early on, so that the phase after it
  // starts without waiting on scalar memory.  A tile is full when its four
  // validity words are all ones.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const __attribute__((address_space(4))) u32x4* tbits4 =
      (const __attribute__((address_space(4))) u32x4*)tile_bits;
  int32_t kt_cur = tile_of(0), kt_nxt = tile_of(1);
  u32x4 bits_cur = tbits4[max(kt_cur, 0)];

  // VALU phase of tile i: the copies of K(i+1) and V^T(i) (their buffers
  // were last read in the MFMA phase just finished) and softmax(i).
  auto valu_phase = [&](int32_t i) {
    const int32_t kt = kt_cur;
    // K(i+1) is copied on the last step too (tile 0 then, never read): a
    // branch around each copy costs more issue cycles than the copy.
    const KCopy ck(krsrc, (i + 1 < n_own ? max(kt_nxt, 0) : 0) * C::kTileBytes, ks, klo, qw);
    const VCopy cv(vrsrc, max(kt, 0) * C::kTileBytes, vsg, vlo, qw);
    static_assert(C::kCopies == 4 || C::kCopies == 8, "copy schedule below");
    // Copy slot S of 8, each followed by a barrier to the scheduler so that
    // the slots stay spread through the softmax (a wave stalls at a copy
    // while the memory pipeline is full, so a burst would hold back the
    // arithmetic behind it).  Slots take two copies each in the order K 0-3,
    // V^T 0-3, K 4-7, V^T 4-7, so that the LDS base changes once per four
    // copies.
    auto copies = [&](auto slot) {
      constexpr int S = decltype(slot)::value;
      constexpr int U = (S / 4) * 4 + (S % 2) * 2;
      if constexpr (U < C::kCopies) {
        if constexpr (S % 4 < 2) {
          ck.template issue<U>();
          ck.template issue<U + 1>();
        } else {
          cv.template issue<U>();
          cv.template issue<U + 1>();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    poison_share<C::kCopies>(ks, qw, lane);
    poison_share<C::kCopies>(vsg, qw, lane);
    copies(I0{});
    // The next step's scalars (in flight during the softmax).
    const int32_t kt_n2 = tile_of(i + 2);
    const u32x4 bits_n = tbits4[max(kt_nxt, 0)];
    const u32x4 bits = kt >= 0 ? bits_cur : u32x4{0u, 0u, 0u, 0u};
    const bool partial = (bits.x & bits.y & bits.z & bits.w) != 0xFFFFFFFFu;
    // Row max over the tile (raw dot products; the scale is positive).
    auto row_max = [&]() {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BS / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[kb][r]);
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(m),
                                                       __float_as_uint(m), false, false);
      return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));   // max with lane ^ 32
    };
    float mx = row_max();
    copies(I1{});
    // Pad keys have all-zero K rows, so they score exactly 0, and all-zero
    // V^T columns, so their weights add nothing to O.  When every query's
    // tile maximum is positive it comes from a valid key and a pad weight
    // 2^(0 - m) stays within 2^8: the pads are left unmasked and their
    // weights are taken out of the row sum afterwards.  Otherwise (and for a
    // masked tile, kt < 0, whose copies hold tile 0) they are set to -inf.
    bool pads_in_sum = false;
    if (partial) {
      if (kt < 0 || __ballot(!(mx > 0.f)) != 0) {
        // Keys of lane group g sit at bit 8g + (16(a/2) + 4(a%2) + b).
#pragma unroll
        for (int kb = 0; kb < BS / 32; ++kb) {
          const uint32_t word = kb == 0 ? bits.x : kb == 1 ? bits.y : kb == 2 ? bits.z : bits.w;
          const uint32_t bits = word >> (8 * g);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int a = r / 4, b = r % 4;
            if (!((bits >> (16 * (a / 2) + 4 * (a % 2) + b)) & 1u)) s[kb][r] = -INFINITY;
          }
        }
        mx = row_max();
      } else {
        pads_in_sum = true;
      }
    }
    // Lazy rescaling: the running max only moves (and O, l are rescaled)
    // when some query's tile max exceeds it by more than 8 in log2 units;
    // otherwise weights stay below 2^8 relative to the stale max, which
    // fp32 accumulation and bf16 P absorb, and the final 1/l uses the same
    // reference.  While no valid key has been seen the max stays -inf.
    const float mt = mx * scale_log2;
    if (__ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    // Row sum of the fp32 weights by plain adds, a tree per eight (a chain
    // of dot-product instructions over the bf16 weights is several times
    // slower while the other wave of the SIMD issues MFMAs).
    float lsum = l_run;
    auto weights = [&](auto kbh) {
      constexpr int kb = decltype(kbh)::value / 2, h = decltype(kbh)::value % 2;
      f32x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * h + e], scale_log2, neg_m));
      pb[kb][h] = __builtin_convertvector(p, bf16x8);
      lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // Pure arithmetic may otherwise be moved across the copies: the empty
      // asm (ordered with them) needs this block's weights done.
      asm volatile("" : "+v"(lsum));
    };
    static_assert(BS / 32 * 2 == 8, "weight blocks below");
    // The remaining copy pairs go out between the first weight blocks.
    using std::integral_constant;
    weights(integral_constant<int, 0>{});
    copies(integral_constant<int, 2>{});
    weights(integral_constant<int, 1>{});
    copies(integral_constant<int, 3>{});
    weights(integral_constant<int, 2>{});
    copies(integral_constant<int, 4>{});
    weights(integral_constant<int, 3>{});
    copies(integral_constant<int, 5>{});
    weights(integral_constant<int, 4>{});
    copies(integral_constant<int, 6>{});
    weights(integral_constant<int, 5>{});
    copies(integral_constant<int, 7>{});
    weights(integral_constant<int, 6>{});
    weights(integral_constant<int, 7>{});
    if (pads_in_sum) {
      // Each pad key of this lane's half of the tile (bits 8g + {0..7,
      // 16..23} of each validity word) scored exactly 0 and so got the
      // weight 2^(0 - m).
      const uint32_t half = g ? 0xFF00FF00u : 0x00FF00FFu;
      const uint32_t npad = __popc(~bits.x & half) + __popc(~bits.y & half) +
                            __popc(~bits.z & half) + __popc(~bits.w & half);
      lsum -= float(npad) * __builtin_amdgcn_exp2f(neg_m);
    }
    l_run = lsum;
    // The wait stays after the softmax, which it would otherwise precede.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the copies have landed
    // The next step's scalars have arrived too (forced here, before the
    // barrier, so that no scalar load is in flight during the MFMA phase,
    // where it would coarsen the LDS waits).
    asm volatile("" ::"s"(kt_n2), "s"(bits_n.x), "s"(bits_n.y), "s"(bits_n.z),
                 "s"(bits_n.w));
    kt_cur = kt_nxt;
    kt_nxt = kt_n2;
    bits_cur = bits_n;
  };

  if (n_own > 0) {
    poison_share<C::kCopies>(ks, qw, lane);
    copy_k(kt_cur);
  }
  // Every scalar the loop reads is resident before it starts: a scalar load
  // still pending at the loop entry would make the compiler wait on all LDS
  // reads at once (lgkmcnt(0)) at the start of each MFMA phase.
  asm volatile("" ::"s"(kt_nxt), "s"(bits_cur.x), "s"(bits_cur.y), "s"(bits_cur.z),
               "s"(bits_cur.w), "s"(scale_log2), "s"(n_grp), "s"(n_own), "s"(row_len));
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __builtin_amdgcn_s_barrier();
  // Phase pairs i = 0 .. n_grp: group 0 runs MFMA(i) then VALU(i); group 1
  // runs VALU(i-1) then MFMA(i).  MFMA(i) takes the PV of step i - 1 and the
  // scores of step i where those steps are the group's own (i - 1 < n_own,
  // i < n_own), and VALU(i) runs for i < n_own (n_own is n_grp for group 0).
  // Both groups take the same number of barriers.  One loop per group, so
  // that each loop carries either P or the scores, not both.
  if (grp == 0) {
    for (int32_t i = 0; i <= n_grp; ++i) {
      mfma_phase(i >= 1, i < n_grp);
      __builtin_amdgcn_s_barrier();
      if (i < n_grp) valu_phase(i);
      __builtin_amdgcn_s_barrier();
    }
  } else {
    for (int32_t i = 0; i <= n_grp; ++i) {
      const bool own_prev = i >= 1 && i - 1 < n_own;
      if (own_prev) valu_phase(i - 1);
      __builtin_amdgcn_s_barrier();
      mfma_phase(own_prev, i < n_own);
      __builtin_amdgcn_s_barrier();
    }
  }

  // Merge: group 1 publishes O (register quads, lane-contiguous), m and l;
  // group 0 combines them with its own and stores.
  float4* ob = reinterpret_cast<float4*>(lds);
  constexpr int kQuads = D / 32 * 4;
  constexpr int kMergeBytes = C::kGroupWaves * kQuads * 64 * 16;
  static_assert(kMergeBytes + 2 * C::kGroupWaves * 64 * 4 <= 4 * C::kTileBytes, "merge space");
  float* const m_buf = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + kMergeBytes);
  float* const l_buf = m_buf + C::kGroupWaves * 64;
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
  const float l_own = l_run * fa + l_b * fb;
  const float l_tot = l_own + __shfl_xor(l_own, 32);
  const int qs = qw * 32 + li;
  const bool qvalid = (tile_bits[qtile * 4 + qs / 32] >> (qs % 32)) & 1u;
  const float inv = (qvalid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const float ca = fa * inv, cb = fb * inv;
  const int64_t iorow = io_row(io, qrow);
  if (iorow < 0) return;                      // pad slot of a raster output
  if (lse != nullptr && g == 0) lse[bh * io.rows + iorow] = lse_of(m_t, l_tot, qvalid);
  // Lane (li, g) holds O^T[dd = db*32 + 8a + 4g + b][query li].
  __bf16* dst = op + (bh * io.rows + iorow) * D + 4 * g;
  typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float4 x = ob[((qw * kQuads + db * 4 + a) * 64) + lane];
      const f32x4 f = {o[db][4 * a] * ca + x.x * cb, o[db][4 * a + 1] * ca + x.y * cb,
                       o[db][4 * a + 2] * ca + x.z * cb, o[db][4 * a + 3] * ca + x.w * cb};
      *reinterpret_cast<bf16x4*>(dst + db * 32 + 8 * a) = __builtin_convertvector(f, bf16x4);
    }
  }
}

// ---------------------------------------------------------------- fp32

template <int D, int BS>
__global__ __launch_bounds__(BS) void attn_f32_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp,
    const float* __restrict__ vt, const int32_t* __restrict__ kept,
    float* __restrict__ op, float* __restrict__ lse, RowIo io,
    const uint32_t* __restrict__ tile_bits,
    const int32_t* __restrict__ tile_count, int64_t Lt, int32_t BH,
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
  const float* kh = kp + bh * Lt * D;
  const float* vh = vt + bh * int64_t(n_tiles) * D * BS;
  const rf::RowRef rr = rf::row_ref(kept + bh * nnz, qtile, nb, row_len_video, n_tiles);
  const int32_t* row = kept + bh * nnz + rr.offset;
  const int32_t row_len = rr.len;

  const int64_t iorow = io_row(io, qrow);
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = iorow >= 0 ? qp[(bh * io.rows + iorow) * D + c] : 0.f;
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
        ks[r][cc] = kh[slot * D + cc];
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
  const bool qvalid = (tile_bits[qtile * 4 + t / 32] >> (t % 32)) & 1u;
  const float inv = (qvalid && l_run > 0.f) ? 1.f / l_run : 0.f;
  if (iorow < 0) return;                      // pad slot of a raster output
  if (lse != nullptr)
    lse[bh * io.rows + iorow] = (qvalid && l_run > 0.f) ? m_run + logf(l_run) : -INFINITY;
  float* dst = op + (bh * io.rows + iorow) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) dst[c] = o[c] * inv;
}

template <int D, int BS>
void launch_bf16(const rf_plan* p, const void* qp, const void* kp,
                 const void* vt, const int32_t* kept, void* op, float* lse, RowIo io,
                 int BH, int32_t row_len_video, int64_t nnz, float scale, hipStream_t st) {
  const int nb = p->sz.nb, n_tt = p->sz.n_text_tiles;
  dim3 grid(BH * (nb + n_tt));
  if constexpr (BS == 128) {
    hipLaunchKernelGGL((attn_bf16_pp_kernel<D>), grid, dim3(PpCfg<D>::kThreads), 0, st,
                       static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp),
                       static_cast<const __bf16*>(vt), kept, static_cast<__bf16*>(op), lse, io,
                       p->tile_bits, p->tile_count, p->sz.Lt, BH, nb, n_tt,
                       row_len_video, nnz,
                       scale * 1.4426950408889634f);
    return;
  }
  hipLaunchKernelGGL((attn_bf16_kernel<D, BS>), grid,
                     dim3(Bf16Cfg<D, BS>::kThreads), 0, st,
                     static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp),
                     static_cast<const __bf16*>(vt), kept, static_cast<__bf16*>(op), lse, io,
                     p->tile_bits, p->tile_count, p->sz.Lt, BH, nb, n_tt,
                     row_len_video, nnz,
                     scale * 1.4426950408889634f);
}

template <int D, int BS>
void launch_f32(const rf_plan* p, const void* qp, const void* kp,
                const void* vt, const int32_t* kept, void* op, float* lse, RowIo io,
                int BH, int32_t row_len_video, int64_t nnz, float scale, hipStream_t st) {
  const int nb = p->sz.nb, n_tt = p->sz.n_text_tiles;
  dim3 grid(BH * (nb + n_tt));
  hipLaunchKernelGGL((attn_f32_kernel<D, BS>), grid, dim3(BS), 0, st,
                     static_cast<const float*>(qp), static_cast<const float*>(kp),
                     static_cast<const float*>(vt), kept, static_cast<float*>(op), lse, io,
                     p->tile_bits, p->tile_count, p->sz.Lt, BH, nb, n_tt,
                     row_len_video, nnz, scale);
}

// Shared by both entry points: row_len_video > 0 is the rf_predict_mask
// layout, row_len_video = -width the padded-row layout.
rf_status sparse_attn(const rf_plan* plan, const void* qp, const void* kp,
                      const void* vt, const int32_t* kept_idx,
                      int32_t row_len_video, int64_t nnz, void* op, float* lse, int32_t B,
                      int32_t H, int32_t d, float scale, rf_dtype dtype,
                      hipStream_t stream, const char* fn, bool raster = false) {
  rf_status st = rf::check_call(plan, B, H, d, dtype, fn);
  if (st != RF_OK) return st;
  if (!rf::aligned16(qp) || !rf::aligned16(kp) || !rf::aligned16(vt) ||
      !rf::aligned16(kept_idx) || !rf::aligned16(op))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: null or misaligned buffer", fn);
  if (reinterpret_cast<uintptr_t>(lse) & 3u)
    return rf::fail(RF_ERR_INVALID_ARG, "%s: misaligned lse", fn);
  if (!(scale > 0.f) || !(scale < 1e30f))
    return rf::fail(RF_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  const int BH = B * H;
  if (int64_t(BH) * plan->sz.n_tiles >= (int64_t(1) << 31))
    return rf::fail(RF_ERR_UNSUPPORTED, "%s: too many tiles", fn);
  const int bs = plan->sz.bs;
  const int32_t rl = row_len_video;
  const RowIo io = raster ? RowIo{plan->slot_src, plan->sz.L} : RowIo{nullptr, plan->sz.Lt};
  if (dtype == RF_BF16) {
    if (d == 128 && bs == 128) launch_bf16<128, 128>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
    else if (d == 128 && bs == 64) launch_bf16<128, 64>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
    else if (d == 64 && bs == 128) launch_bf16<64, 128>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
    else launch_bf16<64, 64>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
  } else {
    if (d == 128 && bs == 128) launch_f32<128, 128>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
    else if (d == 128 && bs == 64) launch_f32<128, 64>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
    else if (d == 64 && bs == 128) launch_f32<64, 128>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
    else launch_f32<64, 64>(plan, qp, kp, vt, kept_idx, op, lse, io, BH, rl, nnz, scale, stream);
  }
  return rf::check_launch(fn);
}

}  // namespace

extern "C" rf_status rf_sparse_attn(const rf_plan* plan, const void* qp,
                                    const void* kp, const void* vt,
                                    const int32_t* kept_idx,
                                    int32_t sparsity_pct, void* op,
                                    float* lse_or_null, int32_t B, int32_t H,
                                    int32_t d, float scale, rf_dtype dtype,
                                    hipStream_t stream) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn: null plan");
  rf_keep kc;
  rf_status st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  return sparse_attn(plan, qp, kp, vt, kept_idx, kc.row_len_video, kc.nnz_per_head,
                     op, lse_or_null, B, H, d, scale, dtype, stream, "rf_sparse_attn");
}

extern "C" rf_status rf_sparse_attn_raster(const rf_plan* plan, const void* q,
                                           const void* kp, const void* vt,
                                           const int32_t* kept_idx,
                                           int32_t sparsity_pct, void* o,
                                           float* lse_or_null, int32_t B, int32_t H,
                                           int32_t d, float scale, rf_dtype dtype,
                                           hipStream_t stream) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_raster: null plan");
  rf_keep kc;
  rf_status st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  if (q == o && q != nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_raster: q and o must not overlap");
  return sparse_attn(plan, q, kp, vt, kept_idx, kc.row_len_video, kc.nnz_per_head, o,
                     lse_or_null, B, H, d, scale, dtype, stream, "rf_sparse_attn_raster",
                     true);
}

extern "C" rf_status rf_sparse_attn_rows(const rf_plan* plan, const void* qp,
                                         const void* kp, const void* vt,
                                         const int32_t* kept_rows,
                                         int32_t row_width, void* op,
                                         float* lse_or_null, int32_t B, int32_t H,
                                         int32_t d, float scale, rf_dtype dtype,
                                         hipStream_t stream) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_rows: null plan");
  if (row_width < 1 || row_width > plan->sz.n_tiles)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_sparse_attn_rows: row_width %d outside [1, %d]",
                    row_width, plan->sz.n_tiles);
  return sparse_attn(plan, qp, kp, vt, kept_rows, -row_width,
                     int64_t(plan->sz.n_tiles) * row_width, op, lse_or_null, B, H, d,
                     scale, dtype, stream, "rf_sparse_attn_rows");
}
