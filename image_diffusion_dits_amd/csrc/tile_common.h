// Helpers shared by the attention kernels: the XCD-aware numbering of
// (head, query tile) jobs, the XOR swizzle of LDS tile rows and the
// global -> LDS tile copies through buffer resources.
#pragma once

#include <type_traits>

#include "rf_internal.h"

namespace rf_tile {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;

struct TileJob {
  int64_t bh;
  int32_t tile;
};

// Workgroup id -> (b*H + h, query tile).  Text query tiles of all heads come
// first.  Video tiles, in (head, tile) order, are dealt in segments of
// kXcds * kXcdWindow: XCD x (ids congruent to x mod 8) takes the x-th run of
// kXcdWindow consecutive tiles of each segment.  The workgroups an XCD runs
// at once then work on neighbouring tiles, which share many kept K/V tiles
// through its L2, and all XCDs stay on the same head at a time, so the K/V
// tiles they stream stay within the memory-side cache.  A final partial
// segment is taken in id order.
constexpr int kXcdWindow = 32;

__device__ inline TileJob job_of(int32_t pid, int32_t BH, int32_t nb,
                                 int32_t n_tt) {
  const int32_t n_text_jobs = BH * n_tt;
  if (pid < n_text_jobs) return {pid / n_tt, nb + pid % n_tt};
  const int32_t p = pid - n_text_jobs;
  constexpr int32_t kSeg = kXcds * kXcdWindow;
  const int32_t full = (BH * nb) / kSeg * kSeg;
  int32_t logical = p;
  if (p < full) {
    const int32_t x = p % kXcds, idx = p / kXcds;
    logical = (idx / kXcdWindow) * kSeg + x * kXcdWindow + idx % kXcdWindow;
  }
  return {logical / nb, logical % nb};
}

// XOR swizzle of the 16-byte chunks of LDS rows of RB bytes: the 16 rows
// read by one ds_read_b128 phase (one chunk column of 16 consecutive rows,
// or the sigma image of them) land on 16 distinct bank groups.
template <int RB>
__device__ inline int swz_rows(int r) {
  return (r / (256 / RB)) % (RB / 16);
}

// Byte offset, inside a tile with LDS rows of RB bytes (global rows GROW
// bytes apart), of the 16-byte chunk that lane `lane` of group wave `w`
// moves in copy 0: the copy writes LDS bytes [w * 1024, +1024), so lane l
// lands on LDS chunk q = w*64 + l: row q / (RB/16), position q % (RB/16),
// which holds global chunk position ^ swizzle.  Copy u moves the rows
// u * WAVES * 64 / (RB/16) further on, a multiple of 16, so the swizzle and
// the lane offset are the same for every copy.
template <int RB, int GROW, int WAVES>
__device__ inline uint32_t dma_offset(int w, int lane) {
  constexpr int cpr = RB / 16;
  static_assert((WAVES * 64 / cpr) % 16 == 0, "copy-invariant swizzle");
  const int q = w * 64 + lane;
  const int r = q / cpr, pc = q % cpr;
  return uint32_t(r * GROW + (pc ^ swz_rows<RB>(r)) * 16);
}

// Calls f(std::integral_constant<int, u>) for u = U .. N-1, in order.
template <int N, int U = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (U < N) {
    f(std::integral_constant<int, U>{});
    static_for<N, U + 1>(f);
  }
}

// Word 3 of a raw buffer resource (untyped dword access) on gfx9-family
// GPUs.
constexpr int kBufferWord3 = 0x00020000;

// Copies one tile into LDS at `dst`: the tile at byte offset tile_off of the
// buffer rsrc covers.  Copy u of group wave w writes
// LDS [dst + (u*WAVES + w) * 1024, +1024) from lane offset voff + u * the
// bytes one copy covers.  The wave's offset passes through an empty asm so
// that the compiler recomputes the LDS addresses at each call instead of
// keeping every one of them in a scalar register across the loop (which
// spilled them to VGPR lanes).
template <int COPIES, int WAVES>
__device__ __forceinline__ void dma_tile_at(__amdgpu_buffer_rsrc_t rsrc, int tile_off,
                                            void* dst, uint32_t voff, int w) {
  constexpr int kStride = WAVES * 64 * 16;
  int woff = w * 1024;
  asm volatile("" : "+s"(woff));
#pragma unroll
  for (int u = 0; u < COPIES; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (lds_void*)(static_cast<char*>(dst) + woff + u * WAVES * 1024), 16, voff,
        tile_off + u * kStride, 0, 0);
}

// Tile copies issued one at a time, so that a caller can spread them
// between other instructions, with each group wave taking a contiguous
// share of the tile: copy u of wave w writes LDS [dst + (w*COPIES + u)*1024,
// +1024), the same LDS layout as dma_tile_at (row r at r * RB, its 16-byte
// chunks swizzled by swz_rows), from the matching global bytes.  The
// swizzle repeats every 16 rows, i.e. every P = RB / 64 copies, so the lane
// offsets are P registers (lane_offsets).  A copy's instruction offset moves
// its LDS and global addresses alike, by up to 3 KB, so four consecutive
// copies share one LDS base (one write of M0 instead of four): copy u takes
// base (u & ~3) KB into the wave's share and offset (u & 3) KB.
template <int RB, int COPIES>
struct ContigTileCopy {
  static constexpr int P = RB / 64;
  static_assert(P >= 1 && P <= 4 && COPIES % 4 == 0 && COPIES % P == 0,
                "a wave's share starts on a swizzle period");
  __amdgpu_buffer_rsrc_t rsrc;
  char* dst;           // LDS start of the wave's share
  int soff;            // byte offset of the wave's share in the tile
  uint32_t voff[P];
  // The tile at byte offset tile_off of the buffer r covers (e.g. one head's
  // tiles): the offset goes to the scalar offset, so the resource stays the
  // same for every tile.
  __device__ __forceinline__ ContigTileCopy(__amdgpu_buffer_rsrc_t r, int tile_off, void* lds,
                                            const uint32_t (&v)[P], int w)
      : rsrc(r) {
#pragma unroll
    for (int j = 0; j < P; ++j) voff[j] = v[j];
    int woff = w * COPIES * 1024;
    asm volatile("" : "+s"(woff));
    dst = static_cast<char*>(lds) + woff;
    soff = tile_off + woff;
  }
  // Lane offsets within a 1 KB copy for the P swizzle phases: lane l moves
  // chunk l % (RB/16) of row l / (RB/16) of the piece, whose first row is
  // 1024/RB * j modulo the 16-row period.
  __device__ static void lane_offsets(int lane, uint32_t (&v)[P]) {
    constexpr int cpr = RB / 16;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int r = j * (1024 / RB) + lane / cpr;
      v[j] = uint32_t((lane / cpr) * RB + ((lane % cpr) ^ swz_rows<RB>(r)) * 16);
    }
  }
  template <int U>
  __device__ __forceinline__ void issue() const {
    static_assert(U >= 0 && U < COPIES, "copy index");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (U & ~3) * 1024), 16,
                                             voff[U % P], soff + (U & ~3) * 1024,
                                             (U & 3) * 1024, 0);
  }
};

// As dma_tile_at, with copy u reading from lane offset voff + soff[u]: for
// tiles whose LDS rows are a permutation of the global rows.
template <int COPIES, int WAVES>
__device__ __forceinline__ void dma_tile_perm_at(__amdgpu_buffer_rsrc_t rsrc, int tile_off,
                                                 void* dst, uint32_t voff, int w,
                                                 const uint32_t (&soff)[COPIES]) {
  int woff = w * 1024;
  asm volatile("" : "+s"(woff));
#pragma unroll
  for (int u = 0; u < COPIES; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (lds_void*)(static_cast<char*>(dst) + woff + u * WAVES * 1024), 16, voff,
        tile_off + soff[u], 0, 0);
}

// Debug build (-DRF_POISON_LDS): before a wave's tile copy lands, the LDS
// bytes that copy will overwrite (copy u of group wave w writes
// [dst + (u*WAVES + w) * 1024, +1024)) are filled with 0x7fff halves, a NaN
// as bf16 and NaN bytes as e4m3, and the fill is waited for, so it is in
// LDS before the copy is issued.  An operand read that is not ordered after
// its copy then returns NaN instead of stale numbers and fails parity.  In
// the normal build this does nothing.
template <int COPIES, int WAVES>
__device__ __forceinline__ void poison_tile(void* dst, int w, int lane) {
#ifdef RF_POISON_LDS
  const uint4 nan = make_uint4(0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu);
  char* d = static_cast<char*>(dst) + w * 1024 + lane * 16;
#pragma unroll
  for (int u = 0; u < COPIES; ++u)
    *reinterpret_cast<uint4*>(d + u * WAVES * 1024) = nan;
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the fill is in LDS
#else
  (void)dst; (void)w; (void)lane;
#endif
}

// poison_tile for the copies of ContigTileCopy: wave w's copy u writes
// [dst + (w*COPIES + u) * 1024, +1024).
template <int COPIES>
__device__ __forceinline__ void poison_share(void* dst, int w, int lane) {
#ifdef RF_POISON_LDS
  const uint4 nan = make_uint4(0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu);
  char* d = static_cast<char*>(dst) + w * COPIES * 1024 + lane * 16;
#pragma unroll
  for (int u = 0; u < COPIES; ++u)
    *reinterpret_cast<uint4*>(d + u * 1024) = nan;
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the fill is in LDS
#else
  (void)dst; (void)w; (void)lane;
#endif
}

// Natural-log softmax normaliser of one query from the reference maximum m
// (log2 units of the scaled logits) and the weight sum l taken relative to
// it: ln sum_j exp(logit_j) = (m + log2 l) ln 2.  -inf for a pad query or a
// query that saw no valid key.
__device__ inline float lse_of(float m, float l, bool valid) {
  return (valid && l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace rf_tile
