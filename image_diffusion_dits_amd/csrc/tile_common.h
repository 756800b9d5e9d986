// Helpers shared by the attention kernels: the XCD-aware numbering of
// (head, query tile) jobs, the XOR swizzle of LDS tile rows and the
// global -> LDS tile copies through buffer resources.
#pragma once

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

// Word 3 of a raw buffer resource (untyped dword access) on gfx9-family
// GPUs.
constexpr int kBufferWord3 = 0x00020000;

// Copies one tile of `bytes` bytes at `base` into LDS at `dst` through a
// buffer resource spanning exactly the tile: copy u of group wave w writes
// LDS [dst + (u*WAVES + w) * 1024, +1024) from lane offset voff + u * the
// bytes one copy covers.  The wave's offset passes through an empty asm so
// that the compiler recomputes the LDS addresses at each call instead of
// keeping every one of them in a scalar register across the loop (which
// spilled them to VGPR lanes).
template <int COPIES, int WAVES>
__device__ __forceinline__ void dma_tile(const char* base, int bytes, void* dst,
                                         uint32_t voff, int w) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kBufferWord3);
  constexpr int kStride = WAVES * 64 * 16;
  int woff = w * 1024;
  asm volatile("" : "+s"(woff));
#pragma unroll
  for (int u = 0; u < COPIES; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (lds_void*)(static_cast<char*>(dst) + woff + u * WAVES * 1024), 16, voff,
        u * kStride, 0, 0);
}

// The copies of dma_tile issued one at a time, so that a caller can spread
// them between other instructions: a wave stalls at a tile copy while the
// memory pipeline is still taking the previous ones, so a burst of copies
// holds back the arithmetic queued behind it.
template <int WAVES>
struct TileCopy {
  __amdgpu_buffer_rsrc_t rsrc;
  char* dst;
  uint32_t voff;
  __device__ __forceinline__ TileCopy(const char* base, int bytes, void* lds, uint32_t v, int w)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kBufferWord3)),
        voff(v) {
    int woff = w * 1024;
    asm volatile("" : "+s"(woff));
    dst = static_cast<char*>(lds) + woff;
  }
  // Copy u: LDS [dst + u*WAVES*1024, +1024) from lane offset voff + u * the
  // bytes one copy covers, as in dma_tile.
  template <int U>
  __device__ __forceinline__ void issue() const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + U * WAVES * 1024), 16,
                                             voff, U * WAVES * 64 * 16, 0, 0);
  }
};

// As dma_tile, with copy u reading from lane offset voff + soff[u]: for
// tiles whose LDS rows are a permutation of the global rows.
template <int COPIES, int WAVES>
__device__ __forceinline__ void dma_tile_perm(const char* base, int bytes, void* dst,
                                              uint32_t voff, int w,
                                              const uint32_t (&soff)[COPIES]) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kBufferWord3);
  int woff = w * 1024;
  asm volatile("" : "+s"(woff));
#pragma unroll
  for (int u = 0; u < COPIES; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (lds_void*)(static_cast<char*>(dst) + woff + u * WAVES * 1024), 16, voff,
        soff[u], 0, 0);
}

// Natural-log softmax normaliser of one query from the reference maximum m
// (log2 units of the scaled logits) and the weight sum l taken relative to
// it: ln sum_j exp(logit_j) = (m + log2 l) ln 2.  -inf for a pad query or a
// query that saw no valid key.
__device__ inline float lse_of(float m, float l, bool valid) {
  return (valid && l > 0.f) ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace rf_tile
