// Layout sizes, index tables, keep counts, plans and error reporting.
//
// The tables encode the 3D window permutation of the RainFusion2.0 page
// (Abstract, key insight (2); TL;DR "3D window permutation") and its
// first-frame sink (Abstract, key insight (3)): blocks are taken row-major
// over the block coordinates of the grid padded up to whole windows, tokens
// row-major inside a block; pad slots carry no token.  With the permutation
// off, slots are raster tokens and the last block is padded.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "rf_internal.h"

namespace {

thread_local char g_err[512] = "";

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Geometry {
  int64_t nT, nH, nW;  // window counts per axis (permute mode)
};

rf_status compute_sizes(const rf_layout* lay, rf_sizes* sz, Geometry* g) {
  if (lay == nullptr || sz == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_layout_sizes: null pointer");
  if (lay->T < 1 || lay->H < 1 || lay->W < 1)
    return rf::fail(RF_ERR_INVALID_ARG, "grid %dx%dx%d must be positive",
                    lay->T, lay->H, lay->W);
  if (lay->wt < 1 || lay->wh < 1 || lay->ww < 1)
    return rf::fail(RF_ERR_INVALID_ARG, "window %dx%dx%d must be positive",
                    lay->wt, lay->wh, lay->ww);
  if (lay->n_text < 0)
    return rf::fail(RF_ERR_INVALID_ARG, "n_text %d is negative", lay->n_text);
  if ((lay->permute != 0 && lay->permute != 1) ||
      (lay->sink != 0 && lay->sink != 1))
    return rf::fail(RF_ERR_INVALID_ARG, "permute and sink must be 0 or 1");
  const int64_t bs = int64_t(lay->wt) * lay->wh * lay->ww;
  if (bs != 64 && bs != 128)
    return rf::fail(RF_ERR_UNSUPPORTED,
                    "block size wt*wh*ww = %lld (need 64 or 128)",
                    (long long)bs);
  const int64_t N = int64_t(lay->T) * lay->H * lay->W;
  int64_t nb;
  Geometry geo{0, 0, 0};
  if (lay->permute) {
    geo.nT = ceil_div(lay->T, lay->wt);
    geo.nH = ceil_div(lay->H, lay->wh);
    geo.nW = ceil_div(lay->W, lay->ww);
    nb = geo.nT * geo.nH * geo.nW;
  } else {
    nb = ceil_div(N, bs);
  }
  const int64_t Np = nb * bs;
  const int64_t ntt = ceil_div(lay->n_text, bs);
  const int64_t Lp = Np + lay->n_text;
  if ((nb + ntt) * bs >= (int64_t(1) << 31) - 256 || N >= (int64_t(1) << 31))
    return rf::fail(RF_ERR_INVALID_ARG, "sequence of %lld slots is too long",
                    (long long)Lp);
  sz->N = N;
  sz->Np = Np;
  sz->L = N + lay->n_text;
  sz->Lp = Lp;
  sz->Lt = (nb + ntt) * bs;
  sz->bs = int32_t(bs);
  sz->nb = int32_t(nb);
  sz->n_text_tiles = int32_t(ntt);
  sz->n_tiles = int32_t(nb + ntt);
  if (!lay->sink)
    sz->n_sink = 0;
  else if (lay->permute)
    sz->n_sink = int32_t(geo.nH * geo.nW);  // every block with bt = 0
  else
    sz->n_sink = int32_t(ceil_div(int64_t(lay->H) * lay->W, bs));
  if (g) *g = geo;
  return RF_OK;
}

// Slot of raster token n (video tokens only).
int64_t slot_of(const rf_layout& lay, const rf_sizes& sz, const Geometry& g,
                int64_t n) {
  if (!lay.permute) return n;
  const int64_t w = n % lay.W, h = (n / lay.W) % lay.H, t = n / (int64_t(lay.W) * lay.H);
  const int64_t blk = ((t / lay.wt) * g.nH + h / lay.wh) * g.nW + w / lay.ww;
  const int64_t in = ((t % lay.wt) * lay.wh + h % lay.wh) * lay.ww + w % lay.ww;
  return blk * sz.bs + in;
}

struct HostTables {
  std::vector<int32_t> slot_src, tok_slot, tile_count, tile_rank;
  std::vector<uint32_t> tile_bits;
  std::vector<uint8_t> is_sink;
};

// Position of each video tile when the tiles are sorted by (h, w, t) of
// their first valid token: the spatial-major order in which the temporal
// head pattern of the v1 page (RainFusion review, "What carries the
// argument": temporal heads attend to one local region across frames) is a
// band.  With the window order this is (bh, bw, bt) order.
void build_rank(const rf_layout& lay, const rf_sizes& sz,
                const std::vector<int32_t>& slot_src, std::vector<int32_t>* rank) {
  struct Key { int64_t h, w, t; int32_t tile; };
  std::vector<Key> keys(sz.nb);
  const int64_t hw = int64_t(lay.H) * lay.W;
  for (int32_t i = 0; i < sz.nb; ++i) {
    int64_t n = -1;
    for (int32_t s = 0; s < sz.bs && n < 0; ++s) n = slot_src[int64_t(i) * sz.bs + s];
    keys[i] = {(n % hw) / lay.W, n % lay.W, n / hw, i};
  }
  std::sort(keys.begin(), keys.end(), [](const Key& a, const Key& b) {
    if (a.h != b.h) return a.h < b.h;
    if (a.w != b.w) return a.w < b.w;
    return a.t < b.t;
  });
  rank->assign(sz.nb, 0);
  for (int32_t r = 0; r < sz.nb; ++r) (*rank)[keys[r].tile] = r;
}

void build_tables(const rf_layout& lay, const rf_sizes& sz, const Geometry& g,
                  HostTables* t) {
  t->slot_src.assign(sz.Lt, -1);
  t->tok_slot.assign(sz.L, 0);
  t->tile_count.assign(sz.n_tiles, 0);
  t->tile_bits.assign(size_t(sz.n_tiles) * 4, 0u);
  t->is_sink.assign(sz.nb, 0);
  for (int64_t n = 0; n < sz.N; ++n) {
    const int64_t s = slot_of(lay, sz, g, n);
    t->slot_src[s] = int32_t(n);
    t->tok_slot[n] = int32_t(s);
  }
  for (int64_t j = 0; j < lay.n_text; ++j) {
    t->slot_src[sz.Np + j] = int32_t(sz.N + j);
    t->tok_slot[sz.N + j] = int32_t(sz.Np + j);
  }
  for (int64_t s = 0; s < sz.Lp; ++s) {
    if (t->slot_src[s] < 0) continue;
    const int64_t tile = s / sz.bs, bit = s % sz.bs;
    t->tile_count[tile] += 1;
    t->tile_bits[tile * 4 + bit / 32] |= 1u << (bit % 32);
  }
  if (lay.sink) {
    // Blocks holding a token of frame 0 (raster tokens 0 .. H*W-1).
    for (int64_t n = 0; n < int64_t(lay.H) * lay.W; ++n)
      t->is_sink[t->tok_slot[n] / sz.bs] = 1;
  }
  build_rank(lay, sz, t->slot_src, &t->tile_rank);
}

}  // namespace

namespace rf {

rf_status fail(rf_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rf_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(RF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return RF_OK;
}

rf_status check_call(const rf_plan* plan, int32_t B, int32_t H, int32_t d,
                     rf_dtype dtype, const char* fn) {
  if (plan == nullptr) return fail(RF_ERR_INVALID_ARG, "%s: null plan", fn);
  if (B < 1 || H < 1 || int64_t(B) * H > 65535)
    return fail(RF_ERR_INVALID_ARG, "%s: B=%d H=%d out of range", fn, B, H);
  if (dtype != RF_BF16 && dtype != RF_F32)
    return fail(RF_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dtype));
  if (d != 64 && d != 128)
    return fail(RF_ERR_UNSUPPORTED, "%s: head dim %d (need 64 or 128)", fn, d);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(RF_ERR_INVALID_ARG,
                "%s: current device %d is not the plan's device %d", fn, dev,
                plan->device);
  return RF_OK;
}

}  // namespace rf

extern "C" {

rf_status rf_layout_sizes(const rf_layout* lay, rf_sizes* out) {
  return compute_sizes(lay, out, nullptr);
}

rf_status rf_layout_tables(const rf_layout* lay, int32_t* slot_src,
                           int64_t cap_slot_src, int32_t* tok_slot,
                           int64_t cap_tok_slot, int32_t* tile_count,
                           int64_t cap_tile_count, uint8_t* is_sink,
                           int64_t cap_is_sink) {
  rf_sizes sz;
  Geometry g;
  rf_status st = compute_sizes(lay, &sz, &g);
  if (st != RF_OK) return st;
  if (!slot_src || !tok_slot || !tile_count || !is_sink)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_layout_tables: null buffer");
  if (cap_slot_src < sz.Lt || cap_tok_slot < sz.L ||
      cap_tile_count < sz.n_tiles || cap_is_sink < sz.nb)
    return rf::fail(RF_ERR_BUFFER_TOO_SMALL,
                    "rf_layout_tables: need %lld/%lld/%d/%d elements",
                    (long long)sz.Lt, (long long)sz.L, sz.n_tiles, sz.nb);
  HostTables t;
  build_tables(*lay, sz, g, &t);
  memcpy(slot_src, t.slot_src.data(), sizeof(int32_t) * sz.Lt);
  memcpy(tok_slot, t.tok_slot.data(), sizeof(int32_t) * sz.L);
  memcpy(tile_count, t.tile_count.data(), sizeof(int32_t) * sz.n_tiles);
  memcpy(is_sink, t.is_sink.data(), sz.nb);
  return RF_OK;
}

rf_status rf_layout_keep(const rf_layout* lay, int32_t sparsity_pct,
                         rf_keep* out) {
  rf_sizes sz;
  rf_status st = compute_sizes(lay, &sz, nullptr);
  if (st != RF_OK) return st;
  if (out == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_layout_keep: null output");
  if (sparsity_pct < 0 || sparsity_pct > 99)
    return rf::fail(RF_ERR_INVALID_ARG, "sparsity %d%% outside [0, 99]",
                    sparsity_pct);
  const int64_t k = (int64_t(sz.nb) * (100 - sparsity_pct) + 50) / 100;
  int64_t keff = k > sz.n_sink ? k : sz.n_sink;
  if (keff < 1) keff = 1;
  out->k = int32_t(k);
  out->k_eff = int32_t(keff);
  out->row_len_video = int32_t(keff + sz.n_text_tiles);
  out->row_len_text = sz.n_tiles;
  out->nnz_per_head = int64_t(sz.nb) * out->row_len_video +
                      int64_t(sz.n_text_tiles) * out->row_len_text;
  return RF_OK;
}

rf_status rf_keep_count(const rf_plan* plan, int32_t sparsity_pct, int32_t* k_eff,
                        int64_t* nnz_per_head) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_keep_count: null plan");
  rf_keep kc;
  rf_status st = rf_layout_keep(&plan->lay, sparsity_pct, &kc);
  if (st != RF_OK) return st;
  if (k_eff) *k_eff = kc.k_eff;
  if (nnz_per_head) *nnz_per_head = kc.nnz_per_head;
  return RF_OK;
}

rf_status rf_band_tiles(const rf_layout* lay, double bandwidth, int32_t* band) {
  rf_sizes sz;
  rf_status st = compute_sizes(lay, &sz, nullptr);
  if (st != RF_OK) return st;
  if (band == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_band_tiles: null output");
  if (!(bandwidth >= 0.0 && bandwidth <= 1.0))
    return rf::fail(RF_ERR_INVALID_ARG, "bandwidth %g outside [0, 1]", bandwidth);
  // Half-width of the band in video tiles, rounded to nearest (halves up):
  // the band |i - j| <= w then covers 1 - (1 - b)^2 of the unit square.
  *band = int32_t(std::floor(bandwidth * sz.nb + 0.5));
  return RF_OK;
}

rf_status rf_tile_rank(const rf_layout* lay, int32_t* rank, int64_t cap) {
  rf_sizes sz;
  Geometry g;
  rf_status st = compute_sizes(lay, &sz, &g);
  if (st != RF_OK) return st;
  if (rank == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_tile_rank: null buffer");
  if (cap < sz.nb)
    return rf::fail(RF_ERR_BUFFER_TOO_SMALL, "rf_tile_rank: need %d elements", sz.nb);
  HostTables t;
  build_tables(*lay, sz, g, &t);
  memcpy(rank, t.tile_rank.data(), sizeof(int32_t) * sz.nb);
  return RF_OK;
}

rf_status rf_pattern_row_width(const rf_layout* lay, int32_t band, int32_t tau,
                               int32_t* width) {
  rf_sizes sz;
  rf_status st = compute_sizes(lay, &sz, nullptr);
  if (st != RF_OK) return st;
  if (width == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_pattern_row_width: null output");
  if (band < 0 || tau < 1)
    return rf::fail(RF_ERR_INVALID_ARG, "band %d must be >= 0 and tau %d >= 1", band, tau);
  // Longest video row: a band row keeps at most 2*band + 1 tiles, a
  // checkerboard row at most ceil(nb / tau); text tiles follow.
  const int64_t b = std::min<int64_t>(2 * int64_t(band) + 1, sz.nb);
  const int64_t c = ceil_div(sz.nb, tau);
  int64_t w = std::max(b, c) + sz.n_text_tiles;
  if (sz.n_text_tiles > 0) w = std::max<int64_t>(w, sz.n_tiles);
  *width = int32_t(w);
  return RF_OK;
}

rf_status rf_arm_sample_count(const rf_layout* lay, int32_t local,
                              int32_t stride, int32_t* n) {
  rf_sizes sz;
  rf_status st = compute_sizes(lay, &sz, nullptr);
  if (st != RF_OK) return st;
  if (n == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_arm_sample_count: null output");
  if (stride < 1) return rf::fail(RF_ERR_INVALID_ARG, "ARM stride %d must be >= 1", stride);
  const int64_t limit = local ? int64_t(lay->H) * lay->W : sz.N;
  *n = int32_t(ceil_div(limit, stride));
  return RF_OK;
}

const char* rf_status_str(rf_status s) {
  switch (s) {
    case RF_OK: return "ok";
    case RF_ERR_INVALID_ARG: return "invalid argument";
    case RF_ERR_UNSUPPORTED: return "unsupported";
    case RF_ERR_HIP: return "HIP runtime error";
    case RF_ERR_BUFFER_TOO_SMALL: return "buffer too small";
  }
  return "unknown status";
}

const char* rf_last_error(void) { return g_err; }

void rf_plan_destroy(rf_plan* p) {
  if (p == nullptr) return;
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (cur != p->device) (void)hipSetDevice(p->device);
  (void)hipFree(p->slot_src);
  (void)hipFree(p->tok_slot);
  (void)hipFree(p->tile_bits);
  (void)hipFree(p->tile_count);
  (void)hipFree(p->is_sink);
  (void)hipFree(p->tile_rank);
  if (cur >= 0 && cur != p->device) (void)hipSetDevice(cur);
  delete p;
}

rf_status rf_plan_create(const rf_layout* lay, rf_plan** out) {
  if (out == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_plan_create: null output");
  *out = nullptr;
  rf_sizes sz;
  Geometry g;
  rf_status st = compute_sizes(lay, &sz, &g);
  if (st != RF_OK) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return rf::fail(RF_ERR_HIP, "rf_plan_create: no HIP device (%s)",
                    hipGetErrorString(e));
  st = rf::prepare_mask_kernels();
  if (st != RF_OK) return st;
  HostTables t;
  build_tables(*lay, sz, g, &t);
  rf_plan* p = new rf_plan();
  p->lay = *lay;
  p->sz = sz;
  p->device = dev;
  struct Item { void** dst; const void* src; size_t bytes; };
  Item items[] = {
      {(void**)&p->slot_src, t.slot_src.data(), sizeof(int32_t) * t.slot_src.size()},
      {(void**)&p->tok_slot, t.tok_slot.data(), sizeof(int32_t) * t.tok_slot.size()},
      {(void**)&p->tile_bits, t.tile_bits.data(), sizeof(uint32_t) * t.tile_bits.size()},
      {(void**)&p->tile_count, t.tile_count.data(), sizeof(int32_t) * t.tile_count.size()},
      {(void**)&p->is_sink, t.is_sink.data(), t.is_sink.size()},
      {(void**)&p->tile_rank, t.tile_rank.data(), sizeof(int32_t) * t.tile_rank.size()},
  };
  for (const Item& it : items) {
    e = hipMalloc(it.dst, it.bytes > 0 ? it.bytes : 4);
    if (e == hipSuccess && it.bytes > 0)
      e = hipMemcpy(*it.dst, it.src, it.bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      rf_plan_destroy(p);
      return rf::fail(RF_ERR_HIP, "rf_plan_create: %s", hipGetErrorString(e));
    }
  }
  *out = p;
  return RF_OK;
}

rf_status rf_plan_sizes(const rf_plan* plan, rf_sizes* out) {
  if (plan == nullptr || out == nullptr)
    return rf::fail(RF_ERR_INVALID_ARG, "rf_plan_sizes: null pointer");
  *out = plan->sz;
  return RF_OK;
}

rf_status rf_plan_info(const rf_plan* plan, int64_t* N, int64_t* Np, int32_t* nb,
                       int32_t* bs, int32_t* n_sink, int32_t* n_text_tiles) {
  if (plan == nullptr) return rf::fail(RF_ERR_INVALID_ARG, "rf_plan_info: null plan");
  if (N) *N = plan->sz.N;
  if (Np) *Np = plan->sz.Np;
  if (nb) *nb = plan->sz.nb;
  if (bs) *bs = plan->sz.bs;
  if (n_sink) *n_sink = plan->sz.n_sink;
  if (n_text_tiles) *n_text_tiles = plan->sz.n_text_tiles;
  return RF_OK;
}

}  // extern "C"
