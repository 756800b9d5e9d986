"""Plain fp64 CPU oracle for RainFusion2.0's online block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library or its Python binding, and imports nothing from them.

Sources (cited by page title and section; no line numbers):
  [RF2]  "RainFusion2.0: Temporal-Spatial Awareness and Hardware-Efficient
         Block-wise Sparse Attention" (arXiv 2512.24086): Abstract, key
         insights (1) block-wise mean values as representative tokens for
         sparse mask prediction, (2) spatiotemporal-aware token permutation,
         (3) first-frame sink; TL;DR ("3D window permutation"); Figure 3
         caption (80% sparsity with and without the 3D permutation).
  [RF1]  "RainFusion: Adaptive Video Generation Acceleration via
         Multi-Dimensional Visual Redundancy" (arXiv 2505.21036): Abstract;
         the pith.science review's "Assumptions" list (softmax attention,
         Eq. (1)) and "What carries the argument" (masked recall R').

The pages give no formula for the mask rule, the permutation order or the
kernel.  Where they are silent this module takes the readings listed here;
each function restates the one it uses.
  R1  Window order: blocks in row-major order of (bt, bh, bw), tokens inside
      a block in row-major order of (dt, dh, dw); the grid is padded up to a
      multiple of the window along each axis; pad slots hold zeros.
  R2  Raster mode (permutation off): slot = raster token index; blocks are
      runs of bs consecutive tokens; the last block is padded.
  R3  Representative token of a block = arithmetic mean over its valid
      (non-pad) tokens, per batch and head.
  R4  Block score l_ij = Qbar_i . Kbar_j / sqrt(d); P = row softmax of l over
      video key blocks.  Ranking by l equals ranking by P.
  R5  Keep rule per video query-block row: n = video key blocks,
      k = floor((n (100 - s) + 50) / 100), S = first-frame sink blocks,
      k_eff = max(k, |S|, 1); kept = S plus the k_eff - |S| highest-scoring
      non-sink blocks, ties to the lower block index.
  R6  First frame = latent frame 0; sink = every key block holding a frame-0
      token (only when the sink is switched on).
  R7  Text tokens follow the video tokens, form ceil(n_text / bs) tiles, are
      not pooled, are appended to every video row's kept list, and text
      query tiles attend to every tile.
  R8  Attention: o = sum_j softmax_j(q . k_j / sqrt(d)) v_j over the valid
      tokens of the row's kept tiles; pad query rows are 0.
  R9  Attention recall (RF1 review, "What carries the argument": the masked
      recall R' = S(Q', K', M') / S(Q', K', M_init), the attention mass that
      survives a mask over the mass with no mask): for one query token,
      R = sum of exp(q . k_j / sqrt(d)) over the valid tokens of its row's
      kept tiles, divided by the same sum over every valid token of the
      sequence.  Computed on chosen query tiles; pad query slots are NaN.
  R10 v1 head patterns as tile masks (RF1 review, "What carries the
      argument", "Core claim" and the free-parameter list: striped bands for
      spatial and temporal heads, bandwidth 1/4 giving a 9/16 cut; the
      checkerboard C = {a_ij : i mod tau = k and j mod tau = k}, tau = 2).
      Tiles play the role of tokens.  Band half-width w = floor(b nb + 1/2)
      video tiles for bandwidth b, so the kept area of the band on the unit
      square is 1 - (1 - b)^2 (7/16 at b = 1/4).  Spatial: video query tile i
      keeps video tile j when |i - j| <= w, tiles in frame-major order (the
      block index).  Temporal: |r(i) - r(j)| <= w with r the rank of a tile
      in spatial-major order, i.e. tiles sorted by (h, w, t) of their first
      valid token.  Textural: j = i (mod tau).  Text tiles are appended to
      every video row and text query rows keep every tile (R7).
  R11 ARM, the v1 online classifier (RF1 review, "What carries the argument"
      and "Core claim"): the local sample is every omega_l-th raster token of
      frame 0, the global sample every omega_g-th raster token of the video;
      queries and keys are the same sampled tokens.  Per sampled query the
      recall is R' of R9 restricted to the sampled keys, with the candidate
      mask evaluated on the tiles that hold the two tokens: the temporal mask
      on the local sample (bR), the spatial mask on the global sample (eR).
      A head's recall is the mean over its sample.  Class: temporal if
      bR >= alpha, else spatial if eR >= alpha, else textural.  The pages give
      neither alpha nor omega; alpha = 0.9 follows the 90% recall target of
      the v1 page's RainFusion+ variant, and the strides are parameters.
"""
import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Layout:
    """Latent grid (T frames of H x W tokens), window, text and switches."""
    T: int
    H: int
    W: int
    wt: int
    wh: int
    ww: int
    n_text: int = 0
    permute: int = 1
    sink: int = 0


def _ceil_div(a, b):
    return -(-a // b)


def sizes(lay: Layout) -> dict:
    """Derived sizes of a layout.  [RF2 TL;DR, 3D window permutation] with
    readings R1 (padding to whole windows), R2 (raster blocks) and R7."""
    bs = lay.wt * lay.wh * lay.ww
    N = lay.T * lay.H * lay.W
    if lay.permute:
        nT, nH, nW = (_ceil_div(lay.T, lay.wt), _ceil_div(lay.H, lay.wh),
                      _ceil_div(lay.W, lay.ww))
        Np = nT * nH * nW * bs
        nb = nT * nH * nW
    else:
        nT = nH = nW = 0
        nb = _ceil_div(N, bs)
        Np = nb * bs
    n_tt = _ceil_div(lay.n_text, bs)
    return dict(bs=bs, N=N, Np=Np, nb=nb, nT=nT, nH=nH, nW=nW,
                n_text=lay.n_text, n_text_tiles=n_tt, n_tiles=nb + n_tt,
                L=N + lay.n_text, Lp=Np + lay.n_text)


def slot_of_token(lay: Layout) -> np.ndarray:
    """pi(n): the slot of raster token n = (t H + h) W + w.

    [RF2 Abstract, insight (2); TL;DR "3D window permutation"], reading R1:
    t = bt wt + dt (same for h, w), block = (bt nH + bh) nW + bw,
    slot = block bs + (dt wh + dh) ww + dw.  Reading R2 when the permutation
    is off: slot = n."""
    z = sizes(lay)
    if not lay.permute:
        return np.arange(z["N"], dtype=np.int64)
    t, h, w = np.meshgrid(np.arange(lay.T), np.arange(lay.H), np.arange(lay.W),
                          indexing="ij")
    bt, dt = np.divmod(t, lay.wt)
    bh, dh = np.divmod(h, lay.wh)
    bw, dw = np.divmod(w, lay.ww)
    block = (bt * z["nH"] + bh) * z["nW"] + bw
    inner = (dt * lay.wh + dh) * lay.ww + dw
    return (block * z["bs"] + inner).reshape(-1).astype(np.int64)


def slot_valid(lay: Layout) -> np.ndarray:
    """Boolean per slot of the permuted sequence (video slots, then text):
    True where the slot holds a real token.  Readings R1, R2, R7."""
    z = sizes(lay)
    valid = np.zeros(z["Lp"], dtype=bool)
    valid[slot_of_token(lay)] = True
    valid[z["Np"]:] = True
    return valid


def permute(x: np.ndarray, lay: Layout) -> np.ndarray:
    """Scatter raster tokens into window order.  x: [..., N + n_text, d] ->
    [..., Np + n_text, d]; pad slots 0; text copied after Np.
    [RF2 Abstract, insight (2)], readings R1, R2, R7."""
    z = sizes(lay)
    out = np.zeros(x.shape[:-2] + (z["Lp"], x.shape[-1]), dtype=x.dtype)
    out[..., slot_of_token(lay), :] = x[..., :z["N"], :]
    out[..., z["Np"]:, :] = x[..., z["N"]:, :]
    return out


def unpermute(xp: np.ndarray, lay: Layout) -> np.ndarray:
    """Inverse of `permute`: gather each raster token from its slot; pad
    dropped, text copied back.  [RF2 Abstract, insight (2)]."""
    z = sizes(lay)
    out = np.empty(xp.shape[:-2] + (z["L"], xp.shape[-1]), dtype=xp.dtype)
    out[..., :z["N"], :] = xp[..., slot_of_token(lay), :]
    out[..., z["N"]:, :] = xp[..., z["Np"]:, :]
    return out


def block_counts(lay: Layout) -> np.ndarray:
    """c_b: valid tokens in each video block."""
    z = sizes(lay)
    return slot_valid(lay)[:z["Np"]].reshape(z["nb"], z["bs"]).sum(axis=1)


def block_means(xp: np.ndarray, lay: Layout) -> np.ndarray:
    """Representative token of each video block: the mean of its valid
    tokens, in fp64.  [RF2 Abstract, insight (1)], reading R3.
    xp: [B, H, Np + n_text, d] -> [B, H, nb, d]."""
    z = sizes(lay)
    valid = slot_valid(lay)[:z["Np"]].reshape(z["nb"], z["bs"])
    blocks = xp[..., :z["Np"], :].astype(np.float64)
    blocks = blocks.reshape(xp.shape[:-2] + (z["nb"], z["bs"], xp.shape[-1]))
    sums = (blocks * valid[:, :, None]).sum(axis=-2)
    return sums / valid.sum(axis=1)[:, None]


def block_scores(qbar: np.ndarray, kbar: np.ndarray):
    """Block logits l = Qbar Kbar^T / sqrt(d) and their row softmax P over
    the video key blocks, fp64.  [RF2 Abstract, insight (1)], reading R4."""
    d = qbar.shape[-1]
    l = np.matmul(qbar, np.swapaxes(kbar, -1, -2)) / math.sqrt(d)
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return l, e / e.sum(axis=-1, keepdims=True)


def sink_blocks(lay: Layout) -> np.ndarray:
    """Ascending ids of the key blocks that hold a frame-0 token, or none when
    the sink is off.  [RF2 Abstract, insight (3) first-frame sink], R6."""
    if not lay.sink:
        return np.zeros(0, dtype=np.int64)
    z = sizes(lay)
    first = slot_of_token(lay)[: lay.H * lay.W]
    return np.unique(first // z["bs"])


def keep_count(n: int, sparsity_pct: int, n_sink: int):
    """(k, k_eff) of reading R5, in integer arithmetic."""
    k = (n * (100 - sparsity_pct) + 50) // 100
    return k, max(k, n_sink, 1)


def predict_mask(qbar: np.ndarray, kbar: np.ndarray, lay: Layout,
                 sparsity_pct: int):
    """Kept key tiles per query tile, for every (b, h).

    Returns (kept, l): kept[b][h] is a list over query tiles (video blocks,
    then text tiles) of ascending int arrays of key-tile ids (video blocks
    0..nb-1, text tiles nb..); l is the logit array [B, H, nb, nb].
    [RF2 Abstract, insights (1) and (3); TL;DR], readings R4-R7."""
    z = sizes(lay)
    nb, n_tt = z["nb"], z["n_text_tiles"]
    l, _ = block_scores(qbar, kbar)
    sinks = sink_blocks(lay)
    is_sink = np.zeros(nb, dtype=bool)
    is_sink[sinks] = True
    _, k_eff = keep_count(nb, sparsity_pct, len(sinks))
    n_pick = k_eff - len(sinks)
    text_tiles = np.arange(nb, nb + n_tt)
    all_tiles = np.arange(nb + n_tt)
    idx = np.arange(nb)
    kept = []
    B, H = qbar.shape[:2]
    for b in range(B):
        per_head = []
        for h in range(H):
            rows = []
            for i in range(nb):
                cand = idx[~is_sink]
                order = np.lexsort((cand, -l[b, h, i, cand]))
                chosen = np.concatenate([sinks, cand[order[:n_pick]]])
                rows.append(np.concatenate([np.sort(chosen), text_tiles]))
            for _ in range(n_tt):
                rows.append(all_tiles.copy())
            per_head.append(rows)
        kept.append(per_head)
    return kept, l


def sparse_attention(qp, kp, vp, kept, lay: Layout, scale=None,
                     query_tiles=None):
    """Block-sparse softmax attention over the kept tiles, fp64.

    For each valid query token of tile i: o = sum_j softmax_j(q . k_j * scale)
    v_j over the valid tokens of the tiles in kept[b][h][i]; pad query rows
    are 0.  [RF2 Abstract, skipping insignificant tokens; RF1 review,
    Assumptions, Eq. (1) softmax attention], reading R8.

    qp, kp, vp: [B, H, Np + n_text, d] in window order.  query_tiles: None
    (all) or a dict {(b, h): iterable of tile ids}.  Tiles not computed are
    NaN in the result so that an accidental comparison fails."""
    z = sizes(lay)
    bs, Lp = z["bs"], z["Lp"]
    d = qp.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    valid = slot_valid(lay)
    B, H = qp.shape[:2]
    out = np.full(qp.shape, np.nan, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            tiles = (range(z["n_tiles"]) if query_tiles is None
                     else query_tiles.get((b, h), ()))
            for i in tiles:
                rows = np.arange(i * bs, min((i + 1) * bs, Lp))
                out[b, h, rows] = 0.0
                qrows = rows[valid[rows]]
                keys = np.concatenate([
                    np.arange(j * bs, min((j + 1) * bs, Lp))
                    for j in kept[b][h][i]])
                keys = keys[valid[keys]]
                q = qp[b, h, qrows].astype(np.float64)
                k = kp[b, h, keys].astype(np.float64)
                v = vp[b, h, keys].astype(np.float64)
                s = (q @ k.T) * scale
                p = np.exp(s - s.max(axis=1, keepdims=True))
                out[b, h, qrows] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def attention_lse(qp, kp, kept, lay: Layout, scale=None, query_tiles=None):
    """Natural log of each query's softmax denominator over its kept tiles,
    fp64: lse = log sum_j exp(q . k_j * scale) over the valid tokens of
    kept[b][h][i] (reading R8's sum); pad query slots are -inf, query tiles
    not computed NaN.  qp, kp: [B, H, Np + n_text, d].  Returns [B, H, Lp]."""
    z = sizes(lay)
    bs, Lp = z["bs"], z["Lp"]
    d = qp.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    valid = slot_valid(lay)
    B, H = qp.shape[:2]
    out = np.full((B, H, Lp), np.nan)
    for b in range(B):
        for h in range(H):
            tiles = (range(z["n_tiles"]) if query_tiles is None
                     else query_tiles.get((b, h), ()))
            for i in tiles:
                rows = np.arange(i * bs, min((i + 1) * bs, Lp))
                out[b, h, rows] = -np.inf
                qrows = rows[valid[rows]]
                keys = np.concatenate([np.arange(j * bs, min((j + 1) * bs, Lp))
                                       for j in kept[b][h][i]])
                keys = keys[valid[keys]]
                s = (qp[b, h, qrows].astype(np.float64) @
                     kp[b, h, keys].astype(np.float64).T) * scale
                mx = s.max(axis=1, keepdims=True)
                out[b, h, qrows] = (mx + np.log(np.exp(s - mx).sum(axis=1, keepdims=True)))[:, 0]
    return out


def kept_dense(kept, lay: Layout) -> np.ndarray:
    """The kept lists as a 0/1 matrix [B, H, n_tiles, n_tiles] (row i, column
    j = 1 when query tile i keeps key tile j)."""
    z = sizes(lay)
    B, H = len(kept), len(kept[0])
    m = np.zeros((B, H, z["n_tiles"], z["n_tiles"]), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            for i, row in enumerate(kept[b][h]):
                m[b, h, i, np.asarray(row, dtype=np.int64)] = 1
    return m


def attention_recall(qp, kp, kept, lay: Layout, query_tiles, scale=None):
    """Share of each query's dense softmax mass inside its kept tiles, fp64.

    Reading R9 of the masked recall R' [RF1 review, "What carries the
    argument"]: numerator over the valid keys of kept[b][h][i], denominator
    over all valid keys.  qp, kp: [B, H, Np + n_text, d] in window order;
    query_tiles: {(b, h): iterable of tile ids}.  Returns {(b, h, i): array
    of bs recalls} with NaN at pad query slots."""
    z = sizes(lay)
    bs, Lp = z["bs"], z["Lp"]
    d = qp.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    valid = slot_valid(lay)
    all_keys = np.flatnonzero(valid)
    out = {}
    for (b, h), tiles in query_tiles.items():
        k_all = kp[b, h, all_keys].astype(np.float64)
        for i in tiles:
            r = np.full(bs, np.nan)
            rows = np.arange(i * bs, min((i + 1) * bs, Lp))
            rows = rows[valid[rows]]
            kept_keys = np.concatenate([
                np.arange(j * bs, min((j + 1) * bs, Lp)) for j in kept[b][h][i]])
            in_kept = np.isin(all_keys, kept_keys)
            if len(rows):
                s = (qp[b, h, rows].astype(np.float64) @ k_all.T) * scale
                e = np.exp(s - s.max(axis=1, keepdims=True))
                r[rows - i * bs] = e[:, in_kept].sum(axis=1) / e.sum(axis=1)
            out[(b, h, i)] = r
    return out


SPATIAL, TEMPORAL, TEXTURAL = 0, 1, 2


def band_halfwidth(lay: Layout, bandwidth: float) -> int:
    """w = floor(b nb + 1/2) video tiles, reading R10."""
    return int(math.floor(bandwidth * sizes(lay)["nb"] + 0.5))


def tile_rank(lay: Layout) -> np.ndarray:
    """r(i): position of video tile i when the tiles are sorted by (h, w, t)
    of their first valid token (spatial-major order), reading R10."""
    z = sizes(lay)
    src = np.full(z["Np"], -1, dtype=np.int64)
    src[slot_of_token(lay)] = np.arange(z["N"])
    first = []
    for i in range(z["nb"]):
        toks = src[i * z["bs"]:(i + 1) * z["bs"]]
        first.append(toks[toks >= 0][0])
    first = np.array(first)
    t, rem = np.divmod(first, lay.H * lay.W)
    h, w = np.divmod(rem, lay.W)
    order = np.lexsort((t, w, h))          # last key is the primary one
    rank = np.empty(z["nb"], dtype=np.int64)
    rank[order] = np.arange(z["nb"])
    return rank


def pattern_keeps(lay: Layout, pattern: int, w: int, tau: int) -> np.ndarray:
    """Boolean [nb, nb] video-tile mask of one v1 head pattern, reading R10.
    [RF1 review, "What carries the argument"; free parameters bandwidth and
    tau]."""
    nb = sizes(lay)["nb"]
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    if pattern == SPATIAL:
        return np.abs(i - j) <= w
    if pattern == TEMPORAL:
        r = tile_rank(lay)
        return np.abs(r[:, None] - r[None, :]) <= w
    if pattern == TEXTURAL:
        # the union over k of {i mod tau = k and j mod tau = k}
        return np.logical_or.reduce([(i % tau == k) & (j % tau == k)
                                     for k in range(tau)])
    raise ValueError(f"pattern {pattern}")


def pattern_mask(lay: Layout, head_pattern, w: int, tau: int):
    """Kept tiles per query tile for every (b, h), in the list-of-rows form
    of `predict_mask`: video rows from `pattern_keeps` of the head's pattern
    plus the text tiles, text rows every tile (R7, R10).
    head_pattern: int array [B, H]."""
    z = sizes(lay)
    nb, n_tiles = z["nb"], z["n_tiles"]
    text_tiles = np.arange(nb, n_tiles)
    masks = {}
    kept = []
    hp = np.asarray(head_pattern)
    for b in range(hp.shape[0]):
        per_head = []
        for h in range(hp.shape[1]):
            p = int(hp[b, h])
            if p not in masks:
                masks[p] = pattern_keeps(lay, p, w, tau)
            rows = [np.concatenate([np.flatnonzero(masks[p][i]), text_tiles])
                    for i in range(nb)]
            rows += [np.arange(n_tiles) for _ in range(z["n_text_tiles"])]
            per_head.append(rows)
        kept.append(per_head)
    return kept


def arm_samples(lay: Layout, local: bool, stride: int) -> np.ndarray:
    """Raster ids of ARM's sampled tokens, reading R11: every stride-th token
    of frame 0 (local) or of the whole video (global)."""
    limit = lay.H * lay.W if local else lay.T * lay.H * lay.W
    return np.arange(0, limit, stride, dtype=np.int64)


def arm_recall(q, k, lay: Layout, pattern: int, w: int, tau: int, tokens,
               scale=None) -> np.ndarray:
    """Per sampled query, the share of its softmax mass over the sampled keys
    that falls on keys its tile keeps under `pattern`, fp64.  Reading R11 of
    R' = S(Q', K', M') / S(Q', K', M_init) [RF1 review, "What carries the
    argument"].  q, k: raster [B, H, N + n_text, d].  Returns [B, H, n]."""
    z = sizes(lay)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    tokens = np.asarray(tokens)
    tile = slot_of_token(lay)[tokens] // z["bs"]
    m = pattern_keeps(lay, pattern, w, tau)[tile[:, None], tile[None, :]]
    qs = q[:, :, tokens].astype(np.float64)
    ks = k[:, :, tokens].astype(np.float64)
    s = np.matmul(qs, np.swapaxes(ks, -1, -2)) * scale
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return (e * m).sum(axis=-1) / e.sum(axis=-1)


def arm_classify(local_recall, global_recall, alpha: float) -> np.ndarray:
    """Head pattern from the per-sample recalls [B, H, n], reading R11:
    temporal if mean local >= alpha, else spatial if mean global >= alpha,
    else textural.  [RF1 review, "Core claim", classification order]."""
    bR = np.mean(local_recall, axis=-1)
    eR = np.mean(global_recall, axis=-1)
    return np.where(bR >= alpha, TEMPORAL,
                    np.where(eR >= alpha, SPATIAL, TEXTURAL))


E4M3_MAX = 448.0


def e4m3(x) -> np.ndarray:
    """Round to the nearest OCP e4m3 value, ties to even (reading R12).
    Normal numbers |x| >= 2^-6 have 3 fraction bits, so the spacing is
    2^(E - 3) for |x| in [2^E, 2^(E+1)); below 2^-6 the spacing is the
    subnormal step 2^-9.  Values that round above 448 are not representable
    and raise."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.exp2(np.maximum(E, -6.0) - 3.0)
    r = np.round(a / step) * step          # np.round: half to even
    if np.any(r > E4M3_MAX):
        raise ValueError("value outside the e4m3 range")
    return np.copysign(r, x)


def pow2_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e; 0 for amax == 0 (R12)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_tiles(xp, lay: Layout):
    """Per-(b, h, tile) power-of-two scaled e4m3 of a permuted tensor
    [B, H, Lp, d] (reading R12).  Returns (dequantized values, fp64, same
    shape; exponents [B, H, n_tiles])."""
    z = sizes(lay)
    bs = z["bs"]
    B, H, Lp, d = xp.shape
    out = np.empty(xp.shape, dtype=np.float64)
    ex = np.zeros((B, H, z["n_tiles"]), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for t in range(z["n_tiles"]):
                rows = slice(t * bs, min((t + 1) * bs, Lp))
                x = xp[b, h, rows].astype(np.float64)
                e = pow2_exponent(np.abs(x).max() if x.size else 0.0)
                ex[b, h, t] = e
                out[b, h, rows] = e4m3(x * 2.0 ** -e) * 2.0 ** e
    return out, ex


def quantize_channels(xp):
    """Per-(b, h, feature) power-of-two scaled e4m3 over all slots of a
    permuted tensor [B, H, Lp, d] (reading R12).  Returns (dequantized
    values, exponents [B, H, d])."""
    B, H, _, d = xp.shape
    x = xp.astype(np.float64)
    amax = np.abs(x).max(axis=2)
    ex = np.vectorize(pow2_exponent, otypes=[np.int64])(amax)
    scale = np.exp2(ex)[:, :, None, :]
    return e4m3(x / scale) * scale, ex


def sparse_attention_fp8(qp, kp, vp, kept, lay: Layout, scale=None,
                         query_tiles=None):
    """Block-sparse attention over e4m3-quantized Q, K (per tile) and V (per
    feature), reading R12: `sparse_attention` on the dequantized values."""
    q8, _ = quantize_tiles(qp, lay)
    k8, _ = quantize_tiles(kp, lay)
    v8, _ = quantize_channels(vp)
    return sparse_attention(q8, k8, v8, kept, lay, scale=scale,
                            query_tiles=query_tiles)


def run(q, k, v, lay: Layout, sparsity_pct: int, query_tiles=None):
    """The whole path on raster inputs [B, H, N + n_text, d] (any float
    dtype; computed in fp64): permute, pool, predict, attend, unpermute."""
    qp, kp, vp = (permute(np.asarray(x, dtype=np.float64), lay)
                  for x in (q, k, v))
    qbar, kbar = block_means(qp, lay), block_means(kp, lay)
    kept, l = predict_mask(qbar, kbar, lay, sparsity_pct)
    op = sparse_attention(qp, kp, vp, kept, lay, query_tiles=query_tiles)
    return dict(qp=qp, kp=kp, vp=vp, qbar=qbar, kbar=kbar, l=l, kept=kept,
                op=op, o=unpermute(op, lay))
