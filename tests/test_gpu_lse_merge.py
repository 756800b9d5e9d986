"""The optional log-sum-exp merges partial attentions, at the full 720p size.

Softmax attention over a union of disjoint key sets is the LSE-weighted mean
of the attentions over each set, and its LSE is the log of the summed
exponentials of theirs.  Each row's kept tiles are split into the tiles at
even and at odd positions of the row.  Both halves are attended through the
padded-row entry point, the two partial outputs are merged with their LSEs
in fp32, and the result must match the attention over the whole row.  The
property holds at any size, so it checks the whole 720p / 80% call (40 heads,
75,600 tokens) with no oracle.

Bounds.  bf16 keeps 8 significant bits, so rounding to it moves a value by
at most 2^-8 of itself.  Each kernel rounds its weights to bf16 for the PV
product while its row sum stays fp32, so its output is within 2^-8 a of the
exact attention, with a = sum_j w_j |v_j| / sum_j w_j: the attention of |V|,
which the same kernel computes on the absolute values.  The merged halves
carry that error once and the whole row once more, and each of the three
bf16 outputs adds at most 2^-8 of its magnitude.  So per element
|merged - whole| <= 2^-7 a (1 + 2^-6) + 2^-8 (max(|o_1|, |o_2|) + |o|) + 1e-5,
the last terms covering fp32 accumulation order.  Each LSE is within 1e-4 of
the exact value (fp32 sums of the fp32 weights), so the merged and the
whole-row LSE are within 2e-4 + 1e-6 |lse| of each other.
"""
import sys

import pytest
import torch

from image_diffusion_dits_amd import configs, inputs, rf

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_lse_merges_two_halves_of_every_row_video720():
    cfg = configs.VIDEO720
    s = 80
    say(f"[lse merge] {cfg.name}, {cfg.H} heads, s={s}: even/odd halves of every row")
    q, k, v = inputs.make_qkv(cfg, "cuda")
    plan = rf.Plan(cfg.layout)
    z = plan.sizes
    kc = plan.keep(s)
    assert z["n_text_tiles"] == 0 and kc["row_len_video"] % 2 == 0
    qp, qb = rf.permute_means(plan, q)
    kp, kb = rf.permute_means(plan, k)
    vt = rf.permute(plan, v, order=rf.TILES_T)
    del q, k, v
    kept = rf.predict_mask(plan, qb, kb, s)
    o_full, lse_full = rf.sparse_attn(plan, qp, kp, vt, kept, s, lse=True)
    a_abs = rf.sparse_attn(plan, qp, kp, vt.abs(), kept, s).float()

    B, H = qp.shape[:2]
    rows = kept.view(B, H, z["nb"], kc["row_len_video"])
    o1, lse1 = rf.sparse_attn_rows(plan, qp, kp, vt, rows[..., 0::2].contiguous(), lse=True)
    o2, lse2 = rf.sparse_attn_rows(plan, qp, kp, vt, rows[..., 1::2].contiguous(), lse=True)
    torch.cuda.synchronize()

    pad = torch.isneginf(lse_full)
    assert torch.equal(pad, torch.isneginf(lse1)) and torch.equal(pad, torch.isneginf(lse2))
    valid = ~pad
    m = torch.maximum(lse1, lse2)
    w1 = torch.where(valid, torch.exp(lse1 - m), torch.zeros_like(m))
    w2 = torch.where(valid, torch.exp(lse2 - m), torch.zeros_like(m))
    wsum = torch.where(valid, w1 + w2, torch.ones_like(m))
    merged = (o1.float() * w1[..., None] + o2.float() * w2[..., None]) / wsum[..., None]
    lse_m = m + torch.log(wsum)

    of = o_full.float()
    bound = (2.0 ** -7 * (1 + 2.0 ** -6) * a_abs
             + 2.0 ** -8 * (torch.maximum(o1.float().abs(), o2.float().abs()) + of.abs())
             + 1e-5)
    err = (merged - of).abs()
    ratio = (err / bound)[valid].max().item()
    lse_err = (lse_m - lse_full).abs()[valid]
    lse_ratio = (lse_err / (2e-4 + 1e-6 * lse_full.abs()[valid])).max().item()
    say(f"[lse merge] output max-abs {err[valid].max().item():.2e} "
        f"({ratio:.2f} of its bound), LSE max-abs {lse_err.max().item():.2e} "
        f"({lse_ratio:.2f} of its bound)")
    assert torch.all(o_full[pad] == 0) and torch.all(o1[pad] == 0) and torch.all(o2[pad] == 0)
    assert ratio <= 1.0
    assert lse_ratio <= 1.0
    plan.close()
