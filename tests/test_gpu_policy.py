"""A layer under the timestep policy runs exactly the library's path: dense
steps equal the sparsity-0 path (dense attention, checked against the
oracle), predicted steps equal a fresh run, reused steps apply the earlier
mask to the new inputs."""
import sys

import numpy as np
import pytest
import torch

import parity
from image_diffusion_dits_amd import configs, inputs, rf
from image_diffusion_dits_amd.policy import SparseAttention, StepPolicy
from oracle import rainfusion_oracle as orc

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_policy_steps_match_the_library_path():
    cfg = configs.IMAGE
    say(f"[policy] {cfg.name}: dense, predict and reuse steps")
    q, k, v = inputs.make_qkv(cfg, "cuda", H=4)
    q2, k2, v2 = (inputs.random_tensor(q.shape, s, device="cuda", dtype=q.dtype)
                  for s in (91, 92, 93))
    pol = StepPolicy(10, dense_fraction=0.1, sparsity_pct=cfg.sparsity[0], refresh_every=2)
    assert pol.schedule()[:4] == ["dense", "predict", "reuse", "predict"]
    layer = SparseAttention(cfg.layout, pol, cfg.B, 4, cfg.d, q.dtype, "cuda")
    plan = rf.Plan(cfg.layout)
    s = cfg.sparsity[0]

    o_dense = layer(q, k, v, 0).clone()
    ref0, _ = rf.sparse_attention(q, k, v, plan, 0)
    torch.cuda.synchronize()
    assert torch.equal(o_dense, ref0)
    # Dense step = dense attention (oracle, all tokens, two heads).
    lay = parity.olayout(cfg)
    for h in (0, 3):
        sl = (slice(0, 1), slice(h, h + 1))
        qv, kv, vv = (parity.values(x[sl]) for x in (q, k, v))
        s_ = qv[0, 0] @ kv[0, 0].T / np.sqrt(cfg.d)
        p = np.exp(s_ - s_.max(axis=1, keepdims=True))
        want = (p / p.sum(axis=1, keepdims=True)) @ vv[0, 0]
        err = np.abs(parity.values(o_dense[sl])[0, 0] - want)
        assert err.max() <= parity.TOL["bf16"][0] and err.mean() <= parity.TOL["bf16"][1]

    o_pred = layer(q, k, v, 1).clone()
    ref1, kept1 = rf.sparse_attention(q, k, v, plan, s)
    torch.cuda.synchronize()
    assert torch.equal(o_pred, ref1)

    o_reuse = layer(q2, k2, v2, 2).clone()
    qp2, kp2 = rf.permute(plan, q2), rf.permute(plan, k2)
    vt2 = rf.permute(plan, v2, order=rf.TILES_T)
    ref2 = rf.unpermute(plan, rf.sparse_attn(plan, qp2, kp2, vt2, kept1, s))
    fresh2, kept_fresh = rf.sparse_attention(q2, k2, v2, plan, s)
    torch.cuda.synchronize()
    assert torch.equal(o_reuse, ref2)
    assert not torch.equal(kept_fresh, kept1)      # the new inputs would pick other tiles
    assert not torch.equal(o_reuse, fresh2)

    o_pred2 = layer(q2, k2, v2, 3).clone()
    torch.cuda.synchronize()
    assert torch.equal(o_pred2, fresh2)
    layer.close()
    plan.close()
