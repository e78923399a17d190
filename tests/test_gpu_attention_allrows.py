"""Every attention row at the large workloads, against a plain fp32 PyTorch computation.

The parity tests compare the full-size workloads with the fp64 oracle on a sample of
rows, since the oracle computes rows one by one. This test checks every live row of C2,
C3 (B = 256, 512) and C4: the trees and ancestor masks come from the oracle, the tree
attention from the library, and the reference is the definition written with PyTorch
fp32 matrix products on the device (scores of the prefix keys and of the visible tree
keys, one softmax over both, the weighted sum of the values). Its fp32 rounding is far
below the bf16 tolerances it is held to (the same as the oracle comparisons: elementwise
2e-2 + 1e-2 |ref|, row L2 1e-2, log-sum-exp 4e-3).
"""
import math

import numpy as np
import pytest
import torch

import block_diffusion_draft_position_amd as ddt
import oracle
from ddt_synthetic import configs, gen

from _cases import attempts
from _gpu import BF16_ATOL, BF16_ROW_L2, BF16_RTOL, dev_tensor, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load()


def _reference(q, kp, vp, kt, vt, vis, scale):
    """q [R, D], prefix kp/vp [P, D], tree kt/vt [N, D], vis [R, N] bool -> (o [R, D], lse [R])."""
    sp = (q @ kp.T) * scale
    st = (q @ kt.T) * scale
    st = st.masked_fill(~vis, -math.inf)
    s = torch.cat([sp, st], dim=1)
    lse = torch.logsumexp(s, dim=1)
    p = torch.exp(s - lse[:, None])
    P = kp.shape[0]
    return p[:, :P] @ vp + p[:, P:] @ vt, lse


@pytest.mark.parametrize("name", ["C2", "C3-B256", "C3-B512", "C4"])
def test_every_row_against_fp32_definition(name):
    cfg = configs.get(name)
    print(f"[case] all rows {cfg.name} S={cfg.S} B={cfg.B} P={cfg.prefix} Hq={cfg.Hq} Hkv={cfg.Hkv}",
          flush=True)
    torch.backends.cuda.matmul.allow_tf32 = False
    b = gen.batch(cfg, attempts(cfg))
    S, N, G, D = cfg.S, cfg.N, cfg.Hq // cfg.Hkv, cfg.D
    W = (N + 31) // 32
    masks = np.zeros((S, N, W), dtype=np.uint32)
    nn = np.zeros(S, dtype=np.int32)
    for s in range(S):
        tok, lq = oracle.topk(b["draft_logits"][s], cfg.K)
        t = oracle.build_tree(tok, lq, int(b["bonus"][s]), cfg.B)
        nn[s] = int(t["num_nodes"])
        masks[s] = oracle.tree_mask(t["parent"], nn[s], N)
    d = upload(b)
    mask_d = dev_tensor(masks.view(np.int32))
    scale = 1.0 / math.sqrt(D)
    out, lse = ddt.ddt_tree_attention(d["q"], d["k_cache"], d["v_cache"], d["cu_prefix"], d["k_tree"],
                                      d["v_tree"], mask_d, dev_tensor(nn), scale)
    torch.cuda.synchronize()
    # visibility of tree key j from node n: bit j of the node's mask words
    bits = torch.arange(N, device="cuda")
    words = mask_d.view(torch.int32).long() & 0xFFFFFFFF  # [S, N, W]
    cu = b["cu_prefix"]
    worst = 0.0
    for s in range(S):
        n_s = int(nn[s])
        vis_nodes = ((words[s][:, bits // 32] >> (bits % 32)) & 1).bool()  # [N, N]
        vis_nodes[:, n_s:] = False
        vis = vis_nodes[:n_s].repeat_interleave(G, dim=0)  # rows n * G + h % G
        p0, p1 = int(cu[s]), int(cu[s + 1])
        for g in range(cfg.Hkv):
            qg = d["q"][s, :n_s, g * G:(g + 1) * G, :].float().reshape(n_s * G, D)
            ref_o, ref_l = _reference(qg, d["k_cache"][p0:p1, g].float(), d["v_cache"][p0:p1, g].float(),
                                      d["k_tree"][s, :, g].float(), d["v_tree"][s, :, g].float(), vis, scale)
            got = out[s, :n_s, g * G:(g + 1) * G, :].float().reshape(n_s * G, D)
            diff = (got - ref_o).abs()
            bad = diff > BF16_ATOL + BF16_RTOL * ref_o.abs()
            assert not bool(bad.any()), (f"{name} seq {s} KV head {g}: {int(bad.sum())} elements off, "
                                         f"worst {float(diff.max()):.3g}")
            rl2 = diff.norm(dim=1) / ref_o.norm(dim=1).clamp_min(1e-30)
            assert float(rl2.max()) <= BF16_ROW_L2, f"{name} seq {s} KV head {g}: row L2 {float(rl2.max()):.3g}"
            gl = lse[s, :n_s, g * G:(g + 1) * G].reshape(n_s * G)
            dl = (gl - ref_l).abs().max()
            assert float(dl) <= 4e-3, f"{name} seq {s} KV head {g}: lse off by {float(dl):.3g}"
            worst = max(worst, float(diff.max()))
        # rows of absent nodes: zeros and -inf
        if n_s < N:
            assert bool((out[s, n_s:] == 0).all()) and bool(torch.isneginf(lse[s, n_s:]).all())
    print(f"[done] {name}: {int(nn.sum()) * cfg.Hq} rows, worst |d| {worst:.3g}", flush=True)
