"""The seeded generator: determinism, planted structure, bf16 rounding."""
import numpy as np
import torch

from ddt_synthetic import configs, gen


def test_deterministic_and_attempt_redraws():
    c = configs.C1
    a, b = gen.draft(c, 0, 0), gen.draft(c, 0, 0)
    assert np.array_equal(a["logits"], b["logits"]) and a["bonus"] == b["bonus"]
    assert not np.array_equal(a["logits"], gen.draft(c, 0, 1)["logits"])
    assert np.array_equal(gen.qkv(configs.C0, 0)["q"], gen.qkv(configs.C0, 0)["q"])


def test_planted_chain_boost():
    c = configs.custom("t", L=16, V=1000, K=4, B=4)
    d = gen.draft(c, 0, 0)
    z = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c.cfg_id, 0, 0, 0])))
    chain = z.integers(0, c.V, size=c.L + 1)
    z.integers(0, c.V)
    base = (np.float32(2.0) * z.standard_normal((c.L, c.V), dtype=np.float32)).astype(np.float32)
    assert np.array_equal(chain, d["chain"])
    diff = d["logits"].astype(np.float64) - base
    for i in range(1, c.L + 1):
        nz = np.flatnonzero(diff[i - 1])
        if i == 15:                      # 6 - 0.4 * 15 = 0: nothing planted
            assert nz.tolist() == []
            continue
        assert nz.tolist() == [chain[i - 1]]
        assert abs(diff[i - 1, chain[i - 1]] - (6 - 0.4 * i)) < 1e-5


def test_target_is_function_of_path():
    c = configs.C0
    d = gen.draft(c, 0, 0)
    keep = gen.keep_flags(c, 0, 0)
    r1 = gen.target_row(c, 0, 0, (3, 4), d["chain"], keep)
    r2 = gen.target_row(c, 0, 0, (3, 4), d["chain"], keep)
    r3 = gen.target_row(c, 0, 0, (4, 3), d["chain"], keep)
    assert np.array_equal(r1, r2) and not np.array_equal(r1, r3)
    on = gen.target_row(c, 0, 0, tuple(int(t) for t in d["chain"][:2]), d["chain"], keep)
    if keep[2]:
        assert int(np.argmax(on)) == int(d["chain"][2])


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties to even
    bits = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = gen.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_batch_layout():
    c = configs.custom("t", S=3, L=3, V=20, K=2, B=5, prefix=(4, 9), Hq=4, Hkv=2, D=8, dtype="bf16")
    b = gen.batch(c)
    P = b["prefix_lens"]
    assert b["cu_prefix"].tolist() == [0, P[0], P[0] + P[1], P.sum()]
    assert b["k_cache"].shape == (P.sum(), 2, 8) and b["k_cache"].dtype == np.uint16
    assert b["q"].shape == (3, 6, 4, 8)
    x1 = gen.qkv(c, 1)
    assert np.array_equal(b["k_cache"][P[0]:P[0] + P[1]], x1["k_prefix"])
    assert np.all((4 <= P) & (P <= 9))
