"""GPU parity on seeded random problem shapes: batch, heads, query and key
lengths, head dim (any multiple of 8 up to 128), input type and causality
drawn from a fixed generator, so that one run crosses the launch choices
(direct 4- and 8-wave, key-split, split-key with its merge) at shapes no
other test names. Each case is checked against the fp64 oracle at the forward
tests' bars (4e-3 fp16 / 3.2e-2 bf16 on O, 1e-3 relative on lse) through
fa.fwd with the suggested split count. Two more draws add padding lengths and
windows, and heavy-tailed scores (q x 4).
"""

import random

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_forward_fwd_amd as fa
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 3.2e-2}


def draw_cases(n, seed):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        B, H = rng.choice([1, 2, 3, 4]), rng.choice([1, 2, 4, 8, 16, 32])
        Nq = rng.choice([1, 7, 32, 33, 100, 257, 640, 1000, 1500])
        Nk = rng.choice([1, 31, 64, 200, 511, 1000, 2048, 3000])
        d = rng.choice([8, 16, 24, 32, 40, 64, 72, 96, 104, 128])
        dtype = rng.choice(["bf16", "fp16"])
        causal = rng.random() < 0.5
        if B * H * Nq * Nk > 40_000_000:  # keep the oracle at a second or two
            continue
        cases.append((B, H, Nq, Nk, d, dtype, causal))
    return cases


CASES = draw_cases(40, 2024)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{c[5]}{'c' if c[6] else ''}"
                                             for c in CASES])
def test_random_shape(case):
    B, H, Nq, Nk, d, dtype, causal = case
    q = make_qkv(B, H, Nq, d, dtype, 800 + Nq + d)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, 801 + Nk)
    code = fa.dtype_code(q.dtype)
    plan = fa.fa_plan_qk(B, H, Nq, Nk, d, int(causal), code)
    splits = fa.fa_split_count(B, H, Nq, Nk, d, int(causal))
    launch = "split" if splits > 1 else ("key-split" if plan["block_m"] == 32 else f"direct {plan['block_m']}-row")
    print(f"[case] {case} -> {launch}", flush=True)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale)
    og = o.cpu().float().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    err_o = float(np.abs(og - o64).max())
    err_l = float((np.abs(lg - l64) / np.maximum(1.0, np.abs(l64))).max())
    print(f"[parity] random {case} {launch} max|dO|={err_o:.3e} ({100 * err_o / TOL_O[q.dtype]:.0f}% of bar) "
          f"max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[q.dtype] and err_l <= 1e-3
    if causal:
        assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def draw_masked_cases(n, seed):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        B, H = rng.choice([1, 2, 3, 4]), rng.choice([1, 2, 4, 8])
        Nq = rng.choice([1, 33, 100, 257, 640, 1000])
        Nk = rng.choice([31, 64, 200, 511, 1000, 2048])
        d = rng.choice([16, 40, 64, 96, 128])
        dtype = rng.choice(["bf16", "fp16"])
        causal = rng.random() < 0.5
        wl = rng.choice([-1, -1, 0, 17, 128, 1000])
        wr = -1 if causal else rng.choice([-1, -1, 0, 5, 300])
        key_lens = [rng.randint(0, Nk) for _ in range(B)] if rng.random() < 0.6 else None
        if wl == -1 and wr == -1 and key_lens is None:
            continue  # no mask in effect: covered above
        if B * H * Nq * Nk > 30_000_000:
            continue
        cases.append((B, H, Nq, Nk, d, dtype, causal, wl, wr, key_lens))
    return cases


MASKED_CASES = draw_masked_cases(24, 2025)


@pytest.mark.parametrize("case", MASKED_CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{c[5]}{'c' if c[6] else ''}"
                                                    f"w{c[7]}_{c[8]}{'p' if c[9] else ''}" for c in MASKED_CASES])
def test_random_masked_shape(case):
    B, H, Nq, Nk, d, dtype, causal, wl, wr, key_lens = case
    q = make_qkv(B, H, Nq, d, dtype, 900 + Nq + d)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, 901 + Nk)
    splits = fa.fa_split_count(B, H, Nq, Nk, d, int(causal))
    print(f"[case] masked {case} splits={splits}", flush=True)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, window_left=wl, window_right=wr,
                    key_lens=key_lens)
    torch.cuda.synchronize()
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale, window_left=wl, window_right=wr, key_lens=key_lens)
    og = o.cpu().float().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(l64)
    # rows that see no key: O = 0 and lse = -inf exactly
    assert np.array_equal(np.isfinite(lg), fin) and np.all(og[~fin] == 0)
    err_o = float(np.abs(og - o64).max())
    err_l = float((np.abs(lg[fin] - l64[fin]) / np.maximum(1.0, np.abs(l64[fin]))).max()) if fin.any() else 0.0
    print(f"[parity] random masked {case} max|dO|={err_o:.3e} ({100 * err_o / TOL_O[q.dtype]:.0f}% of bar) "
          f"max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[q.dtype] and err_l <= 1e-3


def draw_heavy_cases(n, seed):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        B, H = rng.choice([1, 2, 4]), rng.choice([1, 4, 8, 16])
        Nq = rng.choice([1, 33, 257, 640, 1000, 1500, 2048])
        Nk = rng.choice([64, 511, 1000, 2048, 3000])
        d = rng.choice([32, 64, 96, 128])
        dtype = rng.choice(["bf16", "fp16"])
        causal = rng.random() < 0.5
        if B * H * Nq * Nk > 40_000_000:
            continue
        cases.append((B, H, Nq, Nk, d, dtype, causal))
    return cases


HEAVY_CASES = draw_heavy_cases(12, 2026)


@pytest.mark.parametrize("case", HEAVY_CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{c[5]}{'c' if c[6] else ''}"
                                                   for c in HEAVY_CASES])
def test_random_heavy_tailed_shape(case):
    # q x 4 spreads the scores over about 4x the log2 range, so later key tiles
    # raise the running max and the lazy-max refresh runs in every launch kind
    B, H, Nq, Nk, d, dtype, causal = case
    q = make_qkv(B, H, Nq, d, dtype, 1000 + Nq + d, q_scale=4.0)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, 1001 + Nk)
    splits = fa.fa_split_count(B, H, Nq, Nk, d, int(causal))
    print(f"[case] heavy {case} splits={splits}", flush=True)
    scale = fa.default_scale(d)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale)
    og = o.cpu().float().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    err_o = float(np.abs(og - o64).max())
    err_l = float((np.abs(lg - l64) / np.maximum(1.0, np.abs(l64))).max())
    print(f"[parity] random heavy {case} max|dO|={err_o:.3e} ({100 * err_o / TOL_O[q.dtype]:.0f}% of bar) "
          f"max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[q.dtype] and err_l <= 1e-3
