"""GPU parity of the key-split forward (small grids: four waves share 32 query
rows and split their key tiles, merged in LDS) against the fp64 oracle, at the
forward tests' tolerances (4e-3 fp16 / 3.2e-2 bf16 on O, 1e-3 relative on
lse). Every case first checks through fa_plan_qk that the launch it makes is a
key-split one (32-row workgroups, 32-key tiles), so the kernel under test is
the one that runs.
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_forward_fwd_amd as fa
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 3.2e-2}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()


def qk_inputs(B, H, Nq, Nk, d, dtype, seed, q_scale=1.0):
    q = make_qkv(B, H, Nq, d, dtype, seed, q_scale=q_scale)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed + 1)
    return q, k, v


def run_and_check(q, k, v, causal, label):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    code = fa.dtype_code(q.dtype)
    plan = fa.fa_plan_qk(B, H, Nq, Nk, d, int(causal), code)
    assert (plan["block_m"], plan["block_n"], plan["threads"]) == (32, 32, 256), (label, plan)
    assert fa.fa_split_count(B, H, Nq, Nk, d, int(causal)) == 1
    print(f"[case] key-split {label} causal={causal}", flush=True)
    scale = fa.default_scale(d)
    n = q.numel()
    base = torch.full((n + 4096,), float("nan"), dtype=q.dtype, device="cuda")
    out = base[:n].view(q.shape)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, out=out)
    o2, lse2 = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isnan(base[n:]).all(), f"{label}: write past the output"
    assert torch.equal(o, o2) and torch.equal(lse, lse2), f"{label}: not deterministic"
    o, lse = o.cpu(), lse.cpu()
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale)
    err_o = float(np.abs(o.float().numpy().astype(np.float64) - o64).max())
    err_l = float((np.abs(lse.numpy().astype(np.float64) - l64) / np.maximum(1.0, np.abs(l64))).max())
    print(f"[parity] key-split {label} causal={causal} max|dO|={err_o:.3e} ({100 * err_o / TOL_O[q.dtype]:.0f}% of bar) "
          f"max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[q.dtype], f"{label}: O error {err_o:.3e}"
    assert err_l <= TOL_LSE, f"{label}: lse error {err_l:.3e}"
    if causal:
        assert torch.equal(o[:, :, 0], v[:, :, 0]), f"{label}: causal row 0 is not V[0]"


@pytest.mark.parametrize("B,H,N,d,dtype", [(2, 4, 1000, 64, "bf16"), (2, 4, 1000, 128, "fp16"),
                                           (1, 2, 2048, 128, "bf16"), (1, 1, 513, 64, "fp16"),
                                           (1, 3, 520, 128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_key_split_square(B, H, N, d, dtype, causal):
    # ragged key counts (513, 520: the last wave gets fewer tiles) and the
    # longest key range it takes (2048); 520 keys give 17 tiles of 32
    # (5, 5, 5, 2)
    q, k, v = qk_inputs(B, H, N, N, d, dtype, 700 + N + d)
    run_and_check(q, k, v, causal, f"B{B} H{H} N{N} d{d} {dtype}")


@pytest.mark.parametrize("Nq,Nk,causal", [(300, 2000, False), (700, 2000, True), (1500, 600, False),
                                          (1500, 600, True), (33, 2048, False)])
def test_key_split_query_and_key_lengths(Nq, Nk, causal):
    # causal rows past the last key see every key (top-left alignment)
    q, k, v = qk_inputs(1, 4, Nq, Nk, 64, "bf16", 710)
    run_and_check(q, k, v, causal, f"Nq{Nq} Nk{Nk}")


@pytest.mark.parametrize("d,dtype", [(96, "bf16"), (80, "fp16"), (40, "bf16"), (24, "fp16"), (120, "bf16")])
def test_key_split_other_head_dims(d, dtype):
    q, k, v = qk_inputs(1, 2, 777, 777, d, dtype, 720 + d)
    for causal in (False, True):
        run_and_check(q, k, v, causal, f"d{d} {dtype}")


def test_key_split_heavy_tailed_scores():
    # q x 4 spreads the scores so that later tiles refresh the running max
    # and the waves' maxima differ widely before the merge
    q, k, v = qk_inputs(1, 4, 1024, 1024, 128, "bf16", 730, q_scale=4.0)
    for causal in (False, True):
        run_and_check(q, k, v, causal, "q x 4")


def test_key_split_one_dominant_key_in_the_last_range():
    # every query row leans on one direction u, and key 1000 (in the last
    # wave's range) is 5 sqrt(d) u: its score is about 10 against about
    # N(0, 0.56) for the others, so the other waves' partial sums must get
    # almost no weight in the merge
    q, k, v = qk_inputs(1, 2, 256, 1024, 64, "bf16", 740)
    g = torch.Generator().manual_seed(741)
    u = torch.randn(64, generator=g, dtype=torch.float64)
    u = u / u.norm()
    qf = q.double() * 0.5 + 2.0 * u
    kf = k.double()
    kf[:, :, 1000] = 5.0 * 8.0 * u
    q, k = qf.to(q.dtype), kf.to(k.dtype)
    run_and_check(q, k, v, False, "dominant late key")


def test_key_split_query_prefix_bitwise():
    # causal rows of a query prefix (a whole number of 32-row blocks: the
    # lazy-max refresh is decided per wave) see the same key tiles, split
    # among the waves the same way, as in the square problem: bit for bit
    q, k, v = make_qkv(1, 2, 1500, 128, "bf16", 750)
    for nq in (1500, 704):
        plan = fa.fa_plan_qk(1, 2, nq, 1500, 128, 1, fa.FA_DTYPE_BF16)
        assert plan["block_m"] == 32
    o_sq, l_sq = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    o_pre, l_pre = fa.fwd(q[:, :, :704].contiguous().cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_pre, o_sq[:, :, :704]) and torch.equal(l_pre, l_sq[:, :, :704])


@pytest.mark.parametrize("Nq,Nk,causal,d", [(100, 1, False, 64), (100, 1, True, 128), (40, 31, False, 64),
                                            (33, 65, True, 128), (35, 97, False, 40), (1000, 33, True, 64),
                                            (257, 100, False, 128)])
def test_key_split_waves_without_keys(Nq, Nk, causal, d):
    # fewer than four 32-key tiles: the later waves get empty ranges and must
    # get weight zero in the merge; 33-35 query rows leave a block of 1-3 rows
    q, k, v = qk_inputs(1, 3, Nq, Nk, d, "fp16", 760 + Nq + Nk)
    run_and_check(q, k, v, causal, f"Nq{Nq} Nk{Nk} d{d}")
