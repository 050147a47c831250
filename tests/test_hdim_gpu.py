"""GPU parity at head dims other than 64 and 128 (a multiple of 8 up to 128),
which libfa runs with the d = 64 or d = 128 kernel's tiles and the missing
dims held at zero, computing only d rounded up to 32. Checked against the
fp64 oracle at the same tolerances as the other forward tests (4e-3 fp16 /
3.2e-2 bf16 on O, 1e-3 relative on lse), and against the d = 64 / 128 kernel
on the same inputs zero-padded: bit for bit where the arithmetic is the same
(the skipped dims only add zeros), within one output ulp where the row sums
are added in another order (96 computed dims).
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_forward_fwd_amd as fa
from fa_inputs import make_qkv, sample_rows

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 3.2e-2}
TOL_LSE = 1e-3
DIMS = [8, 16, 32, 40, 48, 56, 72, 80, 96, 112, 120]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()


def qk_inputs(B, H, Nq, Nk, d, dtype, seed):
    q = make_qkv(B, H, Nq, d, dtype, seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed + 1)
    return q, k, v


def guarded_out(shape, dtype):
    """A contiguous output tensor followed by a NaN guard region."""
    n = int(np.prod(shape))
    base = torch.full((n + 4096,), float("nan"), dtype=dtype, device="cuda")
    return base, base[:n].view(shape)


def check(q, k, v, causal, rows=None, label="", **kw):
    d = q.shape[-1]
    scale = fa.default_scale(d)
    base, out = guarded_out(q.shape, q.dtype)
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.isnan(base[out.numel():]).all(), f"{label}: write past the output"
    o, lse = o.cpu(), lse.cpu()
    okw = {key: kw[key] for key in ("window_left", "window_right", "key_lens") if key in kw}
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale, rows=rows, **okw)
    og = o.float().numpy().astype(np.float64)
    lg = lse.numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    fin = np.isfinite(l64)
    assert np.array_equal(np.isfinite(lg), fin) and np.all(og[~fin] == 0)
    err_o = float(np.abs(og - o64).max())
    err_l = float((np.abs(lg[fin] - l64[fin]) / np.maximum(1.0, np.abs(l64[fin]))).max()) if fin.any() else 0.0
    print(f"[parity] hdim {label} causal={causal} max|dO|={err_o:.3e} max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[q.dtype], f"{label}: O error {err_o:.3e}"
    assert err_l <= TOL_LSE, f"{label}: lse error {err_l:.3e}"
    if causal and not okw:
        assert torch.equal(o[:, :, 0], v[:, :, 0])
    return o, lse


@pytest.mark.parametrize("d", DIMS)
def test_head_dim_parity(d):
    dtype = "bf16" if d % 16 else "fp16"
    print(f"[case] d={d} {dtype}", flush=True)
    q, k, v = qk_inputs(2, 3, 333, 333, d, dtype, 300 + d)
    for causal in (False, True):
        check(q, k, v, causal, label=f"d={d} N=333 {dtype}")


@pytest.mark.parametrize("d,D", [(96, 128), (72, 128), (40, 64), (120, 128), (8, 64), (32, 64)])
def test_equals_the_native_kernel_on_zero_padded_inputs(d, D):
    # 96 computed dims sum each row per 32-key block (the d = 64 order), the
    # d = 128 kernel over all 64 keys of a tile: the fp32 row sums then differ
    # in their last bits, which moves an output by at most one bf16 ulp
    same_order = -(-d // 32) * 32 != 96
    # large enough for the 256-row non-causal shape, ragged in N
    for B, H, N in ((8, 16, 1000), (1, 2, 257)):
        q, k, v = make_qkv(B, H, N, d, "bf16", 310 + d)
        pad = lambda t: torch.nn.functional.pad(t, (0, D - d)).contiguous().cuda()
        scale = fa.default_scale(d)
        for causal in (False, True):
            o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
            o_n, lse_n = fa.fwd(pad(q), pad(k), pad(v), causal=causal, scale=scale)
            torch.cuda.synchronize()
            o_n = o_n[..., :d]
            if same_order:
                assert torch.equal(o, o_n) and torch.equal(lse, lse_n), (d, B, H, N, causal)
            else:
                a, b = o.float(), o_n.float()
                assert bool(((a - b).abs() <= 2.0 ** -7 * b.abs()).all()), (d, B, H, N, causal)
                assert float((lse - lse_n).abs().max()) <= 1e-5, (d, B, H, N, causal)


@pytest.mark.parametrize("d,dtype", [(96, "bf16"), (48, "fp16")])
def test_head_dim_query_and_key_lengths(d, dtype):
    q, k, v = qk_inputs(2, 2, 300, 1000, d, dtype, 320)
    for causal in (False, True):
        check(q, k, v, causal, label=f"d={d} Nq=300 Nk=1000")


@pytest.mark.parametrize("d", [80, 40])
def test_head_dim_split_decode(d):
    B, H, Nq, Nk = 4, 8, 1, 8192
    q, k, v = qk_inputs(B, H, Nq, Nk, d, "bf16", 330)
    splits = fa.fa_split_count(B, H, Nq, Nk, d, 0)
    assert splits > 1
    check(q, k, v, False, label=f"d={d} decode s{splits}", splits=splits)
    check(q, k, v, False, label=f"d={d} decode padded s{splits}", splits=splits, key_lens=[8192, 5000, 1, 0])


@pytest.mark.parametrize("d", [96, 24])
def test_head_dim_masks(d):
    q, k, v = make_qkv(2, 2, 700, d, "fp16", 340)
    check(q, k, v, True, label=f"d={d} window 100", window_left=100)
    check(q, k, v, False, label=f"d={d} padding", key_lens=[700, 313])
    check(q, k, v, True, label=f"d={d} window+padding", window_left=50, key_lens=[700, 300])


def test_head_dim_96_headline_shape_sampled():
    B, H, N, d = 4, 16, 4096, 96
    q, k, v = make_qkv(B, H, N, d, "bf16", 350)
    rows = sample_rows(N)
    for causal in (False, True):
        check(q, k, v, causal, rows=rows, label="B4 H16 N4096 d96")
