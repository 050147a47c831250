"""GPU parity of the fp32 forward (fa_fwd_f32) against the fp64 oracle.

fa_fwd_f32 forms every product of Q K^T and P V from bf16 hi/lo parts
(hi*hi + hi*lo + lo*hi), about 16 significant bits per product. The bar is
max |O - O_64| <= 1e-4 and |d lse| <= 5e-5 * max(1, |lse_64|): with N(0,1)
inputs the split products alone err by at most 1.5e-5 on O and 7.4e-6 on lse
at N = 1000 (fp64 simulation of the split), and the bar lies well below what
bf16-rounded inputs give (1e-3 to 8e-3; tests/test_f32_tolerance.py checks
that on the CPU).
"""

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_forward_fwd_amd as fa
from fa_inputs import make_qkv, sample_rows

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-4, 5e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()


def qk_inputs(B, H, Nq, Nk, d, seed):
    q = make_qkv(B, H, Nq, d, "fp32", seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, "fp32", seed + 1)
    return q, k, v


def check(q, k, v, causal, rows=None, label=""):
    scale = fa.default_scale(q.shape[-1])
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert o.dtype == torch.float32
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale, rows=rows)
    og, lg = o.numpy().astype(np.float64), lse.numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    err_o = float(np.abs(og - o64).max())
    err_l = float((np.abs(lg - l64) / np.maximum(1.0, np.abs(l64))).max())
    print(f"[parity] fp32 {label} causal={causal} max|dO|={err_o:.3e} max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O, f"{label}: O error {err_o:.3e}"
    assert err_l <= TOL_LSE, f"{label}: lse error {err_l:.3e}"


def test_pages_fp32_case():
    # the test id that failed on the page: one batch, 200 queries, 96 keys,
    # D = 128, non-causal, fp32 inputs
    q, k, v = qk_inputs(1, 1, 200, 96, 128, 400)
    check(q, k, v, False, label="B1 Nq200 Nk96 d128")
    check(q, k, v, True, label="B1 Nq200 Nk96 d128")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 129, 1000, 1025])
def test_f32_lengths(N, d):
    q, k, v = make_qkv(2, 2, N, d, "fp32", 410 + N)
    for causal in (False, True):
        check(q, k, v, causal, label=f"N={N} d={d}")


@pytest.mark.parametrize("Nq,Nk", [(300, 1000), (1000, 300), (1, 4096)])
def test_f32_query_and_key_lengths(Nq, Nk):
    q, k, v = qk_inputs(2, 3, Nq, Nk, 128, 420)
    for causal in (False, True):
        check(q, k, v, causal, label=f"Nq={Nq} Nk={Nk}")


def test_f32_headline_shape_sampled():
    q, k, v = make_qkv(4, 16, 4096, 128, "fp32", 430)
    for causal in (False, True):
        check(q, k, v, causal, rows=sample_rows(4096), label="B4 H16 N4096 d128")


def test_f32_deterministic_and_workspace_checked():
    q, k, v = (t.cuda() for t in make_qkv(1, 4, 700, 64, "fp32", 440))
    a = fa.fwd(q, k, v, causal=True)
    b = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    need = fa.fa_f32_workspace_bytes(1, 4, 700, 64)
    assert need == 8 * 4 * 700 * 64
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, workspace=torch.empty(need // 2 - 1, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, key_lens=[100])
    with pytest.raises(fa.FaError):
        q96 = torch.zeros(1, 1, 16, 96, device="cuda")
        fa.fwd(q96, q96, q96)
