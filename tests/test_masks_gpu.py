"""GPU parity of padding masks and sliding windows (fa_fwd_masked and
fa_fwd_split_masked) against the masked fp64 oracle on the same seeded inputs.

Tolerances are those of the unmasked forward: max |O_gpu - O_64| <= 4e-3 for
fp16 and <= 3.2e-2 for bf16, lse within 1e-3 relative (|d lse| <= 1e-3 *
max(1, |lse_64|)). A row that sees no key must come back as O = 0 exactly and
lse = -inf exactly, never NaN.
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


def run_masked(q, k, v, causal, wl=-1, wr=-1, key_lens=None, splits=1, scale=None):
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, splits=splits,
                    window_left=wl, window_right=wr, key_lens=key_lens)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_masked(q, k, v, causal, wl=-1, wr=-1, key_lens=None, splits=1, rows=None, label=""):
    d = q.shape[-1]
    scale = fa.default_scale(d)
    o, lse = run_masked(q, k, v, causal, wl, wr, key_lens, splits, scale)
    o64, l64 = oracle.attention_fwd(q, k, v, causal, scale, rows=rows, window_left=wl,
                                    window_right=wr, key_lens=key_lens)
    og = o.float().numpy().astype(np.float64)
    lg = lse.numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    empty = ~np.isfinite(l64)
    assert np.all(l64[empty] == -np.inf)
    assert np.array_equal(lg == -np.inf, empty), f"{label}: rows with no visible key differ"
    assert np.all(og[empty] == 0.0), f"{label}: a row with no visible key has O != 0"
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg[~empty])), f"{label}: non-finite output"
    err_o = float(np.abs(og - o64).max()) if og.size else 0.0
    fin = ~empty
    err_l = float((np.abs(lg[fin] - l64[fin]) / np.maximum(1.0, np.abs(l64[fin]))).max()) if fin.any() else 0.0
    print(f"[parity] masked {label} causal={causal} wl={wl} wr={wr} empty rows={int(empty.sum())} "
          f"max|dO|={err_o:.3e} max rel dlse={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[q.dtype], f"{label}: O error {err_o:.3e}"
    assert err_l <= TOL_LSE, f"{label}: lse error {err_l:.3e}"
    return o, lse


# (label, B, H, Nq, Nk, d, dtype, causal, window_left, window_right, key_lens)
CASES = [
    ("padding nc d128", 4, 2, 1000, 1000, 128, "bf16", False, -1, -1, [1000, 777, 64, 1]),
    ("padding causal d64 with an empty batch", 4, 2, 1000, 1000, 64, "fp16", True, -1, -1, [1000, 500, 0, 129]),
    ("sliding window 256 causal d128", 2, 4, 2048, 2048, 128, "bf16", True, 255, -1, None),
    ("sliding window 101 causal d64 ragged", 1, 3, 1025, 1025, 64, "fp16", True, 100, -1, None),
    ("band 64/64 nc d128", 2, 2, 700, 700, 128, "fp16", False, 64, 64, None),
    ("window + padding leaves rows empty", 2, 2, 600, 600, 128, "bf16", True, 50, -1, [600, 300]),
    ("right window only nc d64", 1, 2, 500, 500, 64, "bf16", False, -1, 0, None),
    ("Nq < Nk band + padding", 2, 2, 300, 1000, 128, "bf16", False, -1, 200, [1000, 400]),
    ("Nq > Nk causal window + padding", 2, 2, 1000, 300, 64, "fp16", True, 120, -1, [300, 77]),
    ("8-wave d64 padding", 8, 16, 1000, 1000, 64, "bf16", False, -1, -1, [1000, 999, 513, 512, 511, 65, 64, 2]),
    ("large grid d128 padding", 8, 16, 1000, 1000, 128, "bf16", False, 300, -1, [1000, 640, 333, 1, 1000, 900, 128, 700]),
    ("tiny", 1, 1, 1, 1, 128, "bf16", True, 0, -1, [1]),
    ("tiny empty", 1, 1, 5, 3, 64, "fp16", False, -1, -1, [0]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].replace(" ", "_") for c in CASES])
def test_masked_parity(case):
    label, B, H, Nq, Nk, d, dtype, causal, wl, wr, kl = case
    print(f"[case] {label}", flush=True)
    q, k, v = qk_inputs(B, H, Nq, Nk, d, dtype, 200 + Nq % 97)
    check_masked(q, k, v, causal, wl, wr, kl, label=label)


@pytest.mark.parametrize("d,dtype", [(64, "fp16"), (128, "bf16")])
def test_window_zero_returns_values_bitwise(d, dtype):
    # causal with window 0: row i sees key i alone, so P = 1 and O_i = V_i exactly
    q, k, v = make_qkv(2, 3, 777, d, dtype, 210)
    o, lse = run_masked(q, k, v, True, wl=0)
    assert torch.equal(o, v)


def test_padding_equals_truncated_keys_bitwise():
    # a padding length L gives what the unmasked kernel gives on the first L
    # keys (same workgroup shape and exp path at d = 64; 20 heads keep both
    # grids 4-wave and the unmasked one off the key-split kernel)
    B, H, N, d = 3, 20, 900, 64
    q, k, v = make_qkv(B, H, N, d, "fp16", 220)
    lens = [900, 450, 63]
    for causal in (False, True):
        o, lse = run_masked(q, k, v, causal, key_lens=lens)
        for b, L in enumerate(lens):
            o_t, l_t = fa.fwd(q[b:b + 1].cuda(), k[b:b + 1, :, :L].contiguous().cuda(),
                              v[b:b + 1, :, :L].contiguous().cuda(), causal=causal, splits=1)
            assert torch.equal(o[b:b + 1], o_t.cpu()) and torch.equal(lse[b:b + 1], l_t.cpu()), (causal, L)


def test_wide_window_equals_no_window():
    # 10 heads: the unmasked launch takes the direct kernel, not the key split
    for d, dtype in ((64, "fp16"), (128, "bf16")):
        q, k, v = make_qkv(2, 10, 1000, d, dtype, 230 + d)
        for causal in (False, True):
            o_n, l_n = run_masked(q, k, v, causal)
            o_w, l_w = run_masked(q, k, v, causal, wl=5000, wr=5000)
            if d == 64:  # same workgroup shape and exp path: bit for bit
                assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w)
            else:
                assert (o_n.float() - o_w.float()).abs().max() <= TOL_O[q.dtype]
                assert (l_n - l_w).abs().max() <= 1e-5


def test_key_lens_are_clamped():
    q, k, v = qk_inputs(3, 2, 100, 300, 64, "bf16", 240)
    a = run_masked(q, k, v, False, key_lens=[-7, 300 + 50, 120])
    b = run_masked(q, k, v, False, key_lens=[0, 300, 120])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.all(a[1][0] == -float("inf")) and torch.all(a[0][0] == 0)


def test_key_lens_tensor_on_the_gpu():
    q, k, v = qk_inputs(2, 2, 64, 640, 128, "bf16", 245)
    kl = torch.tensor([640, 100], dtype=torch.int32, device="cuda")
    a = run_masked(q, k, v, False, key_lens=kl)
    b = run_masked(q, k, v, False, key_lens=[640, 100])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    with pytest.raises(ValueError):
        run_masked(q, k, v, False, key_lens=kl.to(torch.int64))


# (label, B, H, Nq, Nk, d, dtype, causal, wl, wr, key_lens, splits): decode over
# caches of different lengths, one of them empty, and chunked bands
SPLIT_CASES = [
    ("decode padded caches", 4, 8, 1, 16384, 128, "bf16", False, -1, -1, [16384, 9000, 1, 0], None),
    ("decode padded d64", 3, 4, 7, 4096, 64, "fp16", False, -1, -1, [4096, 100, 2049], None),
    ("split band + padding", 2, 2, 33, 5000, 128, "bf16", False, -1, 3000, [5000, 2500], 4),
    ("split causal window", 1, 2, 300, 1000, 64, "bf16", True, 200, -1, [1000], 3),
    ("split window + padding, empty chunks", 2, 2, 300, 1000, 128, "fp16", False, 100, 40, [1000, 10], 16),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0].replace(" ", "_") for c in SPLIT_CASES])
def test_split_masked_parity(case):
    label, B, H, Nq, Nk, d, dtype, causal, wl, wr, kl, splits = case
    if splits is None:
        splits = fa.fa_split_count(B, H, Nq, Nk, d, int(causal))
        assert splits > 1
    print(f"[case] split {label} splits={splits}", flush=True)
    q, k, v = qk_inputs(B, H, Nq, Nk, d, dtype, 250 + Nq % 31)
    check_masked(q, k, v, causal, wl, wr, kl, splits=splits, label=f"{label} s{splits}")


def test_sliding_window_long_sequence_sampled():
    # long causal sequence with a 4096-key window, in the launch the sweep
    # times; sampled rows against the oracle
    B, H, N, d = 1, 16, 16384, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", 260)
    check_masked(q, k, v, True, wl=4095, rows=sample_rows(N), label="N16384 window 4096")


def test_padded_batch_headline_shape_sampled():
    B, H, N, d = 4, 16, 4096, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", 270)
    check_masked(q, k, v, False, key_lens=[4096, 3072, 2048, 1024], rows=sample_rows(N),
                 label="B4 H16 N4096 padded")
