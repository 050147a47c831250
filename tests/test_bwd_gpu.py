"""GPU parity of the backward pass (fa_bwd) against the fp64 backward oracle.

The GPU gradients use the forward's rounded O and its lse, round P and dS to
the input type before the MFMA products (as the forward rounds P), and round
the outputs; the oracle is exact. The bar is on the error relative to the
largest entry of each gradient tensor (at least 1e-3): <= 2e-2 for bf16 and
<= 3e-3 for fp16, about 8x the input type's unit roundoff (2^-8, 2^-11), which
covers one rounding of P or dS per product and one of the output; measured
errors are 2e-3 to 5e-3 (bf16) and 2e-4 to 7e-4 (fp16).
"""

import random

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_forward_fwd_amd as fa
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float16: 3e-3}


def grads_gpu(q, k, v, dout, causal):
    qd, kd, vd, dd = (t.cuda() for t in (q, k, v, dout))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, splits=1)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dd, causal=causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check_bwd(B, H, N, d, dtype, causal, seed, Nk=None):
    q, k, v = make_qkv(B, H, N, d, dtype, seed)
    if Nk is not None:  # fewer or more keys than queries
        _, k, v = make_qkv(B, H, Nk, d, dtype, seed + 3)
    dout = make_qkv(B, H, N, d, dtype, seed + 7)[0]
    scale = fa.default_scale(d)
    g = grads_gpu(q, k, v, dout, causal)
    ref = oracle.attention_bwd(q, k, v, dout, causal, scale)
    errs = []
    for name, a, b in zip(("dq", "dk", "dv"), g, ref):
        a = a.float().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), f"{name}: non-finite"
        # relative to the tensor's largest entry; the floor keeps exact zeros
        # (dQ and dK of a single key) checked absolutely
        err = float(np.abs(a - b).max() / max(float(np.abs(b).max()), 1e-3))
        errs.append(err)
    print(f"[bwd] B{B} H{H} N{N} Nk{Nk or N} d{d} {dtype} causal={causal} rel err dq={errs[0]:.2e} "
          f"dk={errs[1]:.2e} dv={errs[2]:.2e}", flush=True)
    tol = TOL[q.dtype]
    assert max(errs) <= tol, f"gradient error {max(errs):.3e} > {tol}"
    return g


CASES = [(1, 2, 128, 64, "fp16"), (1, 2, 128, 128, "bf16"), (2, 3, 300, 128, "bf16"),
         (1, 2, 1000, 64, "fp16"), (2, 2, 64, 128, "fp16"), (1, 1, 17, 64, "bf16"),
         (1, 2, 513, 128, "fp16"), (1, 1, 1, 128, "bf16")]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[4]}" for c in CASES])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_oracle(case, causal):
    B, H, N, d, dtype = case
    print(f"[case] bwd {case} causal={causal}", flush=True)
    check_bwd(B, H, N, d, dtype, causal, 500 + N)


def test_backward_deterministic():
    q, k, v = (t.cuda() for t in make_qkv(2, 4, 700, 128, "bf16", 520))
    dout = make_qkv(2, 4, 700, 128, "bf16", 527)[0].cuda()
    for causal in (False, True):
        o, lse = fa.fwd(q, k, v, causal=causal)
        a = fa.bwd(q, k, v, o, lse, dout, causal=causal)
        b = fa.bwd(q, k, v, o, lse, dout, causal=causal)
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_headline_shape_four_heads():
    # the headline shape B=4 H=16 N=4096 d=128 bf16 on the GPU, checked on one
    # head of each batch, at different head indices (the oracle's full
    # backward of all 64 heads would take minutes)
    B, H, N, d = 4, 16, 4096, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", 530)
    dout = make_qkv(B, H, N, d, "bf16", 537)[0]
    for causal in (False, True):
        g = grads_gpu(q, k, v, dout, causal)
        for b, h in ((0, 0), (1, 5), (2, 10), (3, 15)):
            sl = (slice(b, b + 1), slice(h, h + 1))
            ref = oracle.attention_bwd(q[sl], k[sl], v[sl], dout[sl], causal, fa.default_scale(d))
            for name, a, r in zip(("dq", "dk", "dv"), g, ref):
                a = a[sl].float().numpy().astype(np.float64)
                err = float(np.abs(a - r).max() / max(float(np.abs(r).max()), 1e-3))
                print(f"[bwd] headline head ({b},{h}) causal={causal} {name} rel err {err:.2e}", flush=True)
                assert err <= TOL[torch.bfloat16]


# (B, H, Nq, Nk, d, dtype): cross-attention shapes, ragged both ways, a key
# block wholly past every causal row, and a single query
QK_CASES = [(2, 2, 300, 1000, 128, "bf16"), (2, 2, 1000, 300, 64, "fp16"), (1, 3, 129, 700, 64, "bf16"),
            (1, 2, 700, 129, 128, "fp16"), (1, 2, 1, 513, 128, "bf16"), (1, 1, 64, 1024, 64, "fp16")]


@pytest.mark.parametrize("case", QK_CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{c[5]}" for c in QK_CASES])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_query_and_key_lengths(case, causal):
    B, H, Nq, Nk, d, dtype = case
    print(f"[case] bwd {case} causal={causal}", flush=True)
    dq, dk, dv = check_bwd(B, H, Nq, d, dtype, causal, 540 + Nq % 50, Nk=Nk)
    if causal and Nq < Nk:  # keys past the last query row are seen by no row
        assert torch.all(dk[:, :, Nq:] == 0) and torch.all(dv[:, :, Nq:] == 0)


# (B, H, Nq, Nk, d, dtype, causal, window_left, window_right, key_lens): the
# masks of fa_fwd_masked through the forward and fa_bwd_masked
MASK_CASES = [(3, 2, 500, 500, 128, "bf16", False, -1, -1, [500, 250, 0]),
              (1, 2, 700, 700, 128, "bf16", True, 100, -1, None),
              (2, 2, 600, 600, 64, "fp16", False, 64, 64, None),
              (2, 1, 600, 600, 128, "fp16", True, 50, -1, [600, 300]),
              (2, 2, 300, 1000, 64, "bf16", False, -1, 200, [1000, 400]),
              (1, 2, 1000, 300, 128, "fp16", True, 120, -1, [300]),
              (8, 4, 333, 333, 128, "bf16", False, -1, -1, [333, 1, 64, 65, 300, 0, 200, 333])]


@pytest.mark.parametrize("case", MASK_CASES, ids=[f"q{c[2]}k{c[3]}d{c[4]}{c[5]}c{int(c[6])}wl{c[7]}wr{c[8]}"
                                                  for c in MASK_CASES])
def test_backward_masks_match_oracle(case):
    B, H, Nq, Nk, d, dtype, causal, wl, wr, kl = case
    print(f"[case] bwd masks {case}", flush=True)
    q = make_qkv(B, H, Nq, d, dtype, 560 + Nq % 40)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, 563 + Nq % 40)
    dout = make_qkv(B, H, Nq, d, dtype, 567 + Nq % 40)[0]
    scale = fa.default_scale(d)
    qd, kd, vd, dd = (t.cuda() for t in (q, k, v, dout))
    mk = dict(window_left=wl, window_right=wr, key_lens=kl)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, splits=1, **mk)
    g = [t.cpu() for t in fa.bwd(qd, kd, vd, o, lse, dd, causal=causal, **mk)]
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, dout, causal, scale, **mk)
    # structural zeros: rows that see no key (dQ) and keys that no row sees (dK, dV)
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    vis = np.ones((B, Nq, Nk), dtype=bool)
    if wl >= 0:
        vis &= (j >= i - wl)[None]
    vis &= (j <= i)[None] if causal else ((j <= i + wr)[None] if wr >= 0 else True)
    if kl is not None:
        vis &= np.arange(Nk)[None, None, :] < np.asarray(kl)[:, None, None]
    no_key = ~vis.any(axis=2)      # [B, Nq]
    no_row = ~vis.any(axis=1)      # [B, Nk]
    errs = []
    for name, a, b in zip(("dq", "dk", "dv"), g, ref):
        a = a.float().numpy().astype(np.float64)
        assert np.all(np.isfinite(a)), f"{name}: non-finite"
        errs.append(float(np.abs(a - b).max() / max(float(np.abs(b).max()), 1e-3)))
        zero = no_key if name == "dq" else no_row
        assert np.all(a[zero[:, None, :].repeat(H, axis=1)] == 0), f"{name}: nonzero gradient of an unseen row or key"
    print(f"[bwd] masks {case[:7]} wl={wl} wr={wr} rel err dq={errs[0]:.2e} dk={errs[1]:.2e} "
          f"dv={errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL[q.dtype]


# head dims other than 64 and 128 (a multiple of 8 up to 128): the d = 64 or
# d = 128 kernels with the missing dims held at zero
HDIM_CASES = [(2, 2, 300, 300, 8, "bf16"), (1, 3, 257, 257, 32, "fp16"), (2, 2, 333, 333, 40, "bf16"),
              (1, 2, 300, 300, 72, "fp16"), (2, 2, 500, 500, 96, "bf16"), (1, 2, 129, 129, 120, "fp16"),
              (2, 2, 300, 1000, 96, "bf16"), (1, 2, 700, 129, 48, "fp16")]


@pytest.mark.parametrize("case", HDIM_CASES, ids=[f"q{c[2]}k{c[3]}d{c[4]}{c[5]}" for c in HDIM_CASES])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_head_dims_match_oracle(case, causal):
    B, H, Nq, Nk, d, dtype = case
    print(f"[case] bwd head dim {case} causal={causal}", flush=True)
    check_bwd(B, H, Nq, d, dtype, causal, 580 + d, Nk=None if Nk == Nq else Nk)


@pytest.mark.parametrize("d,D", [(96, 128), (40, 64), (120, 128), (8, 64)])
def test_backward_head_dim_equals_the_native_kernel_on_zero_padded_inputs(d, D):
    # same tiles, same LDS contents and the same MFMA sums: bit for bit, and
    # the native kernel's gradients past d are zero. Both backward calls take
    # the same O and lse (the native forward's), so only the backward is
    # compared (the forward at 96 computed dims adds its row sums in another
    # order than the d = 128 kernel)
    B, H, N = 2, 3, 333
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, "bf16", 600 + d))
    dout = make_qkv(B, H, N, d, "bf16", 607 + d)[0].cuda()
    pad = lambda t: torch.nn.functional.pad(t, (0, D - d)).contiguous()
    sc = fa.default_scale(d)  # the padded calls take d's scale, not D's
    for causal in (False, True):
        o_n, lse_n = fa.fwd(pad(q), pad(k), pad(v), causal=causal, scale=sc, splits=1)
        g = fa.bwd(q, k, v, o_n[..., :d].contiguous(), lse_n, dout, causal=causal, scale=sc)
        g_n = fa.bwd(pad(q), pad(k), pad(v), o_n, lse_n, pad(dout), causal=causal, scale=sc)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), g, g_n):
            assert torch.equal(a, b[..., :d]), (d, causal, name)
            assert torch.all(b[..., d:] == 0), (d, causal, name)


def test_backward_head_dim_masks_and_guard_regions():
    # masks at d = 96 through the C entry point, each output followed by a NaN
    # guard that no store may touch
    B, H, Nq, Nk, d = 2, 2, 600, 600, 96
    q = make_qkv(B, H, Nq, d, "fp16", 620)[0]
    _, k, v = make_qkv(B, H, Nk, d, "fp16", 621)
    dout = make_qkv(B, H, Nq, d, "fp16", 622)[0]
    scale = fa.default_scale(d)
    mk = dict(window_left=50, window_right=-1, key_lens=[600, 300])
    qd, kd, vd, dd = (t.cuda() for t in (q, k, v, dout))
    o, lse = fa.fwd(qd, kd, vd, causal=True, splits=1, **mk)
    outs = []
    for t in (qd, kd, vd):
        base = torch.full((t.numel() + 4096,), float("nan"), dtype=t.dtype, device="cuda")
        outs.append((base, base[:t.numel()].view(t.shape)))
    delta = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    kl = torch.tensor(mk["key_lens"], dtype=torch.int32, device="cuda")
    rc = fa.fa_bwd_masked(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dd.data_ptr(),
                          lse.data_ptr(), outs[0][1].data_ptr(), outs[1][1].data_ptr(), outs[2][1].data_ptr(),
                          delta.data_ptr(), B, H, Nq, Nk, d, 1, 50, -1, kl.data_ptr(), scale,
                          fa.dtype_code(q.dtype), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == fa.FA_OK, fa.fa_status_string(rc)
    ref = oracle.attention_bwd(q, k, v, dout, True, scale, **mk)
    for name, (base, g), r in zip(("dq", "dk", "dv"), outs, ref):
        assert torch.isnan(base[g.numel():]).all(), f"{name}: write past the output"
        a = g.cpu().float().numpy().astype(np.float64)
        err = float(np.abs(a - r).max() / max(float(np.abs(r).max()), 1e-3))
        print(f"[bwd] d96 masks {name} rel err {err:.2e}", flush=True)
        assert err <= TOL[torch.float16]
    # keys past a batch's length get zero gradients
    assert torch.all(outs[1][1][1, :, 300:] == 0) and torch.all(outs[2][1][1, :, 300:] == 0)


def draw_bwd_cases(n, seed):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        B, H = rng.choice([1, 2, 3]), rng.choice([1, 2, 4])
        Nq = rng.choice([1, 31, 64, 100, 257, 600])
        Nk = rng.choice([1, 33, 64, 200, 511, 900])
        d = rng.choice([16, 24, 40, 64, 80, 96, 128])
        dtype = rng.choice(["bf16", "fp16"])
        causal = rng.random() < 0.5
        if B * H * Nq * Nk > 4_000_000:
            continue
        cases.append((B, H, Nq, Nk, d, dtype, causal))
    return cases


RANDOM_CASES = draw_bwd_cases(16, 2027)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}{c[5]}{'c' if c[6] else ''}"
                                                    for c in RANDOM_CASES])
def test_backward_random_shapes(case):
    # seeded random shapes: ragged query and key counts both ways, every
    # head-dim class, both input types and flags
    B, H, Nq, Nk, d, dtype, causal = case
    print(f"[case] bwd random {case}", flush=True)
    check_bwd(B, H, Nq, d, dtype, causal, 580 + Nq % 70, Nk=Nk)
