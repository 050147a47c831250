"""Pins for the fp64 oracle: checks against facts other than the oracle itself.

Each pin takes ``fwd`` (a callable with the signature of
``oracle.attention_fwd``) and raises ``AssertionError`` when the oracle
disagrees with what the pages and the mathematics fix. They are run against
the real oracle in ``test_oracle_pins.py`` and against deliberately broken
copies of it in ``test_oracle_mutants.py`` (every broken copy must fail at
least one pin).

What pins what:
  decimal_bruteforce   the definition itself, at 50 digits, on tiny shapes
  torch_sdpa           a library routine computing the same definition (fp64)
  keys_zero            closed form: uniform softmax, O = mean of visible V, lse = ln|J|
  causal_row0          row 0 attends only to itself: O_0 = V_0 exactly
  causal_last_row      causal row N-1 sees every key: equals the non-causal row
  prefix_truncation    causal rows < N' do not depend on keys >= N'
  v_ones               rows of the softmax sum to one
  v_identity           O = P when V = I; checked against scipy's softmax
  online_equals_twopass  the online-softmax identity, several tile sizes
  linearity            O is linear in V
  permutation          non-causal O is invariant to permuting keys with values
  single_key           N = 1: O = V, lse = s_00
  shift                adding a vector to every key shifts each row's scores
                       by a constant: O unchanged, lse shifted (also needs the
                       max subtraction at scores of several thousand)
  qk_decimal_bruteforce  Nq != Nk: the definition at 50 digits, including the
                       shapes "Programming an attention kernel in Triton"
                       validates in "Kernel 4" (5 x 15 and 1 x 10 keys)
  qk_torch_sdpa        Nq != Nk against the library routine, whose causal mask
                       is also aligned at the top-left corner
  qk_square_prefix     causal Nq < Nk: rows equal the first Nq rows of the
                       square problem (the diagonal starts at the top left)
  qk_rows_past_keys    causal Nq > Nk: every row i >= Nk - 1 sees all keys and
                       equals the non-causal row
  masked_decimal       padding and sliding-window masks against the definition
                       at 50 digits, including rows with no visible key
                       (O = 0, lse = -inf)
  masked_torch         the same masks as an explicit boolean matrix built with
                       broadcast comparisons, fp64 masked softmax in torch
  padding_is_truncation  a padding length L per batch equals attention over
                       the first L keys only, bit for bit
  wide_window_is_none  a window at least as wide as the keys equals no window,
                       bit for bit
"""

from decimal import Decimal, getcontext

import numpy as np
import scipy.special
import torch

from fa_inputs import make_qkv


def _f(x):
    return x.float().numpy().astype(np.float64) if hasattr(x, "float") else np.asarray(x, np.float64)


def _close(a, b, rtol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= rtol, f"{what}: max scaled error {err:.3e} > {rtol:.1e}"


def _visible(i, Nk, causal, wl=-1, wr=-1, klen=None):
    """Visible keys of row i as a Python list, straight from the mask rules."""
    return [j for j in range(Nk)
            if (klen is None or j < klen) and (wl < 0 or j >= i - wl)
            and (j <= i if causal else (wr < 0 or j <= i + wr))]


def _decimal_attention(q, k, v, causal, scale, wl=-1, wr=-1, klen=None):
    """Attention of one head, q [Nq, d] and k, v [Nk, d] float inputs, evaluated in
    50-digit decimal. A causal row i sees keys j <= i; a row with no visible key
    gives O = 0 and lse = -inf."""
    getcontext().prec = 50
    N, d = q.shape
    Nk = k.shape[0]
    Q = [[Decimal(float(x)) for x in row] for row in q]
    K = [[Decimal(float(x)) for x in row] for row in k]
    V = [[Decimal(float(x)) for x in row] for row in v]
    sc = Decimal(float(scale))
    o = np.zeros((N, d))
    lse = np.zeros(N)
    for i in range(N):
        J = _visible(i, Nk, causal, wl, wr, klen)
        if not J:
            lse[i] = -np.inf
            continue
        s = [sc * sum(Q[i][c] * K[j][c] for c in range(d)) for j in J]
        e = [x.exp() for x in s]
        den = sum(e)
        for c in range(d):
            o[i, c] = float(sum(e[t] * V[j][c] for t, j in enumerate(J)) / den)
        lse[i] = float(den.ln())
    return o, lse


def decimal_bruteforce(fwd):
    for seed, (B, H, N, d) in enumerate([(1, 1, 1, 4), (1, 1, 5, 3), (2, 2, 8, 8), (1, 3, 7, 1)]):
        q, k, v = make_qkv(B, H, N, d, "fp16", 100 + seed)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, scale)
            for b in range(B):
                for h in range(H):
                    od, ld = _decimal_attention(_f(q[b, h]), _f(k[b, h]), _f(v[b, h]), causal, scale)
                    _close(o[b, h], od, 1e-14, f"decimal O {B,H,N,d} causal={causal}")
                    _close(lse[b, h], ld, 1e-14, f"decimal lse {B,H,N,d} causal={causal}")


def _torch_reference(q, k, v, causal, scale):
    q64, k64, v64 = (t.to(torch.float64) for t in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(q64, k64, v64, is_causal=causal, scale=scale)
    s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def torch_sdpa(fwd):
    for dtype, (B, H, N, d), qs in [("fp16", (2, 3, 67, 16), 1.0), ("bf16", (1, 2, 130, 64), 1.0),
                                   ("bf16", (1, 2, 96, 32), 4.0)]:
        q, k, v = make_qkv(B, H, N, d, dtype, 7, q_scale=qs)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, scale)
            ot, lt = _torch_reference(q, k, v, causal, scale)
            _close(o, ot, 1e-12, f"sdpa O {dtype} {B,H,N,d} q*{qs} causal={causal}")
            _close(lse, lt, 1e-12, f"sdpa lse {dtype} {B,H,N,d} q*{qs} causal={causal}")


def keys_zero(fwd):
    B, H, N, d = 2, 2, 1000, 64
    q, _, v = make_qkv(B, H, N, d, "bf16", 11)
    k = torch.zeros_like(q)
    scale = 0.125
    vf = _f(v)
    counts = np.arange(1, N + 1, dtype=np.float64)
    for causal in (False, True):
        o, lse = fwd(q, k, v, causal, scale)
        if causal:
            mean = np.cumsum(vf, axis=2) / counts[None, None, :, None]
            lse_exp = np.broadcast_to(np.log(counts), (B, H, N))
        else:
            mean = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
            lse_exp = np.full((B, H, N), np.log(N))
        _close(o, mean, 1e-12, f"K=0 mean of V causal={causal}")
        _close(lse, lse_exp, 1e-13, f"K=0 lse = ln|J| causal={causal}")


def causal_row0(fwd):
    for dtype in ("fp16", "bf16"):
        q, k, v = make_qkv(2, 3, 50, 64, dtype, 12)
        scale = 0.125
        o, lse = fwd(q, k, v, True, scale)
        assert np.array_equal(o[:, :, 0, :], _f(v[:, :, 0, :])), "causal row 0 must equal V[0] exactly"
        s00 = scale * np.einsum("bhc,bhc->bh", _f(q[:, :, 0, :]), _f(k[:, :, 0, :]))
        _close(lse[:, :, 0], s00, 1e-14, "causal lse_0 = s_00")


def causal_last_row(fwd):
    q, k, v = make_qkv(1, 2, 333, 64, "fp16", 13)
    o_c, l_c = fwd(q, k, v, True, 0.125)
    o_n, l_n = fwd(q, k, v, False, 0.125)
    assert np.array_equal(o_c[:, :, -1], o_n[:, :, -1]), "causal last row != non-causal last row"
    assert np.array_equal(l_c[:, :, -1], l_n[:, :, -1])
    assert not np.allclose(o_c[:, :, :-1], o_n[:, :, :-1]), "causal and non-causal must differ above"


def prefix_truncation(fwd):
    q, k, v = make_qkv(1, 2, 1024, 64, "bf16", 14)
    o_full, l_full = fwd(q, k, v, True, 0.125)
    n2 = 1000
    o_pre, l_pre = fwd(q[:, :, :n2].contiguous(), k[:, :, :n2].contiguous(), v[:, :, :n2].contiguous(),
                       True, 0.125)
    assert np.array_equal(o_full[:, :, :n2], o_pre), "causal rows < N' depend on keys >= N'"
    assert np.array_equal(l_full[:, :, :n2], l_pre)


def v_ones(fwd):
    q, k, _ = make_qkv(2, 2, 257, 64, "fp16", 15)
    v = torch.ones_like(q)
    for causal in (False, True):
        o, _ = fwd(q, k, v, causal, 0.125)
        _close(o, np.ones_like(o), 1e-14, f"V=1 gives O=1 causal={causal}")


def v_identity(fwd):
    N = d = 64
    q, k, _ = make_qkv(1, 1, N, d, "bf16", 16)
    v = torch.eye(N, dtype=torch.float32).reshape(1, 1, N, N)
    s = 0.125 * (_f(q[0, 0]) @ _f(k[0, 0]).T)
    for causal in (False, True):
        o, _ = fwd(q, k, v, causal, 0.125)
        p = o[0, 0]
        _close(p.sum(axis=1), np.ones(N), 1e-14, f"rows of P sum to 1 causal={causal}")
        sm = s.copy()
        if causal:
            sm[np.triu_indices(N, 1)] = -np.inf
            assert np.all(p[np.triu_indices(N, 1)] == 0.0), "causal P must be 0 above the diagonal"
        _close(p, scipy.special.softmax(sm, axis=1), 1e-13, f"P vs scipy softmax causal={causal}")


def online_equals_twopass(fwd):
    q, k, v = make_qkv(1, 2, 1000, 64, "fp16", 17)
    for causal in (False, True):
        o2, l2 = fwd(q, k, v, causal, 0.125)
        for tn in (1, 7, 16, 64, 128, 1000, 1024):
            ot, lt = fwd(q, k, v, causal, 0.125, tile_n=tn)
            _close(ot, o2, 1e-12, f"online (tile {tn}) vs two-pass O causal={causal}")
            _close(lt, l2, 1e-12, f"online (tile {tn}) vs two-pass lse causal={causal}")


def linearity(fwd):
    g = torch.Generator().manual_seed(18)
    q, k, _ = make_qkv(1, 2, 200, 32, "fp16", 18)
    v1 = torch.randint(-8, 9, (1, 2, 200, 32), generator=g).float()
    v2 = torch.randint(-8, 9, (1, 2, 200, 32), generator=g).float()
    for causal in (False, True):
        o1, _ = fwd(q, k, v1, causal, 0.125)
        o2, _ = fwd(q, k, v2, causal, 0.125)
        o3, _ = fwd(q, k, 3 * v1 - 2 * v2, causal, 0.125)
        _close(o3, 3 * o1 - 2 * o2, 1e-12, f"linearity in V causal={causal}")


def permutation(fwd):
    q, k, v = make_qkv(1, 2, 300, 64, "bf16", 19)
    g = torch.Generator().manual_seed(19)
    perm = torch.randperm(300, generator=g)
    o, lse = fwd(q, k, v, False, 0.125)
    o_k, lse_k = fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, 0.125)
    _close(o_k, o, 1e-13, "permuting keys with values leaves O unchanged")
    _close(lse_k, lse, 1e-13, "permuting keys with values leaves lse unchanged")
    o_q, lse_q = fwd(q[:, :, perm].contiguous(), k, v, False, 0.125)
    assert np.array_equal(o_q, o[:, :, perm.numpy()]), "permuting queries must permute O rows"
    assert np.array_equal(lse_q, lse[:, :, perm.numpy()])


def single_key(fwd):
    q, k, v = make_qkv(2, 2, 1, 64, "fp16", 20)
    for causal in (False, True):
        o, lse = fwd(q, k, v, causal, 0.125)
        assert np.array_equal(o, _f(v)), "N=1: O must equal V"
        s00 = 0.125 * np.einsum("bhnc,bhnc->bhn", _f(q), _f(k))
        _close(lse, s00, 1e-14, "N=1: lse = s_00")


def shift(fwd):
    g = torch.Generator().manual_seed(21)
    B, H, N, d = 1, 2, 96, 64
    # values on a 1/8 grid: every product and sum below is exact in double
    q = torch.round(torch.randn(B, H, N, d, generator=g) * 8) / 8
    k = torch.round(torch.randn(B, H, N, d, generator=g) * 8) / 8
    v = torch.randn(B, H, N, d, generator=g)
    for mag in (1.0, 4096.0):
        u = torch.round(torch.randn(d, generator=g) * 4) / 4 * mag
        qu = 0.125 * (_f(q) @ _f(u))  # [B, H, N]: the per-row constant added to the scores
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, 0.125)
            o_s, lse_s = fwd(q, k + u, v, causal, 0.125)
            _close(o_s, o, 1e-12, f"shifted keys leave O unchanged (|u|~{mag}) causal={causal}")
            _close(lse_s, lse + qu, 1e-12, f"shifted keys shift lse (|u|~{mag}) causal={causal}")


def _qk_inputs(B, H, Nq, Nk, d, dtype, seed, q_scale=1.0):
    q = make_qkv(B, H, Nq, d, dtype, seed, q_scale=q_scale)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed + 1)
    return q, k, v


def qk_decimal_bruteforce(fwd):
    shapes = [(1, 1, 5, 15, 32), (1, 1, 1, 10, 64), (2, 1, 9, 4, 3), (1, 2, 3, 8, 4)]
    for seed, (B, H, Nq, Nk, d) in enumerate(shapes):
        q, k, v = _qk_inputs(B, H, Nq, Nk, d, "bf16", 300 + 2 * seed)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, scale)
            for b in range(B):
                for h in range(H):
                    od, ld = _decimal_attention(_f(q[b, h]), _f(k[b, h]), _f(v[b, h]), causal, scale)
                    _close(o[b, h], od, 1e-14, f"decimal O Nq={Nq} Nk={Nk} causal={causal}")
                    _close(lse[b, h], ld, 1e-14, f"decimal lse Nq={Nq} Nk={Nk} causal={causal}")


def qk_torch_sdpa(fwd):
    for B, H, Nq, Nk, d in [(2, 3, 37, 130, 16), (1, 2, 200, 70, 64), (3, 1, 1, 257, 32)]:
        q, k, v = _qk_inputs(B, H, Nq, Nk, d, "fp16", 400 + Nq)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        q64, k64, v64 = (t.to(torch.float64) for t in (q, k, v))
        s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * scale
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, scale)
            ot = torch.nn.functional.scaled_dot_product_attention(q64, k64, v64, is_causal=causal,
                                                                  scale=scale)
            sm = s.masked_fill(torch.ones(Nq, Nk, dtype=torch.bool).triu(1), float("-inf")) if causal else s
            _close(o, ot.numpy(), 1e-12, f"sdpa O Nq={Nq} Nk={Nk} causal={causal}")
            _close(lse, torch.logsumexp(sm, dim=-1).numpy(), 1e-12, f"sdpa lse Nq={Nq} Nk={Nk} causal={causal}")


def qk_square_prefix(fwd):
    B, H, Nq, Nk, d = 2, 2, 50, 180, 32
    q_sq, k, v = make_qkv(B, H, Nk, d, "bf16", 500)
    q = q_sq[:, :, :Nq].contiguous()
    o, lse = fwd(q, k, v, True, 0.2)
    o_sq, lse_sq = fwd(q_sq, k, v, True, 0.2)
    assert np.array_equal(o, o_sq[:, :, :Nq]) and np.array_equal(lse, lse_sq[:, :, :Nq]), \
        "causal Nq < Nk differs from the first Nq rows of the square problem"


def qk_rows_past_keys(fwd):
    B, H, Nq, Nk, d = 1, 3, 120, 45, 64
    q, k, v = _qk_inputs(B, H, Nq, Nk, d, "fp16", 600)
    o_c, lse_c = fwd(q, k, v, True, 0.125)
    o_n, lse_n = fwd(q, k, v, False, 0.125)
    assert np.array_equal(o_c[:, :, Nk - 1:], o_n[:, :, Nk - 1:]), "causal rows >= Nk-1 differ from non-causal"
    assert np.array_equal(lse_c[:, :, Nk - 1:], lse_n[:, :, Nk - 1:])
    assert not np.array_equal(o_c[:, :, :Nk - 1], o_n[:, :, :Nk - 1])


# (B, H, Nq, Nk, d, causal, window_left, window_right, key_lens)
MASK_CASES = [
    (2, 1, 9, 9, 4, True, 3, -1, [9, 5]),       # causal sliding window, one batch padded
    (1, 2, 7, 12, 3, False, 2, 1, None),        # banded, Nq < Nk
    (2, 1, 8, 6, 4, False, -1, -1, [0, 4]),     # a fully padded batch: no visible key anywhere
    (1, 1, 10, 10, 2, True, 0, -1, None),       # window 0: each row sees itself only
    (1, 1, 6, 10, 3, False, 1, 0, [3]),         # rows past the padding see nothing
]


def masked_decimal(fwd):
    for seed, (B, H, Nq, Nk, d, causal, wl, wr, kl) in enumerate(MASK_CASES):
        q, k, v = _qk_inputs(B, H, Nq, Nk, d, "fp16", 700 + 2 * seed)
        scale = 0.3
        o, lse = fwd(q, k, v, causal, scale, window_left=wl, window_right=wr, key_lens=kl)
        for b in range(B):
            for h in range(H):
                od, ld = _decimal_attention(_f(q[b, h]), _f(k[b, h]), _f(v[b, h]), causal, scale,
                                            wl, wr, None if kl is None else kl[b])
                fin = np.isfinite(ld)
                assert np.array_equal(np.isfinite(lse[b, h]), fin), f"masked rows differ {seed}"
                assert np.all(lse[b, h][~fin] == -np.inf) and np.all(o[b, h][~fin] == 0.0)
                _close(o[b, h], od, 1e-14, f"masked decimal O case {seed}")
                _close(lse[b, h][fin], ld[fin], 1e-14, f"masked decimal lse case {seed}")


def masked_torch(fwd):
    B, H, Nq, Nk, d = 2, 2, 70, 90, 16
    q, k, v = _qk_inputs(B, H, Nq, Nk, d, "bf16", 720)
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    for causal, wl, wr, kl in [(True, 20, -1, [90, 33]), (False, 5, 9, [60, 90]), (False, -1, -1, [1, 0])]:
        allow = torch.ones(B, Nq, Nk, dtype=torch.bool)
        if wl >= 0:
            allow &= (j >= i - wl)[None]
        allow &= (j <= i)[None] if causal else ((j <= i + wr)[None] if wr >= 0 else True)
        allow &= torch.arange(Nk)[None, None, :] < torch.tensor(kl)[:, None, None]
        s = torch.matmul(q.double(), k.double().transpose(-1, -2).contiguous()) * 0.25
        s = s.masked_fill(~allow[:, None], float("-inf"))
        lse_t = torch.logsumexp(s, dim=-1)
        p = torch.exp(s - lse_t[..., None]).nan_to_num(0.0)
        o_t = torch.matmul(p, v.double())
        o, lse = fwd(q, k, v, causal, 0.25, window_left=wl, window_right=wr, key_lens=kl)
        _close(o, o_t.numpy(), 1e-12, f"masked torch O causal={causal} wl={wl} wr={wr}")
        fin = np.isfinite(lse_t.numpy())
        assert np.array_equal(np.isfinite(lse), fin)
        _close(lse[fin], lse_t.numpy()[fin], 1e-12, f"masked torch lse causal={causal}")


def padding_is_truncation(fwd):
    B, H, Nq, Nk, d = 3, 2, 40, 50, 16
    q, k, v = _qk_inputs(B, H, Nq, Nk, d, "fp16", 740)
    kl = [50, 17, 1]
    for causal in (False, True):
        o, lse = fwd(q, k, v, causal, 0.25, key_lens=kl)
        for b, L in enumerate(kl):
            o_t, lse_t = fwd(q[b:b + 1], k[b:b + 1, :, :L].contiguous(), v[b:b + 1, :, :L].contiguous(),
                             causal, 0.25)
            assert np.array_equal(o[b:b + 1], o_t) and np.array_equal(lse[b:b + 1], lse_t), \
                f"padding to {L} keys differs from truncation causal={causal}"


def wide_window_is_none(fwd):
    q, k, v = _qk_inputs(1, 2, 33, 45, 8, "bf16", 750)
    for causal in (False, True):
        o, lse = fwd(q, k, v, causal, 0.25)
        o_w, lse_w = fwd(q, k, v, causal, 0.25, window_left=45, window_right=45)
        assert np.array_equal(o, o_w) and np.array_equal(lse, lse_w)
        o_n, _ = fwd(q, k, v, causal, 0.25, window_left=3)
        assert not np.array_equal(o, o_n)


ALL_PINS = [decimal_bruteforce, torch_sdpa, keys_zero, causal_row0, causal_last_row,
            prefix_truncation, v_ones, v_identity, online_equals_twopass, linearity,
            permutation, single_key, shift, qk_decimal_bruteforce, qk_torch_sdpa,
            qk_square_prefix, qk_rows_past_keys, masked_decimal, masked_torch,
            padding_is_truncation, wide_window_is_none]
