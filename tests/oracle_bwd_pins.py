"""Pins for the fp64 backward oracle: checks against facts other than the oracle itself.

Each pin takes ``bwd`` (a callable with the signature of
``oracle.attention_bwd``) and raises ``AssertionError`` when the oracle
disagrees with what the mathematics fixes. ``test_oracle_bwd_pins.py`` runs
them against the real oracle and ``test_oracle_bwd_mutants.py`` against
deliberately broken copies (each broken copy must fail at least one pin).

What pins what:
  finite_differences   central differences of the forward oracle's sum(dO * O)
                       (the quantity whose gradient this is), on tiny shapes
  torch_autograd       a library autograd of the same forward, in fp64
  dk_sums_to_zero      sum_j dS_ij = 0 for every row, hence sum_j dK_j = 0
  equal_keys_zero_dq   identical keys give every query the same softmax, so dQ = 0
  uniform_dv           Q = 0: P is uniform over the visible keys, and dV has a
                       closed form (mean of dO, or a causal suffix sum)
  linear_in_dout       the gradients are linear in dO
  masked_finite_differences  central differences of the masked forward oracle
                       (padding, windows, rows that see no key)
  masked_torch_autograd  fp64 autograd through an explicit boolean mask
  masked_padding_is_truncation  a padding length L gives the gradients of the
                       first L keys, bit for bit, and zero for the rest
"""

import numpy as np
import torch

import oracle
from fa_inputs import make_qkv


def _f(x):
    return x.float().numpy().astype(np.float64) if hasattr(x, "float") else np.asarray(x, np.float64)


def _close(a, b, tol, what, scale_floor=1.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b)) / max(scale_floor, float(np.max(np.abs(b))))) if a.size else 0.0
    assert err <= tol, f"{what}: max error {err:.3e} > {tol:.1e}"


def _inputs(B, H, Nq, Nk, d, dtype, seed):
    q = make_qkv(B, H, Nq, d, dtype, seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed + 1)
    dout = make_qkv(B, H, Nq, d, dtype, seed + 2)[0]
    return q, k, v, dout


def finite_differences(bwd):
    rng = np.random.default_rng(5)
    for (B, H, Nq, Nk, d), causal in [((1, 2, 5, 7, 4), False), ((1, 1, 6, 6, 3), True),
                                      ((2, 1, 7, 3, 5), True)]:
        q, k, v, dout = (_f(t) for t in _inputs(B, H, Nq, Nk, d, "fp16", 200 + Nq))
        scale = 0.4
        dq, dk, dv = bwd(q, k, v, dout, causal, scale)

        def loss(q_, k_, v_):
            o, _ = oracle.attention_fwd(q_.astype(np.float32), k_.astype(np.float32),
                                        v_.astype(np.float32), causal, scale)
            return float(np.sum(o * dout))
        # the forward oracle takes fp32 inputs, so perturb by a power of two that fp32 holds exactly
        h = 2.0 ** -10
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(6):
                idx = tuple(rng.integers(0, s) for s in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name], args_m[name] = xp, xm
                fd = (loss(**{a + "_": b for a, b in args_p.items()}) -
                      loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
                assert abs(fd - g[idx]) <= 2e-5 * max(1.0, abs(fd)), \
                    f"d{name}{idx}: finite difference {fd:.8f} vs {g[idx]:.8f} causal={causal}"


def torch_autograd(bwd):
    for (B, H, Nq, Nk, d), causal, dtype in [((2, 2, 37, 37, 16), False, "bf16"),
                                             ((1, 3, 50, 50, 32), True, "fp16"),
                                             ((1, 2, 20, 45, 8), True, "bf16"),
                                             ((2, 1, 45, 20, 8), False, "fp16")]:
        q, k, v, dout = _inputs(B, H, Nq, Nk, d, dtype, 220 + Nq)
        scale = 0.3
        q64, k64, v64 = (t.to(torch.float64).requires_grad_() for t in (q, k, v))
        s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * scale
        if causal:
            s = s.masked_fill(torch.ones(Nq, Nk, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), v64)
        o.backward(dout.to(torch.float64))
        dq, dk, dv = bwd(q, k, v, dout, causal, scale)
        for name, a, b in (("dq", dq, q64.grad), ("dk", dk, k64.grad), ("dv", dv, v64.grad)):
            _close(a, b.numpy(), 1e-12, f"autograd {name} {(B, H, Nq, Nk, d)} causal={causal}")


def dk_sums_to_zero(bwd):
    for causal in (False, True):
        q, k, v, dout = _inputs(2, 3, 64, 80, 16, "bf16", 240)
        dq, dk, dv = bwd(q, k, v, dout, causal, 0.25)
        assert np.max(np.abs(dk)) > 1e-3
        _close(dk.sum(axis=2), np.zeros_like(dk.sum(axis=2)), 1e-12, f"sum_j dK_j causal={causal}")


def equal_keys_zero_dq(bwd):
    q, _, v, dout = _inputs(1, 2, 40, 30, 16, "fp16", 250)
    k = make_qkv(1, 2, 1, 16, "fp16", 251)[1].expand(1, 2, 30, 16).contiguous()
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, dout, causal, 0.5)
        assert np.max(np.abs(dv)) > 1e-3
        _close(dq, np.zeros_like(dq), 1e-13, f"equal keys give dQ = 0 causal={causal}")


def uniform_dv(bwd):
    B, H, Nq, Nk, d = 1, 2, 24, 24, 8
    _, k, v, dout = _inputs(B, H, Nq, Nk, d, "bf16", 260)
    q = torch.zeros(B, H, Nq, d, dtype=torch.bfloat16)
    D = _f(dout)
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, dout, causal, 0.5)
        if causal:
            w = D / np.arange(1, Nq + 1)[None, None, :, None]   # row i spreads dO_i over keys 0..i
            expect = np.cumsum(w[:, :, ::-1], axis=2)[:, :, ::-1]
        else:
            expect = np.broadcast_to(D.mean(axis=2, keepdims=True), dv.shape)
        _close(dv, expect, 1e-13, f"dV with uniform P causal={causal}")
        _close(dk, np.zeros_like(dk), 1e-13, f"dK with Q = 0 causal={causal}")


def linear_in_dout(bwd):
    q, k, v, d1 = _inputs(1, 2, 33, 33, 16, "fp16", 270)
    d2 = make_qkv(1, 2, 33, 16, "fp16", 273)[0]
    for causal in (False, True):
        g1 = bwd(q, k, v, d1, causal, 0.25)
        g2 = bwd(q, k, v, d2, causal, 0.25)
        g3 = bwd(q, k, v, (d1.float() * 2 - d2.float() * 3), causal, 0.25)
        for a, b, c, name in zip(g1, g2, g3, ("dq", "dk", "dv")):
            _close(c, 2 * a - 3 * b, 1e-12, f"{name} linear in dO causal={causal}")


# (B, H, Nq, Nk, d, causal, window_left, window_right, key_lens)
MASKS = [(2, 1, 7, 9, 4, True, 2, -1, [9, 3]),      # causal window; padding empties rows of batch 1
         (1, 2, 6, 8, 3, False, 1, 2, None),        # band
         (2, 1, 5, 6, 4, False, -1, -1, [0, 4])]    # a batch with no key at all


def masked_finite_differences(bwd):
    rng = np.random.default_rng(7)
    for (B, H, Nq, Nk, d, causal, wl, wr, kl) in MASKS:
        q, k, v, dout = (_f(t) for t in _inputs(B, H, Nq, Nk, d, "fp16", 300 + Nq))
        scale = 0.4
        dq, dk, dv = bwd(q, k, v, dout, causal, scale, window_left=wl, window_right=wr, key_lens=kl)

        def loss(q_, k_, v_):
            o, _ = oracle.attention_fwd(q_.astype(np.float32), k_.astype(np.float32),
                                        v_.astype(np.float32), causal, scale, window_left=wl,
                                        window_right=wr, key_lens=kl)
            return float(np.sum(o * dout))
        h = 2.0 ** -10
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(8):
                idx = tuple(rng.integers(0, s) for s in x.shape)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name], args_m[name] = xp, xm
                fd = (loss(**{a + "_": b for a, b in args_p.items()}) -
                      loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
                assert abs(fd - g[idx]) <= 2e-5 * max(1.0, abs(fd)), \
                    f"masked d{name}{idx}: finite difference {fd:.8f} vs {g[idx]:.8f}"


def masked_torch_autograd(bwd):
    B, H, Nq, Nk, d = 2, 2, 40, 56, 16
    q, k, v, dout = _inputs(B, H, Nq, Nk, d, "bf16", 320)
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    for causal, wl, wr, kl in [(True, 9, -1, [56, 20]), (False, 4, 7, [30, 56]), (False, -1, -1, [56, 0])]:
        allow = torch.ones(B, 1, Nq, Nk, dtype=torch.bool)
        if wl >= 0:
            allow = allow & (j >= i - wl)
        allow = allow & ((j <= i) if causal else ((j <= i + wr) if wr >= 0 else True))
        allow = allow & (torch.arange(Nk)[None, None, None, :] < torch.tensor(kl)[:, None, None, None])
        rows = allow.any(dim=-1, keepdim=True)  # rows that see some key
        q64, k64, v64 = (t.to(torch.float64).requires_grad_() for t in (q, k, v))
        s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * 0.3
        s = torch.where(allow, s, torch.tensor(float("-inf"), dtype=torch.float64))
        s = torch.where(rows, s, torch.zeros((), dtype=torch.float64))  # finite softmax on empty rows
        o = torch.matmul(torch.softmax(s, dim=-1), v64) * rows
        o.backward(dout.to(torch.float64))
        dq, dk, dv = bwd(q, k, v, dout, causal, 0.3, window_left=wl, window_right=wr, key_lens=kl)
        for name, a, b in (("dq", dq, q64.grad), ("dk", dk, k64.grad), ("dv", dv, v64.grad)):
            _close(a, b.numpy(), 1e-12, f"masked autograd {name} causal={causal} wl={wl} wr={wr}")


def masked_padding_is_truncation(bwd):
    B, H, Nq, Nk, d = 3, 2, 30, 40, 8
    q, k, v, dout = _inputs(B, H, Nq, Nk, d, "fp16", 330)
    lens = [40, 13, 1]
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, dout, causal, 0.25, key_lens=lens)
        for b, L in enumerate(lens):
            t = bwd(q[b:b + 1], k[b:b + 1, :, :L].contiguous(), v[b:b + 1, :, :L].contiguous(),
                    dout[b:b + 1], causal, 0.25)
            assert np.array_equal(dq[b:b + 1], t[0]), f"dq padded to {L} causal={causal}"
            assert np.array_equal(dk[b:b + 1, :, :L], t[1]) and np.array_equal(dv[b:b + 1, :, :L], t[2])
            assert np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


ALL_PINS = [finite_differences, torch_autograd, dk_sums_to_zero, equal_keys_zero_dq, uniform_dv,
            linear_in_dout, masked_finite_differences, masked_torch_autograd, masked_padding_is_truncation]
