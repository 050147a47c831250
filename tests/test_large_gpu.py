"""GPU checks at the largest sizes the API takes, through closed forms that
hold at any size (the oracle would need minutes here).

With K = 0 every visible score is 0, so each row's softmax is uniform over
its visible keys: O_i is the mean of the visible V rows and lse_i = ln(count)
(the closed form the oracle pins use at small sizes). The inputs are seeded
and generated on the GPU; the expected values are fp64 means on the GPU.
Tolerances are those of the other forward tests (3.2e-2 bf16, 4e-3 fp16 on O;
lse 1e-3 relative).

* 4 heads x 8M keys x d=128: element offsets past 2^31, a 2 GiB head in one
  buffer descriptor, the split-key path and its merge, and padding.
* a causal 1M-token sequence: prefix means for every row.
"""

import math

import pytest
import torch

import tiled_attention_forward_fwd_amd as fa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def seeded_normal(shape, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dtype)


def test_eight_million_keys_past_int32_offsets():
    B, H, Nq, Nk, d = 1, 4, 64, 1 << 23, 128
    assert B * H * Nk * d > 2 ** 31 and Nk * d * 2 == 2 ** 31
    q = seeded_normal((B, H, Nq, d), torch.bfloat16, 600)
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    v = seeded_normal((B, H, Nk, d), torch.bfloat16, 601)
    mean = v.mean(dim=2, dtype=torch.float64)  # [B, H, d], reduced in fp64 without a copy
    splits = fa.fa_split_count(B, H, Nq, Nk, d, 0)
    assert splits > 1
    o, lse = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    err_o = (o.double() - mean[:, :, None, :]).abs().max().item()
    err_l = (lse.double() - math.log(Nk)).abs().max().item() / math.log(Nk)
    print(f"[large] 4 x 8M keys: splits={splits} max|dO|={err_o:.3e} rel dlse={err_l:.3e}", flush=True)
    assert err_o <= 3.2e-2 and err_l <= 1e-3
    # padding: the last head's batch sees only its first L keys
    L = Nk - 12345
    o2, lse2 = fa.fwd(q, k, v, key_lens=[L])
    torch.cuda.synchronize()
    mean_l = v[:, :, :L].mean(dim=2, dtype=torch.float64)
    err_o2 = (o2.double() - mean_l[:, :, None, :]).abs().max().item()
    err_l2 = (lse2.double() - math.log(L)).abs().max().item() / math.log(L)
    print(f"[large] padded to {L}: max|dO|={err_o2:.3e} rel dlse={err_l2:.3e}", flush=True)
    assert err_o2 <= 3.2e-2 and err_l2 <= 1e-3


def test_causal_one_million_tokens_prefix_means():
    B, H, N, d = 1, 1, 1 << 20, 64
    q = seeded_normal((B, H, N, d), torch.float16, 610)
    k = torch.zeros((B, H, N, d), dtype=torch.float16, device="cuda")
    v = seeded_normal((B, H, N, d), torch.float16, 611)
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    cnt = torch.arange(1, N + 1, device="cuda", dtype=torch.float64)
    prefix = v.double().cumsum(dim=2) / cnt[None, None, :, None]
    err_o = (o.double() - prefix).abs().max().item()
    err_l = ((lse.double() - cnt.log()).abs() / cnt.log().clamp(min=1.0)).max().item()
    print(f"[large] causal 1M tokens: max|dO|={err_o:.3e} rel dlse={err_l:.3e}", flush=True)
    assert err_o <= 4e-3 and err_l <= 1e-3
    assert torch.equal(o[:, :, 0], v[:, :, 0])


def test_sliding_window_long_sequence_prefix_means():
    # causal window of 1000 keys over 65536 tokens: row i averages rows
    # max(0, i - 1000) .. i of V
    B, H, N, d, w = 1, 2, 1 << 16, 128, 1000
    q = seeded_normal((B, H, N, d), torch.bfloat16, 620)
    k = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    v = seeded_normal((B, H, N, d), torch.bfloat16, 621)
    o, lse = fa.fwd(q, k, v, causal=True, window_left=w)
    torch.cuda.synchronize()
    c = torch.nn.functional.pad(v.double().cumsum(dim=2), (0, 0, 1, 0))  # c[j] = sum of rows < j
    i = torch.arange(N, device="cuda")
    lo = (i - w).clamp(min=0)
    cnt = (i + 1 - lo).double()
    ref = (c[:, :, i + 1] - c[:, :, lo]) / cnt[None, None, :, None]
    err_o = (o.double() - ref).abs().max().item()
    err_l = ((lse.double() - cnt.log()).abs() / cnt.log().clamp(min=1.0)).max().item()
    print(f"[large] window {w} over {N}: max|dO|={err_o:.3e} rel dlse={err_l:.3e}", flush=True)
    assert err_o <= 3.2e-2 and err_l <= 1e-3
