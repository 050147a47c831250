"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on ROCm).

libfa allocates nothing, clears nothing with memset and never synchronises,
so a call made on a capturing stream records only its kernels. Each test
captures calls once, then replays the graph several times with new values
written into the captured inputs between replays (eager work and a
synchronisation in between, as a caller's step loop would have), and checks
every replay bit for bit against an eager call on the same values.
"""

import pytest
import torch

import tiled_attention_forward_fwd_amd as fa
from fa_inputs import make_qkv

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load_library()
    yield
    torch.cuda.synchronize()


def seeded(shape_src, dtype, seed):
    """Fresh seeded values with the shape of q (from the shared generator)."""
    B, H, N, d = shape_src.shape
    return make_qkv(B, H, N, d, dtype, seed)[0].cuda()


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph; returns (graph, outputs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def replay_and_check(g, outs, inputs, eager, dtype, seed0):
    """Between replays, write new values into inputs[0] (q), run the eager call on them and
    compare every output of the replay with it, bit for bit."""
    for r in range(REPLAYS):
        inputs[0].copy_(seeded(inputs[0], dtype, seed0 + r))
        ref = eager()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r} differs from the eager call"
        print(f"[graph] replay {r} equal to eager", flush=True)


# (B, H): the key-split launch of a small grid, and the direct kernel
@pytest.mark.parametrize("B,H,key_split", [(2, 4, True), (4, 16, False)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_in_a_graph(causal, B, H, key_split):
    assert (fa.fa_plan_qk(B, H, 1000, 1000, 128, int(causal), fa.FA_DTYPE_BF16)["block_m"] == 32) == key_split
    q, k, v = (t.cuda() for t in make_qkv(B, H, 1000, 128, "bf16", 700))
    f = lambda: fa.fwd(q, k, v, causal=causal, splits=1)  # noqa: E731
    g, outs = capture(f)
    replay_and_check(g, outs, (q, k, v), f, "bf16", 710)


def test_split_decode_in_a_graph():
    # one query against a 16384-key cache: split kernel, workspace and merge
    B, H, Nk, d = 4, 8, 16384, 128
    q = make_qkv(B, H, 1, d, "bf16", 720)[0].cuda()
    _, k, v = (t.cuda() for t in make_qkv(B, H, Nk, d, "bf16", 721))
    splits = fa.fa_split_count(B, H, 1, Nk, d, 0)
    assert splits > 1
    f = lambda: fa.fwd(q, k, v, splits=splits)  # noqa: E731
    g, outs = capture(f)
    replay_and_check(g, outs, (q, k, v), f, "bf16", 730)


def test_masked_decode_in_a_graph():
    # caches of different lengths, key_lens already on the GPU (a host list
    # would need a copy, which capture does not allow)
    B, H, Nk, d = 4, 4, 8192, 64
    q = make_qkv(B, H, 3, d, "fp16", 740)[0].cuda()
    _, k, v = (t.cuda() for t in make_qkv(B, H, Nk, d, "fp16", 741))
    kl = torch.tensor([8192, 5000, 1, 0], dtype=torch.int32, device="cuda")
    splits = fa.fa_split_count(B, H, 3, Nk, d, 0)
    f = lambda: fa.fwd(q, k, v, splits=splits, key_lens=kl)  # noqa: E731
    g, outs = capture(f)
    replay_and_check(g, outs, (q, k, v), f, "fp16", 750)


def test_backward_in_a_graph():
    q, k, v = (t.cuda() for t in make_qkv(1, 4, 700, 96, "bf16", 760))
    dout = make_qkv(1, 4, 700, 96, "bf16", 767)[0].cuda()

    def f():
        o, lse = fa.fwd(q, k, v, causal=True, splits=1)
        return (o, lse) + tuple(fa.bwd(q, k, v, o, lse, dout, causal=True))
    g, outs = capture(f)
    replay_and_check(g, outs, (q, k, v), f, "bf16", 770)
