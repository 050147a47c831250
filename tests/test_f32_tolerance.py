"""CPU check that the fp32 parity bar (tests/test_f32_gpu.py: |dO| <= 1e-4,
|d lse| <= 5e-5 relative) excludes a kernel that merely rounds its fp32
inputs to bf16: the oracle on bf16-rounded inputs lies far outside it."""

import numpy as np

import oracle
from fa_inputs import make_qkv


def test_bf16_rounded_inputs_fail_the_fp32_bar():
    q, k, v = make_qkv(1, 2, 300, 128, "fp32", 450)
    scale = float(np.float32(1 / np.sqrt(128)))
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, causal, scale)
        rounded = [t.bfloat16().float() for t in (q, k, v)]
        o_b, lse_b = oracle.attention_fwd(*rounded, causal, scale)
        assert np.abs(o_b - o).max() > 5 * 1e-4
        assert (np.abs(lse_b - lse) / np.maximum(1, np.abs(lse))).max() > 2 * 5e-5
