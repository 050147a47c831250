"""CPU checks of the C ABI: the library loads, exports what include/fa.h
declares, rejects bad arguments before touching the device, and its host
logic (tile ranges, FLOP counts) reproduces the figures the pages print."""

import ctypes
import json
import os
import re

import pytest

import tiled_attention_forward_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "page_counts.json")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from tiled_attention_forward_fwd_amd import build
        build.build()
    return fa.load_library()


def declared_functions():
    names = []
    for hdr in os.listdir(os.path.join(ROOT, "include")):
        text = open(os.path.join(ROOT, "include", hdr)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_names():
    assert sorted(fa.EXPORTED) == declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libfa.so does not export {name}"


# 16-byte aligned fake addresses: every call below fails validation first,
# so nothing is ever dereferenced or launched.
P = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000]


def call(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, causal=0,
             scale=0.125, dtype=fa.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                     a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=P[1] + 8), fa.FA_ERR_INVALID_ARG),      # misaligned
    (dict(lse=P[4] + 2), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),              # empty sequence
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(d=100), fa.FA_ERR_UNSUPPORTED),            # not a multiple of 8
    (dict(d=136), fa.FA_ERR_UNSUPPORTED),            # above 128
    (dict(d=0), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(o=P[0]), fa.FA_ERR_INVALID_ARG),           # o aliases q
    (dict(o=P[2] + 16), fa.FA_ERR_INVALID_ARG),      # o overlaps v
    (dict(lse=P[3] + 64), fa.FA_ERR_INVALID_ARG),    # lse inside o
    (dict(B=65536, H=65536), fa.FA_ERR_INVALID_ARG),  # grid too large
    (dict(N=1 << 24, d=128), fa.FA_ERR_INVALID_ARG),  # one head >= 4 GiB
])
def test_fa_fwd_rejects_before_any_hip_call(lib, kw, status):
    assert call(**kw) == status
    assert fa.fa_status_string(status)


def test_status_strings(lib):
    assert fa.fa_status_string(fa.FA_OK) == "FA_OK"
    assert "unknown" in fa.fa_status_string(99)


def test_tile_counts_match_the_causal_skip_figures(lib):
    g = GOLDEN["causal_tile_pairs_BM64_BN32_N4096"]
    assert fa.fa_tile_counts(4096, 64, 32, 1) == (g["all"], g["visited"], g["unmasked"],
                                                  g["diagonal_masked"])


def test_executed_ops_with_pages_tiling(lib):
    g = GOLDEN["causal_executed_ops_BM64_BN32_B4_H8_N4096_D64"]
    _, visited, _, _ = fa.fa_tile_counts(4096, 64, 32, 1)
    ops = 4 * 64 * 64 * 32 * visited * 4 * 8
    assert abs(ops - g["value"]) <= g["printed_digits"]


@pytest.mark.parametrize("N,bm,bn", [(1000, 128, 64), (1000, 64, 32), (1, 128, 64), (129, 128, 128),
                                     (4096, 128, 64), (16384, 128, 64), (777, 64, 128)])
def test_tile_counts_cover_every_visible_key_once(lib, N, bm, bn):
    total, visited, unmasked, masked = fa.fa_tile_counts(N, bm, bn, 0)
    n_qt, n_kt = -(-N // bm), -(-N // bn)
    assert total == n_qt * n_kt and visited == total
    assert masked == (n_qt if N % bn else 0)
    # causal: brute-force the pairs that hold at least one visible (q, k <= q) entry
    need = 0
    for i in range(n_qt):
        last_q = min(N, (i + 1) * bm) - 1
        need += last_q // bn + 1
    total, visited, unmasked, masked = fa.fa_tile_counts(N, bm, bn, 1)
    assert visited == need
    # an unmasked pair must be fully visible: inside [0, N) and its last key at
    # or below the tile's first query; the rest of the visited pairs get the mask
    fully_visible = sum(1 for i in range(n_qt) for j in range(n_kt)
                        if (j + 1) * bn <= N and (j + 1) * bn - 1 <= i * bm)
    assert unmasked <= fully_visible
    assert unmasked + masked == visited
    assert masked <= n_qt * (-(-bm // bn) + 1)


def test_plan_flops_match_printed_counts(lib):
    nc = fa.fa_plan(4, 8, 4096, 64, 0, fa.FA_DTYPE_BF16)
    c = fa.fa_plan(4, 8, 4096, 64, 1, fa.FA_DTYPE_BF16)
    g = GOLDEN["flops_noncausal_B4_H8_N4096_D64"]
    assert abs(nc["algo_flops"] - g["value"]) <= g["printed_digits"]
    g = GOLDEN["flops_causal_needed_B4_H8_N4096_D64"]
    assert abs(c["algo_flops"] - g["value"]) <= g["printed_digits"]
    # non-causal with tile-divisible N: the matrix cores execute exactly the
    # algorithm's FLOPs; causal adds the masked part of the diagonal tiles
    assert nc["mfma_flops"] == nc["algo_flops"]
    assert c["mfma_flops"] > c["algo_flops"]
    # waves skip the diagonal key tiles past their own rows, so the executed
    # work is below the visited tile pairs' full count
    assert c["mfma_flops"] < 4 * 64 * c["block_m"] * c["block_n"] * c["pairs_visited"]
    assert c["mfma_flops"] == _walked_mfma_flops(4, 8, 4096, 4096, 64, 1, c["threads"] // 64)


def _key_split_launch(B, H, Nq, Nk, D, causal):
    """The rule that sends a direct launch to the key-split kernel, restated:
    more than 32 query rows, at most 256 (D = 128) or 512 (D = 64) workgroups
    of 32 rows, and at most 2048 keys seen by the longest query block."""
    keys = min(Nq, Nk) if causal else Nk
    return Nq > 32 and B * H * -(-Nq // 32) <= (512 if D <= 64 else 256) and keys <= 2048


def _walked_mfma_flops(B, H, Nq, Nk, D, causal, waves):
    """The forward kernel's step loop walked one step at a time (no masks, no
    split): each wave counts the 32 x 64 blocks whose S = Q K^T and whose P V
    it computes. Restates the kernel's control flow, not the plan's interval
    arithmetic. A key-split launch computes every 32-key tile of each 32-row
    block once (one wave each), S and P V of 32 x 32."""
    if _key_split_launch(B, H, Nq, Nk, D, causal):
        tiles = 0
        for q0 in range(0, Nq, 32):
            last = min(q0 + 32, Nq, Nk) if causal else Nk  # keys the block's rows see
            tiles += -(-last // 32)
        return tiles * 2 * 2 * 32 * 32 * D * B * H
    BM, BN = 32 * waves, 64  # every unmasked, unpadded direct launch fuses the exp work
    blocks = 0
    for q0 in range(0, Nq, BM):
        full_end = (Nk // BN) * BN
        if causal:
            un_end = min((q0 // BN) * BN, full_end)
            m_end = min(q0 + BM, Nq, Nk)
        else:
            un_end, m_end = full_end, Nk
        u_hi = un_end // BN
        je = u_hi + -(-(m_end - un_end) // BN)
        for w in range(waves):
            n_wave = min(je, (q0 + (w + 1) * 32 - 1) // BN + 1) if causal else je
            sees = lambda t: t < n_wave  # noqa: E731
            blocks += 1  # the first tile's scores, before the loop
            for j in range(0, je - 1):
                G = j >= u_hi  # masked step: per-wave limits apply
                if not G or sees(j):
                    blocks += 1 if (not G or sees(j + 1)) else 0  # scores of tile j+1
                    blocks += 1  # P V of tile j
            j = je - 1
            blocks += 1 if (j < u_hi or sees(j)) else 0  # the last tile's P V
    return blocks * 2 * 32 * 64 * D * B * H


@pytest.mark.parametrize("Nq,Nk", [(4096, 4096), (1000, 1000), (300, 1000), (1000, 300), (129, 64),
                                   (1, 16384), (4097, 4097)])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("d", [64, 128])
def test_plan_mfma_flops_follow_the_kernel_loop(lib, Nq, Nk, causal, d):
    for B, H in ((1, 2), (8, 16)):  # both workgroup shapes
        p = fa.fa_plan_qk(B, H, Nq, Nk, d, causal, fa.FA_DTYPE_BF16)
        assert p["mfma_flops"] == _walked_mfma_flops(B, H, Nq, Nk, d, causal, p["threads"] // 64)
        assert p["mfma_flops"] >= p["algo_flops"] * (1.0 if not causal else 0.999)


def test_plan_mfma_flops_of_the_headline_causal_launch(lib):
    # B4 H16 N4096 d128 causal: 4-wave workgroups of 128 rows; in query tile
    # i, waves 0-1 compute 2i+1 key tiles and waves 2-3 compute 2i+2, i.e.
    # 8i+6 blocks of 32 rows x 64 keys per workgroup for each of S and P V:
    # 64 heads x sum_i (8i+6) x 2 x 2*32*64*128 FLOPs = 279.17 G
    c = fa.fa_plan(4, 16, 4096, 128, 1, fa.FA_DTYPE_BF16)
    per_head = sum(8 * i + 6 for i in range(32))
    assert c["mfma_flops"] == 64 * per_head * 2 * 2 * 32 * 64 * 128
    assert abs(c["mfma_flops"] - 279.17e9) < 0.01e9


def test_plan_flop_convention_matches_t4_table(lib):
    g = GOLDEN["t4_sequence_sweep"]
    for N, impl, ms, tflops in g["rows"]:
        flops = fa.fa_plan(1, 16, N, 64, 0, fa.FA_DTYPE_F16)["algo_flops"]  # B*H*d = 1024
        assert abs(flops / (ms * 1e-3) / 1e12 - tflops) <= 0.006 + 0.005 * tflops, (N, impl)


def test_plan_rejects_like_fa_fwd(lib):
    with pytest.raises(fa.FaError) as e:
        fa.fa_plan(1, 1, 16, 84, 0, fa.FA_DTYPE_BF16)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FaError):
        fa.fa_plan(1, 1, 0, 64, 0, fa.FA_DTYPE_BF16)


def test_plan_picks_workgroup_shape(lib):
    # non-causal problems that give every CU a 256-row workgroup use 8 waves
    big = fa.fa_plan(4, 16, 4096, 128, 0, fa.FA_DTYPE_BF16)
    assert (big["block_m"], big["threads"], big["workgroups"]) == (256, 512, 1024)
    # causal problems and small grids keep 128-row, 4-wave workgroups
    causal = fa.fa_plan(4, 16, 4096, 128, 1, fa.FA_DTYPE_BF16)
    assert (causal["block_m"], causal["threads"], causal["workgroups"]) == (128, 256, 2048)
    short = fa.fa_plan(4, 16, 512, 64, 0, fa.FA_DTYPE_F16)
    assert (short["block_m"], short["threads"], short["workgroups"]) == (128, 256, 4 * 16 * 4)
    # when every 32-row workgroup fits on the chip at once (512 at d <= 64, 256
    # above) and the rows see at most 2048 keys, the key-split kernel runs:
    # 32-row workgroups of 4 waves over 32-key tiles
    small = fa.fa_plan(2, 4, 1000, 64, 0, fa.FA_DTYPE_F16)
    assert (small["block_m"], small["block_n"], small["threads"], small["workgroups"]) == (32, 32, 256, 2 * 4 * 32)
    assert small["lds_bytes"] == 4 * 4 * 32 * 64 * 2
    assert fa.fa_plan(1, 1, 128, 64, 1, fa.FA_DTYPE_F16)["block_m"] == 32
    assert fa.fa_plan(2, 8, 1000, 64, 0, fa.FA_DTYPE_F16)["block_m"] == 32      # 512 workgroups
    assert fa.fa_plan(4, 8, 1000, 64, 0, fa.FA_DTYPE_F16)["block_m"] == 128     # 1024
    assert fa.fa_plan(1, 8, 1500, 128, 0, fa.FA_DTYPE_BF16)["block_m"] == 128   # 376 at d = 128
    assert fa.fa_plan(1, 2, 2048, 96, 1, fa.FA_DTYPE_BF16)["lds_bytes"] == 4 * 4 * 32 * 128 * 2
    # computing 128 dims it keeps a third K tile per wave (the next tile's scores come first)
    assert fa.fa_plan(1, 2, 2048, 128, 1, fa.FA_DTYPE_BF16)["lds_bytes"] == 4 * 5 * 32 * 128 * 2
    assert fa.fa_plan(1, 2, 2048, 128, 1, fa.FA_DTYPE_BF16)["block_m"] == 32
    assert fa.fa_plan(1, 2, 4096, 128, 0, fa.FA_DTYPE_BF16)["block_m"] == 128   # 4096 keys
    assert fa.fa_plan_qk(1, 2, 32, 2048, 128, 0, fa.FA_DTYPE_BF16)["block_m"] == 128  # decode-like: split path
    assert fa.fa_plan_qk(1, 2, 600, 4096, 128, 1, fa.FA_DTYPE_BF16)["block_m"] == 32  # sees 600 keys
    # at most 128 query rows: 128-row workgroups whatever the grid, so that
    # no workgroup holds a CU's waves for one block of rows
    for nq in (1, 16, 128):
        few = fa.fa_plan_qk(64, 32, nq, 8192, 128, 0, fa.FA_DTYPE_BF16)
        assert (few["block_m"], few["threads"], few["workgroups"]) == (128, 256, 64 * 32)
    more = fa.fa_plan_qk(64, 32, 129, 8192, 128, 0, fa.FA_DTYPE_BF16)
    assert (more["block_m"], more["threads"], more["workgroups"]) == (256, 512, 64 * 32)


def test_plan_lds_bytes(lib):
    # two K and two V tiles of 64 rows; the 8-wave launches without masks or
    # padding also hold their 256-row Q tile; the staged epilogue (32 rows of
    # D + 8 elements per wave) needs more than the tiles only for 8-wave
    # launches that hold no Q tile
    big = fa.fa_plan(4, 16, 4096, 128, 0, fa.FA_DTYPE_BF16)
    assert big["lds_bytes"] == 4 * 64 * 128 * 2 + 256 * 128 * 2
    assert fa.fa_plan(4, 16, 4096, 128, 1, fa.FA_DTYPE_BF16)["lds_bytes"] == 4 * 64 * 128 * 2
    assert fa.fa_plan(4, 16, 4096, 64, 0, fa.FA_DTYPE_BF16)["lds_bytes"] == 4 * 64 * 64 * 2 + 256 * 64 * 2
    # padded d = 96 runs the d = 128 kernel: no Q tile, staged epilogue
    assert fa.fa_plan(4, 16, 4096, 96, 0, fa.FA_DTYPE_BF16)["lds_bytes"] == 8 * 32 * 136 * 2
    # padded d = 32: neither
    assert fa.fa_plan(4, 16, 4096, 32, 0, fa.FA_DTYPE_F16)["lds_bytes"] == 4 * 64 * 64 * 2
    # masks: staged epilogue, no Q tile
    m = fa.fa_plan_masked(4, 16, 4096, 4096, 64, 0, 100, -1, None, fa.FA_DTYPE_BF16)
    assert m["threads"] == 512 and m["lds_bytes"] == 8 * 32 * 72 * 2


# ---- Nq != Nk (fa_fwd_qk, fa_tile_counts_qk, fa_plan_qk)

def call_qk(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, Nq=16, Nk=48, d=64, causal=0,
             scale=0.125, dtype=fa.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_qk(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                        a["Nk"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-5), fa.FA_ERR_INVALID_ARG),
    (dict(d=4), fa.FA_ERR_UNSUPPORTED),
    (dict(d=81), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=1 << 24, d=128), fa.FA_ERR_INVALID_ARG),   # one key head >= 4 GiB
    (dict(Nq=1 << 24, d=128), fa.FA_ERR_INVALID_ARG),   # one query head >= 4 GiB
    (dict(o=P[1] + 32 * 64 * 2), fa.FA_ERR_INVALID_ARG),  # o inside k's 48 rows (not q's 16)
    (dict(lse=P[3] + 16 * 64 * 2 - 4), fa.FA_ERR_INVALID_ARG),  # lse overlaps o's tail
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
])
def test_fa_fwd_qk_rejects_before_any_hip_call(lib, kw, status):
    assert call_qk(**kw) == status


@pytest.mark.parametrize("Nq,Nk,bm,bn", [(5, 15, 128, 64), (1, 10, 128, 64), (1000, 300, 128, 64),
                                         (300, 1000, 128, 64), (257, 64, 256, 64), (64, 4097, 128, 64),
                                         (1, 16384, 128, 64), (700, 129, 64, 128)])
def test_tile_counts_qk_cover_every_visible_key(lib, Nq, Nk, bm, bn):
    n_qt, n_kt = -(-Nq // bm), -(-Nk // bn)
    total, visited, unmasked, masked = fa.fa_tile_counts_qk(Nq, Nk, bm, bn, 0)
    assert total == n_qt * n_kt and visited == total and masked == (n_qt if Nk % bn else 0)
    # causal (top-left): a query tile needs key tiles up to min(last query, Nk - 1)
    need = sum(min(min(Nq, (i + 1) * bm) - 1, Nk - 1) // bn + 1 for i in range(n_qt))
    total, visited, unmasked, masked = fa.fa_tile_counts_qk(Nq, Nk, bm, bn, 1)
    assert visited == need
    # an unmasked pair is fully visible: inside [0, Nk) and at or below the tile's first query
    fully_visible = sum(1 for i in range(n_qt) for j in range(n_kt)
                        if (j + 1) * bn <= Nk and (j + 1) * bn - 1 <= i * bm)
    assert unmasked <= fully_visible and unmasked + masked == visited


def test_tile_counts_qk_square_case_is_fa_tile_counts(lib):
    for N in (1, 100, 4096):
        for causal in (0, 1):
            assert fa.fa_tile_counts_qk(N, N, 128, 64, causal) == fa.fa_tile_counts(N, 128, 64, causal)


def test_plan_qk_flops_and_bytes(lib):
    B, H, d = 2, 3, 64
    for Nq, Nk in [(100, 300), (300, 100), (4096, 4096), (1, 16384)]:
        nc = fa.fa_plan_qk(B, H, Nq, Nk, d, 0, fa.FA_DTYPE_F16)
        c = fa.fa_plan_qk(B, H, Nq, Nk, d, 1, fa.FA_DTYPE_F16)
        assert nc["algo_flops"] == 4 * B * H * Nq * Nk * d
        area = Nq * Nq / 2 if Nq <= Nk else Nk * Nk / 2 + (Nq - Nk) * Nk
        assert c["algo_flops"] == 4 * B * H * area * d
        assert nc["algo_bytes"] == 2 * B * H * d * (2 * Nq + 2 * Nk) + 4 * B * H * Nq
        assert nc["workgroups"] == B * H * -(-Nq // nc["block_m"])
    assert fa.fa_plan_qk(4, 8, 4096, 4096, 64, 1, 1) == fa.fa_plan(4, 8, 4096, 64, 1, 1)


# ---- padding lengths and sliding windows (fa_fwd_masked, fa_fwd_split_masked,
# fa_tile_counts_masked, fa_plan_masked)

def _visible_matrix(Nq, Nk, causal, wl, wr, klen):
    """[Nq, Nk] booleans straight from the mask rules."""
    import numpy as np
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    vis = np.broadcast_to(j < klen, (Nq, Nk)).copy()
    if wl >= 0:
        vis = vis & (j >= i - wl)
    if causal:
        vis = vis & (j <= i)
    elif wr >= 0:
        vis = vis & (j <= i + wr)
    return vis


MASK_GRID = [(Nq, Nk, causal, wl, wr, klen, bm)
             for (Nq, Nk) in [(1, 1), (5, 300), (257, 130), (300, 513), (640, 640)]
             for causal in (0, 1)
             for (wl, wr) in [(-1, -1), (0, -1), (63, 5), (100, 0), (200, 150)]
             for klen in sorted({Nk, 0, 1, Nk // 2})
             for bm in (128, 256)]


@pytest.mark.parametrize("Nq,Nk,causal,wl,wr,klen,bm", MASK_GRID)
def test_tile_counts_masked_are_exact(lib, Nq, Nk, causal, wl, wr, klen, bm):
    """Visited key tiles are exactly those holding a visible key of some row of the
    query tile; unmasked ones are exactly those every row of the tile sees in full."""
    bn = 64
    vis = _visible_matrix(Nq, Nk, causal, wl, wr, klen)
    n_qt, n_kt = -(-Nq // bm), -(-Nk // bn)
    visited = unmasked = 0
    for qt in range(n_qt):
        rows = vis[qt * bm:(qt + 1) * bm]
        for kt in range(n_kt):
            block = rows[:, kt * bn:(kt + 1) * bn]
            visited += bool(block.any())
            unmasked += bool(block.all()) and (kt + 1) * bn <= Nk
    total, v, u, m = fa.fa_tile_counts_masked(Nq, Nk, bm, bn, causal, wl, wr, klen)
    assert (total, v, u, m) == (n_qt * n_kt, visited, unmasked, visited - unmasked)


def test_tile_counts_masked_without_masks_visit_what_fa_tile_counts_visits(lib):
    for Nq, Nk in [(1000, 1000), (300, 1000), (1000, 300), (4096, 4096)]:
        for causal in (0, 1):
            plain = fa.fa_tile_counts_qk(Nq, Nk, 128, 64, causal)
            masked = fa.fa_tile_counts_masked(Nq, Nk, 128, 64, causal, -1, -1, Nk)
            assert masked[:2] == plain[:2]
            assert masked[2] >= plain[2]  # the masked split is exact, the plain one conservative


def test_plan_masked_counts_visible_pairs_and_keys(lib):
    B, H, d = 3, 2, 64
    for Nq, Nk, causal, wl, wr, kls in [(300, 513, 0, 63, 5, [513, 100, 0]),
                                        (257, 130, 1, 200, -1, [130, 1, 65]),
                                        (640, 640, 1, 100, -1, None),
                                        (64, 4096, 0, -1, -1, [4096, 2048, 17])]:
        plan = fa.fa_plan_masked(B, H, Nq, Nk, d, causal, wl, wr, kls, fa.FA_DTYPE_BF16)
        pairs = keys = 0
        for b in range(B):
            vis = _visible_matrix(Nq, Nk, causal, wl, wr, Nk if kls is None else kls[b])
            pairs += int(vis.sum())
            keys += int(vis.any(axis=0).sum())
        assert plan["algo_flops"] == 4 * H * pairs * d
        assert plan["algo_bytes"] == 4 * H * (B * Nq + keys) * d + 4 * B * H * Nq
        tiles = sum(fa.fa_tile_counts_masked(Nq, Nk, plan["block_m"], 64, causal, wl, wr,
                                             Nk if kls is None else kls[b])[1] for b in range(B))
        assert plan["pairs_visited"] == H * tiles
        # every visible pair is computed (at the kernel's head dim, here d);
        # no wave computes more than every visited tile pair plus the one
        # leading tile a wave whose range starts inside the query tile takes
        waves = plan["threads"] // 64
        assert plan["mfma_flops"] >= plan["algo_flops"]
        n_qt = -(-Nq // plan["block_m"])
        assert plan["mfma_flops"] <= 4 * d * plan["block_m"] * 64 * plan["pairs_visited"] + \
            B * H * n_qt * waves * 2 * 2 * 32 * 64 * d


def test_plan_masked_shape(lib):
    # masked d = 128 keeps 128-row workgroups; d = 64 takes the unmasked choice
    p128 = fa.fa_plan_masked(4, 16, 4096, 4096, 128, 0, -1, -1, [4096] * 4, fa.FA_DTYPE_BF16)
    assert (p128["block_m"], p128["threads"]) == (128, 256)
    p64 = fa.fa_plan_masked(4, 16, 4096, 4096, 64, 0, -1, -1, [4096] * 4, fa.FA_DTYPE_BF16)
    assert (p64["block_m"], p64["threads"]) == (256, 512)
    # no mask in effect: the unmasked launch and its plan
    off = fa.fa_plan_masked(4, 16, 4096, 4096, 128, 1, -1, 7, None, fa.FA_DTYPE_BF16)
    assert off["block_m"] == fa.fa_plan_qk(4, 16, 4096, 4096, 128, 1, 1)["block_m"]
    small = fa.fa_plan_masked(2, 4, 1000, 1000, 64, 0, -1, -1, None, fa.FA_DTYPE_BF16)
    ref = fa.fa_plan_qk(2, 4, 1000, 1000, 64, 0, fa.FA_DTYPE_BF16)
    assert ref["block_m"] == 32  # the key-split launch, also through the masked entry point
    for key in ("block_m", "block_n", "threads", "lds_bytes", "workgroups", "pairs_visited", "mfma_flops",
                "algo_flops", "algo_bytes"):
        assert small[key] == ref[key], key
    with pytest.raises(fa.FaError):
        fa.fa_plan_masked(2, 1, 64, 64, 64, 0, -1, -1, [64, 65], fa.FA_DTYPE_BF16)
    with pytest.raises(fa.FaError):
        fa.fa_plan_masked(1, 1, 64, 64, 64, 0, -2, -1, None, fa.FA_DTYPE_BF16)


KL = 0x60000  # fake 4-byte aligned device address for key_lens


def call_masked(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=1, Nq=16, Nk=48, d=64, causal=0,
             wl=-1, wr=-1, kl=KL, scale=0.125, dtype=fa.FA_DTYPE_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                            a["Nk"], a["d"], a["causal"], a["wl"], a["wr"], a["kl"], a["scale"],
                            a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(wl=-2), dict(wr=-5), dict(kl=KL + 2),            # bad window, misaligned key_lens
    dict(kl=P[3] + 8), dict(kl=P[4]),                     # key_lens inside o or lse
    dict(Nk=0), dict(q=None), dict(scale=0.0),
])
def test_fa_fwd_masked_rejects_before_any_hip_call(lib, kw):
    assert call_masked(**kw) == fa.FA_ERR_INVALID_ARG


def test_fa_fwd_split_masked_rejects_before_any_hip_call(lib):
    ws = 0x100000
    base = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=1, Nq=16, Nk=4096, d=64,
                causal=0, wl=-1, wr=-1, kl=KL, scale=0.125, dtype=fa.FA_DTYPE_BF16, n=4,
                ws=ws, wsb=fa.fa_split_workspace_bytes(2, 1, 16, 64, 4))

    def run(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_fwd_split_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                      a["Nq"], a["Nk"], a["d"], a["causal"], a["wl"], a["wr"],
                                      a["kl"], a["scale"], a["dtype"], a["n"], a["ws"], a["wsb"],
                                      None)
    for kw in [dict(wl=-3), dict(n=0), dict(n=65), dict(ws=None), dict(wsb=base["wsb"] - 4),
               dict(kl=ws + 64), dict(ws=ws + 8)]:
        assert run(**kw) == fa.FA_ERR_INVALID_ARG, kw


def test_split_count_suggestion(lib):
    # decode grids are split to about 512 workgroups, a full grid is not, short
    # key sequences stay direct
    assert fa.fa_split_count(1, 32, 1, 16384, 128, 0) == 16
    assert fa.fa_split_count(1, 32, 1, 1024, 128, 0) == 8     # chunks of two key tiles
    assert fa.fa_split_count(4, 32, 1, 2048, 128, 0) == 4
    assert fa.fa_split_count(4, 32, 1, 16384, 128, 0) == 8    # long caches: 8 chunks
    assert fa.fa_split_count(16, 32, 1, 2048, 128, 0) == 1    # a large grid of short caches
    assert fa.fa_split_count(16, 32, 1, 8192, 128, 0) == 2
    assert fa.fa_split_count(2, 32, 128, 8192, 128, 0) == 4   # full query tiles: at most 256 workgroups
    assert fa.fa_split_count(2, 32, 128, 4096, 128, 0) == 4   # ... with chunks of 16 key tiles
    assert fa.fa_split_count(1, 32, 128, 3072, 128, 0) == 3
    assert fa.fa_split_count(1, 16, 128, 4096, 128, 0) == 8   # 16 workgroups: chunks of 8 key tiles
    # the key-split kernel (up to 2048 keys, its workgroups all resident)
    # shortens these in one launch
    assert fa.fa_split_count(2, 32, 128, 2048, 128, 0) == 1
    assert fa.fa_split_count(1, 16, 128, 1536, 128, 0) == 1
    assert fa.fa_split_count(2, 4, 1000, 1000, 64, 0) == 1
    assert fa.fa_split_count(2, 4, 3000, 3000, 64, 0) == 1    # 192 workgroups of 128 rows
    assert fa.fa_split_count(1, 1, 8192, 8192, 64, 1) == 4
    assert fa.fa_split_count(2, 32, 128, 8192, 128, 1) == 1   # causal: the queries see 128 keys
    assert fa.fa_split_count(8, 32, 128, 8192, 128, 0) == 1
    assert fa.fa_split_count(4, 16, 4096, 4096, 128, 0) == 1
    assert fa.fa_split_count(1, 1, 1, 512, 64, 0) == 1
    assert fa.fa_split_count(1, 1, 1, 960, 64, 0) == 1       # under 16 key tiles
    assert fa.fa_split_count(0, 1, 1, 512, 64, 0) == 0  # invalid
    for B, H, Nq, Nk in [(1, 1, 1, 100000), (2, 8, 300, 5000), (16, 32, 1, 2048), (1, 64, 129, 65536),
                         (1, 1, 32, 1024), (3, 5, 33, 7777), (64, 32, 1, 8192)]:
        s = fa.fa_split_count(B, H, Nq, Nk, 128, 0)
        n_kt = -(-Nk // 64)
        assert 1 <= s <= max(1, n_kt // 2)
        if min(Nq, 128) > 32:
            assert s <= max(1, n_kt // 8)


# ---- head dims other than 64 and 128 (run padded by the d = 64 / 128 kernels)

@pytest.mark.parametrize("d", [8, 16, 32, 40, 48, 56, 72, 80, 96, 112, 120])
def test_plan_other_head_dims(lib, d):
    D = 64 if d <= 64 else 128
    DC = -(-d // 32) * 32  # the dims the kernel's MFMAs cover
    for causal in (0, 1):
        p = fa.fa_plan_qk(2, 8, 1000, 1500, d, causal, fa.FA_DTYPE_BF16)
        ref = fa.fa_plan_qk(2, 8, 1000, 1500, D, causal, fa.FA_DTYPE_BF16)
        # same grid and tiles as the kernel head dim; algorithmic work at d,
        # executed MFMA work at d rounded up to 32
        for key in ("block_m", "block_n", "threads", "lds_bytes", "workgroups", "pairs_visited"):
            assert p[key] == ref[key], key
        assert p["mfma_flops"] == ref["mfma_flops"] * DC / D
        assert p["algo_flops"] == ref["algo_flops"] * d / D
        assert p["algo_bytes"] == 4 * 2 * 8 * (1000 + 1500) * d + 4 * 2 * 8 * 1000
    assert fa.fa_split_workspace_bytes(1, 4, 3, d, 5) == 5 * 4 * 3 * (D + 1) * 4


@pytest.mark.parametrize("d", [0, 4, 100, 127, 136, 256])
def test_backward_rejects_head_dims_it_does_not_build(lib, d):
    # the backward takes the forward's head dims: multiples of 8 from 8 to 128
    args = [P[0], P[1], P[2], P[3], P[4], 0x60000, 0x70000, 0x80000, 0x90000, 0xa0000]
    assert fa.fa_bwd(*args, 1, 1, 16, d, 0, 0.1, fa.FA_DTYPE_BF16, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_masked(*args, 1, 1, 16, 16, d, 1, 4, -1, None, 0.1, fa.FA_DTYPE_F16,
                            None) == fa.FA_ERR_UNSUPPORTED


def test_fa_fwd_f32_rejects_before_any_hip_call(lib):
    ws = 0x200000
    base = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, Nq=16, Nk=16, d=64, causal=0,
                scale=0.125, ws=ws, wsb=fa.fa_f32_workspace_bytes(1, 1, 16, 64))

    def run(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_fwd_f32(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                             a["d"], a["causal"], a["scale"], a["ws"], a["wsb"], None)
    assert fa.fa_f32_workspace_bytes(2, 3, 100, 128) == 8 * 2 * 3 * 100 * 128
    assert fa.fa_f32_workspace_bytes(1, 1, 16, 96) == 0
    for kw, st in [(dict(ws=None), fa.FA_ERR_INVALID_ARG), (dict(wsb=base["wsb"] - 1), fa.FA_ERR_INVALID_ARG),
                   (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(ws=ws + 8), fa.FA_ERR_INVALID_ARG),
                   (dict(o=P[0]), fa.FA_ERR_INVALID_ARG), (dict(ws=P[2]), fa.FA_ERR_INVALID_ARG),
                   (dict(scale=0.0), fa.FA_ERR_INVALID_ARG), (dict(Nk=0), fa.FA_ERR_INVALID_ARG)]:
        assert run(**kw) == st, kw


def test_fa_bwd_masked_rejects_before_any_hip_call(lib):
    p = [0x10000 * (i + 1) for i in range(10)]
    base = dict(B=2, H=1, Nq=16, Nk=32, d=64, causal=0, wl=-1, wr=-1, kl=0xB00000, scale=0.125)

    def run(**kw):
        a = dict(base)
        a.update(kw)
        return fa.fa_bwd_masked(*p, a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["causal"], a["wl"],
                                a["wr"], a["kl"], a["scale"], fa.FA_DTYPE_BF16, None)
    for kw, st in [(dict(wl=-2), fa.FA_ERR_INVALID_ARG), (dict(kl=0xB00002), fa.FA_ERR_INVALID_ARG),
                   (dict(kl=p[7] + 16), fa.FA_ERR_INVALID_ARG),   # key_lens inside dk
                   (dict(d=100), fa.FA_ERR_UNSUPPORTED), (dict(Nk=0), fa.FA_ERR_INVALID_ARG)]:
        assert run(**kw) == st, kw


def test_noalloc_split_rejects_before_any_hip_call(lib):
    # the static scratch holds FA_NOALLOC_SCRATCH_BYTES (16 MiB); a problem
    # whose split workspace is larger is refused before any HIP call, as are
    # the usual argument errors (fake, non-overlapping device addresses)
    B, H, Nq, Nk, d = 16, 32, 128, 8192, 128
    assert fa.fa_split_workspace_bytes(B, H, Nq, d, 64) > fa.NOALLOC_SCRATCH_BYTES
    p = [(i + 1) << 36 for i in range(5)]
    rc = fa.fa_fwd_split_qk_noalloc(*p, B, H, Nq, Nk, d, 0, 0.088, fa.FA_DTYPE_BF16, 64, None)
    assert rc == fa.FA_ERR_UNSUPPORTED and "static scratch" in fa.fa_status_string(rc)
    assert fa.fa_fwd_split_qk_noalloc(*p, B, H, Nq, Nk, d, 0, 0.088, fa.FA_DTYPE_BF16, 0, None) == \
        fa.FA_ERR_INVALID_ARG
    assert fa.fa_fwd_split_qk_noalloc(*p, B, H, Nq, Nk, d, 0, 0.088, fa.FA_DTYPE_BF16, 129, None) == \
        fa.FA_ERR_INVALID_ARG
    p16 = list(p)
    p16[1] += 8  # k not 16-byte aligned
    assert fa.fa_fwd_split_qk_noalloc(*p16, 1, 1, 1, 1024, 64, 0, 0.125, fa.FA_DTYPE_BF16, 2, None) == \
        fa.FA_ERR_INVALID_ARG
    assert fa.fa_fwd_split_qk_noalloc(*p, 1, 1, 1, 1024, 100, 0, 0.1, fa.FA_DTYPE_BF16, 2, None) == \
        fa.FA_ERR_UNSUPPORTED
