// fa_tiles.h -- key-tile ranges of one query tile (host and device).
//
// The split follows "How to optimise a Triton FlashAttention-2 kernel step by
// step with a profiler", Round 4, "Causal tile-skipping": key tiles that lie
// wholly below the first query of the tile and wholly inside the sequence are
// visited without a mask; the tiles from there up to the last query of the
// tile (or to the key count) are visited with the mask; nothing above the
// diagonal is visited. Without causality only a ragged last key tile is
// masked. Query row i and key j are absolute positions (causal: j <= i), so
// with fewer or more queries than keys the diagonal starts at the top-left
// corner, as in the page's keep test.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// Whether a forward kernel variant interleaves the exp2 work of tile j with
// the score MFMAs of tile j+1. DC: the head dims the kernel computes (the
// head dim rounded up to 32). Every 32-row variant does, except the 4-wave
// kernels computing 128 dims with a split, masks or padding, which run out of
// registers fused. The kernel and the host's count of executed MFMA work
// (fa_plan) both take it from here.
FA_HD constexpr bool fuses_exp(int DC, int waves, bool split, bool masks, bool padded)
{
    return !(DC == 128 && waves == 4 && (split || masks || padded));
}

struct KeyRange {
    int64_t unmasked_end;  // keys [0, unmasked_end) need no mask; a multiple of block_n
    int64_t masked_end;    // keys [unmasked_end, masked_end) are visited with the mask
};

// n_queries bounds the rows of the last query tile: with fewer queries than
// keys, no key tile above the last real row is visited (the pages' split
// takes the two counts equal, where this clip changes nothing).
FA_HD inline KeyRange key_range(int64_t q0, int64_t block_m, int64_t block_n, int64_t n_queries,
                                int64_t n_keys, bool causal)
{
    const int64_t full_end = (n_keys / block_n) * block_n;  // key tiles wholly inside [0, n_keys)
    KeyRange r;
    if (causal) {
        const int64_t below = (q0 / block_n) * block_n;  // rounded down to a key-tile boundary
        r.unmasked_end = below < full_end ? below : full_end;
        int64_t diag = q0 + block_m;  // one past the tile's last query row
        if (diag > n_queries) diag = n_queries;
        r.masked_end = diag < n_keys ? diag : n_keys;
    } else {
        r.unmasked_end = full_end;
        r.masked_end = n_keys;
    }
    return r;
}

// Key tiles visited by the query tile at q0: [0, unmasked) unmasked, then
// [unmasked, total) masked. Tile j covers keys [j*block_n, (j+1)*block_n).
struct TileSpan {
    int64_t unmasked;
    int64_t total;
};

FA_HD inline TileSpan tile_span(int64_t q0, int64_t block_m, int64_t block_n, int64_t n_queries,
                                int64_t n_keys, bool causal)
{
    const KeyRange r = key_range(q0, block_m, block_n, n_queries, n_keys, causal);
    TileSpan s;
    s.unmasked = r.unmasked_end / block_n;
    s.total = s.unmasked + (r.masked_end - r.unmasked_end + block_n - 1) / block_n;
    return s;
}

// Padding and sliding-window masks. "How to optimise a Triton FlashAttention-2
// kernel step by step with a profiler" ("Future articles") names them as the
// case where a row can see no key at all. Row i of a batch with key_len keys
// sees key j iff j < key_len, j >= i - window_left (window_left >= 0) and
// j <= i (causal) or j <= i + window_right (not causal, window_right >= 0);
// -1 leaves a window unbounded. The visible keys form one range [lo, hi),
// with lo and hi non-decreasing in i; an empty row has hi <= lo. A row can
// only be empty when hi is capped by key_len or the key count (the caps
// i + 1 and i + window_right + 1 always exceed i - window_left), and since lo
// keeps growing every later row is empty too: the non-empty rows of a tile
// are a prefix of it, and their ranges overlap or touch, so their union is
// the one range [lo of the first row, hi of the last row).
struct RowKeys {
    int64_t lo, hi;
};

FA_HD inline RowKeys row_keys(int64_t i, int64_t n_keys, bool causal, int64_t window_left,
                              int64_t window_right, int64_t key_len)
{
    int64_t hi = causal ? i + 1 : (window_right >= 0 ? i + window_right + 1 : n_keys);
    if (hi > n_keys) hi = n_keys;
    if (hi > key_len) hi = key_len;
    const int64_t lo = (window_left >= 0 && i - window_left > 0) ? i - window_left : 0;
    RowKeys r;
    r.lo = lo;
    r.hi = hi;
    return r;
}

// Key tiles of the rows [q0, min(q0 + block_m, n_queries)) under the masks:
// tiles [first, end) are exactly those holding a key some row sees (none when
// the first row is empty); within them the tiles [unmasked_begin,
// unmasked_end) are seen in full by every row and need no mask. Since lo and
// hi grow with the row, the first row bounds the start of the visited range
// and the end of the unmasked one, and the last row the other two.
struct MaskedSpan {
    int64_t first, unmasked_begin, unmasked_end, end;
};

FA_HD inline MaskedSpan masked_span(int64_t q0, int64_t block_m, int64_t block_n, int64_t n_queries,
                                    int64_t n_keys, bool causal, int64_t window_left,
                                    int64_t window_right, int64_t key_len)
{
    const int64_t last = (q0 + block_m < n_queries ? q0 + block_m : n_queries) - 1;
    const RowKeys a = row_keys(q0, n_keys, causal, window_left, window_right, key_len);
    const RowKeys z = row_keys(last, n_keys, causal, window_left, window_right, key_len);
    MaskedSpan s;
    s.first = a.lo / block_n;
    s.end = (z.hi + block_n - 1) / block_n;
    if (a.hi <= a.lo || s.end < s.first) s.end = s.first;
    int64_t ub = (z.lo + block_n - 1) / block_n, ue = a.hi / block_n;
    ub = ub < s.first ? s.first : (ub > s.end ? s.end : ub);
    ue = ue < ub ? ub : (ue > s.end ? s.end : ue);
    s.unmasked_begin = ub;
    s.unmasked_end = ue;
    return s;
}

}  // namespace fa
