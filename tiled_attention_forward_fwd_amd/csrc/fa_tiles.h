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

}  // namespace fa
