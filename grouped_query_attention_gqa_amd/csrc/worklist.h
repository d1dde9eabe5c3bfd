// worklist.h -- the flat tile list shared by the row-attention kernels
// (internal).
//
// Every (query row, KV group) item is cut into tiles of `tt` keys; the tiles
// of all items of one launch form one flat list, ordered by row, then KV
// group, then key.  Workgroup w of W takes the contiguous slice
// [w*T/W, (w+1)*T/W) of the T tiles, so ragged and paged contexts are
// balanced exactly.  The per-row tables live in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace gqa {

// End of the visible keys of query row `row` (b * Sq + i): keys below it
// may be seen; clamped to the cache capacity.
__device__ __forceinline__ int row_visible(const RowAttnParams &p, int64_t row)
{
    const int b = (int)(row / p.Sq);
    const int i = (int)(row % p.Sq);
    int64_t n;
    if (!p.prefill) {
        n = p.ctx_lens[b];
    } else {
        const int64_t start = p.start_pos[b];
        n = p.causal ? start + i + 1 : start + p.Sq;
    }
    if (n > p.cache.capacity) n = p.cache.capacity;
    if (n < 0) n = 0;
    return (int)n;
}

// First visible key of the row: 0, or with a sliding window of W positions
// (inference-optimisation page §6.4.1) the oldest of the W most recent
// positions up to the row's own, qpos + 1 - W.  A decode row that carries mq
// query positions (the newest mq tokens) takes the window of the oldest.
__device__ __forceinline__ int row_first(const RowAttnParams &p, int64_t row, int n_end)
{
    if (p.window <= 0) return 0;
    const int b = (int)(row / p.Sq);
    const int i = (int)(row % p.Sq);
    const int64_t qpos = p.prefill ? (int64_t)p.start_pos[b] + i : (int64_t)p.ctx_lens[b] - (p.mq > 1 ? p.mq : 1);
    int64_t lo = qpos + 1 - p.window;
    if (lo < 0) lo = 0;
    if (lo > n_end) lo = n_end;
    return (int)lo;
}

// Tiles of `tt` keys an item with visible keys [lo, n) covers: tiles lo/tt
// .. ceil(n/tt)-1 of the row.
__device__ __forceinline__ int item_tiles(int lo, int n, int tt) { return n > lo ? (n + tt - 1) / tt - lo / tt : 0; }

// For the rows of this launch (local rows 0 .. rows-1, at most kStreamRows):
// keys first[r] .. nvis[r]-1 are visible, prefix[r] = K * sum_{r' < r} tiles(r'),
// prefix[rows] = the number of tiles T.  Every thread of the workgroup calls
// it; thread i handles the consecutive rows i*per .. i*per+per-1, so any row
// count up to kStreamRows is covered whatever the workgroup size.
// With `newest` (decode step only), newest[r] is the key of the row's newest
// token, ctx - 1, or -1 when it lies past the cache capacity.
template <int NT>
__device__ void build_tables(const RowAttnParams &p, int tt, int32_t *prefix, int32_t *nvis, int32_t *first,
                             int *lds_waves, int32_t *newest = nullptr)
{
    static_assert(kStreamRows % NT == 0, "rows per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rows = p.rows;
    const int per = (rows + NT - 1) / NT;
    const int r0 = tid * per;
    const int items = p.cache.K * (p.kv_split > 1 ? p.kv_split : 1);   // items per row
    int local = 0;
    for (int k = 0; k < per; ++k) {
        const int r = r0 + k;
        if (r < rows) {
            const int n = row_visible(p, p.row0 + r);
            const int lo = row_first(p, p.row0 + r, n);
            nvis[r] = n;
            first[r] = lo;
            if (newest != nullptr) {
                const int raw = p.ctx_lens[p.row0 + r];
                newest[r] = raw >= 1 && raw <= p.cache.capacity ? raw - 1 : -1;
            }
            local += item_tiles(lo, n, tt);
        }
    }
    int x = local;   // inclusive scan over the wave, then over the waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) lds_waves[wave] = x;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += lds_waves[w];
    int run = before + x - local;
    for (int k = 0; k < per; ++k) {
        const int r = r0 + k;
        if (r < rows) {
            prefix[r] = run * items;
            run += item_tiles(first[r], nvis[r], tt);
        }
    }
    if (tid == NT - 1) prefix[rows] = (before + x) * items;
    __syncthreads();
}

struct Cursor {
    int row;       // local query row
    int g;         // KV group
    int j;         // tile within the item (the item's tile 0 is tile jlo of the row)
    int tiles;     // tiles of the item
    int n_vis;     // end of the visible keys of the row
    int lo;        // first visible key of the row
    int jlo;       // row tile of the item's first tile (lo / tt)
    int item0;     // flat index of the item's first tile
};

__device__ __forceinline__ Cursor cursor_at(const int32_t *prefix, const int32_t *nvis, const int32_t *first, int rows,
                                            int tau, int tt)
{
    // last row whose prefix is <= tau (rows without tiles share their prefix)
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= tau) lo = mid; else hi = mid - 1;
    }
    Cursor c;
    c.row = lo;
    c.n_vis = nvis[lo];
    c.lo = first[lo];
    c.jlo = c.lo / tt;
    c.tiles = item_tiles(c.lo, c.n_vis, tt);
    const int off = tau - prefix[lo];
    c.g = off / c.tiles;
    c.j = off % c.tiles;
    c.item0 = prefix[lo] + c.g * c.tiles;
    return c;
}

__device__ __forceinline__ void cursor_next(const int32_t *nvis, const int32_t *first, int rows, int K, Cursor &c,
                                            int tt)
{
    if (++c.j < c.tiles) return;
    c.j = 0;
    c.item0 += c.tiles;
    if (++c.g < K) return;
    c.g = 0;
    do {
        ++c.row;
        if (c.row >= rows) return;
        c.n_vis = nvis[c.row];
        c.lo = first[c.row];
        c.jlo = c.lo / tt;
        c.tiles = item_tiles(c.lo, c.n_vis, tt);
    } while (c.tiles == 0);
}

__device__ __forceinline__ int64_t slice_start(int64_t w, int64_t T, int64_t W) { return w * T / W; }

// The workgroup whose slice holds flat tile x: the last w whose slice starts
// at or before x, i.e. the largest w with w T < (x + 1) W.  Its slice is never
// empty (it runs to the next start, which lies past x).
__device__ __forceinline__ int64_t slice_owner(int64_t x, int64_t T, int64_t W) { return ((x + 1) * W - 1) / T; }

// With no more tiles than workgroups (T <= W) a slice holds at most one tile,
// so the partial of tile x is its slice's first segment, in workspace slot 0.
__device__ __forceinline__ int64_t sparse_slot(int64_t x, int64_t T, int64_t W) { return 2 * slice_owner(x, T, W); }

}  // namespace gqa
