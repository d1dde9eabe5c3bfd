// decode_waves.hip -- the bf16 decode step for groups of up to 8 query heads
// per KV head: the memory-bound hot path.
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps
// 2-4): for every sequence b and KV group g, the G query heads g*G ..
// g*G+G-1 of the single new query row attend to K/V head g of the cache,
// softmax(q K_g^T * scale) V_g over the ctx[b] cached keys.
//
// How (designed for CDNA4; flash-decoding on the inference-optimisation page
// §10.2-§10.3 is prior art, not the blueprint):
//  * Work list.  The (sequence, KV group) items are cut into tiles of 8 KB of
//    K (32 keys at d = 128); the flat tile list is cut into equal contiguous
//    slices, one per workgroup (two per CU).  Inside a slice, the run of
//    tiles that belongs to one item (a segment) is dealt round-robin to the
//    four waves.
//  * No barrier per tile.  Each wave streams its own tiles: the K and V rows
//    of the next tile are loaded straight into registers (coalesced 16-byte
//    loads, 1 KB per wave instruction) while the current tile is computed, so
//    every wave keeps 16 KB in flight and no LDS stage limits the depth.
//  * Scores: the wave copies its K tile into its own LDS buffer (rows padded
//    by 16 bytes) and lane (key t, head set) then reads the whole row t and
//    the q rows of its heads (an LDS broadcast) and forms full dot products
//    with v_dot2_f32_bf16.  One K row read from HBM serves all G heads.
//  * Online softmax per wave (inference-optimisation page §9.2.1) in exp2
//    units with a lazy reference maximum: it moves only when a score exceeds
//    it by 2^8, checked with one wave vote per tile, so the accumulators are
//    rarely rescaled (the final o / l cancels the reference).  P is rounded to
//    bf16 and l sums the rounded values.
//  * Weighted V sum straight from the V registers: lane (row group, 8-byte
//    column chunk) pairs two keys per v_perm and adds p_t v_t + p_t' v_t' for
//    all G heads with one v_dot2 per column; 4 columns x G heads of fp32
//    accumulators per lane.
//  * At the end of a segment the four waves' (m, l, o) are merged in LDS with
//    their common maximum (page §10.2); an item that lies wholly in the
//    segment is normalised and stored, a cut item leaves one partial per
//    workgroup for the merge kernel.
#include "common.h"
#include "kernels.h"
#include "worklist.h"

namespace gqa {
namespace {

constexpr int NT = 256;            // threads per workgroup; two workgroups per CU
constexpr int NW = NT / kWave;     // waves per workgroup
constexpr float TAU = 8.0f;        // lazy-rescale threshold (log2 units)

template <int D, int GP>
struct WCfg {
    static constexpr int RB = D * 2;            // bytes per cache row
    static constexpr int CPR = RB / 16;         // 16-byte chunks per row
    static constexpr int RPL = kWave / CPR;     // rows per 1 KB wave load
    static constexpr int TT = 8192 / RB;        // keys per tile (8 KB of K)
    static constexpr int NL = TT / RPL;         // 16-byte K loads per lane per tile
    static constexpr int VCPR = RB / 8;         // 8-byte V chunks per row
    static constexpr int VRPL = kWave / VCPR;   // V rows per 512 B wave load
    static constexpr int VNL = TT / VRPL;       // 8-byte V loads per lane per tile
    static constexpr int NP = VNL / 2;          // key pairs per lane per tile
    static constexpr int NGR = TT / 16;         // 16-key groups per tile
    static constexpr int KRS = RB + 16;         // LDS row stride of K: 16 lanes reading 16 rows hit distinct banks
    static constexpr int HS0 = kWave / TT;
    static constexpr int HS = HS0 < GP ? HS0 : GP;    // head sets in the score phase
    static constexpr int HPL = GP / HS;              // heads per score lane
    static constexpr int KD = GP >= 8 ? 1 : 2;       // K tiles in flight per wave (register budget)
    static constexpr int K_WAVE = TT * KRS;          // LDS K buffer per wave
    static constexpr int P_WAVE = VRPL * NP * GP;    // P words per wave (bf16 pairs)
    static constexpr int Q_BYTES = GP * RB;
    static constexpr int CMB = NW * GP * D * 4;      // wave partials, in the K buffers
    static_assert(NL == 8 && VNL == 16 && NP == 8, "tile shape");
    static_assert(GP >= 1 && GP <= 8 && (GP & (GP - 1)) == 0, "heads per group");
    static_assert(CMB <= NW * K_WAVE, "the merge area fits in the K buffers");
};

template <int N>
__device__ __forceinline__ void read_p(const uint32_t *src, uint32_t (&pp)[N])
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const uint4 x = *reinterpret_cast<const uint4 *>(src + i);
            pp[i] = x.x; pp[i + 1] = x.y; pp[i + 2] = x.z; pp[i + 3] = x.w;
        }
    } else if constexpr (N == 2) {
        const uint2 x = *reinterpret_cast<const uint2 *>(src);
        pp[0] = x.x; pp[1] = x.y;
    } else {
        pp[0] = src[0];
    }
}

template <int D, int GP>
__global__ __launch_bounds__(NT, 2) void decode_waves_kernel(RowAttnParams p)
{
    using C = WCfg<D, GP>;
    __shared__ __attribute__((aligned(16))) char lds_k[NW * C::K_WAVE];
    __shared__ __attribute__((aligned(16))) char lds_q[C::Q_BYTES];
    __shared__ __attribute__((aligned(16))) uint32_t lds_p[NW][C::P_WAVE];
    __shared__ float lds_alpha[NW][GP];
    __shared__ float lds_ml[NW][GP][2];
    __shared__ int32_t lds_prefix[kStreamRows + 1];
    __shared__ int32_t lds_nvis[kStreamRows];
    __shared__ int32_t lds_first[kStreamRows];
    __shared__ int32_t lds_newest[kStreamRows];
    __shared__ int lds_waves[NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
    const CacheView &cache = p.cache;
    const int G = p.G, H = p.H;

    // ---- decode step: the newest token's K/V rows into the cache ----------
    // The same bytes and the same skips as the append kernel.  This launch
    // never reads those cache rows (it takes the token from k_new / v_new),
    // so the copy only has to be done somewhere in it: thread (item, K or V,
    // 16-byte piece) loads its piece now and stores it once the first tiles
    // are on their way; further items, if any, are copied at the end.
    constexpr int IPW = NT / (2 * C::CPR);   // items per workgroup pass
    const int64_t cp_items = p.k_new != nullptr ? (int64_t)p.rows * cache.K : 0;
    const int64_t cp_stride = (int64_t)gridDim.x * IPW;
    const int64_t cp_first = (int64_t)blockIdx.x * IPW + tid / (2 * C::CPR);
    auto copy_dst = [&](int64_t it, int64_t &src) -> char * {
        const int which = (tid / C::CPR) & 1, piece = tid % C::CPR;
        const int b = (int)(p.row0 + it / cache.K), g = (int)(it % cache.K);
        const int pos = p.ctx_lens[b] - 1;
        if (pos < 0 || pos >= cache.capacity) return nullptr;
        const int64_t row = cache_row(cache, b, g, pos);
        if (row < 0) return nullptr;
        src = ((int64_t)b * cache.K + g) * C::RB + piece * 16 + (which ? p.v_new - p.k_new : 0);
        return (which ? cache.v : cache.k) + row * C::RB + piece * 16;
    };
    auto copy_rest = [&]() {
        for (int64_t it = cp_first + cp_stride; it < cp_items; it += cp_stride) {
            int64_t src = 0;
            char *dst = copy_dst(it, src);
            if (dst != nullptr) st16(dst, ld16(p.k_new + src));
        }
    };
    char *cp_to = nullptr;
    uint4 cp_val = make_uint4(0u, 0u, 0u, 0u);
    if (cp_first < cp_items) {
        int64_t src = 0;
        cp_to = copy_dst(cp_first, src);
        if (cp_to != nullptr) cp_val = ld16(p.k_new + src);
    }

    // ---- the flat tile list and this workgroup's slice ---------------------
    build_tables<NT>(p, C::TT, lds_prefix, lds_nvis, lds_first, lds_waves, p.k_new != nullptr ? lds_newest : nullptr);
    if (blockIdx.x == 0 && p.prefix != nullptr)   // the merge kernel reads it from the workspace
        for (int r = tid; r <= p.rows; r += NT) p.prefix[r] = lds_prefix[r];
    const int T = lds_prefix[p.rows];
    const int64_t W = gridDim.x;
    const int tau0 = (int)slice_start(blockIdx.x, T, W), tau1 = (int)slice_start(blockIdx.x + 1, T, W);
    if (tau0 >= tau1) {   // an empty slice (fewer tiles than workgroups)
        if (cp_to != nullptr) st16(cp_to, cp_val);
        copy_rest();
        return;
    }

    // K loads: lane = (row krow, 16-byte chunk kc); score phase: lane = (key
    // st, head set sh); V phase: lane = (row vr, 8-byte chunk vc: columns 4 vc ..)
    const int krow = lane / C::CPR, kc = lane % C::CPR;
    const int st = lane % C::TT, sh = lane / C::TT;
    const bool s_lane = sh < C::HS;
    const int qh = s_lane ? sh : 0;
    const int vr = lane / C::VCPR, vc = lane % C::VCPR;
    char *kw = lds_k + wave * C::K_WAVE;
    uint32_t *pw = lds_p[wave];
    uint16_t *pw16 = reinterpret_cast<uint16_t *>(pw);
    // where the score lane's probability goes: key st is V row st % VRPL of
    // V load 2 kk + half, so it pairs with the key VRPL rows away
    const int p_slot = (((st % C::VRPL) * C::NP + st / (2 * C::VRPL)) * GP + qh * C::HPL) * 2 + ((st / C::VRPL) & 1);

    // One segment: the tiles [tau, end) of the slice that belong to one item.
    struct Seg {
        int64_t row_g;    // query row (sequence) of the item
        int b, g;         // sequence and KV group
        int n_vis;        // end of the item's visible keys
        int new_key;      // decode step: the key read from k_new / v_new (-1: none)
        int lo, jlo;      // first visible key; its tile (the item's tile 0)
        int j_first;      // tile of the item at tau
        int tau, end;     // flat tile range
        int item0, tiles; // the item's flat range
        int n_w;          // tiles of this wave: j_first + wave + NW * i, i < n_w
    };
    auto make_seg = [&](int at) {
        const Cursor c = cursor_at(lds_prefix, lds_nvis, lds_first, p.rows, at, C::TT);
        Seg sg;
        sg.row_g = p.row0 + c.row;
        sg.b = (int)(sg.row_g / p.Sq);
        sg.g = c.g;
        sg.n_vis = c.n_vis;
        sg.new_key = p.k_new != nullptr ? lds_newest[c.row] : -1;
        sg.lo = c.lo;
        sg.jlo = c.jlo;
        sg.j_first = c.j;
        sg.tau = at;
        sg.end = min(tau1, c.item0 + c.tiles);
        sg.item0 = c.item0;
        sg.tiles = c.tiles;
        const int n_seg = sg.end - at;
        sg.n_w = n_seg > wave ? (n_seg - wave + NW - 1) / NW : 0;
        return sg;
    };

    // Where the rows of tile j of an item live.  A wave load covers rows of
    // one 16-key group, whose cache rows are consecutive (contiguous cache, or
    // one block of >= 16 tokens): a wave-uniform row base per group plus a
    // 32-bit lane offset.
    // A sliding window can leave the first keys of the item's first tile
    // outside: those keys are masked, and a 16-key group wholly outside is
    // not read at all (its block may have been recycled).
    struct TileRows {
        int64_t base[C::NGR];   // cache row of key 16 gi of the tile, -1: none
        int nvalid;             // keys of the tile below the end (<= 0: none)
        int first;              // first visible key of the tile
        int new_row;            // tile row read from k_new / v_new (-1: none)
        int64_t new_off;        // byte offset of that row in k_new / v_new
    };
    auto tile_rows = [&](int lb, int lg, int l_lo, int l_nvis, int l_new, int j) {
        TileRows t;
        const int key0 = j * C::TT;   // j: tile of the row
        t.nvalid = min(C::TT, l_nvis - key0);
        t.first = max(0, l_lo - key0);
        t.new_row = l_new >= key0 && l_new < key0 + C::TT ? l_new - key0 : -1;
        t.new_off = ((int64_t)lb * cache.K + lg) * C::RB;
#pragma unroll
        for (int gi = 0; gi < C::NGR; ++gi)
            t.base[gi] = 16 * gi < t.nvalid && 16 * gi + 16 > t.first ? cache_row_wave(cache, lb, lg, key0 + 16 * gi) : -1;
        return t;
    };
    const uint32_t k_off = (uint32_t)(krow * C::RB + kc * 16);
    const uint32_t v_off = (uint32_t)(vr * C::RB + vc * 8);
    auto load_k = [&](const TileRows &t, uint4 (&kr)[C::NL]) {
#pragma unroll
        for (int i = 0; i < C::NL; ++i) {
            const int r0 = i * C::RPL;                       // first tile row of the load
            const int64_t base = t.base[r0 / 16];
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (base >= 0 && r0 + krow < t.nvalid)
                x = ld16_nt(r0 + krow == t.new_row ? p.k_new + t.new_off + kc * 16 : cache.k + (base + r0 % 16) * C::RB + k_off);
            kr[i] = x;
        }
    };
    auto load_v = [&](const TileRows &t, uint2 (&vv)[C::VNL]) {
#pragma unroll
        for (int i = 0; i < C::VNL; ++i) {
            const int r0 = i * C::VRPL;
            const int64_t base = t.base[r0 / 16];
            uint2 y = make_uint2(0u, 0u);
            if (base >= 0 && r0 + vr < t.nvalid)
                y = ld8_nt(r0 + vr == t.new_row ? p.v_new + t.new_off + vc * 8
                                                : cache.v + (base + r0 % 16) * C::RB + v_off);
            vv[i] = y;
        }
    };
    // this thread's 16 bytes of the q rows of a segment's item (padded heads are zero)
    const bool q_thread = tid < GP * C::CPR;
    const int q_r = tid / C::CPR, q_ch = tid % C::CPR;
    auto load_q = [&](const Seg &sg) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (q_thread && q_r < G) x = ld16(p.q + ((sg.row_g * H + (int64_t)sg.g * G + q_r) * D) * 2 + q_ch * 16);
        return x;
    };

    // The first two tiles of this wave's stream at or after flat tile `at`:
    // the wave's tiles of the segments from there on (none: no rows).
    auto no_rows = [&]() {
        TileRows t;
#pragma unroll
        for (int gi = 0; gi < C::NGR; ++gi) t.base[gi] = -1;
        t.nvalid = 0;
        t.first = 0;
        t.new_row = -1;
        t.new_off = 0;
        return t;
    };
    auto stream_from = [&](int at, TileRows &t1, TileRows &t2) {
        t1 = no_rows();
        t2 = no_rows();
        int found = 0;
        while (at < tau1 && found < C::KD) {
            const Seg sg = make_seg(at);
            for (int k = 0; k < sg.n_w && found < C::KD; ++k, ++found) {
                const TileRows t = tile_rows(sg.b, sg.g, sg.lo, sg.n_vis, sg.new_key, sg.jlo + sg.j_first + wave + NW * k);
                if (found == 0) t1 = t;
                else t2 = t;
            }
            at = sg.end;
        }
    };

    // The wave's tiles form one stream across segments.  Step i (stream
    // position gi): copy K(i) from its register buffer to LDS and start
    // K(i + KD) into that buffer; add P(i-1) V(i-1) from the V registers;
    // start V(i) into them; score tile i into P(i).  K has KD steps to
    // arrive, V one, and V needs a single register buffer.
    uint4 kA[C::NL], kB[C::NL];
    uint2 vbuf[C::VNL];
    int gi = 0;
    Seg cur = make_seg(tau0);
    TileRows r1, r2;   // rows of the stream's next tiles (K already started)
    stream_from(tau0, r1, r2);
    {
        const uint4 x = load_q(cur);
        load_k(r1, kA);
        if constexpr (C::KD == 2) load_k(r2, kB);
        if (q_thread) *reinterpret_cast<uint4 *>(lds_q + q_r * C::RB + q_ch * 16) = x;
        if (cp_to != nullptr) st16(cp_to, cp_val);
        __syncthreads();
    }
    for (;;) {
        const bool has_next = cur.end < tau1;
        const Seg nxt = has_next ? make_seg(cur.end) : cur;
        const int n_w = cur.n_w;
        TileRows after1, after2;   // the stream's first tiles after this segment
        stream_from(cur.end, after1, after2);

        // ---- this wave's tiles of the segment: j_first + wave + NW * i -------
        float m_ref[C::HPL], l_run[C::HPL];
#pragma unroll
        for (int h = 0; h < C::HPL; ++h) { m_ref[h] = -INFINITY; l_run[h] = 0.f; }
        float acc[GP][4];
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;

        // o = o * alpha + sum_t p_t v_t for the tile whose V is in vbuf
        auto pv = [&](bool rescale) {
            if (rescale) {
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    const float al = lds_alpha[wave][h];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[h][e] *= al;
                }
            }
#pragma unroll
            for (int kk = 0; kk < C::NP; ++kk) {
                const uint2 a = vbuf[2 * kk], bb = vbuf[2 * kk + 1];   // rows 2kk*VRPL + vr and VRPL later
                uint32_t vv[4];
                vv[0] = pair_lo(a.x, bb.x); vv[1] = pair_hi(a.x, bb.x);
                vv[2] = pair_lo(a.y, bb.y); vv[3] = pair_hi(a.y, bb.y);
                uint32_t pp[GP];
                read_p<GP>(pw + (vr * C::NP + kk) * GP, pp);
#pragma unroll
                for (int h = 0; h < GP; ++h)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[h][e] = dot2_bf16(pp[h], vv[e], acc[h][e]);
            }
        };

        bool pend_rescale = false;
        for (int i = 0; i < n_w; ++i, ++gi) {
            const TileRows rows = r1;   // tile i
            // rows of the tile KD steps ahead in the stream
            const int ia = i + C::KD;
            const TileRows ra = ia < n_w ? tile_rows(cur.b, cur.g, cur.lo, cur.n_vis, cur.new_key, cur.jlo + cur.j_first + wave + NW * ia)
                                         : (ia == n_w ? after1 : after2);
            // K(i) -> this wave's LDS buffer (padded rows); start K(i + KD) in its place
            auto k_step = [&](uint4 (&kx)[C::NL]) {
#pragma unroll
                for (int ii = 0; ii < C::NL; ++ii)
                    *reinterpret_cast<uint4 *>(kw + (ii * C::RPL + krow) * C::KRS + kc * 16) = kx[ii];
                load_k(ra, kx);
            };
            if (C::KD == 2 && (gi & 1)) k_step(kB);
            else k_step(kA);
            if constexpr (C::KD == 2) { r1 = r2; r2 = ra; }
            else r1 = ra;
            // P(i-1) V(i-1), then start V(i)
            if (i > 0) pv(pend_rescale);
            load_v(rows, vbuf);

            // ---- scores of tile i ----------------------------------------------
            float sc[C::HPL];
            {
                float a0[C::HPL], a1[C::HPL];
#pragma unroll
                for (int h = 0; h < C::HPL; ++h) { a0[h] = 0.f; a1[h] = 0.f; }
#pragma unroll
                for (int ch = 0; ch < C::CPR; ++ch) {
                    const uint4 kv = *reinterpret_cast<const uint4 *>(kw + st * C::KRS + ch * 16);
#pragma unroll
                    for (int h = 0; h < C::HPL; ++h) {
                        const uint4 qv = *reinterpret_cast<const uint4 *>(lds_q + (qh * C::HPL + h) * C::RB + ch * 16);
                        a0[h] = dot2_bf16(qv.x, kv.x, a0[h]);
                        a1[h] = dot2_bf16(qv.y, kv.y, a1[h]);
                        a0[h] = dot2_bf16(qv.z, kv.z, a0[h]);
                        a1[h] = dot2_bf16(qv.w, kv.w, a1[h]);
                    }
                }
                const bool valid = s_lane && st < rows.nvalid && st >= rows.first;
#pragma unroll
                for (int h = 0; h < C::HPL; ++h) sc[h] = valid ? (a0[h] + a1[h]) * p.scale_log2 : -INFINITY;
            }

            // ---- lazy reference maximum: one vote per tile ---------------------
            bool need = false;
#pragma unroll
            for (int h = 0; h < C::HPL; ++h) need |= sc[h] > m_ref[h] + TAU;
            const bool rescale = __ballot(need) != 0;
            if (rescale) {
#pragma unroll
                for (int h = 0; h < C::HPL; ++h) {
                    const float mt = group_max<C::TT>(sc[h]);
                    const float mn = mt > m_ref[h] + TAU ? mt : m_ref[h];
                    const float al = mn == m_ref[h] ? 1.f : fast_exp2(m_ref[h] - mn);   // 0 on the first tile
                    l_run[h] *= al;
                    m_ref[h] = mn;
                    if (s_lane && st == 0) lds_alpha[wave][qh * C::HPL + h] = al;
                }
            }
            pend_rescale = rescale;
            // ---- P (bf16) for the V sum; l sums the rounded values -------------
#pragma unroll
            for (int h = 0; h < C::HPL; ++h) {
                const float pk = fast_exp2(sc[h] - m_ref[h]);   // 0 for keys past the end
                const uint32_t pb = f32_to_bf16_rne(pk);
                l_run[h] += __uint_as_float(pb << 16);
                if (s_lane) pw16[p_slot + 2 * h] = (uint16_t)pb;
            }
        }
        if (n_w > 0) pv(pend_rescale);   // the last tile's V sum

        // the next item's q rows are loaded while the pieces are merged
        const uint4 q_next = has_next ? load_q(nxt) : make_uint4(0u, 0u, 0u, 0u);

        // ---- merge the waves' pieces of the segment ---------------------------
#pragma unroll
        for (int h = 0; h < GP; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (C::VCPR <= 16) acc[h][e] = sum_xor<16>(acc[h][e]);
                acc[h][e] = sum_xor<32>(acc[h][e]);
            }
#pragma unroll
        for (int h = 0; h < C::HPL; ++h) l_run[h] = group_sum<C::TT>(l_run[h]);
        __syncthreads();   // every wave is done with its K buffer and q: the K buffers become the merge area
        float *cmb = reinterpret_cast<float *>(lds_k);   // [NW][GP][D]
        if (lane < C::VCPR) {
#pragma unroll
            for (int h = 0; h < GP; ++h)
                *reinterpret_cast<float4 *>(cmb + (wave * GP + h) * D + lane * 4) =
                    make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        }
        if (s_lane && st == 0) {
#pragma unroll
            for (int h = 0; h < C::HPL; ++h) {
                lds_ml[wave][qh * C::HPL + h][0] = n_w > 0 ? m_ref[h] : -INFINITY;
                lds_ml[wave][qh * C::HPL + h][1] = n_w > 0 ? l_run[h] : 0.f;
            }
        }
        __syncthreads();
        const bool whole = cur.tau == cur.item0 && cur.end == cur.item0 + cur.tiles;
        const int slot = tau0 < cur.item0 ? 1 : 0;
        const int64_t head0 = cur.row_g * H + (int64_t)cur.g * G;
        for (int idx = tid; idx < GP * D / 4; idx += NT) {
            const int h = idx / (D / 4), col = (idx % (D / 4)) * 4;
            if (h >= G) continue;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_ml[w][h][0]);
            float L = 0.f;
            float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = lds_ml[w][h][0];
                if (mw == -INFINITY) continue;   // a wave without tiles in the segment
                const float wt = fast_exp2(mw - M);
                L += lds_ml[w][h][1] * wt;
                const float4 o = *reinterpret_cast<const float4 *>(cmb + (w * GP + h) * D + col);
                O.x += o.x * wt;
                O.y += o.y * wt;
                O.z += o.z * wt;
                O.w += o.w * wt;
            }
            if (whole) {
                const float inv = 1.f / L;
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + (head0 + h) * D + col) =
                    make_uint2(pack_bf16x2(O.x * inv, O.y * inv), pack_bf16x2(O.z * inv, O.w * inv));
            } else {
                const int64_t sr = ((int64_t)blockIdx.x * 2 + slot) * G + h;
                *reinterpret_cast<float4 *>(p.ws_o + sr * D + col) = O;
                if (col == 0) {
                    p.ws_ml[sr * 2] = M;
                    p.ws_ml[sr * 2 + 1] = L;
                }
            }
        }
        if (!has_next) break;
        if (q_thread) *reinterpret_cast<uint4 *>(lds_q + q_r * C::RB + q_ch * 16) = q_next;
        __syncthreads();   // the merge area is free again and the next q is in place
        cur = nxt;
    }
    copy_rest();
}

template <int D, int GP>
hipError_t launch_w(const RowAttnParams &p0, hipStream_t s)
{
    RowAttnParams p = p0;
    if (p.wgs_override > 0) p.num_wgs = p.wgs_override;
    hipLaunchKernelGGL((decode_waves_kernel<D, GP>), dim3(p.num_wgs), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_pieces(p, WCfg<D, GP>::TT, p.num_wgs, s);
}

template <int D>
hipError_t launch_wd(const RowAttnParams &p, int gp, hipStream_t s)
{
    switch (gp) {
    case 1: return launch_w<D, 1>(p, s);
    case 2: return launch_w<D, 2>(p, s);
    case 4: return launch_w<D, 4>(p, s);
    case 8: return launch_w<D, 8>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_waves_supported(const RowAttnParams &p, int gp)
{
    // paged caches need blocks of at least 16 tokens (a wave load stays in one block)
    return !p.prefill && !p.whole_items && p.cache.elem_bytes == 2 && gp <= 8 &&
           (p.cache.d == 64 || p.cache.d == 128) && p.num_wgs <= kStreamWGs &&
           (p.cache.block_table == nullptr || p.cache.log2_bs >= 4);
}

hipError_t launch_decode_waves(const RowAttnParams &p, int gp, hipStream_t stream)
{
    if (!decode_waves_supported(p, gp)) return hipErrorInvalidValue;
    return p.cache.d == 128 ? launch_wd<128>(p, gp, stream) : launch_wd<64>(p, gp, stream);
}

}  // namespace gqa
