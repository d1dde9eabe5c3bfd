// stream_attention.hip -- grouped-query attention of single query rows on the
// vector ALUs: the decode step (memory-bound) and the fp32 prefill.
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps 2-4):
// for every query row and every KV group g, the G query heads g*G .. g*G+G-1
// attend to K/V head g with softmax(q K_g^T * scale) V_g over the row's
// visible keys.
//
// How (designed for CDNA4; flash-decoding on the inference-optimisation page
// §10.2-§10.3 is prior art, not the blueprint):
//  * Work list.  Every (query row, KV group) item is cut into tiles of 8 KB
//    of K (32 keys at d = 128 in bf16); the tiles of all items form one flat
//    list and each of the W workgroups (two per CU) takes an equal contiguous
//    slice of it.  Ragged and paged contexts are
//    balanced exactly, and no workgroup starts just to find nothing to do.
//  * Memory pipeline.  K, V (and the item's q rows) of the next tiles are in
//    flight as LDS-direct loads (global_load_lds_dwordx4: HBM -> LDS without
//    registers) while the scores of one tile and the V sum of the previous
//    one are computed, with one barrier per tile; the loads of a tile are
//    waited for with an explicit vmcnt, so the pipeline also runs across
//    item boundaries.  Every K and V row is read from HBM once and
//    then serves all G heads of its group from LDS (the group broadcast).
//  * Scores: thread (head r, key t) computes the full dot product of its
//    register-resident q row with the K row from LDS (v_dot2_f32_bf16: two
//    bf16 products per instruction into fp32).  K rows are XOR-swizzled in LDS
//    so 16 lanes reading 16 rows hit 16 bank groups.
//  * Online softmax per item (inference-optimisation page §9.2.1), in exp2
//    units; the reference maximum only moves when a tile maximum exceeds it
//    by 2^8, so the accumulators are rarely rescaled (the final o / l
//    cancels the reference).
//  * Weighted V sum: wave w owns column pieces w*CPW .. (w+1)*CPW-1 of all G
//    heads; a lane holds fp32 accumulators for up to 8 heads x 8 columns and
//    two keys at a time are paired (v_perm) so one v_dot2 adds
//    p_t v_t + p_t+1 v_t+1.  Key groups are reduced with lane shuffles.
//  * An item whose tiles all fall in one workgroup is normalised and stored
//    there; an item cut by slice boundaries leaves one partial (m, l, o) per
//    workgroup and merge_pieces_kernel combines them with their global max
//    and sum (page §10.2) after the main kernel.
#include <utility>

#include "common.h"
#include "kernels.h"
#include "worklist.h"

namespace gqa {
namespace {

constexpr int NT = 256;            // threads per workgroup (4 waves); two workgroups per CU
constexpr int NW = NT / kWave;     // waves per workgroup
constexpr float TAU = 8.0f;        // lazy-rescale threshold (log2 units)
constexpr int LDS_LIMIT = 80 * 1024;   // half of a CU's 160 KB: two workgroups per CU
constexpr int K_TILE_BYTES = 8192; // bytes of K (and of V) per tile

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// 16 zero bytes: the source of LDS-direct loads for rows past the end of an
// item and for padded heads.
__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};

// One LDS-direct 16-byte load per lane: lane i's bytes land at
// lds_wave_base + 16 i.  Written as inline assembly so that the compiler does
// not track these loads: it would otherwise wait for every one in flight
// before each LDS read.  The kernel waits for them itself (wait_tiles).
__device__ __forceinline__ void dma16(const void *src, void *lds_wave_base)
{
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_t *)lds_wave_base;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
#pragma clang diagnostic pop
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt vmcnt(n) for a run-time n in [0, kMaxWait]: a branch tree over
// the immediates (n is wave-uniform, so this is scalar code).
constexpr int kMaxWait = 31;
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_range(int n)
{
    if constexpr (LO == HI) {
        wait_vm<LO>();
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n <= MID) wait_vm_range<LO, MID>(n);
        else wait_vm_range<MID + 1, HI>(n);
    }
}
// Loads return in issue order, so "at most n loads in flight" means every
// load issued before the last n has landed.  n above the range waits for
// more than needed, which is always safe.
__device__ __forceinline__ void wait_vm_dyn(int n) { wait_vm_range<0, kMaxWait>(n < kMaxWait ? n : kMaxWait); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

// Workgroup barrier without the memory fence of __syncthreads() (that fence
// would wait for every LDS-direct load in flight).  LDS stores are completed
// first; the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier()
{
    wait_lds();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D, int GP, bool BF16>
struct Cfg {
    static constexpr int ES = BF16 ? 2 : 4;           // element bytes
    static constexpr int RB = D * ES;                 // row bytes
    static constexpr int CPR = RB / 16;               // 16-byte pieces per row
    static constexpr int CE = 16 / ES;                // elements per piece
    static constexpr int TT = K_TILE_BYTES / RB;      // keys per tile
    static constexpr int RPK = 1024 / RB;             // rows per 1 KB load block
    static constexpr int LK = TT * RB / 1024 / NW;    // LDS-direct loads per wave per tile, each of K and V
    static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
    static constexpr int Q_BYTES = GP * RB;
    static constexpr int QN = (Q_BYTES + 1023) / 1024; // 1 KB q loads per tile
    static constexpr int Q_SLOT = QN * 1024;
    static constexpr int K_BYTES = TT * RB;
    static constexpr int STAGE = 2 * K_BYTES + Q_SLOT;
    // score phase
    static constexpr int TPH0 = (NT / GP) < kWave ? (NT / GP) : kWave;
    static constexpr int TPH = TPH0 < TT ? TPH0 : TT;  // threads per head
    static constexpr int NS = TT / TPH;                // keys per score thread
    static constexpr int S_THREADS = GP * TPH;
    static constexpr int QW = RB / 4;                  // 32-bit words of a q row
    // weighted-sum phase
    static constexpr int CPW = CPR / NW;               // column pieces per wave
    static constexpr int HPT = GP < 8 ? GP : 8;        // heads per lane
    static constexpr int HG = GP / HPT;                // head sets
    static constexpr int TGL = kWave / (CPW * HG);     // key groups per wave
    static constexpr int TPT = TT / TGL;               // keys per lane per tile
    // LDS
    static constexpr int P_BYTES = TT * GP * (BF16 ? 2 : 4);
    static constexpr int OTHER = 2 * P_BYTES + 6 * GP * 4 + (2 * kStreamRows + 1) * 4 + NW * 4 + 256;
    // two workgroups per CU when three stages fit in half the LDS, else one
    static constexpr int LIMIT = (LDS_LIMIT - OTHER) / STAGE >= 3 ? LDS_LIMIT : 2 * LDS_LIMIT;
    static constexpr int NBUF0 = (LIMIT - OTHER) / STAGE;
    static constexpr int NBUF = NBUF0 > 6 ? 6 : NBUF0;
    static constexpr int A = NBUF - 1;                 // tiles in flight
    // q loads per wave of a tile that needs q (waves below Q_EXTRA load one more block)
    static constexpr int QL = QN / NW;
    static constexpr int Q_EXTRA = QN % NW;
    // loads one wave issues per pipeline iteration (K and q of one tile, V of another)
    static constexpr int MAX_ITER_LOADS = 2 * LK + QL + (Q_EXTRA ? 1 : 0);

    static_assert(LK >= 1 && LK * 1024 * NW == K_BYTES, "K tile does not split into 1 KB loads per wave");
    static_assert(CPW >= 1 && CPW * NW == CPR, "column pieces do not split over the waves");
    static_assert(TGL >= 1 && TGL * CPW * HG == kWave, "weighted-sum lanes");
    static_assert(!BF16 || TPT % 2 == 0, "key pairs need an even key count per lane");
    static_assert(NS * TPH == TT && S_THREADS <= NT, "score layout");
    static_assert(NBUF >= 2, "stage count");
    static_assert(MAX_ITER_LOADS < 32 && (A - 1) * MAX_ITER_LOADS <= kMaxWait, "load counts of the pipeline waits");
};

// ---------------------------------------------------------------------------
// main kernel
// ---------------------------------------------------------------------------

template <int D, int GP, bool BF16>
__global__ __launch_bounds__(NT, (Cfg<D, GP, BF16>::LIMIT > LDS_LIMIT ? 1 : 2)) void stream_attention_kernel(RowAttnParams p)
{
    using C = Cfg<D, GP, BF16>;
    __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::STAGE];
    __shared__ __attribute__((aligned(16))) char lds_p[2 * C::P_BYTES];   // double-buffered
    __shared__ float lds_alpha[2][GP], lds_m[2][GP], lds_l[2][GP];
    __shared__ int32_t lds_prefix[kStreamRows + 1];
    __shared__ int32_t lds_nvis[kStreamRows];
    __shared__ int32_t lds_first[kStreamRows];
    __shared__ int lds_waves[NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const CacheView &cache = p.cache;
    const int G = p.G, H = p.H;

    // ---- the flat tile list and this workgroup's slice ---------------------
    build_tables<NT>(p, C::TT, lds_prefix, lds_nvis, lds_first, lds_waves);
    if (blockIdx.x == 0 && p.prefix != nullptr)   // the merge kernel reads it from the workspace
        for (int r = tid; r <= p.rows; r += NT) p.prefix[r] = lds_prefix[r];
    const int T = lds_prefix[p.rows];
    const int64_t W = gridDim.x;
    int tau0 = (int)slice_start(blockIdx.x, T, W), tau1 = (int)slice_start(blockIdx.x + 1, T, W);
    if (p.whole_items) {
        // slices start at item starts, so no item is cut (no partial pieces)
        auto snap = [&](int tau) {
            if (tau >= T) return T;
            const Cursor c = cursor_at(lds_prefix, lds_nvis, lds_first, p.rows, tau, C::TT);
            return c.j == 0 ? tau : c.item0 + c.tiles;
        };
        tau0 = snap(tau0);
        tau1 = snap(tau1);
        if (blockIdx.x == 0) {
            // rows without a visible key (a violated contract) get zeros
            for (int r = 0; r < p.rows; ++r) {
                if (lds_nvis[r] > 0) continue;
                for (int idx = tid; idx < H * D; idx += NT) {
                    const int64_t o = ((int64_t)p.row0 + r) * H * D + idx;
                    if constexpr (BF16) reinterpret_cast<uint16_t *>(p.out)[o] = 0;
                    else reinterpret_cast<float *>(p.out)[o] = 0.f;
                }
            }
        }
    }
    if (tau0 >= tau1) return;
    const bool q_extra = wave < C::Q_EXTRA;
    const int q_loads = C::QL + (q_extra ? 1 : 0);

    // ---- LDS-direct loads of one tile's K (and q) or V into a stage ----------
    // Source address of this lane's 16 bytes in 1 KB block `blk` of the tile
    // (nullptr: the row is past the item's keys or its block id is invalid).
    auto row_src = [&](const Cursor &c, int blk) -> int64_t {
        const int tile0 = (c.jlo + c.j) * C::TT;
        const int nvalid = min(C::TT, c.n_vis - tile0);
        const int first = c.lo - tile0;   // keys of the tile before it are outside a sliding window
        const int t = blk * C::RPK + lane / C::CPR;
        if (blk * C::RPK >= nvalid || blk * C::RPK + C::RPK <= first) return -1;
        const int b = (int)(((int64_t)p.row0 + c.row) / p.Sq);
        if (cache.block_table == nullptr || cache.log2_bs >= 4) {
            // the block's RPK consecutive rows lie in one 16-row group,
            // hence in one cache block: one lookup per wave
            const int64_t r0 = cache_row_wave(cache, b, c.g, tile0 + blk * C::RPK);
            return (r0 >= 0 && t < nvalid && t >= first) ? r0 + (t - blk * C::RPK) : -1;
        }
        return t < nvalid && t >= first ? cache_row(cache, b, c.g, tile0 + t) : -1;   // blocks shorter than 16 rows
    };
    // K rows are stored XOR-swizzled: piece x of row t lands in slot x ^ (t & SWZ).
    auto issue_k = [&](const Cursor &c, bool with_q, int stage) -> int {
        char *base = smem + stage * C::STAGE;
#pragma unroll
        for (int k = 0; k < C::LK; ++k) {
            const int blk = wave + NW * k;
            const int t = blk * C::RPK + lane / C::CPR;
            const int piece = lane % C::CPR;
            const int64_t r = row_src(c, blk);
            const void *src = r >= 0 ? (const void *)(cache.k + r * C::RB + (piece ^ (t & C::SWZ)) * 16)
                                     : (const void *)&kZero16;
            dma16(src, base + blk * 1024);
        }
        if (!with_q) return C::LK;
        const int64_t row_g = (int64_t)p.row0 + c.row;
        for (int k = 0; k < q_loads; ++k) {
            const int qblk = wave + NW * k;
            const int off = qblk * 1024 + lane * 16;
            const int r = off / C::RB;
            const void *src = &kZero16;
            if (r < G)
                src = p.q + ((row_g * H + (int64_t)c.g * G + r) * D) * C::ES + (off % C::RB);
            dma16(src, base + 2 * C::K_BYTES + qblk * 1024);
        }
        return C::LK + q_loads;
    };
    auto issue_v = [&](const Cursor &c, int stage) -> int {
        char *base = smem + stage * C::STAGE + C::K_BYTES;
#pragma unroll
        for (int k = 0; k < C::LK; ++k) {
            const int blk = wave + NW * k;
            const int piece = lane % C::CPR;
            const int64_t r = row_src(c, blk);
            const void *src = r >= 0 ? (const void *)(cache.v + r * C::RB + piece * 16) : (const void *)&kZero16;
            dma16(src, base + blk * 1024);
        }
        return C::LK;
    };

    // ---- per-thread state ---------------------------------------------------
    const bool s_thread = tid < C::S_THREADS;
    const int s_r = tid / C::TPH;                     // head (padded group)
    const int s_j = tid % C::TPH;
    uint32_t qw[C::QW];
    float m_ref = -INFINITY, l_run = 0.f;

    const int v_cl = lane % C::CPW;                   // column piece within the wave
    const int v_rest = lane / C::CPW;
    const int v_hg = v_rest % C::HG;
    const int v_tg = v_rest / C::HG;
    const int v_c = wave * C::CPW + v_cl;             // column piece of the row
    float acc[C::HPT][C::CE];
#pragma unroll
    for (int i = 0; i < C::HPT; ++i)
#pragma unroll
        for (int e = 0; e < C::CE; ++e) acc[i][e] = 0.f;

    // ---- software pipeline ---------------------------------------------------
    // Iteration tau (one barrier each) computes the scores of tile tau and the
    // V sum of tile tau-1; they touch different halves of the double-buffered
    // P / alpha / (m, l) arrays.  Tile t lives in stage (t - tau0) % NBUF.
    // Its K (with q when it starts an item or the slice) is issued A = NBUF-1
    // iterations ahead and its V one iteration later, because the V sum of a
    // tile runs one iteration after its scores: A tiles are in flight while
    // only one stage's K and one stage's V are being read.
    // Virtual iteration i issues K(i + A) and V(i + A - 1); iterations
    // tau0 - A .. tau0 - 1 form the prologue.
    constexpr int A = C::A;
    Cursor kc = cursor_at(lds_prefix, lds_nvis, lds_first, p.rows, tau0, C::TT);   // next K to issue
    Cursor vc = kc;                                                     // next V to issue
    uint32_t hist = 0;   // loads of the last virtual iterations, 5 bits each (newest lowest)
    auto issue_iter = [&](int i) {
        int n = 0;
        const int tk = i + A, tv = i + A - 1;
        if (tk >= tau0 && tk < tau1) {
            n += issue_k(kc, kc.j == 0 || tk == tau0, (tk - tau0) % C::NBUF);
            cursor_next(lds_nvis, lds_first, p.rows, cache.K, kc, C::TT);
        }
        if (tv >= tau0 && tv < tau1) {
            n += issue_v(vc, (tv - tau0) % C::NBUF);
            cursor_next(lds_nvis, lds_first, p.rows, cache.K, vc, C::TT);
        }
        hist = (hist << 5) | (uint32_t)n;
    };
    for (int i = tau0 - A; i < tau0; ++i) issue_iter(i);
    Cursor cs = cursor_at(lds_prefix, lds_nvis, lds_first, p.rows, tau0, C::TT);   // tile of the score phase
    Cursor cv = cs;                                                    // tile of the V phase
    int piece0 = tau0;                                // first tile of the V phase's piece

    for (int tau = tau0; tau <= tau1; ++tau) {
        // K(tau) and V(tau-1) came from virtual iteration tau - A; the loads
        // of the A - 1 iterations after it may stay in flight.
        int after = 0;
#pragma unroll
        for (int k = 0; k < A - 1; ++k) after += (hist >> (5 * k)) & 31;
        wait_vm_dyn(after);
        barrier();
        issue_iter(tau);
        const bool do_s = tau < tau1;
        const bool do_v = tau > tau0;
        const int buf = tau & 1;                      // P / alpha / (m, l) half written by this S phase

        // ---- scores and online softmax of tile tau ----------------------------
        if (do_s) {
            const char *base = smem + ((tau - tau0) % C::NBUF) * C::STAGE;
            const uint4 *Ks = reinterpret_cast<const uint4 *>(base);
            const uint4 *Qs = reinterpret_cast<const uint4 *>(base + 2 * C::K_BYTES);
            const int nvalid = min(C::TT, cs.n_vis - (cs.jlo + cs.j) * C::TT);
            const int vfirst = cs.lo - (cs.jlo + cs.j) * C::TT;   // first key inside a sliding window
            const bool s_first = cs.j == 0 || tau == tau0;
            const bool s_last = cs.j == cs.tiles - 1 || tau == tau1 - 1;
            if (s_first) {
                if (s_thread) {
#pragma unroll
                    for (int w = 0; w < C::QW / 4; ++w) {
                        const uint4 x = Qs[s_r * C::CPR + w];
                        qw[4 * w + 0] = x.x; qw[4 * w + 1] = x.y; qw[4 * w + 2] = x.z; qw[4 * w + 3] = x.w;
                    }
                }
                m_ref = -INFINITY;
                l_run = 0.f;
            }
            if (s_thread) {
                float sc[C::NS];
                float mt = -INFINITY;
#pragma unroll
                for (int k = 0; k < C::NS; ++k) {
                    const int t = s_j + k * C::TPH;
                    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
                    for (int pcs = 0; pcs < C::CPR; ++pcs) {
                        const uint4 kv = Ks[t * C::CPR + (pcs ^ (t & C::SWZ))];
                        if constexpr (BF16) {
                            a0 = dot2_bf16(qw[4 * pcs + 0], kv.x, a0);
                            a1 = dot2_bf16(qw[4 * pcs + 1], kv.y, a1);
                            a2 = dot2_bf16(qw[4 * pcs + 2], kv.z, a2);
                            a3 = dot2_bf16(qw[4 * pcs + 3], kv.w, a3);
                        } else {
                            a0 = fmaf(__uint_as_float(qw[4 * pcs + 0]), __uint_as_float(kv.x), a0);
                            a1 = fmaf(__uint_as_float(qw[4 * pcs + 1]), __uint_as_float(kv.y), a1);
                            a2 = fmaf(__uint_as_float(qw[4 * pcs + 2]), __uint_as_float(kv.z), a2);
                            a3 = fmaf(__uint_as_float(qw[4 * pcs + 3]), __uint_as_float(kv.w), a3);
                        }
                    }
                    sc[k] = (t < nvalid && t >= vfirst) ? ((a0 + a1) + (a2 + a3)) * p.scale_log2 : -INFINITY;
                    mt = fmaxf(mt, sc[k]);
                }
                mt = group_max<C::TPH>(mt);
                float alpha = 1.f;
                if (mt > m_ref + TAU) {
                    alpha = fast_exp2(m_ref - mt);   // 0 on an item's first tile
                    m_ref = mt;
                }
                float ps = 0.f;
                char *pbuf = lds_p + buf * C::P_BYTES;
#pragma unroll
                for (int k = 0; k < C::NS; ++k) {
                    const int t = s_j + k * C::TPH;
                    const float pk = fast_exp2(sc[k] - m_ref);
                    if constexpr (BF16) {
                        const uint32_t pb = f32_to_bf16_rne(pk);
                        ps += __uint_as_float(pb << 16);   // the sum of what the V product uses
                        reinterpret_cast<uint16_t *>(pbuf)[((t >> 1) * GP + s_r) * 2 + (t & 1)] = (uint16_t)pb;
                    } else {
                        ps += pk;
                        reinterpret_cast<float *>(pbuf)[t * GP + s_r] = pk;
                    }
                }
                ps = group_sum<C::TPH>(ps);
                l_run = l_run * alpha + ps;
                if (s_j == 0) {
                    lds_alpha[buf][s_r] = alpha;
                    if (s_last) {
                        lds_m[buf][s_r] = m_ref;
                        lds_l[buf][s_r] = l_run;
                    }
                }
            }
        }

        // ---- o = o * alpha + sum_t p_t v_t of tile tau-1 ----------------------
        if (do_v) {
            const int tv = tau - 1;
            const int vb = buf ^ 1;
            const char *base = smem + ((tv - tau0) % C::NBUF) * C::STAGE;
            const uint4 *Vs = reinterpret_cast<const uint4 *>(base + C::K_BYTES);
            const bool v_first = cv.j == 0 || tv == tau0;
            const bool v_last = cv.j == cv.tiles - 1 || tv == tau1 - 1;
            if (v_first) {
#pragma unroll
                for (int i = 0; i < C::HPT; ++i)
#pragma unroll
                    for (int e = 0; e < C::CE; ++e) acc[i][e] = 0.f;
                piece0 = tv;
            }
            float al[C::HPT];
            bool any = false;
#pragma unroll
            for (int i = 0; i < C::HPT; ++i) {
                al[i] = lds_alpha[vb][v_hg * C::HPT + i];
                any |= (al[i] != 1.f);
            }
            if (any) {
#pragma unroll
                for (int i = 0; i < C::HPT; ++i)
#pragma unroll
                    for (int e = 0; e < C::CE; ++e) acc[i][e] *= al[i];
            }
            const char *pbuf = lds_p + vb * C::P_BYTES;
            if constexpr (BF16) {
                const uint32_t *P2 = reinterpret_cast<const uint32_t *>(pbuf);
#pragma unroll
                for (int kp = 0; kp < C::TPT / 2; ++kp) {
                    const int t = v_tg * C::TPT + 2 * kp;
                    const uint4 a = Vs[t * C::CPR + v_c];
                    const uint4 bb = Vs[(t + 1) * C::CPR + v_c];
                    uint32_t vv[8];
                    vv[0] = pair_lo(a.x, bb.x); vv[1] = pair_hi(a.x, bb.x);
                    vv[2] = pair_lo(a.y, bb.y); vv[3] = pair_hi(a.y, bb.y);
                    vv[4] = pair_lo(a.z, bb.z); vv[5] = pair_hi(a.z, bb.z);
                    vv[6] = pair_lo(a.w, bb.w); vv[7] = pair_hi(a.w, bb.w);
#pragma unroll
                    for (int i = 0; i < C::HPT; ++i) {
                        const uint32_t pp = P2[(t >> 1) * GP + v_hg * C::HPT + i];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[i][e] = dot2_bf16(pp, vv[e], acc[i][e]);
                    }
                }
            } else {
                const float *Pf = reinterpret_cast<const float *>(pbuf);
#pragma unroll
                for (int k = 0; k < C::TPT; ++k) {
                    const int t = v_tg * C::TPT + k;
                    const uint4 a = Vs[t * C::CPR + v_c];
                    const float vf[4] = {__uint_as_float(a.x), __uint_as_float(a.y),
                                         __uint_as_float(a.z), __uint_as_float(a.w)};
#pragma unroll
                    for (int i = 0; i < C::HPT; ++i) {
                        const float pk = Pf[t * GP + v_hg * C::HPT + i];
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(pk, vf[e], acc[i][e]);
                    }
                }
            }

            // ---- end of a piece: reduce the key groups and store --------------
            if (v_last) {
#pragma unroll
                for (int m = C::CPW * C::HG; m < kWave; m <<= 1)
#pragma unroll
                    for (int i = 0; i < C::HPT; ++i)
#pragma unroll
                        for (int e = 0; e < C::CE; ++e) acc[i][e] += __shfl_xor(acc[i][e], m, kWave);
                const bool whole = (piece0 == cv.item0) && (cv.j == cv.tiles - 1);
                const int64_t head0 = ((int64_t)p.row0 + cv.row) * H + (int64_t)cv.g * G;
                if (v_tg == 0) {
#pragma unroll
                    for (int i = 0; i < C::HPT; ++i) {
                        const int r = v_hg * C::HPT + i;
                        if (r >= G) continue;
                        const int col = v_c * C::CE;
                        if (whole) {
                            const float inv = 1.f / lds_l[vb][r];
                            const int64_t o = (head0 + r) * D + col;
                            if constexpr (BF16) {
                                uint4 w;
                                w.x = pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv);
                                w.y = pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv);
                                w.z = pack_bf16x2(acc[i][4] * inv, acc[i][5] * inv);
                                w.w = pack_bf16x2(acc[i][6] * inv, acc[i][7] * inv);
                                *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(p.out) + o) = w;
                            } else {
                                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.out) + o) =
                                    make_float4(acc[i][0] * inv, acc[i][1] * inv, acc[i][2] * inv, acc[i][3] * inv);
                            }
                        } else {
                            const int slot = (tau0 < cv.item0) ? 1 : 0;
                            float *dst = p.ws_o + (((int64_t)blockIdx.x * 2 + slot) * G + r) * D + col;
#pragma unroll
                            for (int e = 0; e < C::CE; e += 4)
                                *reinterpret_cast<float4 *>(dst + e) =
                                    make_float4(acc[i][e], acc[i][e + 1], acc[i][e + 2], acc[i][e + 3]);
                            if (v_c == 0) {
                                float *ml = p.ws_ml + (((int64_t)blockIdx.x * 2 + slot) * G + r) * 2;
                                ml[0] = lds_m[vb][r];
                                ml[1] = lds_l[vb][r];
                            }
                        }
                    }
                }
                // These stores share the vector-memory counter with the loads in
                // flight; they can only make the next waits longer, never shorter.
            }
            cursor_next(lds_nvis, lds_first, p.rows, cache.K, cv, C::TT);
        }
        if (do_s) cursor_next(lds_nvis, lds_first, p.rows, cache.K, cs, C::TT);
    }
}

// Merge of the pieces of one (row, KV group) item with their global max and
// sum: M = max_s m_s, L = sum_s l_s 2^(m_s - M), out = sum_s o_s 2^(m_s - M) / L
// (m in log2 units).  Items held by one workgroup were stored by it; rows
// without a visible key get zeros.  Block (g, row, z) handles heads
// z*kMergeHeads .. of the item; the workspace slots of its pieces follow
// from the tile table.
constexpr int kMergeHeads = 8;

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_pieces_kernel(RowAttnParams p, int tt, int W)
{
    const int g = blockIdx.x;
    const int row = blockIdx.y;                       // local row of this launch
    const int G = p.G;
    const int h0 = blockIdx.z * kMergeHeads;
    if (h0 >= G) return;
    const int nh = min(kMergeHeads, G - h0);
    const int64_t head0 = ((int64_t)p.row0 + row) * p.H + (int64_t)g * G + h0;
    const int n_vis = row_visible(p, (int64_t)p.row0 + row);
    if (n_vis <= 0) {
        for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
            const int64_t o = head0 * D + idx;
            if constexpr (BF16) reinterpret_cast<uint16_t *>(p.out)[o] = 0;
            else reinterpret_cast<float *>(p.out)[o] = 0.f;
        }
        return;
    }
    const int64_t T = p.prefix[p.rows];
    const int64_t tiles = item_tiles(row_first(p, (int64_t)p.row0 + row, n_vis), n_vis, tt);
    const int64_t a = p.prefix[row] + (int64_t)g * tiles, e = a + tiles - 1;
    const int64_t wa = slice_owner(a, T, W), wb = slice_owner(e, T, W);
    if (wa == wb) return;
    // the workspace slots of the pieces: with at least one tile per slice
    // (T >= W) they are the slices wa .. wb, the first in slot 1 when the
    // item starts inside it; otherwise every tile of the item is a piece of
    // its own, in slot 0 of its slice
    const bool dense = T >= W;
    const int ns = dense ? (int)(wb - wa + 1) : (int)(e - a + 1);
    const int slot0 = (int)(wa * 2 + (slice_start(wa, T, W) < a ? 1 : 0));
    auto slot_of = [&](int k) {
        return dense ? (k == 0 ? slot0 : (int)(wa + k) * 2) : (int)sparse_slot(a + k, T, W);
    };
    for (int idx = threadIdx.x; idx < nh * D / 4; idx += 256) {
        const int r = h0 + (4 * idx) / D, col = (4 * idx) % D;
        // pieces in batches whose loads are issued together; the running
        // maximum rescales what is summed so far (in slot order)
        constexpr int BATCH = 4;
        float M = -INFINITY, L = 0.f;
        float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k0 = 0; k0 < ns; k0 += BATCH) {
            float mm[BATCH], ll[BATCH];
            float4 oo[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                mm[j] = -INFINITY;
                ll[j] = 0.f;
                oo[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (k0 + j < ns) {
                    const int64_t sr = (int64_t)slot_of(k0 + j) * G + r;
                    mm[j] = p.ws_ml[sr * 2];
                    ll[j] = p.ws_ml[sr * 2 + 1];
                    oo[j] = *reinterpret_cast<const float4 *>(p.ws_o + sr * D + col);
                }
            }
            float Mn = M;
#pragma unroll
            for (int j = 0; j < BATCH; ++j) Mn = fmaxf(Mn, mm[j]);
            if (Mn == -INFINITY) continue;
            const float a_old = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
            L *= a_old;
            O.x *= a_old; O.y *= a_old; O.z *= a_old; O.w *= a_old;
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                if (mm[j] == -INFINITY) continue;
                const float wt = fast_exp2(mm[j] - Mn);
                L += ll[j] * wt;
                O.x += oo[j].x * wt;
                O.y += oo[j].y * wt;
                O.z += oo[j].z * wt;
                O.w += oo[j].w * wt;
            }
            M = Mn;
        }
        const float inv = 1.f / L;
        const int64_t o = (head0 - h0 + r) * D + col;
        if constexpr (BF16) {
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + o) =
                make_uint2(pack_bf16x2(O.x * inv, O.y * inv), pack_bf16x2(O.z * inv, O.w * inv));
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.out) + o) =
                make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
        }
    }
}

// Workgroups per launch: the caller's count (two per CU) when two fit in a
// CU's LDS, half of it when one workgroup needs more than half the LDS (a
// second wave of slices would only run after the first).
template <int D, int GP, bool BF16>
hipError_t launch_g(const RowAttnParams &p0, hipStream_t s)
{
    using C = Cfg<D, GP, BF16>;
    RowAttnParams p = p0;
    if (p.wgs_override > 0) p.num_wgs = p.wgs_override;
    else if (C::LIMIT > LDS_LIMIT && p.num_wgs > 1) p.num_wgs /= 2;
    hipLaunchKernelGGL((stream_attention_kernel<D, GP, BF16>), dim3(p.num_wgs), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.whole_items) return e;
    return launch_merge_pieces(p, C::TT, p.num_wgs, s);
}

template <int D, bool BF16>
hipError_t launch_d(const RowAttnParams &p, int gp, hipStream_t s)
{
    switch (gp) {
    case 1: return launch_g<D, 1, BF16>(p, s);
    case 2: return launch_g<D, 2, BF16>(p, s);
    case 4: return launch_g<D, 4, BF16>(p, s);
    case 8: return launch_g<D, 8, BF16>(p, s);
    case 16: return launch_g<D, 16, BF16>(p, s);
    case 32: return launch_g<D, 32, BF16>(p, s);
    case 64: return launch_g<D, 64, BF16>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_merge_pieces(const RowAttnParams &p, int tt, int W, hipStream_t s)
{
    const dim3 grid(p.cache.K, p.rows, (p.G + kMergeHeads - 1) / kMergeHeads);
    const bool bf16 = p.cache.elem_bytes != 4;   // a 1-byte (FP8 or INT8) cache has bf16 outputs
    if (p.cache.d == 128) {
        if (bf16) hipLaunchKernelGGL((merge_pieces_kernel<128, true>), grid, dim3(256), 0, s, p, tt, W);
        else hipLaunchKernelGGL((merge_pieces_kernel<128, false>), grid, dim3(256), 0, s, p, tt, W);
    } else if (p.cache.d == 64) {
        if (bf16) hipLaunchKernelGGL((merge_pieces_kernel<64, true>), grid, dim3(256), 0, s, p, tt, W);
        else hipLaunchKernelGGL((merge_pieces_kernel<64, false>), grid, dim3(256), 0, s, p, tt, W);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Rows are processed in launches of at most kStreamRows rows (the row tables
// live in LDS); launches on one stream run in order and share the workspace.
hipError_t launch_row_attention(const RowAttnParams &p0, int gp, hipStream_t stream)
{
    if (p0.total_rows <= 0) return hipSuccess;
    if (p0.cache.K > 65535 || p0.num_wgs <= 0 || p0.num_wgs > kStreamWGs) return hipErrorInvalidValue;
    const bool bf16 = p0.cache.elem_bytes == 2;
    for (int64_t r0 = 0; r0 < p0.total_rows; r0 += kStreamRows) {
        RowAttnParams p = p0;
        p.row0 = r0;
        p.rows = (int32_t)(p0.total_rows - r0 < kStreamRows ? p0.total_rows - r0 : kStreamRows);
        hipError_t e = hipErrorInvalidValue;
        // bf16 at d = 128 and 64 and 1-byte codes at d = 128: the matrix-core kernel,
        // whatever the group size; the rest (fp32, bf16 paged in blocks under
        // 16 tokens, more than 64 rows per KV head): this file's kernel
        if (decode_mfma_supported(p)) e = launch_decode_mfma(p, stream);
        else if (p.mq > 1) return hipErrorInvalidValue;   // several positions: the matrix-core kernel only
        else if (p.cache.elem_bytes == 1) return hipErrorInvalidValue;   // FP8 / INT8: the matrix-core kernel only
        else if (p.cache.d == 128) e = bf16 ? launch_d<128, true>(p, gp, stream) : launch_d<128, false>(p, gp, stream);
        else if (p.cache.d == 64) e = bf16 ? launch_d<64, true>(p, gp, stream) : launch_d<64, false>(p, gp, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gqa
