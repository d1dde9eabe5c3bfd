// prefill_mfma.hip -- causal (or full) grouped-query attention of a block of
// new query tokens on the CDNA4 matrix cores, bf16 in, fp32 accumulate.
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps 2-4):
// out[b,i,h] = softmax(q[b,i,h] K_g^T * scale) V_g, g = h / G, over the keys
// visible to row i: keys 0 .. start_pos[b]+i when causal (a token attends to
// itself and to every earlier token), keys 0 .. start_pos[b]+s-1 otherwise.
// The new tokens' K/V are already in the cache (the append kernel runs first
// on the same stream).
//
// How (designed for gfx950; FlashAttention on the inference-optimisation
// page §9 is prior art for the tiling idea only):
//  * A workgroup (8 waves, two per SIMD) owns 256 (position, head) rows of
//    one sequence and one KV group: 256/G consecutive positions x the G heads.
//    Every K/V tile it loads therefore serves all G heads of the group.  Each
//    wave owns one 32-row block.
//  * K/V tiles of 64 keys move HBM -> LDS with LDS-direct loads
//    (global_load_lds_dwordx4, no registers), four stages deep, with explicit
//    vmcnt waits; one barrier per tile.
//  * Scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16),
//    so a lane holds 32 scores of ONE query row: the row max is lane-local
//    plus one exchange with the lane 32 away, and the row sum is kept per
//    lane until the end.  Q^T stays in registers for the whole key loop.
//  * The accumulator layout of S^T, rounded to bf16 (hardware RNE), is the
//    B operand P^T of O^T += V^T P^T as it stands.  The matching V^T operand
//    is read straight from the row-major V tile with the gfx950 transposing
//    LDS read (ds_read_b64_tr_b16): sixteen lanes fetch four 4-key x
//    4-column pieces and each lane receives four consecutive keys of one
//    column.  K and V rows are XOR-swizzled in 16-byte chunks so that these
//    reads hit distinct banks.
//  * Online softmax in fp32 and exp2 units (inference-optimisation page
//    §9.2.1): scale folded into one FMA, the running max only moved when a
//    tile max exceeds it by 2^8 (checked with one wave vote), masking only on
//    the tiles that cross the causal diagonal or the end of the keys.
//  * The two waves of each SIMD run the tile loop half a phase apart (one
//    scores tile t while the other finishes tile t-1), so one wave's softmax
//    overlaps the other's matrix work; the K and V^T fragments are read from
//    LDS a few matrix instructions ahead of their use.
//  * Paged caches (a block table, blocks of 16 or more tokens): a 64-key tile
//    spans at most four blocks, whose ids come from one scalar load of four
//    table entries per tile; each 1 KB load's rows lie in one of them, so its
//    lanes take a wave-uniform base plus the same offsets as a contiguous
//    tile.  A separate instantiation, so the contiguous kernel is unchanged.
//  * Persistent workgroups, one per CU: the query blocks are taken heaviest
//    first (largest causal key range) in rounds of one block per workgroup,
//    the order reversed every other round so that each workgroup's blocks
//    sum to about the same work.  A workgroup goes from one block to the
//    next without the hand-over between workgroups (~2.5 us per block).
#include <type_traits>
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int BN = kKeyTile;       // keys per tile (64)
constexpr int ROWS = 256;          // (position, head) rows per workgroup
constexpr int NS = 5;              // LDS stages (160 KB)
constexpr float TAU = 8.0f;

__device__ const uint4 kZero16P = {0u, 0u, 0u, 0u};

__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One LDS-direct 16-byte load per lane (lane i's bytes land at base + 16 i),
// written as inline assembly so the compiler does not wait for it before LDS
// reads; the kernel waits with explicit vmcnt.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
#pragma clang diagnostic pop
}
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS accesses are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The transposing LDS read: 64 bits per lane, see the header comment.
__device__ __forceinline__ uint2 lds_read_tr16(const char *p)
{
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(lds_void_t *)p);
    return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

// NT_ = 512: 8 waves (two per SIMD), one 32-row block each.
template <int D, int GP, int NT_>
struct PCfg {
    static constexpr int NT = NT_;
    static constexpr int NW = NT / kWave;
    static constexpr int RPW = ROWS / NW;         // rows per wave
    static constexpr int RBW = RPW / 32;          // 32-row blocks per wave
    static constexpr int QB = ROWS / GP;          // positions per workgroup
    static constexpr int RB = D * 2;              // bytes per K/V row
    static constexpr int CPR = RB / 16;           // 16-byte chunks per row
    // 16-byte slot swizzles, chosen so that the LDS reads of the scores (16
    // lanes read 16 bytes of 16 consecutive keys) and of V^T (32 lanes read 8
    // bytes of 4 consecutive keys) spread over all 64 LDS banks: K row r keeps
    // chunk c in slot c ^ ksw(r), V row r in slot c ^ vsw(r).
    __device__ static constexpr int ksw(int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & (CPR - 1)); }
    __device__ static constexpr int vsw(int r) { return CPR >= 16 ? 4 * (r & 3) : 2 * (r & 3); }
    static constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    static constexpr int TILE = BN * RB;          // bytes of K (or V) per tile
    static constexpr int STAGE = 2 * TILE;        // K then V
    static constexpr int RPK = 1024 / RB;         // rows per 1 KB load
    static constexpr int LPW = TILE / 1024 / NW;  // 1 KB loads per wave per tile, each of K and V
    static constexpr int LOADS = 2 * LPW;         // loads per wave per tile
    static_assert(QB * GP == ROWS, "rows split into positions x heads");
    static_assert(LPW >= 1 && LPW * NW * 1024 == TILE, "tile load split");
    static_assert(NS * STAGE <= 160 * 1024, "LDS");
};

// PAGED: the cache goes through a block table (blocks of any size); else it
// is contiguous.  Two instantiations, so that the contiguous kernel carries
// none of the paged path's registers.
template <int D, int GP, int NT_, bool PAGED>
__global__ __launch_bounds__(NT_) void prefill_mfma_kernel(PrefillParams p)
{
    using C = PCfg<D, GP, NT_>;
    constexpr int NW = C::NW, RPW = C::RPW, RBW = C::RBW;
    __shared__ __attribute__((aligned(1024))) char smem[NS * C::STAGE];

    const CacheView &cache = p.cache;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nq = lane & 31, hh = lane >> 5;
    const int num_qb = (p.s + C::QB - 1) / C::QB;
    // Block order: the heaviest query blocks (longest causal key range) of
    // every (sequence, group) come first, and the K (x B) blocks of one query
    // position range follow each other.
    const int kb_pairs = p.cache.K * p.B;
    const int total_blocks = num_qb * kb_pairs;
    // block k*N + j of the heaviest-first order goes to workgroup j in even
    // rounds k and to workgroup N-1-j in odd ones (N = gridDim.x), so that
    // every workgroup's rounds sum to about the same number of tiles
    for (int kr = 0;; ++kr) {
        const int bid = kr * (int)gridDim.x + ((kr & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x);
        if (bid >= total_blocks) break;
        if (kr > 0) barrier();   // every wave is past the previous block's stages
        const int qb = num_qb - 1 - bid / kb_pairs;
        const int g = (bid % kb_pairs) % p.cache.K;
        const int b = (bid % kb_pairs) / p.cache.K;
        const int q0 = qb * C::QB;
        const int start = p.start_pos[b];
        const int G = p.G, H = p.H;
        const int kv_len = (int)min((int64_t)start + p.s, (int64_t)cache.capacity);
        const int kv_end = p.causal ? (int)min((int64_t)start + q0 + C::QB, (int64_t)kv_len) : kv_len;
        const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
        // keys at or past this one may be masked for some row of the workgroup
        const int mask_from = p.causal ? (int)min((int64_t)start + q0 + 1, (int64_t)kv_len) : kv_len;
        // Sliding window of W positions (inference-optimisation page §6.4.1): row
        // i sees keys from qpos + 1 - W on.  The workgroup's first row sets the
        // first tile; tiles below the last row's first key need the mask.
        const int win = p.window;
        const int kv_begin = win > 0 ? (int)min(max((int64_t)0, (int64_t)start + q0 + 1 - win), (int64_t)kv_len) : 0;
        const int t_first = kv_begin / BN;
        const int lo_last = win > 0 ? (int)min(max((int64_t)0, (int64_t)start + q0 + C::QB - win), (int64_t)kv_len) : 0;
        const int t_lo_end = (lo_last + BN - 1) / BN;   // tiles below this one need the window mask

        // ---- this lane's two query rows and their Q^T fragments -------------------
        int row_r[RBW], row_i[RBW], qpos[RBW], row_lo[RBW];
        bool row_ok[RBW];
        uint4 qf[RBW][C::KS];
    #pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const int rho = wave * RPW + rb * 32 + nq;
            row_r[rb] = rho % GP;
            row_i[rb] = q0 + rho / GP;
            row_ok[rb] = row_r[rb] < G && row_i[rb] < p.s;
            qpos[rb] = start + row_i[rb];
            row_lo[rb] = win > 0 ? max(0, qpos[rb] + 1 - win) : 0;
            const uint4 *qrow = reinterpret_cast<const uint4 *>(
                p.q + ((((int64_t)b * p.s + (row_ok[rb] ? row_i[rb] : 0)) * H + (int64_t)g * G +
                        (row_ok[rb] ? row_r[rb] : 0)) * D) * 2);
    #pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                qf[rb][ks] = row_ok[rb] ? qrow[2 * ks + hh] : make_uint4(0, 0, 0, 0);
        }

        // ---- LDS-direct loads of tile t into stage t % NS --------------------------
        // K: row r's 16-byte chunk c lands in slot c ^ ksw(r); V: slot c ^ vsw(r).
        // Lane offsets of the full-tile path (contiguous cache): tile row r_k of
        // this lane's k-th load and its swizzled 16-byte slot, for K and for V.
        uint32_t koff[C::LPW], voff[C::LPW];
    #pragma unroll
        for (int k = 0; k < C::LPW; ++k) {
            const int r = (wave + NW * k) * C::RPK + lane / C::CPR;
            const int slot = lane % C::CPR;
            koff[k] = (uint32_t)(r * C::RB + (slot ^ C::ksw(r)) * 16);
            voff[k] = (uint32_t)(r * C::RB + (slot ^ C::vsw(r)) * 16);
        }
        const bool contiguous = !PAGED && cache.block_table == nullptr;
        const bool small_blocks = !contiguous && cache.log2_bs < 4;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;   // LDS address of the stages
        const char *kseq = cache.k + ((int64_t)b * cache.K + g) * cache.S_max * C::RB;
        const char *vseq = cache.v + ((int64_t)b * cache.K + g) * cache.S_max * C::RB;
        // Lane source pointers of tile t's loads (K then V for each of this
        // wave's 1 KB blocks); rows outside the keys, and tiles past the last,
        // read a zero constant.
        auto plan = [&](int t, const char *(&src)[2 * C::LPW]) __attribute__((always_inline)) {
            const int j0 = t * BN;
            if (t < ntiles && contiguous && j0 >= kv_begin && j0 + BN <= kv_len) {
                // every row of the tile is in the cache: a uniform base and lane offsets
    #pragma unroll
                for (int k = 0; k < C::LPW; ++k) {
                    src[2 * k] = kseq + (int64_t)j0 * C::RB + koff[k];
                    src[2 * k + 1] = vseq + (int64_t)j0 * C::RB + voff[k];
                }
                return;
            }
            if constexpr (PAGED) {
                // paged, blocks of 16 or more, every row of the tile visible: each
                // load's rows lie in one 16-key group, whose block comes from one
                // table read per tile; uniform bases and the same lane offsets
                int id[4];
                if (t < ntiles && !small_blocks && j0 >= kv_begin && j0 + BN <= kv_len &&
                    tile_block_ids(cache, b, j0, id)) {
                    bool ok = true;
                    int64_t row[C::LPW];
    #pragma unroll
                    for (int k = 0; k < C::LPW; ++k) {
                        const int r0 = (wave + NW * k) * C::RPK;   // the load's first tile row
                        const int blk_id = id[r0 / 16];
                        ok = ok && blk_id >= 0 && blk_id < cache.num_blocks;
                        row[k] = (((int64_t)blk_id * cache.K + g) << cache.log2_bs) +
                                 ((j0 + r0) & ((1 << cache.log2_bs) - 1));
                    }
                    if (ok) {
    #pragma unroll
                        for (int k = 0; k < C::LPW; ++k) {
                            const uint32_t rel = (uint32_t)((wave + NW * k) * C::RPK * C::RB);
                            src[2 * k] = cache.k + row[k] * C::RB + (koff[k] - rel);
                            src[2 * k + 1] = cache.v + row[k] * C::RB + (voff[k] - rel);
                        }
                        return;
                    }
                }
            }
    #pragma unroll
            for (int k = 0; k < C::LPW; ++k) {
                const int blk = wave + NW * k;                // 1 KB block of the tile
                const int r = blk * C::RPK + lane / C::CPR;   // tile row of this lane
                const int slot = lane % C::CPR;
                const char *srck = reinterpret_cast<const char *>(&kZero16P), *srcv = srck;
                // rows below kv_begin are outside every row's window: not read
                if (t < ntiles && j0 + blk * C::RPK < kv_len && j0 + blk * C::RPK + C::RPK > kv_begin) {
                    int64_t row = -1;
                    if (small_blocks) {
                        // blocks of fewer than 16 tokens: the load's RPK rows may
                        // span several cache blocks, so each lane looks up its own
                        if (j0 + r < kv_len && j0 + r >= kv_begin) row = cache_row(cache, b, g, j0 + r);
                    } else {
                        // the load's rows lie in one 16-row group, hence in one cache block
                        const int64_t row0 = cache_row_wave(cache, b, g, j0 + blk * C::RPK);
                        if (row0 >= 0 && j0 + r < kv_len && j0 + r >= kv_begin) row = row0 + (r - blk * C::RPK);
                    }
                    if (row >= 0) {
                        srck = cache.k + row * C::RB + (slot ^ C::ksw(r)) * 16;
                        srcv = cache.v + row * C::RB + (slot ^ C::vsw(r)) * 16;
                    }
                }
                src[2 * k] = srck;
                src[2 * k + 1] = srcv;
            }
        };
        // LDS address of load i (K or V of block k = i / 2) of tile t
        auto lds_at = [&](int t, int i) __attribute__((always_inline)) {
            return lds0 + (uint32_t)((t % NS) * C::STAGE + (i & 1) * C::TILE + (wave + NW * (i / 2)) * 1024);
        };
        auto issue = [&](int t) __attribute__((always_inline)) {
            const char *src[2 * C::LPW];
            plan(t, src);
    #pragma unroll
            for (int i = 0; i < 2 * C::LPW; ++i) dma16(src[i], lds_at(t, i));
        };
        // wait until tile t's loads have landed, given how many tiles were issued after it
        auto wait_tile = [&](int after) __attribute__((always_inline)) {
            if (after <= 0) wait_vm<0>();
            else if (after == 1) wait_vm<C::LOADS>();
            else wait_vm<2 * C::LOADS>();
        };

        // ---- per-lane softmax state and accumulators --------------------------------
        float m_ref[RBW], l_run[RBW];
        f32x16_t acc[RBW][C::DB];
    #pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            m_ref[rb] = -INFINITY;
            l_run[rb] = 0.f;
    #pragma unroll
            for (int db = 0; db < C::DB; ++db)
    #pragma unroll
                for (int i = 0; i < 16; ++i) acc[rb][db][i] = 0.f;
        }

        // S^T of tile t for both row blocks
        // S^T of tile t.  The K fragments are read KPF steps ahead of their
        // matrix instruction so that LDS latency overlaps the matrix pipeline.
        constexpr int SSTEPS = C::KS * 2;   // (k-step, 32-key block) pairs
        constexpr int KPF = 4;
        auto k_frag = [&](const char *kt, int st) __attribute__((always_inline)) {
            const int ks = st / 2, kb = st % 2;
            const int key = kb * 32 + nq;
            return *reinterpret_cast<const uint4 *>(kt + key * C::RB + (((2 * ks + hh) ^ C::ksw(key)) * 16));
        };
        auto scores = [&](int t, f32x16_t (&s)[RBW][2]) __attribute__((always_inline)) {
            const char *kt = smem + (t % NS) * C::STAGE;
            uint4 kf[KPF];
    #pragma unroll
            for (int st = 0; st < KPF; ++st) kf[st] = k_frag(kt, st);
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                    for (int i = 0; i < 16; ++i) s[rb][kb][i] = 0.f;
    #pragma unroll
            for (int st = 0; st < SSTEPS; ++st) {
                const uint4 a = kf[st % KPF];
                if (st + KPF < SSTEPS) kf[st % KPF] = k_frag(kt, st + KPF);
                const int ks = st / 2, kb = st % 2;
    #pragma unroll
                for (int rb = 0; rb < RBW; ++rb) s[rb][kb] = mfma32x32x16(a, qf[rb][ks], s[rb][kb]);
            }
        };

        // Softmax of tile t in three parts: the tile maximum (with the causal
        // mask on the tiles that need it) and the vote on a rescale; the rare
        // rescale of the accumulators; the bf16 probabilities P^T and their sum.
        auto tile_max = [&](int t, f32x16_t (&s)[RBW][2], bool masked, float (&mt)[RBW]) __attribute__((always_inline)) {
            const int j0 = t * BN;
            bool need = false;
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                if (masked) {
                    const int lim = p.causal ? min(qpos[rb] + 1, kv_len) : kv_len;
    #pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = j0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                            if (key >= lim || key < row_lo[rb]) s[rb][kb][i] = -INFINITY;
                        }
                }
                float m = -INFINITY;
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                    for (int i = 0; i < 16; ++i) m = fmaxf(m, s[rb][kb][i]);
                m = max_xor32(m);
                mt[rb] = m * p.scale_log2;   // scale > 0, so the max commutes with it
                need |= mt[rb] > m_ref[rb] + TAU;
            }
            return __ballot(need) != 0;
        };
        auto rescale = [&](const float (&mt)[RBW]) __attribute__((always_inline)) {
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                if (mt[rb] > m_ref[rb] + TAU) {
                    const float alpha = fast_exp2(m_ref[rb] - mt[rb]);   // 0 on the first tile
                    m_ref[rb] = mt[rb];
                    l_run[rb] *= alpha;
    #pragma unroll
                    for (int db = 0; db < C::DB; ++db)
    #pragma unroll
                        for (int i = 0; i < 16; ++i) acc[rb][db][i] *= alpha;
                }
            }
        };
        auto probs = [&](const f32x16_t (&s)[RBW][2], uint4 (&pb)[RBW][2][2]) __attribute__((always_inline)) {
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                const float mu = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
                float ps = 0.f;
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        uint32_t w[4];
    #pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float p0 = fast_exp2(fmaf(s[rb][kb][half * 8 + 2 * j], p.scale_log2, -mu));
                            const float p1 = fast_exp2(fmaf(s[rb][kb][half * 8 + 2 * j + 1], p.scale_log2, -mu));
                            w[j] = cvt_pk_bf16(p0, p1);
                            ps = dot2_bf16(w[j], 0x3F803F80u, ps);   // + both rounded probabilities
                        }
                        pb[rb][kb][half] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                l_run[rb] += ps;
            }
        };

        // O^T += V^T P^T for tile t: the V^T operand of (key step, 32 columns) via
        // two transposing reads (keys +0..3 and +8..11 of this lane's 16-key step)
        const int tr_g = lane >> 4, tr_j = lane & 15;
        constexpr int PSTEPS = C::DB * 4;   // (32-column block, 16-key step) pairs
        constexpr int VPF = 2;
        // step st: key step st / DB (kb, half), column block st % DB, so that the
        // first matrix instructions need only the first probabilities
        auto v_frag = [&](const char *vt, int st) __attribute__((always_inline)) {
            const int db = st % C::DB, kb = st / C::DB / 2, half = (st / C::DB) % 2;
            uint2 part[2];
    #pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int row = kb * 32 + half * 16 + 4 * (tr_g >> 1) + 8 * rd + (tr_j >> 2);
                const int col = db * 32 + 16 * (tr_g & 1) + 4 * (tr_j & 3);
                const int chunk = (col >> 3) ^ C::vsw(row);
                part[rd] = lds_read_tr16(vt + row * C::RB + chunk * 16 + (col & 7) * 2);
            }
            return make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
        };
        auto pv = [&](int t, const uint4 (&pb)[RBW][2][2]) __attribute__((always_inline)) {
            const char *vt = smem + (t % NS) * C::STAGE + C::TILE;
            uint4 vf[VPF];
    #pragma unroll
            for (int st = 0; st < VPF; ++st) vf[st] = v_frag(vt, st);
    #pragma unroll
            for (int st = 0; st < PSTEPS; ++st) {
                const uint4 a = vf[st % VPF];
                if (st + VPF < PSTEPS) vf[st % VPF] = v_frag(vt, st + VPF);
                const int db = st % C::DB, kb = st / C::DB / 2, half = (st / C::DB) % 2;
    #pragma unroll
                for (int rb = 0; rb < RBW; ++rb) acc[rb][db] = mfma32x32x16(a, pb[rb][kb][half], acc[rb][db]);
            }
        };

        // ---- the pipeline -----------------------------------------------------------
        // Iteration t: wait for tile t+1, barrier (every wave is past iteration
        // t-1, so the stage of tile t-1 is free), start tile t+NS-1 into it.
        // Then, in one wave: the scores of tile t+1 on the matrix cores while the
        // vector units take the maximum of tile t; the rare rescale; the V product
        // of tile t on the matrix cores while the vector units form the
        // probabilities of tile t.  The instruction groups are interleaved
        // explicitly (one matrix instruction, then a few LDS reads and vector
        // instructions) so that one wave keeps both units busy.
        // Tiles start PD iterations ahead.  The barrier is taken every second
        // iteration, so the stage a load fills must have been free since the
        // barrier before the previous iteration: PD = NS - 2.
        constexpr int PD = NS - 2;
        for (int t = t_first; t < t_first + PD && t < ntiles; ++t) issue(t);
        if (ntiles > t_first) {
            wait_vm<0>();
            barrier();
        }
        // tiles in [t_lo_end, t_mask) need no mask; the steady loop runs over
        // them while a next tile exists
        const int t_mask = min(ntiles, mask_from / BN);
        const int t_steady = min(t_mask, ntiles - 1);
        f32x16_t sA[RBW][2], sB[RBW][2];
        uint4 pbuf[RBW][2][2];
        if (ntiles > t_first) scores(t_first, sA);
        // One probability pair of tile t: k-step ksp (keys kb*32 + half*16 ..),
        // pair j of its four, into pw and the running sum.
        auto prob_pair = [&](int rb, const f32x16_t (&s)[RBW][2], float mu, int ksp, int j, uint32_t (&pw)[RBW][4][4],
                             float &ps) __attribute__((always_inline)) {
            const int kb = ksp / 2, half = ksp % 2;
            const float p0 = fast_exp2(fmaf(s[rb][kb][half * 8 + 2 * j], p.scale_log2, -mu));
            const float p1 = fast_exp2(fmaf(s[rb][kb][half * 8 + 2 * j + 1], p.scale_log2, -mu));
            pw[rb][ksp][j] = cvt_pk_bf16(p0, p1);
            ps = dot2_bf16(pw[rb][ksp][j], 0x3F803F80u, ps);   // + both rounded probabilities
        };
        // The steady iteration, written as a sequence of small groups fenced from
        // each other: each group holds one matrix instruction, the LDS reads a
        // few matrix instructions ahead, and a share of the softmax of tile t.
        // bar: iteration t takes the barrier (every second one); before it, the
        // tiles t+1 and t+2 (the latest issued) must have landed.
        auto steady = [&](int t, f32x16_t (&sc)[RBW][2], f32x16_t (&sn)[RBW][2], bool bar) __attribute__((always_inline)) {
            if (bar) {
                wait_vm<0>();
                barrier();
            }
            // tile t+PD goes into the stage of tile t-2 (free since the last
            // barrier); its loads are spread over the score steps (issued
            // together, they would stall the wave on the full memory queue)
            const int tn = t + PD;
            const char *src[2 * C::LPW];
            plan(tn, src);
            __builtin_amdgcn_sched_barrier(0);
            // -- S(t+1) = K(t+1) Q^T, with the maximum of S(t) alongside
            const char *kt = smem + ((t + 1) % NS) * C::STAGE;
            uint4 kf[KPF];
    #pragma unroll
            for (int st = 0; st < KPF; ++st) kf[st] = k_frag(kt, st);
            float m[RBW];
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                m[rb] = -INFINITY;
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb)
    #pragma unroll
                    for (int i = 0; i < 16; ++i) sn[rb][kb][i] = 0.f;
            }
    #pragma unroll
            for (int st = 0; st < SSTEPS; ++st) {
                const uint4 a = kf[st % KPF];
                if (st + KPF < SSTEPS) kf[st % KPF] = k_frag(kt, st + KPF);
                const int ks = st / 2, kb = st % 2;
    #pragma unroll
                for (int rb = 0; rb < RBW; ++rb) sn[rb][kb] = mfma32x32x16(a, qf[rb][ks], sn[rb][kb]);
                // 32 scores per lane over 16 steps: two per step
                const int e = 2 * st;
    #pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
                    m[rb] = fmaxf(fmaxf(m[rb], sc[rb][e / 16][e % 16]), sc[rb][e / 16][e % 16 + 1]);
                constexpr int EVERY = SSTEPS / (2 * C::LPW);
                if (st % EVERY == EVERY / 2) dma16(src[st / EVERY], lds_at(tn, st / EVERY));
                __builtin_amdgcn_sched_barrier(0);
            }
            float mt[RBW];
            bool need = false;
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                mt[rb] = max_xor32(m[rb]) * p.scale_log2;   // scale > 0, so the max commutes with it
                need |= mt[rb] > m_ref[rb] + TAU;
            }
            if (__builtin_expect(__ballot(need) != 0, 0)) {
                // rare: kept as a branch (the empty volatile asm stops the compiler
                // from flattening it into multiplies on every tile)
                asm volatile("" ::: "memory");
                rescale(mt);
            }
            // -- O^T += V^T(t) P^T(t), forming the probabilities one k-step ahead
            const char *vt = smem + (t % NS) * C::STAGE + C::TILE;
            uint4 vf[VPF];
    #pragma unroll
            for (int st = 0; st < VPF; ++st) vf[st] = v_frag(vt, st);
            uint32_t pw[RBW][4][4];
            float mu[RBW], ps[RBW][2];   // two partial row sums: shorter dependency chains
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                mu[rb] = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
                ps[rb][0] = 0.f;
                ps[rb][1] = 0.f;
    #pragma unroll
                for (int j = 0; j < 4; ++j) prob_pair(rb, sc, mu[rb], 0, j, pw, ps[rb][j & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
            constexpr int PPS = 4 / C::DB;   // probability pairs per matrix instruction
    #pragma unroll
            for (int st = 0; st < PSTEPS; ++st) {
                const uint4 a = vf[st % VPF];
                if (st + VPF < PSTEPS) vf[st % VPF] = v_frag(vt, st + VPF);
                const int db = st % C::DB, ksp = st / C::DB;
    #pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
                    acc[rb][db] = mfma32x32x16(a, make_uint4(pw[rb][ksp][0], pw[rb][ksp][1], pw[rb][ksp][2], pw[rb][ksp][3]),
                                               acc[rb][db]);
                if (ksp + 1 < 4) {
    #pragma unroll
                    for (int rb = 0; rb < RBW; ++rb)
    #pragma unroll
                        for (int q = 0; q < PPS; ++q)
                            prob_pair(rb, sc, mu[rb], ksp + 1, db * PPS + q, pw, ps[rb][(db * PPS + q) & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) l_run[rb] += ps[rb][0] + ps[rb][1];
        };
        // One iteration with a barrier of its own and the mask where the tile
        // needs it: the tiles below the window's edge, the tiles at the causal
        // diagonal or the end of the keys, and the last tile.
        auto general = [&](int t) __attribute__((always_inline)) {
            const bool has_next = t + 1 < ntiles;
            wait_vm<0>();
            barrier();
            if (t + PD < ntiles) issue(t + PD);
            if (has_next) scores(t + 1, sB);
            float mt[RBW];
            if (tile_max(t, sA, t >= t_mask || t < t_lo_end, mt)) rescale(mt);
            probs(sA, pbuf);
            pv(t, pbuf);
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) { sA[rb][0] = sB[rb][0]; sA[rb][1] = sB[rb][1]; }
        };
        int t = t_first;
        for (; t < t_lo_end && t < ntiles; ++t) general(t);
        for (; t + 1 < t_steady; t += 2) {
            steady(t, sA, sB, true);
            steady(t + 1, sB, sA, false);
        }
        if (t < t_steady) {
            steady(t, sA, sB, true);
            ++t;
    #pragma unroll
            for (int rb = 0; rb < RBW; ++rb) { sA[rb][0] = sB[rb][0]; sA[rb][1] = sB[rb][1]; }
        }
        // the rest: tiles that need the mask, and the last tile
        for (; t < ntiles; ++t) general(t);

        // ---- normalise and store: lane owns 16 columns per 32-column block ----------
    #pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const float l = sum_xor32(l_run[rb]);
            if (!row_ok[rb]) continue;
            const float inv = l > 0.f ? 1.f / l : 0.f;
            uint16_t *orow = reinterpret_cast<uint16_t *>(p.out) +
                             (((int64_t)b * p.s + row_i[rb]) * H + (int64_t)g * G + row_r[rb]) * D;
    #pragma unroll
            for (int db = 0; db < C::DB; ++db)
    #pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int d0 = db * 32 + i4 * 8 + hh * 4;
                    const uint2 v = make_uint2(cvt_pk_bf16(acc[rb][db][4 * i4 + 0] * inv, acc[rb][db][4 * i4 + 1] * inv),
                                               cvt_pk_bf16(acc[rb][db][4 * i4 + 2] * inv, acc[rb][db][4 * i4 + 3] * inv));
                    *reinterpret_cast<uint2 *>(orow + d0) = v;
                }
        }
    }
}

// Compute units of the current device (looked up once per device).
int compute_units()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int D, int GP, int NT_>
hipError_t launch_gp(const PrefillParams &p, dim3 grid, hipStream_t s)
{
    if (p.cache.block_table != nullptr)
        hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, NT_, true>), grid, dim3(NT_), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, NT_, false>), grid, dim3(NT_), 0, s, p);
    return hipGetLastError();
}

template <int D, int NT_>
hipError_t launch_d(const PrefillParams &p, int gp, hipStream_t s)
{
    const int64_t qb_pos = ROWS / gp;
    const int64_t nqb = (p.s + qb_pos - 1) / qb_pos;
    if (nqb * p.cache.K * p.B > 0x7fffffffLL) return hipErrorInvalidValue;
    // one persistent workgroup per compute unit (one fits, by its LDS)
    const dim3 grid((unsigned)std::min<int64_t>(nqb * p.cache.K * p.B, compute_units()));
    switch (gp) {
    case 1: return launch_gp<D, 1, NT_>(p, grid, s);
    case 2: return launch_gp<D, 2, NT_>(p, grid, s);
    case 4: return launch_gp<D, 4, NT_>(p, grid, s);
    case 8: return launch_gp<D, 8, NT_>(p, grid, s);
    case 16: return launch_gp<D, 16, NT_>(p, grid, s);
    case 32: return launch_gp<D, 32, NT_>(p, grid, s);
    case 64: return launch_gp<D, 64, NT_>(p, grid, s);
    default: return hipErrorInvalidValue;
    }
}

constexpr int kPrefillThreads = 512;   // workgroup shape of the prefill kernel

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams &p, hipStream_t stream)
{
    const int gp = pow2_at_least(p.G);
    if (p.cache.elem_bytes != 2) return hipErrorInvalidValue;
    if (p.cache.d == 128) return launch_d<128, kPrefillThreads>(p, gp, stream);
    if (p.cache.d == 64) return launch_d<64, kPrefillThreads>(p, gp, stream);
    return hipErrorInvalidValue;
}

}  // namespace gqa
