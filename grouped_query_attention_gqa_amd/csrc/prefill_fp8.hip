// prefill_fp8.hip -- causal (or full) grouped-query attention of a block of
// new query tokens over an FP8 E4M3 (or INT8) KV cache with one fp32 scale
// per cached row, on the CDNA4 matrix cores (bf16 products, fp32
// accumulation).
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps 2-4,
// over the quantised cache of the inference-optimisation page §15.5.1):
// out[b,i,h] = softmax(q[b,i,h] K_g^T * scale) V_g, g = h / G, where cached
// row j of K (and V) stands for k_scale[j] * E4M3(code_j) (k_scale[j] * code_j
// for INT8).  The new tokens
// were quantised into the cache by the append kernel first, so the prefix and
// the new rows are read the same way; the visible keys are those of the bf16
// prefill (causal from start_pos, optional sliding window).
//
// How (the bf16 prefill's tiling, with one conversion step per tile):
//  * A workgroup of 8 waves owns 256 (position, head) rows of one sequence
//    and one KV group; each wave one 32-row block.  Tiles of 64 keys.
//  * The 1-byte rows and the tile's 64 K and 64 V scales move HBM -> LDS by
//    LDS-direct loads, NS stages deep (16.5 KB per stage, half the bytes of a
//    bf16 stage).
//  * Once a tile's codes have landed, the workgroup converts them into a bf16
//    tile (every E4M3 value and every integer of magnitude <= 127 is a bf16
//    value, so the conversion is exact),
//    laid out and swizzled as the bf16 prefill's stages, together with a copy
//    of the scales.  Two such tiles alternate: tile t + 1 is converted while
//    the matrix cores work on tile t, with one barrier per tile.
//  * Scores S^T = K Q^T on the codes; each key's score is multiplied by its
//    K scale before the softmax.  The probabilities are rounded to bf16 and
//    summed for the row sum, and each key's V scale multiplies its
//    probability before the bf16 rounding of the V product's operand, so the
//    V product runs on the codes (the decode kernel's rule).
//  * Online softmax in exp2 units with the lazy maximum (threshold 2^8), the
//    causal / window mask on the tiles that need it.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int D = 128;            // head dim (the FP8 cache is offered at d = 128)
constexpr int BN = kKeyTile;      // keys per tile (64)
constexpr int ROWS = 256;         // (position, head) rows per workgroup
constexpr int NT = 512;           // 8 waves
constexpr int NW = NT / kWave;
constexpr int RB = D * 2;         // bytes per bf16 row
constexpr int CB = D;             // bytes per code row
constexpr int CPR = RB / 16;      // 16-byte chunks per bf16 row
constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
constexpr int DB = D / 32;        // 32-row blocks of O^T
constexpr int NS = 4;             // code stages
constexpr float TAU = 8.0f;
// code stage: K codes, V codes, 64 K scales, 64 V scales
constexpr int ST_CODES = BN * CB;                 // 8 KB
constexpr int ST_KSC = 2 * ST_CODES;
constexpr int ST_VSC = ST_KSC + BN * 4;
constexpr int STAGE = ST_VSC + BN * 4;            // 16.5 KB
// converted tile: K and V as bf16 (swizzled as the bf16 prefill's stages) and the scales
constexpr int CT_V = BN * RB;
constexpr int CT_KSC = 2 * BN * RB;
constexpr int CT_VSC = CT_KSC + BN * 4;
constexpr int CTILE = CT_VSC + BN * 4;            // 32.5 KB
constexpr int JUNK = 256;                         // target of the waves' unused scale loads
constexpr int LDS_BYTES = NS * STAGE + 2 * CTILE + JUNK;
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
constexpr int LOADS = 3;          // LDS-direct loads per wave per tile: K codes, V codes, scales

__device__ const uint4 kZero16F = {0u, 0u, 0u, 0u};

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
// LDS-direct loads (lane i's bytes land at lds + 16 i, or lds + 4 i), as inline
// assembly so that the compiler does not wait for them before LDS reads; the
// kernel waits with explicit vmcnt.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void dma4(const void *src, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
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
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint2 lds_read_tr16(const char *p)
{
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(lds_void_t *)p);
    return __builtin_bit_cast(uint2, v);
}
// bf16 tile swizzles (those of the bf16 prefill at d = 128): K row r keeps its
// 16-byte chunk c in slot c ^ (r & 15), V row r in slot c ^ 4 (r & 3)
__device__ __forceinline__ constexpr int ksw(int r) { return r & 15; }
__device__ __forceinline__ constexpr int vsw(int r) { return 4 * (r & 3); }
// eight E4M3 codes -> eight bf16 values, exactly
template <bool HI>
__device__ __forceinline__ uint32_t f8x2_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// eight 1-byte codes -> eight bf16 values, exactly: E4M3 codes, or INT8
// codes with I8
template <bool I8>
__device__ __forceinline__ uint4 c8x8_bf16x8(uint32_t lo, uint32_t hi)
{
    if constexpr (I8) {
        const uint2 a = i8x4_bf16x4(lo), b = i8x4_bf16x4(hi);
        return make_uint4(a.x, a.y, b.x, b.y);
    }
    return make_uint4(f8x2_bf16x2<false>(lo), f8x2_bf16x2<true>(lo), f8x2_bf16x2<false>(hi), f8x2_bf16x2<true>(hi));
}

template <int GP, bool I8>
__global__ __launch_bounds__(NT) void prefill_fp8_kernel(PrefillParams p)
{
    constexpr int RPW = ROWS / NW;        // 32 rows per wave
    constexpr int QB = ROWS / GP;         // positions per workgroup
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    const CacheView &cache = p.cache;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nq = lane & 31, hh = lane >> 5;
    const int num_qb = (p.s + QB - 1) / QB;
    // heaviest query blocks first (as in the bf16 prefill)
    const int kb_pairs = cache.K * p.B;
    const int qb = num_qb - 1 - (int)(blockIdx.x / kb_pairs);
    const int g = (int)(blockIdx.x % kb_pairs) % cache.K;
    const int b = (int)(blockIdx.x % kb_pairs) / cache.K;
    const int q0 = qb * QB;
    const int start = p.start_pos[b];
    const int G = p.G, H = p.H;
    const int kv_len = (int)min((int64_t)start + p.s, (int64_t)cache.capacity);
    const int kv_end = p.causal ? (int)min((int64_t)start + q0 + QB, (int64_t)kv_len) : kv_len;
    const int ntiles = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    const int mask_from = p.causal ? (int)min((int64_t)start + q0 + 1, (int64_t)kv_len) : kv_len;
    const int win = p.window;
    const int kv_begin = win > 0 ? (int)min(max((int64_t)0, (int64_t)start + q0 + 1 - win), (int64_t)kv_len) : 0;
    const int t_first = kv_begin / BN;
    const int lo_last = win > 0 ? (int)min(max((int64_t)0, (int64_t)start + q0 + QB - win), (int64_t)kv_len) : 0;
    const int t_lo_end = (lo_last + BN - 1) / BN;
    const int t_mask = min(ntiles, mask_from / BN);

    // ---- this lane's query row and its Q^T fragments ----------------------------
    const int rho = wave * RPW + nq;
    const int row_r = rho % GP, row_i = q0 + rho / GP;
    const bool row_ok = row_r < G && row_i < p.s;
    const int qpos = start + row_i;
    const int row_lo = win > 0 ? max(0, qpos + 1 - win) : 0;
    uint4 qf[KS];
    {
        const uint4 *qrow = reinterpret_cast<const uint4 *>(
            p.q + ((((int64_t)b * p.s + (row_ok ? row_i : 0)) * H + (int64_t)g * G + (row_ok ? row_r : 0)) * D) * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = row_ok ? qrow[2 * ks + hh] : make_uint4(0, 0, 0, 0);
    }

    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    const bool small_blocks = cache.block_table != nullptr && cache.log2_bs < 4;
    // ---- LDS-direct loads of tile t's codes and scales into stage t % NS --------
    // Wave w loads code rows 8w .. 8w + 7 of K and of V (lane: row 8w + lane / 8,
    // 16-byte chunk lane % 8, unswizzled); wave 0 loads the 64 K scales and
    // wave 1 the 64 V scales (one per lane), the other waves a zero word into
    // the junk area, so that every wave issues LOADS loads per tile.  Rows
    // outside [kv_begin, kv_len), and tiles past the last, read zeros.
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int j0 = t * BN;
        const uint32_t st = lds0 + (uint32_t)((t % NS) * STAGE);
        const int r = 8 * wave + lane / 8, chunk = lane % 8;
        const char *srck = reinterpret_cast<const char *>(&kZero16F), *srcv = srck;
        if (t < ntiles && j0 + 8 * wave < kv_len && j0 + 8 * wave + 8 > kv_begin) {
            int64_t row = -1;
            if (small_blocks) {
                if (j0 + r < kv_len && j0 + r >= kv_begin) row = cache_row(cache, b, g, j0 + r);
            } else {
                // the 8 rows lie in one 16-row group, hence in one cache block
                const int64_t row0 = cache_row_wave(cache, b, g, j0 + 8 * wave);
                if (row0 >= 0 && j0 + r < kv_len && j0 + r >= kv_begin) row = row0 + (lane / 8);
            }
            if (row >= 0) {
                srck = cache.k + row * CB + chunk * 16;
                srcv = cache.v + row * CB + chunk * 16;
            }
        }
        dma16(srck, st + (uint32_t)(8 * wave * CB));
        dma16(srcv, st + (uint32_t)(ST_CODES + 8 * wave * CB));
        // scales: key j0 + lane
        const char *srcs = reinterpret_cast<const char *>(&kZero16F);
        if (wave < 2 && t < ntiles) {
            const int key = j0 + lane;
            int64_t row = -1;
            if (key < kv_len && key >= kv_begin) {
                if (small_blocks || cache.block_table == nullptr) {
                    row = cache_row(cache, b, g, key);
                } else {
                    // one scalar table read per 16-key group, the lane picks its group's
                    const int64_t r0 = cache_row_wave(cache, b, g, j0);
                    const int64_t r1 = cache_row_wave(cache, b, g, j0 + 16);
                    const int64_t r2 = cache_row_wave(cache, b, g, j0 + 32);
                    const int64_t r3 = cache_row_wave(cache, b, g, j0 + 48);
                    const int grp = lane >> 4;
                    const int64_t rg = grp == 0 ? r0 : grp == 1 ? r1 : grp == 2 ? r2 : r3;
                    row = rg >= 0 ? rg + (lane & 15) : -1;
                }
            }
            if (row >= 0) srcs = reinterpret_cast<const char *>((wave == 0 ? cache.k_scale : cache.v_scale) + row);
        }
        const uint32_t dsts = wave == 0 ? st + ST_KSC : wave == 1 ? st + ST_VSC : lds0 + (uint32_t)(NS * STAGE + 2 * CTILE);
        dma4(srcs, dsts);
    };
    // Conversion of tile t's codes (stage t % NS) into converted tile t & 1:
    // thread i converts the 16 codes of chunk i % 8 of row i / 8, for K and V;
    // threads 0-63 copy a K scale, 64-127 a V scale.  Split into the reads and
    // the conversion with its stores, K and V apart, so that both can sit
    // beside matrix work.
    const int cv_r = tid / 8, cv_c = tid % 8;
    auto conv_read = [&](int t, bool v) __attribute__((always_inline)) {
        return *reinterpret_cast<const uint4 *>(smem + (t % NS) * STAGE + (v ? ST_CODES : 0) + cv_r * CB + cv_c * 16);
    };
    auto scale_read = [&](int t) __attribute__((always_inline)) {
        return tid < 2 * BN ? *reinterpret_cast<const float *>(smem + (t % NS) * STAGE + ST_KSC + tid * 4) : 0.f;
    };
    auto conv_write = [&](int t, bool v, uint4 x) __attribute__((always_inline)) {
        // 16 codes = bf16 chunks 2c and 2c + 1 of the row
        char *ct = smem + NS * STAGE + (t & 1) * CTILE + (v ? CT_V : 0) + cv_r * RB;
        const int sw = v ? vsw(cv_r) : ksw(cv_r);
        *reinterpret_cast<uint4 *>(ct + (((2 * cv_c) ^ sw) * 16)) = c8x8_bf16x8<I8>(x.x, x.y);
        *reinterpret_cast<uint4 *>(ct + (((2 * cv_c + 1) ^ sw) * 16)) = c8x8_bf16x8<I8>(x.z, x.w);
    };
    auto scale_write = [&](int t, float x) __attribute__((always_inline)) {
        if (tid < 2 * BN) *reinterpret_cast<float *>(smem + NS * STAGE + (t & 1) * CTILE + CT_KSC + tid * 4) = x;
    };
    auto convert = [&](int t) __attribute__((always_inline)) {
        conv_write(t, false, conv_read(t, false));
        conv_write(t, true, conv_read(t, true));
        scale_write(t, scale_read(t));
    };

    // ---- softmax state and accumulators ------------------------------------------
    float m_ref = -INFINITY, l_run = 0.f;
    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

    const int tr_g = lane >> 4, tr_j = lane & 15;
    // fragments from converted tile ct: K (key block kb, k-step ks) and V^T
    // (key block kb, 16-key step half, 32-column block db)
    auto k_frag = [&](const char *ct, int kb, int ks) __attribute__((always_inline)) {
        const int key = kb * 32 + nq;
        return *reinterpret_cast<const uint4 *>(ct + key * RB + (((2 * ks + hh) ^ ksw(key)) * 16));
    };
    auto v_frag = [&](const char *ct, int kb, int half, int db) __attribute__((always_inline)) {
        uint2 part[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int row = kb * 32 + half * 16 + 4 * (tr_g >> 1) + 8 * rd + (tr_j >> 2);
            const int col = db * 32 + 16 * (tr_g & 1) + 4 * (tr_j & 3);
            const int chunk = (col >> 3) ^ vsw(row);
            part[rd] = lds_read_tr16(ct + CT_V + row * RB + chunk * 16 + (col & 7) * 2);
        }
        return make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
    };
    // element i of a score block holds key kb * 32 + (i / 4) * 8 + 4 hh + i % 4
    // of this lane's row: four consecutive keys per group of four elements
    auto scales4 = [&](const char *ct, int off, int kb, int gq) __attribute__((always_inline)) {
        return *reinterpret_cast<const float4 *>(ct + off + (kb * 32 + gq * 8 + 4 * hh) * 4);
    };
    // K scale, mask and running maximum of elements 4 gq .. 4 gq + 3 of s
    auto scale_max4 = [&](const char *ct, int t, int kb, int gq, f32x16_t &s, auto masked, int lim, float &m)
        __attribute__((always_inline)) {
        const float4 k4 = scales4(ct, CT_KSC, kb, gq);
        const float kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * gq + e;
            s[i] *= kq[e];   // the key's K scale
            if constexpr (decltype(masked)::value) {
                const int key = t * BN + kb * 32 + gq * 8 + hh * 4 + e;
                if (key >= lim || key < row_lo) s[i] = -INFINITY;
            }
            m = fmaxf(m, s[i]);
        }
    };
    auto vote = [&](float m) __attribute__((always_inline)) {
        // (the maximum is of the K-scaled scores; scale > 0 commutes with it)
        const float mt = max_xor32(m) * p.scale_log2;
        if (__builtin_expect(__ballot(mt > m_ref + TAU) != 0, 0)) {
            asm volatile("" ::: "memory");   // keep the rare rescale a branch
            if (mt > m_ref + TAU) {
                const float alpha = fast_exp2(m_ref - mt);   // 0 on the first tile
                m_ref = mt;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
            }
        }
    };
    // probabilities of pair j of k-step half (keys 8 half + 2 j, +1 of the
    // block's elements): the bf16 values into the row sum, and times the keys'
    // V scales as the V product's operand.  Every key of a loaded tile is
    // either a cached row visible to the workgroup's first row (whose scale
    // the cache's contract makes finite) or a row loaded as zeros, so a
    // masked key's 0 probability times its scale stays 0.
    auto prob_pair = [&](const char *ct, int kb, const f32x16_t &s, int half, int j, float mu, uint32_t (&w)[2][4],
                         float &ps) __attribute__((always_inline)) {
        const int e0 = half * 8 + 2 * j;
        const float4 v4 = scales4(ct, CT_VSC, kb, e0 / 4);
        const float vq0 = (e0 & 2) ? v4.z : v4.x, vq1 = (e0 & 2) ? v4.w : v4.y;
        const float p0 = fast_exp2(fmaf(s[e0], p.scale_log2, -mu));
        const float p1 = fast_exp2(fmaf(s[e0 + 1], p.scale_log2, -mu));
        ps = dot2_bf16(pack_bf16x2(p0, p1), 0x3F803F80u, ps);   // + both rounded probabilities
        w[half][j] = pack_bf16x2(p0 * vq0, p1 * vq1);
    };
    // V product of key block kb with the probabilities of its scores s,
    // formed one k-step ahead; `side(st)` runs beside matrix step st
    auto pv_block = [&](const char *ct, int kb, const f32x16_t &s, auto &&side) __attribute__((always_inline)) {
        const float mu = m_ref == -INFINITY ? 0.f : m_ref;
        uint32_t w[2][4];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) prob_pair(ct, kb, s, 0, j, mu, w, (j & 1) ? ps1 : ps0);
        uint4 vf = v_frag(ct, kb, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < 2 * DB; ++st) {
            const int db = st % DB, half = st / DB;
            const uint4 a = vf;
            if (st + 1 < 2 * DB) vf = v_frag(ct, kb, (st + 1) / DB, (st + 1) % DB);
            acc[db] = mfma32(a, make_uint4(w[half][0], w[half][1], w[half][2], w[half][3]), acc[db]);
            if (half == 0) prob_pair(ct, kb, s, 1, db, mu, w, (db & 1) ? ps1 : ps0);
            side(st);
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run += ps0 + ps1;
    };
    // Tile t from converted tile t & 1, in two 32-key halves so that one
    // half's softmax runs beside the other's matrix work:
    //   S0 = K0 Q^T (beside: the reads of tile t + 1's K codes, then their
    //   conversion); S1 = K1 Q^T (beside: scale, mask and maximum of S0); the
    //   V product of half 0 (beside: its probabilities, and scale, mask and
    //   maximum of S1); the V product of half 1 (beside: its probabilities,
    //   and tile t + 1's V codes and scales).  With `conv`, tile t + 1 is
    //   converted into the other converted tile.  `masked` (the tile needs
    //   the causal or window mask) is a compile-time flag, and so is `conv` on
    //   the steady tiles, which run without branches.
    auto math = [&](int t, auto masked, auto conv_c) __attribute__((always_inline)) {
        const bool conv = conv_c;   // a constant where conv_c is std::true_type
        const char *ct = smem + NS * STAGE + (t & 1) * CTILE;
        const int lim = p.causal ? min(qpos + 1, kv_len) : kv_len;
        f32x16_t s0, s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
        uint4 ck = make_uint4(0u, 0u, 0u, 0u);
        {
            uint4 kf = k_frag(ct, 0, 0);
            if (conv) ck = conv_read(t + 1, false);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 a = kf;
                if (ks + 1 < KS) kf = k_frag(ct, 0, ks + 1);
                s0 = mfma32(a, qf[ks], s0);
                if (conv && ks == 2) conv_write(t + 1, false, ck);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        float m0 = -INFINITY;
        {
            uint4 kf = k_frag(ct, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 a = kf;
                if (ks + 1 < KS) kf = k_frag(ct, 1, ks + 1);
                s1 = mfma32(a, qf[ks], s1);
                if (ks % 2 == 1) scale_max4(ct, t, 0, ks / 2, s0, masked, lim, m0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        vote(m0);
        float m1 = -INFINITY;
        pv_block(ct, 0, s0, [&](int st) __attribute__((always_inline)) {
            if (st % 2 == 1) scale_max4(ct, t, 1, st / 2, s1, masked, lim, m1);
        });
        vote(m1);
        uint4 cv = make_uint4(0u, 0u, 0u, 0u);
        float sc = 0.f;
        pv_block(ct, 1, s1, [&](int st) __attribute__((always_inline)) {
            if (conv) {
                if (st == 0) {
                    cv = conv_read(t + 1, true);
                    sc = scale_read(t + 1);
                }
                if (st == 3) {
                    conv_write(t + 1, true, cv);
                    scale_write(t + 1, sc);
                }
            }
        });
    };

    // ---- the pipeline ---------------------------------------------------------------
    // Iteration t: tile t + 1's codes have landed (waited for), barrier (every
    // wave is past the math of tile t - 1, so converted tile (t + 1) & 1 is
    // free, and past the conversion of tile t, so stage t % NS is free), tile
    // t + NS starts into stage t % NS, tile t's math runs with the conversion
    // of tile t + 1 beside it.  Every wave issues LOADS loads per tile (zeros
    // past the last).
    if (ntiles > t_first) {
#pragma unroll
        for (int k = 0; k < NS; ++k) issue(t_first + k);
        // every load so far, the query fragments included: a wait the
        // compiler would place for them inside the key loop would drain the
        // tile loads in flight on every iteration
        wait_vm<0>();
        barrier();
        convert(t_first);
        auto step = [&](int t, auto masked, auto conv) __attribute__((always_inline)) {
            wait_vm<(NS - 2) * LOADS>();   // tile t + 1 has landed
            barrier();
            issue(t + NS);
            math(t, masked, conv);
        };
        // tiles below the window's lower edge, then the steady tiles (no mask,
        // a next tile to convert), then the tiles at the causal diagonal or
        // the end of the keys and the last tile
        const int t_steady = min(t_mask, ntiles - 1);
        int t = t_first;
        for (; t < ntiles && t < t_lo_end; ++t) step(t, std::true_type{}, t + 1 < ntiles);
        for (; t < t_steady; ++t) step(t, std::false_type{}, std::true_type{});
        for (; t < ntiles; ++t) step(t, std::true_type{}, t + 1 < ntiles);
        wait_vm<0>();   // the loads past the last tile have landed before the LDS is released
    }

    // ---- normalise and store ----------------------------------------------------------
    const float l = sum_xor32(l_run);
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t *orow = reinterpret_cast<uint16_t *>(p.out) + (((int64_t)b * p.s + row_i) * H + (int64_t)g * G + row_r) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = db * 32 + i4 * 8 + hh * 4;
            *reinterpret_cast<uint2 *>(orow + d0) =
                make_uint2(pack_bf16x2(acc[db][4 * i4 + 0] * inv, acc[db][4 * i4 + 1] * inv),
                           pack_bf16x2(acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv));
        }
}

template <bool I8>
hipError_t launch_gp(const PrefillParams &p, int gp, dim3 grid, hipStream_t s)
{
    switch (gp) {
    case 1: hipLaunchKernelGGL((prefill_fp8_kernel<1, I8>), grid, dim3(NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((prefill_fp8_kernel<2, I8>), grid, dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((prefill_fp8_kernel<4, I8>), grid, dim3(NT), 0, s, p); break;
    case 8: hipLaunchKernelGGL((prefill_fp8_kernel<8, I8>), grid, dim3(NT), 0, s, p); break;
    case 16: hipLaunchKernelGGL((prefill_fp8_kernel<16, I8>), grid, dim3(NT), 0, s, p); break;
    case 32: hipLaunchKernelGGL((prefill_fp8_kernel<32, I8>), grid, dim3(NT), 0, s, p); break;
    case 64: hipLaunchKernelGGL((prefill_fp8_kernel<64, I8>), grid, dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp8(const PrefillParams &p, hipStream_t s)
{
    if (p.cache.elem_bytes != 1 || p.cache.d != D) return hipErrorInvalidValue;
    const int gp = pow2_at_least(p.G);
    const int64_t nqb = (p.s + ROWS / gp - 1) / (ROWS / gp);
    if (nqb * p.cache.K * p.B > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(nqb * p.cache.K * p.B));
    return p.cache.int8 ? launch_gp<true>(p, gp, grid, s) : launch_gp<false>(p, gp, grid, s);
}

}  // namespace gqa
