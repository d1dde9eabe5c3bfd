// decode_mfma.hip -- decode on the matrix cores for bf16 caches at head size
// 128 and 64 and 1-byte (FP8 E4M3 or INT8) caches at 128: every group size
// up to G = 64 (the multi-query end) and a block of several newest query
// positions per sequence (speculative-verify shaped).
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps
// 2-4): for sequence b and KV group g, the R = mq * G rows -- query position i
// of the sequence's mq newest tokens, head g*G + j -- attend to K/V head g.
// Row i sits at position ctx[b] - mq + i and sees the keys up to and including
// its own position (the causal rule, so the block is causal among itself),
// from 0 or, with a sliding window of W positions (inference-optimisation
// page §6.4.1), from its position + 1 - W.
//
// How (flash-decoding on the inference-optimisation page §10.2 is prior art
// for the split; the tiling is for CDNA4):
//  * Work list and slices as in the vector decode: the (sequence, KV group)
//    items are cut into 16-key tiles, the flat tile list into one slice per
//    workgroup, and the tiles of one item in a slice (a segment) are dealt
//    round-robin to the 4 waves, which need no barrier per tile.
//  * Each wave streams its tiles through a ring of NSTG stages of its own in
//    LDS (8 KB: the 16 K rows and the 16 V rows), filled NSTG - 1 tiles ahead
//    by LDS-direct loads (global_load_lds_dwordx4: no registers hold data in
//    flight) with explicit vmcnt waits.  Rows are XOR-swizzled in 16-byte
//    slots so that the fragment reads below hit distinct banks.
//  * Scores transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16: the A
//    operand is K (lane: key l%16, 16 bytes of each 32-dimension step), the B
//    operand Q^T stays in registers for the whole item.  A lane then holds 4
//    keys of one row.
//  * Those 4 scores, as bf16 probabilities, are the B operand P^T of
//    O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 exactly as they lie.  V^T
//    comes from the wave's V tile in LDS through the transposing read
//    (ds_read_b64_tr_b16): each lane receives 4 consecutive keys of one
//    column.
//  * Online softmax per row in exp2 units (inference-optimisation page
//    §9.2.1) with a lazy maximum that moves only by >= 2^8; the 4 lanes of a
//    row combine through permlane swaps.
//  * More than 32 rows per KV head (large groups, the multi-query end): the
//    G heads form two items of G / 2 heads over the same K/V head, each
//    streamed by the 32-row kernel.  Each tile is read twice, the second time
//    mostly from the caches; with half the rows per wave the per-item costs
//    (query fragments, the merge of the waves, the store) halve and each
//    wave streams twice as many tiles.
//  * At the end of a segment the 4 waves' (m, l, O) are merged in LDS in wave
//    order (deterministic); a whole item is normalised and stored, a cut item
//    leaves one partial per workgroup that merge_rows_kernel combines with
//    their global max and sum (page §10.2).
//  * FP8 E4M3 cache with a scale per row (inference-optimisation page
//    §15.5.1): the stages hold the 1-byte rows and the tile's 16 K and 16 V
//    scales; K fragments become bf16 in registers (every E4M3 value is a bf16
//    value), the V tile is converted once into a bf16 tile in LDS for the
//    transposing reads, the K scale multiplies the key's score and the V
//    scale its probability (so the V product runs on codes).
//  * A decode step (one position, k_new / v_new given): the newest key and
//    value of every item are loaded from k_new / v_new instead of the cache,
//    and the kernel also copies them into the cache (the bytes the append
//    kernel would write; no launch of this kernel reads those rows).
#include "common.h"
#include "kernels.h"
#include "worklist.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int NT = 256;            // threads per workgroup; two workgroups per CU
constexpr int NW = NT / kWave;     // waves
constexpr int TT = 16;             // keys per tile
constexpr float TAU = 8.0f;        // lazy-rescale threshold (log2 units)
constexpr int MAX_ROWS = 64;       // R = mq * G
// Head dimensions: 128 (bf16 and 1-byte caches) and 64 (bf16).  A bf16 row of D
// values is CPR 16-byte chunks, and one 1 KB LDS-direct load fills RPL rows.
template <int D> struct Dim {
    static constexpr int RB = D * 2;          // bytes per bf16 K/V row
    static constexpr int KS = D / 32;         // 32-dimension steps of S^T = K Q^T
    static constexpr int DB = D / 16;         // 16-dimension blocks of O^T
    static constexpr int CPR = RB / 16;       // 16-byte chunks per row
    static constexpr int RPL = 64 / CPR;      // rows per 1 KB load
    static constexpr int LPT = TT / RPL;      // 1 KB loads per tile, for K and again for V
};
// Workgroups per CU: two up to 16 rows (the registers allow it), one above.
// LDS stages per wave: two in every case.  More stages measured slower: 4
// against 2 at one workgroup per CU (MQA 27.9 against 26.9 us), 3 against 2
// for FP8 (43.9 against 42.0 us), 6 against 2 for FP8 at one workgroup per CU
// (an FP8 MQA decode, 34.2 against 30.6 us), 4 against 2 at d = 64 (38.1
// against 37.1 us).
constexpr int NSTG = 2;
__host__ __device__ constexpr int occ_of(int rbw) { return rbw == 1 ? 2 : 1; }
// FP8: K row r keeps its 16-byte chunk c (of 8) in slot c ^ (r & 7)
__device__ __forceinline__ constexpr int ksw8(int r) { return r & 7; }
// two E4M3 codes (bytes 0-1, or 2-3 with HI) -> a bf16 pair, exactly
template <bool HI>
__device__ __forceinline__ uint32_t f8x2_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// four INT8 codes c (byte i of w) -> the bf16 values of c + 128, exactly
// (integers 1 .. 255 have at most 8 significant bits): one byte-to-float
// conversion per code and a byte permute per pair
__device__ __forceinline__ uint2 i8x4_biased_bf16x4(uint32_t w)
{
    const uint32_t u = w ^ 0x80808080u;
    const float f0 = (float)(u & 0xFFu), f1 = (float)((u >> 8) & 0xFFu);
    const float f2 = (float)((u >> 16) & 0xFFu), f3 = (float)(u >> 24);
    return make_uint2(__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
                      __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u));
}
// eight 1-byte codes -> eight bf16 values, exactly: E4M3 codes, or with I8
// INT8 codes biased by +128 (the kernel takes the bias back out of the
// scores and the weighted sum, see the decode kernel)
template <bool I8>
__device__ __forceinline__ uint4 c8x8_bf16x8(uint2 x)
{
    if constexpr (I8) {
        const uint2 a = i8x4_biased_bf16x4(x.x), b = i8x4_biased_bf16x4(x.y);
        return make_uint4(a.x, a.y, b.x, b.y);
    }
    return make_uint4(f8x2_bf16x2<false>(x.x), f8x2_bf16x2<true>(x.x), f8x2_bf16x2<false>(x.y), f8x2_bf16x2<true>(x.y));
}
// A stage: the tile's K rows, its V rows and (FP8) its 16 K and 16 V scales
template <bool F8, int D> struct Stage {
    static constexpr int ROWB = F8 ? D : D * 2;                 // bytes per cached row
    static constexpr int KV = TT * ROWB;                        // bytes of K (and of V) per tile
    static constexpr int BYTES = 2 * KV + (F8 ? 2 * TT * 4 : 0);
    static constexpr int DMA = 2 * KV / 1024 + (F8 ? 1 : 0);   // LDS-direct loads per tile
};

__device__ const uint4 kZero16M = {0u, 0u, 0u, 0u};

// One LDS-direct 16-byte load per lane: lane i's bytes land at lds + 16 i.
// Inline assembly, so that the compiler does not wait for these loads before
// LDS reads; the kernel waits with explicit vmcnt.  Non-temporal (nt): every
// cached byte is read once per call, and the streaming policy keeps these
// lines from displacing the rest of the caches' contents (measured 12-14%
// faster decode than the default policy).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
#pragma clang diagnostic pop
}
// The same with 4 bytes per lane (lane i's bytes land at lds + 4 i).
__device__ __forceinline__ void dma4(const void *src, uint32_t lds)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off nt"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
#pragma clang diagnostic pop
}
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// K row r keeps its 16-byte chunk c in slot c ^ ksw(r): the 16 lanes of an
// A-operand read (16 keys, one chunk) then fall on 16 different bank groups
// (at d = 64 two rows share the 64 banks, so consecutive row pairs take
// consecutive slots)
template <int D>
__device__ __forceinline__ constexpr int ksw(int r) { return Dim<D>::CPR >= 16 ? (r & 15) : ((r >> 1) & (Dim<D>::CPR - 1)); }

__device__ __forceinline__ f32x4_t mfma_s(uint4 a, uint4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_o(uint2 a, uint2 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b),
                                                     c, 0, 0, 0);
}
// V row r keeps its 16-byte chunk c in slot c ^ vsw(r): the transposing reads
// (16 lanes, 4 rows x 4 pieces of 4 columns) then spread over the banks
template <int D>
__device__ __forceinline__ constexpr int vsw(int r) { return Dim<D>::CPR >= 16 ? 4 * (r & 3) : 2 * (r & 3); }
__device__ __forceinline__ uint2 lds_read_tr16(const char *p)
{
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(lds_void_t *)p);
    return __builtin_bit_cast(uint2, v);
}
// the sum / max over the 4 lanes of a row (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float row_sum(float x)
{
    const float2 a = swap_pair16(x);
    x = a.x + a.y;
    const float2 b = swap_pair32(x);
    return b.x + b.y;
}
__device__ __forceinline__ float row_max(float x)
{
    const float2 a = swap_pair16(x);
    x = fmaxf(a.x, a.y);
    const float2 b = swap_pair32(x);
    return fmaxf(b.x, b.y);
}

// RBW: 16-row blocks (R <= 16 * RBW); occ_of(RBW) workgroups per CU; F8: the
// cache holds E4M3 codes and a scale per row (d = 128); D: the head dimension
template <int RBW, bool F8, int D, bool I8 = false>
__global__ __launch_bounds__(NT, occ_of(RBW)) void decode_mfma_kernel(RowAttnParams p)
{
    static_assert(!F8 || D == 128, "FP8 caches at d = 128");
    constexpr int RB = Dim<D>::RB, KS = Dim<D>::KS, DB = Dim<D>::DB;
    constexpr int CPR = Dim<D>::CPR, RPL = Dim<D>::RPL, LPT = Dim<D>::LPT;
    constexpr int RP = 16 * RBW;
    constexpr int STG = Stage<F8, D>::BYTES, DMA_PER_TILE = Stage<F8, D>::DMA, CRB = Stage<F8, D>::ROWB;
    __shared__ __attribute__((aligned(1024))) char lds_stage[NW][NSTG * STG];
    __shared__ __attribute__((aligned(16))) char lds_vbf[F8 ? NW : 1][F8 ? TT * RB : 16];   // FP8: the tile's V as bf16
    // the merge area of a segment's end reuses the stages (every load has
    // landed and every wave is past its reads when it is written); row r keeps
    // its 16-byte chunk c in slot c ^ (r & 15), so that the 16 rows a store
    // instruction touches fall on different banks without padding
    constexpr int C4 = D / 4;   // 16-byte chunks per merge-area row
    // one region per wave where they fit (one round of writes), else two
    // regions that the other two waves add to
    constexpr int NREG = 4 * RP * D * 4 <= NW * NSTG * STG ? 4 : 2 * RP * D * 4 <= NW * NSTG * STG ? 2 : 1;
    static_assert(NREG * RP * D * 4 <= NW * NSTG * STG, "merge area fits in the stages");
    float4 (*lds_o)[RP][C4] = reinterpret_cast<float4 (*)[RP][C4]>(&lds_stage[0][0]);
    __shared__ float lds_row[RP][2];   // the merged (max, sum) of each row
    __shared__ float lds_ml[NW][RP][2];
    __shared__ int32_t lds_prefix[kStreamRows + 1];
    __shared__ int32_t lds_nvis[kStreamRows];
    __shared__ int32_t lds_first[kStreamRows];
    __shared__ int32_t lds_newest[kStreamRows];   // ctx - 1 (the newest position), -1 past the capacity
    __shared__ int lds_waves[NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const CacheView &cache = p.cache;
    const int G = p.G, H = p.H, mq = p.mq > 1 ? p.mq : 1;
    const int R = mq * G;
    const int nr = lane & 15, lg = lane >> 4;   // row within a 16-row block; lane group
    const int ls = p.kv_split > 1 ? __builtin_ctz((unsigned)p.kv_split) : 0;   // items per KV head: 2^ls

    // decode step: thread (item, K or V, 16-byte piece) loads its piece of a
    // new row now and stores it into the cache once the tables are built
    constexpr int IPW = NT / (2 * (RB / 16));   // items per workgroup pass
    const bool with_new = p.k_new != nullptr;
    const int64_t cp_items = with_new ? (int64_t)p.rows * cache.K : 0;
    const int cp_which = (tid / (RB / 16)) & 1, cp_piece = tid % (RB / 16);
    auto copy_dst = [&](int64_t it, int64_t &src) -> char * {
        const int b = (int)(p.row0 + it / cache.K), g = (int)(it % cache.K);
        const int pos = p.ctx_lens[b] - 1;
        if (pos < 0 || pos >= cache.capacity) return nullptr;
        const int64_t row = cache_row(cache, b, g, pos);
        if (row < 0) return nullptr;
        src = ((int64_t)b * cache.K + g) * RB + cp_piece * 16;
        return (cp_which ? cache.v : cache.k) + row * RB + cp_piece * 16;
    };
    char *cp_to = nullptr;
    uint4 cp_val = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t it = (int64_t)blockIdx.x * IPW + tid / (2 * (RB / 16)); it < cp_items; it += (int64_t)gridDim.x * IPW) {
        int64_t src = 0;
        char *dst = copy_dst(it, src);
        if (dst == nullptr) continue;
        const uint4 x = ld16((cp_which ? p.v_new : p.k_new) + src);
        if (it == (int64_t)blockIdx.x * IPW + tid / (2 * (RB / 16))) {
            cp_to = dst;   // the first item's store waits until the tables are built
            cp_val = x;
        } else {
            st16(dst, x);
        }
    }

    build_tables<NT>(p, TT, lds_prefix, lds_nvis, lds_first, lds_waves, lds_newest);
    if (cp_to != nullptr) st16(cp_to, cp_val);
    if (blockIdx.x == 0 && p.prefix != nullptr)   // the merge kernel reads it from the workspace
        for (int r = tid; r <= p.rows; r += NT) p.prefix[r] = lds_prefix[r];
    const int T = lds_prefix[p.rows];
    const int64_t W = gridDim.x;
    const int tau0 = (int)slice_start(blockIdx.x, T, W), tau1 = (int)slice_start(blockIdx.x + 1, T, W);
    if (tau0 >= tau1) return;

    char *sw = lds_stage[wave];
    const uint32_t lds_w = (uint32_t)(uintptr_t)(lds_void_t *)sw;
    // LDS-direct load i of a tile (i < 4: K, else V) fills rows 4 (i % 4) + lg,
    // slot nr, with chunk nr ^ swizzle(row) of that row.
    // Transposing reads: lane (group lg, index nr) addresses V row 4 lg + nr / 4,
    // columns 16 db + 4 (nr % 4) .. +3
    const int tr_row = 4 * lg + (nr >> 2);
    // Byte offsets of this lane's piece in the loads of a tile whose rows are
    // all visible (the common case): load i fills tile row 4 (i % 4) + lg
    // (bf16) or 8 (i % 2) + lane / 8 (FP8), K first, then V; the tile's first
    // cache row is added as a wave-uniform base.
    uint32_t lane_off[F8 ? 4 : DMA_PER_TILE];
#pragma unroll
    for (int i = 0; i < (F8 ? 4 : DMA_PER_TILE); ++i) {
        if constexpr (!F8) {
            const int r = RPL * (i % LPT) + lane / CPR, slot = lane % CPR;
            lane_off[i] = (uint32_t)(r * RB + (slot ^ (i >= LPT ? vsw<D>(r) : ksw<D>(r))) * 16);
        } else {
            const int r = 8 * (i % 2) + lane / 8, slot = lane % 8;
            lane_off[i] = (uint32_t)(r * CRB + (i >= 2 ? slot : slot ^ ksw8(r)) * 16);
        }
    }

    int at = tau0;
    while (at < tau1) {
        const Cursor c = cursor_at(lds_prefix, lds_nvis, lds_first, p.rows, at, TT);
        const int64_t seq = p.row0 + c.row;
        const int b = (int)seq, g = c.g;
        const int gc = g >> ls;   // the item's KV head
        const int n_vis = c.n_vis, lo = c.lo;
        const int new_key = with_new ? lds_newest[c.row] : -1;   // read from k_new / v_new
        const int end = min(tau1, c.item0 + c.tiles);
        const int n_seg = end - at;
        const int n_w = n_seg > wave ? (n_seg - wave + NW - 1) / NW : 0;
        // the context length from the table (a length past the capacity is clamped to it)
        const int ctx_b = lds_newest[c.row] >= 0 ? lds_newest[c.row] + 1 : n_vis;
        // tile k of this wave in the segment: row tile c.jlo + (at - item0) + wave + NW k
        const int j_first = at - c.item0;
        auto tile_key0 = [&](int k) { return (c.jlo + j_first + wave + NW * k) * TT; };
        // the LDS-direct loads of tile k into stage k % NSTG; rows outside
        // [lo, n_vis), and tiles past the wave's last, read a zero constant
        auto issue = [&](int k) {
            const int key0 = tile_key0(k);
            const int64_t base = k < n_w ? cache_row_wave(cache, b, gc, key0) : -1;   // 16 keys: one cache block
            const uint32_t dst = lds_w + (uint32_t)((k % NSTG) * STG);
            // every row of the tile visible and none of them the newest token:
            // a uniform base plus the lane offsets, no per-lane tests
            const int full = __builtin_amdgcn_readfirstlane(
                (int)(base >= 0 && key0 >= lo && key0 + TT <= n_vis && (unsigned)(new_key - key0) >= (unsigned)TT));
            if (full) {
                const char *kb = cache.k + base * CRB, *vb = cache.v + base * CRB;
#pragma unroll
                for (int i = 0; i < (F8 ? 4 : DMA_PER_TILE); ++i)
                    dma16((i >= (F8 ? 2 : LPT) ? vb : kb) + lane_off[i], dst + (uint32_t)(i * 1024));
                if constexpr (F8) {
                    // the 16 K scales (lanes 0-15) and the 16 V scales (lanes 16-31)
                    if (lane < 32)
                        dma4(reinterpret_cast<const char *>((lane >= 16 ? cache.v_scale : cache.k_scale) + base + lane % 16),
                             dst + (uint32_t)(2 * Stage<F8, D>::KV));
                }
                return;
            }
            if constexpr (!F8) {
#pragma unroll
                for (int i = 0; i < DMA_PER_TILE; ++i) {
                    const bool is_v = i >= LPT;
                    const int r = RPL * (i % LPT) + lane / CPR;
                    const int chunk = (lane % CPR) ^ (is_v ? vsw<D>(r) : ksw<D>(r));
                    const char *src = reinterpret_cast<const char *>(&kZero16M);
                    if (base >= 0 && key0 + r < n_vis && key0 + r >= lo)
                        src = key0 + r == new_key ? (is_v ? p.v_new : p.k_new) + ((int64_t)b * cache.K + gc) * RB + chunk * 16
                                                  : (is_v ? cache.v : cache.k) + (base + r) * RB + chunk * 16;
                    dma16(src, dst + (uint32_t)(i * 1024));
                }
            } else {
                // K: rows 8 i + lane / 8, slot lane % 8 (chunk slot ^ ksw8(row));
                // V: the same rows, unswizzled
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool is_v = i >= 2;
                    const int r = 8 * (i % 2) + lane / 8, slot = lane % 8;
                    const int chunk = is_v ? slot : slot ^ ksw8(r);
                    const char *src = reinterpret_cast<const char *>(&kZero16M);
                    if (base >= 0 && key0 + r < n_vis && key0 + r >= lo)
                        src = (is_v ? cache.v : cache.k) + (base + r) * CRB + chunk * 16;
                    dma16(src, dst + (uint32_t)(i * 1024));
                }
                // the 16 K scales (lanes 0-15) and the 16 V scales (lanes 16-31),
                // one per lane; a key outside the visible range reads zero
                if (lane < 32) {
                    const int r = lane % 16;
                    const char *src = reinterpret_cast<const char *>(&kZero16M);
                    if (base >= 0 && key0 + r < n_vis && key0 + r >= lo)
                        src = reinterpret_cast<const char *>((lane >= 16 ? cache.v_scale : cache.k_scale) + base + r);
                    dma4(src, dst + (uint32_t)(2 * Stage<F8, D>::KV));
                }
            }
        };

        float m_ref[RBW], l_run[RBW];
        // INT8: the sum of the V product's operands (the bf16 weights), for
        // the +128 bias of the converted V codes
        float w_run[RBW];
        f32x4_t acc[RBW][DB];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            m_ref[rb] = -INFINITY;
            l_run[rb] = 0.f;
            w_run[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[rb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        // the first tiles start, then the q fragments load behind them; one
        // full wait then covers both (a wait the compiler inserts itself for
        // the q loads, unaware of the tile loads, would land inside the loop)
#pragma unroll
        for (int k = 0; k < NSTG - 1; ++k) issue(k);
        // this lane's rows: rho = 16 rb + nr -> query position i = rho / G, head j = rho % G
        uint4 qf[RBW][KS];
        int lim[RBW], rlo[RBW];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const int rho = 16 * rb + nr;
            const bool ok = rho < R;
            const int i = ok ? rho / G : 0, j = ok ? rho % G : 0;
            const int64_t qpos = (int64_t)ctx_b - mq + i;
            lim[rb] = ok ? (int)min(max(qpos + 1, (int64_t)0), (int64_t)n_vis) : 0;
            rlo[rb] = p.window > 0 ? (int)max((int64_t)0, qpos + 1 - p.window) : 0;
            const char *qrow = p.q + (((seq * mq + i) * H + (int64_t)g * G + j) * D) * 2;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[rb][ks] = ok ? *reinterpret_cast<const uint4 *>(qrow + ks * 64 + lg * 16) : make_uint4(0, 0, 0, 0);
        }

        // keys [rlo_max, lim_min) are visible to every row of the item: the
        // oldest position's limit and the newest position's window start
        const int lim_min = (int)min(max((int64_t)ctx_b - mq + 1, (int64_t)0), (int64_t)n_vis);
        const int rlo_max = p.window > 0 ? (int)max((int64_t)0, (int64_t)ctx_b - p.window) : 0;

        // INT8: 128 times the sum of each row's query values, the bias the
        // +128-biased K codes add to every score of the row (exact for the
        // integer-valued rows of the exact tests; otherwise the fp32
        // cancellation error is ~2^-24 of 128 sum |q| per score)
        float qbias[RBW];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) qbias[rb] = 0.f;
        wait_vm<0>();
        if constexpr (I8) {
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                float qs = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    qs = dot2_bf16(qf[rb][ks].x, 0x3F803F80u, qs);
                    qs = dot2_bf16(qf[rb][ks].y, 0x3F803F80u, qs);
                    qs = dot2_bf16(qf[rb][ks].z, 0x3F803F80u, qs);
                    qs = dot2_bf16(qf[rb][ks].w, 0x3F803F80u, qs);
                }
                qbias[rb] = 128.f * row_sum(qs);
            }
        }
        // last: the wave's last tile of the segment, after which nothing is
        // issued (so the wait is for every load the wave has in flight)
        auto step = [&](int k, bool last) {
            const int key0 = tile_key0(k);
            if (!last) {
                // tile k + NSTG - 1 goes into the stage read in the previous step
                issue(k + NSTG - 1);
                wait_vm<(NSTG - 1) * DMA_PER_TILE>();   // tile k has landed
            } else {
                wait_vm<0>();
            }
            const char *kt = sw + (k % NSTG) * STG;
            const char *vt = F8 ? lds_vbf[F8 ? wave : 0] : kt + Stage<F8, D>::KV;
            uint4 kf[KS];
            float ksc[4] = {1.f, 1.f, 1.f, 1.f}, vsc[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (!F8) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[ks] = *reinterpret_cast<const uint4 *>(kt + nr * RB + (((4 * ks + lg) ^ ksw<D>(nr)) * 16));
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int chunk = 2 * ks + (lg >> 1);
                    kf[ks] = c8x8_bf16x8<I8>(*reinterpret_cast<const uint2 *>(kt + nr * CRB + ((chunk ^ ksw8(nr)) * 16) +
                                                                          (lg & 1) * 8));
                }
                // scales of this lane's keys 4 lg .. 4 lg + 3
                const float4 k4 = *reinterpret_cast<const float4 *>(kt + 2 * Stage<F8, D>::KV + 16 * lg);
                const float4 v4 = *reinterpret_cast<const float4 *>(kt + 2 * Stage<F8, D>::KV + 64 + 16 * lg);
                ksc[0] = k4.x; ksc[1] = k4.y; ksc[2] = k4.z; ksc[3] = k4.w;
                vsc[0] = v4.x; vsc[1] = v4.y; vsc[2] = v4.z; vsc[3] = v4.w;
                // the V tile as bf16 (swizzled as a bf16 tile): lane i converts
                // the 32 bytes of row i / 4 at columns 32 (i % 4) ..
                const char *vsrc = kt + Stage<F8, D>::KV + lane * 32;
                char *vdst = lds_vbf[F8 ? wave : 0];
                const int vr = lane >> 2;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 x = *reinterpret_cast<const uint4 *>(vsrc + 16 * h);
                    const int c0 = 4 * (lane & 3) + 2 * h;   // logical bf16 chunk of the first 8 columns
                    *reinterpret_cast<uint4 *>(vdst + vr * RB + ((c0 ^ vsw<D>(vr)) * 16)) = c8x8_bf16x8<I8>(make_uint2(x.x, x.y));
                    *reinterpret_cast<uint4 *>(vdst + vr * RB + (((c0 + 1) ^ vsw<D>(vr)) * 16)) = c8x8_bf16x8<I8>(make_uint2(x.z, x.w));
                }
            }
            // S^T = K Q^T: lane holds keys key0 + 4 lg + e of row 16 rb + nr
            f32x4_t s[RBW];
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                s[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) s[rb] = mfma_s(kf[ks], qf[rb][ks], s[rb]);
            }
            // mask (only where the tile reaches past some row's visible keys),
            // tile maximum, lazy rescale
            if constexpr (F8) {
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (I8) s[rb][e] -= qbias[rb];   // the +128 bias of the K codes
                        s[rb][e] *= ksc[e];                        // the key's K scale
                    }
            }
            if (key0 < rlo_max || key0 + TT > lim_min) {
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = key0 + 4 * lg + e;
                        if (key >= lim[rb] || key < rlo[rb]) s[rb][e] = -INFINITY;
                    }
            }
            bool need = false;
            float mt[RBW];
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                float m = -INFINITY;
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, s[rb][e]);
                mt[rb] = row_max(m) * p.scale_log2;   // scale > 0: the max commutes with it
                need |= mt[rb] > m_ref[rb] + TAU;
            }
            if (__ballot(need) != 0) {
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb) {
                    if (mt[rb] > m_ref[rb] + TAU) {
                        const float al = fast_exp2(m_ref[rb] - mt[rb]);   // 0 on the first tile
                        m_ref[rb] = mt[rb];
                        l_run[rb] *= al;
                        if constexpr (I8) w_run[rb] *= al;
#pragma unroll
                        for (int db = 0; db < DB; ++db) acc[rb][db] *= al;
                    }
                }
            }
            // P^T (bf16, rounded) and the running sum of the rounded values
            uint2 pw[RBW];
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                const float mu = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
                const float p0 = fast_exp2(fmaf(s[rb][0], p.scale_log2, -mu));
                const float p1 = fast_exp2(fmaf(s[rb][1], p.scale_log2, -mu));
                const float p2 = fast_exp2(fmaf(s[rb][2], p.scale_log2, -mu));
                const float p3 = fast_exp2(fmaf(s[rb][3], p.scale_log2, -mu));
                pw[rb] = make_uint2(pack_bf16x2(p0, p1), pack_bf16x2(p2, p3));
                l_run[rb] = dot2_bf16(pw[rb].x, 0x3F803F80u, l_run[rb]);
                l_run[rb] = dot2_bf16(pw[rb].y, 0x3F803F80u, l_run[rb]);
                if constexpr (F8) {
                    // the key's V scale rides on its probability (a masked key's
                    // probability is 0 and its scale is not looked at)
                    const float w0 = p0 > 0.f ? p0 * vsc[0] : 0.f, w1 = p1 > 0.f ? p1 * vsc[1] : 0.f;
                    const float w2 = p2 > 0.f ? p2 * vsc[2] : 0.f, w3 = p3 > 0.f ? p3 * vsc[3] : 0.f;
                    pw[rb] = make_uint2(pack_bf16x2(w0, w1), pack_bf16x2(w2, w3));
                    if constexpr (I8) {
                        w_run[rb] = dot2_bf16(pw[rb].x, 0x3F803F80u, w_run[rb]);
                        w_run[rb] = dot2_bf16(pw[rb].y, 0x3F803F80u, w_run[rb]);
                    }
                }
            }
            // O^T += V^T P^T, one 16-column block of V^T per transposing read
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int col = 16 * db + 4 * (nr & 3);
                const int chunk = (col >> 3) ^ vsw<D>(tr_row);
                const uint2 vf = lds_read_tr16(vt + tr_row * RB + chunk * 16 + (col & 7) * 2);
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb) acc[rb][db] = mfma_o(vf, pw[rb], acc[rb][db]);
            }
        };
        for (int k = 0; k + 1 < n_w; ++k) step(k, false);
        if (n_w > 0) step(n_w - 1, true);
        wait_vm<0>();   // (a wave with no tile here: its first-tile loads) before the stages are reused

        // ---- merge the 4 waves' pieces in LDS, in wave order ------------------
        if constexpr (I8) {
            // take the +128 bias of the V codes out: sum w (c + 128) - 128 sum w
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) {
                const float wb = 128.f * row_sum(w_run[rb]);
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[rb][db] -= wb;
            }
        }
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            l_run[rb] = row_sum(l_run[rb]);
            if (lg == 0) {
                lds_ml[wave][16 * rb + nr][0] = n_w > 0 ? m_ref[rb] : -INFINITY;
                lds_ml[wave][16 * rb + nr][1] = n_w > 0 ? l_run[rb] : 0.f;
            }
        }
        __syncthreads();
        float wt[RBW];
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            const int row = 16 * rb + nr;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_ml[w][row][0]);
            wt[rb] = (n_w > 0 && m_ref[rb] != -INFINITY) ? fast_exp2(m_ref[rb] - M) : 0.f;
        }
        // region wave % NREG: written by the first NREG waves, added to by the rest
        for (int round = 0; round < NW / NREG; ++round) {
            if (wave / NREG == round) {
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        float4 *o = &lds_o[wave % NREG][16 * rb + nr][(4 * db + lg) ^ nr];
                        float4 x = make_float4(acc[rb][db][0] * wt[rb], acc[rb][db][1] * wt[rb], acc[rb][db][2] * wt[rb],
                                               acc[rb][db][3] * wt[rb]);
                        if (round > 0) {
                            const float4 y = *o;
                            x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
                        }
                        *o = x;
                    }
            }
            __syncthreads();
        }
        // each row's merged maximum and sum, once
        if (tid < R) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_ml[w][tid][0]);
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = lds_ml[w][tid][0];
                if (mw != -INFINITY) L += lds_ml[w][tid][1] * fast_exp2(mw - M);
            }
            lds_row[tid][0] = M;
            lds_row[tid][1] = L;
        }
        __syncthreads();
        const bool whole = at == c.item0 && end == c.item0 + c.tiles;
        const int slot = tau0 < c.item0 ? 1 : 0;
        for (int idx = tid; idx < R * (D / 4); idx += NT) {
            const int rho = idx / (D / 4), col = (idx % (D / 4)) * 4;
            const float M = lds_row[rho][0], L = lds_row[rho][1];
            const int c4 = (col >> 2) ^ (rho & 15);
            float4 O = lds_o[0][rho][c4];
#pragma unroll
            for (int r = 1; r < NREG; ++r) {
                const float4 y = lds_o[r][rho][c4];
                O.x += y.x; O.y += y.y; O.z += y.z; O.w += y.w;
            }
            if (whole) {
                const int i = rho / G, j = rho % G;
                const float inv = L > 0.f ? 1.f / L : 0.f;   // a row with no visible key is zero
                *reinterpret_cast<uint2 *>(p.out + (((seq * mq + i) * H + (int64_t)g * G + j) * D + col) * 2) =
                    make_uint2(pack_bf16x2(O.x * inv, O.y * inv), pack_bf16x2(O.z * inv, O.w * inv));
            } else {
                const int64_t sr = ((int64_t)blockIdx.x * 2 + slot) * R + rho;
                *reinterpret_cast<float4 *>(p.ws_o + sr * D + col) = O;
                if (col == 0) {
                    p.ws_ml[sr * 2] = M;
                    p.ws_ml[sr * 2 + 1] = L;
                }
            }
        }
        __syncthreads();   // lds_o and lds_ml are free again
        at = end;
    }
}

// The pieces of the items cut by slice boundaries: workgroup (g, row, z)
// merges rows 4 z .. 4 z + 3 of item (sequence row0 + row, group g) with
// their global max and sum (inference-optimisation page §10.2), one float4
// of a row per thread; an item with no visible key gets zero rows.  With
// PG > 1 the pieces are dealt to PG thread groups (piece k to group k % PG),
// so that an item cut into many pieces loads them all in one memory round
// trip; the groups' partial results are then combined in group order.
constexpr int kMergeRows = 4;   // rows per workgroup (more workgroups for the many-piece items of large groups)
template <int PG, int D>
__global__ __launch_bounds__(PG * kMergeRows * (D / 4)) void merge_rows_kernel(RowAttnParams p, int W)
{
    constexpr int TPG = kMergeRows * (D / 4);   // threads per piece group
    __shared__ float4 lds_o[PG > 1 ? PG : 1][TPG];
    __shared__ float2 lds_ml[PG > 1 ? PG : 1][TPG];
    const int g = blockIdx.x, row = blockIdx.y;
    const int G = p.G, H = p.H, mq = p.mq > 1 ? p.mq : 1;
    const int R = mq * G;
    // the piece group is uniform over a wave (TPG is two waves), so the slot
    // arithmetic below stays scalar
    const int pg = PG > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / TPG) : 0;
    const int t = (int)threadIdx.x % TPG;
    const int rho = blockIdx.z * kMergeRows + t / (D / 4), col = (t % (D / 4)) * 4;
    const int64_t seq = p.row0 + row;
    // the table entries and the context length are read together (one
    // memory round trip instead of two)
    const int64_t T = p.prefix[p.rows], pre = p.prefix[row];
    const int n_vis = row_visible(p, seq);
    const int lo = row_first(p, seq, n_vis);
    uint16_t *dst = reinterpret_cast<uint16_t *>(p.out) +
                    ((seq * mq + rho / G) * H + (int64_t)g * G + rho % G) * D + col;
    if (n_vis <= lo) {
        if (rho < R && pg == 0) *reinterpret_cast<uint2 *>(dst) = make_uint2(0u, 0u);
        return;
    }
    const int64_t tiles = item_tiles(lo, n_vis, TT);
    const int64_t a = pre + (int64_t)g * tiles, e = a + tiles - 1;
    const int64_t wa = slice_owner(a, T, W), wb = slice_owner(e, T, W);
    if (wa == wb) return;   // one piece: the main kernel stored the rows
    // the workspace slots of the pieces: with at least one tile per slice
    // (T >= W) the pieces are the slices wa .. wb, the first one in slot 1
    // when the item starts inside it; otherwise every tile of the item is a
    // piece of its own, in slot 0 of its slice
    const bool dense = T >= W;
    if constexpr (PG == 1) {
        if (rho >= R) return;
    }
    const bool live = PG == 1 || rho < R;   // with PG > 1 every thread reaches the barrier below
    const int ns = dense ? (int)(wb - wa + 1) : (int)(e - a + 1);
    const int slot0 = (int)(wa * 2 + (slice_start(wa, T, W) < a ? 1 : 0));
    auto slot_of = [&](int k) {
        return dense ? (k == 0 ? slot0 : (int)(wa + k) * 2) : (int)sparse_slot(a + k, T, W);
    };
    // this group's pieces pg, pg + PG, ... in batches of 8 whose loads are
    // issued together; within a batch and from batch to batch the running
    // maximum rescales what is summed
    constexpr int BATCH = 8;
    float M = -INFINITY, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = pg; k0 < ns; k0 += BATCH * PG) {
        float mm[BATCH], ll[BATCH];
        float4 oo[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            mm[j] = -INFINITY;
            ll[j] = 0.f;
            oo[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            const int k = k0 + j * PG;
            if (live && k < ns) {
                const int64_t sr = (int64_t)slot_of(k) * R + rho;
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
    if constexpr (PG > 1) {
        // the groups' (max, sum, row) combined by group 0, in group order
        lds_o[pg][t] = O;
        lds_ml[pg][t] = make_float2(M, L);
        __syncthreads();
        if (pg != 0) return;
        float Mx = M;
#pragma unroll
        for (int q = 1; q < PG; ++q) Mx = fmaxf(Mx, lds_ml[q][t].x);
        float Ls = 0.f;
        float4 Os = make_float4(0.f, 0.f, 0.f, 0.f);
        if (Mx != -INFINITY) {
#pragma unroll
            for (int q = 0; q < PG; ++q) {
                const float2 ml = lds_ml[q][t];
                if (ml.x == -INFINITY) continue;
                const float wt = fast_exp2(ml.x - Mx);
                const float4 o = lds_o[q][t];
                Ls += ml.y * wt;
                Os.x += o.x * wt; Os.y += o.y * wt; Os.z += o.z * wt; Os.w += o.w * wt;
            }
        }
        L = Ls;
        O = Os;
    }
    if (!live) return;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(O.x * inv, O.y * inv), pack_bf16x2(O.z * inv, O.w * inv));
}

template <int RBW, int D>
hipError_t launch_m(const RowAttnParams &p0, hipStream_t s)
{
    RowAttnParams p = p0;
    // slices resident at once: occ_of(RBW) per CU, unless the caller fixed the count
    p.num_wgs = p0.wgs_override > 0 ? p0.wgs_override : p0.num_wgs * occ_of(RBW) / 2;
    if (p.cache.elem_bytes == 1) {
        if constexpr (D == 128) {
            if (p.cache.int8) hipLaunchKernelGGL((decode_mfma_kernel<RBW, true, D, true>), dim3(p.num_wgs), dim3(NT), 0, s, p);
            else hipLaunchKernelGGL((decode_mfma_kernel<RBW, true, D, false>), dim3(p.num_wgs), dim3(NT), 0, s, p);
        }
        else return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((decode_mfma_kernel<RBW, false, D>), dim3(p.num_wgs), dim3(NT), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int R = (p.mq > 1 ? p.mq : 1) * p.G;
    const dim3 mgrid(p.cache.K * (p.kv_split > 1 ? p.kv_split : 1), p.rows, (R + kMergeRows - 1) / kMergeRows);
    // items of 32 rows or more (large groups: few, long items) are cut into
    // many pieces; their merge loads the pieces in four groups at once
    if (R >= 32) hipLaunchKernelGGL((merge_rows_kernel<4, D>), mgrid, dim3(4 * kMergeRows * (D / 4)), 0, s, p, p.num_wgs);
    else hipLaunchKernelGGL((merge_rows_kernel<1, D>), mgrid, dim3(kMergeRows * (D / 4)), 0, s, p, p.num_wgs);
    return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const RowAttnParams &p)
{
    const int mq = p.mq > 1 ? p.mq : 1;
    // paged caches need blocks of at least 16 tokens (a tile stays in one block)
    // bf16 at d = 128 or 64, or 1-byte codes (FP8 E4M3 or INT8) with row
    // scales at d = 128 (whose new rows the quantising append writes)
    const bool f8 = p.cache.elem_bytes == 1;
    return !p.prefill && !p.whole_items && (p.cache.elem_bytes == 2 || f8) &&
           (p.cache.d == 128 || (p.cache.d == 64 && !f8)) &&
           (p.k_new == nullptr || (mq == 1 && !f8)) &&
           mq * p.G <= MAX_ROWS && p.num_wgs <= kStreamWGs && (p.cache.block_table == nullptr || p.cache.log2_bs >= 4);
}

namespace {

template <int D>
hipError_t launch_decode_mfma_d(const RowAttnParams &p, hipStream_t stream)
{
    const int R = (p.mq > 1 ? p.mq : 1) * p.G;
    if (R <= 16) return launch_m<1, D>(p, stream);
    if (R <= 32) return launch_m<2, D>(p, stream);
    if (p.G % 2 == 0) {
        // more than 32 rows per KV head (the multi-query end): two items of
        // G / 2 heads each read the head's K/V (the second read mostly from
        // the caches) in the 32-row kernel; measured faster than one 64-row
        // item (and than four 16-row items, or two at two workgroups per CU)
        RowAttnParams q = p;
        q.kv_split = 2;
        q.G = p.G / 2;
        return launch_m<2, D>(q, stream);
    }
    return launch_m<4, D>(p, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const RowAttnParams &p, hipStream_t stream)
{
    if (!decode_mfma_supported(p)) return hipErrorInvalidValue;
    return p.cache.d == 64 ? launch_decode_mfma_d<64>(p, stream) : launch_decode_mfma_d<128>(p, stream);
}

}  // namespace gqa
