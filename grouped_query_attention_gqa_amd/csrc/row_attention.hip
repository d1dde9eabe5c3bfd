// row_attention.hip -- grouped-query attention of single query rows on the
// vector ALUs: the decode step (memory-bound) and the fp32 prefill.
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps 2-4):
// for every query row and every KV group g, the G query heads g*G .. g*G+G-1
// attend to K/V head g with softmax(q K_g^T * scale) V_g over the row's
// visible keys.
//
// How (a design for CDNA4, not a port):
//  * One workgroup = one (query row, KV group, key split).  The keys of a
//    row are cut into splits of `split` keys (flash-decoding, inference-
//    optimisation page §10.2, parallel over batch x head as in §10.3); each
//    split keeps an online-softmax state (m, l, o) per head (same page
//    §9.2.1) and the splits are merged with their global max and sum.
//  * The split's keys stream through LDS in 64-key tiles.  Every K and V row
//    is read from HBM once, with coalesced 16-byte loads, and is then used by
//    all G heads of the group from LDS (the group broadcast the concept page
//    names under 上游 for FlashAttention's GQA support).
//  * Scores: thread (head r, key t) computes the full dot product of its
//    register-resident q row with the K row from LDS (v_dot2_f32_bf16: two
//    bf16 products per instruction into fp32).  K rows are XOR-swizzled in LDS
//    so that 16 lanes reading 16 different rows hit 16 different bank groups.
//  * Weighted V sum: thread (key group, column piece, head set) holds
//    fp32 accumulators for up to 8 heads x 8 columns; two keys at a time are
//    paired (v_perm) so that one v_dot2 adds p_t v_t + p_t+1 v_t+1.  The
//    key groups are reduced with lane shuffles and one LDS pass at the end.
//  * The running maximum is only moved when a tile's maximum exceeds it by
//    more than 2^8 (in exp2 units), so the accumulators are rescaled rarely;
//    exp2 of a score minus any reference <= the true max is exact algebra,
//    the final o / l cancels the reference.
//  * A row whose keys fit one split is normalised and stored by its single
//    workgroup; otherwise every split stores (m, l, o) in the workspace and a
//    small second kernel merges them (a kernel boundary orders the stores
//    without any cache-flushing fence inside the hot kernel).
#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

constexpr int NT = 256;      // threads per workgroup (4 waves)
constexpr int TT = kKeyTile; // keys per tile
constexpr float TAU = 8.0f;  // lazy-rescale threshold (log2 units)

template <int D, int GP, bool BF16>
struct Cfg {
    static constexpr int ES = BF16 ? 2 : 4;          // element bytes
    static constexpr int RB = D * ES;                // row bytes
    static constexpr int CPR = RB / 16;              // 16-byte pieces per row
    static constexpr int CE = 16 / ES;               // elements per piece
    static constexpr int LPT = TT * CPR / NT;        // pieces per thread per tile (each of K, V)
    static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
    // score phase
    static constexpr int TPH = (NT / GP) < kWave ? (NT / GP) : kWave;  // threads per head
    static constexpr int NS = TT / TPH;              // keys per score thread
    static constexpr int S_THREADS = GP * TPH;
    static constexpr int QW = RB / 4;                // 32-bit words of a q row
    // weighted-sum phase
    static constexpr int NC = CPR;                   // column pieces
    static constexpr int HPT = GP < 8 ? GP : 8;      // heads per thread
    static constexpr int HG = GP / HPT;              // head sets
    static constexpr int TG = NT / (NC * HG);        // key groups
    static constexpr int TPT = TT / TG;              // keys per thread per tile
    static constexpr int LANE_TG = TG < (kWave / NC) ? TG : (kWave / NC);
    static constexpr int WAVE_TG = TG / LANE_TG;
    // LDS
    static constexpr int KV_BYTES = TT * RB;
    static constexpr int P_BYTES = TT * GP * (BF16 ? 2 : 4);
    static constexpr int RED_BYTES = WAVE_TG * GP * D * 4;

    static_assert(LPT >= 1 && TT * CPR % NT == 0, "tile does not split over the threads");
    static_assert(TG >= 1 && NC * HG * TG == NT, "weighted-sum layout does not cover the threads");
    static_assert(!BF16 || TPT % 2 == 0, "key pairs need an even key count per thread");
    static_assert(RED_BYTES <= 2 * KV_BYTES, "reduction buffer does not fit the tile buffers");
    static_assert(NS * TPH == TT, "score layout does not cover the tile");
};

struct RowCtx {
    int64_t rowseq;   // b * Sq + i
    int b;
    int n_vis;        // visible keys of this row (already clamped to the capacity)
};

__device__ __forceinline__ RowCtx row_context(const RowAttnParams &p, int64_t rowseq)
{
    RowCtx r;
    r.rowseq = rowseq;
    r.b = (int)(rowseq / p.Sq);
    const int i = (int)(rowseq % p.Sq);
    int64_t n;
    if (!p.prefill) {
        n = p.ctx_lens[r.b];
    } else {
        const int64_t start = p.start_pos[r.b];
        n = p.causal ? start + i + 1 : start + p.Sq;
    }
    if (n > p.cache.capacity) n = p.cache.capacity;
    if (n > (int64_t)p.split * p.max_splits) n = (int64_t)p.split * p.max_splits;
    if (n < 0) n = 0;
    r.n_vis = (int)n;
    return r;
}

template <int D, int GP, bool BF16>
__global__ __launch_bounds__(NT) void row_attention_kernel(RowAttnParams p)
{
    using C = Cfg<D, GP, BF16>;
    __shared__ __attribute__((aligned(16))) char lds_kv[2 * C::KV_BYTES];
    __shared__ __attribute__((aligned(16))) char lds_p[C::P_BYTES];
    __shared__ float lds_alpha[GP];
    __shared__ float lds_m[GP];
    __shared__ float lds_l[GP];

    uint4 *Ks = reinterpret_cast<uint4 *>(lds_kv);
    uint4 *Vs = reinterpret_cast<uint4 *>(lds_kv + C::KV_BYTES);

    const int tid = threadIdx.x;
    const int split_idx = blockIdx.x;
    const int g = blockIdx.y;
    const RowCtx rc = row_context(p, blockIdx.z);
    const CacheView &cache = p.cache;
    const int K = cache.K;
    const int G = p.G;
    const int H = p.H;

    const int n_splits = (rc.n_vis + p.split - 1) / p.split;
    if (rc.n_vis <= 0) {
        // no visible key: an all-zero output row (documented contract)
        if (split_idx == 0) {
            for (int idx = tid; idx < G * D; idx += NT) {
                const int r = idx / D, col = idx % D;
                const int64_t o = (rc.rowseq * H + (int64_t)g * G + r) * D + col;
                if (BF16) reinterpret_cast<uint16_t *>(p.out)[o] = 0;
                else reinterpret_cast<float *>(p.out)[o] = 0.f;
            }
        }
        return;
    }
    if (split_idx >= n_splits) return;
    const int key0 = split_idx * p.split;
    const int key1 = min(key0 + p.split, rc.n_vis);

    // ---- score-thread state: q row of head r in registers -----------------
    const bool s_thread = tid < C::S_THREADS;
    const int s_r = tid / C::TPH;          // head (within the padded group)
    const int s_j = tid % C::TPH;
    uint32_t qw[C::QW];
    {
        const bool real = s_thread && s_r < G;
        const uint4 *qrow = reinterpret_cast<const uint4 *>(
            p.q + ((rc.rowseq * H + (int64_t)g * G + (real ? s_r : 0)) * D) * C::ES);
#pragma unroll
        for (int w = 0; w < C::QW / 4; ++w) {
            uint4 x = real ? qrow[w] : make_uint4(0, 0, 0, 0);
            qw[4 * w + 0] = x.x; qw[4 * w + 1] = x.y; qw[4 * w + 2] = x.z; qw[4 * w + 3] = x.w;
        }
    }
    float m_ref = -INFINITY;   // reference maximum (log2 units), uniform per head
    float l_run = 0.f;

    // ---- weighted-sum-thread state ----------------------------------------
    const int v_c = tid % C::NC;
    const int v_rest = tid / C::NC;
    const int v_tg = v_rest % C::TG;
    const int v_hg = v_rest / C::TG;
    float acc[C::HPT][C::CE];
#pragma unroll
    for (int i = 0; i < C::HPT; ++i)
#pragma unroll
        for (int e = 0; e < C::CE; ++e) acc[i][e] = 0.f;

    // ---- tile loads: global -> registers ----------------------------------
    uint4 kreg[C::LPT], vreg[C::LPT];
    auto load_tile = [&](int tile0) {
        const int nvalid = min(TT, key1 - tile0);
#pragma unroll
        for (int li = 0; li < C::LPT; ++li) {
            const int pidx = tid + li * NT;
            const int t = pidx / C::CPR, pc = pidx % C::CPR;
            kreg[li] = make_uint4(0, 0, 0, 0);
            vreg[li] = make_uint4(0, 0, 0, 0);
            if (t < nvalid) {
                // a wave's 64 / CPR rows lie in one 16-row group of the tile
                const int64_t row = cache_row_wave(cache, rc.b, g, tile0 + t);
                if (row >= 0) {
                    const int64_t off = row * C::RB + pc * 16;
                    kreg[li] = ld16(cache.k + off);
                    vreg[li] = ld16(cache.v + off);
                }
            }
        }
    };

    load_tile(key0);
    for (int tile0 = key0; tile0 < key1; tile0 += TT) {
        const int nvalid = min(TT, key1 - tile0);
        __syncthreads();   // previous tile fully consumed
#pragma unroll
        for (int li = 0; li < C::LPT; ++li) {
            const int pidx = tid + li * NT;
            const int t = pidx / C::CPR, pc = pidx % C::CPR;
            Ks[t * C::CPR + (pc ^ (t & C::SWZ))] = kreg[li];
            Vs[t * C::CPR + pc] = vreg[li];
        }
        __syncthreads();
        if (tile0 + TT < key1) load_tile(tile0 + TT);   // overlaps the compute below

        // ---- scores and online softmax (score threads) ---------------------
        if (s_thread) {
            float s[C::NS];
            float mt = -INFINITY;
#pragma unroll
            for (int k = 0; k < C::NS; ++k) {
                const int t = s_j + k * C::TPH;
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int pc = 0; pc < C::CPR; ++pc) {
                    const uint4 kv = Ks[t * C::CPR + (pc ^ (t & C::SWZ))];
                    if constexpr (BF16) {
                        a0 = dot2_bf16(qw[4 * pc + 0], kv.x, a0);
                        a1 = dot2_bf16(qw[4 * pc + 1], kv.y, a1);
                        a0 = dot2_bf16(qw[4 * pc + 2], kv.z, a0);
                        a1 = dot2_bf16(qw[4 * pc + 3], kv.w, a1);
                    } else {
                        a0 = fmaf(__uint_as_float(qw[4 * pc + 0]), __uint_as_float(kv.x), a0);
                        a1 = fmaf(__uint_as_float(qw[4 * pc + 1]), __uint_as_float(kv.y), a1);
                        a0 = fmaf(__uint_as_float(qw[4 * pc + 2]), __uint_as_float(kv.z), a0);
                        a1 = fmaf(__uint_as_float(qw[4 * pc + 3]), __uint_as_float(kv.w), a1);
                    }
                }
                s[k] = (t < nvalid) ? (a0 + a1) * p.scale_log2 : -INFINITY;
                mt = fmaxf(mt, s[k]);
            }
            mt = group_max<C::TPH>(mt);
            float alpha = 1.f;
            if (mt > m_ref + TAU) {
                alpha = fast_exp2(m_ref - mt);   // 0 on the first tile
                m_ref = mt;
            }
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < C::NS; ++k) {
                const int t = s_j + k * C::TPH;
                const float pk = fast_exp2(s[k] - m_ref);
                if constexpr (BF16) {
                    const uint32_t pb = f32_to_bf16_rne(pk);
                    ps += __uint_as_float(pb << 16);   // sum what the V product uses
                    reinterpret_cast<uint16_t *>(lds_p)[((t >> 1) * GP + s_r) * 2 + (t & 1)] = (uint16_t)pb;
                } else {
                    ps += pk;
                    reinterpret_cast<float *>(lds_p)[t * GP + s_r] = pk;
                }
            }
            ps = group_sum<C::TPH>(ps);
            l_run = l_run * alpha + ps;
            if (s_j == 0) lds_alpha[s_r] = alpha;
        }
        __syncthreads();

        // ---- o = o * alpha + sum_t p_t v_t (weighted-sum threads) ----------
        {
            float al[C::HPT];
            bool any = false;
#pragma unroll
            for (int i = 0; i < C::HPT; ++i) {
                al[i] = lds_alpha[v_hg * C::HPT + i];
                any |= (al[i] != 1.f);
            }
            if (any) {
#pragma unroll
                for (int i = 0; i < C::HPT; ++i)
#pragma unroll
                    for (int e = 0; e < C::CE; ++e) acc[i][e] *= al[i];
            }
            if constexpr (BF16) {
                const uint32_t *P2 = reinterpret_cast<const uint32_t *>(lds_p);
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
                const float *Pf = reinterpret_cast<const float *>(lds_p);
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
        }
    }

    // ---- reduce the key groups: lane shuffles, then one LDS pass -----------
#pragma unroll
    for (int m = C::NC; m < C::NC * C::LANE_TG; m <<= 1)
#pragma unroll
        for (int i = 0; i < C::HPT; ++i)
#pragma unroll
            for (int e = 0; e < C::CE; ++e) acc[i][e] += __shfl_xor(acc[i][e], m, kWave);
    __syncthreads();   // the tile buffers become the reduction buffer
    float *red = reinterpret_cast<float *>(lds_kv);
    if (v_tg % C::LANE_TG == 0) {
        const int w = v_tg / C::LANE_TG;
#pragma unroll
        for (int i = 0; i < C::HPT; ++i)
#pragma unroll
            for (int e = 0; e < C::CE; ++e)
                red[(w * GP + v_hg * C::HPT + i) * D + v_c * C::CE + e] = acc[i][e];
    }
    if (s_thread && s_j == 0) {
        lds_m[s_r] = m_ref;
        lds_l[s_r] = l_run;
    }
    __syncthreads();

    // ---- single split: normalise and store ---------------------------------
    if (n_splits == 1) {
        for (int idx = tid; idx < G * D / 2; idx += NT) {
            const int r = (2 * idx) / D, col = (2 * idx) % D;
            float o0 = 0.f, o1 = 0.f;
#pragma unroll
            for (int w = 0; w < C::WAVE_TG; ++w) {
                o0 += red[(w * GP + r) * D + col];
                o1 += red[(w * GP + r) * D + col + 1];
            }
            const float inv = 1.f / lds_l[r];
            const int64_t o = (rc.rowseq * H + (int64_t)g * G + r) * D + col;
            if constexpr (BF16)
                reinterpret_cast<uint32_t *>(p.out)[o / 2] = pack_bf16x2(o0 * inv, o1 * inv);
            else
                *reinterpret_cast<float2 *>(reinterpret_cast<float *>(p.out) + o) = make_float2(o0 * inv, o1 * inv);
        }
        return;
    }

    // ---- several splits: publish the partial state; the merge kernel below
    // combines them once every split of the launch has finished -------------
    const int64_t head0 = rc.rowseq * H + (int64_t)g * G;
    for (int idx = tid; idx < G * D; idx += NT) {
        const int r = idx / D, col = idx % D;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < C::WAVE_TG; ++w) o += red[(w * GP + r) * D + col];
        p.ws_o[((head0 + r) * p.max_splits + split_idx) * D + col] = o;
    }
    if (tid < G) {
        p.ws_ml[((head0 + tid) * p.max_splits + split_idx) * 2 + 0] = lds_m[tid];
        p.ws_ml[((head0 + tid) * p.max_splits + split_idx) * 2 + 1] = lds_l[tid];
    }
}

// Merge of the split partials of one (row, KV group) with their global max
// and sum: M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// out = sum_s o_s 2^(m_s - M) / L (m in log2 units).  Rows that fit one split
// were finished by the split kernel and are skipped.
template <int D, bool BF16>
__global__ __launch_bounds__(NT) void merge_splits_kernel(RowAttnParams p)
{
    const int g = blockIdx.x;
    const RowCtx rc = row_context(p, blockIdx.y);
    const int n_splits = (rc.n_vis + p.split - 1) / p.split;
    if (n_splits <= 1) return;
    const int G = p.G;
    const int64_t head0 = rc.rowseq * p.H + (int64_t)g * G;
    for (int idx = threadIdx.x; idx < G * D / 4; idx += NT) {
        const int r = (4 * idx) / D, col = (4 * idx) % D;
        const float *ml = p.ws_ml + (head0 + r) * p.max_splits * 2;
        float M = -INFINITY;
        for (int sp = 0; sp < n_splits; ++sp) M = fmaxf(M, ml[2 * sp]);
        float L = 0.f;
        float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < n_splits; ++sp) {
            const float w = fast_exp2(ml[2 * sp] - M);
            L += ml[2 * sp + 1] * w;
            const float4 os = *reinterpret_cast<const float4 *>(p.ws_o + ((head0 + r) * p.max_splits + sp) * D + col);
            O.x += os.x * w;
            O.y += os.y * w;
            O.z += os.z * w;
            O.w += os.w * w;
        }
        const float inv = 1.f / L;
        const int64_t o = (head0 + r) * D + col;
        if constexpr (BF16) {
            uint2 packed = make_uint2(pack_bf16x2(O.x * inv, O.y * inv), pack_bf16x2(O.z * inv, O.w * inv));
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.out) + o) = packed;
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.out) + o) =
                make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
        }
    }
}

template <int D, bool BF16>
hipError_t launch_d(const RowAttnParams &p, int gp, dim3 grid, hipStream_t s)
{
    switch (gp) {
    case 1: hipLaunchKernelGGL((row_attention_kernel<D, 1, BF16>), grid, dim3(NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((row_attention_kernel<D, 2, BF16>), grid, dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((row_attention_kernel<D, 4, BF16>), grid, dim3(NT), 0, s, p); break;
    case 8: hipLaunchKernelGGL((row_attention_kernel<D, 8, BF16>), grid, dim3(NT), 0, s, p); break;
    case 16: hipLaunchKernelGGL((row_attention_kernel<D, 16, BF16>), grid, dim3(NT), 0, s, p); break;
    case 32: hipLaunchKernelGGL((row_attention_kernel<D, 32, BF16>), grid, dim3(NT), 0, s, p); break;
    case 64: hipLaunchKernelGGL((row_attention_kernel<D, 64, BF16>), grid, dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.max_splits <= 1) return e;
    hipLaunchKernelGGL((merge_splits_kernel<D, BF16>), dim3(grid.y, grid.z), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_row_attention(const RowAttnParams &p, int gp, hipStream_t stream)
{
    const int64_t rows = (int64_t)p.B * p.Sq;
    if (rows <= 0) return hipSuccess;
    if (rows > 65535 || p.max_splits > 0x7fffffff || p.cache.K > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.max_splits, (unsigned)p.cache.K, (unsigned)rows);
    const bool bf16 = p.cache.elem_bytes == 2;
    if (p.cache.d == 128) return bf16 ? launch_d<128, true>(p, gp, grid, stream) : launch_d<128, false>(p, gp, grid, stream);
    if (p.cache.d == 64) return bf16 ? launch_d<64, true>(p, gp, grid, stream) : launch_d<64, false>(p, gp, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gqa
