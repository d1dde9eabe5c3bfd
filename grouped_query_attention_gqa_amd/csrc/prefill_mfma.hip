// prefill_mfma.hip -- causal (or full) grouped-query attention of a block of
// new query tokens on the CDNA4 matrix cores, bf16 in, fp32 accumulate.
//
// What it computes ("Grouped-Query Attention" concept page, 技术原理 steps 2-4):
// out[b,i,h] = softmax(q[b,i,h] K_g^T * scale) V_g, g = h / G, over the keys
// visible to row i: keys 0 .. start_pos[b]+i when causal (a token attends to
// itself and to every earlier token, inference-optimisation page §5.1), keys
// 0 .. start_pos[b]+s-1 otherwise.  The new tokens' K/V are already in the
// cache (the append kernel runs first on the same stream).
//
// How (designed for gfx950, prior art only for the ideas):
//  * One workgroup owns a block of QB consecutive query positions of one
//    sequence and ALL G heads of one KV group g: 128*RBW rows (position,
//    head) that share every K/V tile, so each K/V tile is fetched once per
//    group (the group broadcast), and every row of the workgroup has the same
//    causal key range.
//  * Keys stream in 64-key tiles (the tile and the 16-token cache block
//    align, inference-optimisation page §9.4) through LDS; the tile for the
//    next step is loaded into registers while the current one is used.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K comes from LDS (rows XOR-swizzled over
//    16-byte chunks, so 16 lanes reading 16 keys hit 16 bank groups), Q^T
//    stays in registers for the whole key loop.  In the accumulator layout
//    each lane then owns one query row, so the row max and sum need a single
//    exchange with the lane 32 away.
//  * Online softmax in fp32 (inference-optimisation page §9.2.1), with the
//    running max only moved when a tile max exceeds it by 2^8 (exp2 units);
//    the probabilities are rounded to bf16 and used directly as the B operand
//    of O^T += V^T P^T -- the accumulator layout of S^T is already the operand
//    layout of P^T once both MFMAs use the same order of keys, so P never
//    leaves registers.  V is stored transposed in LDS (rows padded to 136 B so
//    32 lanes reading one key column hit distinct banks).
//  * Heaviest query blocks (largest causal key range) are launched first.
#include "common.h"
#include "kernels.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int NT = 256;
constexpr int BN = kKeyTile;   // keys per tile
constexpr float TAU = 8.0f;

__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D, int GP, int RBW>
struct PCfg {
    static constexpr int ROWS = 128 * RBW;        // (position, head) rows per workgroup
    static constexpr int QB = ROWS / GP;          // positions per workgroup
    static constexpr int CPR = D * 2 / 16;        // 16-byte chunks per K row
    static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
    static constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;             // 32-row blocks of O^T
    static constexpr int VT = BN + 4;             // V^T row stride (bf16 elements)
    static constexpr int LPT_K = BN * CPR / NT;   // K chunks per thread per tile
    static constexpr int NCK = D / 8;             // 8-element chunks per V row
    static constexpr int KPT_V = BN * NCK / NT;   // consecutive keys per thread for V
    static_assert(QB >= 1 && QB * GP == ROWS, "rows must split into positions x heads");
    static_assert(LPT_K >= 1 && KPT_V >= 2 && KPT_V <= 4, "tile split");
};

template <int D, int GP, int RBW>
__global__ __launch_bounds__(NT) void prefill_mfma_kernel(PrefillParams p)
{
    using C = PCfg<D, GP, RBW>;
    __shared__ uint4 Kl[BN * C::CPR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * C::VT];

    const CacheView &cache = p.cache;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nq = lane & 31, hh = lane >> 5;
    const int num_qb = (p.s + C::QB - 1) / C::QB;
    const int qb = num_qb - 1 - (int)blockIdx.x;   // heaviest first
    const int g = blockIdx.y, b = blockIdx.z;
    const int q0 = qb * C::QB;
    const int start = p.start_pos[b];
    const int G = p.G, H = p.H;
    const int kv_len = (int)min((int64_t)start + p.s, (int64_t)cache.capacity);
    const int kv_end = p.causal ? (int)min((int64_t)start + q0 + C::QB, (int64_t)kv_len) : kv_len;

    // ---- this lane's query rows and their Q^T fragments ---------------------
    int row_r[RBW], row_i[RBW];
    bool row_ok[RBW];
    uint4 qf[RBW][C::KS];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        const int rho = (wave * RBW + rb) * 32 + nq;
        row_r[rb] = rho / C::QB;
        row_i[rb] = q0 + rho % C::QB;
        row_ok[rb] = row_r[rb] < G && row_i[rb] < p.s;
        const uint4 *qrow = reinterpret_cast<const uint4 *>(
            p.q + ((((int64_t)b * p.s + (row_ok[rb] ? row_i[rb] : 0)) * H + (int64_t)g * G +
                    (row_ok[rb] ? row_r[rb] : 0)) * D) * 2);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            qf[rb][ks] = row_ok[rb] ? qrow[2 * ks + hh] : make_uint4(0, 0, 0, 0);
    }

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

    // ---- tile loads: global -> registers -----------------------------------
    uint4 kreg[C::LPT_K], vreg[C::KPT_V];
    const int v_c = tid % C::NCK, v_kq = tid / C::NCK;
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int li = 0; li < C::LPT_K; ++li) {
            const int pidx = tid + li * NT;
            const int key = pidx / C::CPR, ch = pidx % C::CPR;
            kreg[li] = make_uint4(0, 0, 0, 0);
            if (j0 + key < kv_len) {
                // a wave's 64 / CPR keys lie in one 16-key group of the tile
                const int64_t row = cache_row_wave(cache, b, g, j0 + key);
                if (row >= 0) kreg[li] = ld16(cache.k + row * (D * 2) + ch * 16);
            }
        }
#pragma unroll
        for (int k = 0; k < C::KPT_V; ++k) {
            const int key = v_kq * C::KPT_V + k;
            vreg[k] = make_uint4(0, 0, 0, 0);
            if (j0 + key < kv_len) {
                // a wave covers keys 16w .. 16w+15 of the tile
                const int64_t row = cache_row_wave(cache, b, g, j0 + key);
                if (row >= 0) vreg[k] = ld16(cache.v + row * (D * 2) + v_c * 16);
            }
        }
    };

    if (kv_end > 0) load_tile(0);
    for (int j0 = 0; j0 < kv_end; j0 += BN) {
        __syncthreads();   // everyone is done with the previous tile
#pragma unroll
        for (int li = 0; li < C::LPT_K; ++li) {
            const int pidx = tid + li * NT;
            const int key = pidx / C::CPR, ch = pidx % C::CPR;
            Kl[key * C::CPR + (ch ^ (key & C::SWZ))] = kreg[li];
        }
        {
            // V^T[d][key]: this thread holds keys v_kq*KPT_V .. +KPT_V-1 of columns 8*v_c .. 8*v_c+7
            const uint32_t *w[4];
#pragma unroll
            for (int k = 0; k < C::KPT_V; ++k) w[k] = reinterpret_cast<const uint32_t *>(&vreg[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t *dst = Vt + (8 * v_c + e) * C::VT + v_kq * C::KPT_V;
                if constexpr (C::KPT_V == 4) {
                    const uint32_t w0 = (e & 1) ? pair_hi(w[0][e >> 1], w[1][e >> 1]) : pair_lo(w[0][e >> 1], w[1][e >> 1]);
                    const uint32_t w1 = (e & 1) ? pair_hi(w[2][e >> 1], w[3][e >> 1]) : pair_lo(w[2][e >> 1], w[3][e >> 1]);
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(w0, w1);
                } else {
                    const uint32_t w0 = (e & 1) ? pair_hi(w[0][e >> 1], w[1][e >> 1]) : pair_lo(w[0][e >> 1], w[1][e >> 1]);
                    *reinterpret_cast<uint32_t *>(dst) = w0;
                }
            }
        }
        __syncthreads();
        if (j0 + BN < kv_end) load_tile(j0 + BN);

        const bool need_mask = (j0 + BN > kv_len) || (p.causal && j0 + BN - 1 > start + q0);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            // S^T = K Q^T for the two 32-key halves of the tile
            f32x16_t sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int key = kb * 32 + nq;
                    const uint4 a = Kl[key * C::CPR + ((2 * ks + hh) ^ (key & C::SWZ))];
                    sacc[kb] = mfma32x32x16(a, qf[rb][ks], sacc[kb]);
                }
            }
            // scale, mask, row max (lane pairs l, l^32 share a query row)
            const int qpos = start + row_i[rb];
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sacc[kb][i] * p.scale_log2;
                    if (need_mask) {
                        const int key = j0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
                        if (key >= kv_len || (p.causal && key > qpos)) x = -INFINITY;
                    }
                    sacc[kb][i] = x;
                    mt = fmaxf(mt, x);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
            float alpha = 1.f;
            if (mt > m_ref[rb] + TAU) {
                alpha = fast_exp2(m_ref[rb] - mt);
                m_ref[rb] = mt;
            }
            const float m_use = (m_ref[rb] == -INFINITY) ? 0.f : m_ref[rb];
            // probabilities -> bf16 operand pairs; the sum uses the rounded values
            uint4 pb[2][2];
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    uint32_t wv[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float p0 = fast_exp2(sacc[kb][half * 8 + 2 * j] - m_use);
                        const float p1 = fast_exp2(sacc[kb][half * 8 + 2 * j + 1] - m_use);
                        const uint32_t u = pack_bf16x2(p0, p1);
                        ps += __uint_as_float(u << 16) + __uint_as_float(u & 0xffff0000u);
                        wv[j] = u;
                    }
                    pb[kb][half] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                }
            ps += __shfl_xor(ps, 32, kWave);
            l_run[rb] = l_run[rb] * alpha + ps;
            if (alpha != 1.f) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[rb][db][i] *= alpha;
            }
            // O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const uint16_t *vrow = Vt + (db * 32 + nq) * C::VT;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int k0 = kb * 32 + half * 16 + hh * 4;
                        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + k0);
                        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + k0 + 8);
                        acc[rb][db] = mfma32x32x16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb[kb][half], acc[rb][db]);
                    }
            }
        }
    }

    // ---- normalise and store: lane owns 16 columns per 32-column block -----
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        if (!row_ok[rb]) continue;
        const float inv = l_run[rb] > 0.f ? 1.f / l_run[rb] : 0.f;
        uint16_t *orow = reinterpret_cast<uint16_t *>(p.out) +
                         (((int64_t)b * p.s + row_i[rb]) * H + (int64_t)g * G + row_r[rb]) * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = db * 32 + i4 * 8 + hh * 4;
                const uint2 v = make_uint2(pack_bf16x2(acc[rb][db][4 * i4 + 0] * inv, acc[rb][db][4 * i4 + 1] * inv),
                                           pack_bf16x2(acc[rb][db][4 * i4 + 2] * inv, acc[rb][db][4 * i4 + 3] * inv));
                *reinterpret_cast<uint2 *>(orow + d0) = v;
            }
    }
}

template <int D, int RBW>
hipError_t launch_gp(const PrefillParams &p, int gp, hipStream_t s)
{
    const int64_t rows = 128 * RBW;
    const int64_t qb_pos = rows / gp;
    const int64_t nqb = (p.s + qb_pos - 1) / qb_pos;
    if (nqb > 0x7fffffffLL || p.cache.K > 65535 || p.B > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nqb, (unsigned)p.cache.K, (unsigned)p.B);
    switch (gp) {
    case 1: hipLaunchKernelGGL((prefill_mfma_kernel<D, 1, RBW>), grid, dim3(NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<D, 2, RBW>), grid, dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<D, 4, RBW>), grid, dim3(NT), 0, s, p); break;
    case 8: hipLaunchKernelGGL((prefill_mfma_kernel<D, 8, RBW>), grid, dim3(NT), 0, s, p); break;
    case 16: hipLaunchKernelGGL((prefill_mfma_kernel<D, 16, RBW>), grid, dim3(NT), 0, s, p); break;
    case 32: hipLaunchKernelGGL((prefill_mfma_kernel<D, 32, RBW>), grid, dim3(NT), 0, s, p); break;
    case 64: hipLaunchKernelGGL((prefill_mfma_kernel<D, 64, RBW>), grid, dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams &p, hipStream_t stream)
{
    const int gp = pow2_at_least(p.G);
    if (p.cache.elem_bytes != 2) return hipErrorInvalidValue;
    if (p.cache.d == 128) return launch_gp<128, 1>(p, gp, stream);
    if (p.cache.d == 64) return launch_gp<64, 1>(p, gp, stream);
    return hipErrorInvalidValue;
}

}  // namespace gqa
