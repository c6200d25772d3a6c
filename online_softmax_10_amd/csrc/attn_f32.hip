// Fused attention forward with fp32 inputs, fp32 products and fp32
// accumulation throughout (v_mfma_f32_32x32x2_f32), for gfx950.
//
// Same recurrence as the bf16 kernel (running max m, running sum l,
// unnormalised accumulator rescaled by e^{m_old - m_new}, o = o~/l,
// LSE = m + log l): "从原始Softmax到在线Softmax" page, online softmax
// derivation; "Online Softmax and Flash Attention" page, eq. (8).
//
// Layout: a workgroup owns 128 query rows (four waves x 32); key tiles of 32
// keys go through LDS in natural row-major layout.  Scores are computed
// transposed (S^T = K Q^T) so a lane owns one query; the fp32 MFMA consumes
// one element per lane per operand, so the probabilities P^T feed the P.V
// product straight from the score accumulators (register u of the
// accumulator is key row 8*(u/4) + 4*half + u%4) and V is read at those rows.
// Probabilities stay fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace osa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int BR = 32 * NW;
constexpr int BC = kF32KeyTile;  // 32 keys per tile
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.4426950408889634f;

template <int D>
struct Layout {
    static constexpr int KS = D + 2;  // K row stride (floats): lanes read column 2*kk+half of 32 rows
    static constexpr int VS = D + 8;  // V row stride (floats): the two halves read rows 4 apart
    static constexpr int LOADS = BC * D / 4 / NT;  // float4 chunks per thread per tile (K and V each)
    static_assert(LOADS * NT * 4 == BC * D, "tile split");
};

__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT, 1) void attn_fwd_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ o, float *__restrict__ lse, float *__restrict__ part_o, float *__restrict__ part_lse,
    int BH, int N, int M, float c, float qsign, int ntq, int splits, int tiles_per_split,
    const int32_t *__restrict__ kv_len, int H, int coff, const float *__restrict__ bias, int64_t bias_sb,
    int64_t bias_sh, int64_t bias_sn) {
    using Lay = Layout<D>;
    __shared__ __attribute__((aligned(16))) float Ks[BC * Lay::KS];
    __shared__ __attribute__((aligned(16))) float Vs[BC * Lay::VS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    const int b = blockIdx.x;
    const int bh = b % BH;
    const int rest = b / BH;
    const int sp = rest % splits;
    const int qt = ntq - 1 - rest / splits;
    const int q0 = qt * BR;
    const int qrow = q0 + wave * 32 + l32;
    const int wq_lo = q0 + wave * 32;

    const int kb = sp * tiles_per_split * BC;
    int ke = min(M, kb + tiles_per_split * BC);
    if (kv_len != nullptr) ke = min(ke, max(kv_len[bh / H], 0));
    if (CAUSAL) ke = min(ke, q0 + BR + coff);
    const int ntiles = ke > kb ? (ke - kb + BC - 1) / BC : 0;

    // Additive bias: this lane's row (rows past N read row N - 1).  With a
    // bias the scores are brought to base-2 units (bias included) right after
    // the product and the rest runs with cs = 1.
    const bool has_bias = bias != nullptr;
    const float *brow = has_bias ? bias + (int64_t)(bh / H) * bias_sb + (int64_t)(bh % H) * bias_sh +
                                       (int64_t)min(qrow, N - 1) * bias_sn
                                 : nullptr;
    const float cs = has_bias ? 1.f : c;

    const float *qh = q + (size_t)bh * N * D;
    const float *kh = k + (size_t)bh * M * D;
    const float *vh = v + (size_t)bh * M * D;

    // Q^T operand: lane (query l32, half hh) holds q[qrow][2*kk + hh].
    float qop[D / 2];
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) qop[kk] = qrow < N ? qh[(size_t)qrow * D + 2 * kk + hh] * qsign : 0.f;

    f32x4 kreg[Lay::LOADS], vreg[Lay::LOADS];
    auto fetch = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < Lay::LOADS; ++i) {
            const int id = tid + i * NT;
            const int row = id / (D / 4), c4 = id % (D / 4);
            const int key = kv0 + row;
            const bool ok = key < ke;
            kreg[i] = ok ? *reinterpret_cast<const f32x4 *>(kh + (size_t)key * D + 4 * c4) : f32x4{};
            vreg[i] = ok ? *reinterpret_cast<const f32x4 *>(vh + (size_t)key * D + 4 * c4) : f32x4{};
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < Lay::LOADS; ++i) {
            const int id = tid + i * NT;
            const int row = id / (D / 4), c4 = id % (D / 4);
            // K rows are padded by 2 floats, so 16-byte alignment is not guaranteed: store as float2.
            float *kd = &Ks[row * Lay::KS + 4 * c4];
            kd[0] = kreg[i][0];
            kd[1] = kreg[i][1];
            kd[2] = kreg[i][2];
            kd[3] = kreg[i][3];
            *reinterpret_cast<f32x4 *>(&Vs[row * Lay::VS + 4 * c4]) = vreg[i];
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = NEG_INF;
    float l_run = 0.f;

    if (ntiles > 0) fetch(kb);
    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = kb + t * BC;
        __syncthreads();
        stash();
        __syncthreads();
        if (t + 1 < ntiles) fetch(kv0 + BC);
        if (CAUSAL && kv0 > wq_lo + 31 + coff) continue;

        // Bias of this lane's scores (register r: key kv0 + 8*(r/4) + 4*hh + r%4),
        // fetched before the product so the loads overlap it; keys past M read 0.
        f32x4 bv[4];
        if (has_bias) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int key = kv0 + 8 * g + 4 * hh;
                if (key + 4 <= M) {
                    bv[g] = *reinterpret_cast<const f32x4 *>(brow + key);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[g][e] = key + e < M ? brow[key + e] : 0.f;
                }
            }
        }
        f32x16 s = f32x16{};
        const float *krow = &Ks[l32 * Lay::KS + hh];
#pragma unroll
        for (int kk = 0; kk < D / 2; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * kk], qop[kk], s, 0, 0, 0);
        if (has_bias) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], c, bv[r >> 2][r & 3] * LOG2E);
        }

        // Register r holds key kv0 + 8*(r/4) + 4*hh + r%4.
        const bool need_mask = (kv0 + BC > ke) || (CAUSAL && kv0 + BC - 1 > wq_lo + coff);
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool ok = key < ke && (!CAUSAL || key <= qrow + coff);
                s[r] = ok ? s[r] : NEG_INF;
            }
        }
        float mx = NEG_INF;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = xhalf_max(mx);
        const float m_tile = mx == NEG_INF ? NEG_INF : mx * cs;
        const float m_new = fmaxf(m_run, m_tile);
        const float m_use = m_new == NEG_INF ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], cs, -m_use));
            if (need_mask) e = s[r] == NEG_INF ? 0.f : e;
            s[r] = e;
            lsum += e;
        }
        l_run = alpha * l_run + lsum;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int row = 8 * (u >> 2) + 4 * hh + (u & 3);
                const float va = Vs[row * Lay::VS + 32 * db + l32];
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[u], oacc[db], 0, 0, 0);
            }
        }
    }

    const float l_tot = xhalf_sum(l_run);
    if (qrow >= N) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float row_lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * LN2 : NEG_INF;
    float *orow;
    if constexpr (!SPLIT) {
        orow = o + ((size_t)bh * N + qrow) * D;
        if (hh == 0) lse[(size_t)bh * N + qrow] = row_lse;
    } else {
        const size_t prow = ((size_t)sp * BH + bh) * N + qrow;
        orow = part_o + prow * D;
        if (hh == 0) part_lse[prow] = row_lse;
    }
    // O^T register r of block db holds d index 32*db + 8*(r/4) + 4*hh + r%4.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                       oacc[db][4 * g + 3] * inv};
            *reinterpret_cast<f32x4 *>(orow + 32 * db + 8 * g + 4 * hh) = x;
        }
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_t(const AttnProblem &p, hipStream_t stream) {
    const int ntq = (p.N + BR - 1) / BR;
    const int64_t blocks = (int64_t)p.BH * ntq * p.splits;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL, SPLIT>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       static_cast<const float *>(p.q), static_cast<const float *>(p.k),
                       static_cast<const float *>(p.v), static_cast<float *>(p.o), p.lse, p.part_o, p.part_lse,
                       p.BH, p.N, p.M, p.c, p.negate_q ? -1.f : 1.f, ntq, p.splits, p.tiles_per_split, p.kv_len,
                       p.H, p.causal_off, p.bias, p.bias_sb, p.bias_sh, p.bias_sn);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnProblem &p, hipStream_t stream) {
    const bool split = p.splits > 1;
    if (p.causal) return split ? launch_t<D, true, true>(p, stream) : launch_t<D, true, false>(p, stream);
    return split ? launch_t<D, false, true>(p, stream) : launch_t<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_f32(const AttnProblem &p, hipStream_t stream) {
    return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace osa
