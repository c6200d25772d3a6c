// Attention forward for heads with very few query rows (decode shape:
// N <= 4 queries against a long key sequence), split over the keys, plus the
// merge of split partials that every split path shares.
//
// The work per key is tiny (N dot products of length d), so this path is
// bound by streaming K and V from HBM, not by arithmetic: it uses plain fp32
// VALU FMAs instead of MFMA (whose 32-wide query dimension would be >= 87%
// padding here) and spends its registers on keeping many 16-byte loads in
// flight.  K and V are read exactly once, so the loads are non-temporal (no
// cache allocation for data nobody reads again).
//
// Recurrence (per query row, per group of keys): running max m, running sum
// l, accumulator o~ rescaled by e^{m_old - m_new}: "从原始Softmax到在线Softmax"
// page, online softmax derivation.  Partial states over disjoint key sets are
// combined with the block merge of the same page (m = max, each side scaled by
// e^{m_side - m}); the split merge uses it in LSE form: with lse_s = m_s + log
// l_s, lse = log sum_s e^{lse_s} and o = sum_s e^{lse_s - lse} o_s.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace osa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int U = 8;  // key groups per wave per iteration (loads in flight)
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994531f;

// Element type traits: EPL elements per 16-byte load, widened to fp32.
template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
    static constexpr int EPL = 8;
    __device__ static void widen(const u32x4 &x, float *f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(x[i] << 16);
            f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
        }
    }
};
template <>
struct Elem<false> {
    static constexpr int EPL = 4;
    __device__ static void widen(const u32x4 &x, float *f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
    }
};

// Sum over aligned groups of LPK lanes (LPK a power of two <= 32).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <int D, bool BF16, int NQ, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void attn_decode_kernel(const void *__restrict__ qv, const void *__restrict__ kv,
                                                            const void *__restrict__ vv, float *__restrict__ part_o,
                                                            float *__restrict__ part_lse, int BH, int N, int M,
                                                            float c, float qsign, int splits, int keys_per_split,
                                                            const int32_t *__restrict__ kv_len, int H, int coff) {
    using E = Elem<BF16>;
    constexpr int EPL = E::EPL;
    constexpr int LPK = D / EPL;      // lanes per key row
    constexpr int KPW = 64 / LPK;     // keys per wave per load step
    constexpr int NG = NW * KPW;      // key groups per workgroup (independent partial states)
    constexpr int ESZ = BF16 ? 2 : 4; // bytes per element

    __shared__ float sm_m[NG][NQ];
    __shared__ float sm_l[NG][NQ];
    __shared__ float sm_o[NG][NQ][D];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane / LPK;         // key group within the wave
    const int e0 = (lane % LPK) * EPL; // first d index this lane covers

    const int bh = blockIdx.x % BH;
    const int sp = blockIdx.x / BH;
    const int kb = sp * keys_per_split;
    int ke = min(M, kb + keys_per_split);
    if (kv_len != nullptr) ke = min(ke, max(kv_len[bh / H], 0));

    const char *qh = static_cast<const char *>(qv) + (size_t)bh * N * D * ESZ;
    const char *kh = static_cast<const char *>(kv) + (size_t)bh * M * D * ESZ;
    const char *vh = static_cast<const char *>(vv) + (size_t)bh * M * D * ESZ;

    float qf[NQ][EPL];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (n < N) x = *reinterpret_cast<const u32x4 *>(qh + ((size_t)n * D + e0) * ESZ);
        E::widen(x, qf[n]);
#pragma unroll
        for (int i = 0; i < EPL; ++i) qf[n][i] *= qsign;
    }

    float m[NQ], l[NQ], acc[NQ][EPL];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        m[n] = NEG_INF;
        l[n] = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[n][i] = 0.f;
    }

    // Keys are visited in chunks of NW*KPW*U; inside a chunk wave w takes
    // KPW*U consecutive keys, key group g of the wave takes every KPW-th.
    constexpr int CHUNK = NW * KPW * U;
    for (int base = kb; base < ke; base += CHUNK) {
        u32x4 kr[U], vr[U];
        int key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            key[u] = base + wave * KPW * U + u * KPW + g;
            // past the range: reload the last valid key (masked below, weight exactly 0)
            const int kc = min(key[u], ke - 1);
            kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kh + ((size_t)kc * D + e0) * ESZ));
            vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vh + ((size_t)kc * D + e0) * ESZ));
        }
        float kf[U][EPL], vf[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            E::widen(kr[u], kf[u]);
            E::widen(vr[u], vf[u]);
        }
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            float s[U];
            float mx = NEG_INF;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < EPL; ++i) dot = __builtin_fmaf(qf[n][i], kf[u][i], dot);
                dot = group_sum<LPK>(dot);
                const bool ok = key[u] < ke && (!CAUSAL || key[u] <= n + coff);
                s[u] = ok ? dot * c : NEG_INF;
                mx = fmaxf(mx, s[u]);
            }
            const float m_new = fmaxf(m[n], mx);
            if (m_new == NEG_INF) continue;  // nothing visible yet for this row in this group
            const float alpha = __builtin_amdgcn_exp2f(m[n] - m_new);
            float p[U], psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = __builtin_amdgcn_exp2f(s[u] - m_new);
                psum += p[u];
            }
            l[n] = alpha * l[n] + psum;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                float a = acc[n][i] * alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) a = __builtin_fmaf(p[u], vf[u][i], a);
                acc[n][i] = a;
            }
            m[n] = m_new;
        }
    }

    // Combine the NG partial states of this workgroup through LDS.
    const int grp = wave * KPW + g;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        if (lane % LPK == 0) {
            sm_m[grp][n] = m[n];
            sm_l[grp][n] = l[n];
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) sm_o[grp][n][e0 + i] = acc[n][i];
    }
    __syncthreads();
    for (int idx = tid; idx < NQ * D; idx += NT) {
        const int n = idx / D, e = idx % D;
        if (n >= N) continue;
        float mm = NEG_INF;
        for (int t = 0; t < NG; ++t) mm = fmaxf(mm, sm_m[t][n]);
        float ll = 0.f, oo = 0.f;
        if (mm != NEG_INF) {
            for (int t = 0; t < NG; ++t) {
                const float w = __builtin_amdgcn_exp2f(sm_m[t][n] - mm);
                ll += w * sm_l[t][n];
                oo += w * sm_o[t][n][e];
            }
        }
        const size_t prow = ((size_t)sp * BH + bh) * N + n;
        part_o[prow * D + e] = ll > 0.f ? oo / ll : 0.f;
        if (e == 0) part_lse[prow] = ll > 0.f ? (mm + log2f(ll)) * LN2 : NEG_INF;
    }
}

// One wave per output row: merge the split partials.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void split_merge_kernel(const float *__restrict__ part_o,
                                                          const float *__restrict__ part_lse, void *__restrict__ o,
                                                          float *__restrict__ lse, int64_t rows, int splits) {
    constexpr int EPT = D / 64;  // elements per lane
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    float mx = NEG_INF;
    for (int s = 0; s < splits; ++s) mx = fmaxf(mx, part_lse[(size_t)s * rows + row]);
    float wsum = 0.f;
    float acc[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) acc[i] = 0.f;
    if (mx != NEG_INF) {
        for (int s = 0; s < splits; ++s) {
            const float ls = part_lse[(size_t)s * rows + row];
            const float w = expf(ls - mx);
            wsum += w;
            const float *po = part_o + ((size_t)s * rows + row) * D + lane * EPT;
#pragma unroll
            for (int i = 0; i < EPT; ++i) acc[i] = __builtin_fmaf(w, po[i], acc[i]);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if constexpr (BF16) {
        uint16_t *orow = static_cast<uint16_t *>(o) + (size_t)row * D + lane * EPT;
#pragma unroll
        for (int i = 0; i < EPT; ++i) orow[i] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i] * inv));
    } else {
        float *orow = static_cast<float *>(o) + (size_t)row * D + lane * EPT;
#pragma unroll
        for (int i = 0; i < EPT; ++i) orow[i] = acc[i] * inv;
    }
    if (lane == 0) lse[row] = wsum > 0.f ? mx + logf(wsum) : NEG_INF;
}

template <int D, bool BF16, int NQ, bool CAUSAL>
hipError_t launch_decode_t(const AttnProblem &p, hipStream_t stream) {
    const int keys_per_split = p.tiles_per_split * kDecodeKeyTile;
    hipLaunchKernelGGL((attn_decode_kernel<D, BF16, NQ, CAUSAL>), dim3((unsigned)((int64_t)p.BH * p.splits)),
                       dim3(NT), 0, stream, p.q, p.k, p.v, p.part_o, p.part_lse, p.BH, p.N, p.M, p.c,
                       p.negate_q ? -1.f : 1.f, p.splits, keys_per_split, p.kv_len, p.H, p.causal_off);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_decode_d(const AttnProblem &p, hipStream_t stream) {
    if (p.causal) {
        if (p.N == 1) return launch_decode_t<D, BF16, 1, true>(p, stream);
        if (p.N == 2) return launch_decode_t<D, BF16, 2, true>(p, stream);
        return launch_decode_t<D, BF16, 4, true>(p, stream);
    }
    if (p.N == 1) return launch_decode_t<D, BF16, 1, false>(p, stream);
    if (p.N == 2) return launch_decode_t<D, BF16, 2, false>(p, stream);
    return launch_decode_t<D, BF16, 4, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_decode(const AttnProblem &p, bool bf16, hipStream_t stream) {
    if (p.d == 64) return bf16 ? launch_decode_d<64, true>(p, stream) : launch_decode_d<64, false>(p, stream);
    return bf16 ? launch_decode_d<128, true>(p, stream) : launch_decode_d<128, false>(p, stream);
}

hipError_t launch_split_merge(const AttnProblem &p, bool bf16, hipStream_t stream) {
    const int64_t rows = (int64_t)p.BH * p.N;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (p.d == 64) {
        if (bf16)
            hipLaunchKernelGGL((split_merge_kernel<64, true>), grid, dim3(256), 0, stream, p.part_o, p.part_lse, p.o,
                               p.lse, rows, p.splits);
        else
            hipLaunchKernelGGL((split_merge_kernel<64, false>), grid, dim3(256), 0, stream, p.part_o, p.part_lse,
                               p.o, p.lse, rows, p.splits);
    } else {
        if (bf16)
            hipLaunchKernelGGL((split_merge_kernel<128, true>), grid, dim3(256), 0, stream, p.part_o, p.part_lse,
                               p.o, p.lse, rows, p.splits);
        else
            hipLaunchKernelGGL((split_merge_kernel<128, false>), grid, dim3(256), 0, stream, p.part_o, p.part_lse,
                               p.o, p.lse, rows, p.splits);
    }
    return hipGetLastError();
}

}  // namespace osa
