// Fused attention forward, bf16 inputs, fp32 accumulation, for gfx950 (CDNA4).
//
// Method: exact attention softmax(Q K^T * scale) V computed with the online
// softmax recurrence -- per query row a running max m and running exponential
// sum l; each new key block rescales l and the unnormalised accumulator o~ by
// e^{m_old - m_new} and adds the block's terms; finally o = o~ / l and
// LSE = m + log l.  Sources: "从原始Softmax到在线Softmax" page, online softmax
// derivation (m, l, o~ recurrences) and LSE definition; "Online Softmax and
// Flash Attention" page, eq. (8) and the fused loop of eq. (20)-(22); the
// "Softmax与Flash-Attention" page's FlashAttention core idea (tiles of Q, K, V
// stay on chip, S and P never reach HBM; queries outer, keys inner).
//
// Mapping to the chip (all of it specific to this design, not the pages'):
//  * A workgroup owns BR = 128 query rows of one (batch, head): four 64-wide
//    waves, 32 rows each.  A wave keeps its 32 query rows in VGPRs as the B
//    operand of v_mfma_f32_32x32x16_bf16 for the whole key loop.
//  * Key tiles of BC = 64 keys stream through LDS: K row-major, V transposed
//    (d-major) so both MFMA operands are single 16-byte LDS reads.  The next
//    tile is fetched from HBM into registers while the current one is used.
//  * Scores are computed transposed, S^T = K Q^T, so each lane owns one query
//    (column) and 16 keys per 32x32 block: the row max and row sum are
//    in-lane plus one exchange between the two wave halves
//    (v_permlane32_swap).  The K rows fed to the MFMA are permuted (bits 2
//    and 3 of the row index swapped) so that the accumulator registers that
//    form the next MFMA's B operand hold 8 consecutive keys: P^T goes from
//    accumulators to bf16 operand registers with no data movement.
//  * O^T = V^T P^T keeps one query per lane again, so the per-row rescale
//    e^{m_old - m_new} and the final 1/l are per-lane scalars.
//  * Scores stay in base-2 units: c = |scale| * log2(e) is folded into one
//    FMA before v_exp_f32; a negative scale flips q's sign bit on load.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace osa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;            // waves per workgroup
constexpr int NT = 64 * NW;      // threads per workgroup
constexpr int BR = 32 * NW;      // query rows per workgroup
constexpr int BC = kBf16KeyTile; // keys per tile
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994531f;
constexpr float RESCALE_SLACK = 8.f;  // base-2 units: probabilities stay below 2^8

template <int D>
struct Layout {
    static constexpr int KS = D + 8;                 // K row stride in LDS (bf16)
    static constexpr int VS = BC + 8;                // V^T row stride in LDS (bf16)
    static constexpr int K_LOADS = BC * D / 8 / NT;  // 16-byte K chunks per thread
    static constexpr int V_KPT = BC * D / 8 / NT;    // keys per thread in the V transpose
    static constexpr int V_GROUPS = BC / V_KPT;      // key groups across threads
    static constexpr int LDS_BYTES = (BC * KS + D * VS) * 2;
    static_assert(K_LOADS * NT * 8 == BC * D, "K tile split");
    static_assert(V_KPT == 2 || V_KPT == 4, "V transpose width");
};

// Row r of a 32-row MFMA A operand reads K row perm32(r): bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Reduce across the two 32-lane halves of the wave.
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Low (sel=0) or high (sel=1) bf16 halves of a and b packed as (a_half | b_half << 16).
__device__ __forceinline__ uint32_t pack_halves(uint32_t a, uint32_t b, int sel) {
    return __builtin_amdgcn_perm(b, a, sel ? 0x07060302u : 0x05040100u);
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ part_o,
    float *__restrict__ part_lse, int BH, int N, int M, float c, uint32_t qsign, int ntq,
    int splits, int tiles_per_split) {
    using Lay = Layout<D>;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * Lay::KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * Lay::VS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, keeps tile skips scalar
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // Workgroup -> (head, split, query tile); heads vary fastest so that
    // consecutive workgroups share no K/V and the longest causal tiles go first.
    const int b = blockIdx.x;
    const int bh = b % BH;
    const int rest = b / BH;
    const int sp = rest % splits;
    const int qt = ntq - 1 - rest / splits;
    const int q0 = qt * BR;
    const int qrow = q0 + wave * 32 + l32;  // this lane's query row
    const int wq_lo = q0 + wave * 32;

    const int kb = sp * tiles_per_split * BC;
    int ke = min(M, kb + tiles_per_split * BC);
    if (CAUSAL) ke = min(ke, q0 + BR);
    const int ntiles = ke > kb ? (ke - kb + BC - 1) / BC : 0;

    const uint16_t *qh = q + (size_t)bh * N * D;
    const uint16_t *kh = k + (size_t)bh * M * D;
    const uint16_t *vh = v + (size_t)bh * M * D;

    // Q^T operands: lane (query l32, half hh) holds q[qrow][16*kk + 8*hh .. +8].
    bf16x8 qop[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < N) {
            x = *reinterpret_cast<const u32x4 *>(qh + (size_t)qrow * D + 16 * kk + 8 * hh);
            x ^= qsign;
        }
        qop[kk] = __builtin_bit_cast(bf16x8, x);
    }

    // Register staging for the next K/V tile.
    u32x4 kreg[Lay::K_LOADS];
    u32x4 vreg[Lay::V_KPT];
    const int v_kg = tid % Lay::V_GROUPS;  // key group (V_KPT keys) of this thread
    const int v_c8 = tid / Lay::V_GROUPS;  // 8-wide d chunk of this thread

    // Keys past the end of the range are clamped to the last valid key: their
    // scores are masked to -inf and their probabilities are exactly 0, so the
    // (finite) duplicated rows contribute nothing, and the loads need no branch.
    auto fetch = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < Lay::K_LOADS; ++i) {
            const int id = tid + i * NT;
            const int row = id / (D / 8), c8 = id % (D / 8);
            const int key = min(kv0 + row, ke - 1);
            kreg[i] = *reinterpret_cast<const u32x4 *>(kh + (size_t)key * D + c8 * 8);
        }
#pragma unroll
        for (int i = 0; i < Lay::V_KPT; ++i) {
            const int key = min(kv0 + Lay::V_KPT * v_kg + i, ke - 1);
            vreg[i] = *reinterpret_cast<const u32x4 *>(vh + (size_t)key * D + v_c8 * 8);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < Lay::K_LOADS; ++i) {
            const int id = tid + i * NT;
            const int row = id / (D / 8), c8 = id % (D / 8);
            *reinterpret_cast<u32x4 *>(&Ks[row * Lay::KS + c8 * 8]) = kreg[i];
        }
        // Transpose V_KPT keys x 8 d-values into 8 rows of V^T.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int dv = v_c8 * 8 + j;
            if constexpr (Lay::V_KPT == 4) {
                u32x2 w;
                w[0] = pack_halves(vreg[0][j >> 1], vreg[1][j >> 1], j & 1);
                w[1] = pack_halves(vreg[2][j >> 1], vreg[3][j >> 1], j & 1);
                *reinterpret_cast<u32x2 *>(&Vt[dv * Lay::VS + 4 * v_kg]) = w;
            } else {
                *reinterpret_cast<uint32_t *>(&Vt[dv * Lay::VS + 2 * v_kg]) =
                    pack_halves(vreg[0][j >> 1], vreg[1][j >> 1], j & 1);
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = NEG_INF;  // running max, base-2 units
    float l_run = 0.f;      // this lane's share of the running sum

    if (ntiles > 0) fetch(kb);
    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = kb + t * BC;
        __syncthreads();  // previous tile fully consumed
        stash();
        __syncthreads();
        if (t + 1 < ntiles) fetch(kv0 + BC);

        // (A wave whose rows all precede the tile still runs it fully masked:
        // the workgroup waits at the next barrier anyway, and a skip branch
        // here makes the compiler copy the accumulators every tile.)

        // S^T = K Q^T for two 32-key blocks.
        f32x16 s[2] = {f32x16{}, f32x16{}};
        const uint16_t *krow = &Ks[perm32(l32) * Lay::KS + 8 * hh];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(krow + 32 * cb * Lay::KS + 16 * kk);
                s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], s[cb], 0, 0, 0);
            }

        // Accumulator register r of block cb holds key kv0 + 32*cb + 16*(r/8) + 8*hh + r%8.
        const bool need_mask = (kv0 + BC > ke) || (CAUSAL && kv0 + BC - 1 > wq_lo);
        if (need_mask) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * cb + 16 * (r >> 3) + 8 * hh + (r & 7);
                    const bool ok = key < ke && (!CAUSAL || key <= qrow);
                    s[cb][r] = ok ? s[cb][r] : NEG_INF;
                }
        }

        float mx = NEG_INF;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[cb][r]);
        mx = xhalf_max(mx);
        // Lazy rescale: the running shift m_run only moves when the tile max
        // exceeds it by more than RESCALE_SLACK (base-2 units), so most tiles
        // need no rescale of l and o~; probabilities then stay below
        // 2^RESCALE_SLACK.  Any shift gives the same softmax, as long as the
        // numerator and denominator share it and nothing overflows.
        const float m_tile = mx == NEG_INF ? NEG_INF : mx * c;
        const bool move = m_tile > m_run + RESCALE_SLACK;
        const float m_new = move ? m_tile : m_run;
        const float m_use = m_new == NEG_INF ? 0.f : m_new;
        const float alpha = move ? exp2_fast(m_run - m_use) : 1.f;
        const bool any_move = __builtin_amdgcn_ballot_w64(move) != 0;
        m_run = m_new;

        float lsum = 0.f;
        bf16x8 pop[BC / 16];
#pragma unroll
        for (int t4 = 0; t4 < BC / 16; ++t4) {
            f32x8 p;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sv = s[t4 >> 1][8 * (t4 & 1) + i];
                float e = exp2_fast(__builtin_fmaf(sv, c, -m_use));
                if (need_mask) e = sv == NEG_INF ? 0.f : e;
                p[i] = e;
                lsum += e;
            }
            pop[t4] = __builtin_convertvector(p, bf16x8);
        }
        l_run = alpha * l_run + lsum;
        if (any_move) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }

        // O^T += V^T P^T
        const uint16_t *vrow = &Vt[l32 * Lay::VS + 8 * hh];
#pragma unroll
        for (int t4 = 0; t4 < BC / 16; ++t4)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x8 vop = *reinterpret_cast<const bf16x8 *>(vrow + 32 * db * Lay::VS + 16 * t4);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[t4], oacc[db], 0, 0, 0);
            }
    }

    const float l_tot = xhalf_sum(l_run);
    if (qrow >= N) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float row_lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * LN2 : NEG_INF;
    // O^T register r of block db holds d index 32*db + 8*(r/4) + 4*hh + r%4.
    if constexpr (!SPLIT) {
        uint16_t *orow = o + ((size_t)bh * N + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                           oacc[db][4 * g + 3] * inv};
                *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * g + 4 * hh) =
                    __builtin_convertvector(x, bf16x4);
            }
        if (hh == 0) lse[(size_t)bh * N + qrow] = row_lse;
    } else {
        const size_t prow = ((size_t)sp * BH + bh) * N + qrow;
        float *orow = part_o + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                           oacc[db][4 * g + 3] * inv};
                *reinterpret_cast<f32x4 *>(orow + 32 * db + 8 * g + 4 * hh) = x;
            }
        if (hh == 0) part_lse[prow] = row_lse;
    }
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_t(const AttnProblem &p, hipStream_t stream) {
    const int ntq = (p.N + BR - 1) / BR;
    const int64_t blocks = (int64_t)p.BH * ntq * p.splits;
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, SPLIT>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                       static_cast<const uint16_t *>(p.v), static_cast<uint16_t *>(p.o), p.lse, p.part_o,
                       p.part_lse, p.BH, p.N, p.M, p.c, qsign, ntq, p.splits, p.tiles_per_split);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnProblem &p, hipStream_t stream) {
    const bool split = p.splits > 1;
    if (p.causal) return split ? launch_t<D, true, true>(p, stream) : launch_t<D, true, false>(p, stream);
    return split ? launch_t<D, false, true>(p, stream) : launch_t<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnProblem &p, hipStream_t stream) {
    return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace osa
