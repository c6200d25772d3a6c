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
constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor, 32-bit data

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

// Q^T operand: lane (query row, half hh) holds q[row][2*kk + hh], kk < D/2,
// times qsign (0 for a row past N).  Whole 16-byte chunks of a row that
// exists (rows past N read row N - 1), all issued before any is used.
template <int D>
__device__ __forceinline__ void load_q_operand(const float *qh, int N, int row, int hh, float qsign,
                                               float (&qop)[D / 2]) {
    const float *qr = qh + (size_t)min(row, N - 1) * D;
    const float f = row < N ? qsign : 0.f;
    f32x4 x[D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) x[i] = *reinterpret_cast<const f32x4 *>(qr + 4 * i);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        qop[2 * i] = (hh ? x[i][1] : x[i][0]) * f;
        qop[2 * i + 1] = (hh ? x[i][3] : x[i][2]) * f;
    }
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
    load_q_operand<D>(qh, N, qrow, hh, qsign, qop);

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

// Small problems: one workgroup per 16-row query block, its KW waves each
// taking every KW-th 32-key tile (a split over keys inside the workgroup;
// tiles interleaved so causal ranges share out evenly), with K and V staged
// in each wave's own LDS region.  Each wave keeps the running max, sum and
// unnormalised accumulator of its tiles; at the end the waves' states are
// merged in LDS with the same rule as any two blocks of the recurrence
// (L = sum_w l_w 2^{m_w - M}, O = sum_w o~_w 2^{m_w - M} / L, M the largest
// m_w): "从原始Softmax到在线Softmax" page, the merge of two (m, l, o~)
// states.  One launch, no workspace.  No bias (the four-wave kernel above
// takes those).
//
// Products on v_mfma_f32_16x16x4_f32 (A 16x4, B 4x16, one value per lane per
// operand; result register r of lane l is row 4*(l/16) + r, column l%16).
// Scores are computed transposed, S^T = K Q^T, 16 keys x 16 queries per
// block, so lane l owns query l%16 and keys 4*(l/16) + r of the block.  The
// feature index of product step kk for lane group g = l/16 is 16*g + kk, so a
// lane reads 16 consecutive floats of its key row (and of its query row).
// P^T feeds O^T += V^T P^T straight from the score registers: step r of a
// key block takes key 4*g + r in lane group g, which is register r.
template <int D>
struct Small {
    static constexpr int KW = D == 64 ? kF32SmallWaves64 : kF32SmallWaves128;  // waves per workgroup
    static constexpr int KS = D + 4, VS = D + 4;         // LDS row strides (floats): conflict-free reads
    static constexpr int REGION = BC * (KS + VS);        // floats per wave: a K tile and a V tile
    static constexpr int LOADS = BC * D / 4 / 64;        // float4 chunks per lane per tile (K and V each)
    static constexpr int OS = D + 4;                     // row stride (floats) of a wave's scaled o~ in the merge
    static_assert(REGION >= 16 * OS + 32, "the merge state fits a wave's region");
};

// Max and sum over the four 16-lane rows of a wave (the keys of one query).
__device__ __forceinline__ float rows4_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    return xhalf_max(x);
}
__device__ __forceinline__ float rows4_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    return xhalf_sum(x);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * Small<D>::KW, 1) void attn_fwd_f32_small_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v, float *__restrict__ o,
    float *__restrict__ lse, int BH, int N, int M, float c, float qsign, int nrb, const int32_t *__restrict__ kv_len,
    int H, int coff) {
    using S = Small<D>;
    __shared__ __attribute__((aligned(16))) float smem[S::KW * S::REGION];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;  // this lane's query in the block
    const int g = lane >> 4;    // lane group: keys 4g..4g+3 of a 16-key block, features 16g..16g+15
    float *Ks = smem + wave * S::REGION;
    float *Vs = Ks + BC * S::KS;

    // Workgroup -> (head, 16-row block); the longest causal blocks first.
    const int bh = blockIdx.x % BH;
    const int rb = nrb - 1 - blockIdx.x / BH;
    const int r0 = rb * 16;
    const int qrow = r0 + l16;
    int ke = M;
    if (kv_len != nullptr) ke = min(ke, max(kv_len[bh / H], 0));
    if (CAUSAL) ke = min(ke, r0 + 16 + coff);
    const int ntiles = ke > 0 ? (ke + BC - 1) / BC : 0;

    const float *qh = q + (size_t)bh * N * D;
    const float *kh = k + (size_t)bh * M * D;
    const float *vh = v + (size_t)bh * M * D;
    // This wave's next tile in registers, read through buffer descriptors
    // that end at key ke, so keys at or past ke (and whole tiles past the
    // last) read as 0 without a branch; they are masked.  The first tile is
    // requested before Q so that the two arrive in one round trip; each later
    // tile is requested while the tile before it is in the matrix cores.
    const int kv_bytes = max(ke, 0) * D * 4;  // ke <= M <= kF32SmallMaxKeys
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(kh), 0, kv_bytes,
                                                                         kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(vh), 0, kv_bytes,
                                                                         kBufferWord3);
    f32x4 kr[S::LOADS], vr[S::LOADS];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i) {
            const int id = lane + 64 * i;
            const int off = ((t * BC + id / (D / 4)) * D + 4 * (id % (D / 4))) * 4;
            kr[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
            vr[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
        }
    };
    load_tile(wave);
    // Q operand: lane (query l16, group g) holds q[qrow][16g + kk], kk < 16,
    // per D/64 feature chunks, times qsign (0 for a row past N; rows past N
    // read row N - 1).
    float qop[D / 4];
    {
        const float *qr = qh + (size_t)min(qrow, N - 1) * D;
        const float f = qrow < N ? qsign : 0.f;
        f32x4 x[D / 16];
#pragma unroll
        for (int ch = 0; ch < D / 64; ++ch)
#pragma unroll
            for (int j = 0; j < 4; ++j) x[4 * ch + j] = *reinterpret_cast<const f32x4 *>(qr + 64 * ch + 16 * g + 4 * j);
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) qop[4 * i + e] = x[i][e] * f;
    }

    // O^T accumulator: block db, register r is feature 16*db + 4g + r of query l16.
    f32x4 oacc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{};
    float m_run = NEG_INF;
    float l_run = 0.f;

    for (int t = wave; t < ntiles; t += S::KW) {
        const int kv0 = t * BC;
        __builtin_amdgcn_wave_barrier();  // the wave is done reading the previous tile
#pragma unroll
        for (int i = 0; i < S::LOADS; ++i) {
            const int id = lane + 64 * i;
            const int row = id / (D / 4), c4 = id % (D / 4);
            *reinterpret_cast<f32x4 *>(&Ks[row * S::KS + 4 * c4]) = kr[i];
            *reinterpret_cast<f32x4 *>(&Vs[row * S::VS + 4 * c4]) = vr[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        load_tile(t + S::KW);  // zeros once past the last tile
        // S^T for the tile's two 16-key blocks.
        f32x4 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4{};
            const float *krow = &Ks[(16 * kb + l16) * S::KS + 16 * g];
#pragma unroll
            for (int ch = 0; ch < D / 64; ++ch) {
                f32x4 kop[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) kop[j] = *reinterpret_cast<const f32x4 *>(krow + 64 * ch + 4 * j);
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kop[kk / 4][kk % 4], qop[16 * ch + kk], s[kb], 0, 0,
                                                                 0);
            }
        }
        // The next tile's loads go out one per two products of this tile.
#pragma unroll
        for (int i = 0; i < 2 * S::LOADS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        // Register r of block kb holds key kv0 + 16*kb + 4g + r.
        const bool need_mask = (kv0 + BC > ke) || (CAUSAL && kv0 + BC - 1 > r0 + coff);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kv0 + 16 * kb + 4 * g + r;
                    const bool ok = key < ke && (!CAUSAL || key <= qrow + coff);
                    s[kb][r] = ok ? s[kb][r] : NEG_INF;
                }
        }
        float mx = NEG_INF;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = rows4_max(mx);
        const float m_tile = mx == NEG_INF ? NEG_INF : mx * c;
        const float m_new = fmaxf(m_run, m_tile);
        const float m_use = m_new == NEG_INF ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_use));
                if (need_mask) e = s[kb][r] == NEG_INF ? 0.f : e;
                s[kb][r] = e;
                lsum += e;
            }
        l_run = alpha * l_run + lsum;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float *vrow = &Vs[(16 * kb + 4 * g + r) * S::VS + l16];
#pragma unroll
                for (int db = 0; db < D / 16; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * db], s[kb][r], oacc[db], 0, 0, 0);
            }
    }

    // Merge.  Each wave publishes the m and l of its 16 rows; every wave
    // then forms the row's M = max_w m_w and L = sum_w l_w 2^{m_w - M} (the
    // same reads in the same order, so the same values), scales its own o~
    // by 2^{m_w - M} / L and stores it; the workgroup sums the KW scaled
    // tiles.  A row with L = 0 (no visible key) gets o = 0 and LSE = -inf.
    const float l_tot = rows4_sum(l_run);
    float *own = smem + wave * S::REGION;  // this wave's K/V staging, now free
    __builtin_amdgcn_wave_barrier();
    if (g == 0) {
        own[16 * S::OS + l16] = m_run;
        own[16 * S::OS + 16 + l16] = l_tot;
    }
    __syncthreads();
    float mm = NEG_INF;
#pragma unroll
    for (int w = 0; w < S::KW; ++w) mm = fmaxf(mm, smem[w * S::REGION + 16 * S::OS + l16]);
    float ll = 0.f;
    if (mm != NEG_INF) {
#pragma unroll
        for (int w = 0; w < S::KW; ++w) {
            const float *st = smem + w * S::REGION + 16 * S::OS;
            ll += __builtin_amdgcn_exp2f(st[l16] - mm) * st[16 + l16];  // 0 for an empty wave
        }
    }
    const float wt = ll > 0.f ? __builtin_amdgcn_exp2f(m_run - mm) / ll : 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4 *>(&own[l16 * S::OS + 16 * db + 4 * g]) = oacc[db] * wt;
    if (wave == 0 && g == 0 && qrow < N)
        lse[(size_t)bh * N + qrow] = ll > 0.f ? (mm + log2f(ll)) * LN2 : NEG_INF;
    __syncthreads();
    // Thread t sums float4 chunks t, t + 64*KW, ... of the 16 x D output.
    for (int f = tid; f < 16 * D / 4; f += 64 * S::KW) {
        const int row = f / (D / 4), c4 = f % (D / 4);
        f32x4 acc = *reinterpret_cast<const f32x4 *>(&smem[row * S::OS + 4 * c4]);
#pragma unroll
        for (int w = 1; w < S::KW; ++w) acc += *reinterpret_cast<const f32x4 *>(&smem[w * S::REGION + row * S::OS + 4 * c4]);
        if (r0 + row < N) *reinterpret_cast<f32x4 *>(&o[((size_t)bh * N + r0 + row) * D + 4 * c4]) = acc;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_small_t(const AttnProblem &p, hipStream_t stream) {
    using S = Small<D>;
    const int nrb = (p.N + 15) / 16;
    hipLaunchKernelGGL((attn_fwd_f32_small_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)p.BH * nrb)),
                       dim3(64 * S::KW), 0, stream, static_cast<const float *>(p.q),
                       static_cast<const float *>(p.k), static_cast<const float *>(p.v), static_cast<float *>(p.o),
                       p.lse, p.BH, p.N, p.M, p.c, p.negate_q ? -1.f : 1.f, nrb, p.kv_len, p.H, p.causal_off);
    return hipGetLastError();
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

hipError_t launch_attn_f32_small(const AttnProblem &p, hipStream_t stream) {
    // Single pass, no bias, and at most kF32SmallMaxKeys keys.
    if (p.splits != 1 || p.bias != nullptr || p.M > kF32SmallMaxKeys) return hipErrorInvalidValue;
    if (p.d == 64) return p.causal ? launch_small_t<64, true>(p, stream) : launch_small_t<64, false>(p, stream);
    return p.causal ? launch_small_t<128, true>(p, stream) : launch_small_t<128, false>(p, stream);
}

}  // namespace osa
