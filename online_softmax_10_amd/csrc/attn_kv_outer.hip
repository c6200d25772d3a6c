// The key/value-outer loop order of the first FlashAttention formulation, as
// a measured alternative to the query-outer order of attn_bf16.hip: one
// launch per key/value block j (the outer loop, on the host); in launch j
// every (head, 128-row query tile) that sees a key of block j merges the
// block into its rows' state held in HBM -- the normalised output O, the max
// m and the sum l -- and writes the state back:
//     m~ = rowmax(S_ij),  P~ = e^{S_ij - m~},  l~ = rowsum(P~),
//     m_new = max(m_i, m~),  l_new = e^{m_i - m_new} l_i + e^{m~ - m_new} l~,
//     O_i <- (e^{m_i - m_new} l_i O_i + e^{m~ - m_new} P~ V_j) / l_new.
// Source: "从原始Softmax到在线Softmax" page, the blocked online-softmax code
// under "softmax实际代码实现" (key/value blocks outer, query blocks inner,
// scale_old / scale_new, normalised O written back per block); the same
// recurrence as eq. (20)-(22) of the "Online Softmax and Flash Attention" page.
// The last block a tile sees writes the bf16 output and the LSE instead.
//
// Per tile and block the state round trip costs 2 x 128 x (4d + 8) bytes of
// HBM traffic, and Q is re-read: the traffic the query-outer order avoids.
// The per-wave math (S^T on MFMA, transposed V reads, base-2 exponentials)
// is that of attn_bf16_common.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bf16_common.h"
#include "kernels.h"

namespace osa {
namespace {

using namespace bf16;

constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int BR = 32 * NW;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void attn_kv_block_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ ws_o, float *__restrict__ ws_m,
    float *__restrict__ ws_l, int BH, int N, int M, float c, uint32_t qsign, int ntq, int j, int nkv) {
    using T = Tile<D>;
    constexpr int LOADS = T::LOADS / NW;
    __shared__ __attribute__((aligned(1024))) char lds_k[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v[T::BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int bh = blockIdx.x % BH;
    const int q0 = (blockIdx.x / BH) * BR;
    const int kv0 = j * BC;
    // Blocks this tile sees: all, or (causal) up to the one holding its last row.
    const int last = CAUSAL ? min(nkv - 1, (min(N, q0 + BR) - 1) / BC) : nkv - 1;
    if (j > last) return;  // whole workgroup: no key of block j is visible to the tile
    const int ke = min(M, kv0 + BC);

    const u32x4 krs = make_rsrc(k + (size_t)bh * M * D, (uint32_t)M * T::RB);
    const u32x4 vrs = make_rsrc(v + (size_t)bh * M * D, (uint32_t)M * T::RB);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int off = (int)((uint32_t)kv0 * T::RB + (uint32_t)load_src_offset<D>(wave * LOADS + i, lane));
        lds_direct_load16(krs, lds_addr(lds_k + (wave * LOADS + i) * 1024), off);
        lds_direct_load16(vrs, lds_addr(lds_v + (wave * LOADS + i) * 1024), off);
    }

    WaveTile<D, CAUSAL> wt;
    wt.init(q + (size_t)bh * N * D, N, q0 + wave * 32, lane, c, qsign, 0);
    wait_loads_and_barrier<0>();

    // Block scores, block max, block probabilities and their sum, P~ V_j.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) wt.score_step(lds_k, kk, s);
    wt.mask(kv0, ke, s);
    float mx = NEG_INF;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[cb][r]);
    const float m_blk = xhalf_max(mx) * c;  // base-2 units; -inf: no visible key in this block
    bf16x8 pop[BC / 16];
    const float l_blk = xhalf_sum(wt.probs(s, m_blk == NEG_INF ? 0.f : m_blk, pop));
#pragma unroll
    for (int slot = 0; slot < 4 * (D / 32); ++slot) {
        const int t4 = slot / (D / 32), db = slot % (D / 32);
        wt.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wt.vread(lds_v, slot), pop[t4], wt.oacc[db], 0, 0, 0);
    }

    // Merge with the row state in HBM (none before the first block).
    const int qrow = wt.qrow;
    if (qrow >= N) return;
    const size_t row = (size_t)bh * N + qrow;
    float m_i = NEG_INF, l_i = 0.f;
    f32x4 o_i[D / 32][4];
    if (j > 0) {
        m_i = ws_m[row];
        l_i = ws_l[row];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                o_i[db][g] = *reinterpret_cast<const f32x4 *>(ws_o + row * D + 32 * db + 8 * g + 4 * wt.hh);
    } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) o_i[db][g] = f32x4{};
    }
    const float m_new = fmaxf(m_i, m_blk);
    const float m_use = m_new == NEG_INF ? 0.f : m_new;
    const float so = exp2_fast(m_i - m_use);   // 0 when m_i = -inf
    const float sn = exp2_fast(m_blk - m_use); // 0 when the block has no visible key
    const float l_new = so * l_i + sn * l_blk;
    const float inv = l_new > 0.f ? 1.f / l_new : 0.f;
    const float a = so * l_i * inv;  // weight of the old normalised O
    const float b = sn * inv;        // weight of the unnormalised block output P~ V_j
    if (j < last) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = a * o_i[db][g][e] + b * wt.oacc[db][4 * g + e];
                *reinterpret_cast<f32x4 *>(ws_o + row * D + 32 * db + 8 * g + 4 * wt.hh) = x;
            }
        if (wt.hh == 0) {
            ws_m[row] = m_new;
            ws_l[row] = l_new;
        }
    } else {
        uint16_t *orow = o + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = a * o_i[db][g][e] + b * wt.oacc[db][4 * g + e];
                *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * g + 4 * wt.hh) = __builtin_convertvector(x, bf16x4);
            }
        if (wt.hh == 0) lse[row] = l_new > 0.f ? (m_new + log2f(l_new)) * LN2 : NEG_INF;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_t(const AttnProblem &p, float *ws_o, float *ws_m, float *ws_l, hipStream_t stream) {
    const int ntq = (p.N + BR - 1) / BR;
    const int nkv = (p.M + BC - 1) / BC;
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    for (int j = 0; j < nkv; ++j) {
        hipLaunchKernelGGL((attn_kv_block_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)p.BH * ntq)), dim3(NT), 0,
                           stream, static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                           static_cast<const uint16_t *>(p.v), static_cast<uint16_t *>(p.o), p.lse, ws_o, ws_m,
                           ws_l, p.BH, p.N, p.M, p.c, qsign, ntq, j, nkv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_attn_kv_outer(const AttnProblem &p, float *ws_o, float *ws_m, float *ws_l, hipStream_t stream) {
    if (p.d == 64) return p.causal ? launch_t<64, true>(p, ws_o, ws_m, ws_l, stream)
                                   : launch_t<64, false>(p, ws_o, ws_m, ws_l, stream);
    return p.causal ? launch_t<128, true>(p, ws_o, ws_m, ws_l, stream)
                    : launch_t<128, false>(p, ws_o, ws_m, ws_l, stream);
}

}  // namespace osa
