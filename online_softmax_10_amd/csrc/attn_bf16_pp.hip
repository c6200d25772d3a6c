// Fused attention forward, bf16 inputs, fp32 accumulation, for gfx950 (CDNA4):
// the eight-wave "ping-pong" kernel (256 query rows per workgroup, one
// workgroup per CU), used when a problem has enough 256-row query tiles to
// fill the chip.
//
// Method and per-wave tile math: attn_bf16_common.h (online softmax
// recurrence; "从原始Softmax到在线Softmax" page, online softmax derivation and
// LSE; "Online Softmax and Flash Attention" page, eq. (8)); the FlashAttention
// idea of keeping the tiles on chip ("Softmax与Flash-Attention" page).
//
// Mapping.  Waves w and w+4 of a workgroup run on the same SIMD.  Waves 0-3
// (group A) and 4-7 (group B) own 128 query rows each and share every K/V
// tile, so a tile crosses HBM/L2 -> LDS once per 256 rows.  The two groups run
// the same recurrence half an iteration apart:
//     iteration j, group A:  S_j = K_j Q^T;  softmax(S_j);  O += V_j^T P_j
//     iteration j, group B:  softmax(S_{j-1});  O += V_{j-1}^T P_{j-1};  S_j = K_j Q^T
// so on each SIMD one wave issues MFMAs while the other runs the softmax on
// the VALU.  K/V tiles are loaded two tiles ahead into four LDS stages each
// (K_{j+2}, V_{j+2} are issued during iteration j's score MFMAs into the
// stages of tile j-2, whose last reader finished in iteration j-1); one
// wait + barrier per iteration lands tile j+1.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bf16_common.h"
#include "kernels.h"

namespace osa {
namespace {

using namespace bf16;

constexpr int NW = 8;        // waves per workgroup
constexpr int NT = 64 * NW;  // threads per workgroup
constexpr int BR = 32 * NW;  // query rows per workgroup
constexpr int STAGES = 4;    // LDS stages per K and per V

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_pp_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ part_o,
    float *__restrict__ part_lse, int BH, int N, int M, float c, uint32_t qsign, int ntq,
    int splits, int tiles_per_split) {
    using T = Tile<D>;
    constexpr int LOADS = T::LOADS / NW;  // per wave per tile, for K and for V
    static_assert(LOADS * NW == T::LOADS && LOADS >= 1, "tile split");
    __shared__ __attribute__((aligned(1024))) char lds_k[STAGES][T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v[STAGES][T::BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const bool group_b = wave >= 4;

    const int b = blockIdx.x;
    const int bh = b % BH;
    const int rest = b / BH;
    const int sp = rest % splits;
    const int qt = ntq - 1 - rest / splits;
    const int q0 = qt * BR;

    const int kb = sp * tiles_per_split * BC;
    int ke = min(M, kb + tiles_per_split * BC);
    if (CAUSAL) ke = min(ke, q0 + BR);
    const int ntiles = ke > kb ? (ke - kb + BC - 1) / BC : 0;

    const u32x4 krs = make_rsrc(k + (size_t)bh * M * D, (uint32_t)M * T::RB);
    const u32x4 vrs = make_rsrc(v + (size_t)bh * M * D, (uint32_t)M * T::RB);

    WaveTile<D, CAUSAL> wt;
    wt.init(q + (size_t)bh * N * D, N, q0 + wave * 32, lane, c, qsign);

    int ld_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) ld_off[i] = load_src_offset<D>(wave * LOADS + i, lane);
    auto issue = [&](int tile, int stage, int i) {
        const int blk = (wave * LOADS + i) * 1024;
        const int off = (int)((uint32_t)(kb + tile * BC) * T::RB + (uint32_t)ld_off[i]);  // unsigned: M*d < 2^31
        lds_direct_load16(krs, lds_addr(&lds_k[stage][blk]), off);
        lds_direct_load16(vrs, lds_addr(&lds_v[stage][blk]), off);
    };

    // S = K Q^T from the stage of tile j, with this wave's loads of tile j+2
    // spread between the MFMAs.
    auto scores = [&](int j, f32x16 (&s)[2]) {
        s[0] = f32x16{};
        s[1] = f32x16{};
        const char *ks = lds_k[j % STAGES];
        const bool load = j + 2 < ntiles;
        constexpr int EVERY = (D / 16) / LOADS;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            wt.score_step(ks, kk, s);
            if (load && kk % EVERY == 0) issue(j + 2, (j + 2) % STAGES, kk / EVERY);
        }
    };
    auto finish = [&](int j, f32x16 (&s)[2]) {
        wt.mask(kb + j * BC, ke, s);
        bf16x8 pop[BC / 16];
        wt.softmax(s, pop);
        wt.pv(lds_v[j % STAGES], pop);
    };
    auto barrier = [&](int j) {
        if (j + 2 < ntiles) wait_loads_and_barrier<2 * LOADS>();
        else wait_loads_and_barrier<0>();
    };
    // The whole key loop of one group; both groups pass the same barriers.
    // Group B carries the scores of tile j across the barrier of iteration j.
    auto run_a = [&]() {
        for (int j = 0; j < ntiles; ++j) {
            f32x16 s[2];
            scores(j, s);
            finish(j, s);
            barrier(j);
        }
    };
    auto run_b = [&]() {
        f32x16 s[2];
        for (int j = 0; j < ntiles; ++j) {
            if (j > 0) finish(j - 1, s);
            scores(j, s);
            barrier(j);
        }
        finish(ntiles - 1, s);
    };

    if (ntiles > 0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) issue(0, 0, i);
        if (ntiles > 1) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) issue(1, 1, i);
            wait_loads_and_barrier<2 * LOADS>();
        } else {
            wait_loads_and_barrier<0>();
        }
        if (group_b) run_b();
        else run_a();
    }

    wt.template store<SPLIT>(N, o + (size_t)bh * N * D, lse + (size_t)bh * N,
                             part_o + ((size_t)sp * BH + bh) * N * D, part_lse + ((size_t)sp * BH + bh) * N);
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_t(const AttnProblem &p, hipStream_t stream) {
    const int ntq = (p.N + BR - 1) / BR;
    const int64_t blocks = (int64_t)p.BH * ntq * p.splits;
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    hipLaunchKernelGGL((attn_fwd_bf16_pp_kernel<D, CAUSAL, SPLIT>), dim3((unsigned)blocks), dim3(NT), 0, stream,
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

hipError_t launch_attn_bf16_pp(const AttnProblem &p, hipStream_t stream) {
    return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace osa
