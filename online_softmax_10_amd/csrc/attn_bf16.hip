// Fused attention forward, bf16 inputs, fp32 accumulation, for gfx950 (CDNA4):
// the four-wave kernel (128 query rows per workgroup, two workgroups per CU).
// Used for problems with too few 256-row query tiles to fill the chip with
// the eight-wave kernel (attn_bf16_pp.hip), and for split partials.
//
// Method and per-wave tile math: attn_bf16_common.h (online softmax
// recurrence; "从原始Softmax到在线Softmax" page, online softmax derivation and
// LSE; "Online Softmax and Flash Attention" page, eq. (8)).  The
// FlashAttention idea of keeping Q, K, V tiles on chip so S and P never reach
// HBM ("Softmax与Flash-Attention" page, FlashAttention core idea) with the
// query-outer loop order of its v2 section.
//
// Mapping: four 64-wide waves own 32 rows each.  Key tiles of 64 keys go
// HBM -> LDS by LDS-direct buffer loads into two stages; one wait + barrier
// at the top of tile t lands tile t and retires every read of the other
// stage, and tile t+1's loads are spread between tile t's score MFMAs.  The
// buffer range check returns zeros past key M.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bf16_common.h"
#include "kernels.h"

namespace osa {
namespace {

using namespace bf16;

constexpr int NW = 4;        // waves per workgroup
constexpr int NT = 64 * NW;  // threads per workgroup
constexpr int BR = 32 * NW;  // query rows per workgroup

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ part_o,
    float *__restrict__ part_lse, int BH, int N, int M, float c, uint32_t qsign, int ntq,
    int splits, int tiles_per_split) {
    using T = Tile<D>;
    constexpr int LOADS = T::LOADS / NW;  // per wave per tile, for K and for V
    static_assert(LOADS * NW == T::LOADS, "tile split");
    __shared__ __attribute__((aligned(1024))) char lds_k0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_k1[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v1[T::BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;

    // Workgroup -> (head, split, query tile); heads vary fastest and the
    // longest causal tiles go first.
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
    auto issue = [&](int kv0, char *kdst, char *vdst, int i) {
        const int blk = (wave * LOADS + i) * 1024;
        const int off = (int)((uint32_t)kv0 * T::RB + (uint32_t)ld_off[i]);  // unsigned: M*d < 2^31
        lds_direct_load16(krs, lds_addr(kdst + blk), off);
        lds_direct_load16(vrs, lds_addr(vdst + blk), off);
    };

    // The tile at kv0 from stages (ks, vs); its score MFMAs carry the loads
    // of the next tile (at nkv0, if has_next) into the other stages.
    auto compute_tile = [&](int kv0, const char *ks, const char *vs, bool has_next, int nkv0, char *nks,
                            char *nvs) {
        f32x16 s[2] = {f32x16{}, f32x16{}};
        constexpr int EVERY = (D / 16) / LOADS;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            wt.score_step(ks, kk, s);
            if (has_next && kk % EVERY == 0) issue(nkv0, nks, nvs, kk / EVERY);
        }
        wt.mask(kv0, ke, s);
        bf16x8 pop[BC / 16];
        wt.softmax(s, pop);
        wt.pv(vs, pop);
    };

    if (ntiles > 0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) issue(kb, lds_k0, lds_v0, i);
    }
    for (int t = 0; t < ntiles; t += 2) {
        const int kv0 = kb + t * BC;
        wait_loads_and_barrier<0>();
        compute_tile(kv0, lds_k0, lds_v0, t + 1 < ntiles, kv0 + BC, lds_k1, lds_v1);
        if (t + 1 >= ntiles) break;
        wait_loads_and_barrier<0>();
        compute_tile(kv0 + BC, lds_k1, lds_v1, t + 2 < ntiles, kv0 + 2 * BC, lds_k0, lds_v0);
    }

    wt.template store<SPLIT>(N, o + (size_t)bh * N * D, lse + (size_t)bh * N,
                             part_o + ((size_t)sp * BH + bh) * N * D, part_lse + ((size_t)sp * BH + bh) * N);
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
