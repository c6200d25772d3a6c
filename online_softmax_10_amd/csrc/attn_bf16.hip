// Fused attention forward, bf16 inputs, fp32 accumulation, for gfx950 (CDNA4).
//
// Method and per-wave pieces: attn_bf16_common.h (online softmax recurrence;
// "从原始Softmax到在线Softmax" page, online softmax derivation and LSE; "Online
// Softmax and Flash Attention" page, eq. (8)).  The FlashAttention idea of
// keeping the Q, K, V tiles on chip so S and P never reach HBM
// ("Softmax与Flash-Attention" page, FlashAttention core idea), with the
// query-outer loop order of its v2 section.
//
// One kernel body, three forms:
//   attn_fwd_bf16_w8_kernel  8 waves, 256 query rows per workgroup, one per CU
//                            (problems whose 256-row tiles fill the chip; single
//                            pass), so a K/V tile crosses L2 -> LDS once per 256
//                            rows;
//   attn_fwd_bf16_kh_kernel  8 waves on 128 query rows, in two sets of four that
//                            take alternate key tiles (each with its own K/V
//                            stages) and merge their states at the end (problems
//                            whose 128-row tiles number at most 256: one per CU;
//                            single pass);
//   attn_fwd_bf16_kernel     4 waves, 128 query rows per workgroup, two
//                            workgroups per CU (the other problems, split
//                            partials).
// Each SIMD runs two waves.  attn_fwd_bf16_w8_bias_kernel and
// attn_fwd_bf16_bias_kernel are the 256- and 128-row forms with an additive
// score bias.
//
// Software pipeline.  Iteration j of a wave's key loop, with the scores
// S(j) of tile j already in registers, shifted and masked:
//   - one wait + barrier: K(j+1) and V(j) have landed in LDS, and every wave
//     is done with the stages the iteration's loads overwrite;
//   - the 16 score MFMAs of S(j+1) = K(j+1) Q^T, each followed by the K
//     operand read two MFMAs ahead and by the probabilities of tile j's
//     remaining scores (exp2, bf16 pack, dot2 into the sum), so the matrix
//     cores and the VALU work side by side; K(j+2) and V(j+1) are loaded
//     between;
//   - the rare exact-shift path (attn_bf16_common.h);
//   - the 16 MFMAs of O^T += V(j)^T P(j)^T with the transposed V reads two
//     MFMAs ahead, each followed by the shift (and on diagonal tiles the
//     mask) of two of tile j+1's scores and, in the first slots, the
//     probabilities of its first pairs.
// sched_barrier fences keep this order: the compiler's own schedule puts the
// MFMAs and the softmax in separate runs.  K/V tiles of 64 keys go HBM -> LDS
// by LDS-direct buffer loads into two stages each; the buffer range check
// returns zeros past key M.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_bf16_common.h"
#include "kernels.h"

namespace osa {
namespace {

using namespace bf16;

// Nothing is scheduled across this point.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

template <int NW, int D, bool CAUSAL, bool SPLIT, bool BIAS, int KH = 1>
__device__ __forceinline__ void attn_body(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                          const uint16_t *__restrict__ v, uint16_t *__restrict__ o,
                                          float *__restrict__ lse, float *__restrict__ part_o,
                                          float *__restrict__ part_lse, int BH, int N, int M, float c,
                                          uint32_t qsign, int ntq, int splits, int tiles_per_split,
                                          const int32_t *__restrict__ kv_len, int H, int coff,
                                          const float *__restrict__ bias, uint32_t bias_bytes, int64_t bias_sb,
                                          int64_t bias_sh, int64_t bias_sn) {
    using T = Tile<D>;
    constexpr int BR = 32 * NW;           // query rows per workgroup
    constexpr int LOADS = T::LOADS / NW;  // LDS-direct loads per wave per tile, for K and for V
    constexpr int SLOTS = 2 * (D / 16);   // score MFMAs per tile
    constexpr int PSLOTS = 4 * (D / 32);  // P.V MFMAs per tile
    constexpr int EVERY = SLOTS / LOADS;  // score slots per load pair
    static_assert(LOADS * NW == T::LOADS && LOADS >= 1 && EVERY >= 1, "tile split");
    // Scores arrive shifted: the previous P.V phase brought them to base-2
    // units against the shift (with a bias, in the FMA that adds it).  Paired
    // A/B per launch against shifting in the score phase: 2x16x4096^2 causal
    // -3.8 % at d = 128 (-6.7 % at d = 64), 1x8x16384^2 causal -2.5 %;
    // 4x8x1024^2 at d = 64, one wave per SIMD, unchanged; with an [N, M]
    // bias -2.5 % at d = 64 and -1.5 % at d = 128.  MASK_LATE: with a bias
    // at d = 128 the mask is applied at the start of the iteration (masking
    // during the P.V phase made that kernel spill in its key loop, +7.4 %).
    constexpr bool MASK_LATE = BIAS && D == 128;
    // Probability pairs of the next tile formed during the P.V phase
    // (the rest in the score phase); their packed values and sum carry over.
    // 4 of the 16 (paired A/B: 2x16x4096^2 causal -1.4 %, 1x8x16384^2 causal
    // -0.3 %; 2 or 6 pairs did worse, 8 gained nothing);
    // none with a bias, whose runs are added during the first half of the
    // P.V phase.
    constexpr int EARLY = BIAS ? 0 : 4;
    // The four-wave width at d = 64 (one wave per SIMD where it runs alone,
    // as on 4x8x1024^2) reads the first V operands of the P.V phase at the
    // start of the iteration: eight more registers live through the score
    // phase, which it has to spare (-1.5 % per launch on 4x8x1024^2 in
    // interleaved A/B).  At d = 128 the same move spills in the key loop.
    constexpr bool EARLY_V = NW == 4 && D == 64;
    uint32_t popw[BC / 16][4];
    float lsum_early = 0.f;
    // KH = 2: the workgroup holds two sets of NW waves on the same rows, set
    // h taking the key tiles t = 2j + h of the range, each with its own LDS
    // stages; their states are merged at the end.
    static_assert(KH == 1 || (KH == 2 && (!BIAS || D == 64)), "key halves: a bias only at d = 64 (LDS)");
    __shared__ __attribute__((aligned(1024))) char lds_k0[KH * T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_k1[KH * T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v0[KH * T::BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_v1[KH * T::BYTES];

    const int tid = threadIdx.x;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = KH == 1 ? 0 : wave_all / NW;    // which key half
    const int wave = KH == 1 ? wave_all : wave_all % NW;  // wave within its half (row block)
    const int lane = tid & 63;
    char *const k0 = lds_k0 + half * T::BYTES;
    char *const k1 = lds_k1 + half * T::BYTES;
    char *const v0 = lds_v0 + half * T::BYTES;
    char *const v1 = lds_v1 + half * T::BYTES;

    // Workgroup -> (head, split, query tile); heads vary fastest and the
    // longest causal tiles go first.
    const int b = blockIdx.x;
    const int bh = b % BH;
    const int rest = b / BH;
    const int sp = rest % splits;
    const int qt = ntq - 1 - rest / splits;
    const int q0 = qt * BR;

    const int kb = sp * tiles_per_split * BC;
    // Visible keys of this workgroup: its split's range, the batch's key
    // length, and (causal) the last row's limit.
    int ke = min(M, kb + tiles_per_split * BC);
    if (kv_len != nullptr) ke = min(ke, max(kv_len[bh / H], 0));
    if (CAUSAL) ke = min(ke, q0 + BR + coff);
    const int tiles_wg = ke > kb ? (ke - kb + BC - 1) / BC : 0;
    // This half's tiles are t = KH*j + half (first key tkey(j)); every wave
    // of the workgroup passes niter barriers in the key loop.
    const int ntiles = tiles_wg > half ? (tiles_wg - half + KH - 1) / KH : 0;
    const int niter = (tiles_wg + KH - 1) / KH;
    auto tkey = [&](int j) { return kb + (KH * j + half) * BC; };

    const u32x4 krs = make_rsrc(k + (size_t)bh * M * D, (uint32_t)M * T::RB);
    const u32x4 vrs = make_rsrc(v + (size_t)bh * M * D, (uint32_t)M * T::RB);

    WaveTile<D, CAUSAL> wt;
    wt.init(q + (size_t)bh * N * D, N, q0 + wave * 32, lane, c, qsign, coff);
    // This lane's bias row as a byte offset into the bias buffer (rows past N
    // read row N - 1); the front end keeps the bias extent below 2^32 bytes.
    u32x4 brs{};
    uint32_t brow = 0;
    char *bregion = nullptr;  // this wave's 8 KiB bias stage in LDS
    if constexpr (BIAS) {
        __shared__ __attribute__((aligned(1024))) char lds_b[KH * NW * 8192];
        bregion = lds_b + wave_all * 8192;
        brs = make_rsrc(bias, bias_bytes);
        brow = 4u * (uint32_t)((int64_t)(bh / H) * bias_sb + (int64_t)(bh % H) * bias_sh +
                               (int64_t)min(wt.qrow, N - 1) * bias_sn);
    }

    int ld_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) ld_off[i] = load_src_offset<D>(wave * LOADS + i, lane);
    // This wave's share i of tile `tile` of K (or V) into an LDS stage.
    // Unsigned offsets: M * d < 2^31, so M * 2d < 2^32.
    auto load = [&](const u32x4 &rs, int tile, char *dst, int i) {
        const int off = (int)((uint32_t)tkey(tile) * T::RB + (uint32_t)ld_off[i]);
        lds_direct_load16(rs, lds_addr(dst + (wave * LOADS + i) * 1024), off);
    };

    // On entry s_cur = S(j); after the barrier K(j+1) is in ks_next and V(j)
    // in vs_cur.  FULL: this wave computes tile j+1 too (its scores go to
    // s_nxt).  LOADS: tile j+1 exists for the workgroup, so this wave issues
    // its share of K(j+2) and V(j+1) into the stages every wave has finished
    // with.  Load tile indices past the last are clamped to it: a harmless
    // reload into a free stage that keeps the block free of branches.
    // bias_next: this wave computes tile j+2 too (its bias is fetched here).
    // s_cur arrives shifted (x = c*s - sh, sh the shift base when it was
    // shifted) and, unless MASK_LATE, masked: the P.V phase of the previous
    // iteration (the prologue for tile 0) did both while its MFMAs ran, and
    // this iteration does the same for s_nxt.
    auto iteration = [&](auto full, auto loads, int j, bool bias_next, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                         const char *ks_next, char *ks_free, const char *vs_cur, char *vs_free) {
        constexpr bool FULL = decltype(full)::value;
        constexpr bool LOADS_ON = decltype(loads)::value;
        wait_loads_and_barrier<0>();
        // Key halves: the score phase issues at a raised wave priority and the
        // P.V phase at the lowest, so that a SIMD's wave that is still in its
        // score phase goes before its partner that has reached the P.V phase
        // (-2 to -3 % per launch on 4x8x1024^2, bit-identical; on the other
        // widths the same change makes no difference).
        if constexpr (KH == 2) __builtin_amdgcn_s_setprio(2);
        if constexpr (MASK_LATE) wt.mask(tkey(j), ke, s_cur);
        float lsum0 = 0.f, lsum1 = 0.f;
        bf16x8 kop[3];
        if constexpr (FULL) {
            s_nxt[0] = f32x16{};
            s_nxt[1] = f32x16{};
            kop[0] = wt.kread(ks_next, 0);
            kop[1] = wt.kread(ks_next, 1);
        }
        // V(j) landed with the barrier too: where the registers allow (EARLY_V),
        // the first two V operands are read now, so that the P.V phase does
        // not start on an LDS round trip.
        bf16x8 vop[3];
        if constexpr (EARLY_V) {
            vop[0] = wt.vread(vs_cur, 0);
            vop[1] = wt.vread(vs_cur, 1);
        }
        fence();
#pragma unroll
        for (int slot = 0; slot < SLOTS; ++slot) {
            if constexpr (FULL) {
                s_nxt[slot & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[slot % 3], wt.qop[slot >> 1],
                                                                          s_nxt[slot & 1], 0, 0, 0);
                if (slot + 2 < SLOTS) kop[(slot + 2) % 3] = wt.kread(ks_next, slot + 2);
            }
            // 32 scores over SLOTS slots: two per slot at d = 128, four at d = 64.
            {
                // the pairs left after the early ones, spread over the slots
                constexpr int LEFT = 16 - EARLY;
#pragma unroll
                for (int pp = EARLY + (slot * LEFT) / SLOTS; pp < EARLY + ((slot + 1) * LEFT) / SLOTS; ++pp)
                    wt.prob_pair_x(s_cur, 2 * pp, popw, (pp & 1) ? lsum1 : lsum0);
            }
            if constexpr (LOADS_ON) {
                if (slot % EVERY == EVERY - 1) {
                    load(krs, min(j + 2, ntiles - 1), ks_free, slot / EVERY);
                    load(vrs, j + 1, vs_free, slot / EVERY);
                }
            }
            fence();
        }
        bf16x8 pop[BC / 16];
#pragma unroll
        for (int g = 0; g < BC / 16; ++g)
            pop[g] = __builtin_bit_cast(bf16x8, (u32x4{popw[g][0], popw[g][1], popw[g][2], popw[g][3]}));
        float lsum = lsum0 + lsum1 + lsum_early;
        // Some row's tile sum above the limit or not finite, or a row without
        // a shift yet: the exact path.
        float alpha = 1.f;
        if (__builtin_amdgcn_ballot_w64(wt.needs_exact_x(lsum)) != 0) alpha = wt.exact_shift_x(s_cur, pop, lsum);
        wt.l_run = alpha * wt.l_run + lsum;
        const float sh = wt.shift_base();  // for tile j+1's scores

        if constexpr (!EARLY_V) {
            vop[0] = wt.vread(vs_cur, 0);
            vop[1] = wt.vread(vs_cur, 1);
        }
        // The next tile's scores are masked first (its early pairs are formed
        // below); a masked -inf stays -inf when shifted.
        if constexpr (FULL && !MASK_LATE) wt.mask(tkey(j + 1), ke, s_nxt);
        float le0 = 0.f, le1 = 0.f;
        fence();
        if constexpr (KH == 2) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int slot = 0; slot < PSLOTS; ++slot) {
            const int t4 = slot / (D / 32), db = slot % (D / 32);
            wt.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[slot % 3], pop[t4], wt.oacc[db], 0, 0, 0);
            if (slot + 2 < PSLOTS) vop[(slot + 2) % 3] = wt.vread(vs_cur, slot + 2);
            // The VALU is free here.  Without a bias: tile j+1's scores are
            // shifted, 32 / PSLOTS per slot.  With a bias: the bias of tile
            // j+1 (staged during the last iteration, landed with this
            // iteration's wait) goes into its scores, run by run; then tile
            // j+2's bias is fetched into the same region, once every read of
            // it has returned.
            if constexpr (FULL && !BIAS) {
#pragma unroll
                for (int u = 0; u < 32 / PSLOTS; u += 2) wt.shift_pair(s_nxt, slot * (32 / PSLOTS) + u, sh);
                // early pair slot-1 (shifted in the previous slot)
                if (slot >= 1 && slot - 1 < EARLY) wt.prob_pair_x(s_nxt, 2 * (slot - 1), popw, ((slot - 1) & 1) ? le1 : le0);
            }
            if constexpr (BIAS && FULL) {
                constexpr int PER = (8 + PSLOTS / 2 - 1) / (PSLOTS / 2);  // runs per slot over the first half
                if (slot < PSLOTS / 2) {
#pragma unroll
                    for (int t = slot * PER; t < slot * PER + PER && t < 8; ++t) wt.bias_apply(bregion, t, lane, s_nxt, c, sh);
                }
                if (slot == PSLOTS / 2 && bias_next) {
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wt.bias_dma(brs, brow, tkey(j + 2), bregion);
                }
            }
            fence();
        }
        if constexpr (FULL) lsum_early = le0 + le1;
    };
    using Full = std::integral_constant<bool, true>;
    using Last = std::integral_constant<bool, false>;
    using LoadsOn = std::integral_constant<bool, true>;
    using LoadsOff = std::integral_constant<bool, false>;

    // Tiles this wave computes: those holding a key visible to one of its
    // rows (with a causal mask the last ones of the workgroup's range are
    // fully masked for its first waves; rows past N need none).  Its
    // remaining iterations only pass the barriers and issue its share of the
    // loads, so every wave passes the same ntiles barriers.
    int nw = 0;
    {
        const int row_lo = q0 + wave * 32;
        const int row_hi = min(N, row_lo + 32) - 1;
        int last_key = ke - 1;
        if (CAUSAL) last_key = min(last_key, row_hi + coff);
        if (row_hi >= row_lo && last_key >= kb) {
            const int tl = (last_key - kb) / BC;  // last tile of the range with a visible key
            nw = tl >= half ? (tl - half) / KH + 1 : 0;
        }
        nw = __builtin_amdgcn_readfirstlane(nw);
    }


    if (niter > 0) {
        // Prologue: every stage is free, so K(0), V(0) and K(1) load together
        // (one memory latency).  S(0) needs only Q and K(0) (and tile 0's
        // bias), issued first: it is computed once they have landed, while
        // V(0) and K(1) -- the last 2 * LOADS loads of each wave -- may still
        // be on their way (the first iteration waits for them).
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            if (ntiles > 0) load(krs, 0, k0, i);
        if constexpr (BIAS) {
            if (nw > 0) wt.bias_dma(brs, brow, tkey(0), bregion);
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            if (ntiles > 0) {
                load(vrs, 0, v0, i);
                load(krs, min(1, ntiles - 1), k1, i);
            }
        }
        wait_loads_and_barrier<2 * LOADS>();
        f32x16 sa[2] = {f32x16{}, f32x16{}}, sb[2];
        // Stages alternate with the parity of j: even j reads K(j+1) from k1
        // and V(j) from v0, and refills k0 and v1.
        int j = 0;
        if (nw > 0) {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) wt.score_step(k0, kk, sa);
            {
                // Tile 0 masked, shifted against base 0 (no shift yet) -- with
                // a bias by adding it (landed with the prologue's wait) --,
                // its early pairs formed.
                if constexpr (!MASK_LATE) wt.mask(tkey(0), ke, sa);
                if constexpr (BIAS) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) wt.bias_apply(bregion, t, lane, sa, c, 0.f);
                } else {
#pragma unroll
                    for (int e = 0; e < 32; e += 2) wt.shift_pair(sa, e, 0.f);
                }
                // With tile 0 masked, its row max is the row's first shift, so
                // the first iteration needs no exact path (a row with no
                // visible key in tile 0 keeps none).  Unmasked (MASK_LATE), a
                // masked key could set a shift under which the visible ones
                // vanish: the exact path of the first iteration sets it then.
                if constexpr (!MASK_LATE) wt.first_shift(sa);
                float le = 0.f;
#pragma unroll
                for (int e = 0; e < 2 * EARLY; e += 2) wt.prob_pair_x(sa, e, popw, le);
                lsum_early = le;
            }
            if constexpr (BIAS) {
                // Tile 1's bias follows tile 0's.
                if (nw > 1) {
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wt.bias_dma(brs, brow, tkey(1), bregion);
                }
            }
            for (; j + 2 < nw; j += 2) {
                iteration(Full{}, LoadsOn{}, j, true, sa, sb, k1, k0, v0, v1);
                iteration(Full{}, LoadsOn{}, j + 1, j + 3 < nw, sb, sa, k0, k1, v1, v0);
            }
            // This wave's last tile: loads still go on while the workgroup has more.
            if (j + 2 == nw) {
                iteration(Full{}, LoadsOn{}, j, false, sa, sb, k1, k0, v0, v1);
                ++j;
                if (j + 1 < ntiles) iteration(Last{}, LoadsOn{}, j, false, sb, sa, k0, k1, v1, v0);
                else iteration(Last{}, LoadsOff{}, j, false, sb, sa, k0, k1, v1, v0);
            } else {
                if (j + 1 < ntiles) iteration(Last{}, LoadsOn{}, j, false, sa, sb, k1, k0, v0, v1);
                else iteration(Last{}, LoadsOff{}, j, false, sa, sb, k1, k0, v0, v1);
            }
            ++j;
        }
        // Loads only, for the tiles other waves still compute.
        for (; j < niter; ++j) {
            wait_loads_and_barrier<0>();
            if (j + 1 < ntiles) {
                char *kdst = (j & 1) ? k1 : k0;
                char *vdst = (j & 1) ? v0 : v1;
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    load(krs, min(j + 2, ntiles - 1), kdst, i);
                    load(vrs, j + 1, vdst, i);
                }
            }
        }
        // The last iteration issues no loads and starts with a full wait, so
        // no LDS-direct load is in flight past this point.
    }

    // The K/V stages are free once every wave is past its last tile: each
    // wave stages its 32 output rows in its own 64 * D bytes of them.
    constexpr int TILE = 64 * D;  // bytes of one wave's 32 x D bf16 rows
    static_assert(TILE * ((NW + 3) / 4) <= T::BYTES, "staged rows fit the stages");
    char *stage = (wave & 3) == 0 ? lds_k0 : (wave & 3) == 1 ? lds_k1 : (wave & 3) == 2 ? lds_v0 : lds_v1;
    if constexpr (KH == 2) {
        // The two sets' states of the same rows merged by the rule for two
        // blocks ("从原始Softmax到在线Softmax" page).  Each wave and its
        // partner (the other set's wave on the same rows) share the two copies
        // of this stage: a wave puts the accumulator blocks its partner merges
        // into the partner's copy and its shift and sum at the end of its own.
        // With a bf16 output each wave then merges and stores half the
        // columns (set 0 the first half and the LSE); the float32 form is
        // merged and stored by set 0.
        constexpr int NB = D / 32, NBH = NB / 2;
        wait_loads_and_barrier<0>();
        char *own = stage + half * T::BYTES;
        char *partner = stage + (1 - half) * T::BYTES;
        float *ml_own = reinterpret_cast<float *>(own + T::BYTES - 512);
        const float *ml_partner = reinterpret_cast<const float *>(partner + T::BYTES - 512);
        static_assert(NB * 4096 <= T::BYTES && NBH * 4096 + 512 <= T::BYTES && 32 * D <= NBH * 4096,
                      "merge blocks, shift and sum, staged half rows fit a stage copy");
        if constexpr (SPLIT) {
            if (half == 1) {
                wt.template put_blocks<0, NB>(partner, lane);
                ml_own[lane] = wt.m_run;
                ml_own[64 + lane] = wt.l_run;
            }
            __syncthreads();
            if (half == 1) return;
            wt.template merge_blocks<0, NB, true>(own, ml_partner[lane], ml_partner[64 + lane], lane);
            wt.template store<true>(N, o + (size_t)bh * N * D, lse + (size_t)bh * N,
                                    part_o + ((size_t)sp * BH + bh) * N * D, part_lse + ((size_t)sp * BH + bh) * N);
        } else {
            if (half == 0) wt.template put_blocks<NBH, NBH>(partner, lane);
            else wt.template put_blocks<0, NBH>(partner, lane);
            ml_own[lane] = wt.m_run;
            ml_own[64 + lane] = wt.l_run;
            __syncthreads();
            const float m_o = ml_partner[lane], l_o = ml_partner[64 + lane];
            uint16_t *o_head = o + (size_t)bh * N * D;
            float *lse_head = lse + (size_t)bh * N;
            // (the staged half rows go where the partner's blocks were read)
            if (half == 0) {
                wt.template merge_blocks<0, NBH, true>(own, m_o, l_o, lane);
                wt.template store_cols<0, NBH>(N, q0 + wave * 32, o_head, lse_head, own, lane, true);
            } else {
                wt.template merge_blocks<NBH, NBH, false>(own, m_o, l_o, lane);
                wt.template store_cols<NBH, NBH>(N, q0 + wave * 32, o_head, lse_head, own, lane, false);
            }
        }
    } else if constexpr (SPLIT) {
        wt.template store<true>(N, o + (size_t)bh * N * D, lse + (size_t)bh * N,
                                part_o + ((size_t)sp * BH + bh) * N * D, part_lse + ((size_t)sp * BH + bh) * N);
    } else {
        wait_loads_and_barrier<0>();
        wt.store_rows(N, q0 + wave * 32, o + (size_t)bh * N * D, lse + (size_t)bh * N, stage + (wave >> 2) * TILE,
                      lane);
    }
}

#define ATTN_KERNEL_ARGS                                                                                       \
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,           \
        uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ part_o,                        \
        float *__restrict__ part_lse, int BH, int N, int M, float c, uint32_t qsign, int ntq, int splits,     \
        int tiles_per_split, const int32_t *__restrict__ kv_len, int H, int coff
#define ATTN_KERNEL_PASS \
    q, k, v, o, lse, part_o, part_lse, BH, N, M, c, qsign, ntq, splits, tiles_per_split, kv_len, H, coff

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(ATTN_KERNEL_ARGS) {
    attn_body<4, D, CAUSAL, SPLIT, false>(ATTN_KERNEL_PASS, nullptr, 0u, 0, 0, 0);
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_w8_kernel(ATTN_KERNEL_ARGS) {
    attn_body<8, D, CAUSAL, SPLIT, false>(ATTN_KERNEL_PASS, nullptr, 0u, 0, 0, 0);
}

// The four-wave width with the keys split between two sets of four waves on
// the same 128 rows (eight waves, two per SIMD), for problems whose 128-row
// workgroups would each run alone on a CU (one wave per SIMD).
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kh_kernel(ATTN_KERNEL_ARGS) {
    attn_body<4, D, CAUSAL, SPLIT, false, 2>(ATTN_KERNEL_PASS, nullptr, 0u, 0, 0, 0);
}

// Both widths with an additive score bias (staged through 8 KiB of LDS per
// wave: at d = 128 the four-wave width then needs 96 KiB, one workgroup per CU).
#define ATTN_BIAS_ARGS \
    ATTN_KERNEL_ARGS, const float *__restrict__ bias, uint32_t bias_bytes, int64_t bias_sb, int64_t bias_sh, int64_t bias_sn
template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void attn_fwd_bf16_bias_kernel(ATTN_BIAS_ARGS) {
    attn_body<4, D, CAUSAL, SPLIT, true>(ATTN_KERNEL_PASS, bias, bias_bytes, bias_sb, bias_sh, bias_sn);
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_w8_bias_kernel(ATTN_BIAS_ARGS) {
    attn_body<8, D, CAUSAL, SPLIT, true>(ATTN_KERNEL_PASS, bias, bias_bytes, bias_sb, bias_sh, bias_sn);
}

// Key halves with a bias, at d = 64 (each of the eight waves has its own bias
// stage: 64 KiB of LDS beside the 64 KiB of K/V stages).
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kh_bias_kernel(ATTN_BIAS_ARGS) {
    attn_body<4, 64, CAUSAL, false, true, 2>(ATTN_KERNEL_PASS, bias, bias_bytes, bias_sb, bias_sh, bias_sn);
}

template <int NW, int D, bool CAUSAL, bool SPLIT>
hipError_t launch_t(const AttnProblem &p, hipStream_t stream) {
    const int rows = 32 * NW;
    const int ntq = (p.N + rows - 1) / rows;
    const dim3 grid((unsigned)((int64_t)p.BH * ntq * p.splits));
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    const uint16_t *q = static_cast<const uint16_t *>(p.q), *k = static_cast<const uint16_t *>(p.k),
                   *v = static_cast<const uint16_t *>(p.v);
    uint16_t *o = static_cast<uint16_t *>(p.o);
    if (p.bias != nullptr) {
        if constexpr (NW == 8 && SPLIT)
            return hipErrorInvalidValue;  // never asked: partials with a bias take the four-wave width
        else if constexpr (NW == 8)
            hipLaunchKernelGGL((attn_fwd_bf16_w8_bias_kernel<D, CAUSAL, SPLIT>), grid, dim3(512), 0, stream, q, k, v, o,
                               p.lse, p.part_o, p.part_lse, p.BH, p.N, p.M, p.c, qsign, ntq, p.splits,
                               p.tiles_per_split, p.kv_len, p.H, p.causal_off, p.bias, p.bias_bytes, p.bias_sb,
                               p.bias_sh, p.bias_sn);
        else
            hipLaunchKernelGGL((attn_fwd_bf16_bias_kernel<D, CAUSAL, SPLIT>), grid, dim3(256), 0, stream, q, k, v, o,
                               p.lse, p.part_o, p.part_lse, p.BH, p.N, p.M, p.c, qsign, ntq, p.splits,
                               p.tiles_per_split, p.kv_len, p.H, p.causal_off, p.bias, p.bias_bytes, p.bias_sb,
                               p.bias_sh, p.bias_sn);
    } else if constexpr (NW == 8) {
        hipLaunchKernelGGL((attn_fwd_bf16_w8_kernel<D, CAUSAL, SPLIT>), grid, dim3(512), 0, stream, q, k, v, o, p.lse,
                           p.part_o, p.part_lse, p.BH, p.N, p.M, p.c, qsign, ntq, p.splits, p.tiles_per_split,
                           p.kv_len, p.H, p.causal_off);
    } else {
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, SPLIT>), grid, dim3(256), 0, stream, q, k, v, o, p.lse,
                           p.part_o, p.part_lse, p.BH, p.N, p.M, p.c, qsign, ntq, p.splits, p.tiles_per_split,
                           p.kv_len, p.H, p.causal_off);
    }
    return hipGetLastError();
}

template <int NW, int D>
hipError_t launch_d(const AttnProblem &p, hipStream_t stream) {
    // The partial-store form also writes a float32 o (one split).
    const bool split = p.splits > 1 || p.out_f32;
    if (p.causal) return split ? launch_t<NW, D, true, true>(p, stream) : launch_t<NW, D, true, false>(p, stream);
    return split ? launch_t<NW, D, false, true>(p, stream) : launch_t<NW, D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnProblem &p, hipStream_t stream) {
    // Also the kernel for calls with a bias.
    return p.d == 64 ? launch_d<4, 64>(p, stream) : launch_d<4, 128>(p, stream);
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch_kh_t(const AttnProblem &p, hipStream_t stream) {
    const int ntq = (p.N + 127) / 128;
    if constexpr (D == 64 && !SPLIT) {
        if (p.bias != nullptr) {
            hipLaunchKernelGGL((attn_fwd_bf16_kh_bias_kernel<CAUSAL>), dim3((unsigned)((int64_t)p.BH * ntq)), dim3(512),
                               0, stream, static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                               static_cast<const uint16_t *>(p.v), static_cast<uint16_t *>(p.o), p.lse, p.part_o,
                               p.part_lse, p.BH, p.N, p.M, p.c, p.negate_q ? 0x80008000u : 0u, ntq, 1,
                               p.tiles_per_split, p.kv_len, p.H, p.causal_off, p.bias, p.bias_bytes, p.bias_sb,
                               p.bias_sh, p.bias_sn);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attn_fwd_bf16_kh_kernel<D, CAUSAL, SPLIT>), dim3((unsigned)((int64_t)p.BH * ntq)), dim3(512), 0,
                       stream, static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                       static_cast<const uint16_t *>(p.v), static_cast<uint16_t *>(p.o), p.lse, p.part_o, p.part_lse,
                       p.BH, p.N, p.M, p.c, p.negate_q ? 0x80008000u : 0u, ntq, 1, p.tiles_per_split, p.kv_len, p.H,
                       p.causal_off);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_w8(const AttnProblem &p, hipStream_t stream) {
    // Single pass only (a float32 o through the partial-store form, without a
    // bias): the front end never asks this width for split partials.
    if (p.splits != 1 || (p.out_f32 && p.bias != nullptr)) return hipErrorInvalidValue;
    if (p.out_f32) {
        if (p.d == 64) return p.causal ? launch_t<8, 64, true, true>(p, stream) : launch_t<8, 64, false, true>(p, stream);
        return p.causal ? launch_t<8, 128, true, true>(p, stream) : launch_t<8, 128, false, true>(p, stream);
    }
    if (p.d == 64) return p.causal ? launch_t<8, 64, true, false>(p, stream) : launch_t<8, 64, false, false>(p, stream);
    return p.causal ? launch_t<8, 128, true, false>(p, stream) : launch_t<8, 128, false, false>(p, stream);
}

hipError_t launch_attn_bf16_kh(const AttnProblem &p, hipStream_t stream) {
    // Single pass (a float32 o through the partial-store form); a bias only
    // at d = 64 with a bf16 o.
    if (p.splits != 1 || (p.bias != nullptr && (p.d != 64 || p.out_f32))) return hipErrorInvalidValue;
    if (p.out_f32) {
        if (p.d == 64) return p.causal ? launch_kh_t<64, true, true>(p, stream) : launch_kh_t<64, false, true>(p, stream);
        return p.causal ? launch_kh_t<128, true, true>(p, stream) : launch_kh_t<128, false, true>(p, stream);
    }
    if (p.d == 64) return p.causal ? launch_kh_t<64, true, false>(p, stream) : launch_kh_t<64, false, false>(p, stream);
    return p.causal ? launch_kh_t<128, true, false>(p, stream) : launch_kh_t<128, false, false>(p, stream);
}

}  // namespace osa
