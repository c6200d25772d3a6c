// Shared device code of the bf16 attention kernels for gfx950: operand
// layouts, LDS swizzle, LDS-direct loads and the per-wave pieces of the
// online-softmax recurrence (scores, masking, probabilities against a lazily
// moved shift, the exact fallback, the epilogue).
//
// Recurrence: per query row a running shift m and running exponential sum l;
// each new key block rescales l and the unnormalised accumulator o~ by
// e^{m_old - m_new} when the shift moves and adds the block's terms; finally
// o = o~ / l and LSE = m + log l.  Sources: "从原始Softmax到在线Softmax" page,
// online softmax derivation (m, l, o~ recurrences) and LSE definition;
// "Online Softmax and Flash Attention" page, eq. (8) and the fused loop of
// eq. (20)-(22).
//
// One wave owns 32 query rows.  Scores are computed transposed,
// S^T = K Q^T on v_mfma_f32_32x32x16_bf16, so each lane owns one query and 16
// keys per 32x32 block: row max and row sum are in-lane plus one exchange
// between the wave halves (v_permlane32_swap).  The K rows fed to the MFMA are
// permuted (bits 2 and 3 of the row index swapped) so the accumulator
// registers forming the next MFMA's B operand hold 8 consecutive keys: P^T
// goes from accumulators to operands in place.  O^T = V^T P^T takes its V^T
// operand from ds_read_b64_tr_b16 (a transposing LDS read) on the
// natural-layout V tile, so the rescale and the final 1/l are per-lane
// scalars.  Scores stay in base-2 units: c = |scale| * log2(e) (at least the
// smallest normal float, so masked scores of -inf give exactly 0) is folded
// into one FMA before v_exp_f32; a negative scale flips q's sign bit on load.
//
// Lazy shift: the probabilities of a tile are first formed against the
// current shift, with no row max.  Only when some row's tile sum exceeds 2^40
// or is not finite, or a row has no shift yet (its first tile with a visible
// key), does the wave take the exact path: row max, new shift, rescale of l
// and o~, and the probabilities again.  Any shift gives the same softmax as
// long as numerator and denominator share it and nothing overflows.  A
// tile's scores are brought to base-2 units against the shift (x = c*s - m)
// before its softmax, while the previous tile's P.V MFMAs run.
//
// An additive score bias (an elementwise mask(), which eq. (8) leaves open)
// is staged through LDS per wave and folded into the scores in the same FMA:
// x = c * s + (log2(e) * bias - m).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace osa {
namespace bf16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BC = kBf16KeyTile;  // keys per tile
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E = 1.4426950408889634f;
// Largest tile sum kept against a stale shift: 2^40.  Probabilities stay at
// most 2^40 (bf16 keeps its 8-bit relative precision at any magnitude); the
// fp32 sum and accumulator, at most 2^40 x |v| per tile, stay below overflow
// for |v| < 2^68 over a million tiles.  Against a limit of 2^16 it spares
// exact paths on peaked softmaxes (1x8x16384^2 causal with logits up to +-54:
// -4.1 % per launch at 2^30, about -5 % at 2^40 and at 2^60; 2x16x4096^2
// causal with N(0,1) inputs: unchanged).
constexpr float SHIFT_SUM_LIMIT = 1099511627776.f;
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer descriptor, 32-bit data

template <int D>
struct Tile {
    static constexpr int RB = 2 * D;        // bytes per K/V row
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int BYTES = BC * RB;   // bytes per K (or V) tile
    static constexpr int ROWS_PER_LOAD = 1024 / RB;
    static constexpr int LOADS = BYTES / 1024;  // 1 KiB LDS-direct loads per tile
};

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).
// d = 128 (one row per 256-byte bank line): 16 consecutive rows get 16
// distinct values (K reads: 32 rows, one chunk column), and rows 4m..4m+3
// move whole 64-byte groups apart (V transposed reads: 4 rows x 64 bytes).
// d = 64 (two rows per bank line): the same two properties per row parity.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Row r of a 32-row MFMA A operand reads K row perm32(r): bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until at most N LDS-direct loads of this wave are outstanding, then
// synchronise the workgroup.  The memory clobber keeps LDS accesses on their
// side of the barrier.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One LDS-direct buffer load: each lane's 16 bytes at byte offset voff of the
// buffer land at LDS address lds_base + 16*lane.  Issued as inline assembly so
// that the compiler does not track these writes (it would otherwise wait for
// every outstanding load before each LDS read); completion is ordered
// explicitly by wait_loads_and_barrier.  No memory clobber: the loads may be
// scheduled among the LDS reads of other stages; they stay on their side of
// the (volatile) barrier statements.  M0 holds the LDS base of the load: the
// "{m0}" operand makes the compiler set it (and know that it did).  A write
// of M0 needs one wait state before an LDS-direct load reads it, and the
// compiler's hazard check does not look inside the asm: hence the s_nop.
__device__ __forceinline__ void lds_direct_load16(u32x4 rsrc, uint32_t lds_base, int voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_base));
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Raw buffer descriptor over nbytes at p (wave-uniform); loads past nbytes return 0.
__device__ __forceinline__ u32x4 make_rsrc(const void *p, uint32_t nbytes) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)), nbytes, kBufferWord3};
}

// Copies of one K (or V) tile into LDS are split into Tile::LOADS loads of
// 1 KiB; load i covers rows ROWS_PER_LOAD*i .. and lane l writes the block's
// byte 16*l, i.e. row ROWS_PER_LOAD*i + l/CPR, physical chunk l%CPR.  Returns
// the byte offset, within a tile, of the source chunk of this lane.
template <int D>
__device__ __forceinline__ int load_src_offset(int i, int lane) {
    using T = Tile<D>;
    const int row = T::ROWS_PER_LOAD * i + lane / T::CPR;
    const int lc = (lane % T::CPR) ^ swz<D>(row);
    return row * T::RB + lc * 16;
}

// The per-wave state and tile math for 32 query rows.
template <int D, bool CAUSAL>
struct WaveTile {
    using T = Tile<D>;
    bf16x8 qop[D / 16];   // Q^T operand: lane (query l32, half hh) holds q[row][16*kk + 8*hh .. +8]
    f32x16 oacc[D / 32];  // O^T accumulator: register r of block db is d index 32*db + 8*(r/4) + 4*hh + r%4
    float m_run;          // running shift (max), base-2 units
    float l_run;          // this lane's share of the running sum
    int k_off[D / 16];    // K operand byte offsets (block cb adds 32 rows)
    int v_off[2][D / 32]; // V^T operand byte offsets (key chunk t4 adds 16 rows)
    int l32, hh, qrow, wq_lo;
    int coff;  // causal offset: key j visible for query i iff j <= i + coff
    float c;

    __device__ __forceinline__ void init(const uint16_t *qh, int N, int row0, int lane, float c_, uint32_t qsign,
                                         int coff_) {
        l32 = lane & 31;
        hh = lane >> 5;
        wq_lo = row0;
        qrow = row0 + l32;
        coff = coff_;
        c = c_;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < N) {
                x = *reinterpret_cast<const u32x4 *>(qh + (size_t)qrow * D + 16 * kk + 8 * hh);
                x ^= qsign;
            }
            qop[kk] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
        m_run = NEG_INF;
        l_run = 0.f;
        {
            const int row = perm32(l32);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = row * T::RB + (((2 * kk + hh) ^ swz<D>(row)) * 16);
        }
        // Transposing read r of dv block db: lane l of 16-lane group G points at
        // key row 8*(G/2) + 4*r + (l%16)/4 and dv 32*db + 16*(G%2) + 4*(l%4); the
        // read returns to lane i of the group the 4 keys of that group at dv
        // 32*db + 16*(G%2) + i.
        const int G = lane >> 4, L = lane & 15;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int row = 8 * (G >> 1) + 4 * r + (L >> 2);
                const int dv = 32 * db + 16 * (G & 1) + 4 * (L & 3);
                v_off[r][db] = row * T::RB + (((dv >> 3) ^ swz<D>(row)) * 16) + (dv & 7) * 2;
            }
    }

    // One MFMA step kk of S^T = K Q^T for both 32-key blocks.
    __device__ __forceinline__ void score_step(const char *ks, int kk, f32x16 (&s)[2]) const {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(ks + cb * 32 * T::RB + k_off[kk]);
            s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], s[cb], 0, 0, 0);
        }
    }

    // Masked scores become -inf (then P is exactly 0).
    __device__ __forceinline__ void mask(int kv0, int ke, f32x16 (&s)[2]) const {
        // Accumulator register r of block cb holds key kv0 + 32*cb + 16*(r/8) + 8*hh + r%8.
        const bool need_mask = (kv0 + BC > ke) || (CAUSAL && kv0 + BC - 1 > wq_lo + coff);
        if (need_mask) {
            // Key kv0 + 8*hh + off is visible iff off <= lim (key < ke, and
            // key <= qrow + coff when causal): one compare with a constant per score.
            int lim = ke - 1 - kv0 - 8 * hh;
            if (CAUSAL) lim = min(lim, qrow + coff - kv0 - 8 * hh);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 32 * cb + 16 * (r >> 3) + (r & 7);
                    s[cb][r] = off <= lim ? s[cb][r] : NEG_INF;
                }
        }
    }

    // Additive bias, staged through an 8 KiB LDS region of this wave.  The
    // 32 bias values of a lane's scores of the tile at kv0 form eight runs of
    // four keys (register r of block cb is key kv0 + 32*cb + 16*(r/8) + 8*hh
    // + r%8, so run t = 4*cb + 2*(r/8) + (r%8)/4); LDS-direct load t has every
    // lane fetch its own run t from its query's bias row (byte offset row_off
    // in the buffer brs), which lands at region + 1024*t + 16*lane.  The
    // buffer's range check returns 0 past the bias (those keys are masked).
    __device__ __forceinline__ void bias_dma(const u32x4 &brs, uint32_t row_off, int kv0, char *region) const {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int key = kv0 + 32 * (t >> 2) + 16 * ((t >> 1) & 1) + 8 * hh + 4 * (t & 1);
            lds_direct_load16(brs, lds_addr(region + 1024 * t), (int)(row_off + 4u * (uint32_t)key));
        }
    }

    // Run t of the staged bias into s: s <- c_scale * s + log2(e) * bias - sh,
    // the scores in base-2 units with the bias added, against shift sh.
    __device__ __forceinline__ void bias_apply(const char *region, int t, int lane, f32x16 (&s)[2],
                                               float c_scale, float sh) const {
        const f32x4 b = *reinterpret_cast<const f32x4 *>(region + 1024 * t + 16 * lane);
        const int cb = t >> 2, r0 = 8 * ((t >> 1) & 1) + 4 * (t & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[cb][r0 + e] = __builtin_fmaf(s[cb][r0 + e], c_scale, __builtin_fmaf(b[e], LOG2E, -sh));
    }

    // P = 2^(c*s - m) for shift m, rounded to bf16 as the operands of P.V;
    // returns their sum in fp32 (v_dot2c_f32_bf16 against (1,1)).  l sums the
    // same rounded values, so o = o~/l is a weighted mean with consistent
    // weights: with a peaked softmax the rounding of the dominant weights
    // cancels.
    __device__ __forceinline__ float probs(const f32x16 (&s)[2], float m, bf16x8 (&pop)[BC / 16]) const {
        return probs_scaled(s, c, m, pop);
    }
    // The same with the scale given: P = 2^(cs*s - m).
    __device__ __forceinline__ float probs_scaled(const f32x16 (&s)[2], float cs, float m, bf16x8 (&pop)[BC / 16]) const {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float lsum[2] = {0.f, 0.f};  // two chains of v_dot2c
#pragma unroll
        for (int t4 = 0; t4 < BC / 16; ++t4) {
            f32x8 p;
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = exp2_fast(__builtin_fmaf(s[t4 >> 1][8 * (t4 & 1) + i], cs, -m));
            pop[t4] = __builtin_convertvector(p, bf16x8);
            float &acc = lsum[t4 & 1];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pop[t4], pop[t4], 0, 1), ones, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pop[t4], pop[t4], 2, 3), ones, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pop[t4], pop[t4], 4, 5), ones, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pop[t4], pop[t4], 6, 7), ones, acc, false);
        }
        return lsum[0] + lsum[1];
    }

    // K operand of score MFMA `slot` (32-key block slot&1, feature step slot>>1).
    __device__ __forceinline__ bf16x8 kread(const char *ks, int slot) const {
        return *reinterpret_cast<const bf16x8 *>(ks + (slot & 1) * 32 * T::RB + k_off[slot >> 1]);
    }

    // V^T operand of P.V MFMA `slot` (key group slot / (D/32), d block
    // slot % (D/32)): two transposing reads.
    __device__ __forceinline__ bf16x8 vread(const char *vs, int slot) const {
        const int t4 = slot / (D / 32), db = slot % (D / 32);
        const char *vt = vs + t4 * 16 * T::RB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_off[0][db]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_off[1][db]));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }

    // The shift a tile's scores are taken against before the tile is seen:
    // the running one, or 0 for a row that has no shift yet (no visible key
    // so far).
    __device__ __forceinline__ float shift_base() const { return m_run == NEG_INF ? 0.f : m_run; }

    // Scores e, e+1 (e even) brought to base-2 units against shift sh, in
    // place: x = c*s - sh.  Done for the next tile while the P.V MFMAs of this
    // one run, so the score phase is left with the exponentials
    // (prob_pair_x); a masked -inf stays -inf.
    __device__ __forceinline__ void shift_pair(f32x16 (&s)[2], int e, float sh) const {
        s[e >> 4][e & 15] = __builtin_fmaf(s[e >> 4][e & 15], c, -sh);
        s[(e + 1) >> 4][(e + 1) & 15] = __builtin_fmaf(s[(e + 1) >> 4][(e + 1) & 15], c, -sh);
    }

    // Probabilities of shifted scores e, e+1 (e even; register r of block cb
    // is score 16*cb + r): P = 2^x, packed to bf16 into word e/2 of popw,
    // their sum (of the rounded values) added to acc.
    __device__ __forceinline__ void prob_pair_x(const f32x16 (&x)[2], int e, uint32_t (&popw)[BC / 16][4],
                                                float &acc) const {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        const float p0 = exp2_fast(x[e >> 4][e & 15]);
        const float p1 = exp2_fast(x[(e + 1) >> 4][(e + 1) & 15]);
        const bf16x2 pp = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
        popw[e >> 3][(e & 7) >> 1] = __builtin_bit_cast(uint32_t, pp);
        acc = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc, false);
    }

    // A row's first shift from its first tile of shifted scores x = c*s
    // (shift base 0, masked): m = max x, and x -= m in place.  A row with no
    // visible key there keeps no shift.
    __device__ __forceinline__ void first_shift(f32x16 (&x)[2]) {
        float mx = NEG_INF;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[cb][r]);
        mx = xhalf_max(mx);
        if (mx != NEG_INF) {
            m_run = mx;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) x[cb][r] -= mx;
        }
    }

    // Whether this lane's row needs the exact path for a tile of shifted
    // scores with probability sum lsum: the sum is above the limit or not
    // finite, or the row has no shift yet (its first tile: scores far below
    // the base 0 would otherwise underflow to a zero sum).
    __device__ __forceinline__ bool needs_exact_x(float lsum) const {
        return !(lsum <= SHIFT_SUM_LIMIT) || m_run == NEG_INF;
    }

    // Exact path for shifted scores x = c*s - sh (sh = shift_base()): the row
    // max of c*s is sh + max x; the shift becomes the larger of that and the
    // running one, and P = 2^(x - (m_new - sh)).  A row with no visible key
    // in this tile keeps its shift (and, with none so far, its zero state).
    __device__ __forceinline__ float exact_shift_x(const f32x16 (&x)[2], bf16x8 (&pop)[BC / 16], float &lsum) {
        float mx = NEG_INF;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[cb][r]);
        mx = xhalf_max(mx);
        const float sh = shift_base();
        const float m_new = mx == NEG_INF ? m_run : fmaxf(m_run, sh + mx);
        const float delta = mx == NEG_INF ? 0.f : m_new - sh;
        const float alpha = m_new == NEG_INF ? 1.f : exp2_fast(m_run - m_new);  // 0 when m_run was -inf
        m_run = m_new;
        lsum = probs_scaled(x, 1.f, delta, pop);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        return alpha;
    }

    // Final o = o~ / l (bf16) and LSE, with the rows staged in LDS so each
    // store instruction writes whole rows: region holds this wave's 32 x D
    // bf16 tile (16-byte chunk c of row r at chunk c ^ (r % CPR), conflict-
    // free for the writes and the reads); lane t then stores chunk t % CPR of
    // row t / CPR + ROWS*i.  The caller makes sure no wave still reads the
    // region.
    __device__ __forceinline__ void store_rows(int N, int q_wave, uint16_t *o_head, float *lse_head, char *region,
                                               int lane) {
        store_cols<0, D / 32>(N, q_wave, o_head, lse_head, region, lane, true);
    }

    // store_rows for the 32-column blocks [B0, B0 + NB) of the rows only (the
    // staged tile is 32 x 32*NB); the LSE is written if write_lse.
    template <int B0, int NB>
    __device__ __forceinline__ void store_cols(int N, int q_wave, uint16_t *o_head, float *lse_head, char *region,
                                               int lane, bool write_lse) {
        constexpr int W = 32 * NB;      // columns stored
        constexpr int CPR = W / 8;      // 16-byte chunks per staged row
        constexpr int ROWS = 64 / CPR;  // rows per store instruction
        const float l_tot = xhalf_sum(l_run);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (write_lse && qrow < N && hh == 0) lse_head[qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * LN2 : NEG_INF;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16 &a = oacc[B0 + b];
                f32x4 x = {a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
                const int chunk = (4 * b + g) ^ (l32 % CPR);
                *reinterpret_cast<bf16x4 *>(region + l32 * (2 * W) + chunk * 16 + 8 * hh) = __builtin_convertvector(x, bf16x4);
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's rows are in LDS
        const int c = lane % CPR;
#pragma unroll
        for (int i = 0; i < 32 / ROWS; ++i) {
            const int r = lane / CPR + ROWS * i;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(region + r * (2 * W) + ((c ^ (r % CPR)) * 16));
            if (q_wave + r < N) *reinterpret_cast<u32x4 *>(o_head + (size_t)(q_wave + r) * D + 32 * B0 + 8 * c) = val;
        }
    }

    // Key halves: this wave's accumulator blocks [B0, B0 + NB) for its
    // partner wave (the other set, same rows) into xfer, 16 bytes per lane per
    // instruction (conflict-free).
    template <int B0, int NB>
    __device__ __forceinline__ void put_blocks(char *xfer, int lane) const {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16 &a = oacc[B0 + b];
                *reinterpret_cast<f32x4 *>(xfer + (4 * b + g) * 1024 + 16 * lane) =
                    f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
            }
    }

    // ... and the merge of the partner's state into this wave's: blocks
    // [B0, B0 + NB) from xfer (as put_blocks wrote them), the partner's shift
    // m_o and sum share l_o; the rule for two blocks of keys (the larger
    // shift, each side scaled by 2^(its shift - that one); a side without a
    // key (shift -inf) weighs 0).  Both waves of a pair evaluate every sum in
    // the same order, set 0's term first (SET0: this wave is in set 0), so
    // that whichever stores a column gives the same bits.
    template <int B0, int NB, bool SET0>
    __device__ __forceinline__ void merge_blocks(const char *xfer, float m_o, float l_o, int lane) {
        const float mm = fmaxf(m_run, m_o);
        const float w_me = m_run == NEG_INF ? 0.f : exp2_fast(m_run - mm);
        const float w_o = m_o == NEG_INF ? 0.f : exp2_fast(m_o - mm);
        const float w0 = SET0 ? w_me : w_o, w1 = SET0 ? w_o : w_me;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(xfer + (4 * b + g) * 1024 + 16 * lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float mine = oacc[B0 + b][4 * g + i];
                    const float x0 = SET0 ? mine : y[i], x1 = SET0 ? y[i] : mine;
                    oacc[B0 + b][4 * g + i] = __builtin_fmaf(x0, w0, x1 * w1);
                }
            }
        const float l0 = SET0 ? l_run : l_o, l1 = SET0 ? l_o : l_run;
        l_run = __builtin_fmaf(l0, w0, l1 * w1);
        m_run = mm;
    }

    // Final o = o~ / l and LSE; bf16 output or fp32 split partial.
    template <bool SPLIT>
    __device__ __forceinline__ void store(int N, uint16_t *o_head, float *lse_head, float *part_o_rows,
                                          float *part_lse_rows) {
        const float l_tot = xhalf_sum(l_run);
        if (qrow >= N) return;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float row_lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * LN2 : NEG_INF;
        if constexpr (!SPLIT) {
            uint16_t *orow = o_head + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                               oacc[db][4 * g + 3] * inv};
                    *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * g + 4 * hh) = __builtin_convertvector(x, bf16x4);
                }
            if (hh == 0) lse_head[qrow] = row_lse;
        } else {
            float *orow = part_o_rows + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                               oacc[db][4 * g + 3] * inv};
                    *reinterpret_cast<f32x4 *>(orow + 32 * db + 8 * g + 4 * hh) = x;
                }
            if (hh == 0) part_lse_rows[qrow] = row_lse;
        }
    }
};

}  // namespace bf16
}  // namespace osa
