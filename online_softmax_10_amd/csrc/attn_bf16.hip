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
// Mapping to the chip (specific to this design, not the pages'):
//  * A workgroup owns BR = 128 query rows of one (batch, head): four 64-wide
//    waves, 32 rows each; two workgroups share a compute unit, so each SIMD
//    runs two waves whose MFMA and VALU phases overlap.  A wave keeps its 32
//    query rows in VGPRs as the B operand of v_mfma_f32_32x32x16_bf16.
//  * Key tiles of BC = 64 keys are copied HBM -> LDS by buffer loads with
//    the LDS-direct path (no staging registers), into two LDS stages: tile
//    t+1 streams in while tile t is used.  The buffer range check returns
//    zeros past key M, so ragged tails need no clamping.  Rows are stored in
//    natural layout with an XOR swizzle of their 16-byte chunks.
//  * Scores are computed transposed, S^T = K Q^T, so each lane owns one query
//    and 16 keys per 32x32 block: row max and row sum are in-lane plus one
//    exchange between the wave halves (v_permlane32_swap).  The K rows fed to
//    the MFMA are permuted (bits 2 and 3 of the row index swapped) so the
//    accumulator registers forming the next MFMA's B operand hold 8
//    consecutive keys: P^T goes from accumulators to operands in place.
//  * O^T = V^T P^T: the V^T operand is read from the natural-layout V tile
//    with ds_read_b64_tr_b16 (a transposing LDS read), so V is never
//    transposed in registers; each lane again owns one query, so the rescale
//    and the final 1/l are per-lane scalars.
//  * Scores stay in base-2 units: c = |scale| * log2(e) (at least the
//    smallest normal float, so masked scores of -inf always give exactly 0)
//    is folded into one FMA before v_exp_f32; a negative scale flips q's sign
//    bit on load.  The running max only moves when a tile exceeds it by
//    2^RESCALE_SLACK, so most tiles skip the rescale of l and o~.

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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int NW = 4;            // waves per workgroup
constexpr int NT = 64 * NW;      // threads per workgroup
constexpr int BR = 32 * NW;      // query rows per workgroup
constexpr int BC = kBf16KeyTile; // keys per tile
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994531f;
constexpr float RESCALE_SLACK = 8.f;            // base-2 units: probabilities stay below 2^8
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer descriptor, 32-bit data

template <int D>
struct Layout {
    static constexpr int RB = 2 * D;                 // bytes per K/V row
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int TILE = BC * RB;             // bytes per K (or V) tile
    static constexpr int LOADS = TILE / 1024 / NW;   // 1 KiB LDS-direct loads per wave per tile
    static constexpr int ROWS_PER_LOAD = 1024 / RB;
    static_assert(LOADS * NW * 1024 == TILE, "tile split");
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
// scheduled among the LDS reads of the other stage; they stay on their side of
// the (volatile) barrier statements.  M0, the LDS base of the load, is a
// register the compiler reserves and keeps no live value in here.
__device__ __forceinline__ void lds_direct_load16(u32x4 rsrc, uint32_t lds_base, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "s"(lds_base), "v"(voff), "s"(rsrc));
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ part_o,
    float *__restrict__ part_lse, int BH, int N, int M, float c, uint32_t qsign, int ntq,
    int splits, int tiles_per_split) {
    using Lay = Layout<D>;
    __shared__ __attribute__((aligned(1024))) char lds_k0[Lay::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_k1[Lay::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v0[Lay::TILE];
    __shared__ __attribute__((aligned(1024))) char lds_v1[Lay::TILE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // Workgroup -> (head, split, query tile); heads vary fastest and the
    // longest causal tiles go first.
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
    if (CAUSAL) ke = min(ke, q0 + BR);
    const int ntiles = ke > kb ? (ke - kb + BC - 1) / BC : 0;

    const uint16_t *qh = q + (size_t)bh * N * D;
    // Buffer descriptors over this head's K and V; reads past key M return 0.
    const uint64_t kaddr = (uint64_t)(uintptr_t)(k + (size_t)bh * M * D);
    const uint64_t vaddr = (uint64_t)(uintptr_t)(v + (size_t)bh * M * D);
    const uint32_t nbytes = (uint32_t)M * Lay::RB;
    const u32x4 krs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)kaddr),
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(kaddr >> 32)), nbytes, kBufferWord3};
    const u32x4 vrs = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)vaddr),
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(vaddr >> 32)), nbytes, kBufferWord3};

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

    // LDS-direct loads: load i of this wave fills the 1 KiB block (wave*LOADS+i)
    // of the tile; lane l writes the block's byte 16*l, i.e. row
    // ROWS_PER_LOAD*(wave*LOADS+i) + l/CPR, physical chunk l%CPR.
    int ld_off[Lay::LOADS];  // byte offset within a tile of this lane's source chunk
#pragma unroll
    for (int i = 0; i < Lay::LOADS; ++i) {
        const int row = Lay::ROWS_PER_LOAD * (wave * Lay::LOADS + i) + lane / Lay::CPR;
        const int lc = (lane % Lay::CPR) ^ swz<D>(row);
        ld_off[i] = row * Lay::RB + lc * 16;
    }
    // Offsets are unsigned 32-bit byte offsets within the head (M*d < 2^31 elements).
    auto issue_tile = [&](int kv0, char *kdst, char *vdst) {
        const uint32_t base = (uint32_t)kv0 * Lay::RB;
#pragma unroll
        for (int i = 0; i < Lay::LOADS; ++i) {
            const int blk = (wave * Lay::LOADS + i) * 1024;
            const int off = (int)(base + (uint32_t)ld_off[i]);
            lds_direct_load16(krs, lds_addr(kdst + blk), off);
            lds_direct_load16(vrs, lds_addr(vdst + blk), off);
        }
    };

    // K operand byte offsets (block cb adds 32 rows): row perm32(l32), logical
    // chunk 2*kk + hh.
    int k_off[D / 16];
    {
        const int row = perm32(l32);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) k_off[kk] = row * Lay::RB + (((2 * kk + hh) ^ swz<D>(row)) * 16);
    }
    // V^T operand byte offsets for transposing read r of dv block db (key
    // chunk t4 adds 16 rows): lane l of 16-lane group G points at key row
    // 8*(G/2) + 4*r + (l%16)/4 and dv 32*db + 16*(G%2) + 4*(l%4); the read
    // returns to lane i of the group the 4 keys of that group at dv
    // 32*db + 16*(G%2) + i.
    int v_off[2][D / 32];
    {
        const int G = lane >> 4, L = lane & 15;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int row = 8 * (G >> 1) + 4 * r + (L >> 2);
                const int dv = 32 * db + 16 * (G & 1) + 4 * (L & 3);
                v_off[r][db] = row * Lay::RB + (((dv >> 3) ^ swz<D>(row)) * 16) + (dv & 7) * 2;
            }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = NEG_INF;  // running shift (max), base-2 units
    float l_run = 0.f;      // this lane's share of the running sum

    // Computes the tile at kv0 from stages (ks, vs) and, spread between its
    // score MFMAs, issues the loads of the next tile (at nkv0, if any) into
    // the other stages (nks, nvs).
    auto compute_tile = [&](int kv0, const char *ks, const char *vs, bool has_next, int nkv0, char *nks,
                            char *nvs) {
        // S^T = K Q^T for two 32-key blocks, accumulator chains interleaved.
        f32x16 s[2] = {f32x16{}, f32x16{}};
        const uint32_t nbase = (uint32_t)nkv0 * Lay::RB;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(ks + cb * 32 * Lay::RB + k_off[kk]);
                s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[kk], s[cb], 0, 0, 0);
            }
            constexpr int EVERY = (D / 16) / Lay::LOADS;
            if (has_next && kk % EVERY == 0) {
                const int i = kk / EVERY;
                const int blk = (wave * Lay::LOADS + i) * 1024;
                const int off = (int)(nbase + (uint32_t)ld_off[i]);
                lds_direct_load16(krs, lds_addr(nks + blk), off);
                lds_direct_load16(vrs, lds_addr(nvs + blk), off);
            }
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
        // Lazy rescale: any shift gives the same softmax as long as numerator
        // and denominator share it and nothing overflows.
        const float m_tile = mx * c;  // -inf stays -inf (c > 0)
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
                p[i] = exp2_fast(__builtin_fmaf(s[t4 >> 1][8 * (t4 & 1) + i], c, -m_use));
                lsum += p[i];
            }
            pop[t4] = __builtin_convertvector(p, bf16x8);
        }
        l_run = alpha * l_run + lsum;
        if (any_move) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }

        // O^T += V^T P^T; each V^T operand is two transposing reads.
#pragma unroll
        for (int t4 = 0; t4 < BC / 16; ++t4)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const char *vt = vs + t4 * 16 * Lay::RB;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_off[0][db]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + v_off[1][db]));
                const s16x8 w8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w8), pop[t4],
                                                                   oacc[db], 0, 0, 0);
            }
    };

    // Two LDS stages, one barrier per tile: the wait + barrier at the top of
    // tile t lands tile t (its loads were issued during tile t-1) and retires
    // every read of the other stage, which tile t's loads then refill.
    // Unrolled by two so each stage is a distinct LDS array.
    if (ntiles > 0) issue_tile(kb, lds_k0, lds_v0);
    for (int t = 0; t < ntiles; t += 2) {
        const int kv0 = kb + t * BC;
        wait_loads_and_barrier<0>();
        compute_tile(kv0, lds_k0, lds_v0, t + 1 < ntiles, kv0 + BC, lds_k1, lds_v1);
        if (t + 1 >= ntiles) break;
        wait_loads_and_barrier<0>();
        compute_tile(kv0 + BC, lds_k1, lds_v1, t + 2 < ntiles, kv0 + 2 * BC, lds_k0, lds_v0);
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
                *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * g + 4 * hh) = __builtin_convertvector(x, bf16x4);
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
