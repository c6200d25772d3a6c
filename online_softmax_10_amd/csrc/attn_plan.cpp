// Host-side planning of an attention call (no HIP): argument validation,
// the work decomposition, the kernel choice and the split workspace size.
// Contracts of the public entry points are in include/attn.h; the internal
// interface is attn_plan.h.

#include "attn_plan.h"

#include <float.h>
#include <math.h>
#include <stdint.h>

namespace osa {
namespace {

constexpr int64_t kMaxBlocks = int64_t(1) << 24;  // grid.x * 256 threads stays below 2^32
constexpr int64_t kI32Max = 0x7fffffff;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

struct Plan {
    // SMALL: single pass of the small fp32 kernel (keys split inside a workgroup).
    enum Kind { SINGLE, SPLIT, DECODE, SMALL } kind;
    int splits;
    int tiles_per_split;  // in units of the chosen kernel's key tile
};

// Work decomposition.  num_splits: 0 = choose, 1 = single pass, >= 2 = split.
// Calls with a bias never take the decode kernel.
// A split costs a workspace, the merge kernel and their host calls -- about
// 15-20 us per call on MI355X against a single pass of the same small
// problem.  It pays only when a workgroup's key loop is long: measured on
// twelve shapes (256-8192 queries, 256-16384 keys, d = 64 and 128, causal or
// not) the single pass won below 64 units of work per query tile and the split
// above 128, a unit being 64 keys at d = 64 in bf16; the fp32 kernel (matrix
// rate 1/16 of bf16) counts 32 units per bf16 unit.
constexpr int64_t kMinSplitUnits = 96;

Plan plan_for(int64_t BH, int64_t N, int64_t M, int d, bool bf16, int num_splits, bool bias = false) {
    const bool few_queries = N <= kDecodeMaxQueries && !bias;
    if (num_splits == 1) return Plan{Plan::SINGLE, 1, 0};
    if (few_queries) {
        // Decode shape: stream K/V with enough workgroups in flight; each split
        // keeps at least 256 keys.
        const int tile = kDecodeKeyTile;
        int s = num_splits;
        if (s == 0) {
            s = ceil_div(2048, BH);
            const int cap = ceil_div(M, 256);
            if (s > cap) s = cap;
            if (s > ATTN_MAX_SPLITS) s = ATTN_MAX_SPLITS;
            if (s < 1) s = 1;
        }
        const int tps = ceil_div(ceil_div(M, s), tile);
        return Plan{Plan::DECODE, s, tps};
    }
    const int tile = bf16 ? kBf16KeyTile : kF32KeyTile;
    const int row_tiles = ceil_div(N, 128);
    // Small fp32 problems that cannot fill the chip with 128-row workgroups,
    // with at most kF32SmallMaxKeys keys (8 tiles per wave of the small
    // kernel): one launch, the keys split among the waves of each 16-row
    // workgroup.
    if (!bf16 && !bias && num_splits == 0 && BH * row_tiles < 256 && M <= kF32SmallMaxKeys)
        return Plan{Plan::SMALL, 1, 0};
    int s = num_splits;
    if (s == 0) {
        // Split only when the query tiles alone cannot fill the 256 compute
        // units and the key range is long enough to share out.
        const int64_t wgs = BH * row_tiles;
        if (wgs >= 256) return Plan{Plan::SINGLE, 1, 0};
        const int64_t units = ((M + 63) / 64) * (d / 64) * (bf16 ? 1 : 32);
        if (units < kMinSplitUnits) return Plan{Plan::SINGLE, 1, 0};
        s = ceil_div(512, wgs);
        const int cap = ceil_div(M, 4 * tile);
        if (s > cap) s = cap;
        if (s > ATTN_MAX_SPLITS) s = ATTN_MAX_SPLITS;
        if (s <= 1) return Plan{Plan::SINGLE, 1, 0};
    }
    const int tps = ceil_div(ceil_div(M, s), tile);
    return Plan{Plan::SPLIT, s, tps};
}

int validate_args(const void *q, const void *k, const void *v, const void *o, const float *lse, int64_t B,
                  int64_t H, int64_t N, int64_t M, int d, float scale, int dtype, int num_splits,
                  const attn_mask *mask) {
    if (B < 0 || H < 0 || N < 0 || M < 0) return ATTN_ERR_SHAPE;
    if (mask && (mask->causal < ATTN_CAUSAL_NONE || mask->causal > ATTN_CAUSAL_BOTTOM_RIGHT)) return ATTN_ERR_MASK;
    if (mask && mask->kv_len && (reinterpret_cast<uintptr_t>(mask->kv_len) & 3u)) return ATTN_ERR_ALIGN;
    if (mask && mask->bias) {
        if (mask->bias_stride_b < 0 || mask->bias_stride_h < 0 || mask->bias_stride_n < 0) return ATTN_ERR_SHAPE;
        if (!aligned16(mask->bias) || ((mask->bias_stride_b | mask->bias_stride_h | mask->bias_stride_n) & 3))
            return ATTN_ERR_ALIGN;
    }
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_BF16_OUT_F32) return ATTN_ERR_DTYPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
    if (B == 0 || H == 0 || N == 0) return ATTN_OK;  // nothing to compute
    if (M < 1) return ATTN_ERR_SHAPE;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
    if (B > kI32Max || H > kI32Max || B * H > kI32Max) return ATTN_ERR_OVERFLOW;
    if (N > kI32Max / d || M > kI32Max / d) return ATTN_ERR_OVERFLOW;
    if (B * H * ceil_div(N, 128) > kMaxBlocks) return ATTN_ERR_OVERFLOW;
    return ATTN_OK;
}

MainKernel main_kernel(const Plan &plan, int64_t BH, int64_t N, int64_t M, int d, bool bf16, bool bias = false,
                       bool out_f32 = false) {
    if (plan.kind == Plan::DECODE) return MainKernel::DECODE;
    if (plan.kind == Plan::SMALL) return MainKernel::F32_SMALL;
    if (!bf16) return MainKernel::F32;
    // fp32 output with a bias: the four-wave width (its partial-store form
    // fits the registers; the eight-wave one would spill).
    if (bias && out_f32) return MainKernel::BF16_BIAS;
    // The eight-wave kernel shares each K/V tile among 256 rows; use it for
    // single-pass problems whose 256-row tiles alone give every compute unit
    // a workgroup.
    if (plan.kind == Plan::SINGLE && BH * ceil_div(N, kBf16WideRows) >= 256)
        return bias ? MainKernel::BF16_8W_BIAS : MainKernel::BF16_8W;
    // A single pass whose 128-row workgroups run one per CU (one wave per
    // SIMD) over enough key tiles: the keys of each workgroup split between
    // two sets of four waves, two waves per SIMD.  Measured against the
    // four-wave width on 4x8x1024xM, d = 64: M = 384 +5.5 %, 512 +2 %, 640
    // +1 %, 768 -1.5 %, 1024 -4 % (causal -8 %); d = 128: M = 512 +6 %, 1024
    // -0.3 % (1x16x1024^2: -3 %, causal -4 %).
    // With a bias only at d = 64, where the eight waves' bias stages fit in
    // LDS beside the K/V stages (and never with a float32 o and a bias, taken
    // above).
    if (plan.kind == Plan::SINGLE && (!bias || d == 64) && BH * ceil_div(N, 128) <= 256 &&
        ceil_div(M, kBf16KeyTile) >= (d == 64 ? kBf16KhMinTiles64 : kBf16KhMinTiles128))
        return bias ? MainKernel::BF16_KH_BIAS : MainKernel::BF16_KH;
    return bias ? MainKernel::BF16_BIAS : MainKernel::BF16_4W;
}

}  // namespace

const char *main_kernel_name(MainKernel k) {
    switch (k) {
    case MainKernel::F32: return "attn_fwd_f32_kernel";
    case MainKernel::F32_SMALL: return "attn_fwd_f32_small_kernel";
    case MainKernel::BF16_4W: return "attn_fwd_bf16_kernel";
    case MainKernel::BF16_8W: return "attn_fwd_bf16_w8_kernel";
    case MainKernel::BF16_KH: return "attn_fwd_bf16_kh_kernel";
    case MainKernel::DECODE: return "attn_decode_kernel";
    case MainKernel::BF16_BIAS: return "attn_fwd_bf16_bias_kernel";
    case MainKernel::BF16_8W_BIAS: return "attn_fwd_bf16_w8_bias_kernel";
    case MainKernel::BF16_KH_BIAS: return "attn_fwd_bf16_kh_bias_kernel";
    }
    return "";
}


int validate_attn(const void *q, const void *k, const void *v, const void *o, const float *lse, int64_t B,
                  int64_t H, int64_t N, int64_t M, int d, float scale, int dtype, int num_splits,
                  const attn_mask *mask) {
    return validate_args(q, k, v, o, lse, B, H, N, M, d, scale, dtype, num_splits, mask);
}

int plan_attn(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H, int64_t N,
              int64_t M, int d, float scale, const attn_mask *mask, int dtype, int num_splits, PlannedCall *out,
              bool *nothing) {
    *nothing = false;
    const int rc = validate_args(q, k, v, o, lse, B, H, N, M, d, scale, dtype, num_splits, mask);
    if (rc != ATTN_OK) return rc;
    if (B == 0 || H == 0 || N == 0) {
        *nothing = true;
        return ATTN_OK;
    }
    const bool bf16 = dtype != ATTN_F32;
    const int64_t BH = B * H;
    AttnProblem p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.BH = (int)BH;
    p.N = (int)N;
    p.M = (int)M;
    p.d = d;
    p.H = (int)H;
    const int causal = mask ? mask->causal : ATTN_CAUSAL_NONE;
    p.kv_len = mask ? mask->kv_len : nullptr;
    p.bias = mask ? mask->bias : nullptr;
    if (p.bias) {
        p.bias_sb = mask->bias_stride_b;
        p.bias_sh = mask->bias_stride_h;
        p.bias_sn = mask->bias_stride_n;
        // The kernels address the bias with 32-bit byte offsets from its base.
        const double extent = 4.0 * ((double)(B - 1) * p.bias_sb + (double)(H - 1) * p.bias_sh +
                                     (double)(N - 1) * p.bias_sn + (double)M);
        if (extent > 4294967296.0 - 4096.0) return ATTN_ERR_OVERFLOW;
        p.bias_bytes = (uint32_t)extent;
    }
    p.causal_off = causal == ATTN_CAUSAL_BOTTOM_RIGHT ? (int)(M - N) : 0;
    // Scores are kept in base-2 units.  c is at least the smallest normal float
    // so that a masked score (-inf) times c is -inf, never NaN; for scale = 0
    // this changes the (uniform) result by less than 2^-100 relative.
    p.c = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
    p.negate_q = signbit(scale) != 0;
    p.causal = causal != ATTN_CAUSAL_NONE;
    p.out_f32 = dtype == ATTN_BF16_OUT_F32;

    const Plan plan = plan_for(BH, N, M, d, bf16, num_splits, p.bias != nullptr);
    const int64_t blocks = plan.kind == Plan::DECODE  ? BH * plan.splits
                           : plan.kind == Plan::SMALL ? BH * ceil_div(N, 16)
                                                      : BH * ceil_div(N, 128) * plan.splits;
    if (blocks > kMaxBlocks) return ATTN_ERR_OVERFLOW;
    out->kernel = main_kernel(plan, BH, N, M, d, bf16, p.bias != nullptr, p.out_f32);
    out->bf16 = bf16;
    p.splits = plan.splits;
    p.tiles_per_split = plan.tiles_per_split;
    out->split = plan.kind == Plan::SPLIT || plan.kind == Plan::DECODE;
    out->workspace_bytes = 0;
    if (!out->split) {
        p.tiles_per_split = ceil_div(M, bf16 ? kBf16KeyTile : kF32KeyTile);
        if (p.out_f32) {
            // One "split" whose normalised fp32 partial and LSE are the outputs.
            p.part_o = static_cast<float *>(o);
            p.part_lse = lse;
        }
    } else {
        // Partials: o [splits, BH, N, d] fp32, then lse [splits, BH, N] fp32.
        const size_t rows = (size_t)BH * (size_t)N;
        out->workspace_bytes = (size_t)plan.splits * rows * ((size_t)d + 1) * sizeof(float);
    }
    out->p = p;
    return ATTN_OK;
}

}  // namespace osa

extern "C" {

const char *attn_fwd_plan(int64_t B, int64_t H, int64_t N, int64_t M, int d, int dtype, int num_splits,
                          int *splits) {
    using namespace osa;
    if (splits) *splits = 0;
    if (B < 1 || H < 1 || N < 1 || M < 1) return nullptr;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_BF16_OUT_F32) return nullptr;
    if (d != 64 && d != 128) return nullptr;
    if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return nullptr;
    if (B > kI32Max || H > kI32Max || B * H > kI32Max || N > kI32Max / d || M > kI32Max / d) return nullptr;
    const bool bf16 = dtype != ATTN_F32;
    const Plan plan = plan_for(B * H, N, M, d, bf16, num_splits);
    if (splits) *splits = plan.splits;
    return main_kernel_name(main_kernel(plan, B * H, N, M, d, bf16, false, dtype == ATTN_BF16_OUT_F32));
}

const char *attn_strerror(int code) {
    switch (code) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (negative size, or M < 1 / n < 1 with work to do)";
    case ATTN_ERR_HEADDIM: return "unsupported head dim (compiled for d = 64 and d = 128)";
    case ATTN_ERR_DTYPE: return "unsupported dtype (ATTN_F32, ATTN_BF16 or ATTN_BF16_OUT_F32)";
    case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ATTN_ERR_OVERFLOW: return "sizes exceed the kernels' index range";
    case ATTN_ERR_HIP: return "HIP launch or allocation failed";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_SPLITS: return "num_splits outside [0, ATTN_MAX_SPLITS]";
    case ATTN_ERR_MASK: return "unknown causal mode in attn_mask";
    case ATTN_ERR_WORKSPACE: return "the split workspace exceeds the static scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
    }
}

}  // extern "C"
