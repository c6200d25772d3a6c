// C-ABI front end of libattn.so: the HIP side of each entry point -- the
// launches of a call planned by attn_plan.cpp (validation, kernel choice and
// split heuristic, no HIP) and the stream-ordered split workspace.  The
// declarations and their contracts are in include/attn.h.

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"
#include "kernels.h"

namespace {

constexpr int64_t kI32Max = 0x7fffffff;

thread_local char g_detail[256] = "";

void set_detail(const char *what, hipError_t e) {
    snprintf(g_detail, sizeof(g_detail), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

void osa::set_hip_detail(const char *what, hipError_t e) { set_detail(what, e); }

// Launches a planned call.  A split plan writes its partials to workspace
// (plan.workspace_bytes, stream-ordered on `stream`) and merges them.
int osa::launch_planned(const osa::PlannedCall &plan, void *workspace, hipStream_t stream) {
    osa::AttnProblem p = plan.p;
    if (!plan.split) {
        const bool w8 = plan.kernel == osa::MainKernel::BF16_8W || plan.kernel == osa::MainKernel::BF16_8W_BIAS;
        const hipError_t e = plan.kernel == osa::MainKernel::F32         ? osa::launch_attn_f32(p, stream)
                             : plan.kernel == osa::MainKernel::F32_SMALL ? osa::launch_attn_f32_small(p, stream)
                             : w8                                        ? osa::launch_attn_bf16_w8(p, stream)
                             : plan.kernel == osa::MainKernel::BF16_KH || plan.kernel == osa::MainKernel::BF16_KH_BIAS
                                 ? osa::launch_attn_bf16_kh(p, stream)
                                                                         : osa::launch_attn_bf16(p, stream);
        if (e != hipSuccess) {
            set_detail("attention kernel launch", e);
            return ATTN_ERR_HIP;
        }
        return ATTN_OK;
    }
    const size_t o_bytes = (size_t)p.splits * (size_t)p.BH * (size_t)p.N * (size_t)p.d * sizeof(float);
    p.part_o = static_cast<float *>(workspace);
    p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + o_bytes);
    const bool bf16 = plan.bf16;
    hipError_t e;
    if (plan.kernel == osa::MainKernel::DECODE)
        e = osa::launch_attn_decode(p, bf16, stream);
    else
        e = plan.kernel == osa::MainKernel::F32 ? osa::launch_attn_f32(p, stream) : osa::launch_attn_bf16(p, stream);
    if (e != hipSuccess) {
        set_detail("split attention kernel launch", e);
        return ATTN_ERR_HIP;
    }
    e = osa::launch_split_merge(p, bf16 && !p.out_f32, stream);
    if (e != hipSuccess) {
        set_detail("split merge kernel launch", e);
        return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

namespace {

int run_attn(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H, int64_t N,
             int64_t M, int d, float scale, const attn_mask *mask, int dtype, int num_splits, void *stream_v) {
    osa::PlannedCall plan;
    bool nothing = false;
    const int rc = osa::plan_attn(q, k, v, o, lse, B, H, N, M, d, scale, mask, dtype, num_splits, &plan, &nothing);
    if (rc != ATTN_OK || nothing) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    if (!plan.split) return osa::launch_planned(plan, nullptr, stream);
    // Split paths: partials in a stream-ordered workspace.
    void *ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, plan.workspace_bytes, stream);
    if (e != hipSuccess) {
        set_detail("hipMallocAsync of the split workspace", e);
        return ATTN_ERR_HIP;
    }
    const int lrc = osa::launch_planned(plan, ws, stream);
    const hipError_t ef = hipFreeAsync(ws, stream);
    if (lrc != ATTN_OK) return lrc;
    if (ef != hipSuccess) {
        set_detail("hipFreeAsync of the split workspace", ef);
        return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H, int64_t N,
             int64_t M, int d, float scale, int causal, int dtype, void *stream) {
    const attn_mask m{causal ? ATTN_CAUSAL_TOP_LEFT : ATTN_CAUSAL_NONE, nullptr};
    return run_attn(q, k, v, o, lse, B, H, N, M, d, scale, &m, dtype, 0, stream);
}

int attn_fwd_splits(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                    int64_t N, int64_t M, int d, float scale, int causal, int dtype, int num_splits, void *stream) {
    const attn_mask m{causal ? ATTN_CAUSAL_TOP_LEFT : ATTN_CAUSAL_NONE, nullptr};
    return run_attn(q, k, v, o, lse, B, H, N, M, d, scale, &m, dtype, num_splits, stream);
}

int attn_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                    int64_t N, int64_t M, int d, float scale, const attn_mask *mask, int dtype, int num_splits,
                    void *stream) {
    return run_attn(q, k, v, o, lse, B, H, N, M, d, scale, mask, dtype, num_splits, stream);
}

int attn_fwd_kv_outer(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                      int64_t N, int64_t M, int d, float scale, int causal, int dtype, void *stream_v) {
    const attn_mask m{causal ? ATTN_CAUSAL_TOP_LEFT : ATTN_CAUSAL_NONE, nullptr};
    const int rc = osa::validate_attn(q, k, v, o, lse, B, H, N, M, d, scale, dtype, 0, &m);
    if (rc != ATTN_OK || B == 0 || H == 0 || N == 0) return rc;
    if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    osa::AttnProblem p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.BH = (int)(B * H);
    p.N = (int)N;
    p.M = (int)M;
    p.d = d;
    p.H = (int)H;
    p.c = fmaxf(fabsf(scale) * 1.4426950408889634f, FLT_MIN);
    p.negate_q = signbit(scale) != 0;
    p.causal = causal != 0;
    p.splits = 1;
    const size_t rows = (size_t)B * H * N;
    const size_t bytes = rows * (size_t)d * sizeof(float) + 2 * rows * sizeof(float);
    void *ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, bytes, stream);
    if (e != hipSuccess) {
        set_detail("hipMallocAsync of the row-state workspace", e);
        return ATTN_ERR_HIP;
    }
    float *ws_o = static_cast<float *>(ws);
    float *ws_m = ws_o + rows * (size_t)d;
    float *ws_l = ws_m + rows;
    e = osa::launch_attn_kv_outer(p, ws_o, ws_m, ws_l, stream);
    if (e != hipSuccess) set_detail("key/value-outer kernel launch", e);
    const hipError_t ef = hipFreeAsync(ws, stream);
    if (e != hipSuccess) return ATTN_ERR_HIP;
    if (ef != hipSuccess) {
        set_detail("hipFreeAsync of the row-state workspace", ef);
        return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

int online_softmax_lse(const float *x, float *y, float *lse, int64_t rows, int64_t n, void *stream) {
    if (rows < 0 || n < 0) return ATTN_ERR_SHAPE;
    if (rows == 0) return ATTN_OK;
    if (n < 1) return ATTN_ERR_SHAPE;
    if (!x || (!y && !lse)) return ATTN_ERR_NULL;
    if (!aligned16(x) || (y && !aligned16(y)) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return ATTN_ERR_ALIGN;
    if (n > kI32Max || rows > (int64_t(1) << 62) / n) return ATTN_ERR_OVERFLOW;
    const hipError_t e = osa::launch_online_softmax(x, y, lse, rows, n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        set_detail("online softmax kernel launch", e);
        return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

int online_softmax(const float *x, float *y, int64_t rows, int64_t n, void *stream) {
    if (rows > 0 && n > 0 && !y) return ATTN_ERR_NULL;
    return online_softmax_lse(x, y, nullptr, rows, n, stream);
}

int softmax_xent(const float *x, const int64_t *labels, float *loss, float *lse, float *mean, int64_t rows,
                 int64_t n, void *stream) {
    if (rows < 0 || n < 0) return ATTN_ERR_SHAPE;
    if (rows == 0) return ATTN_OK;
    if (n < 1) return ATTN_ERR_SHAPE;
    if (!x || !labels || !loss) return ATTN_ERR_NULL;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(labels) & 7u) || (reinterpret_cast<uintptr_t>(loss) & 3u) ||
        (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (mean && (reinterpret_cast<uintptr_t>(mean) & 3u)))
        return ATTN_ERR_ALIGN;
    if (n > kI32Max || rows > (int64_t(1) << 62) / n) return ATTN_ERR_OVERFLOW;
    const hipError_t e =
        osa::launch_softmax_xent(x, labels, loss, lse, mean, rows, n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        set_detail("softmax cross-entropy kernel launch", e);
        return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

const char *attn_last_error_detail(void) { return g_detail; }

}  // extern "C"
