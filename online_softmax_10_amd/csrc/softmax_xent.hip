// Softmax cross-entropy per row, fp32, for gfx950: loss_i = LSE_i - x[i, c_i]
// with LSE_i = log sum_j e^{x[i,j]}, and the batch mean of the losses.
//
// The loss needs only the row's log-sum-exp and the label's logit, so one
// streaming pass over the logits suffices: the one-pass normaliser (running
// max m and sum s with s rescaled by e^{m_old - m_new} whenever the max moves)
// gives LSE = m + log s without a second read.  Sources: "从原始Softmax到在线
// Softmax" page, "softmax实际代码实现" (the cross-entropy loss as the negated
// log probability of the label, averaged over the batch) and "softmax形式推导"
// (log-softmax = z - LSE); "Online Softmax and Flash Attention" page, section
// "Online softmax", eq. (3)-(7) (the one-pass normaliser).
//
// Each lane folds float4 chunks of the row into a (max m, sum s) state with
// s = sum_j 2^{(x_j - m) log2(e)}: the differences x_j - m are exact for
// nearby values, so logits of any magnitude work, and s is accumulated in
// fp64 across the fp32 partial sums of the chunks (rows of 10^5 terms keep
// the LSE to fp32 rounding).  The lane states are merged within the wave by
// shuffles and, for long rows, across the row's waves in LDS.  The loss is
// formed as (m - z) + log s: no cancellation between two large numbers.
// Each row takes 16 to 1024 threads (about sixteen float4 chunks per thread);
// rows of 16 or 32 threads share a wave.  The logits are read once, with
// non-temporal loads.  The mean is a second, single-workgroup kernel that adds
// the row losses in fp64 in a fixed order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace osa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float NEG_INF = -__builtin_inff();
constexpr float LOG2E = 1.4426950408889634f;

// m = max_j x_j, s = sum_j 2^{(x_j - m) log2(e)}.
struct MS {
    float m;
    double s;
};

// 2^{(a - b) log2(e)} = e^{a - b} for a <= b (0 for a = -inf).
__device__ __forceinline__ float exp_diff(float a, float b) { return __builtin_amdgcn_exp2f((a - b) * LOG2E); }

template <int CNT>
__device__ __forceinline__ void absorb(MS &st, const float *x) {
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < CNT; ++i) mx = fmaxf(mx, x[i]);
    const float m_new = fmaxf(st.m, mx);
    if (m_new == NEG_INF) return;  // only -inf seen so far
    float add = 0.f;
#pragma unroll
    for (int i = 0; i < CNT; ++i) add += exp_diff(x[i], m_new);
    st.s = (st.m == m_new ? st.s : st.s * (double)exp_diff(st.m, m_new)) + (double)add;
    st.m = m_new;
}

__device__ __forceinline__ MS merge(MS a, MS b) {
    const float m = fmaxf(a.m, b.m);
    if (m == NEG_INF) return a;
    const double sa = a.m == NEG_INF ? 0.0 : a.s * (double)exp_diff(a.m, m);
    const double sb = b.m == NEG_INF ? 0.0 : b.s * (double)exp_diff(b.m, m);
    return MS{m, sa + sb};
}

// TPR threads per row (16 ... 1024); a workgroup of max(256, TPR) threads takes
// max(256, TPR) / TPR rows.  Thread 0 of a row fetches the label and its logit
// before the streaming loop so their latency overlaps it.
template <int TPR, bool VEC>
__global__ __launch_bounds__(TPR > 256 ? TPR : 256) void softmax_xent_kernel(
    const float *__restrict__ x, const int64_t *__restrict__ labels, float *__restrict__ loss,
    float *__restrict__ lse, int64_t rows, int64_t n) {
    constexpr int NT = TPR > 256 ? TPR : 256;
    constexpr int RPW = NT / TPR;              // rows per workgroup
    constexpr int WPR = TPR > 64 ? TPR / 64 : 1;  // waves per row
    __shared__ MS part[TPR > 64 ? WPR : 1];
    const int t = threadIdx.x % TPR, sub = threadIdx.x / TPR;
    const int lane = threadIdx.x & 63, wave_in_row = t >> 6;
    for (int64_t base = (int64_t)blockIdx.x * RPW; base < rows; base += (int64_t)gridDim.x * RPW) {
        const int64_t row = base + sub;
        MS st{NEG_INF, 0.0};
        int64_t c = 0;
        float z = 0.f;
        if (row < rows) {
            const float *xr = x + row * n;
            if (t == 0) {
                c = labels[row];
                z = xr[(c >= 0 && c < n) ? c : 0];
            }
            if constexpr (VEC) {
                const int64_t nv = n >> 2;
#pragma unroll 4
                for (int64_t i = t; i < nv; i += TPR) {
                    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(xr) + i);
                    const float c4[4] = {v[0], v[1], v[2], v[3]};
                    absorb<4>(st, c4);
                }
            } else {
#pragma unroll 4
                for (int64_t i = t; i < n; i += TPR) {
                    const float c1[1] = {__builtin_nontemporal_load(xr + i)};
                    absorb<1>(st, c1);
                }
            }
        }
#pragma unroll
        for (int off = (TPR < 64 ? TPR : 64) / 2; off >= 1; off >>= 1) {
            MS o{__shfl_xor(st.m, off, 64), __shfl_xor(st.s, off, 64)};
            st = merge(st, o);
        }
        if constexpr (TPR > 64) {
            if (lane == 0) part[wave_in_row] = st;
            __syncthreads();
            st = part[0];
#pragma unroll
            for (int w = 1; w < WPR; ++w) st = merge(st, part[w]);
            __syncthreads();  // part[] is rewritten for the next row
        }
        if (row < rows && t == 0) {
            // log sum_j e^{x_j - m} = log s.  m = -inf only for a row of -inf
            // logits: LSE = -inf, loss NaN.
            const float tail = st.m == NEG_INF ? 0.f : (float)log(st.s);
            const bool valid = c >= 0 && c < n;
            loss[row] = valid ? (st.m - z) + tail : __builtin_nanf("");
            if (lse != nullptr) lse[row] = st.m + tail;
        }
    }
}

// mean = (sum of loss[0..rows)) / rows, added in fp64 in a fixed order:
// thread t adds indices t + 1024 k in rounds of 32 independent loads (one
// memory latency per round), then a tree over the 1024 threads.
__global__ __launch_bounds__(1024) void xent_mean_kernel(const float *__restrict__ loss, float *__restrict__ mean,
                                                         int64_t rows) {
    constexpr int U = 32;
    __shared__ double part[1024];
    const int t = threadIdx.x;
    double acc = 0.0;
    for (int64_t i0 = t; i0 < rows; i0 += (int64_t)U * 1024) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + (int64_t)u * 1024;
            v[u] = i < rows ? loss[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (double)v[u];
    }
    part[t] = acc;
    __syncthreads();
    for (int w = 512; w >= 1; w >>= 1) {
        if (t < w) part[t] += part[t + w];
        __syncthreads();
    }
    if (t == 0) mean[0] = (float)(part[0] / (double)rows);
}

template <int TPR>
hipError_t launch_t(const float *x, const int64_t *labels, float *loss, float *lse, int64_t rows, int64_t n,
                    hipStream_t stream) {
    constexpr int NT = TPR > 256 ? TPR : 256;
    constexpr int RPW = NT / TPR;
    const int64_t want = (rows + RPW - 1) / RPW;
    const dim3 grid((unsigned)(want < 65536 ? want : 65536));
    if ((n & 3) == 0)
        hipLaunchKernelGGL((softmax_xent_kernel<TPR, true>), grid, dim3(NT), 0, stream, x, labels, loss, lse, rows, n);
    else
        hipLaunchKernelGGL((softmax_xent_kernel<TPR, false>), grid, dim3(NT), 0, stream, x, labels, loss, lse, rows,
                           n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax_xent(const float *x, const int64_t *labels, float *loss, float *lse, float *mean,
                               int64_t rows, int64_t n, hipStream_t stream) {
    // About sixteen chunks (float4, or single logits when n % 4 != 0) per
    // thread, between 16 and 1024 threads per row.
    const int64_t per = ((n & 3) == 0 ? n >> 2 : n) / 16;
    hipError_t e = per <= 16    ? launch_t<16>(x, labels, loss, lse, rows, n, stream)
                   : per <= 32  ? launch_t<32>(x, labels, loss, lse, rows, n, stream)
                   : per <= 64  ? launch_t<64>(x, labels, loss, lse, rows, n, stream)
                   : per <= 512 ? launch_t<256>(x, labels, loss, lse, rows, n, stream)
                                : launch_t<1024>(x, labels, loss, lse, rows, n, stream);
    if (e != hipSuccess || mean == nullptr) return e;
    hipLaunchKernelGGL(xent_mean_kernel, dim3(1), dim3(1024), 0, stream, loss, mean, rows);
    return hipGetLastError();
}

}  // namespace osa
