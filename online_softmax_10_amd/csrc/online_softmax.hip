// Row-wise softmax with the one-pass normaliser, fp32, for gfx950.
//
// Pass 1 keeps, per lane, the running max m and running sum s of the
// elements it visits (m_i = max(m_{i-1}, x_i), s_i = s_{i-1} e^{m_{i-1}-m_i}
// + e^{x_i - m_i}), a chunk of four elements at a time; the 64 lane states are
// merged with the same rule (max of the two maxima, each sum rescaled to it).
// Pass 2 writes y = e^{x - m} / s.  Optionally the row's log-sum-exp
// LSE = m + log s goes out too, and with y absent pass 2 is skipped (one read
// per element: the log-sum-exp reduction alone).  Two reads and one write per element,
// against three reads and one write for the three-pass safe softmax.  Rows
// whose length is a multiple of 4 and at most 65536 stay in registers between
// the passes, so they are read once: up to 4096 elements in one wave, longer
// rows in a 1024-thread workgroup that merges its 16 wave states through LDS.
// Sources: "Online Softmax and Flash Attention" page, section "Online softmax",
// eq. (3)-(7) and the pass counts in its introduction; "Softmax与Flash-Attention"
// page, online-softmax derivation.
//
// One 64-wide wave per row (or a 1024-thread workgroup for long rows).
// Exponentials are v_exp_f32 on base-2 arguments, e^{x - m} = 2^{(x - m)
// log2(e)}: the difference x - m is exact for nearby values, so logits of any
// magnitude work.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace osa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float NEG_INF = -__builtin_inff();
constexpr float LOG2E = 1.4426950408889634f;

// Running state of the recurrence: the max m so far and s = sum_i e^{x_i - m}.
struct MS {
    float m, s;
};

// e^{a - b} = 2^{(a - b) log2(e)} (0 for a = -inf, b finite).
__device__ __forceinline__ float exp_diff(float a, float b) { return __builtin_amdgcn_exp2f((a - b) * LOG2E); }

// Fold the values x[0..CNT) into the state.
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
    st.s = st.s * exp_diff(st.m, m_new) + add;
    st.m = m_new;
}

__device__ __forceinline__ MS merge(MS a, MS b) {
    const float m = fmaxf(a.m, b.m);
    if (m == NEG_INF) return a;
    const float sa = a.m == NEG_INF ? 0.f : a.s * exp_diff(a.m, m);
    const float sb = b.m == NEG_INF ? 0.f : b.s * exp_diff(b.m, m);
    return MS{m, sa + sb};
}

// Lane 0 writes the row's LSE = m + log s (natural log) when asked.
__device__ __forceinline__ void write_lse(float *lse_r, MS st, int lane) {
    if (lse_r != nullptr && lane == 0) *lse_r = st.m + logf(st.s);
}

template <bool VEC>
__device__ __forceinline__ void softmax_row(const float *xr, float *yr, float *lse_r, int64_t n, int lane) {
    MS st{NEG_INF, 0.f};
    if constexpr (VEC) {
        const int64_t nv = n >> 2;
        for (int64_t i = lane; i < nv; i += 64) {
            const f32x4 v = reinterpret_cast<const f32x4 *>(xr)[i];
            const float t[4] = {v[0], v[1], v[2], v[3]};
            absorb<4>(st, t);
        }
    } else {
        for (int64_t i = lane; i < n; i += 64) {
            const float t[1] = {xr[i]};
            absorb<1>(st, t);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        MS o{__shfl_xor(st.m, off, 64), __shfl_xor(st.s, off, 64)};
        st = merge(st, o);
    }
    write_lse(lse_r, st, lane);
    if (yr == nullptr) return;
    const float m = st.m;
    const float inv = 1.f / st.s;
    if constexpr (VEC) {
        const int64_t nv = n >> 2;
        for (int64_t i = lane; i < nv; i += 64) {
            const f32x4 v = reinterpret_cast<const f32x4 *>(xr)[i];
            f32x4 r;
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = exp_diff(v[j], m) * inv;
            reinterpret_cast<f32x4 *>(yr)[i] = r;
        }
    } else {
        for (int64_t i = lane; i < n; i += 64) yr[i] = exp_diff(xr[i], m) * inv;
    }
}

// Rows of n <= 256*R elements (n % 4 == 0) held in registers: each lane keeps
// R float4 chunks (chunk i + 64 r of the row), so the row is read once.
template <int R>
__device__ __forceinline__ void softmax_row_regs(const float *xr, float *yr, float *lse_r, int64_t n, int lane) {
    const int64_t nv = n >> 2;
    f32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = lane + 64 * r;
        v[r] = i < nv ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(xr) + i)
                      : f32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    }
    MS st{NEG_INF, 0.f};
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float t[4] = {v[r][0], v[r][1], v[r][2], v[r][3]};
        absorb<4>(st, t);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        MS o{__shfl_xor(st.m, off, 64), __shfl_xor(st.s, off, 64)};
        st = merge(st, o);
    }
    write_lse(lse_r, st, lane);
    if (yr == nullptr) return;
    const float m = st.m;
    const float inv = 1.f / st.s;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = lane + 64 * r;
        if (i < nv) {
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = exp_diff(v[r][j], m) * inv;
            __builtin_nontemporal_store(y, reinterpret_cast<f32x4 *>(yr) + i);
        }
    }
}

template <int R>
__global__ __launch_bounds__(256) void online_softmax_regs_kernel(const float *x, float *y, float *lse, int64_t rows,
                                                                  int64_t n) {
    const int lane = threadIdx.x & 63;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4)
        softmax_row_regs<R>(x + row * n, y ? y + row * n : nullptr, lse ? lse + row : nullptr, n, lane);
}

// Rows of 4096 < n <= 1024*4*R elements (n % 4 == 0): one 1024-thread
// workgroup per row, R float4 chunks per thread (chunk t + 1024 r), wave
// states merged through LDS.
template <int R>
__global__ __launch_bounds__(1024) void online_softmax_wide_kernel(const float *x, float *y, float *lse, int64_t rows,
                                                                   int64_t n) {
    __shared__ MS part[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t nv = n >> 2;
    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const f32x4 *xr = reinterpret_cast<const f32x4 *>(x + row * n);
        f32x4 *yr = y ? reinterpret_cast<f32x4 *>(y + row * n) : nullptr;
        f32x4 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t i = t + 1024 * r;
            v[r] = i < nv ? __builtin_nontemporal_load(xr + i) : f32x4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        }
        MS st{NEG_INF, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float tt[4] = {v[r][0], v[r][1], v[r][2], v[r][3]};
            absorb<4>(st, tt);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            MS o{__shfl_xor(st.m, off, 64), __shfl_xor(st.s, off, 64)};
            st = merge(st, o);
        }
        if (lane == 0) part[wave] = st;
        __syncthreads();
        MS all = part[0];
#pragma unroll
        for (int w = 1; w < 16; ++w) all = merge(all, part[w]);
        __syncthreads();  // part[] is rewritten by the next row
        write_lse(lse ? lse + row : nullptr, all, t);
        if (yr == nullptr) continue;
        const float m = all.m;
        const float inv = 1.f / all.s;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t i = t + 1024 * r;
            if (i < nv) {
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = exp_diff(v[r][j], m) * inv;
                __builtin_nontemporal_store(o, yr + i);
            }
        }
    }
}

// Grid-stride over rows, one wave per row.
template <bool VEC>
__global__ __launch_bounds__(256) void online_softmax_kernel(const float *x, float *y, float *lse, int64_t rows,
                                                             int64_t n) {
    const int lane = threadIdx.x & 63;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += (int64_t)gridDim.x * 4)
        softmax_row<VEC>(x + row * n, y ? y + row * n : nullptr, lse ? lse + row : nullptr, n, lane);
}

}  // namespace

hipError_t launch_online_softmax(const float *x, float *y, float *lse, int64_t rows, int64_t n, hipStream_t stream) {
    const int64_t want = (rows + 3) / 4;
    const dim3 grid((unsigned)(want < 65536 ? want : 65536));
    if ((n & 3) == 0 && n <= 4096) {
        // Smallest power-of-two chunk count per lane that holds the row.
        if (n <= 256)
            hipLaunchKernelGGL((online_softmax_regs_kernel<1>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
        else if (n <= 512)
            hipLaunchKernelGGL((online_softmax_regs_kernel<2>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
        else if (n <= 1024)
            hipLaunchKernelGGL((online_softmax_regs_kernel<4>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
        else if (n <= 2048)
            hipLaunchKernelGGL((online_softmax_regs_kernel<8>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
        else
            hipLaunchKernelGGL((online_softmax_regs_kernel<16>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
    } else if ((n & 3) == 0 && n <= 65536) {
        const dim3 wgrid((unsigned)(rows < 65536 ? rows : 65536));
        if (n <= 8192)
            hipLaunchKernelGGL((online_softmax_wide_kernel<2>), wgrid, dim3(1024), 0, stream, x, y, lse, rows, n);
        else if (n <= 16384)
            hipLaunchKernelGGL((online_softmax_wide_kernel<4>), wgrid, dim3(1024), 0, stream, x, y, lse, rows, n);
        else if (n <= 32768)
            hipLaunchKernelGGL((online_softmax_wide_kernel<8>), wgrid, dim3(1024), 0, stream, x, y, lse, rows, n);
        else
            hipLaunchKernelGGL((online_softmax_wide_kernel<16>), wgrid, dim3(1024), 0, stream, x, y, lse, rows, n);
    } else if ((n & 3) == 0)
        hipLaunchKernelGGL((online_softmax_kernel<true>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
    else
        hipLaunchKernelGGL((online_softmax_kernel<false>), grid, dim3(256), 0, stream, x, y, lse, rows, n);
    return hipGetLastError();
}

}  // namespace osa
