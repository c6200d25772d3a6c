// Internal launcher interface between the C-ABI front end (attn_api.cpp) and
// the HIP kernels.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osa {

// One attention problem, already validated by the front end.
struct AttnProblem {
    const void *q, *k, *v;  // [BH,N,d] / [BH,M,d] / [BH,M,d], dtype elements
    void *o;                 // [BH,N,d] dtype (unused when writing partials)
    float *lse;              // [BH,N]          (unused when writing partials)
    int BH, N, M, d;
    int H;                   // heads per batch (batch of head bh = bh / H)
    const int32_t *kv_len;   // [B] valid keys per batch (device; clamped to [0, M]), or nullptr
    // Additive score bias, fp32, or nullptr: element (b, h, i, j) at
    // bias[b*bias_sb + h*bias_sh + i*bias_sn + j]; 16-byte aligned rows.
    const float *bias;
    uint32_t bias_bytes;     // bytes from bias to the end of its last element (< 2^32)
    int64_t bias_sb, bias_sh, bias_sn;
    int causal_off;          // causal: key j visible for query i iff j <= i + causal_off
    float c;                 // |scale| * log2(e): scores are kept in base-2 units
    bool negate_q;           // scale < 0: q's sign is flipped on load so c >= 0
    bool causal;
    bool out_f32;            // bf16 inputs, float32 o: single pass uses the partial-store path on o
    // Split over keys: split s covers tiles [s*tiles_per_split, (s+1)*tiles_per_split)
    // of the kernel's key tile size.  splits == 1 writes o and lse directly.
    int splits;
    int tiles_per_split;
    float *part_o;           // [splits,BH,N,d] fp32, normalised partial outputs
    float *part_lse;         // [splits,BH,N]   fp32, natural-log partial LSE (-inf if empty)
};

// Key tile sizes (the unit of a split range) of each kernel family.
constexpr int kBf16KeyTile = 64;
constexpr int kF32KeyTile = 32;
constexpr int kDecodeKeyTile = 64;
constexpr int kDecodeMaxQueries = 4;

// Four-wave bf16 kernel: 128 query rows per workgroup (any size; split partials).
hipError_t launch_attn_bf16(const AttnProblem &p, hipStream_t stream);
// Eight-wave bf16 kernel: 256 query rows per workgroup, single pass only.
hipError_t launch_attn_bf16_w8(const AttnProblem &p, hipStream_t stream);
constexpr int kBf16WideRows = 256;
hipError_t launch_attn_f32(const AttnProblem &p, hipStream_t stream);
// Few queries per head (N <= kDecodeMaxQueries), bf16 or fp32 inputs, always
// writes partials (p.splits >= 1).
hipError_t launch_attn_decode(const AttnProblem &p, bool bf16, hipStream_t stream);
// lse = log sum_s e^{part_lse}, o = sum_s e^{part_lse - lse} part_o.
hipError_t launch_split_merge(const AttnProblem &p, bool bf16, hipStream_t stream);

// Key/value-outer loop order (one launch per key block, row state in the
// fp32 workspace ws_o [BH,N,d], ws_m, ws_l [BH,N]); bf16, single pass, no mask
// beyond top-left causal.
hipError_t launch_attn_kv_outer(const AttnProblem &p, float *ws_o, float *ws_m, float *ws_l, hipStream_t stream);
// y and lse may each be nullptr (not both): softmax rows, row LSE, or both.
hipError_t launch_online_softmax(const float *x, float *y, float *lse, int64_t rows, int64_t n, hipStream_t stream);
// loss[i] = LSE_i - x[i, labels[i]] (NaN for a label outside [0, n)); lse and
// mean optional (nullptr): the row LSE and the mean of the losses.
hipError_t launch_softmax_xent(const float *x, const int64_t *labels, float *loss, float *lse, float *mean,
                               int64_t rows, int64_t n, hipStream_t stream);

}  // namespace osa
