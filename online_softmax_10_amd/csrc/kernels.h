// Internal launcher interface between the C-ABI front end (attn_api.cpp) and
// the HIP kernels.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_plan.h"

namespace osa {

// Launches a call planned by plan_attn; a split plan's partials go to
// `workspace` (at least plan.workspace_bytes of device memory, stream-ordered
// on `stream`).  Returns ATTN_OK or ATTN_ERR_HIP (detail recorded).
int launch_planned(const PlannedCall &plan, void *workspace, hipStream_t stream);
// Records the detail string that attn_last_error_detail returns.
void set_hip_detail(const char *what, hipError_t e);

// Four-wave bf16 kernel: 128 query rows per workgroup (any size; split partials).
hipError_t launch_attn_bf16(const AttnProblem &p, hipStream_t stream);
// Eight-wave bf16 kernel: 256 query rows per workgroup, single pass only.
hipError_t launch_attn_bf16_w8(const AttnProblem &p, hipStream_t stream);
// Key-halves bf16 kernel: 128 query rows per workgroup of eight waves, the
// key tiles alternating between two sets of four waves and merged in LDS;
// single pass (bf16 output, or a float32 one through the partial-store form);
// an additive bias at d = 64 with a bf16 output.
hipError_t launch_attn_bf16_kh(const AttnProblem &p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnProblem &p, hipStream_t stream);
// fp32, small problems: one workgroup per 16-row block, keys split over its
// waves and merged in LDS; single pass, no bias.
hipError_t launch_attn_f32_small(const AttnProblem &p, hipStream_t stream);
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
