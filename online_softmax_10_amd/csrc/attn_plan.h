// Host-side planning of an attention call, free of HIP: argument validation,
// the work decomposition (single pass, key splits, decode), kernel choice and
// the size of the split workspace.  Internal to libattn.so (not installed);
// it is also built on its own, with the host sanitizers, by the CPU tests.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace osa {

// One attention problem, validated and planned.
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
constexpr int kBf16WideRows = 256;  // query rows per workgroup of the eight-wave kernel
// 64-key tiles a workgroup needs before its keys are split in halves (d = 64,
// d = 128): below them the second set's fixed costs (its first loads, the
// merge) outweigh the second wave per SIMD.
constexpr int kBf16KhMinTiles64 = 12;
constexpr int kBf16KhMinTiles128 = 16;
constexpr int kF32SmallWaves64 = 4;  // waves per workgroup of the small fp32 kernel at d = 64
constexpr int kF32SmallWaves128 = 4; // ... and at d = 128
constexpr int kF32SmallMaxKeys = 1024;  // keys the small fp32 kernel takes (its buffer offsets are 32-bit)

// The kernel that carries the attention itself (the split paths add the
// merge kernel).
enum class MainKernel { F32, F32_SMALL, BF16_4W, BF16_8W, BF16_KH, DECODE, BF16_BIAS, BF16_8W_BIAS, BF16_KH_BIAS };
const char *main_kernel_name(MainKernel k);

struct PlannedCall {
    AttnProblem p;
    MainKernel kernel;
    bool bf16;               // q, k, v are bf16 (ATTN_BF16 or ATTN_BF16_OUT_F32)
    bool split;              // partials in a workspace, then the merge kernel
    size_t workspace_bytes;  // bytes of that workspace (0 for a single pass)
};

// The argument checks of attn_fwd_masked (no HIP call, no dereference):
// ATTN_OK or the error code include/attn.h documents.
int validate_attn(const void *q, const void *k, const void *v, const void *o, const float *lse, int64_t B,
                  int64_t H, int64_t N, int64_t M, int d, float scale, int dtype, int num_splits,
                  const attn_mask *mask);

// Validates the arguments of attn_fwd_masked and plans the call without any
// HIP call and without dereferencing a pointer.  Returns ATTN_OK and fills
// *out, or an error code; *nothing is set when there is nothing to compute
// (B*H*N == 0; then *out is not filled).
int plan_attn(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H, int64_t N,
              int64_t M, int d, float scale, const attn_mask *mask, int dtype, int num_splits, PlannedCall *out,
              bool *nothing);

}  // namespace osa
