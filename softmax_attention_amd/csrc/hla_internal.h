// Host-side plumbing shared by the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hla.h"

namespace hla {

// Work split and workspace layout of the gated linear attention for one call.
struct LinearPlan {
  int C = 0;               // token chunks per (b, h) in the state pass
  int T = 0;               // tokens per chunk (multiple of 64)
  int P = 0;               // workgroups per (b, h) in the output pass
  size_t part_off = 0;     // fp32 partial states [BH][C][D*D + D]
  size_t state_off = 0;    // reduced state in the output pass's operand form
  size_t state_bytes = 0;  // bytes per (b, h) of that form
  size_t total = 0;        // workspace bytes
};

LinearPlan linear_plan(const hla_dims& d);

// Work-split overrides for tuning sweeps, fixed when the library is compiled
// (-DHLA_LINEAR_CHUNKS=C, -DHLA_LINEAR_OUT_WGS=P); 0 keeps the built-in choice.
// Nothing read at run time changes the split, so equal calls sum in equal order.
#ifndef HLA_LINEAR_CHUNKS
#define HLA_LINEAR_CHUNKS 0
#endif
#ifndef HLA_LINEAR_OUT_WGS
#define HLA_LINEAR_OUT_WGS 0
#endif
constexpr int kLinearChunksOverride = HLA_LINEAR_CHUNKS;  // C override
constexpr int kLinearOutWgsOverride = HLA_LINEAR_OUT_WGS;  // P override
// Token groups each output-pass wave keeps in flight ahead of the one it
// computes, for bf16 and for fp8 inputs.
#ifndef HLA_LINEAR_OUT_PREFETCH
#define HLA_LINEAR_OUT_PREFETCH 2
#endif
#ifndef HLA_LINEAR_OUT_PREFETCH_F8
#define HLA_LINEAR_OUT_PREFETCH_F8 2
#endif
constexpr int kLinearOutPrefetch = HLA_LINEAR_OUT_PREFETCH;
constexpr int kLinearOutPrefetchF8 = HLA_LINEAR_OUT_PREFETCH_F8;

// w: write-gate logits [B,H,N] (in_dtype) for the write-gated variant, or NULL
hipError_t launch_linear_bf16(const hla_dims& d, const void* q, const void* k, const void* v,
                              const void* g, const void* w, void* out, int accumulate, float eps,
                              void* ws, const LinearPlan& plan, hipStream_t stream);
hipError_t launch_linear_f32(const hla_dims& d, const void* q, const void* k, const void* v,
                             const void* g, const void* w, void* out, int accumulate, float eps,
                             void* ws, const LinearPlan& plan, hipStream_t stream);
// Workspace of the bf16 anchor: V repacked as V^T per head, keys padded to 64.
size_t anchor_workspace_bytes(const hla_dims& d);
// fp8_p: P rounded to e4m3 and P V on the fp8 matrix cores (fp8 inputs only)
hipError_t launch_anchor_bf16(const hla_dims& d, const void* q, const void* k, const void* v,
                              const void* g, void* out, int accumulate, float scale, void* ws,
                              hipStream_t stream, bool fp8_p = false);
hipError_t launch_anchor_f32(const hla_dims& d, const void* q, const void* k, const void* v,
                             const void* g, void* out, int accumulate, float scale,
                             hipStream_t stream);

// Block summaries of the attention-residual routing, passed to the kernel by value.
constexpr int kMaxAttnResBlocks = 16;
struct AttnResBlocks {
  const float* p[kMaxAttnResBlocks];
};
// x, summaries, out: fp32 [B,H,N,D]; w: bf16 [D,D]; 1 <= n_blocks <= kMaxAttnResBlocks
hipError_t launch_attnres_route(const hla_dims& d, int n_blocks, const AttnResBlocks& blocks,
                                const void* x, const void* w, void* out, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace hla
