// C ABI of the hybrid linear-softmax attention library (declared in include/hla.h).
//
// Every argument is validated on the host before any HIP call, so an invalid
// call enqueues nothing and leaves the output untouched; the validation path
// runs without a GPU. Valid calls enqueue kernels on the caller's stream and
// return without synchronising.
#include <math.h>

#include <mutex>

#include "hla_internal.h"

namespace hla {

namespace {

constexpr int64_t kMaxIndex = 0x7fffffffLL;  // per-head offsets are 32-bit in places

bool in_dtype_ok(int32_t x) { return x == HLA_F32 || x == HLA_BF16 || x == HLA_FP8_E4M3; }
bool out_dtype_ok(int32_t x) { return x == HLA_F32 || x == HLA_BF16; }

// Shape and dtype checks shared by all entry points.
hla_status check_dims(const hla_dims* d) {
  if (!d) return HLA_ERR_NULL_PTR;
  if (d->B < 0 || d->H < 0 || d->N < 0 || d->D <= 0) return HLA_ERR_BAD_SHAPE;
  if (!in_dtype_ok(d->in_dtype) || !out_dtype_ok(d->out_dtype)) return HLA_ERR_UNSUPPORTED;
  if (d->in_dtype == HLA_F32) {
    if (d->out_dtype != HLA_F32) return HLA_ERR_UNSUPPORTED;
    if (d->D != 32 && d->D != 64 && d->D != 128) return HLA_ERR_UNSUPPORTED;
  } else {
    if (d->D != 64 && d->D != 128) return HLA_ERR_UNSUPPORTED;
  }
  // every count must fit: B*H (grid), N*D (per-head offsets), B*H*N*D*4 bytes
  if (d->B > kMaxIndex || d->H > kMaxIndex || d->N > kMaxIndex) return HLA_ERR_BAD_SHAPE;
  const int64_t bh = d->B * d->H;  // < 2^62, no overflow
  if (bh > 65535 * 1024LL) return HLA_ERR_BAD_SHAPE;
  // per-head byte offsets are 32-bit (buffer loads), with room for one tile past N
  if (d->N * d->D > kMaxIndex - 65536) return HLA_ERR_BAD_SHAPE;
  if (bh > 0 && d->N * d->D > INT64_MAX / 4 / bh) return HLA_ERR_BAD_SHAPE;
  // anchor grid: B*H * ceil(N/128) workgroups in one dimension
  if (bh * ((d->N + 127) / 128) > kMaxIndex) return HLA_ERR_BAD_SHAPE;
  return HLA_OK;
}

bool empty(const hla_dims* d) { return d->B * d->H * d->N == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hla_status check_tensors(const void* q, const void* k, const void* v, const void* g,
                         const void* out) {
  if (!q || !k || !v || !g || !out) return HLA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(out))
    return HLA_ERR_ALIGN;
  return HLA_OK;
}

hla_status from_hip(hipError_t e) { return e == hipSuccess ? HLA_OK : HLA_ERR_HIP; }

// hipGetLastError() also reports errors left pending by the caller's earlier
// runtime calls (a failed pointer query, for instance). Clear that state right
// before launching, so the check after the launches sees only this call's.
void clear_pending_error() { (void)hipGetLastError(); }

}  // namespace

LinearPlan linear_plan(const hla_dims& d) {
  LinearPlan p;
  const int64_t BH = d.B * d.H, N = d.N, D = d.D;
  if (BH <= 0 || N <= 0) return p;
  // state pass: aim at ~512 workgroups (two per CU) with chunks of >= 64 tokens
  const int64_t max_c = (N + 63) / 64;
  int64_t c = kLinearChunksOverride > 0 ? kLinearChunksOverride : (512 + BH - 1) / BH;
  c = c < 1 ? 1 : (c > max_c ? max_c : c);
  int64_t T = (N + c - 1) / c;
  T = (T + 63) / 64 * 64;
  c = (N + T - 1) / T;  // every chunk non-empty
  p.C = int(c);
  p.T = int(T);
  // output pass: workgroups per head
  int64_t P = kLinearOutWgsOverride > 0 ? kLinearOutWgsOverride : (512 + BH - 1) / BH;
  const int64_t max_p = (N + 63) / 64;
  P = P < 1 ? 1 : (P > max_p ? max_p : P);
  p.P = int(P);
  // per chunk: fp32 S and z (fp32 path), or bf16 S and fp32 z (bf16 and fp8 paths)
  const size_t per_chunk = d.in_dtype != HLA_F32 ? size_t(D * D) * 2 + size_t(D) * 4
                                                 : size_t(D * D + D) * 4;
  const size_t part = size_t(BH) * size_t(c) * per_chunk;
  if (d.in_dtype != HLA_F32)
    p.state_bytes = size_t((D / 16 + 1) * (D / 32)) * 1024;  // MFMA operand fragments
  else
    p.state_bytes = size_t(D * D + D) * 4;                   // fp32 S and z
  p.part_off = 0;
  p.state_off = align_up(part, 256);
  p.total = p.state_off + align_up(size_t(BH) * p.state_bytes, 256);
  return p;
}

}  // namespace hla

using namespace hla;

// Checks and launch shared by the plain and the write-gated linear entry points.
static hla_status linear_common(const hla_dims* d, const void* q, const void* k, const void* v,
                                const void* g, const void* w, bool gated, void* out,
                                int accumulate, float eps, void* workspace,
                                size_t workspace_bytes, void* stream) {
  hla_status st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!isfinite(eps) || eps < 0.f || (accumulate != 0 && accumulate != 1)) return HLA_ERR_BAD_ARG;
  if (empty(d)) return HLA_OK;
  if ((st = check_tensors(q, k, v, g, out)) != HLA_OK) return st;
  if (gated) {
    if (!w) return HLA_ERR_NULL_PTR;
    if (!aligned16(w)) return HLA_ERR_ALIGN;
  }
  const LinearPlan plan = linear_plan(*d);
  if (!workspace) return HLA_ERR_NULL_PTR;
  if (!aligned16(workspace)) return HLA_ERR_ALIGN;
  if (workspace_bytes < plan.total) return HLA_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_pending_error();
  if (d->in_dtype != HLA_F32)  // bf16, or fp8 converted to bf16 on load
    return from_hip(launch_linear_bf16(*d, q, k, v, g, w, out, accumulate, eps, workspace, plan, s));
  return from_hip(launch_linear_f32(*d, q, k, v, g, w, out, accumulate, eps, workspace, plan, s));
}

// Scratch memory of the allocation-free linear entry point: one copy per GPU
// (each device that loads the library holds it until the process ends). The
// array's name is a host-side stand-in in host code; kernels get the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[HLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Address of the current device's scratch array, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int hla_abi_version(void) { return HLA_ABI_VERSION; }

const char* hla_status_str(int s) {
  switch (s) {
    case HLA_OK: return "HLA_OK";
    case HLA_ERR_NULL_PTR: return "HLA_ERR_NULL_PTR";
    case HLA_ERR_BAD_SHAPE: return "HLA_ERR_BAD_SHAPE";
    case HLA_ERR_UNSUPPORTED: return "HLA_ERR_UNSUPPORTED";
    case HLA_ERR_BAD_ARG: return "HLA_ERR_BAD_ARG";
    case HLA_ERR_ALIGN: return "HLA_ERR_ALIGN";
    case HLA_ERR_WORKSPACE: return "HLA_ERR_WORKSPACE";
    case HLA_ERR_HIP: return "HLA_ERR_HIP";
    default: return "HLA_UNKNOWN";
  }
}

size_t hla_linear_workspace_bytes(const hla_dims* d) {
  if (check_dims(d) != HLA_OK || empty(d)) return 0;
  return linear_plan(*d).total;
}

size_t hla_softmax_anchor_workspace_bytes(const hla_dims* d) {
  if (check_dims(d) != HLA_OK || empty(d)) return 0;
  return anchor_workspace_bytes(*d);
}

hla_status hla_linear_fwd(const hla_dims* d, const void* q, const void* k, const void* v,
                          const void* g, void* out, int accumulate, float eps, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return linear_common(d, q, k, v, g, nullptr, false, out, accumulate, eps, workspace,
                       workspace_bytes, stream);
}

hla_status hla_linear_fwd_noalloc(const hla_dims* d, const void* q, const void* k, const void* v,
                                  const void* g, void* out, int accumulate, float eps,
                                  void* stream) {
  hla_status st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!isfinite(eps) || eps < 0.f || (accumulate != 0 && accumulate != 1)) return HLA_ERR_BAD_ARG;
  if (empty(d)) return HLA_OK;
  if ((st = check_tensors(q, k, v, g, out)) != HLA_OK) return st;
  if (linear_plan(*d).total > size_t(HLA_NOALLOC_SCRATCH_BYTES)) return HLA_ERR_WORKSPACE;
  void* ws = nullptr;
  clear_pending_error();
  if (scratch_address(&ws) != hipSuccess) return HLA_ERR_HIP;
  return linear_common(d, q, k, v, g, nullptr, false, out, accumulate, eps, ws,
                       HLA_NOALLOC_SCRATCH_BYTES, stream);
}

hla_status hla_linear_write_gated_fwd(const hla_dims* d, const void* q, const void* k,
                                      const void* v, const void* g, const void* w, void* out,
                                      int accumulate, float eps, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return linear_common(d, q, k, v, g, w, true, out, accumulate, eps, workspace, workspace_bytes,
                       stream);
}

static hla_status anchor_common(const hla_dims* d, const void* q, const void* k, const void* v,
                                const void* g, void* out, int accumulate, float scale,
                                void* workspace, size_t workspace_bytes, void* stream, bool fp8_p) {
  hla_status st = check_dims(d);
  if (st != HLA_OK) return st;
  if (fp8_p && d->in_dtype != HLA_FP8_E4M3) return HLA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || scale <= 0.f || (accumulate != 0 && accumulate != 1))
    return HLA_ERR_BAD_ARG;
  if (empty(d)) return HLA_OK;
  if ((st = check_tensors(q, k, v, g, out)) != HLA_OK) return st;
  const size_t need = anchor_workspace_bytes(*d);
  if (need > 0) {
    if (!workspace) return HLA_ERR_NULL_PTR;
    if (!aligned16(workspace)) return HLA_ERR_ALIGN;
    if (workspace_bytes < need) return HLA_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_pending_error();
  if (d->in_dtype != HLA_F32)
    return from_hip(launch_anchor_bf16(*d, q, k, v, g, out, accumulate, scale, workspace, s, fp8_p));
  return from_hip(launch_anchor_f32(*d, q, k, v, g, out, accumulate, scale, s));
}

hla_status hla_softmax_anchor_fwd(const hla_dims* d, const void* q, const void* k, const void* v,
                                  const void* g, void* out, int accumulate, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return anchor_common(d, q, k, v, g, out, accumulate, scale, workspace, workspace_bytes, stream,
                       false);
}

hla_status hla_softmax_anchor_fp8p_fwd(const hla_dims* d, const void* q, const void* k,
                                       const void* v, const void* g, void* out, int accumulate,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return anchor_common(d, q, k, v, g, out, accumulate, scale, workspace, workspace_bytes, stream,
                       true);
}

hla_status hla_hybrid_stack_fwd(const hla_dims* d, int n_layers, const int32_t* kinds,
                                const void* const* q, const void* const* k,
                                const void* const* v, const void* const* g, void* x, float eps,
                                float scale, void* workspace, size_t workspace_bytes,
                                void* stream) {
  hla_status st = check_dims(d);
  if (st != HLA_OK) return st;
  if (n_layers <= 0) return HLA_ERR_BAD_ARG;
  if (!kinds || !q || !k || !v || !g) return HLA_ERR_NULL_PTR;
  if (!isfinite(eps) || eps < 0.f || !isfinite(scale) || scale <= 0.f) return HLA_ERR_BAD_ARG;
  bool any_linear = false, any_softmax = false;
  for (int l = 0; l < n_layers; ++l) {
    if (kinds[l] != HLA_LAYER_LINEAR && kinds[l] != HLA_LAYER_SOFTMAX) return HLA_ERR_BAD_ARG;
    any_linear |= kinds[l] == HLA_LAYER_LINEAR;
    any_softmax |= kinds[l] == HLA_LAYER_SOFTMAX;
  }
  if (empty(d)) return HLA_OK;
  for (int l = 0; l < n_layers; ++l)
    if ((st = check_tensors(q[l], k[l], v[l], g[l], x)) != HLA_OK) return st;
  LinearPlan plan;
  size_t need = 0;
  if (any_linear) {
    plan = linear_plan(*d);
    need = plan.total;
  }
  if (any_softmax) need = need > anchor_workspace_bytes(*d) ? need : anchor_workspace_bytes(*d);
  if (need > 0) {
    if (!workspace) return HLA_ERR_NULL_PTR;
    if (!aligned16(workspace)) return HLA_ERR_ALIGN;
    if (workspace_bytes < need) return HLA_ERR_WORKSPACE;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = d->in_dtype != HLA_F32;  // bf16 or fp8 kernels
  clear_pending_error();
  for (int l = 0; l < n_layers; ++l) {
    hipError_t e;
    if (kinds[l] == HLA_LAYER_LINEAR)
      e = bf ? launch_linear_bf16(*d, q[l], k[l], v[l], g[l], nullptr, x, 1, eps, workspace, plan, s)
             : launch_linear_f32(*d, q[l], k[l], v[l], g[l], nullptr, x, 1, eps, workspace, plan, s);
    else
      e = bf ? launch_anchor_bf16(*d, q[l], k[l], v[l], g[l], x, 1, scale, workspace, s)
             : launch_anchor_f32(*d, q[l], k[l], v[l], g[l], x, 1, scale, s);
    if (e != hipSuccess) return HLA_ERR_HIP;
  }
  return HLA_OK;
}

hla_status hla_attnres_route_fwd(const hla_dims* d, int n_blocks, const void* const* summaries,
                                 const void* x, const void* w_router, void* out, void* stream) {
  hla_status st = check_dims(d);
  if (st != HLA_OK) return st;
  if (d->in_dtype != HLA_F32 || d->out_dtype != HLA_F32 || (d->D != 64 && d->D != 128))
    return HLA_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > kMaxAttnResBlocks) return HLA_ERR_BAD_ARG;
  if (n_blocks > 0 && !summaries) return HLA_ERR_NULL_PTR;
  if (empty(d)) return HLA_OK;
  if (!x || !out) return HLA_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(out)) return HLA_ERR_ALIGN;
  AttnResBlocks blocks{};
  if (n_blocks > 0) {
    if (!w_router) return HLA_ERR_NULL_PTR;
    if (!aligned16(w_router)) return HLA_ERR_ALIGN;
    for (int i = 0; i < n_blocks; ++i) {
      if (!summaries[i]) return HLA_ERR_NULL_PTR;
      if (!aligned16(summaries[i])) return HLA_ERR_ALIGN;
      blocks.p[i] = reinterpret_cast<const float*>(summaries[i]);
    }
  }
  if (n_blocks == 0 && out == x) return HLA_OK;  // no completed block, in place: nothing to do
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  clear_pending_error();
  if (n_blocks == 0) {  // no completed block: the stream passes unchanged
    const size_t bytes = size_t(d->B * d->H * d->N * d->D) * 4;
    return from_hip(hipMemcpyAsync(out, x, bytes, hipMemcpyDeviceToDevice, s));
  }
  return from_hip(launch_attnres_route(*d, n_blocks, blocks, x, w_router, out, s));
}

}  // extern "C"
