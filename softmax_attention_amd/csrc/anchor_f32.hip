// Gated softmax anchor, fp32 inputs, fp32 arithmetic throughout (vector ALU).
//
// One lane per query row; keys and values stream through LDS 32 at a time and
// the row softmax is accumulated online (running max, rescaled sum and
// accumulator). Serves the fp32 workloads, which are small; the bf16 path on
// the matrix cores is the fast one.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kKeys = 32;

template <int D>
__global__ __launch_bounds__(64) void anchor_f32(const float* __restrict__ Q,
                                                 const float* __restrict__ K,
                                                 const float* __restrict__ V,
                                                 const float* __restrict__ G,
                                                 float* __restrict__ out, int N, float scale,
                                                 int accumulate) {
  __shared__ float Ks[kKeys][D];
  __shared__ float Vs[kKeys][D];
  const int tid = threadIdx.x, bh = blockIdx.y;
  const int qi = blockIdx.x * 64 + tid;
  const size_t base = (size_t)bh * N * D;
  const bool live = qi < N;

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Q[base + (size_t)qi * D + d] * scale : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int k0 = 0; k0 < N; k0 += kKeys) {
    const int nk = min(kKeys, N - k0);
    __syncthreads();
    for (int e = tid; e < kKeys * D; e += 64) {
      const int row = e / D, col = e % D;
      Ks[row][col] = row < nk ? K[base + (size_t)(k0 + row) * D + col] : 0.f;
      Vs[row][col] = row < nk ? V[base + (size_t)(k0 + row) * D + col] : 0.f;
    }
    __syncthreads();
    float s[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[j][d], acc);
      s[j] = j < nk ? acc : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    const float alpha = expf(m - mn);  // 0 on the first tile (m = -inf)
    m = mn;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[j][d], o[d]);
    }
  }
  if (!live) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const size_t off = base + (size_t)qi * D + d;
    const float gate = 1.0f / (1.0f + expf(-G[off]));
    float r = gate * (o[d] * inv);
    if (accumulate) r += out[off];
    out[off] = r;
  }
}

template <int D>
hipError_t launch_d(const hla_dims& d, const void* q, const void* k, const void* v, const void* g,
                    void* out, int accumulate, float scale, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  hipLaunchKernelGGL(anchor_f32<D>, dim3((N + 63) / 64, BH), dim3(64), 0, stream,
                     reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(k),
                     reinterpret_cast<const float*>(v), reinterpret_cast<const float*>(g),
                     reinterpret_cast<float*>(out), N, scale, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_anchor_f32(const hla_dims& d, const void* q, const void* k, const void* v,
                             const void* g, void* out, int accumulate, float scale,
                             hipStream_t stream) {
  switch (d.D) {
    case 32: return launch_d<32>(d, q, k, v, g, out, accumulate, scale, stream);
    case 64: return launch_d<64>(d, q, k, v, g, out, accumulate, scale, stream);
    default: return launch_d<128>(d, q, k, v, g, out, accumulate, scale, stream);
  }
}

}  // namespace hla
