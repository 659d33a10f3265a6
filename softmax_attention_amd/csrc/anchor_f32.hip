// Gated softmax anchor, fp32 inputs, fp32 arithmetic throughout (vector ALU).
//
// One lane per query row; keys and values stream through LDS 16 at a time and
// the row softmax is accumulated online (running max, rescaled sum and
// accumulator), split over the four waves of a workgroup. Serves the fp32
// workloads, which are small; the bf16 path on the matrix cores is the fast one.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kKeys = 16;   // keys per LDS tile
constexpr int kSplit = 4;   // waves per workgroup; wave w takes key tiles w, w+4, ...

// One lane per query row, 64 query rows per workgroup; the four waves of the
// workgroup each run the online softmax over a quarter of the key tiles, and
// their (running max, sum, accumulator) are merged through LDS at the end.
template <int D>
__global__ __launch_bounds__(256) void anchor_f32(const float* __restrict__ Q,
                                                  const float* __restrict__ K,
                                                  const float* __restrict__ V,
                                                  const float* __restrict__ G,
                                                  float* __restrict__ out, int N, float scale,
                                                  int accumulate) {
  static_assert(2 * kSplit * kKeys * D >= 64 * (D + 2), "merge buffer fits in the tiles");
  __shared__ float lds[2 * kSplit * kKeys * D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, bh = blockIdx.y;
  const int qi = blockIdx.x * 64 + lane;
  const size_t base = (size_t)bh * N * D;
  const bool live = qi < N;
  float (*Ks)[D] = reinterpret_cast<float (*)[D]>(lds + w * kKeys * D);
  float (*Vs)[D] = reinterpret_cast<float (*)[D]>(lds + (kSplit + w) * kKeys * D);

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Q[base + (size_t)qi * D + d] * scale : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int ntiles = (N + kKeys - 1) / kKeys;
  const int rounds = (ntiles + kSplit - 1) / kSplit;
  for (int r = 0; r < rounds; ++r) {
    const int k0 = (r * kSplit + w) * kKeys;
    const int nk = max(0, min(kKeys, N - k0));
    __syncthreads();
    for (int e = lane; e < kKeys * D; e += 64) {
      const int row = e / D, col = e % D;
      Ks[row][col] = row < nk ? K[base + (size_t)(k0 + row) * D + col] : 0.f;
      Vs[row][col] = row < nk ? V[base + (size_t)(k0 + row) * D + col] : 0.f;
    }
    __syncthreads();
    if (nk == 0) continue;  // a tile past the last key (wave-uniform)
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
    const float alpha = expf(m - mn);  // 0 on the wave's first tile (m = -inf)
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

  // merge waves 1..3 into wave 0, one at a time through the tile memory
  float* red = lds + lane * (D + 2);
  for (int src = 1; src < kSplit; ++src) {
    __syncthreads();
    if (w == src) {
      red[0] = m;
      red[1] = l;
#pragma unroll
      for (int d = 0; d < D; ++d) red[2 + d] = o[d];
    }
    __syncthreads();
    if (w == 0 && red[0] != -INFINITY) {  // that wave saw at least one key
      const float m2 = red[0], mn = fmaxf(m, m2);
      const float a = expf(m - mn), b = expf(m2 - mn);
      l = l * a + red[1] * b;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = o[d] * a + red[2 + d] * b;
      m = mn;
    }
  }
  if (w != 0 || !live) return;
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
  hipLaunchKernelGGL(anchor_f32<D>, dim3((N + 63) / 64, BH), dim3(64 * kSplit), 0, stream,
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
