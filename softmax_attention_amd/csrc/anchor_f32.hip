// Gated softmax anchor, fp32 inputs, fp32 arithmetic throughout (vector ALU).
//
// Four lanes per query row, each holding a quarter of the row's features of q
// and of the output accumulator; keys and values stream through LDS 16 at a
// time and the row softmax is accumulated online (running max, rescaled sum and
// accumulator), split over the waves of a workgroup. Serves the fp32 workloads,
// which are small; the bf16 path on the matrix cores is the fast one.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kKeys = 16;  // keys per LDS tile
// Waves per workgroup, wave w taking key tiles w, w + kSplit, ...: as many as
// keep the K and V tiles at 64 KiB of LDS (16 for D = 32, 8 for 64, 4 for 128),
// so that short sequences still spread over many waves.
template <int D>
constexpr int split_for() { return 4 * 128 / D; }

// 16 query rows per workgroup: lane = 4 * (row in the wave) + part, where part
// holds features part * D/4 .. +D/4. A score is the sum of the four parts'
// partial dot products (two lane exchanges; every lane of the row ends with the
// same value, as fp32 addition is commutative), so the four lanes keep identical
// running max and sum. The waves each run the online softmax over their share
// of the key tiles, and their (running max, sum, accumulator) are merged in a
// fixed binary tree through LDS at the end.
template <int D, int kSplit = split_for<D>()>
__global__ __launch_bounds__(64 * kSplit) void anchor_f32(const float* __restrict__ Q,
                                                          const float* __restrict__ K,
                                                          const float* __restrict__ V,
                                                          const float* __restrict__ G,
                                                          float* __restrict__ out, int N,
                                                          float scale, int accumulate) {
  constexpr int DP = D / 4;  // features per lane
  static_assert(2 * kSplit * kKeys * D >= kSplit / 2 * 64 * (DP + 2), "merge buffer fits in the tiles");
  __shared__ float lds[2 * kSplit * kKeys * D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, bh = blockIdx.y;
  const int part = lane & 3, qi = blockIdx.x * 16 + (lane >> 2);
  const size_t base = (size_t)bh * N * D;
  const bool live = qi < N;
  const float* Kt = lds + w * kKeys * D + part * DP;
  const float* Vt = lds + (kSplit + w) * kKeys * D + part * DP;

  // Every load is unconditional and 16 bytes wide: a row past the last query
  // reads row 0 and a key slot past the last key reads the last key, and the
  // values are then discarded, so the compiler can issue all of a tile's loads
  // before it waits (a load under a per-lane condition makes it wait for each).
  float q[DP], o[DP];
  const f32x4* Qr = reinterpret_cast<const f32x4*>(Q + base + (size_t)(live ? qi : 0) * D + part * DP);
#pragma unroll
  for (int x = 0; x < DP / 4; ++x) {
    const f32x4 t = Qr[x];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[4 * x + e] = live ? t[e] * scale : 0.f;
      o[4 * x + e] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;

  constexpr int NV = kKeys * D / 4 / 64;  // 16-byte loads per lane and tensor for one tile
  const f32x4* K4 = reinterpret_cast<const f32x4*>(K + base);
  const f32x4* V4 = reinterpret_cast<const f32x4*>(V + base);
  f32x4* Ks4 = reinterpret_cast<f32x4*>(lds + w * kKeys * D);
  f32x4* Vs4 = reinterpret_cast<f32x4*>(lds + (kSplit + w) * kKeys * D);
  const int ntiles = (N + kKeys - 1) / kKeys;
  const int rounds = (ntiles + kSplit - 1) / kSplit;
  for (int r = 0; r < rounds; ++r) {
    const int k0 = (r * kSplit + w) * kKeys;
    const int nk = max(0, min(kKeys, N - k0));
    f32x4 kv[NV], vv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i, row = e / (D / 4), c4 = e % (D / 4);
      const size_t src = (size_t)min(k0 + row, N - 1) * (D / 4) + c4;
      kv[i] = K4[src];
      vv[i] = V4[src];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i, row = e / (D / 4);
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      Ks4[e] = row < nk ? kv[i] : zero;
      Vs4[e] = row < nk ? vv[i] : zero;
    }
    __syncthreads();
    if (nk == 0) continue;  // a tile past the last key (wave-uniform)
    float s[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < DP; ++d) acc = fmaf(q[d], Kt[j * D + d], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      s[j] = j < nk ? acc : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mn = fmaxf(m, mt);
    const float alpha = expf(m - mn);  // 0 on the wave's first tile (m = -inf)
    m = mn;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < DP; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m);
      l += p;
#pragma unroll
      for (int d = 0; d < DP; ++d) o[d] = fmaf(p, Vt[j * D + d], o[d]);
    }
  }

  // binary-tree merge: at each step the upper half of the remaining waves hands
  // its state to the lower half through the tile memory
#pragma unroll
  for (int step = kSplit / 2; step >= 1; step >>= 1) {
    __syncthreads();
    if (w >= step && w < 2 * step) {
      float* red = lds + ((w - step) * 64 + lane) * (DP + 2);
      red[0] = m;
      red[1] = l;
#pragma unroll
      for (int d = 0; d < DP; ++d) red[2 + d] = o[d];
    }
    __syncthreads();
    if (w < step) {
      const float* red = lds + (w * 64 + lane) * (DP + 2);
      if (red[0] != -INFINITY) {  // that wave saw at least one key
        const float m2 = red[0], mn = fmaxf(m, m2);
        const float a = expf(m - mn), b = expf(m2 - mn);
        l = l * a + red[1] * b;
#pragma unroll
        for (int d = 0; d < DP; ++d) o[d] = o[d] * a + red[2 + d] * b;
        m = mn;
      }
    }
  }
  if (w != 0 || !live) return;
  const float inv = 1.0f / l;
  const size_t off = base + (size_t)qi * D + part * DP;
  const f32x4* G4 = reinterpret_cast<const f32x4*>(G + off);
  f32x4* O4 = reinterpret_cast<f32x4*>(out + off);
  f32x4 gv[DP / 4], pv[DP / 4];
#pragma unroll
  for (int x = 0; x < DP / 4; ++x) gv[x] = G4[x];
  if (accumulate) {
#pragma unroll
    for (int x = 0; x < DP / 4; ++x) pv[x] = O4[x];
  }
#pragma unroll
  for (int x = 0; x < DP / 4; ++x) {
    f32x4 rv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gate = 1.0f / (1.0f + expf(-gv[x][e]));
      rv[e] = gate * (o[4 * x + e] * inv);
    }
    if (accumulate) rv += pv[x];
    O4[x] = rv;
  }
}

template <int D>
hipError_t launch_d(const hla_dims& d, const void* q, const void* k, const void* v, const void* g,
                    void* out, int accumulate, float scale, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  hipLaunchKernelGGL(anchor_f32<D>, dim3((N + 15) / 16, BH), dim3(64 * split_for<D>()), 0, stream,
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
