// Gated linear attention, fp32 inputs, fp32 arithmetic throughout (vector ALU).
//
// Same three steps as the bf16 path -- per-chunk partial state, fixed-order
// reduce, output pass -- but with plain fp32 FMAs so the result stays within
// fp32 rounding of the exact operator. It serves the fp32 workloads, which are
// small; the bf16 path is the fast one.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kTileF = 32;  // tokens per LDS tile

// partial S_c = phi(K_c)^T V_c and z_c; thread (ty, tx) owns an R x R block of S.
// W (optional, [B,H,N]): write-gate logits; token n's phi(K_n) is scaled by
// sigma(W_n) in both S and z.
template <int D>
__global__ __launch_bounds__(256) void linear_state_f32(const float* __restrict__ K,
                                                        const float* __restrict__ V,
                                                        const float* __restrict__ W,
                                                        float* __restrict__ part, int N, int T,
                                                        int C) {
  constexpr int R = D / 16;
  __shared__ float Ks[kTileF][D];
  __shared__ float Vs[kTileF][D];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int n0 = c * T, n1 = min(N, n0 + T);
  const size_t base = (size_t)bh * N * D;
  float acc[R][R];
  float z[R];
#pragma unroll
  for (int x = 0; x < R; ++x) {
    z[x] = 0.f;
#pragma unroll
    for (int y = 0; y < R; ++y) acc[x][y] = 0.f;
  }
  // Tile loads are unconditional 16-byte loads (a row past the chunk reads the
  // chunk's last row and is then zeroed), so they are all in flight at once.
  constexpr int NV = kTileF * D / 4 / 256;  // 16-byte loads per thread and tensor
  const f32x4* K4 = reinterpret_cast<const f32x4*>(K + base);
  const f32x4* V4 = reinterpret_cast<const f32x4*>(V + base);
  f32x4* Ks4 = reinterpret_cast<f32x4*>(&Ks[0][0]);
  f32x4* Vs4 = reinterpret_cast<f32x4*>(&Vs[0][0]);
  for (int t0 = n0; t0 < n1; t0 += kTileF) {
    f32x4 kv[NV], vv[NV];
    float wl[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, row = e / (D / 4), c4 = e % (D / 4);
      const int src = min(t0 + row, n1 - 1);
      kv[i] = K4[(size_t)src * (D / 4) + c4];
      vv[i] = V4[(size_t)src * (D / 4) + c4];
      wl[i] = W != nullptr ? W[(size_t)bh * N + src] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, row = e / (D / 4);
      const bool live = t0 + row < n1;
      const float beta = W != nullptr ? sigmoid(wl[i]) : 1.f;
      f32x4 kk, vz;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        kk[x] = live ? fmaxf(kv[i][x], 0.f) * beta : 0.f;
        vz[x] = live ? vv[i][x] : 0.f;
      }
      Ks4[e] = kk;
      Vs4[e] = vz;
    }
    __syncthreads();
    for (int n = 0; n < kTileF; ++n) {
      float a[R], b[R];
#pragma unroll
      for (int x = 0; x < R; ++x) {
        a[x] = Ks[n][ty * R + x];
        b[x] = Vs[n][tx * R + x];
      }
#pragma unroll
      for (int x = 0; x < R; ++x) {
        z[x] += a[x];
#pragma unroll
        for (int y = 0; y < R; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
      }
    }
  }
  float* P = part + ((size_t)bh * C + c) * (size_t)(D * D + D);
#pragma unroll
  for (int x = 0; x < R; ++x)
#pragma unroll
    for (int y = 0; y < R; ++y) P[(ty * R + x) * D + tx * R + y] = acc[x][y];
  if (tx == 0) {
#pragma unroll
    for (int x = 0; x < R; ++x) P[D * D + ty * R + x] = z[x];
  }
}

// S = sum_c S_c, z = sum_c z_c in chunk order; state is [BH][D*D + D] fp32
template <int D>
__global__ __launch_bounds__(256) void linear_reduce_f32(const float* __restrict__ part,
                                                         float* __restrict__ state, int C) {
  const size_t stride = (size_t)D * D + D;
  const int e = blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (e >= (int)stride) return;
  const float* P = part + (size_t)bh * C * stride + e;
  float s = 0.f;
  for (int c = 0; c < C; ++c) s += P[c * stride];
  state[(size_t)bh * stride + e] = s;
}

// O = sigma(G) (.) (phi(Q) S) / (phi(Q) . z + eps); thread (n, jg) owns D/8
// outputs of token n; S streams through LDS 32 rows at a time
template <int D>
__global__ __launch_bounds__(256) void linear_out_f32(const float* __restrict__ Q,
                                                      const float* __restrict__ G,
                                                      float* __restrict__ out,
                                                      const float* __restrict__ state, int N,
                                                      float eps, int accumulate) {
  constexpr int J = D / 8;
  __shared__ float Qs[32][D];
  __shared__ float Ss[32][D];
  const int tid = threadIdx.x, n = tid >> 3, jg = tid & 7;
  const int bh = blockIdx.y, t0 = blockIdx.x * 32;
  const size_t base = (size_t)bh * N * D;
  const float* S = state + (size_t)bh * (D * D + D);
  const float* z = S + D * D;
  // unconditional 16-byte loads, as in the state pass (rows past N read row N-1)
  constexpr int NV = 32 * D / 4 / 256;
  {
    const f32x4* Q4 = reinterpret_cast<const f32x4*>(Q + base);
    f32x4 qv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, row = e / (D / 4), c4 = e % (D / 4);
      qv[i] = Q4[(size_t)min(t0 + row, N - 1) * (D / 4) + c4];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i, row = e / (D / 4);
      f32x4 r;
#pragma unroll
      for (int x = 0; x < 4; ++x) r[x] = t0 + row < N ? fmaxf(qv[i][x], 0.f) : 0.f;
      reinterpret_cast<f32x4*>(&Qs[0][0])[e] = r;
    }
  }
  float acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = 0.f;
  const f32x4* S4 = reinterpret_cast<const f32x4*>(S);
#pragma unroll 1
  for (int i0 = 0; i0 < D; i0 += 32) {
    f32x4 sv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) sv[i] = S4[i0 * (D / 4) + tid + 256 * i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) reinterpret_cast<f32x4*>(&Ss[0][0])[tid + 256 * i] = sv[i];
    __syncthreads();
    for (int ii = 0; ii < 32; ++ii) {
      const float a = Qs[n][i0 + ii];
#pragma unroll
      for (int j = 0; j < J; ++j) acc[j] = fmaf(a, Ss[ii][jg * J + j], acc[j]);
    }
  }
  float den = 0.f;
#pragma unroll 8
  for (int i = 0; i < D; ++i) den = fmaf(Qs[n][i], z[i], den);
  den += eps;
  const int tok = t0 + n;
  if (tok >= N) return;
  // J consecutive outputs: their gate (and previous output) loads go out together
  const size_t off = base + (size_t)tok * D + jg * J;
  const f32x4* G4 = reinterpret_cast<const f32x4*>(G + off);
  f32x4* O4 = reinterpret_cast<f32x4*>(out + off);
  f32x4 gv[J / 4], pv[J / 4];
#pragma unroll
  for (int x = 0; x < J / 4; ++x) gv[x] = G4[x];
  if (accumulate) {
#pragma unroll
    for (int x = 0; x < J / 4; ++x) pv[x] = O4[x];
  }
#pragma unroll
  for (int x = 0; x < J / 4; ++x) {
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gate = 1.0f / (1.0f + expf(-gv[x][e]));
      o[e] = gate * (acc[4 * x + e] / den);
    }
    if (accumulate) o += pv[x];
    O4[x] = o;
  }
}

template <int D>
hipError_t launch_d(const hla_dims& d, const void* q, const void* k, const void* v, const void* g,
                    const void* wg, void* out, int accumulate, float eps, void* ws,
                    const LinearPlan& plan, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  char* w = reinterpret_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w + plan.part_off);
  float* state = reinterpret_cast<float*>(w + plan.state_off);
  hipLaunchKernelGGL(linear_state_f32<D>, dim3(plan.C, BH), dim3(256), 0, stream,
                     reinterpret_cast<const float*>(k), reinterpret_cast<const float*>(v),
                     reinterpret_cast<const float*>(wg), part, N, plan.T, plan.C);
  hipLaunchKernelGGL(linear_reduce_f32<D>, dim3((D * D + D + 255) / 256, BH), dim3(256), 0,
                     stream, part, state, plan.C);
  hipLaunchKernelGGL(linear_out_f32<D>, dim3((N + 31) / 32, BH), dim3(256), 0, stream,
                     reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(g),
                     reinterpret_cast<float*>(out), state, N, eps, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_f32(const hla_dims& d, const void* q, const void* k, const void* v,
                             const void* g, const void* w, void* out, int accumulate, float eps,
                             void* ws, const LinearPlan& plan, hipStream_t stream) {
  switch (d.D) {
    case 32: return launch_d<32>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
    case 64: return launch_d<64>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
    default: return launch_d<128>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
  }
}

}  // namespace hla
