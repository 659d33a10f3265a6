// Block attention residuals (AttnRes): routing the summaries of completed
// 8-layer blocks into the residual stream a later linear layer reads.
//
// SANA-Video 2.0 groups consecutive layers into blocks of 8 and routes a summary
// of each completed block directly into later linear layers, through a router
// whose query projection is shared across depth (ai-papers.net summary, section
// on attention residuals; lode.cx article, "The Core Innovation"; SANA-Video 2.0
// abstract). The pages give no formula; the reading built here is, per token n
// of one (b, h):
//   q_n = x_n W                         (W: D x D bf16, one matrix for all layers)
//   a_i = q_n . s_i,n / sqrt(D)         (s_i: summary of completed block i)
//   out_n = x_n + sum_i softmax_i(a)_i s_i,n
// x, the summaries and out are fp32 [B, H, N, D] (the residual stream).
//
// One pass over HBM: each wave takes 16 tokens at a time, moved as whole 1 KB
// runs through a per-wave LDS tile; in registers lane (n = lane & 15,
// g = lane >> 4) owns features 32t + 8g .. +7 (t < D/32) of token n. q comes
// from 16x16x32 bf16 MFMAs with W^T fragments in LDS and x split into a bf16
// hi + lo pair as the B operands (about 16 significant bits of x: the scores are
// exponentiated, so an 8-bit x would move them by up to ~0.1 when they spread
// over tens of units), and lands in the same lanes and features as the lane's x slice,
// so the score of block i is the lane's partial dot product summed over the
// four lanes of the token. The blocks are streamed once each through an online
// softmax (running max, running sum, running weighted summary), so any number
// of blocks costs one read of each.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

// Fragment (j, t) of W^T for the 16x16x32 MFMA: A[i][k] = W[32t + k][c(j, i)] with
// c(j, i) = 32(j>>1) + 8(i>>2) + 4(j&1) + (i&3), so output lane (n, g) ends with
// q at features 32t + 8g + 0..7 from fragments j = 2t, 2t+1 (as its x slice).
template <int D>
__device__ __forceinline__ u32x4 w_fragment(const uint16_t* __restrict__ W, int j, int t, int l) {
  const int i = l & 15, k0 = 8 * (l >> 4);
  const int col = 32 * (j >> 1) + 8 * (i >> 2) + 4 * (j & 1) + (i & 3);
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = 32 * t + k0 + 2 * p;
    w[p] = uint32_t(W[row * D + col]) | (uint32_t(W[(row + 1) * D + col]) << 16);
  }
  return (u32x4){w[0], w[1], w[2], w[3]};
}

// 16-byte chunk c of token row t (R = D / 4 chunks per fp32 row, 16 or 32) in a
// wave's staging tile: t R + (c ^ (t mod 16)), so the 16 lanes of one 16-byte LDS
// access (16 consecutive chunks of a 1 KB run, or one chunk of 16 rows) land on 16
// distinct bank groups.
template <int R>
__device__ __forceinline__ int run_slot(int t, int c) { return t * R + (c ^ (t & 15)); }

// A wave's tile is written by some lanes and read by others; a wave's LDS
// instructions execute in issue order, so keeping the compiler from moving them
// across this point is all the ordering needed.
__device__ __forceinline__ void wave_order() { asm volatile("" ::: "memory"); }

// X may be out itself (in place): no __restrict__ on either.
template <int D>
__global__ __launch_bounds__(256, 2) void attnres_route(const float* X,
                                                        AttnResBlocks S, int M,
                                                        const uint16_t* __restrict__ W,
                                                        float* out, int N) {
  constexpr int NT = D / 32, NJ = D / 16, NF = NJ * NT;
  constexpr int R = D / 4;         // 16-byte chunks per fp32 token row
  constexpr int NL = 16 * R / 64;  // 1 KB runs per 16-token group and tensor
  __shared__ u32x4 fr[NF * 64];
  __shared__ f32x4 tile[4][16 * R];  // per wave: one tensor's group at a time
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int x = tid; x < NF * 64; x += 256) {
    const int f = x >> 6;
    fr[x] = w_fragment<D>(W, f / NT, f % NT, x & 63);
  }
  __syncthreads();

  const int bh = blockIdx.y, n = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * N * D;
  const float c = kLog2e * rsqrtf((float)D);  // scores in log2 units
  const int stride = gridDim.x * 4;
  f32x4* const tl = tile[wave];
  // Every tensor moves through HBM as whole 1 KB runs (lane l of run u: chunk
  // 64u + l of the group's 16 rows), read once with the non-temporal cache
  // policy; the tile turns them into the operand layout -- lane (n, g) takes
  // chunks 8t + 2g and 8t + 2g + 1 of token n (features 32t + 8g .. +7) -- and the
  // result back into runs. Rows past N read as zeros and are never stored.
  for (int grp = blockIdx.x * 4 + wave; grp * 16 < N; grp += stride) {
    const size_t gbase = base + (size_t)grp * 16 * D;
    auto load_runs = [&](const float* T, f32x4* raw) {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int k = 64 * u + lane;
        raw[u] = grp * 16 + k / R < N ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(T + gbase + 4 * k))
                                      : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    };
    auto stage = [&](const f32x4* raw, f32x4* v) {
      wave_order();
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int k = 64 * u + lane;
        tl[run_slot<R>(k / R, k % R)] = raw[u];
      }
      wave_order();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        v[2 * t] = tl[run_slot<R>(n, 8 * t + 2 * g)];
        v[2 * t + 1] = tl[run_slot<R>(n, 8 * t + 2 * g + 1)];
      }
    };
    f32x4 raw[NL], sraw[NL], xv[2 * NT];
    load_runs(X, raw);
    if (M > 0) load_runs(S.p[0], sraw);
    stage(raw, xv);

    // q = x W on the matrix cores. The fragments are re-read from LDS every
    // group: an opaque (always equal) offset keeps the compiler from hoisting all
    // of them into registers, which would spill.
    int fo = lane;
    asm volatile("" : "+v"(fo));
    f32x4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float v[8], lo[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = xv[2 * t][e];
        v[4 + e] = xv[2 * t + 1][e];
      }
      u32x4 bh, bl;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        bh[p] = pack_bf16(v[2 * p], v[2 * p + 1]);
        lo[2 * p] = v[2 * p] - bf_lo(bh[p]);
        lo[2 * p + 1] = v[2 * p + 1] - bf_hi(bh[p]);
        bl[p] = pack_bf16(lo[2 * p], lo[2 * p + 1]);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 a = fr[(j * NT + t) * 64 + fo];
        acc[j] = mfma16x16x32(a, bh, acc[j]);
        acc[j] = mfma16x16x32(a, bl, acc[j]);
      }
    }

    // online softmax over the blocks
    float m = -INFINITY, l = 0.f;
    f32x4 r[2 * NT];
#pragma unroll
    for (int x = 0; x < 2 * NT; ++x) r[x] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < M; ++i) {
      f32x4 cur[2 * NT];
      stage(sraw, cur);
      if (i + 1 < M) load_runs(S.p[i + 1], sraw);  // next block in flight
      float part = 0.f;
#pragma unroll
      for (int x = 0; x < 2 * NT; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(acc[x][e], cur[x][e], part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      // rounded on its own (the empty asm pins the product): a fused
      // c * part - m_new would leave the product's rounding error where a - m_new
      // must be exactly 0 for the largest score
      float a = part * c;
      asm volatile("" : "+v"(a));
      const float m_new = fmaxf(m, a);
      const float corr = exp2_fast(m - m_new), p = exp2_fast(a - m_new);
      l = fmaf(l, corr, p);
#pragma unroll
      for (int x = 0; x < 2 * NT; ++x) r[x] = r[x] * corr + p * cur[x];
      m = m_new;
    }
    const float inv = M > 0 ? 1.0f / l : 0.f;
    wave_order();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      tl[run_slot<R>(n, 8 * t + 2 * g)] = xv[2 * t] + r[2 * t] * inv;
      tl[run_slot<R>(n, 8 * t + 2 * g + 1)] = xv[2 * t + 1] + r[2 * t + 1] * inv;
    }
    wave_order();
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int k = 64 * u + lane;
      const f32x4 o = tl[run_slot<R>(k / R, k % R)];
      if (grp * 16 + k / R < N) *reinterpret_cast<f32x4*>(out + gbase + 4 * k) = o;
    }
  }
}

}  // namespace

hipError_t launch_attnres_route(const hla_dims& d, int n_blocks, const AttnResBlocks& blocks,
                                const void* x, const void* w, void* out, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  const int groups = (N + 15) / 16;
  int P = (1024 + BH - 1) / BH;  // about four workgroups per CU in all
  const int maxp = (groups + 3) / 4;
  P = P < 1 ? 1 : (P > maxp ? maxp : P);
  const float* X = reinterpret_cast<const float*>(x);
  const uint16_t* W = reinterpret_cast<const uint16_t*>(w);
  float* O = reinterpret_cast<float*>(out);
  if (d.D == 128)
    hipLaunchKernelGGL(attnres_route<128>, dim3(P, BH), dim3(256), 0, stream, X, blocks, n_blocks, W, O, N);
  else
    hipLaunchKernelGGL(attnres_route<64>, dim3(P, BH), dim3(256), 0, stream, X, blocks, n_blocks, W, O, N);
  return hipGetLastError();
}

}  // namespace hla
