// Gated softmax anchor, bf16 inputs, on gfx950 matrix cores.
//
// O = sigma(G) (.) softmax_rows(scale * Q K^T) V, non-causal: the periodic
// gated-softmax layer of SANA-Video 2.0 that restores exact token interactions
// between gated linear layers (SANA-Video 2.0 abstract, thelatestinai.com
// listing; lode.cx article, "The Core Innovation" and "How It Works").
//
// Flash-style single pass: a workgroup owns 128 query rows (4 waves x 32) of
// one (b, h) and streams all keys through LDS in tiles of 64, double-buffered.
// Per tile and wave:
//   S^T = K Q^T      32x32x16 bf16 MFMA, K from LDS, Q^T held in registers; the
//                    transposed product puts one query per lane (and its
//                    partner lane ^ 32), so row max and row sum need one swap.
//   online softmax   in log2 units with a lazily updated running max: the
//                    accumulator is rescaled only when a row's max grows by
//                    more than 2^8, which keeps exp2 arguments <= 8 and the
//                    result exact up to rounding.
//   O^T += V^T P^T   P^T stays in registers (the MFMA result layout is reused as
//                    the next B operand by permuting the key order inside each
//                    k-step); V is stored transposed in LDS so each lane reads
//                    its 8 keys as two 8-byte loads.
// The epilogue divides by the row sum, applies the sigmoid gate and stores O
// (bf16) or adds it into an fp32 residual stream.
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per LDS tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void anchor_bf16(const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ G,
                                                      void* __restrict__ out, int N, int nqb,
                                                      int total, float c, int accumulate) {
  constexpr int KS = D + 8;        // K tile row stride (elements)
  constexpr int VS = kBC + 4;      // V^T tile row stride (elements)
  constexpr int NK = D / 16;       // k-steps of S^T
  constexpr int ND = D / 32;       // 32-row blocks of O^T
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int KLOADS = kBC * CH / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBC * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VS];

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // each XCD runs a contiguous range of (b, h, query block) and the query
  // blocks of one head share that XCD's L2 while streaming its K and V.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int logical =
      xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int bh = logical / nqb, qb = logical - bh * nqb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const int qrow = qb * kBR + wave * 32 + r;

  u32x4 qf[NK];
#pragma unroll
  for (int t = 0; t < NK; ++t)
    qf[t] = qrow < N ? ldg16(Qh + (size_t)qrow * D + 16 * t + 8 * h) : (u32x4){0, 0, 0, 0};

  // tile loaders: K row-major, V as 4 keys x 8 features per thread
  const int kq = tid & 15, dc = tid >> 4;
  const bool vload = dc < CH;
  u32x4 kr[KLOADS], vr[4];
  auto load_tile = [&](int j) {
    const int k0 = j * kBC;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int chunk = tid + 256 * i;
      const int key = k0 + chunk / CH, col = (chunk % CH) * 8;
      kr[i] = key < N ? ldg16(Kh + (size_t)key * D + col) : (u32x4){0, 0, 0, 0};
    }
    if (vload) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + 4 * kq + i;
        vr[i] = key < N ? ldg16(Vh + (size_t)key * D + 8 * dc) : (u32x4){0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int chunk = tid + 256 * i;
      const int row = chunk / CH, col = (chunk % CH) * 8;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KS + col]) = kr[i];
    }
    if (vload) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t e0 = (vr[0][p] & 0xffffu) | (vr[1][p] << 16);
        const uint32_t e1 = (vr[2][p] & 0xffffu) | (vr[3][p] << 16);
        const uint32_t o0 = (vr[0][p] >> 16) | (vr[1][p] & 0xffff0000u);
        const uint32_t o1 = (vr[2][p] >> 16) | (vr[3][p] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(&Vt[buf][(8 * dc + 2 * p) * VS + 4 * kq]) = (u32x2){e0, e1};
        *reinterpret_cast<u32x2*>(&Vt[buf][(8 * dc + 2 * p + 1) * VS + 4 * kq]) = (u32x2){o0, o1};
      }
    }
  };

  f32x16 acc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) acc[b] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // row of V^T that MFMA row r reads, so each lane ends with 16 consecutive
  // output features: d = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3)
  const int vrow = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);

  const int ntiles = (N + kBC - 1) / kBC;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);

    // S^T (keys x queries) for two 32-key blocks
    f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int t = 0; t < NK; ++t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[buf][(kb * 32 + r) * KS + 16 * t + 8 * h]);
        s[kb] = mfma32x32x16(a, qf[t], s[kb]);
      }
    }
    // keys past N in the last tile
    if ((j + 1) * kBC > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int key = j * kBC + kb * 32 + (x >> 2) * 8 + 4 * h + (x & 3);
          if (key >= N) s[kb][x] = -INFINITY;
        }
    }
    // row max over this tile (own 32 scores, then the partner lane's)
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int x = 0; x < 16; ++x) mt = fmaxf(mt, s[kb][x]);
    mt = fmaxf(mt, swap_halves(mt)) * c;
    const bool need = mt > m_run + kTau;
    if (__any(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < ND; ++b) acc[b] *= alpha;
      m_run = m_new;
    }
    // P = 2^(s*c - m), row sum, pack to bf16 B operands (4 k-steps of 16 keys)
    u32x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        p[x] = exp2_fast(fmaf(s[kb][x], c, -m_run));
        l_run += p[x];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qq = half * 2;
        pb[kb * 2 + half] = (u32x4){pack_bf16(p[qq * 4 + 0], p[qq * 4 + 1]),
                                    pack_bf16(p[qq * 4 + 2], p[qq * 4 + 3]),
                                    pack_bf16(p[qq * 4 + 4], p[qq * 4 + 5]),
                                    pack_bf16(p[qq * 4 + 6], p[qq * 4 + 7])};
      }
    }
    // O^T += V^T P^T; k-slot s of half h is key 16ks + 8(s>>2) + 4h + (s&3)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int b = 0; b < ND; ++b) {
        const uint16_t* vp = &Vt[buf][(b * 32 + vrow) * VS + ks * 16 + 4 * h];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
        acc[b] = mfma32x32x16((u32x4){lo[0], lo[1], hi[0], hi[1]}, pb[ks], acc[b]);
      }
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane (query r, half h) holds features 32b + 16h + 0..15 of block b
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow >= N) return;
#pragma unroll
  for (int b = 0; b < ND; ++b) {
    const size_t off = base + (size_t)qrow * D + 32 * b + 16 * h;
    const u32x4 g0 = ldg16(G + off), g1 = ldg16(G + off + 8);
    float o[16];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      o[2 * p] = (acc[b][2 * p] * inv) * sigmoid(bf_lo(g0[p]));
      o[2 * p + 1] = (acc[b][2 * p + 1] * inv) * sigmoid(bf_hi(g0[p]));
      o[8 + 2 * p] = (acc[b][8 + 2 * p] * inv) * sigmoid(bf_lo(g1[p]));
      o[8 + 2 * p + 1] = (acc[b][8 + 2 * p + 1] * inv) * sigmoid(bf_hi(g1[p]));
    }
    if (OUT_F32) {
      float* dst = reinterpret_cast<float*>(out) + off;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        f32x4 v = (f32x4){o[4 * x], o[4 * x + 1], o[4 * x + 2], o[4 * x + 3]};
        if (accumulate) v += *reinterpret_cast<const f32x4*>(dst + 4 * x);
        *reinterpret_cast<f32x4*>(dst + 4 * x) = v;
      }
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(out) + off;
      if (accumulate) {
        const u32x4 p0 = ldg16(dst), p1 = ldg16(dst + 8);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          o[2 * p] += bf_lo(p0[p]);
          o[2 * p + 1] += bf_hi(p0[p]);
          o[8 + 2 * p] += bf_lo(p1[p]);
          o[8 + 2 * p + 1] += bf_hi(p1[p]);
        }
      }
      stg16(dst, (u32x4){pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
                         pack_bf16(o[6], o[7])});
      stg16(dst + 8, (u32x4){pack_bf16(o[8], o[9]), pack_bf16(o[10], o[11]),
                             pack_bf16(o[12], o[13]), pack_bf16(o[14], o[15])});
    }
  }
}

template <int D>
hipError_t launch_d(const hla_dims& d, const void* q, const void* k, const void* v, const void* g,
                    void* out, int accumulate, float scale, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  const int nqb = (N + kBR - 1) / kBR;
  const int total = BH * nqb;
  const float c = scale * kLog2e;
  if (d.out_dtype == HLA_F32)
    hipLaunchKernelGGL((anchor_bf16<D, true>), dim3(total), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                       reinterpret_cast<const uint16_t*>(v), reinterpret_cast<const uint16_t*>(g),
                       out, N, nqb, total, c, accumulate);
  else
    hipLaunchKernelGGL((anchor_bf16<D, false>), dim3(total), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                       reinterpret_cast<const uint16_t*>(v), reinterpret_cast<const uint16_t*>(g),
                       out, N, nqb, total, c, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_anchor_bf16(const hla_dims& d, const void* q, const void* k, const void* v,
                              const void* g, void* out, int accumulate, float scale,
                              hipStream_t stream) {
  if (d.D == 128) return launch_d<128>(d, q, k, v, g, out, accumulate, scale, stream);
  return launch_d<64>(d, q, k, v, g, out, accumulate, scale, stream);
}

}  // namespace hla
