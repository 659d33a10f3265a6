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
//                    k-step); V stays row-major in LDS and the V^T operand comes
//                    from two LDS transpose reads per MFMA.
// K and V tiles arrive through buffer loads, which return zeros past the end of
// the head, so the last partial tile needs no predicated loads.
// The epilogue divides by the row sum, applies the sigmoid gate and stores O
// (bf16) or adds it into an fp32 residual stream.
#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per LDS tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

// LDS tiles are row-major (one key per row) with XOR swizzles of whole chunks
// instead of padding:
//   K: 16-byte chunk c of row k sits at chunk c ^ (k & 15) (c ^ (k & 7) for D=64),
//      so the 32 rows one S^T operand read touches spread over all banks;
//   V: 8-byte chunk c of row k sits at chunk c ^ kVx[k & 3], which keeps the
//      transposed (ds_read_b64_tr_b16) operand reads of 16 lanes on 16 distinct
//      bank pairs.
template <int D>
struct AnchorSwz;
template <>
struct AnchorSwz<128> {
  static constexpr int kmask = 15;
  __device__ static int vx8(int k) { return (0x18120a00 >> (8 * (k & 3))) & 0xff; }  // 0,10,18,24
};
template <>
struct AnchorSwz<64> {
  static constexpr int kmask = 7;
  __device__ static int vx8(int k) { return (0x08020a00 >> (8 * (k & 3))) & 0xff; }  // 0,10,2,8
};

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void anchor_bf16(const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ G,
                                                      void* __restrict__ out, int N, int nqb,
                                                      int total, float c, int accumulate) {
  constexpr int NK = D / 16;              // k-steps of S^T
  constexpr int ND = D / 32;              // 32-row blocks of O^T
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int LOADS = kBC * CH / 256;   // 16-byte loads per thread per tensor per tile
  constexpr uint32_t kTileBytes = kBC * D * 2;
  using Swz = AnchorSwz<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBC * D];

  // Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
  // each XCD runs a contiguous range of (b, h, query block) and the query
  // blocks of one head share that XCD's L2 while streaming its K and V.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int logical =
      xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int bh = logical / nqb, qb = logical - bh * nqb;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index, made visibly wave-uniform (it selects the M0 LDS base of the
  // direct-to-LDS loads, which must be a scalar)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const int qrow = qb * kBR + wave * 32 + r;

  u32x4 qf[NK];
  {
    const rsrc_t Qr = make_rsrc(Q + base, head_bytes);
    const uint32_t qoff = qrow < N ? (uint32_t)qrow * D * 2 : head_bytes;  // past N reads 0
#pragma unroll
    for (int t = 0; t < NK; ++t) qf[t] = buf_load16(Qr, qoff + (16 * t + 8 * h) * 2);
  }

  // Tiles go global -> LDS directly (buffer_load ... lds): instruction i of
  // wave w fills the 1 KB LDS block bw = LOADS*w + i, i.e. rows 4bw..4bw+3 with
  // lane l at row 4bw + l/16, physical 16-byte chunk l%16. Each lane fetches
  // the logical chunk that the swizzle puts there.
  constexpr int ROWS_PER_BLK = 1024 / (D * 2);   // 4 rows of 256 B (8 for D=64)
  uint32_t goff_k[LOADS], goff_v[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int blk = LOADS * wave + i;
    const int row = blk * ROWS_PER_BLK + lane / CH, pc = lane % CH;
    const int ck = pc ^ (row & Swz::kmask);
    const int cv = (2 * pc ^ Swz::vx8(row)) / 2;
    goff_k[i] = (row * D + ck * 8) * 2;
    goff_v[i] = (row * D + cv * 8) * 2;
  }
  // issue tile j into LDS buffer buf (completion: wait_all_memory + barrier)
  auto load_tile = [&](int j, int buf) {
    const uint32_t done = (uint32_t)j * kTileBytes;
    const uint32_t left = done < head_bytes ? head_bytes - done : 0u;
    const rsrc_t kr = make_rsrc_uniform(K + base + (size_t)j * kBC * D, left);
    const rsrc_t vr = make_rsrc_uniform(V + base + (size_t)j * kBC * D, left);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int blk = LOADS * wave + i;
      buf_load16_lds(kr, goff_k[i], &Ks[buf][blk * 512]);
      buf_load16_lds(vr, goff_v[i], &Vs[buf][blk * 512]);
    }
  };

  // S^T operand A (key rows): lane reads row kb*32 + r, chunk 2t + h (swizzled)
  int koff[NK];
#pragma unroll
  for (int t = 0; t < NK; ++t) koff[t] = r * D + (((2 * t + h) ^ (r & Swz::kmask)) * 8);
  // O^T operand A (V^T) through transposed reads: source lane (e = (lane>>2)&3,
  // q = lane&3) of each 16-lane group points at key 4h + e (+16 ks, +8 for the
  // upper four k-slots) and at the 4 features of output rows R = 16 g + 4 q..+3,
  // where MFMA row R maps to feature 16((R>>2)&1) + 4(R>>3) + (R&3) of block b.
  const int ve = (lane >> 2) & 3, vq = lane & 3, vg = (lane >> 4) & 1;
  const int vkey = 4 * h + ve;
  int voff[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) {
    const int chunk8 = b * 8 + 4 * (vq & 1) + (vq >> 1) + 2 * vg;
    voff[b] = vkey * D + ((chunk8 ^ Swz::vx8(vkey)) * 4);
  }

  f32x16 acc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) acc[b] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  // One key tile: tile j sits in LDS buffer BUF (= j & 1, a compile-time
  // constant so every LDS address is a per-lane base plus an immediate); MASK
  // marks the ragged last tile, the only one that needs keys >= N masked.
  const int ntiles = (N + kBC - 1) / kBC;
  auto step = [&](auto buf_c, auto mask_c, int j) {
    constexpr int BUF = decltype(buf_c)::value;
    constexpr bool MASK = decltype(mask_c)::value;
    if (j + 1 < ntiles) load_tile(j + 1, BUF ^ 1);
    const uint16_t* Kb = Ks[BUF];
    const uint16_t* Vb = Vs[BUF];

    // S^T (keys x queries) for two 32-key blocks
    f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int t = 0; t < NK; ++t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Kb[kb * 32 * D + koff[t]]);
        s[kb] = mfma32x32x16(a, qf[t], s[kb]);
      }
    }
    if (MASK) {
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
      // a real branch: the empty volatile asm keeps the compiler from turning
      // this rarely taken rescale into straight-line code run on every tile
      asm volatile("");
      const float m_new = need ? mt : m_run;
      const float alpha = exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < ND; ++b) acc[b] *= alpha;
      m_run = m_new;
    }
    // P = 2^(s*c - m) packed to bf16 B operands (4 k-steps of 16 keys); the row
    // sum adds the same rounded values the MFMA consumes
    u32x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) p[x] = exp2_fast(fmaf(s[kb][x], c, -m_run));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qq = half * 8;
        pb[kb * 2 + half] = (u32x4){pack_bf16(p[qq + 0], p[qq + 1]), pack_bf16(p[qq + 2], p[qq + 3]),
                                    pack_bf16(p[qq + 4], p[qq + 5]), pack_bf16(p[qq + 6], p[qq + 7])};
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int x = 0; x < 4; ++x) l_run = add_bf16x2(pb[ks][x], l_run);
    // O^T += V^T P^T; k-slot s of half h is key 16ks + 8(s>>2) + 4h + (s&3)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int b = 0; b < ND; ++b) {
        const u32x2 lo = lds_read_tr16(&Vb[ks * 16 * D + voff[b]]);
        const u32x2 hi = lds_read_tr16(&Vb[(ks * 16 + 8) * D + voff[b]]);
        acc[b] = mfma32x32x16((u32x4){lo[0], lo[1], hi[0], hi[1]}, pb[ks], acc[b]);
      }
    }
    wait_all_memory();  // tile j + 1 has landed in LDS
    __syncthreads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using Full = std::false_type;
  using Ragged = std::true_type;

  load_tile(0, 0);
  wait_all_memory();
  __syncthreads();
  const int nfull = N / kBC;
  int j = 0;
  for (; j + 2 <= nfull; j += 2) {
    step(B0{}, Full{}, j);
    step(B1{}, Full{}, j + 1);
  }
  if (j < nfull) {
    step(B0{}, Full{}, j);
    ++j;
    if (j < ntiles) step(B1{}, Ragged{}, j);
  } else if (j < ntiles) {
    step(B0{}, Ragged{}, j);
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
