// Gated softmax anchor, bf16 or fp8 (OCP e4m3) inputs, on gfx950 matrix cores.
//
// O = sigma(G) (.) softmax_rows(scale * Q K^T) V, non-causal: the periodic
// gated-softmax layer of SANA-Video 2.0 that restores exact token interactions
// between gated linear layers (SANA-Video 2.0 abstract, thelatestinai.com
// listing; lode.cx article, "The Core Innovation" and "How It Works").
//
// Flash-style single pass: a workgroup owns 256 query rows (8 waves x 32, two
// waves per SIMD) of one (b, h) and streams all keys through LDS in tiles of
// 64, four buffers deep with one barrier per two tiles; the eight waves share
// each tile, so K and V cross from L2 into LDS once per 256 queries.
// Per tile and wave:
//   S^T = K Q^T      32x32x16 bf16 MFMA (32x32x64 fp8 MFMA for fp8 inputs, exact
//                    products), K from LDS, Q^T held in registers; the
//                    transposed product puts one query per lane (and its
//                    partner lane ^ 32), so row max and row sum need one swap.
//   online softmax   in log2 units with a lazily updated running max: the
//                    accumulator is rescaled only when a row's max grows by
//                    more than 2^8, which keeps exp2 arguments <= 8 and the
//                    result exact up to rounding.
//   O^T += V^T P^T   P^T stays in registers (the MFMA result layout is reused as
//                    the next B operand by permuting the key order inside each
//                    k-step). V is repacked once per call into V^T rows (a
//                    workspace, zero keys past N) in the key order P^T uses,
//                    so each V^T operand is one 16-byte LDS read (two for fp8).
//                    By default P is rounded to bf16 and V^T is bf16 (fp8 V
//                    converts exactly): 32x32x16 bf16 MFMA. In the fp8-P mode
//                    (fp8 inputs only) P is rounded to e4m3 (P <= 2^8 by the
//                    lazy max) and V^T stays e4m3: one 32x32x64 fp8 MFMA per
//                    64-key tile and 32-row block. The row sum always adds the
//                    same rounded P the matrix cores consume.
// K and V^T tiles go from HBM straight into LDS through buffer loads, which
// return zeros past the end of the head, so the last partial tile needs no
// predicated loads; only its scores past N are masked.
// The epilogue divides by the row sum, applies the sigmoid gate and stores O
// (bf16) or adds it into an fp32 residual stream.
#include <type_traits>

#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

constexpr int kWaves = 8;               // waves per workgroup, 32 query rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;        // query rows per workgroup
constexpr int kBC = 64;   // keys per LDS tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kMaxPieces = 1024;  // most key-range pieces one call splits its last batch into

// LDS tiles use XOR swizzles of whole 16-byte chunks instead of padding. A
// 16-byte LDS read serves 16 lanes per cycle from the 64 banks (16 bank groups
// of 16 bytes), and the 16 lanes read the same logical chunk of 16 consecutive
// rows, so the swizzle must put those on 16 distinct bank groups:
//   K   (row = key, CH = D * element size / 16 chunks): chunk c of row k sits at
//       c ^ k_swz<CH>(k), k_swz = (k / (16 / CH)) mod CH: rows that share bank
//       groups (k mod 16/CH equal) get CH distinct chunk positions;
//   V^T (row = feature, 8 chunks of 8 keys): chunk c of row d sits at
//       c ^ vt_swz(d), which puts the 16 rows one P V operand read touches on
//       16 distinct bank groups.
template <int CH>
__device__ __forceinline__ int k_swz(int k) { return (k / (16 / CH)) & (CH - 1); }
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) & 3) | ((d >> 2) & 4); }

// Position of key k16 (0..15) of a 16-key group in the repacked V^T rows: MFMA
// lane half h takes k-slots s = 0..7 = keys 4h + (s & 3) + 8 (s >> 2), so the
// group is stored as [keys 0-3, 8-11 | keys 4-7, 12-15] and each half reads
// its 8 keys as one 16-byte chunk.
__device__ __forceinline__ int vt_pos(int k16) { return 8 * ((k16 >> 2) & 1) + 4 * (k16 >> 3) + (k16 & 3); }

// fp8 V^T rows (64 bytes per 64-key tile). The P V instruction's k index
// p = 32h + 16kb + 4q + e of lane half h takes score element 4q + e of 32-key
// block kb of that lane, which is key 32kb + 8q + 4h + e (the S^T MFMA result
// layout), so position p of a tile row holds that key. The four 16-byte
// chunks of row d sit at c ^ vt8_swz(d): the 16 rows one operand read touches
// (features vrow(r), r < 16, or 16 <= r < 32) land on 16 distinct bank groups.
__device__ __forceinline__ int vt8_key(int p) {
  return 32 * ((p >> 4) & 1) + 8 * ((p >> 2) & 3) + 4 * (p >> 5) + (p & 3);
}
__device__ __forceinline__ int vt8_swz(int d) { return ((d >> 2) & 1) | ((d >> 3) & 2); }

// ---------------------------------------------------------------------------
// V -> V^T repack (once per call): per head, V^T[d][n_pad] with the key order
// of vt_pos inside every 16-key group and zeros for keys >= N.
// ---------------------------------------------------------------------------
template <int D, typename TIn>
__global__ __launch_bounds__(256) void anchor_pack_vt(const TIn* __restrict__ V,
                                                      uint16_t* __restrict__ VT, int N,
                                                      int n_pad) {
  constexpr int CH = D / 8;
  __shared__ uint32_t tile[64][D / 2 + 1];  // 64 keys x D features, odd word stride
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const TIn* Vh = V + (size_t)bh * N * D;
  uint16_t* VTh = VT + (size_t)bh * D * n_pad;
  for (int c = tid; c < 64 * CH; c += 256) {
    const int key = c / CH, col = (c % CH) * 8, n = j * 64 + key;
    const u32x4 v = n < N ? load8_bf16(Vh + (size_t)n * D + col) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) tile[key][col / 2 + p] = v[p];
  }
  __syncthreads();
  // output: D rows x 8 chunks of 8 keys; chunk pc holds positions 8pc..8pc+7
  for (int c = tid; c < D * 8; c += 256) {
    const int d = c >> 3, pc = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t e[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pos = 8 * pc + 2 * p + u;           // position within the tile
        const int g16 = pos >> 4, r = pos & 15;       // group, position in group
        // invert vt_pos: r = 8h + 4(k>>3) + (k&3) -> k = 4h + 8(r>>2 & 1) + (r&3)
        const int k16 = 4 * (r >> 3) + 8 * ((r >> 2) & 1) + (r & 3);
        const uint32_t word = tile[g16 * 16 + k16][d >> 1];
        e[u] = (d & 1) ? (word >> 16) : (word & 0xffffu);
      }
      w[p] = e[0] | (e[1] << 16);
    }
    stg16(VTh + (size_t)d * n_pad + j * 64 + pc * 8, (u32x4){w[0], w[1], w[2], w[3]});
  }
}

// fp8-P mode: V^T stays e4m3, per head [D][n_pad] bytes in vt8_key order
// inside every 64-key tile, zeros for keys >= N.
template <int D>
__global__ __launch_bounds__(256) void anchor_pack_vt8(const uint8_t* __restrict__ V,
                                                       uint8_t* __restrict__ VT, int N, int n_pad) {
  constexpr int CH = D / 16;                 // 16-byte chunks per key row
  __shared__ uint32_t tile[64][D / 4 + 1];   // 64 keys x D bytes, odd word stride
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const uint8_t* Vh = V + (size_t)bh * N * D;
  uint8_t* VTh = VT + (size_t)bh * D * n_pad;
  for (int c = tid; c < 64 * CH; c += 256) {
    const int key = c / CH, col = (c % CH) * 16, n = j * 64 + key;
    const u32x4 v = n < N ? ldg16(Vh + (size_t)n * D + col) : (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) tile[key][col / 4 + p] = v[p];
  }
  __syncthreads();
  // output: D rows x 4 chunks of 16 positions
  for (int c = tid; c < D * 4; c += 256) {
    const int d = c >> 2, pc = c & 3;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t word = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t src = tile[vt8_key(16 * pc + 4 * p + u)][d >> 2];
        word |= ((src >> (8 * (d & 3))) & 0xffu) << (8 * u);
      }
      w[p] = word;
    }
    stg16(VTh + (size_t)d * n_pad + j * 64 + pc * 16, (u32x4){w[0], w[1], w[2], w[3]});
  }
}

// P8: the fp8-P mode (TIn must be uint8_t).
template <int D, bool OUT_F32, typename TIn, bool P8>
__global__ __launch_bounds__(kThreads, 1) void anchor_bf16(const TIn* __restrict__ Q,
                                                      const TIn* __restrict__ K,
                                                      const TIn* __restrict__ G,
                                                      const void* __restrict__ VTv,
                                                      void* __restrict__ out, int N, int n_pad,
                                                      int nqb, int nmain, int split, float c,
                                                      int accumulate, float* __restrict__ part,
                                                      float* __restrict__ part_ml) {
  constexpr int ES = sizeof(TIn);         // bytes per input element: 2 bf16, 1 fp8
  constexpr bool F8 = ES == 1;
  constexpr int CPO = F8 ? 2 : 1;         // 16-byte K chunks per S^T operand
  constexpr int NK = D * ES / (32 * CPO);  // k-steps of S^T (16 bf16 or 64 fp8 features)
  constexpr int ND = D / 32;              // 32-row blocks of O^T
  constexpr int RB = D * ES;              // bytes per K row
  constexpr int CH = RB / 16;             // 16-byte chunks per K row
  constexpr int KBLK = kBC * RB / 1024;   // 1 KB direct-to-LDS blocks per K tile
  constexpr int LK = KBLK > kWaves ? KBLK / kWaves : 1;  // K blocks per loading wave
  constexpr int KW = KBLK / LK;           // waves that load K (4 for fp8, D = 64)
  static_assert(!P8 || F8, "fp8 P needs fp8 inputs");
  using VE = std::conditional_t<P8, uint8_t, uint16_t>;  // V^T element: e4m3 or bf16
  constexpr int VES = sizeof(VE);
  constexpr int VBLK = kBC * D * VES / 1024;              // 1 KB blocks per V^T tile
  constexpr int LV = VBLK > kWaves ? VBLK / kWaves : 1;    // V^T blocks per loading wave
  constexpr int VW = VBLK / LV;                            // waves that load V^T
  constexpr int VCH = kBC * VES / 16;     // 16-byte chunks per V^T row
  constexpr int VRPB = 1024 / (kBC * VES);  // V^T rows per block
  constexpr int RPB = 1024 / RB;          // K rows per block
  constexpr uint32_t kTileBytes = kBC * RB;
  using QOp = std::conditional_t<F8, u32x8, u32x4>;
  const VE* __restrict__ VT = reinterpret_cast<const VE*>(VTv);
  // Four separate LDS arrays rather than two [2][...] ones: the compiler then
  // knows that the direct-to-LDS loads filling one buffer do not alias the
  // reads of the other, and does not make every LDS read wait for them.
  __shared__ __attribute__((aligned(16))) TIn Ks0[kBC * D];
  __shared__ __attribute__((aligned(16))) TIn Ks1[kBC * D];
  __shared__ __attribute__((aligned(16))) TIn Ks2[kBC * D];
  __shared__ __attribute__((aligned(16))) TIn Ks3[kBC * D];
  __shared__ __attribute__((aligned(16))) VE Vs0[kBC * D];
  __shared__ __attribute__((aligned(16))) VE Vs1[kBC * D];
  __shared__ __attribute__((aligned(16))) VE Vs2[kBC * D];
  __shared__ __attribute__((aligned(16))) VE Vs3[kBC * D];
  // buffer b of each tensor: a compile-time b names one array, which lets the
  // compiler keep LDS reads of one buffer independent of the DMA into another;
  // a run-time b (rare edge iterations) selects among them
  auto kbuf = [&](auto b) -> TIn* {
    if constexpr (std::is_integral_v<decltype(b)>) {
      const int x = b & 3;
      return x == 0 ? Ks0 : x == 1 ? Ks1 : x == 2 ? Ks2 : Ks3;
    } else {
      constexpr int B = decltype(b)::value & 3;
      if constexpr (B == 0) return Ks0;
      else if constexpr (B == 1) return Ks1;
      else if constexpr (B == 2) return Ks2;
      else return Ks3;
    }
  };
  auto vbuf = [&](auto b) -> VE* {
    if constexpr (std::is_integral_v<decltype(b)>) {
      const int x = b & 3;
      return x == 0 ? Vs0 : x == 1 ? Vs1 : x == 2 ? Vs2 : Vs3;
    } else {
      constexpr int B = decltype(b)::value & 3;
      if constexpr (B == 0) return Vs0;
      else if constexpr (B == 1) return Vs1;
      else if constexpr (B == 2) return Vs2;
      else return Vs3;
    }
  };

  // The first nmain workgroups each own one query block over all keys. They are
  // dispatched round-robin over the 8 XCDs; renumber them so each XCD runs a
  // contiguous range of (b, h, query block) and the query blocks of one head
  // share that XCD's L2 while streaming its K and V. The workgroups after them
  // (dispatched last) split each remaining query block into `split` key ranges,
  // so the last batch of workgroups is short; they leave unnormalised partial
  // results in `part` for anchor_combine.
  const int bid = blockIdx.x;
  int logical, piece = -1;
  if (bid < nmain) {
    const int xcd = bid & 7, local = bid >> 3;
    const int per = nmain >> 3, rem = nmain & 7;
    logical = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  } else {
    piece = bid - nmain;
    logical = nmain + piece / split;
  }
  const int bh = logical / nqb, qb = logical - bh * nqb;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index, made visibly wave-uniform (it selects the M0 LDS base of the
  // direct-to-LDS loads, which must be a scalar)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * RB;
  const int qrow = qb * kBR + wave * 32 + r;

  // Q^T operand of k-step t: query qrow, bytes 32t + 16h (bf16) or 64t + 32h (fp8)
  QOp qf[NK];
  {
    const rsrc_t Qr = make_rsrc(Q + base, head_bytes);
    const uint32_t qoff = qrow < N ? (uint32_t)qrow * RB : head_bytes;  // past N reads 0
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      if constexpr (F8)
        qf[t] = concat(buf_load16(Qr, qoff + 64 * t + 32 * h), buf_load16(Qr, qoff + 64 * t + 32 * h + 16));
      else
        qf[t] = buf_load16(Qr, qoff + 32 * t + 16 * h);
    }
  }

  // Tiles go global -> LDS directly (buffer_load ... lds): instruction i of
  // wave w fills 1 KB LDS block bw = L*w + i in lane order. K tiles hold RPB key
  // rows of RB bytes per block (4 x 256 B for bf16 D=128, 8 x 128 B for bf16
  // D=64 and fp8 D=128, 16 x 64 B for fp8 D=64): lane l lands in row
  // RPB bw + l/CH, physical chunk l%CH. V^T tiles hold VRPB feature rows per
  // block (8 x 128 B of 64 bf16 keys, or 16 x 64 B of 64 fp8 keys): lane l lands
  // in row VRPB bw + l/VCH, physical chunk l%VCH. Each lane fetches the logical
  // chunk that the swizzle puts there.
  uint32_t goff_k[LK], goff_v[LV];
#pragma unroll
  for (int i = 0; i < LK; ++i) {
    const int row = (LK * wave + i) * RPB + lane / CH, pc = lane % CH;
    goff_k[i] = row * RB + (pc ^ k_swz<CH>(row)) * 16;
  }
#pragma unroll
  for (int i = 0; i < LV; ++i) {
    const int vd = (LV * wave + i) * VRPB + lane / VCH, vpc = lane % VCH;
    const int sw = P8 ? vt8_swz(vd) : vt_swz(vd);
    goff_v[i] = (uint32_t)vd * n_pad * VES + (uint32_t)(vpc ^ sw) * 16;
  }
  const uint32_t vt_head_bytes = (uint32_t)D * n_pad * VES;
  // issue K (or V^T) tile j into LDS buffer buf (completion: wait_all_memory + barrier).
  // No branch on the tile index: a tile past the end gets a zero-size descriptor,
  // so its loads touch no memory and fill LDS with zeros that nothing reads.
  auto load_k = [&](int j, auto buf_c) {
    if (KW < kWaves && wave >= KW) return;  // wave-uniform
    const uint32_t done = (uint32_t)j * kTileBytes;
    const uint32_t left = done < head_bytes ? head_bytes - done : 0u;
    const rsrc_t kr = make_rsrc_uniform(K + base + (size_t)j * kBC * D, left);
#pragma unroll
    for (int i = 0; i < LK; ++i)
      buf_load16_lds(kr, goff_k[i], kbuf(buf_c) + (LK * wave + i) * (1024 / ES));
  };
  auto load_v = [&](int j, auto buf_c) {
    if (VW < kWaves && wave >= VW) return;  // wave-uniform
    const uint32_t done = (uint32_t)j * kBC * VES;
    const uint32_t left = j * kBC < n_pad ? vt_head_bytes - done : 0u;
    const rsrc_t vr = make_rsrc_uniform(VT + (size_t)bh * D * n_pad + (size_t)j * kBC, left);
#pragma unroll
    for (int i = 0; i < LV; ++i)
      buf_load16_lds(vr, goff_v[i], vbuf(buf_c) + (LV * wave + i) * (1024 / VES));
  };

  // S^T operand A (key rows): lane reads row kb*32 + r, logical chunks
  // CPO (2t + h) + u, u < CPO (swizzled); offsets in elements
  int koff[NK][CPO];
#pragma unroll
  for (int t = 0; t < NK; ++t)
#pragma unroll
    for (int u = 0; u < CPO; ++u)
      koff[t][u] = r * D + ((CPO * (2 * t + h) + u) ^ k_swz<CH>(r)) * (16 / ES);
  // O^T operand A (V^T rows): MFMA row r of block b is feature
  // d = 32b + vrow, vrow = 16((r>>2)&1) + 4(r>>3) + (r&3), so each lane ends with
  // 16 consecutive output features; its 8 keys of k-step ks are logical chunk
  // 2ks + h of that row
  // (bf16 V^T); for e4m3 V^T its 32 keys of the tile are logical chunks 2h and 2h + 1
  const int vrow = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
  int voff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if constexpr (P8) voff[ks] = vrow * kBC + (((2 * h + (ks & 1)) ^ vt8_swz(vrow)) * 16);
    else voff[ks] = vrow * kBC + (((2 * ks + h) ^ vt_swz(vrow)) * 8);
  }

  f32x16 acc[ND];
#pragma unroll
  for (int b = 0; b < ND; ++b) acc[b] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  // fp8-P mode: the row sum is a fifth accumulator, ones^T P^T on the matrix
  // cores (every row of it holds the query's sum of the rounded P), rescaled
  // with the others; the bf16 mode sums on the VALU into l_run
  f32x16 acc_l = (f32x16){};
  const u32x4 ones8 = {0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};  // e4m3 1.0
  const int ntiles = (N + kBC - 1) / kBC;
  const bool ragged = (N % kBC) != 0;
  // key tiles [t0, t1) of this workgroup
  const int t0 = piece < 0 ? 0 : (piece % split) * ntiles / split;
  const int t1 = piece < 0 ? ntiles : (piece % split + 1) * ntiles / split;

  // ---- building blocks -----------------------------------------------------
  // S^T of the tile held in K buffer KB (two 32-key blocks)
  auto s_tile = [&](auto kb_c, f32x16* s) {
    const TIn* Kb = kbuf(kb_c);
    s[0] = (f32x16){};
    s[1] = (f32x16){};
#pragma unroll
    for (int t = 0; t < NK; ++t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Kb[kb * 32 * D + koff[t][0]]);
        if constexpr (F8) {
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(&Kb[kb * 32 * D + koff[t][1]]);
          s[kb] = mfma32x32x64_fp8(concat(a, a1), qf[t], s[kb]);
        } else {
          s[kb] = mfma32x32x16(a, qf[t], s[kb]);
        }
      }
    }
  };
  // O^T += V^T P^T for the tile held in V buffer VB; k-slot s of half h is
  // key 16ks + 8(s>>2) + 4h + (s&3)
  // (bf16 P; for e4m3 P, pb[0..1] is the 32-byte operand of the whole tile)
  auto pv_tile = [&](auto vb_c, const u32x4* pb) {
    const VE* Vb = vbuf(vb_c);
    if constexpr (P8) {
#pragma unroll
      for (int b = 0; b < ND; ++b) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(&Vb[b * 32 * kBC + voff[0]]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(&Vb[b * 32 * kBC + voff[1]]);
        acc[b] = mfma32x32x64_fp8(concat(a0, a1), concat(pb[0], pb[1]), acc[b]);
      }
      acc_l = mfma32x32x64_fp8(concat(ones8, ones8), concat(pb[0], pb[1]), acc_l);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int b = 0; b < ND; ++b) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&Vb[b * 32 * kBC + voff[ks]]);
          acc[b] = mfma32x32x16(a, pb[ks], acc[b]);
        }
      }
    }
  };
  // online softmax of S^T for tile j: returns the P^T operands in pb (bf16:
  // four 16-byte k-steps; e4m3: pb[kb] holds score elements 0..15 of 32-key
  // block kb as bytes) and the factor alpha by which the accumulator must be
  // rescaled (1 if none)
  auto softmax = [&](f32x16* s, u32x4* pb, int j, bool mask) -> float {
    if (mask) {
      asm volatile("");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int key = j * kBC + kb * 32 + (x >> 2) * 8 + 4 * h + (x & 3);
          if (key >= N) s[kb][x] = -INFINITY;
        }
    }
    // row max: two chains of 3-input maxima, then the partner half-wave.
    // maximum (NaN-propagating) needs no canonicalizing of the MFMA results,
    // which fmaxf would add for every score.
    float m2[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      m2[kb] = s[kb][0];
#pragma unroll
      for (int x = 1; x < 16; ++x) m2[kb] = __builtin_elementwise_maximum(m2[kb], s[kb][x]);
    }
    float m16[1] = {__builtin_elementwise_maximum(m2[0], m2[1])};
    const float mt = max_halves(m16[0]) * c;
    const bool need = mt > m_run + kTau;
    const float m_new = need ? mt : m_run;
    const float alpha = exp2_fast(m_run - m_new);  // 1 unless the max moved up
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) p[x] = exp2_fast(fmaf(s[kb][x], c, -m_run));
      if constexpr (P8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) pb[kb][w] = pack_fp8x4(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3]);
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int qq = half * 8;
          pb[kb * 2 + half] = (u32x4){pack_bf16(p[qq + 0], p[qq + 1]), pack_bf16(p[qq + 2], p[qq + 3]),
                                      pack_bf16(p[qq + 4], p[qq + 5]), pack_bf16(p[qq + 6], p[qq + 7])};
        }
      }
    }
    // the row sum adds the same rounded values the MFMA consumes (4 chains)
    if constexpr (!P8) {
      float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) l4[ks] = add_bf16x2(pb[ks][x], l4[ks]);
      l_run += (l4[0] + l4[1]) + (l4[2] + l4[3]);
    }
    return alpha;
  };
  auto rescale = [&](float alpha) {
    // a real branch: the empty volatile asm keeps the compiler from turning
    // this rarely taken rescale into straight-line code run on every tile
    if (__any(alpha != 1.0f)) {
      asm volatile("");
#pragma unroll
      for (int b = 0; b < ND; ++b) acc[b] *= alpha;
      if constexpr (P8) acc_l *= alpha;
    }
  };

  // ---- software pipeline ------------------------------------------------------
  // Iteration j overlaps the softmax of tile j (VALU) with the MFMAs of P V for
  // tile j-1 and of S^T for tile j+1, which do not depend on it: K runs one
  // tile ahead of the softmax and V one tile behind. The accumulator rescale
  // for tile j waits until P V of tile j-1 has been added.
  f32x16 s_cur[2];
  u32x4 p_prev[4];
  // Four K and four V buffers; local tile t lives in buffer t % 4. Iterations go
  // in pairs: the first of a pair issues K(j+3), K(j+4), V(j+1), V(j+2), the
  // second ends with the barrier, so each pair reads only tiles issued by the
  // previous one and overwrites only buffers that pair has finished reading.
  // jm_c: jl % 4, as a compile-time constant in the unrolled steady loop or
  // as an int in the few edge iterations
  auto iteration = [&](auto jm_c, auto steady_c, int jl) __attribute__((always_inline)) {
    constexpr bool STEADY = decltype(steady_c)::value;
    constexpr bool RT = std::is_integral_v<decltype(jm_c)>;
    auto shifted = [&](auto d_c) {
      constexpr int Dd = decltype(d_c)::value;
      if constexpr (RT) return int((jm_c + Dd) & 3);
      else return std::integral_constant<int, (decltype(jm_c)::value + Dd) & 3>{};
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    bool first;
    if constexpr (RT) first = (jm_c & 1) == 0;
    else first = (decltype(jm_c)::value & 1) == 0;
    const int j = t0 + jl;
    asm volatile("" : "+v"(s_cur[0]), "+v"(s_cur[1]));
    if (first) {
      load_k(j + 3, shifted(S3{}));
      load_k(j + 4, shifted(S0{}));
      load_v(j + 1, shifted(S1{}));
      load_v(j + 2, shifted(S2{}));
    }
    u32x4 p_cur[4];
    const bool mask = !STEADY && ragged && j == ntiles - 1;
    const float alpha = softmax(s_cur, p_cur, j, mask);
    if (STEADY || jl > 0) pv_tile(shifted(S3{}), p_prev);
    f32x16 s_next[2];
    if (STEADY || j + 1 < t1) s_tile(shifted(S1{}), s_next);
    if constexpr (P8) asm volatile("" ::"v"(p_cur[0]), "v"(p_cur[1]), "v"(l_run));
    else asm volatile("" ::"v"(p_cur[0]), "v"(p_cur[1]), "v"(p_cur[2]), "v"(p_cur[3]), "v"(l_run));
    rescale(alpha);
#pragma unroll
    for (int ks = 0; ks < (P8 ? 2 : 4); ++ks) p_prev[ks] = p_cur[ks];
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
    if (!first) {
      wait_all_memory();  // the pair's tiles have landed in LDS
      __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using Steady = std::true_type;
  using Edge = std::false_type;
  // prologue: K(t0), K(t0+1), K(t0+2), V(t0) in; S^T of tile t0
  const int nt = t1 - t0;
  load_k(t0, std::integral_constant<int, 0>{});
  load_k(t0 + 1, std::integral_constant<int, 1>{});
  load_k(t0 + 2, std::integral_constant<int, 2>{});
  load_v(t0, std::integral_constant<int, 0>{});
  wait_all_memory();
  __syncthreads();
  s_tile(std::integral_constant<int, 0>{}, s_cur);
  __syncthreads();  // K buffer 0 is free for K(t0+4)

  auto run = [&](int jl, auto steady_c) __attribute__((always_inline)) {
    iteration(int(jl & 3), steady_c, jl);
  };
  iteration(std::integral_constant<int, 0>{}, Edge{}, 0);
  int jl = 1;
  for (; jl + 4 <= nt - 1; jl += 4) {  // local tiles 1 .. nt-2 are steady
    iteration(std::integral_constant<int, 1>{}, Steady{}, jl);
    iteration(std::integral_constant<int, 2>{}, Steady{}, jl + 1);
    iteration(std::integral_constant<int, 3>{}, Steady{}, jl + 2);
    iteration(std::integral_constant<int, 0>{}, Steady{}, jl + 3);
  }
  for (; jl <= nt - 2; ++jl) run(jl, Steady{});
  if (jl == nt - 1 && jl > 0) run(jl, Edge{});
  // an odd-length range ends on the first iteration of a pair: no barrier was
  // needed after it, and none is needed now (only registers remain)
  // P V of the last tile
  pv_tile(int((nt - 1) & 3), p_prev);

  if (piece >= 0) {
    // partial result of a key range: unnormalised O, running max and row sum
    const float l_tot = P8 ? acc_l[0] : add_halves(l_run);
    const int row = wave * 32 + r;
    float* po = part + ((size_t)piece * kBR + row) * D;
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
      for (int x = 0; x < 4; ++x)
        *reinterpret_cast<f32x4*>(po + 32 * b + 16 * h + 4 * x) =
            (f32x4){acc[b][4 * x], acc[b][4 * x + 1], acc[b][4 * x + 2], acc[b][4 * x + 3]};
    if (h == 0) {
      float* pml = part_ml + ((size_t)piece * kBR + row) * 2;
      pml[0] = m_run;
      pml[1] = l_tot;
    }
    return;
  }

  // epilogue: lane (query r, half h) holds features 32b + 16h + 0..15 of block b
  const float l_tot = P8 ? acc_l[0] : add_halves(l_run);
  const float inv = 1.0f / l_tot;
  if (qrow >= N) return;
#pragma unroll
  for (int b = 0; b < ND; ++b) {
    const size_t off = base + (size_t)qrow * D + 32 * b + 16 * h;
    float o[16];
    load16_f32(G + off, o);
#pragma unroll
    for (int x = 0; x < 16; ++x) o[x] = (acc[b][x] * inv) * sigmoid(o[x]);
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

// ---------------------------------------------------------------------------
// Merge the key-range pieces of the split query blocks: with per-piece running
// max m_p (log2 units), row sum l_p and unnormalised O_p, the full row is
// O = sum_p 2^(m_p - m) O_p / sum_p 2^(m_p - m) l_p, m = max_p m_p; then the
// gate and the store, as in the main epilogue. Each thread takes 8 features of
// one query row; 16 rows per workgroup, kBR / 16 workgroups per split block.
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32, typename TIn>
__global__ __launch_bounds__(256) void anchor_combine(const float* __restrict__ part,
                                                      const float* __restrict__ part_ml,
                                                      const TIn* __restrict__ G,
                                                      void* __restrict__ out, int N, int nqb,
                                                      int nmain, int split, int accumulate) {
  constexpr int TPR = D / 8;                 // threads per row
  constexpr int RPB = 256 / TPR;             // rows per workgroup
  constexpr int WPB = kBR / RPB;             // workgroups per split block
  const int tb = blockIdx.x / WPB;
  const int row = (blockIdx.x % WPB) * RPB + threadIdx.x / TPR;
  const int f = (threadIdx.x % TPR) * 8;
  const int logical = nmain + tb;
  const int bh = logical / nqb, qb = logical - bh * nqb;
  const int qrow = qb * kBR + row;
  if (qrow >= N) return;
  const float* ml = part_ml + ((size_t)tb * split * kBR + row) * 2;  // piece p at + p kBR 2
  const float* po = part + ((size_t)tb * split * kBR + row) * D + f;  // piece p at + p kBR D
  float m = -INFINITY;
  for (int p = 0; p < split; ++p) m = fmaxf(m, ml[(size_t)p * kBR * 2]);
  float wsum = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < split; ++p) {
    const float wp = exp2_fast(ml[(size_t)p * kBR * 2] - m);
    wsum = fmaf(wp, ml[(size_t)p * kBR * 2 + 1], wsum);
    const f32x4 a = *reinterpret_cast<const f32x4*>(po + (size_t)p * kBR * D);
    const f32x4 b = *reinterpret_cast<const f32x4*>(po + (size_t)p * kBR * D + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = fmaf(wp, a[e], o[e]);
      o[4 + e] = fmaf(wp, b[e], o[4 + e]);
    }
  }
  const float inv = 1.0f / wsum;
  const size_t base = ((size_t)bh * N + qrow) * D + f;
  float gf[8];
  load8_f32(G + base, gf);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (o[e] * inv) * sigmoid(gf[e]);
  if (OUT_F32) {
    float* dst = reinterpret_cast<float*>(out) + base;
    f32x4 lo = (f32x4){o[0], o[1], o[2], o[3]}, hi = (f32x4){o[4], o[5], o[6], o[7]};
    if (accumulate) {
      lo += *reinterpret_cast<const f32x4*>(dst);
      hi += *reinterpret_cast<const f32x4*>(dst + 4);
    }
    *reinterpret_cast<f32x4*>(dst) = lo;
    *reinterpret_cast<f32x4*>(dst + 4) = hi;
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + base;
    if (accumulate) {
      const u32x4 prev = ldg16(dst);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] += bf_lo(prev[e]);
        o[2 * e + 1] += bf_hi(prev[e]);
      }
    }
    stg16(dst, (u32x4){pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]),
                       pack_bf16(o[6], o[7])});
  }
}

// Compute units of the current device (one anchor workgroup fits per CU).
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

struct AnchorLayout {
  size_t vt_bytes, part_off, ml_off, total;
  int pieces_cap;
};
// fp8_p: the fp8-P mode, whose V^T copy takes one byte per element (else two)
AnchorLayout anchor_layout(const hla_dims& d, bool fp8_p) {
  AnchorLayout L;
  const int64_t BH = d.B * d.H, N = d.N, D = d.D;
  const int64_t n_pad = (N + kBC - 1) / kBC * kBC;
  const int64_t nqb = (N + kBR - 1) / kBR, ntiles = n_pad / kBC;
  const int64_t cap = BH * nqb * ntiles;
  L.pieces_cap = int(cap < kMaxPieces ? cap : kMaxPieces);
  const int64_t ves = fp8_p ? 1 : 2;  // V^T bytes per element
  L.vt_bytes = align_up(size_t(BH * D * n_pad * ves), 256);
  L.part_off = L.vt_bytes;
  L.ml_off = L.part_off + align_up(size_t(L.pieces_cap) * kBR * D * 4, 256);
  L.total = L.ml_off + align_up(size_t(L.pieces_cap) * kBR * 2 * 4, 256);
  return L;
}

template <int D, typename TIn, bool P8>
hipError_t launch_d(const hla_dims& d, const void* q, const void* k, const void* v, const void* g,
                    void* out, int accumulate, float scale, void* ws, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  const int n_pad = (N + kBC - 1) / kBC * kBC;
  const int ntiles = n_pad / kBC;
  const int nqb = (N + kBR - 1) / kBR;
  const int total = BH * nqb;
  const float c = scale * kLog2e;
  const AnchorLayout L = anchor_layout(d, P8);
  char* w = reinterpret_cast<char*>(ws);
  void* vt = w;
  float* part = reinterpret_cast<float*>(w + L.part_off);
  float* part_ml = reinterpret_cast<float*>(w + L.ml_off);
  // Workgroups run in batches of one per CU. The query blocks of an
  // incomplete last batch are split along the keys so that batch takes a
  // fraction of a full one.
  const int slots = device_cus();
  // Split each of the `tail` blocks into k pieces. The last batch then lasts
  // ceil(tail k / slots) / k rounds; take the smallest k within 0.02 rounds of
  // the shortest (more pieces cost partial results and combine work), within
  // the piece cap and at least one key tile per piece.
  int tail = total % slots, split = 1;
  if (tail > 0) {
    const int kmax_t = ntiles, kmax_p = L.pieces_cap / tail;
    const int kmax = kmax_t < kmax_p ? kmax_t : kmax_p;
    int best_num = 1, best_den = 1;  // shortest length in rounds, as a fraction
    for (int k = 2; k <= kmax; ++k) {
      const int num = (tail * k + slots - 1) / slots;
      if (num * best_den < best_num * k) {
        best_num = num;
        best_den = k;
      }
    }
    for (int k = 2; k <= kmax; ++k) {
      const int num = (tail * k + slots - 1) / slots;
      if (50 * num * best_den <= (50 * best_num + best_den) * k) {  // num/k <= best + 1/50
        split = k;
        break;
      }
    }
  }
  if (split < 2) {
    tail = 0;
    split = 1;
  }
  const int nmain = total - tail;
  const int grid = nmain + tail * split;
  if constexpr (P8)
    hipLaunchKernelGGL((anchor_pack_vt8<D>), dim3(n_pad / kBC, BH), dim3(256), 0, stream,
                       reinterpret_cast<const uint8_t*>(v), reinterpret_cast<uint8_t*>(vt), N, n_pad);
  else
    hipLaunchKernelGGL((anchor_pack_vt<D, TIn>), dim3(n_pad / kBC, BH), dim3(256), 0, stream,
                       reinterpret_cast<const TIn*>(v), reinterpret_cast<uint16_t*>(vt), N, n_pad);
  const TIn* Qp = reinterpret_cast<const TIn*>(q);
  const TIn* Kp = reinterpret_cast<const TIn*>(k);
  const TIn* Gp = reinterpret_cast<const TIn*>(g);
  if (d.out_dtype == HLA_F32) {
    hipLaunchKernelGGL((anchor_bf16<D, true, TIn, P8>), dim3(grid), dim3(kThreads), 0, stream, Qp, Kp,
                       Gp, vt, out, N, n_pad, nqb, nmain, split, c, accumulate, part, part_ml);
    if (tail > 0)
      hipLaunchKernelGGL((anchor_combine<D, true, TIn>), dim3(tail * (D / 8)), dim3(256), 0, stream,
                         part, part_ml, Gp, out, N, nqb, nmain, split, accumulate);
  } else {
    hipLaunchKernelGGL((anchor_bf16<D, false, TIn, P8>), dim3(grid), dim3(kThreads), 0, stream, Qp, Kp,
                       Gp, vt, out, N, n_pad, nqb, nmain, split, c, accumulate, part, part_ml);
    if (tail > 0)
      hipLaunchKernelGGL((anchor_combine<D, false, TIn>), dim3(tail * (D / 8)), dim3(256), 0,
                         stream, part, part_ml, Gp, out, N, nqb, nmain, split, accumulate);
  }
  return hipGetLastError();
}

}  // namespace

size_t anchor_workspace_bytes(const hla_dims& d) {
  if (d.in_dtype == HLA_F32) return 0;
  return anchor_layout(d, false).total;
}

hipError_t launch_anchor_bf16(const hla_dims& d, const void* q, const void* k, const void* v,
                              const void* g, void* out, int accumulate, float scale, void* ws,
                              hipStream_t stream, bool fp8_p) {
  if (d.in_dtype == HLA_FP8_E4M3) {
    if (fp8_p) {
      if (d.D == 128)
        return launch_d<128, uint8_t, true>(d, q, k, v, g, out, accumulate, scale, ws, stream);
      return launch_d<64, uint8_t, true>(d, q, k, v, g, out, accumulate, scale, ws, stream);
    }
    if (d.D == 128)
      return launch_d<128, uint8_t, false>(d, q, k, v, g, out, accumulate, scale, ws, stream);
    return launch_d<64, uint8_t, false>(d, q, k, v, g, out, accumulate, scale, ws, stream);
  }
  if (d.D == 128)
    return launch_d<128, uint16_t, false>(d, q, k, v, g, out, accumulate, scale, ws, stream);
  return launch_d<64, uint16_t, false>(d, q, k, v, g, out, accumulate, scale, ws, stream);
}

}  // namespace hla
