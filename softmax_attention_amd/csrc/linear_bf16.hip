// Gated linear attention, bf16 or fp8 (OCP e4m3) inputs, on gfx950 matrix cores.
//
// Three launches per call:
//   1. state pass   per (token chunk, b, h): S_c = phi(K_c)^T V_c and
//                   z_c = sum phi(K_c), with the contraction over tokens on
//                   32x32x16 bf16 MFMA (fp32 accumulate); partials to workspace
//                   (S_c rounded to bf16, z_c in fp32).
//   2. reduce       per (b, h): S = sum_c S_c and z = sum_c z_c in fp32 in a fixed
//                   chunk order (deterministic, no float atomics), written straight into
//                   the operand fragments the output pass feeds to the MFMA:
//                   S^T rounded to bf16, z split into a bf16 hi + lo pair.
//   3. output pass  per (b, h, token group): O = sigma(G) (.) (phi(Q) S) /
//                   (phi(Q) . z + eps) with 16x16x32 bf16 MFMA, streaming Q and G
//                   from HBM and writing O once, each as whole 1 KB runs that a
//                   per-wave LDS tile turns into (and back from) operand layout.
// The operator is the O(N) fixed-size-state token mixer of SANA-Video 2.0
// (ai-papers.net summary, section on hybrid linear attention; SANA-Video 2.0
// abstract on thelatestinai.com).
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {
namespace {

// fp8 inputs are converted exactly to bf16 where a kernel consumes them, not
// where it loads them, so the loads of the next tile stay in flight meanwhile.
// Every global load is 16 bytes: 8 bf16 or 16 fp8 elements.
__device__ __forceinline__ u32x4 fp8_half(u32x4 raw, int hi) {
  return fp8x8_to_bf16(hi ? (u32x2){raw[2], raw[3]} : (u32x2){raw[0], raw[1]});
}

// buf_load16 with the non-temporal cache policy (cache-policy bit 1: nt), for
// data read exactly once.
__device__ __forceinline__ u32x4 buf_load16_stream(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2));
}

// ---------------------------------------------------------------------------
// Operand fragments of the output pass (16x16x32 MFMA: A rows i = lane & 15,
// k = 8*(lane>>4) + e). Numerator fragment (jb, t) holds A[i][k] =
// S[row(t, k)][col(jb, i)], ordered so that an output lane's Q slice (its B
// operand) and its output features are whole 16-byte runs of its token's row:
//   bf16 (8 features per run):  row = 32t + k,
//                               col = 32(jb>>1) + 8(i>>2) + 4(jb&1) + (i&3);
//   fp8 (16 features per run):  row = 64(t>>1) + 16(k>>3) + 8(t&1) + (k&7),
//                               col = 64(jb>>2) + 16(i>>2) + 4(jb&3) + (i&3).
// frag_pos gives the fp32 slot of S[row][col] among the D*D partial-state
// slots: ((jb * D/32 + t) * 64 + lane) * 8 + e, lane = 16(k>>3) + i, e = k&7.
// ---------------------------------------------------------------------------
template <int D, bool F8>
__device__ __forceinline__ int frag_pos(int row, int col) {
  constexpr int NT = D / 32;
  int t, kg, jb, i;
  if constexpr (F8) {
    t = 2 * (row >> 6) + ((row >> 3) & 1);
    kg = (row >> 4) & 3;
    jb = 4 * (col >> 6) + ((col >> 2) & 3);
    i = 4 * ((col >> 4) & 3) + (col & 3);
  } else {
    t = row >> 5;
    kg = (row >> 3) & 3;
    jb = 2 * (col >> 5) + ((col >> 2) & 1);
    i = 4 * ((col >> 3) & 3) + (col & 3);
  }
  return ((jb * NT + t) * 64 + 16 * kg + i) * 8 + (row & 7);
}
// first z entry of the 8 that k-step t, k-group kg of a denominator fragment holds
template <int D, bool F8>
__device__ __forceinline__ int z_run(int t, int kg) {
  return F8 ? 64 * (t >> 1) + 16 * kg + 8 * (t & 1) : 32 * t + 8 * kg;
}

// One chunk's partial state in the workspace: D*D bf16 of S in frag_pos order,
// then D fp32 of z. S is rounded to bf16 once more before the fp32 sum of the
// chunks (the sum is rounded to bf16 for the output pass anyway), which halves
// the partials' traffic; z, which sets every output's normaliser, stays fp32.
template <int D>
struct Partial {
  static constexpr size_t kSBytes = size_t(D) * D * 2;
  static constexpr size_t kBytes = kSBytes + size_t(D) * 4;
};

// ---------------------------------------------------------------------------
// 1. state pass
// ---------------------------------------------------------------------------
// Both MFMA operands have tokens along k: A = phi(K)^T (rows = features) and
// B = V (cols = features), each lane holding 8 consecutive tokens of one
// feature. So the tiles are stored feature-major in LDS: each thread loads an
// 8-token x 8-feature block (8 coalesced 16-byte loads, one per token row),
// transposes it in registers with byte permutes and writes 8 feature rows of 8
// tokens, and every operand is then one 16-byte LDS read. Threads 0-127 take K
// blocks (ReLU, the write gate and the normaliser z on the way), 128-255 V
// blocks; a tile of TILE tokens holds exactly 128 blocks per tensor.
// Wave w owns a (D/2 x D/2) quadrant of S: 32-row blocks [(w>>1)*RB, +RB) and
// 32-column blocks [(w&1)*RB, +RB).
// With WG (the write-gated variant) each token's phi(K) row is first scaled by
// its write strength sigma(W_n), W one logit per token and head ([B,H,N]); the
// scaled row, rounded to bf16, feeds both the MFMA and the normaliser sum.
// TIn: uint16_t for bf16 inputs, uint8_t for fp8 (16 features per load, so two
// 8 x 8 blocks per load row).

// Physical 16-byte chunk of logical chunk c in feature row `row` of a tile with
// CH chunks per row: c ^ t_swz<CH>(row). The 16 lanes of one operand read take
// 16 consecutive rows (one bank group each); the 16 lanes of one block write take
// rows 8 or 16 apart, spread at most two to a bank group.
template <int CH>
__device__ __forceinline__ int t_swz(int row) {
  if constexpr (CH >= 16) return (row ^ (row >> 3)) & 15;
  else return ((row >> 1) ^ (row >> 3)) & 7;
}

// 8 x 8 transpose of bf16: in[i] holds 8 features of token i, out[h] the 8
// tokens of feature h (v_perm_b32 takes bytes 0-3 from its second operand and
// 4-7 from its first).
__device__ __forceinline__ void transpose8x8(const u32x4* in, u32x4* out) {
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t sel = (h & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      out[h][d] = __builtin_amdgcn_perm(in[2 * d + 1][h >> 1], in[2 * d][h >> 1], sel);
  }
}

// A wave's quadrant of a chunk's partial S, stored in the output pass's
// fragment order (bf16, see frag_pos) so the reduce reads and writes whole
// fragments contiguously. C-tile element (q*4 + e) of lane (col r, half h2) is
// row q*8 + 4h2 + e: 4 consecutive slots.
template <int D, bool F8, int RB>
__device__ __forceinline__ void store_partial_s(const f32x16 (&acc)[RB][RB], char* Pc, int ib0,
                                                int jb0, int lane) {
  uint16_t* PS = reinterpret_cast<uint16_t*>(Pc);
  const int r = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int y = 0; y < RB; ++y)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = (ib0 + x) * 32 + 8 * q + 4 * h2, col = (jb0 + y) * 32 + r;
        *reinterpret_cast<u32x2*>(&PS[frag_pos<D, F8>(row, col)]) =
            (u32x2){pack_bf16(acc[x][y][q * 4], acc[x][y][q * 4 + 1]),
                    pack_bf16(acc[x][y][q * 4 + 2], acc[x][y][q * 4 + 3])};
      }
}

template <int D, bool WG, typename TIn>
__global__ __launch_bounds__(256) void linear_state_bf16(const TIn* __restrict__ K,
                                                         const TIn* __restrict__ V,
                                                         const TIn* __restrict__ W,
                                                         char* __restrict__ part, int N, int T,
                                                         int C) {
  constexpr bool F8 = sizeof(TIn) == 1;
  constexpr int EPL = 16 / sizeof(TIn);    // features per 16-byte load
  constexpr int HALVES = EPL / 8;          // 8 x 8 blocks per load row
  constexpr int FC = D / EPL;              // feature chunks per token row
  constexpr int TILE = 1024 * EPL / D;     // tokens per tile: 128 blocks per tensor
  constexpr int TG = TILE / 8;             // 8-token groups per tile
  constexpr int CH = TILE / 8;             // 16-byte chunks per feature row
  constexpr int RB = D / 64;               // 32-wide blocks per wave per side
  static_assert(TG * FC == 128, "one block per thread and tensor");
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int n0 = c * T;
  const int n1 = min(N, n0 + T);
  const size_t base = (size_t)bh * N * D;
  const bool isk = tid < 128;  // waves 0-1: K blocks, waves 2-3: V blocks
  const int jb = tid & 127, fc = jb % FC, tg = jb / FC;
  const TIn* src = (isk ? K : V) + base + fc * EPL;
  uint16_t* tile = isk ? Kt : Vt;
  const TIn* Wh = WG ? W + (size_t)bh * N : nullptr;

  u32x4 raw[8];  // rows 8tg .. 8tg+7 of the tile, raw bytes as loaded
  TIn wr[8];
  float zacc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) zacc[e] = 0.f;
  f32x16 acc[RB][RB];
#pragma unroll
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int y = 0; y < RB; ++y) acc[x][y] = (f32x16){};

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = t0 + 8 * tg + i;
      if (n < n1) {
        raw[i] = ldg16_stream(src + (size_t)n * D);
        if (WG) wr[i] = isk ? Wh[n] : TIn(0);
      } else {
        raw[i] = (u32x4){0, 0, 0, 0};
        if (WG) wr[i] = 0;
      }
    }
  };

  const int r = lane & 31, h2 = lane >> 5;
  const int ib0 = (wave >> 1) * RB, jb0 = (wave & 1) * RB;
  const int ntiles = (n1 - n0 + TILE - 1) / TILE;

  load_tile(n0);
  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();  // every wave is done reading the previous tile
    float beta[8];
    if (WG && isk) {
#pragma unroll
      for (int i = 0; i < 8; ++i) beta[i] = sigmoid(elem_f32(wr[i]));
    }
#pragma unroll
    for (int hh = 0; hh < HALVES; ++hh) {
      u32x4 rows[8], cols[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rows[i] = F8 ? fp8_half(raw[i], hh) : raw[i];
      if (isk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          rows[i] = relu_bf16x8(rows[i]);
          if (WG) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
              rows[i][p] = pack_bf16(bf_lo(rows[i][p]) * beta[i], bf_hi(rows[i][p]) * beta[i]);
          }
        }
      }
      transpose8x8(rows, cols);
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const int row = fc * EPL + 8 * hh + h;
        *reinterpret_cast<u32x4*>(&tile[row * TILE + ((tg ^ t_swz<CH>(row)) * 8)]) = cols[h];
        if (isk) {
          // the normaliser sums the same rounded values the MFMA consumes
#pragma unroll
          for (int d = 0; d < 4; ++d) zacc[8 * hh + h] = add_bf16x2(cols[h][d], zacc[8 * hh + h]);
        }
      }
    }
    __syncthreads();
    if (it + 1 < ntiles) load_tile(n0 + (it + 1) * TILE);  // in flight during the MFMAs
#pragma unroll
    for (int s = 0; s < TILE / 16; ++s) {
      const int lc = 2 * s + h2;  // logical chunk: tokens 16s + 8h2 .. +7
      u32x4 a[RB], b[RB];
#pragma unroll
      for (int x = 0; x < RB; ++x) {
        const int fi = (ib0 + x) * 32 + r;
        const int fj = (jb0 + x) * 32 + r;
        a[x] = *reinterpret_cast<const u32x4*>(&Kt[fi * TILE + ((lc ^ t_swz<CH>(fi)) * 8)]);
        b[x] = *reinterpret_cast<const u32x4*>(&Vt[fj * TILE + ((lc ^ t_swz<CH>(fj)) * 8)]);
      }
#pragma unroll
      for (int x = 0; x < RB; ++x)
#pragma unroll
        for (int y = 0; y < RB; ++y) acc[x][y] = mfma32x32x16(a[x], b[y], acc[x][y]);
    }
  }

  char* Pc = part + ((size_t)bh * C + c) * Partial<D>::kBytes;
  float* Pz = reinterpret_cast<float*>(Pc + Partial<D>::kSBytes);
  store_partial_s<D, F8, RB>(acc, Pc, ib0, jb0, lane);

  // partial z: the K thread of block (fc, tg) holds features fc*EPL .. +EPL over
  // its token groups; sum the TG groups of each feature in a fixed order
  __syncthreads();
  float* zred = reinterpret_cast<float*>(Kt);  // TG * D floats fit in the K tile
  if (isk) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) zred[tg * D + fc * EPL + e] = zacc[e];
  }
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
    for (int g = 0; g < TG; ++g) sum += zred[g * D + tid];
    Pz[tid] = sum;
  }
}

// fp8 inputs without a write gate: the tiles stay e4m3 and the contraction runs
// on the 32x32x64 fp8 matrix instruction (products exact in fp32, fp32 sums),
// so a tile costs the LDS bytes and matrix-core cycles of a bf16 tile of half
// as many tokens. Same block scheme as linear_state_bf16: each thread loads an
// 8-token x 16-feature block, clears negative K bytes (phi), and transposes it
// with byte permutes into 16 feature rows of 8 tokens; an A or B operand (32
// consecutive tokens of one feature) is then two 16-byte LDS reads. z = phi(K)^T 1
// comes from the same instruction with a B operand of ones (e4m3 1.0 = 0x38),
// on the two waves whose quadrant starts at column 0.
template <int D>
__global__ __launch_bounds__(256) void linear_state_fp8(const uint8_t* __restrict__ K,
                                                        const uint8_t* __restrict__ V,
                                                        char* __restrict__ part, int N, int T,
                                                        int C) {
  constexpr int FC = D / 16;    // 16-feature chunks per token row
  constexpr int TG = 128 / FC;  // 8-token groups per tile: one block per thread and tensor
  constexpr int TILE = 8 * TG;  // tokens per tile (one byte each per feature row)
  constexpr int CH = TILE / 16; // 16-byte chunks per feature row
  constexpr int RB = D / 64;    // 32-wide blocks per wave per side
  __shared__ __attribute__((aligned(16))) uint8_t Kt[D * TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[D * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int n0 = c * T;
  const int n1 = min(N, n0 + T);
  const size_t base = (size_t)bh * N * D;
  const bool isk = tid < 128;  // waves 0-1: K blocks, waves 2-3: V blocks
  const int jb = tid & 127, fc = jb % FC, tg = jb / FC;
  const uint8_t* src = (isk ? K : V) + base + fc * 16;
  uint8_t* tile = isk ? Kt : Vt;

  u32x4 raw[8];  // tokens 8tg .. 8tg+7 of the tile, features 16fc .. +15
  f32x16 acc[RB][RB], zacc[RB];
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    zacc[x] = (f32x16){};
#pragma unroll
    for (int y = 0; y < RB; ++y) acc[x][y] = (f32x16){};
  }
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = t0 + 8 * tg + i;
      raw[i] = n < n1 ? ldg16_stream(src + (size_t)n * D) : (u32x4){0, 0, 0, 0};
    }
  };
  auto lds_chunk = [&](const uint8_t* t, int row, int lc) {
    return *reinterpret_cast<const u32x4*>(&t[row * TILE + ((lc ^ t_swz<CH>(row)) * 16)]);
  };

  const int r = lane & 31, h2 = lane >> 5;
  const int ib0 = (wave >> 1) * RB, jb0 = (wave & 1) * RB;
  const bool zwave = (wave & 1) == 0;
  const u32x8 ones = {0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u,
                      0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};
  const int ntiles = (n1 - n0 + TILE - 1) / TILE;

  load_tile(n0);
  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();  // every wave is done reading the previous tile
    if (isk) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) raw[i][d] = relu_fp8x4(raw[i][d]);
    }
    // 4 x 4 byte transposes: dword d of tokens 4th .. 4th+3 -> features
    // 4d .. 4d+3, four tokens each (v_perm_b32 takes bytes 0-3 from its second
    // operand and 4-7 from its first)
    uint32_t cols[16][2];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int i0 = 4 * th;
        const uint32_t a = __builtin_amdgcn_perm(raw[i0 + 1][d], raw[i0][d], 0x05010400u);
        const uint32_t b = __builtin_amdgcn_perm(raw[i0 + 1][d], raw[i0][d], 0x07030602u);
        const uint32_t e = __builtin_amdgcn_perm(raw[i0 + 3][d], raw[i0 + 2][d], 0x05010400u);
        const uint32_t f = __builtin_amdgcn_perm(raw[i0 + 3][d], raw[i0 + 2][d], 0x07030602u);
        cols[4 * d + 0][th] = __builtin_amdgcn_perm(e, a, 0x05040100u);
        cols[4 * d + 1][th] = __builtin_amdgcn_perm(e, a, 0x07060302u);
        cols[4 * d + 2][th] = __builtin_amdgcn_perm(f, b, 0x05040100u);
        cols[4 * d + 3][th] = __builtin_amdgcn_perm(f, b, 0x07060302u);
      }
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      const int row = fc * 16 + h;
      *reinterpret_cast<u32x2*>(&tile[row * TILE + (((tg >> 1) ^ t_swz<CH>(row)) * 16) + (tg & 1) * 8]) =
          (u32x2){cols[h][0], cols[h][1]};
    }
    __syncthreads();
    if (it + 1 < ntiles) load_tile(n0 + (it + 1) * TILE);  // in flight during the MFMAs
#pragma unroll
    for (int s = 0; s < TILE / 64; ++s) {
      const int lc = 4 * s + 2 * h2;  // logical chunks: tokens 64s + 32h2 .. +31
      u32x8 a[RB], b[RB];
#pragma unroll
      for (int x = 0; x < RB; ++x) {
        const int fi = (ib0 + x) * 32 + r;
        const int fj = (jb0 + x) * 32 + r;
        a[x] = concat(lds_chunk(Kt, fi, lc), lds_chunk(Kt, fi, lc + 1));
        b[x] = concat(lds_chunk(Vt, fj, lc), lds_chunk(Vt, fj, lc + 1));
      }
#pragma unroll
      for (int x = 0; x < RB; ++x)
#pragma unroll
        for (int y = 0; y < RB; ++y) acc[x][y] = mfma32x32x64_fp8(a[x], b[y], acc[x][y]);
      if (zwave) {
#pragma unroll
        for (int x = 0; x < RB; ++x) zacc[x] = mfma32x32x64_fp8(a[x], ones, zacc[x]);
      }
    }
  }

  char* Pc = part + ((size_t)bh * C + c) * Partial<D>::kBytes;
  store_partial_s<D, true, RB>(acc, Pc, ib0, jb0, lane);
  // every column of zacc holds z; lane (r = 0, h2) writes rows q*8 + 4h2 .. +3
  if (zwave && r == 0) {
    float* Pz = reinterpret_cast<float*>(Pc + Partial<D>::kSBytes);
#pragma unroll
    for (int x = 0; x < RB; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(&Pz[(ib0 + x) * 32 + 8 * q + 4 * h2]) =
            (f32x4){zacc[x][4 * q], zacc[x][4 * q + 1], zacc[x][4 * q + 2], zacc[x][4 * q + 3]};
  }
}

// ---------------------------------------------------------------------------
// 2. fixed-order reduce of the partial states into output-pass fragments
// ---------------------------------------------------------------------------
// The state pass already stored its partials in the numerator fragments' order
// (frag_pos). Fragment (NJ, t) of the denominator holds z_hi[row(t, k)] in rows
// 0..7 and z_lo[row(t, k)] in rows 8..15. Chunks are summed in fp32 in order
// c = 0, 1, ..., C-1, with the loads of eight chunks in flight at a time.
template <int D, bool F8>
__global__ __launch_bounds__(256) void linear_reduce_bf16(const char* __restrict__ part,
                                                          uint32_t* __restrict__ state, int C) {
  constexpr int NT = D / 32, NJ = D / 16, NF = (NJ + 1) * NT;
  constexpr int NUM_WG = D * D / 8 / 256;  // workgroups for the numerator fragments
  constexpr size_t kStride = Partial<D>::kBytes;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const char* P = part + (size_t)bh * C * kStride;
  uint32_t* St = state + (size_t)bh * NF * 256;
  // 8 consecutive S slots (16 bytes of bf16) at slot `off`, summed over the chunks
  auto sum8_s = [&](size_t off, float* v) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int c = 0;
    auto add = [&](const u32x4 w) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[2 * q] += bf_lo(w[q]);
        a[2 * q + 1] += bf_hi(w[q]);
      }
    };
    for (; c + 8 <= C; c += 8) {
      u32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = ldg16(P + (c + u) * kStride + off * 2);
#pragma unroll
      for (int u = 0; u < 8; ++u) add(x[u]);
    }
    for (; c < C; ++c) add(ldg16(P + c * kStride + off * 2));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = a[e];
  };
  // 8 consecutive z entries (fp32) from entry `off`, summed over the chunks
  auto sum8_z = [&](size_t off, float* v) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    const char* Z = P + Partial<D>::kSBytes + off * 4;
    int c = 0;
    for (; c + 8 <= C; c += 8) {
      f32x4 x[16];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x[2 * u] = *reinterpret_cast<const f32x4*>(Z + (c + u) * kStride);
        x[2 * u + 1] = *reinterpret_cast<const f32x4*>(Z + (c + u) * kStride + 16);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a0 += x[2 * u];
        a1 += x[2 * u + 1];
      }
    }
    for (; c < C; ++c) {
      a0 += *reinterpret_cast<const f32x4*>(Z + c * kStride);
      a1 += *reinterpret_cast<const f32x4*>(Z + c * kStride + 16);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a0[e];
      v[4 + e] = a1[e];
    }
  };
  float v[8];
  if (blockIdx.x < NUM_WG) {
    const int x = blockIdx.x * 256 + tid;  // (fragment, lane) pair; 8 slots each
    sum8_s((size_t)x * 8, v);
    *reinterpret_cast<u32x4*>(St + (size_t)x * 4) =
        (u32x4){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
  } else if (tid < NT * 64) {
    const int t = tid >> 6, l = tid & 63, i = l & 15, g = l >> 4;
    sum8_z((size_t)z_run<D, F8>(t, g), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float hi = bf16_to_f32(f32_to_bf16(v[e]));
      v[e] = (i < 8) ? hi : (v[e] - hi);
    }
    *reinterpret_cast<u32x4*>(St + ((size_t)(NJ * NT + t) * 64 + l) * 4) =
        (u32x4){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
  }
}

// ---------------------------------------------------------------------------
// 3. output pass
// ---------------------------------------------------------------------------
// Each wave takes 16 tokens at a time. Q and G of the group move from HBM as
// whole 1 KB runs (64 lanes x 16 contiguous bytes per load instruction: four
// 256-byte token rows, or eight 128-byte fp8 rows) and pass through the wave's
// own LDS tile into the operand layout: lane (n = lane & 15, g = lane >> 4) then
// holds 16 bytes of Q and of G of token n per run, features 32u + 8g .. +7
// (bf16) or 64u + 16g .. +15 (fp8, two k-steps). That is both its B-operand
// slice and, by the fragment order (frag_pos), the feature run of its output
// values. O goes back through the same tile and leaves as 1 KB runs too (an
// fp32 O added into the stream at those runs); only a bf16 O added into is
// stored from the operand layout (16-byte accesses, 64 bytes per token and
// instruction), so that each sum is rounded to bf16 once, as before.
//
// Tile slots are 16-byte chunks: chunk c of token row t (R chunks per row) sits
// at t R + (c ^ ((t / (16 / R)) mod R)) for R <= 16 and at t R + (c ^ (t mod 16))
// for wider rows (an fp32 O), so the 16 lanes of one 16-byte LDS
// access (16 consecutive chunks of the 1 KB run, or one chunk of 16 rows) land
// on 16 distinct bank groups.
template <int R>
__device__ __forceinline__ int out_slot(int t, int c) {
  if constexpr (R >= 16) return t * R + (c ^ (t & 15));
  else return t * R + (c ^ ((t / (16 / R)) & (R - 1)));
}

// A wave's LDS tile is written by some lanes and read by others; a wave's LDS
// instructions execute in issue order, so keeping the compiler from moving
// them across this point is all the ordering needed.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

template <int D, bool OUT_F32, typename TIn>
__global__ __launch_bounds__(256, 2) void linear_out_bf16(const TIn* __restrict__ Q,
                                                       const TIn* __restrict__ G,
                                                       void* __restrict__ out,
                                                       const uint32_t* __restrict__ state, int N,
                                                       float eps, int accumulate) {
  constexpr bool F8 = sizeof(TIn) == 1;
  constexpr int NT = D / 32, NJ = D / 16, NF = (NJ + 1) * NT;
  constexpr int EPL = 16 / sizeof(TIn);  // features per run
  constexpr int NU = D / 4 / EPL;        // runs per lane and token (= load instructions per group)
  constexpr int JPU = NJ / NU;           // output fragments per run
  constexpr int CPR = D * (int)sizeof(TIn) / 16;  // 16-byte chunks per token row of Q or G
  constexpr int OCPR = D / 8;                     // 16-byte chunks per token row of a bf16 O
  constexpr int TILE = 16 * CPR;                  // chunks of Q (or G) per group
  constexpr int FCPR = D / 4;                     // 16-byte chunks per token row of an fp32 O
  constexpr int XS = OUT_F32 && 16 * FCPR > 2 * TILE ? 16 * FCPR : 2 * TILE;
  static_assert(CPR == 4 * NU && 16 * OCPR <= 2 * TILE, "tile shapes");
  __shared__ u32x4 fr[NF * 64];
  __shared__ u32x4 xs[4][XS];  // per wave: Q and G of its group, then its O
  // fp8 gates take 256 values: sigma of each, computed once per workgroup with
  // the same sigmoid, replaces an exp and a reciprocal per output element
  __shared__ float sig_tab[F8 ? 256 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.y;
  const int n = lane & 15, g = lane >> 4;
  const size_t base = (size_t)bh * N * D;
  const TIn* Qh = Q + base;
  const TIn* Gh = G + base;
  const int stride = gridDim.x * 4;
  int grp = blockIdx.x * 4 + wave;
  u32x4* const tq = xs[wave];
  u32x4* const tg = xs[wave] + TILE;

  // Buffer loads over the head: a token past N reads zeros without touching
  // memory, so every prefetch is issued unconditionally and the compiler can
  // wait for exactly the oldest group instead of draining every load. (Offsets
  // of prefetches beyond the last group may wrap 32 bits; they stay inside the
  // head, and their values are never used.) Q and G are read once, with the
  // non-temporal cache policy: with whole 1 KB runs that made the layer 0-11 %
  // faster than plain loads (with 64-byte pieces per token it had been slower).
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * sizeof(TIn));
  const rsrc_t Qr = make_rsrc(Qh, head_bytes), Gr = make_rsrc(Gh, head_bytes);
  auto load = [&](int gi, u32x4* qd, u32x4* gd) {
    const uint32_t off = (uint32_t)gi * (uint32_t)(16 * D * sizeof(TIn)) + 16u * lane;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      qd[u] = buf_load16_stream(Qr, off + 1024u * u);
      gd[u] = buf_load16_stream(Gr, off + 1024u * u);
    }
  };

  // The head's state fragments go to LDS; the first PF groups' Q and G loads
  // are issued after the fragment loads and before the wait for them, so the
  // latencies overlap (loads complete in order: waiting for the fragments
  // leaves the newer Q/G loads in flight).
  constexpr int FPT = (NF * 64 + 255) / 256;  // fragment loads per thread
  const rsrc_t Sr = make_rsrc(state + (size_t)bh * NF * 256, NF * 64 * 16);
  u32x4 frv[FPT];
#pragma unroll
  for (int i = 0; i < FPT; ++i) frv[i] = buf_load16(Sr, (tid + 256 * i) * 16);
  // PF groups ahead in flight, in PF + 1 register sets used in turn (the loop
  // is unrolled by PF + 1, so no set is copied into another: a copy would have
  // to wait for the loads it reads).
  constexpr int PF = F8 ? kLinearOutPrefetchF8 : kLinearOutPrefetch;
  u32x4 qs[PF + 1][NU], gs[PF + 1][NU];
#pragma unroll
  for (int s = 0; s < PF; ++s) load(grp + s * stride, qs[s], gs[s]);
#pragma unroll
  for (int i = 0; i < FPT; ++i)
    if (tid + 256 * i < NF * 64) fr[tid + 256 * i] = frv[i];
  if constexpr (F8) sig_tab[tid] = sigmoid(fp8_to_f32((uint8_t)tid));  // 256 threads, 256 codes
  __syncthreads();
  if (grp * 16 >= N) return;

  // sigma of the EPL gate values of one run
  auto gate_values = [&](const u32x4& gw, float* sg) __attribute__((always_inline)) {
    if constexpr (F8) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) sg[4 * q + e] = sig_tab[(gw[q] >> (8 * e)) & 0xffu];
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        sg[2 * p] = sigmoid(bf_lo(gw[p]));
        sg[2 * p + 1] = sigmoid(bf_hi(gw[p]));
      }
    }
  };
  auto compute = [&](int gi, const u32x4* qraw, const u32x4* graw) __attribute__((always_inline)) {
    // the 1 KB runs into the tile, then this lane's operand chunks out of it
    wave_lds_order();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int k = 64 * u + lane, sl = out_slot<CPR>(k / CPR, k % CPR);
      tq[sl] = qraw[u];
      tg[sl] = graw[u];
    }
    wave_lds_order();
    u32x4 qv[NU], gv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int sl = out_slot<CPR>(n, 4 * u + g);
      qv[u] = tq[sl];
      gv[u] = tg[sl];
    }
    // Re-read the fragments from LDS every group: an opaque (always zero)
    // offset keeps the compiler from hoisting all of them into registers,
    // which would cost the occupancy this streaming loop needs.
    int fo = lane;
    asm volatile("" : "+v"(fo));
    f32x4 acc[NJ], accd = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 b = relu_bf16x8(F8 ? fp8_half(qv[t >> 1], t & 1) : qv[t]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = mfma16x16x32(fr[(j * NT + t) * 64 + fo], b, acc[j]);
      accd = mfma16x16x32(fr[(NJ * NT + t) * 64 + fo], b, accd);
    }
    const float den = add_halves(accd[0]) + eps;
    const float rden = 1.0f / den;

    const int tok = gi * 16 + n;
    if (!OUT_F32 && !accumulate) {
      // bf16 O through the tile: this lane's runs in, 1 KB runs out (rows past N
      // are computed from zero Q and never stored)
      wave_lds_order();
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float o[EPL], sg[EPL];
#pragma unroll
        for (int jj = 0; jj < JPU; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[4 * jj + e] = acc[JPU * u + jj][e];
        gate_values(gv[u], sg);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = sg[e] * (o[e] * rden);
#pragma unroll
        for (int x = 0; x < EPL / 8; ++x)
          tq[out_slot<OCPR>(n, (4 * u + g) * (EPL / 8) + x)] =
              (u32x4){pack_bf16(o[8 * x], o[8 * x + 1]), pack_bf16(o[8 * x + 2], o[8 * x + 3]),
                      pack_bf16(o[8 * x + 4], o[8 * x + 5]), pack_bf16(o[8 * x + 6], o[8 * x + 7])};
      }
      wave_lds_order();
      uint16_t* dst = reinterpret_cast<uint16_t*>(out) + base + (size_t)gi * 16 * D;
#pragma unroll
      for (int v = 0; v < OCPR / 4; ++v) {
        const int k = 64 * v + lane, t = k / OCPR;
        const u32x4 ov = tq[out_slot<OCPR>(t, k % OCPR)];
        if (gi * 16 + t < N) stg16(dst + 8 * k, ov);
      }
    } else if (OUT_F32) {
      // fp32 O through the tile the same way; added into the stream at the
      // run positions when accumulating
      wave_lds_order();
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float o[EPL], sg[EPL];
#pragma unroll
        for (int jj = 0; jj < JPU; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[4 * jj + e] = acc[JPU * u + jj][e];
        gate_values(gv[u], sg);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = sg[e] * (o[e] * rden);
#pragma unroll
        for (int x = 0; x < EPL / 4; ++x)
          tq[out_slot<FCPR>(n, (4 * u + g) * (EPL / 4) + x)] = __builtin_bit_cast(
              u32x4, (f32x4){o[4 * x], o[4 * x + 1], o[4 * x + 2], o[4 * x + 3]});
      }
      wave_lds_order();
      float* dst = reinterpret_cast<float*>(out) + base + (size_t)gi * 16 * D;
#pragma unroll
      for (int v = 0; v < FCPR / 4; ++v) {
        const int k = 64 * v + lane, t = k / FCPR;
        f32x4 ov = __builtin_bit_cast(f32x4, tq[out_slot<FCPR>(t, k % FCPR)]);
        if (gi * 16 + t < N) {
          if (accumulate) ov += *reinterpret_cast<const f32x4*>(dst + 4 * k);
          *reinterpret_cast<f32x4*>(dst + 4 * k) = ov;
        }
      }
    } else if (tok < N) {
      // a bf16 O added into: from the operand layout, each run's sum rounded once
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        // run u: fragments JPU*u .. +JPU-1, 4 consecutive features each
        float o[EPL], sg[EPL];
#pragma unroll
        for (int jj = 0; jj < JPU; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[4 * jj + e] = acc[JPU * u + jj][e];
        gate_values(gv[u], sg);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = sg[e] * (o[e] * rden);
        uint16_t* dst = reinterpret_cast<uint16_t*>(out) + base + (size_t)tok * D + 4 * EPL * u + EPL * g;
#pragma unroll
        for (int x = 0; x < EPL / 8; ++x) {
          const u32x4 prev = ldg16(dst + 8 * x);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            o[8 * x + 2 * p] += bf_lo(prev[p]);
            o[8 * x + 2 * p + 1] += bf_hi(prev[p]);
          }
          stg16(dst + 8 * x, (u32x4){pack_bf16(o[8 * x], o[8 * x + 1]), pack_bf16(o[8 * x + 2], o[8 * x + 3]),
                                     pack_bf16(o[8 * x + 4], o[8 * x + 5]),
                                     pack_bf16(o[8 * x + 6], o[8 * x + 7])});
        }
      }
    }
  };
  for (;;) {
#pragma unroll
    for (int s = 0; s <= PF; ++s) {
      load(grp + PF * stride, qs[(s + PF) % (PF + 1)], gs[(s + PF) % (PF + 1)]);
      compute(grp, qs[s], gs[s]);
      if ((grp += stride) * 16 >= N) return;
    }
  }
}

template <int D, typename TIn>
hipError_t launch_d(const hla_dims& d, const void* q, const void* k, const void* v, const void* g,
                    const void* w, void* out, int accumulate, float eps, void* ws,
                    const LinearPlan& plan, hipStream_t stream) {
  const int BH = int(d.B * d.H), N = int(d.N);
  char* wsb = reinterpret_cast<char*>(ws);
  char* part = wsb + plan.part_off;
  uint32_t* state = reinterpret_cast<uint32_t*>(wsb + plan.state_off);
  const TIn* Kp = reinterpret_cast<const TIn*>(k);
  const TIn* Vp = reinterpret_cast<const TIn*>(v);
  const TIn* Qp = reinterpret_cast<const TIn*>(q);
  const TIn* Gp = reinterpret_cast<const TIn*>(g);
  if (w)
    hipLaunchKernelGGL((linear_state_bf16<D, true, TIn>), dim3(plan.C, BH), dim3(256), 0, stream,
                       Kp, Vp, reinterpret_cast<const TIn*>(w), part, N, plan.T, plan.C);
  else if constexpr (sizeof(TIn) == 1)
    hipLaunchKernelGGL((linear_state_fp8<D>), dim3(plan.C, BH), dim3(256), 0, stream, Kp, Vp, part,
                       N, plan.T, plan.C);
  else
    hipLaunchKernelGGL((linear_state_bf16<D, false, TIn>), dim3(plan.C, BH), dim3(256), 0, stream,
                       Kp, Vp, nullptr, part, N, plan.T, plan.C);
  hipLaunchKernelGGL((linear_reduce_bf16<D, sizeof(TIn) == 1>), dim3(D * D / 8 / 256 + 1, BH),
                     dim3(256), 0, stream, part, state, plan.C);
  if (d.out_dtype == HLA_F32)
    hipLaunchKernelGGL((linear_out_bf16<D, true, TIn>), dim3(plan.P, BH), dim3(256), 0, stream,
                       Qp, Gp, out, state, N, eps, accumulate);
  else
    hipLaunchKernelGGL((linear_out_bf16<D, false, TIn>), dim3(plan.P, BH), dim3(256), 0, stream,
                       Qp, Gp, out, state, N, eps, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bf16(const hla_dims& d, const void* q, const void* k, const void* v,
                              const void* g, const void* w, void* out, int accumulate, float eps,
                              void* ws, const LinearPlan& plan, hipStream_t stream) {
  if (d.in_dtype == HLA_FP8_E4M3) {
    if (d.D == 128)
      return launch_d<128, uint8_t>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
    return launch_d<64, uint8_t>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
  }
  if (d.D == 128)
    return launch_d<128, uint16_t>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
  return launch_d<64, uint16_t>(d, q, k, v, g, w, out, accumulate, eps, ws, plan, stream);
}

}  // namespace hla
