// Micro-benchmarks of the gfx950 units the attention kernels depend on: the
// bf16 matrix-core rate and the shader clock it sustains for operand data of
// different switching activity (register-fed, and fed from LDS as the anchor
// feeds it), the transcendental (v_exp_f32) rate, the LDS 16-byte read rate,
// and HBM streaming under the linear output pass's two candidate byte
// patterns. They back the hardware figures the kernels' rooflines are
// discussed against. Built into a library of its own (libhla_probes.so),
// separate from the attention library; callers pass device buffers and a
// stream, and time the launches themselves. hla_probe_cvt_fp8 runs the
// attention kernels' own fp32 -> e4m3 rounding (pack_fp8x4) on given values, so
// that tests can pin it to the format's definition.
//
// The compute probes write one float per thread to `out` (so the compiler keeps
// the work) and, from thread 0 of each workgroup, the workgroup's elapsed shader
// clock cycles (s_memtime, read after a barrier at the start and at the end of
// the timed loop, so the count spans every wave) to `clk`. Buffers:
// out >= grid * 512 floats, clk >= grid int64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hla_device.h"

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_p __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
// two finite bf16 values in [1, 2) with random mantissas
__device__ __forceinline__ uint32_t bf16_pair_near_one(uint32_t x) {
  return (x & 0x007f007fu) | 0x3f803f80u;
}

// MODE 0: A and B random bf16 (fixed per lane); 1: A and B zero; 2: one random
// register used as both A and B. WAVES waves per workgroup, one workgroup per
// CU; each wave issues iters * 8 MFMAs into four independent accumulators.
template <int MODE, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void probe_mfma(float* out, long long* clk, int iters) {
  const int tid = threadIdx.x;
  u32x4_p A[2], B[2];
  for (int i = 0; i < 2; ++i) {
    const uint32_t s = (blockIdx.x * 512u + tid) * 16u + i * 8u;
    A[i] = (u32x4_p){bf16_pair_near_one(mix(s)), bf16_pair_near_one(mix(s + 1)),
                     bf16_pair_near_one(mix(s + 2)), bf16_pair_near_one(mix(s + 3))};
    B[i] = (u32x4_p){bf16_pair_near_one(mix(s + 4)), bf16_pair_near_one(mix(s + 5)),
                     bf16_pair_near_one(mix(s + 6)), bf16_pair_near_one(mix(s + 7))};
    if (MODE == 1) A[i] = B[i] = (u32x4_p){0, 0, 0, 0};
    if (MODE == 2) B[i] = A[i];
  }
  f32x16_p acc[4];
  for (int i = 0; i < 4; ++i) acc[i] = (f32x16_p){};
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_p, A[m & 1]),
                                                           __builtin_bit_cast(bf16x8_p, B[m >> 2]),
                                                           acc[m & 3], 0, 0, 0);
  }
  __syncthreads();
  const long long t1 = clock64();
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int x = 0; x < 16; ++x) s += acc[i][x];
  out[blockIdx.x * 512 + tid] = s;
  if (tid == 0) clk[blockIdx.x] = t1 - t0;
}

// The same MFMA stream with LDS-fed A operands, as the attention kernels read
// their K and V^T operands: per iteration each lane reads R 16-byte chunks
// (lane-consecutive, conflict-free; the address advances with the iteration
// through a 64 KiB array of random bf16 pairs) and the wave issues 8 MFMAs, the
// A operand of MFMA m from read m * R / 8, the B operand one of two random
// registers. R = 8: one read per MFMA; R = 4: each read feeds two MFMAs with
// different B operands.
template <int R, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void probe_mfma_lds(float* out, long long* clk, int iters) {
  __shared__ u32x4_p lds[4096];  // 64 KiB
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 4096; i += 64 * WAVES) {
    const uint32_t s = (uint32_t)i * 4u + 0x9e37u;
    lds[i] = (u32x4_p){bf16_pair_near_one(mix(s)), bf16_pair_near_one(mix(s + 1)),
                       bf16_pair_near_one(mix(s + 2)), bf16_pair_near_one(mix(s + 3))};
  }
  u32x4_p B[2];
  for (int i = 0; i < 2; ++i) {
    const uint32_t s = (blockIdx.x * 512u + tid) * 16u + i * 8u + 4u;
    B[i] = (u32x4_p){bf16_pair_near_one(mix(s)), bf16_pair_near_one(mix(s + 1)),
                     bf16_pair_near_one(mix(s + 2)), bf16_pair_near_one(mix(s + 3))};
  }
  f32x16_p acc[4];
  for (int i = 0; i < 4; ++i) acc[i] = (f32x16_p){};
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    const int base = (it & 7) * 512 + lane;  // + 64 r + 512 (it & 7) <= 4095
    u32x4_p a[R];
#pragma unroll
    for (int r = 0; r < R; ++r) a[r] = lds[base + 64 * r];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_p, a[m * R / 8]),
                                                           __builtin_bit_cast(bf16x8_p, B[m & 1]),
                                                           acc[m & 3], 0, 0, 0);
  }
  __syncthreads();
  const long long t1 = clock64();
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int x = 0; x < 16; ++x) s += acc[i][x];
  out[blockIdx.x * 512 + tid] = s;
  if (tid == 0) clk[blockIdx.x] = t1 - t0;
}

// 16 independent chains per thread of x <- 2^x - 1.5 (a contraction towards a
// fixed point near -0.86, so values stay ordinary floats): iters * 16 v_exp_f32
// per thread, 512 threads per workgroup.
__global__ __launch_bounds__(512, 1) void probe_exp(float* out, long long* clk, int iters) {
  const int tid = threadIdx.x;
  float e[16];
  for (int i = 0; i < 16; ++i) e[i] = (float)(mix(tid * 16u + i) & 255u) * (1.0f / 256.0f) - 0.5f;
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(e[i]) - 1.5f;
  }
  __syncthreads();
  const long long t1 = clock64();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += e[i];
  out[blockIdx.x * 512 + tid] = s;
  if (tid == 0) clk[blockIdx.x] = t1 - t0;
}

// ds_read_b128 stream: 512 threads, 8 reads of 16 bytes per iteration at fixed
// addresses (lane-consecutive chunks, conflict-free, 8 KiB apart) inside a
// 64 KiB LDS array. The eight reads and their wait are one asm block, so all
// eight are in flight together and stay 16-byte reads although only one dword
// of each feeds the running XOR (one VALU op per read).
__global__ __launch_bounds__(512, 1) void probe_lds(float* out, long long* clk, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[16384];  // 64 KiB
  const int tid = threadIdx.x;
  for (int i = tid; i < 16384; i += 512) lds[i] = mix(i);
  __syncthreads();
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  // LDS byte address of this lane's chunk in the first 8 KiB; reads at +8 KiB * m
  const uint32_t a = (uint32_t)(uintptr_t)((lds_u32*)lds) + (uint32_t)(tid & 511) * 16u;
  uint32_t x = 0;
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    u32x4_p v0, v1, v2, v3, v4, v5, v6, v7;
    asm volatile(
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %8 offset:8192\n"
        "ds_read_b128 %2, %8 offset:16384\n"
        "ds_read_b128 %3, %8 offset:24576\n"
        "ds_read_b128 %4, %8 offset:32768\n"
        "ds_read_b128 %5, %8 offset:40960\n"
        "ds_read_b128 %6, %8 offset:49152\n"
        "ds_read_b128 %7, %8 offset:57344\n"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
        : "v"(a)
        : "memory");
    x ^= v0[0] ^ v1[1] ^ v2[2] ^ v3[3] ^ v4[0] ^ v5[1] ^ v6[2] ^ v7[3];
  }
  __syncthreads();
  const long long t1 = clock64();
  out[blockIdx.x * 512 + tid] = __uint_as_float(x & 0x3fffffffu);
  if (tid == 0) clk[blockIdx.x] = t1 - t0;
}

// Streaming with the gated linear output pass's byte pattern and no arithmetic:
// read two bf16 tensors [BH][N][128], write a third (o = q ^ g, bitwise), each
// wave taking 16-token groups (grid (P, BH), four waves per workgroup, the
// next two groups' loads in flight). Per 16-byte access, MODE 0 uses the
// operand layout (lane (n, g) takes token n, features 8g + 32u .. +7: each
// instruction touches 16 tokens x 64 bytes); MODE 1 moves 1 KB of consecutive
// bytes per instruction; MODE 2 loads as MODE 1 and stores as MODE 0; MODE 3
// loads as MODE 0 and stores as MODE 1 (the last two write o to permuted
// places; only their timing means something).
template <int MODE>
__global__ __launch_bounds__(256, 2) void probe_stream(const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ G,
                                                      uint16_t* __restrict__ O, int N) {
  constexpr int D = 128, PF = 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const size_t base = (size_t)blockIdx.y * N * D;
  const uint32_t head_bytes = (uint32_t)((size_t)N * D * 2);
  const hla::rsrc_t Qr = hla::make_rsrc(Q + base, head_bytes), Gr = hla::make_rsrc(G + base, head_bytes);
  const int stride = gridDim.x * 4;
  int grp = blockIdx.x * 4 + wave;
  // byte offset in the head of access u of group gi; `pieces` selects the operand layout
  auto off_of = [&](int gi, int u, bool pieces) -> uint32_t {
    return pieces ? ((uint32_t)(gi * 16 + n) * D + 8 * g + 32 * u) * 2
                  : (uint32_t)gi * 4096u + 1024u * u + 16u * lane;
  };
  constexpr bool kLoadPieces = MODE == 0 || MODE == 3, kStorePieces = MODE == 0 || MODE == 2;
  auto load = [&](int gi, u32x4_p* qd, u32x4_p* gd) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qd[u] = __builtin_bit_cast(u32x4_p, hla::buf_load16(Qr, off_of(gi, u, kLoadPieces)));
      gd[u] = __builtin_bit_cast(u32x4_p, hla::buf_load16(Gr, off_of(gi, u, kLoadPieces)));
    }
  };
  u32x4_p qs[PF + 1][4], gs[PF + 1][4];
#pragma unroll
  for (int s = 0; s < PF; ++s) load(grp + s * stride, qs[s], gs[s]);
  if (grp * 16 >= N) return;
  auto store = [&](int gi, const u32x4_p* qv, const u32x4_p* gv) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = kStorePieces ? gi * 16 + n : gi * 16 + 4 * u + (lane >> 4);
      if (tok < N) *reinterpret_cast<u32x4_p*>(O + base + off_of(gi, u, kStorePieces) / 2) = qv[u] ^ gv[u];
    }
  };
  for (;;) {
#pragma unroll
    for (int s = 0; s <= PF; ++s) {
      load(grp + PF * stride, qs[(s + PF) % (PF + 1)], gs[(s + PF) % (PF + 1)]);
      store(grp, qs[s], gs[s]);
      if ((grp += stride) * 16 >= N) return;
    }
  }
}

// out[i] = e4m3 bytes of in[4i .. 4i+3], as the anchor packs its probabilities
__global__ __launch_bounds__(256) void probe_cvt_fp8(const float* __restrict__ in,
                                                      uint32_t* __restrict__ out, int n4) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n4) out[i] = hla::pack_fp8x4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
}

}  // namespace

extern "C" {

// Status: 0 on success, 1 for an unsupported argument, 2 for a launch error.
int hla_probe_mfma(int mode, int waves_per_simd, int grid, int iters, float* out, long long* clk,
                   void* stream) {
  if (grid <= 0 || iters <= 0 || !out || !clk || mode < 0 || mode > 2 ||
      (waves_per_simd != 1 && waves_per_simd != 2))
    return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 g(grid);
  if (waves_per_simd == 1) {
    if (mode == 0) hipLaunchKernelGGL((probe_mfma<0, 4>), g, dim3(256), 0, s, out, clk, iters);
    if (mode == 1) hipLaunchKernelGGL((probe_mfma<1, 4>), g, dim3(256), 0, s, out, clk, iters);
    if (mode == 2) hipLaunchKernelGGL((probe_mfma<2, 4>), g, dim3(256), 0, s, out, clk, iters);
  } else {
    if (mode == 0) hipLaunchKernelGGL((probe_mfma<0, 8>), g, dim3(512), 0, s, out, clk, iters);
    if (mode == 1) hipLaunchKernelGGL((probe_mfma<1, 8>), g, dim3(512), 0, s, out, clk, iters);
    if (mode == 2) hipLaunchKernelGGL((probe_mfma<2, 8>), g, dim3(512), 0, s, out, clk, iters);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// reads_per_8: LDS operand reads per 8 MFMAs (8 or 4)
int hla_probe_mfma_lds(int reads_per_8, int waves_per_simd, int grid, int iters, float* out,
                       long long* clk, void* stream) {
  if (grid <= 0 || iters <= 0 || !out || !clk || (reads_per_8 != 8 && reads_per_8 != 4) ||
      (waves_per_simd != 1 && waves_per_simd != 2))
    return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 g(grid);
  if (waves_per_simd == 1) {
    if (reads_per_8 == 8) hipLaunchKernelGGL((probe_mfma_lds<8, 4>), g, dim3(256), 0, s, out, clk, iters);
    else hipLaunchKernelGGL((probe_mfma_lds<4, 4>), g, dim3(256), 0, s, out, clk, iters);
  } else {
    if (reads_per_8 == 8) hipLaunchKernelGGL((probe_mfma_lds<8, 8>), g, dim3(512), 0, s, out, clk, iters);
    else hipLaunchKernelGGL((probe_mfma_lds<4, 8>), g, dim3(512), 0, s, out, clk, iters);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// q, g, o: bf16 [BH][N][128]; P workgroups per head
int hla_probe_stream(int mode, int P, int BH, int N, const void* q, const void* g, void* o,
                     void* stream) {
  if (P <= 0 || BH <= 0 || BH > 65535 || N <= 0 || (long long)N * 256 >= (1LL << 32) || !q || !g ||
      !o || mode < 0 || mode > 3)
    return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(P, BH);
  const uint16_t *qq = static_cast<const uint16_t*>(q), *gg = static_cast<const uint16_t*>(g);
  uint16_t* oo = static_cast<uint16_t*>(o);
  if (mode == 0) hipLaunchKernelGGL(probe_stream<0>, grid, dim3(256), 0, s, qq, gg, oo, N);
  if (mode == 1) hipLaunchKernelGGL(probe_stream<1>, grid, dim3(256), 0, s, qq, gg, oo, N);
  if (mode == 2) hipLaunchKernelGGL(probe_stream<2>, grid, dim3(256), 0, s, qq, gg, oo, N);
  if (mode == 3) hipLaunchKernelGGL(probe_stream<3>, grid, dim3(256), 0, s, qq, gg, oo, N);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int hla_probe_exp(int grid, int iters, float* out, long long* clk, void* stream) {
  if (grid <= 0 || iters <= 0 || !out || !clk) return 1;
  hipLaunchKernelGGL(probe_exp, dim3(grid), dim3(512), 0, reinterpret_cast<hipStream_t>(stream), out,
                     clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// n4 groups of four floats -> n4 words of four e4m3 bytes
int hla_probe_cvt_fp8(const float* in, uint32_t* out, int n4, void* stream) {
  if (n4 <= 0 || !in || !out) return 1;
  hipLaunchKernelGGL(probe_cvt_fp8, dim3((n4 + 255) / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), in, out, n4);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int hla_probe_lds(int grid, int iters, float* out, long long* clk, void* stream) {
  if (grid <= 0 || iters <= 0 || !out || !clk) return 1;
  hipLaunchKernelGGL(probe_lds, dim3(grid), dim3(512), 0, reinterpret_cast<hipStream_t>(stream), out,
                     clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
