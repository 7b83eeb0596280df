// sk_microbench.hip -- kernels that measure the MFMA issue rate, the HBM
// read rate and the LDS read rate this MI355X sustains
// (include/sk_microbench.h).  Built into libskmb.so, apart from the GEMM
// library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sk_microbench.h"

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u2_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t *lds_v4s_t;

// A value in [-1, 1) from a hash of (lane, j, e): operands that differ from
// one MFMA to the next, so the datapath toggles as it does on real data (a
// single constant operand draws less power and lets the clock rise).
__device__ __forceinline__ float hval(int lane, int j, int e) {
  uint32_t x = (uint32_t)(lane * 977 + j * 131 + e * 31 + 7) * 2654435761u;
  x ^= x >> 15;
  x *= 2246822519u;
  x ^= x >> 13;
  return (float)(x >> 8) * (1.f / 8388608.f) - 1.f;
}

// Eight independent accumulators per wave, as in the GEMM kernels' wave
// tiles: four A fragments times two B fragments.
template <int DT>
__global__ __launch_bounds__(256) void mfma_kernel(int rounds, float *sink) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
  if constexpr (DT == 0) {
    float a[4], b[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = hval(lane, j, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = hval(lane, 4 + j, 0);
    f4_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f4_t{0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < rounds; r += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j & 3], b[j >> 2], c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  } else {
    using V8 = typename std::conditional<DT == 1, h8_t, b8_t>::type;
    using T = typename std::conditional<DT == 1, _Float16, __bf16>::type;
    V8 a[4], b[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j][e] = (T)hval(lane, j, e);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j][e] = (T)hval(lane, 4 + j, e);
    }
    f16v_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
    for (int r = 0; r < rounds; r += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (DT == 1)
            c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j & 3], b[j >> 2], c[j], 0, 0, 0);
          else
            c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[j >> 2], c[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += c[j][e];
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each wave reads blocks of 8 KiB (eight 1 KiB loads in flight, 16 bytes per
// lane each), blocks dealt round-robin to the waves; a tail of fewer than
// 8 KiB is read 16 bytes per lane.
__global__ __launch_bounds__(256) void read_kernel(const u4_t *src, int64_t n16, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int64_t blocks = n16 / 512;  // 512 pieces of 16 bytes = 8 KiB
  u4_t x = {0u, 0u, 0u, 0u};
  for (int64_t b = wave; b < blocks; b += waves) {
    const u4_t *p = src + b * 512 + lane;
    u4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[u * 64];
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  for (int64_t i = blocks * 512 + wave * 64 + lane; i < n16; i += waves * 64) x ^= src[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// LDS read rate: each workgroup fills 32 KiB of LDS, then every wave runs
// `rounds` rounds of 8 reads over it: MODE 0 reads 16 bytes per lane (1 KiB
// per instruction, lanes in order: no bank conflicts), MODE 1 reads 8 bytes
// per lane with the transposing read ds_read_b64_tr_b16 (512 bytes per
// instruction, lanes in order).  The round's offsets change from round to
// round and a compiler barrier between rounds keeps every read in the loop.
__device__ __attribute__((always_inline)) inline v4s_t tr_read(lds_v4s_t __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

template <int MODE>
__global__ __launch_bounds__(256) void lds_kernel(int rounds, uint32_t *sink) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[8192];
  for (int i = threadIdx.x; i < 8192; i += 256) buf[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const char *base = reinterpret_cast<const char *>(buf);
  uint32_t x = 0;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int blk = (r * 8 + u + w * 8) & 31;  // one of 32 blocks of 1 KiB
      if constexpr (MODE == 0) {
        const u4_t v = *reinterpret_cast<const u4_t *>(base + blk * 1024 + lane * 16);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else {
        const v4s_t v = tr_read((lds_v4s_t)(__attribute__((address_space(3))) void *)(base + blk * 1024 + lane * 8));
        const u2_t b = __builtin_bit_cast(u2_t, v);  // the same XOR work per byte as mode 0
        x ^= b[0] ^ b[1];
      }
    }
    asm volatile("" ::: "memory");
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

extern "C" int skmb_lds(int mode, int rounds, int grid, uint32_t *sink, hipStream_t stream) {
  if (rounds <= 0 || grid <= 0 || !sink || mode < 0 || mode > 1) return (int)hipErrorInvalidValue;
  if (mode == 0)
    hipLaunchKernelGGL(lds_kernel<0>, dim3(grid), dim3(256), 0, stream, rounds, sink);
  else
    hipLaunchKernelGGL(lds_kernel<1>, dim3(grid), dim3(256), 0, stream, rounds, sink);
  return (int)hipGetLastError();
}

extern "C" int skmb_mfma(int dtype, int rounds, int grid, float *sink, hipStream_t stream) {
  if (rounds <= 0 || rounds % 4 || grid <= 0 || !sink || dtype < 0 || dtype > 2) return (int)hipErrorInvalidValue;
  const dim3 g(grid), b(256);
  if (dtype == 0)
    hipLaunchKernelGGL(mfma_kernel<0>, g, b, 0, stream, rounds, sink);
  else if (dtype == 1)
    hipLaunchKernelGGL(mfma_kernel<1>, g, b, 0, stream, rounds, sink);
  else
    hipLaunchKernelGGL(mfma_kernel<2>, g, b, 0, stream, rounds, sink);
  return (int)hipGetLastError();
}

extern "C" int skmb_read(const void *src, int64_t bytes, int grid, uint32_t *sink, hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || grid <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const u4_t *>(src), bytes / 16,
                     sink);
  return (int)hipGetLastError();
}
