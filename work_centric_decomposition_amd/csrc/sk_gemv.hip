// sk_gemv.hip -- matrix-vector products (m == 1 or n == 1) for CDNA4
// (gfx950): the even split of the work (the KBLAS page's block-row split,
// section 6.2, which is Stream-K's work-centric idea at the level of dot
// products), with the chunk sums combined in a fixed order by a second
// kernel instead of the page's atomic additions, so results are reproducible
// and beta is applied by the one writer of each output (the page needs a
// separate scaling kernel first, section 6.4).  Two forms, by the matrix
// operand's storage: rows contiguous along k (one dot product per output,
// split in k-chunks), or contiguous along the output (the page's transposed
// case: a wave owns a block of outputs and accumulates rows scaled by the
// vector's entries, the rows split in chunks).  The path is bound by HBM
// bandwidth: the matrix is read once, with 16-byte loads of 1 KiB per wave
// instruction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sk_internal.h"

namespace sk {
namespace dev {

typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));

// Storage type of each sk_dtype; products and sums are fp32, outputs are
// rounded once (to nearest even) by the conversion.
template <int DT> struct GvElem;
template <> struct GvElem<SK_F32> { using T = float; };
template <> struct GvElem<SK_F16> { using T = _Float16; };
template <> struct GvElem<SK_BF16> { using T = __bf16; };

// out[r] = alpha * (M row r) . v + beta * out[r] for r < R, M rows of K
// elements at M + r * ldm (k-contiguous, 16-byte aligned rows), v
// contiguous.  Task t = (r, s) is chunk s of row r: elements
// [s * chunk, min((s + 1) * chunk, K)).  Each wave takes tasks t = wave,
// wave + waves, ...; lane l multiplies 16-byte pieces l, l + 64, ... of the
// chunk (fp32 products and sums), eight pieces in flight per lane (four
// gave 6 % less bandwidth on a 16384 x 16384 matrix), the
// partial sums are reduced across the wave, and the wave's lane 0 writes
// the chunk sum to part[r * S + s] = part[t] (S > 1) or the result itself
// (S == 1).
template <int DT>
__global__ __launch_bounds__(256) void gemv_kernel(const void *M, int64_t ldm, const void *v, int64_t R,
                                                   int64_t K, int64_t chunk, int64_t S, float *part, void *out,
                                                   int64_t ldo, float alpha, float beta) {
  using T = typename GvElem<DT>::T;
  constexpr int VEC = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t tasks = R * S;
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); t < tasks; t += waves) {
    const int64_t r = t / S, s = t - r * S;
    const int64_t k0 = s * chunk, k1 = k0 + chunk < K ? k0 + chunk : K;
    const T *row = static_cast<const T *>(M) + r * ldm;
    const T *vec = static_cast<const T *>(v);
    float acc = 0.f;
    // whole 16-byte pieces of this chunk (chunks start on piece boundaries)
    const int64_t pieces = (k1 - k0) / VEC;
    int64_t p = lane;
    for (; p + 7 * 64 < pieces; p += 8 * 64) {
      u4_t mv[8], vv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        mv[u] = *reinterpret_cast<const u4_t *>(row + k0 + (p + u * 64) * VEC);
        vv[u] = *reinterpret_cast<const u4_t *>(vec + k0 + (p + u * 64) * VEC);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const T *mx = reinterpret_cast<const T *>(&mv[u]);
        const T *vx = reinterpret_cast<const T *>(&vv[u]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += (float)mx[e] * (float)vx[e];
      }
    }
    for (; p < pieces; p += 64) {
      const u4_t mv = *reinterpret_cast<const u4_t *>(row + k0 + p * VEC);
      const u4_t vv = *reinterpret_cast<const u4_t *>(vec + k0 + p * VEC);
      const T *mx = reinterpret_cast<const T *>(&mv);
      const T *vx = reinterpret_cast<const T *>(&vv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc += (float)mx[e] * (float)vx[e];
    }
    // the last (K mod VEC) elements of the row, in the chunk that ends at K
    for (int64_t kk = k0 + pieces * VEC + lane; kk < k1; kk += 64) acc += (float)row[kk] * (float)vec[kk];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) {
      if (S > 1) {
        part[t] = acc;
      } else {
        float o = alpha * acc;
        if (beta != 0.f) o += beta * (float)static_cast<const T *>(out)[r * ldo];
        static_cast<T *>(out)[r * ldo] = (T)o;
      }
    }
  }
}

// out[r] = alpha * sum_s part[r * S + s] + beta * out[r], RT threads per row
// (one wave, or the whole workgroup when there are many chunks): thread j
// adds chunks j, j + RT, ... in increasing order (loads issued eight at a
// time, the sums still taken one after another), the wave's lanes are
// combined by a fixed butterfly and, with RT = 256, the four wave sums in
// wave order, so repeated calls agree bitwise.
template <int DT, int RT>
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float *part, int64_t R, int64_t S, void *out,
                                                          int64_t ldo, float alpha, float beta) {
  using T = typename GvElem<DT>::T;
  static_assert(RT == 64 || RT == 256, "threads per row");
  __shared__ float wsum[4];
  const int j = threadIdx.x % RT, lane = threadIdx.x & 63;
  const int64_t rows_per_block = 256 / RT;
  for (int64_t r = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / RT; r < R;
       r += (int64_t)gridDim.x * rows_per_block) {
    const float *pr = part + r * S;
    float acc = 0.f;
    int64_t s = j;
    for (; s + 7 * RT < S; s += 8 * RT) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pr[s + u * RT];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; s < S; s += RT) acc += pr[s];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (RT == 256) {
      if (lane == 0) wsum[threadIdx.x >> 6] = acc;
      __syncthreads();
      acc = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
      __syncthreads();  // wsum is reused by the next row
    }
    if (j == 0) {
      float o = alpha * acc;
      if (beta != 0.f) o += beta * (float)static_cast<const T *>(out)[r * ldo];
      static_cast<T *>(out)[r * ldo] = (T)o;
    }
  }
}

// The axpy form: out[j * ldo] = alpha * sum_r v[r * incv] M[r * ldm + j] +
// beta * out[j * ldo] for j < R, r < K, the rows of M contiguous along the
// output (16-byte aligned base and rows).  Task t = s * blocks + b takes
// output block b (W = 64 VEC elements: lane l holds elements b W + l VEC
// .. + VEC - 1) over rows [s * chunk, min((s + 1) * chunk, K)) in order,
// eight rows' 16-byte pieces in flight (a wave reads 1 KiB of each row);
// fp32 products and sums.  The block's partial goes to part[s * R + j]
// (S > 1) or, with alpha and beta, to the output (S == 1).  The piece that
// holds the output's end, if partial, is read element by element.
template <int DT>
__global__ __launch_bounds__(256) void gemv_axpy_kernel(const void *M, int64_t ldm, const void *v, int64_t incv,
                                                        int64_t R, int64_t K, int64_t chunk, int64_t S, float *part,
                                                        void *out, int64_t ldo, float alpha, float beta) {
  using T = typename GvElem<DT>::T;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int64_t W = 64 * VEC;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t blocks = (R + W - 1) / W, tasks = blocks * S;
  const T *vp = static_cast<const T *>(v);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); t < tasks; t += waves) {
    const int64_t s = t / blocks, b = t - s * blocks;
    const int64_t r0 = s * chunk, r1 = r0 + chunk < K ? r0 + chunk : K;
    const int64_t j = b * W + (int64_t)lane * VEC;
    const T *col = static_cast<const T *>(M) + j;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    int64_t r = r0;
    if (j + VEC <= R) {
      for (; r + 8 <= r1; r += 8) {
        u4_t mv[8];
        float xv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          mv[u] = *reinterpret_cast<const u4_t *>(col + (r + u) * ldm);
          xv[u] = (float)vp[(r + u) * incv];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const T *mx = reinterpret_cast<const T *>(&mv[u]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] += xv[u] * (float)mx[e];
        }
      }
      for (; r < r1; ++r) {
        const u4_t mv = *reinterpret_cast<const u4_t *>(col + r * ldm);
        const float xr = (float)vp[r * incv];
        const T *mx = reinterpret_cast<const T *>(&mv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += xr * (float)mx[e];
      }
    } else if (j < R) {
      for (; r < r1; ++r) {
        const float xr = (float)vp[r * incv];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (j + e < R) acc[e] += xr * (float)col[r * ldm + e];
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (j + e >= R) break;
      if (S > 1) {
        part[s * R + j + e] = acc[e];
      } else {
        float o = alpha * acc[e];
        if (beta != 0.f) o += beta * (float)static_cast<const T *>(out)[(j + e) * ldo];
        static_cast<T *>(out)[(j + e) * ldo] = (T)o;
      }
    }
  }
}

// Output o < NO (o = i * R + j: vector i, output j) is
// out[i * ld_i + j * ld_j] = alpha * sum_s part[s * NO + o] + beta * (the
// same): a workgroup per 64 outputs, its wave w adding chunks
// [w S / 4, (w + 1) S / 4) of each in increasing order (eight loads in
// flight), then the four wave sums added in wave order, so repeated calls
// agree bitwise.
template <int DT>
__global__ __launch_bounds__(256) void gemv_part_reduce_kernel(const float *part, int64_t NO, int64_t R, int64_t S,
                                                               void *out, int64_t ld_i, int64_t ld_j, float alpha,
                                                               float beta) {
  using T = typename GvElem<DT>::T;
  __shared__ float wsum[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t s0 = S * w / 4, s1 = S * (w + 1) / 4;
  for (int64_t o0 = (int64_t)blockIdx.x * 64; o0 < NO; o0 += (int64_t)gridDim.x * 64) {
    const int64_t o = o0 + lane;
    float acc = 0.f;
    if (o < NO) {
      int64_t s = s0;
      for (; s + 8 <= s1; s += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(s + u) * NO + o];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      for (; s < s1; ++s) acc += part[s * NO + o];
    }
    wsum[w][lane] = acc;
    __syncthreads();
    if (w == 0 && o < NO) {
      const int64_t i = o / R, j = o - i * R;
      T *dst = static_cast<T *>(out) + i * ld_i + j * ld_j;
      float r = alpha * (((wsum[0][lane] + wsum[1][lane]) + wsum[2][lane]) + wsum[3][lane]);
      if (beta != 0.f) r += beta * (float)*dst;
      *dst = (T)r;
    }
    __syncthreads();  // wsum is reused by the next block of outputs
  }
}

// The multi form: D[i][r] = sum_k X[i][k] M[r][k] for vectors i < V (<= 16),
// rows r < R, both k-contiguous (16-byte aligned base and rows).  Task
// t = s * blocks + b takes rows [16 NB b, 16 NB (b + 1)) (NB blocks of 16)
// over k-chunk s, in slabs of one 16-byte load per lane and block: lane l
// loads row 16 (NB b + q) + (l & 15) of M for each block q and row (l & 15)
// of X (once for the NB blocks) at k offset VEC (l >> 4) of the slab, rows or
// vectors past the end as zeros, and the MFMAs sum over the slab (fp16 and
// bf16: one v_mfma_f32_16x16x32 per block and 32-k slab with X as the first
// operand; fp32: four v_mfma_f32_16x16x4 steps per block and 16-k slab, step
// e taking the e-th of every lane's four values, so that the lane groups
// cover k = 4 (l >> 4) + e).  U slabs' loads are in flight.  Lane l then
// holds D for vectors 4 (l >> 4) + e and rows 16 (NB b + q) + (l & 15).  A slab
// holding the end of k loads element by element, zeros past k.  The
// partials go to part[s * V R + i R + r] (S > 1) or, with alpha and beta, to
// out[i ld_v + r ld_r] (S == 1).
template <int DT, int NB, int U>
__global__ __launch_bounds__(256) void gemv_multi_kernel(const void *M, int64_t ldm, const void *X, int64_t ldx,
                                                         int V, int64_t R, int64_t K, int64_t chunk, int64_t S,
                                                         float *part, void *out, int64_t ld_v, int64_t ld_r,
                                                         float alpha, float beta) {
  using T = typename GvElem<DT>::T;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int64_t SLAB = 4 * VEC;
  const int lane = threadIdx.x & 63, li = lane & 15, kg = lane >> 4;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t blocks = (R + 16 * NB - 1) / (16 * NB), tasks = blocks * S;
  const bool xrow = li < V;
  const T *xp = static_cast<const T *>(X) + (xrow ? li : 0) * ldx + kg * VEC;
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); t < tasks; t += waves) {
    const int64_t s = t / blocks, b = t - s * blocks;
    const int64_t k0 = s * chunk, k1 = k0 + chunk < K ? k0 + chunk : K;
    bool mrow[NB];
    const T *mp[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int64_t row = b * 16 * NB + 16 * q + li;
      mrow[q] = row < R;
      mp[q] = static_cast<const T *>(M) + (mrow[q] ? row : 0) * ldm + kg * VEC;
    }
    f4_t acc[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) acc[q] = f4_t{0.f, 0.f, 0.f, 0.f};
    auto step = [&](f4_t &c, const u4_t &mv, const u4_t &xv) {
      if constexpr (DT == SK_F32) {
        const f4_t mf = __builtin_bit_cast(f4_t, mv), xf = __builtin_bit_cast(f4_t, xv);
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[e], mf[e], c, 0, 0, 0);
      } else if constexpr (DT == SK_F16) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xv), __builtin_bit_cast(h8_t, mv), c, 0,
                                                   0, 0);
      } else {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, xv), __builtin_bit_cast(b8_t, mv), c,
                                                    0, 0, 0);
      }
    };
    const u4_t zero = {0u, 0u, 0u, 0u};
    const int64_t kfull = k0 + (k1 - k0) / SLAB * SLAB;  // whole slabs of this chunk
    int64_t k = k0;
    for (; k + U * SLAB <= kfull; k += U * SLAB) {
      u4_t mv[U][NB], xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        xv[u] = xrow ? *reinterpret_cast<const u4_t *>(xp + k + u * SLAB) : zero;
#pragma unroll
        for (int q = 0; q < NB; ++q) mv[u][q] = mrow[q] ? *reinterpret_cast<const u4_t *>(mp[q] + k + u * SLAB) : zero;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < NB; ++q) step(acc[q], mv[u][q], xv[u]);
    }
    for (; k < kfull; k += SLAB) {
      const u4_t xv = xrow ? *reinterpret_cast<const u4_t *>(xp + k) : zero;
#pragma unroll
      for (int q = 0; q < NB; ++q) step(acc[q], mrow[q] ? *reinterpret_cast<const u4_t *>(mp[q] + k) : zero, xv);
    }
    if (k < k1) {  // the slab holding the end of k
      T xe[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) xe[e] = xrow && k + kg * VEC + e < k1 ? xp[k + e] : (T)0.f;
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        T me[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) me[e] = mrow[q] && k + kg * VEC + e < k1 ? mp[q][k + e] : (T)0.f;
        step(acc[q], __builtin_bit_cast(u4_t, me), __builtin_bit_cast(u4_t, xe));
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int64_t r = b * 16 * NB + 16 * q + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * kg + e;
        if (i >= V || r >= R) continue;
        if (S > 1) {
          part[s * (int64_t)V * R + i * R + r] = acc[q][e];
        } else {
          T *dst = static_cast<T *>(out) + i * ld_v + r * ld_r;
          float o = alpha * acc[q][e];
          if (beta != 0.f) o += beta * (float)*dst;
          *dst = (T)o;
        }
      }
    }
  }
}

}  // namespace dev

namespace {
void launch_reduce_parts(int dtype, const float *part, int64_t NO, int64_t R, int64_t S, void *out, int64_t ld_i,
                         int64_t ld_j, float alpha, float beta, hipStream_t stream) {
  const int64_t rb = (NO + 63) / 64;
  const dim3 g((unsigned)(rb < 8192 ? rb : 8192)), b(256);
  if (dtype == SK_F32)
    hipLaunchKernelGGL(dev::gemv_part_reduce_kernel<SK_F32>, g, b, 0, stream, part, NO, R, S, out, ld_i, ld_j, alpha,
                       beta);
  else if (dtype == SK_F16)
    hipLaunchKernelGGL(dev::gemv_part_reduce_kernel<SK_F16>, g, b, 0, stream, part, NO, R, S, out, ld_i, ld_j, alpha,
                       beta);
  else
    hipLaunchKernelGGL(dev::gemv_part_reduce_kernel<SK_BF16>, g, b, 0, stream, part, NO, R, S, out, ld_i, ld_j,
                       alpha, beta);
}

template <int DT>
void launch_axpy(const GemvPlan &g, float *part, float alpha, float beta, hipStream_t stream) {
  hipLaunchKernelGGL(dev::gemv_axpy_kernel<DT>, dim3(g.grid), dim3(256), 0, stream, g.M, g.ldm, g.v, g.incv, g.R,
                     g.K, g.chunk, g.S, part, g.out, g.ldo, alpha, beta);
  if (g.S > 1 && hipPeekAtLastError() == hipSuccess)
    launch_reduce_parts(DT, part, g.R, g.R, g.S, g.out, 0, g.ldo, alpha, beta, stream);
}

// Rows per task and slabs in flight, per element type: fp32 shares each
// vector load among four 16-row blocks (its vector loads otherwise rival the
// matrix's); fp16 and bf16 keep one block and eight slabs in flight.
template <int DT>
void launch_multi(const GemvPlan &g, float *part, float alpha, float beta, hipStream_t stream) {
  constexpr int NB = DT == SK_F32 ? 4 : 1, U = DT == SK_F32 ? 4 : 8;
  hipLaunchKernelGGL((dev::gemv_multi_kernel<DT, NB, U>), dim3(g.grid), dim3(256), 0, stream, g.M, g.ldm, g.v, g.ldv, g.V,
                     g.R, g.K, g.chunk, g.S, part, g.out, g.ld_v, g.ld_r, alpha, beta);
  if (g.S > 1 && hipPeekAtLastError() == hipSuccess)
    launch_reduce_parts(DT, part, (int64_t)g.V * g.R, g.R, g.S, g.out, g.ld_v, g.ld_r, alpha, beta, stream);
}

template <int DT>
void launch_dot(const GemvPlan &g, float *part, float alpha, float beta, hipStream_t stream) {
  hipLaunchKernelGGL(dev::gemv_kernel<DT>, dim3(g.grid), dim3(256), 0, stream, g.M, g.ldm, g.v, g.R, g.K, g.chunk,
                     g.S, part, g.out, g.ldo, alpha, beta);
  if (g.S == 1 || hipPeekAtLastError() != hipSuccess) return;
  // many chunks per row (few, long rows): a workgroup per row
  const bool wide = g.S >= 512;
  const int64_t rb = wide ? g.R : (g.R + 3) / 4;
  const dim3 rg((unsigned)(rb < 4096 ? rb : 4096));
  if (wide)
    hipLaunchKernelGGL((dev::gemv_reduce_kernel<DT, 256>), rg, dim3(256), 0, stream, part, g.R, g.S, g.out, g.ldo,
                       alpha, beta);
  else
    hipLaunchKernelGGL((dev::gemv_reduce_kernel<DT, 64>), rg, dim3(256), 0, stream, part, g.R, g.S, g.out, g.ldo,
                       alpha, beta);
}

}  // namespace

template <int DT>
void launch_form(const GemvPlan &g, float *part, float alpha, float beta, hipStream_t stream) {
  if (g.form == kGemvAxpy)
    launch_axpy<DT>(g, part, alpha, beta, stream);
  else if (g.form == kGemvMulti)
    launch_multi<DT>(g, part, alpha, beta, stream);
  else
    launch_dot<DT>(g, part, alpha, beta, stream);
}

int launch_gemv(int dtype, const GemvPlan &g, float *part, float alpha, float beta, hipStream_t stream) {
  if (dtype == SK_F32)
    launch_form<SK_F32>(g, part, alpha, beta, stream);
  else if (dtype == SK_F16)
    launch_form<SK_F16>(g, part, alpha, beta, stream);
  else
    launch_form<SK_BF16>(g, part, alpha, beta, stream);
  return (int)hipGetLastError();
}

}  // namespace sk
