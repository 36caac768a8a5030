// Rank-r LoRA adapter path in fp32, every reduction in a fixed order.
//
// Gate walkthrough ("Soup layer-streamed NF4 training measured") section 2.1:
// LoRA r16 on q_proj and v_proj over the frozen NF4 base; section 2.2 check 2:
// the adapter gradients are non-zero in every layer; section 2.5: with B = 0
// the gradient of A vanishes structurally.
//
//   lora_fwd: u  = x . A^T                     [M, r]   (row dots over k_in)
//   lora_bwd: du = scale * dy . B              [M, r]   (row dots over n_out)
//             dB = scale * dy^T . u            [n_out, r] (column dots over M)
//             dA = du^T . x                    [r, k_in]  (column dots over M)
//
// Row dots: one wave per 4 rows, lanes stride the long dimension 8 elements at
// a time, the 64 partial sums are folded by a fixed butterfly. Column dots: a
// thread owns two adjacent columns and all r, the M rows are split over the
// grid's y dimension, and the split partials are summed in split order by a
// second kernel.
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int RCH = 16;        // rank handled per pass
constexpr int ROWS = 4;        // rows per wave in the row-dot kernel
constexpr int MSPLIT_ROWS = 32;  // rows per split in the column-dot kernel

__device__ __forceinline__ void bf16x8_to_f32(uint4 u, float* v) {
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  v[4] = __uint_as_float(u.z << 16);
  v[5] = __uint_as_float(u.z & 0xFFFF0000u);
  v[6] = __uint_as_float(u.w << 16);
  v[7] = __uint_as_float(u.w & 0xFFFF0000u);
}

// out[m, r0 + j] = scale * sum_k X[m, k] * W(j, k), j < 16, where W(j, k) is
// Wm[(r0 + j) * K + k] (TRANS_W = false, A[r, K]) or Wm[k * r + r0 + j]
// (TRANS_W = true, B[K, r]).
template <bool TRANS_W>
__global__ __launch_bounds__(256) void k_rowdot(const uint16_t* __restrict__ X, int64_t M,
                                                int64_t K, const float* __restrict__ Wm, int r,
                                                float scale, float* __restrict__ out) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t mbase = ((int64_t)blockIdx.x * 4 + wave) * ROWS;
  const int r0 = blockIdx.y * RCH;
  float acc[ROWS][RCH];
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
#pragma unroll
    for (int j = 0; j < RCH; ++j) acc[i][j] = 0.0f;

  for (int64_t k = (int64_t)lane * 8; k < K; k += 512) {
    float w[RCH][8];
#pragma unroll
    for (int j = 0; j < RCH; ++j) {
      const int rr = r0 + j;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[j][e] = (rr < r) ? (TRANS_W ? Wm[(k + e) * r + rr] : Wm[(int64_t)rr * K + k + e]) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      const int64_t m = mbase + i;
      if (m >= M) break;
      float xv[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(X + m * K + k), xv);
#pragma unroll
      for (int j = 0; j < RCH; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][j] = __builtin_fmaf(xv[e], w[j][e], acc[i][j]);
    }
  }
  // fixed butterfly over the 64 lanes; every lane ends with the full sum
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
#pragma unroll
    for (int j = 0; j < RCH; ++j)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc[i][j] += __shfl_xor(acc[i][j], o, 64);
  if (lane < RCH) {
    const int rr = r0 + lane;
    if (rr < r) {
#pragma unroll
      for (int i = 0; i < ROWS; ++i) {
        const int64_t m = mbase + i;
        if (m >= M) break;
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < RCH; ++j)
          if (j == lane) v = acc[i][j];
        out[m * r + rr] = scale * v;
      }
    }
  }
}

// part[s, n, j] = sum over rows m of split s of G[m, n] * U[m, r0 + j].
__global__ __launch_bounds__(256) void k_coldot(const uint16_t* __restrict__ G, int64_t M,
                                                int64_t N, const float* __restrict__ U, int r,
                                                int r0, float* __restrict__ part) {
  const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  const int s = blockIdx.y;
  const int64_t mb = (int64_t)s * MSPLIT_ROWS;
  const int64_t me = (mb + MSPLIT_ROWS < M) ? mb + MSPLIT_ROWS : M;
  if (n >= N) return;
  float acc0[RCH], acc1[RCH];
#pragma unroll
  for (int j = 0; j < RCH; ++j) acc0[j] = acc1[j] = 0.0f;
  for (int64_t m = mb; m < me; ++m) {
    const uint32_t gv = *reinterpret_cast<const uint32_t*>(G + m * N + n);
    const float g0 = __uint_as_float(gv << 16);
    const float g1 = __uint_as_float(gv & 0xFFFF0000u);
#pragma unroll
    for (int j = 0; j < RCH; ++j) {
      const float u = (r0 + j < r) ? U[m * r + r0 + j] : 0.0f;
      acc0[j] = __builtin_fmaf(g0, u, acc0[j]);
      acc1[j] = __builtin_fmaf(g1, u, acc1[j]);
    }
  }
  float* p0 = part + ((int64_t)s * N + n) * RCH;
#pragma unroll
  for (int j = 0; j < RCH; ++j) {
    p0[j] = acc0[j];
    p0[RCH + j] = acc1[j];
  }
}

// out (+)= scale * sum_s part[s, n, j], s in order; out is [N, r] (dB) or,
// with TRANS_OUT, [r, N] (dA).
template <bool TRANS_OUT>
__global__ __launch_bounds__(256) void k_colsum(const float* __restrict__ part, int splits,
                                                int64_t N, int r, int r0, float scale,
                                                int accumulate, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over N * RCH
  if (i >= N * RCH) return;
  const int64_t n = i / RCH;
  const int j = (int)(i % RCH);
  if (r0 + j >= r) return;
  float s = part[i];
  for (int p = 1; p < splits; ++p) s += part[(int64_t)p * N * RCH + i];
  s = scale * s;
  float* o = TRANS_OUT ? out + (int64_t)(r0 + j) * N + n : out + n * r + r0 + j;
  *o = accumulate ? *o + s : s;
}

template <bool TRANS_OUT>
hipError_t coldot(const uint16_t* G, int64_t M, int64_t N, const float* U, int r, float scale,
                  int accumulate, float* out, float* part, hipStream_t s) {
  const int splits = (int)((M + MSPLIT_ROWS - 1) / MSPLIT_ROWS);
  for (int r0 = 0; r0 < r; r0 += RCH) {
    hipLaunchKernelGGL(k_coldot, dim3((unsigned)((N / 2 + 255) / 256), (unsigned)splits),
                       dim3(256), 0, s, G, M, N, U, r, r0, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_colsum<TRANS_OUT>, dim3((unsigned)((N * RCH + 255) / 256)), dim3(256), 0, s, part,
                       splits, N, r, r0, scale, accumulate, out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t lora_bwd_ws_bytes(int64_t M, int64_t k_in, int64_t n_out) {
  const int64_t splits = (M + MSPLIT_ROWS - 1) / MSPLIT_ROWS;
  const int64_t n = k_in > n_out ? k_in : n_out;
  return (size_t)splits * (size_t)n * RCH * sizeof(float);
}

hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t k_in, const float* A, int r,
                           float* u, hipStream_t s) {
  const dim3 grid((unsigned)((M + 4 * ROWS - 1) / (4 * ROWS)), (unsigned)((r + RCH - 1) / RCH));
  hipLaunchKernelGGL(k_rowdot<false>, grid, dim3(256), 0, s, x, M, k_in, A, r, 1.0f, u);
  return hipGetLastError();
}

hipError_t launch_lora_bwd(const uint16_t* x, const uint16_t* dy, const float* u, int64_t M,
                           int64_t k_in, int64_t n_out, const float* B, int r, float scale,
                           float* dA, float* dB, float* du, int accumulate, void* ws,
                           hipStream_t s) {
  // du = scale * dy . B
  const dim3 grid((unsigned)((M + 4 * ROWS - 1) / (4 * ROWS)), (unsigned)((r + RCH - 1) / RCH));
  hipLaunchKernelGGL(k_rowdot<true>, grid, dim3(256), 0, s, dy, M, n_out, B, r, scale, du);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* part = static_cast<float*>(ws);
  // dB = scale * dy^T . u
  e = coldot<false>(dy, M, n_out, u, r, scale, accumulate, dB, part, s);
  if (e != hipSuccess) return e;
  // dA = du^T . x
  return coldot<true>(x, M, k_in, du, r, 1.0f, accumulate, dA, part, s);
}

}  // namespace nf4s
