// Rank-r LoRA adapter path on the matrix cores, every reduction in a fixed order.
//
// Gate walkthrough ("Soup layer-streamed NF4 training measured") section 2.1:
// LoRA r16 on q_proj and v_proj over the frozen NF4 base; section 2.2 check 2:
// the adapter gradients are non-zero in every layer; section 2.5: with B = 0
// the gradient of A vanishes structurally.
//
//   lora_fwd: u  = x . A^T            [M, r]     contraction over k_in
//   lora_bwd: du = scale * dy . B     [M, r]     contraction over n_out
//             dB = scale * dy^T . u   [n_out, r] contraction over M
//             dA = du^T . x           [r, k_in]  contraction over M
//
// Every product pairs a bf16 activation (x or dy, exact) with an fp32 adapter
// quantity F (A, B, u or du). F is split as F = hi + lo with hi = bf16(F) and
// lo = bf16(F - hi), and the 16 rank columns of hi and the 16 of lo form the
// 32 rows of one v_mfma_f32_32x32x16_bf16 operand; the two partial products
// land in accumulator rows j and j + 16 of the same lane and are added there.
// The split keeps about 17 bits of F, so the result carries fp32-level error
// while running on the matrix cores.
//
// Row kernel (u, du): one workgroup per 32 rows of the output and 512-wide
// chunk of the long contraction, its 4 waves take interleaved 16-wide slices,
// their tiles are summed through LDS in wave order, and a second kernel adds
// the chunks' partials in chunk order. Column kernel (dA, dB): one
// workgroup per 32 output columns, its 16 waves take sixteenths of M, summed the
// same way.
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int RCH = 16;  // rank columns per pass

__device__ __forceinline__ uint32_t bf16_bits(float v) {
  return pack_bf16x2(v, 0.0f) & 0xFFFFu;
}

// hi part (first) or lo part (second) of v, as bf16 bits
__device__ __forceinline__ uint32_t split_part(float v, bool lo) {
  const uint32_t h = bf16_bits(v);
  if (!lo) return h;
  return bf16_bits(v - __uint_as_float(h << 16));
}

__device__ __forceinline__ bf16x8_t frag_from_f32(const float* v, bool lo) {
  uint4 u;
  u.x = split_part(v[0], lo) | (split_part(v[1], lo) << 16);
  u.y = split_part(v[2], lo) | (split_part(v[3], lo) << 16);
  u.z = split_part(v[4], lo) | (split_part(v[5], lo) << 16);
  u.w = split_part(v[6], lo) | (split_part(v[7], lo) << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

constexpr int ROW_WAVES = 4;
constexpr int UNR = 8;                        // 16-wide slices per wave, loads issued together
constexpr int ROW_CHUNK = ROW_WAVES * UNR * 16;  // contraction handled by one workgroup (512)

// Adapters of one launch (the projections that read one input, e.g. q and
// v): the grid's last dimension runs over them.
constexpr int LORA_MAX = NF4S_MAX_LORA_GROUP;
struct RowsSeg {
  const uint16_t* X;  // [M, K]
  const float* F;     // A [r, K] or B [K, r]
  float* part;        // [nks, M, r] chunk partials
  float* out;         // [M, r]
  int64_t K;
  int nks;            // 512-wide chunks of K
};
struct RowsArgs {
  RowsSeg seg[LORA_MAX];
};

// Partial row dots: part[ks, m, r0 + j] = sum over k in chunk ks of
// X[m, k] * F(r0 + j, k), for one 32-row tile of m. F(j, k) = Fm[j * K + k]
// (TRANS_F = false: A [r, K]) or Fm[k * r + j] (TRANS_F = true: B [K, r]).
// MFMA view: C[rho, m] = sum_k F'[rho, k] X[m, k], rho < 16 the hi halves,
// rho >= 16 the lo halves. Wave w takes slices w, w + 4, ... of the chunk; the
// UNR loads of a wave are issued before its MFMAs; the 4 wave tiles are summed
// through LDS in wave order. blockIdx.z = rank chunk + rch * adapter.
template <bool TRANS_F>
__global__ __launch_bounds__(ROW_WAVES * 64) void k_lora_rows(RowsArgs ra, int64_t M, int r, int rch) {
  __shared__ float s_part[ROW_WAVES][64][8];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int lane = threadIdx.x & 63;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int ks = blockIdx.y;
  const int ad = blockIdx.z / rch;
  const int r0 = (blockIdx.z % rch) * RCH;
  const RowsSeg& sg = ra.seg[ad];
  if (ks >= sg.nks) return;  // uniform: this adapter's contraction has fewer chunks
  const uint16_t* __restrict__ X = sg.X;
  const float* __restrict__ Fm = sg.F;
  float* __restrict__ part = sg.part;
  const int64_t K = sg.K;
  const int rho = lane & 31;
  const bool lo = rho >= 16;
  const int j = r0 + (rho & 15);
  const int jc = j < r ? j : r - 1;
  const int kq = (lane >> 5) * 8;
  const int64_t m = m0 + rho;
  const int64_t mc = m < M ? m : M - 1;  // rows past M feed unstored columns
  float f[UNR][8];
  uint4 xv[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int64_t k = (int64_t)ks * ROW_CHUNK + (int64_t)(u * ROW_WAVES + wave) * 16 + kq;
    const bool ok = k < K;  // K % 8 == 0, so k < K covers all 8 elements
    const int64_t kc = ok ? k : K - 8;
    if (TRANS_F) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[u][e] = Fm[(kc + e) * r + jc];
    } else {
      const float4 a = *reinterpret_cast<const float4*>(Fm + (int64_t)jc * K + kc);
      const float4 b = *reinterpret_cast<const float4*>(Fm + (int64_t)jc * K + kc + 4);
      f[u][0] = a.x; f[u][1] = a.y; f[u][2] = a.z; f[u][3] = a.w;
      f[u][4] = b.x; f[u][5] = b.y; f[u][6] = b.z; f[u][7] = b.w;
    }
    if (!(ok && j < r)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[u][e] = 0.0f;
    }
    xv[u] = *reinterpret_cast<const uint4*>(X + mc * K + kc);
  }
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const bf16x8_t fa = frag_from_f32(f[u], lo);
    const bf16x8_t fb = __builtin_bit_cast(bf16x8_t, xv[u]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
  }
  // register r (< 8) holds rank row 8*(r/4) + 4*(lane/32) + r%4 (hi), r + 8 its lo
#pragma unroll
  for (int i = 0; i < 8; ++i) s_part[wave][lane][i] = acc[i] + acc[i + 8];
  __syncthreads();
  if (wave == 0) {
    const int64_t mo = m0 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sum = s_part[0][lane][i];
      for (int w = 1; w < ROW_WAVES; ++w) sum += s_part[w][lane][i];
      const int jj = r0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (mo < M && jj < r) part[((int64_t)ks * M + mo) * r + jj] = sum;
    }
  }
}

// out[m, j] = scale * sum_ks part[ks, m, j], ks in order; blockIdx.y = adapter.
__global__ __launch_bounds__(256) void k_rows_sum(RowsArgs ra, int64_t n, float scale) {
  const RowsSeg& sg = ra.seg[blockIdx.y];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // the partials in chunk order; loads issued eight at a time ahead of
  // their adds, which keep that order
  float s = sg.part[i];
  for (int p = 1; p < sg.nks; p += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (p + q < sg.nks) v[q] = sg.part[(int64_t)(p + q) * n + i];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (p + q < sg.nks) s += v[q];
  }
  sg.out[i] = scale * s;
}

int64_t row_chunks(int64_t K) { return (K + ROW_CHUNK - 1) / ROW_CHUNK; }

// n adapters: X[i] [M, K[i]] against F[i]; partials packed one after the other in ws
hipError_t rowdot(bool trans_f, int n, const uint16_t* const* X, int64_t M, const int64_t* K,
                  const float* const* F, int r, float scale, float* const* out, float* ws,
                  hipStream_t s) {
  RowsArgs ra = {};
  int64_t nks_max = 0;
  float* part = ws;
  for (int i = 0; i < n; ++i) {
    RowsSeg& sg = ra.seg[i];
    sg.X = X[i];
    sg.F = F[i];
    sg.out = out[i];
    sg.K = K[i];
    sg.nks = (int)row_chunks(K[i]);
    sg.part = part;
    part += (size_t)sg.nks * (size_t)M * (size_t)r;
    nks_max = sg.nks > nks_max ? sg.nks : nks_max;
  }
  const int rch = (r + RCH - 1) / RCH;
  const dim3 grid((unsigned)((M + 31) / 32), (unsigned)nks_max, (unsigned)(rch * n));
  if (trans_f)
    hipLaunchKernelGGL(k_lora_rows<true>, grid, dim3(ROW_WAVES * 64), 0, s, ra, M, r, rch);
  else
    hipLaunchKernelGGL(k_lora_rows<false>, grid, dim3(ROW_WAVES * 64), 0, s, ra, M, r, rch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nel = M * r;
  hipLaunchKernelGGL(k_rows_sum, dim3((unsigned)((nel + 255) / 256), (unsigned)n), dim3(256), 0, s, ra,
                     nel, scale);
  return hipGetLastError();
}

constexpr int COL_WAVES = 16;

struct ColsSeg {
  const uint16_t* G;  // [M, N]
  const float* L;     // [M, r]
  float* out;         // [r, N] or [N, r]
  int64_t N;
};
struct ColsArgs {
  ColsSeg seg[LORA_MAX];
};

// out(r0 + j, c) (+)= scale * sum_m L[m, r0 + j] * G[m, c] for one 32-column
// tile of c; out is [r, N] (dA) or, with TRANS_OUT, [N, r] (dB).
// MFMA view: C[rho, c] = sum_m L'[rho, m] G[m, c]. The waves take consecutive
// stretches of M in 16-row slices. The contraction runs over M, which is G's
// row index, while each lane of the B operand needs 8 consecutive rows of
// one column: a wave reads its 16 x 32 slice of G with one 16-byte load per
// lane (a row's 8 consecutive columns) and the 16 x 16 slice of L with four
// 4-byte loads per lane, writes both into LDS of its own (G transposed), and
// reads the operands back -- lanes of one wave, whose LDS accesses complete
// in issue order, so no workgroup barrier is needed. blockIdx.z = adapter.
constexpr int CT_STRIDE = 24;  // bf16 per transposed row (16 rows + 8 pad: 16-B reads, 2-way writes)
constexpr int CL_STRIDE = 17;  // fp32 per staged L row
constexpr int COL_WAVE_LDS = 32 * CT_STRIDE * 2 + 16 * CL_STRIDE * 4;  // bytes per wave
constexpr int COL_SMEM = (COL_WAVES * COL_WAVE_LDS > COL_WAVES * 64 * 8 * 4) ? COL_WAVES * COL_WAVE_LDS
                                                                              : COL_WAVES * 64 * 8 * 4;

template <bool TRANS_OUT>
__global__ __launch_bounds__(COL_WAVES * 64) void k_lora_cols(ColsArgs ca, int64_t M, int r,
                                                              float scale, int accumulate) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[COL_SMEM];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int lane = threadIdx.x & 63;
  const int64_t c0 = (int64_t)blockIdx.x * 32;
  const int r0 = blockIdx.y * RCH;
  const ColsSeg& sg = ca.seg[blockIdx.z];
  const int64_t N = sg.N;
  if (c0 >= N) return;  // uniform: this adapter is narrower than the grid
  const uint16_t* __restrict__ G = sg.G;
  const float* __restrict__ Lm = sg.L;
  float* __restrict__ out = sg.out;
  uint16_t* const Ts = reinterpret_cast<uint16_t*>(smem + wave * COL_WAVE_LDS);  // [32 c][CT_STRIDE]
  float* const Ls = reinterpret_cast<float*>(smem + wave * COL_WAVE_LDS + 32 * CT_STRIDE * 2);  // [16 m][CL_STRIDE]
  // loads: lane l takes slice row l / 4, columns 8 (l % 4) .. +8 of G and
  // ranks 4 (l % 4) .. +4 of L
  const int lrow = lane >> 2, lq = lane & 3;
  const int64_t gc = c0 + 8 * lq;  // N % 8 == 0: the 8 columns are all in or all out
  // operands: lane l is MFMA row / column l % 32, contraction half l / 32
  const int rho = lane & 31, hf = lane >> 5;
  const bool lo = rho >= 16;
  const int per = (int)(((M + COL_WAVES * 16 - 1) / (COL_WAVES * 16)) * 16);
  const int64_t mb = (int64_t)wave * per;
  const int64_t me = (mb + per < M) ? mb + per : M;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  for (int64_t m1 = mb; m1 < me; m1 += 16) {
    const int64_t m = m1 + lrow;
    const bool okm = m < me;
    uint4 gv = make_uint4(0u, 0u, 0u, 0u);
    if (okm && gc < N) gv = *reinterpret_cast<const uint4*>(G + m * N + gc);
    float lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int jj = r0 + 4 * lq + q;
      lv[q] = (okm && jj < r) ? Lm[m * r + jj] : 0.0f;
    }
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      Ts[(8 * lq + e) * CT_STRIDE + lrow] = (uint16_t)((e & 1) ? (gw[e >> 1] >> 16) : (gw[e >> 1] & 0xFFFFu));
#pragma unroll
    for (int q = 0; q < 4; ++q) Ls[lrow * CL_STRIDE + 4 * lq + q] = lv[q];
    __builtin_amdgcn_wave_barrier();
    const uint4 bv = *reinterpret_cast<const uint4*>(Ts + rho * CT_STRIDE + 8 * hf);
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = Ls[(8 * hf + e) * CL_STRIDE + (rho & 15)];
    __builtin_amdgcn_wave_barrier();
    const bf16x8_t fa = frag_from_f32(f, lo);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
  }
  __syncthreads();  // every wave is done with its staging area before the partials reuse it
  float (*s_part)[64][8] = reinterpret_cast<float (*)[64][8]>(smem);
#pragma unroll
  for (int i = 0; i < 8; ++i) s_part[wave][lane][i] = acc[i] + acc[i + 8];
  __syncthreads();
  if (wave == 0) {
    const int64_t co = c0 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sacc = s_part[0][lane][i];
      for (int w = 1; w < COL_WAVES; ++w) sacc += s_part[w][lane][i];
      const int jj = r0 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (co < N && jj < r) {
        float* o = TRANS_OUT ? out + co * r + jj : out + (int64_t)jj * N + co;
        const float v = scale * sacc;
        *o = accumulate ? *o + v : v;
      }
    }
  }
}

}  // namespace

size_t lora_fwd_ws_bytes(int64_t M, int64_t k_in, int r) {
  return (size_t)row_chunks(k_in) * (size_t)M * (size_t)r * sizeof(float);
}

size_t lora_bwd_ws_bytes(int64_t M, int64_t n_out, int r) {
  return (size_t)row_chunks(n_out) * (size_t)M * (size_t)r * sizeof(float);
}

hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t k_in, const float* A, int r,
                           float* u, void* ws, hipStream_t s) {
  return launch_lora_fwd_grouped(x, M, k_in, &A, 1, r, &u, ws, s);
}

hipError_t launch_lora_fwd_grouped(const uint16_t* x, int64_t M, int64_t k_in, const float* const* A,
                                   int n, int r, float* const* u, void* ws, hipStream_t s) {
  const uint16_t* X[LORA_MAX];
  int64_t K[LORA_MAX];
  for (int i = 0; i < n; ++i) {
    X[i] = x;
    K[i] = k_in;
  }
  return rowdot(false, n, X, M, K, A, r, 1.0f, u, static_cast<float*>(ws), s);
}

hipError_t launch_lora_bwd(const uint16_t* x, const uint16_t* dy, const float* u, int64_t M,
                           int64_t k_in, int64_t n_out, const float* B, int r, float scale,
                           float* dA, float* dB, float* du, int accumulate, void* ws,
                           hipStream_t s) {
  return launch_lora_bwd_grouped(x, &dy, &u, M, k_in, &n_out, &B, 1, r, scale, &dA, &dB, &du,
                                 accumulate, ws, s);
}

hipError_t launch_lora_bwd_grouped(const uint16_t* x, const uint16_t* const* dy,
                                   const float* const* u, int64_t M, int64_t k_in,
                                   const int64_t* n_out, const float* const* B, int n, int r,
                                   float scale, float* const* dA, float* const* dB,
                                   float* const* du, int accumulate, void* ws, hipStream_t s) {
  const unsigned rch = (unsigned)((r + RCH - 1) / RCH);
  // du = scale * dy . B
  hipError_t e = rowdot(true, n, dy, M, n_out, B, r, scale, du, static_cast<float*>(ws), s);
  if (e != hipSuccess) return e;
  ColsArgs cb = {}, ca = {};
  int64_t nmax = 0;
  for (int i = 0; i < n; ++i) {
    cb.seg[i] = ColsSeg{dy[i], u[i], dB[i], n_out[i]};
    ca.seg[i] = ColsSeg{x, du[i], dA[i], k_in};
    nmax = n_out[i] > nmax ? n_out[i] : nmax;
  }
  // dB = scale * dy^T . u   ([n_out, r])
  hipLaunchKernelGGL(k_lora_cols<true>, dim3((unsigned)((nmax + 31) / 32), rch, (unsigned)n),
                     dim3(COL_WAVES * 64), 0, s, cb, M, r, scale, accumulate);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dA = du^T . x           ([r, k_in])
  hipLaunchKernelGGL(k_lora_cols<false>, dim3((unsigned)((k_in + 31) / 32), rch, (unsigned)n),
                     dim3(COL_WAVES * 64), 0, s, ca, M, r, 1.0f, accumulate);
  return hipGetLastError();
}

}  // namespace nf4s
