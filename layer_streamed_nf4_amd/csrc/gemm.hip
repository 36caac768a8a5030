// Fused NF4-dequant bf16 MFMA GEMMs for the frozen linears.
//
// Forward  y[M, n_out]  = x[M, k_in] . W'^T   (+ s . u . B^T)
// Backward dx[M, k_in]  = dy[M, n_out] . W'   (+ du . A)
// Gate walkthrough ("Soup layer-streamed NF4 training measured") section 2.1:
// the NF4 weight is rebuilt from the streamed bytes on every call and used with
// bf16 compute; section 4.4: the frozen base needs dL/dx but no dL/dW.
//
// Both directions are one kernel template computing C[M, Nc] = A[M, Kc] . B,
// where A is the bf16 activation (x or dy, row stride Kc) and B[Kc, Nc] is the
// dequantised weight seen either transposed (forward: B[k][n] = W'[n][k]) or
// as is (backward: B[k][n] = W'[k][n]). The packed codes are read from HBM once
// per workgroup, decoded in registers with the block scale
// a' = fp32(fp32(C8[q8]*nested) + offset) and W' = bf16_rne(fp32(C4[code]*a')),
// and written to LDS as bf16 in the column-major-by-contraction layout the
// matrix cores read; W' never goes back to HBM. The backward orientation is
// transposed on the way into LDS for free: a thread decodes a 4x8 patch and
// pairs values along the contraction when it packs bf16.
//
// Tiling for gfx950: 256 threads (4 wave64), output tile 256x128, contraction
// step 64 (exactly one NF4 block per weight row in the forward direction),
// v_mfma_f32_32x32x16_bf16 with each wave owning a 128x64 sub-tile (4x2 MFMA
// tiles, 128 fp32 accumulators per lane), double-buffered LDS (stage n+1 is
// fetched into registers while stage n feeds the matrix cores). LDS rows are
// padded to 144 B so the 16-byte fragment reads of 8 consecutive lanes cover
// all 32 banks. When the output has too few tiles to occupy the chip, the
// contraction is split; each split writes fp32 partials and a second kernel
// sums them in split order (deterministic, no atomics).
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDS_STRIDE = 72;  // bf16 elements per LDS row (64 + 8 pad = 144 B)
constexpr int THREADS = 256;

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* q8;
  const float* nested;
  const float* offset;
  const uint16_t* a;  // bf16 [M, Kc]
  int64_t M, Kc, Nc;
  int64_t n_out, k_in;
  uint16_t* out;       // bf16 [M, Nc]
  float* part;         // fp32 [splits, M, Nc] (splits > 1)
  int64_t kc_chunk;
  const float* lora_l;  // fp32 [M, r]
  const float* lora_r;  // fwd: B fp32 [n_out, r]; bwd: A fp32 [r, k_in]
  int r;
  float scale;
};

template <bool BWD>
struct BRegs;

// Forward: thread t owns weight row n0 + t/2, contraction half t%2 (32 codes).
template <>
struct BRegs<false> {
  uint4 w;
  uint32_t q;
  float nest;
  bool valid;
};

// Backward: thread t owns weight rows k0 + 4*(t/16) + i (i < 4) and output
// columns n0 + 8*(t%16) + j (j < 8): four packed words, four scales.
template <>
struct BRegs<true> {
  uint32_t w[4];
  uint32_t q[4];
  float nest[4];
  bool valid[4];
};

__device__ __forceinline__ void load_a(const GemmArgs& g, int64_t m0, int64_t k0, uint4 (&ra)[8]) {
  const int t = threadIdx.x;
  const int c = t & 7;
  const int64_t kk = k0 + c * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + (t >> 3) + 32 * i;
    if (row < g.M && kk < g.Kc)
      ra[i] = *reinterpret_cast<const uint4*>(g.a + row * g.Kc + kk);
    else
      ra[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_a(uint16_t* As, const uint4 (&ra)[8]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (t >> 3) + 32 * i;
    *reinterpret_cast<uint4*>(As + row * LDS_STRIDE + c * 8) = ra[i];
  }
}

__device__ __forceinline__ void load_b(const GemmArgs& g, int64_t n0, int64_t k0, BRegs<false>& rb) {
  const int t = threadIdx.x;
  const int64_t n = n0 + (t >> 1);
  const int half = t & 1;
  rb.valid = n < g.n_out;
  if (rb.valid) {
    const int64_t e = n * g.k_in + k0 + half * 32;
    rb.w = *reinterpret_cast<const uint4*>(g.packed + e / 2);
    const int64_t blk = (n * g.k_in + k0) / 64;
    rb.q = g.q8[blk];
    rb.nest = g.nested[blk >> 8];
  }
}

__device__ __forceinline__ void store_b(uint16_t* Bs, const BRegs<false>& rb, float off,
                                        const float* c4, const float* c8) {
  const int t = threadIdx.x;
  const int row = t >> 1;
  const int half = t & 1;
  uint4* dst = reinterpret_cast<uint4*>(Bs + row * LDS_STRIDE + half * 32);
  if (!rb.valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = make_uint4(0, 0, 0, 0);
    return;
  }
  const float a = decode_scale(c8[rb.q], rb.nest, off);
  const uint32_t words[4] = {rb.w.x, rb.w.y, rb.w.z, rb.w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t o[4];
    dequant_word(words[j], a, c4, o);
    dst[j] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__device__ __forceinline__ void load_b(const GemmArgs& g, int64_t n0, int64_t k0, BRegs<true>& rb) {
  const int t = threadIdx.x;
  const int64_t col = n0 + 8 * (t & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = k0 + 4 * (t >> 4) + i;
    rb.valid[i] = row < g.n_out && col < g.k_in;
    if (rb.valid[i]) {
      const int64_t e = row * g.k_in + col;
      rb.w[i] = *reinterpret_cast<const uint32_t*>(g.packed + e / 2);
      const int64_t blk = e / 64;
      rb.q[i] = g.q8[blk];
      rb.nest[i] = g.nested[blk >> 8];
    }
  }
}

__device__ __forceinline__ void store_b(uint16_t* Bs, const BRegs<true>& rb, float off,
                                        const float* c4, const float* c8) {
  const int t = threadIdx.x;
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (rb.valid[i]) {
      const float a = decode_scale(c8[rb.q[i]], rb.nest[i], off);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = __fmul_rn(c4[nib(rb.w[i], j)], a);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
  }
  const int cb = 8 * (t & 15);
  const int rbase = 4 * (t >> 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint2 pk;
    pk.x = pack_bf16x2(v[0][j], v[1][j]);
    pk.y = pack_bf16x2(v[2][j], v[3][j]);
    *reinterpret_cast<uint2*>(Bs + (cb + j) * LDS_STRIDE + rbase) = pk;
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* base, int row, int kofs) {
  return *reinterpret_cast<const bf16x8_t*>(base + row * LDS_STRIDE + kofs);
}

__device__ __forceinline__ bf16x8_t f32x8_to_bf16(const float* v) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// SPLIT selects the output path (fp32 partials vs bf16 result) at compile time,
// so the two variants also carry distinct kernel names in profiles.
template <bool BWD, bool SPLIT>
__global__ __launch_bounds__(THREADS, 1) void k_gemm(GemmArgs g, Tables tab) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  __shared__ float s_c4[16];
  __shared__ float s_c8[256];

  const int t = threadIdx.x;
  if (t < 16) s_c4[t] = tab.c4[t];
  s_c8[t] = tab.c8[t];

  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int split = blockIdx.z;
  const int64_t kb = split * g.kc_chunk;
  const int64_t ke = (kb + g.kc_chunk < g.Kc) ? kb + g.kc_chunk : g.Kc;
  const int nk = (int)((ke - kb + BK - 1) / BK);
  const float off = g.offset[0];

  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave >> 1;  // 128-row half of the tile
  const int wn = wave & 1;   // 64-column half of the tile
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 ra[8];
  BRegs<BWD> rb;
  load_a(g, m0, kb, ra);
  load_b(g, n0, kb, rb);
  __syncthreads();  // tables in LDS
  store_a(As[0], ra);
  store_b(Bs[0], rb, off, s_c4, s_c8);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_a(g, m0, kb + (int64_t)(kt + 1) * BK, ra);
      load_b(g, n0, kb + (int64_t)(kt + 1) * BK, rb);
    }
    const uint16_t* as = As[st];
    const uint16_t* bs = Bs[st];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = lds_frag(as, wm * 128 + i * 32 + lrow, kk * 16 + lk);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = lds_frag(bs, wn * 64 + j * 32 + lrow, kk * 16 + lk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_a(As[st ^ 1], ra);
      store_b(Bs[st ^ 1], rb, off, s_c4, s_c8);
    }
    __syncthreads();
  }

  // LoRA term, contracted on the matrix cores in chunks of 16 over the rank:
  // forward  + u[m, :] . (s * B[n, :]),  backward + du[m, :] . A[:, n].
  if (g.lora_l != nullptr && split == 0) {
    for (int r0 = 0; r0 < g.r; r0 += 16) {
      bf16x8_t fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 128 + i * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (row < g.M && rr < g.r) ? g.lora_l[row * g.r + rr] : 0.0f;
        }
        fa[i] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 64 + j * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          float x = 0.0f;
          if (col < g.Nc && rr < g.r)
            x = BWD ? g.lora_r[(int64_t)rr * g.k_in + col] : g.scale * g.lora_r[col * g.r + rr];
          v[e] = x;
        }
        fb[j] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 tile.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + lrow;
      if (col >= g.Nc) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        if (SPLIT) {
          g.part[((int64_t)split * g.M + row) * g.Nc + col] = acc[i][j][r];
        } else {
          bf16x2_t h;
          h[0] = (__bf16)acc[i][j][r];
          g.out[row * g.Nc + col] = __builtin_bit_cast(uint32_t, h) & 0xFFFFu;
        }
      }
    }
  }
}

// Sum of the split partials in split order, rounded once to bf16.
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int splits,
                                                   int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    float4 s = *reinterpret_cast<const float4*>(part + i);
    for (int p = 1; p < splits; ++p) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)p * n + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(out + i) = o;
  } else {
    for (int64_t e = i; e < n; ++e) {
      float s = part[e];
      for (int p = 1; p < splits; ++p) s += part[(int64_t)p * n + e];
      bf16x2_t h;
      h[0] = (__bf16)s;
      out[e] = __builtin_bit_cast(uint32_t, h) & 0xFFFFu;
    }
  }
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t n_cols, int64_t k_contract) {
  GemmPlan p;
  p.bm = BM;
  p.bn = BN;
  const int64_t tiles = ((M + BM - 1) / BM) * ((n_cols + BN - 1) / BN);
  const int64_t nk = (k_contract + BK - 1) / BK;
  int splits = 1;
  // Split the contraction while the grid is short of the chip's 256 CUs and
  // each split keeps at least 8 contraction steps.
  while (tiles * splits < 192 && nk / (2 * splits) >= 8) splits *= 2;
  const int64_t steps_per = (nk + splits - 1) / splits;
  p.kc_chunk = steps_per * BK;
  p.splits = (int)((nk + steps_per - 1) / steps_per);
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)n_cols * sizeof(float) : 0;
  return p;
}

hipError_t launch_linear(bool backward, const QPtrs& q, int64_t n_out, int64_t k_in,
                         const uint16_t* a, int64_t M, uint16_t* out, const float* lora_l,
                         const float* lora_r, int r, float scale, void* ws, hipStream_t s) {
  GemmArgs g;
  g.packed = q.packed;
  g.q8 = q.q8;
  g.nested = q.nested;
  g.offset = q.offset;
  g.a = a;
  g.M = M;
  g.Kc = backward ? n_out : k_in;
  g.Nc = backward ? k_in : n_out;
  g.n_out = n_out;
  g.k_in = k_in;
  g.out = out;
  const GemmPlan p = plan_gemm(M, g.Nc, g.Kc);
  g.part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
  g.kc_chunk = p.kc_chunk;
  g.lora_l = lora_l;
  g.lora_r = lora_r;
  g.r = r;
  g.scale = scale;
  const dim3 grid((unsigned)((g.Nc + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)p.splits);
  const bool split = p.splits > 1;
  if (backward && split)
    hipLaunchKernelGGL((k_gemm<true, true>), grid, dim3(THREADS), 0, s, g, host_tables());
  else if (backward)
    hipLaunchKernelGGL((k_gemm<true, false>), grid, dim3(THREADS), 0, s, g, host_tables());
  else if (split)
    hipLaunchKernelGGL((k_gemm<false, true>), grid, dim3(THREADS), 0, s, g, host_tables());
  else
    hipLaunchKernelGGL((k_gemm<false, false>), grid, dim3(THREADS), 0, s, g, host_tables());
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = M * g.Nc;
  const dim3 g2((unsigned)((n / 4 + 1 + 255) / 256));
  hipLaunchKernelGGL(k_split_sum, g2, dim3(256), 0, s, g.part, p.splits, n, out);
  return hipGetLastError();
}

}  // namespace nf4s
