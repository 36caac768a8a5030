// Kernels of the decoder around the streamed NF4 linears: embedding gather,
// RMSNorm, rotary embedding, causal attention with grouped KV heads, SwiGLU,
// cross-entropy, AdamW and the small conversions between them.
//
// "Soup layer-streamed NF4 training measured", sections 2.1-2.2 and 4.3: a
// llama decoder (SmolLM2-135M, Llama-3.1-8B) whose layer linears are the
// streamed NF4 weights with bf16 compute, resident bf16 embeddings/lm_head,
// checkpointed layer bodies. The operations follow llama's definitions:
// RMSNorm y = x / sqrt(mean(x^2) + eps) * w; rotate-half rotary embedding with
// angle t * theta^(-2j/d) for pair (j, j + d/2) at position t of a sequence;
// softmax(q k^T / sqrt(d)) v with a causal mask and KV head h / (H / Hkv);
// SwiGLU silu(g) * u; mean token cross-entropy; AdamW with decoupled weight
// decay. Storage: bf16 for every tensor that feeds a product or the
// attention, fp32 for the residual stream, norms' statistics, softmax
// statistics and reductions; all arithmetic in fp32. Every reduction runs in a
// fixed order (no atomics), so results do not depend on timing.
#include <math.h>

#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu); }

// Sum over a 256-thread workgroup in a fixed tree; every thread gets the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
#pragma unroll
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
#pragma unroll
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] = fmaxf(red[t], red[t + s]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// h[t, :] = E[ids[t], :] (bf16 -> fp32 residual stream); an id outside
// [0, V) gives a row of NaNs instead of a read outside the table.
__global__ __launch_bounds__(256) void k_embed(const uint16_t* __restrict__ E, int64_t V,
                                               const int64_t* __restrict__ ids, int64_t H,
                                               float* __restrict__ h) {
  const int64_t t = blockIdx.x;
  const int64_t id = ids[t];
  const bool ok = id >= 0 && id < V;
  const uint16_t* row = E + (ok ? id : 0) * H;
  for (int64_t j = threadIdx.x; j < H; j += 256) h[t * H + j] = ok ? bf2f(row[j]) : __builtin_nanf("");
}

// y = bf16(x * rstd * w), rstd = 1/sqrt(mean(x^2) + eps); one workgroup per row
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const float* __restrict__ x,
                                                     const float* __restrict__ w, int64_t H,
                                                     float eps, uint16_t* __restrict__ y,
                                                     float* __restrict__ rstd) {
  __shared__ float red[256];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * H;
  float ss = 0.0f;
  for (int64_t j = threadIdx.x; j < H; j += 256) ss += xr[j] * xr[j];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (threadIdx.x == 0) rstd[t] = r;
  for (int64_t j = threadIdx.x; j < H; j += 256) y[t * H + j] = f2bf(xr[j] * r * w[j]);
}

// dh (+)= rstd * g - x * rstd^3 * mean(g * x), g = w * (sum of the n bf16 inputs)
struct DyPtrs {
  const uint16_t* p[3];
};

__global__ __launch_bounds__(256) void k_rmsnorm_bwd(DyPtrs dys, int n_dy, const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ rstd, int64_t H,
                                                     int accumulate, float* __restrict__ dh) {
  __shared__ float red[256];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * H;
  const float r = rstd[t];
  auto dy_at = [&](int64_t j) {
    float s = bf2f(dys.p[0][t * H + j]);
    if (n_dy > 1) s += bf2f(dys.p[1][t * H + j]);
    if (n_dy > 2) s += bf2f(dys.p[2][t * H + j]);
    return s;
  };
  float acc = 0.0f;
  for (int64_t j = threadIdx.x; j < H; j += 256) acc += dy_at(j) * w[j] * xr[j];
  acc = block_sum(acc, red);
  const float c = r * r * r * acc / (float)H;
  for (int64_t j = threadIdx.x; j < H; j += 256) {
    const float d = r * dy_at(j) * w[j] - xr[j] * c;
    dh[t * H + j] = accumulate ? dh[t * H + j] + d : d;
  }
}

// In-place rotary embedding of bf16 x[T, heads * d]; row t is position t % S.
__global__ __launch_bounds__(256) void k_rope(uint16_t* __restrict__ x, int64_t T, int64_t S,
                                              int heads, int d, double theta, int inverse) {
  const int64_t n = T * heads * (d / 2);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int half = d / 2;
  const int j = (int)(i % half);
  const int64_t th = i / half;  // (row, head)
  const int64_t row = th / heads;
  const int64_t pos = row % S;
  const double ang = (double)pos * pow(theta, -2.0 * j / d);
  const float c = (float)cos(ang);
  const float s = inverse ? -(float)sin(ang) : (float)sin(ang);
  uint16_t* v = x + th * d;
  const float x1 = bf2f(v[j]), x2 = bf2f(v[j + half]);
  v[j] = f2bf(x1 * c - x2 * s);
  v[j + half] = f2bf(x2 * c + x1 * s);
}

// ---- attention --------------------------------------------------------------
// A workgroup owns 64 query rows of one (sequence, head); 4 lanes per query,
// each holding d/4 of the query and of the output accumulator. Key/value
// blocks of 64 rows are staged in LDS as bf16. Online softmax in fp32.
constexpr int QB = 64;  // queries (and keys) per block
constexpr int MAXD = 128;

template <int D>
__global__ __launch_bounds__(256) void k_attn_fwd(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v, int64_t S,
                                                  int H, int Hkv, uint16_t* __restrict__ o,
                                                  float* __restrict__ o_f32,
                                                  float* __restrict__ lse) {
  constexpr int DL = D / 4;  // dims per lane
  __shared__ uint16_t Ks[QB * D];
  __shared__ uint16_t Vs[QB * D];
  const int t = threadIdx.x, qi = t >> 2, part = t & 3;
  const int64_t nqb = (S + QB - 1) / QB;
  const int64_t b = blockIdx.x / (H * nqb);
  const int h = (int)((blockIdx.x / nqb) % H);
  const int64_t qb = blockIdx.x % nqb;
  const int g = h / (H / Hkv);
  const int64_t qpos = qb * QB + qi;  // position within the sequence
  const bool qvalid = qpos < S;
  const float scale = 1.0f / sqrtf((float)D);
  float qv[DL], acc[DL];
  const int64_t qrow = b * S + (qvalid ? qpos : S - 1);
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qv[e] = bf2f(q[qrow * (int64_t)H * D + (int64_t)h * D + part * DL + e]) * scale;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int64_t kb = 0; kb <= qb; ++kb) {
    __syncthreads();
    for (int idx = t; idx < QB * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      const int64_t kpos = kb * QB + r;
      const int64_t krow = b * S + (kpos < S ? kpos : S - 1);
      Ks[idx] = k[krow * (int64_t)Hkv * D + (int64_t)g * D + c];
      Vs[idx] = v[krow * (int64_t)Hkv * D + (int64_t)g * D + c];
    }
    __syncthreads();
    const int jmax = (int)min((int64_t)QB, S - kb * QB);
    for (int j = 0; j < jmax; ++j) {
      const int64_t kpos = kb * QB + j;
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < DL; ++e) s += qv[e] * bf2f(Ks[j * D + part * DL + e]);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (kpos > qpos) continue;  // causal (uniform within a query's 4 lanes)
      if (s > m) {
        const float corr = __expf(m - s);
        l *= corr;
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[e] *= corr;
        m = s;
      }
      const float p = __expf(s - m);
      l += p;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] += p * bf2f(Vs[j * D + part * DL + e]);
    }
  }
  if (!qvalid) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    const int64_t idx = qrow * (int64_t)H * D + (int64_t)h * D + part * DL + e;
    o[idx] = f2bf(acc[e] * inv);
    if (o_f32 != nullptr) o_f32[idx] = acc[e] * inv;
  }
  if (part == 0) lse[(b * H + h) * S + qpos] = m + logf(l);
}

// Dsum[row, h] = sum_j P_ij dP_ij = dO_i . O_i with the unrounded (fp32)
// attention output; one thread per (row, head).
__global__ __launch_bounds__(256) void k_attn_dsum(const float* __restrict__ o,
                                                   const uint16_t* __restrict__ dout, int64_t T,
                                                   int H, int D, float* __restrict__ dsum) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * H) return;
  float s = 0.0f;
  for (int e = 0; e < D; ++e) s += o[i * D + e] * bf2f(dout[i * D + e]);
  dsum[i] = s;
}

// dQ for 64 query rows of one (sequence, head).
template <int D>
__global__ __launch_bounds__(256) void k_attn_dq(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v,
                                                 const uint16_t* __restrict__ dout,
                                                 const float* __restrict__ lse,
                                                 const float* __restrict__ dsum, int64_t S, int H,
                                                 int Hkv, uint16_t* __restrict__ dq) {
  constexpr int DL = D / 4;
  __shared__ uint16_t Ks[QB * D];
  __shared__ uint16_t Vs[QB * D];
  const int t = threadIdx.x, qi = t >> 2, part = t & 3;
  const int64_t nqb = (S + QB - 1) / QB;
  const int64_t b = blockIdx.x / (H * nqb);
  const int h = (int)((blockIdx.x / nqb) % H);
  const int64_t qb = blockIdx.x % nqb;
  const int g = h / (H / Hkv);
  const int64_t qpos = qb * QB + qi;
  const bool qvalid = qpos < S;
  const float scale = 1.0f / sqrtf((float)D);
  const int64_t qrow = b * S + (qvalid ? qpos : S - 1);
  float qv[DL], dov[DL], acc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    const int64_t idx = qrow * (int64_t)H * D + (int64_t)h * D + part * DL + e;
    qv[e] = bf2f(q[idx]) * scale;
    dov[e] = bf2f(dout[idx]);
    acc[e] = 0.0f;
  }
  const float L = lse[(b * H + h) * S + (qvalid ? qpos : S - 1)];
  const float Di = dsum[qrow * H + h];
  for (int64_t kb = 0; kb <= qb; ++kb) {
    __syncthreads();
    for (int idx = t; idx < QB * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      const int64_t kpos = kb * QB + r;
      const int64_t krow = b * S + (kpos < S ? kpos : S - 1);
      Ks[idx] = k[krow * (int64_t)Hkv * D + (int64_t)g * D + c];
      Vs[idx] = v[krow * (int64_t)Hkv * D + (int64_t)g * D + c];
    }
    __syncthreads();
    const int jmax = (int)min((int64_t)QB, S - kb * QB);
    for (int j = 0; j < jmax; ++j) {
      const int64_t kpos = kb * QB + j;
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        s += qv[e] * bf2f(Ks[j * D + part * DL + e]);
        dp += dov[e] * bf2f(Vs[j * D + part * DL + e]);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      if (kpos > qpos) continue;
      const float p = __expf(s - L);
      const float ds = p * (dp - Di) * scale;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] += ds * bf2f(Ks[j * D + part * DL + e]);
    }
  }
  if (!qvalid) return;
#pragma unroll
  for (int e = 0; e < DL; ++e) dq[qrow * (int64_t)H * D + (int64_t)h * D + part * DL + e] = f2bf(acc[e]);
}

// dK, dV for 64 key rows of one (sequence, KV head), summed over the heads of
// the group in head order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_dkv(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  const uint16_t* __restrict__ dout,
                                                  const float* __restrict__ lse,
                                                  const float* __restrict__ dsum, int64_t S, int H,
                                                  int Hkv, uint16_t* __restrict__ dk,
                                                  uint16_t* __restrict__ dv) {
  constexpr int DL = D / 4;
  __shared__ uint16_t Qs[QB * D];
  __shared__ uint16_t Os[QB * D];
  __shared__ float Ls[QB];
  __shared__ float Ds[QB];
  const int t = threadIdx.x, ki = t >> 2, part = t & 3;
  const int64_t nkb = (S + QB - 1) / QB;
  const int64_t b = blockIdx.x / (Hkv * nkb);
  const int g = (int)((blockIdx.x / nkb) % Hkv);
  const int64_t kb = blockIdx.x % nkb;
  const int grp = H / Hkv;
  const int64_t kpos = kb * QB + ki;
  const bool kvalid = kpos < S;
  const float scale = 1.0f / sqrtf((float)D);
  const int64_t krow = b * S + (kvalid ? kpos : S - 1);
  float kv_[DL], vv[DL], dka[DL], dva[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    const int64_t idx = krow * (int64_t)Hkv * D + (int64_t)g * D + part * DL + e;
    kv_[e] = bf2f(k[idx]);
    vv[e] = bf2f(v[idx]);
    dka[e] = 0.0f;
    dva[e] = 0.0f;
  }
  for (int hh = 0; hh < grp; ++hh) {
    const int h = g * grp + hh;
    for (int64_t qb = kb; qb < nkb; ++qb) {
      __syncthreads();
      for (int idx = t; idx < QB * D; idx += 256) {
        const int r = idx / D, c = idx % D;
        const int64_t qp = qb * QB + r;
        const int64_t qrow = b * S + (qp < S ? qp : S - 1);
        Qs[idx] = q[qrow * (int64_t)H * D + (int64_t)h * D + c];
        Os[idx] = dout[qrow * (int64_t)H * D + (int64_t)h * D + c];
      }
      if (t < QB) {
        const int64_t qp = qb * QB + t;
        const int64_t qc = qp < S ? qp : S - 1;
        Ls[t] = lse[(b * H + h) * S + qc];
        Ds[t] = dsum[(b * S + qc) * H + h];
      }
      __syncthreads();
      const int imax = (int)min((int64_t)QB, S - qb * QB);
      for (int i = 0; i < imax; ++i) {
        const int64_t qp = qb * QB + i;
        float s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
          s += bf2f(Qs[i * D + part * DL + e]) * kv_[e];
          dp += bf2f(Os[i * D + part * DL + e]) * vv[e];
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dp += __shfl_xor(dp, 1);
        dp += __shfl_xor(dp, 2);
        if (qp < kpos) continue;
        const float p = __expf(s * scale - Ls[i]);
        const float ds = p * (dp - Ds[i]) * scale;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
          dva[e] += p * bf2f(Os[i * D + part * DL + e]);
          dka[e] += ds * bf2f(Qs[i * D + part * DL + e]);
        }
      }
    }
  }
  if (!kvalid) return;
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    const int64_t idx = krow * (int64_t)Hkv * D + (int64_t)g * D + part * DL + e;
    dk[idx] = f2bf(dka[e]);
    dv[idx] = f2bf(dva[e]);
  }
}

// ---- elementwise ------------------------------------------------------------
__global__ __launch_bounds__(256) void k_swiglu_fwd(const uint16_t* __restrict__ g,
                                                    const uint16_t* __restrict__ u, int64_t n,
                                                    uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gv = bf2f(g[i]);
  out[i] = f2bf(gv / (1.0f + __expf(-gv)) * bf2f(u[i]));
}

__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t* __restrict__ ds,
                                                    const uint16_t* __restrict__ g,
                                                    const uint16_t* __restrict__ u, int64_t n,
                                                    uint16_t* __restrict__ dg,
                                                    uint16_t* __restrict__ du) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gv = bf2f(g[i]), uv = bf2f(u[i]), d = bf2f(ds[i]);
  const float sg = 1.0f / (1.0f + __expf(-gv));
  dg[i] = f2bf(d * uv * (sg * (1.0f + gv * (1.0f - sg))));
  du[i] = f2bf(d * gv * sg);
}

// out = h + y (fp32 residual stream plus a bf16 branch output); out may be h
__global__ __launch_bounds__(256) void k_residual_add(const float* h, const uint16_t* __restrict__ y,
                                                      int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = h[i] + bf2f(y[i]);
}

__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* __restrict__ x, int64_t n,
                                                     uint16_t* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = f2bf(x[i]);
}

// Cross-entropy of one row of bf16 logits: row loss and bf16 gradient
// (softmax - onehot) / T. A target outside [0, V) makes the row loss NaN.
__global__ __launch_bounds__(256) void k_ce_rows(const uint16_t* __restrict__ logits,
                                                 const int64_t* __restrict__ targets, int64_t T,
                                                 int64_t V, float* __restrict__ row_loss,
                                                 uint16_t* __restrict__ dlogits) {
  __shared__ float red[256];
  const int64_t t = blockIdx.x;
  const uint16_t* z = logits + t * V;
  float m = -INFINITY;
  for (int64_t j = threadIdx.x; j < V; j += 256) m = fmaxf(m, bf2f(z[j]));
  m = block_max(m, red);
  float s = 0.0f;
  for (int64_t j = threadIdx.x; j < V; j += 256) s += expf(bf2f(z[j]) - m);
  s = block_sum(s, red);
  const float lse = m + logf(s);
  const int64_t tg = targets[t];
  const bool ok = tg >= 0 && tg < V;
  if (threadIdx.x == 0) row_loss[t] = ok ? lse - bf2f(z[tg]) : __builtin_nanf("");
  const float invT = 1.0f / (float)T;
  for (int64_t j = threadIdx.x; j < V; j += 256) {
    float p = expf(bf2f(z[j]) - lse);
    if (j == tg) p -= 1.0f;
    dlogits[t * V + j] = f2bf(p * invT);
  }
}

// loss = mean of the row losses, summed in a fixed order by one workgroup
__global__ __launch_bounds__(256) void k_mean(const float* __restrict__ x, int64_t n,
                                              float* __restrict__ out) {
  __shared__ float red[256];
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += x[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) out[0] = s / (float)n;
}

__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ p, const float* __restrict__ g,
                                               float* __restrict__ m, float* __restrict__ v,
                                               int64_t n, float lr, float b1, float b2, float eps,
                                               float wd, float bc1, float bc2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gi = g[i];
  const float mi = b1 * m[i] + (1.0f - b1) * gi;
  const float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
  m[i] = mi;
  v[i] = vi;
  const float mhat = mi / bc1, vhat = vi / bc2;
  p[i] = p[i] * (1.0f - lr * wd) - lr * mhat / (sqrtf(vhat) + eps);
}

inline unsigned grid_of(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_embed(const uint16_t* E, int64_t V, const int64_t* ids, int64_t T, int64_t H,
                        float* h, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3((unsigned)T), dim3(256), 0, s, E, V, ids, H, h);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_fwd(const float* x, const float* w, int64_t T, int64_t H, float eps,
                              uint16_t* y, float* rstd, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm_fwd, dim3((unsigned)T), dim3(256), 0, s, x, w, H, eps, y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* const* dys, int n_dy, const float* x, const float* w,
                              const float* rstd, int64_t T, int64_t H, int accumulate, float* dh,
                              hipStream_t s) {
  DyPtrs d{{dys[0], n_dy > 1 ? dys[1] : nullptr, n_dy > 2 ? dys[2] : nullptr}};
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3((unsigned)T), dim3(256), 0, s, d, n_dy, x, w, rstd, H,
                     accumulate, dh);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* x, int64_t T, int64_t S, int heads, int d, double theta,
                       int inverse, hipStream_t s) {
  hipLaunchKernelGGL(k_rope, dim3(grid_of(T * heads * (d / 2))), dim3(256), 0, s, x, T, S, heads, d,
                     theta, inverse);
  return hipGetLastError();
}

#define NF4S_DISPATCH_D(D_, CALL) \
  switch (D_) {                   \
    case 16: CALL(16); break;     \
    case 32: CALL(32); break;     \
    case 64: CALL(64); break;     \
    case 128: CALL(128); break;   \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                int64_t S, int H, int Hkv, int D, uint16_t* o, float* o_f32,
                                float* lse, hipStream_t s) {
  const unsigned grid = (unsigned)(B * H * ((S + QB - 1) / QB));
#define CALL(DD) hipLaunchKernelGGL(k_attn_fwd<DD>, dim3(grid), dim3(256), 0, s, q, k, v, S, H, Hkv, o, o_f32, lse)
  NF4S_DISPATCH_D(D, CALL)
#undef CALL
  return hipGetLastError();
}

size_t attention_bwd_ws_bytes(int64_t B, int64_t S, int H) { return (size_t)(B * S * H) * sizeof(float); }

hipError_t launch_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* o_f32, const uint16_t* dout, const float* lse,
                                int64_t B, int64_t S, int H, int Hkv, int D, uint16_t* dq,
                                uint16_t* dk, uint16_t* dv, void* ws, hipStream_t s) {
  float* dsum = static_cast<float*>(ws);
  hipLaunchKernelGGL(k_attn_dsum, dim3(grid_of(B * S * H)), dim3(256), 0, s, o_f32, dout, B * S, H,
                     D, dsum);
  const unsigned gq = (unsigned)(B * H * ((S + QB - 1) / QB));
  const unsigned gk = (unsigned)(B * Hkv * ((S + QB - 1) / QB));
#define CALL(DD)                                                                                   \
  hipLaunchKernelGGL(k_attn_dq<DD>, dim3(gq), dim3(256), 0, s, q, k, v, dout, lse, dsum, S, H, Hkv, dq); \
  hipLaunchKernelGGL(k_attn_dkv<DD>, dim3(gk), dim3(256), 0, s, q, k, v, dout, lse, dsum, S, H, Hkv, dk, dv)
  NF4S_DISPATCH_D(D, CALL)
#undef CALL
  return hipGetLastError();
}
#undef NF4S_DISPATCH_D

hipError_t launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_swiglu_fwd, dim3(grid_of(n)), dim3(256), 0, s, g, u, n, out);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* ds, const uint16_t* g, const uint16_t* u, int64_t n,
                             uint16_t* dg, uint16_t* du, hipStream_t s) {
  hipLaunchKernelGGL(k_swiglu_bwd, dim3(grid_of(n)), dim3(256), 0, s, ds, g, u, n, dg, du);
  return hipGetLastError();
}

hipError_t launch_residual_add(const float* h, const uint16_t* y, int64_t n, float* out,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_residual_add, dim3(grid_of(n)), dim3(256), 0, s, h, y, n, out);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* x, int64_t n, uint16_t* y, hipStream_t s) {
  hipLaunchKernelGGL(k_f32_to_bf16, dim3(grid_of(n)), dim3(256), 0, s, x, n, y);
  return hipGetLastError();
}

size_t cross_entropy_ws_bytes(int64_t T) { return (size_t)T * sizeof(float); }

hipError_t launch_cross_entropy(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                                float* loss, uint16_t* dlogits, void* ws, hipStream_t s) {
  float* rows = static_cast<float*>(ws);
  hipLaunchKernelGGL(k_ce_rows, dim3((unsigned)T), dim3(256), 0, s, logits, targets, T, V, rows, dlogits);
  hipLaunchKernelGGL(k_mean, dim3(1), dim3(256), 0, s, rows, T, loss);
  return hipGetLastError();
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float b1,
                        float b2, float eps, float wd, int64_t step, hipStream_t s) {
  const float bc1 = (float)(1.0 - pow((double)b1, (double)step));
  const float bc2 = (float)(1.0 - pow((double)b2, (double)step));
  hipLaunchKernelGGL(k_adamw, dim3(grid_of(n)), dim3(256), 0, s, p, g, m, v, n, lr, b1, b2, eps, wd,
                     bc1, bc2);
  return hipGetLastError();
}

}  // namespace nf4s
