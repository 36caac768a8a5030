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

#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu); }

// Sum over a 256-thread workgroup in a fixed order (butterfly within each
// wave, then the four wave sums in wave order); every thread gets the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();  // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Eight consecutive bf16 values (16 bytes) as fp32.
__device__ __forceinline__ void load8_bf16(const uint16_t* p, float* f) {
  const u32x4v u = *reinterpret_cast<const u32x4v*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void store8_bf16(uint16_t* p, const float* f) {
  u32x4v u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  *reinterpret_cast<u32x4v*>(p) = u;
}

__device__ __forceinline__ void load8_f32(const float* p, float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ void store8_f32(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
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

// y = bf16(x * rstd * w), rstd = 1/sqrt(mean(x^2) + eps); one workgroup per
// row, 8 elements (16- and 32-byte accesses) per thread and step.
// packed (nullable): y also in MFMA fragment order (K = H), for the GEMMs
// One workgroup per row. Workgroups are dealt to the 8 XCDs round-robin by
// id; xcd_row gives each XCD a contiguous range of rows, so that rows that
// share the 64-byte segments of a fragment-order copy (4 consecutive rows)
// are written through one L2. Launch xcd_rows(T) workgroups.
__device__ __forceinline__ int64_t xcd_row(int64_t b, int64_t T) {
  const int64_t rpx = (T + 7) / 8;
  return (b % 8) * rpx + b / 8;
}
inline unsigned xcd_rows(int64_t T) { return (unsigned)(8 * ((T + 7) / 8)); }

__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const float* __restrict__ x,
                                                     const float* __restrict__ w, int64_t H,
                                                     float eps, uint16_t* __restrict__ y,
                                                     float* __restrict__ rstd,
                                                     uint8_t* __restrict__ packed, int64_t T) {
  __shared__ float red[4];
  const int64_t t = xcd_row(blockIdx.x, T);
  if (t >= T) return;  // uniform per workgroup
  const float* xr = x + t * H;
  const int nc = (int)(H / 8);
  float ss = 0.0f;
  for (int c = threadIdx.x; c < nc; c += 256) {
    float f[8];
    load8_f32(xr + 8 * c, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (threadIdx.x == 0) rstd[t] = r;
  for (int c = threadIdx.x; c < nc; c += 256) {
    float f[8], g[8];
    load8_f32(xr + 8 * c, f);
    load8_f32(w + 8 * c, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f[e] * r * g[e];
    u32x4v o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    *reinterpret_cast<u32x4v*>(y + t * H + 8 * c) = o;
    if (packed) {
      const int64_t kb = (H + 63) / 64 * 4;
      *reinterpret_cast<u32x4v*>(packed + frag_offset(t, 8 * c, kb)) = o;
      if (c == nc - 1) frag_zero_tail(packed, t, H, kb);
    }
  }
}

// chunks of 8 of the row a thread of the norm backward keeps in registers
// between its two passes (rows up to 8192 wide are read once)
constexpr int RC = 4;

// dh (+)= rstd * g - x * rstd^3 * mean(g * x), g = w * (sum of the n bf16 inputs)
struct DyPtrs {
  const uint16_t* p[3];
};

__device__ __forceinline__ void dy_sum8(const DyPtrs& dys, int n_dy, int64_t off, float* f) {
  load8_bf16(dys.p[0] + off, f);
  for (int i = 1; i < n_dy; ++i) {
    float u[8];
    load8_bf16(dys.p[i] + off, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] += u[e];
  }
}

// y, packed (nullable): the resulting dh row also as bf16, row-major and in
// MFMA fragment order (the next GEMM's input), as k_f32_to_bf16 writes them.
// The first RC chunks of the summed dy and of x stay in registers for the
// second pass.
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(DyPtrs dys, int n_dy, const float* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ rstd, int64_t H,
                                                     int accumulate, float* __restrict__ dh,
                                                     uint16_t* __restrict__ y,
                                                     uint8_t* __restrict__ packed, int64_t T) {
  __shared__ float red[4];
  const int64_t t = xcd_row(blockIdx.x, T);
  if (t >= T) return;  // uniform per workgroup
  const float* xr = x + t * H;
  const float r = rstd[t];
  const int nc = (int)(H / 8);
  float acc = 0.0f, dyc[RC][8], xc[RC][8];
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nc) {
      float g[8];
      dy_sum8(dys, n_dy, t * H + 8 * c, dyc[i]);
      load8_f32(xr + 8 * c, xc[i]);
      load8_f32(w + 8 * c, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += dyc[i][e] * g[e] * xc[i][e];
    }
  }
  for (int c = threadIdx.x + 256 * RC; c < nc; c += 256) {
    float dy[8], f[8], g[8];
    dy_sum8(dys, n_dy, t * H + 8 * c, dy);
    load8_f32(xr + 8 * c, f);
    load8_f32(w + 8 * c, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += dy[e] * g[e] * f[e];
  }
  acc = block_sum(acc, red);
  const float cc = r * r * r * acc / (float)H;
  auto emit = [&](int c, const float* dy, const float* f) {
    float g[8], o[8];
    load8_f32(w + 8 * c, g);
    if (accumulate) load8_f32(dh + t * H + 8 * c, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = r * dy[e] * g[e] - f[e] * cc;
      o[e] = accumulate ? o[e] + d : d;
    }
    store8_f32(dh + t * H + 8 * c, o);
    if (y) {
      u32x4v b;
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
      *reinterpret_cast<u32x4v*>(y + t * H + 8 * c) = b;
      if (packed) {
        const int64_t kb = (H + 63) / 64 * 4;
        *reinterpret_cast<u32x4v*>(packed + frag_offset(t, 8 * c, kb)) = b;
        if (c == nc - 1) frag_zero_tail(packed, t, H, kb);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nc) emit(c, dyc[i], xc[i]);
  }
  for (int c = threadIdx.x + 256 * RC; c < nc; c += 256) {
    float dy[8], f[8];
    dy_sum8(dys, n_dy, t * H + 8 * c, dy);
    load8_f32(xr + 8 * c, f);
    emit(c, dy, f);
  }
}

// In-place rotary embedding of bf16 x[T, heads * d]; row t is position t % S.
// inv[j] = theta^(-2j/d) (computed on the host in fp64); the angle and its
// sine and cosine are fp64, the rotation fp32.
struct InvFreq {
  double f[128];
};

// One workgroup per row t and both tensors (queries and keys; none second
// when x2 is null): the d/2 cosines and sines of position t % S are computed
// once into LDS (fp64, rounded to fp32), then every head is rotated, four
// pairs per thread and item. p1 / p2 (nullable): the rotated rows also in
// MFMA fragment order (K = heads * d), as the GEMMs that read them next take
// them (k_frag_pack's layout, the columns past K up to a multiple of 64 zero).
// One workgroup per row, rows dealt to XCDs by xcd_row. A thread rotates G
// consecutive columns of each half of a head: G = 8 where the half is a
// multiple of 8 and the rows are 16-byte aligned (one fragment slot per
// packed store), else G = 4.
template <int G>
__global__ __launch_bounds__(256) void k_rope_rows(uint16_t* __restrict__ x1, int heads1,
                                                   uint8_t* __restrict__ p1, uint16_t* __restrict__ x2,
                                                   int heads2, uint8_t* __restrict__ p2, int64_t T,
                                                   int64_t S, int d, InvFreq inv, int inverse) {
  using V = typename std::conditional<G == 8, u32x4v, uint2>::type;
  __shared__ float2 cs[128];
  const int64_t t = xcd_row(blockIdx.x, T);
  if (t >= T) return;  // uniform per workgroup
  const int half = d / 2, qg = half / G;
  for (int j = threadIdx.x; j < half; j += 256) {
    double sd, cd;
    sincos((double)(t % S) * inv.f[j], &sd, &cd);
    cs[j] = make_float2((float)cd, inverse ? -(float)sd : (float)sd);
  }
  __syncthreads();
  const int n1 = heads1 * qg, n = n1 + (x2 ? heads2 * qg : 0);
  for (int i = threadIdx.x; i < n; i += 256) {
    const bool second = i >= n1;
    const int ii = second ? i - n1 : i;
    uint16_t* const x = second ? x2 : x1;
    uint8_t* const p = second ? p2 : p1;
    const int heads = second ? heads2 : heads1;
    const int h = ii / qg, j0 = G * (ii % qg);
    const int64_t K = (int64_t)heads * d;
    uint16_t* const v = x + t * K + (int64_t)h * d;
    const V a = *reinterpret_cast<const V*>(v + j0);
    const V b = *reinterpret_cast<const V*>(v + j0 + half);
    const uint32_t* const aw = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* const bw = reinterpret_cast<const uint32_t*>(&b);
    float o1[G], o2[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const float c = cs[j0 + e].x, sn = cs[j0 + e].y;
      const uint32_t wa = aw[e >> 1], wb = bw[e >> 1];
      const float x1v = __uint_as_float((e & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
      const float x2v = __uint_as_float((e & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
      o1[e] = x1v * c - x2v * sn;
      o2[e] = x2v * c + x1v * sn;
    }
    V ra, rb;
    uint32_t* const raw = reinterpret_cast<uint32_t*>(&ra);
    uint32_t* const rbw = reinterpret_cast<uint32_t*>(&rb);
#pragma unroll
    for (int e = 0; e < G / 2; ++e) {
      raw[e] = pack_bf16x2(o1[2 * e], o1[2 * e + 1]);
      rbw[e] = pack_bf16x2(o2[2 * e], o2[2 * e + 1]);
    }
    *reinterpret_cast<V*>(v + j0) = ra;
    *reinterpret_cast<V*>(v + j0 + half) = rb;
    if (p) {  // G consecutive columns inside one fragment slot of 8
      const int64_t kb = (K + 63) / 64 * 4;
      const int64_t c1 = (int64_t)h * d + j0, c2 = c1 + half;
      *reinterpret_cast<V*>(p + frag_offset(t, c1 & ~7ll, kb) + (c1 & 7) * 2) = ra;
      *reinterpret_cast<V*>(p + frag_offset(t, c2 & ~7ll, kb) + (c2 & 7) * 2) = rb;
    }
  }
  if (threadIdx.x == 0) {
    if (p1) frag_zero_tail(p1, t, (int64_t)heads1 * d, ((int64_t)heads1 * d + 63) / 64 * 4);
    if (x2 && p2) frag_zero_tail(p2, t, (int64_t)heads2 * d, ((int64_t)heads2 * d + 63) / 64 * 4);
  }
}

// ---- attention on the matrix cores -------------------------------------------
// One wave per 32-row block of one (sequence, head), v_mfma_f32_32x32x16_bf16.
// Operand layouts of that instruction: lane l supplies row (A) or column (B)
// l%32 and the 8 contraction values 8*(l/32) .. +8 of a 16-wide step; result
// register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
//
// The query-side kernels compute the transposed products S^T = K . Q^T and
// O^T = V^T . P^T (dQ^T = K^T . dS^T), so that lane l owns query l%32: the
// softmax statistics and the rescaling of the output stay in the lane, and
// the row reductions are in-register plus one exchange between the two
// half-waves. The key-side kernel computes S = Q . K^T and dV^T = dO^T . P,
// dK^T = Q^T . dS with lane l owning key l%32.
//
// The probabilities (and dS) feed the next product without moving: its
// contraction index is taken in the order the score registers hold it --
// step kk, lane half hf, slot e <-> position 16kk + 8(e/4) + 4hf + e%4 of the
// 32-block -- and the other operand is read in that same order from the
// row-major LDS tile of its block, transposed by the LDS transpose read (two
// reads of four consecutive positions; no transposed copy). P and dS
// enter the matrix cores as a bf16 high part plus a bf16 low part (about 16
// significant bits), K, Q, V and dO are bf16 already, and accumulation is
// fp32, so the attention arithmetic keeps fp32-level accuracy.
constexpr int AB = 32;  // rows per block (queries or keys)

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.0f;
  return z;
}

// Eight fp32 values as bf16 high and low parts (hi + lo carries ~16 bits).
__device__ __forceinline__ void split8(const float* x, bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hp = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xFFFF0000u);
    h[i] = hp;
    l[i] = pack_bf16x2(x[2 * i] - h0, x[2 * i + 1] - h1);
  }
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}

// Row offset of result register r in its 32x32 tile for lane half hf.
__device__ __forceinline__ int crow(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// A 32-row block of a [rows, ld] bf16 matrix (rows r0 .. r0 + 31 of one
// sequence, clamped to it; columns c0 .. c0 + D) in the registers of one wave:
// item it = lane + 64 x covers rows 4(it / (D/8)) .. +4 and columns 8(it % (D/8))
// .. +8, as four 16-byte loads. The forward loads each block one step ahead
// of its use, hiding the memory latency behind the current block's products;
// the backward kernels load just before use and leave the latency to the
// second workgroup on their CU.
template <int D>
struct BlockRegs {
  static constexpr int ITEMS = 8 * (D / 8);           // 4-row x 8-column items per block
  static constexpr int PER_LANE = (ITEMS + 63) / 64;
  u32x4_t v[PER_LANE][4];
};

// The rows of one sequence of a [rows, ld] bf16 matrix, columns c0 .. c0 + D,
// read through a buffer resource with 32-bit byte offsets (a sequence of the
// attention calls holds fewer than 2^30 bytes); rows past the sequence are
// clamped to its last one.
template <int D>
struct SeqRows {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t ld2;   // bytes per row
  uint32_t last;  // byte offset of the sequence's last row
};

template <int D>
__device__ __forceinline__ SeqRows<D> seq_rows(const uint16_t* __restrict__ src, int64_t ld, int64_t c0,
                                               int64_t base_row, int64_t S) {
  SeqRows<D> sr;
  sr.rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + base_row * ld + c0), (short)0, (int)0xFFFFFFFFu,
                                            0x00020000);
  sr.ld2 = (uint32_t)ld * 2u;
  sr.last = (uint32_t)(S - 1) * sr.ld2;
  return sr;
}

// A lane's byte offsets inside a block of rows of ld2 bytes: load (x, i) is
// row 4(it / (D/8)) + i, column 8(it % (D/8)) of item it = lane + 64 x; the
// same for every block and for every matrix of that row length.
template <int D>
struct BlockLanes {
  uint32_t off[BlockRegs<D>::PER_LANE][4];
  uint32_t col[BlockRegs<D>::PER_LANE];
};

template <int D>
__device__ __forceinline__ BlockLanes<D> block_lanes(uint32_t ld2, int lane) {
  constexpr int CH = D / 8;
  BlockLanes<D> bl;
#pragma unroll
  for (int x = 0; x < BlockRegs<D>::PER_LANE; ++x) {
    const int it = lane + 64 * x;
    bl.col[x] = (uint32_t)(16 * (it % CH));
#pragma unroll
    for (int i = 0; i < 4; ++i) bl.off[x][i] = (uint32_t)(4 * (it / CH) + i) * ld2 + bl.col[x];
  }
  return bl;
}

// Rows r0 .. r0 + 31 of the sequence into the registers of one wave: the
// block's byte offset as the scalar offset of every load, except for a block
// that runs past the sequence, whose rows are clamped one by one.
template <int D>
__device__ __forceinline__ void load_block(const SeqRows<D>& sr, const BlockLanes<D>& bl, int r0, int S,
                                           BlockRegs<D>& br, int lane) {
  const uint32_t base = (uint32_t)r0 * sr.ld2;
  if (r0 + AB <= S) {  // uniform
#pragma unroll
    for (int x = 0; x < BlockRegs<D>::PER_LANE; ++x)
      if (lane + 64 * x < BlockRegs<D>::ITEMS)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          br.v[x][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr.rs, bl.off[x][i], (int)base, 0));
  } else {
#pragma unroll
    for (int x = 0; x < BlockRegs<D>::PER_LANE; ++x)
      if (lane + 64 * x < BlockRegs<D>::ITEMS)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t ro = base + bl.off[x][i] - bl.col[x];
          const uint32_t off = (ro < sr.last ? ro : sr.last) + bl.col[x];
          br.v[x][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr.rs, off, 0, 0));
        }
  }
}

// Zero that the compiler cannot see through: added to the offset of a load
// inside a loop, it keeps the compiler from hoisting a loop-invariant load
// (and then spilling its registers) where the loop re-reads on purpose.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// Row `row` (clamped to the sequence) as the lane's operand fragments, the
// 16-wide steps of the head dimension (half hf of each).
template <int D>
__device__ __forceinline__ void row_frags(const SeqRows<D>& sr, int row, int hf, bf16x8_t* f,
                                          uint32_t extra = 0) {
  const uint32_t ro = (uint32_t)row * sr.ld2;
  const uint32_t off = (ro < sr.last ? ro : sr.last) + 16u * (uint32_t)hf + extra;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    f[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(sr.rs, off + 32u * kk, 0, 0));
}

// The block into LDS, row-major with row stride RS: 16-byte stores.
template <int D, int RS = D + 8>
__device__ __forceinline__ void store_block(const BlockRegs<D>& br, uint16_t* rm, int lane) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int x = 0; x < BlockRegs<D>::PER_LANE; ++x) {
    const int it = lane + 64 * x;
    if (it < BlockRegs<D>::ITEMS) {
      const int rg = it / CH, ch = it % CH;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_t*>(rm + (4 * rg + i) * RS + 8 * ch) = br.v[x][i];
    }
  }
}

// A operand from a row-major LDS tile: row l%32, contraction values
// 16kk + 8*(l/32) .. +8.
template <int D>
__device__ __forceinline__ bf16x8_t frag_rm(const uint16_t* rm, int c, int hf, int kk) {
  return *reinterpret_cast<const bf16x8_t*>(rm + c * (D + 8) + 16 * kk + 8 * hf);
}

// A operand of the transposed products (row d = col0 + l%32, contraction
// positions in the score-register order of step kk), read straight from a
// row-major LDS tile (row = position, RS bf16 per row) with the LDS transpose
// read ds_read_b64_tr_b16: within each group of 16 lanes, lane s gives the
// address of 4 consecutive columns 4(s%4) .. of row s/4 and receives column s
// of those 4 rows (element e from the lane that addressed row e). Lane l
// thus gets column col0 + l%32 at positions 16kk + 4(l/32) + 0..3 and, from a
// second read, + 8 .. + 11. RS = D + 16 puts 8 consecutive rows on disjoint
// 8-bank spans (conflict-free); tiles that are also read row by row keep
// D + 8, which is conflict-free for those reads.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

template <int RS>
__device__ __forceinline__ bf16x8_t frag_trr(const uint16_t* rm, int col0, int lane, int kk) {
  const int grp = lane >> 4, s = lane & 15;
  const int row = 16 * kk + 4 * (grp >> 1) + (s >> 2);
  const int col = col0 + 16 * (grp & 1) + 4 * (s & 3);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(rm + row * RS + col));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(rm + (row + 8) * RS + col));
  u32x4_t u;
  u[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  u[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  u[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  u[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

// Operand with lane l = row l%32 of a global bf16 matrix (a query or key row),
// the 16-wide contraction steps of the head dimension.
template <int D>
__device__ __forceinline__ void row_frags(const uint16_t* __restrict__ rowp, int hf, bf16x8_t* f) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) f[kk] = *reinterpret_cast<const bf16x8_t*>(rowp + 16 * kk + 8 * hf);
}

// Work split: a workgroup of AW waves owns one 32-row block; wave w walks the
// other side's blocks w, w + AW, ... of the causal range with its own LDS
// tiles (no workgroup barrier inside the walk), and the waves' partial results
// are combined through LDS in wave order at the end.
constexpr int AW = 4;
constexpr int RM_ELEMS(int D) { return AB * (D + 8); }
constexpr int RV_ELEMS(int D) { return AB * (D + 16); }  // a tile read only transposed

// Per-lane partial results of the AW waves go through LDS lane-major:
// part[((w * 64 + lane) * NV) + i].
template <int NV>
__device__ __forceinline__ void park(float* part, int wave, int lane, const float* v) {
#pragma unroll
  for (int i = 0; i < NV; i += 4)
    *reinterpret_cast<float4*>(part + (wave * 64 + lane) * NV + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
}

template <int D>
__global__ __launch_bounds__(64 * AW, 2) void k_attn_fwd(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int64_t S,
                                                         int H, int Hkv, uint16_t* __restrict__ o,
                                                         float* __restrict__ o_f32,
                                                         float* __restrict__ lse,
                                                         uint8_t* __restrict__ packed) {
  constexpr int KS = D / 16, DT = D / 32, WS = RM_ELEMS(D) + RV_ELEMS(D);
  constexpr int STAGE = AW * 64 * (DT * 16 + 2) * 2;  // the waves' partial results (bf16 units)
  __shared__ __attribute__((aligned(16))) uint16_t smem[AW * WS > STAGE ? AW * WS : STAGE];
  const int t = threadIdx.x, lane = t & 63, hf = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: the walk over blocks is scalar
  uint16_t* const Ks = smem + wave * WS;
  uint16_t* const Vs = Ks + RM_ELEMS(D);
  const int64_t nqb = (S + AB - 1) / AB;
  // the longest causal ranges (the last query blocks) are dispatched first
  const int64_t nbh = gridDim.x / nqb;  // sequences x heads
  const int64_t qb = nqb - 1 - blockIdx.x / nbh;
  const int64_t b = (blockIdx.x % nbh) / H;
  const int h = (int)(blockIdx.x % nbh % H);
  const int g = h / (H / Hkv);
  const int64_t ldq = (int64_t)H * D, ldk = (int64_t)Hkv * D;
  const int64_t qpos = qb * AB + c;
  const int64_t qrow = b * S + (qpos < S ? qpos : S - 1);
  const float scale = 1.0f / sqrtf((float)D);
  bf16x8_t qf[KS];
  row_frags<D>(seq_rows<D>(q, ldq, (int64_t)h * D, b * S, S), (int)qpos, hf, qf);
  float acc[DT][16];
#pragma unroll
  for (int j = 0; j < DT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f;
  BlockRegs<D> rk, rv;
  const SeqRows<D> sk = seq_rows<D>(k, ldk, (int64_t)g * D, b * S, S);
  const SeqRows<D> sv = seq_rows<D>(v, ldk, (int64_t)g * D, b * S, S);
  const BlockLanes<D> bl = block_lanes<D>(sk.ld2, lane);
  const int qp = (int)qpos, S32 = (int)S;
  if (wave <= qb) {
    load_block<D>(sk, bl, wave * AB, S32, rk, lane);
    load_block<D>(sv, bl, wave * AB, S32, rv, lane);
  }
  for (int kb = wave; kb <= (int)qb; kb += AW) {
    store_block<D>(rk, Ks, lane);
    store_block<D, D + 16>(rv, Vs, lane);
    if (kb + AW <= qb) {
      load_block<D>(sk, bl, (kb + AW) * AB, S32, rk, lane);
      load_block<D>(sv, bl, (kb + AW) * AB, S32, rv, lane);
    }
    f32x16_t st = zero16();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) st = mfma32(frag_rm<D>(Ks, c, hf, kk), qf[kk], st);
    float mt = -INFINITY;
    if (kb < qb && (kb + 1) * AB <= S32) {  // every key of the block precedes every query
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] *= scale;
        mt = fmaxf(mt, st[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * AB + crow(r, hf);
        st[r] = (key <= qp && key < S32) ? st[r] * scale : -INFINITY;
        mt = fmaxf(mt, st[r]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);  // finite: key kb*32 <= qpos and < S
    const float corr = __expf(m - mn);
    float p[16], ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __expf(st[r] - mn);
      ps += p[r];
    }
    ps += __shfl_xor(ps, 32);
    lsum = lsum * corr + ps;
    m = mn;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t ph, pl;
      split8(p + 8 * kk, ph, pl);
#pragma unroll
      for (int j = 0; j < DT; ++j) {
        f32x16_t a;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = kk == 0 ? acc[j][r] * corr : acc[j][r];
        const bf16x8_t va = frag_trr<D + 16>(Vs, 32 * j, lane, kk);
        a = mfma32(va, ph, a);
        a = mfma32(va, pl, a);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = a[r];
      }
    }
  }
  // combine the waves: O = sum_w O_w e^(m_w - m) / sum_w l_w e^(m_w - m)
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);          // [AW][64][DT * 16]
  float* ml = part + AW * 64 * DT * 16;                  // [AW][64][2]
  park<DT * 16>(part, wave, lane, &acc[0][0]);
  ml[(wave * 64 + lane) * 2] = m;
  ml[(wave * 64 + lane) * 2 + 1] = lsum;
  __syncthreads();
  if (wave >= DT) return;  // wave w combines output tile j = w
  float mw[AW], mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < AW; ++w) {
    mw[w] = ml[(w * 64 + lane) * 2];
    mx = fmaxf(mx, mw[w]);
  }
  float ltot = 0.0f, f[AW];
#pragma unroll
  for (int w = 0; w < AW; ++w) {
    f[w] = __expf(mw[w] - mx);
    ltot += ml[(w * 64 + lane) * 2 + 1] * f[w];
  }
  if (qpos >= S) return;
  const int j = wave;
  const float inv = 1.0f / ltot;
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) {
    float4 fo;
    float* fv = &fo.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sacc = 0.0f;
#pragma unroll
      for (int w = 0; w < AW; ++w) sacc += part[(w * 64 + lane) * DT * 16 + j * 16 + 4 * rq + e] * f[w];
      fv[e] = sacc * inv;
    }
    const int d0 = 32 * j + 8 * rq + 4 * hf;
    const int64_t idx = qrow * ldq + (int64_t)h * D + d0;
    uint2 wv;
    wv.x = pack_bf16x2(fo.x, fo.y);
    wv.y = pack_bf16x2(fo.z, fo.w);
    *reinterpret_cast<uint2*>(o + idx) = wv;
    if (o_f32 != nullptr) *reinterpret_cast<float4*>(o_f32 + idx) = fo;
    // the o projection's input in fragment order: the two half-waves write
    // the two 8-byte halves of a row's 16-byte chunk, the 32 rows of a query
    // block 512 consecutive bytes
    if (packed != nullptr)
      *reinterpret_cast<uint2*>(packed + frag_offset(qrow, (int64_t)h * D + d0, (ldq + 63) / 64 * 4) +
                                8 * hf) = wv;
  }
  if (packed != nullptr && ldq % 64 != 0 && h == H - 1 && j == 0 && hf == 0)
    frag_zero_tail(packed, qrow, ldq, (ldq + 63) / 64 * 4);
  if (j == 0 && hf == 0) lse[(b * H + h) * S + qpos] = mx + logf(ltot);
}

// dQ of a 32-query block of one head (the key blocks split over AW waves,
// the partial dQ summed in wave order); also writes Dsum = dO . O (fp32) of
// its queries for the key-side kernel.
template <int D>
__global__ __launch_bounds__(64 * AW, 2) void k_attn_dq(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const float* __restrict__ o_f32,
                                                        const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ lse, int64_t S,
                                                        int H, int Hkv, float* __restrict__ dsum,
                                                        uint16_t* __restrict__ dq) {
  constexpr int KS = D / 16, DT = D / 32, WS = RM_ELEMS(D);
  constexpr int STAGE = AW * 64 * DT * 16 * 2;  // the waves' partial dQ (bf16 units)
  __shared__ __attribute__((aligned(16))) uint16_t smem[AW * WS > STAGE ? AW * WS : STAGE];
  const int t = threadIdx.x, lane = t & 63, hf = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: the walk over blocks is scalar
  uint16_t* const Ks = smem + wave * WS;
  const int64_t nqb = (S + AB - 1) / AB;
  // the longest causal ranges (the last query blocks) are dispatched first
  const int64_t nbh = gridDim.x / nqb;  // sequences x heads
  const int64_t qb = nqb - 1 - blockIdx.x / nbh;
  const int64_t b = (blockIdx.x % nbh) / H;
  const int h = (int)(blockIdx.x % nbh % H);
  const int g = h / (H / Hkv);
  const int64_t ldq = (int64_t)H * D, ldk = (int64_t)Hkv * D;
  const int64_t qpos = qb * AB + c;
  const int64_t qrow = b * S + (qpos < S ? qpos : S - 1);
  const float scale = 1.0f / sqrtf((float)D);
  bf16x8_t qf[KS], df[KS];
  row_frags<D>(seq_rows<D>(q, ldq, (int64_t)h * D, b * S, S), (int)qpos, hf, qf);
  row_frags<D>(seq_rows<D>(dout, ldq, (int64_t)h * D, b * S, S), (int)qpos, hf, df);
  // Dsum over the lane's half of the head dimension, then both halves
  float di = 0.0f;
  {
    const float* orow = o_f32 + qrow * ldq + (int64_t)h * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const u32x4_t u = __builtin_bit_cast(u32x4_t, df[kk]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dv = __uint_as_float((e & 1) ? (u[e >> 1] & 0xFFFF0000u) : (u[e >> 1] << 16));
        di += dv * orow[16 * kk + 8 * hf + e];
      }
    }
    di += __shfl_xor(di, 32);
  }
  if (wave == 0 && hf == 0 && qpos < S) dsum[qrow * H + h] = di;
  const float L = lse[(b * H + h) * S + (qpos < S ? qpos : S - 1)];
  float acc[DT][16];
#pragma unroll
  for (int j = 0; j < DT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  // Two workgroups share a CU: the key block goes through LDS (row-major; the
  // dQ product reads it transposed) without a register prefetch, and the
  // value rows, which only ever serve as A operands of their own lane, come
  // straight from memory.
  const SeqRows<D> sk = seq_rows<D>(k, ldk, (int64_t)g * D, b * S, S);
  const SeqRows<D> sv = seq_rows<D>(v, ldk, (int64_t)g * D, b * S, S);
  const BlockLanes<D> bl = block_lanes<D>(sk.ld2, lane);
  const int qp = (int)qpos, S32 = (int)S;
  for (int kb = wave; kb <= (int)qb; kb += AW) {
    {
      BlockRegs<D> rk;
      load_block<D>(sk, bl, kb * AB, S32, rk, lane);
      store_block<D>(rk, Ks, lane);
    }
    bf16x8_t vf[KS];
    row_frags<D>(sv, kb * AB + c, hf, vf);
    f32x16_t st = zero16(), dp = zero16();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      st = mfma32(frag_rm<D>(Ks, c, hf, kk), qf[kk], st);
      dp = mfma32(vf[kk], df[kk], dp);
    }
    float ds[16];
    if (kb < qb && (kb + 1) * AB <= S32) {  // every key of the block precedes every query
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = __expf(st[r] * scale - L) * (dp[r] - di) * scale;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * AB + crow(r, hf);
        const float pr = (key <= qp && key < S32) ? __expf(st[r] * scale - L) : 0.0f;
        ds[r] = pr * (dp[r] - di) * scale;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t sh, sl;
      split8(ds + 8 * kk, sh, sl);
#pragma unroll
      for (int j = 0; j < DT; ++j) {
        f32x16_t a;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = acc[j][r];
        const bf16x8_t ka = frag_trr<D + 8>(Ks, 32 * j, lane, kk);
        a = mfma32(ka, sh, a);
        a = mfma32(ka, sl, a);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = a[r];
      }
    }
  }
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);  // [AW][64][DT * 16]
  static_assert(AW * 64 * DT * 16 * 4 <= sizeof(smem), "partial staging fits the LDS");
  park<DT * 16>(part, wave, lane, &acc[0][0]);
  __syncthreads();
  if (wave >= DT || qpos >= S) return;
  const int j = wave;
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) {
    float sv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float sacc = 0.0f;
#pragma unroll
      for (int w = 0; w < AW; ++w) sacc += part[(w * 64 + lane) * DT * 16 + j * 16 + 4 * rq + e];
      sv[e] = sacc;
    }
    const int d0 = 32 * j + 8 * rq + 4 * hf;
    uint2 wv;
    wv.x = pack_bf16x2(sv[0], sv[1]);
    wv.y = pack_bf16x2(sv[2], sv[3]);
    *reinterpret_cast<uint2*>(dq + qrow * ldq + (int64_t)h * D + d0) = wv;
  }
}

// dK, dV of a 32-key block for one query head (the query blocks split over AW
// waves and summed in wave order; fp32 partials per head, the heads of a KV
// group summed afterwards in head order). Two workgroups share a CU (at most
// 256 registers and 80 KB of LDS each): each query and dO block goes through
// LDS without a register prefetch, and the key and value rows, operands of
// their own lane only, are read from memory for every block (they stay in
// L2); the waves' dK partials and then their dV partials are
// combined through the same 64 KB of LDS.
template <int D>
__global__ __launch_bounds__(64 * AW, 2) void k_attn_dkv(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const uint16_t* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ dsum, int64_t S,
                                                         int H, int Hkv, float* __restrict__ pk,
                                                         float* __restrict__ pv) {
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int WS = 2 * RM_ELEMS(D) + 4 * AB;  // + lse and Dsum (fp32) of the block
  constexpr int STAGE = AW * 64 * DT * 16 * 2;  // the waves' partial dK or dV (bf16 units)
  __shared__ __attribute__((aligned(16))) uint16_t smem[AW * WS > STAGE ? AW * WS : STAGE];
  const int t = threadIdx.x, lane = t & 63, hf = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: the walk over blocks is scalar
  uint16_t* const Qs = smem + wave * WS;
  uint16_t* const Os = Qs + RM_ELEMS(D);
  float* const Ls = reinterpret_cast<float*>(Os + RM_ELEMS(D));
  float* const Dl = Ls + AB;
  const int64_t nkb = (S + AB - 1) / AB;
  // the longest causal ranges (the first key blocks) are dispatched first
  const int64_t nbh = gridDim.x / nkb;  // sequences x heads
  const int64_t kb = blockIdx.x / nbh;
  const int64_t b = (blockIdx.x % nbh) / H;
  const int h = (int)(blockIdx.x % nbh % H);
  const int g = h / (H / Hkv);
  const int64_t ldq = (int64_t)H * D, ldk = (int64_t)Hkv * D;
  const int64_t kpos = kb * AB + c;
  const int64_t krow = b * S + (kpos < S ? kpos : S - 1);
  const float scale = 1.0f / sqrtf((float)D);
  const SeqRows<D> sk = seq_rows<D>(k, ldk, (int64_t)g * D, b * S, S);
  const SeqRows<D> sv = seq_rows<D>(v, ldk, (int64_t)g * D, b * S, S);
  float adk[DT][16], adv[DT][16];
#pragma unroll
  for (int j = 0; j < DT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      adk[j][r] = 0.0f;
      adv[j][r] = 0.0f;
    }
  const SeqRows<D> sq = seq_rows<D>(q, ldq, (int64_t)h * D, b * S, S);
  const SeqRows<D> so = seq_rows<D>(dout, ldq, (int64_t)h * D, b * S, S);
  const BlockLanes<D> bl = block_lanes<D>(sq.ld2, lane);
  const int kp = (int)kpos, S32 = (int)S;
  for (int qb = (int)kb + wave; qb < (int)nkb; qb += AW) {
    {
      BlockRegs<D> rb;
      load_block<D>(sq, bl, qb * AB, S32, rb, lane);
      store_block<D>(rb, Qs, lane);
      load_block<D>(so, bl, qb * AB, S32, rb, lane);
      store_block<D>(rb, Os, lane);
    }
    if (lane < AB) {
      const int qc = qb * AB + lane < S32 ? qb * AB + lane : S32 - 1;
      Ls[lane] = lse[(b * H + h) * S + qc];
      Dl[lane] = dsum[(b * S + qc) * H + h];
    }
    f32x16_t st = zero16(), dp = zero16();
    {
      bf16x8_t kf[KS];
      row_frags<D>(sk, kp, hf, kf, opaque_zero());
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) st = mfma32(frag_rm<D>(Qs, c, hf, kk), kf[kk], st);
    }
    {
      bf16x8_t vf[KS];
      row_frags<D>(sv, kp, hf, vf, opaque_zero());
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) dp = mfma32(frag_rm<D>(Os, c, hf, kk), vf[kk], dp);
    }
    float p[16], ds[16];
    if (qb > (int)kb && (qb + 1) * AB <= S32) {  // every query of the block follows every key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = crow(r, hf);
        p[r] = __expf(st[r] * scale - Ls[qr]);
        ds[r] = p[r] * (dp[r] - Dl[qr]) * scale;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = crow(r, hf);
        const int qp = qb * AB + qr;
        p[r] = (kp <= qp && qp < S32) ? __expf(st[r] * scale - Ls[qr]) : 0.0f;
        ds[r] = p[r] * (dp[r] - Dl[qr]) * scale;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t ph, pl, sh, sl;
      split8(p + 8 * kk, ph, pl);
      split8(ds + 8 * kk, sh, sl);
#pragma unroll
      for (int j = 0; j < DT; ++j) {
        f32x16_t a, bq;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          a[r] = adv[j][r];
          bq[r] = adk[j][r];
        }
        const bf16x8_t oa = frag_trr<D + 8>(Os, 32 * j, lane, kk);
        a = mfma32(oa, ph, a);
        a = mfma32(oa, pl, a);
        const bf16x8_t qa = frag_trr<D + 8>(Qs, 32 * j, lane, kk);
        bq = mfma32(qa, sh, bq);
        bq = mfma32(qa, sl, bq);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          adv[j][r] = a[r];
          adk[j][r] = bq[r];
        }
      }
    }
  }
  // combine the waves: dK first, then dV through the same LDS
  float* part = reinterpret_cast<float*>(smem);  // [AW][64][DT * 16]
  static_assert(AW * 64 * DT * 16 * 4 <= sizeof(smem), "partial staging fits the LDS");
  const int64_t prow = (krow * H + h) * D;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
    park<DT * 16>(part, wave, lane, pass == 0 ? &adk[0][0] : &adv[0][0]);
    __syncthreads();
    if (wave < DT && kpos < S) {
      const int j = wave;
      float* const dst = pass == 0 ? pk : pv;
#pragma unroll
      for (int rq2 = 0; rq2 < 4; ++rq2) {
        float sm[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float a = 0.0f;
#pragma unroll
          for (int w = 0; w < AW; ++w) a += part[(w * 64 + lane) * DT * 16 + j * 16 + 4 * rq2 + e];
          sm[e] = a;
        }
        const int d0 = 32 * j + 8 * rq2 + 4 * hf;
        *reinterpret_cast<float4*>(dst + prow + d0) = make_float4(sm[0], sm[1], sm[2], sm[3]);
      }
    }
  }
}

// dk[row, g, :] = bf16(sum over the heads of group g, in head order, of the
// per-head partials); one thread per (row, kv head, 4 dims). dv_packed
// (nullable): dv also in MFMA fragment order (K = Hkv * D), as k_frag_pack
// lays it out, for the v projection's backward.
__global__ __launch_bounds__(256) void k_attn_group_sum(const float* __restrict__ pk,
                                                        const float* __restrict__ pv, int64_t T,
                                                        int H, int Hkv, int D,
                                                        uint16_t* __restrict__ dk,
                                                        uint16_t* __restrict__ dv,
                                                        uint8_t* __restrict__ dv_packed) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n4 = T * Hkv * (D / 4);
  if (i >= n4) return;
  const int d4 = (int)(i % (D / 4));
  const int64_t rg = i / (D / 4);
  const int g = (int)(rg % Hkv);
  const int64_t row = rg / Hkv;
  const int grp = H / Hkv;
  float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
  for (int hh = 0; hh < grp; ++hh) {
    const int64_t off = (row * H + g * grp + hh) * D + 4 * d4;
    const float4 a = *reinterpret_cast<const float4*>(pk + off);
    const float4 bq = *reinterpret_cast<const float4*>(pv + off);
    sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
    sv.x += bq.x; sv.y += bq.y; sv.z += bq.z; sv.w += bq.w;
  }
  const int64_t out = (row * Hkv + g) * D + 4 * d4;
  uint2 wk, wv;
  wk.x = pack_bf16x2(sk.x, sk.y);
  wk.y = pack_bf16x2(sk.z, sk.w);
  wv.x = pack_bf16x2(sv.x, sv.y);
  wv.y = pack_bf16x2(sv.z, sv.w);
  *reinterpret_cast<uint2*>(dk + out) = wk;
  *reinterpret_cast<uint2*>(dv + out) = wv;
  if (dv_packed) {
    // four consecutive columns are one half of a fragment's 16-byte slot
    const int64_t K = (int64_t)Hkv * D, kb = (K + 63) / 64 * 4;
    const int64_t c = (int64_t)g * D + 4 * d4;
    *reinterpret_cast<uint2*>(dv_packed + frag_offset(row, c & ~7ll, kb) + (c & 7) * 2) = wv;
    if (g == Hkv - 1 && d4 == 0) frag_zero_tail(dv_packed, row, K, kb);
  }
}

// ---- elementwise ------------------------------------------------------------
// Element-wise kernels over a [T, W] matrix (W a multiple of 8), one
// workgroup per 32 x 64 tile (one 64-wide step of one 32-row block): thread t
// takes row t/8, columns 8*(t%8) .. +8 of the tile, so row-major reads and
// writes are 128 contiguous bytes per 8 lanes. With a packed pointer the bf16
// result also goes through LDS and leaves in MFMA fragment order (K = W):
// the tile's four fragments, 4 KB contiguous, for the GEMM that reads it
// next; rows past T are not written, columns past W are written as zeros.
constexpr int EW_STRIDE = 144;  // bytes per staged row (128 + 16: conflict-free reads)

struct EwTile {
  int64_t rb, st;  // the workgroup's 32-row block and 64-wide step
  int64_t m, c;    // the thread's row and first column
  bool ok;         // m < T and c < W
};

__device__ __forceinline__ EwTile ew_tile(int64_t T, int64_t W) {
  EwTile e;
  const int64_t steps = (W + 63) / 64;
  e.rb = (int64_t)blockIdx.x / steps;
  e.st = (int64_t)blockIdx.x % steps;
  e.m = 32 * e.rb + (threadIdx.x >> 3);
  e.c = 64 * e.st + 8 * (threadIdx.x & 7);
  e.ok = e.m < T && e.c < W;
  return e;
}

// Writes the thread's 8 results (row-major when out is set, packed when
// packed is set); stage is 32 * EW_STRIDE bytes of LDS. Every thread of the
// workgroup must call it (it holds a barrier).
__device__ __forceinline__ void ew_store(const EwTile& e, int64_t T, int64_t W, uint16_t* out,
                                         uint8_t* packed, uint8_t* stage, const float* f) {
  u32x4v o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  if (!e.ok) o = u32x4v{0u, 0u, 0u, 0u};
  if (out && e.ok) *reinterpret_cast<u32x4v*>(out + e.m * W + e.c) = o;
  if (!packed) return;
  *reinterpret_cast<u32x4v*>(stage + (threadIdx.x >> 3) * EW_STRIDE + (threadIdx.x & 7) * 16) = o;
  __syncthreads();
  const int f16 = threadIdx.x >> 6, lane = threadIdx.x & 63;  // 16-wide block of the step, lane
  const int64_t row = 32 * e.rb + (lane & 31);
  if (row < T) {
    const u32x4v w = *reinterpret_cast<const u32x4v*>(stage + (lane & 31) * EW_STRIDE +
                                                      (2 * f16 + (lane >> 5)) * 16);
    const int64_t kb = (W + 63) / 64 * 4;
    const int64_t frag = e.rb * kb + 4 * e.st + f16;
    *reinterpret_cast<u32x4v*>(packed + (frag * 64 + lane) * 16) = w;
  }
}

__global__ __launch_bounds__(256) void k_swiglu_fwd(const uint16_t* __restrict__ g,
                                                    const uint16_t* __restrict__ u, int64_t T,
                                                    int64_t W, uint16_t* __restrict__ out,
                                                    uint8_t* __restrict__ packed) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[32 * EW_STRIDE];
  const EwTile e = ew_tile(T, W);
  float o[8] = {};
  if (e.ok) {
    float gv[8], uv[8];
    load8_bf16(g + e.m * W + e.c, gv);
    load8_bf16(u + e.m * W + e.c, uv);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = swiglu_val(gv[i], uv[i]);
  }
  ew_store(e, T, W, out, packed, stage, o);
}

__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t* __restrict__ ds,
                                                    const uint16_t* __restrict__ g,
                                                    const uint16_t* __restrict__ u, int64_t T,
                                                    int64_t W, uint16_t* __restrict__ dg,
                                                    uint16_t* __restrict__ du,
                                                    uint8_t* __restrict__ dg_packed,
                                                    uint8_t* __restrict__ du_packed) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2][32 * EW_STRIDE];
  const EwTile e = ew_tile(T, W);
  float og[8] = {}, ou[8] = {};
  if (e.ok) {
    float gv[8], uv[8], d[8];
    load8_bf16(g + e.m * W + e.c, gv);
    load8_bf16(u + e.m * W + e.c, uv);
    load8_bf16(ds + e.m * W + e.c, d);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = 1.0f / (1.0f + __expf(-gv[i]));
      og[i] = d[i] * uv[i] * (sg * (1.0f + gv[i] * (1.0f - sg)));
      ou[i] = d[i] * gv[i] * sg;
    }
  }
  ew_store(e, T, W, dg, dg_packed, stage[0], og);
  ew_store(e, T, W, du, du_packed, stage[1], ou);
}

// out = h + y (fp32 residual stream plus a bf16 branch output); out may be h
__global__ __launch_bounds__(256) void k_residual_add(const float* h, const uint16_t* __restrict__ y,
                                                      int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = h[i] + bf2f(y[i]);
}

__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* __restrict__ x, int64_t T,
                                                     int64_t W, uint16_t* __restrict__ y,
                                                     uint8_t* __restrict__ packed) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[32 * EW_STRIDE];
  const EwTile e = ew_tile(T, W);
  float f[8] = {};
  if (e.ok) load8_f32(x + e.m * W + e.c, f);
  ew_store(e, T, W, y, packed, stage, f);
}

// ---- rows of logits: one 1024-thread workgroup per row ----------------------
// A row of a large vocabulary (128,256 bf16 = 256 KB) is read twice: once
// for its log-sum-exp, with a running maximum and a sum rescaled whenever the
// maximum grows (one exponential per element), and once for the gradient.
// Rows whose length is a multiple of 8 and whose start is 16-byte aligned are
// read 16 bytes per lane. The partial (max, sum) pairs are combined in a
// fixed order: a butterfly inside each wave, then the 16 waves in order.
constexpr int ROW_THREADS = 1024;

__device__ __forceinline__ void ms_add(float& m, float& s, float x) {
  if (x > m) {
    s = s * expf(m - x) + 1.0f;
    m = x;
  } else if (x != -INFINITY) {
    s += expf(x - m);
  }
}

__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both parts empty
  s = (m == -INFINITY ? 0.0f : s * expf(m - M)) + (m2 == -INFINITY ? 0.0f : s2 * expf(m2 - M));
  m = M;
}

__device__ __forceinline__ bool row_vec(const uint16_t* z, int64_t V) {
  return V % 8 == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0;
}

// log-sum-exp of z[0, V) (fp32); red holds 2 * 16 floats
__device__ __forceinline__ float row_lse(const uint16_t* __restrict__ z, int64_t V, float* red) {
  float m = -INFINITY, s = 0.0f;
  if (row_vec(z, V)) {
    for (int64_t j = threadIdx.x; j < V / 8; j += ROW_THREADS) {
      float x[8];
      load8_bf16(z + 8 * j, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) ms_add(m, s, x[e]);
    }
  } else {
    for (int64_t j = threadIdx.x; j < V; j += ROW_THREADS) ms_add(m, s, bf2f(z[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    ms_merge(m, s, m2, s2);
  }
  __syncthreads();  // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) {
    red[2 * (threadIdx.x >> 6)] = m;
    red[2 * (threadIdx.x >> 6) + 1] = s;
  }
  __syncthreads();
  float M = red[0], S = red[1];
  for (int w = 1; w < ROW_THREADS / 64; ++w) ms_merge(M, S, red[2 * w], red[2 * w + 1]);
  return M + logf(S);
}

// out[j] = bf16(w * (exp(z[j] - lse) - [j == tg])) over the row
__device__ __forceinline__ void row_grad(const uint16_t* __restrict__ z, int64_t V, float lse, int64_t tg, float w,
                         uint16_t* __restrict__ out) {
  if (row_vec(z, V) && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    for (int64_t j = threadIdx.x; j < V / 8; j += ROW_THREADS) {
      float x[8];
      load8_bf16(z + 8 * j, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = expf(x[e] - lse);
        if (8 * j + e == tg) p -= 1.0f;
        x[e] = w * p;
      }
      store8_bf16(out + 8 * j, x);
    }
  } else {
    for (int64_t j = threadIdx.x; j < V; j += ROW_THREADS) {
      float p = expf(bf2f(z[j]) - lse);
      if (j == tg) p -= 1.0f;
      out[j] = f2bf(w * p);
    }
  }
}

// Cross-entropy of one row of bf16 logits: row loss and bf16 gradient
// (softmax - onehot) / T. A target outside [0, V) makes the row loss NaN.
__global__ __launch_bounds__(ROW_THREADS) void k_ce_rows(const uint16_t* __restrict__ logits,
                                                         const int64_t* __restrict__ targets, int64_t T,
                                                         int64_t V, float* __restrict__ row_loss,
                                                         uint16_t* __restrict__ dlogits) {
  __shared__ float red[2 * ROW_THREADS / 64];
  const int64_t t = blockIdx.x;
  const uint16_t* z = logits + t * V;
  const float lse = row_lse(z, V, red);
  const int64_t tg = targets[t];
  const bool ok = tg >= 0 && tg < V;
  if (threadIdx.x == 0) row_loss[t] = ok ? lse - bf2f(z[tg]) : __builtin_nanf("");
  row_grad(z, V, lse, tg, 1.0f / (float)T, dlogits + t * V);
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

// ---- preference step (DPO) ---------------------------------------------------
// Per-token negative log-probability of the target, logsumexp(z_t) - z_t[y_t]
// (fp32; NaN for a target outside [0, V)); one workgroup per row.
__global__ __launch_bounds__(ROW_THREADS) void k_token_nll(const uint16_t* __restrict__ logits,
                                                           const int64_t* __restrict__ targets,
                                                           int64_t V, float* __restrict__ nll) {
  __shared__ float red[2 * ROW_THREADS / 64];
  const int64_t t = blockIdx.x;
  const uint16_t* z = logits + t * V;
  const float lse = row_lse(z, V, red);
  const int64_t tg = targets[t];
  const bool ok = tg >= 0 && tg < V;
  if (threadIdx.x == 0) nll[t] = ok ? lse - bf2f(z[tg]) : __builtin_nanf("");
}

__device__ __forceinline__ float log_sigmoid(float x) {
  return -(fmaxf(-x, 0.0f) + log1pf(expf(-fabsf(x))));
}

// DPO over n_seq = 2 * pairs sequences of S tokens (chosen, rejected per
// pair): lp / lr = -sum of mask * nll (policy / reference) per sequence, in
// a fixed order; delta = beta * ((lp_c - lr_c) - (lp_r - lr_r));
// loss = -mean log sigmoid(delta); coef[s] = dL/d(sum of masked nll of s).
// One workgroup.
__global__ __launch_bounds__(256) void k_dpo(const float* __restrict__ nll_p,
                                             const float* __restrict__ nll_r,
                                             const float* __restrict__ mask, int64_t pairs,
                                             int64_t S, float beta, float* __restrict__ loss,
                                             float* __restrict__ coef) {
  __shared__ float red[4];
  float total = 0.0f;
  for (int64_t p = 0; p < pairs; ++p) {
    float v[4];  // lp_c, lr_c, lp_r, lr_r
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t base = (2 * p + (q >> 1)) * S;
      const float* src = (q & 1) ? nll_r : nll_p;
      float a = 0.0f;
      for (int64_t j = threadIdx.x; j < S; j += 256) a += mask[base + j] * src[base + j];
      v[q] = -block_sum(a, red);
    }
    const float delta = beta * ((v[0] - v[1]) - (v[2] - v[3]));
    const float sig_neg = expf(log_sigmoid(-delta));  // sigmoid(-delta)
    const float g = sig_neg / (float)pairs;           // -dL/d delta
    if (threadIdx.x == 0) {
      coef[2 * p] = beta * g;
      coef[2 * p + 1] = -beta * g;
    }
    total += log_sigmoid(delta);
  }
  if (threadIdx.x == 0) loss[0] = -total / (float)pairs;
}

// dlogits[t] = bf16(coef[t / S] * mask[t] * (softmax(z_t) - onehot(y_t))).
__global__ __launch_bounds__(ROW_THREADS) void k_logit_grad(const uint16_t* __restrict__ logits,
                                                            const int64_t* __restrict__ targets,
                                                            const float* __restrict__ coef,
                                                            const float* __restrict__ mask, int64_t S,
                                                            int64_t V, uint16_t* __restrict__ dlogits) {
  __shared__ float red[2 * ROW_THREADS / 64];
  const int64_t t = blockIdx.x;
  const uint16_t* z = logits + t * V;
  const float lse = row_lse(z, V, red);
  row_grad(z, V, lse, targets[t], coef[t / S] * mask[t], dlogits + t * V);
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

// one workgroup per 32 x 64 tile of a [T, W] matrix (T * W < 2^40: < 2^29 tiles)
inline dim3 ew_grid(int64_t T, int64_t W) {
  return dim3((unsigned)(((T + 31) / 32) * ((W + 63) / 64)));
}

}  // namespace

hipError_t launch_embed(const uint16_t* E, int64_t V, const int64_t* ids, int64_t T, int64_t H,
                        float* h, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3((unsigned)T), dim3(256), 0, s, E, V, ids, H, h);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_fwd(const float* x, const float* w, int64_t T, int64_t H, float eps,
                              uint16_t* y, float* rstd, void* packed, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm_fwd, dim3(xcd_rows(T)), dim3(256), 0, s, x, w, H, eps, y, rstd,
                     static_cast<uint8_t*>(packed), T);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* const* dys, int n_dy, const float* x, const float* w,
                              const float* rstd, int64_t T, int64_t H, int accumulate, float* dh,
                              uint16_t* y, void* packed, hipStream_t s) {
  DyPtrs d{{dys[0], n_dy > 1 ? dys[1] : nullptr, n_dy > 2 ? dys[2] : nullptr}};
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(xcd_rows(T)), dim3(256), 0, s, d, n_dy, x, w, rstd, H,
                     accumulate, dh, y, static_cast<uint8_t*>(packed), T);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* x, int64_t T, int64_t S, int heads, int d, double theta,
                       int inverse, hipStream_t s) {
  return launch_rope_pair(x, heads, nullptr, 0, T, S, d, theta, inverse, nullptr, nullptr, s);
}

hipError_t launch_rope_pair(uint16_t* x1, int heads1, uint16_t* x2, int heads2, int64_t T, int64_t S,
                            int d, double theta, int inverse, void* p1, void* p2, hipStream_t s) {
  InvFreq inv;
  for (int j = 0; j < 128; ++j) inv.f[j] = j < d / 2 ? pow(theta, -2.0 * j / d) : 0.0;
  const bool wide = (d / 2) % 8 == 0 && reinterpret_cast<uintptr_t>(x1) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(x2) % 16 == 0;
  if (wide)
    hipLaunchKernelGGL(k_rope_rows<8>, dim3(xcd_rows(T)), dim3(256), 0, s, x1, heads1,
                       static_cast<uint8_t*>(p1), x2, heads2, static_cast<uint8_t*>(p2), T, S, d, inv, inverse);
  else
    hipLaunchKernelGGL(k_rope_rows<4>, dim3(xcd_rows(T)), dim3(256), 0, s, x1, heads1,
                       static_cast<uint8_t*>(p1), x2, heads2, static_cast<uint8_t*>(p2), T, S, d, inv, inverse);
  return hipGetLastError();
}

#define NF4S_DISPATCH_D(D_, CALL) \
  switch (D_) {                   \
    case 32: CALL(32); break;     \
    case 64: CALL(64); break;     \
    case 128: CALL(128); break;   \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                int64_t S, int H, int Hkv, int D, uint16_t* o, float* o_f32,
                                float* lse, void* packed, hipStream_t s) {
  const unsigned grid = (unsigned)(B * H * ((S + AB - 1) / AB));
  uint8_t* const pk = static_cast<uint8_t*>(packed);
#define CALL(DD) hipLaunchKernelGGL(k_attn_fwd<DD>, dim3(grid), dim3(64 * AW), 0, s, q, k, v, S, H, Hkv, o, o_f32, lse, pk)
  NF4S_DISPATCH_D(D, CALL)
#undef CALL
  return hipGetLastError();
}

// Workspace: Dsum [B*S, H] fp32, then the per-head dK and dV partials
// [B*S, H, D] fp32 each (256-byte aligned sections).
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t attention_bwd_ws_bytes(int64_t B, int64_t S, int H, int D) {
  const size_t rows = (size_t)(B * S);
  return align256(rows * H * sizeof(float)) + 2 * align256(rows * H * D * sizeof(float));
}

hipError_t launch_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* o_f32, const uint16_t* dout, const float* lse,
                                int64_t B, int64_t S, int H, int Hkv, int D, uint16_t* dq,
                                uint16_t* dk, uint16_t* dv, void* dv_packed, void* ws, hipStream_t s) {
  const size_t rows = (size_t)(B * S);
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* dsum = reinterpret_cast<float*>(w);
  float* pk = reinterpret_cast<float*>(w + align256(rows * H * sizeof(float)));
  float* pv = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(pk) + align256(rows * H * D * sizeof(float)));
  const unsigned grid = (unsigned)(B * H * ((S + AB - 1) / AB));
#define CALL(DD)                                                                                   \
  hipLaunchKernelGGL(k_attn_dq<DD>, dim3(grid), dim3(64 * AW), 0, s, q, k, v, o_f32, dout, lse, S, H, Hkv, \
                     dsum, dq);                                                                    \
  hipLaunchKernelGGL(k_attn_dkv<DD>, dim3(grid), dim3(64 * AW), 0, s, q, k, v, dout, lse, dsum, S, H, Hkv, \
                     pk, pv)
  NF4S_DISPATCH_D(D, CALL)
#undef CALL
  const int64_t n4 = (int64_t)rows * Hkv * (D / 4);
  hipLaunchKernelGGL(k_attn_group_sum, dim3(grid_of(n4)), dim3(256), 0, s, pk, pv, (int64_t)rows, H,
                     Hkv, D, dk, dv, static_cast<uint8_t*>(dv_packed));
  return hipGetLastError();
}
#undef NF4S_DISPATCH_D

hipError_t launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t T, int64_t W,
                             uint16_t* out, void* packed, hipStream_t s) {
  hipLaunchKernelGGL(k_swiglu_fwd, ew_grid(T, W), dim3(256), 0, s, g, u, T, W, out,
                     static_cast<uint8_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* ds, const uint16_t* g, const uint16_t* u, int64_t T,
                             int64_t W, uint16_t* dg, uint16_t* du, void* dg_packed,
                             void* du_packed, hipStream_t s) {
  hipLaunchKernelGGL(k_swiglu_bwd, ew_grid(T, W), dim3(256), 0, s, ds, g, u, T, W, dg, du,
                     static_cast<uint8_t*>(dg_packed), static_cast<uint8_t*>(du_packed));
  return hipGetLastError();
}

hipError_t launch_residual_add(const float* h, const uint16_t* y, int64_t n, float* out,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_residual_add, dim3(grid_of(n)), dim3(256), 0, s, h, y, n, out);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* x, int64_t T, int64_t W, uint16_t* y, void* packed,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_f32_to_bf16, ew_grid(T, W), dim3(256), 0, s, x, T, W, y,
                     static_cast<uint8_t*>(packed));
  return hipGetLastError();
}

size_t cross_entropy_ws_bytes(int64_t T) { return (size_t)T * sizeof(float); }

hipError_t launch_cross_entropy(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                                float* loss, uint16_t* dlogits, void* ws, hipStream_t s) {
  float* rows = static_cast<float*>(ws);
  hipLaunchKernelGGL(k_ce_rows, dim3((unsigned)T), dim3(ROW_THREADS), 0, s, logits, targets, T, V, rows,
                     dlogits);
  hipLaunchKernelGGL(k_mean, dim3(1), dim3(256), 0, s, rows, T, loss);
  return hipGetLastError();
}

hipError_t launch_token_nll(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                            float* nll, hipStream_t s) {
  hipLaunchKernelGGL(k_token_nll, dim3((unsigned)T), dim3(ROW_THREADS), 0, s, logits, targets, V, nll);
  return hipGetLastError();
}

hipError_t launch_dpo(const float* nll_p, const float* nll_r, const float* mask, int64_t pairs,
                      int64_t S, float beta, float* loss, float* coef, hipStream_t s) {
  hipLaunchKernelGGL(k_dpo, dim3(1), dim3(256), 0, s, nll_p, nll_r, mask, pairs, S, beta, loss, coef);
  return hipGetLastError();
}

hipError_t launch_logit_grad(const uint16_t* logits, const int64_t* targets, const float* coef,
                             const float* mask, int64_t T, int64_t S, int64_t V, uint16_t* dlogits,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_logit_grad, dim3((unsigned)T), dim3(ROW_THREADS), 0, s, logits, targets, coef,
                     mask, S, V, dlogits);
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
