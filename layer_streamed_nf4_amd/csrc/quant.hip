// Offline NF4 double-quant sharder and the standalone dequantiser.
//
// Gate walkthrough ("Soup layer-streamed NF4 training measured"), section 2.1:
// each tensor is quantised once, offline, blockwise 64, into packed 4-bit codes
// plus the absmax sidecar, which double quant replaces by 8-bit codes, a nested
// absmax per 256 blocks and one offset; section 2.3: the result is byte-for-byte
// deterministic. Three passes, all with fixed reduction orders:
//   1. per 64-block absmax, NF4 codes, nibble packing (16 lanes per block),
//      and each workgroup's double-double sum of its 64 absmax values;
//   2. the offset = mean of the absmax, summed exactly (double-double, the
//      workgroup partials in a fixed order) then divided once in fp64 and
//      rounded to fp32;
//   3. per 256-block nested absmax of (absmax - offset) and the 8-bit codes.
#include <cmath>

#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int kLanesPerBlock = 16;  // 16 lanes x 4 elements = one 64-block

// #{i : v > m_i} over ascending thresholds m[0..n-2] (n a power of two): the
// nearest level with ties to the lower code.
template <int N>
__device__ __forceinline__ int code_of(float v, const float* m) {
  int idx = 0;
#pragma unroll
  for (int step = N / 2; step >= 1; step >>= 1)
    if (v > m[idx + step - 1]) idx += step;
  return idx;
}

// A workgroup takes kItems consecutive chunks of 256 x 4 elements; in chunk j
// thread t handles elements 4t..4t+3 (block t/16 of the chunk), so every load
// and store instruction of a wave covers contiguous bytes, and all kItems
// loads of a thread are issued before the first is used.
constexpr int kItems = 4;
constexpr int kChunkElems = 256 * 4;

// Double-double helpers (error-free transformations; no multiplications).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
__device__ __forceinline__ void dd_add(double& hi, double& lo, double xhi, double xlo) {
  double s, e;
  two_sum(hi, xhi, s, e);
  e += lo + xlo;
  hi = s + e;
  lo = e - (hi - s);
}

// Fixed pairwise tree over the 64 lanes of a wave (lane l takes lane l + w,
// w = 1, 2, ..., 32); lane 0 ends with the sum.
__device__ __forceinline__ void dd_wave_tree(double& hi, double& lo) {
  const int l = (int)(threadIdx.x & 63);
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) {
    const double ph = __shfl_down(hi, w, 64), pl = __shfl_down(lo, w, 64);
    if ((l & (2 * w - 1)) == 0) dd_add(hi, lo, ph, pl);
  }
}

// The NF4 code of n = fl(v / m) is #{i : n > t_i} over the 15 thresholds. It
// is found without the division: an fp64 estimate of v / m picks one of 257
// buckets of width 1/128 on [-1, 1]; the bucket's count c of thresholds below
// it makes t_c the only threshold that can lie inside it, and fl(v / m) > t_c
// is decided exactly as v > B_c * m in fp64, with B_c the midpoint between t_c
// and the next fp32 above it: a quotient above B_c rounds above t_c, one below
// rounds to t_c or lower. B_c's significand has 25 bits and ends in a one, so
// B_c * m (exact in fp64: 25 + 24 bits) never fits an fp32 and v / m never
// equals B_c, the only case round-to-nearest-even would have to settle. No
// threshold lies within 1/64 of a bucket width of a bucket edge (checked on
// the host when the table is built), far beyond the estimate's error, so an
// estimate that lands in the neighbouring bucket gives the same code. m = 0
// gives n = 0.
template <int DTYPE>
__global__ __launch_bounds__(256) void k_absmax_codes(const void* __restrict__ w, int64_t nb,
                                                       uint8_t* __restrict__ packed,
                                                       float* __restrict__ absmax,
                                                       int32_t* __restrict__ status, Buckets4 bk,
                                                       double2* __restrict__ part) {
  __shared__ double s_b[16];
  __shared__ uint32_t s_code[65];
  __shared__ float s_am[kItems * 16];  // the workgroup's absmax, in block order
  const int lane = (int)(threadIdx.x % kLanesPerBlock);
  const int64_t base = (int64_t)blockIdx.x * kItems * kChunkElems + threadIdx.x * 4;
  const int64_t ne = nb * 64;
  float v[kItems][4];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t e0 = base + j * kChunkElems;
    if (e0 >= ne) continue;  // whole blocks: a block is either in range or not
    if (DTYPE == NF4S_DTYPE_F32) {
      const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + e0);
      v[j][0] = t.x; v[j][1] = t.y; v[j][2] = t.z; v[j][3] = t.w;
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + e0);
      v[j][0] = __uint_as_float(t.x << 16);
      v[j][1] = __uint_as_float(t.x & 0xFFFF0000u);
      v[j][2] = __uint_as_float(t.y << 16);
      v[j][3] = __uint_as_float(t.y & 0xFFFF0000u);
    }
  }
  // the bucket table, filled while the loads are in flight
  if (threadIdx.x < 16) s_b[threadIdx.x] = bk.b_mid[threadIdx.x];
  if (threadIdx.x < 65) s_code[threadIdx.x] = reinterpret_cast<const uint32_t*>(bk.code)[threadIdx.x];
  __syncthreads();
  const uint8_t* const codes = reinterpret_cast<const uint8_t*>(s_code);
  bool finite = true;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t e0 = base + j * kChunkElems;
    float m = 0.0f;
    if (e0 < ne) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        finite = finite && __builtin_isfinite(v[j][i]);
        m = fmaxf(m, fabsf(v[j][i]));
      }
    }
    // max over the 16 lanes of this block (exact, order-free); the lanes of
    // a block are all in range or all out, and every lane takes part
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kLanesPerBlock));
    if (lane == 0) s_am[j * 16 + threadIdx.x / kLanesPerBlock] = m;  // 0 past the last block
    if (e0 >= ne) continue;
    const double md = (m > 0.0f) ? (double)m : 1.0;
    const double rd = __builtin_amdgcn_rcp(md);  // estimate only
    int c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double vd = (double)v[j][i];
      const double pos = fmin(fmax(__builtin_fma(vd * rd, 128.0, 128.0), 0.0), 256.0);
      const int cb = codes[(int)pos];
      c[i] = cb + (int)(vd > s_b[cb] * md);
    }
    const uint32_t b0 = (uint32_t)((c[0] << 4) | c[1]);
    const uint32_t b1 = (uint32_t)((c[2] << 4) | c[3]);
    reinterpret_cast<uint16_t*>(packed)[e0 / 4] = (uint16_t)(b0 | (b1 << 8));
    if (lane == 0) absmax[e0 / 64] = m;
  }
  if (!finite && status) {
    volatile int32_t* st = status;
    *st = 1;
  }
  // first pass of the offset sum: this workgroup's kItems * 16 absmax values
  // added in double-double over a fixed pairwise tree
  __syncthreads();
  if (threadIdx.x < 64) {
    double hi = (double)s_am[threadIdx.x], lo = 0.0;
    dd_wave_tree(hi, lo);
    if (threadIdx.x == 0) part[blockIdx.x] = make_double2(hi, lo);
  }
}

// The offset sum in two fixed-order passes: k_absmax_codes adds the absmax of
// each of its workgroups (kItems * 16 consecutive blocks) into one
// double-double partial, and one workgroup adds the partials (thread t the
// partials t, t + T, ... in order, then a fixed tree over the threads) and
// divides once. The
// partition is a function of nb only, so the result is the same on every run;
// every addition is double-double.
constexpr int kFinalThreads = 1024;
constexpr int64_t kBlocksPerPart = kItems * 16;

int64_t offset_parts(int64_t nb) {
  const int64_t g = (nb + kBlocksPerPart - 1) / kBlocksPerPart;
  return g < 1 ? 1 : g;
}

__global__ __launch_bounds__(kFinalThreads) void k_offset_final(const double2* __restrict__ part,
                                                                 int64_t parts, int64_t nb,
                                                                 float* __restrict__ offset) {
  __shared__ double s_hi[kFinalThreads / 64];
  __shared__ double s_lo[kFinalThreads / 64];
  const int t = threadIdx.x;
  double hi = 0.0, lo = 0.0;
  // partials t, t + T, t + 2T, ... in order, eight loads issued at a time
  constexpr int kBatch = 8;
  for (int64_t i0 = t; i0 < parts; i0 += (int64_t)kBatch * kFinalThreads) {
    double2 v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int64_t i = i0 + (int64_t)q * kFinalThreads;
      v[q] = i < parts ? part[i] : make_double2(0.0, 0.0);
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) dd_add(hi, lo, v[q].x, v[q].y);
  }
  dd_wave_tree(hi, lo);
  if ((t & 63) == 0) {
    s_hi[t >> 6] = hi;
    s_lo[t >> 6] = lo;
  }
  __syncthreads();
  if (t < 64) {
    hi = t < kFinalThreads / 64 ? s_hi[t] : 0.0;
    lo = t < kFinalThreads / 64 ? s_lo[t] : 0.0;
    dd_wave_tree(hi, lo);
    if (t == 0) {
      const double sum = hi + lo;  // one rounding of the exact sum
      offset[0] = (float)(sum / (double)nb);
    }
  }
}

__global__ __launch_bounds__(256) void k_nested(const float* __restrict__ absmax, int64_t nb,
                                                const float* __restrict__ offset,
                                                float* __restrict__ nested,
                                                uint8_t* __restrict__ q8, Mids8 mids) {
  __shared__ float s_m[255];
  __shared__ float s_wmax[4];
  for (int i = threadIdx.x; i < 255; i += 256) s_m[i] = mids.m[i];
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float off = offset[0];
  const float c = (b < nb) ? __fsub_rn(absmax[b], off) : 0.0f;
  float m = fabsf(c);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) s_wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  const float nm = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  if (threadIdx.x == 0) nested[blockIdx.x] = nm;
  if (b < nb) {
    const float u = (nm > 0.0f) ? __fdiv_rn(c, nm) : 0.0f;
    q8[b] = (uint8_t)code_of<256>(u, s_m);
  }
}

// Standalone dequantiser: 8 elements (one packed word) per thread.
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ packed,
                                                 const uint8_t* __restrict__ q8,
                                                 const float* __restrict__ nested,
                                                 const float* __restrict__ offset,
                                                 int64_t nwords, uint4* __restrict__ out,
                                                 Tables tab) {
  __shared__ float s_c4[16];
  __shared__ float s_c8[256];
  if (threadIdx.x < 16) s_c4[threadIdx.x] = tab.c4[threadIdx.x];
  s_c8[threadIdx.x] = tab.c8[threadIdx.x];
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int64_t blk = i >> 3;  // 8 words per 64-block
  const float a = decode_scale(s_c8[q8[blk]], nested[blk >> 8], offset[0]);
  uint32_t o[4];
  dequant_word(packed[i], a, s_c4, o);
  out[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

// absmax fp32 [nb], then the offset pass's double-double partials
static size_t absmax_bytes(int64_t nb) { return ((size_t)nb * sizeof(float) + 255) / 256 * 256; }

size_t quantize_ws_bytes(int64_t n_out, int64_t k_in) {
  const int64_t nb = n_out * k_in / 64;
  return absmax_bytes(nb) + (size_t)offset_parts(nb) * sizeof(double2);
}

hipError_t launch_quantize(const void* w, int dtype, int64_t n_out, int64_t k_in, uint8_t* packed,
                           uint8_t* q8, float* nested, float* offset, int32_t* status, void* ws,
                           hipStream_t s) {
  if (!host_buckets4().ok) return hipErrorInvalidValue;  // the bucket search's premise
  const int64_t nb = n_out * k_in / 64;
  float* absmax = static_cast<float*>(ws);
  const int64_t parts = offset_parts(nb);
  double2* part = reinterpret_cast<double2*>(static_cast<uint8_t*>(ws) + absmax_bytes(nb));
  const int64_t per_wg = (int64_t)kItems * kChunkElems;
  const dim3 grid((unsigned)((nb * 64 + per_wg - 1) / per_wg));
  if (dtype == NF4S_DTYPE_F32)
    hipLaunchKernelGGL(k_absmax_codes<NF4S_DTYPE_F32>, grid, dim3(256), 0, s, w, nb, packed, absmax,
                       status, host_buckets4(), part);
  else
    hipLaunchKernelGGL(k_absmax_codes<NF4S_DTYPE_BF16>, grid, dim3(256), 0, s, w, nb, packed,
                       absmax, status, host_buckets4(), part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_offset_final, dim3(1), dim3(kFinalThreads), 0, s, part, parts, nb, offset);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nn = (nb + 255) / 256;
  hipLaunchKernelGGL(k_nested, dim3((unsigned)nn), dim3(256), 0, s, absmax, nb, offset, nested, q8,
                     host_mids8());
  return hipGetLastError();
}

hipError_t launch_dequant(const QPtrs& q, int64_t n_out, int64_t k_in, uint16_t* out,
                          hipStream_t s) {
  const int64_t nwords = n_out * k_in / 8;
  const dim3 grid((unsigned)((nwords + 255) / 256));
  hipLaunchKernelGGL(k_dequant, grid, dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(q.packed), q.q8, q.nested, q.offset, nwords,
                     reinterpret_cast<uint4*>(out), host_tables());
  return hipGetLastError();
}

}  // namespace nf4s
