// Offline NF4 double-quant sharder and the standalone dequantiser.
//
// Gate walkthrough ("Soup layer-streamed NF4 training measured"), section 2.1:
// each tensor is quantised once, offline, blockwise 64, into packed 4-bit codes
// plus the absmax sidecar, which double quant replaces by 8-bit codes, a nested
// absmax per 256 blocks and one offset; section 2.3: the result is byte-for-byte
// deterministic. Three passes, all with fixed reduction orders:
//   1. per 64-block absmax, NF4 codes, nibble packing (16 lanes per block);
//   2. the offset = mean of the absmax, summed exactly (double-double, fixed
//      chunks over many workgroups then a fixed tree over their partials)
//      then divided once in fp64 and rounded to fp32;
//   3. per 256-block nested absmax of (absmax - offset) and the 8-bit codes.
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

template <int DTYPE>
__global__ __launch_bounds__(256) void k_absmax_codes(const void* __restrict__ w, int64_t nb,
                                                       uint8_t* __restrict__ packed,
                                                       float* __restrict__ absmax,
                                                       int32_t* __restrict__ status, Mids4 mids) {
  __shared__ float s_m[15];
  if (threadIdx.x < 15) s_m[threadIdx.x] = mids.m[threadIdx.x];
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid / kLanesPerBlock;
  const int lane = (int)(gid % kLanesPerBlock);
  if (blk >= nb) return;
  const int64_t e0 = blk * 64 + lane * 4;
  float v[4];
  if (DTYPE == NF4S_DTYPE_F32) {
    const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + e0);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + e0);
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xFFFF0000u);
  }
  bool finite = true;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    finite = finite && __builtin_isfinite(v[i]);
    m = fmaxf(m, fabsf(v[i]));
  }
  // max over the 16 lanes of this block (exact, order-free)
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kLanesPerBlock));
  if (!finite && status) {
    volatile int32_t* st = status;
    *st = 1;
  }
  int c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float n = (m > 0.0f) ? __fdiv_rn(v[i], m) : 0.0f;
    c[i] = code_of<16>(n, s_m);
  }
  const uint32_t b0 = (uint32_t)((c[0] << 4) | c[1]);
  const uint32_t b1 = (uint32_t)((c[2] << 4) | c[3]);
  reinterpret_cast<uint16_t*>(packed)[e0 / 4] = (uint16_t)(b0 | (b1 << 8));
  if (lane == 0) absmax[blk] = m;
}

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

// The offset sum in two fixed-order passes: workgroup g adds the contiguous
// chunk [g*chunk, (g+1)*chunk) of the absmax (each thread a strided subset,
// then a fixed tree over the workgroup), and one workgroup adds the partials
// in a fixed tree and divides once. The partition is a function of nb only,
// so the result is the same on every run; every addition is double-double.
constexpr int kPartThreads = 256;
constexpr int kFinalThreads = 1024;
constexpr int64_t kChunk = 4096;          // absmax values per first-pass workgroup
constexpr int kMaxParts = kFinalThreads;  // first-pass workgroups at most

int64_t offset_parts(int64_t nb) {
  int64_t g = (nb + kChunk - 1) / kChunk;
  return g < 1 ? 1 : (g > kMaxParts ? kMaxParts : g);
}

template <int T>
__device__ __forceinline__ void dd_tree(double* s_hi, double* s_lo, int t) {
  for (int half = T / 2; half >= 1; half >>= 1) {
    if (t < half) {
      double h = s_hi[t], l = s_lo[t];
      dd_add(h, l, s_hi[t + half], s_lo[t + half]);
      s_hi[t] = h;
      s_lo[t] = l;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kPartThreads) void k_offset_part(const float* __restrict__ absmax,
                                                               int64_t nb, int64_t chunk,
                                                               double2* __restrict__ part) {
  __shared__ double s_hi[kPartThreads];
  __shared__ double s_lo[kPartThreads];
  const int t = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = b0 + chunk < nb ? b0 + chunk : nb;
  double hi = 0.0, lo = 0.0;
  for (int64_t i = b0 + t; i < b1; i += kPartThreads) dd_add(hi, lo, (double)absmax[i], 0.0);
  s_hi[t] = hi;
  s_lo[t] = lo;
  __syncthreads();
  dd_tree<kPartThreads>(s_hi, s_lo, t);
  if (t == 0) part[blockIdx.x] = make_double2(s_hi[0], s_lo[0]);
}

__global__ __launch_bounds__(kFinalThreads) void k_offset_final(const double2* __restrict__ part,
                                                                 int parts, int64_t nb,
                                                                 float* __restrict__ offset) {
  __shared__ double s_hi[kFinalThreads];
  __shared__ double s_lo[kFinalThreads];
  const int t = threadIdx.x;
  const double2 v = t < parts ? part[t] : make_double2(0.0, 0.0);
  s_hi[t] = v.x;
  s_lo[t] = v.y;
  __syncthreads();
  dd_tree<kFinalThreads>(s_hi, s_lo, t);
  if (t == 0) {
    const double sum = s_hi[0] + s_lo[0];  // one rounding of the exact sum
    offset[0] = (float)(sum / (double)nb);
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
  const int64_t nb = n_out * k_in / 64;
  float* absmax = static_cast<float*>(ws);
  const int64_t threads = nb * kLanesPerBlock;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (dtype == NF4S_DTYPE_F32)
    hipLaunchKernelGGL(k_absmax_codes<NF4S_DTYPE_F32>, grid, dim3(256), 0, s, w, nb, packed, absmax,
                       status, host_mids4());
  else
    hipLaunchKernelGGL(k_absmax_codes<NF4S_DTYPE_BF16>, grid, dim3(256), 0, s, w, nb, packed,
                       absmax, status, host_mids4());
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t parts = offset_parts(nb);
  const int64_t chunk = (nb + parts - 1) / parts;
  double2* part = reinterpret_cast<double2*>(static_cast<uint8_t*>(ws) + absmax_bytes(nb));
  hipLaunchKernelGGL(k_offset_part, dim3((unsigned)parts), dim3(kPartThreads), 0, s, absmax, nb, chunk,
                     part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_offset_final, dim3(1), dim3(kFinalThreads), 0, s, part, (int)parts, nb, offset);
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
