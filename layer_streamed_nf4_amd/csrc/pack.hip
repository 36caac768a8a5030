// Activation packing for the fused NF4 GEMMs.
//
// The 32x32x16 bf16 MFMA takes its activation operand per lane as 16 bytes:
// lane l holds row l%32 of a 32-row block and 8 contraction values of a
// 16-wide block. Read straight from a row-major matrix those loads put
// consecutive lanes in different rows, which the vector memory path serves at
// a quarter of its rate, so the GEMMs read a copy in fragment order instead:
// fragment (b, s) = 1 KB at offset (b * KB + s) * 1024, lane after lane, with
// KB = 4 * ceil(K/64), rows zero-padded to a multiple of PACK_ROWS (256) and
// the contraction to a multiple of PACK_COLS (64). The activations are the
// bf16 inputs of the frozen linears (gate walkthrough "Soup layer-streamed
// NF4 training measured", section 2.1: bf16 compute); packing changes their
// order only.
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int TILES_PER_BLOCK = 4;  // (32-row block, 64-wide step) tiles per workgroup
constexpr int TILE_STRIDE = 144;    // bytes per staged row (128 + 16 pad: conflict-free reads)

// Workgroup w packs tiles 4w .. 4w+3, i.e. four consecutive 64-wide steps of
// one 32-row block: it reads 8 lanes per 128-byte row segment (whole 512-byte
// runs per row), transposes through LDS and writes 16 KB of consecutive
// fragments. All four loads of a thread are in flight together.
__global__ __launch_bounds__(256) void k_frag_pack(const uint16_t* __restrict__ a, int64_t M,
                                                   int64_t K, int64_t steps, int64_t ntiles,
                                                   uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TILES_PER_BLOCK][32 * TILE_STRIDE];
  const int t = threadIdx.x;
  const int r = t >> 3, c = t & 7;
  u32x4 v[TILES_PER_BLOCK];
#pragma unroll
  for (int u = 0; u < TILES_PER_BLOCK; ++u) {
    const int64_t id = (int64_t)blockIdx.x * TILES_PER_BLOCK + u;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (id < ntiles) {
      const int64_t row = 32 * (id / steps) + r;
      const int64_t k = 64 * (id % steps) + 8 * c;
      if (row < M && k < K) v[u] = *reinterpret_cast<const u32x4*>(a + row * K + k);
    }
  }
#pragma unroll
  for (int u = 0; u < TILES_PER_BLOCK; ++u)
    *reinterpret_cast<u32x4*>(&tile[u][r * TILE_STRIDE + c * 16]) = v[u];
  __syncthreads();
  const int f = t >> 6, lane = t & 63;  // 16-wide block within the step, and its lane
#pragma unroll
  for (int u = 0; u < TILES_PER_BLOCK; ++u) {
    const int64_t id = (int64_t)blockIdx.x * TILES_PER_BLOCK + u;
    if (id >= ntiles) break;
    const int64_t b = id / steps, st = id % steps;
    const u32x4 w = *reinterpret_cast<const u32x4*>(
        &tile[u][(lane & 31) * TILE_STRIDE + (2 * f + (lane >> 5)) * 16]);
    *reinterpret_cast<u32x4*>(out + ((b * 4 * steps + 4 * st + f) * 64 + lane) * 16) = w;
  }
}

// Writes the 32-bit pattern v (little-endian, repeated) over `bytes` bytes at p
// (16-byte aligned): 16-byte stores for the bulk, byte stores for a ragged
// tail (the slot pool's poison mode).
__global__ __launch_bounds__(256) void k_fill_u32(uint8_t* __restrict__ p, int64_t bytes, uint32_t v) {
  const int64_t n = bytes / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = t; i < n; i += stride) reinterpret_cast<u32x4*>(p)[i] = u32x4{v, v, v, v};
  if (t == 0)
    for (int64_t b = n * 16; b < bytes; ++b) p[b] = (uint8_t)(v >> (8 * (b % 4)));
}

}  // namespace

hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t v, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const int64_t words = (int64_t)(bytes / 16);
  int64_t blocks = (words + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint8_t*>(p),
                     (int64_t)bytes, v);
  return hipGetLastError();
}

size_t packed_activation_bytes(int64_t M, int64_t K) {
  return (size_t)((M + PACK_ROWS - 1) / PACK_ROWS * PACK_ROWS) *
         (size_t)((K + PACK_COLS - 1) / PACK_COLS * PACK_COLS) * 2;
}

hipError_t launch_pack(const uint16_t* a, int64_t M, int64_t K, uint8_t* packed, hipStream_t s) {
  const int64_t steps = (K + PACK_COLS - 1) / PACK_COLS;
  const int64_t ntiles = (M + PACK_ROWS - 1) / PACK_ROWS * (PACK_ROWS / 32) * steps;
  const int64_t blocks = (ntiles + TILES_PER_BLOCK - 1) / TILES_PER_BLOCK;
  hipLaunchKernelGGL(k_frag_pack, dim3((unsigned)blocks), dim3(256), 0, s, a, M, K, steps, ntiles,
                     packed);
  return hipGetLastError();
}

}  // namespace nf4s
