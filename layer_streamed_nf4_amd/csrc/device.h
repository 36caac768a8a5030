// Device helpers shared by the kernels: bf16 packing, scale decode, NF4 decode.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4s {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Two fp32 values -> one dword of two bf16, round to nearest even
// (v_cvt_pk_bf16_f32); `lo` lands in the low half (the lower address).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// SwiGLU of one element: silu(g) * u = g / (1 + e^-g) * u in fp32 (the
// decoder's MLP activation), the quotient as g times the hardware reciprocal
// (v_rcp_f32, within 1 ulp) -- one definition for the elementwise kernel and
// the GEMM epilogue that fuses it, so both give the same bits.
__device__ __forceinline__ float swiglu_val(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Block scale: a' = fp32(fp32(C8[q8] * nested) + offset), two separate
// roundings (never a fused multiply-add).
__device__ __forceinline__ float decode_scale(float c8v, float nested, float offset) {
  return __fadd_rn(__fmul_rn(c8v, nested), offset);
}

// 4-bit code of element e (0..7) of a little-endian packed word: byte e/2,
// even elements in the high nibble.
__device__ __forceinline__ uint32_t nib(uint32_t word, int e) {
  return (word >> (8 * (e >> 1) + ((e & 1) ? 0 : 4))) & 0xFu;
}

// Eight NF4 codes of one packed word times one scale -> four bf16 pairs.
__device__ __forceinline__ void dequant_word(uint32_t word, float a, const float* c4,
                                             uint32_t out[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float v0 = __fmul_rn(c4[nib(word, 2 * p)], a);
    const float v1 = __fmul_rn(c4[nib(word, 2 * p + 1)], a);
    out[p] = pack_bf16x2(v0, v1);
  }
}

// Byte offset of the 16 bytes holding row m, columns c .. c+7 (c a multiple of
// 8) of a bf16 [M, K] matrix in MFMA fragment order (the layout k_frag_pack
// writes): fragment (m/32, c/16), lane m%32 + 32*((c/8)%2); kb = 16-wide
// blocks per 32-row block, 4 * ceil(K/64).
__device__ __forceinline__ int64_t frag_offset(int64_t m, int64_t c, int64_t kb) {
  return (((m >> 5) * kb + (c >> 4)) * 64 + (m & 31) + 32 * ((c >> 3) & 1)) * 16;
}

// Zero the padding of row m past K (up to the next multiple of 64), which
// the GEMMs contract with zero weights and so must not be NaN.
__device__ __forceinline__ void frag_zero_tail(uint8_t* packed, int64_t m, int64_t K, int64_t kb) {
  for (int64_t c = K; c < kb * 16; c += 8)
    *reinterpret_cast<uint4*>(packed + frag_offset(m, c, kb)) = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace nf4s
