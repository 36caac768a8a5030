// Internal declarations shared by the host API and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/nf4stream.h"

namespace nf4s {

// The code tables as kernel arguments (by value; 1.1 KB of kernarg space).
struct Tables {
  float c4[16];
  float c8[256];
};
struct Mids4 {
  float m[15];
};
struct Mids8 {
  float m[255];
};

// Host-side tables, computed once at first use (see tables.cpp).
const Tables& host_tables();
const Mids4& host_mids4();
const Mids8& host_mids8();
uint64_t host_table_hash();

// Pointers into one quantised tensor (resolved from shard base + descriptor).
struct QPtrs {
  const uint8_t* packed;
  const uint8_t* q8;
  const float* nested;
  const float* offset;
};

// Packed activation layout shared by the packer (pack.hip) and the GEMMs
// (gemm.hip): 1 KB fragments of (32 rows x 16 contraction values), rows padded
// to a multiple of PACK_ROWS, contraction to a multiple of PACK_COLS.
constexpr int PACK_ROWS = 256;
constexpr int PACK_COLS = 64;
constexpr int FRAG_BYTES = 1024;

// Launch configuration of the dequant GEMMs, a function of the shape only.
struct GemmPlan {
  int bm, bn;        // output tile
  int splits;        // split of the contraction (1 = none)
  int64_t kc_chunk;   // contraction elements per split (multiple of 64)
  size_t frag_bytes;  // packed activation (start of the workspace of the unpacked calls)
  size_t part_bytes;  // fp32 partials when splits > 1
  size_t ws_bytes;    // frag_bytes + part_bytes
};
GemmPlan plan_gemm(int64_t M, int64_t n_cols, int64_t k_contract);
size_t packed_activation_bytes(int64_t M, int64_t K);

// Kernel launchers (return hipError_t of the launch).
hipError_t launch_quantize(const void* w, int dtype, int64_t n_out, int64_t k_in,
                           uint8_t* packed, uint8_t* q8, float* nested, float* offset,
                           int32_t* status, void* ws, hipStream_t s);
size_t quantize_ws_bytes(int64_t n_out, int64_t k_in);

hipError_t launch_dequant(const QPtrs& q, int64_t n_out, int64_t k_in, uint16_t* out,
                          hipStream_t s);

hipError_t launch_pack(const uint16_t* a, int64_t M, int64_t K, uint8_t* packed, hipStream_t s);
hipError_t launch_linear_packed(bool backward, const QPtrs& q, int64_t n_out, int64_t k_in,
                                const uint8_t* a_packed, int64_t M, uint16_t* out,
                                const float* lora_l, const float* lora_r, int r, float scale,
                                void* part_ws, hipStream_t s);

hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t k_in, const float* A, int r,
                           float* u, void* ws, hipStream_t s);
size_t lora_fwd_ws_bytes(int64_t M, int64_t k_in, int r);
hipError_t launch_lora_bwd(const uint16_t* x, const uint16_t* dy, const float* u, int64_t M,
                           int64_t k_in, int64_t n_out, const float* B, int r, float scale,
                           float* dA, float* dB, float* du, int accumulate, void* ws,
                           hipStream_t s);
size_t lora_bwd_ws_bytes(int64_t M, int64_t n_out, int r);

}  // namespace nf4s
