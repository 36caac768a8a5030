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
// The NF4 code search of the quantiser (quant.hip): bucket b of v / m, of
// width 1/128 from -1, counts code[b] thresholds below it; b_mid[i] is the fp64
// midpoint between threshold i and the next fp32 above it (b_mid[15] = +inf).
// ok: every threshold lies at least 1/64 of a bucket width from a bucket edge.
struct Buckets4 {
  double b_mid[16];
  uint8_t code[260];
  int ok;
};

// Sets the calling thread's last-error message (nf4s_last_error) and returns code.
int set_error(int code, const char* fmt, ...);

// Host-side tables, computed once at first use (see tables.cpp).
const Tables& host_tables();
const Mids4& host_mids4();
const Mids8& host_mids8();
const Buckets4& host_buckets4();
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

// Weights one grouped forward launch covers (q, k and v read the same input).
constexpr int GEMM_MAX_SEG = 3;

// Launch configuration of the dequant GEMMs, a function of the shape only.
struct GemmPlan {
  int bm, bn;        // output tile
  int splits;        // split of the contraction (1 = none)
  int64_t kc_chunk;   // contraction elements per split (multiple of 64)
  size_t frag_bytes;  // packed activation (start of the workspace of the unpacked calls)
  size_t part_bytes;  // fp32 partials when splits > 1
  size_t ws_bytes;    // frag_bytes + part_bytes
};
// fwd_nf4: the forward NF4 kernel (512-row tiles); else k_gemm (256-row tiles).
GemmPlan plan_gemm(int64_t M, int64_t n_cols, int64_t k_contract, bool fwd_nf4);
// The same for a grouped forward of nseg weights of n_cols[i] outputs.
GemmPlan plan_gemm_grouped(int64_t M, const int64_t* n_cols, int nseg, int64_t k_contract,
                           bool fwd_nf4);
size_t packed_activation_bytes(int64_t M, int64_t K);

// Kernel launchers (return hipError_t of the launch).
hipError_t launch_quantize(const void* w, int dtype, int64_t n_out, int64_t k_in,
                           uint8_t* packed, uint8_t* q8, float* nested, float* offset,
                           int32_t* status, void* ws, hipStream_t s);
size_t quantize_ws_bytes(int64_t n_out, int64_t k_in);

hipError_t launch_dequant(const QPtrs& q, int64_t n_out, int64_t k_in, uint16_t* out,
                          hipStream_t s);

hipError_t launch_pack(const uint16_t* a, int64_t M, int64_t K, uint8_t* packed, hipStream_t s);
// Writes the 32-bit pattern v over `bytes` bytes at p (16-byte aligned).
hipError_t launch_fill_u32(void* p, size_t bytes, uint32_t v, hipStream_t s);
hipError_t launch_linear_packed(bool backward, const QPtrs& q, int64_t n_out, int64_t k_in,
                                const uint8_t* a_packed, int64_t M, uint16_t* out,
                                const float* lora_l, const float* lora_r, int r, float scale,
                                void* part_ws, hipStream_t s);
// The forward with the residual stream: y as launch_linear_packed writes it,
// and h_out = h_in + y (fp32 [M, n_out]), summed with the split partials or,
// unsplit, by k_residual_add.
hipError_t launch_linear_fwd_residual(const QPtrs& q, int64_t n_out, int64_t k_in,
                                      const uint8_t* x_packed, int64_t M, uint16_t* y,
                                      const float* lora_u, const float* lora_B, int r, float scale,
                                      const float* h_in, float* h_out, void* part_ws, hipStream_t s);
// Forward of nseg (<= GEMM_MAX_SEG) NF4 linears reading the same packed
// activation, in one launch (lora_us / lora_Bs entries may be null).
// gate + up forward with the SwiGLU epilogue: out = bf16(silu(g) * u) for
// g, u the two weights' bf16 outputs (q[0] gate, q[1] up, both width x k_in);
// out and out_packed (fragment order) nullable. swiglu_fused_ok: the launch
// needs no split of the contraction (the only case it supports).
bool swiglu_fused_ok(int64_t M, int64_t width, int64_t k_in);
// The fused launch's tile (rows, gate + up columns); false where unsupported.
bool swiglu_tiles(int64_t M, int64_t width, int64_t k_in, int* bm, int* bn);
hipError_t launch_linear_swiglu_fwd(const QPtrs* q, int64_t width, int64_t k_in, const uint8_t* x_packed,
                                    int64_t M, uint16_t* out, uint8_t* out_packed,
                                    const float* const* lora_us, const float* const* lora_Bs, int r,
                                    float scale, hipStream_t s);
hipError_t launch_linear_grouped_fwd(const QPtrs* q, int nseg, const int64_t* n_outs, int64_t k_in,
                                     const uint8_t* x_packed, int64_t M, uint16_t* const* ys,
                                     const float* const* lora_us, const float* const* lora_Bs,
                                     int r, float scale, void* part_ws, hipStream_t s);

// Backward of n (<= GEMM_MAX_SEG) NF4 linears that read the same input:
// dx = sum_j (dy_j . W'_j + du_j . A_j), one contraction over the n weights
// (every n_outs[j] a multiple of 64 when n > 1) rounded to bf16 once;
// dy_packed[j] is dy_j packed (lora_dus / lora_As entries may be null).
struct BwdGroupPlan {
  int bm;                          // tile rows: 256 (k_gemm) or 512 (k_gemm_bwd512)
  int cmax;                        // contraction steps of the longest split
  int splits[GEMM_MAX_SEG];        // splits of each weight's contraction
  int64_t kc_chunk[GEMM_MAX_SEG];  // contraction rows per split
  int total;                       // all splits (partials when > 1)
  size_t part_bytes;               // fp32 partials [total, M, k_in]
};
BwdGroupPlan plan_bwd_grouped(int64_t M, const int64_t* n_outs, int n, int64_t k_in);
hipError_t launch_linear_grouped_bwd(const QPtrs* q, int n, const int64_t* n_outs, int64_t k_in,
                                     const uint8_t* const* dy_packed, int64_t M, uint16_t* dx,
                                     const float* const* lora_dus, const float* const* lora_As,
                                     int r, void* part_ws, hipStream_t s);

// The same GEMMs with a dense bf16 weight w[n_out, k_in] (the resident lm_head).
hipError_t launch_dense_packed(bool backward, const uint16_t* w, int64_t n_out, int64_t k_in,
                               const uint8_t* a_packed, int64_t M, uint16_t* out, void* part_ws,
                               hipStream_t s);

hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t k_in, const float* A, int r,
                           float* u, void* ws, hipStream_t s);
size_t lora_fwd_ws_bytes(int64_t M, int64_t k_in, int r);
hipError_t launch_lora_bwd(const uint16_t* x, const uint16_t* dy, const float* u, int64_t M,
                           int64_t k_in, int64_t n_out, const float* B, int r, float scale,
                           float* dA, float* dB, float* du, int accumulate, void* ws,
                           hipStream_t s);
size_t lora_bwd_ws_bytes(int64_t M, int64_t n_out, int r);
// n (<= 3) adapters reading one input x in one launch of each kernel; their
// workspaces (as above) follow each other in ws
hipError_t launch_lora_fwd_grouped(const uint16_t* x, int64_t M, int64_t k_in, const float* const* A,
                                   int n, int r, float* const* u, void* ws, hipStream_t s);
hipError_t launch_lora_bwd_grouped(const uint16_t* x, const uint16_t* const* dy,
                                   const float* const* u, int64_t M, int64_t k_in,
                                   const int64_t* n_out, const float* const* B, int n, int r,
                                   float scale, float* const* dA, float* const* dB,
                                   float* const* du, int accumulate, void* ws, hipStream_t s);

// Decoder kernels (decoder.hip).
hipError_t launch_embed(const uint16_t* E, int64_t V, const int64_t* ids, int64_t T, int64_t H,
                        float* h, hipStream_t s);
// packed (nullable): y also in MFMA fragment order, as k_frag_pack writes it
// except for rows past T (left as they are; the GEMMs never store them)
hipError_t launch_rmsnorm_fwd(const float* x, const float* w, int64_t T, int64_t H, float eps,
                              uint16_t* y, float* rstd, void* packed, hipStream_t s);
// y, packed (nullable): the resulting dh also as bf16 (and in fragment order)
hipError_t launch_rmsnorm_bwd(const uint16_t* const* dys, int n_dy, const float* x, const float* w,
                              const float* rstd, int64_t T, int64_t H, int accumulate, float* dh,
                              uint16_t* y, void* packed, hipStream_t s);
hipError_t launch_rope(uint16_t* x, int64_t T, int64_t S, int heads, int d, double theta,
                       int inverse, hipStream_t s);
// x1 and x2 (heads1 / heads2 heads, x2 nullable) in one launch; p1 / p2
// (nullable): the results also in MFMA fragment order
hipError_t launch_rope_pair(uint16_t* x1, int heads1, uint16_t* x2, int heads2, int64_t T, int64_t S,
                            int d, double theta, int inverse, void* p1, void* p2, hipStream_t s);
// packed (nullable): o also in fragment order (width H*D), as the producers above
hipError_t launch_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                int64_t S, int H, int Hkv, int D, uint16_t* o, float* o_f32,
                                float* lse, void* packed, hipStream_t s);
size_t attention_bwd_ws_bytes(int64_t B, int64_t S, int H, int D);
hipError_t launch_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* o_f32, const uint16_t* dout, const float* lse,
                                int64_t B, int64_t S, int H, int Hkv, int D, uint16_t* dq,
                                uint16_t* dk, uint16_t* dv, void* dv_packed, void* ws, hipStream_t s);
hipError_t launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t T, int64_t W,
                             uint16_t* out, void* packed, hipStream_t s);
hipError_t launch_swiglu_bwd(const uint16_t* ds, const uint16_t* g, const uint16_t* u, int64_t T,
                             int64_t W, uint16_t* dg, uint16_t* du, void* dg_packed,
                             void* du_packed, hipStream_t s);
hipError_t launch_residual_add(const float* h, const uint16_t* y, int64_t n, float* out,
                               hipStream_t s);
hipError_t launch_f32_to_bf16(const float* x, int64_t T, int64_t W, uint16_t* y, void* packed,
                              hipStream_t s);
size_t cross_entropy_ws_bytes(int64_t T);
hipError_t launch_cross_entropy(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                                float* loss, uint16_t* dlogits, void* ws, hipStream_t s);
hipError_t launch_token_nll(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                            float* nll, hipStream_t s);
hipError_t launch_dpo(const float* nll_p, const float* nll_r, const float* mask, int64_t pairs,
                      int64_t S, float beta, float* loss, float* coef, hipStream_t s);
hipError_t launch_logit_grad(const uint16_t* logits, const int64_t* targets, const float* coef,
                             const float* mask, int64_t T, int64_t S, int64_t V, uint16_t* dlogits,
                             hipStream_t s);
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float b1,
                        float b2, float eps, float wd, int64_t step, hipStream_t s);

}  // namespace nf4s
