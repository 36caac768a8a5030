/*
 * nf4stream.h -- C ABI of the layer-streamed NF4 + LoRA hot path (MI355X, gfx950).
 *
 * Frozen decoder linears are stored as NF4 blockwise 4-bit weights with
 * double-quantised absmax (block 64, nested block 256, about 0.516 bytes per
 * parameter), dequantised on the GPU and contracted in bf16 with fp32
 * accumulation, forward y = x.W'^T + s.(x.A^T).B^T and backward
 * dx = dy.W' + du.A, with the rank-r LoRA gradients. Layer shards stream from
 * pinned host memory into a pool of 2..8 device slots on a side stream.
 *
 * Sources (web pages on the Soup tool's stream_layers feature), cited by page
 * title and section:
 *   [G]  "Soup layer-streamed NF4 training measured" (gate walkthrough):
 *        s1.3 resident-NF4 reference and the double-quant flag; s2.1 offline
 *        per-tensor quantisation, per-call weight reconstruction from slot
 *        bytes plus two shared tables, checkpointed layer body; s2.3
 *        deterministic quantiser; s2.4 bytes per weight and the two constant
 *        tables (asserted, never assumed); s2.5 zero-B adapter pitfall; s4.4
 *        no weight gradient for the frozen base.
 *   [E]  "Fine-Tune 8B Models on 4GB VRAM: Soup's Layer Streaming", section
 *        "The Principle of Layer Streaming": 2-8 VRAM buffers, prefetch of
 *        layer i+1 (forward) / i-1 (backward) on a dedicated stream, each
 *        layer read twice per step; the slot-aliasing gradient bug of NF4
 *        layers above ~165 MiB.
 *
 * Conventions for every function:
 *   - Return 0 (NF4S_OK) or a negative NF4S_E* code; nf4s_last_error() gives a
 *     thread-local message for the last failure. No exception crosses the ABI.
 *   - All arguments are validated on the host before anything is enqueued; on
 *     error nothing is launched and outputs are untouched. There is no
 *     fallback path: an unsupported case is an error, never a slower variant.
 *   - The caller owns every buffer, stream and event it passes. Device
 *     pointers are device (HBM) addresses; "host_pinned" pointers must come
 *     from hipHostMalloc (torch pin_memory). The library allocates no device
 *     memory; scratch comes in through (ws, ws_bytes), sized by
 *     nf4s_workspace_bytes(). Streams are hipStream_t passed as void*; 0 is the
 *     null stream. Calls are asynchronous on the given stream and never
 *     synchronise the device.
 *   - bf16 tensors are uint16_t bit patterns, row-major, contiguous.
 *   - Results do not depend on pointer values, on slot indices or on the
 *     pool size: the launch configuration is a function of the shapes only.
 */
#ifndef NF4STREAM_H
#define NF4STREAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define NF4S_OK 0
#define NF4S_EINVAL -1      /* null pointer, bad enum, non-finite scale, r out of range */
#define NF4S_ESHAPE -2      /* K_in % 64 != 0, odd element count, M/N <= 0, GEMM M > 2^23, size overflow */
#define NF4S_EALIGN -3      /* pointer not aligned (16 B for tensors, 256 B for shards/slots) */
#define NF4S_ETABLE -4      /* descriptor's table hash differs from the library's tables */
#define NF4S_EKEY -5        /* method / block / nested block / double-quant flag mismatch */
#define NF4S_ESLOT -6       /* slot too small, pool size outside [2, 8], unknown layer */
#define NF4S_ENOTPINNED -7  /* host source is not page-locked */
#define NF4S_EHIP -8        /* a HIP runtime call failed (message kept) */
#define NF4S_EWORKSPACE -9  /* workspace missing or smaller than nf4s_workspace_bytes() */

/* ---- format ------------------------------------------------------------- */
#define NF4S_METHOD_NF4 1
#define NF4S_BLOCK 64
#define NF4S_NESTED_BLOCK 256
#define NF4S_SECTION_ALIGN 256
#define NF4S_MAX_RANK 64

#define NF4S_DTYPE_F32 0
#define NF4S_DTYPE_BF16 1

/*
 * Where one quantised tensor W[n_out, k_in] lives inside a shard (a device or
 * host byte buffer). [G] s2.1/s2.4: uint8 packed codes, 8-bit absmax codes,
 * fp32 nested absmax, one fp32 offset. Offsets are bytes from the shard base
 * and are multiples of NF4S_SECTION_ALIGN.
 *   packed: uint8 [n_out*k_in/2], row-major, element 2j in the high nibble of
 *           byte j;
 *   q8:     uint8 [nb], nb = n_out*k_in/64, block b = elements [64b, 64b+64);
 *   nested: float [nn], nn = ceil(nb/256), nested block j = blocks [256j, 256j+256);
 *   offset: float [1], the mean of the fp32 absmax the q8 codes are centred on.
 * table_hash is FNV-1a-64 over the fp32 bytes of the NF4 table then the nested
 * table; a descriptor whose hash differs from nf4s_table_hash() is refused
 * ([G] s2.4: a per-weight table would silently dequantise with wrong constants).
 */
typedef struct nf4s_tensor_desc {
  int64_t n_out;
  int64_t k_in;
  int32_t method;        /* NF4S_METHOD_NF4 */
  int32_t blocksize;     /* NF4S_BLOCK */
  int32_t nested_block;  /* NF4S_NESTED_BLOCK */
  int32_t double_quant;  /* 1 ([G] s1.3: the flag must agree between sharder and reader) */
  uint64_t off_packed;
  uint64_t off_q8;
  uint64_t off_nested;
  uint64_t off_offset;
  uint64_t end;          /* first byte after this tensor's sections */
  uint64_t table_hash;
} nf4s_tensor_desc;

/* Library identification and the last error of the calling thread. */
const char* nf4s_version(void);
const char* nf4s_last_error(void);

/*
 * Payload bytes of one tensor, [G] s2.4: N/2 + ceil(N/64) + 4*ceil(N/16384) + 4
 * for N = n_out*k_in (about 0.516 bytes per parameter). Section padding is not
 * included (see nf4s_tensor_layout). Returns 0 for invalid shapes.
 */
uint64_t nf4_shard_bytes(int64_t n_out, int64_t k_in);

/*
 * Fill *out with the section offsets of a tensor placed at byte `base` of a
 * shard (base must be a multiple of 256); out->end is where the next tensor
 * may start. Errors: ESHAPE (k_in % 64, n_out <= 0), EALIGN (base), EINVAL.
 */
int nf4s_tensor_layout(int64_t n_out, int64_t k_in, uint64_t base, nf4s_tensor_desc* out);

/*
 * Copy out the library's code tables ([G] s2.4: 16 fp32 NF4 levels and 256
 * fp32 nested levels, ascending, shared by every tensor) and their hash.
 * The NF4 levels are normal quantiles (QLoRA section 3); the nested table is
 * the signed dynamic-tree map (8-bit Optimizers section 2). Either pointer may
 * be NULL.
 */
int nf4_code_tables(float* c4_16, float* c8_256);
uint64_t nf4s_table_hash(void);

/*
 * Scratch bytes an operation needs for the given shape (0 means none; ws may
 * then be NULL). op: NF4S_OP_QUANTIZE (n_out, k_in), NF4S_OP_LINEAR_FWD and
 * NF4S_OP_LINEAR_BWD (the packed activation plus split partials),
 * NF4S_OP_LINEAR_FWD_PACKED and NF4S_OP_LINEAR_BWD_PACKED (split partials
 * only), NF4S_OP_LORA_FWD and NF4S_OP_LORA_BWD (M, n_out, k_in; the adapter
 * sizes cover any rank up to NF4S_MAX_RANK). The value depends on shapes only.
 */
#define NF4S_OP_QUANTIZE 1
#define NF4S_OP_LINEAR_FWD 2
#define NF4S_OP_LINEAR_BWD 3
#define NF4S_OP_LORA_BWD 4
#define NF4S_OP_LORA_FWD 5
#define NF4S_OP_LINEAR_FWD_PACKED 6
#define NF4S_OP_LINEAR_BWD_PACKED 7
#define NF4S_OP_DENSE_FWD_PACKED 8   /* split partials of dense_linear_fwd_packed */
#define NF4S_OP_DENSE_BWD_PACKED 9   /* split partials of dense_linear_bwd_packed */
#define NF4S_OP_ATTENTION_BWD 10     /* M = tokens, n_out = heads, k_in = head_dim */
#define NF4S_OP_CROSS_ENTROPY 11     /* M = tokens (n_out, k_in ignored) */
int nf4s_workspace_bytes(int op, int64_t M, int64_t n_out, int64_t k_in, size_t* bytes);

/*
 * Offline NF4 double-quant of one tensor, [G] s2.1 (quantised once, one tensor
 * at a time, written as packed bytes plus sidecars) and s2.3 (deterministic).
 *   w_dev:     W[n_out, k_in] on the device, dtype NF4S_DTYPE_F32 or _BF16;
 *   shard_dev: device buffer receiving the sections at desc's offsets
 *              (desc from nf4s_tensor_layout, base 256-B aligned);
 *   status_dev: nullable device int32, set to 1 if W held a non-finite value
 *              (codes for such a tensor are meaningless), else left as is;
 *   ws:        nf4s_workspace_bytes(NF4S_OP_QUANTIZE) bytes.
 * Per 64-block: absmax, v = w/absmax (IEEE fp32 division), code = nearest NF4
 * level (ties to the lower code; all-zero block -> level 0). Offset = mean of
 * the absmax (exact sum, one fp64 division, rounded to fp32); nested absmax =
 * max |absmax - offset| over 256 blocks; q8 = nearest nested level of
 * (absmax - offset)/nested. Errors: EINVAL, ESHAPE, EALIGN, EKEY, EWORKSPACE.
 */
int nf4_quantize_shard(const void* w_dev, int dtype, int64_t n_out, int64_t k_in,
                       void* shard_dev, const nf4s_tensor_desc* desc, int32_t* status_dev,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantise one tensor to bf16, [G] s2.1 (NF4 weight rebuilt per call from
 * the streamed bytes and the two shared tables, bf16 compute):
 *   a'[b] = fp32(fp32(C8[q8[b]] * nested[b/256]) + offset)  (two roundings)
 *   W'[e] = bf16_rne(fp32(C4[code[e]] * a'[e/64]))
 * w_bf16_dev: uint16 [n_out, k_in]. Errors: EINVAL, EALIGN, ETABLE, EKEY.
 */
int nf4_dequant(const void* shard_dev, const nf4s_tensor_desc* d, uint16_t* w_bf16_dev,
                void* stream);

/*
 * Forward of a frozen NF4 linear with an optional LoRA adapter, [G] s2.1
 * (matmul over the NF4 weight with bf16 compute; LoRA r16 on the target
 * projections):  y = bf16( x.W'^T + scale * u.B^T ),  fp32 accumulation, W'
 * dequantised tile by tile on chip (never written to HBM).
 *   x:      bf16 [M, k_in];  y: bf16 [M, n_out];
 *   lora_u: nullable fp32 [M, r] = x.A^T from lora_fwd;
 *   lora_B: fp32 [n_out, r] (required iff lora_u is given); r in [1, 64];
 *   ws:     nf4s_workspace_bytes(NF4S_OP_LINEAR_FWD, M, n_out, k_in) bytes.
 * The LoRA term is contracted in bf16 on the matrix cores (u and scale*B
 * rounded to bf16). Errors: EINVAL, ESHAPE, EALIGN, ETABLE, EKEY, EWORKSPACE.
 */
int streamed_linear_fwd(const void* shard_dev, const nf4s_tensor_desc* d, const uint16_t* x,
                        int64_t M, uint16_t* y, const float* lora_u, const float* lora_B, int r,
                        float scale, void* ws, size_t ws_bytes, void* stream);

/*
 * streamed_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The same kernels and results, bit for
 * bit; their scratch (packed x and split partials) lives in a library-owned
 * device array of NF4S_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends. Arguments and errors as streamed_linear_fwd, plus EWORKSPACE when
 * nf4s_workspace_bytes(NF4S_OP_LINEAR_FWD, M, n_out, k_in) exceeds that size
 * (checked before anything is enqueued; e.g. every 8B projection up to
 * M = 2048 fits). Allocates nothing. All calls on one GPU share the array:
 * calls that overlap on one GPU (two streams, two host threads) race.
 */
#define NF4S_NOALLOC_SCRATCH_BYTES (64ull << 20)
int streamed_linear_fwd_noalloc(const void* shard_dev, const nf4s_tensor_desc* d, const uint16_t* x,
                                int64_t M, uint16_t* y, const float* lora_u, const float* lora_B,
                                int r, float scale, void* stream);

/*
 * Backward (input gradient only) of the same linear, [G] s4.4 (frozen base:
 * dL/dx and no dL/dW) and [E] (dL/dx needs W again, hence the second read):
 *   dx = bf16( dy.W' + du.A ),  fp32 accumulation.
 *   dy: bf16 [M, n_out];  dx: bf16 [M, k_in];
 *   lora_du: nullable fp32 [M, r] (= scale * dy.B, from lora_bwd);
 *   lora_A:  fp32 [r, k_in] (required iff lora_du is given).
 * Errors as streamed_linear_fwd. For both directions M * max(n_out, k_in)
 * must stay below 2^31 and the packed activation below 2^32 bytes.
 */
int streamed_linear_bwd(const void* shard_dev, const nf4s_tensor_desc* d, const uint16_t* dy,
                        int64_t M, uint16_t* dx, const float* lora_du, const float* lora_A,
                        int r, void* ws, size_t ws_bytes, void* stream);

/*
 * Activation packing. The matrix cores take their activation operand as
 * 16-byte fragments (lane l: row l%32 of a 32-row block, 8 contraction values
 * of a 16-wide block), so the GEMMs read it in that order: packed[(b*KB + s)
 * *64 + l] = the 16 bytes of row 32b + l%32, columns 16s + 8(l/32) .. +8,
 * with KB = 4*ceil(K/64), rows padded with zeros to a multiple of 256 and
 * columns to a multiple of 64. The unpacked linear calls pack into their
 * workspace on every call; a caller whose projections read the same input
 * (q, k and v; gate and up) packs it once and calls the _packed variants.
 *   nf4s_packed_activation_bytes: size of the packed form of a bf16 [M, K]
 *     matrix (0 for M <= 0 or K not a positive multiple of 8).
 *   nf4s_pack_activation: a bf16 [M, K] row-major (16-B aligned) -> packed
 *     (256-B aligned, at least packed_bytes). Errors: EINVAL, ESHAPE, EALIGN,
 *     EWORKSPACE.
 */
uint64_t nf4s_packed_activation_bytes(int64_t M, int64_t K);
int nf4s_pack_activation(const uint16_t* a, int64_t M, int64_t K, void* packed, size_t packed_bytes,
                         void* stream);

/*
 * streamed_linear_fwd / _bwd on an activation already packed with
 * nf4s_pack_activation (x with K = k_in; dy with K = n_out) for the same M.
 * ws: nf4s_workspace_bytes(NF4S_OP_LINEAR_FWD_PACKED / _BWD_PACKED) bytes
 * (zero when the contraction is not split). Results are bit-identical to the
 * unpacked calls. Errors as streamed_linear_fwd.
 */
int streamed_linear_fwd_packed(const void* shard_dev, const nf4s_tensor_desc* d,
                               const void* x_packed, int64_t M, uint16_t* y, const float* lora_u,
                               const float* lora_B, int r, float scale, void* ws, size_t ws_bytes,
                               void* stream);
int streamed_linear_bwd_packed(const void* shard_dev, const nf4s_tensor_desc* d,
                               const void* dy_packed, int64_t M, uint16_t* dx,
                               const float* lora_du, const float* lora_A, int r, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * Forward of n (1..3) NF4 linears of one shard that read the same input, in
 * one launch ([G] s2.1: q, k and v read the normed hidden state, as do gate
 * and up): for each i, ys[i] is streamed_linear_fwd_packed of descs[i] on
 * x_packed. One grid covers the column tiles of all n weights, so projections
 * too narrow to fill the chip alone (k and v under grouped-query attention)
 * share a launch, and the contraction is split for the group as a whole.
 *   descs:   host array of n descriptors of the shard, all with the same k_in;
 *   x_packed: nf4s_pack_activation of bf16 x [M, k_in] (256-B aligned);
 *   ys:      host array of n device pointers, bf16 [M, descs[i].n_out];
 *   lora_us, lora_Bs: nullable host arrays of n device pointers; entry i is
 *            fp32 [M, r] / [descs[i].n_out, r] or NULL in both (no adapter);
 *   ws:      nf4s_grouped_workspace_bytes(n, n_outs, k_in, M) bytes (zero
 *            when the contraction is not split).
 * Outputs equal the single calls' up to the grouping of the fp32 accumulation
 * (the group's split count may differ from a single weight's); deterministic.
 * Errors: EINVAL (n out of range, unpaired LoRA operands), ESHAPE (k_in
 * differs, sizes), EALIGN, ETABLE, EKEY, EWORKSPACE.
 */
int nf4s_grouped_workspace_bytes(int n, const int64_t* n_outs, int64_t k_in, int64_t M,
                                 size_t* bytes);

/*
 * The launch plan of streamed_linear_fwd_grouped (swiglu = 0; n = 1 is the
 * plan of streamed_linear_fwd_packed) or of streamed_linear_fwd_swiglu
 * (swiglu = 1, n = 2 equal widths) for these shapes: the output tile
 * (*tile_rows x *tile_cols; 512 x 128 is the one-wave-per-SIMD forward
 * kernel, 256 x 128 the general one; for the SwiGLU launch the columns count
 * gate and up together) and the split of the contraction (1 = none).
 * Host-only, depends on the shapes alone. Errors: EINVAL (NULL outputs, n
 * out of range, SwiGLU widths differ), ESHAPE (sizes; a SwiGLU launch that
 * would need a split).
 */
int nf4s_linear_fwd_plan(int n, const int64_t* n_outs, int64_t k_in, int64_t M, int swiglu,
                         int* tile_rows, int* tile_cols, int* splits);

/*
 * Forward into the residual stream (the o and down projections of a llama
 * layer, [G] s2.1): y as streamed_linear_fwd_packed writes it, and
 *   h_out = h_in + y        fp32 [M, n_out], y's bf16 values added in fp32
 * (h_in may be h_out). When the contraction is split the sum of the partials
 * writes both at once; otherwise a residual kernel follows the GEMM. The
 * results equal streamed_linear_fwd_packed followed by nf4s_residual_add bit
 * for bit. ws as for streamed_linear_fwd_packed. Errors: as there, and EINVAL
 * / EALIGN for h_in, h_out (16-byte aligned).
 */
int streamed_linear_fwd_residual(const void* shard_dev, const nf4s_tensor_desc* d,
                                 const void* x_packed, int64_t M, uint16_t* y, const float* lora_u,
                                 const float* lora_B, int r, float scale, const float* h_in,
                                 float* h_out, void* ws, size_t ws_bytes, void* stream);
int streamed_linear_fwd_grouped(const void* shard_dev, const nf4s_tensor_desc* descs, int n,
                                const void* x_packed, int64_t M, uint16_t* const* ys,
                                const float* const* lora_us, const float* const* lora_Bs, int r,
                                float scale, void* ws, size_t ws_bytes, void* stream);

/*
 * The gate and up projections of a llama MLP ([G] s2.1: the unmodified layer
 * body around the streamed linears, SwiGLU between them) as one launch whose
 * epilogue applies the activation:
 *   out = bf16( silu(g) * u ),  g = bf16(x.W'_gate^T + s.u_g.B_g^T),
 *                               u = bf16(x.W'_up^T + s.u_u.B_u^T),
 * silu(g) * u = g / (1 + e^-g) * u in fp32 -- the same bits as
 * streamed_linear_fwd_grouped on (gate, up) followed by nf4s_swiglu_fwd, with
 * half the output bytes and no g, u tensors.
 *   d_gate, d_up: descriptors of the shard, both width x k_in, width a
 *              multiple of 64;
 *   x_packed:  nf4s_pack_activation of bf16 x [M, k_in];
 *   out:       nullable bf16 [M, width]; out_packed: nullable, the same
 *              values in fragment order (nf4s_packed_activation_bytes(M,
 *              width) bytes, 256-B aligned; rows past M are not written),
 *              the input of the down projection; at least one is given;
 *   lora_us, lora_Bs: nullable host arrays of 2 device pointers (gate, up),
 *              as for streamed_linear_fwd_grouped.
 * Only shapes whose launch needs no split of the contraction are supported
 * (nf4s_swiglu_fused_supported returns 1; e.g. 8B widths at M >= 512); others
 * are refused with ESHAPE. No workspace. Errors: EINVAL, ESHAPE, EALIGN,
 * ETABLE, EKEY, EWORKSPACE (out_packed too small).
 */
int nf4s_swiglu_fused_supported(int64_t M, int64_t width, int64_t k_in);
int streamed_linear_fwd_swiglu(const void* shard_dev, const nf4s_tensor_desc* d_gate,
                               const nf4s_tensor_desc* d_up, const void* x_packed, int64_t M,
                               uint16_t* out, void* out_packed, size_t out_packed_bytes,
                               const float* const* lora_us, const float* const* lora_Bs, int r,
                               float scale, void* stream);

/*
 * Grouped backward ([G] s2.1 and s4.4: the input gradient of the layer's
 * normed input is the sum over the projections that read it, q, k and v, or
 * gate and up): for n in [1, 3] weights sharing k_in,
 *   dx = bf16( sum_i (dy_i.W'_i + du_i.A_i) )
 * as one contraction over the dy_i placed one after the other, rounded to
 * bf16 once (the sum of the single calls' outputs rounds each term).
 *   descs:     host array of n descriptors of the shard, all with the same
 *              k_in; with n > 1 every n_out a multiple of 64;
 *   dy_packed: host array of n device pointers, nf4s_pack_activation of bf16
 *              dy_i [M, descs[i].n_out] (256-B aligned);
 *   dx:        bf16 [M, k_in];
 *   lora_dus, lora_As: nullable host arrays of n device pointers; entry i is
 *              fp32 [M, r] / [r, k_in] or NULL in both (no adapter);
 *   ws:        nf4s_grouped_bwd_workspace_bytes(n, n_outs, k_in, M) bytes
 *              (fp32 partials of the split contraction; zero when unsplit).
 * Each weight's contraction is split on its own, so a workgroup reads one
 * weight; the partials of all weights are summed in a fixed order
 * (deterministic). A group of one equals streamed_linear_bwd_packed bit for
 * bit. Errors: EINVAL (n out of range, unpaired LoRA operands), ESHAPE
 * (k_in differs, n_out not a multiple of 64 in a group, sizes), EALIGN,
 * ETABLE, EKEY, EWORKSPACE.
 */
int nf4s_grouped_bwd_workspace_bytes(int n, const int64_t* n_outs, int64_t k_in, int64_t M,
                                     size_t* bytes);
int streamed_linear_bwd_grouped(const void* shard_dev, const nf4s_tensor_desc* descs, int n,
                                const void* const* dy_packed, int64_t M, uint16_t* dx,
                                const float* const* lora_dus, const float* const* lora_As, int r,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * LoRA down-projection, u = x.A^T in fp32 ([G] s2.1, adapter on q/v):
 *   x: bf16 [M, k_in]; A: fp32 [r, k_in] (16-byte aligned); u_out: fp32 [M, r];
 *   ws: nf4s_workspace_bytes(NF4S_OP_LORA_FWD, M, n_out, k_in) bytes (partials
 *       of the split contraction).
 * Runs on the matrix cores with A split into bf16 hi + lo parts (about 17
 * significant bits kept), fp32 accumulation. Deterministic (fixed reduction
 * order). Errors: EINVAL, ESHAPE, EALIGN, EWORKSPACE.
 */
int lora_fwd(const uint16_t* x, int64_t M, int64_t k_in, const float* A, int r, float* u_out,
             void* ws, size_t ws_bytes, void* stream);

/*
 * LoRA gradients for L with upstream dy ([G] s2.2 check 2: non-zero in every
 * layer; s2.5: with B = 0, dA is structurally zero):
 *   du_out = scale * dy.B        fp32 [M, r]
 *   dB    (+)= scale * dy^T.u     fp32 [n_out, r]
 *   dA    (+)= du^T.x             fp32 [r, k_in]
 * x: bf16 [M, k_in]; dy: bf16 [M, n_out]; u: fp32 [M, r] (x.A^T);
 * B: fp32 [n_out, r]. accumulate = 0 overwrites dA/dB, 1 adds to them.
 * The fp32 operand of each product (B, u, du) is split into bf16 hi + lo
 * parts for the matrix cores; accumulation is fp32.
 * ws: nf4s_workspace_bytes(NF4S_OP_LORA_BWD, M, n_out, k_in) bytes.
 * Reductions run in a fixed order, so results are bit-reproducible.
 * Errors: EINVAL, ESHAPE, EALIGN, EWORKSPACE.
 */
int lora_bwd(const uint16_t* x, const uint16_t* dy, const float* u, int64_t M, int64_t k_in,
             int64_t n_out, const float* B, int r, float scale, float* dA, float* dB,
             float* du_out, int accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped adapters ([G] s2.1: the q and v adapters of a layer read the same
 * normed input x): n in [1, NF4S_MAX_LORA_GROUP] adapters in one launch of
 * each kernel. The array arguments are host arrays of n device pointers (or,
 * for n_outs, of n output widths); entry i is what the single call of adapter
 * i takes, with the same alignment and shape rules:
 *   lora_fwd_grouped: u_out[i] = x.A[i]^T;
 *   lora_bwd_grouped: du_out[i], dB[i], dA[i] as lora_bwd(x, dy[i], u[i],
 *     n_outs[i], B[i]), one scale and accumulate flag for the group.
 * Results are bit-identical to the n single calls (same kernels and
 * reduction order per adapter).
 * ws: nf4s_lora_grouped_workspace_bytes(n, n_outs, k_in, M, backward) bytes
 * (the sum of the single calls' workspaces; the forward ignores n_outs'
 * values but takes the array). Errors: EINVAL (n out of range, NULL arrays),
 * ESHAPE, EALIGN, EWORKSPACE.
 */
#define NF4S_MAX_LORA_GROUP 3
int nf4s_lora_grouped_workspace_bytes(int n, const int64_t* n_outs, int64_t k_in, int64_t M,
                                      int backward, size_t* bytes);
int lora_fwd_grouped(const uint16_t* x, int64_t M, int64_t k_in, const float* const* A, int n, int r,
                     float* const* u_out, void* ws, size_t ws_bytes, void* stream);
int lora_bwd_grouped(const uint16_t* x, const uint16_t* const* dy, const float* const* u, int64_t M,
                     int64_t k_in, const int64_t* n_outs, const float* const* B, int n, int r,
                     float scale, float* const* dA, float* const* dB, float* const* du_out,
                     int accumulate, void* ws, size_t ws_bytes, void* stream);

/* ---- the decoder around the streamed linears ----------------------------
 *
 * [G] s2.1-s2.2 and s4.3: a llama decoder (SmolLM2-135M, Llama-3.1-8B) whose
 * seven layer projections are the streamed NF4 linears; the embedding table
 * and the lm_head stay resident and unquantised in bf16, every layer body is
 * checkpointed (recomputed in the backward), compute is bf16. The operations
 * follow llama's published definitions (the pages name the architecture, not
 * the formulas). Storage: bf16 for every tensor that feeds a product or the
 * attention; fp32 for the residual stream h, norm statistics, softmax
 * statistics and the adapters' optimiser state. All arithmetic is fp32, every
 * reduction runs in a fixed order (results are bit-reproducible), and calls
 * are asynchronous on `stream`. Tokens are rows t = b*S + s (batch-major).
 */

/*
 * Resident bf16 linear (the lm_head, [G] s4.3: embed/lm_head stay bf16):
 *   fwd: y[M, n_out] = bf16(x.W^T),  bwd: dx[M, k_in] = bf16(dy.W),
 * fp32 accumulation on the matrix cores, W bf16 [n_out, k_in] row-major,
 * activations packed with nf4s_pack_activation (x: K = k_in; dy: K = n_out).
 * Shapes as the streamed linears (k_in % 64 == 0, n_out % 8 == 0).
 * ws: nf4s_workspace_bytes(NF4S_OP_DENSE_FWD_PACKED / _BWD_PACKED) bytes.
 * Errors: EINVAL, ESHAPE, EALIGN, EWORKSPACE, EHIP.
 */
int dense_linear_fwd_packed(const uint16_t* w, int64_t n_out, int64_t k_in, const void* x_packed,
                            int64_t M, uint16_t* y, void* ws, size_t ws_bytes, void* stream);
int dense_linear_bwd_packed(const uint16_t* w, int64_t n_out, int64_t k_in, const void* dy_packed,
                            int64_t M, uint16_t* dx, void* ws, size_t ws_bytes, void* stream);

/*
 * Token embedding ([G] s4.3: resident bf16 embed_tokens, a lookup):
 * h[t, :] = fp32(table[ids[t], :]). table bf16 [vocab, hidden]; ids int64 [T]
 * (device); h fp32 [T, hidden]. An id outside [0, vocab) yields a NaN row
 * (the table is never read out of bounds). Errors: EINVAL, ESHAPE, EALIGN.
 */
int nf4s_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int64_t* ids, int64_t T,
               float* h, void* stream);

/*
 * Packed outputs. The producers of GEMM inputs below take an optional
 * `packed` pointer (NULL: none): the bf16 result [T, width] is then also
 * written in the MFMA fragment order of nf4s_pack_activation (256-B aligned,
 * nf4s_packed_activation_bytes(T, width) bytes), ready for the _packed GEMM
 * calls without a separate packing pass. It equals nf4s_pack_activation's
 * output except in the rows past T, which are left as they were (the GEMMs
 * compute them but never store them); the columns past width up to the next
 * multiple of 64 are written as zeros.
 *
 * (nf4s_attention_fwd writes o this way too, width = heads*head_dim.)
 *
 * RMSNorm: rstd[t] = 1/sqrt(mean_j x[t,j]^2 + eps), y = bf16(x * rstd * w).
 * x fp32 [T, H]; w fp32 [H]; y bf16 [T, H] (and packed, see above); rstd fp32
 * [T] (kept for the backward); H a multiple of 8, x, w, y, dys and dh 16-byte
 * aligned. Backward: with g = w * (dys[0] + ... + dys[n_dy-1]) (n_dy bf16
 * [T, H] gradients of y, 1..3, summed in fp32 in that order),
 *   d = rstd * g - x * rstd^3 * mean_j(g * x),
 * written to dh (accumulate = 0) or added to it (accumulate = 1). dys is a
 * host array of device pointers. y (nullable) receives the resulting dh as
 * bf16 [T, H] (what nf4s_to_bf16 would write), packed (nullable, needs y)
 * also in fragment order, so the next GEMM's input leaves with the norm's
 * backward. Errors: EINVAL, ESHAPE, EALIGN.
 */
int nf4s_rmsnorm_fwd(const float* x, const float* w, int64_t T, int64_t H, float eps, uint16_t* y,
                     float* rstd, void* packed, void* stream);
int nf4s_rmsnorm_bwd(const uint16_t* const* dys, int n_dy, const float* x, const float* w,
                     const float* rstd, int64_t T, int64_t H, int accumulate, float* dh,
                     uint16_t* y, void* packed, void* stream);

/*
 * Rotary embedding, rotate-half form, in place on bf16 x [T, heads*head_dim]:
 * row t is position t % S; pair (j, j + d/2) of each head is rotated by the
 * angle (t % S) * theta^(-2j/d) (inverse = 1: by minus that angle, which is
 * the backward of the rotation); the angle, its sine and cosine are fp64,
 * the rotation fp32, results rounded to bf16. head_dim a multiple of 8, at
 * most 256; T a multiple of S; x 8-byte aligned. Errors: EINVAL, ESHAPE,
 * EALIGN.
 */
int nf4s_rope(uint16_t* x, int64_t T, int64_t S, int heads, int head_dim, double theta, int inverse,
              void* stream);
/* The same on queries q [T, q_heads*head_dim] and keys k [T, k_heads*head_dim]
 * in one launch (each element as nf4s_rope rotates it). q_packed / k_packed
 * (nullable, 256-B aligned, nf4s_packed_activation_bytes(T, heads*head_dim)
 * bytes): the rotated tensors also as nf4s_pack_activation lays them out, for
 * the GEMMs that read them next (the backward's dq and dk). */
int nf4s_rope_pair(uint16_t* q, int q_heads, uint16_t* k, int k_heads, int64_t T, int64_t S,
                   int head_dim, double theta, int inverse, void* q_packed, void* k_packed,
                   void* stream);

/*
 * Causal softmax attention with grouped KV heads (head h reads KV head
 * h / (heads / kv_heads)), scale 1/sqrt(head_dim), fp32 online softmax:
 *   q bf16 [B*S, heads*d]; k, v bf16 [B*S, kv_heads*d];
 *   o bf16 [B*S, heads*d]; o_f32 nullable fp32 [B*S, heads*d] (the same
 *   output before rounding, needed by the backward); lse fp32 [B, heads, S]
 *   (log-sum-exp of each row's scaled scores).
 * Backward from dout bf16 [B*S, heads*d]: dq bf16 (like q), dk, dv bf16 (like
 * k, summed over the heads of a group in head order), with
 * dS = P * (dP - rowsum(P * dP)) and rowsum(P * dP) = dout . o_f32.
 * ws: nf4s_workspace_bytes(NF4S_OP_ATTENTION_BWD, B*S, heads, head_dim)
 * bytes (rowsum and per-head fp32 partials of dk, dv, summed per group in
 * head order). The products run on the matrix cores with P and dS split into
 * bf16 high + low parts (about 16 significant bits), fp32 accumulation.
 * dv_packed (nullable, 256-B aligned, nf4s_packed_activation_bytes(B*S,
 * kv_heads*d) bytes): dv also as nf4s_pack_activation lays it out, for the v
 * projection's backward. head_dim in {32, 64, 128}; heads % kv_heads == 0;
 * every tensor argument except lse 16-byte aligned. Errors: EINVAL, ESHAPE,
 * EALIGN, EWORKSPACE.
 */
int nf4s_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                       int64_t S, int heads, int kv_heads, int head_dim, uint16_t* o, float* o_f32,
                       float* lse, void* packed, void* stream);
int nf4s_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o_f32,
                       const uint16_t* dout, const float* lse, int64_t B, int64_t S, int heads,
                       int kv_heads, int head_dim, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                       void* dv_packed, void* ws, size_t ws_bytes, void* stream);

/*
 * SwiGLU: out = bf16(silu(g) * u), silu(z) = z / (1 + e^-z); backward from ds:
 * dg = bf16(ds * u * s * (1 + g * (1 - s))), du = bf16(ds * g * s), s the
 * logistic of g. All bf16 [T, width], width a multiple of 8, 16-byte aligned;
 * packed outputs as above (out; dg and du). dg (du) may be NULL when
 * dg_packed (du_packed) is given: only the packed form is then written.
 * Errors: EINVAL, ESHAPE, EALIGN.
 */
int nf4s_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t T, int64_t width, uint16_t* out,
                    void* packed, void* stream);
int nf4s_swiglu_bwd(const uint16_t* ds, const uint16_t* g, const uint16_t* u, int64_t T,
                    int64_t width, uint16_t* dg, uint16_t* du, void* dg_packed, void* du_packed,
                    void* stream);

/* Residual update out[i] = h[i] + y[i] (fp32 h and out, bf16 y; out may be
 * h), and rounding y = bf16(x) of an fp32 [T, width] matrix (width a multiple
 * of 8, 16-byte aligned; packed output as above). */
int nf4s_residual_add(const float* h, const uint16_t* y, int64_t n, float* out, void* stream);
int nf4s_to_bf16(const float* x, int64_t T, int64_t width, uint16_t* y, void* packed, void* stream);

/*
 * Mean token cross-entropy over bf16 logits [T, V] against int64 targets [T]:
 * loss (device fp32 [1]) = mean_t (logsumexp(z_t) - z_t[target_t]), and
 * dlogits bf16 [T, V] = (softmax(z_t) - onehot(target_t)) / T. A target
 * outside [0, V) makes the loss NaN. ws: nf4s_workspace_bytes(
 * NF4S_OP_CROSS_ENTROPY, T, 0, 0) bytes. Errors: EINVAL, ESHAPE, EALIGN,
 * EWORKSPACE.
 */
int nf4s_cross_entropy(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                       float* loss, uint16_t* dlogits, void* ws, size_t ws_bytes, void* stream);

/*
 * Preference step (DPO), "Soup v0.72.4 technical analysis" s3.1-3.3: the
 * reference model is the same streamed base with the adapters off, the policy
 * the base with them on; no second model. Sequences are rows of S tokens,
 * ordered chosen, rejected per pair; mask fp32 [T] weights the tokens that
 * count (the response).
 *   nf4s_token_nll:  nll[t] = logsumexp(z_t) - z_t[target_t] (fp32 [T]; NaN
 *                    for a target outside [0, V)); logits bf16 [T, V].
 *   nf4s_dpo_loss:   lp / lr = -sum_t mask * nll over each sequence (policy /
 *                    reference), delta = beta ((lp_c - lr_c) - (lp_r - lr_r)),
 *                    loss (device fp32 [1]) = -mean over pairs of
 *                    log sigmoid(delta) (the DPO objective of Rafailov et al.
 *                    2023, the pages name the method, not its formula);
 *                    seq_coef fp32 [2 pairs] = dL/d(masked nll sum) of each
 *                    sequence. Fixed-order sums.
 *   nf4s_logit_grad: dlogits[t] = bf16(seq_coef[t/S] * mask[t] *
 *                    (softmax(z_t) - onehot(target_t))), the logits' gradient.
 * Errors: EINVAL, ESHAPE, EALIGN.
 */
int nf4s_token_nll(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V, float* nll,
                   void* stream);
int nf4s_dpo_loss(const float* nll_policy, const float* nll_ref, const float* mask, int64_t pairs,
                  int64_t S, float beta, float* loss, float* seq_coef, void* stream);
int nf4s_logit_grad(const uint16_t* logits, const int64_t* targets, const float* seq_coef,
                    const float* mask, int64_t T, int64_t S, int64_t V, uint16_t* dlogits,
                    void* stream);

/*
 * One AdamW step on fp32 parameters (the adapters' optimiser; [G] s4.1 uses a
 * paged 8-bit AdamW, whose paging is an allocation strategy): with t = step
 * (from 1), m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2,
 * p = p (1 - lr wd) - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps).
 * p, m, v updated in place; g read. Errors: EINVAL, ESHAPE, EALIGN.
 */
int nf4s_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1,
               float beta2, float eps, float weight_decay, int64_t step, void* stream);

/*
 * Enqueue one layer-shard copy host -> device slot on copy_stream, [E] (a
 * dedicated stream prefetches the next layer while the current one computes):
 * wait wait_slot_free (nullable; the event recorded after the slot's last
 * reader), hipMemcpyAsync H2D, record record_ready (nullable).
 * Errors: EINVAL, EALIGN (slot), ESLOT (bytes > slot_bytes), ENOTPINNED
 * (host_pinned_src not page-locked: a pageable source would make the copy
 * synchronous), EHIP.
 */
int layer_prefetch(void* slot_dev, size_t slot_bytes, const void* host_pinned_src, size_t bytes,
                   void* copy_stream, void* wait_slot_free, void* record_ready);

/* Events for layer_prefetch and cross-stream ordering (timing disabled). */
int nf4s_event_create(void** event_out);
int nf4s_event_destroy(void* event);
int nf4s_event_record(void* event, void* stream);
int nf4s_stream_wait_event(void* stream, void* event);

/*
 * Slot pool: n_slots device slots that layer shards stream through, [E]
 * (2..8 buffers, default 2; forward prefetches i+1, backward i-1). The pool
 * tracks which layer each slot holds and orders every overwrite after the
 * slot's last reader with a per-slot free event, and every read after its copy
 * with a per-slot ready event -- the ordering whose absence corrupted
 * gradients but not the forward pass in the pages' slot-aliasing bug ([E],
 * the NF4 layers above ~165 MiB). A layer still resident in a slot is not
 * copied again.
 *   nf4s_pool_create:   slots are caller-owned device buffers (256-B aligned,
 *                       slot_bytes > 0 each, pairwise disjoint: EINVAL if two
 *                       overlap); n_slots in [2, 8]; copy and compute are
 *                       distinct streams.
 *   nf4s_pool_set_layer: register layer `layer`'s pinned host shard; a copy
 *                       of an earlier registration still in a slot is
 *                       dropped (ESLOT while a reader holds it).
 *   nf4s_pool_prefetch: reserve `layer` for its next acquire: if it is
 *                       resident or in flight it is only marked reserved;
 *                       otherwise it is copied into a slot no reader holds
 *                       and no earlier prefetch reserved (an empty slot
 *                       first, else the least recently used one). When every
 *                       slot no reader holds is reserved, nothing is copied
 *                       (the acquire copies) and NF4S_OK is returned; ESLOT
 *                       if every slot is held. A caller may thus prefetch up
 *                       to n_slots - 1 layers ahead without evicting a layer
 *                       it prefetched earlier.
 *   nf4s_pool_acquire:  make `layer` resident (copying now if needed, into an
 *                       empty, else unreserved, else reserved slot, least
 *                       recently used first), make the compute stream wait
 *                       for it, return its slot. It may block the calling
 *                       thread until that slot's copy is enqueued (below).
 *   nf4s_pool_release:  record the slot's free event on the compute stream
 *                       after the last kernel that reads it was enqueued.
 *   nf4s_pool_stats:    copies issued and bytes copied so far.
 * prefetch, acquire and release return ESLOT for a layer index that was never
 * registered (negative included).
 * Copies are enqueued on the copy stream by a host thread the pool owns, in
 * the order they were asked for, each once the free event it follows has
 * completed on the device (so the copy stream never waits on a pending
 * event, which costs tens of microseconds per copy); the host sources must
 * stay valid until then. A failure of that thread is returned by the next
 * prefetch, acquire or release. nf4s_pool_destroy lets it enqueue what was
 * asked, then stops it.
 *   nf4s_pool_set_debug: NF4S_POOL_POISON_ON_RELEASE makes every release also
 *                       overwrite the slot with 0xFF bytes (NaN block scales)
 *                       on the copy stream, ordered after the free event as a
 *                       copy would be, and forget the layer it held; a kernel
 *                       that read a slot after its release would then compute
 *                       with NaN weights. For tests of the slot ordering; it
 *                       adds one fill and, later, one copy per release.
 */
typedef struct nf4s_pool nf4s_pool;
int nf4s_pool_create(int n_slots, void* const* slots, size_t slot_bytes, void* copy_stream,
                     void* compute_stream, nf4s_pool** out);
int nf4s_pool_destroy(nf4s_pool* pool);
int nf4s_pool_set_layer(nf4s_pool* pool, int layer, const void* host_pinned_src, size_t bytes);
int nf4s_pool_prefetch(nf4s_pool* pool, int layer);
int nf4s_pool_acquire(nf4s_pool* pool, int layer, void** slot_dev_out);
int nf4s_pool_release(nf4s_pool* pool, int layer);
int nf4s_pool_stats(const nf4s_pool* pool, uint64_t* copies, uint64_t* bytes);
#define NF4S_POOL_POISON_ON_RELEASE 1
int nf4s_pool_set_debug(nf4s_pool* pool, int flags);

#ifdef __cplusplus
}
#endif
#endif /* NF4STREAM_H */
