// Host side of the C ABI: argument validation (before anything is enqueued),
// descriptor and table-key checks, dispatch to the kernels, events, the
// layer prefetch and the slot pool. No device memory is allocated here.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "common.h"

using namespace nf4s;

namespace {

// Rows of a GEMM operand: 256-row tiles keep the grid's y dimension far below
// its limit of 65535.
constexpr int64_t kMaxRows = 1ll << 23;

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

}  // namespace

int nf4s::set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(NF4S_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Shapes the kernels support: n_out a positive multiple of 8 (16-byte rows of
// bf16 activations), k_in a positive multiple of 64 (whole NF4 blocks per row),
// element count below 2^40.
int check_shape(int64_t n_out, int64_t k_in) {
  if (n_out <= 0 || k_in <= 0) return fail(NF4S_ESHAPE, "n_out=%lld k_in=%lld must be positive", (long long)n_out, (long long)k_in);
  if (k_in % 64) return fail(NF4S_ESHAPE, "k_in=%lld is not a multiple of 64", (long long)k_in);
  if (n_out % 8) return fail(NF4S_ESHAPE, "n_out=%lld is not a multiple of 8", (long long)n_out);
  if (n_out > (1ll << 26) || k_in > (1ll << 26) || n_out * k_in > (1ll << 40))
    return fail(NF4S_ESHAPE, "tensor too large");
  return NF4S_OK;
}

int check_desc(const nf4s_tensor_desc* d) {
  if (!d) return fail(NF4S_EINVAL, "descriptor is NULL");
  int rc = check_shape(d->n_out, d->k_in);
  if (rc) return rc;
  if (d->method != NF4S_METHOD_NF4 || d->blocksize != NF4S_BLOCK ||
      d->nested_block != NF4S_NESTED_BLOCK || d->double_quant != 1)
    return fail(NF4S_EKEY,
                "descriptor key mismatch: method=%d block=%d nested=%d double_quant=%d "
                "(library: NF4, 64, 256, 1)",
                d->method, d->blocksize, d->nested_block, d->double_quant);
  if (d->table_hash != host_table_hash())
    return fail(NF4S_ETABLE, "descriptor table hash %016llx differs from library tables %016llx",
                (unsigned long long)d->table_hash, (unsigned long long)host_table_hash());
  nf4s_tensor_desc ref;
  const uint64_t base = d->off_packed;
  if (base % NF4S_SECTION_ALIGN) return fail(NF4S_EALIGN, "packed section not 256-B aligned");
  if (nf4s_tensor_layout(d->n_out, d->k_in, base, &ref)) return NF4S_ESHAPE;
  if (ref.off_q8 != d->off_q8 || ref.off_nested != d->off_nested ||
      ref.off_offset != d->off_offset || ref.end != d->end)
    return fail(NF4S_EKEY, "descriptor section offsets do not follow the shard layout");
  return NF4S_OK;
}

QPtrs resolve(const void* shard, const nf4s_tensor_desc* d) {
  const uint8_t* b = static_cast<const uint8_t*>(shard);
  QPtrs q;
  q.packed = b + d->off_packed;
  q.q8 = b + d->off_q8;
  q.nested = reinterpret_cast<const float*>(b + d->off_nested);
  q.offset = reinterpret_cast<const float*>(b + d->off_offset);
  return q;
}

int check_ptr(const void* p, const char* name, uintptr_t align = 16) {
  if (!p) return fail(NF4S_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(NF4S_EALIGN, "%s is not %u-byte aligned", name, (unsigned)align);
  return NF4S_OK;
}

int check_rank(int r) {
  if (r < 1 || r > NF4S_MAX_RANK) return fail(NF4S_EINVAL, "rank r=%d outside [1, %d]", r, NF4S_MAX_RANK);
  return NF4S_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return NF4S_OK;
  if (!ws || have < need)
    return fail(NF4S_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? have : 0);
  if (!aligned(ws, 256)) return fail(NF4S_EALIGN, "workspace not 256-byte aligned");
  return NF4S_OK;
}

int check_pinned(const void* p) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(NF4S_ENOTPINNED, "host source %p is not page-locked (%s)", p, hipGetErrorString(e));
  }
  if (attr.type != hipMemoryTypeHost)
    return fail(NF4S_ENOTPINNED, "source %p is not page-locked host memory (type %d)", p, (int)attr.type);
  return NF4S_OK;
}

}  // namespace

extern "C" {

const char* nf4s_version(void) { return "nf4stream 0.1 gfx950"; }
const char* nf4s_last_error(void) { return g_err.c_str(); }

uint64_t nf4_shard_bytes(int64_t n_out, int64_t k_in) {
  if (n_out <= 0 || k_in <= 0) return 0;
  const uint64_t n = (uint64_t)n_out * (uint64_t)k_in;
  if (n % 2) return 0;
  const uint64_t nb = (n + 63) / 64;
  const uint64_t nn = (nb + 255) / 256;
  return n / 2 + nb + 4 * nn + 4;
}

int nf4s_tensor_layout(int64_t n_out, int64_t k_in, uint64_t base, nf4s_tensor_desc* out) {
  if (!out) return fail(NF4S_EINVAL, "out is NULL");
  int rc = check_shape(n_out, k_in);
  if (rc) return rc;
  if (base % NF4S_SECTION_ALIGN) return fail(NF4S_EALIGN, "base %llu not 256-byte aligned", (unsigned long long)base);
  const uint64_t n = (uint64_t)n_out * (uint64_t)k_in;
  const uint64_t nb = n / 64;
  const uint64_t nn = (nb + 255) / 256;
  nf4s_tensor_desc d;
  memset(&d, 0, sizeof d);
  d.n_out = n_out;
  d.k_in = k_in;
  d.method = NF4S_METHOD_NF4;
  d.blocksize = NF4S_BLOCK;
  d.nested_block = NF4S_NESTED_BLOCK;
  d.double_quant = 1;
  d.off_packed = base;
  d.off_q8 = round_up(d.off_packed + n / 2, NF4S_SECTION_ALIGN);
  d.off_nested = round_up(d.off_q8 + nb, NF4S_SECTION_ALIGN);
  d.off_offset = round_up(d.off_nested + 4 * nn, NF4S_SECTION_ALIGN);
  d.end = round_up(d.off_offset + 4, NF4S_SECTION_ALIGN);
  d.table_hash = host_table_hash();
  *out = d;
  return NF4S_OK;
}

int nf4_code_tables(float* c4_16, float* c8_256) {
  const Tables& t = host_tables();
  if (c4_16) memcpy(c4_16, t.c4, sizeof t.c4);
  if (c8_256) memcpy(c8_256, t.c8, sizeof t.c8);
  return NF4S_OK;
}

uint64_t nf4s_table_hash(void) { return host_table_hash(); }

int nf4s_workspace_bytes(int op, int64_t M, int64_t n_out, int64_t k_in, size_t* bytes) {
  if (!bytes) return fail(NF4S_EINVAL, "bytes is NULL");
  if (op == NF4S_OP_ATTENTION_BWD || op == NF4S_OP_CROSS_ENTROPY) {
    if (M <= 0 || M > kMaxRows) return fail(NF4S_ESHAPE, "M=%lld out of range", (long long)M);
    if (op == NF4S_OP_CROSS_ENTROPY) {
      *bytes = cross_entropy_ws_bytes(M);
      return NF4S_OK;
    }
    if (n_out <= 0 || n_out > 1024) return fail(NF4S_ESHAPE, "heads=%lld out of range", (long long)n_out);
    if (k_in != 32 && k_in != 64 && k_in != 128)
      return fail(NF4S_ESHAPE, "head_dim=%lld not one of 32, 64, 128", (long long)k_in);
    *bytes = attention_bwd_ws_bytes(1, M, (int)n_out, (int)k_in);
    return NF4S_OK;
  }
  int rc = check_shape(n_out, k_in);
  if (rc) return rc;
  switch (op) {
    case NF4S_OP_QUANTIZE:
      *bytes = quantize_ws_bytes(n_out, k_in);
      return NF4S_OK;
    case NF4S_OP_LINEAR_FWD:
    case NF4S_OP_LINEAR_BWD:
    case NF4S_OP_LINEAR_FWD_PACKED:
    case NF4S_OP_LINEAR_BWD_PACKED:
    case NF4S_OP_DENSE_FWD_PACKED:
    case NF4S_OP_DENSE_BWD_PACKED: {
      if (M <= 0 || M > kMaxRows) return fail(NF4S_ESHAPE, "M=%lld out of range", (long long)M);
      const bool bwd = op == NF4S_OP_LINEAR_BWD || op == NF4S_OP_LINEAR_BWD_PACKED ||
                       op == NF4S_OP_DENSE_BWD_PACKED;
      const bool dense = op == NF4S_OP_DENSE_FWD_PACKED || op == NF4S_OP_DENSE_BWD_PACKED;
      const GemmPlan p = plan_gemm(M, bwd ? k_in : n_out, bwd ? n_out : k_in, !bwd && !dense);
      const bool packed = op != NF4S_OP_LINEAR_FWD && op != NF4S_OP_LINEAR_BWD;
      *bytes = packed ? p.part_bytes : p.ws_bytes;
      return NF4S_OK;
    }
    case NF4S_OP_LORA_FWD:
      if (M <= 0) return fail(NF4S_ESHAPE, "M=%lld must be positive", (long long)M);
      *bytes = lora_fwd_ws_bytes(M, k_in, NF4S_MAX_RANK);
      return NF4S_OK;
    case NF4S_OP_LORA_BWD:
      if (M <= 0) return fail(NF4S_ESHAPE, "M=%lld must be positive", (long long)M);
      *bytes = lora_bwd_ws_bytes(M, n_out, NF4S_MAX_RANK);
      return NF4S_OK;
    default:
      return fail(NF4S_EINVAL, "unknown op %d", op);
  }
}

int nf4_quantize_shard(const void* w_dev, int dtype, int64_t n_out, int64_t k_in, void* shard_dev,
                       const nf4s_tensor_desc* desc, int32_t* status_dev, void* ws,
                       size_t ws_bytes, void* stream) {
  int rc;
  if (dtype != NF4S_DTYPE_F32 && dtype != NF4S_DTYPE_BF16) return fail(NF4S_EINVAL, "dtype %d", dtype);
  if ((rc = check_shape(n_out, k_in))) return rc;
  if ((rc = check_desc(desc))) return rc;
  if (desc->n_out != n_out || desc->k_in != k_in)
    return fail(NF4S_ESHAPE, "descriptor shape %lldx%lld differs from %lldx%lld",
                (long long)desc->n_out, (long long)desc->k_in, (long long)n_out, (long long)k_in);
  if ((rc = check_ptr(w_dev, "w_dev"))) return rc;
  if ((rc = check_ptr(shard_dev, "shard_dev", 256))) return rc;
  if ((rc = check_ws(ws, ws_bytes, quantize_ws_bytes(n_out, k_in)))) return rc;
  uint8_t* b = static_cast<uint8_t*>(shard_dev);
  hipError_t e = launch_quantize(w_dev, dtype, n_out, k_in, b + desc->off_packed, b + desc->off_q8,
                                 reinterpret_cast<float*>(b + desc->off_nested),
                                 reinterpret_cast<float*>(b + desc->off_offset), status_dev, ws,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "quantize launch");
}

int nf4_dequant(const void* shard_dev, const nf4s_tensor_desc* d, uint16_t* w_bf16_dev, void* stream) {
  int rc;
  if ((rc = check_desc(d))) return rc;
  if ((rc = check_ptr(shard_dev, "shard_dev", 256))) return rc;
  if ((rc = check_ptr(w_bf16_dev, "w_bf16_dev"))) return rc;
  hipError_t e = launch_dequant(resolve(shard_dev, d), d->n_out, d->k_in, w_bf16_dev,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "dequant launch");
}

// Packed activations are addressed with 32-bit offsets.
static int check_packed_shape(int64_t M, int64_t K) {
  if (M <= 0 || M > kMaxRows) return fail(NF4S_ESHAPE, "M=%lld out of range", (long long)M);
  if (K <= 0 || K % 8) return fail(NF4S_ESHAPE, "K=%lld must be a positive multiple of 8", (long long)K);
  if (packed_activation_bytes(M, K) >= (1ull << 32))
    return fail(NF4S_ESHAPE, "packed activation of %lldx%lld exceeds 32-bit offsets", (long long)M,
                (long long)K);
  return NF4S_OK;
}

// Shared validation of the linear calls; fills the plan.
static int linear_checks(bool bwd, const void* shard_dev, const nf4s_tensor_desc* d, int64_t M,
                         uint16_t* out, const float* lora_l, const float* lora_r, int r,
                         float scale, GemmPlan* plan) {
  int rc;
  if ((rc = check_desc(d))) return rc;
  if (M <= 0 || M > kMaxRows) return fail(NF4S_ESHAPE, "M=%lld out of range", (long long)M);
  // the kernels address outputs and packed weights with 32-bit offsets
  const int64_t widest = d->n_out > d->k_in ? d->n_out : d->k_in;
  if (M * widest >= (1ll << 31) || d->n_out * d->k_in >= (1ll << 33))
    return fail(NF4S_ESHAPE, "M=%lld with a %lldx%lld weight exceeds 32-bit offsets", (long long)M,
                (long long)d->n_out, (long long)d->k_in);
  if ((rc = check_packed_shape(M, bwd ? d->n_out : d->k_in))) return rc;
  if ((rc = check_ptr(shard_dev, "shard_dev", 256))) return rc;
  if ((rc = check_ptr(out, bwd ? "dx" : "y"))) return rc;
  if ((lora_l == nullptr) != (lora_r == nullptr))
    return fail(NF4S_EINVAL, "LoRA operands must be given together");
  if (lora_l) {
    if ((rc = check_rank(r))) return rc;
    if ((rc = check_ptr(lora_l, bwd ? "lora_du" : "lora_u", 4))) return rc;
    if ((rc = check_ptr(lora_r, bwd ? "lora_A" : "lora_B", 4))) return rc;
    if (!std::isfinite(scale)) return fail(NF4S_EINVAL, "scale is not finite");
  }
  *plan = plan_gemm(M, bwd ? d->k_in : d->n_out, bwd ? d->n_out : d->k_in, !bwd);
  return NF4S_OK;
}

static int linear_common(bool bwd, const void* shard_dev, const nf4s_tensor_desc* d,
                         const uint16_t* a, int64_t M, uint16_t* out, const float* lora_l,
                         const float* lora_r, int r, float scale, void* ws, size_t ws_bytes,
                         void* stream) {
  int rc;
  GemmPlan p;
  if ((rc = linear_checks(bwd, shard_dev, d, M, out, lora_l, lora_r, r, scale, &p))) return rc;
  if ((rc = check_ptr(a, bwd ? "dy" : "x"))) return rc;
  if ((rc = check_ws(ws, ws_bytes, p.ws_bytes))) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* packed = static_cast<uint8_t*>(ws);
  hipError_t e = launch_pack(a, M, bwd ? d->n_out : d->k_in, packed, st);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  e = launch_linear_packed(bwd, resolve(shard_dev, d), d->n_out, d->k_in, packed, M, out, lora_l,
                           lora_r, lora_l ? r : 0, scale, packed + p.frag_bytes, st);
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "linear launch");
}

static int linear_packed(bool bwd, const void* shard_dev, const nf4s_tensor_desc* d,
                         const void* a_packed, int64_t M, uint16_t* out, const float* lora_l,
                         const float* lora_r, int r, float scale, void* ws, size_t ws_bytes,
                         void* stream) {
  int rc;
  GemmPlan p;
  if ((rc = linear_checks(bwd, shard_dev, d, M, out, lora_l, lora_r, r, scale, &p))) return rc;
  if ((rc = check_ptr(a_packed, bwd ? "dy_packed" : "x_packed", 256))) return rc;
  if (p.part_bytes && (rc = check_ws(ws, ws_bytes, p.part_bytes))) return rc;
  hipError_t e = launch_linear_packed(bwd, resolve(shard_dev, d), d->n_out, d->k_in,
                                      static_cast<const uint8_t*>(a_packed), M, out, lora_l, lora_r,
                                      lora_l ? r : 0, scale, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "linear launch");
}

uint64_t nf4s_packed_activation_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 8) return 0;
  return packed_activation_bytes(M, K);
}

int nf4s_pack_activation(const uint16_t* a, int64_t M, int64_t K, void* packed, size_t packed_bytes,
                         void* stream) {
  int rc;
  if ((rc = check_packed_shape(M, K))) return rc;
  if ((rc = check_ptr(a, "a"))) return rc;
  if ((rc = check_ptr(packed, "packed", 256))) return rc;
  const size_t need = packed_activation_bytes(M, K);
  if (packed_bytes < need)
    return fail(NF4S_EWORKSPACE, "packed buffer of %zu bytes needed, %zu given", need, packed_bytes);
  hipError_t e = launch_pack(a, M, K, static_cast<uint8_t*>(packed), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "pack launch");
}

int streamed_linear_fwd(const void* shard_dev, const nf4s_tensor_desc* d, const uint16_t* x,
                        int64_t M, uint16_t* y, const float* lora_u, const float* lora_B, int r,
                        float scale, void* ws, size_t ws_bytes, void* stream) {
  return linear_common(false, shard_dev, d, x, M, y, lora_u, lora_B, r, scale, ws, ws_bytes, stream);
}

int streamed_linear_bwd(const void* shard_dev, const nf4s_tensor_desc* d, const uint16_t* dy,
                        int64_t M, uint16_t* dx, const float* lora_du, const float* lora_A, int r,
                        void* ws, size_t ws_bytes, void* stream) {
  return linear_common(true, shard_dev, d, dy, M, dx, lora_du, lora_A, r, 1.0f, ws, ws_bytes, stream);
}

int streamed_linear_fwd_packed(const void* shard_dev, const nf4s_tensor_desc* d,
                               const void* x_packed, int64_t M, uint16_t* y, const float* lora_u,
                               const float* lora_B, int r, float scale, void* ws, size_t ws_bytes,
                               void* stream) {
  return linear_packed(false, shard_dev, d, x_packed, M, y, lora_u, lora_B, r, scale, ws, ws_bytes,
                       stream);
}

int streamed_linear_fwd_residual(const void* shard_dev, const nf4s_tensor_desc* d,
                                 const void* x_packed, int64_t M, uint16_t* y, const float* lora_u,
                                 const float* lora_B, int r, float scale, const float* h_in,
                                 float* h_out, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  GemmPlan p;
  if ((rc = linear_checks(false, shard_dev, d, M, y, lora_u, lora_B, r, scale, &p))) return rc;
  if ((rc = check_ptr(x_packed, "x_packed", 256))) return rc;
  if ((rc = check_ptr(h_in, "h_in")) || (rc = check_ptr(h_out, "h_out"))) return rc;
  if (p.part_bytes && (rc = check_ws(ws, ws_bytes, p.part_bytes))) return rc;
  hipError_t e = launch_linear_fwd_residual(resolve(shard_dev, d), d->n_out, d->k_in,
                                            static_cast<const uint8_t*>(x_packed), M, y, lora_u, lora_B,
                                            lora_u ? r : 0, scale, h_in, h_out, ws,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "linear launch");
}

int streamed_linear_bwd_packed(const void* shard_dev, const nf4s_tensor_desc* d,
                               const void* dy_packed, int64_t M, uint16_t* dx,
                               const float* lora_du, const float* lora_A, int r, void* ws,
                               size_t ws_bytes, void* stream) {
  return linear_packed(true, shard_dev, d, dy_packed, M, dx, lora_du, lora_A, r, 1.0f, ws,
                       ws_bytes, stream);
}

static int check_group(int n, const int64_t* n_outs, int64_t k_in, int64_t M) {
  if (n < 1 || n > GEMM_MAX_SEG)
    return fail(NF4S_EINVAL, "group of %d weights (1..%d allowed)", n, GEMM_MAX_SEG);
  if (!n_outs) return fail(NF4S_EINVAL, "n_outs is NULL");
  int rc;
  if ((rc = check_packed_shape(M, k_in))) return rc;
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_shape(n_outs[i], k_in))) return rc;
    const int64_t widest = n_outs[i] > k_in ? n_outs[i] : k_in;
    if (M * widest >= (1ll << 31))
      return fail(NF4S_ESHAPE, "M=%lld with a %lldx%lld weight exceeds 32-bit offsets", (long long)M,
                  (long long)n_outs[i], (long long)k_in);
    tiles += (n_outs[i] + 127) / 128;
  }
  if (tiles >= (1ll << 31)) return fail(NF4S_ESHAPE, "too many column tiles");
  return NF4S_OK;
}

int nf4s_grouped_workspace_bytes(int n, const int64_t* n_outs, int64_t k_in, int64_t M,
                                 size_t* bytes) {
  if (!bytes) return fail(NF4S_EINVAL, "bytes is NULL");
  int rc;
  if ((rc = check_group(n, n_outs, k_in, M))) return rc;
  *bytes = plan_gemm_grouped(M, n_outs, n, k_in, true).part_bytes;
  return NF4S_OK;
}

int streamed_linear_fwd_grouped(const void* shard_dev, const nf4s_tensor_desc* descs, int n,
                                const void* x_packed, int64_t M, uint16_t* const* ys,
                                const float* const* lora_us, const float* const* lora_Bs, int r,
                                float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!descs || !ys) return fail(NF4S_EINVAL, "descs and ys must be given");
  if (n < 1 || n > GEMM_MAX_SEG)
    return fail(NF4S_EINVAL, "group of %d weights (1..%d allowed)", n, GEMM_MAX_SEG);
  int64_t n_outs[GEMM_MAX_SEG];
  QPtrs q[GEMM_MAX_SEG];
  bool any_lora = false;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_desc(&descs[i]))) return rc;
    if (descs[i].k_in != descs[0].k_in)
      return fail(NF4S_ESHAPE, "weight %d has k_in=%lld, weight 0 has %lld", i,
                  (long long)descs[i].k_in, (long long)descs[0].k_in);
    n_outs[i] = descs[i].n_out;
    if ((rc = check_ptr(ys[i], "ys[i]"))) return rc;
    const float* u = lora_us ? lora_us[i] : nullptr;
    const float* B = lora_Bs ? lora_Bs[i] : nullptr;
    if ((u == nullptr) != (B == nullptr))
      return fail(NF4S_EINVAL, "LoRA operands of weight %d must be given together", i);
    if (u) {
      any_lora = true;
      if ((rc = check_ptr(u, "lora_us[i]", 4))) return rc;
      if ((rc = check_ptr(B, "lora_Bs[i]", 4))) return rc;
    }
  }
  const int64_t k_in = descs[0].k_in;
  if ((rc = check_group(n, n_outs, k_in, M))) return rc;
  for (int i = 0; i < n; ++i)
    if (descs[i].n_out * k_in >= (1ll << 33))
      return fail(NF4S_ESHAPE, "a %lldx%lld weight exceeds 32-bit offsets", (long long)descs[i].n_out,
                  (long long)k_in);
  if (any_lora) {
    if ((rc = check_rank(r))) return rc;
    if (!std::isfinite(scale)) return fail(NF4S_EINVAL, "scale is not finite");
  }
  if ((rc = check_ptr(shard_dev, "shard_dev", 256))) return rc;
  if ((rc = check_ptr(x_packed, "x_packed", 256))) return rc;
  const GemmPlan p = plan_gemm_grouped(M, n_outs, n, k_in, true);
  if (p.part_bytes && (rc = check_ws(ws, ws_bytes, p.part_bytes))) return rc;
  for (int i = 0; i < n; ++i) q[i] = resolve(shard_dev, &descs[i]);
  hipError_t e = launch_linear_grouped_fwd(q, n, n_outs, k_in, static_cast<const uint8_t*>(x_packed),
                                           M, ys, lora_us, lora_Bs, any_lora ? r : 0, scale, ws,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "grouped linear launch");
}

int nf4s_linear_fwd_plan(int n, const int64_t* n_outs, int64_t k_in, int64_t M, int swiglu,
                         int* tile_rows, int* tile_cols, int* splits) {
  if (!tile_rows || !tile_cols || !splits) return fail(NF4S_EINVAL, "plan outputs must be given");
  int rc;
  if ((rc = check_group(n, n_outs, k_in, M))) return rc;
  if (swiglu) {
    if (n != 2 || n_outs[0] != n_outs[1])
      return fail(NF4S_EINVAL, "the SwiGLU launch takes gate and up of one width");
    if (!swiglu_tiles(M, n_outs[0], k_in, tile_rows, tile_cols))
      return fail(NF4S_ESHAPE, "no unsplit SwiGLU launch for M=%lld width=%lld k_in=%lld", (long long)M,
                  (long long)n_outs[0], (long long)k_in);
    *splits = 1;
    return NF4S_OK;
  }
  const GemmPlan p = plan_gemm_grouped(M, n_outs, n, k_in, true);
  *tile_rows = p.bm;
  *tile_cols = p.bn;
  *splits = p.splits;
  return NF4S_OK;
}

int nf4s_swiglu_fused_supported(int64_t M, int64_t width, int64_t k_in) {
  if (M <= 0 || M > kMaxRows || width <= 0 || k_in <= 0 || width % 64 || k_in % 64) return 0;
  return swiglu_fused_ok(M, width, k_in) ? 1 : 0;
}

int streamed_linear_fwd_swiglu(const void* shard_dev, const nf4s_tensor_desc* d_gate,
                               const nf4s_tensor_desc* d_up, const void* x_packed, int64_t M,
                               uint16_t* out, void* out_packed, size_t out_packed_bytes,
                               const float* const* lora_us, const float* const* lora_Bs, int r,
                               float scale, void* stream) {
  int rc;
  if ((rc = check_desc(d_gate)) || (rc = check_desc(d_up))) return rc;
  if (d_gate->n_out != d_up->n_out || d_gate->k_in != d_up->k_in)
    return fail(NF4S_ESHAPE, "gate %lldx%lld and up %lldx%lld differ", (long long)d_gate->n_out,
                (long long)d_gate->k_in, (long long)d_up->n_out, (long long)d_up->k_in);
  const int64_t width = d_gate->n_out, k_in = d_gate->k_in;
  const int64_t n_outs[2] = {width, width};
  if ((rc = check_group(2, n_outs, k_in, M))) return rc;
  if (width % 64)
    return fail(NF4S_ESHAPE, "width %lld is not a multiple of 64 (whole 64-column tiles)", (long long)width);
  if (!swiglu_fused_ok(M, width, k_in))
    return fail(NF4S_ESHAPE,
                "M=%lld, width %lld, k_in %lld needs a split contraction; the fused SwiGLU launch has "
                "none (use streamed_linear_fwd_grouped and nf4s_swiglu_fwd)",
                (long long)M, (long long)width, (long long)k_in);
  if (!out && !out_packed) return fail(NF4S_EINVAL, "out and out_packed are both NULL");
  if (out && (rc = check_ptr(out, "out"))) return rc;
  if (out_packed) {
    if ((rc = check_ptr(out_packed, "out_packed", 256))) return rc;
    const size_t need = packed_activation_bytes(M, width);
    if (out_packed_bytes < need)
      return fail(NF4S_EWORKSPACE, "out_packed of %zu bytes needed, %zu given", need, out_packed_bytes);
  }
  bool any_lora = false;
  for (int i = 0; i < 2; ++i) {
    const float* u = lora_us ? lora_us[i] : nullptr;
    const float* B = lora_Bs ? lora_Bs[i] : nullptr;
    if ((u == nullptr) != (B == nullptr))
      return fail(NF4S_EINVAL, "LoRA operands of weight %d must be given together", i);
    if (u) {
      any_lora = true;
      if ((rc = check_ptr(u, "lora_us[i]", 4)) || (rc = check_ptr(B, "lora_Bs[i]", 4))) return rc;
    }
  }
  if (any_lora) {
    if ((rc = check_rank(r))) return rc;
    if (!std::isfinite(scale)) return fail(NF4S_EINVAL, "scale is not finite");
  }
  if ((rc = check_ptr(shard_dev, "shard_dev", 256))) return rc;
  if ((rc = check_ptr(x_packed, "x_packed", 256))) return rc;
  const QPtrs q[2] = {resolve(shard_dev, d_gate), resolve(shard_dev, d_up)};
  hipError_t e = launch_linear_swiglu_fwd(q, width, k_in, static_cast<const uint8_t*>(x_packed), M, out,
                                          static_cast<uint8_t*>(out_packed), lora_us, lora_Bs,
                                          any_lora ? r : 0, scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "swiglu linear launch");
}

static int check_bwd_group(int n, const int64_t* n_outs, int64_t k_in, int64_t M) {
  if (n < 1 || n > GEMM_MAX_SEG)
    return fail(NF4S_EINVAL, "group of %d weights (1..%d allowed)", n, GEMM_MAX_SEG);
  if (!n_outs) return fail(NF4S_EINVAL, "n_outs is NULL");
  if (M <= 0 || M > kMaxRows) return fail(NF4S_ESHAPE, "M=%lld out of range", (long long)M);
  int rc;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_shape(n_outs[i], k_in))) return rc;
    if ((rc = check_packed_shape(M, n_outs[i]))) return rc;
    if (n > 1 && n_outs[i] % 64)
      return fail(NF4S_ESHAPE, "n_out=%lld of a grouped backward must be a multiple of 64",
                  (long long)n_outs[i]);
    const int64_t widest = n_outs[i] > k_in ? n_outs[i] : k_in;
    if (M * widest >= (1ll << 31) || n_outs[i] * k_in >= (1ll << 33))
      return fail(NF4S_ESHAPE, "M=%lld with a %lldx%lld weight exceeds 32-bit offsets", (long long)M,
                  (long long)n_outs[i], (long long)k_in);
  }
  return NF4S_OK;
}

int nf4s_grouped_bwd_workspace_bytes(int n, const int64_t* n_outs, int64_t k_in, int64_t M,
                                     size_t* bytes) {
  if (!bytes) return fail(NF4S_EINVAL, "bytes is NULL");
  int rc;
  if ((rc = check_bwd_group(n, n_outs, k_in, M))) return rc;
  *bytes = plan_bwd_grouped(M, n_outs, n, k_in).part_bytes;
  return NF4S_OK;
}

int streamed_linear_bwd_grouped(const void* shard_dev, const nf4s_tensor_desc* descs, int n,
                                const void* const* dy_packed, int64_t M, uint16_t* dx,
                                const float* const* lora_dus, const float* const* lora_As, int r,
                                void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!descs || !dy_packed) return fail(NF4S_EINVAL, "descs and dy_packed must be given");
  if (n < 1 || n > GEMM_MAX_SEG)
    return fail(NF4S_EINVAL, "group of %d weights (1..%d allowed)", n, GEMM_MAX_SEG);
  int64_t n_outs[GEMM_MAX_SEG];
  QPtrs q[GEMM_MAX_SEG];
  const uint8_t* dyp[GEMM_MAX_SEG];
  bool any_lora = false;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_desc(&descs[i]))) return rc;
    if (descs[i].k_in != descs[0].k_in)
      return fail(NF4S_ESHAPE, "weight %d has k_in=%lld, weight 0 has %lld", i,
                  (long long)descs[i].k_in, (long long)descs[0].k_in);
    n_outs[i] = descs[i].n_out;
    if ((rc = check_ptr(dy_packed[i], "dy_packed[i]", 256))) return rc;
    dyp[i] = static_cast<const uint8_t*>(dy_packed[i]);
    const float* du = lora_dus ? lora_dus[i] : nullptr;
    const float* A = lora_As ? lora_As[i] : nullptr;
    if ((du == nullptr) != (A == nullptr))
      return fail(NF4S_EINVAL, "LoRA operands of weight %d must be given together", i);
    if (du) {
      any_lora = true;
      if ((rc = check_ptr(du, "lora_dus[i]", 4))) return rc;
      if ((rc = check_ptr(A, "lora_As[i]", 4))) return rc;
    }
  }
  const int64_t k_in = descs[0].k_in;
  if ((rc = check_bwd_group(n, n_outs, k_in, M))) return rc;
  if (any_lora && (rc = check_rank(r))) return rc;
  if ((rc = check_ptr(shard_dev, "shard_dev", 256))) return rc;
  if ((rc = check_ptr(dx, "dx"))) return rc;
  const BwdGroupPlan bp = plan_bwd_grouped(M, n_outs, n, k_in);
  if (bp.part_bytes && (rc = check_ws(ws, ws_bytes, bp.part_bytes))) return rc;
  for (int i = 0; i < n; ++i) q[i] = resolve(shard_dev, &descs[i]);
  hipError_t e = launch_linear_grouped_bwd(q, n, n_outs, k_in, dyp, M, dx, lora_dus, lora_As,
                                           any_lora ? r : 0, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "grouped backward launch");
}

int lora_fwd(const uint16_t* x, int64_t M, int64_t k_in, const float* A, int r, float* u_out,
             void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (M <= 0 || k_in <= 0 || k_in % 64) return fail(NF4S_ESHAPE, "M=%lld k_in=%lld", (long long)M, (long long)k_in);
  if ((rc = check_rank(r))) return rc;
  if ((rc = check_ptr(x, "x"))) return rc;
  if ((rc = check_ptr(A, "A"))) return rc;
  if ((rc = check_ptr(u_out, "u_out", 4))) return rc;
  if (M * k_in >= (1ll << 31)) return fail(NF4S_ESHAPE, "M x k_in too large");
  if ((rc = check_ws(ws, ws_bytes, lora_fwd_ws_bytes(M, k_in, r)))) return rc;
  hipError_t e = launch_lora_fwd(x, M, k_in, A, r, u_out, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "lora_fwd launch");
}

int lora_bwd(const uint16_t* x, const uint16_t* dy, const float* u, int64_t M, int64_t k_in,
             int64_t n_out, const float* B, int r, float scale, float* dA, float* dB,
             float* du_out, int accumulate, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (M <= 0) return fail(NF4S_ESHAPE, "M=%lld must be positive", (long long)M);
  if ((rc = check_shape(n_out, k_in))) return rc;
  if ((rc = check_rank(r))) return rc;
  if (!std::isfinite(scale)) return fail(NF4S_EINVAL, "scale is not finite");
  if (accumulate != 0 && accumulate != 1) return fail(NF4S_EINVAL, "accumulate must be 0 or 1");
  if ((rc = check_ptr(x, "x"))) return rc;
  if ((rc = check_ptr(dy, "dy"))) return rc;
  if ((rc = check_ptr(u, "u", 4))) return rc;
  if ((rc = check_ptr(B, "B", 4))) return rc;
  if ((rc = check_ptr(dA, "dA", 4))) return rc;
  if ((rc = check_ptr(dB, "dB", 4))) return rc;
  if ((rc = check_ptr(du_out, "du_out", 4))) return rc;
  if ((rc = check_ws(ws, ws_bytes, lora_bwd_ws_bytes(M, n_out, r)))) return rc;
  if (M * (n_out > k_in ? n_out : k_in) >= (1ll << 31) || M * r >= (1ll << 31))
    return fail(NF4S_ESHAPE, "M x width too large for the adapter kernels");
  hipError_t e = launch_lora_bwd(x, dy, u, M, k_in, n_out, B, r, scale, dA, dB, du_out, accumulate,
                                 ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "lora_bwd launch");
}

namespace {
int check_lora_group(int n, const int64_t* n_outs, int64_t k_in, int64_t M) {
  if (n < 1 || n > NF4S_MAX_LORA_GROUP)
    return fail(NF4S_EINVAL, "group of %d adapters (1..%d allowed)", n, NF4S_MAX_LORA_GROUP);
  if (!n_outs) return fail(NF4S_EINVAL, "n_outs is NULL");
  if (M <= 0) return fail(NF4S_ESHAPE, "M=%lld must be positive", (long long)M);
  int rc;
  for (int i = 0; i < n; ++i) {
    if ((rc = check_shape(n_outs[i], k_in))) return rc;
    if (M * (n_outs[i] > k_in ? n_outs[i] : k_in) >= (1ll << 31))
      return fail(NF4S_ESHAPE, "M x width too large for the adapter kernels");
  }
  return NF4S_OK;
}

size_t lora_group_ws(int n, const int64_t* n_outs, int64_t k_in, int64_t M, int r, bool bwd) {
  size_t b = 0;
  for (int i = 0; i < n; ++i)
    b += bwd ? lora_bwd_ws_bytes(M, n_outs[i], r) : lora_fwd_ws_bytes(M, k_in, r);
  return b;
}

int check_ptrs(const void* const* p, int n, const char* what, int align) {
  if (!p) return fail(NF4S_EINVAL, "%s is NULL", what);
  int rc;
  for (int i = 0; i < n; ++i)
    if ((rc = check_ptr(p[i], what, align))) return rc;
  return NF4S_OK;
}
}  // namespace

int nf4s_lora_grouped_workspace_bytes(int n, const int64_t* n_outs, int64_t k_in, int64_t M,
                                      int backward, size_t* bytes) {
  if (!bytes) return fail(NF4S_EINVAL, "bytes is NULL");
  int rc;
  if ((rc = check_lora_group(n, n_outs, k_in, M))) return rc;
  *bytes = lora_group_ws(n, n_outs, k_in, M, NF4S_MAX_RANK, backward != 0);
  return NF4S_OK;
}

int lora_fwd_grouped(const uint16_t* x, int64_t M, int64_t k_in, const float* const* A, int n, int r,
                     float* const* u_out, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  int64_t n_outs[NF4S_MAX_LORA_GROUP];
  if (n >= 1 && n <= NF4S_MAX_LORA_GROUP)
    for (int i = 0; i < n; ++i) n_outs[i] = 64;  // the forward reads no output width
  if ((rc = check_lora_group(n, n_outs, k_in, M))) return rc;
  if ((rc = check_rank(r))) return rc;
  if ((rc = check_ptr(x, "x"))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(A), n, "A", 4))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(u_out), n, "u_out", 4))) return rc;
  if ((rc = check_ws(ws, ws_bytes, lora_group_ws(n, n_outs, k_in, M, r, false)))) return rc;
  hipError_t e =
      launch_lora_fwd_grouped(x, M, k_in, A, n, r, u_out, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "lora_fwd_grouped launch");
}

int lora_bwd_grouped(const uint16_t* x, const uint16_t* const* dy, const float* const* u, int64_t M,
                     int64_t k_in, const int64_t* n_outs, const float* const* B, int n, int r,
                     float scale, float* const* dA, float* const* dB, float* const* du_out,
                     int accumulate, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_lora_group(n, n_outs, k_in, M))) return rc;
  if ((rc = check_rank(r))) return rc;
  if (!std::isfinite(scale)) return fail(NF4S_EINVAL, "scale is not finite");
  if (accumulate != 0 && accumulate != 1) return fail(NF4S_EINVAL, "accumulate must be 0 or 1");
  if ((rc = check_ptr(x, "x"))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(dy), n, "dy", 16))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(u), n, "u", 4))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(B), n, "B", 4))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(dA), n, "dA", 4))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(dB), n, "dB", 4))) return rc;
  if ((rc = check_ptrs(reinterpret_cast<const void* const*>(du_out), n, "du_out", 4))) return rc;
  if (M * r >= (1ll << 31)) return fail(NF4S_ESHAPE, "M x r too large for the adapter kernels");
  if ((rc = check_ws(ws, ws_bytes, lora_group_ws(n, n_outs, k_in, M, r, true)))) return rc;
  hipError_t e = launch_lora_bwd_grouped(x, dy, u, M, k_in, n_outs, B, n, r, scale, dA, dB, du_out,
                                         accumulate, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "lora_bwd_grouped launch");
}

int layer_prefetch(void* slot_dev, size_t slot_bytes, const void* host_pinned_src, size_t bytes,
                   void* copy_stream, void* wait_slot_free, void* record_ready) {
  int rc;
  if ((rc = check_ptr(slot_dev, "slot_dev", 256))) return rc;
  if (!host_pinned_src) return fail(NF4S_EINVAL, "host source is NULL");
  if (bytes == 0 || bytes > slot_bytes)
    return fail(NF4S_ESLOT, "shard of %zu bytes does not fit a slot of %zu bytes", bytes, slot_bytes);
  if ((rc = check_pinned(host_pinned_src))) return rc;
  hipStream_t s = static_cast<hipStream_t>(copy_stream);
  hipError_t e;
  if (wait_slot_free && (e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(wait_slot_free), 0)) != hipSuccess)
    return hip_fail(e, "hipStreamWaitEvent");
  if ((e = hipMemcpyAsync(slot_dev, host_pinned_src, bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync");
  if (record_ready && (e = hipEventRecord(static_cast<hipEvent_t>(record_ready), s)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  return NF4S_OK;
}

// ---- resident dense linear (lm_head) -------------------------------------

static int dense_common(bool bwd, const uint16_t* w, int64_t n_out, int64_t k_in,
                        const void* a_packed, int64_t M, uint16_t* out, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc;
  if ((rc = check_shape(n_out, k_in))) return rc;
  if (M <= 0 || M > kMaxRows) return fail(NF4S_ESHAPE, "M=%lld out of range", (long long)M);
  const int64_t widest = n_out > k_in ? n_out : k_in;
  if (M * widest >= (1ll << 31)) return fail(NF4S_ESHAPE, "M x width exceeds 32-bit offsets");
  if ((rc = check_packed_shape(M, bwd ? n_out : k_in))) return rc;
  if ((rc = check_ptr(w, "w"))) return rc;
  if ((rc = check_ptr(a_packed, bwd ? "dy_packed" : "x_packed", 256))) return rc;
  if ((rc = check_ptr(out, bwd ? "dx" : "y"))) return rc;
  const GemmPlan p = plan_gemm(M, bwd ? k_in : n_out, bwd ? n_out : k_in, false);
  if (p.part_bytes && (rc = check_ws(ws, ws_bytes, p.part_bytes))) return rc;
  hipError_t e = launch_dense_packed(bwd, w, n_out, k_in, static_cast<const uint8_t*>(a_packed), M,
                                     out, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "dense linear launch");
}

int dense_linear_fwd_packed(const uint16_t* w, int64_t n_out, int64_t k_in, const void* x_packed,
                            int64_t M, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  return dense_common(false, w, n_out, k_in, x_packed, M, y, ws, ws_bytes, stream);
}

int dense_linear_bwd_packed(const uint16_t* w, int64_t n_out, int64_t k_in, const void* dy_packed,
                            int64_t M, uint16_t* dx, void* ws, size_t ws_bytes, void* stream) {
  return dense_common(true, w, n_out, k_in, dy_packed, M, dx, ws, ws_bytes, stream);
}

// ---- decoder glue ----------------------------------------------------------

static int check_rows(int64_t T, int64_t H) {
  if (T <= 0 || H <= 0 || T > (1ll << 31) - 1 || H > (1ll << 24) || T * H >= (1ll << 40))
    return fail(NF4S_ESHAPE, "rows=%lld width=%lld out of range", (long long)T, (long long)H);
  return NF4S_OK;
}

static int check_count(int64_t n) {
  if (n <= 0 || n >= (1ll << 40)) return fail(NF4S_ESHAPE, "element count %lld out of range", (long long)n);
  return NF4S_OK;
}

static int launched(hipError_t e, const char* what) {
  return e == hipSuccess ? NF4S_OK : hip_fail(e, what);
}

int nf4s_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int64_t* ids, int64_t T,
               float* h, void* stream) {
  int rc;
  if ((rc = check_rows(T, hidden))) return rc;
  if (vocab <= 0 || vocab * hidden >= (1ll << 40)) return fail(NF4S_ESHAPE, "vocab=%lld", (long long)vocab);
  if ((rc = check_ptr(table, "table", 2))) return rc;
  if ((rc = check_ptr(ids, "ids", 8))) return rc;
  if ((rc = check_ptr(h, "h", 4))) return rc;
  return launched(launch_embed(table, vocab, ids, T, hidden, h, static_cast<hipStream_t>(stream)),
                  "embed launch");
}

// The norms move 8 elements (16/32 bytes) per access.
static int check_norm_width(int64_t H) {
  if (H % 8) return fail(NF4S_ESHAPE, "width=%lld is not a multiple of 8", (long long)H);
  return NF4S_OK;
}

// an optional packed output: 256-B aligned, offsets within 32 bits
static int check_packed_out(const void* packed, int64_t T, int64_t W) {
  if (!packed) return NF4S_OK;
  int rc;
  if ((rc = check_packed_shape(T, W))) return rc;
  return check_ptr(packed, "packed", 256);
}

int nf4s_rmsnorm_fwd(const float* x, const float* w, int64_t T, int64_t H, float eps, uint16_t* y,
                     float* rstd, void* packed, void* stream) {
  int rc;
  if ((rc = check_rows(T, H)) || (rc = check_norm_width(H))) return rc;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(NF4S_EINVAL, "eps must be positive and finite");
  if ((rc = check_ptr(x, "x")) || (rc = check_ptr(w, "w")) || (rc = check_ptr(y, "y")) ||
      (rc = check_ptr(rstd, "rstd", 4)) || (rc = check_packed_out(packed, T, H)))
    return rc;
  return launched(launch_rmsnorm_fwd(x, w, T, H, eps, y, rstd, packed, static_cast<hipStream_t>(stream)),
                  "rmsnorm_fwd launch");
}

int nf4s_rmsnorm_bwd(const uint16_t* const* dys, int n_dy, const float* x, const float* w,
                     const float* rstd, int64_t T, int64_t H, int accumulate, float* dh,
                     uint16_t* y, void* packed, void* stream) {
  int rc;
  if ((rc = check_rows(T, H)) || (rc = check_norm_width(H))) return rc;
  if (!dys) return fail(NF4S_EINVAL, "dys is NULL");
  if (n_dy < 1 || n_dy > 3) return fail(NF4S_EINVAL, "n_dy=%d outside [1, 3]", n_dy);
  for (int i = 0; i < n_dy; ++i)
    if ((rc = check_ptr(dys[i], "dys[i]"))) return rc;
  if (accumulate != 0 && accumulate != 1) return fail(NF4S_EINVAL, "accumulate must be 0 or 1");
  if ((rc = check_ptr(x, "x")) || (rc = check_ptr(w, "w")) || (rc = check_ptr(rstd, "rstd", 4)) ||
      (rc = check_ptr(dh, "dh")))
    return rc;
  if (packed && !y) return fail(NF4S_EINVAL, "packed output needs y");
  if (y && (rc = check_ptr(y, "y"))) return rc;
  if (packed && (rc = check_packed_out(packed, T, H))) return rc;
  return launched(launch_rmsnorm_bwd(dys, n_dy, x, w, rstd, T, H, accumulate, dh, y, packed,
                                     static_cast<hipStream_t>(stream)),
                  "rmsnorm_bwd launch");
}

static int check_heads(int heads, int head_dim) {
  if (heads <= 0 || heads > 1024) return fail(NF4S_ESHAPE, "heads=%d out of range", heads);
  if (head_dim <= 0 || head_dim > 256 || head_dim % 2)
    return fail(NF4S_ESHAPE, "head_dim=%d must be even and at most 256", head_dim);
  return NF4S_OK;
}

int nf4s_rope(uint16_t* x, int64_t T, int64_t S, int heads, int head_dim, double theta, int inverse,
              void* stream) {
  int rc;
  if ((rc = check_heads(heads, head_dim))) return rc;
  if (head_dim % 8) return fail(NF4S_ESHAPE, "head_dim=%d is not a multiple of 8", head_dim);
  if (S <= 0 || T <= 0 || T % S) return fail(NF4S_ESHAPE, "rows=%lld must be a positive multiple of seq=%lld", (long long)T, (long long)S);
  if ((rc = check_rows(T, (int64_t)heads * head_dim))) return rc;
  if (!(theta > 1.0) || !std::isfinite(theta)) return fail(NF4S_EINVAL, "theta must be finite and > 1");
  if (inverse != 0 && inverse != 1) return fail(NF4S_EINVAL, "inverse must be 0 or 1");
  if ((rc = check_ptr(x, "x", 8))) return rc;
  return launched(launch_rope(x, T, S, heads, head_dim, theta, inverse, static_cast<hipStream_t>(stream)),
                  "rope launch");
}

int nf4s_rope_pair(uint16_t* q, int q_heads, uint16_t* k, int k_heads, int64_t T, int64_t S,
                   int head_dim, double theta, int inverse, void* q_packed, void* k_packed,
                   void* stream) {
  int rc;
  if ((rc = check_heads(q_heads, head_dim)) || (rc = check_heads(k_heads, head_dim))) return rc;
  if (head_dim % 8) return fail(NF4S_ESHAPE, "head_dim=%d is not a multiple of 8", head_dim);
  if (S <= 0 || T <= 0 || T % S) return fail(NF4S_ESHAPE, "rows=%lld must be a positive multiple of seq=%lld", (long long)T, (long long)S);
  if ((rc = check_rows(T, (int64_t)q_heads * head_dim)) || (rc = check_rows(T, (int64_t)k_heads * head_dim)))
    return rc;
  if (!(theta > 1.0) || !std::isfinite(theta)) return fail(NF4S_EINVAL, "theta must be finite and > 1");
  if (inverse != 0 && inverse != 1) return fail(NF4S_EINVAL, "inverse must be 0 or 1");
  if ((rc = check_ptr(q, "q", 8)) || (rc = check_ptr(k, "k", 8))) return rc;
  if ((rc = check_packed_out(q_packed, T, (int64_t)q_heads * head_dim)) ||
      (rc = check_packed_out(k_packed, T, (int64_t)k_heads * head_dim)))
    return rc;
  return launched(launch_rope_pair(q, q_heads, k, k_heads, T, S, head_dim, theta, inverse, q_packed,
                                   k_packed, static_cast<hipStream_t>(stream)),
                  "rope launch");
}

static int check_attention(int64_t B, int64_t S, int heads, int kv_heads, int head_dim) {
  int rc;
  if ((rc = check_heads(heads, head_dim))) return rc;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(NF4S_ESHAPE, "head_dim=%d not one of 32, 64, 128", head_dim);
  if (kv_heads <= 0 || heads % kv_heads)
    return fail(NF4S_ESHAPE, "heads=%d is not a multiple of kv_heads=%d", heads, kv_heads);
  if (B <= 0 || S <= 0 || B * S > (1ll << 24) || B * heads * ((S + 63) / 64) >= (1ll << 31))
    return fail(NF4S_ESHAPE, "batch=%lld seq=%lld out of range", (long long)B, (long long)S);
  if (B * S * heads * head_dim >= (1ll << 31) / 4)
    return fail(NF4S_ESHAPE, "attention of %lld tokens x %d heads too large", (long long)(B * S), heads);
  return NF4S_OK;
}

int nf4s_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                       int64_t S, int heads, int kv_heads, int head_dim, uint16_t* o, float* o_f32,
                       float* lse, void* packed, void* stream) {
  int rc;
  if ((rc = check_attention(B, S, heads, kv_heads, head_dim))) return rc;
  if (packed && (rc = check_packed_out(packed, B * S, (int64_t)heads * head_dim))) return rc;
  // the kernels move 16-byte fragments of q, k, v and store o / o_f32 in 8- and 16-byte pieces
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, "o")) || (rc = check_ptr(lse, "lse", 4)))
    return rc;
  if (o_f32 && (rc = check_ptr(o_f32, "o_f32"))) return rc;
  return launched(launch_attention_fwd(q, k, v, B, S, heads, kv_heads, head_dim, o, o_f32, lse, packed,
                                       static_cast<hipStream_t>(stream)),
                  "attention_fwd launch");
}

int nf4s_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* o_f32,
                       const uint16_t* dout, const float* lse, int64_t B, int64_t S, int heads,
                       int kv_heads, int head_dim, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                       void* dv_packed, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_attention(B, S, heads, kv_heads, head_dim))) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o_f32, "o_f32")) || (rc = check_ptr(dout, "dout")) ||
      (rc = check_ptr(lse, "lse", 4)) || (rc = check_ptr(dq, "dq")) || (rc = check_ptr(dk, "dk")) ||
      (rc = check_ptr(dv, "dv")) || (rc = check_packed_out(dv_packed, B * S, (int64_t)kv_heads * head_dim)))
    return rc;
  if ((rc = check_ws(ws, ws_bytes, attention_bwd_ws_bytes(B, S, heads, head_dim)))) return rc;
  return launched(launch_attention_bwd(q, k, v, o_f32, dout, lse, B, S, heads, kv_heads, head_dim, dq,
                                       dk, dv, dv_packed, ws, static_cast<hipStream_t>(stream)),
                  "attention_bwd launch");
}

int nf4s_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t T, int64_t width, uint16_t* out,
                    void* packed, void* stream) {
  int rc;
  if ((rc = check_rows(T, width)) || (rc = check_norm_width(width))) return rc;
  if ((rc = check_ptr(g, "g")) || (rc = check_ptr(u, "u")) || (rc = check_ptr(out, "out")) ||
      (rc = check_packed_out(packed, T, width)))
    return rc;
  return launched(launch_swiglu_fwd(g, u, T, width, out, packed, static_cast<hipStream_t>(stream)),
                  "swiglu_fwd launch");
}

int nf4s_swiglu_bwd(const uint16_t* ds, const uint16_t* g, const uint16_t* u, int64_t T,
                    int64_t width, uint16_t* dg, uint16_t* du, void* dg_packed, void* du_packed,
                    void* stream) {
  int rc;
  if ((rc = check_rows(T, width)) || (rc = check_norm_width(width))) return rc;
  if ((rc = check_ptr(ds, "ds")) || (rc = check_ptr(g, "g")) || (rc = check_ptr(u, "u")) ||
      (rc = check_packed_out(dg_packed, T, width)) || (rc = check_packed_out(du_packed, T, width)))
    return rc;
  // a row-major result may be left out when its packed form is written
  if ((dg || !dg_packed) && (rc = check_ptr(dg, "dg"))) return rc;
  if ((du || !du_packed) && (rc = check_ptr(du, "du"))) return rc;
  return launched(launch_swiglu_bwd(ds, g, u, T, width, dg, du, dg_packed, du_packed,
                                    static_cast<hipStream_t>(stream)),
                  "swiglu_bwd launch");
}

int nf4s_residual_add(const float* h, const uint16_t* y, int64_t n, float* out, void* stream) {
  int rc;
  if ((rc = check_count(n))) return rc;
  if ((rc = check_ptr(h, "h", 4)) || (rc = check_ptr(y, "y", 2)) || (rc = check_ptr(out, "out", 4))) return rc;
  return launched(launch_residual_add(h, y, n, out, static_cast<hipStream_t>(stream)),
                  "residual_add launch");
}

int nf4s_to_bf16(const float* x, int64_t T, int64_t width, uint16_t* y, void* packed, void* stream) {
  int rc;
  if ((rc = check_rows(T, width)) || (rc = check_norm_width(width))) return rc;
  if ((rc = check_ptr(x, "x")) || (rc = check_ptr(y, "y")) || (rc = check_packed_out(packed, T, width)))
    return rc;
  return launched(launch_f32_to_bf16(x, T, width, y, packed, static_cast<hipStream_t>(stream)),
                  "to_bf16 launch");
}

int nf4s_cross_entropy(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V,
                       float* loss, uint16_t* dlogits, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_rows(T, V))) return rc;
  if ((rc = check_ptr(logits, "logits", 2)) || (rc = check_ptr(targets, "targets", 8)) ||
      (rc = check_ptr(loss, "loss", 4)) || (rc = check_ptr(dlogits, "dlogits", 2)))
    return rc;
  if ((rc = check_ws(ws, ws_bytes, cross_entropy_ws_bytes(T)))) return rc;
  return launched(launch_cross_entropy(logits, targets, T, V, loss, dlogits, ws,
                                       static_cast<hipStream_t>(stream)),
                  "cross_entropy launch");
}

int nf4s_token_nll(const uint16_t* logits, const int64_t* targets, int64_t T, int64_t V, float* nll,
                   void* stream) {
  int rc;
  if ((rc = check_rows(T, V))) return rc;
  if ((rc = check_ptr(logits, "logits", 2)) || (rc = check_ptr(targets, "targets", 8)) ||
      (rc = check_ptr(nll, "nll", 4)))
    return rc;
  return launched(launch_token_nll(logits, targets, T, V, nll, static_cast<hipStream_t>(stream)),
                  "token_nll launch");
}

int nf4s_dpo_loss(const float* nll_policy, const float* nll_ref, const float* mask, int64_t pairs,
                  int64_t S, float beta, float* loss, float* seq_coef, void* stream) {
  int rc;
  if (pairs <= 0 || pairs > 4096 || S <= 0 || 2 * pairs * S >= (1ll << 31))
    return fail(NF4S_ESHAPE, "pairs=%lld seq=%lld out of range", (long long)pairs, (long long)S);
  if (!std::isfinite(beta) || !(beta > 0.0f)) return fail(NF4S_EINVAL, "beta must be positive and finite");
  if ((rc = check_ptr(nll_policy, "nll_policy", 4)) || (rc = check_ptr(nll_ref, "nll_ref", 4)) ||
      (rc = check_ptr(mask, "mask", 4)) || (rc = check_ptr(loss, "loss", 4)) ||
      (rc = check_ptr(seq_coef, "seq_coef", 4)))
    return rc;
  return launched(launch_dpo(nll_policy, nll_ref, mask, pairs, S, beta, loss, seq_coef,
                             static_cast<hipStream_t>(stream)),
                  "dpo launch");
}

int nf4s_logit_grad(const uint16_t* logits, const int64_t* targets, const float* seq_coef,
                    const float* mask, int64_t T, int64_t S, int64_t V, uint16_t* dlogits,
                    void* stream) {
  int rc;
  if ((rc = check_rows(T, V))) return rc;
  if (S <= 0 || T % S) return fail(NF4S_ESHAPE, "rows=%lld must be a multiple of seq=%lld", (long long)T, (long long)S);
  if ((rc = check_ptr(logits, "logits", 2)) || (rc = check_ptr(targets, "targets", 8)) ||
      (rc = check_ptr(seq_coef, "seq_coef", 4)) || (rc = check_ptr(mask, "mask", 4)) ||
      (rc = check_ptr(dlogits, "dlogits", 2)))
    return rc;
  return launched(launch_logit_grad(logits, targets, seq_coef, mask, T, S, V, dlogits,
                                    static_cast<hipStream_t>(stream)),
                  "logit_grad launch");
}

int nf4s_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1,
               float beta2, float eps, float weight_decay, int64_t step, void* stream) {
  int rc;
  if ((rc = check_count(n))) return rc;
  if (step < 1) return fail(NF4S_EINVAL, "step=%lld must count from 1", (long long)step);
  if (!std::isfinite(lr) || lr < 0.0f || !(beta1 >= 0.0f && beta1 < 1.0f) ||
      !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) || !std::isfinite(weight_decay))
    return fail(NF4S_EINVAL, "AdamW hyper-parameters out of range");
  if ((rc = check_ptr(p, "p", 4)) || (rc = check_ptr(g, "g", 4)) || (rc = check_ptr(m, "m", 4)) ||
      (rc = check_ptr(v, "v", 4)))
    return rc;
  return launched(launch_adamw(p, g, m, v, n, lr, beta1, beta2, eps, weight_decay, step,
                               static_cast<hipStream_t>(stream)),
                  "adamw launch");
}

int nf4s_event_create(void** event_out) {
  if (!event_out) return fail(NF4S_EINVAL, "event_out is NULL");
  hipEvent_t ev;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  *event_out = ev;
  return NF4S_OK;
}

int nf4s_event_destroy(void* event) {
  if (!event) return NF4S_OK;
  hipError_t e = hipEventDestroy(static_cast<hipEvent_t>(event));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "hipEventDestroy");
}

int nf4s_event_record(void* event, void* stream) {
  if (!event) return fail(NF4S_EINVAL, "event is NULL");
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "hipEventRecord");
}

int nf4s_stream_wait_event(void* stream, void* event) {
  if (!event) return fail(NF4S_EINVAL, "event is NULL");
  hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(event), 0);
  return e == hipSuccess ? NF4S_OK : hip_fail(e, "hipStreamWaitEvent");
}

}  // extern "C"

// ---- slot pool -----------------------------------------------------------

// The pool's copies are enqueued on the copy stream by a host thread of its
// own (the issuer), each only once the free event it must follow has
// completed, so the copy stream never holds a wait on a pending event: the
// runtime resolves such a wait tens of microseconds after the event
// completes, a gap before every layer copy of a copy-bound sweep (measured
// on MI355X: a median 68 us between back-to-back 112.5 MB copies). The
// issuer takes requests in order; an acquire waits on the host until the
// copy (and ready event) of its slot is enqueued, then makes the compute
// stream wait for the ready event as before.
struct nf4s_pool {
  struct Slot {
    void* ptr = nullptr;
    hipEvent_t ready = nullptr;  // recorded on the copy stream after the copy
    hipEvent_t free = nullptr;   // recorded on the compute stream after the last reader
    int layer = -1;              // layer held (or being copied), -1 = none
    bool held = false;           // between acquire and release
    bool reserved = false;       // prefetched (or asked for again) and not yet acquired
    bool free_recorded = false;  // a free event exists to wait on
    uint64_t last_use = 0;       // 0 = never, or emptied
    uint64_t asked = 0;          // copies and fills requested of the issuer for this slot
    uint64_t issued = 0;         // of those, the ones it has enqueued (under mu)
  };
  struct Layer {
    const void* src = nullptr;
    size_t bytes = 0;
  };
  struct Job {
    bool fill = false;  // poison fill instead of a copy
    int slot = 0;
    uint64_t seq = 0;   // the slot's request number
    const void* src = nullptr;
    size_t bytes = 0;
    bool wait_free = false;
  };
  int n = 0;
  size_t slot_bytes = 0;
  hipStream_t copy = nullptr, compute = nullptr;
  int device = 0;
  int debug = 0;  // NF4S_POOL_POISON_ON_RELEASE
  Slot slots[8];
  std::vector<Layer> layers;
  uint64_t tick = 0, copies = 0, bytes = 0;
  std::mutex mu;
  std::condition_variable cv;  // a job queued, or a job enqueued on the copy stream
  std::deque<Job> jobs;
  bool stop = false;
  hipError_t issue_error = hipSuccess;  // the first failure of the issuer
  std::thread issuer;
};

namespace {

int pool_find(const nf4s_pool* p, int layer) {
  if (layer < 0) return -1;  // -1 marks an empty slot, never a layer
  for (int i = 0; i < p->n; ++i)
    if (p->slots[i].layer == layer) return i;
  return -1;
}

int pool_check_layer(const nf4s_pool* p, int layer) {
  if (layer < 0 || layer >= (int)p->layers.size() || !p->layers[layer].src)
    return fail(NF4S_ESLOT, "layer %d was not registered", layer);
  return NF4S_OK;
}

// The slot a copy may overwrite: one that no reader holds, preferring an
// empty slot, then the least recently used slot that no earlier prefetch
// reserved; a reserved slot only when take_reserved (an acquire that must
// make room).
int pool_victim(const nf4s_pool* p, bool take_reserved) {
  int v = -1;
  for (int pass = 0; pass < (take_reserved ? 2 : 1) && v < 0; ++pass) {
    for (int i = 0; i < p->n; ++i) {
      const auto& s = p->slots[i];
      if (s.held || (pass == 0 && s.reserved)) continue;
      if (s.layer < 0) return i;
      if (v < 0 || s.last_use < p->slots[v].last_use) v = i;
    }
  }
  return v;
}

// The issuer: wait for the slot's free event on the host, then enqueue the
// copy and record the ready event (or enqueue the poison fill); requests in
// the order they were made. Stops once asked to and every request is done.
void pool_issue_loop(nf4s_pool* p) {
  const hipError_t dev_e = hipSetDevice(p->device);  // the device is per thread
  if (dev_e != hipSuccess) {
    std::lock_guard<std::mutex> lk(p->mu);
    p->issue_error = dev_e;
  }
  for (;;) {
    nf4s_pool::Job j;
    {
      std::unique_lock<std::mutex> lk(p->mu);
      p->cv.wait(lk, [p] { return p->stop || !p->jobs.empty(); });
      if (p->jobs.empty()) return;
      j = p->jobs.front();
      p->jobs.pop_front();
    }
    auto& s = p->slots[j.slot];
    hipError_t e = dev_e;  // after a failure every request is still marked issued, never enqueued
    if (e == hipSuccess && j.wait_free) e = hipEventSynchronize(s.free);
    if (e == hipSuccess) {
      if (j.fill) {
        e = launch_fill_u32(s.ptr, p->slot_bytes, 0xFFFFFFFFu, p->copy);
      } else {
        e = hipMemcpyAsync(s.ptr, j.src, j.bytes, hipMemcpyHostToDevice, p->copy);
        if (e == hipSuccess) e = hipEventRecord(s.ready, p->copy);
      }
    }
    {
      std::lock_guard<std::mutex> lk(p->mu);
      if (e != hipSuccess && p->issue_error == hipSuccess) p->issue_error = e;
      s.issued = j.seq;
    }
    p->cv.notify_all();
  }
}

void pool_request(nf4s_pool* p, nf4s_pool::Job j) {
  auto& s = p->slots[j.slot];
  j.seq = ++s.asked;
  j.wait_free = s.free_recorded;
  {
    std::lock_guard<std::mutex> lk(p->mu);
    p->jobs.push_back(j);
  }
  p->cv.notify_all();
}

// Block until every request for slot v is enqueued on the copy stream;
// the issuer's first failure, if any.
int pool_wait_issued(nf4s_pool* p, int v) {
  auto& s = p->slots[v];
  std::unique_lock<std::mutex> lk(p->mu);
  p->cv.wait(lk, [&] { return s.issued == s.asked; });
  if (p->issue_error != hipSuccess) return hip_fail(p->issue_error, "slot copy (pool issuer)");
  return NF4S_OK;
}

int pool_issue_status(nf4s_pool* p) {
  std::lock_guard<std::mutex> lk(p->mu);
  return p->issue_error == hipSuccess ? NF4S_OK : hip_fail(p->issue_error, "slot copy (pool issuer)");
}

int pool_copy_into(nf4s_pool* p, int layer, int v) {
  auto& s = p->slots[v];
  const auto& L = p->layers[layer];
  nf4s_pool::Job j;
  j.slot = v;
  j.src = L.src;
  j.bytes = L.bytes;
  pool_request(p, j);
  s.layer = layer;
  s.last_use = ++p->tick;
  p->copies += 1;
  p->bytes += L.bytes;
  return NF4S_OK;
}

}  // namespace

extern "C" {

int nf4s_pool_create(int n_slots, void* const* slots, size_t slot_bytes, void* copy_stream,
                     void* compute_stream, nf4s_pool** out) {
  if (!out || !slots) return fail(NF4S_EINVAL, "NULL argument");
  if (n_slots < 2 || n_slots > 8) return fail(NF4S_ESLOT, "pool size %d outside [2, 8]", n_slots);
  if (slot_bytes == 0) return fail(NF4S_ESLOT, "slot_bytes is 0");
  if (copy_stream == compute_stream)
    return fail(NF4S_EINVAL, "copy and compute streams must differ (the copy overlaps compute)");
  for (int i = 0; i < n_slots; ++i) {
    int rc = check_ptr(slots[i], "slot", 256);
    if (rc) return rc;
  }
  // two slots sharing memory would let a copy overwrite a layer another
  // slot's reader still holds
  for (int i = 0; i < n_slots; ++i)
    for (int j = i + 1; j < n_slots; ++j) {
      const uintptr_t a = (uintptr_t)slots[i], b = (uintptr_t)slots[j];
      if (a < b + slot_bytes && b < a + slot_bytes)
        return fail(NF4S_EINVAL, "slots %d and %d overlap (slot_bytes %zu)", i, j, slot_bytes);
    }
  nf4s_pool* p = new nf4s_pool();
  p->n = n_slots;
  p->slot_bytes = slot_bytes;
  p->copy = static_cast<hipStream_t>(copy_stream);
  p->compute = static_cast<hipStream_t>(compute_stream);
  hipError_t e0 = hipGetDevice(&p->device);
  if (e0 != hipSuccess) {
    delete p;
    return hip_fail(e0, "hipGetDevice");
  }
  for (int i = 0; i < n_slots; ++i) {
    p->slots[i].ptr = slots[i];
    hipError_t e1 = hipEventCreateWithFlags(&p->slots[i].ready, hipEventDisableTiming);
    hipError_t e2 = hipEventCreateWithFlags(&p->slots[i].free, hipEventDisableTiming);
    if (e1 != hipSuccess || e2 != hipSuccess) {
      nf4s_pool_destroy(p);
      return hip_fail(e1 != hipSuccess ? e1 : e2, "hipEventCreateWithFlags");
    }
  }
  p->issuer = std::thread(pool_issue_loop, p);
  *out = p;
  return NF4S_OK;
}

int nf4s_pool_destroy(nf4s_pool* p) {
  if (!p) return NF4S_OK;
  if (p->issuer.joinable()) {  // let the issuer enqueue what was asked, then stop it
    {
      std::lock_guard<std::mutex> lk(p->mu);
      p->stop = true;
    }
    p->cv.notify_all();
    p->issuer.join();
  }
  for (int i = 0; i < p->n; ++i) {
    if (p->slots[i].ready) (void)hipEventDestroy(p->slots[i].ready);
    if (p->slots[i].free) (void)hipEventDestroy(p->slots[i].free);
  }
  delete p;
  return NF4S_OK;
}

int nf4s_pool_set_debug(nf4s_pool* p, int flags) {
  if (!p) return fail(NF4S_EINVAL, "pool is NULL");
  if (flags & ~NF4S_POOL_POISON_ON_RELEASE) return fail(NF4S_EINVAL, "unknown debug flags %d", flags);
  p->debug = flags;
  return NF4S_OK;
}

int nf4s_pool_set_layer(nf4s_pool* p, int layer, const void* src, size_t bytes) {
  if (!p || !src) return fail(NF4S_EINVAL, "NULL argument");
  if (layer < 0 || layer > (1 << 20)) return fail(NF4S_ESLOT, "layer index %d", layer);
  if (bytes == 0 || bytes > p->slot_bytes)
    return fail(NF4S_ESLOT, "shard of %zu bytes does not fit a slot of %zu bytes", bytes, p->slot_bytes);
  int rc = check_pinned(src);
  if (rc) return rc;
  // a re-registered layer is stale wherever it is resident; one that a reader
  // holds cannot be replaced under it
  const int i = pool_find(p, layer);
  if (i >= 0 && p->slots[i].held)
    return fail(NF4S_ESLOT, "layer %d is acquired; release it before registering it again", layer);
  if ((int)p->layers.size() <= layer) p->layers.resize(layer + 1);
  p->layers[layer].src = src;
  p->layers[layer].bytes = bytes;
  if (i >= 0) {
    p->slots[i].layer = -1;
    p->slots[i].reserved = false;
    p->slots[i].last_use = 0;
  }
  return NF4S_OK;
}

int nf4s_pool_prefetch(nf4s_pool* p, int layer) {
  if (!p) return fail(NF4S_EINVAL, "pool is NULL");
  int rc = pool_check_layer(p, layer);
  if (rc || (rc = pool_issue_status(p))) return rc;
  const int i = pool_find(p, layer);
  if (i >= 0) {  // resident or in flight: keep it for its next reader
    if (!p->slots[i].held) p->slots[i].reserved = true;
    return NF4S_OK;
  }
  const int v = pool_victim(p, false);
  if (v < 0) {
    for (int j = 0; j < p->n; ++j)
      if (!p->slots[j].held) return NF4S_OK;  // every free slot is reserved: the acquire copies
    return fail(NF4S_ESLOT, "every slot is held; release one before prefetching");
  }
  rc = pool_copy_into(p, layer, v);
  if (rc) return rc;
  p->slots[v].reserved = true;
  return NF4S_OK;
}

int nf4s_pool_acquire(nf4s_pool* p, int layer, void** slot_dev_out) {
  if (!p || !slot_dev_out) return fail(NF4S_EINVAL, "NULL argument");
  int rc = pool_check_layer(p, layer);
  if (rc) return rc;
  int i = pool_find(p, layer);
  if (i >= 0 && p->slots[i].held) return fail(NF4S_ESLOT, "layer %d is already acquired", layer);
  if (i < 0) {
    i = pool_victim(p, true);
    if (i < 0) return fail(NF4S_ESLOT, "every slot is held; release one before acquiring layer %d", layer);
    if ((rc = pool_copy_into(p, layer, i))) return rc;
  }
  if ((rc = pool_wait_issued(p, i))) return rc;
  auto& s = p->slots[i];
  hipError_t e = hipStreamWaitEvent(p->compute, s.ready, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  s.held = true;
  s.reserved = false;
  s.last_use = ++p->tick;
  *slot_dev_out = s.ptr;
  return NF4S_OK;
}

int nf4s_pool_release(nf4s_pool* p, int layer) {
  if (!p) return fail(NF4S_EINVAL, "pool is NULL");
  int rc = pool_check_layer(p, layer);
  if (rc) return rc;
  const int i = pool_find(p, layer);
  if (i < 0 || !p->slots[i].held) return fail(NF4S_ESLOT, "layer %d is not acquired", layer);
  auto& s = p->slots[i];
  hipError_t e = hipEventRecord(s.free, p->compute);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  s.free_recorded = true;
  s.held = false;
  if (p->debug & NF4S_POOL_POISON_ON_RELEASE) {
    // Overwrite the slot with NaN bytes on the copy stream, issued after the
    // free event exactly as the next copy into the slot would be: a kernel
    // that still read the slot after its release would see NaN weights.
    s.layer = -1;
    s.reserved = false;
    s.last_use = 0;
    nf4s_pool::Job j;
    j.fill = true;
    j.slot = i;
    pool_request(p, j);
  }
  return pool_issue_status(p);
}

int nf4s_pool_stats(const nf4s_pool* p, uint64_t* copies, uint64_t* bytes) {
  if (!p) return fail(NF4S_EINVAL, "pool is NULL");
  if (copies) *copies = p->copies;
  if (bytes) *bytes = p->bytes;
  return NF4S_OK;
}

}  // extern "C"
