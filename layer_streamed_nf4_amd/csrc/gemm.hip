// Fused NF4-dequant bf16 MFMA GEMMs for the frozen linears.
//
// Forward  y[M, n_out]  = x[M, k_in] . W'^T   (+ s . u . B^T)
// Backward dx[M, k_in]  = dy[M, n_out] . W'   (+ du . A)
// Gate walkthrough ("Soup layer-streamed NF4 training measured") section 2.1:
// the NF4 weight is rebuilt from the streamed bytes on every call and used with
// bf16 compute; section 4.4: the frozen base needs dL/dx but no dL/dW.
//
// Both directions are one kernel template computing C[M, Nc] = A[M, Kc] . B,
// where A is the bf16 activation (x or dy, row stride Kc) and B[Kc, Nc] is the
// dequantised weight seen either transposed (forward: B[k][n] = W'[n][k]) or
// as is (backward: B[k][n] = W'[k][n]). The packed codes are read from HBM once
// per workgroup, decoded in registers with the block scale
// a' = fp32(fp32(C8[q8]*nested) + offset) and W' = bf16_rne(fp32(C4[code]*a')),
// and written to LDS as bf16 in the contraction-major layout the matrix cores
// read; W' never goes back to HBM. A packed byte holds two codes, and one LDS
// read of a 256-entry table gives both of their NF4 levels; the table is
// replicated 16 times so that lane l always reads the copy that lives in bank
// pair (2(l%16), 2(l%16)+1), which makes the random lookups conflict-free.
// The backward orientation is transposed on the way into LDS for free: a
// thread decodes a 4x8 patch and pairs values along the contraction when it
// packs bf16.
//
// Tiling for gfx950: 512 threads (8 wave64, two per SIMD so that one wave's
// LDS and memory waits are covered by the other's MFMAs), output tile
// 256x128, contraction step 64 (exactly one NF4 block per weight row in the
// forward direction), v_mfma_f32_32x32x16_bf16 with each wave owning a 64x64
// sub-tile (2x2 MFMA tiles, 64 fp32 accumulators per lane), double-buffered
// LDS, and register rings that keep the weight stream and the activation tile
// two steps ahead.
// All per-lane addresses are loop-invariant 32-bit offsets from per-step
// uniform bases, so a step spends its vector instructions on decoding only.
// LDS rows are padded to 144 B so the 16-byte fragment reads of 8 consecutive
// lanes cover all 32 banks. When the output has too few tiles to occupy the
// chip, the contraction is split; each split writes fp32 partials and a second
// kernel sums them in split order (deterministic, no atomics).
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDS_STRIDE = 72;  // bf16 elements per LDS row (64 + 8 pad = 144 B)
constexpr int THREADS = 512;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* q8;
  const float* nested;
  const float* offset;
  const uint16_t* a;  // bf16 [M, Kc]
  int64_t M, Kc, Nc;
  int64_t n_out, k_in;
  uint16_t* out;       // bf16 [M, Nc]
  float* part;         // fp32 [splits, M, Nc] (splits > 1)
  int64_t kc_chunk;
  const float* lora_l;  // fp32 [M, r]
  const float* lora_r;  // fwd: B fp32 [n_out, r]; bwd: A fp32 [r, k_in]
  int r;
  float scale;
};

// A contraction step covers [k0, k0 + 64). When the contraction length Kc is
// not a multiple of 64 (backward with n_out % 64 != 0) the last step reads the
// window [Kc - 64, Kc) instead, and the weight rows it has already consumed
// (below its nominal start) decode to zero.
struct Step {
  int64_t win;  // first contraction index actually read
  int64_t nom;  // nominal first index; rows below it are masked
};

// ---- activation tile (A): 4 rows x 16 bytes per thread -------------------
constexpr int A_CHUNKS = BM * BK / 8 / THREADS;  // 16-byte chunks per thread (4)
constexpr int A_ROW_STEP = THREADS / 8;          // rows between a thread's chunks (64)

struct ALanes {
  uint32_t off[A_CHUNKS];  // byte offsets of the thread's chunks at contraction 0
};

__device__ __forceinline__ ALanes a_lanes(const GemmArgs& g, int64_t m0) {
  const int t = threadIdx.x;
  ALanes L;
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    int64_t row = m0 + (t >> 3) + A_ROW_STEP * i;
    row = row < g.M ? row : g.M - 1;  // rows past M feed output rows never stored
    L.off[i] = (uint32_t)((row * g.Kc + (t & 7) * 8) * 2);
  }
  return L;
}

__device__ __forceinline__ void load_a(const GemmArgs& g, const ALanes& L, int64_t win,
                                       u32x4 (&ra)[A_CHUNKS]) {
  const char* base = reinterpret_cast<const char*>(g.a + win);
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *reinterpret_cast<const u32x4*>(base + L.off[i]);
}

__device__ __forceinline__ void store_a(uint16_t* As, const u32x4 (&ra)[A_CHUNKS]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int row = (t >> 3) + A_ROW_STEP * i;
    *reinterpret_cast<u32x4*>(As + row * LDS_STRIDE + c * 8) = ra[i];
  }
}

// ---- weight tile (B) ------------------------------------------------------
template <bool BWD>
struct WLanes;
template <bool BWD>
struct BRegs;

// Forward: thread t owns weight row n0 + t/4 and contraction quarter t%4
// (16 codes, two packed words).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <>
struct WLanes<false> {
  uint32_t woff;  // byte offset of the thread's 8 packed bytes at contraction 0
  uint32_t blk0;  // 64-block index at contraction 0
  bool valid;     // row < n_out
};
template <>
struct BRegs<false> {
  u32x2 w;
  uint32_t q;
  float nest;
};

__device__ __forceinline__ WLanes<false> w_lanes_fwd(const GemmArgs& g, int64_t n0) {
  const int t = threadIdx.x;
  WLanes<false> L;
  int64_t n = n0 + (t >> 2);
  L.valid = n < g.n_out;
  n = L.valid ? n : g.n_out - 1;
  L.woff = (uint32_t)(n * (g.k_in / 2) + (t & 3) * 8);
  L.blk0 = (uint32_t)(n * (g.k_in / 64));
  return L;
}

__device__ __forceinline__ void load_b(const GemmArgs& g, const WLanes<false>& L, Step s,
                                       BRegs<false>& rb) {
  rb.w = *reinterpret_cast<const u32x2*>(g.packed + s.win / 2 + L.woff);
  const uint32_t blk = L.blk0 + (uint32_t)(s.win / 64);
  rb.q = g.q8[blk];
  rb.nest = g.nested[blk >> 8];
}

// Backward: thread t owns weight rows k0 + 2*(t/16) + i (i < 2) and output
// columns n0 + 8*(t%16) + j (j < 8): two packed words, two 8-bit scale codes
// packed in one register, two nested scales, a 2-bit validity mask.
constexpr int BW_ROWS = 2;
template <>
struct WLanes<true> {
  uint32_t woff[BW_ROWS];  // byte offsets of the packed words at contraction 0
  uint32_t blk0[BW_ROWS];  // 64-block indices at contraction 0
  bool cvalid;             // columns < k_in
};
template <>
struct BRegs<true> {
  uint32_t w[BW_ROWS];
  uint32_t q;
  float nest[BW_ROWS];
  uint32_t vmask;
};

__device__ __forceinline__ WLanes<true> w_lanes_bwd(const GemmArgs& g, int64_t n0) {
  const int t = threadIdx.x;
  WLanes<true> L;
  int64_t col = n0 + 8 * (t & 15);
  L.cvalid = col < g.k_in;
  col = L.cvalid ? col : g.k_in - 8;
#pragma unroll
  for (int i = 0; i < BW_ROWS; ++i) {
    const int64_t row = BW_ROWS * (t >> 4) + i;  // relative to the step's window
    L.woff[i] = (uint32_t)((row * g.k_in + col) / 2);
    L.blk0[i] = (uint32_t)((row * g.k_in + col) / 64);
  }
  return L;
}

__device__ __forceinline__ void load_b(const GemmArgs& g, const WLanes<true>& L, Step s,
                                       BRegs<true>& rb) {
  const int t = threadIdx.x;
  const uint8_t* base = g.packed + s.win * (g.k_in / 2);
  const uint32_t bstep = (uint32_t)(s.win * (g.k_in / 64));
  rb.q = 0;
  rb.vmask = 0;
#pragma unroll
  for (int i = 0; i < BW_ROWS; ++i) {
    rb.w[i] = *reinterpret_cast<const uint32_t*>(base + L.woff[i]);
    const uint32_t blk = bstep + L.blk0[i];
    rb.q |= (uint32_t)g.q8[blk] << (8 * i);
    rb.nest[i] = g.nested[blk >> 8];
    const int64_t row = s.win + BW_ROWS * (t >> 4) + i;
    rb.vmask |= (L.cvalid && row >= s.nom) ? (1u << i) : 0u;
  }
}

// ---- decoding -------------------------------------------------------------
// Pair table: entry b = (C4[b >> 4], C4[b & 15]), both levels of a packed byte,
// the even element (high nibble) first. Copy c of entry b sits at float2 index
// 16*b + c, i.e. dwords 32*b + 2c and 32*b + 2c + 1: the copy fixes the LDS
// bank pair whatever b is. `ptab` below is already offset by the lane's copy.
constexpr int PAIR_COPIES = 16;

__device__ __forceinline__ float2 pair_of(const float2* ptab, uint32_t word, int byte) {
  return ptab[((word >> (8 * byte)) & 0xFFu) * PAIR_COPIES];
}

__device__ __forceinline__ float stage_scale(const BRegs<false>& rb, bool valid, float off,
                                             const float* c8) {
  return valid ? decode_scale(c8[rb.q], rb.nest, off) : 0.0f;
}

// Quarter Q of a forward stage: half Q%2 of packed word Q/2 (4 codes) -> 4
// bf16 in LDS.
template <int Q>
__device__ __forceinline__ void store_b_quarter(uint16_t* Bs, const BRegs<false>& rb, float a,
                                                const float2* ptab) {
  const int t = threadIdx.x;
  const uint32_t word = rb.w[Q >> 1];
  u32x2 o;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float2 c = pair_of(ptab, word, 2 * (Q & 1) + p);
    o[p] = pack_bf16x2(__fmul_rn(c.x, a), __fmul_rn(c.y, a));
  }
  *reinterpret_cast<u32x2*>(Bs + (t >> 2) * LDS_STRIDE + (t & 3) * 16 + Q * 4) = o;
}

struct Scales4 {
  float a[BW_ROWS];
};

__device__ __forceinline__ Scales4 stage_scale(const BRegs<true>& rb, bool, float off,
                                               const float* c8) {
  Scales4 s;
#pragma unroll
  for (int i = 0; i < BW_ROWS; ++i)
    s.a[i] = ((rb.vmask >> i) & 1u) ? decode_scale(c8[(rb.q >> (8 * i)) & 0xFFu], rb.nest[i], off)
                                    : 0.0f;
  return s;
}

// Quarter Q of a backward stage: output columns 2Q and 2Q+1 of the thread's
// 2x8 patch (byte Q of each row's word), each written as 2 consecutive
// contraction values -- the transpose into the matrix-core layout happens here,
// in the bf16 pairing.
template <int Q>
__device__ __forceinline__ void store_b_quarter(uint16_t* Bs, const BRegs<true>& rb,
                                                const Scales4& sc, const float2* ptab) {
  const int t = threadIdx.x;
  const int cb = 8 * (t & 15) + 2 * Q;
  const int rbase = BW_ROWS * (t >> 4);
  const float2 c0 = pair_of(ptab, rb.w[0], Q);
  const float2 c1 = pair_of(ptab, rb.w[1], Q);
  const uint32_t p0 = pack_bf16x2(__fmul_rn(c0.x, sc.a[0]), __fmul_rn(c1.x, sc.a[1]));
  const uint32_t p1 = pack_bf16x2(__fmul_rn(c0.y, sc.a[0]), __fmul_rn(c1.y, sc.a[1]));
  *reinterpret_cast<uint32_t*>(Bs + cb * LDS_STRIDE + rbase) = p0;
  *reinterpret_cast<uint32_t*>(Bs + (cb + 1) * LDS_STRIDE + rbase) = p1;
}

template <typename R, typename S>
__device__ __forceinline__ void store_b_all(uint16_t* Bs, const R& rb, const S& sc,
                                            const float2* ptab) {
  store_b_quarter<0>(Bs, rb, sc, ptab);
  store_b_quarter<1>(Bs, rb, sc, ptab);
  store_b_quarter<2>(Bs, rb, sc, ptab);
  store_b_quarter<3>(Bs, rb, sc, ptab);
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* base, int row, int kofs) {
  return *reinterpret_cast<const bf16x8_t*>(base + row * LDS_STRIDE + kofs);
}

__device__ __forceinline__ bf16x8_t f32x8_to_bf16(const float* v) {
  u32x4 u;
  u[0] = pack_bf16x2(v[0], v[1]);
  u[1] = pack_bf16x2(v[2], v[3]);
  u[2] = pack_bf16x2(v[4], v[5]);
  u[3] = pack_bf16x2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ WLanes<false> w_lanes(const GemmArgs& g, int64_t n0, WLanes<false>*) {
  return w_lanes_fwd(g, n0);
}
__device__ __forceinline__ WLanes<true> w_lanes(const GemmArgs& g, int64_t n0, WLanes<true>*) {
  return w_lanes_bwd(g, n0);
}

// SPLIT selects the output path (fp32 partials vs bf16 result) at compile time,
// so the two variants also carry distinct kernel names in profiles.
template <bool BWD, bool SPLIT>
__global__ __launch_bounds__(THREADS, 1) void k_gemm(GemmArgs g, Tables tab) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];
  __shared__ float2 s_pair_all[256 * PAIR_COPIES];
  __shared__ float s_c8[256];

  const int t = threadIdx.x;
  if (t < 256) {
    const float2 e = make_float2(tab.c4[t >> 4], tab.c4[t & 15]);
#pragma unroll
    for (int c = 0; c < PAIR_COPIES; ++c) s_pair_all[t * PAIR_COPIES + c] = e;
    s_c8[t] = tab.c8[t];
  }
  const float2* s_pair = s_pair_all + (t & (PAIR_COPIES - 1));

  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int split = blockIdx.z;
  const int64_t kb = split * g.kc_chunk;
  const int64_t ke = (kb + g.kc_chunk < g.Kc) ? kb + g.kc_chunk : g.Kc;
  const int nk = (int)((ke - kb + BK - 1) / BK);
  const float off = g.offset[0];

  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave >> 1;  // 64-row quarter of the tile
  const int wn = wave & 1;   // 64-column half of the tile
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const ALanes al = a_lanes(g, m0);
  const WLanes<BWD> wl = w_lanes(g, n0, static_cast<WLanes<BWD>*>(nullptr));
  bool fwd_valid = true;
  if constexpr (!BWD) fwd_valid = wl.valid;

  // step kt (clamped to the last one for prefetches past the end)
  auto step_of = [&](int kt) {
    const int k = kt < nk ? kt : nk - 1;
    Step s;
    s.nom = kb + (int64_t)k * BK;
    s.win = s.nom + BK <= g.Kc ? s.nom : g.Kc - BK;
    return s;
  };

  // Software pipeline over contraction steps. Weight stage k lives in register
  // slot k%4 and activation stage k in slot k%2; both are fetched two steps
  // before use. Step kt feeds the matrix cores from LDS stage kt%2 while it
  // decodes weight stage kt+1 into the other LDS stage (a quarter before each
  // group of 8 MFMAs), fetches weight stage kt+3 and activation stage kt+2, and
  // finally stores activation stage kt+1.
  BRegs<BWD> rb0, rb1, rb2, rb3;
  u32x4 ra0[A_CHUNKS], ra1[A_CHUNKS];
  load_b(g, wl, step_of(0), rb0);
  load_b(g, wl, step_of(1), rb1);
  load_b(g, wl, step_of(2), rb2);
  load_a(g, al, step_of(0).win, ra0);
  load_a(g, al, step_of(1).win, ra1);
  __syncthreads();  // tables in LDS
  store_a(As[0], ra0);
  store_b_all(Bs[0], rb0, stage_scale(rb0, fwd_valid, off, s_c8), s_pair);
  __syncthreads();

  // MFMAs of one step from LDS stage st, fragments double-buffered across the
  // four 16-wide sub-steps, with one quarter of the next weight stage decoded
  // into the other LDS stage before each group of 8 MFMAs.
  auto mma_and_decode = [&](int st, const BRegs<BWD>& w_deq) {
    const auto sc = stage_scale(w_deq, fwd_valid, off, s_c8);
    const uint16_t* as = As[st];
    const uint16_t* bs = Bs[st];
    uint16_t* bnext = Bs[st ^ 1];
    bf16x8_t fa[2][2], fb[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[0][i] = lds_frag(as, wm * 64 + i * 32 + lrow, lk);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[0][j] = lds_frag(bs, wn * 64 + j * 32 + lrow, lk);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          fa[cur ^ 1][i] = lds_frag(as, wm * 64 + i * 32 + lrow, (kk + 1) * 16 + lk);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[cur ^ 1][j] = lds_frag(bs, wn * 64 + j * 32 + lrow, (kk + 1) * 16 + lk);
      }
      if (kk == 0) store_b_quarter<0>(bnext, w_deq, sc, s_pair);
      if (kk == 1) store_b_quarter<1>(bnext, w_deq, sc, s_pair);
      if (kk == 2) store_b_quarter<2>(bnext, w_deq, sc, s_pair);
      if (kk == 3) store_b_quarter<3>(bnext, w_deq, sc, s_pair);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
  };

  // One step over named ring registers (a macro, so nothing is address-taken
  // and every ring slot stays in VGPRs).
#define NF4S_GEMM_STEP(KT, WL, WD, AL, AS)            \
  do {                                                \
    const int kt_ = (KT);                             \
    load_b(g, wl, step_of(kt_ + 3), WL);              \
    load_a(g, al, step_of(kt_ + 2).win, AL);          \
    __builtin_amdgcn_sched_barrier(0);                \
    mma_and_decode(kt_ & 1, WD);                      \
    store_a(As[(kt_ & 1) ^ 1], AS);                   \
    __syncthreads();                                  \
  } while (0)

  const int nk4 = nk - nk % 4;
  for (int kt = 0; kt < nk4; kt += 4) {
    NF4S_GEMM_STEP(kt, rb3, rb1, ra0, ra1);
    NF4S_GEMM_STEP(kt + 1, rb0, rb2, ra1, ra0);
    NF4S_GEMM_STEP(kt + 2, rb1, rb3, ra0, ra1);
    NF4S_GEMM_STEP(kt + 3, rb2, rb0, ra1, ra0);
  }
  if (nk4 < nk) NF4S_GEMM_STEP(nk4, rb3, rb1, ra0, ra1);
  if (nk4 + 1 < nk) NF4S_GEMM_STEP(nk4 + 1, rb0, rb2, ra1, ra0);
  if (nk4 + 2 < nk) NF4S_GEMM_STEP(nk4 + 2, rb1, rb3, ra0, ra1);
#undef NF4S_GEMM_STEP

  // LoRA term, contracted on the matrix cores in chunks of 16 over the rank:
  // forward  + u[m, :] . (s * B[n, :]),  backward + du[m, :] . A[:, n].
  if (g.lora_l != nullptr && split == 0) {
    for (int r0 = 0; r0 < g.r; r0 += 16) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t row = m0 + wm * 64 + i * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (row < g.M && rr < g.r) ? g.lora_l[row * g.r + rr] : 0.0f;
        }
        fa[i] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 64 + j * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          float x = 0.0f;
          if (col < g.Nc && rr < g.r)
            x = BWD ? g.lora_r[(int64_t)rr * g.k_in + col] : g.scale * g.lora_r[col * g.r + rr];
          v[e] = x;
        }
        fb[j] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 tile.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + lrow;
      if (col >= g.Nc) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        if (SPLIT) {
          g.part[((int64_t)split * g.M + row) * g.Nc + col] = acc[i][j][r];
        } else {
          g.out[row * g.Nc + col] = (uint16_t)(pack_bf16x2(acc[i][j][r], 0.0f) & 0xFFFFu);
        }
      }
    }
  }
}

// Sum of the split partials in split order, rounded once to bf16.
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int splits,
                                                   int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    float4 s = *reinterpret_cast<const float4*>(part + i);
    for (int p = 1; p < splits; ++p) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)p * n + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(out + i) = o;
  } else {
    for (int64_t e = i; e < n; ++e) {
      float s = part[e];
      for (int p = 1; p < splits; ++p) s += part[(int64_t)p * n + e];
      out[e] = (uint16_t)(pack_bf16x2(s, 0.0f) & 0xFFFFu);
    }
  }
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t n_cols, int64_t k_contract) {
  GemmPlan p;
  p.bm = BM;
  p.bn = BN;
  const int64_t tiles = ((M + BM - 1) / BM) * ((n_cols + BN - 1) / BN);
  const int64_t nk = (k_contract + BK - 1) / BK;
  int splits = 1;
  // Split the contraction while the grid is short of the chip's 256 CUs and
  // each split keeps at least 8 contraction steps.
  while (tiles * splits < 192 && nk / (2 * splits) >= 8) splits *= 2;
  const int64_t steps_per = (nk + splits - 1) / splits;
  p.kc_chunk = steps_per * BK;
  p.splits = (int)((nk + steps_per - 1) / steps_per);
  p.ws_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)n_cols * sizeof(float) : 0;
  return p;
}

hipError_t launch_linear(bool backward, const QPtrs& q, int64_t n_out, int64_t k_in,
                         const uint16_t* a, int64_t M, uint16_t* out, const float* lora_l,
                         const float* lora_r, int r, float scale, void* ws, hipStream_t s) {
  GemmArgs g;
  g.packed = q.packed;
  g.q8 = q.q8;
  g.nested = q.nested;
  g.offset = q.offset;
  g.a = a;
  g.M = M;
  g.Kc = backward ? n_out : k_in;
  g.Nc = backward ? k_in : n_out;
  g.n_out = n_out;
  g.k_in = k_in;
  g.out = out;
  const GemmPlan p = plan_gemm(M, g.Nc, g.Kc);
  g.part = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
  g.kc_chunk = p.kc_chunk;
  g.lora_l = lora_l;
  g.lora_r = lora_r;
  g.r = r;
  g.scale = scale;
  const dim3 grid((unsigned)((g.Nc + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)p.splits);
  const bool split = p.splits > 1;
  if (backward && split)
    hipLaunchKernelGGL((k_gemm<true, true>), grid, dim3(THREADS), 0, s, g, host_tables());
  else if (backward)
    hipLaunchKernelGGL((k_gemm<true, false>), grid, dim3(THREADS), 0, s, g, host_tables());
  else if (split)
    hipLaunchKernelGGL((k_gemm<false, true>), grid, dim3(THREADS), 0, s, g, host_tables());
  else
    hipLaunchKernelGGL((k_gemm<false, false>), grid, dim3(THREADS), 0, s, g, host_tables());
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = M * g.Nc;
  const dim3 g2((unsigned)((n / 4 + 1 + 255) / 256));
  hipLaunchKernelGGL(k_split_sum, g2, dim3(256), 0, s, g.part, p.splits, n, out);
  return hipGetLastError();
}

}  // namespace nf4s
