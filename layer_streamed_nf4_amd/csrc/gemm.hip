// Fused NF4-dequant bf16 MFMA GEMMs for the frozen linears.
//
// Forward  y[M, n_out]  = x[M, k_in] . W'^T   (+ s . u . B^T)
// Backward dx[M, k_in]  = dy[M, n_out] . W'   (+ du . A)
// Gate walkthrough ("Soup layer-streamed NF4 training measured") section 2.1:
// the NF4 weight is rebuilt from the streamed bytes on every call and used with
// bf16 compute; section 4.4: the frozen base needs dL/dx but no dL/dW.
//
// Both directions are one kernel template computing C[M, Nc] = A[M, Kc] . B,
// where A is the bf16 activation (x or dy) and B[Kc, Nc] is the dequantised
// weight seen either transposed (forward: B[k][n] = W'[n][k]) or as is
// (backward: B[k][n] = W'[k][n]). The packed codes are read from HBM once per
// workgroup, decoded in registers with the block scale
// a' = fp32(fp32(C8[q8]*nested) + offset) and W' = bf16_rne(fp32(C4[code]*a')),
// and written to LDS as bf16 in the contraction-major layout the matrix cores
// read; W' never goes back to HBM. A packed byte holds two codes, and one LDS
// read of a 256-entry table gives both of their NF4 levels; the table is
// replicated 16 times so that lane l always reads the copy that lives in bank
// pair (2(l%16), 2(l%16)+1), which makes the random lookups conflict-free.
// The backward orientation is transposed on the way into LDS for free: a
// thread decodes a 2x8 patch and pairs values along the contraction when it
// packs bf16.
//
// Tiling for gfx950, sized by its LDS bandwidth (about 128 B per clock per
// CU), its vector-memory path (about 64 B per clock per CU, and only when
// every four consecutive lanes read contiguous bytes) and the issue slots a
// wave leaves between its MFMAs:
//  * output tile 256x128 per workgroup, contraction step 64 (one NF4 block per
//    weight row in the forward direction), v_mfma_f32_32x32x16_bf16;
//  * 512 threads = 8 waves, two per SIMD. Waves w and w+4 own the same 64
//    output rows x all 128 columns (2x4 MFMA tiles, 128 fp32 accumulators per
//    lane) and split every step's contraction: w takes sub-steps 0-1, w+4
//    sub-steps 2-3. Their accumulators are summed through LDS once, at the
//    end. Each SIMD thus runs 32 MFMAs per step from two waves, so one wave's
//    decode work and waits overlap the other's matrix work;
//  * the activation operand never touches LDS: a first kernel rewrites it in
//    MFMA fragment order (k_frag_pack), and each wave loads its fragments
//    with contiguous 1 KB reads into a register ring two steps ahead;
//  * the decoded weights go through a three-stage LDS ring: step s multiplies
//    stage s, decodes stage s+2 and, before its barrier, already reads the
//    first fragments of stage s+1, so the matrix cores restart without an
//    LDS round trip after the barrier.
// LDS traffic per step: 64 KB of weight fragments, 32 KB of table lookups and
// 16 KB of decoded stores, against 1024 MFMA cycles per SIMD.
// LDS rows are padded to 144 B so the 16-byte fragment reads of 8 consecutive
// lanes cover all 32 banks; in the backward orientation the 16-byte chunks of
// a column are XOR-swizzled by the column's 8-group so the transposing stores
// of a row of lanes spread over the banks. When the output has too few tiles
// to occupy the chip, the contraction is split; each split writes fp32
// partials and a second kernel sums them in split order (deterministic, no
// atomics).
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int WAVE_ROWS = 64;         // output rows per wave (waves w and w+4 share them)
constexpr int NSTAGE = 3;             // LDS ring of decoded weight stages
constexpr int LDS_STRIDE = 72;        // bf16 elements per LDS row (64 + 8 pad = 144 B)
constexpr int STAGE_ELEMS = BN * LDS_STRIDE;
constexpr int PAIR_COPIES = 16;
constexpr int SMEM_BYTES = NSTAGE * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8 + 256 * 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* q8;
  const float* nested;
  const float* offset;
  const uint8_t* afrag;  // activation in fragment order (see k_frag_pack)
  int64_t kblocks;       // 16-wide contraction blocks per 32-row block of afrag
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

// A contraction step covers [k0, k0 + 64). The packed activation is zero past
// the contraction length Kc, and in the backward direction (Kc = n_out, a
// multiple of 8 only) weight rows at or past Kc decode to zero.
struct Step {
  int64_t k0;
};

// ---- activation operand (A) -----------------------------------------------
// For sub-step kk the 32x32x16 MFMA takes from lane l row l%32 of its 32-row
// tile and contraction elements kk*16 + 8*(l/32) .. +8 (16 bytes). A row-major
// activation puts consecutive lanes in different rows, which the vector memory
// path serves at a quarter of its rate, so a first kernel rewrites A in
// fragment order: 1 KB per (32-row block, 16-wide contraction block), lane
// after lane, zero-padded to whole 256-row tiles and 64-wide steps. Every
// fragment load of the GEMM is then one contiguous 1 KB read.
constexpr int FRAG_BYTES = 1024;

// One workgroup per (32-row block, 64-wide contraction step): read the 32x64
// bf16 tile row by row (8 lanes per 128-byte row), transpose it through LDS,
// write the four 1 KB fragments in lane order. Both global sides move whole
// 64-byte runs per 4 lanes.
__global__ __launch_bounds__(256) void k_frag_pack(const uint16_t* __restrict__ a, int64_t M,
                                                   int64_t Kc, int64_t kblocks,
                                                   uint8_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[32 * 144];
  const int t = threadIdx.x;
  const int64_t steps = kblocks / 4;
  const int64_t b = blockIdx.x / steps;  // 32-row block
  const int64_t st = blockIdx.x % steps; // 64-wide step
  {
    const int r = t >> 3, c = t & 7;
    const int64_t row = 32 * b + r;
    const int64_t k = 64 * st + 8 * c;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < M && k < Kc) v = *reinterpret_cast<const u32x4*>(a + row * Kc + k);
    *reinterpret_cast<u32x4*>(tile + r * 144 + c * 16) = v;
  }
  __syncthreads();
  const int f = t >> 6, lane = t & 63;  // fragment (16-wide block) and its lane
  const u32x4 v = *reinterpret_cast<const u32x4*>(tile + (lane & 31) * 144 + (2 * f + (lane >> 5)) * 16);
  *reinterpret_cast<u32x4*>(out + ((b * kblocks + 4 * st + f) * 64 + lane) * 16) = v;
}

struct AFrags {
  u32x4 f[2][2];  // [row tile i][own sub-step]
};

struct ALanes {
  uint32_t off[2];  // byte offsets of the lane's chunk in its two 32-row blocks at contraction 0
};

// Wave rows: group g = wave % 4; contraction half h = wave / 4.
__device__ __forceinline__ ALanes a_lanes(const GemmArgs& g, int64_t m0, int grp, int half,
                                          int lane) {
  ALanes L;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t blk = (m0 + grp * WAVE_ROWS + i * 32) / 32;
    L.off[i] = (uint32_t)(blk * g.kblocks * FRAG_BYTES + (2 * half) * FRAG_BYTES + lane * 16);
  }
  return L;
}

__device__ __forceinline__ void load_a(const GemmArgs& g, const ALanes& L, int64_t k0,
                                       AFrags& r) {
  const uint8_t* base = g.afrag + (k0 / 16) * FRAG_BYTES;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      r.f[i][kk] = *reinterpret_cast<const u32x4*>(base + L.off[i] + kk * FRAG_BYTES);
}

// ---- weight tile (B) ------------------------------------------------------
template <bool BWD>
struct WLanes;
template <bool BWD>
struct BRegs;

// Forward: thread t owns weight row n0 + t/4 and contraction quarter t%4
// (16 codes, two packed words).
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
  rb.w = *reinterpret_cast<const u32x2*>(g.packed + s.k0 / 2 + L.woff);
  const uint32_t blk = L.blk0 + (uint32_t)(s.k0 / 64);
  rb.q = g.q8[blk];
  rb.nest = g.nested[blk >> 8];
}

// Backward: thread t owns weight rows k0 + 2*(t/16) + i (i < 2) and output
// columns n0 + 8*(t%16) + j (j < 8): two packed words, two 8-bit scale codes
// packed in one register, two nested scales, a 2-bit validity mask.
template <>
struct WLanes<true> {
  uint32_t woff[2];  // byte offsets of the packed words at contraction 0
  uint32_t blk0[2];  // 64-block indices at contraction 0
  uint32_t col;      // first (clamped) column
  bool cvalid;       // columns < k_in
};
template <>
struct BRegs<true> {
  uint32_t w[2];
  uint32_t q;
  float nest[2];
  uint32_t vmask;
};

__device__ __forceinline__ WLanes<true> w_lanes_bwd(const GemmArgs& g, int64_t n0) {
  const int t = threadIdx.x;
  WLanes<true> L;
  int64_t col = n0 + 8 * (t & 15);
  L.cvalid = col < g.k_in;
  col = L.cvalid ? col : g.k_in - 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t row = 2 * (t >> 4) + i;  // relative to the step's start
    L.woff[i] = (uint32_t)((row * g.k_in + col) / 2);
    L.blk0[i] = (uint32_t)((row * g.k_in + col) / 64);
  }
  L.col = (uint32_t)col;
  return L;
}

__device__ __forceinline__ void load_b(const GemmArgs& g, const WLanes<true>& L, Step s,
                                       BRegs<true>& rb) {
  const int t = threadIdx.x;
  rb.q = 0;
  if (s.k0 + BK <= g.Kc) {  // uniform: every row of the step exists
    const uint8_t* base = g.packed + s.k0 * (g.k_in / 2);
    const uint32_t bstep = (uint32_t)(s.k0 * (g.k_in / 64));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rb.w[i] = *reinterpret_cast<const uint32_t*>(base + L.woff[i]);
      const uint32_t blk = bstep + L.blk0[i];
      rb.q |= (uint32_t)g.q8[blk] << (8 * i);
      rb.nest[i] = g.nested[blk >> 8];
    }
    rb.vmask = L.cvalid ? 0x3u : 0u;
  } else {  // the last step of a contraction that is not a multiple of 64
    rb.vmask = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = s.k0 + 2 * (t >> 4) + i;
      const bool ok = row < g.Kc;
      const int64_t e = (ok ? row : g.Kc - 1) * g.k_in + L.col;  // code index
      rb.w[i] = *reinterpret_cast<const uint32_t*>(g.packed + e / 2);
      const uint32_t blk = (uint32_t)(e / 64);
      rb.q |= (uint32_t)g.q8[blk] << (8 * i);
      rb.nest[i] = g.nested[blk >> 8];
      rb.vmask |= (L.cvalid && ok) ? (1u << i) : 0u;
    }
  }
}

// ---- decoding -------------------------------------------------------------
// Pair table: entry b = (C4[b >> 4], C4[b & 15]), both levels of a packed byte,
// the even element (high nibble) first. Copy c of entry b sits at float2 index
// 16*b + c, i.e. dwords 32*b + 2c and 32*b + 2c + 1: the copy fixes the LDS
// bank pair whatever b is. `ptab` below is already offset by the lane's copy.
__device__ __forceinline__ float2 pair_of(const float2* ptab, uint32_t word, int byte) {
  return ptab[((word >> (8 * byte)) & 0xFFu) * PAIR_COPIES];
}

// All table reads of a stage are issued together, ahead of the arithmetic
// that consumes them, so their LDS latencies overlap.
struct Pairs {
  float2 v[8];  // forward: [word * 4 + byte]; backward: [byte * 2 + row]
};

__device__ __forceinline__ float stage_scale(const BRegs<false>& rb, bool valid, float off,
                                             const float* c8) {
  const float a = decode_scale(c8[rb.q], rb.nest, off);
  return valid ? a : 0.0f;
}

__device__ __forceinline__ void load_pairs(const BRegs<false>& rb, const float2* ptab, Pairs& pr) {
#pragma unroll
  for (int jw = 0; jw < 2; ++jw)
#pragma unroll
    for (int p = 0; p < 4; ++p) pr.v[jw * 4 + p] = pair_of(ptab, rb.w[jw], p);
}

// Forward stage: the thread's 16 codes -> 16 bf16 of its weight row in LDS.
__device__ __forceinline__ void store_b(uint16_t* Bs, const Pairs& pr, float a) {
  const int t = threadIdx.x;
#pragma unroll
  for (int jw = 0; jw < 2; ++jw) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float2 c = pr.v[jw * 4 + p];
      o[p] = pack_bf16x2(__fmul_rn(c.x, a), __fmul_rn(c.y, a));
    }
    *reinterpret_cast<u32x4*>(Bs + (t >> 2) * LDS_STRIDE + (t & 3) * 16 + jw * 8) = o;
  }
}

struct Scales2 {
  float a[2];
};

__device__ __forceinline__ Scales2 stage_scale(const BRegs<true>& rb, bool, float off,
                                               const float* c8) {
  Scales2 s;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float a = decode_scale(c8[(rb.q >> (8 * i)) & 0xFFu], rb.nest[i], off);
    s.a[i] = ((rb.vmask >> i) & 1u) ? a : 0.0f;
  }
  return s;
}

__device__ __forceinline__ void load_pairs(const BRegs<true>& rb, const float2* ptab, Pairs& pr) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 2; ++i) pr.v[q * 2 + i] = pair_of(ptab, rb.w[i], q);
}

// Backward LDS layout: stage[col][k] with the 16-byte chunk k/8 of column col
// stored at chunk (k/8) ^ ((col/8) % 8).
__device__ __forceinline__ int bwd_swizzle_off(int col, int k) {
  return ((((k >> 3) ^ (col >> 3)) & 7) << 3) | (k & 7);
}

// Backward stage: byte q of each of the thread's two row words gives output
// columns 2q and 2q+1 of its 2x8 patch, each written as 2 consecutive
// contraction values -- the transpose into the matrix-core layout happens
// here, in the bf16 pairing.
__device__ __forceinline__ void store_b(uint16_t* Bs, const Pairs& pr, const Scales2& sc) {
  const int t = threadIdx.x;
  const int r0 = 2 * (t >> 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float2 c0 = pr.v[q * 2 + 0];
    const float2 c1 = pr.v[q * 2 + 1];
    const int cb = 8 * (t & 15) + 2 * q;
    const uint32_t p0 = pack_bf16x2(__fmul_rn(c0.x, sc.a[0]), __fmul_rn(c1.x, sc.a[1]));
    const uint32_t p1 = pack_bf16x2(__fmul_rn(c0.y, sc.a[0]), __fmul_rn(c1.y, sc.a[1]));
    *reinterpret_cast<uint32_t*>(Bs + cb * LDS_STRIDE + bwd_swizzle_off(cb, r0)) = p0;
    *reinterpret_cast<uint32_t*>(Bs + (cb + 1) * LDS_STRIDE + bwd_swizzle_off(cb + 1, r0)) = p1;
  }
}

// B fragment j (columns 32j .. 32j+31) of sub-step kk from an LDS stage:
// lane l reads column 32j + l%32, contraction kk*16 + 8*(l/32) .. +8.
template <bool BWD>
__device__ __forceinline__ bf16x8_t b_frag(const uint16_t* bs, int lane, int j, int kk) {
  const int col = 32 * j + (lane & 31);
  const int k = kk * 16 + 8 * (lane >> 5);
  const int e = BWD ? bwd_swizzle_off(col, k) : k;
  return *reinterpret_cast<const bf16x8_t*>(bs + col * LDS_STRIDE + e);
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
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_BYTES];
  uint16_t* const Bs0 = reinterpret_cast<uint16_t*>(smem);
  float2* const s_pair_all = reinterpret_cast<float2*>(smem + NSTAGE * STAGE_ELEMS * 2);
  float* const s_c8 = reinterpret_cast<float*>(smem + NSTAGE * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8);

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
  const int grp = wave & 3;   // 64-row group of the tile
  const int half = wave >> 2;  // contraction half of every step
  const int lane = t & 63;
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const ALanes al = a_lanes(g, m0, grp, half, lane);
  const WLanes<BWD> wl = w_lanes(g, n0, static_cast<WLanes<BWD>*>(nullptr));
  bool fwd_valid = true;
  if constexpr (!BWD) fwd_valid = wl.valid;

  // step kt (clamped to the last one for prefetches past the end)
  auto step_of = [&](int kt) {
    const int k = kt < nk ? kt : nk - 1;
    Step s;
    s.k0 = kb + (int64_t)k * BK;
    return s;
  };
  auto stage = [&](int st) { return Bs0 + st * STAGE_ELEMS; };
  auto decode = [&](uint16_t* bs, const BRegs<BWD>& W) {
    const auto sc = stage_scale(W, fwd_valid, off, s_c8);
    Pairs pr;
    load_pairs(W, s_pair, pr);
    store_b(bs, pr, sc);
  };

  // Pipeline: activation stage k lives in register slot k%3 and is fetched two
  // steps before use; weight stage k lives in register slot k%3, is fetched
  // two steps before it is decoded, and is decoded into LDS stage k%3 two
  // steps before the matrix cores read it.
  BRegs<BWD> wb0, wb1, wb2;
  AFrags ar0, ar1, ar2;
  load_b(g, wl, step_of(0), wb0);
  load_b(g, wl, step_of(1), wb1);
  load_b(g, wl, step_of(2), wb2);
  load_a(g, al, step_of(0).k0, ar0);
  load_a(g, al, step_of(1).k0, ar1);
  __syncthreads();  // tables in LDS
  decode(stage(0), wb0);
  load_b(g, wl, step_of(3), wb0);
  decode(stage(1), wb1);
  __syncthreads();

  const int kk0 = 2 * half;  // the wave's first sub-step
  bf16x8_t fb0[4];           // its fragments of the stage about to be multiplied
#pragma unroll
  for (int j = 0; j < 4; ++j) fb0[j] = b_frag<BWD>(stage(0), lane, j, kk0);

  auto mfma_kk = [&](const AFrags& A, int kk, const bf16x8_t* fb) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, A.f[i][kk]), fb[j], acc[i][j], 0, 0, 0);
  };

  // One step: multiply the wave's two sub-steps of LDS stage `bs` (the first
  // one's fragments already in fb0), decode weight registers `W` into LDS
  // stage `bdec`, and read the first fragments of the next stage `bnext`.
  auto compute = [&](const uint16_t* bs, uint16_t* bdec, const uint16_t* bnext, const AFrags& A,
                     const BRegs<BWD>& W) {
    const auto sc = stage_scale(W, fwd_valid, off, s_c8);
    Pairs pr;
    load_pairs(W, s_pair, pr);
    bf16x8_t fb1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fb1[j] = b_frag<BWD>(bs, lane, j, kk0 + 1);
    mfma_kk(A, 0, fb0);
    store_b(bdec, pr, sc);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb0[j] = b_frag<BWD>(bnext, lane, j, kk0);
    mfma_kk(A, 1, fb1);
  };

  // One step over named ring registers (a macro, so nothing is address-taken
  // and every ring slot stays in VGPRs). SM = step % 3.
#define NF4S_GEMM_STEP(KT, SM, ACUR, ALD, WDEC, WLD)                                  \
  do {                                                                                \
    const int kt_ = (KT);                                                             \
    load_a(g, al, step_of(kt_ + 2).k0, ALD);                                          \
    load_b(g, wl, step_of(kt_ + 4), WLD);                                             \
    __builtin_amdgcn_sched_barrier(0);                                                \
    compute(stage(SM), stage(((SM) + 2) % 3), stage(((SM) + 1) % 3), ACUR, WDEC);     \
    __syncthreads();                                                                  \
  } while (0)

  const int nk3 = nk - nk % 3;
  for (int kt = 0; kt < nk3; kt += 3) {
    NF4S_GEMM_STEP(kt, 0, ar0, ar2, wb2, wb1);
    NF4S_GEMM_STEP(kt + 1, 1, ar1, ar0, wb0, wb2);
    NF4S_GEMM_STEP(kt + 2, 2, ar2, ar1, wb1, wb0);
  }
  if (nk3 < nk) NF4S_GEMM_STEP(nk3, 0, ar0, ar2, wb2, wb1);
  if (nk3 + 1 < nk) NF4S_GEMM_STEP(nk3 + 1, 1, ar1, ar0, wb0, wb2);
#undef NF4S_GEMM_STEP

  // Sum the two contraction halves through LDS (the weight ring is free now):
  // the wave of half h finishes column tiles j = 2h, 2h+1, so it hands the
  // other two to its partner. Exchange slot of a tile: 16 registers x 64 lanes.
  {
    float* xch = reinterpret_cast<float*>(smem);
    auto slot = [&](int g4, int i, int jj, int r) { return ((((g4 * 2 + i) * 2 + jj) * 16 + r) * 64 + lane); };
    // round h: the half-(1-h) waves export tiles j = 2h + jj, the half-h waves add them
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (half != h) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) xch[slot(grp, i, jj, r)] = acc[i][2 * h + jj][r];
      }
      __syncthreads();
      if (half == h) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][2 * h + jj][r] += xch[slot(grp, i, jj, r)];
      }
      __syncthreads();
    }
  }

  // From here each wave owns row tiles i = 0, 1 of its group and column tiles
  // j = 2*half + jj.
  // LoRA term, contracted on the matrix cores in chunks of 16 over the rank:
  // forward  + u[m, :] . (s * B[n, :]),  backward + du[m, :] . A[:, n].
  if (g.lora_l != nullptr && split == 0) {
    for (int r0 = 0; r0 < g.r; r0 += 16) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t row = m0 + grp * WAVE_ROWS + i * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (row < g.M && rr < g.r) ? g.lora_l[row * g.r + rr] : 0.0f;
        }
        fa[i] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int64_t col = n0 + (2 * half + jj) * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          float x = 0.0f;
          if (col < g.Nc && rr < g.r)
            x = BWD ? g.lora_r[(int64_t)rr * g.k_in + col] : g.scale * g.lora_r[col * g.r + rr];
          v[e] = x;
        }
        fb[jj] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          f32x16_t& c = half ? acc[i][2 + jj] : acc[i][jj];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[jj], c, 0, 0, 0);
        }
    }
  }

  // Accumulator layout of v_mfma_f32_32x32x16: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 tile. The tile goes
  // out through LDS so that every global store writes 16 contiguous bytes
  // (bf16: the whole 256x128 tile at once; fp32 partials: 128 rows at a time).
  __syncthreads();  // the exchange buffer is reused
  if constexpr (!SPLIT) {
    constexpr int OS = BN + 8;  // bf16 per LDS row
    uint16_t* ot = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const f32x16_t& c = half ? acc[i][2 + jj] : acc[i][jj];
        const int col = (2 * half + jj) * 32 + lrow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = grp * WAVE_ROWS + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          ot[row * OS + col] = (uint16_t)(pack_bf16x2(c[r], 0.0f) & 0xFFFFu);
        }
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < BM * BN / 8 / THREADS; ++it) {
      const int q = it * THREADS + t;  // 16-byte chunk of the tile
      const int row = q / (BN / 8), c8 = q % (BN / 8);
      const int64_t grow = m0 + row, gcol = n0 + 8 * c8;
      if (grow < g.M && gcol < g.Nc)
        *reinterpret_cast<u32x4*>(g.out + grow * g.Nc + gcol) =
            *reinterpret_cast<const u32x4*>(ot + row * OS + 8 * c8);
    }
  } else {
    constexpr int OS = BN + 4;  // fp32 per LDS row
    float* ot = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {  // rows [128 ph, 128 ph + 128): groups 2ph, 2ph+1
      if ((grp >> 1) == ph) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const f32x16_t& c = half ? acc[i][2 + jj] : acc[i][jj];
            const int col = (2 * half + jj) * 32 + lrow;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = (grp & 1) * WAVE_ROWS + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              ot[row * OS + col] = c[r];
            }
          }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 128 * BN / 4 / THREADS; ++it) {
        const int q = it * THREADS + t;
        const int row = q / (BN / 4), c4 = q % (BN / 4);
        const int64_t grow = m0 + 128 * ph + row, gcol = n0 + 4 * c4;
        if (grow < g.M && gcol < g.Nc)
          *reinterpret_cast<u32x4*>(g.part + ((int64_t)split * g.M + grow) * g.Nc + gcol) =
              *reinterpret_cast<const u32x4*>(ot + row * OS + 4 * c4);
      }
      __syncthreads();
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

size_t packed_activation_bytes(int64_t M, int64_t K) {
  return (size_t)((M + BM - 1) / BM * BM) * (size_t)((K + BK - 1) / BK * BK) * 2;
}

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
  p.frag_bytes = packed_activation_bytes(M, k_contract);
  p.part_bytes = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)n_cols * sizeof(float) : 0;
  p.ws_bytes = p.frag_bytes + p.part_bytes;
  return p;
}

hipError_t launch_pack(const uint16_t* a, int64_t M, int64_t K, uint8_t* packed, hipStream_t s) {
  const int64_t kblocks = (K + BK - 1) / BK * (BK / 16);
  const int64_t packs = (int64_t)(packed_activation_bytes(M, K) / (4 * FRAG_BYTES));
  hipLaunchKernelGGL(k_frag_pack, dim3((unsigned)packs), dim3(256), 0, s, a, M, K, kblocks, packed);
  return hipGetLastError();
}

hipError_t launch_linear_packed(bool backward, const QPtrs& q, int64_t n_out, int64_t k_in,
                                const uint8_t* a_packed, int64_t M, uint16_t* out,
                                const float* lora_l, const float* lora_r, int r, float scale,
                                void* part_ws, hipStream_t s) {
  GemmArgs g;
  g.packed = q.packed;
  g.q8 = q.q8;
  g.nested = q.nested;
  g.offset = q.offset;
  g.M = M;
  g.Kc = backward ? n_out : k_in;
  g.Nc = backward ? k_in : n_out;
  g.n_out = n_out;
  g.k_in = k_in;
  g.out = out;
  const GemmPlan p = plan_gemm(M, g.Nc, g.Kc);
  g.afrag = a_packed;
  g.kblocks = (g.Kc + BK - 1) / BK * (BK / 16);
  g.part = p.splits > 1 ? static_cast<float*>(part_ws) : nullptr;
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
