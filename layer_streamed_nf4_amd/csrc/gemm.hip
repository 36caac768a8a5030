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
// replicated 32 times so that lane l always reads the copy that lives in bank
// pair (2(l%32), 2(l%32)+1) of the 64 LDS banks, which makes the random
// lookups of a half-wave conflict-free.
// The backward orientation is transposed on the way into LDS for free: a
// thread decodes a 4x8 patch and pairs values along the contraction when it
// packs bf16.
//
// Tiling for gfx950, sized by its LDS bandwidth (about 128 B per clock per
// CU), its vector-memory path (about 64 B per clock per CU, and only when
// every four consecutive lanes read contiguous bytes) and the issue slots a
// wave leaves between its MFMAs:
//  * output tile 256x128 per workgroup, contraction step 64 (one NF4 block per
//    weight row in the forward direction), v_mfma_f32_32x32x16_bf16;
//  * 512 threads = 8 waves, two per SIMD, with split roles. Waves 0-3 are the
//    consumers: each owns 64 output rows x all 128 columns (2x4 MFMA tiles,
//    128 fp32 accumulators per lane) and only loads its activation fragments
//    and multiplies. Waves 4-7 are the producers: they only stream the packed
//    weights and decode them into LDS. Every SIMD thus runs one wave of each
//    kind, so the decode's vector work and LDS waits overlap the other wave's
//    matrix work instead of competing with it step for step;
//  * the activation operand never touches LDS: it arrives in MFMA fragment
//    order (k_frag_pack, pack.hip), and each consumer loads its fragments
//    with contiguous 1 KB reads; a sub-step's registers are refilled for the
//    step two ahead as soon as its MFMAs are issued;
//  * the decoded weights go through a four-stage LDS ring with one barrier
//    per step: in step s the consumers multiply stage s and, before the
//    barrier, read the first fragments of stage s+1; the producers finish
//    stage s+2 from table lookups issued in step s-1, issue the lookups of
//    stage s+3, and fetch the packed codes of stage s+5.
// LDS traffic per step: 64 KB of weight fragments, 32 KB of table lookups and
// 16 KB of decoded stores, against 1024 MFMA cycles per SIMD.
// LDS rows are padded to 144 B so the 16-byte fragment reads of 8 consecutive
// lanes cover all 32 banks; in the backward orientation the 16-byte chunks of
// a column are XOR-swizzled by the column's 16-group so the transposing stores
// of a row of lanes spread over the banks. When the output has too few tiles
// to occupy the chip, the contraction is split; each split writes fp32
// partials and a second kernel sums them in split order (deterministic, no
// atomics).
#include "common.h"
#include "device.h"

namespace nf4s {
namespace {

constexpr int BM = PACK_ROWS;  // the packed activation is padded to whole output tiles
constexpr int BN = 128;
constexpr int BK = PACK_COLS;
constexpr int CONSUMERS = 4;          // waves 0-3 multiply, waves 4-7 decode
constexpr int THREADS = 64 * 2 * CONSUMERS;
constexpr int WAVE_ROWS = BM / CONSUMERS;  // 64 output rows per consumer wave
constexpr int NSTAGE = 4;             // LDS ring of decoded weight stages
constexpr int LDS_STRIDE = 72;        // bf16 elements per LDS row (64 + 8 pad = 144 B)
constexpr int STAGE_ELEMS = BN * LDS_STRIDE;
constexpr int PAIR_COPIES = 32;
// backward: the block scales of a stage (2 column blocks x 64 rows), a ring of NSTAGE
constexpr int SCALE_FLOATS = 2 * 64;
constexpr int SMEM_BYTES = NSTAGE * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8 + 256 * 4 +
                           NSTAGE * SCALE_FLOATS * 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs

// One weight of a grouped launch. Forward: up to GEMM_MAX_SEG NF4 linears
// that read the same activation (q, k and v; gate and up) run as one grid
// whose column tiles are dealt to the weights in order. Backward: the dx of
// such a group is one sum, dx = sum_j dy_j . W'_j, so the weights lie along
// the contraction instead; the grid's split index z is dealt to them in
// order (splits z0_j .. z0_{j+1}-1 cover weight j, each with its own dy_j),
// every split writes its own fp32 partial and one sum adds them all.
struct GemmSeg {
  const uint8_t* packed;
  const uint8_t* q8;
  const float* nested;
  const float* offset;
  uint16_t* out;         // bf16 [M, Nc]
  float* part;           // fp32 [splits, M, Nc] (splits > 1)
  const float* lora_l;   // fp32 [M, r]
  const float* lora_r;   // fwd: B fp32 [n_out, r]; bwd: A fp32 [r, k_in]
  int64_t n_out;
  int tile0;             // forward: first column tile of this weight
  int z0;                // backward: first split of this weight
  const uint8_t* afrag;  // backward: dy_j in fragment order
  int64_t kblocks;       // backward: its 16-wide blocks per 32-row block
  int64_t kc_chunk;      // backward: contraction rows per split of this weight
};

struct GemmArgs {
  const uint16_t* wd;  // dense bf16 weight [n_out, k_in] (DENSE kernels only)
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
  int nseg;             // weights in the launch (1 unless a grouped forward)
  GemmSeg seg[GEMM_MAX_SEG];
  uint8_t* out_packed;  // SwiGLU epilogue: its output again in fragment order (nullable)
  int xcd_pairs;        // backward: deal the tiles of a (row tile, split) pair to shared XCDs
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
// path serves at a quarter of its rate, so the activation arrives rewritten
// in fragment order (pack.hip): 1 KB per (32-row block, 16-wide contraction
// block), lane after lane, zero-padded to whole 256-row tiles and 64-wide
// steps. Every fragment load of the GEMM is then one contiguous 1 KB read.


struct AFrags {
  u32x4 f[2][4];  // [row tile i][sub-step kk]
};

struct ALanes {
  uint32_t off[2];  // byte offsets of the lane's chunk in its two 32-row blocks at contraction 0
};

__device__ __forceinline__ ALanes a_lanes(const GemmArgs& g, int64_t m0, int wave, int lane) {
  ALanes L;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t blk = (m0 + wave * WAVE_ROWS + i * 32) / 32;
    L.off[i] = (uint32_t)(blk * g.kblocks * FRAG_BYTES + lane * 16);
  }
  return L;
}

__device__ __forceinline__ void load_a(const GemmArgs& g, const ALanes& L, int64_t k0,
                                       AFrags& r) {
  const uint8_t* base = g.afrag + (k0 / 16) * FRAG_BYTES;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      r.f[i][kk] = *reinterpret_cast<const u32x4*>(base + L.off[i] + kk * FRAG_BYTES);
}

// ---- weight tile (B), producer side ---------------------------------------
// pt = producer thread index 0..255.
template <bool BWD>
struct WLanes;
template <bool BWD>
struct BRegs;

// Forward: producer thread pt owns weight row n0 + pt/2 and contraction half
// pt%2 (32 codes, four packed words).
template <>
struct WLanes<false> {
  uint32_t woff;  // byte offset of the thread's 16 packed bytes at contraction 0
  uint32_t blk0;  // 64-block index at contraction 0
  bool valid;     // row < n_out
};
template <>
struct BRegs<false> {
  u32x4 w;
  uint32_t q;
  float nest;
};

__device__ __forceinline__ WLanes<false> w_lanes(const GemmArgs& g, int64_t n0, int pt,
                                                 WLanes<false>*) {
  WLanes<false> L;
  int64_t n = n0 + (pt >> 1);
  L.valid = n < g.n_out;
  n = L.valid ? n : g.n_out - 1;
  L.woff = (uint32_t)(n * (g.k_in / 2) + (pt & 1) * 16);
  L.blk0 = (uint32_t)(n * (g.k_in / 64));
  return L;
}

__device__ __forceinline__ void load_b(const GemmArgs& g, const WLanes<false>& L, Step s, int,
                                       BRegs<false>& rb) {
  rb.w = *reinterpret_cast<const u32x4*>(g.packed + s.k0 / 2 + L.woff);
  const uint32_t blk = L.blk0 + (uint32_t)(s.k0 / 64);
  rb.q = g.q8[blk];
  rb.nest = g.nested[blk >> 8];
}

// Backward patch of producer thread pt: output-column group m (columns
// 8m .. 8m+7 of the tile) and contraction group kg (rows 4kg .. 4kg+3 of the
// step). Lane bit 0 is kg's bit 0, lane bits 1-3 are m's bits 1-3, lane bit 4
// is m's bit 0, lane bit 5 is kg's bit 1 and the wave gives kg's bits 2-3, so
// every 16 consecutive lanes hold 8 column groups of distinct m/2, each at
// both halves of a 16-byte LDS chunk: with the XOR by col/16 below, the
// 8-byte stores of any 16 (or 32) consecutive lanes hit distinct banks. For a
// fixed row the lanes still cover 16 consecutive column groups (64
// contiguous bytes of packed codes).
__device__ __forceinline__ int bwd_m(int pt) { return (((pt >> 1) & 7) << 1) | ((pt >> 4) & 1); }
__device__ __forceinline__ int bwd_kg(int pt) { return (pt & 1) | (((pt >> 5) & 1) << 1) | ((pt >> 6) << 2); }

// Backward: producer thread pt owns weight rows k0 + 4*bwd_kg(pt) + i (i < 4)
// and output columns n0 + 8*bwd_m(pt) + j (j < 8): four packed words. The 128
// block scales of a step (64 rows x 2 column blocks of 64) are loaded and
// decoded once, by producer threads 0..127 (row pt/2, column block pt%2),
// and shared through LDS; a scale is 0 for a row past the contraction or a
// column block past k_in, which zeroes the decoded weights there.
template <>
struct WLanes<true> {
  uint32_t woff[4];  // byte offsets of the packed words at contraction 0
  uint32_t col;      // first (clamped) column
  bool cvalid;       // columns < k_in
  bool sload;        // this thread loads a block scale
  bool scol;         // its column block lies inside k_in
  uint32_t sblk;     // its column block index (clamped)
};
template <>
struct BRegs<true> {
  uint32_t w[4];
  uint32_t q;    // (scale loaders) raw 8-bit scale code
  float nest;    // (scale loaders) nested scale
  bool sok;      // (scale loaders) row and column block inside the weight
};

__device__ __forceinline__ WLanes<true> w_lanes(const GemmArgs& g, int64_t n0, int pt,
                                                WLanes<true>*) {
  WLanes<true> L;
  int64_t col = n0 + 8 * bwd_m(pt);
  L.cvalid = col < g.k_in;
  col = L.cvalid ? col : g.k_in - 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = 4 * bwd_kg(pt) + i;  // relative to the step's start
    L.woff[i] = (uint32_t)((row * g.k_in + col) / 2);
  }
  L.col = (uint32_t)col;
  L.sload = pt < 2 * 64;
  const int64_t bcol = n0 + 64 * (pt & 1);
  L.scol = bcol < g.k_in;
  L.sblk = (uint32_t)((L.scol ? bcol : 0) / 64);
  return L;
}

__device__ __forceinline__ void load_b(const GemmArgs& g, const WLanes<true>& L, Step s, int pt,
                                       BRegs<true>& rb) {
  if (s.k0 + BK <= g.Kc) {  // uniform: every row of the step exists
    const uint8_t* base = g.packed + s.k0 * (g.k_in / 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb.w[i] = *reinterpret_cast<const uint32_t*>(base + L.woff[i]);
  } else {  // the last step of a contraction that is not a multiple of 64
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = s.k0 + 4 * bwd_kg(pt) + i;
      const int64_t e = (row < g.Kc ? row : g.Kc - 1) * g.k_in + L.col;  // code index
      rb.w[i] = *reinterpret_cast<const uint32_t*>(g.packed + e / 2);
    }
  }
  if (L.sload) {  // uniform per wave
    const int64_t row = s.k0 + (pt >> 1);
    rb.sok = L.scol && row < g.Kc;
    const uint32_t blk = (uint32_t)((row < g.Kc ? row : g.Kc - 1) * (g.k_in / 64)) + L.sblk;
    rb.q = g.q8[blk];
    rb.nest = g.nested[blk >> 8];
  }
}

// ---- decoding -------------------------------------------------------------
// Pair table: entry b = (C4[b >> 4], C4[b & 15]), both levels of a packed byte,
// the even element (high nibble) first. Copy c of entry b sits at float2 index
// 32*b + c, i.e. dwords 64*b + 2c and 64*b + 2c + 1: the copy fixes the LDS
// bank pair whatever b is. The byte offset of copy c of entry b, 256 b + 8 c,
// is one byte permute of the code word (byte 1 the code byte, byte 0 the
// copy's offset 8 c < 256, bytes 2 and 3 zero).
struct PairTab {
  const uint8_t* base;  // the table in LDS
  uint32_t copy8;       // 8 * the lane's copy
};
__device__ __forceinline__ float2 pair_of(const PairTab& pt, uint32_t word, int byte) {
  const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)byte) << 8);
  return *reinterpret_cast<const float2*>(pt.base + __builtin_amdgcn_perm(word, pt.copy8, sel));
}

// Fill the pair table and the nested-code table in LDS (threads t < 256).
// 16-byte slot f = 256 i + t holds copies 2(t%16) and 2(t%16)+1 of entry
// e = f/16 = 16 i + t/16, i.e. (C4[i], C4[t/16]): consecutive lanes store
// consecutive 16 bytes, so the stores meet no bank conflicts.
__device__ __forceinline__ void fill_tables(float2* s_pair, float* s_c8, const Tables& tab, int t) {
  static_assert(PAIR_COPIES == 32, "16-byte slots of 16 per entry");
  const float lo = tab.c4[t >> 4];
  float4* const p4 = reinterpret_cast<float4*>(s_pair);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float hi = tab.c4[i];
    p4[i * 256 + t] = make_float4(hi, lo, hi, lo);
  }
  s_c8[t] = tab.c8[t];
}

// The LDS reads of a stage's decode (scale-code lookups and pair table) are
// issued one step before the arithmetic that consumes them, so the producer
// never waits on LDS latency inside a step.
template <int NR>
struct Prep {
  float2 v[16];  // forward: [word * 4 + byte]; backward: [byte * 4 + row]
  float c8v[NR];
};

__device__ __forceinline__ void prep_reads(const BRegs<false>& rb, const PairTab& ptab,
                                           const float* c8, Prep<1>& pp) {
  pp.c8v[0] = c8[rb.q];
#pragma unroll
  for (int jw = 0; jw < 4; ++jw)
#pragma unroll
    for (int p = 0; p < 4; ++p) pp.v[jw * 4 + p] = pair_of(ptab, rb.w[jw], p);
}

// Forward stage: the producer thread's 32 codes -> 32 bf16 of its weight row.
__device__ __forceinline__ void finish_stage(uint16_t* Bs, const BRegs<false>& rb, const Prep<1>& pp,
                                             bool valid, float off, int pt) {
  const float a = valid ? decode_scale(pp.c8v[0], rb.nest, off) : 0.0f;
#pragma unroll
  for (int jw = 0; jw < 4; ++jw) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float2 c = pp.v[jw * 4 + p];
      o[p] = pack_bf16x2(__fmul_rn(c.x, a), __fmul_rn(c.y, a));
    }
    *reinterpret_cast<u32x4*>(Bs + (pt >> 1) * LDS_STRIDE + (pt & 1) * 32 + jw * 8) = o;
  }
}

// Backward LDS layout: stage[col][k] with the 16-byte chunk k/8 of column col
// stored at chunk (k/8) ^ ((col/16) % 8). A 144-byte row puts column col's
// chunk c on 16-byte bank group (9 col + c) mod 16 of the 64 banks, so the
// fragment reads (16 consecutive columns, one chunk: the XOR term constant)
// cover all 16 groups; and the decode's 8-byte stores of a half-wave (columns
// 8m + c for m = 0..15, two halves of one chunk) see m/2 through the XOR, so
// the even m and the odd m each take 8 different chunks: 32 different 8-byte
// slots. (The XOR by col/8 used before mapped m and m + 8 to one slot.)
__device__ __forceinline__ int bwd_swizzle_off(int col, int k) {
  return ((((k >> 3) ^ (col >> 4)) & 7) << 3) | (k & 7);
}

// Also decodes and publishes the thread's block scale (scale loaders), for
// the stage's decode after the next workgroup barrier; sc is the stage's
// slot of the scale ring.
__device__ __forceinline__ void prep_reads(const BRegs<true>& rb, const PairTab& ptab,
                                           const float* c8, Prep<1>& pp, float* sc, float off,
                                           int pt) {
  float cq = 0.0f;
  if (pt < 2 * 64) cq = c8[rb.q];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) pp.v[q * 4 + i] = pair_of(ptab, rb.w[i], q);
  if (pt < 2 * 64) sc[(pt & 1) * 64 + (pt >> 1)] = rb.sok ? decode_scale(cq, rb.nest, off) : 0.0f;
}

// Backward stage: byte q of each of the thread's four row words gives output
// columns 2q and 2q+1 of its 4x8 patch, each written as 4 consecutive
// contraction values -- the transpose into the matrix-core layout happens
// here, in the bf16 pairing.
__device__ __forceinline__ void finish_stage(uint16_t* Bs, const BRegs<true>&, const Prep<1>& pp,
                                             const float* sc, int pt) {
  const int r0 = 4 * bwd_kg(pt);
  const float4 a4 = *reinterpret_cast<const float4*>(sc + (bwd_m(pt) >> 3) * 64 + r0);
  const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v0[4], v1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v0[i] = __fmul_rn(pp.v[q * 4 + i].x, a[i]);
      v1[i] = __fmul_rn(pp.v[q * 4 + i].y, a[i]);
    }
    const int cb = 8 * bwd_m(pt) + 2 * q;
    uint2 p0, p1;
    p0.x = pack_bf16x2(v0[0], v0[1]);
    p0.y = pack_bf16x2(v0[2], v0[3]);
    p1.x = pack_bf16x2(v1[0], v1[1]);
    p1.y = pack_bf16x2(v1[2], v1[3]);
    *reinterpret_cast<uint2*>(Bs + cb * LDS_STRIDE + bwd_swizzle_off(cb, r0)) = p0;
    *reinterpret_cast<uint2*>(Bs + (cb + 1) * LDS_STRIDE + bwd_swizzle_off(cb + 1, r0)) = p1;
  }
}

// ---- dense bf16 weight tile (the resident lm_head), producer side ---------
// Same thread-to-tile map and LDS layouts as the NF4 producer, without the
// decode: the forward copies 64 B of a weight row per thread, the backward
// loads a 4x8 patch and pairs its values along the contraction on the way
// into LDS. Rows and columns outside the weight load as zeros.
template <bool BWD>
struct DLanes;
template <>
struct DLanes<false> {
  const uint16_t* row;  // the thread's weight row at contraction 0, plus its half
  bool valid;
};
template <>
struct DLanes<true> {
  int64_t col;  // first (clamped) column
  bool cvalid;
};
struct DRegs {
  u32x4 w[4];
};

__device__ __forceinline__ DLanes<false> d_lanes(const GemmArgs& g, int64_t n0, int pt,
                                                 DLanes<false>*) {
  DLanes<false> L;
  int64_t n = n0 + (pt >> 1);
  L.valid = n < g.n_out;
  n = L.valid ? n : g.n_out - 1;
  L.row = g.wd + n * g.k_in + (pt & 1) * 32;
  return L;
}

__device__ __forceinline__ void load_d(const GemmArgs&, const DLanes<false>& L, Step s, int,
                                       DRegs& rb) {
#pragma unroll
  for (int jw = 0; jw < 4; ++jw) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(L.row + s.k0 + jw * 8);
    rb.w[jw] = L.valid ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void finish_dense(uint16_t* Bs, const DRegs& rb, int pt,
                                             DLanes<false>*) {
#pragma unroll
  for (int jw = 0; jw < 4; ++jw)
    *reinterpret_cast<u32x4*>(Bs + (pt >> 1) * LDS_STRIDE + (pt & 1) * 32 + jw * 8) = rb.w[jw];
}

__device__ __forceinline__ DLanes<true> d_lanes(const GemmArgs& g, int64_t n0, int pt,
                                                DLanes<true>*) {
  DLanes<true> L;
  const int64_t col = n0 + 8 * bwd_m(pt);
  L.cvalid = col < g.k_in;
  L.col = L.cvalid ? col : g.k_in - 8;
  return L;
}

__device__ __forceinline__ void load_d(const GemmArgs& g, const DLanes<true>& L, Step s, int pt,
                                       DRegs& rb) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = s.k0 + 4 * bwd_kg(pt) + i;
    const bool ok = L.cvalid && row < g.Kc;
    const u32x4 v = *reinterpret_cast<const u32x4*>(g.wd + (ok ? row : 0) * g.k_in + L.col);
    rb.w[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

// Word q of row i holds columns 2q (low half) and 2q+1 (high half); column c
// of the patch goes to LDS as its four contraction values r0..r0+3.
__device__ __forceinline__ void finish_dense(uint16_t* Bs, const DRegs& rb, int pt, DLanes<true>*) {
  const int r0 = 4 * bwd_kg(pt);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w0 = rb.w[0][q], w1 = rb.w[1][q], w2 = rb.w[2][q], w3 = rb.w[3][q];
    const int cb = 8 * bwd_m(pt) + 2 * q;
    uint2 p0, p1;
    p0.x = (w0 & 0xFFFFu) | (w1 << 16);
    p0.y = (w2 & 0xFFFFu) | (w3 << 16);
    p1.x = (w0 >> 16) | (w1 & 0xFFFF0000u);
    p1.y = (w2 >> 16) | (w3 & 0xFFFF0000u);
    *reinterpret_cast<uint2*>(Bs + cb * LDS_STRIDE + bwd_swizzle_off(cb, r0)) = p0;
    *reinterpret_cast<uint2*>(Bs + (cb + 1) * LDS_STRIDE + bwd_swizzle_off(cb + 1, r0)) = p1;
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

// SPLIT selects the output path (fp32 partials vs bf16 result) at compile time,
// so the two variants also carry distinct kernel names in profiles. DENSE
// swaps the NF4 producer for the plain bf16 one.
template <bool BWD, bool SPLIT, bool DENSE>
__global__ __launch_bounds__(THREADS, 1) void k_gemm(GemmArgs ga, Tables tab) {
  // Tile order. Workgroups are dispatched in flattened-id order and dealt to
  // the 8 XCDs round-robin; each XCD has its own L2. NF4 weights stream at
  // 0.52 B per weight, an eighth of the activation bytes a tile reads, so the
  // launch order is kept: the workgroups running together share one row
  // tile of the activation in L2. A dense bf16 weight is 4x heavier and the
  // lm_head grid spans many waves, so there ids are mapped to put all row
  // tiles of a column tile on one XCD at the same time (ids ct%8 + 8*rt in a
  // block of 8*R ids) and each weight tile leaves HBM once.
  // The NF4 backward reads a different activation block per (row tile,
  // split) pair -- the dy rows of the tile over the split's share of the
  // contraction, e.g. 3.7 MB at the grouped gate+up backward -- and every
  // column tile of the pair reads all of it. Dealt in launch order, each XCD
  // would hold tiles of every pair and fetch all their blocks (8 x 29 MB);
  // instead the ids are mapped so that a pair's column tiles share XCDs: with
  // P pairs dividing or divided by 8, id 8 s + x (x the XCD) is pair
  // x / G + 8 (s / C') and column tile (s % C') G + x % G, G = max(1, 8 / P)
  // XCDs per pair, C' = C / G tiles per XCD (used when G divides C). The
  // host asks for it when the blocks together exceed two L2s: where they fit
  // the launch order is faster (measured: 6% slower q+k+v backward at M =
  // 512 with the mapping, 4-6% faster gate+up backward).
  const int C = (int)gridDim.x, R = (int)gridDim.y;
  const int id = (int)blockIdx.x + C * (int)blockIdx.y;
  const int full = C / 8 * 8;
  int ct, rt, zz = (int)blockIdx.z;
  if (!DENSE && BWD && ga.xcd_pairs) {
    const int P = R * (int)gridDim.z;
    const int G = P >= 8 ? 1 : 8 / P;
    const int flat = id + C * R * (int)blockIdx.z;
    if ((P % 8 == 0 || 8 % P == 0) && C % G == 0) {
      const int x = flat % 8, sl = flat / 8, cg = C / G;
      const int pair = x / G + 8 * (sl / cg);
      ct = (sl % cg) * G + x % G;
      rt = pair % R;
      zz = pair / R;
    } else {
      ct = (int)blockIdx.x;
      rt = (int)blockIdx.y;
    }
  } else if (!DENSE) {
    ct = (int)blockIdx.x;
    rt = (int)blockIdx.y;
  } else if (id < full * R) {
    const int w = id % (8 * R);
    ct = id / (8 * R) * 8 + w % 8;
    rt = w / 8;
  } else {
    const int j = id - full * R;
    ct = full + j / R;
    rt = j % R;
  }
  // the weight this workgroup belongs to (uniform per workgroup): by column
  // tile in the forward, by split in the backward
  int sgi = 0;
#pragma unroll
  for (int q = 1; q < GEMM_MAX_SEG; ++q)
    if (q < ga.nseg && (BWD ? zz >= ga.seg[q].z0 : ct >= ga.seg[q].tile0)) sgi = q;
  GemmArgs g = ga;
  g.packed = ga.seg[sgi].packed;
  g.q8 = ga.seg[sgi].q8;
  g.nested = ga.seg[sgi].nested;
  g.offset = ga.seg[sgi].offset;
  g.out = ga.seg[sgi].out;
  g.part = ga.seg[sgi].part;
  g.lora_l = ga.seg[sgi].lora_l;
  g.lora_r = ga.seg[sgi].lora_r;
  g.n_out = ga.seg[sgi].n_out;
  if (!BWD) g.Nc = g.n_out;
  if (BWD) {  // the weight's own dy, contraction length and split chunk
    g.afrag = ga.seg[sgi].afrag;
    g.kblocks = ga.seg[sgi].kblocks;
    g.kc_chunk = ga.seg[sgi].kc_chunk;
    g.Kc = g.n_out;
  }
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_BYTES];
  uint16_t* const Bs0 = reinterpret_cast<uint16_t*>(smem);
  float2* const s_pair_all = reinterpret_cast<float2*>(smem + NSTAGE * STAGE_ELEMS * 2);
  float* const s_c8 = reinterpret_cast<float*>(smem + NSTAGE * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8);
  float* const s_scale =
      reinterpret_cast<float*>(smem + NSTAGE * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8 + 256 * 4);

  const int t = threadIdx.x;
  if (!DENSE && t < 256) fill_tables(s_pair_all, s_c8, tab, t);

  const int64_t n0 = (int64_t)(ct - ga.seg[sgi].tile0) * BN;
  const int64_t m0 = (int64_t)rt * BM;
  const int zpart = zz;                                 // the partial this workgroup writes
  const int split = zpart - (BWD ? ga.seg[sgi].z0 : 0);  // its split of the weight's contraction
  const int64_t kb = split * g.kc_chunk;
  const int64_t ke = (kb + g.kc_chunk < g.Kc) ? kb + g.kc_chunk : g.Kc;
  const int nk = (int)((ke - kb + BK - 1) / BK);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: role branches are scalar
  const int lane = t & 63;
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;

  // step kt (clamped to the last one for prefetches past the end)
  auto step_of = [&](int kt) {
    const int k = kt < nk ? kt : nk - 1;
    Step s;
    s.k0 = kb + (int64_t)k * BK;
    return s;
  };
  auto stage = [&](int st) { return Bs0 + st * STAGE_ELEMS; };

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Both roles pass the same barriers: 2 in the prologue, 1 per step.
  if (wave < CONSUMERS) {
    // ---- consumer: activation stage k in register slot k%2; sub-step kk of
    // stage k+2 is fetched into the slot as soon as the MFMAs of sub-step kk
    // of stage k are issued
    const ALanes al = a_lanes(g, m0, wave, lane);
    AFrags ar0, ar1;
    load_a(g, al, step_of(0).k0, ar0);
    load_a(g, al, step_of(1).k0, ar1);
    __syncthreads();  // tables in LDS
    if constexpr (BWD && !DENSE) {
      __syncthreads();  // block scales of stage 0 published
      __syncthreads();  // block scales of stage 1 published
    }
    __syncthreads();  // weight stages 0 and 1 decoded
    bf16x8_t fb0[4];  // fragments of sub-step 0 of the stage about to be multiplied
#pragma unroll
    for (int j = 0; j < 4; ++j) fb0[j] = b_frag<BWD>(stage(0), lane, j, 0);

    auto mfma_kk = [&](const AFrags& A, int kk, const bf16x8_t* fb) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              fb[j], __builtin_bit_cast(bf16x8_t, A.f[i][kk]), acc[i][j], 0, 0, 0);
    };
    auto refill = [&](AFrags& A, int kk, int64_t k0) {
      const uint8_t* base = g.afrag + (k0 / 16) * FRAG_BYTES + kk * FRAG_BYTES;
#pragma unroll
      for (int i = 0; i < 2; ++i) A.f[i][kk] = *reinterpret_cast<const u32x4*>(base + al.off[i]);
    };
    // One step: multiply LDS stage `bs` (sub-step 0 fragments already in fb0)
    // with activation slot A, reading each sub-step's fragments one sub-step
    // ahead and refilling A for the step two ahead; end with the sub-step 0
    // fragments of the next stage `bnext`. The scheduling barriers keep this
    // order: left alone, the compiler hoists the MFMAs of a sub-step above
    // the workgroup barrier and then issues the next fragment reads right
    // before their first use, exposing the LDS latency.
    auto multiply = [&](const uint16_t* bs, const uint16_t* bnext, AFrags& A, int64_t knext) {
      bf16x8_t fb1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb1[j] = b_frag<BWD>(bs, lane, j, 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_kk(A, 0, fb0);
      refill(A, 0, knext);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb0[j] = b_frag<BWD>(bs, lane, j, 2);
      __builtin_amdgcn_sched_barrier(0);
      mfma_kk(A, 1, fb1);
      refill(A, 1, knext);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb1[j] = b_frag<BWD>(bs, lane, j, 3);
      __builtin_amdgcn_sched_barrier(0);
      mfma_kk(A, 2, fb0);
      refill(A, 2, knext);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb0[j] = b_frag<BWD>(bnext, lane, j, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_kk(A, 3, fb1);
      refill(A, 3, knext);
    };
#define NF4S_CONSUMER_STEP(KT, SM, ACUR)                                              \
  do {                                                                                \
    multiply(stage(SM), stage(((SM) + 1) % NSTAGE), ACUR, step_of((KT) + 2).k0);      \
    __builtin_amdgcn_sched_barrier(0);                                                \
    __syncthreads();                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                \
  } while (0)
    const int nk4 = nk - nk % 4;
    for (int kt = 0; kt < nk4; kt += 4) {
      NF4S_CONSUMER_STEP(kt, 0, ar0);
      NF4S_CONSUMER_STEP(kt + 1, 1, ar1);
      NF4S_CONSUMER_STEP(kt + 2, 2, ar0);
      NF4S_CONSUMER_STEP(kt + 3, 3, ar1);
    }
    if (nk4 < nk) NF4S_CONSUMER_STEP(nk4, 0, ar0);
    if (nk4 + 1 < nk) NF4S_CONSUMER_STEP(nk4 + 1, 1, ar1);
    if (nk4 + 2 < nk) NF4S_CONSUMER_STEP(nk4 + 2, 2, ar0);
#undef NF4S_CONSUMER_STEP

    // LoRA term, contracted on the matrix cores in chunks of 16 over the rank:
    // forward  + u[m, :] . (s * B[n, :]),  backward + du[m, :] . A[:, n].
    if (g.lora_l != nullptr && split == 0) {
      for (int r0 = 0; r0 < g.r; r0 += 16) {
        bf16x8_t fa[2], fb[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int64_t row = m0 + wave * WAVE_ROWS + i * 32 + lrow;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rr = r0 + lk + e;
            v[e] = (row < g.M && rr < g.r) ? g.lora_l[row * g.r + rr] : 0.0f;
          }
          fa[i] = f32x8_to_bf16(v);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = n0 + j * 32 + lrow;
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
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
      }
    }
  } else if constexpr (DENSE) {
    // ---- dense producer: the same ring without the decode; stage k is
    // fetched in step k-5 and stored into LDS stage k%4 in step k-2
    const int pt = t - 64 * CONSUMERS;
    const DLanes<BWD> dl = d_lanes(g, n0, pt, static_cast<DLanes<BWD>*>(nullptr));
    DRegs wb0, wb1, wb2, wb3;
    load_d(g, dl, step_of(0), pt, wb0);
    load_d(g, dl, step_of(1), pt, wb1);
    load_d(g, dl, step_of(2), pt, wb2);
    load_d(g, dl, step_of(3), pt, wb3);
    __syncthreads();  // tables in LDS (unused here; the barrier count is shared)
    finish_dense(stage(0), wb0, pt, static_cast<DLanes<BWD>*>(nullptr));
    load_d(g, dl, step_of(4), pt, wb0);
    finish_dense(stage(1), wb1, pt, static_cast<DLanes<BWD>*>(nullptr));
    __syncthreads();
#define NF4S_DENSE_STEP(KT, SM, WFIN, WLD)                                          \
  do {                                                                              \
    load_d(g, dl, step_of((KT) + 5), pt, WLD);                                      \
    finish_dense(stage(((SM) + 2) % NSTAGE), WFIN, pt, static_cast<DLanes<BWD>*>(nullptr)); \
    __syncthreads();                                                                \
  } while (0)
    const int nk4 = nk - nk % 4;
    for (int kt = 0; kt < nk4; kt += 4) {
      NF4S_DENSE_STEP(kt, 0, wb2, wb1);
      NF4S_DENSE_STEP(kt + 1, 1, wb3, wb2);
      NF4S_DENSE_STEP(kt + 2, 2, wb0, wb3);
      NF4S_DENSE_STEP(kt + 3, 3, wb1, wb0);
    }
    if (nk4 < nk) NF4S_DENSE_STEP(nk4, 0, wb2, wb1);
    if (nk4 + 1 < nk) NF4S_DENSE_STEP(nk4 + 1, 1, wb3, wb2);
    if (nk4 + 2 < nk) NF4S_DENSE_STEP(nk4 + 2, 2, wb0, wb3);
#undef NF4S_DENSE_STEP
  } else {
    // ---- producer: weight stage k lives in register slot k%4, is fetched in
    // step k-5, has its table lookups issued in step k-3 and is decoded into
    // LDS stage k%4 in step k-2
    const int pt = t - 64 * CONSUMERS;
    const WLanes<BWD> wl = w_lanes(g, n0, pt, static_cast<WLanes<BWD>*>(nullptr));
    bool valid = true;
    if constexpr (!BWD) valid = wl.valid;
    const float off = g.offset[0];
    const PairTab s_pair{reinterpret_cast<const uint8_t*>(s_pair_all),
                         (uint32_t)(t & (PAIR_COPIES - 1)) * 8u};
    BRegs<BWD> wb0, wb1, wb2, wb3;
    Prep<1> pp;
    // table lookups of stage st (backward: also publish its block scales)
    auto prep = [&](const BRegs<BWD>& rb, int st) {
      if constexpr (BWD) prep_reads(rb, s_pair, s_c8, pp, s_scale + st * SCALE_FLOATS, off, pt);
      else prep_reads(rb, s_pair, s_c8, pp);
    };
    auto fin = [&](const BRegs<BWD>& rb, int st) {
      if constexpr (BWD) finish_stage(stage(st), rb, pp, s_scale + st * SCALE_FLOATS, pt);
      else finish_stage(stage(st), rb, pp, valid, off, pt);
    };
    load_b(g, wl, step_of(0), pt, wb0);
    load_b(g, wl, step_of(1), pt, wb1);
    load_b(g, wl, step_of(2), pt, wb2);
    load_b(g, wl, step_of(3), pt, wb3);
    __syncthreads();  // tables in LDS
    prep(wb0, 0);
    if constexpr (BWD) __syncthreads();  // block scales of stage 0 published
    fin(wb0, 0);
    load_b(g, wl, step_of(4), pt, wb0);
    prep(wb1, 1);
    if constexpr (BWD) __syncthreads();  // block scales of stage 1 published
    fin(wb1, 1);
    prep(wb2, 2);
    __syncthreads();
// (the scheduling barriers keep the next stage's decode arithmetic below the
// workgroup barrier, so the table lookups issued here overlap the wait)
#define NF4S_PRODUCER_STEP(KT, SM, WFIN, WPREP, WLD)                                 \
  do {                                                                               \
    load_b(g, wl, step_of((KT) + 5), pt, WLD);                                       \
    fin(WFIN, ((SM) + 2) % NSTAGE);                                                  \
    prep(WPREP, ((SM) + 3) % NSTAGE);                                                \
    __builtin_amdgcn_sched_barrier(0);                                               \
    __syncthreads();                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                               \
  } while (0)
    const int nk4 = nk - nk % 4;
    for (int kt = 0; kt < nk4; kt += 4) {
      NF4S_PRODUCER_STEP(kt, 0, wb2, wb3, wb1);
      NF4S_PRODUCER_STEP(kt + 1, 1, wb3, wb0, wb2);
      NF4S_PRODUCER_STEP(kt + 2, 2, wb0, wb1, wb3);
      NF4S_PRODUCER_STEP(kt + 3, 3, wb1, wb2, wb0);
    }
    if (nk4 < nk) NF4S_PRODUCER_STEP(nk4, 0, wb2, wb3, wb1);
    if (nk4 + 1 < nk) NF4S_PRODUCER_STEP(nk4 + 1, 1, wb3, wb0, wb2);
    if (nk4 + 2 < nk) NF4S_PRODUCER_STEP(nk4 + 2, 2, wb0, wb1, wb3);
#undef NF4S_PRODUCER_STEP
  }

  // The products are formed transposed (weight fragment first), so register
  // r of lane l holds output row l%32 and column 8*(r/4) + 4*(l/32) + r%4 of
  // its 32x32 tile: registers 4q..4q+3 are four adjacent columns, one LDS
  // store. The tile goes out through LDS so that every global store writes
  // 16 contiguous bytes (bf16: the whole 256x128 tile at once; fp32
  // partials: 128 rows at a time). The weight ring is free: the last step
  // ended with a barrier.
  if constexpr (!SPLIT) {
    constexpr int OS = BN + 8;  // bf16 per LDS row
    uint16_t* ot = reinterpret_cast<uint16_t*>(smem);
    if (wave < CONSUMERS) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wave * WAVE_ROWS + i * 32 + lrow;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 v;
            v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<uint2*>(ot + row * OS + j * 32 + 8 * q + 4 * (lane >> 5)) = v;
          }
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
    for (int ph = 0; ph < 2; ++ph) {  // rows [128 ph, 128 ph + 128): consumers 2ph, 2ph+1
      if (wave < CONSUMERS && (wave >> 1) == ph) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = (wave & 1) * WAVE_ROWS + i * 32 + lrow;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]);
              *reinterpret_cast<float4*>(ot + row * OS + j * 32 + 8 * q + 4 * (lane >> 5)) = v;
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
          *reinterpret_cast<u32x4*>(g.part + ((int64_t)zpart * g.M + grow) * g.Nc + gcol) =
              *reinterpret_cast<const u32x4*>(ot + row * OS + 4 * c4);
      }
      __syncthreads();
    }
  }
}

// ---- forward kernel: one wave per SIMD ------------------------------------
// The forward orientation (x . W'^T, NF4 weight) runs on a second design that
// gives each wave the whole matrix-core register budget: 256 threads = 4
// waves, one per SIMD, each owning 128 output rows x 128 columns (4x4 MFMA
// tiles, 256 fp32 accumulators per lane in the accumulation registers); the
// workgroup tile is 512 rows x 128 columns, so every decoded weight tile
// feeds twice the rows of k_gemm and each wave reads half the LDS bytes per
// MFMA. Every wave also decodes its quarter of the weight tile; that work is
// placed between the MFMAs in a fixed order (one scheduling barrier per
// MFMA) so it runs while the matrix pipe is busy:
//  * sub-step g of step s: 16 MFMAs; after the first four, the B fragments
//    of the next sub-step (or of the next stage's sub-step 0) are read; after
//    every fourth, one activation fragment is refilled for step s+2;
//  * sub-step 0 issues the pair-table lookups of stage s+2, sub-step 1 does
//    its arithmetic, sub-step 2 stores it, sub-step 3 fetches the packed
//    codes of step s+4;
//  * three LDS stages: stage s+1 is complete at the barrier that ends step
//    s-1, so its first fragments are read before the barrier of step s;
//  * the packed codes of even and odd steps live in two register sets that
//    are never copied (a copy of a value still in flight would wait for every
//    older load);
//  * the loop is unrolled by six steps (two register sets x three stages), so
//    the stage addresses are constants.
// The decode and the contraction order per output element are those of
// k_gemm: results are bit-identical for the same split of the contraction.
constexpr int FBM = 512;
constexpr int FTHREADS = 256;
constexpr int FNST = 3;
constexpr int F_SMEM_BYTES = FNST * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8 + 256 * 4;

struct FSlot {
  u32x4 w;     // 32 packed codes of the thread's weight row half
  uint32_t q;  // 8-bit scale code of the row's 64-block
  float nest;  // nested scale of that block
};

// SWIGLU: the launch holds the gate (weight 0) and up (weight 1) projections of
// one MLP; column tile ct covers gate rows and up rows 64 ct .. 64 ct + 63
// (waves 0-1 decode the gate rows into tile columns 0-63, waves 2-3 the up
// rows into columns 64-127), and the epilogue writes silu(g) * u of the two
// bf16-rounded results instead of g and u.
template <bool SWIGLU>
__global__ __launch_bounds__(FTHREADS, 1) void k_gemm_fwd(GemmArgs ga, Tables tab) {
  const int ct = (int)blockIdx.x;
  int sgi = 0;
  if constexpr (SWIGLU) {
    sgi = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 7);  // the weight this wave decodes
  } else {
#pragma unroll
    for (int q = 1; q < GEMM_MAX_SEG; ++q)
      if (q < ga.nseg && ct >= ga.seg[q].tile0) sgi = q;
  }
  const uint8_t* const packed = ga.seg[sgi].packed;
  const uint8_t* const q8 = ga.seg[sgi].q8;
  const float* const nested = ga.seg[sgi].nested;
  const float off = ga.seg[sgi].offset[0];
  const int64_t n_out = ga.seg[sgi].n_out;
  const int64_t n0 = SWIGLU ? (int64_t)ct * (BN / 2) : (int64_t)(ct - ga.seg[sgi].tile0) * BN;
  const int64_t m0 = (int64_t)blockIdx.y * FBM;
  const int split = blockIdx.z;
  const int64_t M = ga.M, k_in = ga.k_in;
  const int64_t kb = split * ga.kc_chunk;
  const int64_t ke = (kb + ga.kc_chunk < ga.Kc) ? kb + ga.kc_chunk : ga.Kc;
  const int nk = (int)((ke - kb + BK - 1) / BK);

  __shared__ __attribute__((aligned(16))) uint8_t smem[F_SMEM_BYTES];
  uint16_t* const Bs0 = reinterpret_cast<uint16_t*>(smem);
  float2* const s_pair_all = reinterpret_cast<float2*>(smem + FNST * STAGE_ELEMS * 2);
  float* const s_c8 = reinterpret_cast<float*>(smem + FNST * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8);
  const int t = threadIdx.x;
  fill_tables(s_pair_all, s_c8, tab, t);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  auto stage = [&](int st) { return Bs0 + st * STAGE_ELEMS; };

  // activation fragments: the rows of a wave past the packed activation (a
  // last tile of fewer than 512 rows) re-read its last 32-row block; those
  // rows are never stored
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc((void*)ga.afrag, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const int64_t nblk = (M + PACK_ROWS - 1) / PACK_ROWS * (PACK_ROWS / 32);
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t b = (m0 + wave * 128 + i * 32) / 32;
    b = b < nblk ? b : nblk - 1;
    aoff[i] = (uint32_t)(b * ga.kblocks * FRAG_BYTES + lane * 16);
  }
  // contraction step k (clamped to the last one) -> activation byte offset of its sub-step 0
  auto a_soff = [&](int k) {
    const int kc = k < nk ? k : nk - 1;
    return (int)(((kb + (int64_t)kc * BK) / 16) * FRAG_BYTES);
  };

  // weights: thread t owns row n0 + t/2 (SWIGLU: n0 + (t/2) % 64 of its
  // wave's weight; clamped, scale forced to 0 past n_out) and the contraction
  // half t%2 of every step
  int64_t wrow = n0 + (SWIGLU ? ((t >> 1) & (BN / 2 - 1)) : (t >> 1));
  const bool valid = wrow < n_out;
  wrow = valid ? wrow : n_out - 1;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)packed, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const __amdgpu_buffer_rsrc_t qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)q8, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const __amdgpu_buffer_rsrc_t nr =
      __builtin_amdgcn_make_buffer_rsrc((void*)nested, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const uint32_t woff = (uint32_t)(wrow * (k_in / 2) + (t & 1) * 16);
  const uint32_t blk0 = (uint32_t)(wrow * (k_in / 64));
  // (all loads of the loop are buffer loads: one return-order class, so the
  // compiler's wait counts stay exact)
  auto load_w = [&](int k, FSlot& sl) {
    const int kc = k < nk ? k : nk - 1;
    const int64_t k0 = kb + (int64_t)kc * BK;
    sl.w = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, (int)(k0 / 2), 0);
    const uint32_t blk = blk0 + (uint32_t)(k0 / 64);
    sl.q = __builtin_amdgcn_raw_buffer_load_b8(qr, blk, 0, 0);
    sl.nest = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(nr, (blk >> 8) * 4, 0, 0));
  };
  const PairTab ptab{reinterpret_cast<const uint8_t*>(s_pair_all), (uint32_t)(t & (PAIR_COPIES - 1)) * 8u};
  float2 pv[16];
  float pc, ascale;
  uint32_t ow[16];
  auto lookup = [&](const FSlot& sl, int u) { pv[u] = pair_of(ptab, sl.w[u >> 2], u & 3); };
  auto unit = [&](int u) { ow[u] = pack_bf16x2(__fmul_rn(pv[u].x, ascale), __fmul_rn(pv[u].y, ascale)); };
  auto store_w = [&](int jw, int st) {
    u32x4 o;
    o[0] = ow[jw * 4];
    o[1] = ow[jw * 4 + 1];
    o[2] = ow[jw * 4 + 2];
    o[3] = ow[jw * 4 + 3];
    *reinterpret_cast<u32x4*>(stage(st) + (t >> 1) * LDS_STRIDE + (t & 1) * 32 + jw * 8) = o;
  };
  auto decode_all = [&](const FSlot& sl, int st) {  // prologue: a whole stage at once
    pc = s_c8[sl.q];
#pragma unroll
    for (int u = 0; u < 16; ++u) lookup(sl, u);
    ascale = valid ? decode_scale(pc, sl.nest, off) : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) unit(u);
#pragma unroll
    for (int jw = 0; jw < 4; ++jw) store_w(jw, st);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // prologue: every load is issued before the first decode, so the
  // activation's latency overlaps the decode of stages 0 and 1. After the
  // codes of steps 0 and 1 come the activation of step 0 and the codes of
  // step 2, then the activation of step 1 and the codes of step 3, in the
  // order a step of the loop issues them (the codes after the second
  // activation refill of sub-step 3), so the wait counts the compiler derives
  // at the loop head are the steady-state ones on both paths into it
  FSlot p0, p1, sa, sb;
  u32x4 A0[4][4], A1[4][4];
  load_w(0, p0);
  load_w(1, p1);
  __builtin_amdgcn_sched_barrier(0);
  auto issue_a = [&](u32x4 (&A)[4][4], int k, FSlot& sl, int kw) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i][g] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], a_soff(k) + g * FRAG_BYTES, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (g == 3 && i == 1) {
          load_w(kw, sl);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  };
  issue_a(A0, 0, sa, 2);
  issue_a(A1, 1, sb, 3);
  __syncthreads();  // tables in LDS
  decode_all(p0, 0);
  decode_all(p1, 1);
  __syncthreads();
  bf16x8_t fb0[4], fb1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fb0[j] = b_frag<false>(stage(0), lane, j, 0);

  // st = s % FNST, a constant where the loop below is unrolled by six
  auto step = [&](int s, int st, u32x4 (&A)[4][4], FSlot& sl) __attribute__((always_inline)) {
    const int s1 = st + 1 < FNST ? st + 1 : st + 1 - FNST;
    const int s2 = st + 2 < FNST ? st + 2 : st + 2 - FNST;
    const int a2 = a_soff(s + 2);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x8_t(&fc)[4] = (g & 1) ? fb1 : fb0;
      bf16x8_t(&fn)[4] = (g & 1) ? fb0 : fb1;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc[j], __builtin_bit_cast(bf16x8_t, A[i][g]),
                                                            acc[i][j], 0, 0, 0);
        if (m < 4) fn[m] = (g < 3) ? b_frag<false>(stage(st), lane, m, g + 1) : b_frag<false>(stage(s1), lane, m, 0);
        if (j == 3) A[i][g] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], a2 + g * FRAG_BYTES, 0);
        if (g == 0) {
          if (m == 4) pc = s_c8[sl.q];
          if (m >= 4) lookup(sl, m - 4);
          if (m >= 12) lookup(sl, m);
        }
        if (g == 1) {
          if (m == 0) ascale = valid ? decode_scale(pc, sl.nest, off) : 0.0f;
          unit(m);
        }
        if (g == 2 && (m & 3) == 1) store_w(m >> 2, s2);
        if (g == 3 && m == 8) load_w(s + 4, sl);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s + 5 < nk; s += 6) {
    step(s, 0, A0, sa);
    step(s + 1, 1, A1, sb);
    step(s + 2, 2, A0, sa);
    step(s + 3, 0, A1, sb);
    step(s + 4, 1, A0, sa);
    step(s + 5, 2, A1, sb);
  }
  for (; s + 1 < nk; s += 2) {
    step(s, s % FNST, A0, sa);
    step(s + 1, (s + 1) % FNST, A1, sb);
  }
  if (s < nk) step(s, s % FNST, A0, sa);

  // LoRA term on the matrix cores, in chunks of 16 over the rank (split 0):
  // + u[m, :] . (s * B[n, :]); SWIGLU: gate's adapter on column tiles 0-1,
  // up's on 2-3
  for (int lw = 0; lw < (SWIGLU ? 2 : 1); ++lw) {
    const int ls = SWIGLU ? lw : sgi;
    if (ga.seg[ls].lora_l == nullptr || split != 0) continue;
    const float* const lu = ga.seg[ls].lora_l;
    const float* const lb = ga.seg[ls].lora_r;
    const int64_t ln_out = ga.seg[ls].n_out;
    const int64_t ln0 = SWIGLU ? (int64_t)ct * (BN / 2) : n0;
    for (int r0 = 0; r0 < ga.r; r0 += 16) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wave * 128 + i * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (row < M && rr < ga.r) ? lu[row * ga.r + rr] : 0.0f;
        }
        fa[i] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // SWIGLU: tile column j*32 + lrow is column (j%2)*32 + lrow of weight j/2
        const int64_t col = ln0 + (SWIGLU ? (j & 1) : j) * 32 + lrow;
        const bool mine = !SWIGLU || (j >> 1) == lw;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (mine && col < ln_out && rr < ga.r) ? ga.scale * lb[col * ga.r + rr] : 0.0f;
        }
        fb[j] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!SWIGLU || (j >> 1) == lw)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  // Output through LDS (the ring is free after the last barrier) so that
  // every global store writes 16 contiguous bytes. The products are formed
  // transposed (weight fragment as the first operand), so accumulator
  // register r of lane l holds output row l%32 and column 8*(r/4) + 4*(l/32)
  // + r%4 of its 32x32 tile: registers 4q..4q+3 are four adjacent columns,
  // one 8-byte LDS store.
  if constexpr (SWIGLU) {
    // tile columns c and 64 + c are gate and up column n0 + c (accumulator
    // tiles j and j + 2): round both to bf16 as the unfused launch stores
    // them, then silu(g) * u as the elementwise kernel computes it; the 512 x
    // 64 result leaves row-major and, when asked, in fragment order
    constexpr int OS = BN / 2 + 8;  // bf16 per LDS row, all 512 rows at once
    uint16_t* const ot = reinterpret_cast<uint16_t*>(smem);
    auto bf = [](float x) { return __uint_as_float(pack_bf16x2(x, 0.0f) << 16); };
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wave * 128 + i * 32 + lrow;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float sv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sv[e] = swiglu_val(bf(acc[i][j][4 * q + e]), bf(acc[i][j + 2][4 * q + e]));
          uint2 v;
          v.x = pack_bf16x2(sv[0], sv[1]);
          v.y = pack_bf16x2(sv[2], sv[3]);
          *reinterpret_cast<uint2*>(ot + row * OS + j * 32 + 8 * q + 4 * (lane >> 5)) = v;
        }
      }
    __syncthreads();
    uint16_t* const out = ga.seg[0].out;
    const int64_t width = ga.seg[0].n_out;
#pragma unroll
    for (int it = 0; it < FBM * (BN / 2) / 8 / FTHREADS; ++it) {
      const int q = it * FTHREADS + t;
      const int row = q / (BN / 16), c8 = q % (BN / 16);
      const int64_t grow = m0 + row, gcol = n0 + 8 * c8;
      if (out && grow < M && gcol < width)
        *reinterpret_cast<u32x4*>(out + grow * width + gcol) = *reinterpret_cast<const u32x4*>(ot + row * OS + 8 * c8);
    }
    if (ga.out_packed) {
      // fragment (32-row block b, 16-wide block s) of the tile: lane l holds
      // row 32 b + l%32, columns 16 s + 8 (l/32) .. + 8
      const int64_t kbw = (width + 63) / 64 * 4;
#pragma unroll
      for (int it = 0; it < FBM * (BN / 2) / 8 / FTHREADS; ++it) {
        const int q = it * FTHREADS + t;
        const int f = q >> 6, l = q & 63;
        const int row = 32 * (f >> 2) + (l & 31), col = 16 * (f & 3) + 8 * (l >> 5);
        const int64_t grow = m0 + row, gcol = n0 + col;
        if (grow < M && gcol < width)
          *reinterpret_cast<u32x4*>(ga.out_packed + frag_offset(grow, gcol, kbw)) =
              *reinterpret_cast<const u32x4*>(ot + row * OS + col);
      }
    }
    return;
  }
  constexpr int OS = BN + 8;  // bf16 per LDS row; 256 rows (two waves) per pass
  uint16_t* const ot = reinterpret_cast<uint16_t*>(smem);
  uint16_t* const out = ga.seg[sgi].out;
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
    if ((wave >> 1) == ph) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = (wave & 1) * 128 + i * 32 + lrow;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = j * 32 + 8 * q + 4 * (lane >> 5);
            uint2 v;
            v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<uint2*>(ot + row * OS + col) = v;
          }
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 256 * BN / 8 / FTHREADS; ++it) {
      const int q = it * FTHREADS + t;
      const int row = q / (BN / 8), c8 = q % (BN / 8);
      const int64_t grow = m0 + 256 * ph + row, gcol = n0 + 8 * c8;
      if (grow < M && gcol < n_out)
        *reinterpret_cast<u32x4*>(out + grow * n_out + gcol) = *reinterpret_cast<const u32x4*>(ot + row * OS + 8 * c8);
    }
    __syncthreads();
  }
}

// ---- backward kernel: one wave per SIMD -----------------------------------
// k_gemm_fwd's construction for the backward orientation, dx = dy . W': 256
// threads = 4 waves, one per SIMD, each owning 128 output rows x 128 columns
// (4x4 MFMA tiles, 256 fp32 accumulators); the workgroup tile is 512 rows x
// 128 columns (columns = k_in), the contraction (n_out) in steps of 64 rows
// of W. The decode is k_gemm's backward producer, done by all 256 threads
// (thread t = producer thread pt of k_gemm): a 4x8 patch of codes per thread
// and step, paired along the contraction as it is packed, stored transposed
// into the XOR-swizzled LDS layout; the 128 block scales of a stage are
// decoded twice over (threads t and t+128 alike) and published through a
// two-slot LDS ring. Stage X:
//  * step X-5: its scale codes are fetched; step X-3: its block scale is
//    decoded and published (the barrier that ends the step makes it visible);
//  * step X-4: its patch codes are fetched; step X-2: the pair lookups run
//    through sub-step 0 and the products, bf16 pairs and 8-byte LDS stores
//    every other MFMA of sub-step 1, so no lookup lives across a step;
//  * three LDS stages, one barrier per step;
//  * the per-element contraction order is k_gemm's: same bits for the same
//    split of the contraction.
// With 512-row tiles the grid has half k_gemm's tiles, so where that needs
// more splits the fp32 partials double; the plan takes this kernel for groups
// of two or more weights (always split: every weight has its own splits)
// where the grid still fills the chip with long splits, and for a single
// weight where its grid needs no split at all (SPLIT = false: bf16 output).
template <bool SPLIT>
__global__ __launch_bounds__(FTHREADS, 1) void k_gemm_bwd512(GemmArgs ga, Tables tab) {
  // tile order as k_gemm's backward: the column tiles of one (row tile,
  // split) pair share XCDs when the host asks for it
  const int C = (int)gridDim.x, R = (int)gridDim.y;
  const int id = (int)blockIdx.x + C * (int)blockIdx.y;
  int ct = (int)blockIdx.x, rt = (int)blockIdx.y, zz = (int)blockIdx.z;
  if (ga.xcd_pairs) {
    const int P = R * (int)gridDim.z;
    const int G = P >= 8 ? 1 : 8 / P;
    const int flat = id + C * R * (int)blockIdx.z;
    if ((P % 8 == 0 || 8 % P == 0) && C % G == 0) {
      const int x = flat % 8, sl = flat / 8, cg = C / G;
      const int pair = x / G + 8 * (sl / cg);
      ct = (sl % cg) * G + x % G;
      rt = pair % R;
      zz = pair / R;
    }
  }
  int sgi = 0;
#pragma unroll
  for (int q = 1; q < GEMM_MAX_SEG; ++q)
    if (q < ga.nseg && zz >= ga.seg[q].z0) sgi = q;
  const GemmSeg& sg = ga.seg[sgi];
  const int64_t M = ga.M, k_in = ga.k_in, Nc = ga.Nc, Kc = sg.n_out;

  __shared__ __attribute__((aligned(16))) uint8_t smem[F_SMEM_BYTES + 2 * SCALE_FLOATS * 4];
  uint16_t* const Bs0 = reinterpret_cast<uint16_t*>(smem);
  float2* const s_pair_all = reinterpret_cast<float2*>(smem + FNST * STAGE_ELEMS * 2);
  float* const s_c8 = reinterpret_cast<float*>(smem + FNST * STAGE_ELEMS * 2 + 256 * PAIR_COPIES * 8);
  float* const s_scale = reinterpret_cast<float*>(smem + F_SMEM_BYTES);  // [2][SCALE_FLOATS]
  const int t = threadIdx.x;
  fill_tables(s_pair_all, s_c8, tab, t);
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  auto stage = [&](int st) { return Bs0 + st * STAGE_ELEMS; };

  const int64_t n0 = (int64_t)ct * BN;
  const int64_t m0 = (int64_t)rt * FBM;
  const int zpart = zz;
  const int split = zpart - sg.z0;
  const int64_t kb = split * sg.kc_chunk;
  const int64_t ke = (kb + sg.kc_chunk < Kc) ? kb + sg.kc_chunk : Kc;
  const int nk = (int)((ke - kb + BK - 1) / BK);

  // activation (dy) fragments, as in k_gemm_fwd
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc((void*)sg.afrag, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const int64_t nblk = (M + PACK_ROWS - 1) / PACK_ROWS * (PACK_ROWS / 32);
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t b = (m0 + wave * 128 + i * 32) / 32;
    b = b < nblk ? b : nblk - 1;
    aoff[i] = (uint32_t)(b * sg.kblocks * FRAG_BYTES + lane * 16);
  }
  auto a_soff = [&](int k) {
    const int kc = k < nk ? k : nk - 1;
    return (int)(((kb + (int64_t)kc * BK) / 16) * FRAG_BYTES);
  };

  // weights (k_gemm's backward producer map, pt = t): rows 4 kg + i of a
  // step, columns n0 + mcol .. + 8 (clamped inside k_in; the block scale of
  // a column block past k_in is 0). Every contraction length here is a
  // multiple of 64 (the plan's condition), so every step is whole and every
  // code offset is the thread's own offset plus a wave-uniform row offset.
  // Every thread loads the block scale of row (pt/2)%64, column block pt%2:
  // threads pt and pt+128 load and publish the same one, which keeps the
  // loop free of branches.
  const int pt = t;
  const int kg = bwd_kg(pt), mcol = 8 * bwd_m(pt), r0p = 4 * kg;
  const uint32_t kin2 = (uint32_t)(k_in / 2), kblk = (uint32_t)(k_in / 64);
  int64_t col = n0 + mcol;
  col = col < k_in ? col : k_in - 8;
  const int64_t bcol = n0 + 64 * (pt & 1);
  const bool scol = bcol < k_in;
  const uint32_t sblk = (uint32_t)((scol ? bcol : 0) / 64);
  const int srow = (pt >> 1) & 63;
  const uint32_t woff0 = (uint32_t)r0p * kin2 + (uint32_t)(col / 2);  // the thread's part
  const uint32_t sbase = (uint32_t)srow * kblk + sblk;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)sg.packed, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const __amdgpu_buffer_rsrc_t qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)sg.q8, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const __amdgpu_buffer_rsrc_t nr =
      __builtin_amdgcn_make_buffer_rsrc((void*)sg.nested, (short)0, (int)0xFFFFFFFFu, 0x00020000);
  const float off = sg.offset[0];
  // a stage's codes: four packed words (the patch), and the scale code and
  // nested scale of the thread's block scale, fetched at different times
  struct WCodes {
    uint32_t w[4];
  };
  struct QCodes {
    uint32_t q;
    float nest;
  };
  auto load_w = [&](int k, WCodes& c) {
    const int kc = k < nk ? k : nk - 1;
    const uint32_t k0 = (uint32_t)(kb + kc * BK);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c.w[i] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff0, (int)((k0 + i) * kin2), 0);
  };
  auto load_q = [&](int k, QCodes& c) {
    const int kc = k < nk ? k : nk - 1;
    const uint32_t blk = sbase + (uint32_t)(kb + kc * BK) * kblk;
    c.q = __builtin_amdgcn_raw_buffer_load_b8(qr, blk, 0, 0);
    c.nest = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(nr, (blk >> 8) * 4, 0, 0));
  };
  const PairTab ptab{reinterpret_cast<const uint8_t*>(s_pair_all), (uint32_t)(t & (PAIR_COPIES - 1)) * 8u};
  float2 pv[16];  // pair lookups of the stage being decoded: [byte q * 4 + row i]
  float cq = 0.0f;
  float4 a4;      // the block scales of the thread's four rows
  // the block scale of stage x into ring slot x%2: scale code lookup, then
  // the decode and store
  auto scale_code = [&](const QCodes& c) { cq = s_c8[c.q]; };
  auto scale_put = [&](const QCodes& c, int x) {
    s_scale[(x & 1) * SCALE_FLOATS + (pt & 1) * 64 + srow] = scol ? decode_scale(cq, c.nest, off) : 0.0f;
  };
  // decoding stage x into LDS stage st: pair lookups, the four block scales
  // (published one step earlier), then half h (byte q = h/2, column 2q + h%2
  // of the patch) -- four products, two bf16 pairs along the contraction,
  // one 8-byte store (k_gemm's backward decode, in pieces)
  auto lookup = [&](const WCodes& c, int u) { pv[u] = pair_of(ptab, c.w[u & 3], u >> 2); };
  auto fin_scales = [&](int x) {
    a4 = *reinterpret_cast<const float4*>(s_scale + (x & 1) * SCALE_FLOATS + (bwd_m(pt) >> 3) * 64 + r0p);
  };
  // column mcol + c of the patch lands at wbase + c * LDS_STRIDE: the
  // swizzle bwd_swizzle_off(mcol + c, r0p) is the same for c < 8, since
  // mcol is a multiple of 8
  const int wbase = mcol * LDS_STRIDE + bwd_swizzle_off(mcol, r0p);
  auto fin_half = [&](int st, int h) {
    const int q = h >> 1, hi = h & 1;
    const float a[4] = {a4.x, a4.y, a4.z, a4.w};
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __fmul_rn(hi ? pv[q * 4 + i].y : pv[q * 4 + i].x, a[i]);
    uint2 p;
    p.x = pack_bf16x2(v[0], v[1]);
    p.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(stage(st) + wbase + (2 * q + hi) * LDS_STRIDE) = p;
  };
  auto decode_all = [&](const WCodes& c, int x, int st) {
#pragma unroll
    for (int u = 0; u < 16; ++u) lookup(c, u);
    fin_scales(x);
#pragma unroll
    for (int h = 0; h < 8; ++h) fin_half(st, h);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // stage X: scale codes fetched in step X-5, block scale published in step
  // X-3, patch codes fetched in step X-4, looked up and decoded into LDS in
  // step X-2 -- the pair lookups never live across a step
  WCodes w0, w1;  // patch codes of even and odd stages
  QCodes q0, q1;  // scale codes of even and odd stages
  u32x4 A0[4][4], A1[4][4];
  auto issue_a = [&](u32x4 (&A)[4][4], int k) {
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i][gg] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], a_soff(k) + gg * FRAG_BYTES, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // prologue: stages 0 and 1 decoded, the scale of stage 2 published, the
  // patch codes of stages 2 and 3 and the scale codes of 3 and 4 in flight
  load_w(0, w0);
  load_q(0, q0);
  load_w(1, w1);
  load_q(1, q1);
  issue_a(A0, 0);
  issue_a(A1, 1);
  __syncthreads();  // tables in LDS
  scale_code(q0);
  scale_put(q0, 0);
  scale_code(q1);
  scale_put(q1, 1);
  load_q(2, q0);
  load_q(3, q1);
  __syncthreads();  // scales of stages 0 and 1 published
  decode_all(w0, 0, 0);
  decode_all(w1, 1, 1);
  load_w(2, w0);
  load_w(3, w1);
  __syncthreads();  // every thread is past the scales of stages 0 and 1
  scale_code(q0);
  scale_put(q0, 2);
  load_q(4, q0);
  __syncthreads();  // stages 0 and 1 in LDS, the scale of stage 2 published
  // b_frag<true>(bs, lane, j, kk) with its swizzle split into a lane part
  // and a constant: for column 32 j + l%32 and contraction 16 kk + 8 (l/32)
  // the swizzled offset is 16 (kk ^ j) + 8 ((l/32) ^ (l/16 % 2))
  const int fbase = (lane & 31) * LDS_STRIDE + 8 * (((lane >> 5) ^ (lane >> 4)) & 1);
  auto bfrag = [&](int st, int j, int kk) {
    return *reinterpret_cast<const bf16x8_t*>(stage(st) + fbase + 32 * j * LDS_STRIDE + 16 * (kk ^ j));
  };
  bf16x8_t fb0[4], fb1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fb0[j] = bfrag(0, j, 0);

  // step s: multiply LDS stage st = s % FNST (activation set A); decode
  // stage s+2 (patch codes wc) into LDS stage (s+2) % FNST; publish the
  // scale of stage s+3 (scale codes qc); fetch the patch codes of stage s+4
  // into wc and the scale codes of stage s+5 into qc
  auto step = [&](int s, int st, u32x4 (&A)[4][4], WCodes& wc, QCodes& qc) __attribute__((always_inline)) {
    const int s1 = st + 1 < FNST ? st + 1 : st + 1 - FNST;
    const int s2 = st + 2 < FNST ? st + 2 : st + 2 - FNST;
    const int a2 = a_soff(s + 2);
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      bf16x8_t(&fc)[4] = (gg & 1) ? fb1 : fb0;
      bf16x8_t(&fn)[4] = (gg & 1) ? fb0 : fb1;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc[j], __builtin_bit_cast(bf16x8_t, A[i][gg]),
                                                            acc[i][j], 0, 0, 0);
        if (m < 4) fn[m] = (gg < 3) ? bfrag(st, m, gg + 1) : bfrag(s1, m, 0);
        if (j == 3) A[i][gg] = __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[i], a2 + gg * FRAG_BYTES, 0);
        // stage s+2: lookups through sub-step 0, scales, then a half-column
        // every other MFMA of sub-step 1
        if (gg == 0) lookup(wc, m);
        if (gg == 0 && m == 15) fin_scales(s + 2);
        if (gg == 1 && (m & 1)) fin_half(s2, m >> 1);
        // stage s+3's block scale; then the codes of s+4 and s+5
        if (gg == 2 && m == 0) scale_code(qc);
        if (gg == 2 && m == 4) scale_put(qc, s + 3);
        if (gg == 3 && m == 8) {
          load_w(s + 4, wc);
          load_q(s + 5, qc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // stage s+2 is in set (s+2)%2 = s%2 of the patch codes, stage s+3 in set
  // (s+3)%2 = (s+1)%2 of the scale codes
  int s = 0;
  for (; s + 5 < nk; s += 6) {
    step(s, 0, A0, w0, q1);
    step(s + 1, 1, A1, w1, q0);
    step(s + 2, 2, A0, w0, q1);
    step(s + 3, 0, A1, w1, q0);
    step(s + 4, 1, A0, w0, q1);
    step(s + 5, 2, A1, w1, q0);
  }
  for (; s + 1 < nk; s += 2) {
    step(s, s % FNST, A0, w0, q1);
    step(s + 1, (s + 1) % FNST, A1, w1, q0);
  }
  if (s < nk) step(s, s % FNST, A0, w0, q1);

  // LoRA term (split 0): + du[m, :] . A[:, n], in chunks of 16 over the rank
  if (sg.lora_l != nullptr && split == 0) {
    for (int r0 = 0; r0 < ga.r; r0 += 16) {
      bf16x8_t fa[4], fbl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wave * 128 + i * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (row < M && rr < ga.r) ? sg.lora_l[row * ga.r + rr] : 0.0f;
        }
        fa[i] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + j * 32 + lrow;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = r0 + lk + e;
          v[e] = (col < Nc && rr < ga.r) ? sg.lora_r[(int64_t)rr * k_in + col] : 0.0f;
        }
        fbl[j] = f32x8_to_bf16(v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fbl[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  // output through LDS: bf16, 256 rows (two waves) per pass, or the fp32
  // partial of this split, 128 rows (one wave) per pass
  if constexpr (!SPLIT) {
    constexpr int OS = BN + 8;
    uint16_t* const ot = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      if ((wave >> 1) == ph) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = (wave & 1) * 128 + i * 32 + lrow;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint2 v;
              v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
              v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              *reinterpret_cast<uint2*>(ot + row * OS + j * 32 + 8 * q + 4 * (lane >> 5)) = v;
            }
          }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 256 * BN / 8 / FTHREADS; ++it) {
        const int q = it * FTHREADS + t;
        const int row = q / (BN / 8), c8 = q % (BN / 8);
        const int64_t grow = m0 + 256 * ph + row, gcol = n0 + 8 * c8;
        if (grow < M && gcol < Nc)
          *reinterpret_cast<u32x4*>(sg.out + grow * Nc + gcol) = *reinterpret_cast<const u32x4*>(ot + row * OS + 8 * c8);
      }
      __syncthreads();
    }
  } else {
    constexpr int OS = BN + 4;
    float* const ot = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int ph = 0; ph < 4; ++ph) {
      if (wave == ph) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = i * 32 + lrow;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(ot + row * OS + j * 32 + 8 * q + 4 * (lane >> 5)) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 128 * BN / 4 / FTHREADS; ++it) {
        const int q = it * FTHREADS + t;
        const int row = q / (BN / 4), c4 = q % (BN / 4);
        const int64_t grow = m0 + 128 * ph + row, gcol = n0 + 4 * c4;
        if (grow < M && gcol < Nc)
          *reinterpret_cast<u32x4*>(sg.part + ((int64_t)zpart * M + grow) * Nc + gcol) =
              *reinterpret_cast<const u32x4*>(ot + row * OS + 4 * c4);
      }
      __syncthreads();
    }
  }
}

// Sum of the split partials in split order, rounded once to bf16; blockIdx.y
// selects the weight of a grouped launch. With res_out, also the residual
// stream res_out = res_in + bf16 result in fp32 (what k_residual_add computes
// from the bf16 output).
struct SumSegs {
  const float* part[GEMM_MAX_SEG];
  uint16_t* out[GEMM_MAX_SEG];
  int64_t n[GEMM_MAX_SEG];
  const float* res_in[GEMM_MAX_SEG];
  float* res_out[GEMM_MAX_SEG];
};

__global__ __launch_bounds__(256) void k_split_sum(SumSegs sg, int splits) {
  const int sgi = blockIdx.y;
  const float* __restrict__ part = sg.part[sgi];
  uint16_t* __restrict__ out = sg.out[sgi];
  const int64_t n = sg.n[sgi];
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  if (i + 4 <= n) {
    // every load issued ahead of the adds, which keep split order
    const bool res = sg.res_out[sgi] != nullptr;
    float4 h = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (res) h = *reinterpret_cast<const float4*>(sg.res_in[sgi] + i);
    float4 s = *reinterpret_cast<const float4*>(part + i);
    for (int p = 1; p < splits; p += 8) {
      float4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (p + q < splits) v[q] = *reinterpret_cast<const float4*>(part + (int64_t)(p + q) * n + i);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (p + q < splits) {
          s.x += v[q].x; s.y += v[q].y; s.z += v[q].z; s.w += v[q].w;
        }
    }
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *reinterpret_cast<uint2*>(out + i) = o;
    if (res) {
      float4 r;
      r.x = h.x + __uint_as_float(o.x << 16);
      r.y = h.y + __uint_as_float(o.x & 0xFFFF0000u);
      r.z = h.z + __uint_as_float(o.y << 16);
      r.w = h.w + __uint_as_float(o.y & 0xFFFF0000u);
      *reinterpret_cast<float4*>(sg.res_out[sgi] + i) = r;
    }
  } else {
    for (int64_t e = i; e < n; ++e) {
      float s = part[e];
      for (int p = 1; p < splits; ++p) s += part[(int64_t)p * n + e];
      const uint32_t b = pack_bf16x2(s, 0.0f) & 0xFFFFu;
      out[e] = (uint16_t)b;
      if (sg.res_out[sgi]) sg.res_out[sgi][e] = sg.res_in[sgi][e] + __uint_as_float(b << 16);
    }
  }
}

}  // namespace


static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// A backward's activation blocks are kept on shared XCDs (k_gemm's tile
// mapping) when all of them together exceed two 4 MB L2s.
constexpr int64_t kXcdPairBytes = 8ll << 20;

static GemmPlan plan_tiles(int64_t M, const int64_t* n_cols, int nseg, int64_t k_contract, int bm) {
  GemmPlan p;
  p.bm = bm;
  p.bn = BN;
  int64_t col_tiles = 0;
  for (int q = 0; q < nseg; ++q) col_tiles += (n_cols[q] + BN - 1) / BN;
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * col_tiles;
  const int64_t nk = (k_contract + BK - 1) / BK;
  int splits = 1;
  // Split the contraction while the grid is short of the chip's 256 CUs and
  // each split keeps at least 8 contraction steps.
  while (tiles * splits < 192 && nk / (2 * splits) >= 8) splits *= 2;
  const int64_t steps_per = (nk + splits - 1) / splits;
  p.kc_chunk = steps_per * BK;
  p.splits = (int)((nk + steps_per - 1) / steps_per);
  p.frag_bytes = packed_activation_bytes(M, k_contract);
  p.part_bytes = 0;
  if (p.splits > 1)
    for (int q = 0; q < nseg; ++q)
      p.part_bytes += round256((size_t)p.splits * (size_t)M * (size_t)n_cols[q] * sizeof(float));
  p.ws_bytes = p.frag_bytes + p.part_bytes;
  return p;
}

// The forward NF4 GEMM runs on k_gemm_fwd (512-row tiles) when that grid
// needs no split of the contraction; otherwise on k_gemm, whose 256-row tiles
// give twice the tiles and so at most half the splits: at M = 512 the fp32
// partials of a split launch cost more than the faster kernel saves. Both
// kernels give the same bits for the same split.
GemmPlan plan_gemm_grouped(int64_t M, const int64_t* n_cols, int nseg, int64_t k_contract,
                           bool fwd_nf4) {
  if (fwd_nf4) {
    const GemmPlan wide = plan_tiles(M, n_cols, nseg, k_contract, FBM);
    if (wide.splits == 1) return wide;
  }
  return plan_tiles(M, n_cols, nseg, k_contract, BM);
}

GemmPlan plan_gemm(int64_t M, int64_t n_cols, int64_t k_contract, bool fwd_nf4) {
  return plan_gemm_grouped(M, &n_cols, 1, k_contract, fwd_nf4);
}

// A single NF4 backward runs on k_gemm_bwd512 (no split) where its 512-row
// grid alone fills the chip (plan_tiles' 192 tiles), so that it needs no split
// of the contraction; k_gemm's 256-row grid then needs none either, so the
// workspace is the same. Smaller grids keep k_gemm's twice as many tiles.
static bool bwd512_unsplit(int64_t M, int64_t n_out, int64_t k_in) {
  if (n_out % BK != 0 || n_out * (k_in / 2) >= ((int64_t)1 << 31)) return false;
  return ((M + FBM - 1) / FBM) * ((k_in + BN - 1) / BN) >= 192;
}

// Launches the GEMM (and the split sum when the contraction is split) for
// C[M, Nc] = A . B with the weight given either as NF4 tensors (q: nseg of
// them, forward only when nseg > 1) or as a dense bf16 matrix (wd).
static hipError_t launch_gemm(bool backward, const QPtrs* q, int nseg, const uint16_t* wd,
                              const int64_t* n_outs, int64_t k_in, const uint8_t* a_packed,
                              int64_t M, uint16_t* const* outs, const float* const* lora_ls,
                              const float* const* lora_rs, int r, float scale, void* part_ws,
                              hipStream_t s, const float* res_in = nullptr,
                              float* res_out = nullptr) {
  GemmArgs g = {};
  g.wd = wd;
  g.M = M;
  g.k_in = k_in;
  g.Kc = backward ? n_outs[0] : k_in;
  g.Nc = backward ? k_in : n_outs[0];
  g.n_out = n_outs[0];
  int64_t ncols[GEMM_MAX_SEG];
  for (int i = 0; i < nseg; ++i) ncols[i] = backward ? k_in : n_outs[i];
  const bool fwd_nf4 = !backward && wd == nullptr;
  const GemmPlan p = plan_gemm_grouped(M, ncols, nseg, g.Kc, fwd_nf4);
  g.afrag = a_packed;
  g.kblocks = (g.Kc + BK - 1) / BK * (BK / 16);
  g.kc_chunk = p.kc_chunk;
  g.r = r;
  g.scale = scale;
  g.nseg = nseg;
  SumSegs sum = {};
  int tile0 = 0;
  int64_t max_n = 0;
  uint8_t* part = static_cast<uint8_t*>(part_ws);
  for (int i = 0; i < nseg; ++i) {
    GemmSeg& sg = g.seg[i];
    if (q) {
      sg.packed = q[i].packed;
      sg.q8 = q[i].q8;
      sg.nested = q[i].nested;
      sg.offset = q[i].offset;
    }
    sg.out = outs[i];
    if (backward) {  // the single weight along the contraction
      sg.afrag = a_packed;
      sg.kblocks = g.kblocks;
      sg.kc_chunk = p.kc_chunk;
    }
    sg.lora_l = lora_ls ? lora_ls[i] : nullptr;
    sg.lora_r = lora_rs ? lora_rs[i] : nullptr;
    sg.n_out = n_outs[i];
    sg.tile0 = tile0;
    tile0 += (int)((ncols[i] + BN - 1) / BN);
    const int64_t n = M * ncols[i];
    if (p.splits > 1) {
      sg.part = reinterpret_cast<float*>(part);
      part += round256((size_t)p.splits * (size_t)n * sizeof(float));
    }
    sum.part[i] = sg.part;
    sum.out[i] = sg.out;
    sum.n[i] = n;
    sum.res_in[i] = res_in;
    sum.res_out[i] = res_out;
    max_n = n > max_n ? n : max_n;
  }
  const bool split = p.splits > 1;
  // a single NF4 backward whose 512-row grid needs no split: k_gemm_bwd512
  const bool bwd_wide = backward && wd == nullptr && nseg == 1 && bwd512_unsplit(M, n_outs[0], k_in);
  const int bm = bwd_wide ? FBM : p.bm;
  const dim3 grid((unsigned)tile0, (unsigned)((M + bm - 1) / bm), (unsigned)p.splits);
  g.xcd_pairs = backward && wd == nullptr && 2 * M * g.Kc > kXcdPairBytes;
  const Tables& tab = host_tables();
  // forward NF4 without a split: k_gemm_fwd; everything else: k_gemm
#define NF4S_GEMM(B_, S_, D_) hipLaunchKernelGGL((k_gemm<B_, S_, D_>), grid, dim3(THREADS), 0, s, g, tab)
  if (fwd_nf4 && p.bm == FBM) {
    hipLaunchKernelGGL(k_gemm_fwd<false>, grid, dim3(FTHREADS), 0, s, g, tab);
  } else if (bwd_wide) {
    hipLaunchKernelGGL(k_gemm_bwd512<false>, grid, dim3(FTHREADS), 0, s, g, tab);
  } else if (wd == nullptr) {
    if (backward && split) NF4S_GEMM(true, true, false);
    else if (backward) NF4S_GEMM(true, false, false);
    else if (split) NF4S_GEMM(false, true, false);
    else NF4S_GEMM(false, false, false);
  } else {
    if (backward && split) NF4S_GEMM(true, true, true);
    else if (backward) NF4S_GEMM(true, false, true);
    else if (split) NF4S_GEMM(false, true, true);
    else NF4S_GEMM(false, false, true);
  }
#undef NF4S_GEMM
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits == 1)  // the residual from the bf16 output, as a kernel of its own
    return res_out ? launch_residual_add(res_in, outs[0], M * n_outs[0], res_out, s) : hipSuccess;
  const dim3 g2((unsigned)((max_n / 4 + 1 + 255) / 256), (unsigned)nseg);
  hipLaunchKernelGGL(k_split_sum, g2, dim3(256), 0, s, sum, p.splits);
  return hipGetLastError();
}

hipError_t launch_linear_packed(bool backward, const QPtrs& q, int64_t n_out, int64_t k_in,
                                const uint8_t* a_packed, int64_t M, uint16_t* out,
                                const float* lora_l, const float* lora_r, int r, float scale,
                                void* part_ws, hipStream_t s) {
  return launch_gemm(backward, &q, 1, nullptr, &n_out, k_in, a_packed, M, &out, &lora_l, &lora_r, r,
                     scale, part_ws, s);
}

hipError_t launch_linear_fwd_residual(const QPtrs& q, int64_t n_out, int64_t k_in,
                                      const uint8_t* x_packed, int64_t M, uint16_t* y,
                                      const float* lora_u, const float* lora_B, int r, float scale,
                                      const float* h_in, float* h_out, void* part_ws, hipStream_t s) {
  return launch_gemm(false, &q, 1, nullptr, &n_out, k_in, x_packed, M, &y, &lora_u, &lora_B, r, scale,
                     part_ws, s, h_in, h_out);
}

hipError_t launch_linear_grouped_fwd(const QPtrs* q, int nseg, const int64_t* n_outs, int64_t k_in,
                                     const uint8_t* x_packed, int64_t M, uint16_t* const* ys,
                                     const float* const* lora_us, const float* const* lora_Bs,
                                     int r, float scale, void* part_ws, hipStream_t s) {
  return launch_gemm(false, q, nseg, nullptr, n_outs, k_in, x_packed, M, ys, lora_us, lora_Bs, r,
                     scale, part_ws, s);
}

// The gate + up forward with the SwiGLU epilogue runs on k_gemm_fwd<true>,
// which has no split path: it is planned only where the grid of 512-row
// tiles of 64 gate and 64 up columns needs no split by plan_tiles' rule.
bool swiglu_fused_ok(int64_t M, int64_t width, int64_t k_in) {
  const int64_t tiles = ((M + FBM - 1) / FBM) * ((width + BN / 2 - 1) / (BN / 2));
  const int64_t nk = (k_in + BK - 1) / BK;
  return tiles >= 192 || nk / 2 < 8;
}

bool swiglu_tiles(int64_t M, int64_t width, int64_t k_in, int* bm, int* bn) {
  *bm = FBM;
  *bn = BN;
  return swiglu_fused_ok(M, width, k_in);
}

hipError_t launch_linear_swiglu_fwd(const QPtrs* q, int64_t width, int64_t k_in, const uint8_t* x_packed,
                                    int64_t M, uint16_t* out, uint8_t* out_packed,
                                    const float* const* lora_us, const float* const* lora_Bs, int r,
                                    float scale, hipStream_t s) {
  GemmArgs g = {};
  g.M = M;
  g.k_in = k_in;
  g.Kc = k_in;
  g.Nc = width;
  g.n_out = width;
  g.afrag = x_packed;
  g.kblocks = (k_in + BK - 1) / BK * (BK / 16);
  g.kc_chunk = (k_in + BK - 1) / BK * BK;
  g.r = r;
  g.scale = scale;
  g.nseg = 2;
  g.out_packed = out_packed;
  for (int i = 0; i < 2; ++i) {
    GemmSeg& sg = g.seg[i];
    sg.packed = q[i].packed;
    sg.q8 = q[i].q8;
    sg.nested = q[i].nested;
    sg.offset = q[i].offset;
    sg.out = out;
    sg.lora_l = lora_us ? lora_us[i] : nullptr;
    sg.lora_r = lora_Bs ? lora_Bs[i] : nullptr;
    sg.n_out = width;
  }
  const dim3 grid((unsigned)((width + BN / 2 - 1) / (BN / 2)), (unsigned)((M + FBM - 1) / FBM), 1u);
  hipLaunchKernelGGL(k_gemm_fwd<true>, grid, dim3(FTHREADS), 0, s, g, host_tables());
  return hipGetLastError();
}

// Splits of a grouped backward: split j's contraction into S_j chunks of c
// steps, the smallest c for which the grid still fits one wave of 256
// workgroups (so the slowest workgroup runs as few steps as possible), never
// below 8 steps; a group of one plans as the single call. Planned for
// k_gemm's 256-row tiles and for k_gemm_bwd512's 512-row tiles; the latter
// is taken where its splits keep at least 32 steps (its per-step cost is
// about 1.6 times k_gemm's for twice the rows, and its partials are twice as
// many, which long splits amortise).
static BwdGroupPlan plan_bwd_tiles(int64_t M, const int64_t* n_outs, int n, int64_t k_in, int bm) {
  BwdGroupPlan bp = {};
  bp.bm = bm;
  const int64_t tiles = ((M + bm - 1) / bm) * ((k_in + BN - 1) / BN);
  int64_t steps[GEMM_MAX_SEG], cmax = 0;
  for (int j = 0; j < n; ++j) {
    steps[j] = (n_outs[j] + BK - 1) / BK;
    cmax = steps[j] > cmax ? steps[j] : cmax;
  }
  int64_t best = cmax;
  for (int64_t c = cmax; c >= 8; --c) {
    int64_t sz = 0;
    for (int j = 0; j < n; ++j) sz += (steps[j] + c - 1) / c;
    if (tiles * sz > 256) break;
    best = c;
  }
  bp.total = 0;
  bp.cmax = 0;
  for (int j = 0; j < n; ++j) {
    const int64_t c = best < steps[j] ? best : steps[j];
    bp.splits[j] = (int)((steps[j] + c - 1) / c);
    bp.kc_chunk[j] = c * BK;
    bp.total += bp.splits[j];
    bp.cmax = c > bp.cmax ? (int)c : bp.cmax;
  }
  bp.part_bytes = bp.total > 1 ? round256((size_t)bp.total * (size_t)M * (size_t)k_in * sizeof(float)) : 0;
  return bp;
}

BwdGroupPlan plan_bwd_grouped(int64_t M, const int64_t* n_outs, int n, int64_t k_in) {
  if (n == 1) {
    BwdGroupPlan bp = {};
    const GemmPlan p = plan_gemm(M, k_in, n_outs[0], false);
    bp.bm = bwd512_unsplit(M, n_outs[0], k_in) ? FBM : BM;
    bp.splits[0] = p.splits;
    bp.kc_chunk[0] = p.kc_chunk;
    bp.total = p.splits;
    bp.cmax = (int)(p.kc_chunk / BK);
    bp.part_bytes = bp.total > 1 ? round256((size_t)bp.total * (size_t)M * (size_t)k_in * sizeof(float)) : 0;
    return bp;
  }
  // k_gemm_bwd512 addresses a weight's codes with 32-bit offsets and takes
  // whole 64-row contraction steps only
  bool fits = true;
  for (int j = 0; j < n; ++j) fits = fits && n_outs[j] * (k_in / 2) < ((int64_t)1 << 31) && n_outs[j] % BK == 0;
  const BwdGroupPlan wide = plan_bwd_tiles(M, n_outs, n, k_in, FBM);
  if (fits && wide.cmax >= 32) return wide;
  return plan_bwd_tiles(M, n_outs, n, k_in, BM);
}

hipError_t launch_linear_grouped_bwd(const QPtrs* q, int n, const int64_t* n_outs, int64_t k_in,
                                     const uint8_t* const* dy_packed, int64_t M, uint16_t* dx,
                                     const float* const* lora_dus, const float* const* lora_As,
                                     int r, void* part_ws, hipStream_t s) {
  const BwdGroupPlan bp = plan_bwd_grouped(M, n_outs, n, k_in);
  GemmArgs g = {};
  g.M = M;
  g.k_in = k_in;
  g.Nc = k_in;
  g.r = r;
  g.nseg = n;
  int z0 = 0;
  for (int j = 0; j < n; ++j) {
    GemmSeg& sg = g.seg[j];
    sg.packed = q[j].packed;
    sg.q8 = q[j].q8;
    sg.nested = q[j].nested;
    sg.offset = q[j].offset;
    sg.out = dx;
    sg.part = bp.total > 1 ? static_cast<float*>(part_ws) : nullptr;
    sg.lora_l = lora_dus ? lora_dus[j] : nullptr;
    sg.lora_r = lora_As ? lora_As[j] : nullptr;
    sg.n_out = n_outs[j];
    sg.z0 = z0;
    sg.afrag = dy_packed[j];
    sg.kblocks = (n_outs[j] + BK - 1) / BK * (BK / 16);
    sg.kc_chunk = bp.kc_chunk[j];
    z0 += bp.splits[j];
  }
  const dim3 grid((unsigned)((k_in + BN - 1) / BN), (unsigned)((M + bp.bm - 1) / bp.bm), (unsigned)bp.total);
  int64_t a_bytes = 0;
  for (int j = 0; j < n; ++j) a_bytes += 2 * M * n_outs[j];
  g.xcd_pairs = a_bytes > kXcdPairBytes;
  const Tables& tab = host_tables();
  if (bp.bm == FBM) {
    if (bp.total > 1) hipLaunchKernelGGL(k_gemm_bwd512<true>, grid, dim3(FTHREADS), 0, s, g, tab);
    else hipLaunchKernelGGL(k_gemm_bwd512<false>, grid, dim3(FTHREADS), 0, s, g, tab);
  } else if (bp.total > 1) {
    hipLaunchKernelGGL((k_gemm<true, true, false>), grid, dim3(THREADS), 0, s, g, tab);
  } else {
    hipLaunchKernelGGL((k_gemm<true, false, false>), grid, dim3(THREADS), 0, s, g, tab);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || bp.total == 1) return e;
  SumSegs sum = {};
  sum.part[0] = static_cast<const float*>(part_ws);
  sum.out[0] = dx;
  sum.n[0] = M * k_in;
  hipLaunchKernelGGL(k_split_sum, dim3((unsigned)((M * k_in / 4 + 1 + 255) / 256), 1u), dim3(256), 0, s,
                     sum, bp.total);
  return hipGetLastError();
}

hipError_t launch_dense_packed(bool backward, const uint16_t* w, int64_t n_out, int64_t k_in,
                               const uint8_t* a_packed, int64_t M, uint16_t* out, void* part_ws,
                               hipStream_t s) {
  return launch_gemm(backward, nullptr, 1, w, &n_out, k_in, a_packed, M, &out, nullptr, nullptr, 0,
                     0.0f, part_ws, s);
}

}  // namespace nf4s
