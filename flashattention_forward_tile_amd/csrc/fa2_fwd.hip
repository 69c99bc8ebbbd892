// fa2_fwd.hip -- FlashAttention-2 forward pass for gfx950 (MI355X, CDNA4).
//
// One workgroup owns one query tile and streams every key/value tile of its
// K/V head through LDS, keeping the running softmax state and the output
// accumulator in registers, so the N x N score matrix never reaches HBM (the
// fusion described in the abstract of "A Case Study in CUDA Kernel Fusion:
// Implementing FlashAttention-2 on NVIDIA Hopper Architecture using the
// CUTLASS Library" and in "Flash Attention 2 from scratch on Ampere", Part 1,
// "Why Flash Attention?").  The per-workgroup flow (query tile held on chip,
// loop over the j-th key/value tile) follows that page's Notation section.
//
// CDNA4 mapping (prior art re-designed, not translated):
//  * Both products run on 32x32 MFMA (16x16 at d = 256).  The first is
//    computed transposed, S^T = K_j Q_i^T, so each lane of a wave owns one
//    query column: lanes l and l+32 hold the two halves of that query's keys
//    (four lanes hold quarters with 16x16), and the softmax needs no
//    cross-lane reduction except exchanges between those lanes.
//  * The S^T accumulator layout is exactly the B-operand layout of the second
//    product O^T += V_j^T P^T once V_j^T is read in the matching key order,
//    which ds_read_b64_tr_b16 does from the row-major V tile, so P never
//    leaves registers.
//  * K_j and V_j go HBM -> LDS by buffer loads that write LDS directly, into
//    XOR-swizzled tiles (bank conflicts were the largest single gain in the
//    Ampere series' table, kernel 2).  Each cycles through a ring of four
//    slots with loads two iterations ahead of their use and the next
//    iteration's first operands read before the closing barrier (kernels 3
//    and 5 of that table pipeline one tile ahead).
//  * d = 256 gives each wave 16 query rows on 16x16x32 MFMA, so its output
//    accumulator and query fragments fit the register budget of two waves
//    per SIMD.
//  * Softmax in fp32 registers with exp2 and the scale folded into one FMA
//    (kernel 6), against a lazy reference max: it moves only when a row's
//    tile sum of p would exceed kSumLimit, which keeps the result exact
//    because every p and l then share the same stale reference.
//  * The query heads that share a K/V head are tiled together (their rows are
//    adjacent in memory), and workgroup ids are remapped so all query tiles of
//    a K/V head land on one XCD and share that XCD's L2 copy of its K and V.
//  * The INT8 and FP8 key/value cache kernels (Q8) quantize each query row in
//    the kernel, run the first product on int8 or FP8 (E4M3) MFMA and widen V
//    to fp16 in LDS.
//  * Key splits (SPLIT): when query tiles are too few to fill the chip (a
//    few query rows against a long cache, as in decoding), each query tile's
//    key tiles are divided among several workgroups, which write fp32
//    partial outputs and logsumexps to a workspace; a second kernel merges
//    them (the softmax of a union of key sets from the parts' logsumexps).

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "fa2.h"

namespace fa2 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

template <bool FP16> struct Vec;
template <> struct Vec<false> {
  using x8 = bf16x8; using x4 = bf16x4; using x2 = bf16x2; using e = __bf16;
};
template <> struct Vec<true> {
  using x8 = f16x8; using x4 = f16x4; using x2 = f16x2; using e = _Float16;
};

template <bool FP16>
__device__ __forceinline__ f32x16 mfma32x32x16(typename Vec<FP16>::x8 a,
                                               typename Vec<FP16>::x8 b,
                                               f32x16 c) {
  if constexpr (FP16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
template <bool FP16>
__device__ __forceinline__ f32x4 mfma16x16x32(typename Vec<FP16>::x8 a, typename Vec<FP16>::x8 b,
                                              f32x4 c) {
  if constexpr (FP16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS tiles are row-major with 16-byte chunks XOR-swizzled per row.  The
// K tile is read with ds_read_b128 by 16 lanes at 16 consecutive rows and one
// logical chunk; the V tile is read with ds_read_b64_tr_b16, for 32x32
// products by 32 lanes at 4 consecutive rows and 4 consecutive chunks, for
// 16x16 products (MS = 16) at 8 consecutive rows and 2 consecutive chunks.
// Each swizzle spreads its pattern over distinct bank groups; CPR is the row
// length in chunks.
template <int CPR>
__device__ __forceinline__ int k_swizzle(int row, int chunk) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16 || CPR == 32, "row of 64 to 512 B");
  if constexpr (CPR >= 16)
    return chunk ^ (row & 15);
  else if constexpr (CPR == 8)  // 128 B rows: two rows share one sweep of the banks
    return chunk ^ ((row >> 1) & 7);
  else  // 64 B rows (8-bit codes at d = 64): four rows share one sweep
    return chunk ^ ((row >> 2) & 3);
}
template <int CPR, int MS = 32>
__device__ __forceinline__ int v_swizzle(int row, int chunk) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "row of 128, 256 or 512 B");
  static_assert(MS == 32 || CPR >= 16, "16x16 reads of rows of 256 B or more");
  if constexpr (MS == 16)
    return chunk ^ ((row & 7) << 1);
  else if constexpr (CPR >= 16)
    return chunk ^ ((row & 3) << 2);
  else
    return chunk ^ (((row >> 1) & 1) << 2);
}

// x of lane l ^ 32: v_permlane32_swap exchanges lanes 32..63 of its first
// operand with lanes 0..31 of its second; with x in both, the second result
// holds the upper half's values in the lower lanes and the first the lower
// half's values in the upper lanes.
__device__ __forceinline__ float other_half(float x, int lane) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
}

// The OCP E4M3 code nearest to t (1 sign, 4 exponent bits with bias 7, 3
// mantissa bits; below 2^-6 the subnormals m * 2^-9), ties to the even code,
// magnitudes above 448 saturating to 448; t is not NaN.  Normal range: the
// binary32 mantissa is rounded to 3 bits in place (a carry moves into the
// exponent) and the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, t);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __builtin_fabsf(t);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // m = 0..8; 8 is 2^-6, the code 0x08
  } else {
    uint32_t u = bits & 0x7fffffffu;
    u += 0x7ffffu + ((u >> 20) & 1u);
    code = (u >> 20) - (120u << 3);
    code = code > 0x7eu ? 0x7eu : code;
  }
  return sign | code;
}

// s_waitcnt with only vmcnt(0): every buffer load of this wave, including
// the ones that write LDS directly, has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but this wave's N most recent buffer loads have
// landed (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer descriptor words 2 and 3: num_records = `bytes`, then a raw untyped
// 32-bit buffer format; loads past `bytes` return zeros.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufferWord3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The same descriptor as four wave-uniform words, for the inline-asm loads.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kBufferWord3;
  return r;
}

// 16 bytes per lane from buffer offset `voff` straight into LDS: lane l writes
// LDS bytes [m0 + 16 l, m0 + 16 l + 16).  Written as inline asm so the compiler
// does not guard every later LDS read with a wait on these loads (it cannot
// tell the double buffers apart); the caller waits with wait_vmem() before
// the barrier that publishes the tile.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// Tile shape per head dimension: key rows per tile (BC), waves per workgroup
// (NW), MS-query blocks per wave (QB), the waves per SIMD the register
// budget is sized for (OCC), whether the iteration block carries explicit
// MFMA / LDS / VALU interleave hints (SGB), the LDS slots per K and V ring
// (RING), how many K and V operands of each product are read from LDS one
// iteration early (PK, PV), and the matrix instruction shape (MS = 32:
// 32x32x16, MS = 16: 16x16x32), which is also the query rows of one block.
// Each K or V operand read from LDS feeds QB matrix instructions, so LDS
// bytes per FLOP fall as 1/QB.
//
// d = 256 uses the 16x16x32 shape: a wave of 32 query rows would hold 128
// accumulator and 64 query-fragment registers, more than two waves per SIMD
// allow, while 16 rows hold half of each.  Every wave still reads all of each
// K and V tile, so the LDS bytes per FLOP are twice those of the 32-row
// waves at d = 128 (the transposed-read pattern of V then spans 8 rows, which
// its swizzle spreads over the banks).
//
// K and V tiles cycle through rings of RING = 4 LDS slots: tile t sits in
// slot t % 4, K_t is loaded during iteration t - 4 and V_t during iteration
// t - 2, and each iteration waits only for the loads of the one before it,
// so every load has two iterations to land and the operands an iteration
// reads were published one barrier early (which is what lets PK, PV > 0).
// At d = 256 the rings take 128 KiB of a workgroup's LDS.
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int BC = 64, NW = 4, QB = 1, OCC = 2, SGB = 1, RING = 4, PK = 4, PV = 2, MS = 32; };
template <> struct Cfg<128> { static constexpr int BC = 32, NW = 8, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 4, PV = 2, MS = 32; };
template <> struct Cfg<256> { static constexpr int BC = 32, NW = 8, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 4, PV = 2, MS = 16; };

// Tile shapes of the INT8 and FP8 key/value cache kernels.
template <int D> struct Cfg8;
template <> struct Cfg8<128> { static constexpr int BC = 32, NW = 8, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 2, PV = 2, MS = 32; };
// d = 64: 64-key tiles, so a code tile (4 KiB) and its fp16 widening (8 KiB)
// split into whole loads and chunks over the eight waves.
template <> struct Cfg8<64> { static constexpr int BC = 64, NW = 8, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 2, PV = 2, MS = 32; };
// d = 256: 16-row waves on the 16x16 int8 / FP8 shapes, as the 16-bit d = 256
// kernels.
template <> struct Cfg8<256> { static constexpr int BC = 32, NW = 8, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 1, PV = 2, MS = 16; };
// The quantized caches with key splits: 128-row tiles (four 32-row waves, or
// eight 16-row waves at d = 256), as the 16-bit split kernels, so that
// decoding forms one tile per K/V head.
template <int D> struct Cfg8S;
template <> struct Cfg8S<128> { static constexpr int BC = 32, NW = 4, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 2, PV = 2, MS = 32; };
template <> struct Cfg8S<64> { static constexpr int BC = 64, NW = 4, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 2, PV = 2, MS = 32; };
template <> struct Cfg8S<256> { static constexpr int BC = 32, NW = 8, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 2, PV = 2, MS = 16; };
// Short key sequences at d = 128 (at most kShortKeys keys): half the query
// rows per workgroup, so two workgroups share a CU and one's prologue and
// epilogue overlap the other's loop.  The same shape serves grids too small
// to give every CU a full-height workgroup.
template <int D> struct CfgS;
template <> struct CfgS<128> { static constexpr int BC = 32, NW = 4, QB = 1, OCC = 2, SGB = 0, RING = 4, PK = 4, PV = 2, MS = 32; };
constexpr int kShortKeys = 1024;
// Persistent workgroups (one per CU, walking several items): the d = 128
// shape, and at d = 64 eight waves of 32 rows (a four-wave workgroup's ring
// and query/output areas, twice over, would not fit two per CU in LDS).
template <int D> struct CfgP : Cfg<D> {};
template <> struct CfgP<64> { static constexpr int BC = 64, NW = 8, QB = 1, OCC = 2, SGB = 1, RING = 4, PK = 4, PV = 2, MS = 32; };
template <int D, bool Q8, bool SHORT, bool PERSIST>
using KCfg = std::conditional_t<
    Q8, std::conditional_t<SHORT, Cfg8S<D>, Cfg8<D>>,
    std::conditional_t<SHORT, CfgS<D>, std::conditional_t<PERSIST, CfgP<D>, Cfg<D>>>>;
// Ring slots and loop phases as compile-time constants.
template <int X> using Ic = std::integral_constant<int, X>;

// p = exp2(t - m_ref) is summed over each lane's keys of a tile; while that
// sum stays at or below kSumLimit no p exceeds it, and the reference max is
// left alone.  Otherwise the row's reference moves to its true running max.
// The limit only has to keep every p, rounded to the 16-bit type of the
// second product, finite with room to spare (fp16 tops out at 65504); a
// higher limit lets the reference move less often when the running max keeps
// climbing (peaky rows: 2^14 instead of 2^8 takes about a third of the
// tiles of N(0, 16) logits off the rescale path).
constexpr float kSumLimit = 16384.0f;

// Race-check build (-DFA2_SYNC_CHECK=1, a second library used by the tests):
// every iteration waits for all of its loads and synchronises the workgroup
// right after issuing them, and the persistent epilogue waits as well, so no
// tile is read before it has landed whatever the ring's deferred waits
// assume.  The arithmetic and its order are unchanged: both builds must give
// the same bits.
#ifndef FA2_SYNC_CHECK
#define FA2_SYNC_CHECK 0
#endif
constexpr bool kSyncCheck = FA2_SYNC_CHECK != 0;

// Sign of the folded scale c = scale * log2(e): the running extreme of the raw
// logits is a max for c > 0 and a min for c < 0; c == 0 is uniform attention.
enum ScaleMode { kPositive = 0, kNegative = 1, kZero = 2 };

// Kernel arguments.  q, o: [B][hq][nq][D]; k, v: [B][hkv][nk][D]; lse:
// [B][hq][nq].  Query head h reads key/value head h / (hq / hkv).  The query
// heads of one K/V head are adjacent, so their rows form one block of
// rows = (hq / hkv) * nq rows in q, o and lse; workgroups tile that block
// (query-head packing), and packed row r is row r % nq of its head.  With
// the causal option row i of a head sees keys j <= i + causal_off
// (causal_off = nk - nq).
struct Problem {
  const uint16_t* q;
  const char* k;     // 16-bit elements, or 8-bit codes for the INT8 / FP8 caches
  const char* v;
  uint16_t* o;
  float* lse;
  const float* ks;   // quantized caches only: per-channel scales [B][hkv][D]
  const float* vs;
  int nq, nk;        // query rows per query head, key rows per K/V head
  int rows;          // query rows per K/V head (its query heads back to back)
  int q_tiles;       // query tiles per K/V head
  int n_groups;      // workgroups in the grid
  int causal_off;
  float c;           // scale * log2(e) (1 when the scale is 0)
};

// Arguments of the key-split kernels (the others keep Problem alone, so
// their argument block and register allocation do not change): each item's
// key tiles are shared out among `splits` workgroups (consecutive ids),
// which write fp32 partials: part_o [splits][part_rows][D] (O of the part's
// keys, normalised by their own sum) and part_lse [splits][part_rows]
// (natural log; -inf: no key seen).  part_rows = B * hq * nq, rows indexed
// as in lse.  With part_o null (one part, splits = 1) the kernel writes o and
// lse itself.
struct SplitProblem : Problem {
  float* part_o;
  float* part_lse;
  int64_t part_rows;
  int splits;
};

// QK selects a quantized key/value cache (Q8 below): 1, int8 codes; 2, FP8
// (OCP E4M3) codes (F8).  K and V arrive as codes with per-channel scales;
// the first product runs on int8 or FP8 matrix instructions against the
// in-kernel quantized query, and V is widened to fp16 in LDS for the second
// product (see the header of fa2.h for the schemes).
// PERSIST: one workgroup per CU walks several (K/V head, query tile) items,
// and the key/value ring runs on from one item into the next (see below).
// SPLIT: key splits (see SplitProblem); non-persistent kernels only.
template <int D, bool FP16, int MODE, bool CAUSAL, int QK, bool SHORT, bool PERSIST, bool SPLIT>
__global__ void __attribute__((amdgpu_flat_work_group_size(KCfg<D, QK != 0, SHORT, PERSIST>::NW * 64,
                                                           KCfg<D, QK != 0, SHORT, PERSIST>::NW * 64),
                               amdgpu_waves_per_eu(KCfg<D, QK != 0, SHORT, PERSIST>::OCC,
                                                   KCfg<D, QK != 0, SHORT, PERSIST>::OCC)))
fa2_fwd_kernel(const std::conditional_t<SPLIT, SplitProblem, Problem> P) {
  constexpr bool Q8 = QK != 0;  // a quantized key/value cache (8-bit codes)
  constexpr bool F8 = QK == 2;  // its codes are FP8 (E4M3) values
  using C = KCfg<D, Q8, SHORT, PERSIST>;
  const int N = P.nk;  // keys per head
  const float c = P.c;
  constexpr int BC = C::BC;
  constexpr int NW = C::NW;
  constexpr int QB = C::QB;
  // Matrix instruction shape: 32x32x16 (MS = 32: a wave block of 32 query
  // rows, lanes l and l+32 share a row) or 16x16x32 (MS = 16: 16 query rows,
  // lanes l, l+16, l+32, l+48 share a row).
  constexpr int MS = C::MS;
  static_assert(MS == 32 || (MS == 16 && !PERSIST), "16x16 blocking");
  constexpr int BR = NW * MS * QB;    // query rows per workgroup
  constexpr int CPR = D / 8;          // 16-byte chunks per (16-bit) V row
  constexpr int RB = D * 2;           // bytes per (16-bit) V row in LDS
  constexpr int TBYTES = BC * RB;     // one V tile in LDS
  constexpr int RBK = Q8 ? D : RB;    // bytes per K row in LDS (int8 or 16-bit)
  constexpr int CPRK = RBK / 16;      // 16-byte chunks per K row
  constexpr int TBK = BC * RBK;       // one K tile in LDS (and one 8-bit V tile)
  // HBM -> LDS loads move 16 bytes per lane.  A tile smaller than one such
  // load per lane of the workgroup (8-bit tiles of 4 KiB over eight waves)
  // is loaded by its first LNW waves only.
  constexpr int LW = 16;
  constexpr int LNW = TBK / (64 * LW) < NW ? TBK / (64 * LW) : NW;  // waves that load K / V
  constexpr int LOADS = TBK / (LNW * 64 * LW);  // K loads per loading thread per tile (V: the same)
  // contraction depth of one first-product MFMA (16 bytes of codes per lane,
  // 32 for FP8, 8 16-bit values otherwise)
  constexpr int KD = F8 ? (MS == 16 ? 128 : 64) : Q8 ? (MS == 16 ? 64 : 32) : MS == 16 ? 32 : 16;
  constexpr int KS = D / KD;          // k-steps of the first product
  constexpr int KPM = MS == 32 ? 16 : 32;  // keys per second-product MFMA
  constexpr int ST = BC / KPM;        // k-steps of the second product
  constexpr int KB = BC / MS;         // MS-key blocks per tile
  constexpr int DB = D / MS;          // MS-dim blocks of the output
  constexpr int NACC = MS * MS / 64;  // accumulator registers per lane of one block
  static_assert(TBK % (LNW * 64 * LW) == 0, "tile must split into wave loads");
  static_assert(BC % 32 == 0 && D % 32 == 0, "MFMA blocking");
  // Q and O are bf16 or fp16; P and V meet on fp16 matrix instructions in the
  // INT8 kernels (V is widened exactly), on the input type otherwise.
  constexpr bool F16B = FP16 || Q8;
  using X8 = typename Vec<F16B>::x8;  // operands of the second product
  using X4 = typename Vec<FP16>::x4;
  using X2 = typename Vec<F16B>::x2;
  using E = typename Vec<FP16>::e;    // element type of Q and O
  using EP = typename Vec<F16B>::e;   // element type of P
  // A operand of the first product: 8 16-bit, 16 int8 or 32 FP8 values
  using KOp = std::conditional_t<F8, i32x8, std::conditional_t<Q8, i32x4, X8>>;
  using FAcc = std::conditional_t<MS == 32, f32x16, f32x4>;  // fp32 accumulator block
  using SAcc = std::conditional_t<Q8 && !F8, std::conditional_t<MS == 32, i32x16, i32x4>, FAcc>;  // the first product's

  constexpr int PK = C::PK;           // K operands read one iteration early
  constexpr int PV = C::PV;           // V operands read one iteration early
  constexpr int KO = KS * KB;         // K operands (A of the first product) per tile and wave
  constexpr int VO = ST * DB;         // V operands (A of the second product) per tile and wave
  constexpr int RING = C::RING;
  static_assert(RING == 4, "ring of four slots");
  static_assert(PK <= KO && PV <= VO, "prefetch depth");
  // V_t is loaded during iteration t - VAHEAD: as int8 into a staging ring
  // three iterations ahead (Q8; widened to fp16 during iteration t - 1), else
  // straight into the V ring.
  constexpr int VAHEAD = Q8 ? 3 : 2;
  // LDS: the K ring [RING][BC][D] at 0, the (16-bit) V ring at VBASE, and with
  // Q8 the int8 V staging ring at SBASE; tiles row-major, K and V swizzled.
  constexpr int VBASE = RING * TBK;
  constexpr int SBASE = VBASE + RING * TBYTES;
  constexpr int RING_BYTES = SBASE + (Q8 ? RING * TBK : 0);
  // After the loop the same LDS stages the output: each wave's MS*QB rows of
  // O, row-major, rows padded by 16 bytes (OROW) against bank conflicts.
  constexpr int OROW = D * 2 + 16;
  constexpr int OBYTES = NW * MS * QB * OROW;
  // PERSIST keeps the ring apart from a query / output area at QOBASE: the
  // next item's query tile is staged there while the current one runs, and
  // the output is staged there while the next item's first K/V tiles sit in
  // the ring.
  constexpr int QTB = BR * RB;  // one query tile
  static_assert(!PERSIST || (!Q8 && QB == 1), "persistent kernels");
  static_assert(!SPLIT || !PERSIST, "key splits");
  constexpr int QOBASE = PERSIST ? RING_BYTES : 0;
  constexpr int QOBYTES = QTB > OBYTES ? QTB : OBYTES;
  __shared__ __attribute__((aligned(16)))
  char smem[PERSIST ? RING_BYTES + QOBYTES
                    : (RING_BYTES > OBYTES ? RING_BYTES : OBYTES)];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  // The lane's query row within an MFMA block, and its k-group (the lanes of
  // one row: MS = 32, l and l + 32; MS = 16, l + 16 g for g = 0..3).
  const int lq = lane & (MS - 1);
  const int lg = lane / MS;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Work items are (K/V head bh = b * hkv + g, query tile qt) pairs, G =
  // n_groups of them.  All query tiles of one K/V head go to one XCD
  // (dispatch is round-robin over the 8 XCDs): the k-th workgroup on XCD x
  // takes logical item x*G/8 + k.  With the causal mask the later (longer)
  // query tiles start first.  A persistent workgroup (gridDim.x of them, a
  // multiple of 8, one per CU) takes items k, k + gridDim.x/8, ... of its XCD;
  // with the causal mask it takes pairs of query tiles of one K/V head,
  // q_tiles-1-i then i, whose key-tile counts always add up to the same.
  const int id = blockIdx.x;
  auto locate = [&](int r, int& bh_r, int& qt_r) -> bool {  // this workgroup's r-th item
    const int per_xcd = P.n_groups >> 3;
    if constexpr (PERSIST && CAUSAL) {
      const int half_tiles = P.q_tiles >> 1;
      const int x = id & 7, k = (id >> 3) + (r >> 1) * (int)(gridDim.x >> 3);
      if (2 * k >= per_xcd) return false;
      const int pair = x * (per_xcd >> 1) + k;
      bh_r = pair / half_tiles;
      const int pi = pair - bh_r * half_tiles;
      qt_r = (r & 1) ? pi : P.q_tiles - 1 - pi;
      return true;
    } else if constexpr (PERSIST) {
      const int x = id & 7, k = (id >> 3) + r * (int)(gridDim.x >> 3);
      if (k >= per_xcd) return false;
      const int logical = x * per_xcd + k;
      bh_r = logical / P.q_tiles;
      qt_r = logical - bh_r * P.q_tiles;
      return true;
    }
    if constexpr (SPLIT) {
      // the splits of one item are consecutive workgroups (on different
      // XCDs, reading different keys); with the causal mask the later
      // (longer) query tiles start first
      const int item = id / P.splits;
      bh_r = item / P.q_tiles;
      qt_r = item - bh_r * P.q_tiles;
      if constexpr (CAUSAL) qt_r = P.q_tiles - 1 - qt_r;
      return r == 0;
    }
    if ((P.n_groups & 7) == 0) {
      const int x = id & 7, kx = id >> 3;  // k-th workgroup dispatched on XCD x
      if (CAUSAL && per_xcd % P.q_tiles == 0) {
        // this XCD's heads, longest query tiles of all of them first
        const int heads = per_xcd / P.q_tiles;
        bh_r = x * heads + kx % heads;
        qt_r = P.q_tiles - 1 - kx / heads;
      } else {
        const int logical = x * per_xcd + kx;
        bh_r = logical / P.q_tiles;
        qt_r = logical - bh_r * P.q_tiles;
        if constexpr (CAUSAL) qt_r = P.q_tiles - 1 - qt_r;
      }
    } else {
      bh_r = id / P.q_tiles;
      qt_r = id - bh_r * P.q_tiles;
      if constexpr (CAUSAL) qt_r = P.q_tiles - 1 - qt_r;
    }
    return r == 0;
  };
  int bh = 0, qt = 0;
  if (!locate(0, bh, qt)) return;  // a persistent workgroup left without items
  constexpr int KE = Q8 ? 1 : 2;  // bytes per K / V element in HBM
  // Buffer descriptors of an item: its group's query rows, its K and V.
  auto q_words = [&](int bh_r) {
    return make_rsrc_words(P.q + (int64_t)bh_r * P.rows * D, (uint32_t)P.rows * D * 2);
  };
  auto k_words = [&](int bh_r) {
    return make_rsrc_words(P.k + (int64_t)bh_r * N * D * KE, (uint32_t)N * D * KE);
  };
  auto v_words = [&](int bh_r) {
    return make_rsrc_words(P.v + (int64_t)bh_r * N * D * KE, (uint32_t)N * D * KE);
  };
  int64_t q_head = (int64_t)bh * P.rows * D;  // the group's first query row
  __amdgpu_buffer_rsrc_t q_rs = make_rsrc(P.q + q_head, (uint32_t)P.rows * D * 2);
  i32x4 k_rs = k_words(bh);
  i32x4 v_rs = v_words(bh);
  // PERSIST: the next item (if any), whose query tile and first K/V tiles
  // are loaded during this item's iterations; nx_delta is the byte distance
  // from this item's K (and V) head to the next one's.  Without a next item
  // those loads fetch this item's own tiles again, unused.
  int bh_nx = 0, qt_nx = 0;
  bool has_next = false;
  int64_t nx_delta = 0;
  auto look_ahead = [&](int r) {
    has_next = locate(r + 1, bh_nx, qt_nx);
    if (!has_next) {
      bh_nx = bh;
      qt_nx = qt;
    }
    nx_delta = (int64_t)(bh_nx - bh) * N * D * KE;
  };
  // The descriptor rs with its base moved by `delta` bytes.
  auto rebase = [](i32x4 rs, int64_t delta) {
    const uint64_t b = ((uint64_t)((uint32_t)rs[1] & 0xffffu) << 32 | (uint32_t)rs[0]) + (uint64_t)delta;
    rs[0] = (int)(uint32_t)b;
    rs[1] = (int)((uint32_t)(b >> 32) & 0xffffu);
    return rs;
  };
  if constexpr (PERSIST) look_ahead(0);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Global -> LDS without registers: each wave load moves 64 lanes x 16 bytes
  // (lane l to byte 16*l of its piece).  The swizzles (on 16-byte chunks) are
  // applied on the global side: a lane fetches the bytes that belong at its
  // LDS position.  With Q8 the 8-bit V tile is staged unswizzled.  Rows past N
  // read as zeros (buffer range check); their keys are masked later.
  uint32_t k_src[LOADS], v_src[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = ((i * LNW + wave) * 64 + lane) * LW;  // byte in the LDS tile (wave < LNW)
    const int row = pos / RBK, pc = (pos % RBK) / 16;
    k_src[i] = (uint32_t)(row * RBK + k_swizzle<CPRK>(row, pc) * 16);
    v_src[i] = Q8 ? (uint32_t)pos : (uint32_t)(row * RB + v_swizzle<CPR, MS>(row, pc) * 16);
  }
  // `s` (an integral constant) is t modulo 4, known at compile time in the
  // loop (unrolled by 4), so the ring slot t % RING and its LDS offsets fold
  // into instruction immediates.
  auto slot = [](int, auto s) { return decltype(s)::value % RING; };
  // Tiles past the last one read as zeros (buffer range check) and are never
  // used; loading them keeps the per-iteration load count fixed.
  // PERSIST: with `nx` (a compile-time flag) tile t is tile t - n_cur of
  // the next item, n_cur being the current item's key-tile count.
  int n_cur = (N + BC - 1) / BC;
  auto issue_k = [&](int t, auto s, auto nx) {
    const uint32_t dst = lds_base + slot(t, s) * TBK + wave * 64 * LW;
    i32x4 rs = k_rs;
    if constexpr (decltype(nx)::value) {
      rs = rebase(k_rs, nx_delta);
      t -= n_cur;
    }
    if (LNW == NW || wave < LNW)
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        load_lds16(rs, (uint32_t)t * TBK + k_src[i], dst + i * LNW * 64 * LW);
  };
  // V_t into the V ring, or with Q8 into the int8 staging ring.
  auto issue_v = [&](int t, auto s, auto nx) {
    const uint32_t dst = lds_base + (Q8 ? SBASE + slot(t, s) * TBK : VBASE + slot(t, s) * TBYTES) +
                         wave * 64 * LW;
    i32x4 rs = v_rs;
    if constexpr (decltype(nx)::value) {
      rs = rebase(v_rs, nx_delta);
      t -= n_cur;
    }
    if (LNW == NW || wave < LNW)
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        load_lds16(rs, (uint32_t)t * TBK + v_src[i], dst + i * LNW * 64 * LW);
  };
  // PERSIST: query tile qt_r of the group that descriptor rs covers into the
  // query / output area, swizzled like K (QLOADS 16-byte loads per thread).
  // Load i moves the pieces (i*NW + wave)*64 + lane, rows 16 apart or more
  // from load i-1, so the swizzle (row & 15) is that of load 0.
  constexpr int QLOADS = QTB / (NW * 64 * 16);
  constexpr int QSTEP = NW * 64 * 16;  // bytes of the tile per load
  static_assert(!PERSIST || (QTB % QSTEP == 0 && QSTEP % (16 * RB) == 0), "query tile loads");
  auto issue_q = [&](const i32x4& rs, int qt_r) {
    if constexpr (PERSIST) {
      // recomputed per item rather than held in registers through the loop
      int ln = lane;
      uint32_t dst = lds_base + QOBASE + wave * 1024;
      asm volatile("" : "+v"(ln), "+s"(dst));
      const int lin = wave * 64 + ln, row = lin / CPR;
      // unsigned: a group's query rows may span up to 2^32 - 2^21 bytes
      const uint32_t src = (uint32_t)qt_r * QTB + (uint32_t)(row * RB + k_swizzle<CPR>(row, lin % CPR) * 16);
#pragma unroll
      for (int i = 0; i < QLOADS; ++i) load_lds16(rs, src + i * QSTEP, dst + i * QSTEP);
    }
  };

  // Per-lane LDS byte offsets of the MFMA operands within a tile.  The
  // swizzle term depends only on the lane (row bits below the MS-row block),
  // so every other index becomes an instruction immediate.
  //   K (A operand of S^T): row kb*MS + lq, logical chunk ks*KCH + lg (FP8:
  //   the two chunks ks*KCH + 2 lg and ks*KCH + 2 lg + 1).
  //   V^T (A operand of O^T), via ds_read_b64_tr_b16 (in each 16-lane group
  //   lane i receives element i%4 of the 8-byte pieces that lanes i/4,
  //   4+i/4, 8+i/4, 12+i/4 address).  MS = 32: the 16-lane group g reads rows
  //   st*16 + sg*8 + half*4 + (lane%16)/4 and 4 elements at column
  //   db*32 + 16*(g&1) + 4*(lane%4); lane l then holds V[key][db*32 + l32] for
  //   keys st*16 + sg*8 + half*4 + 0..3.  MS = 16: group g reads rows
  //   st*32 + sg*16 + 4g + (lane%16)/4 at column db*16 + 4*(lane%4); lane l
  //   then holds V[key][db*16 + lq] for keys st*32 + sg*16 + 4g + 0..3.
  //   Either way these are the keys whose probabilities the lane holds in
  //   the matching slots of its B operand (the S^T accumulator layout).
  // The swizzles touch only the low 4 bits of a chunk index, so offsets
  // repeat every 16 chunks (256 B) along a row: keep one K offset per k-step
  // and one V offset per output block within 256 B, and reach the rest with
  // an immediate.  The V offsets include the V ring's base and are opaque to
  // the compiler, so that the immediate of an LDS read (16 bits) only has to
  // hold the slot and the rows: at d = 256 the V ring starts at 64 KiB.
  constexpr int KCH = KD * (Q8 ? 1 : 2) / 16;  // 16-byte chunks of a K row per k-step
  constexpr int KPB = 16 / KCH;       // first-product k-steps per 256 B of a row
  constexpr int KOFF = KS < KPB ? KS : KPB;
  constexpr int VPB = 128 / MS;       // output blocks per 256 B of a row
  constexpr int VOFF = DB < VPB ? DB : VPB;
  uint32_t k_off[KOFF], k_off2[F8 ? KOFF : 1];
#pragma unroll
  for (int ks = 0; ks < KOFF; ++ks) {
    const int ch = F8 ? ks * KCH + 2 * lg : ks * KCH + lg;
    k_off[ks] = (uint32_t)(lq * RBK + k_swizzle<CPRK>(lq, ch) * 16);
    if constexpr (F8) k_off2[ks] = (uint32_t)(lq * RBK + k_swizzle<CPRK>(lq, ch + 1) * 16);
  }
  const int tr_row = MS == 32 ? half * 4 + ((lane & 15) >> 2) : 4 * lg + ((lane & 15) >> 2);
  const int tr_col = MS == 32 ? 16 * ((lane >> 4) & 1) + 4 * (lane & 3) : 4 * (lane & 3);
  uint32_t v_off[VOFF];
#pragma unroll
  for (int db = 0; db < VOFF; ++db) {
    const int col = db * MS + tr_col;
    v_off[db] = (uint32_t)(VBASE + tr_row * RB + v_swizzle<CPR, MS>(tr_row, col >> 3) * 16 +
                           (col & 7) * 2);
    asm volatile("" : "+v"(v_off[db]));
  }

  // Q_i fragments: the B operands of S^T = K_j Q_i^T, held for the whole
  // loop.  Query block b of this wave is packed rows q0 + MS*b + lq.
  int q0 = qt * BR + wave * MS * QB;

  // Limits of the current item (recomputed for each item of a persistent
  // workgroup).  Causal: a lane's last visible key (its row within its head
  // plus causal_off), and the smallest such row among the wave's rows (packed
  // rows wrap to 0 at a head boundary); the last key tile any row of the wave
  // sees (-1: none), from its largest row within a head (nq - 1 if its rows
  // wrap to the next head).  n_tiles: the key tiles this workgroup needs, all
  // of them or with the causal mask those up to the last key its rows see (a
  // workgroup whose rows see no key writes O = 0 and lse = -inf).  n_clear:
  // the leading tiles that no wave of the workgroup masks, whole tiles of keys
  // and with the causal mask those whose last key every row of the workgroup
  // sees (its smallest row within a head; 0 if it spans a head boundary).
  // SPLIT: the workgroup takes the key tiles [lo, hi) of its item's n_tiles
  // (split id % splits of `splits` near-equal shares); key_base = lo * BC is
  // its first key, and tile counts and wave_last become relative to lo.
  int row_lim[QB];
  int wave_row_min = 0, wave_last = 0, n_tiles = 0, n_clear = 0, key_base = 0;
  auto item_limits = [&]() {
    if constexpr (CAUSAL) {
      const int r0 = q0 % P.nq;
#pragma unroll
      for (int b = 0; b < QB; ++b) row_lim[b] = (q0 + MS * b + lq) % P.nq + P.causal_off;
      wave_row_min = r0 + MS * QB - 1 < P.nq ? r0 : 0;
      const int row_max = r0 + MS * QB - 1 < P.nq ? r0 + MS * QB - 1 : P.nq - 1;
      const int last_key = min(row_max + P.causal_off, N - 1);
      wave_last = last_key < 0 ? -1 : last_key / BC;
    }
    n_tiles = (N + BC - 1) / BC;
    n_clear = N / BC;
    if constexpr (CAUSAL) {
      const int first = qt * BR, last = min(P.rows, first + BR) - 1;
      const bool spans = first / P.nq != last / P.nq;
      const int row_max = spans ? P.nq - 1 : last % P.nq;
      const int last_key = row_max + P.causal_off;  // may be < 0
      n_tiles = last_key < 0 ? 0 : min(n_tiles, last_key / BC + 1);
      const int row_min = spans ? 0 : first % P.nq;
      const int seen = row_min + P.causal_off + 1;  // keys every row sees
      n_clear = seen <= 0 ? 0 : min(n_clear, seen / BC);
    }
    if constexpr (SPLIT) {
      const int sp = id % P.splits;
      const int lo = (int)((int64_t)n_tiles * sp / P.splits);
      const int hi = (int)((int64_t)n_tiles * (sp + 1) / P.splits);
      key_base = lo * BC;
      n_clear = max(0, min(n_clear, hi) - lo);
      if constexpr (CAUSAL) wave_last -= lo;
      n_tiles = hi - lo;
    }
    n_cur = n_tiles;
  };
  // Causal: whether any row of this wave sees a key of tile t (always true
  // without the mask).
  // SKIP (the key-split kernels, and the 16-bit d = 256 ones): a wave whose
  // query rows all lie past the item's last row (the padding of a short
  // query block: decoding fills one of four waves) runs neither product and
  // reads no operands; it still issues its share of the loads, widens its
  // share of V and meets every barrier.  Its logits stay 0 (set once below),
  // so its softmax is cheap and never takes the rare path after the first
  // tile; its rows are never written.  (The other kernels compute such waves:
  // the check cost them 5-12% in register allocation at 254-256 VGPRs.)
  constexpr bool SKIP = SPLIT || (D == 256 && !Q8 && !PERSIST);
  const bool live = !SKIP || q0 < P.rows;
  auto sees = [&](int t) -> bool { return live && (!CAUSAL || t <= wave_last); };
  item_limits();
  if constexpr (SPLIT) {
    // K and V from the split's first key on; key_base < N unless there are
    // no tiles at all (then 0), so the range stays within the head
    const int64_t off = ((int64_t)bh * N + key_base) * D * KE;
    const uint32_t len = (uint32_t)(N - key_base) * D * KE;
    k_rs = make_rsrc_words(P.k + off, len);
    v_rs = make_rsrc_words(P.v + off, len);
  }
  // c_q: the lane's logit multiplier (scale * log2 e, times the query row
  // scale with Q8).
  using QOp = KOp;
  QOp qf[QB][KS];
  float c_q[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    c_q[b] = c;
    const uint32_t qrow_off = (uint32_t)(q0 + MS * b + lq) * RB;  // unsigned, as above
    if constexpr (PERSIST) {
      // fragments come through LDS (load_qf below)
    } else if constexpr (!Q8) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[b][ks] = __builtin_bit_cast(
            X8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, qrow_off + (ks * KD + lg * 8) * 2, 0, 0));
    } else if constexpr (F8 && MODE != kZero) {
      // In-kernel quantization of the query row to E4M3 (the lanes of a row,
      // k-group lg = lane / MS, hold its parts): for k-step ks this lane
      // holds channels KD ks + 32 lg + 0..31.  u = q * ks in binary32; amax
      // over the row; codes e4m3_rne(u * (448 / amax)) and sq = amax / 448,
      // both divisions correctly rounded (a zero row: codes 0, sq 0).
      using Q16 = typename Vec<FP16>::x8;
      const float* ksp = P.ks + (int64_t)bh * D;
      float u[KS][32];
      float amax = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int h4 = 0; h4 < 4; ++h4) {
          const int ch = KD * ks + 32 * lg + 8 * h4;
          const Q16 qv = __builtin_bit_cast(
              Q16, __builtin_amdgcn_raw_buffer_load_b128(q_rs, qrow_off + ch * 2, 0, 0));
          const float4 s0 = *(const float4*)(ksp + ch);
          const float4 s1 = *(const float4*)(ksp + ch + 4);
          const float sk[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = (float)qv[e] * sk[e];
            u[ks][8 * h4 + e] = v;
            amax = fmaxf(amax, fabsf(v));
          }
        }
      }
      if constexpr (MS == 16) amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, other_half(amax, lane));
      const bool nonzero = amax > 0.0f;
      const float to448 = nonzero ? __fdiv_rn(448.0f, amax) : 0.0f;
      const float sq = nonzero ? __fdiv_rn(amax, 448.0f) : 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        i32x8 w;
#pragma unroll
        for (int k4 = 0; k4 < 8; ++k4) {
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) packed |= e4m3_rne(u[ks][4 * k4 + e] * to448) << (8 * e);
          w[k4] = (int)packed;
        }
        qf[b][ks] = w;
      }
      const float cq = c * sq;
      c_q[b] = cq != 0.0f ? cq : (MODE == kNegative ? -FLT_MIN : FLT_MIN);
    } else if constexpr (MODE != kZero) {
      // In-kernel quantization of the query row (the lanes of a row, k-group
      // lg = lane / MS, hold its parts): for k-step ks this lane holds
      // channels KD ks + 16 lg + 0..15.  u = q * ks in binary32; amax over the row; codes
      // clamp(rint(u * (127 / amax)), +-127) and sq = amax / 127, both
      // divisions correctly rounded (a zero row: codes 0, sq 0).
      using Q16 = typename Vec<FP16>::x8;
      const float* ksp = P.ks + (int64_t)bh * D;
      float u[KS][16];
      float amax = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = KD * ks + 16 * lg;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const Q16 qv = __builtin_bit_cast(
              Q16, __builtin_amdgcn_raw_buffer_load_b128(q_rs, qrow_off + (ch + 8 * h2) * 2, 0, 0));
          const float4 s0 = *(const float4*)(ksp + ch + 8 * h2);
          const float4 s1 = *(const float4*)(ksp + ch + 8 * h2 + 4);
          const float sk[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = (float)qv[e] * sk[e];
            u[ks][8 * h2 + e] = v;
            amax = fmaxf(amax, fabsf(v));
          }
        }
      }
      if constexpr (MS == 16) amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, other_half(amax, lane));
      const bool nonzero = amax > 0.0f;
      const float inv = nonzero ? __fdiv_rn(127.0f, amax) : 0.0f;
      const float sq = nonzero ? __fdiv_rn(amax, 127.0f) : 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        i32x4 w;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float code = fminf(fmaxf(__builtin_rintf(u[ks][4 * k4 + e] * inv), -127.0f), 127.0f);
            packed |= ((uint32_t)(int)code & 0xFFu) << (8 * e);
          }
          w[k4] = (int)packed;
        }
        qf[b][ks] = w;
      }
      // A zero (or underflowing) multiplier would turn the -inf of masked keys
      // into NaN; the smallest normal keeps every unmasked logit at 0 instead.
      const float cq = c * sq;
      c_q[b] = cq != 0.0f ? cq : (MODE == kNegative ? -FLT_MIN : FLT_MIN);
    }
  }

  FAcc acc[QB][DB];
  float m_ref[QB], l_part[QB];  // reference max (log2 units), lane's row sum
#pragma unroll
  for (int b = 0; b < QB; ++b) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < NACC; ++i) acc[b][db][i] = 0.0f;
    m_ref[b] = -INFINITY;
    l_part[b] = 0.0f;
  }

  // PERSIST: this wave's query fragments from the query tile in LDS, at the
  // K operand offsets (the tile is swizzled like K and the wave's rows start
  // at a multiple of 32).  The wave's base is made opaque here so that the
  // compiler does not keep every offset plus base in a register between uses.
  auto load_qf = [&]() {
    if constexpr (PERSIST) {
      uint32_t qbase = QOBASE + wave * 32 * QB * RB;
      asm volatile("" : "+s"(qbase));
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qf[b][ks] = __builtin_bit_cast(
              X8, *(const __attribute__((address_space(3))) u32x4*)(
                      lds + qbase + 32 * b * RB + k_off[ks % KOFF] + (ks / KOFF) * 256));
    }
  };

  // First operands of the next products, read one iteration early.
  KOp kpre[PK > 0 ? PK : 1];
  X8 vpre[PV > 0 ? PV : 1];

  // Operand o of the first product, o = ks*KB + kk: rows kk*MS .. +MS-1 of
  // K_t (k-step ks), as the A operand of S^T = K_t Q_i^T.
  auto k_operand = [&](int t, auto s, int o) -> KOp {
    const int ks = o / KB, kk = o % KB;
    const lds_char* kb = lds + slot(t, s) * TBK;
    const u32x4 a = *(const __attribute__((address_space(3))) u32x4*)(
        kb + kk * MS * RBK + k_off[ks % KOFF] + (ks / KOFF) * 256);
    if constexpr (F8) {
      const u32x4 b = *(const __attribute__((address_space(3))) u32x4*)(
          kb + kk * MS * RBK + k_off2[ks % KOFF] + (ks / KOFF) * 256);
      return __builtin_bit_cast(KOp, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return __builtin_bit_cast(KOp, a);
    }
  };
  // Operand o of the second product, o = st*DB + db: V_t^T for output rows
  // db*MS .. +MS-1 and keys st*KPM .. +KPM-1 in the S^T accumulator's key
  // order, from the row-major V tile through two transposing LDS reads of 4
  // keys.
  auto v_operand = [&](int t, auto s, int o) -> X8 {
    const int st = o / DB, db = o % DB;
    const lds_char* vb = lds + slot(t, s) * TBYTES;  // v_off holds VBASE
    const uint32_t vo = v_off[db % VOFF] + (db / VOFF) * 256;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vb + vo + (st * KPM) * RB));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vb + vo + (st * KPM + KPM / 2) * RB));
    return __builtin_bit_cast(X8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T_t = K_t Q_i^T : [BC keys] x [MS queries] per wave.  The first PK
  // operands come from `pre` (read during the previous iteration), the rest
  // from LDS.  With a zero scale every logit is 0 whatever Q and K hold, so S
  // stays 0 and c is taken as 1 (x = s - m_ref keeps masked keys at -inf).
  auto gemm1 = [&](int t, auto s, const KOp (&pre)[PK > 0 ? PK : 1], SAcc (&sd)[QB][KB]) {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int i = 0; i < NACC; ++i) sd[b][kk][i] = 0;
    if constexpr (MODE == kZero) return;
#pragma unroll
    for (int o = 0; o < KO; ++o) {
      const KOp a = o < PK ? pre[o < PK ? o : 0] : k_operand(t, s, o);
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        if constexpr (F8 && MS == 32)  // E4M3 x E4M3 (format 0 for both operands), fp32 sums, no block scales
          sd[b][o % KB] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[b][o / KB], sd[b][o % KB],
                                                                          0, 0, 0, 0, 0, 0);
        else if constexpr (F8)
          sd[b][o % KB] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qf[b][o / KB], sd[b][o % KB],
                                                                           0, 0, 0, 0, 0, 0);
        else if constexpr (Q8 && MS == 32)  // exact int32 dot products of the codes
          sd[b][o % KB] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[b][o / KB], sd[b][o % KB], 0, 0, 0);
        else if constexpr (Q8)
          sd[b][o % KB] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qf[b][o / KB], sd[b][o % KB], 0, 0, 0);
        else if constexpr (MS == 32)
          sd[b][o % KB] = mfma32x32x16<FP16>(a, qf[b][o / KB], sd[b][o % KB]);
        else
          sd[b][o % KB] = mfma16x16x32<FP16>(a, qf[b][o / KB], sd[b][o % KB]);
      }
    }
  };

  // O^T += V_t^T P_t^T : [D] x [MS queries] per wave; the first PV operands
  // come from `pre`.
  auto gemm2 = [&](int t, auto s, const X8 (&pre)[PV > 0 ? PV : 1], const X8 (&pf)[QB][ST]) {
#pragma unroll
    for (int o = 0; o < VO; ++o) {
      const X8 a = o < PV ? pre[o < PV ? o : 0] : v_operand(t, s, o);
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        if constexpr (MS == 32)
          acc[b][o % DB] = mfma32x32x16<F16B>(a, pf[b][o / DB], acc[b][o % DB]);
        else
          acc[b][o % DB] = mfma16x16x32<F16B>(a, pf[b][o / DB], acc[b][o % DB]);
      }
    }
  };

  // The first PK / PV operands of the next iteration's products.
  auto prefetch_k = [&](int t, auto s, KOp (&pre)[PK > 0 ? PK : 1]) {
    if constexpr (MODE == kZero) return;
#pragma unroll
    for (int o = 0; o < PK; ++o) pre[o] = k_operand(t, s, o);
  };
  auto prefetch_v = [&](int t, auto s, X8 (&pre)[PV > 0 ? PV : 1]) {
#pragma unroll
    for (int o = 0; o < PV; ++o) pre[o] = v_operand(t, s, o);
  };

  // Q8: widen V_t from its 8-bit staging slot into the 16-bit V ring as exact
  // fp16.  Each thread writes whole 16-byte chunks of the swizzled tile from
  // the 8 codes of the logical chunk that belongs there.  int8: with u =
  // code + 128 (the byte xor 0x80), the fp16 pattern 0x6400 | u is 1024 + u,
  // and subtracting 1152 leaves the code.  FP8: every E4M3 value is an fp16
  // value; the conversion instruction takes two codes at a time (scale 1).
  auto convert_v = [&](int t, auto s) {
    if constexpr (Q8) {
      using h16x8 = _Float16 __attribute__((ext_vector_type(8)));
      constexpr int CH = TBYTES / 16;  // 16-byte fp16 chunks per tile
      static_assert(CH % (NW * 64) == 0, "whole chunks per thread");
#pragma unroll
      for (int i = 0; i < CH / (NW * 64); ++i) {
        const int lin = i * NW * 64 + tid;
        const int row = lin / CPR, pc = lin % CPR;
        const int lc = v_swizzle<CPR, MS>(row, pc);
        const u32x2 codes = *(const __attribute__((address_space(3))) u32x2*)(
            lds + SBASE + slot(t, s) * TBK + row * D + lc * 8);
        u32x4 w;
        h16x8 v;
        if constexpr (F8) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            w[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[h], 1.0f, false));
            w[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes[h], 1.0f, true));
          }
          v = __builtin_bit_cast(h16x8, w);
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t biased = codes[h] ^ 0x80808080u;
            w[2 * h] = __builtin_amdgcn_perm(0x64646464u, biased, 0x04010400u);
            w[2 * h + 1] = __builtin_amdgcn_perm(0x64646464u, biased, 0x04030402u);
          }
          v = __builtin_bit_cast(h16x8, w) - (_Float16)1152.0f;
        }
        *(__attribute__((address_space(3))) u32x4*)(lds + VBASE + slot(t, s) * TBYTES + lin * 16) =
            __builtin_bit_cast(u32x4, v);
      }
    }
  };

  // Reductions over the lanes that hold one query row; the exchange of the
  // two 32-lane halves is one v_permlane32_swap (no LDS round trip).
  auto row_max = [&](float x) -> float {
    if constexpr (MS == 16) x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, other_half(x, lane));
  };
  auto row_sum = [&](float x) -> float {
    if constexpr (MS == 16) x += __shfl_xor(x, 16);
    return x + other_half(x, lane);
  };

  // P_t^T as the B operands of the second product.  MS = 32: k-step st
  // takes keys 16 st .. +15, this lane's 8 of them the accumulator elements
  // 8 (st % 2) .. +7 of key block st / 2.  MS = 16: k-step st takes key
  // blocks 2 st and 2 st + 1, this lane's 4 keys of each.
  auto probs = [&](const FAcc (&sc)[KB], X8 (&pf)[ST], float m, float cl) -> float {
    // A causal row that has seen no key yet has m = -inf and only masked
    // logits; reference 0 gives them p = 0 rather than NaN.
    if constexpr (CAUSAL) m = m == -INFINITY ? 0.0f : m;
    float rs = 0.0f;
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = MS == 32 ? st >> 1 : 2 * st + (e >> 1);
        const int i0 = MS == 32 ? (st & 1) * 8 + 2 * e : 2 * (e & 1);
        const float x0 = __builtin_fmaf(sc[kb][i0], cl, -m);
        const float x1 = __builtin_fmaf(sc[kb][i0 + 1], cl, -m);
        const float p0 = __builtin_amdgcn_exp2f(x0);
        const float p1 = __builtin_amdgcn_exp2f(x1);
        rs += p0;
        rs += p1;
        const X2 pair = {(EP)p0, (EP)p1};
        w[e] = __builtin_bit_cast(uint32_t, pair);
      }
      pf[st] = __builtin_bit_cast(X8, w);
    }
    return rs;
  };

  // One iteration j, as a single straight-line block for the scheduler:
  // S_{j+1} = K_{j+1} Q^T and O += P_{j-1} V_{j-1} on the matrix cores while
  // the VALU turns S_j into P_j.  The loads issued here are K_{j+RING} and
  // V_{j+VAHEAD}; each goes to the ring slot whose previous tile (K_j;
  // V_{j-2}, or the int8 V_{j-1} widened during iteration j-2) was last read
  // before the barrier that ended iteration j-1.  With Q8 the iteration also
  // widens V_{j+1} (staged during iteration j-2) into its slot of the V ring,
  // whose previous tile V_{j-3} was last read in iteration j-2.
  // With RING = 4 the iteration then reads the first operands of iteration
  // j+1 (K_{j+2}, V_j: loaded during iteration j-2 and published by the last
  // barrier) and waits only for the loads issued during iteration j-1.  The
  // last iteration's S_{j+1} product reads a tile past the end and is
  // dropped.  `ph` is j % 4.  `tail` (compile-time): bit 3, no wave masks
  // this tile (the check, a branch that splits the block, is left out).
  // PERSIST marks the last iterations of an item with bit 0, the K tile
  // loaded is the next item's; bit 1, the V tile; bit 2, S_{j+1} is the next
  // item's S_0 (its query fragments are read first).
  auto step = [&](auto first, auto ph, int j, SAcc (&s_cur)[QB][KB], SAcc (&s_nxt)[QB][KB],
                  const X8 (&p_prev)[QB][ST], X8 (&p_cur)[QB][ST], auto tail) {
    constexpr int p = decltype(ph)::value;
    constexpr int TL = decltype(tail)::value;
    using S0 = Ic<p>;
    using S1 = Ic<(p + 1) % 4>;
    using S2 = Ic<(p + 2) % 4>;
    using S3 = Ic<(p + 3) % 4>;
    issue_k(j + RING, S0{}, std::bool_constant<(TL & 1) != 0>{});
    issue_v(j + VAHEAD, Ic<(p + VAHEAD) % 4>{}, std::bool_constant<(TL & 2) != 0>{});
    convert_v(j + 1, S1{});
    // PERSIST: the next item's query tile, needed by this item's last product
    // (issued after this iteration's K/V loads, also when there is no next
    // item, so that the wait below counts it; waited by the next iteration)
    if constexpr (PERSIST && decltype(first)::value) issue_q(q_words(bh_nx), qt_nx);
    if constexpr (kSyncCheck) {
      wait_vmem();
      __syncthreads();
    }

    // The logits of this tile in fp32 (converted from the int32 products
    // of the INT8 cache; the FP8 products are fp32 already).
    constexpr bool CONV = Q8 && !F8;
    FAcc s_conv[CONV ? QB : 1][CONV ? KB : 1];
    if constexpr (CONV) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int i = 0; i < NACC; ++i) s_conv[b][kk][i] = (float)s_cur[b][kk][i];
    }
    auto& sf = [&]() -> auto& {
      if constexpr (CONV)
        return s_conv;
      else
        return s_cur;
    }();

    // Mask keys past N and, with the causal option, keys past a row's
    // diagonal (key > row + causal_off).  Decided per wave, from its
    // smallest row within a head.
    const int key0 = j * BC + (SPLIT ? key_base : 0);
    bool masked = false;
    if constexpr ((TL & 8) == 0) {
      masked = key0 + BC > N;
      if constexpr (CAUSAL) masked |= key0 + BC - 1 > wave_row_min + P.causal_off;
    }
    if (masked) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int lim = CAUSAL ? min(N - 1, row_lim[b]) : N - 1;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int i = 0; i < NACC; ++i) {
            const int key = MS == 32 ? key0 + kk * 32 + (i >> 2) * 8 + half * 4 + (i & 3)
                                     : key0 + kk * 16 + lg * 4 + i;
            if (key > lim) sf[b][kk][i] = MODE == kNegative ? INFINITY : -INFINITY;
          }
      }
    }

    // PERSIST: the last iteration's S_{j+1} is the next item's S_0, against
    // its query tile (landed by the end of iteration 1).
    if constexpr ((TL & 4) != 0) load_qf();
    // Causal, past the diagonal: a wave whose rows see no key of tile j+1
    // skips S_{j+1}, and one whose rows saw no key of tile j-1 skips its P V
    // product (P is 0), leaving the MFMA pipe of its SIMD to the other wave.
    // The stale S registers are never used: the next iteration masks every
    // key of that tile for this wave (to -inf, so P is 0), as it would the
    // computed logits.
    if (((TL & 8) != 0 || (TL & 4) != 0 || sees(j + 1)) && live) gemm1(j + 1, S1{}, kpre, s_nxt);
    if constexpr (!decltype(first)::value) {
      if (((TL & 8) != 0 || sees(j - 1)) && live) gemm2(j - 1, S3{}, vpre, p_prev);
    }
    float rs[QB];
    bool over = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      if constexpr (decltype(first)::value) {
        // The first tile: every reference is still -inf, so every row takes
        // the path below, which forms the probabilities.
        rs[b] = INFINITY;
        over = true;
      } else {
        rs[b] = probs(sf[b], p_cur[b], m_ref[b], c_q[b]);
        over |= !(rs[b] <= kSumLimit);  // also true for inf / NaN
        // Causal rows that see no key keep m_ref = -inf; they take the rare
        // path, which leaves their p at 0.
        if constexpr (CAUSAL) over |= m_ref[b] == -INFINITY;
      }
    }
    constexpr int MF = QB * ((MODE == kZero ? 0 : KO) + (decltype(first)::value ? 0 : VO));
#pragma unroll
    for (int t = 0; t < (C::SGB ? MF : 0); ++t) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }

    // First operands of the next iteration: K_{j+2} and V_j, both published
    // by the barrier that ended the previous iteration.
    if (live) {
      prefetch_k(j + 2, S2{}, kpre);
      prefetch_v(j, S0{}, vpre);
    }

    // While the unrounded sum of a lane's p stays at or below kSumLimit no p
    // exceeds it and the reference max stands.  Otherwise (always on the
    // first tile, where no reference exists yet) rows whose sum outgrew the
    // limit move their reference to their running max, rescale O and l, and
    // get their p recomputed; other rows keep their reference, so a row's
    // arithmetic never depends on its wave-mates.
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        float ext = sf[b][0][0];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int i = 0; i < NACC; ++i)
            ext = MODE == kNegative ? fminf(ext, sf[b][kk][i]) : fmaxf(ext, sf[b][kk][i]);
        const float t_max = __builtin_isfinite(ext) ? ext * c_q[b] : -INFINITY;
        const float t_row = row_max(t_max);
        const float mine = !(rs[b] <= kSumLimit) ? 1.0f : 0.0f;
        // a row still at -inf takes its first reference from any visible key
        const bool move = row_max(mine) > 0.0f || m_ref[b] == -INFINITY;
        const float m_new = move ? fmaxf(m_ref[b], t_row) : m_ref[b];
        const float alpha =
            m_new == m_ref[b] ? 1.0f : __builtin_amdgcn_exp2f(m_ref[b] - m_new);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < NACC; ++i) acc[b][db][i] *= alpha;
        l_part[b] *= alpha;
        m_ref[b] = m_new;
        rs[b] = probs(sf[b], p_cur[b], m_ref[b], c_q[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) l_part[b] += rs[b];

    // The loads issued during iteration j-1 have landed (waves past LNW have
    // none in flight: LNW < NW only with 8-bit tiles, never persistent, so
    // such a wave issues no query loads either).  (PERSIST: the first
    // iteration's query loads may stay in flight too.)
    if constexpr (kSyncCheck)
      wait_vmem();
    else
      wait_vmem_but<2 * LOADS + (PERSIST && decltype(first)::value ? QLOADS : 0)>();
    __syncthreads();
  };

  // Both products' S and P register sets; with PERSIST they carry the next
  // item's S_0 from one item into the next.
  SAcc sA[QB][KB], sB[QB][KB];
  X8 pA[QB][ST], pB[QB][ST];
  if constexpr (SKIP) {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int i = 0; i < NACC; ++i) sA[b][kk][i] = sB[b][kk][i] = 0;
  }
  if (n_tiles > 0) {
    // Prologue: Q, K_0 .. K_{RING-1} and V_0 .. V_{RING-3} resident, S_0
    // computed, the first operands of K_1 in registers.  Everything retires
    // before the loop: vmcnt is a counter, so a load still in flight at the
    // loop head would make every iteration wait on it.  (Later persistent
    // items find all of this done by the item before.)
    issue_q(q_words(bh), qt);
    issue_k(0, Ic<0>{}, std::false_type{});
    issue_k(1, Ic<1>{}, std::false_type{});
    issue_k(2, Ic<2>{}, std::false_type{});
    issue_k(3, Ic<3>{}, std::false_type{});
    issue_v(0, Ic<0>{}, std::false_type{});
    issue_v(1, Ic<1>{}, std::false_type{});
    if constexpr (VAHEAD > 2) issue_v(2, Ic<2>{}, std::false_type{});
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (F8) {  // 8 registers: one operand each (the constraint takes at most 128 bits)
#pragma unroll
          for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(qf[b][ks][e]));
        } else {
          asm volatile("" ::"v"(qf[b][ks]));
        }
      }
    wait_vmem();
    __syncthreads();

    load_qf();              // PERSIST: Q from LDS (read before the next tile lands there)
    convert_v(0, Ic<0>{});  // Q8: V_0 widened; published by the barrier below
    if (live) {
      prefetch_k(0, Ic<0>{}, kpre);
      gemm1(0, Ic<0>{}, kpre, sA);
      prefetch_k(1, Ic<1>{}, kpre);
    }
    __syncthreads();  // every wave is done with K_0 before K_RING may overwrite it
  }

  for (int item = 0;; ++item) {
  if (n_tiles > 0) {

    // Iterations run in groups of 4 so ring slots and the S / P register
    // sets (even j: S_j in sA, S_{j+1} into sB, P_j into pA) are compile-time.
    step(std::true_type{}, Ic<0>{}, 0, sA, sB, pB, pA, Ic<PERSIST && !CAUSAL ? 8 : 0>{});
    int j = 1;
    if constexpr (PERSIST) {
      // n_tiles % 4 == 0 and n_tiles >= 8: the loop leaves the last seven
      // iterations, of which the last four load the next item's K tiles 0..3
      // and the last two its V tiles 0..1; the last computes its S_0.
      // Without the causal mask only the last tile can be masked; with it,
      // the tiles from n_clear on (the diagonal block) take the check.
      constexpr int NM = CAUSAL ? 0 : 8;
      if constexpr (CAUSAL) {
        for (; j + 7 < n_tiles && j + 3 < n_clear; j += 4) {
          step(std::false_type{}, Ic<1>{}, j, sB, sA, pA, pB, Ic<8>{});
          step(std::false_type{}, Ic<2>{}, j + 1, sA, sB, pB, pA, Ic<8>{});
          step(std::false_type{}, Ic<3>{}, j + 2, sB, sA, pA, pB, Ic<8>{});
          step(std::false_type{}, Ic<0>{}, j + 3, sA, sB, pB, pA, Ic<8>{});
        }
      }
      for (; j + 7 < n_tiles; j += 4) {
        step(std::false_type{}, Ic<1>{}, j, sB, sA, pA, pB, Ic<NM>{});
        step(std::false_type{}, Ic<2>{}, j + 1, sA, sB, pB, pA, Ic<NM>{});
        step(std::false_type{}, Ic<3>{}, j + 2, sB, sA, pA, pB, Ic<NM>{});
        step(std::false_type{}, Ic<0>{}, j + 3, sA, sB, pB, pA, Ic<NM>{});
      }
      step(std::false_type{}, Ic<1>{}, j, sB, sA, pA, pB, Ic<NM>{});
      step(std::false_type{}, Ic<2>{}, j + 1, sA, sB, pB, pA, Ic<NM>{});
      step(std::false_type{}, Ic<3>{}, j + 2, sB, sA, pA, pB, Ic<NM>{});
      step(std::false_type{}, Ic<0>{}, j + 3, sA, sB, pB, pA, Ic<1 | NM>{});
      step(std::false_type{}, Ic<1>{}, j + 4, sB, sA, pA, pB, Ic<1 | NM>{});
      step(std::false_type{}, Ic<2>{}, j + 5, sA, sB, pB, pA, Ic<3 | NM>{});
      step(std::false_type{}, Ic<3>{}, j + 6, sB, sA, pA, pB, Ic<7>{});
      if (sees(j + 6)) gemm2(j + 6, Ic<3>{}, vpre, pB);
    } else {
      // First the tiles no wave masks, then the rest with the per-wave check.
      for (; j + 3 < n_clear; j += 4) {
        step(std::false_type{}, Ic<1>{}, j, sB, sA, pA, pB, Ic<8>{});
        step(std::false_type{}, Ic<2>{}, j + 1, sA, sB, pB, pA, Ic<8>{});
        step(std::false_type{}, Ic<3>{}, j + 2, sB, sA, pA, pB, Ic<8>{});
        step(std::false_type{}, Ic<0>{}, j + 3, sA, sB, pB, pA, Ic<8>{});
      }
      for (; j + 3 < n_tiles; j += 4) {
        step(std::false_type{}, Ic<1>{}, j, sB, sA, pA, pB, Ic<0>{});
        step(std::false_type{}, Ic<2>{}, j + 1, sA, sB, pB, pA, Ic<0>{});
        step(std::false_type{}, Ic<3>{}, j + 2, sB, sA, pA, pB, Ic<0>{});
        step(std::false_type{}, Ic<0>{}, j + 3, sA, sB, pB, pA, Ic<0>{});
      }
      // Up to three iterations left (j % 4 == 1), then O += P_{n-1} V_{n-1}.
      if (j < n_tiles) {
        step(std::false_type{}, Ic<1>{}, j, sB, sA, pA, pB, Ic<0>{});
        if (j + 1 < n_tiles) {
          step(std::false_type{}, Ic<2>{}, j + 1, sA, sB, pB, pA, Ic<0>{});
          if (j + 2 < n_tiles) {
            step(std::false_type{}, Ic<3>{}, j + 2, sB, sA, pA, pB, Ic<0>{});
            if (sees(j + 2)) gemm2(j + 2, Ic<3>{}, vpre, pB);
          } else {
            if (sees(j + 1)) gemm2(j + 1, Ic<2>{}, vpre, pA);
          }
        } else {
          if (sees(j)) gemm2(j, Ic<1>{}, vpre, pB);
        }
      } else {
        if (sees(j - 1)) gemm2(j - 1, Ic<0>{}, vpre, pA);
      }
    }
  }

  // ---- epilogue: O = acc / l, lse = (m_ref + log2 l) * ln 2; a row that saw
  // no key (l = 0) gets O = 0 and lse = -inf.  O goes through LDS so that the
  // global stores are whole rows: a lane holds 4-element pieces of one row,
  // which written straight out would be 8-byte pieces of 32 rows per store.
  // The LDS is reused only once every wave is done with the K and V tiles
  // and every load into it has landed: the last iterations still load tiles
  // past the end (waited one iteration late), whose writes must not fall
  // into the staged output.  PERSIST stages the output apart from the ring,
  // where the next item's first tiles are still landing, in the area of the
  // next item's query tile, which every wave read before the barrier that
  // ended the last iteration: no further wait.
  if constexpr (!PERSIST || kSyncCheck) {
    wait_vmem();
    __syncthreads();
  }
  // SPLIT with part_o set: the part's fp32 output (normalised by the part's
  // own sum) and logsumexp, straight from registers: a lane holds 4
  // consecutive channels of one row per store.  Without part_o (one part,
  // no workspace) the kernel writes O and lse itself, below.
  if constexpr (SPLIT) if (P.part_o != nullptr) {
    const int sp = id % P.splits;
    const int64_t prow0 = (int64_t)sp * P.part_rows + (int64_t)bh * P.rows;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int qrow = q0 + MS * b + lq;
      const float l_tot = row_sum(l_part[b]);
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      if (qrow < P.rows) {
        float* const po = P.part_o + (prow0 + qrow) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < NACC / 4; ++g4) {
            const int ch = db * MS + g4 * 8 + lg * 4;
            float vsc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (Q8) {  // the per-channel value scales of the quantized cache
              const float4 f = *(const float4*)(P.vs + (int64_t)bh * D + ch);
              vsc[0] = f.x; vsc[1] = f.y; vsc[2] = f.z; vsc[3] = f.w;
            }
            const float4 v = {acc[b][db][g4 * 4] * vsc[0] * inv, acc[b][db][g4 * 4 + 1] * vsc[1] * inv,
                              acc[b][db][g4 * 4 + 2] * vsc[2] * inv, acc[b][db][g4 * 4 + 3] * vsc[3] * inv};
            *(float4*)(po + ch) = v;
          }
        if (lg == 0)
          P.part_lse[prow0 + qrow] = l_tot > 0.0f ? (m_ref[b] + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
    break;
  }
  // PERSIST: the lane's addresses here are recomputed per item rather than
  // held in registers through the loop.
  int el = lane;
  if constexpr (PERSIST) asm volatile("" : "+v"(el));
  const int elq = el & (MS - 1), elg = el / MS;
  lds_char* const ow = lds + QOBASE + wave * (MS * QB) * OROW;  // this wave's rows
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int qrow = q0 + MS * b + elq;
    const float l_tot = row_sum(l_part[b]);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < NACC / 4; ++g4) {
        // output channels ch .. ch+3
        const int ch = db * MS + g4 * 8 + elg * 4;
        float vsc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (Q8) {  // the per-channel value scales of the quantized cache
          const float4 f = *(const float4*)(P.vs + (int64_t)bh * D + ch);
          vsc[0] = f.x; vsc[1] = f.y; vsc[2] = f.z; vsc[3] = f.w;
        }
        X4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ov[e] = (E)(Q8 ? acc[b][db][g4 * 4 + e] * vsc[e] * inv : acc[b][db][g4 * 4 + e] * inv);
        *(__attribute__((address_space(3))) u32x2*)(ow + (MS * b + elq) * OROW + ch * 2) =
            __builtin_bit_cast(u32x2, ov);
      }
    if (elg == 0 && qrow < P.rows)
      P.lse[(int64_t)bh * P.rows + qrow] =
          l_tot > 0.0f ? (m_ref[b] + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
  // The wave reads back only its own rows (LDS operations of one wave are
  // ordered): D/8 lanes per row, 16 bytes each, so a store covers 64 / (D/8)
  // whole rows.  O is written once and not read again here: the stores carry
  // the non-temporal hint.
  constexpr int CPO = D / 8;                         // 16-byte pieces per O row
  constexpr int OPIECES = MS * QB * CPO;             // pieces per wave
  static_assert(OPIECES % 64 == 0, "whole stores per wave");
#pragma unroll
  for (int s = 0; s < OPIECES / 64; ++s) {
    const int lin = s * 64 + el;
    const int r = lin / CPO, pc = lin % CPO;
    const u32x4 piece = *(const __attribute__((address_space(3))) u32x4*)(ow + r * OROW + pc * 16);
    if (q0 + r < P.rows)
      __builtin_nontemporal_store(piece, (u32x4*)(P.o + q_head + (int64_t)(q0 + r) * D + pc * 8));
  }
  if constexpr (!PERSIST) {
    break;
  } else {
    if (!has_next) break;
    // The next item: its S_0 is in sA and the first operands of its K_1 in
    // kpre (this item's last iteration), its first K/V tiles in the ring.
    bh = bh_nx;
    qt = qt_nx;
    q_head = (int64_t)bh * P.rows * D;
    q0 = qt * BR + wave * MS * QB;
    item_limits();
    k_rs = rebase(k_rs, nx_delta);
    v_rs = rebase(v_rs, nx_delta);
    look_ahead(item + 1);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[b][db][i] = 0.0f;
      m_ref[b] = -INFINITY;
      l_part[b] = 0.0f;
    }
    __syncthreads();  // the staged output is read before the next query tile lands there
  }
  }
}

typedef void (*kernel_fn)(const Problem);

template <int D, bool FP16, bool CAUSAL, int QK, bool SHORT, bool PERSIST = false>
kernel_fn pick_mode(int mode) {
  switch (mode) {
    case kNegative: return fa2_fwd_kernel<D, FP16, kNegative, CAUSAL, QK, SHORT, PERSIST, false>;
    case kZero: return fa2_fwd_kernel<D, FP16, kZero, CAUSAL, QK, SHORT, PERSIST, false>;
    default: return fa2_fwd_kernel<D, FP16, kPositive, CAUSAL, QK, SHORT, PERSIST, false>;
  }
}

template <int D, int QK, bool SHORT = false>
kernel_fn pick(bool fp16, int mode, bool causal) {
  if (fp16)
    return causal ? pick_mode<D, true, true, QK, SHORT>(mode)
                  : pick_mode<D, true, false, QK, SHORT>(mode);
  return causal ? pick_mode<D, false, true, QK, SHORT>(mode)
                : pick_mode<D, false, false, QK, SHORT>(mode);
}

// Key-split kernels: 128-query-row tiles at every head dimension (the d = 128
// half-height shape), so that few query rows still make many workgroups.
template <int D> struct SplitCfg { using C = Cfg<D>; };
template <> struct SplitCfg<128> { using C = CfgS<128>; };
template <int D>
constexpr int kSplitRows = SplitCfg<D>::C::NW * SplitCfg<D>::C::MS * SplitCfg<D>::C::QB;
template <int D>
constexpr int kSplitKeys = SplitCfg<D>::C::BC;
constexpr int kMaxSplits = 128;

// Merge of the key splits' partials (see SplitProblem): for each row, with
// m the largest part logsumexp and w_s = exp(lse_s - m), O = sum_s w_s O_s /
// sum_s w_s and lse = m + log(sum_s w_s), which is the softmax over the
// union of the parts' keys (every part's O_s is normalised by its own sum
// exp(lse_s)).  A row that no part saw (every lse_s = -inf) gets O = 0,
// lse = -inf.  Each thread owns 4 channels of one row.  There are few rows
// when splits pay (decoding), so the merge is bound by load latency, not
// bytes: the parts are read 8 at a time, every load of a chunk issued
// before any is used, and folded into running sums whose reference m moves
// chunk by chunk as in an online softmax.
constexpr int kMergeThreads = 256;
template <int D, bool FP16>
__global__ void __launch_bounds__(kMergeThreads)
fa2_split_merge_kernel(const float* part_o, const float* part_lse, uint16_t* o, float* lse,
                       int64_t rows, int splits) {
  using X4 = typename Vec<FP16>::x4;
  using E = typename Vec<FP16>::e;
  constexpr int TPR = D / 4;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t r = gid / TPR;
  const int c4 = (int)(gid - r * TPR);
  if (r >= rows) return;
  float m = -INFINITY, wsum = 0.0f;
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto fold = [&](int s0, auto count) {
    constexpr int U = decltype(count)::value;
    float ls[U];
    float4 po[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = (int64_t)(s0 + u) * rows + r;
      ls[u] = part_lse[row];
      po[u] = *(const float4*)(part_o + row * D + c4 * 4);
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mc = fmaxf(mc, ls[u]);
    if (mc == -INFINITY) return;  // no part so far saw a key
    const float alpha = __builtin_amdgcn_exp2f((m - mc) * kLog2e);  // 0 while m = -inf
    wsum *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __builtin_amdgcn_exp2f((ls[u] - mc) * kLog2e);
      wsum += w;
      a[0] += w * po[u].x;
      a[1] += w * po[u].y;
      a[2] += w * po[u].z;
      a[3] += w * po[u].w;
    }
    m = mc;
  };
  int s = 0;
  for (; s + 8 <= splits; s += 8) fold(s, Ic<8>{});
  for (; s < splits; ++s) fold(s, Ic<1>{});
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const X4 out = {(E)(a[0] * inv), (E)(a[1] * inv), (E)(a[2] * inv), (E)(a[3] * inv)};
  *(u32x2*)(o + r * D + c4 * 4) = __builtin_bit_cast(u32x2, out);
  if (c4 == 0) lse[r] = wsum > 0.0f ? m + __log2f(wsum) * kLn2 : -INFINITY;
}

template <int D, bool FP16, bool CAUSAL>
const void* pick_split_mode(int mode) {
  constexpr bool S = D == 128;  // the half-height shape at d = 128
  switch (mode) {
    case kNegative: return (const void*)fa2_fwd_kernel<D, FP16, kNegative, CAUSAL, 0, S, false, true>;
    case kZero: return (const void*)fa2_fwd_kernel<D, FP16, kZero, CAUSAL, 0, S, false, true>;
    default: return (const void*)fa2_fwd_kernel<D, FP16, kPositive, CAUSAL, 0, S, false, true>;
  }
}

// Quantized caches (QK 1: INT8, 2: FP8), 128-row tiles.
template <int D, int QK, bool FP16, bool CAUSAL>
const void* pick_split_q8_mode(int mode) {
  switch (mode) {
    case kNegative: return (const void*)fa2_fwd_kernel<D, FP16, kNegative, CAUSAL, QK, true, false, true>;
    case kZero: return (const void*)fa2_fwd_kernel<D, FP16, kZero, CAUSAL, QK, true, false, true>;
    default: return (const void*)fa2_fwd_kernel<D, FP16, kPositive, CAUSAL, QK, true, false, true>;
  }
}

template <int D, int QK>
const void* pick_split_q8(bool fp16, int mode, bool causal) {
  if (fp16)
    return causal ? pick_split_q8_mode<D, QK, true, true>(mode) : pick_split_q8_mode<D, QK, true, false>(mode);
  return causal ? pick_split_q8_mode<D, QK, false, true>(mode) : pick_split_q8_mode<D, QK, false, false>(mode);
}
static_assert(kSplitRows<128> == Cfg8S<128>::NW * Cfg8S<128>::MS * Cfg8S<128>::QB &&
                  kSplitKeys<128> == Cfg8S<128>::BC &&
                  kSplitRows<64> == Cfg8S<64>::NW * Cfg8S<64>::MS * Cfg8S<64>::QB &&
                  kSplitKeys<64> == Cfg8S<64>::BC &&
                  kSplitRows<256> == Cfg8S<256>::NW * Cfg8S<256>::MS * Cfg8S<256>::QB &&
                  kSplitKeys<256> == Cfg8S<256>::BC,
              "the quantized split kernels share the 16-bit split plan");

template <int D>
const void* pick_split(bool fp16, int mode, bool causal) {
  if (fp16)
    return causal ? pick_split_mode<D, true, true>(mode) : pick_split_mode<D, true, false>(mode);
  return causal ? pick_split_mode<D, false, true>(mode) : pick_split_mode<D, false, false>(mode);
}

// Compute units of the current device (0 if unknown), cached per device.
// The cache entries are atomics: threads that race on a first call each
// query the attribute and store the same value.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The fixed scratch of fa2_fwd_split_noalloc (key-split partials for
// callers that cannot allocate): one array per device, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it only names the symbol): scratch_ptr() looks up each device's copy
// once, with that device current, and every use goes through that pointer.
constexpr int64_t kScratchBytes = (int64_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// This device's scratch address (nullptr if the lookup fails), cached per
// device; threads that race on a first lookup store the same value.
void* scratch_ptr() {
  static std::atomic<void*> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    cache[dev].store(p, std::memory_order_release);
  }
  return p;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace fa2

extern "C" {

const char* fa2_strerror(int status) {
  switch (status) {
    case FA2_OK: return "success";
    case FA2_ERR_NULL: return "a required pointer is NULL";
    case FA2_ERR_SHAPE: return "a size is negative, heads do not group, or sizes are too large";
    case FA2_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA2_ERR_DTYPE: return "dtype must be FA2_BF16 or FA2_FP16";
    case FA2_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA2_ERR_SCALE: return "scale must be finite";
    case FA2_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case FA2_ERR_HIP: return "kernel launch failed";
    case FA2_ERR_OPTION: return "causal must be 0 or 1, and a split count 0 to 128";
    case FA2_ERR_WORKSPACE: return "the key-split workspace is NULL or too small";
    case FA2_ERR_SCRATCH: return "the key-split partials exceed the 16 MiB fixed scratch";
    default: return "unknown status";
  }
}

int fa2_tile_config(int64_t d, int dtype, int* block_q, int* block_k, int* waves) {
  if (!block_q || !block_k || !waves) return FA2_ERR_NULL;
  if (dtype != FA2_BF16 && dtype != FA2_FP16) return FA2_ERR_DTYPE;
  switch (d) {
    case 64: *block_q = fa2::Cfg<64>::NW * fa2::Cfg<64>::MS * fa2::Cfg<64>::QB; *block_k = fa2::Cfg<64>::BC; *waves = fa2::Cfg<64>::NW; break;
    case 128: *block_q = fa2::Cfg<128>::NW * fa2::Cfg<128>::MS * fa2::Cfg<128>::QB; *block_k = fa2::Cfg<128>::BC; *waves = fa2::Cfg<128>::NW; break;
    case 256: *block_q = fa2::Cfg<256>::NW * fa2::Cfg<256>::MS * fa2::Cfg<256>::QB; *block_k = fa2::Cfg<256>::BC; *waves = fa2::Cfg<256>::NW; break;
    default: return FA2_ERR_HEADDIM;
  }
  return FA2_OK;
}

}  // extern "C"

namespace fa2 {

// The key-split plan of a call whose shape has passed validation: the split
// count (splits = 0: enough splits for one workgroup per CU over the call's
// query tiles, two with a quantized cache (qk != 0), each split keeping at
// least 8 key tiles, at most kMaxSplits; 1 when that leaves a single
// split), the query tiles per K/V head and the workspace bytes (0 without
// splits).  Those targets measured best for decoding shapes (one to 128
// query rows per K/V head, 8K to 128K keys: 4.8-5.6 TB/s of 16-bit K/V reads
// at d = 64 to 256, 3.0-4.4 TB/s of INT8 / FP8 codes, whose kernels also
// widen V and quantize the query); more splits only add partials to write
// and merge.
struct SplitPlan {
  int splits;
  int64_t q_tiles;
  int64_t bytes;
};
SplitPlan plan_split(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                     int qk, int splits) {
  const int64_t rows = Hq / Hkv * Nq;
  const int64_t br = d == 64 ? kSplitRows<64> : d == 128 ? kSplitRows<128> : kSplitRows<256>;
  const int64_t bc = d == 64 ? kSplitKeys<64> : d == 128 ? kSplitKeys<128> : kSplitKeys<256>;
  SplitPlan p;
  p.q_tiles = (rows + br - 1) / br;
  if (splits == 0) {
    const int64_t items = B * Hkv * p.q_tiles;
    const int64_t cus = cu_count();
    const int64_t k_tiles = (Nk + bc - 1) / bc;
    const int64_t per_cu = qk != 0 ? 2 : 1;
    int64_t want = cus > 0 ? (per_cu * cus + items - 1) / items : 1;
    // Items whose rows fill at most half a tile (a few query rows per K/V
    // head, as in decoding) take at least two parts once the keys are long
    // enough, even when the items alone fill the GPU: the split kernels'
    // half-height tiles leave their padding waves idle, which the unsplit
    // ones do not.
    if (rows * 2 <= br && k_tiles >= 64 && want < 2) want = 2;
    want = want < k_tiles / 8 ? want : k_tiles / 8;
    want = want < kMaxSplits ? want : kMaxSplits;
    splits = (int)(want > 1 ? want : 1);
  }
  p.splits = splits;
  p.bytes = splits > 1 ? (int64_t)splits * (B * Hq * Nq) * (d + 1) * 4 : 0;
  return p;
}

// Shape checks shared by the entry points (no pointer is looked at).
// Returns FA2_OK, an error, or 1 when the call has no output rows.
int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                int causal, int dtype, bool q8) {
  if (dtype != FA2_BF16 && dtype != FA2_FP16) return FA2_ERR_DTYPE;
  if (d != 64 && d != 128 && d != 256) return FA2_ERR_HEADDIM;
  if (causal != 0 && causal != 1) return FA2_ERR_OPTION;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return FA2_ERR_SHAPE;
  if (B == 0 || Hq == 0 || Nq == 0) return 1;  // no output rows
  if (Hkv == 0 || Hq % Hkv != 0) return FA2_ERR_SHAPE;
  // The query rows of one K/V head's group (group * Nq) and the key rows of
  // one K/V head are addressed with 32-bit offsets (plus slack for the loads
  // of tiles past the end); the workgroup count fits a 1-D grid.
  const int64_t lim = ((int64_t)1 << 31) - ((int64_t)1 << 20);
  if (Nq > (int64_t)1 << 30 || Nk > (int64_t)1 << 30 || Nk * d > lim) return FA2_ERR_SHAPE;
  const int64_t group = Hq / Hkv;
  if (group > lim / (Nq * d)) return FA2_ERR_SHAPE;
  const int64_t rows = group * Nq;  // query rows per K/V head
  if (B > (((int64_t)1 << 31) - 1) / Hq) return FA2_ERR_SHAPE;
  // The workgroup count fits a 1-D grid for every tile height the call may
  // take (the smallest, 128 query rows, gives the most workgroups).
  int bq = 0, bk = 0, nw = 0;
  fa2_tile_config(d, dtype, &bq, &bk, &nw);
  const int64_t bq_min = q8 ? (d == 64 ? Cfg8<64>::NW * Cfg8<64>::MS * Cfg8<64>::QB
                               : d == 128 ? Cfg8<128>::NW * Cfg8<128>::MS * Cfg8<128>::QB
                                          : Cfg8<256>::NW * Cfg8<256>::MS * Cfg8<256>::QB)
                       : d == 128 ? CfgS<128>::NW * CfgS<128>::MS * CfgS<128>::QB : bq;
  if (B * Hkv > (((int64_t)1 << 31) - 1) / ((rows + bq_min - 1) / bq_min)) return FA2_ERR_SHAPE;
  return FA2_OK;
}

// The split plan of a call that passed check_shape, with its own limits:
// the split count in range, the grids of both kernels within a 1-D grid.
int check_split(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                int qk, int splits, SplitPlan* plan) {
  if (splits < 0 || splits > kMaxSplits) return FA2_ERR_OPTION;
  *plan = plan_split(B, Hq, Hkv, Nq, Nk, d, qk, splits);
  if (plan->splits == 1) return FA2_OK;
  const int64_t grid_max = ((int64_t)1 << 31) - 1;
  if (B * Hkv * plan->q_tiles > grid_max / plan->splits) return FA2_ERR_SHAPE;
  if ((B * Hq * Nq * (d / 4) + kMergeThreads - 1) / kMergeThreads > grid_max) return FA2_ERR_SHAPE;
  return FA2_OK;
}

// Validation and launch shared by the entry points.  qk selects a quantized
// key/value cache: 1, INT8 (k, v int8 codes); 2, FP8 (k, v E4M3 codes); ks,
// vs are then their per-channel scales.  splits != 1 (16-bit only): key
// splits (0: planned here) with the partials in `ws`, ws_bytes long.
int launch(const void* q, const void* k, const void* v, const float* ks, const float* vs,
           void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
           int64_t d, float scale, int causal, int dtype, void* stream, int qk,
           int splits = 1, void* ws = nullptr, int64_t ws_bytes = 0) {
  const bool q8 = qk != 0;
  const int shape = check_shape(B, Hq, Hkv, Nq, Nk, d, causal, dtype, q8);
  if (shape < 0) return shape;
  // logits in log2 units: t = s * scale * log2(e), which must stay finite
  const float c = (float)((double)scale * 1.4426950408889634074);
  if (!__builtin_isfinite(scale) || !__builtin_isfinite(c)) return FA2_ERR_SCALE;
  if (splits < 0 || splits > kMaxSplits) return FA2_ERR_OPTION;
  if (shape == 1) return FA2_OK;  // no output rows
  const int64_t rows = Hq / Hkv * Nq;  // query rows per K/V head
  const int64_t bh = B * Hq;
  int bq = 0, bk = 0, nw = 0;
  fa2_tile_config(d, dtype, &bq, &bk, &nw);
  if (!q || !o || !lse || (Nk > 0 && (!k || !v))) return FA2_ERR_NULL;
  if (q8 && (!ks || !vs)) return FA2_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA2_ERR_ALIGN;
  if (((uintptr_t)ks | (uintptr_t)vs | (uintptr_t)ws) & 15) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA2_ERR_ALIGN;
  const size_t qbytes = (size_t)(bh * Nq * d) * 2;
  const size_t kbytes = (size_t)(B * Hkv * Nk * d) * (q8 ? 1 : 2);
  const size_t sbytes = q8 ? (size_t)(B * Hkv * d) * 4 : 0;
  const size_t lbytes = (size_t)(bh * Nq) * 4;
  const void* in[5] = {q, k, v, ks, vs};
  const size_t in_bytes[5] = {qbytes, kbytes, kbytes, sbytes, sbytes};
  for (int i = 0; i < 5; ++i)
    if (overlaps(o, qbytes, in[i], in_bytes[i]) || overlaps(lse, lbytes, in[i], in_bytes[i]))
      return FA2_ERR_ALIAS;
  if (overlaps(lse, lbytes, o, qbytes)) return FA2_ERR_ALIAS;
  // The split plan (for splits = 0 it queries the device's CU count), then
  // the workspace it needs.
  SplitPlan plan;
  if (splits != 1) {
    const int sc = check_split(B, Hq, Hkv, Nq, Nk, d, qk, splits, &plan);
    if (sc != FA2_OK) return sc;
    splits = plan.splits;
  }
  if (splits > 1) {
    if (!ws || ws_bytes < plan.bytes) return FA2_ERR_WORKSPACE;
    const size_t wbytes = (size_t)plan.bytes;
    for (int i = 0; i < 5; ++i)
      if (overlaps(ws, wbytes, in[i], in_bytes[i])) return FA2_ERR_ALIAS;
    if (overlaps(ws, wbytes, o, qbytes) || overlaps(ws, wbytes, lse, lbytes)) return FA2_ERR_ALIAS;
  }

  // Launch shape (the arguments are valid; from here on HIP may be queried).
  // Persistent workgroups (one per CU) when every one gets at least two items
  // whose key-tile counts the ring's four slots divide and are at least 8 (the
  // ring then carries on from one item into the next at slot 0), also for
  // short key sequences: at d = 128 (256-row items) and, without the mask, at
  // d = 64 (the CfgP shape, 256-row items of 64-key tiles).  Without the mask
  // every item has all key tiles.  With it (d = 128), query tile i of a head
  // needs (256 (i + 1) + Nk - Nq) / 32 key tiles when Nq is a multiple of the
  // 256-row tile (no tile straddles two query heads), Nk of 128 and Nk >= Nq;
  // workgroups then take pairs of query tiles i and T-1-i of one K/V head
  // (T of them, an even number), which all cost the same.
  const int64_t items_full = B * Hkv * ((rows + bq - 1) / bq);  // full-height workgroups
  bool persist = false;
  int cus = 0;
  if (!q8 && d == 64 && !causal) {
    constexpr int64_t BRP = CfgP<64>::NW * CfgP<64>::MS * CfgP<64>::QB;
    const int64_t items_p = B * Hkv * ((rows + BRP - 1) / BRP);
    const int64_t k_tiles = (Nk + CfgP<64>::BC - 1) / CfgP<64>::BC;
    if (k_tiles >= 8 && k_tiles % CfgP<64>::RING == 0 && items_p % 8 == 0) {
      cus = cu_count();
      persist = cus > 0 && cus % 8 == 0 && items_p >= 2 * (int64_t)cus;
    }
  }
  if (!q8 && d == 128) {
    constexpr int64_t BR128 = Cfg<128>::NW * Cfg<128>::MS * Cfg<128>::QB;
    const int64_t k_tiles = (Nk + Cfg<128>::BC - 1) / Cfg<128>::BC;
    const bool shape_ok =
        !causal ? (k_tiles >= 8 && k_tiles % Cfg<128>::RING == 0 && items_full % 8 == 0)
                : (Nq % BR128 == 0 && Nk % (Cfg<128>::BC * Cfg<128>::RING) == 0 && Nk >= Nq &&
                   (rows / BR128) % 2 == 0 && items_full % 16 == 0);
    if (shape_ok) {
      cus = cu_count();
      persist = cus > 0 && cus % 8 == 0 && items_full >= 2 * (int64_t)cus;
    }
  }
  // Half-height workgroups for short key sequences, and when the full-height
  // grid would leave compute units without a workgroup (few heads and query
  // rows, as in a prefill chunk against a cache): twice the workgroups.
  bool short_keys = !persist && !q8 && d == 128 && Nk <= kShortKeys;
  if (!persist && !q8 && d == 128 && !short_keys) {
    const int n_cu = cu_count();
    short_keys = n_cu > 0 && items_full < n_cu;
  }
  if (q8) {
    bq = d == 64 ? Cfg8<64>::NW * Cfg8<64>::MS * Cfg8<64>::QB
       : d == 128 ? Cfg8<128>::NW * Cfg8<128>::MS * Cfg8<128>::QB
                  : Cfg8<256>::NW * Cfg8<256>::MS * Cfg8<256>::QB;
    nw = d == 64 ? Cfg8<64>::NW : d == 128 ? Cfg8<128>::NW : Cfg8<256>::NW;
  } else if (persist && d == 64) {
    bq = CfgP<64>::NW * CfgP<64>::MS * CfgP<64>::QB;
    nw = CfgP<64>::NW;
  } else if (short_keys) {
    bq = CfgS<128>::NW * CfgS<128>::MS * CfgS<128>::QB;
    nw = CfgS<128>::NW;
  }
  const int64_t q_tiles = (rows + bq - 1) / bq;
  const int64_t groups = B * Hkv * q_tiles;

  const bool fp16 = dtype == FA2_FP16;
  const int mode = c > 0.0f ? kPositive : c < 0.0f ? kNegative : kZero;
  Problem P;
  P.q = (const uint16_t*)q;
  P.k = (const char*)k;
  P.v = (const char*)v;
  P.o = (uint16_t*)o;
  P.lse = lse;
  P.ks = ks;
  P.vs = vs;
  P.nq = (int)Nq;
  P.nk = (int)Nk;
  P.rows = (int)rows;
  P.q_tiles = (int)q_tiles;
  P.n_groups = (int)groups;
  P.causal_off = (int)(Nk - Nq);
  P.c = mode == kZero ? 1.0f : c;  // zero mode: logits are 0, t = s
  // Items of at most one key-split tile's rows (a few query rows per K/V
  // head, as in decoding) run on the key-split kernels also without splits,
  // as one part that writes O and lse itself: their 128-row tiles leave the
  // padding waves idle, which the other kernels' 256-row tiles compute.  The 16-bit
  // kernels take that route only once the items fill the compute units (on
  // fewer workgroups the half-height kernels ran 0-16% faster); the 8-bit
  // caches always (10-49% faster).
  const int64_t sbr = d == 64 ? kSplitRows<64> : d == 128 ? kSplitRows<128> : kSplitRows<256>;
  bool one_part = splits == 1 && rows <= sbr;
  if (one_part && !q8) {
    const int n_cu = cu_count();
    one_part = n_cu > 0 && B * Hkv * ((rows + sbr - 1) / sbr) >= n_cu;
  }
  // The same tiles are the 8-bit caches' half-height shape: taken also for
  // longer query blocks when the 256-row grid would leave compute units idle
  // (as the 16-bit half-height kernels are; 8-26% faster), except at d = 256
  // (no gain).
  if (splits == 1 && q8 && !one_part && d != 256) {
    const int n_cu = cu_count();
    one_part = n_cu > 0 && groups < n_cu;
  }
  if (splits > 1 || one_part) {
    // Key splits: the split kernel over items x splits workgroups, then the
    // merge, both on `stream` (one part: the split kernel alone).
    SplitProblem SP;
    static_cast<Problem&>(SP) = P;
    SP.q_tiles = (int)((rows + sbr - 1) / sbr);
    SP.n_groups = (int)(B * Hkv * SP.q_tiles * splits);
    SP.part_rows = bh * Nq;
    SP.part_o = one_part ? nullptr : (float*)ws;
    SP.part_lse = one_part ? nullptr : (float*)ws + (int64_t)splits * SP.part_rows * d;
    SP.splits = splits;
    const void* sfn = qk == 2 ? (d == 64 ? pick_split_q8<64, 2>(fp16, mode, causal)
                                 : d == 128 ? pick_split_q8<128, 2>(fp16, mode, causal)
                                            : pick_split_q8<256, 2>(fp16, mode, causal))
                    : qk == 1 ? (d == 64 ? pick_split_q8<64, 1>(fp16, mode, causal)
                                 : d == 128 ? pick_split_q8<128, 1>(fp16, mode, causal)
                                            : pick_split_q8<256, 1>(fp16, mode, causal))
                    : d == 64 ? pick_split<64>(fp16, mode, causal)
                    : d == 128 ? pick_split<128>(fp16, mode, causal)
                               : pick_split<256>(fp16, mode, causal);
    const int snw = q8 ? (d == 64 ? Cfg8S<64>::NW : d == 128 ? Cfg8S<128>::NW : Cfg8S<256>::NW)
                  : d == 64 ? SplitCfg<64>::C::NW : d == 128 ? SplitCfg<128>::C::NW
                                                             : SplitCfg<256>::C::NW;
    void* sargs[] = {&SP};
    hipError_t err = hipLaunchKernel(sfn, dim3((unsigned)SP.n_groups),
                                     dim3((unsigned)(snw * 64)), sargs, 0, (hipStream_t)stream);
    if (err != hipSuccess) return FA2_ERR_HIP;
    if (one_part) return FA2_OK;
    const float* po = SP.part_o;
    const float* pl = SP.part_lse;
    uint16_t* oo = SP.o;
    float* ll = lse;
    int64_t mrows = SP.part_rows;
    int msplits = splits;
    void* margs[] = {&po, &pl, &oo, &ll, &mrows, &msplits};
    const int64_t mblocks = (mrows * (d / 4) + kMergeThreads - 1) / kMergeThreads;
    const void* mfn = d == 64 ? (fp16 ? (const void*)fa2_split_merge_kernel<64, true>
                                      : (const void*)fa2_split_merge_kernel<64, false>)
                    : d == 128 ? (fp16 ? (const void*)fa2_split_merge_kernel<128, true>
                                       : (const void*)fa2_split_merge_kernel<128, false>)
                               : (fp16 ? (const void*)fa2_split_merge_kernel<256, true>
                                       : (const void*)fa2_split_merge_kernel<256, false>);
    err = hipLaunchKernel(mfn, dim3((unsigned)mblocks), dim3(kMergeThreads), margs, 0,
                          (hipStream_t)stream);
    return err == hipSuccess ? FA2_OK : FA2_ERR_HIP;
  }
  kernel_fn fn = qk == 2 ? (d == 64 ? pick<64, 2>(fp16, mode, causal)
                           : d == 128 ? pick<128, 2>(fp16, mode, causal) : pick<256, 2>(fp16, mode, causal))
               : q8 ? (d == 64 ? pick<64, 1>(fp16, mode, causal)
                       : d == 128 ? pick<128, 1>(fp16, mode, causal) : pick<256, 1>(fp16, mode, causal))
               : d == 64 ? pick<64, 0>(fp16, mode, causal)
               : d == 128 ? (short_keys ? pick<128, 0, true>(fp16, mode, causal)
                                        : pick<128, 0>(fp16, mode, causal))
                          : pick<256, 0>(fp16, mode, causal);
  int64_t grid = groups;
  if (persist) {
    if (d == 64)
      fn = fp16 ? pick_mode<64, true, false, 0, false, true>(mode)
                : pick_mode<64, false, false, 0, false, true>(mode);
    else
      fn = fp16 ? (causal ? pick_mode<128, true, true, 0, false, true>(mode)
                          : pick_mode<128, true, false, 0, false, true>(mode))
                : (causal ? pick_mode<128, false, true, 0, false, true>(mode)
                          : pick_mode<128, false, false, 0, false, true>(mode));
    grid = cus;
  }
  void* args[] = {&P};
  hipError_t err = hipLaunchKernel((const void*)fn, dim3((unsigned)grid),
                                   dim3((unsigned)(nw * 64)), args, 0,
                                   (hipStream_t)stream);
  return err == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

}  // namespace fa2

extern "C" {

int fa2_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                float scale, int causal, int dtype, void* stream) {
  return fa2::launch(q, k, v, nullptr, nullptr, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                     dtype, stream, 0);
}

int fa2_fwd_kv_int8(const void* q, const int8_t* kq, const float* ks, const int8_t* vq,
                    const float* vs, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                    void* stream) {
  return fa2::launch(q, kq, vq, ks, vs, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype,
                     stream, 1);
}

int fa2_fwd_kv_fp8(const void* q, const uint8_t* kq, const float* ks, const uint8_t* vq,
                   const float* vs, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                   void* stream) {
  return fa2::launch(q, kq, vq, ks, vs, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype,
                     stream, 2);
}

int fa2_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                  float scale, int causal, int dtype, int splits, void* workspace,
                  int64_t workspace_bytes, void* stream) {
  return fa2::launch(q, k, v, nullptr, nullptr, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                     dtype, stream, 0, splits, workspace, workspace_bytes);
}

int64_t fa2_fwd_split_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                int64_t d, int causal, int dtype, int cache, int splits) {
  if (cache != 0 && cache != FA2_CACHE_INT8 && cache != FA2_CACHE_FP8) return FA2_ERR_OPTION;
  const int shape = fa2::check_shape(B, Hq, Hkv, Nq, Nk, d, causal, dtype, cache != 0);
  if (shape < 0) return shape;
  if (splits < 0 || splits > fa2::kMaxSplits) return FA2_ERR_OPTION;
  if (shape == 1 || splits == 1) return 0;
  fa2::SplitPlan plan;
  const int sc = fa2::check_split(B, Hq, Hkv, Nq, Nk, d, cache, splits, &plan);
  if (sc != FA2_OK) return sc;
  return plan.bytes;
}

int fa2_fwd_kv_split(const void* q, const void* kq, const float* ks, const void* vq,
                     const float* vs, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                     int cache, int splits, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  if (cache != FA2_CACHE_INT8 && cache != FA2_CACHE_FP8) return FA2_ERR_OPTION;
  return fa2::launch(q, kq, vq, ks, vs, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype,
                     stream, cache == FA2_CACHE_INT8 ? 1 : 2, splits, workspace,
                     workspace_bytes);
}

int fa2_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                          int64_t d, float scale, int causal, int dtype, int splits,
                          void* stream) {
  int64_t need = fa2_fwd_split_workspace(B, Hq, Hkv, Nq, Nk, d, causal, dtype, 0, splits);
  if (need < 0) return (int)need;
  if (need > fa2::kScratchBytes && splits == 0) {
    // The library's own count does not fit: the most parts that do, or none.
    const int64_t per_part = fa2_fwd_split_workspace(B, Hq, Hkv, Nq, Nk, d, causal, dtype, 0, 2) / 2;
    const int64_t fit = per_part > 0 ? fa2::kScratchBytes / per_part : 0;
    splits = fit >= 2 ? (int)fit : 1;
    need = fit >= 2 ? fit * per_part : 0;
  }
  if (need > fa2::kScratchBytes) return FA2_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    ws = fa2::scratch_ptr();
    if (ws == nullptr) return FA2_ERR_HIP;
  }
  return fa2::launch(q, k, v, nullptr, nullptr, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                     dtype, stream, 0, splits, ws, fa2::kScratchBytes);
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype,
            void* stream) {
  return fa2_fwd_ext(q, k, v, o, lse, B, H, H, N, N, d, scale, 0, dtype, stream);
}

}  // extern "C"
