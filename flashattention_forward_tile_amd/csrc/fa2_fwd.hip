// fa2_fwd.hip -- FlashAttention-2 forward pass for gfx950 (MI355X, CDNA4).
//
// One workgroup owns one (batch, head, query tile) and streams every key/value
// tile of that head through LDS, keeping the running softmax state and the
// output accumulator in registers, so the N x N score matrix never reaches
// HBM (the fusion described in the abstract of "A Case Study in CUDA Kernel
// Fusion: Implementing FlashAttention-2 on NVIDIA Hopper Architecture using the
// CUTLASS Library" and in "Flash Attention 2 from scratch on Ampere", Part 1,
// "Why Flash Attention?").  The per-workgroup flow (query tile held on chip,
// loop over the j-th key/value tile) follows that page's Notation section.
//
// CDNA4 mapping (prior art re-designed, not translated):
//  * Both products run on v_mfma_f32_32x32x16_{bf16,f16}.  The first product is
//    computed transposed, S^T = K_j Q_i^T, so each lane of a wave owns one query
//    column: lanes l and l+32 hold the two halves of that query's keys.  The
//    row max and row sum of the softmax are then in-lane reductions plus one
//    exchange between the two lane halves.
//  * The S^T accumulator layout is exactly the B-operand layout of the second
//    product O^T += V_j^T P^T, once V_j^T is stored in LDS in the matching key
//    order, so P never leaves registers.
//  * K_j is staged row-major and V_j transposed into XOR-swizzled LDS (bank
//    conflicts were the largest single gain in the Ampere series' table,
//    kernel 2), double-buffered, with tile j+1's global loads in flight while
//    tile j is computed (kernels 3 and 5 of that table).
//  * Softmax in fp32 registers with exp2 and the scale folded into one FMA
//    (kernel 6); the running-max rescale of O is skipped unless some row's max
//    grew by more than kRescaleSlack (log2 units), which keeps the result exact
//    because every p and l then share the same stale reference max.
//  * Workgroup ids are remapped so all query tiles of a head land on one XCD
//    and share that XCD's L2 copy of the head's K and V.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa2.h"

namespace fa2 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// p = exp2(t - m_ref) may reach 2^kRescaleSlack before O is rescaled.
constexpr float kRescaleSlack = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;

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

// XOR swizzle of 16-byte chunks within an LDS row of CPR chunks, chosen so the
// 16 lanes of a ds_read_b128 phase that read one logical chunk from 16
// consecutive rows hit 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swizzle(int row, int chunk) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16 || CPR == 32,
                "row of 64, 128, 256 or 512 B");
  if constexpr (CPR >= 16)
    return chunk ^ (row & 15);  // rows start on the same bank: spread by row
  else if constexpr (CPR == 8)
    return chunk ^ ((row ^ (row >> 3)) & 7);  // 128 B rows: two rows per sweep
  else
    return chunk ^ ((row >> 2) & 3);  // 64 B rows: four rows per sweep
}

// Tile shape per head dimension: D, key rows per tile, waves per workgroup,
// waves per SIMD the register budget is sized for.
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int BC = 64, NW = 4, OCC = 2; };
template <> struct Cfg<128> { static constexpr int BC = 64, NW = 4, OCC = 2; };
template <> struct Cfg<256> { static constexpr int BC = 32, NW = 4, OCC = 1; };

template <int D, bool FP16, bool NEG>
__global__ void __attribute__((amdgpu_flat_work_group_size(Cfg<D>::NW * 64,
                                                           Cfg<D>::NW * 64),
                               amdgpu_waves_per_eu(Cfg<D>::OCC, Cfg<D>::OCC)))
fa2_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
               float* __restrict__ lse, int N, int q_tiles, int n_groups,
               float c) {
  constexpr int BC = Cfg<D>::BC;
  constexpr int NW = Cfg<D>::NW;
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;        // query rows per workgroup
  constexpr int CPR = D / 8;         // 16-byte chunks per K row
  constexpr int CPRV = BC / 8;       // 16-byte chunks per V^T row
  constexpr int KCH = BC * CPR / NT; // K chunks staged per thread
  constexpr int VUNITS = (BC / 4) * CPR;       // 4 keys x 8 dims per unit
  constexpr int VU = (VUNITS + NT - 1) / NT;   // units per thread
  constexpr int KBYTES = BC * D * 2;
  static_assert(BC * CPR % NT == 0, "K staging must divide evenly");
  static_assert(BC % 32 == 0 && D % 32 == 0, "MFMA 32x32 blocking");
  using X8 = typename Vec<FP16>::x8;
  using X4 = typename Vec<FP16>::x4;
  using E = typename Vec<FP16>::e;

  __shared__ __attribute__((aligned(16))) char smem[4 * KBYTES];
  char* const k_lds = smem;                 // [2][BC][D] row-major, swizzled
  char* const v_lds = smem + 2 * KBYTES;    // [2][D][BC] transposed, swizzled

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // All query tiles of one head go to one XCD (dispatch is round-robin over
  // the 8 XCDs): the k-th workgroup on XCD x takes logical tile x*G/8 + k.
  int id = blockIdx.x;
  if ((n_groups & 7) == 0) id = (id & 7) * (n_groups >> 3) + (id >> 3);
  const int bh = id / q_tiles;
  const int qt = id - bh * q_tiles;
  const int64_t head = (int64_t)bh * N * D;
  const uint16_t* __restrict__ qh = q + head;
  const uint16_t* __restrict__ kh = k + head;
  const uint16_t* __restrict__ vh = v + head;

  // Q_i fragments: the B operand of S^T = K_j Q_i^T, held for the whole loop.
  const int qrow = qt * BR + wave * 32 + l32;
  const int qrow_c = qrow < N ? qrow : N - 1;
  X8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = __builtin_bit_cast(
        X8, *(const u32x4*)(qh + (int64_t)qrow_c * D + ks * 16 + half * 8));

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  float m_ref = -INFINITY;  // reference max of this query, log2 units
  float l_part = 0.0f;      // this lane's share of the row sum

  u32x4 kst[KCH];
  u32x4 vst[VU][4];

  auto load_tile = [&](int key0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + NT * i;
      const int row = ch / CPR, cc = ch % CPR;
      int kr = key0 + row;
      kr = kr < N ? kr : N - 1;
      kst[i] = *(const u32x4*)(kh + (int64_t)kr * D + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + NT * i;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int g4 = u / CPR, dc = u % CPR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int vr = key0 + 4 * g4 + r;
          vr = vr < N ? vr : N - 1;
          vst[i][r] = *(const u32x4*)(vh + (int64_t)vr * D + dc * 8);
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* kb = k_lds + buf * KBYTES;
    char* vb = v_lds + buf * KBYTES;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + NT * i;
      const int row = ch / CPR, cc = ch % CPR;
      *(u32x4*)(kb + row * (D * 2) + swizzle<CPR>(row, cc) * 16) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = tid + NT * i;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int g4 = u / CPR, dc = u % CPR;
        // Key group g4 = 4 consecutive keys.  Within each 16-key step the
        // second and third groups trade places, matching the key order of the
        // S^T accumulator (lane half h, slot s -> key (s/4)*8 + h*4 + s%4).
        const int gi = g4 & 3;
        const int pg = ((gi & 1) << 1) | (gi >> 1);
        const int chunk = (g4 >> 2) * 2 + (pg >> 1);
        const int hoff = (pg & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          uint32_t lo, hi;
          if (e & 1) {
            lo = (vst[i][0][w] >> 16) | (vst[i][1][w] & 0xffff0000u);
            hi = (vst[i][2][w] >> 16) | (vst[i][3][w] & 0xffff0000u);
          } else {
            lo = (vst[i][0][w] & 0xffffu) | (vst[i][1][w] << 16);
            hi = (vst[i][2][w] & 0xffffu) | (vst[i][3][w] << 16);
          }
          const int d = dc * 8 + e;
          u32x2 pk;
          pk[0] = lo;
          pk[1] = hi;
          *(u32x2*)(vb + d * (BC * 2) + swizzle<CPRV>(d, chunk) * 16 + hoff) = pk;
        }
      }
    }
  };

  const int n_tiles = (N + BC - 1) / BC;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < n_tiles;
    if (more) load_tile((j + 1) * BC);

    const char* kb = k_lds + buf * KBYTES;
    const char* vb = v_lds + buf * KBYTES;

    // ---- S^T = K_j Q_i^T : [BC keys] x [32 queries] per wave
    f32x16 s[BC / 32];
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb32][i] = 0.0f;
      const int row = kb32 * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const X8 a = __builtin_bit_cast(
            X8, *(const u32x4*)(kb + row * (D * 2) +
                                swizzle<CPR>(row, ks * 2 + half) * 16));
        s[kb32] = mfma32x32x16<FP16>(a, qf[ks], s[kb32]);
      }
    }

    // ---- online softmax (fp32, log2 units, scale folded into c)
    const int key0 = j * BC;
    const bool tail = key0 + BC > N;  // wave-uniform
    auto key_of = [&](int kb32, int i) {
      return key0 + kb32 * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
    };
    if (tail) {
#pragma unroll
      for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key_of(kb32, i) >= N) s[kb32][i] = NEG ? INFINITY : -INFINITY;
    }
    float ext = s[0][0];
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        ext = NEG ? fminf(ext, s[kb32][i]) : fmaxf(ext, s[kb32][i]);
    const float t_max = __builtin_isfinite(ext) ? ext * c : -INFINITY;

    if (__builtin_amdgcn_ballot_w64(t_max > m_ref + kRescaleSlack) != 0) {
      // Only rows whose own max outgrew the slack move their reference, so a
      // row's arithmetic never depends on the other rows sharing its wave.
      const float t_row = fmaxf(t_max, __shfl_xor(t_max, 32));
      const float m_new = t_row > m_ref + kRescaleSlack ? t_row : m_ref;
      const float alpha =
          m_new == m_ref ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      l_part *= alpha;
      m_ref = m_new;
    }

    // p in fp32; the row sum takes the unrounded p, the second product takes
    // p rounded to the input type.
    float rs = 0.0f;
#pragma unroll
    for (int kb32 = 0; kb32 < BC / 32; ++kb32)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb32][i], c, -m_ref));
        if (tail && key_of(kb32, i) >= N) p = 0.0f;
        s[kb32][i] = p;
        rs += p;
      }
    l_part += rs;

    using X2 = typename Vec<FP16>::x2;
    X8 pf[BC / 16];
#pragma unroll
    for (int st = 0; st < BC / 16; ++st) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const X2 pair = {(E)s[st >> 1][(st & 1) * 8 + 2 * e],
                         (E)s[st >> 1][(st & 1) * 8 + 2 * e + 1]};
        w[e] = __builtin_bit_cast(uint32_t, pair);
      }
      pf[st] = __builtin_bit_cast(X8, w);
    }

    // ---- O^T += V_j^T P^T : [D] x [32 queries] per wave
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + l32;
#pragma unroll
      for (int st = 0; st < BC / 16; ++st) {
        const X8 a = __builtin_bit_cast(
            X8, *(const u32x4*)(vb + d * (BC * 2) +
                                swizzle<CPRV>(d, st * 2 + half) * 16));
        acc[db] = mfma32x32x16<FP16>(a, pf[st], acc[db]);
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, lse = (m_ref + log2 l) * ln 2
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l_tot;
  if (qrow < N) {
    uint16_t* orow = o + head + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        X4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (E)(acc[db][g * 4 + e] * inv);
        *(u32x2*)(orow + db * 32 + g * 8 + half * 4) = __builtin_bit_cast(u32x2, ov);
      }
    if (half == 0)
      lse[(int64_t)bh * N + qrow] = (m_ref + __log2f(l_tot)) * kLn2;
  }
}

typedef void (*kernel_fn)(const uint16_t*, const uint16_t*, const uint16_t*,
                          uint16_t*, float*, int, int, int, float);

template <int D>
kernel_fn pick(bool fp16, bool neg) {
  if (fp16) return neg ? fa2_fwd_kernel<D, true, true> : fa2_fwd_kernel<D, true, false>;
  return neg ? fa2_fwd_kernel<D, false, true> : fa2_fwd_kernel<D, false, false>;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace fa2

extern "C" {

const char* fa2_strerror(int status) {
  switch (status) {
    case FA2_OK: return "success";
    case FA2_ERR_NULL: return "a required pointer is NULL";
    case FA2_ERR_SHAPE: return "B, H or N negative, or sizes too large";
    case FA2_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA2_ERR_DTYPE: return "dtype must be FA2_BF16 or FA2_FP16";
    case FA2_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA2_ERR_SCALE: return "scale must be finite";
    case FA2_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case FA2_ERR_HIP: return "kernel launch failed";
    default: return "unknown status";
  }
}

int fa2_tile_config(int64_t d, int dtype, int* block_q, int* block_k, int* waves) {
  if (!block_q || !block_k || !waves) return FA2_ERR_NULL;
  if (dtype != FA2_BF16 && dtype != FA2_FP16) return FA2_ERR_DTYPE;
  switch (d) {
    case 64: *block_q = fa2::Cfg<64>::NW * 32; *block_k = fa2::Cfg<64>::BC; *waves = fa2::Cfg<64>::NW; break;
    case 128: *block_q = fa2::Cfg<128>::NW * 32; *block_k = fa2::Cfg<128>::BC; *waves = fa2::Cfg<128>::NW; break;
    case 256: *block_q = fa2::Cfg<256>::NW * 32; *block_k = fa2::Cfg<256>::BC; *waves = fa2::Cfg<256>::NW; break;
    default: return FA2_ERR_HEADDIM;
  }
  return FA2_OK;
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype,
            void* stream) {
  if (dtype != FA2_BF16 && dtype != FA2_FP16) return FA2_ERR_DTYPE;
  if (d != 64 && d != 128 && d != 256) return FA2_ERR_HEADDIM;
  if (B < 0 || H < 0 || N < 0) return FA2_ERR_SHAPE;
  if (!__builtin_isfinite(scale)) return FA2_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return FA2_OK;
  // N*d elements of one head are addressed with 32-bit row offsets; the
  // workgroup count must fit a 1-D grid.
  if (N > (int64_t)1 << 30 || N * d > ((int64_t)1 << 31) - 1) return FA2_ERR_SHAPE;
  int bq = 0, bk = 0, nw = 0;
  fa2_tile_config(d, dtype, &bq, &bk, &nw);
  const int64_t q_tiles = (N + bq - 1) / bq;
  if (B > ((int64_t)1 << 31) / H) return FA2_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > (((int64_t)1 << 31) - 1) / q_tiles) return FA2_ERR_SHAPE;
  const int64_t groups = bh * q_tiles;
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA2_ERR_ALIGN;
  if ((uintptr_t)lse & 3) return FA2_ERR_ALIGN;
  const size_t tbytes = (size_t)(bh * N * d) * 2;
  const size_t lbytes = (size_t)(bh * N) * 4;
  if (fa2::overlaps(o, tbytes, q, tbytes) || fa2::overlaps(o, tbytes, k, tbytes) ||
      fa2::overlaps(o, tbytes, v, tbytes) || fa2::overlaps(lse, lbytes, q, tbytes) ||
      fa2::overlaps(lse, lbytes, k, tbytes) || fa2::overlaps(lse, lbytes, v, tbytes) ||
      fa2::overlaps(lse, lbytes, o, tbytes))
    return FA2_ERR_ALIAS;

  // logits in log2 units: t = s * scale * log2(e)
  const float c = (float)((double)scale * 1.4426950408889634074);
  const bool fp16 = dtype == FA2_FP16;
  const bool neg = c < 0.0f;
  fa2::kernel_fn fn = d == 64 ? fa2::pick<64>(fp16, neg)
                    : d == 128 ? fa2::pick<128>(fp16, neg)
                               : fa2::pick<256>(fp16, neg);
  const uint16_t* qp = (const uint16_t*)q;
  const uint16_t* kp = (const uint16_t*)k;
  const uint16_t* vp = (const uint16_t*)v;
  uint16_t* op = (uint16_t*)o;
  int n32 = (int)N, qt32 = (int)q_tiles, g32 = (int)groups;
  void* args[] = {&qp, &kp, &vp, &op, &lse, &n32, &qt32, &g32, (void*)&c};
  hipError_t err = hipLaunchKernel((const void*)fn, dim3((unsigned)groups),
                                   dim3((unsigned)(nw * 64)), args, 0,
                                   (hipStream_t)stream);
  return err == hipSuccess ? FA2_OK : FA2_ERR_HIP;
}

}  // extern "C"
