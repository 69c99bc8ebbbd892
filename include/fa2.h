/*
 * fa2.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward pass.
 *
 * The operation is the forward pass of FlashAttention-2: non-causal scaled
 * dot-product attention computed tile by tile with an online softmax, so the
 * N x N score matrix never reaches HBM ("A Case Study in CUDA Kernel Fusion:
 * Implementing FlashAttention-2 on NVIDIA Hopper Architecture using the CUTLASS
 * Library", abstract; "Flash Attention 2 from scratch on Ampere", Part 1,
 * sections "Why Flash Attention?" and "Kernel Specification").  For every
 * batch b, head h and query row i:
 *
 *     s_ij  = scale * sum_c q[b,h,i,c] * k[b,h,j,c]
 *     o[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp(s_ij)
 *
 * Scope follows the Kernel Specification section of the Ampere Part 1 page:
 * forward only, non-causal, no dropout, no KV cache, equal query and key
 * lengths, 16-bit (bf16 or fp16) inputs and outputs, softmax in fp32.  The head
 * dimension may be 64, 128 (the page's) or 256.  Unlike the page, N need not
 * be a multiple of the block size: the last key tile is masked.  fa2_fwd_ext
 * adds causal masking, Nq != Nk and grouped key/value heads.
 *
 * All entry points are plain C.  Pointers are device pointers unless stated.
 */
#ifndef FA2_H
#define FA2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
enum fa2_dtype {
  FA2_BF16 = 0, /* bfloat16 (8-bit exponent, 7-bit mantissa) */
  FA2_FP16 = 1  /* IEEE binary16 */
};

/* Code format of a quantized key/value cache (fa2_fwd_kv_split). */
enum fa2_cache {
  FA2_CACHE_INT8 = 1, /* int8 codes, the scheme of fa2_fwd_kv_int8 */
  FA2_CACHE_FP8 = 2   /* OCP E4M3 codes, the scheme of fa2_fwd_kv_fp8 */
};

/* Return codes.  Every negative code except FA2_ERR_HIP is detected on the
 * host before any kernel is launched, and nothing is written; before any HIP
 * call at all, except that fa2_fwd_split with splits = 0 queries the
 * device's compute-unit count before it checks the workspace. */
enum fa2_status {
  FA2_OK = 0,
  FA2_ERR_NULL = -1,    /* a required pointer is NULL */
  FA2_ERR_SHAPE = -2,   /* a size is negative, Hq is not a multiple of Hkv,
                           the grid overflows, or the query rows of one K/V
                           head ((Hq/Hkv)*Nq*d) or its key rows (Nk*d) exceed
                           2^31 - 2^20 elements */
  FA2_ERR_HEADDIM = -3, /* d is not 64, 128 or 256 */
  FA2_ERR_DTYPE = -4,   /* dtype is not an fa2_dtype */
  FA2_ERR_ALIGN = -5,   /* q, k, v, o or a workspace not 16-byte aligned, lse
                           not 4-byte */
  FA2_ERR_SCALE = -6,   /* scale is NaN or infinite, or scale * log2(e)
                           overflows fp32 (|scale| above about 2.36e38) */
  FA2_ERR_ALIAS = -7,   /* o, lse or a workspace overlaps q, k, v, or each
                           other */
  FA2_ERR_HIP = -8,     /* the kernel launch failed (HIP error) */
  FA2_ERR_OPTION = -9,  /* causal is not 0 or 1, or a split count is out of
                           range */
  FA2_ERR_WORKSPACE = -10, /* the key-split workspace is NULL or too small */
  FA2_ERR_SCRATCH = -11   /* fa2_fwd_split_noalloc: the partials would exceed
                             its 16 MiB fixed scratch */
};

/*
 * fa2_fwd -- attention forward for B*H independent heads.
 *
 *   q, k, v  in : [B][H][N][d] contiguous, element type `dtype`; element
 *                 (b,h,n,c) at ((b*H + h)*N + n)*d + c.  16-byte aligned.
 *   o        out: same shape, layout and type as q.  16-byte aligned.
 *   lse      out: [B][H][N] contiguous fp32, lse(b,h,n) at (b*H + h)*N + n:
 *                 the natural-log logsumexp of row n's scaled logits.
 *   B, H, N  : batch, heads, sequence length (queries = keys = N), each >= 0.
 *              If B*H*N == 0 the call returns FA2_OK and touches nothing
 *              (pointers may then be NULL).
 *   d        : head dimension, 64, 128 or 256.
 *   scale    : multiplies the logits; any finite value whose product with
 *              log2(e) is a finite float, |scale| <= about 2.36e38
 *              (1/sqrt(d) is usual; 0 gives uniform attention, negative
 *              values are allowed).
 *   dtype    : an fa2_dtype.
 *   stream   : a hipStream_t, or NULL for the default stream.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing and
 * keeps no state between calls (it only caches each device's compute-unit
 * count, race-free), so concurrent calls on any streams and host threads are
 * safe as long as their outputs do not overlap.  o and lse must not overlap q, k, v or
 * each other.
 *
 * Asynchrony: the work is enqueued on `stream` and the call returns at once;
 * synchronise the stream before reading o or lse.
 *
 * Numerics: logits are accumulated in fp32 from the exact 16-bit inputs; the
 * softmax runs in fp32 with exp2; probabilities are rounded to `dtype` for the
 * second product, accumulated in fp32; o is rounded to `dtype` (nearest even).
 * Non-finite inputs propagate and are not diagnosed.
 *
 * Returns FA2_OK, or a negative fa2_status.
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int64_t B, int64_t H, int64_t N, int64_t d, float scale,
            int dtype, void* stream);

/*
 * fa2_fwd_ext -- the same operation widened along the rows the "Kernel
 * Specification" section of the Ampere Part 1 page leaves out: causal
 * masking, unequal query and key lengths (cross-attention, a key/value
 * cache), and grouped key/value heads (MQA/GQA, the setting of the Colfax
 * "FlashAttention-3 for Inference" post).  The query heads that share a key/value
 * head are processed together: their rows are tiled as one block, so short
 * query blocks (a prefill chunk, a few decode rows) still fill the tiles.
 *
 *   q, o     : [B][Hq][Nq][d] contiguous, element type `dtype`.
 *   k, v     : [B][Hkv][Nk][d] contiguous; query head h reads key/value head
 *              h / (Hq / Hkv).  Hq must be a multiple of Hkv >= 1.
 *   lse      : [B][Hq][Nq] fp32.
 *   causal   : 0 = every row sees all Nk keys; 1 = row i sees keys
 *              j <= i + Nk - Nq (the last row sees every key; with Nq == Nk
 *              this is the usual lower-triangular mask).
 *   A row that sees no key (causal with Nq > Nk, or Nk == 0) gets O = 0 and
 *   lse = -inf.  k and v may be NULL when Nk == 0.
 *
 * Other arguments, alignment, ownership, asynchrony, numerics and return
 * codes are those of fa2_fwd; fa2_fwd(q, k, v, o, lse, B, H, N, d, ...) is
 * fa2_fwd_ext(q, k, v, o, lse, B, H, H, N, N, d, scale, 0, dtype, stream).
 * B*Hq*Nq == 0 returns FA2_OK and touches nothing.
 */
int fa2_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                int64_t d, float scale, int causal, int dtype, void* stream);

/*
 * fa2_fwd_kv_int8 -- attention over an INT8 key/value cache.  The Colfax
 * author page lists "FlashAttention-3 for Inference: INT8 Quantization and
 * Query Head Packing for MQA/GQA" by title only; this is the library's
 * reading of it.  Keys and values arrive as int8 codes with fp32 per-channel
 * scales of their key/value head:
 *
 *     k[b,g,j,c] = ks[b,g,c] * kq[b,g,j,c],   v[b,g,j,c] = vs[b,g,c] * vq[b,g,j,c].
 *
 * Each query row is quantized to int8 inside the kernel after the key scales
 * are folded into it, every step in IEEE binary32 with round-half-to-even:
 *
 *     u[c]  = q[c] * ks[c],   amax = max_c |u[c]|,
 *     qq[c] = clamp(rint(u[c] * (127 / amax)), -127, 127),   sq = amax / 127
 *     (a zero row: qq = 0, sq = 0),
 *
 * and s_j = scale * sq * sum_c qq[c] * kq[j][c] (an exact integer dot product
 * on int8 matrix instructions).  The softmax, O and lse then follow fa2_fwd
 * with the dequantized v; P and V meet on fp16 matrix instructions (V widened
 * exactly), O is written in `dtype`.
 *
 *   q, o     : [B][Hq][Nq][d], element type `dtype` (bf16 or fp16).
 *   kq, vq   : [B][Hkv][Nk][d] int8 codes (may be NULL when Nk == 0).
 *   ks, vs   : [B][Hkv][d] fp32 scales (required).
 *   lse      : [B][Hq][Nq] fp32.
 *   d        : 64, 128 or 256 (FA2_ERR_HEADDIM otherwise).
 *   Alignment: q, kq, vq, o, ks, vs 16-byte aligned, lse 4-byte.  No output
 *   may overlap an input or the other output.
 *
 * Heads, lengths, causal, packing of query heads, asynchrony and return codes
 * are those of fa2_fwd_ext.
 */
int fa2_fwd_kv_int8(const void* q, const int8_t* kq, const float* ks, const int8_t* vq,
                    const float* vs, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                    void* stream);

/*
 * fa2_fwd_kv_fp8 -- attention over an FP8 key/value cache: the scheme of
 * fa2_fwd_kv_int8 with 8-bit floating-point codes (this library's second
 * reading of the same post title; gfx950 multiplies FP8 matrices at twice the
 * 16-bit rate).  Every code is an OCP FP8 E4M3 value: 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits, exponent field 0 holding the subnormals
 * m * 2^-9, 0x7F and 0xFF NaN (not diagnosed), largest magnitude 448.
 *
 *     k[b,g,j,c] = ks[b,g,c] * e4m3(kq[b,g,j,c]),   v[b,g,j,c] = vs[b,g,c] * e4m3(vq[b,g,j,c]).
 *
 * Each query row is quantized inside the kernel after the key scales are
 * folded into it, every step in IEEE binary32 up to the last rounding:
 *
 *     u[c]  = q[c] * ks[c],   amax = max_c |u[c]|,
 *     qq[c] = e4m3_rne(u[c] * (448 / amax)),   sq = amax / 448
 *     (a zero row: qq = 0, sq = 0),
 *
 * where e4m3_rne rounds to the nearest E4M3 value, ties to the code with an
 * even last mantissa bit (both divisions correctly rounded).  The logits are
 * s_j = scale * sq * sum_c e4m3(qq[c]) * e4m3(kq[j][c]), on FP8 matrix
 * instructions with fp32 sums; the softmax, O and lse follow fa2_fwd with the
 * dequantized v, P and V meeting on fp16 matrix instructions (V widened
 * exactly).
 *
 *   q, o     : [B][Hq][Nq][d], element type `dtype` (bf16 or fp16).
 *   kq, vq   : [B][Hkv][Nk][d] E4M3 codes (may be NULL when Nk == 0).
 *   ks, vs   : [B][Hkv][d] fp32 scales (required).
 *   d        : 64, 128 or 256 (FA2_ERR_HEADDIM otherwise).
 *
 * Alignment, heads, lengths, causal, asynchrony and return codes are those
 * of fa2_fwd_kv_int8.
 */
int fa2_fwd_kv_fp8(const void* q, const uint8_t* kq, const float* ks, const uint8_t* vq,
                   const float* vs, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                   void* stream);

/*
 * fa2_fwd_split -- fa2_fwd_ext with key splits, for calls whose query rows
 * are too few to fill the GPU (decoding, or a short chunk, against a long
 * key/value cache: the inference setting of the Colfax "FlashAttention-3 for
 * Inference" post, title and teaser only).  Each query tile's visible key
 * tiles are divided into `splits` near-equal parts, each run by its own
 * workgroup, which leaves an fp32 partial result in `workspace`: O_s, the
 * output over the part's keys normalised by their own sum, and lse_s, their
 * logsumexp (-inf for a part with no visible key).  A second kernel on the
 * same stream merges them into o and lse:
 *
 *     m = max_s lse_s,  w_s = exp(lse_s - m),
 *     o = sum_s w_s O_s / sum_s w_s,   lse = m + ln sum_s w_s,
 *
 * which is the softmax over the union of the parts' keys, exactly (up to
 * rounding), since each part's weights sum to exp(lse_s).  Results match
 * fa2_fwd_ext up to floating-point rounding (not bit for bit).
 *
 *   q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream:
 *              as in fa2_fwd_ext (16-bit inputs; d = 64, 128 or 256).
 *   splits   : 1..128 key parts per query tile (a part may get no key tile:
 *              then it contributes nothing), 1 = fa2_fwd_ext itself, or 0 =
 *              chosen here: enough parts for one workgroup per compute unit
 *              of the current device over the call's 128-row query tiles,
 *              and at least 2 when each K/V head has at most 64 query rows
 *              (Hq / Hkv * Nq) and at least 64 key tiles (of 32 keys; 64
 *              at d = 64), each part keeping at least 8 key tiles (1 if
 *              that leaves one part).  The
 *              choice queries the device's compute-unit count
 *              (a HIP attribute query, after every argument check except the
 *              workspace's).
 *   workspace: device memory of at least fa2_fwd_split_workspace(...) bytes
 *              for the same arguments (cache = 0), 16-byte aligned, overlapping no
 *              input or output; unused (may be NULL) when the call runs
 *              without splits.  The caller owns it; its contents are scratch
 *              (overwritten, never read before written), and two calls in
 *              flight at once need two workspaces.
 *   workspace_bytes: its size in bytes.
 *
 * Returns FA2_OK or a negative fa2_status: those of fa2_fwd_ext, and
 * FA2_ERR_OPTION (splits out of range), FA2_ERR_WORKSPACE (workspace NULL or
 * smaller than needed), FA2_ERR_ALIGN, FA2_ERR_ALIAS (workspace overlapping
 * an input or output).  B*Hq*Nq == 0 returns FA2_OK and touches nothing.
 */
int fa2_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                  float scale, int causal, int dtype, int splits, void* workspace,
                  int64_t workspace_bytes, void* stream);

/*
 * fa2_fwd_split_workspace -- bytes of workspace fa2_fwd_split (cache = 0) or
 * fa2_fwd_kv_split (cache = FA2_CACHE_INT8 or FA2_CACHE_FP8) needs
 * for these arguments: splits * B*Hq*Nq * (d + 1) * 4 (the partial outputs,
 * then the partial logsumexps), or 0 when the call runs without splits.
 * With splits = 0 the count is chosen as those calls choose it on the
 * current device (one workgroup per compute unit, two for a quantized
 * cache).  Returns the byte count (>= 0) or a negative fa2_status for
 * arguments those calls would reject (shape, head dimension, dtype, causal,
 * cache, splits).
 */
int64_t fa2_fwd_split_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                int64_t d, int causal, int dtype, int cache, int splits);

/*
 * fa2_fwd_kv_split -- key splits (as in fa2_fwd_split) over a quantized
 * key/value cache: the operation of fa2_fwd_kv_int8 (cache = FA2_CACHE_INT8)
 * or fa2_fwd_kv_fp8 (cache = FA2_CACHE_FP8), for decoding against a long
 * INT8 or FP8 cache.  Each part quantizes its query rows exactly as the
 * unsplit call does, so the parts' logits are those of fa2_fwd_kv_int8 /
 * fa2_fwd_kv_fp8; their partials are merged as in fa2_fwd_split.
 *
 *   q, kq, ks, vq, vs, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
 *   dtype, stream: as in fa2_fwd_kv_int8 (kq, vq void: int8 or E4M3 codes).
 *   cache    : an fa2_cache (FA2_ERR_OPTION otherwise).
 *   splits, workspace, workspace_bytes: as in fa2_fwd_split (splits = 0
 *              targets two workgroups per compute unit here); the workspace
 *              size is fa2_fwd_split_workspace(B, Hq, Hkv, Nq, Nk, 128,
 *              causal, dtype, cache, splits).
 *
 * Returns the codes of fa2_fwd_kv_int8 and fa2_fwd_split.
 */
int fa2_fwd_kv_split(const void* q, const void* kq, const float* ks, const void* vq,
                     const float* vs, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, int dtype,
                     int cache, int splits, void* workspace, int64_t workspace_bytes,
                     void* stream);

/*
 * fa2_fwd_split_noalloc -- fa2_fwd_split for callers that cannot allocate
 * device memory, not even a workspace to pass in (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * partials go to a fixed scratch array of 16 MiB in the library's device
 * memory, one per GPU, held until the process ends; the call allocates
 * nothing.  Its first call on a device (with that device current) looks up
 * that device's array.
 *
 *   Arguments as in fa2_fwd_split, without workspace and workspace_bytes.
 *   A call whose partials (fa2_fwd_split_workspace bytes for the same
 *   arguments) exceed 16 MiB returns FA2_ERR_SCRATCH and launches nothing;
 *   e.g. with d = 128 that is splits * B*Hq*Nq above 32513 rows.  With
 *   splits = 0 the library's count is lowered instead to the most parts
 *   that fit, or to none (fa2_fwd_ext) when two do not.
 *
 * Every call on one GPU shares that GPU's array, and a call only writes
 * partials before reading them (nothing needs to start at zero), so calls
 * in sequence on one stream are safe; calls that overlap in time on one GPU
 * (other streams, other host threads) race on the array and may corrupt
 * each other's results.  Returns the codes of fa2_fwd_split, FA2_ERR_SCRATCH,
 * or FA2_ERR_HIP if the array's address cannot be looked up.
 */
int fa2_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                          int64_t d, float scale, int causal, int dtype, int splits,
                          void* stream);

/* Static description of a status code (never NULL). */
const char* fa2_strerror(int status);

/*
 * fa2_tile_config -- the tile shape fa2_fwd uses for head dimension d and
 * dtype: *block_q query rows per workgroup, *block_k key rows per K/V tile,
 * *waves wavefronts (of 64 lanes) per workgroup.  At d = 128 a call with at
 * most 1024 keys uses half the waves and query rows instead (two workgroups
 * then share a compute unit), unless it is large enough for one persistent
 * workgroup per compute unit; so does a call whose full-height workgroups
 * would be fewer than the compute units.  Persistent workgroups (one per
 * compute unit, each walking several query tiles) hold 256 query rows with 8
 * waves at d = 64 (non-causal) and d = 128 (also causal, tiles taken in
 * pairs of equal total cost).  At d = 256 each wave holds 16 query rows
 * (16x16x32 matrix instructions), elsewhere 32.  A call whose K/V heads
 * have at most 128 query rows each (Hq / Hkv * Nq, as in decoding) runs on
 * the 128-row tiles of the key-split kernels, as one part: over a quantized
 * cache always, with 16-bit K/V once B*Hkv is at least the number of
 * compute units.  Over a quantized cache at d = 64 or 128 any call whose
 * 256-row workgroups would be fewer than the compute units does the same.
 * block_q here is
 * always a multiple of the smaller shapes and divides the larger.
 * Host-only, no HIP call.  Returns FA2_OK, FA2_ERR_HEADDIM, FA2_ERR_DTYPE or
 * FA2_ERR_NULL.
 */
int fa2_tile_config(int64_t d, int dtype, int* block_q, int* block_k,
                    int* waves);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
