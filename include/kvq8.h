/*
 * kvq8.h -- C ABI of the int8 / int4 KV-cache decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes single-query (decode) attention over a paged KV cache
 * whose keys and values are stored as int8 codes with one float32 step per
 * (token, kv-head) row of 128 values, and fills that cache from float K/V
 * (the write path).  An int4 group variant keeps older tokens as 4-bit codes.
 *
 * Sources, cited by short name:
 *   [P1] "Day 9-3: q8 KV precision comparison" (jianying88.com news/32654):
 *        Sec. 2 states the per-(token, head) max-abs/127 rule.
 *   [P2] "0.8MB runs Qwen part 9-1: q8 KV halves cache and decode bandwidth"
 *        (developer.aliyun.com article 1767759): Sec. 2 gives the allocation
 *        (paged int8 blocks of kv_bs tokens, one float scale per token per
 *        head) and the write path that quantizes each new token's heads.
 *   [P3] "Day 9-2: flash_attn_single_q_q8_neon" (dtytms.com news/32657):
 *        Sec. 2 gives the decode kernel's arguments and its three segments
 *        (query quantized once in 32-blocks; integer block dot products
 *        scaled afterwards, online softmax, int8 V times float weights;
 *        one division at the end).
 *   [P4] "UltraQuant 4-bit KV cache on AMD" (seekfood.cn news/2668800):
 *        Sec. 3.2 group-64 asymmetric INT4 with scale and zero point,
 *        Sec. 3.3 higher precision for recent tokens, Sec. 5.2 the scale
 *        floor and zero-point range.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - Pointers marked (device) are HIP device pointers; (host) are host
 *    pointers.  The caller owns every buffer.  The library keeps no global
 *    state and allocates no memory.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without synchronizing.  Results are valid
 *    once the stream has reached that point.
 *  - Arguments are validated on the host before anything is launched; a
 *    violation returns a negative status and launches nothing.  A launch
 *    that the runtime rejects returns KVQ8_EHIP; the status is that of this
 *    call's own launches (an error left pending by an earlier, unrelated
 *    HIP call is neither reported nor cleared).
 *  - Device-side index data (slots, block tables, context lengths) is
 *    bounds-checked in the kernels: a slot or block id outside the pool is
 *    skipped (the token is neither written nor read) and context lengths are
 *    clamped to [0, min(max_ctx_len, max_blocks_per_seq * kv_bs)].
 *  - hd (head dimension) must be 128.  kv_bs (tokens per cache block) must
 *    be a power of two in [8, 1024].  nq must be a multiple of nkv and
 *    nq / nkv in [1, 8]; query head h reads kv-head h / (nq / nkv).
 *
 * Cache layout (the pages' token-major paged layout, [P2] Sec. 2, [P3] Sec. 2)
 * --------------------------------------------------------------------------
 *  int8 codes   cache[n_blocks][kv_bs][nkv * 128]
 *  float steps  scale[n_blocks][kv_bs][nkv]
 *  Token t of sequence b lives in block  block_tables[b][t / kv_bs],  row
 *  t % kv_bs.  A "slot" is block_id * kv_bs + row; with an identity block
 *  table the step array is the pages' [max_seq][nkv] array byte for byte.
 *  The codes of slot s form one row of nkv x 128 bytes, in which kv-head kh
 *  sits at column  (kh & ~(P - 1)) | ((kh + s) & (P - 1))  (byte offset
 *  128 times that), P = the largest power of two dividing nkv, at most 8:
 *  within each aligned group of P heads the heads rotate with the slot
 *  (nkv odd: column kh, the pages' order).  Every kernel reading or writing
 *  int8 code rows uses this order; it spreads each head's rows over all
 *  column positions, which the memory system serves faster than one fixed
 *  column of many rows.
 */
#ifndef KVQ8_H
#define KVQ8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum kvq8_status {
    KVQ8_OK = 0,
    KVQ8_EINVAL = -1,     /* null pointer, negative count, unknown dtype */
    KVQ8_ESHAPE = -2,     /* unsupported hd, kv_bs, head grouping or chunk */
    KVQ8_EWORKSPACE = -3, /* workspace missing or smaller than required */
    KVQ8_EHIP = -4        /* a HIP launch or runtime call failed */
};

/* Element types of float inputs to the write paths. */
enum kvq8_dtype { KVQ8_F32 = 0, KVQ8_BF16 = 1, KVQ8_F16 = 2 };

/* A static, NUL-terminated description of a status code. */
const char* kvq8_status_string(int status);

/* Library version, e.g. "kvq8 1.0 gfx950". */
const char* kvq8_version(void);

/*
 * kvq8_quantize_append -- the write path ([P2] Sec. 2; rule of [P1] Sec. 2).
 *
 * For each new token i and kv-head kh, quantizes the 128-value K row and the
 * 128-value V row independently: amax = max |x| (amax < 1e-6 is replaced by
 * 1); step d = amax / 127 (IEEE float32 division); code = roundf(x / d)
 * (IEEE division, ties away from zero) clamped to [-127, 127].  Codes go to
 * the cache at slots[i], the step to scale[slots[i]][kh].  All arithmetic is
 * float32; results are bit-exact across runs.  (The codes are those of the
 * division; the kernel rounds x times a reciprocal of d and divides only
 * where that product is near a half-integer, the one place the two can
 * round apart.  The int4 and Q4_0 write paths do the same.)
 *
 *   k_cache, v_cache  (device) int8 [n_blocks][kv_bs][nkv * hd] in the storage
 *                     order above, written
 *   k_scale, v_scale  (device) float [n_blocks][kv_bs][nkv], written
 *   k_new, v_new      (device) [n_tokens][nkv][hd] of `dtype` (KVQ8_F32,
 *                     KVQ8_BF16 or KVQ8_F16), read; 16-byte aligned
 *   slots             (device) int32 [n_tokens]: block_id * kv_bs + row;
 *                     a slot outside [0, n_blocks * kv_bs) is skipped
 *   n_tokens          may be 0 (nothing is launched)
 * Errors: KVQ8_ESHAPE for hd != 128, an invalid kv_bs (a power of two in
 * [8, 1024]), nkv < 1, n_blocks < 1, n_tokens * nkv * 2 rows above
 * 2^31 - 65, or a pool of 2^32 or more rows (n_blocks * kv_bs * nkv; such
 * a pool would hold 512 GiB of codes); KVQ8_EINVAL for a null or misaligned
 * pointer, a bad dtype or n_tokens < 0.  Tokens with equal slots race (one
 * of them wins).
 */
int kvq8_quantize_append(int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                         int n_blocks, int kv_bs, int nkv, int hd,
                         const void* k_new, const void* v_new, int dtype, int n_tokens,
                         const int32_t* slots, void* stream);

/*
 * kvq8_decode_chunk_tokens -- the context chunk (tokens per split-K work
 * item) that kvq8_decode_attn uses when called with chunk = 0.  A multiple
 * of 256.  Pure host arithmetic.
 */
int kvq8_decode_chunk_tokens(int batch, int nkv, int max_ctx_len);

/*
 * kvq8_decode_workspace_size -- bytes of device workspace kvq8_decode_attn
 * needs for these sizes (chunk = 0 selects the default chunk).  Returns 0
 * for invalid sizes.  Pure host arithmetic.
 */
size_t kvq8_decode_workspace_size(int batch, int nq, int nkv, int max_ctx_len, int chunk);

/*
 * kvq8_decode_attn -- single-query decode attention over the int8 cache
 * ([P3] Sec. 1-2, generalized to a batch of sequences, paged blocks and
 * grouped query heads).
 *
 * For sequence b and query head h (kv-head kh = h / (nq / nkv)):
 *   1. the query row is quantized once in four 32-value blocks: qm = max |q|
 *      (qm < 1e-6 -> 1), block scale qsc = qm * (1/127), codes
 *      roundf(q * (127 / qm)) clamped to [-128, 127]   ([P3] Sec. 2 seg. 1);
 *   2. token t's score is sm_scale * kstep_t * sum_b qsc_b * dot_b with
 *      dot_b the int32 dot product of block b's query and key codes
 *      ([P3] Sec. 2 seg. 2);
 *   3. out = sum_t softmax(score)_t * vstep_t * vcodes_t
 *      ([P3] Sec. 2 seg. 2-3).
 * The context is split into chunks processed in parallel, each keeping its
 * own running max and sum (online softmax per chunk); a second kernel merges
 * the chunks and divides by the total sum.  The integer dot products and the
 * value accumulation run on the matrix cores (each weight is carried as an
 * f16 high part of 11 significant bits plus the f16 of the remainder,
 * rounded toward zero, together within 2^-21 relative); accumulation is
 * float32 and the result
 * matches the exact float64 value of the definition to about 1e-5 relative.
 * A sequence with context length 0 gets a zero output row.  The pool may
 * hold at most 2^32 - 1 rows (n_blocks * kv_bs * nkv), else KVQ8_ESHAPE.
 *
 *   out               (device) float [batch][nq][hd], written
 *   q                 (device) float [batch][nq][hd], read; 16-byte aligned
 *   k_cache, v_cache  (device) int8 [n_blocks][kv_bs][nkv * hd] in the storage
 *                     order above, read
 *   k_scale, v_scale  (device) float [n_blocks][kv_bs][nkv], read
 *   block_tables      (device) int32 [batch][max_blocks_per_seq]
 *   ctx_lens          (device) int32 [batch]
 *   max_ctx_len       (host) an upper bound of ctx_lens; sizes the grid
 *   sm_scale          score scale; 0 or a negative value selects the
 *                     method's 1 / sqrt(hd) ([P1] Sec. 1-2); NaN or an
 *                     infinite value returns KVQ8_EINVAL
 *   chunk             tokens per work item: 0 (default) or a multiple of
 *                     256; must equal the value given to
 *                     kvq8_decode_workspace_size
 *   workspace         (device) at least kvq8_decode_workspace_size(...)
 *                     bytes, 16-byte aligned; contents need no
 *                     initialization and are overwritten
 */
int kvq8_decode_attn(float* out, const float* q, int batch, int nq,
                     const int8_t* k_cache, const int8_t* v_cache,
                     const float* k_scale, const float* v_scale,
                     int n_blocks, int kv_bs, int nkv, int hd,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* ctx_lens, int max_ctx_len, float sm_scale,
                     int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq8_decode_attn_noalloc -- kvq8_decode_attn for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, computation and results as kvq8_decode_attn (bit for bit,
 * with the same chunk), without `workspace` and `workspace_bytes`: the chunk
 * partials go to a library-owned device array of KVQ8_DECODE_SCRATCH_BYTES
 * (16 MiB) that every device the library runs on holds until the process
 * ends.  Its address is looked up on the first call on each device (the
 * current device); the call allocates nothing and frees nothing.
 *
 * Limits and errors: sizes whose kvq8_decode_workspace_size exceeds
 * KVQ8_DECODE_SCRATCH_BYTES return KVQ8_EWORKSPACE (nothing launched);
 * a `stream` that belongs to a device other than the current one returns
 * KVQ8_EINVAL; other errors as for kvq8_decode_attn.  All calls on one
 * device share that device's array and nothing needs clearing between them
 * (each call writes every partial it reads), but calls whose executions
 * overlap on one device -- on different streams, or in different threads
 * without stream ordering -- race on it: order them on one stream.
 */
#define KVQ8_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

int kvq8_decode_attn_noalloc(float* out, const float* q, int batch, int nq,
                             const int8_t* k_cache, const int8_t* v_cache,
                             const float* k_scale, const float* v_scale,
                             int n_blocks, int kv_bs, int nkv, int hd,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* ctx_lens, int max_ctx_len, float sm_scale,
                             int chunk, void* stream);

/*
 * kvq8_append_decode_attn -- one decode step of a layer: the write path for
 * each sequence's newest token, then decode attention over its whole
 * context, in one pass over the cache ([P2] Sec. 2 write path followed by
 * [P3] Sec. 2, as the layer runs them).
 *
 * Sequence b's newest token is at position ctx_lens[b] - 1; its K and V rows
 * (k_new[b], v_new[b], [nkv][hd] of `dtype`) are quantized exactly as
 * kvq8_quantize_append does, stored in the slot the block table assigns to
 * that position (skipped when the block id is outside the pool), and used
 * by the attention.  The cache bytes and the output equal those of
 * kvq8_quantize_append followed by kvq8_decode_attn.  Sequences with
 * ctx_lens[b] = 0 write nothing and get a zero row.  A sequence whose
 * ctx_lens[b] exceeds the bound (max_ctx_len, or max_blocks_per_seq * kv_bs)
 * is attended over the clamped length like in kvq8_decode_attn, and its new
 * token, which lies past that length, is not written: no cached token is
 * overwritten.  Other arguments as for
 * kvq8_decode_attn (same workspace size); the cache pools are written.
 */
int kvq8_append_decode_attn(float* out, const float* q, int batch, int nq,
                            const void* k_new, const void* v_new, int dtype,
                            int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale,
                            int n_blocks, int kv_bs, int nkv, int hd,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* ctx_lens, int max_ctx_len, float sm_scale,
                            int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq8_quantize_q -- step 1 of kvq8_decode_attn alone, exported so that the
 * query codes and block scales can be checked bit for bit ([P3] Sec. 2
 * seg. 1).  Runs the same device code the decode kernel runs.
 *
 *   qi    (device) int8 [n_vectors][hd], written
 *   qsc   (device) float [n_vectors][hd / 32], written
 *   q     (device) float [n_vectors][hd], read; 16-byte aligned
 */
int kvq8_quantize_q(int8_t* qi, float* qsc, const float* q, int n_vectors, int hd, void* stream);

/*
 * kvq8_qk_partials -- the int32 block dot products of step 2 for every
 * (sequence, query head, token), exported for bit-exact checking
 * ([P3] Sec. 2 seg. 2).  Runs the same tile loader and dot-product code the
 * decode kernel runs.
 *
 *   partials  (device) int32 [batch][nq][max_ctx_len][4], written for
 *             t < ctx_len (clamped as above); other entries are untouched
 *   remaining arguments as for kvq8_decode_attn
 */
int kvq8_qk_partials(int32_t* partials, const float* q, int batch, int nq,
                     const int8_t* k_cache, int n_blocks, int kv_bs, int nkv, int hd,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* ctx_lens, int max_ctx_len, void* stream);

/* ------------------------------------------------------------------------
 * int4 group variant ([P4] Sec. 3.2, 3.3)
 *
 * int4 pool layout (head-major inside each block: the kv_bs rows of one
 * (block, kv-head) are contiguous, so a decode work item, which reads one
 * kv-head, reads whole cache lines):
 *   packed codes  cache4[n_blocks4][nkv][kv_bs][64] uint8, two consecutive
 *                 codes per byte, even-indexed value in the high nibble;
 *                 key rows hold the pair starting at element 64h + 16c + 2j
 *                 (h = 0, 1; c = 0..3; j = 0..7) in byte 16c + 8h + j, value
 *                 rows hold the pair starting at element 64g + 4m + 2k in
 *                 byte 4m + 2g + k
 *   scale, zero   [n_blocks4][nkv][kv_bs][2] IEEE binary16 (as uint16 bits),
 *                 one per 64-value group
 * Slot s = block * kv_bs + offset of kv-head kh is row (block * nkv + kh) *
 * kv_bs + offset of each array.  Recent tokens stay in an int8 pool laid
 * out as above ([n_blocks][kv_bs][nkv * 128]).
 * ------------------------------------------------------------------------ */

/*
 * kvq4_quantize_append -- int4 write path ([P4] Sec. 3.2 with the
 * Sec. 5.2 checklist).  Per 64-value group: scale = (max - min) / 15 in
 * float32 (1.0 when max == min), floored at 1e-7 and rounded to binary16;
 * with s the stored binary16 scale, zero = clamp(rint(-min / s), 0, 15)
 * (stored as binary16, exact); code = clamp(rint(x / s + zero), 0, 15);
 * rint is round-half-to-even.  Value rows store the pair of elements
 * 64g + 4m + 2k, 64g + 4m + 2k + 1 (group g, m = 0..15, k = 0, 1) at byte
 * 4m + 2g + k, key rows the pair 64h + 16c + 2j, +1 (h = 0, 1, c = 0..3,
 * j = 0..7) at byte 16c + 8h + j; in both the even element is in the high
 * nibble.  Arguments and errors as for
 * kvq8_quantize_append.
 */
int kvq4_quantize_append(uint8_t* k_cache, uint8_t* v_cache,
                         uint16_t* k_scale, uint16_t* k_zero, uint16_t* v_scale, uint16_t* v_zero,
                         int n_blocks, int kv_bs, int nkv, int hd,
                         const void* k_new, const void* v_new, int dtype, int n_tokens,
                         const int32_t* slots, void* stream);

/*
 * kvq4_requantize_q8 -- move tokens from the int8 pool (the recent window)
 * into the int4 pool as they age ([P4] Sec. 3.3 practical notes: the oldest
 * time block is re-quantized from 8-bit to 4-bit as the sequence grows,
 * off the decode's critical path).
 *
 * Pair i reads int8 slot src_slots[i] (block id * kv_bs + offset) of both
 * the K and the V pool, takes the values code * step (one float32
 * multiplication each) and writes them to int4 slot dst_slots[i] exactly as
 * kvq4_quantize_append would write those float32 values.  A pair with either
 * slot outside its pool is skipped.  The int8 pool is only read, so a
 * decode may keep using it until the caller switches the tokens' table
 * entries.
 *
 *   k_cache4 .. v_zero4  (device) the int4 pool as in kvq4_quantize_append,
 *                        written; caches 16-byte aligned
 *   k_cache8 .. v_scale8 (device) the int8 pool as in kvq8_quantize_append,
 *                        read; caches 16-byte aligned
 *   n_blocks4, n_blocks8 blocks in each pool (same kv_bs and nkv)
 *   src_slots, dst_slots (device) int32 [n_tokens]
 *
 * Returns KVQ8_ESHAPE for a bad hd, kv_bs or nkv, for more than 2^31 - 129
 * rows (n_tokens * nkv * 2: rows are indexed with 32-bit integers) and for a
 * destination pool of 2^32 or more rows (n_blocks * kv_bs * nkv), and
 * KVQ8_EINVAL for a null or misaligned pointer or n_tokens < 0.
 */
int kvq4_requantize_q8(uint8_t* k_cache4, uint8_t* v_cache4, uint16_t* k_scale4, uint16_t* k_zero4,
                       uint16_t* v_scale4, uint16_t* v_zero4, int n_blocks4,
                       const int8_t* k_cache8, const int8_t* v_cache8,
                       const float* k_scale8, const float* v_scale8, int n_blocks8,
                       int kv_bs, int nkv, int hd, int n_tokens,
                       const int32_t* src_slots, const int32_t* dst_slots, void* stream);

/* Default chunk and workspace size for kvq4_decode_attn (see the kvq8
 * counterparts).  max_len4 / max_len8 bound lens4 / lens8. */
int kvq4_decode_chunk_tokens(int batch, int nkv, int max_len4, int max_len8);
size_t kvq4_decode_workspace_size(int batch, int nq, int nkv, int max_len4, int max_len8, int chunk);

/*
 * kvq4_decode_attn -- decode attention over a sequence split between an
 * int4 pool (older tokens; lens4[b] of them, positions 0.. through
 * block_tables4) and an int8 pool (the recent window; lens8[b] tokens
 * through block_tables8).  Attention does not depend on token order, so
 * the split only sets each token's precision ([P4] Sec. 2.2, 3.3).
 *
 * The query is quantized as in kvq8_decode_attn.  For an int4 key row with
 * codes c, group scale s_g and zero z_g, block b's score term is
 * qsc_b * s_g * (P_b - z_g * R_b) with P_b = sum qi * c and R_b = sum qi
 * (int32); values contribute weight * s_g * (c - z_g).  Both pools' chunks
 * are merged as in kvq8_decode_attn.  Both products run on the matrix cores
 * (the int4 values enter as c - z_g, exact in f16; the weights p * s_g as in
 * kvq8_decode_attn).  Other arguments as there; the int4 and int8 pools
 * share kv_bs and nkv.  The four binary16 arrays (k_scale4 .. v_zero4) must
 * be 4-byte aligned (a row's two groups are read as one word), else
 * KVQ8_EINVAL; each pool may hold at most 2^32 - 1 rows, else KVQ8_ESHAPE.
 */
int kvq4_decode_attn(float* out, const float* q, int batch, int nq,
                     const uint8_t* k_cache4, const uint8_t* v_cache4,
                     const uint16_t* k_scale4, const uint16_t* k_zero4,
                     const uint16_t* v_scale4, const uint16_t* v_zero4,
                     int n_blocks4, const int32_t* block_tables4, int max_blocks_per_seq4,
                     const int32_t* lens4, int max_len4,
                     const int8_t* k_cache8, const int8_t* v_cache8,
                     const float* k_scale8, const float* v_scale8,
                     int n_blocks8, const int32_t* block_tables8, int max_blocks_per_seq8,
                     const int32_t* lens8, int max_len8,
                     int kv_bs, int nkv, int hd, float sm_scale,
                     int chunk, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Q4_0 KV mode ([P2] Sec. 1 and Sec. 3: the --kv-q4 switch, a Q4_0 payload
 * cache about 1.65x denser than q8 whose decode dot reads the nibbles
 * without dequantizing them).
 *
 * A (token, kv-head) row of 128 values is four blocks of 32.  Per block:
 * step = m / -8 (float32, exact) where m is the value of largest magnitude
 * (the negative one when a positive and a negative value tie); a block of
 * zeros has step +0 and all codes 8; otherwise
 * code = min(15, floor(x / step + 8.5)) with an IEEE float32 division and
 * one float32 addition, and the value it stands for is (code - 8) * step.
 * 64 code bytes + 4 float32 steps = 80 B per row (q8: 132 B, 1.65x).
 *
 * Pools (caller-owned device memory, 16-byte aligned):
 *   k_cache, v_cache  uint8 [n_blocks][nkv][kv_bs][64], two codes per byte:
 *                     key row byte j = code[j] | code[64 + j] << 4;
 *                     value row byte 4m + k = code[32k + 2m] |
 *                     code[32k + 2m + 1] << 4  (k = 0..3, m = 0..15);
 *                     rows head-major inside each block as in the int4
 *                     pool: slot s = block * kv_bs + offset of kv-head kh
 *                     is row (block * nkv + kh) * kv_bs + offset
 *   k_step, v_step    float32 [n_blocks][nkv][kv_bs][4], one per block,
 *                     rows in the same order
 * ------------------------------------------------------------------------ */

/*
 * kvq4_0_quantize_append -- Q4_0 write path: quantize n_tokens new rows of
 * K and V (k_new, v_new [n_tokens][nkv][128], 16-byte aligned, dtype as in
 * kvq8_quantize_append) into slot slots[i] = block * kv_bs + offset.  Slots
 * outside [0, n_blocks * kv_bs) are skipped.  Errors: KVQ8_ESHAPE for
 * hd != 128, an invalid kv_bs (a power of two in [8, 1024]), nkv < 1 or
 * n_blocks < 1; KVQ8_EINVAL for a null or misaligned pointer, a bad dtype
 * or n_tokens < 0; KVQ8_ESHAPE also for more than 2^31 - 129 rows
 * (n_tokens * nkv * 2) and for a pool of 2^32 or more rows (n_blocks *
 * kv_bs * nkv; such a pool would hold over 320 GiB).  n_tokens == 0
 * enqueues nothing.
 */
int kvq4_0_quantize_append(uint8_t* k_cache, uint8_t* v_cache, float* k_step, float* v_step,
                           int n_blocks, int kv_bs, int nkv, int hd,
                           const void* k_new, const void* v_new, int dtype, int n_tokens,
                           const int32_t* slots, void* stream);

/* Default chunk and workspace size for kvq4_0_decode_attn (see the kvq8
 * counterparts; the same rules). */
int kvq4_0_decode_chunk_tokens(int batch, int nkv, int max_ctx_len);
size_t kvq4_0_decode_workspace_size(int batch, int nq, int nkv, int max_ctx_len, int chunk);

/*
 * kvq4_0_decode_attn -- decode attention over the Q4_0 cache.  The query is
 * quantized as in kvq8_decode_attn (int8 codes qi and a float32 scale qsc
 * per 32-block); the score of a token is
 *   sm_scale * sum_b qsc_b * kstep_b * (P_b - 8 R_b),
 *   P_b = sum over block b of qi * code (int32),  R_b = sum of qi (int32),
 * i.e. the dot product of the dequantized query and key, taken without
 * dequantizing; values contribute weight * vstep_b * (code - 8).  Split-K
 * chunks and merge as in kvq8_decode_attn; both products run on the matrix
 * cores.  Arguments, workspace, errors and the 2^32 - 1 row limit as in
 * kvq8_decode_attn, with the pools above (k_step / v_step 16-byte aligned).
 */
int kvq4_0_decode_attn(float* out, const float* q, int batch, int nq,
                       const uint8_t* k_cache, const uint8_t* v_cache,
                       const float* k_step, const float* v_step,
                       int n_blocks, int kv_bs, int nkv, int hd,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* ctx_lens, int max_ctx_len, float sm_scale,
                       int chunk, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * 2-bit band of the group variant ([P4] Sec. 2.2 time-adaptive bits and
 * Sec. 3.3 band schedule: the oldest tokens take 2 bits, the middle band
 * int4, the recent window int8; the page's example edges are 2048 and 16384
 * tokens from the newest).  The caller decides which tokens sit in which
 * band through the three pools' block tables and lengths.
 *
 * Codes: the [P4] Sec. 3.2 group quantizer with two bits, on groups of 64
 * values: scale = (max - min) / 3 in float32 (1.0 when max == min), floored
 * at 1e-7 and rounded to binary16; with s the stored binary16 scale,
 * zero = clamp(rint(-min / s), 0, 3) (stored as binary16, exact);
 * code = clamp(rint(x / s + zero), 0, 3); rint rounds half to even; the
 * value a code stands for is (code - zero) * s.
 *
 * 2-bit pool layout (this library's packing, four codes per byte; rows
 * head-major inside each block as in the int4 pool):
 *   packed codes  cache2[n_blocks2][nkv][kv_bs][32] uint8;
 *                 key rows: 32-bit word 2g + h holds element
 *                 64h + 16g + 4k + j at bits 8j + 2k (g, j, k = 0..3);
 *                 value rows: 16-bit word m holds element
 *                 64(s / 4) + 4m + s % 4 at bits 2s (s = 0..7, m = 0..15)
 *   scale, zero   [n_blocks2][nkv][kv_bs][2] IEEE binary16 (as uint16 bits)
 * 32 + 32 code bytes + 8 + 8 scale / zero bytes = 80 B per (token, kv-head)
 * (int4: 144 B, int8: 264 B).
 * ------------------------------------------------------------------------ */

/*
 * kvq2_quantize_append -- 2-bit write path: quantize n_tokens new rows of K
 * and V (k_new, v_new [n_tokens][nkv][128], 16-byte aligned, dtype as in
 * kvq8_quantize_append) into 2-bit slot slots[i] = block * kv_bs + offset.
 * Arguments, skipped slots and errors as for kvq4_quantize_append.
 */
int kvq2_quantize_append(uint8_t* k_cache, uint8_t* v_cache,
                         uint16_t* k_scale, uint16_t* k_zero, uint16_t* v_scale, uint16_t* v_zero,
                         int n_blocks, int kv_bs, int nkv, int hd,
                         const void* k_new, const void* v_new, int dtype, int n_tokens,
                         const int32_t* slots, void* stream);

/*
 * kvq2_requantize_q4 -- move tokens from the int4 pool into the 2-bit pool
 * as they leave the int4 band ([P4] Sec. 3.3 practical notes: the oldest
 * time block drops to fewer bits, off the decode's critical path).
 *
 * Pair i reads int4 slot src_slots[i] of both the K and the V pool, takes
 * the values (code - zero) * scale (exact in float32) and writes them to
 * 2-bit slot dst_slots[i] exactly as kvq2_quantize_append would write those
 * float32 values.  A pair with either slot outside its pool is skipped; the
 * int4 pool is only read.
 *
 *   k_cache2 .. v_zero2  (device) the 2-bit pool, written; caches 16-byte
 *                        aligned
 *   k_cache4 .. v_zero4  (device) the int4 pool as in kvq4_quantize_append,
 *                        read; caches 16-byte aligned
 *   n_blocks2, n_blocks4 blocks in each pool (same kv_bs and nkv)
 *   src_slots, dst_slots (device) int32 [n_tokens]
 *
 * Errors as for kvq4_requantize_q8 (here either pool of 2^32 or more rows
 * is rejected).
 */
int kvq2_requantize_q4(uint8_t* k_cache2, uint8_t* v_cache2, uint16_t* k_scale2, uint16_t* k_zero2,
                       uint16_t* v_scale2, uint16_t* v_zero2, int n_blocks2,
                       const uint8_t* k_cache4, const uint8_t* v_cache4,
                       const uint16_t* k_scale4, const uint16_t* k_zero4,
                       const uint16_t* v_scale4, const uint16_t* v_zero4, int n_blocks4,
                       int kv_bs, int nkv, int hd, int n_tokens,
                       const int32_t* src_slots, const int32_t* dst_slots, void* stream);

/* Default chunk and workspace size for kvq2_decode_attn (the kvq4 rules over
 * the three bands' lengths together). */
int kvq2_decode_chunk_tokens(int batch, int nkv, int max_len2, int max_len4, int max_len8);
size_t kvq2_decode_workspace_size(int batch, int nq, int nkv, int max_len2, int max_len4, int max_len8,
                                  int chunk);

/*
 * kvq2_decode_attn -- decode attention over a sequence split into three
 * bands: lens2[b] tokens in the 2-bit pool (block_tables2), lens4[b] in the
 * int4 pool (block_tables4) and lens8[b] in the int8 pool (block_tables8).
 * Attention does not depend on token order, so the bands only set each
 * token's precision.
 *
 * A 2-bit key row contributes qsc_b * s_g * (P_b - z_g * R_b) per query
 * block as an int4 row does (P_b = sum qi * c, R_b = sum qi, int32), a
 * value row weight * s_g * (c - z_g); int4 and int8 rows as in
 * kvq4_decode_attn.  All three bands' chunks share one launch and one
 * merge.  The pools share kv_bs and nkv; the eight binary16 arrays must be
 * 4-byte aligned, each pool may hold at most 2^32 - 1 rows; other arguments,
 * workspace and errors as in kvq4_decode_attn.
 */
int kvq2_decode_attn(float* out, const float* q, int batch, int nq,
                     const uint8_t* k_cache2, const uint8_t* v_cache2,
                     const uint16_t* k_scale2, const uint16_t* k_zero2,
                     const uint16_t* v_scale2, const uint16_t* v_zero2,
                     int n_blocks2, const int32_t* block_tables2, int max_blocks_per_seq2,
                     const int32_t* lens2, int max_len2,
                     const uint8_t* k_cache4, const uint8_t* v_cache4,
                     const uint16_t* k_scale4, const uint16_t* k_zero4,
                     const uint16_t* v_scale4, const uint16_t* v_zero4,
                     int n_blocks4, const int32_t* block_tables4, int max_blocks_per_seq4,
                     const int32_t* lens4, int max_len4,
                     const int8_t* k_cache8, const int8_t* v_cache8,
                     const float* k_scale8, const float* v_scale8,
                     int n_blocks8, const int32_t* block_tables8, int max_blocks_per_seq8,
                     const int32_t* lens8, int max_len8,
                     int kv_bs, int nkv, int hd, float sm_scale,
                     int chunk, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ8_H */
