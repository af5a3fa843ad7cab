/*
 * rq.h -- C ABI of the ResidualQuant decode hot path on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of the paper "KV Cache Quantization for Looped
 * Transformers with 2-Bit Residuals" (ResidualQuant); section numbers below
 * refer to it. A looped Transformer produces keys/values X_r for every loop
 * r = 1..L. The cache stores
 *   - an anchor (loop L under the Last-loop policy, §3.2; with loop groups,
 *     one anchor per group), group-quantized in the rotated domain:
 *     A = D(Q(H X_L));
 *   - for every other loop r, a least-squares coefficient
 *     alpha_r = <Z_r, A> / |A|^2 (Z_r = H X_r, stored fp16; §3.2 "Scaling
 *     coefficient", App. G.1) and the group-quantized rotated residual
 *     Q(Z_r - alpha_r A) (§3.2, §3.3), with a bit width chosen per loop (§3.4).
 * Decode rebuilds zhat_r = alpha_r A + D(c_r) tile by tile inside the attention
 * kernel, scores keys against the rotated query H_K q and rotates the value sum
 * back once (§4.1, App. G.2 "Reconstruction and attention"). The current
 * token stays bf16 until the final loop, then all its loops are quantized and
 * appended (§3.2, §4.2 "Decode").
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers unless stated otherwise; the
 *     descriptor and layer-cache structs themselves live in host memory.
 *   - The caller owns all memory. The library never allocates, keeps no state
 *     between calls and may be called from several host threads.
 *   - Every call validates its arguments on the host first; on error it returns
 *     a non-zero rq_status and enqueues nothing. Otherwise it enqueues its
 *     kernels on `stream` (a hipStream_t; NULL = default stream), does not
 *     synchronize, and returns RQ_OK, or RQ_E_HIP if a launch fails. Faults of
 *     enqueued work surface at the caller's next synchronization.
 *   - Token counts that change every step (positions, cached lengths) are read
 *     from device memory by the kernels, so a decode step can be captured once
 *     in a hipGraph and replayed. Kernels clamp them to [0, max_tokens] and, if
 *     `dev_err` (device int32, may be NULL) is given, OR an RQ_DEVERR_* bit into it.
 *   - Alignment of device arrays: codes, rot, kv, q, k_cur, v_cur, k_cache and
 *     v_cache 16 bytes; meta 4 bytes (8 for loops in groups of 16); out 4
 *     bytes; alpha 2 bytes; the workspace 256 bytes. Otherwise the call
 *     returns RQ_E_ALIGN (RQ_E_WORKSPACE for the workspace). Every allocation of the HIP or torch allocators meets this.
 *   - No C++ exception crosses this interface.
 *
 * Data types: bf16 and fp16 values travel as uint16_t bit patterns.
 */
#ifndef RQ_H
#define RQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RQ_MAX_LOOPS 32

typedef enum {
  RQ_OK = 0,
  RQ_E_NULL = 1,         /* a required pointer is NULL */
  RQ_E_SHAPE = 2,        /* batch/heads/head_dim/loops/max_tokens/n out of range */
  RQ_E_BITS = 3,         /* a bit width or group size is not supported */
  RQ_E_CAPACITY = 4,     /* a host-known size exceeds max_tokens */
  RQ_E_WORKSPACE = 5,    /* workspace too small (see rq_workspace_bytes) */
  RQ_E_UNSUPPORTED = 6,  /* valid request this build has no kernel for */
  RQ_E_HIP = 7,          /* a HIP launch failed */
  RQ_E_POLICY = 8,       /* unknown reference policy */
  RQ_E_LOOP = 9,         /* loop index out of range */
  RQ_E_ALIGN = 10,       /* a device array is not aligned as documented below */
  RQ_E_SCRATCH = 11      /* rq_decode_attn_noalloc: the request needs more than RQ_SCRATCH_BYTES */
} rq_status;

/* Device-side error bits (OR-ed into *dev_err when given). */
#define RQ_DEVERR_CAPACITY 1  /* append: pos[b] + n > max_tokens; tokens past capacity were dropped */
#define RQ_DEVERR_LENGTH 2    /* decode: past_len[b] outside [0, max_tokens]; it was clamped */
#define RQ_DEVERR_BLOCK 4     /* paged cache: a block-table entry a token needs is outside [0, num_blocks);
                               * append dropped the token, decode read it as zeros */
#define RQ_DEVERR_RANGE 8     /* append: an offset, scale or LS coefficient fell outside the fp16 range and
                               * was stored as +-65504 (see rq_quantize_append) */

/* Reference policy (§3.2, App. D), applied inside every loop group (see
 * rq_desc.loop_group; by default all L loops form one group).
 * LAST_LOOP: the anchor is the group's last loop; every other loop r of the
 *   group stores Q(Z_r - alpha_r A). Decoding loop r reads two components.
 * FIRST_LOOP: the same with the group's first loop as anchor (§3.2 "Reference
 *   KV": the shared-anchor alternative to Previous-loop; ablated in Table 3).
 * PREV_LOOP: the anchor is the group's first loop; loop r refers to the
 *   reconstruction of loop r-1 (a chain: zhat_r = alpha_r zhat_{r-1} + D(c_r)),
 *   so decoding the j-th loop of a group reads j stored components (App. D).
 *   Kept as the comparator the paper measures against. The decode kernels take
 *   up to 8 components per call, for the chains rq_check_decode describes;
 *   other chains return RQ_E_UNSUPPORTED at decode (their append works). */
typedef enum { RQ_POLICY_LAST_LOOP = 0, RQ_POLICY_PREV_LOOP = 1, RQ_POLICY_FIRST_LOOP = 2 } rq_policy;

/* Decode flag: score the cached keys against the rotated query held in 21-bit
 * instead of 14-bit fixed point (§4.1 keeps softmax in FP32; App. G.2). The
 * query's rounding is the only error of the key path, relative 2^-15 (default)
 * or 2^-22 of each 32-channel group's largest |q'|, so the score error grows
 * with the size of the logits; set the flag for sharp softmax distributions. It
 * costs a few percent of the streaming kernel's time. Decode calls only. */
#define RQ_FLAG_PRECISE_QUERY 1

/* Rotation storage: the matrices rq_layer_cache.rot[kv] (and rq_decode_combine's
 * rot_v) are fp16 instead of fp32, as the learned rotations are stored once
 * calibrated (App. G: fixed matrices kept in FP16, multiplied with FP16 inputs
 * and FP32 accumulation). Every kernel converts the entries to fp32/fp64
 * exactly and keeps its arithmetic, so caches and outputs are bit-identical to
 * those made with an fp32 copy holding the same values; the matrices take half
 * the bytes (half the rotation reads of every decode and append call). A
 * property of the cache: append and decode calls on it must agree. */
#define RQ_FLAG_ROT_F16 2

/* Shapes and the quantization plan of one layer's cache. */
typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t heads;       /* H >= 1 */
  int32_t head_dim;    /* D: 64, 96 or 128 */
  int32_t loops;       /* L: 1 .. RQ_MAX_LOOPS */
  int32_t max_tokens;  /* T_max >= 1: token capacity of every cache buffer */
  int32_t policy;      /* rq_policy */
  int32_t loop_group;  /* G: loops per anchor group; 0 = all L loops form one group, else a divisor of L.
                        * Loops gG .. gG+G-1 (0-based) are quantized against an anchor of their own
                        * (§5 "Models": a model with many loops, e.g. 32, split into groups of 4). */
  int32_t block_size;  /* 0: contiguous cache. Else a paged cache (§4.2: the cache lives in the
                        * serving engine's paged KV blocks): tokens per block, a power of two in
                        * [16, 4096] dividing max_tokens; see rq_layer_cache.block_table */
  int32_t num_blocks;  /* paged cache: blocks in every buffer's pool (>= 1) */
  int32_t flags;       /* RQ_FLAG_PRECISE_QUERY | RQ_FLAG_ROT_F16, or 0 (other bits: RQ_E_SHAPE) */
  uint8_t bits[RQ_MAX_LOOPS];   /* bit width per loop (0-based), 2 or 4 (§2.1, §3.4) */
  uint8_t group[RQ_MAX_LOOPS];  /* group size per loop along the rotated head_dim: 32, or 16 for
                                 * 2-bit loops (§5 "Quantization setup": g = 16 for INT2) */
} rq_desc;

/* Device buffers of one layer's compressed cache. kv index 0 = keys, 1 = values;
 * loop index is 0-based.
 *   codes[kv][r]: uint8 [B][H][T_max][D*bits[r]/8]. Each group of g = group[r]
 *     consecutive channels of the rotated vector occupies g*bits/8 bytes, i.e.
 *     g*bits/32 little-endian 32-bit words. Element e of a group lies in half
 *     h = e/(g/2) at index k = e%(g/2); bits-wide codes fill 16-bit half-words,
 *     16/bits per half-word, element k at bit offset bits*(k%(16/bits)) of
 *     half-word k/(16/bits); 32-bit word j = half-word j of half 0 (bits 0..15)
 *     | half-word j of half 1 (bits 16..31). (Pairs e, e+g/2 share bit
 *     positions, so one mask yields a pair of codes.)
 *   meta[kv][r]: fp16 [B][H][T_max][D/g][2] = (offset o, scale s) per group;
 *     dequantized value = o + s*code (§2.1).
 *   alpha[kv][r]: fp16 [B][H][T_max], the LS coefficient; unused (may be NULL)
 *     for the anchor loop of each group.
 *   rot[kv]: fp32 [H][D][D] row-major (fp16 with RQ_FLAG_ROT_F16), z = rot[h] x.
 *     Any orthogonal matrix works (randomized Hadamard, §2.2, or learned
 *     rotations such as OptR-H, §3.3); the kernels use the entries as given.
 * Paged cache (desc.block_size = BS > 0): every codes, meta and alpha buffer is
 *   a pool [num_blocks][H][BS][row] with the rows above; token t of sequence b,
 *   head h, is row (block_table[b][t / BS] * H + h) * BS + t % BS. Each of a
 *   block's heads thus holds BS consecutive tokens. Every pool buffer must stay
 *   below 4 GiB - 64 KiB (RQ_E_SHAPE otherwise). */
typedef struct {
  uint8_t* codes[2][RQ_MAX_LOOPS];
  uint16_t* meta[2][RQ_MAX_LOOPS];
  uint16_t* alpha[2][RQ_MAX_LOOPS];
  const void* rot[2];
  const int32_t* block_table;  /* paged cache only (else ignored, may be NULL): device int32
                                * [B][max_tokens / block_size]; entry [b][j] is the pool block
                                * holding tokens j*BS .. j*BS+BS-1 of sequence b. Entries covering
                                * tokens an append writes or a decode reads must lie in
                                * [0, num_blocks); others are never read. */
} rq_layer_cache;

/* Bytes of one cache buffer of `loop` for one tensor (K or V): kind 0 = codes,
 * 1 = meta, 2 = alpha. Returns 0 if the descriptor or arguments are invalid. */
size_t rq_buffer_bytes(const rq_desc* desc, int kind, int loop);

/* Bytes of device workspace rq_decode_attn / rq_decode_attn_bf16 need (0 if
 * invalid). The split of the token axis, and so this size, depends on the
 * compute-unit count of the current device. */
size_t rq_workspace_bytes(const rq_desc* desc);

/* Host-side check of a descriptor: RQ_OK or the first problem found. */
rq_status rq_check_desc(const rq_desc* desc);

/* Host-side check that rq_decode_attn / rq_decode_attn_partial have a kernel for
 * decoding loop `loop` (0-based) under desc, its flags included: RQ_OK, a
 * descriptor error as rq_check_desc, RQ_E_LOOP, or RQ_E_UNSUPPORTED. Touches no
 * device. Kernels exist for every decode that reads one or two stored
 * components (every Last-loop and First-loop plan, any widths and group sizes)
 * and for Previous-loop chains of three to eight components whose INT4 loops
 * all come before their INT2 loops, the INT2 loops in one group size (§3.2,
 * §3.4: the descending plans); chains of five to eight need a contiguous cache,
 * at most two INT4 loops and groups of 32. */
rq_status rq_check_decode(const rq_desc* desc, int32_t loop);

/* Quantize and store n tokens per sequence (§4.2 "Prefill" bulk store and
 * "Decode" deferred store; App. G.1 recipe).
 *   kv:  bf16 [2][L][B][H][n][D] keys (index 0) and values (1) of all loops of
 *        n consecutive tokens, original (unrotated) domain.
 *   pos: device int32 [B], the cache position of the first of the n tokens of
 *        each sequence; token i goes to position pos[b] + i.
 * For every (tensor, b, h, token): Z_r = rot x_r (fp64 accumulation), anchor
 * group quantization, alpha_r (fp64, stored fp16 nearest-even), residual
 * E_r = Z_r - alpha_r * ref, group quantization of E_r, packing. Offsets are
 * rounded toward -inf and scales toward +inf to fp16, codes to nearest-even,
 * so every group's range is covered. Tokens at positions >= max_tokens are
 * dropped (RQ_DEVERR_CAPACITY). n == 0 is a no-op.
 * Accepted range: the metadata are fp16, so every rotated value (and every
 * residual E_r) must lie within +-65504 and every group's range within
 * (2^bits - 1) * 65504; LS coefficients must stay below 65504 in magnitude.
 * Outside it, an offset, scale or coefficient whose fp16 rounding overflows is
 * stored as the largest finite fp16 magnitude of its sign (values beyond the
 * group's covered range then clip to the end codes) and RQ_DEVERR_RANGE is set;
 * the cache stays finite. Inputs must be finite bf16. */
rq_status rq_quantize_append(const rq_desc* desc, const rq_layer_cache* cache,
                             const uint16_t* kv, const int32_t* pos, int32_t n,
                             int32_t* dev_err, void* stream);

/* rq_quantize_append for nlayers layers that share one descriptor (§4.2
 * "Decode": the store of the current token is deferred until after the final
 * loop, when every layer's keys and values of all loops are known, so one call
 * can store them for the whole layer stack).
 *   caches: host array of nlayers layer caches (copied during the call).
 *   kv:     bf16 [nlayers][2][L][B][H][n][D], layer l's input as in
 *           rq_quantize_append, the layers back to back.
 *   pos:    as in rq_quantize_append, the same positions for every layer.
 * Each layer's buffers receive exactly the bytes rq_quantize_append(desc,
 * &caches[l], kv + l*2*L*B*H*n*D, pos, n, ...) would write. For n <= 8 (or
 * more than 16 loops) the layers share launches: their cache pointers travel in
 * the kernel arguments, as many layers per launch as fit (16 at 4 loops, 8 at
 * 8 loops); larger n takes one bulk launch per layer. Every cache is checked
 * before the first launch, so an error status means nothing was launched.
 * nlayers == 0 or n == 0 is a no-op; nlayers < 0 is RQ_E_SHAPE. */
rq_status rq_quantize_append_layers(const rq_desc* desc, const rq_layer_cache* caches,
                                    int32_t nlayers, const uint16_t* kv, const int32_t* pos,
                                    int32_t n, int32_t* dev_err, void* stream);

/* Decode attention of loop `loop` (0-based) over the compressed cache plus the
 * current token held in bf16 (§4.1, §4.2 "Decode", App. G.2).
 *   q, k_cur, v_cur: bf16 [B][H][D], original domain (current token's q/k/v of
 *     this loop).
 *   past_len: device int32 [B], cached tokens of each sequence (positions
 *     0 .. past_len[b]-1 are attended, then the current token).
 *   out: fp32 [B][H][D] = softmax(scale [q.k_t ..., q.k_cur]) [v_t ..., v_cur].
 *   workspace: device, >= rq_workspace_bytes(desc) bytes, 256-byte aligned; it
 *     holds the per-split partial results (no initial contents needed). Calls
 *     that share a workspace must not overlap in time.
 * Two kernel launches: every workgroup of the first rotates the query
 * (q' = scale H_K q), scores a contiguous range of cached tokens against the
 * rotated keys and accumulates the rotated value sum; the second merges the
 * ranges of each (b, h) with the current token and applies H_V^T once. */
rq_status rq_decode_attn(const rq_desc* desc, const rq_layer_cache* cache, int32_t loop,
                         const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                         const int32_t* past_len, float softmax_scale, float* out,
                         void* workspace, size_t workspace_bytes, int32_t* dev_err, void* stream);

/* Split of the token axis used by the decode calls (§4.1 "split-K"): every
 * (b, h) has *nsplit slots (chosen from the current device's compute-unit
 * count). Slot i of sequence b covers cached tokens [i*c_b, (i+1)*c_b) with
 * c_b = u * ceil(ceil(past_len[b] / nsplit) / u), at least u, where
 * u = *unit is the kernel's tile; so the slots of every sequence are equally
 * long whatever its length, and slots starting at or past past_len[b] are
 * unused (slot 0 always counts). */
rq_status rq_split_plan(const rq_desc* desc, int32_t* unit, int32_t* nsplit);

/* The two launches of rq_decode_attn as separate calls, for callers that merge
 * partial results themselves (for instance over a token axis split across
 * devices, or with partials of another cache) or time the streaming kernel
 * alone. rq_decode_attn(...) is exactly rq_decode_attn_partial(...) followed by
 * rq_decode_combine(..., cache->rot[1], ...) on the same stream and workspace.
 *
 * rq_decode_attn_partial: rotates q (q' = scale H_K q) and scores the cached
 *   tokens of each slot that holds any of the past_len[b] tokens (slot 0 always
 *   counts, even when past_len[b] == 0). For each such (b, h, slot) it writes
 *   float part[b][h][slot][D + 4] = (m, l, unused, unused, acc[0..D-1]) into
 *   the workspace, with scores x_t = log2(e) * scale * <q', zhat_K,t> over the
 *   slot's tokens, m = max_t x_t (-inf for an empty slot), l = sum_t 2^(x_t - m),
 *   acc = sum_t 2^(x_t - m) zhat_V,t (rotated value domain). Slots past the
 *   last used one are not written. The current token is not included.
 * rq_decode_combine: merges the written slots of each (b, h) with the current
 *   token (score log2(e) * scale * <q, k_cur> in the original domain) and
 *   writes out = (rot_v^T acc + p_cur v_cur) / l, all slots rescaled to one
 *   max. rot_v: [H][D][D] (the cache's value rotation; fp16 when desc has
 *   RQ_FLAG_ROT_F16, else fp32), or NULL when the partials are already in the
 *   original domain (as rq_decode_attn_bf16's are). Only batch, heads, head_dim,
 *   max_tokens and RQ_FLAG_ROT_F16 of desc are used; desc must be the one the
 *   partials were made with. The workspace is only read. */
rq_status rq_decode_attn_partial(const rq_desc* desc, const rq_layer_cache* cache, int32_t loop,
                                 const uint16_t* q, const int32_t* past_len, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, void* stream);
rq_status rq_decode_combine(const rq_desc* desc, const void* rot_v, const uint16_t* q, const uint16_t* k_cur,
                            const uint16_t* v_cur, const int32_t* past_len, float softmax_scale, float* out,
                            const void* workspace, size_t workspace_bytes, int32_t* dev_err, void* stream);

/* rq_decode_attn for callers that cannot allocate device memory (code under
 * hipGraph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, bit for bit, with the split partials kept in a
 * static device array of RQ_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends, instead of a caller workspace. The call
 * allocates nothing. Its first call on a device looks up that device's array
 * (hipGetSymbolAddress, with the device current); make that first call outside
 * stream capture. Requests whose partials, rq_workspace_bytes(desc), exceed
 * RQ_SCRATCH_BYTES return RQ_E_SCRATCH and enqueue nothing. All calls on one
 * GPU share its array and it keeps the last call's contents (nothing in it needs
 * to start at zero): calls that overlap in time on one GPU, from any stream or
 * thread, race and must be ordered by the caller. Other arguments and errors as
 * rq_decode_attn. */
#define RQ_SCRATCH_BYTES (8u << 20)
rq_status rq_decode_attn_noalloc(const rq_desc* desc, const rq_layer_cache* cache, int32_t loop,
                                 const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                                 const int32_t* past_len, float softmax_scale, float* out, int32_t* dev_err,
                                 void* stream);

/* BF16 decode baseline (the paper's comparison point, §5.3): the same attention
 * over an uncompressed cache. k_cache, v_cache: bf16 [B][H][T_max][D]. Only
 * batch, heads, head_dim and max_tokens of desc are used.
 * rq_decode_attn_bf16 is rq_decode_attn_bf16_partial followed by
 * rq_decode_combine(desc, NULL, ...); the partial writes the same slots and
 * layout as rq_decode_attn_partial, in the original (unrotated) domain. */
rq_status rq_decode_attn_bf16_partial(const rq_desc* desc, const uint16_t* k_cache, const uint16_t* v_cache,
                                      const uint16_t* q, const int32_t* past_len, float softmax_scale,
                                      void* workspace, size_t workspace_bytes, void* stream);
rq_status rq_decode_attn_bf16(const rq_desc* desc, const uint16_t* k_cache, const uint16_t* v_cache,
                              const uint16_t* q, const uint16_t* k_cur, const uint16_t* v_cur,
                              const int32_t* past_len, float softmax_scale, float* out,
                              void* workspace, size_t workspace_bytes, int32_t* dev_err, void* stream);

/* Prefill attention of one loop (§4.2 "Prefill"): every prompt token attends
 * causally over the prompt's own BF16 K/V of that loop, before anything is
 * quantized; after the final loop the caller stores the prompt with
 * rq_quantize_append (all loops at once). Row i of a sequence's output is
 * sum_{j <= i} softmax_j(scale <q_i, k_j>) v_j.
 *   q, k, v: bf16 [B][H][n][D] (one loop's prompt), 16-byte aligned;
 *   lens: device int32 [B], the prompt length of each sequence (clamped to
 *     [0, n]; RQ_DEVERR_LENGTH if outside); rows past it are not written;
 *   out: fp32 [B][H][n][D], 16-byte aligned;
 *   workspace: device memory of rq_prefill_workspace_bytes(desc, n) bytes,
 *     256-byte aligned (a first pass writes V transposed in fp16 there).
 * Only batch, heads and head_dim of desc are used (n is the prompt capacity,
 * independent of max_tokens). softmax_scale must be positive (RQ_E_SHAPE).
 * The matrix products run in bf16 (scores) and fp16 (probabilities times
 * values) with fp32 accumulation; values must lie within the fp16 range
 * (|v| < 65504). n == 0 is a no-op. */
size_t rq_prefill_workspace_bytes(const rq_desc* desc, int32_t n);
rq_status rq_prefill_attn(const rq_desc* desc, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* lens, int32_t n, float softmax_scale, float* out, void* workspace,
                          size_t workspace_bytes, int32_t* dev_err, void* stream);

/* Static description of a status code. */
const char* rq_status_str(rq_status status);

/* Library version string. */
const char* rq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RQ_H */
