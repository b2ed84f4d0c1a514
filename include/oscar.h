/*
 * oscar.h — C ABI of liboscar: the OSCAR INT2 KV-cache write and the
 * mixed-precision paged decode attention over that cache, for AMD gfx950.
 *
 * Method: "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV
 * Cache Quantization" (arXiv:2605.17757). Passages are cited by page and
 * section:
 *   [abs]   the arXiv v2 abstract (paperdot.bitmofang.com listing);
 *   [nl]    gist.science/nl technical summary ("Technische Samenvatting");
 *   [fr]    gist.science/fr technical summary ("Résumé technique").
 *
 * Every pointer argument is a plain pointer; "device" means memory the HIP
 * runtime can address on the current device, "host" means CPU memory.
 * The caller owns every buffer; the library allocates no memory on the device
 * (work areas are caller workspaces, sized by the *_workspace_bytes calls,
 * or the fixed scratch array of oscar_decode_attn_noalloc).  Its state is a
 * thread-local error string, a per-device cache of the device check and the
 * scratch array's address.  All calls except the calibration calls are
 * asynchronous on the given stream.
 *
 * Return value: OSCAR_OK (0) or a negative code; oscar_last_error() then
 * holds a message.  Arguments are validated on the host before any launch;
 * a call that fails validation launches nothing.  No call aborts and no C++
 * exception crosses this boundary.
 */
#ifndef OSCAR_H_
#define OSCAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define OSCAR_API __attribute__((visibility("default")))
#else
#define OSCAR_API
#endif

/* hipStream_t without the HIP headers: an opaque stream handle (NULL = the
 * default stream). */
typedef struct ihipStream_t *oscar_stream_t;

/* ---------------------------------------------------------------------------
 * Fixed shape of the cache.
 *   head_dim 128, 16-token pages; the first 16 tokens ("sink") and the last
 *   128 tokens ("recent") of every request stay BF16, the middle ("history")
 *   is rotated, clipped and stored as INT2 ([nl] §2.2.B, [fr] §2.2.B; the
 *   pages give no sizes, these are the values this library fixes).
 * ------------------------------------------------------------------------- */
#define OSCAR_HEAD_DIM 128
#define OSCAR_PAGE 16
#define OSCAR_N_SINK 16
#define OSCAR_N_RECENT 128
/* BF16 pages per request: entry 0 = sink page, entries 1..8 = ring pages. */
#define OSCAR_BF16_PAGES_PER_REQ 9

enum {
  OSCAR_OK = 0,
  OSCAR_EINVAL = -1,       /* null pointer, negative or inconsistent size    */
  OSCAR_EUNSUPPORTED = -2, /* G, code_bits or Hq/Hkv outside what is built */
  OSCAR_EWORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes() */
  OSCAR_EHIP = -4,         /* HIP runtime or launch error (text appended)    */
  OSCAR_ENODEV = -5        /* no usable gfx950 device                        */
};

/* Bits a kernel ORs into *status (oscar_layer_cache.status) when it meets
 * data it must not follow; the offending work item is skipped. */
#define OSCAR_STATUS_BAD_PAGE 1u   /* page id outside [0, n_pages)          */
#define OSCAR_STATUS_BAD_LEN 2u    /* seq_len < 1 or > the host bound       */

/* ---------------------------------------------------------------------------
 * Position → storage (one request of current length L; positions 0..L-1).
 *   p < 16                         sink:    bf16 page bf16_pt[b][0], row p
 *   16 <= p < L-128   (L > 144)    history: h = p-16, INT2 page
 *                                           hist_pt[b][h/16], row h%16
 *   max(16, L-128) <= p < L        recent:  ring slot s = p % 128, bf16 page
 *                                           bf16_pt[b][1 + s/16], row s%16
 * Appending one token at position L moves position L-128 (when >= 16) from
 * its ring slot into history; the new token takes that same slot.  History
 * page j always holds positions 16+16j .. 16+16j+15, so a page depends only
 * on its own tokens and may be shared between requests (prefix caching,
 * [nl] §2.2.B, [abs]).  Page tables may repeat page ids.
 *
 * BF16 pool: uint16 (bf16 bits) [n_bf16_pages][Hkv][2][16][128]; index 0 of
 * the "2" axis is K, 1 is V.  Rows hold raw, unrotated vectors.
 *
 * History pool: uint8 [n_hist_pages][Hkv][B_hist(G, bits)], one block per
 * (page, KV head):
 *     [ K codes A B | K meta 64*NG B | V codes A B | V meta 64*NG B ]
 *   NG = 128/G groups; A = 512 B for INT2 codes (code_bits 2), 1024 B for
 *   INT4 (code_bits 4); B_hist = 2A + 128*NG  (INT2: 1536, 1280, 1152 B,
 *   INT4: 2560, 2304, 2176 B for G = 32, 64, 128).
 *
 * Meta: entry (group g, row t) at byte 4*(16*g + t) of the meta area:
 *   fp16 scale s at +0, fp16 zero z at +2.  Dequantised value of a code c:
 *   c*s + z, in the rotated basis.
 *
 * Codes: 2-bit values 0..3.  A code area is 128 dwords; dword w (byte 4w,
 * little-endian) belongs to "lane" l = w/2, half d = w%2, with
 * a = l%16, q = l/16.  Inside a dword, slot u (0..7) holds two codes, the
 * first at bit LO[u] and the second at bit HI[u] (each 2 bits wide):
 *     LO = { 8,  6, 12, 10,  4,  2, 16, 14 }
 *     HI = {24, 22, 28, 26, 20, 18,  0, 30 }
 *   K code area (token-major): a = row (token) t, q selects channels;
 *     slot u of half d holds channels  c0 = 32*(2d + u/4) + 8q + 2*(u%4)
 *     (first) and c0+1 (second), both of token t.
 *   V code area (channel-major): a = channel offset m inside a block of 16,
 *     q selects a quad of rows; slot u of half d holds channel
 *     c = 16*(4d + u/2) + m for rows t0 = 4q + 2*(u%2) (first) and t0+1
 *     (second).
 * This order lets the decode expand a dword into eight fp16 pairs with one
 * AND-OR each (after at most one shift), in exactly the register order the
 * gfx950 matrix-core instructions read: K as 16x16x32 operands (16 tokens,
 * 32 channels per block), V as 16x16x16 operands (16 channels x 16 tokens).
 *
 * INT4 codes (code_bits 4): 4-bit values 0..15, asymmetric min-max over 15
 * steps (the INT4 comparison point of [nl] §4 / [fr] §4), meta as above.  A
 * code area is 256 dwords; lane l = w/4 owns dwords 4l..4l+3 (i = w%4), with
 * a = l%16, q = l/16; nibble e (0..7) of a dword sits at bits 4e..4e+3.
 *   K: a = row (token) t; dword i holds channels 32i + 8q + j of token t,
 *      channel offset j = 2*(e%4) + e/4 in nibble e.
 *   V: a = channel offset m; dword i holds channels 16*(2i + h) + m, h =
 *      (e/2)%2, rows 4q + k, k = 2*(e%2) + e/4, in nibble e.
 * Nibbles e and e+4 hold neighbouring channels (K) or rows (V), so one
 * shift and one AND-OR place them in the two halves of an fp16 pair.
 * ------------------------------------------------------------------------- */

typedef struct oscar_layer_cache {
  int32_t n_kv_heads;      /* Hkv >= 1                                       */
  int32_t group;           /* G: 32, 64 or 128 channels per (scale, zero)    */
  uint8_t *hist;           /* device history pool, layout above              */
  int64_t n_hist_pages;
  uint16_t *bf16;          /* device BF16 pool, layout above                 */
  int64_t n_bf16_pages;
  const int32_t *hist_pt;  /* device int32 [batch][hist_pt_stride]          */
  int32_t hist_pt_stride;  /* >= history pages of the longest request       */
  const int32_t *bf16_pt;  /* device int32 [batch][9]                        */
  uint32_t *status;        /* device, may be NULL: OSCAR_STATUS_* bits       */
  int32_t code_bits;       /* history code width: 2 (INT2; 0 also means 2)
                              or 4 (INT4)                                  */
} oscar_layer_cache;

/* Device forms of one fixed per-layer rotation R = U*H*P ([nl] §2.2.A
 * "Formule", [fr] §2.2.A.3; row-vector convention x_rot = x*R) and its clip
 * threshold ([nl]/[fr] §2.2.A, [abs] "fixed per-layer rotations and clipping
 * thresholds").  `forms` is written by oscar_prepare_rotation.
 *
 * Per-KV-head rotations (optional, an extension of the pages' per-layer
 * rule): n_heads equal to the cache's n_kv_heads (at most
 * OSCAR_MAX_HEAD_ROTATIONS) gives each KV head h its own rotation, whose
 * forms start h * oscar_rotation_bytes() bytes into `forms` (each written
 * by oscar_prepare_rotation), and its own clip head_clips[h] (host array,
 * read during the call only; each as `clip` below, which is then unused).
 * n_heads 0 or 1: one rotation for every head (head_clips unused).  Both
 * rotations of a call may use either form independently.  Errors:
 * OSCAR_EINVAL for another n_heads, a NULL head_clips or a clip outside
 * (0, 65504]. */
#define OSCAR_MAX_HEAD_ROTATIONS 32
typedef struct oscar_rotation {
  const void *forms;       /* device, n_heads (at least 1) consecutive forms
                              of oscar_rotation_bytes() bytes each        */
  float clip;              /* > 0 and finite; values clamp to [-clip, clip]  */
  int32_t n_heads;         /* 0 or 1: one rotation; else n_kv_heads         */
  const float *head_clips; /* host float[n_heads] when n_heads > 1         */
} oscar_rotation;

OSCAR_API const char *oscar_last_error(void);
OSCAR_API const char *oscar_version(void);

/* Bytes of one INT2 history block for group size G (0 if G is unsupported). */
OSCAR_API size_t oscar_hist_block_bytes(int32_t group);

/* Bytes of one history block for group size G and code width code_bits
 * (2 or 4); 0 if either is unsupported. */
OSCAR_API size_t oscar_hist_block_bytes_bits(int32_t group, int32_t code_bits);

/* Bytes of the device buffer that holds the forms of one rotation. */
OSCAR_API size_t oscar_rotation_bytes(void);

/* Converts R (device fp64 [128][128], row-major, R[i][j]) into the device
 * forms the kernels read (fp32 R and R^T, and R^T split into an fp16 high
 * part plus a 2^11-scaled fp16 low part for the matrix cores).
 * forms: device buffer of oscar_rotation_bytes(). */
OSCAR_API int oscar_prepare_rotation(const double *R, void *forms, oscar_stream_t stream);

/* Calibration workspaces.  Every calibration call works in a device
 * workspace the caller provides (any alignment >= 256 B, contents on entry
 * irrelevant); these give its size in bytes (0 for invalid sizes):
 *   oscar_calibrate_workspace_bytes: fp64 moments, the causal attention
 *     outputs (n_tokens * Hq * 1 KiB), |k R| / |v R| (n_tokens * Hkv *
 *     1 KiB), the moment partials (32 MiB) and the quantile's selection;
 *   oscar_calib_accumulate_workspace_bytes: attention outputs and partials;
 *   oscar_calib_rotations_workspace_bytes: two 128 x 128 fp64 matrices;
 *   oscar_clip_threshold_workspace_bytes: R and |x R| (n_vec * 1 KiB). */
OSCAR_API size_t oscar_calibrate_workspace_bytes(int64_t n_tokens, int32_t n_q_heads, int32_t n_kv_heads);
OSCAR_API size_t oscar_calib_accumulate_workspace_bytes(int64_t n_tokens, int32_t n_q_heads,
                                                        int32_t n_kv_heads);
OSCAR_API size_t oscar_calib_rotations_workspace_bytes(void);
OSCAR_API size_t oscar_clip_threshold_workspace_bytes(int64_t n_vec);

/* Calibration over many sequences ([nl]/[fr] §2.2.A; the moments are sums,
 * so they accumulate over any number of calibration sequences):
 * oscar_calib_accumulate adds one sequence's second-moment sums to sums,
 *   sums[0] += sum over tokens and query heads of q q^T,
 *   sums[1] += sum over tokens and query heads of o o^T, o the causal
 *              softmax(q K^T / sqrt(128)) V output of this sequence (query
 *              head h reads KV head h / (Hq/Hkv)),
 * and the caller adds n_tokens * Hq to its count.  oscar_calib_rotations
 * divides by count and returns R_K = U_Q H P_br and R_V = U_S H P_br as
 * oscar_calibrate_rotation does; the clips then come from
 * oscar_clip_threshold over the calibration K and V vectors.
 * q_cal: device bf16 [n_tokens][Hq][128]; k_cal, v_cal: device bf16
 * [n_tokens][Hkv][128]; sums: device fp64 [2][128][128], zeroed by the
 * caller before the first sequence; R_K, R_V: host fp64 [128][128] out;
 * workspace: device, the sizes above.  Both calls synchronise the stream.
 * Errors: OSCAR_EINVAL (NULL pointers, n_tokens outside [1, 65536], count
 * not positive, non-finite moments, an eigen-iteration that did not reach
 * its tolerance), OSCAR_EUNSUPPORTED (head counts), OSCAR_EWORKSPACE,
 * OSCAR_EHIP. */
OSCAR_API int oscar_calib_accumulate(const uint16_t *q_cal, const uint16_t *k_cal,
                           const uint16_t *v_cal, int64_t n_tokens, int32_t n_q_heads,
                           int32_t n_kv_heads, double *sums, void *workspace,
                           size_t workspace_bytes, oscar_stream_t stream);
OSCAR_API int oscar_calib_rotations(const double *sums, double count, double *R_K, double *R_V,
                          void *workspace, size_t workspace_bytes, oscar_stream_t stream);

/* Per-KV-head moments, for per-head rotations (an extension of the pages'
 * per-layer rule): as oscar_calib_accumulate, but KV head h's sums only
 * take the Hq/Hkv query heads that read it (h*Hq/Hkv ..), each with its
 * causal attention output over KV head h:
 *   sums[h][0] += sum over tokens and those query heads of q q^T,
 *   sums[h][1] += the same of o o^T.
 * sums: device fp64 [Hkv][2][128][128], zeroed by the caller before the
 * first sequence; KV head h's count grows by n_tokens * Hq/Hkv.  Then
 * oscar_calib_rotations on sums + h * 2*128*128 gives head h's R_K and R_V,
 * and oscar_clip_threshold over head h's K and V vectors its clips.
 * Workspace, synchronisation and errors as oscar_calib_accumulate. */
OSCAR_API int oscar_calib_accumulate_heads(const uint16_t *q_cal, const uint16_t *k_cal,
                                           const uint16_t *v_cal, int64_t n_tokens, int32_t n_q_heads,
                                           int32_t n_kv_heads, double *sums, void *workspace,
                                           size_t workspace_bytes, oscar_stream_t stream);

/* Clip threshold of one fixed rotation ([nl]/[fr] §2.2.A "clipping
 * thresholds"): the clip_quantile quantile (linear interpolation between
 * order statistics) of |x R| over every vector and channel of x_cal, the
 * same rule oscar_calibrate_rotation applies to its own R_K and R_V.  It
 * serves rotations chosen by the caller, such as the Hadamard-only
 * (QuaRot-style) R = H P_br and the identity of plain INT2 that the pages
 * compare OSCAR with ([abs]; [nl]/[fr] §2.1).  The order statistics are
 * selected on the device (radix selection over the fp64 bit patterns): host
 * memory does not grow with n_vec.
 * x_cal: device bf16 [n_vec][128]; R: host fp64 [128][128] (row-vector
 * convention, x R); clip: host float out; workspace: device,
 * oscar_clip_threshold_workspace_bytes(n_vec).  Synchronises the stream.
 * Errors: OSCAR_EINVAL for NULL pointers, n_vec outside [1, 2^31 - 1] or
 * clip_quantile outside (0, 1]; OSCAR_EWORKSPACE; OSCAR_EHIP. */
OSCAR_API int oscar_clip_threshold(const uint16_t *x_cal, int64_t n_vec, const double *R,
                         double clip_quantile, float *clip, void *workspace,
                         size_t workspace_bytes, oscar_stream_t stream);

/* Offline calibration ([nl] §2.2.A, [fr] §2.2.A, [abs]):
 *   C_Q = mean over tokens and query heads of the outer product q q^T;
 *   C_S = mean over tokens and query heads of o o^T, o = S V the causal
 *         softmax(q K^T / sqrt(128)) attention output of the calibration
 *         sequence (query head h reads KV head h / (Hq/Hkv));
 *   U_Q, U_S = eigenbases (eigenvalues descending, each column's
 *         largest-magnitude entry positive);
 *   R_K = U_Q H P_br, R_V = U_S H P_br (H = normalised 128-point Sylvester
 *         Hadamard, P_br = 7-bit bit-reversal permutation);
 *   clip_K / clip_V = the clip_quantile quantile (linear interpolation
 *         between order statistics) of |k R_K| / |v R_V| over every
 *         calibration token, KV head and channel.
 * q_cal: device bf16 [n_tokens][Hq][128]; k_cal, v_cal: device bf16
 * [n_tokens][Hkv][128].  Outputs R_K, R_V (host fp64 [128][128]) and
 * clip_K, clip_V (host).  workspace: device,
 * oscar_calibrate_workspace_bytes(n_tokens, Hq, Hkv).  Synchronises the
 * stream.  n_tokens in [1, 65536], clip_quantile in (0, 1].  Errors as
 * oscar_calib_accumulate. */
OSCAR_API int oscar_calibrate_rotation(const uint16_t *q_cal, const uint16_t *k_cal,
                             const uint16_t *v_cal, int64_t n_tokens,
                             int32_t n_q_heads, int32_t n_kv_heads,
                             double clip_quantile, double *R_K, double *R_V,
                             float *clip_K, float *clip_V, void *workspace,
                             size_t workspace_bytes, oscar_stream_t stream);

/* Fused KV write ([abs] "fused ... write ... kernels", [nl]/[fr] §2.2.B):
 * appends new tokens to every request of the batch.  Request b gets
 * n_b = cu_new[b+1]-cu_new[b] tokens at positions len_before[b] ..
 * len_before[b]+n_b-1 from rows cu_new[b].. of k_new / v_new (device bf16
 * [total_tokens][Hkv][128]).  Tokens that end up in the sink or recent
 * window are stored raw (bf16); tokens that end up in history, including
 * ring tokens pushed out by this call, are rotated by R (x*R), clamped to
 * [-clip, clip], split into groups of G consecutive rotated channels, and
 * stored as codes c = clamp(rint((x - z)/s), 0, 3) with z = fp16(min),
 * s = fp16((max - min)/3) (all codes 0 when s == 0); with code_bits 4 the
 * same over 15 steps: c in 0..15, s = fp16((max - min)/15).  The rotation keeps
 * fp32 dot-product accuracy with fp16 operands on the matrix cores: entries
 * of k_new / v_new beyond the fp16 range (|x| > 65504) are saturated to
 * +-65504 before rotating.
 * cu_new: device int32 [batch+1]; len_before: device int32 [batch].
 * max_new: host upper bound of n_b (sizes the grid).  History pages a call
 * writes must not be shared with another live request (caller's duty). */
OSCAR_API int oscar_write_kv(const oscar_layer_cache *cache, const oscar_rotation *rot_k,
                   const oscar_rotation *rot_v, const uint16_t *k_new,
                   const uint16_t *v_new, const int32_t *cu_new,
                   const int32_t *len_before, int32_t batch,
                   int64_t total_tokens, int32_t max_new,
                   oscar_stream_t stream);

/* Workspace for oscar_decode_attn and oscar_decode_step (device, any
 * alignment >= 256 B): the partial results of the splits, then one counter
 * per (request, KV head) that elects the workgroup which merges them.  Fill
 * it with zeros before its first call; every call that runs to completion
 * leaves the counters at zero again, so a workspace is reused without
 * clearing (after a call that faulted on the device, clear it again).  Calls
 * that share a workspace must not run concurrently. */
OSCAR_API size_t oscar_decode_workspace_bytes(int32_t batch, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t max_seq_len);

/* Mixed-precision paged decode attention ([nl]/[fr] §2.2.B "kernel
 * integration", [abs]): one query per request attends to all seq_lens[b]
 * cached tokens: BF16 sink/recent tokens directly, INT2 history through
 * dequantisation.  History keys stay in the rotated basis and are scored
 * against q*R_K; the history part of the output is brought back with R_V^T
 * once per partial sum over a split of pages (never per token).  softmax
 * scale sm_scale; query head h uses
 * KV head h / (Hq/Hkv).
 * q: device bf16 [batch][Hq][128]; seq_lens: device int32 [batch], each in
 * [1, max_seq_len]; out: device fp32 [batch][Hq][128]; workspace: see
 * oscar_decode_workspace_bytes (zero-filled before its first use).  Reads
 * INT2 or INT4 history (cache->code_bits). */
OSCAR_API int oscar_decode_attn(const oscar_layer_cache *cache,
                      const oscar_rotation *rot_k, const oscar_rotation *rot_v,
                      const uint16_t *q, int32_t n_q_heads,
                      const int32_t *seq_lens, int32_t batch,
                      int32_t max_seq_len, float sm_scale, float *out,
                      void *workspace, size_t workspace_bytes,
                      oscar_stream_t stream);

/* oscar_decode_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the partials and merge counters live in a
 * scratch array inside the library, one per GPU, held until the process
 * ends.  Same arguments, layout and results as oscar_decode_attn (the same
 * kernels and split plan), minus the workspace.  This call allocates
 * nothing.  Limit: at most 4096 (request, KV head) units and
 * oscar_decode_noalloc_max_bytes() bytes of scratch in all (16 MiB, of
 * which 1 MiB holds the counters); beyond that it returns OSCAR_EWORKSPACE
 * and launches nothing.  All calls on one GPU share its scratch array:
 * calls that overlap on one GPU (several streams or host threads at once)
 * race and must be serialised by the caller; a call that faulted on the
 * device may leave the counters dirty for later calls in this process. */
OSCAR_API size_t oscar_decode_noalloc_max_bytes(void);
OSCAR_API int oscar_decode_attn_noalloc(const oscar_layer_cache *cache,
                                        const oscar_rotation *rot_k, const oscar_rotation *rot_v,
                                        const uint16_t *q, int32_t n_q_heads,
                                        const int32_t *seq_lens, int32_t batch,
                                        int32_t max_seq_len, float sm_scale, float *out,
                                        oscar_stream_t stream);

/* One generation step of a layer: write-on-append of one token per request
 * followed by the decode over the grown cache ([abs] "fused Triton write and
 * decode kernels"; [nl]/[fr] §2.2.B).  Request b's new token k_new[b],
 * v_new[b] (device bf16 [batch][Hkv][128]) goes to position len_before[b]
 * (device int32 [batch]); a token leaving the recent window moves to history
 * exactly as in oscar_write_kv.  Then q (device bf16 [batch][Hq][128])
 * attends over all len_before[b] + 1 tokens as in oscar_decode_attn, which
 * must be <= max_seq_len.  Same result as oscar_write_kv with one token per
 * request followed by oscar_decode_attn, in one kernel launch.  The
 * workspace is the one of oscar_decode_attn (oscar_decode_workspace_bytes,
 * zero-filled before its first use).  INT2 or INT4 caches. */
OSCAR_API int oscar_decode_step(const oscar_layer_cache *cache,
                                const oscar_rotation *rot_k,
                                const oscar_rotation *rot_v,
                                const uint16_t *k_new, const uint16_t *v_new,
                                const int32_t *len_before, const uint16_t *q,
                                int32_t n_q_heads, int32_t batch,
                                int32_t max_seq_len, float sm_scale,
                                float *out, void *workspace,
                                size_t workspace_bytes, oscar_stream_t stream);

/* Extend (chunked-prefill) attention over the cache ([abs]: paged KV layouts
 * with prefix caching; [nl]/[fr] §2.2.B: the fused kernel dequantises and
 * inverse-rotates the INT2 history inside the attention).  Request b has a
 * cached prefix of len_before[b] tokens (device int32 [batch], each in
 * [0, max_prefix]) and new tokens at rows cu_new[b] .. cu_new[b+1]-1
 * (device int32 [batch+1], non-decreasing, cu_new[0] = 0, at most max_new
 * per request) of q (device bf16 [total_tokens][Hq][128]) and k_new, v_new
 * (device bf16 [total_tokens][Hkv][128]), at positions len_before[b] + i.
 * New token i attends to the whole prefix as oscar_decode_attn reads it
 * (BF16 sink and recent window, INT2 history scored against q*R_K, its
 * output part brought back with R_V^T once per query) and causally to new
 * tokens 0..i of its request at bf16.  The chunk is not written: call
 * oscar_write_kv with the same rows afterwards to append it.  Softmax scale
 * sm_scale; query head h uses KV head h / (Hq/Hkv).  out: device fp32
 * [total_tokens][Hq][128].  Needs no workspace.  A request whose length or
 * chunk is out of range sets OSCAR_STATUS_BAD_LEN and leaves its rows
 * unwritten; a page id out of range sets OSCAR_STATUS_BAD_PAGE and that
 * page is left out.  INT2 or INT4 caches. */
OSCAR_API int oscar_extend_attn(const oscar_layer_cache *cache,
                                const oscar_rotation *rot_k,
                                const oscar_rotation *rot_v,
                                const uint16_t *q, int32_t n_q_heads,
                                const uint16_t *k_new, const uint16_t *v_new,
                                const int32_t *cu_new, const int32_t *len_before,
                                int32_t batch, int64_t total_tokens,
                                int32_t max_new, int32_t max_prefix,
                                float sm_scale, float *out,
                                oscar_stream_t stream);

/* Workspace for oscar_bf16_paged_decode (device, any alignment >= 256 B):
 * the partials of the splits, then one merge counter per (request, KV head),
 * with the contract of oscar_decode_workspace_bytes: zero-filled before its
 * first use, left with zero counters by every call that completes. */
OSCAR_API size_t oscar_bf16_decode_workspace_bytes(int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads,
                                         int32_t max_seq_len);

/* Plain BF16 paged decode attention (the BF16 baseline the pages compare
 * against, [abs] "over BF16"): every token raw bf16, no rotation.
 * kv_pages: device bf16 [n_pages][Hkv][2][16][128] (same page format as
 * the BF16 pool); pt: device int32 [batch][pt_stride] — token p of request
 * b is row p%16 of page pt[b][p/16]; other arguments as oscar_decode_attn.
 * status: device uint32 or NULL (OSCAR_STATUS_* bits).  Split plan and
 * merge as in oscar_decode_attn (one round of one workgroup per CU with the
 * merge inside the kernel when the batch allows).  The workspace
 * (oscar_bf16_decode_workspace_bytes) is zero-filled before its first use;
 * calls that share a workspace must not run concurrently. */
OSCAR_API int oscar_bf16_paged_decode(const uint16_t *q, const uint16_t *kv_pages,
                            int64_t n_pages, const int32_t *pt,
                            int32_t pt_stride, const int32_t *seq_lens,
                            int32_t batch, int32_t max_seq_len,
                            int32_t n_q_heads, int32_t n_kv_heads,
                            float sm_scale, float *out, uint32_t *status,
                            void *workspace, size_t workspace_bytes,
                            oscar_stream_t stream);

/* Instrumentation for benchmarks: the next decode or write call on this host
 * thread (oscar_decode_attn, oscar_decode_step, oscar_bf16_paged_decode:
 * their split-K attention kernel; oscar_write_kv: its history write kernel)
 * launches that kernel with hipExtLaunchKernelGGL so that event `before` is
 * recorded when it starts and `after` when it ends, then forgets both.  before, after: hipEvent_t handles created by the
 * caller, or both NULL to cancel.  Returns OSCAR_EINVAL if exactly one of
 * them is NULL. */
OSCAR_API int oscar_profile_events(void *before, void *after);

/* Instrumentation for benchmarks: the read ceiling of the device.  Reads
 * n_blocks blocks of block_bytes bytes each with 16-byte vector loads --
 * block i is slot ids[i] of buf (slot k = bytes k*block_bytes ..
 * (k+1)*block_bytes-1), or slot i itself when ids is NULL -- and adds every
 * 32-bit word read, modulo 2^32, to *sink, so that no read can be left out.
 * Contiguous slots measure streaming reads; a permuted ids array measures
 * gathers of page-sized blocks, the access pattern of the decode's history
 * reads.  The decode kernels' bandwidth is reported against both ceilings.
 * buf: device, buf_bytes long; ids: device int32 [n_blocks] or NULL; sink:
 * device uint32.  Ids outside [0, buf_bytes / block_bytes) are skipped.
 * The next launch is timed by oscar_profile_events like the decode kernels.
 * Errors: OSCAR_EINVAL for NULL buf or sink, block_bytes not a multiple of
 * 16 in [16, 4096], n_blocks < 1, or (ids NULL) n_blocks * block_bytes >
 * buf_bytes; OSCAR_EHIP. */
OSCAR_API int oscar_read_probe(const void *buf, int64_t buf_bytes, int64_t n_blocks, int32_t block_bytes,
                               const int32_t *ids, uint32_t *sink, oscar_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H_ */
