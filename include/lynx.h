/*
 * lynx.h: C ABI of the MI355X (gfx950) Lynx split-stream KV codec.
 *
 * The operations are those of "Lynx: Progressive Speculative Quantization
 * for accelerating KV Transfer in Long-Context Inference" (Han et al.):
 *   - lynx_quantize_pages: Section 4.1, Algorithm 1 (Stages 1-4) and
 *     Eq. (3) on every page block of a KV set, producing the Anchor stream,
 *     the Residual stream and the metadata {gamma_min, gamma_scale, mu,
 *     sigma} (Section 4.2, prefill workflow: the quantization kernel turns
 *     each KV object into Q_anc, Q_res and the metadata);
 *   - lynx_dequant_anchor: the anchor phase of the decode workflow
 *     (Section 4.2, Figure 7(b)): approximate KV from Q_anc and metadata;
 *   - lynx_dequant_full: the residual phase (Section 4.2, Figure 7(c)):
 *     Q_res combined with the stored metadata refines the KV to Q_full;
 *   - lynx_page_stats / lynx_block_stats: Stage 1 and Stage 2 statistics of
 *     Algorithm 1 on their own (the same arithmetic as the fused quantize);
 *   - lynx_split_stream_transfer: the prioritized transmission of Section
 *     4.2 (Figure 7) emulated on one GPU through a wire buffer;
 *   - lynx_spec_verify: the verification that closes a speculative round
 *     (Section 4.3): accepted prefix and corrected next token;
 *   - lynx_decode_attn_dequant: attention O = softmax(Q K^T scale) V
 *     (Section 2.1) over K, V rebuilt on the fly from their streams: one
 *     query token (decode on the draft or verification precision) or T
 *     draft tokens with a causal tail (the single parallel forward pass of
 *     the verification, Section 4.3).
 *
 * Terms
 *   KV set      num_tensors token-major bf16 tensors [num_tokens][num_channels]
 *               (e.g. layers x {K, V}); tensor k starts tensor_stride elements
 *               after tensor k-1, token rows are row_stride elements apart.
 *   page block  X in R^{H x P}: H = 128 consecutive channels (one KV head)
 *               x P = 256 consecutive tokens of one tensor; chunk = C = 32
 *               consecutive tokens of one channel inside a page block.
 *   block index b = ((tensor * (num_tokens / P)) + page) * (num_channels / H)
 *               + head.  Every per-block output below is stored at block b.
 *
 * Stream and metadata layouts (all outputs are plain device buffers)
 *   anchor      uint8 [nblocks][P/C][H/2][C], chunk-tiled: byte
 *               [b][j][k][i] holds token 32 j + i of channel pair k, the
 *               4-bit two's-complement anchor of channel 2k in its low
 *               nibble and of channel 2k+1 in its high nibble.  16384 bytes
 *               per block, each chunk one 2048-byte tile, blocks back to
 *               back: one contiguous stream.
 *   residual    uint8 [nblocks][P/C][H/2][C], same layout, 4-bit signed
 *               residual (code = (anchor magnitude << 4) - residual).
 *   With anchor_bits = a other than 4 (the other splits of the 8-bit code,
 *   b = 8 - a residual bits): each (chunk j, pair k) holds a run of 8 w
 *   bytes (w = a for the anchor, b for the residual) at byte
 *   [b][j][k] x 8 w of the block's 4096 w bytes: an LSB-first bit stream
 *   of 64 two's-complement w-bit fields, field 2 i + e (token 32 j + i,
 *   channel 2k + e) at bit w (2 i + e).  For w = 4 this is the nibble
 *   layout above.  A single stream (residual_bits = 0) is the anchor layout
 *   alone, each field the whole code: magnitude I, one's-complemented when
 *   the value is negative.
 *   gamma_min, gamma_scale   float32 [nblocks][H]
 *   mu, sigma               float32 [nblocks][P/C][H]
 *   (bfloat16 bit patterns instead of float32 with meta_bits = 16)
 *
 * Numerics: binary32 with one IEEE round-to-nearest-even rounding per step
 * of Algorithm 1 (no contraction); the compander code is the exact
 * real-arithmetic rounding (half-up) of Eq. (3) applied to the binary32
 * X_final with the compander scaled to code_scale (default 120, so every
 * code fits the 4 + 4 split; with 127 codes above 120 are clipped so the
 * anchor fits 4 bits; with a anchor bits the clip is at 128 - 2^(7 - a),
 * the largest code whose anchor magnitude (code + 2^(7-a) - 1) >> (8 - a)
 * fits a bits); reconstruction is
 * ((S * L[code]) * (sigma + eps) + mu) * (gamma_scale + eps) + gamma_min with
 * L[k] = ((1 + alpha)^(k / code_scale) - 1) / alpha rounded to binary32, then
 * bf16 round-to-nearest-even.  Anchor-only uses code = anchor magnitude << 4
 * (<< (8 - a) in general).
 * Results are deterministic and independent of launch geometry.
 * Non-finite inputs, and channels whose max - min overflows binary32, give
 * unspecified (but in-bounds) outputs.
 *
 * Ownership and errors: the caller allocates and owns every buffer; the
 * library allocates no device memory and keeps no device state (its only
 * state is a host-side cache of the compander tables, keyed by the
 * parameters and guarded by a mutex).  Every call validates its arguments
 * before launching anything and returns a status code; on an error nothing
 * is launched and no output is written.  Successful calls are asynchronous
 * on `stream` (NULL = the default stream): results are visible once the
 * stream is synchronised.  Apart from the blocking
 * lynx_split_stream_transfer, a call only enqueues kernels on `stream` (no
 * allocation, memset, copy or synchronisation), so it may be recorded into a
 * HIP graph and replayed.  Device pointers must be 16-byte aligned, row and
 * tensor strides multiples of 8 elements, and row_stride at most 4210744
 * elements (a page block's 256 rows are addressed with 32-bit byte offsets;
 * larger strides give LYNX_ESHAPE).
 */
#ifndef LYNX_H
#define LYNX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LYNX_OK 0
#define LYNX_EINVAL (-1) /* null pointer, negative size, bad parameter     */
#define LYNX_ESHAPE (-2) /* tokens % 256, channels % 128, stride or align   */
#define LYNX_EHIP (-3)   /* a HIP call or launch failed (see status string) */
#define LYNX_ESCRATCH (-4) /* more than LYNX_ATTN_SCRATCH_BYTES of scratch
                              needed (lynx_decode_attn_dequant_noalloc)     */

/* Geometry fixed by the GPU kernels. */
#define LYNX_PAGE_TOKENS 256
#define LYNX_CHUNK_TOKENS 32
#define LYNX_BLOCK_CHANNELS 128

/* Output element type of lynx_decode_attn_dequant. */
#define LYNX_OUT_BF16 0
#define LYNX_OUT_F32 1

/* Method parameters (Algorithm 1 and Eq. (3)).  alpha > 0 controls the
 * skew of the alpha-law (default 255); eps > 0 is added to both scales
 * (default 1e-6); code_scale is the top of the compander's code range: the
 * default 120 is the largest code a 4-bit anchor plus a 4-bit residual can
 * carry (anchor magnitude (code + 7) >> 4 <= 7), so every |X_final| in
 * [0, 1] keeps its code; 127 (the 2^7 - 1 printed in Eq. (3)) is accepted and
 * then codes above 120 are clipped to 120.  page_tokens, chunk_tokens and
 * block_channels must be 256, 32 and 128.  anchor_bits a and residual_bits
 * b are the field widths (default 4 and 4 = the paper's split): a split of
 * the 8-bit code has a = 3..6 and b = 8 - a (the bias of Stage 4 is
 * 2^(b - 1) - 1, +7 for b = 4; codes above 128 - 2^(b - 1) are clipped);
 * b = 0 with a = 4 or 8 is a single a-bit stream (the paper's Lynx-INT4 /
 * Lynx-INT8 configurations, Section 5: Algorithm 1 into one precision, no
 * split; set code_scale to 2^(a - 1) - 1 = 7 or 127, codes above that are
 * clipped).  The anchor and residual streams take 4096 a and 4096 b bytes
 * per block.  Only quantize and the two dequant calls accept other widths
 * than 4 + 4.  meta_bits is 32 (binary32 metadata, default) or 16: bfloat16
 * metadata for the 4 + 4 split, each statistic rounded where Algorithm 1
 * produces it and used rounded from there on (gamma_scale and sigma up,
 * mu to nearest; gamma_min is already a bfloat16 value); the four lynx_meta
 * pointers then address arrays of bfloat16 bit patterns (uint16) with the
 * same element counts, half the bytes.  Only lynx_quantize_pages and the two
 * dequant calls accept 16. */
typedef struct lynx_params {
    float alpha;
    float eps;
    float code_scale;
    int32_t page_tokens;
    int32_t chunk_tokens;
    int32_t block_channels;
    int32_t anchor_bits;
    int32_t residual_bits;
    int32_t meta_bits;
    int32_t layout;
} lynx_params;

/* Code layouts (lynx_params.layout).
 *   LYNX_LAYOUT_SEPARATE (default): the anchor stream and the four metadata
 *     arrays are separate buffers (the layouts at the top of this file).
 *   LYNX_LAYOUT_PACKED: the transmission buffer of the paper's Section 4.2
 *     (prefill workflow, step 3) and Section 5 ("Compression Kernel"): the
 *     anchor of every page block followed immediately by its scalars.  The
 *     `anchor` buffer then holds one record per block, back to back, of
 *     lynx_anchor_block_bytes(params) bytes: the block's 4096 a bytes of
 *     anchor stream, then its gamma_min[128], gamma_scale[128],
 *     mu[8][128] and sigma[8][128] (binary32, or bfloat16 with
 *     meta_bits = 16): 25600 bytes per block for the paper's 4 + 4 split.
 *     A run of blocks is one contiguous byte range, so a KV object's anchor
 *     and metadata move in one copy.  Every lynx_meta argument must then be
 *     all NULL (LYNX_EINVAL otherwise).  The residual stream is unchanged.
 *     Accepted by lynx_quantize_pages, the two dequant calls, the two
 *     attention calls and lynx_split_stream_transfer; the statistics calls
 *     refuse it. */
#define LYNX_LAYOUT_SEPARATE 0
#define LYNX_LAYOUT_PACKED 1

/* Shape of a KV set (element strides, bf16 elements). */
typedef struct lynx_kv_shape {
    int64_t num_tensors;
    int64_t tensor_stride;
    int64_t num_tokens;
    int64_t num_channels;
    int64_t row_stride;
} lynx_kv_shape;

/* Device pointers to the four metadata arrays (layouts above). */
typedef struct lynx_meta {
    float *gamma_min;
    float *gamma_scale;
    float *mu;
    float *sigma;
} lynx_meta;

/* Fills *p with alpha = 255, eps = 1e-6, code_scale = 120, P = 256,
 * C = 32, H = 128, anchor_bits = residual_bits = 4, meta_bits = 32,
 * layout = LYNX_LAYOUT_SEPARATE. */
void lynx_default_params(lynx_params *p);

/* Number of page blocks of a shape, or a negative status if the shape is
 * invalid. */
int64_t lynx_num_blocks(const lynx_kv_shape *shape);

/* Bytes of one stream (anchor or residual) and number of floats of each
 * metadata array, for a shape; 0 if the shape is invalid.
 * lynx_stream_bytes is the 4-bit stream of the paper's split;
 * lynx_field_stream_bytes the stream of field_bits-bit fields (1..8),
 * nblocks x 4096 x field_bits. */
size_t lynx_stream_bytes(const lynx_kv_shape *shape);
size_t lynx_field_stream_bytes(const lynx_kv_shape *shape, int field_bits);
size_t lynx_gamma_floats(const lynx_kv_shape *shape);

/* Bytes per page block of the anchor-side buffer for `params` (NULL =
 * defaults): 4096 anchor_bits (separate layout), or the packed record of the
 * anchor stream and the metadata (4096 anchor_bits + 2304 meta_bits / 8).
 * 0 for invalid parameters.  Host only. */
size_t lynx_anchor_block_bytes(const lynx_params *params);
size_t lynx_chunk_floats(const lynx_kv_shape *shape);

/* Eq. (1) of the paper (Section 2.2): Size_KV = K_factor * L * D *
 * N_layers * Precision bytes (K_factor 2 for K and V, 1 for MLA; D = heads
 * x head dimension; precision in bytes).  0 on overflow or bad input. */
uint64_t lynx_kv_bytes(int64_t k_factor, int64_t seq_len, int64_t hidden,
                       int64_t layers, int64_t precision_bytes);

/* The 128 compander thresholds the kernels use for `params` (NULL =
 * defaults): thr[k], k = 1..120, is the smallest binary32 magnitude whose
 * Eq. (3) value reaches k - 1/2 (so code(|x|) = #{k : |x| >= thr[k]});
 * thr[0] = 0 and thr[k] = +inf for codes above 120 (above the largest
 * storable code of the field widths in general) or out of reach.  Host
 * only, no GPU needed.  Returns LYNX_EINVAL for bad parameters. */
int lynx_compander_thresholds(const lynx_params *params, float *thr128);

/* Human-readable text for a status code, or the last HIP error text of the
 * calling thread for LYNX_EHIP. */
const char *lynx_status_string(int status);

/*
 * Algorithm 1 on every page block of the KV set `kv` (bf16, layout given
 * by `shape`): writes anchor, residual (nblocks * 16384 bytes each; nblocks
 * * 4096 * anchor_bits and nblocks * 4096 * residual_bits for other field
 * widths) and the four metadata arrays.  `params` NULL means the defaults.
 * residual must be NULL exactly when residual_bits is 0 (a single stream),
 * else LYNX_EINVAL.
 */
int lynx_quantize_pages(const void *kv, const lynx_kv_shape *shape,
                        const lynx_params *params, uint8_t *anchor,
                        uint8_t *residual, lynx_meta meta, hipStream_t stream);

/*
 * Anchor phase: rebuilds every page block from the anchor stream and the
 * metadata (code = anchor magnitude << residual_bits: << 4 for the paper's
 * split, the whole code for a single stream) into `out` (bf16, layout given
 * by `shape`; the shape's strides describe `out`).  meta.* are only read.
 */
int lynx_dequant_anchor(const uint8_t *anchor, lynx_meta meta,
                        const lynx_kv_shape *shape, const lynx_params *params,
                        void *out, hipStream_t stream);

/*
 * Residual phase: rebuilds every page block at the verification precision
 * from anchor + residual and the metadata into `out`.  LYNX_EINVAL for a
 * single stream (residual_bits = 0).
 */
int lynx_dequant_full(const uint8_t *anchor, const uint8_t *residual,
                      lynx_meta meta, const lynx_kv_shape *shape,
                      const lynx_params *params, void *out,
                      hipStream_t stream);

/*
 * Algorithm 1 Stage 1 alone: gamma_min (canonical +0 for a zero minimum)
 * and gamma_scale = max - gamma_min of every channel of every page block.
 */
int lynx_page_stats(const void *kv, const lynx_kv_shape *shape,
                    const lynx_params *params, float *gamma_min,
                    float *gamma_scale, hipStream_t stream);

/*
 * Algorithm 1 Stage 2 statistics alone, given the Stage 1 statistics
 * (read from gamma_min / gamma_scale): mu (balanced pairwise tree mean of
 * the 32 normalised values) and sigma = max |X - mu| of every chunk.
 * Both statistics calls write binary32 (meta_bits must be 32).
 */
int lynx_block_stats(const void *kv, const lynx_kv_shape *shape,
                     const lynx_params *params, const float *gamma_min,
                     const float *gamma_scale, float *mu, float *sigma,
                     hipStream_t stream);

/* Workspace bytes lynx_decode_attn_dequant needs for these sizes (0 for
 * invalid sizes).  Host only. */
size_t lynx_attn_workspace_bytes(int t_q, int num_q_heads, int num_kv_heads,
                                 int64_t ctx_len);

/*
 * Grouped-query attention over Lynx-coded K and V:
 *   out[r][h] = softmax_p( q[r][h] . K^[p][h / g] * scale ) V^[p][h / g],
 * g = num_q_heads / num_kv_heads, p over the context positions a query sees.
 *   q            bf16 [t_q][num_q_heads][128] (device);
 *   out          [t_q][num_q_heads][128] (device) of LYNX_OUT_BF16 (bf16,
 *                the binary32 result rounded to nearest even) or
 *                LYNX_OUT_F32 (binary32) elements, per out_dtype;
 *   k_*, v_*     the streams and metadata of one quantized tensor each, of
 *                shape [ctx_len][num_kv_heads * 128] (the outputs of
 *                lynx_quantize_pages for num_tensors = 1); k_residual /
 *                v_residual NULL = anchor-only reconstruction.  K^ and V^
 *                follow Eq. (4) as one fused multiply-add per element with
 *                the coefficients folded per chunk and channel, so they
 *                equal lynx_dequant_anchor / _full up to rounding order (at
 *                most one bf16 unit apart, on rare elements);
 *   ctx_len      multiple of 256; head_dim must be 128;
 *   causal_tail  0: every query sees all ctx_len positions; 1: the t_q
 *                queries are the last t_q positions and row r sees positions
 *                0 .. ctx_len - t_q + r;
 *   workspace    >= lynx_attn_workspace_bytes(...) bytes of device memory,
 *                overwritten (split partials).
 * Scores, the softmax and the accumulation are binary32 (bf16 x bf16
 * products are exact).  g must be <= 64 and the field widths 4 + 4.  The
 * kernels take at most 64 query rows (t_q * g) per KV head: a call with
 * more query tokens runs in passes of floor(64 / g) tokens (each reading
 * the codes again), one after the other on `stream`, sharing the workspace,
 * whose size is that of the first pass.  Errors as above.
 */
int lynx_decode_attn_dequant(const void *q, int t_q, int num_q_heads,
                             const uint8_t *k_anchor, const uint8_t *k_residual,
                             lynx_meta k_meta, const uint8_t *v_anchor,
                             const uint8_t *v_residual, lynx_meta v_meta,
                             int64_t ctx_len, int num_kv_heads, int head_dim,
                             float scale, int causal_tail,
                             const lynx_params *params, void *out,
                             int out_dtype, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch of lynx_decode_attn_dequant_noalloc. */
#define LYNX_ATTN_SCRATCH_BYTES (24u << 20)

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): lynx_decode_attn_dequant
 * without a workspace argument.  Same arguments, results and errors, bit
 * for bit the same output; the split partials go to a fixed device array of
 * LYNX_ATTN_SCRATCH_BYTES (24 MiB) inside the library instead, and the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine;
 * the caller passes q, the codes and out).  Each GPU the library runs on
 * holds its own copy of the array from the first call on that device until
 * the process ends.  The first call on a device looks up that device's
 * array address (with the device current).  Calls whose partials need more
 * than the array holds (lynx_attn_workspace_bytes(...) above
 * LYNX_ATTN_SCRATCH_BYTES, which takes 64 query rows per KV head and more
 * than 128 KV heads) return LYNX_ESCRATCH before launching anything.  Every call on
 * one GPU shares that GPU's array and leaves its partials there (every
 * partial a call reads was written by the same call, so nothing needs
 * clearing): calls that overlap on one GPU (on different streams, or from
 * different host threads) race on it and must be serialised by the caller.
 */
int lynx_decode_attn_dequant_noalloc(const void *q, int t_q, int num_q_heads,
                                     const uint8_t *k_anchor,
                                     const uint8_t *k_residual, lynx_meta k_meta,
                                     const uint8_t *v_anchor,
                                     const uint8_t *v_residual, lynx_meta v_meta,
                                     int64_t ctx_len, int num_kv_heads,
                                     int head_dim, float scale, int causal_tail,
                                     const lynx_params *params, void *out,
                                     int out_dtype, hipStream_t stream);

/* Streams and metadata of a KV set in one memory space (device memory or
 * pinned host memory), layouts as above. */
typedef struct lynx_codes {
    uint8_t *anchor;
    uint8_t *residual;
    lynx_meta meta;
} lynx_codes;

/* Milestones of lynx_split_stream_transfer, in milliseconds after its start
 * (HIP events on the streams that reach them). */
typedef struct lynx_transfer_times {
    float quantized;          /* sender: last object quantized             */
    float anchor_arrived;     /* last anchor + metadata object in rx        */
    float residual_arrived;   /* last residual object in rx                 */
    float first_anchor_ready; /* receiver: first object rebuilt from anchor */
    float anchor_ready;       /* receiver: every object rebuilt from anchor */
    float full_ready;         /* receiver: every object refined             */
} lynx_transfer_times;

#define LYNX_TRANSFER_COPIES_ONLY 1 /* move the codes only: no quantize, no
                                       rebuild (the link's own time)       */

/*
 * Progressive split-stream transfer of a KV set through a wire buffer, on
 * one GPU (the paper's Section 4.2, Figure 7: the serializer quantizes KV
 * objects into Q_anc, Q_res and metadata, pushes the Anchor and the Residual
 * through two queues with the Anchor drained first, and overlaps the
 * transmission of object i with the quantization of object i + 1; the
 * deserializer rebuilds the cache from the Anchor first and refines it when
 * the Residual arrives).
 *
 * The set's page blocks (block order of the layouts above) are cut into
 * objects of object_blocks blocks (1 .. 2^22, at most 4096 objects; else
 * LYNX_EINVAL).  The wire has two hops, out (tx ->
 * wire) and in (wire -> rx), one stream each, so the two directions of the
 * link run at once.  Per object i:
 *   sender stream:   quantize the object into tx;
 *   link_out:        after it, copy its anchor and metadata tx -> wire;
 *   link_in:         after that, copy them wire -> rx;
 *   receiver stream: after that, rebuild the object from the anchor into
 *                    kv_anchor;
 * and only after every object's anchor copy on the same link stream (the
 * anchor queue is drained first on both hops), per object: its residual
 * tx -> wire on link_out, wire -> rx on link_in, and once every object is
 * rebuilt from its anchor, its rebuild from anchor + residual into
 * kv_full on the receiver stream.
 *   kv, shape, params  as lynx_quantize_pages (field widths must be 4 + 4);
 *   tx, wire, rx       code buffers of the whole set: tx and rx device
 *                      memory, wire pinned host memory (or device memory);
 *   kv_anchor, kv_full device bf16 outputs laid out by shape;
 *   flags              0, or LYNX_TRANSFER_COPIES_ONLY (kv, kv_anchor and
 *                      kv_full unused and may be NULL; tx must hold codes);
 *   times              if not NULL, the milestones.
 * Blocking: returns when all four streams have finished the transfer.  No
 * memory is allocated (HIP events only).  Errors as above; a HIP failure
 * mid-way still waits for the streams before returning LYNX_EHIP.
 */
int lynx_split_stream_transfer(const void *kv, const lynx_kv_shape *shape,
                               const lynx_params *params, int64_t object_blocks,
                               lynx_codes tx, lynx_codes wire, lynx_codes rx,
                               void *kv_anchor, void *kv_full, int flags,
                               hipStream_t sender, hipStream_t link_out,
                               hipStream_t link_in, hipStream_t receiver,
                               lynx_transfer_times *times);

/*
 * A stream for the codec kernels of a transfer (the sender and receiver
 * streams of lynx_split_stream_transfer) that leaves reserved_cus compute
 * units of the current device to other work: its kernels run only on the
 * remaining units (a CU mask; the reserved units are spread evenly over the
 * XCDs, whether the mask's bits go to the XCDs in turn or XCD after XCD).  The runtime runs most device-to-
 * pinned-host copies as shader copy kernels; on streams without such a
 * reserve those kernels wait until the quantize or rebuild kernels' own
 * workgroups drain, which stalls the link by up to a kernel's duration per
 * object.  reserved_cus = 0 gives a plain stream.  The stream is a blocking
 * stream (ordered with the NULL stream, as hipStreamCreate's) of the
 * current device; release it with lynx_stream_destroy.
 *   reserved_cus  0 .. (compute units of the device) - 1, else LYNX_EINVAL;
 *   stream        out: the new stream (NULL: LYNX_EINVAL).
 * Host only; LYNX_EHIP if the runtime refuses the stream.
 */
int lynx_codec_stream_create(int reserved_cus, hipStream_t *stream);
int lynx_stream_destroy(hipStream_t stream);

/* Workspace bytes of lynx_spec_verify (0 for invalid sizes).  Host only. */
size_t lynx_spec_verify_workspace_bytes(int t_draft, int vocab);

/*
 * Speculative verification of t_draft draft tokens (the paper's Section 4.3:
 * the drafts decoded on the Anchor-only cache are checked in one forward
 * pass on the full cache, the longest valid prefix is accepted and the first
 * divergence corrected; the notes' Eq. (10) and Eq. (11)).
 *   draft_logits   float32 [t_draft][vocab] (device): the logits the drafts
 *                  were drawn from, q_t = softmax(row t);
 *   target_logits  float32 [t_draft + 1][vocab] (device): p_t on Q_full;
 *   draft_tokens   int32 [t_draft] (device); u_accept float64 [t_draft]
 *                  (device), uniforms in [0, 1); u_sample in [0, 1);
 *   out            int32 [2] (device): accepted drafts k (0..t_draft) and the
 *                  next token.
 * Draft t is accepted when u_accept[t] < p_t(s_t) / q_t(s_t); at the first
 * rejection k the next token is the smallest x whose running sum of
 * max(0, p_k - q_k) exceeds u_sample times its total; if all drafts pass it
 * is drawn the same way from p_{t_draft}.  Softmaxes in binary64.  A draft
 * token outside [0, vocab) counts as rejected.  t_draft <= 64.  Errors as
 * above.
 */
int lynx_spec_verify(const float *draft_logits, const float *target_logits,
                     const int32_t *draft_tokens, const double *u_accept,
                     double u_sample, int t_draft, int vocab, int32_t *out,
                     void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LYNX_H */
