/*
 * octopus.h -- C ABI of the OCTOPUS KV-cache codec and the attention kernels
 * that read it (gfx950 / MI355X).
 *
 * The method is the one of "OCTOPUS: Optimized KV Cache for Transformers via
 * Octahedral Parametrization Under optimal Squared error quantization"
 * (arXiv 2605.21226).  A key (or value) k in R^d is stored as the compressed
 * state S(k) = (gamma, I_dir, I_nrm) of its Sec. 3: the norm gamma, a packed
 * stream of octahedral-coordinate indices and a packed stream of triplet-norm
 * indices, optionally plus the 1-bit QJL residual (sigma, gamma_r) of Sec. 3.6.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes inside these calls and keeps no
 *     mutable global state; calls are asynchronous on `stream` and re-entrant.
 *   - Every argument that can be checked on the host is checked before any
 *     launch; on failure nothing is launched and a status other than OCTO_OK is
 *     returned.  octo_last_error() then returns a thread-local message.
 *     No exception crosses this boundary.
 *   - Device-resident lengths (seq_lens) cannot be checked on the host; the
 *     kernels clamp them to [0, min(max_seq_len, capacity)].
 *   - Outputs are bitwise deterministic for identical inputs (no atomics in any
 *     reduction; the split-K merge order is fixed).
 *   - Supported now: head_dim = 128; (b_dir, b_nrm) in {(3,1), (4,2), (5,3)}
 *     (the paper's (b+1, b-1) split for b = 2, 3, 4; Sec. 3.3) and the uniform
 *     splits {(2,2), (3,3), (4,4)}; for decode, 1 to 16 query heads per KV
 *     head; QJL on keys only, in the decode path only; the group-wise codec
 *     (group 16 or 32, b = 2, 3, 4; described below) for values, and for
 *     keys in the chunk path.  octo_encode, octo_decode_tokens and
 *     octo_record_sizes also take the other splits of the (b + delta,
 *     b - delta) sweep of Sec. 3.3 (b = 2, 3, 4; delta = -2 .. 2, so b_dir and
 *     b_nrm from 0 to 6), for quality measurement; the attention entry points
 *     do not.  Anything else returns OCTO_ERR_UNSUPPORTED.
 *
 * Cache layout (OCTO_LAYOUT_TILE64).  The paper fixes no bit layout; this one
 * is this library's.  A stream is a little-endian LSB-first bit string: field
 * j of width w occupies bits [j*w, (j+1)*w).  The index stream `idx` holds the
 * bits of I_dir and I_nrm interleaved per triplet: n_tri fields of
 * B_tri = 2*b_dir + b_nrm bits (the triplet budget of Sec. 3.3), field i being
 *     xi_i | eta_i << b_dir | rho_i << (2*b_dir)
 * (the triplet's two octahedral-coordinate indices, then its norm index).  The
 * QJL stream holds d one-bit fields (1 where sigma_j = -1).  Each stream is
 * zero-padded to whole 32-bit words (W words per token).  In a
 * (batch b, kv head h) plane of `capacity` tokens (a multiple of 64), word w
 * of token t is stored at word index
 *     ((b*kv_heads + h)*(capacity/64) + t/64)*W*64 + w*64 + t%64,
 * i.e. each 64-token tile keeps its W words as W rows of 64 consecutive words,
 * so that one wavefront reading word w of 64 tokens reads 256 contiguous bytes.
 * gamma (fp32) and gamma_r (fp16 bit pattern) are plain [B][H][capacity].
 *
 * Group-wise value codec (codec.group = 16 or 32).  The OCTOPUS paper's
 * experiments share one value codec with a value-side group size of 16 or
 * 32 (Sec. 4, default recipe; Sec. 4.2) without defining it; it is read from
 * "Quantized Keys Steal Attention" (Sec. 3, quantization granularity and the
 * Hadamard rotation; Sec. 4.3, FP8 E4M3 scales and BF16 zero-points,
 * B_eff = b + 24/g; Sec. 5, asymmetric round-to-nearest):
 *     u = R v (the same R = H diag(s) as above, /sqrt(d)), and per group j
 *     of g consecutive coordinates: Delta = (max - min) / (2^b - 1) in fp32,
 *     stored as E4M3 (round to nearest even, saturating at 448); z = min
 *     stored as BF16 (round to nearest even); code c = clamp(rint((u_c - z) /
 *     Delta), 0, 2^b - 1) in fp32 (0 where Delta rounds to 0);
 *     v^ = R^T (Delta code + z).
 * Its record is one index-stream record of W = (128 b + 24 * 128/g) / 32
 * words: 128 fields of b bits (the codes, coordinate order), then 128/g
 * fields of 8 bits (E4M3 scales), then 128/g fields of 16 bits (BF16
 * zero-points), in the same tile-64 layout.  It has no gamma, QJL or
 * codebooks.
 */
#ifndef OCTOPUS_H
#define OCTOPUS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OCTO_ABI_VERSION 4u

typedef enum {
  OCTO_OK = 0,
  OCTO_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad enum   */
  OCTO_ERR_UNSUPPORTED = 2,        /* valid but not implemented (d, bits, G)  */
  OCTO_ERR_ALIGNMENT = 3,          /* pointer or stride not suitably aligned  */
  OCTO_ERR_CAPACITY = 4,           /* token range beyond the cache capacity   */
  OCTO_ERR_WORKSPACE_TOO_SMALL = 5,
  OCTO_ERR_VERSION = 6,            /* descriptor built for another ABI        */
  OCTO_ERR_HIP = 7                 /* a HIP launch reported an error          */
} octo_status;

/* The enums below name the values of plain int32_t arguments and fields:
   a caller may pass any int, and a value outside the enum is rejected
   with OCTO_ERR_INVALID_ARGUMENT rather than read as an enum.            */
typedef enum { OCTO_DTYPE_F32 = 0, OCTO_DTYPE_BF16 = 1 } octo_dtype;

/* Encoder rounding (OCTOPUS paper Sec. 3.5; App. A/E summaries).
 * LOCAL3X3: the 3x3 joint rounding around the scalar Lloyd seed (default).
 * SCALAR:   Delta = {(0,0)}: independent nearest-centroid xi, eta and rho.   */
typedef enum { OCTO_ROUND_LOCAL3X3 = 0, OCTO_ROUND_SCALAR = 1 } octo_rounding;

typedef enum { OCTO_LAYOUT_TILE64 = 0 } octo_layout;

/* One codec (one for K, one for V).  Sec. 3.3-3.4: the triplet budget is
 * B_tri = 2*b_dir + b_nrm; codebooks depend only on (d, b_dir, b_nrm).
 * The rotation R = H diag(s) (Sec. 3.1, App. C.2) takes its signs s_j,
 * j < d, from the j-th output of SplitMix64 seeded with `seed` (bit 63 set ->
 * -1); the QJL rotation R' uses outputs d..2d-1.                             */
typedef struct {
  uint32_t abi_version;   /* must be OCTO_ABI_VERSION                          */
  int32_t head_dim;       /* d (power of two; 128 supported)                   */
  int32_t bits;           /* b; with b_dir = b_nrm = 0 selects (b+1, b-1)      */
  int32_t b_dir;          /* explicit bits per octahedral coordinate, or 0     */
  int32_t b_nrm;          /* explicit bits per triplet norm, or 0              */
  int32_t rounding;       /* octo_rounding                                     */
  int32_t qjl;            /* 1: keys carry the QJL sign sketch (Sec. 3.6)      */
  int32_t group;          /* 0: OCTOPUS codec; 16 or 32: the group-wise value
                             codec described above (bits in 2..4, b_dir =
                             b_nrm = 0, no QJL, rounding and codebooks ignored)*/
  uint64_t seed;          /* rotation seed                                     */
  const float* c_xi;      /* host, 2^b_dir fp32 centroids, ascending           */
  const float* c_rho;     /* host, 2^b_nrm fp32 centroids, ascending           */
} octo_codec_desc;

/* A packed cache for one tensor (K or V), layout OCTO_LAYOUT_TILE64.        */
typedef struct {
  uint32_t* idx;          /* B*H*capacity*W_idx words                          */
  float* gamma;           /* B*H*capacity; unused (may be NULL) for a group codec */
  uint32_t* qjl;          /* B*H*capacity*W_qjl words, NULL unless codec.qjl   */
  uint16_t* gamma_r;      /* B*H*capacity fp16 bits, NULL unless codec.qjl     */
  int32_t batch;          /* B                                                 */
  int32_t kv_heads;       /* H                                                 */
  int32_t capacity;       /* tokens per (b, h) plane, multiple of 64           */
  int32_t layout;         /* octo_layout                                       */
} octo_cache_view;

/* 32-bit words per token of each stream for a codec.                        */
typedef struct {
  int32_t idx_words;      /* ceil(n_triplets * (2*b_dir + b_nrm) / 32); for a
                             group codec the record's (128 b + 24*128/g) / 32   */
  int32_t qjl_words;
  int32_t n_triplets;     /* ceil(d / 3); 0 for a group codec                  */
  int32_t b_dir;          /* the resolved split (0, 0 for a group codec)       */
  int32_t b_nrm;
} octo_stream_sizes;

uint32_t octo_abi_version(void);
/* Name of a status code; "OCTO_ERR_UNKNOWN" for any other value.  The code
   is taken as a plain int, so a value outside the enum is well defined.     */
const char* octo_status_string(int32_t s);
/* Message of the last failing call on this thread ("" if none).             */
const char* octo_last_error(void);

/* Resolves the bit split and fills `out`.  Host only.                        */
octo_status octo_record_sizes(const octo_codec_desc* codec, octo_stream_sizes* out);

/* octo_encode -- OCTOPUS encoder (paper Sec. 3.1-3.6; App. A summary).
 * For every b < B, h < H, t < T encodes x[b,h,t,:] and writes token
 * token_offset + t of plane (b, h) of `dst`: gamma = ||x||_2, u = R x/gamma,
 * zero-pad to 3*ceil(d/3), triplets, octahedral map (Eq. 5), Lloyd seeds,
 * 3x3 joint rounding (or scalar rounding), packing; with codec.qjl also the
 * QJL signs of R'(u - u^) and gamma_r = fp16(||u - u^||).  With a group
 * codec it writes the group record of R x instead (no gamma).
 *   x          device, element (b,h,t,e) at x + b*s0 + h*s1 + t*s2 + e*s3,
 *              x_strides = {s0,s1,s2,s3} in elements, s3 must be 1, the
 *              others >= 0; x aligned to its element size.
 *   x_dtype    OCTO_DTYPE_F32 or OCTO_DTYPE_BF16.
 *   dst        cache with batch == B, kv_heads == H and
 *              token_offset + T <= capacity (else OCTO_ERR_CAPACITY).
 * Zero vectors encode as gamma = 0 with the placeholder direction (0, 0).   */
octo_status octo_encode(const octo_codec_desc* codec, const void* x, int32_t x_dtype,
                        int32_t B, int32_t H, int32_t T, const int64_t x_strides[4],
                        const octo_cache_view* dst, int32_t token_offset,
                        hipStream_t stream);

/* octo_decode_tokens -- the explicit reconstruction of packed tokens:
 * out[b, h, t - t0, :] = gamma R^T u^[:d] for t in [t0, t0 + T) of every
 * plane (paper Sec. 3.6 Eq. 13 and App. C.14: the factorized score is
 * q . x^).  For quality measurement and for callers that need dense vectors;
 * the attention entry points never materialize K^.  With a QJL codec this is
 * the MSE reconstruction alone (the sign sketch estimates inner products and
 * reconstructs nothing).  A group codec gives R^T (Delta code + z).
 *   out   device fp32 [B, H, T, d], contiguous.
 * Tokens beyond capacity return OCTO_ERR_CAPACITY; T = 0 does nothing.      */
octo_status octo_decode_tokens(const octo_codec_desc* codec, const octo_cache_view* cache,
                               int32_t t0, int32_t T, float* out, hipStream_t stream);

/* Workspace bytes needed by octo_attend_decode for these shapes.            */
octo_status octo_decode_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                        int32_t num_q_heads, int32_t kv_heads,
                                        int32_t max_seq_len, size_t* bytes);

/* octo_attend_decode -- one query per sequence over the packed cache
 * (paper Sec. 3.6 Eq. 13 score factorization; App. A summary: split-K
 * flash decoding with fused unpack, centroid lookup, octahedral decode,
 * value dequantization and online softmax).  For query head h on KV head
 * g = h / (num_q_heads / kv_heads):
 *   score_j = gamma_j * (R q_h) . u^_j  [+ gamma_j sqrt(pi/(2d)) gamma_r,j (R'R q_h).sigma_j]
 *   out[b,h,:] = R_v^T sum_j softmax(softmax_scale * score)_j gamma_v,j u^_v,j
 * over tokens j < min(seq_lens[b], max_seq_len, capacity).  K^ is never
 * materialized.  An empty context gives a zero output row.
 *   q          device [B, num_q_heads, d], fp32 or bf16, contiguous.
 *   seq_lens   device int32 [B].
 *   softmax_scale  <= 0 selects 1/sqrt(d).
 *   out        device fp32 [B, num_q_heads, d].
 *   workspace  device, >= octo_decode_workspace_bytes(...), 256-byte aligned;
 *              holds the per-split partial results (no state between calls).
 *              Calls that share a workspace must not overlap in time.
 * Both contractions run on MFMA with fp16 hi/lo operand pairs and fp32
 * accumulation (about 2^-20 relative per product); softmax and the merge of
 * the splits are fp32.  Any finite value norm is supported: a token whose
 * norm is 128 or more enters the running maximum with its score raised by
 * its norm's binary exponent, so that every weight p gamma_v stays below
 * 2^15, inside the fp16 operands.  K and V caches must share B, kv_heads, capacity and
 * (b_dir, b_nrm); V must not carry QJL.  V may instead use the group codec
 * (group 16 or 32) when K uses the (b+1, b-1) split and V has the same b
 * (the symmetric K = V bit width of the paper's comparisons); its products
 * take Delta * code, exact in fp16, against the hi/lo weights, and the
 * zero-point term sum_j p_j z_j in fp32.  K must use the OCTOPUS codec here
 * (the group codec for keys is taken by octo_attend_chunk only).            */
octo_status octo_attend_decode(const octo_codec_desc* k_codec, const octo_codec_desc* v_codec,
                               const octo_cache_view* k_cache, const octo_cache_view* v_cache,
                               const void* q, int32_t q_dtype, int32_t num_q_heads,
                               const int32_t* seq_lens, int32_t max_seq_len,
                               float softmax_scale, float* out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* octo_attend_decode_noalloc -- octo_attend_decode without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results as octo_attend_decode, bit for bit; the per-split
 * partials live in a static device array of OCTO_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library keeps on each device it runs on until the
 * process ends.  The call allocates and frees nothing.  Shapes whose
 * partials need more (octo_decode_workspace_bytes > 16 MiB) return
 * OCTO_ERR_CAPACITY before any launch.  Every call on one device uses that
 * device's one array, which keeps the last call's partials: calls that
 * overlap in time on one device (different streams, or a capture replayed
 * beside another call) race and must be ordered by the caller.  Nothing in
 * the array has to start at any particular value.                         */
#define OCTO_NOALLOC_SCRATCH_BYTES (16u << 20)
octo_status octo_attend_decode_noalloc(const octo_codec_desc* k_codec,
                                       const octo_codec_desc* v_codec,
                                       const octo_cache_view* k_cache,
                                       const octo_cache_view* v_cache, const void* q,
                                       int32_t q_dtype, int32_t num_q_heads,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       float softmax_scale, float* out, hipStream_t stream);

/* Workspace bytes needed by octo_decode_step for these shapes.              */
octo_status octo_decode_step_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                             int32_t num_q_heads, int32_t kv_heads,
                                             int32_t max_packed_len, size_t* bytes);

/* octo_decode_step -- one decode step with a residual window of native-
 * precision tokens beside the packed cache (the OCTOPUS paper's experiments
 * keep the most recent tokens at native precision, Sec. 4 "default recipe";
 * Sec. 4.2 uses 32).  The paper gives no mechanism; this call's:
 *   State of sequence b: the packed caches hold tokens [0, P_b), the rings
 *   hold tokens [P_b, P_b + n_b), n_b < window, token j in ring slot
 *   j mod window.  P_b = packed_lens[b], n_b = window_lens[b].
 *   1. k_new[b], v_new[b] become token t = P_b + n_b, written to ring slot
 *      t mod window;
 *   2. out[b, h] = softmax attention of q[b, h] over the packed tokens
 *      [0, P_b) (as octo_attend_decode, QJL term included) and the native
 *      rows of tokens P_b .. t, in one softmax (fp32 over the native rows);
 *   3. if n_b + 1 == window, token P_b is encoded from its ring row into
 *      packed slot P_b of k_cache and v_cache (as octo_encode would) and
 *      P_b += 1; otherwise n_b += 1.  packed_lens and window_lens are
 *      updated on the device by the call's second kernel.
 * So the attention always sees the last min(window, t + 1) tokens at native
 * precision, and a token is compressed when it leaves the window.
 *   q           device [B, num_q_heads, d], fp32 or bf16.
 *   k_new, v_new  device bf16 [B, kv_heads, d], 16-byte aligned.
 *   k_window, v_window  device bf16 rings [B, kv_heads, window, d], 16-byte
 *               aligned, owned by the caller, read and written.
 *   window      1 .. 256.
 *   packed_lens, window_lens  device int32 [B], read and updated in place.
 *   max_packed_len  host bound: every P_b <= max_packed_len <= capacity
 *               (the split plan is sized by it).  A larger P_b breaks this
 *               precondition: its packed tokens past max_packed_len are then
 *               left out of the attention, while the ring slots, the
 *               eviction and the length updates still follow P_b itself.
 *   workspace   device, >= octo_decode_step_workspace_bytes(...), 256-byte
 *               aligned.
 * Device-resident preconditions (not checked on the host): 0 <= n_b < window;
 * P_b < capacity when the ring is full (else nothing is encoded and the
 * lengths keep their values).  Two kernels: the scan of octo_attend_decode
 * over the packed tokens, then the merge, which folds in the native rows and
 * in which one more workgroup per sequence does steps 1 and 3 and updates
 * the lengths.  Codec combinations as for octo_attend_decode.                */
octo_status octo_decode_step(const octo_codec_desc* k_codec, const octo_codec_desc* v_codec,
                             const octo_cache_view* k_cache, const octo_cache_view* v_cache,
                             const void* q, int32_t q_dtype, int32_t num_q_heads,
                             const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_window,
                             uint16_t* v_window, int32_t window, int32_t* packed_lens,
                             int32_t* window_lens, int32_t max_packed_len, float softmax_scale,
                             float* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Flags of octo_attend_chunk.
 * OCTO_CHUNK_JENSEN_CORRECTION: subtract from every cached token's logit the
 * Jensen bias of "Quantized Keys Steal Attention" (Sec. 4.2, Eq. 15; its
 * appendix on the rotation): b = tau^2 / 24 * sum_j Delta_j^2 ||(R q)_j||^2
 * over the key's groups j, tau the softmax scale (Eq. 15 has tau = 1/sqrt(d)).
 * It models round-to-nearest noise, so the keys must use the group codec.  */
#define OCTO_CHUNK_JENSEN_CORRECTION 1u

/* Workspace bytes needed by octo_attend_chunk for these shapes and flags.   */
octo_status octo_chunk_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                       int32_t num_q_heads, int32_t kv_heads, int32_t Tq,
                                       int32_t cached_tokens, int32_t Tc, uint32_t flags,
                                       size_t* bytes);

/* octo_attend_chunk -- chunk-wise attention ("Quantized Keys Steal Attention",
 * Sec. 3, Token Structure and Attention Decomposition; OCTOPUS paper Sec. 4.3
 * chunk-wise video diffusion): every one of the Tq queries of the current
 * chunk attends, in one softmax and without a mask, to the first
 * `cached_tokens` tokens of the packed cache and to the Tc current-chunk keys
 * and values held at full precision.  Query head h uses KV head
 * h / (num_q_heads / kv_heads).  QK^T and PV run on MFMA with fp16 operands
 * and fp32 accumulation, everything in the rotated frames: R_k q, R_k k_cur,
 * R_v v_cur and gamma u^ of the cached tokens (Eq. 13); the epilogue applies
 * R_v^T.  The cached window is decoded inside the attention kernel, tile by
 * tile, into on-chip memory: it is read once per query tile as packed words
 * and never written out.  The queries are rotated inside the attention
 * kernel too; the workspace receives only the fp16 rotated key and value
 * rows of the current chunk, which every query tile of a plane reads.
 *   q          device bf16 [B, num_q_heads, Tq, d] contiguous, 16-byte aligned.
 *   k_cur,v_cur device bf16 [B, kv_heads, Tc, d] contiguous, 16-byte aligned
 *              (may be NULL if Tc == 0).
 *   out        device fp32 [B, num_q_heads, Tq, d].
 *   workspace  device, >= octo_chunk_workspace_bytes(...), 256-byte aligned.
 * Keys must not carry QJL in this path; keys and values may use the group
 * codec, any b and g.  flags: 0 or OCTO_CHUNK_JENSEN_CORRECTION (above; the
 * bias is one more MFMA k-slice per 16 keys, the product of fp16 query
 * features -16 log2(e) tau^2/24 ||(R q)_j||^2 and key features Delta_j^2/16,
 * so it shares the fp16 range limits below).  Operand range and precision:
 * the fp16 operands require |rotated entries| < 65504 (for cached keys and
 * values, gamma rho^ < 65504) and round each operand to 11 significant bits, so this
 * path is meant for inputs without large outlier channels (the decode path
 * computes in fp32).  Tq == 0 is a no-op; an empty window gives zero output
 * rows.  A plane whose current value rows (Tc rounded up to 32, times 256
 * bytes) or packed records (capacity times record bytes) exceed 2 GiB
 * returns OCTO_ERR_UNSUPPORTED.                                            */
octo_status octo_attend_chunk(const octo_codec_desc* k_codec, const octo_codec_desc* v_codec,
                              const octo_cache_view* k_cache, const octo_cache_view* v_cache,
                              int32_t cached_tokens, const void* q, const void* k_cur,
                              const void* v_cur, int32_t num_q_heads, int32_t Tq, int32_t Tc,
                              float softmax_scale, uint32_t flags, float* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* OCTOPUS_H */
