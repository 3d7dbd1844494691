/*
 * libwaveprune -- WavePrune (RoPE first-period truncation) attention on
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The method: "WavePrune: One period is often enough for RoPE"
 * (arXiv 2610.06963), as described on the cc.laoqi.cc reading notes
 * ("WavePrune：RoPE 通常只需一个旋转周期", cited below as [notes]) and the
 * first author's thread on sotwe.com ([thread]).  Every 2-D RoPE channel c
 * adds to the query-key logit only while the query-key distance stays within
 * its wavelength w_c = 2*pi/f_c; a truncated channel adds 0 and the key stays
 * in the causal softmax ([notes] section 2.1, Eq. (6); [thread] 3/7).
 * Head dims are grouped in G consecutive dims that share the largest cutoff
 * inside the group ([notes] section 2.3, Eq. (8)), and every
 * (query block, key block) tile is classified per group as skip, partial or
 * full ([notes] section 2.3, classification table; [thread] 6/7).
 *
 * Conventions shared by every call
 *  - Channel c of a head vector is the interleaved pair of dims (2c, 2c+1).
 *  - Tensors are bf16 unless stated; d_h is innermost and contiguous; the
 *    other axes take explicit strides counted in ELEMENTS.  Base pointers must
 *    be 16-byte aligned and every stride a multiple of 8 elements.
 *  - Device buffers are owned by the caller.  The library allocates nothing,
 *    keeps no mutable global state, never synchronizes, and enqueues all work
 *    on `stream` (a hipStream_t; NULL is the null stream).
 *  - Arguments are validated on the host before any HIP call.  On error the
 *    call returns a negative wp_status, enqueues nothing, and
 *    wp_last_error() (thread-local) describes the problem.  Nothing is thrown
 *    across the ABI and nothing aborts.  Faults inside kernels surface at the
 *    caller's next synchronization of `stream`.
 *  - Supported: d_h in {64, 128}; Hq a multiple of Hkv; G in {16, 32}
 *    everywhere, and also G in {2, 4, 8} for the tiling / tile-count
 *    queries, wp_prefill, wp_prefill_backward and wp_decode.  G = 2 gives
 *    every channel its own cutoff: the exact per-channel rule of [notes]
 *    section 2.1, Eq. (6), which section 2.3 approximates by groups (kept
 *    for quality ablations; a tile mixing classes inside one 16-dim MFMA
 *    step costs extra masked MFMAs).  The compact K store (wp_kcache_*,
 *    wp_decode_kcache) takes G in {16, 32} only (WP_ERR_UNSUPPORTED
 *    otherwise).
 */
#ifndef WAVEPRUNE_H
#define WAVEPRUNE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t wp_status;
#define WP_OK               0
#define WP_ERR_NULL        (-1)  /* a required pointer is NULL */
#define WP_ERR_SHAPE       (-2)  /* a size is out of range or inconsistent */
#define WP_ERR_UNSUPPORTED (-3)  /* d_h or G outside the supported set */
#define WP_ERR_ALIGN       (-4)  /* pointer or stride misaligned */
#define WP_ERR_WORKSPACE   (-5)  /* workspace too small */
#define WP_ERR_ARG         (-6)  /* bad scalar argument (theta, scale, cutoffs, flags) */
#define WP_ERR_HIP         (-7)  /* the HIP runtime reported an error at launch */

#define WP_DTYPE_BF16 0
#define WP_DTYPE_F32  1

/* Flags for wp_prefill / wp_decode. */
#define WP_FLAG_DENSE 1u  /* ignore the cutoffs: every group is full (plain RoPE
                             attention; the in-house dense baseline) */
#define WP_FLAG_COUNT 2u  /* add tile-class counts into `counters` */
#define WP_FLAG_MFMA16 4u /* wp_prefill only, d_h = 128 and G = 32: run the
                             v_mfma_f32_16x16x32_bf16 kernel (one MFMA step per
                             32-dim group) instead of the 32x32x16 one; same
                             tiles, same results up to summation order */

/* Largest cutoff value: a group with this cutoff is never pruned. */
#define WP_NEVER_PRUNE 2147483647

/*
 * wp_group_cutoffs -- the per-group integer cutoff table D'_g (host only).
 *
 * f_c = theta^(-2c/d_h) / pos_scale ([notes] section 1.1, Eq. 2-5: the
 * cutoffs come from the scaled frequencies when position scaling is on; a
 * linear position scale s divides every frequency by s).  The per-channel
 * cutoff is D_c = floor(2*pi / f_c) (integer distances, [notes] section 2.1),
 * and D'_g = max of D_c over the channels of dims [g*G, (g+1)*G)
 * ([notes] section 2.3, Eq. 8).  Values at or above 2^31-1 clamp to
 * WP_NEVER_PRUNE.  G = 2 yields the per-channel (exact-rule) table.
 *
 * theta > 0 and pos_scale > 0, finite.  d_h even, G even, G divides d_h
 * (any such G is accepted here, not only the kernels' 16/32).
 * out: host int32[out_len], out_len == d_h / G.  Output is non-decreasing.
 */
wp_status wp_group_cutoffs(double theta, int32_t d_h, int32_t G, double pos_scale,
                           int32_t* out, int32_t out_len);

/*
 * wp_cutoffs_from_freqs -- the group cutoff table from any per-channel
 * frequency vector (host only).
 *
 * freqs: host double[n_ch], n_ch = d_h / 2, the angular frequency of each
 * channel in radians per position exactly as the model rotates (any
 * per-channel or position scaling already applied: the cutoffs follow the
 * scaled frequencies, [notes] section 1.1).  Channel c < trunc_channels keeps
 * integer distances <= floor(alpha * pi / freqs[c]); channels from
 * trunc_channels on are never pruned ([notes] section 2.1, the paragraph
 * after Eq. (6): alpha = 2 is one period and alpha -> infinity prunes
 * nothing; truncating only the first high-frequency channels is one of the
 * ablations summarised around Fig. 8a and Appendix E).  A group of G dims
 * takes the largest cutoff of its channels (section 2.3, Eq. (8)); values
 * at or above 2^31-1 clamp to WP_NEVER_PRUNE.
 * alpha > 0 (+infinity allowed); every freqs[c] finite and > 0;
 * 0 <= trunc_channels <= n_ch; G even and dividing 2*n_ch;
 * out: host int32[out_len], out_len == 2*n_ch / G.
 * wp_prefill and wp_decode need a non-decreasing table: if the group
 * cutoffs would decrease, the call returns WP_ERR_ARG and leaves out
 * untouched.  With freqs[c] = theta^(-2c/d_h) / pos_scale, alpha = 2 and
 * trunc_channels = n_ch the result equals wp_group_cutoffs.
 */
wp_status wp_cutoffs_from_freqs(const double* freqs, int32_t n_ch, double alpha, int32_t trunc_channels,
                                int32_t G, int32_t* out, int32_t out_len);

/*
 * wp_rope_apply -- rotate every channel of x by its position's angle.
 *
 * x: [B, n, H, d_h], dtype WP_DTYPE_BF16 or WP_DTYPE_F32, strides
 *    x_strides = {batch, token, head} in elements.
 * y: [B, n, H, d_h] bf16, strides y_strides.  y may be x itself (in place)
 *    only when x is bf16 with identical strides; any other overlap is an error
 *    the library cannot detect.
 * pos_start: device int64[B] or NULL (all zero).  Token t of batch b sits at
 *    position p = pos_start[b] + t.
 * Channel c rotates by a = p * theta^(-2c/d_h) / pos_scale:
 *    (x, y) -> (x cos a - y sin a, x sin a + y cos a)
 *    ([notes] section 1.1; the rotation matrix in the kongchang.com article's
 *    RoPE paragraph).  The angle is reduced modulo 2*pi in float64; the
 *    rotation runs in float32 and rounds to bf16 (nearest even).
 */
wp_status wp_rope_apply(const void* x, int32_t x_dtype, void* y,
                        int32_t B, int32_t n, int32_t H, int32_t d_h,
                        const int64_t x_strides[3], const int64_t y_strides[3],
                        const int64_t* pos_start, double theta, double pos_scale,
                        void* stream);

/*
 * wp_prefill -- causal WavePrune attention, grouped rule.
 *
 * q [B, n, Hq, d_h], k and v [B, n, Hkv, d_h]: bf16, q and k already rotated
 * (wp_rope_apply).  o [B, n, Hq, d_h] bf16 output.  strides[12] =
 * {q_b, q_t, q_h, k_b, k_t, k_h, v_b, v_t, v_h, o_b, o_t, o_h} in elements.
 * lse: device float[B][Hq][n] (natural-log log-sum-exp of each row) or NULL.
 * Query row i sees keys j <= i at distance i - j; query head h reads kv head
 * h / (Hq / Hkv).  Logit = (1/sqrt(d_h)) * sum over groups g with
 * i - j <= cutoffs[g] of q_g . k_g ([notes] section 2.1, Eq. 6, with the
 * grouped cutoffs of section 2.3, Eq. 8).  Softmax and P.V are unchanged.
 * cutoffs: host int32[d_h/G], non-decreasing, >= 0 (wp_group_cutoffs); may be
 * NULL with WP_FLAG_DENSE.
 * Tiles: (BM queries of one head) x (BN keys) from wp_prefill_tiling; a tile
 * is visited when it holds a causal pair; per group it is skip
 * (cutoff < l_D: no MFMA work), partial (l_D <= cutoff < r_D: compute then
 * mask) or full (cutoff >= r_D), with l_D = max(0, i0 - j1), r_D = i1 - j0
 * on the tile clipped to n.
 * counters (WP_FLAG_COUNT): device int64[3*(d_h/G) + 1]; counters[3g + cls]
 * gains the number of visited tiles whose group g has class cls
 * (0 skip, 1 partial, 2 full), summed over batches and query heads, and
 * counters[3*(d_h/G)] the number of visited tiles.  Counts are added; the
 * caller zeroes the buffer.  May be NULL otherwise.
 * n >= 1, B >= 1, Hkv >= 1, Hq % Hkv == 0.  The k and v token strides must be
 * >= d_h and below 2^30 elements, and one 64-token tile, 63 * token_stride +
 * d_h elements, must span less than 2^31 bytes (K/V tiles are read through
 * 32-bit-addressed buffer resources based at each tile; a sequence may span
 * any number of bytes); otherwise WP_ERR_SHAPE.
 */
wp_status wp_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                     int32_t B, int32_t n, int32_t Hq, int32_t Hkv, int32_t d_h,
                     const int64_t strides[12], const int32_t* cutoffs, int32_t G,
                     uint32_t flags, int64_t* counters, void* stream);

/*
 * wp_prefill_backward -- gradients of the scalar <dO, O> of wp_prefill with
 * respect to q, k and v.
 *
 * With P = exp(S - lse) and Dsum_i = dO_i . O_i: dV_j = sum_i P_ij dO_i,
 * dS_ij = P_ij (dO_i . V_j - Dsum_i), and per group g the same mask as the
 * forward logit: dQ_i,g = (1/sqrt(d_h)) sum_j [i-j <= D'_g] dS_ij k_j,g,
 * dK_j,g = (1/sqrt(d_h)) sum_i [i-j <= D'_g] dS_ij q_i,g; dK and dV are
 * summed over the query heads of a kv head.  The reading notes' section 2.3
 * (its summary of the paper's Appendix C) describes this backward: the head
 * dimension becomes an output axis, the gradient operands are masked per
 * group, and dQ and dK share one mask.  Tiles are classified per group as
 * in wp_prefill; skipped groups contribute nothing.
 * q, k, v, o, dout as wp_prefill's q, k, v, o (o = the forward output), lse
 * the forward's natural-log LSE [B][Hq][n]; dq [B, n, Hq, d_h], dk and dv
 * [B, n, Hkv, d_h] bf16, written (not accumulated).  strides[24] = {q, k, v,
 * o, dout, dq, dk, dv} x {batch, token, head} in elements; the q, k, v and
 * dout token strides must be >= d_h and one 64-token tile of each must span
 * less than 2^31 bytes (as in wp_prefill).  cutoffs and G as in wp_prefill; flags: WP_FLAG_DENSE or
 * 0.  workspace: device memory of at least
 * wp_prefill_backward_workspace_size(B, n, Hq) bytes, 256-byte aligned (two
 * floats per query row: its LSE in base 2 and its row sum Dsum).
 * Asynchronous on stream.
 */
wp_status wp_prefill_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int32_t B, int32_t n,
                              int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[24],
                              const int32_t* cutoffs, int32_t G, uint32_t flags, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Workspace bytes wp_prefill_backward needs. */
size_t wp_prefill_backward_workspace_size(int32_t B, int32_t n, int32_t Hq);

/*
 * wp_decode -- one new query token per sequence against a KV cache.
 *
 * q [B, Hq, d_h] bf16 rotated; k_cache, v_cache [B, Lmax, Hkv, d_h] bf16 (K
 * rotated at its own positions); o [B, Hq, d_h] bf16.
 * strides[10] = {q_b, q_h, k_b, k_t, k_h, v_b, v_t, v_h, o_b, o_h}.
 * cache_len, q_pos: device int32[B].  Cached key j sits at position j; the
 * query at q_pos[b]; keys 0 .. cache_len[b]-1 are attended at distance
 * q_pos[b] - j.  The caller guarantees 1 <= cache_len[b] <= Lmax and
 * q_pos[b] >= cache_len[b] - 1 (not checked: device data); a sequence with
 * cache_len[b] <= 0 gets o = 0.
 * Same rule as wp_prefill; per key block of BN keys (wp_decode_tiling) the K
 * dims of skipped groups are not read ([notes] section 2.3: skipped groups
 * read no K cache).
 * The key blocks are dealt to num_splits splits (0 = automatic, see
 * wp_decode_num_splits; at most one split per key block): split s takes
 * blocks s, s + S, s + 2S, ...  Splits are computed independently, then
 * merged.  Up to 32 query heads of a kv head are computed together, in one
 * pass over the cache; more (Hq / Hkv > 32) run in passes of 32, each
 * reading the cache again.
 * workspace: device memory of at least wp_decode_workspace_size(...) bytes,
 * 256-byte aligned, used for the per-split partial results.
 * counters (WP_FLAG_COUNT): device int64[3*(d_h/G)+1], as in wp_prefill but
 * counted per (sequence, kv head, key block).
 * The cache token strides must be >= d_h and one 32-token block of the cache,
 * 31 * token_stride + d_h elements, must span less than 2^31 bytes (each
 * block is read through its own 32-bit-addressed buffer resources; a cache
 * may span any number of bytes); WP_ERR_SHAPE otherwise.
 */
wp_status wp_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                    const int32_t* cache_len, const int32_t* q_pos,
                    int32_t B, int32_t Lmax, int32_t Hq, int32_t Hkv, int32_t d_h,
                    const int64_t strides[10], const int32_t* cutoffs, int32_t G,
                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                    uint32_t flags, int64_t* counters, void* stream);

/*
 * Group-major compact K cache.
 *
 * Group g of a key is only read while the query is within D'_g of it, and a
 * decoding query never moves back, so group g needs only the keys of the
 * last D'_g + 1 positions.  Keeping just those turns decode's skipped K
 * reads into allocated-capacity savings: the pages leave per-channel
 * eviction of expired K entries as future work and note that fewer reads
 * and a smaller allocated cache are separate gains ([notes] section 2.3,
 * the closing paragraph on what the implementation optimises).
 *
 * The store of one (sequence, kv head) is ng = d_h/G rings, one per group,
 * concatenated: group g has cap[g] = min(Lmax, cutoffs[g] + 1) slots of G
 * bf16 elements at element offset off[g] (off[0] = 0, off[g+1] = off[g] +
 * cap[g]*G); key j of group g sits in slot j % cap[g], so the keys of a
 * group are contiguous and a decode step reads each kept group as one dense
 * run.  A store is addressed with two strides, sequence and kv head, in
 * elements.  The cutoffs passed to every call on one store must be the same
 * table.
 */

/* wp_kcache_layout -- ring sizes caps[ng] and element offsets offsets[ng+1]
 * (offsets[ng] = elements per (sequence, kv head)) of the compact K store
 * (host only).  cutoffs: host int32[d_h/G], non-decreasing, >= 0. */
wp_status wp_kcache_layout(int32_t Lmax, int32_t d_h, int32_t G, const int32_t* cutoffs, int32_t* caps,
                           int64_t* offsets);

/*
 * wp_kcache_append -- write T rotated keys per sequence into the compact
 * store.  k [B, T, Hkv, d_h] bf16, k_strides = {batch, token, head}; token
 * t of sequence b is position pos0[b] + t (pos0: device int32[B], >= 0;
 * the caller keeps pos0[b] + T <= Lmax).  For each group, a key that a
 * later token of the same call replaces in its ring is not written, so the
 * result is the ring after appending the tokens in order.  Appends must be
 * in position order across calls (prefill once, then one token per step).
 * store_strides = {sequence, kv head} >= offsets[ng] elements, regions not
 * overlapping.  Asynchronous on stream.
 */
wp_status wp_kcache_append(const void* k, int32_t B, int32_t T, int32_t Hkv, int32_t d_h,
                           const int64_t k_strides[3], const int32_t* pos0, void* store,
                           const int64_t store_strides[2], int32_t Lmax, const int32_t* cutoffs, int32_t G,
                           void* stream);

/*
 * wp_decode_kcache -- wp_decode with K read from the compact store.
 * strides[9] = {q_b, q_h, store_b, store_h, v_b, v_t, v_h, o_b, o_h}.  The
 * store must hold the keys of positions 0 .. cache_len[b]-1 (appended in
 * order); V is the ordinary cache [B, Lmax, Hkv, d_h].  Keys are read only
 * for groups a key block keeps; a partial group's keys beyond its cutoff may
 * find their slot reused and are masked, as in wp_decode.  Same results as
 * wp_decode on the full cache (the same arithmetic in the same order).
 * WP_FLAG_DENSE is rejected (WP_ERR_ARG); cutoffs must not be NULL;
 * Lmax <= 2^24.  Workspace as for wp_decode.
 */
wp_status wp_decode_kcache(const void* q, const void* k_store, const void* v_cache, void* o,
                           const int32_t* cache_len, const int32_t* q_pos, int32_t B, int32_t Lmax,
                           int32_t Hq, int32_t Hkv, int32_t d_h, const int64_t strides[9],
                           const int32_t* cutoffs, int32_t G, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, uint32_t flags, int64_t* counters, void* stream);

/* Number of key splits wp_decode uses when num_splits == 0: the count that
 * spreads B * Hkv * splits workgroups over the current device's compute
 * units with the fewest keys per unit (at least 128 keys per split). */
int32_t wp_decode_num_splits(int32_t B, int32_t Lmax, int32_t Hkv);

/* Workspace bytes wp_decode needs for these sizes (num_splits 0 = automatic). */
size_t wp_decode_workspace_size(int32_t B, int32_t Lmax, int32_t Hq, int32_t Hkv,
                                int32_t d_h, int32_t num_splits);

/*
 * wp_decode_noalloc -- wp_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, kernels and results as wp_decode
 * (bit-identical for the same num_splits), but the per-split partial
 * results live in a fixed device array inside the library instead of a
 * caller workspace: WP_DECODE_SCRATCH_BYTES (8 MiB) on each GPU, held from
 * the first call on that GPU until the process ends.  The call allocates and
 * frees nothing (no hipMalloc, hipFree or allocating library routine).
 * Errors: WP_ERR_WORKSPACE when wp_decode_workspace_size(B, Lmax, Hq, Hkv,
 * d_h, num_splits) exceeds WP_DECODE_SCRATCH_BYTES (e.g. at d_h = 128,
 * B * Hq * splits above about 16000); WP_ERR_HIP if the array's device
 * address cannot be looked up; otherwise the errors of wp_decode.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (on different streams, or from
 * different threads) race and must be ordered by the caller.
 */
#define WP_DECODE_SCRATCH_BYTES (8u << 20)
wp_status wp_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                            const int32_t* cache_len, const int32_t* q_pos,
                            int32_t B, int32_t Lmax, int32_t Hq, int32_t Hkv, int32_t d_h,
                            const int64_t strides[10], const int32_t* cutoffs, int32_t G,
                            int32_t num_splits, uint32_t flags, int64_t* counters, void* stream);

/* The classification tile of the prefill kernel: BM queries x BN keys. */
wp_status wp_prefill_tiling(int32_t d_h, int32_t G, int32_t* BM, int32_t* BN);

/* The key block of the decode kernel. */
wp_status wp_decode_tiling(int32_t d_h, int32_t G, int32_t* BN);

/*
 * Host-side tile classifier, the same rule and grid the kernels use
 * ([notes] section 2.3 table).  For one (sequence, query head) of length n
 * (prefill) or one (sequence, kv head) with the query at q_pos over keys
 * 0..cache_len-1 (decode).  counts: host int64[3*ng + 1], overwritten, laid
 * out as the kernels' counters.  cutoffs: host int32[ng], non-decreasing.
 */
wp_status wp_prefill_tile_counts(int32_t n, int32_t d_h, int32_t G,
                                 const int32_t* cutoffs, int64_t* counts);
wp_status wp_decode_tile_counts(int32_t q_pos, int32_t cache_len, int32_t d_h, int32_t G,
                                const int32_t* cutoffs, int64_t* counts);

/* Static description of a status code. */
const char* wp_status_string(wp_status s);

/* Message for the last error returned on the calling thread ("" if none). */
const char* wp_last_error(void);

/* Library version, "major.minor.patch". */
const char* wp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WAVEPRUNE_H */
