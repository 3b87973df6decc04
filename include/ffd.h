/*
 * ffd.h -- C ABI of libffd, MI355X-native (gfx950) Faster Flash Decoding.
 *
 * Source of the method: "Faster Than Flash: Exploiting Attention Sparsity for Efficient
 * Long-Context Decoding" (arXiv 2609.00097).  For one new token per sequence, a decode step
 *   1. scans a low-bit copy of every full key block (Sec. 3.1, App. A),
 *   2. estimates a pseudo-max from the sink block and the local block (Sec. 3.2, Eq. 3),
 *   3. keeps a block when its estimated maximum logit is within delta of the pseudo-max
 *      (Sec. 3.2, Eq. 1; no sort, no cross-block synchronization),
 *   4. runs exact softmax(q K^T / sqrt(d)) V over the kept blocks only (Alg. 1, refinement), and
 *   5. merges the per-split partial softmax states with a log-sum-exp combine (the split-KV
 *      decoding of Sec. 2, FlashDecoding).  Steps 1-5 run in one kernel launch; the merge is done
 *      by the last work-group of each work unit (query heads of one kv head) to finish.
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, contiguous device allocations owned by the caller.
 *     The library allocates and frees nothing and keeps no state between calls.
 *   - Every pointer must be 16-byte aligned.
 *   - Shapes (B = batch, Hq = query heads, Hkv = kv heads, d = head_dim = 128, T = block):
 *         q        [B, Hq, d]             dims.dtype (fp32 or bf16)
 *         K, V     [B, Hkv, seq_cap, d]   dims.dtype
 *         Kq       [B, Hkv, seq_cap, d/2] uint8: byte i of a token row holds the 4-bit code of
 *                                         channel 2i in bits 0-3 and of channel 2i+1 in bits 4-7
 *         scales   [B, Hkv, seq_cap/T, d] bf16 bit patterns (uint16): one scale per (block,
 *                                         channel), the binary32 s = RN(max|x| / 7.5) of App. A
 *                                         rounded to nearest bf16 (ties to even)
 *         out      [B, Hq, d]             fp32
 *         lse      [B, Hq]                fp32, natural log of the softmax denominator
 *         keep_mask[B, Hq, ceil(L/T)]     uint8, 1 = block used for that query head
 *     Query head h reads kv head h / (Hq/Hkv) (contiguous groups).
 *   - Query groups: any G = Hq/Hkv >= 1 (Llama-3's 4, Qwen2.5's 7, ...).  A kernel works on a
 *     unit of G_u query heads of one kv head, G_u = 1, 2, 4 or 8, the narrowest that holds G;
 *     other group sizes run padded (3 as 4; 5, 6 and 7 as 8): the padding heads cost arithmetic
 *     but no memory traffic.  Groups of more than 8 are cut into ceil(G/8) units of 8, each of
 *     which reads the kv head's keys (and scans them) on its own.  Units = B * Hkv * ceil(G/8)
 *     must not exceed 65535.
 *   - Calls are asynchronous on `stream` and never synchronize.  They are thread-safe: no
 *     mutable global state.  No C++ exception crosses the ABI.
 *   - Argument validation runs before any HIP call: on failure a call returns
 *     FFD_ERR_INVALID_ARG or FFD_ERR_UNSUPPORTED and launches nothing.  A HIP error reported
 *     right after a launch returns FFD_ERR_HIP.
 *   - NaN or Inf in q, K or V gives unspecified results.
 *
 * Low-bit code and scan definitions (fixed readings of what the paper leaves open):
 *   code u in 0..15 of channel c of a token in block j stands for (u - 7.5) * s[j][c] with
 *   s = RN(amax / 7.5) and amax = max |K| over the block's T tokens in that channel (App. A,
 *   Eqs. 5-7 with 16 levels instead of 4); u = clamp(floor(RN(x * RN(7.5 / amax))) + 8, 0, 15);
 *   amax = 0 gives s = 0 and u = 8.
 *   Estimated block score of query head h (Alg. 1 scan): w_c = RN(q_c * s_c), W = max|w_c|,
 *   wi_c = rint(RN(w_c * RN(127 / W))), E_t = sum_c wi_c * (2 u_tc - 15) in exact integers,
 *   shat_j = RN(float(max_t E_t) * RN(W * kappa)) with kappa = (float)(0.5 / (127 sqrt(d))),
 *   and shat_j = 0 when W = 0.  Pseudo-max: mtilde = max(shat_0, shat_{nf-1}), nf = floor(L/T).
 *   Block j is kept iff j = 0, j >= nf - 1 (local block and a partial tail), or
 *   shat_j >= RN(mtilde - delta).  With nf = 0 every token is kept.
 */
#ifndef FFD_H
#define FFD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FFD_ABI_VERSION 2
#define FFD_BITS 4          /* bits per key channel in the scanned copy */
#define FFD_SINK_BLOCKS 1   /* S_global of Eq. 3: block 0 */
#define FFD_LOCAL_BLOCKS 1  /* S_local of Eq. 3: the last full block */
#define FFD_HEAD_DIM 128    /* the only supported head dimension */

typedef enum {
    FFD_OK = 0,
    FFD_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, NaN/negative delta */
    FFD_ERR_UNSUPPORTED = 2, /* valid but not implemented: head_dim != 128, block not 64/128,
                                more than 65535 work units (see "Query groups") */
    FFD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than ffd_workspace_bytes() */
    FFD_ERR_HIP = 4          /* the HIP runtime reported an error for a launch */
} ffd_status;

typedef enum { FFD_F32 = 0, FFD_BF16 = 1 } ffd_dtype;

typedef struct {
    int32_t batch;      /* B >= 0 (B = 0: every call is a no-op returning FFD_OK) */
    int32_t n_q_heads;  /* Hq >= 1, a multiple of n_kv_heads */
    int32_t n_kv_heads; /* Hkv >= 1 */
    int32_t head_dim;   /* d, must be 128 */
    int32_t seq_len;    /* L >= 1 valid tokens per sequence (the same for every sequence) */
    int32_t seq_cap;    /* row stride of K, V and Kq in tokens: >= seq_len, multiple of block */
    int32_t dtype;      /* ffd_dtype of q, K and V */
} ffd_dims;

/*
 * Low-bit copy of the keys (App. A quantizer; the "K quantization" stage of Fig. 2).
 * Quantizes every block j (0 <= j < seq_cap/block) whose last token index (j+1)*block-1 lies in
 * [tok_begin, tok_end): those are the blocks that become complete when tokens tok_begin..tok_end-1
 * are appended.  Writes rows j*block..(j+1)*block-1 of Kq and row j of scales; leaves every other
 * byte untouched.  Requires 0 <= tok_begin <= tok_end <= seq_len.  Calling it once with (0, L)
 * quantizes a whole cache; calling it once per appended token gives the same bytes.
 */
ffd_status ffd_quantize_k_append(const ffd_dims* dims, const void* K, int32_t tok_begin,
                                 int32_t tok_end, int32_t block, uint8_t* Kq, uint16_t* scales,
                                 hipStream_t stream);

/*
 * Sparse decode step: scan, pseudo-max, top-delta selection, exact attention over kept blocks
 * and split-KV log-sum-exp combine (Alg. 1; Sec. 3.2-3.3).
 *   delta      >= 0, or +inf (keeps every block); NaN is rejected.
 *   block      T in {64, 128}; Kq and scales must hold the quantized full blocks of K.
 *   out, lse   results; lse may be NULL.
 *   keep_mask  optional (NULL) per-(b, query head, block) selection, written as 0/1.
 *   workspace  caller-owned device memory of at least ffd_workspace_bytes(dims, block) bytes,
 *              prepared once by ffd_workspace_init; it holds a counter per work unit (see
 *              "Query groups"), which every call returns to zero, and the per-split partial
 *              softmax states.  Calls that share a workspace must not overlap in time (run them
 *              on one stream).
 */
ffd_status ffd_decode_sparse(const ffd_dims* dims, const void* q, const void* K, const void* V,
                             const uint8_t* Kq, const uint16_t* scales, float delta, int32_t block,
                             float* out, float* lse, uint8_t* keep_mask, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Dense decode step (the exact flash-decoding baseline of Sec. 4.2): softmax(q K^T / sqrt(d)) V
 * over all seq_len tokens, split along the sequence and merged with the same combine.
 * `block` only sets the work granularity (64 or 128); results do not depend on it beyond
 * floating-point rounding.
 */
ffd_status ffd_decode_dense(const ffd_dims* dims, const void* q, const void* K, const void* V,
                            int32_t block, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Residual storage form of the keys (Sec. 3.1 and Fig. 2: a low-bit "thumbnail" plus an 8-bit
 * residual replace the 16-bit keys of full blocks; Alg. 1 rebuilds each kept key with Dequant,
 * Eq. 4 being the same score written as q.k_quant + q.k_res).
 * Writes, for every block completed by tokens [tok_begin, tok_end) (as in ffd_quantize_k_append):
 *   Kc         [B, Hkv, seq_cap, d*bits/8] uint8: thumbnail codes, channel c at bit
 *              (c % (8/bits)) * bits of byte c / (8/bits) of the token row (App. A quantizer
 *              with 2^bits levels: value (u - (2^bits-1)/2) * s; bits = 2 is App. A exactly)
 *   scales     [B, Hkv, seq_cap/T, d] bf16 bits: thumbnail scale, the binary32
 *              RN(max|x| / ((2^bits-1)/2)) rounded to nearest bf16 (ties to even); the codes use
 *              the binary32 reciprocal RN(((2^bits-1)/2) / max|x|), the residual the stored s
 *   Kr         [B, Hkv, seq_cap, d] int8: residual code of r = RN(x - RN((u - half) s)),
 *              clamp(rint(RN(r * RN(127 / max|r|))), -127, 127), max over the block's T tokens
 *   res_scales [B, Hkv, seq_cap/T, d] fp32: s_r = RN(max|r| / 127) (0 when max|r| = 0)
 * K must be bf16 (dims.dtype == FFD_BF16); bits must be 2 or 4 (else FFD_ERR_UNSUPPORTED).
 * Rebuilt key (Dequant): (u - half) * s + r_q * s_r, within s_r / 2 of the stored key.
 */
ffd_status ffd_quantize_k_residual_append(const ffd_dims* dims, const void* K, int32_t tok_begin,
                                          int32_t tok_end, int32_t block, int32_t bits,
                                          uint8_t* Kc, uint16_t* scales, int8_t* Kr,
                                          float* res_scales, hipStream_t stream);

/*
 * Sparse decode step in the residual storage form: the scan reads the bits-wide thumbnail; the
 * refinement attends over the kept blocks with Dequant keys (fp32, fed to the bf16 MFMA as a
 * high/low bf16 pair) and bf16 values.  K_tail [B, Hkv, seq_cap, d] bf16 supplies the keys of
 * the partial tail block (rows floor(L/T)*T .. L-1 only; NULL is allowed when L % T == 0).
 * Same outputs, workspace and errors as ffd_decode_sparse; q and V bf16 only.
 */
ffd_status ffd_decode_sparse_residual(const ffd_dims* dims, const void* q, const void* K_tail,
                                      const void* V, const uint8_t* Kc, const uint16_t* scales,
                                      const int8_t* Kr, const float* res_scales, int32_t bits,
                                      float delta, int32_t block, float* out, float* lse,
                                      uint8_t* keep_mask, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * Decode loop (Sec. 3.3: the fused step runs once per generated token; Fig. 2: the low-bit key
 * copy is maintained as blocks complete; App. G / Table 9: the step is replayed as a graph).
 * Everything a step needs lives in device memory, so one captured step (append + decode) can be
 * replayed for every token, across block boundaries, with no re-capture.
 *
 * ffd_append_token: for every sequence b (and every kv head), writes the new token's key and value
 * rows k_new[b, g, :] and v_new[b, g, :] at position seq_lens[b] of K and V; if that token
 * completes key block j = seq_lens[b] / block, quantizes block j into Kq/scales exactly as
 * ffd_quantize_k_append does; then increments seq_lens[b].
 *   k_new, v_new  [B, Hkv, d] in dims->dtype
 *   K, V, Kq, scales  the caches (layouts of ffd_decode_sparse), updated in place
 *   seq_lens   device int32 [B], the current lengths; a sequence already at dims->seq_cap (or
 *              with a negative length) is left unchanged and nothing of it is written
 * dims->seq_len is not used (it must still be valid). One kernel launch, no host synchronisation.
 */
ffd_status ffd_append_token(const ffd_dims* dims, const void* k_new, const void* v_new, void* K,
                            void* V, int32_t* seq_lens, int32_t block, uint8_t* Kq,
                            uint16_t* scales, hipStream_t stream);

/*
 * Sparse (and dense) decode step with per-sequence lengths read from device memory: sequence b
 * attends over its first seq_lens[b] tokens, clamped to [0, dims->seq_len]; dims->seq_len is the
 * bound the splits cover (normally dims->seq_cap) and sizes the workspace.  Everything else is as
 * in ffd_decode_sparse / ffd_decode_dense; keep_mask rows are ceil(dims->seq_len / block) long,
 * and entries past a sequence's own blocks are not written.  A sequence of length 0 gets out = 0
 * and lse = -inf.
 */
ffd_status ffd_decode_sparse_varlen(const ffd_dims* dims, const void* q, const void* K,
                                    const void* V, const uint8_t* Kq, const uint16_t* scales,
                                    const int32_t* seq_lens, float delta, int32_t block,
                                    float* out, float* lse, uint8_t* keep_mask, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);
ffd_status ffd_decode_dense_varlen(const ffd_dims* dims, const void* q, const void* K,
                                   const void* V, const int32_t* seq_lens, int32_t block,
                                   float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * One decode-loop step in one launch (Sec. 3.3: one fused kernel per generated token; App. G /
 * Table 9: the step replayed as a graph): ffd_append_token followed by ffd_decode_sparse_varlen,
 * with the same results, bytes and lengths as that pair of calls when dims->seq_len is the
 * capacity (the pair appends below the capacity; this call below dims->seq_len, the length its
 * splits cover).  For every sequence b whose
 * length l = seq_lens[b] satisfies 0 <= l < dims->seq_len: the rows k_new[b, g, :] and
 * v_new[b, g, :] go to position l of K and V, the key block they complete (if any) is quantized
 * into Kq/scales, the sequence attends over its first l + 1 tokens, and seq_lens[b] becomes
 * l + 1.  Any other sequence is decoded at its clamped length and left unchanged.
 *   k_new, v_new  [B, Hkv, d] in dims->dtype, 16-byte aligned
 *   K, V, Kq, scales, seq_lens  updated in place (layouts of ffd_decode_sparse)
 * dims->seq_len is the bound the splits cover (normally dims->seq_cap), as in the varlen call.
 * The workspace's counter region also holds one count per sequence (its top B slots), returned to
 * zero by the call; FFD_ERR_UNSUPPORTED when work units + B exceed its 65535 slots.
 */
ffd_status ffd_decode_sparse_append(const ffd_dims* dims, const void* q, const void* k_new,
                                   const void* v_new, void* K, void* V, uint8_t* Kq,
                                   uint16_t* scales, int32_t* seq_lens, float delta, int32_t block,
                                   float* out, float* lse, uint8_t* keep_mask, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Selection comparators and fidelity diagnostics (Sec. 4.5 Table 3: top-delta against top-k and
 * top-p at a matched keep ratio; Sec. 5.1 Fig. 6: a Quest-style min/max scan as the comparator;
 * Sec. 3.2 Eq. 3 and Sec. 5.2 Fig. 5: the pseudo-max from exact scores and its gap to the true
 * maximum).  Unlike ffd_decode_sparse, which decides each block as it scans it, these run as
 * separate steps: per-block scores, then a rule over every block of a (sequence, query head),
 * then exact attention over the chosen blocks.
 */
typedef enum {
    FFD_SCORE_SCAN = 0,    /* the scan estimate of the block's largest score (Alg. 1), from Kq/scales */
    FFD_SCORE_BOUNDS = 1,  /* sum_c max(q_c kmin_c, q_c kmax_c) / sqrt(d): an upper bound from the
                              block's per-channel min/max (Quest-style page metadata) */
    FFD_SCORE_EXACT = 2    /* the block's exact largest score max_t q.k_t / sqrt(d), from K */
} ffd_score_kind;

typedef enum {
    FFD_SELECT_TOP_DELTA = 0,  /* Eq. 1: keep s_j >= RN(mtilde - param); mtilde = pseudo_max[row]
                                  if given, else max(s_0, s_{nf-1}) (Alg. 1) */
    FFD_SELECT_TOP_K = 1,      /* the floor(param) highest-scoring full blocks */
    FFD_SELECT_TOP_P = 2       /* the fewest highest-scoring full blocks whose share
                                  exp(s_j - max s) / sum_i exp(s_i - max s) reaches param */
} ffd_select_rule;

/* Per-channel min and max over every key block completed by tokens [tok_begin, tok_end) (the
 * blocks of ffd_quantize_k_append): kmin, kmax [B, Hkv, seq_cap/block, d] in dims->dtype. */
ffd_status ffd_block_bounds(const ffd_dims* dims, const void* K, int32_t tok_begin,
                            int32_t tok_end, int32_t block, void* kmin, void* kmax,
                            hipStream_t stream);

/* Scores of every full block (nf = dims->seq_len / block of them) for every query head:
 * scores [B, Hq, nf] fp32.  FFD_SCORE_SCAN needs Kq and scales (bit-identical to the decode
 * kernel's estimates), FFD_SCORE_BOUNDS kmin and kmax, FFD_SCORE_EXACT K; the other inputs may
 * be NULL.  q is [B, Hq, d] in dims->dtype. */
ffd_status ffd_block_scores(const ffd_dims* dims, int32_t kind, const void* q, const void* K,
                            const uint8_t* Kq, const uint16_t* scales, const void* kmin,
                            const void* kmax, int32_t block, float* scores, hipStream_t stream);

/* One selection rule over every row of scores [B, Hq, nf] -> keep_mask [B, Hq, ceil(seq_len /
 * block)] (0/1).  Every rule also keeps block 0, the last full block and a partial tail.  Full
 * blocks are ranked by score, ties going to the lower index.  param: delta (>= 0 or +inf) for
 * top-delta, k (>= 0) for top-k, p in (0, 1] for top-p; pseudo_max [B, Hq] (optional, top-delta
 * only) replaces Alg. 1's max(s_0, s_{nf-1}), e.g. by the exact-score maximum of Eq. 3.  Top-k and
 * top-p hold each row in LDS: nf <= 16384 (else FFD_ERR_UNSUPPORTED).  Top-p evaluates each mass
 * in fp32 and sums them exactly as integer multiples of 2^-40. */
ffd_status ffd_select_blocks(const ffd_dims* dims, int32_t rule, const float* scores,
                             const float* pseudo_max, float param, int32_t block,
                             uint8_t* keep_mask, hipStream_t stream);

/* Exact attention and split combine over the blocks a caller-made keep_mask [B, Hq,
 * ceil(seq_len / block)] marks (per query head), e.g. from ffd_select_blocks; otherwise as
 * ffd_decode_sparse (same workspace).  A head with no kept block gets out = 0, lse = -inf. */
ffd_status ffd_decode_masked(const ffd_dims* dims, const void* q, const void* K, const void* V,
                             const uint8_t* keep_mask, int32_t block, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Running-max variant of the sparse step (Sec. 1 Fig. 1: a threshold relative to the local max,
 * with no global sort or synchronisation; Alg. 1's pseudo-max as the starting point).  The
 * sequence is cut into windows of `window` blocks, each one split (work-group) of the step; in
 * each window, per query head and in increasing block order, a full block that is not forced is
 * kept iff its scan estimate is >= RN(M - delta), where M is the maximum of Alg. 1's pseudo-max
 * and the estimates of the window's earlier non-forced full blocks.  Forced blocks (0, the last
 * full block, a partial tail) are kept.  So the kept set is a subset of ffd_decode_sparse's at the
 * same delta, equal to it for window = 1.  Arguments as ffd_decode_sparse, plus
 *   window     blocks per window, 1 <= window <= 256, with ceil(seq_len / block / window) <= 256
 *              (else FFD_ERR_UNSUPPORTED)
 *   workspace  at least ffd_workspace_bytes_window(dims, block, window) bytes. */
ffd_status ffd_decode_sparse_running(const ffd_dims* dims, const void* q, const void* K,
                                     const void* V, const uint8_t* Kq, const uint16_t* scales,
                                     float delta, int32_t block, int32_t window, float* out,
                                     float* lse, uint8_t* keep_mask, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc): ffd_decode_sparse with the library's own fixed scratch area
 * in place of a caller's workspace.  Same arguments (minus the workspace), same kernels, same
 * results as ffd_decode_sparse.
 *   - The scratch area is a file-scope device array of FFD_NOALLOC_SCRATCH_BYTES (16 MiB) per
 *     GPU, held from the first call on that GPU until the process ends.  A call whose dims need
 *     more (ffd_workspace_bytes is an upper bound of the need) returns FFD_ERR_WORKSPACE and
 *     launches nothing.
 *   - The first call on a device (the current device) looks up the area's address and zeroes its
 *     counters with a kernel on `stream`; it should not be the call under graph capture.  Nothing
 *     is allocated, then or later (no hipMalloc, hipFree or allocating library routine).
 *   - Every call on a GPU shares that GPU's area: calls that overlap in time on one GPU (other
 *     streams, other threads) race and give wrong results.  Serialize them (one stream).
 */
#define FFD_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
ffd_status ffd_decode_sparse_noalloc(const ffd_dims* dims, const void* q, const void* K,
                                     const void* V, const uint8_t* Kq, const uint16_t* scales,
                                     float delta, int32_t block, float* out, float* lse,
                                     uint8_t* keep_mask, hipStream_t stream);

/* Workspace bytes of ffd_decode_sparse_running for this window; 0 for invalid arguments. */
size_t ffd_workspace_bytes_window(const ffd_dims* dims, int32_t block, int32_t window);

/* Workspace bytes needed by ffd_decode_sparse / ffd_decode_dense for these dims and block
 * (the maximum of the two); 0 for invalid dims.  The size depends on the split count, which the
 * environment variable FFD_NUM_SPLITS (a positive integer) overrides. */
size_t ffd_workspace_bytes(const ffd_dims* dims, int32_t block);

/* Prepares a workspace for the decode calls: zeroes its counter region (the first 524,288
 * bytes: one 8-byte counter for each of the at most 65535 work units of a call, rounded up to
 * 256) with a small kernel on `stream` (no memset, so it may be recorded into a graph).
 * FFD_ERR_WORKSPACE if workspace_bytes is smaller than that region; each decode call checks its
 * own size.  Needed once per new allocation: every completed decode call returns the counters it
 * used to zero, so a prepared workspace stays prepared for later calls with any dims and block it
 * is large enough for (dims and block are validated but do not change what is zeroed). */
ffd_status ffd_workspace_init(const ffd_dims* dims, int32_t block, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Number of sequence splits (work-groups per (sequence, kv head)) that ffd_decode_sparse (sparse
 * != 0) or ffd_decode_dense (sparse == 0) uses for these dims and block; 0 for invalid dims. */
int32_t ffd_num_splits(const ffd_dims* dims, int32_t block, int32_t sparse);

/* Static description of a status code. */
const char* ffd_status_string(ffd_status status);

/* FFD_ABI_VERSION of the loaded library. */
int32_t ffd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFD_H */
