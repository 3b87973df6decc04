/*
 * ffd_oracle.c -- CPU oracle for Faster Flash Decoding (FFD) sparse decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, obviously-correct reference that the
 * tests, the package's smoke check and the benchmark's CPU-baseline leg call to check the HIP
 * library.  The product path never links, loads or calls it, and it shares no code, header,
 * table or constant generator with the HIP library.
 *
 * Source: the paper "Faster Than Flash: Exploiting Attention Sparsity for Efficient
 * Long-Context Decoding" (arXiv 2609.00097), cited below as FTF.
 *
 * What it computes, for one new token per sequence (one query vector per query head):
 *   O1  quantize     App. A, Eqs. 5-7: symmetric mid-rise (zero-free) uniform quantizer of each
 *                    channel vector of a block of keys, generalized from 4 levels to 2^bits levels.
 *   O2  scan         Alg. 1, top-delta selection stage: estimated score of every token of every
 *                    full block from the low-bit keys; block score = max over the block.
 *   O5  pseudo-max   Eq. 3 and Alg. 1, pseudo-max stage: max estimated score over the sink block
 *                    and the local block.
 *   O6/O7 select     Eq. 1 with the pseudo-max in place of the true max: keep block j iff its
 *                    estimated max >= pseudo-max - delta.
 *   O8  attention    Alg. 1, refinement stage: exact softmax(q K^T / sqrt(d)) V over the tokens of
 *                    the kept blocks, in double precision.
 *   O9  dense        the same over every token (FlashAttention-style exact decode, FTF Sec. 2).
 *   R1-R4 residual storage form (Sec. 3.1, Fig. 2, Alg. 1 Dequant, Eq. 4): a 2- or 4-bit
 *                    thumbnail plus an 8-bit residual replaces the 16-bit keys of full blocks;
 *                    the scan reads the thumbnail, the refinement attends over Dequant keys
 *                    (see the section at the end of this file for its readings).
 *
 * Readings of points the paper leaves open (each is also listed in the design notes):
 *   - Quantizer levels: value of code u is (u - (2^bits-1)/2) * s, s = amax / ((2^bits-1)/2).
 *     For bits = 2 this is exactly App. A (codebook {-1.5,-0.5,+0.5,+1.5}, s = max|x| / 1.5).
 *   - Quantizer rounding: s = RN(amax/half), inv = RN(half/amax), y = RN(x*inv),
 *     u = clamp(floor(y) + 2^(bits-1), 0, 2^bits - 1).  floor(y) + 2^(bits-1) is the index of the
 *     nearest codeword (Eq. 7); a value exactly on a bin boundary goes to the upper bin.
 *     amax == 0 gives s = 0 and every code = 2^(bits-1).
 *   - Scale group: one scale per (block of T tokens, channel).
 *   - Scale storage: each block scale is kept as bf16, the binary32 s rounded to the nearest
 *     bf16 value (8 significant bits), ties to even.  The codes are those of the binary32
 *     quantizer above; the scan and Dequant read the stored bf16 scale.
 *   - Scan arithmetic (integer-exact): per (query head, block) w_c = RN(q_c * s_c) (s_c the
 *     stored bf16 scale),
 *     W = max_c |w_c|; if W == 0 all estimates are 0; otherwise rho = RN(127/W),
 *     wi_c = rint_even(RN(w_c*rho)) clamped to [-127,127], E_t = sum_c wi_c * (2u_tc - (2^bits-1))
 *     (exact integer), f = RN(W * kappa) with kappa = (float)(0.5 / (127 * sqrt(d))) and the
 *     estimated score shat_t = RN((float)E_t * f).  The 1/sqrt(d) of Eq. 1 is included so that
 *     estimates, pseudo-max and delta share logit units.
 *   - Pseudo-max source: the estimated scores (as in Alg. 1's pseudo-max stage), over sink block 0
 *     and the last full block (the local block).
 *   - Forced blocks: block 0, the last full block and a partial tail block are always kept; the
 *     tail has no low-bit copy and is not part of the pseudo-max.  With no full block every token
 *     is kept.
 *   - Threshold: theta = RN(mtilde - delta) in float; keep iff shat_block >= theta.
 *   - Exact scores use the stored key (bf16 or fp32 values), not the dequantized low-bit key.
 *
 * All float operations above are single IEEE binary32 operations, round-to-nearest-even; the
 * file is built with -ffp-contract=off and without fast-math so that none are fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FFDO_DTYPE_F32 0
#define FFDO_DTYPE_BF16 1

int ffdo_version(void) { return 1; }

/* Element t*ld + c of a key/value array stored as fp32 or as bf16 bit patterns. */
static float load_elem(const void* base, int dtype, size_t idx)
{
    if (dtype == FFDO_DTYPE_F32) return ((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16; /* bf16 = top half of fp32 */
    float v;
    memcpy(&v, &bits, sizeof v);
    return v;
}

/*
 * Storage of a block scale: round-to-nearest-even from binary32 to bf16 (the upper 16 bits of a
 * binary32 whose lower 16 bits are zero).  Adding 0x7FFF plus the lowest kept bit to the bit
 * pattern and truncating rounds to nearest with ties to even, also across a binade and up to
 * infinity; a NaN keeps its sign and becomes a quiet NaN.
 */
static uint16_t round_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static float bf16_value(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

/* round_to_bf16 over an array (exported so that its rounding can be pinned). */
void ffdo_round_bf16(const float* x, uint16_t* y, int n)
{
    for (int i = 0; i < n; ++i) y[i] = round_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* O1: App. A quantizer for one channel vector x[0..n) (stride `stride` floats).               */
/* ------------------------------------------------------------------------------------------ */
void ffdo_quantize_channel(const float* x, int n, int stride, int bits, uint8_t* codes,
                           float* scale_out)
{
    const int levels = 1 << bits;
    const float half = (float)(levels - 1) * 0.5f; /* 1.5 for 2 bits, 7.5 for 4 bits */
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(x[(size_t)i * stride]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale_out = 0.0f;
        for (int i = 0; i < n; ++i) codes[i] = (uint8_t)(levels / 2);
        return;
    }
    const float s = amax / half;   /* Eq. 6, one rounding */
    const float inv = half / amax; /* one rounding */
    *scale_out = s;
    for (int i = 0; i < n; ++i) {
        const float y = x[(size_t)i * stride] * inv; /* one rounding */
        int u = (int)floorf(y) + levels / 2;        /* nearest codeword index, Eq. 7 */
        if (u < 0) u = 0;
        if (u > levels - 1) u = levels - 1;
        codes[i] = (uint8_t)u;
    }
}

/*
 * O1 for one (batch, kv-head) slice.  K is [L_cap][d] (fp32 or bf16 bits).  Every full block j
 * whose last token index (j+1)*T-1 lies in [tok_begin, tok_end) is quantized:
 *   Kq[t][i] = code(t, 2i) | code(t, 2i+1) << 4      (4-bit codes, two channels per byte)
 *   scales[j][c] = s of channel c of block j, stored as bf16 bits.
 * Returns the number of blocks written.
 */
int ffdo_quantize_k(const void* K, int dtype, int L_cap, int d, int T, int tok_begin,
                    int tok_end, uint8_t* Kq, uint16_t* scales)
{
    if (d % 2 || T <= 0 || L_cap % T) return -1;
    const int n_cap_blocks = L_cap / T;
    float* x = (float*)malloc(sizeof(float) * (size_t)T);
    uint8_t* codes = (uint8_t*)malloc((size_t)T * (size_t)d);
    uint8_t* col = (uint8_t*)malloc((size_t)T);
    int written = 0;
    for (int j = 0; j < n_cap_blocks; ++j) {
        const int last = (j + 1) * T - 1;
        if (last < tok_begin || last >= tok_end) continue;
        for (int c = 0; c < d; ++c) {
            for (int t = 0; t < T; ++t) x[t] = load_elem(K, dtype, (size_t)(j * T + t) * d + c);
            float s;
            ffdo_quantize_channel(x, T, 1, 4, col, &s);
            scales[(size_t)j * d + c] = round_to_bf16(s);
            for (int t = 0; t < T; ++t) codes[(size_t)t * d + c] = col[t];
        }
        for (int t = 0; t < T; ++t) {
            uint8_t* row = Kq + (size_t)(j * T + t) * (d / 2);
            for (int i = 0; i < d / 2; ++i)
                row[i] = (uint8_t)(codes[(size_t)t * d + 2 * i] |
                                   (codes[(size_t)t * d + 2 * i + 1] << 4));
        }
        ++written;
    }
    free(x);
    free(codes);
    free(col);
    return written;
}

/* ------------------------------------------------------------------------------------------ */
/* O2: integer-exact scan.                                                                     */
/* ------------------------------------------------------------------------------------------ */
float ffdo_kappa(int d) { return (float)(0.5 / (127.0 * sqrt((double)d))); }

/*
 * Requantization of w = q (.) s for one (query head, block): writes wi[0..d) and returns
 * f = RN(W*kappa) (0 when W == 0, in which case every wi is 0).
 */
float ffdo_requant(const float* qh, const float* s, int d, int32_t* wi)
{
    float W = 0.0f;
    for (int c = 0; c < d; ++c) {
        const float w = qh[c] * s[c];
        if (fabsf(w) > W) W = fabsf(w);
    }
    if (W == 0.0f) {
        for (int c = 0; c < d; ++c) wi[c] = 0;
        return 0.0f;
    }
    const float rho = 127.0f / W;
    for (int c = 0; c < d; ++c) {
        const float w = qh[c] * s[c];
        float v = rintf(w * rho); /* ties to even under the default rounding mode */
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        wi[c] = (int32_t)v;
    }
    return W * ffdo_kappa(d);
}

/* The stored bf16 scales of one block as binary32 values. */
static void block_scales(const uint16_t* scales, int j, int d, float* s)
{
    for (int c = 0; c < d; ++c) s[c] = bf16_value(scales[(size_t)j * d + c]);
}

/*
 * Scan of one query head over the full blocks of its kv-head slice.
 *   qh[d]                      query (fp32 values)
 *   Kq[n_full*T][d/2]          packed 4-bit codes
 *   scales[n_full][d]          bf16 bits
 * Outputs: shat_block[n_full] (block estimate = max over its tokens) and, if non-NULL,
 * shat_tok[n_full*T] and E_tok[n_full*T] (the exact integer sums).
 */
void ffdo_scan_head(const float* qh, const uint8_t* Kq, const uint16_t* scales, int n_full,
                    int T, int d, float* shat_block, float* shat_tok, int32_t* E_tok)
{
    int32_t* wi = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
    float* sf = (float*)malloc(sizeof(float) * (size_t)d);
    for (int j = 0; j < n_full; ++j) {
        block_scales(scales, j, d, sf);
        const float f = ffdo_requant(qh, sf, d, wi);
        float best = -INFINITY;
        for (int t = 0; t < T; ++t) {
            const uint8_t* row = Kq + (size_t)(j * T + t) * (d / 2);
            int64_t E = 0;
            for (int c = 0; c < d; ++c) {
                const int u = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 15);
                E += (int64_t)wi[c] * (int64_t)(2 * u - 15);
            }
            const float sh = (float)E * f;
            if (shat_tok) shat_tok[(size_t)j * T + t] = sh;
            if (E_tok) E_tok[(size_t)j * T + t] = (int32_t)E;
            if (sh > best) best = sh;
        }
        shat_block[j] = best;
    }
    free(wi);
    free(sf);
}

/* ------------------------------------------------------------------------------------------ */
/* O5-O7: relative threshold and block mask of one query head (Eq. 1 with Eq. 3).              */
/* ------------------------------------------------------------------------------------------ */
/*
 * Eq. 1 keeps a block when its largest score is no more than delta below the largest score of
 * the whole attention row.  That maximum is unknown before every block has been scored, so Eq. 3
 * stands a reference in for it: the largest score over a few anchor blocks on which attention
 * concentrates, the sink at the start of the sequence and the most recent tokens.  Here the
 * scores are the scan estimates, the anchors are block 0 and the last full block, and the
 * anchors, together with a partial tail block (which has no low-bit copy), are kept with no test.
 *
 * est[n_full] are the estimates of the full blocks; keep[n_blocks] receives 0/1, n_blocks =
 * ceil(L/T).  ref_out and cut_out (may be NULL) receive the reference and the cut RN(ref - delta);
 * both are NaN when there is no full block, and then every block is kept.
 */
static int anchor_or_tail(int j, int n_full) { return j == 0 || j >= n_full - 1; }

void ffdo_select_head(const float* est, int n_full, int n_blocks, float delta, uint8_t* keep,
                      float* ref_out, float* cut_out)
{
    if (n_full == 0) {
        memset(keep, 1, (size_t)n_blocks);
        if (ref_out) *ref_out = NAN;
        if (cut_out) *cut_out = NAN;
        return;
    }
    const int anchors[2] = {0, n_full - 1};
    float ref = -INFINITY;
    for (int a = 0; a < 2; ++a)
        if (est[anchors[a]] > ref) ref = est[anchors[a]];
    const float cut = ref - delta; /* one binary32 subtraction; delta = +inf gives -inf */
    for (int j = 0; j < n_blocks; ++j)
        keep[j] = (uint8_t)(anchor_or_tail(j, n_full) || est[j] >= cut);
    if (ref_out) *ref_out = ref;
    if (cut_out) *cut_out = cut;
}

/* ------------------------------------------------------------------------------------------ */
/* O8/O9: exact attention over the tokens of kept blocks, in double precision.                 */
/* ------------------------------------------------------------------------------------------ */
/*
 * One query head.  K, V: [L_cap][d] slices (fp32 or bf16 bits), tokens 0..L-1 valid.
 * keep: [ceil(L/T)] block mask, or NULL for dense.  out[d] and lse receive
 * o = sum_t p_t V_t with p = softmax over kept tokens of s_t = q.K_t / sqrt(d), and
 * lse = log sum_t exp(s_t).
 */
void ffdo_attend_head(const float* qh, const void* K, const void* V, int dtype, int L, int d,
                      int T, const uint8_t* keep, double* out, double* lse)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
        if (keep && !keep[t / T]) { s[t] = -INFINITY; continue; }
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += (double)qh[c] * (double)load_elem(K, dtype, (size_t)t * d + c);
        s[t] = acc * inv_sqrt_d;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int t = 0; t < L; ++t) {
        if (s[t] == -INFINITY) continue;
        const double p = exp(s[t] - m);
        l += p;
        for (int c = 0; c < d; ++c) out[c] += p * (double)load_elem(V, dtype, (size_t)t * d + c);
    }
    for (int c = 0; c < d; ++c) out[c] /= l;
    *lse = m + log(l);
    free(s);
}

/* ------------------------------------------------------------------------------------------ */
/* Batch driver: the whole decode step, OpenMP over (batch, query head).                       */
/* ------------------------------------------------------------------------------------------ */
/*
 * q       [B][Hq][d]              fp32 or bf16 bits
 * K, V    [B][Hkv][L_cap][d]      fp32 or bf16 bits
 * Kq      [B][Hkv][L_cap][d/2]    packed codes      (sparse mode only)
 * scales  [B][Hkv][L_cap/T][d]    bf16 bits         (sparse mode only)
 * sparse  1: O2-O8, 0: O9 (dense)
 * out     [B][Hq][d] double, lse [B][Hq] double
 * keep    [B][Hq][ceil(L/T)] (sparse, may be NULL)
 * shat    [B][Hq][floor(L/T)] block estimates (sparse, may be NULL)
 * mtilde  [B][Hq] (sparse, may be NULL)
 * Query head h reads kv head h / (Hq/Hkv).  Returns the number of (b, h) rows done.
 */
int ffdo_decode(int B, int Hq, int Hkv, int d, int L, int L_cap, int T, int dtype,
                const void* q, const void* K, const void* V, const uint8_t* Kq,
                const uint16_t* scales, float delta, int sparse, double* out, double* lse,
                uint8_t* keep, float* shat, float* mtilde, int n_threads)
{
    if (Hkv <= 0 || Hq % Hkv || d % 2 || T <= 0 || L < 0 || L > L_cap || L_cap % T) return -1;
    const int G = Hq / Hkv;
    const int n_full = L / T;
    const int n_blocks = (L + T - 1) / T;
    const size_t esz = dtype == FFDO_DTYPE_F32 ? 4 : 2;
    const int rows = B * Hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int r = 0; r < rows; ++r) {
        const int b = r / Hq, h = r % Hq, g = h / G;
        float* qh = (float*)malloc(sizeof(float) * (size_t)d);
        for (int c = 0; c < d; ++c) qh[c] = load_elem(q, dtype, (size_t)r * d + c);
        const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)L_cap * d;
        const char* Kbg = (const char*)K + kv_off * esz;
        const char* Vbg = (const char*)V + kv_off * esz;
        uint8_t* kp = NULL;
        if (sparse) {
            const uint8_t* Kq_bg = Kq + ((size_t)b * Hkv + g) * (size_t)L_cap * (d / 2);
            const uint16_t* sc_bg = scales + ((size_t)b * Hkv + g) * (size_t)(L_cap / T) * d;
            float* sb = (float*)malloc(sizeof(float) * (size_t)(n_full > 0 ? n_full : 1));
            kp = (uint8_t*)malloc((size_t)(n_blocks > 0 ? n_blocks : 1));
            ffdo_scan_head(qh, Kq_bg, sc_bg, n_full, T, d, sb, NULL, NULL);
            float mt;
            ffdo_select_head(sb, n_full, n_blocks, delta, kp, &mt, NULL);
            if (keep) memcpy(keep + (size_t)r * n_blocks, kp, (size_t)n_blocks);
            if (shat) memcpy(shat + (size_t)r * n_full, sb, sizeof(float) * (size_t)n_full);
            if (mtilde) mtilde[r] = mt;
            free(sb);
        }
        ffdo_attend_head(qh, Kbg, Vbg, dtype, L, d, T, kp, out + (size_t)r * d, lse + r);
        free(kp);
        free(qh);
    }
    return rows;
}

/* ========================================================================================== */
/* Storage form of FTF Sec. 3.1 / Fig. 2: the key cache split into a low-bit thumbnail and an  */
/* 8-bit residual; Alg. 1's Dequant rebuilds the key for the refinement stage (Eq. 4 is the    */
/* same quantity written as two dot products).                                                 */
/*                                                                                             */
/* Readings (the paper fixes the thumbnail quantizer, App. A, but not the residual's):         */
/*   - thumbnail: the App. A quantizer with 2^bits levels, bits = 2 (App. A exactly) or 4;     */
/*     codes packed little-endian in bytes, channel c at bit (c % (8/bits)) * bits of byte     */
/*     c / (8/bits) of its token row;                                                          */
/*   - the thumbnail scale s is stored as bf16 (as in the 4-bit key copy), and the residual    */
/*     is taken against the stored value: r = RN(x - RN((u - half) * s)) in fp32;             */
/*   - residual quantizer: symmetric 8-bit per (block, channel): s_r = RN(max|r| / 127),       */
/*     r_q = clamp(rint(RN(r * RN(127 / max|r|))), -127, 127); max|r| = 0 gives s_r = 0, r_q=0;*/
/*   - Dequant: k = (u - half) * s + r_q * s_r (evaluated in double here);                     */
/*   - a partial tail block (tokens after the last full block) has no low-bit copy: its keys   */
/*     are read from a 16-bit key buffer.                                                      */
/* ========================================================================================== */

static int code_at(const uint8_t* row, int c, int bits)
{
    const int per = 8 / bits;
    return (row[c / per] >> ((c % per) * bits)) & ((1 << bits) - 1);
}

/* Residual quantizer for one channel vector r[0..n) (stride 1). */
void ffdo_quantize_residual(const float* r, int n, int8_t* rq, float* scale_out)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float a = fabsf(r[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale_out = 0.0f;
        for (int i = 0; i < n; ++i) rq[i] = 0;
        return;
    }
    *scale_out = amax / 127.0f;
    const float inv = 127.0f / amax;
    for (int i = 0; i < n; ++i) {
        float v = rintf(r[i] * inv);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        rq[i] = (int8_t)v;
    }
}

/*
 * Thumbnail + residual of the completed blocks of one (batch, kv-head) slice K [L_cap][d]
 * (fp32 or bf16 bits); blocks whose last token lies in [tok_begin, tok_end) are written:
 *   Kc [L_cap][d*bits/8] packed codes, sc [L_cap/T][d] thumbnail scales (bf16 bits),
 *   Kr [L_cap][d] int8 residual codes, sr [L_cap/T][d] residual scales.
 * Returns the number of blocks written (or -1 for bad sizes).
 */
int ffdo_quantize_k_res(const void* K, int dtype, int L_cap, int d, int T, int bits,
                        int tok_begin, int tok_end, uint8_t* Kc, uint16_t* sc, int8_t* Kr,
                        float* sr)
{
    if ((bits != 2 && bits != 4) || d % (8 / bits) || T <= 0 || L_cap % T) return -1;
    const int per = 8 / bits;
    const int row_bytes = d / per;
    const float half = (float)((1 << bits) - 1) * 0.5f;
    float* x = (float*)malloc(sizeof(float) * (size_t)T);
    float* r = (float*)malloc(sizeof(float) * (size_t)T);
    uint8_t* codes = (uint8_t*)malloc((size_t)T);
    int8_t* rq = (int8_t*)malloc((size_t)T);
    int written = 0;
    for (int j = 0; j < L_cap / T; ++j) {
        const int last = (j + 1) * T - 1;
        if (last < tok_begin || last >= tok_end) continue;
        for (int t = 0; t < T; ++t) memset(Kc + (size_t)(j * T + t) * row_bytes, 0, (size_t)row_bytes);
        for (int c = 0; c < d; ++c) {
            for (int t = 0; t < T; ++t) x[t] = load_elem(K, dtype, (size_t)(j * T + t) * d + c);
            float s32;
            ffdo_quantize_channel(x, T, 1, bits, codes, &s32);
            const uint16_t s16 = round_to_bf16(s32);
            const float s = bf16_value(s16);
            for (int t = 0; t < T; ++t) {
                const float xh = ((float)codes[t] - half) * s;
                r[t] = x[t] - xh;
            }
            float s_r;
            ffdo_quantize_residual(r, T, rq, &s_r);
            sc[(size_t)j * d + c] = s16;
            sr[(size_t)j * d + c] = s_r;
            for (int t = 0; t < T; ++t) {
                uint8_t* row = Kc + (size_t)(j * T + t) * row_bytes;
                row[c / per] |= (uint8_t)(codes[t] << ((c % per) * bits));
                Kr[(size_t)(j * T + t) * d + c] = rq[t];
            }
        }
        ++written;
    }
    free(x);
    free(r);
    free(codes);
    free(rq);
    return written;
}

/* Alg. 1 Dequant of key element (t, c) of a slice, in double. */
double ffdo_dequant(const uint8_t* Kc, const uint16_t* sc, const int8_t* Kr, const float* sr,
                    int d, int T, int bits, int t, int c)
{
    const int row_bytes = d * bits / 8;
    const int u = code_at(Kc + (size_t)t * row_bytes, c, bits);
    const double half = (double)((1 << bits) - 1) * 0.5;
    const size_t sidx = (size_t)(t / T) * d + c;
    return ((double)u - half) * (double)bf16_value(sc[sidx]) +
           (double)Kr[(size_t)t * d + c] * (double)sr[sidx];
}

/*
 * Integer-exact scan of one query head over the thumbnail codes (bits = 2 or 4); the same
 * arithmetic as ffdo_scan_head with E_t = sum_c wi_c * (2 u_tc - (2^bits - 1)).
 */
void ffdo_scan_head_bits(const float* qh, const uint8_t* Kc, const uint16_t* scales,
                         int n_full, int T, int d, int bits, float* shat_block, float* shat_tok,
                         int32_t* E_tok)
{
    const int row_bytes = d * bits / 8;
    const int top = (1 << bits) - 1;
    int32_t* wi = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
    float* sf = (float*)malloc(sizeof(float) * (size_t)d);
    for (int j = 0; j < n_full; ++j) {
        block_scales(scales, j, d, sf);
        const float f = ffdo_requant(qh, sf, d, wi);
        float best = -INFINITY;
        for (int t = 0; t < T; ++t) {
            const uint8_t* row = Kc + (size_t)(j * T + t) * row_bytes;
            int64_t E = 0;
            for (int c = 0; c < d; ++c)
                E += (int64_t)wi[c] * (int64_t)(2 * code_at(row, c, bits) - top);
            const float sh = (float)E * f;
            if (shat_tok) shat_tok[(size_t)j * T + t] = sh;
            if (E_tok) E_tok[(size_t)j * T + t] = (int32_t)E;
            if (sh > best) best = sh;
        }
        shat_block[j] = best;
    }
    free(wi);
    free(sf);
}

/*
 * Exact attention of one head over the kept blocks with Dequant keys (full blocks) and the
 * 16-bit tail keys Ktail [L_cap][d] (bf16 bits; rows n_full*T .. L-1 are read, may be NULL when
 * L % T == 0).  V [L_cap][d] in `dtype`.  keep = NULL for all blocks.
 */
void ffdo_attend_head_res(const float* qh, const uint8_t* Kc, const uint16_t* sc, const int8_t* Kr,
                          const float* sr, const void* Ktail, const void* V, int dtype, int L,
                          int d, int T, int bits, const uint8_t* keep, double* out, double* lse)
{
    const int n_full = L / T;
    double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
        if (keep && !keep[t / T]) { s[t] = -INFINITY; continue; }
        double acc = 0.0;
        for (int c = 0; c < d; ++c) {
            const double k = t < n_full * T
                                 ? ffdo_dequant(Kc, sc, Kr, sr, d, T, bits, t, c)
                                 : (double)load_elem(Ktail, FFDO_DTYPE_BF16, (size_t)t * d + c);
            acc += (double)qh[c] * k;
        }
        s[t] = acc * inv_sqrt_d;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int t = 0; t < L; ++t) {
        if (s[t] == -INFINITY) continue;
        const double p = exp(s[t] - m);
        l += p;
        for (int c = 0; c < d; ++c) out[c] += p * (double)load_elem(V, dtype, (size_t)t * d + c);
    }
    for (int c = 0; c < d; ++c) out[c] /= l;
    *lse = m + log(l);
    free(s);
}

/*
 * Whole decode step in the residual storage form (q, Ktail, V bf16 bits; thumbnail + residual of
 * the full blocks), OpenMP over (batch, query head).  sparse = 0 attends over every token with
 * the same Dequant keys.  Outputs as ffdo_decode.
 */
int ffdo_decode_res(int B, int Hq, int Hkv, int d, int L, int L_cap, int T, int bits,
                    const void* q, const void* Ktail, const void* V, const uint8_t* Kc,
                    const uint16_t* sc, const int8_t* Kr, const float* sr, float delta, int sparse,
                    double* out, double* lse, uint8_t* keep, float* shat, float* mtilde,
                    int n_threads)
{
    if (Hkv <= 0 || Hq % Hkv || (bits != 2 && bits != 4) || d % (8 / bits) || T <= 0 || L < 0 ||
        L > L_cap || L_cap % T)
        return -1;
    if (L % T && !Ktail) return -1;
    const int G = Hq / Hkv;
    const int n_full = L / T;
    const int n_blocks = (L + T - 1) / T;
    const int row_bytes = d * bits / 8;
    const int rows = B * Hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int r = 0; r < rows; ++r) {
        const int b = r / Hq, h = r % Hq, g = h / G;
        const size_t bg = (size_t)b * Hkv + g;
        float* qh = (float*)malloc(sizeof(float) * (size_t)d);
        for (int c = 0; c < d; ++c) qh[c] = load_elem(q, FFDO_DTYPE_BF16, (size_t)r * d + c);
        const uint8_t* Kc_bg = Kc + bg * (size_t)L_cap * row_bytes;
        const uint16_t* sc_bg = sc + bg * (size_t)(L_cap / T) * d;
        const int8_t* Kr_bg = Kr + bg * (size_t)L_cap * d;
        const float* sr_bg = sr + bg * (size_t)(L_cap / T) * d;
        const char* Kt_bg = Ktail ? (const char*)Ktail + bg * (size_t)L_cap * d * 2 : NULL;
        const char* V_bg = (const char*)V + bg * (size_t)L_cap * d * 2;
        uint8_t* kp = NULL;
        if (sparse) {
            float* sb = (float*)malloc(sizeof(float) * (size_t)(n_full > 0 ? n_full : 1));
            kp = (uint8_t*)malloc((size_t)(n_blocks > 0 ? n_blocks : 1));
            ffdo_scan_head_bits(qh, Kc_bg, sc_bg, n_full, T, d, bits, sb, NULL, NULL);
            float mt;
            ffdo_select_head(sb, n_full, n_blocks, delta, kp, &mt, NULL);
            if (keep) memcpy(keep + (size_t)r * n_blocks, kp, (size_t)n_blocks);
            if (shat) memcpy(shat + (size_t)r * n_full, sb, sizeof(float) * (size_t)n_full);
            if (mtilde) mtilde[r] = mt;
            free(sb);
        }
        ffdo_attend_head_res(qh, Kc_bg, sc_bg, Kr_bg, sr_bg, Kt_bg, V_bg, FFDO_DTYPE_BF16, L, d,
                             T, bits, kp, out + (size_t)r * d, lse + r);
        free(kp);
        free(qh);
    }
    return rows;
}
