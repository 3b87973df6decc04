// ffd_api.cpp -- C ABI of libffd (declared in include/ffd.h): argument validation, the split
// heuristic, workspace layout and kernel launches.  Validation happens before any HIP call.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/ffd.h"
#include "ffd_internal.h"

namespace {

using ffd::kHeadDim;
using ffd::kMaxBlocksPerSplit;
using ffd::kMaxSplits;
using ffd::kWaves;

// the ranked selection rules sort a row of block scores in LDS (8-byte keys)
constexpr int kMaxRankedBlocks = 16384;
// work units per call: a grid dimension of the score kernel, and the workspace's counter slots
constexpr int64_t kMaxUnits = ffd::kCounterSlots;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Work units: the G = Hq / Hkv query heads of a kv head are handled G_unit at a time, G_unit
// being the narrowest kernel width (1, 2, 4, 8) that holds them, or 8 with several units per kv
// head for groups of more than 8 (each unit then reads the kv head's keys and values itself).
int group_of(const ffd_dims* d) { return d->n_q_heads / d->n_kv_heads; }
int64_t n_units(const ffd_dims* d)
{
    return (int64_t)d->batch * d->n_kv_heads * ffd::units_per_kv(group_of(d));
}

// Shape checks shared by every call.  `block` must be known (64/128) for the decode calls.
ffd_status check_dims(const ffd_dims* d, int32_t block)
{
    if (!d) return FFD_ERR_INVALID_ARG;
    if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
        d->seq_len < 1 || d->seq_cap < d->seq_len || block < 1)
        return FFD_ERR_INVALID_ARG;
    if (d->n_q_heads % d->n_kv_heads) return FFD_ERR_INVALID_ARG;
    if (d->dtype != FFD_F32 && d->dtype != FFD_BF16) return FFD_ERR_INVALID_ARG;
    if (d->head_dim != kHeadDim) return FFD_ERR_UNSUPPORTED;
    if (block != 64 && block != 128) return FFD_ERR_UNSUPPORTED;
    if (d->seq_cap % block) return FFD_ERR_INVALID_ARG;
    // grid and table limits: at most 65535 work units (a grid dimension of the score kernel),
    // at most kMaxSplits splits of at most kMaxBlocksPerSplit blocks
    if (n_units(d) > kMaxUnits) return FFD_ERR_UNSUPPORTED;
    const int64_t n_blocks = ((int64_t)d->seq_len + block - 1) / block;
    if (n_blocks > (int64_t)kMaxSplits * kMaxBlocksPerSplit) return FFD_ERR_UNSUPPORTED;
    return FFD_OK;
}

int splits_for(const ffd_dims* d, int32_t block, bool sparse)
{
    const int n_blocks = (d->seq_len + block - 1) / block;
    const int64_t bh = n_units(d);
    const int min_s = (n_blocks + kMaxBlocksPerSplit - 1) / kMaxBlocksPerSplit;
    int64_t s;
    const char* env = getenv("FFD_NUM_SPLITS");
    if (env && atoi(env) >= 1) {
        s = atoi(env);
        if (s > n_blocks) s = n_blocks;
    } else {
        // one work-group per CU: fewer, longer streams measured faster than more resident
        // work-groups at every occupancy tried.  A split keeps at least two blocks per wave,
        // except that a short sequence may go down to two blocks per split (at most 32 splits):
        // such a step is latency-bound, and more work-groups finish it sooner (a 4K-token,
        // one-head step: 22 us at 8 splits, 14 us at 32)
        const int64_t target_wgs = 256;
        s = bh > 0 ? (target_wgs + bh - 1) / bh : 1;
        const int64_t few = n_blocks / 2 < 32 ? n_blocks / 2 : 32;
        int64_t max_s = n_blocks / (2 * kWaves);
        if (max_s < few) max_s = few;
        if (max_s < 1) max_s = 1;
        if (s > max_s) s = max_s;
        // sparse: a split shorter than one block per wave leaves waves without scan work; one
        // block per wave is faster while the work-groups still fill half of the CUs (4K tokens
        // in blocks of 64, 8 kv heads: 9.3-9.5 against 10.0 us at 16 splits instead of 32)
        if (sparse) {
            const int64_t s_wave = n_blocks / kWaves;
            if (s > s_wave && s_wave >= 1 && bh * s_wave >= target_wgs / 2) s = s_wave;
        }
        // dense: splits of at most 8192 tokens.  Its work per split is uniform, and the
        // dispatcher balances the extra work-groups (128K x 8: 697 against 710 us at 16 splits
        // instead of 8; 64K x 16: 708 against 717 us at 8 instead of 4); the sparse step, whose
        // splits carry a per-split pseudo-max, ramp and partial, measured slower with them
        if (!sparse) {
            const int64_t s_tok = d->seq_len / 8192;
            if (s < s_tok) s = s_tok;
        }
    }
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < min_s) s = min_s;
    if (s < 1) s = 1;
    return (int)s;
}

// Workspace layout: counters [kMaxUnits] u64 | ml [units*S*G_unit] float2 |
// o [units*S*G_unit*d] fp32, each region starting on a 256-byte boundary.  The counter region has
// a fixed size (one slot for every unit any call may have), so that a workspace prepared once
// serves every later call whatever its dims: each call returns the slots it used to zero.
struct WsLayout {
    size_t off_ml, off_o, total;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr size_t kCounterBytes = ((size_t)kMaxUnits * sizeof(unsigned long long) + 255) & ~(size_t)255;
static_assert(FFD_NOALLOC_SCRATCH_BYTES == ffd::kScratchBytes, "header and library disagree");

WsLayout ws_layout(const ffd_dims* d, int S)
{
    const size_t bh = (size_t)n_units(d);
    const size_t rec = bh * (size_t)S * (size_t)ffd::unit_heads(group_of(d));
    WsLayout w;
    w.off_ml = kCounterBytes;
    w.off_o = w.off_ml + round256(rec * 2 * sizeof(float));
    w.total = w.off_o + rec * kHeadDim * sizeof(float);
    return w;
}

ffd_status finish(hipError_t e) { return e == hipSuccess ? FFD_OK : FFD_ERR_HIP; }

ffd_status decode_common(const ffd_dims* dims, const void* q, const void* K, const void* V,
                         const uint8_t* Kq, const uint16_t* scales, float delta, int32_t block,
                         float* out, float* lse, uint8_t* keep_mask, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, bool sparse,
                         const int8_t* Kr = nullptr, const float* res_scales = nullptr,
                         int bits = 0, const int32_t* seq_lens = nullptr,
                         const uint8_t* ext_mask = nullptr, int window = 0,
                         bool noalloc = false, const void* k_new = nullptr,
                         const void* v_new = nullptr, int32_t* seq_lens_out = nullptr)
{
    const bool res = bits != 0;
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (res && (dims->dtype != FFD_BF16 || (bits != 2 && bits != 4))) return FFD_ERR_UNSUPPORTED;
    if (dims->batch == 0) return FFD_OK;
    // the residual form reads 16-bit keys only for a partial tail block
    const bool need_K = !res || dims->seq_len % block != 0;
    if (!q || (need_K && !K) || !V || !out) return FFD_ERR_INVALID_ARG;
    if (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u)) return FFD_ERR_INVALID_ARG;
    if (!aligned16(q) || (K && !aligned16(K)) || !aligned16(V) || !aligned16(out) ||
        (lse && !aligned16(lse)) || (keep_mask && !aligned16(keep_mask)))
        return FFD_ERR_INVALID_ARG;
    if (sparse && !ext_mask) {
        if (!Kq || !scales || !aligned16(Kq) || !aligned16(scales)) return FFD_ERR_INVALID_ARG;
        if (isnan(delta) || delta < 0.0f) return FFD_ERR_INVALID_ARG;
    }
    if (res && (!Kr || !res_scales || !aligned16(Kr) || !aligned16(res_scales)))
        return FFD_ERR_INVALID_ARG;
    // the running-max variant splits the sequence into the caller's windows
    const int n_blk = (dims->seq_len + block - 1) / block;
    if (window != 0 && (window < 1 || window > kMaxBlocksPerSplit ||
                        (n_blk + window - 1) / window > kMaxSplits))
        return FFD_ERR_UNSUPPORTED;
    const int S = window != 0 ? (n_blk + window - 1) / window : splits_for(dims, block, sparse);
    const WsLayout lay = ws_layout(dims, S);
    if (noalloc) {
        // the library's fixed scratch area in place of a caller's workspace: sizes beyond it are
        // rejected before any HIP call; its address is looked up (and its counters zeroed) at
        // the first call on the device
        if (lay.total > ffd::kScratchBytes) return FFD_ERR_WORKSPACE;
        if (ffd::scratch_area(kCounterBytes, stream, &workspace) != hipSuccess) return FFD_ERR_HIP;
        workspace_bytes = ffd::kScratchBytes;
    }
    if (!workspace || !aligned16(workspace)) return FFD_ERR_WORKSPACE;
    if (workspace_bytes < lay.total) return FFD_ERR_WORKSPACE;

    ffd::DecodeParams p{};
    p.q = q;
    p.K = K;
    p.V = V;
    p.Kq = Kq;
    p.scales = scales;
    p.Kr = Kr;
    p.res_scales = res_scales;
    p.out = out;
    p.lse = lse;
    p.keep_mask = keep_mask;
    char* wsb = static_cast<char*>(workspace);
    p.counters = reinterpret_cast<unsigned long long*>(wsb);
    p.part_ml = reinterpret_cast<float2*>(wsb + lay.off_ml);
    p.part_o = reinterpret_cast<float*>(wsb + lay.off_o);
    p.B = dims->batch;
    p.Hq = dims->n_q_heads;
    p.Hkv = dims->n_kv_heads;
    p.G = group_of(dims);
    p.GP = ffd::unit_heads(p.G);
    p.NSUB = ffd::units_per_kv(p.G);
    p.L = dims->seq_len;
    p.cap = dims->seq_cap;
    p.T = block;
    p.n_full = dims->seq_len / block;
    p.n_blocks = (dims->seq_len + block - 1) / block;
    p.S = S;
    p.R = window != 0 ? window : (p.n_blocks + S - 1) / S;
    p.stream = p.R >= (sparse ? ffd::kStreamBlocks : ffd::kStreamBlocksDense) ? 1 : 0;
    p.running = window != 0 ? 1 : 0;
    p.seq_lens = seq_lens;
    p.k_new = k_new;
    p.v_new = v_new;
    p.seq_lens_out = seq_lens_out;
    p.mask_stride = p.n_blocks;
    p.ext_mask = ext_mask;
    p.delta = delta;
    p.kappa = (float)(0.5 / (127.0 * sqrt((double)kHeadDim)));
    p.c_log2 = (float)(1.4426950408889634 / sqrt((double)kHeadDim));
    if (res) return finish(ffd::launch_decode_res(p, bits, stream));
    return finish(ffd::launch_decode(p, dims->dtype == FFD_BF16, sparse, stream));
}

// Blocks j with tok_begin <= (j+1)*block - 1 < tok_end, as [j_first, j_last]; validation shared
// by both append calls.
ffd_status append_range(const ffd_dims* dims, int32_t tok_begin, int32_t tok_end, int32_t block,
                        int* j_first, int* j_last)
{
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (tok_begin < 0 || tok_end < tok_begin || tok_end > dims->seq_len) return FFD_ERR_INVALID_ARG;
    *j_first = (tok_begin + 1 + block - 1) / block - 1;
    *j_last = tok_end / block - 1;
    return FFD_OK;
}

}  // namespace

extern "C" {

int32_t ffd_abi_version(void) { return FFD_ABI_VERSION; }

const char* ffd_status_string(ffd_status s)
{
    switch (s) {
    case FFD_OK: return "ok";
    case FFD_ERR_INVALID_ARG: return "invalid argument";
    case FFD_ERR_UNSUPPORTED: return "unsupported configuration";
    case FFD_ERR_WORKSPACE: return "workspace missing or too small";
    case FFD_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t ffd_workspace_bytes(const ffd_dims* dims, int32_t block)
{
    if (check_dims(dims, block) != FFD_OK) return 0;
    const int s_sparse = splits_for(dims, block, true), s_dense = splits_for(dims, block, false);
    return ws_layout(dims, s_sparse > s_dense ? s_sparse : s_dense).total;
}

ffd_status ffd_workspace_init(const ffd_dims* dims, int32_t block, void* workspace,
                              size_t workspace_bytes, hipStream_t stream)
{
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (dims->batch == 0) return FFD_OK;
    if (!workspace || !aligned16(workspace)) return FFD_ERR_WORKSPACE;
    // only the counters are prepared, all of their fixed region: any workspace holding it
    // qualifies (a decode call checks its own size requirement, which depends on its dims)
    if (workspace_bytes < kCounterBytes) return FFD_ERR_WORKSPACE;
    return finish(ffd::launch_zero_counters(static_cast<uint32_t*>(workspace),
                                            (int)(kCounterBytes / sizeof(uint32_t)), stream));
}

int32_t ffd_num_splits(const ffd_dims* dims, int32_t block, int32_t sparse)
{
    if (check_dims(dims, block) != FFD_OK) return 0;
    return splits_for(dims, block, sparse != 0);
}

ffd_status ffd_quantize_k_append(const ffd_dims* dims, const void* K, int32_t tok_begin,
                                 int32_t tok_end, int32_t block, uint8_t* Kq, uint16_t* scales,
                                 hipStream_t stream)
{
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (tok_begin < 0 || tok_end < tok_begin || tok_end > dims->seq_len) return FFD_ERR_INVALID_ARG;
    if (dims->batch == 0) return FFD_OK;
    if (!K || !Kq || !scales || !aligned16(K) || !aligned16(Kq) || !aligned16(scales))
        return FFD_ERR_INVALID_ARG;
    // blocks j with tok_begin <= (j+1)*block - 1 < tok_end
    const int j_first = (tok_begin + 1 + block - 1) / block - 1;
    const int j_last = tok_end / block - 1;
    if (j_last < j_first) return FFD_OK;
    ffd::QuantParams p{};
    p.K = K;
    p.Kq = Kq;
    p.scales = scales;
    p.B = dims->batch;
    p.Hkv = dims->n_kv_heads;
    p.cap = dims->seq_cap;
    p.T = block;
    p.j_first = j_first;
    p.n_blocks = j_last - j_first + 1;
    return finish(ffd::launch_quantize(p, dims->dtype == FFD_BF16, stream));
}

ffd_status ffd_decode_sparse(const ffd_dims* dims, const void* q, const void* K, const void* V,
                             const uint8_t* Kq, const uint16_t* scales, float delta, int32_t block,
                             float* out, float* lse, uint8_t* keep_mask, void* workspace,
                             size_t workspace_bytes, hipStream_t stream)
{
    return decode_common(dims, q, K, V, Kq, scales, delta, block, out, lse, keep_mask, workspace,
                         workspace_bytes, stream, true);
}

ffd_status ffd_decode_sparse_noalloc(const ffd_dims* dims, const void* q, const void* K,
                                     const void* V, const uint8_t* Kq, const uint16_t* scales,
                                     float delta, int32_t block, float* out, float* lse,
                                     uint8_t* keep_mask, hipStream_t stream)
{
    return decode_common(dims, q, K, V, Kq, scales, delta, block, out, lse, keep_mask, nullptr, 0,
                         stream, true, nullptr, nullptr, 0, nullptr, nullptr, 0, true);
}

ffd_status ffd_quantize_k_residual_append(const ffd_dims* dims, const void* K, int32_t tok_begin,
                                          int32_t tok_end, int32_t block, int32_t bits,
                                          uint8_t* Kc, uint16_t* scales, int8_t* Kr,
                                          float* res_scales, hipStream_t stream)
{
    int j_first, j_last;
    ffd_status st = append_range(dims, tok_begin, tok_end, block, &j_first, &j_last);
    if (st != FFD_OK) return st;
    if (dims->dtype != FFD_BF16 || (bits != 2 && bits != 4)) return FFD_ERR_UNSUPPORTED;
    if (dims->batch == 0) return FFD_OK;
    if (!K || !Kc || !scales || !Kr || !res_scales || !aligned16(K) || !aligned16(Kc) ||
        !aligned16(scales) || !aligned16(Kr) || !aligned16(res_scales))
        return FFD_ERR_INVALID_ARG;
    if (j_last < j_first) return FFD_OK;
    ffd::QuantParams p{};
    p.K = K;
    p.Kq = Kc;
    p.scales = scales;
    p.Kr = Kr;
    p.res_scales = res_scales;
    p.B = dims->batch;
    p.Hkv = dims->n_kv_heads;
    p.cap = dims->seq_cap;
    p.T = block;
    p.j_first = j_first;
    p.n_blocks = j_last - j_first + 1;
    return finish(ffd::launch_quantize_res(p, bits, stream));
}

ffd_status ffd_decode_sparse_residual(const ffd_dims* dims, const void* q, const void* K_tail,
                                      const void* V, const uint8_t* Kc, const uint16_t* scales,
                                      const int8_t* Kr, const float* res_scales, int32_t bits,
                                      float delta, int32_t block, float* out, float* lse,
                                      uint8_t* keep_mask, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream)
{
    if (bits == 0) return FFD_ERR_UNSUPPORTED;
    return decode_common(dims, q, K_tail, V, Kc, scales, delta, block, out, lse, keep_mask,
                         workspace, workspace_bytes, stream, true, Kr, res_scales, bits);
}

ffd_status ffd_decode_dense(const ffd_dims* dims, const void* q, const void* K, const void* V,
                            int32_t block, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream)
{
    return decode_common(dims, q, K, V, nullptr, nullptr, 0.0f, block, out, lse, nullptr,
                         workspace, workspace_bytes, stream, false);
}

ffd_status ffd_decode_sparse_varlen(const ffd_dims* dims, const void* q, const void* K,
                                    const void* V, const uint8_t* Kq, const uint16_t* scales,
                                    const int32_t* seq_lens, float delta, int32_t block,
                                    float* out, float* lse, uint8_t* keep_mask, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream)
{
    if (!seq_lens) return FFD_ERR_INVALID_ARG;
    return decode_common(dims, q, K, V, Kq, scales, delta, block, out, lse, keep_mask, workspace,
                         workspace_bytes, stream, true, nullptr, nullptr, 0, seq_lens);
}

ffd_status ffd_decode_sparse_append(const ffd_dims* dims, const void* q, const void* k_new,
                                   const void* v_new, void* K, void* V, uint8_t* Kq,
                                   uint16_t* scales, int32_t* seq_lens, float delta, int32_t block,
                                   float* out, float* lse, uint8_t* keep_mask, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    if (!seq_lens || !k_new || !v_new || !K) return FFD_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return FFD_ERR_INVALID_ARG;
    // the per-sequence counts take the top counter slots, above those of the work units
    if (dims && check_dims(dims, block) == FFD_OK && n_units(dims) + dims->batch > kMaxUnits)
        return FFD_ERR_UNSUPPORTED;
    return decode_common(dims, q, K, V, Kq, scales, delta, block, out, lse, keep_mask, workspace,
                         workspace_bytes, stream, true, nullptr, nullptr, 0, seq_lens, nullptr, 0,
                         false, k_new, v_new, seq_lens);
}

ffd_status ffd_decode_sparse_running(const ffd_dims* dims, const void* q, const void* K,
                                     const void* V, const uint8_t* Kq, const uint16_t* scales,
                                     float delta, int32_t block, int32_t window, float* out,
                                     float* lse, uint8_t* keep_mask, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream)
{
    if (window < 1) return FFD_ERR_UNSUPPORTED;
    return decode_common(dims, q, K, V, Kq, scales, delta, block, out, lse, keep_mask, workspace,
                         workspace_bytes, stream, true, nullptr, nullptr, 0, nullptr, nullptr,
                         window);
}

size_t ffd_workspace_bytes_window(const ffd_dims* dims, int32_t block, int32_t window)
{
    if (check_dims(dims, block) != FFD_OK || window < 1 || window > kMaxBlocksPerSplit) return 0;
    const int n_blk = (dims->seq_len + block - 1) / block;
    const int S = (n_blk + window - 1) / window;
    if (S > kMaxSplits) return 0;
    return ws_layout(dims, S).total;
}

ffd_status ffd_decode_dense_varlen(const ffd_dims* dims, const void* q, const void* K,
                                   const void* V, const int32_t* seq_lens, int32_t block,
                                   float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream)
{
    if (!seq_lens) return FFD_ERR_INVALID_ARG;
    return decode_common(dims, q, K, V, nullptr, nullptr, 0.0f, block, out, lse, nullptr,
                         workspace, workspace_bytes, stream, false, nullptr, nullptr, 0,
                         seq_lens);
}

ffd_status ffd_append_token(const ffd_dims* dims, const void* k_new, const void* v_new, void* K,
                            void* V, int32_t* seq_lens, int32_t block, uint8_t* Kq,
                            uint16_t* scales, hipStream_t stream)
{
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (dims->batch == 0) return FFD_OK;
    if (!k_new || !v_new || !K || !V || !seq_lens || !Kq || !scales) return FFD_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(K) || !aligned16(V) ||
        !aligned16(Kq) || !aligned16(scales) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return FFD_ERR_INVALID_ARG;
    ffd::AppendParams a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.K = K;
    a.V = V;
    a.seq_lens = seq_lens;
    a.Kq = Kq;
    a.scales = scales;
    a.B = dims->batch;
    a.Hkv = dims->n_kv_heads;
    a.cap = dims->seq_cap;
    a.T = block;
    return finish(ffd::launch_append(a, dims->dtype == FFD_BF16, stream));
}

ffd_status ffd_decode_masked(const ffd_dims* dims, const void* q, const void* K, const void* V,
                             const uint8_t* keep_mask, int32_t block, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!keep_mask) return FFD_ERR_INVALID_ARG;
    return decode_common(dims, q, K, V, nullptr, nullptr, 0.0f, block, out, lse, nullptr,
                         workspace, workspace_bytes, stream, true, nullptr, nullptr, 0, nullptr,
                         keep_mask);
}

ffd_status ffd_block_bounds(const ffd_dims* dims, const void* K, int32_t tok_begin,
                            int32_t tok_end, int32_t block, void* kmin, void* kmax,
                            hipStream_t stream)
{
    int j_first = 0, j_last = -1;
    ffd_status st = append_range(dims, tok_begin, tok_end, block, &j_first, &j_last);
    if (st != FFD_OK) return st;
    if (dims->batch == 0) return FFD_OK;
    if (!K || !kmin || !kmax || !aligned16(K) || !aligned16(kmin) || !aligned16(kmax))
        return FFD_ERR_INVALID_ARG;
    ffd::BoundsParams b{};
    b.K = K;
    b.kmin = kmin;
    b.kmax = kmax;
    b.B = dims->batch;
    b.Hkv = dims->n_kv_heads;
    b.cap = dims->seq_cap;
    b.T = block;
    b.j_first = j_first;
    b.n_blocks = j_last - j_first + 1;
    return finish(ffd::launch_bounds(b, dims->dtype == FFD_BF16, stream));
}

ffd_status ffd_block_scores(const ffd_dims* dims, int32_t kind, const void* q, const void* K,
                            const uint8_t* Kq, const uint16_t* scales, const void* kmin,
                            const void* kmax, int32_t block, float* scores, hipStream_t stream)
{
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (kind < FFD_SCORE_SCAN || kind > FFD_SCORE_EXACT) return FFD_ERR_INVALID_ARG;
    if (dims->batch == 0) return FFD_OK;
    if (!q || !scores || !aligned16(q) || !aligned16(scores)) return FFD_ERR_INVALID_ARG;
    if (kind == FFD_SCORE_SCAN && (!Kq || !scales || !aligned16(Kq) || !aligned16(scales)))
        return FFD_ERR_INVALID_ARG;
    if (kind == FFD_SCORE_BOUNDS && (!kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)))
        return FFD_ERR_INVALID_ARG;
    if (kind == FFD_SCORE_EXACT && (!K || !aligned16(K))) return FFD_ERR_INVALID_ARG;
    ffd::ScoreParams p{};
    p.q = q;
    p.K = K;
    p.Kq = Kq;
    p.scales = scales;
    p.kmin = kmin;
    p.kmax = kmax;
    p.scores = scores;
    p.B = dims->batch;
    p.Hq = dims->n_q_heads;
    p.Hkv = dims->n_kv_heads;
    p.G = group_of(dims);
    p.GP = ffd::unit_heads(p.G);
    p.NSUB = ffd::units_per_kv(p.G);
    p.cap = dims->seq_cap;
    p.T = block;
    p.n_full = dims->seq_len / block;
    p.kappa = (float)(0.5 / (127.0 * sqrt((double)kHeadDim)));
    p.inv_sqrt_d = (float)(1.0 / sqrt((double)kHeadDim));
    return finish(ffd::launch_scores(p, kind, dims->dtype == FFD_BF16, stream));
}

ffd_status ffd_select_blocks(const ffd_dims* dims, int32_t rule, const float* scores,
                             const float* pseudo_max, float param, int32_t block,
                             uint8_t* keep_mask, hipStream_t stream)
{
    ffd_status st = check_dims(dims, block);
    if (st != FFD_OK) return st;
    if (rule < FFD_SELECT_TOP_DELTA || rule > FFD_SELECT_TOP_P || isnan(param))
        return FFD_ERR_INVALID_ARG;
    if (rule == FFD_SELECT_TOP_DELTA && param < 0.0f) return FFD_ERR_INVALID_ARG;
    if (rule == FFD_SELECT_TOP_K && !(param >= 0.0f && param < 2147483648.0f))
        return FFD_ERR_INVALID_ARG;
    if (rule == FFD_SELECT_TOP_P && !(param > 0.0f && param <= 1.0f)) return FFD_ERR_INVALID_ARG;
    const int n_full = dims->seq_len / block;
    if (rule != FFD_SELECT_TOP_DELTA && n_full > kMaxRankedBlocks) return FFD_ERR_UNSUPPORTED;
    if (dims->batch == 0) return FFD_OK;
    if (!scores || !keep_mask || (pseudo_max && (reinterpret_cast<uintptr_t>(pseudo_max) & 3u)) ||
        (reinterpret_cast<uintptr_t>(scores) & 3u))
        return FFD_ERR_INVALID_ARG;
    ffd::SelectParams p{};
    p.scores = scores;
    p.pseudo_max = rule == FFD_SELECT_TOP_DELTA ? pseudo_max : nullptr;
    p.keep = keep_mask;
    p.rows = dims->batch * dims->n_q_heads;
    p.n_full = n_full;
    p.n_blocks = (dims->seq_len + block - 1) / block;
    int n2 = 1;
    while (n2 < n_full) n2 <<= 1;
    p.n_pow2 = n2;
    p.param = param;
    return finish(ffd::launch_select(p, rule, stream));
}

}  // extern "C"
