// ffd_internal.h -- launch parameters shared by the C-ABI layer and the gfx950 kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>

namespace ffd {

constexpr int kHeadDim = 128;
constexpr int kWaves = 4;                  // waves per work-group of the decode kernels
constexpr int kMaxBlocksPerSplit = 256;    // LDS sizing of the per-split block tables
constexpr int kMaxSplits = 256;            // LDS sizing of the final split merge
constexpr int kMaxUnitHeads = 8;           // query heads per work unit (the kernels' widest group)
constexpr size_t kScratchBytes = (size_t)16 << 20;  // the fixed scratch area of the no-allocation
                                                    // entry point, per device

// Query heads per work unit for a group of G query heads per kv head: the narrowest kernel width
// (1, 2, 4 or 8) that holds the group, or 8 for larger groups, which are cut into units of 8
// heads (each unit reads the kv head's keys and values on its own).
inline int unit_heads(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : kMaxUnitHeads; }
inline int units_per_kv(int G) { return (G + kMaxUnitHeads - 1) / kMaxUnitHeads; }

struct DecodeParams {
    const void* q;
    const void* K;
    const void* V;
    const uint8_t* Kq;      // scanned codes (4 bits; 2 or 4 bits in the residual form)
    const uint16_t* scales;  // their block scales, bf16 bits [B*Hkv][cap/T][d]
    const int8_t* Kr;       // residual form: 8-bit residual codes [B*Hkv][cap][d]
    const float* res_scales;  // residual form: residual scales [B*Hkv][cap/T][d]
    float* out;
    float* lse;
    uint8_t* keep_mask;
    unsigned long long* counters;  // [units] finished splits (high half) and, for S <= 32, a
                                   // mask of the splits with a partial (low half); zero between
                                   // calls
    float2* part_ml;     // [units][S][GP] per-split (max in log2 units, sum of exp2)
    float* part_o;       // [units][S][GP][d] per-split unnormalized output
    int B, Hq, Hkv, G;   // G = Hq / Hkv query heads per kv head (any value)
    int GP, NSUB;        // query heads per work unit (the kernel's width: 1, 2, 4 or 8; the
                         // unit's last heads are padding when G is not a multiple) and units per
                         // kv head; units = B * Hkv * NSUB, counters and partials are per unit
    int L, cap, T;
    int n_full, n_blocks;
    int S, R;       // splits per (b, kv head), blocks per split
    float delta;    // top-delta threshold (logit units)
    float kappa;    // (float)(0.5 / (127 sqrt(d)))
    float c_log2;   // (float)(log2(e) / sqrt(d))
    const int32_t* seq_lens;  // optional [B] per-sequence lengths in device memory, each clamped
                              // to [0, L]; L, n_full and n_blocks are then the bounds the splits
                              // cover and each work-group derives its sequence's own
    int mask_stride;          // keep_mask row length in blocks
    const uint8_t* ext_mask;  // optional [B][Hq][mask_stride] selection made by the caller: the
                              // sparse kernel then attends over these blocks and scans nothing
    int running;              // sparse: top-delta against the running maximum of each split (the
                              // splits are then the caller's windows of R blocks)
    int stream;               // the launch uses the kernels whose streamed reads (the scan's codes
                              // and scales, the exact stage's values, the dense step's keys) take
                              // the streaming (non-temporal) cache policy: set for long splits
    // Fused decode-loop step (sparse, stored keys, with seq_lens): when k_new is set, the step's
    // own token k_new/v_new [B][Hkv][d] (q's dtype) goes to position seq_lens[b] of K and V (if
    // that is below L) and is attended to; the key block it completes is quantized into Kq and
    // scales (K, V, Kq and scales are then written: the caller's buffers are mutable); and once
    // every unit of sequence b has read its length, seq_lens_out[b] (= seq_lens) is advanced.
    // The per-sequence count lives in counter slot kCounterSlots - 1 - b.
    const void* k_new;
    const void* v_new;
    int32_t* seq_lens_out;
};

// Counter slots of a workspace (its fixed first region): one per work unit of any call, the fused
// decode-loop step also using the top B slots for its per-sequence counts.
constexpr int kCounterSlots = 65535;

// Splits of at least this many blocks run the streaming-policy kernels.  Measured (alternating
// builds, graph replay): sparse 128K x 8 (256 blocks per split) 214 -> 193 us, 256K (64 blocks)
// 33.4 -> 31.3 us, 128K (32 blocks) 22.3 -> 20.8 us; slower on shorter splits, whose steps are
// bound by latency (32K, 8 blocks: +0.2 us; 4K: +0.6 us).  The dense step gains from 4 blocks per
// split (32K: 31.5 -> 28.6 us; 256K: 183 -> 155 us) and not on 2 (a 4K-token fp32 head).
constexpr int kStreamBlocks = 32;
constexpr int kStreamBlocksDense = 4;

struct QuantParams {
    const void* K;
    uint8_t* Kq;
    uint16_t* scales;   // bf16 bits
    int8_t* Kr;         // residual form only
    float* res_scales;  // residual form only
    int B, Hkv, cap, T;
    int j_first, n_blocks;  // blocks j_first .. j_first + n_blocks - 1
};

// One decode-loop step of the cache: the new token's key and value rows go to position
// seq_lens[b] of every (b, kv head), and the key block they complete (if any) is quantized.
struct AppendParams {
    const void* k_new;  // [B][Hkv][d]
    const void* v_new;  // [B][Hkv][d]
    void* K;            // [B][Hkv][cap][d]
    void* V;
    int32_t* seq_lens;  // [B], device
    uint8_t* Kq;
    uint16_t* scales;   // bf16 bits
    int B, Hkv, cap, T;
};

// Per-block metadata of the selection comparators: min and max of every channel of a key block.
struct BoundsParams {
    const void* K;
    void* kmin;  // [B][Hkv][cap/T][d], in K's dtype
    void* kmax;
    int B, Hkv, cap, T;
    int j_first, n_blocks;
};

// Block scores for the selection comparators: kind 0 = the scan estimate (Alg. 1), 1 = the
// min/max upper bound, 2 = the exact largest score of the block.
struct ScoreParams {
    const void* q;
    const void* K;
    const uint8_t* Kq;
    const uint16_t* scales;  // bf16 bits
    const void* kmin;
    const void* kmax;
    float* scores;  // [B][Hq][n_full]
    int B, Hq, Hkv, G, cap, T, n_full;
    int GP, NSUB;      // as DecodeParams
    float kappa;       // as DecodeParams
    float inv_sqrt_d;  // (float)(1 / sqrt(d))
};

// One selection rule over per-block scores, one work-group per (b, query head) row.
struct SelectParams {
    const float* scores;      // [rows][n_full]
    const float* pseudo_max;  // optional [rows] (top-delta)
    uint8_t* keep;            // [rows][n_blocks]
    int rows, n_full, n_blocks, n_pow2;
    float param;              // delta, k or p
};

// Launchers (ffd_kernels.hip).  Return the hipError_t of the launch.
hipError_t launch_bounds(const BoundsParams& p, bool bf16, hipStream_t stream);
hipError_t launch_scores(const ScoreParams& p, int kind, bool bf16, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, int rule, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, bool bf16, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, bool bf16, bool sparse, hipStream_t stream);
hipError_t launch_quantize(const QuantParams& p, bool bf16, hipStream_t stream);
hipError_t launch_decode_res(const DecodeParams& p, int bits, hipStream_t stream);
hipError_t launch_quantize_res(const QuantParams& p, int bits, hipStream_t stream);
hipError_t launch_zero_counters(uint32_t* counters, int n, hipStream_t stream);
// the streaming-policy decode kernels (bf16 inputs, p.stream set), in their own translation unit
hipError_t launch_decode_stream(const DecodeParams& p, bool sparse, hipStream_t stream);
hipError_t launch_decode_res_stream(const DecodeParams& p, int bits, hipStream_t stream);

// The current device's fixed scratch area (kScratchBytes, 256-byte aligned; ffd_scratch.hip):
// its device address, looked up at the first call on the device, when its first counter_bytes
// bytes are also zeroed on `stream`.  No allocation.
hipError_t scratch_area(size_t counter_bytes, hipStream_t stream, void** ptr);

}  // namespace ffd
