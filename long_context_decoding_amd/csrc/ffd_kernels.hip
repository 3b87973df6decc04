// ffd_kernels.hip -- gfx950 (CDNA4) kernels of libffd.
//
// Method: "Faster Than Flash: Exploiting Attention Sparsity for Efficient Long-Context Decoding"
// (arXiv 2609.00097), written FTF below.
//
//   quantize_kernel  App. A quantizer (16 levels) of each completed key block -> packed int4 codes
//                    and one fp32 scale per (block, channel).
//   quantize_res_kernel
//                    the residual storage form (Sec. 3.1, Fig. 2): App. A thumbnail at 2 or 4 bits
//                    plus a symmetric 8-bit code of the residual x - (u - half) s, both with one
//                    fp32 scale per (block, channel).
//   decode_kernel    one work-group per (sequence, kv head, split of the sequence):
//                      scan     int4 codes x int8-requantized (q . s) on the int8 MFMA (Alg. 1 scan)
//                      select   pseudo-max over the sink and local blocks (Eq. 3), keep a block
//                               iff its estimated max >= pseudo-max - delta (Eq. 1)
//                      exact    bf16/fp32 MFMA for the G x 16 score tile, online softmax with
//                               fp32 probabilities, PV on the bf16 MFMA with each probability
//                               as a bf16 high/low pair (fp32 values: on the VALU) (Alg. 1
//                               refinement)
//                      combine  one partial (o, m, l) per query head; the last work-group of the
//                               (sequence, kv head) merges the splits' partials with the
//                               log-sum-exp rule (split-KV decoding, FTF Sec. 2)
//                    The dense baseline is the same kernel with every block kept and no scan.
//                    In the residual storage form the scan reads the 2- or 4-bit thumbnail and the
//                    exact stage rebuilds each kept key (Alg. 1 Dequant) from thumbnail and
//                    residual, as a bf16 high/low pair, so that q.k_quant + q.k_res (Eq. 4) is
//                    accumulated on the bf16 MFMA.
//
// Wave layout conventions (wave64):
//   lane = 16 * kg + col, kg = lane >> 4 in 0..3, col = lane & 15.
//   16x16 MFMA outputs: lane holds rows 4*kg + v (v = 0..3) of column col.
//   The A and B operands of a 16x16 MFMA hold row/column `col` and the k-slice selected by kg;
//   any assignment of channels to k works as long as A and B use the same one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ffd_internal.h"

// This file is compiled twice: as itself (FFD_PART 0: every kernel but the streaming-policy decode
// kernels, and every launcher) and through ffd_kernels_stream.hip (FFD_PART 1: the streaming-policy
// decode kernels and their launchers), so that the two halves compile in parallel.
#ifndef FFD_PART
#define FFD_PART 0
#endif

namespace ffd {
namespace {

constexpr int D = kHeadDim;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kResWaves = 8;  // decode waves per work-group in the residual storage form

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Loads of data that is read once (the scan's codes and scales, the exact stage's values, the
// dense step's keys and values) can use the streaming (non-temporal) cache policy, which streams
// faster on this chip (decode_kernel's STREAM variants, launched for long splits:
// kStreamBlocks).  The kept keys of the sparse step stay on the default policy (measured slower
// with streaming loads).
template <bool B>
struct Flag {
    static constexpr bool value = B;
};
// 16-byte load (streaming cache policy when NT)
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p)
{
    if constexpr (NT) {
        typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
        const v4u_t x = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
        return make_uint4(x[0], x[1], x[2], x[3]);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}
template <bool NT>
__device__ __forceinline__ float4 ld16f(const void* p)
{
    const uint4 u = ld16<NT>(p);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
}
typedef unsigned int u32;

__device__ __forceinline__ float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ int as_i(float x) { return __builtin_bit_cast(int, x); }

template <int CTRL>
__device__ __forceinline__ int dpp(int x)
{
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}

// Reductions over the 16 lanes of a row (all lanes receive the result):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, as_f(dpp<0xB1>(as_i(x))));
    x = fmaxf(x, as_f(dpp<0x4E>(as_i(x))));
    x = fmaxf(x, as_f(dpp<0x141>(as_i(x))));
    x = fmaxf(x, as_f(dpp<0x140>(as_i(x))));
    return x;
}

__device__ __forceinline__ int row16_sum(int x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

// Exchanges across the 16-lane rows on the VALU (gfx950 permlane swaps, no LDS round trip).
// The two results of permlane16_swap(x, x) hold, in every lane l, the values of lanes l & ~16 and
// l | 16, so an operation on them forms op(x_l, x_{l^16}) with the same operand order in both
// lanes of a pair; permlane32_swap does the same for l ^ 32.
__device__ __forceinline__ void pair16(int x, int& a, int& b)
{
    const auto r = __builtin_amdgcn_permlane16_swap((u32)x, (u32)x, false, false);
    a = (int)r[0];
    b = (int)r[1];
}
__device__ __forceinline__ void pair32(int x, int& a, int& b)
{
    const auto r = __builtin_amdgcn_permlane32_swap((u32)x, (u32)x, false, false);
    a = (int)r[0];
    b = (int)r[1];
}
__device__ __forceinline__ float fmax16(float x)
{
    int a, b;
    pair16(as_i(x), a, b);
    return fmaxf(as_f(a), as_f(b));
}
__device__ __forceinline__ float fmax32(float x)
{
    int a, b;
    pair32(as_i(x), a, b);
    return fmaxf(as_f(a), as_f(b));
}
__device__ __forceinline__ float fsum16(float x)
{
    int a, b;
    pair16(as_i(x), a, b);
    return as_f(a) + as_f(b);
}
__device__ __forceinline__ float fsum32(float x)
{
    int a, b;
    pair32(as_i(x), a, b);
    return as_f(a) + as_f(b);
}
__device__ __forceinline__ int imax16(int x)
{
    int a, b;
    pair16(x, a, b);
    return max(a, b);
}
__device__ __forceinline__ int imax32(int x)
{
    int a, b;
    pair32(x, a, b);
    return max(a, b);
}

// Value of lane h of this lane's 16-lane row (DPP row_newbcast), h < 8 known after unrolling.
__device__ __forceinline__ float row_bcast(float x, int h)
{
    switch (h) {
    case 0: return as_f(dpp<0x150>(as_i(x)));
    case 1: return as_f(dpp<0x151>(as_i(x)));
    case 2: return as_f(dpp<0x152>(as_i(x)));
    case 3: return as_f(dpp<0x153>(as_i(x)));
    case 4: return as_f(dpp<0x154>(as_i(x)));
    case 5: return as_f(dpp<0x155>(as_i(x)));
    case 6: return as_f(dpp<0x156>(as_i(x)));
    default: return as_f(dpp<0x157>(as_i(x)));
    }
}

// Orders this wave's LDS accesses (LDS executes one wave's instructions in order; this only
// stops the compiler from moving accesses across the point).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool C, class A, class B>
struct pick {
    typedef A type;
};
template <class A, class B>
struct pick<false, A, B> {
    typedef B type;
};

__device__ __forceinline__ float bf16_lo(u32 x) { return as_f((int)(x << 16)); }
__device__ __forceinline__ float bf16_hi(u32 x) { return as_f((int)(x & 0xFFFF0000u)); }

// Block scales are kept as bf16: the binary32 value rounded to nearest, ties to even (adding
// 0x7FFF plus the lowest kept bit, then truncating, also carries correctly into the next binade
// and to infinity); a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t scale_bits(float x)
{
    const u32 u = (u32)as_i(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float scale_value(uint16_t b) { return as_f((int)((u32)b << 16)); }

// ------------------------------------------------------------------------------------------
// Per-wave LDS scratch
// ------------------------------------------------------------------------------------------
template <int G>
struct __attribute__((aligned(16))) WaveScratch {
    int8_t wB[2][G][4][16];  // scan MFMA B operand: [k-step][head][kg][16 int8]
    float f[G];              // per-head scan factor RN(W * kappa)
    int wsum[G];             // per-head sum of the requantized weights
    float4 rsc[96];          // residual form, four channels an entry: the current block's s
                             // (0-31), s_r (32-63), -half * s (64-95)
};

// ------------------------------------------------------------------------------------------
// Scan of one full block (FTF Alg. 1, scan stage; App. B Eq. 8 for what it approximates).
// ------------------------------------------------------------------------------------------
template <int BITS>
struct CodeSlice;  // the packed codes of 32 channels of one token row
template <>
struct CodeSlice<4> {
    typedef uint4 type;
};
template <>
struct CodeSlice<2> {
    typedef uint2 type;
};

template <int T, int BITS>
struct ScanRegs {
    typename CodeSlice<BITS>::type kq[T / 16];  // token row (16*i + col), channels 32*kg .. +31
    uint4 s;                                    // bf16 scales of channels 8*col .. 8*col+7
};

template <int T, int BITS, bool NT>
__device__ __forceinline__ void scan_load(ScanRegs<T, BITS>& r, const uint8_t* __restrict__ kq_blk,
                                          const uint16_t* __restrict__ sc_blk, int lane)
{
    const int col = lane & 15, kg = lane >> 4;
    constexpr int RB = D * BITS / 8, CB = 32 * BITS / 8;  // bytes per row, per 32 channels
#pragma unroll
    for (int i = 0; i < T / 16; ++i) {
        const uint8_t* a = kq_blk + (size_t)(i * 16 + col) * RB + kg * CB;
        if constexpr (BITS == 4) {
            r.kq[i] = ld16<NT>(a);
        } else if constexpr (NT) {
            typedef u32 v2u_t __attribute__((ext_vector_type(2)));
            const v2u_t x = __builtin_nontemporal_load(reinterpret_cast<const v2u_t*>(a));
            r.kq[i] = make_uint2(x[0], x[1]);
        } else {
            r.kq[i] = *reinterpret_cast<const uint2*>(a);
        }
    }
    r.s = ld16<NT>(sc_blk + col * 8);
}

// Estimated block maximum of every query head of the group.  Requantization lanes: row kg
// handles head kg (+4 for G = 8), 8 channels 8*col..8*col+7.  Result valid in lanes with
// col < G (head col), identical across kg.
//
// The A operand holds 16 channels c0..c0+15 per 16 bytes.  At 4 bits each packed dword
// (channels c..c+7, two per byte) unpacks into lo = d & 0x0F0F0F0F (channels c, c+2, c+4, c+6)
// and hi = (d >> 4) & 0x0F0F0F0F (c+1, c+3, c+5, c+7); at 2 bits a dword (channels c..c+15,
// four per byte) unpacks into (d >> 2m) & 0x03030303 (channels c+m, c+m+4, c+m+8, c+m+12),
// m = 0..3.  The B operand stores the requantized weights in the same channel order.
// Codes enter as u in 0..2^BITS-1 (positive int8), so D_t = sum_c wi_c u_tc and
// E_t = sum_c wi_c (2 u_tc - (2^BITS - 1)) = 2 D_t - (2^BITS - 1) sum_c wi_c, exact in int32.
template <int T, int G, int BITS>
__device__ __forceinline__ float scan_compute(const ScanRegs<T, BITS>& r,
                                              const float (&qw)[(G + 3) / 4][8], float kappa,
                                              WaveScratch<G>& ws, int lane)
{
    constexpr int HPL = (G + 3) / 4;
    const int col = lane & 15, kg = lane >> 4;
    const float s[8] = {bf16_lo(r.s.x), bf16_hi(r.s.x), bf16_lo(r.s.y), bf16_hi(r.s.y),
                        bf16_lo(r.s.z), bf16_hi(r.s.z), bf16_lo(r.s.w), bf16_hi(r.s.w)};
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
        const int h = kg + 4 * k;
        float w[8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = __fmul_rn(qw[k][i], s[i]);
            amax = fmaxf(amax, fabsf(w[i]));
        }
        const float W = row16_max(amax);
        int wi[8];
        if (W > 0.0f) {
            const float rho = __fdiv_rn(127.0f, W);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float v = rintf(__fmul_rn(w[i], rho));
                v = fminf(fmaxf(v, -127.0f), 127.0f);
                wi[i] = (int)v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) wi[i] = 0;
        }
        const int wsum =
            row16_sum(wi[0] + wi[1] + wi[2] + wi[3] + wi[4] + wi[5] + wi[6] + wi[7]);
        if (G >= 4 || h < G) {
            // channel 8*col + i: kg' = col / 4, k-step (col % 4) / 2, offset 8 * (col % 2) + i
            // within the k-step's 16 channels
            const int kgw = col >> 2, ks = (col & 3) >> 1;
            int8_t* dst = &ws.wB[ks][h][kgw][0];
            if constexpr (BITS == 4) {
                const u32 d0 = (u32)(wi[0] & 255) | ((u32)(wi[2] & 255) << 8) |
                               ((u32)(wi[4] & 255) << 16) | ((u32)(wi[6] & 255) << 24);
                const u32 d1 = (u32)(wi[1] & 255) | ((u32)(wi[3] & 255) << 8) |
                               ((u32)(wi[5] & 255) << 16) | ((u32)(wi[7] & 255) << 24);
                *reinterpret_cast<uint2*>(dst + (col & 1) * 8) = make_uint2(d0, d1);
            } else {
                // offset o = 8 * (col % 2) + i sits at byte 4 * (o % 4) + o / 4
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint16_t*>(dst + 4 * i + 2 * (col & 1)) =
                        (uint16_t)((wi[i] & 255) | ((wi[i + 4] & 255) << 8));
            }
            if (col == 0) {
                ws.f[h] = __fmul_rn(W, kappa);
                ws.wsum[h] = wsum;
            }
        }
    }
    wave_sync();
    const int hB = col % G;
    const v4i B0 = *reinterpret_cast<const v4i*>(&ws.wB[0][hB][kg][0]);
    const v4i B1 = *reinterpret_cast<const v4i*>(&ws.wB[1][hB][kg][0]);
    int dmax = -2147483647 - 1;
#pragma unroll
    for (int i = 0; i < T / 16; ++i) {
        v4i A0, A1;
        if constexpr (BITS == 4) {
            constexpr u32 M = 0x0F0F0F0Fu;
            const uint4 p = r.kq[i];
            A0 = v4i{(int)(p.x & M), (int)((p.x >> 4) & M), (int)(p.y & M), (int)((p.y >> 4) & M)};
            A1 = v4i{(int)(p.z & M), (int)((p.z >> 4) & M), (int)(p.w & M), (int)((p.w >> 4) & M)};
        } else {
            constexpr u32 M = 0x03030303u;
            const uint2 p = r.kq[i];
            A0 = v4i{(int)(p.x & M), (int)((p.x >> 2) & M), (int)((p.x >> 4) & M),
                     (int)((p.x >> 6) & M)};
            A1 = v4i{(int)(p.y & M), (int)((p.y >> 2) & M), (int)((p.y >> 4) & M),
                     (int)((p.y >> 6) & M)};
        }
        v4i acc = {0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B1, acc, 0, 0, 0);
        dmax = max(dmax, max(max(acc[0], acc[1]), max(acc[2], acc[3])));
    }
    dmax = imax32(imax16(dmax));
    const int E = 2 * dmax - ((1 << BITS) - 1) * ws.wsum[hB];
    const float shat = __fmul_rn((float)E, ws.f[hB]);
    wave_sync();
    return shat;
}

// ------------------------------------------------------------------------------------------
// Exact attention on one 16-token tile (FTF Alg. 1, refinement stage).
// ------------------------------------------------------------------------------------------
template <bool BF16>
struct TileRegs;
template <>
struct TileRegs<true> {
    uint4 k[4];  // k-step ks: 8 bf16 of token row col, channels 32*ks + 8*kg ..
    uint4 v[4];  // token 4*kg + i, 8 bf16 channels 8*col ..
};
template <>
struct TileRegs<false> {
    float4 k[8];  // token row col, channels 32*kg + 4*i ..
    float4 v[8];  // token 4*kg + i/2, channels 8*col + 4*(i%2) ..
};

template <bool BF16, bool NTK, bool NTV>
__device__ __forceinline__ void tile_load(TileRegs<BF16>& r, const void* __restrict__ Kbg,
                                          const void* __restrict__ Vbg, int t0, int lane)
{
    const int col = lane & 15, kg = lane >> 4;
    if constexpr (BF16) {
        const __bf16* Kp = static_cast<const __bf16*>(Kbg);
        const __bf16* Vp = static_cast<const __bf16*>(Vbg);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            r.k[ks] = ld16<NTK>(Kp + (size_t)(t0 + col) * D + ks * 32 + kg * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.v[i] = ld16<NTV>(Vp + (size_t)(t0 + 4 * kg + i) * D + col * 8);
    } else {
        const float* Kp = static_cast<const float*>(Kbg);
        const float* Vp = static_cast<const float*>(Vbg);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r.k[i] = ld16f<NTK>(Kp + (size_t)(t0 + col) * D + kg * 32 + i * 4);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r.v[i] = ld16f<NTV>(Vp + (size_t)(t0 + 4 * kg + i / 2) * D + col * 8 +
                                        (i & 1) * 4);
    }
}

// Online-softmax state of one lane.  m and l belong to head col % G (the lane's score column).
// The unnormalized output o depends on how P.V is computed:
//   bf16 values (MF): on the MFMA, o[j] is the 16 x 16 accumulator of channels 8 r + j (r = 16
//     rows) against the 16 columns (heads col % G, replicated): lane (kg, col) holds channels
//     32 kg + 8 v + j, v = 0..3, of head col, summed over every token;
//   fp32 values: on the VALU, o[h][c] is channel 8 col + c of head h, summed over this lane's
//     tokens (4 kg + v), to be summed over kg at the end.
template <int G, bool MF>
struct SoftState;
template <int G>
struct SoftState<G, true> {
    v4f o[8];
    float m;
    float l;
};
template <int G>
struct SoftState<G, false> {
    float o[G][8];
    float m;
    float l;
};

// Scores S[token t0 + 4 kg + v][head col % G] of a 16-token tile with stored keys.  B operand:
// query head col % G, the same channel slice as the key row in the A operand: for bf16 the four
// k-steps' 8 channels 32 ks + 8 kg .. held in registers (qv), for fp32 channels 32 kg + 4 i ..
// read from the query row in LDS.
template <bool BF16>
__device__ __forceinline__ v4f tile_scores(const TileRegs<BF16>& r, const void* __restrict__ qrow,
                                           const v8bf* qv, int lane)
{
    const int kg = lane >> 4;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r.k[ks]), qv[ks],
                                                          acc, 0, 0, 0);
    } else {
        const float* qf = static_cast<const float*>(qrow);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 qv = *reinterpret_cast<const float4*>(qf + kg * 32 + 4 * i);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[i].x, qv.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[i].y, qv.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[i].z, qv.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[i].w, qv.w, acc, 0, 0, 0);
        }
    }
    return acc;
}

// Online softmax (base 2) of a tile's scores and P.V into the lane's running state.  r.v holds
// the tile's values: 4 x uint4 of bf16 (token 4*kg + i, channels 8*col ..) or 8 x float4.
template <int G, bool VBF16, typename TR>
__device__ __forceinline__ void softmax_pv(v4f acc, const TR& r, SoftState<G, VBF16>& st, int t0,
                                           int L, u32 kbits, float c_log2, int lane)
{
    const int col = lane & 15, kg = lane >> 4;
    const bool head_keep = (kbits >> (col % G)) & 1u;
    float s2[4];
    float tmax = kNegInf;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const bool valid = head_keep && (t0 + 4 * kg + v) < L;
        s2[v] = valid ? acc[v] * c_log2 : kNegInf;
        tmax = fmaxf(tmax, s2[v]);
    }
    tmax = fmax32(fmax16(tmax));
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = (m_new == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(st.m - m_new);
    v4f p;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        p[v] = (s2[v] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(s2[v] - m_new);
        psum += p[v];
    }
    psum = fsum32(fsum16(psum));
    st.l = st.l * alpha + psum;
    st.m = m_new;

    if constexpr (VBF16) {
        // P.V on the bf16 MFMA, O^T[channel][head] += V^T[channel][token] P^T[token][head], one
        // 16x16x32 product per 16 channels 8 r + j (r = 0..15) and j = 0..7.  The K dimension holds
        // every token twice: k = 8 kg + i is token 4 kg + (i % 4), with the bf16 high part of its
        // probability for i < 4 and the low part p - hi for i >= 4, so the fp32 probabilities
        // enter to within 2^-17 relative and the sum over tokens needs no cross-lane step.
        // B: this lane's own probabilities (column col = head col % G, tokens 4 kg + v).
        v8bf bp;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const __bf16 hi = (__bf16)p[v];
            bp[v] = hi;
            bp[v + 4] = (__bf16)(p[v] - (float)hi);
        }
        // A: row r = col holds channel 8 col + j of tokens 4 kg + i: the j-th bf16 of r.v[i];
        // rows past the sequence are zeroed (they may hold anything, even NaN)
        u32 wv[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool in = t0 + 4 * kg + i < L;
            const uint4 x = r.v[i];
            wv[i][0] = in ? x.x : 0u;
            wv[i][1] = in ? x.y : 0u;
            wv[i][2] = in ? x.z : 0u;
            wv[i][3] = in ? x.w : 0u;
        }
        typedef u32 v4u __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32 sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each word
            const u32 d0 = __builtin_amdgcn_perm(wv[1][j >> 1], wv[0][j >> 1], sel);
            const u32 d1 = __builtin_amdgcn_perm(wv[3][j >> 1], wv[2][j >> 1], sel);
            const v8bf a = __builtin_bit_cast(v8bf, (v4u){d0, d1, d0, d1});
            st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp, st.o[j] * alpha, 0, 0, 0);
        }
        return;
    } else {
    // move probabilities to the PV layout: lane (kg, col) needs p[4 kg + v] of every head h of
    // the group, and its rescale factor, from lane h of its own row (column h of the score tile)
    float pp[G][4];
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        al[h] = row_bcast(alpha, h);
#pragma unroll
        for (int v = 0; v < 4; ++v) pp[h][v] = row_bcast(p[v], h);
    }

#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) st.o[h][c] *= al[h];

#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float vv[8];
        if constexpr (VBF16) {
            const uint4 x = r.v[v];
            vv[0] = bf16_lo(x.x); vv[1] = bf16_hi(x.x);
            vv[2] = bf16_lo(x.y); vv[3] = bf16_hi(x.y);
            vv[4] = bf16_lo(x.z); vv[5] = bf16_hi(x.z);
            vv[6] = bf16_lo(x.w); vv[7] = bf16_hi(x.w);
        } else {
            const float4 a = r.v[2 * v], b = r.v[2 * v + 1];
            vv[0] = a.x; vv[1] = a.y; vv[2] = a.z; vv[3] = a.w;
            vv[4] = b.x; vv[5] = b.y; vv[6] = b.z; vv[7] = b.w;
        }
        if (t0 + 4 * kg + v >= L) {  // rows past the sequence may hold anything (even NaN)
#pragma unroll
            for (int c = 0; c < 8; ++c) vv[c] = 0.0f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) st.o[h][c] = fmaf(pp[h][v], vv[c], st.o[h][c]);
    }
    }
}

template <int G, bool BF16>
__device__ __forceinline__ void tile_compute(const TileRegs<BF16>& r, const void* __restrict__ qrow,
                                             const v8bf* qv, SoftState<G, BF16>& st, int t0, int L,
                                             u32 kbits, float c_log2, int lane)
{
    softmax_pv<G, BF16>(tile_scores<BF16>(r, qrow, qv, lane), r, st, t0, L, kbits, c_log2, lane);
}

// ------------------------------------------------------------------------------------------
// Exact attention on one 16-token tile in the residual storage form.  Lane (kg, col) holds
// token row col, channels 32*kg .. 32*kg+31 (the A operand of k-step ks takes channels
// 32*kg + 8*ks ..; the query side reads the same channels).
// ------------------------------------------------------------------------------------------
struct TileRes {
    // full block: a[0] = the 32 channels' codes (16 B at 4 bits, 8 B + 8 unused at 2 bits),
    // a[1..2] = their 8-bit residual codes, a[3] = 16 B of the block's scales (lanes 0-31: the
    // bf16 s of channels 8*(lane%16) .., lanes 32-63: the fp32 s_r of channels 4*(lane-32) ..).
    // Tail block (no low-bit copy): a[0..3] = the 32 channels' 16-bit keys.
    uint4 a[4];
    uint4 v[4];  // as TileRegs<true>::v
};

template <int BITS, bool NT>
__device__ __forceinline__ void tile_load_res(TileRes& r, const uint8_t* __restrict__ kc_bg,
                                              const uint16_t* __restrict__ sc_bg,
                                              const int8_t* __restrict__ kr_bg,
                                              const float* __restrict__ sr_bg,
                                              const __bf16* __restrict__ kt_bg,
                                              const __bf16* __restrict__ V_bg, int t0, int T,
                                              bool tail, int lane)
{
    const int col = lane & 15, kg = lane >> 4;
    constexpr int RB = D * BITS / 8, CB = 32 * BITS / 8;
    const size_t row = (size_t)(t0 + col);
    const size_t blk = (size_t)(t0 / T);
    // the same four loads into the same registers whichever the source, so that the wait
    // counter tracks them alike on both paths
    const char* a0;
    const char* a1;
    const char* a2;
    const char* a3;
    if (tail) {
        const __bf16* kt = kt_bg + row * D + kg * 32;
        a0 = reinterpret_cast<const char*>(kt);
        a1 = reinterpret_cast<const char*>(kt + 8);
        a2 = reinterpret_cast<const char*>(kt + 16);
        a3 = reinterpret_cast<const char*>(kt + 24);
    } else {
        a0 = reinterpret_cast<const char*>(kc_bg + row * RB + kg * CB);
        a1 = reinterpret_cast<const char*>(kr_bg + row * D + kg * 32);
        a2 = a1 + 16;
        a3 = lane < 32 ? reinterpret_cast<const char*>(sc_bg + blk * D + (lane & 15) * 8)
                       : reinterpret_cast<const char*>(sr_bg + blk * D + (lane - 32) * 4);
    }
    if constexpr (BITS == 4) {
        r.a[0] = *reinterpret_cast<const uint4*>(a0);
    } else {
        const uint2 lo = *reinterpret_cast<const uint2*>(a0);
        const uint2 hi = *reinterpret_cast<const uint2*>(tail ? a0 + 8 : a0);
        r.a[0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    r.a[1] = ld16<false>(a1);
    r.a[2] = ld16<false>(a2);
    r.a[3] = *reinterpret_cast<const uint4*>(a3);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.v[i] = ld16<NT>(V_bg + (size_t)(t0 + 4 * kg + i) * D + col * 8);
}

__device__ __forceinline__ u32 byte_of(const uint4& x, int b)
{
    const u32 w = (b >> 2) == 0 ? x.x : (b >> 2) == 1 ? x.y : (b >> 2) == 2 ? x.z : x.w;
    return (w >> ((b & 3) * 8)) & 255u;
}

// Scores of a residual-form tile: Dequant k = (u - half) s + r_q s_r in fp32 (Alg. 1; two fused
// multiply-adds, within an ulp or two of the separately rounded products and sum), split into
// bf16 k_hi = RN_bf16(k) and k_lo = RN_bf16(k - k_hi) (|k - k_hi - k_lo| <= 2^-16 |k|), so that
// q.k_quant + q.k_res accumulates on the bf16 MFMA with fp32 sums (Eq. 4).
// qv: the query operand of k-step ks, channels 32 kg + 8 ks .., in registers.
template <int BITS, int G>
__device__ __forceinline__ v4f tile_scores_res(const TileRes& r, const v8bf* qv,
                                               WaveScratch<G>& ws, bool tail, int lane)
{
    const int kg = lane >> 4;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (tail) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r.a[ks]), qv[ks],
                                                          acc, 0, 0, 0);
        return acc;
    }
    constexpr float half = (float)((1 << BITS) - 1) * 0.5f;
    if (lane >= 32) {
        ws.rsc[lane] = __builtin_bit_cast(float4, r.a[3]);  // s_r
    } else if (lane < 16) {
        const uint4 b = r.a[3];  // the bf16 s of channels 8*lane .. 8*lane+7
        const float4 s0 = make_float4(bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y));
        const float4 s1 = make_float4(bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w));
        ws.rsc[2 * lane] = s0;
        ws.rsc[2 * lane + 1] = s1;
        ws.rsc[64 + 2 * lane] = make_float4(-half * s0.x, -half * s0.y, -half * s0.z, -half * s0.w);
        ws.rsc[65 + 2 * lane] = make_float4(-half * s1.x, -half * s1.y, -half * s1.z, -half * s1.w);
    }
    wave_sync();
    const float* sq = reinterpret_cast<const float*>(ws.rsc) + kg * 32;  // s of my channels
    const float* sr = sq + 128;                                           // s_r of my channels
    const float* nhs = sq + 256;                                          // -half * s
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        v8bf hi, lo;
        // (u - half) s + r_q s_r evaluated as u s + (r_q s_r - half s) with fused multiply-adds
        // (the exact stage only has to stay within the output tolerance), then the high/low
        // split two channels at a time: one packed conversion gives both highs, whose fp32
        // values are the packed word's halves shifted into place
        // the codes of a dword, channel c' at bits BITS*c', spread one per byte:
        // (word >> BITS*m) & mask holds channel (8/BITS) b + m in byte b
        float k[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 8 * ks + i;  // channel 32*kg + c
            constexpr int PER = 32 / BITS;  // channels per dword
            constexpr int PB = 8 / BITS;    // channels per byte
            constexpr u32 M = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
            const int dw = c / PER, cc = c % PER;
            const u32 wd = dw == 0 ? r.a[0].x : dw == 1 ? r.a[0].y : dw == 2 ? r.a[0].z : r.a[0].w;
            const u32 spread = (wd >> (BITS * (cc % PB))) & M;
            const float u = (float)((spread >> (8 * (cc / PB))) & 0xFFu);
            const int rq = (int)(int8_t)byte_of(c < 16 ? r.a[1] : r.a[2], c & 15);
            k[i] = fmaf(u, sq[c], fmaf((float)rq, sr[c], nhs[c]));
        }
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const v2bf h = __builtin_convertvector((v2f){k[i], k[i + 1]}, v2bf);
            const u32 hb = __builtin_bit_cast(u32, h);
            const v2bf l = __builtin_convertvector(
                (v2f){k[i] - as_f((int)(hb << 16)), k[i + 1] - as_f((int)(hb & 0xFFFF0000u))}, v2bf);
            hi[i] = h[0];
            hi[i + 1] = h[1];
            lo[i] = l[0];
            lo[i + 1] = l[1];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, qv[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, qv[ks], acc, 0, 0, 0);
    }
    wave_sync();
    return acc;
}

template <int G, int BITS>
__device__ __forceinline__ void tile_compute_res(const TileRes& r, const v8bf* qv,
                                                 SoftState<G, true>& st, WaveScratch<G>& ws, int t0,
                                                 int L, u32 kbits, float c_log2, bool tail,
                                                 int lane)
{
    softmax_pv<G, true>(tile_scores_res<BITS, G>(r, qv, ws, tail, lane), r, st, t0, L, kbits,
                        c_log2, lane);
}

// ------------------------------------------------------------------------------------------
// Low-bit key copy of one block (App. A, Eqs. 5-7)
// ------------------------------------------------------------------------------------------
// App. A quantizer of one whole block by a work-group of 256 threads (quantize_kernel runs one
// per (b, kv head, block); the fused decode-loop step runs it at a block boundary).
// Thread (rg, cg) = (t / 16, t % 16) loads channels 8 cg .. 8 cg + 7 of rows rg, rg + 16, ...
// (16-byte loads, 16 threads per row), takes their absolute maxima over its rows, and the
// per-channel maxima over the 16 row groups meet in LDS.  It then writes the codes of its eight
// channels of each of its rows as one 4-byte word (low nibble = even channel).  The arithmetic is
// quantize_block's, so the codes and scales are the same bytes: s = RN(amax / 7.5),
// u = clamp(floor(RN(x * RN(7.5 / amax))) + 8, 0, 15), and u = 8 for an all-zero channel (its
// stored reciprocal is 0).
template <int T, bool BF16>
__device__ __forceinline__ void quantize_block_wg(const void* __restrict__ K,
                                                  uint8_t* __restrict__ Kq,
                                                  uint16_t* __restrict__ scales, int cap, int bg,
                                                  int j, float (*part)[D], float* inv_s)
{
    constexpr int RPT = T / 16;  // rows per thread
    const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
    const size_t row0 = (size_t)bg * cap + (size_t)j * T;
    float x[RPT][8];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const size_t e0 = (row0 + rg + 16 * r) * D + cg * 8;
        if constexpr (BF16) {
            const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(K) + e0);
            x[r][0] = bf16_lo(v.x); x[r][1] = bf16_hi(v.x);
            x[r][2] = bf16_lo(v.y); x[r][3] = bf16_hi(v.y);
            x[r][4] = bf16_lo(v.z); x[r][5] = bf16_hi(v.z);
            x[r][6] = bf16_lo(v.w); x[r][7] = bf16_hi(v.w);
        } else {
            const float4* fp = reinterpret_cast<const float4*>(static_cast<const float*>(K) + e0);
            const float4 a = fp[0], b = fp[1];
            x[r][0] = a.x; x[r][1] = a.y; x[r][2] = a.z; x[r][3] = a.w;
            x[r][4] = b.x; x[r][5] = b.y; x[r][6] = b.z; x[r][7] = b.w;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float am = 0.0f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) am = fmaxf(am, fabsf(x[r][i]));
        part[rg][cg * 8 + i] = am;
    }
    __syncthreads();
    if (t < D) {
        float amax = 0.0f;
#pragma unroll
        for (int g = 0; g < 16; ++g) amax = fmaxf(amax, part[g][t]);
        float s = 0.0f, inv = 0.0f;
        if (amax > 0.0f) {
            s = __fdiv_rn(amax, 7.5f);
            inv = __fdiv_rn(7.5f, amax);
        }
        scales[((size_t)bg * (cap / T) + j) * D + t] = scale_bits(s);
        inv_s[t] = inv;
    }
    __syncthreads();
    float iv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) iv[i] = inv_s[cg * 8 + i];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        u32 word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int u = (int)floorf(__fmul_rn(x[r][i], iv[i])) + 8;
            u = min(max(u, 0), 15);
            word |= (u32)u << (4 * i);
        }
        *reinterpret_cast<u32*>(Kq + (row0 + rg + 16 * r) * (D / 2) + cg * 4) = word;
    }
}

// ------------------------------------------------------------------------------------------
// Decode kernel (sparse and dense)
// ------------------------------------------------------------------------------------------
template <int G, int NW>
struct __attribute__((aligned(16))) DecodeShared {
    WaveScratch<G> wave[NW];
    union {
        struct {                                            // the waves' softmax states
            float o[NW][G][D];
            float m[NW][G];
            float l[NW][G];
        } merge;
        struct {                                            // final merge of the splits
            float wgt[G][kMaxSplits];                       // weight of each non-empty split
            uint16_t idx[G][kMaxSplits];                    // its index
            float M[G], Lsum[G];
            int cnt[G];
        } fin;
        struct {                                            // final merge, fast path: the
            v4f acc[NW * 64];                               // threads' shares of the splits
            float M[NW * 64], L[NW * 64];
        } share;
        struct {                                            // running-max selection
            float s[kMaxBlocksPerSplit][G];                 // scan estimates of the split's blocks
            float mt[G];                                    // Alg. 1 pseudo-max of each head
            u32 bits[kMaxBlocksPerSplit];                   // heads that keep each block
        } run;
        struct {                                            // fused decode-loop step: the block
            float part[16][D];                              // the new token completes, quantized
            float inv[D];                                   // by the work-group (before the scan)
        } quant;
    } u;
    float4 q[G * D / 4];                   // the group's query rows (bf16 or fp32 bytes)
    uint8_t kbits[kMaxBlocksPerSplit];     // per-block head mask (bit h = query head h of group)
    uint8_t list[NW][kMaxBlocksPerSplit];  // kept blocks (offsets in the split), per wave
    int is_last;
    u32 mask;                              // non-empty splits (when S <= 32)
};

__device__ __forceinline__ float wave_max(float x)
{
    return fmax32(fmax16(row16_max(x)));
}

__device__ __forceinline__ float wave_sum(float x)
{
    x += as_f(dpp<0xB1>(as_i(x)));
    x += as_f(dpp<0x4E>(as_i(x)));
    x += as_f(dpp<0x141>(as_i(x)));
    x += as_f(dpp<0x140>(as_i(x)));
    return fsum32(fsum16(x));
}

// Device-scope (agent) relaxed atomic loads and stores: on gfx950 these are plain global loads
// and stores with the device-scope cache policy (sc1), which write through to, and read from,
// the point where all XCDs' accesses are coherent.  The split partials travel this way so that
// the merging work-group needs no cache-wide writeback or invalidate (an agent-scope fence costs
// a walk of the XCD's L2 per work-group).
__device__ __forceinline__ void st_dev(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev2(float2* p, float a, float b)
{
    const unsigned long long v = (unsigned long long)(u32)as_i(a) |
                                 ((unsigned long long)(u32)as_i(b) << 32);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float2* p)
{
    const unsigned long long v = __hip_atomic_load(
        reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(as_f((int)(u32)v), as_f((int)(u32)(v >> 32)));
}

// 16- and 8-byte device-scope accesses through a buffer resource (raw buffer, no swizzle, the
// gfx9 default format word), with the same cache policy as the relaxed agent-scope atomics above
// (sc1).  A buffer access outside the resource's byte range reads zero and writes nothing.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kCpolDevice = 16;  // sc1
__device__ __forceinline__ rsrc_t dev_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev16(rsrc_t r, int off, v4f v)
{
    typedef u32 v4u __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, kCpolDevice);
}
__device__ __forceinline__ v4f ld_dev16(rsrc_t r, int off)
{
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDevice));
}
__device__ __forceinline__ void st_dev8(rsrc_t r, int off, float a, float b)
{
    typedef u32 v2u __attribute__((ext_vector_type(2)));
    const v2u v = {(u32)as_i(a), (u32)as_i(b)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpolDevice);
}
__device__ __forceinline__ float2 ld_dev8(rsrc_t r, int off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolDevice);
    return make_float2(as_f((int)v[0]), as_f((int)v[1]));
}

// One work-group per (sequence b, kv head g, split of the sequence).  Phases:
//   1. scan and select (sparse only): every wave scans the sink and local blocks (its own
//      pseudo-max), then its share of the split's other full blocks, two items in flight, and
//      applies the top-delta test to each block as soon as it is scanned;
//   2. compaction of the kept blocks into a per-wave LDS list, in increasing order;
//   3. exact attention over the kept blocks' 16-token tiles (pipelined the same way);
//   4. merge of the waves' softmax states -> one (o, m, l) partial per query head;
//   5. the last work-group of (b, g) to finish (atomic counter) merges the splits' partials
//      with the log-sum-exp rule into out and lse, and resets the counter.
// BITS is the width of the scanned codes; RES selects the residual storage form (thumbnail +
// 8-bit residual instead of stored keys; bf16 values; sparse only).
template <int T, int G, bool BF16, bool SPARSE, int BITS, bool RES, bool STREAM>
__global__ __launch_bounds__((RES ? kResWaves : kWaves) * 64, 2) void decode_kernel(DecodeParams p)
{
    // waves per work-group: eight in the residual form, whose exact tiles cost more arithmetic
    constexpr int NW = RES ? kResWaves : kWaves;
    __shared__ DecodeShared<G, NW> sh;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int col = lane & 15, kg = lane >> 4;

    // work-group -> (unit, split).  A unit is G query heads (the kernel's width) of one (b, kv
    // head): the whole group, its padded form, or one of several slices of a group wider than
    // the kernel.  Sparse: the S splits of one unit are consecutive work-groups, which the
    // dispatcher deals round-robin to the XCDs, so every XCD holds splits of every unit and the
    // exact work of a unit that keeps many blocks is spread over all of them.  Ranks 0 and 1
    // are the splits holding the sink (0) and the local block (S-1), which always carry exact
    // work; the ranks of a unit start at work-group offset S - unit mod S, so that these forced
    // splits of different units fall on different XCDs.  Dense (the same work in every split):
    // all splits of one unit share blockIdx.x mod units, one XCD when the unit count is a
    // multiple of 8.  Each layout measured faster than the other for its kernel.
    const int n_units = p.B * p.Hkv * p.NSUB;
    const int id = blockIdx.x;
    const int unit = SPARSE ? id / p.S : id % n_units;
    const int rank = SPARSE ? (id % p.S + unit) % p.S : id / n_units;
    int split = rank;
    if (SPARSE && p.S > 1) split = rank == 0 ? 0 : (rank == 1 ? p.S - 1 : rank - 1);
    const int bg = unit / p.NSUB;  // (b, kv head) whose keys and values the unit reads
    const int sub = unit % p.NSUB;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    // real query heads of the unit: the first nh of its G; the others are padding, with a zero
    // query in the exact stage, never kept and never written
    const int nh = min(G, p.G - sub * G);
    // this sequence's length: the common one, or (decode loops) its own from device memory
    int L_b = p.L;
    if (p.seq_lens) L_b = min(max(p.seq_lens[b], 0), p.L);
    // fused decode-loop step: the new token at position pos = seq_lens[b] (if below L) is part of
    // this step; nobody writes the length before every unit of the sequence has read it
    int pos = -1;
    if constexpr (SPARSE && !RES) {
        if (p.k_new) {
            const int l0 = p.seq_lens[b];
            if (l0 >= 0 && l0 < p.L) {
                pos = l0;
                L_b = l0 + 1;
            }
        }
    }
    const int nf_b = L_b / T;            // full blocks
    const int nb_b = (L_b + T - 1) / T;  // blocks, the last one possibly partial
    const int jb = split * p.R;
    const int je = min(nb_b, jb + p.R);

    const size_t esz = BF16 ? 2 : 4;
    const size_t kv_off = (size_t)bg * p.cap * D;
    const char* Kbg = p.K ? static_cast<const char*>(p.K) + kv_off * esz : nullptr;
    const char* Vbg = static_cast<const char*>(p.V) + kv_off * esz;
    const int h0 = b * p.Hq + g * p.G + sub * G;  // first query row of the unit

    if constexpr (SPARSE && !RES) {
        if (pos >= 0) {
            // The new key and value rows go to position pos.  The split that holds that block
            // writes both (it alone reads them, in its exact stage); when the token completes
            // the block, every work-group of the kv head also writes the key row and quantizes
            // the block itself, because every one of them scans it as its local block: all
            // write the same bytes, and each reads back only what it wrote itself (after the
            // barrier), so no work-group waits for another.
            static_assert(NW * 64 == 256, "the block quantizer runs on 256 threads");
            const int jt = pos / T;
            const bool completes = (pos + 1) % T == 0;
            const bool owner = jt / p.R == split;
            constexpr int kRow16 = (int)(D * (BF16 ? 2 : 4) / 16);  // 16-byte pieces of a row
            const size_t src = (size_t)bg * D * esz;
            const size_t dst = ((size_t)bg * p.cap + pos) * D * esz;
            const int t = (int)threadIdx.x;
            char* Kw = static_cast<char*>(const_cast<void*>(p.K));
            char* Vw = static_cast<char*>(const_cast<void*>(p.V));
            const char* kn = static_cast<const char*>(p.k_new);
            const char* vn = static_cast<const char*>(p.v_new);
            if ((owner || completes) && t < kRow16)
                reinterpret_cast<uint4*>(Kw + dst)[t] = reinterpret_cast<const uint4*>(kn + src)[t];
            if (owner && t >= kRow16 && t < 2 * kRow16)
                reinterpret_cast<uint4*>(Vw + dst)[t - kRow16] =
                    reinterpret_cast<const uint4*>(vn + src)[t - kRow16];
            if (completes) {
                __syncthreads();  // the key row is written
                quantize_block_wg<T, BF16>(p.K, const_cast<uint8_t*>(p.Kq),
                                           const_cast<uint16_t*>(p.scales), p.cap, bg, jt,
                                           sh.u.quant.part, sh.u.quant.inv);
                __syncthreads();  // codes and scales written
            }
        }
    }

    WaveScratch<G>& ws = sh.wave[w];
    constexpr int NT = T / 16;
    int n_kept;

    // the unit's query rows (at most 16 bytes per thread), copied to LDS once the first scan
    // loads are in flight; the load is unconditional (clamped index, inside the real rows) so
    // that it is issued before them and the copy waits only for itself; padding rows are zero
    constexpr int kRow16 = (int)(D * (BF16 ? 2 : 4) / 16);
    constexpr int kQ16 = G * kRow16;
    static_assert(kQ16 <= NW * 64, "query rows exceed one 16-byte load per thread");
    const int q16_real = nh * kRow16;
    const float4 qcopy = reinterpret_cast<const float4*>(
        static_cast<const char*>(p.q) + (size_t)h0 * D * esz)[min((int)threadIdx.x, q16_real - 1)];
    auto publish_q = [&]() {
        if ((int)threadIdx.x < kQ16)
            sh.q[threadIdx.x] = (int)threadIdx.x < q16_real ? qcopy : make_float4(0.f, 0.f, 0.f, 0.f);
    };

    if constexpr (SPARSE) {
        if (!p.ext_mask) {
            constexpr int HPL = (G + 3) / 4;
            float qw[HPL][8];
    #pragma unroll
            for (int k = 0; k < HPL; ++k) {
                const int h = (G >= 4) ? (kg + 4 * k) : (kg % G);
                const int hq = h0 + min(h, nh - 1);  // a padding head scans a real head's row
                if constexpr (BF16) {
                    const uint4 x = *reinterpret_cast<const uint4*>(
                        static_cast<const __bf16*>(p.q) + (size_t)hq * D + col * 8);
                    qw[k][0] = bf16_lo(x.x); qw[k][1] = bf16_hi(x.x);
                    qw[k][2] = bf16_lo(x.y); qw[k][3] = bf16_hi(x.y);
                    qw[k][4] = bf16_lo(x.z); qw[k][5] = bf16_hi(x.z);
                    qw[k][6] = bf16_lo(x.w); qw[k][7] = bf16_hi(x.w);
                } else {
                    const float4* qp = reinterpret_cast<const float4*>(
                        static_cast<const float*>(p.q) + (size_t)hq * D + col * 8);
                    const float4 a = qp[0], c = qp[1];
                    qw[k][0] = a.x; qw[k][1] = a.y; qw[k][2] = a.z; qw[k][3] = a.w;
                    qw[k][4] = c.x; qw[k][5] = c.y; qw[k][6] = c.z; qw[k][7] = c.w;
                }
            }

            const uint8_t* kq_bg = p.Kq + (size_t)bg * p.cap * (D * BITS / 8);
            const uint16_t* sc_bg = p.scales + (size_t)bg * (p.cap / T) * D;
            const int nf = nf_b;
            const u32 all_heads = (1u << nh) - 1u;
            // Forced blocks of the split (sink 0, the local block nf-1 and a partial tail) are kept
            // for every head; every other block of the split is a scan item of exactly one wave.
            if (w == 0) {
                for (int t = lane; t < je - jb; t += 64) {
                    const int j = jb + t;
                    if (j == 0 || j >= nf - 1) {
                        sh.kbits[t] = (uint8_t)all_heads;
                        if (p.keep_mask)
                            for (int h = 0; h < nh; ++h) p.keep_mask[(size_t)(h0 + h) * p.mask_stride + j] = 1;
                    } else if (p.running) {
                        sh.kbits[t] = 0;  // decided after the scan
                    }
                    if (p.running) sh.u.run.bits[t] = 0u;
                }
            }
            // Scan items of this wave: the sink and local blocks (each wave forms the pseudo-max of
            // Eq. 3 itself, so that it can apply Eq. 1 to its own blocks at once), then the split's
            // non-forced full blocks j_lo + w, j_lo + w + NW, ...
            const int n_pro = nf >= 1 ? 2 : 0;
            const int j_lo = max(jb, 1);
            const int j_hi = min(je, nf - 1);
            const int n_main = max(j_hi - j_lo, 0);
            const int n_items = n_pro + (n_main > w ? (n_main - w + NW - 1) / NW : 0);
            auto block_of = [&](int k) -> int {
                if (k < n_pro) return k == 0 ? 0 : nf - 1;
                return j_lo + w + (k - n_pro) * NW;
            };
            if (n_items > 0) {
                float pro0 = 0.0f, theta = 0.0f;  // lanes < G: head = lane
                auto load = [&](ScanRegs<T, BITS>& r, int k, auto nt) {
                    const int j = block_of(k);
                    scan_load<T, BITS, decltype(nt)::value>(
                        r, kq_bg + (size_t)j * T * (D * BITS / 8), sc_bg + (size_t)j * D, lane);
                };
                auto process = [&](const ScanRegs<T, BITS>& r, int k) {
                    const float shat = scan_compute<T, G, BITS>(r, qw, p.kappa, ws, lane);
                    if (k == 0) {
                        pro0 = shat;
                    } else if (k == 1) {
                        theta = __fsub_rn(fmaxf(pro0, shat), p.delta);
                        if (p.running && w == 0 && lane < G) sh.u.run.mt[lane] = fmaxf(pro0, shat);
                    } else if (p.running) {
                        // running-max variant: the estimate is kept for the decision after the
                        // scan, which needs every earlier block of the split
                        if (lane < G) sh.u.run.s[block_of(k) - jb][lane] = shat;
                    } else {
                        // selection, Eq. 1 with the pseudo-max: shat >= mtilde - delta
                        const int j = block_of(k);
                        const bool keep = lane < nh && shat >= theta;
                        const u32 bits = (u32)__ballot(keep) & all_heads;
                        if (lane == 0) sh.kbits[j - jb] = (uint8_t)bits;
                        if (p.keep_mask && lane < nh)
                            p.keep_mask[(size_t)(h0 + lane) * p.mask_stride + j] = keep ? 1 : 0;
                    }
                };
                // Two items in flight: item k + 1 is loaded while item k is computed.  The steady
                // loop issues loads only for items that exist and the epilogue issues none past the
                // end, so no load is left outstanding.  The scheduling barriers keep each prefetch
                // issued before the computation that follows it in program order (otherwise the
                // scheduler hoists that computation's first use of its buffer above the loads, and
                // the in-order wait counter then waits for the prefetch too).
                auto pipeline = [&](auto nt) {
                    ScanRegs<T, BITS> ra, rb;
                    load(ra, 0, nt);
                    __builtin_amdgcn_sched_barrier(0);
                    publish_q();
                    int k = 0;
                    for (; k + 2 < n_items; k += 2) {
                        load(rb, k + 1, nt);
                        __builtin_amdgcn_sched_barrier(0);
                        process(ra, k);
                        load(ra, k + 2, nt);
                        __builtin_amdgcn_sched_barrier(0);
                        process(rb, k + 1);
                    }
                    if (k + 1 < n_items) {
                        load(rb, k + 1, nt);
                        __builtin_amdgcn_sched_barrier(0);
                        process(ra, k);
                        process(rb, k + 1);
                    } else {
                        process(ra, k);
                    }
                };
                pipeline(Flag<STREAM>{});
            } else {
                publish_q();
            }
        } else {
            // selection made outside (a comparator rule): every block's head mask is read from
            // the caller's keep mask; nothing is scanned
            for (int t = threadIdx.x; t < je - jb; t += NW * 64) {
                u32 bits = 0;
                for (int h = 0; h < nh; ++h)
                    bits |= (p.ext_mask[(size_t)(h0 + h) * p.mask_stride + jb + t] != 0 ? 1u : 0u)
                            << h;
                sh.kbits[t] = (uint8_t)bits;
            }
            publish_q();
        }
        __syncthreads();  // kbits complete, query rows in LDS

        if (p.running && !p.ext_mask) {
            // Running-max variant of Eq. 1: per head, the split's scanned blocks in increasing
            // order; block j is kept iff shat_j >= RN(M - delta), M the maximum of mtilde and the
            // estimates of the split's earlier scanned blocks.  One wave per head, 64 blocks at a
            // time: an exclusive prefix maximum over the lanes plus the earlier chunks' maximum.
            const int nf = nf_b;
            for (int h = w; h < nh; h += NW) {
                float carry = sh.u.run.mt[h];
                for (int base = 0; base < je - jb; base += 64) {
                    const int t = base + lane;
                    const int j = jb + t;
                    const bool scanned = t < je - jb && j >= 1 && j < nf - 1;
                    const float sv = scanned ? sh.u.run.s[t][h] : kNegInf;
                    float inc = sv;
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const float o = __shfl_up(inc, d);
                        if (lane >= d) inc = fmaxf(inc, o);
                    }
                    float before = __shfl_up(inc, 1);
                    if (lane == 0) before = kNegInf;
                    const bool keep = scanned && sv >= __fsub_rn(fmaxf(carry, before), p.delta);
                    if (keep) atomicOr(&sh.u.run.bits[t], 1u << h);
                    if (scanned && p.keep_mask)
                        p.keep_mask[(size_t)(h0 + h) * p.mask_stride + j] = keep ? 1 : 0;
                    carry = fmaxf(carry, __shfl(inc, 63));
                }
            }
            __syncthreads();
            for (int t = threadIdx.x; t < je - jb; t += NW * 64)
                sh.kbits[t] |= (uint8_t)sh.u.run.bits[t];
            __syncthreads();
        }

        // every wave compacts the kept blocks of the split, in increasing order, into its own
        // list (identical in all waves)
        int n = 0;
        for (int base = 0; base < je - jb; base += 64) {
            const int t = base + lane;
            const u32 bits = t < je - jb ? sh.kbits[t] : 0u;
            const unsigned long long ball = __ballot(bits != 0);
            const int pos = __popcll(ball & ((1ull << lane) - 1ull));
            if (bits != 0) sh.list[w][n + pos] = (uint8_t)t;
            n += __popcll(ball);
        }
        n_kept = n;
    } else {
        n_kept = max(je - jb, 0);
        publish_q();
        __syncthreads();  // query rows in LDS
    }

    // the exact stage reads head col % G's query row from LDS: for 16-bit inputs once, into
    // the MFMA operand registers of the four k-steps (channels 32 ks + 8 kg .. for stored keys,
    // 32 kg + 8 ks .. in the residual form), for fp32 at every tile
    const void* qrow = reinterpret_cast<const char*>(sh.q) + (size_t)(col % G) * D * esz;
    v8bf qv[4];
    if constexpr (BF16) {
        const __bf16* qb = static_cast<const __bf16*>(qrow);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qv[ks] = *reinterpret_cast<const v8bf*>(qb + (RES ? kg * 32 + ks * 8 : ks * 32 + kg * 8));
    }

    // exact attention over the kept blocks, 16-token tiles dealt round-robin to the waves,
    // pipelined like the scan (two tiles in flight, no load past the last tile)
    constexpr bool MF = BF16;  // P.V on the MFMA for 16-bit values (see SoftState)
    SoftState<G, MF> st;
    if constexpr (MF) {
#pragma unroll
        for (int j = 0; j < 8; ++j) st.o[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) st.o[h][c] = 0.0f;
    }
    st.m = kNegInf;
    st.l = 0.0f;
    {
        const int n_tiles = n_kept * NT;
        const int n_w = n_tiles > w ? (n_tiles - w + NW - 1) / NW : 0;
        if (n_w > 0) {
            auto tile_of = [&](int k, int& t0, u32& kb) {
                const int it = w + k * NW;
                const int kk = it / NT;
                int off;
                if constexpr (SPARSE) {
                    off = sh.list[w][kk];
                    kb = sh.kbits[off];
                } else {
                    off = kk;
                    kb = (1u << nh) - 1u;
                }
                t0 = (jb + off) * T + (it % NT) * 16;
            };
            typedef typename pick<RES, TileRes, TileRegs<BF16>>::type TR;
            // residual form: tiles of full blocks are rebuilt from thumbnail + residual, the tiles
            // of a partial tail block (no low-bit copy) read the 16-bit keys
            const int full_end = nf_b * T;
            // STREAM: the streaming policy for the values (and, in the dense step, the keys); the
            // kept keys of the sparse step keep the default policy (measured slower otherwise)
            auto load_tile = [&](TR& r, int t0, auto nt) {
                constexpr bool NT = decltype(nt)::value;
                if constexpr (RES)
                    tile_load_res<BITS, NT>(
                        r, p.Kq + (size_t)bg * p.cap * (D * BITS / 8),
                        p.scales + (size_t)bg * (p.cap / T) * D, p.Kr + (size_t)bg * p.cap * D,
                        p.res_scales + (size_t)bg * (p.cap / T) * D,
                        reinterpret_cast<const __bf16*>(Kbg), reinterpret_cast<const __bf16*>(Vbg),
                        t0, T, t0 >= full_end, lane);
                else
                    tile_load<BF16, NT && !SPARSE, NT>(r, Kbg, Vbg, t0, lane);
            };
            auto compute_tile = [&](const TR& r, int t0, u32 kb) {
                if constexpr (RES)
                    tile_compute_res<G, BITS>(r, qv, st, ws, t0, L_b, kb, p.c_log2,
                                              t0 >= full_end, lane);
                else
                    tile_compute<G, BF16>(r, qrow, qv, st, t0, L_b, kb, p.c_log2, lane);
            };
            auto pipeline = [&](auto nt) {
                TR ta, tb;
                int t0a, t0b;
                u32 kba, kbb;
                tile_of(0, t0a, kba);
                load_tile(ta, t0a, nt);
                int k = 0;
                for (; k + 2 < n_w; k += 2) {
                    tile_of(k + 1, t0b, kbb);
                    load_tile(tb, t0b, nt);
                    __builtin_amdgcn_sched_barrier(0);
                    compute_tile(ta, t0a, kba);
                    tile_of(k + 2, t0a, kba);
                    load_tile(ta, t0a, nt);
                    __builtin_amdgcn_sched_barrier(0);
                    compute_tile(tb, t0b, kbb);
                }
                if (k + 1 < n_w) {
                    tile_of(k + 1, t0b, kbb);
                    load_tile(tb, t0b, nt);
                    __builtin_amdgcn_sched_barrier(0);
                    compute_tile(ta, t0a, kba);
                    compute_tile(tb, t0b, kbb);
                } else {
                    compute_tile(ta, t0a, kba);
                }
            };
            pipeline(Flag<STREAM>{});
        }
    }

    if constexpr (!MF) {
        // sum the four token subsets (kg) of every lane's channels
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float x = st.o[h][c];
                x = fsum32(fsum16(x));
                st.o[h][c] = x;
            }
    }

    // merge the waves' softmax states into this split's partial
    __syncthreads();  // the shat table is reused as the merge buffer
    if constexpr (MF) {
        // lane (kg, col < G): channels 32 kg + 8 v + j of head col are st.o[j][v]
        if (col < G) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float4* dst = reinterpret_cast<float4*>(&sh.u.merge.o[w][col][32 * kg + 8 * v]);
                dst[0] = make_float4(st.o[0][v], st.o[1][v], st.o[2][v], st.o[3][v]);
                dst[1] = make_float4(st.o[4][v], st.o[5][v], st.o[6][v], st.o[7][v]);
            }
            if (kg == 0) {
                sh.u.merge.m[w][col] = st.m;
                sh.u.merge.l[w][col] = st.l;
            }
        }
    } else if (kg == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float4* dst = reinterpret_cast<float4*>(&sh.u.merge.o[w][h][col * 8]);
            dst[0] = make_float4(st.o[h][0], st.o[h][1], st.o[h][2], st.o[h][3]);
            dst[1] = make_float4(st.o[h][4], st.o[h][5], st.o[h][6], st.o[h][7]);
        }
        if (col < G) {
            sh.u.merge.m[w][col] = st.m;
            sh.u.merge.l[w][col] = st.l;
        }
    }
    __syncthreads();
    const size_t rec0 = ((size_t)unit * p.S + split) * G;
    const bool fast = p.S <= 32;  // the counter word can carry a mask of the non-empty splits
    if (n_kept > 0) {
        // one 16-byte store per four channels of a real head, (m, l) with the first four
        const rsrc_t ro = dev_rsrc(p.part_o + rec0 * D, G * D * 4);
        const rsrc_t rml = dev_rsrc(p.part_ml + rec0, G * 8);
        for (int e = threadIdx.x; e < nh * (D / 4); e += NW * 64) {
            const int h = e / (D / 4), c = (e % (D / 4)) * 4;
            float M = kNegInf;
#pragma unroll
            for (int v = 0; v < NW; ++v) M = fmaxf(M, sh.u.merge.m[v][h]);
            v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
            float l = 0.0f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float mv = sh.u.merge.m[v][h];
                const float sc = (mv == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
                const v4f ov = *reinterpret_cast<const v4f*>(&sh.u.merge.o[v][h][c]);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = fmaf(ov[i], sc, o[i]);
                l = fmaf(sh.u.merge.l[v][h], sc, l);
            }
            st_dev16(ro, e * 16, o);
            if (c == 0) st_dev8(rml, h * 8, M, l);
        }
    } else if (!fast && (int)threadIdx.x < nh) {
        st_dev2(&p.part_ml[rec0 + threadIdx.x], kNegInf, 0.0f);
    }

    // split-KV combine by the last work-group of (b, g) to finish.  Every thread waits until its
    // device-scope partial stores have completed (s_waitcnt 0) before the barrier; only then does
    // one thread count this split as done.  The counter word holds the number of finished
    // splits in its high half and, when S <= 32, a bit per split that wrote a partial in its low
    // half (each split adds its bit once, so no carry).  The work-group that brings the count to
    // S reads the partials with device-scope loads, issued after its counter update returned.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long add =
            (1ull << 32) | ((fast && n_kept > 0) ? (1ull << split) : 0ull);
        const unsigned long long old = __hip_atomic_fetch_add(
            &p.counters[unit], add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.is_last = (u32)(old >> 32) == (u32)(p.S - 1);
        sh.mask = (u32)(old | add);
    }
    __syncthreads();
    if (!sh.is_last) return;
    if (threadIdx.x == 0) {  // ready for the next call
        __hip_atomic_store(&p.counters[unit], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (SPARSE && !RES) {
            if (p.k_new) {
                // every work-group of this unit has read the length; the last unit of the
                // sequence to get here advances it (and returns the count to zero)
                unsigned long long* sc = p.counters + (kCounterSlots - 1 - b);
                const unsigned long long seen =
                    __hip_atomic_fetch_add(sc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (seen == (unsigned long long)(p.Hkv * p.NSUB - 1)) {
                    __hip_atomic_store(sc, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (pos >= 0) p.seq_lens_out[b] = pos + 1;
                }
            }
        }
    }

    const size_t base = (size_t)unit * p.S * G;
    if (fast) {
        // Thread (part, e) merges four channels e of one head over a share of the non-empty
        // splits: those of rank part, part + P, ... among them, in increasing split order, read
        // with 16-byte device-scope loads in rounds of kMB splits.  The P shares are then merged
        // in part order through LDS, so the result does not depend on timing.
        constexpr int NT = NW * 64;
        constexpr int NE4 = G * (D / 4);
        static_assert(NT % NE4 == 0, "the group's outputs must tile the work-group");
        constexpr int P = NT / NE4;
        constexpr int kMB = P == 1 ? 16 : 8;
        const int e = (int)threadIdx.x % NE4, part = (int)threadIdx.x / NE4;
        const int h = e / (D / 4), c = (e % (D / 4)) * 4;
        const bool real = h < nh;  // padding heads read and write nothing
        u32 mine = real ? sh.mask : 0u;
        if constexpr (P > 1) {
            u32 rest = mine;
            mine = 0u;
            for (int r = 0; rest != 0u; ++r) {
                const u32 low = rest & (0u - rest);
                if (r % P == part) mine |= low;
                rest ^= low;
            }
        }
        const rsrc_t ro = dev_rsrc(p.part_o + base * D, p.S * G * D * 4);
        const rsrc_t rml = dev_rsrc(p.part_ml + base, p.S * G * 8);
        float M = kNegInf, Ls = 0.0f;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        while (mine != 0u) {
            int sidx[kMB];
            int nb = 0;
#pragma unroll
            for (int u = 0; u < kMB; ++u) {
                sidx[u] = mine ? __builtin_ctz(mine) : 0;
                if (mine) {
                    mine &= mine - 1u;
                    ++nb;
                }
            }
            float2 ml[kMB];
            v4f v[kMB];
#pragma unroll
            for (int u = 0; u < kMB; ++u) {
                if (u < nb) {
                    const int r = sidx[u] * G + h;
                    ml[u] = ld_dev8(rml, r * 8);
                    v[u] = ld_dev16(ro, (r * D + c) * 4);
                } else {
                    ml[u] = make_float2(kNegInf, 0.0f);
                    v[u] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            // a head may have kept nothing in a split that another head used (m = -inf)
            float Mb = M;
#pragma unroll
            for (int u = 0; u < kMB; ++u)
                if (ml[u].y > 0.0f) Mb = fmaxf(Mb, ml[u].x);
            const float a = (M == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(M - Mb);
            v4f sa = acc * a;
            float sl = Ls * a;
#pragma unroll
            for (int u = 0; u < kMB; ++u) {
                const float wgt = ml[u].y > 0.0f ? __builtin_amdgcn_exp2f(ml[u].x - Mb) : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) sa[i] = fmaf(v[u][i], wgt, sa[i]);
                sl = fmaf(ml[u].y, wgt, sl);
            }
            M = Mb;
            acc = sa;
            Ls = sl;
        }
        if constexpr (P > 1) {
            sh.u.share.acc[threadIdx.x] = acc;
            sh.u.share.M[threadIdx.x] = M;
            sh.u.share.L[threadIdx.x] = Ls;
            __syncthreads();
            if (part != 0) return;
            float Mb = M;
#pragma unroll
            for (int q = 1; q < P; ++q)
                if (sh.u.share.L[q * NE4 + e] > 0.0f) Mb = fmaxf(Mb, sh.u.share.M[q * NE4 + e]);
            const float a = (M == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(M - Mb);
            acc = acc * a;
            Ls = Ls * a;
#pragma unroll
            for (int q = 1; q < P; ++q) {
                const float Lq = sh.u.share.L[q * NE4 + e];
                const float wgt =
                    Lq > 0.0f ? __builtin_amdgcn_exp2f(sh.u.share.M[q * NE4 + e] - Mb) : 0.0f;
                const v4f vq = sh.u.share.acc[q * NE4 + e];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(vq[i], wgt, acc[i]);
                Ls = fmaf(Lq, wgt, Ls);
            }
            M = Mb;
        }
        if (!real) return;
        // an empty sequence (length 0) has no softmax: out = 0, lse = -inf
        v4f r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = Ls > 0.0f ? acc[i] / Ls : 0.0f;
        *reinterpret_cast<v4f*>(p.out + (size_t)(h0 + h) * D + c) = r;
        if (p.lse && c == 0)
            p.lse[h0 + h] = Ls > 0.0f ? (M + __log2f(Ls)) * 0.69314718055994530942f : kNegInf;
        return;
    }

    // general path: (m, l) of every split first, then o of the non-empty ones
    for (int h = w; h < nh; h += NW) {
        float M = kNegInf;
        for (int s = lane; s < p.S; s += 64)
            M = fmaxf(M, ld_dev2(&p.part_ml[base + (size_t)s * G + h]).x);
        M = wave_max(M);
        float Lsum = 0.0f;
        int cnt = 0;
        for (int s0 = 0; s0 < p.S; s0 += 64) {
            const int s = s0 + lane;
            float wgt = 0.0f, l = 0.0f;
            if (s < p.S) {
                const float2 ml = ld_dev2(&p.part_ml[base + (size_t)s * G + h]);
                if (ml.x != kNegInf && ml.y > 0.0f) {
                    wgt = __builtin_amdgcn_exp2f(ml.x - M);
                    l = ml.y;
                }
            }
            Lsum = fmaf(wgt, l, Lsum);
            const unsigned long long ball = __ballot(wgt > 0.0f);
            const int pos = __popcll(ball & ((1ull << lane) - 1ull));
            if (wgt > 0.0f) {
                sh.u.fin.wgt[h][cnt + pos] = wgt;
                sh.u.fin.idx[h][cnt + pos] = (uint16_t)s;
            }
            cnt += __popcll(ball);
        }
        Lsum = wave_sum(Lsum);
        if (lane == 0) {
            sh.u.fin.M[h] = M;
            sh.u.fin.Lsum[h] = Lsum;
            sh.u.fin.cnt[h] = cnt;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nh * D; e += NW * 64) {
        const int h = e / D, c = e % D;
        const int n = sh.u.fin.cnt[h];
        float acc = 0.0f;
        for (int k0 = 0; k0 < n; k0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = sh.u.fin.idx[h][min(k0 + u, n - 1)];
                v[u] = ld_dev(&p.part_o[(base + (size_t)s * G + h) * D + c]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (k0 + u < n) acc = fmaf(sh.u.fin.wgt[h][k0 + u], v[u], acc);
        }
        const float L = sh.u.fin.Lsum[h];
        p.out[(size_t)(h0 + h) * D + c] = L > 0.0f ? acc / L : 0.0f;
        if (p.lse && c == 0)
            p.lse[h0 + h] =
                L > 0.0f ? (sh.u.fin.M[h] + __log2f(L)) * 0.69314718055994530942f : kNegInf;
    }
}

#if FFD_PART == 0
__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}
#endif

// ------------------------------------------------------------------------------------------
// App. A quantizer, 16 levels, of key block j of slice bg: one thread per channel c (a
// work-group of 128 threads; neighbouring channels share a byte).
// ------------------------------------------------------------------------------------------
template <int T, bool BF16>
__device__ __forceinline__ void quantize_block(QuantParams p, int bg, int j, int c)
{
    const size_t row0 = (size_t)bg * p.cap + (size_t)j * T;
    float x[T];
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if constexpr (BF16) {
            const unsigned short bits =
                static_cast<const unsigned short*>(p.K)[(row0 + t) * D + c];
            x[t] = as_f((int)((u32)bits << 16));
        } else {
            x[t] = static_cast<const float*>(p.K)[(row0 + t) * D + c];
        }
        amax = fmaxf(amax, fabsf(x[t]));
    }
    float s = 0.0f, inv = 0.0f;
    if (amax > 0.0f) {
        s = __fdiv_rn(amax, 7.5f);
        inv = __fdiv_rn(7.5f, amax);
    }
    p.scales[((size_t)bg * (p.cap / T) + j) * D + c] = scale_bits(s);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        int u = 8;
        if (amax > 0.0f) {
            u = (int)floorf(__fmul_rn(x[t], inv)) + 8;
            u = min(max(u, 0), 15);
        }
        const int partner = __shfl_xor(u, 1);
        if ((c & 1) == 0) p.Kq[(row0 + t) * (D / 2) + c / 2] = (uint8_t)(u | (partner << 4));
    }
}

template <int T, bool BF16>
__global__ __launch_bounds__(256) void quantize_kernel(QuantParams p)
{
    __shared__ float part[16][D];
    __shared__ float inv_s[D];
    quantize_block_wg<T, BF16>(p.K, p.Kq, p.scales, p.cap, blockIdx.y, p.j_first + blockIdx.x, part,
                               inv_s);
}

// One decode-loop step of the cache, in one launch.  One work-group per sequence b; thread
// (gi, c) handles channel c of kv heads g = gi, gi + nh, ... (nh = blockDim.x / d): the new key and
// value rows go to position seq_lens[b], and the key block they complete, if any, is quantized
// (this thread wrote the block's last key of its channel; the other rows are older).  Every thread
// reads the length before the barrier and thread 0 advances it after, so no thread of the launch
// sees the advanced value.
constexpr int kAppendHeads = 4;  // kv heads handled side by side by one work-group (a column
                                 // of T keys per thread stays in registers at 512 threads)
template <int T, bool BF16>
__global__ __launch_bounds__(kAppendHeads * 128) void append_kernel(AppendParams a)
{
    const int b = blockIdx.x;
    const int c = threadIdx.x % D;
    const int nh = blockDim.x / D;
    const int pos = a.seq_lens[b];
    const bool ok = pos >= 0 && pos < a.cap;  // uniform over the work-group
    if (ok) {
        // the kv head is uniform over a wave (D = 2 waves per head): held in a scalar register,
        // the block's row addresses stay scalar
#pragma unroll 1
        for (int g = __builtin_amdgcn_readfirstlane((int)threadIdx.x / D); g < a.Hkv; g += nh) {
            const int bg = b * a.Hkv + g;
            const size_t src = (size_t)bg * D + c;
            const size_t dst = ((size_t)bg * a.cap + pos) * D + c;
            if constexpr (BF16) {
                static_cast<unsigned short*>(a.K)[dst] =
                    static_cast<const unsigned short*>(a.k_new)[src];
                static_cast<unsigned short*>(a.V)[dst] =
                    static_cast<const unsigned short*>(a.v_new)[src];
            } else {
                static_cast<float*>(a.K)[dst] = static_cast<const float*>(a.k_new)[src];
                static_cast<float*>(a.V)[dst] = static_cast<const float*>(a.v_new)[src];
            }
            if ((pos + 1) % T == 0) {
                QuantParams q{};
                q.K = a.K;
                q.Kq = a.Kq;
                q.scales = a.scales;
                q.cap = a.cap;
                q.T = T;
                quantize_block<T, BF16>(q, bg, pos / T, c);
            }
        }
    }
    __syncthreads();
    if (ok && threadIdx.x == 0) a.seq_lens[b] = pos + 1;
}

// ------------------------------------------------------------------------------------------
// Residual storage form of the keys (Sec. 3.1, Fig. 2): App. A thumbnail at BITS bits and the
// symmetric 8-bit code of the residual, per (block, channel); one thread per channel, the same
// fp32 operations as the oracle: xh = RN((u - half) s), r = RN(x - xh), s_r = RN(max|r| / 127),
// r_q = clamp(rint(RN(r * RN(127 / max|r|))), -127, 127).
// ------------------------------------------------------------------------------------------
template <int T, int BITS>
__global__ __launch_bounds__(256) void quantize_res_kernel(QuantParams p)
{
    // one 256-thread work-group per (block, b g): thread (rg, cg) = (t / 16, t % 16) holds
    // channels 8 cg .. 8 cg + 7 of rows rg, rg + 16, ... (16-byte loads); the per-channel maxima
    // of the keys and then of the residuals meet in LDS; an all-zero channel gets reciprocal 0,
    // which gives the same codes (the middle one) as the per-channel form
    constexpr float half = (float)((1 << BITS) - 1) * 0.5f;
    constexpr int top = (1 << BITS) - 1;
    constexpr int RPT = T / 16;  // rows per thread
    __shared__ float part[16][D];
    __shared__ float sc_s[D], sc_inv[D];
    const int t = threadIdx.x, rg = t >> 4, cg = t & 15;
    const int j = p.j_first + blockIdx.x;
    const int bg = blockIdx.y;
    const size_t row0 = (size_t)bg * p.cap + (size_t)j * T;
    const size_t srow = ((size_t)bg * (p.cap / T) + j) * D;
    float x[RPT][8];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            static_cast<const unsigned short*>(p.K) + (row0 + rg + 16 * r) * D + cg * 8);
        x[r][0] = bf16_lo(v.x); x[r][1] = bf16_hi(v.x);
        x[r][2] = bf16_lo(v.y); x[r][3] = bf16_hi(v.y);
        x[r][4] = bf16_lo(v.z); x[r][5] = bf16_hi(v.z);
        x[r][6] = bf16_lo(v.w); x[r][7] = bf16_hi(v.w);
    }
    // 1. the thumbnail scale of each channel
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float am = 0.0f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) am = fmaxf(am, fabsf(x[r][i]));
        part[rg][cg * 8 + i] = am;
    }
    __syncthreads();
    if (t < D) {
        float amax = 0.0f;
#pragma unroll
        for (int g = 0; g < 16; ++g) amax = fmaxf(amax, part[g][t]);
        float sv = 0.0f, inv = 0.0f;
        if (amax > 0.0f) {
            sv = __fdiv_rn(amax, half);
            inv = __fdiv_rn(half, amax);
        }
        // the codes use the binary32 reciprocal; the residual is taken against the stored
        // (bf16) scale, which Dequant reads
        const uint16_t sb = scale_bits(sv);
        p.scales[srow + t] = sb;
        sc_s[t] = scale_value(sb);
        sc_inv[t] = inv;
    }
    __syncthreads();
    // 2. codes, the residual in place of x, and the residual scale of each channel
    int u[RPT][8];
    {
        float sv[8], iv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sv[i] = sc_s[cg * 8 + i];
            iv[i] = sc_inv[cg * 8 + i];
        }
        float rm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) rm[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int v = min(max((int)floorf(__fmul_rn(x[r][i], iv[i])) + (1 << (BITS - 1)), 0),
                                  top);
                u[r][i] = v;
                x[r][i] = __fsub_rn(x[r][i], __fmul_rn((float)v - half, sv[i]));
                rm[i] = fmaxf(rm[i], fabsf(x[r][i]));
            }
        // part[] was last read before the previous barrier
#pragma unroll
        for (int i = 0; i < 8; ++i) part[rg][cg * 8 + i] = rm[i];
    }
    __syncthreads();
    if (t < D) {
        float ramax = 0.0f;
#pragma unroll
        for (int g = 0; g < 16; ++g) ramax = fmaxf(ramax, part[g][t]);
        float s_r = 0.0f, inv_r = 0.0f;
        if (ramax > 0.0f) {
            s_r = __fdiv_rn(ramax, 127.0f);
            inv_r = __fdiv_rn(127.0f, ramax);
        }
        p.res_scales[srow + t] = s_r;
        sc_inv[t] = inv_r;
    }
    __syncthreads();
    // 3. the 8-bit residual codes (8 bytes per row) and the packed thumbnail codes (channel i of
    // the eight at bit i * BITS of a 4- or 2-byte word)
    float ir[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ir[i] = sc_inv[cg * 8 + i];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const size_t row = row0 + rg + 16 * r;
        u32 rq_lo = 0, rq_hi = 0, code = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float rq = fminf(fmaxf(rintf(__fmul_rn(x[r][i], ir[i])), -127.0f), 127.0f);
            const u32 byte = (u32)(uint8_t)(int8_t)(int)rq;
            if (i < 4) rq_lo |= byte << (8 * i);
            else rq_hi |= byte << (8 * (i - 4));
            code |= (u32)u[r][i] << (i * BITS);
        }
        *reinterpret_cast<uint2*>(p.Kr + row * D + cg * 8) = make_uint2(rq_lo, rq_hi);
        if constexpr (BITS == 4)
            *reinterpret_cast<u32*>(p.Kq + row * (D / 2) + cg * 4) = code;
        else
            *reinterpret_cast<uint16_t*>(p.Kq + row * (D / 4) + cg * 2) = (uint16_t)code;
    }
}

// The streaming-policy kernels (p.stream, set for long splits) exist for 16-bit inputs only.
template <int T, int G>
hipError_t launch_stream_t(const DecodeParams& p, bool sparse, hipStream_t stream)
{
    const dim3 grid(p.B * p.Hkv * p.NSUB * p.S), block(kWaves * 64);
    if (sparse)
        hipLaunchKernelGGL((decode_kernel<T, G, true, true, 4, false, true>), grid, block, 0,
                           stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<T, G, true, false, 4, false, true>), grid, block, 0,
                           stream, p);
    return hipGetLastError();
}

template <int T, int G, bool BF16>
hipError_t launch_decode_t(const DecodeParams& p, bool sparse, hipStream_t stream)
{
    const dim3 grid(p.B * p.Hkv * p.NSUB * p.S), block(kWaves * 64);
    if (BF16 && p.stream) {
        return launch_decode_stream(p, sparse, stream);  // the other half of this file
    } else if (sparse) {
        hipLaunchKernelGGL((decode_kernel<T, G, BF16, true, 4, false, false>), grid, block, 0,
                           stream, p);
    } else {
        hipLaunchKernelGGL((decode_kernel<T, G, BF16, false, 4, false, false>), grid, block, 0,
                           stream, p);
    }
    return hipGetLastError();
}

template <int T, bool BF16>
hipError_t launch_decode_g(const DecodeParams& p, bool sparse, hipStream_t stream)
{
    switch (p.GP) {
    case 1: return launch_decode_t<T, 1, BF16>(p, sparse, stream);
    case 2: return launch_decode_t<T, 2, BF16>(p, sparse, stream);
    case 4: return launch_decode_t<T, 4, BF16>(p, sparse, stream);
    case 8: return launch_decode_t<T, 8, BF16>(p, sparse, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int T, int BITS, bool STREAM>
hipError_t launch_res_s(const DecodeParams& p, hipStream_t stream)
{
    const dim3 grid(p.B * p.Hkv * p.NSUB * p.S), block(kResWaves * 64);
    switch (p.GP) {
    case 1: hipLaunchKernelGGL((decode_kernel<T, 1, true, true, BITS, true, STREAM>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, 2, true, true, BITS, true, STREAM>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, 4, true, true, BITS, true, STREAM>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<T, 8, true, true, BITS, true, STREAM>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
template <int T, int BITS>
hipError_t launch_res_g(const DecodeParams& p, hipStream_t stream)
{
    return p.stream ? launch_decode_res_stream(p, BITS, stream) : launch_res_s<T, BITS, false>(p, stream);
}

// ------------------------------------------------------------------------------------------
// Selection comparators (Sec. 4.5 Table 3; Sec. 5.1 Fig. 6; Sec. 5.2 Fig. 5): per-block scores
// written out, then one rule per (b, query head) row.  They are unfused on purpose: the rules
// other than top-delta need every block's score of a row before they can decide.
// ------------------------------------------------------------------------------------------

// Min and max of every channel over a key block's T tokens (one thread per channel), stored in
// K's dtype (the min and max of bf16 values are bf16 values).
template <int T, bool BF16>
__global__ __launch_bounds__(128) void bounds_kernel(BoundsParams p)
{
    const int j = p.j_first + blockIdx.x;
    const int bg = blockIdx.y;
    const int c = threadIdx.x;
    const size_t row0 = (size_t)bg * p.cap + (size_t)j * T;
    const size_t o = ((size_t)bg * (p.cap / T) + j) * D + c;
    if constexpr (BF16) {
        const unsigned short* K = static_cast<const unsigned short*>(p.K);
        unsigned short bmn = K[row0 * D + c], bmx = bmn;
        float mn = as_f((int)((u32)bmn << 16)), mx = mn;
        for (int t = 1; t < T; ++t) {
            const unsigned short b = K[(row0 + t) * D + c];
            const float x = as_f((int)((u32)b << 16));
            if (x < mn) { mn = x; bmn = b; }
            if (x > mx) { mx = x; bmx = b; }
        }
        static_cast<unsigned short*>(p.kmin)[o] = bmn;
        static_cast<unsigned short*>(p.kmax)[o] = bmx;
    } else {
        const float* K = static_cast<const float*>(p.K);
        float mn = K[row0 * D + c], mx = mn;
        for (int t = 1; t < T; ++t) {
            const float x = K[(row0 + t) * D + c];
            mn = fminf(mn, x);
            mx = fmaxf(mx, x);
        }
        static_cast<float*>(p.kmin)[o] = mn;
        static_cast<float*>(p.kmax)[o] = mx;
    }
}

__device__ __forceinline__ float elem(const void* base, size_t i, bool bf16)
{
    return bf16 ? as_f((int)((u32) static_cast<const unsigned short*>(base)[i] << 16))
                : static_cast<const float*>(base)[i];
}

// Block scores of the full blocks, one work-group (4 waves) per (b, kv head, 16 blocks); wave w
// takes blocks w, w + 4, ... of the chunk.  KIND 0: the scan estimate shat of Alg. 1 (the decode
// kernel's integer scan); KIND 1: sum_c max(q_c mn_c, q_c mx_c) / sqrt(d) (a Quest-style upper
// bound; fp32, lane-parallel over channels, fixed reduction order); KIND 2: the exact largest
// q.k / sqrt(d) of the block (bf16 or fp32 MFMA over its 16-token tiles).
template <int T, int G, bool BF16, int KIND>
__global__ __launch_bounds__(kWaves * 64) void score_kernel(ScoreParams p)
{
    constexpr int kChunk = 16;
    __shared__ WaveScratch<G> wsh[kWaves];
    __shared__ float4 qs[G * D * (BF16 ? 2 : 4) / 16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int col = lane & 15, kg = lane >> 4;
    // blockIdx.y = work unit: G query heads (the kernel's width) of one (b, kv head), the last
    // ones padding when the group is narrower (as in decode_kernel)
    const int unit = blockIdx.y;
    const int bg = unit / p.NSUB, sub = unit % p.NSUB;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int h0 = b * p.Hq + g * p.G + sub * G;
    const int nh = min(G, p.G - sub * G);  // real heads of the unit
    const int j0 = blockIdx.x * kChunk;
    const int j1 = min(p.n_full, j0 + kChunk);
    const size_t esz = BF16 ? 2 : 4;
    if constexpr (KIND == 2) {
        constexpr int kRow16 = D * (BF16 ? 2 : 4) / 16;
        constexpr int kQ16 = G * kRow16;
        const float4* src =
            reinterpret_cast<const float4*>(static_cast<const char*>(p.q) + (size_t)h0 * D * esz);
        for (int i = threadIdx.x; i < kQ16; i += kWaves * 64)
            qs[i] = i < nh * kRow16 ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        __syncthreads();
    }
    if constexpr (KIND == 0) {
        constexpr int HPL = (G + 3) / 4;
        float qw[HPL][8];
#pragma unroll
        for (int k = 0; k < HPL; ++k) {
            const int h = min((G >= 4) ? (kg + 4 * k) : (kg % G), nh - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                qw[k][i] = elem(p.q, (size_t)(h0 + h) * D + col * 8 + i, BF16);
        }
        const uint8_t* kq_bg = p.Kq + (size_t)bg * p.cap * (D / 2);
        const uint16_t* sc_bg = p.scales + (size_t)bg * (p.cap / T) * D;
        for (int j = j0 + w; j < j1; j += kWaves) {
            ScanRegs<T, 4> r;
            scan_load<T, 4, false>(r, kq_bg + (size_t)j * T * (D / 2), sc_bg + (size_t)j * D, lane);
            const float shat = scan_compute<T, G, 4>(r, qw, p.kappa, wsh[w], lane);
            if (lane < nh) p.scores[(size_t)(h0 + lane) * p.n_full + j] = shat;
        }
    } else if constexpr (KIND == 1) {
        const size_t mrow = (size_t)bg * (p.cap / T);
        for (int j = j0 + w; j < j1; j += kWaves) {
            const size_t mo = (mrow + j) * D;
            const float mn0 = elem(p.kmin, mo + 2 * lane, BF16);
            const float mn1 = elem(p.kmin, mo + 2 * lane + 1, BF16);
            const float mx0 = elem(p.kmax, mo + 2 * lane, BF16);
            const float mx1 = elem(p.kmax, mo + 2 * lane + 1, BF16);
            for (int h = 0; h < nh; ++h) {
                const float q0 = elem(p.q, (size_t)(h0 + h) * D + 2 * lane, BF16);
                const float q1 = elem(p.q, (size_t)(h0 + h) * D + 2 * lane + 1, BF16);
                float x = fmaxf(__fmul_rn(q0, mn0), __fmul_rn(q0, mx0)) +
                          fmaxf(__fmul_rn(q1, mn1), __fmul_rn(q1, mx1));
                x = wave_sum(x);
                if (lane == 0) p.scores[(size_t)(h0 + h) * p.n_full + j] = x * p.inv_sqrt_d;
            }
        }
    } else {
        const void* qrow = reinterpret_cast<const char*>(qs) + (size_t)(col % G) * D * esz;
        v8bf qv[4];
        if constexpr (BF16) {
            const __bf16* qb = static_cast<const __bf16*>(qrow);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qv[ks] = *reinterpret_cast<const v8bf*>(qb + ks * 32 + kg * 8);
        }
        const char* Kbg = static_cast<const char*>(p.K) + (size_t)bg * p.cap * D * esz;
        for (int j = j0 + w; j < j1; j += kWaves) {
            float m = kNegInf;
            for (int t = 0; t < T / 16; ++t) {
                TileRegs<BF16> r;
                const int t0 = j * T + 16 * t;
                if constexpr (BF16) {
                    const __bf16* Kp = reinterpret_cast<const __bf16*>(Kbg);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        r.k[ks] = *reinterpret_cast<const uint4*>(Kp + (size_t)(t0 + col) * D +
                                                                  ks * 32 + kg * 8);
                } else {
                    const float* Kp = reinterpret_cast<const float*>(Kbg);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        r.k[i] = *reinterpret_cast<const float4*>(Kp + (size_t)(t0 + col) * D +
                                                                  kg * 32 + i * 4);
                }
                const v4f acc = tile_scores<BF16>(r, qrow, qv, lane);
                m = fmaxf(m, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
            }
            m = fmax32(fmax16(m));  // over the four token groups: column col = head col % G
            if (kg == 0 && col < nh) p.scores[(size_t)(h0 + col) * p.n_full + j] = m * p.inv_sqrt_d;
        }
    }
}

// Order-preserving map of a float's bits to an unsigned integer, and its inverse.
__device__ __forceinline__ u32 f_ord(float x)
{
    const u32 u = (u32)as_i(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f_unord(u32 o)
{
    return as_f((int)((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o));
}

// One selection rule over a row of block scores (one work-group of 256 threads per (b, query
// head)).  RULE 0 top-delta: theta = RN(mtilde - delta), mtilde the given pseudo-max or
// max(s_0, s_{nf-1}); keep s_j >= theta.  RULE 1 top-k and RULE 2 top-p keep a prefix of the row
// ranked by descending score, ties to the lower index: top-k the first k, top-p the shortest
// prefix whose mass exp(s - s_max) reaches p of the row's total.  Neither needs the ranking
// itself, only the prefix's last key: a radix select over the keys ~ord(s_j) (ascending key =
// descending score) finds it in four 8-bit passes, each a histogram in LDS of the weights of the
// keys that share the bits found so far -- weight 1 for top-k, the mass as an integer multiple of
// 2^-40 for top-p (integer sums: exact and independent of the order of the atomics).  The prefix
// is then every key below the last one plus, of the keys equal to it, the first ones in index
// order.  Every rule keeps block 0, the last full block and a partial tail.
constexpr float kMassScale = 1099511627776.0f;  // 2^40

// ceil(t * p) for 0 < p <= 1, exactly: p = m 2^-sh with a 24-bit integer m, the 128-bit product
// t m shifted right by sh, rounding up (integer arithmetic only)
__device__ __forceinline__ unsigned long long ceil_mul(unsigned long long t, float p)
{
    const u32 bits = (u32)as_i(p);
    const int e = (int)((bits >> 23) & 0xFFu);
    const unsigned long long m = (bits & 0x7FFFFFu) | (e != 0 ? 0x800000u : 0u);
    const int sh = 150 - (e != 0 ? e : 1);  // >= 23
    const unsigned long long lo = t * m, hi = __umul64hi(t, m);
    unsigned long long q, rem;
    if (sh < 64) {
        q = (lo >> sh) | (hi << (64 - sh));
        rem = lo & ((1ull << sh) - 1ull);
    } else if (sh < 128) {
        q = hi >> (sh - 64);
        rem = lo | (hi & ((1ull << (sh - 64)) - 1ull));
    } else {
        q = 0ull;
        rem = lo | hi;
    }
    return q + (rem != 0ull ? 1ull : 0ull);
}

template <int RULE>
__global__ __launch_bounds__(256) void select_kernel(SelectParams p)
{
    extern __shared__ u32 keys[];  // n_full keys, then n_blocks keep flags
    __shared__ unsigned long long hist[256];
    __shared__ unsigned long long s_total, s_above;
    __shared__ u32 s_min, s_prefix;
    __shared__ int s_ties[4];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int nf = p.n_full, nb = p.n_blocks;
    const float* s = p.scores + (size_t)row * nf;
    uint8_t* keep = p.keep + (size_t)row * nb;
    auto forced = [&](int j) { return j == 0 || j >= nf - 1; };
    if (RULE == 0 || nf == 0) {
        float theta = kNegInf;
        if (nf > 0) {
            const float mt = p.pseudo_max ? p.pseudo_max[row] : fmaxf(s[0], s[nf - 1]);
            theta = __fsub_rn(mt, p.param);
        }
        for (int j = tid; j < nb; j += 256) {
            bool k = forced(j);  // every j >= nf - 1 is forced, so s[j] is read only for j < nf
            if (!k && RULE == 0) k = s[j] >= theta;
            keep[j] = k ? 1 : 0;
        }
        return;
    }
    uint8_t* flag = reinterpret_cast<uint8_t*>(keys + nf);
    if (tid == 0) {
        s_min = 0xFFFFFFFFu;
        s_total = 0ull;
        s_above = 0ull;
        s_prefix = 0u;
    }
    __syncthreads();
    u32 kmin = 0xFFFFFFFFu;
    for (int i = tid; i < nf; i += 256) {
        const u32 k = ~f_ord(s[i]);
        keys[i] = k;
        kmin = min(kmin, k);
    }
    for (int j = tid; j < nb; j += 256) flag[j] = forced(j) ? 1 : 0;
    float smax = 0.0f;
    if constexpr (RULE == 2) {
        atomicMin(&s_min, kmin);
        __syncthreads();
        smax = f_unord(~s_min);
    }
    // weight of a key: 1, or its mass exp(s - s_max) in units of 2^-40 (truncated)
    auto weight = [&](u32 k) -> unsigned long long {
        if constexpr (RULE == 1) {
            return 1ull;
        } else {
            const float x = f_unord(~k);
            const float m = (x == smax) ? 1.0f
                                        : __builtin_amdgcn_exp2f((x - smax) * 1.4426950408889634f);
            return (unsigned long long)(m * kMassScale);
        }
    };
    // target weight of the prefix; all = every full block is kept
    unsigned long long target;
    bool all = false, none = false;
    if constexpr (RULE == 1) {
        const float kk = p.param;
        none = !(kk >= 1.0f);
        all = kk >= (float)nf;
        target = none || all ? 0ull : (unsigned long long)(u32)kk;
    } else {
        unsigned long long tot = 0ull;
        for (int i = tid; i < nf; i += 256) tot += weight(keys[i]);
        atomicAdd(&s_total, tot);
        __syncthreads();
        // the shortest prefix with mass >= p of the total: weight >= ceil(p total)
        const float pp = p.param;
        all = !(pp <= 1.0f);  // p above 1 (or NaN): every block
        target = all ? 0ull : (pp > 0.0f ? ceil_mul(s_total, pp) : 1ull);
        if (target == 0ull && !all) target = 1ull;  // p <= 0 or tiny: the top block
    }
    if (!none) {
        if (all) {
            for (int i = tid; i < nf; i += 256) flag[i] = 1;
        } else {
            // radix select: after the pass at bit sh, s_prefix holds the last key's bits from sh
            // up and s_above the weight of every key below the keys with those bits
            for (int sh = 24; sh >= 0; sh -= 8) {
                hist[tid] = 0ull;
                __syncthreads();
                const u32 pre = s_prefix;
                const u32 hi_mask = sh == 24 ? 0u : (0xFFFFFFFFu << (sh + 8));
                for (int i = tid; i < nf; i += 256) {
                    const u32 k = keys[i];
                    if (((k ^ pre) & hi_mask) == 0u)
                        atomicAdd(&hist[(k >> sh) & 255u], weight(k));
                }
                __syncthreads();
                if (w == 0) {
                    // lane l holds bins 4l .. 4l + 3; inclusive scan over the lanes
                    unsigned long long b4[4], loc = 0ull;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        b4[u] = hist[4 * lane + u];
                        loc += b4[u];
                    }
                    unsigned long long inc = loc;
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const unsigned long long o = __shfl_up(inc, d);
                        if (lane >= d) inc += o;
                    }
                    const unsigned long long above = s_above;
                    // first bin whose inclusive weight reaches the target
                    const bool hit = above + inc >= target;
                    const unsigned long long ball = __ballot(hit);
                    const int L0 = (int)__builtin_ctzll(ball);  // exists: the range holds the target
                    if (lane == L0) {
                        unsigned long long run = above + inc - loc;  // weight below bin 4 L0
                        int bin = 4 * L0;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            if (run + b4[u] >= target) break;
                            run += b4[u];
                            ++bin;
                        }
                        s_prefix = pre | ((u32)bin << sh);
                        s_above = run;
                    }
                }
                __syncthreads();
            }
            // keys below the last key v: kept; keys equal to v: the first c in index order
            const u32 v = s_prefix;
            const unsigned long long rest = target - s_above;
            const unsigned long long wv = weight(v);
            const int c = (int)((rest + wv - 1ull) / wv);
            int taken = 0;  // ties already met in earlier chunks
            for (int base = 0; base < nf; base += 256) {
                const int i = base + tid;
                const u32 k = i < nf ? keys[i] : 0xFFFFFFFFu;
                if (k < v) flag[i] = 1;
                const bool tie = i < nf && k == v;
                const unsigned long long ball = __ballot(tie);
                if (lane == 0) s_ties[w] = (int)__popcll(ball);
                __syncthreads();
                int before = taken;
                for (int u = 0; u < w; ++u) before += s_ties[u];
                const int rank = before + (int)__popcll(ball & ((1ull << lane) - 1ull));
                if (tie && rank < c) flag[i] = 1;
                taken += s_ties[0] + s_ties[1] + s_ties[2] + s_ties[3];
                __syncthreads();
            }
        }
    }
    __syncthreads();
    for (int j = tid; j < nb; j += 256) keep[j] = flag[j];
}

}  // namespace

#if FFD_PART == 0
hipError_t launch_decode(const DecodeParams& p, bool bf16, bool sparse, hipStream_t stream)
{
    if (p.T == 64)
        return bf16 ? launch_decode_g<64, true>(p, sparse, stream)
                    : launch_decode_g<64, false>(p, sparse, stream);
    if (p.T == 128)
        return bf16 ? launch_decode_g<128, true>(p, sparse, stream)
                    : launch_decode_g<128, false>(p, sparse, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_res(const DecodeParams& p, int bits, hipStream_t stream)
{
    if (p.T == 64) return bits == 2 ? launch_res_g<64, 2>(p, stream) : launch_res_g<64, 4>(p, stream);
    if (p.T == 128)
        return bits == 2 ? launch_res_g<128, 2>(p, stream) : launch_res_g<128, 4>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_res(const QuantParams& p, int bits, hipStream_t stream)
{
    if (p.n_blocks <= 0) return hipSuccess;
    const dim3 grid(p.n_blocks, p.B * p.Hkv), block(256);
    if (p.T == 64) {
        if (bits == 2) hipLaunchKernelGGL((quantize_res_kernel<64, 2>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((quantize_res_kernel<64, 4>), grid, block, 0, stream, p);
    } else if (p.T == 128) {
        if (bits == 2) hipLaunchKernelGGL((quantize_res_kernel<128, 2>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((quantize_res_kernel<128, 4>), grid, block, 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_zero_counters(uint32_t* counters, int n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, counters, n);
    return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, bool bf16, hipStream_t stream)
{
    if (p.B <= 0) return hipSuccess;
    const dim3 grid(p.B), block(D * (p.Hkv < kAppendHeads ? p.Hkv : kAppendHeads));
    if (p.T == 64) {
        if (bf16) hipLaunchKernelGGL((append_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((append_kernel<64, false>), grid, block, 0, stream, p);
    } else if (p.T == 128) {
        if (bf16) hipLaunchKernelGGL((append_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((append_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, bool bf16, hipStream_t stream)
{
    if (p.n_blocks <= 0) return hipSuccess;
    const dim3 grid(p.n_blocks, p.B * p.Hkv), block(256);
    if (p.T == 64) {
        if (bf16) hipLaunchKernelGGL((quantize_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((quantize_kernel<64, false>), grid, block, 0, stream, p);
    } else if (p.T == 128) {
        if (bf16) hipLaunchKernelGGL((quantize_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((quantize_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bounds(const BoundsParams& p, bool bf16, hipStream_t stream)
{
    if (p.n_blocks <= 0) return hipSuccess;
    const dim3 grid(p.n_blocks, p.B * p.Hkv), block(D);
    if (p.T == 64) {
        if (bf16) hipLaunchKernelGGL((bounds_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bounds_kernel<64, false>), grid, block, 0, stream, p);
    } else if (p.T == 128) {
        if (bf16) hipLaunchKernelGGL((bounds_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bounds_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

namespace {
template <int T, int G, bool BF16>
void launch_scores_k(const ScoreParams& p, int kind, hipStream_t stream)
{
    const dim3 grid((p.n_full + 15) / 16, p.B * p.Hkv * p.NSUB), block(kWaves * 64);
    if (kind == 0) hipLaunchKernelGGL((score_kernel<T, G, BF16, 0>), grid, block, 0, stream, p);
    else if (kind == 1) hipLaunchKernelGGL((score_kernel<T, G, BF16, 1>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((score_kernel<T, G, BF16, 2>), grid, block, 0, stream, p);
}
template <int T, bool BF16>
hipError_t launch_scores_g(const ScoreParams& p, int kind, hipStream_t stream)
{
    switch (p.GP) {
    case 1: launch_scores_k<T, 1, BF16>(p, kind, stream); break;
    case 2: launch_scores_k<T, 2, BF16>(p, kind, stream); break;
    case 4: launch_scores_k<T, 4, BF16>(p, kind, stream); break;
    case 8: launch_scores_k<T, 8, BF16>(p, kind, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_scores(const ScoreParams& p, int kind, bool bf16, hipStream_t stream)
{
    if (p.n_full <= 0 || p.B <= 0) return hipSuccess;
    if (p.T == 64) return bf16 ? launch_scores_g<64, true>(p, kind, stream)
                               : launch_scores_g<64, false>(p, kind, stream);
    if (p.T == 128) return bf16 ? launch_scores_g<128, true>(p, kind, stream)
                                : launch_scores_g<128, false>(p, kind, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectParams& p, int rule, hipStream_t stream)
{
    if (p.rows <= 0) return hipSuccess;
    const size_t dyn = rule == 0 ? 0 : (size_t)p.n_full * 4 + (size_t)((p.n_blocks + 15) & ~15);
    if (rule == 0)
        hipLaunchKernelGGL(select_kernel<0>, dim3(p.rows), dim3(256), dyn, stream, p);
    else if (rule == 1)
        hipLaunchKernelGGL(select_kernel<1>, dim3(p.rows), dim3(256), dyn, stream, p);
    else
        hipLaunchKernelGGL(select_kernel<2>, dim3(p.rows), dim3(256), dyn, stream, p);
    return hipGetLastError();
}

#else  // FFD_PART == 1
hipError_t launch_decode_stream(const DecodeParams& p, bool sparse, hipStream_t stream)
{
    switch (p.T * 16 + p.GP) {
    case 64 * 16 + 1: return launch_stream_t<64, 1>(p, sparse, stream);
    case 64 * 16 + 2: return launch_stream_t<64, 2>(p, sparse, stream);
    case 64 * 16 + 4: return launch_stream_t<64, 4>(p, sparse, stream);
    case 64 * 16 + 8: return launch_stream_t<64, 8>(p, sparse, stream);
    case 128 * 16 + 1: return launch_stream_t<128, 1>(p, sparse, stream);
    case 128 * 16 + 2: return launch_stream_t<128, 2>(p, sparse, stream);
    case 128 * 16 + 4: return launch_stream_t<128, 4>(p, sparse, stream);
    case 128 * 16 + 8: return launch_stream_t<128, 8>(p, sparse, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_res_stream(const DecodeParams& p, int bits, hipStream_t stream)
{
    if (p.T == 64)
        return bits == 2 ? launch_res_s<64, 2, true>(p, stream) : launch_res_s<64, 4, true>(p, stream);
    if (p.T == 128)
        return bits == 2 ? launch_res_s<128, 2, true>(p, stream) : launch_res_s<128, 4, true>(p, stream);
    return hipErrorInvalidValue;
}
#endif

}  // namespace ffd
