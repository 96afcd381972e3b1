// ssq_device.h -- device building blocks of the quantized state update (gfx950).
//
// A state row is N = 128 entries.  LPR lanes of a wave64 cooperate on a row,
// each holding E = 128/LPR consecutive entries in registers, so a wave covers
// 64/LPR rows at once.  Cross-lane reductions over the LPR lanes of a row use
// DPP (quad_perm, row_half_mirror, row_mirror), never LDS.
//
// Evaluation order (identical in every kernel, so that the decode step, the
// scan and the state initialisation round the same way):
//   lambda  = fl32(exp_double(fl(dt*A))),  w = fl(dt*x)
//   hh_n    = fl(s*fl(c_n - z))                    the stored entry (z = 0: symmetric grid)
//   h'_n    = fma(lambda, hh_n, fl(w*B_n))         the fp32 recurrence on it
//   refit   (asymmetric) s' = fl(fl(mx-mn)/(2^b-1)), inv = fl(1/s'),
//           z' = -rne(mn*inv);  (symmetric) s' = fl(amax/(2^(b-1)-1))
//   code    = clamp(rne(h'*inv + z')), the product exact, ties to the even code
//
// The rounding uses the 1.5*2^23 trick: floats in [2^23, 2^24) are the
// integers, so fma(h, inv, 1.5*2^23 + z) is 1.5*2^23 + rne(h*inv + z) for the
// exact product, as long as 1.5*2^23 + z is exact (|z| < 2^21 here).  Rows
// with |z| >= 2^21 (a spread below ~2^-13 of the row's offset) take a slow
// path in double, where h*inv + z is exact by Sterbenz's lemma.  The clamped
// value's bit pattern minus that of 1.5*2^23 is the code itself, so packing
// needs no float-to-int conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssq_internal.h"

namespace ssq {

enum Format : int { FP32 = 0, INT8_SYM = 1, INT8_ASYM = 2, INT4_SYM = 3, INT4_ASYM = 4 };

template <int F> struct Traits;
template <> struct Traits<FP32> {
    static constexpr bool quant = false, asym = false;
    static constexpr int bits = 32, lo = 0, hi = 0;
};
template <> struct Traits<INT8_SYM> {
    static constexpr bool quant = true, asym = false;
    static constexpr int bits = 8, lo = -127, hi = 127;
};
template <> struct Traits<INT8_ASYM> {
    static constexpr bool quant = true, asym = true;
    static constexpr int bits = 8, lo = 0, hi = 255;
};
template <> struct Traits<INT4_SYM> {
    static constexpr bool quant = true, asym = false;
    static constexpr int bits = 4, lo = -7, hi = 7;
};
template <> struct Traits<INT4_ASYM> {
    static constexpr bool quant = true, asym = true;
    static constexpr int bits = 4, lo = 0, hi = 15;
};

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kSlowZero = 2097152.0f; // 2^21
constexpr float kFltMin = 1.17549435e-38f;

// ---------------------------------------------------------------------------
// DPP cross-lane helpers (every lane of a 16-lane DPP row is a valid source)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dppf(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// min / max of a lane and its DPP partner in one v_min_f32_dpp / v_max_f32_dpp.
// Written out because the compiler, to keep fminf's NaN rules, would move the
// partner with v_mov_b32_dpp and canonicalize it first (four instructions per
// step); the values here are finite.  The s_nop gives the two wait states a DPP
// read needs after a VALU write of its source.
#define SSQ_DPP_MINMAX(NAME, OP)                                                                  \
    template <int CTRL>                                                                           \
    __device__ __forceinline__ float NAME(float v)                                                \
    {                                                                                             \
        float r;                                                                                  \
        if constexpr (CTRL == 0xB1)                                                               \
            asm("s_nop 1\n\t" OP " %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"   \
                : "=v"(r) : "v"(v));                                                              \
        else if constexpr (CTRL == 0x4E)                                                          \
            asm("s_nop 1\n\t" OP " %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"   \
                : "=v"(r) : "v"(v));                                                              \
        else if constexpr (CTRL == 0x141)                                                         \
            asm("s_nop 1\n\t" OP " %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf"       \
                : "=v"(r) : "v"(v));                                                              \
        else                                                                                      \
            asm("s_nop 1\n\t" OP " %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf"            \
                : "=v"(r) : "v"(v));                                                              \
        return r;                                                                                 \
    }
SSQ_DPP_MINMAX(dpp_min, "v_min_f32_dpp")
SSQ_DPP_MINMAX(dpp_max, "v_max_f32_dpp")
#undef SSQ_DPP_MINMAX

// xor 1, xor 2 inside a quad; lane i <-> 7-i inside 8; lane i <-> 15-i inside 16
template <int LPR>
__device__ __forceinline__ float group_min(float v)
{
    if constexpr (LPR >= 2) v = dpp_min<0xB1>(v);
    if constexpr (LPR >= 4) v = dpp_min<0x4E>(v);
    if constexpr (LPR >= 8) v = dpp_min<0x141>(v);
    if constexpr (LPR >= 16) v = dpp_min<0x140>(v);
    return v;
}
template <int LPR>
__device__ __forceinline__ float group_max(float v)
{
    if constexpr (LPR >= 2) v = dpp_max<0xB1>(v);
    if constexpr (LPR >= 4) v = dpp_max<0x4E>(v);
    if constexpr (LPR >= 8) v = dpp_max<0x141>(v);
    if constexpr (LPR >= 16) v = dpp_max<0x140>(v);
    return v;
}
// every lane of the group ends with the same sum (each step adds a value and its mirror)
template <int LPR>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (LPR >= 2) v = v + dppf<0xB1>(v);
    if constexpr (LPR >= 4) v = v + dppf<0x4E>(v);
    if constexpr (LPR >= 8) v = v + dppf<0x141>(v);
    if constexpr (LPR >= 16) v = v + dppf<0x140>(v);
    return v;
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone).  Used at the end of a rarely
// taken block that loads, so that nothing from that block is still pending where the
// paths merge: otherwise the merge point itself must wait for every outstanding
// vector memory operation, which on this counter includes the ring's prefetches.
__device__ __forceinline__ void wait_vmem_all()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Orders the wave's LDS accesses on either side: writes of some lanes before reads of
// others (and reads before a later overwrite).  A wave executes its LDS instructions in
// order; this keeps the compiler from moving one across another when it cannot tell that
// the lanes' addresses overlap.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// lambda = exp(dt*A): the fp32 product, exponentiated in double, rounded once
__device__ __forceinline__ float decay(float dt, float A)
{
    const float e = dt * A;
    return (float)exp((double)e);
}

// ---------------------------------------------------------------------------
// codes <-> fp32 for one lane's E entries held in NW = E*bits/32 words
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ubyte_f(uint32_t w, int k)
{
    return (float)((w >> (8 * k)) & 0xFFu); // v_cvt_f32_ubyte{k}
}

// v_and_b32 the compiler cannot see through: with a visible mask it folds the
// shift-and-mask of each nibble into v_bfe_u32 + v_cvt_f32_ubyte0 (two ops);
// hidden, every byte converts with a single v_cvt_f32_ubyte{k}
__device__ __forceinline__ uint32_t and_0f(uint32_t w)
{
    uint32_t r;
    asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(r) : "v"(w));
    return r;
}

// c_n as float (sym: the signed code; asym: 0..2^b-1)
template <int F, int E>
__device__ __forceinline__ void unpack_codes(const uint32_t* w, float* c)
{
    if constexpr (F == INT8_ASYM) {
#pragma unroll
        for (int i = 0; i < E / 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) c[4 * i + k] = ubyte_f(w[i], k);
    } else if constexpr (F == INT8_SYM) {
#pragma unroll
        for (int i = 0; i < E / 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) c[4 * i + k] = (float)(int)(int8_t)(w[i] >> (8 * k));
    } else if constexpr (F == INT4_ASYM) {
#pragma unroll
        for (int i = 0; i < E / 8; ++i) {
            const uint32_t lo = and_0f(w[i]), hi = and_0f(w[i] >> 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[8 * i + 2 * k] = ubyte_f(lo, k);
                c[8 * i + 2 * k + 1] = ubyte_f(hi, k);
            }
        }
    } else if constexpr (F == INT4_SYM) {
        // two's complement nibble x becomes x + 8 after flipping its sign bit
#pragma unroll
        for (int i = 0; i < E / 8; ++i) {
            const uint32_t b = w[i] ^ 0x88888888u;
            const uint32_t lo = and_0f(b), hi = and_0f(b >> 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[8 * i + 2 * k] = ubyte_f(lo, k) - 8.0f;
                c[8 * i + 2 * k + 1] = ubyte_f(hi, k) - 8.0f;
            }
        }
    }
}

// byte 0 of four words -> one word (v_perm_b32: bytes 0-3 of the 2nd operand, 4-7 of the 1st)
__device__ __forceinline__ uint32_t gather_b0(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// f[e] = 1.5*2^23 + code: the low bits of its pattern are the code
template <int F, int E>
__device__ __forceinline__ void pack_codes(const float* f, uint32_t* w)
{
    if constexpr (F == INT8_ASYM || F == INT8_SYM) {
#pragma unroll
        for (int i = 0; i < E / 4; ++i)
            w[i] = gather_b0(__float_as_uint(f[4 * i]), __float_as_uint(f[4 * i + 1]),
                             __float_as_uint(f[4 * i + 2]), __float_as_uint(f[4 * i + 3]));
    } else {
#pragma unroll
        for (int i = 0; i < E / 8; ++i) {
            const uint32_t ev = gather_b0(__float_as_uint(f[8 * i]), __float_as_uint(f[8 * i + 2]),
                                          __float_as_uint(f[8 * i + 4]), __float_as_uint(f[8 * i + 6]));
            const uint32_t od = gather_b0(__float_as_uint(f[8 * i + 1]), __float_as_uint(f[8 * i + 3]),
                                          __float_as_uint(f[8 * i + 5]), __float_as_uint(f[8 * i + 7]));
            if constexpr (F == INT4_ASYM)
                w[i] = ev | (od << 4); // codes < 16: no carry between nibbles
            else
                w[i] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
        }
    }
}

// h = fma(a, h, c), one rounding, written back into the register that holds h: the same
// instruction as __builtin_fmaf.  For a value carried from one token to the next, the
// compiler picks the form that writes the addend's register (v_fmac) and then copies every
// result back, one move per entry and token.
__device__ __forceinline__ void fma_in_place(float a, float& h, float c)
{
    asm("v_fma_f32 %0, %1, %0, %2" : "+v"(h) : "v"(a), "v"(c));
}

// ---------------------------------------------------------------------------
// refit of one row from its statistics (every lane of the row computes it)
// ---------------------------------------------------------------------------
struct RowGrid {
    float s;     // stored scale
    float z;     // stored zero point (0 for symmetric)
    float inv;   // 1/s, or 0 for a degenerate row (all codes 0)
    float Mz;    // 1.5*2^23 + z on the fast path
    float Mr;    // 1.5*2^23 + the z the readout subtracts: f - Mr = c - z
    float zc;    // z used for coding (0 for a degenerate row)
    bool slow;   // |z| >= 2^21
};

template <int F>
__device__ __forceinline__ RowGrid refit(float mn, float mx, float amax)
{
    RowGrid g;
    g.slow = false;
    if constexpr (Traits<F>::asym) {
        constexpr float qmax = (float)Traits<F>::hi;
        const float range = mx - mn;
        const float s = range / qmax;
        if (!(s >= kFltMin)) {
            // the row is kept as the constant mn: s = |mn|, z = -sign(mn), codes 0
            g.s = fabsf(mn);
            g.z = -(mn > 0.0f ? 1.0f : (mn < 0.0f ? -1.0f : 0.0f)) + 0.0f; // a zero zero point is +0
            g.inv = 0.0f;
            g.zc = 0.0f;
            g.Mz = kMagic;      // every code 0 ...
            g.Mr = kMagic + g.z; // ... standing for s*(0 - z) = mn
        } else {
            const float inv = 1.0f / s;
            // the product of two floats is exact in double; rint rounds half to even
            const float z = -(float)rint((double)mn * (double)inv) + 0.0f; // +0, never -0
            g.s = s;
            g.z = z;
            g.inv = inv;
            g.zc = z;
            g.slow = fabsf(z) >= kSlowZero;
            g.Mz = kMagic + z;
            g.Mr = g.Mz; // inexact only when |z| >= 2^22, where f - Mr is within 2^-21 relative of c - z
        }
    } else {
        constexpr float qmax = (float)Traits<F>::hi;
        const float s = amax / qmax;
        g.z = 0.0f;
        g.zc = 0.0f;
        g.Mz = kMagic;
        g.Mr = kMagic;
        if (!(s >= kFltMin)) {
            g.s = 0.0f;
            g.inv = 0.0f;
        } else {
            g.s = s;
            g.inv = 1.0f / s;
        }
    }
    return g;
}

// f = 1.5*2^23 + clamp(rne(h*inv + z)) for E entries; `slow_any` is wave-uniform
template <int F, int E>
__device__ __forceinline__ void round_codes(const float* h, const RowGrid& g, bool slow_any, float* f)
{
    constexpr float flo = kMagic + (float)Traits<F>::lo;
    constexpr float fhi = kMagic + (float)Traits<F>::hi;
    if (!slow_any) {
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = __builtin_amdgcn_fmed3f(__builtin_fmaf(h[e], g.inv, g.Mz), flo, fhi);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float t;
            if (g.slow) {
                // h*inv + z is exact in double here: h*inv lies within Qa+1 of -z and |z| >= 2^21
                const double p = (double)h[e] * (double)g.inv + (double)g.zc;
                t = kMagic + (float)rint(p);
            } else {
                t = __builtin_fmaf(h[e], g.inv, g.Mz);
            }
            f[e] = __builtin_amdgcn_fmed3f(t, flo, fhi);
        }
    }
}

// ---------------------------------------------------------------------------
// stochastic rounding ("ssm-state-quantization" README, Findings 9): the code
// is floor(v + U) for the exact real v = h*inv + z and U uniform in [0, 1), on
// the grid round-to-nearest refits.  U = K/2^16: counter ctr takes the 16-bit
// piece k = ctr mod 4 (bits 16k .. 16k+15) of SplitMix64 (Steele, Lea and Flood,
// OOPSLA 2014) output number ctr/4 + 1 for the state's seed, i.e. of the state
// advanced ctr/4 + 1 times by the golden gamma and mixed.
// ---------------------------------------------------------------------------
constexpr uint64_t kGoldenGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix_mix(uint64_t x)
{
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

// f = 1.5*2^23 + clamp(floor(h*inv + z + U)) for E entries (E a multiple of 8) whose
// uniforms are counters ctr0 .. ctr0 + E - 1 (ctr0 a multiple of 4): one generator
// output per four entries.  Off the fast path, with p = h*inv (exact in double) and K
// integer, floor(p + K/2^16) = floor(p) + [t + K >= 2^16], t = floor(2^16 p) - 2^16 floor(p),
// every term an exact integer in double.
//
// On the fast path (inv <= 2^100) the decision is taken in fp32 with the wave's rounding
// mode set to round toward -infinity (RD).  With A = 2^16 inv (exact), X = h*A + (2^23 + K)
// is 2^23 + 2^16 (h inv + K/2^16) exactly and v = fma(h, A, 2^23 + K) under RD is RD(X).
// Multiples of 2^16 (below 2^40) are representable and RD never rounds above X, so
// floor(v / 2^16) = floor(X / 2^16) for every X; with z an integer,
// f = RD(v * 2^-16 + (1.5*2^23 + z - 128)) = 1.5*2^23 + z + floor(v / 2^16) - 128
//   = 1.5*2^23 + floor(h inv + z + K/2^16)
// (one rounding of an exact sum inside the magic number's range).  Two fp32 operations per
// entry and no exceptions.  The two operations and the mode switches sit in one asm block,
// so that no other floating-point instruction is scheduled while the mode is RD.  Rows
// whose A would leave the fp32 range take double.
template <int F>
__device__ __forceinline__ bool sr_f32_ok(const RowGrid& g)
{
    return g.inv <= 0x1p100f;
}

// MODE register, FP_ROUND bits 1:0 (single precision): 0 nearest even, 2 toward -infinity
#define SSQ_MODE_ROUND_F32 "hwreg(HW_REG_MODE, 0, 2)"

// kz[i] = RD(RD(h[i]*A + kz[i]) * 2^-16 + M) for 8 entries, the mode RD only inside the
// block (s_nop 1: the two wait states between a mode write and a VALU that reads it).
__device__ __forceinline__ void sr_decide8_rd(const float* h, float A, float M, float* kz)
{
    asm volatile("s_setreg_imm32_b32 " SSQ_MODE_ROUND_F32 ", 2\n\t"
                 "s_nop 1\n\t"
                 "v_fmac_f32 %0, %8, %16\n\t"
                 "v_fmac_f32 %1, %9, %16\n\t"
                 "v_fmac_f32 %2, %10, %16\n\t"
                 "v_fmac_f32 %3, %11, %16\n\t"
                 "v_fmac_f32 %4, %12, %16\n\t"
                 "v_fmac_f32 %5, %13, %16\n\t"
                 "v_fmac_f32 %6, %14, %16\n\t"
                 "v_fmac_f32 %7, %15, %16\n\t"
                 "v_fmamk_f32 %0, %0, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %1, %1, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %2, %2, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %3, %3, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %4, %4, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %5, %5, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %6, %6, 0x37800000, %17\n\t"
                 "v_fmamk_f32 %7, %7, 0x37800000, %17\n\t"
                 "s_setreg_imm32_b32 " SSQ_MODE_ROUND_F32 ", 0\n\t"
                 "s_nop 1"
                 : "+v"(kz[0]), "+v"(kz[1]), "+v"(kz[2]), "+v"(kz[3]), "+v"(kz[4]), "+v"(kz[5]), "+v"(kz[6]),
                   "+v"(kz[7])
                 : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]), "v"(h[6]), "v"(h[7]),
                   "v"(A), "v"(M));
}

// The token the call's stochastic rounding starts at: the state's counter, read at the start
// of every wave (the call's own counter kernel advances it after the step kernels).
__device__ __forceinline__ uint64_t sr_token(const SrArgs& a)
{
    return *a.ctr;
}

template <int F, int E, bool FAST>
__device__ __forceinline__ void round_codes_sr(const float* h, const RowGrid& g, uint64_t seed, uint64_t ctr0,
                                               float* f)
{
    static_assert(E % 8 == 0, "eight entries per fp32 decision block");
    constexpr float flo = kMagic + (float)Traits<F>::lo;
    constexpr float fhi = kMagic + (float)Traits<F>::hi;
    const double inv16 = (double)g.inv * 65536.0;
    const float A = g.inv * 65536.0f;                 // exact
    const float Mz128 = g.Mz - 128.0f;               // 1.5*2^23 + z - 2^23/2^16, exact
    uint64_t x = seed + ((ctr0 >> 2) + 1) * kGoldenGamma;
#pragma unroll
    for (int q8 = 0; q8 < E / 8; ++q8) {
        uint32_t K[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint64_t o = splitmix_mix(x);
            x += kGoldenGamma;
            const uint32_t lo32 = (uint32_t)o, hi32 = (uint32_t)(o >> 32);
            K[4 * half + 0] = lo32 & 0xFFFFu;
            K[4 * half + 1] = lo32 >> 16;
            K[4 * half + 2] = hi32 & 0xFFFFu;
            K[4 * half + 3] = hi32 >> 16;
        }
        const int e0 = 8 * q8;
        if constexpr (FAST) {
            float kz[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                kz[k] = __uint_as_float(K[k] | 0x4B000000u); // 2^23 + K
            sr_decide8_rd(h + e0, A, Mz128, kz);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                f[e0 + k] = __builtin_amdgcn_fmed3f(kz[k], flo, fhi);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = e0 + k;
                const double P = (double)h[e] * inv16; // 2^16 h inv, exact
                const double fl = floor((double)h[e] * (double)g.inv);
                const double t = __builtin_fma(-65536.0, fl, floor(P));
                double c = fl + (double)g.zc + (t + (double)K[k] >= 65536.0 ? 1.0 : 0.0);
                c = fmin(fmax(c, (double)Traits<F>::lo), (double)Traits<F>::hi);
                f[e] = kMagic + (float)c;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fast refit: the same s, inv and z as refit(), with fewer instructions, for
// rows inside the ranges where the shortcuts were verified exhaustively
// (every fp32 mantissa, against IEEE division):
//   a / Qa    = fma(fma(-q, Qa, a), r, q), q = a*r, r = RN(1/Qa)  (normal a/Qa)
//   1 / s     = fma(fma(-s, y, 1), y, y),  y = v_rcp_f32(s)       (2^-126 < 1/s)
//   rne(mn*inv) = fma(mn, inv, 1.5*2^23) - 1.5*2^23               (|mn*inv| < 2^22)
// It also checks that no code leaves its range, so the rounding needs no
// clamp: the bottom asymmetric code is 0 by construction and the largest entry
// is the only one that can pass the top.  A row outside these conditions makes
// its wave take refit() and round_codes() instead.
// ---------------------------------------------------------------------------
template <int Q>
__device__ __forceinline__ float div_by_const(float a)
{
    constexpr float qf = (float)Q;
    constexpr float r = 1.0f / (float)Q;
    const float q = a * r;
    return __builtin_fmaf(__builtin_fmaf(-q, qf, a), r, q);
}

__device__ __forceinline__ float recip_rn(float s)
{
    const float y = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
}

// SR: the row is also rounded stochastically, which on this path needs sr_f32_ok
template <int F, bool SR = false>
__device__ __forceinline__ bool refit_fast(float mn, float mx, float amax, RowGrid& g)
{
    constexpr float lo_ok = 7.88860905e-31f; // 2^-100
    constexpr float hi_ok = 1.26765060e+30f; // 2^100
    g.slow = false;
    if constexpr (Traits<F>::asym) {
        const float range = mx - mn;
        const float s = div_by_const<Traits<F>::hi>(range);
        const float inv = recip_rn(s);
        const float z = kMagic - __builtin_fmaf(mn, inv, kMagic) + 0.0f;
        g.s = s;
        g.z = z;
        g.inv = inv;
        g.zc = z;
        g.Mz = kMagic + z;
        g.Mr = g.Mz;
        const float top = __builtin_fmaf(mx, inv, g.Mz);
        return range >= lo_ok && range <= hi_ok && fabsf(z) < kSlowZero &&
               top <= kMagic + (float)Traits<F>::hi && (!SR || sr_f32_ok<F>(g));
    } else {
        const float s = div_by_const<Traits<F>::hi>(amax);
        const float inv = recip_rn(s);
        g.s = s;
        g.z = 0.0f;
        g.inv = inv;
        g.zc = 0.0f;
        g.Mz = kMagic;
        g.Mr = kMagic;
        const float top = __builtin_fmaf(amax, inv, kMagic);
        return amax >= lo_ok && amax <= hi_ok && top <= kMagic + (float)Traits<F>::hi;
    }
}


// ---------------------------------------------------------------------------
// vector memory helpers: NW consecutive 32-bit words at a 4*NW-byte aligned address
// ---------------------------------------------------------------------------
// The state is streamed: every byte is read once and written once per step.
// SSQ_NT_LD / SSQ_NT_ST put the non-temporal hint on the state's loads / stores.
// The hint pays where one store instruction covers whole 64-byte segments (a
// quantized row's lanes hold adjacent 16-byte pieces).  Where a lane's pieces
// are 16 bytes at a wider stride (fp32 rows, half rows), the hinted stores
// leave partial segments that reach HBM unmerged: those rows go without it
// (an fp32 decode step took 2.9x as long with it).
#ifndef SSQ_NT
#define SSQ_NT 1
#endif
#ifndef SSQ_NT_LD
#define SSQ_NT_LD SSQ_NT
#endif
#ifndef SSQ_NT_ST
#define SSQ_NT_ST SSQ_NT
#endif

template <typename T, bool NT = true>
__device__ __forceinline__ T ld_stream(const T* p)
{
    if constexpr (NT && SSQ_NT_LD) return __builtin_nontemporal_load(p);
    else return *p;
}
template <typename T, bool NT = true>
__device__ __forceinline__ void st_stream(T* p, T v)
{
    if constexpr (NT && SSQ_NT_ST) __builtin_nontemporal_store(v, p);
    else *p = v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// buffer (descriptor) addressing: a wave-uniform base and byte range in scalar
// registers, a per-lane 32-bit offset and a uniform offset.  An access outside
// the range reads 0 and writes nothing, so a wrong offset cannot fault.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000; // gfx9 family: 32-bit data format, no swizzle, no stride
// cache-policy bits of the state's buffer loads and stores: sc0 = 1, nt = 2, sc1 = 16.
// kAuxStoreWhole is for stores whose instruction covers whole 64-byte segments (a lane
// holding 16 contiguous bytes of a row, so a row's lanes store it at once): sc1 | nt
// measured 2.6% faster than nt alone on the 370m int4 decode step.  Where a lane's pieces
// leave partial segments (two 16-byte pieces 32 bytes apart) sc1 doubled the step's time:
// those keep nt.
#ifndef SSQ_STORE_POLICY
#define SSQ_STORE_POLICY (SSQ_NT_ST ? 2 : 0)
#endif
#ifndef SSQ_STORE_POLICY_WHOLE
#define SSQ_STORE_POLICY_WHOLE (SSQ_NT_ST ? 18 : 0)
#endif
constexpr int kAuxLoad = SSQ_NT_LD ? 2 : 0; // the non-temporal hint on state loads
constexpr int kAuxStore = SSQ_STORE_POLICY;
constexpr int kAuxStoreWhole = SSQ_STORE_POLICY_WHOLE;
constexpr int kAuxStoreSc1 = 16; // write-through alone: y of a decode iteration of 16 rows

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

template <int NW, int AUX>
__device__ __forceinline__ void buf_load_words(Rsrc r, uint32_t voff, uint32_t soff, uint32_t* w)
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * i, soff, AUX);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else if constexpr (NW == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
        w[0] = v.x; w[1] = v.y;
    } else {
        static_assert(NW == 1, "unsupported lane width");
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
    }
}

template <int NW, int AUX>
__device__ __forceinline__ void buf_store_words(Rsrc r, uint32_t voff, uint32_t soff, const uint32_t* w)
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff + 16 * i, soff, AUX);
        }
    } else if constexpr (NW == 2) {
        const u32x2 v = {w[0], w[1]};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, AUX);
    } else {
        static_assert(NW == 1, "unsupported lane width");
        __builtin_amdgcn_raw_buffer_store_b32(w[0], r, voff, soff, AUX);
    }
}

template <int AUX>
__device__ __forceinline__ float buf_load_f32(Rsrc r, uint32_t voff, uint32_t soff)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
}
template <int AUX>
__device__ __forceinline__ void buf_store_f32(float v, Rsrc r, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, AUX);
}

template <int NW, bool NT = true>
__device__ __forceinline__ void load_words(const void* p, uint32_t* w)
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = ld_stream<u32x4, NT>(reinterpret_cast<const u32x4*>(p) + i);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else if constexpr (NW == 2) {
        const u32x2 v = ld_stream<u32x2, NT>(reinterpret_cast<const u32x2*>(p));
        w[0] = v.x; w[1] = v.y;
    } else {
        static_assert(NW == 1, "unsupported lane width");
        w[0] = ld_stream<uint32_t, NT>(reinterpret_cast<const uint32_t*>(p));
    }
}

template <int NW, bool NT = true>
__device__ __forceinline__ void store_words(void* p, const uint32_t* w)
{
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
            st_stream<u32x4, NT>(reinterpret_cast<u32x4*>(p) + i, v);
        }
    } else if constexpr (NW == 2) {
        const u32x2 v = {w[0], w[1]};
        st_stream<u32x2, NT>(reinterpret_cast<u32x2*>(p), v);
    } else {
        st_stream<uint32_t, NT>(reinterpret_cast<uint32_t*>(p), w[0]);
    }
}

template <int E>
__device__ __forceinline__ void load_f32(const float* p, float* v)
{
    static_assert(E % 4 == 0, "E must be a multiple of 4");
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
        const float4 t = reinterpret_cast<const float4*>(p)[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
}

template <int E>
__device__ __forceinline__ void store_f32(float* p, const float* v)
{
#pragma unroll
    for (int i = 0; i < E / 4; ++i)
        reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

} // namespace ssq
