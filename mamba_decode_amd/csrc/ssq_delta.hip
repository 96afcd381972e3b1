// ssq_delta.hip -- delta-rule (Gated DeltaNet / KDA style) matrix-state step
// with the state stored quantized per key row, for gfx950.
//
//   S' = alpha*(I - beta*k*k^T)*S + beta*k*v^T = alpha*S + k*w^T,
//   w  = beta*(v - alpha*u),  u = k^T S,   o = S'^T q
// ("Mamba state quantization for inference": one dk x dv matrix per head, the
// query reads it, decay and a delta-rule correction write the next version;
// the kernel of the DAMP paragraph reconstructs the low-precision tier,
// computes the recurrence in FP32, derives new quantization parameters and
// writes the state back -- here with a single int8/int4 tier).
//
// Mapping: one 256-thread workgroup per (sequence, head) matrix of 128 key
// rows x 128 values.  Thread t owns rows {t/8 + 32k : k < 4} and the 16
// columns 16*(t%8) .. +15, so each row is held by 8 lanes of one wave and its
// min/max and refit use DPP only.  The two column reductions (u = k^T S before
// the update and o = S'^T q after it) cross rows: every thread reduces its four
// rows in registers, then the 32 partial rows meet in LDS.  u is accumulated in
// double and rounded once, so its reduction order only matters where the sum
// lies within double rounding of an fp32 midpoint; o is an output only.  The whole matrix (16 KiB of int8
// codes) is read once and written once.  Each key row is reconstructed once,
// fl(s*fl(c - z)), and the fp32 values stay in registers from u to the update.
#include "ssq_device.h"
#include "ssq_internal.h"

namespace ssq {

// waves per SIMD the register budget is sized for
#ifndef SSQ_DELTA_WAVES
#define SSQ_DELTA_WAVES 4
#endif
#ifndef SSQ_DAMP_WAVES
#define SSQ_DAMP_WAVES 3
#endif

// A quantized key row's piece (4*NW bytes at `off` within the block's rows) stored through a
// buffer descriptor over the block's own rows, with the write-through streaming policy: the
// row's 8 lanes store it whole with one instruction.
template <int NW>
__device__ __forceinline__ void store_row_piece(uint8_t* rows_base, uint32_t rows_bytes, uint32_t off,
                                                const uint32_t* w)
{
    buf_store_words<NW, kAuxStoreWhole>(make_rsrc(rows_base, rows_bytes), off, 0u, w);
}

// Partial rows in LDS, 128 columns per row group r, column c stored at r*128 + (c ^ x(c)):
// u in double with x = 2*(c/16), o in float with x = 4*(c/32).  The XOR stays inside the
// aligned pair (u) or quad (o) that one 16-byte write carries, so thread (r, part) still
// writes its 16 columns with 16-byte writes.  gfx950's LDS serves a 16-byte write 8 lanes at
// a time over 32 four-byte banks, an 8-byte read 16 lanes at a time and a 4-byte read 32
// lanes at a time over the same 32 banks (and a 16-byte read 16 lanes at a time over 64
// banks); with these swizzles the eight parts of a write land in eight distinct 16-byte bank
// windows, and the 16 (u) or 32 (o) consecutive columns that one read serves land in
// distinct banks, so neither side has a bank conflict.
__device__ __forceinline__ int part_idx(int r, int c) { return r * 128 + (c ^ (2 * (c >> 4))); }
__device__ __forceinline__ int part_idx_o(int r, int c) { return r * 128 + (c ^ (4 * (c >> 5))); }
constexpr int kPartElems = 32 * 128; // doubles; the float rows of o use the first half of the bytes
// thread (r, part)'s 16 columns 16*part .. 16*part + 15: pairs (u) or quads (o) at the
// swizzled offsets, one 16-byte write each
__device__ __forceinline__ void store_part_u(double* pu, int r, int part, const double* v)
{
    double* const row = pu + r * 128 + part * 16;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2)
        *reinterpret_cast<double2*>(row + 2 * (e2 ^ part)) = make_double2(v[2 * e2], v[2 * e2 + 1]);
}
__device__ __forceinline__ void store_part_o(float* po, int r, int part, const float* v)
{
    float* const row = po + r * 128 + part * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(row + 4 * (q ^ (part >> 1))) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}
// Column c's sum over the 32 partial rows, as four interleaved chains (rows r = k mod 4)
// added pairwise at the end: a dependent chain of 8 + 2 adds instead of 32.  u is summed in
// double and rounded once and o is an output, so neither fixes this order.
// T = double: the partial rows of u (part_idx); T = float: those of o (part_idx_o).
template <typename T>
__device__ __forceinline__ T column_sum(const T* rows, int c)
{
    auto at = [&](int r) { return rows[sizeof(T) == 8 ? part_idx(r, c) : part_idx_o(r, c)]; };
    T a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
    for (int r = 0; r < 32; r += 4) {
        a0 += at(r);
        a1 += at(r + 1);
        a2 += at(r + 2);
        a3 += at(r + 3);
    }
    return (a0 + a1) + (a2 + a3);
}

// w is shared through LDS with 4 floats of padding after every 64: column j sits at
// j + 4*(j/64), so the eight parts' 16-byte reads (16 lanes, two row groups, per pass) fall in
// eight distinct 16-byte windows of the 64 banks.
constexpr int kWPad = 136;
__device__ __forceinline__ int w_idx(int j) { return j + 4 * (j >> 6); }

// The matrix the step starts from, reconstructed in fp32 (fl(s_i*fl(c_ij - z_i)) for a
// quantized key row), stays in registers from the u reduction to the update: each entry is
// reconstructed once.
// KDA: a decay per key channel (alpha [matrices][128]), S' = (I - beta k k^T) Diag(alpha) S
// + beta k v^T, evaluated as u = k^T Diag(alpha) S, w = beta*(v - u), S' = alpha_i*S + k w^T
template <int F, bool PRE, bool SR, bool KDA>
__global__ __launch_bounds__(256, SSQ_DELTA_WAVES) void k_delta_step(DeltaArgs a)
{
    using Tr = Traits<F>;
    constexpr int LPR = 8, E = 16, RG = 32, KR = 4; // lanes per row, columns per lane, row groups, rows per thread
    constexpr int NW = Tr::quant ? E * Tr::bits / 32 : E;
    constexpr int ROWB = Tr::quant ? 128 * Tr::bits / 8 : 512;
    __shared__ __attribute__((aligned(16))) double part_u[kPartElems]; // reused for the fp32 partials of o
    __shared__ __attribute__((aligned(16))) float w_s[kWPad];

    const int t = threadIdx.x;
    const int rg = t >> 3, part = t & 7, j0 = part * E;
    const int64_t mat = blockIdx.x;
    const int64_t mrow0 = mat * 128; // first state row of the matrix
    const float alpha = KDA ? 0.0f : a.alpha[mat], beta = a.beta[mat];
    const uint64_t sr_step = SR ? sr_token(a.sr) : 0;

    float kk[KR], qq[KR], al[KR];
    float Sh[KR][E]; // this thread's 16 columns of its four key rows, in fp32
    {
        uint32_t cw[KR][NW];
        float s_old[KR], z_old[KR];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const int i = rg + RG * r;
            kk[r] = a.k[mrow0 + i];
            qq[r] = a.q[mrow0 + i];
            al[r] = KDA ? a.alpha[mrow0 + i] : alpha; // the key row's decay
            const int64_t row = mrow0 + i;
            if constexpr (Tr::quant) {
                load_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw[r]);
                s_old[r] = a.scale[row];
                z_old[r] = Tr::asym ? a.zero[row] : 0.0f;
            } else {
                load_f32<E>(a.h32 + row * 128 + j0, Sh[r]);
            }
        }
        if constexpr (Tr::quant) {
#pragma unroll
            for (int r = 0; r < KR; ++r) {
                unpack_codes<F, E>(cw[r], Sh[r]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = Tr::asym ? Sh[r][e] - z_old[r] : Sh[r][e];
                    Sh[r][e] = s_old[r] * d;
                }
            }
        }
    }
    // column t's value of v, for the threads that form w_t
    const float vcol = t < 128 ? a.v[mrow0 + t] : 0.0f;

    // u = k^T S (KDA: k^T Diag(alpha) S), products and sums in double, rounded once
    {
        double up[E];
#pragma unroll
        for (int e = 0; e < E; ++e) up[e] = 0.0;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const double kd = KDA ? (double)kk[r] * (double)al[r] : (double)kk[r];
#pragma unroll
            for (int e = 0; e < E; ++e) up[e] = __builtin_fma(kd, (double)Sh[r][e], up[e]);
        }
        store_part_u(part_u, rg, part, up);
    }
    __syncthreads();
    if (t < 128) {
        const double acc = column_sum(part_u, t);
        // w_t = beta*(v_t - alpha*u_t), or beta*(v_t - u_t) for KDA (the decay is
        // already in u), formed once per column and shared
        const float u = (float)acc;
        const float au = KDA ? u : alpha * u;
        const float vm = vcol - au;
        w_s[w_idx(t)] = beta * vm;
    }
    __syncthreads();

    // S' = alpha*S + k w^T, row by row; refit, round and store each row.  w is read from LDS
    // for each row (four 16-byte reads) rather than held in 16 registers across the rows.
    float op[E];
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const int64_t row = mrow0 + rg + RG * r;
        float* const S = Sh[r];
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 w4 = reinterpret_cast<const float4*>(w_s + w_idx(j0))[q];
            const float wq[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float kw = kk[r] * wq[k];
                S[4 * q + k] = __builtin_fmaf(al[r], S[4 * q + k], kw);
            }
        }
        if constexpr (!Tr::quant || PRE) {
#pragma unroll
            for (int e = 0; e < E; ++e) op[e] = __builtin_fmaf(qq[r], S[e], op[e]);
        }
        if constexpr (Tr::quant) {
            float mn = 0.0f, mx = 0.0f, am = 0.0f;
            if constexpr (Tr::asym) {
                mn = S[0];
                mx = S[0];
#pragma unroll
                for (int e = 1; e < E; ++e) {
                    mn = fminf(mn, S[e]);
                    mx = fmaxf(mx, S[e]);
                }
                mn = group_min<LPR>(mn);
                mx = group_max<LPR>(mx);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) am = fmaxf(am, fabsf(S[e]));
                am = group_max<LPR>(am);
            }
            RowGrid g;
            float f[E];
            // stochastic rounding: this lane's first counter, (step*rows + row)*128 + j0
            const uint64_t ctr0 = SR ? ((sr_step * (uint64_t)a.sr.rows + (uint64_t)row) * 128u + (uint64_t)j0) : 0;
            if (__all(refit_fast<F, SR>(mn, mx, am, g))) {
                if constexpr (SR) {
                    round_codes_sr<F, E, true>(S, g, a.sr.seed, ctr0, f);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) f[e] = __builtin_fmaf(S[e], g.inv, g.Mz);
                }
            } else {
                g = refit<F>(mn, mx, am);
                if constexpr (SR) {
                    round_codes_sr<F, E, false>(S, g, a.sr.seed, ctr0, f);
                } else {
                    const bool slow_any = Tr::asym && __any(g.slow);
                    round_codes<F, E>(S, g, slow_any, f);
                }
            }
            uint32_t ow[NW];
            pack_codes<F, E>(f, ow);
            store_row_piece<NW>(a.codes + mrow0 * ROWB, 128u * ROWB,
                                (uint32_t)((row - mrow0) * ROWB + part * (NW * 4)), ow);
            if (part == 0) {
                a.scale[row] = g.s;
                if constexpr (Tr::asym) a.zero[row] = g.z;
            }
            if constexpr (!PRE) {
                const float qs = qq[r] * g.s;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float cz = f[e] - g.Mr; // c - z (the readout is an output)
                    op[e] = __builtin_fmaf(qs, cz, op[e]);
                }
            }
        } else {
            store_f32<E>(a.h32 + row * 128 + j0, S);
        }
    }

    // o = S'^T q: 32 partial rows meet in LDS
    float* part_o = reinterpret_cast<float*>(part_u);
    store_part_o(part_o, rg, part, op);
    __syncthreads();
    if (t < 128) {
        a.o[mrow0 + t] = column_sum(part_o, t);
    }
}

template <int F, bool KDA>
static hipError_t launch_delta_fk(DeltaArgs a, bool pre, hipStream_t st)
{
    const unsigned blocks = (unsigned)a.nmat;
    if constexpr (Traits<F>::quant) {
        if (a.sr.on) {
            if (pre)
                hipLaunchKernelGGL((k_delta_step<F, true, true, KDA>), dim3(blocks), dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL((k_delta_step<F, false, true, KDA>), dim3(blocks), dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
    if (pre)
        hipLaunchKernelGGL((k_delta_step<F, true, false, KDA>), dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_delta_step<F, false, false, KDA>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int F>
static hipError_t launch_delta_f(DeltaArgs a, bool pre, hipStream_t st)
{
    return a.kda ? launch_delta_fk<F, true>(a, pre, st) : launch_delta_fk<F, false>(a, pre, st);
}

hipError_t launch_delta_step(int fmt, DeltaArgs a, bool pre, hipStream_t st)
{
    switch (fmt) {
    case FP32: return launch_delta_f<FP32>(a, pre, st);
    case INT8_SYM: return launch_delta_f<INT8_SYM>(a, pre, st);
    case INT8_ASYM: return launch_delta_f<INT8_ASYM>(a, pre, st);
    case INT4_SYM: return launch_delta_f<INT4_SYM>(a, pre, st);
    case INT4_ASYM: return launch_delta_f<INT4_ASYM>(a, pre, st);
    }
    return hipErrorInvalidValue;
}

} // namespace ssq

// ===========================================================================
// two-tier delta state ("Mamba state quantization for inference", "Mixed
// precision spends bits on persistent channels"): every key row rotated by
// Hs = H_128/16 along the value dimension, key rows 0..15 of each matrix kept
// as IEEE half values, rows 16..127 as asymmetric uint8 codes with a per-row
// fp32 scale and zero point.  The step is the scalar-decay delta rule in the
// rotated coordinates, v rotated in and o rotated out (Hs Hs = I/2).
// ===========================================================================
namespace ssq {

constexpr int kNhi = 16, kNlo = 112;

// (-1)^popcount(i & j) / 16: entry (i, j) of the Sylvester-ordered Hadamard matrix over 16
__device__ __forceinline__ double hs(int i, int j)
{
    return (__builtin_popcount(i & j) & 1) ? -0.0625 : 0.0625;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
// The fp32 value rounded to the nearest half (ties to even).  The value is made opaque
// first: the compiler would otherwise fold the fp32 rounding of the fma or double sum that
// produced it into one rounding straight to half (v_fma_mix*), which differs from rounding
// twice exactly when the fp32 value sits on a half midpoint.
__device__ __forceinline__ uint32_t float_to_half_bits(float x)
{
    asm volatile("" : "+v"(x));
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// H_128 x (Sylvester order, unscaled) of the 128 values x held one per thread by threads
// 0..127, in double: butterflies over lane distances 1..32, the last level through LDS.
// Each output is a sum of the 128 inputs with signs; it is exact (so equal to any other
// summation order) while the inputs span less than 2^29 in magnitude.  Holds a barrier:
// every thread of the block calls it; threads 128..255 return their x unchanged.
__device__ __forceinline__ double wht128(double x, double* xch)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
        const double p = __shfl_xor(x, h);
        x = (t & h) ? p - x : x + p;
    }
    if (t < 128) xch[t] = x;
    __syncthreads();
    if (t < 128) {
        const double p = xch[t ^ 64];
        x = (t & 64) ? p - x : x + p;
    }
    return x;
}

// Mapping as k_delta_step: thread t owns key rows t/8 + 32k (k < 4) and 16 columns.  Row
// k = 0 of threads 0..127 (waves 0 and 1) is a half row, every other row a uint8 row, so
// the tier of a row is uniform across its wave.
template <bool PRE, bool SR>
__global__ __launch_bounds__(256, SSQ_DAMP_WAVES) void k_damp_step(DeltaArgs a)
{
    constexpr int F = INT8_ASYM;
    constexpr int LPR = 8, E = 16, RG = 32, KR = 4, NW = 4, ROWB = 128;
    __shared__ __attribute__((aligned(16))) double part_u[kPartElems]; // reused for the fp32 partials of the readout
    __shared__ __attribute__((aligned(16))) float w_s[kWPad];
    __shared__ double xch[128];

    const int t = threadIdx.x;
    const int rg = t >> 3, part = t & 7, j0 = part * E;
    const int64_t mat = blockIdx.x;
    const int64_t mrow0 = mat * 128;
    const float alpha = a.alpha[mat], beta = a.beta[mat];
    const bool hi_wave = rg < kNhi; // row k = 0 of this thread is a half row
    const uint64_t sr_step = SR ? sr_token(a.sr) : 0;

    const double vj = t < 128 ? (double)a.v[mrow0 + t] : 0.0;

    float kk[KR], qq[KR];
    float Sh[KR][E]; // the stored rows in fp32: half values, or fl(s*fl(c - z)) of the uint8 rows
    {
        uint32_t cw[KR][2 * NW]; // uint8 rows: 4 words of codes; half rows: 8 words of halves
        float s_old[KR], z_old[KR];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const int i = rg + RG * r;
            kk[r] = a.k[mrow0 + i];
            qq[r] = a.q[mrow0 + i];
            if (r == 0 && hi_wave) {
                load_words<2 * NW, false>(a.hi + (mat * kNhi + i) * 128 + j0, cw[r]);
                s_old[r] = 1.0f;
                z_old[r] = 0.0f;
            } else {
                const int64_t lrow = mat * kNlo + (i - kNhi);
                load_words<NW>(a.codes + lrow * ROWB + part * (NW * 4), cw[r]);
                s_old[r] = a.scale[lrow];
                z_old[r] = a.zero[lrow];
            }
        }
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            if (r == 0 && hi_wave) {
#pragma unroll
                for (int q = 0; q < NW * 2; ++q) {
                    Sh[r][2 * q] = half_bits_to_float(cw[r][q] & 0xFFFFu);
                    Sh[r][2 * q + 1] = half_bits_to_float(cw[r][q] >> 16);
                }
            } else {
                unpack_codes<F, E>(cw[r], Sh[r]);
#pragma unroll
                for (int e = 0; e < E; ++e) Sh[r][e] = s_old[r] * (Sh[r][e] - z_old[r]);
            }
        }
    }
    // ut = k^T St in double, rounded once
    {
        double up[E];
#pragma unroll
        for (int e = 0; e < E; ++e) up[e] = 0.0;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const double kd = (double)kk[r];
#pragma unroll
            for (int e = 0; e < E; ++e) up[e] = __builtin_fma(kd, (double)Sh[r][e], up[e]);
        }
        store_part_u(part_u, rg, part, up);
    }
    // vt = Hs v, rounded once; thread t < 128 holds column t (here, where the partial sums
    // of u no longer hold registers)
    const float vt = (float)(wht128(vj, xch) * 0.0625);
    __syncthreads();
    if (t < 128) {
        const double acc = column_sum(part_u, t);
        // wt = beta*(vt - alpha*ut), formed once per column and shared
        const float au = alpha * (float)acc;
        const float vm = vt - au;
        w_s[w_idx(t)] = beta * vm;
    }
    __syncthreads();

    float op[E];
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const int i = rg + RG * r;
        float* const S = Sh[r];
        // every row: St' = fma(alpha, St, fl(k*wt)), wt read from LDS for each row
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 w4 = reinterpret_cast<const float4*>(w_s + w_idx(j0))[q];
            const float wq[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float kw = kk[r] * wq[k];
                S[4 * q + k] = __builtin_fmaf(alpha, S[4 * q + k], kw);
            }
        }
        if constexpr (PRE) {
#pragma unroll
            for (int e = 0; e < E; ++e) op[e] = __builtin_fmaf(qq[r], S[e], op[e]);
        }
        if (r == 0 && hi_wave) {
            // half row: round to half
            uint32_t hw[2 * NW];
#pragma unroll
            for (int q = 0; q < 2 * NW; ++q) {
                const uint32_t lo = float_to_half_bits(S[2 * q]), hi = float_to_half_bits(S[2 * q + 1]);
                hw[q] = lo | (hi << 16);
                S[2 * q] = half_bits_to_float(lo);
                S[2 * q + 1] = half_bits_to_float(hi);
            }
            store_words<2 * NW, false>(a.hi + (mat * kNhi + i) * 128 + j0, hw);
            if constexpr (!PRE) {
#pragma unroll
                for (int e = 0; e < E; ++e) op[e] = __builtin_fmaf(qq[r], S[e], op[e]);
            }
        } else {
            const int64_t lrow = mat * kNlo + (i - kNhi);
            float mn = S[0], mx = S[0];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                mn = fminf(mn, S[e]);
                mx = fmaxf(mx, S[e]);
            }
            mn = group_min<LPR>(mn);
            mx = group_max<LPR>(mx);
            RowGrid g;
            float f[E];
            const uint64_t ctr0 = SR ? ((sr_step * (uint64_t)a.sr.rows + (uint64_t)lrow) * 128u + (uint64_t)j0) : 0;
            if (__all(refit_fast<F, SR>(mn, mx, 0.0f, g))) {
                if constexpr (SR) {
                    round_codes_sr<F, E, true>(S, g, a.sr.seed, ctr0, f);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) f[e] = __builtin_fmaf(S[e], g.inv, g.Mz);
                }
            } else {
                g = refit<F>(mn, mx, 0.0f);
                if constexpr (SR) {
                    round_codes_sr<F, E, false>(S, g, a.sr.seed, ctr0, f);
                } else {
                    const bool slow_any = __any(g.slow);
                    round_codes<F, E>(S, g, slow_any, f);
                }
            }
            uint32_t ow[NW];
            pack_codes<F, E>(f, ow);
            store_row_piece<NW>(a.codes + mat * kNlo * ROWB, (uint32_t)(kNlo * ROWB),
                                (uint32_t)((lrow - mat * kNlo) * ROWB + part * (NW * 4)), ow);
            if (part == 0) {
                a.scale[lrow] = g.s;
                a.zero[lrow] = g.z;
            }
            if constexpr (!PRE) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float r_ij = g.s * ((f[e] - kMagic) - g.z); // the stored value, fl(s*fl(c - z))
                    op[e] = __builtin_fmaf(qq[r], r_ij, op[e]);
                }
            }
        }
    }

    // ot = St'^T q meets in LDS; o = 2 Hs ot
    float* part_o = reinterpret_cast<float*>(part_u);
    store_part_o(part_o, rg, part, op);
    __syncthreads();
    float ot = 0.0f;
    if (t < 128) ot = column_sum(part_o, t);
    const double x = wht128((double)ot, xch);
    if (t < 128) a.o[mrow0 + t] = (float)(x * 0.125);
}

// Rows of a two-tier state, 8 lanes per key row (16 columns each).  init: rotate the fp32
// row (each output a sum over the input row in order, in double, rounded once), then round
// the half rows to half and refit and round the uint8 rows; dequant: S = 2 St Hs.
template <bool DEQ>
__global__ __launch_bounds__(256) void k_damp_rows(QArgs a)
{
    constexpr int F = INT8_ASYM;
    constexpr int LPR = 8, E = 16, NW = 4, ROWB = 128;
    const int lane = threadIdx.x & 63, sub = lane >> 3, part = lane & 7, j0 = part * E;
    const int64_t row = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 8 + sub;
    const bool live = row < a.rows; // rows come in whole matrices of 128, so a wave is all live or not
    if (!__any(live)) return;
    const int64_t mat = row / 128;
    const int i = (int)(row % 128);
    const bool hi_row = i < kNhi;
    const int64_t lrow = mat * kNlo + (i - kNhi);
    if constexpr (!DEQ) {
        const float* src = a.in + row * 128;
        float rv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < 128; ++c) acc = __builtin_fma((double)src[c], hs(c, j0 + e), acc);
            rv[e] = (float)acc;
        }
        if (hi_row) {
            uint32_t hw[2 * NW];
#pragma unroll
            for (int q = 0; q < 2 * NW; ++q)
                hw[q] = float_to_half_bits(rv[2 * q]) | (float_to_half_bits(rv[2 * q + 1]) << 16);
            store_words<2 * NW, false>(a.hi + (mat * kNhi + i) * 128 + j0, hw);
        } else {
            float mn = rv[0], mx = rv[0];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                mn = fminf(mn, rv[e]);
                mx = fmaxf(mx, rv[e]);
            }
            // a row's 8 lanes are all half rows or all uint8 rows; reduce within them
            mn = group_min<LPR>(mn);
            mx = group_max<LPR>(mx);
            const RowGrid g = refit<F>(mn, mx, 0.0f);
            float f[E];
            round_codes<F, E>(rv, g, g.slow, f);
            uint32_t ow[NW];
            pack_codes<F, E>(f, ow);
            store_words<NW>(a.codes + lrow * ROWB + part * (NW * 4), ow);
            if (part == 0) {
                a.scale[lrow] = g.s;
                a.zero[lrow] = g.z;
            }
        }
    } else {
        // every lane reconstructs the whole stored row, then forms its 16 outputs
        float r128[128];
        if (hi_row) {
            const uint16_t* hp = a.hi + (mat * kNhi + i) * 128;
            for (int c = 0; c < 128; ++c) r128[c] = half_bits_to_float(hp[c]);
        } else {
            const uint8_t* cp = a.codes + lrow * ROWB;
            const float s = a.scale[lrow], z = a.zero[lrow];
            for (int c = 0; c < 128; ++c) r128[c] = s * ((float)cp[c] - z);
        }
        float out[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int c = 0; c < 128; ++c) acc = __builtin_fma((double)r128[c], hs(c, j0 + e), acc);
            out[e] = (float)(2.0 * acc);
        }
        store_f32<E>(a.out + row * 128 + j0, out);
    }
}

hipError_t launch_damp_step(DeltaArgs a, bool pre, hipStream_t st)
{
    const unsigned blocks = (unsigned)a.nmat;
    if (a.sr.on) {
        if (pre) hipLaunchKernelGGL((k_damp_step<true, true>), dim3(blocks), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_damp_step<false, true>), dim3(blocks), dim3(256), 0, st, a);
    } else {
        if (pre) hipLaunchKernelGGL((k_damp_step<true, false>), dim3(blocks), dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_damp_step<false, false>), dim3(blocks), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_damp_rows(QArgs a, bool dequant, hipStream_t st)
{
    const int64_t waves = (a.rows + 7) / 8;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (dequant) hipLaunchKernelGGL((k_damp_rows<true>), dim3(blocks), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_damp_rows<false>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

} // namespace ssq
