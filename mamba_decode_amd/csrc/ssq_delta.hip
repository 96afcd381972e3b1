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
// codes) is read once and written once.  The codes stay packed in registers between
// the two phases (4 waves per SIMD, 4 matrices per CU in flight).
#include "ssq_device.h"
#include "ssq_internal.h"

namespace ssq {

// waves per SIMD the register budget is sized for
#ifndef SSQ_DELTA_WAVES
#define SSQ_DELTA_WAVES 4
#endif

// KDA: a decay per key channel (alpha [matrices][128]), S' = (I - beta k k^T) Diag(alpha) S
// + beta k v^T, evaluated as u = k^T Diag(alpha) S, w = beta*(v - u), S' = alpha_i*S + k w^T
template <int F, bool PRE, bool SR, bool KDA>
__global__ __launch_bounds__(256, SSQ_DELTA_WAVES) void k_delta_step(DeltaArgs a)
{
    using Tr = Traits<F>;
    constexpr int LPR = 8, E = 16, RG = 32, KR = 4; // lanes per row, columns per lane, row groups, rows per thread
    constexpr int NW = Tr::quant ? E * Tr::bits / 32 : E;
    constexpr int NS = NW; // registers per row part (packed codes, or fp32 values)
    constexpr int ROWB = Tr::quant ? 128 * Tr::bits / 8 : 512;
    __shared__ double part_u[RG * 128]; // reused for the fp32 partials of o
    __shared__ float u_s[128];

    const int t = threadIdx.x;
    const int rg = t >> 3, part = t & 7, j0 = part * E;
    const int64_t mat = blockIdx.x;
    const int64_t mrow0 = mat * 128; // first state row of the matrix
    const float alpha = KDA ? 0.0f : a.alpha[mat], beta = a.beta[mat];

    float kk[KR], qq[KR], s_old[KR], z_old[KR], al[KR];
    // the codes stay packed in registers (or the fp32 rows, for the fp32 state) and are
    // unpacked where they are used, once for u and once for the update: fewer live
    // registers, more waves per SIMD to overlap the matrix loads
    uint32_t cw[KR][NW];
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
            load_f32<E>(a.h32 + row * 128 + j0, reinterpret_cast<float*>(cw[r]));
            s_old[r] = 1.0f;
            z_old[r] = 0.0f;
        }
    }
    auto row_values = [&](int r, float* f) {
        if constexpr (Tr::quant) unpack_codes<F, E>(cw[r], f); // the codes c_ij as floats
        else {
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = __uint_as_float(cw[r][e]);
        }
    };
    float vv[E];
    load_f32<E>(a.v + mrow0 + j0, vv);

    // u = k^T S in double: sum_i kap_i*c_ij - sum_i kap_i*z_i with kap_i = k_i*s_i exact
    // (quantized), or sum_i k_i*S_ij (fp32); the z term is the same for every column.
    // KDA folds the row's decay in: kap_i = (k_i*alpha_i)*s_i.
    {
        double kaps[KR];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const double kd = KDA ? (double)kk[r] * (double)al[r] : (double)kk[r];
            kaps[r] = Tr::quant ? kd * (double)s_old[r] : kd;
        }
        double up[E];
        double zt = 0.0;
        if constexpr (Tr::asym) {
#pragma unroll
            for (int r = 0; r < KR; ++r) zt = __builtin_fma(kaps[r], (double)z_old[r], zt);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) up[e] = -zt;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const double kap = kaps[r];
            float f[E];
            row_values(r, f);
#pragma unroll
            for (int e = 0; e < E; ++e) up[e] = __builtin_fma(kap, (double)f[e], up[e]);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) part_u[rg * 128 + j0 + e] = up[e];
    }
    __syncthreads();
    if (t < 128) {
        double acc = 0.0;
#pragma unroll 8
        for (int r = 0; r < RG; ++r) acc += part_u[r * 128 + t];
        u_s[t] = (float)acc;
    }
    __syncthreads();

    // w = beta*(v - alpha*u), or beta*(v - u) for KDA (the decay is already in u)
    float ww[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float au = KDA ? u_s[j0 + e] : alpha * u_s[j0 + e];
        const float vm = vv[e] - au;
        ww[e] = beta * vm;
    }

    // S' = alpha*S + k w^T, row by row; refit, round and store each row
    float op[E];
#pragma unroll
    for (int e = 0; e < E; ++e) op[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < KR; ++r) {
        const int64_t row = mrow0 + rg + RG * r;
        // unpack again rather than keep the first unpacking alive across the u reduction
#pragma unroll
        for (int q = 0; q < NS; ++q) asm volatile("" : "+v"(cw[r][q]));
        float S[E];
        row_values(r, S);
        if constexpr (Tr::quant) {
            // alpha*s*(c - z) + k*w = fma(as, c, fma(k, w, -as*z)): the decay acts on the scale
            const float as = al[r] * s_old[r];
            const float az = as * z_old[r];
#pragma unroll
            for (int e = 0; e < E; ++e) S[e] = __builtin_fmaf(as, S[e], __builtin_fmaf(kk[r], ww[e], -az));
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float kw = kk[r] * ww[e];
                S[e] = __builtin_fmaf(al[r], S[e], kw);
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
            const uint64_t ctr0 = SR ? ((a.sr.step * (uint64_t)a.sr.rows + (uint64_t)row) * 128u + (uint64_t)j0) : 0;
            if (__all(refit_fast<F>(mn, mx, am, g))) {
                if constexpr (SR) {
                    round_codes_sr<F, E>(S, g, a.sr.seed, ctr0, f);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) f[e] = __builtin_fmaf(S[e], g.inv, g.Mz);
                }
            } else {
                g = refit<F>(mn, mx, am);
                if constexpr (SR) {
                    round_codes_sr<F, E>(S, g, a.sr.seed, ctr0, f);
                } else {
                    const bool slow_any = Tr::asym && __any(g.slow);
                    round_codes<F, E>(S, g, slow_any, f);
                }
            }
            uint32_t ow[NW];
            pack_codes<F, E>(f, ow);
            store_words<NW>(a.codes + row * ROWB + part * (NW * 4), ow);
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
#pragma unroll
    for (int e = 0; e < E; ++e) part_o[rg * 128 + j0 + e] = op[e];
    __syncthreads();
    if (t < 128) {
        float acc = 0.0f;
#pragma unroll 8
        for (int r = 0; r < RG; ++r) acc += part_o[r * 128 + t];
        a.o[mrow0 + t] = acc;
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
