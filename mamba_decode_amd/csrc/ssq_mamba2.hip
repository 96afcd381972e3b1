// ssq_mamba2.hip -- Mamba-2 decode step, fused scan, row quantization and
// dequantization kernels for gfx950.
//
// What a row update computes ("ssm-state-quantization" README, Setup): the
// head decays its state by lambda = exp(dt*A), the token writes dt*x*B, the
// output y = C.h + D*x is read from the quantized state, and the row's scale
// (and zero point) is refit before rounding to nearest.
//
// Work mapping.  A wave64 handles 64/LPR rows at a time ("an iteration"),
// LPR lanes per row and E = 128/LPR entries per lane, so each lane moves 16
// contiguous bytes of int8 or int4 codes (32 for fp32) and a wave's access is
// one contiguous run of rows.  The decode kernel gives each wave a contiguous
// range of iterations; B and C of the current (sequence, group) stay in
// registers while consecutive rows reuse them, and the per-head decay is
// computed once for up to 64 heads in parallel lanes and broadcast with
// v_readlane.  The next row's codes are loaded before the current row is
// processed.  Nothing is shared between waves, so there is no LDS and no
// barrier; the kernel is bound by HBM traffic (codes + metadata in and out).
#include "ssq_device.h"
#include "ssq_internal.h"

namespace ssq {

template <int F>
struct RowBytes {
    static constexpr int value = Traits<F>::quant ? 128 * Traits<F>::bits / 8 : 512;
};

// uniform wave index (an SGPR), so that every per-iteration value below is scalar
__device__ __forceinline__ int64_t wave_id()
{
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    return (int64_t)blockIdx.x * (blockDim.x >> 6) + w;
}

// ---------------------------------------------------------------------------
// one row, one token: dequantize, decay + write, refit, round, pack.
// Returns the lane's share of the readout sum (before the group reduction).
// ---------------------------------------------------------------------------
template <int F, int LPR, bool PRE>
struct RowStep {
    static constexpr int E = 128 / LPR;
    static constexpr int NW = Traits<F>::quant ? E * Traits<F>::bits / 32 : E;

    // quantized formats: cw in -> ow out, s/z in -> grid out
    __device__ __forceinline__ static float run_q(const uint32_t* cw, float s_old, float z_old, float lam,
                                                  float w, const float* Bv, const float* Cv, uint32_t* ow,
                                                  RowGrid& g, bool& slow_any)
    {
        using Tr = Traits<F>;
        float h[E];
        unpack_codes<F, E>(cw, h);
        const float ls = lam * s_old;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float d = Tr::asym ? h[e] - z_old : h[e];
            const float wb = w * Bv[e];
            h[e] = __builtin_fmaf(ls, d, wb);
        }
        float acc = 0.0f;
        if constexpr (PRE) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc = __builtin_fmaf(Cv[e], h[e], acc);
        }
        float mn = 0.0f, mx = 0.0f, am = 0.0f;
        if constexpr (Tr::asym) {
            mn = h[0];
            mx = h[0];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                mn = fminf(mn, h[e]);
                mx = fmaxf(mx, h[e]);
            }
            mn = group_min<LPR>(mn);
            mx = group_max<LPR>(mx);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) am = fmaxf(am, fabsf(h[e]));
            am = group_max<LPR>(am);
        }
        g = refit<F>(mn, mx, am);
        slow_any = Tr::asym && __any(g.slow);
        float f[E];
        round_codes<F, E>(h, g, slow_any, f);
        pack_codes<F, E>(f, ow);
        if constexpr (!PRE) {
            if (!slow_any) {
#pragma unroll
                for (int e = 0; e < E; ++e) acc = __builtin_fmaf(Cv[e], f[e] - g.Mz, acc);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) acc = __builtin_fmaf(Cv[e], code_minus_z(f[e], g), acc);
            }
        }
        return acc;
    }

    // fp32 control: hv in/out
    __device__ __forceinline__ static float run_f(float* hv, float lam, float w, const float* Bv,
                                                  const float* Cv)
    {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float wb = w * Bv[e];
            hv[e] = __builtin_fmaf(lam, hv[e], wb);
            acc = __builtin_fmaf(Cv[e], hv[e], acc);
        }
        return acc;
    }
};

// lane share of sum_n C_n over the row (only needed by degenerate asymmetric rows)
template <int LPR, int E>
__device__ __forceinline__ float row_csum(const float* Cv)
{
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) cs += Cv[e];
    return group_sum<LPR>(cs);
}

// final readout of a row (value valid in every lane of the row group)
template <int F, bool PRE>
__device__ __forceinline__ float row_y(float acc, const RowGrid& g, float csum_if_needed, float dx)
{
    if constexpr (!Traits<F>::quant || PRE) return acc + dx;
    const float t = acc - g.zadj * csum_if_needed;
    return g.s * t + dx;
}

// ---------------------------------------------------------------------------
// decode step
// ---------------------------------------------------------------------------
template <int F, int LPR, bool PRE>
__global__ __launch_bounds__(256) void k_m2_step(M2Args a)
{
    using Tr = Traits<F>;
    using RS = RowStep<F, LPR, PRE>;
    constexpr int E = RS::E, NW = RS::NW, RPW = 64 / LPR, ROWB = RowBytes<F>::value;
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it0 = wave_id() * a.iters_per_wave;
    if (it0 >= a.total_iters) return;
    const int64_t it1 = min(it0 + (int64_t)a.iters_per_wave, a.total_iters);
    const int64_t nbh = (int64_t)a.Bsz * a.H;
    const int64_t bh0 = (it0 * RPW) / a.P;

    // decay of up to 64 heads, one per lane
    float dt_l = 0.0f, lam_l = 0.0f;
    if (bh0 + lane < nbh) {
        const int64_t bh = bh0 + lane;
        dt_l = a.dt[bh];
        lam_l = decay(dt_l, a.A[bh % a.H]);
    }
    const int hpg = a.H / a.G;
    int64_t key = -1;
    float Bv[E], Cv[E];

    // state of the current row (prefetched one iteration ahead)
    uint32_t cw[NW];
    float hv[Tr::quant ? 1 : E];
    float s_old = 0.0f, z_old = 0.0f, xv;
    auto load_row = [&](int64_t it, uint32_t* w, float* hf, float& s, float& z, float& xx) {
        const int64_t row = it * RPW + sub;
        if constexpr (Tr::quant) {
            load_words<NW>(a.codes + row * ROWB + part * (NW * 4), w);
            s = a.scale[row];
            if constexpr (Tr::asym) z = a.zero[row];
        } else {
            load_f32<E>(a.h32 + row * 128 + part * E, hf);
        }
        xx = a.x[row];
    };
    load_row(it0, cw, hv, s_old, z_old, xv);

    for (int64_t it = it0; it < it1; ++it) {
        const int64_t row0 = it * RPW;
        const int64_t bh = row0 / a.P;
        const int b = (int)(bh / a.H), h = (int)(bh % a.H);
        const int64_t k = (int64_t)b * a.G + h / hpg;
        if (k != key) {
            key = k;
            load_f32<E>(a.Bm + k * 128 + part * E, Bv);
            load_f32<E>(a.Cm + k * 128 + part * E, Cv);
        }
        const int li = (int)(bh - bh0);
        const float lam = readlane_f(lam_l, li);
        const float dtv = readlane_f(dt_l, li);
        const float Dh = a.D[h];
        const int64_t row = row0 + sub;

        // prefetch the next row
        uint32_t nw[NW];
        float nh[Tr::quant ? 1 : E];
        float ns = 0.0f, nz = 0.0f, nx = 0.0f;
        if (it + 1 < it1) load_row(it + 1, nw, nh, ns, nz, nx);

        const float w = dtv * xv;
        const float dx = Dh * xv;
        if constexpr (Tr::quant) {
            uint32_t ow[NW];
            RowGrid g;
            bool slow_any;
            float acc = RS::run_q(cw, s_old, z_old, lam, w, Bv, Cv, ow, g, slow_any);
            acc = group_sum<LPR>(acc);
            float csum = 0.0f;
            if (!PRE && Tr::asym && __any(g.zadj != 0.0f)) csum = row_csum<LPR, E>(Cv);
            store_words<NW>(a.codes + row * ROWB + part * (NW * 4), ow);
            if (part == 0) {
                a.scale[row] = g.s;
                if constexpr (Tr::asym) a.zero[row] = g.z;
                a.y[row] = row_y<F, PRE>(acc, g, csum, dx);
            }
        } else {
            float acc = RS::run_f(hv, lam, w, Bv, Cv);
            acc = group_sum<LPR>(acc);
            store_f32<E>(a.h32 + row * 128 + part * E, hv);
            if (part == 0) a.y[row] = acc + dx;
        }

        if (it + 1 < it1) {
#pragma unroll
            for (int i = 0; i < NW; ++i) cw[i] = nw[i];
            if constexpr (!Tr::quant) {
#pragma unroll
                for (int e = 0; e < E; ++e) hv[e] = nh[e];
            }
            s_old = ns;
            z_old = nz;
            xv = nx;
        }
    }
}

// ---------------------------------------------------------------------------
// fused scan: each wave keeps one iteration's rows in registers for T tokens
// ---------------------------------------------------------------------------
template <int F, int LPR, bool PRE>
__global__ __launch_bounds__(256) void k_m2_scan(M2Args a)
{
    using Tr = Traits<F>;
    using RS = RowStep<F, LPR, PRE>;
    constexpr int E = RS::E, NW = RS::NW, RPW = 64 / LPR, ROWB = RowBytes<F>::value;
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it = wave_id();
    if (it >= a.total_iters) return;
    const int64_t row0 = it * RPW;
    const int64_t bh = row0 / a.P;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const int g = h / (a.H / a.G);
    const int64_t row = row0 + sub;
    const int p = (int)(row % a.P);
    const int T = a.T, H = a.H, P = a.P, G = a.G;
    const float Ah = a.A[h], Dh = a.D[h];

    uint32_t cw[NW];
    float hv[Tr::quant ? 1 : E];
    float s = 0.0f, z = 0.0f;
    if constexpr (Tr::quant) {
        load_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw);
        s = a.scale[row];
        if constexpr (Tr::asym) z = a.zero[row];
    } else {
        load_f32<E>(a.h32 + row * 128 + part * E, hv);
    }

    auto bc_ptr = [&](const float* base, int t) { return base + (((int64_t)b * T + t) * G + g) * 128 + part * E; };
    auto x_idx = [&](int t) { return (((int64_t)b * T + t) * H + h) * P + p; };

    float Bv[E], Cv[E], xv;
    load_f32<E>(bc_ptr(a.Bm, 0), Bv);
    load_f32<E>(bc_ptr(a.Cm, 0), Cv);
    xv = a.x[x_idx(0)];
    float dt_l = 0.0f, lam_l = 0.0f;

    for (int t = 0; t < T; ++t) {
        if ((t & 63) == 0) {
            const int tt = t + lane;
            if (tt < T) {
                dt_l = a.dt[((int64_t)b * T + tt) * H + h];
                lam_l = decay(dt_l, Ah);
            }
        }
        const float lam = readlane_f(lam_l, t & 63);
        const float dtv = readlane_f(dt_l, t & 63);

        // prefetch the next token's inputs
        float nB[E], nC[E], nx = 0.0f;
        if (t + 1 < T) {
            load_f32<E>(bc_ptr(a.Bm, t + 1), nB);
            load_f32<E>(bc_ptr(a.Cm, t + 1), nC);
            nx = a.x[x_idx(t + 1)];
        }

        const float w = dtv * xv;
        const float dx = Dh * xv;
        float yv;
        if constexpr (Tr::quant) {
            uint32_t ow[NW];
            RowGrid gr;
            bool slow_any;
            float acc = RS::run_q(cw, s, z, lam, w, Bv, Cv, ow, gr, slow_any);
            acc = group_sum<LPR>(acc);
            float csum = 0.0f;
            if (!PRE && Tr::asym && __any(gr.zadj != 0.0f)) csum = row_csum<LPR, E>(Cv);
            yv = row_y<F, PRE>(acc, gr, csum, dx);
#pragma unroll
            for (int i = 0; i < NW; ++i) cw[i] = ow[i];
            s = gr.s;
            z = gr.z;
        } else {
            float acc = RS::run_f(hv, lam, w, Bv, Cv);
            yv = group_sum<LPR>(acc) + dx;
        }
        if (part == 0) a.y[x_idx(t)] = yv;

        if (t + 1 < T) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                Bv[e] = nB[e];
                Cv[e] = nC[e];
            }
            xv = nx;
        }
    }

    if constexpr (Tr::quant) {
        store_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw);
        if (part == 0) {
            a.scale[row] = s;
            if constexpr (Tr::asym) a.zero[row] = z;
        }
    } else {
        store_f32<E>(a.h32 + row * 128 + part * E, hv);
    }
}

// ---------------------------------------------------------------------------
// quantize fp32 rows into a state (state initialisation), and dequantize
// ---------------------------------------------------------------------------
template <int F, int LPR>
__global__ __launch_bounds__(256) void k_quantize_rows(QArgs a)
{
    using Tr = Traits<F>;
    constexpr int E = 128 / LPR, RPW = 64 / LPR, NW = Tr::quant ? E * Tr::bits / 32 : E;
    constexpr int ROWB = RowBytes<F>::value;
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it = wave_id();
    const int64_t row = it * RPW + sub;
    if (row >= a.rows) return; // whole row groups leave together, so DPP never reads an idle lane
    float h[E];
    load_f32<E>(a.in + row * 128 + part * E, h);
    if constexpr (!Tr::quant) {
        store_f32<E>(a.h32 + row * 128 + part * E, h);
    } else {
        float mn = 0.0f, mx = 0.0f, am = 0.0f;
        if constexpr (Tr::asym) {
            mn = h[0];
            mx = h[0];
#pragma unroll
            for (int e = 1; e < E; ++e) {
                mn = fminf(mn, h[e]);
                mx = fmaxf(mx, h[e]);
            }
            mn = group_min<LPR>(mn);
            mx = group_max<LPR>(mx);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) am = fmaxf(am, fabsf(h[e]));
            am = group_max<LPR>(am);
        }
        const RowGrid g = refit<F>(mn, mx, am);
        const bool slow_any = Tr::asym && __any(g.slow);
        float f[E];
        round_codes<F, E>(h, g, slow_any, f);
        uint32_t ow[NW];
        pack_codes<F, E>(f, ow);
        store_words<NW>(a.codes + row * ROWB + part * (NW * 4), ow);
        if (part == 0) {
            a.scale[row] = g.s;
            if constexpr (Tr::asym) a.zero[row] = g.z;
        }
    }
}

template <int F, int LPR>
__global__ __launch_bounds__(256) void k_dequant_rows(QArgs a)
{
    using Tr = Traits<F>;
    constexpr int E = 128 / LPR, RPW = 64 / LPR, NW = Tr::quant ? E * Tr::bits / 32 : E;
    constexpr int ROWB = RowBytes<F>::value;
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it = wave_id();
    const int64_t row = it * RPW + sub;
    if (row >= a.rows) return;
    float h[E];
    if constexpr (!Tr::quant) {
        load_f32<E>(a.h32 + row * 128 + part * E, h);
    } else {
        uint32_t cw[NW];
        load_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw);
        unpack_codes<F, E>(cw, h);
        const float s = a.scale[row];
        const float z = Tr::asym ? a.zero[row] : 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float d = Tr::asym ? h[e] - z : h[e];
            h[e] = s * d;
        }
    }
    store_f32<E>(a.out + row * 128 + part * E, h);
}

__global__ __launch_bounds__(256) void k_zero_fill(uint4* p, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int F>
constexpr int lanes_per_row()
{
    return F == FP32 ? 16 : (Traits<F>::bits == 8 ? 8 : 4);
}

template <int F>
static hipError_t launch_step_f(M2Args a, bool pre, int num_cus, hipStream_t st)
{
    constexpr int LPR = lanes_per_row<F>();
    constexpr int RPW = 64 / LPR;
    a.total_iters = (int64_t)a.Bsz * a.H * a.P / RPW;
    // enough waves to fill every CU several times over; each wave then walks a contiguous range
    const int64_t target_waves = (int64_t)num_cus * 16;
    int64_t ipw = (a.total_iters + target_waves - 1) / target_waves;
    // a wave's rows span at most ipw*RPW/P + 1 heads; with ipw <= 32, RPW <= 16 <= P that is
    // at most 33, so the per-head decay fits one lane per head
    if (ipw < 1) ipw = 1;
    if (ipw > 32) ipw = 32;
    a.iters_per_wave = (int)ipw;
    const int64_t waves = (a.total_iters + ipw - 1) / ipw;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (pre)
        hipLaunchKernelGGL((k_m2_step<F, LPR, true>), dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_m2_step<F, LPR, false>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_m2_step(int fmt, M2Args a, bool pre, int num_cus, hipStream_t st)
{
    switch (fmt) {
    case FP32: return launch_step_f<FP32>(a, pre, num_cus, st);
    case INT8_SYM: return launch_step_f<INT8_SYM>(a, pre, num_cus, st);
    case INT8_ASYM: return launch_step_f<INT8_ASYM>(a, pre, num_cus, st);
    case INT4_SYM: return launch_step_f<INT4_SYM>(a, pre, num_cus, st);
    case INT4_ASYM: return launch_step_f<INT4_ASYM>(a, pre, num_cus, st);
    }
    return hipErrorInvalidValue;
}

template <int F>
static hipError_t launch_scan_f(M2Args a, bool pre, hipStream_t st)
{
    constexpr int LPR = lanes_per_row<F>();
    constexpr int RPW = 64 / LPR;
    a.total_iters = (int64_t)a.Bsz * a.H * a.P / RPW;
    a.iters_per_wave = 1;
    const unsigned blocks = (unsigned)((a.total_iters + 3) / 4);
    if (pre)
        hipLaunchKernelGGL((k_m2_scan<F, LPR, true>), dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_m2_scan<F, LPR, false>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_m2_scan(int fmt, M2Args a, bool pre, hipStream_t st)
{
    switch (fmt) {
    case FP32: return launch_scan_f<FP32>(a, pre, st);
    case INT8_SYM: return launch_scan_f<INT8_SYM>(a, pre, st);
    case INT8_ASYM: return launch_scan_f<INT8_ASYM>(a, pre, st);
    case INT4_SYM: return launch_scan_f<INT4_SYM>(a, pre, st);
    case INT4_ASYM: return launch_scan_f<INT4_ASYM>(a, pre, st);
    }
    return hipErrorInvalidValue;
}

template <int F>
static hipError_t launch_rows_f(QArgs a, bool dequant, hipStream_t st)
{
    constexpr int LPR = lanes_per_row<F>();
    constexpr int RPW = 64 / LPR;
    const int64_t waves = (a.rows + RPW - 1) / RPW;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (dequant)
        hipLaunchKernelGGL((k_dequant_rows<F, LPR>), dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_quantize_rows<F, LPR>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_rows(int fmt, QArgs a, bool dequant, hipStream_t st)
{
    switch (fmt) {
    case FP32: return launch_rows_f<FP32>(a, dequant, st);
    case INT8_SYM: return launch_rows_f<INT8_SYM>(a, dequant, st);
    case INT8_ASYM: return launch_rows_f<INT8_ASYM>(a, dequant, st);
    case INT4_SYM: return launch_rows_f<INT4_SYM>(a, dequant, st);
    case INT4_ASYM: return launch_rows_f<INT4_ASYM>(a, dequant, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)p, n16);
    return hipGetLastError();
}

} // namespace ssq
