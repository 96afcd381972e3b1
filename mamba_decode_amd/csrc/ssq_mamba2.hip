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
// one row, one token: dequantize, decay + write, refit, round, pack, read out.
// ---------------------------------------------------------------------------
template <int F, int LPR, bool PRE>
struct RowStep {
    static constexpr int E = 128 / LPR;
    static constexpr int NW = Traits<F>::quant ? E * Traits<F>::bits / 32 : E;

    // B and C of the current (sequence, group): E consecutive entries each
    struct RowIn {
        float B[E];
        float C[E];
        __device__ __forceinline__ void load(const float* Bp, const float* Cp)
        {
            load_f32<E>(Bp, B);
            load_f32<E>(Cp, C);
        }
    };

    // quantized formats: the old codes as floats (h, overwritten) in -> the new packed codes
    // ow out; returns y (valid in every lane of the row).  ls = fl(lambda*s) and
    // lz = fl(ls*z) of the old row, w = fl(dt*x), dx = fl(D*x).
    __device__ __forceinline__ static float run_q(float* h, float ls, float lz, float w, float dx,
                                                  const RowIn& in, uint32_t* ow, RowGrid& g)
    {
        using Tr = Traits<F>;
        // lambda*s*(c - z) + w*B = fma(ls, c, fma(w, B, -ls*z)): the decay acts on the scale
        if constexpr (Tr::asym) {
#pragma unroll
            for (int e = 0; e < E; ++e) h[e] = __builtin_fmaf(ls, h[e], __builtin_fmaf(w, in.B[e], -lz));
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float wb = w * in.B[e];
                h[e] = __builtin_fmaf(ls, h[e], wb);
            }
        }
        float acc = 0.0f;
        if constexpr (PRE) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc = __builtin_fmaf(in.C[e], h[e], acc);
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
        // h becomes f = 1.5*2^23 + code in place
        bool slow_any = false;
        if (__all(refit_fast<F>(mn, mx, am, g))) {
            // every row of the wave is inside the verified ranges and needs no clamp
#pragma unroll
            for (int e = 0; e < E; ++e) h[e] = __builtin_fmaf(h[e], g.inv, g.Mz);
        } else {
            g = refit<F>(mn, mx, am);
            slow_any = Tr::asym && __any(g.slow);
            round_codes<F, E>(h, g, slow_any, h);
        }
        pack_codes<F, E>(h, ow);
        if constexpr (PRE) return group_sum<LPR>(acc) + dx;
        // y = s * sum_n C_n*(c_n - z) + dx, read from the new codes
        if (!slow_any) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc = __builtin_fmaf(in.C[e], h[e] - g.Mz, acc);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) acc = __builtin_fmaf(in.C[e], code_minus_z(h[e], g), acc);
        }
        acc = group_sum<LPR>(acc);
        if (__any(g.zadj != 0.0f)) {
            // a degenerate row codes everything as 0 around z = 0 but stands for the constant -z*s
            float cs = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) cs += in.C[e];
            acc = acc - g.zadj * group_sum<LPR>(cs);
        }
        return g.s * acc + dx;
    }

    // fp32 control: hv in/out, returns y
    __device__ __forceinline__ static float run_f(float* hv, float lam, float w, float dx, const RowIn& in)
    {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float wb = w * in.B[e];
            hv[e] = __builtin_fmaf(lam, hv[e], wb);
            acc = __builtin_fmaf(in.C[e], hv[e], acc);
        }
        return group_sum<LPR>(acc) + dx;
    }
};

// ---------------------------------------------------------------------------
// decode step
// ---------------------------------------------------------------------------
// Wave w takes iterations [it_base + w*K, it_base + (w+1)*K), all of them
// valid, as straight-line code: the state words of iteration i + D are loaded
// while iteration i is processed.  With no loop and no optional store, the
// compiler's s_waitcnt before each use covers exactly the loads that use needs;
// a loop-carried prefetch made it wait for younger loads as well.  Every lane
// of a row stores the row's scale, zero point and y (the same value to the same
// address), so no store sits behind a branch either.  Leftover iterations (fewer
// than K) are run by a second launch with K = 1.
template <int F, int LPR, bool PRE, int K, int D>
__global__ __launch_bounds__(256) void k_m2_step(M2Args a, int64_t it_base)
{
    using Tr = Traits<F>;
    using RS = RowStep<F, LPR, PRE>;
    constexpr int E = RS::E, NW = RS::NW, RPW = 64 / LPR, ROWB = RowBytes<F>::value;
    constexpr int NS = Tr::quant ? NW : E; // registers per slot for the row's words
    constexpr int DD = D < K ? D : K;
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it0 = it_base + wave_id() * K;
    if (it0 + K > a.total_iters) return;

    const int ipH = a.P / RPW; // iterations per head (RPW divides P)
    int64_t bh = it0 / ipH;
    int jh = (int)(it0 - bh * ipH);
    int h = (int)(bh % a.H);
    int64_t b = bh / a.H;
    const int64_t nbh = (int64_t)a.Bsz * a.H;
    const int hpg = a.H / a.G;
    int gi = h / hpg, hg = h - gi * hpg; // B/C group of head h and the head's place in it

    uint32_t ring[DD][NS];
    float rs[DD], rz[DD], rx[DD];
    auto issue = [&](int slot, int64_t it) {
        const int64_t row = it * RPW + sub;
        if constexpr (Tr::quant) {
            load_words<NW>(a.codes + row * ROWB + part * (NW * 4), ring[slot]);
            rs[slot] = ld_stream(a.scale + row);
            if constexpr (Tr::asym) rz[slot] = ld_stream(a.zero + row);
            else rz[slot] = 0.0f;
        } else {
            load_f32<E>(a.h32 + row * 128 + part * E, reinterpret_cast<float*>(ring[slot]));
            rs[slot] = 0.0f;
            rz[slot] = 0.0f;
        }
        rx[slot] = a.x[row];
    };
    // decay, dt and D of the heads this wave covers (at most K*RPW/P + 1 <= 64), one per lane,
    // read by the iterations with v_readlane; and B, C of the first row.  Issued before the
    // state prefetches: the memory counter retires in order, so waiting for these does not
    // wait for the prefetches.
    const int64_t bh0 = bh;
    float dt_l = 0.0f, A_l = 0.0f, d_l = 0.0f;
    if (bh0 + lane < nbh) {
        const int64_t q = bh0 + lane;
        const int hq = (int)(q % a.H);
        dt_l = a.dt[q];
        A_l = a.A[hq];
        d_l = a.D[hq];
    }
    int64_t key = b * a.G + gi;
    typename RS::RowIn rin;
    rin.load(a.Bm + key * 128 + part * E, a.Cm + key * 128 + part * E);
#pragma unroll
    for (int j = 0; j < DD; ++j) issue(j, it0 + j);
    const float lam_l = decay(dt_l, A_l);

#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int j = i % DD;
        const int64_t it = it0 + i;
        const int64_t row = it * RPW + sub;
        const int li = (int)(bh - bh0);
        const float lam = readlane_f(lam_l, li);
        const float dtv = readlane_f(dt_l, li);
        const float Dh = readlane_f(d_l, li);
        float cf[E];
        if constexpr (Tr::quant) unpack_codes<F, E>(ring[j], cf);
        else {
#pragma unroll
            for (int e = 0; e < E; ++e) cf[e] = __uint_as_float(ring[j][e]);
        }
        const float w = dtv * rx[j];
        const float dx = Dh * rx[j];
        const float ls = lam * rs[j];
        const float lz = ls * rz[j];
        if (i + DD < K) issue(j, it + DD);

        const int64_t k = b * a.G + gi;
        if (k != key) {
            // the wave crossed into another sequence or group: new B and C
            key = k;
            rin.load(a.Bm + k * 128 + part * E, a.Cm + k * 128 + part * E);
            wait_vmem_all();
        }
        if constexpr (Tr::quant) {
            uint32_t ow[NW];
            RowGrid g;
            const float yv = RS::run_q(cf, ls, lz, w, dx, rin, ow, g);
            store_words<NW>(a.codes + row * ROWB + part * (NW * 4), ow);
            st_stream(a.scale + row, g.s);
            if constexpr (Tr::asym) st_stream(a.zero + row, g.z);
            a.y[row] = yv;
        } else {
            const float yv = RS::run_f(cf, lam, w, dx, rin);
            store_f32<E>(a.h32 + row * 128 + part * E, cf);
            a.y[row] = yv;
        }
        if (++jh == ipH) {
            jh = 0;
            ++bh;
            if (++h == a.H) {
                h = 0;
                ++b;
                gi = 0;
                hg = 0;
            } else if (++hg == hpg) {
                hg = 0;
                ++gi;
            }
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

    // B/C of the current token; the next token's raw B/C are prefetched
    typename RS::RowIn rin;
    rin.load(bc_ptr(a.Bm, 0), bc_ptr(a.Cm, 0));
    float xv = a.x[x_idx(0)];
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
            float cf[E];
            unpack_codes<F, E>(cw, cf);
            const float ls = lam * s;
            const float lz = ls * z;
            yv = RS::run_q(cf, ls, lz, w, dx, rin, ow, gr);
#pragma unroll
            for (int i = 0; i < NW; ++i) cw[i] = ow[i];
            s = gr.s;
            z = gr.z;
        } else {
            yv = RS::run_f(hv, lam, w, dx, rin);
        }
        if (part == 0) a.y[x_idx(t)] = yv;

        if (t + 1 < T) {
#pragma unroll
            for (int e = 0; e < E; ++e) rin.B[e] = nB[e];
#pragma unroll
            for (int e = 0; e < E; ++e) rin.C[e] = nC[e];
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
// lanes per 128-entry row (each lane then holds 128/LPR entries) and the depth
// of the decode step's prefetch ring: build-time tuning knobs
#ifndef SSQ_LPR_INT4
#define SSQ_LPR_INT4 4
#endif
#ifndef SSQ_LPR_INT8
#define SSQ_LPR_INT8 4
#endif
#ifndef SSQ_LPR_FP32
#define SSQ_LPR_FP32 16
#endif
template <int F>
constexpr int lanes_per_row()
{
    return F == FP32 ? SSQ_LPR_FP32 : (Traits<F>::bits == 8 ? SSQ_LPR_INT8 : SSQ_LPR_INT4);
}

// iterations per wave (straight-line code) and prefetch distance of the decode
// step, per code width
#ifndef SSQ_ITERS_INT4
#define SSQ_ITERS_INT4 16
#endif
#ifndef SSQ_RING_INT4
#define SSQ_RING_INT4 4
#endif
#ifndef SSQ_ITERS_INT8
#define SSQ_ITERS_INT8 8
#endif
#ifndef SSQ_RING_INT8
#define SSQ_RING_INT8 3
#endif
#ifndef SSQ_ITERS_FP32
#define SSQ_ITERS_FP32 8
#endif
#ifndef SSQ_RING_FP32
#define SSQ_RING_FP32 3
#endif

template <int F>
constexpr int step_iters()
{
    return F == FP32 ? SSQ_ITERS_FP32 : (Traits<F>::bits == 8 ? SSQ_ITERS_INT8 : SSQ_ITERS_INT4);
}
template <int F>
constexpr int step_ring()
{
    return F == FP32 ? SSQ_RING_FP32 : (Traits<F>::bits == 8 ? SSQ_RING_INT8 : SSQ_RING_INT4);
}

template <int F, bool PRE>
static hipError_t launch_step_fp(M2Args a, hipStream_t st)
{
    constexpr int LPR = lanes_per_row<F>();
    constexpr int RPW = 64 / LPR;
    a.total_iters = (int64_t)a.Bsz * a.H * a.P / RPW;
    constexpr int kStepIters = step_iters<F>();
    constexpr int kStepRing = step_ring<F>();
    static_assert(kStepRing >= 1 && kStepRing <= kStepIters, "prefetch ring deeper than the iterations");
    a.iters_per_wave = kStepIters;
    // main launch: whole groups of K iterations per wave
    const int64_t main_waves = a.total_iters / kStepIters;
    if (main_waves > 0) {
        const unsigned blocks = (unsigned)((main_waves + 3) / 4);
        hipLaunchKernelGGL((k_m2_step<F, LPR, PRE, kStepIters, kStepRing>), dim3(blocks), dim3(256), 0, st, a,
                           (int64_t)0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // leftover iterations, one per wave
    const int64_t done = main_waves * kStepIters;
    const int64_t rest = a.total_iters - done;
    if (rest > 0) {
        const unsigned blocks = (unsigned)((rest + 3) / 4);
        hipLaunchKernelGGL((k_m2_step<F, LPR, PRE, 1, 1>), dim3(blocks), dim3(256), 0, st, a, done);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int F>
static hipError_t launch_step_f(M2Args a, bool pre, int /*num_cus*/, hipStream_t st)
{
    return pre ? launch_step_fp<F, true>(a, st) : launch_step_fp<F, false>(a, st);
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
