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
// one contiguous run of rows.  The decode kernel gives each wave a fixed run
// of consecutive iterations; B and C of the current (sequence, group) are
// staged once in the wave's own slice of LDS (quantized formats; registers for
// fp32) and re-read by every row, and the per-head decay is computed once for
// up to 64 heads in parallel lanes and broadcast with v_readlane.  The codes of
// later iterations are in flight while the current one is processed.  Waves
// share nothing, so there is no barrier; row reductions are DPP within the
// row's lane group.
#include <type_traits>

#include "ssq_device.h"
#include "ssq_internal.h"

namespace ssq {

// lanes per 128-entry row (each lane then holds 128/LPR entries): build-time tuning knobs.
// The scan, prefill and row kernels use lanes_per_row, the decode step step_lanes_per_row.
#ifndef SSQ_LPR_INT4
#define SSQ_LPR_INT4 4
#endif
#ifndef SSQ_LPR_INT8
#define SSQ_LPR_INT8 4
#endif
#ifndef SSQ_LPR_FP32
#define SSQ_LPR_FP32 4
#endif
template <int F>
constexpr int lanes_per_row()
{
    return F == FP32 ? SSQ_LPR_FP32 : (Traits<F>::bits == 8 ? SSQ_LPR_INT8 : SSQ_LPR_INT4);
}
// The decode step spreads an int8 row over 8 lanes: a lane then holds 16 contiguous bytes
// of the row, one store instruction writes whole rows (with the write-through streaming
// policy), and shorter waves keep more rows in flight; 8B-shaped int8 step 120.8 to about
// 100 us.  The scan and prefill keep 4: they store the state once per launch, and with
// 16 entries per lane their per-token refit would cost twice the VALU per entry.
#ifndef SSQ_STEP_LPR_INT8
#define SSQ_STEP_LPR_INT8 8
#endif
template <int F>
constexpr int step_lanes_per_row()
{
    return F != FP32 && Traits<F>::bits == 8 ? SSQ_STEP_LPR_INT8 : lanes_per_row<F>();
}

// B and C of the decode step in LDS (quantized formats) rather than in registers
#ifndef SSQ_BC_LDS
#define SSQ_BC_LDS 1
#endif

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

// Workgroups are dispatched to the 8 XCDs in turn (workgroup i to XCD i mod 8), each XCD with
// its own L2.  Numbered this way instead, each XCD runs one contiguous range of rows, so the
// waves of a sequence share an XCD and its L2 fetches that sequence's B and C once per token
// rather than once per XCD.  A permutation of the waves: any grid stays correct.
__device__ __forceinline__ int64_t wave_id_xcd_grouped()
{
    constexpr int kXcds = 8;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t nb = gridDim.x, bid = blockIdx.x;
    const int64_t lb = nb % kXcds == 0 ? (bid % kXcds) * (nb / kXcds) + bid / kXcds : bid;
    return lb * (blockDim.x >> 6) + w;
}

// ---------------------------------------------------------------------------
// one row, one token: dequantize, decay + write, refit, round, pack, read out.
// ---------------------------------------------------------------------------
template <int F, int LPR, bool PRE>
struct RowStep {
    static constexpr int E = 128 / LPR;
    static constexpr int NW = Traits<F>::quant ? E * Traits<F>::bits / 32 : E;

    // B and C of the current (sequence, group): E consecutive entries each, in registers
    struct RowIn {
        float B[E];
        float C[E];
        __device__ __forceinline__ void load(const float* Bp, const float* Cp)
        {
            load_f32<E>(Bp, B);
            load_f32<E>(Cp, C);
        }
        __device__ __forceinline__ float b(int e) const { return B[e]; }
        __device__ __forceinline__ float c(int e) const { return C[e]; }
        __device__ __forceinline__ float4 b4(int q) const { return make_float4(B[4 * q], B[4 * q + 1], B[4 * q + 2], B[4 * q + 3]); }
        __device__ __forceinline__ float4 c4(int q) const { return make_float4(C[4 * q], C[4 * q + 1], C[4 * q + 2], C[4 * q + 3]); }
    };
    // ... or in LDS: the wave's copy of B and C, E entries per lane group, rows of E + 4
    // floats so that the LPR groups' 16-byte reads fall in different banks
    static constexpr int LDS_PITCH = E + 4;
    static constexpr int LDS_FLOATS = LPR * LDS_PITCH;
    struct RowInLds {
        const float* Bp; // this lane's E entries of B in LDS, 16-byte aligned
        const float* Cp;
        __device__ __forceinline__ float b(int e) const { return Bp[e]; }
        __device__ __forceinline__ float c(int e) const { return Cp[e]; }
        // four entries with one 16-byte read: written out, so that no inline asm in a loop
        // that uses them keeps the compiler from merging the reads
        __device__ __forceinline__ float4 b4(int q) const { return reinterpret_cast<const float4*>(Bp)[q]; }
        __device__ __forceinline__ float4 c4(int q) const { return reinterpret_cast<const float4*>(Cp)[q]; }
    };

    // The readout sum of E entries of this lane and its row's other lanes, sum_n C_n*val(n).
    // Each lane sums chains of CH consecutive entries with fmas from zero; with two chains per
    // lane their sum is taken first, then the lanes' partial sums meet in the DPP tree of
    // group_sum.  A lane holding 2*CH entries on LPR lanes thus adds in the same order as one
    // holding CH entries on 2*LPR lanes: the scan (4 lanes per int8 row) returns the y of the
    // decode step (8 lanes per int8 row) bit for bit.
    template <int CH, typename In, typename V>
    __device__ __forceinline__ static float readout(const In& in, V val)
    {
        static_assert(E % CH == 0 && (E / CH == 1 || E / CH == 2), "one or two readout chains per lane");
        float a0 = 0.0f;
#pragma unroll
        for (int e = 0; e < CH; ++e) a0 = __builtin_fmaf(in.c(e), val(e), a0);
        if constexpr (E / CH == 2) {
            float a1 = 0.0f;
#pragma unroll
            for (int e = CH; e < E; ++e) a1 = __builtin_fmaf(in.c(e), val(e), a1);
            a0 = a0 + a1;
        }
        return group_sum<LPR>(a0);
    }

    // Quantized formats, one token.  d: the stored row up to its scale, d_n = fl(c_n - z) (the
    // code itself on the symmetric grid), overwritten; s: the row's scale; lam = fl32(exp(dt*A)),
    // w = fl(dt*x), dx = fl(D*x).  Every entry is reconstructed, hh_n = fl(s*d_n), and the fp32
    // recurrence runs on it, h'_n = fma(lam, hh_n, fl(w*B_n)); the row is then refit and
    // rounded, and y is read from the new codes (or from h' with PRE).  Returns y (valid in
    // every lane of the row).
    // PACK: the new codes are packed into ow; otherwise d ends holding fl(c'_n - z') of the
    // new row, what the next token of a scan starts from.  SR: round stochastically with the
    // uniforms of counters ctr0 .. ctr0 + E - 1.  CH: entries per readout chain (readout()).
    template <bool PACK = true, bool SR = false, int CH = E, typename In>
    __device__ __forceinline__ static float run_q(float* d, float s, float lam, float w, float dx,
                                                  const In& in, uint32_t* ow, RowGrid& g, uint64_t sr_seed = 0,
                                                  uint64_t ctr0 = 0)
    {
        using Tr = Traits<F>;
        float* const h = d;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float hh = s * d[e];
            const float wb = w * in.b(e);
            h[e] = __builtin_fmaf(lam, hh, wb);
        }
        float y_pre = 0.0f;
        if constexpr (PRE) y_pre = readout<CH>(in, [&](int e) { return h[e]; });
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
        const bool fast = __all(refit_fast<F, SR>(mn, mx, am, g));
        if (fast) {
            // every row of the wave is inside the verified ranges and needs no clamp
            if constexpr (SR) {
                round_codes_sr<F, E, true>(h, g, sr_seed, ctr0, h);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) h[e] = __builtin_fmaf(h[e], g.inv, g.Mz);
            }
        } else {
            g = refit<F>(mn, mx, am);
            if constexpr (SR) {
                round_codes_sr<F, E, false>(h, g, sr_seed, ctr0, h);
            } else {
                const bool slow_any = Tr::asym && __any(g.slow);
                round_codes<F, E>(h, g, slow_any, h);
            }
        }
        if constexpr (PACK) pack_codes<F, E>(h, ow);
        // h becomes d'_n = fl(c'_n - z') of the new row: f - Mr on the fast path, where
        // |z'| < 2^21 makes Mr = 1.5*2^23 + z' and the difference exact; (f - 1.5*2^23) - z'
        // otherwise.  It is the next token's input in a scan and the readout's operand:
        // y = s' * sum_n C_n*d'_n + dx.
        if constexpr (!PACK || !PRE) {
            if (fast) {
#pragma unroll
                for (int e = 0; e < E; ++e) h[e] = h[e] - g.Mr;
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) h[e] = (h[e] - kMagic) - g.z;
            }
        }
        if constexpr (PRE) return y_pre + dx;
        return g.s * readout<CH>(in, [&](int e) { return h[e]; }) + dx;
    }

    // refit and round the fp32 row h in place: h becomes f = 1.5*2^23 + code, g the new grid
    template <bool SR>
    __device__ __forceinline__ static void requant(float* h, RowGrid& g, uint64_t sr_seed, uint64_t ctr0)
    {
        using Tr = Traits<F>;
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
        if (__all(refit_fast<F, SR>(mn, mx, am, g))) {
            if constexpr (SR) {
                round_codes_sr<F, E, true>(h, g, sr_seed, ctr0, h);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) h[e] = __builtin_fmaf(h[e], g.inv, g.Mz);
            }
        } else {
            g = refit<F>(mn, mx, am);
            if constexpr (SR) {
                round_codes_sr<F, E, false>(h, g, sr_seed, ctr0, h);
            } else {
                const bool slow_any = Tr::asym && __any(g.slow);
                round_codes<F, E>(h, g, slow_any, h);
            }
        }
    }

    // fp32 control: hv in/out, returns y
    template <typename In>
    __device__ __forceinline__ static float run_f(float* hv, float lam, float w, float dx, const In& in)
    {
        // h = fma(lambda, h, w*B) written into h's own register (fma_in_place): the
        // compiler's own form accumulates into w*B's register and copies every entry back
        float acc = 0.0f;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 b = in.b4(q), c = in.c4(q);
            const float bb[4] = {b.x, b.y, b.z, b.w}, cc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                fma_in_place(lam, hv[4 * q + k], w * bb[k]);
                acc = __builtin_fmaf(cc[k], hv[4 * q + k], acc);
            }
        }
        return group_sum<LPR>(acc) + dx;
    }
};

// Progress-based wave priority.  The waves of a SIMD share its VALU and the arbiter prefers the
// oldest ready wave, so with equal priorities the first wave of a SIMD ran ahead and finished
// after about half the launch while the last ones finished alone on a half-idle SIMD (370m
// int4 layer: waves ending 10.7-21.2 us, the last wave of every SIMD at 19.1-21.2 us).  A wave
// therefore lowers its own priority as it gets ahead: 3 for the first half of its K iterations,
// 2 for the third quarter, 1 and 0 for the two halves of the last quarter (3,3,3,3,2,2,1,0 for
// K = 8), so that the waves behind it are issued first.  Measured on the 370m int4 layer, A/B
// on one box: 7.8% faster (stochastic rounding: 10%), the 8B int4 layer unchanged; of the
// schedules tried this one was fastest (3,3,2,2,1,1,0,0: 6%; 3,2,1,0,...: 3%; the reverse
// order: no gain).  The int8 step (four iterations per wave, held by memory) keeps priority 0;
// the fp32 step (eight iterations) takes the same schedule.  SSQ_STEP_PRIO=0 switches it off.
#ifndef SSQ_STEP_PRIO
#define SSQ_STEP_PRIO 1
#endif
template <int K>
__device__ __forceinline__ void step_priority(int i)
{
    if constexpr (SSQ_STEP_PRIO != 0 && K >= 8 && K % 8 == 0) {
        if (i == 0) __builtin_amdgcn_s_setprio(3);
        else if (i == K / 2) __builtin_amdgcn_s_setprio(2);
        else if (i == 3 * K / 4) __builtin_amdgcn_s_setprio(1);
        else if (i == 7 * K / 8) __builtin_amdgcn_s_setprio(0);
    }
}

// The same for the token loop of a scan of a quantized state: 3 for the first half of the T
// tokens, then 2, 1, 0 (t is uniform, so these are scalar compares).  A/B on one box: the 130m
// int8 scans 7% faster, the 8B int4 scan 12%; the fp32 scan unchanged and the prefill 4%
// slower, so those two keep priority 0.
#ifndef SSQ_SCAN_PRIO
#define SSQ_SCAN_PRIO 1
#endif
template <bool ON>
__device__ __forceinline__ void token_priority(int t, int T)
{
    if constexpr (ON && SSQ_SCAN_PRIO != 0) {
        if (t == 0) __builtin_amdgcn_s_setprio(3);
        else if (t == T / 2) __builtin_amdgcn_s_setprio(2);
        else if (t == 3 * (T / 4)) __builtin_amdgcn_s_setprio(1);
        else if (t == 7 * (T / 8)) __builtin_amdgcn_s_setprio(0);
    }
}

// ---------------------------------------------------------------------------
// decode step
// ---------------------------------------------------------------------------
// Wave w takes iterations [it_base + w*K, it_base + (w+1)*K), all of them
// valid: the state words of iteration i + D are loaded while iteration i is
// processed.  K = 8 compiles to straight-line code, where the compiler's
// s_waitcnt before each use covers exactly the loads that use needs (a
// loop-carried prefetch made it wait for younger loads as well); the compiler
// keeps a loop for K = 16 and 32, which pay off only where they spare the
// launch later rounds of waves (see the launcher).  Every lane
// of a row stores the row's scale, zero point and y (the same value to the same
// address), so no store sits behind a branch either.  Leftover iterations (fewer
// than K) are run by a second launch with K = 1.
template <int F, int LPR, bool PRE, int K, int D, int W, bool SR>
__global__ __launch_bounds__(256, W) void k_m2_step(M2Args a, int64_t it_base)
{
    using Tr = Traits<F>;
    using RS = RowStep<F, LPR, PRE>;
    constexpr int E = RS::E, NW = RS::NW, RPW = 64 / LPR, ROWB = RowBytes<F>::value;
    constexpr int NS = Tr::quant ? NW : E; // registers per slot for the row's words
    constexpr int DD = D < K ? D : K;
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it0 = it_base + wave_id() * K; // round-robin over the XCDs: grouping the
    // decode's workgroups by XCD (as the scan does) made it 7-8% slower
    if (it0 + K > a.total_iters) return;
    const uint64_t sr_step = SR ? sr_token(a.sr) : 0;

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
    // The wave's K*RPW consecutive rows as buffer descriptors: a uniform base and range in
    // scalar registers, one fixed 32-bit offset per lane and a constant offset per
    // iteration, so that no per-iteration address occupies vector registers.
    const int64_t row_first = it0 * RPW;
    constexpr uint32_t SPAN = (uint32_t)(K * RPW);
    constexpr uint32_t WB = Tr::quant ? (uint32_t)ROWB : 512u; // state bytes per row
    const Rsrc r_w = make_rsrc(Tr::quant ? (const void*)(a.codes + row_first * ROWB)
                                         : (const void*)(a.h32 + row_first * 128), SPAN * WB);
    const Rsrc r_s = make_rsrc(a.scale + row_first, Tr::quant ? SPAN * 4 : 0);
    const Rsrc r_z = make_rsrc(a.zero + row_first, Tr::asym ? SPAN * 4 : 0);
    const Rsrc r_x = make_rsrc(a.x + row_first, SPAN * 4);
    const Rsrc r_y = make_rsrc(a.y + row_first, SPAN * 4);
    const uint32_t off_w = (uint32_t)(sub * WB + part * (Tr::quant ? NW * 4 : E * 4));
    const uint32_t off_r = (uint32_t)(sub * 4);
    auto issue = [&](int slot, int i) {
        const uint32_t sw = (uint32_t)i * RPW * WB, sr = (uint32_t)i * RPW * 4;
        if constexpr (Tr::quant) {
            buf_load_words<NW, kAuxLoad>(r_w, off_w, sw, ring[slot]);
            rs[slot] = buf_load_f32<kAuxLoad>(r_s, off_r, sr);
            if constexpr (Tr::asym) rz[slot] = buf_load_f32<kAuxLoad>(r_z, off_r, sr);
            else rz[slot] = 0.0f;
        } else {
            buf_load_words<E, 0>(r_w, off_w, sw, ring[slot]); // fp32 rows: no hint
            rs[slot] = 0.0f;
            rz[slot] = 0.0f;
        }
        rx[slot] = buf_load_f32<0>(r_x, off_r, sr);
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
    // B and C: in this wave's slice of LDS (each lane staging two entries of each), or in
    // registers when built with SSQ_BC_LDS=0
    constexpr bool BCL = SSQ_BC_LDS != 0;
    constexpr int PITCH = RS::LDS_PITCH, LDSF = RS::LDS_FLOATS;
    __shared__ float4 bc_lds[BCL ? 4 * 2 * LDSF / 4 : 1];
    float* const lds_b = reinterpret_cast<float*>(bc_lds) + (threadIdx.x >> 6) * (2 * LDSF);
    float* const lds_c = lds_b + LDSF;
    typename RS::RowIn rin;
    const typename RS::RowInLds rin_l{lds_b + part * PITCH, lds_c + part * PITCH};
    float2 bv, cv;
    auto bc_fetch = [&](int64_t k) {
        bv = *reinterpret_cast<const float2*>(a.Bm + k * 128 + 2 * lane);
        cv = *reinterpret_cast<const float2*>(a.Cm + k * 128 + 2 * lane);
    };
    // Lanes write entries that other lanes of the wave read: each write is ordered after the
    // wave's earlier reads of the slice and before its later ones (wave_lds_sync).
    auto bc_stage = [&]() {
        const int n = 2 * lane, off = (n / E) * PITCH + n % E;
        wave_lds_sync();
        *reinterpret_cast<float2*>(lds_b + off) = bv;
        *reinterpret_cast<float2*>(lds_c + off) = cv;
        wave_lds_sync();
    };
    if constexpr (BCL) bc_fetch(key);
    else rin.load(a.Bm + key * 128 + part * E, a.Cm + key * 128 + part * E);
#ifndef SSQ_STEP_FIRST
#define SSQ_STEP_FIRST 1
#endif
    // iterations whose loads go out before the decay and the B/C staging (0: all DD).  With
    // only the first one ahead of them, its rows compete with fewer requests and the rest
    // still arrive before they are needed: 0.6-0.9% faster on the 370m and 8B layers.
    constexpr int FIRST = SSQ_STEP_FIRST > 0 && SSQ_STEP_FIRST < DD ? SSQ_STEP_FIRST : DD;
#pragma unroll
    for (int j = 0; j < FIRST; ++j) issue(j, j);
    const float lam_l = decay(dt_l, A_l);
    if constexpr (BCL) bc_stage();
#pragma unroll
    for (int j = FIRST; j < DD; ++j) issue(j, j);

#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int j = i % DD;
        const uint32_t sw = (uint32_t)i * RPW * WB, sr = (uint32_t)i * RPW * 4;
        step_priority<K>(i);
        const int li = (int)(bh - bh0);
        const float lam = readlane_f(lam_l, li);
        const float dtv = readlane_f(dt_l, li);
        const float Dh = readlane_f(d_l, li);
        float cf[E]; // quantized: fl(c - z) of the stored row; fp32: the row
        if constexpr (Tr::quant) {
            unpack_codes<F, E>(ring[j], cf);
            if constexpr (Tr::asym) {
#pragma unroll
                for (int e = 0; e < E; ++e) cf[e] = cf[e] - rz[j];
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) cf[e] = __uint_as_float(ring[j][e]);
        }
        const float w = dtv * rx[j];
        const float dx = Dh * rx[j];
        const float sc = rs[j];
        if (i + DD < K) issue(j, i + DD);

        const int64_t k = b * a.G + gi;
        if (k != key) {
            // the wave crossed into another sequence or group: new B and C
            key = k;
            if constexpr (BCL) bc_fetch(k);
            else rin.load(a.Bm + k * 128 + part * E, a.Cm + k * 128 + part * E);
            wait_vmem_all();
            if constexpr (BCL) bc_stage();
        }
        if constexpr (Tr::quant) {
            uint32_t ow[NW];
            RowGrid g;
            // this lane's first counter of stochastic rounding: (step*rows + row)*128 + part*E
            const uint64_t ctr0 =
                SR ? ((sr_step * (uint64_t)a.sr.rows + (uint64_t)(row_first + (int64_t)i * RPW + sub)) * 128u +
                      (uint64_t)(part * E))
                   : 0;
            float yv;
            if constexpr (BCL) yv = RS::template run_q<true, SR>(cf, sc, lam, w, dx, rin_l, ow, g, a.sr.seed, ctr0);
            else yv = RS::template run_q<true, SR>(cf, sc, lam, w, dx, rin, ow, g, a.sr.seed, ctr0);
            // a lane's 16 bytes of a row: one store instruction writes whole rows
            constexpr int AUXS = 128 * Tr::bits / 8 / LPR == 16 ? kAuxStoreWhole : kAuxStore;
            buf_store_words<NW, AUXS>(r_w, off_w, sw, ow);
            buf_store_f32<AUXS>(g.s, r_s, off_r, sr);
            if constexpr (Tr::asym) buf_store_f32<AUXS>(g.z, r_z, off_r, sr);
            // y of 16 rows is one whole 64-byte segment: written through (sc1); 8 rows'
            // 32 bytes go without a hint
            buf_store_f32<RPW == 16 ? kAuxStoreSc1 : 0>(yv, r_y, off_r, sr);
        } else {
            float yv;
            if constexpr (BCL) yv = RS::run_f(cf, lam, w, dx, rin_l);
            else yv = RS::run_f(cf, lam, w, dx, rin);
            buf_store_words<E, 0>(r_w, off_w, sw, reinterpret_cast<const uint32_t*>(cf)); // fp32 rows: no hint
            buf_store_f32<0>(yv, r_y, off_r, sr);
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
// The rows stay on-chip as codes in float form (no packing between tokens) with
// their scale and zero point.  B and C of each token go through two LDS buffers
// per wave: token t reads buffer t&1 while token t+1's B and C, loaded during
// token t-1, are written to the other one and token t+2's are being loaded, so
// every global load has a full token of work to arrive.  All loads are
// unconditional (the token index is clamped at the end), and every lane of a
// row stores that row's y.
#ifndef SSQ_SCAN_WAVES
#define SSQ_SCAN_WAVES 4
#endif
template <int F, int LPR, bool PRE, bool SR, int W>
__global__ __launch_bounds__(256, PRE ? W - 1 : W) void k_m2_scan(M2Args a)
{
    using Tr = Traits<F>;
    using RS = RowStep<F, LPR, PRE>;
    constexpr int E = RS::E, NW = RS::NW, RPW = 64 / LPR, ROWB = RowBytes<F>::value;
    constexpr int PITCH = RS::LDS_PITCH, LDSF = RS::LDS_FLOATS;
    __shared__ float4 bc_lds[4 * 2 * 2 * LDSF / 4]; // [wave][buffer][B, C][LDSF]
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it = wave_id_xcd_grouped();
    if (it >= a.total_iters) return;
    const uint64_t sr_step = SR ? sr_token(a.sr) : 0;
    const int64_t row0 = it * RPW;
    const int64_t bh = row0 / a.P;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const int g = h / (a.H / a.G);
    const int64_t row = row0 + sub;
    const int p = (int)(row % a.P);
    const int T = a.T, H = a.H, P = a.P, G = a.G;
    const float Ah = a.A[h], Dh = a.D[h];

    // quantized: fl(c - z) of the row (the code itself on the symmetric grid), carried from
    // token to token; fp32: the row's values
    float cf[E];
    float s = 0.0f;
    if constexpr (Tr::quant) {
        uint32_t cw[NW];
        load_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw);
        s = a.scale[row];
        unpack_codes<F, E>(cw, cf);
        if constexpr (Tr::asym) {
            const float z = a.zero[row];
#pragma unroll
            for (int e = 0; e < E; ++e) cf[e] = cf[e] - z;
        }
    } else {
        load_f32<E>(a.h32 + row * 128 + part * E, cf);
    }

    float* const wl = reinterpret_cast<float*>(bc_lds) + (threadIdx.x >> 6) * (4 * LDSF);
    const int n2 = 2 * lane, st_off = (n2 / E) * PITCH + n2 % E; // this lane's two entries
    auto bc_at = [&](const float* base, int t) {
        return *reinterpret_cast<const float2*>(base + (((int64_t)b * T + t) * G + g) * 128 + n2);
    };
    // lanes write entries that other lanes read (wave_lds_sync on both sides)
    auto stage = [&](int buf, float2 bv, float2 cv) {
        wave_lds_sync();
        *reinterpret_cast<float2*>(wl + buf * (2 * LDSF) + st_off) = bv;
        *reinterpret_cast<float2*>(wl + buf * (2 * LDSF) + LDSF + st_off) = cv;
        wave_lds_sync();
    };
    auto x_idx = [&](int t) { return (((int64_t)b * T + t) * H + h) * P + p; };

    // token 0 into buffer 0; token 1 in registers
    stage(0, bc_at(a.Bm, 0), bc_at(a.Cm, 0));
    const int t1 = T > 1 ? 1 : 0;
    float2 bn = bc_at(a.Bm, t1), cn = bc_at(a.Cm, t1);
    float xv = a.x[x_idx(0)], xn = a.x[x_idx(t1)];
    float dt_l = 0.0f, lam_l = 0.0f;
    // the y readout in the decode step's summation order: chains of 128/(its lanes per row)
    constexpr int CH = 128 / step_lanes_per_row<F>();
    uint32_t ow[NW];  // the packed codes after the last token
    RowGrid gr;

    // one token; LAST packs the new codes instead of carrying fl(c - z) on
    auto token = [&](int t, auto last) {
        constexpr bool LAST = decltype(last)::value;
        token_priority<Tr::quant>(t, T);
        if ((t & 63) == 0) {
            const int tt = t + lane;
            if (tt < T) {
                dt_l = a.dt[((int64_t)b * T + tt) * H + h];
                lam_l = decay(dt_l, Ah);
            }
        }
        const float lam = readlane_f(lam_l, t & 63);
        const float dtv = readlane_f(dt_l, t & 63);

        // token t+2's inputs (clamped to the last token)
        const int t2 = t + 2 < T ? t + 2 : T - 1;
        const float2 bf = bc_at(a.Bm, t2), cf2 = bc_at(a.Cm, t2);
        const float xf = a.x[x_idx(t2)];

        const float* const cur = wl + (t & 1) * (2 * LDSF);
        const typename RS::RowInLds in{cur + part * PITCH, cur + LDSF + part * PITCH};
        const float w = dtv * xv;
        const float dx = Dh * xv;
        float yv;
        if constexpr (Tr::quant) {
            const uint64_t ctr0 =
                SR ? (((sr_step + (uint64_t)t) * (uint64_t)a.sr.rows + (uint64_t)row) * 128u + (uint64_t)(part * E))
                   : 0;
            yv = RS::template run_q<LAST, SR, CH>(cf, s, lam, w, dx, in, ow, gr, a.sr.seed, ctr0);
            s = gr.s;
        } else {
            yv = RS::run_f(cf, lam, w, dx, in);
        }
        a.y[x_idx(t)] = yv;

        // token t+1's B and C into the other buffer
        stage((t + 1) & 1, bn, cn);
        bn = bf;
        cn = cf2;
        xv = xn;
        xn = xf;
    };
    for (int t = 0; t < T - 1; ++t) token(t, std::false_type{});
    token(T - 1, std::true_type{});

    if constexpr (Tr::quant) {
        store_words<NW>(a.codes + row * ROWB + part * (NW * 4), ow);
        if (part == 0) {
            a.scale[row] = gr.s;
            if constexpr (Tr::asym) a.zero[row] = gr.z;
        }
    } else {
        store_f32<E>(a.h32 + row * 128 + part * E, cf);
    }
}

// ---------------------------------------------------------------------------
// prefill: the fp32 recurrence inside each chunk, the state quantized at chunk ends
// ---------------------------------------------------------------------------
// Same row mapping and B/C pipeline as the scan.  Each row is dequantized once,
// s*(c - z), and kept in fp32; every token applies h = fma(lambda, h, w*B) and
// reads y from it; at the end of each chunk of `chunk` tokens, and after the last
// token, the row is refit and rounded (to nearest or stochastically), y follows
// the readout flag, and the row continues from its dequantized new codes.  The
// packed codes of the last chunk end are stored once at the end.
#ifndef SSQ_PREFILL_WAVES
#define SSQ_PREFILL_WAVES 3
#endif
template <int F, int LPR, bool PRE, bool SR>
__global__ __launch_bounds__(256, PRE ? SSQ_PREFILL_WAVES - 1 : SSQ_PREFILL_WAVES) void k_m2_prefill(M2Args a, int chunk)
{
    using Tr = Traits<F>;
    static_assert(Tr::quant, "the fp32 state's prefill is the scan");
    using RS = RowStep<F, LPR, PRE>;
    constexpr int E = RS::E, NW = RS::NW, RPW = 64 / LPR, ROWB = RowBytes<F>::value;
    constexpr int PITCH = RS::LDS_PITCH, LDSF = RS::LDS_FLOATS;
    __shared__ float4 bc_lds[4 * 2 * 2 * LDSF / 4]; // [wave][buffer][B, C][LDSF]
    const int lane = threadIdx.x & 63, sub = lane / LPR, part = lane % LPR;
    const int64_t it = wave_id_xcd_grouped();
    if (it >= a.total_iters) return;
    const uint64_t sr_step = SR ? sr_token(a.sr) : 0;
    const int64_t row0 = it * RPW;
    const int64_t bh = row0 / a.P;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const int g = h / (a.H / a.G);
    const int64_t row = row0 + sub;
    const int p = (int)(row % a.P);
    const int T = a.T, H = a.H, P = a.P, G = a.G;
    const float Ah = a.A[h], Dh = a.D[h];

    uint32_t cw[NW];
    load_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw);
    float s = a.scale[row];
    float z = Tr::asym ? a.zero[row] : 0.0f;
    float hv[E];
    unpack_codes<F, E>(cw, hv);
#pragma unroll
    for (int e = 0; e < E; ++e) hv[e] = s * (hv[e] - z); // the stored row's value, fl(s*fl(c - z))

    float* const wl = reinterpret_cast<float*>(bc_lds) + (threadIdx.x >> 6) * (4 * LDSF);
    const int n2 = 2 * lane, st_off = (n2 / E) * PITCH + n2 % E;
    auto bc_at = [&](const float* base, int t) {
        return *reinterpret_cast<const float2*>(base + (((int64_t)b * T + t) * G + g) * 128 + n2);
    };
    auto stage = [&](int buf, float2 bv, float2 cv) {
        wave_lds_sync();
        *reinterpret_cast<float2*>(wl + buf * (2 * LDSF) + st_off) = bv;
        *reinterpret_cast<float2*>(wl + buf * (2 * LDSF) + LDSF + st_off) = cv;
        wave_lds_sync();
    };
    auto x_idx = [&](int t) { return (((int64_t)b * T + t) * H + h) * P + p; };

    stage(0, bc_at(a.Bm, 0), bc_at(a.Cm, 0));
    const int t1 = T > 1 ? 1 : 0;
    float2 bn = bc_at(a.Bm, t1), cn = bc_at(a.Cm, t1);
    float xv = a.x[x_idx(0)], xn = a.x[x_idx(t1)];
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
        const int t2 = t + 2 < T ? t + 2 : T - 1;
        const float2 bf = bc_at(a.Bm, t2), cf2 = bc_at(a.Cm, t2);
        const float xf = a.x[x_idx(t2)];

        const float* const cur = wl + (t & 1) * (2 * LDSF);
        const typename RS::RowInLds in{cur + part * PITCH, cur + LDSF + part * PITCH};
        const float w = dtv * xv;
        const float dx = Dh * xv;
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 b = in.b4(q);
            const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) fma_in_place(lam, hv[4 * q + k], w * bb[k]);
        }
        const bool end = (t + 1) % chunk == 0 || t == T - 1; // wave-uniform
        float acc = 0.0f;
        if (!end || PRE) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc = __builtin_fmaf(in.c(e), hv[e], acc);
        }
        if (end) {
            RowGrid gr;
            const uint64_t ctr0 =
                SR ? (((sr_step + (uint64_t)t) * (uint64_t)a.sr.rows + (uint64_t)row) * 128u + (uint64_t)(part * E))
                   : 0;
            RS::template requant<SR>(hv, gr, a.sr.seed, ctr0);
            pack_codes<F, E>(hv, cw);
            s = gr.s;
            z = gr.z;
#pragma unroll
            for (int e = 0; e < E; ++e) hv[e] = s * ((hv[e] - kMagic) - z); // fl(s*fl(c - z))
            if constexpr (!PRE) {
#pragma unroll
                for (int e = 0; e < E; ++e) acc = __builtin_fmaf(in.c(e), hv[e], acc);
            }
        }
        a.y[x_idx(t)] = group_sum<LPR>(acc) + dx;

        stage((t + 1) & 1, bn, cn);
        bn = bf;
        cn = cf2;
        xv = xn;
        xn = xf;
    }

    store_words<NW>(a.codes + row * ROWB + part * (NW * 4), cw);
    if (part == 0) {
        a.scale[row] = s;
        if constexpr (Tr::asym) a.zero[row] = z;
    }
}

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

// The state's stochastic-rounding token counter set to `value`, or advanced by `tokens` after
// a call's step kernels (one thread, through a vector atomic; kernels rather than memsets or
// copies, so that the calls may also sit in a captured graph).
__global__ __launch_bounds__(64) void k_set_counter(uint64_t* ctr, uint64_t value)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicExch(reinterpret_cast<unsigned long long*>(ctr), value);
}
__global__ __launch_bounds__(64) void k_advance_counter(uint64_t* ctr, uint64_t tokens)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicAdd(reinterpret_cast<unsigned long long*>(ctr), tokens);
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
// iterations per wave (straight-line code), prefetch distance and the waves per
// SIMD the register budget is sized for (launch bounds), per code width.  With B
// and C in LDS and buffer addressing both quantized widths fit 128 registers
// (4 waves per SIMD); int4: K = 8 makes one round of resident waves at 370m shape;
// int8 (8 rows per wave-iteration): K = 4 with every iteration's loads issued up front
// measured fastest (K = 8 with a ring of 4 about 3% slower, K = 1 or a ring of 3 about 20%;
// on the 8B-shaped layer K = 2 31% slower and K = 8 with all eight up front 9%).
#ifndef SSQ_ITERS_INT4
#define SSQ_ITERS_INT4 8
#endif
#ifndef SSQ_RING_INT4
#define SSQ_RING_INT4 4
#endif
#ifndef SSQ_WAVES_INT4
#define SSQ_WAVES_INT4 4
#endif
#ifndef SSQ_ITERS_INT8
#define SSQ_ITERS_INT8 4
#endif
#ifndef SSQ_RING_INT8
#define SSQ_RING_INT8 4
#endif
#ifndef SSQ_WAVES_INT8
#define SSQ_WAVES_INT8 4
#endif
#ifndef SSQ_ITERS_FP32
#define SSQ_ITERS_FP32 8
#endif
#ifndef SSQ_RING_FP32
#define SSQ_RING_FP32 2
#endif
#ifndef SSQ_WAVES_FP32
#define SSQ_WAVES_FP32 3
#endif

// stochastic rounding keeps the generator's state live beside the ring: its own ring depth
#ifndef SSQ_RING_INT4_SR
#define SSQ_RING_INT4_SR 2
#endif
#ifndef SSQ_RING_INT8_SR
#define SSQ_RING_INT8_SR SSQ_RING_INT8
#endif
#ifndef SSQ_WAVES_INT4_SR
#define SSQ_WAVES_INT4_SR SSQ_WAVES_INT4
#endif

template <int F>
constexpr int step_iters()
{
    return F == FP32 ? SSQ_ITERS_FP32 : (Traits<F>::bits == 8 ? SSQ_ITERS_INT8 : SSQ_ITERS_INT4);
}
template <int F, bool SR>
constexpr int step_ring()
{
    if constexpr (SR) return Traits<F>::bits == 8 ? SSQ_RING_INT8_SR : SSQ_RING_INT4_SR;
    return F == FP32 ? SSQ_RING_FP32 : (Traits<F>::bits == 8 ? SSQ_RING_INT8 : SSQ_RING_INT4);
}
// the pre-rounding readout keeps C live through the update: one wave less
template <int F, bool PRE, bool SR>
constexpr int step_waves()
{
    constexpr int w = F == FP32 ? SSQ_WAVES_FP32
                                : (Traits<F>::bits == 8 ? SSQ_WAVES_INT8 : (SR ? SSQ_WAVES_INT4_SR : SSQ_WAVES_INT4));
    return PRE && w > 2 ? w - 1 : w;
}

template <int F, bool PRE, bool SR, int kStepIters>
static hipError_t launch_step_k(M2Args a, hipStream_t st)
{
    constexpr int LPR = step_lanes_per_row<F>();
    constexpr int RPW = 64 / LPR;
    a.total_iters = (int64_t)a.Bsz * a.H * a.P / RPW;
    constexpr int kStepRing = step_ring<F, SR>();
    static_assert(kStepRing >= 1 && kStepRing <= kStepIters, "prefetch ring deeper than the iterations");
    a.iters_per_wave = kStepIters;
    // main launch: whole groups of K iterations per wave
    const int64_t main_waves = a.total_iters / kStepIters;
    if (main_waves > 0) {
        const unsigned blocks = (unsigned)((main_waves + 3) / 4);
        hipLaunchKernelGGL((k_m2_step<F, LPR, PRE, kStepIters, kStepRing, step_waves<F, PRE, SR>(), SR>), dim3(blocks),
                           dim3(256), 0, st, a,
                           (int64_t)0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // leftover iterations, one per wave
    const int64_t done = main_waves * kStepIters;
    const int64_t rest = a.total_iters - done;
    if (rest > 0) {
        const unsigned blocks = (unsigned)((rest + 3) / 4);
        hipLaunchKernelGGL((k_m2_step<F, LPR, PRE, 1, 1, 1, SR>), dim3(blocks), dim3(256), 0, st, a, done);
        return hipGetLastError();
    }
    return hipSuccess;
}

// Iterations per wave for this layer: int4 rows (16 per wave-iteration) take 16 or 32 when the
// layer has enough of them to give every resident wave slot that many, so that the waves
// run in one round (8B-shaped layer: 4.6% faster with 32 than with four rounds of 8, A/B on one
// box).  The longer forms are compiled as a loop; the 370m-shaped layer, one round of 8, is
// slower with them (fewer waves than slots).  int8 rows (8 per wave-iteration) keep 4 at
// every size (8 or 16 on the 8B-shaped layer: 7% and 16% slower), as does stochastic
// rounding.
template <int F, bool PRE, bool SR>
static hipError_t launch_step_fp(M2Args a, int num_cus, hipStream_t st)
{
    constexpr int K0 = step_iters<F>();
    if constexpr (Traits<F>::quant && Traits<F>::bits == 4 && !SR) {
        constexpr int RPW = 64 / step_lanes_per_row<F>();
        const int64_t iters = (int64_t)a.Bsz * a.H * a.P / RPW;
        const int64_t slots = (int64_t)num_cus * 16; // 4 SIMDs x 4 waves: every int4 form fits 128 registers
        if (iters >= 4 * K0 * slots) return launch_step_k<F, PRE, SR, 4 * K0>(a, st);
        if (iters >= 2 * K0 * slots) return launch_step_k<F, PRE, SR, 2 * K0>(a, st);
    }
    return launch_step_k<F, PRE, SR, K0>(a, st);
}

template <int F>
static hipError_t launch_step_f(M2Args a, bool pre, int num_cus, hipStream_t st)
{
    if constexpr (Traits<F>::quant) {
        if (a.sr.on) return pre ? launch_step_fp<F, true, true>(a, num_cus, st) : launch_step_fp<F, false, true>(a, num_cus, st);
    }
    return pre ? launch_step_fp<F, true, false>(a, num_cus, st) : launch_step_fp<F, false, false>(a, num_cus, st);
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

template <int F, bool PRE, int W>
static hipError_t launch_scan_k(M2Args a, hipStream_t st)
{
    constexpr int LPR = lanes_per_row<F>();
    constexpr int RPW = 64 / LPR;
    a.total_iters = (int64_t)a.Bsz * a.H * a.P / RPW;
    a.iters_per_wave = 1;
    const unsigned blocks = (unsigned)((a.total_iters + 3) / 4);
    if constexpr (Traits<F>::quant) {
        if (a.sr.on) {
            hipLaunchKernelGGL((k_m2_scan<F, LPR, PRE, true, W>), dim3(blocks), dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_m2_scan<F, LPR, PRE, false, W>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// Rows with a zero point need more than 128 registers in the scan: with a budget of 4 waves
// per SIMD they spill to scratch, with 3 they do not.  The 3-wave form is taken where every
// wave of the scan fits at 3 per SIMD (130m-shaped layer, 3,072 waves: int8 asymmetric scan 2%
// faster); a layer with more waves keeps 4 per SIMD rather than run a second round (8B-shaped
// int4 scan, 4,096 waves: 45% slower with 3).
template <int F>
static hipError_t launch_scan_f(M2Args a, bool pre, int num_cus, hipStream_t st)
{
    if (pre) return launch_scan_k<F, true, SSQ_SCAN_WAVES>(a, st);
    if constexpr (Traits<F>::asym) {
        const int64_t waves = (int64_t)a.Bsz * a.H * a.P / (64 / lanes_per_row<F>());
        if (waves <= (int64_t)num_cus * 4 * (SSQ_SCAN_WAVES - 1))
            return launch_scan_k<F, false, SSQ_SCAN_WAVES - 1>(a, st);
    }
    return launch_scan_k<F, false, SSQ_SCAN_WAVES>(a, st);
}

template <int F>
static hipError_t launch_prefill_f(M2Args a, int chunk, bool pre, int num_cus, hipStream_t st)
{
    if constexpr (!Traits<F>::quant) {
        return launch_scan_f<F>(a, pre, num_cus, st); // the fp32 state's prefill is the scan
    } else {
        constexpr int LPR = lanes_per_row<F>();
        constexpr int RPW = 64 / LPR;
        a.total_iters = (int64_t)a.Bsz * a.H * a.P / RPW;
        a.iters_per_wave = 1;
        const unsigned blocks = (unsigned)((a.total_iters + 3) / 4);
        if (a.sr.on) {
            if (pre)
                hipLaunchKernelGGL((k_m2_prefill<F, LPR, true, true>), dim3(blocks), dim3(256), 0, st, a, chunk);
            else
                hipLaunchKernelGGL((k_m2_prefill<F, LPR, false, true>), dim3(blocks), dim3(256), 0, st, a, chunk);
        } else {
            if (pre)
                hipLaunchKernelGGL((k_m2_prefill<F, LPR, true, false>), dim3(blocks), dim3(256), 0, st, a, chunk);
            else
                hipLaunchKernelGGL((k_m2_prefill<F, LPR, false, false>), dim3(blocks), dim3(256), 0, st, a, chunk);
        }
        return hipGetLastError();
    }
}

hipError_t launch_m2_prefill(int fmt, M2Args a, int chunk, bool pre, int num_cus, hipStream_t st)
{
    switch (fmt) {
    case FP32: return launch_prefill_f<FP32>(a, chunk, pre, num_cus, st);
    case INT8_SYM: return launch_prefill_f<INT8_SYM>(a, chunk, pre, num_cus, st);
    case INT8_ASYM: return launch_prefill_f<INT8_ASYM>(a, chunk, pre, num_cus, st);
    case INT4_SYM: return launch_prefill_f<INT4_SYM>(a, chunk, pre, num_cus, st);
    case INT4_ASYM: return launch_prefill_f<INT4_ASYM>(a, chunk, pre, num_cus, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_m2_scan(int fmt, M2Args a, bool pre, int num_cus, hipStream_t st)
{
    switch (fmt) {
    case FP32: return launch_scan_f<FP32>(a, pre, num_cus, st);
    case INT8_SYM: return launch_scan_f<INT8_SYM>(a, pre, num_cus, st);
    case INT8_ASYM: return launch_scan_f<INT8_ASYM>(a, pre, num_cus, st);
    case INT4_SYM: return launch_scan_f<INT4_SYM>(a, pre, num_cus, st);
    case INT4_ASYM: return launch_scan_f<INT4_ASYM>(a, pre, num_cus, st);
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

hipError_t launch_set_counter(uint64_t* ctr, uint64_t value, hipStream_t st)
{
    hipLaunchKernelGGL(k_set_counter, dim3(1), dim3(64), 0, st, ctr, value);
    return hipGetLastError();
}

hipError_t launch_advance_counter(uint64_t* ctr, uint64_t tokens, hipStream_t st)
{
    hipLaunchKernelGGL(k_advance_counter, dim3(1), dim3(64), 0, st, ctr, tokens);
    return hipGetLastError();
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
