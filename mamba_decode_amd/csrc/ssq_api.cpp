// ssq_api.cpp -- the C ABI of include/ssq.h: argument validation, state
// layout and ownership, launch configuration and error reporting.  Every
// argument is checked before anything is enqueued, so a rejected call changes
// nothing; kernels run asynchronously on the caller's stream.
#include "ssq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "ssq_internal.h"

struct ssq_state {
    ssq_desc desc;
    ssq_layout lay;
    void* storage;
    bool owned;
    int device;
    int32_t rounding; // ssq_rounding
    uint64_t sr_seed; // stochastic rounding: generator seed (the next token is in the storage)
};

namespace {

thread_local std::string g_last_error;

ssq_status fail(ssq_status st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

ssq_status ok()
{
    g_last_error.clear();
    return SSQ_OK;
}

bool fmt_valid(int f) { return f >= SSQ_FP32 && f <= SSQ_DAMP; }
bool fmt_quant(int f) { return f != SSQ_FP32; }
bool fmt_asym(int f) { return f == SSQ_INT8_ASYM || f == SSQ_INT4_ASYM || f == SSQ_DAMP; }
int fmt_bits(int f)
{
    return f == SSQ_FP32 ? 32 : (f == SSQ_INT8_SYM || f == SSQ_INT8_ASYM || f == SSQ_DAMP ? 8 : 4);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool mul_ok(size_t a, size_t b, size_t* out)
{
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

ssq_status check_desc(const ssq_desc* d, ssq_layout* lay)
{
    if (!d) return fail(SSQ_ERR_INVALID_ARG, "desc is NULL");
    if (d->kind != SSQ_MAMBA2 && d->kind != SSQ_DELTA) return fail(SSQ_ERR_INVALID_ARG, "unknown state kind");
    if (!fmt_valid(d->format)) return fail(SSQ_ERR_INVALID_ARG, "unknown format");
    if (d->batch <= 0 || d->nheads <= 0 || d->ngroups <= 0 || d->rows_per_head <= 0 || d->row_len <= 0)
        return fail(SSQ_ERR_INVALID_ARG, "every dimension must be positive");
    if (d->nheads % d->ngroups != 0) return fail(SSQ_ERR_INVALID_ARG, "ngroups must divide nheads");
    if (d->kind == SSQ_DELTA && d->ngroups != 1) return fail(SSQ_ERR_INVALID_ARG, "a delta state has ngroups == 1");
    if (d->row_len != 128) return fail(SSQ_ERR_UNSUPPORTED, "kernels are built for row_len == 128");
    if (d->kind == SSQ_MAMBA2 && d->rows_per_head % 16 != 0)
        return fail(SSQ_ERR_UNSUPPORTED, "Mamba-2 kernels need rows_per_head to be a multiple of 16");
    if (d->kind == SSQ_DELTA && d->rows_per_head != 128)
        return fail(SSQ_ERR_UNSUPPORTED, "delta kernels are built for dk == 128");
    if (d->format == SSQ_DAMP && d->kind != SSQ_DELTA)
        return fail(SSQ_ERR_UNSUPPORTED, "the two-tier format is a delta-rule state");

    ssq_layout l;
    size_t rows;
    if (!mul_ok((size_t)d->batch, (size_t)d->nheads, &rows) || !mul_ok(rows, (size_t)d->rows_per_head, &rows))
        return fail(SSQ_ERR_INVALID_ARG, "state size overflows size_t");
    const int bits = fmt_bits(d->format);
    l.rows = rows;
    l.row_bytes = (size_t)d->row_len * (size_t)bits / 8;
    // the two-tier format keeps its uint8 rows in codes/scale/zero and the half rows apart
    size_t qrows = rows, hi_bytes = 0;
    if (d->format == SSQ_DAMP) {
        const size_t mats = rows / (size_t)d->rows_per_head;
        qrows = mats * (size_t)(d->rows_per_head - SSQ_DAMP_NHI);
        hi_bytes = mats * SSQ_DAMP_NHI * (size_t)d->row_len * 2;
    }
    size_t codes_bytes, meta_bytes;
    if (!mul_ok(qrows, l.row_bytes, &codes_bytes) || !mul_ok(qrows, 4, &meta_bytes) || codes_bytes > SIZE_MAX / 2)
        return fail(SSQ_ERR_INVALID_ARG, "state size overflows size_t");
    l.codes_offset = 0;
    size_t end = align256(codes_bytes);
    l.scale_offset = 0;
    l.zero_offset = 0;
    if (fmt_quant(d->format)) {
        l.scale_offset = end;
        end = align256(end + meta_bytes);
        if (fmt_asym(d->format)) {
            l.zero_offset = end;
            end = align256(end + meta_bytes);
        }
    }
    l.hi_offset = 0;
    if (hi_bytes) {
        l.hi_offset = end;
        end = align256(end + hi_bytes);
    }
    // quantized formats: the stochastic-rounding token counter
    l.counter_offset = 0;
    if (fmt_quant(d->format)) {
        l.counter_offset = end;
        end = align256(end + 8);
    }
    l.total_bytes = end;
    if (lay) *lay = l;
    return SSQ_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// compute units of a device, cached (read-only after the first query)
int num_cus(int dev)
{
    static std::atomic<int> cache[64];
    if (dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

ssq_status from_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ok();
    return fail(SSQ_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

ssq_status check_device(const ssq_state* st)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, "hipGetDevice");
    if (dev != st->device) return fail(SSQ_ERR_INVALID_ARG, "the state lives on another device than the current one");
    return SSQ_OK;
}

uint8_t* codes_ptr(const ssq_state* st) { return (uint8_t*)st->storage + st->lay.codes_offset; }
float* scale_ptr(const ssq_state* st)
{
    return fmt_quant(st->desc.format) ? (float*)((uint8_t*)st->storage + st->lay.scale_offset) : nullptr;
}
float* zero_ptr(const ssq_state* st)
{
    return fmt_asym(st->desc.format) ? (float*)((uint8_t*)st->storage + st->lay.zero_offset) : nullptr;
}
uint64_t* counter_ptr(const ssq_state* st)
{
    return fmt_quant(st->desc.format) ? (uint64_t*)((uint8_t*)st->storage + st->lay.counter_offset) : nullptr;
}
uint16_t* hi_ptr(const ssq_state* st)
{
    return st->desc.format == SSQ_DAMP ? (uint16_t*)((uint8_t*)st->storage + st->lay.hi_offset) : nullptr;
}
// rows of the state that are rounded to a grid (the counter space of stochastic rounding)
int64_t grid_rows(const ssq_state* st)
{
    if (st->desc.format != SSQ_DAMP) return (int64_t)st->lay.rows;
    return (int64_t)(st->lay.rows / 128) * (128 - SSQ_DAMP_NHI);
}

#define SSQ_REQUIRE(cond, status, msg)            \
    do {                                           \
        if (!(cond)) return fail((status), (msg)); \
    } while (0)

} // namespace

extern "C" {

size_t ssq_state_bytes(const ssq_desc* desc)
{
    ssq_layout l;
    if (check_desc(desc, &l) != SSQ_OK) return 0;
    return l.total_bytes;
}

ssq_status ssq_state_layout(const ssq_desc* desc, ssq_layout* layout)
{
    SSQ_REQUIRE(layout, SSQ_ERR_INVALID_ARG, "layout is NULL");
    ssq_status s = check_desc(desc, layout);
    return s == SSQ_OK ? ok() : s;
}

ssq_status ssq_alloc_state(const ssq_desc* desc, void* storage, const float* init, void* stream, ssq_state** out)
{
    SSQ_REQUIRE(out, SSQ_ERR_INVALID_ARG, "out is NULL");
    ssq_layout lay;
    ssq_status s = check_desc(desc, &lay);
    if (s != SSQ_OK) return s;
    SSQ_REQUIRE(aligned(storage, 256), SSQ_ERR_INVALID_ARG, "storage must be 256-byte aligned");
    SSQ_REQUIRE(aligned(init, 16), SSQ_ERR_INVALID_ARG, "init must be 16-byte aligned");
    if (!storage) {
        const char* hook = std::getenv("SSQ_TEST_FAIL_ALLOC");
        if (hook && hook[0] == '1') return fail(SSQ_ERR_ALLOC, "allocation failure forced by SSQ_TEST_FAIL_ALLOC");
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, "hipGetDevice");

    ssq_state* st = new (std::nothrow) ssq_state;
    SSQ_REQUIRE(st, SSQ_ERR_ALLOC, "out of host memory");
    st->desc = *desc;
    st->lay = lay;
    st->device = dev;
    st->owned = false;
    st->storage = storage;
    st->rounding = SSQ_ROUND_NEAREST;
    st->sr_seed = 0;
    if (!storage) {
        void* p = nullptr;
        e = hipMalloc(&p, lay.total_bytes);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            delete st;
            return fail(SSQ_ERR_ALLOC, std::string("hipMalloc: ") + hipGetErrorString(e));
        }
        st->storage = p;
        st->owned = true;
    }
    hipStream_t hs = (hipStream_t)stream;
    // every byte of the storage is written: zero first (padding, the token counter), then the
    // quantized rows of `init`
    e = ssq::launch_zero_fill(st->storage, lay.total_bytes, hs);
    if (e == hipSuccess && init) {
        ssq::QArgs a{};
        a.codes = codes_ptr(st);
        a.scale = scale_ptr(st);
        a.zero = zero_ptr(st);
        a.h32 = (float*)codes_ptr(st);
        a.hi = hi_ptr(st);
        a.in = init;
        a.rows = (int64_t)lay.rows;
        e = desc->format == SSQ_DAMP ? ssq::launch_damp_rows(a, false, hs)
                                     : ssq::launch_rows(desc->format, a, false, hs);
    }
    if (e != hipSuccess) {
        if (st->owned) (void)hipFree(st->storage);
        delete st;
        return from_hip(e, "state initialisation launch");
    }
    *out = st;
    return ok();
}

ssq_status ssq_free_state(ssq_state* st)
{
    if (!st) return ok();
    hipError_t e = hipSuccess;
    if (st->owned) e = hipFree(st->storage);
    delete st;
    return from_hip(e, "hipFree");
}

ssq_status ssq_state_info(const ssq_state* st, ssq_desc* desc, void** storage, ssq_layout* layout)
{
    SSQ_REQUIRE(st, SSQ_ERR_INVALID_ARG, "state is NULL");
    if (desc) *desc = st->desc;
    if (storage) *storage = st->storage;
    if (layout) *layout = st->lay;
    return ok();
}

// the stochastic-rounding arguments of the next call on a state (the launcher sets the
// call's wave count and the tokens it consumes)
static ssq::SrArgs sr_args(const ssq_state* st)
{
    ssq::SrArgs r{};
    r.on = st->rounding == SSQ_ROUND_STOCHASTIC;
    r.seed = st->sr_seed;
    r.rows = grid_rows(st);
    r.ctr = counter_ptr(st);
    return r;
}

// after a stochastically rounded call's step kernels: the state's next token moves on
static ssq_status advance(const ssq_state* st, uint64_t tokens, hipStream_t stream)
{
    if (st->rounding != SSQ_ROUND_STOCHASTIC) return ok();
    return from_hip(ssq::launch_advance_counter(counter_ptr(st), tokens, stream), "token counter launch");
}

ssq_status ssq_set_rounding(ssq_state* st, int32_t mode, uint64_t seed, uint64_t step, void* stream)
{
    SSQ_REQUIRE(st, SSQ_ERR_INVALID_ARG, "state is NULL");
    SSQ_REQUIRE(mode == SSQ_ROUND_NEAREST || mode == SSQ_ROUND_STOCHASTIC, SSQ_ERR_INVALID_ARG,
                "unknown rounding mode");
    SSQ_REQUIRE(mode == SSQ_ROUND_NEAREST || fmt_quant(st->desc.format), SSQ_ERR_UNSUPPORTED,
                "the fp32 state is not rounded");
    SSQ_REQUIRE(mode == SSQ_ROUND_STOCHASTIC || step == 0 || fmt_quant(st->desc.format), SSQ_ERR_UNSUPPORTED,
                "the fp32 state has no token counter");
    ssq_status s = check_device(st);
    if (s != SSQ_OK) return s;
    if (fmt_quant(st->desc.format)) {
        s = from_hip(ssq::launch_set_counter(counter_ptr(st), step, (hipStream_t)stream), "token counter launch");
        if (s != SSQ_OK) return s;
    }
    st->rounding = mode;
    st->sr_seed = seed;
    return ok();
}

ssq_status ssq_get_rounding(const ssq_state* st, int32_t* mode, uint64_t* seed, uint64_t* step, void* stream)
{
    SSQ_REQUIRE(st, SSQ_ERR_INVALID_ARG, "state is NULL");
    uint64_t next = 0;
    if (step && fmt_quant(st->desc.format)) {
        ssq_status s = check_device(st);
        if (s != SSQ_OK) return s;
        hipError_t e = hipMemcpyAsync(&next, counter_ptr(st), sizeof next, hipMemcpyDeviceToHost, (hipStream_t)stream);
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) return from_hip(e, "reading the token counter");
    }
    if (mode) *mode = st->rounding;
    if (seed) *seed = st->sr_seed;
    if (step) *step = next;
    return ok();
}

static ssq_status fill_m2(ssq_state* st, const float* x, const float* dt, const float* A, const float* B,
                          const float* C, const float* D, float* y, int32_t readout, ssq::M2Args* a)
{
    SSQ_REQUIRE(st, SSQ_ERR_INVALID_ARG, "state is NULL");
    SSQ_REQUIRE(st->desc.kind == SSQ_MAMBA2, SSQ_ERR_KIND_MISMATCH, "a Mamba-2 call on a delta state");
    SSQ_REQUIRE(x && dt && A && B && C && D && y, SSQ_ERR_INVALID_ARG, "an input or output pointer is NULL");
    SSQ_REQUIRE(aligned(x, 4) && aligned(dt, 4) && aligned(A, 4) && aligned(D, 4) && aligned(y, 4),
                SSQ_ERR_INVALID_ARG, "x, dt, A, D and y must be 4-byte aligned");
    SSQ_REQUIRE(aligned(B, 16) && aligned(C, 16), SSQ_ERR_INVALID_ARG, "B and C must be 16-byte aligned");
    SSQ_REQUIRE(readout == SSQ_READ_POST_QUANT || readout == SSQ_READ_PRE_QUANT, SSQ_ERR_INVALID_ARG,
                "unknown readout");
    ssq_status s = check_device(st);
    if (s != SSQ_OK) return s;
    *a = ssq::M2Args{};
    a->codes = codes_ptr(st);
    a->scale = scale_ptr(st);
    a->zero = zero_ptr(st);
    a->h32 = (float*)codes_ptr(st);
    a->x = x;
    a->dt = dt;
    a->A = A;
    a->Bm = B;
    a->Cm = C;
    a->D = D;
    a->y = y;
    a->Bsz = st->desc.batch;
    a->H = st->desc.nheads;
    a->G = st->desc.ngroups;
    a->P = st->desc.rows_per_head;
    a->T = 1;
    return SSQ_OK;
}

ssq_status ssq_decode_step(ssq_state* st, const float* x, const float* dt, const float* A, const float* B,
                           const float* C, const float* D, float* y, int32_t readout, void* stream)
{
    ssq::M2Args a;
    ssq_status s = fill_m2(st, x, dt, A, B, C, D, y, readout, &a);
    if (s != SSQ_OK) return s;
    a.sr = sr_args(st);
    s = from_hip(ssq::launch_m2_step(st->desc.format, a, readout == SSQ_READ_PRE_QUANT, num_cus(st->device),
                                     (hipStream_t)stream),
                 "decode step launch");
    return s == SSQ_OK ? advance(st, 1, (hipStream_t)stream) : s;
}

ssq_status ssq_scan(ssq_state* st, int32_t T, const float* x, const float* dt, const float* A, const float* B,
                    const float* C, const float* D, float* y, int32_t readout, void* stream)
{
    ssq::M2Args a;
    ssq_status s = fill_m2(st, x, dt, A, B, C, D, y, readout, &a);
    if (s != SSQ_OK) return s;
    SSQ_REQUIRE(T > 0, SSQ_ERR_INVALID_ARG, "T must be positive");
    a.T = T;
    a.sr = sr_args(st);
    s = from_hip(ssq::launch_m2_scan(st->desc.format, a, readout == SSQ_READ_PRE_QUANT, num_cus(st->device),
                                     (hipStream_t)stream),
                 "scan launch");
    return s == SSQ_OK ? advance(st, (uint64_t)T, (hipStream_t)stream) : s;
}

ssq_status ssq_prefill(ssq_state* st, int32_t T, int32_t chunk, const float* x, const float* dt, const float* A,
                       const float* B, const float* C, const float* D, float* y, int32_t readout, void* stream)
{
    ssq::M2Args a;
    ssq_status s = fill_m2(st, x, dt, A, B, C, D, y, readout, &a);
    if (s != SSQ_OK) return s;
    SSQ_REQUIRE(T > 0, SSQ_ERR_INVALID_ARG, "T must be positive");
    SSQ_REQUIRE(chunk > 0, SSQ_ERR_INVALID_ARG, "chunk must be positive");
    a.T = T;
    a.sr = sr_args(st);
    s = from_hip(ssq::launch_m2_prefill(st->desc.format, a, chunk, readout == SSQ_READ_PRE_QUANT, num_cus(st->device),
                                        (hipStream_t)stream),
                 "prefill launch");
    return s == SSQ_OK ? advance(st, (uint64_t)T, (hipStream_t)stream) : s;
}

static ssq_status delta_common(ssq_state* st, const float* q, const float* k, const float* v, const float* alpha,
                               const float* beta, float* o, int32_t readout, void* stream, bool kda)
{
    SSQ_REQUIRE(st, SSQ_ERR_INVALID_ARG, "state is NULL");
    SSQ_REQUIRE(st->desc.kind == SSQ_DELTA, SSQ_ERR_KIND_MISMATCH, "a delta-rule call on a Mamba-2 state");
    SSQ_REQUIRE(q && k && v && alpha && beta && o, SSQ_ERR_INVALID_ARG, "an input or output pointer is NULL");
    SSQ_REQUIRE(aligned(q, 4) && aligned(k, 4) && aligned(alpha, 4) && aligned(beta, 4) && aligned(o, 4),
                SSQ_ERR_INVALID_ARG, "q, k, alpha, beta and o must be 4-byte aligned");
    SSQ_REQUIRE(aligned(v, 16), SSQ_ERR_INVALID_ARG, "v must be 16-byte aligned");
    SSQ_REQUIRE(readout == SSQ_READ_POST_QUANT || readout == SSQ_READ_PRE_QUANT, SSQ_ERR_INVALID_ARG,
                "unknown readout");
    ssq_status s = check_device(st);
    if (s != SSQ_OK) return s;
    ssq::DeltaArgs a{};
    a.codes = codes_ptr(st);
    a.scale = scale_ptr(st);
    a.zero = zero_ptr(st);
    a.h32 = (float*)codes_ptr(st);
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.o = o;
    a.nmat = (int64_t)st->desc.batch * st->desc.nheads;
    a.kda = kda ? 1 : 0;
    a.sr = sr_args(st);
    a.hi = hi_ptr(st);
    if (st->desc.format == SSQ_DAMP) {
        SSQ_REQUIRE(!kda, SSQ_ERR_UNSUPPORTED, "the two-tier state takes the scalar-decay step only");
        s = from_hip(ssq::launch_damp_step(a, readout == SSQ_READ_PRE_QUANT, (hipStream_t)stream),
                     "two-tier delta step launch");
    } else {
        s = from_hip(ssq::launch_delta_step(st->desc.format, a, readout == SSQ_READ_PRE_QUANT, (hipStream_t)stream),
                     kda ? "KDA step launch" : "delta step launch");
    }
    return s == SSQ_OK ? advance(st, 1, (hipStream_t)stream) : s;
}

ssq_status ssq_delta_step(ssq_state* st, const float* q, const float* k, const float* v, const float* alpha,
                          const float* beta, float* o, int32_t readout, void* stream)
{
    return delta_common(st, q, k, v, alpha, beta, o, readout, stream, false);
}

ssq_status ssq_kda_step(ssq_state* st, const float* q, const float* k, const float* v, const float* alpha,
                        const float* beta, float* o, int32_t readout, void* stream)
{
    return delta_common(st, q, k, v, alpha, beta, o, readout, stream, true);
}

ssq_status ssq_dequant(const ssq_state* st, float* out, void* stream)
{
    SSQ_REQUIRE(st, SSQ_ERR_INVALID_ARG, "state is NULL");
    SSQ_REQUIRE(out, SSQ_ERR_INVALID_ARG, "out is NULL");
    SSQ_REQUIRE(aligned(out, 16), SSQ_ERR_INVALID_ARG, "out must be 16-byte aligned");
    ssq_status s = check_device(st);
    if (s != SSQ_OK) return s;
    ssq::QArgs a{};
    a.codes = codes_ptr(st);
    a.scale = scale_ptr(st);
    a.zero = zero_ptr(st);
    a.h32 = (float*)codes_ptr(st);
    a.out = out;
    a.rows = (int64_t)st->lay.rows;
    a.hi = hi_ptr(st);
    if (st->desc.format == SSQ_DAMP)
        return from_hip(ssq::launch_damp_rows(a, true, (hipStream_t)stream), "dequant launch");
    return from_hip(ssq::launch_rows(st->desc.format, a, true, (hipStream_t)stream), "dequant launch");
}

ssq_status ssq_stream_copy(void* dst, const void* src, size_t bytes, void* stream)
{
    SSQ_REQUIRE(dst && src, SSQ_ERR_INVALID_ARG, "dst and src must not be NULL");
    SSQ_REQUIRE(aligned(dst, 16) && aligned(src, 16), SSQ_ERR_INVALID_ARG, "dst and src must be 16-byte aligned");
    SSQ_REQUIRE(bytes % 16 == 0, SSQ_ERR_INVALID_ARG, "bytes must be a multiple of 16");
    SSQ_REQUIRE(bytes <= ((size_t)1 << 40), SSQ_ERR_INVALID_ARG, "bytes must not exceed 2^40");
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    SSQ_REQUIRE(d + bytes <= s || s + bytes <= d, SSQ_ERR_INVALID_ARG, "dst and src must not overlap");
    return from_hip(ssq::launch_stream_copy(dst, src, (int64_t)bytes, (hipStream_t)stream), "copy launch");
}

const char* ssq_status_string(int32_t status)
{
    switch (status) {
    case SSQ_OK: return "SSQ_OK";
    case SSQ_ERR_INVALID_ARG: return "SSQ_ERR_INVALID_ARG: invalid argument";
    case SSQ_ERR_UNSUPPORTED: return "SSQ_ERR_UNSUPPORTED: size or format not supported by the kernels";
    case SSQ_ERR_KIND_MISMATCH: return "SSQ_ERR_KIND_MISMATCH: call does not match the state kind";
    case SSQ_ERR_ALLOC: return "SSQ_ERR_ALLOC: device allocation failed";
    case SSQ_ERR_DEVICE: return "SSQ_ERR_DEVICE: HIP runtime error";
    }
    return "unknown ssq_status";
}

const char* ssq_last_error(void) { return g_last_error.c_str(); }

} // extern "C"
