// ssq_internal.h -- kernel argument blocks and launchers shared by the HIP
// sources and the C-ABI layer (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssq {

// stochastic rounding of the codes: off, or entry n of state row r at token step + t
// draws the uniform of counter ((step + t)*rows + r)*128 + n.  `step` is the state's token
// counter in device memory (*ctr), read by every wave at its start; the call advances it with
// a one-thread kernel enqueued after its step kernels (launch_advance_counter), so that a
// call replayed from a graph draws the next tokens' uniforms.
struct SrArgs {
    int on;
    uint64_t seed;
    int64_t rows;
    const uint64_t* ctr; // the state's next token
};

// Mamba-2 decode step / scan of one layer
struct M2Args {
    uint8_t* codes; // quantized formats: [rows][128*bits/8]
    float* scale;   // [rows]
    float* zero;    // [rows] (asymmetric formats)
    float* h32;     // fp32 format: [rows][128]
    const float* x;
    const float* dt;
    const float* A;
    const float* Bm;
    const float* Cm;
    const float* D;
    float* y;
    int Bsz, H, G, P, T;
    int64_t total_iters;
    int iters_per_wave;
    SrArgs sr;
};

// row quantization (state initialisation) and dequantization
struct QArgs {
    uint8_t* codes;
    float* scale;
    float* zero;
    float* h32;
    uint16_t* hi;    // two-tier delta state: the half rows
    const float* in; // quantize: source rows [rows][128]
    float* out;      // dequantize: destination rows [rows][128]
    int64_t rows;
};

// delta-rule step of one layer: Bsz*H matrices of 128 key rows x 128 values
struct DeltaArgs {
    uint8_t* codes;
    float* scale;
    float* zero;
    float* h32;
    const float* q;
    const float* k;
    const float* v;
    const float* alpha; // [nmat], or [nmat][128] with kda (a decay per key channel)
    const float* beta;
    float* o;
    int64_t nmat;
    int kda;
    SrArgs sr;
    uint16_t* hi; // two-tier state: [nmat][16][128] half rows (codes/scale/zero: the uint8 rows)
};

hipError_t launch_m2_step(int fmt, M2Args a, bool pre, int num_cus, hipStream_t st);
hipError_t launch_m2_scan(int fmt, M2Args a, bool pre, int num_cus, hipStream_t st);
hipError_t launch_m2_prefill(int fmt, M2Args a, int chunk, bool pre, int num_cus, hipStream_t st);
hipError_t launch_rows(int fmt, QArgs a, bool dequant, hipStream_t st);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st);
hipError_t launch_delta_step(int fmt, DeltaArgs a, bool pre, hipStream_t st);
hipError_t launch_damp_step(DeltaArgs a, bool pre, hipStream_t st);
hipError_t launch_damp_rows(QArgs a, bool dequant, hipStream_t st);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t st);
hipError_t launch_set_counter(uint64_t* ctr, uint64_t value, hipStream_t st);
hipError_t launch_advance_counter(uint64_t* ctr, uint64_t tokens, hipStream_t st);

} // namespace ssq
