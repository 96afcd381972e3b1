/*
 * ssq.h -- quantized recurrent-state update on MI355X (gfx950): C ABI.
 *
 * A recurrent layer keeps one fixed-size state per live sequence and, for
 * every generated token, reads it, applies the recurrence, requantizes it and
 * writes it back ("Mamba state quantization for inference": "Recurrent state
 * is fixed per request, not free"; the DAMP paragraph of "Mamba state
 * quantization changes persistent state").  This library stores that state
 * quantized per row and updates it in place with hand-written HIP kernels.
 *
 * Two state kinds:
 *  - SSQ_MAMBA2: the Mamba-2 selective-SSM state, [batch][nheads][P][N] with
 *    head dimension P and state size N.  A row is (sequence, head, p) over the
 *    N state entries ("ssm-state-quantization" README, Setup: one scale per
 *    row, i.e. per head and head_dim, over the 128 state entries).
 *  - SSQ_DELTA: the delta-rule (Gated DeltaNet / Kimi Delta Attention style)
 *    matrix state, one dk x dv matrix per (sequence, head) ("Mamba state
 *    quantization for inference", "Mamba state quantization changes
 *    persistent state").  A row is one key channel over the value dimension.
 *
 * Formats: fp32 (unquantized control), and symmetric or asymmetric per-row
 * grids at 8 or 4 bits, refit at every step (README, Setup: symmetric grid
 * [-amax, amax] with step amax/(2^(b-1)-1); asymmetric grid [min, max] with an
 * integer zero point and step (max-min)/(2^b-1); Findings 1: round to
 * nearest at 8 and 4 bits).
 *
 * Fixed fp32 evaluation order of one row (fl() = one fp32 rounding; results
 * are bit-reproducible and independent of the launch configuration):
 *   lambda = fl32(exp(fl(dt*A)))  (exp evaluated in double, rounded once)
 *   w      = fl(dt*x)
 *   quantized state (scale s, zero point z, codes c): each entry is
 *   reconstructed, then the fp32 recurrence runs on it (the README's Setup
 *   applies the decay and the write to the state; "Mamba state quantization
 *   for inference", "Mixed precision spends bits on persistent channels":
 *   reconstruct, recur in FP32, refit, write back):
 *     hh_n = fl(s*fl(c_n - z)),  h'_n = fma(lambda, hh_n, fl(w*B_n))
 *   fp32 state:  h'_n = fma(lambda, h_n, fl(w*B_n))
 *   asymmetric refit: s' = fl(fl(max-min)/(2^b-1)), inv = fl(1/s'),
 *     z' = -rne(min*inv), c'_n = clamp(rne(h'_n*inv + z'), 0, 2^b-1)
 *   symmetric refit: s' = fl(amax/(2^(b-1)-1)), inv = fl(1/s'),
 *     c'_n = clamp(rne(h'_n*inv), -(2^(b-1)-1), 2^(b-1)-1)
 *   where rne() rounds the exact real value (the product is not rounded
 *     first) to the nearest integer, a tie going to the even integer, and a
 *     zero point of zero is stored as +0
 *   a zero or subnormal s' marks a degenerate row: asymmetric rows become the
 *     constant min (s' = |min|, z' = -sign(min), codes 0), symmetric rows zero
 *   y = sum_n C_n*r_n + D*x, r = the dequantized new row s'*fl(c'-z')
 *     (default: the README reads the output from the quantized state) or the
 *     new row before rounding (SSQ_READ_PRE_QUANT); y and the delta-rule
 *     output o are outputs only, their summation order is unspecified.
 *
 * Conventions for every call:
 *  - Pointers named as device pointers must be device memory of the current
 *    HIP device, fp32, contiguous, row-major in the shapes given, and 16-byte
 *    aligned.  The caller owns every input and output buffer.
 *  - Calls only enqueue work on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream) and return without synchronizing.  Inputs must
 *    stay valid until the stream has passed the call.  Calls on one state
 *    must be ordered on one stream by the caller; distinct states are
 *    independent.
 *  - Every argument is validated before anything is enqueued; a rejected
 *    call returns a non-zero status, changes nothing and leaves a detail
 *    message for ssq_last_error().  Non-finite inputs are not checked: the
 *    codes, scales and outputs of the rows they reach (for the delta rule,
 *    the matrices) are unspecified; the call completes and every other row
 *    is computed as usual.
 *  - Kernels support row_len == 128, and rows_per_head a multiple of 16 for
 *    SSQ_MAMBA2, dk == 128 for SSQ_DELTA.
 */
#ifndef SSQ_H
#define SSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSQ_OK = 0,
    SSQ_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad alignment, ngroups not dividing nheads, T <= 0 */
    SSQ_ERR_UNSUPPORTED = 2,   /* a size or format the kernels are not built for */
    SSQ_ERR_KIND_MISMATCH = 3, /* a Mamba-2 call on a delta state or the reverse */
    SSQ_ERR_ALLOC = 4,         /* device allocation failed */
    SSQ_ERR_DEVICE = 5         /* the HIP runtime reported an error */
} ssq_status;

typedef enum {
    SSQ_FP32 = 0,
    SSQ_INT8_SYM = 1,  /* int8_t codes in [-127, 127], fp32 scale */
    SSQ_INT8_ASYM = 2, /* uint8_t codes in [0, 255], fp32 scale and integer-valued fp32 zero point */
    SSQ_INT4_SYM = 3,  /* 4-bit two's complement codes in [-7, 7], two per byte, fp32 scale */
    SSQ_INT4_ASYM = 4, /* 4-bit codes in [0, 15], two per byte, fp32 scale and zero point */
    SSQ_DAMP = 5       /* SSQ_DELTA only: two tiers, see below */
} ssq_format;

/* SSQ_DAMP: the two-tier delta-rule state of "Mamba state quantization for
 * inference", "Mixed precision spends bits on persistent channels" (a Hadamard
 * transform along each key channel's value dimension; the protected key
 * channels in FP16, the rest in INT8 with scale and zero point, the protected
 * channels permuted to be contiguous).  Here: key channels 0 .. SSQ_DAMP_NHI-1
 * of every matrix are the protected ones (the model's key projection is
 * permuted offline so that they come first); every row is stored rotated,
 * St = S Hs with Hs = H_128/16 (Sylvester-ordered Hadamard, Hs Hs = I/2); the
 * protected rows as IEEE half values (round to nearest even), the others as
 * asymmetric uint8 codes with an fp32 scale and zero point, refit every step.
 * 9.44 bits per value.  A step is the scalar-decay delta rule in the rotated
 * coordinates: vt = Hs v (exact sum in double, rounded once), ut = k^T St,
 * wt = beta*(vt - alpha*ut), St' = alpha*St + k wt^T on the stored rows in
 * fp32 (half values, uint8 rows reconstructed as fl(s*fl(c - z))), each entry
 * fma(alpha, St_ij, fl(k_i*wt_j)), and o = 2 Hs (St'^T q).  ssq_dequant
 * returns S = 2 St Hs. */
#define SSQ_DAMP_NHI 16

typedef enum { SSQ_MAMBA2 = 0, SSQ_DELTA = 1 } ssq_kind;

typedef enum { SSQ_READ_POST_QUANT = 0, SSQ_READ_PRE_QUANT = 1 } ssq_readout;

typedef enum { SSQ_ROUND_NEAREST = 0, SSQ_ROUND_STOCHASTIC = 1 } ssq_rounding;

/* Shape and format of one layer's state for all sequences of a batch. */
typedef struct {
    int32_t kind;          /* ssq_kind */
    int32_t format;        /* ssq_format */
    int32_t batch;         /* sequences */
    int32_t nheads;        /* heads */
    int32_t ngroups;       /* SSQ_MAMBA2: B/C groups, each shared by nheads/ngroups heads; SSQ_DELTA: 1 */
    int32_t rows_per_head; /* SSQ_MAMBA2: head dimension P; SSQ_DELTA: key dimension dk */
    int32_t row_len;       /* SSQ_MAMBA2: state size N; SSQ_DELTA: value dimension dv */
} ssq_desc;

/* Byte layout of a state in its storage (public, so that checkpoints and
 * tests can read it):
 *   codes  at codes_offset: rows x row_len*bits/8 bytes, row-major with rows
 *          ordered [batch][nheads][rows_per_head]; int4 puts entry 2j in the
 *          low nibble of byte j.  For SSQ_FP32 this region is the fp32 state.
 *   scale  at scale_offset: one fp32 per row (quantized formats, else 0)
 *   zero   at zero_offset:  one fp32 per row (asymmetric formats, else 0)
 *   SSQ_DAMP: codes, scale and zero hold the uint8 rows only,
 *          [batch][nheads][dk - SSQ_DAMP_NHI], and the half rows sit at
 *          hi_offset.  `rows` counts every key row.
 *   counter at counter_offset (quantized formats, else 0): the uint64 token
 *          the next stochastically rounded call starts at (see ssq_set_rounding)
 * Every region starts 256-byte aligned; ssq_alloc_state writes every byte of
 * the storage (padding 0).  A zero state has all bytes 0. */
typedef struct {
    size_t rows;
    size_t row_bytes;
    size_t codes_offset;
    size_t scale_offset;
    size_t zero_offset;
    size_t total_bytes;
    size_t hi_offset; /* SSQ_DAMP: the half rows [batch][nheads][SSQ_DAMP_NHI][128]; else 0 */
    size_t counter_offset; /* quantized formats: the stochastic-rounding token counter; else 0 */
} ssq_layout;

typedef struct ssq_state ssq_state; /* opaque handle: one layer's state */

/* Size in bytes of the storage a state with this description needs (the
 * layout's total_bytes), or 0 if the description is invalid.  For 30 delta
 * layers of batch 256 x 32 heads x 128 x 128 fp32 this is 30 x 512 MiB =
 * 15 GiB, the 15 GB of recurrent state at decode batch 256 reported in
 * "Recurrent state is fixed per request, not free". */
size_t ssq_state_bytes(const ssq_desc *desc);

/* Fill *layout for desc.  SSQ_ERR_INVALID_ARG / SSQ_ERR_UNSUPPORTED as for
 * ssq_alloc_state. */
ssq_status ssq_state_layout(const ssq_desc *desc, ssq_layout *layout);

/* Create a state.  storage: device memory of at least ssq_state_bytes(desc)
 * bytes, 256-byte aligned, owned by the caller and outliving the handle; or
 * NULL, and the library allocates it (hipMalloc) and frees it in
 * ssq_free_state.  init: NULL for the zero state, else a device pointer to
 * the fp32 state [batch][nheads][rows_per_head][row_len] that is quantized
 * row by row with the refit above (the prompt's state written into the
 * cache, "Mamba state quantization needs phase-aware benchmarks").  The
 * storage is written on `stream`.  *out receives the handle. */
ssq_status ssq_alloc_state(const ssq_desc *desc, void *storage, const float *init, void *stream,
                           ssq_state **out);

/* Destroy a handle: the end of a request, whose fixed-size state is then no
 * longer held ("Mamba state quantization for inference", "Recurrent state is
 * fixed per request, not free": every active request owns one).  Frees the
 * storage only if the library allocated it.  NULL is accepted.  The caller
 * must make sure no enqueued call still uses the state. */
ssq_status ssq_free_state(ssq_state *state);

/* The description, storage pointer and layout of a state (any out pointer
 * may be NULL). */
ssq_status ssq_state_info(const ssq_state *state, ssq_desc *desc, void **storage, ssq_layout *layout);

/* How the state's codes are rounded by the calls below ("ssm-state-quantization"
 * README, Findings 9: stochastic rounding of the state as the alternative to
 * round to nearest).  SSQ_ROUND_NEAREST (the default) is the rule above.
 * SSQ_ROUND_STOCHASTIC keeps the same grid (scale, zero point) and sets each
 * code to floor(v + U) for the exact real v = h'*inv + z', clamped to the
 * code range, so a row rounds up with probability equal to the fractional
 * part of v taken down to a multiple of 2^-16.  Entry n of state row r at
 * token t draws U = K * 2^-16 for the counter ctr = (t*rows + r)*row_len + n:
 * K is bits 16k .. 16k+15, k = ctr mod 4, of SplitMix64 output number
 * ctr/4 + 1 for `seed` (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), rows = the state's rows (for the two-tier
 * state, its uint8 rows).
 * `step` is the token the next call starts at.  It is kept in the state's
 * storage (the layout's counter), so it belongs to the stream's order, not to
 * the host: in SSQ_ROUND_STOCHASTIC mode ssq_decode_step and ssq_delta_step
 * use it and advance it by one, ssq_scan and ssq_prefill use step .. step+T-1
 * and advance it by T, with a one-thread kernel the call enqueues after its
 * step kernels (round to nearest leaves it as it is, and enqueues none).  A call captured in a graph
 * therefore draws the next tokens' uniforms at every replay.  The storage
 * bytes plus this mode and seed are all a state holds: copied into new
 * storage under a new handle with the same mode and seed they continue bit
 * for bit.  The fp32 state is never rounded and has no counter:
 * SSQ_ROUND_STOCHASTIC on it, or a non-zero step, gives SSQ_ERR_UNSUPPORTED.
 * Mode and seed take effect for calls made after this one; the counter is
 * written on `stream` (a one-thread kernel, so this call may also be
 * captured). */
ssq_status ssq_set_rounding(ssq_state *state, int32_t mode, uint64_t seed, uint64_t step, void *stream);

/* The state's rounding mode, seed and next token (any out pointer may be
 * NULL).  Reading the token copies it from device memory on `stream` and
 * waits for the stream to reach that copy. */
ssq_status ssq_get_rounding(const ssq_state *state, int32_t *mode, uint64_t *seed, uint64_t *step,
                            void *stream);

/* One Mamba-2 decode token for every row of the layer (README, Setup: decay
 * lambda = exp(dt*A) per head, write dt*B*x, per-row refit every step, round
 * to nearest; output read from the state selected by `readout`).
 *   x [batch][nheads][P], dt [batch][nheads] (positive, already through
 *   softplus), A [nheads] (negative), B, C [batch][ngroups][N], D [nheads];
 *   y [batch][nheads][P] is written.  The state is updated in place. */
ssq_status ssq_decode_step(ssq_state *state, const float *x, const float *dt, const float *A,
                           const float *B, const float *C, const float *D, float *y,
                           int32_t readout, void *stream);

/* T Mamba-2 tokens in one launch, the state rounded after every token (the
 * sequential per-token scan of the README's Setup, which rounds the state at
 * every step).  The state it leaves and every y are bit-identical to T calls
 * of ssq_decode_step, in every format.
 *   x [batch][T][nheads][P], dt [batch][T][nheads], B, C [batch][T][ngroups][N],
 *   A, D [nheads]; y [batch][T][nheads][P] is written. */
ssq_status ssq_scan(ssq_state *state, int32_t T, const float *x, const float *dt, const float *A,
                    const float *B, const float *C, const float *D, float *y, int32_t readout,
                    void *stream);

/* A prompt of T tokens with the state quantized only at chunk ends ("Mamba
 * state quantization for inference", "Mamba state quantization needs
 * phase-aware benchmarks": DAMP computes the prefill recurrence in FP32 inside
 * each chunk and writes the chunk-final state into the packed cache, which
 * decode then reads and rewrites).  Each row is dequantized once,
 * fl(s*fl(c - z)); every token applies h'_n = fma(lambda, h_n, fl(w*B_n)) in
 * fp32 and y is read from that fp32 row; after every `chunk` tokens and after
 * the last one the row is refit and rounded (the state's rounding mode; a
 * stochastic chunk end at token t draws the uniforms of token step + t), y of
 * that token follows `readout`, and the row continues from its dequantized new
 * codes.  The fp32 state runs the plain fp32 recurrence (the scan).  Shapes as
 * ssq_scan; T > 0, chunk > 0 (a chunk of T or more quantizes once, at the
 * end). */
ssq_status ssq_prefill(ssq_state *state, int32_t T, int32_t chunk, const float *x, const float *dt,
                       const float *A, const float *B, const float *C, const float *D, float *y,
                       int32_t readout, void *stream);

/* One delta-rule step for every (sequence, head) matrix S:
 *   S' = alpha*(I - beta*k*k^T)*S + beta*k*v^T,  o = S'^T q
 * ("Mamba state quantization for inference": the query reads the matrix,
 * decay and a delta-rule correction write the next version; the update
 * S_t = A_t S_(t-1) + W_t of "Quantization error returns on the next token"),
 * evaluated on the reconstructed matrix S_ij = fl(s_i*fl(c_ij - z_i)) (the
 * fp32 state as stored): u = k^T S (products and sum in double, rounded
 * once), w_j = fl(beta*fl(v_j - fl(alpha*u_j))), S'_ij = fma(alpha, S_ij,
 * fl(k_i*w_j)), then each key row refit and rounded as above.
 *   q, k [batch][nheads][dk], v [batch][nheads][dv], alpha, beta
 *   [batch][nheads]; o [batch][nheads][dv] is written. */
ssq_status ssq_delta_step(ssq_state *state, const float *q, const float *k, const float *v,
                          const float *alpha, const float *beta, float *o, int32_t readout,
                          void *stream);

/* One Kimi-Delta-Attention-style step: the delta rule with a decay per key
 * channel ("Mamba state quantization for inference" names KDA beside Gated
 * DeltaNet and reports persistence differing across KDA key channels):
 *   S' = (I - beta*k*k^T) * Diag(alpha) * S + beta*k*v^T,  o = S'^T q
 * evaluated on the reconstructed matrix S_ij = fl(s_i*fl(c_ij - z_i)):
 * u = k^T Diag(alpha) S (products and sum in double, rounded once),
 * w_j = fl(beta*fl(v_j - u_j)), S'_ij = fma(alpha_i, S_ij, fl(k_i*w_j)), then
 * each key row refit and rounded as above.
 *   alpha [batch][nheads][dk] (each in (0, 1]); q, k, v, beta, o as in
 *   ssq_delta_step.  Errors as ssq_delta_step. */
ssq_status ssq_kda_step(ssq_state *state, const float *q, const float *k, const float *v,
                        const float *alpha, const float *beta, float *o, int32_t readout,
                        void *stream);

/* The fp32 value the state stands for, fl(s*fl(c - z)) per entry (the stored
 * fp32 for SSQ_FP32): the reconstruction every step starts from ("Mamba
 * state quantization for inference", "Mixed precision spends bits on
 * persistent channels": the low tier is reconstructed before the FP32
 * recurrence; README, Setup: a row's value is its scale times its code
 * offset by the zero point).  out [batch][nheads][rows_per_head][row_len]. */
ssq_status ssq_dequant(const ssq_state *state, float *out, void *stream);

/* A streaming copy of `bytes` bytes from device memory src to device memory dst,
 * enqueued on `stream`: the plain read-and-write kernel a state step's bandwidth is
 * compared with on the same device (one 16-byte load and store per lane, with the
 * non-temporal hint).  Not part of the state update.  bytes: a multiple of 16, at most
 * 2^40 (0 enqueues nothing); dst and src 16-byte aligned and not overlapping, else
 * SSQ_ERR_INVALID_ARG before anything is enqueued.  The caller owns both buffers. */
ssq_status ssq_stream_copy(void *dst, const void *src, size_t bytes, void *stream);

/* Static text for a status code (an ssq_status value); any other value gives
 * "unknown ssq_status".  Taken as int32_t so that an out-of-range code is an
 * ordinary argument, not an invalid enum value. */
const char *ssq_status_string(int32_t status);

/* Detail of the last failed call on this thread ("" if none). */
const char *ssq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSQ_H */
