/*
 * ssd.h -- C ABI of libssd, a gfx950 (MI355X) implementation of the Mamba-2
 * state-space-duality (SSD) chunked forward scan and its O(1) decode step.
 *
 * What is computed.  For batch row b and head h (group g = h / (H/G)):
 *     S_t = exp(dt_t * A_h) * S_{t-1} + dt_t * x_t (outer) B_t        (P x N)
 *     y_t = C_t . S_t + D_h * x_t
 * with S_{-1} = h0 (or 0).  The decay exp(delta*A) is the discretisation of
 * "3.3 Hardware-Aware algorithms and GPU memory hierarchy optimisation",
 * section 2.1; the recurrence and its output through C are its sections 3 and
 * 4.1.  Mamba-2 uses one scalar A per head and the input term dt * B.
 * The chunked method cuts the sequence into chunks of Q tokens and splits the
 * work into an in-chunk cumulative sum of dt*A, chunk states, a chunk-order
 * state pass and a fused in-chunk output -- the three kernels described on the
 * devotd.net page on the NVIDIA / Jane Street cuTile Mamba-2 forward kernels,
 * section 2 (the state kernel is split here into two calls).  The decode step
 * is the fixed-size, on-device state update of "Compiler-First State Space
 * Duality and Portable O(1) Autoregressive Caching for Inference",
 * Methodology.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers, contiguous, row-major, in the
 *     layouts listed below.  `stream` is a hipStream_t passed as void* (NULL =
 *     the null stream).  Calls only enqueue work; they never synchronise.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory and keeps no state between calls (a per-thread error
 *     string aside), so it is re-entrant across threads and streams.
 *   - Arguments are validated before anything is enqueued; a non-OK status
 *     means nothing was launched, and ssd_last_error() describes why.
 *     SSD_ERR_HIP is returned when a launch itself fails.  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - x, B, C, y, h0, final_state, states and the decode state must be
 *     16-byte aligned (the kernels move them in 16-byte vectors); a
 *     misaligned pointer returns SSD_ERR_UNSUPPORTED.  dt, A, D and the
 *     per-position float32 arrays have no alignment rule beyond their type.
 *   - io dtype (ssd_dims.io) is the element type of x, dt, B, C and y:
 *     SSD_F32 (float) or SSD_BF16 (bfloat16).  A, D, h0, the final state, the
 *     decode state and every intermediate are float32.
 *
 * Layouts (b = batch, L = seqlen, H = nheads, P = headdim, N = dstate,
 * G = ngroups, Q = chunk, nC = ceil(L / Q)):
 *     x, y              (b, L, H, P)        io dtype
 *     dt                (b, L, H)           io dtype   (final positive step)
 *     A, D              (H)                 float32    (A < 0 expected)
 *     B, C              (b, L, G, N)        io dtype
 *     h0, final_state   (b, H, P, N)        float32
 *     dt_t, dA_cs_log2  (b, H, nC, Q)       float32
 *     states            (b, nC, H, P, N)    float32
 *     step: x, y (b, H, P); dt (b, H); B, C (b, G, N); state (b, H, P, N)
 * Tokens at positions >= L inside the last chunk are treated as dt = 0,
 * which leaves the state unchanged; their rows are never written.
 *
 * Supported sizes: P and N multiples of 16 with P <= 256 and N <= 1024;
 * Q a multiple of 16 in [16, 512] -- or a multiple of 64 up to 4096 for bf16
 * with P = 64 and N in {64, 128, 256, 512}, the shapes served by the fast chunk
 * kernels; H divisible by G; b, L >= 0 (an empty batch or sequence is a valid
 * no-op).  Other sizes return SSD_ERR_UNSUPPORTED.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 1

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a dimension is negative/zero where it must not be, or H % G != 0 */
    SSD_ERR_DTYPE = 3,       /* io is not SSD_F32 or SSD_BF16 */
    SSD_ERR_UNSUPPORTED = 4, /* sizes outside the supported set (see above) */
    SSD_ERR_WORKSPACE = 5,   /* workspace missing or smaller than ssd_forward_workspace_bytes() */
    SSD_ERR_ALIAS = 6,       /* an output overlaps an input it may not overlap */
    SSD_ERR_HIP = 7          /* a HIP launch failed; see ssd_last_error() */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
    int64_t batch;    /* b */
    int64_t seqlen;   /* L */
    int64_t nheads;   /* H */
    int64_t headdim;  /* P */
    int64_t dstate;   /* N */
    int64_t ngroups;  /* G: head h reads B, C of group h / (H / G) */
    int64_t chunk;    /* Q; 0 = let ssd_forward choose (the staged calls need Q > 0) */
    int32_t io;       /* ssd_dtype of x, dt, B, C, y */
    int32_t reserved; /* must be 0 */
} ssd_dims;

/*
 * Optional dt front-end of the *_ex calls, applied wherever the kernels read
 * dt (the plain calls behave as if it were all zero: dt is the final step).
 * For head h, with d the raw dt:
 *     d <- d + dt_bias[h]                    (dt_bias: (H) float32, or NULL)
 *     d <- log(1 + exp(d))                   if softplus
 *     d <- min(max(d, dt_min), dt_max)       if clamp
 * d is then the decay step (exp(d A)).  The input term uses d, or with zoh
 * the zero-order-hold factor (exp(d A) - 1) / A (d where A == 0): the
 * scalar-A form of the ZOH discretisation B-bar in "3.3 Hardware-Aware
 * algorithms and GPU memory hierarchy optimisation", section 2.1.  In
 * ssd_chunk_cumsum_ex, dt_t receives that input step and dA_cs_log2 sums the
 * decay steps, so ssd_chunk_state and ssd_chunk_scan need no change.
 * reserved must be 0; clamp needs finite dt_min <= dt_max (SSD_ERR_SHAPE
 * otherwise); dt_bias must not overlap any output.
 */
typedef struct {
    const float* dt_bias; /* (H) float32 device pointer, or NULL */
    int32_t softplus;     /* nonzero: d <- softplus(d) */
    int32_t zoh;          /* nonzero: zero-order-hold input step (exp(d A) - 1) / A */
    int32_t clamp;        /* nonzero: d <- min(max(d, dt_min), dt_max) after the softplus */
    int32_t reserved;     /* must be 0 */
    float dt_min, dt_max;
} ssd_dt_frontend;

/*
 * In-chunk cumulative sum (cuTile page, section 2, first kernel and its
 * listing): for chunk c and position i < Q,
 *     dA_cs_log2[b,h,c,i] = log2(e) * sum_{k<=i} dt[b,cQ+k,h] * A[h]
 *     dt_t[b,h,c,i]       = dt[b,cQ+i,h] as float32
 * (log2 units, so later stages decay with exp2).  Positions past L read 0.
 * dt_t and dA_cs_log2 must not overlap dt or A, nor each other.
 */
ssd_status ssd_chunk_cumsum(const ssd_dims* dims, const void* dt, const float* A,
                            float* dt_t, float* dA_cs_log2, void* stream);

/*
 * Chunk-local states (cuTile page, section 2, first half of the state kernel):
 * the state each chunk produces from a zero start,
 *     states[b,c,h,p,n] = sum_{j<Q} 2^(l[Q-1] - l[j]) * dt_t[j] * x[b,cQ+j,h,p] * B[b,cQ+j,g,n]
 * with l = dA_cs_log2[b,h,c,:].  states must not overlap any input.
 */
ssd_status ssd_chunk_state(const ssd_dims* dims, const void* x, const void* B,
                           const float* dt_t, const float* dA_cs_log2,
                           float* states, void* stream);

/*
 * Chunk-order state passing (cuTile page, section 2, second half of the state
 * kernel: chunk order kept, independent state elements in parallel).  On
 * entry states holds the chunk-local states; on return it holds the state
 * BEFORE each chunk:
 *     S_0 = h0 (or 0),  states[c] <- S_c,  S_{c+1} = 2^(l_c[Q-1]) S_c + local_c,
 *     final_state = S_nC.
 * h0 may be NULL.  final_state must not overlap states, h0 or dA_cs_log2.
 */
ssd_status ssd_state_passing(const ssd_dims* dims, float* states, const float* dA_cs_log2,
                             const float* h0, float* final_state, void* stream);

/*
 * Chunk output from the chunk-start states (cuTile page, section 2, third
 * kernel), for i < Q in chunk c:
 *     y_i = 2^(l_i) C_i . S_c + sum_{j<=i} (C_i . B_j) 2^(l_i - l_j) dt_t[j] x_j + D_h x_i
 * The in-chunk matrix stays in registers and LDS.  D may be NULL (no skip
 * term).  y must not overlap any input.
 */
ssd_status ssd_chunk_scan(const ssd_dims* dims, const void* x, const void* B, const void* C,
                          const float* dt_t, const float* dA_cs_log2,
                          const float* chunk_start_states, const float* D,
                          void* y, void* stream);

/* ssd_chunk_cumsum with the dt front-end above (fe may be NULL). */
ssd_status ssd_chunk_cumsum_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* dt,
                               const float* A, float* dt_t, float* dA_cs_log2, void* stream);

/* Bytes of device workspace ssd_forward needs for these dims (0 on invalid dims). */
size_t ssd_forward_workspace_bytes(const ssd_dims* dims);

/*
 * One-shot forward: y and the final state from (x, dt, A, B, C, D, h0), the
 * four stages above composed (or fused) on `stream`.  dims->chunk = 0 lets
 * the library pick the chunk size; the result does not depend on it beyond
 * rounding.  D and h0 may be NULL.  workspace must hold at least
 * ssd_forward_workspace_bytes(dims) bytes (256-byte aligned) and may not
 * overlap anything else; its contents on entry are ignored.  y and
 * final_state must not overlap the inputs.
 */
ssd_status ssd_forward(const ssd_dims* dims, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* h0,
                       void* y, float* final_state, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ssd_forward with the dt front-end above (fe may be NULL); same workspace. */
ssd_status ssd_forward_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* x, const void* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          const float* h0, void* y, float* final_state, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * ssd_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The forward's intermediates go to a static device
 * scratch of 128 MiB that the library holds on each GPU it runs on until the
 * process ends; this call allocates nothing and frees nothing.  Shapes whose
 * ssd_forward_workspace_bytes() exceeds 128 MiB return SSD_ERR_WORKSPACE
 * (the 2.7B-shaped forward at 64K tokens needs about 108 MB).  All other
 * arguments, validation and results are those of ssd_forward.  Every call on
 * one GPU shares that GPU's scratch: calls that may overlap in time on one GPU
 * (different streams, or different host threads) race and must be ordered by
 * the caller.  The first call on a device looks up the scratch's address.
 */
ssd_status ssd_forward_noalloc(const ssd_dims* dims, const void* x, const void* dt, const float* A,
                               const void* B, const void* C, const float* D, const float* h0,
                               void* y, float* final_state, void* stream);

/*
 * O(1) decode step for one token per (b, h), in place on state (dims->seqlen
 * must be 1; dims->chunk is ignored):
 *     S <- exp(dt A) S + dt x (outer) B;   y = C . S + D x   (after the update)
 * y must not overlap the inputs or the state.  D may be NULL.
 */
ssd_status ssd_step(const ssd_dims* dims, float* state, const void* x, const void* dt,
                    const float* A, const void* B, const void* C, const float* D,
                    void* y, void* stream);

/* ssd_step with the dt front-end above (fe may be NULL). */
ssd_status ssd_step_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, float* state, const void* x,
                       const void* dt, const float* A, const void* B, const void* C, const float* D,
                       void* y, void* stream);

/*
 * K decode steps in one call, over inputs that are all on the device before
 * the call (pre-staged: teacher forcing, scoring, speculative verification):
 * the on-device multi-step decode loop of the "Compiler-First State Space
 * Duality ..." page (Methodology; Results), with the state read from and
 * written to HBM once per call instead of once per step.  K = dims->seqlen
 * (K = 0 is a no-op); dims->chunk is ignored.  For k < K, in order:
 *     S <- exp(dt_k A) S + dt_k x_k (outer) B_k;   y_k = C_k . S + D x_k
 * Inputs use the forward's layouts with K as the sequence axis:
 *     x, y (b, K, H, P);  dt (b, K, H);  B, C (b, K, G, N);  state (b, H, P, N)
 * fp32, updated in place.  The result equals K calls of ssd_step on the
 * slices [:, k] (up to summation order in y).  state, x, B, C and y must be
 * 16-byte aligned (SSD_ERR_UNSUPPORTED otherwise); y must not overlap the
 * inputs or the state; D may be NULL.  The state stays in registers across
 * the K steps when P divides 256 and N / (256 / P) is 4, 8, 16, 32 or 64 (and
 * a block of 16 steps fits 64 KiB of LDS); other shapes run one step kernel
 * per token on `stream`, still without a host round trip.
 */
ssd_status ssd_step_multi(const ssd_dims* dims, float* state, const void* x, const void* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          void* y, void* stream);

/* ssd_step_multi with the dt front-end above (fe may be NULL). */
ssd_status ssd_step_multi_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, float* state,
                             const void* x, const void* dt, const float* A, const void* B,
                             const void* C, const float* D, void* y, void* stream);

/*
 * Backward pass of ssd_forward (plain input step dt, no front-end): the
 * gradients of a loss through y and the final state, for training ("3.3
 * Hardware-Aware algorithms and GPU memory hierarchy optimisation", section 6:
 * the forward's states are recomputed, not stored).  Given dy (the gradient
 * of y, layout of x) and dfinal (of the final state, (b, H, P, N) fp32, or
 * NULL for zero), it writes
 *     dx (b, L, H, P), ddt (b, L, H), dB, dC (b, L, G, N)   in the io dtype
 *     dA (H), dD (H), dh0 (b, H, P, N)                       float32
 * dB and dC sum over the heads of each group; dA and dD over batch rows and
 * tokens.  D, h0 and dfinal may be NULL (then D = 0, h0 = 0, dfinal = 0); dD
 * and dh0 may be NULL (not written).  dims->chunk is the chunk of the
 * internal scans: 0 for the library's choice, else a multiple of 16 up to 512
 * whose fp32 tiles fit LDS.  Supported: dstate <= 256 besides the forward's
 * limits (SSD_ERR_UNSUPPORTED otherwise).  The decay gradient is formed chunk
 * by chunk from each chunk's starting state and adjoint.  bf16 inputs with
 * headdim 64, dstate 64 or 128 and chunk 64 or 128 (the library's choice) run
 * every scan on the bf16 chunk kernels; other inputs run fp32 scans.
 * workspace: ssd_backward_workspace_bytes(dims) bytes, 256-byte aligned
 * (about (2 s + 4) P + 8 N + 2 s N G / H + 8 P N / chunk + 30 bytes per
 * token-head with fp32 scans, s = the io element size; on the bf16 chunk
 * kernels about max(2 N, 4 P N / chunk) + 4 P N / chunk + 2.5 chunk G / H +
 * 70 when H is a multiple of 4 and G N <= 1024, else 4 N + 8 P N / chunk +
 * 2.5 chunk G / H + 70); no output may
 * overlap an input, another output or the workspace.  x, B, C, dy, dx, dB,
 * dC, h0, dfinal and dh0 must be 16-byte aligned (SSD_ERR_UNSUPPORTED
 * otherwise).
 */
size_t ssd_backward_workspace_bytes(const ssd_dims* dims);
ssd_status ssd_backward(const ssd_dims* dims, const void* x, const void* dt, const float* A,
                        const void* B, const void* C, const float* D, const float* h0,
                        const void* dy, const float* dfinal, void* dx, void* ddt, float* dA,
                        void* dB, void* dC, float* dD, float* dh0, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Mamba-1 selective scan: a per-channel diagonal state with a per-entry decay
 * rate, discretised, scanned and read out through C in one fused call ("3.3
 * Hardware-Aware algorithms and GPU memory hierarchy optimisation": section
 * 2.1 for the discretisation abar = exp(delta A) and the zero-order-hold
 * bbar, section 3 for the fused load / discretise / scan / output steps,
 * section 4.1 for the associativity that lets the sequence run in segments).
 * For every batch row b and channel d (group g = d / (Dc / G)), n < N:
 *     h[n] <- h0[b, d, n] (or 0)
 *     for t < L:  e = exp(delta[b,t,d] A[d,n])
 *                 h[n] <- e h[n] + f x[b,t,d] B[b,t,g,n],
 *                        f = (e - 1) / A[d,n]  (zero-order hold; delta where A[d,n] == 0)
 *                        f = delta[b,t,d]      (without zoh)
 *                 y[b,t,d] = sum_n C[b,t,g,n] h[n] + D[d] x[b,t,d]
 *     final_state[b, d] = h
 * dims: batch = b, seqlen = L, nheads = the channel count Dc, headdim = 1,
 * dstate = N, ngroups = G, io = dtype of x, delta, B, C and y; chunk = the
 * length of the sequence segments the call scans in parallel (0: the
 * library's choice; otherwise a multiple of 64).  The result does not depend
 * on the segment length beyond rounding.
 * fe (may be NULL): the step front-end of ssd_dt_frontend, per channel
 * (dt_bias has Dc entries): delta <- clamp(softplus(delta + bias)); zoh
 * selects the zero-order-hold input (else delta B).  A NULL fe means the raw
 * delta is the step and the input is delta B.
 * Layouts (row-major, contiguous): x, delta, y (b, L, Dc); A (Dc, N) and D (Dc)
 * float32; B, C (b, L, G, N); h0, final_state (b, Dc, N) float32.  D and h0
 * may be NULL.  x, delta, B, C and y must be 16-byte aligned.
 * Supported: N in {16, 32, 48, 64} and Dc / G a multiple of 16
 * (SSD_ERR_UNSUPPORTED otherwise).
 * workspace: ssd_selective_scan_workspace_bytes(dims) bytes, 256-byte aligned
 * (NULL allowed when that is 0: a single segment).  y and final_state must not
 * overlap the inputs, each other or the workspace.
 */
size_t ssd_selective_scan_workspace_bytes(const ssd_dims* dims);
ssd_status ssd_selective_scan(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* x,
                              const void* delta, const float* A, const void* B, const void* C,
                              const float* D, const float* h0, void* y, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* ssd_status_string(ssd_status status);

/* Detail for the last non-OK status returned on the calling thread ("" if none). */
const char* ssd_last_error(void);

/* SSD_ABI_VERSION of the loaded library. */
int ssd_abi_version(void);

/*
 * The tiling ssd_forward would use for these dims: the chunk size, the
 * P-tile and the number of heads per workgroup of its output kernel, and the
 * number of 64-token sub-chunks its chunk kernels walk in registers per chunk
 * (1 = the generic kernels, which do not sub-chunk).  Any pointer may be NULL.
 */
ssd_status ssd_query_config(const ssd_dims* dims, int* chunk, int* tile_p, int* heads_per_wg,
                            int* chunks_per_segment);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
