// launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Validated problem sizes; io = 0 (fp32) or 1 (bf16).
struct Shape {
    int64_t b, L, H, P, N, G, Q, nC;
    int io;
};

// dt front-end, applied where dt is read: d = raw (+ bias[h]); softplus; clamp to
// [lo, hi]; the decay uses d and the input term d, or (exp(d A) - 1) / A with zoh.
// All zero = the raw dt is the step.
struct DtFront {
    const float* bias;
    int softplus, zoh, clamp;
    float lo, hi;
};

hipError_t launch_chunk_cumsum(const Shape& s, const DtFront& fe, const void* dt, const float* A, float* dt_t,
                               float* cs, hipStream_t st);
hipError_t launch_chunk_state(const Shape& s, const void* x, const void* B, const float* dt_t,
                              const float* cs, float* states, hipStream_t st);
hipError_t launch_state_passing(const Shape& s, float* states, const float* cs, const float* h0,
                                float* final_state, hipStream_t st);
hipError_t launch_chunk_scan(const Shape& s, const void* x, const void* B, const void* C, const float* dt_t,
                             const float* cs, const float* start, const float* D, void* y, hipStream_t st);
// The generic chunk kernels alone, with inputs x, B, C in dtype in_io (0 fp32, 1 bf16; bf16
// compute needs bf16 inputs), computing in s.io, and head h reading x head h / xrep.
hipError_t launch_chunk_state_in(const Shape& s, int in_io, int xrep, const void* x, const void* B,
                                 const float* dt_t, const float* cs, float* states, hipStream_t st);
hipError_t launch_chunk_scan_in(const Shape& s, int in_io, int xrep, const void* x, const void* B, const void* C,
                                const float* dt_t, const float* cs, const float* start, const float* D, void* y,
                                hipStream_t st);
hipError_t launch_step(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, void* y, hipStream_t st);
// K = s.L decode steps over pre-staged (b, K, ...) inputs; the state stays on chip
// when N / 16 is 4, 8, 16, 32 or 64 and P * N <= 16384 (a 16 x 16 thread grid of
// P/16 x N/16 register blocks), else one launch per step.
bool step_multi_on_chip(const Shape& s);
hipError_t launch_step_multi(const Shape& s, const DtFront& fe, float* state, const void* x, const void* dt,
                             const float* A, const void* B, const void* C, const float* D, void* y, hipStream_t st);

// Where the fast kernels read x: rows of hx heads, and the head pair starting at head h0 reads the x heads
// h0 / div * mul and the next one.  The identity is {H, 1, 1}.  The backward's transposed scans run
// 2H half-heads (the two 64-column halves of each head) whose x is B or C of the head's group:
// {2G, 2 H / G, 2}.  rows > 0 (chunk state and chunk scan only, L a multiple of 64): the inputs x, B and
// C hold `rows` tokens per batch row in forward time and the kernels walk them backwards -- their token
// t (of L) is input row L - 1 - t, and the tokens t < L - rows (past the inputs' start) read as zero.
// The chunk scan then writes its output in forward time too (`rows` rows per batch row, nothing for the
// padding tokens), as y = s * (C.S + in-chunk term) + D x with s = rowscale[b, row, h] (an io-dtype
// (b, rows, H) array, e.g. the step dt) or 1 when rowscale is NULL.
// tap (chunk scan over sub-chunk-local decay arrays): the fp32 state the kernel carries is also stored
// at every position that is a multiple of tapq (the state entering it), as (b, L / tapq, H, P, N), and
// the state update then splits its scaled operand into hi + lo bf16 (fp32-level states).  tap_tr > 0:
// the scan is a transposed one with tap_tr half-heads per head, and its taps go to the original heads'
// layout (b, L / tapq, H / tap_tr, N, 64 tap_tr): kernel head h2's state row i and column j become element
// (j, 64 (h2 % tap_tr) + i) of head h2 / tap_tr.  start_tr: the chunk-start states are those of a
// transposed scan, (b, nC, (N / 64) H, 64, P).
struct XMap {
    int hx, div, mul;
    int64_t rows;
    const void* rowscale;
    float* tap;
    int tapq;
    int start_tr;
    int tap_tr;
};
// The backward's chunk kernels over sub-chunk-local decay arrays (dtl, lw: (b, H, ceil(L / 64), 64), from
// launch_subchunk_decay_bwd), with the reading options of XMap; the chunk state also writes each chunk's
// total log2 decay (b, H, nC) for the state pass (run with Q = 1 over those totals).  dstate 64 or 128.
hipError_t launch_chunk_state_sub(const Shape& s, const void* x, const void* B, const float* dtl, const float* lw,
                                  float* states, float* totals, hipStream_t st, const XMap* xm);
hipError_t launch_chunk_scan_sub(const Shape& s, const void* x, const void* B, const void* C, const float* dtl,
                                 const float* lw, const float* start, const float* D, void* y, hipStream_t st,
                                 const XMap* xm);
// Up to three sets of sub-chunk-local decay arrays in one launch.  A set covers H kernel heads over L
// tokens (b batch rows) from a bf16 dt of (b, Ls, H / hdiv): kernel head h takes dt head h / hdiv and
// A[h / hdiv]; rev: token t takes the decay step of dt row L - t (none where that row is past the end);
// unit: the input step is 1.
struct DecaySet {
    float *dtl, *lw;
    int64_t b, L, Ls;
    int H, hdiv;
    bool rev, unit;
};
hipError_t launch_subchunk_decay_bwd_sets(const DecaySet* sets, int nsets, const void* dt, const float* A,
                                          hipStream_t st);
// Fast chunk-state / chunk-scan kernels (bf16, headdim 64, dstate 64 or 128, chunk a multiple of 64).
bool fast_chunk_supported(const Shape& s);
int fast_forward_chunk(const Shape& s);   // chunk size the forward uses on the fast path
int fast_heads_per_wg(const Shape& s);
hipError_t launch_chunk_state_fast(const Shape& s, const void* x, const void* B, const float* dt_t, const float* cs,
                                   float* states, hipStream_t st, const XMap* xm = nullptr);
hipError_t launch_chunk_scan_fast(const Shape& s, const void* x, const void* B, const void* C, const float* dt_t,
                                  const float* cs, const float* start, const float* D, void* y, hipStream_t st,
                                  const XMap* xm = nullptr);

// The forward on the fast path: the decays restart at every 64-token sub-chunk (one coalesced pass over
// dt writes them, or, for short inputs at dstate <= 128, the chunk kernels form them from dt themselves),
// the chunk states also yield each chunk's total decay, the state pass runs over those totals, then the
// output kernel.  Workspace byte offsets: dt and decay (b, H, ceil(L/64), 64; empty when the kernels form
// them), chunk states (b, nC, H, P, N), chunk totals (b, H, nC), all fp32.
struct FastFwdLayout {
    size_t dtl, lw, states, totals, total;
};
FastFwdLayout fast_forward_layout(const Shape& s);
hipError_t launch_forward_fast(const Shape& s, const DtFront& fe, const void* x, const void* dt, const float* A,
                               const void* B,
                               const void* C, const float* D, const float* h0, void* y, float* final_state,
                               void* workspace, hipStream_t st);

// Mamba-1 selective scan (selective.hip): x, delta, y (b, L, Dc); A (Dc, N); B, C
// (b, L, G, N); D (Dc); h0, final (b, Dc, N).  Supported: N in {16, 32, 48, 64}
// and Dc / G a multiple of 16.  The sequence runs in nseg segments of seg_len
// tokens (a multiple of 64); with more than one segment the workspace holds the
// segment states (b, nseg - 1, Dc, N) and step sums (b, nseg - 1, Dc), fp32.
struct SelectiveLayout {
    int64_t seg_len;
    int nseg;
    size_t states, sums, total;
};
bool selective_supported(int64_t Dc, int64_t N, int64_t G);
SelectiveLayout selective_layout(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G, int64_t seg_len);
hipError_t launch_selective_scan(int64_t b, int64_t L, int64_t Dc, int64_t N, int64_t G, int io, const DtFront& fe,
                                 const void* x, const void* delta, const float* A, const void* B, const void* C,
                                 const float* D, const float* h0, void* y, float* final_state, int64_t seg_len,
                                 void* workspace, hipStream_t st);

// Backward pass (backward.hip): three fp32 chunked scans on converted copies of the
// inputs.  Byte offsets of the workspace pieces (all 256-byte aligned).
struct BackwardLayout {
    size_t xr, dyr, Cr, Br, drev, dfwd, dt_t, cs, states, u_r, v_r, w, G0, dfT, h0T, finT, fscr, q, dxy,
        dA_part, dD_part, states_b, R, sub, totals, stT, cbt, total;
    int64_t Qt;  // chunk of the half-head transposed scans (local flow)
    int64_t Lr;  // rows of the time-reversed copies (the sequence, front-padded to whole chunks when local)
    bool local;  // the decay gradient is formed chunk by chunk (decay_grad.hip)
};
// The chunk-local decay gradient (decay_grad.hip): bf16 io, headdim 64, dstate 64 or 128, chunk 64 or 128
// (a multiple of 64 for the fast chunk kernels that supply its states, at most 128 for its tiles).
bool decay_grad_supported(const Shape& s);
// R (b, H, L): R_k = a_k <G_k, S_{k-1}> from the step dt (b, L, H) bf16 and A (the chunks' decays are
// formed in the kernel), the forward chunk-start states S0 (b, nC, H, P, N) and the reversed adjoint
// scan's chunk-start states Gst (same layout, reversed chunk order); dxy (b, H, L) = dy_t . x_t.  cbt:
// scratch of decay_grad_tile_bytes(s) bytes for the chunks' C . B tiles (shared by the heads of a group).
size_t decay_grad_tile_bytes(const Shape& s);
hipError_t launch_decay_grad(const Shape& s, const void* x, const void* dy, const void* B, const void* C,
                             const void* dt, const float* A, const float* S0, const float* Gst, float* cbt, float* R,
                             float* dxy, hipStream_t st);
BackwardLayout backward_layout(const Shape& s);
hipError_t launch_backward(const Shape& s, const void* x, const void* dt, const float* A, const void* B,
                           const void* C, const float* D, const float* h0, const void* dy, const float* dfinal,
                           void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, void* workspace,
                           hipStream_t st);

// The static device scratch of ssd_forward_noalloc (noalloc.hip): its size, and its
// device address on the current device (taken with hipGetSymbolAddress on the first
// call per device, then cached).
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
hipError_t static_scratch(void** ptr);

// LDS bytes the generic chunk kernels need; used by validation.
size_t chunk_state_lds_bytes(const Shape& s);
size_t chunk_scan_lds_bytes(const Shape& s);

}  // namespace ssd
