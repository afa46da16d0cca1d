// api.cpp -- the C ABI of libssd: argument validation, workspace layout,
// tuning choice and launches.  Validation never touches the HIP runtime, so a
// rejected call enqueues nothing (and works on a machine without a GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>

#include "../../include/ssd.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

ssd_status fail(ssd_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

ssd_status ok() {
    g_last_error.clear();
    return SSD_OK;
}

ssd_status hip_fail(hipError_t e, const char* where) {
    return fail(SSD_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxGrid = 0x7fffffffLL;

// ---------------------------------------------------------------------------
// dims validation
// ---------------------------------------------------------------------------
enum class Need { kStaged, kCumsum, kForward, kStep, kStepMulti };

ssd_status check_dims(const ssd_dims* d, Need need, ssd::Shape* out) {
    if (!d) return fail(SSD_ERR_NULL, "dims is NULL");
    if (d->io != SSD_F32 && d->io != SSD_BF16) return fail(SSD_ERR_DTYPE, "io dtype %d is not SSD_F32/SSD_BF16", d->io);
    if (d->reserved != 0) return fail(SSD_ERR_SHAPE, "dims.reserved must be 0");
    if (d->batch < 0 || d->seqlen < 0) return fail(SSD_ERR_SHAPE, "batch and seqlen must be >= 0");
    if (d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
        return fail(SSD_ERR_SHAPE, "nheads, headdim, dstate and ngroups must be > 0");
    if (d->nheads % d->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "nheads (%lld) is not a multiple of ngroups (%lld)", (long long)d->nheads,
                    (long long)d->ngroups);
    if (d->chunk < 0) return fail(SSD_ERR_SHAPE, "chunk must be >= 0");
    if (d->headdim % 16 || d->headdim > 256)
        return fail(SSD_ERR_UNSUPPORTED, "headdim %lld: need a multiple of 16 up to 256", (long long)d->headdim);
    if (d->dstate % 16 || d->dstate > 1024)
        return fail(SSD_ERR_UNSUPPORTED, "dstate %lld: need a multiple of 16 up to 1024", (long long)d->dstate);
    ssd::Shape s{};
    s.b = d->batch;
    s.L = d->seqlen;
    s.H = d->nheads;
    s.P = d->headdim;
    s.N = d->dstate;
    s.G = d->ngroups;
    s.io = d->io;
    if (need == Need::kStep || need == Need::kStepMulti) {
        if (need == Need::kStep && d->seqlen != 1)
            return fail(SSD_ERR_SHAPE, "ssd_step needs seqlen == 1 (got %lld)", (long long)d->seqlen);
        if (s.b * s.H > kMaxGrid) return fail(SSD_ERR_UNSUPPORTED, "batch * nheads too large");
        s.Q = 1;
        s.nC = 1;
        *out = s;
        return SSD_OK;
    }
    int64_t Q = d->chunk;
    if (Q == 0) {
        if (need != Need::kForward) return fail(SSD_ERR_UNSUPPORTED, "the staged calls need an explicit chunk > 0");
        // the forward's own choice: a large chunk on the fast path, else 256
        s.Q = 64;
        Q = ssd::fast_chunk_supported(s) ? ssd::fast_forward_chunk(s) : 256;
    }
    s.Q = Q;
    // the cumulative sum has no headdim/dstate dependence: any chunk the other calls accept
    const bool fast = Q % 64 == 0 && (need == Need::kCumsum || ssd::fast_chunk_supported(s));
    if (Q % 16 || Q < 16 || Q > (fast ? 4096 : 512))
        return fail(SSD_ERR_UNSUPPORTED, "chunk %lld: need a multiple of 16 in [16, 512] (multiple of 64 up to "
                    "4096 for bf16 with headdim 64 and dstate 64/128/256/512)", (long long)Q);
    s.nC = (s.L + Q - 1) / Q;
    if (s.b * s.nC * s.H * s.N > kMaxGrid || s.H > 65535 || s.b > 65535)
        return fail(SSD_ERR_UNSUPPORTED, "problem too large for one launch grid");
    if (!fast && (ssd::chunk_scan_lds_bytes(s) > 160 * 1024 || ssd::chunk_state_lds_bytes(s) > 160 * 1024))
        return fail(SSD_ERR_UNSUPPORTED, "tile shapes exceed the 160 KiB LDS");
    *out = s;
    return SSD_OK;
}

// ---------------------------------------------------------------------------
// pointers and aliasing
// ---------------------------------------------------------------------------
struct Span {
    const void* p;
    size_t bytes;
    const char* name;
};

bool overlap(const Span& a, const Span& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

ssd_status need_ptr(const Span& s) {
    if (s.bytes > 0 && !s.p) return fail(SSD_ERR_NULL, "%s is NULL", s.name);
    return SSD_OK;
}

// The kernels read and write the io and state arrays with 16-byte vector accesses.
ssd_status need_align16(std::initializer_list<Span> spans) {
    for (const Span& p : spans)
        if (p.p && reinterpret_cast<uintptr_t>(p.p) % 16)
            return fail(SSD_ERR_UNSUPPORTED, "%s must be 16-byte aligned", p.name);
    return SSD_OK;
}

ssd_status no_alias(const Span& out, const Span* ins, int n) {
    for (int i = 0; i < n; ++i)
        if (overlap(out, ins[i])) return fail(SSD_ERR_ALIAS, "%s overlaps %s", out.name, ins[i].name);
    return SSD_OK;
}

// the dt front-end of the *_ex calls (NULL: the raw dt is the step)
ssd_status front_end(const ssd_dt_frontend* f, int64_t H, ssd::DtFront* out, Span* sbias) {
    *out = ssd::DtFront{nullptr, 0, 0, 0, 0.0f, 0.0f};
    *sbias = Span{nullptr, 0, "dt_bias"};
    if (!f) return SSD_OK;
    if (f->reserved != 0) return fail(SSD_ERR_SHAPE, "ssd_dt_frontend.reserved must be 0");
    if (f->clamp && !(std::isfinite(f->dt_min) && std::isfinite(f->dt_max) && f->dt_min <= f->dt_max))
        return fail(SSD_ERR_SHAPE, "the dt clamp needs finite dt_min <= dt_max");
    *out = ssd::DtFront{f->dt_bias, f->softplus != 0, f->zoh != 0, f->clamp != 0, f->dt_min, f->dt_max};
    *sbias = Span{f->dt_bias, f->dt_bias ? (size_t)H * 4 : 0, "dt_bias"};
    return SSD_OK;
}

#define SSD_TRY(expr)                       \
    do {                                    \
        ssd_status _st = (expr);            \
        if (_st != SSD_OK) return _st;      \
    } while (0)

size_t esz(const ssd::Shape& s) { return s.io == SSD_BF16 ? 2 : 4; }

struct Sizes {
    size_t x, dt, bc, A, hstate, cs, states;
};

Sizes sizes(const ssd::Shape& s) {
    Sizes z;
    z.x = (size_t)(s.b * s.L * s.H * s.P) * esz(s);
    z.dt = (size_t)(s.b * s.L * s.H) * esz(s);
    z.bc = (size_t)(s.b * s.L * s.G * s.N) * esz(s);
    z.A = (size_t)s.H * 4;
    z.hstate = (size_t)(s.b * s.H * s.P * s.N) * 4;
    z.cs = (size_t)(s.b * s.H * s.nC * s.Q) * 4;
    z.states = (size_t)(s.b * s.nC * s.H * s.P * s.N) * 4;
    return z;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct FwdLayout {
    size_t dt_t, cs, states, total;
};

FwdLayout fwd_layout(const ssd::Shape& s) {
    Sizes z = sizes(s);
    FwdLayout f;
    if (ssd::fast_chunk_supported(s)) {  // the fast forward keeps no per-position arrays
        f.dt_t = f.cs = f.states = 0;
        f.total = ssd::fast_forward_layout(s).total;
        return f;
    }
    f.dt_t = 0;
    f.cs = align256(z.cs);
    f.states = f.cs + align256(z.cs);
    f.total = f.states + align256(z.states);
    return f;
}

}  // namespace

extern "C" {

const char* ssd_status_string(ssd_status st) {
    switch (st) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "null pointer";
        case SSD_ERR_SHAPE: return "invalid shape";
        case SSD_ERR_DTYPE: return "invalid dtype";
        case SSD_ERR_UNSUPPORTED: return "unsupported size";
        case SSD_ERR_WORKSPACE: return "workspace too small";
        case SSD_ERR_ALIAS: return "forbidden aliasing";
        case SSD_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* ssd_last_error(void) { return g_last_error.c_str(); }

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

ssd_status ssd_query_config(const ssd_dims* dims, int* chunk, int* tile_p, int* heads_per_wg,
                            int* chunks_per_segment) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kForward, &s));
        const bool fast = ssd::fast_chunk_supported(s);
        if (chunk) *chunk = (int)s.Q;
        if (tile_p) *tile_p = 16;
        if (heads_per_wg) *heads_per_wg = fast ? ssd::fast_heads_per_wg(s) : 1;
        if (chunks_per_segment) *chunks_per_segment = fast ? (int)(s.Q / 64) : 1;
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

ssd_status ssd_chunk_cumsum_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* dt, const float* A,
                               float* dt_t, float* dA_cs_log2, void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kCumsum, &s));
        Sizes z = sizes(s);
        ssd::DtFront f;
        Span sbias;
        SSD_TRY(front_end(fe, s.H, &f, &sbias));
        Span sdt{dt, z.dt, "dt"}, sA{A, z.A, "A"}, sdtt{dt_t, z.cs, "dt_t"}, scs{dA_cs_log2, z.cs, "dA_cs_log2"};
        for (const Span& p : {sdt, sA, sdtt, scs}) SSD_TRY(need_ptr(p));
        Span ins[] = {sdt, sA, sbias};
        SSD_TRY(no_alias(sdtt, ins, 3));
        SSD_TRY(no_alias(scs, ins, 3));
        Span o1[] = {sdtt};
        SSD_TRY(no_alias(scs, o1, 1));
        hipError_t e = ssd::launch_chunk_cumsum(s, f, dt, A, dt_t, dA_cs_log2, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ssd_chunk_cumsum");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

ssd_status ssd_chunk_cumsum(const ssd_dims* dims, const void* dt, const float* A, float* dt_t, float* dA_cs_log2,
                            void* stream) {
    return ssd_chunk_cumsum_ex(dims, nullptr, dt, A, dt_t, dA_cs_log2, stream);
}

ssd_status ssd_chunk_state(const ssd_dims* dims, const void* x, const void* B, const float* dt_t,
                           const float* dA_cs_log2, float* states, void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kStaged, &s));
        Sizes z = sizes(s);
        Span sx{x, z.x, "x"}, sB{B, z.bc, "B"}, sdtt{dt_t, z.cs, "dt_t"}, scs{dA_cs_log2, z.cs, "dA_cs_log2"},
            sst{states, z.states, "states"};
        for (const Span& p : {sx, sB, sdtt, scs, sst}) SSD_TRY(need_ptr(p));
        SSD_TRY(need_align16({sx, sB, sst}));
        Span ins[] = {sx, sB, sdtt, scs};
        SSD_TRY(no_alias(sst, ins, 4));
        hipError_t e = ssd::launch_chunk_state(s, x, B, dt_t, dA_cs_log2, states, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ssd_chunk_state");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

ssd_status ssd_state_passing(const ssd_dims* dims, float* states, const float* dA_cs_log2, const float* h0,
                             float* final_state, void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kStaged, &s));
        Sizes z = sizes(s);
        Span sst{states, z.states, "states"}, scs{dA_cs_log2, z.cs, "dA_cs_log2"}, sh0{h0, h0 ? z.hstate : 0, "h0"},
            sfin{final_state, z.hstate, "final_state"};
        for (const Span& p : {sst, scs, sfin}) SSD_TRY(need_ptr(p));
        SSD_TRY(need_align16({sst, sh0, sfin}));
        Span ins[] = {sst, scs, sh0};
        SSD_TRY(no_alias(sfin, ins, 3));
        Span ins2[] = {scs, sh0};
        SSD_TRY(no_alias(sst, ins2, 2));
        hipError_t e = ssd::launch_state_passing(s, states, dA_cs_log2, h0, final_state, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ssd_state_passing");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

ssd_status ssd_chunk_scan(const ssd_dims* dims, const void* x, const void* B, const void* C, const float* dt_t,
                          const float* dA_cs_log2, const float* chunk_start_states, const float* D, void* y,
                          void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kStaged, &s));
        Sizes z = sizes(s);
        Span sx{x, z.x, "x"}, sB{B, z.bc, "B"}, sC{C, z.bc, "C"}, sdtt{dt_t, z.cs, "dt_t"},
            scs{dA_cs_log2, z.cs, "dA_cs_log2"}, sst{chunk_start_states, z.states, "chunk_start_states"},
            sD{D, D ? z.A : 0, "D"}, sy{y, z.x, "y"};
        for (const Span& p : {sx, sB, sC, sdtt, scs, sst, sy}) SSD_TRY(need_ptr(p));
        SSD_TRY(need_align16({sx, sB, sC, sst, sy}));
        Span ins[] = {sx, sB, sC, sdtt, scs, sst, sD};
        SSD_TRY(no_alias(sy, ins, 7));
        hipError_t e = ssd::launch_chunk_scan(s, x, B, C, dt_t, dA_cs_log2, chunk_start_states, D, y,
                                              (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ssd_chunk_scan");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

size_t ssd_forward_workspace_bytes(const ssd_dims* dims) {
    try {
        ssd::Shape s;
        if (check_dims(dims, Need::kForward, &s) != SSD_OK) return 0;
        return fwd_layout(s).total;
    } catch (...) {
        return 0;
    }
}

}  // extern "C"

namespace {

// ssd_forward_ex, or with use_static the same forward on the library's static scratch
// (ssd_forward_noalloc): every argument is validated before the first HIP call.
ssd_status forward_common(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* x, const void* dt,
                          const float* A, const void* B, const void* C, const float* D, const float* h0, void* y,
                          float* final_state, void* workspace, size_t workspace_bytes, bool use_static,
                          void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kForward, &s));
        Sizes z = sizes(s);
        FwdLayout f = fwd_layout(s);
        ssd::DtFront dfe;
        Span sbias;
        SSD_TRY(front_end(fe, s.H, &dfe, &sbias));
        Span sx{x, z.x, "x"}, sdt{dt, z.dt, "dt"}, sA{A, z.A, "A"}, sB{B, z.bc, "B"}, sC{C, z.bc, "C"},
            sD{D, D ? z.A : 0, "D"}, sh0{h0, h0 ? z.hstate : 0, "h0"}, sy{y, z.x, "y"},
            sfin{final_state, z.hstate, "final_state"}, sws{workspace, f.total, "workspace"};
        for (const Span& p : {sx, sdt, sA, sB, sC, sy, sfin}) SSD_TRY(need_ptr(p));
        SSD_TRY(need_align16({sx, sB, sC, sy, sh0, sfin}));
        if (use_static && f.total > ssd::kStaticScratchBytes)
            return fail(SSD_ERR_WORKSPACE, "ssd_forward_noalloc: this shape needs %zu bytes of scratch, above the "
                        "%zu-byte static scratch (use ssd_forward with a workspace)", f.total, ssd::kStaticScratchBytes);
        if (!use_static && s.b > 0 && s.L > 0) {
            if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", f.total);
            if (workspace_bytes < f.total)
                return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, f.total);
            if (reinterpret_cast<uintptr_t>(workspace) % 256)
                return fail(SSD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        }
        Span ins[] = {sx, sdt, sA, sB, sC, sD, sh0, sbias};
        SSD_TRY(no_alias(sy, ins, 8));
        SSD_TRY(no_alias(sfin, ins, 8));
        Span o1[] = {sy};
        SSD_TRY(no_alias(sfin, o1, 1));
        if (!use_static && s.b > 0 && s.L > 0) {
            Span all[] = {sx, sdt, sA, sB, sC, sD, sh0, sy, sfin, sbias};
            SSD_TRY(no_alias(sws, all, 10));
        }
        hipStream_t st = (hipStream_t)stream;
        if (s.b == 0) return ok();
        if (use_static && s.L > 0) {  // validation is complete: the first HIP call of this entry point
            hipError_t e = ssd::static_scratch(&workspace);
            if (e != hipSuccess) return hip_fail(e, "ssd_forward_noalloc (static scratch address)");
        }
        if (ssd::fast_chunk_supported(s)) {
            if (s.L == 0) {  // no tokens: the final state is h0 (or zero)
                hipError_t e = ssd::launch_state_passing(s, nullptr, nullptr, h0, final_state, st);
                return e == hipSuccess ? ok() : hip_fail(e, "ssd_forward/state_passing");
            }
            hipError_t e = ssd::launch_forward_fast(s, dfe, x, dt, A, B, C, D, h0, y, final_state, workspace, st);
            return e == hipSuccess ? ok() : hip_fail(e, "ssd_forward (fast path)");
        }
        char* ws = static_cast<char*>(workspace);
        float* dt_t = reinterpret_cast<float*>(ws + f.dt_t);
        float* cs = reinterpret_cast<float*>(ws + f.cs);
        float* states = reinterpret_cast<float*>(ws + f.states);
        hipError_t e;
        if (s.nC > 0) {
            e = ssd::launch_chunk_cumsum(s, dfe, dt, A, dt_t, cs, st);
            if (e != hipSuccess) return hip_fail(e, "ssd_forward/cumsum");
            e = ssd::launch_chunk_state(s, x, B, dt_t, cs, states, st);
            if (e != hipSuccess) return hip_fail(e, "ssd_forward/chunk_state");
        }
        e = ssd::launch_state_passing(s, states, cs, h0, final_state, st);
        if (e != hipSuccess) return hip_fail(e, "ssd_forward/state_passing");
        if (s.nC > 0) {
            e = ssd::launch_chunk_scan(s, x, B, C, dt_t, cs, states, D, y, st);
            if (e != hipSuccess) return hip_fail(e, "ssd_forward/chunk_scan");
        }
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

}  // namespace

extern "C" {

ssd_status ssd_forward_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* x, const void* dt,
                          const float* A, const void* B, const void* C, const float* D, const float* h0, void* y,
                          float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_common(dims, fe, x, dt, A, B, C, D, h0, y, final_state, workspace, workspace_bytes, false, stream);
}

ssd_status ssd_forward_noalloc(const ssd_dims* dims, const void* x, const void* dt, const float* A, const void* B,
                               const void* C, const float* D, const float* h0, void* y, float* final_state,
                               void* stream) {
    return forward_common(dims, nullptr, x, dt, A, B, C, D, h0, y, final_state, nullptr, ssd::kStaticScratchBytes,
                          true, stream);
}

ssd_status ssd_forward(const ssd_dims* dims, const void* x, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, const float* h0, void* y, float* final_state,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return ssd_forward_ex(dims, nullptr, x, dt, A, B, C, D, h0, y, final_state, workspace, workspace_bytes, stream);
}

ssd_status ssd_step_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, float* state, const void* x, const void* dt,
                       const float* A, const void* B, const void* C, const float* D, void* y, void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kStep, &s));
        ssd::DtFront dfe;
        Span sbias;
        SSD_TRY(front_end(fe, s.H, &dfe, &sbias));
        const size_t e = esz(s);
        Span sst{state, (size_t)(s.b * s.H * s.P * s.N) * 4, "state"}, sx{x, (size_t)(s.b * s.H * s.P) * e, "x"},
            sdt{dt, (size_t)(s.b * s.H) * e, "dt"}, sA{A, (size_t)s.H * 4, "A"}, sB{B, (size_t)(s.b * s.G * s.N) * e, "B"},
            sC{C, (size_t)(s.b * s.G * s.N) * e, "C"}, sD{D, D ? (size_t)s.H * 4 : 0, "D"},
            sy{y, (size_t)(s.b * s.H * s.P) * e, "y"};
        for (const Span& p : {sst, sx, sdt, sA, sB, sC, sy}) SSD_TRY(need_ptr(p));
        SSD_TRY(need_align16({sst, sx, sB, sC, sy}));
        Span ins[] = {sx, sdt, sA, sB, sC, sD, sbias};
        SSD_TRY(no_alias(sst, ins, 7));
        Span ins2[] = {sx, sdt, sA, sB, sC, sD, sst, sbias};
        SSD_TRY(no_alias(sy, ins2, 8));
        hipError_t he = ssd::launch_step(s, dfe, state, x, dt, A, B, C, D, y, (hipStream_t)stream);
        if (he != hipSuccess) return hip_fail(he, "ssd_step");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

ssd_status ssd_step(const ssd_dims* dims, float* state, const void* x, const void* dt, const float* A,
                    const void* B, const void* C, const float* D, void* y, void* stream) {
    return ssd_step_ex(dims, nullptr, state, x, dt, A, B, C, D, y, stream);
}

ssd_status ssd_step_multi_ex(const ssd_dims* dims, const ssd_dt_frontend* fe, float* state, const void* x,
                             const void* dt, const float* A, const void* B, const void* C, const float* D, void* y,
                             void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_dims(dims, Need::kStepMulti, &s));
        ssd::DtFront dfe;
        Span sbias;
        SSD_TRY(front_end(fe, s.H, &dfe, &sbias));
        const size_t e = esz(s);
        const size_t K = (size_t)s.L;
        Span sst{state, (size_t)(s.b * s.H * s.P * s.N) * 4, "state"},
            sx{x, (size_t)(s.b * s.H * s.P) * K * e, "x"}, sdt{dt, (size_t)(s.b * s.H) * K * e, "dt"},
            sA{A, (size_t)s.H * 4, "A"}, sB{B, (size_t)(s.b * s.G * s.N) * K * e, "B"},
            sC{C, (size_t)(s.b * s.G * s.N) * K * e, "C"}, sD{D, D ? (size_t)s.H * 4 : 0, "D"},
            sy{y, (size_t)(s.b * s.H * s.P) * K * e, "y"};
        for (const Span& p : {sst, sx, sdt, sA, sB, sC, sy}) SSD_TRY(need_ptr(p));
        Span ins[] = {sx, sdt, sA, sB, sC, sD, sbias};
        SSD_TRY(no_alias(sst, ins, 7));
        Span ins2[] = {sx, sdt, sA, sB, sC, sD, sst, sbias};
        SSD_TRY(no_alias(sy, ins2, 8));
        SSD_TRY(need_align16({sst, sx, sB, sC, sy}));
        hipError_t he = ssd::launch_step_multi(s, dfe, state, x, dt, A, B, C, D, y, (hipStream_t)stream);
        if (he != hipSuccess) return hip_fail(he, "ssd_step_multi");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

ssd_status ssd_step_multi(const ssd_dims* dims, float* state, const void* x, const void* dt, const float* A,
                          const void* B, const void* C, const float* D, void* y, void* stream) {
    return ssd_step_multi_ex(dims, nullptr, state, x, dt, A, B, C, D, y, stream);
}

// ---------------------------------------------------------------------------
// backward pass
// ---------------------------------------------------------------------------
// The backward runs three scans: the adjoint (headdim P, dstate N) and two transposed ones (headdim N,
// dstate P, one group per head).  Whatever path runs them (the fp32 generic kernels, or for bf16 inputs
// with headdim 64 the chunk-local decay gradient and the bf16 chunk kernels), the chunk must suit the fp32
// generic tiles, which every shape can fall back to.
static bool backward_chunk_ok(const ssd::Shape& s, int64_t Q) {
    if (Q % 16 || Q < 16 || Q > 512) return false;
    ssd::Shape a = s, t = s;
    a.io = t.io = 0;
    a.Q = t.Q = Q;
    t.P = s.N;
    t.N = s.P;
    t.G = s.H;
    for (const ssd::Shape& x : {a, t})
        if (ssd::chunk_scan_lds_bytes(x) > 160 * 1024 || ssd::chunk_state_lds_bytes(x) > 160 * 1024) return false;
    return true;
}

static ssd_status check_backward(const ssd_dims* d, ssd::Shape* out) {
    if (!d) return fail(SSD_ERR_NULL, "dims is NULL");
    ssd_dims d2 = *d;
    if (d2.chunk == 0) d2.chunk = 64;  // validated below with the backward's own choice
    ssd::Shape s;
    SSD_TRY(check_dims(&d2, Need::kStaged, &s));
    if (s.N > 256)
        return fail(SSD_ERR_UNSUPPORTED, "dstate %lld: the backward needs dstate <= 256", (long long)s.N);
    if ((2 * s.G * s.N + s.H) * 4 > 64 * 1024)
        return fail(SSD_ERR_UNSUPPORTED, "the backward stages B and C of all groups of a token in 64 KiB of LDS");
    int64_t Q = d->chunk;
    if (Q == 0) {
        for (int64_t cand : {128, 256, 64})  // 128: fewest in-chunk flops per chunk state (measured)
            if (backward_chunk_ok(s, cand)) {
                Q = cand;
                break;
            }
        if (Q == 0) return fail(SSD_ERR_UNSUPPORTED, "no chunk size fits the backward's tiles in LDS");
    } else if (!backward_chunk_ok(s, Q)) {
        return fail(SSD_ERR_UNSUPPORTED, "chunk %lld: the backward needs a multiple of 16 up to 512 whose fp32 "
                    "tiles fit the 160 KiB LDS", (long long)Q);
    }
    s.Q = Q;
    s.nC = (s.L + Q - 1) / Q;
    if (s.b * s.L * s.H > kMaxGrid * 4 || s.b * s.nC * s.H * s.N > kMaxGrid)
        return fail(SSD_ERR_UNSUPPORTED, "problem too large for one launch grid");
    *out = s;
    return SSD_OK;
}

size_t ssd_backward_workspace_bytes(const ssd_dims* dims) {
    try {
        ssd::Shape s;
        if (check_backward(dims, &s) != SSD_OK) return 0;
        return ssd::backward_layout(s).total;
    } catch (...) {
        return 0;
    }
}

ssd_status ssd_backward(const ssd_dims* dims, const void* x, const void* dt, const float* A, const void* B,
                        const void* C, const float* D, const float* h0, const void* dy, const float* dfinal,
                        void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, float* dh0, void* workspace,
                        size_t workspace_bytes, void* stream) {
    try {
        ssd::Shape s;
        SSD_TRY(check_backward(dims, &s));
        Sizes z = sizes(s);
        const size_t need = ssd::backward_layout(s).total;
        Span sx{x, z.x, "x"}, sdt{dt, z.dt, "dt"}, sA{A, z.A, "A"}, sB{B, z.bc, "B"}, sC{C, z.bc, "C"},
            sD{D, D ? z.A : 0, "D"}, sh0{h0, h0 ? z.hstate : 0, "h0"}, sdy{dy, z.x, "dy"},
            sdf{dfinal, dfinal ? z.hstate : 0, "dfinal"}, sdx{dx, z.x, "dx"}, sddt{ddt, z.dt, "ddt"},
            sdA{dA, z.A, "dA"}, sdB{dB, z.bc, "dB"}, sdC{dC, z.bc, "dC"}, sdD{dD, dD ? z.A : 0, "dD"},
            sdh0{dh0, dh0 ? z.hstate : 0, "dh0"}, sws{workspace, need, "workspace"};
        for (const Span& p : {sx, sdt, sA, sB, sC, sdy, sdx, sddt, sdA, sdB, sdC}) SSD_TRY(need_ptr(p));
        SSD_TRY(need_align16({sx, sB, sC, sdy, sdx, sdB, sdC, sh0, sdf, sdh0}));
        if (s.b > 0 && s.L > 0) {
            if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
            if (workspace_bytes < need)
                return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, need);
            if (reinterpret_cast<uintptr_t>(workspace) % 256)
                return fail(SSD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        }
        Span ins[] = {sx, sdt, sA, sB, sC, sD, sh0, sdy, sdf};
        Span outs[] = {sdx, sddt, sdA, sdB, sdC, sdD, sdh0};
        for (const Span& o : outs) {
            SSD_TRY(no_alias(o, ins, 9));
            for (const Span& o2 : outs)
                if (&o2 != &o && overlap(o, o2)) return fail(SSD_ERR_ALIAS, "%s overlaps %s", o.name, o2.name);
        }
        if (s.b > 0 && s.L > 0) {
            Span all[] = {sx, sdt, sA, sB, sC, sD, sh0, sdy, sdf, sdx, sddt, sdA, sdB, sdC, sdD, sdh0};
            SSD_TRY(no_alias(sws, all, 16));
        }
        hipError_t e = ssd::launch_backward(s, x, dt, A, B, C, D, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dh0,
                                            workspace, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "ssd_backward");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

// ---------------------------------------------------------------------------
// Mamba-1 selective scan
// ---------------------------------------------------------------------------
static ssd_status check_selective(const ssd_dims* d, ssd::SelectiveLayout* lay) {
    if (!d) return fail(SSD_ERR_NULL, "dims is NULL");
    if (d->io != SSD_F32 && d->io != SSD_BF16) return fail(SSD_ERR_DTYPE, "io dtype %d is not SSD_F32/SSD_BF16", d->io);
    if (d->reserved != 0) return fail(SSD_ERR_SHAPE, "dims.reserved must be 0");
    if (d->batch < 0 || d->seqlen < 0) return fail(SSD_ERR_SHAPE, "batch and seqlen must be >= 0");
    if (d->nheads <= 0 || d->dstate <= 0 || d->ngroups <= 0)
        return fail(SSD_ERR_SHAPE, "nheads (channels), dstate and ngroups must be > 0");
    if (d->headdim != 1) return fail(SSD_ERR_SHAPE, "the selective scan needs headdim == 1 (got %lld)",
                                     (long long)d->headdim);
    if (d->nheads % d->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "channels (%lld) is not a multiple of ngroups (%lld)", (long long)d->nheads,
                    (long long)d->ngroups);
    if (d->chunk < 0) return fail(SSD_ERR_SHAPE, "chunk must be >= 0");
    if (d->chunk % 64) return fail(SSD_ERR_UNSUPPORTED, "segment length %lld: need 0 or a multiple of 64",
                                   (long long)d->chunk);
    if (!ssd::selective_supported(d->nheads, d->dstate, d->ngroups))
        return fail(SSD_ERR_UNSUPPORTED, "dstate %lld, channels per group %lld: need dstate in {16, 32, 48, 64} and "
                    "a multiple of 16 channels per group", (long long)d->dstate,
                    (long long)(d->nheads / d->ngroups));
    if (d->batch > 65535 || d->batch * (d->nheads / 16) * ((d->seqlen + 63) / 64 + 1) > kMaxGrid)
        return fail(SSD_ERR_UNSUPPORTED, "problem too large for one launch grid");
    *lay = ssd::selective_layout(d->batch, d->seqlen, d->nheads, d->dstate, d->ngroups, d->chunk);
    return SSD_OK;
}

size_t ssd_selective_scan_workspace_bytes(const ssd_dims* dims) {
    try {
        ssd::SelectiveLayout f;
        if (check_selective(dims, &f) != SSD_OK) return 0;
        return f.total;
    } catch (...) {
        return 0;
    }
}

ssd_status ssd_selective_scan(const ssd_dims* dims, const ssd_dt_frontend* fe, const void* x, const void* delta,
                              const float* A, const void* B, const void* C, const float* D, const float* h0,
                              void* y, float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        ssd::SelectiveLayout f;
        SSD_TRY(check_selective(dims, &f));
        const int64_t b = dims->batch, L = dims->seqlen, Dc = dims->nheads, N = dims->dstate, G = dims->ngroups;
        ssd::DtFront dfe;
        Span sbias;
        SSD_TRY(front_end(fe, Dc, &dfe, &sbias));
        const size_t e = dims->io == SSD_BF16 ? 2 : 4;
        Span sx{x, (size_t)(b * L * Dc) * e, "x"}, sdl{delta, (size_t)(b * L * Dc) * e, "delta"},
            sA{A, (size_t)(Dc * N) * 4, "A"}, sB{B, (size_t)(b * L * G * N) * e, "B"},
            sC{C, (size_t)(b * L * G * N) * e, "C"}, sD{D, D ? (size_t)Dc * 4 : 0, "D"},
            sh0{h0, h0 ? (size_t)(b * Dc * N) * 4 : 0, "h0"}, sy{y, (size_t)(b * L * Dc) * e, "y"},
            sfin{final_state, (size_t)(b * Dc * N) * 4, "final_state"}, sws{workspace, f.total, "workspace"};
        for (const Span& p : {sx, sdl, sA, sB, sC, sy, sfin}) SSD_TRY(need_ptr(p));
        if (b > 0 && L > 0 && f.total > 0) {
            if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", f.total);
            if (workspace_bytes < f.total)
                return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, f.total);
            if (reinterpret_cast<uintptr_t>(workspace) % 256)
                return fail(SSD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        }
        Span ins[] = {sx, sdl, sA, sB, sC, sD, sh0, sbias};
        SSD_TRY(no_alias(sy, ins, 8));
        SSD_TRY(no_alias(sfin, ins, 8));
        Span o1[] = {sy};
        SSD_TRY(no_alias(sfin, o1, 1));
        if (b > 0 && L > 0 && f.total > 0) {
            Span all[] = {sx, sdl, sA, sB, sC, sD, sh0, sy, sfin, sbias};
            SSD_TRY(no_alias(sws, all, 10));
        }
        for (const Span& p : {sx, sdl, sB, sC, sy})
            if (reinterpret_cast<uintptr_t>(p.p) % 16)
                return fail(SSD_ERR_UNSUPPORTED, "%s must be 16-byte aligned", p.name);
        hipError_t he = ssd::launch_selective_scan(b, L, Dc, N, G, dims->io == SSD_BF16 ? 1 : 0, dfe, x, delta, A,
                                                   B, C, D, h0, y, final_state, dims->chunk, workspace,
                                                   (hipStream_t)stream);
        if (he != hipSuccess) return hip_fail(he, "ssd_selective_scan");
        return ok();
    } catch (...) {
        return fail(SSD_ERR_HIP, "internal error");
    }
}

}  // extern "C"
