// abi_driver.cpp -- drives the host-side code of the C ABI (argument checks,
// workspace sizes, the chunk rule) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  api.cpp is compiled host-only with the
// sanitizers and linked ahead of libssd.so (see tests/test_sanitizers.py), so
// these calls run the instrumented copy.  Every pointer is a fake address that
// is never dereferenced: each call below must be rejected before any launch.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/ssd.h"

static int fails = 0;
static void expect(ssd_status got, ssd_status want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "FAILED: %s: status %d, expected %d (%s)\n", what, (int)got, (int)want,
                     ssd_last_error());
        ++fails;
    }
}
static void* P(uint64_t off) { return reinterpret_cast<void*>(0x100000000ull + off); }
static float* F(uint64_t off) { return static_cast<float*>(P(off)); }

static ssd_dims dims(int64_t b, int64_t L, int64_t H, int64_t Pd, int64_t N, int64_t G, int64_t Q, int io) {
    ssd_dims d;
    std::memset(&d, 0, sizeof(d));
    d.batch = b, d.seqlen = L, d.nheads = H, d.headdim = Pd, d.dstate = N, d.ngroups = G, d.chunk = Q, d.io = io;
    return d;
}

int main() {
    const uint64_t GB = 1ull << 30;
    ssd_dims d = dims(1, 512, 4, 64, 128, 1, 256, SSD_BF16);
    // status strings and version
    for (int s = 0; s < 9; ++s)
        if (!ssd_status_string((ssd_status)s)) ++fails;
    if (ssd_abi_version() != SSD_ABI_VERSION) ++fails;
    // forward: dims, pointers, workspace, alignment, aliasing
    expect(ssd_forward(nullptr, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB),
                       F(7 * GB), P(8 * GB), 1ull << 40, nullptr),
           SSD_ERR_NULL, "forward dims NULL");
    ssd_dims bad = d;
    bad.ngroups = 3;
    expect(ssd_forward(&bad, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB), F(7 * GB),
                       P(8 * GB), 1ull << 40, nullptr),
           SSD_ERR_SHAPE, "forward H % G");
    bad = d;
    bad.chunk = 100;
    expect(ssd_forward(&bad, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB), F(7 * GB),
                       P(8 * GB), 1ull << 40, nullptr),
           SSD_ERR_UNSUPPORTED, "forward chunk");
    const size_t need = ssd_forward_workspace_bytes(&d);
    if (need == 0) ++fails;
    expect(ssd_forward(&d, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB), F(7 * GB),
                       P(8 * GB), need - 1, nullptr),
           SSD_ERR_WORKSPACE, "forward workspace size");
    expect(ssd_forward(&d, P(8), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB), F(7 * GB),
                       P(8 * GB), need, nullptr),
           SSD_ERR_UNSUPPORTED, "forward x misaligned");
    expect(ssd_forward(&d, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(96), F(7 * GB),
                       P(8 * GB), need, nullptr),
           SSD_ERR_ALIAS, "forward y over x");
    // the allocation-free forward: same validation, and a shape above its static scratch is refused
    ssd_dims big = dims(1, 262144, 80, 64, 128, 1, 0, SSD_BF16);
    expect(ssd_forward_noalloc(&big, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB),
                               F(7 * GB), nullptr),
           SSD_ERR_WORKSPACE, "noalloc oversize");
    expect(ssd_forward_noalloc(&d, nullptr, P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB),
                               F(7 * GB), nullptr),
           SSD_ERR_NULL, "noalloc x NULL");
    // staged calls
    expect(ssd_chunk_state(&d, P(0), nullptr, F(2 * GB), F(3 * GB), F(4 * GB), nullptr), SSD_ERR_NULL,
           "chunk_state B NULL");
    expect(ssd_chunk_scan(&d, P(0), P(GB), P(2 * GB + 8), F(3 * GB), F(4 * GB), F(5 * GB), nullptr, P(6 * GB),
                          nullptr),
           SSD_ERR_UNSUPPORTED, "chunk_scan C misaligned");
    expect(ssd_state_passing(&d, F(0), F(GB), nullptr, F(128), nullptr), SSD_ERR_ALIAS, "state_passing alias");
    expect(ssd_chunk_cumsum(&d, P(0), F(GB), F(0), F(3 * GB), nullptr), SSD_ERR_ALIAS, "cumsum alias");
    // step and multi-step
    ssd_dims s1 = dims(64, 1, 80, 64, 128, 1, 0, SSD_BF16);
    expect(ssd_step(&s1, F(0), P(GB), P(2 * GB), F(3 * GB), P(4 * GB), P(5 * GB), nullptr, P(16), nullptr),
           SSD_ERR_ALIAS, "step y over state");
    expect(ssd_step(&s1, F(8), P(GB), P(2 * GB), F(3 * GB), P(4 * GB), P(5 * GB), nullptr, P(6 * GB), nullptr),
           SSD_ERR_UNSUPPORTED, "step state misaligned");
    ssd_dims s8 = dims(2, 8, 4, 64, 128, 1, 0, 9);
    expect(ssd_step_multi(&s8, F(0), P(GB), P(2 * GB), F(3 * GB), P(4 * GB), P(5 * GB), nullptr, P(6 * GB), nullptr),
           SSD_ERR_DTYPE, "step_multi dtype");
    // front-end validation
    ssd_dt_frontend fe;
    std::memset(&fe, 0, sizeof(fe));
    fe.clamp = 1;
    fe.dt_min = 1.0f;
    fe.dt_max = 0.5f;
    expect(ssd_forward_ex(&d, &fe, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(6 * GB),
                          F(7 * GB), P(8 * GB), need, nullptr),
           SSD_ERR_SHAPE, "front-end clamp order");
    // the chunk rule and the configuration query over a grid of shapes (host-only arithmetic)
    const int64_t Ls[] = {0, 1, 63, 64, 1000, 1024, 4096, 65536, 262144};
    const int64_t Ns[] = {16, 64, 128, 256, 512};
    for (int64_t L : Ls)
        for (int64_t N : Ns)
            for (int io = 0; io < 2; ++io) {
                ssd_dims q = dims(1, L, 80, 64, N, 1, 0, io);
                int chunk = -1, tp = -1, hpw = -1, cps = -1;
                ssd_status st = ssd_query_config(&q, &chunk, &tp, &hpw, &cps);
                if (st == SSD_OK && (chunk <= 0 || hpw <= 0)) ++fails;
                (void)ssd_forward_workspace_bytes(&q);
            }
    // backward and selective scan sizes / validation
    expect(ssd_backward(&bad, P(0), P(GB), F(2 * GB), P(3 * GB), P(4 * GB), nullptr, nullptr, P(5 * GB), nullptr,
                        P(6 * GB), P(7 * GB), F(8 * GB), P(9 * GB), P(10 * GB), nullptr, F(11 * GB), P(12 * GB),
                        1ull << 40, nullptr),
           SSD_ERR_UNSUPPORTED, "backward chunk");
    (void)ssd_backward_workspace_bytes(&d);
    ssd_dims sel = dims(1, 4096, 5120, 1, 16, 1, 0, SSD_BF16);
    (void)ssd_selective_scan_workspace_bytes(&sel);
    expect(ssd_selective_scan(&sel, nullptr, P(0), P(GB), F(2 * GB), P(3 * GB + 8), P(4 * GB), nullptr, nullptr,
                              P(5 * GB), F(6 * GB), P(7 * GB), 1ull << 40, nullptr),
           SSD_ERR_UNSUPPORTED, "selective B misaligned");
    if (fails) {
        std::fprintf(stderr, "%d check(s) failed\n", fails);
        return 1;
    }
    std::printf("abi driver: all checks passed\n");
    return 0;
}
