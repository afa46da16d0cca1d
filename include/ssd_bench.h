/*
 * ssd_bench.h -- measurement helpers exported by libssd next to the calls of
 * ssd.h.  They compute nothing of the state-space model; they exist so that a
 * benchmark can time, in the same process and under the same conditions, the
 * access pattern a kernel of ssd.h is bound by.
 */
#ifndef SSD_BENCH_H
#define SSD_BENCH_H

#include <stddef.h>

#include "ssd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * In place, for i < n: buf[i] <- a * buf[i] + b (fp32), on `stream`.  Every
 * element is read once and written once: the byte pattern of ssd_step's
 * state update (2 x 4 bytes per state element) with none of its other work.
 * buf is a device pointer, 16-byte aligned, n a multiple of 4
 * (SSD_ERR_UNSUPPORTED otherwise; SSD_ERR_NULL for a NULL buf with n > 0).
 * Nothing is validated beyond that and nothing synchronises.
 */
ssd_status ssd_bench_rmw_stream(float* buf, size_t n, float a, float b, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_BENCH_H */
