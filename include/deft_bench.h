/*
 * deft_bench.h - measurement aid shipped beside libdeft (libdeft_bench.so):
 * a plain streaming read of device memory, timed by the benchmark to give the
 * HBM bandwidth this device actually reaches, against which the attention
 * kernels' achieved bandwidth is also reported (the pages compare engines by
 * kernel latency and memory traffic: DeFT Guide, "Empirical Benchmark
 * Evaluation"; the calibration itself is not part of the method).
 *
 * Conventions as in deft.h: device pointers, hipStream_t passed as void*,
 * asynchronous on the stream, DEFT_OK (0) or a negative code.
 */
#ifndef DEFT_BENCH_H
#define DEFT_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` of device memory at `src` (16-byte aligned, bytes a multiple
 * of 16) once, with 16-byte vector loads in a grid-stride loop over a grid
 * that fills the device, and writes one float per work-group to `sink`
 * (device memory of at least deft_bench_stream_read_sink_floats() floats;
 * the sum of the data read, so the loads cannot be dropped).  Returns -1 for
 * NULL pointers or misaligned arguments, -4 if the launch fails.
 */
int deft_bench_stream_read(const void* src, size_t bytes, float* sink, void* stream);

/* Floats the sink of deft_bench_stream_read needs. */
size_t deft_bench_stream_read_sink_floats(void);

#ifdef __cplusplus
}
#endif

#endif /* DEFT_BENCH_H */
