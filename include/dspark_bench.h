/*
 * dspark_bench.h — C ABI of libdspark_bench.so, the benchmark's measurement
 * library.  It is not part of the verification library (libdspark.so) and the
 * pages define nothing in it: it holds the yardstick with which the streaming
 * pass's bandwidth is compared.
 */
#ifndef DSPARK_BENCH_H
#define DSPARK_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dspark_bench_read_probe — plain contiguous read of a device buffer.
 *
 * Reads `bytes` bytes at `x` (device memory, 16-byte aligned) once, in the
 * launch shape of the streaming pass (one 512-thread workgroup per compute
 * unit, 8 KB tiles of coalesced 16-byte loads per wave), and computes nothing
 * from them that reaches memory: `sink` (one uint32_t of device memory) is
 * written only if a checksum of the data equals a fixed constant.  Work goes
 * onto `stream` (a hipStream_t as void*); nothing is allocated.
 * Returns 0 on success, 1 for a NULL x or sink, 7 for bytes zero or not a
 * multiple of 16 or x misaligned, 6 if the launch failed (the status values
 * of dspark.h).
 */
__attribute__((visibility("default"))) int dspark_bench_read_probe(const void* x, size_t bytes,
                                                                   uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_BENCH_H */
