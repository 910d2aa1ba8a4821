/*
 * mns_probe.h -- C ABI of libmns_probe.so, a measurement aid beside the optimizer-step
 * library (not part of the optimizer path; nothing in libmuon_ns.so uses it).
 *
 * The published dense float16 MFMA peak of the MI355X (2.5 PFLOP/s) assumes the 2.4 GHz
 * clock. Under sustained matrix load the part holds that clock only while the operands
 * barely toggle: with random operands its power limit brings the clock down, and with it
 * the rate any kernel can reach. This probe measures that ceiling on the running part: a
 * kernel made only of v_mfma_f32_32x32x16_f16 instructions (the ones the library's GEMMs
 * issue), with no memory traffic in its loop, on every compute unit.
 *
 * Rules (as in muon_ns.h): pointers marked (host) are host memory; launches are
 * asynchronous on `stream` (a hipStream_t; NULL = the null stream); arguments are checked
 * before anything is enqueued. Return values: 0 = OK, 4 = an argument is out of range,
 * 6 = a HIP call failed (the muon_ns.h status codes). The probe keeps one static device
 * array (its result sink, 4 MiB) and allocates nothing.
 */
#ifndef MNS_PROBE_H
#define MNS_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one launch of the MFMA-only kernel on the current device: 8 workgroups of 4
 * waves per compute unit, each wave `iters` (1 .. 1e6) times 8 MFMAs on 4 independent
 * accumulators, its operands rotating through 8 register fragments filled from a linear
 * congruential sequence of the thread index (float16 values in [-1, 1]), or all zero when
 * `zero_operands` is non-zero. (host) *flops_per_launch receives the launch's float16 FLOPs
 * (2 * 32 * 32 * 16 per MFMA). */
int mns_probe_mfma_launch(int iters, int zero_operands, void* stream, double* flops_per_launch);

/* Synchronously read back the sum of the absolute values of the first `n` (1 .. 65536)
 * per-thread results of the last launch into (host) *sum: zero for zero operands, finite and
 * proportional to `iters` otherwise. */
int mns_probe_mfma_checksum(int n, double* sum);

#ifdef __cplusplus
}
#endif

#endif /* MNS_PROBE_H */
