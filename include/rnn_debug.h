/*
 * rnn_debug.h - extra exports of the debug build of the layer engine
 * (librnn_timers.so, compiled with RNN_STEP_TIMERS; the normal librnn.so
 * does not have them).
 *
 * In that build thread 0 of every workgroup of a persistent recurrent kernel
 * writes the shader clock (s_memtime) at eight fixed points of every step,
 * the per-step latency evidence that the CUDA fragment page's persistent
 * kernel gives no means to observe (its only time structure is the wait on
 * the previous step's data). Points, forward and backward alike:
 *   0 step start, 1 step counters seen (wave 0), 2 contraction issued,
 *   3 partial sums written to LDS, 4 past the workgroup barrier,
 *   5 gate epilogue done (exchange stores issued), 6 step counter published,
 *   7 stores for later kernels issued.
 * Records cover blocks [0, wgs) (launch order) and steps [0, steps)
 * (processing order); each kernel launch overwrites what it reaches.
 */
#ifndef RNN_DEBUG_H_
#define RNN_DEBUG_H_

#ifdef __cplusplus
extern "C" {
#endif

/* Zeroes the per-workgroup calibration pairs: after the next launch, a
 * block whose pairs are still zero did no work (padded placements launch
 * blocks that return at once). RNN_ERR_DEVICE if the copy fails. */
int rnn_step_timers_reset(void);

/* Dimensions of the timer array: wgs x steps x phases 64-bit ticks. */
int rnn_step_timers_shape(int* wgs, int* steps, int* phases);

/* Copies the timers (wgs*steps*phases uint64, s_memtime ticks) and, per
 * workgroup, (s_memtime, s_memrealtime) at kernel start and at kernel end
 * (wgs*4 uint64; s_memrealtime counts at 100 MHz) to host memory, after the
 * caller has synchronised. RNN_ERR_INVALID_ARG for NULL, RNN_ERR_DEVICE if a
 * copy fails. */
int rnn_step_timers_read(unsigned long long* timers, unsigned long long* cal);

#ifdef __cplusplus
}
#endif
#endif /* RNN_DEBUG_H_ */
