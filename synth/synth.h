/*
 * synth.h -- seeded synthetic-input generator (test and benchmark infrastructure).
 *
 * The routed-expert FFN workloads are evaluated on trained checkpoints that are not
 * available here, so every weight, activation and logit is synthetic.  This module
 * turns (seed, stream, element index) into a value through a counter-based generator,
 * so the same element can be produced on the host (for the oracle) and on the GPU (for
 * the kernels under test) bit for bit, in any order and in any subset.  It holds none
 * of the layer's arithmetic: it only makes inputs.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11).  Counter = (index lo, index hi, stream lo, stream hi),
 * key = (seed lo, seed hi).
 *
 * Normal approximation: Irwin-Hall of four 22-bit uniforms from one Philox call,
 *   S = sum_k (r_k >> 10) - 2*(2^22 - 1)        (an exact integer, |S| < 2^23)
 *   value = (float)S * c,  c = (float)(sigma * sqrt(3) / 2^22)
 * which has mean 0 and variance sigma^2 (1 - 2^-44), bounded at 3.46 sigma.  The one
 * fp32 multiply is IEEE round-to-nearest-even on both sides.
 *
 * bf16: round-to-nearest-even of that fp32 value by integer bit operations.
 * MXFP4 (OCP Microscaling Formats v1.0, e2m1 elements with one e8m0 scale per 32
 * consecutive elements along a row): scale exponent floor(log2(amax)) - 2, elements
 * rounded to nearest-even on the e2m1 grid {0,0.5,1,1.5,2,3,4,6} and saturated at 6;
 * an all-zero block has scale byte 0 and codes 0; a zero element is code 0; the even
 * element sits in the low nibble.  Codes and scales are separate arrays.
 *
 * All functions return 0 on success and a negative value on a bad argument.
 * Host functions write host memory; device functions enqueue on the given HIP stream
 * (NULL = default stream) and write device memory.
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The fp32 multiplier c for a target standard deviation sigma. */
float synth_scale_for_sigma(double sigma);

/* Raw Philox4x32-10 block: out[4] for counter ctr[4], key key[2] (known-answer tests). */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Elements [first, first+n) of stream (seed, stream) as fp32 / bf16 bits. nthreads <= 0: all cores. */
int synth_normal_f32_host(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                          float scale, float* out, int nthreads);
int synth_normal_bf16_host(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                           float scale, uint16_t* out, int nthreads);
/* Rows [row0, row0+rows) of a row-major [*, cols] matrix quantised to MXFP4.
 * codes: rows*cols/2 bytes; scales: rows*cols/32 bytes.  cols % 32 == 0. */
int synth_mxfp4_host(uint64_t seed, uint64_t stream, uint64_t row0, uint64_t rows,
                     uint64_t cols, float scale, uint8_t* codes, uint8_t* scales, int nthreads);

int synth_normal_f32_device(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                            float scale, float* out, void* hip_stream);
int synth_normal_bf16_device(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                             float scale, uint16_t* out, void* hip_stream);
int synth_mxfp4_device(uint64_t seed, uint64_t stream, uint64_t row0, uint64_t rows,
                       uint64_t cols, float scale, uint8_t* codes, uint8_t* scales,
                       void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
