/*
 * mla_inputs.h -- device twin of the seeded synthetic-input generator
 * (libmla_inputs.so).  Not part of the MLA computation: it only writes
 * numbers, so that large pools and weights can be produced in device memory
 * with exactly the bits the host generator gives for the same (key, index).
 *
 * Element i of a stream with 64-bit key K is SplitMix64's output mix of
 * K + (i+1)*0x9E3779B97F4A7C15 (Steele, Lea & Flood, OOPSLA 2014).  The value
 * written is the centred sum of the word's four 16-bit fields (an integer in
 * [-131070, 131070]) times `scale` in one fp32 multiply; bf16 output rounds to
 * nearest even.
 */
#ifndef MLA_INPUTS_H_
#define MLA_INPUTS_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Writes elements start .. start+n-1 of stream `key` to dst[0 .. n-1].
 * dtype: 0 = fp32, 1 = bf16.  dst is a device pointer (n elements).
 * Returns 0, -1 for a NULL dst with n > 0 or n < 0, -3 for an unknown dtype,
 * -5 if the launch fails. */
int32_t mla_fill_normal(void* dst, int64_t n, int32_t dtype, uint64_t key, uint64_t start,
                        float scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_INPUTS_H_ */
