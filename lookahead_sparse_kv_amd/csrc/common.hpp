// common.hpp -- shared device types and host helpers of the LSA HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

// ---------------------------------------------------------------- device types
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Matrix-core products used here (CDNA4 bf16 MFMA with 8 operands per lane).
// 16x16x32: lane l supplies A[l%16][8*(l/16) + j] and B[8*(l/16) + j][l%16];
//           it receives D[4*(l/16) + v][l%16], v = 0..3.
// 32x32x16: lane l supplies A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32];
//           it receives D[8*(v/4) + 4*(l/32) + v%4][l%32], v = 0..15.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

// max(x, 0) in one integer instruction: an fp32 value with its sign bit clear
// is a non-negative int32, one with it set (-0.0 included) a negative one, so
// max_i32(bits, 0) returns x for x >= +0.0 and +0.0 otherwise (a NaN keeps its
// bits).  fmaxf(x, 0.0f) costs two instructions on a matrix-core result, which
// the compiler first canonicalises.
__device__ __forceinline__ float relu_bits(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// Word 3 of a buffer resource for plain raw buffer loads on gfx950; a load
// past num_records (or through a range of 0) reads no memory.
constexpr int kBufferWord3 = 0x00020000;

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order); LDS and export counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations retire
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads, so copies of later data stay in flight across it;
// a wave that copies into LDS waits for its own copies with wait_vmcnt first.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
}

// ------------------------------------------------------------------ host side
// Thread-local detail string for lsa_last_error(); returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread-local error message.
void clear_error();
// LSA_OK if the current device is gfx950, else LSA_ERR_UNSUPPORTED/LSA_ERR_HIP
// (the answer is cached per device).  Also returns the CU count.
int check_device(int* num_cus);
// Converts a HIP launch status into LSA_OK / LSA_ERR_HIP.
int launch_status(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace lsa
