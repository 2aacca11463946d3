// libvlf_probe.so: a probe of the gfx950 matrix unit for the measurement harness (not part of
// the attention path). Each wave keeps four independent 32x32 accumulators and issues nothing
// but v_mfma_f32_32x32x16_bf16 in its loop, so with two waves per SIMD the matrix unit never
// waits on a dependence; the shader-clock and constant-clock tick counts around the loop give
// the clock the chip ran at while doing so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/vlf_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

thread_local std::string g_error;

int fail(int status, const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

__global__ void __launch_bounds__(256) mfma_probe(int32_t iters, uint64_t *record) {
    const int lane = (int)(threadIdx.x & 63);
    bf16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(1.0f + 0.001f * (lane + k));
        b[k] = (__bf16)(0.5f - 0.001f * (lane - k));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    __syncthreads();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c3, 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        sum += c0[k] + c1[k] + c2[k] + c3[k];
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        uint64_t *o = record + 4 * (uint64_t)blockIdx.x;
        o[0] = t1 - t0;
        o[1] = r1 - r0;
        o[2] = (uint64_t)__float_as_uint(sum);
        o[3] = r0;
    }
}

}  // namespace

extern "C" {

int vlf_probe_mfma(int32_t iters, int32_t blocks, uint64_t *record_dev, void *stream) {
    if (iters < 1 || iters > (1 << 24))
        return fail(-1, "iters = %d outside 1 .. 2^24", iters);
    if (blocks < 1 || blocks > (1 << 20))
        return fail(-1, "blocks = %d outside 1 .. 2^20", blocks);
    if (!record_dev || ((uintptr_t)record_dev & 7) != 0)
        return fail(-1, "record_dev %p is null or not 8-byte aligned", (void *)record_dev);
    void *args[] = {(void *)&iters, (void *)&record_dev};
    const hipError_t e = hipLaunchKernel((const void *)mfma_probe, dim3((unsigned)blocks),
                                         dim3(256), args, 0, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(-3, "probe launch failed: %s", hipGetErrorString(e));
    return 0;
}

const char *vlf_probe_last_error(void) { return g_error.c_str(); }

}  // extern "C"
