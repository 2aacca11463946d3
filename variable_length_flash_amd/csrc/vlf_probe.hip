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
#include <type_traits>

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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Byte offset of a lane's first operand in LDS at step i (the step's operands lie 1 KiB apart).
__device__ __forceinline__ int base_of(int i, int lane) { return (i & 3) * 1024 + lane * 16; }

// One role's loop (see vlf_probe_overlap). Every result feeds the returned checksum, so nothing
// is dropped; the vector roles carry eight independent chains.
template <int ROLE>
__device__ __forceinline__ float role_loop(int iters, int lane, const uint8_t *lds) {
    u32x4 a = {0x3c003c00u + lane, 0x3b003b00u, 0x3c00u, 0x3a00u}, b = a ^ 0x00010001u;
    u32x4 a2 = a ^ 0x00020002u, b2 = b ^ 0x00040004u;
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, d0 = {}, d1 = {}, d2 = {}, d3 = {};
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = -0.01f * (lane + k + 1);
    float l = 0.f;
    uint32_t acc = 0;
    u32x4 ops[16];
    if constexpr (ROLE == 7 || ROLE == 8 || ROLE == 10) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            ops[k] = *(const u32x4 *)(lds + ((base_of(0, lane) + k * 1024) & 16383));
    }
    for (int i = 0; i < iters; ++i) {
        if constexpr (ROLE == 1 || ROLE == 5) {
            c0 = mma(a, b, c0); c1 = mma(b, a, c1); c2 = mma(a2, b2, c2); c3 = mma(b2, a2, c3);
            c0 = mma(a2, b, c0); c1 = mma(b2, a, c1); c2 = mma(a, b2, c2); c3 = mma(b, a2, c3);
        }
        if constexpr (ROLE == 5) {
            c0 = mma(a, b2, c0); c1 = mma(b, a2, c1); c2 = mma(a2, b, c2); c3 = mma(b2, a, c3);
            c0 = mma(a2, b2, c0); c1 = mma(b2, a2, c1); c2 = mma(a, b, c2); c3 = mma(b, a, c3);
        }
        if constexpr (ROLE == 6) {
            // 16 products whose A operands come from LDS, one 16-byte read each
            const int base = base_of(i, lane);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const u32x4 op = *(const u32x4 *)(lds + ((base + k * 1024) & 16383));
                f32x16 &c = (k & 3) == 0 ? c0 : (k & 3) == 1 ? c1 : (k & 3) == 2 ? c2 : c3;
                c = mma(op, b, c);
            }
        }
        if constexpr (ROLE == 7) {
            // the same 16 LDS operands, all read one step ahead of their products
            const int nbase = ((i + 1) & 3) * 1024 + lane * 16;
            u32x4 nxt[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                nxt[k] = *(const u32x4 *)(lds + ((nbase + k * 1024) & 16383));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                f32x16 &c = (k & 3) == 0 ? c0 : (k & 3) == 1 ? c1 : (k & 3) == 2 ? c2 : c3;
                c = mma(ops[k], b, c);
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                ops[k] = nxt[k];
        }
        if constexpr (ROLE == 8) {
            // the same 16 LDS operands, each read four products ahead of its own
            const int nbase = ((i + 1) & 3) * 1024 + lane * 16;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                f32x16 &c = (k & 3) == 0 ? c0 : (k & 3) == 1 ? c1 : (k & 3) == 2 ? c2 : c3;
                c = mma(ops[k & 3], b, c);
                const int off = k < 12 ? base_of(i, lane) + (k + 4) * 1024 : nbase + (k - 12) * 1024;
                ops[k & 3] = *(const u32x4 *)(lds + (off & 16383));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (ROLE == 9) {
            // the 16 LDS reads alone, all issued before the first is used
            u32x4 r[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                r[k] = *(const u32x4 *)(lds + ((base_of(i, lane) + k * 1024) & 16383));
#pragma unroll
            for (int k = 0; k < 16; ++k)
                acc ^= r[k][0] ^ r[k][1] ^ r[k][2] ^ r[k][3];
        }
        if constexpr (ROLE == 10) {
            // a 64-row step: every operand read (four products ahead) feeds two products, one
            // per 32-row block, and the softmax covers 64 scores per lane
            const int nbase = ((i + 1) & 3) * 1024 + lane * 16;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                f32x16 &c = (k & 3) == 0 ? c0 : (k & 3) == 1 ? c1 : (k & 3) == 2 ? c2 : c3;
                f32x16 &d = (k & 3) == 0 ? d0 : (k & 3) == 1 ? d1 : (k & 3) == 2 ? d2 : d3;
                c = mma(ops[k & 3], b, c);
                d = mma(ops[k & 3], b2, d);
                const int off = k < 12 ? base_of(i, lane) + (k + 4) * 1024 : nbase + (k - 12) * 1024;
                ops[k & 3] = *(const u32x4 *)(lds + (off & 16383));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (ROLE == 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = __builtin_amdgcn_exp2f(v[k]);
        }
        if constexpr (ROLE == 3) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = __builtin_fmaf(v[k], 0.999f, -0.001f);
        }
        if constexpr (ROLE >= 4 && ROLE != 9) {
            // the softmax of 32 scores per lane (64 for the 64-row step): fma, exp2, row-sum
            // add, bf16 pair conversion
#pragma unroll
            for (int r = 0; r < (ROLE == 10 ? 8 : 4); ++r) {
                float e[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[k], 1.4427f, -0.5f));
                    l += e[k];
                }
                asm volatile("" : "+v"(l));
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    acc ^= pack2(e[2 * k], e[2 * k + 1]);
                v[r & 7] += __uint_as_float(acc & 0x3f800000u) * 1e-9f;
            }
        }
    }
    float s = l + __uint_as_float(acc);
#pragma unroll
    for (int k = 0; k < 16; ++k)
        s += c0[k] + c1[k] + c2[k] + c3[k] + d0[k] + d1[k] + d2[k] + d3[k];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        s += v[k];
    if constexpr (ROLE == 7 || ROLE == 8 || ROLE == 10) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            s += __uint_as_float(ops[k][0] & 0x3fffffffu);
    }
    return s;
}

template <int ROLE>
__device__ __forceinline__ float run_role(int iters, int lane, const uint8_t *lds) {
    return role_loop<ROLE>(iters, lane, lds);
}

__device__ __forceinline__ float dispatch_role(int role, int iters, int lane, const uint8_t *lds) {
    switch (role) {
    case 1: return run_role<1>(iters, lane, lds);
    case 2: return run_role<2>(iters, lane, lds);
    case 3: return run_role<3>(iters, lane, lds);
    case 4: return run_role<4>(iters, lane, lds);
    case 5: return run_role<5>(iters, lane, lds);
    case 6: return run_role<6>(iters, lane, lds);
    case 7: return run_role<7>(iters, lane, lds);
    case 8: return run_role<8>(iters, lane, lds);
    case 9: return run_role<9>(iters, lane, lds);
    case 10: return run_role<10>(iters, lane, lds);
    default: return 0.f;
    }
}

__global__ void __launch_bounds__(512) overlap_probe(int32_t lo_role, int32_t hi_role,
                                                     int32_t iters, float *sink,
                                                     uint64_t *record) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[16384];
    for (int i = threadIdx.x; i < 4096; i += 512)
        ((uint32_t *)lds)[i] = 0x3c003c00u ^ (i & 0x00ff00ffu);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const float s = dispatch_role(wave < 4 ? lo_role : hi_role, iters, lane, lds);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    sink[blockIdx.x * 512 + threadIdx.x] = s;
    uint64_t *rec = record + 4 * (uint64_t)blockIdx.x;
    if (threadIdx.x == 256)
        rec[3] = t1 - t0;  // wave 4's own loop
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t t2 = __builtin_amdgcn_s_memtime(), r2 = __builtin_amdgcn_s_memrealtime();
        rec[0] = t2 - t0;  // both halves, to the last wave's end
        rec[1] = r2 - r0;
        rec[2] = t1 - t0;  // wave 0's own loop
    }
}

// ---- phase schedules of the forward's wave step -------------------------------------------
// One workgroup per CU whose waves rotate through the roles of a 32-row, 64-key step with the
// forward's dataflow: a product phase (the output product of tile t from the V image in LDS and
// the packed probabilities, and the scores of tile t+1 from the K image and the query operand,
// four independent accumulator chains), and softmax phases (exp2 of score * log2 e minus a
// reference, the row sum, pair conversions to bf16) that split the step's 32 scores per lane.
// Groups of four waves (one per SIMD) take the roles in turn, a barrier per phase, so that each
// SIMD holds one product wave and the rest softmax waves: NG = 3 (each softmax wave half a
// step) or NG = 4 (a third). DROP = 1 leaves the softmax phases empty, DROP = 2 the products,
// to show what each side costs alone. The compiler may not move work across a phase barrier
// (sched_barrier), or it would fold the softmax parts into one phase.

constexpr float PROBE_LOG2E = 1.4426950408889634f;

__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int NG, int DROP>
__global__ void __launch_bounds__(256 * NG) __attribute__((amdgpu_waves_per_eu(NG)))
schedule_probe(int32_t steps, float *sink, uint64_t *record) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * 16384];
    for (int i = threadIdx.x; i < 16384; i += 256 * NG)
        ((uint32_t *)ring)[i] = 0x3c003c00u ^ ((i * 2654435761u) & 0x007f007fu);
    const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >> 2;
    int cof[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
        cof[kc] = n * 128 + 16 * ((2 * kc + g) ^ ((n >> 1) & 7));
    u32x4 qop[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        qop[c] = u32x4{0x3c003c00u + lane, 0x3b003b00u, 0x3c00u + c, 0x3a00u};
    f32x16 o0 = {}, o1 = {}, s0 = {}, s1 = {};
    u32x4 pk[4] = {};
    float l = 0.f;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    // softmax of scores [a, b) of the lane's 32 (s0 then s1) and the packs of their pairs
    auto part = [&](int a, int b) __attribute__((always_inline)) {
        if (DROP == 1)
            return;
        float rs = 0.f;
#pragma unroll
        for (int i = a; i < b; ++i) {
            if (i < 16) {
                s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], PROBE_LOG2E, -0.75f));
                rs += s0[i];
            } else {
                s1[i - 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i - 16], PROBE_LOG2E, -0.75f));
                rs += s1[i - 16];
            }
        }
#pragma unroll
        for (int i = a; i < b; i += 2) {
            const float x0 = i < 16 ? s0[i] : s1[i - 16];
            const float x1 = i + 1 < 16 ? s0[i + 1] : s1[i - 15];
            pk[i / 8][(i % 8) / 2] = pack2(x0, x1);
        }
        l += rs;
        asm volatile("" : "+v"(l), "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]), "+v"(pk[3]));
    };
    auto product = [&](int cur) __attribute__((always_inline)) {
        if (DROP == 2) {
            s0[0] += 1.0f;
            s1[0] += 1.0f;
            o0[0] += __uint_as_float(pk[0][0] & 0x3f000000u);
            return;
        }
        __builtin_amdgcn_s_setprio(1);
        const uint8_t *kt = ring + ((cur + 1) & 3) * 16384, *vt = ring + cur * 16384 + 8192;
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            o0 = mma(*(const u32x4 *)(vt + cof[c]), pk[c], o0);
            s0 = mma(*(const u32x4 *)(kt + cof[c]), qop[c], s0);
            o1 = mma(*(const u32x4 *)(vt + 4096 + cof[c]), pk[c], o1);
            s1 = mma(*(const u32x4 *)(kt + 4096 + cof[c]), qop[c], s1);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // Group r runs its role sequence rotated by r phases; the roles of one step are the product
    // (role 0) and the softmax parts (roles 1 .. NG - 1). Four steps unrolled keep ring slots
    // constant.
    auto role = [&](int r, int u) __attribute__((always_inline)) {
        if (r == 0)
            product(u);
        else if (NG == 3)
            part(r == 1 ? 0 : 16, r == 1 ? 16 : 32);
        else
            part(r == 1 ? 0 : r == 2 ? 10 : 22, r == 1 ? 10 : r == 2 ? 22 : 32);
    };
    auto run = [&](auto shift) __attribute__((always_inline)) {
        constexpr int SH = decltype(shift)::value;
        for (int t = 0; t < steps; t += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int ph = 0; ph < NG; ++ph) {
                    role((ph + NG - SH) % NG, u);
                    phase_barrier();
                }
        }
    };
    if (grp == 0)
        run(std::integral_constant<int, 0>{});
    else if (grp == 1)
        run(std::integral_constant<int, 1>{});
    else if (grp == 2)
        run(std::integral_constant<int, 2>{});
    else if (NG == 4)
        run(std::integral_constant<int, 3>{});
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    float sum = l;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        sum += o0[k] + o1[k] + s0[k] + s1[k];  // (the scores too, so no product is dropped)
    sink[blockIdx.x * 1024 + threadIdx.x] = sum;
    if (threadIdx.x == 0)
        record[16 * blockIdx.x] = t1 - t0;
}

// The matrix unit's toll on the vector unit: waves 0-3 (one per SIMD) issue four independent
// v_mfma_f32_32x32x16_bf16 per iteration (MFMA = true) or nothing; waves 4-11 (two per SIMD)
// 16 v_fma_f32 (EXP = false) or v_exp_f32 per iteration on eight chains. Every wave records its
// own loop time.
template <bool MFMA, bool EXP>
__global__ void __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3)))
toll_probe(int32_t iters, float *sink, uint64_t *record) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    float s = 0.f;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    if (wv < 4) {
        if (MFMA) {
            u32x4 a = {0x3c003c00u + lane, 0x3b003b00u, 0x3c00u, 0x3a00u}, b = a ^ 0x00010001u;
            f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
            for (int i = 0; i < iters; ++i) {
                c0 = mma(a, b, c0);
                c1 = mma(b, a, c1);
                c2 = mma(a, a, c2);
                c3 = mma(b, b, c3);
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                s += c0[k] + c1[k] + c2[k] + c3[k];
        }
    } else {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = -0.01f * (lane + k + 1);
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = EXP ? __builtin_amdgcn_exp2f(v[k]) : __builtin_fmaf(v[k], 0.999f, -0.001f);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            s += v[k];
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    sink[blockIdx.x * 1024 + threadIdx.x] = s;
    if (lane == 0)
        record[blockIdx.x * 16 + wv] = t1 - t0;
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

int vlf_probe_overlap(int32_t lo_role, int32_t hi_role, int32_t iters, int32_t blocks,
                      float *sink_dev, uint64_t *record_dev, void *stream) {
    if (lo_role < 0 || lo_role > 10 || hi_role < 0 || hi_role > 10)
        return fail(-1, "roles %d, %d outside 0 .. 10", lo_role, hi_role);
    if (iters < 1 || iters > (1 << 24))
        return fail(-1, "iters = %d outside 1 .. 2^24", iters);
    if (blocks < 1 || blocks > (1 << 20))
        return fail(-1, "blocks = %d outside 1 .. 2^20", blocks);
    if (!sink_dev || ((uintptr_t)sink_dev & 3) != 0 || !record_dev ||
        ((uintptr_t)record_dev & 7) != 0)
        return fail(-1, "null or misaligned sink_dev / record_dev");
    void *args[] = {(void *)&lo_role, (void *)&hi_role, (void *)&iters, (void *)&sink_dev,
                    (void *)&record_dev};
    const hipError_t e = hipLaunchKernel((const void *)overlap_probe, dim3((unsigned)blocks),
                                         dim3(512), args, 0, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(-3, "probe launch failed: %s", hipGetErrorString(e));
    return 0;
}

int vlf_probe_schedule(int32_t kind, int32_t steps, int32_t blocks, float *sink_dev,
                       uint64_t *record_dev, void *stream) {
    if (kind < 0 || kind > 9)
        return fail(-1, "kind = %d outside 0 .. 9", kind);
    if (steps < 4 || steps > (1 << 22) || steps % 4 != 0)
        return fail(-1, "steps = %d: a multiple of 4 in 4 .. 2^22", steps);
    if (blocks < 1 || blocks > (1 << 20))
        return fail(-1, "blocks = %d outside 1 .. 2^20", blocks);
    if (!sink_dev || ((uintptr_t)sink_dev & 3) != 0 || !record_dev ||
        ((uintptr_t)record_dev & 7) != 0)
        return fail(-1, "null or misaligned sink_dev / record_dev");
    static const void *const fns[10] = {
        (const void *)schedule_probe<3, 0>, (const void *)schedule_probe<3, 1>,
        (const void *)schedule_probe<3, 2>, (const void *)schedule_probe<4, 0>,
        (const void *)schedule_probe<4, 1>, (const void *)schedule_probe<4, 2>,
        (const void *)toll_probe<false, false>, (const void *)toll_probe<true, false>,
        (const void *)toll_probe<false, true>, (const void *)toll_probe<true, true>};
    const unsigned threads = kind < 3 ? 768 : kind < 6 ? 1024 : 768;
    void *args[] = {(void *)&steps, (void *)&sink_dev, (void *)&record_dev};
    const hipError_t e = hipLaunchKernel(fns[kind], dim3((unsigned)blocks), dim3(threads), args,
                                         0, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(-3, "probe launch failed: %s", hipGetErrorString(e));
    return 0;
}

const char *vlf_probe_last_error(void) { return g_error.c_str(); }

}  // extern "C"
