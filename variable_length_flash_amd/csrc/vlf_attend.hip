// The forward kernel of packed variable-length attention for gfx950 (MI355X), and its launcher.
//
// What is computed is the `attend` kernel of hanzo-kernel 0.2.42 src/packed.rs: one tile of
// `br` query rows of one head against every key tile its window reaches; queries and keys rotated
// by position within their sequence (half-split pairs m, m+32) in float32, the query also scaled,
// both rounded to the storage type; scores and the output product on the matrix units; the
// softmax online per row with masked keys weighing exactly zero; out = O / l rounded to the
// storage type and lse = m + ln l in float32.
//
// How it is laid out on CDNA4 (this file's own design):
//   * A workgroup is one (tile, head); each 64-lane wave owns 32 query rows (br = 32 * waves).
//   * Scores are computed transposed, S^T = K~ Q~^T, with v_mfma_f32_32x32x16_{bf16,f16}: the
//     32x32 accumulator gives lane l the column of query l % 32 and 16 of the key rows, so a row
//     max or row sum is a local reduction plus one exchange between lanes l and l ^ 32.
//   * The query operand (B of that product) is rotated, scaled and rounded in registers and
//     stays there for the whole key loop.
//   * Keys are rotated in registers and staged row-major in LDS (rows padded to 144 B so the
//     16-byte operand reads of 8 consecutive lanes fall on distinct banks).
//   * Values are staged transposed, V^T [dim][key] (rows padded to 136 B), so the output is
//     computed transposed too, O^T += V^T P^T: the probabilities leave the score accumulator
//     registers directly as the B operand (after rounding), with the key order inside each
//     16-key step permuted to match the accumulator layout; no LDS round trip for P. The O^T
//     accumulator again gives each lane one query, so the per-row rescale is a lane-local
//     multiply.
//   * exp is exp2 with log2(e) folded into one FMA per score.
//   * Masks are evaluated only on tiles that touch a sequence end or a window edge; waves with
//     no visible pair in a key tile skip it.
//   * The 1-D grid is remapped so that consecutive work items land on the same XCD (blocks are
//     dealt round-robin over the 8 XCDs): all tiles of one (sequence, head) share one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vlf.h"
#include "vlf_internal.h"

namespace vlf {
namespace {

constexpr int D = 64;      // head dimension
constexpr int BC = 64;     // keys per key tile
constexpr int KS = 72;     // LDS row stride of the rotated key tile, elements (144 B)
constexpr int VS = 68;     // LDS row stride of the transposed value tile, elements (136 B)
constexpr int XCDS = 8;    // accelerator complex dies on MI355X
constexpr float LOG2E = 1.4426950408889634f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Storage-type helpers: widen the low / high element of a packed pair, round a pair of floats
// to the storage type (round-to-nearest-even), and the 32x32x16 matrix instruction.
struct BF16 {
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return __uint_as_float(w & 0xffff0000u);
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct F16 {
    static __device__ __forceinline__ float lo(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
    static __device__ __forceinline__ float hi(uint32_t w) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

// Rotate 8 pairs: x1 holds elements m .. m+7, x2 elements m+32 .. m+39, c / s the table entries
// for m .. m+7 at the row's position. Each output is one float32 rounding of x1 c - x2 s (or
// x1 s + x2 c): the products of two storage-type values are exact in float32, so the fma
// rounds once. Then times `scale` (exact for a power of two) and rounded to the storage type.
template <class E>
__device__ __forceinline__ void rotate8(u32x4 x1, u32x4 x2, u32x4 c, u32x4 s, float scale,
                                        u32x4 &y1, u32x4 &y2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a0 = E::lo(x1[k]), a1 = E::hi(x1[k]);
        const float b0 = E::lo(x2[k]), b1 = E::hi(x2[k]);
        const float c0 = E::lo(c[k]), c1 = E::hi(c[k]);
        const float s0 = E::lo(s[k]), s1 = E::hi(s[k]);
        const float p0 = __builtin_fmaf(a0, c0, -(b0 * s0)) * scale;
        const float p1 = __builtin_fmaf(a1, c1, -(b1 * s1)) * scale;
        const float q0 = __builtin_fmaf(a0, s0, b0 * c0) * scale;
        const float q1 = __builtin_fmaf(a1, s1, b1 * c1) * scale;
        y1[k] = E::pack(p0, p1);
        y2[k] = E::pack(q0, q1);
    }
}

// Max / sum of a value with the same lane's value in the other half of the wave (lane ^ 32).
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class E, int NW>
__global__ void __launch_bounds__(NW * 64)
attend_fwd(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
           const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
           const uint32_t *__restrict__ tiles, uint16_t *__restrict__ out,
           float *__restrict__ lse, int32_t num_tiles, int32_t T, int32_t S, int32_t H, int32_t P,
           int32_t window, float scale) {
    constexpr int BR = 32 * NW;
    constexpr int NTHR = 64 * NW;
    __shared__ __attribute__((aligned(16))) uint16_t ks[BC * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

    // XCD-aware work index: block b runs on XCD b % 8; give each XCD a contiguous range.
    const int nb = (int)gridDim.x;
    const int b = (int)blockIdx.x;
    const int xcd = b % XCDS, slot = b / XCDS;
    const int per = nb / XCDS, extra = nb % XCDS;
    const int work = xcd * per + min(xcd, extra) + slot;
    const int h = work / num_tiles;
    const int tile = work - h * num_tiles;

    const uint32_t seq = tiles[2 * tile];
    const int i0 = (int)tiles[2 * tile + 1];
    if (seq >= (uint32_t)S)
        return;
    const int start = cu[seq];
    const int len = cu[seq + 1] - start;
    if (i0 < 0 || i0 >= len || len > P || start < 0 || (int64_t)start + len > T)
        return;  // a tile that does not match cu reads nothing (uniform over the block)

    const int64_t ld = 3LL * H * D;  // elements per token row of qkv
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int qi = i0 + 32 * wv + n;  // this lane's query position

    // ---- query operand: rotated, scaled, rounded; rows past the sequence are zero.
    // Lane (n, g) holds, for k-step c, dims 16c + 8g .. 16c + 8g + 7 of query n.
    u32x4 qop[4];
    if (qi < len) {
        const uint16_t *qr = qkv + (int64_t)(start + qi) * ld + h * D;
        const u32x4 xa = *(const u32x4 *)(qr + 8 * g);
        const u32x4 xb = *(const u32x4 *)(qr + 16 + 8 * g);
        const u32x4 xc = *(const u32x4 *)(qr + 32 + 8 * g);
        const u32x4 xd = *(const u32x4 *)(qr + 48 + 8 * g);
        const uint16_t *cr = cos_t + qi * 32, *sr = sin_t + qi * 32;
        const u32x4 ca = *(const u32x4 *)(cr + 8 * g), cb = *(const u32x4 *)(cr + 16 + 8 * g);
        const u32x4 sa = *(const u32x4 *)(sr + 8 * g), sb = *(const u32x4 *)(sr + 16 + 8 * g);
        rotate8<E>(xa, xc, ca, sa, scale, qop[0], qop[2]);
        rotate8<E>(xb, xd, cb, sb, scale, qop[1], qop[3]);
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            qop[c] = u32x4{0, 0, 0, 0};
    }

    // ---- the key span this tile's window reaches (whole key tiles of BC)
    int lo = 0, hi = len;
    if (window > 0) {
        if (i0 + 1 > window)
            lo = (i0 + 1 - window) / BC * BC;
        if ((int64_t)i0 + BR + window - 1 < len)
            hi = i0 + BR + window - 1;
    }

    const int w0 = i0 + 32 * wv;            // first row of this wave
    const bool wave_live = w0 < len;
    const int w1 = min(w0 + 31, len - 1);   // last real row of this wave

    float m_run = -__builtin_inff();  // running max of this row's scores
    float l_run = 0.f;                // this lane's share of the row's exp-sum
    f32x16 o0 = {}, o1 = {};          // O^T: dims 0..31 and 32..63 of query n

    const uint16_t *kbase = qkv + (int64_t)start * ld + hd + h * D;
    const uint16_t *vbase = qkv + (int64_t)start * ld + 2 * hd + h * D;

    for (int j0 = lo; j0 < hi; j0 += BC) {
        // ---- stage the key tile (rotated) and the value tile (transposed); zero past the end
        for (int u = tid; u < BC * 4; u += NTHR) {
            const int kk = u >> 2, pp = u & 3;
            const int j = j0 + kk;
            u32x4 y1 = {0, 0, 0, 0}, y2 = {0, 0, 0, 0};
            if (j < len) {
                const uint16_t *kr = kbase + (int64_t)j * ld;
                const u32x4 x1 = *(const u32x4 *)(kr + 8 * pp);
                const u32x4 x2 = *(const u32x4 *)(kr + 32 + 8 * pp);
                const u32x4 c = *(const u32x4 *)(cos_t + j * 32 + 8 * pp);
                const u32x4 s = *(const u32x4 *)(sin_t + j * 32 + 8 * pp);
                rotate8<E>(x1, x2, c, s, 1.0f, y1, y2);
            }
            *(u32x4 *)(ks + kk * KS + 8 * pp) = y1;
            *(u32x4 *)(ks + kk * KS + 32 + 8 * pp) = y2;
        }
        for (int u = tid; u < (BC / 2) * 8; u += NTHR) {
            const int kp = u >> 3, dc = u & 7;
            const int j = j0 + 2 * kp;
            u32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
            const uint16_t *vr = vbase + (int64_t)j * ld + 8 * dc;
            if (j < len)
                va = *(const u32x4 *)vr;
            if (j + 1 < len)
                vb = *(const u32x4 *)(vr + ld);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t a = (e & 1) ? (va[e >> 1] >> 16) : (va[e >> 1] & 0xffffu);
                const uint32_t bb = (e & 1) ? (vb[e >> 1] & 0xffff0000u) : (vb[e >> 1] << 16);
                *(uint32_t *)(vt + (8 * dc + e) * VS + 2 * kp) = a | bb;
            }
        }
        __syncthreads();

        bool any = wave_live;
        if (window > 0)
            any = any && (j0 <= w1 + window - 1) && (j0 + BC - 1 >= w0 - window + 1);
        if (any) {
            // ---- S^T = K~ Q~^T: block 0 keys j0 .. j0+31, block 1 keys j0+32 .. j0+63.
            // Lane (n, g), register i holds key 8(i/4) + 4g + (i%4) of the block, query n.
            f32x16 s0 = {}, s1 = {};
            const uint16_t *k0 = ks + n * KS + 8 * g;
            const uint16_t *k1 = ks + (32 + n) * KS + 8 * g;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s0 = E::mfma(*(const u32x4 *)(k0 + 16 * c), qop[c], s0);
                s1 = E::mfma(*(const u32x4 *)(k1 + 16 * c), qop[c], s1);
            }

            const bool edge = (j0 + BC > len) ||
                              (window > 0 && (w0 + 31 - j0 >= window || j0 + BC - 1 - w0 >= window));
            if (edge) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = j0 + 8 * (i >> 2) + 4 * g + (i & 3);
                    const int ja = j, jb = j + 32;
                    const int da = qi > ja ? qi - ja : ja - qi;
                    const int db = qi > jb ? qi - jb : jb - qi;
                    const bool va = ja < len && (window == 0 || da < window);
                    const bool vb = jb < len && (window == 0 || db < window);
                    s0[i] = va ? s0[i] : -__builtin_inff();
                    s1[i] = vb ? s1[i] : -__builtin_inff();
                }
            }

            // ---- online softmax for query n
            float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int i = 1; i < 16; ++i)
                mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
            mx = pair_max(mx);
            const float m_new = fmaxf(m_run, mx);
            // no visible key yet: any finite reference keeps exp2(-inf) = 0
            const float m_ref = m_new == -__builtin_inff() ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_ref) * LOG2E);
            m_run = m_new;
            const float mb = m_ref * LOG2E;
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], LOG2E, -mb));
                s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], LOG2E, -mb));
                rs += s0[i] + s1[i];
            }
            l_run = l_run * alpha + rs;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                o0[i] *= alpha;
                o1[i] *= alpha;
            }

            // ---- P rounded to the storage type, as the B operand of 16-key steps: step kc
            // takes registers 8(kc%2) .. 8(kc%2)+7 of block kc/2, i.e. keys
            // 16kc + 8(e/4) + 4g + (e%4) for slot e.
            u32x4 pk[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                pk[0][k] = E::pack(s0[2 * k], s0[2 * k + 1]);
                pk[1][k] = E::pack(s0[8 + 2 * k], s0[8 + 2 * k + 1]);
                pk[2][k] = E::pack(s1[2 * k], s1[2 * k + 1]);
                pk[3][k] = E::pack(s1[8 + 2 * k], s1[8 + 2 * k + 1]);
            }

            // ---- O^T += V^T P^T; the A operand for lane (n, g) at step kc is V^T row (dim) n
            // (or 32 + n), keys 16kc + 4g + 0..3 and 16kc + 8 + 4g + 0..3.
            const uint16_t *v0 = vt + n * VS + 4 * g;
            const uint16_t *v1 = vt + (32 + n) * VS + 4 * g;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const u32x2 a0 = *(const u32x2 *)(v0 + 16 * kc);
                const u32x2 a1 = *(const u32x2 *)(v0 + 16 * kc + 8);
                const u32x2 b0 = *(const u32x2 *)(v1 + 16 * kc);
                const u32x2 b1 = *(const u32x2 *)(v1 + 16 * kc + 8);
                o0 = E::mfma(u32x4{a0[0], a0[1], a1[0], a1[1]}, pk[kc], o0);
                o1 = E::mfma(u32x4{b0[0], b0[1], b1[0], b1[1]}, pk[kc], o1);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: out = O / l, lse = m + ln l, for rows inside the sequence
    const float l_tot = pair_sum(l_run);
    if (qi < len) {
        const float inv = 1.0f / l_tot;
        uint16_t *orow = out + (int64_t)(start + qi) * hd + h * D;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x2 wa = {E::pack(o0[4 * q] * inv, o0[4 * q + 1] * inv),
                              E::pack(o0[4 * q + 2] * inv, o0[4 * q + 3] * inv)};
            const u32x2 wb = {E::pack(o1[4 * q] * inv, o1[4 * q + 1] * inv),
                              E::pack(o1[4 * q + 2] * inv, o1[4 * q + 3] * inv)};
            *(u32x2 *)(orow + 8 * q + 4 * g) = wa;
            *(u32x2 *)(orow + 32 + 8 * q + 4 * g) = wb;
        }
        if (g == 0)
            lse[(int64_t)h * T + start + qi] = m_run + logf(l_tot);
    }
}

template <class E, int NW>
int launch_typed(const AttendArgs &a) {
    const int64_t blocks = (int64_t)a.num_tiles * a.H;
    if (blocks > INT32_MAX)
        return fail(VLF_EINVAL, "%lld workgroups exceed the grid limit", (long long)blocks);
    const uint16_t *qkv = (const uint16_t *)a.qkv;
    const uint16_t *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin;
    uint16_t *out = (uint16_t *)a.out;
    int32_t num_tiles = a.num_tiles, T = a.T, S = a.S, H = a.H, P = a.table_rows, W = a.window;
    float scale = a.scale;
    void *args[] = {(void *)&qkv, (void *)&cs,        (void *)&sn, (void *)&a.cu,
                    (void *)&a.tiles, (void *)&out,   (void *)&a.lse, (void *)&num_tiles,
                    (void *)&T,   (void *)&S,         (void *)&H,  (void *)&P,
                    (void *)&W,   (void *)&scale};
    hipError_t e = hipLaunchKernel((const void *)attend_fwd<E, NW>, dim3((unsigned)blocks),
                                   dim3(NW * 64), args, 0, (hipStream_t)a.stream);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "attend launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}

}  // namespace

int launch_attend(const AttendArgs &a) {
    if (a.dtype == VLF_BF16)
        return a.br == 128 ? launch_typed<BF16, 4>(a) : launch_typed<BF16, 2>(a);
    return a.br == 128 ? launch_typed<F16, 4>(a) : launch_typed<F16, 2>(a);
}

}  // namespace vlf
