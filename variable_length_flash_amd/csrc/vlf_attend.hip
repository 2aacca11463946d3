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
//   * The key loop is software-pipelined over 64-key tiles. Step t: the scores of tile t+1 run
//     on the matrix unit while the probabilities of tile t are formed (block A); tile t's output
//     product runs while its row sum is taken and tile t+2 is rotated and written to LDS
//     (block B); then tile t+1 is masked (edge tiles only) and its row maximum taken. LDS holds
//     a ring of three tiles (values of t, keys of t+1, tile t+2 being staged); one barrier per
//     step.
//   * Key/value rows come in through raw buffer loads whose descriptors are rebased per tile in
//     scalar registers: rows past the sequence read as zero in hardware and the per-thread
//     offsets never change. Loads run two steps ahead in two register sets.
//   * Over the full window, each query tile starts its sweep at a different key tile and wraps
//     around, so the workgroups of one (sequence, head) do not all miss L2 on the same tile.
//   * Keys sit row-major in LDS (rows padded to 144 B: the 16-byte operand reads of 16
//     consecutive lanes fall on distinct banks).
//   * Values sit transposed, V^T [dim][key] (rows of 144 B), so the output is computed
//     transposed too, O^T += V^T P^T: the probabilities leave the score accumulators directly as
//     the B operand (after rounding). Inside each 16-key step the accumulator holds keys
//     {0-3, 8-11} in lanes 0-31 and {4-7, 12-15} in lanes 32-63; V^T stores every 16 keys in
//     that order, so each A operand is one 16-byte LDS read. The lanes staging values write
//     rows 8 apart in the two wave halves, which puts a wave's 64 stores on 64 distinct banks.
//     The O^T accumulator gives each lane one query, so the per-row rescale is lane-local.
//   * The softmax keeps, per row, a reference maximum that is only raised when a tile's maximum
//     exceeds it by more than TAU (natural-log units); probabilities stay <= e^TAU, and the
//     rescale of O is skipped for the whole wave when no row needs it. The result is the same
//     as rescaling at every tile (the reference cancels in O / l and is added back in lse).
//   * exp is exp2 with log2(e) folded into one FMA per score.
//   * The 1-D grid is remapped so that consecutive work items land on the same XCD (blocks are
//     dealt round-robin over the 8 XCDs): all tiles of one (sequence, head) share one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/vlf.h"
#include "vlf_internal.h"

namespace vlf {
namespace {

constexpr int D = 64;      // head dimension
constexpr int BC = 64;     // keys per key tile
constexpr int KS = 72;     // LDS row stride of the rotated key tile, elements (144 B)
constexpr int VS = 72;     // LDS row stride of the transposed value tile, elements (144 B)
constexpr int XCDS = 8;    // accelerator complex dies on MI355X
constexpr float LOG2E = 1.4426950408889634f;
constexpr float TAU = 8.0f;  // headroom of the reference maximum, natural-log units
constexpr int RSRC_WORD3 = 0x00020000;  // buffer descriptor word 3: 32-bit data format

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// Storage-type helpers: widen the low / high element of a packed pair, round a pair of floats
// to the storage type (round-to-nearest-even), and the 32x32x16 matrix instruction.
struct BF16 {
    // headroom of the workspace path's reference maximum (natural-log units): probabilities stay
    // below e^16, far inside bfloat16's range
    static constexpr float TAU_PRE = 16.0f;
    // a fixed reference may sit up to this far above a row's largest score: bfloat16 has
    // float32's exponent range, so e^-40 times the probabilities stays normal
    static constexpr float FIX_SLACK = 40.0f;
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
    // e^10 < 65504 (the largest binary16 value), so a rounded probability cannot overflow
    static constexpr float TAU_PRE = 10.0f;
    // a fixed reference never exceeds a row's largest score: the largest probability stays at
    // least 1, as with the running maximum, and small ones keep binary16's normal range
    static constexpr float FIX_SLACK = 0.0f;
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

// Rotate 2*W pairs held as W packed words each: x1 has elements m.., x2 elements m+32.., c / s
// the table entries for m.. at the row's position. Each output is one float32 rounding of
// x1 c - x2 s (or x1 s + x2 c): the products of two storage-type values are exact in float32,
// so the fma rounds once. Then times `scale` (a power of two in practice, so exact) and rounded
// to the storage type.
template <class E, int W>
__device__ __forceinline__ void rotate(const uint32_t *x1, const uint32_t *x2, const uint32_t *c,
                                       const uint32_t *s, float scale, uint32_t *y1,
                                       uint32_t *y2) {
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const float a0 = E::lo(x1[k]), a1 = E::hi(x1[k]);
        const float b0 = E::lo(x2[k]), b1 = E::hi(x2[k]);
        const float c0 = E::lo(c[k]), c1 = E::hi(c[k]);
        const float s0 = E::lo(s[k]), s1 = E::hi(s[k]);
        float p0 = __builtin_fmaf(a0, c0, -(b0 * s0)) * scale;
        float p1 = __builtin_fmaf(a1, c1, -(b1 * s1)) * scale;
        float q0 = __builtin_fmaf(a0, s0, b0 * c0) * scale;
        float q1 = __builtin_fmaf(a1, s1, b1 * c1) * scale;
        // Materialise the float32 results: the storage-type rounding must see them. Left to
        // itself the compiler fuses an fma with the narrowing (v_fma_mix*_f16), which rounds
        // the exact value once and differs wherever the float32 result is a binary16 tie.
        asm volatile("" : "+v"(p0), "+v"(p1), "+v"(q0), "+v"(q1));
        y1[k] = E::pack(p0, p1);
        y2[k] = E::pack(q0, q1);
    }
}

// out row = O / l in float32, then the storage-type rounding (the float32 quotient is
// materialised first so that no fused operation rounds the exact quotient instead). The
// quotient takes one reciprocal of l per row and, per element, the product and one Newton
// correction y + (o - l y) r: within one float32 ulp of the correctly rounded quotient, at 3
// instructions instead of a full division's 10. l lies in float32's normal range (the largest
// probability is at least e^-40).
// Lane (n, g) holds dims 8q + 4g .. +3 (o0) and 32 + 8q + 4g .. +3 (o1) of its query.
__device__ __forceinline__ float quotient(float o, float l, float r) {
    const float y = o * r;
    return __builtin_fmaf(__builtin_fmaf(-l, y, o), r, y);
}

template <class E>
__device__ __forceinline__ void store_out(const f32x16 &o0, const f32x16 &o1, float l,
                                          uint16_t *orow, int g) {
    const float r = __builtin_amdgcn_rcpf(l);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float a[4], b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = quotient(o0[4 * q + e], l, r);
            b[e] = quotient(o1[4 * q + e], l, r);
        }
        asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
        asm volatile("" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
        *(u32x2 *)(orow + 8 * q + 4 * g) = u32x2{E::pack(a[0], a[1]), E::pack(a[2], a[3])};
        *(u32x2 *)(orow + 32 + 8 * q + 4 * g) = u32x2{E::pack(b[0], b[1]), E::pack(b[2], b[3])};
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

// Position of key k (0..63) of a tile inside a V^T row: within each 16 keys, swap bits 2 and 3
// of the index, so keys {0-3, 8-11} come first and {4-7, 12-15} second.
__device__ __forceinline__ int vt_slot(int k) {
    return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// A buffer resource over `bytes` bytes from base. Every resource here is built from
// wave-uniform values (an item's, tile's or sequence's); they are read from the first lane so
// that the compiler keeps the resource in scalar registers instead of wrapping each load that
// uses it in a loop over the lanes' distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes),
                                             RSRC_WORD3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t *base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffLL ? 0xffffffffLL : bytes);
    return make_rsrc(base, (uint32_t)n);
}

__device__ __forceinline__ u32x2 load8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// One thread's share of staging a 64-key tile, for NTHR threads.
//   keys:   KP pairs (m, m+32) of key row kk, m = pp .. pp+KP-1;
//   values: key rows 2kp and 2kp+1 (kp = lane % 32), VD dims in chunks of 4; the chunk index C
//           (dims 4C .. 4C+3) has bit 1 equal to the wave half, so the two halves of a wave
//           write V^T rows 8 apart.
template <int NTHR>
struct Staging {
    static constexpr int KP = 2048 / NTHR;    // key pairs per thread (64 keys x 32 pairs)
    static constexpr int KW = KP / 2;         // packed words per operand
    static constexpr int TPK = 32 / KP;       // threads per key row
    static constexpr int VC = 512 / NTHR;     // 4-dim value chunks per thread (16 x 32 pairs)
    int kk, pp, kp;
    int vchunk[VC];
    int koff, toff, voff;                     // byte offsets inside the tile's descriptors

    __device__ void init(int tid, int64_t ld) {
        kk = tid / TPK;
        pp = (tid % TPK) * KP;
        const int lane = tid & 63, w = tid >> 6, half = lane >> 5;
        kp = lane & 31;
        constexpr int per = VC;  // chunks per (wave, half) = 8 / waves
#pragma unroll
        for (int q = 0; q < VC; ++q) {
            const int k = w * per + q;  // 0..7 over the waves of the block
            vchunk[q] = (k & 1) | (half << 1) | ((k >> 1) << 2);
        }
        koff = (int)(kk * ld * 2) + pp * 2;
        toff = kk * 64 + pp * 2;
        voff = (int)(2 * kp * ld * 2);
    }
};

template <int NTHR>
struct TileRegs {
    uint32_t x1[Staging<NTHR>::KW], x2[Staging<NTHR>::KW];
    uint32_t c[Staging<NTHR>::KW], s[Staging<NTHR>::KW];
    u32x2 va[Staging<NTHR>::VC], vb[Staging<NTHR>::VC];
};

// Where a workgroup's key/value rows and table rows come from. With FIXED, one descriptor per
// source covers the whole sequence (32-bit offsets reach every row) and a tile's row offset is
// added to the per-thread offsets; otherwise the descriptors are rebased on every tile.
template <bool FIXED>
struct Sources {
    const uint16_t *kbase, *vbase, *cos_t, *sin_t;
    int len, P;
    int64_t ld;
    int row_bytes;
    __amdgpu_buffer_rsrc_t kr, vr, cr, sr;  // FIXED only

    __device__ void init(const uint16_t *k, const uint16_t *v, const uint16_t *c,
                         const uint16_t *sn, int len_, int P_, int64_t ld_) {
        kbase = k, vbase = v, cos_t = c, sin_t = sn, len = len_, P = P_, ld = ld_;
        row_bytes = (int)(ld * 2);
        if (FIXED) {
            kr = rsrc(kbase, (int64_t)len * row_bytes);
            vr = rsrc(vbase, (int64_t)len * row_bytes);
            cr = rsrc(cos_t, (int64_t)P * 64);
            sr = rsrc(sin_t, (int64_t)P * 64);
        }
    }
};

template <int NTHR, bool FIXED>
__device__ __forceinline__ void stage_load(TileRegs<NTHR> &r, const Staging<NTHR> &sg,
                                           const Sources<FIXED> &src, int j0) {
    using S = Staging<NTHR>;
    __amdgpu_buffer_rsrc_t kr, vr, cr, sr;
    int kdelta, tdelta;
    if (FIXED) {
        kr = src.kr, vr = src.vr, cr = src.cr, sr = src.sr;
        kdelta = j0 * src.row_bytes;
        tdelta = j0 * 64;
    } else {
        kr = rsrc(src.kbase + (int64_t)j0 * src.ld, (int64_t)(src.len - j0) * src.row_bytes);
        vr = rsrc(src.vbase + (int64_t)j0 * src.ld, (int64_t)(src.len - j0) * src.row_bytes);
        cr = rsrc(src.cos_t + (int64_t)j0 * 32, (int64_t)(src.P - j0) * 64);
        sr = rsrc(src.sin_t + (int64_t)j0 * 32, (int64_t)(src.P - j0) * 64);
        kdelta = 0;
        tdelta = 0;
    }
    const int koff = sg.koff + kdelta, toff = sg.toff + tdelta;
#pragma unroll
    for (int w = 0; w < S::KW; w += 2) {
        const u32x2 a = load8(kr, koff + 4 * w);
        const u32x2 b = load8(kr, koff + 64 + 4 * w);
        const u32x2 cc = load8(cr, toff + 4 * w);
        const u32x2 ss = load8(sr, toff + 4 * w);
        r.x1[w] = a[0], r.x1[w + 1] = a[1];
        r.x2[w] = b[0], r.x2[w + 1] = b[1];
        r.c[w] = cc[0], r.c[w + 1] = cc[1];
        r.s[w] = ss[0], r.s[w + 1] = ss[1];
    }
    const int va = sg.voff + kdelta, vb = sg.voff + src.row_bytes + kdelta;
#pragma unroll
    for (int q = 0; q < S::VC; ++q) {
        r.va[q] = load8(vr, va + sg.vchunk[q] * 8);
        r.vb[q] = load8(vr, vb + sg.vchunk[q] * 8);
    }
}

// Rotates and rounds this thread's keys into K~ and transposes its values into V^T.
template <class E, int NTHR>
__device__ __forceinline__ void stage_keys(const TileRegs<NTHR> &r, const Staging<NTHR> &sg,
                                           uint16_t *ks) {
    using S = Staging<NTHR>;
    uint32_t y1[S::KW], y2[S::KW];
    rotate<E, S::KW>(r.x1, r.x2, r.c, r.s, 1.0f, y1, y2);
#pragma unroll
    for (int w = 0; w < S::KW; w += 2) {
        *(u32x2 *)(ks + sg.kk * KS + sg.pp + 2 * w) = u32x2{y1[w], y1[w + 1]};
        *(u32x2 *)(ks + sg.kk * KS + 32 + sg.pp + 2 * w) = u32x2{y2[w], y2[w + 1]};
    }
}

template <int NTHR>
__device__ __forceinline__ void stage_values(const TileRegs<NTHR> &r, const Staging<NTHR> &sg,
                                             uint16_t *vt) {
    using S = Staging<NTHR>;
    const int slot = vt_slot(2 * sg.kp);
#pragma unroll
    for (int q = 0; q < S::VC; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t wa = r.va[q][e >> 1], wb = r.vb[q][e >> 1];
            const uint32_t a = (e & 1) ? (wa >> 16) : (wa & 0xffffu);
            const uint32_t b = (e & 1) ? (wb & 0xffff0000u) : (wb << 16);
            *(uint32_t *)(vt + (4 * sg.vchunk[q] + e) * VS + slot) = a | b;
        }
    }
}

// keys false: this thread's key rows are never read, so they are not staged
template <class E, int NTHR>
__device__ __forceinline__ void stage_store(const TileRegs<NTHR> &r, const Staging<NTHR> &sg,
                                            uint16_t *ks, uint16_t *vt, bool keys = true) {
    if (keys)
        stage_keys<E, NTHR>(r, sg, ks);
    stage_values<NTHR>(r, sg, vt);
}

// Raw inputs of one lane's query operand: dims 8g .. 8g+7, 16+8g .., 32+8g .., 48+8g .. of the
// query row and the table entries for dims 8g .., 16+8g .. at its position (zero past the
// sequence).
struct QueryRaw {
    u32x4 x[4], c[2], s[2];
};

__device__ __forceinline__ void query_load(QueryRaw &r, const uint16_t *qkv,
                                           const uint16_t *cos_t, const uint16_t *sin_t,
                                           int64_t ld, int start, int qi, int len, int h, int g) {
    u32x4 x0 = {0, 0, 0, 0}, x1 = x0, x2 = x0, x3 = x0, c0 = x0, c1 = x0, s0 = x0, s1 = x0;
    if (qi < len) {
        const uint16_t *qr = qkv + (int64_t)(start + qi) * ld + h * D + 8 * g;
        x0 = *(const u32x4 *)qr;
        x1 = *(const u32x4 *)(qr + 16);
        x2 = *(const u32x4 *)(qr + 32);
        x3 = *(const u32x4 *)(qr + 48);
        const uint16_t *cr = cos_t + qi * 32 + 8 * g, *sr = sin_t + qi * 32 + 8 * g;
        c0 = *(const u32x4 *)cr;
        c1 = *(const u32x4 *)(cr + 16);
        s0 = *(const u32x4 *)sr;
        s1 = *(const u32x4 *)(sr + 16);
    }
    r.x[0] = x0, r.x[1] = x1, r.x[2] = x2, r.x[3] = x3;
    r.c[0] = c0, r.c[1] = c1, r.s[0] = s0, r.s[1] = s1;
}

// Query operand of one 32-row block: rows rotated, scaled, rounded; rows past the sequence are
// zero (a zero row rotates to zero). Lane (n, g) holds, for k-step c, dims 16c + 8g .. 16c +
// 8g + 7 of its query.
template <class E>
__device__ __forceinline__ void query_make(const QueryRaw &r, float scale, u32x4 (&qop)[4]) {
    uint32_t y[4][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t x1[4] = {r.x[k][0], r.x[k][1], r.x[k][2], r.x[k][3]};
        const uint32_t x2[4] = {r.x[k + 2][0], r.x[k + 2][1], r.x[k + 2][2], r.x[k + 2][3]};
        const uint32_t c[4] = {r.c[k][0], r.c[k][1], r.c[k][2], r.c[k][3]};
        const uint32_t s[4] = {r.s[k][0], r.s[k][1], r.s[k][2], r.s[k][3]};
        rotate<E, 4>(x1, x2, c, s, scale, y[k], y[k + 2]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
        qop[c] = u32x4{y[c][0], y[c][1], y[c][2], y[c][3]};
}

template <class E>
__device__ __forceinline__ void query_operand(const uint16_t *qkv, const uint16_t *cos_t,
                                              const uint16_t *sin_t, int64_t ld, int start,
                                              int qi, int len, int h, int g, float scale,
                                              u32x4 (&qop)[4]) {
    QueryRaw r;
    query_load(r, qkv, cos_t, sin_t, ld, start, qi, len, h, g);
    query_make<E>(r, scale, qop);
}

// Scores of one key tile for one 32-row block: S^T = K~ Q~^T from the key tile in LDS. Block 0
// holds keys 0..31 of the tile, block 1 keys 32..63; lane (n, g), register i holds key
// 8(i/4) + 4g + (i%4) of the block for query n.
template <class E>
__device__ __forceinline__ void scores(const uint16_t *kt, const u32x4 (&qop)[4], int n, int g,
                                       f32x16 &s0, f32x16 &s1) {
    const uint16_t *k0 = kt + n * KS + 8 * g;
    const uint16_t *k1 = kt + (32 + n) * KS + 8 * g;
    u32x4 a[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        a[2 * c] = *(const u32x4 *)(k0 + 16 * c);
        a[2 * c + 1] = *(const u32x4 *)(k1 + 16 * c);
    }
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        s0 = E::mfma(a[2 * c], qop[c], s0);
        s1 = E::mfma(a[2 * c + 1], qop[c], s1);
    }
}

// Masks the scores of the key tile at j0 to the keys lo <= j < hi: register i of block b holds
// key j0 + 32b + 8(i/4) + 4g + i%4 (one subtraction, one comparison and one select each).
__device__ __forceinline__ void mask_band(f32x16 &s0, f32x16 &s1, int lo, int hi, int j0,
                                          int g) {
    const int a = lo - j0 - 4 * g;
    const uint32_t span = (uint32_t)max(hi - lo, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int o = 8 * (i >> 2) + (i & 3);
        s0[i] = (uint32_t)(o - a) < span ? s0[i] : -__builtin_inff();
        s1[i] = (uint32_t)(o + 32 - a) < span ? s1[i] : -__builtin_inff();
    }
}

// The window as two reaches: row x sees keys x - back <= j <= x + ahead of its sequence. The
// symmetric window W >= 1 is back = ahead = W - 1, the causal window W >= 1 is back = W - 1 and
// ahead = 0, and REACH_ALL (on both sides, or behind for the causal full window) reaches every
// key. The host turns the caller's window into the two.
constexpr int32_t REACH_ALL = 0x7fffffff;

// The visible keys [lo, hi) of row x of a sequence of `len` rows.
__device__ __forceinline__ void row_keys(int x, int len, int back, int ahead, int &lo, int &hi) {
    lo = x > back ? x - back : 0;
    hi = (int)min((int64_t)x + ahead + 1, (int64_t)len);
}

// The whole 64-key tiles [lo, hi) that rows [r0, r0 + rows) reach (hi clipped to the sequence).
__device__ __forceinline__ void key_span(int r0, int rows, int len, int back, int ahead, int &lo,
                                         int &hi) {
    lo = r0 > back ? (r0 - back) / BC * BC : 0;
    hi = (int64_t)r0 + rows + ahead < len ? r0 + rows + ahead : len;
}

// Whether some pair of rows [w0, w0 + 32) and keys [j0, j0 + 64) lies outside the window or the
// sequence: the tile then needs masks.
__device__ __forceinline__ bool tile_edge(int w0, int j0, int len, int back, int ahead) {
    return j0 + BC > len || w0 + 31 - j0 > back || j0 + BC - 1 - w0 > ahead;
}

// Masks the scores of the 64-key tile at j0 for query qi (keys past the sequence and outside
// the window weigh nothing).
__device__ __forceinline__ void mask_scores(f32x16 &s0, f32x16 &s1, int j0, int len, int back,
                                            int ahead, int qi, int g) {
    int lo, hi;
    row_keys(qi, len, back, ahead, lo, hi);
    mask_band(s0, s1, lo, hi, j0, g);
}

// Maximum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x = __builtin_fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Which wave group a sweep of attend_pre_ph runs for (true: the late group).
template <bool F>
struct LateGroup {
    static constexpr bool value = F;
};

// Row maximum over the 64-key tile, shared by lanes n and n + 32.
__device__ __forceinline__ float row_max(const f32x16 &s0, const f32x16 &s1) {
    float mx = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i)
        mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[i]), s1[i]);
    return pair_max(mx);
}

// ---- pre-rotated key tiles --------------------------------------------------------------------
// A workspace block holds key tile u of sequence s for head h as two 8 KB LDS images: the
// rotated, rounded keys K~ [key][dim] and the values V^T [dim][slot] (slots in the order of
// vt_slot). Each image has 64 rows of 128 B; 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7), so the operand reads of 16 consecutive lanes (rows n .. n+15, one chunk
// each) cover all 16 chunk positions of two 128-byte rows and fall on distinct banks. The block
// index floor(cu[s] / 64) + s + u keeps the sequences' blocks apart without a prefix sum.
constexpr int IMG = 8192;     // bytes of one 64 x 64 image
constexpr int BLK = 2 * IMG;  // bytes of one key tile's block

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Margin on a computed norm: the float32 sum of 64 squares and v_sqrt_f32 are each within a few
// ulp, so a factor 1 + 2^-10 makes the result an upper bound of the exact norm.
constexpr float NORM_MARGIN = 1.0f + 1.0f / 1024.0f;

// ---- the fixed reference maximum of the workspace path ----------------------------------------
// A sweep over pre-rotated key tiles fixes each row's reference maximum before its loop, so no
// step takes a row maximum or rescales the accumulators (the reference cancels in O / l and
// returns in lse = m_ref + ln l). Every score of the row is at most bq = |q~| times the largest
// key norm among the swept blocks (both upper bounds), so a reference at or above bq - TAU_PRE
// keeps each probability within e^TAU_PRE. With m0 any value no larger than the row's largest
// score, max(m0, bq - TAU_PRE) also keeps the row's largest probability at least e^-FIX_SLACK
// when bq - TAU_PRE - m0 <= FIX_SLACK. Where that fails for a row, its wave first sweeps the
// scores alone for the exact row maximum and takes that as the reference.

// Largest key norm bound among the ntiles blocks from knorm[kb]: the first 128 are read before
// the caller's copies start (kn0, kn1), the rest after.
__device__ __forceinline__ void key_norm_reads(const float *knorm, int kb, int ntiles, int lane,
                                               float &kn0, float &kn1) {
    kn0 = lane < ntiles ? knorm[kb + lane] : 0.f;
    kn1 = lane + 64 < ntiles ? knorm[kb + lane + 64] : 0.f;
}
__device__ __forceinline__ float key_norm_max(const float *knorm, int kb, int ntiles, int lane,
                                              float kn0, float kn1) {
    float kmax = __builtin_fmaxf(kn0, kn1);
    for (int u = lane + 128; u < ntiles; u += 64)
        kmax = __builtin_fmaxf(kmax, knorm[kb + u]);
    return wave_max(kmax);
}

// Score of row qi with its own key (always visible), from the workspace block that holds it;
// -inf for rows past the sequence. Shared by lanes n and n + 32. own_key reads the lane's half
// of the key row (zero past the sequence), own_dot forms the score from it, so that the read
// can be issued before the query operand exists.
__device__ __forceinline__ void own_key(const uint8_t *wblock, int qi, int len, int g,
                                        u32x4 (&kw)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        kw[c] = u32x4{0, 0, 0, 0};
    if (qi < len) {
        const int r = qi % BC;
        const uint8_t *krow = wblock + (int64_t)(qi / BC) * BLK + r * 128;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            kw[c] = *(const u32x4 *)(krow + 16 * ((2 * c + g) ^ swz(r)));
    }
}
template <class E>
__device__ __forceinline__ float own_dot(const u32x4 (&kw)[4], const u32x4 (&qop)[4], int qi,
                                         int len) {
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            d = __builtin_fmaf(E::lo(qop[c][w]), E::lo(kw[c][w]), d);
            d = __builtin_fmaf(E::hi(qop[c][w]), E::hi(kw[c][w]), d);
        }
    d = pair_sum(d);
    return qi < len ? d : -__builtin_inff();
}
template <class E>
__device__ __forceinline__ float own_score(const uint8_t *wblock, const u32x4 (&qop)[4], int qi,
                                           int len, int g) {
    u32x4 kw[4];
    own_key(wblock, qi, len, g, kw);
    return own_dot<E>(kw, qop, qi, len);
}

// The reference of each row of a wave: m_tile is the row maximum of one swept tile (masked),
// s_own the row's own score, bq its score bound. `exact` returns the exact row maximum.
template <class E, class Exact>
__device__ __forceinline__ float fixed_reference(float m_tile, float s_own, float bq, bool valid,
                                                 Exact exact) {
    const float m0 = __builtin_fmaxf(m_tile, s_own);
    const bool ok = !valid || bq - E::TAU_PRE - m0 <= E::FIX_SLACK;
    if (__builtin_amdgcn_ballot_w64(!ok))
        return exact();
    return __builtin_fmaxf(m0, bq - E::TAU_PRE);
}

// Exact row maximum over tiles key(0) .. key(ntiles - 1): the scores alone, each tile's key
// image read from its workspace block in global memory (the same bytes and products as the
// sweep's, so the same scores).
template <class E, class KeyF, class EdgeF>
__device__ __forceinline__ float exact_row_max(const uint8_t *wblock,
                                                         const u32x4 (&qop)[4],
                                                         const int (&cof)[4], int ntiles,
                                                         KeyF key, EdgeF edge, int len,
                                                         int back, int ahead, int qi, int g) {
    float mx = -__builtin_inff();
    for (int u = 0; u < ntiles; ++u) {
        const int ju = key(u);
        const uint8_t *kg = wblock + (int64_t)(ju / BC) * BLK;
        f32x16 a0 = {}, a1 = {};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            a0 = E::mfma(*(const u32x4 *)(kg + cof[c]), qop[c], a0);
            a1 = E::mfma(*(const u32x4 *)(kg + 4096 + cof[c]), qop[c], a1);
        }
        if (edge(ju))
            mask_scores(a0, a1, ju, len, back, ahead, qi, g);
        mx = __builtin_fmaxf(mx, row_max(a0, a1));
    }
    return mx;
}

// One workgroup per block and group of four heads writes those heads' blocks: keys rotated and
// rounded exactly as the staging of the other path does, values transposed; keys past the
// sequence are zero. The rotation table rows are read once for the four heads, and every key
// and value row is requested before the first is used. It also writes an upper bound of the
// largest Euclidean norm among each block's rounded keys into the norm array that follows the
// blocks (index h * NB + block).
constexpr int PREP_HEADS = 4;  // heads one prep_tiles workgroup rotates for its block

template <class E>
__global__ void __launch_bounds__(256)
prep_tiles(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
           const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
           uint8_t *__restrict__ ws, int32_t NB, int32_t T, int32_t S, int32_t H, int32_t P) {
    __shared__ uint16_t vrow[PREP_HEADS][64][72];
    __shared__ float wmax[PREP_HEADS][4];
    __shared__ int owner;
    // block b of heads h0 .. h0 + PREP_HEADS - 1 (the table rows are read once for all of them)
    const int b = (int)(blockIdx.x % (uint32_t)NB);
    const int h0 = (int)(blockIdx.x / (uint32_t)NB) * PREP_HEADS;
    const int tid = (int)threadIdx.x;
    // The sequence owning block b: the largest s with floor(cu[s] / 64) + s <= b, i.e. the one
    // s with key(s) <= b < key(s + 1) for key(s) = floor(cu[s] / 64) + s, which rises with s.
    // A search narrows it to at most 256 candidates, then one thread per candidate tests it:
    // one memory round trip for batches of up to 256 sequences.
    int lo = 0, hi = S - 1;
    while (hi - lo >= 256) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] / 64 + mid <= b)
            lo = mid;
        else
            hi = mid - 1;
    }
    if (tid == 0)
        owner = lo;
    __syncthreads();
    if (tid > 0 && lo + tid <= hi && cu[lo + tid] / 64 + lo + tid <= b &&
        (lo + tid == hi || cu[lo + tid + 1] / 64 + lo + tid + 1 > b))
        owner = lo + tid;
    __syncthreads();
    const int s = owner;
    const int start = cu[s];
    const int len = cu[s + 1] - start;
    if (start < 0 || len <= 0 || len > P || (int64_t)start + len > T)
        return;
    const int u = b - (start / 64 + s);
    if (u < 0 || u >= (len + BC - 1) / BC)
        return;  // a block no tile of this sequence uses (uniform over the workgroup)
    const int j0 = BC * u;
    const int nvalid = min(BC, len - j0);
    const int64_t ld = 3LL * H * D;

    // thread (r, q): key row r, pairs m = 8q .. 8q+7 (dims m and m+32), value dims 16q .. 16q+15;
    // every head's rows and the table entries are requested before any is used
    const int r = tid >> 2, q = tid & 3;
    u32x4 c = {0, 0, 0, 0}, sn = {0, 0, 0, 0};
    u32x4 x1[PREP_HEADS], x2[PREP_HEADS], va[PREP_HEADS], vb[PREP_HEADS];
#pragma unroll
    for (int k = 0; k < PREP_HEADS; ++k)
        x1[k] = x2[k] = va[k] = vb[k] = u32x4{0, 0, 0, 0};
    if (r < nvalid) {
        const uint16_t *krow = qkv + (int64_t)(start + j0 + r) * ld + H * D;
#pragma unroll
        for (int k = 0; k < PREP_HEADS; ++k) {
            if (h0 + k < H) {
                const uint16_t *kr = krow + (h0 + k) * D, *vr = kr + H * D;
                x1[k] = *(const u32x4 *)(kr + 8 * q);
                x2[k] = *(const u32x4 *)(kr + 32 + 8 * q);
                va[k] = *(const u32x4 *)(vr + 16 * q);
                vb[k] = *(const u32x4 *)(vr + 16 * q + 8);
            }
        }
        c = *(const u32x4 *)(cos_t + (j0 + r) * 32 + 8 * q);
        sn = *(const u32x4 *)(sin_t + (j0 + r) * 32 + 8 * q);
    }
    const uint32_t c_[4] = {c[0], c[1], c[2], c[3]}, s_[4] = {sn[0], sn[1], sn[2], sn[3]};
#pragma unroll
    for (int k = 0; k < PREP_HEADS; ++k) {
        if (h0 + k >= H)
            break;  // uniform over the workgroup
        uint8_t *blk = ws + ((int64_t)(h0 + k) * NB + b) * BLK;
        uint32_t y1[4], y2[4];
        {
            const uint32_t a_[4] = {x1[k][0], x1[k][1], x1[k][2], x1[k][3]};
            const uint32_t b_[4] = {x2[k][0], x2[k][1], x2[k][2], x2[k][3]};
            rotate<E, 4>(a_, b_, c_, s_, 1.0f, y1, y2);
        }
        *(u32x4 *)(blk + r * 128 + 16 * (q ^ swz(r))) = u32x4{y1[0], y1[1], y1[2], y1[3]};
        *(u32x4 *)(blk + r * 128 + 16 * ((4 + q) ^ swz(r))) = u32x4{y2[0], y2[1], y2[2], y2[3]};
        *(u32x4 *)&vrow[k][r][16 * q] = va[k];
        *(u32x4 *)&vrow[k][r][16 * q + 8] = vb[k];
        // squared norm of key row r (its 64 rounded elements sit in lanes 4r .. 4r+3), then
        // the largest over the wave's 16 rows
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a0 = E::lo(y1[e]), a1 = E::hi(y1[e]), b0 = E::lo(y2[e]), b1 = E::hi(y2[e]);
            sq = __builtin_fmaf(a0, a0, sq);
            sq = __builtin_fmaf(a1, a1, sq);
            sq = __builtin_fmaf(b0, b0, sq);
            sq = __builtin_fmaf(b1, b1, sq);
        }
        sq += __shfl_xor(sq, 1);
        sq += __shfl_xor(sq, 2);
#pragma unroll
        for (int off = 4; off < 64; off <<= 1)
            sq = fmaxf(sq, __shfl_xor(sq, off));
        if ((tid & 63) == 0)
            wmax[k][tid >> 6] = sq;
    }
    __syncthreads();
    // V^T and the norm bound of each head's block
    const int d = tid >> 2;
#pragma unroll
    for (int k = 0; k < PREP_HEADS; ++k) {
        if (h0 + k >= H)
            break;
        uint8_t *blk = ws + ((int64_t)(h0 + k) * NB + b) * BLK;
        if (tid == 0) {
            const float m = fmaxf(fmaxf(wmax[k][0], wmax[k][1]), fmaxf(wmax[k][2], wmax[k][3]));
            float *norms = (float *)(ws + (int64_t)H * NB * BLK);
            norms[(int64_t)(h0 + k) * NB + b] = __builtin_sqrtf(m) * NORM_MARGIN;
        }
        // thread (d, q) writes chunks 2q and 2q+1 of row d; chunk ch holds slots 8ch .. 8ch+7
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int ch = 2 * q + e;
            uint32_t wv4[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int k0 = vt_slot(8 * ch + 2 * jj), k1 = vt_slot(8 * ch + 2 * jj + 1);
                wv4[jj] = (uint32_t)vrow[k][k0][d] | ((uint32_t)vrow[k][k1][d] << 16);
            }
            *(u32x4 *)(blk + IMG + d * 128 + 16 * (ch ^ swz(d))) =
                u32x4{wv4[0], wv4[1], wv4[2], wv4[3]};
        }
    }
}

template <class E, int NW, bool FIXED>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
attend_fwd(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
           const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
           const uint32_t *__restrict__ tiles, uint16_t *__restrict__ out,
           float *__restrict__ lse, int32_t num_tiles, int32_t T, int32_t S, int32_t H, int32_t P,
           int32_t back, int32_t ahead, float scale) {
    constexpr int BR = 32 * NW;
    constexpr int NTHR = 64 * NW;
    constexpr int RING = 3;  // key/value tiles in LDS: t (values), t+1 (keys), t+2 (being staged)
    __shared__ __attribute__((aligned(16))) uint16_t ks[RING][BC * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vt[RING][D * VS];

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
    const int w0 = i0 + 32 * __builtin_amdgcn_readfirstlane(wv);  // first row of this wave
    const int qi = w0 + n;        // this lane's query position

    // ---- the key span this tile's window reaches (whole key tiles of BC)
    int lo, hi;
    key_span(i0, BR, len, back, ahead, lo, hi);
    const int ntiles = (hi - lo + BC - 1) / BC;
    // Over the full window every query tile of a sequence reads every key tile: start each at
    // a different key tile (and wrap around) so the workgroups of one (sequence, head), which
    // run side by side on one XCD, do not all miss L2 on the same tile at the same time. The
    // online softmax does not depend on the order of the keys.
    const int offset = (back < REACH_ALL || ahead < REACH_ALL)
                           ? 0
                           : (int)((int64_t)(i0 / BR) * ntiles / ((len + BR - 1) / BR));
    // first key of the t-th tile in this workgroup's order (t <= ntiles)
    auto key = [&](int t) {
        int u = t + offset;
        if (u >= ntiles)
            u -= ntiles;
        return lo + u * BC;
    };

    const uint16_t *kbase = qkv + (int64_t)start * ld + hd + h * D;
    const uint16_t *vbase = qkv + (int64_t)start * ld + 2 * hd + h * D;

    // ---- prologue: tiles 0 and 1 staged in LDS, tiles 2 and 3 in flight to registers
    Staging<NTHR> sg;
    sg.init(tid, ld);
    Sources<FIXED> src;
    src.init(kbase, vbase, cos_t, sin_t, len, P, ld);
    TileRegs<NTHR> ra, rb;
    // (tiles past the span are neither loaded nor staged: a sequence of one key tile costs one)
    stage_load(ra, sg, src, key(0));
    if (ntiles > 1)
        stage_load(rb, sg, src, key(1));
    u32x4 qop[4];
    query_operand<E>(qkv, cos_t, sin_t, ld, start, qi, len, h, g, scale, qop);
    stage_store<E, NTHR>(ra, sg, ks[0], vt[0]);
    if (ntiles > 2)
        stage_load(ra, sg, src, key(2));
    if (ntiles > 1)
        stage_store<E, NTHR>(rb, sg, ks[1], vt[1]);
    if (ntiles > 3)
        stage_load(rb, sg, src, key(3));
    __syncthreads();

    // A tile needs masks when it reaches past the sequence or some pair of this wave's rows
    // and its keys lies outside the window.
    auto edge = [&](int j0) {
        return tile_edge(w0, j0, len, back, ahead);
    };

    float m_ref = -__builtin_inff();  // reference maximum, natural-log units
    float l_run = 0.f;                // this lane's share of the row's exp-sum
    f32x16 o0 = {}, o1 = {};          // O^T: dims 0..31 and 32..63 of query n
    f32x16 sa0, sa1, sb0, sb1;        // scores of the current and the next key tile

    scores<E>(ks[0], qop, n, g, sa0, sa1);
    if (edge(key(0)))
        mask_scores(sa0, sa1, key(0), len, back, ahead, qi, g);
    float mx = row_max(sa0, sa1);

    // One key tile t: c0/c1 hold its masked scores and mx their row maximum; n0/n1 receive the
    // scores of tile t+1. LDS ring slots: values of t in `cur`, keys of t+1 in the next slot;
    // tile t+2 (register set `st`) is staged into the slot after, then set `st` receives tile
    // t+4. Past the span nothing is loaded or staged; the scores of a tile past the span read
    // a stale slot and are never used.
    auto step = [&](f32x16 &c0, f32x16 &c1, f32x16 &n0, f32x16 &n1, TileRegs<NTHR> &st, int t,
                    int cur) {
        const int nxt = cur == RING - 1 ? 0 : cur + 1;
        const int fut = nxt == RING - 1 ? 0 : nxt + 1;
        const int j1 = key(t + 1);

        // raise the reference maximum where this tile exceeds it by more than TAU; lanes that
        // keep it scale by exactly 1 (their m_ref may still be -inf, where the difference
        // would be NaN); a first reference scales the zero state by 0
        const bool raise = mx > m_ref + TAU;  // false while nothing is visible
        const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mx) * LOG2E) : 1.0f;
        m_ref = raise ? mx : m_ref;
        l_run *= alpha;
        if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                o0[i] *= alpha;
                o1[i] *= alpha;
            }
        }
        // no visible key yet: any finite reference keeps exp2(-inf) = 0
        const float mb = m_ref == -__builtin_inff() ? 0.f : m_ref * LOG2E;

        // ---- block A: the scores of tile t+1 on the matrix unit while the probabilities of
        // tile t are formed and rounded: the B operand of 16-key step kc takes registers
        // 8(kc%2) .. 8(kc%2)+7 of block kc/2, i.e. keys 16kc + 8(e/4) + 4g + (e%4).
        scores<E>(ks[nxt], qop, n, g, n0, n1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            c0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(c0[i], LOG2E, -mb));
            c1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(c1[i], LOG2E, -mb));
        }
        u32x4 pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pk[0][k] = E::pack(c0[2 * k], c0[2 * k + 1]);
            pk[1][k] = E::pack(c0[8 + 2 * k], c0[8 + 2 * k + 1]);
            pk[2][k] = E::pack(c1[2 * k], c1[2 * k + 1]);
            pk[3][k] = E::pack(c1[8 + 2 * k], c1[8 + 2 * k + 1]);
        }

        // ---- block B: O^T += V^T P^T for tile t while the row sum is taken and tile t+2 is
        // rotated and staged. The A operand for lane (n, g) at step kc is V^T row (dim) n (or
        // 32 + n), slots 16kc + 8g .. +7 = keys 16kc + 4g + 0..3 and 16kc + 8 + 4g + 0..3.
        const uint16_t *v0 = vt[cur] + n * VS + 8 * g;
        const uint16_t *v1 = vt[cur] + (32 + n) * VS + 8 * g;
        u32x4 va[8];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            va[2 * kc] = *(const u32x4 *)(v0 + 16 * kc);
            va[2 * kc + 1] = *(const u32x4 *)(v1 + 16 * kc);
        }
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            o0 = E::mfma(va[2 * kc], pk[kc], o0);
            o1 = E::mfma(va[2 * kc + 1], pk[kc], o1);
        }
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            rs += c0[i] + c1[i];
        l_run += rs;
        if (t + 2 < ntiles)
            stage_store<E, NTHR>(st, sg, ks[fut], vt[fut]);
        if (t + 4 < ntiles)
            stage_load(st, sg, src, key(t + 4));

        // ---- masks (edge tiles only) and row maximum of tile t+1
        if (edge(j1))
            mask_scores(n0, n1, j1, len, back, ahead, qi, g);
        mx = row_max(n0, n1);
        __syncthreads();
    };

    int t = 0, cur = 0;
    for (; t + 1 < ntiles; t += 2) {
        step(sa0, sa1, sb0, sb1, ra, t, cur);
        cur = cur == RING - 1 ? 0 : cur + 1;
        step(sb0, sb1, sa0, sa1, rb, t + 1, cur);
        cur = cur == RING - 1 ? 0 : cur + 1;
    }
    if (t < ntiles)
        step(sa0, sa1, sb0, sb1, ra, t, cur);

    // ---- epilogue: out = O / l, lse = m + ln l, for rows inside the sequence
    const float l_tot = pair_sum(l_run);
    if (qi < len) {
        uint16_t *orow = out + (int64_t)(start + qi) * hd + h * D;
        store_out<E>(o0, o1, l_tot, orow, g);
        if (g == 0)
            lse[(int64_t)h * T + start + qi] = m_ref + logf(l_tot);
    }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Wait until at most N of this wave's tile copies are in flight and its LDS reads have returned,
// then the workgroup barrier. The empty asm statements keep the compiler from moving memory
// accesses across; no release fence is wanted here (one would wait for every copy in flight).
template <int N>
__device__ __forceinline__ void ring_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // vmcnt(N) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The forward over pre-rotated key tiles. Same arithmetic, order and outputs as attend_fwd;
// the key loop streams each 16 KB block straight into a four-slot LDS ring with buffer loads
// that write LDS (no registers, no ALU work): tile t+3 is requested at the start of step t into
// the slot tile t-1 left (every wave passed the barrier after its last read), and the end of
// step t waits for tile t+2, so each copy has two steps to land.
// At 64 rows (two waves) the compiler keeps part of the loop state in AGPRs and the kernel runs
// one wave per SIMD; the binding never takes the workspace path at that height (its key span
// is too short to repay the key tiles), so only an explicit request runs it.
template <class E, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 2 ? 1 : 2)))
attend_pre(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
           const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
           const uint32_t *__restrict__ tiles, const uint8_t *__restrict__ ws,
           uint16_t *__restrict__ out, float *__restrict__ lse, int32_t num_tiles, int32_t T,
           int32_t S, int32_t H, int32_t P, int32_t NB, int32_t back, int32_t ahead,
           float scale) {
    constexpr int BR = 32 * NW;
    constexpr int RING = 4;
    constexpr int PIECES = 16 / NW;  // 16-byte copies per thread per tile
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RING * BLK];

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
        return;

    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int w0 = i0 + 32 * __builtin_amdgcn_readfirstlane(wv);
    const int qi = w0 + n;

    int lo, hi;
    key_span(i0, BR, len, back, ahead, lo, hi);
    const int ntiles = (hi - lo + BC - 1) / BC;
    const int offset = (back < REACH_ALL || ahead < REACH_ALL)
                           ? 0
                           : (int)((int64_t)(i0 / BR) * ntiles / ((len + BR - 1) / BR));
    auto key = [&](int t) {
        int u = t + offset;
        if (u >= ntiles)
            u -= ntiles;
        return lo + u * BC;
    };

    // copies of tile t (t < ntiles) into ring slot sl: piece j of wave wv covers bytes
    // 1024 (NW j + wv) .. +1023 of the block, 16 per lane
    const uint8_t *wblock = ws + ((int64_t)h * NB + start / BC + (int)seq) * BLK;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int voff = 16 * lane;
    auto copy = [&](int t, int sl) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(wblock + (int64_t)(key(t) / BC) * BLK, BLK);
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const int off = 1024 * (NW * j + wvu);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)((lds_u8 *)ring + sl * BLK + off), 16, voff, off, 0, 0);
        }
    };

    // Every global read of the prologue is issued before the first wait: the query rows and
    // their table entries, the own key rows, the key norms and the copies of tiles 0 .. 2 (one
    // memory latency in all rather than one after another).
    QueryRaw qr;
    query_load(qr, qkv, cos_t, sin_t, ld, start, qi, len, h, g);
    u32x4 kw[4];
    own_key(wblock, qi, len, g, kw);
    // the blocks' key norm bounds: every score of tile t is at most qn * knorm[key(t) / BC]
    const float *knorm = (const float *)(ws + (int64_t)H * NB * BLK) + (int64_t)h * NB +
                         start / BC + (int)seq;
    float kn0, kn1;
    key_norm_reads(knorm, lo / BC, ntiles, lane, kn0, kn1);
    asm volatile("" ::: "memory");
    copy(0, 0);
    if (ntiles > 1)
        copy(1, 1);
    if (ntiles > 2)
        copy(2, 2);
    u32x4 qop[4];
    query_make<E>(qr, scale, qop);
    // upper bound of this row's rounded query norm (lanes n and n + 32 hold 32 elements each)
    float qn;
    {
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a0 = E::lo(qop[c][w]), a1 = E::hi(qop[c][w]);
                sq = __builtin_fmaf(a0, a0, sq);
                sq = __builtin_fmaf(a1, a1, sq);
            }
        qn = __builtin_sqrtf(pair_sum(sq)) * NORM_MARGIN;
    }
    // upper bound of every score of this row
    const float bq = qn * key_norm_max(knorm, lo / BC, ntiles, lane, kn0, kn1);
    const float s_own = own_dot<E>(kw, qop, qi, len);
    if (ntiles > 2)
        ring_barrier<PIECES>();
    else
        ring_barrier<0>();

    // byte offset of operand chunk 2kc + g of row n (and of row 32 + n, 4096 further on)
    int cof[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
        cof[kc] = n * 128 + 16 * ((2 * kc + g) ^ swz(n));

    auto edge = [&](int j0) {
        return tile_edge(w0, j0, len, back, ahead);
    };
    auto kscores = [&](int sl, f32x16 &s0, f32x16 &s1) {
        const uint8_t *kt = ring + sl * BLK;
        u32x4 a[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            a[2 * c] = *(const u32x4 *)(kt + cof[c]);
            a[2 * c + 1] = *(const u32x4 *)(kt + 4096 + cof[c]);
        }
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s0 = E::mfma(a[2 * c], qop[c], s0);
            s1 = E::mfma(a[2 * c + 1], qop[c], s1);
        }
    };

    float l_run = 0.f;
    f32x16 o0 = {}, o1 = {};
    f32x16 sa0, sa1, sb0, sb1;
    kscores(0, sa0, sa1);
    if (edge(key(0)))
        mask_scores(sa0, sa1, key(0), len, back, ahead, qi, g);
    const float m_ref =
        fixed_reference<E>(row_max(sa0, sa1), s_own, bq,
                           qi < len, [&] {
                               return exact_row_max<E>(wblock, qop, cof, ntiles, key, edge, len,
                                                       back, ahead, qi, g);
                           });
    const float mb = m_ref == -__builtin_inff() ? 0.f : m_ref * LOG2E;

    // Step t with tile t in slot cur (cur = t % 4, a constant after unrolling): the scores of
    // tile t+1 alongside the softmax and output product of tile t, the copy of tile t+3 and the
    // ring wait. With the reference fixed the body is one branch-free stretch.
    auto step = [&](f32x16 &c0, f32x16 &c1, f32x16 &n0, f32x16 &n1, int t, int cur) {
        const int nxt = (cur + 1) & 3;
        const bool more = t + 3 < ntiles;
        if (more)
            copy(t + 3, (cur + 3) & 3);
        const int j1 = key(t + 1);
        kscores(nxt, n0, n1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            c0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(c0[i], LOG2E, -mb));
            c1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(c1[i], LOG2E, -mb));
        }
        u32x4 pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pk[0][k] = E::pack(c0[2 * k], c0[2 * k + 1]);
            pk[1][k] = E::pack(c0[8 + 2 * k], c0[8 + 2 * k + 1]);
            pk[2][k] = E::pack(c1[2 * k], c1[2 * k + 1]);
            pk[3][k] = E::pack(c1[8 + 2 * k], c1[8 + 2 * k + 1]);
        }
        const uint8_t *vt = ring + cur * BLK + IMG;
        u32x4 va[8];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            va[2 * kc] = *(const u32x4 *)(vt + cof[kc]);
            va[2 * kc + 1] = *(const u32x4 *)(vt + 4096 + cof[kc]);
        }
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            o0 = E::mfma(va[2 * kc], pk[kc], o0);
            o1 = E::mfma(va[2 * kc + 1], pk[kc], o1);
        }
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            rs += c0[i] + c1[i];
        l_run += rs;
        // keep the sum in its step (the compiler would defer it and hold the probabilities)
        asm volatile("" : "+v"(l_run));
        // past the last tile the scores of "tile t+1" come from a stale slot: never used
        if (t + 1 < ntiles && edge(j1))
            mask_scores(n0, n1, j1, len, back, ahead, qi, g);
        if (more)
            ring_barrier<PIECES>();
        else
            ring_barrier<0>();
    };

    int t = 0;
    for (; t + 3 < ntiles; t += 4) {
        step(sa0, sa1, sb0, sb1, t, 0);
        step(sb0, sb1, sa0, sa1, t + 1, 1);
        step(sa0, sa1, sb0, sb1, t + 2, 2);
        step(sb0, sb1, sa0, sa1, t + 3, 3);
    }
    if (t < ntiles)
        step(sa0, sa1, sb0, sb1, t, 0);
    if (t + 1 < ntiles)
        step(sb0, sb1, sa0, sa1, t + 1, 1);
    if (t + 2 < ntiles)
        step(sa0, sa1, sb0, sb1, t + 2, 2);

    const float l_tot = pair_sum(l_run);
    if (qi < len) {
        uint16_t *orow = out + (int64_t)(start + qi) * hd + h * D;
        store_out<E>(o0, o1, l_tot, orow, g);
        if (g == 0)
            lse[(int64_t)h * T + start + qi] = m_ref + logf(l_tot);
    }
}

// Blocks of the key-tile workspace per head: floor(T / 64) + S.
int64_t tile_blocks(const AttendArgs &a) { return (int64_t)(a.T / BC) + a.S; }

template <class E>
int launch_rotate(const AttendArgs &a) {
    const int64_t NB = tile_blocks(a);
    const int64_t blocks = NB * ((a.H + PREP_HEADS - 1) / PREP_HEADS);
    if (blocks > INT32_MAX)
        return fail(VLF_EINVAL, "%lld workgroups exceed the grid limit", (long long)blocks);
    const uint16_t *qkv = (const uint16_t *)a.qkv;
    const uint16_t *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin;
    uint8_t *ws = (uint8_t *)a.workspace;
    int32_t nb32 = (int32_t)NB, T = a.T, S = a.S, H = a.H, P = a.table_rows;
    void *args[] = {(void *)&qkv, (void *)&cs, (void *)&sn, (void *)&a.cu, (void *)&ws,
                    (void *)&nb32, (void *)&T, (void *)&S,  (void *)&H,   (void *)&P};
    hipError_t e = hipLaunchKernel((const void *)prep_tiles<E>, dim3((unsigned)blocks),
                                   dim3(256), args, 0, (hipStream_t)a.stream);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "key tile launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}

// The workspace path at 256 rows in two wave groups half a step apart (waves 0-3 and 4-7, one
// of each on every SIMD): while one group runs a phase of matrix products (tile t's output
// product, tile t+1's scores) the other runs a softmax phase, so the vector instructions of one
// wave issue while the matrix unit works for the other (a wave's own products and vector work
// do not overlap). Four waves per SIMD (two workgroups per CU, 2 x 64 KB of LDS).
template <class E>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
attend_pre_ph(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
              const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
              const uint32_t *__restrict__ tiles, const uint8_t *__restrict__ ws,
              uint16_t *__restrict__ out, float *__restrict__ lse, int32_t num_tiles, int32_t T,
              int32_t S, int32_t H, int32_t P, int32_t NB, int32_t back, int32_t ahead,
              float scale) {
    constexpr int NW = 8;
    constexpr int BR = 32 * NW;
    constexpr int RING = 4;
    constexpr int PIECES = 16 / NW;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RING * BLK];

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
        return;
    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int w0 = i0 + 32 * __builtin_amdgcn_readfirstlane(wv);
    const int qi = w0 + n;
    int lo, hi;
    key_span(i0, BR, len, back, ahead, lo, hi);
    const int ntiles = (hi - lo + BC - 1) / BC;
    // every query tile sweeps its keys in order: the tiles of one (sequence, head) then read
    // the same blocks at about the same time, which keeps two such pairs per XCD within its L2
    // (the staggered start of attend_fwd measured 1% slower here)
    const int offset = 0;
    auto key = [&](int t) {
        int u = t + offset;
        if (u >= ntiles)
            u -= ntiles;
        return lo + u * BC;
    };
    const uint8_t *wblock = ws + ((int64_t)h * NB + start / BC + (int)seq) * BLK;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int voff = 16 * lane;
    auto copy = [&](int t, int sl) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(wblock + (int64_t)(key(t) / BC) * BLK, BLK);
#pragma unroll
        for (int j = 0; j < PIECES; ++j) {
            const int off = 1024 * (NW * j + wvu);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)((lds_u8 *)ring + sl * BLK + off), 16, voff, off, 0, 0);
        }
    };
    u32x4 qop[4];
    query_operand<E>(qkv, cos_t, sin_t, ld, start, qi, len, h, g, scale, qop);
    float qn;
    {
        float sq = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a0 = E::lo(qop[c][w]), a1 = E::hi(qop[c][w]);
                sq = __builtin_fmaf(a0, a0, sq);
                sq = __builtin_fmaf(a1, a1, sq);
            }
        qn = __builtin_sqrtf(pair_sum(sq)) * NORM_MARGIN;
    }
    const float *knorm = (const float *)(ws + (int64_t)H * NB * BLK) + (int64_t)h * NB +
                         start / BC + (int)seq;
    float kn0, kn1;
    key_norm_reads(knorm, lo / BC, ntiles, lane, kn0, kn1);
    asm volatile("" ::: "memory");
    // tiles 0 .. 2 in flight; tile 0 must land before step 0
    copy(0, 0);
    if (ntiles > 1)
        copy(1, 1);
    if (ntiles > 2)
        copy(2, 2);
    const float bq = qn * key_norm_max(knorm, lo / BC, ntiles, lane, kn0, kn1);
    if (ntiles > 2)
        ring_barrier<2 * PIECES>();
    else if (ntiles > 1)
        ring_barrier<PIECES>();
    else
        ring_barrier<0>();
    int cof[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
        cof[kc] = n * 128 + 16 * ((2 * kc + g) ^ swz(n));
    auto edge = [&](int j0) {
        return tile_edge(w0, j0, len, back, ahead);
    };
    // the two groups: waves 0-3 and 4-7 (one of each on every SIMD)
    const bool late = __builtin_amdgcn_readfirstlane(wv) >= 4;
    float m_ref = -__builtin_inff(), mb = 0.f;
    const float s_own = own_score<E>(wblock, qop, qi, len, g);
    float l_run = 0.f;
    f32x16 o0 = {}, o1 = {}, s0, s1;
    u32x4 pk[4];
    auto plain_barrier = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // scores of the key tile in slot sl into s0, s1
    auto scores = [&](int sl) __attribute__((always_inline)) {
        const uint8_t *kt = ring + sl * BLK;
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s0 = E::mfma(*(const u32x4 *)(kt + cof[c]), qop[c], s0);
            s1 = E::mfma(*(const u32x4 *)(kt + 4096 + cof[c]), qop[c], s1);
        }
    };
    // tile 0's scores and the reference
    auto first = [&]() __attribute__((always_inline)) {
        scores(0);
        if (edge(key(0)))
            mask_scores(s0, s1, key(0), len, back, ahead, qi, g);
        m_ref = fixed_reference<E>(row_max(s0, s1), s_own, bq, qi < len, [&] {
            return exact_row_max<E>(wblock, qop, cof, ntiles, key, edge, len, back, ahead, qi, g);
        });
        mb = m_ref == -__builtin_inff() ? 0.f : m_ref * LOG2E;
    };
    // softmax of tile t (scores in s0, s1; tile 0 was masked by first()): pk and the row sum
    auto softmax = [&](int t) __attribute__((always_inline)) {
        const int j0 = key(t);
        if (t > 0 && edge(j0))
            mask_scores(s0, s1, j0, len, back, ahead, qi, g);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], LOG2E, -mb));
            s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], LOG2E, -mb));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pk[0][k] = E::pack(s0[2 * k], s0[2 * k + 1]);
            pk[1][k] = E::pack(s0[8 + 2 * k], s0[8 + 2 * k + 1]);
            pk[2][k] = E::pack(s1[2 * k], s1[2 * k + 1]);
            pk[3][k] = E::pack(s1[8 + 2 * k], s1[8 + 2 * k + 1]);
        }
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            rs += s0[i] + s1[i];
        l_run += rs;
        // keep the sum in its phase (the compiler would defer it and hold the probabilities)
        asm volatile("" : "+v"(l_run));
    };
    // output product of tile t (pk, slot cur), then the scores of tile t+1 (next slot)
    // The products run at a raised wave priority: the arbiter then issues them ahead of the
    // other group's vector work and the matrix unit idles less (measured 2.5% faster).
    auto product = [&](int t, int cur) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        const uint8_t *vt = ring + cur * BLK + IMG;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            o0 = E::mfma(*(const u32x4 *)(vt + cof[kc]), pk[kc], o0);
            o1 = E::mfma(*(const u32x4 *)(vt + 4096 + cof[kc]), pk[kc], o1);
        }
        if (t + 1 < ntiles)
            scores((cur + 1) & 3);
        __builtin_amdgcn_s_setprio(0);
    };
    // end of phase 2t+1: tile t+2 has landed (tile t+3, copied at phase 2t, may be in flight)
    auto odd_end = [&](int t) __attribute__((always_inline)) {
        if (t + 3 < ntiles)
            ring_barrier<PIECES>();
        else
            ring_barrier<0>();
    };
    // Global phase 2t: the early group runs tile t's product (and tile t+1's scores), the late
    // group tile t's softmax; phase 2t+1: early softmax of t+1, late product of t. Every phase
    // ends at a barrier. Tile t+3 is copied at phase 2t into the slot of tile t-1, whose last
    // reads (the late group's product of t-1) ended with phase 2t-1; it is first read at phase
    // 2t+4 and waited for at the end of phase 2t+3.
    auto run = [&](auto late_group) __attribute__((always_inline)) {
        constexpr bool LATE = decltype(late_group)::value;
        auto phases = [&](int t, int cur) __attribute__((always_inline)) {
            if (t + 3 < ntiles)
                copy(t + 3, (cur + 3) & 3);
            if constexpr (LATE)
                softmax(t);
            else
                product(t, cur);
            plain_barrier();
            if constexpr (LATE) {
                product(t, cur);
            } else {
                if (t + 1 < ntiles)
                    softmax(t + 1);
            }
            odd_end(t);
        };
        // phases -2 and -1
        if constexpr (LATE) {
            plain_barrier();
            first();
        } else {
            first();
            plain_barrier();
            softmax(0);
        }
        odd_end(-1);
        int t = 0;
        for (; t + 3 < ntiles; t += 4) {
            phases(t, 0);
            phases(t + 1, 1);
            phases(t + 2, 2);
            phases(t + 3, 3);
        }
        if (t < ntiles)
            phases(t, 0);
        if (t + 1 < ntiles)
            phases(t + 1, 1);
        if (t + 2 < ntiles)
            phases(t + 2, 2);
    };
    if (late)
        run(LateGroup<true>{});
    else
        run(LateGroup<false>{});
    const float l_tot = pair_sum(l_run);
    if (qi < len) {
        uint16_t *orow = out + (int64_t)(start + qi) * hd + h * D;
        store_out<E>(o0, o1, l_tot, orow, g);
        if (g == 0)
            lse[(int64_t)h * T + start + qi] = m_ref + logf(l_tot);
    }
}

template <class E, int NW>
int launch_pre(const AttendArgs &a) {
    const int64_t blocks = (int64_t)a.num_tiles * a.H;
    if (blocks > INT32_MAX || tile_blocks(a) * a.H > INT32_MAX)
        return fail(VLF_EINVAL, "%lld workgroups exceed the grid limit", (long long)blocks);
    const uint16_t *qkv = (const uint16_t *)a.qkv;
    const uint16_t *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin;
    const uint8_t *ws = (const uint8_t *)a.workspace;
    uint16_t *out = (uint16_t *)a.out;
    int32_t nb32 = (int32_t)tile_blocks(a), num_tiles = a.num_tiles, T = a.T, S = a.S, H = a.H;
    int32_t P = a.table_rows, Bk = a.back, Ah = a.ahead;
    float scale = a.scale;
    void *args[] = {(void *)&qkv, (void *)&cs,  (void *)&sn,    (void *)&a.cu,
                    (void *)&a.tiles, (void *)&ws, (void *)&out, (void *)&a.lse,
                    (void *)&num_tiles, (void *)&T, (void *)&S,   (void *)&H,
                    (void *)&P,   (void *)&nb32, (void *)&Bk,  (void *)&Ah, (void *)&scale};
    const void *fn;
    if constexpr (NW == 8)
        fn = (const void *)attend_pre_ph<E>;
    else
        fn = (const void *)attend_pre<E, NW>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(NW * 64), args, 0,
                                   (hipStream_t)a.stream);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "attend launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}

// Query tiles of 64 rows (two waves) with a single key-tile slot: each key tile is loaded,
// rotated, staged and consumed in turn, without attend_fwd's software pipeline. Registers and
// LDS (18 KB) stay small, so many workgroups share a CU, which is what batches of short
// sequences need: most of their tiles see one key tile and are bound by load latency, not by
// the matrix unit. Same arithmetic as attend_fwd, tile by tile.
// SINGLE serves batches of sequences of at most 64 tokens, where every query tile reaches one
// key tile: without a second tile to load ahead, the kernel fits 128 registers, so four waves
// share a SIMD and eight workgroups a CU. A tile that reaches more keys (a sequence longer than
// the caller's max_len said) is left unwritten.
template <class E, bool FIXED, bool SINGLE>
__global__ void __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(SINGLE ? 4 : 2)))
attend_one(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
           const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
           const uint32_t *__restrict__ tiles, uint16_t *__restrict__ out,
           float *__restrict__ lse, int32_t num_tiles, int32_t T, int32_t S, int32_t H, int32_t P,
           int32_t back, int32_t ahead, float scale) {
    constexpr int BR = 64;
    constexpr int NTHR = 128;
    __shared__ __attribute__((aligned(16))) uint16_t ks[BC * KS];
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

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
        return;

    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int w0 = i0 + 32 * __builtin_amdgcn_readfirstlane(wv);
    const int qi = w0 + n;

    int lo, hi;
    key_span(i0, BR, len, back, ahead, lo, hi);
    const int ntiles = (hi - lo + BC - 1) / BC;
    if (SINGLE && ntiles > 1)
        return;

    Staging<NTHR> sg;
    sg.init(tid, ld);
    Sources<FIXED> src;
    src.init(qkv + (int64_t)start * ld + hd + h * D, qkv + (int64_t)start * ld + 2 * hd + h * D,
             cos_t, sin_t, len, P, ld);
    TileRegs<NTHR> r;
    stage_load(r, sg, src, lo);
    // a wave whose rows all lie past the sequence (half the waves of a batch of short
    // sequences) only stages and waits
    const bool idle = __builtin_amdgcn_readfirstlane(w0) >= len;
    u32x4 qop[4];
    if (!idle)
        query_operand<E>(qkv, cos_t, sin_t, ld, start, qi, len, h, g, scale, qop);

    float m_ref = -__builtin_inff();
    float l_run = 0.f;
    f32x16 o0 = {}, o1 = {};
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = lo + t * BC;
        if (t > 0) {
            stage_load(r, sg, src, j0);
            __syncthreads();  // every wave is done with the previous tile
        }
        // wave v stages key rows 32v .. 32v+31 of the tile; past the sequence they are never
        // read (the second half of such a tile is skipped below)
        stage_store<E, NTHR>(r, sg, ks, vt, __builtin_amdgcn_readfirstlane(j0 + 32 * wv) < len);
        __syncthreads();
        if (idle)
            continue;
        // keys j0 + 32 .. j0 + 63 all past the sequence (a sequence of at most 32 tokens): that
        // half's products, probabilities and sums are skipped, its scores are -inf
        const bool h1 = j0 + 32 < len;
        f32x16 s0, s1;
        if (h1) {
            scores<E>(ks, qop, n, g, s0, s1);
        } else {
            const uint16_t *k0 = ks + n * KS + 8 * g;
            s0 = f32x16{};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                s0 = E::mfma(*(const u32x4 *)(k0 + 16 * c), qop[c], s0);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                s1[i] = -__builtin_inff();
        }
        if (tile_edge(w0, j0, len, back, ahead))
            mask_scores(s0, s1, j0, len, back, ahead, qi, g);
        const float mx = row_max(s0, s1);
        const bool raise = mx > m_ref + TAU;
        const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mx) * LOG2E) : 1.0f;
        m_ref = raise ? mx : m_ref;
        l_run *= alpha;
        if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                o0[i] *= alpha;
                o1[i] *= alpha;
            }
        }
        const float mb = m_ref == -__builtin_inff() ? 0.f : m_ref * LOG2E;
        u32x4 pk[4];
        const uint16_t *v0 = vt + n * VS + 8 * g;
        const uint16_t *v1 = vt + (32 + n) * VS + 8 * g;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], LOG2E, -mb));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pk[0][k] = E::pack(s0[2 * k], s0[2 * k + 1]);
            pk[1][k] = E::pack(s0[8 + 2 * k], s0[8 + 2 * k + 1]);
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            o0 = E::mfma(*(const u32x4 *)(v0 + 16 * kc), pk[kc], o0);
            o1 = E::mfma(*(const u32x4 *)(v1 + 16 * kc), pk[kc], o1);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            rs += s0[i];
        if (h1) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], LOG2E, -mb));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                pk[2][k] = E::pack(s1[2 * k], s1[2 * k + 1]);
                pk[3][k] = E::pack(s1[8 + 2 * k], s1[8 + 2 * k + 1]);
            }
#pragma unroll
            for (int kc = 2; kc < 4; ++kc) {
                o0 = E::mfma(*(const u32x4 *)(v0 + 16 * kc), pk[kc], o0);
                o1 = E::mfma(*(const u32x4 *)(v1 + 16 * kc), pk[kc], o1);
            }
            float r1 = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                r1 += s1[i];
            rs += r1;
        }
        l_run += rs;
    }

    const float l_tot = pair_sum(l_run);
    if (qi < len) {
        uint16_t *orow = out + (int64_t)(start + qi) * hd + h * D;
        store_out<E>(o0, o1, l_tot, orow, g);
        if (g == 0)
            lse[(int64_t)h * T + start + qi] = m_ref + logf(l_tot);
    }
}

// ---- windows that fit in LDS: query tiles walked in table order, keys kept between them -------
// With a window of at most 129 keys, the keys that a 256-row query tile reaches span at most
// eight 64-key tiles, and the next query tile of the same sequence shares all but four of them.
// attend_slide serves 256-row tiles whose reached keys span at most eight key tiles: a window of
// at most 129 keys (causal: 257), or any window over sequences of at most 512 tokens, whose
// whole key range then fits the ring.
// attend_slide runs one 8-wave workgroup per CU over a contiguous run of the (head, tile) items:
// an 8-slot LDS ring holds the current item's key tiles (key tile u of the sequence in slot
// u % 8, as block images), each new key tile is rotated and staged once per run instead of once
// per query tile that reads it, and the next item's new key tiles and query rows are loaded into
// registers while the current item computes. Each wave sweeps only the key tiles its own 32 rows
// reach. The arithmetic per key tile is that of attend_one.

// A thread's share of staging one key tile, by role (t = tid % 256):
//   keys:   key row t / 4, dims 8 (t % 4) .. +7 and 32 + 8 (t % 4) .. +7, and their table entries;
//   values: keys 2 (t / 8) and 2 (t / 8) + 1, dims 8 (t % 8) .. +7.
// Eight consecutive lanes read one 128-byte row (keys: two 64-byte halves).
struct SlideKeys {
    u32x4 x1, x2, c, s;
};
struct SlideVals {
    u32x4 va, vb;
};

// Where the current item's key and value rows come from. With FIXED (every sequence, and the
// tables, within 2^31 bytes of their first row), one descriptor per item covers its sequence
// and a tile's byte offset is added to the lane offsets; otherwise descriptors are rebased on
// each tile. Either way they end at the sequence (table) end, so rows past it read as zero.
template <bool FIXED>
struct SlideSrc {
    const uint16_t *kbase, *vbase, *cos_t, *sin_t;
    int64_t ld;
    int len, P, row_bytes;
    int koff, toff, voff;                   // this thread's byte offsets inside a tile
    __amdgpu_buffer_rsrc_t kr, vr, cr, sr;  // FIXED only

    __device__ void set(const uint16_t *k, const uint16_t *v, int len_) {
        kbase = k, vbase = v, len = len_;
        if (FIXED) {
            kr = rsrc(kbase, (int64_t)len * row_bytes);
            vr = rsrc(vbase, (int64_t)len * row_bytes);
        }
    }
};

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Loads of the key tile at j0 (< len).
template <bool FIXED>
__device__ __forceinline__ void slide_load_keys(SlideKeys &r, const SlideSrc<FIXED> &q, int j0) {
    __amdgpu_buffer_rsrc_t kr, cr, sr;
    int kd = 0, td = 0;
    if (FIXED) {
        kr = q.kr, cr = q.cr, sr = q.sr;
        kd = j0 * q.row_bytes;
        td = j0 * 64;
    } else {
        kr = rsrc(q.kbase + (int64_t)j0 * q.ld, (int64_t)(q.len - j0) * q.row_bytes);
        cr = rsrc(q.cos_t + (int64_t)j0 * 32, (int64_t)(q.P - j0) * 64);
        sr = rsrc(q.sin_t + (int64_t)j0 * 32, (int64_t)(q.P - j0) * 64);
    }
    r.x1 = load16(kr, q.koff + kd);
    r.x2 = load16(kr, q.koff + kd + 64);
    r.c = load16(cr, q.toff + td);
    r.s = load16(sr, q.toff + td);
}
template <bool FIXED>
__device__ __forceinline__ void slide_load_vals(SlideVals &r, const SlideSrc<FIXED> &q, int j0) {
    __amdgpu_buffer_rsrc_t vr;
    int vd = 0;
    if (FIXED) {
        vr = q.vr;
        vd = j0 * q.row_bytes;
    } else {
        vr = rsrc(q.vbase + (int64_t)j0 * q.ld, (int64_t)(q.len - j0) * q.row_bytes);
    }
    r.va = load16(vr, q.voff + vd);
    r.vb = load16(vr, q.voff + vd + q.row_bytes);
}

// Rotates and rounds the keys into the block image at blk (the layout prep_tiles writes).
template <class E>
__device__ __forceinline__ void slide_store_keys(const SlideKeys &r, uint8_t *blk, int t) {
    const int kr = t >> 2, q = t & 3;
    uint32_t a[4], b[4], c[4], s[4], y1[4], y2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        a[k] = r.x1[k], b[k] = r.x2[k], c[k] = r.c[k], s[k] = r.s[k];
    rotate<E, 4>(a, b, c, s, 1.0f, y1, y2);
    *(u32x4 *)(blk + kr * 128 + 16 * (q ^ swz(kr))) = u32x4{y1[0], y1[1], y1[2], y1[3]};
    *(u32x4 *)(blk + kr * 128 + 16 * ((4 + q) ^ swz(kr))) = u32x4{y2[0], y2[1], y2[2], y2[3]};
}

// Transposes the values into the V^T image: row d, slot p holds key vt_slot(p); keys 2kp and
// 2kp + 1 sit in slots p and p + 1, one 32-bit word per dim.
__device__ __forceinline__ void slide_store_vals(const SlideVals &r, uint8_t *blk, int t) {
    const int kp = t >> 3, c = t & 7;
    const int p = vt_slot(2 * kp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * c + e;
        const uint32_t wa = r.va[e >> 1], wb = r.vb[e >> 1];
        const uint32_t lo = (e & 1) ? (wa >> 16) : (wa & 0xffffu);
        const uint32_t hi = (e & 1) ? (wb & 0xffff0000u) : (wb << 16);
        *(uint32_t *)(blk + IMG + d * 128 + 16 * ((p >> 3) ^ swz(d)) + 2 * (p & 7)) = lo | hi;
    }
}

// Sequences attend_slide ranks itself for its snake order (larger batches take equal runs of
// the table's order).
constexpr int SNAKE_SEQ = 256;

// One (head, query tile) item of attend_slide, with the key tiles [ta, tb) its window reaches.
struct SlideItem {
    int h, seq, i0, start, len, ta, tb;
    bool ok;
};

template <class E, bool FIXED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
attend_slide(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
             const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
             const uint32_t *__restrict__ tiles, uint16_t *__restrict__ out,
             float *__restrict__ lse, int32_t num_tiles, int32_t T, int32_t S, int32_t H,
             int32_t P, int32_t back, int32_t ahead, float scale, int32_t snake) {
    constexpr int NW = 8;
    constexpr int BR = 32 * NW;
    constexpr int RING = 8;   // key tiles held in LDS
    constexpr int DESC = 64;  // items described in LDS at a time
    __shared__ __attribute__((aligned(1024))) uint8_t ring[RING * BLK];
    __shared__ int32_t desc[DESC][8];  // seq (-1: skip), i0, start, len, h, ta, tb
    __shared__ int32_t plist[DESC];    // snake order: seq << 24 | tile << 16 | h
    __shared__ int32_t cost[SNAKE_SEQ], ranked[SNAKE_SEQ];
    __shared__ int32_t plist_n;

    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int tid = (int)threadIdx.x;
    int ua, ub;
    if (snake && S <= SNAKE_SEQ) {
        // Snake order: the sequences ranked by cost (tiles x key tiles they reach, most first,
        // ties by index), run r = (rank floor(r / H), head r mod H) of all their tiles goes to
        // workgroup r mod G, in rounds of G that alternate direction. The table's order is not
        // used: the runs cover the tiles of every sequence cu describes, which is the set of
        // the table's entries.
        for (int x = tid; x < S; x += NW * 64) {
            const int start = cu[x], len = cu[x + 1] - start;
            int c = -1;
            if (len > 0 && len <= P && start >= 0 && (int64_t)start + len <= T) {
                c = 0;
                for (int i0 = 0; i0 < len; i0 += BR) {
                    int lo, hi;
                    key_span(i0, BR, len, back, ahead, lo, hi);
                    c += 2 + (hi - lo + BC - 1) / BC;
                }
            }
            cost[x] = c;
        }
        __syncthreads();
        for (int x = tid; x < S; x += NW * 64) {
            const int c = cost[x];
            if (c >= 0) {
                int rank = 0;
                for (int y = 0; y < S; ++y) {
                    const int cy = cost[y];
                    rank += cy > c || (cy == c && y < x);
                }
                ranked[rank] = x;
            }
        }
        __syncthreads();
        if (tid == 0) {
            int sn = 0;
            for (int y = 0; y < S; ++y)
                sn += cost[y] >= 0;
            const int runs = sn * H;
            int np = 0;
            for (int j = 0; j * G < runs; ++j) {
                const int r = j * G + ((j & 1) ? G - 1 - b : b);
                if (r >= runs)
                    continue;
                const int x = ranked[r / H], h = r - (r / H) * H;
                const int len = cu[x + 1] - cu[x];
                // (the host sizes the list for every run; the bound only guards it)
                for (int tile = 0; tile * BR < len && np < DESC; ++tile)
                    plist[np++] =
                        (int32_t)(((uint32_t)x << 24) | ((uint32_t)tile << 16) | (uint32_t)h);
            }
            plist_n = np;
        }
        __syncthreads();
        ua = 0;
        ub = plist_n;
    } else {
        // this workgroup's run of items u = h * num_tiles + tile (the host keeps the count
        // below 2^31)
        snake = 0;
        const int items = num_tiles * H;
        ua = (int)((int64_t)items * b / G);
        ub = (int)((int64_t)items * (b + 1) / G);
    }
    if (ua >= ub)
        return;

    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int t = tid & 255, gp = __builtin_amdgcn_readfirstlane(wv) >> 2;
    int cof[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
        cof[kc] = n * 128 + 16 * ((2 * kc + g) ^ swz(n));

    // ---- item descriptors, DESC at a time (one lane each)
    int base = ua;
    auto fill = [&](int from) {
        if (tid < DESC) {
            int32_t e[8] = {-1, 0, 0, 0, 0, 0, 0, 0};
            const int u = from + tid;
            if (u < ub) {
                int h;
                uint32_t seq;
                int i0;
                if (snake) {
                    const int pe = plist[u];
                    seq = (uint32_t)pe >> 24;
                    i0 = ((pe >> 16) & 255) * BR;
                    h = pe & 0xffff;
                } else {
                    h = u / num_tiles;
                    const int tile = u - h * num_tiles;
                    seq = tiles[2 * tile];
                    i0 = (int)tiles[2 * tile + 1];
                }
                if (seq < (uint32_t)S) {
                    const int start = cu[seq];
                    const int len = cu[seq + 1] - start;
                    int lo, hi;
                    key_span(i0, BR, len, back, ahead, lo, hi);
                    // a tile that does not match cu, or reaches more key tiles than the ring
                    // holds (the host admits no such window), reads and writes nothing
                    if (i0 >= 0 && i0 < len && len <= P && start >= 0 &&
                        (int64_t)start + len <= T && (hi + BC - 1) / BC - lo / BC <= RING) {
                        e[0] = (int)seq, e[1] = i0, e[2] = start, e[3] = len;
                        e[5] = lo / BC, e[6] = (hi + BC - 1) / BC;
                    }
                }
                e[4] = h;
            }
            *(u32x4 *)&desc[tid][0] = u32x4{(uint32_t)e[0], (uint32_t)e[1], (uint32_t)e[2],
                                            (uint32_t)e[3]};
            *(u32x4 *)&desc[tid][4] = u32x4{(uint32_t)e[4], (uint32_t)e[5], (uint32_t)e[6], 0u};
        }
        base = from;
    };
    auto decode = [&](int u, SlideItem &it) {
        const int k = u - base;
        it.seq = __builtin_amdgcn_readfirstlane(desc[k][0]);
        it.i0 = __builtin_amdgcn_readfirstlane(desc[k][1]);
        it.start = __builtin_amdgcn_readfirstlane(desc[k][2]);
        it.len = __builtin_amdgcn_readfirstlane(desc[k][3]);
        it.h = __builtin_amdgcn_readfirstlane(desc[k][4]);
        it.ta = __builtin_amdgcn_readfirstlane(desc[k][5]);
        it.tb = __builtin_amdgcn_readfirstlane(desc[k][6]);
        it.ok = it.seq >= 0;
    };

    // The ring holds key tiles [ra, rb) of (rseq, rh). An item keeps them when it belongs to
    // the same (sequence, head) and its range starts inside them; its new tiles are then
    // [max(rb, ta), tb), all within eight consecutive tiles, so no kept tile shares a slot
    // with a new one.
    int rseq = -1, rh = -1, ra = 0, rb = 0;
    auto keeps = [&](const SlideItem &it) {
        return it.seq == rseq && it.h == rh && it.ta >= ra && it.ta <= rb;
    };
    auto fresh = [&](const SlideItem &it, int &na, int &nb) {
        na = nb = 0;
        if (!it.ok)
            return;
        na = keeps(it) ? max(rb, it.ta) : it.ta;
        nb = max(na, it.tb);
    };
    auto advance = [&](const SlideItem &it) {
        if (!it.ok)
            return;  // nothing was staged or read
        rb = keeps(it) ? max(it.tb, rb) : it.tb;
        ra = it.ta;
        rseq = it.seq;
        rh = it.h;
    };

    SlideSrc<FIXED> src;
    src.cos_t = cos_t;
    src.sin_t = sin_t;
    src.ld = ld;
    src.P = P;
    src.row_bytes = (int)(ld * 2);
    if (FIXED) {
        src.cr = rsrc(cos_t, (int64_t)P * 64);
        src.sr = rsrc(sin_t, (int64_t)P * 64);
    }
    src.koff = (t >> 2) * src.row_bytes + 16 * (t & 3);
    src.toff = (t >> 2) * 64 + 16 * (t & 3);
    src.voff = 2 * (t >> 3) * src.row_bytes + 16 * (t & 7);
    auto set_src = [&](const SlideItem &it) {
        const uint16_t *k = qkv + (int64_t)it.start * ld + hd + it.h * D;
        src.set(k, k + hd, it.len);
    };

    // New tiles travel in pairs (x, x + 1): waves 0-3 take the keys of x and the values of
    // x + 1, waves 4-7 the other way round, so each thread holds one of each per pair.
    SlideKeys kk[2];
    SlideVals vv[2];
    QueryRaw qr;
    auto load_pair = [&](SlideKeys &k, SlideVals &v, int x, int nb) {
        const int tk = x + gp, tv = x + 1 - gp;
        if (tk < nb)
            slide_load_keys(k, src, tk * BC);
        if (tv < nb)
            slide_load_vals(v, src, tv * BC);
    };
    auto store_pair = [&](const SlideKeys &k, const SlideVals &v, int x, int nb) {
        const int tk = x + gp, tv = x + 1 - gp;
        if (tk < nb)
            slide_store_keys<E>(k, ring + (tk & (RING - 1)) * BLK, t);
        if (tv < nb)
            slide_store_vals(v, ring + (tv & (RING - 1)) * BLK, t);
    };
    // the loads of an item's first four new key tiles and of its query rows, in three parts
    // (the key-tile pairs, then the query rows): the vector memory path moves about 64 bytes per
    // clock per CU, so the item's 160 KB are issued a part per key tile of the computation
    // rather than at once
    auto prefetch = [&](int part, const SlideItem &it, int na, int nb) {
        if (part < 2) {
            if (it.ok)
                load_pair(kk[part], vv[part], na + 2 * part, nb);
        } else {
            // (an item that reads nothing loads zero rows)
            query_load(qr, qkv, cos_t, sin_t, ld, it.start, it.ok ? it.i0 + 32 * wv + n : 0,
                       it.ok ? it.len : 0, it.h, g);
        }
    };

    fill(ua);
    __syncthreads();
    SlideItem cur, nxt, nn;
    int na, nb;
    decode(ua, cur);
    nxt.ok = false;
    if (ua + 1 < ub)
        decode(ua + 1, nxt);
    fresh(cur, na, nb);
    if (cur.ok)
        set_src(cur);
#pragma unroll
    for (int part = 0; part < 3; ++part)
        prefetch(part, cur, na, nb);

    for (int u = ua; u < ub; ++u) {
        // ---- stage the item's new key tiles (every wave is done with the previous item)
        __syncthreads();
        if (cur.ok) {
            store_pair(kk[0], vv[0], na, nb);
            store_pair(kk[1], vv[1], na + 2, nb);
            // a cold ring (first item of a run or of a sequence) needs more than four
            for (int x = na + 4; x < nb; x += 4) {
                load_pair(kk[0], vv[0], x, nb);
                load_pair(kk[1], vv[1], x + 2, nb);
                store_pair(kk[0], vv[0], x, nb);
                store_pair(kk[1], vv[1], x + 2, nb);
            }
        }
        advance(cur);
        u32x4 qop[4];
        query_make<E>(qr, scale, qop);
        // the next item's loads (into the registers just consumed) are issued during this
        // item's key loop, one part per key tile
        int na2 = 0, nb2 = 0;
        const bool more = u + 1 < ub;
        if (more) {
            fresh(nxt, na2, nb2);
            if (nxt.ok)
                set_src(nxt);
        }
        auto issue = [&](int part) __attribute__((always_inline)) {
            if (more)
                prefetch(part, nxt, na2, nb2);
        };
        int issued = 0;
        // descriptors of the items after the next (all reads of the old ones are done)
        if (u + 2 < ub && u + 2 >= base + DESC)
            fill(u + 2);
        __syncthreads();
        nn.ok = false;
        if (u + 2 < ub)
            decode(u + 2, nn);

        // ---- this wave's 32 rows against the key tiles they reach
        const int w0 = cur.i0 + 32 * __builtin_amdgcn_readfirstlane(wv);
        if (cur.ok && w0 < cur.len) {
            const int len = cur.len;
            const int qi = w0 + n;
            int lo, hi;
            key_span(w0, 32, len, back, ahead, lo, hi);
            // this row's visible keys: jlo <= j < jhi
            int jlo, jhi;
            row_keys(qi, len, back, ahead, jlo, jhi);
            const int nt = (hi - lo + BC - 1) / BC;
            issued = min(nt, 3);
            float m_ref = -__builtin_inff();
            float l_run = 0.f;
            f32x16 o0 = {}, o1 = {};
            auto step = [&](int tt) __attribute__((always_inline)) {
                const int j0 = lo + tt * BC;
                const uint8_t *kt = ring + ((j0 / BC) & (RING - 1)) * BLK;
                f32x16 s0 = {}, s1 = {};
                // Every operand read of a product goes out before its first MFMA (the
                // scheduling barrier keeps them there): left to itself the compiler issued
                // each read right before its MFMA and waited for it.
                u32x4 op0[4], op1[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    op0[c] = *(const u32x4 *)(kt + cof[c]);
                    op1[c] = *(const u32x4 *)(kt + 4096 + cof[c]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    s0 = E::mfma(op0[c], qop[c], s0);
                    s1 = E::mfma(op1[c], qop[c], s1);
                }
                if (tile_edge(w0, j0, len, back, ahead))
                    mask_band(s0, s1, jlo, jhi, j0, g);
                const float mx = row_max(s0, s1);
                const bool raise = mx > m_ref + TAU;
                const float alpha = raise ? __builtin_amdgcn_exp2f((m_ref - mx) * LOG2E) : 1.0f;
                m_ref = raise ? mx : m_ref;
                l_run *= alpha;
                if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        o0[i] *= alpha;
                        o1[i] *= alpha;
                    }
                }
                const float mb = m_ref == -__builtin_inff() ? 0.f : m_ref * LOG2E;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], LOG2E, -mb));
                    s1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], LOG2E, -mb));
                }
                u32x4 pk[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    pk[0][k] = E::pack(s0[2 * k], s0[2 * k + 1]);
                    pk[1][k] = E::pack(s0[8 + 2 * k], s0[8 + 2 * k + 1]);
                    pk[2][k] = E::pack(s1[2 * k], s1[2 * k + 1]);
                    pk[3][k] = E::pack(s1[8 + 2 * k], s1[8 + 2 * k + 1]);
                }
                // the row sum before the output product, so the probabilities are dead by the
                // time its operands arrive
                float rs = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    rs += s0[i] + s1[i];
                l_run += rs;
                const uint8_t *vt = kt + IMG;
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    op0[kc] = *(const u32x4 *)(vt + cof[kc]);
                    op1[kc] = *(const u32x4 *)(vt + 4096 + cof[kc]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    o0 = E::mfma(op0[kc], pk[kc], o0);
                    o1 = E::mfma(op1[kc], pk[kc], o1);
                }
            };
            // the first three key tiles, each after issuing a part of the next item's loads
            if (nt > 0) {
                issue(0);
                step(0);
            }
            if (nt > 1) {
                issue(1);
                step(1);
            }
            if (nt > 2) {
                issue(2);
                step(2);
            }
            for (int tt = 3; tt < nt; ++tt)
                step(tt);
            const float l_tot = pair_sum(l_run);
            if (qi < len) {
                uint16_t *orow = out + (int64_t)(cur.start + qi) * hd + cur.h * D;
                store_out<E>(o0, o1, l_tot, orow, g);
                if (g == 0)
                    lse[(int64_t)cur.h * T + cur.start + qi] = m_ref + logf(l_tot);
            }
        }
        // (waves that swept fewer than three key tiles)
        if (issued < 1)
            issue(0);
        if (issued < 2)
            issue(1);
        if (issued < 3)
            issue(2);
        cur = nxt;
        nxt = nn;
        na = na2;
        nb = nb2;
    }
}

template <class E, int NW, bool FIXED>
int launch_typed(const AttendArgs &a) {
    const int64_t blocks = (int64_t)a.num_tiles * a.H;
    if (blocks > INT32_MAX)
        return fail(VLF_EINVAL, "%lld workgroups exceed the grid limit", (long long)blocks);
    const uint16_t *qkv = (const uint16_t *)a.qkv;
    const uint16_t *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin;
    uint16_t *out = (uint16_t *)a.out;
    int32_t num_tiles = a.num_tiles, T = a.T, S = a.S, H = a.H, P = a.table_rows;
    int32_t Bk = a.back, Ah = a.ahead;
    float scale = a.scale;
    void *args[] = {(void *)&qkv, (void *)&cs,        (void *)&sn, (void *)&a.cu,
                    (void *)&a.tiles, (void *)&out,   (void *)&a.lse, (void *)&num_tiles,
                    (void *)&T,   (void *)&S,         (void *)&H,  (void *)&P,
                    (void *)&Bk,  (void *)&Ah, (void *)&scale};
    // 64-row tiles take the unpipelined kernel (short sequences; the single-tile form when no
    // sequence is longer than one key tile), taller ones the pipeline
    const void *fn;
    if constexpr (NW == 2)
        fn = a.max_len <= BC ? (const void *)attend_one<E, FIXED, true>
                             : (const void *)attend_one<E, FIXED, false>;
    else
        fn = (const void *)attend_fwd<E, NW, FIXED>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(NW * 64), args, 0,
                                   (hipStream_t)a.stream);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "attend launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}

template <class E, bool FIXED>
int launch_slide(const AttendArgs &a) {
    const int64_t items = (int64_t)a.num_tiles * a.H;
    if (items > INT32_MAX)
        return fail(VLF_EINVAL, "%lld items exceed the grid limit", (long long)items);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus < 1)
        return fail(VLF_EHIP, "device query failed: %s", hipGetErrorString(e));
    // one workgroup per CU (the 128 KB ring admits no second one)
    const int64_t grid = items < cus ? items : cus;
    // Snake order where there are at least two runs of whole (sequence, head) pairs per
    // workgroup and the sequences are few enough for each workgroup to rank them: a run per
    // workgroup and round evens out the load far better than equal counts of consecutive
    // entries. Each workgroup's list holds at most ceil(S H / grid) runs of at most
    // ceil(P / 256) tiles (a longer sequence is skipped, as the tables do not reach it).
    const int64_t runs = (int64_t)a.S * a.H;
    const int64_t per = (runs + grid - 1) / grid, tiles_per = ((int64_t)a.table_rows + 255) / 256;
    int32_t snake = a.S <= SNAKE_SEQ && runs >= 2 * grid && per * tiles_per <= 64;
    const uint16_t *qkv = (const uint16_t *)a.qkv;
    const uint16_t *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin;
    uint16_t *out = (uint16_t *)a.out;
    int32_t num_tiles = a.num_tiles, T = a.T, S = a.S, H = a.H, P = a.table_rows;
    int32_t Bk = a.back, Ah = a.ahead;
    float scale = a.scale;
    void *args[] = {(void *)&qkv, (void *)&cs,        (void *)&sn, (void *)&a.cu,
                    (void *)&a.tiles, (void *)&out,   (void *)&a.lse, (void *)&num_tiles,
                    (void *)&T,   (void *)&S,         (void *)&H,  (void *)&P,
                    (void *)&Bk,  (void *)&Ah, (void *)&scale, (void *)&snake};
    e = hipLaunchKernel((const void *)attend_slide<E, FIXED>, dim3((unsigned)grid), dim3(512),
                        args, 0, (hipStream_t)a.stream);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "attend launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}

template <class E>
int launch_pre_br(const AttendArgs &a) {
    switch (a.br) {  // the host side admits 64, 128 and 256 only
    case 64: return launch_pre<E, 2>(a);
    case 128: return launch_pre<E, 4>(a);
    case 256: return launch_pre<E, 8>(a);
    default: return fail(VLF_EUNSUPPORTED, "br = %d", a.br);
    }
}

template <class E, bool FIXED>
int launch_br(const AttendArgs &a) {
    switch (a.br) {  // the host side admits 64, 128 and 256 only
    case 64: return launch_typed<E, 2, FIXED>(a);
    case 128: return launch_typed<E, 4, FIXED>(a);
    case 256: return launch_typed<E, 8, FIXED>(a);
    default: return fail(VLF_EUNSUPPORTED, "br = %d", a.br);
    }
}


// ---- backward: the gradient of sum(out * dout) with respect to qkv ---------------------------
// hanzo-kernel 0.2.42 src/packed.rs, `delta`, `attend_back` and `rotate_back`: P is recomputed
// from the forward's lse and dS = P (dP - delta) with delta = rowsum(dO * O). The page sums dK
// and dV per key tile and adds dQ into float32 with atomics; here dQ has a pass of its own, over
// query tiles, that recomputes S and dP (two more products) and writes dQ once, rotated back and
// scaled: no atomics, and the same dqkv bits on every run.
//
// back_prep writes, per row and head, -delta and -lse (float32, natural log; the passes apply
// log2(e) where they form P). On tiles taller than 64 rows (128 or 256) it also writes, once per
// 64-row tile and head, the operand images both passes stage from: Q~ rows, Q~^T, dO^T, K~ rows
// and K~^T (rotated, scaled and rounded as the forward rounds them); back_kv and back_q then fill
// LDS with plain 16-byte copies (buffer loads straight into LDS), dO and V rows coming from their
// tensors the same way. On 64-row tiles the passes load, rotate and store each step's operands
// themselves and no image is written. Every kernel walks the tile table of the call's tile
// height (64, 128 or 256 rows).

constexpr int BIMG = 5 * IMG;  // one tile's images: Q~, Q~^T, dO^T (24 KB), K~, K~^T (16 KB)
constexpr int BS = 64;         // streamed rows per step of back_kv and back_q

// Byte offset of the images in the workspace: -delta and -lse, float32 [H, T] each, then
// padding to 256 bytes.
__host__ __device__ __forceinline__ int64_t back_img_offset(int32_t T, int32_t H) {
    return ((int64_t)8 * T * H + 255) / 256 * 256;
}

// XCD-aware work index of the block (block b runs on XCD b % 8).
__device__ __forceinline__ int xcd_work() {
    const int nb = (int)gridDim.x, b = (int)blockIdx.x;
    const int xcd = b % XCDS, slot = b / XCDS;
    const int per = nb / XCDS, extra = nb % XCDS;
    return xcd * per + min(xcd, extra) + slot;
}

// The (sequence, first row) of a table entry, or false for an entry that names no tile.
__device__ __forceinline__ bool back_tile(const uint32_t *tiles, const int32_t *cu, int tile,
                                          int32_t S, int32_t T, int32_t P, int &seq, int &start,
                                          int &len, int &i0) {
    const uint32_t s = tiles[2 * tile];
    i0 = (int)tiles[2 * tile + 1];
    if (s >= (uint32_t)S)
        return false;
    seq = (int)s;
    start = cu[s];
    len = cu[s + 1] - start;
    return !(i0 < 0 || i0 >= len || len > P || start < 0 || (int64_t)start + len > T);
}

// Element (d, slot) of a transposed image: 128-byte rows, 16-byte chunk c at c ^ swz(d).
__device__ __forceinline__ int tr_at(int d, int slot) {
    return d * 128 + 16 * ((slot >> 3) ^ swz(d)) + 2 * (slot & 7);
}

// Dims 8c4 .. 8c4+7 (w1) and 32+8c4 .. (w2) of row `row` into the transposed image t at slot
// vt_slot(row): the order in which a score accumulator holds a 16-row group.
__device__ __forceinline__ void stage_transposed(const uint32_t (&w1)[4], const uint32_t (&w2)[4],
                                                 uint8_t *t, int row, int c4) {
    const int slot = vt_slot(row);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int d1 = 8 * c4 + 2 * w + e;
            const int sh = e ? 16 : 0;
            *(uint16_t *)(t + tr_at(d1, slot)) = (uint16_t)(w1[w] >> sh);
            *(uint16_t *)(t + tr_at(d1 + 32, slot)) = (uint16_t)(w2[w] >> sh);
        }
}

// The same dims of row `row`, rotated by (c, s), times `scale`, rounded to E: into the row image
// xs (chunk c at c ^ swz(row)) and the transposed image xt.
template <class E>
__device__ __forceinline__ void stage_rotated(const u32x4 &x1, const u32x4 &x2, const u32x4 &c,
                                              const u32x4 &s, float scale, uint8_t *xs,
                                              uint8_t *xt, int row, int c4) {
    const uint32_t a_[4] = {x1[0], x1[1], x1[2], x1[3]};
    const uint32_t b_[4] = {x2[0], x2[1], x2[2], x2[3]};
    const uint32_t c_[4] = {c[0], c[1], c[2], c[3]};
    const uint32_t s_[4] = {s[0], s[1], s[2], s[3]};
    uint32_t p1[4], p2[4];
    rotate<E, 4>(a_, b_, c_, s_, scale, p1, p2);
    const int sw = swz(row);
    *(u32x4 *)(xs + row * 128 + 16 * (c4 ^ sw)) = u32x4{p1[0], p1[1], p1[2], p1[3]};
    *(u32x4 *)(xs + row * 128 + 16 * ((4 + c4) ^ sw)) = u32x4{p2[0], p2[1], p2[2], p2[3]};
    stage_transposed(p1, p2, xt, row, c4);
}

// 16-byte chunks of row i of a [*, ld] tensor at column col: dims 8c4 .. and 32 + 8c4 ..
// (zeros past the sequence).
__device__ __forceinline__ void load_halves(const uint16_t *base, int64_t ld, int start, int i,
                                            int len, int c4, u32x4 &a, u32x4 &b) {
    const u32x4 z = {0, 0, 0, 0};
    u32x4 x = z, y = z;
    if (i < len) {
        const uint16_t *r = base + (int64_t)(start + i) * ld + 8 * c4;
        x = *(const u32x4 *)r;
        y = *(const u32x4 *)(r + 32);
    }
    a = x, b = y;
}

// The rotation table entries of position i for dims 8c4 .. 8c4+7 (zeros past the sequence).
__device__ __forceinline__ void load_table_row(const uint16_t *cos_t, const uint16_t *sin_t, int i,
                                               int len, int c4, u32x4 &c, u32x4 &s) {
    const u32x4 z = {0, 0, 0, 0};
    u32x4 cv = z, sv = z;
    if (i < len) {
        cv = *(const u32x4 *)(cos_t + (int64_t)i * 32 + 8 * c4);
        sv = *(const u32x4 *)(sin_t + (int64_t)i * 32 + 8 * c4);
    }
    c = cv, s = sv;
}

// The operand images of the 64-row tiles of one table entry (R rows) and head, with -delta and
// -lse of their rows. Built in LDS (four lanes per row, 16 dims each) and copied out in 16-byte
// pieces. Rows past the sequence are zero in every image. Without IMAGES only the two per-row
// floats are written (the passes then stage their operands themselves).
template <class E, int R, bool IMAGES>
__global__ void __launch_bounds__(256)
back_prep(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
          const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
          const uint32_t *__restrict__ tiles, const uint16_t *__restrict__ out,
          const uint16_t *__restrict__ dout, const float *__restrict__ lse,
          uint8_t *__restrict__ ws, int32_t num_tiles, int32_t T, int32_t S, int32_t H,
          int32_t P, float scale) {
    __shared__ __attribute__((aligned(16))) uint8_t im[IMAGES ? BIMG : 16];
    const int work = xcd_work();
    const int h = work / num_tiles;
    int seq, start, len, i0;
    if (!back_tile(tiles, cu, work - h * num_tiles, S, T, P, seq, start, len, i0))
        return;
    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int row = tid >> 2, c4 = tid & 3;
    float *ndelta = (float *)ws + (int64_t)h * T, *nlse = (float *)ws + (int64_t)(H + h) * T;
    const int64_t nb = T / BC + S;
    uint8_t *blocks = ws + back_img_offset(T, H) + ((int64_t)h * nb + start / BC + seq) * BIMG;
#pragma unroll 1
    for (int t = i0; t < i0 + R && t < len; t += BC) {
        const int i = t + row;
        u32x4 o1, o2, y1, y2;
        load_halves(dout + h * D, hd, start, i, len, c4, y1, y2);
        load_halves(out + h * D, hd, start, i, len, c4, o1, o2);
        if constexpr (IMAGES) {
            u32x4 q1, q2, k1, k2, c, s;
            load_halves(qkv + h * D, ld, start, i, len, c4, q1, q2);
            load_halves(qkv + hd + h * D, ld, start, i, len, c4, k1, k2);
            load_table_row(cos_t, sin_t, i, len, c4, c, s);
            stage_rotated<E>(q1, q2, c, s, scale, im, im + IMG, row, c4);
            const uint32_t w1[4] = {y1[0], y1[1], y1[2], y1[3]};
            const uint32_t w2[4] = {y2[0], y2[1], y2[2], y2[3]};
            stage_transposed(w1, w2, im + 2 * IMG, row, c4);
            stage_rotated<E>(k1, k2, c, s, 1.0f, im + 3 * IMG, im + 4 * IMG, row, c4);
        }
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            acc = __builtin_fmaf(E::lo(o1[k]), E::lo(y1[k]), acc);
            acc = __builtin_fmaf(E::hi(o1[k]), E::hi(y1[k]), acc);
            acc = __builtin_fmaf(E::lo(o2[k]), E::lo(y2[k]), acc);
            acc = __builtin_fmaf(E::hi(o2[k]), E::hi(y2[k]), acc);
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        if (i < len && c4 == 0) {
            ndelta[start + i] = -acc;
            nlse[start + i] = -lse[(int64_t)h * T + start + i];
        }
        if constexpr (IMAGES) {
            __syncthreads();
            uint8_t *blk = blocks + (int64_t)(t / BC) * BIMG;
#pragma unroll
            for (int j = 0; j < BIMG / 4096; ++j)
                *(u32x4 *)(blk + 4096 * j + 16 * tid) =
                    *(const u32x4 *)(im + 4096 * j + 16 * tid);
            __syncthreads();
        }
    }
}

// dims 16c + 8g .. 16c+8g+7 of row i of a tensor (zeros past the sequence)
__device__ __forceinline__ void back_row_operand(const uint16_t *base, int64_t ld, int start,
                                                 int i, int len, int g, u32x4 (&op)[4]) {
    const u32x4 z = {0, 0, 0, 0};
    u32x4 v0 = z, v1 = z, v2 = z, v3 = z;
    if (i < len) {
        const uint16_t *r = base + (int64_t)(start + i) * ld + 8 * g;
        v0 = *(const u32x4 *)r;
        v1 = *(const u32x4 *)(r + 16);
        v2 = *(const u32x4 *)(r + 32);
        v3 = *(const u32x4 *)(r + 48);
    }
    op[0] = v0, op[1] = v1, op[2] = v2, op[3] = v3;
}

// The rows a row sees through the window (empty for a row past the sequence): the keys
// [lo, hi) of query x (x - back <= j <= x + ahead), or the queries [lo, hi) that see key x
// (x - ahead <= i <= x + back: pass the reaches swapped).
__device__ __forceinline__ void back_visible(int x, int len, int back, int ahead, int &lo,
                                             int &hi) {
    lo = 0, hi = 0;
    if (x < len)
        row_keys(x, len, back, ahead, lo, hi);
}

// The streamed rows a tile [t0, t0 + rows) reaches: [a, b), a a multiple of BS. For a key tile
// (the queries that see it) pass the reaches swapped.
__device__ __forceinline__ void back_span(int t0, int rows, int len, int back, int ahead, int &a,
                                          int &b) {
    a = t0 > back ? (t0 - back) / BS * BS : 0;
    b = (int64_t)t0 + rows + ahead < len ? t0 + rows + ahead : len;
}

// True when every pair of the 32-row query block [q0, q0+32) and key block [k0, k0+32) of one
// sequence is visible: no masking needed.
__device__ __forceinline__ bool back_full(int q0, int k0, int len, int back, int ahead) {
    return q0 + 32 <= len && k0 + 32 <= len && q0 + 31 - k0 <= back && k0 + 31 - q0 <= ahead;
}

// The steps [fa, fb) of a sweep whose 64 streamed rows (it = a + 64 st, two 32-row blocks) and
// the 32-row block at b0 are visible in every pair, for a sweep of `steps` steps: an interval of
// st, since each condition of back_full bounds it on one side. Streamed rows are queries when
// Q is true (back_kv: b0 is the wave's key block), keys otherwise (back_q: b0 its query block).
// The bounds are taken in 64 bits (a reach may be INT32_MAX) and then checked with back_full
// itself, so a step outside [fa, fb) is only ever masked when it need not be.
template <bool Q>
__device__ __forceinline__ void full_steps(int a, int steps, int b0, int len, int back, int ahead,
                                           int &fa, int &fb) {
    // streamed block x and fixed block b0: x + 32 <= len, b0 + 32 <= len, and the offset
    // x - b0 (queries minus keys) within [-ahead + 31, back - 31] when Q, swapped otherwise
    auto full = [&](int st) {
        const int x = a + BS * st;
        return Q ? back_full(x, b0, len, back, ahead) && back_full(x + 32, b0, len, back, ahead)
                 : back_full(b0, x, len, back, ahead) && back_full(b0, x + 32, len, back, ahead);
    };
    const int64_t hi_q = Q ? (int64_t)b0 + back - 63 : (int64_t)b0 + ahead - 63;
    const int64_t lo_q = Q ? (int64_t)b0 + 31 - ahead : (int64_t)b0 + 31 - back;
    const int64_t top = min((int64_t)len - 64, hi_q);  // largest streamed start that fits
    int64_t lo = lo_q - a <= 0 ? 0 : (lo_q - a + BS - 1) / BS;
    int64_t hi = top - a < 0 ? 0 : (top - a) / BS + 1;
    if (b0 + 32 > len)
        hi = 0;
    lo = min(lo, (int64_t)steps);
    hi = min(hi, (int64_t)steps);
    int f0 = (int)lo, f1 = (int)max(lo, hi);
    while (f0 < f1 && !full(f0))
        ++f0;
    while (f1 > f0 && !full(f1 - 1))
        --f1;
    if (f0 >= f1)
        f0 = f1 = steps;
    fa = f0, fb = f1;
}

// Buffer resource over rows [r0, len) of a [*, ld] tensor from column col: rows past the
// sequence read as zeros. Offsets stay below 64 rows, so 32 bits hold them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t back_rows(const uint16_t *base, int64_t ld,
                                                            int start, int r0, int len) {
    // (wave-uniform: the arithmetic then stays on the scalar unit)
    const int row = __builtin_amdgcn_readfirstlane(start + r0);
    const int rows = __builtin_amdgcn_readfirstlane(len - r0);
    const int64_t bytes = (int64_t)(rows - 1) * ld * 2 + 128;
    return rsrc(base + (int64_t)row * ld, bytes);
}

// Copies 64 rows of a [*, ld] tensor (128 bytes each from the resource's column) into a row
// image (chunk c of row r at c ^ swz(r)): piece p = 8 rows = 1 KB, 16 bytes per lane.
template <int NW>
__device__ __forceinline__ void copy_rows(__amdgpu_buffer_rsrc_t r, int64_t ld, lds_u8 *dst,
                                          int wvu, int lane) {
#pragma unroll
    for (int j = 0; j < 8 / NW; ++j) {
        const int p = NW * j + wvu;
        const int row = 8 * p + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + 1024 * p), 16,
                                                 (int)(row * ld * 2 + 16 * chunk), 0, 0, 0);
    }
}

// Copies `bytes` (a multiple of 1 KB) of a workspace block into LDS, 1 KB pieces by wave.
template <int NW, int BYTES>
__device__ __forceinline__ void copy_block(const uint8_t *src, lds_u8 *dst, int wvu, int lane) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, BYTES);
#pragma unroll
    for (int j = 0; j < BYTES / 1024 / NW; ++j) {
        const int off = 1024 * (NW * j + wvu);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + off), 16, 16 * lane, off,
                                                 0, 0);
    }
}

// 64 floats of rows [r0, r0 + 64) of a per-row float array into LDS (zeros past the sequence;
// a range that starts past it reads nothing and leaves zeros).
__device__ __forceinline__ void copy_floats(const float *base, int start, int r0, int len,
                                            lds_u8 *dst, int lane) {
    const int rows = len > r0 ? len - r0 : 0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + start + (rows > 0 ? r0 : 0), 4 * rows);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 4, 4 * lane, 0, 0, 0);
}

// Compile-time choice of the masked or the unmasked step.
template <bool B>
struct Masked {
    static constexpr bool value = B;
};

// P = exp(S - lse) and dS = P (dP - delta) of a 32 x 32 accumulator block whose register i holds
// row 8(i/4) + 4g + i%4 (sc holds S - lse and dp holds dP - delta: the products started from
// -lse and -delta), packed to E as the B operands of the next products. With MASK, only rows r
// with r - a in [0, span) count (a is relative to register 0 of the lane's group).
template <class E, bool MASK>
__device__ __forceinline__ void back_pds(f32x16 &sc, f32x16 &dp, int a, uint32_t span,
                                         u32x4 (&pp)[2], u32x4 (&pd)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(sc[i] * LOG2E);
        if (MASK)
            p = (uint32_t)(8 * (i >> 2) + (i & 3) - a) < span ? p : 0.f;
        sc[i] = p;
        dp[i] = p * dp[i];
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pp[kc][k] = E::pack(sc[8 * kc + 2 * k], sc[8 * kc + 2 * k + 1]);
            pd[kc][k] = E::pack(dp[8 * kc + 2 * k], dp[8 * kc + 2 * k + 1]);
        }
}

// The same for a transposed block (one row per lane), dS only.
template <class E, bool MASK>
__device__ __forceinline__ void back_ds(const f32x16 &st, f32x16 &dp, int a, uint32_t span,
                                        u32x4 (&pd)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(st[i] * LOG2E);
        if (MASK)
            p = (uint32_t)(8 * (i >> 2) + (i & 3) - a) < span ? p : 0.f;
        dp[i] = p * dp[i];
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            pd[kc][k] = E::pack(dp[8 * kc + 2 * k], dp[8 * kc + 2 * k + 1]);
}

// dK and dV of one key tile (32 NW keys) of one head over every query row its window reaches,
// 64 rows a step (FlashAttention-2's backward without dQ). Wave w owns keys 32w .. 32w+31 of
// the tile and keeps their rotated keys K~ and values V in registers as the B operands of
// S = Q~ K~^T and dP = dO V^T, whose accumulators hold one key per lane and 16 query rows per
// 32-row block. A step's Q~, Q~^T and dO^T images come from back_prep and its dO rows from dout,
// straight into one of two LDS slots while the other slot's step is computed; P and dS go from
// the accumulators into the B operands of dV^T += dO^T P and dK^T += Q~^T dS.
// SL slots of 33 KB: copies run SL - 1 steps ahead. Eight waves take two a SIMD and the CU's
// LDS for four slots; four take two a SIMD with two workgroups of two slots a CU; two take one.
template <class E, int NW, int SL, bool DIRECT>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 2 ? 1 : 2)))
back_kv(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
        const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
        const uint32_t *__restrict__ tiles, const uint16_t *__restrict__ dout,
        const uint8_t *__restrict__ ws, uint16_t *__restrict__ dqkv, int32_t num_tiles,
        int32_t T, int32_t S, int32_t H, int32_t P, int32_t back, int32_t ahead, float scale) {
    // Q~, Q~^T, dO^T, dO rows, then -lse and -delta of the step's 64 rows and of the next 64
    constexpr int SLOT = 4 * IMG + 1024;
    // buffer loads a wave issues per copy (waves 0 and 1 issue one more)
    constexpr int PIECES = 3 * IMG / 1024 / NW + 8 / NW;
    __shared__ __attribute__((aligned(16))) uint8_t lds[SL * SLOT];

    const int work = xcd_work();
    const int h = work / num_tiles;
    int seq, start, len, j0;
    if (!back_tile(tiles, cu, work - h * num_tiles, S, T, P, seq, start, len, j0))
        return;
    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int n = lane & 31, g = lane >> 5;
    const int kw0 = j0 + 32 * wvu;  // the wave's first key
    const int kj = kw0 + n;         // this lane's key
    const bool idle = kw0 >= len;   // the wave's keys all lie past the sequence: copies only

    // the lane's key (rotated and rounded as the forward rounds it) and value, dims 16c + 8g ..
    u32x4 kop[4], vop[4];
    {
        QueryRaw r;
        query_load(r, qkv + hd, cos_t, sin_t, ld, start, kj, len, h, g);
        query_make<E>(r, 1.0f, kop);
    }
    back_row_operand(qkv + 2 * hd + h * D, ld, start, kj, len, g, vop);

    int qa, qb, vlo, vhi;
    back_span(j0, 32 * NW, len, ahead, back, qa, qb);  // the queries that see the tile's keys
    back_visible(kj, len, ahead, back, vlo, vhi);
    const uint32_t span = (uint32_t)(vhi - vlo);

    const float *nlse = (const float *)ws + (int64_t)(H + h) * T;
    const float *ndelta = (const float *)ws + (int64_t)h * T;
    const uint8_t *imgs =
        ws + back_img_offset(T, H) + ((int64_t)h * (T / BC + S) + start / BC + seq) * BIMG;
    lds_u8 *const base = (lds_u8 *)lds;
    auto copy = [&](int it, int sl) {
        if constexpr (DIRECT) {
            // the step's rows loaded, rotated and stored here: four lanes a row
            uint8_t *dg = lds + sl * SLOT;
            const int c4 = tid & 3;
            for (int r = tid >> 2; r < BS; r += 16 * NW) {
                const int i = it + r;
                u32x4 q1, q2, y1, y2, c, s;
                load_halves(qkv + h * D, ld, start, i, len, c4, q1, q2);
                load_halves(dout + h * D, hd, start, i, len, c4, y1, y2);
                load_table_row(cos_t, sin_t, i, len, c4, c, s);
                stage_rotated<E>(q1, q2, c, s, scale, dg, dg + IMG, r, c4);
                const uint32_t w1[4] = {y1[0], y1[1], y1[2], y1[3]};
                const uint32_t w2[4] = {y2[0], y2[1], y2[2], y2[3]};
                stage_transposed(w1, w2, dg + 2 * IMG, r, c4);
                *(u32x4 *)(dg + 3 * IMG + r * 128 + 16 * (c4 ^ swz(r))) = y1;
                *(u32x4 *)(dg + 3 * IMG + r * 128 + 16 * ((4 + c4) ^ swz(r))) = y2;
                if (c4 == 0) {
                    float *fl = (float *)(dg + 4 * IMG);
                    fl[r] = i < len ? nlse[start + i] : 0.f;
                    fl[64 + r] = i + BS < len ? nlse[start + i + BS] : 0.f;
                    fl[128 + r] = i < len ? ndelta[start + i] : 0.f;
                    fl[192 + r] = i + BS < len ? ndelta[start + i + BS] : 0.f;
                }
            }
            return;
        }
        lds_u8 *d = base + sl * SLOT;
        copy_block<NW, 3 * IMG>(imgs + (int64_t)(it / BC) * BIMG, d, wvu, lane);
        copy_rows<NW>(back_rows(dout + h * D, hd, start, it, len), hd, d + 3 * IMG, wvu, lane);
        // the step's -lse and -delta, and the next step's (read at the end of this step)
        if (wvu == 0) {
            copy_floats(nlse, start, it, len, d + 4 * IMG, lane);
            copy_floats(nlse, start, it + BS, len, d + 4 * IMG + 256, lane);
        }
        if (wvu == 1) {
            copy_floats(ndelta, start, it, len, d + 4 * IMG + 512, lane);
            copy_floats(ndelta, start, it + BS, len, d + 4 * IMG + 768, lane);
        }
    };
    const int steps = (qb - qa + BS - 1) / BS;
    for (int k = 0; k < SL - 1 && k < steps; ++k)
        copy(qa + k * BS, k);
    if (steps >= SL - 1)
        ring_barrier<PIECES * (SL - 2)>();
    else
        ring_barrier<0>();

    f32x16 dv0 = {}, dv1 = {}, dk0 = {}, dk1 = {};
    // S - lse and dP - delta of 32-row block rb of a step, register i holding query row
    // 32rb + 8(i/4) + 4g + i%4: the accumulators start at -lse and -delta. A step's values are
    // read from the LDS slot of the step before (its second half) as soon as that step's block
    // rb has formed its P and dS, so that they have landed when the block's first products of
    // the next step need them.
    f32x16 sc[2], dp[2];
    auto start_values = [&](const float *nl, const float *nd, int rb) __attribute__((always_inline)) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const f32x4 x = *(const f32x4 *)(nl + 32 * rb + 8 * gi + 4 * g);
            const f32x4 y = *(const f32x4 *)(nd + 32 * rb + 8 * gi + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sc[rb][4 * gi + e] = x[e], dp[rb][4 * gi + e] = y[e];
        }
    };
    if (!idle && steps > 0) {
        const float *nl = (const float *)(lds + 4 * IMG);
        start_values(nl, nl + 128, 0);
        start_values(nl, nl + 128, 1);
    }
    // One step: the copy SL - 1 steps ahead, the products of step st (unless the wave is idle),
    // the ring wait. The masked and unmasked steps run in loops of their own (below): with both
    // bodies behind a branch in one loop the compiler gives the accumulators different
    // registers in the two and copies all of them at the join, every step.
    auto step = [&](int st, auto masked) __attribute__((always_inline)) {
        const int it = qa + st * BS;
        const bool more = st + SL - 1 < steps;
        if (more)
            copy(it + (SL - 1) * BS, (st + SL - 1) % SL);
        if (!idle) {
            const uint8_t *qs = lds + (st % SL) * SLOT, *qt = qs + IMG, *ot = qs + 2 * IMG;
            const uint8_t *os = qs + 3 * IMG;
            // the next step's -lse and -delta (second halves of this slot's float arrays)
            const float *nl = (const float *)(qs + 4 * IMG) + BS, *nd = nl + 128;
            // both 32-row blocks in one stretch, so that the softmax of one overlaps the
            // products of the other
            {
                constexpr bool MASK = decltype(masked)::value;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int off = (32 * rb + n) * 128 + 16 * ((2 * c + g) ^ swz(n));
                        sc[rb] = E::mfma(*(const u32x4 *)(qs + off), kop[c], sc[rb]);
                        dp[rb] = E::mfma(*(const u32x4 *)(os + off), vop[c], dp[rb]);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    u32x4 pp[2], pd[2];
                    back_pds<E, MASK>(sc[rb], dp[rb], vlo - it - 32 * rb - 4 * g, span, pp, pd);
                    start_values(nl, nd, rb);
                    // dV^T += dO^T P and dK^T += Q~^T dS (dims 0..31 and 32..63)
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        const int ch = 4 * rb + 2 * kc + g;
                        const int f0 = n * 128 + 16 * (ch ^ swz(n));
                        const int f1 = (32 + n) * 128 + 16 * (ch ^ swz(32 + n));
                        dv0 = E::mfma(*(const u32x4 *)(ot + f0), pp[kc], dv0);
                        dv1 = E::mfma(*(const u32x4 *)(ot + f1), pp[kc], dv1);
                        dk0 = E::mfma(*(const u32x4 *)(qt + f0), pd[kc], dk0);
                        dk1 = E::mfma(*(const u32x4 *)(qt + f1), pd[kc], dk1);
                    }
                }
            }
        }
        // the next step's copies have landed (later steps' may still be in flight)
        if (more)
            ring_barrier<PIECES * (SL - 2)>();
        else
            ring_barrier<0>();
    };
    // steps [fa, fb) see every pair of the wave's keys and skip the mask
    int fa, fb;
    full_steps<true>(qa, steps, kw0, len, back, ahead, fa, fb);
    for (int st = 0; st < fa; ++st)
        step(st, Masked<true>{});
    for (int st = fa; st < fb; ++st)
        step(st, Masked<false>{});
    for (int st = fb; st < steps; ++st)
        step(st, Masked<true>{});

    // dK rotated back to the key's position, and dV; register i of block b holds dim
    // 32b + 8(i/4) + 4g + i%4 of key kj
    if (kj < len) {
        const uint16_t *cr = cos_t + (int64_t)kj * 32, *sr = sin_t + (int64_t)kj * 32;
        uint16_t *o = dqkv + (int64_t)(start + kj) * ld + h * D;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int m0 = 8 * gi + 4 * g;
            const u32x2 cw = *(const u32x2 *)(cr + m0), sw = *(const u32x2 *)(sr + m0);
            float a[4], bb[4], v0[4], v1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float cm = (e & 1) ? E::hi(cw[e >> 1]) : E::lo(cw[e >> 1]);
                const float sm = (e & 1) ? E::hi(sw[e >> 1]) : E::lo(sw[e >> 1]);
                const float x1 = dk0[4 * gi + e], x2 = dk1[4 * gi + e];
                a[e] = x1 * cm + x2 * sm;
                bb[e] = x2 * cm - x1 * sm;
                v0[e] = dv0[4 * gi + e];
                v1[e] = dv1[4 * gi + e];
            }
            asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
            asm volatile("" : "+v"(bb[0]), "+v"(bb[1]), "+v"(bb[2]), "+v"(bb[3]));
            *(u32x2 *)(o + hd + m0) = u32x2{E::pack(a[0], a[1]), E::pack(a[2], a[3])};
            *(u32x2 *)(o + hd + 32 + m0) = u32x2{E::pack(bb[0], bb[1]), E::pack(bb[2], bb[3])};
            *(u32x2 *)(o + 2 * hd + m0) = u32x2{E::pack(v0[0], v0[1]), E::pack(v0[2], v0[3])};
            *(u32x2 *)(o + 2 * hd + 32 + m0) =
                u32x2{E::pack(v1[0], v1[1]), E::pack(v1[2], v1[3])};
        }
    }
}

// dQ of one query tile (32 NW rows) of one head over every key its window reaches, 64 keys a
// step. Wave w owns query rows 32w .. 32w+31 and keeps Q~ and dO in registers as the B operands
// of S^T = K~ Q~^T and dP^T = V dO^T, whose accumulators hold one query per lane (so lse and
// delta are one value per lane) and 16 keys per 32-key block. A step's K~ and K~^T images come
// from back_prep and its V rows from qkv, straight into one of two LDS slots; dS^T goes from the
// accumulators into the B operand of dQ^T += K~^T dS^T. dQ is rotated back to the row's
// position, scaled and written once.
template <class E, int NW, int SL, bool DIRECT>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
back_q(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
       const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
       const uint32_t *__restrict__ tiles, const uint16_t *__restrict__ dout,
       const uint8_t *__restrict__ ws, uint16_t *__restrict__ dqkv, int32_t num_tiles,
       int32_t T, int32_t S, int32_t H, int32_t P, int32_t back, int32_t ahead, float scale) {
    constexpr int SLOT = 3 * IMG;  // K~, K~^T, V rows
    constexpr int PIECES = 2 * IMG / 1024 / NW + 8 / NW;  // buffer loads a wave issues per copy
    __shared__ __attribute__((aligned(16))) uint8_t lds[SL * SLOT];

    const int work = xcd_work();
    const int h = work / num_tiles;
    int seq, start, len, i0;
    if (!back_tile(tiles, cu, work - h * num_tiles, S, T, P, seq, start, len, i0))
        return;
    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int n = lane & 31, g = lane >> 5;
    const int qw0 = i0 + 32 * wvu;  // the wave's first query row
    const int qi = qw0 + n;         // this lane's query row
    const bool idle = qw0 >= len;

    // the lane's rotated, scaled query (as the forward rounds it) and its dO, dims 16c + 8g ..
    u32x4 qop[4], oop[4];
    {
        QueryRaw r;
        query_load(r, qkv, cos_t, sin_t, ld, start, qi, len, h, g);
        query_make<E>(r, scale, qop);
    }
    back_row_operand(dout + h * D, hd, start, qi, len, g, oop);
    float nl = 0.f, nd = 0.f;  // -lse and -delta of the lane's row
    if (qi < len) {
        nl = ((const float *)ws)[(int64_t)(H + h) * T + start + qi];
        nd = ((const float *)ws)[(int64_t)h * T + start + qi];
    }
    f32x16 nlv, ndv;  // where the S^T and dP^T blocks start: -lse and -delta in every register
#pragma unroll
    for (int i = 0; i < 16; ++i)
        nlv[i] = nl, ndv[i] = nd;

    int ka, kb, klo, khi;
    back_span(i0, 32 * NW, len, back, ahead, ka, kb);
    back_visible(qi, len, back, ahead, klo, khi);
    const uint32_t span = (uint32_t)(khi - klo);

    const uint8_t *imgs = ws + back_img_offset(T, H) +
                          ((int64_t)h * (T / BC + S) + start / BC + seq) * BIMG + 3 * IMG;
    lds_u8 *const base = (lds_u8 *)lds;
    auto copy = [&](int jt, int sl) {
        if constexpr (DIRECT) {
            uint8_t *dg = lds + sl * SLOT;
            const int c4 = tid & 3;
            for (int r = tid >> 2; r < BS; r += 16 * NW) {
                const int i = jt + r;
                u32x4 k1, k2, v1, v2, c, s;
                load_halves(qkv + hd + h * D, ld, start, i, len, c4, k1, k2);
                load_halves(qkv + 2 * hd + h * D, ld, start, i, len, c4, v1, v2);
                load_table_row(cos_t, sin_t, i, len, c4, c, s);
                stage_rotated<E>(k1, k2, c, s, 1.0f, dg, dg + IMG, r, c4);
                *(u32x4 *)(dg + 2 * IMG + r * 128 + 16 * (c4 ^ swz(r))) = v1;
                *(u32x4 *)(dg + 2 * IMG + r * 128 + 16 * ((4 + c4) ^ swz(r))) = v2;
            }
            return;
        }
        lds_u8 *d = base + sl * SLOT;
        copy_block<NW, 2 * IMG>(imgs + (int64_t)(jt / BC) * BIMG, d, wvu, lane);
        copy_rows<NW>(back_rows(qkv + 2 * hd + h * D, ld, start, jt, len), ld, d + 2 * IMG, wvu,
                      lane);
    };
    const int steps = (kb - ka + BS - 1) / BS;
    for (int k = 0; k < SL - 1 && k < steps; ++k)
        copy(ka + k * BS, k);
    if (steps >= SL - 1)
        ring_barrier<PIECES * (SL - 2)>();
    else
        ring_barrier<0>();

    f32x16 dq0 = {}, dq1 = {};
    // One step (see back_kv: masked and unmasked steps run in loops of their own)
    auto step = [&](int st_i, auto masked) __attribute__((always_inline)) {
        const int jt = ka + st_i * BS;
        const bool more = st_i + SL - 1 < steps;
        if (more)
            copy(jt + (SL - 1) * BS, (st_i + SL - 1) % SL);
        if (!idle) {
            const uint8_t *ks = lds + (st_i % SL) * SLOT, *kt = ks + IMG, *vs = ks + 2 * IMG;
            {
                constexpr bool MASK = decltype(masked)::value;
                f32x16 st[2], dp[2];
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) {
                    // S^T - lse and dP^T - delta of keys jt + 32kb2 + 8(i/4) + 4g + i%4: the
                    // first products add to -lse and -delta (nlv and ndv stay as they are)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int off = (32 * kb2 + n) * 128 + 16 * ((2 * c + g) ^ swz(n));
                        st[kb2] = E::mfma(*(const u32x4 *)(ks + off), qop[c],
                                          c == 0 ? nlv : st[kb2]);
                        dp[kb2] = E::mfma(*(const u32x4 *)(vs + off), oop[c],
                                          c == 0 ? ndv : dp[kb2]);
                    }
                }
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) {
                    u32x4 pd[2];
                    back_ds<E, MASK>(st[kb2], dp[kb2], klo - jt - 32 * kb2 - 4 * g, span, pd);
                    // dQ^T += K~^T dS^T (dims 0..31 and 32..63)
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        const int ch = 4 * kb2 + 2 * kc + g;
                        dq0 = E::mfma(*(const u32x4 *)(kt + n * 128 + 16 * (ch ^ swz(n))), pd[kc],
                                      dq0);
                        dq1 = E::mfma(
                            *(const u32x4 *)(kt + (32 + n) * 128 + 16 * (ch ^ swz(32 + n))),
                            pd[kc], dq1);
                    }
                }
            }
        }
        if (more)
            ring_barrier<PIECES * (SL - 2)>();
        else
            ring_barrier<0>();
    };
    // steps [fa, fb) see every pair of the wave's rows and skip the mask
    int fa, fb;
    full_steps<false>(ka, steps, qw0, len, back, ahead, fa, fb);
    for (int st_i = 0; st_i < fa; ++st_i)
        step(st_i, Masked<true>{});
    for (int st_i = fa; st_i < fb; ++st_i)
        step(st_i, Masked<false>{});
    for (int st_i = fb; st_i < steps; ++st_i)
        step(st_i, Masked<true>{});

    // dQ rotated back to the row's position (the transpose of the half-split rotation) and
    // scaled; register i of block b holds dim 32b + 8(i/4) + 4g + i%4 of row qi
    if (qi < len) {
        const uint16_t *cr = cos_t + (int64_t)qi * 32, *sr = sin_t + (int64_t)qi * 32;
        uint16_t *o = dqkv + (int64_t)(start + qi) * ld + h * D;
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int m0 = 8 * gi + 4 * g;
            const u32x2 cw = *(const u32x2 *)(cr + m0), sw = *(const u32x2 *)(sr + m0);
            float a[4], bb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float cm = (e & 1) ? E::hi(cw[e >> 1]) : E::lo(cw[e >> 1]);
                const float sm = (e & 1) ? E::hi(sw[e >> 1]) : E::lo(sw[e >> 1]);
                const float x1 = dq0[4 * gi + e], x2 = dq1[4 * gi + e];
                a[e] = scale * (x1 * cm + x2 * sm);
                bb[e] = scale * (x2 * cm - x1 * sm);
            }
            asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
            asm volatile("" : "+v"(bb[0]), "+v"(bb[1]), "+v"(bb[2]), "+v"(bb[3]));
            *(u32x2 *)(o + m0) = u32x2{E::pack(a[0], a[1]), E::pack(a[2], a[3])};
            *(u32x2 *)(o + 32 + m0) = u32x2{E::pack(bb[0], bb[1]), E::pack(bb[2], bb[3])};
        }
    }
}

template <class E, int NW>
int launch_backward_tiles(const BackArgs &a) {
    const int64_t blocks = (int64_t)a.num_tiles * a.H;
    if (blocks > INT32_MAX)
        return fail(VLF_EINVAL, "%lld workgroups exceed the grid limit", (long long)blocks);
    const uint16_t *qkv = (const uint16_t *)a.qkv, *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin, *out = (const uint16_t *)a.out;
    const uint16_t *dout = (const uint16_t *)a.dout;
    uint16_t *dqkv = (uint16_t *)a.dqkv;
    uint8_t *ws = (uint8_t *)a.workspace;
    const uint8_t *wsc = ws;
    const float *lse = a.lse;
    int32_t num_tiles = a.num_tiles, T = a.T, S = a.S, H = a.H, P = a.table_rows;
    int32_t Bk = a.back, Ah = a.ahead;
    float scale = a.scale;
    hipStream_t st = (hipStream_t)a.stream;
    void *args1[] = {(void *)&qkv, (void *)&cs,   (void *)&sn,        (void *)&a.cu,
                     (void *)&a.tiles, (void *)&out, (void *)&dout, (void *)&lse,
                     (void *)&ws,  (void *)&num_tiles, (void *)&T, (void *)&S,
                     (void *)&H,   (void *)&P,    (void *)&scale};
    // 64-row tiles stage their operands in the passes (sequences of one or two steps gain
    // nothing from images written once); taller ones stream the images back_prep writes
    constexpr bool DIRECT = NW == 2;
    hipError_t e = hipLaunchKernel((const void *)back_prep<E, 32 * NW, !DIRECT>,
                                   dim3((unsigned)blocks), dim3(256), args1, 0, st);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "backward prep launch failed: %s", hipGetErrorString(e));
    constexpr int SL = NW == 8 ? 4 : 2;
    void *args3[] = {(void *)&qkv, (void *)&cs, (void *)&sn, (void *)&a.cu, (void *)&a.tiles,
                     (void *)&dout, (void *)&wsc, (void *)&dqkv, (void *)&num_tiles,
                     (void *)&T, (void *)&S, (void *)&H, (void *)&P, (void *)&Bk, (void *)&Ah,
                     (void *)&scale};
    e = hipLaunchKernel((const void *)back_kv<E, NW, SL, DIRECT>, dim3((unsigned)blocks),
                        dim3(64 * NW), args3, 0, st);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "dK/dV launch failed: %s", hipGetErrorString(e));
    e = hipLaunchKernel((const void *)back_q<E, NW, SL, DIRECT>, dim3((unsigned)blocks),
                        dim3(64 * NW), args3, 0, st);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "dQ launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}

template <class E>
int launch_backward_typed(const BackArgs &a) {
    if (a.br == 256)
        return launch_backward_tiles<E, 8>(a);
    return a.br == 128 ? launch_backward_tiles<E, 4>(a) : launch_backward_tiles<E, 2>(a);
}

// ---- the unfused baseline's rotation pass ------------------------------------------------------
// The forward's rotation as a pass of its own, writing qkv' with q' = the query rotated at its
// position and times `scale`, k' = the key rotated, v' = v, each rounded exactly as the fused
// kernels round their operands. The forward over qkv' with identity tables (cos 1, sin 0) and
// scale 1 then multiplies the same rounded operands as the fused forward over qkv. R rows of one
// table entry and one head per workgroup, four lanes a row.
template <class E, int R>
__global__ void __launch_bounds__(256)
rotate_qkv(const uint16_t *__restrict__ qkv, const uint16_t *__restrict__ cos_t,
           const uint16_t *__restrict__ sin_t, const int32_t *__restrict__ cu,
           const uint32_t *__restrict__ tiles, uint16_t *__restrict__ dst, int32_t num_tiles,
           int32_t T, int32_t S, int32_t H, int32_t P, float scale) {
    const int work = xcd_work();
    const int h = work / num_tiles;
    int seq, start, len, i0;
    if (!back_tile(tiles, cu, work - h * num_tiles, S, T, P, seq, start, len, i0))
        return;
    const int64_t ld = 3LL * H * D;
    const int hd = H * D;
    const int tid = (int)threadIdx.x;
    const int row = tid >> 2, c4 = tid & 3;
#pragma unroll 1
    for (int t = i0; t < i0 + R && t < len; t += BC) {
        const int i = t + row;
        if (i >= len)
            continue;
        const uint16_t *src = qkv + (int64_t)(start + i) * ld + h * D + 8 * c4;
        uint16_t *o = dst + (int64_t)(start + i) * ld + h * D + 8 * c4;
        const u32x4 c = *(const u32x4 *)(cos_t + (int64_t)i * 32 + 8 * c4);
        const u32x4 sn = *(const u32x4 *)(sin_t + (int64_t)i * 32 + 8 * c4);
        const uint32_t c_[4] = {c[0], c[1], c[2], c[3]}, s_[4] = {sn[0], sn[1], sn[2], sn[3]};
#pragma unroll
        for (int part = 0; part < 2; ++part) {  // the query, then the key
            const u32x4 x1 = *(const u32x4 *)(src + part * hd);
            const u32x4 x2 = *(const u32x4 *)(src + part * hd + 32);
            const uint32_t a_[4] = {x1[0], x1[1], x1[2], x1[3]};
            const uint32_t b_[4] = {x2[0], x2[1], x2[2], x2[3]};
            uint32_t y1[4], y2[4];
            rotate<E, 4>(a_, b_, c_, s_, part == 0 ? scale : 1.0f, y1, y2);
            *(u32x4 *)(o + part * hd) = u32x4{y1[0], y1[1], y1[2], y1[3]};
            *(u32x4 *)(o + part * hd + 32) = u32x4{y2[0], y2[1], y2[2], y2[3]};
        }
        *(u32x4 *)(o + 2 * hd) = *(const u32x4 *)(src + 2 * hd);
        *(u32x4 *)(o + 2 * hd + 32) = *(const u32x4 *)(src + 2 * hd + 32);
    }
}

template <class E>
int launch_rotate_qkv_typed(const RotateArgs &a) {
    const int64_t blocks = (int64_t)a.num_tiles * a.H;
    if (blocks > INT32_MAX)
        return fail(VLF_EINVAL, "%lld workgroups exceed the grid limit", (long long)blocks);
    const uint16_t *qkv = (const uint16_t *)a.qkv, *cs = (const uint16_t *)a.cos;
    const uint16_t *sn = (const uint16_t *)a.sin;
    uint16_t *dst = (uint16_t *)a.dst;
    int32_t num_tiles = a.num_tiles, T = a.T, S = a.S, H = a.H, P = a.table_rows;
    float scale = a.scale;
    void *args[] = {(void *)&qkv, (void *)&cs, (void *)&sn, (void *)&a.cu, (void *)&a.tiles,
                    (void *)&dst, (void *)&num_tiles, (void *)&T, (void *)&S, (void *)&H,
                    (void *)&P, (void *)&scale};
    const void *k = a.br == 256   ? (const void *)rotate_qkv<E, 256>
                    : a.br == 128 ? (const void *)rotate_qkv<E, 128>
                                  : (const void *)rotate_qkv<E, 64>;
    const hipError_t e =
        hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)a.stream);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "rotation pass launch failed: %s", hipGetErrorString(e));
    return VLF_OK;
}
}  // namespace

// ---- the forward's key-tile workspace in a fixed device array ---------------------------------
// For callers that cannot allocate device memory (code under stream capture, serving loops that
// forbid it): vlf_attend_static runs the workspace path on this array instead of a caller's
// workspace. Every GPU the library runs on holds its own copy, at its own address, until the
// process ends. Host code never passes `scratch` itself to a kernel (in host code the name
// stands for a host-side shadow, not device memory): the device address is looked up once per
// device, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[VLF_STATIC_WORKSPACE_BYTES];

int static_scratch(void **ptr) {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static void *addr[kDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(VLF_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kDevices)
        return fail(VLF_EUNSUPPORTED, "device %d beyond the %d the library tracks", dev, kDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(VLF_EHIP, "device address of the static workspace on device %d: %s",
                        dev, hipGetErrorString(e));
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return VLF_OK;
}

int64_t backward_workspace_bytes(int32_t T, int32_t S, int32_t H, int32_t br) {
    if (T == 0)
        return 0;
    const int64_t floats = back_img_offset(T, H);
    return br == 64 ? floats : floats + (int64_t)H * (T / BC + S) * BIMG;
}

int launch_backward(const BackArgs &a) {
    return a.dtype == VLF_BF16 ? launch_backward_typed<BF16>(a) : launch_backward_typed<F16>(a);
}

int launch_rotate_qkv(const RotateArgs &a) {
    return a.dtype == VLF_BF16 ? launch_rotate_qkv_typed<BF16>(a)
                               : launch_rotate_qkv_typed<F16>(a);
}

int launch_attend(const AttendArgs &a, Launch what) {
    const bool bf = a.dtype == VLF_BF16;
    if (what == Launch::kRotate || what == Launch::kBoth) {
        const int rc = bf ? launch_rotate<BF16>(a) : launch_rotate<F16>(a);
        if (rc || what == Launch::kRotate)
            return rc;
    }
    if (what != Launch::kDirect)
        return bf ? launch_pre_br<BF16>(a) : launch_pre_br<F16>(a);
    // Whole-sequence descriptors need every row of the longest sequence (at most min(P, T)
    // rows) plus a tile past it to be reachable with a 31-bit byte offset.
    const int64_t rows = (int64_t)(a.table_rows < a.T ? a.table_rows : a.T) + 2 * BC;
    const bool fixed = rows * 3 * a.H * D * 2 < ((int64_t)1 << 31);
    if (a.br == 256 && ring_holds(a.back, a.ahead, a.max_len)) {
        if (bf)
            return fixed ? launch_slide<BF16, true>(a) : launch_slide<BF16, false>(a);
        return fixed ? launch_slide<F16, true>(a) : launch_slide<F16, false>(a);
    }
    if (bf)
        return fixed ? launch_br<BF16, true>(a) : launch_br<BF16, false>(a);
    return fixed ? launch_br<F16, true>(a) : launch_br<F16, false>(a);
}

}  // namespace vlf
