// Internal declarations shared by the host translation unit (vlf_host.cpp) and the kernel
// translation unit (vlf_attend.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace vlf {

// Everything the launcher needs after the host side has validated the arguments.
struct AttendArgs {
    const void *qkv;
    const void *cos;
    const void *sin;
    int32_t table_rows;
    int32_t max_len;  // the longest sequence (at most table_rows)
    const int32_t *cu;
    const uint32_t *tiles;
    int32_t num_tiles;
    int32_t br;
    int32_t T, S, H;
    int32_t back, ahead;  // row x sees keys x - back .. x + ahead (window_reaches)
    float scale;
    int32_t dtype;
    void *workspace;  // NULL: every workgroup rotates the key tiles it reads
    void *out;
    float *lse;
    void *stream;
};

// The window of the ABI (W, or W | VLF_CAUSAL) as the reaches the kernels take: row x sees the
// keys x - back .. x + ahead of its sequence, 0x7fffffff reaching every key on that side.
void window_reaches(int32_t window, int32_t &back, int32_t &ahead);

// Bytes of the key-tile workspace for T tokens, S sequences and H heads.
int64_t workspace_bytes(int32_t T, int32_t S, int32_t H);

// Whether a 256-row query tile's keys under the reaches span at most eight 64-key tiles: from
// i0 - 64 ceil(back / 64) (i0 a multiple of 64) to i0 + 255 + ahead. The direct path then runs
// the kernel that keeps them in an LDS ring (attend_slide).
bool ring_fits(int32_t back, int32_t ahead);

// Whether every 256-row query tile's keys span at most eight 64-key tiles for a batch whose
// longest sequence is max_len: the window fits (ring_fits), or no sequence is longer than eight
// tiles, so the whole sequence fits. The direct path then runs attend_slide.
bool ring_holds(int32_t back, int32_t ahead, int32_t max_len);

// What launch_attend queues.
enum class Launch {
    kDirect,   // the forward, every workgroup rotating the key tiles it reads
    kRotate,   // the key-tile workspace only
    kRotated,  // the forward over a workspace written before
    kBoth,     // kRotate, then kRotated
};

// Queue the forward kernels; returns a vlf_status.
int launch_attend(const AttendArgs &a, Launch what);

// The current device's address of the fixed workspace array (VLF_STATIC_WORKSPACE_BYTES),
// looked up on the first call on that device; returns a vlf_status.
int static_scratch(void **ptr);

// The backward's arguments after validation; tiles are the tile table for br-row tiles.
struct BackArgs {
    const void *qkv;
    const void *cos;
    const void *sin;
    int32_t table_rows;
    const int32_t *cu;
    const uint32_t *tiles;
    int32_t num_tiles;
    int32_t br;  // 64, 128 or 256
    int32_t T, S, H;
    int32_t back, ahead;
    float scale;
    int32_t dtype;
    const void *out;
    const void *dout;
    const float *lse;
    void *workspace;  // -delta and -lse (float32 [H, T] each), then, above 64 rows, the images
    void *dqkv;
    void *stream;
};

// Bytes of the backward's workspace on br-row tiles (the images only above 64 rows).
int64_t backward_workspace_bytes(int32_t T, int32_t S, int32_t H, int32_t br);

// Queue the backward kernels (prep, dK/dV, dQ); returns a vlf_status.
int launch_backward(const BackArgs &a);

// The unfused baseline's rotation pass after validation.
struct RotateArgs {
    const void *qkv;
    const void *cos;
    const void *sin;
    int32_t table_rows;
    const int32_t *cu;
    const uint32_t *tiles;
    int32_t num_tiles;
    int32_t br;  // 64, 128 or 256
    int32_t T, S, H;
    float scale;
    int32_t dtype;
    void *dst;
    void *stream;
};

// Queue the rotation pass; returns a vlf_status.
int launch_rotate_qkv(const RotateArgs &a);

// Record the calling thread's error message (printf-style) and return `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace vlf
