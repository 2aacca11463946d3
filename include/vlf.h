/*
 * vlf.h — C ABI of libvlf.so: packed variable-length attention with rotary position embeddings
 * applied inside the kernel and an optional symmetric (or causal) window, forward and backward,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one hanzo-kernel 0.2.42 `src/packed.rs` defines: its module contract
 * (layouts of qkv, cu, tiles, cos/sin and the window value), the host `layout` function (the tile
 * table), the `attend` kernel (rotation, masking, online softmax, outputs and log-sum-exp) and
 * its backward (`delta`, `attend_back`, `rotate_back`). vlf_rotate_qkv is the rotation as a pass
 * of its own, the baseline that measures what its fusion saves.
 *
 * Conventions for every call:
 *   - Head dimension is 64. H heads; a token's row of qkv holds 3*H*64 elements: the H query
 *     heads, then the H key heads, then the H value heads, each head's 64 elements contiguous.
 *   - cu [S+1] int32: cu[0] = 0, non-decreasing, cu[S] = T. Sequence s owns tokens
 *     cu[s] .. cu[s+1]-1. Zero-length sequences are allowed.
 *   - window: 0 = every key of the query's own sequence; W >= 1 = keys j with |i - j| < W
 *     (i, j positions within the sequence). ORed with VLF_CAUSAL it is the causal sliding
 *     window instead: keys j with i - W < j <= i (W >= 1), or j <= i (W = 0). The causal mode
 *     is not on the page's `attend`, which takes the symmetric one; the convention is that of
 *     the array library page's sliding-window mask.
 *   - Status codes are returned; nothing aborts or throws across this boundary. After a
 *     non-zero status, vlf_last_error() returns a message (per calling thread).
 *   - Pointers marked "host" are read by the CPU during the call only. Pointers marked
 *     "device" are HIP device memory owned by the caller; the library keeps no reference after
 *     the call returns and allocates no device memory.
 *   - There are two ways to run the forward. With a workspace, the keys are rotated once per
 *     call into 64-key tile images that every query tile then streams; this is the faster
 *     choice when sequences span several query tiles. Without one, every workgroup rotates the
 *     key tiles it reads. Both round the same operands and run the same products. They may
 *     subtract different reference maxima before the exp, which cancel in the results, so the
 *     probabilities are rounded at different scales: lse agrees to float32 rounding and out
 *     to about one storage-type ulp.
 */
#ifndef VLF_H
#define VLF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vlf_status {
    VLF_OK = 0,
    VLF_EINVAL = -1,       /* malformed argument (cu, sizes, null pointer, window, ...) */
    VLF_EUNSUPPORTED = -2, /* dtype or tile height the library does not build */
    VLF_EHIP = -3,         /* the HIP runtime reported an error (launch, device) */
};

enum vlf_dtype {
    VLF_F16 = 0,  /* IEEE binary16 */
    VLF_BF16 = 1, /* bfloat16 */
};

/* Flag ORed into `window` for the causal sliding window (see the conventions above). */
#define VLF_CAUSAL 0x40000000

/* Library ABI version (this header: 5). */
int32_t vlf_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
const char *vlf_last_error(void);

/*
 * Validate cu and size the tile table for `br`-row query tiles.
 * hanzo-kernel 0.2.42 src/packed.rs, `layout`: every sequence contributes ceil(L_s / br) tiles.
 *   cu_host    host, [S+1] int32, checked as described above.
 *   br         tile height >= 1 (vlf_attend runs 64, 128 and 256).
 *   num_tiles  out: number of tiles (may be 0).
 *   max_len    out: the longest sequence (0 if none). May be NULL.
 * Errors: VLF_EINVAL for a malformed cu, br < 1 or a total above INT32_MAX tiles.
 */
int vlf_tile_count(const int32_t *cu_host, int32_t S, int32_t T, int32_t br, int32_t *num_tiles,
                   int32_t *max_len);

/*
 * Write the tile table: for each sequence s in order and each first row i0 = 0, br, 2*br, ...
 * below L_s, the pair (s, i0), as consecutive uint32 values (hanzo-kernel 0.2.42
 * src/packed.rs, `layout`). Zero-length sequences get no tiles.
 *   tiles_host  host, capacity >= 2 * num_tiles uint32 (num_tiles from vlf_tile_count).
 *   capacity    number of uint32 slots in tiles_host.
 * Errors: VLF_EINVAL (bad cu, br < 1, capacity too small).
 */
int vlf_tile_table(const int32_t *cu_host, int32_t S, int32_t T, int32_t br, uint32_t *tiles_host,
                   int64_t capacity);

/*
 * The tile table in the order vlf_attend runs it best at this schedule: the entries of
 * vlf_tile_table (hanzo-kernel 0.2.42 src/packed.rs, `layout`), permuted. Where the direct path
 * runs attend_slide (br = 256, prerotate 0, every tile's reached keys within eight key tiles,
 * as vlf_forward_kernel names it), each CU takes an equal count of consecutive entries, so
 * whole sequences (their entries kept adjacent and in row order) are ordered by the work of
 * their entries: the most costly, the least costly, the second most, the second least, and so
 * on (ties by sequence index). An entry's cost is 2 plus the 64-key tiles its 256 rows reach.
 * Every other schedule gets the canonical order of vlf_tile_table.
 *   cu_host, S, T, br   as in vlf_tile_table.
 *   prerotate, window   as the batch will be run (vlf_choose_schedule, vlf_attend).
 *   tiles_host          out, host, [num_tiles, 2] uint32.   capacity  as in vlf_tile_table.
 * Host time O(S log S + num_tiles). Errors: those of vlf_tile_table; window < 0 (VLF_EINVAL).
 */
int vlf_launch_table(const int32_t *cu_host, int32_t S, int32_t T, int32_t br, int32_t prerotate,
                     int32_t window, uint32_t *tiles_host, int64_t capacity);

/*
 * The number of (query, key) pairs one head computes: for each row i of each sequence, the
 * keys j of the same sequence the window admits (the masking of hanzo-kernel 0.2.42
 * src/packed.rs `attend`, or the causal window with VLF_CAUSAL). Effective FLOPs of one call
 * are 4 * 64 * pairs * H.
 *   cu_host  host, [S+1]. pairs  out.
 * Errors: VLF_EINVAL (bad cu, window < 0).
 */
int vlf_visible_pairs(const int32_t *cu_host, int32_t S, int32_t T, int32_t window,
                      uint64_t *pairs);

/*
 * Device workspace vlf_attend needs to pre-rotate keys for T tokens in S sequences and H heads:
 * NB = floor(T / 64) + S blocks of 16384 bytes per head, then H * NB float32 values, in all
 * H * NB * 16388 bytes. Key tile u (keys 64u .. 64u+63) of sequence s and head h occupies block
 * h * NB + floor(cu[s] / 64) + s + u; these indices never collide for a valid cu. A block holds
 * two 8192-byte images: the rotated, rounded keys [key][dim] and the values transposed
 * [dim][key], 64 rows of 128 bytes each. The float32 at the same index bounds the Euclidean norm
 * of the block's rounded keys from above.
 *   bytes  out: the size (0 when T, S or H is 0).
 * Errors: VLF_EINVAL (negative size, H > 65536, null bytes).
 */
int vlf_workspace_bytes(int32_t T, int32_t S, int32_t H, int64_t *bytes);

/*
 * The schedule rule: which tile height and forward path serve a batch best, from two statistics
 * of its lengths, and which tile height the backward takes. The page picks its launch shape per
 * batch by measurement (hanzo-kernel 0.2.42 src/packed.rs, `attend_tuned` and
 * `attend_back_tuned`, with `usable` / `fits` checking capacity); this rule was fitted to such
 * measurements on MI355X and is what vlf_choose_schedule and vlf_choose_backward apply.
 *   max_len     the longest sequence (vlf_tile_count).
 *   typical     the length of the sequence an average token sits in, sum(L^2) / sum(L)
 *               (vlf_typical_length); work per token grows with it.
 *   window      as in vlf_attend.
 *   br_request  0: choose the tile height; 64, 128 or 256: take it and choose only the path.
 *   br          out: 64 when no sequence is longer than 64 (one key tile per query tile);
 *               256 once typical >= 256 where the direct path keeps every key a 256-row tile
 *               reaches in LDS (vlf_forward_kernel names attend_slide: a window of at most
 *               eight key tiles, or max_len <= 512); 128 under other windows of at most 512;
 *               for wider or full windows 256 once typical >= 448, else 128.
 *   prerotate   out: 1 to rotate keys once into a workspace (vlf_attend with a workspace),
 *               0 for the direct path. 1 when a query tile's key span (typical, or
 *               br + back + ahead + 1 for a window) reaches three tiles at 64 or 128 rows,
 *               1.75 tiles at 256 rows; 0 where the direct path runs attend_slide.
 *   backward_br out (may be NULL): the backward's tile height, 128 once typical >= 128,
 *               else 64.
 * Errors: VLF_EINVAL (negative max_len or typical, window < 0, br_request not 0, 64, 128 or
 * 256, null br or prerotate).
 */
int vlf_schedule_rule(int32_t max_len, double typical, int32_t window, int32_t br_request,
                      int32_t *br, int32_t *prerotate, int32_t *backward_br);

/*
 * sum(L^2) / sum(L) over the sequences of cu (0 for a batch without tokens).
 *   cu_host  host, [S+1].   typical  out.
 * Errors: VLF_EINVAL (bad cu, null typical).
 */
int vlf_typical_length(const int32_t *cu_host, int32_t S, int32_t T, double *typical);

/*
 * The forward's schedule for a batch: vlf_schedule_rule applied to cu's statistics.
 *   cu_host          host, [S+1], checked as vlf_tile_count checks it.
 *   H, window        as in vlf_attend.
 *   br, prerotate    out: as vlf_schedule_rule returns them.
 *   max_len          out (may be NULL): the longest sequence, vlf_attend's max_len.
 *   workspace_bytes  out (may be NULL): vlf_workspace_bytes(T, S, H) when prerotate is 1,
 *                    else 0: what the caller allocates for vlf_attend.
 * Errors: VLF_EINVAL (bad cu, H out of range, window < 0, null br or prerotate).
 */
int vlf_choose_schedule(const int32_t *cu_host, int32_t S, int32_t T, int32_t H, int32_t window,
                        int32_t *br, int32_t *prerotate, int32_t *max_len,
                        int64_t *workspace_bytes);

/*
 * The backward's schedule for a batch: its tile height (vlf_schedule_rule's backward_br) and
 * the workspace vlf_attend_backward needs at that height.
 *   cu_host, H, window  as in vlf_choose_schedule.
 *   br               out: 64 or 128.
 *   workspace_bytes  out (may be NULL): vlf_backward_workspace_bytes(T, S, H, br).
 * Errors: VLF_EINVAL (bad cu, H out of range, window < 0, null br).
 */
int vlf_choose_backward(const int32_t *cu_host, int32_t S, int32_t T, int32_t H, int32_t window,
                        int32_t *br, int64_t *workspace_bytes);

/*
 * Name of the forward kernel vlf_attend launches for a tile height, path, window and longest
 * sequence (the key-tile kernel prep_tiles runs before it when prerotate is 1): "attend_pre_ph"
 * (workspace, 256 rows), "attend_pre" (workspace, 64 or 128 rows), "attend_slide" (direct, 256
 * rows, every key a tile reaches kept in an LDS ring of eight key tiles: a window with
 * 1 <= W <= 129, or causal 1 <= W <= 257, or any window when max_len <= 512), "attend_one"
 * (direct, 64 rows) or "attend_fwd" (direct, 128 or 256 rows); "" for a tile height the library
 * does not run, a negative window or a negative max_len. A static string.
 */
const char *vlf_forward_kernel(int32_t br, int32_t prerotate, int32_t window, int32_t max_len);

/*
 * The forward pass (hanzo-kernel 0.2.42 src/packed.rs, `attend`): for each tile in tiles_dev
 * and each head h, query rows i0 .. i0+br-1 of sequence s against the keys of s the window
 * reaches.
 *
 *   For a row at position i of sequence s (token t = cu[s] + i) and head h:
 *     q~ = storage-type rounding of (rot(q_t, i) * scale), rotation and scale in float32;
 *     k~_j = storage-type rounding of rot(k_{cu[s]+j}, j);
 *     rot(x, p)[m] = x[m] cos[p][m] - x[m+32] sin[p][m],
 *     rot(x, p)[m+32] = x[m] sin[p][m] + x[m+32] cos[p][m]   (m < 32);
 *     scores s_ij = <q~, k~_j> (float32 accumulation) for visible j;
 *     out[t][h*64 + d] = sum_j softmax_j(s_ij) v_j[d], rounded to the storage type;
 *     lse[h*T + t]     = ln sum_j exp(s_ij)  (float32, natural log of the scaled scores).
 *
 *   qkv        device, [T, 3*H*64] elements of `dtype`, rows contiguous.
 *   cos, sin   device, [table_rows, 32] elements of `dtype`: entry [p][m] for position p.
 *   table_rows P, rows of the tables.
 *   max_len    the longest sequence of cu (vlf_tile_count's max_len). The call fails with
 *              VLF_EINVAL when P < max_len. It also picks the kernel (vlf_forward_kernel): at
 *              max_len <= 512 the direct path at 256 rows holds whole sequences in an LDS ring,
 *              and at max_len <= 64 the direct path at 64 rows sweeps one key tile per tile.
 *              The library cannot read cu_dev to check it, so a max_len that understates is
 *              the caller's error with a defined outcome: a tile naming a sequence longer than
 *              P, or (on that ring) one whose keys span more than eight key tiles, or (at 64
 *              rows with max_len <= 64) one whose keys span more than one key tile, is skipped
 *              (its rows left unwritten) rather than read past the tables or the ring.
 *   cu_dev     device, [S+1] int32, the same values as the cu the tiles were built from.
 *   tiles_dev  device, [num_tiles, 2] uint32 (sequence, first row) pairs built for the same cu
 *              and `br` (vlf_tile_table, or any permutation of it: the order is the launch
 *              order). Tiles naming a sequence >= S or a row beyond the sequence are skipped.
 *              Without a workspace, at br = 256 where every tile's reached keys span at most
 *              eight key tiles (1 <= W <= 129, causal 1 <= W <= 257, or max_len <= 512), each
 *              CU walks a run of consecutive entries and keeps the keys that one entry shares
 *              with the next of the same sequence in LDS: any order gives the same results;
 *              vlf_launch_table's is the fastest (entries of a sequence adjacent and in row
 *              order, sequences interleaved by cost). There, when S <= 256, S * H is at least
 *              twice the number of CUs and each CU's share of whole (sequence, head) runs fits
 *              its list (ceil(S H / CUs) * ceil(table_rows / 256) <= 64), the kernel instead
 *              ranks the sequences cu describes by cost and deals whole runs to the CUs in
 *              snake order; the table's order is then not used (its entries must still be a
 *              permutation of vlf_tile_table's).
 *   br         64, 128 or 256: rows per tile, as the table was built.
 *   T, S, H    tokens, sequences, heads (1 <= H <= 65536; T = 0 or num_tiles = 0 launches
 *              nothing).
 *   window     0 or W >= 1, optionally | VLF_CAUSAL, as above.
 *   scale      multiplies the rotated query before rounding (1/8 for head dimension 64).
 *   dtype      VLF_BF16 or VLF_F16: storage type of qkv, cos, sin and out.
 *   workspace  device (16-byte aligned) or NULL. With workspace_bytes >=
 *              vlf_workspace_bytes(T, S, H), the call
 *              first rotates every key tile once into it (vlf_rotate_keys, then
 *              vlf_attend_rotated: two kernels on `stream`); its
 *              previous contents are ignored and overwritten, so calls that may overlap in
 *              time need separate workspaces. NULL (and workspace_bytes 0): no workspace is
 *              used.
 *   workspace_bytes  size of `workspace` in bytes.
 *   out        device, [T, H*64] elements of `dtype`. Every row of every tiled sequence is
 *              written; nothing else is.
 *   lse        device, [H, T] float32, written for the same rows.
 *   stream     hipStream_t to launch on (NULL = the null stream). The call is asynchronous:
 *              it never synchronises, never allocates, and returns once the launch is queued.
 *
 * Errors: VLF_EINVAL (null pointer with work to do, H out of range, window < 0, negative sizes,
 * T or S inconsistent with each other, num_tiles < 0, max_len < 0, table_rows < max_len, a
 * workspace not 16-byte aligned or smaller than vlf_workspace_bytes or a size without a
 * pointer), VLF_EUNSUPPORTED (dtype, br), VLF_EHIP (launch failure, from hipGetLastError).
 * Device-side contents (cu_dev, tiles_dev) cannot be checked here; the kernel skips tiles that
 * would read out of range.
 */
int vlf_attend(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
               int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
               int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H, int32_t window,
               float scale, int32_t dtype, void *workspace, int64_t workspace_bytes, void *out,
               float *lse, void *stream);

/* Bytes of the fixed device array vlf_attend_static uses as its key-tile workspace. */
#define VLF_STATIC_WORKSPACE_BYTES (128LL << 20)

/*
 * vlf_attend on the key-tile workspace path, for callers that cannot allocate device memory
 * (code under stream capture, serving loops and harnesses that forbid allocation): the
 * workspace is a fixed array of VLF_STATIC_WORKSPACE_BYTES in the library's device memory,
 * one per GPU, held until the process ends, instead of a caller's buffer. The call allocates
 * and frees nothing. Arguments and results as in vlf_attend without `workspace` and
 * `workspace_bytes`: the same two kernels on `stream` (key tiles, then the forward over them),
 * so the same bits as vlf_attend with a workspace of its own. The array's address on the
 * current device is looked up on the first call there.
 *   Every call on one GPU shares that GPU's array: calls that may overlap in time on one GPU
 *   (other streams, other threads) race on it and must be ordered by the caller. Each call
 *   writes every block and norm bound it reads before reading it, so nothing in the array
 *   needs clearing and the previous call's contents never reach a result.
 * Errors: as vlf_attend; VLF_EINVAL also when vlf_workspace_bytes(T, S, H) exceeds
 * VLF_STATIC_WORKSPACE_BYTES (the message gives both sizes); VLF_EHIP when the array's device
 * address cannot be obtained.
 */
int vlf_attend_static(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                      int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                      int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                      int32_t window, float scale, int32_t dtype, void *out, float *lse,
                      void *stream);

/*
 * The first half of vlf_attend with a workspace: rotate every key tile of cu once and write it,
 * with its values, into `workspace` (the blocks vlf_workspace_bytes describes; the rotation and
 * rounding of k~ in vlf_attend's formula). Arguments as in vlf_attend. One kernel on `stream`;
 * asynchronous; allocates nothing.
 * Errors: VLF_EINVAL (null pointer with work to do, H out of range, negative sizes, T or S
 * inconsistent, table_rows < max_len, workspace missing or smaller than vlf_workspace_bytes),
 * VLF_EUNSUPPORTED (dtype), VLF_EHIP (launch failure).
 */
int vlf_rotate_keys(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                    int32_t max_len, const int32_t *cu_dev, int32_t T, int32_t S, int32_t H,
                    int32_t dtype, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The second half of vlf_attend with a workspace: the forward over key tiles a previous
 * vlf_rotate_keys wrote into `workspace` for the same qkv, cos, sin, cu and H (queued earlier on
 * the same stream, or otherwise complete). Arguments and results as in vlf_attend; `workspace`
 * is read, not written, and may be shared by calls that overlap in time. One kernel on `stream`.
 * Errors: as vlf_attend; the workspace is required.
 */
int vlf_attend_rotated(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                       int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                       int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                       int32_t window, float scale, int32_t dtype, const void *workspace,
                       int64_t workspace_bytes, void *out, float *lse, void *stream);

/*
 * Device workspace vlf_attend_backward needs for T tokens in S sequences and H heads on br-row
 * tiles: float32 -delta and -lse (natural log), [H, T] each, padded to a multiple of 256 bytes;
 * then, for br = 128 or 256 only, per head floor(T / 64) + S blocks of 40 KiB (the operand images
 * of one 64-row tile: rotated queries, their transpose, the transposed output gradient, rotated
 * keys and their transpose). Calls on 64-row tiles stage their operands inside the passes and
 * need no blocks.
 *   br     64, 128 or 256.
 *   bytes  out: the size (0 when T is 0).
 * Errors: VLF_EINVAL (negative size, H > 65536, br, null bytes).
 */
int vlf_backward_workspace_bytes(int32_t T, int32_t S, int32_t H, int32_t br, int64_t *bytes);

/*
 * The backward pass (hanzo-kernel 0.2.42 src/packed.rs: `delta`, `attend_back`, `rotate_back`):
 * dqkv = d sum(out * dout) / d qkv for the forward of vlf_attend with the same arguments.
 *
 *   For each sequence and head, with q~, k~ and the visible set of vlf_attend's formula:
 *     delta_i = <dout_i, out_i> (float32, from the stored out);
 *     p_ij    = exp(<q~_i, k~_j> - lse_i) for visible j, 0 otherwise (from the stored lse);
 *     ds_ij   = p_ij (<dout_i, v_j> - delta_i);
 *     dv_j    = sum_i p_ij dout_i;
 *     dk_j    = the transposed rotation at position j of sum_i ds_ij q~_i;
 *     dq_i    = scale times the transposed rotation at position i of sum_j ds_ij k~_j.
 *   p and ds are rounded to the storage type where they enter matrix products; every sum is
 *   float32 in registers and every element of dqkv is written once (no atomics: the same
 *   inputs give the same bits). dq has a pass of its own that recomputes p and ds; the page
 *   adds dq into float32 with atomics instead.
 *
 *   qkv, cos, sin, table_rows, max_len, cu_dev, T, S, H, window, scale, dtype  as in
 *              vlf_attend.
 *   tiles_dev, num_tiles  the tile table for br-row tiles (vlf_tile_table with this br, or any
 *              permutation of it): each entry is a key tile of the dK/dV pass and a query tile
 *              of the dQ pass.
 *   br         64, 128 or 256: the rows of a tile, 32 per wave of the two passes.
 *   out        device, [T, H*64] of `dtype`: the forward's output for these inputs.
 *   dout       device, [T, H*64] of `dtype`: the gradient of the loss with respect to out.
 *   lse        device, [H, T] float32: the forward's log-sum-exp for these inputs.
 *   workspace  device, at least vlf_backward_workspace_bytes(T, S, H, br) bytes, 16-byte
 *              aligned; overwritten.
 *   dqkv       device, [T, 3*H*64] of `dtype`: every row of every tiled sequence written.
 *   stream     hipStream_t (NULL = the null stream). Three kernels; asynchronous; allocates
 *              nothing. Calls that may overlap in time need separate workspaces.
 *
 * Errors: VLF_EINVAL (null pointer with work to do, H out of range, window < 0, br not 64, 128
 * or 256, negative sizes, T or S inconsistent, table_rows < max_len, a workspace smaller than
 * vlf_backward_workspace_bytes or not 16-byte aligned), VLF_EUNSUPPORTED (dtype), VLF_EHIP
 * (launch failure).
 */
int vlf_attend_backward(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                        int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                        int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                        int32_t window, float scale, int32_t dtype, const void *out,
                        const void *dout, const float *lse, void *workspace,
                        int64_t workspace_bytes, void *dqkv, void *stream);

/*
 * The unfused baseline's rotation pass: the forward's rotation as a kernel of its own (the page
 * applies it inside `attend`; this pass exists to measure what that fusion saves). For every
 * row i of every tiled sequence and every head it writes
 *     qkv_out q part = RNE_dtype(RN_f32(rot(q, i)) * scale),
 *     qkv_out k part = RNE_dtype(RN_f32(rot(k, i))),
 *     qkv_out v part = v,
 * the operands exactly as vlf_attend rounds them, so vlf_attend over qkv_out with identity
 * tables (cos 1, sin 0) and scale 1 gives the bits vlf_attend gives over qkv.
 *
 *   qkv, cos, sin, table_rows, max_len, cu_dev, T, S, H, scale, dtype  as in vlf_attend.
 *   tiles_dev, num_tiles, br  a tile table (vlf_tile_table) for br = 64, 128 or 256.
 *   qkv_out    device, [T, 3*H*64] of `dtype`, not qkv; rows no tile covers are not written.
 *   stream     hipStream_t (NULL = the null stream). One kernel; asynchronous.
 *
 * Errors: VLF_EINVAL (null pointer with work to do, qkv_out == qkv, H out of range, br, negative
 * sizes, T or S inconsistent, table_rows < max_len), VLF_EUNSUPPORTED (dtype), VLF_EHIP (launch
 * failure).
 */
int vlf_rotate_qkv(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                   int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                   int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H, float scale,
                   int32_t dtype, void *qkv_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VLF_H */
