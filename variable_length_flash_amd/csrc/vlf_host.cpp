// Host side of libvlf.so: argument checks, the tile table, the visible-pair count and the
// schedule rule (tile height and path per batch).
//
// The tile table is the host-built index of hanzo-kernel 0.2.42 src/packed.rs (`layout`): one
// (sequence, first row) pair per `br` query rows of every sequence, in sequence order. The pair
// count follows the masking of that page's `attend` kernel: a query at position i sees key j of
// its own sequence when the window is 0 or |i - j| < window.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/vlf.h"

#include "vlf_internal.h"

namespace vlf {

static thread_local std::string g_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

// cu[0] = 0, non-decreasing, cu[S] = T. Reports the longest sequence.
static int check_cu(const int32_t *cu, int32_t S, int32_t T, int32_t *max_len) {
    if (S < 0 || T < 0)
        return fail(VLF_EINVAL, "negative size: S=%d T=%d", S, T);
    if (!cu)
        return fail(VLF_EINVAL, "cu is NULL");
    if (cu[0] != 0)
        return fail(VLF_EINVAL, "cu[0] = %d, expected 0", cu[0]);
    int32_t longest = 0;
    for (int32_t s = 0; s < S; ++s) {
        if (cu[s + 1] < cu[s])
            return fail(VLF_EINVAL, "cu decreases at s=%d (%d > %d)", s, cu[s], cu[s + 1]);
        int32_t L = cu[s + 1] - cu[s];
        if (L > longest)
            longest = L;
    }
    if (cu[S] != T)
        return fail(VLF_EINVAL, "cu[S] = %d, expected T = %d", cu[S], T);
    if (max_len)
        *max_len = longest;
    return VLF_OK;
}

static bool supported_br(int32_t br) { return br == 64 || br == 128 || br == 256; }

int64_t workspace_bytes(int32_t T, int32_t S, int32_t H) {
    if (T <= 0 || S <= 0 || H <= 0)
        return 0;
    return (int64_t)H * ((int64_t)(T / 64) + S) * (16384 + 4);
}

constexpr int32_t kReachAll = 0x7fffffff;

void window_reaches(int32_t window, int32_t &back, int32_t &ahead) {
    const int32_t W = window & ~VLF_CAUSAL;
    back = W > 0 ? W - 1 : kReachAll;
    ahead = (window & VLF_CAUSAL) ? 0 : back;
}

bool ring_fits(int32_t back, int32_t ahead) {
    if (back == kReachAll || ahead == kReachAll)
        return false;
    const int64_t behind = ((int64_t)back + 63) / 64 * 64;
    return (behind + 256 + ahead + 63) / 64 <= 8;
}

bool ring_holds(int32_t back, int32_t ahead, int32_t max_len) {
    return ring_fits(back, ahead) || max_len <= 8 * 64;
}

// sum(L^2) / sum(L): the length of the sequence an average token sits in.
static double typical_of(const int32_t *cu, int32_t S) {
    double sq = 0, total = 0;
    for (int32_t s = 0; s < S; ++s) {
        const double L = (double)cu[s + 1] - (double)cu[s];
        sq += L * L;
        total += L;
    }
    return total > 0 ? sq / total : 0.0;
}

// The rule vlf_schedule_rule documents; arguments already checked.
static void rule(int32_t max_len, double typical, int32_t window, int32_t br_request,
                 int32_t &br, int32_t &prerotate, int32_t &backward_br) {
    int32_t back, ahead;
    window_reaches(window, back, ahead);
    const bool ring = ring_holds(back, ahead, max_len);
    const int32_t W = window & ~VLF_CAUSAL;
    if (br_request) {
        br = br_request;
    } else if (max_len <= 64) {
        br = 64;  // one key tile per query tile: the unpipelined kernel
    } else if (ring && typical >= 256) {
        br = 256;  // the reached keys stay in an LDS ring across consecutive tiles
    } else if (W > 0 && W <= 512) {
        br = 128;  // taller tiles would compute more masked pairs (span br + 2W - 1)
    } else {
        br = typical >= 448 ? 256 : 128;
    }
    if (br == 256 && ring) {
        prerotate = 0;  // attend_slide keeps the reached keys in LDS already
    } else {
        // a query tile's key span: the typical length, or the window's reach
        double span = typical;
        if (back != kReachAll && ahead != kReachAll) {
            const double reach = (double)br + back + ahead + 1;
            span = reach < span ? reach : span;
        }
        prerotate = span >= (br < 256 ? 3.0 * br : 7.0 * br / 4) ? 1 : 0;
    }
    backward_br = typical >= 128 ? 128 : 64;
}

}  // namespace vlf

using namespace vlf;

extern "C" {

int32_t vlf_version(void) { return 5; }

const char *vlf_last_error(void) { return g_error.c_str(); }

int vlf_tile_count(const int32_t *cu_host, int32_t S, int32_t T, int32_t br, int32_t *num_tiles,
                   int32_t *max_len) {
    if (br < 1)
        return fail(VLF_EINVAL, "br = %d < 1", br);
    if (!num_tiles)
        return fail(VLF_EINVAL, "num_tiles is NULL");
    int32_t longest = 0;
    int rc = check_cu(cu_host, S, T, &longest);
    if (rc)
        return rc;
    int64_t n = 0;
    for (int32_t s = 0; s < S; ++s)
        n += ((int64_t)(cu_host[s + 1] - cu_host[s]) + br - 1) / br;
    if (n > INT32_MAX)
        return fail(VLF_EINVAL, "%lld tiles exceed INT32_MAX", (long long)n);
    *num_tiles = (int32_t)n;
    if (max_len)
        *max_len = longest;
    return VLF_OK;
}

int vlf_tile_table(const int32_t *cu_host, int32_t S, int32_t T, int32_t br, uint32_t *tiles_host,
                   int64_t capacity) {
    int32_t n = 0;
    int rc = vlf_tile_count(cu_host, S, T, br, &n, nullptr);
    if (rc)
        return rc;
    if (capacity < 2 * (int64_t)n)
        return fail(VLF_EINVAL, "capacity %lld < %lld", (long long)capacity, 2 * (long long)n);
    if (n > 0 && !tiles_host)
        return fail(VLF_EINVAL, "tiles_host is NULL");
    int64_t k = 0;
    for (int32_t s = 0; s < S; ++s) {
        const int32_t L = cu_host[s + 1] - cu_host[s];
        for (int64_t i0 = 0; i0 < L; i0 += br) {
            tiles_host[k++] = (uint32_t)s;
            tiles_host[k++] = (uint32_t)i0;
        }
    }
    return VLF_OK;
}

int vlf_launch_table(const int32_t *cu_host, int32_t S, int32_t T, int32_t br, int32_t prerotate,
                     int32_t window, uint32_t *tiles_host, int64_t capacity) {
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    int32_t n = 0, max_len = 0;
    int rc = vlf_tile_count(cu_host, S, T, br, &n, &max_len);
    if (rc)
        return rc;
    rc = vlf_tile_table(cu_host, S, T, br, tiles_host, capacity);
    if (rc)
        return rc;
    int32_t back, ahead;
    window_reaches(window, back, ahead);
    if (n == 0 || prerotate || br != 256 || !ring_holds(back, ahead, max_len))
        return VLF_OK;  // one workgroup per entry: the canonical order
    // attend_slide gives each CU an equal count of consecutive entries. Whole sequences (their
    // entries stay adjacent, so the key ring still carries over between them) are ordered
    // most costly, least costly, second most, second least, ..., so that every run mixes costly
    // and cheap entries. The cost of an entry is what its waves sweep: a fixed 2 plus the key
    // tiles its 256 rows reach (the kernel's key span).
    std::vector<std::pair<int64_t, int32_t>> cost;  // (cost, sequence), sequences with rows
    std::vector<int64_t> first((size_t)S + 1, 0);    // index of a sequence's first entry
    int64_t k = 0;
    for (int32_t s = 0; s < S; ++s) {
        first[s] = k;
        const int32_t L = cu_host[s + 1] - cu_host[s];
        int64_t c = 0;
        for (int64_t i0 = 0; i0 < L; i0 += 256, ++k) {
            const int64_t lo = i0 > back ? (i0 - back) / 64 * 64 : 0;
            const int64_t hi = i0 + 256 + (int64_t)ahead < L ? i0 + 256 + ahead : L;
            c += 2 + (hi - lo + 63) / 64;
        }
        if (L > 0)
            cost.emplace_back(c, s);
    }
    first[S] = k;
    std::stable_sort(cost.begin(), cost.end(),
                     [](const std::pair<int64_t, int32_t> &a,
                        const std::pair<int64_t, int32_t> &b) { return a.first > b.first; });
    std::vector<uint32_t> out;
    out.reserve(2 * (size_t)n);
    size_t a = 0, b = cost.size();
    bool front = true;
    while (a < b) {
        const int32_t s = front ? cost[a++].second : cost[--b].second;
        front = !front;
        for (int64_t e = first[s]; e < first[s + 1]; ++e) {
            out.push_back((uint32_t)s);
            out.push_back(tiles_host[2 * e + 1]);
        }
    }
    std::copy(out.begin(), out.end(), tiles_host);
    return VLF_OK;
}

int vlf_visible_pairs(const int32_t *cu_host, int32_t S, int32_t T, int32_t window,
                      uint64_t *pairs) {
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    const bool causal = (window & VLF_CAUSAL) != 0;
    window &= ~VLF_CAUSAL;
    if (!pairs)
        return fail(VLF_EINVAL, "pairs is NULL");
    int rc = check_cu(cu_host, S, T, nullptr);
    if (rc)
        return rc;
    uint64_t total = 0;
    for (int32_t s = 0; s < S; ++s) {
        const uint64_t L = (uint64_t)(cu_host[s + 1] - cu_host[s]);
        if (causal) {
            // row i sees min(i + 1, W) keys: L(L + 1)/2 while L <= W, then W per row
            const uint64_t W = window == 0 ? L : (uint64_t)window;
            total += L <= W ? L * (L + 1) / 2 : W * (W + 1) / 2 + (L - W) * W;
        } else if (window == 0 || L <= (uint64_t)window) {
            total += L * L;  // every key of the sequence
        } else {
            // rows see min(L, i + W) - max(0, i - W + 1) keys; summed over i this is
            // L(2W - 1) - W(W - 1) for L >= W
            const uint64_t W = (uint64_t)window;
            total += L * (2 * W - 1) - W * (W - 1);
        }
    }
    *pairs = total;
    return VLF_OK;
}

int vlf_workspace_bytes(int32_t T, int32_t S, int32_t H, int64_t *bytes) {
    if (!bytes)
        return fail(VLF_EINVAL, "bytes is NULL");
    if (T < 0 || S < 0 || H < 0)
        return fail(VLF_EINVAL, "negative size: T=%d S=%d H=%d", T, S, H);
    if (H > 65536)
        return fail(VLF_EINVAL, "H = %d above 65536", H);
    *bytes = workspace_bytes(T, S, H);
    return VLF_OK;
}

int vlf_schedule_rule(int32_t max_len, double typical, int32_t window, int32_t br_request,
                      int32_t *br, int32_t *prerotate, int32_t *backward_br) {
    if (!br || !prerotate)
        return fail(VLF_EINVAL, "null br or prerotate");
    if (max_len < 0 || !(typical >= 0))
        return fail(VLF_EINVAL, "max_len = %d, typical = %g", max_len, typical);
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    if (br_request != 0 && !supported_br(br_request))
        return fail(VLF_EINVAL, "br_request = %d; 0, 64, 128 or 256", br_request);
    int32_t b, p, bb;
    rule(max_len, typical, window, br_request, b, p, bb);
    *br = b;
    *prerotate = p;
    if (backward_br)
        *backward_br = bb;
    return VLF_OK;
}

int vlf_typical_length(const int32_t *cu_host, int32_t S, int32_t T, double *typical) {
    if (!typical)
        return fail(VLF_EINVAL, "typical is NULL");
    int rc = check_cu(cu_host, S, T, nullptr);
    if (rc)
        return rc;
    *typical = typical_of(cu_host, S);
    return VLF_OK;
}

int vlf_choose_schedule(const int32_t *cu_host, int32_t S, int32_t T, int32_t H, int32_t window,
                        int32_t *br, int32_t *prerotate, int32_t *max_len,
                        int64_t *workspace_bytes_) {
    if (!br || !prerotate)
        return fail(VLF_EINVAL, "null br or prerotate");
    if (H < 1 || H > 65536)
        return fail(VLF_EINVAL, "H = %d outside 1 .. 65536", H);
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    int32_t longest = 0;
    int rc = check_cu(cu_host, S, T, &longest);
    if (rc)
        return rc;
    int32_t b, p, bb;
    rule(longest, typical_of(cu_host, S), window, 0, b, p, bb);
    *br = b;
    *prerotate = p;
    if (max_len)
        *max_len = longest;
    if (workspace_bytes_)
        *workspace_bytes_ = p ? workspace_bytes(T, S, H) : 0;
    return VLF_OK;
}

int vlf_choose_backward(const int32_t *cu_host, int32_t S, int32_t T, int32_t H, int32_t window,
                        int32_t *br, int64_t *workspace_bytes_) {
    if (!br)
        return fail(VLF_EINVAL, "br is NULL");
    if (H < 1 || H > 65536)
        return fail(VLF_EINVAL, "H = %d outside 1 .. 65536", H);
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    int32_t longest = 0;
    int rc = check_cu(cu_host, S, T, &longest);
    if (rc)
        return rc;
    int32_t b, p, bb;
    rule(longest, typical_of(cu_host, S), window, 0, b, p, bb);
    *br = bb;
    if (workspace_bytes_)
        *workspace_bytes_ = backward_workspace_bytes(T, S, H, bb);
    return VLF_OK;
}

const char *vlf_forward_kernel(int32_t br, int32_t prerotate, int32_t window, int32_t max_len) {
    if (!supported_br(br) || window < 0 || max_len < 0)
        return "";
    if (prerotate)
        return br == 256 ? "attend_pre_ph" : "attend_pre";
    int32_t back, ahead;
    window_reaches(window, back, ahead);
    if (br == 256 && ring_holds(back, ahead, max_len))
        return "attend_slide";
    return br == 64 ? "attend_one" : "attend_fwd";
}

// Checks shared by the three launching calls. `work`: the call launches something (pointers
// are checked only then); `need_ws`: the call cannot run without a workspace.
static int check_launch(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                        int32_t max_len, const int32_t *cu_dev, int32_t T, int32_t S, int32_t H,
                        int32_t dtype, const void *workspace, int64_t ws_bytes, bool work,
                        bool need_ws) {
    if (dtype != VLF_BF16 && dtype != VLF_F16)
        return fail(VLF_EUNSUPPORTED, "dtype = %d; supported: VLF_F16 (0), VLF_BF16 (1)", dtype);
    if (H < 1 || H > 65536)
        return fail(VLF_EINVAL, "H = %d outside 1 .. 65536", H);
    if (T < 0 || S < 0 || table_rows < 0 || max_len < 0)
        return fail(VLF_EINVAL, "negative size: T=%d S=%d table_rows=%d max_len=%d", T, S,
                    table_rows, max_len);
    if (max_len > T)
        return fail(VLF_EINVAL, "max_len = %d above T = %d", max_len, T);
    if (T > 0 && S == 0)
        return fail(VLF_EINVAL, "T = %d tokens but no sequence", T);
    if ((int64_t)T * 3 * H * 64 > ((int64_t)1 << 40))
        return fail(VLF_EINVAL, "qkv of %lld elements is beyond this library's indexing",
                    (long long)T * 3 * H * 64);
    if (ws_bytes < 0)
        return fail(VLF_EINVAL, "workspace_bytes = %lld < 0", (long long)ws_bytes);
    if (!workspace && ws_bytes > 0)
        return fail(VLF_EINVAL, "workspace_bytes = %lld without a workspace",
                    (long long)ws_bytes);
    if (need_ws && !workspace && work)
        return fail(VLF_EINVAL, "this call needs a workspace");
    if (((uintptr_t)workspace & 15) != 0)
        return fail(VLF_EINVAL, "workspace %p is not 16-byte aligned", workspace);
    if (workspace && ws_bytes < workspace_bytes(T, S, H))
        return fail(VLF_EINVAL, "workspace of %lld bytes; T=%d S=%d H=%d need %lld",
                    (long long)ws_bytes, T, S, H, (long long)workspace_bytes(T, S, H));
    if (!work)
        return VLF_OK;
    if (!qkv || !cos || !sin || !cu_dev)
        return fail(VLF_EINVAL, "null device pointer (qkv=%p cos=%p sin=%p cu=%p)", qkv, cos,
                    sin, (const void *)cu_dev);
    if (table_rows == 0)
        return fail(VLF_EINVAL, "empty rotary tables with %d tokens", T);
    if (table_rows < max_len)
        return fail(VLF_EINVAL, "rotary tables have %d rows; the longest sequence has %d",
                    table_rows, max_len);
    return VLF_OK;
}

static int attend_common(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                         int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                         int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                         int32_t window, float scale, int32_t dtype, const void *workspace,
                         int64_t ws_bytes, void *out, float *lse, void *stream, Launch what) {
    if (dtype != VLF_BF16 && dtype != VLF_F16)
        return fail(VLF_EUNSUPPORTED, "dtype = %d; supported: VLF_F16 (0), VLF_BF16 (1)", dtype);
    if (!supported_br(br))
        return fail(VLF_EUNSUPPORTED, "br = %d; supported: 64, 128, 256", br);
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    if (num_tiles < 0)
        return fail(VLF_EINVAL, "negative size: num_tiles=%d", num_tiles);
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(VLF_EINVAL, "scale is not finite");
    const bool work = T > 0 && num_tiles > 0;
    int rc = check_launch(qkv, cos, sin, table_rows, max_len, cu_dev, T, S, H, dtype, workspace,
                          ws_bytes, work, what == Launch::kRotated);
    if (rc)
        return rc;
    if (!work)
        return VLF_OK;
    if (!tiles_dev || !out || !lse)
        return fail(VLF_EINVAL, "null device pointer (tiles=%p out=%p lse=%p)",
                    (const void *)tiles_dev, out, (void *)lse);
    int32_t back, ahead;
    window_reaches(window, back, ahead);
    AttendArgs a{qkv,    cos,   sin,   table_rows, max_len, cu_dev, tiles_dev, num_tiles,
                 br,     T,     S,     H,          back,    ahead,  scale,
                 dtype,  const_cast<void *>(workspace), out, lse, stream};
    return launch_attend(a, what);
}

int vlf_attend(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
               int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
               int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H, int32_t window,
               float scale, int32_t dtype, void *workspace, int64_t workspace_bytes_, void *out,
               float *lse, void *stream) {
    return attend_common(qkv, cos, sin, table_rows, max_len, cu_dev, tiles_dev, num_tiles, br, T,
                         S, H, window, scale, dtype, workspace, workspace_bytes_, out, lse, stream,
                         workspace ? Launch::kBoth : Launch::kDirect);
}

int vlf_attend_static(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                      int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                      int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                      int32_t window, float scale, int32_t dtype, void *out, float *lse,
                      void *stream) {
    if (T < 0 || S < 0 || H < 1 || H > 65536)
        return fail(VLF_EINVAL, "T = %d, S = %d, H = %d", T, S, H);
    const int64_t need = workspace_bytes(T, S, H);
    if (need > VLF_STATIC_WORKSPACE_BYTES)
        return fail(VLF_EINVAL,
                    "the key-tile workspace of %lld bytes (T=%d S=%d H=%d) exceeds the static "
                    "array of %lld bytes; use vlf_attend with a workspace of its own",
                    (long long)need, T, S, H, (long long)VLF_STATIC_WORKSPACE_BYTES);
    void *ws = nullptr;
    int64_t ws_bytes = 0;
    if (T > 0 && num_tiles > 0) {
        const int rc = static_scratch(&ws);
        if (rc)
            return rc;
        ws_bytes = VLF_STATIC_WORKSPACE_BYTES;
    }
    return attend_common(qkv, cos, sin, table_rows, max_len, cu_dev, tiles_dev, num_tiles, br, T,
                         S, H, window, scale, dtype, ws, ws_bytes, out, lse, stream,
                         Launch::kBoth);
}

int vlf_attend_rotated(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                       int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                       int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                       int32_t window, float scale, int32_t dtype, const void *workspace,
                       int64_t workspace_bytes_, void *out, float *lse, void *stream) {
    return attend_common(qkv, cos, sin, table_rows, max_len, cu_dev, tiles_dev, num_tiles, br, T,
                         S, H, window, scale, dtype, workspace, workspace_bytes_, out, lse, stream,
                         Launch::kRotated);
}

int vlf_backward_workspace_bytes(int32_t T, int32_t S, int32_t H, int32_t br, int64_t *bytes) {
    if (!bytes)
        return fail(VLF_EINVAL, "null bytes");
    if (T < 0 || S < 0 || H < 0 || H > 65536)
        return fail(VLF_EINVAL, "T = %d, S = %d, H = %d", T, S, H);
    if (!supported_br(br))
        return fail(VLF_EINVAL, "br = %d; the backward runs on 64-, 128- or 256-row tiles", br);
    *bytes = backward_workspace_bytes(T, S, H, br);
    return VLF_OK;
}

int vlf_attend_backward(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                        int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                        int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H,
                        int32_t window, float scale, int32_t dtype, const void *out,
                        const void *dout, const float *lse, void *workspace,
                        int64_t workspace_bytes_, void *dqkv, void *stream) {
    if (dtype != VLF_BF16 && dtype != VLF_F16)
        return fail(VLF_EUNSUPPORTED, "dtype = %d; supported: VLF_F16 (0), VLF_BF16 (1)", dtype);
    if (window < 0)
        return fail(VLF_EINVAL, "window = %d < 0", window);
    if (num_tiles < 0)
        return fail(VLF_EINVAL, "negative size: num_tiles=%d", num_tiles);
    if (br != 64 && br != 128 && br != 256)
        return fail(VLF_EINVAL, "br = %d; the backward runs on 64-, 128- or 256-row tiles", br);
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(VLF_EINVAL, "scale is not finite");
    const bool work = T > 0 && num_tiles > 0;
    // the forward's checks, without its workspace (this call's workspace is checked below)
    int rc = check_launch(qkv, cos, sin, table_rows, max_len, cu_dev, T, S, H, dtype, nullptr, 0,
                          work, false);
    if (rc)
        return rc;
    if (workspace_bytes_ < 0)
        return fail(VLF_EINVAL, "workspace_bytes = %lld < 0", (long long)workspace_bytes_);
    if (!work)
        return VLF_OK;
    if (((uintptr_t)workspace & 15) != 0)
        return fail(VLF_EINVAL, "workspace %p is not 16-byte aligned", workspace);
    if (!workspace || workspace_bytes_ < backward_workspace_bytes(T, S, H, br))
        return fail(VLF_EINVAL, "workspace of %lld bytes; T=%d S=%d H=%d br=%d need %lld",
                    (long long)(workspace ? workspace_bytes_ : 0), T, S, H, br,
                    (long long)backward_workspace_bytes(T, S, H, br));
    if (!tiles_dev || !out || !dout || !lse || !dqkv)
        return fail(VLF_EINVAL, "null device pointer (tiles=%p out=%p dout=%p lse=%p dqkv=%p)",
                    (const void *)tiles_dev, out, dout, (const void *)lse, dqkv);
    int32_t back, ahead;
    window_reaches(window, back, ahead);
    BackArgs a{qkv,  cos,   sin,   table_rows, cu_dev, tiles_dev, num_tiles, br,  T,
               S,    H,     back,  ahead,      scale,  dtype,     out,       dout, lse,
               workspace, dqkv, stream};
    return launch_backward(a);
}

int vlf_rotate_qkv(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                   int32_t max_len, const int32_t *cu_dev, const uint32_t *tiles_dev,
                   int32_t num_tiles, int32_t br, int32_t T, int32_t S, int32_t H, float scale,
                   int32_t dtype, void *qkv_out, void *stream) {
    if (num_tiles < 0)
        return fail(VLF_EINVAL, "negative size: num_tiles=%d", num_tiles);
    if (br != 64 && br != 128 && br != 256)
        return fail(VLF_EINVAL, "br = %d; tiles of 64, 128 or 256 rows", br);
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(VLF_EINVAL, "scale is not finite");
    const bool work = T > 0 && num_tiles > 0;
    int rc = check_launch(qkv, cos, sin, table_rows, max_len, cu_dev, T, S, H, dtype, nullptr, 0,
                          work, false);
    if (rc || !work)
        return rc;
    if (!tiles_dev || !qkv_out)
        return fail(VLF_EINVAL, "null device pointer (tiles=%p qkv_out=%p)",
                    (const void *)tiles_dev, qkv_out);
    if (qkv_out == qkv)
        return fail(VLF_EINVAL, "qkv_out must not be qkv");
    RotateArgs a{qkv, cos, sin, table_rows, cu_dev, tiles_dev, num_tiles, br, T,
                 S,   H,   scale, dtype,    qkv_out, stream};
    return launch_rotate_qkv(a);
}

int vlf_rotate_keys(const void *qkv, const void *cos, const void *sin, int32_t table_rows,
                    int32_t max_len, const int32_t *cu_dev, int32_t T, int32_t S, int32_t H,
                    int32_t dtype, void *workspace, int64_t workspace_bytes_, void *stream) {
    int rc = check_launch(qkv, cos, sin, table_rows, max_len, cu_dev, T, S, H, dtype, workspace,
                          workspace_bytes_, T > 0, true);
    if (rc || T == 0)
        return rc;
    AttendArgs a{qkv, cos, sin, table_rows, max_len, cu_dev,    nullptr, 0,       0, T,
                 S,   H,   0,   0,          1.f,     dtype,     workspace, nullptr, nullptr, stream};
    return launch_attend(a, Launch::kRotate);
}

}  // extern "C"
