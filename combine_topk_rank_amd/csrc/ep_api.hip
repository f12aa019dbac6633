// ep_api.hip — host-side helpers of the C ABI: shape validation, row sizes,
// workspace layout and status strings.

#include <stdio.h>

#include "ep_common.h"

namespace ep {

namespace {
thread_local char g_last_error[256] = "";
}

void record_hip_error(hipError_t e, const char* what) {
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

void record_error(const char* what) { snprintf(g_last_error, sizeof g_last_error, "%s", what); }

size_t row_bytes(int32_t H, int32_t fmt) {
    if (fmt == EP_FMT_BF16) return (size_t)2 * H;
    // H code bytes, one float scale per 128 elements, then zero bytes up to a
    // whole number of 128-byte lines, so that rows never share a cache line
    return ((size_t)H + (size_t)4 * (H / 128) + 127) / 128 * 128;
}

int validate_shape(const ep_shape_t* p) {
    if (!p) return EP_ERR_INVALID_ARG;
    const ep_shape_t& s = *p;
    if (s.T < 0 || s.H < 8 || s.H % 8 != 0 || s.H > kMaxH) return EP_ERR_INVALID_ARG;
    if (s.fmt != EP_FMT_BF16 && s.fmt != EP_FMT_FP8_E4M3_B128) return EP_ERR_INVALID_ARG;
    if (s.fmt == EP_FMT_FP8_E4M3_B128 && s.H % 128 != 0) return EP_ERR_INVALID_ARG;
    if (s.R < 1 || s.R > kMaxR || s.E < 1 || s.E > kMaxE || s.E % s.R != 0) return EP_ERR_INVALID_ARG;
    if (s.k < 1 || s.k > kMaxK || s.k > s.E) return EP_ERR_INVALID_ARG;
    const int64_t m = s.k > s.R ? s.k : s.R;
    if ((int64_t)s.T * m >= ((int64_t)1 << 31)) return EP_ERR_INVALID_ARG;
    if ((int64_t)s.T * (s.H / 8) >= ((int64_t)1 << 40)) return EP_ERR_INVALID_ARG;
    return EP_OK;
}

namespace {
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
}

size_t workspace_bytes(const ep_shape_t& s) {
    const int64_t nb = layout_blocks(s.T);
    size_t b = kWsHeader;                      // barrier words, arrival counters
    b += align256((size_t)nb * s.R * 4);       // blk_rank_cnt
    b += align256((size_t)nb * s.E * 4);       // blk_exp_cnt
    b += align256((size_t)wave_blocks(s.T) * s.R * 4);   // wave_rank_cnt
    b += align256((size_t)(s.R + 1) * 4);      // msg_base
    b += align256((size_t)(max_messages(s) + s.E) * 4);   // msg_arrivals + msgs_done
    return b;
}

Workspace carve_workspace(const ep_shape_t& s, void* base) {
    Workspace w{};
    uint8_t* p = reinterpret_cast<uint8_t*>(base);
    const int64_t nb = layout_blocks(s.T);
    w.layout_blocks = (int32_t)nb;
    w.barrier = reinterpret_cast<uint32_t*>(p);
    w.arrive = reinterpret_cast<uint32_t*>(p + kBarrierBytes);
    p += kWsHeader;
    w.blk_rank_cnt = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)nb * s.R * 4);
    w.blk_exp_cnt = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)nb * s.E * 4);
    w.wave_rank_cnt = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)wave_blocks(s.T) * s.R * 4);
    w.msg_base = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)(s.R + 1) * 4);
    w.max_msgs = max_messages(s);
    w.msg_arrivals = reinterpret_cast<int32_t*>(p);
    w.msgs_done = w.msg_arrivals + w.max_msgs;
    w.counters_n = w.max_msgs + s.E;
    return w;
}

}  // namespace ep

using namespace ep;

extern "C" size_t ep_row_bytes(int32_t H, int32_t fmt) {
    if (H < 8 || H % 8 != 0) return 0;
    if (fmt == EP_FMT_FP8_E4M3_B128 && H % 128 != 0) return 0;
    if (fmt != EP_FMT_BF16 && fmt != EP_FMT_FP8_E4M3_B128) return 0;
    return row_bytes(H, fmt);
}

extern "C" size_t ep_workspace_bytes(const ep_shape_t* shape) {
    if (validate_shape(shape) != EP_OK) return 0;
    return workspace_bytes(*shape);
}

extern "C" const char* ep_last_error(void) { return g_last_error; }

extern "C" const char* ep_status_str(int st) {
    switch (st) {
        case EP_OK: return "ok";
        case EP_ERR_INVALID_ARG: return "invalid argument";
        case EP_ERR_BAD_EXPERT: return "expert id out of range";
        case EP_ERR_CAPACITY: return "send buffer capacity exceeded";
        case EP_ERR_RING_TIMEOUT: return "transfer ring full for longer than its timeout";
        case EP_ERR_HIP: return "HIP runtime error";
        case EP_ERR_BUSY: return "ring busy (proxy threads running)";
        case EP_ERR_TIMEOUT: return "a device-side wait for other workgroups timed out";
        default: return "unknown status";
    }
}
