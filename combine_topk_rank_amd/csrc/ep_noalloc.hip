// ep_noalloc.hip — the one-call dispatch (routing layout + pack + descriptor
// emission) for callers that cannot allocate device memory: code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation.
//
// It is ep_dispatch_fused with its workspace taken from a file-scope device
// array instead of an argument.  The array's name is only a host-side stand-in
// for device memory: host code must never pass it to a kernel.  The first call
// on each device looks up the array's device address on that device with
// hipGetSymbolAddress (each GPU holds its own copy) and from then on passes
// only that address.  Nothing here allocates: no hipMalloc, hipFree or
// allocating library routine.

#include <mutex>

#include "ep_common.h"

namespace ep {
namespace {

// Largest workspace the array serves (ep_workspace_bytes of the shape); the
// train and skewed workloads need under 200 KB.
constexpr size_t kScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;

}  // namespace
}  // namespace ep

// One per device; zero-filled by the first call on the device, kept until
// the process ends.
static __device__ __align__(256) uint8_t scratch[ep::kScratchBytes];

namespace ep {
namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];      // device address of `scratch` on each device
bool g_cleared[kMaxDevices];       // its zero fill has been enqueued

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = uint4{0, 0, 0, 0};
}

// The current device's scratch address, zero-filled on `stream` before its
// first use on the device or when `clear` is set.
int device_scratch(hipStream_t stream, bool clear, void** out) {
    int dev = 0;
    EP_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) {
        record_error("ep_dispatch_fused_noalloc: device index beyond the library's table");
        return EP_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        EP_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        g_scratch[dev] = p;
    }
    if (clear || !g_cleared[dev]) {
        clear_hip_error();
        hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream,
                           reinterpret_cast<uint4*>(g_scratch[dev]), kScratchBytes / 16);
        EP_HIP_CHECK(hipGetLastError());
        g_cleared[dev] = true;
    }
    *out = g_scratch[dev];
    return EP_OK;
}

}  // namespace
}  // namespace ep

using namespace ep;

extern "C" int ep_dispatch_fused_noalloc(
    const ep_shape_t* shape, const void* x, const int32_t* topk_idx, const float* topk_w,
    int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert, int32_t* rank_offset,
    int32_t* expert_offset, uint8_t* is_token_in_rank, int32_t* send_slot, void* send_buf,
    int64_t capacity_rows, int32_t* slot_src, int32_t* slot_local_idx, float* slot_local_w,
    ep_ring_t* ring, int32_t clear_scratch, int32_t* dev_status, hipStream_t stream) {
    const int v = validate_shape(shape);
    if (v != EP_OK) return v;
    if (workspace_bytes(*shape) > kScratchBytes) {
        record_error("ep_dispatch_fused_noalloc: the shape needs more than the 4 MiB of "
                     "device scratch this call owns; use ep_dispatch_fused with a workspace");
        return EP_ERR_INVALID_ARG;
    }
    void* ws = nullptr;
    const int st = device_scratch(stream, clear_scratch != 0, &ws);
    if (st != EP_OK) return st;
    return ep_dispatch_fused(shape, x, topk_idx, topk_w, num_tokens_per_rank,
                             num_tokens_per_expert, rank_offset, expert_offset, is_token_in_rank,
                             send_slot, send_buf, capacity_rows, slot_src, slot_local_idx,
                             slot_local_w, ring, ws, kScratchBytes, dev_status, stream);
}
