// noalloc.hip -- attn_decode_noalloc: the decode entry point for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its kernels are attn_decode's; the
// per-share partial records they need go to a fixed device array that the
// library holds for the life of the process instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_internal.h"
#include "sdpa_flash.h"

namespace {

// Largest workspace the entry point serves: 32 MiB (for instance the fp16
// decode of 64 entries x 8 kv heads x 4-head groups at head dim 128 needs
// 5.4 MiB).  Every GPU the library runs on holds one copy until the process
// ends.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];          // device address of `scratch` on each device
hipError_t g_status[kMaxDevices];

}  // namespace

extern "C" attn_status attn_decode_noalloc(const attn_problem* p, const void* q, const void* k,
                                           const void* v, void* o, const float* mask,
                                           const int32_t* key_lens, float* lse, void* stream) {
    size_t need = 0;
    const attn_status st = attn_workspace_size(p, ATTN_OP_DECODE, &need);
    if (st != ATTN_OK) return st;
    if (need > kScratchBytes)
        return sdpa::set_error(ATTN_ERR_WORKSPACE,
                               "decode needs %zu workspace bytes, more than the %zu this entry "
                               "point holds; use attn_decode with a workspace",
                               need, kScratchBytes);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return sdpa::set_error(ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return sdpa::set_error(ATTN_ERR_UNSUPPORTED, "device %d is beyond the %d this entry point "
                                                     "serves", dev, kMaxDevices);
    // Once per device, with that device current: the address of this device's
    // copy of the array (the array's name is only a host-side stand-in).
    std::call_once(g_once[dev], [dev] {
        g_status[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    });
    if (g_status[dev] != hipSuccess)
        return sdpa::set_error(ATTN_ERR_HIP, "hipGetSymbolAddress: %s",
                               hipGetErrorString(g_status[dev]));
    return attn_decode(p, q, k, v, o, mask, key_lens, lse, g_scratch[dev], kScratchBytes, stream);
}
