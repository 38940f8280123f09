// gdn_prefill_ex_noalloc: gdn_prefill_ex with its workspace in a static device array of
// the library instead of caller memory, for callers that cannot allocate (see gdn.h).
//
// The array lives in the library's code object: every device the library runs on holds
// its own copy (allocated when the code object is loaded there) until the process ends.
// On the host the name `scratch` is only a stand-in for the symbol, never a device
// address; the address is obtained once per device with hipGetSymbolAddress, with that
// device current, and used everywhere the kernels need the buffer.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(128) << 20;   // the documented maximum
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of the array, looked up on the first call made with it current.
gdn_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GDN_ERR_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GDN_OK;
}

}  // namespace

namespace gdn {
// (gdn_api.cpp) the workspace of one prefill call, for its own packing and fusion; 0 for
// arguments that gdn_prefill_ex rejects
size_t prefill_call_workspace_bytes(const gdn_params* p, const gdn_fusion* fusion, int B, int L, int N, int chunk,
                                    bool ragged);
}  // namespace gdn

extern "C" gdn_status gdn_prefill_ex_noalloc(const gdn_params* p, const gdn_fusion* fusion, int32_t B,
                                             int32_t L, const void* qkv, const void* gate,
                                             const void* beta, const void* conv_weight,
                                             const void* conv_state_in, void* conv_state_out,
                                             float* S, float* o, const int32_t* cu_seqlens,
                                             int32_t N, int32_t chunk, void* stream) {
    // 0 for arguments gdn_prefill_ex rejects: it reports them itself below
    const size_t need = gdn::prefill_call_workspace_bytes(p, fusion, B, L, N, chunk, cu_seqlens != nullptr);
    if (need > kScratchBytes) return GDN_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (need > 0) {
        const gdn_status st = scratch_of_current_device(&ws);
        if (st != GDN_OK) return st;
    }
    return gdn_prefill_ex(p, fusion, B, L, qkv, gate, beta, conv_weight, conv_state_in, conv_state_out,
                          S, o, cu_seqlens, N, chunk, ws, need > 0 ? kScratchBytes : 0, stream);
}
