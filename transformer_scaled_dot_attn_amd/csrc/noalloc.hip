// Allocation-free entry point: attn_fwd_ex with its temporary memory taken
// from a fixed device array instead of a workspace, for callers that may not
// allocate device memory (code under stream capture, tight serving loops).
//
// The array lives in the library's code object, so every device the library
// runs on holds one copy of it from load until the process ends.  Its device
// address differs per device: host code never names the array itself (in
// host code that name is only a stand-in), it uses the address that
// hipGetSymbolAddress returned on that device, taken once per device with
// the device current.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn.h"
#include "launch.h"

namespace tsda {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];  // device address of `scratch` on each device, once taken

// Address of the current device's copy of the array (set-up on first use).
int scratch_address(void** out) {
    int dev = -1;
    if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return launch_status(e);
    if (dev < 0 || dev >= kMaxDevices) return ATTN_E_UNSUPPORTED;
    std::lock_guard<std::mutex> g(g_mu);
    if (g_addr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return launch_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
        }
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return ATTN_OK;
}

}  // namespace
}  // namespace tsda

using namespace tsda;

extern "C" {

size_t attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H,
                     int H_kv, int Sq, int Skv, int d, int d_v, float scale, int causal,
                     const int32_t* kv_lens, const uint8_t* mask, int64_t mask_sb,
                     int64_t mask_sh, int64_t mask_si, int dtype, void* stream) {
    int st = attn_validate_ex(q, k, v, out, B, H, H_kv, Sq, Skv, d, d_v, scale, causal, mask,
                              mask_sb, mask_sh, mask_si, dtype);
    if (st != ATTN_OK) return st;
    const size_t need =
        attn_workspace_bytes_ex(B, H, H_kv, Sq, Skv, d, d_v, dtype, mask != nullptr ? 1 : 0);
    if (need > kScratchBytes) return ATTN_E_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != ATTN_OK) return st;
    }
    return run_with_workspace(q, k, v, out, B, H, H_kv, Sq, Skv, d, d_v, scale, causal, kv_lens,
                              mask, mask_sb, mask_sh, mask_si, dtype, stream, ws,
                              need > 0 ? kScratchBytes : 0);
}

}  // extern "C"
