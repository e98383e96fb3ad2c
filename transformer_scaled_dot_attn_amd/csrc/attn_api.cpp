// C-ABI front end: argument checks, kernel choice, workspace, timing.
//
// The checks are a pure host function (attn_validate) that runs before any
// HIP call.  Requests outside the kernels' support matrix are refused with
// ATTN_E_UNSUPPORTED instead of running a slower path without saying so
// ("Attention from First Principles", section 8, on silent kernel
// fallbacks).  Prefill and decode get different kernels, since their shapes
// and bottlenecks are opposite (same page, sections 6 and 8).
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "attn.h"
#include "launch.h"

namespace tsda {

// HIP error behind this thread's last ATTN_E_LAUNCH (hipSuccess: none yet)
thread_local hipError_t g_last_hip = hipSuccess;

int launch_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    g_last_hip = e;
    return ATTN_E_LAUNCH;
}

namespace {

enum Path { kPathNone = -1, kPathGenericF32 = 0, kPathPrefill = 1, kPathDecode = 2 };

Path choose_path(int Sq, int d, int dtype, int dv) {
    if (dtype == ATTN_F32) return d <= 128 && dv <= 128 ? kPathGenericF32 : kPathNone;
    if (dtype == ATTN_BF16 && (d == 64 || d == 128) && (dv == 64 || dv == 128))
        return Sq == 1 ? kPathDecode : kPathPrefill;
    return kPathNone;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int B, int H, int Hkv, int Sq, int Skv, int d, int dv) {
    if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || d <= 0 || dv <= 0 || Sq > Skv)
        return ATTN_E_SHAPE;
    if (Hkv <= 0 || H % Hkv != 0) return ATTN_E_SHAPE;
    // element counts of the q/k/v tensors and the launch grids must stay in range
    const long double kv = (long double)B * H * Skv * (d > dv ? d : dv);  // >= every tensor's count
    if (kv > (long double)(INT64_MAX / 8)) return ATTN_E_SHAPE;
    const long double rows = (long double)B * H * ((Sq + 63) / 64);
    if (rows > (long double)INT_MAX) return ATTN_E_SHAPE;
    const long double splits = (long double)B * H * ((Skv + 63) / 64);
    if (splits > (long double)INT_MAX) return ATTN_E_SHAPE;
    return ATTN_OK;
}

// Library-owned workspaces, one per (device, stream): calls on different
// streams never share temporary memory, and calls on one stream are ordered
// by the stream itself.
struct StreamWorkspace {
    int device;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
};
std::mutex g_ws_mu;
std::vector<StreamWorkspace> g_ws;

// ---- timing -------------------------------------------------------------
struct Record {
    int kernel;
    hipEvent_t start, stop;
};

class EventTimer final : public KernelTimer {
  public:
    void begin(int kernel, hipStream_t s) override {
        std::lock_guard<std::mutex> g(mu_);
        Record r{kernel, take(), take()};
        (void)hipEventRecord(r.start, s);
        open_.push_back(r);
    }
    void end(int kernel, hipStream_t s) override {
        std::lock_guard<std::mutex> g(mu_);
        for (size_t i = open_.size(); i-- > 0;) {
            if (open_[i].kernel == kernel) {
                (void)hipEventRecord(open_[i].stop, s);
                done_.push_back(open_[i]);
                open_.erase(open_.begin() + i);
                return;
            }
        }
    }
    int read(int kernel, long* launches, double* total_ms) {
        std::lock_guard<std::mutex> g(mu_);
        long n = 0;
        double ms = 0.0;
        for (const Record& r : done_) {
            if (r.kernel != kernel) continue;
            if (const hipError_t e = hipEventSynchronize(r.stop); e != hipSuccess)
                return launch_status(e);
            float t = 0.0f;
            if (const hipError_t e = hipEventElapsedTime(&t, r.start, r.stop); e != hipSuccess)
                return launch_status(e);
            ms += t;
            ++n;
        }
        if (launches) *launches = n;
        if (total_ms) *total_ms = ms;
        return ATTN_OK;
    }
    // Durations (ms) of the first `cap` recorded launches of `kernel`, in
    // launch order; *n receives the number of recorded launches.
    int samples(int kernel, double* ms_out, long cap, long* n_out) {
        std::lock_guard<std::mutex> g(mu_);
        long n = 0;
        for (const Record& r : done_) {
            if (r.kernel != kernel) continue;
            if (n < cap && ms_out != nullptr) {
                if (const hipError_t e = hipEventSynchronize(r.stop); e != hipSuccess)
                    return launch_status(e);
                float t = 0.0f;
                if (const hipError_t e = hipEventElapsedTime(&t, r.start, r.stop); e != hipSuccess)
                    return launch_status(e);
                ms_out[n] = t;
            }
            ++n;
        }
        if (n_out) *n_out = n;
        return ATTN_OK;
    }
    void reset() {
        std::lock_guard<std::mutex> g(mu_);
        for (Record& r : done_) { give(r.start); give(r.stop); }
        for (Record& r : open_) { give(r.start); give(r.stop); }
        done_.clear();
        open_.clear();
    }
    ~EventTimer() override {
        reset();
        for (hipEvent_t e : pool_) (void)hipEventDestroy(e);
    }

  private:
    hipEvent_t take() {
        if (!pool_.empty()) {
            hipEvent_t e = pool_.back();
            pool_.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        (void)hipEventCreate(&e);
        return e;
    }
    void give(hipEvent_t e) {
        if (e) pool_.push_back(e);
    }
    std::mutex mu_;
    std::vector<Record> open_, done_;
    std::vector<hipEvent_t> pool_;
};

// Launches read these without the lock: the timer is created once (under it)
// and never freed, and the switch is a flag.
std::atomic<EventTimer*> g_timer{nullptr};
std::atomic<bool> g_timing_on{false};
std::mutex g_timer_mu;

// Allowed-mask layout checks: strides >= 0 and multiples of 4, base 4-byte
// aligned, every byte offset a kernel may touch representable.
int check_mask(const uint8_t* mask, int64_t sb, int64_t sh, int64_t si, int B, int H, int Sq,
               int Skv) {
    if (mask == nullptr) return ATTN_OK;
    if (sb < 0 || sh < 0 || si < 0) return ATTN_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(mask) & 3u) != 0 || (sb & 3) || (sh & 3) || (si & 3))
        return ATTN_E_ALIGN;
    const long double last = (long double)sb * (B - 1) + (long double)sh * (H - 1) +
                             (long double)si * (Sq - 1) + (long double)Skv + 3;
    if (last > (long double)(INT64_MAX / 2)) return ATTN_E_SHAPE;
    // the prefill kernel addresses a wave's 32 rows as 32-bit offsets
    if ((long double)si * 32 + Skv + 4 > (long double)UINT32_MAX) return ATTN_E_UNSUPPORTED;
    return ATTN_OK;
}

// Additive-bias layout checks: strides >= 0 and multiples of 4 elements,
// base 16-byte aligned, every element offset a kernel may touch
// representable, and a wave's 32 rows addressable with 32-bit byte offsets.
int check_bias(const void* bias, int64_t sb, int64_t sh, int64_t si, int B, int H, int Sq,
               int Skv, int elem) {
    if (bias == nullptr) return ATTN_OK;
    if (sb < 0 || sh < 0 || si < 0) return ATTN_E_SHAPE;
    if (!aligned16(bias) || (sb & 3) || (sh & 3) || (si & 3)) return ATTN_E_ALIGN;
    const long double last = (long double)sb * (B - 1) + (long double)sh * (H - 1) +
                             (long double)si * (Sq - 1) + (long double)Skv + 3;
    if (last * elem > (long double)(INT64_MAX / 2)) return ATTN_E_SHAPE;
    if (((long double)si * 32 + Skv + 4) * elem > (long double)UINT32_MAX)
        return ATTN_E_UNSUPPORTED;
    return ATTN_OK;
}

// Every host-side check of attn_fwd_bias (and so of attn_fwd_ex), in the
// documented order.
int validate_all(const void* q, const void* k, const void* v, void* out, int B, int H, int Hkv,
                 int Sq, int Skv, int d, int dv, float scale, int dtype, const uint8_t* mask,
                 int64_t msb, int64_t msh, int64_t msi, const void* bias = nullptr,
                 int64_t bsb = 0, int64_t bsh = 0, int64_t bsi = 0) {
    if (!q || !k || !v || !out) return ATTN_E_NULL;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_E_DTYPE;
    int st = check_shape(B, H, Hkv, Sq, Skv, d, dv);
    if (st != ATTN_OK) return st;
    if (!std::isfinite(scale)) return ATTN_E_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_E_ALIGN;
    if (choose_path(Sq, d, dtype, dv) == kPathNone) return ATTN_E_UNSUPPORTED;
    // the bf16 kernels address a head's K and V rows with 32-bit byte offsets
    if (dtype == ATTN_BF16 && (long double)Skv * (d > dv ? d : dv) * 2 > (long double)UINT32_MAX)
        return ATTN_E_UNSUPPORTED;
    st = check_mask(mask, msb, msh, msi, B, H, Sq, Skv);
    if (st != ATTN_OK) return st;
    return check_bias(bias, bsb, bsh, bsi, B, H, Sq, Skv, dtype == ATTN_F32 ? 4 : 2);
}

int run(const void* q, const void* k, const void* v, void* out, int B, int H, int Hkv, int Sq,
        int Skv, int d, float scale, int causal, const int32_t* kv_lens, int dtype, void* stream,
        void* workspace, size_t workspace_bytes, bool library_ws, const uint8_t* mask = nullptr,
        int64_t msb = 0, int64_t msh = 0, int64_t msi = 0, int dv = -1,
        const void* bias = nullptr, int64_t bsb = 0, int64_t bsh = 0, int64_t bsi = 0) {
    if (dv < 0) dv = d;
    int st = validate_all(q, k, v, out, B, H, Hkv, Sq, Skv, d, dv, scale, dtype, mask, msb, msh,
                          msi, bias, bsb, bsh, bsi);
    if (st != ATTN_OK) return st;
    const Path path = choose_path(Sq, d, dtype, dv);
    const size_t need = attn_workspace_bytes_ex(B, H, Hkv, Sq, Skv, d, dv, dtype, mask != nullptr);
    if (library_ws) {
        workspace = nullptr;
        if (need > 0) {
            int dev = 0;
            if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return launch_status(e);
            const hipStream_t hs = static_cast<hipStream_t>(stream);
            std::lock_guard<std::mutex> g(g_ws_mu);
            StreamWorkspace* w = nullptr;
            for (StreamWorkspace& x : g_ws)
                if (x.device == dev && x.stream == hs) w = &x;
            if (w == nullptr) {
                g_ws.push_back(StreamWorkspace{dev, hs, nullptr, 0});
                w = &g_ws.back();
            }
            if (w->bytes < need) {
                // earlier calls on this stream may still be using the old buffer
                if (const hipError_t e = hipStreamSynchronize(hs); e != hipSuccess)
                    return launch_status(e);
                if (w->ptr) (void)hipFree(w->ptr);
                w->ptr = nullptr;
                w->bytes = 0;
                if (hipMalloc(&w->ptr, need) != hipSuccess) {
                    w->ptr = nullptr;
                    return ATTN_E_NOMEM;
                }
                w->bytes = need;
            }
            workspace = w->ptr;
            workspace_bytes = w->bytes;
        }
    } else {
        if (workspace_bytes < need) return ATTN_E_WORKSPACE;
        if (need > 0 && (workspace == nullptr)) return ATTN_E_NULL;
        if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_E_ALIGN;
    }
    LaunchArgs a{q, k, v, out, B, H, Hkv, Sq, Skv, d, dv, scale, causal ? 1 : 0, kv_lens,
                 static_cast<hipStream_t>(stream), workspace, workspace_bytes, mask, msb, msh,
                 msi, bias, bsb, bsh, bsi};
    hipError_t e = hipSuccess;
    switch (path) {
        case kPathGenericF32: e = launch_generic_f32(a); break;
        case kPathPrefill: e = launch_prefill_bf16(a); break;
        case kPathDecode: e = launch_decode_bf16(a); break;
        default: return ATTN_E_UNSUPPORTED;
    }
    return launch_status(e);
}

}  // namespace

int run_with_workspace(const void* q, const void* k, const void* v, void* out, int B, int H,
                       int Hkv, int Sq, int Skv, int d, int dv, float scale, int causal,
                       const int32_t* kv_lens, const uint8_t* mask, int64_t msb, int64_t msh,
                       int64_t msi, int dtype, void* stream, void* workspace,
                       size_t workspace_bytes) {
    return run(q, k, v, out, B, H, Hkv, Sq, Skv, d, scale, causal, kv_lens, dtype, stream,
               workspace, workspace_bytes, false, mask, msb, msh, msi, dv);
}

KernelTimer* active_timer() {
    return g_timing_on.load(std::memory_order_acquire) ? g_timer.load(std::memory_order_acquire)
                                                       : nullptr;
}

}  // namespace tsda

using namespace tsda;

extern "C" {

int attn_validate_gqa(const void* q, const void* k, const void* v, void* out, int B, int H,
                      int Hkv, int Sq, int Skv, int d, float scale, int causal, int dtype) {
    (void)causal;
    return validate_all(q, k, v, out, B, H, Hkv, Sq, Skv, d, d, scale, dtype, nullptr, 0, 0, 0);
}

int attn_validate(const void* q, const void* k, const void* v, void* out, int B, int H, int Sq,
                  int Skv, int d, float scale, int causal, int dtype) {
    return attn_validate_gqa(q, k, v, out, B, H, H, Sq, Skv, d, scale, causal, dtype);
}

const char* attn_kernel_for(int Sq, int Skv, int d, int dtype) {
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return nullptr;
    if (check_shape(1, 1, 1, Sq, Skv, d, d) != ATTN_OK) return nullptr;
    switch (choose_path(Sq, d, dtype, d)) {
        case kPathGenericF32: return "generic_f32";
        case kPathPrefill: return "prefill_bf16_mfma";
        case kPathDecode: return "decode_bf16_stream";
        default: return nullptr;
    }
}

size_t attn_workspace_bytes_gqa(int B, int H, int Hkv, int Sq, int Skv, int d, int dtype) {
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
    if (check_shape(B, H, Hkv, Sq, Skv, d, d) != ATTN_OK) return 0;
    switch (choose_path(Sq, d, dtype, d)) {
        case kPathDecode: return decode_workspace_bytes(B, H, Hkv, Skv, d, d);
        case kPathPrefill: return prefill_workspace_bytes(B, H, Sq, Skv, d);
        default: return 0;
    }
}

size_t attn_workspace_bytes_ex(int B, int H, int Hkv, int Sq, int Skv, int d, int dv, int dtype,
                               int masked) {
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
    if (check_shape(B, H, Hkv, Sq, Skv, d, dv) != ATTN_OK) return 0;
    switch (choose_path(Sq, d, dtype, dv)) {
        case kPathDecode:
            return decode_workspace_bytes(B, H, Hkv, Skv, d, dv) +
                   (masked ? decode_mask_workspace_bytes(B, H, Hkv, Skv, d, dv) : 0);
        case kPathPrefill:
            return prefill_workspace_bytes(B, H, Sq, Skv, dv) +
                   (masked ? prefill_mask_workspace_bytes(B, Sq, Skv) : 0);
        default: return 0;
    }
}

size_t attn_workspace_bytes(int B, int H, int Sq, int Skv, int d, int dtype) {
    return attn_workspace_bytes_gqa(B, H, H, Sq, Skv, d, dtype);
}

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, int B, int H, int Hkv,
                 int Sq, int Skv, int d, float scale, int causal, const int32_t* kv_lens,
                 int dtype, void* stream) {
    return run(q, k, v, out, B, H, Hkv, Sq, Skv, d, scale, causal, kv_lens, dtype, stream,
               nullptr, 0, true);
}

int attn_fwd_gqa_ws(const void* q, const void* k, const void* v, void* out, int B, int H,
                    int Hkv, int Sq, int Skv, int d, float scale, int causal,
                    const int32_t* kv_lens, int dtype, void* stream, void* workspace,
                    size_t workspace_bytes) {
    return run(q, k, v, out, B, H, Hkv, Sq, Skv, d, scale, causal, kv_lens, dtype, stream,
               workspace, workspace_bytes, false);
}

int attn_validate_ex(const void* q, const void* k, const void* v, void* out, int B, int H,
                     int Hkv, int Sq, int Skv, int d, int dv, float scale, int causal,
                     const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int64_t mask_si,
                     int dtype) {
    (void)causal;
    return validate_all(q, k, v, out, B, H, Hkv, Sq, Skv, d, dv, scale, dtype, mask, mask_sb,
                        mask_sh, mask_si);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int Hkv,
                int Sq, int Skv, int d, int dv, float scale, int causal, const int32_t* kv_lens,
                const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int64_t mask_si, int dtype,
                void* stream, void* workspace, size_t workspace_bytes) {
    return run(q, k, v, out, B, H, Hkv, Sq, Skv, d, scale, causal, kv_lens, dtype, stream,
               workspace, workspace_bytes, workspace == nullptr, mask, mask_sb, mask_sh, mask_si,
               dv);
}

int attn_validate_bias(const void* q, const void* k, const void* v, void* out, int B, int H,
                       int Hkv, int Sq, int Skv, int d, int dv, float scale, int causal,
                       const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int64_t mask_si,
                       const void* bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_si,
                       int dtype) {
    (void)causal;
    return validate_all(q, k, v, out, B, H, Hkv, Sq, Skv, d, dv, scale, dtype, mask, mask_sb,
                        mask_sh, mask_si, bias, bias_sb, bias_sh, bias_si);
}

int attn_fwd_bias(const void* q, const void* k, const void* v, void* out, int B, int H, int Hkv,
                  int Sq, int Skv, int d, int dv, float scale, int causal,
                  const int32_t* kv_lens, const uint8_t* mask, int64_t mask_sb, int64_t mask_sh,
                  int64_t mask_si, const void* bias, int64_t bias_sb, int64_t bias_sh,
                  int64_t bias_si, int dtype, void* stream, void* workspace,
                  size_t workspace_bytes) {
    return run(q, k, v, out, B, H, Hkv, Sq, Skv, d, scale, causal, kv_lens, dtype, stream,
               workspace, workspace_bytes, workspace == nullptr, mask, mask_sb, mask_sh, mask_si,
               dv, bias, bias_sb, bias_sh, bias_si);
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int Sq,
             int Skv, int d, float scale, int causal, const int32_t* kv_lens, int dtype,
             void* stream) {
    return run(q, k, v, out, B, H, H, Sq, Skv, d, scale, causal, kv_lens, dtype, stream, nullptr,
               0, true);
}

int attn_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int Sq,
                int Skv, int d, float scale, int causal, const int32_t* kv_lens, int dtype,
                void* stream, void* workspace, size_t workspace_bytes) {
    return run(q, k, v, out, B, H, H, Sq, Skv, d, scale, causal, kv_lens, dtype, stream,
               workspace, workspace_bytes, false);
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_E_NULL: return "null pointer argument";
        case ATTN_E_SHAPE:
            return "invalid shape (a size <= 0, Sq > Skv, H not a multiple of H_kv, or too large)";
        case ATTN_E_UNSUPPORTED:
            return "unsupported combination of dtype and head sizes (or mask row stride)";
        case ATTN_E_DTYPE: return "unknown dtype";
        case ATTN_E_ALIGN:
            return "pointer not aligned (16 bytes; workspace 256 bytes; mask and its strides 4 "
                   "bytes; bias strides 4 elements)";
        case ATTN_E_WORKSPACE: return "workspace too small";
        case ATTN_E_ARG: return "scale is not finite";
        case ATTN_E_LAUNCH: return "HIP launch or runtime failure";
        case ATTN_E_NOMEM: return "device allocation failed";
        case ATTN_E_SCRATCH:
            return "problem needs more temporary memory than the fixed scratch area "
                   "(attn_noalloc_scratch_bytes) holds";
        default: return "unknown status";
    }
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

int attn_last_hip_error(void) { return static_cast<int>(g_last_hip); }

int attn_prefill_plan(int B, int H, int H_kv, int Sq, int Skv, int d, int d_v, int masked,
                      int general, int* key_splits, int* rows_per_block, int* key_groups) {
    const int st = check_shape(B, H, H_kv, Sq, Skv, d, d_v);
    if (st != ATTN_OK) return st;
    if (choose_path(Sq, d, ATTN_BF16, d_v) != kPathPrefill) return ATTN_E_UNSUPPORTED;
    const PrefillPlan p = prefill_plan(B, H, Sq, Skv, d, d_v, masked != 0, general != 0);
    if (key_splits) *key_splits = p.nsplit;
    if (rows_per_block) *rows_per_block = p.bm;
    if (key_groups) *key_groups = p.kg;
    return ATTN_OK;
}

const char* attn_last_hip_error_name(void) { return hipGetErrorName(g_last_hip); }

void attn_release(void) {
    std::lock_guard<std::mutex> g(g_ws_mu);
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (StreamWorkspace& w : g_ws) {
        if (w.ptr) {
            (void)hipSetDevice(w.device);
            (void)hipFree(w.ptr);
        }
    }
    g_ws.clear();
    if (have_cur) (void)hipSetDevice(cur);
}

int attn_profile_enable(int on) {
    std::lock_guard<std::mutex> g(g_timer_mu);
    if (!g_timer.load()) g_timer.store(new EventTimer(), std::memory_order_release);
    g_timer.load()->reset();
    g_timing_on.store(on != 0, std::memory_order_release);
    return ATTN_OK;
}

int attn_profile_reset(void) {
    std::lock_guard<std::mutex> g(g_timer_mu);
    if (EventTimer* tm = g_timer.load()) tm->reset();
    return ATTN_OK;
}

int attn_profile_read(int kernel, long* launches, double* total_ms) {
    if (kernel < 0 || kernel >= kNumKernels) return ATTN_E_ARG;
    std::lock_guard<std::mutex> g(g_timer_mu);
    EventTimer* tm = g_timer.load();
    if (!tm) {
        if (launches) *launches = 0;
        if (total_ms) *total_ms = 0.0;
        return ATTN_OK;
    }
    return tm->read(kernel, launches, total_ms);
}

int attn_profile_samples(int kernel, double* ms, long cap, long* launches) {
    if (kernel < 0 || kernel >= kNumKernels || cap < 0) return ATTN_E_ARG;
    std::lock_guard<std::mutex> g(g_timer_mu);
    EventTimer* tm = g_timer.load();
    if (!tm) {
        if (launches) *launches = 0;
        return ATTN_OK;
    }
    return tm->samples(kernel, ms, cap, launches);
}

const char* attn_profile_name(int kernel) {
    switch (kernel) {
        case kPrefillBf16: return "prefill_bf16_mfma";
        case kDecodePartialBf16: return "decode_bf16_partial";
        case kDecodeCombineBf16: return "decode_bf16_combine";
        case kGenericF32: return "generic_f32";
        case kPrefillCombineBf16: return "prefill_bf16_combine";
        case kPrefillMaskTiles: return "prefill_mask_tiles";
        case kDecodeMaskTiles: return "decode_mask_tiles";
        default: return nullptr;
    }
}

}  // extern "C"
