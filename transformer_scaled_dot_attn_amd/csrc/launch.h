// Internal interface between the C-ABI front end and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tsda {

struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int B, H, Hkv, Sq, Skv, d;  // Hkv key/value heads; query head h reads K/V head h / (H / Hkv)
    int dv;                     // value / output width
    float scale;
    int causal;
    const int32_t* kv_lens;
    hipStream_t stream;
    void* workspace;
    size_t workspace_bytes;
    // optional allowed-mask: byte (b, h, i, j) at mask[b*msb + h*msh + i*msi + j],
    // nonzero = visible; 4-byte aligned, strides multiples of 4 (checked by the
    // front end), each row readable up to Skv rounded up to 4.  nullptr: none.
    const uint8_t* mask;
    long long msb, msh, msi;
    // optional additive bias, elements of the inputs' type: element (b, h, i,
    // j) at bias[b*bsb + h*bsh + i*bsi + j], added to the scaled logit; -inf
    // hides the key.  16-byte aligned, strides multiples of 4 (checked by the
    // front end), each row readable up to Skv rounded up to 4.  nullptr: none.
    const void* bias;
    long long bsb, bsh, bsi;
};

// Last 4-element group offset of a bias row that a kernel may read.
__host__ __device__ inline int bias_last_group(int Skv) { return ((Skv + 3) & ~3) - 4; }

// Last 4-byte word offset of a mask row that a kernel may read.
__host__ __device__ inline int mask_last_word(int Skv) { return ((Skv + 3) & ~3) - 4; }

// Decode workspace: the stream kernel's partials and pair spans; with an
// allowed-mask, plus decode_mask_workspace_bytes for the pairs' visible-tile
// counts and lists.
size_t decode_workspace_bytes(int B, int H, int Hkv, int Skv, int d, int dv);
size_t decode_mask_workspace_bytes(int B, int H, int Hkv, int Skv, int d, int dv);

// Prefill plan: key-range splits per query tile (1 = none, no workspace).
struct PrefillPlan {
    int nsplit;  // key-range splits per query tile (1: none)
    int bm;      // query rows per block: 256, or 128 / 64 on small unsplit grids
    int kg;      // key groups per block: 2 splits each block's keys between two wave sets
};
// masked: an allowed-mask is given; general: a bias, or a scale that is not positive
PrefillPlan prefill_plan(int B, int H, int Sq, int Skv, int d = 128, int dv = 128,
                         bool masked = false, bool general = false);
size_t prefill_workspace_bytes(int B, int H, int Sq, int Skv, int dv);  // dv: partial width
// extra bytes a masked prefill needs for its key-tile marks (after the above)
size_t prefill_mask_workspace_bytes(int B, int Sq, int Skv);

inline size_t round_up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Profiling hook: the front end brackets each launch when timing is on.
struct KernelTimer {
    virtual void begin(int kernel, hipStream_t s) = 0;
    virtual void end(int kernel, hipStream_t s) = 0;
    virtual ~KernelTimer() = default;
};
KernelTimer* active_timer();  // nullptr when timing is off

enum KernelId { kPrefillBf16 = 0, kDecodePartialBf16 = 1, kDecodeCombineBf16 = 2, kGenericF32 = 3,
                kPrefillCombineBf16 = 4, kPrefillMaskTiles = 5, kDecodeMaskTiles = 6,
                kNumKernels = 7 };

// ATTN_OK for hipSuccess; otherwise records e as this thread's last HIP
// error (attn_last_hip_error) and returns ATTN_E_LAUNCH.
int launch_status(hipError_t e);

// attn_fwd_ex on a caller-supplied workspace (checks, kernel choice, launch).
int run_with_workspace(const void* q, const void* k, const void* v, void* out, int B, int H,
                       int Hkv, int Sq, int Skv, int d, int dv, float scale, int causal,
                       const int32_t* kv_lens, const uint8_t* mask, int64_t msb, int64_t msh,
                       int64_t msi, int dtype, void* stream, void* workspace,
                       size_t workspace_bytes);

hipError_t launch_generic_f32(const LaunchArgs& a);
hipError_t launch_prefill_bf16(const LaunchArgs& a);
hipError_t launch_decode_bf16(const LaunchArgs& a);

}  // namespace tsda
