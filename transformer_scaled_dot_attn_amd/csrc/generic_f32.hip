// Float32 attention forward on the vector ALUs (any d, d_v <= 128, any Sq <= Skv).
//
// One wavefront per block and one query row per lane; the block's 64 query
// rows share K/V tiles of 32 keys staged in LDS (every lane reads the same
// LDS word, a broadcast).  Per tile each lane computes its 32 logits, then
// updates its running maximum m and normaliser l and rescales its output
// accumulator once (the online-softmax recurrence), so the score matrix is
// never materialised ("Scaled dot-product attention with masking", section
// "The memory problem").  Keys past the valid length are never read; rows
// past the valid query count are written as zeros.  With grouped key/value
// heads, query head h reads K/V head h / (H / Hkv) ("Attention from First
// Principles", section "MHA, GQA, MQA -- the KV cache lever").  An
// explicit allowed-mask (MASK: a byte per query row and key, nonzero =
// visible, ANDed with the causal and length rules) is read as eight 4-byte
// words of the lane's row per tile; a row with no visible key is 0.  The
// value width d_v may differ from d (the d_v != d_k case of "Attention from
// Scratch", KubeDojo module 1.4.3, Part 2): K rows have d features, V and
// output rows d_v.  An additive bias (the float mask of that page's Part 7,
// added to the scaled logits; -inf hides the key) is read as eight 16-byte
// groups of the lane's row per tile.  The kernel keeps the maximum of the
// scaled logits, so any finite scale works.
#include "device_common.h"
#include "launch.h"

namespace tsda {

namespace {

constexpr int kRows = 64;   // query rows per block
constexpr int kKeys = 32;   // keys per LDS tile

template <int DP, int DPV, bool MASK>  // DP, DPV: d, d_v rounded up to 16, 32, 64 or 128
__global__ __launch_bounds__(64) void generic_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ out, const int32_t* __restrict__ kv_lens, int H, int Hkv, int Sq, int Skv,
    int d, int dv, float scale_log2, int causal, const uint8_t* __restrict__ mask, long long msb,
    long long msh, long long msi, const float* __restrict__ bias, long long bsb, long long bsh,
    long long bsi) {
    __shared__ float ks[kKeys][DP];
    __shared__ float vs[kKeys][DPV];

    const int lane = threadIdx.x;
    const int nqt = (Sq + kRows - 1) / kRows;
    const int bh = blockIdx.x / nqt;
    const int b = bh / H;
    const int L = valid_length(kv_lens, b, Skv);
    const int n = Sq < L ? Sq : L;
    const int row0 = (blockIdx.x - bh * nqt) * kRows;
    const int i = row0 + lane;
    const bool live = i < n;
    const int p = L - n + i;  // absolute position of this lane's query

    // keys any row of this block may see
    int kv_hi = L;
    if (causal) {
        const int last = (row0 + kRows < n ? row0 + kRows : n) - 1;
        kv_hi = min(L, L - n + last + 1);
    }
    if (row0 >= n) kv_hi = 0;

    float qr[DP];
    float acc[DPV];
    const float* qrow = q + ((size_t)bh * Sq + (live ? i : 0)) * d;
#pragma unroll
    for (int c = 0; c < DP; ++c) qr[c] = (live && c < d) ? qrow[c] : 0.0f;
#pragma unroll
    for (int c = 0; c < DPV; ++c) acc[c] = 0.0f;
    float m = -INFINITY, l = 0.0f;

    const int bk = b * Hkv + (bh - b * H) / (H / Hkv);  // this head's K/V head
    const uint8_t* mrow = nullptr;  // this lane's allowed-mask row
    if constexpr (MASK)
        mrow = mask + b * msb + (long long)(bh - b * H) * msh + (long long)(live ? i : 0) * msi;
    const int mlast = mask_last_word(Skv);
    // this lane's bias row (groups past the row's end are clamped: their keys
    // are >= Skv >= L and hidden)
    const float* brow = nullptr;
    if (bias != nullptr)
        brow = bias + b * bsb + (long long)(bh - b * H) * bsh + (long long)(live ? i : 0) * bsi;
    const int blast = bias_last_group(Skv);
    const float* kb = k + (size_t)bk * Skv * d;
    const float* vb = v + (size_t)bk * Skv * dv;
    for (int j0 = 0; j0 < kv_hi; j0 += kKeys) {
        const int nk = min(kKeys, kv_hi - j0);
        __syncthreads();
        // stage the tile: the tile is contiguous in global memory
        for (int e = lane; e < kKeys * d; e += 64) {
            const int r = e / d, c = e - r * d;
            ks[r][c] = r < nk ? kb[(size_t)j0 * d + e] : 0.0f;
        }
        for (int e = lane; e < kKeys * dv; e += 64) {
            const int r = e / dv, c = e - r * dv;
            vs[r][c] = r < nk ? vb[(size_t)j0 * dv + e] : 0.0f;
        }
        if (d < DP) {
            for (int e = lane; e < kKeys * (DP - d); e += 64) {
                const int r = e / (DP - d), c = d + e - r * (DP - d);
                ks[r][c] = 0.0f;
            }
        }
        if (dv < DPV) {
            for (int e = lane; e < kKeys * (DPV - dv); e += 64) {
                const int r = e / (DPV - dv), c = dv + e - r * (DPV - dv);
                vs[r][c] = 0.0f;
            }
        }
        __syncthreads();

        uint32_t mbits = ~0u;  // bit r: the mask allows key j0 + r
        if constexpr (MASK) {
            // words past the row's end are clamped (their keys are >= Skv >= L)
#pragma unroll
            for (int w = 0; w < kKeys / 4; ++w) {
                const uint32_t word = ldg_word(mrow + min(j0 + 4 * w, mlast));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!byte_set(word, e)) mbits &= ~(1u << (4 * w + e));
            }
        }
        f32x4 bw[kKeys / 4];  // the bias of keys j0 + 4 w .. +3, times log2 e
#pragma unroll
        for (int w = 0; w < kKeys / 4; ++w) bw[w] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (brow != nullptr) {
#pragma unroll
            for (int w = 0; w < kKeys / 4; ++w)
                bw[w] = *reinterpret_cast<const f32x4*>(brow + min(j0 + 4 * w, blast)) * kLog2e;
        }
        float s[kKeys];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            float dot = 0.0f;
#pragma unroll
            for (int c = 0; c < DP; ++c) dot = fmaf(qr[c], ks[r][c], dot);
            const int j = j0 + r;
            bool vis = r < nk && (!causal || j <= p);
            if constexpr (MASK) vis = vis & (((mbits >> r) & 1u) != 0);  // no short circuit: keeps the loop straight-line
            s[r] = vis ? fmaf(dot, scale_log2, bw[r >> 2][r & 3]) : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m - m_use);
        l *= alpha;
#pragma unroll
        for (int c = 0; c < DPV; ++c) acc[c] *= alpha;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            const float pr = fast_exp2(s[r] - m_use);
            l += pr;
#pragma unroll
            for (int c = 0; c < DPV; ++c) acc[c] = fmaf(pr, vs[r][c], acc[c]);
        }
        m = m_new;
    }

    if (i < Sq) {
        float* orow = out + ((size_t)bh * Sq + i) * dv;
        const float inv = (live && l > 0.0f) ? 1.0f / l : 0.0f;
#pragma unroll
        for (int c = 0; c < DPV; ++c)
            if (c < dv) orow[c] = live ? acc[c] * inv : 0.0f;
    }
}

// Calls go(generic_f32_kernel<16 << wd, 16 << wv, mask>) for run-time
// width indices wd, wv in 0..3 and the mask flag.
template <int WD = 0, int WV = 0, class Go>
void dispatch(Go&& go, int wd, int wv, bool mask) {
    if constexpr (WD < 3) {
        if (wd > WD) return dispatch<WD + 1, WV>(go, wd, wv, mask);
    }
    if constexpr (WV < 3) {
        if (wv > WV) return dispatch<WD, WV + 1>(go, wd, wv, mask);
    }
    constexpr int DP = 16 << WD, DPV = 16 << WV;
    mask ? go(generic_f32_kernel<DP, DPV, true>) : go(generic_f32_kernel<DP, DPV, false>);
}

}  // namespace

hipError_t launch_generic_f32(const LaunchArgs& a) {
    dim3 grid((unsigned)(((a.Sq + kRows - 1) / kRows) * (long)a.B * a.H));
    dim3 block(64);
    const float sl = a.scale * kLog2e;
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.out);
    KernelTimer* t = active_timer();
    if (t) t->begin(kGenericF32, a.stream);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, a.stream, q, k, v, o, a.kv_lens, a.H, a.Hkv, a.Sq,
                           a.Skv, a.d, a.dv, sl, a.causal, a.mask, a.msb, a.msh, a.msi,
                           static_cast<const float*>(a.bias), a.bsb, a.bsh, a.bsi);
    };
    // d and d_v rounded up to 16, 32, 64 or 128 (d, d_v <= 128 is checked by the front end)
    auto width = [](int x) { return x <= 16 ? 0 : x <= 32 ? 1 : x <= 64 ? 2 : 3; };
    dispatch(go, width(a.d), width(a.dv), a.mask != nullptr);
    hipError_t e = hipGetLastError();
    if (t) t->end(kGenericF32, a.stream);
    return e;
}

}  // namespace tsda
