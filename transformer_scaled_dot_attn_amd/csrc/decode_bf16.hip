// bfloat16 decode: one query per (b, h) against a KV cache, split over keys.
//
// Decode reads the whole valid cache and does little arithmetic per byte
// ("Attention from First Principles", section 6: a matrix-vector product
// whose intensity is about 1 for multi-head attention), so this path is
// built for HBM bandwidth, not for the matrix cores:
//   * partial kernel: one block per (b, K/V head, group of HB query heads,
//     split of `chunk` keys).  With grouped key/value heads (GQA / MQA:
//     query head h reads K/V head h / (H / H_kv), "Attention from First
//     Principles", section "MHA, GQA, MQA -- the KV cache lever") the block
//     scores each K/V row against all HB query heads it serves, so K and V
//     are read once per group instead of once per query head -- the rise in
//     decode intensity to H / H_kv that the same page's section 6 derives.
//     Each key
//     row (d bf16 = 2d bytes) is read by d/8 lanes with one 16-byte load
//     each, so every wave-wide load covers whole contiguous rows.  Logits use
//     v_dot2 on the raw bf16 pairs (exact products, fp32 sums), reduced over
//     the row's lanes with DPP.  K and V are read once, with non-temporal
//     loads; each lane keeps two steps of 4 rows in flight.  Each lane group keeps a running maximum m,
//     normaliser l and an fp32 accumulator for its 8 columns (the online
//     softmax recurrence); the block merges its groups in LDS and writes one
//     (m, l, acc[d]) partial.  Keys past the valid length are never loaded.
//   * combine kernel: per (b, h), merges the partials with the log-sum-exp
//     rule  M = max m_s,  l = sum l_s 2^(m_s - M),
//     out = (sum acc_s 2^(m_s - M)) / l, and rounds to bf16.  L_b = 0 gives 0.
// Logits are kept in base 2 (scale * log2 e folded in), which leaves the
// softmax unchanged.
#include "device_common.h"
#include "launch.h"

namespace tsda {

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;  // key rows per lane per step (two steps in flight)

template <int D, int HB>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ kv_lens, int H, int Hkv,
    int Skv, float scale_log2, int chunk, int nsplit, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml) {
    constexpr int G = D / 8;            // lanes per key row
    constexpr int KPW = 64 / G;         // key rows per wave per load
    constexpr int SLOTS = kWaves * KPW; // key rows per block per load
    __shared__ float s_m[HB][SLOTS];
    __shared__ float s_l[HB][SLOTS];
    __shared__ float s_acc[SLOTS][D];

    const int unit = blockIdx.x;
    const int gunit = unit / nsplit;  // (b, K/V head, query-head group)
    const int split = unit - gunit * nsplit;
    const int group = H / Hkv;        // query heads per K/V head
    const int ngrp = group / HB;      // blocks per K/V head
    const int bk = gunit / ngrp;      // b * Hkv + K/V head
    const int hg = gunit - bk * ngrp;
    const int b = bk / Hkv;
    const int h0 = (bk - b * Hkv) * group + hg * HB;  // first query head served
    const int L = valid_length(kv_lens, b, Skv);
    const int k0 = split * chunk;
    if (k0 >= L) return;  // the combine kernel reads only splits below L
    const int k1 = min(k0 + chunk, L);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int slot = (tid >> 6) * KPW + lane / G;
    const int part = lane % G;

    u32x4 qw[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i) qw[i] = ldg16(q + ((size_t)b * H + h0 + i) * D + part * 8);
    const uint16_t* kp = k + (size_t)bk * Skv * D + part * 8;
    const uint16_t* vp = v + (size_t)bk * Skv * D + part * 8;

    float m[HB], l[HB];
    float acc[HB][8];
#pragma unroll
    for (int i = 0; i < HB; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
    }

    // Rows of one step: base + u*SLOTS + slot for u < kUnroll.  Loads are
    // branch-free (a row past k1 is redirected to row k0, which is valid, and
    // its logit is masked), so the next step's loads stay in flight while the
    // current step is computed.
    constexpr int kStep = SLOTS * kUnroll;
    auto load = [&](int base, u32x4 (&kr)[kUnroll], u32x4 (&vr)[kUnroll]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = base + u * SLOTS + slot;
            const size_t row = (size_t)(j < k1 ? j : k0) * D;
            kr[u] = ldg16_stream(kp + row);
            vr[u] = ldg16_stream(vp + row);
        }
    };
    auto consume = [&](int base, const u32x4 (&kr)[kUnroll], const u32x4 (&vr)[kUnroll]) {
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            float s[kUnroll];
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float dot = 0.0f;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    dot = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kr[u][c]), as_bf16x2(qw[i][c]),
                                                          dot, false);
                dot = group_sum<G>(dot);
                const int j = base + u * SLOTS + slot;
                s[u] = j < k1 ? dot * scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[u]);
            }
            const float m_new = fmaxf(m[i], mx);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = fast_exp2(m[i] - m_use);
            l[i] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float pw = fast_exp2(s[u] - m_use);
                l[i] += pw;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc[i][2 * c] = fmaf(pw, bf16_lo(vr[u][c]), acc[i][2 * c]);
                    acc[i][2 * c + 1] = fmaf(pw, bf16_hi(vr[u][c]), acc[i][2 * c + 1]);
                }
            }
            m[i] = m_new;
        }
    };
    u32x4 ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
    load(k0, ka, va);
    for (int base = k0; base < k1; base += 2 * kStep) {
        if (base + kStep < k1) load(base + kStep, kb, vb);
        consume(base, ka, va);
        if (base + kStep >= k1) break;
        if (base + 2 * kStep < k1) load(base + 2 * kStep, ka, va);
        consume(base + kStep, kb, vb);
    }

    // merge the block's SLOTS row groups, one query head at a time
    if (part == 0) {
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            s_m[i][slot] = m[i];
            s_l[i][slot] = l[i];
        }
    }
#pragma unroll
    for (int i = 0; i < HB; ++i) {
        if (i > 0) __syncthreads();  // the previous head's merge has read s_acc
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[slot][part * 8 + e] = acc[i][e];
        __syncthreads();
        if (tid < D) {
            float M = -INFINITY;
#pragma unroll
            for (int s2 = 0; s2 < SLOTS; ++s2) M = fmaxf(M, s_m[i][s2]);
            float lt = 0.0f, at = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < SLOTS; ++s2) {
                const float w = s_m[i][s2] == -INFINITY ? 0.0f : fast_exp2(s_m[i][s2] - M);
                lt = fmaf(s_l[i][s2], w, lt);
                at = fmaf(s_acc[s2][tid], w, at);
            }
            const size_t uq = ((size_t)b * H + h0 + i) * nsplit + split;  // partial of head h0+i
            ws_acc[uq * D + tid] = at;
            if (tid == 0) {
                ws_ml[uq * 2] = M;
                ws_ml[uq * 2 + 1] = lt;
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(2 * D) void decode_combine_kernel(
    const int32_t* __restrict__ kv_lens, int H, int Skv, int chunk, int nsplit,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, uint16_t* __restrict__ out) {
    // Two halves of the block each merge every other split of one (b, h)
    // (independent loads, unrolled), then one thread per column merges the
    // two halves.
    __shared__ float s_m[2], s_l[2];
    __shared__ float s_a[2][D];
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int t = threadIdx.x % D;
    const int h2 = threadIdx.x / D;
    const int L = valid_length(kv_lens, b, Skv);
    uint16_t* o = out + (size_t)bh * D;
    if (L == 0) {
        if (h2 == 0) o[t] = 0;
        return;
    }
    const int nv = (L + chunk - 1) / chunk;
    const float* ml = ws_ml + (size_t)bh * nsplit * 2;
    const float* ac = ws_acc + (size_t)bh * nsplit * D;
    float M = -INFINITY;
#pragma unroll 4
    for (int s = h2; s < nv; s += 2) M = fmaxf(M, ml[2 * s]);
    float lt = 0.0f, at = 0.0f;
#pragma unroll 4
    for (int s = h2; s < nv; s += 2) {
        const float w = fast_exp2(ml[2 * s] - M);
        lt = fmaf(ml[2 * s + 1], w, lt);
        at = fmaf(ac[(size_t)s * D + t], w, at);
    }
    if (t == 0) {
        s_m[h2] = M;
        s_l[h2] = lt;
    }
    s_a[h2][t] = at;
    __syncthreads();
    if (h2 == 0) {
        // a half with no split has M = -inf and contributes nothing
        const float Mt = fmaxf(s_m[0], s_m[1]);
        const float w0 = s_m[0] == -INFINITY ? 0.0f : fast_exp2(s_m[0] - Mt);
        const float w1 = s_m[1] == -INFINITY ? 0.0f : fast_exp2(s_m[1] - Mt);
        const float l = s_l[0] * w0 + s_l[1] * w1;
        o[t] = to_bf16((s_a[0][t] * w0 + s_a[1][t] * w1) / l);
    }
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int decode_heads_per_block(int H, int Hkv) {
    const int group = H / Hkv;
    for (int hb = 8; hb > 1; hb >>= 1)
        if (group % hb == 0) return hb;
    return 1;
}

DecodePlan decode_plan(int B, int H, int Hkv, int Skv) {
    // Multi-head: splits of 128 keys (64 KiB of K+V at d = 128) measured
    // fastest on the ragged decode workload: many short units spread the
    // reads of the valid prefixes of all caches evenly over the memory
    // system.  Smaller problems split finer so the grid still fills the GPU.
    // A block serving several query heads does several times the vector work
    // per row and merges one partial per head at its end, so it takes the
    // longest split (up to 1024 keys) that still leaves 8 blocks per CU:
    // 1024 measured 1.25x faster than 128 at 8 K/V heads.
    const int hb = decode_heads_per_block(H, Hkv);
    const long groups = (long)B * Hkv * (H / Hkv / hb);
    int chunk = 128;
    if (hb > 1) {
        while (chunk < 1024 && groups * ((Skv + 2 * chunk - 1) / (2 * chunk)) >= 2048) chunk *= 2;
    } else if (groups * ((Skv + chunk - 1) / chunk) < 8192) {
        chunk = 64;
    }
    return DecodePlan{chunk, (Skv + chunk - 1) / chunk};
}

size_t decode_workspace_bytes(int B, int H, int Hkv, int Skv, int d) {
    const DecodePlan p = decode_plan(B, H, Hkv, Skv);
    const size_t units = (size_t)B * H * p.nsplit;  // one partial per query head and split
    return round256(units * d * sizeof(float)) + round256(units * 2 * sizeof(float));
}

namespace {

template <int D, int HB>
void launch_partial(const LaunchArgs& a, const DecodePlan& p, float sl, float* ws_acc,
                    float* ws_ml) {
    const size_t blocks = (size_t)a.B * a.H / HB * p.nsplit;
    hipLaunchKernelGGL((decode_partial_kernel<D, HB>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       a.kv_lens, a.H, a.Hkv, a.Skv, sl, p.chunk, p.nsplit, ws_acc, ws_ml);
}

template <int D>
void launch_partial_d(const LaunchArgs& a, const DecodePlan& p, float sl, float* ws_acc,
                      float* ws_ml) {
    switch (decode_heads_per_block(a.H, a.Hkv)) {
        case 8: launch_partial<D, 8>(a, p, sl, ws_acc, ws_ml); break;
        case 4: launch_partial<D, 4>(a, p, sl, ws_acc, ws_ml); break;
        case 2: launch_partial<D, 2>(a, p, sl, ws_acc, ws_ml); break;
        default: launch_partial<D, 1>(a, p, sl, ws_acc, ws_ml); break;
    }
}

}  // namespace

hipError_t launch_decode_bf16(const LaunchArgs& a) {
    const DecodePlan p = decode_plan(a.B, a.H, a.Hkv, a.Skv);
    const size_t units = (size_t)a.B * a.H * p.nsplit;
    float* ws_acc = static_cast<float*>(a.workspace);
    float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                            round256(units * a.d * sizeof(float)));
    uint16_t* o = static_cast<uint16_t*>(a.out);
    const float sl = a.scale * kLog2e;
    KernelTimer* t = active_timer();
    hipError_t e;
    if (t) t->begin(kDecodePartialBf16, a.stream);
    if (a.d == 128)
        launch_partial_d<128>(a, p, sl, ws_acc, ws_ml);
    else
        launch_partial_d<64>(a, p, sl, ws_acc, ws_ml);
    e = hipGetLastError();
    if (t) t->end(kDecodePartialBf16, a.stream);
    if (e != hipSuccess) return e;
    if (t) t->begin(kDecodeCombineBf16, a.stream);
    const unsigned pairs = (unsigned)((size_t)a.B * a.H);
    if (a.d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(pairs), dim3(256), 0, a.stream,
                           a.kv_lens, a.H, a.Skv, p.chunk, p.nsplit, ws_acc, ws_ml, o);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(pairs), dim3(128), 0, a.stream,
                           a.kv_lens, a.H, a.Skv, p.chunk, p.nsplit, ws_acc, ws_ml, o);
    e = hipGetLastError();
    if (t) t->end(kDecodeCombineBf16, a.stream);
    return e;
}

}  // namespace tsda
