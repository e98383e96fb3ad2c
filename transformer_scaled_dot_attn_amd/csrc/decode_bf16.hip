// bfloat16 decode: one query per (b, h) against a KV cache, split over keys.
//
// Decode reads the whole valid cache and does little arithmetic per byte
// ("Attention from First Principles", section 6: a matrix-vector product
// whose intensity is about 1 for multi-head attention), so this path is
// built for HBM bandwidth.  With grouped key/value heads (GQA / MQA: query
// head h reads K/V head h / (H / H_kv), same page, section "MHA, GQA, MQA --
// the KV cache lever") each K/V row serves H / H_kv query heads, the rise in
// decode intensity that section 6 derives, and the kernels read it once per
// group of query heads:
//   * stream kernel (every call without an allowed-mask): the query heads a
//     K/V head serves are the columns of 32x32 MFMA tiles (one live column
//     for multi-head attention: the loop is bound by K/V bytes either way),
//     and a fixed grid of waves shares all key tiles of all caches equally
//     (below).
//   * split kernels (calls with an allowed-mask), one unit per split of
//     `chunk` keys, so that a split the mask hides from every head it serves
//     writes an empty partial without reading its K/V rows:
//       - vector kernel (1 or 2 query heads per K/V head): one block per
//         (b, K/V head, group of HB query heads, split).  Each key row
//         (d bf16 = 2d bytes) is read by d/8 lanes with one 16-byte load
//         each, so every wave-wide load covers whole contiguous rows.
//         Logits use v_dot2 on the raw bf16 pairs (exact products, fp32
//         sums), reduced over the row's lanes with DPP, once per served head.
//         K and V are read once, with non-temporal loads; each lane keeps two
//         steps of 4 rows in flight.  Each lane group keeps a running maximum
//         m, normaliser l and an fp32 accumulator for its 8 columns per head
//         (the online softmax recurrence); the block merges its groups in LDS
//         and writes one (m, l, acc[d]) partial per head.  Keys past the
//         valid length are never loaded.
//       - matrix-core split kernel (4 or more query heads per K/V head): the
//         stream kernel's loop over one split.
//   * combine kernels: per (b, h), merge the partials with the log-sum-exp
//     rule  M = max m_s,  l = sum l_s 2^(m_s - M),
//     out = (sum acc_s 2^(m_s - M)) / l, and round to bf16.  L_b = 0 gives 0.
// Logits are kept in base 2 (scale * log2 e folded in), which leaves the
// softmax unchanged.
// An explicit allowed-mask (the MASK instantiations: a byte per query head
// and key, nonzero = visible, ANDed with the length rule) is read next to
// the K/V rows it gates; a split whose keys are all hidden leaves a partial
// with m = -inf and l = 0, which the combine weighs as zero, and a head with
// no visible key at all is written as 0.  A split the mask hides entirely
// from every head it serves writes that empty partial without reading its
// K/V rows (a left-padded cache then streams only its visible keys).
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "launch.h"

namespace tsda {

namespace {

constexpr int kWaves = 4;
constexpr int kUnroll = 4;  // key rows per lane per step (two steps in flight)

template <int D, int HB, bool MASK>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ kv_lens, int H, int Hkv,
    int Skv, float scale_log2, int chunk, int nsplit, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, const uint8_t* __restrict__ mask, long long msb, long long msh) {
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
    // allowed-mask bytes: lane `part` of a row group reads the byte of query
    // head h0 + part % HB (HB <= G), and the group's lanes share them below
    const uint8_t* mrow = nullptr;
    if constexpr (MASK) {
        mrow = mask + b * msb + (long long)(h0 + part % HB) * msh;
        // does any served head see any key of the split?
        const int nk = k1 - k0;
        int vis = 0;
        for (int e = tid; e < HB * nk; e += 256) {
            const int i = e / nk;
            vis |= mask[b * msb + (long long)(h0 + i) * msh + k0 + (e - i * nk)];
        }
        if (!__syncthreads_or(vis)) {
            for (int e = tid; e < HB * D; e += 256) {
                const size_t uq = ((size_t)b * H + h0 + e / D) * nsplit + split;
                ws_acc[uq * D + e % D] = 0.0f;
                if (e % D == 0) {
                    ws_ml[uq * 2] = -INFINITY;
                    ws_ml[uq * 2 + 1] = 0.0f;
                }
            }
            return;
        }
    }

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
    auto load = [&](int base, u32x4 (&kr)[kUnroll], u32x4 (&vr)[kUnroll],
                    uint32_t (&mk)[kUnroll]) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = base + u * SLOTS + slot;
            const int jc = j < k1 ? j : k0;
            const size_t row = (size_t)jc * D;
            kr[u] = ldg16_stream(kp + row);
            vr[u] = ldg16_stream(vp + row);
            if constexpr (MASK) mk[u] = mrow[jc];
        }
    };
    const int grp0 = lane & ~(G - 1);  // first lane of this row group
    auto consume = [&](int base, const u32x4 (&kr)[kUnroll], const u32x4 (&vr)[kUnroll],
                       const uint32_t (&mk)[kUnroll]) {
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
                bool vis = j < k1;
                if constexpr (MASK) {
                    const uint32_t mb =
                        HB > 1 ? (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (grp0 + i), (int)mk[u])
                               : mk[u];
                    vis = vis & (mb != 0);
                }
                s[u] = vis ? dot * scale_log2 : -INFINITY;
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
    uint32_t ma[kUnroll], mb[kUnroll];
    load(k0, ka, va, ma);
    for (int base = k0; base < k1; base += 2 * kStep) {
        if (base + kStep < k1) load(base + kStep, kb, vb, mb);
        consume(base, ka, va, ma);
        if (base + kStep >= k1) break;
        if (base + 2 * kStep < k1) load(base + 2 * kStep, ka, va, ma);
        consume(base + kStep, kb, vb, mb);
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

// Matrix-core decode for grouped K/V heads.  The query heads a K/V head
// serves are the 32 columns of one MFMA tile (heads past the group are zero
// columns), so per 32-key tile a wave computes S^T = K Q^T with d/16
// v_mfma_f32_32x32x16_bf16 -- K from the tile staged in LDS as the A operand,
// Q^T held as the B operand -- and O^T += V^T P^T with d/16 more, V^T read
// through ds_read_b64_tr_b16 from the staged V tile.  K and V both arrive by
// whole-row, non-temporal 16-byte loads (a wave-wide load covers 1 KiB of
// contiguous rows), issued for the next tile at the top of each iteration;
// K loaded straight into the A-operand layout instead (32 bytes of each of 32
// rows per load) measured 17 % slower at 8 K/V heads.  In both accumulators a
// lane owns one query head, so the online softmax is lane-local plus one half
// swap, as in the prefill kernel.  The matrix cores have ample headroom (16
// MFMAs per 16 KiB of K+V): decode stays bound by the bytes of K and V,
// read once per group of up to 32 query heads.  A copy of the loop with its
// arithmetic removed runs no faster, so how the grid meets memory decides the
// speed.  Two kernels drive the loop:
//   * stream kernel (no allowed-mask, any number of query heads per K/V
//     head): a fixed grid of as many waves as the GPU holds at once.  The
//     (b, K/V head, head group) pairs, each cut into ceil(L_b / 32) key
//     tiles, are laid end to end and wave w takes the w-th equal share of
//     that sequence, crossing pair boundaries as it goes and writing one
//     partial per pair it touches (the stream-K decomposition of Osama et
//     al., 2023, applied to the key axis).  Every wave streams the same
//     bytes, so ragged lengths leave no part-filled last round of waves.  On
//     lengths U[512, 8192] (B = 64, H = 32), fixed splits measured 12 %
//     slower at 32 K/V heads (the vector kernel), 29 % at 16 and 20-25 % at
//     4 and 8 (the split kernel); with short caches in a large capacity
//     (lengths U[16, 512] of 8192) the vector kernel's grid of mostly empty
//     splits took 4.8x as long.
//   * split kernel (allowed-mask, 4 or more query heads per K/V head): one
//     wave per (b, K/V head, head group, split of `chunk` keys), so that a
//     split the mask hides from every head skips its K/V reads.
template <int D>
struct MfmaDecode {
    static constexpr int kKSteps = D / 16;      // MFMA k-steps of K Q^T
    static constexpr int kDBlocks = D / 32;     // 32-row blocks of O^T
    static constexpr int kStrideV = D + 16;     // padded LDS row of V (elements)
    static constexpr int kStrideK = D + 8;      // padded LDS row of K: 8 consecutive rows start in
                                                // 8 different 16-byte bank groups (A-operand reads)
    static constexpr int kChunks = D / 8;       // 16-byte chunks per row
    static constexpr int kRows = 64 / kChunks;  // K or V rows per wave-wide load
    static constexpr int kLoads = 32 / kRows;   // wave-wide loads per 32-row K or V tile
    static constexpr int kAheadK = 2;           // K operand k-steps read ahead of their MFMA
};

// Q^T fragments (B operand) of query heads h0 .. h0+31 of batch item b: lane
// l holds features 16*ks + 8*(l/32) .. +7 of head h0 + l%32 (zero when the
// lane's head is not served).
template <int D>
__device__ __forceinline__ void mfma_load_q(const uint16_t* __restrict__ q, int b, int H, int h0,
                                            bool live, u32x4 (&qf)[D / 16]) {
    const int lane = threadIdx.x;
    const uint16_t* qrow =
        q + ((size_t)b * H + h0 + (live ? (lane & 31) : 0)) * D + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = live ? ldg16(qrow + ks * 16) : u32x4{0, 0, 0, 0};
}

// Online softmax of the 32 query-head columns in qf over keys k0 .. k1-1
// (k0 < k1) of the K/V head whose rows start at kb and vb, from scratch:
// running maximum m_run (raw logit units), normaliser l_run over this lane's
// half of the keys, and the O^T accumulators.  With MASK, mrow is the
// allowed-mask row of the lane's query head (words past mlast never read).
template <int D, bool MASK>
__device__ __forceinline__ void mfma_keys(const u32x4 (&qf)[D / 16], const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int k0, int k1,
                                          float scale_log2, const uint8_t* __restrict__ mrow,
                                          int mlast, uint16_t* lds_k, uint16_t* lds_v,
                                          f32x16 (&oacc)[D / 32], float& m_run, float& l_run) {
    using C = MfmaDecode<D>;
    const int lane = threadIdx.x;
    const int half = lane >> 5;
    const int jh = lane & 31;

    // allowed-mask words of this lane's query head for a 32-key tile: word g
    // holds keys 8 g + 4 half .. +3, the keys of score elements 4 g .. +3
    // (offsets clamped to the row's last readable word; keys past it are
    // >= Skv >= L and hidden anyway)
    uint32_t mw[4], mw_next[4];
    auto load_m = [&](int t0, uint32_t (&dst)[4]) {
        if constexpr (MASK) {
#pragma unroll
            for (int g = 0; g < 4; ++g) dst[g] = ldg_word(mrow + min(t0 + 8 * g + 4 * half, mlast));
        }
    };

    // K and V tile rows whole (kRows rows per load, lane%kChunks the 16-byte
    // chunk).  Rows at or past k1 are redirected to row k0 (valid; their
    // logits are masked).
    u32x4 kr[C::kLoads], vr[C::kLoads];
    auto load_kv = [&](int t0) {
#pragma unroll
        for (int c = 0; c < C::kLoads; ++c) {
            const int row = t0 + c * C::kRows + lane / C::kChunks;
            const size_t off = (size_t)(row < k1 ? row : k0) * D + (lane % C::kChunks) * 8;
            kr[c] = ldg16_stream(kb + off);
            vr[c] = ldg16_stream(vb + off);
        }
    };
    // K operand of S^T from LDS: row lane%32, features 16*ks + 8*(lane/32)
    const int k_rd = jh * C::kStrideK + half * 8;
    //  V^T operand via ds_read_b64_tr_b16 (the prefill kernel's mapping):
    //  within each 16-lane group, source lane i reads features col0 + 4*(i%4)
    //  .. +3 of key row key0 + i/4; lanes of the second half take keys 4..7
    //  (and 12..15) of each 16-key step, matching their P^T fragment.
    const int n16 = lane & 15;
    const int v_rd =
        (4 * half + (n16 >> 2)) * C::kStrideV + 16 * ((lane >> 4) & 1) + 4 * (n16 & 3);

#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    m_run = -INFINITY;
    l_run = 0.0f;

    load_kv(k0);
    load_m(k0, mw);
    for (int t0 = k0; t0 < k1; t0 += 32) {
        // K(t0), V(t0) to LDS; the next tile's loads reuse their registers
#pragma unroll
        for (int c = 0; c < C::kLoads; ++c) {
            const int r = c * C::kRows + lane / C::kChunks, col = (lane % C::kChunks) * 8;
            *reinterpret_cast<u32x4*>(lds_k + r * C::kStrideK + col) = kr[c];
            *reinterpret_cast<u32x4*>(lds_v + r * C::kStrideV + col) = vr[c];
        }
        __syncthreads();
        const bool next = t0 + 32 < k1;
        if (next) {
            load_kv(t0 + 32);
            load_m(t0 + 32, mw_next);
        }

        // S^T = K Q^T for 32 keys x 32 heads, K operands read kAheadK ahead
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
        u32x4 ka[C::kAheadK + 1];
#pragma unroll
        for (int ks = 0; ks < C::kAheadK; ++ks)
            ka[ks] = *reinterpret_cast<const u32x4*>(lds_k + k_rd + ks * 16);
#pragma unroll
        for (int ks = 0; ks < C::kKSteps; ++ks) {
            if (ks + C::kAheadK < C::kKSteps)
                ka[(ks + C::kAheadK) % (C::kAheadK + 1)] =
                    *reinterpret_cast<const u32x4*>(lds_k + k_rd + (ks + C::kAheadK) * 16);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, ka[ks % (C::kAheadK + 1)]),
                __builtin_bit_cast(bf16x8, qf[ks]), sacc, 0, 0, 0);
        }
        bool cut = t0 + 32 > k1;
        if constexpr (MASK) {
            uint32_t z = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) z |= has_zero_byte(mw[g]);
            cut = cut || __builtin_amdgcn_ballot_w64(z != 0) != 0;
        }
        if (cut) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
                bool vis = j < k1;
                if constexpr (MASK) vis = vis & byte_set(mw[r >> 2], r & 3);  // no short circuit
                if (!vis) sacc[r] = -INFINITY;
            }
        }
        if constexpr (MASK) {
#pragma unroll
            for (int g = 0; g < 4; ++g) mw[g] = mw_next[g];
        }
        // online softmax, lazy per-lane reference (as the prefill kernel)
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        mx = halves_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const bool grow = (m_new - m_run) * scale_log2 > 8.0f;  // true if m_run = -inf
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float alpha = grow ? fast_exp2((m_run - m_new) * scale_log2) : 1.0f;
            m_run = grow ? m_new : m_run;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float mc = m_run == -INFINITY ? 0.0f : m_run * scale_log2;
        u32x4 pf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a0 = fast_exp2(fmaf(sacc[8 * h2 + 2 * i], scale_log2, -mc));
                const float a1 = fast_exp2(fmaf(sacc[8 * h2 + 2 * i + 1], scale_log2, -mc));
                pf[h2][i] = pack_bf16(a0, a1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pf[h2][i]),
                                                        as_bf16x2(0x3F803F80u), l_run, false);
            }
        // O^T += V^T P^T, output blocks innermost
#pragma unroll
        for (int st = 0; st < 2 * C::kDBlocks; ++st) {
            const int db = st % C::kDBlocks, kk = st / C::kDBlocks;
            const uint16_t* a1 = lds_v + v_rd + kk * 16 * C::kStrideV + db * 32;
            const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TSDA_LDS i16x4*)(a1));
            const i16x4 x1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((TSDA_LDS i16x4*)(a1 + 8 * C::kStrideV));
            u32x4 a;
            a[0] = (uint32_t)(uint16_t)x0[0] | ((uint32_t)(uint16_t)x0[1] << 16);
            a[1] = (uint32_t)(uint16_t)x0[2] | ((uint32_t)(uint16_t)x0[3] << 16);
            a[2] = (uint32_t)(uint16_t)x1[0] | ((uint32_t)(uint16_t)x1[1] << 16);
            a[3] = (uint32_t)(uint16_t)x1[2] | ((uint32_t)(uint16_t)x1[3] << 16);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pf[kk]), oacc[db], 0, 0,
                0);
        }
        __syncthreads();  // the K and V tiles are read before the next ones are stored
    }
}

// One partial per served query head: acc[D] at arow (the lane's head) and
// (m, l) in exp2 units at ml.  Every lane of the wave calls it.
template <int D>
__device__ __forceinline__ void mfma_write_partial(const f32x16 (&oacc)[D / 32], float m_run,
                                                   float l_run, float scale_log2, bool live,
                                                   float* __restrict__ arow,
                                                   float* __restrict__ ml) {
    const int half = threadIdx.x >> 5;
    const float l_tot = halves_sum(l_run);
    if (live) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = db * 32 + 8 * rg + 4 * half;
                const f32x4 w4 = {oacc[db][4 * rg], oacc[db][4 * rg + 1], oacc[db][4 * rg + 2],
                                  oacc[db][4 * rg + 3]};
                *reinterpret_cast<f32x4*>(arow + d0) = w4;
            }
        if (half == 0) {
            ml[0] = m_run * scale_log2;
            ml[1] = l_tot;
        }
    }
}

// Split kernel: one wavefront per (b, K/V head, group of up to 32 query
// heads, split of `chunk` keys), with an allowed-mask.
template <int D, bool MASK>
__global__ __launch_bounds__(64, 2) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ kv_lens, int H, int Hkv,
    int Skv, float scale_log2, int chunk, int nsplit, int hgroups, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, const uint8_t* __restrict__ mask, long long msb, long long msh) {
    using C = MfmaDecode<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[32 * C::kStrideV];
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[32 * C::kStrideK];

    const int lane = threadIdx.x;
    const int half = lane >> 5;
    const int unit = blockIdx.x;
    const int split = unit % nsplit;
    const int g = unit / nsplit;
    const int hgrp = g % hgroups;
    const int bk = g / hgroups;                // b * Hkv + K/V head
    const int b = bk / Hkv;
    const int group = H / Hkv;
    const int h0 = (bk - b * Hkv) * group + hgrp * 32;  // first query head served
    const int nh = min(32, group - hgrp * 32);          // query heads served
    const int L = valid_length(kv_lens, b, Skv);
    const int k0 = split * chunk;
    if (k0 >= L) return;  // the combine kernel reads only splits below L
    const int k1 = min(k0 + chunk, L);

    const int jh = lane & 31;
    const bool live = jh < nh;
    u32x4 qf[C::kKSteps];
    mfma_load_q<D>(q, b, H, h0, live, qf);
    const uint16_t* kb = k + (size_t)bk * Skv * D;
    const uint16_t* vb = v + (size_t)bk * Skv * D;

    const uint8_t* mrow = nullptr;
    if constexpr (MASK) mrow = mask + b * msb + (long long)(h0 + (live ? jh : 0)) * msh;
    const int mlast = mask_last_word(Skv);
    if constexpr (MASK) {
        if (msh == 0) {
            // a mask shared by all heads: does it open any key of the split?
            // (lane l checks the words at 4 l, 4 (l + 64), ...; keys >= k1 are
            // excluded byte by byte)
            uint32_t vis = 0;
            for (int j = k0 + 4 * lane; j < k1; j += 256) {
                const uint32_t wd = ldg_word(mask + b * msb + min(j, mlast));
#pragma unroll
                for (int e = 0; e < 4; ++e) vis |= (j + e < k1) & byte_set(wd, e);
            }
            if (__builtin_amdgcn_ballot_w64(vis != 0) == 0) {
                if (live) {
                    const size_t uq = ((size_t)b * H + h0 + jh) * nsplit + split;
                    for (int c = half; c < D; c += 2) ws_acc[uq * D + c] = 0.0f;
                    if (half == 0) {
                        ws_ml[uq * 2] = -INFINITY;
                        ws_ml[uq * 2 + 1] = 0.0f;
                    }
                }
                return;
            }
        }
    }
    f32x16 oacc[C::kDBlocks];
    float m_run, l_run;
    mfma_keys<D, MASK>(qf, kb, vb, k0, k1, scale_log2, mrow, mlast, lds_k, lds_v, oacc, m_run,
                       l_run);
    const size_t uq = ((size_t)b * H + h0 + jh) * nsplit + split;
    mfma_write_partial<D>(oacc, m_run, l_run, scale_log2, live, ws_acc + uq * D, ws_ml + uq * 2);
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// Stream kernel: wave w of the grid's W waves takes tiles [w T' / W',
// (w+1) T' / W') of the T' key tiles of all pairs laid end to end, pair
// p = (b * H_kv + K/V head) * hgroups + head group holding tiles
// ceil(L_b / 32) of them, where W' = min(W, max(T' / min_tiles,
// min(T', min_waves))) (waves past W' exit): shares of at least min_tiles
// tiles, unless that leaves fewer than min_waves waves, then down to one tile
// per wave.  The partial of pair p computed by wave w goes to slot
// w + p (distinct: along the sequence each new segment raises the wave or the
// pair index), head row jh of it; span[2p] and span[2p+1] receive the waves
// that hold the pair's first and last tile, so the combine reads slots
// span[2p] + p .. span[2p+1] + p.
template <int D>
__global__ __launch_bounds__(64, 2) void decode_mfma_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ kv_lens, int B, int H, int Hkv,
    int Skv, float scale_log2, int hgroups, int min_tiles, int min_waves,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int* __restrict__ span) {
    using C = MfmaDecode<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[32 * C::kStrideV];
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[32 * C::kStrideK];

    const int lane = threadIdx.x;
    const int jh = lane & 31;
    const int w = blockIdx.x;
    const int group = H / Hkv;
    const int G = Hkv * hgroups;     // pairs per batch item
    const int nhs = min(32, group);  // head rows per partial slot

    // tiles per pair of batch item b: ceil(L_b / 32).  Lane l sums the items
    // l*per .. l*per+per-1 (independent loads, issued together) and a wave
    // scan gives it the tiles before them.
    const int per = (B + 63) / 64;
    const int b_lo = min(lane * per, B), b_hi = min(b_lo + per, B);
    uint32_t mine = 0;
#pragma unroll 8
    for (int bb = b_lo; bb < b_hi; ++bb) mine += (uint32_t)(valid_length(kv_lens, bb, Skv) + 31) >> 5;
    const uint32_t inc = wave_incl_scan(mine);
    const long long T = (long long)(uint32_t)__builtin_amdgcn_readlane((int)inc, 63) * G;
    const long long nw =
        min((long long)gridDim.x, max(T / min_tiles, min(T, (long long)min_waves)));
    if (w >= nw) return;
    const long long s = w * T / nw, e = (w + 1) * T / nw;  // this wave's tiles
    if (s >= e) return;

    // the batch item b holding tile s, and `base`, the first tile of its
    // pairs: first the lane whose items hold it, then, one item per lane, a
    // second scan over that lane's items
    const uint64_t hit = __builtin_amdgcn_ballot_w64(
        mine > 0 && (long long)(inc - mine) * G <= s && s < (long long)inc * G);
    if (hit == 0) return;  // unreachable: s < T
    const int src = __builtin_ctzll(hit);
    const int b_first = __builtin_amdgcn_readlane(b_lo, src);
    const int cnt = __builtin_amdgcn_readlane(b_hi, src) - b_first;
    long long base = (long long)(uint32_t)__builtin_amdgcn_readlane((int)(inc - mine), src) * G;
    int b = -1, L = 0;
    for (int c = 0; c < cnt; c += 64) {
        const int Lb = c + lane < cnt ? valid_length(kv_lens, b_first + c + lane, Skv) : 0;
        const uint32_t n = (uint32_t)(Lb + 31) >> 5;
        const uint32_t inc2 = wave_incl_scan(n);
        const uint64_t hit2 = __builtin_amdgcn_ballot_w64(
            n > 0 && base + (long long)(inc2 - n) * G <= s && s < base + (long long)inc2 * G);
        if (hit2 != 0) {
            const int src2 = __builtin_ctzll(hit2);
            b = b_first + c + src2;
            L = __builtin_amdgcn_readlane(Lb, src2);
            base += (long long)(uint32_t)__builtin_amdgcn_readlane((int)(inc2 - n), src2) * G;
            break;
        }
        base += (long long)(uint32_t)__builtin_amdgcn_readlane((int)inc2, 63) * G;
    }
    if (b < 0) return;  // unreachable
    int nb = (L + 31) >> 5;
    int j = (int)((s - base) / nb);               // pair within batch item b
    int t = (int)(s - base - (long long)j * nb);  // tile within the pair
    long long pos = s;
    for (;;) {
        const int seg = (int)min((long long)(nb - t), e - pos);  // tiles of this pair
        const int kvh = j / hgroups;
        const int hg = j - kvh * hgroups;
        const bool live = jh < min(32, group - hg * 32);
        u32x4 qf[C::kKSteps];
        mfma_load_q<D>(q, b, H, kvh * group + hg * 32, live, qf);
        const size_t kvo = ((size_t)b * Hkv + kvh) * Skv * D;
        f32x16 oacc[C::kDBlocks];
        float m_run, l_run;
        mfma_keys<D, false>(qf, k + kvo, v + kvo, 32 * t, min(32 * (t + seg), L), scale_log2,
                            nullptr, 0, lds_k, lds_v, oacc, m_run, l_run);
        const long long pr = (long long)b * G + j;
        const size_t uq = (size_t)(w + pr) * nhs + jh;
        mfma_write_partial<D>(oacc, m_run, l_run, scale_log2, live, ws_acc + uq * D,
                              ws_ml + uq * 2);
        if (lane == 0) {
            if (t == 0) span[2 * pr] = w;
            if (t + seg == nb) span[2 * pr + 1] = w;
        }
        pos += seg;
        if (pos >= e) return;
        t = 0;
        if (++j == G) {  // next batch item with keys
            j = 0;
            do {
                if (++b >= B) return;  // unreachable: pos < e <= T
                L = valid_length(kv_lens, b, Skv);
            } while (L == 0);
            nb = (L + 31) >> 5;
        }
    }
}

// Final step of a combine block of 2 D threads: thread (h2, t) holds the
// merge (M, lt, at) of half h2 of the partials for column t; the halves are
// merged in LDS and column t of the output row o is written (0 when no key
// was visible: l = 0).
template <int D>
__device__ __forceinline__ void merge_halves(float M, float lt, float at, uint16_t* __restrict__ o) {
    __shared__ float s_m[2], s_l[2];
    __shared__ float s_a[2][D];
    const int t = threadIdx.x % D;
    const int h2 = threadIdx.x / D;
    if (t == 0) {
        s_m[h2] = M;
        s_l[h2] = lt;
    }
    s_a[h2][t] = at;
    __syncthreads();
    if (h2 == 0) {
        // a half with no partial has M = -inf and contributes nothing
        const float Mt = fmaxf(s_m[0], s_m[1]);
        const float w0 = s_m[0] == -INFINITY ? 0.0f : fast_exp2(s_m[0] - Mt);
        const float w1 = s_m[1] == -INFINITY ? 0.0f : fast_exp2(s_m[1] - Mt);
        const float l = s_l[0] * w0 + s_l[1] * w1;
        o[t] = l > 0.0f ? to_bf16((s_a[0][t] * w0 + s_a[1][t] * w1) / l) : 0;  // 0: no visible key
    }
}

template <int D>
__global__ __launch_bounds__(2 * D) void decode_combine_kernel(
    const int32_t* __restrict__ kv_lens, int H, int Skv, int chunk, int nsplit,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, uint16_t* __restrict__ out) {
    // Two halves of the block each merge every other split of one (b, h)
    // (independent loads, unrolled), then one thread per column merges the
    // two halves.
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
        // a split whose keys are all masked has m = -inf, l = 0: weight 0
        const float w = ml[2 * s] == -INFINITY ? 0.0f : fast_exp2(ml[2 * s] - M);
        lt = fmaf(ml[2 * s + 1], w, lt);
        at = fmaf(ac[(size_t)s * D + t], w, at);
    }
    merge_halves<D>(M, lt, at, o);
}

// Stream combine: per (b, h), merges the partials of the head's pair, slots
// span[2p] + p .. span[2p+1] + p (head row h mod 32 of the pair's group), each
// half of the block taking every other slot, four at a time with one running
// maximum.
template <int D>
__global__ __launch_bounds__(2 * D) void decode_combine_stream_kernel(
    const int32_t* __restrict__ kv_lens, int H, int Hkv, int Skv, int hgroups,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int* __restrict__ span, uint16_t* __restrict__ out) {
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int t = threadIdx.x % D;
    const int h2 = threadIdx.x / D;
    const int L = valid_length(kv_lens, b, Skv);
    uint16_t* o = out + (size_t)bh * D;
    if (L == 0) {
        if (h2 == 0) o[t] = 0;
        return;
    }
    const int group = H / Hkv, nhs = min(32, group);
    const int kvh = h / group, r = h - kvh * group;
    const long long pr = ((long long)b * Hkv + kvh) * hgroups + r / 32;
    const int hh = r % 32;
    const int w0 = span[2 * pr], w1 = span[2 * pr + 1];
    float M = -INFINITY, lt = 0.0f, at = 0.0f;
    for (int w = w0 + h2; w <= w1; w += 8) {
        float mv[4], lv[4], av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ww = w + 2 * i;
            const bool ok = ww <= w1;
            const size_t u = (size_t)((ww + pr) * nhs + hh);
            mv[i] = ok ? ws_ml[u * 2] : -INFINITY;
            lv[i] = ok ? ws_ml[u * 2 + 1] : 0.0f;
            av[i] = ok ? ws_acc[u * D + t] : 0.0f;
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < 4; ++i) Mn = fmaxf(Mn, mv[i]);
        const float f = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
        lt *= f;
        at *= f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float wt = mv[i] == -INFINITY ? 0.0f : fast_exp2(mv[i] - Mn);
            lt = fmaf(lv[i], wt, lt);
            at = fmaf(av[i], wt, at);
        }
        M = Mn;
    }
    merge_halves<D>(M, lt, at, o);
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
    const int group = H / Hkv;
    if (group >= 4) {
        // Matrix-core split kernel (with an allowed-mask; without one the
        // stream kernel runs), one wave per (b, K/V head, 32 query heads,
        // split).  Splits of 512 keys measured best at 8 and at 1 K/V heads
        // (64 to 1024 tried); smaller problems split finer, down to 64 keys,
        // until there are 1024 waves.
        const int hgroups = (group + 31) / 32;
        const long pairs = (long)B * Hkv * hgroups;
        int chunk = 512;
        while (chunk > 64 && pairs * ((Skv + chunk - 1) / chunk) < 1024) chunk /= 2;
        return DecodePlan{chunk, (Skv + chunk - 1) / chunk, hgroups};
    }
    // Vector split kernel (with an allowed-mask): splits of 128 keys (64 KiB
    // of K+V at d = 128) measured fastest on the ragged decode workload: many
    // short units spread the reads of the valid prefixes of all caches evenly
    // over the memory system.  Smaller problems split finer so the grid still fills the GPU.
    // A block serving two query heads does twice the vector work per row and
    // merges one partial per head at its end, so it takes the longest split
    // (up to 1024 keys) that still leaves 8 blocks per CU.
    const int hb = decode_heads_per_block(H, Hkv);
    const long groups = (long)B * Hkv * (group / hb);
    int chunk = 128;
    if (hb > 1) {
        while (chunk < 1024 && groups * ((Skv + 2 * chunk - 1) / (2 * chunk)) >= 2048) chunk *= 2;
    } else if (groups * ((Skv + chunk - 1) / chunk) < 8192) {
        chunk = 64;
    }
    return DecodePlan{chunk, (Skv + chunk - 1) / chunk, 0};
}

namespace {

// Stream kernel (every bf16 decode without an allowed-mask).  Shares of a
// wave: at least 16 key tiles when a partial holds 16 or more query heads
// (its bytes then come near a K+V tile's), else 4; but never fewer waves than
// a quarter of those the GPU holds, down to one tile each, so that short
// caches still spread over the chip.  Measured (B = 64, H = 32, d = 128):
// lengths U[512, 8192] at 1 and 2 K/V heads, floors of 8 are 20-25 % slower
// than 16 and 32; lengths U[16, 512] in caches of 8192, floors of 16 are
// 25-100 % slower than 2-4 at 1, 8 and 32 K/V heads.
int stream_min_tiles(int H, int Hkv) { return std::min(32, H / Hkv) >= 16 ? 16 : 4; }
// Most stream waves launched on a d = 128 or d = 64 decode (workspace bound):
// 256 compute units with 8 or 16 resident waves.
long stream_max_waves(int d) { return d == 128 ? 2048 : 4096; }

// Waves the stream kernel can use on this problem: at most one per key tile
// of caches all Skv long.
long stream_wave_cap(int B, int Hkv, int hgroups, int Skv, int d) {
    const long tmax = (long)B * Hkv * hgroups * ((Skv + 31) / 32);
    return std::min(stream_max_waves(d), std::max(1L, tmax));
}

// Stream workspace: partial slots (wave + pair, at most cap + pairs) of nhs
// head rows: acc[d] floats, then (m, l), then two wave indices per pair.
struct StreamLayout {
    size_t ml, span, total;
};
StreamLayout stream_layout(int B, int H, int Hkv, int Skv, int d) {
    const int group = H / Hkv, hg = (group + 31) / 32, nhs = std::min(32, group);
    const size_t pairs = (size_t)B * Hkv * hg;
    const size_t rows = ((size_t)stream_wave_cap(B, Hkv, hg, Skv, d) + pairs) * nhs;
    StreamLayout l;
    l.ml = round256(rows * d * sizeof(float));
    l.span = l.ml + round256(rows * 2 * sizeof(float));
    l.total = l.span + round256(pairs * 2 * sizeof(int));
    return l;
}

// Waves of the stream kernel the current device holds at once (compute
// units x resident waves per unit), cached per device and head size.
int stream_resident_waves(int d) {
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices][2];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const int di = d == 128 ? 0 : 1;
    const bool cached = dev >= 0 && dev < kDevices;
    if (cached) {
        const int c = cache[dev][di].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per = 0;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess || cus <= 0)
        cus = 256;
    const hipError_t e =
        d == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &per, decode_mfma_stream_kernel<128>, 64, 0)
                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &per, decode_mfma_stream_kernel<64>, 64, 0);
    if (e != hipSuccess || per <= 0) {
        (void)hipGetLastError();  // a failed query leaves no error for the launches
        per = d == 128 ? 8 : 16;
    }
    const int waves = (int)std::min((long)cus * per, stream_max_waves(d));
    if (cached) cache[dev][di].store(waves, std::memory_order_relaxed);
    return waves;
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int Hkv, int Skv, int d) {
    const DecodePlan p = decode_plan(B, H, Hkv, Skv);
    const size_t units = (size_t)B * H * p.nsplit;  // one partial per query head and split
    const size_t split = round256(units * d * sizeof(float)) + round256(units * 2 * sizeof(float));
    // split kernels with an allowed-mask, else the stream kernel
    return std::max(split, stream_layout(B, H, Hkv, Skv, d).total);
}

namespace {

template <int D, int HB>
void launch_partial(const LaunchArgs& a, const DecodePlan& p, float sl, float* ws_acc,
                    float* ws_ml) {
    const size_t blocks = (size_t)a.B * a.H / HB * p.nsplit;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                           static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                           static_cast<const uint16_t*>(a.v), a.kv_lens, a.H, a.Hkv, a.Skv, sl,
                           p.chunk, p.nsplit, ws_acc, ws_ml, a.mask, a.msb, a.msh);
    };
    a.mask ? go(decode_partial_kernel<D, HB, true>) : go(decode_partial_kernel<D, HB, false>);
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
    // the front end sizes the workspace; refuse rather than write through a bad one
    if (a.workspace == nullptr ||
        a.workspace_bytes < decode_workspace_bytes(a.B, a.H, a.Hkv, a.Skv, a.d))
        return hipErrorInvalidValue;
    const size_t units = (size_t)a.B * a.H * p.nsplit;
    float* ws_acc = static_cast<float*>(a.workspace);
    float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                            round256(units * a.d * sizeof(float)));
    uint16_t* o = static_cast<uint16_t*>(a.out);
    const float sl = a.scale * kLog2e;
    KernelTimer* t = active_timer();
    hipError_t e;
    if (a.mask == nullptr) {
        const int hgroups = (a.H / a.Hkv + 31) / 32;
        const StreamLayout l = stream_layout(a.B, a.H, a.Hkv, a.Skv, a.d);
        char* ws = static_cast<char*>(a.workspace);
        float* acc = reinterpret_cast<float*>(ws);
        float* ml = reinterpret_cast<float*>(ws + l.ml);
        int* span = reinterpret_cast<int*>(ws + l.span);
        const int resident = stream_resident_waves(a.d);
        const int waves =
            (int)std::min((long)resident, stream_wave_cap(a.B, a.Hkv, hgroups, a.Skv, a.d));
        const int min_tiles = stream_min_tiles(a.H, a.Hkv);
        const int min_waves = std::max(1, resident / 4);
        const uint16_t* q = static_cast<const uint16_t*>(a.q);
        const uint16_t* k = static_cast<const uint16_t*>(a.k);
        const uint16_t* v = static_cast<const uint16_t*>(a.v);
        if (t) t->begin(kDecodePartialBf16, a.stream);
        if (a.d == 128)
            hipLaunchKernelGGL(decode_mfma_stream_kernel<128>, dim3(waves), dim3(64), 0, a.stream,
                               q, k, v, a.kv_lens, a.B, a.H, a.Hkv, a.Skv, sl, hgroups,
                               min_tiles, min_waves, acc, ml, span);
        else
            hipLaunchKernelGGL(decode_mfma_stream_kernel<64>, dim3(waves), dim3(64), 0, a.stream,
                               q, k, v, a.kv_lens, a.B, a.H, a.Hkv, a.Skv, sl, hgroups,
                               min_tiles, min_waves, acc, ml, span);
        e = hipGetLastError();
        if (t) t->end(kDecodePartialBf16, a.stream);
        if (e != hipSuccess) return e;
        if (t) t->begin(kDecodeCombineBf16, a.stream);
        const unsigned pairs = (unsigned)((size_t)a.B * a.H);
        if (a.d == 128)
            hipLaunchKernelGGL(decode_combine_stream_kernel<128>, dim3(pairs), dim3(256), 0,
                               a.stream, a.kv_lens, a.H, a.Hkv, a.Skv, hgroups, acc, ml, span,
                               o);
        else
            hipLaunchKernelGGL(decode_combine_stream_kernel<64>, dim3(pairs), dim3(128), 0,
                               a.stream, a.kv_lens, a.H, a.Hkv, a.Skv, hgroups, acc, ml, span,
                               o);
        e = hipGetLastError();
        if (t) t->end(kDecodeCombineBf16, a.stream);
        return e;
    }
    if (t) t->begin(kDecodePartialBf16, a.stream);
    if (p.hgroups > 0) {
        const unsigned blocks = (unsigned)((size_t)a.B * a.Hkv * p.hgroups * p.nsplit);
        const uint16_t* q = static_cast<const uint16_t*>(a.q);
        const uint16_t* k = static_cast<const uint16_t*>(a.k);
        const uint16_t* v = static_cast<const uint16_t*>(a.v);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(blocks), dim3(64), 0, a.stream, q, k, v, a.kv_lens, a.H,
                               a.Hkv, a.Skv, sl, p.chunk, p.nsplit, p.hgroups, ws_acc, ws_ml,
                               a.mask, a.msb, a.msh);
        };
        if (a.d == 128)
            a.mask ? go(decode_mfma_kernel<128, true>) : go(decode_mfma_kernel<128, false>);
        else
            a.mask ? go(decode_mfma_kernel<64, true>) : go(decode_mfma_kernel<64, false>);
    } else if (a.d == 128) {
        launch_partial_d<128>(a, p, sl, ws_acc, ws_ml);
    } else {
        launch_partial_d<64>(a, p, sl, ws_acc, ws_ml);
    }
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
