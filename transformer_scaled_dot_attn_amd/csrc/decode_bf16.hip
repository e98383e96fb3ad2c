// bfloat16 decode: one query per (b, h) against a KV cache, split over keys.
//
// Decode reads the whole valid cache and does little arithmetic per byte
// ("Attention from First Principles", section 6: a matrix-vector product
// whose intensity is about 1 for multi-head attention), so this path is
// built for HBM bandwidth.  With grouped key/value heads (GQA / MQA: query
// head h reads K/V head h / (H / H_kv), same page, section "MHA, GQA, MQA --
// the KV cache lever") each K/V row serves H / H_kv query heads, the rise in
// decode intensity that section 6 derives, and the kernels read it once per
// group of query heads.
//
// Key loop.  The query heads a K/V head serves are the 32 columns of one
// MFMA tile (heads past the group are zero columns; one live column for
// multi-head attention), so per 32-key tile a wave computes S^T = K Q^T with
// d/16 v_mfma_f32_32x32x16_bf16 -- K from the tile staged in LDS as the A
// operand, Q^T held as the B operand -- and O^T += V^T P^T with d/16 more,
// V^T read through ds_read_b64_tr_b16 from the staged V tile.  K and V both
// arrive by whole-row, non-temporal 16-byte loads (a wave-wide load covers
// 1 KiB of contiguous rows), issued for the next tile at the top of each
// iteration; K loaded straight into the A-operand layout instead (32 bytes of
// each of 32 rows per load) measured 17 % slower at 8 K/V heads.  In both
// accumulators a lane owns one query head, so the online softmax is
// lane-local plus one half swap, as in the prefill kernel.  The matrix cores
// have ample headroom (16 MFMAs per 16 KiB of K+V): a copy of the loop with
// its arithmetic removed runs no faster, so decode stays bound by the bytes
// of K and V, and how the grid meets memory decides the speed.
//
// Stream kernel.  A fixed grid of as many waves as the GPU holds at once.
// The (b, K/V head, head group) pairs, each cut into ceil(L_b / 32) key
// tiles, are laid end to end and wave w takes the w-th equal share of that
// sequence, crossing pair boundaries as it goes and writing one partial
// (m, l, acc[d]) per pair it touches (the stream-K decomposition of Osama et
// al., 2023, applied to the key axis).  Every wave streams the same bytes, so
// ragged lengths leave no part-filled last round of waves.  On lengths
// U[512, 8192] (B = 64, H = 32), grids of fixed key splits measured 12 %
// slower at 32 K/V heads, 29 % at 16 and 20-25 % at 4 and 8; with short caches
// in a large capacity (lengths U[16, 512] of 8192) a grid of 128-key splits,
// almost all empty, took 4.8x as long.
//
// V rows and outputs may have a width DV other than the D of K (each 64 or
// 128): Q K^T runs over D, P V over DV, and the partials hold DV columns.
//
// Allowed-mask (the MASK instantiations: a byte per query head and key,
// nonzero = visible, ANDed with the length rule).  A pre-pass lists, per
// pair, the key tiles that some served head may see; the stream kernel shares
// out only those tiles, so a hidden tile costs neither reads nor a place in a
// wave's share, and reads each listed tile's mask words next to its K/V rows.
// A pair with no visible tile writes no partial, and its heads are written as
// 0, as is a head whose visible tiles hold no key it may see (l = 0).
//
// General logits (the GEN instantiations): with an additive bias (the
// float mask of "Attention from Scratch", KubeDojo module 1.4.3, Part 7,
// added to each scaled logit; -inf hides the key) or a scale that is not
// positive, each score becomes scale * s + bias before the online softmax,
// which then tracks the maximum of those logits.  The lane's 16 bias values
// of a tile (8-byte groups of 4 keys of its query head's row) are loaded
// with the next tile's K/V rows; without a bias a zero array is read.
//
// Combine kernel: per (b, h), merges the pair's partials with the
// log-sum-exp rule  M = max m_s,  l = sum l_s 2^(m_s - M),
// out = (sum acc_s 2^(m_s - M)) / l, and rounds to bf16.  L_b = 0 gives 0.
// Logits are kept in base 2 (scale * log2 e folded in), which leaves the
// softmax unchanged.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace tsda {

namespace {

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

// Online softmax of the 32 query-head columns in qf over n key tiles (n >= 1)
// of the K/V head whose rows start at kb and vb, from scratch: running
// maximum m_run (raw logit units), normaliser l_run over this lane's half of
// the keys, and the O^T accumulators.  Tile i holds keys key_i .. key_i+31,
// those at or past klim hidden.  Without MASK the tiles are consecutive,
// key_i = k0 + 32 i; with MASK, key_i = 32 tl[i] (a list of visible tiles)
// and mrow is the allowed-mask row of the lane's query head (words past mlast
// never read).
template <int D, int DV, bool MASK, bool GEN>
__device__ __forceinline__ void mfma_keys(const u32x4 (&qf)[D / 16], const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ vb, int k0, int n, int klim,
                                          const int* __restrict__ tl, float scale_log2,
                                          const uint8_t* __restrict__ mrow, int mlast,
                                          const uint16_t* __restrict__ brow, int blast, float scale,
                                          uint16_t* lds_k, uint16_t* lds_v,
                                          f32x16 (&oacc)[DV / 32], float& m_run, float& l_run) {
    using C = MfmaDecode<D>;    // the key side (D features)
    using CV = MfmaDecode<DV>;  // the value side (DV features)
    const int lane = threadIdx.x;
    const int half = lane >> 5;
    const int jh = lane & 31;

    // MASK: list entries c .. c+63 (la) and c+64 .. c+127 (lb), one per lane;
    // the tile of entry i (c <= i < c+128) is read out with readlane, and lb
    // is loaded 64 entries before it is needed
    int c = 0, la = 0, lb = 0;
    if constexpr (MASK) {
        la = lane < n ? tl[lane] : 0;
        lb = 64 + lane < n ? tl[64 + lane] : 0;
    }
    auto tile_key = [&](int i) -> int {
        if constexpr (MASK) {
            const int r = i - c;
            return 32 * __builtin_amdgcn_readlane(r < 64 ? la : lb, r & 63);
        } else {
            return k0 + 32 * i;
        }
    };

    // allowed-mask words of this lane's query head for a 32-key tile: word g
    // holds keys 8 g + 4 half .. +3, the keys of score elements 4 g .. +3
    // (offsets clamped to the row's last readable word; keys past it are
    // >= Skv >= klim and hidden anyway)
    uint32_t mw[4], mw_next[4];
    auto load_m = [&](int t0, uint32_t (&dst)[4]) {
        if constexpr (MASK) {
#pragma unroll
            for (int g = 0; g < 4; ++g) dst[g] = ldg_word(mrow + min(t0 + 8 * g + 4 * half, mlast));
        }
    };

    // GEN: bias of this lane's query head for a 32-key tile: group g holds
    // keys 8 g + 4 half .. +3, those of score elements 4 g .. +3 (offsets
    // clamped to the row's last readable group, as the mask words are)
    u32x2 bw[4], bw_next[4];
    auto load_b = [&](int t0, u32x2 (&dst)[4]) {
        if constexpr (GEN) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                dst[g] = *reinterpret_cast<const u32x2*>(brow + min(t0 + 8 * g + 4 * half, blast));
        }
    };

    // K and V tile rows whole (kRows rows per load, lane%kChunks the 16-byte
    // chunk).  Rows at or past klim are clamped to row klim - 1 (valid: klim
    // <= L; their logits are masked).  Addresses are a wave-uniform base plus
    // a 32-bit byte offset per lane (a head's rows span less than 4 GiB), so
    // a load costs a min and a multiply-add.
    const char* kbase = reinterpret_cast<const char*>(kb);
    const char* vbase = reinterpret_cast<const char*>(vb);
    const uint32_t kcol = (uint32_t)(lane % C::kChunks) * 16u;
    const uint32_t vcol = (uint32_t)(lane % CV::kChunks) * 16u;
    u32x4 kr[C::kLoads], vr[CV::kLoads];
    auto load_kv = [&](int t0) {
        if constexpr (D == DV) {  // K and V rows of one tile side by side
#pragma unroll
            for (int c2 = 0; c2 < C::kLoads; ++c2) {
                const int row = min(t0 + c2 * C::kRows + lane / C::kChunks, klim - 1);
                const uint32_t off = (uint32_t)row * (2u * D) + kcol;
                kr[c2] = ldg16_stream(kbase + off);
                vr[c2] = ldg16_stream(vbase + off);
            }
        } else {
#pragma unroll
            for (int c2 = 0; c2 < C::kLoads; ++c2) {
                const int row = min(t0 + c2 * C::kRows + lane / C::kChunks, klim - 1);
                kr[c2] = ldg16_stream(kbase + ((uint32_t)row * (2u * D) + kcol));
            }
#pragma unroll
            for (int c2 = 0; c2 < CV::kLoads; ++c2) {
                const int row = min(t0 + c2 * CV::kRows + lane / CV::kChunks, klim - 1);
                vr[c2] = ldg16_stream(vbase + ((uint32_t)row * (2u * DV) + vcol));
            }
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
        (4 * half + (n16 >> 2)) * CV::kStrideV + 16 * ((lane >> 4) & 1) + 4 * (n16 & 3);

#pragma unroll
    for (int db = 0; db < CV::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    m_run = -INFINITY;
    l_run = 0.0f;

    int t0 = tile_key(0);
    load_kv(t0);
    load_m(t0, mw);
    load_b(t0, bw);
    for (int i = 0; i < n; ++i) {
        // K(t0), V(t0) to LDS; the next tile's loads reuse their registers
#pragma unroll
        for (int c2 = 0; c2 < C::kLoads; ++c2) {
            const int r = c2 * C::kRows + lane / C::kChunks, col = (lane % C::kChunks) * 8;
            *reinterpret_cast<u32x4*>(lds_k + r * C::kStrideK + col) = kr[c2];
            if constexpr (D == DV) *reinterpret_cast<u32x4*>(lds_v + r * CV::kStrideV + col) = vr[c2];
        }
        if constexpr (D != DV) {
#pragma unroll
            for (int c2 = 0; c2 < CV::kLoads; ++c2) {
                const int r = c2 * CV::kRows + lane / CV::kChunks, col = (lane % CV::kChunks) * 8;
                *reinterpret_cast<u32x4*>(lds_v + r * CV::kStrideV + col) = vr[c2];
            }
        }
        __syncthreads();
        if constexpr (MASK) {
            if (i - c == 64) {  // entries c+64 .. move down, the next 64 are loaded
                c += 64;
                la = lb;
                lb = c + 64 + lane < n ? tl[c + 64 + lane] : 0;
            }
        }
        const bool next = i + 1 < n;
        const int t1 = next ? tile_key(i + 1) : t0;
        if (next) {
            load_kv(t1);
            load_m(t1, mw_next);
            load_b(t1, bw_next);
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
        if constexpr (GEN) {
            // logits scale * s + bias
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t wd = bw[r >> 2][(r & 3) >> 1];
                sacc[r] = fmaf(sacc[r], scale, (r & 1) ? bf16_hi(wd) : bf16_lo(wd));
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) bw[g] = bw_next[g];
        }
        bool cut = t0 + 32 > klim;
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
                bool vis = j < klim;
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
            for (int db = 0; db < CV::kDBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        const float mc = m_run == -INFINITY ? 0.0f : m_run * scale_log2;
        u32x4 pf[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a0 = fast_exp2(fmaf(sacc[8 * h2 + 2 * e], scale_log2, -mc));
                const float a1 = fast_exp2(fmaf(sacc[8 * h2 + 2 * e + 1], scale_log2, -mc));
                pf[h2][e] = pack_bf16(a0, a1);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pf[h2][e]),
                                                        as_bf16x2(0x3F803F80u), l_run, false);
            }
        // O^T += V^T P^T, output blocks innermost
#pragma unroll
        for (int st = 0; st < 2 * CV::kDBlocks; ++st) {
            const int db = st % CV::kDBlocks, kk = st / CV::kDBlocks;
            const uint16_t* a1 = lds_v + v_rd + kk * 16 * CV::kStrideV + db * 32;
            const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TSDA_LDS i16x4*)(a1));
            const i16x4 x1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((TSDA_LDS i16x4*)(a1 + 8 * CV::kStrideV));
            u32x4 a;
            a[0] = (uint32_t)(uint16_t)x0[0] | ((uint32_t)(uint16_t)x0[1] << 16);
            a[1] = (uint32_t)(uint16_t)x0[2] | ((uint32_t)(uint16_t)x0[3] << 16);
            a[2] = (uint32_t)(uint16_t)x1[0] | ((uint32_t)(uint16_t)x1[1] << 16);
            a[3] = (uint32_t)(uint16_t)x1[2] | ((uint32_t)(uint16_t)x1[3] << 16);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pf[kk]), oacc[db], 0, 0,
                0);
        }
        t0 = t1;
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

// Mask pre-pass: one 256-thread block per pair p = (b * H_kv + K/V head) *
// hgroups + head group.  Key tile t (keys 32 t .. 32 t + 31 below L_b) is
// listed when some head of the group (the one shared row when msh = 0) may
// see one of its keys: lists[p * ntmax + i] is the i-th such tile, in
// ascending order, counts[p] their number.  The mask is read once, a 4-key
// word per thread, consecutive threads on consecutive words of a row.
constexpr int kMaskChunk = 2048;  // key tiles flagged per pass through LDS
__global__ __launch_bounds__(256) void decode_mask_tiles_kernel(
    const uint8_t* __restrict__ mask, long long msb, long long msh,
    const int32_t* __restrict__ kv_lens, int H, int Hkv, int Skv, int hgroups, int ntmax,
    int* __restrict__ counts, int* __restrict__ lists) {
    __shared__ uint8_t flag[kMaskChunk];
    __shared__ uint32_t wsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int p = blockIdx.x;
    const int G = Hkv * hgroups;
    const int b = p / G, j = p - b * G;
    const int group = H / Hkv;
    const int kvh = j / hgroups, hg = j - kvh * hgroups;
    const int h0 = kvh * group + hg * 32;
    const int heads = msh == 0 ? 1 : min(32, group - hg * 32);
    const int L = valid_length(kv_lens, b, Skv);
    const int nt = (L + 31) >> 5;
    const int mlast = mask_last_word(Skv);
    const uint8_t* mrow = mask + b * msb + (long long)h0 * msh;
    int* list = lists + (size_t)p * ntmax;
    int total = 0;
    for (int c0 = 0; c0 < nt; c0 += kMaskChunk) {
        const int nc = min(kMaskChunk, nt - c0);
        for (int i = tid; i < nc; i += 256) flag[i] = 0;
        __syncthreads();
        const int words = nc * 8;  // 4-key words of the chunk, per head
        const int nwords = heads * words;
        if (heads > 1) {
            // several head rows: eight words per thread in flight before any
            // is tested (one memory round trip per eight)
            for (int i0 = tid; i0 < nwords; i0 += 8 * 256) {
                uint32_t wd[8];
                int wk[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int idx = i0 + u * 256;
                    const int hh = idx / words, w = idx - hh * words;
                    const int key = c0 * 32 + 4 * w;
                    const bool ok = idx < nwords && key < L;
                    wd[u] = ok ? ldg_word(mrow + hh * msh + min(key, mlast)) : 0u;
                    wk[u] = ok ? w : -1;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (wk[u] < 0) continue;
                    const int key = c0 * 32 + 4 * wk[u];
                    uint32_t any = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) any |= (key + e < L) & byte_set(wd[u], e);
                    if (any) flag[wk[u] >> 3] = 1;
                }
            }
        } else {
            for (int idx = tid; idx < nwords; idx += 256) {
                const int w = idx;
                const int key = c0 * 32 + 4 * w;
                if (key < L) {
                    const uint32_t wd = ldg_word(mrow + min(key, mlast));
                    uint32_t any = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) any |= (key + e < L) & byte_set(wd, e);
                    if (any) flag[w >> 3] = 1;
                }
            }
        }
        __syncthreads();
        // compaction: thread tid owns flags 8 tid .. 8 tid + 7
        uint32_t mine = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) mine += 8 * tid + e < nc ? flag[8 * tid + e] : 0;
        const uint32_t inc = wave_incl_scan(mine);
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        uint32_t before = inc - mine;
        for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
        const uint32_t chunk_total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 8 * tid + e;
            if (i < nc && flag[i]) list[total + before++] = c0 + i;
        }
        total += (int)chunk_total;
        __syncthreads();  // flags and sums are read before the next chunk resets them
    }
    if (tid == 0) counts[p] = total;
}

// Stream kernel: wave w of the grid's W waves takes tiles [w T / W', (w+1) T /
// W') of the T key tiles of all pairs laid end to end, where W' = min(W,
// max(T / min_tiles, min(T, min_waves))) (waves past W' exit): shares of at
// least min_tiles tiles, unless that leaves fewer than min_waves waves, then
// down to one tile per wave.  Pair p = (b * H_kv + K/V head) * hgroups + head
// group holds ceil(L_b / 32) tiles, or with MASK its counts[p] listed tiles.
// The partial of pair p computed by wave w goes to slot w + p (distinct:
// along the sequence each new segment raises the wave or the pair index),
// head row jh of it; span[2p] and span[2p+1] receive the waves that hold the
// pair's first and last tile, so the combine reads slots span[2p] + p ..
// span[2p+1] + p.
// Zero bias for GEN calls without one (read as its first 4-element group).
__device__ __attribute__((aligned(16))) uint16_t g_zero_bias_dec[8];

template <int D, int DV, bool MASK, bool GEN>
__global__ __launch_bounds__(64, 2) void decode_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ kv_lens, int B, int H, int Hkv,
    int Skv, float scale_log2, int hgroups, int min_tiles, int min_waves,
    float* __restrict__ ws_acc, float* __restrict__ ws_ml, int* __restrict__ span,
    const uint8_t* __restrict__ mask, long long msb, long long msh,
    const int* __restrict__ counts, const int* __restrict__ lists, int ntmax,
    const uint16_t* __restrict__ bias, long long bsb, long long bsh, float scale) {
    using C = MfmaDecode<D>;
    using CV = MfmaDecode<DV>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[32 * CV::kStrideV];
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[32 * C::kStrideK];

    const int lane = threadIdx.x;
    const int jh = lane & 31;
    const int w = blockIdx.x;
    const int group = H / Hkv;
    const int G = Hkv * hgroups;     // pairs per batch item
    const int nhs = min(32, group);  // head rows per partial slot

    // Items laid end to end: batch items of G pairs with ceil(L_b / 32) tiles
    // each, or (MASK) single pairs with their listed tiles.  Lane l sums the
    // items l*per .. l*per+per-1 (independent loads, issued together) and a
    // wave scan gives it the tiles before them.
    const int nitems = MASK ? B * G : B;
    const int gi = MASK ? 1 : G;  // pairs per item
    auto item_tiles = [&](int it, int& Lb) -> uint32_t {
        if constexpr (MASK) {
            return (uint32_t)counts[it];
        } else {
            Lb = valid_length(kv_lens, it, Skv);
            return (uint32_t)(Lb + 31) >> 5;
        }
    };
    const int per = (nitems + 63) / 64;
    const int i_lo = min(lane * per, nitems), i_hi = min(i_lo + per, nitems);
    uint32_t mine = 0;
#pragma unroll 8
    for (int it = i_lo; it < i_hi; ++it) {
        int unused;
        mine += item_tiles(it, unused);
    }
    const uint32_t inc = wave_incl_scan(mine);
    const long long T = (long long)(uint32_t)__builtin_amdgcn_readlane((int)inc, 63) * gi;
    const long long nw =
        min((long long)gridDim.x, max(T / min_tiles, min(T, (long long)min_waves)));
    if (w >= nw) return;
    const long long s = w * T / nw, e = (w + 1) * T / nw;  // this wave's tiles
    if (s >= e) return;

    // the item holding tile s, and `base`, its first tile: first the lane
    // whose items hold it, then, one item per lane, a second scan over them
    const uint64_t hit = __builtin_amdgcn_ballot_w64(
        mine > 0 && (long long)(inc - mine) * gi <= s && s < (long long)inc * gi);
    if (hit == 0) return;  // unreachable: s < T
    const int src = __builtin_ctzll(hit);
    const int i_first = __builtin_amdgcn_readlane(i_lo, src);
    const int cnt = __builtin_amdgcn_readlane(i_hi, src) - i_first;
    long long base = (long long)(uint32_t)__builtin_amdgcn_readlane((int)(inc - mine), src) * gi;
    int item = -1, nb = 0, L = 0;
    for (int c = 0; c < cnt; c += 64) {
        int Lb = 0;
        const uint32_t n = c + lane < cnt ? item_tiles(i_first + c + lane, Lb) : 0u;
        const uint32_t inc2 = wave_incl_scan(n);
        const uint64_t hit2 = __builtin_amdgcn_ballot_w64(
            n > 0 && base + (long long)(inc2 - n) * gi <= s && s < base + (long long)inc2 * gi);
        if (hit2 != 0) {
            const int src2 = __builtin_ctzll(hit2);
            item = i_first + c + src2;
            nb = __builtin_amdgcn_readlane((int)n, src2);
            L = __builtin_amdgcn_readlane(Lb, src2);
            base += (long long)(uint32_t)__builtin_amdgcn_readlane((int)(inc2 - n), src2) * gi;
            break;
        }
        base += (long long)(uint32_t)__builtin_amdgcn_readlane((int)inc2, 63) * gi;
    }
    if (item < 0) return;  // unreachable
    int b, j, t;  // batch item, pair within it, tile within the pair
    if constexpr (MASK) {
        b = item / G;
        j = item - b * G;
        t = (int)(s - base);
        L = valid_length(kv_lens, b, Skv);
    } else {
        b = item;
        j = (int)((s - base) / nb);
        t = (int)(s - base - (long long)j * nb);
    }
    const int mlast = mask_last_word(Skv);
    long long pos = s;
    for (;;) {
        const int seg = (int)min((long long)(nb - t), e - pos);  // tiles of this pair
        const int kvh = j / hgroups;
        const int hg = j - kvh * hgroups;
        const int h0 = kvh * group + hg * 32;
        const bool live = jh < min(32, group - hg * 32);
        const long long pr = (long long)b * G + j;
        u32x4 qf[C::kKSteps];
        mfma_load_q<D>(q, b, H, h0, live, qf);
        const size_t kvo = ((size_t)b * Hkv + kvh) * Skv * D;
        const size_t vvo = ((size_t)b * Hkv + kvh) * Skv * DV;
        f32x16 oacc[CV::kDBlocks];
        float m_run, l_run;
        // the bias row of the lane's query head (Sq = 1: row 0), or the zero array
        const uint16_t* brow = nullptr;
        int blast = 0;
        if constexpr (GEN) {
            brow = g_zero_bias_dec;
            if (bias != nullptr) {
                brow = bias + b * bsb + (long long)(h0 + (live ? jh : 0)) * bsh;
                blast = bias_last_group(Skv);
            }
        }
        if constexpr (MASK) {
            const uint8_t* mrow = mask + b * msb + (long long)(h0 + (live ? jh : 0)) * msh;
            mfma_keys<D, DV, true, GEN>(qf, k + kvo, v + vvo, 0, seg, L, lists + pr * ntmax + t,
                                    scale_log2, mrow, mlast, brow, blast, scale, lds_k, lds_v,
                                    oacc, m_run, l_run);
        } else {
            mfma_keys<D, DV, false, GEN>(qf, k + kvo, v + vvo, 32 * t, seg, min(32 * (t + seg), L),
                                     nullptr, scale_log2, nullptr, 0, brow, blast, scale, lds_k,
                                     lds_v, oacc, m_run, l_run);
        }
        const size_t uq = (size_t)(w + pr) * nhs + jh;
        mfma_write_partial<DV>(oacc, m_run, l_run, scale_log2, live, ws_acc + uq * DV,
                              ws_ml + uq * 2);
        if (lane == 0) {
            if (t == 0) span[2 * pr] = w;
            if (t + seg == nb) span[2 * pr + 1] = w;
        }
        pos += seg;
        if (pos >= e) return;
        t = 0;
        if constexpr (MASK) {  // next pair with a listed tile
            long long p2 = pr;
            do {
                if (++p2 >= (long long)B * G) return;  // unreachable: pos < e <= T
                nb = counts[p2];
            } while (nb == 0);
            const int b2 = (int)(p2 / G);
            j = (int)(p2 - (long long)b2 * G);
            if (b2 != b) {
                b = b2;
                L = valid_length(kv_lens, b, Skv);
            }
        } else if (++j == G) {  // next batch item with keys
            j = 0;
            do {
                if (++b >= B) return;  // unreachable: pos < e <= T
                L = valid_length(kv_lens, b, Skv);
            } while (L == 0);
            nb = (L + 31) >> 5;
        }
    }
}

// Combine: per (b, h), merges the partials of the head's pair, slots
// span[2p] + p .. span[2p+1] + p (head row h mod 32 of the pair's group).  The
// block's 256 threads form kG groups of D/4 threads, each thread holding 4
// columns (16-byte loads); group g takes every kG-th slot, kU at a time with
// one running maximum, and the groups are merged in LDS.  A pair with no tile
// (L_b = 0, or with a mask no listed tile: counts[p] = 0) wrote no partial;
// its heads are 0, as is a head with no visible key (l = 0).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const int32_t* __restrict__ kv_lens, int H, int Hkv, int Skv, int hgroups,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
    const int* __restrict__ span, const int* __restrict__ counts, uint16_t* __restrict__ out) {
    constexpr int kC = D / 4;     // threads per partial row
    constexpr int kG = 256 / kC;  // groups of slots: 8 at d = 128, 16 at d = 64
    constexpr int kU = 4;         // slots per group per step
    __shared__ float s_m[kG], s_l[kG];
    __shared__ __attribute__((aligned(16))) float s_a[kG][D];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x;
    const int g = tid / kC, c = (tid % kC) * 4;
    const int group = H / Hkv, nhs = min(32, group);
    const int kvh = h / group, r = h - kvh * group;
    const long long pr = ((long long)b * Hkv + kvh) * hgroups + r / 32;
    const int hh = r % 32;
    uint16_t* o = out + (size_t)bh * D;
    // the span is read with the length (unused when the pair has no tile)
    const int w0 = span[2 * pr], w1 = span[2 * pr + 1];
    if (valid_length(kv_lens, b, Skv) == 0 || (counts != nullptr && counts[pr] == 0)) {
        if (tid < kC) *reinterpret_cast<u32x2*>(o + c) = u32x2{0, 0};
        return;
    }
    float M = -INFINITY, lt = 0.0f;
    f32x4 at = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int w = w0 + g; w <= w1; w += kG * kU) {
        float mv[kU], lv[kU];
        f32x4 av[kU];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int ww = w + kG * i;
            const bool ok = ww <= w1;
            const size_t u = (size_t)((ww + pr) * nhs + hh);
            mv[i] = ok ? ws_ml[u * 2] : -INFINITY;
            lv[i] = ok ? ws_ml[u * 2 + 1] : 0.0f;
            av[i] = ok ? *reinterpret_cast<const f32x4*>(ws_acc + u * D + c)
                       : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < kU; ++i) Mn = fmaxf(Mn, mv[i]);
        const float f = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
        lt *= f;
        at *= f;
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const float wt = mv[i] == -INFINITY ? 0.0f : fast_exp2(mv[i] - Mn);
            lt = fmaf(lv[i], wt, lt);
            at += av[i] * wt;
        }
        M = Mn;
    }
    if (c == 0) {
        s_m[g] = M;
        s_l[g] = lt;
    }
    *reinterpret_cast<f32x4*>(&s_a[g][c]) = at;
    __syncthreads();
    if (tid < kC) {
        // a group with no slot has M = -inf and contributes nothing
        float Mt = -INFINITY;
#pragma unroll
        for (int gg = 0; gg < kG; ++gg) Mt = fmaxf(Mt, s_m[gg]);
        float l = 0.0f;
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int gg = 0; gg < kG; ++gg) {
            const float wt = s_m[gg] == -INFINITY ? 0.0f : fast_exp2(s_m[gg] - Mt);
            l = fmaf(s_l[gg], wt, l);
            a += *reinterpret_cast<const f32x4*>(&s_a[gg][c]) * wt;
        }
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // 0: no visible key
        const u32x2 wv = {pack_bf16(a[0] * inv, a[1] * inv), pack_bf16(a[2] * inv, a[3] * inv)};
        *reinterpret_cast<u32x2*>(o + c) = wv;
    }
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shares of a wave: at least 32 key tiles when a partial holds 16 or more
// query heads (its bytes then come near a K+V tile's), else 4; but never
// fewer waves than a quarter of those the GPU holds, down to one tile each,
// so that short caches still spread over the chip.  Measured (B = 64,
// H = 32, d = 128, capacity 8192): at 1 and 2 K/V heads, floors of 32 beat
// 16 by 4-8 % (fewer partials to write and merge) and floors of 8 lose
// 10-25 %, while 256 waves lose 23 %; with lengths U[16, 512], floors of 16
// are 25-100 % slower than 2-4 at 1, 8 and 32 K/V heads.
int stream_min_tiles(int H, int Hkv) { return std::min(32, H / Hkv) >= 16 ? 32 : 4; }
// Most stream waves launched on a d = 128 or d = 64 decode (workspace bound):
// 256 compute units with 8 or 16 resident waves.
long stream_max_waves(int d) { return d == 128 ? 2048 : 4096; }

// Waves the stream kernel can use on this problem: at most one per key tile
// of caches all Skv long.
long stream_wave_cap(int B, int Hkv, int hgroups, int Skv, int d) {
    const long tmax = (long)B * Hkv * hgroups * ((Skv + 31) / 32);
    return std::min(stream_max_waves(d), std::max(1L, tmax));
}

// Workspace: partial slots (wave + pair, at most cap + pairs) of nhs head
// rows: acc[d] floats, then (m, l), then two wave indices per pair; with a
// mask, then the pairs' tile counts and tile lists.
struct StreamLayout {
    size_t ml, span, counts, lists, total, masked_total;
    int ntmax;
};
StreamLayout stream_layout(int B, int H, int Hkv, int Skv, int d, int dv) {
    const int group = H / Hkv, hg = (group + 31) / 32, nhs = std::min(32, group);
    const size_t pairs = (size_t)B * Hkv * hg;
    const size_t rows = ((size_t)stream_wave_cap(B, Hkv, hg, Skv, d) + pairs) * nhs;
    StreamLayout l;
    l.ntmax = (Skv + 31) / 32;
    l.ml = round256(rows * dv * sizeof(float));
    l.span = l.ml + round256(rows * 2 * sizeof(float));
    l.total = l.span + round256(pairs * 2 * sizeof(int));
    l.counts = l.total;
    l.lists = l.counts + round256(pairs * sizeof(int));
    l.masked_total = l.lists + round256(pairs * (size_t)l.ntmax * sizeof(int));
    return l;
}

// Calls go(decode_stream_kernel<D, DV, MASK, GEN>) for d, dv in {64, 128}.
template <class Go>
void with_stream_kernel(int d, int dv, bool masked, bool gen, Go&& go) {
    auto pick = [&](auto dk, auto dvk) {
        constexpr int D = decltype(dk)::value, DV = decltype(dvk)::value;
        if (gen)
            masked ? go(decode_stream_kernel<D, DV, true, true>)
                   : go(decode_stream_kernel<D, DV, false, true>);
        else
            masked ? go(decode_stream_kernel<D, DV, true, false>)
                   : go(decode_stream_kernel<D, DV, false, false>);
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    if (d == 128)
        dv == 128 ? pick(I128{}, I128{}) : pick(I128{}, I64{});
    else
        dv == 128 ? pick(I64{}, I128{}) : pick(I64{}, I64{});
}

// Waves of the stream kernel the current device holds at once (compute
// units x resident waves per unit), cached per device, head size and mask
// and general-logit flags (the masked and general kernels hold more
// registers).
int stream_resident_waves(int d, int dv, bool masked, bool gen) {
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices][16];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const int ki = (d == 128 ? 0 : 8) + (dv == 128 ? 0 : 4) + (gen ? 2 : 0) + (masked ? 1 : 0);
    const bool cached = dev >= 0 && dev < kDevices;
    if (cached) {
        const int c = cache[dev][ki].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per = 0;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess || cus <= 0)
        cus = 256;
    auto query = [&](auto kern) {
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 64, 0);
    };
    hipError_t e = hipSuccess;
    with_stream_kernel(d, dv, masked, gen, [&](auto kern) { e = query(kern); });
    if (e != hipSuccess || per <= 0) {
        (void)hipGetLastError();  // a failed query leaves no error for the launches
        per = d == 128 ? 8 : 12;
    }
    const int waves = (int)std::min((long)cus * per, stream_max_waves(d));
    if (cached) cache[dev][ki].store(waves, std::memory_order_relaxed);
    return waves;
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int Hkv, int Skv, int d, int dv) {
    return stream_layout(B, H, Hkv, Skv, d, dv).total;
}

size_t decode_mask_workspace_bytes(int B, int H, int Hkv, int Skv, int d, int dv) {
    const StreamLayout l = stream_layout(B, H, Hkv, Skv, d, dv);
    return l.masked_total - l.total;
}

hipError_t launch_decode_bf16(const LaunchArgs& a) {
    const StreamLayout l = stream_layout(a.B, a.H, a.Hkv, a.Skv, a.d, a.dv);
    // the front end sizes the workspace; refuse rather than write through a bad one
    if (a.workspace == nullptr || a.workspace_bytes < (a.mask ? l.masked_total : l.total))
        return hipErrorInvalidValue;
    const int hgroups = (a.H / a.Hkv + 31) / 32;
    char* ws = static_cast<char*>(a.workspace);
    float* acc = reinterpret_cast<float*>(ws);
    float* ml = reinterpret_cast<float*>(ws + l.ml);
    int* span = reinterpret_cast<int*>(ws + l.span);
    int* counts = a.mask ? reinterpret_cast<int*>(ws + l.counts) : nullptr;
    int* lists = a.mask ? reinterpret_cast<int*>(ws + l.lists) : nullptr;
    // the general instantiation for a bias or a scale that is not positive
    const bool gen = a.bias != nullptr || !(a.scale > 0.0f);
    const int resident = stream_resident_waves(a.d, a.dv, a.mask != nullptr, gen);
    const int waves =
        (int)std::min((long)resident, stream_wave_cap(a.B, a.Hkv, hgroups, a.Skv, a.d));
    const int min_tiles = stream_min_tiles(a.H, a.Hkv);
    const int min_waves = std::max(1, resident / 4);
    const float sl = gen ? kLog2e : a.scale * kLog2e;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* o = static_cast<uint16_t*>(a.out);
    const unsigned pairs = (unsigned)((size_t)a.B * a.Hkv * hgroups);
    KernelTimer* t = active_timer();
    hipError_t e;
    if (a.mask) {
        if (t) t->begin(kDecodeMaskTiles, a.stream);
        hipLaunchKernelGGL(decode_mask_tiles_kernel, dim3(pairs), dim3(256), 0, a.stream, a.mask,
                           a.msb, a.msh, a.kv_lens, a.H, a.Hkv, a.Skv, hgroups, l.ntmax, counts,
                           lists);
        e = hipGetLastError();
        if (t) t->end(kDecodeMaskTiles, a.stream);
        if (e != hipSuccess) return e;
    }
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, a.stream, q, k, v, a.kv_lens, a.B, a.H,
                           a.Hkv, a.Skv, sl, hgroups, min_tiles, min_waves, acc, ml, span, a.mask,
                           a.msb, a.msh, counts, lists, l.ntmax,
                           static_cast<const uint16_t*>(a.bias), a.bsb, a.bsh, a.scale);
    };
    if (t) t->begin(kDecodePartialBf16, a.stream);
    with_stream_kernel(a.d, a.dv, a.mask != nullptr, gen, go);
    e = hipGetLastError();
    if (t) t->end(kDecodePartialBf16, a.stream);
    if (e != hipSuccess) return e;
    if (t) t->begin(kDecodeCombineBf16, a.stream);
    const unsigned heads = (unsigned)((size_t)a.B * a.H);
    if (a.dv == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(heads), dim3(256), 0, a.stream,
                           a.kv_lens, a.H, a.Hkv, a.Skv, hgroups, acc, ml, span, counts, o);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(heads), dim3(256), 0, a.stream,
                           a.kv_lens, a.H, a.Hkv, a.Skv, hgroups, acc, ml, span, counts, o);
    e = hipGetLastError();
    if (t) t->end(kDecodeCombineBf16, a.stream);
    return e;
}

}  // namespace tsda
