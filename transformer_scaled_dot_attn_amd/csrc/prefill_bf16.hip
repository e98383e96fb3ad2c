// bfloat16 prefill: causal / padded attention on the gfx950 matrix cores.
//
// Both products of the method are dense contractions -- the scores Q K^T
// and the mixture P V ("Attention from First Principles", section 5: score
// computation and attn @ V are the O(S^2 d) terms) -- so both run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, and the S x S score
// matrix never leaves registers.
//
// Block = 4 wavefronts = 128 query rows of one (b, h); wave w owns rows
// 32w..32w+31.  The block walks the keys in tiles of 64, staged K and V
// tiles in LDS (two buffers: the next tile's global loads are in flight
// while the current tile is computed).
//
// Transposed products.  Each wave computes S^T = K Q^T (K from LDS as the A
// operand, Q^T held in registers as the B operand).  In the accumulator of
// a 32x32 MFMA a lane holds one column, so every lane owns ONE query and 16
// of its keys; lane l and lane l^32 hold the other 16.  Row maximum and row
// sum are therefore lane-local plus one permlane32 swap.  The mixture is
// computed as O^T = V^T P^T: P^T is the B operand straight from the score
// registers (cast to bf16, as the "Attention from scratch" readable model
// casts its fp32 softmax weights before multiplying by V), and V^T is read
// from the row-major V tile with ds_read_b64_tr_b16 transposing loads.  The
// output accumulator again has one query per lane, so the online-softmax
// rescale is a per-lane scalar multiply.
//
// Masking.  Key j is visible to the query at absolute position p iff
// j < L_b and (not causal or j <= p).  Tiles past the block's last visible
// key are never visited, and a wave stops computing at its own last visible
// key ("Attention from First Principles", section 5: half of the causal
// score matrix is discarded, and good kernels skip it).  Only tiles that cut
// the diagonal or the valid length get per-element masks (-inf logits, so
// exactly zero weight).  Key rows >= L_b are never loaded (the LDS rows are
// zero-filled instead), and query rows >= n_b are written as zeros.
//
// Order.  Block ids are mapped heaviest query tile first, and consecutive
// ids walk the (b, h) pairs, so the tiles of one head land on one XCD (ids
// are dealt round-robin over the 8 XCDs) and share its L2.
#include "device_common.h"
#include "launch.h"

namespace tsda {

namespace {

constexpr int kBM = 128;   // query rows per block
constexpr int kBN = 64;    // keys per tile
constexpr int kThreads = 256;

template <int D>
struct Shape {
    static constexpr int kChunks = D / 8;                     // 16-byte chunks per row
    static constexpr int kKSteps = D / 16;                    // MFMA k-steps of Q K^T
    static constexpr int kDBlocks = D / 32;                   // 32-row blocks of O^T
    static constexpr int kTile = kBN * D;                     // elements per K or V tile
    static constexpr int kPerThread = kBN * kChunks / kThreads;  // 16-byte loads per thread
    static_assert(kPerThread * kThreads == kBN * kChunks, "tile must split evenly");
};

// Position of 16-byte chunk c of LDS row r.  The XOR keeps both access
// patterns free of bank conflicts: 8 consecutive rows reading one chunk
// (the K operand loads) and 4 consecutive rows reading two neighbouring
// chunks (the transposing V loads).
template <int D>
__device__ __forceinline__ int swizzle(int r, int c) {
    if constexpr (D == 128)
        return c ^ ((r & 7) << 1);
    else
        return c ^ (((r >> 1) & 3) << 1);
}

template <int D>
__device__ __forceinline__ int lds_offset(int r, int c) {
    return r * D + swizzle<D>(r, c) * 8;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
    const int32_t* __restrict__ kv_lens, int BH, int H, int Sq, int Skv, float scale_log2,
    int causal, int nqt) {
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][S::kTile];  // [buffer][K, V]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;

    const int bid = blockIdx.x;
    const int qt = nqt - 1 - bid / BH;
    const int bh = bid - (bid / BH) * BH;
    const int b = bh / H;
    const int L = valid_length(kv_lens, b, Skv);
    const int n = Sq < L ? Sq : L;
    const int off = L - n;
    const int q0 = qt * kBM;

    uint16_t* obase = out + (size_t)bh * Sq * D;
    if (q0 >= n) {
        // every row of this tile is padding: write zeros
        const int rows = min(kBM, Sq - q0);
        const u32x4 z = {0, 0, 0, 0};
        for (int e = tid; e < rows * S::kChunks; e += kThreads)
            *reinterpret_cast<u32x4*>(obase + (size_t)q0 * D + e * 8) = z;
        return;
    }

    // keys the whole block may see, and this wave's limits
    const int kv_hi = causal ? min(L, off + min(q0 + kBM, n)) : L;
    const int ntiles = (kv_hi + kBN - 1) / kBN;
    const int qw = q0 + wave * 32;
    const bool wave_live = qw < n;
    const int p_lo = off + qw;
    const int p_hi = off + min(qw + 32, n) - 1;
    const int kv_hi_w = wave_live ? (causal ? min(L, p_hi + 1) : L) : 0;
    const int kfull_w = causal ? min(L, p_lo + 1) : L;

    // this lane's query
    const int qi = qw + (lane & 31);
    const int p = off + qi;
    const bool q_live = qi < n;

    // Q^T fragments: B operand of S^T = K Q^T.  Lane l holds 8 consecutive
    // features 16*ks + 8*(l/32) .. +7 of query (l%32).
    u32x4 qf[S::kKSteps];
    {
        const uint16_t* qrow = q + ((size_t)bh * Sq + (q_live ? qi : 0)) * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks)
            qf[ks] = q_live ? ldg16(qrow + ks * 16) : u32x4{0, 0, 0, 0};
    }

    const uint16_t* kg = k + (size_t)bh * Skv * D;
    const uint16_t* vg = v + (size_t)bh * Skv * D;

    u32x4 kreg[S::kPerThread], vreg[S::kPerThread];
    auto fetch = [&](int tile) {
        const int kbase = tile * kBN;
#pragma unroll
        for (int i = 0; i < S::kPerThread; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / S::kChunks, c = idx % S::kChunks;
            if (kbase + r < L) {
                const size_t g = (size_t)(kbase + r) * D + c * 8;
                kreg[i] = ldg16(kg + g);
                vreg[i] = ldg16(vg + g);
            } else {
                kreg[i] = u32x4{0, 0, 0, 0};
                vreg[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < S::kPerThread; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / S::kChunks, c = idx % S::kChunks;
            const int o = lds_offset<D>(r, c);
            *reinterpret_cast<u32x4*>(&lds[buf][0][o]) = kreg[i];
            *reinterpret_cast<u32x4*>(&lds[buf][1][o]) = vreg[i];
        }
    };

    f32x16 oacc[S::kDBlocks];
#pragma unroll
    for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m_run = -INFINITY;  // running maximum of raw logits (this lane's query)
    float l_run = 0.0f;       // this lane's share of the normaliser

    fetch(0);
    stash(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int kbase = t * kBN;
        if (t + 1 < ntiles) fetch(t + 1);

        if (kbase < kv_hi_w) {
            const uint16_t* kl = lds[buf][0];
            const uint16_t* vl = lds[buf][1];

            // ---- S^T = K Q^T: two 32-key blocks
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
                const int row = kb * 32 + (lane & 31);
#pragma unroll
                for (int ks = 0; ks < S::kKSteps; ++ks) {
                    const u32x4 a =
                        *reinterpret_cast<const u32x4*>(kl + lds_offset<D>(row, 2 * ks + half));
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a),
                                                                       as_bf16x8(qf[ks]),
                                                                       sacc[kb], 0, 0, 0);
                }
            }

            // ---- mask (diagonal / length tiles only)
            if (kbase + kBN > kfull_w) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = kbase + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                        const bool vis = j < L && (!causal || j <= p);
                        if (!vis) sacc[kb][r] = -INFINITY;
                    }
            }

            // ---- online softmax, base 2
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = halves_max(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = fast_exp2((m_run - m_use) * scale_log2);
            const float mc = m_use * scale_log2;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m_run = m_new;

            u32x4 pf[2][2];  // P^T fragments: [key block][16-key step]
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float pr[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pr[r] = fast_exp2(fmaf(sacc[kb][r], scale_log2, -mc));
                    l_run += pr[r];
                }
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pf[kb][h2][i] = pack_bf16(pr[8 * h2 + 2 * i], pr[8 * h2 + 2 * i + 1]);
            }

            // ---- O^T += V^T P^T
            const int g16 = lane >> 4;   // 16-lane group
            const int n16 = lane & 15;
#pragma unroll
            for (int db = 0; db < S::kDBlocks; ++db) {
                const int col = db * 32 + 16 * (g16 & 1) + 4 * (n16 & 3);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int r1 = kb * 32 + h2 * 16 + 4 * half + (n16 >> 2);
                        const int r2 = r1 + 8;
                        const uint16_t* a1 = vl + lds_offset<D>(r1, col >> 3) + (col & 7);
                        const uint16_t* a2 = vl + lds_offset<D>(r2, col >> 3) + (col & 7);
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (TSDA_LDS i16x4*)(a1));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (TSDA_LDS i16x4*)(a2));
                        u32x4 a;
                        a[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
                        a[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
                        a[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
                        a[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            as_bf16x8(a), as_bf16x8(pf[kb][h2]), oacc[db], 0, 0, 0);
                    }
            }
        }

        if (t + 1 < ntiles) stash(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: out = acc / l, rows past n_b are zero
    if (qi < Sq) {
        const float l_tot = halves_sum(l_run);
        const float inv = (q_live && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = obase + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < S::kDBlocks; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = db * 32 + 8 * rg + 4 * half;
                u32x2 w = {0, 0};
                if (q_live) {
                    w[0] = pack_bf16(oacc[db][4 * rg] * inv, oacc[db][4 * rg + 1] * inv);
                    w[1] = pack_bf16(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
                }
                *reinterpret_cast<u32x2*>(orow + d0) = w;
            }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const LaunchArgs& a) {
    const int nqt = (a.Sq + kBM - 1) / kBM;
    const int BH = a.B * a.H;
    const dim3 grid((unsigned)((long)nqt * BH));
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* o = static_cast<uint16_t*>(a.out);
    const float sl = a.scale * kLog2e;
    KernelTimer* t = active_timer();
    if (t) t->begin(kPrefillBf16, a.stream);
    if (a.d == 128)
        hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(kThreads), 0, a.stream, q, k, v, o,
                           a.kv_lens, BH, a.H, a.Sq, a.Skv, sl, a.causal, nqt);
    else
        hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(kThreads), 0, a.stream, q, k, v, o,
                           a.kv_lens, BH, a.H, a.Sq, a.Skv, sl, a.causal, nqt);
    hipError_t e = hipGetLastError();
    if (t) t->end(kPrefillBf16, a.stream);
    return e;
}

}  // namespace tsda
