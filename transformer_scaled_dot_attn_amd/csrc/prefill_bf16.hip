// bfloat16 prefill: causal / padded attention on the gfx950 matrix cores.
//
// Both products of the method are dense contractions -- the scores Q K^T
// and the mixture P V ("Attention from First Principles", section 5: score
// computation and attn @ V are the O(S^2 d) terms) -- so both run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, and the S x S score
// matrix never leaves registers.
//
// Block = 8 wavefronts = 256 query rows of one (b, h); wave w owns rows
// 32w..32w+31, and two waves share each SIMD.  The block walks the keys in
// tiles of 64, staging K and V tiles in two-slot LDS rings.  Grids of at
// most 128 such blocks run blocks of 4 wavefronts = 128 rows instead, and
// grids of at most 64 blocks of 2 wavefronts = 64 rows, so more CUs share
// the walk; a row's arithmetic is the same at every block height.  On such
// small grids (and on plain grids of up to 256 blocks, with 128-row blocks)
// a block may also run two key groups: twice the waves, the second set
// computing the odd key tiles of the same rows, merged at the end.
//
// Transposed products.  Each wave computes S^T = K Q^T (K from LDS as the A
// operand, Q^T held in registers as the B operand).  In the accumulator of
// a 32x32 MFMA a lane holds one column, so every lane owns ONE query and 16
// of its keys; lane l and lane l^32 hold the other 16.  Row maximum and row
// sum are therefore lane-local plus one permlane32 swap.  The mixture is
// computed as O^T = V^T P^T: P^T is the B operand straight from the score
// registers (cast to bf16, as the readable model of "Attention from
// scratch", Open LLM Engineering, casts its fp32 softmax weights before
// multiplying by V), and V^T is read from the row-major V tile with
// ds_read_b64_tr_b16 transposing loads.  The output accumulator again has
// one query per lane, so the online-softmax rescale is a per-lane scalar
// multiply.
//
// Staging.  All threads of the block load the next K and V tiles with
// branch-free 16-byte loads issued between compute blocks and write them to
// LDS at the end of the iteration, one barrier per tile.
//
// Software pipeline.  Within a wave the work of a tile is a chain: Q K^T on
// the matrix cores, then the softmax on the vector ALU, then P V on the
// matrix cores.  Each iteration t overlaps two tiles: the MFMAs of
// S^T(t+1) = K(t+1) Q^T are interleaved with the exponentials of tile t,
// and the P V MFMAs of tile t with the row-maximum scan of tile t+1.  The
// scores of two tiles are therefore live at once (two register sets that
// swap roles every iteration), and the vector work runs while the matrix
// cores are busy instead of between MFMA phases.
//
// Masking.  Key j is visible to the query at absolute position p iff
// j < L_b and (not causal or j <= p).  Tiles past the block's last visible
// key are never visited, and a wave stops computing at its own last visible
// key ("Attention from First Principles", section 5: half of the causal
// score matrix is discarded, and good kernels skip it).  Only tiles that cut
// the diagonal or the valid length get per-element masks (-inf logits, so
// exactly zero weight).  Key rows >= L_b are never loaded (their LDS rows
// hold copies of row L_b - 1, whose weight there is exactly zero), and query
// rows >= n_b are written as zeros.
//
// Explicit allowed-mask (the MASK instantiation).  A byte per (query row,
// key), nonzero = visible, ANDed with the rules above (the boolean allowed-
// mask of "Attention from Scratch", KubeDojo module 1.4.3, Part 3).  Each
// lane needs the 32 bytes of its query row that its score registers hold.
// They are loaded one iteration ahead (under the P V MFMAs) -- by the block
// as coalesced 16-byte chunks of its rows where the rows allow it, else by
// each lane as eight 4-byte words -- and stored into per-lane LDS slots of
// the buffer of the tile's parity before the iteration's barrier, so they
// hold no registers across the score MFMAs.  After the barrier each lane
// reads its words back, the wave decides once whether any of its lanes
// hides a key of the tile, and the per-element pass reads them again.  A
// tile that the mask hides entirely from every live row of a wave is skipped
// by that wave (its weights would all be exactly zero and its maximum -inf).  For a mask shared by all heads, a
// small kernel first reads it once (prefill_mask_tiles_kernel) and marks,
// per query tile and key tile, whether any row of the query tile may see a
// key of the key tile (a mask with one row for all queries and at most 64
// key tiles is marked by the blocks themselves, from that row); each block
// compacts its query tile's marks into an ascending list of key tiles and
// stages and walks only those, so structured masks -- left padding, packed
// documents, sliding windows -- cost only the tiles they open.  The loop
// then runs over list positions: LDS ring slots follow the position, key
// offsets and masks the listed tile.
// The marks also tell a tile that the mask opens whole (every byte of it
// that the causal rule leaves visible is set) from one it cuts; a block
// whose listed tiles are consecutive and all open whole runs the loop of
// the unmasked kernel over them and reads no mask byte, so an all-true mask
// or one that only pads keys costs the tile pre-pass and nothing else.
//
// General logits (the GEN instantiation).  An additive bias (the float mask
// of "Attention from Scratch", KubeDojo module 1.4.3, Part 7: a value added
// to each scaled logit before the softmax; -inf hides the key), or a scale
// that is not positive: each score is rewritten as scale * s + bias before
// the online softmax, which then tracks the maximum of those logits.  The
// lane's 32 bias values of a tile (8-byte groups of 4 keys) are loaded two
// tiles ahead, under the P V MFMAs, and parked in per-lane LDS slots like
// the mask words (coalesced, through two buffers, when there is no mask;
// with a mask, by each lane into one buffer at the next step's start).
// Without a bias the kernel reads a zero array instead.
//
// Order.  Block ids are mapped heaviest query tile first; within a query
// tile rank the (b, h) pairs are laid out so that each XCD (ids are dealt
// round-robin over the 8 XCDs) runs whole heads -- every tile of a head, and
// the query heads that share one K/V head, use one L2 -- with the (b, K/V
// head) units dealt to the XCDs in turn, so that every XCD holds heads of
// every batch item and ragged lengths load the XCDs evenly.
//
// Grouped key/value heads (GQA / MQA): query head h reads K/V head
// h / (H / Hkv) ("Attention from First Principles", section "MHA, GQA, MQA
// -- the KV cache lever"); nothing else changes.
//
// Value width.  V rows and outputs have DV features, K rows D (each 64 or
// 128): softmax(Q K^T) V needs V's rows to line up with K's, not its width
// to match (the d_k = 4, d_v = 2 example of "Attention from Scratch",
// KubeDojo module 1.4.3, Part 2).  Q K^T runs over D, P V over DV.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace tsda {

namespace {

constexpr int kBM = 256;   // query rows per block (128 or 64 on small grids: BM below)
constexpr int kBN = 64;    // keys per tile
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kMaxListTiles = 2048;   // key tiles a block's tile list may hold (Skv <= 131072)

template <int D, int T>  // T: threads of the block
struct Shape {
    static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
    static constexpr int kKSteps = D / 16;                       // MFMA k-steps of Q K^T
    static constexpr int kDBlocks = D / 32;                      // 32-row blocks of O^T
    static constexpr int kPerThread = kBN * kChunks / T;         // 16-byte loads per thread
    static constexpr int kRowsPerPass = T / kChunks;             // tile rows per load pass
    static_assert(kPerThread >= 1 && kPerThread * T == kBN * kChunks,
                  "tile must split evenly");
    // LDS row strides in elements.  LDS reads are served 256 bytes (16
    // groups of 16 bytes) per cycle.  A K row is padded by 16 bytes, so the
    // 16 consecutive rows that 16 lanes read at one chunk (the K operand
    // loads) start in 16 different 16-byte bank groups.  A V row is padded
    // by 64 bytes (for D = 128 row r starts at group 4 r mod 16; for D = 64
    // at 12 r mod 16), so the 4 consecutive rows x 64 bytes that 32 lanes
    // read with one transposing load cover the 16 groups once.  (With a
    // 32-byte pad the 4 rows start 2 groups apart and cover 10 groups:
    // 8.5 M conflict cycles per 4096-token prefill were measured, none with
    // the 64-byte pad.)
    // Every LDS address is then a per-lane base plus a constant.
    static constexpr int kStrideK = D + 8;
    static constexpr int kStrideV = D + 32;
    static constexpr int kTileK = kBN * kStrideK;
    static constexpr int kTileV = kBN * kStrideV;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Scheduling fence: the compiler moves no instruction across it, which keeps
// a batch of LDS reads issued ahead of the MFMAs that consume them.
__device__ __forceinline__ void pin_schedule() { __builtin_amdgcn_sched_barrier(0); }

// Zero bias for GEN calls without one (read as its first 4-element group).
__device__ __attribute__((aligned(16))) uint16_t g_zero_bias[8];

// BM: query rows per block (256, or 128 or 64 on grids that leave CUs
// idle); a wave owns 32 of them.
template <int D, int DV, bool MASK, bool GEN, int BM, int KG>
__global__ __launch_bounds__(2 * BM * KG, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
    const int32_t* __restrict__ kv_lens, int BH, int H, int Hkv, int Sq, int Skv, float scale_log2,
    int causal, int nqt, int nsplit, float* __restrict__ ws_acc, float* __restrict__ ws_ml,
    const uint8_t* __restrict__ allowed, long long msb, long long msh, long long msi,
    const uint8_t* __restrict__ tmap, int nkt, const uint16_t* __restrict__ bias, long long bsb,
    long long bsh, long long bsi, float scale) {
    constexpr int kBMb = BM;            // query rows of this block
    constexpr int kRowWaves = BM / 32;  // waves per key group, 32 rows each
    constexpr int kThreads = 64 * kRowWaves * KG;
    static_assert(KG == 1 || (KG == 2 && !MASK && !GEN), "key groups: unmasked plain logits");
    using S = Shape<D, kThreads>;    // the key side: Q K^T over D features
    using SV = Shape<DV, kThreads>;  // the value side: V rows and outputs of DV features
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][S::kTileK];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][SV::kTileV];
    // parked mask words, 32 bytes per lane, two buffers (list positions of each parity)
    __shared__ u32x4 lds_m[MASK ? 4 * kThreads : 1];
    __shared__ int lds_tl[MASK ? kMaxListTiles : 1];  // this query tile's listed key tiles
    __shared__ int lds_tn;                            // their number
    __shared__ int lds_tcut;                          // some listed tile is cut by the mask
    // parked bias, 64 bytes per lane (two buffers without a mask: tiles of each parity)
    __shared__ u32x4 lds_b[GEN ? (MASK ? 1 : 2) * 4 * kThreads : 1];
    // key group 1's (acc, m, l) per lane for the merge (KG = 2)
    __shared__ float lds_x[KG == 2 ? kRowWaves * (SV::kDBlocks * 16 + 2) * 64 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rg = wave % kRowWaves;  // row group: rows 32 rg .. 32 rg + 31 of the block
    const int kg = wave / kRowWaves;  // key group (KG = 2: tiles of parity kg)
    const int half = lane >> 5;

    const int bid = blockIdx.x;
    const int qt = nqt - 1 - bid / (BH * nsplit);
    const int rem = bid - (bid / (BH * nsplit)) * (BH * nsplit);
    const int split = rem / BH;  // key-range split of this query tile
    const int jb = rem - split * BH;
    // Blocks are dealt to the 8 XCDs round-robin by id.  When the (b, K/V
    // head) units, each with the g = H / Hkv query heads that share it, number
    // a multiple of 8, unit u runs on XCD u mod 8: every query tile of a head,
    // and the heads of one K/V group, meet in one L2, and each XCD holds heads
    // of every batch item, so ragged lengths load the XCDs evenly.  Otherwise,
    // with BH a multiple of 8, XCD x runs the contiguous (b, h) pairs
    // x*BH/8 .. (x+1)*BH/8 - 1.
    const int g = H / Hkv;
    const int units = BH / g;
    int bh = jb;
    if ((units & 7) == 0) {
        const int i = jb >> 3;
        bh = ((jb & 7) + 8 * (i / g)) * g + i % g;
    } else if ((BH & 7) == 0) {
        bh = (jb & 7) * (BH >> 3) + (jb >> 3);
    }
    const int b = bh / H;
    const int bk = b * Hkv + (bh - b * H) / (H / Hkv);  // this head's K/V head
    const int L = valid_length(kv_lens, b, Skv);
    const int n = Sq < L ? Sq : L;
    const int off = L - n;
    // Query tile rows.  Without a mask the tiles end at the last valid row
    // (q0 = n - (nqt - qt) BM; rows below 0 are dead), so a sequence's partly
    // filled tile is its first one, whose rows see the fewest keys; the pad
    // rows n .. Sq-1 are zeroed by the blocks of the tiling from row 0 (block
    // qt: rows qt BM .. qt BM + BM - 1).  With a mask the tiles start at
    // row 0, as the key-tile marks do.
    const int qz = qt * kBMb;
    const int q0 = MASK ? qz : n - (nqt - qt) * kBMb;

    uint16_t* obase = out + (size_t)bh * Sq * DV;
    // pad rows are zero (without splits; the split combine zeroes them itself)
    const int z0 = max(qz, n), z1 = min(qz + kBMb, Sq);
    if (nsplit == 1 && z0 < z1 && (!MASK || q0 >= n)) {
        const u32x4 z = {0, 0, 0, 0};
        for (int e = tid; e < (z1 - z0) * SV::kChunks; e += kThreads)
            *reinterpret_cast<u32x4*>(obase + (size_t)z0 * DV + e * 8) = z;
    }
    if (q0 >= n || q0 + kBMb <= 0) return;  // no valid row in this tile

    // keys the whole query tile may see, this block's split of them, and
    // this wave's limits: tiles t0 <= t < t1 of the block, t < t1w of the wave
    const int kv_hi = causal ? min(L, off + min(q0 + kBMb, n)) : L;
    const int ntiles_q = (kv_hi + kBN - 1) / kBN;
    const int per_split = (ntiles_q + nsplit - 1) / nsplit;
    const int t0 = min(ntiles_q, split * per_split);
    const int t1 = min(ntiles_q, t0 + per_split);
    const int qw = q0 + rg * 32;
    const bool wave_live = qw < n && qw + 32 > 0;
    const int p_lo = off + qw;
    const int p_hi = off + min(qw + 32, n) - 1;
    const int kv_hi_w = wave_live ? (causal ? min(L, p_hi + 1) : L) : 0;
    int t1w = min(t1, (kv_hi_w + kBN - 1) / kBN);  // this wave computes t0 <= t < t1w
    const int kfull_w = causal ? min(L, p_lo + 1) : L;
    const int tw = (kv_hi_w + kBN - 1) / kBN;  // key tiles this wave's rules reach

    // this lane's query
    const int qi = qw + (lane & 31);
    const int p = off + qi;
    const bool q_live = qi >= 0 && qi < n;

    // Q^T fragments: B operand of S^T = K Q^T.  Lane l holds 8 consecutive
    // features 16*ks + 8*(l/32) .. +7 of query (l%32).
    // Loaded directly, each of a lane's loads would touch 32 rows, 32 bytes
    // each; so the block reads its Q rows coalesced instead (thread t: the
    // 16-byte chunks t + kThreads i of the row-major tile, consecutive
    // threads on consecutive bytes), together with the walk's first K/V
    // tiles, and hands them to the fragments through per-wave LDS regions
    // (stage_q) before those tiles are stored there.  Rows outside the
    // sequence's queries read as zero.  Where the regions do not fit in the
    // K/V slots (d = 128 with d_v = 64 at 256 rows), lanes load their
    // fragments directly, before the key-tile list is built.
    constexpr int kQRegion = 32 * S::kStrideK;                // one wave's Q rows
    constexpr int kQRegK = 2 * S::kTileK / kQRegion;          // regions in lds_k
    constexpr int kQRegV = 2 * SV::kTileV / kQRegion;         // regions in lds_v
    constexpr bool kQStaged = kQRegK + kQRegV >= kRowWaves;
    constexpr int kQChunks = kQStaged ? kBMb * S::kChunks / kThreads : 1;
    static_assert(!kQStaged || kQChunks * kThreads == kBMb * S::kChunks, "Q tile must split evenly");
    u32x4 qf[S::kKSteps];
    u32x4 qtmp[kQChunks];
    if constexpr (!kQStaged) {
        const uint16_t* qrow = q + ((size_t)bh * Sq + (q_live ? qi : 0)) * D + half * 8;
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks)
            qf[ks] = q_live ? ldg16(qrow + ks * 16) : u32x4{0, 0, 0, 0};
    }
    auto q_region = [&](int w) -> uint16_t* {
        return w < kQRegK ? &lds_k[0][0] + w * kQRegion : &lds_v[0][0] + (w - kQRegK) * kQRegion;
    };
    // Issued with the first K/V loads of the walk (one memory round trip).
    auto load_q = [&]() {
        if constexpr (kQStaged) {
#pragma unroll
            for (int i = 0; i < kQChunks; ++i) {
                const int c = tid + kThreads * i;
                const int r = min(max(q0 + c / S::kChunks, 0), Sq - 1);
                qtmp[i] = ldg16(q + ((size_t)bh * Sq + r) * D + (c % S::kChunks) * 8);
            }
        }
    };
    // Called once by every wave, while no K/V tile is in LDS yet.
    auto stage_q = [&]() {
        if constexpr (kQStaged) {
#pragma unroll
            for (int i = 0; i < kQChunks; ++i) {
                const int c = tid + kThreads * i;
                const int r = c / S::kChunks, qr = q0 + r;
                const u32x4 z = {0, 0, 0, 0};
                *reinterpret_cast<u32x4*>(q_region(r >> 5) + (r & 31) * S::kStrideK +
                                          (c % S::kChunks) * 8) = qr >= 0 && qr < n ? qtmp[i] : z;
            }
            __syncthreads();
            const uint16_t* src = q_region(rg) + (lane & 31) * S::kStrideK + half * 8;
#pragma unroll
            for (int ks = 0; ks < S::kKSteps; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(src + ks * 16);
            __syncthreads();
        }
    };


    // Masked calls walk list positions pp0 <= pos < pp1 of the key tiles the
    // mask opens to this query tile (all tiles when no list is given);
    // tix(pos) is the key tile at a position (positions past the list map to
    // its last tile, a valid one, for the staging run-ahead).
    int pp0 = t0, pp1 = t1;
    bool listed = false;
    bool dense = false;  // the listed tiles are consecutive and all open whole
    int lcount = 0, tl0 = 0;
    if constexpr (MASK) {
        if (tmap != nullptr) {  // the mask is shared by all heads (msh == 0)
            listed = true;
            const uint8_t* tm = tmap + ((size_t)(msb != 0 ? b : 0) * nqt + qt) * nkt;
            // A mask with one row for all queries (msi == 0) and at most 64
            // key tiles (one round below) has no pre-pass: each lane marks its
            // key tile from the row's 64 bytes, counting the bytes the
            // pre-pass would (keys below Skv; under the causal rule, keys up
            // to this query tile's last row's position bound).  Longer rows
            // keep the pre-pass, which costs one launch instead of a memory
            // round trip per round in every block.
            const bool row_marks = msi == 0 && nkt <= 64;
            const uint8_t* mrow = allowed + b * msb;
            const int mrow_last = mask_last_word(Skv);
            const int qlast = min(qz + kBMb, Sq) - 1;
            auto row_mark = [&](int kt) -> int {
                uint32_t wd[16];
#pragma unroll
                for (int w = 0; w < 16; ++w) wd[w] = ldg_word(mrow + min(kt * kBN + 4 * w, mrow_last));
                uint32_t any = 0, hole = 0;
#pragma unroll
                for (int w = 0; w < 16; ++w) {
                    const int c = kt * kBN + 4 * w;
                    int nb = c <= mrow_last ? Skv - c : 0;  // bytes counted: keys c .. c + nb - 1
                    if (causal) nb = min(nb, Skv - Sq + qlast - c + 1);
                    const uint32_t ign = nb >= 4 ? 0u : nb <= 0 ? ~0u : ~0u << (8 * nb);
                    any |= wd[w] & ~ign;
                    hole |= has_zero_byte(wd[w] | ign);
                }
                return any != 0 ? (hole != 0 ? 1 : 2) : 0;
            };
            if (wave == 0) {
                // compact the marks of key tiles 0 .. ntiles_q-1 in ascending
                // order: 64 tiles per round, a lane each, ballot and prefix count
                int base = 0;
                bool cut = false;
                for (int k0 = 0; k0 < ntiles_q; k0 += 64) {
                    const int kt = k0 + lane;
                    const int mk = kt >= ntiles_q ? 0 : row_marks ? row_mark(kt) : tm[min(kt, nkt - 1)];
                    const uint64_t bal = __builtin_amdgcn_ballot_w64(mk != 0);
                    cut |= __builtin_amdgcn_ballot_w64(mk == 1) != 0;
                    if (mk != 0) lds_tl[base + __builtin_popcountll(bal & ((1ull << lane) - 1))] = kt;
                    base += __builtin_popcountll(bal);
                }
                if (lane == 0) {
                    lds_tn = base;
                    lds_tcut = cut;
                }
            }
            __syncthreads();
            lcount = lds_tn;
            tl0 = lcount > 0 ? lds_tl[0] : 0;
            dense = lds_tcut == 0 && lcount > 0 && lds_tl[lcount - 1] - tl0 + 1 == lcount;
            const int per = (lcount + nsplit - 1) / nsplit;
            pp0 = min(lcount, split * per);
            pp1 = min(lcount, pp0 + per);
        }
    }
    auto tix = [&](int pos) -> int {
        if constexpr (MASK) {
            if (listed) return lcount > 0 ? lds_tl[min(pos, lcount - 1)] : 0;
        }
        return pos;
    };

    // ---- allowed-mask words of this lane's query row for one key tile:
    // word w holds keys 32 (w/4) + 8 (w%4) + 4 half .. +3, the keys of
    // score elements 4 (w%4) .. +3 of block w/4.  A list position's words
    // are loaded one step ahead (mload), stored into the LDS buffer of the
    // position's parity before a barrier (mwrite) and read back by their
    // lane after it (mread, which also sets mcut and mnone); mask() reads
    // them from the same buffer.
    // Two ways to load them, the same words either way:
    //  - coalesced (mvec: keys in whole 64-key tiles, 16-byte aligned rows):
    //    the block reads its rows' 64 bytes of the tile as 16-byte chunks,
    //    consecutive threads on consecutive chunks, and mwrite scatters each
    //    chunk's four words to the two lanes that own them;
    //  - per lane: each lane reads its own 8 words, offsets clamped to the
    //    row's last readable word (keys past it are >= Skv >= L and hidden
    //    by the length rule anyway).
    // Reading its own words, each load of a lane touches 32 rows; the
    // coalesced loads were measured 15 % faster on a per-element mask.
    u32x4 mw[2];  // in flight: word w is mw[w / 4][w % 4], or the two chunks (mvec)
    bool mcut = false;   // some lane of the wave hides a key of the parked tile
    bool mnone = false;  // no live lane of the wave sees a key of the parked tile
    int mbuf = 0;        // the LDS buffer of the parked tile
    // per lane: a wave-uniform row base (row min(qw, Sq-1)) plus a 32-bit
    // lane offset (qi - that row) * msi, below 32 * msi <= 2^32; pad lanes
    // read the base row
    // (coalesced: the block's first row as the base, 32-bit row offsets)
    const uint8_t* mbase = nullptr;
    const uint8_t* mblk = nullptr;
    uint32_t mlane = 0;
    bool mvec = false;
    if constexpr (MASK) {
        const int r0 = __builtin_amdgcn_readfirstlane(min(qw, Sq - 1));  // uniform: SGPR base
        const uint8_t* mhead = allowed + b * msb + (long long)(bh - b * H) * msh;
        mbase = mhead + (long long)r0 * msi;
        mblk = mhead + (long long)qz * msi;  // qz < Sq
        mlane = q_live ? (uint32_t)(qi - r0) * (uint32_t)msi : 0u;
        mvec = Skv % kBN == 0 && (reinterpret_cast<uintptr_t>(mblk) & 15u) == 0 && (msi & 15) == 0 &&
               (long long)kBMb * msi + Skv <= (long long)UINT32_MAX;
    }
    const int mlast = mask_last_word(Skv);
    constexpr int kMChunks = kBMb * 4 / kThreads;  // 16-byte chunks per thread (coalesced)
    static_assert(!MASK || kMChunks == 2, "two mask chunks per thread");
    auto mload = [&](int tile) {
        if constexpr (MASK) {
            if (mvec) {
                // run-ahead positions past the last key tile (unlisted masks)
                // read the last tile; their words are never used
                tile = min(tile, Skv / kBN - 1);
#pragma unroll
                for (int i = 0; i < kMChunks; ++i) {
                    const int c = tid + kThreads * i;  // row c / 4, keys 16 (c % 4) ..
                    const uint32_t rr = (uint32_t)min(c / 4, Sq - 1 - qz);
                    mw[i] = ldg16(mblk + (rr * (uint32_t)msi + (uint32_t)(tile * kBN + (c % 4) * 16)));
                }
            } else {
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const int j = tile * kBN + 32 * (w >> 2) + 8 * (w & 3) + 4 * half;
                    mw[w >> 2][w & 3] = ldg_word(mbase + (mlane + (uint32_t)min(j, mlast)));
                }
            }
        }
    };
    // Before a barrier; the buffer's last readers are behind the one before.
    auto mwrite = [&](int pos) {
        if constexpr (MASK) {
            u32x4* buf = lds_m + (pos & 1) * 2 * kThreads;
            if (mvec) {
#pragma unroll
                for (int i = 0; i < kMChunks; ++i) {
                    // chunk part p holds words w0, w0 + 1 (w0 = 4 (p/2) + 2 (p%2)) of
                    // the row's two lanes: its words 0, 2 for half 0, 1, 3 for half 1
                    const int c = tid + kThreads * i;
                    const int r = c / 4, part = c % 4;
                    const int w0 = 4 * (part >> 1) + 2 * (part & 1);
                    const int lt = 64 * (r >> 5) + (r & 31);  // the row's half-0 lane
                    uint32_t* b0 = reinterpret_cast<uint32_t*>(buf + 2 * lt) + w0;
                    uint32_t* b1 = reinterpret_cast<uint32_t*>(buf + 2 * (lt + 32)) + w0;
                    *reinterpret_cast<u32x2*>(b0) = u32x2{mw[i][0], mw[i][2]};
                    *reinterpret_cast<u32x2*>(b1) = u32x2{mw[i][1], mw[i][3]};
                }
            } else {
                buf[2 * tid] = mw[0];
                buf[2 * tid + 1] = mw[1];
            }
        }
    };
    // After the barrier that follows mwrite(pos).
    auto mread = [&](int pos) {
        if constexpr (MASK) {
            mbuf = pos & 1;
            const u32x4* buf = lds_m + mbuf * 2 * kThreads;
            const u32x4 m0 = buf[2 * tid], m1 = buf[2 * tid + 1];
            uint32_t z = 0, nz = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                z |= has_zero_byte(m0[w]) | has_zero_byte(m1[w]);
                nz |= m0[w] | m1[w];
            }
            mcut = __builtin_amdgcn_ballot_w64(z != 0) != 0;
            mnone = __builtin_amdgcn_ballot_w64(q_live && nz != 0) == 0;
        }
    };

    // ---- bias of this lane's query row for one key tile (GEN): group
    // (kb, g) holds keys 32 kb + 8 g + 4 half .. +3, those of score elements
    // 4 g .. 4 g + 3 of block kb.  Addressed like the mask words: a
    // wave-uniform row base plus a 32-bit lane offset; group offsets are
    // clamped to the row's last readable group (keys past it are >= Skv >= L
    // and hidden).  Without a bias every group reads the zero array.
    // Without a mask, where the keys come in whole 64-key tiles and the rows
    // are 16-byte aligned (bvec), the block reads its rows' 128 bytes of the
    // tile coalesced instead, as 16-byte chunks (four per thread, held in
    // bw), and bwrite scatters each chunk's two groups to their lanes through
    // the LDS buffer of the tile's parity (written before a barrier, read
    // after it; the scheme of the mask words below).
    u32x2 bw[2][4];
    const uint8_t* bbase = nullptr;  // byte addresses: 32-bit lane offsets below 2^32
    const uint8_t* bblk = nullptr;   // (bvec: the block's first row in the sequence)
    uint32_t blane = 0;
    int blast = 0;
    int brb = 0;
    bool bvec = false;
    int bbuf = 0;  // the LDS buffer of the parked tile
    if constexpr (GEN) {
        // without a mask a tile's first waves may start at a negative row
        // (tiles end at the last valid row): the base row is clamped to 0
        const int r0 = __builtin_amdgcn_readfirstlane(min(max(qw, 0), Sq - 1));
        if (bias != nullptr) {
            const uint16_t* bhead = bias + b * bsb + (long long)(bh - b * H) * bsh;
            bbase = reinterpret_cast<const uint8_t*>(bhead + (long long)r0 * bsi);
            blane = q_live ? 2u * (uint32_t)(qi - r0) * (uint32_t)bsi : 0u;
            blast = bias_last_group(Skv);
            brb = min(max(q0, 0), Sq - 1);
            bblk = reinterpret_cast<const uint8_t*>(bhead + (long long)brb * bsi);
            bvec = !MASK && Skv % kBN == 0 && (reinterpret_cast<uintptr_t>(bblk) & 15u) == 0 &&
                   (bsi & 7) == 0 && 2LL * kBMb * bsi + 2LL * Skv <= (long long)UINT32_MAX;
        } else {
            bbase = reinterpret_cast<const uint8_t*>(g_zero_bias);
        }
    }
    constexpr int kBChunks = kBMb * 8 / kThreads;  // 16-byte chunks per thread (bvec)
    static_assert(!GEN || kBChunks == 4, "four bias chunks per thread");
    auto bload = [&](int tile) {
        if constexpr (GEN) {
            if (bvec) {
                // the steps load two tiles ahead: past the last key tile they
                // read the last one, never used
                tile = min(tile, Skv / kBN - 1);
#pragma unroll
                for (int i = 0; i < kBChunks; ++i) {
                    const int c = tid + kThreads * i;  // row c / 8, keys 8 (c % 8) ..
                    const int rr = min(max(q0 + c / 8, 0), Sq - 1);
                    const u32x4 ch = ldg16(bblk + (2u * (uint32_t)(rr - brb) * (uint32_t)bsi +
                                                   (uint32_t)(2 * tile * kBN + 16 * (c % 8))));
                    bw[i >> 1][2 * (i & 1)] = u32x2{ch[0], ch[1]};
                    bw[i >> 1][2 * (i & 1) + 1] = u32x2{ch[2], ch[3]};
                }
                return;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int j = tile * kBN + 32 * kb + 8 * g + 4 * half;
                    bw[kb][g] = *reinterpret_cast<const u32x2*>(
                        bbase + (blane + 2u * (uint32_t)min(j, blast)));
                }
        }
    };
    auto bpark = [&]() {
        if constexpr (GEN) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    lds_b[4 * tid + 2 * kb + h2] = u32x4{bw[kb][2 * h2][0], bw[kb][2 * h2][1],
                                                         bw[kb][2 * h2 + 1][0], bw[kb][2 * h2 + 1][1]};
        }
    };
    // Without a mask: before a barrier, into the buffer of the tile's parity,
    // whose last readers are behind the barrier before.
    auto bwrite = [&](int tile) {
        if constexpr (GEN && !MASK) {
            u32x4* buf = lds_b + (tile & 1) * 4 * kThreads;
            if (bvec) {
#pragma unroll
                for (int i = 0; i < kBChunks; ++i) {
                    // chunk part p: group (p / 4, p % 4) of the row's half-0 lane,
                    // then the same group of its half-1 lane
                    const int c = tid + kThreads * i;
                    const int r = c / 8, part = c % 8, kb = part >> 2, g = part & 3;
                    const int lt = 64 * (r >> 5) + (r & 31);
                    *(reinterpret_cast<u32x2*>(buf + 4 * lt + 2 * kb + (g >> 1)) + (g & 1)) =
                        bw[i >> 1][2 * (i & 1)];
                    *(reinterpret_cast<u32x2*>(buf + 4 * (lt + 32) + 2 * kb + (g >> 1)) + (g & 1)) =
                        bw[i >> 1][2 * (i & 1) + 1];
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
                        buf[4 * tid + 2 * kb + h2] = u32x4{bw[kb][2 * h2][0], bw[kb][2 * h2][1],
                                                           bw[kb][2 * h2 + 1][0], bw[kb][2 * h2 + 1][1]};
            }
        }
    };
    // bias of a tile: parked at the step's start with a mask, else written
    // before the last barrier (bwrite) and taken from the tile's buffer
    auto bhere = [&](int tile) {
        if constexpr (MASK) bpark();
        else bbuf = tile & 1;
    };

    // ---- tile staging: thread t moves 16-byte chunks t + 512 i of the
    // row-major tile, so consecutive threads read consecutive global bytes.
    // The loads are branch-free, so they stay in flight through the compute
    // (no wait until the stash): a row at or past L is clamped to row L - 1
    // of the same head (valid, L >= 1 here), so padded rows are never read;
    // the keys it stands for are masked (-inf logits), so its copy adds an
    // exact zero to the mixture (2 % faster than zero-filling it).  K runs two
    // tiles ahead of the scores, V one tile.  Addresses are the head's base
    // (wave-uniform) plus a 32-bit byte offset per lane: a head's rows span
    // less than 4 GiB (the front end refuses larger heads), so a load costs
    // a min and a multiply-add.
    const int st_row = tid / S::kChunks;
    const int st_col = (tid % S::kChunks) * 8;
    const int st_row_v = tid / SV::kChunks;
    const int st_col_v = (tid % SV::kChunks) * 8;
    const char* khead = reinterpret_cast<const char*>(k + (size_t)bk * Skv * D);
    const char* vhead = reinterpret_cast<const char*>(v + (size_t)bk * Skv * DV);
    u32x4 kreg[S::kPerThread], vreg[SV::kPerThread];
    auto fetch_k_to = [&](int tile, u32x4 (&dst)[S::kPerThread]) {
        const int kbase = tile * kBN;
#pragma unroll
        for (int i = 0; i < S::kPerThread; ++i) {
            const int row = min(kbase + st_row + i * S::kRowsPerPass, L - 1);
            dst[i] = ldg16(khead + ((uint32_t)row * (2u * D) + (uint32_t)st_col * 2u));
        }
    };
    auto fetch_v_to = [&](int tile, u32x4 (&dst)[SV::kPerThread]) {
        const int kbase = tile * kBN;
#pragma unroll
        for (int i = 0; i < SV::kPerThread; ++i) {
            const int row = min(kbase + st_row_v + i * SV::kRowsPerPass, L - 1);
            dst[i] = ldg16(vhead + ((uint32_t)row * (2u * DV) + (uint32_t)st_col_v * 2u));
        }
    };
    auto stash_k_from = [&](int tile, const u32x4 (&src)[S::kPerThread]) {
        uint16_t* dk = lds_k[tile & 1] + st_row * S::kStrideK + st_col;
#pragma unroll
        for (int i = 0; i < S::kPerThread; ++i)
            *reinterpret_cast<u32x4*>(dk + i * S::kRowsPerPass * S::kStrideK) = src[i];
    };
    auto stash_v_from = [&](int tile, const u32x4 (&src)[SV::kPerThread]) {
        uint16_t* dv = lds_v[tile & 1] + st_row_v * SV::kStrideV + st_col_v;
#pragma unroll
        for (int i = 0; i < SV::kPerThread; ++i)
            *reinterpret_cast<u32x4*>(dv + i * SV::kRowsPerPass * SV::kStrideV) = src[i];
    };
    auto fetch_k = [&](int tile) { fetch_k_to(tile, kreg); };
    auto fetch_v = [&](int tile) { fetch_v_to(tile, vreg); };
    auto stash_k = [&](int tile) { stash_k_from(tile, kreg); };
    auto stash_v = [&](int tile) { stash_v_from(tile, vreg); };

    // Per-lane LDS read bases (element offsets within a slot).
    //  K operand of S^T: row 32*kb + lane%32, features 16*ks + 8*(lane/32).
    const int k_rd = (lane & 31) * S::kStrideK + half * 8;
    //  V^T operand via ds_read_b64_tr_b16: within each 16-lane group, source
    //  lane i reads features col0 + 4*(i%4) .. +3 of key row key0 + i/4, and
    //  result lane n then holds V[key0 + 0..3][col0 + n].  Lanes of the
    //  second half take keys 4..7 (and 12..15) of each 16-key step, which
    //  matches the keys their P^T fragment holds.
    const int n16 = lane & 15;
    const int v_rd = (4 * half + (n16 >> 2)) * SV::kStrideV + 16 * ((lane >> 4) & 1) + 4 * (n16 & 3);

    f32x16 oacc[SV::kDBlocks];
#pragma unroll
    for (int db = 0; db < SV::kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m_run = -INFINITY;  // reference maximum of raw logits (this lane's query)
    float ref_run = 0.0f;     // m_run * scale_log2, 0 while m_run = -inf (set where m_run moves)
    float l_run = 0.0f;       // this lane's share of the normaliser
    f32x16 s0[2], s1[2];      // S^T of two consecutive tiles (two 32-key blocks each)
    u32x4 pf[2][2];           // P^T fragments of the tile being mixed

    constexpr int kQK = 2 * S::kKSteps;       // MFMAs of S^T per tile
    constexpr int kHalf = 2 * SV::kDBlocks;   // P V MFMAs per 32-key block
    constexpr int kPV = 2 * kHalf;            // P V MFMAs per tile
    constexpr int kAheadK = 2;                // K operand k-steps in flight
    constexpr int kAheadV = 3;                // V operands in flight
    // The 18 weight stages of a tile (below) are split between the MFMAs of
    // the next tile's scores (the first kNA) and the first kHalf P V MFMAs
    // of the tile itself (the rest), which read only the first 32-key block
    // of P: in proportion to the MFMAs that hide them, and at least 9 ahead
    // of P V (stage 8 packs the block's last pair).
    constexpr int kNA = std::clamp((18 * kQK + (kQK + kHalf) / 2) / (kQK + kHalf), 9, 18);

    // ---- pieces of S^T(tile) = K Q^T: two 32-key blocks, chains interleaved
    auto kread = [&](const uint16_t* kl, int ks, u32x4 (&dst)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            dst[kb] = *reinterpret_cast<const u32x4*>(kl + kb * 32 * S::kStrideK + ks * 16);
    };
    // ---- one pair of weights of P = 2^(s*scale*log2e - reference), packed to
    // bf16; the normaliser sums the bf16 weights the mixture uses, in the
    // fixed order kb, h2, i.
    // Three stages per pair e = 8 kb + 4 h2 + i, issued in a rolling window
    // (exponentials of pair e, bf16 packing of pair e-1, normaliser update
    // of pair e-2), so no instruction waits on the result of the one just
    // before it; empty volatile uses keep each stage where it is issued
    // (under the MFMAs) instead of letting it sink to its first reader.
    float ex[2][2];  // exponentials of the two most recent pairs
    auto pair_stage = [&](const f32x16 (&sc)[2], int e, float mc) {
        if (e < 16) {
            const int kb = e >> 3, h2 = (e >> 2) & 1, i = e & 3;
            ex[e & 1][0] = fast_exp2(fmaf(sc[kb][8 * h2 + 2 * i], scale_log2, -mc));
            ex[e & 1][1] = fast_exp2(fmaf(sc[kb][8 * h2 + 2 * i + 1], scale_log2, -mc));
        }
        if (e >= 1 && e - 1 < 16) {
            const int f = e - 1, kb = f >> 3, h2 = (f >> 2) & 1, i = f & 3;
            pf[kb][h2][i] = pack_bf16(ex[f & 1][0], ex[f & 1][1]);
            asm volatile("" : "+v"(pf[kb][h2][i]));
        }
        if (e >= 2 && e - 2 < 16) {
            const int f = e - 2, kb = f >> 3, h2 = (f >> 2) & 1, i = f & 3;
            l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pf[kb][h2][i]), as_bf16x2(0x3F803F80u),
                                                    l_run, false);
            asm volatile("" : "+v"(l_run));
        }
    };
    auto ref_log2 = [&]() { return ref_run; };

    // S^T(tile) into sn; when sc is given, weight stages 0 .. kNA-1 of the
    // tile before it are issued under these MFMAs.
    auto score = [&](int tile, f32x16 (&sn)[2], const f32x16 (*sc)[2]) {
        const uint16_t* kl = lds_k[tile & 1] + k_rd;
        const float mc = ref_log2();
        u32x4 ka[kAheadK + 1][2];
#pragma unroll
        for (int ks = 0; ks < kAheadK; ++ks) kread(kl, ks, ka[ks]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sn[kb][r] = 0.0f;
        pin_schedule();
#pragma unroll
        for (int ks = 0; ks < S::kKSteps; ++ks) {
            if (ks + kAheadK < S::kKSteps) kread(kl, ks + kAheadK, ka[(ks + kAheadK) % (kAheadK + 1)]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(ka[ks % (kAheadK + 1)][kb]), as_bf16x8(qf[ks]), sn[kb], 0, 0, 0);
                if (sc) {
                    const int m = 2 * ks + kb;  // MFMA index: stages kNA m / kQK .. kNA (m+1) / kQK - 1
#pragma unroll
                    for (int e = kNA * m / kQK; e < kNA * (m + 1) / kQK; ++e) pair_stage(*sc, e, mc);
                }
                pin_schedule();
            }
        }
    };
    // weights of a tile with no next tile to score under them
    auto weigh = [&](const f32x16 (&sc)[2]) {
        const float mc = ref_log2();
#pragma unroll
        for (int e = 0; e < 18; ++e) pair_stage(sc, e, mc);
    };
    // per-element mask of S^T(tile) when the tile cuts the diagonal or L,
    // or (MASK) when the allowed-mask hides a key of the tile in some lane.
    // The rules leave keys 0 .. lim visible (lim = min(p, L - 1) causal,
    // L - 1 otherwise), so each element costs one compare against a
    // per-tile constant -- no short-circuit branches.
    const int lim = causal ? min(p, L - 1) : L - 1;
    // UM (the tag's value): the allowed-mask words are read.
    auto mask = [&](auto um, int tile, f32x16 (&sn)[2]) {
        constexpr bool UM = decltype(um)::value;
        const int kbase = tile * kBN;
        if constexpr (GEN) {
            // logits scale * s + bias (the parked bias of this tile)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const u32x4 w4 = lds_b[bbuf * 4 * kThreads + 4 * tid + 2 * kb + h2];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int r = 8 * h2 + e;  // groups 2 h2, 2 h2 + 1: elements 8 h2 .. +7
                        const uint32_t wd = w4[e >> 1];
                        const float bv = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
                        sn[kb][r] = fmaf(sn[kb][r], scale, bv);
                    }
                    pin_schedule();  // one 16-byte group in registers at a time
                }
        }
        u32x4 mk[2] = {{~0u, ~0u, ~0u, ~0u}, {~0u, ~0u, ~0u, ~0u}};
        if (kbase + kBN > kfull_w) {
            // the rules cut this tile (and the allowed-mask may)
            if constexpr (UM) {
                mk[0] = lds_m[mbuf * 2 * kThreads + 2 * tid];
                mk[1] = lds_m[mbuf * 2 * kThreads + 2 * tid + 1];
            }
            const int rel = lim - kbase - 4 * half;  // element visible iff its offset <= rel
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    bool vis = kb * 32 + 8 * (r >> 2) + (r & 3) <= rel;
                    if constexpr (UM) vis = vis & byte_set(mk[kb][r >> 2], r & 3);
                    sn[kb][r] = vis ? sn[kb][r] : -INFINITY;
                }
        } else if constexpr (UM) {
            if (mcut) {
                // only the allowed-mask cuts it
                mk[0] = lds_m[mbuf * 2 * kThreads + 2 * tid];
                mk[1] = lds_m[mbuf * 2 * kThreads + 2 * tid + 1];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sn[kb][r] = byte_set(mk[kb][r >> 2], r & 3) ? sn[kb][r] : -INFINITY;
            }
        }
    };
    // O^T += V^T(tile) P^T, output blocks innermost (consecutive MFMAs
    // independent).  When sc (the tile's scores) is given, weight stages
    // kNA .. 17 are issued under the first kHalf MFMAs, which use only the
    // first 32-key block of P; when sn is given, the maximum of the next
    // tile's scores is scanned under the other kHalf.  Returns that maximum
    // (lane-local).
    auto mix = [&](int tile, const f32x16 (*sn)[2], const f32x16 (*sc)[2]) {
        const uint16_t* vl = lds_v[tile & 1] + v_rd;
        auto vread = [&](int st, i16x4 (&dst)[2]) {
            const int db = st % SV::kDBlocks, kk = st / SV::kDBlocks;  // kk = 2*kb + h2
            const uint16_t* a1 = vl + kk * 16 * SV::kStrideV + db * 32;
            dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TSDA_LDS i16x4*)(a1));
            dst[1] =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((TSDA_LDS i16x4*)(a1 + 8 * SV::kStrideV));
        };
        i16x4 vr[kAheadV + 1][2];
#pragma unroll
        for (int st = 0; st < kAheadV; ++st) vread(st, vr[st]);
        float mx = -INFINITY;
        const float mc = ref_log2();
        pin_schedule();
#pragma unroll
        for (int st = 0; st < kPV; ++st) {
            if (st + kAheadV < kPV) vread(st + kAheadV, vr[(st + kAheadV) % (kAheadV + 1)]);
            const i16x4 (&src)[2] = vr[st % (kAheadV + 1)];
            u32x4 a;
            a[0] = (uint32_t)(uint16_t)src[0][0] | ((uint32_t)(uint16_t)src[0][1] << 16);
            a[1] = (uint32_t)(uint16_t)src[0][2] | ((uint32_t)(uint16_t)src[0][3] << 16);
            a[2] = (uint32_t)(uint16_t)src[1][0] | ((uint32_t)(uint16_t)src[1][1] << 16);
            a[3] = (uint32_t)(uint16_t)src[1][2] | ((uint32_t)(uint16_t)src[1][3] << 16);
            const int db = st % SV::kDBlocks;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(a), as_bf16x8(pf[st / kHalf][(st % kHalf) / SV::kDBlocks]), oacc[db], 0, 0,
                0);
            if (sc && st < kHalf) {
#pragma unroll
                for (int e = kNA + (18 - kNA) * st / kHalf; e < kNA + (18 - kNA) * (st + 1) / kHalf; ++e)
                    pair_stage(*sc, e, mc);
            }
            if (sn && st >= kHalf) {
                constexpr int kPer = 32 / kHalf;
#pragma unroll
                for (int e = 0; e < kPer; ++e) {
                    const int x = (st - kHalf) * kPer + e;
                    mx = fmaxf(mx, (*sn)[x >> 4][x & 15]);
                }
            }
            pin_schedule();
        }
        return mx;
    };
    // Online-softmax reference update from a tile's maximum.  A row's
    // reference moves only when the tile maximum exceeds it by more than
    // kRescaleLog2 (log2 units); otherwise the tile is exponentiated against
    // the old reference, so P stays below 2^kRescaleLog2 and the result is
    // unchanged (weights and normaliser share one reference).  The decision
    // is per row -- a row that does not move multiplies by exactly 1 -- so
    // each row's arithmetic depends on its own keys only; the wave merely
    // skips the multiplies when no row moves.  Runs after every P V MFMA of
    // the tiles before.
    auto reference = [&](float mx) {
        mx = halves_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const bool grow = (m_new - m_run) * scale_log2 > kRescaleLog2;  // true if m_run = -inf
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float alpha = grow ? fast_exp2((m_run - m_new) * scale_log2) : 1.0f;
            m_run = grow ? m_new : m_run;
            ref_run = m_run == -INFINITY ? 0.0f : m_run * scale_log2;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < SV::kDBlocks; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
    };
    auto scan = [&](const f32x16 (&sn)[2]) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sn[kb][r]);
        return mx;
    };

    // One iteration: tile t's scores are in sc and its reference is set; on
    // entry LDS holds K(t+1) and V(t).  The next tiles' loads are issued
    // between the two compute blocks.
    // The staging loads and stores run unconditionally: past the block's
    // last tile they move rows that are in bounds (rows at or past L are
    // clamped) into LDS slots nobody reads again, and with no load under
    // a branch the compiler's wait counts stay exact (each stash waits only
    // for its own loads).
    // No allowed-mask word is read: the unmasked kernel and the masked
    // kernel's blocks whose listed tiles all open whole take this step.
    auto step = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {
        const bool pipe = t + 1 < t1w;  // this wave scores tile t+1
        bhere(t + 1);  // bias of tile t+1
        fetch_k(t + 2);
        // S^T(t+1) under which P(t) is formed
        if (pipe) score(t + 1, sn, &sc);
        fetch_v(t + 1);
        if (pipe) {
            mask(std::false_type{}, t + 1, sn);
            // P(t) V(t) under which the maximum of S^T(t+1) is found
            const float mx = mix(t, &sn, &sc);
            reference(mx);
        } else if (t < t1w) {
            weigh(sc);
            mix(t, nullptr, nullptr);
        }
        bload(t + 2);
        stash_k(t + 2);
        stash_v(t + 1);
        bwrite(t + 2);
        __syncthreads();
    };

    // The masked step: as `step`, but a wave skips the tiles its mask words
    // show fully hidden.  `have` says whether the wave holds the scores of
    // tile t (it skipped tile t otherwise); the four cases chain the score of
    // the next computed tile to the weights of the last one exactly as the
    // prologue, the pipelined step and the wave's last tile do.
    bool have = false;
    auto step_m = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) __attribute__((always_inline)) {  // t: list position
        mread(t + 1);  // mask words of position t+1
        bpark();
        const bool next = t + 1 < pp1 && tix(t + 1) < tw && !mnone;  // this wave computes t+1
        fetch_k(tix(t + 2));
        if (next) {
            if (have) score(t + 1, sn, &sc);
            else score(t + 1, sn, nullptr);
        }
        fetch_v(tix(t + 1));
        mload(tix(t + 2));
        if (next) mask(std::bool_constant<MASK>{}, tix(t + 1), sn);
        if (have && next) {
            const float mx = mix(t, &sn, &sc);
            reference(mx);
        } else if (have) {
            weigh(sc);
            mix(t, nullptr, nullptr);
        } else if (next) {
            reference(scan(sn));
        }
        have = next;
        bload(tix(t + 2));
        stash_k(t + 2);
        stash_v(t + 1);
        mwrite(t + 2);
        __syncthreads();
    };

    // The unmasked walk over key tiles ta <= t < tb.  Prologue: K(ta), V(ta),
    // K(ta+1) staged; S^T(ta) scored and its reference set.
    auto walk = [&](int ta, int tb) __attribute__((always_inline)) {
        load_q();
        bload(ta);
        fetch_k(ta);
        fetch_v(ta);
        u32x4 k1[S::kPerThread];
        fetch_k_to(ta + 1, k1);
        stage_q();
        stash_k(ta);
        stash_v(ta);
        stash_k_from(ta + 1, k1);
        bwrite(ta);
        __syncthreads();
        bhere(ta);
        if (ta < t1w) {
            score(ta, s0, nullptr);
            mask(std::false_type{}, ta, s0);
            reference(scan(s0));
        }
        bload(ta + 1);
        bwrite(ta + 1);
        __syncthreads();  // K(ta) is read by every wave before K(ta+2) replaces it
        for (int t = ta; t < tb; t += 2) {
            step(t, s0, s1);
            if (t + 1 < tb) step(t + 1, s1, s0);
        }
    };
    // The key-group walk (KG = 2, unmasked small grids): waves rg and
    // rg + BM/32 own the same 32 rows, and key group kg computes the tiles
    // ta + kg, ta + kg + 2, ... of them, each with its own online softmax,
    // merged at the end.  The staging moves tiles in pairs (ta + 2s,
    // ta + 2s + 1) into the two LDS slots, so group kg always reads slot kg
    // (ta is 0: these grids are unsplit).  Step s: group kg scores its next
    // tile u + 2 (K of pair s + 1) under the weights of its tile
    // u = ta + 2s + kg and mixes u (V of pair s); after a barrier the block
    // stores K of pair s + 2 and V of pair s + 1, then a second barrier.  Both
    // groups run the same ceil((tb - ta) / 2) steps.
    u32x4 kp0[S::kPerThread], kp1[S::kPerThread], vp0[SV::kPerThread], vp1[SV::kPerThread];
    auto step_kg = [&](int st, f32x16 (&sc)[2], f32x16 (&sn)[2], int ta) __attribute__((always_inline)) {
        const int u = ta + 2 * st + kg;
        const bool pipe = u + 2 < t1w;  // this wave scores its next tile
        // The next pairs' loads are issued after the scores, in each branch
        // (their registers do not fit beside the score phase's at d = d_v =
        // 128; placed once before the branch they spill).
        if (pipe) {
            score(u + 2, sn, &sc);
            fetch_k_to(ta + 2 * st + 4, kp0);
            fetch_k_to(ta + 2 * st + 5, kp1);
            fetch_v_to(ta + 2 * st + 2, vp0);
            fetch_v_to(ta + 2 * st + 3, vp1);
            mask(std::false_type{}, u + 2, sn);
            const float mx = mix(u, &sn, &sc);
            reference(mx);
        } else {
            fetch_k_to(ta + 2 * st + 4, kp0);
            fetch_k_to(ta + 2 * st + 5, kp1);
            fetch_v_to(ta + 2 * st + 2, vp0);
            fetch_v_to(ta + 2 * st + 3, vp1);
            if (u < t1w) {
                weigh(sc);
                mix(u, nullptr, nullptr);
            }
        }
        __syncthreads();  // K of pair s + 1 and V of pair s are read
        stash_k_from(ta + 2 * st + 4, kp0);
        stash_k_from(ta + 2 * st + 5, kp1);
        stash_v_from(ta + 2 * st + 2, vp0);
        stash_v_from(ta + 2 * st + 3, vp1);
        __syncthreads();
    };
    auto walk_kg = [&](int ta, int tb) __attribute__((always_inline)) {
        const int u0 = ta + kg;
        load_q();
        fetch_k_to(ta, kp0);
        fetch_k_to(ta + 1, kp1);
        fetch_v_to(ta, vp0);
        fetch_v_to(ta + 1, vp1);
        stage_q();
        stash_k_from(ta, kp0);
        stash_k_from(ta + 1, kp1);
        fetch_k_to(ta + 2, kp0);
        fetch_k_to(ta + 3, kp1);
        __syncthreads();
        if (u0 < t1w) {
            score(u0, s0, nullptr);
            mask(std::false_type{}, u0, s0);
            reference(scan(s0));
        }
        __syncthreads();  // K of pair 0 is read by every wave before pair 1 replaces it
        stash_k_from(ta + 2, kp0);
        stash_k_from(ta + 3, kp1);
        stash_v_from(ta, vp0);
        stash_v_from(ta + 1, vp1);
        __syncthreads();
        const int nsteps = (tb - ta + 1) >> 1;
        for (int st = 0; st < nsteps; st += 2) {
            step_kg(st, s0, s1, ta);
            if (st + 1 < nsteps) step_kg(st + 1, s1, s0, ta);
        }
    };
    // The masked walk over list positions pp0 <= t < pp1, with the same
    // prologue; the tile scored first is the first one the wave computes.
    auto walk_m = [&]() __attribute__((always_inline)) {
        load_q();
        mload(tix(pp0));
        bload(tix(pp0));
        fetch_k(tix(pp0));
        fetch_v(tix(pp0));
        stage_q();
        stash_k(pp0);
        stash_v(pp0);
        fetch_k(tix(pp0 + 1));
        stash_k(pp0 + 1);
        mwrite(pp0);
        __syncthreads();
        bpark();
        mread(pp0);
        have = pp0 < pp1 && tix(pp0) < tw && !mnone;
        if (have) {
            score(pp0, s0, nullptr);
            mask(std::bool_constant<MASK>{}, tix(pp0), s0);
            reference(scan(s0));
        }
        mload(tix(pp0 + 1));
        bload(tix(pp0 + 1));
        mwrite(pp0 + 1);
        __syncthreads();
        for (int t = pp0; t < pp1; t += 2) {
            step_m(t, s0, s1);
            if (t + 1 < pp1) step_m(t + 1, s1, s0);
        }
    };

    if constexpr (MASK) {
        if (dense) {
            // consecutive tiles, each opened whole: positions map to tiles
            // tl0 + pos and the mask changes no logit
            t1w = min(tl0 + pp1, tw);
            walk(tl0 + pp0, tl0 + pp1);
        } else {
            walk_m();
        }
    } else if constexpr (KG == 2) {
        walk_kg(t0, t1);
        // merge the two key groups' softmax states of each row, in group 0
        constexpr int kO = SV::kDBlocks * 16;
        float* xs = lds_x + (size_t)rg * (kO + 2) * 64;
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < kO; ++i) xs[i * 64 + lane] = oacc[i >> 4][i & 15];
            xs[kO * 64 + lane] = m_run;
            xs[(kO + 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (kg == 0) {
            const float m1 = xs[kO * 64 + lane], l1 = xs[(kO + 1) * 64 + lane];
            const float mn = fmaxf(m_run, m1);
            const float a0 = m_run == -INFINITY ? 0.0f : fast_exp2((m_run - mn) * scale_log2);
            const float a1 = m1 == -INFINITY ? 0.0f : fast_exp2((m1 - mn) * scale_log2);
#pragma unroll
            for (int i = 0; i < kO; ++i)
                oacc[i >> 4][i & 15] = a0 * oacc[i >> 4][i & 15] + a1 * xs[i * 64 + lane];
            l_run = a0 * l_run + a1 * l1;
            m_run = mn;
        }
    } else {
        walk(t0, t1);
    }

    if (KG == 1 && nsplit > 1) {  // (key groups run unsplit grids only)
        // ---- split epilogue: this split's (m, l, acc) of every live row, the
        // reference in exp2 units (-inf with l = 0 when the split saw none of
        // the row's keys); the combine kernel merges the splits.
        if (q_live) {
            const size_t unit = ((size_t)bh * Sq + qi) * nsplit + split;
            const float l_tot = halves_sum(l_run);
            float* arow = ws_acc + unit * DV;
#pragma unroll
            for (int db = 0; db < SV::kDBlocks; ++db)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int d0 = db * 32 + 8 * rg + 4 * half;
                    const f32x4 w4 = {oacc[db][4 * rg], oacc[db][4 * rg + 1], oacc[db][4 * rg + 2],
                                      oacc[db][4 * rg + 3]};
                    *reinterpret_cast<f32x4*>(arow + d0) = w4;
                }
            if (half == 0) {
                ws_ml[unit * 2] = m_run == -INFINITY ? -INFINITY : m_run * scale_log2;
                ws_ml[unit * 2 + 1] = l_tot;
            }
        }
        return;
    }

    // ---- epilogue: out = acc / l; with a mask this tile's rows past n_b are
    // zero too (without one the pad rows were zeroed above).
    // A lane holds 4-feature pieces of one row, so storing them directly
    // writes 8 bytes into each of 32 rows per instruction.  Instead each wave
    // packs its 32 x DV outputs into its own LDS region (the K/V slots are
    // free after the walk's last barrier) and stores whole rows from there:
    // 16 bytes a lane, consecutive lanes on consecutive bytes.
    constexpr int kOutStride = DV + 8;                          // row stride (elements)
    constexpr int kOutRegion = 32 * kOutStride;                 // one wave's rows
    constexpr int kRegionsK = 2 * S::kTileK / kOutRegion;       // regions in lds_k
    constexpr int kRegionsV = 2 * SV::kTileV / kOutRegion;      // regions in lds_v
    constexpr bool kStaged = kRegionsK + kRegionsV >= kRowWaves;
    if constexpr (kStaged) {
        uint16_t* region = rg < kRegionsK ? &lds_k[0][0] + rg * kOutRegion
                                          : &lds_v[0][0] + (rg - kRegionsK) * kOutRegion;
        if (kg == 0) {
            const float l_tot = halves_sum(l_run);
            const float inv = (q_live && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
            uint16_t* lrow = region + (lane & 31) * kOutStride;
#pragma unroll
            for (int db = 0; db < SV::kDBlocks; ++db)
#pragma unroll
                for (int rg4 = 0; rg4 < 4; ++rg4) {
                    const int d0 = db * 32 + 8 * rg4 + 4 * half;
                    u32x2 w = {0, 0};
                    if (q_live) {
                        w[0] = pack_bf16(oacc[db][4 * rg4] * inv, oacc[db][4 * rg4 + 1] * inv);
                        w[1] = pack_bf16(oacc[db][4 * rg4 + 2] * inv, oacc[db][4 * rg4 + 3] * inv);
                    }
                    *reinterpret_cast<u32x2*>(lrow + d0) = w;
                }
        }
        __syncthreads();
        if (kg == 0) {
            constexpr int kRowChunks = DV / 8;  // 16-byte chunks per row
            constexpr int kPer = 32 * kRowChunks / 64;
            // every read first, then the stores (each behind its row's test)
            u32x4 val[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = i * 64 + lane;
                val[i] = *reinterpret_cast<const u32x4*>(region + (c / kRowChunks) * kOutStride +
                                                         (c % kRowChunks) * 8);
            }
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = i * 64 + lane;
                const int qr = qw + c / kRowChunks;
                if (MASK ? qr < Sq : (qr >= 0 && qr < n))
                    *reinterpret_cast<u32x4*>(obase + (size_t)qr * DV + (c % kRowChunks) * 8) = val[i];
            }
        }
        return;
    }
    if ((MASK ? qi < Sq : q_live) && kg == 0) {
        const float l_tot = halves_sum(l_run);
        const float inv = (q_live && l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = obase + (size_t)qi * DV;
#pragma unroll
        for (int db = 0; db < SV::kDBlocks; ++db)
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

// Tile marks of an allowed-mask shared by all heads: one workgroup per
// (mask batch, query tile, key tile) writes 0 if no row of the query tile
// may see a key of the key tile, 2 if every row may see every key of it,
// else 1.  Only the bytes that can matter count: keys below Skv, and with
// the causal rule keys at or before the row's position (row i sits at
// position <= Skv - Sq + i in every batch item, a bound the rules reach
// when the item's length is Skv), so a causal mask given with the causal
// rule still opens its tiles whole.  Each wave reads 64 rows; lane l reads
// 4-byte word l mod 16 of every 4th row from l / 16, so each load
// instruction covers 4 whole 64-byte row segments.  Key tiles past the last
// key a causal row of the tile can reach are marked 0 unread (the prefill
// never visits them).
// VEC: whole 64-key tiles (Skv a multiple of 64) and 16-byte aligned rows;
// then each lane reads 16 keys of a row with one load (4 lanes per row of
// the tile, 16 rows per wave-wide load) instead of one 4-key word, and a
// workgroup marks four consecutive key tiles, its loads of all four issued
// before any is tested.
template <int BM, bool VEC>  // BM: query rows per query tile (the prefill's block)
__global__ __launch_bounds__(BM) void prefill_mask_tiles_kernel(
    const uint8_t* __restrict__ mask, long long msb, long long msi, int Sq, int Skv, int nqt,
    int nkt, int causal, uint8_t* __restrict__ tmap) {
    // VEC: a workgroup marks kKT consecutive key tiles, its loads of all of
    // them in flight together
    constexpr int kKT = VEC ? 4 : 1;
    const int nkg = (nkt + kKT - 1) / kKT;
    const int kt0 = (blockIdx.x % nkg) * kKT;
    const int qt = (blockIdx.x / nkg) % nqt;
    const int bm = blockIdx.x / (nkg * nqt);
    const int q0 = qt * BM;
    uint8_t* marks = tmap + ((size_t)bm * nqt + qt) * nkt;
    __shared__ int flags[kKT][2 * (BM / 64)];
    // keys any row of the query tile may reach: tiles from hi on are marked 0
    // unread (the prefill never visits them)
    const int hi = causal ? Skv - Sq + min(q0 + BM, Sq) : Skv;
    if (kt0 * kBN >= hi) {  // every tile of the workgroup: nothing to read
        if ((int)threadIdx.x < kKT && kt0 + (int)threadIdx.x < nkt) marks[kt0 + threadIdx.x] = 0;
        return;
    }
    const int lane = threadIdx.x & 63;
    uint32_t any[kKT], hole[kKT];  // OR of the counted bytes; nonzero if one is zero
    if constexpr (VEC) {
        const int r0 = q0 + (int)(threadIdx.x >> 6) * 64 + (lane >> 2);
        // a tile that is not marked from its bytes reads the last one that is
        // (or tile 0), which is in bounds
        const int kmax = max(0, min(nkt - 1, (hi - 1) / kBN));
        // all loads first (rows past Sq read row Sq - 1 and count nothing),
        // so they are in flight together
        u32x4 w4[kKT][4];
#pragma unroll
        for (int j = 0; j < kKT; ++j) {
            const int c = min(kt0 + j, kmax) * kBN + 16 * (lane & 3);
#pragma unroll
            for (int it = 0; it < 4; ++it)
                w4[j][it] = ldg16(mask + bm * msb + c + (long long)min(r0 + 16 * it, Sq - 1) * msi);
        }
#pragma unroll
        for (int j = 0; j < kKT; ++j) {
            const int c = (kt0 + j) * kBN + 16 * (lane & 3);  // first key of this lane's 16
            any[j] = hole[j] = 0;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int row = r0 + 16 * it;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // keys c + 4 g .. + 3, below Skv; the causal rule may cut them
                    int nb = row < Sq ? 4 : 0;
                    if (causal) nb = min(nb, Skv - Sq + row - (c + 4 * g) + 1);
                    const uint32_t ign = nb >= 4 ? 0u : nb <= 0 ? ~0u : ~0u << (8 * nb);
                    any[j] |= w4[j][it][g] & ~ign;
                    hole[j] |= has_zero_byte(w4[j][it][g] | ign);
                }
            }
        }
    } else {
        const int r0 = q0 + (int)(threadIdx.x >> 6) * 64 + (lane >> 4);
        const int c = kt0 * kBN + 4 * (lane & 15);  // first key of this lane's word
        const int col = min(c, mask_last_word(Skv));
        const uint8_t* mtile = mask + bm * msb + col;
        uint32_t wd[16];
#pragma unroll
        for (int it = 0; it < 16; ++it)
            wd[it] = ldg_word(mtile + (long long)min(r0 + 4 * it, Sq - 1) * msi);
        any[0] = hole[0] = 0;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = r0 + 4 * it;
            // bytes counted: keys c .. c + nb - 1 (none for a clamped word or row)
            int nb = c == col && row < Sq ? Skv - c : 0;
            if (causal) nb = min(nb, Skv - Sq + row - c + 1);
            const uint32_t ign = nb >= 4 ? 0u : nb <= 0 ? ~0u : ~0u << (8 * nb);
            any[0] |= wd[it] & ~ign;
            hole[0] |= has_zero_byte(wd[it] | ign);
        }
    }
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
        const bool wa = __builtin_amdgcn_ballot_w64(any[j] != 0) != 0;
        const bool wh = __builtin_amdgcn_ballot_w64(hole[j] != 0) != 0;
        if ((threadIdx.x & 63) == 0) {
            flags[j][threadIdx.x >> 6] = wa;
            flags[j][BM / 64 + (threadIdx.x >> 6)] = wh;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < kKT && kt0 + (int)threadIdx.x < nkt) {
        const int j = threadIdx.x, kt = kt0 + j;
        int fa = 0, fh = 0;
        for (int w = 0; w < BM / 64; ++w) {
            fa |= flags[j][w];
            fh |= flags[j][BM / 64 + w];
        }
        marks[kt] = kt * kBN >= hi ? 0 : fa ? (fh ? 1 : 2) : 0;
    }
}

// Merge of the key-range splits of each query row (log-sum-exp rule, as at
// decode): M = max_s m_s, l = sum_s l_s 2^(m_s - M),
// out = (sum_s acc_s 2^(m_s - M)) / l; padded rows are written as zeros.
// Each thread merges 4 consecutive columns of one row with 16-byte loads;
// a block covers 256 / (D/4) rows.  A thread issues the loads of all its
// splits before any arithmetic (one memory round trip); NS >= nsplit bounds
// the register arrays that hold them.
constexpr int kMaxSplit = 16;

template <int D, int NS>
__global__ __launch_bounds__(256) void prefill_combine_kernel(
    const int32_t* __restrict__ kv_lens, int H, int Sq, int Skv, int nsplit, size_t nrows,
    const float* __restrict__ ws_acc, const float* __restrict__ ws_ml, uint16_t* __restrict__ out) {
    constexpr int TPR = D / 4;  // threads per row
    constexpr int ROWS = 256 / TPR;
    const int tid = threadIdx.x;
    const int c = (tid % TPR) * 4;
    const size_t row = (size_t)blockIdx.x * ROWS + tid / TPR;  // (b*H + h)*Sq + i
    if (row >= nrows) return;
    const int bh = (int)(row / Sq);
    const int i = (int)(row - (size_t)bh * Sq);
    const int L = valid_length(kv_lens, bh / H, Skv);
    const int n = Sq < L ? Sq : L;
    u32x2 res = {0, 0};
    if (i < n) {
        // every split's (m, l) and accumulator columns are loaded up front:
        // one memory round trip per row
        const float* ml = ws_ml + row * nsplit * 2;
        const float* ac = ws_acc + row * nsplit * D + c;
        float mv[NS], lv[NS];
        f32x4 av[NS];
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            const bool ok = sp < nsplit;
            mv[sp] = ok ? ml[2 * sp] : -INFINITY;
            lv[sp] = ok ? ml[2 * sp + 1] : 0.0f;
            av[sp] = ok ? *reinterpret_cast<const f32x4*>(ac + (size_t)sp * D)
                        : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float M = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) M = fmaxf(M, mv[sp]);
        float lt = 0.0f;
        f32x4 at = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            const float w = mv[sp] == -INFINITY ? 0.0f : fast_exp2(mv[sp] - M);
            lt = fmaf(lv[sp], w, lt);
#pragma unroll
            for (int e = 0; e < 4; ++e) at[e] = fmaf(av[sp][e], w, at[e]);
        }
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        res[0] = pack_bf16(at[0] * inv, at[1] * inv);
        res[1] = pack_bf16(at[2] * inv, at[3] * inv);
    }
    *reinterpret_cast<u32x2*>(out + row * D + c) = res;
}

}  // namespace

PrefillPlan prefill_plan(int B, int H, int Sq, int Skv, int d, int dv, bool masked, bool general) {
    // Each query tile is one block.  When that leaves CUs idle (short query
    // chunks against a long cache), the key range of every query tile is
    // split over about one block per CU in all, each split at least 16 key
    // tiles, and the splits are merged by a second kernel.  Measured on
    // 1-4 x 32 heads: 512 queries against 4096 keys 117 -> 64 us (4 splits),
    // 256 against 8192 214 -> 66 us (8 splits); grids of 256 blocks or more
    // are faster unsplit, the merge costing more than the idle CUs.
    //
    // Unsplit grids of at most 128 blocks (half the CUs or fewer) use blocks
    // of 128 query rows instead: twice the blocks, each with four waves, so
    // the heaviest block's walk over the keys takes less time per step.
    // Measured (B=1, H=32, d=128, causal): S = 512 23.1 -> 20.5 us, S = 1024
    // 36.8 -> 33.6 us; B=4, H=12, S=512, d=64: 17.0 -> 16.1 us.  Grids of at
    // most 64 such blocks use blocks of 64 rows (two waves), still one block
    // per CU at most: S = 128, 256, 512 at H = 32 11.3 -> 10.2, 14.1 -> 13.0,
    // 20.0 -> 19.1 us against 128-row blocks.  Large grids lose with smaller
    // blocks (prefill4096 150 -> 234 us with 128 rows: one wave per SIMD).
    const long blocks = (long)((Sq + kBM - 1) / kBM) * B * H;
    const long tiles = (Skv + kBN - 1) / kBN;
    long nsplit = 256 / blocks;
    nsplit = std::max(1L, std::min({nsplit, tiles / 16, (long)kMaxSplit}));
    // Plain unmasked grids of up to 256 such blocks with at least 8 key
    // tiles take 128-row blocks with key groups (below) too: B=1, H=32,
    // S=2048 64.6 -> 57.4 us; B=1, H=16, S=4096 116.7 -> 92.6 us (two rounds
    // of blocks, each block's walk halved).  Larger grids lose with them
    // (prefill4096 145 -> 176 us: the pair steps cost more per tile).
    const bool plain = !masked && !general;
    int bm = kBM;
    if (nsplit == 1) {
        if (4 * blocks <= 256)
            bm = 64;
        else if (blocks <= 128 || (plain && blocks <= 256 && tiles >= 8))
            bm = 128;
    }
    // Small unmasked grids with plain logits and at least 8 key tiles split
    // each block's keys between two wave sets (the kernel's key-group walk),
    // halving the longest walk: B=4, H=12, S=512, d=64 15.6 -> 13.7 us;
    // B=1, H=8, S=1024, d=64 22.0 -> 17.0 us; B=1, H=32, S=512, d=128
    // 19.0 -> 17.6 us; B=1, H=32, S=1024, d=128 31.3 -> 27.6 us.  Shorter
    // walks lose (S = 128, 256: +10 %, +1.5 %).
    (void)d;
    (void)dv;
    const int kg = bm < kBM && plain && tiles >= 8 ? 2 : 1;
    return PrefillPlan{(int)nsplit, bm, kg};
}

size_t prefill_workspace_bytes(int B, int H, int Sq, int Skv, int d) {
    const PrefillPlan p = prefill_plan(B, H, Sq, Skv);
    if (p.nsplit == 1) return 0;
    const size_t units = (size_t)B * H * Sq * p.nsplit;
    return round_up256(units * d * sizeof(float)) + round_up256(units * 2 * sizeof(float));
}

size_t prefill_mask_workspace_bytes(int B, int Sq, int Skv) {
    // tile marks of a mask shared by all heads, one byte per (mask batch,
    // query tile, key tile), after the split partials; none past the list
    // size.  Sized for query tiles of 64 rows, the smallest block height.
    const size_t nkt = (Skv + kBN - 1) / kBN;
    if (nkt > (size_t)kMaxListTiles) return 0;
    return round_up256((size_t)B * ((Sq + 63) / 64) * nkt);
}

hipError_t launch_prefill_bf16(const LaunchArgs& a) {
    const PrefillPlan p = prefill_plan(a.B, a.H, a.Sq, a.Skv, a.d, a.dv, a.mask != nullptr,
                                       a.bias != nullptr || !(a.scale > 0.0f));
    const int nqt = (a.Sq + p.bm - 1) / p.bm;
    const int BH = a.B * a.H;
    const dim3 grid((unsigned)((long)nqt * BH * p.nsplit));
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* o = static_cast<uint16_t*>(a.out);
    float* ws_acc = nullptr;
    float* ws_ml = nullptr;
    const size_t ws_split = prefill_workspace_bytes(a.B, a.H, a.Sq, a.Skv, a.dv);
    // a mask shared by all heads gets key-tile lists (marks after the partials)
    const int nkt = (a.Skv + kBN - 1) / kBN;
    const size_t ws_marks = a.mask && a.msh == 0 ? prefill_mask_workspace_bytes(a.B, a.Sq, a.Skv) : 0;
    if (ws_split + ws_marks > 0 &&
        (a.workspace == nullptr || a.workspace_bytes < ws_split + ws_marks))
        return hipErrorInvalidValue;  // the front end sizes it; never write through a bad one
    uint8_t* tmap = ws_marks ? static_cast<uint8_t*>(a.workspace) + ws_split : nullptr;
    if (p.nsplit > 1) {
        const size_t units = (size_t)BH * a.Sq * p.nsplit;
        ws_acc = static_cast<float*>(a.workspace);
        ws_ml = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                         round_up256(units * a.dv * sizeof(float)));
    }
    // the general instantiation for a bias or a scale that is not positive:
    // it forms scale * s + bias and works in exp2 units of those logits
    const bool gen = a.bias != nullptr || !(a.scale > 0.0f);
    const float sl = gen ? kLog2e : a.scale * kLog2e;
    KernelTimer* t = active_timer();
    if (tmap && !(a.msi == 0 && nkt <= 64)) {  // short one-row masks are marked in the prefill
        const int Bm = a.msb != 0 ? a.B : 1;
        if (t) t->begin(kPrefillMaskTiles, a.stream);
        const bool vec = a.Skv % kBN == 0 && (reinterpret_cast<uintptr_t>(a.mask) & 15u) == 0 &&
                         (a.msb & 15) == 0 && (a.msi & 15) == 0;
        // VEC: four key tiles per workgroup
        const dim3 mgrid((unsigned)((long)Bm * nqt * (vec ? (nkt + 3) / 4 : nkt)));
        auto marks = [&](auto kern, int threads) {
            hipLaunchKernelGGL(kern, mgrid, dim3(threads), 0, a.stream, a.mask, a.msb, a.msi,
                               a.Sq, a.Skv, nqt, nkt, a.causal, tmap);
        };
        if (p.bm == 64)
            vec ? marks(prefill_mask_tiles_kernel<64, true>, 64)
                : marks(prefill_mask_tiles_kernel<64, false>, 64);
        else if (p.bm == 128)
            vec ? marks(prefill_mask_tiles_kernel<128, true>, 128)
                : marks(prefill_mask_tiles_kernel<128, false>, 128);
        else
            vec ? marks(prefill_mask_tiles_kernel<kBM, true>, kBM)
                : marks(prefill_mask_tiles_kernel<kBM, false>, kBM);
        hipError_t e = hipGetLastError();
        if (t) t->end(kPrefillMaskTiles, a.stream);
        if (e != hipSuccess) return e;
    }
    if (t) t->begin(kPrefillBf16, a.stream);
    const int kg = p.kg;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(2 * p.bm * kg), 0, a.stream, q, k, v, o, a.kv_lens, BH, a.H,
                           a.Hkv, a.Sq, a.Skv, sl, a.causal, nqt, p.nsplit, ws_acc, ws_ml, a.mask,
                           a.msb, a.msh, a.msi, tmap, nkt, static_cast<const uint16_t*>(a.bias),
                           a.bsb, a.bsh, a.bsi, a.scale);
    };
    const bool m = a.mask != nullptr;
    // instantiations for d, d_v in {64, 128}, the mask, the general logits
    // and the block height
    auto pick_bm = [&](auto dk, auto dvk, auto bmk) {
        constexpr int D = decltype(dk)::value, DV = decltype(dvk)::value;
        constexpr int BM = decltype(bmk)::value;
        if (gen)
            m ? go(prefill_bf16_kernel<D, DV, true, true, BM, 1>)
              : go(prefill_bf16_kernel<D, DV, false, true, BM, 1>);
        else if (m)
            go(prefill_bf16_kernel<D, DV, true, false, BM, 1>);
        else if constexpr (BM < kBM)
            kg == 2 ? go(prefill_bf16_kernel<D, DV, false, false, BM, 2>)
                    : go(prefill_bf16_kernel<D, DV, false, false, BM, 1>);
        else
            go(prefill_bf16_kernel<D, DV, false, false, BM, 1>);
    };
    auto pick = [&](auto dk, auto dvk) {
        if (p.bm == 64)
            pick_bm(dk, dvk, std::integral_constant<int, 64>{});
        else if (p.bm == 128)
            pick_bm(dk, dvk, std::integral_constant<int, 128>{});
        else
            pick_bm(dk, dvk, std::integral_constant<int, kBM>{});
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    if (a.d == 128)
        a.dv == 128 ? pick(I128{}, I128{}) : pick(I128{}, I64{});
    else
        a.dv == 128 ? pick(I64{}, I128{}) : pick(I64{}, I64{});
    hipError_t e = hipGetLastError();
    if (t) t->end(kPrefillBf16, a.stream);
    if (e != hipSuccess || p.nsplit == 1) return e;
    if (t) t->begin(kPrefillCombineBf16, a.stream);
    const size_t rows = (size_t)BH * a.Sq;
    // a bound of 4 splits where it suffices: its register arrays keep twice
    // the waves resident of the 16-split form
    auto merge = [&](auto kern, int rows_per_block) {
        hipLaunchKernelGGL(kern, dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                           dim3(256), 0, a.stream, a.kv_lens, a.H, a.Sq, a.Skv, p.nsplit, rows, ws_acc,
                           ws_ml, o);
    };
    if (a.dv == 128)
        p.nsplit <= 4 ? merge(prefill_combine_kernel<128, 4>, 8)
                      : merge(prefill_combine_kernel<128, kMaxSplit>, 8);
    else
        p.nsplit <= 4 ? merge(prefill_combine_kernel<64, 4>, 16)
                      : merge(prefill_combine_kernel<64, kMaxSplit>, 16);
    e = hipGetLastError();
    if (t) t->end(kPrefillCombineBf16, a.stream);
    return e;
}

}  // namespace tsda
