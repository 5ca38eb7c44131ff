// Remap + sparse attention over the resident rows (split over rows).
//
// [LSO] section 4 "Decode step": the logical top-k positions are remapped
// to physical hot-buffer slots and sparse attention consumes the resident
// K/V (the Copy-SFA operator of the Chinese revision, section 4, fused
// Copy-SFA sub-section).  For every (seq, position, head):
//     z_j = scale * (q . K_j)  over the 576 columns of row j,
//     out = sum_j softmax(z)_j * V_j  over the first 512 (latent) columns,
// j running over the min(k, L_t) winners of that position.
//
// Every slot lives in a physical hot row (slot_row), and the misses of a
// step arrive in spare rows that their victim slots then take over, so the
// rows of a step never move.  Which row a winner reads comes either from the
// list the LRU-update launch wrote (wrow: the default, with the copy done
// early by that launch or late by its own kernel) or from the tables
// (slot_row[cache_slots[token]]).  With one query position and one group of
// 16 heads every winner row is read by exactly one block, which can also
// read a missed row straight from the pinned host pool (device-mapped) and
// write it into its row (the Copy-SFA fusion of the Chinese revision), so
// the host-link transfer of one block overlaps the attention of the others
// and no separate copy kernel runs.  A split launch pair attends the rows
// resident at step start and the missed rows separately (AttnPhase below),
// each writing its own partials.
//
// Layout of the work: a block takes one (seq, position), one group of 16
// heads and a chunk of winners.  Rows are staged 32 at a time in LDS (one
// coalesced 1152-byte read each, gathered by slot); the next tile is fetched
// into registers while the current one is computed.  The four waves split
// the 576-deep contraction S^T = K Q^T (v_mfma_f32_16x16x32_bf16, M = 16
// rows, N = 16 heads) and add their partial tiles through LDS; each wave
// then runs the online softmax and accumulates O^T = V^T P^T for its own
// 128 of the 512 output columns (M = 16 columns, N = 16 heads, K = 32
// rows).  P enters the MFMA in bf16; accumulation is fp32.  Each block
// writes (m, l, acc) partials; k_attn_combine merges them.
#include "sko_common.h"
#include "sko_internal.h"

namespace sko {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRowStrideU4 = kKvRowU4 + 1;  // 16-byte pad per staged row

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// v if keep, else zero: a bit mask rather than a select, so that a load
// feeding it is issued unconditionally (a select of a load becomes a branch
// around the load, and a wait for it inside the branch)
__device__ __forceinline__ uint4 keep_if(uint4 v, bool keep) {
    const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// dword holding bf16 element m (0..7) of a 16-byte vector
__device__ __forceinline__ uint32_t dword_of(uint4 v, int m) {
    return (m >> 1) == 0 ? v.x : (m >> 1) == 1 ? v.y : (m >> 1) == 2 ? v.z : v.w;
}

// ---- per-tile compute, shared by both attention kernels ---------------------
// Four compute waves, lanes (n16, g): n16 = head within the group, g = lane
// / 16.  The 18 k-steps (32 columns each) of S^T = K Q^T for a 32-row tile
// are split over the waves (5, 5, 4, 4); wave w holds the B operand Q^T of
// its k-steps in qv (lane (n16, g): Q[h][32ks + 8g .. +7]).

// This wave's partial S^T tiles of the tile in `rows` (LDS, padded rows)
// for rows 0..15 and 16..31, written to sp[wave].
__device__ __forceinline__ void tile_scores(const uint4* rows, const uint4 (&qv)[5], int ks0, int nks, int n16,
                                            int g, int lane, int wave, f32x4_t (*sp)[2][64]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
        const uint4* rp = rows + (half * 16 + n16) * kRowStrideU4 + g;
#pragma unroll
        for (int q = 0; q < 5; ++q)
            if (q < nks)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rp[4 * (ks0 + q)]), as_bf16x8(qv[q]), c, 0, 0,
                                                            0);
        sp[wave][half][lane] = c;
    }
}

// Once every wave's partial tiles are in sp: the scores of the tile's rows
// r .. r+31 (the four partials added in wave order; rows at or past n
// masked), the online-softmax update of (m_run, l_run) per head (exp2 of
// scaled scores), and O^T += V^T P^T for this wave's 128 output columns
// (P in bf16, fp32 accumulation).
__device__ __forceinline__ void tile_softmax_pv(const uint4* rows, const f32x4_t (*sp)[2][64], int r, int n,
                                                float scale_log2, int n16, int g, int lane, int wave, float& m_run,
                                                float& l_run, f32x4_t (&acc)[8]) {
    float s[2][4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const f32x4_t c = ((sp[0][half][lane] + sp[1][half][lane]) + sp[2][half][lane]) + sp[3][half][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = r + half * 16 + 4 * g + i;
            s[half][i] = (j < n) ? c[i] * scale_log2 : -INFINITY;
        }
    }
    // online softmax per head over the 32 rows (lane groups g share a head)
    float mt = s[0][0];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[half][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    // v_exp_f32 directly: arguments are <= 0 (or -inf: 0), results that
    // would be binary32 subnormals flush to zero
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[2][4];
    float ls = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[half][i] = __builtin_amdgcn_exp2f(s[half][i] - m_new);
            ls += p[half][i];
        }
    l_run = l_run * alpha + ls;
    m_run = m_new;
    // once the running maxima settle, most tiles leave every head's maximum
    // unchanged (alpha exactly 1): the rescale is skipped for the wave
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[m] *= alpha;
    }

    // B operand of O^T = V^T P^T: k-slot s of group g is row 4g+s (s<4)
    // or 16+4g+s-4 (s>=4), i.e. exactly the rows this lane's p covers;
    // P rounded to bf16 (nearest even) two at a time
    uint4 pb;
    pb.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p[0][0], p[0][1]}, bf16x2_t));
    pb.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p[0][2], p[0][3]}, bf16x2_t));
    pb.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p[1][0], p[1][1]}, bf16x2_t));
    pb.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){p[1][2], p[1][3]}, bf16x2_t));

    // A operand: V^T.  Lane reads 8 columns (cb + 8*n16 .. +7) of each of
    // its 8 rows; column cb + 8*n16 + m feeds MFMA m.
    uint4 vr[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
        const int R = (sl < 4) ? (4 * g + sl) : (16 + 4 * g + sl - 4);
        vr[sl] = rows[R * kRowStrideU4 + wave * 16 + n16];
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        // element m of each row: the low half of dword m/2 for even m, the
        // high half for odd m; two rows' elements per dword (v_perm_b32
        // byte select: 0..3 = bytes of the second operand, 4..7 = first)
        const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
        uint32_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = __builtin_amdgcn_perm(dword_of(vr[2 * q + 1], m), dword_of(vr[2 * q], m), sel);
        const uint4 a = make_uint4(d[0], d[1], d[2], d[3]);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(pb), acc[m], 0, 0, 0);
    }
}

// This wave's (m, l, acc) partials: acc of 16 heads x its 128 columns, and
// (m, l) per head from wave 0.
__device__ __forceinline__ void write_partials(float* acc_out, float* ml_out, const f32x4_t (&acc)[8], float m_run,
                                               float l_run, int h, int H, int n16, int g, int wave) {
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
    const int cb = wave * 128;
    if (h < H) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_out[n16 * kVDim + cb + 8 * (4 * g + i) + m] = acc[m][i];
    }
    if (wave == 0 && g == 0) {
        ml_out[2 * n16] = m_run;
        ml_out[2 * n16 + 1] = lt;
    }
}

// How the launch gets the rows that missed into their slots.
// Where a launch finds each winner's row: the tables, the tables plus the
// fused copy of the misses, or the LRU-update launch's row list.
enum AttnRows { kRowsTables = 0, kRowsFusedCopy = 1, kRowsGiven = 2 };

// Which rows of a chunk a launch attends: all of them, only those resident
// at step start (hits), or only those that missed.  A split runs the hits
// while the copy launch brings the misses in, and the misses after it; each
// phase writes its own partials, the combine merges both.
enum AttnPhase { kPhaseAll = 0, kPhaseHits = 1, kPhaseMisses = 2 };

template <int ROWS, int PHASE>
__global__ __launch_bounds__(256) void k_attn_partial(
    const int32_t* __restrict__ topk, const int32_t* __restrict__ cache_slots_layer,
    const int32_t* __restrict__ slot_row_layer, uint4* __restrict__ hot_layer, const uint4* __restrict__ q_attn,
    const uint4* __restrict__ pool_layer, const uint4* __restrict__ recent_layer,
    const int32_t* __restrict__ ntok_layer, float* __restrict__ part_acc, float* __restrict__ part_ml,
    int32_t* __restrict__ phys, const int32_t* __restrict__ wrow, uint32_t* __restrict__ miss_bits, int64_t wpr,
    int D, int H, int HG, int top_k, int S, int R, int64_t cap, int rows_per_block, int nchunk, int pchunks,
    float scale_log2, int nbp, int xc) {
    __shared__ uint4 rows[kAttnTileRows * kRowStrideU4];
    __shared__ int32_t slot_s[kAttnMaxRowsPerBlock];  // row read, relative to the sequence's hot rows
    __shared__ int32_t cp_s[kAttnMaxRowsPerBlock];    // fused copy: pool token of a missed row, else -1
    __shared__ f32x4_t sp[4][2][64];  // per-wave partial S^T tiles
    __shared__ int scratch[256 / 64 + 1];

    // work block (chunk, bp, hg), chunk fastest
    const int wk = split_block(blockIdx.x, xc);
    if (wk < 0 || wk >= nchunk * nbp * HG) return;  // block-uniform
    const int chunk = wk % nchunk, bp = (wk / nchunk) % nbp, hg = wk / (nchunk * nbp);
    const int b = bp / D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const int h = hg * kAttnHeadGroup + n16;
    constexpr bool fused_copy = ROWS == kRowsFusedCopy;
    constexpr bool given = ROWS == kRowsGiven;
    const int r0 = chunk * rows_per_block;
    // list entries this chunk can hold (known without the token count)
    const int rcap = std::min(r0 + rows_per_block, top_k);
    const int32_t* __restrict__ w = topk + (size_t)bp * top_k;

    // The loads that depend on nothing else are issued together, before any
    // of them is waited for: the token count, the chunk's list entries (and
    // rows) and the query operand.
    const int64_t Lt = ntok_layer[b];
    constexpr int kRowsPerThread = kAttnMaxRowsPerBlock / 256;
    int32_t pk[kRowsPerThread], pr[kRowsPerThread];
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        // all rows: thread t takes entries t, t + 256; a split phase keeps
        // the rows in order, so a thread takes two consecutive entries
        const int j = PHASE == kPhaseAll ? tid + 256 * u : tid * kRowsPerThread + u;
        // read in bounds (clamped) and used only below the chunk's row count
        const int jc = std::min(r0 + j, top_k - 1);
        pk[u] = w[jc];
        pr[u] = -1;
        if constexpr (given) pr[u] = wrow[(size_t)bp * top_k + jc];
    }
    // The 18 k-steps (32 columns each) of S^T = K Q^T are split over the 4
    // waves (5, 5, 4, 4); wave w holds the B operand Q^T of its k-steps:
    // lane (n16, g) holds Q[h][32ks + 8g .. +7].
    const int ks0 = wave < 2 ? 5 * wave : 10 + 4 * (wave - 2);
    const int nks = wave < 2 ? 5 : 4;
    uint4 qv[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) {
        // loads stay in bounds (clamped head and step); the select zeroes
        // padding heads and the fifth step of waves that own four
        const int hq = h < H ? h : H - 1;
        const int kq = q < nks ? ks0 + q : ks0;
        qv[q] = keep_if(q_attn[((size_t)bp * H + hq) * kKvRowU4 + 4 * kq + g], h < H && q < nks);
    }

    const int kk = (int)std::min<int64_t>(top_k, Lt);
    const int r1 = std::min(rcap, kk);
    // partials of the chunk: pchunks per (seq, position, head group), the
    // misses phase after the hits phase's nchunk
    const size_t pidx = ((size_t)bp * HG + hg) * pchunks + (PHASE == kPhaseMisses ? nchunk : 0) + chunk;
    float* __restrict__ acc_out = part_acc + pidx * kAttnHeadGroup * kVDim;
    float* __restrict__ ml_out = part_ml + pidx * kAttnHeadGroup * 2;
    if (r0 >= r1) {
        if (tid < kAttnHeadGroup) {
            ml_out[2 * tid] = -INFINITY;
            ml_out[2 * tid + 1] = 0.0f;
        }
        return;
    }
    const int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    const int32_t* __restrict__ srow = slot_row_layer + (size_t)b * S;
    uint4* __restrict__ hb = hot_layer + (size_t)b * R * kKvRowU4;

    // remap: logical winner -> the row to read for the chunk's rows of this
    // phase (a split phase keeps its rows compacted in winner order: rows
    // 0 .. n-1 of the block).  Given rows come with the list; otherwise the
    // winner's slot (cache_slots) and the slot's row (slot_row).  With the
    // given list the miss's bitmap word is cleared for the next step
    // (several blocks may store the same zero).  A row that resolves to none
    // (only possible with a broken invariant, which the LRU-update launch
    // reports) reads row 0 instead of leaving the buffer.
    uint32_t* __restrict__ mbw = miss_bits != nullptr ? miss_bits + (size_t)b * wpr : nullptr;
    auto remap = [&](int j, int32_t packed, int32_t given_row, int q) {
        int32_t rd = -1, cp = -1;
        if constexpr (given) {
            rd = given_row;
            if (mbw != nullptr && packed < 0) mbw[(packed & 0x7FFFFFFF) >> 5] = 0u;
        } else {
            const int32_t tok = packed & 0x7FFFFFFF;
            int32_t slot = (tok < cap) ? cs[tok] : -1;
            if (slot >= S) slot = -1;
            if (slot >= 0) {
                rd = srow[slot];
                if (rd >= R) rd = -1;
            }
            if (fused_copy && packed < 0 && rd >= 0) cp = tok;
            if (hg == 0) phys[(size_t)bp * top_k + r0 + j] = slot;
        }
        slot_s[q] = rd >= 0 ? rd : 0;
        cp_s[q] = cp;
    };
    int n = r1 - r0;
    if constexpr (PHASE == kPhaseAll) {
#pragma unroll
        for (int u = 0; u < kRowsPerThread; ++u) {
            const int j = tid + 256 * u;
            if (j < n) remap(j, pk[u], pr[u], j);
        }
    } else {
        int nmine = 0;
#pragma unroll
        for (int u = 0; u < kRowsPerThread; ++u) {
            const int j = tid * kRowsPerThread + u;
            nmine += (j < r1 - r0 && (PHASE == kPhaseHits) == (pk[u] >= 0)) ? 1 : 0;
        }
        int q = block_exclusive_scan<256>(nmine, &n, scratch);
#pragma unroll
        for (int u = 0; u < kRowsPerThread; ++u) {
            const int j = tid * kRowsPerThread + u;
            if (j < r1 - r0 && (PHASE == kPhaseHits) == (pk[u] >= 0)) remap(j, pk[u], pr[u], q++);
        }
    }
    if (n == 0) {  // block-uniform: no rows of this phase in the chunk
        if (tid < kAttnHeadGroup) {
            ml_out[2 * tid] = -INFINITY;
            ml_out[2 * tid + 1] = 0.0f;
        }
        return;
    }
    // rows past the chunk's own, up to the last tile's end, read a real row
    // (row 0: finite data) whose scores the softmax masks, so the tile
    // loads need no condition
    for (int j = n + tid; j < (n + kAttnTileRows - 1) / kAttnTileRows * kAttnTileRows; j += 256) {
        slot_s[j] = 0;
        cp_s[j] = -1;
    }

    // Fused: the missed rows of this chunk are copied from the pool into
    // their rows first (wave w takes rows w, w+4, ...; lanes 0..63 move
    // 16-byte chunks 0..63 of a row, lanes 0..7 chunks 64..71), and the
    // attention below reads them there.
    if (fused_copy) {
        __syncthreads();
        // one row in flight per wave: more outstanding host reads lowered
        // the link rate of this scattered access pattern
        for (int j = wave; j < n; j += 4) {
            const int32_t c = cp_s[j];
            const int32_t dst = c >= 0 ? slot_s[j] : -1;
            // (the newest token's row from its device copy)
            const uint4* sp = c == Lt - 1 ? recent_layer + (size_t)b * kKvRowU4
                                          : pool_layer + ((size_t)b * cap + (c >= 0 ? c : 0)) * kKvRowU4;
            uint4 a = make_uint4(0u, 0u, 0u, 0u), e = make_uint4(0u, 0u, 0u, 0u);
            if (c >= 0) {
                a = sp[lane];
                if (lane < kKvRowU4 - 64) e = sp[64 + lane];
            }
            if (dst >= 0) {
                uint4* dp = hb + (size_t)dst * kKvRowU4;
                dp[lane] = a;
                if (lane < kKvRowU4 - 64) dp[64 + lane] = e;
            }
        }
        __threadfence_block();
    }

    f32x4_t acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    __syncthreads();

    // rows of a tile: 32 x 72 chunks of 16 bytes, 9 per thread; the next
    // tile is fetched into registers while the current one is computed
    constexpr int kPer = kAttnTileRows * kKvRowU4 / 256;
    // the nine 16-byte chunks of this thread, as named registers (an array
    // here was kept in private memory by the compiler)
    static_assert(kPer == 9, "a tile is 9 chunks of 16 bytes per thread");
    uint4 pre0, pre1, pre2, pre3, pre4, pre5, pre6, pre7, pre8;
#define SKO_FETCH1(u, rbase)                                                                   \
    {                                                                                          \
        const int idx = tid + 256 * u;                                                         \
        const int rr = idx / kKvRowU4;                                                         \
        pre##u = hb[(size_t)slot_s[(rbase) + rr] * kKvRowU4 + (idx - rr * kKvRowU4)];          \
    }
#define SKO_FETCH(rbase)                                                                       \
    SKO_FETCH1(0, rbase) SKO_FETCH1(1, rbase) SKO_FETCH1(2, rbase) SKO_FETCH1(3, rbase)        \
    SKO_FETCH1(4, rbase) SKO_FETCH1(5, rbase) SKO_FETCH1(6, rbase) SKO_FETCH1(7, rbase)        \
    SKO_FETCH1(8, rbase)
#define SKO_STASH1(u)                                                                          \
    {                                                                                          \
        const int idx = tid + 256 * u;                                                         \
        const int rr = idx / kKvRowU4;                                                         \
        rows[rr * kRowStrideU4 + (idx - rr * kKvRowU4)] = pre##u;                              \
    }
#define SKO_STASH()                                                                            \
    SKO_STASH1(0) SKO_STASH1(1) SKO_STASH1(2) SKO_STASH1(3) SKO_STASH1(4) SKO_STASH1(5)        \
    SKO_STASH1(6) SKO_STASH1(7) SKO_STASH1(8)
    SKO_FETCH(0)
    SKO_STASH()
    __syncthreads();

    for (int r = 0; r < n; r += kAttnTileRows) {
        const bool more = r + kAttnTileRows < n;
        if (more) {
            SKO_FETCH(r + kAttnTileRows)
        }
        tile_scores(rows, qv, ks0, nks, n16, g, lane, wave, sp);
        __syncthreads();
        tile_softmax_pv(rows, sp, r, n, scale_log2, n16, g, lane, wave, m_run, l_run, acc);
        __syncthreads();
        if (more) {
            SKO_STASH()
            __syncthreads();
        }
    }
#undef SKO_FETCH1
#undef SKO_FETCH
#undef SKO_STASH1
#undef SKO_STASH

    write_partials(acc_out, ml_out, acc, m_run, l_run, h, H, n16, g, wave);
}

// Merge of the per-chunk partials (m, l, acc) of one (seq, position, head):
// out = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c.  Grid (B*D*H, 4):
// a block takes 128 output columns; the chunk weights are computed once in
// LDS and every thread then sums its column over the chunks.
constexpr int kCombineThreads = 128;
constexpr int kMaxChunks = 1024;

__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(const float* __restrict__ part_acc,
                                                                  const float* __restrict__ part_ml,
                                                                  float* __restrict__ out, int H,
                                                                  int HG, int nchunk, int nbph, int xc) {
    __shared__ float wgt[kMaxChunks];
    __shared__ float red[2 * kCombineThreads / 64];
    // work block (bph, column block), bph fastest
    const int wk = split_block(blockIdx.x, xc);
    if (wk < 0 || wk >= nbph * (kVDim / kCombineThreads)) return;  // block-uniform
    const int bph = wk % nbph, cblk = wk / nbph;
    const int bp = bph / H, h = bph - bp * H;
    const int hg = h / kAttnHeadGroup, hl = h - hg * kAttnHeadGroup;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const size_t pbase = ((size_t)bp * HG + hg) * nchunk;
    // each thread's (m, l) pairs stay in registers between the max and the
    // weights (nchunk <= kMaxChunks: at most kCombinePer per thread)
    constexpr int kCombinePer = kMaxChunks / kCombineThreads;
    float mv[kCombinePer], lv[kCombinePer];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < kCombinePer; ++i) {
        const int c = tid + i * kCombineThreads;
        mv[i] = -INFINITY;
        lv[i] = 0.0f;
        if (c < nchunk) {
            const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((pbase + c) * kAttnHeadGroup + hl) * 2);
            mv[i] = ml.x;
            lv[i] = ml.y;
            if (ml.y > 0.0f) mloc = fmaxf(mloc, ml.x);
        }
    }
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    if (lane == 0) red[wid] = mloc;
    __syncthreads();
    const float M = fmaxf(red[0], red[1]);
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombinePer; ++i) {
        const int c = tid + i * kCombineThreads;
        if (c < nchunk) {
            const float wc = (lv[i] > 0.0f) ? exp2f(mv[i] - M) : 0.0f;
            wgt[c] = wc;
            lsum += wc * lv[i];
        }
    }
    for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) red[2 + wid] = lsum;
    __syncthreads();
    const float L = red[2] + red[3];
    const int col = cblk * kCombineThreads + tid;
    const float* __restrict__ src = part_acc + (pbase * kAttnHeadGroup + hl) * kVDim + col;
    const size_t cstride = (size_t)kAttnHeadGroup * kVDim;
    float acc = 0.0f;
    int c = 0;
    // chunks without rows (weight 0) never wrote their accumulators: they
    // are skipped, not scaled by zero
    for (; c + 8 <= nchunk; c += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(c + u) * cstride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = (wgt[c + u] > 0.0f) ? fmaf(wgt[c + u], v[u], acc) : acc;
    }
    for (; c < nchunk; ++c) acc = (wgt[c] > 0.0f) ? fmaf(wgt[c], src[(size_t)c * cstride], acc) : acc;
    out[((size_t)bp * H + h) * kVDim + col] = (L > 0.0f) ? acc / L : 0.0f;
}

hipError_t launch_attn_partial(hipStream_t st, const int32_t* topk, const int32_t* cache_slots_layer,
                               const int32_t* slot_row_layer, uint16_t* hot_layer, int R, const uint16_t* q_attn,
                               const uint16_t* pool_layer, const uint16_t* recent_layer, const int32_t* ntok_layer,
                               float* part_acc, float* part_ml, int32_t* phys, int B, int D, int H, int top_k, int S,
                               int64_t cap, int rows_per_block, float scale, const int32_t* wrow,
                               uint32_t* miss_bits, int phase, int xc) {
    const int HG = (H + kAttnHeadGroup - 1) / kAttnHeadGroup;
    const int nchunk = (top_k + rows_per_block - 1) / rows_per_block;
    const int pchunks = phase == 0 ? nchunk : 2 * nchunk;
    const float scale_log2 = scale * 1.4426950408889634f;
#define SKO_ATTN_LAUNCH(W, P)                                                                                 \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_attn_partial<W, P>), dim3(split_grid((int64_t)nchunk * B * D * HG, xc)), \
                       dim3(256), 0, st, topk,                                                                   \
                       cache_slots_layer, slot_row_layer, reinterpret_cast<uint4*>(hot_layer),                   \
                       reinterpret_cast<const uint4*>(q_attn), reinterpret_cast<const uint4*>(pool_layer),       \
                       reinterpret_cast<const uint4*>(recent_layer), ntok_layer, part_acc, part_ml, phys, wrow,  \
                       miss_bits, winner_words(cap), D, H, HG, top_k, S, R, cap, rows_per_block, nchunk, pchunks, \
                       scale_log2, B * D, xc)
    if (pool_layer != nullptr && wrow != nullptr) return hipErrorInvalidValue;
    if (phase == 1) {
        // the rows resident at step start: no copy of any kind
        SKO_ATTN_LAUNCH(kRowsTables, kPhaseHits);
    } else if (phase == 2) {
        if (wrow == nullptr) return hipErrorInvalidValue;
        SKO_ATTN_LAUNCH(kRowsGiven, kPhaseMisses);
    } else if (pool_layer != nullptr) {
        SKO_ATTN_LAUNCH(kRowsFusedCopy, kPhaseAll);
    } else if (wrow != nullptr) {
        SKO_ATTN_LAUNCH(kRowsGiven, kPhaseAll);
    } else {
        SKO_ATTN_LAUNCH(kRowsTables, kPhaseAll);
    }
#undef SKO_ATTN_LAUNCH
    return hipGetLastError();
}

// One sequence's rows in slot order (for reading the hot buffer by slot):
// block s copies row slot_row[s] (lanes: 16-byte chunks).
__global__ __launch_bounds__(128) void k_gather_slots(const uint4* __restrict__ hot_seq,
                                                      const int32_t* __restrict__ slot_row_seq, int R,
                                                      uint4* __restrict__ dst) {
    const int s = blockIdx.x;
    const int32_t row = slot_row_seq[s];
    if (row < 0 || row >= R) return;  // never with intact tables
    for (int c = threadIdx.x; c < kKvRowU4; c += 128) dst[(size_t)s * kKvRowU4 + c] = hot_seq[(size_t)row * kKvRowU4 + c];
}

hipError_t launch_gather_slots(hipStream_t st, const uint16_t* hot_seq, const int32_t* slot_row_seq, int S, int R,
                               uint16_t* dst) {
    if (S < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gather_slots, dim3(S), dim3(128), 0, st, reinterpret_cast<const uint4*>(hot_seq),
                       slot_row_seq, R, reinterpret_cast<uint4*>(dst));
    return hipGetLastError();
}

hipError_t launch_attn_combine(hipStream_t st, const float* part_acc, const float* part_ml,
                               float* out, int B, int D, int H, int nchunk, int xc) {
    const int HG = (H + kAttnHeadGroup - 1) / kAttnHeadGroup;
    if (nchunk > kMaxChunks) return hipErrorInvalidValue;
    const int nbph = B * D * H;
    hipLaunchKernelGGL(k_attn_combine, dim3(split_grid((int64_t)nbph * (kVDim / kCombineThreads), xc)),
                       dim3(kCombineThreads), 0, st, part_acc, part_ml, out, H, HG, nchunk, nbph, xc);
    return hipGetLastError();
}

}  // namespace sko
