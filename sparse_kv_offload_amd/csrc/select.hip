// Token append, indexer scoring and the packed top-k selection.
//
// Scoring and selection follow [LSO] section 4 "Decode step" (the indexer
// picks logical top-k positions) and the FlashOffloading explainer's decode
// paragraphs (every winner carries its token index and its residency in one
// int32, so the selection already says hit or miss).  The score of token i
// for query position p is the 64-d dot product q_p . K_i accumulated in
// binary32 by fused multiply-add in index order 0..63 from +0; winners are
// the min(k, L_t) largest (score, -index) pairs.
//
// Selection is a radix select over the monotone 32-bit key of the score:
//   1. k_score_hist: one coalesced pass over the tiled indexer cache (the HBM
//      stream) that builds a 12-bit first-digit histogram per row and keeps
//      the (key, token) candidates whose first digit is at or above the
//      row's floor (set from the previous step's histogram);
//   2. k_topk_filter: every block finds the bucket holding the k-th largest
//      key of its row; keys above it are winners; keys in it are staged (or
//      taken whole when the bucket fits exactly).  It reads the candidates
//      when they hold every winner and rescans the row's tokens otherwise,
//      and sets the rows' floors for the next step.  Appends are aggregated
//      per block;
//   3. the merge kernel (merge_lru.hip) resolves a split bucket exactly on
//      the composite (low 20 key bits, inverted index), so ties go to
//      smaller indices.
// No kernel waits on another block of the same launch: cross-block results
// are handed over at kernel boundaries.
// Winners are written packed (bit 31 = absent from the hot buffer at step
// start) and also marked in a per-sequence bitmap over tokens, which the
// merge stage reads in token order (union and dedupe of the D positions).
#include <hip/hip_fp16.h>

#include <utility>

#include "sko_common.h"
#include "sko_internal.h"

namespace sko {

// ---------------------------------------------------------------- append

// Rows of new tokens.  16-byte chunks 0..7 of a row are the indexer row
// (to the tiled device cache); chunks 8..79 the main-KV row (to the host
// pool through its device mapping, and the last row of each sequence also
// to the device copy of its newest row; skipped when kv_src is null because
// the host already wrote it).  Sets the sequence's token count to base + n.
__global__ __launch_bounds__(256) void k_append_rows(const uint4* __restrict__ idx_src,
                                                     const uint4* __restrict__ kv_src,
                                                     uint4* __restrict__ idx_layer,
                                                     uint4* __restrict__ pool_layer,
                                                     uint4* __restrict__ recent_layer,
                                                     int32_t* __restrict__ ntok_layer, int seq0,
                                                     int64_t n, int64_t cap, int64_t ntiles,
                                                     int32_t base) {
    const int s = blockIdx.y;
    const int b = seq0 + s;
    const int parts = kv_src ? (kIdxRowU4 + kKvRowU4) : kIdxRowU4;
    const int64_t chunks = n * parts;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = c / parts;
        const int part = (int)(c - r * parts);
        const int64_t src_row = (int64_t)s * n + r;
        const int64_t tok = base + r;
        if (part < kIdxRowU4)
            idx_layer[idx_tile_u4((size_t)b * ntiles, tok, part)] = idx_src[src_row * kIdxRowU4 + part];
        else {
            const uint4 v = kv_src[src_row * kKvRowU4 + (part - kIdxRowU4)];
            pool_layer[((int64_t)b * cap + tok) * kKvRowU4 + (part - kIdxRowU4)] = v;
            if (r == n - 1) recent_layer[(int64_t)b * kKvRowU4 + (part - kIdxRowU4)] = v;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) ntok_layer[b] = base + (int32_t)n;
}

hipError_t launch_append_rows(hipStream_t st, const uint16_t* idx_src, const uint16_t* kv_src,
                              uint16_t* idx_layer, uint16_t* pool_layer, uint16_t* recent_layer,
                              int32_t* ntok_layer, int seq0, int nseq, int64_t n, int64_t cap, int64_t ntiles,
                              int32_t base) {
    const int64_t chunks = n * (kv_src ? (kIdxRowU4 + kKvRowU4) : kIdxRowU4);
    int gx = (int)std::min<int64_t>((chunks + 255) / 256, 4096);
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(k_append_rows, dim3(gx, nseq), dim3(256), 0, st,
                       reinterpret_cast<const uint4*>(idx_src), reinterpret_cast<const uint4*>(kv_src),
                       reinterpret_cast<uint4*>(idx_layer), reinterpret_cast<uint4*>(pool_layer),
                       reinterpret_cast<uint4*>(recent_layer), ntok_layer, seq0, n, cap, ntiles, base);
    return hipGetLastError();
}

// ------------------------------------------------------- int8 indexer rows

// One wave rotates and quantizes one bf16 row (LIM C8 of [LSO-zh] section 4:
// Hadamard rotation, then int8 codes with an fp16 dequantization scale).
// Lane i holds x_i and gets code i; every lane gets the scale bits.
//   x'_i = (1/8) sum_j (-1)^popcount(i & j) x_j, a binary32 sum in index
//          order j = 0..63 from +0 (every term exact);
//   s = max_i |x'_i| / 127, code_i = round-half-even(x'_i / s) clamped to
//   [-127, 127]; the scale is s rounded to binary16 (a zero row: all 0).
__device__ __forceinline__ int quant_row_wave(float xi, uint32_t* scale16) {
    const int lane = threadIdx.x & 63;
    float acc = 0.0f;
#pragma unroll 4
    for (int j = 0; j < kIdxDim; ++j) {
        const float xj = __shfl(xi, j);
        acc = (__popc((unsigned)(lane & j)) & 1) ? acc - xj : acc + xj;
    }
    const float xr = acc * 0.125f;
    float a = fabsf(xr);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    if (a == 0.0f) {  // wave-uniform
        *scale16 = 0u;
        return 0;
    }
    const float s = a / 127.0f;  // binary32 division, correctly rounded
    const float r = fminf(127.0f, fmaxf(-127.0f, rintf(xr / s)));
    *scale16 = (uint32_t)__half_as_ushort(__float2half_rn(s));
    return (int)r;
}

// Four lanes' int8 codes packed little-endian into one word: lane 4w + e
// holds code e of word w (the result is valid in lanes 4w).
__device__ __forceinline__ uint32_t pack_codes4(int code) {
    const uint32_t b = (uint32_t)code & 0xFFu;
    const uint32_t b1 = __shfl_down(b, 1), b2 = __shfl_down(b, 2), b3 = __shfl_down(b, 3);
    return b | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Append with the int8 indexer: each wave rotates and quantizes rows and
// writes their codes (tiled) and scales; the threads then copy the
// main-KV rows to the pool as k_append_rows does.
__global__ __launch_bounds__(256) void k_append_rows_c8(const uint16_t* __restrict__ idx_src,
                                                        const uint4* __restrict__ kv_src,
                                                        uint32_t* __restrict__ codes_layer,
                                                        uint16_t* __restrict__ scales_layer,
                                                        uint4* __restrict__ pool_layer,
                                                        uint4* __restrict__ recent_layer,
                                                        int32_t* __restrict__ ntok_layer, int seq0, int64_t n,
                                                        int64_t cap, int64_t ntiles, int32_t base) {
    const int s = blockIdx.y;
    const int b = seq0 + s;
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / 64);
    for (int64_t r = gw; r < n; r += nwaves) {
        const int64_t src_row = (int64_t)s * n + r;
        const int64_t tok = base + r;
        const float xi = __uint_as_float((uint32_t)idx_src[src_row * kIdxDim + lane] << 16);
        uint32_t sc;
        const int code = quant_row_wave(xi, &sc);
        const uint32_t word = pack_codes4(code);
        if ((lane & 3) == 0) {
            const int w = lane >> 2;  // word w of the row: chunk w / 4, word w % 4 of it
            codes_layer[idx_c8_tile_u4((size_t)b * ntiles, tok, w >> 2) * 4 + (w & 3)] = word;
        }
        if (lane == 0) scales_layer[(size_t)b * ntiles * kIdxTile + tok] = (uint16_t)sc;
    }
    if (kv_src) {
        const int64_t chunks = n * kKvRowU4;
        for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
             c += (int64_t)gridDim.x * blockDim.x) {
            const int64_t r = c / kKvRowU4;
            const int part = (int)(c - r * kKvRowU4);
            const uint4 v = kv_src[((int64_t)s * n + r) * kKvRowU4 + part];
            pool_layer[((int64_t)b * cap + base + r) * kKvRowU4 + part] = v;
            if (r == n - 1) recent_layer[(int64_t)b * kKvRowU4 + part] = v;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) ntok_layer[b] = base + (int32_t)n;
}

hipError_t launch_append_rows_c8(hipStream_t st, const uint16_t* idx_src, const uint16_t* kv_src,
                                 uint8_t* idx_layer, uint16_t* scales_layer, uint16_t* pool_layer,
                                 uint16_t* recent_layer, int32_t* ntok_layer, int seq0, int nseq, int64_t n,
                                 int64_t cap, int64_t ntiles, int32_t base) {
    const int64_t by_rows = (n + 3) / 4;
    const int64_t by_kv = kv_src ? (n * kKvRowU4 + 255) / 256 : 1;
    int gx = (int)std::min<int64_t>(std::max(by_rows, by_kv), 4096);
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(k_append_rows_c8, dim3(gx, nseq), dim3(256), 0, st, idx_src,
                       reinterpret_cast<const uint4*>(kv_src), reinterpret_cast<uint32_t*>(idx_layer),
                       scales_layer, reinterpret_cast<uint4*>(pool_layer), reinterpret_cast<uint4*>(recent_layer),
                       ntok_layer, seq0, n, cap, ntiles, base);
    return hipGetLastError();
}

// ---------------------------------------------------------------- threshold

// Block of 256 threads: bucket of the kk-th largest key of one row, and the
// candidate floor for the next step: one bin below the highest bin at which
// the count from the top reaches kFloorCover * kk (0 when it never does).
__device__ void threshold_row(const uint32_t* __restrict__ h, RowMeta* __restrict__ meta, int kk,
                              int* scratch, RowMeta* s_res, int* s_floor) {
    const int hi_bin = kHistBins - 1 - 16 * (int)threadIdx.x;  // thread 0 owns the top bins
    uint32_t loc[16];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        loc[j] = h[hi_bin - j];
        sum += (int)loc[j];
    }
    if (threadIdx.x == 0) {
        *s_res = RowMeta{-1, 0, 0, 0, 0, 0, 0, 0};
        *s_floor = 0;
    }
    int total;
    const int excl = block_exclusive_scan<256>(sum, &total, scratch);
    if (kk > 0 && excl < kk && excl + sum >= kk) {
        int c = excl;
        for (int j = 0; j < 16; ++j) {
            const int cnt = (int)loc[j];
            if (c + cnt >= kk) {
                *s_res = RowMeta{hi_bin - j, c, kk - c, cnt, 0, 0, 0, 0};
                break;
            }
            c += cnt;
        }
    }
    const int cover = kFloorCover * kk;
    if (kk > 0 && excl < cover && excl + sum >= cover) {
        int c = excl;
        for (int j = 0; j < 16; ++j) {
            c += (int)loc[j];
            if (c >= cover) {
                *s_floor = hi_bin - j > 0 ? hi_bin - j - 1 : 0;
                break;
            }
        }
    }
    __syncthreads();
    if (meta != nullptr && threadIdx.x == 0) {
        // the list counters are updated concurrently by other blocks
        meta->bucket = s_res->bucket;
        meta->above = s_res->above;
        meta->need = s_res->need;
        meta->bucket_count = s_res->bucket_count;
    }
}

// ---------------------------------------------------------------- score

// acc = fma(q, k, acc) with q taken from lane E % 16 of the 16-lane row of
// qv (every row of qv holds the same 16 query values): the broadcast rides
// on the DPP source operand of the fused multiply-add, so the query costs
// no scalar or extra vector instruction.
template <int E>
__device__ __forceinline__ float fma_row_bcast(float qv, float k, float acc) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(qv), "v"(k), "n"(E % 16));
    return acc;
}

// The NP chains of one token (the 32 packed key words w; term e is the low
// half of word e/2 for even e, the high half for odd e), term by term: term
// e is unpacked once and feeds the e-th FMA of every position's chain (each
// chain still runs in index order e = 0..63), so the unpacked key never
// needs 64 live registers (measured 3.5 % faster at D = 4 than whole chains
// one position after another).  vq[p][e / 16] holds position p's query
// terms 16*(e/16) .. +15 as above.
template <int NP, int E>
__device__ __forceinline__ void chains_term(const float (&vq)[NP][4], const uint32_t (&w)[32], float (&acc)[NP]) {
    const float kf = (E & 1) ? bf16_hi(w[E / 2]) : bf16_lo(w[E / 2]);
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[p] = fma_row_bcast<E>(vq[p][E / 16], kf, acc[p]);
}

template <int NP, int... E>
__device__ __forceinline__ void score_chains(const float (&vq)[NP][4], const uint32_t (&w)[32], float (&acc)[NP],
                                             std::integer_sequence<int, E...>) {
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[p] = 0.0f;
    (chains_term<NP, E>(vq, w, acc), ...);
}

// A staged candidate (key, token) with the token's residency at step start
// packed in: the low word becomes the packed winner value token | miss << 31.
__device__ __forceinline__ uint2 with_residency(uint2 v, const int32_t* __restrict__ cs) {
    return make_uint2(v.x, v.y | (cs[v.y] == -1 ? 0x80000000u : 0u));
}

// Key of token `token` for one query row, computed exactly as the score pass
// does (64-term binary32 FMA chain in index order from +0; a zero is +0).
// Used by the rescan path of the filter.
__device__ __forceinline__ uint32_t token_key(const uint4* __restrict__ idx_layer, size_t seq_tiles_base,
                                              int64_t token, const uint32_t* __restrict__ qrow) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kIdxRowU4; ++c) {
        const uint4 v = idx_layer[idx_tile_u4(seq_tiles_base, token, c)];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t qw = qrow[4 * c + m];
            acc = __builtin_fmaf(bf16_lo(qw), bf16_lo(w4[m]), acc);
            acc = __builtin_fmaf(bf16_hi(qw), bf16_hi(w4[m]), acc);
        }
    }
    if (acc == 0.0f) acc = 0.0f;
    return score_key(acc);
}

// Key of token `token` with the int8 indexer: the exact int32 dot of the
// codes (any order gives the same sum), then (dot * s_k) * s_q in binary32.
__device__ __forceinline__ uint32_t token_key_c8(const uint4* __restrict__ codes_layer,
                                                 const uint16_t* __restrict__ scales_layer,
                                                 size_t seq_tiles_base, int64_t token,
                                                 const uint32_t* __restrict__ q8row) {
    int dot = 0;
#pragma unroll
    for (int c = 0; c < kIdxC8RowU4; ++c) {
        const uint4 v = codes_layer[idx_c8_tile_u4(seq_tiles_base, token, c)];
        dot = __builtin_amdgcn_sdot4((int)v.x, (int)q8row[4 * c + 0], dot, false);
        dot = __builtin_amdgcn_sdot4((int)v.y, (int)q8row[4 * c + 1], dot, false);
        dot = __builtin_amdgcn_sdot4((int)v.z, (int)q8row[4 * c + 2], dot, false);
        dot = __builtin_amdgcn_sdot4((int)v.w, (int)q8row[4 * c + 3], dot, false);
    }
    const float sk = __half2float(__ushort_as_half(scales_layer[seq_tiles_base * kIdxTile + token]));
    const float sq = __half2float(__ushort_as_half((uint16_t)q8row[kIdxDim / 4]));
    float acc = (float)dot * sk;
    acc = acc * sq;
    if (acc == 0.0f) acc = 0.0f;
    return score_key(acc);
}

// Score pass over the flattened (sequence, tile) space of B * tiles_now
// tiles of 64 tokens: block j takes the contiguous range
// [j * total / nblocks, (j + 1) * total / nblocks), and the launch holds at
// most as many blocks as the chip keeps resident at once, so every block
// gets the same share and no second round of blocks forms a tail.  A range
// is cut at sequence boundaries into segments; within a segment wave w of
// the block's nw waves takes tiles w, w+nw, ...; lane l owns token
// 64*tile + l and reads its row as 8 loads of 16 bytes, each a coalesced
// 1 KB run of the tiled layout.  Every position p0 .. p0+NP-1 runs its
// 64-term FMA chain in index order.
//
// Outputs per row (seq, position):
//   * the first-digit histogram of all keys, counted in LDS and flushed with
//     one 64-bit global atomic per non-empty pair of bins.  Blocks are
//     large (all the waves one CU holds at this kernel's register use), so a
//     row is split over few blocks and its bins receive few atomics;
//   * the candidates: (key, token | miss << 31) of every key whose first digit is at or
//     above the row's floor (set from the previous step's threshold), staged
//     per wave in LDS and appended to pre[row] with one reservation per block
//     and row at the end of a segment (a wave whose staging fills up
//     reserves for itself).  Writing all keys
//     instead would add 4 bytes per token and position to a read-only
//     stream, which costs far more than its size in HBM time;
//   * all keys, only in the KEEP instantiation (kept for inspection).
template <int NP>
constexpr int score_threads() { return NP == 1 ? 640 : 768; }

// The C8 instantiation reads the int8 indexer instead (4 chunks of codes
// and one fp16 scale per token): its queries are rotated and quantized at
// the start of each segment (waves 0..NP-1, one row each, also written to
// qc8 for the filter), and a score is the exact int32 dot of the codes
// (dot4 instructions; every order gives the same sum) times s_k, times s_q.
template <int NP, bool KEEP, bool C8>
__global__ __launch_bounds__(score_threads<NP>()) void k_score_hist(
    const uint4* __restrict__ idx_layer, const uint32_t* __restrict__ q_idx,
    const int32_t* __restrict__ ntok_layer, uint32_t* __restrict__ keys, uint32_t* __restrict__ hist,
    const int32_t* __restrict__ floor_layer, uint2* __restrict__ pre, RowMeta* __restrict__ meta,
    const int32_t* __restrict__ cache_slots_layer, int D, int p0, int64_t kcap, int64_t cap, int64_t ntiles,
    int64_t tiles_now, int64_t total_tiles, const uint16_t* __restrict__ scales_layer,
    uint32_t* __restrict__ qc8, ScoreAppend app, int nwork, int xc) {
    constexpr int nw = score_threads<NP>() / 64;
    constexpr int RU = C8 ? kIdxC8RowU4 : kIdxRowU4;  // 16-byte loads per token
    __shared__ uint32_t sh[NP * kHistBins];
    // C8: per position, the query codes (16 words) then the scale bits,
    // rows of 5 x 16 bytes so the codes are read with 16-byte loads
    __shared__ uint4 sq8[C8 ? NP : 1][5];
    __shared__ uint2 stage[nw][NP][kPreStage];
    __shared__ int s_cnt[nw][NP];
    __shared__ float sq[NP > 1 ? NP * kIdxDim : 1];
    __shared__ int s_base[NP];
    // the fused append: the new token's indexer row of the segment's
    // sequence as the cache holds it (bf16: 32 words; int8: 16 words of
    // codes, then the scale bits)
    __shared__ uint4 snew4[kIdxRowU4];
    uint32_t* const snew = reinterpret_cast<uint32_t*>(snew4);
    const int add = app.idx != nullptr ? 1 : 0;  // tokens appended by this launch, per sequence
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // nwork work blocks, each a contiguous range of the (seq, tile) space
    const int wb = split_block(blockIdx.x, xc);
    if (wb < 0 || wb >= nwork) return;  // block-uniform
    const int64_t r_begin = (int64_t)wb * total_tiles / nwork;
    const int64_t r_end = ((int64_t)wb + 1) * total_tiles / nwork;
    // query terms of positions p0.. of row0's sequence, staged in LDS (the
    // caller synchronizes).  qbits: this thread's bf16 term (thread t holds
    // term t % 64 of position t / 64).  The int8 indexer quantizes each
    // position's rotated query (waves 0..NP-1, one row each) into sq8 and
    // qc8; otherwise the terms go to sq as binary32, where each chain loads
    // its position's terms 16 per register (replicated in the four 16-lane
    // rows): register m, lane l holds term 16*m + (l % 16).
    auto stage_query = [&](size_t row0, uint32_t qbits) {
        if constexpr (C8) {
            if (wave < NP) {
                uint32_t sc;
                const int code = quant_row_wave(__uint_as_float(qbits << 16), &sc);
                const uint32_t word = pack_codes4(code);
                uint32_t* qg = qc8 + (row0 + wave) * kQc8Words;
                uint32_t* ql = reinterpret_cast<uint32_t*>(&sq8[wave][0]);
                if ((lane & 3) == 0) {
                    ql[lane >> 2] = word;
                    qg[lane >> 2] = word;
                }
                if (lane == 0) {
                    ql[kIdxDim / 4] = sc;
                    qg[kIdxDim / 4] = sc;
                }
            }
        } else if constexpr (NP > 1) {
            static_assert(NP == 1 || score_threads<NP>() >= NP * kIdxDim, "one query term per thread");
            if ((int)threadIdx.x < NP * kIdxDim) sq[threadIdx.x] = __uint_as_float(qbits << 16);
        }
    };
    // the fused append: wave NP stages the new token's row (element `elem`
    // of it per lane), quantized for the int8 indexer (the caller
    // synchronizes)
    auto stage_new = [&](uint32_t elem) {
        if (wave == NP) {
            if constexpr (C8) {
                uint32_t sc;
                const int code = quant_row_wave(__uint_as_float(elem << 16), &sc);
                const uint32_t word = pack_codes4(code);
                if ((lane & 3) == 0) snew[lane >> 2] = word;
                if (lane == 0) snew[kIdxDim / 4] = sc;
            } else {
                reinterpret_cast<uint16_t*>(snew)[lane] = (uint16_t)elem;
            }
        }
    };
    // this lane's element of sequence b's new row (any valid row when there
    // is none, so that the load needs no branch)
    auto new_elem = [&](int b) -> uint32_t {
        const uint16_t* src = add ? app.idx + (size_t)b * kIdxDim
                                  : reinterpret_cast<const uint16_t*>(q_idx) + (size_t)b * D * kIdxDim;
        return src[lane];
    };
    // this thread's query term (clamped in bounds; used by threads below
    // NP * 64 only)
    auto query_bits = [&](size_t row0) -> uint32_t {
        return (uint32_t)reinterpret_cast<const uint16_t*>(q_idx)[row0 * kIdxDim +
                                                                  std::min<int>(threadIdx.x, NP * kIdxDim - 1)];
    };
    // Two register tiles per wave (ping-pong, below).  The wave's first tile
    // of the block's first segment is requested before the block's set-up
    // (query staging, histogram clear), so its latency overlaps that work.
    // Every block has at least one tile of the flattened space (the launch
    // holds at most as many blocks as tiles), and the loads below are
    // unconditional on clamped indexes, so the set-up waits only for the
    // query term, not for the tile.
    uint4 ra[RU], rb[RU];
    uint32_t sa = 0u, sb = 0u;  // C8: the lane's token scales
    const int b_first = (int)(r_begin / tiles_now);
    const size_t row0_first = (size_t)b_first * D + p0;
    const uint32_t qpre = (NP > 1 || C8) ? query_bits(row0_first) : 0u;
    const uint32_t npre = new_elem(b_first);
    // keep the query load ahead of the tile loads: loads complete in order,
    // so waiting for it then leaves the tile in flight
    __builtin_amdgcn_sched_barrier(0);
    bool preloaded;  // ra holds this wave's first tile of the first segment
    {
        const int64_t tile0 = r_begin - (int64_t)b_first * tiles_now;
        const int64_t tile_end = std::min<int64_t>(std::min<int64_t>(r_end, ((int64_t)b_first + 1) * tiles_now) -
                                                       (int64_t)b_first * tiles_now,
                                                   (ntok_layer[b_first] + kIdxTile - 1) / kIdxTile);
        const int64_t tile = tile0 + wave;
        preloaded = tile < tile_end;
        // a wave without a tile reads an in-range one it does not use
        const int64_t tl = std::max<int64_t>(0, std::min<int64_t>(tile, tile_end - 1));
        const uint4* __restrict__ st = idx_layer + (size_t)b_first * ntiles * RU * kIdxTile + lane;
#pragma unroll
        for (int c = 0; c < RU; ++c) ra[c] = load_nt_u4(st + (tl * RU + c) * kIdxTile);
        if constexpr (C8) sa = scales_layer[(size_t)b_first * ntiles * kIdxTile + lane + tl * kIdxTile];
    }
    // the first segment's queries while its first tiles are in flight
    stage_query(row0_first, qpre);
    if (add) stage_new(npre);
    for (int i = threadIdx.x; i < NP * kHistBins; i += blockDim.x) sh[i] = 0u;
    __syncthreads();
    for (int64_t seg = r_begin; seg < r_end;) {
        const bool first_segment = seg == r_begin;
        const int b = (int)(seg / tiles_now);
        const int64_t seg_end = std::min<int64_t>(r_end, ((int64_t)b + 1) * tiles_now);
        // Lt: the tokens the cache holds at launch (the tile loop's tokens);
        // the fused append adds token Lt, which the block whose range holds
        // its tile scores on its own, from the staged row
        const int64_t Lt = ntok_layer[b];
        const int64_t tile0 = seg - (int64_t)b * tiles_now;
        const int64_t tile_end = std::min<int64_t>(seg_end - (int64_t)b * tiles_now,
                                                   (Lt + kIdxTile - 1) / kIdxTile);
        const bool own_new = add && Lt / kIdxTile >= tile0 && Lt / kIdxTile < seg_end - (int64_t)b * tiles_now;
        seg = seg_end;
        if (tile0 >= tile_end && !own_new) continue;  // block-uniform: nothing of this sequence here
        const size_t row0 = (size_t)b * D + p0;
        const uint32_t* __restrict__ qb = q_idx + row0 * (kIdxDim / 2);
        uint32_t* __restrict__ keyrow = keys + row0 * kcap;
        const uint4* __restrict__ seq_tiles = idx_layer + (size_t)b * ntiles * RU * kIdxTile + lane;
        const uint16_t* __restrict__ seq_scales = C8 ? scales_layer + (size_t)b * ntiles * kIdxTile + lane : nullptr;
        const int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
        if ((NP > 1 || C8 || add) && !first_segment) {
            stage_query(row0, query_bits(row0));
            if (add) stage_new(new_elem(b));
            __syncthreads();
        }

        uint32_t floor_bin[NP];
        int nstage[NP];  // wave-uniform
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            floor_bin[p] = (uint32_t)floor_layer[row0 + p];
            nstage[p] = 0;
        }
        if (own_new) {  // block-uniform
            // the layer's first launch writes the appended token: its
            // indexer row to the cache (int8: codes and scale), its main-KV
            // row to the device copy of the newest row, the token count
            if (app.write) {
                const int t = threadIdx.x;
                if (t < kKvRowU4) {
                    app.recent[(size_t)b * kKvRowU4 + t] = app.kv[(size_t)b * kKvRowU4 + t];
                } else if (t < kKvRowU4 + RU) {
                    const int c = t - kKvRowU4;
                    uint4* cache = static_cast<uint4*>(app.idx_cache);
                    if constexpr (C8) cache[idx_c8_tile_u4((size_t)b * ntiles, Lt, c)] = snew4[c];
                    else cache[idx_tile_u4((size_t)b * ntiles, Lt, c)] = snew4[c];
                } else if (t == kKvRowU4 + RU) {
                    if constexpr (C8) app.scales[(size_t)b * ntiles * kIdxTile + Lt] = (uint16_t)snew[kIdxDim / 4];
                    app.ntok_out[b] = (int32_t)(Lt + 1);
                }
            }
            // wave NP scores it for every position (lane 0, the same
            // arithmetic as the tile loop) and counts and stages its keys
            if (wave == NP) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    uint32_t key = 0u;
                    if (lane == 0) {
                        float acc;
                        if constexpr (C8) {
                            int dot = 0;
#pragma unroll
                            for (int c = 0; c < kIdxC8RowU4; ++c) {
                                const uint4 qv = sq8[p][c];
                                dot = __builtin_amdgcn_sdot4((int)snew[4 * c + 0], (int)qv.x, dot, false);
                                dot = __builtin_amdgcn_sdot4((int)snew[4 * c + 1], (int)qv.y, dot, false);
                                dot = __builtin_amdgcn_sdot4((int)snew[4 * c + 2], (int)qv.z, dot, false);
                                dot = __builtin_amdgcn_sdot4((int)snew[4 * c + 3], (int)qv.w, dot, false);
                            }
                            const float sq = __half2float(__ushort_as_half((uint16_t)sq8[p][4].x));
                            acc = (float)dot * __half2float(__ushort_as_half((uint16_t)snew[kIdxDim / 4]));
                            acc = acc * sq;
                        } else {
                            acc = 0.0f;
                            const uint32_t* __restrict__ qr = qb + (size_t)p * (kIdxDim / 2);
#pragma unroll
                            for (int j = 0; j < kIdxDim / 2; ++j) {
                                const uint32_t qw = qr[j];
                                acc = __builtin_fmaf(bf16_lo(qw), bf16_lo(snew[j]), acc);
                                acc = __builtin_fmaf(bf16_hi(qw), bf16_hi(snew[j]), acc);
                            }
                        }
                        acc += 0.0f;
                        key = score_key(acc);
                    }
                    key = __shfl(key, 0);
                    const uint32_t bin = key >> (32 - kHistBits);
                    if (lane == 0) {
                        if constexpr (KEEP) keyrow[(size_t)p * kcap + Lt] = key;
                        atomicAdd(&sh[p * kHistBins + bin], 1u);
                    }
                    if (bin >= floor_bin[p]) {  // wave-uniform
                        if (lane == 0) stage[wave][p][0] = make_uint2(key, (uint32_t)Lt);
                        nstage[p] = 1;
                    }
                }
            }
        }
        // append this wave's staged candidates of position p to pre[row]
        auto flush = [&](int p) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&meta[row0 + p].pre_count, nstage[p]);
            base = __shfl(base, 0);
            uint2* __restrict__ dst = pre + (row0 + p) * (size_t)cap + base;
            for (int e = lane; e < nstage[p]; e += 64) dst[e] = with_residency(stage[wave][p][e], cs);
            nstage[p] = 0;
        };
        // Ping-pong over two register tiles: the next tile's 8 loads are in
        // flight while this tile's FMA chains run.  Loads are unconditional
        // (the tile index is clamped to the last valid tile) so that the
        // compiler's wait counts stay "all but the newest 8 loads".
        const int64_t last = tile_end - 1;
        auto load_tile = [&](uint4* r, uint32_t& scv, int64_t tile) {
            const int64_t tl = tile < last ? tile : last;
#pragma unroll
            for (int c = 0; c < RU; ++c) r[c] = load_nt_u4(seq_tiles + (tl * RU + c) * kIdxTile);
            if constexpr (C8) scv = seq_scales[tl * kIdxTile];
        };
        // the chains run for every lane (lanes past the last token compute on
        // a clamped in-bounds row and store nothing), so every loaded
        // register is consumed on every path
        auto score_tile = [&](const uint4* r, uint32_t scv, int64_t tile) {
            const int64_t i = tile * kIdxTile + lane;
            const bool valid = i < Lt;
            uint32_t w[4 * RU];
#pragma unroll
            for (int c = 0; c < RU; ++c) {
                w[4 * c + 0] = r[c].x;
                w[4 * c + 1] = r[c].y;
                w[4 * c + 2] = r[c].z;
                w[4 * c + 3] = r[c].w;
            }
            float accs[NP];
            if constexpr (NP > 1 && !C8) {
                float vq[NP][4];
#pragma unroll
                for (int p = 0; p < NP; ++p)
#pragma unroll
                    for (int m = 0; m < 4; ++m) vq[p][m] = sq[p * kIdxDim + 16 * m + (lane & 15)];
                score_chains<NP>(vq, w, accs, std::make_integer_sequence<int, 64>{});
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float acc;
                if constexpr (C8) {
                    // the query row from LDS (same address in every lane)
                    int dot = 0;
#pragma unroll
                    for (int c = 0; c < kIdxC8RowU4; ++c) {
                        const uint4 qv = sq8[p][c];
                        dot = __builtin_amdgcn_sdot4((int)w[4 * c + 0], (int)qv.x, dot, false);
                        dot = __builtin_amdgcn_sdot4((int)w[4 * c + 1], (int)qv.y, dot, false);
                        dot = __builtin_amdgcn_sdot4((int)w[4 * c + 2], (int)qv.z, dot, false);
                        dot = __builtin_amdgcn_sdot4((int)w[4 * c + 3], (int)qv.w, dot, false);
                    }
                    const float sq = __half2float(__ushort_as_half((uint16_t)sq8[p][4].x));
                    acc = (float)dot * __half2float(__ushort_as_half((uint16_t)scv));
                    acc = acc * sq;
                } else if constexpr (NP == 1) {
                    // one position: its 32 query words fit in scalar registers
                    acc = 0.0f;
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const uint32_t qw = qb[j];
                        acc = __builtin_fmaf(bf16_lo(qw), bf16_lo(w[j]), acc);
                        acc = __builtin_fmaf(bf16_hi(qw), bf16_hi(w[j]), acc);
                    }
                } else {
                    acc = accs[p];
                }
                acc += 0.0f;  // a zero becomes +0 (one add instead of compare and select)
                uint32_t key = score_key(acc);
                asm volatile("" : "+v"(key));  // keep the chain outside the branches below
                const uint32_t bin = key >> (32 - kHistBits);
                if (valid) {
                    if constexpr (KEEP) keyrow[(size_t)p * kcap + i] = key;
                    atomicAdd(&sh[p * kHistBins + bin], 1u);
                }
                const bool take = valid && bin >= floor_bin[p];
                const unsigned long long bal = __ballot(take);
                if (bal != 0ull) {
                    const int n = (int)__popcll(bal);
                    if (nstage[p] + n > kPreStage) flush(p);
                    if (take) {
                        const unsigned long long below = lane == 0 ? 0ull : (bal & (~0ull >> (64 - lane)));
                        stage[wave][p][nstage[p] + (int)__popcll(below)] = make_uint2(key, (uint32_t)i);
                    }
                    nstage[p] += n;
                }
            }
        };
        int64_t tile = tile0 + wave;
        if (tile < tile_end) {
            // (the first segment's first tile was requested at the start)
            if (!(first_segment && preloaded)) load_tile(ra, sa, tile);
            for (; tile < tile_end; tile += 2 * nw) {
                load_tile(rb, sb, tile + nw);
                score_tile(ra, sa, tile);
                if (tile + nw >= tile_end) break;
                load_tile(ra, sa, tile + 2 * nw);
                score_tile(rb, sb, tile + nw);
            }
        }
        // end of segment: one reservation per row for the whole block
        if (lane == 0) {
#pragma unroll
            for (int p = 0; p < NP; ++p) s_cnt[wave][p] = nstage[p];
        }
        __syncthreads();
        if (threadIdx.x < NP) {
            const int p = threadIdx.x;
            int tot = 0;
            for (int v = 0; v < nw; ++v) tot += s_cnt[v][p];
            s_base[p] = tot > 0 ? atomicAdd(&meta[row0 + p].pre_count, tot) : 0;
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            int off = s_base[p];
            for (int v = 0; v < wave; ++v) off += s_cnt[v][p];
            uint2* __restrict__ dst = pre + (row0 + p) * (size_t)cap + off;
            for (int e = lane; e < nstage[p]; e += 64) dst[e] = with_residency(stage[wave][p][e], cs);
        }
        for (int i = threadIdx.x; i < NP * kHistBins / 2; i += blockDim.x) {
            uint2* const pair = reinterpret_cast<uint2*>(sh) + i;
            const uint2 v = *pair;
            if ((v.x | v.y) == 0u) continue;
            *pair = make_uint2(0u, 0u);
            // bins 2m and 2m+1 are adjacent 32-bit counters: one 64-bit
            // atomic adds both (a row holds fewer than 2^31 tokens, so the
            // low counter never carries into the high one)
            const int p = (2 * i) / kHistBins;
            const int bin = 2 * i - p * kHistBins;
            uint32_t* h = hist + (row0 + p) * kHistBins;
            atomicAdd(reinterpret_cast<unsigned long long*>(h + bin),
                      (unsigned long long)v.x | ((unsigned long long)v.y << 32));
        }
        __syncthreads();
    }
}

namespace {
template <int NP, bool C8>
int score_blocks_per_cu() {
    static const int n = [] {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void*>(&k_score_hist<NP, false, C8>),
                                                         score_threads<NP>(), 0) != hipSuccess ||
            v < 1)
            v = 1;
        return v;
    }();
    return n;
}
}  // namespace

hipError_t launch_score_hist(hipStream_t st, const void* idx_layer, const uint16_t* q_idx,
                             const int32_t* ntok_layer, uint32_t* keys, uint32_t* hist,
                             const int32_t* floor_layer, uint2* pre, RowMeta* meta,
                             const int32_t* cache_slots_layer, int B, int D, int64_t kcap, int64_t cap,
                             int64_t ntiles, int64_t max_tokens_now, int cu_count,
                             const uint16_t* scales_layer, uint32_t* qc8, const ScoreAppend& app, int xc) {
    const int64_t tiles_now = std::max<int64_t>(1, (max_tokens_now + kIdxTile - 1) / kIdxTile);
    const int64_t total = (int64_t)B * tiles_now;
    const uint4* kb = reinterpret_cast<const uint4*>(idx_layer);
    const uint32_t* q = reinterpret_cast<const uint32_t*>(q_idx);
    for (int p0 = 0; p0 < D; p0 += 4) {
        const int np = std::min(4, D - p0);
        const int per_cu = scales_layer
                               ? (np == 1 ? score_blocks_per_cu<1, true>() : np == 2 ? score_blocks_per_cu<2, true>()
                                  : np == 3 ? score_blocks_per_cu<3, true>() : score_blocks_per_cu<4, true>())
                               : (np == 1 ? score_blocks_per_cu<1, false>() : np == 2 ? score_blocks_per_cu<2, false>()
                                  : np == 3 ? score_blocks_per_cu<3, false>() : score_blocks_per_cu<4, false>());
        const int nw = (np == 1 ? score_threads<1>() : score_threads<4>()) / 64;
        // one resident round of blocks (on the CUs the launch may use), at
        // least one tile per wave
        const int64_t cus = xc < 0 ? cu_count : (int64_t)cu_count * (kXcds - 1) / kXcds;
        int64_t nb = std::min<int64_t>(cus * per_cu, (total + nw - 1) / nw);
        nb = std::max<int64_t>(nb, 1);
        const dim3 grid(split_grid(nb, xc));
        // every launch scores the appended token; the first one writes it
        ScoreAppend ap = app;
        ap.write = (app.idx != nullptr && p0 == 0) ? 1 : 0;
#define SKO_SCORE_LAUNCH1(N, K, C)                                                                         \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_score_hist<N, K, C>), grid, dim3(score_threads<N>()), 0, st, kb, q,      \
                       ntok_layer, keys, hist, floor_layer, pre, meta, cache_slots_layer, D, p0, kcap, cap, ntiles, \
                       tiles_now, total, scales_layer, qc8, ap, (int)nb, xc)
#define SKO_SCORE_LAUNCH(N)                                   \
    do {                                                      \
        if (scales_layer) {                                   \
            if (keys) SKO_SCORE_LAUNCH1(N, true, true);       \
            else SKO_SCORE_LAUNCH1(N, false, true);           \
        } else {                                              \
            if (keys) SKO_SCORE_LAUNCH1(N, true, false);      \
            else SKO_SCORE_LAUNCH1(N, false, false);          \
        }                                                     \
    } while (0)
        switch (np) {
            case 1: SKO_SCORE_LAUNCH(1); break;
            case 2: SKO_SCORE_LAUNCH(2); break;
            case 3: SKO_SCORE_LAUNCH(3); break;
            default: SKO_SCORE_LAUNCH(4); break;
        }
#undef SKO_SCORE_LAUNCH
#undef SKO_SCORE_LAUNCH1
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------- filter

__device__ __forceinline__ uint32_t pack_winner(int64_t token, const int32_t* __restrict__ cs) {
    const bool miss = cs[token] == -1;
    return (uint32_t)token | (miss ? 0x80000000u : 0u);
}

// Grid (blocks per row, rows), 256 threads.  Every block with items finds
// the row's threshold bucket from the finished histogram; block 0 records it
// for the refinement and sets the row's candidate floor for the next step.
//   * At least kk candidates: the floor was at or below the threshold bucket,
//     so the candidates hold every winner.  Blocks take spans of kFilterSpanC
//     candidate entries (4 per thread, coalesced; the first span's loads are
//     issued with the histogram's).  The entries already carry the packed
//     winner value (token | miss << 31).
//   * Fewer: the threshold fell below the floor, and blocks rescan spans of
//     kFilterSpan tokens of the row, recomputing their keys.
// In both, a key above the bucket (or in it, when the bucket is taken
// whole) is a winner: written packed to topk and marked in the sequence's
// winner bitmap (and, if absent from the hot buffer, in the miss bitmap when
// one is given); a key in a split bucket is staged (packed) in cand.  Each
// pass makes one reservation per list for the block.
constexpr int kFilterSpanC = 256 * 4;

__global__ __launch_bounds__(256) void k_topk_filter(
    const uint32_t* __restrict__ hist, RowMeta* __restrict__ meta, const uint2* __restrict__ pre,
    uint2* __restrict__ cand, int32_t* __restrict__ topk, const int32_t* __restrict__ cache_slots_layer,
    const int32_t* __restrict__ ntok_layer, uint32_t* __restrict__ winners, uint32_t* __restrict__ miss_bits,
    const uint4* __restrict__ idx_layer, const uint32_t* __restrict__ q_idx, int32_t* __restrict__ floor_layer,
    int rescan_all, int D, int64_t cap, int64_t ntiles, int64_t wpr, int top_k,
    const uint16_t* __restrict__ scales_layer, const uint32_t* __restrict__ qc8, int per_row, int nwork, int xc) {
    __shared__ int scratch[8];
    __shared__ int s_bw, s_bs, s_floor;
    __shared__ RowMeta s_res;
    // work block wk: block bx of row `row` (per_row blocks per row)
    const int wk = split_block(blockIdx.x, xc);
    if (wk < 0 || wk >= nwork) return;  // block-uniform
    const int row = wk / per_row;
    const int bx = wk - row * per_row;
    const int b = row / D;
    const int64_t Lt = ntok_layer[b];
    const int kk = (int)std::min<int64_t>(top_k, Lt);
    const int64_t npre = meta[row].pre_count;
    const uint2* __restrict__ pr = pre + (size_t)row * cap;
    // first candidate span, loaded before it is known to be needed (rows
    // hold cap entries, so clamped indexes stay in bounds)
    uint2 e0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t j = (int64_t)bx * kFilterSpanC + 256 * u + threadIdx.x;
        e0[u] = pr[j < cap ? j : cap - 1];
    }
    const bool rescan = npre < kk;
    const int64_t n_items = rescan ? Lt : npre;
    const int span = rescan ? kFilterSpan : kFilterSpanC;
    // a block without items leaves at once (block 0 stays: it records the
    // threshold and the floor)
    if (bx != 0 && (int64_t)bx * span >= n_items) return;
    threshold_row(hist + (size_t)row * kHistBins, bx == 0 ? meta + row : nullptr, kk, scratch, &s_res,
                  &s_floor);
    if (bx == 0 && threadIdx.x == 0) floor_layer[row] = rescan_all ? kFloorRescanAll : s_floor;
    const RowMeta m = s_res;
    if (m.bucket < 0) return;
    const bool take_bucket = m.need == m.bucket_count;
    const int32_t* __restrict__ cs = cache_slots_layer + (size_t)b * cap;
    uint32_t* __restrict__ wb = winners + (size_t)b * wpr;
    uint32_t* __restrict__ mb = miss_bits ? miss_bits + (size_t)b * wpr : nullptr;
    int32_t* __restrict__ w = topk + (size_t)row * top_k;
    uint2* __restrict__ cr = cand + (size_t)row * cap;
    const uint32_t* __restrict__ qrow = q_idx + (size_t)row * (kIdxDim / 2);
    for (int64_t base = (int64_t)bx * span; base < n_items; base += (int64_t)per_row * span) {
        uint32_t kv[kFilterKeysPerThread], tk[kFilterKeysPerThread];  // tk: packed winner value
        uint32_t wmask = 0, smask = 0;
        if (rescan) {
            // tokens base + 256 e + thread of the row (a wave reads whole
            // 1 KB runs of the tiled indexer), keys recomputed
            for (int e = 0; e < kFilterKeysPerThread; ++e) {
                const int64_t i = base + 256 * e + threadIdx.x;
                kv[e] = 0u;
                tk[e] = 0u;
                if (i < n_items) {
                    kv[e] = qc8 ? token_key_c8(idx_layer, scales_layer, (size_t)b * ntiles, i,
                                               qc8 + (size_t)row * kQc8Words)
                                : token_key(idx_layer, (size_t)b * ntiles, i, qrow);
                    const int bin = (int)(kv[e] >> (32 - kHistBits));
                    if (bin > m.bucket || (bin == m.bucket && take_bucket)) wmask |= 1u << e;
                    else if (bin == m.bucket) smask |= 1u << e;
                    if ((wmask | smask) >> e & 1u) tk[e] = pack_winner(i, cs);
                }
            }
        } else {
            // candidate entries base + 256 u + thread
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t j = base + 256 * u + threadIdx.x;
                uint2 v = e0[u];
                if (base != (int64_t)bx * kFilterSpanC) v = pr[j < cap ? j : cap - 1];
                kv[u] = v.x;
                tk[u] = v.y;
                if (j < n_items) {
                    const int bin = (int)(v.x >> (32 - kHistBits));
                    if (bin > m.bucket || (bin == m.bucket && take_bucket)) wmask |= 1u << u;
                    else if (bin == m.bucket) smask |= 1u << u;
                }
            }
        }
        const int nw = __popc(wmask), ns = __popc(smask);
        int total;
        const int excl = block_exclusive_scan<256>(nw | (ns << 16), &total, scratch);
        if (threadIdx.x == 0) {
            s_bw = (total & 0xFFFF) ? atomicAdd(&meta[row].out_count, total & 0xFFFF) : 0;
            s_bs = (total >> 16) ? atomicAdd(&meta[row].cand_count, total >> 16) : 0;
        }
        __syncthreads();
        int pw = s_bw + (excl & 0xFFFF);
        int ps = s_bs + (excl >> 16);
        const int ne = rescan ? kFilterKeysPerThread : 4;
        for (int e = 0; e < ne; ++e) {
            if ((wmask >> e) & 1u) {
                if (pw < top_k) w[pw] = (int32_t)tk[e];
                ++pw;
                const uint32_t tok = tk[e] & 0x7FFFFFFFu;
                atomicOr(&wb[tok >> 5], 1u << (tok & 31u));
                if (mb && (tk[e] & 0x80000000u)) atomicOr(&mb[tok >> 5], 1u << (tok & 31u));
            } else if ((smask >> e) & 1u) {
                if (ps < cap) cr[ps] = make_uint2(kv[e], tk[e]);
                ++ps;
            }
        }
        __syncthreads();  // s_bw / s_bs are reused by the next pass
    }
}

hipError_t launch_topk_filter(hipStream_t st, const uint32_t* hist, RowMeta* meta, const uint2* pre,
                              uint2* cand, int32_t* topk, const int32_t* cache_slots_layer,
                              const int32_t* ntok_layer, uint32_t* winners, uint32_t* miss_bits,
                              const void* idx_layer, const uint16_t* q_idx, int32_t* floor_layer,
                              bool rescan_all, int B, int D, int64_t cap, int64_t ntiles, int top_k,
                              int64_t max_tokens_now, const uint16_t* scales_layer, const uint32_t* qc8, int xc) {
    const int64_t wpr = winner_words(cap);
    const int64_t now = std::max<int64_t>(1, max_tokens_now);
    // blocks per row: one per kFilterSpan tokens of the longest sequence
    // (the rescan path's share), 4 to 32, and at most 1024 blocks in all:
    // most blocks of a row find no candidates and only cost their launch
    // (mtp3, 64 rows: 32 per row 18.3 us, 16 per row 12.4 us; long, 8 rows,
    // keeps 32: 16 per row took 10.9 against 8.0 us)
    const int rows = B * D;
    int per_row = (int)std::min<int64_t>(32, std::max<int64_t>(4, (now + kFilterSpan - 1) / kFilterSpan));
    per_row = std::min(per_row, std::max(4, 1024 / std::max(rows, 1)));
    // one linear grid, block bx of row r at r * per_row + bx
    const int nwork = per_row * rows;
    hipLaunchKernelGGL(k_topk_filter, dim3(split_grid(nwork, xc)), dim3(256), 0, st, hist, meta, pre, cand, topk,
                       cache_slots_layer, ntok_layer, winners, miss_bits, reinterpret_cast<const uint4*>(idx_layer),
                       reinterpret_cast<const uint32_t*>(q_idx), floor_layer, rescan_all ? 1 : 0, D, cap, ntiles,
                       wpr, top_k, scales_layer, qc8, per_row, nwork, xc);
    return hipGetLastError();
}

}  // namespace sko
