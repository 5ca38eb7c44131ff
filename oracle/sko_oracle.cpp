// CPU oracle for the per-layer sparse decode offload step.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
// benchmark's CPU-baseline leg may load this library.  It shares no code,
// header, table or constant with the HIP path under sparse_kv_offload_amd/.
//
// It is a plain, slow, single-threaded brute force of what the step computes,
// following the order of the decode-step list in "Layerwise and Sparse KV
// Cache Offloading Design" (vLLM-Ascend design doc), section 4 "Sparse Decode
// Offload", subsection "Decode step", together with the hot-shelf mechanics
// described in the FlashOffloading explainer on learnaivisually.com
// ("FlashOffloading offloads all KV cache ..."), decode paragraphs: tokens on
// the shelf are hits, misses replace evicted tokens so the shelf size never
// changes, MTP position lists are merged and deduplicated before loading, a
// reverse index (cache_slots, -1 when absent) answers hit-or-miss, and each
// top-k candidate carries its token index and residency in one int32.
//
// Where the pages leave a step open, the oracle takes one plain reading:
//   * score: single 64-d dot product q . k, accumulated in binary32 with
//     fused multiply-add in index order j = 0..63 starting from +0 (exact
//     bf16 products, one rounding per term); a zero result is stored as +0;
//   * candidates: every token present after this step's append;
//   * top-k order: larger score first, equal scores -> smaller token index;
//     min(k, L_t) winners;
//   * packed value: bit 31 set <=> cache_slots[token] == -1 at step start,
//     bits 0..30 = token index;
//   * merged list U ascending by token index; misses M ascending;
//   * LRU: per (layer, seq) table stamped with the layer's step counter t;
//     hits are stamped t first; victims are the slots not stamped t, taken in
//     ascending (last_use, slot) order; the r-th miss takes the r-th victim;
//     an eviction is a victim whose previous owner is a token (>= 0);
//   * attention: K = all 576 columns of a main-KV row, V = its first 512
//     (latent) columns, softmax(scale * q.K) over the selected rows, in
//     float64 from the bf16 values.
//
// The int8 indexer (LIM C8 in the Chinese revision of the same page,
// section 4, fused LIM / Copy-SFA sub-section: the indexer applies a
// Hadamard rotation to query and key, quantizes both to int8, and the
// selection takes the int8 query with fp16 dequantization scales).  The page
// fixes no more than that; the oracle takes these readings:
//   * rotation: x' = (1/8) H x with H the 64 x 64 Sylvester Hadamard matrix,
//     H[i][j] = (-1)^popcount(i & j); each x'[i] is a binary32 sum over
//     j = 0..63 in order from +0 of the exact terms +-x_j, then times 1/8;
//   * quantization of one row: a = max |x'[i]|; a = 0 gives codes 0 and
//     scale 0; else s = a / 127 (binary32), code[i] = round-half-even of
//     x'[i] / s (binary32 division) clamped to [-127, 127], and the stored
//     scale is s rounded to binary16 (nearest-even);
//   * keys on append (per token row), the query per (seq, position) row;
//   * score = (float(dot) * s_k) * s_q in binary32, dot = the exact int32
//     sum of code products; a zero is stored as +0.  Everything after the
//     score (keys, top-k order, residency, LRU, attention) is unchanged.
//
// Parity status: every function below is pinned by tests/test_oracle_pins.py
// (closed forms, brute force, a hand-simulated LRU trace, an independent
// recency-list formulation and invariants).  The decode step and the
// scripted LRU entry point run one merge-and-update routine, and the whole
// step is also replayed against the pinned parts (keys from the per-row
// score, winners by a full sort, misses / victims / tables from the
// recency-list formulation).  The per-step statistics (hit rate, miss count)
// have no printed values on the pages and are pinned only by the invariants.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <utility>
#include <vector>

namespace {

constexpr int IDX_DIM = 64;
constexpr int KV_DIM = 576;
constexpr int V_DIM = 512;

// Planted-mistake switch.  Zero in every real use; the pin tests set it to
// show that each pin rejects a plausible slip in this file.
int g_mutation = 0;
enum Mutation {
    MUT_NONE = 0,
    MUT_SCORE_DROP_LAST_TERM = 1,
    MUT_TIE_LARGER_INDEX = 2,
    MUT_NO_DEDUPE = 3,
    MUT_VICTIM_SLOT_DESC = 4,
    MUT_VICTIM_IGNORE_STAMP = 5,
    MUT_SCALE_512 = 6,
    MUT_V_WRONG_SLICE = 7,
    MUT_HITS_NOT_STAMPED = 8,
    MUT_EVICT_KEEPS_OLD = 9,
    MUT_FLAG_INVERTED = 10,
    MUT_SCORE_SWAP_OPERAND = 11,
    MUT_C8_HADAMARD_SIGN = 12,     // (-1)^popcount(i | j) instead of i & j
    MUT_C8_TRUNCATE = 13,          // codes truncated toward zero
    MUT_C8_QUERY_NOT_ROTATED = 14, // keys rotated, the query not
    MUT_C8_SCALE_255 = 15,         // s = a / 255 (codes saturate)
    MUT_C8_NO_QUERY_SCALE = 16,    // score misses the factor s_q
    // slips confined to the decode step's own path (the scripted LRU entry
    // point and the pin functions stay correct)
    MUT_STEP_VICTIM_SLOT_DESC = 17, // decode step: victims in descending slot order
    MUT_STEP_MISS_DESC = 18,        // decode step: misses paired with victims in descending order
    MUT_APPEND_OFFSET = 19,         // append: indexer rows stored one place later
};

inline float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

inline uint32_t f32_bits(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

// Monotone map from binary32 (finite, non-NaN) to uint32: a < b <=> ord(a) < ord(b).
inline uint32_t ordered_key(float s) {
    uint32_t u = f32_bits(s);
    return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}

// ---- binary16 <-> binary32 (IEEE 754), written from the format definition --
// binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
inline float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const int e = (h >> 10) & 0x1F;
    const uint32_t f = h & 0x3FFu;
    float v;
    if (e == 0x1F) {
        uint32_t u = sign | 0x7F800000u | (f << 13);
        std::memcpy(&v, &u, 4);
        return v;
    }
    // normal: (1 + f / 2^10) 2^(e - 15); subnormal: (f / 2^10) 2^-14 (both exact in binary32)
    v = (e == 0) ? std::ldexp((float)f, -24) : std::ldexp((float)(f + 1024u), e - 25);
    return sign ? -v : v;
}

// Round a binary32 value to the nearest binary16 value, ties to even
// fraction; beyond the largest finite binary16 (65504) rounding gives inf.
inline uint16_t f32_to_f16(float x) {
    uint32_t u = f32_bits(x);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (std::isnan(x)) return (uint16_t)(sign | 0x7E00u);
    const double a = std::fabs((double)x);
    if (std::isinf(x)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    // candidates are multiples of the binary16 spacing at a's binade
    int e2;
    std::frexp(a, &e2);               // a = m 2^e2, m in [0.5, 1)
    int ulp_exp = std::max(e2 - 11, -24);  // spacing 2^(e2 - 11) for normals, 2^-24 subnormal
    const double ulp = std::ldexp(1.0, ulp_exp);
    const double q = a / ulp;          // exact (power-of-two scaling)
    double r = std::floor(q);
    const double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && std::fmod(r, 2.0) != 0.0)) r += 1.0;
    const double v = r * ulp;          // the rounded magnitude
    if (v > 65504.0) return (uint16_t)(sign | 0x7C00u);
    // encode v
    if (v < std::ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(v / std::ldexp(1.0, -24)));
    int ev;
    const double m = std::frexp(v, &ev);  // v = m 2^ev, m in [0.5, 1)
    const int E = ev - 1 + 15;
    const uint32_t frac10 = (uint32_t)((m * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)frac10);
}

// ---- the int8 indexer (readings in the header) -----------------------------
inline int hadamard_sign(int i, int j) {
    const int m = (g_mutation == MUT_C8_HADAMARD_SIGN) ? (i | j) : (i & j);
    return (__builtin_popcount((unsigned)m) & 1) ? -1 : 1;
}

// x' = (1/8) H x, each x'[i] a binary32 sum over j in index order from +0.
void hadamard_rotate(const uint16_t* x, float* out) {
    for (int i = 0; i < IDX_DIM; ++i) {
        float acc = 0.0f;
        for (int j = 0; j < IDX_DIM; ++j) {
            const float term = bf16_to_f32(x[j]);
            acc = hadamard_sign(i, j) > 0 ? acc + term : acc - term;
        }
        out[i] = acc * 0.125f;
    }
}

// Symmetric per-row int8 quantization with an fp16 dequantization scale.
void quantize_row(const float* xr, int8_t* codes, uint16_t* scale16) {
    float a = 0.0f;
    for (int i = 0; i < IDX_DIM; ++i) a = std::max(a, std::fabs(xr[i]));
    if (a == 0.0f) {
        for (int i = 0; i < IDX_DIM; ++i) codes[i] = 0;
        *scale16 = 0;
        return;
    }
    const float s = a / ((g_mutation == MUT_C8_SCALE_255) ? 255.0f : 127.0f);
    for (int i = 0; i < IDX_DIM; ++i) {
        const float q = xr[i] / s;
        float r = (g_mutation == MUT_C8_TRUNCATE) ? std::trunc(q) : std::nearbyint(q);
        r = std::min(127.0f, std::max(-127.0f, r));
        codes[i] = (int8_t)r;
    }
    *scale16 = f32_to_f16(s);
}

// Rotation then quantization of one bf16 row (a key on append, a query).
void quantize_index_row(const uint16_t* x, int8_t* codes, uint16_t* scale16, bool rotate) {
    float xr[IDX_DIM];
    if (rotate) {
        hadamard_rotate(x, xr);
    } else {
        for (int i = 0; i < IDX_DIM; ++i) xr[i] = bf16_to_f32(x[i]);
    }
    quantize_row(xr, codes, scale16);
}

float c8_score(const int8_t* q8, uint16_t sq, const int8_t* k8, uint16_t sk) {
    int32_t dot = 0;
    for (int j = 0; j < IDX_DIM; ++j) dot += (int32_t)q8[j] * (int32_t)k8[j];
    float r = (float)dot * f16_to_f32(sk);
    if (g_mutation != MUT_C8_NO_QUERY_SCALE) r = r * f16_to_f32(sq);
    if (r == 0.0f) r = 0.0f;  // store a zero as +0
    return r;
}

struct Chain {
    int64_t ntok = 0;
    std::vector<int8_t> kidx8;       // [cap][64]  int8 indexer cache (C8 mode)
    std::vector<uint16_t> kscale;    // [cap]      its fp16 scales
    std::vector<uint16_t> kidx;      // [cap][64]  device indexer cache contents
    std::vector<uint16_t> pool;      // [cap][576] host main-KV pool
    std::vector<int32_t> cache_slots;  // [cap] token -> hot slot, -1 when absent
    std::vector<int32_t> slot_token;   // [S] hot slot -> token, -1 when empty
    std::vector<int32_t> last_use;     // [S] step stamp, -1 = never used
    std::vector<uint16_t> hot;       // [S][576] hot buffer contents
};

struct Oracle {
    int L, B, k, S, D, H;
    bool c8 = false;
    int64_t cap;
    float scale;
    std::vector<Chain> chains;       // [L][B]
    std::vector<int64_t> layer_step; // t per layer
    Chain& at(int l, int b) { return chains[(size_t)l * B + b]; }
};

// ---- step 3 of the decode-step list: the indexer scores every token --------
// s_i = sum_j q_j * K_i[j], binary32 FMA chain in index order from +0.
float indexer_score(const uint16_t* q, const uint16_t* krow) {
    float acc = 0.0f;
    int n = (g_mutation == MUT_SCORE_DROP_LAST_TERM) ? IDX_DIM - 1 : IDX_DIM;
    for (int j = 0; j < n; ++j) {
        float a = bf16_to_f32(q[j]);
        float b = bf16_to_f32(krow[(g_mutation == MUT_SCORE_SWAP_OPERAND) ? (IDX_DIM - 1 - j) : j]);
        acc = std::fma(a, b, acc);
    }
    if (acc == 0.0f) acc = 0.0f;  // store a zero as +0
    return acc;
}

// Top-k over (score desc, index asc); returns min(k, n) token indices.
std::vector<int32_t> topk_indices(const std::vector<float>& s, int k) {
    std::vector<int32_t> idx(s.size());
    for (size_t i = 0; i < s.size(); ++i) idx[i] = (int32_t)i;
    auto better = [&](int32_t a, int32_t b) {
        uint32_t ka = ordered_key(s[a]), kb = ordered_key(s[b]);
        if (ka != kb) return ka > kb;
        return (g_mutation == MUT_TIE_LARGER_INDEX) ? a > b : a < b;
    };
    std::sort(idx.begin(), idx.end(), better);
    idx.resize(std::min<size_t>((size_t)k, idx.size()));
    return idx;
}

// Packed int32 candidate: token index with the residency read from cache_slots.
inline int32_t pack_candidate(int32_t token, const int32_t* cache_slots) {
    bool miss = cache_slots[token] == -1;
    if (g_mutation == MUT_FLAG_INVERTED) miss = !miss;
    return (int32_t)((uint32_t)token | (miss ? 0x80000000u : 0u));
}

// What one residency update did to one (layer, seq) table.
struct LruStep {
    int32_t n_union = 0, n_hits = 0;
    std::vector<int32_t> misses, victims, evict_old;  // r-th miss -> r-th victim, its old owner
};

// Merge the position lists and update the residency table: the one routine
// behind both the decode step and the scripted LRU entry point.
//   packed: every position's winners, concatenated, each carrying its
//           residency flag (bit 31 = absent at step start).
// U = the distinct tokens, ascending; H = those flagged resident, M = those
// flagged absent (both ascending).  Hits are stamped t; the victims are the
// slots whose stamp is below t in ascending (last_use, slot) order; the r-th
// miss takes the r-th victim and evicts its previous owner.
// Returns 0, -5 when the slots run out (impossible when S >= D k), or -7 when
// a flag disagrees with the table.
int merge_and_update(int32_t* cache_slots, int32_t* slot_token, int32_t* last_use, int S, int32_t t,
                     std::vector<int32_t> U, bool from_step, LruStep& out) {
    std::sort(U.begin(), U.end(), [](int32_t a, int32_t x) { return (a & 0x7FFFFFFF) < (x & 0x7FFFFFFF); });
    if (g_mutation != MUT_NO_DEDUPE)
        U.erase(std::unique(U.begin(), U.end(), [](int32_t a, int32_t x) {
                    return (a & 0x7FFFFFFF) == (x & 0x7FFFFFFF);
                }), U.end());
    std::vector<int32_t> Hs, Ms;
    for (int32_t v : U) {
        const int32_t tok = v & 0x7FFFFFFF;
        if ((v < 0) != (cache_slots[tok] == -1)) return -7;
        (v < 0 ? Ms : Hs).push_back(tok);
    }
    if (from_step && g_mutation == MUT_STEP_MISS_DESC) std::reverse(Ms.begin(), Ms.end());
    if (g_mutation != MUT_HITS_NOT_STAMPED)
        for (int32_t tok : Hs) last_use[cache_slots[tok]] = t;
    std::vector<std::pair<int32_t, int32_t>> order;  // (last_use, slot)
    for (int s = 0; s < S; ++s)
        if (last_use[s] < t) order.push_back({last_use[s], s});
    if (g_mutation == MUT_VICTIM_SLOT_DESC || (from_step && g_mutation == MUT_STEP_VICTIM_SLOT_DESC))
        std::sort(order.begin(), order.end(), [](auto a, auto x) {
            return a.first != x.first ? a.first < x.first : a.second > x.second;
        });
    else if (g_mutation == MUT_VICTIM_IGNORE_STAMP)
        std::sort(order.begin(), order.end(), [](auto a, auto x) { return a.second < x.second; });
    else
        std::sort(order.begin(), order.end());
    if (Ms.size() > order.size()) return -5;
    for (size_t r = 0; r < Ms.size(); ++r) {
        const int32_t v = order[r].second, m = Ms[r], old = slot_token[v];
        if (old >= 0 && g_mutation != MUT_EVICT_KEEPS_OLD) cache_slots[old] = -1;
        cache_slots[m] = v;
        slot_token[v] = m;
        last_use[v] = t;
        out.misses.push_back(m);
        out.victims.push_back(v);
        out.evict_old.push_back(old);
    }
    out.n_union = (int32_t)U.size();
    out.n_hits = (int32_t)Hs.size();
    return 0;
}

// Step 7: softmax attention over the selected rows (fp64).
void sparse_attention(const Oracle& o, const uint16_t* qa /*[H][576]*/,
                      const std::vector<const uint16_t*>& rows, double* out /*[H][512]*/) {
    const int n = (int)rows.size();
    double scale = (g_mutation == MUT_SCALE_512) ? 1.0 / std::sqrt(512.0) : (double)o.scale;
    int voff = (g_mutation == MUT_V_WRONG_SLICE) ? KV_DIM - V_DIM : 0;
    std::vector<double> z(n), w(n);
    for (int h = 0; h < o.H; ++h) {
        const uint16_t* q = qa + (size_t)h * KV_DIM;
        double* oh = out + (size_t)h * V_DIM;
        for (int c = 0; c < V_DIM; ++c) oh[c] = 0.0;
        if (n == 0) continue;
        double m = -INFINITY;
        for (int j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int c = 0; c < KV_DIM; ++c) acc += (double)bf16_to_f32(q[c]) * (double)bf16_to_f32(rows[j][c]);
            z[j] = scale * acc;
            m = std::max(m, z[j]);
        }
        double l = 0.0;
        for (int j = 0; j < n; ++j) { w[j] = std::exp(z[j] - m); l += w[j]; }
        for (int j = 0; j < n; ++j) {
            double p = w[j] / l;
            for (int c = 0; c < V_DIM; ++c) oh[c] += p * (double)bf16_to_f32(rows[j][voff + c]);
        }
    }
}

}  // namespace

extern "C" {

void oracle_set_mutation(int m) { g_mutation = m; }

void* oracle_create(int L, int B, int64_t cap, int k, int S, int D, int H, float scale) {
    if (L < 1 || B < 1 || cap < 1 || k < 1 || D < 1 || H < 1 || S < (int64_t)D * k) return nullptr;
    Oracle* o = new Oracle();
    o->L = L; o->B = B; o->cap = cap; o->k = k; o->S = S; o->D = D; o->H = H; o->scale = scale;
    o->chains.resize((size_t)L * B);
    for (auto& c : o->chains) {
        c.kidx.assign((size_t)cap * IDX_DIM, 0);
        c.pool.assign((size_t)cap * KV_DIM, 0);
        c.cache_slots.assign((size_t)cap, -1);
        c.slot_token.assign((size_t)S, -1);
        c.last_use.assign((size_t)S, -1);
        c.hot.assign((size_t)S * KV_DIM, 0);
    }
    o->layer_step.assign((size_t)L, 0);
    return o;
}

void oracle_destroy(void* h) { delete static_cast<Oracle*>(h); }

// Switch a fresh oracle (nothing appended yet) to the int8 indexer.
int oracle_set_indexer_c8(void* h, int on) {
    Oracle* o = static_cast<Oracle*>(h);
    for (const Chain& c : o->chains)
        if (c.ntok != 0) return -1;
    o->c8 = on != 0;
    return 0;
}

// Steps 1-2: the new token's rows go to their logical slots: the main-KV row
// to the host pool, the indexer row to the indexer cache.
int oracle_append(void* h, int layer, int seq, const uint16_t* idx_rows, const uint16_t* kv_rows, int64_t n) {
    Oracle* o = static_cast<Oracle*>(h);
    if (layer < 0 || layer >= o->L || seq < 0 || seq >= o->B || n < 0) return -1;
    Chain& c = o->at(layer, seq);
    if (c.ntok + n > o->cap) return -4;
    if (g_mutation == MUT_APPEND_OFFSET) {
        for (int64_t r = 0; r < n; ++r)
            if (c.ntok + r + 1 < o->cap)
                std::memcpy(&c.kidx[(size_t)(c.ntok + r + 1) * IDX_DIM], idx_rows + (size_t)r * IDX_DIM,
                            IDX_DIM * 2);
    } else {
        std::memcpy(&c.kidx[(size_t)c.ntok * IDX_DIM], idx_rows, (size_t)n * IDX_DIM * 2);
    }
    if (o->c8) {
        if (c.kidx8.empty()) {
            c.kidx8.assign((size_t)o->cap * IDX_DIM, 0);
            c.kscale.assign((size_t)o->cap, 0);
        }
        for (int64_t r = 0; r < n; ++r)
            quantize_index_row(idx_rows + (size_t)r * IDX_DIM, &c.kidx8[(size_t)(c.ntok + r) * IDX_DIM],
                               &c.kscale[(size_t)(c.ntok + r)], true);
    }
    std::memcpy(&c.pool[(size_t)c.ntok * KV_DIM], kv_rows, (size_t)n * KV_DIM * 2);
    c.ntok += n;
    return 0;
}

// One decode step of one layer for all sequences.
//   q_idx  [B][D][64]     bf16 indexer queries
//   q_attn [B][D][H][576] bf16 attention queries
int oracle_decode_step(void* h, int layer, const uint16_t* q_idx, const uint16_t* q_attn,
                       int32_t* topk, int32_t* phys, uint32_t* keys, int32_t* counts,
                       int32_t* misses, int32_t* victims, int32_t* evict_old,
                       double* out, double* out_pool) {
    Oracle* o = static_cast<Oracle*>(h);
    if (layer < 0 || layer >= o->L) return -1;
    const int B = o->B, D = o->D, k = o->k, S = o->S, H = o->H;
    const int32_t t = (int32_t)o->layer_step[layer];
    for (int b = 0; b < B; ++b) {
        Chain& c = o->at(layer, b);
        const int64_t Lt = c.ntok;
        const int kk = (int)std::min<int64_t>(k, Lt);

        // Step 3: score all tokens and select the top-k per position.  The
        // residency of every winner is packed in with it, read from the
        // reverse index as it stands before this step's LRU update.
        std::vector<std::vector<int32_t>> W(D);
        for (int p = 0; p < D; ++p) {
            const uint16_t* q = q_idx + ((size_t)b * D + p) * IDX_DIM;
            std::vector<float> s((size_t)Lt);
            if (o->c8) {
                int8_t q8[IDX_DIM];
                uint16_t sq;
                quantize_index_row(q, q8, &sq, g_mutation != MUT_C8_QUERY_NOT_ROTATED);
                for (int64_t i = 0; i < Lt; ++i)
                    s[i] = c8_score(q8, sq, &c.kidx8[(size_t)i * IDX_DIM], c.kscale[(size_t)i]);
            } else {
                for (int64_t i = 0; i < Lt; ++i) s[i] = indexer_score(q, &c.kidx[(size_t)i * IDX_DIM]);
            }
            if (keys)
                for (int64_t i = 0; i < Lt; ++i) keys[((size_t)b * D + p) * o->cap + i] = ordered_key(s[i]);
            std::vector<int32_t> sel = topk_indices(s, k);
            for (int32_t tok : sel) W[p].push_back(pack_candidate(tok, c.cache_slots.data()));
            if (topk) {
                int32_t* dst = topk + ((size_t)b * D + p) * k;
                for (int j = 0; j < k; ++j) dst[j] = j < kk ? W[p][j] : 0;
            }
        }

        // Merge the D position lists, deduplicate and update the residency
        // table (the one routine the scripted LRU entry point also runs);
        // then step 5: copy only the missed rows, host pool -> hot buffer.
        std::vector<int32_t> U;
        for (int p = 0; p < D; ++p)
            for (int32_t v : W[p]) U.push_back(v);
        LruStep st;
        const int rc = merge_and_update(c.cache_slots.data(), c.slot_token.data(), c.last_use.data(),
                                        S, t, U, true, st);
        if (rc < 0) return rc;
        const int nM = (int)st.misses.size();
        int nEv = 0;
        for (int r = 0; r < nM; ++r) {
            const int32_t v = st.victims[r], m = st.misses[r];
            if (st.evict_old[r] >= 0) ++nEv;
            std::memcpy(&c.hot[(size_t)v * KV_DIM], &c.pool[(size_t)m * KV_DIM], KV_DIM * 2);
            if (misses) misses[(size_t)b * D * k + r] = m;
            if (victims) victims[(size_t)b * D * k + r] = v;
            if (evict_old) evict_old[(size_t)b * D * k + r] = st.evict_old[r];
        }
        if (counts) {
            int32_t* cn = counts + (size_t)b * 8;
            cn[0] = st.n_union; cn[1] = st.n_hits; cn[2] = nM; cn[3] = nEv;
            cn[4] = kk; cn[5] = (int32_t)Lt; cn[6] = t; cn[7] = 0;
        }

        // Step 6: remap each position's logical winners to physical slots;
        // step 7: attention over those hot-buffer rows.  The same attention
        // over the pool rows is computed alongside: offload moves data, it
        // must not change the result.
        for (int p = 0; p < D; ++p) {
            std::vector<const uint16_t*> hot_rows, pool_rows;
            for (int j = 0; j < kk; ++j) {
                int32_t tok = W[p][j] & 0x7FFFFFFF;
                int32_t slot = c.cache_slots[tok];
                if (phys) phys[((size_t)b * D + p) * k + j] = slot;
                if (slot < 0) return -6;  // a winner must be resident after the update
                hot_rows.push_back(&c.hot[(size_t)slot * KV_DIM]);
                pool_rows.push_back(&c.pool[(size_t)tok * KV_DIM]);
            }
            const uint16_t* qa = q_attn + ((size_t)b * D + p) * H * KV_DIM;
            if (out) sparse_attention(*o, qa, hot_rows, out + ((size_t)b * D + p) * H * V_DIM);
            if (out_pool) sparse_attention(*o, qa, pool_rows, out_pool + ((size_t)b * D + p) * H * V_DIM);
        }
    }
    o->layer_step[layer] += 1;
    return 0;
}

// Table readers (copies of one (layer, seq) chain's state).
int oracle_read_state(void* h, int layer, int seq, int32_t* cache_slots, int32_t* slot_token,
                      int32_t* last_use, uint16_t* hot, int64_t* ntok) {
    Oracle* o = static_cast<Oracle*>(h);
    if (layer < 0 || layer >= o->L || seq < 0 || seq >= o->B) return -1;
    Chain& c = o->at(layer, seq);
    if (cache_slots) std::memcpy(cache_slots, c.cache_slots.data(), c.cache_slots.size() * 4);
    if (slot_token) std::memcpy(slot_token, c.slot_token.data(), c.slot_token.size() * 4);
    if (last_use) std::memcpy(last_use, c.last_use.data(), c.last_use.size() * 4);
    if (hot) std::memcpy(hot, c.hot.data(), c.hot.size() * 2);
    if (ntok) *ntok = c.ntok;
    return 0;
}

// The int8 indexer rows of one (layer, seq) chain: codes [cap][64], scales [cap].
int oracle_read_indexer_c8(void* h, int layer, int seq, int8_t* codes, uint16_t* scales) {
    Oracle* o = static_cast<Oracle*>(h);
    if (layer < 0 || layer >= o->L || seq < 0 || seq >= o->B || !o->c8) return -1;
    Chain& c = o->at(layer, seq);
    if (c.kidx8.empty()) {
        std::memset(codes, 0, (size_t)o->cap * IDX_DIM);
        std::memset(scales, 0, (size_t)o->cap * 2);
        return 0;
    }
    std::memcpy(codes, c.kidx8.data(), c.kidx8.size());
    std::memcpy(scales, c.kscale.data(), c.kscale.size() * 2);
    return 0;
}

void oracle_hadamard_rotate(const uint16_t* x, float* out) { hadamard_rotate(x, out); }

void oracle_quantize_row(const float* xr, int8_t* codes, uint16_t* scale16) { quantize_row(xr, codes, scale16); }

float oracle_c8_score(const int8_t* q8, uint16_t sq, const int8_t* k8, uint16_t sk) {
    return c8_score(q8, sq, k8, sk);
}

uint16_t oracle_f32_to_f16(float x) { return f32_to_f16(x); }

float oracle_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

// Direct access to one function at a time, for the pin tests.
float oracle_score_one(const uint16_t* q, const uint16_t* krow) { return indexer_score(q, krow); }

uint32_t oracle_ordered_key(float s) { return ordered_key(s); }

// Top-k of n given scores; writes min(k, n) indices.
int oracle_topk(const float* s, int64_t n, int k, int32_t* out_idx) {
    std::vector<float> v(s, s + n);
    std::vector<int32_t> sel = topk_indices(v, k);
    for (size_t i = 0; i < sel.size(); ++i) out_idx[i] = sel[i];
    return (int)sel.size();
}

// LRU unit driven by scripted selections.  State arrays are caller-owned.
//   sel: n packed winners (already carrying flags is not required: the
//   flags are recomputed from cache_slots here), returns nM and fills the
//   miss / victim / old-owner lists.
int oracle_lru_apply(int32_t* cache_slots, int64_t cap, int32_t* slot_token, int32_t* last_use,
                     int S, int32_t t, const int32_t* sel, int n,
                     int32_t* misses, int32_t* victims, int32_t* evict_old, int32_t* n_hits) {
    std::vector<int32_t> packed;
    for (int i = 0; i < n; ++i) {
        const int32_t tok = sel[i] & 0x7FFFFFFF;
        if (tok >= cap) return -1;
        packed.push_back(pack_candidate(tok, cache_slots));
    }
    LruStep st;
    const int rc = merge_and_update(cache_slots, slot_token, last_use, S, t, packed, false, st);
    if (rc < 0) return rc;
    for (size_t r = 0; r < st.misses.size(); ++r) {
        misses[r] = st.misses[r];
        victims[r] = st.victims[r];
        evict_old[r] = st.evict_old[r];
    }
    if (n_hits) *n_hits = st.n_hits;
    return (int)st.misses.size();
}

// Attention over explicit rows (for the closed-form pins).
void oracle_attention(const uint16_t* qa, int H, const uint16_t* rows, int n, float scale, double* out) {
    Oracle o;
    o.H = H;
    o.scale = scale;
    std::vector<const uint16_t*> r;
    for (int j = 0; j < n; ++j) r.push_back(rows + (size_t)j * KV_DIM);
    sparse_attention(o, qa, r, out);
}

}  // extern "C"
