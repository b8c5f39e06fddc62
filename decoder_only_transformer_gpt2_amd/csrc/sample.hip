// Sampled next-token choice over a [B, V] block of fp32 logits: repetition penalty, temperature,
// top-k, top-p and a multinomial draw by inverse CDF ("GPT2模型开发实战：从原理到部署全解析" §8.2
// lists the four knobs; "GPT-2模型架构解析与实现指南" §4.1 draws from softmax(logits / temperature)).
//
// One 1024-thread workgroup per row. Wave w owns the vocabulary span [w*64*NPT, (w+1)*64*NPT) with
// NPT = ceil(V / 1024) rounded up to a multiple of 8 (a template constant, so the per-thread slots
// stay in registers without per-slot guards); lane l holds the order keys of the penalised logits
// of tokens w*64*NPT + i*64 + l, so every load is a coalesced 256-byte wave access and the row is
// read from HBM once. Dividing by the temperature preserves order, so both cut-offs compare the
// penalised logits x themselves and the temperature only enters the weights exp((x - max) / T).
//
// Both cut-offs are thresholds on the order key:
//   top-k keeps key >= kappa, kappa the k-th largest key;
//   top-p keeps key >= tau, tau the smallest key whose strictly-larger kept mass is below p.
// A full pass over the row costs the one CU that owns it a few microseconds of VALU time, so the
// search narrows the candidates first and finishes on a short list:
//   * top-k (the usual case, k <= 64 * the fully populated waves): each such wave takes the q-th
//     largest of its 64 lane maxima, q = ceil(k / waves), by a 32-step ballot search; their minimum
//     is a lower bound of kappa (that many distinct tokens reach it). The tokens at or above it,
//     a few hundred, are copied to LDS with their ids, and wave 0 alone finishes: kappa by a
//     bitwise search on ballot counts, tau by a bitwise search on the kept mass (DPP wave sums),
//     and the draw by a bitwise search over token ids, with no further block barrier;
//   * otherwise a 2048-bin histogram over the distance from the row maximum picks the bin holding
//     the threshold, that bin's tokens are copied to LDS, and four 8-bit radix passes over their
//     keys fix it; the draw then walks the kept mass wave by wave in vocabulary order.
// Softmax weights are 2^-31 fixed point (u32, the largest token weighs 2^31) summed in u64, so every
// sum is exact and no result depends on the order in which lanes add.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int ST = 1024;                // threads per row
constexpr int SWAVES = ST / GPT2_WAVE;  // 16
constexpr int SNPT = 64;                // values per thread: V <= ST * SNPT
constexpr int NCOARSE = 2048;
constexpr int LCAP = 4096;              // candidate list capacity
constexpr float kFix = 2147483648.0f;   // 2^31

struct SampleSmem {
    uint32_t pen[ST * SNPT / 32];     // history membership bits
    uint32_t cnt[NCOARSE];            // histogram counts (radix passes use the first 256)
    uint64_t mass[NCOARSE];           // histogram masses
    uint32_t draw[GPT2_WAVE * SNPT];  // one wave's weights in vocabulary order
    uint32_t list[LCAP];              // candidate keys
    uint32_t list_tok[LCAP];          // their token ids (top-k lists)
    uint64_t wm[SWAVES];
    uint32_t wc[SWAVES];
    uint32_t wk[SWAVES];
    uint32_t lbw[SWAVES];             // per-wave lower bounds of kappa
    int list_n;
    int sel_bin;
    uint32_t sel_c;
    uint64_t sel_m;
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
    const uint32_t lo = __shfl_up((uint32_t)v, d), hi = __shfl_up((uint32_t)(v >> 32), d);
    return ((uint64_t)hi << 32) | lo;
}

__device__ uint64_t block_sum_u64(uint64_t v, SampleSmem& sm) {
    for (int o = 32; o; o >>= 1) v += shfl_xor_u64(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.wm[threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t t = 0;
    for (int i = 0; i < SWAVES; ++i) t += sm.wm[i];
    return t;
}
__device__ uint32_t block_sum_u32(uint32_t v, SampleSmem& sm) {
    for (int o = 32; o; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.wc[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = 0;
    for (int i = 0; i < SWAVES; ++i) t += sm.wc[i];
    return t;
}
// Block maximum of a and minimum of b in one exchange.
__device__ void block_max_min_u32(uint32_t& a, uint32_t& b, SampleSmem& sm) {
    for (int o = 32; o; o >>= 1) {
        a = max(a, (uint32_t)__shfl_xor(a, o));
        b = min(b, (uint32_t)__shfl_xor(b, o));
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        sm.wk[threadIdx.x >> 6] = a;
        sm.wc[threadIdx.x >> 6] = b;
    }
    __syncthreads();
    a = sm.wk[0];
    b = sm.wc[0];
    for (int i = 1; i < SWAVES; ++i) {
        a = max(a, sm.wk[i]);
        b = min(b, sm.wc[i]);
    }
}

// Coarse bin of a value: 0 at the row maximum m, growing with the distance below it (monotone:
// a larger value never lands in a larger bin; equal values share a bin). -inf and NaN go last.
__device__ __forceinline__ int coarse_bin(float x, float m, float scale) {
    const float t = (m - x) * scale;
    return t < (float)NCOARSE ? (int)fmaxf(t, 0.f) : NCOARSE - 1;
}

// A copy of v the compiler cannot see through: values derived from it are recomputed where they are
// used instead of being hoisted out of the passes and kept live for every slot.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// exp((x - m) / T) in 2^-31 fixed point, c = log2(e) / T; x <= m, so the result is at most 2^31.
__device__ __forceinline__ uint32_t fixed_weight(float x, float m, float c) {
    return (uint32_t)(__builtin_amdgcn_exp2f((x - m) * c) * kFix);
}
__device__ __forceinline__ uint32_t key_weight(uint32_t key, float m, float c) {
    return fixed_weight(f32_from_order_key(key), m, c);
}

// Histogram bins [0, nb) are ordered by decreasing value. COUNT mode (top-k): returns the bin b
// whose count range holds the rem-th largest element and lowers rem by the count before b. MASS
// mode (top-p): returns the last non-empty bin b whose mass before it, plus above, is below P, and
// adds that mass to above. Every thread of the block calls it and gets the same result (-1 when no
// bin qualifies, which the callers' invariants rule out).
template <bool MASS>
__device__ int select_bin(int nb, uint32_t& rem, uint64_t& above, uint64_t P, SampleSmem& sm) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int per = nb >= ST ? nb / ST : 1;  // 2 or 1 bins per thread (nb = 2048 or 256)
    const int b0 = t * per;
    uint32_t cb[2] = {0, 0};
    uint64_t mb[2] = {0, 0};
    uint32_t c = 0;
    uint64_t m = 0;
    for (int j = 0; j < 2; ++j)
        if (j < per && b0 + j < nb) {
            cb[j] = sm.cnt[b0 + j];
            if (MASS) mb[j] = sm.mass[b0 + j];
            c += cb[j];
            m += mb[j];
        }
    // block exclusive scan of (c, m)
    uint32_t ic = c;
    uint64_t im = m;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t tc = __shfl_up(ic, o);
        const uint64_t tm = MASS ? shfl_up_u64(im, o) : 0;
        if (lane >= o) {
            ic += tc;
            im += tm;
        }
    }
    if (t == 0) sm.sel_bin = -1;
    __syncthreads();
    if (lane == 63) {
        sm.wc[w] = ic;
        sm.wm[w] = im;
    }
    __syncthreads();
    uint32_t ec = ic - c;
    uint64_t em = im - m;
    for (int i = 0; i < w; ++i) {
        ec += sm.wc[i];
        if (MASS) em += sm.wm[i];
    }
    const uint32_t ec0 = ec;
    const uint64_t em0 = em;
    int cand = -1;
    for (int j = 0; j < 2; ++j)
        if (j < per && b0 + j < nb) {
            if (cb[j] > 0) {
                if (MASS) {
                    if (above + em < P) cand = b0 + j;
                } else if (ec < rem && rem <= ec + cb[j]) {
                    cand = b0 + j;
                }
            }
            ec += cb[j];
            em += mb[j];
        }
    if (cand >= 0) atomicMax(&sm.sel_bin, cand);
    __syncthreads();
    const int bin = sm.sel_bin;
    if (bin >= b0 && bin < b0 + per) {
        sm.sel_c = ec0 + (bin > b0 ? cb[0] : 0u);
        sm.sel_m = em0 + (bin > b0 ? mb[0] : 0ull);
    }
    __syncthreads();
    if (MASS)
        above += sm.sel_m;
    else
        rem -= sm.sel_c;
    return bin;
}

__device__ __forceinline__ void clear_bins(int nb, bool mass, SampleSmem& sm) {
    for (int i = threadIdx.x; i < nb; i += ST) {
        sm.cnt[i] = 0;
        if (mass) sm.mass[i] = 0;
    }
    __syncthreads();
}

// Appends the keys of the slots for which pred(key) holds to sm.list (wave-aggregated: one LDS
// atomic per wave and slot) and returns how many there were (entries past LCAP are dropped).
template <int NPT, class Pred>
__device__ int compact(const uint32_t (&key)[NPT], Pred pred, SampleSmem& sm) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) sm.list_n = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const uint32_t k = opaque(key[i]);
        const bool p = pred(k);
        const uint64_t bal = __builtin_amdgcn_ballot_w64(p);
        if (bal) {
            int at = 0;
            if (lane == 0) at = atomicAdd(&sm.list_n, (int)__popcll(bal));
            at = __builtin_amdgcn_readfirstlane(at);
            if (p) {
                const int idx = at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (idx < LCAP) sm.list[idx] = k;
            }
        }
    }
    __syncthreads();
    return sm.list_n;
}

// compact() that also records each key's token id (slot i of this thread is token base + 64 i).
template <int NPT, class Pred>
__device__ int compact_pairs(const uint32_t (&key)[NPT], int base, Pred pred, SampleSmem& sm) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) sm.list_n = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const uint32_t k = opaque(key[i]);
        const bool p = pred(k);
        const uint64_t bal = __builtin_amdgcn_ballot_w64(p);
        if (bal) {
            int at = 0;
            if (lane == 0) at = atomicAdd(&sm.list_n, (int)__popcll(bal));
            at = __builtin_amdgcn_readfirstlane(at);
            if (p) {
                const int idx = at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                if (idx < LCAP) {
                    sm.list[idx] = k;
                    sm.list_tok[idx] = (uint32_t)(base + i * GPT2_WAVE);
                }
            }
        }
    }
    __syncthreads();
    return sm.list_n;
}

// Radix passes (most significant byte first) over the candidates: the n keys of sm.list when
// IN_LIST, else the register slots that satisfy in_bin. Only keys >= lo_key take part. COUNT
// mode: the rem-th largest candidate key; MASS mode: the smallest candidate key whose strictly
// larger candidate mass plus above is below P.
template <bool MASS, bool IN_LIST, int NPT, class InBin>
__device__ uint32_t radix_threshold(const uint32_t (&key)[NPT], int n, InBin in_bin, float m, float c,
                                    uint32_t lo_key, uint32_t rem, uint64_t P, uint64_t above, SampleSmem& sm) {
    uint32_t prefix = 0;
#pragma unroll 1
    for (int r = 0; r < 4; ++r) {
        const int shift = 24 - 8 * r;
        const int hs = r == 0 ? 0 : shift + 8;
        clear_bins(256, MASS, sm);
        auto add = [&](uint32_t k) {
            if (k >= lo_key && (r == 0 || (k >> hs) == prefix)) {
                const int b = 255 - (int)((k >> shift) & 255u);
                atomicAdd(&sm.cnt[b], 1u);
                if (MASS) atomicAdd((unsigned long long*)&sm.mass[b], (unsigned long long)key_weight(k, m, c));
            }
        };
        if (IN_LIST) {
            for (int j = threadIdx.x; j < n; j += ST) add(sm.list[j]);
        } else {
#pragma unroll
            for (int i = 0; i < NPT; ++i) {
                const uint32_t k = opaque(key[i]);
                if (in_bin(k)) add(k);
            }
        }
        __syncthreads();
        const int b = select_bin<MASS>(256, rem, above, P, sm);
        prefix = (prefix << 8) | (uint32_t)(255 - b);
    }
    return prefix;
}

// Sum over the 64 lanes of a wave through DPP (row_shr 1, 2, 4, 8 inside each row of 16, then
// row_bcast 15 and 31); the total is read from lane 63 and is the same in every lane.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xF, true);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
    v += dpp_u64<0x111, 0xF>(v);  // row_shr:1
    v += dpp_u64<0x112, 0xF>(v);  // row_shr:2
    v += dpp_u64<0x114, 0xF>(v);  // row_shr:4
    v += dpp_u64<0x118, 0xF>(v);  // row_shr:8
    v += dpp_u64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_u64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Number of lanes of the wave whose x is >= c (uniform).
__device__ __forceinline__ int wave_count_ge(uint32_t x, uint32_t c) {
    return (int)__popcll(__builtin_amdgcn_ballot_w64(x >= c));
}

// Bits [0, hb] are searched, hb the highest bit where lo and hi differ; returns the common prefix
// of lo and hi above it (the search start) through start and the bit index (-1: lo == hi).
__device__ __forceinline__ int search_span(uint32_t lo, uint32_t hi, uint32_t& start) {
    const uint32_t d = lo ^ hi;
    if (d == 0) {
        start = lo;
        return -1;
    }
    const int hb = 31 - __builtin_clz(d);
    start = hi & ~(uint32_t)((2ull << hb) - 1);
    return hb;
}

// One wave finishes a top-k row from its n <= 64 * NS candidates (keys lkey, token ids ltok, in LDS
// or global memory: every token with key >= the lower bound lb; the row maximum key is kmax):
// kappa, tau, the draw.
template <int NS>
__device__ void finish_top_k(const uint32_t* lkey, const uint32_t* ltok, int n, uint32_t lb, uint32_t kmax, int top_k,
                             float top_p, float m, float c, float uu, int32_t* out, int32_t* n_kept) {
    const int lane = threadIdx.x & 63;
    uint32_t kl[NS], tk[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int j = s * GPT2_WAVE + lane;
        kl[s] = j < n ? lkey[j] : 0u;
        tk[s] = j < n ? ltok[j] : 0u;
    }
    // kappa: the largest x with count(key >= x) >= k; every candidate key lies in [lb, kmax]
    uint32_t kappa;
    int hb = search_span(lb, kmax, kappa);
#pragma unroll 1
    for (; hb >= 0; --hb) {
        const uint32_t cand = kappa | (1u << hb);
        int cnt = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) cnt += wave_count_ge(kl[s], cand);
        if (cnt >= top_k) kappa = cand;
    }
    uint32_t wl[NS];
    uint64_t part = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        wl[s] = kl[s] >= kappa ? key_weight(kl[s], m, c) : 0u;
        part += wl[s];
    }
    const uint64_t S = wave_sum_u64(part);
    uint32_t theta = kappa;
    uint64_t total = S;
    if (top_p < 1.0f) {
        uint64_t P = (uint64_t)((double)top_p * (double)S);
        if (P == 0) P = 1;
        // the largest x with mass(key > x) >= P lies in [kappa - 1, kmax]; tau is one above it
        uint32_t x;
        int b = search_span(kappa - 1, kmax, x);
#pragma unroll 1
        for (; b >= 0; --b) {
            const uint32_t cand = x | (1u << b);
            uint64_t mp = 0;
#pragma unroll
            for (int s = 0; s < NS; ++s) mp += kl[s] > cand ? wl[s] : 0u;
            if (wave_sum_u64(mp) >= P) x = cand;
        }
        theta = x + 1;
        part = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            wl[s] = kl[s] >= theta ? wl[s] : 0u;
            part += wl[s];
        }
        total = wave_sum_u64(part);
    }
    int kept = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) kept += wave_count_ge(kl[s], theta);
    // the draw: the largest y with (kept mass of tokens < y) <= U is the first token whose
    // cumulative kept mass exceeds U
    const double ud = uu >= 0.f ? (uu < 1.f ? (double)uu : 1.0) : 0.0;
    uint64_t U = (uint64_t)(ud * (double)total);
    if (total > 0 && U >= total) U = total - 1;
    uint32_t y = 0;
#pragma unroll 1
    for (int bit = 16; bit >= 0; --bit) {
        const uint32_t cand = y | (1u << bit);
        uint64_t mp = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) mp += tk[s] < cand ? wl[s] : 0u;
        if (wave_sum_u64(mp) <= U) y = cand;
    }
    if (lane == 0) {
        *out = (int32_t)y;
        if (n_kept) *n_kept = kept;
    }
}

// Threshold through the coarse histogram: pick the coarse bin holding it, then finish on that
// bin's tokens (list, or registers if the bin overflows the list).
template <bool MASS, int NPT>
__device__ uint32_t coarse_threshold(const uint32_t (&key)[NPT], float m, float c, float scale, uint32_t lo_key,
                                     uint32_t rem, uint64_t P, SampleSmem& sm) {
    uint64_t above = 0;
    clear_bins(NCOARSE, MASS, sm);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const uint32_t k = opaque(key[i]);
        if (k >= lo_key) {
            const float x = f32_from_order_key(k);
            const int b = coarse_bin(x, m, scale);
            atomicAdd(&sm.cnt[b], 1u);
            if (MASS) atomicAdd((unsigned long long*)&sm.mass[b], (unsigned long long)fixed_weight(x, m, c));
        }
    }
    __syncthreads();
    const int cb = select_bin<MASS>(NCOARSE, rem, above, P, sm);
    auto in_bin = [&](uint32_t k) { return k >= lo_key && coarse_bin(f32_from_order_key(k), m, scale) == cb; };
    const int n = compact(key, in_bin, sm);
    if (n <= LCAP) return radix_threshold<MASS, true>(key, n, in_bin, m, c, lo_key, rem, P, above, sm);
    return radix_threshold<MASS, false>(key, 0, in_bin, m, c, lo_key, rem, P, above, sm);
}

// Candidates gathered by the chunked top-k kernels (null when they did not run): per row, the count
// cnt and the keys / token ids of the tokens at or above the row's lower bound of kappa (the first
// min(cnt, lcap) of them; the row maximum is among them).
struct SampleList {
    const int32_t* cnt = nullptr;
    const uint32_t* lkey = nullptr;
    const uint32_t* ltok = nullptr;
    int lcap = 0;
};

template <int NPT>
__global__ void __launch_bounds__(ST) sample_kernel(const float* __restrict__ logits, long ld, int V,
                                                     const int32_t* __restrict__ hist, long hist_ld, int n_hist,
                                                     float temperature, int top_k, float top_p, float penalty,
                                                     const float* __restrict__ u, int32_t* __restrict__ out,
                                                     int32_t* __restrict__ n_kept, SampleList cl) {
    __shared__ SampleSmem sm;
    const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (cl.cnt != nullptr) {
        // the chunked kernels collected this row's top-k candidates: one wave finishes from them
        const int n = cl.cnt[b];
        if (n <= 8 * GPT2_WAVE) {
            if (w == 0) {
                const uint32_t* lk = cl.lkey + (long)b * cl.lcap;
                const uint32_t* lt = cl.ltok + (long)b * cl.lcap;
                uint32_t kmax = 0, lb = 0xffffffffu;  // the list holds the row maximum
                for (int i = lane; i < n; i += GPT2_WAVE) {
                    kmax = max(kmax, lk[i]);
                    lb = min(lb, lk[i]);
                }
                for (int o = 32; o; o >>= 1) {
                    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o));
                    lb = min(lb, (uint32_t)__shfl_xor(lb, o));
                }
                const float m = f32_from_order_key(kmax), c = 1.4426950408889634f / temperature;
                if (n <= 4 * GPT2_WAVE)
                    finish_top_k<4>(lk, lt, n, lb, kmax, top_k, top_p, m, c, u[b], out + b, n_kept ? n_kept + b : nullptr);
                else
                    finish_top_k<8>(lk, lt, n, lb, kmax, top_k, top_p, m, c, u[b], out + b, n_kept ? n_kept + b : nullptr);
            }
            return;
        }
    }
    const int base = w * GPT2_WAVE * NPT + lane;  // token of slot i: base + i * 64
    const float* row = logits + (long)b * ld;
    auto none = [](uint32_t) { return false; };

    const bool use_pen = hist != nullptr && n_hist > 0 && penalty != 1.0f;
    if (use_pen) {
        for (int i = t; i < (V + 31) / 32; i += ST) sm.pen[i] = 0;
        __syncthreads();
        const int32_t* h = hist + (long)b * hist_ld;
        for (int i = t; i < n_hist; i += ST) {
            const int id = h[i];
            if (id >= 0 && id < V) atomicOr(&sm.pen[id >> 5], 1u << (id & 31));
        }
        __syncthreads();
    }

    // order keys of the penalised logits; key 0 marks a slot past the vocabulary. Every load is
    // issued before any is used, through a buffer descriptor bounded by the row (a slot past it
    // reads 0 without touching memory), so the row costs one memory latency instead of one per slot.
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, V * 4, 0x00020000);
    uint32_t key[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i)
        key[i] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (base + i * GPT2_WAVE) * 4, 0, 0);
    uint32_t kmax = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int tok = base + i * GPT2_WAVE;
        float x = __builtin_bit_cast(float, key[i]);
        if (use_pen && tok < V && ((sm.pen[tok >> 5] >> (tok & 31)) & 1u)) x = x > 0.f ? x / penalty : x * penalty;
        key[i] = tok < V ? f32_order_key(x) : 0u;
        kmax = max(kmax, key[i]);
    }
    const uint32_t tmax = kmax;  // this thread's largest key (0: no token)
    {
        uint32_t unused = 0;
        block_max_min_u32(kmax, unused, sm);
    }
    const float m = f32_from_order_key(kmax);
    const float c = 1.4426950408889634f / temperature;
    float scale = 0.f;  // coarse-bin scale, set up when a coarse search runs
    auto coarse_setup = [&]() {
        uint32_t kmin = 0xffffffffu, dummy = 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const uint32_t k = opaque(key[i]);
            if (k != 0u && f32_from_order_key(k) > -INFINITY) kmin = min(kmin, k);
        }
        block_max_min_u32(dummy, kmin, sm);
        const float span = m - f32_from_order_key(kmin);
        scale = (kmin != 0xffffffffu && span > 0.f && span < INFINITY) ? (float)(NCOARSE - 1) / span : 0.f;
    };

    uint32_t theta = 1;  // kept: key >= theta
    int kept_list = -1;  // >= 0: every kept token's key is among the first kept_list entries of sm.list
    if (top_k > 0 && top_k < V) {
        const int nfw = min(SWAVES, V / (GPT2_WAVE * NPT));  // waves whose every slot is a token
        const int q = nfw > 0 ? (top_k + nfw - 1) / nfw : GPT2_WAVE + 1;
        if (q <= GPT2_WAVE) {
            // lower bound of kappa: the smallest over those waves of their q-th largest lane maximum
            if (w < nfw) {
                uint32_t sq = 0;
#pragma unroll 1
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t cand = sq | (1u << bit);
                    if (wave_count_ge(tmax, cand) >= q) sq = cand;
                }
                if (lane == 0) sm.lbw[w] = sq;
            }
            __syncthreads();
            // r = ceil(k / q) waves each hold q tokens at or above their own bound, so the r-th
            // largest of the bounds is a lower bound of kappa
            const int r = (top_k + q - 1) / q;
            uint32_t lb = 0;
            for (int i = 0; i < nfw; ++i) {
                int above = 0, atleast = 0;
                for (int j = 0; j < nfw; ++j) {
                    above += sm.lbw[j] > sm.lbw[i];
                    atleast += sm.lbw[j] >= sm.lbw[i];
                }
                if (above < r && r <= atleast) lb = sm.lbw[i];
            }
            const int n = compact_pairs(key, base, [&](uint32_t k) { return k >= lb; }, sm);
            if (n <= 8 * GPT2_WAVE) {
                if (w == 0) {
                    if (n <= 4 * GPT2_WAVE)
                        finish_top_k<4>(sm.list, sm.list_tok, n, lb, kmax, top_k, top_p, m, c, u[b], out + b,
                                        n_kept ? n_kept + b : nullptr);
                    else
                        finish_top_k<8>(sm.list, sm.list_tok, n, lb, kmax, top_k, top_p, m, c, u[b], out + b,
                                        n_kept ? n_kept + b : nullptr);
                }
                return;
            }
            if (n <= LCAP) {
                theta = radix_threshold<false, true>(key, n, none, m, c, 1u, (uint32_t)top_k, 0, 0, sm);
                kept_list = n;
            }
        }
        if (kept_list < 0) {
            coarse_setup();
            theta = coarse_threshold<false>(key, m, c, scale, 1u, (uint32_t)top_k, 0, sm);
        }
    }
    if (top_p < 1.0f) {
        uint64_t s = 0;
        if (kept_list >= 0) {
            for (int j = t; j < kept_list; j += ST) {
                const uint32_t k = sm.list[j];
                if (k >= theta) s += key_weight(k, m, c);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NPT; ++i) {
                const uint32_t k = opaque(key[i]);
                if (k >= theta) s += key_weight(k, m, c);
            }
        }
        s = block_sum_u64(s, sm);
        uint64_t P = (uint64_t)((double)top_p * (double)s);
        if (P == 0) P = 1;
        const uint32_t tau = kept_list >= 0
                                 ? radix_threshold<true, true>(key, kept_list, none, m, c, theta, 0u, P, 0, sm)
                                 : (coarse_setup(), coarse_threshold<true>(key, m, c, scale, theta, 0u, P, sm));
        theta = max(theta, tau);
    }

    // the draw: first token (vocabulary order) whose cumulative kept mass exceeds u * total
    uint64_t mine = 0;
    uint32_t kept = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const uint32_t k = opaque(key[i]);
        if (k >= theta) {
            mine += key_weight(k, m, c);
            ++kept;
        }
    }
    uint64_t wsum = mine;
    for (int o = 32; o; o >>= 1) wsum += shfl_xor_u64(wsum, o);
    kept = block_sum_u32(kept, sm);  // its barriers also order the wave totals below
    if (lane == 0) sm.wm[w] = wsum;
    __syncthreads();
    uint64_t total = 0;
    for (int i = 0; i < SWAVES; ++i) total += sm.wm[i];
    const float uu = u[b];
    const double ud = uu >= 0.f ? (uu < 1.f ? (double)uu : 1.0) : 0.0;
    uint64_t U = (uint64_t)(ud * (double)total);
    if (total > 0 && U >= total) U = total - 1;
    int ws = 0;
    uint64_t before = 0;
    {
        uint64_t acc = 0;
        bool found = false;
        for (int i = 0; i < SWAVES; ++i) {
            if (!found && U < acc + sm.wm[i]) {
                ws = i;
                before = acc;
                found = true;
            }
            acc += sm.wm[i];
        }
    }
    if (w == ws) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const uint32_t k = opaque(key[i]);
            sm.draw[i * GPT2_WAVE + lane] = k >= theta ? key_weight(k, m, c) : 0u;
        }
    }
    __syncthreads();
    if (total == 0 && t == 0) out[b] = 0;  // no finite maximum: the row has no distribution to draw from
    if (w == ws) {
        const uint64_t Uw = U - before;
        uint64_t tl = 0;
#pragma unroll 8
        for (int j = 0; j < NPT; ++j) tl += sm.draw[lane * NPT + j];
        uint64_t il = tl;
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t x = shfl_up_u64(il, o);
            if (lane >= o) il += x;
        }
        const uint64_t el = il - tl;
        if (tl > 0 && el <= Uw && Uw < il) {
            uint64_t acc = el;
            int pick = NPT - 1;
            for (int j = 0; j < NPT; ++j) {
                acc += sm.draw[lane * NPT + j];
                if (acc > Uw) {
                    pick = j;
                    break;
                }
            }
            out[b] = ws * GPT2_WAVE * NPT + lane * NPT + pick;
        }
        if (lane == 0 && n_kept) n_kept[b] = (int32_t)kept;
    }
}

// ---------------------------------------------------------------------------------------------
// Chunked top-k: (chunk, row) workgroups of 256 threads, 8 slots per thread; chunk c holds tokens
// [2048 c, 2048 c + 2048), slot i of thread t is token 2048 c + 256 i + t (coalesced per slot).
// ---------------------------------------------------------------------------------------------
constexpr int CT = 256, CNPT = 8, CHUNK = CT * CNPT, CWAVES = CT / GPT2_WAVE;

// Penalised order keys of this thread's slots (key 0: past the vocabulary), the chunk's history
// bits built in LDS first.
__device__ __forceinline__ void chunk_keys(const float* row, int V, int c0, const int32_t* h, int n_hist, float penalty,
                                           uint32_t (&key)[CNPT], uint32_t* pen) {
    const int t = threadIdx.x;
    const bool use_pen = h != nullptr && n_hist > 0 && penalty != 1.0f;
    if (use_pen) {
        for (int i = t; i < CHUNK / 32; i += CT) pen[i] = 0;
        __syncthreads();
        for (int i = t; i < n_hist; i += CT) {
            const int id = h[i] - c0;
            if (id >= 0 && id < CHUNK && id + c0 < V) atomicOr(&pen[id >> 5], 1u << (id & 31));
        }
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, V * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < CNPT; ++i) key[i] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (c0 + i * CT + t) * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < CNPT; ++i) {
        const int o = i * CT + t, tok = c0 + o;
        float x = __builtin_bit_cast(float, key[i]);
        if (use_pen && tok < V && ((pen[o >> 5] >> (o & 31)) & 1u)) x = x > 0.f ? x / penalty : x * penalty;
        key[i] = tok < V ? f32_order_key(x) : 0u;
    }
}

// Per wave: the q-th largest key among its 512 slots (q tokens of the wave reach it; 0 when the
// wave holds fewer than q tokens).
__global__ void __launch_bounds__(CT) sample_bound_kernel(const float* __restrict__ logits, long ld, int V,
                                                          const int32_t* __restrict__ hist, long hist_ld, int n_hist,
                                                          float penalty, int q, uint32_t* __restrict__ wbound,
                                                          int32_t* __restrict__ cnt) {
    __shared__ uint32_t pen[CHUNK / 32];
    const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int c0 = c * CHUNK, nw = gridDim.x * CWAVES;
    uint32_t key[CNPT];
    chunk_keys(logits + (long)b * ld, V, c0, hist ? hist + (long)b * hist_ld : nullptr, n_hist, penalty, key, pen);
    uint32_t sq = 0;
    if (q == 1) {  // the wave maximum
        for (int i = 0; i < CNPT; ++i) sq = max(sq, key[i]);
        for (int o = 32; o; o >>= 1) sq = max(sq, (uint32_t)__shfl_xor(sq, o));
    } else {
#pragma unroll 1
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = sq | (1u << bit);
            int n = 0;
#pragma unroll
            for (int i = 0; i < CNPT; ++i) n += wave_count_ge(key[i], cand);
            if (n >= q) sq = cand;
        }
    }
    if (lane == 0) wbound[(long)b * nw + c * CWAVES + w] = sq;
    if (c == 0 && t == 0) cnt[b] = 0;
}

// Copies every token with key >= the row's lower bound to the row's list (one global atomic per
// workgroup reserves its range); entries past lcap are counted but not stored.
__global__ void __launch_bounds__(CT) sample_collect_kernel(const float* __restrict__ logits, long ld, int V,
                                                            const int32_t* __restrict__ hist, long hist_ld,
                                                            int n_hist, float penalty, int r,
                                                            const uint32_t* __restrict__ wbound, int32_t* cnt,
                                                            uint32_t* __restrict__ lkey, uint32_t* __restrict__ ltok,
                                                            int lcap) {
    __shared__ uint32_t pen[CHUNK / 32];
    __shared__ int wcnt[CWAVES];
    __shared__ int wbase;
    const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int c0 = c * CHUNK, nw = gridDim.x * CWAVES;
    // the row's lower bound of kappa: the r-th largest of the wave bounds (r waves hold q tokens
    // each at or above their bound, r * q >= k); every wave finds it on its own
    const uint32_t b0 = lane < nw ? wbound[(long)b * nw + lane] : 0u;
    const uint32_t b1 = lane + GPT2_WAVE < nw ? wbound[(long)b * nw + lane + GPT2_WAVE] : 0u;
    uint32_t lb = 0;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = lb | (1u << bit);
        if (wave_count_ge(b0, cand) + wave_count_ge(b1, cand) >= r) lb = cand;
    }
    uint32_t key[CNPT];
    chunk_keys(logits + (long)b * ld, V, c0, hist ? hist + (long)b * hist_ld : nullptr, n_hist, penalty, key, pen);
    // one global atomic per workgroup: count the wave's candidates, reserve the block's range
    uint64_t bal[CNPT];
    int nwave = 0;
#pragma unroll
    for (int i = 0; i < CNPT; ++i) {
        bal[i] = __builtin_amdgcn_ballot_w64(key[i] >= lb);
        nwave += (int)__popcll(bal[i]);
    }
    if (lane == 0) wcnt[w] = nwave;
    __syncthreads();
    if (t == 0) {
        int tot = 0;
        for (int i = 0; i < CWAVES; ++i) tot += wcnt[i];
        wbase = tot ? atomicAdd(cnt + b, tot) : 0;
    }
    __syncthreads();
    int at = wbase;
    for (int i = 0; i < w; ++i) at += wcnt[i];
#pragma unroll
    for (int i = 0; i < CNPT; ++i) {
        if (key[i] >= lb) {
            const int idx = at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], 0u));
            if (idx < lcap) {
                lkey[(long)b * lcap + idx] = key[i];
                ltok[(long)b * lcap + idx] = (uint32_t)(c0 + i * CT + t);
            }
        }
        at += (int)__popcll(bal[i]);
    }
}

constexpr int kListCap = 4096;

// Workspace of the chunked top-k path for B rows of V tokens (bytes; each region 256-byte aligned).
struct SampleWs {
    size_t wbound, cnt, lkey, ltok, total;
    SampleWs(int B, int V) {
        const size_t nw = (size_t)((V + CHUNK - 1) / CHUNK) * CWAVES;
        auto al = [](size_t x) { return (x + 255) / 256 * 256; };
        wbound = 0;
        cnt = wbound + al((size_t)B * nw * 4);
        lkey = cnt + al((size_t)B * 4);
        ltok = lkey + al((size_t)B * kListCap * 4);
        total = ltok + al((size_t)B * kListCap * 4);
    }
};

}  // namespace

size_t sample_workspace_bytes(int B, int V) { return SampleWs(B, V).total; }

hipError_t sample(const float* logits, long ld, int B, int V, const int32_t* hist, long hist_ld, int n_hist,
                  float temperature, int top_k, float top_p, float penalty, const float* u, int32_t* out,
                  int32_t* n_kept, void* ws, size_t ws_bytes, hipStream_t s) {
    SampleList cl;
    if (ws != nullptr && top_k > 0 && top_k < V) {
        const SampleWs L(B, V);
        const int G = (V + CHUNK - 1) / CHUNK;
        // waves whose 8 slots all hold tokens: r = ceil(k / q) <= nfull of them reach their bound
        int nfull = 0;
        for (int c = 0; c < G; ++c)
            for (int w = 0; w < CWAVES; ++w) nfull += c * CHUNK + (CNPT - 1) * CT + w * GPT2_WAVE + GPT2_WAVE - 1 < V;
        const int q = nfull > 0 ? (top_k + nfull - 1) / nfull : CHUNK;
        const int r = (top_k + q - 1) / q;
        if (ws_bytes >= L.total && nfull >= 1 && q <= CHUNK / CWAVES && r <= G * CWAVES) {
            char* p = static_cast<char*>(ws);
            uint32_t* wbound = reinterpret_cast<uint32_t*>(p + L.wbound);
            int32_t* cnt = reinterpret_cast<int32_t*>(p + L.cnt);
            uint32_t* lkey = reinterpret_cast<uint32_t*>(p + L.lkey);
            uint32_t* ltok = reinterpret_cast<uint32_t*>(p + L.ltok);
            sample_bound_kernel<<<dim3(G, B), dim3(CT), 0, s>>>(logits, ld, V, hist, hist_ld, n_hist, penalty, q, wbound,
                                                                 cnt);
            sample_collect_kernel<<<dim3(G, B), dim3(CT), 0, s>>>(logits, ld, V, hist, hist_ld, n_hist, penalty, r,
                                                                   wbound, cnt, lkey, ltok, kListCap);
            cl.cnt = cnt;
            cl.lkey = lkey;
            cl.ltok = ltok;
            cl.lcap = kListCap;
        }
    }
    const int npt = ((V + ST - 1) / ST + 7) / 8 * 8;  // slots per thread, a multiple of 8
#define GPT2_SAMPLE_CASE(N)                                                                                   \
    case N:                                                                                                  \
        sample_kernel<N><<<dim3(B), dim3(ST), 0, s>>>(logits, ld, V, hist, hist_ld, n_hist, temperature, top_k, \
                                                       top_p, penalty, u, out, n_kept, cl);                    \
        break;
    switch (npt) {
        GPT2_SAMPLE_CASE(8)
        GPT2_SAMPLE_CASE(16)
        GPT2_SAMPLE_CASE(24)
        GPT2_SAMPLE_CASE(32)
        GPT2_SAMPLE_CASE(40)
        GPT2_SAMPLE_CASE(48)
        GPT2_SAMPLE_CASE(56)
        GPT2_SAMPLE_CASE(64)
        default: return hipErrorInvalidValue;
    }
#undef GPT2_SAMPLE_CASE
    return hipGetLastError();
}

int sample_max_vocab() { return ST * SNPT; }

}  // namespace gpt2k
