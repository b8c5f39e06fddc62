// Sampled next-token choice over a [B, V] block of fp32 logits: repetition penalty, temperature,
// top-k, top-p and a multinomial draw by inverse CDF ("GPT2模型开发实战：从原理到部署全解析" §8.2
// lists the four knobs; "GPT-2模型架构解析与实现指南" §4.1 draws from softmax(logits / temperature)).
//
// One 1024-thread workgroup per row. Wave w owns the vocabulary span [w*64*NPT, (w+1)*64*NPT) with
// NPT = ceil(V / 1024) rounded up to a multiple of 8 (a template constant, so the per-thread slots
// stay in registers without per-slot guards); lane l holds the order keys of tokens
// w*64*NPT + i*64 + l, so every load is a coalesced 256-byte wave access and the row is read once.
//
// Both cut-offs are found as a threshold on the order-preserving key of the processed logit:
//   top-k keeps key >= kappa, kappa the k-th largest key;
//   top-p keeps key >= tau, tau the smallest key whose strictly-larger kept mass is below p.
// Each threshold is located in two stages: a 2048-bin histogram over the value's distance from the
// row maximum (bins spread the bulk of the distribution, so LDS atomics rarely collide within a
// wave instruction), then four 8-bit radix passes over the exact key restricted to the chosen bin.
// Probability mass is accumulated in 2^-40 fixed point (u64), so every sum is exact and the result
// does not depend on the order in which lanes add.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int ST = 1024;                // threads per row
constexpr int SWAVES = ST / GPT2_WAVE;  // 16
constexpr int SNPT = 64;                // values per thread: V <= ST * SNPT
constexpr int NCOARSE = 2048;
constexpr float kFix = 1099511627776.0f;  // 2^40: fixed-point scale of a softmax weight (max weight 1)

struct SampleSmem {
    uint32_t pen[ST * SNPT / 32];   // history membership bits
    uint32_t cnt[NCOARSE];          // histogram counts (radix passes use the first 256)
    uint64_t mass[NCOARSE];         // histogram masses
    uint64_t draw[GPT2_WAVE * SNPT];  // one wave's weights in vocabulary order
    uint64_t wm[SWAVES];
    uint32_t wc[SWAVES];
    uint32_t wk[SWAVES];
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
template <bool MAX>
__device__ uint32_t block_ext_u32(uint32_t v, SampleSmem& sm) {
    for (int o = 32; o; o >>= 1) {
        const uint32_t x = __shfl_xor(v, o);
        v = MAX ? max(v, x) : min(v, x);
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.wk[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = sm.wk[0];
    for (int i = 1; i < SWAVES; ++i) t = MAX ? max(t, sm.wk[i]) : min(t, sm.wk[i]);
    return t;
}

// Coarse bin of a value: 0 at the row maximum m, growing with the distance below it (monotone:
// a larger value never lands in a larger bin; equal values share a bin). -inf and NaN go last.
__device__ __forceinline__ int coarse_bin(float z, float m, float scale) {
    const float t = (m - z) * scale;
    return t < (float)NCOARSE ? (int)fmaxf(t, 0.f) : NCOARSE - 1;
}

// A copy of v the compiler cannot see through: values derived from it are recomputed where they are
// used instead of being hoisted out of the histogram passes and kept live for every slot.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ uint64_t fixed_weight(float z, float m) {
    return (uint64_t)(__builtin_amdgcn_exp2f((z - m) * 1.4426950408889634f) * kFix);
}

// Histogram bins [0, nb) are ordered by decreasing value. COUNT mode (top-k): returns the bin b
// whose count range holds the rem-th largest element and lowers rem by the count before b. MASS
// mode (top-p): returns the last non-empty bin b whose mass before it, plus above, is below P, and
// adds that mass to above. Every thread of the block calls it and gets the same result.
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

// Threshold key over the elements with key >= lo_key (lo_key >= 1: empty slots hold key 0):
// COUNT mode the rem-th largest key, MASS mode the smallest key whose strictly-larger mass is below P.
template <bool MASS, int NPT>
__device__ uint32_t find_threshold(const uint32_t (&key)[NPT], float m, float scale, uint32_t lo_key, uint32_t rem,
                                   uint64_t P, SampleSmem& sm) {
    uint64_t above = 0;
    // stage 1: coarse bins
    clear_bins(NCOARSE, MASS, sm);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const uint32_t k = opaque(key[i]);
        if (k >= lo_key) {
            const float z = f32_from_order_key(k);
            const int b = coarse_bin(z, m, scale);
            atomicAdd(&sm.cnt[b], 1u);
            if (MASS) atomicAdd((unsigned long long*)&sm.mass[b], (unsigned long long)fixed_weight(z, m));
        }
    }
    __syncthreads();
    const int cbin = select_bin<MASS>(NCOARSE, rem, above, P, sm);
    // stage 2: radix passes over the exact key inside the coarse bin, most significant byte first
    uint32_t prefix = 0;
#pragma unroll 1
    for (int r = 0; r < 4; ++r) {
        const int shift = 24 - 8 * r;
        const int hs = r == 0 ? 31 : shift + 8;  // r == 0: no prefix to match (compare bit 31 with 0 / 1)
        const uint32_t want = r == 0 ? 0xffffffffu : prefix;
        clear_bins(256, MASS, sm);
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const uint32_t k = opaque(key[i]);
            const float z = f32_from_order_key(k);
            const bool in = k >= lo_key && coarse_bin(z, m, scale) == cbin && (r == 0 || (k >> hs) == want);
            if (in) {
                const int b = 255 - (int)((k >> shift) & 255u);
                atomicAdd(&sm.cnt[b], 1u);
                if (MASS) atomicAdd((unsigned long long*)&sm.mass[b], (unsigned long long)fixed_weight(z, m));
            }
        }
        __syncthreads();
        const int b = select_bin<MASS>(256, rem, above, P, sm);
        prefix = (prefix << 8) | (uint32_t)(255 - b);
    }
    return prefix;
}

template <int NPT>
__global__ void __launch_bounds__(ST) sample_kernel(const float* __restrict__ logits, long ld, int V,
                                                     const int32_t* __restrict__ hist, long hist_ld, int n_hist,
                                                     float temperature, int top_k, float top_p, float penalty,
                                                     const float* __restrict__ u, int32_t* __restrict__ out,
                                                     int32_t* __restrict__ n_kept) {
    __shared__ SampleSmem sm;
    const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int base = w * GPT2_WAVE * NPT + lane;  // token of slot i: base + i * 64
    const float* row = logits + (long)b * ld;

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

    // order keys of the processed logits; key 0 marks a slot past the vocabulary
    uint32_t key[NPT];
    uint32_t kmax = 0, kmin = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int tok = base + i * GPT2_WAVE;
        key[i] = 0;
        if (tok < V) {
            float v = __builtin_nontemporal_load(row + tok);
            if (use_pen && ((sm.pen[tok >> 5] >> (tok & 31)) & 1u)) v = v > 0.f ? v / penalty : v * penalty;
            v = v / temperature;
            key[i] = f32_order_key(v);
            kmax = max(kmax, key[i]);
            if (v > -INFINITY) kmin = min(kmin, key[i]);
        }
    }
    kmax = block_ext_u32<true>(kmax, sm);
    kmin = block_ext_u32<false>(kmin, sm);
    const float m = f32_from_order_key(kmax);
    const float zlo = f32_from_order_key(kmin);
    const float span = m - zlo;
    const float scale = (kmin != 0xffffffffu && span > 0.f && span < INFINITY) ? (float)(NCOARSE - 1) / span : 0.f;

    uint32_t theta = 1;  // kept: key >= theta
    if (top_k > 0 && top_k < V) theta = find_threshold<false, NPT>(key, m, scale, 1u, (uint32_t)top_k, 0, sm);
    if (top_p < 1.0f) {
        uint64_t s = 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const uint32_t k = opaque(key[i]);
            if (k >= theta) s += fixed_weight(f32_from_order_key(k), m);
        }
        s = block_sum_u64(s, sm);
        uint64_t P = (uint64_t)((double)top_p * (double)s);
        if (P == 0) P = 1;
        const uint32_t tau = find_threshold<true, NPT>(key, m, scale, theta, 0u, P, sm);
        theta = max(theta, tau);
    }

    // the draw: first token (vocabulary order) whose cumulative kept mass exceeds u * total
    uint64_t mine = 0;
    uint32_t kept = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const uint32_t k = opaque(key[i]);
        if (k >= theta) {
            mine += fixed_weight(f32_from_order_key(k), m);
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
            sm.draw[i * GPT2_WAVE + lane] = k >= theta ? fixed_weight(f32_from_order_key(k), m) : 0ull;
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

}  // namespace

hipError_t sample(const float* logits, long ld, int B, int V, const int32_t* hist, long hist_ld, int n_hist,
                  float temperature, int top_k, float top_p, float penalty, const float* u, int32_t* out,
                  int32_t* n_kept, hipStream_t s) {
    const int npt = ((V + ST - 1) / ST + 7) / 8 * 8;  // slots per thread, a multiple of 8
#define GPT2_SAMPLE_CASE(N)                                                                                   \
    case N:                                                                                                  \
        sample_kernel<N><<<dim3(B), dim3(ST), 0, s>>>(logits, ld, V, hist, hist_ld, n_hist, temperature, top_k, \
                                                       top_p, penalty, u, out, n_kept);                        \
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
