// Causal multi-head self-attention, flash style: the [T, T] score matrix is never stored.
//   o[b,h,i,:] = sum_{j<=i} softmax_j(q_i . k_j / sqrt(64)) v_j
// ("复现GPT-2 124M" §2.1-§2.2 and "GPT-2模型架构解析与实现指南" §2.1: scores scaled by 1/sqrt(d_head),
// keys after the query masked to -inf before the softmax, the diagonal kept.)
//
// bf16 kernel. A workgroup of eight wavefronts owns 128 queries of one (b, h); each wavefront owns
// 16 of them. Key/value tiles of 64 keys are staged in LDS (K as [key][d] with 16-byte chunks
// XOR-swizzled, V transposed to [d][key]), double-buffered: the global loads of tile t+1 are in
// flight in registers while tile t runs, so one barrier per tile remains and the load latency is
// hidden. Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16, so each
// lane's accumulator column is one query: the softmax row statistics are per-lane values combined
// over the four 16-lane groups, and the probabilities are already in the operand layout of the
// second product O^T += V^T P^T. Online softmax in fp32 on the raw scores: exp2(s*c - m*c) is one
// FMA and one v_exp_f32 per score (c = scale * log2 e); the reference maximum moves only when a
// query's maximum grows by more than 2^8, so the accumulators are rarely rescaled. The row sums
// come from the matrix unit as ones x P^T, over the same bf16 probabilities that weight V. Tiles
// wholly above a wavefront's diagonal are skipped; only tiles that cross it are masked (selects).
// Workgroups are issued longest-first (last query tiles first) to even out the causal imbalance.
// When the grid is small, a workgroup runs two groups of eight wavefronts over the same queries,
// each taking every other key tile; group 1 hands its accumulators, denominator and reference
// maximum to group 0 through LDS, which rescales both to the common maximum and adds them.
#include "common.h"

#ifndef GPT2_ATT_WAVES
#define GPT2_ATT_WAVES 8  // 128 queries per workgroup (faster than 32 or 64 on MI355X)
#endif

namespace gpt2k {
namespace {

constexpr int KT = 64;        // keys per LDS tile
constexpr int DH = 64;        // head size
constexpr int VTS = KT + 8;   // row stride (elements) of the transposed V tile: spreads rows over banks

__device__ __forceinline__ int kswz(int key, int chunk) { return key * DH + ((chunk ^ (key & 7)) << 3); }

template <int WAVES, int G>  // 16 queries per wavefront; G groups of WAVES wavefronts share the queries
__global__ __launch_bounds__(64 * WAVES * G) void attn_bf16_kernel(const uint16_t* __restrict__ Q, int64_t qsb,
                                                               int64_t qsh, int64_t qst,
                                                               const uint16_t* __restrict__ K, int64_t ksb,
                                                               int64_t ksh, int64_t kst,
                                                               const uint16_t* __restrict__ V, int64_t vsb,
                                                               int64_t vsh, int64_t vst, uint16_t* __restrict__ O,
                                                               int64_t osb, int64_t osh, int64_t ost, int64_t osx,
                                                               int B, int H,
                                                               int T, float scale_log2) {
    constexpr int QT = 16 * WAVES, NG = 64 * WAVES, CPT = KT * 8 / NG;  // 16-byte chunks per thread per tile
    // sK / sVt: [buffer][group]; after the loop the same bytes hold the partial results of group 1
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][G][KT * DH];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[2][G][DH * VTS];

    const int nqt = (T + QT - 1) / QT;
    const int bh = blockIdx.x % (B * H);
    const int qt = nqt - 1 - blockIdx.x / (B * H);
    const int b = bh / H, h = bh % H;
    const int q0 = qt * QT;
    const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t / GPT2_WAVE), lane = t % GPT2_WAVE;
    const int grp = wave / WAVES, wv = wave % WAVES, tg = t % NG;  // group, wavefront and thread in the group
    const int r16 = lane & 15, g4 = lane >> 4;
    const int qw = q0 + 16 * wv;  // this wavefront's first query
    const int qi = qw + r16;      // this lane's query (accumulator column)

    const uint16_t* Qb = Q + b * qsb + h * qsh;
    const uint16_t* Kb = K + b * ksb + h * ksh;
    const uint16_t* Vb = V + b * vsb + h * vsh;

    // Q^T as the B operand of S^T = K Q^T: lane holds query qi, d = kk*32 + 8*g4 .. +7
    bf16x8_t qf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        u32x4_t u = {0u, 0u, 0u, 0u};
        if (qi < T) u = *reinterpret_cast<const u32x4_t*>(Qb + qi * qst + kk * 32 + g4 * 8);
        qf[kk] = __builtin_bit_cast(bf16x8_t, u);
    }

    const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_u);
    f32x4_t oacc[4];  // [d fragment]; rows d = df*16 + 4*g4 + e, column = query qi
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};  // every row: the running denominator of the column's query
    float mrow = -INFINITY;               // reference maximum of the raw scores of this lane's query

    // tile loader: thread tg of a group moves CPT 16-byte K chunks (key c/8, chunk c%8) and CPT
    // 16-byte V chunks (key c%64, d chunk c/64) of its group's tile, c = tg + i*NG
    auto load_tile = [&](int k0, u32x4_t (&kr)[CPT], u32x4_t (&vr)[CPT]) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tg + i * NG, kkey = c / 8, kch = c % 8, vkey = c % KT, vdc = c / KT;
            kr[i] = u32x4_t{0u, 0u, 0u, 0u};
            vr[i] = u32x4_t{0u, 0u, 0u, 0u};
            if (k0 + kkey < T) kr[i] = *reinterpret_cast<const u32x4_t*>(Kb + (k0 + kkey) * kst + kch * 8);
            if (k0 + vkey < T) vr[i] = *reinterpret_cast<const u32x4_t*>(Vb + (k0 + vkey) * vst + vdc * 8);
        }
    };
    auto store_tile = [&](int buf, const u32x4_t (&kr)[CPT], const u32x4_t (&vr)[CPT]) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tg + i * NG, kkey = c / 8, kch = c % 8, vkey = c % KT, vdc = c / KT;
            *reinterpret_cast<u32x4_t*>(&sK[buf][grp][kswz(kkey, kch)]) = kr[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sVt[buf][grp][(vdc * 8 + 2 * j) * VTS + vkey] = (uint16_t)(vr[i][j] & 0xffffu);
                sVt[buf][grp][(vdc * 8 + 2 * j + 1) * VTS + vkey] = (uint16_t)(vr[i][j] >> 16);
            }
        }
    };

    // step s: group g runs key tile s*G + g
    const int kend = min(T, q0 + QT);
    const int n_kt = (kend + KT - 1) / KT;
    const int n_st = (n_kt + G - 1) / G;
    u32x4_t kr[CPT], vr[CPT];
    load_tile(grp * KT, kr, vr);
    store_tile(0, kr, vr);
    if (n_st > 1) load_tile((G + grp) * KT, kr, vr);
    __syncthreads();

    for (int st = 0; st < n_st; ++st) {
        const int kt = st * G + grp, k0 = kt * KT, buf = st & 1;
        const uint16_t* tK = sK[buf][grp];
        const uint16_t* tV = sVt[buf][grp];
        if (kt < n_kt && k0 <= qw + 15) {  // some key of this tile is visible to some query of this wavefront
            // S^T[key, query] for 64 keys x 16 queries
            f32x4_t s[4];
#pragma unroll
            for (int mf = 0; mf < 4; ++mf) {
                s[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&tK[kswz(mf * 16 + r16, kk * 4 + g4)]);
                    s[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], s[mf], 0, 0, 0);
                }
            }
            if (k0 + KT - 1 > qw || k0 + KT > T) {  // the tile crosses the diagonal or T
#pragma unroll
                for (int mf = 0; mf < 4; ++mf)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = k0 + mf * 16 + 4 * g4 + e;
                        s[mf][e] = (key <= qi && key < T) ? s[mf][e] : -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mf = 0; mf < 4; ++mf) mx = fmaxf(mx, fmaxf(fmaxf(s[mf][0], s[mf][1]), fmaxf(s[mf][2], s[mf][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16, GPT2_WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 32, GPT2_WAVE));
            // The reference maximum moves only when some query's tile maximum exceeds it by more
            // than 8 in log2 units (the softmax does not depend on the constant subtracted, and
            // unscaled probabilities up to 2^8 are exact enough in fp32 and bf16); then the whole
            // wavefront rescales its accumulators, which is rare after the first tiles.
            if (__builtin_amdgcn_ballot_w64((mx - mrow) * scale_log2 > 8.f)) {
                const float mnew = fmaxf(mrow, mx);
                // a query with every key so far masked (only past T) keeps a zero state
                const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mrow - mnew) * scale_log2);
                mrow = mnew;
#pragma unroll
                for (int df = 0; df < 4; ++df) oacc[df] *= alpha;
                lacc *= alpha;
            }
            const float mb = mrow == -INFINITY ? 0.f : mrow * scale_log2;
#pragma unroll
            for (int mf = 0; mf < 4; ++mf)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[mf][e] = __builtin_amdgcn_exp2f(fmaf(s[mf][e], scale_log2, -mb));

            // O^T[d, query] += V^T[d, key] P^T[key, query], 32 keys per MFMA. Slot j of a lane
            // holds key 32*hh + 4*g4 + j (j < 4) or 32*hh + 16 + 4*g4 + (j - 4) on both operands.
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4_t pu;
                pu[0] = pack_bf16x2(s[2 * hh][0], s[2 * hh][1]);
                pu[1] = pack_bf16x2(s[2 * hh][2], s[2 * hh][3]);
                pu[2] = pack_bf16x2(s[2 * hh + 1][0], s[2 * hh + 1][1]);
                pu[3] = pack_bf16x2(s[2 * hh + 1][2], s[2 * hh + 1][3]);
                const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pu);
                lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc, 0, 0, 0);
#pragma unroll
                for (int df = 0; df < 4; ++df) {
                    const uint16_t* vrow = &tV[(df * 16 + r16) * VTS + 32 * hh + 4 * g4];
                    const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
                    const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16);
                    const u32x4_t vu = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[df] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vu), pf, oacc[df],
                                                                       0, 0, 0);
                }
            }
        }
        if (st + 1 < n_st) {
            store_tile(buf ^ 1, kr, vr);  // step st+1 (its loads were issued during step st)
            if (st + 2 < n_st) load_tile(((st + 2) * G + grp) * KT, kr, vr);
        }
        __syncthreads();
    }

    if constexpr (G > 1) {
        // groups 1.. hand their (accumulators, denominator, reference maximum) to group 0, which
        // rescales every part to the common maximum and adds them in group order
        static_assert(G == 2, "the merge area holds one partner group");
        float* part = reinterpret_cast<float*>(&sVt[0][0][0]);  // [wave][lane][18], fits in sVt
        static_assert(sizeof(sVt) >= sizeof(float) * WAVES * 64 * 18, "merge area");
        float* mine = part + ((size_t)wv * 64 + lane) * 18;
        if (grp == 1) {
#pragma unroll
            for (int df = 0; df < 4; ++df)
#pragma unroll
                for (int e = 0; e < 4; ++e) mine[df * 4 + e] = oacc[df][e];
            mine[16] = lacc[0];
            mine[17] = mrow;
        }
        __syncthreads();
        if (grp == 1) return;
        const float m1 = mine[17], mn = fmaxf(mrow, m1);
        const float a0 = mrow == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mrow - mn) * scale_log2);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - mn) * scale_log2);
#pragma unroll
        for (int df = 0; df < 4; ++df)
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[df][e] = oacc[df][e] * a0 + mine[df * 4 + e] * a1;
        lacc[0] = lacc[0] * a0 + mine[16] * a1;
    }

    if (qi < T) {
        const float inv = 1.0f / lacc[0];
        uint16_t* Ob = O + b * osb + h * osh + qi * ost;
#pragma unroll
        for (int df = 0; df < 4; ++df) {
            uint2 u;
            u.x = pack_bf16x2(oacc[df][0] * inv, oacc[df][1] * inv);
            u.y = pack_bf16x2(oacc[df][2] * inv, oacc[df][3] * inv);
            // head dims df*16 + 4*g4 .. +3 lie in half df/2 of the head (32 dims each, osx apart)
            *reinterpret_cast<uint2*>(Ob + (df >> 1) * osx + (df & 1) * 16 + 4 * g4) = u;
        }
    }
}

// fp32 kernel (fp32 compute mode): one wavefront per 64 queries of one (b, h), one query per lane;
// key/value tiles of 64 keys in LDS are read as broadcasts; exact expf online softmax.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ Q, int64_t qsb, int64_t qsh, int64_t qst,
                                                      const float* __restrict__ K, int64_t ksb, int64_t ksh, int64_t kst,
                                                      const float* __restrict__ V, int64_t vsb, int64_t vsh, int64_t vst,
                                                      float* __restrict__ O, int64_t osb, int64_t osh, int64_t ost,
                                                      int B, int H, int T, float scale) {
    __shared__ float sK[64][DH + 1];
    __shared__ float sV[64][DH + 1];
    const int nqt = (T + 63) / 64;
    const int bh = blockIdx.x % (B * H);
    const int qt = nqt - 1 - blockIdx.x / (B * H);
    const int b = bh / H, h = bh % H;
    const int lane = threadIdx.x;
    const int qi = qt * 64 + lane;
    const float* Qb = Q + b * qsb + h * qsh;
    const float* Kb = K + b * ksb + h * ksh;
    const float* Vb = V + b * vsb + h * vsh;
    float q[DH], acc[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) {
        q[c] = qi < T ? Qb[qi * qst + c] : 0.f;
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int kend = min(T, qt * 64 + 64);
    for (int k0 = 0; k0 < kend; k0 += 64) {
        __syncthreads();
        for (int idx = lane; idx < 64 * DH; idx += 64) {
            const int key = idx / DH, c = idx % DH, kg = k0 + key;
            sK[key][c] = kg < T ? Kb[kg * kst + c] : 0.f;
            sV[key][c] = kg < T ? Vb[kg * vst + c] : 0.f;
        }
        __syncthreads();
        const int jn = min(64, kend - k0);
        for (int j = 0; j < jn; ++j) {
            if (k0 + j > qi) break;
            float sdot = 0.f;
#pragma unroll
            for (int c = 0; c < DH; ++c) sdot = fmaf(q[c], sK[j][c], sdot);
            const float sv = sdot * scale;
            const float mnew = fmaxf(m, sv);
            const float alpha = expf(m - mnew), p = expf(sv - mnew);
            l = l * alpha + p;
#pragma unroll
            for (int c = 0; c < DH; ++c) acc[c] = acc[c] * alpha + p * sV[j][c];
            m = mnew;
        }
    }
    if (qi < T) {
        float* Ob = O + b * osb + h * osh + qi * ost;
        const float inv = 1.0f / l;
#pragma unroll
        for (int c = 0; c < DH; ++c) Ob[c] = acc[c] * inv;
    }
}

}  // namespace

hipError_t attention_bf16(const uint16_t* q, const int64_t* qs, const uint16_t* k, const int64_t* ks, const uint16_t* v,
                          const int64_t* vs, uint16_t* o, const int64_t* os, int B, int H, int T, hipStream_t s,
                          int64_t os_half) {
    const float scale_log2 = 0.125f * 1.4426950408889634f;  // (1/sqrt(64)) * log2(e)
    constexpr int WAVES = GPT2_ATT_WAVES;
    const int nqt = (T + 16 * WAVES - 1) / (16 * WAVES);
    // Few workgroups (at most two per CU): two wavefront groups per workgroup split the key tiles,
    // which shortens the longest workgroups; with more, one group per workgroup is faster
    // (measured: B=4 H=12 T=1024 24.2 vs 27.1 us; B=8 42.9 vs 39.3 us).
    const dim3 grid(nqt * B * H);
#define GPT2_ATT_LAUNCH(G)                                                                                         \
    attn_bf16_kernel<WAVES, G><<<grid, dim3(64 * WAVES * G), 0, s>>>(q, qs[0], qs[1], qs[2], k, ks[0], ks[1], ks[2], \
                                                                     v, vs[0], vs[1], vs[2], o, os[0], os[1], os[2],  \
                                                                     os_half, B, H, T, scale_log2)
    if (nqt * B * H <= 512)
        GPT2_ATT_LAUNCH(2);
    else
        GPT2_ATT_LAUNCH(1);
#undef GPT2_ATT_LAUNCH
    return hipGetLastError();
}

hipError_t attention_f32(const float* q, const int64_t* qs, const float* k, const int64_t* ks, const float* v,
                         const int64_t* vs, float* o, const int64_t* os, int B, int H, int T, hipStream_t s) {
    const int nqt = (T + 63) / 64;
    attn_f32_kernel<<<dim3(nqt * B * H), dim3(64), 0, s>>>(q, qs[0], qs[1], qs[2], k, ks[0], ks[1], ks[2], v, vs[0], vs[1],
                                                          vs[2], o, os[0], os[1], os[2], B, H, T, 0.125f);
    return hipGetLastError();
}

}  // namespace gpt2k
