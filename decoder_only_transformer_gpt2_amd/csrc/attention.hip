// Causal multi-head self-attention, flash style: the [T, T] score matrix is never stored.
//   o[b,h,i,:] = sum_{j<=i} softmax_j(q_i . k_j / sqrt(64)) v_j
// ("复现GPT-2 124M" §2.1-§2.2 and "GPT-2模型架构解析与实现指南" §2.1: scores scaled by 1/sqrt(d_head),
// keys after the query masked to -inf before the softmax, the diagonal kept.)
//
// bf16 kernel. A workgroup of four wavefronts owns 128 queries of one (b, h); each wavefront owns
// 32 of them (two 16-query column blocks), so every K and V fragment it reads from LDS feeds two
// MFMAs and the per-tile bookkeeping is shared by twice the queries. Key/value tiles of 64 keys
// are staged in LDS (K as [key][d] with 16-byte chunks XOR-swizzled by key, V transposed to
// [d][key]), double-buffered: the global loads of tile t+1 are in flight in registers while tile t
// runs, so one barrier per tile remains and the load latency is hidden. V is transposed in pairs
// of keys, so each 4-byte LDS write carries both keys of one dimension. Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16, so each lane's accumulator column is one
// query: the softmax row statistics are per-lane values combined over the four 16-lane groups, and
// the probabilities are already in the operand layout of the second product O^T += V^T P^T.
// Online softmax in fp32 on the raw scores: exp2(s*c - m*c) is one FMA and one v_exp_f32 per score
// (c = scale * log2 e); the reference maximum moves only when a query's maximum grows by more than
// 2^8, so the accumulators are rarely rescaled. The row sums come from the matrix unit as
// ones x P^T, over the same bf16 probabilities that weight V. Tiles wholly above a wavefront's
// diagonal are skipped; only tiles that cross it are masked (selects). Workgroups are issued
// longest-first (last query tiles first) to even out the causal imbalance. When the grid is small,
// a workgroup runs two groups of wavefronts over the same queries, each taking every other key
// tile; group 1 hands its accumulators, denominator and reference maximum to group 0 through LDS,
// which rescales both to the common maximum and adds them.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int KT = 64;        // keys per LDS tile
constexpr int DH = 64;        // head size
constexpr int VTS = KT + 4;   // row stride (elements) of the transposed V tile: 34 words, so the
                              // 8-byte fragment reads of 16 rows fall on distinct banks
// Maximum over the four lanes L, L^16, L^32, L^48 (the four 16-lane rows). Only the rare
// rescale path needs it. (The gfx950 row-swap builtins would avoid the LDS crossbar, but this
// toolchain miscompiles them when both operands are the same value.)
__device__ __forceinline__ float max_over_rows(float m) {
    m = fmaxf(m, __shfl_xor(m, 16, GPT2_WAVE));
    return fmaxf(m, __shfl_xor(m, 32, GPT2_WAVE));
}

// K tile element offset of (key, 16-byte chunk): chunks are permuted within a key row by
// (key & 7) ^ ((key >> 3) & 1), which spreads the 16-byte reads of 16 consecutive keys over all
// banks whether a read pass covers 8 or 16 lanes.
__device__ __forceinline__ int kswz(int key, int chunk) {
    return key * DH + ((chunk ^ (key & 7) ^ ((key >> 3) & 1)) << 3);
}

template <int WAVES, int G>  // 32 queries per wavefront; G groups of WAVES wavefronts share the queries
__global__ __launch_bounds__(64 * WAVES * G, 4) void attn_bf16_kernel(
    const uint16_t* __restrict__ Q, int64_t qsb, int64_t qsh, int64_t qst, const uint16_t* __restrict__ K, int64_t ksb,
    int64_t ksh, int64_t kst, const uint16_t* __restrict__ V, int64_t vsb, int64_t vsh, int64_t vst,
    uint16_t* __restrict__ O, int64_t osb, int64_t osh, int64_t ost, int64_t osx, int B, int H, int T,
    float scale_log2) {
    constexpr int NQ = 2, QW = 16 * NQ;          // 16-query column blocks and queries per wavefront
    constexpr int QT = QW * WAVES, NG = 64 * WAVES;
    constexpr int KCPT = KT * 8 / NG;            // 16-byte K chunks per thread per tile
    constexpr int VPPT = KT * 4 / NG;            // (key pair, 16-byte d chunk) V items per thread per tile
    static_assert(KCPT >= 1 && VPPT >= 1 && KT * 4 % NG == 0, "tile loader");
    constexpr int KSZ = KT * DH, VSZ = DH * VTS;  // elements of one K tile and one transposed V tile
    constexpr int RING = 2 * G * (KSZ + VSZ);
    constexpr int MERGE = (G - 1) * WAVES * 64 * (NQ * 18) * 2;  // groups 1.. partial states (floats)
    // [buffer][group] K tiles, then [buffer][group] V tiles; after the loop the merge area
    __shared__ __attribute__((aligned(16))) uint16_t smem[RING > MERGE ? RING : MERGE];
    auto tile_k = [&](int buf, int g) { return smem + (buf * G + g) * KSZ; };
    auto tile_v = [&](int buf, int g) { return smem + 2 * G * KSZ + (buf * G + g) * VSZ; };

    const int nqt = (T + QT - 1) / QT;
    const int bh = blockIdx.x % (B * H);
    const int qt = nqt - 1 - blockIdx.x / (B * H);
    const int b = bh / H, h = bh % H;
    const int q0 = qt * QT;
    const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t / GPT2_WAVE), lane = t % GPT2_WAVE;
    const int grp = wave / WAVES, wv = wave % WAVES, tg = t % NG;  // group, wavefront and thread in the group
    const int r16 = lane & 15, g4 = lane >> 4;
    const int qw = q0 + QW * wv;  // this wavefront's first query; lane's queries: qw + 16*qb + r16

    const uint16_t* Qb = Q + b * qsb + h * qsh;
    const uint16_t* Kb = K + b * ksb + h * ksh;
    const uint16_t* Vb = V + b * vsb + h * vsh;

    // Q^T as the B operand of S^T = K Q^T: lane holds query qw + 16*qb + r16, d = kk*32 + 8*g4 .. +7
    bf16x8_t qf[NQ][2];
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int qi = qw + 16 * qb + r16;
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (qi < T) u = *reinterpret_cast<const u32x4_t*>(Qb + qi * qst + kk * 32 + g4 * 8);
            qf[qb][kk] = __builtin_bit_cast(bf16x8_t, u);
        }

    const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_u);
    f32x4_t oacc[NQ][4];  // [query block][d fragment]; rows d = df*16 + 4*g4 + e, column = query
    f32x4_t lacc[NQ];     // every row: the running denominator of the column's query
    float mrow[NQ];       // reference maximum of the raw scores of this lane's queries
    float mthr[NQ];       // mrow + 8 / scale_log2: scores above it move the reference
    float mbias[NQ];      // mrow * scale_log2 (0 while mrow is -inf)
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[qb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lacc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mrow[qb] = -INFINITY;
        mthr[qb] = -INFINITY;
        mbias[qb] = 0.f;
    }

    // V item c of a group: key pair kp = c / 8 and d chunk vdc = c % 8, so that eight consecutive
    // lanes read one whole 128-byte key row per load
    auto v_item = [](int c, int& kp, int& vdc) {
        kp = c >> 3;
        vdc = c & 7;
    };
    // tile loader: thread tg of a group moves KCPT 16-byte K chunks (key c/8, chunk c%8) and, for
    // VPPT V items, the 16-byte d chunks of both keys of the pair. Keys past T read row T-1 (finite
    // data): their scores are masked to -inf, so they weigh nothing.
    auto load_tile = [&](int k0, u32x4_t (&kr)[KCPT], u32x4_t (&vr)[2 * VPPT]) {
#pragma unroll
        for (int i = 0; i < KCPT; ++i) {
            const int c = tg + i * NG, kkey = c / 8, kch = c % 8;
            kr[i] = *reinterpret_cast<const u32x4_t*>(Kb + min(k0 + kkey, T - 1) * kst + kch * 8);
        }
#pragma unroll
        for (int i = 0; i < VPPT; ++i) {
            int kp, vdc;
            v_item(tg + i * NG, kp, vdc);
            const int key = k0 + 2 * kp;
            vr[2 * i] = *reinterpret_cast<const u32x4_t*>(Vb + min(key, T - 1) * vst + vdc * 8);
            vr[2 * i + 1] = *reinterpret_cast<const u32x4_t*>(Vb + min(key + 1, T - 1) * vst + vdc * 8);
        }
    };
    auto store_tile = [&](int buf, const u32x4_t (&kr)[KCPT], const u32x4_t (&vr)[2 * VPPT]) {
        uint16_t* tK = tile_k(buf, grp);
        uint16_t* tV = tile_v(buf, grp);
#pragma unroll
        for (int i = 0; i < KCPT; ++i) {
            const int c = tg + i * NG, kkey = c / 8, kch = c % 8;
            *reinterpret_cast<u32x4_t*>(&tK[kswz(kkey, kch)]) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < VPPT; ++i) {
            int kp, vdc;
            v_item(tg + i * NG, kp, vdc);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = vr[2 * i][w], bb = vr[2 * i + 1][w];  // d = vdc*8 + 2w, +1 of keys 2kp, 2kp+1
                *reinterpret_cast<uint32_t*>(&tV[(vdc * 8 + 2 * w) * VTS + 2 * kp]) = (a & 0xffffu) | (bb << 16);
                *reinterpret_cast<uint32_t*>(&tV[(vdc * 8 + 2 * w + 1) * VTS + 2 * kp]) = (a >> 16) | (bb & 0xffff0000u);
            }
        }
    };

    // step s: group g runs key tile s*G + g
    const int kend = min(T, q0 + QT);
    const int n_kt = (kend + KT - 1) / KT;
    const int n_st = (n_kt + G - 1) / G;
    u32x4_t kr[KCPT], vr[2 * VPPT];
    load_tile(grp * KT, kr, vr);
    store_tile(0, kr, vr);
    if (n_st > 1) load_tile((G + grp) * KT, kr, vr);
    __syncthreads();

    for (int st = 0; st < n_st; ++st) {
        const int kt = st * G + grp, k0 = kt * KT, buf = st & 1;
        const uint16_t* tK = tile_k(buf, grp);
        const uint16_t* tV = tile_v(buf, grp);
        if (kt < n_kt && k0 <= qw + QW - 1) {  // some key of this tile is visible to some query of this wavefront
            const bool edge = k0 + KT - 1 > qw || k0 + KT > T;  // the tile crosses the diagonal or T
            // The tile runs as two halves of 32 keys, each with its own softmax update (fewer
            // scores live at once). hh = 1 is skipped when all its keys lie above the diagonal.
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if (hh == 1 && k0 + 32 > qw + QW - 1) break;
                // S^T[key, query] for keys k0 + 32*hh .. +31 x 32 queries
                f32x4_t s[NQ][2];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const int mf = 2 * hh + m2;
                    bf16x8_t kf[2];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        kf[kk] = *reinterpret_cast<const bf16x8_t*>(&tK[kswz(mf * 16 + r16, kk * 4 + g4)]);
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        s[qb][m2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < 2; ++kk)
                            s[qb][m2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[qb][kk], s[qb][m2], 0, 0, 0);
                    }
                }
                if (edge) {
                    // key k0 + 16*mf + 4*g4 + e is visible to query qi when it is <= min(qi, T-1)
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        const int lim = min(qw + 16 * qb + r16, T - 1) - k0 - 32 * hh - 4 * g4;
#pragma unroll
                        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                            for (int e = 0; e < 4; ++e) s[qb][m2][e] = 16 * m2 + e <= lim ? s[qb][m2][e] : -INFINITY;
                    }
                }
                // The reference maximum mrow of a query moves only when one of its scores exceeds
                // it by more than 8 in log2 units (the softmax does not depend on the constant
                // subtracted, and unscaled probabilities up to 2^8 are exact enough in fp32 and
                // bf16). Each lane tests its own scores against the threshold; only when some lane
                // of the wavefront crosses it (the first tiles, then rarely) are the four lanes of
                // each query combined, the reference moved and the accumulators rescaled.
                float mloc[NQ];
                bool grow = false;
#pragma unroll
                for (int qb = 0; qb < NQ; ++qb) {
                    mloc[qb] = fmaxf(fmaxf(fmaxf(s[qb][0][0], s[qb][0][1]), fmaxf(s[qb][0][2], s[qb][0][3])),
                                     fmaxf(fmaxf(s[qb][1][0], s[qb][1][1]), fmaxf(s[qb][1][2], s[qb][1][3])));
                    grow |= mloc[qb] > mthr[qb];
                }
                if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb) {
                        const float mnew = fmaxf(mrow[qb], max_over_rows(mloc[qb]));
                        // a query with every key so far masked (only past T) keeps a zero state
                        const float alpha =
                            mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mrow[qb] - mnew) * scale_log2);
                        mrow[qb] = mnew;
                        mthr[qb] = mnew + 8.f / scale_log2;
                        mbias[qb] = mnew == -INFINITY ? 0.f : mnew * scale_log2;
#pragma unroll
                        for (int df = 0; df < 4; ++df) oacc[qb][df] *= alpha;
                        lacc[qb] *= alpha;
                    }
                }
                // P^T in the B-operand layout: slot j of a lane holds key 32*hh + 4*g4 + j (j < 4) or
                // 32*hh + 16 + 4*g4 + (j - 4); V^T fragments use the same key order
                bf16x8_t pf[NQ];
#pragma unroll
                for (int qb = 0; qb < NQ; ++qb) {
                    const float mb = mbias[qb];
                    float p[2][4];
#pragma unroll
                    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            p[m2][e] = __builtin_amdgcn_exp2f(fmaf(s[qb][m2][e], scale_log2, -mb));
                    u32x4_t pu;
                    pu[0] = pack_bf16x2(p[0][0], p[0][1]);
                    pu[1] = pack_bf16x2(p[0][2], p[0][3]);
                    pu[2] = pack_bf16x2(p[1][0], p[1][1]);
                    pu[3] = pack_bf16x2(p[1][2], p[1][3]);
                    pf[qb] = __builtin_bit_cast(bf16x8_t, pu);
                    lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb], lacc[qb], 0, 0, 0);
                }
                // O^T[d, query] += V^T[d, key] P^T[key, query], 32 keys per MFMA
#pragma unroll
                for (int df = 0; df < 4; ++df) {
                    const uint16_t* vrow = &tV[(df * 16 + r16) * VTS + 32 * hh + 4 * g4];
                    const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
                    const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16);
                    const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                    for (int qb = 0; qb < NQ; ++qb)
                        oacc[qb][df] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], oacc[qb][df], 0, 0, 0);
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
        // groups 1..G-1 hand their (accumulators, denominator, reference maximum) to group 0,
        // which rescales every part to the common maximum and adds them in group order. Merge
        // area: value j of a lane at [(group-1) * NQ*18 + j][wave][lane], so that consecutive
        // lanes write consecutive words.
        constexpr int NV = NQ * 18;
        float* part = reinterpret_cast<float*>(smem);
        auto at = [&](int g, int j) -> float& { return part[((g - 1) * NV + j) * NG + wv * 64 + lane]; };
        if (grp > 0) {
#pragma unroll
            for (int qb = 0; qb < NQ; ++qb) {
#pragma unroll
                for (int df = 0; df < 4; ++df)
#pragma unroll
                    for (int e = 0; e < 4; ++e) at(grp, qb * 18 + df * 4 + e) = oacc[qb][df][e];
                at(grp, qb * 18 + 16) = lacc[qb][0];
                at(grp, qb * 18 + 17) = mrow[qb];
            }
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) {
            float mn = mrow[qb];
#pragma unroll
            for (int g = 1; g < G; ++g) mn = fmaxf(mn, at(g, qb * 18 + 17));
            const float a0 = mrow[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mrow[qb] - mn) * scale_log2);
#pragma unroll
            for (int df = 0; df < 4; ++df) oacc[qb][df] *= a0;
            lacc[qb][0] *= a0;
#pragma unroll
            for (int g = 1; g < G; ++g) {
                const float mg = at(g, qb * 18 + 17);
                const float ag = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mg - mn) * scale_log2);
#pragma unroll
                for (int df = 0; df < 4; ++df)
#pragma unroll
                    for (int e = 0; e < 4; ++e) oacc[qb][df][e] += at(g, qb * 18 + df * 4 + e) * ag;
                lacc[qb][0] += at(g, qb * 18 + 16) * ag;
            }
        }
    }

#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
        const int qi = qw + 16 * qb + r16;
        if (qi < T) {
            const float inv = 1.0f / lacc[qb][0];
            uint16_t* Ob = O + b * osb + h * osh + qi * ost;
#pragma unroll
            for (int df = 0; df < 4; ++df) {
                uint2 u;
                u.x = pack_bf16x2(oacc[qb][df][0] * inv, oacc[qb][df][1] * inv);
                u.y = pack_bf16x2(oacc[qb][df][2] * inv, oacc[qb][df][3] * inv);
                // head dims df*16 + 4*g4 .. +3 lie in half df/2 of the head (32 dims each, osx apart)
                *reinterpret_cast<uint2*>(Ob + (df >> 1) * osx + (df & 1) * 16 + 4 * g4) = u;
            }
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
    constexpr int WAVES = 4;  // 128 queries per workgroup
    const int nqt = (T + 32 * WAVES - 1) / (32 * WAVES);
    // The causal grid is uneven (the last query tile attends to all keys). With at most two
    // workgroups per CU, two wavefront groups per workgroup split the key tiles, which halves the
    // longest workgroups; with more workgroups, one group each. Measured at T=1024, H=12: B=4
    // (384 workgroups) 22.4 us with two groups, 26.4 with one, 27.4 with four (one 16-wave
    // workgroup per CU: its wavefronts run in lock step, so MFMA and VALU work no longer overlap
    // across them); B=8 32.4 us with one group, 33.9 with two.
    const int nwg = nqt * B * H;
    const dim3 grid(nwg);
#define GPT2_ATT_LAUNCH(G)                                                                                         \
    attn_bf16_kernel<WAVES, G><<<grid, dim3(64 * WAVES * G), 0, s>>>(q, qs[0], qs[1], qs[2], k, ks[0], ks[1], ks[2], \
                                                                     v, vs[0], vs[1], vs[2], o, os[0], os[1], os[2],  \
                                                                     os_half, B, H, T, scale_log2)
    if (nwg <= 512)
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
