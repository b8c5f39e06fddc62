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

constexpr int KT = 64;         // keys per LDS tile
constexpr int DH = 64;         // head size
constexpr int TSZ = KT * DH;   // elements of one K or V tile (8 KB)

// K and V tiles are both [key][64 dims] in LDS, the eight 16-byte chunks of each key row permuted
// by key & 7. The tiles arrive by LDS DMA (global_load_lds, 16 bytes per lane, a 1 KB block of
// eight key rows per instruction); lane L of a block writes the LDS slot L, i.e. key row L / 8,
// stored chunk L % 8, so it fetches source chunk (L % 8) ^ (L / 8). Reads:
//  * K fragments (16 bytes per lane, sixteen consecutive keys x one chunk): 16-byte reads are
//    served sixteen lanes at a time over 64 banks, the sixteen being lanes 0-7 with 24-31 and 8-15
//    with 16-23; the key & 7 permutation puts each sixteen on distinct banks;
//  * V^T fragments by ds_read_b64_tr_b16: in each group of sixteen lanes, lane 4r + q reads the
//    four dims 4q .. 4q+3 of key row r of a four-key group and receives, transposed, four
//    consecutive keys of one dimension (lane i: dim i of the sixteen) -- the A operand of
//    O^T += V^T P^T. Thirty-two lanes read eight key rows x 32 bytes; under the permutation they
//    fall on distinct banks (8-byte accesses are served 32 lanes at a time over 64 banks).
__device__ __forceinline__ int kvswz(int key, int chunk) { return key * DH + ((chunk ^ (key & 7)) << 3); }
// Maximum over the four lanes L, L^16, L^32, L^48 (the four 16-lane rows). Only the rare
// rescale path needs it. (The gfx950 row-swap builtins would avoid the LDS crossbar, but this
// toolchain miscompiles them when both operands are the same value.)
__device__ __forceinline__ float max_over_rows(float m) {
    m = fmaxf(m, __shfl_xor(m, 16, GPT2_WAVE));
    return fmaxf(m, __shfl_xor(m, 32, GPT2_WAVE));
}

// s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(0): every vector memory access of this wavefront (the LDS
// DMA included) and every LDS access has completed
constexpr int kWaitAllMem = 0x0070;
typedef short short4_t __attribute__((vector_size(8)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
    const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}
__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* lds_block) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_block), 16, 0, 0);
}

// Register budget: with two groups (eight wavefronts, 64 KB of LDS) two workgroups share a CU only
// at 128 VGPRs (four waves per SIMD); with one group, three 4-wave workgroups per CU (three waves per
// SIMD) fill the CUs at B*H = 96, and the 168 VGPRs this allows remove the spills (B=8 H=12 T=1024:
// 25.3 -> 23.6 us).
// LSE: also write each query's base-2 log-sum-exp of the scaled scores, log2 sum_j 2^(c s_j), summed
// in fp32 over the unrounded probabilities (what the backward pass needs to form P again).
template <int WAVES, int G, bool LSE>  // 32 queries per wavefront; G groups of WAVES wavefronts share the queries
__global__ __launch_bounds__(64 * WAVES * G, G == 1 ? 3 : 4) void attn_bf16_kernel(
    const uint16_t* __restrict__ Q, int64_t qsb, int64_t qsh, int64_t qst, const uint16_t* __restrict__ K, int64_t ksb,
    int64_t ksh, int64_t kst, const uint16_t* __restrict__ V, int64_t vsb, int64_t vsh, int64_t vst,
    uint16_t* __restrict__ O, int64_t osb, int64_t osh, int64_t ost, int64_t osx, int B, int H, int T,
    float scale_log2, int n_lone, float* __restrict__ lse_out) {
    static_assert(WAVES == 4, "each wavefront of a group moves two of the eight 1 KB blocks of a K or V tile");
    constexpr int NQ = 2, QW = 16 * NQ;  // 16-query column blocks and queries per wavefront
    constexpr int QT = QW * WAVES, NG = 64 * WAVES;
    constexpr int BUF = G * 2 * TSZ;     // one ring slot: [group][K, V]
    constexpr int NVQ = LSE ? 19 : 18;   // merge values per lane and query block (accumulators, denominator,
                                         // maximum, fp32 sum)
    static_assert((G - 1) * NVQ * NG * 4 <= BUF * 2, "merge area of one query block fits one ring slot");
    // two ring slots as two objects, so that the compiler can tell the slot being read from the slot
    // the DMA is filling
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[BUF];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[BUF];

    const int nqt = (T + QT - 1) / QT;
    // Work unit u: query tiles longest first (u / (B*H) counts down from the last query tile).
    // Workgroups are dispatched one per CU before any CU gets a second, and workgroup n_cu + i shares
    // CU i with workgroup i. With n_lone CUs holding one workgroup (and n_pair = nwg - n_cu CUs two),
    // the longest units go alone (ids n_pair .. n_cu-1) and the pairs match the next longest with
    // the shortest (ids i and n_cu + i). n_lone = 0: plain longest-first order.
    int u = blockIdx.x;
    if (n_lone > 0) {
        const int nwg = (int)gridDim.x, n_pair = nwg - (n_lone + (nwg - n_lone) / 2), n_cu = n_lone + n_pair;
        const int bid = blockIdx.x;
        u = bid >= n_cu ? nwg - 1 - (bid - n_cu) : bid >= n_pair ? bid - n_pair : n_lone + bid;
    }
    const int bh = u % (B * H);
    const int qt = nqt - 1 - u / (B * H);
    const int b = bh / H, h = bh % H;
    const int q0 = qt * QT;
    const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t / GPT2_WAVE), lane = t % GPT2_WAVE;
    const int grp = wave / WAVES, wv = wave % WAVES;  // group and wavefront in the group
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

    f32x4_t oacc[NQ][4];  // [query block][d fragment]; rows d = df*16 + 4*g4 + e, column = query
    f32x4_t lacc[NQ];     // every row: the running denominator of the column's query
    float mrow[NQ];       // reference maximum of the raw scores of this lane's queries
    float mthr[NQ];       // mrow + 8 / scale_log2: scores above it move the reference
    float mbias[NQ];      // mrow * scale_log2 (0 while mrow is -inf)
    float lsum[NQ];       // (LSE) fp32 sum of this lane's unrounded probabilities, relative to mrow
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
        lsum[qb] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[qb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lacc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mrow[qb] = -INFINITY;
        mthr[qb] = -INFINITY;
        mbias[qb] = 0.f;
    }

    const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_u);

    // DMA: wavefront wv of a group moves blocks 2wv and 2wv+1 (key rows 16wv .. 16wv+15) of the K
    // and the V tile. Keys past T read row T-1 (finite data): their scores are masked to -inf, so
    // they weigh nothing.
    const int drow = 16 * wv + (lane >> 3);
    const int dch8 = ((lane & 7) ^ (lane >> 3)) * 8;
    const int64_t koff = (int64_t)drow * kst + dch8, voff = (int64_t)drow * vst + dch8;
    auto issue = [&](uint16_t* slot, int k0) __attribute__((always_inline)) {
        uint16_t* tK = slot + grp * 2 * TSZ + 2 * wv * 512;
        uint16_t* tV = tK + TSZ;
        if (k0 + KT <= T) {
            const uint16_t* ks = Kb + (int64_t)k0 * kst + koff;
            const uint16_t* vs = Vb + (int64_t)k0 * vst + voff;
            lds_dma16(ks, tK);
            lds_dma16(ks + 8 * kst, tK + 512);
            lds_dma16(vs, tV);
            lds_dma16(vs + 8 * vst, tV + 512);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int key = min(k0 + drow + 8 * i, T - 1);
                lds_dma16(Kb + (int64_t)key * kst + dch8, tK + i * 512);
                lds_dma16(Vb + (int64_t)key * vst + dch8, tV + i * 512);
            }
        }
    };

    // V^T fragment reads: lane 4r + q of each sixteen reads dims 4q..4q+3 of key 4*g4 + r of a
    // 16-key group; per d fragment df the chunk is (2df + q/2) ^ (key & 7) (key & 7 does not depend
    // on which 16-key group), so the four per-lane offsets are fixed and the group moves them by
    // whole 16-key strides (immediate offsets)
    int vtr[4];
    {
        const int r = r16 >> 2, q = r16 & 3, key = 4 * g4 + r;
#pragma unroll
        for (int df = 0; df < 4; ++df) vtr[df] = key * DH + (((2 * df + (q >> 1)) ^ (key & 7)) << 3) + 4 * (q & 1);
    }

    // step s: group g runs key tile s*G + g
    const int kend = min(T, q0 + QT);
    const int n_kt = (kend + KT - 1) / KT;
    const int n_st = (n_kt + G - 1) / G;

    auto compute = [&](const uint16_t* slot, int st) __attribute__((always_inline)) {
        const int kt = st * G + grp, k0 = kt * KT;
        const uint16_t* tK = slot + grp * 2 * TSZ;
        const uint16_t* tV = tK + TSZ;
        if (!(kt < n_kt && k0 <= qw + QW - 1)) return;  // no key of this tile is visible to this wavefront
        const bool edge = k0 + KT - 1 > qw || k0 + KT > T;  // the tile crosses the diagonal or T
        // The tile runs as two halves of 32 keys, each with its own softmax update (fewer scores
        // live at once). hh = 1 is skipped when all its keys lie above the diagonal.
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
                    kf[kk] = *reinterpret_cast<const bf16x8_t*>(&tK[kvswz(mf * 16 + r16, kk * 4 + g4)]);
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
            // The reference maximum mrow of a query moves only when one of its scores exceeds it
            // by more than 8 in log2 units (the softmax does not depend on the constant
            // subtracted, and unscaled probabilities up to 2^8 are exact enough in fp32 and bf16).
            // Each lane tests its own scores against the threshold; only when some lane of the
            // wavefront crosses it (the first tiles, then rarely) are the four lanes of each query
            // combined, the reference moved and the accumulators rescaled.
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
                    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mrow[qb] - mnew) * scale_log2);
                    mrow[qb] = mnew;
                    mthr[qb] = mnew + 8.f / scale_log2;
                    mbias[qb] = mnew == -INFINITY ? 0.f : mnew * scale_log2;
#pragma unroll
                    for (int df = 0; df < 4; ++df) oacc[qb][df] *= alpha;
                    lacc[qb] *= alpha;
                    if (LSE) lsum[qb] *= alpha;
                }
            }
            // P^T in the B-operand layout: slot j of a lane holds key 32*hh + 4*g4 + j (j < 4) or
            // 32*hh + 16 + 4*g4 + (j - 4); the V^T fragments use the same key order
            bf16x8_t pf[NQ];
#pragma unroll
            for (int qb = 0; qb < NQ; ++qb) {
                const float mb = mbias[qb];
                float p[2][4];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) p[m2][e] = __builtin_amdgcn_exp2f(fmaf(s[qb][m2][e], scale_log2, -mb));
                if (LSE)
                    lsum[qb] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
                u32x4_t pu;
                pu[0] = pack_bf16x2(p[0][0], p[0][1]);
                pu[1] = pack_bf16x2(p[0][2], p[0][3]);
                pu[2] = pack_bf16x2(p[1][0], p[1][1]);
                pu[3] = pack_bf16x2(p[1][2], p[1][3]);
                pf[qb] = __builtin_bit_cast(bf16x8_t, pu);
                lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qb], lacc[qb], 0, 0, 0);
            }
            // O^T[d, query] += V^T[d, key] P^T[key, query], 32 keys per MFMA; the transposing
            // reads take keys 32hh + 4*g4 + 0..3 (low) and 32hh + 16 + 4*g4 + 0..3 (high)
#pragma unroll
            for (int df = 0; df < 4; ++df) {
                const u32x2_t lo = lds_read_tr16(tV + vtr[df] + (32 * hh) * DH);
                const u32x2_t hi = lds_read_tr16(tV + vtr[df] + (32 * hh + 16) * DH);
                const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
                for (int qb = 0; qb < NQ; ++qb)
                    oacc[qb][df] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], oacc[qb][df], 0, 0, 0);
            }
        }
    };

    // Step st reads ring slot st & 1. It waits for its own DMAs of that slot and meets the other
    // wavefronts (their DMAs have landed too, and nobody still reads the other slot, which step
    // st-1 used), starts the DMA of step st+1 into the other slot, then computes.
    issue(lds0, grp * KT);
    auto step = [&](auto slot_c, int st) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot_c)::value;
        uint16_t* cur = SL == 0 ? lds0 : lds1;
        uint16_t* nxt = SL == 0 ? lds1 : lds0;
        __builtin_amdgcn_s_waitcnt(kWaitAllMem);
        __builtin_amdgcn_s_barrier();
        if (st + 1 < n_st) issue(nxt, ((st + 1) * G + grp) * KT);
        compute(cur, st);
    };
    for (int st = 0; st < n_st; st += 2) {
        step(std::integral_constant<int, 0>{}, st);
        if (st + 1 < n_st) step(std::integral_constant<int, 1>{}, st + 1);
    }

    if constexpr (G > 1) {
        // groups 1..G-1 hand their (accumulators, denominator, reference maximum, fp32 sum) to
        // group 0, which rescales every part to the common maximum and adds them in group order.
        // Merge area: value j of query block qb of a lane at [(group-1) * NVQ + j][wave][lane] of
        // ring slot qb, so that consecutive lanes write consecutive words.
        __builtin_amdgcn_s_waitcnt(kWaitAllMem);
        __syncthreads();  // every wavefront is done with the ring
        auto at = [&](int qb, int g, int j) -> float& {
            float* part = reinterpret_cast<float*>(qb == 0 ? lds0 : lds1);
            return part[((g - 1) * NVQ + j) * NG + wv * 64 + lane];
        };
        if (grp > 0) {
#pragma unroll
            for (int qb = 0; qb < NQ; ++qb) {
#pragma unroll
                for (int df = 0; df < 4; ++df)
#pragma unroll
                    for (int e = 0; e < 4; ++e) at(qb, grp, df * 4 + e) = oacc[qb][df][e];
                at(qb, grp, 16) = lacc[qb][0];
                at(qb, grp, 17) = mrow[qb];
                if (LSE) at(qb, grp, 18) = lsum[qb];
            }
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) {
            float mn = mrow[qb];
#pragma unroll
            for (int g = 1; g < G; ++g) mn = fmaxf(mn, at(qb, g, 17));
            const float a0 = mrow[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mrow[qb] - mn) * scale_log2);
#pragma unroll
            for (int df = 0; df < 4; ++df) oacc[qb][df] *= a0;
            lacc[qb][0] *= a0;
            if (LSE) lsum[qb] *= a0;
#pragma unroll
            for (int g = 1; g < G; ++g) {
                const float mg = at(qb, g, 17);
                const float ag = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mg - mn) * scale_log2);
#pragma unroll
                for (int df = 0; df < 4; ++df)
#pragma unroll
                    for (int e = 0; e < 4; ++e) oacc[qb][df][e] += at(qb, g, df * 4 + e) * ag;
                lacc[qb][0] += at(qb, g, 16) * ag;
                if (LSE) lsum[qb] += at(qb, g, 18) * ag;
            }
            mrow[qb] = mn;  // the reference of the merged state
        }
    }

    if constexpr (LSE) {
        // the four lanes of a query (g4 = 0..3) hold disjoint keys: add their sums
#pragma unroll
        for (int qb = 0; qb < NQ; ++qb) {
            float tot = lsum[qb];
            tot += __shfl_xor(tot, 16, GPT2_WAVE);
            tot += __shfl_xor(tot, 32, GPT2_WAVE);
            const int qi = qw + 16 * qb + r16;
            if (g4 == 0 && qi < T) lse_out[(int64_t)bh * T + qi] = mrow[qb] * scale_log2 + __log2f(tot);
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

// Compute units of the current device (cached per device; 0 when the query fails).
int cu_count() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

hipError_t attention_bf16(const uint16_t* q, const int64_t* qs, const uint16_t* k, const int64_t* ks, const uint16_t* v,
                          const int64_t* vs, uint16_t* o, const int64_t* os, int B, int H, int T, hipStream_t s,
                          int64_t os_half, float* lse_out) {
    const float scale_log2 = 0.125f * 1.4426950408889634f;  // (1/sqrt(64)) * log2(e)
    constexpr int WAVES = 4;  // 128 queries per workgroup
    const int nqt = (T + 32 * WAVES - 1) / (32 * WAVES);
    // The causal grid is uneven (the last query tile attends to all keys). With at most two
    // workgroups per CU, two wavefront groups per workgroup split the key tiles, which halves the
    // longest workgroups; with more workgroups, one group each. Measured at T=1024, H=12 (with the
    // register-staged tiles this kernel had before): B=4 (384 workgroups) 22.4 us with two groups,
    // 26.4 with one, 27.4 with four (one 16-wave workgroup per CU: its wavefronts run in lock step,
    // so MFMA and VALU work no longer overlap across them); B=8 32.4 us with one group, 33.9 with
    // two. Now: B=4 18.3 us, B=8 23.6 us.
    const int nwg = nqt * B * H;
    const int n_cu = cu_count();
    const dim3 grid(nwg);
#define GPT2_ATT_LAUNCH1(G, LSE, LONE)                                                                             \
    attn_bf16_kernel<WAVES, G, LSE><<<grid, dim3(64 * WAVES * G), 0, s>>>(                                         \
        q, qs[0], qs[1], qs[2], k, ks[0], ks[1], ks[2], v, vs[0], vs[1], vs[2], o, os[0], os[1], os[2], os_half, B, H, \
        T, scale_log2, LONE, lse_out)
#define GPT2_ATT_LAUNCH(G, LONE)          \
    do {                                  \
        if (lse_out)                      \
            GPT2_ATT_LAUNCH1(G, true, LONE);  \
        else                              \
            GPT2_ATT_LAUNCH1(G, false, LONE); \
    } while (0)
    if (nwg <= 2 * n_cu) {
        // two workgroups fit a CU: n_cu - (nwg - n_cu) CUs get one
        GPT2_ATT_LAUNCH(2, nwg > n_cu ? 2 * n_cu - nwg : 0);
    } else {
        GPT2_ATT_LAUNCH(1, 0);
    }
#undef GPT2_ATT_LAUNCH
#undef GPT2_ATT_LAUNCH1
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
