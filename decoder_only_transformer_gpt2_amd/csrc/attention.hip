// Causal multi-head self-attention, flash style: the [T, T] score matrix is never stored.
//   o[b,h,i,:] = sum_{j<=i} softmax_j(q_i . k_j / sqrt(64)) v_j
// ("复现GPT-2 124M" §2.1-§2.2 and "GPT-2模型架构解析与实现指南" §2.1: scores scaled by 1/sqrt(d_head),
// keys after the query masked to -inf before the softmax, the diagonal kept.)
//
// bf16 kernel. A 256-thread workgroup owns 128 queries of one (b, h); each wavefront owns 32 of
// them. Key/value tiles of 64 keys are staged in LDS (K as [key][d] with 16-byte chunks XOR-
// swizzled, V transposed to [d][key]). Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16, so each lane's accumulator column is one query: the softmax row
// statistics are then per-lane values combined over the four 16-lane groups, and the
// probabilities are already in the operand layout of the second product O^T += V^T P^T.
// Online softmax in fp32 with exp2 (scale and log2 e folded into one multiplier). Tiles wholly
// above the diagonal are skipped per wavefront; only tiles that cross it are masked. Workgroups
// are issued longest-first (last query tiles first) to even out the causal imbalance.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int QT = 128;    // queries per workgroup
constexpr int KT = 64;     // keys per LDS tile
constexpr int DH = 64;     // head size
constexpr int VTS = KT + 8;  // row stride (elements) of the transposed V tile: spreads rows over banks

__device__ __forceinline__ int kswz(int key, int chunk) { return key * DH + ((chunk ^ (key & 7)) << 3); }

__global__ __launch_bounds__(256) void attn_bf16_kernel(const uint16_t* __restrict__ Q, int64_t qsb, int64_t qsh,
                                                        int64_t qst, const uint16_t* __restrict__ K, int64_t ksb,
                                                        int64_t ksh, int64_t kst, const uint16_t* __restrict__ V,
                                                        int64_t vsb, int64_t vsh, int64_t vst, uint16_t* __restrict__ O,
                                                        int64_t osb, int64_t osh, int64_t ost, int B, int H, int T,
                                                        float scale_log2) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[KT * DH];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[DH * VTS];

    const int nqt = (T + QT - 1) / QT;
    const int bh = blockIdx.x % (B * H);
    const int qt = nqt - 1 - blockIdx.x / (B * H);
    const int b = bh / H, h = bh % H;
    const int q0 = qt * QT;
    const int t = threadIdx.x, wave = t / GPT2_WAVE, lane = t % GPT2_WAVE;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int qw = q0 + 32 * wave;

    const uint16_t* Qb = Q + b * qsb + h * qsh;
    const uint16_t* Kb = K + b * ksb + h * ksh;
    const uint16_t* Vb = V + b * vsb + h * vsh;

    // Q^T as the B operand of S^T = K Q^T: lane holds query qw + qf*16 + r16, d = kk*32 + 8*g4 .. +7
    bf16x8_t qf[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int qi = qw + f * 16 + r16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qi < T) u = *reinterpret_cast<const uint4*>(Qb + qi * qst + kk * 32 + g4 * 8);
            qf[f][kk] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    f32x4_t oacc[4][2];  // [d fragment][query fragment]; rows d = df*16 + 4*g4 + e, column query
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i][0] = oacc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrow[2] = {-INFINITY, -INFINITY};  // running max (log2 domain) of this lane's query
    float lrow[2] = {0.f, 0.f};              // this lane's share of the running denominator

    const int kend = min(T, q0 + QT);
    const int n_kt = (kend + KT - 1) / KT;
    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * KT;
        __syncthreads();  // the previous tile is no longer read
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int key = t / 8 + 32 * i, chunk = t % 8, kg = k0 + key;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (kg < T) u = *reinterpret_cast<const uint4*>(Kb + kg * kst + chunk * 8);
            *reinterpret_cast<uint4*>(&sK[kswz(key, chunk)]) = u;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int key = t % KT, dc = t / KT + 4 * i, kg = k0 + key;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (kg < T) u = *reinterpret_cast<const uint4*>(Vb + kg * vst + dc * 8);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sVt[(dc * 8 + 2 * j) * VTS + key] = (uint16_t)(w[j] & 0xffffu);
                sVt[(dc * 8 + 2 * j + 1) * VTS + key] = (uint16_t)(w[j] >> 16);
            }
        }
        __syncthreads();
        if (k0 > qw) continue;  // every key of this tile is after every query of this wavefront

        // S^T[key, query] for 64 keys x 32 queries
        f32x4_t s[4][2];
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
            s[mf][0] = s[mf][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(&sK[kswz(mf * 16 + r16, kk * 4 + g4)]);
                s[mf][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][kk], s[mf][0], 0, 0, 0);
                s[mf][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][kk], s[mf][1], 0, 0, 0);
            }
        }

        const bool edge = (k0 + KT - 1 > qw) || (k0 + KT > T);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int qi = qw + f * 16 + r16;
            float mx = -INFINITY;
#pragma unroll
            for (int mf = 0; mf < 4; ++mf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = s[mf][f][e] * scale_log2;
                    if (edge) {
                        const int key = k0 + mf * 16 + 4 * g4 + e;
                        if (key > qi || key >= T) v = -INFINITY;
                    }
                    s[mf][f][e] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, GPT2_WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 32, GPT2_WAVE));
            const float mnew = fmaxf(mrow[f], mx);
            const float alpha = __builtin_amdgcn_exp2f(mrow[f] - mnew);
            mrow[f] = mnew;
            float ls = 0.f;
#pragma unroll
            for (int mf = 0; mf < 4; ++mf)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = __builtin_amdgcn_exp2f(s[mf][f][e] - mnew);
                    s[mf][f][e] = p;
                    ls += p;
                }
            lrow[f] = lrow[f] * alpha + ls;
#pragma unroll
            for (int df = 0; df < 4; ++df) oacc[df][f] *= alpha;
        }

        // O^T[d, query] += V^T[d, key] P^T[key, query], 32 keys per MFMA. Slot j of a lane holds key
        // 32*hh + 4*g4 + j (j < 4) or 32*hh + 16 + 4*g4 + (j - 4) on both operands.
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            bf16x8_t pf[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                uint4 u;
                u.x = pack_bf16x2(s[2 * hh][f][0], s[2 * hh][f][1]);
                u.y = pack_bf16x2(s[2 * hh][f][2], s[2 * hh][f][3]);
                u.z = pack_bf16x2(s[2 * hh + 1][f][0], s[2 * hh + 1][f][1]);
                u.w = pack_bf16x2(s[2 * hh + 1][f][2], s[2 * hh + 1][f][3]);
                pf[f] = __builtin_bit_cast(bf16x8_t, u);
            }
#pragma unroll
            for (int df = 0; df < 4; ++df) {
                const uint16_t* vr = &sVt[(df * 16 + r16) * VTS + 32 * hh + 4 * g4];
                uint4 u;
                const uint2 lo = *reinterpret_cast<const uint2*>(vr);
                const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16);
                u.x = lo.x; u.y = lo.y; u.z = hi.x; u.w = hi.y;
                const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u);
                oacc[df][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0], oacc[df][0], 0, 0, 0);
                oacc[df][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[1], oacc[df][1], 0, 0, 0);
            }
        }
    }

    uint16_t* Ob = O + b * osb + h * osh;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        float l = lrow[f];
        l += __shfl_xor(l, 16, GPT2_WAVE);
        l += __shfl_xor(l, 32, GPT2_WAVE);
        const float inv = 1.0f / l;
        const int qi = qw + f * 16 + r16;
        if (qi < T) {
#pragma unroll
            for (int df = 0; df < 4; ++df) {
                uint2 u;
                u.x = pack_bf16x2(oacc[df][f][0] * inv, oacc[df][f][1] * inv);
                u.y = pack_bf16x2(oacc[df][f][2] * inv, oacc[df][f][3] * inv);
                *reinterpret_cast<uint2*>(Ob + qi * ost + df * 16 + 4 * g4) = u;
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
                          const int64_t* vs, uint16_t* o, const int64_t* os, int B, int H, int T, hipStream_t s) {
    const float scale_log2 = 0.125f * 1.4426950408889634f;  // (1/sqrt(64)) * log2(e)
    const int nqt = (T + QT - 1) / QT;
    attn_bf16_kernel<<<dim3(nqt * B * H), dim3(256), 0, s>>>(q, qs[0], qs[1], qs[2], k, ks[0], ks[1], ks[2], v, vs[0],
                                                            vs[1], vs[2], o, os[0], os[1], os[2], B, H, T, scale_log2);
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
