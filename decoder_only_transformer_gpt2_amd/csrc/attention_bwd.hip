// Causal attention backward on the matrix cores (bf16 operands, fp32 accumulation).
//   P = softmax_j(q_i . k_j / 8) over j <= i, o_i = sum_j P_ij v_j (the forward, "复现GPT-2 124M"
//   §2.1-§2.2); given dO: dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with D_i = dO_i . o_i,
//   dQ = dS K / 8, dK = dS^T Q / 8.
// Two kernels, each exact in its own accumulation order (no atomics):
//   attn_bwd_dq_mfma: a workgroup owns 64 queries of one (b, h), a wavefront 16 of them. With each
//     query's log-sum-exp (base 2) from the forward pass, it forms S^T = K Q^T, P^T, dP^T = V dO^T
//     and dS^T over the key tiles, and accumulates dQ^T += K^T dS^T. It also writes D.
//   attn_bwd_dkv_mfma: a workgroup owns 64 keys, a wavefront 16 of them; over the query tiles on
//     and after the diagonal it forms S = Q K^T, P, dP = dO V^T, dS and accumulates
//     dV^T += dO^T P and dK^T += Q^T dS.
// Both write their gradient rows in bf16 into dqkv [B*T, 3 * H * 64] (the output gradient of the
// QKV projection, whose weight and input gradients read it) and the sums of each 64-row tile's
// columns into part [B * ceil(T / 64)][3 * H * 64] (partials of that projection's bias gradient).
// With v_mfma_f32_16x16x32_bf16 a lane's accumulator holds one column (lane % 16) and rows
// 4 (lane / 16) + e; the four accumulators of a 64-row product therefore give every lane the 8
// values of its column at rows {32 h + 4 g + j, 32 h + 16 + 4 g + j} (j < 4), which is directly
// the B operand of the next product over those 32 rows; the A operand (the transposed tile) is read
// from the same [row][d] LDS tile by ds_read_b64_tr_b16 with the same row order.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int BT = 64;        // rows (queries or keys) per tile
constexpr int DHB = 64;       // head size

__device__ __forceinline__ int swz(int row, int chunk) { return row * DHB + ((chunk ^ (row & 7)) << 3); }

// Staging of 64 rows x 64 dims into a swizzled [row][d] LDS tile, split in two so that the next
// tile's global loads are in flight while the current tile is computed: fetch_* loads this
// thread's two 16-byte chunks (rows >= n zero; fp32 rows kept as loaded), put_* rounds fp32 to
// bf16 and writes them.
struct Bf16Chunks {
    u32x4_t u[2];
};
struct F32Chunks {
    f32x4_t a[2], b[2];
};
__device__ __forceinline__ void fetch_bf16(const uint16_t* __restrict__ src, long ld, int n, Bf16Chunks& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = threadIdx.x + 256 * i, r = c >> 3, ch = c & 7;
        f.u[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (r < n) f.u[i] = *reinterpret_cast<const u32x4_t*>(src + (long)r * ld + ch * 8);
    }
}
__device__ __forceinline__ void fetch_f32(const float* __restrict__ src, long ld, int n, F32Chunks& f) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = threadIdx.x + 256 * i, r = c >> 3, ch = c & 7;
        f.a[i] = f.b[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (r < n) {
            f.a[i] = *reinterpret_cast<const f32x4_t*>(src + (long)r * ld + ch * 8);
            f.b[i] = *reinterpret_cast<const f32x4_t*>(src + (long)r * ld + ch * 8 + 4);
        }
    }
}
__device__ __forceinline__ void put_chunk(const u32x4_t& u, int c, uint16_t* tile) {
    const int r = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4_t*>(&tile[swz(r, ch)]) = u;
}
__device__ __forceinline__ void put_bf16(const Bf16Chunks& f, uint16_t* tile) {
#pragma unroll
    for (int i = 0; i < 2; ++i) put_chunk(f.u[i], threadIdx.x + 256 * i, tile);
}
__device__ __forceinline__ void put_f32(const F32Chunks& f, uint16_t* tile) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
        put_chunk(u32x4_t{pack_bf16x2(f.a[i][0], f.a[i][1]), pack_bf16x2(f.a[i][2], f.a[i][3]),
                          pack_bf16x2(f.b[i][0], f.b[i][1]), pack_bf16x2(f.b[i][2], f.b[i][3])},
                  threadIdx.x + 256 * i, tile);
}

// A operand from a swizzled [row][d] tile: row, dims kk * 32 + 8 g .. + 7
__device__ __forceinline__ bf16x8_t a_rows(const uint16_t* tile, int row, int kk, int g) {
    return *reinterpret_cast<const bf16x8_t*>(&tile[swz(row, kk * 4 + g)]);
}
// A operand of the transposed tile, A[d][k] = tile[k][d], read from the swizzled [row][d] tile by
// ds_read_b64_tr_b16: lane (d = df*16 + lane%16, g = lane/16), k-slots = rows {32 h + 4 g + j, 32 h +
// 16 + 4 g + j} (j < 4). In each sixteen lanes, lane 4r + q reads dims df*16 + 4q .. +3 of row
// 32 h + 4 g + r (and of the row 16 further) and receives, transposed, dim df*16 + lane%16 of the
// four rows. The rows' chunk permutation (row & 7) is the same for both row groups.
typedef short short4_t __attribute__((vector_size(8)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
    const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}
__device__ __forceinline__ bf16x8_t a_trans(const uint16_t* tile, int df, int h, int lane) {
    const int j = lane & 15, g = lane >> 4, r = j >> 2, q = j & 3;
    const int row = 32 * h + 4 * g + r;
    const int off = row * DHB + (((2 * df + (q >> 1)) ^ (row & 7)) << 3) + 4 * (q & 1);
    const u32x2_t lo = lds_read_tr16(tile + off);
    const u32x2_t hi = lds_read_tr16(tile + off + 16 * DHB);
    return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}
// B operand over 32 rows from two accumulators (rows 4 g + e of fragments 2 h and 2 h + 1)
__device__ __forceinline__ bf16x8_t b_pack(const f32x4_t& x0, const f32x4_t& x1) {
    return __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                                                 pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])});
}
// This lane's 16 dims (kk * 32 + 8 g .. + 7, kk < 2) of a bf16 row as two B operands.
__device__ __forceinline__ void row_operand(const uint16_t* row, int g, bf16x8_t (&f)[2], bool valid) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        u32x4_t u = {0u, 0u, 0u, 0u};
        if (valid) u = *reinterpret_cast<const u32x4_t*>(row + kk * 32 + g * 8);
        f[kk] = __builtin_bit_cast(bf16x8_t, u);
    }
}

constexpr float kC2 = 0.125f * 1.4426950408889634f;  // (1 / sqrt(64)) * log2(e)

// NG gradients of one 64-row tile (lane: four dims 4 g4 .. 4 g4 + 3 of each 16-dim group df, for
// row 16 w + lane % 16; invalid rows hold zeros) to bf16 row-major out[i] (row stride 3d), and their
// column sums over the tile's rows to part[i] (64 floats each): the tile is staged in LDS (rows of
// 68 floats, so the lanes' 16-byte writes of 16 rows meet distinct banks), each thread sums 16 rows
// of one column, and the four quarter sums are added in order.
constexpr int kStg = DHB + 4;
template <int NG>
__device__ __forceinline__ void tile_grad_out(const f32x4_t (&v)[NG][4], bool valid, uint16_t* const (&out)[NG],
                                              float* const (&part)[NG], float (*stg)[64][kStg], float (*q4)[4][DHB],
                                              int w, int lane) {
    const int r16 = lane & 15, g4 = lane >> 4, row = 16 * w + r16;
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int df = 0; df < 4; ++df) {
            if (valid)
                *reinterpret_cast<u32x2_t*>(out[i] + df * 16 + 4 * g4) =
                    u32x2_t{pack_bf16x2(v[i][df][0], v[i][df][1]), pack_bf16x2(v[i][df][2], v[i][df][3])};
            *reinterpret_cast<f32x4_t*>(&stg[i][row][df * 16 + 4 * g4]) = v[i][df];
        }
    __syncthreads();
    const int c = threadIdx.x & 63, qq = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) a += stg[i][16 * qq + r][c];
        q4[i][qq][c] = a;
    }
    __syncthreads();
    if (threadIdx.x < DHB) {
#pragma unroll
        for (int i = 0; i < NG; ++i) part[i][c] = ((q4[i][0][c] + q4[i][1][c]) + q4[i][2][c]) + q4[i][3][c];
    }
}

__global__ __launch_bounds__(256) void attn_bwd_dq_mfma(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ o,
                                                        const float* __restrict__ dout, uint16_t* __restrict__ dqkv,
                                                        float* __restrict__ part,
                                                        const float* __restrict__ lse_in, float* __restrict__ d_out, int B,
                                                        int H, int T) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[BT * DHB];
    __shared__ __attribute__((aligned(16))) uint16_t sV[BT * DHB];
    const int nqb = (T + BT - 1) / BT;
    const int bh = blockIdx.x % (B * H), qb = nqb - 1 - blockIdx.x / (B * H);  // longest first
    const int b = bh / H, h = bh % H, d = H * DHB;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, r16 = lane & 15, g4 = lane >> 4;
    const int qi = qb * BT + 16 * w + r16;  // this lane's query (accumulator column)
    const bool qv = qi < T;
    const long qrow = (long)b * T + (qv ? qi : 0);
    const uint16_t* base = qkv + (long)b * T * 3 * d + h * DHB;  // q of row r at base + r * 3d

    bf16x8_t qf[2], gf[2];
    row_operand(qkv + qrow * 3 * d + h * DHB, g4, qf, qv);
    // dO row (fp32) as bf16 operands, and D = dO . o over this lane's 16 dims, then over the row
    float dd = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const float* gr = dout + qrow * d + h * DHB + kk * 32 + g4 * 8;
        const uint16_t* orow = o + qrow * d + h * DHB + kk * 32 + g4 * 8;
        f32x4_t a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
        u32x4_t ou = {0u, 0u, 0u, 0u};
        if (qv) {
            a = *reinterpret_cast<const f32x4_t*>(gr);
            c = *reinterpret_cast<const f32x4_t*>(gr + 4);
            ou = *reinterpret_cast<const u32x4_t*>(orow);
        }
        gf[kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                       pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = bf16_bits_to_f32(ou[j] & 0xffffu), hi = bf16_bits_to_f32(ou[j] >> 16);
            dd += (j < 2 ? a[2 * j] : c[2 * j - 4]) * lo + (j < 2 ? a[2 * j + 1] : c[2 * j - 3]) * hi;
        }
    }
    dd += __shfl_xor(dd, 16);
    dd += __shfl_xor(dd, 32);
    // this query's log-sum-exp (base 2, of the scores times c2), written by the forward pass
    const float lse2 = qv ? lse_in[(long)bh * T + qi] : 0.f;

    const int n_kt = qb + 1;  // key tiles up to the diagonal
    // dQ^T += K^T dS^T over the key tiles
    f32x4_t dq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dq[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    Bf16Chunks fk, fv;  // key tile kt + 1 in flight while tile kt is computed
    fetch_bf16(base + d, 3 * d, min(BT, T), fk);
    fetch_bf16(base + 2 * d, 3 * d, min(BT, T), fv);
    for (int kt = 0; kt < n_kt; ++kt) {
        const int k0 = kt * BT;
        __syncthreads();
        put_bf16(fk, sK);
        put_bf16(fv, sV);
        if (kt + 1 < n_kt) {
            const int k1 = k0 + BT, nk1 = min(BT, T - k1);
            fetch_bf16(base + d + (long)k1 * 3 * d, 3 * d, nk1, fk);
            fetch_bf16(base + 2 * d + (long)k1 * 3 * d, 3 * d, nk1, fv);
        }
        __syncthreads();
        if (k0 > qb * BT + 16 * w + 15) continue;
        f32x4_t s[4], dp[4];
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
            s[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                s[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_rows(sK, mf * 16 + r16, kk, g4), qf[kk], s[mf], 0, 0, 0);
                dp[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_rows(sV, mf * 16 + r16, kk, g4), gf[kk], dp[mf], 0, 0, 0);
            }
        }
        // dS^T = P^T * (dP^T - D), P^T = 2^(s c2 - lse2) on visible keys
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = k0 + mf * 16 + 4 * g4 + e;
                const float p = (key <= qi && key < T) ? __builtin_amdgcn_exp2f(fmaf(s[mf][e], kC2, -lse2)) : 0.f;
                s[mf][e] = p * (dp[mf][e] - dd);
            }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x8_t dsf = b_pack(s[2 * hh], s[2 * hh + 1]);
#pragma unroll
            for (int df = 0; df < 4; ++df)
                dq[df] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_trans(sK, df, hh, lane), dsf, dq[df], 0, 0, 0);
        }
    }
    if (qv && g4 == 0) d_out[(long)bh * T + qi] = dd;
    __shared__ __attribute__((aligned(16))) float stg[1][64][kStg];
    __shared__ float q4[1][4][DHB];
    f32x4_t v[1][4];
#pragma unroll
    for (int df = 0; df < 4; ++df) v[0][df] = qv ? dq[df] * 0.125f : f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint16_t* const outs[1] = {dqkv + qrow * 3 * d + h * DHB};
    float* const parts[1] = {part + ((long)b * nqb + qb) * 3 * d + h * DHB};
    tile_grad_out<1>(v, qv, outs, parts, stg, q4, w, lane);
}

__global__ __launch_bounds__(256) void attn_bwd_dkv_mfma(const uint16_t* __restrict__ qkv, const float* __restrict__ dout,
                                                         const float* __restrict__ lse, const float* __restrict__ dvec,
                                                         uint16_t* __restrict__ dqkv, float* __restrict__ part, int B,
                                                         int H, int T) {
    __shared__ __attribute__((aligned(16))) uint16_t sQ[BT * DHB];
    __shared__ __attribute__((aligned(16))) uint16_t sG[BT * DHB];
    __shared__ float sL[BT], sD[BT];
    const int nkb = (T + BT - 1) / BT;
    const int bh = blockIdx.x % (B * H), kb = blockIdx.x / (B * H);  // most query tiles first
    const int b = bh / H, h = bh % H, d = H * DHB;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, r16 = lane & 15, g4 = lane >> 4;
    const int kj = kb * BT + 16 * w + r16;  // this lane's key (accumulator column)
    const bool kv = kj < T;
    const long krow = (long)b * T + (kv ? kj : 0);
    const uint16_t* base = qkv + (long)b * T * 3 * d + h * DHB;
    const float* gbase = dout + (long)b * T * d + h * DHB;

    bf16x8_t kf[2], vf[2];
    row_operand(qkv + krow * 3 * d + d + h * DHB, g4, kf, kv);
    row_operand(qkv + krow * 3 * d + 2 * d + h * DHB, g4, vf, kv);
    f32x4_t dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dk[i] = dv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // query tile qt + 1 (q, dO, lse, D) in flight while tile qt is computed
    Bf16Chunks fq;
    F32Chunks fg;
    float fl = 0.f, fd = 0.f;
    auto fetch_q = [&](int q0) {
        const int nq = min(BT, T - q0);
        fetch_bf16(base + (long)q0 * 3 * d, 3 * d, nq, fq);
        fetch_f32(gbase + (long)q0 * d, d, nq, fg);
        if (t < BT) {
            fl = t < nq ? lse[(long)bh * T + q0 + t] : 0.f;
            fd = t < nq ? dvec[(long)bh * T + q0 + t] : 0.f;
        }
    };
    fetch_q(kb * BT);
    for (int qt = kb; qt < nkb; ++qt) {
        const int q0 = qt * BT;
        __syncthreads();
        put_bf16(fq, sQ);
        put_f32(fg, sG);
        if (t < BT) {
            sL[t] = fl;
            sD[t] = fd;
        }
        if (qt + 1 < nkb) fetch_q(q0 + BT);
        __syncthreads();
        if (q0 + BT - 1 < kb * BT + 16 * w) continue;  // wave-uniform: every query of the tile is before every key
        f32x4_t s[4], dp[4];
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
            s[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dp[mf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                s[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_rows(sQ, mf * 16 + r16, kk, g4), kf[kk], s[mf], 0, 0, 0);
                dp[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_rows(sG, mf * 16 + r16, kk, g4), vf[kk], dp[mf], 0, 0, 0);
            }
        }
        // P[q, key] and dS = P * (dP - D[q]) for visible (query, key) pairs
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int qr = mf * 16 + 4 * g4 + e, q = q0 + qr;
                const float p = (q >= kj && q < T && kv) ? __builtin_amdgcn_exp2f(fmaf(s[mf][e], kC2, -sL[qr])) : 0.f;
                s[mf][e] = p;
                dp[mf][e] = p * (dp[mf][e] - sD[qr]);
            }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x8_t pf = b_pack(s[2 * hh], s[2 * hh + 1]);
            const bf16x8_t dsf = b_pack(dp[2 * hh], dp[2 * hh + 1]);
#pragma unroll
            for (int df = 0; df < 4; ++df) {
                dv[df] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_trans(sG, df, hh, lane), pf, dv[df], 0, 0, 0);
                dk[df] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_trans(sQ, df, hh, lane), dsf, dk[df], 0, 0, 0);
            }
        }
    }
    __shared__ __attribute__((aligned(16))) float stg[2][64][kStg];
    __shared__ float q4[2][4][DHB];
    f32x4_t v[2][4];
    uint16_t* out = dqkv + krow * 3 * d + h * DHB;
    float* pp = part + ((long)b * nkb + kb) * 3 * d + h * DHB;
#pragma unroll
    for (int df = 0; df < 4; ++df) {
        v[0][df] = kv ? dk[df] * 0.125f : f32x4_t{0.f, 0.f, 0.f, 0.f};
        v[1][df] = kv ? dv[df] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    uint16_t* const outs[2] = {out + d, out + 2 * d};
    float* const parts[2] = {pp + d, pp + 2 * d};
    tile_grad_out<2>(v, kv, outs, parts, stg, q4, w, lane);
}

}  // namespace

int attention_backward_parts(int B, int T) { return B * ((T + BT - 1) / BT); }

hipError_t attention_backward_bf16(const uint16_t* qkv, const uint16_t* o, const float* dout, uint16_t* dqkv,
                                   float* part, float* lse, float* dvec, int B, int H, int T, hipStream_t s) {
    const dim3 grid((unsigned)(((T + BT - 1) / BT) * B * H)), block(256);
    attn_bwd_dq_mfma<<<grid, block, 0, s>>>(qkv, o, dout, dqkv, part, lse, dvec, B, H, T);
    attn_bwd_dkv_mfma<<<grid, block, 0, s>>>(qkv, dout, lse, dvec, dqkv, part, B, H, T);
    return hipGetLastError();
}

}  // namespace gpt2k
