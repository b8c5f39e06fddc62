// Kernels of the backward pass of the shifted next-token cross-entropy ("从零手写GPT-2：PyTorch实现
// Transformer解码器核心模块" §4: the loss and loss.backward(); §2.2: the tied wte receives both the
// lm_head gradient and the embedding gradient). The matrix products of the backward are the
// library's GEMM (C = A B^T, both operands K-contiguous) on transposed copies made here.
#include "common.h"

namespace gpt2k {
namespace {

template <bool BF>
struct Act;
template <>
struct Act<true> {
    using T = uint16_t;
    static __device__ __forceinline__ float load(const T* p, long i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(T* p, long i, float v) { p[i] = f32_to_bf16_bits(v); }
};
template <>
struct Act<false> {
    using T = float;
    static __device__ __forceinline__ float load(const T* p, long i) { return p[i]; }
    static __device__ __forceinline__ void store(T* p, long i, float v) { p[i] = v; }
};

// ------------------------------------------------------------------------------ transpose
// dst[c * ldd + r] = src[r * lds + c] for r < R, c < C, and 0 for R <= r < Rp (64x64 tiles via LDS).
template <bool SRC_BF, bool DST_BF>
__global__ void __launch_bounds__(256) transpose_kernel(const void* __restrict__ src, long lds, int R, int C,
                                                        void* __restrict__ dst, long ldd, int Rp) {
    __shared__ float tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, t = threadIdx.x;
    const auto* s = static_cast<const typename Act<SRC_BF>::T*>(src);
    auto* d = static_cast<typename Act<DST_BF>::T*>(dst);
    for (int e = t; e < 64 * 64; e += 256) {
        const int rr = e >> 6, cc = e & 63, r = r0 + rr, c = c0 + cc;
        tile[rr][cc] = (r < R && c < C) ? Act<SRC_BF>::load(s, (long)r * lds + c) : 0.f;
    }
    __syncthreads();
    for (int e = t; e < 64 * 64; e += 256) {
        const int cc = e >> 6, rr = e & 63, r = r0 + rr, c = c0 + cc;
        if (c < C && r < Rp) Act<DST_BF>::store(d, (long)c * ldd + r, tile[rr][cc]);
    }
}

// bf16 or fp32 -> bf16 with 16-byte accesses on both sides (row strides and pointers 16-byte
// aligned): a thread moves two 8-column pieces of source rows into the tile and two 8-row pieces
// of destination rows out of it; element by element only where a piece crosses R, C or Rp. The
// 65-float tile rows keep both the row writes and the column reads of a wavefront on distinct
// banks. The values are the same bits as transpose_kernel's (fp32 sources round to nearest even).
template <bool SRC_BF>
__global__ void __launch_bounds__(256) transpose_vec_kernel(const void* __restrict__ srcv, long lds, int R, int C,
                                                            uint16_t* __restrict__ dst, long ldd, int Rp) {
    __shared__ float tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = t + i * 256, rr = e >> 3, ck = (e & 7) * 8, r = r0 + rr, c = c0 + ck;
        float v[8];
        if (r < R && c + 8 <= C) {
            if constexpr (SRC_BF) {
                const u32x4_t u = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(srcv) + (long)r * lds + c);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = __uint_as_float(u[j] << 16);
                    v[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
                }
            } else {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(srcv) + (long)r * lds + c);
                const float4 a = p[0], b = p[1];
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = (r < R && c + j < C) ? Act<SRC_BF>::load(static_cast<const typename Act<SRC_BF>::T*>(srcv),
                                                                (long)r * lds + c + j)
                                            : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[rr][ck + j] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = t + i * 256, cc = e >> 3, rk = (e & 7) * 8, c = c0 + cc, r = r0 + rk;
        if (c >= C) continue;
        uint16_t* dp = dst + (long)c * ldd + r;
        if (r + 8 <= Rp) {
            u32x4_t u;
#pragma unroll
            for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(tile[rk + 2 * j][cc], tile[rk + 2 * j + 1][cc]);
            *reinterpret_cast<u32x4_t*>(dp) = u;
        } else {
            for (int j = 0; j < 8 && r + j < Rp; ++j) dp[j] = f32_to_bf16_bits(tile[rk + j][cc]);
        }
    }
}

// ------------------------------------------------------------------------------ column sums
// part[b][c] = sum of src[r][c] over the 256 rows r of block b: four row groups of 64 rows per
// column (eight loads in flight per thread), combined in group order.
constexpr int kColRows = 256;
__global__ void __launch_bounds__(256) colsum_partial_kernel(const float* __restrict__ src, long ld, int R, int C,
                                                             float* __restrict__ part) {
    __shared__ float acc4[4][64];
    const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6, c = blockIdx.x * 64 + cl, b = blockIdx.y;
    const int r0 = b * kColRows + grp * 64, r1 = min(R, r0 + 64);
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < C) {
        int r = r0;
        for (; r + 8 <= r1; r += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += src[(long)(r + u) * ld + c];
        }
        for (; r < r1; ++r) a[0] += src[(long)r * ld + c];
    }
    acc4[grp][cl] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (grp == 0 && c < C) part[(long)b * C + c] = ((acc4[0][cl] + acc4[1][cl]) + acc4[2][cl]) + acc4[3][cl];
}
// out[c] = sum over b < nb of part[b][c]: a workgroup owns 16 columns and splits the partial rows
// into 16 groups (eight loads in flight per thread), combined in group order, so short column
// ranges (d = 768) still spread over 48 workgroups.
constexpr int kRedCols = 16, kRedGroups = 16;
__global__ void __launch_bounds__(256) colsum_reduce_kernel(const float* __restrict__ part, int nb, int C,
                                                            float* __restrict__ out) {
    __shared__ float accg[kRedGroups][kRedCols];
    const int cl = threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols, c = blockIdx.x * kRedCols + cl;
    const int per = (nb + kRedGroups - 1) / kRedGroups, b0 = grp * per, b1 = min(nb, b0 + per);
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < C) {
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += part[(long)(b + u) * C + c];
        }
        for (; b < b1; ++b) a[0] += part[(long)b * C + c];
    }
    accg[grp][cl] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (grp == 0 && c < C) {
        float sum = 0.f;
#pragma unroll
        for (int g = 0; g < kRedGroups; ++g) sum += accg[g][cl];
        out[c] = sum;
    }
}

// colsum_reduce_kernel over several independent segments: blockIdx.y picks the segment, the column
// blocks past its C return at once. Same per-column order as colsum_reduce_kernel.
__global__ void __launch_bounds__(256) colsum_reduce_multi_kernel(const ColsumSegs segs) {
    __shared__ float accg[kRedGroups][kRedCols];
    const ColsumSeg sg = segs.seg[blockIdx.y];
    if ((int)blockIdx.x * kRedCols >= sg.C) return;
    const int cl = threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols, c = blockIdx.x * kRedCols + cl;
    const int per = (sg.nb + kRedGroups - 1) / kRedGroups, b0 = grp * per, b1 = min(sg.nb, b0 + per);
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < sg.C) {
        int b = b0;
        for (; b + 8 <= b1; b += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) a[u] += sg.part[(long)(b + u) * sg.C + c];
        }
        for (; b < b1; ++b) a[0] += sg.part[(long)b * sg.C + c];
    }
    accg[grp][cl] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (grp == 0 && c < sg.C) {
        float sum = 0.f;
#pragma unroll
        for (int g = 0; g < kRedGroups; ++g) sum += accg[g][cl];
        sg.out[c] = sum;
    }
}

// ------------------------------------------------------------------------------ LayerNorm backward
// One block per kLnRows rows. For each row: xhat = (x - mean) * rstd, g = dy * gamma,
// dx += rstd * (g - mean(g) - xhat * mean(g * xhat)). The block sums dy * xhat and dy per column over
// its rows and writes them as partial row blockIdx.x of pg / pb [blocks][d]. With y16 the new dx is
// also written in bf16 (row stride d) and its per-column sums as partial row blockIdx.x of pd: the
// output gradient of the projection before this LayerNorm, with its bias gradient's partials.
constexpr int kLnRows = 16, kLnWaves = 8;

// CPL > 0 (d = 64 * CPL): kLnWaves wavefronts, one row at a time each (eight waves for two rows each:
// with four waves per CU the loads in flight did not cover the memory latency), the row and the column
// sums held in registers (lane l owns columns l + 64 j), the waves' sums added in wave order through LDS.
// CPL = 0 (any d, a multiple of 64): one wavefront takes the block's rows in order, re-reading the row
// and accumulating in its partial rows.
template <int CPL>
__global__ void __launch_bounds__(64 * kLnWaves) ln_backward_kernel(const float* __restrict__ x,
                                                                    const float* __restrict__ gamma,
                                                                    const float* __restrict__ dy, float* __restrict__ dx,
                                                                    int M, int d, float eps, float* __restrict__ pg,
                                                                    float* __restrict__ pb, uint16_t* __restrict__ y16,
                                                                    float* __restrict__ pd) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, blk = blockIdx.x;
    float* og = pg + (long)blk * d;
    float* ob = pb + (long)blk * d;
    float* od = y16 ? pd + (long)blk * d : nullptr;
    const float inv_d = 1.0f / (float)d;
    if constexpr (CPL > 0) {
        float ag[CPL], ab[CPL], ad[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) ag[j] = ab[j] = ad[j] = 0.f;
        // the next row's x, dy and dx are loaded while this row is processed
        float xv[CPL], gv[CPL], dv[CPL];
        auto load_row = [&](int m, float* xa, float* ga, float* da) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                xa[j] = x[(long)m * d + lane + 64 * j];
                ga[j] = dy[(long)m * d + lane + 64 * j];
                da[j] = dx[(long)m * d + lane + 64 * j];
            }
        };
        if (blk * kLnRows + w < M) load_row(blk * kLnRows + w, xv, gv, dv);
#pragma unroll
        for (int rr = w; rr < kLnRows; rr += kLnWaves) {
            const int m = blk * kLnRows + rr;
            if (m >= M) break;
            float* dr = dx + (long)m * d;
            float xn[CPL], gn[CPL], dn[CPL];
            const bool has_next = rr + kLnWaves < kLnRows && m + kLnWaves < M;
            if (has_next) load_row(m + kLnWaves, xn, gn, dn);
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) s += xv[j];
            const float mean = wave_sum(s) * inv_d;
            float q = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) q += (xv[j] - mean) * (xv[j] - mean);
            const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + eps);
            float sg = 0.f, sgx = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                xv[j] = (xv[j] - mean) * rstd;
                const float g = gv[j] * gamma[lane + 64 * j];
                sg += g;
                sgx += g * xv[j];
            }
            const float mg = wave_sum(sg) * inv_d, mgx = wave_sum(sgx) * inv_d;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + 64 * j;
                const float g = gv[j] * gamma[c];
                const float nv = dv[j] + rstd * (g - mg - xv[j] * mgx);
                dr[c] = nv;
                if (y16) {
                    y16[(long)m * d + c] = f32_to_bf16_bits(nv);
                    ad[j] += nv;
                }
                ag[j] += gv[j] * xv[j];
                ab[j] += gv[j];
            }
            if (has_next) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    xv[j] = xn[j];
                    gv[j] = gn[j];
                    dv[j] = dn[j];
                }
            }
        }
        // one sum at a time through a [waves][d] buffer, added in wave order
        __shared__ float red[kLnWaves][CPL * 64];
        auto block_sum = [&](const float* a, float* out) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) red[w][lane + 64 * j] = a[j];
            __syncthreads();
            for (int c = threadIdx.x; c < d; c += 64 * kLnWaves) {
                float t = red[0][c];
#pragma unroll
                for (int v = 1; v < kLnWaves; ++v) t += red[v][c];
                out[c] = t;
            }
            __syncthreads();
        };
        block_sum(ag, og);
        block_sum(ab, ob);
        if (od) block_sum(ad, od);
    } else {
        for (int c = lane; c < d; c += 64) {
            og[c] = ob[c] = 0.f;
            if (od) od[c] = 0.f;
        }
        for (int rr = 0; rr < kLnRows; ++rr) {
            const int m = blk * kLnRows + rr;
            if (m >= M) break;
            const float* xr = x + (long)m * d;
            const float* gr = dy + (long)m * d;
            float* dr = dx + (long)m * d;
            float s = 0.f;
            for (int c = lane; c < d; c += 64) s += xr[c];
            const float mean = wave_sum(s) * inv_d;
            float q = 0.f;
            for (int c = lane; c < d; c += 64) q += (xr[c] - mean) * (xr[c] - mean);
            const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + eps);
            float sg = 0.f, sgx = 0.f;
            for (int c = lane; c < d; c += 64) {
                const float xh = (xr[c] - mean) * rstd, g = gr[c] * gamma[c];
                sg += g;
                sgx += g * xh;
            }
            const float mg = wave_sum(sg) * inv_d, mgx = wave_sum(sgx) * inv_d;
            for (int c = lane; c < d; c += 64) {
                const float xh = (xr[c] - mean) * rstd, g = gr[c] * gamma[c];
                const float nv = dr[c] + rstd * (g - mg - xh * mgx);
                dr[c] = nv;
                if (y16) {
                    y16[(long)m * d + c] = f32_to_bf16_bits(nv);
                    od[c] += nv;
                }
                og[c] += gr[c] * xh;
                ob[c] += gr[c];
            }
        }
    }
}

// ------------------------------------------------------------------------------ GELU
// (gelu_tanh_grad / gelu_erf_grad: common.h)
// h = gelu(u) in the compute dtype (the values the fused forward epilogue produces from the same u)
template <bool BF>
__global__ void gelu_forward_kernel(const float* __restrict__ u, void* __restrict__ h, long n, int erf_form) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float x = u[i];
    Act<BF>::store(static_cast<typename Act<BF>::T*>(h), i, erf_form ? gelu_erf_f32(x) : gelu_tanh_fast(x));
}
// g = g * gelu'(u), in place
__global__ void gelu_backward_kernel(const float* __restrict__ u, float* __restrict__ g, long n, int erf_form) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    g[i] *= erf_form ? gelu_erf_grad(u[i]) : gelu_tanh_grad(u[i]);
}
// The same four values per thread (16-byte accesses), n4 = n / 4.
__global__ void gelu_backward_x4_kernel(const float4* __restrict__ u, float4* __restrict__ g, long n4, int erf_form) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 x = u[i];
    float4 y = g[i];
    if (erf_form) {
        y.x *= gelu_erf_grad(x.x); y.y *= gelu_erf_grad(x.y); y.z *= gelu_erf_grad(x.z); y.w *= gelu_erf_grad(x.w);
    } else {
        y.x *= gelu_tanh_grad(x.x); y.y *= gelu_tanh_grad(x.y); y.z *= gelu_tanh_grad(x.z); y.w *= gelu_tanh_grad(x.w);
    }
    g[i] = y;
}
// gelu_forward_kernel with four values per thread (16-byte reads), n4 = n / 4.
template <bool BF>
__global__ void gelu_forward_x4_kernel(const float4* __restrict__ u, void* __restrict__ h, long n4, int erf_form) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 x = u[i];
    float4 y;
    if (erf_form) {
        y.x = gelu_erf_f32(x.x); y.y = gelu_erf_f32(x.y); y.z = gelu_erf_f32(x.z); y.w = gelu_erf_f32(x.w);
    } else {
        y.x = gelu_tanh_fast(x.x); y.y = gelu_tanh_fast(x.y); y.z = gelu_tanh_fast(x.z); y.w = gelu_tanh_fast(x.w);
    }
    if constexpr (BF)
        static_cast<uint2*>(h)[i] = make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
    else
        static_cast<float4*>(h)[i] = y;
}

// ------------------------------------------------------------------------------ cross-entropy
// cnt[0] = number of rows with tgt >= 0.
__global__ void __launch_bounds__(256) count_targets_kernel(const int32_t* __restrict__ tgt, int M, int32_t* cnt) {
    __shared__ int part[4];
    int n = 0;
    for (int m = threadIdx.x; m < M; m += 256) n += tgt[m] >= 0;
    for (int o = 32; o; o >>= 1) n += __shfl_xor(n, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = n;
    __syncthreads();
    if (threadIdx.x == 0) cnt[0] = part[0] + part[1] + part[2] + part[3];
}

// One workgroup per row m of the fp32 logits: lse = log sum exp, nll[m] = lse - z[tgt] (0 when the
// row has no target), and the loss gradient row (exp(z - lse) - [v = tgt]) / n_counted in the
// compute dtype, zero for rows without target and for the padding columns V <= v < Vp.
template <bool BF>
__global__ void __launch_bounds__(256) xent_grad_kernel(const float* __restrict__ logits, long ld, int V, int Vp,
                                                        const int32_t* __restrict__ tgt, const int32_t* __restrict__ cnt,
                                                        float* __restrict__ nll, void* __restrict__ dlogits) {
    __shared__ float sm[4], ss[4];
    const int m = blockIdx.x, t = threadIdx.x;
    const float* z = logits + (long)m * ld;
    const int y = tgt[m];
    auto* out = static_cast<typename Act<BF>::T*>(dlogits) + (long)m * Vp;
    if (y < 0) {
        for (int v = t; v < Vp; v += 256) Act<BF>::store(out, v, 0.f);
        if (t == 0) nll[m] = 0.f;
        return;
    }
    const float L2E = 1.4426950408889634f;
    float mx = -INFINITY, s = 0.f;  // running maximum of z * log2(e) and sum of 2^(.. - max)
    for (int v = t; v < V; v += 256) {
        const float a = z[v] * L2E;
        if (a > mx) {
            s = s * __builtin_amdgcn_exp2f(mx - a) + 1.f;
            mx = a;
        } else {
            s += __builtin_amdgcn_exp2f(a - mx);
        }
    }
    lse_merge(mx, s, __shfl_xor(mx, 32), __shfl_xor(s, 32));
    lse_merge(mx, s, __shfl_xor(mx, 16), __shfl_xor(s, 16));
    lse_merge(mx, s, __shfl_xor(mx, 8), __shfl_xor(s, 8));
    lse_merge(mx, s, __shfl_xor(mx, 4), __shfl_xor(s, 4));
    lse_merge(mx, s, __shfl_xor(mx, 2), __shfl_xor(s, 2));
    lse_merge(mx, s, __shfl_xor(mx, 1), __shfl_xor(s, 1));
    if ((t & 63) == 0) {
        sm[t >> 6] = mx;
        ss[t >> 6] = s;
    }
    __syncthreads();
    mx = sm[0];
    s = ss[0];
    for (int i = 1; i < 4; ++i) lse_merge(mx, s, sm[i], ss[i]);
    const float lse2 = mx + __log2f(s);  // log2 of sum 2^(z log2 e)
    if (t == 0) nll[m] = lse2 / L2E - z[y];
    const float inv_n = 1.0f / (float)max(cnt[0], 1);
    for (int v = t; v < Vp; v += 256) {
        float g = 0.f;
        if (v < V) g = (__builtin_amdgcn_exp2f(z[v] * L2E - lse2) - (v == y ? 1.f : 0.f)) * inv_n;
        Act<BF>::store(out, v, g);
    }
}

// The same with the row held in registers: 512 threads per row, NF float4 per thread (row stride
// ld a multiple of 4, columns V <= v of the row masked by index), so the logits are read once. The
// row maximum and the sum of 2^((z - max) log2 e) are reduced over the wavefront and then over the
// eight wavefronts in a fixed order. Registers are capped at 128 (four waves per SIMD) so that two
// rows share a CU, one loading while the other reduces and stores (with the 168 the compiler chose
// otherwise, a CU held one row at a time; capped, with a few registers spilled, a GPT-2 small
// training step measured 0.4% faster).
constexpr int XG_T = 512;

__device__ __forceinline__ float wave_max_xor(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum_xor(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <bool BF, int NF>
__global__ void __launch_bounds__(XG_T, 4) xent_grad_reg_kernel(const float* __restrict__ logits, long ld, int V, int Vp,
                                                            const int32_t* __restrict__ tgt,
                                                            const int32_t* __restrict__ cnt, float* __restrict__ nll,
                                                            void* __restrict__ dlogits) {
    __shared__ float red[2][XG_T / 64];
    const int m = blockIdx.x, t = threadIdx.x, wave = t >> 6;
    const float* z = logits + (long)m * ld;
    const int y = tgt[m];
    auto* out = static_cast<typename Act<BF>::T*>(dlogits) + (long)m * Vp;
    const int nq = Vp / 4;
    auto store4 = [&](int f, float g0, float g1, float g2, float g3) {
        if constexpr (BF) {
            uint2 p;
            p.x = pack_bf16x2(g0, g1);
            p.y = pack_bf16x2(g2, g3);
            *reinterpret_cast<uint2*>(out + 4 * (long)f) = p;
        } else {
            *reinterpret_cast<float4*>(out + 4 * (long)f) = make_float4(g0, g1, g2, g3);
        }
    };
    if (y < 0) {
        for (int f = t; f < nq; f += XG_T) store4(f, 0.f, 0.f, 0.f, 0.f);
        if (t == 0) nll[m] = 0.f;
        return;
    }
    float4 zr[NF];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int f = t + i * XG_T;
        float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (f < nq) {
            v = *reinterpret_cast<const float4*>(z + 4 * (long)f);
            const int c = 4 * f;
            if (c + 0 >= V) v.x = -INFINITY;
            if (c + 1 >= V) v.y = -INFINITY;
            if (c + 2 >= V) v.z = -INFINITY;
            if (c + 3 >= V) v.w = -INFINITY;
        }
        zr[i] = v;
        mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
    mx = wave_max_xor(mx);
    if ((t & 63) == 0) red[0][wave] = mx;
    __syncthreads();
    mx = red[0][0];
#pragma unroll
    for (int w = 1; w < XG_T / 64; ++w) mx = fmaxf(mx, red[0][w]);
    const float L2E = 1.4426950408889634f;
    const float mb = mx * L2E;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NF; ++i) {  // masked columns: exp2(-inf) = 0
        s += __builtin_amdgcn_exp2f(fmaf(zr[i].x, L2E, -mb)) + __builtin_amdgcn_exp2f(fmaf(zr[i].y, L2E, -mb));
        s += __builtin_amdgcn_exp2f(fmaf(zr[i].z, L2E, -mb)) + __builtin_amdgcn_exp2f(fmaf(zr[i].w, L2E, -mb));
    }
    s = wave_sum_xor(s);
    if ((t & 63) == 0) red[1][wave] = s;
    __syncthreads();
    s = red[1][0];
#pragma unroll
    for (int w = 1; w < XG_T / 64; ++w) s += red[1][w];
    const float lse2 = mb + __log2f(s);  // log2 of sum 2^(z log2 e)
    if (t == 0) nll[m] = lse2 / L2E - z[y];
    const float inv_n = 1.0f / (float)max(cnt[0], 1);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        const int f = t + i * XG_T;
        if (f < nq) {
            const int c = 4 * f;
            auto g = [&](float zz, int v) {
                return (__builtin_amdgcn_exp2f(fmaf(zz, L2E, -lse2)) - (v == y ? 1.f : 0.f)) * inv_n;
            };
            store4(f, c + 0 < V ? g(zr[i].x, c + 0) : 0.f, c + 1 < V ? g(zr[i].y, c + 1) : 0.f,
                   c + 2 < V ? g(zr[i].z, c + 2) : 0.f, c + 3 < V ? g(zr[i].w, c + 3) : 0.f);
        }
    }
}

// ------------------------------------------------------------------------------ attention backward
// fp32 compute mode (the bf16 mode uses the matrix-core kernels of attention_bwd.hip).
// Causal attention of head (b, h) on qkv [B, T, 3, H, 64] (compute dtype), output o [B, T, H, 64],
// output gradient dout fp32 [B, T, H*64]. Two threads per row, each owning 32 of the 64 dimensions;
// a dot product is two half sums joined by a lane swap. Softmax in base 2: p = 2^(s c2 - lse2)
// with c2 = log2(e) / 8. Gradients (fp32) go to dqkv [B, T, 3 * H * 64].
constexpr int AB_ROWS = 64, AB_T = 2 * AB_ROWS;

__device__ __forceinline__ float swap_pair(float v) {
    return __builtin_bit_cast(float, dpp_mov<0xB1>(__builtin_bit_cast(uint32_t, v)));
}

template <bool BF>
__device__ __forceinline__ void load_half(const typename Act<BF>::T* p, float (&r)[32]) {
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = Act<BF>::load(p, c);
}

// Pass over the keys j <= i of query i: lse2[i], D[i] = dout_i . o_i, dq_i.
template <bool BF>
__global__ void __launch_bounds__(AB_T) attn_bwd_q_kernel(const void* __restrict__ qkv_, const void* __restrict__ o_,
                                                          const float* __restrict__ dout, float* __restrict__ dqkv,
                                                          float* __restrict__ lse_out, float* __restrict__ d_out, int H,
                                                          int T) {
    using AT = typename Act<BF>::T;
    __shared__ float sk[AB_ROWS][64];
    __shared__ float sv[AB_ROWS][64];
    const AT* qkv = static_cast<const AT*>(qkv_);
    const AT* o = static_cast<const AT*>(o_);
    const int bh = blockIdx.y, b = bh / H, h = bh % H, qb = blockIdx.x;
    const int r = threadIdx.x >> 1, half = threadIdx.x & 1, i = qb * AB_ROWS + r;
    const int d = H * 64;
    const float c2 = 0.125f * 1.4426950408889634f;
    const bool valid = i < T;
    const long row = (long)b * T + (valid ? i : 0);
    float q[32], g[32], dq[32];
    load_half<BF>(qkv + row * 3 * d + h * 64 + half * 32, q);
#pragma unroll
    for (int c = 0; c < 32; ++c) g[c] = dout[row * d + h * 64 + half * 32 + c];
    float dd = 0.f;
    {
        float oc[32];
        load_half<BF>(o + row * d + h * 64 + half * 32, oc);
#pragma unroll
        for (int c = 0; c < 32; ++c) dd += g[c] * oc[c];
    }
    dd += swap_pair(dd);
    const int last = min(T - 1, qb * AB_ROWS + AB_ROWS - 1);
    const int n_tiles = last / AB_ROWS + 1;
    // pass 1: the row's log-sum-exp (base 2)
    float mx = -INFINITY, s = 0.f;
    for (int kt = 0; kt < n_tiles; ++kt) {
        __syncthreads();
        for (int e = threadIdx.x; e < AB_ROWS * 64; e += AB_T) {
            const int j = kt * AB_ROWS + (e >> 6), c = e & 63;
            sk[e >> 6][c] = j < T ? Act<BF>::load(qkv, ((long)b * T + j) * 3 * d + d + h * 64 + c) : 0.f;
        }
        __syncthreads();
        const int jn = min(AB_ROWS, i - kt * AB_ROWS + 1);  // keys j <= i in this tile
        for (int jj = 0; jj < AB_ROWS; ++jj) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) a += q[c] * sk[jj][half * 32 + c];
            a = (a + swap_pair(a)) * c2;
            if (jj < jn) {
                if (a > mx) {
                    s = s * __builtin_amdgcn_exp2f(mx - a) + 1.f;
                    mx = a;
                } else {
                    s += __builtin_amdgcn_exp2f(a - mx);
                }
            }
        }
    }
    const float lse2 = mx + __log2f(s);
    // pass 2: dq = sum_j p_ij (dout_i . v_j - D_i) k_j / 8
#pragma unroll
    for (int c = 0; c < 32; ++c) dq[c] = 0.f;
    for (int kt = 0; kt < n_tiles; ++kt) {
        __syncthreads();
        for (int e = threadIdx.x; e < AB_ROWS * 64; e += AB_T) {
            const int j = kt * AB_ROWS + (e >> 6), c = e & 63;
            const long base = ((long)b * T + j) * 3 * d + h * 64 + c;
            sk[e >> 6][c] = j < T ? Act<BF>::load(qkv, base + d) : 0.f;
            sv[e >> 6][c] = j < T ? Act<BF>::load(qkv, base + 2 * d) : 0.f;
        }
        __syncthreads();
        const int jn = min(AB_ROWS, i - kt * AB_ROWS + 1);
        for (int jj = 0; jj < AB_ROWS; ++jj) {
            float a = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                a += q[c] * sk[jj][half * 32 + c];
                dp += g[c] * sv[jj][half * 32 + c];
            }
            a = (a + swap_pair(a)) * c2;
            dp += swap_pair(dp);
            const float p = jj < jn ? __builtin_amdgcn_exp2f(a - lse2) : 0.f;
            const float ds = p * (dp - dd);
#pragma unroll
            for (int c = 0; c < 32; ++c) dq[c] += ds * sk[jj][half * 32 + c];
        }
    }
    if (valid) {
#pragma unroll
        for (int c = 0; c < 32; ++c) dqkv[row * 3 * d + h * 64 + half * 32 + c] = dq[c] * 0.125f;
        if (half == 0) {
            lse_out[(long)bh * T + i] = lse2;
            d_out[(long)bh * T + i] = dd;
        }
    }
}

// Pass over the queries i >= j of key j: dk_j, dv_j.
template <bool BF>
__global__ void __launch_bounds__(AB_T) attn_bwd_kv_kernel(const void* __restrict__ qkv_, const float* __restrict__ dout,
                                                           const float* __restrict__ lse, const float* __restrict__ dvec,
                                                           float* __restrict__ dqkv, int H, int T) {
    using AT = typename Act<BF>::T;
    __shared__ float sq[AB_ROWS][64];
    __shared__ float sg[AB_ROWS][64];
    __shared__ float sl[AB_ROWS], sd[AB_ROWS];
    const AT* qkv = static_cast<const AT*>(qkv_);
    const int bh = blockIdx.y, b = bh / H, h = bh % H, kb = blockIdx.x;
    const int r = threadIdx.x >> 1, half = threadIdx.x & 1, j = kb * AB_ROWS + r;
    const int d = H * 64;
    const float c2 = 0.125f * 1.4426950408889634f;
    const bool valid = j < T;
    const long row = (long)b * T + (valid ? j : 0);
    float k[32], v[32], dk[32], dv[32];
    load_half<BF>(qkv + row * 3 * d + d + h * 64 + half * 32, k);
    load_half<BF>(qkv + row * 3 * d + 2 * d + h * 64 + half * 32, v);
#pragma unroll
    for (int c = 0; c < 32; ++c) dk[c] = dv[c] = 0.f;
    const int n_tiles = (T + AB_ROWS - 1) / AB_ROWS;
    for (int qt = kb; qt < n_tiles; ++qt) {
        __syncthreads();
        for (int e = threadIdx.x; e < AB_ROWS * 64; e += AB_T) {
            const int i = qt * AB_ROWS + (e >> 6), c = e & 63;
            const long ri = (long)b * T + i;
            sq[e >> 6][c] = i < T ? Act<BF>::load(qkv, ri * 3 * d + h * 64 + c) : 0.f;
            sg[e >> 6][c] = i < T ? dout[ri * d + h * 64 + c] : 0.f;
        }
        if (threadIdx.x < AB_ROWS) {
            const int i = qt * AB_ROWS + threadIdx.x;
            sl[threadIdx.x] = i < T ? lse[(long)bh * T + i] : 0.f;
            sd[threadIdx.x] = i < T ? dvec[(long)bh * T + i] : 0.f;
        }
        __syncthreads();
        for (int ii = 0; ii < AB_ROWS; ++ii) {
            const int i = qt * AB_ROWS + ii;
            float a = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                a += sq[ii][half * 32 + c] * k[c];
                dp += sg[ii][half * 32 + c] * v[c];
            }
            a = (a + swap_pair(a)) * c2;
            dp += swap_pair(dp);
            const float p = (i >= j && i < T) ? __builtin_amdgcn_exp2f(a - sl[ii]) : 0.f;
            const float ds = p * (dp - sd[ii]);
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                dv[c] += p * sg[ii][half * 32 + c];
                dk[c] += ds * sq[ii][half * 32 + c];
            }
        }
    }
    if (valid) {
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            dqkv[row * 3 * d + d + h * 64 + half * 32 + c] = dk[c] * 0.125f;
            dqkv[row * 3 * d + 2 * d + h * 64 + half * 32 + c] = dv[c];
        }
    }
}

// ------------------------------------------------------------------------------ embedding backward
// gwpe[t] = sum over b of dx[b, t] for t < T, 0 for T <= t < n_ctx (batch order).
__global__ void wpe_grad_kernel(const float* __restrict__ dx, int B, int T, int n_ctx, int d, float* __restrict__ gwpe) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)n_ctx * d) return;
    const int t = (int)(e / d), c = (int)(e % d);
    float acc = 0.f;
    if (t < T)
        for (int b = 0; b < B; ++b) acc += dx[((long)b * T + t) * d + c];
    gwpe[e] = acc;
}
// gwte[tok[m]] += dx[m] (float atomics: tokens that repeat add in an unspecified order).
__global__ void wte_grad_kernel(const int32_t* __restrict__ tok, const float* __restrict__ dx, int M, int d, int V,
                                float* __restrict__ gwte) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= (long)M * d) return;
    const int m = (int)(e / d), c = (int)(e % d), id = tok[m];
    if (id >= 0 && id < V) atomicAdd(gwte + (long)id * d + c, dx[e]);
}

}  // namespace

hipError_t transpose(const void* src, bool src_bf16, long lds, int R, int C, void* dst, bool dst_bf16, long ldd, int Rp,
                     hipStream_t s) {
    const dim3 grid((C + 63) / 64, (Rp + 63) / 64), block(256);
    const bool vec = lds % 8 == 0 && ldd % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dst) % 16 == 0;
    if (src_bf16 && dst_bf16 && vec)
        transpose_vec_kernel<true><<<grid, block, 0, s>>>(src, lds, R, C, static_cast<uint16_t*>(dst), ldd, Rp);
    else if (dst_bf16 && vec)
        transpose_vec_kernel<false><<<grid, block, 0, s>>>(src, lds, R, C, static_cast<uint16_t*>(dst), ldd, Rp);
    else if (src_bf16 && dst_bf16)
        transpose_kernel<true, true><<<grid, block, 0, s>>>(src, lds, R, C, dst, ldd, Rp);
    else if (src_bf16)
        transpose_kernel<true, false><<<grid, block, 0, s>>>(src, lds, R, C, dst, ldd, Rp);
    else if (dst_bf16)
        transpose_kernel<false, true><<<grid, block, 0, s>>>(src, lds, R, C, dst, ldd, Rp);
    else
        transpose_kernel<false, false><<<grid, block, 0, s>>>(src, lds, R, C, dst, ldd, Rp);
    return hipGetLastError();
}

int colsum_blocks(int R) { return (R + kColRows - 1) / kColRows; }

hipError_t colsum_reduce_multi(const ColsumSegs& segs, hipStream_t s) {
    if (segs.n < 1 || segs.n > kColsumSegs) return hipErrorInvalidValue;
    int cmax = 0;
    for (int i = 0; i < segs.n; ++i) cmax = max(cmax, segs.seg[i].C);
    colsum_reduce_multi_kernel<<<dim3((cmax + kRedCols - 1) / kRedCols, segs.n), dim3(256), 0, s>>>(segs);
    return hipGetLastError();
}

hipError_t colsum(const float* src, long ld, int R, int C, float* part, float* out, hipStream_t s) {
    const int nb = colsum_blocks(R);
    colsum_partial_kernel<<<dim3((C + 63) / 64, nb), dim3(256), 0, s>>>(src, ld, R, C, part);
    colsum_reduce_kernel<<<dim3((C + kRedCols - 1) / kRedCols), dim3(256), 0, s>>>(part, nb, C, out);
    return hipGetLastError();
}

int ln_backward_blocks(int M) { return (M + kLnRows - 1) / kLnRows; }

hipError_t ln_backward(const float* x, const float* gamma, const float* dy, float* dx, int M, int d, float eps, float* pg,
                       float* pb, float* dgamma, float* dbeta, hipStream_t s, uint16_t* y16, float* pd) {
    if (y16 && !pd) return hipErrorInvalidValue;
    const int nb = ln_backward_blocks(M);
    const dim3 grid(nb), block(64 * kLnWaves);
    switch (d) {
        case 768: ln_backward_kernel<12><<<grid, block, 0, s>>>(x, gamma, dy, dx, M, d, eps, pg, pb, y16, pd); break;
        case 1024: ln_backward_kernel<16><<<grid, block, 0, s>>>(x, gamma, dy, dx, M, d, eps, pg, pb, y16, pd); break;
        case 1280: ln_backward_kernel<20><<<grid, block, 0, s>>>(x, gamma, dy, dx, M, d, eps, pg, pb, y16, pd); break;
        case 1600: ln_backward_kernel<25><<<grid, block, 0, s>>>(x, gamma, dy, dx, M, d, eps, pg, pb, y16, pd); break;
        default: ln_backward_kernel<0><<<grid, dim3(64), 0, s>>>(x, gamma, dy, dx, M, d, eps, pg, pb, y16, pd); break;
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    ColsumSegs segs;  // the gain and shift gradients in one launch
    segs.seg[0] = {pg, dgamma, nb, d};
    segs.seg[1] = {pb, dbeta, nb, d};
    segs.n = 2;
    return colsum_reduce_multi(segs, s);
}

hipError_t gelu_forward(const float* u, void* h, long n, bool bf16, int erf_form, hipStream_t s) {
    if (n % 4 == 0 && reinterpret_cast<uintptr_t>(u) % 16 == 0 && reinterpret_cast<uintptr_t>(h) % 16 == 0) {
        const dim3 grid4((unsigned)((n / 4 + 255) / 256)), block4(256);
        if (bf16)
            gelu_forward_x4_kernel<true><<<grid4, block4, 0, s>>>(reinterpret_cast<const float4*>(u), h, n / 4, erf_form);
        else
            gelu_forward_x4_kernel<false><<<grid4, block4, 0, s>>>(reinterpret_cast<const float4*>(u), h, n / 4, erf_form);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (bf16)
        gelu_forward_kernel<true><<<grid, block, 0, s>>>(u, h, n, erf_form);
    else
        gelu_forward_kernel<false><<<grid, block, 0, s>>>(u, h, n, erf_form);
    return hipGetLastError();
}

hipError_t gelu_backward(const float* u, float* g, long n, int erf_form, hipStream_t s) {
    if (n % 4 == 0 && reinterpret_cast<uintptr_t>(u) % 16 == 0 && reinterpret_cast<uintptr_t>(g) % 16 == 0) {
        gelu_backward_x4_kernel<<<dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s>>>(
            reinterpret_cast<const float4*>(u), reinterpret_cast<float4*>(g), n / 4, erf_form);
        return hipGetLastError();
    }
    gelu_backward_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(u, g, n, erf_form);
    return hipGetLastError();
}

hipError_t xent_grad(const float* logits, long ld, int M, int V, int Vp, const int32_t* tgt, int32_t* cnt, float* nll,
                     void* dlogits, bool bf16, hipStream_t s) {
    count_targets_kernel<<<dim3(1), dim3(256), 0, s>>>(tgt, M, cnt);
    // the row in registers when it fits (the row stride and Vp multiples of 4), else two passes
    const int nf = (Vp / 4 + XG_T - 1) / XG_T;
    if (ld % 4 == 0 && Vp % 4 == 0 && nf <= 32) {
#define GPT2_XG(NF)                                                                                          \
    do {                                                                                                     \
        if (bf16)                                                                                            \
            xent_grad_reg_kernel<true, NF><<<dim3(M), dim3(XG_T), 0, s>>>(logits, ld, V, Vp, tgt, cnt, nll, dlogits); \
        else                                                                                                 \
            xent_grad_reg_kernel<false, NF><<<dim3(M), dim3(XG_T), 0, s>>>(logits, ld, V, Vp, tgt, cnt, nll,        \
                                                                           dlogits);                         \
        return hipGetLastError();                                                                            \
    } while (0)
        if (nf <= 1) GPT2_XG(1);
        if (nf <= 4) GPT2_XG(4);
        if (nf <= 12) GPT2_XG(12);
        if (nf <= 25) GPT2_XG(25);
        GPT2_XG(32);
#undef GPT2_XG
    }
    if (bf16)
        xent_grad_kernel<true><<<dim3(M), dim3(256), 0, s>>>(logits, ld, V, Vp, tgt, cnt, nll, dlogits);
    else
        xent_grad_kernel<false><<<dim3(M), dim3(256), 0, s>>>(logits, ld, V, Vp, tgt, cnt, nll, dlogits);
    return hipGetLastError();
}

hipError_t attention_backward(const void* qkv, const void* o, const float* dout, float* dqkv, float* lse, float* dvec,
                              int B, int H, int T, bool bf16, hipStream_t s) {
    if (bf16) return hipErrorInvalidValue;  // attention_backward_bf16
    const dim3 grid((T + AB_ROWS - 1) / AB_ROWS, B * H), block(AB_T);
    attn_bwd_q_kernel<false><<<grid, block, 0, s>>>(qkv, o, dout, dqkv, lse, dvec, H, T);
    attn_bwd_kv_kernel<false><<<grid, block, 0, s>>>(qkv, dout, lse, dvec, dqkv, H, T);
    return hipGetLastError();
}

hipError_t embed_backward(const int32_t* tok, const float* dx, int B, int T, int n_ctx, int d, int V, float* gwte,
                          float* gwpe, hipStream_t s) {
    wpe_grad_kernel<<<dim3((unsigned)(((long)n_ctx * d + 255) / 256)), dim3(256), 0, s>>>(dx, B, T, n_ctx, d, gwpe);
    wte_grad_kernel<<<dim3((unsigned)(((long)B * T * d + 255) / 256)), dim3(256), 0, s>>>(tok, dx, B * T, d, V, gwte);
    return hipGetLastError();
}

}  // namespace gpt2k
