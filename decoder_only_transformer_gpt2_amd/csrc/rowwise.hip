// Row-wise HBM-bound kernels: embedding gather-add, LayerNorm, argmax reduction, weight packing.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int kRowsPerBlock = 4;  // one wavefront per row, four wavefronts per workgroup

// x[m, :] = wte[tok[m], :] + wpe[m mod T, :]  (token embedding plus learned position embedding,
// positions from 0; "从零手写GPT-2" §4.1 forward step 1, "复现GPT-2 124M" §2.1).
// Tables are bf16 or fp32; the sum is one fp32 add of the two exactly-upcast entries, so it equals
// the correctly rounded fp32 value of the exact sum. An id outside [0, n_vocab) is clamped for the
// read and recorded in flags[blockIdx.x] (every block writes its slot on every launch).
template <bool BF16>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok, const void* __restrict__ wte,
                                                    const void* __restrict__ wpe, float* __restrict__ x, int M,
                                                    int T, int pos0, int d, int n_vocab, int32_t* __restrict__ flags) {
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int row = blockIdx.x * kRowsPerBlock + wave;
    int bad = 0;
    if (row < M) {
        int t = tok[row];
        if (t < 0 || t >= n_vocab) {
            bad = 1;
            t = t < 0 ? 0 : n_vocab - 1;
        }
        const int pos = pos0 + row % T;
        float4* xr = reinterpret_cast<float4*>(x + (size_t)row * d);
        const int nq = d / 4;
        if (BF16) {
            const uint2* er = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(wte) + (size_t)t * d);
            const uint2* pr = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(wpe) + (size_t)pos * d);
            for (int c = lane; c < nq; c += GPT2_WAVE) {
                const uint2 e = er[c], p = pr[c];
                float4 o;
                o.x = bf16_bits_to_f32(e.x & 0xffffu) + bf16_bits_to_f32(p.x & 0xffffu);
                o.y = bf16_bits_to_f32(e.x >> 16) + bf16_bits_to_f32(p.x >> 16);
                o.z = bf16_bits_to_f32(e.y & 0xffffu) + bf16_bits_to_f32(p.y & 0xffffu);
                o.w = bf16_bits_to_f32(e.y >> 16) + bf16_bits_to_f32(p.y >> 16);
                xr[c] = o;
            }
        } else {
            const float4* er = reinterpret_cast<const float4*>(static_cast<const float*>(wte) + (size_t)t * d);
            const float4* pr = reinterpret_cast<const float4*>(static_cast<const float*>(wpe) + (size_t)pos * d);
            for (int c = lane; c < nq; c += GPT2_WAVE) {
                const float4 e = er[c], p = pr[c];
                xr[c] = make_float4(e.x + p.x, e.y + p.y, e.z + p.z, e.w + p.w);
            }
        }
    }
    const int any_bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) flags[blockIdx.x] = any_bad;
}

// LayerNorm with the biased variance ("复现GPT-2 124M" §2.1: unbiased=False; eps inside the square
// root, "从零手写GPT-2" §3.2). One wavefront per row; the row stays in registers between the two
// passes (mean, then the centred sum of squares), so x is read from memory once.
template <int NV, bool OUT_BF16>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                        const float* __restrict__ b, void* __restrict__ y, int M,
                                                        int n, float eps) {
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int row = blockIdx.x * kRowsPerBlock + wave;
    if (row >= M) return;
    const int nq = n / 4;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * n);
    float4 v[NV];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * GPT2_WAVE + lane;
        v[i] = c < nq ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float mean = wave_sum(s) / (float)n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * GPT2_WAVE + lane;
        if (c < nq) {
            const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
            q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
        }
    }
    const float var = wave_sum(q) / (float)n;
    const float rstd = 1.0f / sqrtf(var + eps);
    const float4* g4 = reinterpret_cast<const float4*>(g);
    const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * GPT2_WAVE + lane;
        if (c < nq) {
            const float4 gg = g4[c], bb = b4[c];
            float4 o;
            o.x = (v[i].x - mean) * rstd * gg.x + bb.x;
            o.y = (v[i].y - mean) * rstd * gg.y + bb.y;
            o.z = (v[i].z - mean) * rstd * gg.z + bb.z;
            o.w = (v[i].w - mean) * rstd * gg.w + bb.w;
            if (OUT_BF16) {
                uint2 p;
                p.x = pack_bf16x2(o.x, o.y);
                p.y = pack_bf16x2(o.z, o.w);
                reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (size_t)row * n)[c] = p;
            } else {
                reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)row * n)[c] = o;
            }
        }
    }
}

// Row argmax from per-tile partials (value, index) written by the logits GEMM epilogue.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                                            int M, int n_part, int32_t* __restrict__ out) {
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int row = blockIdx.x * kRowsPerBlock + wave;
    if (row >= M) return;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = lane; j < n_part; j += GPT2_WAVE)
        argmax_merge(bv, bi, pv[(size_t)row * n_part + j], pi[(size_t)row * n_part + j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float v2 = __shfl_xor(bv, o, GPT2_WAVE);
        const int i2 = __shfl_xor(bi, o, GPT2_WAVE);
        argmax_merge(bv, bi, v2, i2);
    }
    if (lane == 0) out[row] = bi;
}

// Shifted next-token targets ([手写] §4.1: logits of position t are scored against the label of
// position t+1); the ignore index and the last position of each sequence give -1.
constexpr int kIgnoreIndex = -100;

__global__ __launch_bounds__(256) void xent_targets_kernel(const int32_t* __restrict__ labels, int M, int T,
                                                           int n_vocab, int32_t* __restrict__ tgt,
                                                           int32_t* __restrict__ flags) {
    const int m = blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    int t = -1;
    if (m % T != T - 1) {
        const int y = labels[m + 1];
        if (y >= 0 && y < n_vocab)
            t = y;
        else if (y != kIgnoreIndex)
            flags[0] = 1;  // reported by gpt2_check; the position is left out
    }
    tgt[m] = t;
}

// One wavefront per row: log-sum-exp from the per-tile base-2 partials, minus the target logit.
__global__ __launch_bounds__(256) void xent_rows_kernel(const float* __restrict__ pm, const float* __restrict__ ps,
                                                        const int32_t* __restrict__ tgt,
                                                        const float* __restrict__ tgt_logit, int M, int n_part,
                                                        float* __restrict__ nll) {
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int row = blockIdx.x * kRowsPerBlock + wave;
    if (row >= M) return;
    float mx = -INFINITY, sum = 0.f;
    for (int j = lane; j < n_part; j += GPT2_WAVE) {
        const float m2 = pm[(size_t)row * n_part + j], s2 = ps[(size_t)row * n_part + j];
        const float mn = fmaxf(mx, m2), mz = mn == -INFINITY ? 0.f : mn;
        sum = sum * exp2f(mx - mz) + s2 * exp2f(m2 - mz);
        mx = mn;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(mx, o, GPT2_WAVE), s2 = __shfl_xor(sum, o, GPT2_WAVE);
        const float mn = fmaxf(mx, m2), mz = mn == -INFINITY ? 0.f : mn;
        sum = sum * exp2f(mx - mz) + s2 * exp2f(m2 - mz);
        mx = mn;
    }
    if (lane == 0) {
        const float ln2 = 0.6931471805599453f;
        nll[row] = tgt[row] >= 0 ? (mx + log2f(sum)) * ln2 - tgt_logit[row] : 0.f;
    }
}

// One workgroup: the mean over the counted rows, summed in a fixed order (strided per thread,
// then a tree), so the result does not depend on scheduling.
__global__ __launch_bounds__(1024) void xent_mean_kernel(const float* __restrict__ nll, const int32_t* __restrict__ tgt,
                                                         int M, float* __restrict__ loss) {
    __shared__ float ssum[1024];
    __shared__ int scnt[1024];
    float acc = 0.f;
    int cnt = 0;
    for (int m = threadIdx.x; m < M; m += 1024)
        if (tgt[m] >= 0) {
            acc += nll[m];
            ++cnt;
        }
    ssum[threadIdx.x] = acc;
    scnt[threadIdx.x] = cnt;
    __syncthreads();
    for (int w = 512; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) {
            ssum[threadIdx.x] += ssum[threadIdx.x + w];
            scnt[threadIdx.x] += scnt[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[0] = ssum[0] / (float)scnt[0];  // 0 / 0 = NaN when nothing counts
}

// The same with a whole workgroup per row, for long partial lists (the 16-column partials of the
// few-row projection: 3142 per row for the GPT-2 vocabulary).
__global__ __launch_bounds__(256) void argmax_reduce_wide_kernel(const float* __restrict__ pv,
                                                                 const int32_t* __restrict__ pi, int n_part,
                                                                 int32_t* __restrict__ out) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int row = blockIdx.x, wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = threadIdx.x; j < n_part; j += 256)
        argmax_merge(bv, bi, pv[(size_t)row * n_part + j], pi[(size_t)row * n_part + j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float v2 = __shfl_xor(bv, o, GPT2_WAVE);
        const int i2 = __shfl_xor(bi, o, GPT2_WAVE);
        argmax_merge(bv, bi, v2, i2);
    }
    if (lane == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, sv[w], si[w]);
        out[row] = bi;
    }
}

__global__ __launch_bounds__(256) void convert_kernel(const void* __restrict__ src, int src_bf16, void* __restrict__ dst,
                                                      int dst_bf16, long n_src, long n_dst) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n_dst; i += (long)gridDim.x * blockDim.x) {
        float v = 0.f;
        if (i < n_src)
            v = src_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(src)[i]) : static_cast<const float*>(src)[i];
        if (dst_bf16)
            static_cast<uint16_t*>(dst)[i] = f32_to_bf16_bits(v);
        else
            static_cast<float*>(dst)[i] = v;
    }
}

// fp32 -> bf16, eight values per thread (two 16-byte reads, one 16-byte write), zero from n_src8 on;
// the same rounding as convert_kernel.
__global__ __launch_bounds__(256) void convert_f32_bf16_x8_kernel(const float4* __restrict__ src,
                                                                 u32x4_t* __restrict__ dst, long n_src8, long n_dst8) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n_dst8; i += (long)gridDim.x * blockDim.x) {
        u32x4_t o = {0u, 0u, 0u, 0u};
        if (i < n_src8) {
            const float4 a = src[2 * i], b = src[2 * i + 1];
            o[0] = pack_bf16x2(a.x, a.y);
            o[1] = pack_bf16x2(a.z, a.w);
            o[2] = pack_bf16x2(b.x, b.y);
            o[3] = pack_bf16x2(b.z, b.w);
        }
        dst[i] = o;
    }
}

// LayerNorm with a k-blocked bf16 output: WAVES*RPW rows per workgroup (RPW per wavefront, all
// their loads in flight together), normalised into LDS (rows padded by 16 bytes against bank
// conflicts), then written block by block: the rows' 32-column slab of a block is one contiguous
// run of WAVES*RPW*64 bytes, 16 bytes per lane. The statistics and rounding are those of
// layernorm_kernel, so the values are bit-identical to its row-major output.
template <int NV, int RPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void layernorm_kb_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                           const float* __restrict__ b, uint16_t* __restrict__ y,
                                                           int M, int n, float eps, int kb_rows) {
    extern __shared__ __attribute__((aligned(16))) uint16_t sy[];  // [WAVES*RPW][n + 8]
    constexpr int R = WAVES * RPW;
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int r0 = blockIdx.x * R, nq = n / 4, sp = n + 8;
    float4 v[RPW][NV];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int row = r0 + wave * RPW + r;
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)min(row, M - 1) * n);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = i * GPT2_WAVE + lane;
            v[r][i] = c < nq ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    const float4* g4 = reinterpret_cast<const float4*>(g);
    const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) s += (v[r][i].x + v[r][i].y) + (v[r][i].z + v[r][i].w);
        const float mean = wave_sum(s) / (float)n;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = i * GPT2_WAVE + lane;
            if (c < nq) {
                const float a0 = v[r][i].x - mean, a1 = v[r][i].y - mean, a2 = v[r][i].z - mean, a3 = v[r][i].w - mean;
                q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
            }
        }
        const float var = wave_sum(q) / (float)n;
        const float rstd = 1.0f / sqrtf(var + eps);
        uint16_t* srow = sy + (wave * RPW + r) * sp;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = i * GPT2_WAVE + lane;
            if (c < nq) {
                const float4 gg = g4[c], bb = b4[c];
                uint2 p;
                p.x = pack_bf16x2((v[r][i].x - mean) * rstd * gg.x + bb.x, (v[r][i].y - mean) * rstd * gg.y + bb.y);
                p.y = pack_bf16x2((v[r][i].z - mean) * rstd * gg.z + bb.z, (v[r][i].w - mean) * rstd * gg.w + bb.w);
                *reinterpret_cast<uint2*>(srow + 4 * c) = p;
            }
        }
    }
    __syncthreads();
    const int n_chunks = (n / 32) * R * 4;  // 16-byte chunks: per block, R rows of four
    for (int ci = threadIdx.x; ci < n_chunks; ci += blockDim.x) {
        const int blk = ci / (R * 4), rr = (ci / 4) % R, part = ci % 4;
        const int row = r0 + rr;
        if (row < M)
            *reinterpret_cast<u32x4_t*>(y + ((size_t)blk * kb_rows + row) * 32 + part * 8) =
                *reinterpret_cast<const u32x4_t*>(sy + rr * sp + blk * 32 + part * 8);
    }
}

// The embedding gather-add fused with the first block's ln_1, for bf16 tables and a k-blocked bf16
// LayerNorm output: each wavefront forms its row of x in registers with the adds of embed_kernel,
// stores it (the residual stream), and normalises it with the arithmetic of layernorm_kb_kernel
// (the same sums in the same order), so x and the LayerNorm output carry exactly the bits of the two
// launches this one replaces, and x is not read back from memory. Four rows per workgroup, the token
// flags as in embed_kernel.
template <int NV>
__global__ __launch_bounds__(256) void embed_ln_kb_kernel(const int32_t* __restrict__ tok,
                                                          const uint16_t* __restrict__ wte,
                                                          const uint16_t* __restrict__ wpe, float* __restrict__ x,
                                                          const float* __restrict__ g, const float* __restrict__ b,
                                                          uint16_t* __restrict__ y, int M, int T, int pos0, int n,
                                                          int n_vocab, float eps, int kb_rows,
                                                          int32_t* __restrict__ flags) {
    extern __shared__ __attribute__((aligned(16))) uint16_t sy[];  // [kRowsPerBlock][n + 8]
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int r0 = blockIdx.x * kRowsPerBlock, row = r0 + wave, nq = n / 4, sp = n + 8;
    const int rr = min(row, M - 1);  // rows past M compute on a valid row and store nothing
    int t = tok[rr];
    const int bad = row < M && (t < 0 || t >= n_vocab);
    t = t < 0 ? 0 : t >= n_vocab ? n_vocab - 1 : t;
    const int pos = pos0 + rr % T;
    const uint2* er = reinterpret_cast<const uint2*>(wte + (size_t)t * n);
    const uint2* pr = reinterpret_cast<const uint2*>(wpe + (size_t)pos * n);
    float4* xr = reinterpret_cast<float4*>(x + (size_t)rr * n);
    float4 v[NV];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * GPT2_WAVE + lane;
        v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < nq) {
            const uint2 e = er[c], p = pr[c];
            v[i].x = bf16_bits_to_f32(e.x & 0xffffu) + bf16_bits_to_f32(p.x & 0xffffu);
            v[i].y = bf16_bits_to_f32(e.x >> 16) + bf16_bits_to_f32(p.x >> 16);
            v[i].z = bf16_bits_to_f32(e.y & 0xffffu) + bf16_bits_to_f32(p.y & 0xffffu);
            v[i].w = bf16_bits_to_f32(e.y >> 16) + bf16_bits_to_f32(p.y >> 16);
            if (row < M) xr[c] = v[i];
        }
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float mean = wave_sum(s) / (float)n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * GPT2_WAVE + lane;
        if (c < nq) {
            const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
            q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
        }
    }
    const float var = wave_sum(q) / (float)n;
    const float rstd = 1.0f / sqrtf(var + eps);
    const float4* g4 = reinterpret_cast<const float4*>(g);
    const float4* b4 = reinterpret_cast<const float4*>(b);
    uint16_t* srow = sy + wave * sp;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = i * GPT2_WAVE + lane;
        if (c < nq) {
            const float4 gg = g4[c], bb = b4[c];
            uint2 p;
            p.x = pack_bf16x2((v[i].x - mean) * rstd * gg.x + bb.x, (v[i].y - mean) * rstd * gg.y + bb.y);
            p.y = pack_bf16x2((v[i].z - mean) * rstd * gg.z + bb.z, (v[i].w - mean) * rstd * gg.w + bb.w);
            *reinterpret_cast<uint2*>(srow + 4 * c) = p;
        }
    }
    const int any_bad = __syncthreads_or(bad);  // also the barrier before the staged rows are read
    if (threadIdx.x == 0) flags[blockIdx.x] = any_bad;
    const int n_chunks = (n / 32) * kRowsPerBlock * 4;  // 16-byte chunks: per block, four rows of four
    for (int ci = threadIdx.x; ci < n_chunks; ci += blockDim.x) {
        const int blk = ci / (kRowsPerBlock * 4), rl = (ci / 4) % kRowsPerBlock, part = ci % 4;
        const int r = r0 + rl;
        if (r < M)
            *reinterpret_cast<u32x4_t*>(y + ((size_t)blk * kb_rows + r) * 32 + part * 8) =
                *reinterpret_cast<const u32x4_t*>(sy + rl * sp + blk * 32 + part * 8);
    }
}

// One 16-byte chunk (8 columns) per thread: chunk j of row r goes to block j/4 of the k-blocked copy.
__global__ __launch_bounds__(256) void kblock_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     long rows, int K) {
    const int cpr = K / 8;  // chunks per row
    const long n = rows * cpr;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long r = i / cpr;
        const int j = (int)(i % cpr);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + r * K + j * 8);
        *reinterpret_cast<u32x4_t*>(dst + ((long)(j >> 2) * rows + r) * 32 + (j & 3) * 8) = v;
    }
}

template <int NV>
hipError_t launch_ln(const float* x, const float* g, const float* b, void* y, int M, int n, float eps, bool out_bf16,
                     int kb_rows, hipStream_t s) {
    if (kb_rows) {
        const size_t row_bytes = (size_t)(n + 8) * 2;
        // four rows per workgroup (measured at B*T = 4096, d = 768: 16 rows per workgroup leave too
        // few workgroups to hide the load latency; eight gain nothing)
        layernorm_kb_kernel<NV, 1, 4><<<dim3((M + 3) / 4), dim3(256), 4 * row_bytes, s>>>(
            x, g, b, static_cast<uint16_t*>(y), M, n, eps, kb_rows);
        return hipGetLastError();
    }
    dim3 grid((M + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
    if (out_bf16)
        layernorm_kernel<NV, true><<<grid, block, 0, s>>>(x, g, b, y, M, n, eps);
    else
        layernorm_kernel<NV, false><<<grid, block, 0, s>>>(x, g, b, y, M, n, eps);
    return hipGetLastError();
}

}  // namespace

int embed_flag_count(int M) { return (M + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t embed(const int32_t* tok, const void* wte, const void* wpe, float* x, int M, int T, int pos0, int d,
                 int n_vocab, bool bf16, int32_t* flags, hipStream_t s) {
    dim3 grid(embed_flag_count(M)), block(256);
    if (bf16)
        embed_kernel<true><<<grid, block, 0, s>>>(tok, wte, wpe, x, M, T, pos0, d, n_vocab, flags);
    else
        embed_kernel<false><<<grid, block, 0, s>>>(tok, wte, wpe, x, M, T, pos0, d, n_vocab, flags);
    return hipGetLastError();
}

hipError_t embed_ln(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, float* x, const float* g,
                    const float* b, uint16_t* y, int M, int T, int pos0, int n, int n_vocab, float eps, int kb_rows,
                    int32_t* flags, hipStream_t s) {
    if (M < 1 || kb_rows < M || n % 32 || n > 4096) return hipErrorInvalidValue;
    const dim3 grid(embed_flag_count(M)), block(256);
    const size_t lds = (size_t)kRowsPerBlock * (n + 8) * 2;
    const int nq = n / 4;
#define GPT2_EMBED_LN(NV) \
    embed_ln_kb_kernel<NV><<<grid, block, lds, s>>>(tok, wte, wpe, x, g, b, y, M, T, pos0, n, n_vocab, eps, kb_rows, flags)
    if (nq <= 4 * GPT2_WAVE)
        GPT2_EMBED_LN(4);
    else if (nq <= 8 * GPT2_WAVE)
        GPT2_EMBED_LN(8);
    else
        GPT2_EMBED_LN(16);
#undef GPT2_EMBED_LN
    return hipGetLastError();
}

hipError_t layernorm(const float* x, const float* g, const float* b, void* y, int M, int n, float eps, bool out_bf16,
                     hipStream_t s, int kb_rows) {
    if (kb_rows && (!out_bf16 || kb_rows < M || n % 32)) return hipErrorInvalidValue;
    const int nq = n / 4;
    if (nq <= 4 * GPT2_WAVE) return launch_ln<4>(x, g, b, y, M, n, eps, out_bf16, kb_rows, s);
    if (nq <= 8 * GPT2_WAVE) return launch_ln<8>(x, g, b, y, M, n, eps, out_bf16, kb_rows, s);
    return launch_ln<16>(x, g, b, y, M, n, eps, out_bf16, kb_rows, s);  // n <= 4096 (checked by the callers)
}

hipError_t argmax_reduce(const float* pv, const int32_t* pi, int M, int n_part, int32_t* out, hipStream_t s) {
    if (n_part >= 1024)
        argmax_reduce_wide_kernel<<<dim3(M), dim3(256), 0, s>>>(pv, pi, n_part, out);
    else
        argmax_reduce_kernel<<<dim3((M + kRowsPerBlock - 1) / kRowsPerBlock), dim3(256), 0, s>>>(pv, pi, M, n_part, out);
    return hipGetLastError();
}

hipError_t xent_targets(const int32_t* labels, int M, int T, int n_vocab, int32_t* tgt, int32_t* flags,
                        hipStream_t s) {
    xent_targets_kernel<<<dim3((M + 255) / 256), dim3(256), 0, s>>>(labels, M, T, n_vocab, tgt, flags);
    return hipGetLastError();
}

hipError_t xent_rows(const float* pm, const float* ps, const int32_t* tgt, const float* tgt_logit, int M, int n_part,
                     float* nll, hipStream_t s) {
    xent_rows_kernel<<<dim3((M + kRowsPerBlock - 1) / kRowsPerBlock), dim3(256), 0, s>>>(pm, ps, tgt, tgt_logit, M,
                                                                                        n_part, nll);
    return hipGetLastError();
}

hipError_t xent_mean(const float* nll, const int32_t* tgt, int M, float* loss, hipStream_t s) {
    xent_mean_kernel<<<dim3(1), dim3(1024), 0, s>>>(nll, tgt, M, loss);
    return hipGetLastError();
}

hipError_t kblock_bf16(const uint16_t* src, uint16_t* dst, long rows, int K, hipStream_t s) {
    if (K % 32 || rows <= 0) return hipErrorInvalidValue;
    long blocks = (rows * (K / 8) + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    kblock_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(src, dst, rows, K);
    return hipGetLastError();
}

hipError_t convert(const void* src, bool src_bf16, void* dst, bool dst_bf16, long n_src, long n_dst, hipStream_t s) {
    if (n_dst <= 0) return hipSuccess;
    if (!src_bf16 && dst_bf16 && n_src % 8 == 0 && n_dst % 8 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(dst) % 16 == 0) {
        long blocks = (n_dst / 8 + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        convert_f32_bf16_x8_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
            static_cast<const float4*>(src), static_cast<u32x4_t*>(dst), n_src / 8, n_dst / 8);
        return hipGetLastError();
    }
    long blocks = (n_dst + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    convert_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(src, src_bf16, dst, dst_bf16, n_src, n_dst);
    return hipGetLastError();
}

}  // namespace gpt2k
