// Incremental decoding with a key/value cache ([手写] §6.3 and [解析] §4.2: generation feeds one new
// token per step; the keys and values of the earlier positions do not change, so they are kept
// instead of recomputed). Per layer the cache holds K and V as [B][H][n_ctx][64] in the compute
// dtype. A decode step's query attends to keys 0 .. pos: causality makes this the last row of the
// full forward over the extended sequence.
//
// Decode attention is bound by reading the cache (HBM), not by arithmetic: one 1024-thread
// workgroup per (b, h); scores are computed with one key per thread (its 128-byte row against q in LDS), the
// softmax is online over chunks of 1024 keys (fp32, exp2 with the scale folded in), and the
// weighted sum of V is split over 128 key groups x 8 chunks of 8 dimensions, each thread reading
// 16-byte pieces of V rows with four rows in flight; the key groups are summed through LDS.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int DHD = 64;      // head size
constexpr int CHUNK = 1024;  // keys per softmax chunk

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
    if (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    return static_cast<const float*>(p)[i];
}

template <bool BF16>
__global__ __launch_bounds__(256) void kv_append_kernel(const void* __restrict__ qkv, int B, int T, int H, int pos0,
                                                        void* __restrict__ kc, void* __restrict__ vc, int n_ctx) {
    // one thread per 16-byte chunk of a k or v head row
    constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
    constexpr int CPR = DHD / EPC;     // chunks per head row
    const long total = (long)B * T * H * CPR;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int c = (int)(i % CPR);
    const int h = (int)((i / CPR) % H);
    const long row = i / ((long)CPR * H);  // b * T + t
    const int b = (int)(row / T), t = (int)(row % T);
    const int d = H * DHD;
    const size_t esz = BF16 ? 2 : 4;
    const char* src = static_cast<const char*>(qkv) + ((size_t)row * 3 * d + h * DHD + c * EPC) * esz;
    const size_t dst = (((size_t)b * H + h) * n_ctx + pos0 + t) * DHD + c * EPC;
    *reinterpret_cast<u32x4_t*>(static_cast<char*>(kc) + dst * esz) = *reinterpret_cast<const u32x4_t*>(src + d * esz);
    *reinterpret_cast<u32x4_t*>(static_cast<char*>(vc) + dst * esz) =
        *reinterpret_cast<const u32x4_t*>(src + 2 * d * esz);
}

// Eight consecutive elements of a cache row as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t i, float (&v)[8]) {
    if (BF16) {
        const u32x4_t u = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_bits_to_f32(u[e] & 0xffffu);
            v[2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
        }
    } else {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + i);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + i + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = a[e];
            v[4 + e] = b[e];
        }
    }
}

constexpr int DT = 1024;  // threads of a decode-attention workgroup

template <bool BF16>
__global__ __launch_bounds__(DT) void decode_attn_kernel(const void* __restrict__ qkv, const void* __restrict__ kc,
                                                          const void* __restrict__ vc, void* __restrict__ o, int H,
                                                          int n_ctx, int n_keys, float scale_log2) {
    constexpr int KG = DT / 8;  // key groups of the weighted sum (x 8 dimension chunks)
    constexpr int NWV = DT / GPT2_WAVE;
    __shared__ float sq[DHD];
    __shared__ float sp[CHUNK];
    __shared__ float red[NWV];
    __shared__ float so[KG][DHD + 1];
    __shared__ float sl[KG];
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int t = threadIdx.x, wave = t / GPT2_WAVE, lane = t % GPT2_WAVE;
    const int kg = t / 8, dc = t % 8;  // this thread's key group and 8-dimension chunk
    const int d = H * DHD;
    if (t < DHD) sq[t] = load_elem<BF16>(qkv, (size_t)b * 3 * d + h * DHD + t);
    const size_t base = (size_t)bh * n_ctx * DHD;  // this (b, h)'s cache rows
    float m_run = -INFINITY;                       // running maximum (base 2), the same in every thread
    float oacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lacc = 0.f;
    __syncthreads();
    for (int c0 = 0; c0 < n_keys; c0 += CHUNK) {
        const int nk = min(CHUNK, n_keys - c0);
        // scores, one key (a whole 64-element row) per thread
        float lmax = -INFINITY;
        for (int j = t; j < nk; j += DT) {
            const size_t kr = base + (size_t)(c0 + j) * DHD;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < DHD / 8; ++c) {
                float kv8[8];
                load8<BF16>(kc, kr + c * 8, kv8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(sq[c * 8 + e], kv8[e], acc);
            }
            const float sv = acc * scale_log2;
            sp[j] = sv;
            lmax = fmaxf(lmax, sv);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, GPT2_WAVE));
        if (lane == 0) red[wave] = lmax;
        __syncthreads();
        float cmax = red[0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) cmax = fmaxf(cmax, red[w]);
        const float m_new = fmaxf(m_run, cmax);  // finite: every chunk holds at least one key
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        for (int j = t; j < nk; j += DT) sp[j] = __builtin_amdgcn_exp2f(sp[j] - m_new);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[e] *= alpha;
        lacc *= alpha;
        // weighted sum of V: 16-byte pieces of 32 rows per pass, four passes' loads in flight
        int j = kg;
        for (; j + 3 * KG < nk; j += 4 * KG) {
            float v[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) load8<BF16>(vc, base + (size_t)(c0 + j + u * KG) * DHD + dc * 8, v[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float pj = sp[j + u * KG];
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[e] = fmaf(pj, v[u][e], oacc[e]);
                lacc += pj;
            }
        }
        for (; j < nk; j += KG) {
            float v[8];
            load8<BF16>(vc, base + (size_t)(c0 + j) * DHD + dc * 8, v);
            const float pj = sp[j];
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[e] = fmaf(pj, v[e], oacc[e]);
            lacc += pj;
        }
        m_run = m_new;
        __syncthreads();  // sp and red are rewritten by the next chunk
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) so[kg][dc * 8 + e] = oacc[e];
    if (dc == 0) sl[kg] = lacc;
    __syncthreads();
    if (t < DHD) {
        float num = 0.f, den = 0.f;
#pragma unroll 8
        for (int g = 0; g < KG; ++g) {
            num += so[g][t];
            den += sl[g];
        }
        const float r = num / den;
        const size_t oi = (size_t)b * d + h * DHD + t;
        if (BF16)
            static_cast<uint16_t*>(o)[oi] = f32_to_bf16_bits(r);
        else
            static_cast<float*>(o)[oi] = r;
    }
}

__global__ __launch_bounds__(256) void gather_last_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                               int B, int T, int n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)B * n) return;
    const int b = (int)(i / n), c = (int)(i % n);
    dst[i] = src[((size_t)b * T + T - 1) * n + c];
}

}  // namespace

hipError_t kv_append(const void* qkv, int B, int T, int H, int pos0, void* kc, void* vc, int n_ctx, bool bf16,
                     hipStream_t s) {
    const long total = (long)B * T * H * (DHD / (bf16 ? 8 : 4));
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    if (bf16)
        kv_append_kernel<true><<<grid, block, 0, s>>>(qkv, B, T, H, pos0, kc, vc, n_ctx);
    else
        kv_append_kernel<false><<<grid, block, 0, s>>>(qkv, B, T, H, pos0, kc, vc, n_ctx);
    return hipGetLastError();
}

hipError_t decode_attention(const void* qkv, const void* kc, const void* vc, void* o, int B, int H, int n_ctx,
                            int n_keys, bool bf16, hipStream_t s) {
    const float scale_log2 = 0.125f * 1.4426950408889634f;  // (1/sqrt(64)) * log2(e)
    if (bf16)
        decode_attn_kernel<true><<<dim3(B * H), dim3(DT), 0, s>>>(qkv, kc, vc, o, H, n_ctx, n_keys, scale_log2);
    else
        decode_attn_kernel<false><<<dim3(B * H), dim3(DT), 0, s>>>(qkv, kc, vc, o, H, n_ctx, n_keys, scale_log2);
    return hipGetLastError();
}

hipError_t gather_last_rows(const float* src, float* dst, int B, int T, int n, hipStream_t s) {
    const long total = (long)B * n;
    gather_last_rows_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(src, dst, B, T, n);
    return hipGetLastError();
}

}  // namespace gpt2k
