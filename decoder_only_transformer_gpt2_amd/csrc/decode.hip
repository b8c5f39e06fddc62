// Incremental decoding with a key/value cache ([手写] §6.3 and [解析] §4.2: generation feeds one new
// token per step; the keys and values of the earlier positions do not change, so they are kept
// instead of recomputed). Per layer the cache holds K and V as [B][H][n_ctx][64] in the compute
// dtype. A decode step's query attends to keys 0 .. pos: causality makes this the last row of the
// full forward over the extended sequence.
//
// Decode attention is bound by reading the cache (HBM), not by arithmetic: one 1024-thread
// workgroup per (b, h), split into 128 groups of eight lanes. Group g takes keys g, g + 128, ...;
// lane i of a group holds dimensions 8i .. 8i+7 of the query, of each of its keys and of its value
// rows, so a wavefront's load covers eight whole rows. The K and V rows of up to eight keys per
// group (four in fp32) are loaded together, one round trip per batch (1024 keys in bf16); a key's
// score is the sum of the eight lanes' partial dot products (three butterfly steps). Each group
// keeps its own running maximum, sum and weighted sum of V (online softmax in fp32, exp2 with the
// scale folded in); at the end the groups are rescaled to the workgroup's maximum and summed
// through LDS. (Splitting the keys of a (b, h) over several workgroups shortens this kernel, but
// the projection that reads o then has to combine every split's state in each of its workgroups,
// which costs as much as it saves.)
#include "common.h"

namespace gpt2k {
namespace {

constexpr int DHD = 64;      // head size

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

// Eight consecutive elements (bf16 or fp32, 16-byte aligned) as fp32.
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

// 16-byte (bf16) or 32-byte (fp32) piece of a cache row, kept raw until it is used.
template <bool BF16>
struct RowPiece {
    u32x4_t u[BF16 ? 1 : 2];
};
template <bool BF16>
__device__ __forceinline__ RowPiece<BF16> load_piece(const void* base, size_t i) {
    RowPiece<BF16> r;
    if constexpr (BF16) {
        r.u[0] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i);
    } else {
        r.u[0] = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(base) + i);
        r.u[1] = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(base) + i + 4);
    }
    return r;
}
template <bool BF16>
__device__ __forceinline__ float piece_elem(const RowPiece<BF16>& r, int e) {
    if constexpr (BF16)
        return bf16_bits_to_f32(e & 1 ? r.u[0][e >> 1] >> 16 : r.u[0][e >> 1] & 0xffffu);
    else  // (not __builtin_bit_cast on the vector element: hipcc then read element 0 for every e)
        return __uint_as_float(r.u[e >> 2][e & 3]);
}

constexpr int DT = 1024;  // threads of a decode-attention workgroup

template <bool BF16>
__global__ __launch_bounds__(DT) void decode_attn_kernel(const void* __restrict__ qkv, const void* __restrict__ kc,
                                                          const void* __restrict__ vc, void* __restrict__ o, int H,
                                                          int n_ctx, int n_keys, float scale_log2) {
    constexpr int KG = DT / 8;  // key groups of eight lanes
    constexpr int NWV = DT / GPT2_WAVE;
    constexpr int KPB = BF16 ? 8 : 4;  // keys per group and batch
    __shared__ float red[NWV];
    __shared__ float so[KG][DHD + 1];
    __shared__ float sl[KG];
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int t = threadIdx.x, wave = t / GPT2_WAVE, lane = t % GPT2_WAVE;
    const int kg = t / 8, dc = t % 8;  // key group, 8-dimension piece
    const int d = H * DHD;
    float q[8];
    load8<BF16>(qkv, (size_t)b * 3 * d + h * DHD + dc * 8, q);
    const size_t base = (size_t)bh * n_ctx * DHD + dc * 8;  // this lane's piece of row 0 of (b, h)
    float m_run = -INFINITY;  // the group's running maximum (base 2)
    float lacc = 0.f, oacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = kg; j0 < n_keys; j0 += KG * KPB) {
        RowPiece<BF16> kp[KPB], vp[KPB];
#pragma unroll
        for (int u = 0; u < KPB; ++u) {
            const int j = j0 + u * KG;
            if (j < n_keys) {
                kp[u] = load_piece<BF16>(kc, base + (size_t)j * DHD);
                vp[u] = load_piece<BF16>(vc, base + (size_t)j * DHD);
            }
        }
        float sc[KPB];
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < KPB; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(q[e], piece_elem<BF16>(kp[u], e), acc);
            acc += __shfl_xor(acc, 1, 8);
            acc += __shfl_xor(acc, 2, 8);
            acc += __shfl_xor(acc, 4, 8);
            sc[u] = j0 + u * KG < n_keys ? acc * scale_log2 : -INFINITY;
            mb = fmaxf(mb, sc[u]);
        }
        const float m_new = fmaxf(m_run, mb);  // finite: key j0 is valid
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        lacc *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[e] *= alpha;
#pragma unroll
        for (int u = 0; u < KPB; ++u) {
            if (j0 + u * KG < n_keys) {
                const float p = __builtin_amdgcn_exp2f(sc[u] - m_new);
                lacc += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) oacc[e] = fmaf(p, piece_elem<BF16>(vp[u], e), oacc[e]);
            }
        }
        m_run = m_new;
    }
    // the workgroup's maximum, then every group rescaled to it and summed through LDS
    float wm = m_run;
#pragma unroll
    for (int off = 32; off >= 8; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off, GPT2_WAVE));
    if (lane == 0) red[wave] = wm;
    __syncthreads();
    float mx = red[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) mx = fmaxf(mx, red[w]);
    const float sw = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);  // a group without keys: 0
#pragma unroll
    for (int e = 0; e < 8; ++e) so[kg][dc * 8 + e] = oacc[e] * sw;
    if (dc == 0) sl[kg] = lacc * sw;
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
