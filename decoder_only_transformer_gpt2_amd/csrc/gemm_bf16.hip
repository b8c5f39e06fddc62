// bf16 GEMM on the gfx950 matrix cores with fused epilogues:
//   C[M, N] = epi(A[M, K] . W[N, K]^T + bias[N])
// A (activations) and W (nn.Linear weights, [out, in]) are both K-contiguous. Used for c_attn,
// attn.c_proj, mlp.c_fc, mlp.c_proj and the tied lm_head ("复现GPT-2 124M" §2.1 and §2.4,
// "从零手写GPT-2" §4.1).
//
// Tiling: a 256-thread workgroup (4 wavefronts as 2 x 2) owns a BM x BN tile of C and walks K in
// steps of 64. Each step's A and W slabs are staged global -> registers -> LDS (double-buffered,
// one barrier per step); 16-byte chunks are XOR-swizzled by row so the 16-byte fragment reads of
// a wavefront spread over all LDS banks. Each wavefront computes (BM/2) x (BN/2) with
// v_mfma_f32_16x16x32_bf16 and keeps the fp32 accumulators in registers to the epilogue.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int BK = 64;  // K per LDS stage (eight 16-byte chunks per row)

// LDS element offset of (row, 16-byte chunk) in a [rows][64] bf16 slab with the XOR swizzle.
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

template <int ROWS>
__device__ __forceinline__ void load_slab(const uint16_t* __restrict__ g, int ld, int k0, uint4 (&r)[ROWS / 32]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < ROWS / 32; ++i) {
        const int row = t / 8 + 32 * i, chunk = t % 8;
        r[i] = *reinterpret_cast<const uint4*>(g + (size_t)row * ld + k0 + chunk * 8);
    }
}

template <int ROWS>
__device__ __forceinline__ void store_slab(uint16_t* s, const uint4 (&r)[ROWS / 32]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < ROWS / 32; ++i) {
        const int row = t / 8 + 32 * i, chunk = t % 8;
        *reinterpret_cast<uint4*>(s + swz(row, chunk)) = r[i];
    }
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                        const float* __restrict__ bias, void* __restrict__ Cv, int M,
                                                        int N, int K, long ldc, int gelu_erf, int tiles_m,
                                                        float* __restrict__ amax_v, int32_t* __restrict__ amax_i) {
    constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * BK];

    // consecutive workgroups share a W tile (walk down M first)
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int wm = wave / 2, wn = wave % 2;
    const int r16 = lane & 15, g4 = lane >> 4;

    const uint16_t* Ab = A + (size_t)m0 * K;
    const uint16_t* Wb = W + (size_t)n0 * K;

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[BM / 32], rw[BN / 32];
    load_slab<BM>(Ab, K, 0, ra);
    load_slab<BN>(Wb, K, 0, rw);
    store_slab<BM>(sA[0], ra);
    store_slab<BN>(sW[0], rw);
    __syncthreads();

    const int nk = K / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_slab<BM>(Ab, K, (kt + 1) * BK, ra);
            load_slab<BN>(Wb, K, (kt + 1) * BK, rw);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8_t af[FM], wf[FN];
            const int chunk = kk * 4 + g4;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[cur][swz(wm * WM + i * 16 + r16, chunk)]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                wf[j] = *reinterpret_cast<const bf16x8_t*>(&sW[cur][swz(wn * WN + j * 16 + r16, chunk)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            store_slab<BM>(sA[cur ^ 1], ra);
            store_slab<BN>(sW[cur ^ 1], rw);
        }
        __syncthreads();
    }

    // Epilogue. acc[i][j][e] holds C[row, col] with row = wm*WM + i*16 + 4*g4 + e and
    // col = wn*WN + j*16 + r16 (the 16x16 MFMA accumulator layout).
    if (EPI == EPI_LOGITS) {
        float* C = static_cast<float*>(Cv);
        __shared__ float red_v[2][BM];
        __shared__ int red_i[2][BM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = wm * WM + i * 16 + 4 * g4 + e;
                const int m = m0 + rl;
                float bv = -INFINITY;
                int bi = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = n0 + wn * WN + j * 16 + r16;
                    const float v = acc[i][j][e];
                    if (n < N) {
                        if (m < M) C[(size_t)m * ldc + n] = v;
                        argmax_merge(bv, bi, v, n);
                    }
                }
                if (amax_v) {
#pragma unroll
                    for (int o = 8; o >= 1; o >>= 1) {
                        const float v2 = __shfl_xor(bv, o, GPT2_WAVE);
                        const int i2 = __shfl_xor(bi, o, GPT2_WAVE);
                        argmax_merge(bv, bi, v2, i2);
                    }
                    if (r16 == 0) {
                        red_v[wn][rl] = bv;
                        red_i[wn][rl] = bi;
                    }
                }
            }
        }
        if (amax_v) {
            __syncthreads();
            const int tiles_n = (N + BN - 1) / BN;
            for (int rl = threadIdx.x; rl < BM; rl += 256) {
                const int m = m0 + rl;
                if (m < M) {
                    float bv = red_v[0][rl];
                    int bi = red_i[0][rl];
                    argmax_merge(bv, bi, red_v[1][rl], red_i[1][rl]);
                    amax_v[(size_t)m * tiles_n + tn] = bv;
                    amax_i[(size_t)m * tiles_n + tn] = bi;
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + j * 16 + r16;
            if (n >= N) continue;
            const float bn = bias[n];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + wm * WM + i * 16 + 4 * g4 + e;
                    if (m >= M) continue;
                    float v = acc[i][j][e] + bn;
                    if (EPI == EPI_BIAS_RESIDUAL) {
                        float* C = static_cast<float*>(Cv);
                        C[(size_t)m * ldc + n] += v;
                    } else {
                        if (EPI == EPI_BIAS_GELU) v = gelu_erf ? gelu_erf_f32(v) : gelu_tanh_f32(v);
                        static_cast<uint16_t*>(Cv)[(size_t)m * ldc + n] = f32_to_bf16_bits(v);
                    }
                }
            }
        }
    }
}

template <int BM, int BN>
hipError_t launch(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K, long ldc,
                  int epi, int gelu_erf, float* av, int32_t* ai, hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    dim3 grid(tiles_m * tiles_n), block(256);
    switch (epi) {
        case EPI_BIAS:
            gemm_bf16_kernel<BM, BN, EPI_BIAS><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, gelu_erf, tiles_m, av, ai);
            break;
        case EPI_BIAS_GELU:
            gemm_bf16_kernel<BM, BN, EPI_BIAS_GELU><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, gelu_erf, tiles_m, av, ai);
            break;
        case EPI_BIAS_RESIDUAL:
            gemm_bf16_kernel<BM, BN, EPI_BIAS_RESIDUAL><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, gelu_erf, tiles_m, av, ai);
            break;
        default:
            gemm_bf16_kernel<BM, BN, EPI_LOGITS><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, gelu_erf, tiles_m, av, ai);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K, long ldc,
                     int epi, int gelu_erf, float* amax_v, int32_t* amax_i, hipStream_t s) {
    static_assert(kGemmBf16BN == 128, "argmax partial count assumes BN = 128");
    return launch<128, 128>(A, W, bias, C, M, N, K, ldc, epi, gelu_erf, amax_v, amax_i, s);
}

}  // namespace gpt2k
