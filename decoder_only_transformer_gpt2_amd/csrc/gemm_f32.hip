// fp32 GEMM for the fp32 compute mode, same contract and epilogues as the bf16 GEMM:
//   C[M, N] = epi(A[M, K] . W[N, K]^T + bias[N]), A and W K-contiguous.
// A 256-thread workgroup owns a 64 x 64 tile of C; each thread accumulates a 4 x 4 block with
// vector-ALU FMAs. K is walked in steps of 16 through LDS, where both slabs are stored k-major so
// that each thread's four A values and four W values are one 16-byte LDS read each.
#include "common.h"

namespace gpt2k {
namespace {

constexpr int TM = 64, TN = 64, TK = 16, PAD = 4;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                       const float* __restrict__ bias, void* __restrict__ Cv, int M,
                                                       int N, int K, long ldc, int gelu_erf, int tiles_m,
                                                       HeadOut ho) {
    __shared__ __attribute__((aligned(16))) float sA[TK][TM + PAD];
    __shared__ __attribute__((aligned(16))) float sW[TK][TN + PAD];
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int m0 = tm * TM, n0 = tn * TN;
    const int t = threadIdx.x, tx = t % 16, ty = t / 16;
    const int lr = t / 4, lk = (t % 4) * 4;  // loader: row of the slab and first k of its float4

    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
        const float4 a = *reinterpret_cast<const float4*>(A + (size_t)(m0 + lr) * K + k0 + lk);
        const float4 w = *reinterpret_cast<const float4*>(W + (size_t)(n0 + lr) * K + k0 + lk);
        __syncthreads();
        sA[lk + 0][lr] = a.x; sA[lk + 1][lr] = a.y; sA[lk + 2][lr] = a.z; sA[lk + 3][lr] = a.w;
        sW[lk + 0][lr] = w.x; sW[lk + 1][lr] = w.y; sW[lk + 2][lr] = w.z; sW[lk + 3][lr] = w.w;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TK; ++k) {
            const float4 av = *reinterpret_cast<const float4*>(&sA[k][ty * 4]);
            const float4 wv = *reinterpret_cast<const float4*>(&sW[k][tx * 4]);
            const float ar[4] = {av.x, av.y, av.z, av.w}, wr[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], wr[j], acc[i][j]);
        }
    }

    if (EPI == EPI_LSE) {
        // per row: (max of y = logit * log2 e, sum of 2^(y - max)) over this tile's columns, merged
        // over the 16 consecutive lanes that hold the row; the lane holding the target keeps it
        constexpr float LOG2E = 1.4426950408889634f;
        const int tiles_n = (N + TN - 1) / TN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + ty * 4 + i;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n0 + tx * 4 + j < N) mx = fmaxf(mx, acc[i][j] * LOG2E);
            const float ms = mx == -INFINITY ? 0.f : mx;
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n0 + tx * 4 + j < N) sum += exp2f(acc[i][j] * LOG2E - ms);
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                const float m2 = __shfl_xor(mx, o, GPT2_WAVE), s2 = __shfl_xor(sum, o, GPT2_WAVE);
                const float mn = fmaxf(mx, m2), mz = mn == -INFINITY ? 0.f : mn;
                sum = sum * exp2f(mx - mz) + s2 * exp2f(m2 - mz);
                mx = mn;
            }
            if (m < M) {
                const int tc = ho.tgt[m];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (tc == n0 + tx * 4 + j && tc < N) ho.tgt_logit[m] = acc[i][j];
                if (tx == 0) {
                    ho.pv[(size_t)m * tiles_n + tn] = mx;
                    ho.ps[(size_t)m * tiles_n + tn] = sum;
                }
            }
        }
    } else if (EPI == EPI_LOGITS) {
        float* C = static_cast<float*>(Cv);
        const int tiles_n = (N + TN - 1) / TN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + ty * 4 + i;
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + tx * 4 + j;
                if (n < N) {
                    if (m < M && C) C[(size_t)m * ldc + n] = acc[i][j];
                    argmax_merge(bv, bi, acc[i][j], n);
                }
            }
            if (ho.pv) {
                // the 16 threads of one row are 16 consecutive lanes of a wavefront
#pragma unroll
                for (int o = 8; o >= 1; o >>= 1) {
                    const float v2 = __shfl_xor(bv, o, GPT2_WAVE);
                    const int i2 = __shfl_xor(bi, o, GPT2_WAVE);
                    argmax_merge(bv, bi, v2, i2);
                }
                if (tx == 0 && m < M) {
                    ho.pv[(size_t)m * tiles_n + tn] = bv;
                    ho.pi[(size_t)m * tiles_n + tn] = bi;
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + ty * 4 + i;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + tx * 4 + j;
                if (n >= N) continue;
                float v = acc[i][j] + bias[n];
                float* C = static_cast<float*>(Cv);
                if (EPI == EPI_BIAS_RESIDUAL) {
                    C[(size_t)m * ldc + n] += v;
                } else {
                    if (EPI == EPI_BIAS_GELU) v = gelu_erf ? gelu_erf_f32(v) : gelu_tanh_f32(v);
                    C[(size_t)m * ldc + n] = v;
                }
            }
        }
    }
}

}  // namespace

hipError_t gemm_f32(const float* A, const float* W, const float* bias, void* C, int M, int N, int K, long ldc, int epi,
                    int gelu_erf, const HeadOut& ho, hipStream_t s) {
    static_assert(kGemmF32BN == TN, "head partial count assumes BN = 64");
    if (ho.res || ho.u) return hipErrorInvalidValue;  // the tiled bf16 kernel's epilogue options only
    const int tiles_m = (M + TM - 1) / TM, tiles_n = (N + TN - 1) / TN;
    dim3 grid(tiles_m * tiles_n), block(256);
#define GPT2_LAUNCH(E) gemm_f32_kernel<E><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, gelu_erf, tiles_m, ho)
    switch (epi) {
        case EPI_BIAS: GPT2_LAUNCH(EPI_BIAS); break;
        case EPI_BIAS_GELU: GPT2_LAUNCH(EPI_BIAS_GELU); break;
        case EPI_BIAS_RESIDUAL: GPT2_LAUNCH(EPI_BIAS_RESIDUAL); break;
        case EPI_LSE: GPT2_LAUNCH(EPI_LSE); break;
        default: GPT2_LAUNCH(EPI_LOGITS); break;
    }
#undef GPT2_LAUNCH
    return hipGetLastError();
}

}  // namespace gpt2k
