// GEMM for a handful of rows (M <= 16: one token per sequence in cached decoding), same contract
// and epilogues as the tiled bf16 GEMM: C[M, N] = epi(A[M, K] . W[N, K]^T + bias[N]).
//
// With so few rows the product is a stream over W: every weight is read once and used M times,
// so the time is W's bytes over HBM bandwidth if enough of W is in flight. A 256-thread workgroup
// owns 16 output columns; its wavefronts (four, or sixteen for K >= 2048) take interleaved
// 32-wide slices of K and run
// v_mfma_f32_16x16x32_bf16 on 16 (padded) rows of A straight from global memory (A is a few KB and
// stays in L2), so no cross-lane reduction is needed; the partial accumulators are summed
// through LDS and the first wavefront applies the epilogue. The grid has ceil(N/16) workgroups:
// 144 for the QKV projection, 3142 for the vocabulary projection.
#include "common.h"

namespace gpt2k {
namespace {

// Reductions over each group of 16 consecutive lanes (a DPP row), result in every lane.
template <int ROR>
__device__ __forceinline__ uint32_t ror16(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x120 + ROR, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t row16_max_u(uint32_t x) {
    x = max(x, ror16<8>(x));
    x = max(x, ror16<4>(x));
    x = max(x, ror16<2>(x));
    return max(x, ror16<1>(x));
}
__device__ __forceinline__ uint32_t row16_min_u(uint32_t x) {
    x = min(x, ror16<8>(x));
    x = min(x, ror16<4>(x));
    x = min(x, ror16<2>(x));
    return min(x, ror16<1>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, ror16<8>(__builtin_bit_cast(uint32_t, x)));
    x += __builtin_bit_cast(float, ror16<4>(__builtin_bit_cast(uint32_t, x)));
    x += __builtin_bit_cast(float, ror16<2>(__builtin_bit_cast(uint32_t, x)));
    return x + __builtin_bit_cast(float, ror16<1>(__builtin_bit_cast(uint32_t, x)));
}

template <int EPI, int KW, bool LNA>  // KW wavefronts split K; LNA: A = LayerNorm(ex.ln_x)
__global__ __launch_bounds__(64 * KW) void gemm_skinny_kernel(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ W,
                                                              const float* __restrict__ bias, void* __restrict__ Cv,
                                                              int M, int N, int K, int ldc, HeadOut ho,
                                                              SkinnyExtra ex) {
    __shared__ f32x4_t red[KW][64];
    __shared__ float ln_mean[16], ln_rstd[16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / GPT2_WAVE), lane = threadIdx.x % GPT2_WAVE;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int n0 = blockIdx.x * 16;
    // operand fragments: A row r16 (rows >= M are padding; they only reach outputs never stored),
    // W row n0 + r16, each lane 8 consecutive k at 8*g4 within a 32-wide slice
    const uint16_t* ap = A + (size_t)r16 * K + 8 * g4;
    const uint16_t* wp = W + (size_t)(n0 + r16) * K + 8 * g4;
    const bool arow = r16 < M;
    const float* xp = ex.ln_x + (size_t)r16 * K + 8 * g4;
    float a_mean = 0.f, a_rstd = 0.f;  // row r16's statistics, set once they are computed
    auto a_frag = [&](int c) -> bf16x8_t {
        if (!LNA) return *reinterpret_cast<const bf16x8_t*>(ap + c * 32);
        u32x4_t u = {0u, 0u, 0u, 0u};
        if (arow) {
            const int k = c * 32 + 8 * g4;
            const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(xp + c * 32);
            const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(xp + c * 32 + 4);
            const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(ex.ln_g + k);
            const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(ex.ln_g + k + 4);
            const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(ex.ln_b + k);
            const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(ex.ln_b + k + 4);
            u[0] = pack_bf16x2((x0[0] - a_mean) * a_rstd * g0[0] + b0[0], (x0[1] - a_mean) * a_rstd * g0[1] + b0[1]);
            u[1] = pack_bf16x2((x0[2] - a_mean) * a_rstd * g0[2] + b0[2], (x0[3] - a_mean) * a_rstd * g0[3] + b0[3]);
            u[2] = pack_bf16x2((x1[0] - a_mean) * a_rstd * g1[0] + b1[0], (x1[1] - a_mean) * a_rstd * g1[1] + b1[1]);
            u[3] = pack_bf16x2((x1[2] - a_mean) * a_rstd * g1[2] + b1[2], (x1[3] - a_mean) * a_rstd * g1[3] + b1[3]);
        }
        return __builtin_bit_cast(bf16x8_t, u);
    };
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int nch = K / 32;
    // rounds of up to eight slices: every load of a round is in flight before the first MFMA waits
    // (a wavefront has six slices in the decoding shapes, so its W stream is one round trip). The
    // first round's W loads are issued before the LayerNorm statistics, so they overlap.
    bf16x8_t wf[8];
    {
        const int ns = min(8, (nch - wave + KW - 1) / KW);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < ns) wf[u] = *reinterpret_cast<const bf16x8_t*>(wp + (wave + u * KW) * 32);
    }
    if (LNA) {
        for (int m = wave; m < M; m += KW) {
            float mean, rstd;
            row_ln_stats_reg(ex.ln_x + (size_t)m * K, K, ex.ln_eps, mean, rstd);
            if (lane == 0) {
                ln_mean[m] = mean;
                ln_rstd[m] = rstd;
            }
        }
        __syncthreads();
        if (arow) {
            a_mean = ln_mean[r16];
            a_rstd = ln_rstd[r16];
        }
    }
    for (int c = wave; c < nch; c += 8 * KW) {
        const int ns = min(8, (nch - c + KW - 1) / KW);  // wave-uniform
        bf16x8_t af[8];
        if (c != wave) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u < ns) wf[u] = *reinterpret_cast<const bf16x8_t*>(wp + (c + u * KW) * 32);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < ns) af[u] = a_frag(c + u * KW);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < ns) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u], wf[u], acc, 0, 0, 0);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < KW; ++w) acc += red[w][lane];

    // acc[e] = C[row 4*g4 + e, column n0 + r16]
    const int n = n0 + r16;
    const bool ncol = n < N;
    const int n_part = gridDim.x;
    constexpr bool HEAD = EPI == EPI_LOGITS || EPI == EPI_LSE;
    const float b = (!HEAD && ncol) ? bias[n] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = 4 * g4 + e;
        const bool ok = ncol && m < M;
        float v = acc[e] + b;
        if (EPI == EPI_BIAS_GELU) v = gelu_tanh_fast(v);
        if (EPI == EPI_BIAS_GELU_ERF) v = gelu_erf_f32(v);
        if (EPI == EPI_BIAS_RESIDUAL) {
            if (ok) static_cast<float*>(Cv)[(size_t)m * ldc + n] += v;
        } else if (EPI == EPI_LOGITS) {
            if (ok && Cv) static_cast<float*>(Cv)[(size_t)m * ldc + n] = v;
            if (ho.pv) {
                // (max, first column) over the row's 16 columns of this workgroup
                const uint32_t key = ncol ? f32_order_key(v) : 0u;
                const uint32_t kmax = row16_max_u(key);
                const uint32_t col = (ncol && key == kmax) ? (uint32_t)n : 0xffffffffu;
                const uint32_t cmin = row16_min_u(col);
                if (r16 == 0 && m < M) {
                    ho.pv[(size_t)m * n_part + blockIdx.x] = f32_from_order_key(kmax);
                    ho.pi[(size_t)m * n_part + blockIdx.x] = (int32_t)cmin;
                }
            }
        } else if (EPI == EPI_LSE) {
            constexpr float LOG2E = 1.4426950408889634f;
            const float y = ncol ? v * LOG2E : -INFINITY;
            const float mx = f32_from_order_key(row16_max_u(f32_order_key(y)));  // column 0 is always valid
            const float sum = row16_sum(__builtin_amdgcn_exp2f(y - mx));
            if (m < M) {
                if (r16 == 0) {
                    ho.pv[(size_t)m * n_part + blockIdx.x] = mx;
                    ho.ps[(size_t)m * n_part + blockIdx.x] = sum;
                }
                if (ncol && ho.tgt[m] == n) ho.tgt_logit[m] = v;
            }
        } else {
            if (ok) {
                const uint16_t bits = f32_to_bf16_bits(v);
                static_cast<uint16_t*>(Cv)[(size_t)m * ldc + n] = bits;
                if (EPI == EPI_BIAS && ex.kc) {  // fused QKV: k and v of this position into the cache
                    const int d = N / 3, H = d / 64;
                    if (n >= d) {
                        const int nn = n < 2 * d ? n - d : n - 2 * d;
                        uint16_t* cache = n < 2 * d ? ex.kc : ex.vc;
                        cache[(((size_t)m * H + nn / 64) * ex.kv_n_ctx + ex.kv_pos) * 64 + nn % 64] = bits;
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t gemm_bf16_skinny(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K,
                            int ldc, int epi, int gelu_erf, int a_rows, int w_rows, const HeadOut& ho,
                            const SkinnyExtra& ex, hipStream_t s) {
    if (M < 1 || M > kSkinnyM || K % 32 || a_rows < 16 || w_rows < (N + 15) / 16 * 16) return hipErrorInvalidValue;
    if (ex.ln_x && (K % 8 || K > 4096)) return hipErrorInvalidValue;
    if (ex.kc && (epi != EPI_BIAS || N % 3 || (N / 3) % 64)) return hipErrorInvalidValue;
    // long K over few columns: sixteen wavefronts per workgroup keep enough of W in flight
    const bool wide = K >= 2048, lna = ex.ln_x != nullptr;
    const dim3 grid((N + 15) / 16), block(wide ? 1024 : 256);
#define GPT2_LAUNCH_KW(E, KWV)                                                                                  \
    do {                                                                                                        \
        if (lna)                                                                                                \
            gemm_skinny_kernel<E, KWV, true><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, ho, ex);       \
        else                                                                                                    \
            gemm_skinny_kernel<E, KWV, false><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, ho, ex);      \
    } while (0)
#define GPT2_LAUNCH(E)            \
    do {                          \
        if (wide)                 \
            GPT2_LAUNCH_KW(E, 16); \
        else                      \
            GPT2_LAUNCH_KW(E, 4);  \
    } while (0)
    switch (epi) {
        case EPI_BIAS: GPT2_LAUNCH(EPI_BIAS); break;
        case EPI_BIAS_GELU:
            if (gelu_erf)
                GPT2_LAUNCH(EPI_BIAS_GELU_ERF);
            else
                GPT2_LAUNCH(EPI_BIAS_GELU);
            break;
        case EPI_BIAS_RESIDUAL: GPT2_LAUNCH(EPI_BIAS_RESIDUAL); break;
        case EPI_LSE: GPT2_LAUNCH(EPI_LSE); break;
        default: GPT2_LAUNCH(EPI_LOGITS); break;
    }
#undef GPT2_LAUNCH
#undef GPT2_LAUNCH_KW
    return hipGetLastError();
}

}  // namespace gpt2k
