// bf16 products with operands stored reduction-dimension-outermost (gemm_bf16_tn.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace gpt2k {
// C[m][n] (fp32, row stride ldc) = sum_k A(k, m) B(k, n) for m < M, n < N, k < K (K a multiple of
// 64). A(k, m) is A[k * lda + m] when a_mmajor, else A[m * lda + k]; likewise B (b_mmajor must be
// set). a_lim / b_lim bound what is read: the row count of a K-major operand, the row width of an
// M-major one (a multiple of 8); tiles reaching past it read duplicates of valid data, and only
// C[m < M][n < N] is written. Rows k < K of an M-major operand must exist and hold finite values;
// where the other operand's row k is zero they contribute nothing.
// part: optional fp32 scratch of part_elems floats. With room for a few M x N partial products, a
// product with few output tiles or a reduction over thousands of rows is split along K and its
// partial products summed in a fixed order (the result repeats bit for bit from run to run).
// The GELU backward step fused into an input-gradient product (A K-major, B M-major, BM = 64 tiles):
// instead of C, g = C * gelu'(u) (u fp32 [M][ldu], the GELU input; erf selects the erf form) is
// written in bf16 to y [rows][ldy] (rows M .. ceil(M/64)*64 - 1 get 0), and the sums of g over each
// 64-row block to part[block][N] (the bias gradient's partial column sums).
struct TnGeluBack {
    const float* u = nullptr;
    long ldu = 0;
    uint16_t* y = nullptr;
    long ldy = 0;
    float* part = nullptr;
    int erf = 0;
};
hipError_t gemm_bf16_tn(const uint16_t* A, bool a_mmajor, long lda, int a_lim, const uint16_t* B, bool b_mmajor,
                        long ldb, int b_lim, float* C, long ldc, int M, int N, int K, hipStream_t s,
                        float* part = nullptr, size_t part_elems = 0, const TnGeluBack* gb = nullptr,
                        bool b_kb = false);
// (b_kb: B is M-major and k-blocked, [N/32][ldb][32] with ldb >= K rows per block; weight gradients only)
}  // namespace gpt2k
