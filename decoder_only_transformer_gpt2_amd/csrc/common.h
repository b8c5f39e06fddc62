// Device helpers and kernel-launcher declarations shared by the library's translation units.
// gfx950 (CDNA4) only: 64-wide wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16-byte register vector for global/LDS staging. A native vector (not the uint4 struct) so that a
// load and its later store stay two separate instructions instead of being merged into one copy.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define GPT2_WAVE 64

// bf16 is stored as its raw 16-bit pattern (uint16_t) in every buffer.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// Two floats to two bf16 (round to nearest even) in one word, lo in the low half: one
// v_cvt_pk_bf16_f32 (the same rounding as f32_to_bf16_bits).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, bf16x2_v));
}

// GELU forms. tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); erf form: 0.5 x (1 + erf(x/sqrt 2)).
__device__ __forceinline__ float gelu_tanh_f32(float x) {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * x * (1.0f + tanhf(k0 * (x + 0.044715f * x * x * x)));
}
// The tanh form through the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), on the hardware
// exp2 and reciprocal (about 1 ulp each); saturates correctly at both ends (exp -> 0 or inf).
__device__ __forceinline__ float gelu_tanh_fast(float x) {
    const float u = 0.7978845608028654f * fmaf(0.044715f * x, x * x, x);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);  // exp(-2u) = 2^(-2u log2(e))
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_erf_f32(float x) { return 0.5f * x * (1.0f + erff(x * 0.7071067811865476f)); }
// Their derivatives (the backward pass multiplies the output gradient by them).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    const float t = tanhf(c * (x + 0.044715f * x * x * x));
    return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * c * (1.0f + 3.0f * 0.044715f * x * x);
}
__device__ __forceinline__ float gelu_erf_grad(float x) {
    return 0.5f * (1.0f + erff(x * 0.7071067811865476f)) + x * 0.3989422804014327f * expf(-0.5f * x * x);
}

// (value, index) maximum with ties broken toward the smaller index (selects, no branches).
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    const bool take = (v2 > v) | ((v2 == v) & (i2 < i));
    v = take ? v2 : v;
    i = take ? i2 : i;
}

// Order-preserving map of a float to an unsigned integer (negatives bit-inverted, non-negatives
// with the sign bit set; -0 is first turned into +0 so that it ties with +0 as a float compare
// does), and its inverse. Integer max/min then reduce across lanes in one DPP-fused instruction.
__device__ __forceinline__ uint32_t f32_order_key(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t u) {
    return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Maximum / minimum over each group of 4 consecutive lanes (quad permutes [1,0,3,2], [2,3,0,1]).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t x) {
    x = max(x, dpp_mov<0xB1>(x));
    return max(x, dpp_mov<0x4E>(x));
}
__device__ __forceinline__ uint32_t quad_min_u32(uint32_t x) {
    x = min(x, dpp_mov<0xB1>(x));
    return min(x, dpp_mov<0x4E>(x));
}

// Sum over the 64 lanes of a wavefront (butterfly, result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, GPT2_WAVE);
    return v;
}

// LayerNorm statistics of one row of n fp32 values (n % 4 == 0, n <= 4096) by one wavefront, in the
// order the LayerNorm kernel uses (so both give the same bits): float4 c = i*64 + lane, sums of
// (x + y) + (z + w), mean first, then the centred sum of squares; rstd = 1 / sqrt(var + eps).
__device__ __forceinline__ void row_ln_stats(const float* __restrict__ xr, int n, float eps, float& mean, float& rstd) {
    const int lane = threadIdx.x % GPT2_WAVE, nq = n / 4;
    const f32x4_t* x4 = reinterpret_cast<const f32x4_t*>(xr);
    float s = 0.f;
    for (int c = lane; c < nq; c += GPT2_WAVE) {
        const f32x4_t v = x4[c];
        s += (v[0] + v[1]) + (v[2] + v[3]);
    }
    mean = wave_sum(s) / (float)n;
    float q = 0.f;
    for (int c = lane; c < nq; c += GPT2_WAVE) {
        const f32x4_t v = x4[c];
        const float a0 = v[0] - mean, a1 = v[1] - mean, a2 = v[2] - mean, a3 = v[3] - mean;
        q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
    rstd = 1.0f / sqrtf(wave_sum(q) / (float)n + eps);
}

// row_ln_stats with the row read once into registers (n <= 4096): the same order, the same bits.
// row_ln_load reads the row (float4 c = i*64 + lane into v[i], zeros past the end);
// row_ln_stats_v reduces it.
__device__ __forceinline__ void row_ln_load(const float* __restrict__ xr, int n, f32x4_t (&v)[16]) {
    const int lane = threadIdx.x % GPT2_WAVE, nq = n / 4;
    const f32x4_t* x4 = reinterpret_cast<const f32x4_t*>(xr);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = lane + GPT2_WAVE * i;
        v[i] = c < nq ? x4[c] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
}
__device__ __forceinline__ void row_ln_stats_v(const f32x4_t (&v)[16], int n, float eps, float& mean, float& rstd) {
    const int lane = threadIdx.x % GPT2_WAVE, nq = n / 4;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (lane + GPT2_WAVE * i < nq) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    mean = wave_sum(s) / (float)n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (lane + GPT2_WAVE * i < nq) {
            const float a0 = v[i][0] - mean, a1 = v[i][1] - mean, a2 = v[i][2] - mean, a3 = v[i][3] - mean;
            q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
        }
    rstd = 1.0f / sqrtf(wave_sum(q) / (float)n + eps);
}

// Log-sum-exp partials in base 2: (m, s) stands for 2^m * s. Merging two keeps the larger maximum;
// an empty partial has m = -inf and s = 0.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    const float ms = mn == -INFINITY ? 0.f : mn;  // both empty: 0 * 2^-inf + 0 * 2^-inf = 0
    s = s * __builtin_amdgcn_exp2f(m - ms) + s2 * __builtin_amdgcn_exp2f(m2 - ms);
    m = mn;
}
// The same over each group of 4 consecutive lanes.
__device__ __forceinline__ void lse_quad_merge(float& m, float& s) {
    lse_merge(m, s, __builtin_bit_cast(float, dpp_mov<0xB1>(__builtin_bit_cast(uint32_t, m))),
              __builtin_bit_cast(float, dpp_mov<0xB1>(__builtin_bit_cast(uint32_t, s))));
    lse_merge(m, s, __builtin_bit_cast(float, dpp_mov<0x4E>(__builtin_bit_cast(uint32_t, m))),
              __builtin_bit_cast(float, dpp_mov<0x4E>(__builtin_bit_cast(uint32_t, s))));
}

// ---------------------------------------------------------------------------------------------
// Launchers (each returns the hipError_t of the launch). Pointers are device pointers.
// ---------------------------------------------------------------------------------------------
namespace gpt2k {

// 0-3 as in the C ABI; 4 and 5 are internal: the erf GELU and the log-sum-exp head (no logits).
enum Epi {
    EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_RESIDUAL = 2, EPI_LOGITS = 3, EPI_BIAS_GELU_ERF = 4, EPI_LSE = 5,
    EPI_BIAS_GELU_U = 6, EPI_BIAS_GELU_U_ERF = 7
};

// Per-row, per-column-tile outputs of the vocabulary projection's epilogue ([M, n_part] arrays).
//   EPI_LOGITS: pv/pi = (max logit, first column holding it) when pv is set.
//   EPI_LSE:    pv/ps = (max of y, sum of 2^(y - max)) over the tile with y = logit * log2(e), and
//               tgt_logit[m] = logit of column tgt[m] from the tile holding it (tgt[m] < 0: none).
struct HeadOut {
    float* pv = nullptr;
    float* ps = nullptr;
    int32_t* pi = nullptr;
    const int32_t* tgt = nullptr;
    float* tgt_logit = nullptr;
    // Tiled bf16 GEMM only (more than kSkinnyM rows, row-major output):
    //   EPI_BIAS_RESIDUAL with res set: C = res + (A W^T + b), res an fp32 matrix with C's row stride
    //     (the residual read from one buffer and written to another, instead of C += ...);
    //   EPI_BIAS_GELU_U: u = A W^T + b (fp32, row-major with row stride ldc) and C = gelu(u) in bf16
    //     (row-major or k-blocked; tanh form, the erf form with gelu_erf), the values the plain GELU
    //     epilogue stores.
    const float* res = nullptr;
    float* u = nullptr;
};

// Tile width along N the GEMMs use for a shape: the argmax partial count per row is ceil(N / BN).
int gemm_bf16_tile_n(int M, int N, int K);
constexpr int kGemmF32BN = 64;

// x[m] = wte[tok[m]] + wpe[pos0 + m % T] (rows m of [B, T]).
hipError_t embed(const int32_t* tok, const void* wte, const void* wpe, float* x, int M, int T, int pos0, int d,
                 int n_vocab, bool bf16, int32_t* flags, hipStream_t s);
int embed_flag_count(int M);
// The embedding fused with the first LayerNorm (bf16 tables, k-blocked bf16 output y with kb_rows >= M
// rows per block): writes x as embed() does and y as layernorm(x, g, b, y, ..., kb_rows) would, with
// the same bits; the same token flags as embed().
hipError_t embed_ln(const int32_t* tok, const uint16_t* wte, const uint16_t* wpe, float* x, const float* g,
                    const float* b, uint16_t* y, int M, int T, int pos0, int n, int n_vocab, float eps, int kb_rows,
                    int32_t* flags, hipStream_t s);

// k-blocked layout of a bf16 matrix with `rows` rows and K columns (K a multiple of 32): the
// 32-column blocks one after another, each holding all rows, [K/32][rows][32]. Element (r, k) sits
// at (k / 32 * rows + r) * 32 + k % 32, so the 32-column slab of any range of rows is one
// contiguous run of memory, which the GEMM's DMA reads at full cache-line width.

// kb_rows > 0 (bf16 only): y is written k-blocked with that many rows per block (>= M).
hipError_t layernorm(const float* x, const float* g, const float* b, void* y, int M, int n, float eps,
                     bool out_bf16, hipStream_t s, int kb_rows = 0);

// A must have a_rows >= M readable rows and W w_rows >= N (rows past them are never read).
// kb: A and W are k-blocked with a_rows and w_rows rows per block (M > kSkinnyM only).
// c_kb_rows > 0: the bf16 output (bias or GELU epilogues) is written k-blocked with that many rows
// per block (>= M; N a multiple of 32; M > kSkinnyM only).
hipError_t gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K,
                     long ldc, int epi, int gelu_erf, int a_rows, int w_rows, const HeadOut& ho, hipStream_t s,
                     bool kb = false, int c_kb_rows = 0);
hipError_t gemm_f32(const float* A, const float* W, const float* bias, void* C, int M, int N, int K, long ldc,
                    int epi, int gelu_erf, const HeadOut& ho, hipStream_t s);
// The same for M <= kSkinnyM rows (gemm_bf16 dispatches to it): 16 output columns per workgroup,
// so the head partial count per row is ceil(N / 16). Needs a_rows >= 16 and w_rows >= N rounded
// up to 16 readable rows. w_kb: W is k-blocked ([K/32][w_rows][32]) instead of row-major.
constexpr int kSkinnyM = 16;
// Fusions of the few-row GEMM used by cached decoding:
//   ln_x set: A is LayerNorm(ln_x rows; ln_g, ln_b, ln_eps) (fp32 [M, K] in; normalised and rounded
//             to bf16 into LDS, the same bits the LayerNorm kernel writes; K < 2048); the A
//             argument is unused;
//   kc set:   (bias epilogue of the fused QKV projection, N = 3d) columns [d, 2d) and [2d, 3d) of row m
//             are also written as K and V of sequence m, position kv_pos, into the layer's cache
//             ([B][H][kv_n_ctx][64] bf16 each).
struct SkinnyExtra {
    const float* ln_x = nullptr;
    const float* ln_g = nullptr;
    const float* ln_b = nullptr;
    float ln_eps = 0.f;
    uint16_t* kc = nullptr;
    uint16_t* vc = nullptr;
    int kv_n_ctx = 0;
    int kv_pos = 0;
};
hipError_t gemm_bf16_skinny(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K,
                            int ldc, int epi, int gelu_erf, int a_rows, int w_rows, const HeadOut& ho,
                            const SkinnyExtra& ex, hipStream_t s, bool w_kb = false);

hipError_t argmax_reduce(const float* pv, const int32_t* pi, int M, int n_part, int32_t* out, hipStream_t s);

// Shifted next-token targets: tgt[m] = labels[m + 1] for positions t = m % T < T - 1, -1 for the
// last position of each sequence and for the ignore index; a label outside [0, V) that is not the
// ignore index sets flags[0] = 1 and counts as ignored.
hipError_t xent_targets(const int32_t* labels, int M, int T, int n_vocab, int32_t* tgt, int32_t* flags,
                        hipStream_t s);
// nll[m] = log-sum-exp of row m (from the EPI_LSE partials) - tgt_logit[m], or 0 where tgt[m] < 0.
hipError_t xent_rows(const float* pm, const float* ps, const int32_t* tgt, const float* tgt_logit, int M,
                     int n_part, float* nll, hipStream_t s);
// loss[0] = sum of nll over rows with tgt >= 0 / their count (NaN when none), summed in a fixed order.
hipError_t xent_mean(const float* nll, const int32_t* tgt, int M, float* loss, hipStream_t s);

// o element (b, h, t, e) at o + b*os[0] + h*os[1] + t*os[2] + (e / 32) * os_half + e % 32 (os_half = 32
// for a plain row; the k-blocked layout of [B*T, H*64] has os = {T*32, 2*rows*32, 32}, os_half = rows*32).
// lse_out (optional, [B*H*T] fp32): each query's base-2 log-sum-exp of its scaled scores, for the backward.
hipError_t attention_bf16(const uint16_t* q, const int64_t* qs, const uint16_t* k, const int64_t* ks,
                          const uint16_t* v, const int64_t* vs, uint16_t* o, const int64_t* os, int B, int H,
                          int T, hipStream_t s, int64_t os_half = 32, float* lse_out = nullptr);
hipError_t attention_f32(const float* q, const int64_t* qs, const float* k, const int64_t* ks, const float* v,
                         const int64_t* vs, float* o, const int64_t* os, int B, int H, int T, hipStream_t s);

// Key/value cache of one layer: K and V each [B][H][n_ctx][64] in the compute dtype.
// Copies k, v of the rows of qkv [B, T, 3, H, 64] to positions pos0 .. pos0 + T - 1.
hipError_t kv_append(const void* qkv, int B, int T, int H, int pos0, void* kc, void* vc, int n_ctx, bool bf16,
                     hipStream_t s);
// One query per (b, h) (q of row b of qkv [B, 1, 3, H, 64]) against cached keys 0 .. n_keys - 1:
// o[b, h*64 .. h*64+63] = sum_j softmax_j(q . k_j / 8) v_j, fp32 softmax, output in the dtype.
hipError_t decode_attention(const void* qkv, const void* kc, const void* vc, void* o, int B, int H, int n_ctx,
                            int n_keys, bool bf16, hipStream_t s);
// dst[b] = src[b * T + T - 1] for rows of n fp32 values.
hipError_t gather_last_rows(const float* src, float* dst, int B, int T, int n, hipStream_t s);

// Sampled next token of each of B rows of fp32 logits (row stride ld, V <= sample_max_vocab()):
// repetition penalty over hist[b, 0 .. n_hist) (row stride hist_ld, may be null), division by the
// temperature, top-k (0 = off), top-p (1 = off), then the inverse-CDF draw at u[b]. n_kept may be null.
// With a workspace of sample_workspace_bytes(B, V) bytes (256-byte aligned) the top-k case is spread
// over many workgroups per row; ws = null keeps every row on one workgroup.
hipError_t sample(const float* logits, long ld, int B, int V, const int32_t* hist, long hist_ld, int n_hist,
                  float temperature, int top_k, float top_p, float penalty, const float* u, int32_t* out,
                  int32_t* n_kept, void* ws, size_t ws_bytes, hipStream_t s);
size_t sample_workspace_bytes(int B, int V);
int sample_max_vocab();

// Backward pass (train.hip).
// dst[c * ldd + r] = src[r * lds + c] (r < R, c < C) and 0 for R <= r < Rp; fp32 or bf16 each side.
hipError_t transpose(const void* src, bool src_bf16, long lds, int R, int C, void* dst, bool dst_bf16, long ldd, int Rp,
                     hipStream_t s);
// out[c] = sum over rows of src[r * ld + c] (deterministic order); part holds colsum_blocks(R) * C floats.
int colsum_blocks(int R);
hipError_t colsum(const float* src, long ld, int R, int C, float* part, float* out, hipStream_t s);
// out[c] = sum over b < nb of part[b * C + c] for up to kColsumSegs independent (part, nb, C, out)
// segments in one launch, each in the fixed order of colsum.
struct ColsumSeg {
    const float* part;
    float* out;
    int nb, C;
};
constexpr int kColsumSegs = 64;
struct ColsumSegs {
    ColsumSeg seg[kColsumSegs];
    int n = 0;
};
hipError_t colsum_reduce_multi(const ColsumSegs& segs, hipStream_t s);
// LayerNorm backward on rows of x with output gradient dy (fp32 [M, d]): dx += the input gradient,
// dgamma / dbeta = column sums (pg, pb hold ln_backward_blocks(M) * d floats each: partial rows).
// With y16 (and pd, ln_backward_blocks(M) * d floats): the updated dx rows also in bf16 (row stride
// d, rows 0..M-1 only) and their column sums' partial rows in pd, for a later colsum_reduce_multi.
int ln_backward_blocks(int M);
hipError_t ln_backward(const float* x, const float* gamma, const float* dy, float* dx, int M, int d, float eps, float* pg,
                       float* pb, float* dgamma, float* dbeta, hipStream_t s, uint16_t* y16 = nullptr,
                       float* pd = nullptr);
// h = gelu(u) in the compute dtype; g *= gelu'(u) in place (fp32).
hipError_t gelu_forward(const float* u, void* h, long n, bool bf16, int erf_form, hipStream_t s);
hipError_t gelu_backward(const float* u, float* g, long n, int erf_form, hipStream_t s);
// From fp32 logits [M, V] (row stride ld) and targets: cnt[0] = counted rows, nll[m], and the loss
// gradient [M, Vp] (compute dtype; zero past V and on rows without target).
hipError_t xent_grad(const float* logits, long ld, int M, int V, int Vp, const int32_t* tgt, int32_t* cnt, float* nll,
                     void* dlogits, bool bf16, hipStream_t s);
// Causal attention backward, fp32 mode: qkv [B, T, 3, H, 64] and o [B, T, H, 64] with the output
// gradient dout [B, T, H * 64]: dqkv [B, T, 3 * H * 64]; lse, dvec [B * H * T] are scratch.
hipError_t attention_backward(const void* qkv, const void* o, const float* dout, float* dqkv, float* lse, float* dvec,
                              int B, int H, int T, bool bf16, hipStream_t s);
// bf16 mode (matrix cores): dqkv in bf16 (rows 0 .. B*T-1) and the column sums of every 64-row tile
// of each sequence in part ([attention_backward_parts(B, T)][3 * H * 64] floats); lse is the forward's
// attention_bf16 lse_out, dvec [B * H * T] scratch.
int attention_backward_parts(int B, int T);
hipError_t attention_backward_bf16(const uint16_t* qkv, const uint16_t* o, const float* dout, uint16_t* dqkv,
                                   float* part, float* lse, float* dvec, int B, int H, int T, hipStream_t s);
// gwpe[t] = sum_b dx[b, t] (0 for t >= T, all n_ctx rows written); gwte[tok[m]] += dx[m].
hipError_t embed_backward(const int32_t* tok, const float* dx, int B, int T, int n_ctx, int d, int V, float* gwte,
                          float* gwpe, hipStream_t s);

// dst[i] = i < n_src ? convert(src[i]) : 0 for i < n_dst (element types fp32 or bf16).
hipError_t convert(const void* src, bool src_bf16, void* dst, bool dst_bf16, long n_src, long n_dst,
                   hipStream_t s);
// dst = the k-blocked copy of the row-major bf16 matrix src [rows][K] (K a multiple of 32).
hipError_t kblock_bf16(const uint16_t* src, uint16_t* dst, long rows, int K, hipStream_t s);

}  // namespace gpt2k
