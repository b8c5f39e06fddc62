// bf16 products of the backward pass whose operands are stored with the reduction dimension
// outermost: C[m][n] (fp32) = sum_k A(k, m) B(k, n), with A(k, m) at A[m * lda + k] (K-major, the
// nn.Linear layout) or at A[k * lda + m] (M-major), and likewise B. The weight gradient
// dW = dY^T X reduces over the rows of dY and X (both M-major), the input gradient dX = dY W reads
// W [out][in] with the reduction over its rows (B M-major). M-major tiles are staged in LDS as
// [k][m] and turned into matrix-core operands by ds_read_b64_tr_b16, so no transposed copy of any
// operand is made.
//
// Tiling as in the forward projections: a workgroup owns a BM x BN tile of C and walks K in steps of
// 64 through a ring of S LDS stages filled by LDS DMA (global_load_lds, 16 bytes per lane, one 1 KB
// block per instruction), issued S-1 steps ahead. LDS layouts (16-byte chunks permuted so that the
// fragment reads of 32 lanes fall on distinct banks):
//  * K-major operand: [rows][64], chunk c of row r at c ^ (r & 7); a fragment (16 rows x 32 k) is
//    one 16-byte read per lane;
//  * M-major operand of width BX: [64][BX], chunk c of k-row k at c ^ mswz(k); a fragment is two
//    ds_read_b64_tr_b16 per lane (k 8g..8g+3 and 8g+4..8g+7 of its column, g = lane / 16).
// The accumulators are stored straight to C (fp32; 16 consecutive columns per row and instruction).
#include "gemm_bf16_impl.h"
#include "gemm_tn.h"

namespace gpt2k {
namespace {

constexpr int TBK = 64;  // K step

// Chunk permutation of k-row k of an M-major tile of width BX. The two transposing reads of a
// fragment cover, for 32 lanes, k-rows {b, b+1, b+2, b+3, b+8, .., b+11} (b a multiple of 4, the
// second read b+4) x 32 bytes: with 256-byte rows (BX >= 128) the eight rows need eight different
// even chunk offsets, with 128-byte rows (BX = 64; rows k and k+1 lie on different bank halves)
// four per half.
template <int BX>
__device__ __forceinline__ int mswz(int k) {
    if constexpr (BX == 64)
        return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));
    else
        return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
}

typedef short short4_t __attribute__((vector_size(8)));
__device__ __forceinline__ u32x2_t lds_tr16(const uint16_t* p) {
    const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// BKB: the M-major B operand is k-blocked ([N/32][ldb][32]: element (k, n) at ((n / 32) * ldb + k) * 32 + n % 32).
template <int BM, int BN, int S, int WGM, int WGN, bool AMM, bool BMM, int NKT, bool GB = false, bool BKB = false>
__global__ __launch_bounds__(64 * WGM * WGN, S * (BM + BN) * TBK * 2 <= 80 * 1024 ? 2 : 1) void gemm_tn_kernel(
    const uint16_t* __restrict__ A, long lda, int a_lim, const uint16_t* __restrict__ B, long ldb, int b_lim,
    float* __restrict__ C, long ldc, int M, int N, int K, int tiles_m, int ntiles, TnGeluBack gb) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
    constexpr int SA = BM * TBK, SB = BN * TBK, STAGE = SA + SB;  // bf16 elements
    constexpr int NIA = SA / 512, NIB = SB / 512, NI = NIA + NIB;  // 1 KB DMA instructions per stage
    constexpr int PW = (NI + NW - 1) / NW;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
    static_assert(!AMM || BM == 64 || BM == 128 || BM == 256, "M-major width");
    static_assert(!BMM || BN == 64 || BN == 128 || BN == 256, "M-major width");
    static_assert(S >= 2 && S <= 4 && (S - 1) * PW < 64, "ring depth");
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[STAGE];
    __shared__ __attribute__((aligned(S > 2 ? 1024 : 2))) uint16_t lds2[S > 2 ? STAGE : 1];
    __shared__ __attribute__((aligned(S > 3 ? 1024 : 2))) uint16_t lds3[S > 3 ? STAGE : 1];
    auto slot = [&](int i) -> uint16_t* { return i == 0 ? lds0 : i == 1 ? lds1 : i == 2 ? lds2 : lds3; };

    // split along K: workgroup z * ntiles + b computes tile b over K steps [z nk, (z+1) nk) into
    // the z-th M x ldc partial product
    const int z = blockIdx.x / ntiles;
    C += (long)z * M * ldc;
    const TileCoord tc = tile_of(blockIdx.x % ntiles, ntiles, tiles_m, 4, true);
    const int m0 = tc.tm * BM, n0 = tc.tn * BN;
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, g4 = lane >> 4;

    // DMA sources: instruction q of a stage fills 1 KB block q (A's blocks first); lane L writes
    // 16-byte slot L of it and fetches the chunk that belongs there.
    const uint16_t* src[PW];
    int dst[PW];
    long kstep[PW];
#pragma unroll
    for (int p = 0; p < PW; ++p) {
        const int q = min(wave * PW + p, NI - 1);  // past the last instruction, repeat it
        const bool is_a = q < NIA;
        const int qb = is_a ? q : q - NIA;
        const bool mm = is_a ? AMM : BMM;
        const int width = is_a ? BM : BN, base = is_a ? m0 : n0, lim = is_a ? a_lim : b_lim;
        const long ld = is_a ? lda : ldb;
        const uint16_t* X = is_a ? A : B;
        if (mm) {
            const int e = qb * 512 + 8 * lane, kr = e / width, sch = (e % width) / 8;
            const int sw = is_a ? (AMM ? mswz<BM>(kr) : 0) : (BMM ? mswz<BN>(kr) : 0);
            const int col = min(base + 8 * (sch ^ sw), lim - 8);  // columns past the operand: any finite data
            if (BKB && !is_a) {
                src[p] = X + ((long)(col >> 5) * ld + kr) * 32 + (col & 31);
                kstep[p] = TBK * 32;
            } else {
                src[p] = X + (long)kr * ld + col;
                kstep[p] = TBK * ld;
            }
        } else {
            const int row = qb * 8 + (lane >> 3), sch = lane & 7;
            const int g = min(base + row, lim - 1);
            src[p] = X + (long)g * ld + ((sch ^ (row & 7)) << 3);
            kstep[p] = TBK;
        }
        dst[p] = (is_a ? 0 : SA) + qb * 512;
        src[p] += (long)z * (K / TBK) * kstep[p];  // this split's first K step
    }
    auto issue = [&](int st, int kt) __attribute__((always_inline)) {
        uint16_t* b = slot(st);
#pragma unroll
        for (int p = 0; p < PW; ++p)
            __builtin_amdgcn_global_load_lds((const void*)(src[p] + (long)kt * kstep[p]),
                                             (__attribute__((address_space(3))) void*)(b + dst[p]), 16, 0, 0);
    };

    // per-lane fragment offsets (elements, within an operand's part of a stage)
    const int tr_r = r16 >> 2, tr_q = r16 & 3;
    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment of rows/columns c0 .. c0+15 of an operand part, k = kk*32 + 8*g4 .. +7
    auto frag = [&](const uint16_t* part, int c0, int kk, auto mm_c, auto width_c) __attribute__((always_inline)) {
        constexpr bool MM = decltype(mm_c)::value;
        constexpr int BX = decltype(width_c)::value;
        if constexpr (MM) {
            const int k1 = kk * 32 + 8 * g4 + tr_r, k2 = k1 + 4;
            const int ch = (c0 >> 3) + (tr_q >> 1);
            const u32x2_t lo = lds_tr16(part + k1 * BX + ((ch ^ mswz<BX>(k1)) << 3) + 4 * (tr_q & 1));
            const u32x2_t hi = lds_tr16(part + k2 * BX + ((ch ^ mswz<BX>(k2)) << 3) + 4 * (tr_q & 1));
            return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
        } else {
            const int row = c0 + r16;
            return *reinterpret_cast<const bf16x8_t*>(part + row * TBK + (((kk * 4 + g4) ^ (row & 7)) << 3));
        }
    };
    auto compute = [&](int st) __attribute__((always_inline)) {
        const uint16_t* sa = slot(st);
        const uint16_t* sb = sa + SA;
#pragma unroll
        for (int kk = 0; kk < TBK / 32; ++kk) {
            bf16x8_t af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = frag(sa, wm * WM + i * 16, kk, std::integral_constant<bool, AMM>{}, std::integral_constant<int, BM>{});
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = frag(sb, wn * WN + j * 16, kk, std::integral_constant<bool, BMM>{}, std::integral_constant<int, BN>{});
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

#define GPT2_TN_WAIT_BARRIER(after)                                \
    do {                                                           \
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((after) * PW, 0));  \
        __builtin_amdgcn_s_barrier();                              \
    } while (0)
    const int nk = K / TBK;
    if constexpr (NKT > 0) {
        static_for<0, S - 1>([&](auto st) {
            if constexpr (decltype(st)::value < NKT) issue(decltype(st)::value, decltype(st)::value);
        });
        static_for<0, NKT>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            constexpr int later = (k + S - 2 < NKT - 1 ? k + S - 2 : NKT - 1) - k;  // stages issued after k
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(later * PW, 0));
            __builtin_amdgcn_s_barrier();
            if constexpr (k + S - 1 < NKT) issue((k + S - 1) % S, k + S - 1);
            compute(k % S);
        });
    } else {
#pragma unroll
        for (int st = 0; st < S - 1; ++st)
            if (st < nk) issue(st, st);
        int kt = 0;
        for (; kt + 2 * S - 2 < nk; kt += S) {
#pragma unroll
            for (int u = 0; u < S; ++u) {
                GPT2_TN_WAIT_BARRIER(S - 2);
                issue((u + S - 1) % S, kt + u + S - 1);
                compute(u);
            }
        }
        for (; kt < nk; ++kt) {
            const int later = min(kt + S - 2, nk - 1) - kt;
            switch (later) {
                case 0: GPT2_TN_WAIT_BARRIER(0); break;
                case 1: GPT2_TN_WAIT_BARRIER(1); break;
                default: GPT2_TN_WAIT_BARRIER(2); break;
            }
            if (kt + S - 1 < nk) issue((kt + S - 1) % S, kt + S - 1);
            compute(kt % S);
        }
    }
#undef GPT2_TN_WAIT_BARRIER

    // C rows m0 + wm*WM + i*16 + 4*g4 + e, columns n0 + wn*WN + j*16 + r16
    if constexpr (GB) {
        // g = C * gelu'(u) in bf16 (0 on rows past M) and each column's sum of g over the tile's 64
        // rows. The tile goes through LDS ([64][BN + 4] fp32, rows 0-31 in ring slot 0, 32-63 in slot 1)
        // so that u is read and g written in whole 16- and 32-byte pieces per lane.
        static_assert(BM == 64 && BN == 128 && WGM * WGN == 4 && 32 * (BN + 4) * 4 <= STAGE * 2, "tile layout");
        constexpr int TS = BN + 4;
        auto trow = [&](int r) -> float* { return reinterpret_cast<float*>(r < 32 ? lds0 : lds1) + (r & 31) * TS; };
        __syncthreads();  // the ring is idle
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int j = 0; j < FN; ++j) trow(wm * WM + i * 16 + 4 * g4 + e)[wn * WN + j * 16 + r16] = acc[i][j][e];
        __syncthreads();
        const int t = threadIdx.x;
        for (int idx = t; idx < BM * (BN / 8); idx += 64 * WGM * WGN) {
            const int r = idx / (BN / 8), c8 = (idx % (BN / 8)) * 8, m = m0 + r, n = n0 + c8;
            float* tp = trow(r) + c8;
            float g[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) g[k] = 0.f;
            if (m < M) {
                const float* up = gb.u + (long)m * gb.ldu + n;
                if (n + 8 <= N) {
                    const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(up);
                    const f32x4_t u1 = *reinterpret_cast<const f32x4_t*>(up + 4);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        g[k] = tp[k] * (gb.erf ? gelu_erf_grad(u0[k]) : gelu_tanh_grad(u0[k]));
                        g[k + 4] = tp[k + 4] * (gb.erf ? gelu_erf_grad(u1[k]) : gelu_tanh_grad(u1[k]));
                    }
                } else {
                    for (int k = 0; k < 8 && n + k < N; ++k)
                        g[k] = tp[k] * (gb.erf ? gelu_erf_grad(up[k]) : gelu_tanh_grad(up[k]));
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) tp[k] = g[k];
            uint16_t* yp = gb.y + (long)m * gb.ldy + n;
            if (n + 8 <= N) {
                u32x4_t pk;
                pk[0] = pack_bf16x2(g[0], g[1]);
                pk[1] = pack_bf16x2(g[2], g[3]);
                pk[2] = pack_bf16x2(g[4], g[5]);
                pk[3] = pack_bf16x2(g[6], g[7]);
                *reinterpret_cast<u32x4_t*>(yp) = pk;
            } else {
                for (int k = 0; k < 8 && n + k < N; ++k) yp[k] = f32_to_bf16_bits(g[k]);
            }
        }
        __syncthreads();
        if (t < BN && n0 + t < N) {
            float cs = 0.f;
            for (int r = 0; r < BM; ++r) cs += trow(r)[t];
            gb.part[(long)tc.tm * N + n0 + t] = cs;
        }
    } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + wm * WM + i * 16 + 4 * g4 + e;
            if (m >= M) continue;
            float* crow = C + (long)m * ldc;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WN + j * 16 + r16;
                if (n < N) crow[n] = acc[i][j][e];
            }
        }
    }
}

// C[m][n] = sum over z < nsplit of P[z][m][n] (P: nsplit partial products of M x N, row stride N),
// added in increasing z, so the result does not depend on scheduling. Four columns per thread.
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float4* __restrict__ P, int nsplit, int M, int N4,
                                                         float* __restrict__ C, long ldc) {
    const long n = (long)M * N4;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        float4 a = P[i];
        for (int z = 1; z < nsplit; ++z) {
            const float4 b = P[(long)z * n + i];
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        const long m = i / N4;
        *reinterpret_cast<float4*>(C + m * ldc + 4 * (i % N4)) = a;
    }
}

// nsplit > 1: the K range is split into nsplit parts of K / nsplit (a multiple of TBK); their
// partial products go to part (nsplit x M x N floats) and are then summed into C.
template <int BM, int BN, int S, int WGM, int WGN, bool AMM, bool BMM, int NKT, bool GB = false, bool BKB = false>
hipError_t launch_tn(const uint16_t* A, long lda, int a_lim, const uint16_t* B, long ldb, int b_lim, float* C, long ldc,
                     int M, int N, int K, hipStream_t s, int nsplit = 1, float* part = nullptr,
                     const TnGeluBack& gb = TnGeluBack()) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN, ntiles = tiles_m * tiles_n;
    if (nsplit > 1) {
        gemm_tn_kernel<BM, BN, S, WGM, WGN, AMM, BMM, NKT, GB, BKB><<<dim3(ntiles * nsplit), dim3(64 * WGM * WGN), 0, s>>>(
            A, lda, a_lim, B, ldb, b_lim, part, N, M, N, K / nsplit, tiles_m, ntiles, gb);
        const long n4 = (long)M * (N / 4);
        splitk_sum_kernel<<<dim3((unsigned)std::min<long>((n4 + 255) / 256, 4096)), dim3(256), 0, s>>>(
            reinterpret_cast<const float4*>(part), nsplit, M, N / 4, C, ldc);
        return hipGetLastError();
    }
    gemm_tn_kernel<BM, BN, S, WGM, WGN, AMM, BMM, NKT, GB, BKB><<<dim3(ntiles), dim3(64 * WGM * WGN), 0, s>>>(
        A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, tiles_m, ntiles, gb);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16_tn(const uint16_t* A, bool a_mmajor, long lda, int a_lim, const uint16_t* B, bool b_mmajor,
                        long ldb, int b_lim, float* C, long ldc, int M, int N, int K, hipStream_t s, float* part,
                        size_t part_elems, const TnGeluBack* gb, bool b_kb) {
    if (M < 1 || N < 1 || K < TBK || K % TBK || !b_mmajor) return hipErrorInvalidValue;
    const int nk = K / TBK;
    if (b_kb) {
        // weight gradients on a k-blocked activation (ldb = its rows per block, >= K; b_lim a
        // multiple of 32): 64 x 128 tiles, the narrow ones split along K as below
        if (!a_mmajor || gb || ldb < K || b_lim % 32 || M >= 16384) return hipErrorInvalidValue;
        auto fits4 = [&]() {
            return part && N % 4 == 0 && ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
                   (size_t)4 * M * N <= part_elems;
        };
        const long t64 = (long)((M + 63) / 64) * ((N + 127) / 128);
        if (t64 < 128 && nk % 4 == 0 && nk >= 16 && fits4()) {
            if (nk == 64)
                return launch_tn<64, 128, 3, 2, 2, true, true, 16, false, true>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M,
                                                                                N, K, s, 4, part);
            return launch_tn<64, 128, 3, 2, 2, true, true, 0, false, true>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N,
                                                                           K, s, 4, part);
        }
        if (nk == 64)
            return launch_tn<64, 128, 3, 2, 2, true, true, 64, false, true>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N,
                                                                            K, s);
        return launch_tn<64, 128, 3, 2, 2, true, true, 0, false, true>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K,
                                                                       s);
    }
    // input gradient of c_fc's output through the GELU: 64 x 128 tiles, no split, on a two-stage ring
    // (49 KB of LDS: three workgroups per CU, so that two overlap the third's epilogue, which reads
    // the fp32 GELU input; GPT-2 small B=4 T=1024 training step 7.72 -> 7.65 ms, while the plain
    // input gradients measured slower on two stages)
    if (gb) {
        if (a_mmajor || !gb->u || !gb->y || !gb->part || gb->ldu < N || gb->ldy < N || gb->ldu % 4 || gb->ldy % 8 ||
            reinterpret_cast<uintptr_t>(gb->u) % 16 || reinterpret_cast<uintptr_t>(gb->y) % 16)
            return hipErrorInvalidValue;
        if (nk == 12)
            return launch_tn<64, 128, 2, 2, 2, false, true, 12, true>(A, lda, a_lim, B, ldb, b_lim, nullptr, 0, M, N, K,
                                                                      s, 1, nullptr, *gb);
        return launch_tn<64, 128, 2, 2, 2, false, true, 0, true>(A, lda, a_lim, B, ldb, b_lim, nullptr, 0, M, N, K, s,
                                                                 1, nullptr, *gb);
    }
    // Split along K where one pass would leave most CUs idle or run very long chains: a weight
    // gradient with fewer than 128 tiles of 64 x 128 (attn.c_proj of GPT-2 small: 72) in four
    // parts; a reduction over the vocabulary (nk in the hundreds) in six, three or two parts (six for
    // GPT-2's 786 steps: 2304 workgroups fill the 512 slots of two per CU 4.5 times, where three parts
    // filled them 2.25 times with twice the steps each; training step 7.75 -> 7.70 ms).
    auto fits = [&](int ns) {
        return part && N % 4 == 0 && ldc % 4 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
               (size_t)ns * M * N <= part_elems;
    };
    const long tiles64 = (long)((M + 63) / 64) * ((N + 127) / 128);
    if (a_mmajor && M < 16384 && tiles64 < 128 && nk % 4 == 0 && nk >= 16 && fits(4)) {
        if (nk == 64)
            return launch_tn<64, 128, 3, 2, 2, true, true, 16>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s, 4, part);
        return launch_tn<64, 128, 3, 2, 2, true, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s, 4, part);
    }
    if (!a_mmajor && nk >= 256) {
        if (nk % 6 == 0 && fits(6))
            return launch_tn<64, 128, 3, 2, 2, false, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s, 6, part);
        if (nk % 3 == 0 && fits(3))
            return launch_tn<64, 128, 3, 2, 2, false, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s, 3, part);
        if (nk % 2 == 0 && fits(2))
            return launch_tn<64, 128, 3, 2, 2, false, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s, 2, part);
    }
    if (a_mmajor) {
        // weight gradients: 64 x 128 tiles of four wavefronts (32 x 64 each), two workgroups per
        // CU; for very many rows (the tied wte gradient, M = n_vocab) 128 x 128 tiles
        if (M >= 16384) {
            if (nk == 64) return launch_tn<128, 128, 3, 2, 2, true, true, 64>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
            return launch_tn<128, 128, 3, 2, 2, true, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
        }
        if (nk == 64) return launch_tn<64, 128, 3, 2, 2, true, true, 64>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
        return launch_tn<64, 128, 3, 2, 2, true, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
    }
    // input gradients dX = dY W (A K-major, B = W [out][in] M-major)
    switch (nk) {
        case 12: return launch_tn<64, 128, 3, 2, 2, false, true, 12>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
        case 36: return launch_tn<64, 128, 3, 2, 2, false, true, 36>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
        case 48: return launch_tn<64, 128, 3, 2, 2, false, true, 48>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
        default: return launch_tn<64, 128, 3, 2, 2, false, true, 0>(A, lda, a_lim, B, ldb, b_lim, C, ldc, M, N, K, s);
    }
}

}  // namespace gpt2k
