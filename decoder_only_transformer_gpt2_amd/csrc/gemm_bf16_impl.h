#pragma once
// bf16 GEMM on the gfx950 matrix cores with fused epilogues:
//   C[M, N] = epi(A[M, K] . W[N, K]^T + bias[N])
// A (activations) and W (nn.Linear weights, [out, in]) are both K-contiguous. Used for c_attn,
// attn.c_proj, mlp.c_fc, mlp.c_proj and the tied lm_head ("复现GPT-2 124M" §2.1 and §2.4,
// "从零手写GPT-2" §4.1).
//
// Tiling: a workgroup of WGM x WGN wavefronts owns a BM x BN tile of C and walks K in steps of
// BK. The A and W slabs of each step go straight from global memory into a ring of S LDS stages
// (global_load_lds_dwordx4, no staging registers), issued S-1 steps ahead, so up to S-1 stages
// are in flight while one is consumed: the loop is bound by how many bytes are in flight per CU,
// and the DMA ring holds far more than register staging could. Each step waits for its own stage
// with an explicit vmcnt, meets the other wavefronts at a barrier, refills the stage it freed and
// runs its MFMAs (v_mfma_f32_16x16x32_bf16, fp32 accumulators kept in registers until the
// epilogue). 16-byte chunks are XOR-swizzled by row in LDS (the permutation is applied on the
// global side, since a DMA writes 64 consecutive 16-byte lane slots) so that the 16-byte
// fragment reads of a wavefront spread over all banks.
//
// Tile shapes come from a per-shape table chosen so that the grid fills the 256 compute units
// (8 XCDs x 32). The block projections remap workgroup ids so that each XCD (which receives every
// 8th id) works on one contiguous range of tiles, rasterised in groups of row-tiles, so the A rows
// and W rows a group shares stay in that XCD's L2; the vocabulary projection interleaves the XCDs
// instead (see tile_of).
//
// Operands are row-major ([rows][K]) or k-blocked ([K/32][rows][32]); with the k-blocked layout the
// slab of a 32-wide K step is one contiguous run per operand, so each DMA instruction reads whole
// 128-byte lines (row-major slabs are 64-byte pieces of lines, and the DMA rate follows the number
// of lines an instruction touches: measured ~59 against ~115 GB/s per CU).
#include <cstdio>
#include <cstdlib>

#include "common.h"

#include <type_traits>

namespace gpt2k {
namespace {

constexpr int kXcds = 8;

struct TileCoord {
    int tm, tn;
};

// Workgroup id -> (row-tile, column-tile). group_m >= 1000: XCD-interleaved groups (below);
// otherwise optionally remapped so that each XCD (which receives every 8th id) works on one
// contiguous range of tiles, then rasterised in groups of group_m row-tiles (column-major inside a
// group), so neighbouring ids share W rows.
__device__ __forceinline__ TileCoord tile_of(int b, int nblk, int tiles_m, int group_m, bool xcd_remap) {
    if (group_m >= 1000) {
        // XCD-interleaved groups of g row-tiles: inside a group, column tiles go by octets and ids
        // b, b+8, b+16, ... (one XCD, one L2) take the same column tile in consecutive row-tiles,
        // while the eight XCDs work on eight neighbouring column tiles
        const int g = group_m - 1000;
        const int tiles_n = nblk / tiles_m;
        const int per_group = g * tiles_n;
        const int grp = b / per_group, lb = b % per_group;
        const int first_m = grp * g;
        const int gm = min(tiles_m - first_m, g);
        const int full = tiles_n / 8;
        if (lb < full * 8 * gm) {
            const int oct = lb / (8 * gm), w = lb % (8 * gm);
            return {first_m + w / 8, oct * 8 + w % 8};
        }
        const int rem = tiles_n - full * 8, w = lb - full * 8 * gm;
        return {first_m + w / rem, full * 8 + w % rem};
    }
    int logical = b;
    if (xcd_remap) {
        const int xcd = b % kXcds, idx = b / kXcds, q = nblk / kXcds, r = nblk % kXcds;
        logical = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
    }
    const int tiles_n = nblk / tiles_m;
    const int per_group = group_m * tiles_n;
    const int grp = logical / per_group, in = logical % per_group;
    const int first_m = grp * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    return {first_m + in % gm, in / gm};
}

// Waitcnt immediate (gfx9 encoding): wait until at most vm vector-memory and lgkm LDS/scalar
// operations of this wavefront are outstanding (expcnt not waited on).
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

template <int BM, int BN, int BK, int S, int WGM, int WGN, int EPI, bool KB, int NKT>
// NKT > 0: the K loop has exactly NKT steps and is unrolled completely (straight-line code with
// compile-time ring slots and waits): at a loop header the compiler drains every outstanding DMA
// before the first LDS read of the iteration (vmcnt(0) once per ring turn), since it cannot tell
// across the back edge which stage that read depends on.
// Two workgroups per CU (256 registers per lane) wherever the ring fits twice in LDS and the
// wave tile is at most 128 x 64.
__global__ __launch_bounds__(64 * WGM * WGN,
                             (BM / WGM) * (BN / WGN) <= 128 * 64 && S * (BM + BN) * BK * 2 <= 80 * 1024 ? 2 : 1)
void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, const float* __restrict__ bias,
    void* __restrict__ Cv, int M, int N, int K, int ldc, int a_rows, int w_rows, int tiles_m,
    int group_m, int c_kb, HeadOut ho) {
    constexpr int NT = 64 * WGM * WGN, NW = WGM * WGN;
    constexpr bool HEAD = EPI == EPI_LOGITS || EPI == EPI_LSE;  // vocabulary projection: no bias
    constexpr bool GU = EPI == EPI_BIAS_GELU_U || EPI == EPI_BIAS_GELU_U_ERF;  // u in fp32 and gelu(u) in bf16
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
    constexpr int CPR = BK / 8;                  // 16-byte chunks per slab row
    constexpr int RPI = 64 / CPR;                // slab rows one 64-lane DMA instruction fills
    constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage (A slab, then W slab)
    constexpr int NI = (BM + BN) / RPI;          // DMA instructions per stage
    constexpr int PW = (NI + NW - 1) / NW;       // per wavefront (the last ones may repeat a load)
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BM % RPI == 0 && BN % RPI == 0, "a DMA instruction fills rows of one operand");
    static_assert(S >= 2 && S <= 6 && (S - 1) * PW < 64, "ring depth");
    static_assert(S * STAGE * 2 <= 160 * 1024, "LDS");
    // One LDS object per stage: lets the compiler see which outstanding DMA an LDS read depends on.
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[STAGE];
    // (stages past S get a 2-byte placeholder so that they take no LDS)
    __shared__ __attribute__((aligned(S > 2 ? 1024 : 2))) uint16_t lds2[S > 2 ? STAGE : 1];
    __shared__ __attribute__((aligned(S > 3 ? 1024 : 2))) uint16_t lds3[S > 3 ? STAGE : 1];
    __shared__ __attribute__((aligned(S > 4 ? 1024 : 2))) uint16_t lds4[S > 4 ? STAGE : 1];
    __shared__ __attribute__((aligned(S > 5 ? 1024 : 2))) uint16_t lds5[S > 5 ? STAGE : 1];
    auto slot = [&](int i) -> uint16_t* {
        return i == 0 ? lds0 : i == 1 ? lds1 : i == 2 ? lds2 : i == 3 ? lds3 : i == 4 ? lds4 : lds5;
    };

    const TileCoord tc = tile_of(blockIdx.x, gridDim.x, tiles_m, group_m < 0 ? -group_m : group_m, group_m > 0);
    const int m0 = tc.tm * BM, n0 = tc.tn * BN;
    const int wave = threadIdx.x / GPT2_WAVE, lane = threadIdx.x % GPT2_WAVE;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r16 = lane & 15, g4 = lane >> 4;

    // Swizzled chunk position of (row, chunk) within a slab row.
    auto swz_chunk = [](int row, int chunk) { return CPR == 8 ? (chunk ^ (row & 7)) : (chunk ^ ((row >> 1) & 3)); };

    // DMA sources: instruction p of this wavefront fills slab rows [q*RPI, q*RPI+RPI) of the stage
    // (q = wave*PW + p; A rows first, then W rows); lane L writes LDS slot L of that 1 KB block,
    // i.e. row q*RPI + L/CPR, swizzled chunk L%CPR, so it fetches the chunk that belongs there.
    const uint16_t* src[PW];
    int lds_off[PW];
    [[maybe_unused]] int kstep[PW];
#pragma unroll
    for (int p = 0; p < PW; ++p) {
        // past the stage's last instruction, repeat it: the same bytes to the same LDS block, so
        // every wavefront issues PW loads per stage and the waits below stay exact
        const int q = min(wave * PW + p, NI - 1);
        const int srow = q * RPI + lane / CPR;  // row within the stage (A rows, then W rows)
        const int sch = lane % CPR;
        const bool is_a = srow < BM;
        const int row = is_a ? srow : srow - BM;
        const int chunk = swz_chunk(row, sch);
        const int g = is_a ? min(m0 + row, a_rows - 1) : min(n0 + row, w_rows - 1);
        if (KB) {
            // k-blocked operands ([K/32][rows][32]): chunk c of row g at k0 = 0 sits in block c/4
            const int rows = is_a ? a_rows : w_rows;
            src[p] = (is_a ? A : W) + ((size_t)(chunk >> 2) * rows + g) * 32 + (chunk & 3) * 8;
            kstep[p] = rows;
        } else {
            src[p] = (is_a ? A : W) + (size_t)g * K + chunk * 8;
        }
        lds_off[p] = q * RPI * BK;  // element offset of the instruction's 1 KB block
    }
    auto issue = [&](int st, int k0) {
        uint16_t* base = slot(st);
#pragma unroll
        for (int p = 0; p < PW; ++p)
            // k-blocked: block k0/32 starts k0/32 * rows * 32 = k0 * rows elements further on
            __builtin_amdgcn_global_load_lds((const void*)(src[p] + (KB ? (size_t)k0 * kstep[p] : (size_t)k0)),
                                             (__attribute__((address_space(3))) void*)(base + lds_off[p]), 16, 0, 0);
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Epilogue operands are loaded before the K loop, so their memory latency hides behind it: the
    // bias of this lane's column in each 16-column block (0 past N) and, for the residual epilogue
    // with narrow wave tiles, the residual values this lane adds to in the store loop below (four
    // floats per lane and 16-row strip pass, the same order).
    const int row0 = m0 + wm * WM, col0 = n0 + wn * WN;
    // Interior tiles (the common case) take the store and argmax paths without bounds checks.
    const bool interior = m0 + BM <= M && n0 + BN <= N;
    float bcol[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int n = col0 + j * 16 + r16;
        bcol[j] = (!HEAD && n < N) ? bias[n] : 0.f;
    }
    constexpr int RIT = 16 * (WN / 4) / GPT2_WAVE;  // residual store passes per strip
    constexpr bool RPRE = EPI == EPI_BIAS_RESIDUAL && (16 * (WN / 4)) % GPT2_WAVE == 0 && FM * RIT * 4 <= 32;
    const bool rpre = RPRE && interior && (ldc & 3) == 0;
    f32x4_t xres[RPRE ? FM : 1][RPRE ? RIT : 1];
    if constexpr (RPRE) {
        if (rpre) {
            const float* Rb = (ho.res ? ho.res : static_cast<const float*>(Cv)) + (size_t)row0 * ldc + col0;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int it = 0; it < RIT; ++it) {
                    const int idx = it * GPT2_WAVE + lane, r = idx / (WN / 4), c = (idx % (WN / 4)) * 4;
                    xres[i][it] = *reinterpret_cast<const f32x4_t*>(Rb + (size_t)(i * 16 + r) * ldc + c);
                }
        }
    }

    auto compute = [&](int st) {
        const uint16_t* sa = slot(st);
        const uint16_t* sw = sa + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            bf16x8_t af[FM], wf[FN];
            const int chunk = kk * 4 + g4;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WM + i * 16 + r16;
                af[i] = *reinterpret_cast<const bf16x8_t*>(&sa[row * BK + swz_chunk(row, chunk) * 8]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WN + j * 16 + r16;
                wf[j] = *reinterpret_cast<const bf16x8_t*>(&sw[row * BK + swz_chunk(row, chunk) * 8]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
        }
    };

    // Step kt: wait until this wavefront's DMAs of stage kt have landed (at most `after` stages
    // issued later may still be in flight) and its LDS reads of the previous step are done, meet
    // the other wavefronts (their stage kt has landed too, and nobody still reads the slot of step
    // kt-1), refill that slot with stage kt+S-1, then run stage kt.
#define GPT2_WAIT_BARRIER(after)                                              \
    do {                                                                      \
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((after) * PW, 0));             \
        __builtin_amdgcn_s_barrier();                                         \
    } while (0)

    const int nk = K / BK;
    if constexpr (NKT > 0) {
        static_for<0, S - 1>([&](auto st) {
            if constexpr (decltype(st)::value < NKT) issue(decltype(st)::value, decltype(st)::value * BK);
        });
        static_for<0, NKT>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            constexpr int later = (k + S - 2 < NKT - 1 ? k + S - 2 : NKT - 1) - k;  // stages issued after k
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(later * PW, 0));
            __builtin_amdgcn_s_barrier();
            if constexpr (k + S - 1 < NKT) issue((k + S - 1) % S, (k + S - 1) * BK);
            compute(k % S);
        });
    } else {
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < nk) issue(st, st * BK);

    int kt = 0;
    // steady state: every step issues a new stage, so S-2 later stages are always in flight
    for (; kt + 2 * S - 2 < nk; kt += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            GPT2_WAIT_BARRIER(S - 2);
            issue((u + S - 1) % S, (kt + u + S - 1) * BK);
            compute(u);
        }
    }
    // tail: fewer stages left to issue; wait exactly for this step's stage
    for (; kt < nk; ++kt) {
        const int later = min(kt + S - 2, nk - 1) - kt;  // stages issued after kt
        switch (later) {
            case 0: GPT2_WAIT_BARRIER(0); break;
            case 1: GPT2_WAIT_BARRIER(1); break;
            case 2: GPT2_WAIT_BARRIER(2); break;
            case 3: GPT2_WAIT_BARRIER(3); break;
            default: GPT2_WAIT_BARRIER(4); break;
        }
        if (kt + S - 1 < nk) issue((kt + S - 1) % S, (kt + S - 1) * BK);
        compute(kt % S);
    }
    }
#undef GPT2_WAIT_BARRIER
    __syncthreads();  // the ring is idle from here: the epilogue reuses it

    // Epilogue. acc[i][j][e] holds C[row, col] with row = wm*WM + i*16 + 4*g4 + e and
    // col = wn*WN + j*16 + r16 (the 16x16 MFMA accumulator layout: each lane holds four rows of
    // one column). Stores straight from that layout would scatter 2- or 4-byte writes over four
    // rows per instruction, so each wavefront stages one 16-row strip at a time in its own LDS
    // scratch ([16][WN+4] fp32, padded against bank conflicts) and then writes whole row segments
    // with consecutive lanes on consecutive columns.
    constexpr int SP = WN + 4;
    constexpr int SCR_BYTES = 16 * SP * 4;
    constexpr int WAVES_PER_SLOT = (STAGE * 2) / SCR_BYTES;
    static_assert(WAVES_PER_SLOT >= 1 && (NW + WAVES_PER_SLOT - 1) / WAVES_PER_SLOT <= S - 1,
                  "epilogue scratch fits the ring, leaving the last stage for the argmax partials");
    static_assert(WGN * BM * 8 <= STAGE * 2, "argmax partials fit one stage");
    float* scr = reinterpret_cast<float*>(slot(wave / WAVES_PER_SLOT)) + (wave % WAVES_PER_SLOT) * (16 * SP);
    uint32_t* red_v = reinterpret_cast<uint32_t*>(slot(S - 1));  // [WGN][BM] row maximum (order key)
    uint32_t* red_i = red_v + WGN * BM;                            // [WGN][BM] its first column
    float* red_m = reinterpret_cast<float*>(red_v);                // (EPI_LSE) [WGN][BM] base-2 maximum
    float* red_s = reinterpret_cast<float*>(red_i);                // (EPI_LSE) [WGN][BM] sum below it


    // One strip: 16 rows x WN columns staged in scr, then written out (a wavefront's LDS
    // operations complete in order, so its own staged values are visible to its later reads).
    auto strip_out = [&](int i, auto checked) {
        constexpr bool CHK = decltype(checked)::value;
        const int rs = row0 + i * 16;  // first row of the strip (wave-uniform)
        const int rows = M - rs, cols = N - col0;
        if (EPI == EPI_LSE) {
            // Per row over the staged strip, four lanes per row, lane q taking columns 4c + q (so
            // that the 64 lanes' reads fall on distinct banks: SP is 4 more than a multiple of 16):
            // the maximum of y = logit * log2(e) and the sum of 2^(y - max), then both combined over
            // the four lanes. Columns past N are left out. The lane whose columns hold the row's
            // target keeps that logit. Nothing is stored to the logits.
            constexpr int CQ = WN / 4;
            constexpr float LOG2E = 1.4426950408889634f;
            const int ar = lane >> 2, aq = lane & 3;
            const float* sp = scr + ar * SP + aq;
            const int lim = CHK ? cols - aq : WN;  // column 4c + aq is valid when 4c < lim
            float y[CQ];
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < CQ; ++c) {
                y[c] = sp[4 * c] * LOG2E;
                if (CHK) y[c] = 4 * c < lim ? y[c] : -INFINITY;
                mx = fmaxf(mx, y[c]);
            }
            const float ms = mx == -INFINITY ? 0.f : mx;
            float sum = 0.f;
#pragma unroll
            for (int c = 0; c < CQ; ++c) sum += __builtin_amdgcn_exp2f(y[c] - ms);
            lse_quad_merge(mx, sum);
            const int row = rs + ar;
            if (!CHK || row < M) {
                const int tc = ho.tgt[row], rel = tc - col0;
                if (rel >= 0 && rel < WN && (rel & 3) == aq && tc < N) ho.tgt_logit[row] = sp[rel - aq];
            }
            if (aq == 0) {
                const int rl = wn * BM + wm * WM + i * 16 + ar;
                red_m[rl] = mx;
                red_s[rl] = sum;
            }
        } else if (EPI == EPI_LOGITS) {
            if (ho.pv) {
                // Row argmax over the staged strip: four lanes per row, lane q scanning columns
                // 4c + q in increasing order (a strict > keeps the first of equal values; the
                // interleave keeps the 64 lanes' reads on distinct banks), then the row maximum (as
                // an order key) and the smallest column holding it over the four lanes. Columns
                // past N count as -inf; a lane with no column offers none (its -inf seed and its
                // key never beat a real column, whatever the sign of the row's logits: the zero
                // padding rows of wte give exactly 0 past N).
                constexpr int CQ = WN / 4;
                const int ar = lane >> 2, aq = lane & 3;
                const float* sp = scr + ar * SP + aq;
                const int lim = CHK ? cols - aq : WN;  // column 4c + aq is valid when 4c < lim
                const bool has_col = !CHK || lim > 0;
                float bv = has_col ? sp[0] : -INFINITY;
                int bc = 0;
#pragma unroll
                for (int c = 1; c < CQ; ++c) {
                    float x = sp[4 * c];
                    if (CHK) x = 4 * c < lim ? x : -INFINITY;
                    const bool take = x > bv;
                    bv = take ? x : bv;
                    bc = take ? c : bc;
                }
                const uint32_t key = has_col ? f32_order_key(bv) : 0u;
                const uint32_t kmax = quad_max_u32(key);
                const uint32_t col = (key == kmax && has_col) ? (uint32_t)(col0 + 4 * bc + aq) : 0xffffffffu;
                const uint32_t cmin = quad_min_u32(col);
                if (aq == 0) {
                    const int rl = wn * BM + wm * WM + i * 16 + ar;
                    red_v[rl] = kmax;
                    red_i[rl] = cmin;
                }
            }
            // fp32 rows of odd stride: one float per lane, consecutive lanes on consecutive
            // columns, from the strip's origin plus a 32-bit in-strip offset. Streaming stores:
            // the logits are written once and not read back by this pass, so they should not
            // evict the weights and activations from the caches.
            float* Cs = static_cast<float*>(Cv) + (size_t)rs * ldc + col0;
            if (Cv)  // no logits buffer: argmax partials only
#pragma unroll
            for (int it = 0; it < (16 * WN + GPT2_WAVE - 1) / GPT2_WAVE; ++it) {
                const int idx = it * GPT2_WAVE + lane;
                if (16 * WN % GPT2_WAVE != 0 && idx >= 16 * WN) break;
                const int r = idx / WN, c = idx % WN;
                if (!CHK || (r < rows && c < cols)) __builtin_nontemporal_store(scr[r * SP + c], Cs + r * ldc + c);
            }
        } else if (EPI == EPI_BIAS_RESIDUAL) {
            // C += staged (or C = res + staged), four floats per lane
            float* Cs = static_cast<float*>(Cv) + (size_t)rs * ldc + col0;
            const float* Rs = ho.res ? ho.res + (size_t)rs * ldc + col0 : Cs;
            const bool vec = (ldc & 3) == 0;
#pragma unroll
            for (int it = 0; it < (16 * (WN / 4) + GPT2_WAVE - 1) / GPT2_WAVE; ++it) {
                const int idx = it * GPT2_WAVE + lane;
                if (16 * (WN / 4) % GPT2_WAVE != 0 && idx >= 16 * (WN / 4)) break;
                const int r = idx / (WN / 4), c = (idx % (WN / 4)) * 4;
                if (CHK && r >= rows) continue;
                const float* sv = &scr[r * SP + c];
                float* cp = Cs + r * ldc + c;
                const float* rp = Rs + r * ldc + c;
                if ((!CHK || c + 4 <= cols) && vec) {
                    f32x4_t cv;
                    if constexpr (RPRE && !CHK)
                        cv = rpre ? xres[i][it] : *reinterpret_cast<const f32x4_t*>(rp);
                    else
                        cv = *reinterpret_cast<const f32x4_t*>(rp);
                    cv[0] += sv[0]; cv[1] += sv[1]; cv[2] += sv[2]; cv[3] += sv[3];
                    *reinterpret_cast<f32x4_t*>(cp) = cv;
                } else {
                    for (int t = 0; t < 4 && c + t < cols; ++t) cp[t] = rp[t] + sv[t];
                }
            }
        } else {
            // bf16 rows: eight values (16 bytes) per lane (eight columns never straddle a 32-column
            // block of the k-blocked layout)
            uint16_t* Cs = static_cast<uint16_t*>(Cv) + (size_t)rs * ldc + col0;
            const bool vec = c_kb || (ldc & 7) == 0;
#pragma unroll
            for (int it = 0; it < (16 * (WN / 8) + GPT2_WAVE - 1) / GPT2_WAVE; ++it) {
                const int idx = it * GPT2_WAVE + lane;
                if (16 * (WN / 8) % GPT2_WAVE != 0 && idx >= 16 * (WN / 8)) break;
                const int r = idx / (WN / 8), c = (idx % (WN / 8)) * 8;
                if (CHK && r >= rows) continue;
                const float* sv = &scr[r * SP + c];
                uint16_t* cp = Cs + r * ldc + c;
                if (c_kb) {
                    const int col = col0 + c;
                    cp = static_cast<uint16_t*>(Cv) + ((size_t)(col >> 5) * c_kb + rs + r) * 32 + (col & 31);
                }
                // GU: sv holds u; u is stored as is and gelu(u) rounded to bf16
                auto act = [](float v) {
                    return EPI == EPI_BIAS_GELU_U ? gelu_tanh_fast(v) : EPI == EPI_BIAS_GELU_U_ERF ? gelu_erf_f32(v) : v;
                };
                float* up = GU ? ho.u + (size_t)(rs + r) * ldc + col0 + c : nullptr;
                if ((!CHK || c + 8 <= cols) && vec) {
                    u32x4_t pk;
                    pk[0] = pack_bf16x2(act(sv[0]), act(sv[1]));
                    pk[1] = pack_bf16x2(act(sv[2]), act(sv[3]));
                    pk[2] = pack_bf16x2(act(sv[4]), act(sv[5]));
                    pk[3] = pack_bf16x2(act(sv[6]), act(sv[7]));
                    *reinterpret_cast<u32x4_t*>(cp) = pk;
                    if (GU) {
                        *reinterpret_cast<f32x4_t*>(up) = f32x4_t{sv[0], sv[1], sv[2], sv[3]};
                        *reinterpret_cast<f32x4_t*>(up + 4) = f32x4_t{sv[4], sv[5], sv[6], sv[7]};
                    }
                } else {
                    for (int t = 0; t < 8 && c + t < cols; ++t) {
                        cp[t] = f32_to_bf16_bits(act(sv[t]));
                        if (GU) up[t] = sv[t];
                    }
                }
            }
        }
    };

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        // stage the strip (bias and GELU applied; the residual add happens at the store)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = acc[i][j][e];
                if (!HEAD) v += bcol[j];
                if (EPI == EPI_BIAS_GELU) v = gelu_tanh_fast(v);
                if (EPI == EPI_BIAS_GELU_ERF) v = gelu_erf_f32(v);
                scr[(4 * g4 + e) * SP + j * 16 + r16] = v;
            }
        if (interior)
            strip_out(i, std::integral_constant<bool, false>{});
        else
            strip_out(i, std::integral_constant<bool, true>{});
    }

    if (EPI == EPI_LSE) {
        __syncthreads();
        const int tiles_n = (N + BN - 1) / BN;
        for (int rl = threadIdx.x; rl < BM; rl += NT) {
            const int m = m0 + rl;
            if (m < M) {
                float mx = red_m[rl], sum = red_s[rl];
#pragma unroll
                for (int w = 1; w < WGN; ++w) lse_merge(mx, sum, red_m[w * BM + rl], red_s[w * BM + rl]);
                ho.pv[(size_t)m * tiles_n + tc.tn] = mx;
                ho.ps[(size_t)m * tiles_n + tc.tn] = sum;
            }
        }
    }
    if (EPI == EPI_LOGITS && ho.pv) {
        __syncthreads();
        const int tiles_n = (N + BN - 1) / BN;
        for (int rl = threadIdx.x; rl < BM; rl += NT) {
            const int m = m0 + rl;
            if (m < M) {
                uint32_t kv = red_v[rl], ki = red_i[rl];
#pragma unroll
                for (int w = 1; w < WGN; ++w) {
                    const uint32_t v2 = red_v[w * BM + rl], i2 = red_i[w * BM + rl];
                    const bool take = (v2 > kv) | ((v2 == kv) & (i2 < ki));
                    kv = take ? v2 : kv;
                    ki = take ? i2 : ki;
                }
                ho.pv[(size_t)m * tiles_n + tc.tn] = f32_from_order_key(kv);
                ho.pi[(size_t)m * tiles_n + tc.tn] = (int32_t)ki;
            }
        }
    }
}

// ------------------------------------------------------------------------------ tile table
struct TileCfg {
    int bm, bn, bk, stages, wgm, wgn;
};

// Instantiated tile shapes (the ones the dispatcher in gemm_bf16.hip chooses).
constexpr TileCfg kCfgs[] = {
    {64, 96, 64, 4, 2, 2},    // 0: 4 waves (32 x 48 each), 2 workgroups per CU: narrow row-major products
    {256, 192, 64, 2, 2, 4},  // 1: 8 waves (128 x 48): narrow outputs of very many rows (wte gradient)
    {128, 256, 32, 3, 2, 2},  // 2: 4 waves (64 x 128), 72 KB ring, 2 per CU: vocabulary projection
    {192, 256, 32, 5, 2, 4},  // 3: 8 waves (96 x 64), 140 KB ring: N = 2304 (c_attn)
    {256, 192, 32, 5, 2, 4},  // 4: 8 waves (128 x 48), 140 KB ring: N = 3072 on k-blocked operands (c_fc)
    {128, 96, 64, 4, 4, 2},   // 5: 8 waves (4 x 2, 32 x 48 each), 112 KB ring: narrow k-blocked (c_proj)
};

// One epilogue's launch, with the K loop fully unrolled for the step counts that occur: the
// forward's k-blocked projections (K = 768 and 3072; for GPT-2 medium and XL the vocabulary
// projection, c_attn and c_fc, K = d, and the residual projections, K = d and 4d, for d = 1024 and
// 1600) and the plain fp32 products of the backward (K = 768, 2304, 3072 and B*T = 4096 at the
// benchmark shape).
template <int BM, int BN, int BK, int S, int WGM, int WGN, int EPI, bool KB>
void launch_epi(dim3 grid, dim3 block, hipStream_t s, const uint16_t* A, const uint16_t* W, const float* bias,
                void* C, int M, int N, int K, int ldc, int a_rows, int w_rows, int tiles_m, int group_m, int c_kb,
                const HeadOut& ho) {
#define GPT2_LAUNCH_NK(NK)                                                                                       \
    gemm_bf16_kernel<BM, BN, BK, S, WGM, WGN, EPI, KB, NK><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K, ldc, a_rows, \
                                                                                  w_rows, tiles_m, group_m, c_kb, ho)
    const int nk = K / BK;
    constexpr bool HEAD = EPI == EPI_LOGITS || EPI == EPI_LSE;
    if constexpr (KB || EPI == EPI_LOGITS) {
        if constexpr (BK == 32) {
            if (nk == 24) return (void)GPT2_LAUNCH_NK(24);
            // the vocabulary projection of GPT-2 medium and XL (K = d = 1024, 1600), and their c_attn
            // and c_fc on the 256 x 192 tiles
            if constexpr (HEAD || (KB && BM == 256 && BN == 192 && (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU))) {
                if (nk == 32) return (void)GPT2_LAUNCH_NK(32);
                if (nk == 50) return (void)GPT2_LAUNCH_NK(50);
            }
            // attn.c_proj of GPT-2 XL (N = K = 1600) on the 192 x 256 tiles
            if constexpr (KB && BM == 192 && BN == 256 && EPI == EPI_BIAS_RESIDUAL) {
                if (nk == 50) return (void)GPT2_LAUNCH_NK(50);
            }
        } else {
            if (nk == 12) return (void)GPT2_LAUNCH_NK(12);
            if (nk == 48) return (void)GPT2_LAUNCH_NK(48);
            // the residual projections of GPT-2 medium and XL (K = d and 4d)
            if constexpr (KB && EPI == EPI_BIAS_RESIDUAL) {
                if (nk == 16) return (void)GPT2_LAUNCH_NK(16);
                if (nk == 64) return (void)GPT2_LAUNCH_NK(64);
                if (nk == 25) return (void)GPT2_LAUNCH_NK(25);
                if (nk == 100) return (void)GPT2_LAUNCH_NK(100);
            }
            if constexpr (!KB) {
                if (nk == 36) return (void)GPT2_LAUNCH_NK(36);
                if (nk == 64) return (void)GPT2_LAUNCH_NK(64);
            }
        }
    }
    GPT2_LAUNCH_NK(0);
#undef GPT2_LAUNCH_NK
}

template <int BM, int BN, int BK, int S, int WGM, int WGN, bool KB>
hipError_t launch_cfg(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K, long ldc,
                      int epi, int gelu_erf, int a_rows, int w_rows, int c_kb, const HeadOut& ho, hipStream_t s) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    // group_m in [1, 1000): XCD-contiguous remap + groups of group_m row-tiles; < 0: plain order,
    // groups of -group_m; >= 1000: XCD-interleaved groups of group_m - 1000 row-tiles. Measured in
    // the forward (cold caches for the wte operand), vocabulary projection on 128 x 256 tiles:
    // XCD-interleaved groups of 3-6 row-tiles 364-366 us, of 2 392 us, of 8 383 us, of 1 519 us;
    // XCD-contiguous ranges 457 us and more, plain pairs 506 us. With interleaved groups each wte
    // tile is read into one XCD's L2 per group of row-tiles instead of into several, while the eight
    // XCDs sweep neighbouring columns together, so the logits are written in long runs. The block
    // projections are insensitive to the order.
    int group_m = tiles_n >= 64 ? 1004 : 4;
    dim3 grid(tiles_m * tiles_n), block(64 * WGM * WGN);
#define GPT2_LAUNCH(E)                                                                                         \
    launch_epi<BM, BN, BK, S, WGM, WGN, E, KB>(grid, block, s, A, W, bias, C, M, N, K, (int)ldc, a_rows, w_rows, \
                                               tiles_m, group_m, c_kb, ho)
    switch (epi) {
        case EPI_BIAS: GPT2_LAUNCH(EPI_BIAS); break;
        case EPI_BIAS_GELU:
            if (gelu_erf)
                GPT2_LAUNCH(EPI_BIAS_GELU_ERF);
            else
                GPT2_LAUNCH(EPI_BIAS_GELU);
            break;
        case EPI_BIAS_RESIDUAL: GPT2_LAUNCH(EPI_BIAS_RESIDUAL); break;
        case EPI_BIAS_GELU_U:  // (the training forward)
            if (gelu_erf)
                GPT2_LAUNCH(EPI_BIAS_GELU_U_ERF);
            else
                GPT2_LAUNCH(EPI_BIAS_GELU_U);
            break;
        case EPI_LSE: GPT2_LAUNCH(EPI_LSE); break;
        default: GPT2_LAUNCH(EPI_LOGITS); break;
    }
#undef GPT2_LAUNCH
    return hipGetLastError();
}

}  // namespace

// One entry per tile configuration i of kCfgs, each defined in a translation unit of its own so
// that the configurations compile in parallel: launches configuration i for row-major (kb false)
// or k-blocked (kb true) operands.
#define GPT2_GEMM_CFG_PARAMS                                                                                    \
    const uint16_t *A, const uint16_t *W, const float *bias, void *C, int M, int N, int K, long ldc, int epi,     \
        int gelu_erf, int a_rows, int w_rows, int c_kb, const HeadOut &ho, hipStream_t s, bool kb
#define GPT2_GEMM_DECLARE_CFG(i) hipError_t gemm_bf16_cfg_##i(GPT2_GEMM_CFG_PARAMS);
#define GPT2_GEMM_DEFINE_CFG(i)                                                                                 \
    hipError_t gemm_bf16_cfg_##i(GPT2_GEMM_CFG_PARAMS) {                                                        \
        constexpr TileCfg c = kCfgs[i];                                                                         \
        return kb ? launch_cfg<c.bm, c.bn, c.bk, c.stages, c.wgm, c.wgn, true>(A, W, bias, C, M, N, K, ldc, epi,  \
                                                                               gelu_erf, a_rows, w_rows, c_kb,  \
                                                                               ho, s)                           \
                  : launch_cfg<c.bm, c.bn, c.bk, c.stages, c.wgm, c.wgn, false>(A, W, bias, C, M, N, K, ldc, epi, \
                                                                                gelu_erf, a_rows, w_rows, c_kb, \
                                                                                ho, s);                         \
    }
// the configurations the library dispatches to
GPT2_GEMM_DECLARE_CFG(0)
GPT2_GEMM_DECLARE_CFG(1)
GPT2_GEMM_DECLARE_CFG(2)
GPT2_GEMM_DECLARE_CFG(3)
GPT2_GEMM_DECLARE_CFG(4)
GPT2_GEMM_DECLARE_CFG(5)

}  // namespace gpt2k
