// bf16 GEMM dispatch: the tile configuration per GEMM shape (choose_cfg) and the entry point.
// The kernel, its tile table and launchers are in gemm_bf16_impl.h; each configuration the
// library uses is instantiated in a translation unit of its own (gemm_bf16_c<i>.hip).
#include "gemm_bf16_impl.h"

namespace gpt2k {
namespace {

// Tile shape per GEMM shape, from measurements on MI355X at M = 4096 (bf16, K = 768 / 3072).
// The block projections are bound by their operand traffic through L2 (re-reads grow as tiles
// shrink), so the largest tile that still gives every CU about one tile wins: 192 x 256 for
// N = 2304 (198 tiles, a five-stage 32-wide ring), 256 x 192 for N = 3072 (256 tiles; with
// k-blocked operands the five-stage 32-wide ring, else the two-stage 64-wide one). Narrow outputs
// (N <= 1024) on k-blocked operands take 128 x 96 tiles of eight wavefronts (4 x 2, 32 x 48 each)
// with a four-stage 64-wide ring: two wavefronts per SIMD hide the LDS and barrier latency that a
// single one leaves exposed (per forward, mlp.c_proj 392 -> 376 us and attn.c_proj 192 -> 176 us
// against 128 x 96 tiles of four wavefronts and 64 x 96 tiles two per CU); row-major narrow
// products (the backward) keep 64 x 96 tiles with a four-stage ring, two workgroups per CU. The
// vocabulary projection, with tiles for every CU many times over, spends about 40% of its time in
// the epilogue (staging, argmax partials, 824 MB of fp32 logits), which overlaps nothing when one
// workgroup fills a CU; it uses 128 x 256 tiles of four waves with a three-stage ring, two
// workgroups per CU, so that one's epilogue runs beside the other's K loop (in the forward: 364-366
// us; 256 x 256 tiles of eight waves with a five-stage ring, one per CU, 404-418 us; 256 x 128
// tiles two per CU 409 us).
int choose_cfg(int M, int N, int K, bool kb) {
    auto tiles = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (tiles(256, 256) >= 4 * 256) return 2;  // vocabulary projection
    // narrow outputs of very many rows (the wte weight gradient, M = n_vocab): large tiles, since
    // the grid fills the CUs twice over anyway and each tile re-reads less through L2
    if (N <= 1024 && tiles(256, 192) >= 512) return 1;
    // narrow outputs on k-blocked operands (attn.c_proj, mlp.c_proj): 128 x 96 tiles of eight
    // wavefronts (two per SIMD, 32 x 48 each), one wave of 256 workgroups at GPT-2 small B*T = 4096
    // (128 x 128 tiles, fewer waves of workgroups for GPT-2 medium and XL, measured slower: medium
    // B=8 forward 8.58 -> 8.87 ms)
    if (N <= 1024 && kb && tiles(128, 96) >= 192) return 5;
    if (N <= 1024) return 0;
    if (tiles(192, 256) < 128) return 0;  // few rows (weight gradients, short prompts): fill the CUs
    if (tiles(192, 256) <= 256) return 3;
    // k-blocked operands stream at full cache-line width, which favours the deeper 32-wide ring, also
    // when the grid takes several waves (GPT-2 medium B=8 forward 9.06 -> 8.52 ms, XL B=4 20.04 ->
    // 18.41 ms against the two-stage 64-wide ring, with bit-identical logits)
    if (kb) return 4;
    return 1;
}

}  // namespace

// (the vocabulary projection takes the same tile in either operand layout)
int gemm_bf16_tile_n(int M, int N, int K) { return M <= kSkinnyM ? 16 : kCfgs[choose_cfg(M, N, K, false)].bn; }

hipError_t gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C, int M, int N, int K, long ldc,
                     int epi, int gelu_erf, int a_rows, int w_rows, const HeadOut& ho, hipStream_t s, bool kb,
                     int c_kb_rows) {
    if (ldc < N || ldc > (1 << 26)) return hipErrorInvalidValue;  // in-strip offsets are 32-bit
    // a separate residual source and the saved GELU input: tiled kernel, row-major output only
    if (ho.res && (epi != EPI_BIAS_RESIDUAL || M <= kSkinnyM)) return hipErrorInvalidValue;
    if (epi == EPI_BIAS_GELU_U && (!ho.u || M <= kSkinnyM || (ldc & 3))) return hipErrorInvalidValue;
    if (M <= kSkinnyM) {  // a few rows: a stream over W (row-major operands and output only)
        if (kb || c_kb_rows) return hipErrorInvalidValue;
        return gemm_bf16_skinny(A, W, bias, C, M, N, K, (int)ldc, epi, gelu_erf, a_rows, w_rows, ho, SkinnyExtra(), s);
    }
    if (c_kb_rows && (epi == EPI_BIAS_RESIDUAL || epi == EPI_LOGITS || epi == EPI_LSE || c_kb_rows < M || N % 32))
        return hipErrorInvalidValue;  // k-blocked output: bf16 epilogues only
    if (kb && K % 32) return hipErrorInvalidValue;
    switch (choose_cfg(M, N, K, kb)) {
#define GPT2_CFG(i) \
    case i: return gemm_bf16_cfg_##i(A, W, bias, C, M, N, K, ldc, epi, gelu_erf, a_rows, w_rows, c_kb_rows, ho, s, kb);
        GPT2_CFG(0)
        GPT2_CFG(1)
        GPT2_CFG(2)
        GPT2_CFG(3)
        GPT2_CFG(4)
        GPT2_CFG(5)
#undef GPT2_CFG
    }
    return hipErrorInvalidValue;
}

}  // namespace gpt2k
