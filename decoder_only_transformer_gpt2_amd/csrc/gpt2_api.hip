// Host side of the C ABI declared in include/gpt2.h: configuration checks, packed weight layout,
// workspace carving and the launch sequence of the forward pass. Every device buffer belongs to
// the caller; nothing here allocates device memory.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/gpt2.h"
#include "common.h"
#include "gemm_tn.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kRowPad = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct TensorSlot {
    int64_t rows, cols;  // source shape (cols = 0 for a vector)
    int64_t rows_padded;  // matrices: rows rounded up to kRowPad
    size_t offset;        // byte offset in the packed buffer
    bool matrix;
};

// Per-layer tensor indices inside the fixed source order.
enum LayerTensor {
    LN1_W = 0, LN1_B, ATTN_W, ATTN_B, APROJ_W, APROJ_B, LN2_W, LN2_B, FC_W, FC_B, MPROJ_W, MPROJ_B, PER_LAYER
};

struct WorkspaceLayout {
    size_t x, a, qkv, o, hid, amax_v, amax_i, tgt, tgt_logit, xl, al, flags, total;
    int64_t Mp;
    int n_part;
};

// Key/value cache arguments of the trunk: append this call's keys and values at positions pos0 ..
// pos0 + T - 1; with from_cache (one new position per sequence) the attention reads the cache.
struct KVArgs {
    char* cache = nullptr;
    int pos0 = 0;
    bool from_cache = false;
};

}  // namespace

struct gpt2_model {
    gpt2_config_t cfg;
    std::vector<TensorSlot> slots;
    // bf16: byte offset of the k-blocked copy of each GEMM weight (wte and the four projections of
    // every layer), read by the tiled GEMMs of the forward; 0 for other tensors
    std::vector<size_t> kb_offset;
    size_t weight_bytes = 0;
    void* weights = nullptr;  // borrowed device pointer, set by gpt2_load_weights
    bool loaded = false;
};

namespace {

bool is_bf16(const gpt2_model* m) { return m->cfg.dtype == GPT2_BF16; }
size_t act_size(const gpt2_model* m) { return is_bf16(m) ? 2 : 4; }

void build_layout(gpt2_model* m) {
    const gpt2_config_t& c = m->cfg;
    const int64_t d = c.d_model, f = c.d_mlp;
    auto mat = [&](int64_t r, int64_t k) { m->slots.push_back({r, k, round_up(r, kRowPad), 0, true}); };
    auto vec = [&](int64_t n) { m->slots.push_back({n, 0, n, 0, false}); };
    mat(c.n_vocab, d);  // wte (also the lm_head operand)
    mat(c.n_ctx, d);    // wpe
    for (int l = 0; l < c.n_layer; ++l) {
        vec(d); vec(d);
        mat(3 * d, d); vec(3 * d);
        mat(d, d); vec(d);
        vec(d); vec(d);
        mat(f, d); vec(f);
        mat(d, f); vec(d);
    }
    vec(d); vec(d);  // ln_f
    size_t off = 0;
    for (auto& s : m->slots) {
        s.offset = off;
        const size_t bytes = s.matrix ? (size_t)s.rows_padded * s.cols * act_size(m) : (size_t)s.rows * 4;
        off = align_up(off + bytes, kAlign);
    }
    m->kb_offset.assign(m->slots.size(), 0);
    if (c.dtype == GPT2_BF16) {
        auto kb = [&](int i) {
            m->kb_offset[i] = off;
            off = align_up(off + (size_t)m->slots[i].rows_padded * m->slots[i].cols * 2, kAlign);
        };
        kb(0);  // wte as the lm_head operand
        for (int l = 0; l < c.n_layer; ++l)
            for (int t : {ATTN_W, APROJ_W, FC_W, MPROJ_W}) kb(2 + l * PER_LAYER + t);
    }
    m->weight_bytes = off;
}

const void* wptr(const gpt2_model* m, int idx) { return static_cast<const char*>(m->weights) + m->slots[idx].offset; }
const void* wptr_kb(const gpt2_model* m, int idx) {
    return static_cast<const char*>(m->weights) + m->kb_offset[idx];
}
int layer_idx(int l, int t) { return 2 + l * PER_LAYER + t; }

WorkspaceLayout ws_layout(const gpt2_model* m, int B, int T) {
    const gpt2_config_t& c = m->cfg;
    WorkspaceLayout w{};
    const int64_t M = (int64_t)B * T;
    w.Mp = round_up(M, kRowPad);
    const size_t as = act_size(m);
    auto n_part = [&](int rows) {
        const int bn = is_bf16(m) ? gpt2k::gemm_bf16_tile_n(rows, c.n_vocab, c.d_model) : gpt2k::kGemmF32BN;
        return (c.n_vocab + bn - 1) / bn;
    };
    w.n_part = n_part((int)M);
    // the head partials serve the M-row projection and the B-row next-token projection of cached
    // decoding, whose tile width can differ
    const size_t n_head_part = std::max((size_t)M * w.n_part, (size_t)B * n_part(B));
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, kAlign); return o; };
    w.x = take((size_t)w.Mp * c.d_model * 4);
    w.a = take((size_t)w.Mp * c.d_model * as);
    w.qkv = take((size_t)w.Mp * 3 * c.d_model * as);
    w.o = take((size_t)w.Mp * c.d_model * as);
    w.hid = take((size_t)w.Mp * c.d_mlp * as);
    w.amax_v = take(n_head_part * 4);  // head partials: argmax value / base-2 maximum
    w.amax_i = take(n_head_part * 4);  // argmax index / sum below the maximum
    w.tgt = take((size_t)M * 4);                // cross-entropy target column per row
    w.tgt_logit = take((size_t)M * 4);          // and its logit
    // cached decoding: the B rows whose logits are wanted (fp32 residual, ln_f output)
    const int64_t Bp = round_up(B, kRowPad);
    w.xl = take((size_t)B * c.d_model * 4);
    w.al = take((size_t)Bp * c.d_model * as);
    w.flags = take((size_t)gpt2k::embed_flag_count((int)M) * 4);
    w.total = off;
    return w;
}

#define GPT2_HIP(call)                              \
    do {                                            \
        if ((call) != hipSuccess) return GPT2_EHIP; \
    } while (0)

gpt2_status check_run_args(const gpt2_model* m, const int32_t* tokens, int B, int T, const void* out, const void* ws,
                           size_t ws_bytes) {
    if (!m || !tokens || !out || !ws) return GPT2_EINVAL;
    if (!m->loaded) return GPT2_ESTATE;
    if (B < 1 || T < 1 || T > m->cfg.n_ctx) return GPT2_ESHAPE;
    if ((int64_t)B * T > (int64_t)1 << 24) return GPT2_ESHAPE;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return GPT2_EINVAL;
    if (ws_bytes < ws_layout(m, B, T).total) return GPT2_EWORKSPACE;
    return GPT2_OK;
}

// Linear dispatch on the compute dtype. kb (bf16, tiled GEMM): A is k-blocked with M rounded up to
// kRowPad rows per block and the weight's k-blocked copy is read; c_kb: the bf16 output is written
// k-blocked the same way.
hipError_t linear(const gpt2_model* m, const void* A, int widx, int bidx, void* C, int M, int N, int K, long ldc,
                  int epi, const gpt2k::HeadOut& ho, hipStream_t s, bool kb = false, bool c_kb = false) {
    const float* bias = bidx >= 0 ? static_cast<const float*>(wptr(m, bidx)) : nullptr;
    const int ge = m->cfg.gelu == GPT2_GELU_ERF;
    // a few rows: the W-streaming kernel over the weight's k-blocked copy (whole cache lines)
    if (is_bf16(m) && M <= gpt2k::kSkinnyM && !kb && !c_kb && m->kb_offset[widx])
        return gpt2k::gemm_bf16_skinny(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(wptr_kb(m, widx)),
                                       bias, C, M, N, K, (int)ldc, epi, ge, (int)round_up(M, kRowPad),
                                       (int)m->slots[widx].rows_padded, ho, {}, s, true);
    if (is_bf16(m))
        return gpt2k::gemm_bf16(static_cast<const uint16_t*>(A),
                                static_cast<const uint16_t*>(kb ? wptr_kb(m, widx) : wptr(m, widx)), bias, C, M, N, K,
                                ldc, epi, ge, (int)round_up(M, kRowPad), (int)m->slots[widx].rows_padded, ho, s, kb,
                                c_kb ? (int)round_up(M, kRowPad) : 0);
    return gpt2k::gemm_f32(static_cast<const float*>(A), static_cast<const float*>(wptr(m, widx)), bias, C, M, N, K, ldc,
                           epi, ge, ho, s);
}

// Enqueues launches in order, optionally recording caller events around them, or (dry) only
// counts them and reports their kinds.
struct Sequencer {
    hipStream_t s;
    hipEvent_t* before = nullptr;
    hipEvent_t* after = nullptr;
    int n_slots = 0;
    int32_t* kinds = nullptr;
    int cap = 0;
    bool dry = false;
    int idx = 0;
    // launch rep_idx is enqueued rep_n times back to back, with rep_before / rep_after around the
    // group (for timing one kernel without per-launch event gaps)
    int rep_idx = -1, rep_n = 1;
    hipEvent_t rep_before = nullptr, rep_after = nullptr;

    template <class F>
    hipError_t run(int kind, F&& launch) {
        if (kinds && idx < cap) kinds[idx] = kind;
        if (dry) {
            ++idx;
            return hipSuccess;
        }
        const bool slot = idx < n_slots;
        if (slot && before && before[idx] && hipEventRecord(before[idx], s) != hipSuccess) return hipErrorUnknown;
        hipError_t e = hipSuccess;
        if (idx == rep_idx) {
            if (rep_before && hipEventRecord(rep_before, s) != hipSuccess) return hipErrorUnknown;
            for (int r = 0; r < rep_n && e == hipSuccess; ++r) e = launch();
            if (e == hipSuccess && rep_after) e = hipEventRecord(rep_after, s);
        } else {
            e = launch();
        }
        if (e == hipSuccess && slot && after && after[idx]) e = hipEventRecord(after[idx], s);
        ++idx;
        return e;
    }
};

#define GPT2_RUN(kind, expr)                                                   \
    do {                                                                       \
        if (q.run(kind, [&]() { return (expr); }) != hipSuccess) return GPT2_EHIP; \
    } while (0)

// Embedding and the first n_layers blocks; leaves the residual stream in the workspace's x.
size_t kv_layer_elems(const gpt2_model* m, int B) { return (size_t)B * m->cfg.d_model * m->cfg.n_ctx; }

gpt2_status enqueue_trunk(const gpt2_model* m, const int32_t* tokens, int B, int T, int n_layers, char* ws,
                          const WorkspaceLayout& w, Sequencer& q, const KVArgs& kv = KVArgs()) {
    const gpt2_config_t& c = m->cfg;
    const hipStream_t s = q.s;
    const int M = B * T, d = c.d_model, f = c.d_mlp, H = c.n_head;
    const bool bf = is_bf16(m);
    float* x = reinterpret_cast<float*>(ws + w.x);
    void* a = ws + w.a;
    void* qkv = ws + w.qkv;
    void* o = ws + w.o;
    void* hid = ws + w.hid;
    // bf16 with tiled GEMMs: the operands the GEMMs read (the LayerNorm outputs, the attention
    // output and the GELU output) are written k-blocked, Mp rows per 32-column block
    const bool kbl = bf && M > gpt2k::kSkinnyM && !kv.from_cache;
    const int Mp = kbl ? (int)w.Mp : 0;
    // with k-blocked operands the first block's ln_1 is computed by the embedding launch
    const bool embed_ln1 = kbl && n_layers > 0;
    if (embed_ln1)
        GPT2_RUN(GPT2_K_EMBED, gpt2k::embed_ln(tokens, static_cast<const uint16_t*>(wptr(m, 0)),
                                               static_cast<const uint16_t*>(wptr(m, 1)), x,
                                               static_cast<const float*>(wptr(m, layer_idx(0, LN1_W))),
                                               static_cast<const float*>(wptr(m, layer_idx(0, LN1_B))),
                                               static_cast<uint16_t*>(a), M, T, kv.pos0, d, c.n_vocab, c.ln_eps, Mp,
                                               reinterpret_cast<int32_t*>(ws + w.flags), s));
    else
        GPT2_RUN(GPT2_K_EMBED, gpt2k::embed(tokens, wptr(m, 0), wptr(m, 1), x, M, T, kv.pos0, d, c.n_vocab, bf,
                                            reinterpret_cast<int32_t*>(ws + w.flags), s));
    // q, k, v views of qkv [B, T, 3, H, 64]: strides (batch, head, token) in elements
    // cached decoding in bf16 with few rows: LayerNorms and the cache append fused into the
    // projections (fewer, larger launches)
    const bool fuse = kv.from_cache && bf && M <= gpt2k::kSkinnyM && d < 2048;
    auto skinny = [&](int widx, int bidx, void* C, int N, int K, int epi, const gpt2k::SkinnyExtra& ex) {
        return gpt2k::gemm_bf16_skinny(static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(wptr_kb(m, widx)),
                                       static_cast<const float*>(wptr(m, bidx)), C, M, N, K, N, epi,
                                       c.gelu == GPT2_GELU_ERF, (int)w.Mp, (int)m->slots[widx].rows_padded, {}, ex, s,
                                       true);
    };
    const int64_t qs[3] = {(int64_t)T * 3 * d, 64, 3 * d};
    const int64_t os[3] = {kbl ? (int64_t)T * 32 : (int64_t)T * d, kbl ? (int64_t)2 * Mp * 32 : 64, kbl ? 32 : d};
    const int64_t os_half = kbl ? (int64_t)Mp * 32 : 32;
    const size_t as = act_size(m);
    for (int l = 0; l < n_layers; ++l) {
        auto L = [&](int t) { return layer_idx(l, t); };
        auto vecp = [&](int t) { return static_cast<const float*>(wptr(m, L(t))); };
        const char* qb = static_cast<const char*>(qkv);
        char* kc = nullptr;
        char* vc = nullptr;
        if (kv.cache) {
            kc = kv.cache + (size_t)2 * l * kv_layer_elems(m, B) * as;
            vc = kc + kv_layer_elems(m, B) * as;
        }
        if (fuse) {
            // one launch: ln_1, the QKV projection, and this position's k and v into the cache
            gpt2k::SkinnyExtra ex;
            ex.ln_x = x;
            ex.ln_g = vecp(LN1_W);
            ex.ln_b = vecp(LN1_B);
            ex.ln_eps = c.ln_eps;
            ex.kc = reinterpret_cast<uint16_t*>(kc);
            ex.vc = reinterpret_cast<uint16_t*>(vc);
            ex.kv_n_ctx = c.n_ctx;
            ex.kv_pos = kv.pos0;
            GPT2_RUN(GPT2_K_QKV, skinny(L(ATTN_W), L(ATTN_B), qkv, 3 * d, d, gpt2k::EPI_BIAS, ex));
        } else {
            if (!(embed_ln1 && l == 0))
                GPT2_RUN(GPT2_K_LN, gpt2k::layernorm(x, vecp(LN1_W), vecp(LN1_B), a, M, d, c.ln_eps, bf, s, Mp));
            GPT2_RUN(GPT2_K_QKV,
                     linear(m, a, L(ATTN_W), L(ATTN_B), qkv, M, 3 * d, d, 3 * d, gpt2k::EPI_BIAS, {}, s, kbl));
            if (kv.cache) GPT2_RUN(GPT2_K_KV, gpt2k::kv_append(qkv, B, T, H, kv.pos0, kc, vc, c.n_ctx, bf, s));
        }
        if (kv.from_cache)
            GPT2_RUN(GPT2_K_ATTN, gpt2k::decode_attention(qkv, kc, vc, o, B, H, c.n_ctx, kv.pos0 + 1, bf, s));
        else if (bf)
            GPT2_RUN(GPT2_K_ATTN, gpt2k::attention_bf16(reinterpret_cast<const uint16_t*>(qb), qs,
                                                        reinterpret_cast<const uint16_t*>(qb + d * as), qs,
                                                        reinterpret_cast<const uint16_t*>(qb + 2 * d * as), qs,
                                                        static_cast<uint16_t*>(o), os, B, H, T, s, os_half));
        else
            GPT2_RUN(GPT2_K_ATTN, gpt2k::attention_f32(reinterpret_cast<const float*>(qb), qs,
                                                       reinterpret_cast<const float*>(qb + d * as), qs,
                                                       reinterpret_cast<const float*>(qb + 2 * d * as), qs,
                                                       static_cast<float*>(o), os, B, H, T, s));
        GPT2_RUN(GPT2_K_ATTN_PROJ, linear(m, o, L(APROJ_W), L(APROJ_B), x, M, d, d, d, gpt2k::EPI_BIAS_RESIDUAL,
                                          {}, s, kbl));
        if (fuse) {  // ln_2 inside the c_fc projection
            gpt2k::SkinnyExtra ex;
            ex.ln_x = x;
            ex.ln_g = vecp(LN2_W);
            ex.ln_b = vecp(LN2_B);
            ex.ln_eps = c.ln_eps;
            GPT2_RUN(GPT2_K_FC, skinny(L(FC_W), L(FC_B), hid, f, d, gpt2k::EPI_BIAS_GELU, ex));
        } else {
            GPT2_RUN(GPT2_K_LN, gpt2k::layernorm(x, vecp(LN2_W), vecp(LN2_B), a, M, d, c.ln_eps, bf, s, Mp));
            GPT2_RUN(GPT2_K_FC,
                     linear(m, a, L(FC_W), L(FC_B), hid, M, f, d, f, gpt2k::EPI_BIAS_GELU, {}, s, kbl, kbl));
        }
        GPT2_RUN(GPT2_K_MLP_PROJ, linear(m, hid, L(MPROJ_W), L(MPROJ_B), x, M, d, f, d, gpt2k::EPI_BIAS_RESIDUAL,
                                         {}, s, kbl));
    }
    return GPT2_OK;
}

// The whole forward: trunk, ln_f, tied lm_head (+ argmax partials), argmax reduction.
gpt2_status enqueue_forward(const gpt2_model* m, const int32_t* tokens, int B, int T, float* logits, int32_t* argmax,
                            char* ws, Sequencer& q) {
    const gpt2_config_t& c = m->cfg;
    const hipStream_t s = q.s;
    const WorkspaceLayout w = ws_layout(m, B, T);
    const int M = B * T;
    gpt2_status st = enqueue_trunk(m, tokens, B, T, c.n_layer, ws, w, q);
    if (st != GPT2_OK) return st;
    const int ln_f = 2 + c.n_layer * PER_LAYER;
    const bool kbl = is_bf16(m) && M > gpt2k::kSkinnyM;  // the head reads a k-blocked ln_f output
    GPT2_RUN(GPT2_K_LN_F, gpt2k::layernorm(reinterpret_cast<float*>(ws + w.x), static_cast<const float*>(wptr(m, ln_f)),
                                           static_cast<const float*>(wptr(m, ln_f + 1)), ws + w.a, M, c.d_model,
                                           c.ln_eps, is_bf16(m), s, kbl ? (int)w.Mp : 0));
    gpt2k::HeadOut ho;
    if (argmax) {
        ho.pv = reinterpret_cast<float*>(ws + w.amax_v);
        ho.pi = reinterpret_cast<int32_t*>(ws + w.amax_i);
    }
    GPT2_RUN(GPT2_K_LM_HEAD,
             linear(m, ws + w.a, 0, -1, logits, M, c.n_vocab, c.d_model, c.n_vocab, gpt2k::EPI_LOGITS, ho, s, kbl));
    if (argmax) GPT2_RUN(GPT2_K_ARGMAX, gpt2k::argmax_reduce(ho.pv, ho.pi, M, w.n_part, argmax, s));
    return GPT2_OK;
}

// The forward followed by the shifted cross-entropy ([手写] §4.1): trunk, ln_f, targets, the
// vocabulary projection with the log-sum-exp epilogue (no logits stored), per-row losses, mean.
gpt2_status enqueue_forward_loss(const gpt2_model* m, const int32_t* tokens, const int32_t* labels, int B, int T,
                                 float* nll, float* loss, char* ws, Sequencer& q) {
    const gpt2_config_t& c = m->cfg;
    const hipStream_t s = q.s;
    const WorkspaceLayout w = ws_layout(m, B, T);
    const int M = B * T;
    gpt2_status st = enqueue_trunk(m, tokens, B, T, c.n_layer, ws, w, q);
    if (st != GPT2_OK) return st;
    const int ln_f = 2 + c.n_layer * PER_LAYER;
    const bool kbl = is_bf16(m) && M > gpt2k::kSkinnyM;
    GPT2_RUN(GPT2_K_LN_F, gpt2k::layernorm(reinterpret_cast<float*>(ws + w.x), static_cast<const float*>(wptr(m, ln_f)),
                                           static_cast<const float*>(wptr(m, ln_f + 1)), ws + w.a, M, c.d_model,
                                           c.ln_eps, is_bf16(m), s, kbl ? (int)w.Mp : 0));
    int32_t* tgt = reinterpret_cast<int32_t*>(ws + w.tgt);
    GPT2_RUN(GPT2_K_XENT, gpt2k::xent_targets(labels ? labels : tokens, M, T, c.n_vocab, tgt,
                                              reinterpret_cast<int32_t*>(ws + w.flags), s));
    gpt2k::HeadOut ho;
    ho.pv = reinterpret_cast<float*>(ws + w.amax_v);
    ho.ps = reinterpret_cast<float*>(ws + w.amax_i);
    ho.tgt = tgt;
    ho.tgt_logit = reinterpret_cast<float*>(ws + w.tgt_logit);
    GPT2_RUN(GPT2_K_LM_HEAD,
             linear(m, ws + w.a, 0, -1, nullptr, M, c.n_vocab, c.d_model, c.n_vocab, gpt2k::EPI_LSE, ho, s, kbl));
    GPT2_RUN(GPT2_K_XENT, gpt2k::xent_rows(ho.pv, ho.ps, tgt, ho.tgt_logit, M, w.n_part, nll, s));
    GPT2_RUN(GPT2_K_XENT, gpt2k::xent_mean(nll, tgt, M, loss, s));
    return GPT2_OK;
}

// ln_f and the tied lm_head on B rows of the residual (fp32 [B, d] at xr): the next-token logits
// (not stored when logits is NULL) and their argmax.
gpt2_status enqueue_next_token(const gpt2_model* m, const float* xr, int B, float* logits, int32_t* next, char* ws,
                               const WorkspaceLayout& w, Sequencer& q) {
    const gpt2_config_t& c = m->cfg;
    const hipStream_t s = q.s;
    const int ln_f = 2 + c.n_layer * PER_LAYER;
    gpt2k::HeadOut ho;
    if (next) {
        ho.pv = reinterpret_cast<float*>(ws + w.amax_v);
        ho.pi = reinterpret_cast<int32_t*>(ws + w.amax_i);
    }
    // (a separate ln_f: fused into the projection, each of its ~3000 workgroups would redo the
    // row statistics, which measured slower)
    GPT2_RUN(GPT2_K_LN_F, gpt2k::layernorm(xr, static_cast<const float*>(wptr(m, ln_f)),
                                           static_cast<const float*>(wptr(m, ln_f + 1)), ws + w.al, B, c.d_model,
                                           c.ln_eps, is_bf16(m), s));
    GPT2_RUN(GPT2_K_LM_HEAD, linear(m, ws + w.al, 0, -1, logits, B, c.n_vocab, c.d_model, c.n_vocab,
                                    gpt2k::EPI_LOGITS, ho, s));
    if (next) {
        // the partial count of a B-row projection (the tile width depends on the shape)
        const int bn = is_bf16(m) ? gpt2k::gemm_bf16_tile_n(B, c.n_vocab, c.d_model) : gpt2k::kGemmF32BN;
        GPT2_RUN(GPT2_K_ARGMAX, gpt2k::argmax_reduce(ho.pv, ho.pi, B, (c.n_vocab + bn - 1) / bn, next, s));
    }
    return GPT2_OK;
}

size_t kv_cache_bytes(const gpt2_model* m, int B) { return 2 * (size_t)m->cfg.n_layer * kv_layer_elems(m, B) * act_size(m); }

gpt2_status check_cache(const gpt2_model* m, int B, const void* cache, size_t cache_bytes) {
    if (!cache) return GPT2_EINVAL;
    if (reinterpret_cast<uintptr_t>(cache) % kAlign) return GPT2_EINVAL;
    if (cache_bytes < kv_cache_bytes(m, B)) return GPT2_EWORKSPACE;
    return GPT2_OK;
}

// ------------------------------------------------------------------------------ training
// Gradient buffer: the fp32 gradient of source tensor i (in the order of gpt2_tensor_shape) starts
// at grad_offset(i) bytes, every tensor 256-byte aligned, rows unpadded.
size_t grad_offset(const gpt2_model* m, int i) {
    size_t off = 0;
    for (int j = 0; j < i; ++j) {
        const TensorSlot& t = m->slots[j];
        off = align_up(off + (size_t)t.rows * (t.matrix ? t.cols : 1) * 4, kAlign);
    }
    return off;
}

// Training workspace: the forward workspace first (so gpt2_check finds its flags), then the saved
// activations of every layer, the head, and the buffers of the backward.
struct TrainLayout {
    WorkspaceLayout fw;
    size_t layer0, per_layer;
    size_t l_xin, l_xmid, l_a1, l_qkv, l_o, l_a2, l_u, l_h, l_lse;  // inside one layer's block
    size_t splitk, splitk_elems, dact2;
    size_t xfin, xf, logits, dx, dbuf, dbuf2, dact, dT, xT, wT, wteT, dlog, dlogT, part, bpart, lnpg, lnpb, lse, dvec, nll,
        cnt;
    size_t total;
    int64_t M, Mp, Mk, Vp, Vr, wide, rows_w, rows_dT, rows_x;
};

TrainLayout train_layout(const gpt2_model* m, int B, int T) {
    const gpt2_config_t& c = m->cfg;
    TrainLayout L{};
    L.fw = ws_layout(m, B, T);
    const size_t as = act_size(m);
    const int64_t d = c.d_model, f = c.d_mlp;
    L.M = (int64_t)B * T;
    L.Mp = round_up(L.M, kRowPad);     // rows of a GEMM A operand
    L.Mk = round_up(L.M, 64);          // reduction length of the weight-gradient GEMMs
    L.Vp = round_up(c.n_vocab, 64);    // reduction length of the lm_head input gradient
    L.Vr = round_up(c.n_vocab, kRowPad);
    L.wide = std::max(3 * d, f);
    L.rows_w = round_up(std::max(d, f), kRowPad);
    L.rows_dT = round_up(L.wide, kRowPad);
    L.rows_x = round_up(std::max(d, f), kRowPad);
    size_t off = L.fw.total;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, kAlign); return o; };
    size_t lo = 0;
    auto ltake = [&](size_t bytes) { size_t o = lo; lo = align_up(lo + bytes, kAlign); return o; };
    L.l_xin = ltake(L.M * d * 4);
    L.l_xmid = ltake(L.M * d * 4);
    L.l_a1 = ltake(L.Mp * d * as);
    L.l_qkv = ltake(L.Mp * 3 * d * as);
    L.l_o = ltake(L.Mp * d * as);
    L.l_a2 = ltake(L.Mp * d * as);
    L.l_u = ltake(L.M * f * 4);
    L.l_h = ltake(L.Mp * f * as);
    // bf16: each query's log-sum-exp from the forward attention, read by the attention backward
    L.l_lse = ltake(is_bf16(m) ? (size_t)B * c.n_head * T * 4 : 0);
    L.per_layer = lo;
    L.layer0 = take(L.per_layer * c.n_layer);
    L.xfin = take(L.M * d * 4);
    L.xf = take(L.Mp * d * as);
    L.logits = take((size_t)L.M * L.Vp * 4);  // row stride Vp: rows 256-byte aligned for the loss gradient
    L.dx = take(L.M * d * 4);
    L.dbuf = take(L.M * L.wide * 4);
    L.dbuf2 = take(L.M * L.wide * 4);
    L.dact = take(L.Mp * L.wide * as);
    // bf16: c_fc's output gradient, written by the GELU-backward epilogue of mlp.c_proj's input gradient
    L.dact2 = take(is_bf16(m) ? L.Mp * c.d_mlp * 2 : 0);
    // transposed operands (fp32 mode only: the bf16 products read M-major operands directly)
    const bool tr_ops = !is_bf16(m);
    L.dT = take(tr_ops ? L.rows_dT * L.Mk * as : 0);
    L.xT = take(tr_ops ? L.rows_x * L.Mk * as : 0);
    L.wT = take(tr_ops ? L.rows_w * L.wide * as : 0);
    L.wteT = take(tr_ops ? round_up(d, kRowPad) * L.Vp * as : 0);
    L.dlog = take(L.Mp * L.Vp * as);
    L.dlogT = take(tr_ops ? L.Vr * L.Mk * as : 0);
    L.part = take((size_t)std::max<int64_t>(gpt2k::colsum_blocks((int)L.M), (L.Mk + 63) / 64) * L.wide * 4);
    // bf16: the bias gradients' partial column sums of every layer, reduced in one launch at the end
    // (c_fc: one row per 64-row block; c_attn: one per 64-row tile of a sequence, from the attention
    // backward; attn.c_proj, mlp.c_proj: one per LayerNorm-backward block)
    L.bpart = take(is_bf16(m) ? ((size_t)((L.Mk + 63) / 64) * f + (size_t)gpt2k::attention_backward_parts(B, T) * 3 * d +
                                 (size_t)gpt2k::ln_backward_blocks((int)L.M) * 2 * d) * c.n_layer * 4
                              : 0);
    L.lnpg = take((size_t)gpt2k::ln_backward_blocks((int)L.M) * d * 4);
    L.lnpb = take((size_t)gpt2k::ln_backward_blocks((int)L.M) * d * 4);
    L.lse = take(is_bf16(m) ? 0 : (size_t)B * c.n_head * T * 4);  // fp32 mode: the backward finds it
    L.dvec = take((size_t)B * c.n_head * T * 4);
    // partial products of the products split along K (the vocabulary reduction of dxf in six
    // parts, a narrow weight gradient in four)
    L.splitk_elems = is_bf16(m) ? std::max<size_t>((size_t)6 * L.M * d, (size_t)4 * d * d) : 0;
    L.splitk = take(L.splitk_elems * 4);
    L.nll = take(L.M * 4);
    L.cnt = take(4);
    L.total = off;
    return L;
}

// Forward keeping what the backward needs, then the mean shifted cross-entropy and the loss
// gradient with respect to the logits (the GELU input u = a W^T + b is kept in fp32 beside
// h = gelu(u) rounded to the compute dtype, the values the inference epilogue produces).
gpt2_status enqueue_train_forward(const gpt2_model* m, const int32_t* tokens, const int32_t* labels, int B, int T,
                                  float* loss, char* ws, const TrainLayout& L, hipStream_t s) {
    const gpt2_config_t& c = m->cfg;
    const bool bf = is_bf16(m);
    const int M = B * T, d = c.d_model, f = c.d_mlp, H = c.n_head;
    const size_t as = act_size(m);
    const int64_t qs[3] = {(int64_t)T * 3 * d, 64, 3 * d};
    const int64_t os[3] = {(int64_t)T * d, 64, d};
    auto lay = [&](int l, size_t o) { return ws + L.layer0 + (size_t)l * L.per_layer + o; };
    // bf16 on the tiled GEMM (more than kSkinnyM rows): residual sums and the GELU input come from
    // the projections' epilogues
    const bool tiled = bf && M > gpt2k::kSkinnyM;
    const int Mp = (int)L.Mp;
    GPT2_HIP(gpt2k::embed(tokens, wptr(m, 0), wptr(m, 1), reinterpret_cast<float*>(lay(0, L.l_xin)), M, T, 0, d,
                          c.n_vocab, bf, reinterpret_cast<int32_t*>(ws + L.fw.flags), s));
    for (int l = 0; l < c.n_layer; ++l) {
        auto I = [&](int t) { return layer_idx(l, t); };
        auto vecp = [&](int t) { return static_cast<const float*>(wptr(m, I(t))); };
        float* xin = reinterpret_cast<float*>(lay(l, L.l_xin));
        float* xmid = reinterpret_cast<float*>(lay(l, L.l_xmid));
        float* xout = l + 1 < c.n_layer ? reinterpret_cast<float*>(lay(l + 1, L.l_xin)) : reinterpret_cast<float*>(ws + L.xfin);
        char* a1 = lay(l, L.l_a1);
        char* qkv = lay(l, L.l_qkv);
        char* o = lay(l, L.l_o);
        char* a2 = lay(l, L.l_a2);
        float* u = reinterpret_cast<float*>(lay(l, L.l_u));
        char* h = lay(l, L.l_h);
        // tiled bf16: the LayerNorm outputs and the GELU output are k-blocked (the layout the
        // projections stream best; the backward's weight gradients read them that way too)
        GPT2_HIP(gpt2k::layernorm(xin, vecp(LN1_W), vecp(LN1_B), a1, M, d, c.ln_eps, bf, s, tiled ? Mp : 0));
        GPT2_HIP(linear(m, a1, I(ATTN_W), I(ATTN_B), qkv, M, 3 * d, d, 3 * d, gpt2k::EPI_BIAS, {}, s, tiled));
        if (bf)
            GPT2_HIP(gpt2k::attention_bf16(reinterpret_cast<const uint16_t*>(qkv), qs,
                                           reinterpret_cast<const uint16_t*>(qkv + d * as), qs,
                                           reinterpret_cast<const uint16_t*>(qkv + 2 * d * as), qs,
                                           reinterpret_cast<uint16_t*>(o), os, B, H, T, s, 32,
                                           reinterpret_cast<float*>(lay(l, L.l_lse))));
        else
            GPT2_HIP(gpt2k::attention_f32(reinterpret_cast<const float*>(qkv), qs,
                                          reinterpret_cast<const float*>(qkv + d * as), qs,
                                          reinterpret_cast<const float*>(qkv + 2 * d * as), qs,
                                          reinterpret_cast<float*>(o), os, B, H, T, s));
        // each block keeps both residual states: the tiled bf16 GEMM reads the residual from one
        // buffer and writes the sum to the next; otherwise the state is copied and added to in place
        if (tiled) {
            gpt2k::HeadOut hr;
            hr.res = xin;
            GPT2_HIP(linear(m, o, I(APROJ_W), I(APROJ_B), xmid, M, d, d, d, gpt2k::EPI_BIAS_RESIDUAL, hr, s));
        } else {
            GPT2_HIP(hipMemcpyAsync(xmid, xin, (size_t)M * d * 4, hipMemcpyDeviceToDevice, s));
            GPT2_HIP(linear(m, o, I(APROJ_W), I(APROJ_B), xmid, M, d, d, d, gpt2k::EPI_BIAS_RESIDUAL, {}, s));
        }
        GPT2_HIP(gpt2k::layernorm(xmid, vecp(LN2_W), vecp(LN2_B), a2, M, d, c.ln_eps, bf, s, tiled ? Mp : 0));
        if (tiled) {  // u and h = gelu(u) from one epilogue
            gpt2k::HeadOut hu;
            hu.u = u;
            GPT2_HIP(linear(m, a2, I(FC_W), I(FC_B), h, M, f, d, f, gpt2k::EPI_BIAS_GELU_U, hu, s, true, true));
        } else {
            GPT2_HIP(hipMemsetAsync(u, 0, (size_t)M * f * 4, s));
            GPT2_HIP(linear(m, a2, I(FC_W), I(FC_B), u, M, f, d, f, gpt2k::EPI_BIAS_RESIDUAL, {}, s));
            GPT2_HIP(gpt2k::gelu_forward(u, h, (long)M * f, bf, c.gelu == GPT2_GELU_ERF, s));
        }
        if (tiled) {
            gpt2k::HeadOut hr;
            hr.res = xmid;
            GPT2_HIP(linear(m, h, I(MPROJ_W), I(MPROJ_B), xout, M, d, f, d, gpt2k::EPI_BIAS_RESIDUAL, hr, s, true));
        } else {
            GPT2_HIP(hipMemcpyAsync(xout, xmid, (size_t)M * d * 4, hipMemcpyDeviceToDevice, s));
            GPT2_HIP(linear(m, h, I(MPROJ_W), I(MPROJ_B), xout, M, d, f, d, gpt2k::EPI_BIAS_RESIDUAL, {}, s));
        }
    }
    const int ln_f = 2 + c.n_layer * PER_LAYER;
    GPT2_HIP(gpt2k::layernorm(reinterpret_cast<float*>(ws + L.xfin), static_cast<const float*>(wptr(m, ln_f)),
                              static_cast<const float*>(wptr(m, ln_f + 1)), ws + L.xf, M, d, c.ln_eps, bf, s));
    float* logits = reinterpret_cast<float*>(ws + L.logits);
    GPT2_HIP(linear(m, ws + L.xf, 0, -1, logits, M, c.n_vocab, d, L.Vp, gpt2k::EPI_LOGITS, {}, s));
    int32_t* tgt = reinterpret_cast<int32_t*>(ws + L.fw.tgt);
    GPT2_HIP(gpt2k::xent_targets(labels ? labels : tokens, M, T, c.n_vocab, tgt,
                                 reinterpret_cast<int32_t*>(ws + L.fw.flags), s));
    float* nll = reinterpret_cast<float*>(ws + L.nll);
    GPT2_HIP(gpt2k::xent_grad(logits, L.Vp, M, c.n_vocab, (int)L.Vp, tgt, reinterpret_cast<int32_t*>(ws + L.cnt), nll,
                              ws + L.dlog, bf, s));
    GPT2_HIP(gpt2k::xent_mean(nll, tgt, M, loss, s));
    return GPT2_OK;
}

// The backward pass: every gradient into grads (fp32, grad_offset layout), the layers in reverse.
// bf16: each weight gradient dW = dY^T X reduces over the rows of dY and X, read as M-major operands
// (gemm_bf16_tn), and each input gradient dX = dY W reads W [out][in] with the reduction over its
// rows; fp32: both are C = A B^T GEMMs on copies transposed here (K padded with zeros).
gpt2_status enqueue_backward(const gpt2_model* m, const int32_t* tokens, int B, int T, float* grads, char* ws,
                             const TrainLayout& L, hipStream_t s) {
    const gpt2_config_t& c = m->cfg;
    const bool bf = is_bf16(m);
    const int M = B * T, d = c.d_model, f = c.d_mlp, H = c.n_head, V = c.n_vocab;
    const int Mp = (int)L.Mp, Mk = (int)L.Mk, Vp = (int)L.Vp;
    // the tiled bf16 forward left the LayerNorm and GELU outputs k-blocked (Mp rows per 32-column block)
    const bool x_kb = bf && M > gpt2k::kSkinnyM;
    auto lay = [&](int l, size_t o) { return ws + L.layer0 + (size_t)l * L.per_layer + o; };
    auto G = [&](int i) { return grads + grad_offset(m, i) / 4; };
    auto pad = [&](int64_t r) { return (int)round_up(r, kRowPad); };
    float* dx = reinterpret_cast<float*>(ws + L.dx);
    float* dbuf = reinterpret_cast<float*>(ws + L.dbuf);
    float* dbuf2 = reinterpret_cast<float*>(ws + L.dbuf2);
    char* dact = ws + L.dact;
    char* dT = ws + L.dT;
    char* xT = ws + L.xT;
    char* wT = ws + L.wT;
    float* part = reinterpret_cast<float*>(ws + L.part);
    float* splitk = reinterpret_cast<float*>(ws + L.splitk);
    float* lnpg = reinterpret_cast<float*>(ws + L.lnpg);
    float* lnpb = reinterpret_cast<float*>(ws + L.lnpb);
    // C[Mg, Ng] (fp32, row stride ldc) = A[Mg, Kg] B[Ng, Kg]^T in the compute dtype
    auto gemm_nt = [&](const void* A, int a_rows, const void* Bm, int b_rows, float* C, int Mg, int Ng, int Kg,
                       long ldc) {
        if (bf)
            return gpt2k::gemm_bf16(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(Bm), nullptr, C, Mg, Ng,
                                    Kg, ldc, gpt2k::EPI_LOGITS, 0, a_rows, b_rows, {}, s);
        return gpt2k::gemm_f32(static_cast<const float*>(A), static_cast<const float*>(Bm), nullptr, C, Mg, Ng, Kg, ldc,
                               gpt2k::EPI_LOGITS, 0, {}, s);
    };
    // dst (compute dtype) [C rows, ldd] = transpose of src [R, C] (row stride lds), zero for R <= r < Rp
    auto tr = [&](const void* src, bool src_act, long lds, int R, int Cc, void* dst, long ldd, int Rp) {
        return gpt2k::transpose(src, src_act && bf, lds, R, Cc, dst, bf, ldd, Rp, s);
    };
    // row-major fp32 [M, C] -> compute dtype [Mp, C] (rows past M zero)
    auto to_act = [&](const float* src, int Cc, void* dst) {
        return gpt2k::convert(src, false, dst, bf, (long)M * Cc, (long)Mp * Cc, s);
    };
    // bf16: the bias gradients' partial column sums, one region per bias, reduced together at the end
    std::vector<gpt2k::ColsumSeg> bsegs;
    float* bpart = reinterpret_cast<float*>(ws + L.bpart);
    const int nbp = (int)((Mk + 63) / 64);
    // bf16: the weight gradient and the input gradient from the bf16 output gradient dy16 (rows M .. Mk-1
    // zero) whose bias partial sums are at bp; gb: the input gradient goes through the GELU backward
    // into c_fc's output gradient instead (dx_out unused)
    // (x_kb: the activation x is k-blocked with Mp rows per block, as the tiled forward writes it)
    // (nb: the partial rows at bp)
    auto linear_back16 = [&](const uint16_t* dy16, float* bp, int nb, int n_out, const void* x_act, int n_in,
                             bool x_kb, int widx, float* dx_out, const gpt2k::TnGeluBack* gb) -> hipError_t {
        hipError_t e;
        bsegs.push_back({bp, G(widx + 1), nb, n_out});
        // dW [n_out, n_in] = sum over rows m < Mk of dy[m]^T x[m]
        if ((e = gpt2k::gemm_bf16_tn(dy16, true, n_out, n_out, static_cast<const uint16_t*>(x_act), true,
                                     x_kb ? Mp : n_in, n_in, G(widx), n_in, n_out, n_in, Mk, s, splitk,
                                     L.splitk_elems, nullptr, x_kb)) != hipSuccess)
            return e;
        // dX [M, n_in] = dy W, W [n_out][n_in] reduced over its rows
        return gpt2k::gemm_bf16_tn(dy16, false, n_out, Mk, static_cast<const uint16_t*>(wptr(m, widx)), true, n_in,
                                   n_in, dx_out, n_in, M, n_in, n_out, s, nullptr, 0, gb);
    };
    // fp32: the weight gradient and the input gradient of y = x W^T + b for output gradient dy ([M, n_out])
    auto linear_back = [&](const float* dy, int n_out, const void* x_act, int n_in, bool x_kb, int widx,
                           float* dx_out) -> hipError_t {
        hipError_t e;
        if ((e = gpt2k::colsum(dy, n_out, M, n_out, part, G(widx + 1), s)) != hipSuccess) return e;
        if ((e = tr(dy, false, n_out, M, n_out, dT, Mk, Mk)) != hipSuccess) return e;
        if ((e = tr(x_act, true, n_in, M, n_in, xT, Mk, Mk)) != hipSuccess) return e;
        if ((e = gemm_nt(dT, pad(n_out), xT, pad(n_in), G(widx), n_out, n_in, Mk, n_in)) != hipSuccess) return e;
        if ((e = to_act(dy, n_out, dact)) != hipSuccess) return e;
        if ((e = tr(wptr(m, widx), true, n_in, n_out, n_in, wT, n_out, n_out)) != hipSuccess) return e;
        return gemm_nt(dact, Mp, wT, pad(n_in), dx_out, M, n_in, n_out, n_in);
    };
    if (bf && Mk > M) {
        // rows M .. Mk-1 of the M-major operands: zero (the reductions run over Mk rows)
        const size_t pr = (size_t)(Mk - M);
        // (k-blocked: those rows of every 32-column block)
        auto zero_rows = [&](char* p, int n) {
            if (x_kb)
                return hipMemset2DAsync(p + (size_t)M * 64, (size_t)Mp * 64, 0, pr * 64, (size_t)n / 32, s);
            return hipMemsetAsync(p + (size_t)M * n * 2, 0, pr * n * 2, s);
        };
        for (int l = 0; l < c.n_layer; ++l) {
            GPT2_HIP(zero_rows(lay(l, L.l_a1), d));
            GPT2_HIP(hipMemsetAsync(lay(l, L.l_o) + (size_t)M * d * 2, 0, pr * d * 2, s));
            GPT2_HIP(zero_rows(lay(l, L.l_a2), d));
            GPT2_HIP(zero_rows(lay(l, L.l_h), f));
        }
        GPT2_HIP(hipMemsetAsync(ws + L.xf + (size_t)M * d * 2, 0, pr * d * 2, s));
        GPT2_HIP(hipMemsetAsync(ws + L.dlog + (size_t)M * Vp * 2, 0, pr * Vp * 2, s));
    }
    // lm_head: dxf = dlogits wte, dwte (head part) = dlogits^T xf
    if (bf) {
        const uint16_t* dl16 = reinterpret_cast<const uint16_t*>(ws + L.dlog);
        // wte [V rows, zero-padded past V][d], reduced over its rows (Vp of them)
        GPT2_HIP(gpt2k::gemm_bf16_tn(dl16, false, Vp, Mp, static_cast<const uint16_t*>(wptr(m, 0)), true, d, d, dbuf, d,
                                     M, d, Vp, s, splitk, L.splitk_elems));
        GPT2_HIP(gpt2k::gemm_bf16_tn(dl16, true, Vp, Vp, reinterpret_cast<const uint16_t*>(ws + L.xf), true, d, d, G(0),
                                     d, V, d, Mk, s));
    } else {
        GPT2_HIP(tr(wptr(m, 0), true, d, V, d, ws + L.wteT, Vp, Vp));
        GPT2_HIP(gemm_nt(ws + L.dlog, Mp, ws + L.wteT, pad(d), dbuf, M, d, Vp, d));
        GPT2_HIP(tr(ws + L.dlog, true, Vp, M, Vp, ws + L.dlogT, Mk, Mk));
        GPT2_HIP(tr(ws + L.xf, true, d, M, d, xT, Mk, Mk));
        GPT2_HIP(gemm_nt(ws + L.dlogT, (int)L.Vr, xT, pad(d), G(0), V, d, Mk, d));
    }
    GPT2_HIP(hipMemsetAsync(dx, 0, (size_t)M * d * 4, s));
    // bf16: each LayerNorm backward also writes the next projection's bf16 output gradient (dact, row
    // stride d) and that projection's bias partial sums (nbl rows at bp_ln); rows M .. Mk-1 stay zero
    // (the weight gradients reduce over Mk rows)
    uint16_t* dact16 = reinterpret_cast<uint16_t*>(dact);
    const int nbl = gpt2k::ln_backward_blocks(M);
    float* bp_ln = nullptr;
    auto take_ln_part = [&]() {
        bp_ln = bpart;
        bpart += (size_t)nbl * d;
        return bp_ln;
    };
    auto zero_dact_tail = [&]() {
        return Mk > M ? hipMemsetAsync(dact16 + (size_t)M * d, 0, (size_t)(Mk - M) * d * 2, s) : hipSuccess;
    };
    const int ln_f = 2 + c.n_layer * PER_LAYER;
    if (bf) GPT2_HIP(zero_dact_tail());
    GPT2_HIP(gpt2k::ln_backward(reinterpret_cast<float*>(ws + L.xfin), static_cast<const float*>(wptr(m, ln_f)), dbuf, dx,
                                M, d, c.ln_eps, lnpg, lnpb, G(ln_f), G(ln_f + 1), s, bf ? dact16 : nullptr,
                                bf ? take_ln_part() : nullptr));
    for (int l = c.n_layer - 1; l >= 0; --l) {
        auto I = [&](int t) { return layer_idx(l, t); };
        auto vecp = [&](int t) { return static_cast<const float*>(wptr(m, I(t))); };
        // MLP projection, GELU, c_fc, ln_2
        const float* u = reinterpret_cast<const float*>(lay(l, L.l_u));
        if (bf) {
            // mlp.c_proj's output gradient: dact from the LayerNorm backward above; its input gradient
            // goes through the GELU backward in its epilogue, which writes c_fc's bf16 output gradient
            // and its bias partial sums
            float* bp_fc = bpart;
            bpart += (size_t)nbp * f;
            gpt2k::TnGeluBack gb;
            gb.u = u;
            gb.ldu = f;
            gb.y = reinterpret_cast<uint16_t*>(ws + L.dact2);
            gb.ldy = f;
            gb.part = bp_fc;
            gb.erf = c.gelu == GPT2_GELU_ERF;
            GPT2_HIP(linear_back16(dact16, bp_ln, nbl, d, lay(l, L.l_h), f, x_kb, I(MPROJ_W), nullptr, &gb));
            GPT2_HIP(linear_back16(gb.y, bp_fc, nbp, f, lay(l, L.l_a2), d, x_kb, I(FC_W), dbuf2, nullptr));
        } else {
            GPT2_HIP(linear_back(dx, d, lay(l, L.l_h), f, false, I(MPROJ_W), dbuf));
            GPT2_HIP(gpt2k::gelu_backward(u, dbuf, (long)M * f, c.gelu == GPT2_GELU_ERF, s));
            GPT2_HIP(linear_back(dbuf, f, lay(l, L.l_a2), d, false, I(FC_W), dbuf2));
        }
        if (bf) GPT2_HIP(zero_dact_tail());
        GPT2_HIP(gpt2k::ln_backward(reinterpret_cast<const float*>(lay(l, L.l_xmid)), vecp(LN2_W), dbuf2, dx, M, d,
                                    c.ln_eps, lnpg, lnpb, G(I(LN2_W)), G(I(LN2_B)), s, bf ? dact16 : nullptr,
                                    bf ? take_ln_part() : nullptr));
        // attention projection, attention, c_attn, ln_1
        if (bf)
            GPT2_HIP(linear_back16(dact16, bp_ln, nbl, d, lay(l, L.l_o), d, false, I(APROJ_W), dbuf, nullptr));
        else
            GPT2_HIP(linear_back(dx, d, lay(l, L.l_o), d, false, I(APROJ_W), dbuf));
        float* lse = reinterpret_cast<float*>(bf ? lay(l, L.l_lse) : ws + L.lse);  // bf16: written by the forward
        if (bf) {
            // the attention backward writes c_attn's bf16 output gradient and its bias partial sums
            const int nba = gpt2k::attention_backward_parts(B, T);
            if (Mk > M) GPT2_HIP(hipMemsetAsync(dact16 + (size_t)M * 3 * d, 0, (size_t)(Mk - M) * 3 * d * 2, s));
            float* bp_attn = bpart;
            bpart += (size_t)nba * 3 * d;
            GPT2_HIP(gpt2k::attention_backward_bf16(reinterpret_cast<const uint16_t*>(lay(l, L.l_qkv)),
                                                    reinterpret_cast<const uint16_t*>(lay(l, L.l_o)), dbuf, dact16,
                                                    bp_attn, lse, reinterpret_cast<float*>(ws + L.dvec), B, H, T, s));
            GPT2_HIP(linear_back16(dact16, bp_attn, nba, 3 * d, lay(l, L.l_a1), d, x_kb, I(ATTN_W), dbuf, nullptr));
        } else {
            GPT2_HIP(gpt2k::attention_backward(lay(l, L.l_qkv), lay(l, L.l_o), dbuf, dbuf2, lse,
                                               reinterpret_cast<float*>(ws + L.dvec), B, H, T, false, s));
            GPT2_HIP(linear_back(dbuf2, 3 * d, lay(l, L.l_a1), d, x_kb, I(ATTN_W), dbuf));
        }
        // (the layer below's mlp.c_proj output gradient; none below the first layer)
        const bool next16 = bf && l > 0;
        if (next16) GPT2_HIP(zero_dact_tail());
        GPT2_HIP(gpt2k::ln_backward(reinterpret_cast<const float*>(lay(l, L.l_xin)), vecp(LN1_W), dbuf, dx, M, d,
                                    c.ln_eps, lnpg, lnpb, G(I(LN1_W)), G(I(LN1_B)), s, next16 ? dact16 : nullptr,
                                    next16 ? take_ln_part() : nullptr));
    }
    // every bias gradient, kColsumSegs segments per launch
    for (size_t i0 = 0; i0 < bsegs.size(); i0 += gpt2k::kColsumSegs) {
        gpt2k::ColsumSegs part_segs;
        for (size_t i = i0; i < std::min(bsegs.size(), i0 + gpt2k::kColsumSegs); ++i) part_segs.seg[part_segs.n++] = bsegs[i];
        GPT2_HIP(gpt2k::colsum_reduce_multi(part_segs, s));
    }
    GPT2_HIP(gpt2k::embed_backward(tokens, dx, B, T, c.n_ctx, d, V, G(0), G(1), s));
    return GPT2_OK;
}

}  // namespace

// ------------------------------------------------------------------ fixed scratch (no allocation)
// Workspace of gpt2_forward_noalloc: a file-scope device array, one copy per GPU the library runs
// on, held until the process ends. Host code never passes the array's name to a kernel or a copy
// (on the host it is only a stand-in for the symbol): its device address is looked up once per
// device with hipGetSymbolAddress and kept in scratch_addr.
constexpr size_t kScratchBytes = (size_t)80 << 20;  // 80 MiB: GPT-2 small up to B*T = 4096 rows
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

// Device address of this device's scratch array for work enqueued on stream s (looked up on the
// first call for that device, with the device current).
gpt2_status scratch_for(hipStream_t s, char** out) {
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return GPT2_EHIP;
    dev = cur;
    if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return GPT2_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GPT2_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GPT2_EHIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return GPT2_EHIP;
        if (e != hipSuccess || !p) return GPT2_EHIP;
        scratch_addr[dev] = p;
    }
    *out = static_cast<char*>(scratch_addr[dev]);
    return GPT2_OK;
}
}  // namespace

extern "C" {

gpt2_status gpt2_config(const gpt2_config_t* cfg, gpt2_model** out) {
    if (!cfg || !out) return GPT2_EINVAL;
    *out = nullptr;
    const gpt2_config_t& c = *cfg;
    if (c.dtype != GPT2_F32 && c.dtype != GPT2_BF16) return GPT2_EINVAL;
    if (c.gelu != GPT2_GELU_TANH && c.gelu != GPT2_GELU_ERF) return GPT2_EINVAL;
    if (!(c.ln_eps > 0.f)) return GPT2_EINVAL;
    if (c.n_vocab < 1 || c.n_ctx < 1 || c.d_model < 1 || c.n_head < 1 || c.n_layer < 1 || c.d_mlp < 1)
        return GPT2_ESHAPE;
    if (c.d_model % c.n_head != 0 || c.d_model / c.n_head != 64) return GPT2_ESHAPE;
    if (c.d_model % 64 != 0 || c.d_mlp % 64 != 0 || c.d_model > 4096 || c.n_ctx > 65536) return GPT2_ESHAPE;
    gpt2_model* m = new (std::nothrow) gpt2_model();
    if (!m) return GPT2_EINVAL;
    m->cfg = c;
    build_layout(m);
    *out = m;
    return GPT2_OK;
}

void gpt2_destroy(gpt2_model* m) { delete m; }

int32_t gpt2_n_tensors(const gpt2_model* m) { return m ? (int32_t)m->slots.size() : 0; }

gpt2_status gpt2_tensor_shape(const gpt2_model* m, int32_t i, int64_t* rows, int64_t* cols) {
    if (!m || !rows || !cols) return GPT2_EINVAL;
    if (i < 0 || i >= (int32_t)m->slots.size()) return GPT2_EINVAL;
    *rows = m->slots[i].rows;
    *cols = m->slots[i].cols;
    return GPT2_OK;
}

size_t gpt2_weight_bytes(const gpt2_model* m) { return m ? m->weight_bytes : 0; }

size_t gpt2_workspace_bytes(const gpt2_model* m, int32_t B, int32_t T) {
    if (!m || B < 1 || T < 1 || T > m->cfg.n_ctx || (int64_t)B * T > (int64_t)1 << 24) return 0;
    return ws_layout(m, B, T).total;
}

gpt2_status gpt2_load_weights(gpt2_model* m, const void* const* src, int32_t n_src, int32_t src_dtype, void* dst,
                              size_t dst_bytes, hipStream_t stream) {
    if (!m || !src || !dst) return GPT2_EINVAL;
    if (n_src != (int32_t)m->slots.size()) return GPT2_EINVAL;
    if (src_dtype != GPT2_F32 && src_dtype != GPT2_BF16) return GPT2_EINVAL;
    if (reinterpret_cast<uintptr_t>(dst) % kAlign) return GPT2_EINVAL;
    if (dst_bytes < m->weight_bytes) return GPT2_EWORKSPACE;
    for (int i = 0; i < n_src; ++i)
        if (!src[i]) return GPT2_EINVAL;
    const bool sb = src_dtype == GPT2_BF16;
    for (int i = 0; i < n_src; ++i) {
        const TensorSlot& s = m->slots[i];
        char* d = static_cast<char*>(dst) + s.offset;
        if (s.matrix) {
            const long n = (long)s.rows * s.cols, np = (long)s.rows_padded * s.cols;
            GPT2_HIP(gpt2k::convert(src[i], sb, d, is_bf16(m), n, np, stream));
            if (m->kb_offset[i])
                GPT2_HIP(gpt2k::kblock_bf16(reinterpret_cast<const uint16_t*>(d),
                                            reinterpret_cast<uint16_t*>(static_cast<char*>(dst) + m->kb_offset[i]),
                                            s.rows_padded, (int)s.cols, stream));
        } else {
            GPT2_HIP(gpt2k::convert(src[i], sb, d, false, s.rows, s.rows, stream));
        }
    }
    m->weights = dst;
    m->loaded = true;
    return GPT2_OK;
}

gpt2_status gpt2_forward(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, float* logits,
                         int32_t* argmax, void* ws_dev, size_t ws_bytes, hipStream_t s) {
    const gpt2_status st = check_run_args(m, tokens, B, T, logits, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    Sequencer q{s};
    return enqueue_forward(m, tokens, B, T, logits, argmax, static_cast<char*>(ws_dev), q);
}

gpt2_status gpt2_forward_noalloc(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, float* logits,
                                 int32_t* argmax, hipStream_t s) {
    if (!m || !tokens || !logits) return GPT2_EINVAL;
    if (!m->loaded) return GPT2_ESTATE;
    if (B < 1 || T < 1 || T > m->cfg.n_ctx) return GPT2_ESHAPE;
    if ((int64_t)B * T > (int64_t)1 << 24 || ws_layout(m, B, T).total > kScratchBytes) return GPT2_EWORKSPACE;
    char* ws = nullptr;
    const gpt2_status st = scratch_for(s, &ws);
    if (st != GPT2_OK) return st;
    // every workspace buffer of the forward is written before it is read (the residual by the
    // embedding, the head partials and token flags by their producers), so nothing is cleared
    Sequencer q{s};
    return enqueue_forward(m, tokens, B, T, logits, argmax, ws, q);
}

gpt2_status gpt2_forward_loss(const gpt2_model* m, const int32_t* tokens, const int32_t* labels, int32_t B, int32_t T,
                              float* nll, float* loss, void* ws_dev, size_t ws_bytes, hipStream_t s) {
    gpt2_status st = check_run_args(m, tokens, B, T, nll, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    if (!loss) return GPT2_EINVAL;
    if (T < 2) return GPT2_ESHAPE;
    Sequencer q{s};
    return enqueue_forward_loss(m, tokens, labels, B, T, nll, loss, static_cast<char*>(ws_dev), q);
}

size_t gpt2_kv_cache_bytes(const gpt2_model* m, int32_t B) {
    if (!m || B < 1 || (int64_t)B * m->cfg.n_ctx > (int64_t)1 << 30) return 0;
    return kv_cache_bytes(m, B);
}

gpt2_status gpt2_prefill(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, void* cache,
                         size_t cache_bytes, float* logits, int32_t* next, void* ws_dev, size_t ws_bytes, hipStream_t s) {
    gpt2_status st = check_run_args(m, tokens, B, T, cache, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    if ((st = check_cache(m, B, cache, cache_bytes)) != GPT2_OK) return st;
    char* ws = static_cast<char*>(ws_dev);
    const WorkspaceLayout w = ws_layout(m, B, T);
    Sequencer q{s};
    KVArgs kv;
    kv.cache = static_cast<char*>(cache);
    st = enqueue_trunk(m, tokens, B, T, m->cfg.n_layer, ws, w, q, kv);
    if (st != GPT2_OK) return st;
    if (!logits && !next) return GPT2_OK;
    float* xl = reinterpret_cast<float*>(ws + w.xl);
    GPT2_RUN(GPT2_K_LN_F, gpt2k::gather_last_rows(reinterpret_cast<const float*>(ws + w.x), xl, B, T, m->cfg.d_model, s));
    return enqueue_next_token(m, xl, B, logits, next, ws, w, q);
}

gpt2_status gpt2_decode_step(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t pos, void* cache,
                             size_t cache_bytes, float* logits, int32_t* next, void* ws_dev, size_t ws_bytes,
                             hipStream_t s) {
    gpt2_status st = check_run_args(m, tokens, B, 1, cache, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    if ((st = check_cache(m, B, cache, cache_bytes)) != GPT2_OK) return st;
    if (pos < 0 || pos >= m->cfg.n_ctx) return GPT2_ESHAPE;
    char* ws = static_cast<char*>(ws_dev);
    const WorkspaceLayout w = ws_layout(m, B, 1);
    Sequencer q{s};
    KVArgs kv;
    kv.cache = static_cast<char*>(cache);
    kv.pos0 = pos;
    kv.from_cache = true;
    st = enqueue_trunk(m, tokens, B, 1, m->cfg.n_layer, ws, w, q, kv);
    if (st != GPT2_OK) return st;
    if (!logits && !next) return GPT2_OK;
    return enqueue_next_token(m, reinterpret_cast<const float*>(ws + w.x), B, logits, next, ws, w, q);
}

gpt2_status gpt2_forward_timed(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, float* logits,
                               int32_t* argmax, void* ws_dev, size_t ws_bytes, hipStream_t s, hipEvent_t* ev_before,
                               hipEvent_t* ev_after, int32_t n_slots) {
    const gpt2_status st = check_run_args(m, tokens, B, T, logits, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    if (n_slots < 0) return GPT2_EINVAL;
    Sequencer q{s};
    q.before = ev_before;
    q.after = ev_after;
    q.n_slots = n_slots;
    return enqueue_forward(m, tokens, B, T, logits, argmax, static_cast<char*>(ws_dev), q);
}

gpt2_status gpt2_forward_repeat(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, float* logits,
                                int32_t* argmax, void* ws_dev, size_t ws_bytes, hipStream_t s, int32_t launch,
                                int32_t repeats, hipEvent_t ev_before, hipEvent_t ev_after) {
    const gpt2_status st = check_run_args(m, tokens, B, T, logits, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    if (launch < 0 || launch >= gpt2_forward_launches(m, B, T, argmax != nullptr, nullptr, 0) || repeats < 1)
        return GPT2_EINVAL;
    Sequencer q{s};
    q.rep_idx = launch;
    q.rep_n = repeats;
    q.rep_before = ev_before;
    q.rep_after = ev_after;
    return enqueue_forward(m, tokens, B, T, logits, argmax, static_cast<char*>(ws_dev), q);
}

int32_t gpt2_forward_launches(const gpt2_model* m, int32_t B, int32_t T, int32_t with_argmax, int32_t* kinds,
                              int32_t cap) {
    if (!m || B < 1 || T < 1 || T > m->cfg.n_ctx) return 0;
    Sequencer q{nullptr};
    q.dry = true;
    q.kinds = kinds;
    q.cap = kinds ? cap : 0;
    // a dry run touches no memory: the pointers only need to be non-null where the path branches
    int32_t dummy = 0;
    if (enqueue_forward(m, &dummy, B, T, nullptr, with_argmax ? &dummy : nullptr, nullptr, q) != GPT2_OK) return 0;
    return q.idx;
}

gpt2_status gpt2_forward_debug(const gpt2_model* m, const int32_t* tokens, int32_t B, int32_t T, int32_t n_layers,
                               float* resid, void* ws_dev, size_t ws_bytes, hipStream_t s) {
    gpt2_status st = check_run_args(m, tokens, B, T, resid, ws_dev, ws_bytes);
    if (st != GPT2_OK) return st;
    if (n_layers < 0 || n_layers > m->cfg.n_layer) return GPT2_EINVAL;
    char* ws = static_cast<char*>(ws_dev);
    const WorkspaceLayout w = ws_layout(m, B, T);
    Sequencer q{s};
    st = enqueue_trunk(m, tokens, B, T, n_layers, ws, w, q);
    if (st != GPT2_OK) return st;
    GPT2_HIP(hipMemcpyAsync(resid, ws + w.x, (size_t)B * T * m->cfg.d_model * 4, hipMemcpyDeviceToDevice, s));
    return GPT2_OK;
}

gpt2_status gpt2_check(const gpt2_model* m, const void* ws_dev, int32_t B, int32_t T, hipStream_t s) {
    if (!m || !ws_dev) return GPT2_EINVAL;
    if (B < 1 || T < 1 || T > m->cfg.n_ctx) return GPT2_ESHAPE;
    const WorkspaceLayout w = ws_layout(m, B, T);
    const int n = gpt2k::embed_flag_count(B * T);
    std::vector<int32_t> flags(n);
    GPT2_HIP(hipStreamSynchronize(s));
    GPT2_HIP(hipMemcpy(flags.data(), static_cast<const char*>(ws_dev) + w.flags, n * sizeof(int32_t),
                       hipMemcpyDeviceToHost));
    for (int i = 0; i < n; ++i)
        if (flags[i]) return GPT2_ETOKEN;
    return GPT2_OK;
}

gpt2_status gpt2_attention(const void* q, const int64_t* qs, const void* k, const int64_t* ks, const void* v,
                           const int64_t* vs, void* o, const int64_t* os, int32_t B, int32_t H, int32_t T, int32_t dh,
                           int32_t dtype, hipStream_t s) {
    if (!q || !k || !v || !o || !qs || !ks || !vs || !os) return GPT2_EINVAL;
    if (dtype != GPT2_F32 && dtype != GPT2_BF16) return GPT2_EINVAL;
    if (dh != 64 || B < 1 || H < 1 || T < 1) return GPT2_ESHAPE;
    if ((int64_t)B * H * ((T + 127) / 128) > 0x7fffffff) return GPT2_ESHAPE;
    for (const int64_t* st : {qs, ks, vs, os})
        for (int i = 0; i < 3; ++i)
            if (st[i] < 0 || st[i] % 8) return GPT2_EINVAL;
    for (const void* p : {q, k, v, static_cast<const void*>(o)})
        if (reinterpret_cast<uintptr_t>(p) % 16) return GPT2_EINVAL;
    if (dtype == GPT2_BF16)
        GPT2_HIP(gpt2k::attention_bf16(static_cast<const uint16_t*>(q), qs, static_cast<const uint16_t*>(k), ks,
                                       static_cast<const uint16_t*>(v), vs, static_cast<uint16_t*>(o), os, B, H, T, s));
    else
        GPT2_HIP(gpt2k::attention_f32(static_cast<const float*>(q), qs, static_cast<const float*>(k), ks,
                                      static_cast<const float*>(v), vs, static_cast<float*>(o), os, B, H, T, s));
    return GPT2_OK;
}

gpt2_status gpt2_layernorm(const float* x, const float* g, const float* b, void* y, int32_t M, int32_t n, float eps,
                           int32_t out_dtype, hipStream_t s) {
    if (!x || !g || !b || !y) return GPT2_EINVAL;
    if (out_dtype != GPT2_F32 && out_dtype != GPT2_BF16) return GPT2_EINVAL;
    if (M < 1 || n < 4 || n % 4 || n > 4096) return GPT2_ESHAPE;
    if (!(eps > 0.f)) return GPT2_EINVAL;
    GPT2_HIP(gpt2k::layernorm(x, g, b, y, M, n, eps, out_dtype == GPT2_BF16, s));
    return GPT2_OK;
}

gpt2_status gpt2_linear(const void* A, const void* W, const float* bias, void* C, int32_t M, int32_t N, int32_t K,
                        int64_t ldc, int32_t dtype, int32_t epi, int32_t gelu, hipStream_t s) {
    if (!A || !W || !C) return GPT2_EINVAL;
    if (dtype != GPT2_F32 && dtype != GPT2_BF16) return GPT2_EINVAL;
    if (epi < GPT2_EPI_BIAS || epi > GPT2_EPI_LOGITS) return GPT2_EINVAL;
    if (gelu != GPT2_GELU_TANH && gelu != GPT2_GELU_ERF) return GPT2_EINVAL;
    if (epi != GPT2_EPI_LOGITS && !bias) return GPT2_EINVAL;
    if (M < 1 || N < 1 || K < 64 || K % 64 || ldc < N) return GPT2_ESHAPE;
    const int ge = gelu == GPT2_GELU_ERF;
    if (dtype == GPT2_BF16)
        GPT2_HIP(gpt2k::gemm_bf16(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W), bias, C, M, N, K, ldc,
                                  epi, ge, (int)round_up(M, kRowPad), (int)round_up(N, kRowPad), {}, s));
    else
        GPT2_HIP(gpt2k::gemm_f32(static_cast<const float*>(A), static_cast<const float*>(W), bias, C, M, N, K, ldc, epi,
                                 ge, {}, s));
    return GPT2_OK;
}

size_t gpt2_sample_workspace_bytes(int32_t B, int32_t V) {
    if (B < 1 || V < 1 || V > gpt2k::sample_max_vocab()) return 0;
    return gpt2k::sample_workspace_bytes(B, V);
}

gpt2_status gpt2_sample(const float* logits, int64_t ld, int32_t B, int32_t V, const int32_t* hist, int64_t hist_ld,
                        int32_t n_hist, float temperature, int32_t top_k, float top_p, float penalty, const float* u,
                        int32_t* out, int32_t* n_kept, void* ws, size_t ws_bytes, hipStream_t s) {
    if (!logits || !u || !out) return GPT2_EINVAL;
    if (B < 1 || V < 1 || V > gpt2k::sample_max_vocab() || ld < V) return GPT2_ESHAPE;
    if (n_hist < 0 || (n_hist > 0 && (!hist || hist_ld < n_hist))) return GPT2_EINVAL;
    if (!(temperature > 0.f) || !(temperature < INFINITY)) return GPT2_EINVAL;
    if (top_k < 0 || !(top_p > 0.f) || !(top_p <= 1.f)) return GPT2_EINVAL;
    if (!(penalty > 0.f) || !(penalty < INFINITY)) return GPT2_EINVAL;
    if (ws && (reinterpret_cast<uintptr_t>(ws) % 256)) return GPT2_EINVAL;
    if (ws && ws_bytes < gpt2k::sample_workspace_bytes(B, V)) return GPT2_EWORKSPACE;
    GPT2_HIP(gpt2k::sample(logits, ld, B, V, n_hist > 0 ? hist : nullptr, hist_ld, n_hist, temperature, top_k, top_p,
                           penalty, u, out, n_kept, ws, ws_bytes, s));
    return GPT2_OK;
}

size_t gpt2_grad_bytes(const gpt2_model* m) { return m ? grad_offset(m, (int)m->slots.size()) : 0; }

size_t gpt2_grad_offset(const gpt2_model* m, int32_t i) {
    if (!m || i < 0 || i >= (int)m->slots.size()) return (size_t)-1;
    return grad_offset(m, i);
}

size_t gpt2_train_workspace_bytes(const gpt2_model* m, int32_t B, int32_t T) {
    if (!m || B < 1 || T < 2 || T > m->cfg.n_ctx) return 0;
    return train_layout(m, B, T).total;
}

gpt2_status gpt2_backward(const gpt2_model* m, const int32_t* tokens, const int32_t* labels, int32_t B, int32_t T,
                          float* grads, size_t grads_bytes, float* loss, void* ws, size_t ws_bytes, hipStream_t s) {
    if (!m || !tokens || !grads || !loss || !ws) return GPT2_EINVAL;
    if (!m->loaded) return GPT2_ESTATE;
    if (B < 1 || T < 2 || T > m->cfg.n_ctx || (int64_t)B * T > (int64_t)1 << 20) return GPT2_ESHAPE;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign || reinterpret_cast<uintptr_t>(grads) % kAlign) return GPT2_EINVAL;
    const TrainLayout L = train_layout(m, B, T);
    if (ws_bytes < L.total || grads_bytes < grad_offset(m, (int)m->slots.size())) return GPT2_EWORKSPACE;
    char* w = static_cast<char*>(ws);
    gpt2_status st = enqueue_train_forward(m, tokens, labels, B, T, loss, w, L, s);
    if (st != GPT2_OK) return st;
    return enqueue_backward(m, tokens, B, T, grads, w, L, s);
}

const char* gpt2_strerror(gpt2_status s) {
    switch (s) {
        case GPT2_OK: return "ok";
        case GPT2_EINVAL: return "invalid argument";
        case GPT2_ESHAPE: return "unsupported or inconsistent shape";
        case GPT2_EWORKSPACE: return "buffer smaller than required";
        case GPT2_ETOKEN: return "token id (or label) outside [0, n_vocab)";
        case GPT2_EHIP: return "HIP runtime error";
        case GPT2_ESTATE: return "call made in the wrong state";
    }
    return "unknown status";
}

}  // extern "C"
