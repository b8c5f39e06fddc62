"""CPU float64 oracle of the GPT-2 decoder forward pass.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this module. The product path (the HIP library and its Python binding) never
imports, calls or falls back to it, and this module imports nothing from the product path: it
depends on numpy alone and receives its inputs as plain arrays.

Every function is the plain definition of one step, written out in float64 with numpy (matmul
is the only library primitive used as a step). Nothing is blocked, fused or reordered beyond
what the definition states, so each function can be checked against the pages by eye.

Pages cited (titles as they appear on the pages):
  [手写] "从零手写GPT-2：PyTorch实现Transformer解码器核心模块"
  [实战] "GPT2模型开发实战：从原理到部署全解析"
  [解析] "GPT-2模型架构解析与实现指南"
  [复现] "复现GPT-2 124M"
  [指南] "从零实现 GPT-2：PyTorch 版大语言模型构建指南"

Readings taken where the pages are silent or disagree (each one also recorded in the design
notes): learned wpe table; GELU in its tanh form; biases present on all four block Linears and
absent on lm_head; causal mask keeps the diagonal (key j visible to query i iff j <= i); scale
1/sqrt(d_head) applied before the mask; biased variance with eps 1e-5 inside the square root;
dropout is the identity (inference forward); q, k, v are the column blocks [0,d), [d,2d), [2d,3d)
of the fused projection and head h owns columns h*dh .. (h+1)*dh-1 within each block.

Parity pins: every function below is pinned by a CPU test against values the mathematics or
the pages fix (closed forms, brute force on tiny inputs, library special cases, invariants).
The whole-model logits at random init are "parity unpinned" beyond those component pins and the
model-level invariants (shape, parameter count, causality, batch independence, all-ones MLP):
the pages print no logits for any input.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def embed(wte: np.ndarray, wpe: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Token embedding plus learned position embedding.

    x[b, t, :] = wte[tokens[b, t], :] + wpe[t, :] with positions counted from 0
    ([手写] §4.1 forward, steps 1; [复现] §2.1 learned position table; [解析] §1.2).
    Dropout after the sum is the identity in the inference forward.
    """
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    wte = np.asarray(wte, dtype=F64)
    wpe = np.asarray(wpe, dtype=F64)
    return wte[tokens] + wpe[np.arange(T)][None, :, :]


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance.

    mean = E[x]; var = E[(x - mean)^2] (no Bessel correction); out = gamma * (x - mean) /
    sqrt(var + eps) + beta ([复现] §2.1 LayerNorm class, unbiased=False; eps 1e-5 per [手写] §3.2
    and §4.2).
    """
    x = np.asarray(x, dtype=F64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return np.asarray(gamma, F64) * (x - mean) / np.sqrt(var + eps) + np.asarray(beta, F64)


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray | None) -> np.ndarray:
    """nn.Linear semantics: y = x W^T + b with W stored [out, in] (all pages' code listings)."""
    y = np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T
    if b is not None:
        y = y + np.asarray(b, dtype=F64)
    return y


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).

    [复现] §2.4 names this form as the one original GPT-2 used; [手写] §3.4 prints the same
    formula.
    """
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gelu_erf(x: np.ndarray) -> np.ndarray:
    """GELU, erf form 0.5 x (1 + erf(x / sqrt(2))) (the F.gelu default used by [解析] §2.2).

    Kept only for the optional erf configuration; the default reading is the tanh form.
    """
    from math import erf
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + np.vectorize(erf)(x / math.sqrt(2.0)))


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Row softmax with the row maximum subtracted first (exact in float64; -inf gives 0)."""
    s = np.asarray(s, dtype=F64)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Causal scaled dot-product attention per (batch, head); inputs [..., T, dh].

    S = q k^T / sqrt(dh); S[i, j] = -inf for j > i (diagonal kept); P = softmax over keys;
    out = P v ([复现] §2.1 CausalSelfAttention and §2.2; [解析] §2.1; [手写] §3.3: the mask goes
    after the scores and before the softmax). The [T, T] score matrix is materialised on purpose.
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    T, dh = q.shape[-2], q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) * (1.0 / math.sqrt(dh))
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    return softmax(s, axis=-1) @ v


def split_heads(qkv: np.ndarray, n_head: int):
    """[B, T, 3d] -> q, k, v each [B, H, T, dh]: split by d, view (B, T, H, dh), swap T and H.

    ([复现] §2.1 forward: split(n_embd) then view/transpose; [解析] §2.1 reshape(B, T, 3, H, dh).)
    """
    B, T, three_d = qkv.shape
    d = three_d // 3
    dh = d // n_head
    q, k, v = qkv[..., 0:d], qkv[..., d:2 * d], qkv[..., 2 * d:3 * d]
    return tuple(t.reshape(B, T, n_head, dh).transpose(0, 2, 1, 3) for t in (q, k, v))


def merge_heads(o: np.ndarray) -> np.ndarray:
    """[B, H, T, dh] -> [B, T, H*dh] (transpose back, then view)."""
    B, H, T, dh = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, T, H * dh)


def exact(a: np.ndarray) -> np.ndarray:
    """Activations kept exact (float64): the default storage of every intermediate."""
    return a


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Each value rounded to the nearest bfloat16 (8 significant bits, ties to even), as float64.

    bfloat16 keeps fp32's exponent range and 8 significant bits, so a value x = m * 2^e with
    m in [0.5, 1) lies on the grid of spacing 2^(e - 8); np.round rounds halves to even. Used only
    for forward_bf16_activations (values here are far from the subnormal and overflow ranges)."""
    a = np.asarray(a, dtype=F64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, e - 8)
    return np.round(a / step) * step


def attention_block(x: np.ndarray, p: dict, l: int, n_head: int, act=exact) -> np.ndarray:
    """Self-attention sub-layer of block l on its LayerNorm'd input: c_attn, heads, c_proj.
    act stores the fused projection's output and the merged head outputs (identity by default)."""
    pre = f"h.{l}.attn."
    qkv = act(linear(x, p[pre + "c_attn.w"], p[pre + "c_attn.b"]))
    q, k, v = split_heads(qkv, n_head)
    o = act(merge_heads(causal_attention(q, k, v)))
    return linear(o, p[pre + "c_proj.w"], p[pre + "c_proj.b"])


def mlp_block(x: np.ndarray, p: dict, l: int, gelu=gelu_tanh, act=exact) -> np.ndarray:
    """MLP sub-layer: c_fc (d -> d_mlp), GELU, c_proj (d_mlp -> d) ([解析] §2.2; [复现] §2.4).
    act stores the GELU output (identity by default)."""
    pre = f"h.{l}.mlp."
    return linear(act(gelu(linear(x, p[pre + "c_fc.w"], p[pre + "c_fc.b"]))),
                  p[pre + "c_proj.w"], p[pre + "c_proj.b"])


def block(x: np.ndarray, p: dict, l: int, n_head: int, eps: float = 1e-5, gelu=gelu_tanh, act=exact) -> np.ndarray:
    """Pre-LN block: x + attn(ln_1(x)), then + mlp(ln_2(x)) ([手写] §3.2; [实战] §10 and [解析] §1.1
    Block listings; [复现] §2.3). act stores the two LayerNorm outputs (identity by default); the
    residual stream x itself is never passed through it."""
    pre = f"h.{l}."
    x = x + attention_block(act(layer_norm(x, p[pre + "ln_1.w"], p[pre + "ln_1.b"], eps)), p, l, n_head, act)
    x = x + mlp_block(act(layer_norm(x, p[pre + "ln_2.w"], p[pre + "ln_2.b"], eps)), p, l, gelu, act)
    return x


def residual(p: dict, tokens: np.ndarray, n_head: int, n_layers: int, eps: float = 1e-5,
             gelu=gelu_tanh, act=exact) -> np.ndarray:
    """Residual stream [B, T, d] after the embedding and the first n_layers blocks."""
    x = embed(p["wte"], p["wpe"], tokens)
    for l in range(n_layers):
        x = block(x, p, l, n_head, eps, gelu, act)
    return x


def final_hidden(p: dict, tokens: np.ndarray, n_head: int, n_layer: int, eps: float = 1e-5,
                 gelu=gelu_tanh, act=exact) -> np.ndarray:
    """ln_f applied to the residual stream after all blocks ([手写] §4.1 forward, step 3)."""
    x = residual(p, tokens, n_head, n_layer, eps, gelu, act)
    return act(layer_norm(x, p["ln_f.w"], p["ln_f.b"], eps))


def lm_head(h: np.ndarray, wte: np.ndarray) -> np.ndarray:
    """Tied output projection, no bias: logits = h wte^T ([手写] §2.2 item 4 and §4.1)."""
    return linear(h, wte, None)


def forward(p: dict, tokens: np.ndarray, n_head: int, n_layer: int, eps: float = 1e-5,
            gelu=gelu_tanh, act=exact) -> np.ndarray:
    """Whole forward: tokens [B, T] -> logits [B, T, n_vocab] in float64 (every activation exact)."""
    return lm_head(final_hidden(p, tokens, n_head, n_layer, eps, gelu, act), p["wte"])


def forward_bf16_activations(p: dict, tokens: np.ndarray, n_head: int, n_layer: int, eps: float = 1e-5,
                             gelu=gelu_tanh) -> np.ndarray:
    """The forward of a model whose activations are stored in bf16 (the bf16 configuration:
    bf16 weights and activations, fp32 accumulation): the same float64 arithmetic, with the
    activations that configuration stores rounded to bf16 where they are produced -- the LayerNorm
    outputs (ln_1, ln_2, ln_f), the fused q/k/v projection, the merged attention output and the
    GELU output. The residual stream, every statistic and every sum stay exact, and the logits are
    not rounded. Used where a floating-point result decides an integer (the top-1 token), so that
    the decision is taken in the precision the configuration computes in."""
    return forward(p, tokens, n_head, n_layer, eps, gelu, act=round_bf16)


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Index of the largest entry along the last axis; the first such index on ties."""
    return np.argmax(np.asarray(logits), axis=-1)


IGNORE_INDEX = -100  # the default ignore_index of the cross-entropy loss the pages use


def log_sum_exp(logits: np.ndarray) -> np.ndarray:
    """log(sum_v exp(logits[..., v])) along the last axis, with the row maximum subtracted first."""
    z = np.asarray(logits, dtype=F64)
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def shifted_nll(logits: np.ndarray, labels: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Next-token negative log-likelihood as in [手写] §4.1: the logits of positions 0..T-2 are
    scored against the labels of positions 1..T-1, nll = logsumexp(logits) - logits[label].

    logits [B, T, V], labels int [B, T]. Returns (nll [B, T-1], counted [B, T-1] bool): positions
    whose label is the ignore index are not counted and get nll 0."""
    z = np.asarray(logits, dtype=F64)[:, :-1, :]
    y = np.asarray(labels)[:, 1:]
    counted = y != IGNORE_INDEX
    safe = np.where(counted, y, 0)
    picked = np.take_along_axis(z, safe[..., None], axis=-1)[..., 0]
    nll = np.where(counted, log_sum_exp(z) - picked, 0.0)
    return nll, counted


def shifted_cross_entropy(logits: np.ndarray, labels: np.ndarray) -> float:
    """Mean of shifted_nll over the counted positions ([手写] §4.1, mean reduction); NaN when no
    position is counted (0 / 0)."""
    nll, counted = shifted_nll(logits, labels)
    n = int(counted.sum())
    return float(nll.sum() / n) if n else float("nan")


def greedy_generate(p: dict, prompt: np.ndarray, n_new: int, n_head: int, n_layer: int, eps: float = 1e-5,
                    gelu=gelu_tanh) -> np.ndarray:
    """Greedy decoding as in [手写] §6.3: run the forward on the whole sequence so far, take the
    first-index argmax of the last position's logits as the next token, append, repeat.
    prompt int [B, T] -> int [B, T + n_new]. (No cache: each step recomputes every position.)"""
    seq = np.asarray(prompt).copy()
    for _ in range(n_new):
        nxt = argmax_first(forward(p, seq, n_head, n_layer, eps, gelu)[:, -1])
        seq = np.concatenate([seq, nxt[:, None].astype(seq.dtype)], axis=1)
    return seq


def sample_filter(logits: np.ndarray, history: np.ndarray | None = None, temperature: float = 1.0, top_k: int = 0,
                  top_p: float = 1.0, repetition_penalty: float = 1.0):
    """The logit processors of sampled decoding ([实战] §8.2: repetition penalty, temperature, top-k,
    top-p), row by row. Returns (z, keep): z [B, V] the penalised logits divided by the temperature
    and keep [B, V] the tokens that survive both cut-offs. Readings:
      * penalty: each distinct id of the row's history inside [0, V) (others ignored) has its logit
        divided by the penalty when it is positive and multiplied by it otherwise, once per id;
      * top_k = 0 or >= V keeps everything; otherwise every token whose value is at least the k-th
        largest value is kept (ties at the boundary stay);
      * top_p = 1 keeps everything; otherwise, with q the softmax over the tokens kept so far,
        token v stays when the mass of all kept tokens with value <= its own exceeds 1 - top_p
        (ties together; the largest value always stays)."""
    z = np.array(logits, dtype=F64)
    B, V = z.shape
    keep = np.ones((B, V), dtype=bool)
    for b in range(B):
        if history is not None and repetition_penalty != 1.0:
            h = np.asarray(history[b])
            ids = np.unique(h[(h >= 0) & (h < V)])
            v = z[b, ids]
            z[b, ids] = np.where(v > 0, v / repetition_penalty, v * repetition_penalty)
        z[b] = z[b] / temperature
        if 0 < top_k < V:
            kth = np.sort(z[b])[::-1][top_k - 1]
            keep[b] &= z[b] >= kth
        if top_p < 1.0:
            m = z[b][keep[b]].max()
            q = np.where(keep[b], np.exp(z[b] - m), 0.0)
            q /= q.sum()
            # mass of the kept tokens whose value is <= each token's value
            order = np.argsort(z[b], kind="stable")
            zs, qs = z[b][order], q[order]
            cum = np.cumsum(qs)
            # ties: every member of a run of equal values gets the cumulative mass at the run's end
            last = np.searchsorted(zs, zs, side="right") - 1
            below = np.empty(V)
            below[order] = cum[last]
            keep[b] &= below > 1.0 - top_p
    return z, keep


def sample_next(logits: np.ndarray, u: np.ndarray, history: np.ndarray | None = None, temperature: float = 1.0,
                top_k: int = 0, top_p: float = 1.0, repetition_penalty: float = 1.0) -> np.ndarray:
    """One sampled next token per row: the processors of sample_filter, then a multinomial draw
    from the softmax of z over the kept tokens ([解析] §4.1: softmax(logits / temperature), then a
    multinomial draw). logits [B, V]; u [B] uniform numbers in [0, 1) supplied by the caller (the
    randomness of the draw); history int [B, n] token ids seen so far or None. The draw is the
    first token, in vocabulary order, whose cumulative probability over the kept tokens exceeds u."""
    z, keep = sample_filter(logits, history, temperature, top_k, top_p, repetition_penalty)
    out = np.empty(z.shape[0], dtype=np.int64)
    for b in range(z.shape[0]):
        m = z[b][keep[b]].max()
        q = np.where(keep[b], np.exp(z[b] - m), 0.0)
        c = np.cumsum(q) / q.sum()
        idx = int(np.searchsorted(c, u[b], side="right"))  # first index with c > u
        out[b] = min(idx, int(np.nonzero(keep[b])[0][-1]))
    return out


# ------------------------------------------------------------------------------------ backward
# Gradients of the mean shifted cross-entropy ([手写] §4 training loop: loss.backward()) with
# respect to every weight. Each function is the chain rule of one forward step above, written out
# by hand in float64; the tied matrix wte collects both the lm_head gradient and the embedding
# gradient ([手写] §2.2: with weight tying the gradient of wte is the sum of the two).


def layer_norm_backward(x: np.ndarray, gamma: np.ndarray, dy: np.ndarray, eps: float = 1e-5):
    """Gradients of layer_norm (biased variance): with xhat = (x - mean) / sqrt(var + eps) and
    g = dy * gamma, dx = (g - mean(g) - xhat * mean(g * xhat)) / sqrt(var + eps); dgamma and dbeta
    are dy * xhat and dy summed over every leading axis. Returns (dx, dgamma, dbeta)."""
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    g = dy * np.asarray(gamma, F64)
    dx = rstd * (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    d = x.shape[-1]
    return dx, (dy * xhat).reshape(-1, d).sum(axis=0), dy.reshape(-1, d).sum(axis=0)


def linear_backward(x: np.ndarray, w: np.ndarray, dy: np.ndarray):
    """Gradients of y = x W^T + b: dx = dy W, dW = dy^T x (summed over every row), db = sum of dy.
    Returns (dx, dW, db)."""
    x = np.asarray(x, dtype=F64)
    w = np.asarray(w, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    n_out, n_in = w.shape
    return dy @ w, dy.reshape(-1, n_out).T @ x.reshape(-1, n_in), dy.reshape(-1, n_out).sum(axis=0)


def gelu_tanh_backward(x: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """dy * gelu'(x) for the tanh form: with c = sqrt(2/pi), z = c (x + 0.044715 x^3), t = tanh z,
    gelu'(x) = 0.5 (1 + t) + 0.5 x (1 - t^2) c (1 + 3 * 0.044715 x^2)."""
    x = np.asarray(x, dtype=F64)
    c = math.sqrt(2.0 / math.pi)
    t = np.tanh(c * (x + 0.044715 * x ** 3))
    return np.asarray(dy, F64) * (0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x))


def causal_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray):
    """Gradients of causal_attention for the output gradient do (all [..., T, dh]): with P the
    masked softmax of S = q k^T / sqrt(dh), dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
    dQ = dS K / sqrt(dh), dK = dS^T Q / sqrt(dh) (the masked entries have P = 0 and pass nothing).
    Returns (dq, dk, dv)."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    do = np.asarray(do, dtype=F64)
    T, dh = q.shape[-2], q.shape[-1]
    scale = 1.0 / math.sqrt(dh)
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    s = np.where(np.triu(np.ones((T, T), dtype=bool), k=1), -np.inf, s)
    prob = softmax(s, axis=-1)
    dv = np.swapaxes(prob, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = prob * (dp - (prob * dp).sum(axis=-1, keepdims=True))
    return (ds @ k) * scale, (np.swapaxes(ds, -1, -2) @ q) * scale, dv


def causal_attention_backward_terms(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray):
    """Magnitudes of the terms that causal_attention_backward sums, for bounding the rounding error
    of an implementation (the sum of |terms| of a dot product bounds what relative errors in its
    operands can move it). With P the masked softmax, |dP| taken as |dO| |V|^T and the row-sum term
    as rowsum(P |dP|): |dS| <= P (|dP| + rowsum(P |dP|)); then
    dq_terms = |dS| |K| / sqrt(dh), dk_terms = |dS|^T |Q| / sqrt(dh), dv_terms = P^T |dO|.
    (dQ is a sum of dS-weighted keys whose weights sum to zero, so it can be far smaller than
    these terms when the keys share a common part.) Returns (dq_terms, dk_terms, dv_terms)."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    do = np.abs(np.asarray(do, dtype=F64))
    T, dh = q.shape[-2], q.shape[-1]
    scale = 1.0 / math.sqrt(dh)
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    s = np.where(np.triu(np.ones((T, T), dtype=bool), k=1), -np.inf, s)
    prob = softmax(s, axis=-1)
    dp = do @ np.swapaxes(np.abs(v), -1, -2)
    ds = prob * (dp + (prob * dp).sum(axis=-1, keepdims=True))
    return (ds @ np.abs(k)) * scale, (np.swapaxes(ds, -1, -2) @ np.abs(q)) * scale, np.swapaxes(prob, -1, -2) @ do


def shifted_cross_entropy_backward(logits: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """Gradient of shifted_cross_entropy with respect to logits [B, T, V]: for every counted
    position (b, t < T-1), (softmax(logits[b, t]) - onehot(labels[b, t+1])) / n_counted; zero at
    the last position of each row and at ignored positions."""
    z = np.asarray(logits, dtype=F64)
    grad = np.zeros_like(z)
    _, counted = shifted_nll(z, labels)
    n = int(counted.sum())
    if n == 0:
        return grad
    y = np.asarray(labels)[:, 1:]
    g = softmax(z[:, :-1, :], axis=-1)
    b_idx, t_idx = np.nonzero(counted)
    g[b_idx, t_idx, y[b_idx, t_idx]] -= 1.0
    grad[:, :-1, :] = np.where(counted[..., None], g, 0.0) / n
    return grad


def loss_and_grads(p: dict, tokens: np.ndarray, labels: np.ndarray | None, n_head: int, n_layer: int,
                   eps: float = 1e-5, term_scales: bool = False):
    """Mean shifted cross-entropy of the forward (labels None: the tokens themselves) and its
    gradient with respect to every weight of p (same keys). The forward is the one above, step by
    step, keeping what the backward needs; the backward visits the steps in reverse.

    term_scales: also return, per weight, the magnitude its gradient is built from: the backward
    run on magnitudes (_gradient_magnitudes), the scale against which an implementation's rounding
    error in that gradient is measured. Returns (loss, grads) or (loss, grads, scales)."""
    tokens = np.asarray(tokens)
    labels = tokens if labels is None else np.asarray(labels)
    B, T = tokens.shape
    x = embed(p["wte"], p["wpe"], tokens)
    saved = []
    for l in range(n_layer):
        pre = f"h.{l}."
        a1 = layer_norm(x, p[pre + "ln_1.w"], p[pre + "ln_1.b"], eps)
        qkv = linear(a1, p[pre + "attn.c_attn.w"], p[pre + "attn.c_attn.b"])
        q, k, v = split_heads(qkv, n_head)
        o = merge_heads(causal_attention(q, k, v))
        x_mid = x + linear(o, p[pre + "attn.c_proj.w"], p[pre + "attn.c_proj.b"])
        a2 = layer_norm(x_mid, p[pre + "ln_2.w"], p[pre + "ln_2.b"], eps)
        u = linear(a2, p[pre + "mlp.c_fc.w"], p[pre + "mlp.c_fc.b"])
        h = gelu_tanh(u)
        x_out = x_mid + linear(h, p[pre + "mlp.c_proj.w"], p[pre + "mlp.c_proj.b"])
        saved.append((x, a1, q, k, v, o, x_mid, a2, u, h))
        x = x_out
    xf = layer_norm(x, p["ln_f.w"], p["ln_f.b"], eps)
    logits = lm_head(xf, p["wte"])
    loss = shifted_cross_entropy(logits, labels)

    g = {}
    dlogits = shifted_cross_entropy_backward(logits, labels)
    dxf, dwte_head, _ = linear_backward(xf, p["wte"], dlogits)
    dx, g["ln_f.w"], g["ln_f.b"] = layer_norm_backward(x, p["ln_f.w"], dxf, eps)
    for l in reversed(range(n_layer)):
        pre = f"h.{l}."
        x_in, a1, q, k, v, o, x_mid, a2, u, h = saved[l]
        dh, g[pre + "mlp.c_proj.w"], g[pre + "mlp.c_proj.b"] = linear_backward(h, p[pre + "mlp.c_proj.w"], dx)
        du = gelu_tanh_backward(u, dh)
        da2, g[pre + "mlp.c_fc.w"], g[pre + "mlp.c_fc.b"] = linear_backward(a2, p[pre + "mlp.c_fc.w"], du)
        dln2, g[pre + "ln_2.w"], g[pre + "ln_2.b"] = layer_norm_backward(x_mid, p[pre + "ln_2.w"], da2, eps)
        dx_mid = dx + dln2
        do, g[pre + "attn.c_proj.w"], g[pre + "attn.c_proj.b"] = linear_backward(o, p[pre + "attn.c_proj.w"], dx_mid)
        dh_ = do.shape[-1] // n_head
        do_heads = do.reshape(B, T, n_head, dh_).transpose(0, 2, 1, 3)  # the layout split_heads gives q
        dq, dk, dv = causal_attention_backward(q, k, v, do_heads)
        dqkv = np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv)], axis=-1)
        da1, g[pre + "attn.c_attn.w"], g[pre + "attn.c_attn.b"] = linear_backward(a1, p[pre + "attn.c_attn.w"], dqkv)
        dln1, g[pre + "ln_1.w"], g[pre + "ln_1.b"] = layer_norm_backward(x_in, p[pre + "ln_1.w"], da1, eps)
        dx = dx_mid + dln1
    # embedding: x[b, t] = wte[tokens[b, t]] + wpe[t]
    dwte_embed = np.zeros_like(np.asarray(p["wte"], F64))
    np.add.at(dwte_embed, tokens.reshape(-1), dx.reshape(-1, dx.shape[-1]))
    g["wte"] = dwte_head + dwte_embed
    dwpe = np.zeros_like(np.asarray(p["wpe"], F64))
    dwpe[:T] = dx.sum(axis=0)
    g["wpe"] = dwpe
    if not term_scales:
        return loss, g
    return loss, g, _gradient_magnitudes(p, tokens, labels, logits, xf, x, saved, n_head, n_layer, eps)


def _layer_norm_backward_terms(x, gamma, mdy, eps):
    """Magnitudes of the terms of layer_norm_backward for output-gradient magnitudes mdy: with
    |g| = mdy |gamma| and xhat's magnitude taken as |xhat| + 1 (its row RMS),
    |dx| <= rstd (|g| + mean|g| + |xhat| mean|g xhat|); the gain and shift gradients sum
    mdy |xhat| and mdy. Returns (dx, dgamma, dbeta) magnitudes."""
    x = np.asarray(x, dtype=F64)
    mean = x.mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mean) ** 2).mean(axis=-1, keepdims=True) + eps)
    xhat = np.abs((x - mean) * rstd) + 1.0  # |xhat| plus its row RMS (1)
    gm = mdy * np.abs(np.asarray(gamma, F64))
    dx = rstd * (gm + gm.mean(axis=-1, keepdims=True) + xhat * (gm * xhat).mean(axis=-1, keepdims=True))
    d = x.shape[-1]
    return dx, (mdy * xhat).reshape(-1, d).sum(axis=0), mdy.reshape(-1, d).sum(axis=0)


def _gradient_magnitudes(p, tokens, labels, logits, xf, x_last, saved, n_head, n_layer, eps):
    """The backward of loss_and_grads run on magnitudes: every step takes the magnitudes of its
    inputs and returns the sum of the magnitudes of the terms it adds up (|dY| |W| for an input
    gradient, |dY|^T |X| for a weight, sums of |dY| for biases and shifts, and the bounds of
    _layer_norm_backward_terms, |gelu'| mdy and causal_attention_backward_terms), starting from
    the magnitude (softmax + onehot) / n of the loss gradient. A forward activation X enters as
    |X| plus its row's RMS: an implementation computes it with an error on the scale of its row,
    so a small element can be off by far more than its own size. A relative error of e in every
    term of every step moves each gradient by at most about e times its magnitude per step it went
    through (a running error bound). Returns name -> magnitude, shaped like the gradients."""
    B, T = np.asarray(tokens).shape
    labels = np.asarray(tokens if labels is None else labels)
    sc = {}
    ab = lambda a: np.abs(np.asarray(a, dtype=F64))

    def act(a):  # a forward activation's magnitude: |a| plus its row's RMS, since an implementation's
        a = np.asarray(a, dtype=F64)  # error in an element scales with its row, not with the element
        return np.abs(a) + np.sqrt((a * a).mean(axis=-1, keepdims=True))
    # the loss gradient (softmax - onehot) / n: its two parts' magnitudes added
    z = np.asarray(logits, dtype=F64)
    _, counted = shifted_nll(z, labels)
    n = max(int(counted.sum()), 1)
    sm = softmax(z[:, :-1, :], axis=-1)
    mlog = np.zeros_like(z)
    mlog[:, :-1, :] = np.where(counted[..., None], sm, 0.0) / n
    b_idx, t_idx = np.nonzero(counted)
    mlog[b_idx, t_idx, labels[:, 1:][b_idx, t_idx]] += 1.0 / n

    def lin(name, xin, mdy):
        w = ab(p[name + ".w"])
        n_out, n_in = w.shape
        sc[name + ".w"] = mdy.reshape(-1, n_out).T @ act(xin).reshape(-1, n_in)
        sc[name + ".b"] = mdy.reshape(-1, n_out).sum(axis=0)
        return mdy @ w

    mxf = mlog @ ab(p["wte"])
    swte = mlog.reshape(-1, z.shape[-1]).T @ act(xf).reshape(-1, xf.shape[-1])
    mdx, sc["ln_f.w"], sc["ln_f.b"] = _layer_norm_backward_terms(x_last, p["ln_f.w"], mxf, eps)
    c = math.sqrt(2.0 / math.pi)
    for l in reversed(range(n_layer)):
        pre = f"h.{l}."
        x_in, a1, q, k, v, o, x_mid, a2, u, h = saved[l]
        mdh = lin(pre + "mlp.c_proj", h, mdx)
        uu = np.asarray(u, F64)
        t = np.tanh(c * (uu + 0.044715 * uu ** 3))
        mdu = mdh * np.abs(0.5 * (1.0 + t) + 0.5 * uu * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * uu * uu))
        mda2 = lin(pre + "mlp.c_fc", a2, mdu)
        mln2, sc[pre + "ln_2.w"], sc[pre + "ln_2.b"] = _layer_norm_backward_terms(x_mid, p[pre + "ln_2.w"], mda2, eps)
        mdx_mid = mdx + mln2
        mdo = lin(pre + "attn.c_proj", o, mdx_mid)
        dh_ = mdo.shape[-1] // n_head
        mdo_h = mdo.reshape(B, T, n_head, dh_).transpose(0, 2, 1, 3)
        tq, tk, tv = causal_attention_backward_terms(act(q), act(k), act(v), mdo_h)
        mda1 = lin(pre + "attn.c_attn", a1, np.concatenate([merge_heads(tq), merge_heads(tk), merge_heads(tv)], -1))
        mln1, sc[pre + "ln_1.w"], sc[pre + "ln_1.b"] = _layer_norm_backward_terms(x_in, p[pre + "ln_1.w"], mda1, eps)
        mdx = mdx_mid + mln1
    d = mdx.shape[-1]
    np.add.at(swte, tokens.reshape(-1), mdx.reshape(-1, d))
    sc["wte"] = swte
    swpe = np.zeros(np.asarray(p["wpe"]).shape)
    swpe[:T] = mdx.sum(axis=0)
    sc["wpe"] = swpe
    return sc


def param_count(n_vocab: int, n_ctx: int, d: int, n_layer: int, d_mlp: int) -> int:
    """Number of parameters with lm_head tied to wte (counted once).

    wte + wpe + per block (ln_1, c_attn, attn.c_proj, ln_2, c_fc, mlp.c_proj) + ln_f.
    """
    per_block = (2 * d) + (3 * d * d + 3 * d) + (d * d + d) + (2 * d) + (d_mlp * d + d_mlp) + (d * d_mlp + d)
    return n_vocab * d + n_ctx * d + n_layer * per_block + 2 * d
