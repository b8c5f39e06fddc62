"""ctypes binding of libgpt2.so (the C ABI in include/gpt2.h).

Argument marshalling only: every step of the forward runs in the library's HIP kernels. PyTorch
supplies device memory (tensors the caller owns) and the current HIP stream. The library must be
built (``python -m decoder_only_transformer_gpt2_amd.build``); nothing here falls back to any
other implementation when it is missing.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgpt2.so")

OK, EINVAL, ESHAPE, EWORKSPACE, ETOKEN, EHIP, ESTATE = range(7)
F32, BF16 = 0, 1
GELU_TANH, GELU_ERF = 0, 1
EPI_BIAS, EPI_BIAS_GELU, EPI_BIAS_RESIDUAL, EPI_LOGITS = range(4)
KERNEL_KINDS = ("embed", "ln", "qkv", "attn", "attn_proj", "fc", "mlp_proj", "ln_f", "lm_head", "argmax", "xent",
                "kv")

# Every function the header declares, with its ctypes signature (restype, argtypes).
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_I64P = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "gpt2_config": (_I32, [_P, ctypes.POINTER(_P)]),
    "gpt2_destroy": (None, [_P]),
    "gpt2_n_tensors": (_I32, [_P]),
    "gpt2_tensor_shape": (_I32, [_P, _I32, _I64P, _I64P]),
    "gpt2_weight_bytes": (_SZ, [_P]),
    "gpt2_workspace_bytes": (_SZ, [_P, _I32, _I32]),
    "gpt2_load_weights": (_I32, [_P, ctypes.POINTER(_P), _I32, _I32, _P, _SZ, _P]),
    "gpt2_forward": (_I32, [_P, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "gpt2_forward_noalloc": (_I32, [_P, _P, _I32, _I32, _P, _P, _P]),
    "gpt2_forward_loss": (_I32, [_P, _P, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "gpt2_kv_cache_bytes": (_SZ, [_P, _I32]),
    "gpt2_prefill": (_I32, [_P, _P, _I32, _I32, _P, _SZ, _P, _P, _P, _SZ, _P]),
    "gpt2_decode_step": (_I32, [_P, _P, _I32, _I32, _P, _SZ, _P, _P, _P, _SZ, _P]),
    "gpt2_forward_debug": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "gpt2_check": (_I32, [_P, _P, _I32, _I32, _P]),
    "gpt2_forward_launches": (_I32, [_P, _I32, _I32, _I32, ctypes.POINTER(_I32), _I32]),
    "gpt2_forward_repeat": (_I32, [_P, _P, _I32, _I32, _P, _P, _P, _SZ, _P, _I32, _I32, _P, _P]),
    "gpt2_forward_timed": (_I32, [_P, _P, _I32, _I32, _P, _P, _P, _SZ, _P, ctypes.POINTER(_P), ctypes.POINTER(_P), _I32]),
    "gpt2_attention": (_I32, [_P, _I64P, _P, _I64P, _P, _I64P, _P, _I64P, _I32, _I32, _I32, _I32, _I32, _P]),
    "gpt2_layernorm": (_I32, [_P, _P, _P, _P, _I32, _I32, _F, _I32, _P]),
    "gpt2_linear": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P]),
    "gpt2_sample": (_I32, [_P, _I64, _I32, _I32, _P, _I64, _I32, _F, _I32, _F, _F, _P, _P, _P, _P, _SZ, _P]),
    "gpt2_sample_workspace_bytes": (_SZ, [_I32, _I32]),
    "gpt2_grad_bytes": (_SZ, [_P]),
    "gpt2_grad_offset": (_SZ, [_P, _I32]),
    "gpt2_train_workspace_bytes": (_SZ, [_P, _I32, _I32]),
    "gpt2_backward": (_I32, [_P, _P, _P, _I32, _I32, _P, _SZ, _P, _P, _SZ, _P]),
    "gpt2_strerror": (ctypes.c_char_p, [_I32]),
}


class Config(ctypes.Structure):
    _fields_ = [("n_vocab", _I32), ("n_ctx", _I32), ("d_model", _I32), ("n_head", _I32), ("n_layer", _I32),
                ("d_mlp", _I32), ("ln_eps", _F), ("dtype", _I32), ("gelu", _I32)]


class GPT2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Open libgpt2.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decoder_only_transformer_gpt2_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().gpt2_strerror(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise GPT2Error(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _strides(t: torch.Tensor):
    """(s_b, s_h, s_t) element strides of a [B, H, T, dh] view with a contiguous last dim."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("attention operands must be [B, H, T, dh] views with a contiguous last dimension")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("every tensor handed to the library must live on the GPU")


@dataclass(frozen=True)
class ModelConfig:
    n_vocab: int = 50257
    n_ctx: int = 1024
    d_model: int = 768
    n_head: int = 12
    n_layer: int = 12
    d_mlp: int = 3072
    ln_eps: float = 1e-5
    dtype: str = "bf16"   # "bf16" or "f32"
    gelu: str = "tanh"    # "tanh" or "erf"

    def to_c(self) -> Config:
        return Config(self.n_vocab, self.n_ctx, self.d_model, self.n_head, self.n_layer, self.d_mlp, self.ln_eps,
                      BF16 if self.dtype == "bf16" else F32, GELU_ERF if self.gelu == "erf" else GELU_TANH)


def _aligned_empty(nbytes: int, device, align: int = 256) -> torch.Tensor:
    """uint8 device buffer of nbytes whose first byte is align-aligned (a view into a torch tensor)."""
    raw = torch.empty(nbytes + align, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % align
    return raw[off:off + nbytes]


class GPT2:
    """A configured model: packed weights on the device plus the handle that describes them."""

    def __init__(self, cfg: ModelConfig, device: str | torch.device = "cuda:0"):
        self.cfg = cfg
        self.device = torch.device(device)
        self._h = ctypes.c_void_p()
        _check(lib().gpt2_config(ctypes.byref(cfg.to_c()), ctypes.byref(self._h)), "gpt2_config")
        self.weights = None
        self._ws = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and h.value and _lib is not None:
            _lib.gpt2_destroy(h)
            self._h = ctypes.c_void_p()

    # -- sizes -----------------------------------------------------------------------------------
    def n_tensors(self) -> int:
        return lib().gpt2_n_tensors(self._h)

    def tensor_shape(self, i: int):
        r, c = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().gpt2_tensor_shape(self._h, i, ctypes.byref(r), ctypes.byref(c)), "gpt2_tensor_shape")
        return (r.value,) if c.value == 0 else (r.value, c.value)

    def weight_bytes(self) -> int:
        return lib().gpt2_weight_bytes(self._h)

    def workspace_bytes(self, B: int, T: int) -> int:
        return lib().gpt2_workspace_bytes(self._h, B, T)

    # -- weights ---------------------------------------------------------------------------------
    def load_weights(self, tensors, stream=None) -> None:
        """tensors: sequence in the header's fixed order of contiguous fp32 or bf16 device tensors."""
        tensors = list(tensors)
        if len(tensors) != self.n_tensors():
            raise ValueError(f"expected {self.n_tensors()} tensors, got {len(tensors)}")
        dt = tensors[0].dtype
        if dt not in (torch.float32, torch.bfloat16) or any(t.dtype != dt for t in tensors):
            raise ValueError("source tensors must all be float32 or all bfloat16")
        for i, t in enumerate(tensors):
            _require_cuda(t)
            if not t.is_contiguous() or tuple(t.shape) != self.tensor_shape(i):
                raise ValueError(f"tensor {i}: expected contiguous shape {self.tensor_shape(i)}, got {tuple(t.shape)}")
        dst = _aligned_empty(self.weight_bytes(), self.device)
        ptrs = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
        _check(lib().gpt2_load_weights(self._h, ptrs, len(tensors), BF16 if dt == torch.bfloat16 else F32,
                                       _ptr(dst), dst.numel(), _stream(stream)), "gpt2_load_weights")
        # the sources must outlive the asynchronous packing
        torch.cuda.current_stream(self.device).synchronize() if stream is None else stream.synchronize()
        self.weights = dst

    def load_numpy(self, named: dict) -> None:
        """Upload a name -> numpy float32 dict (the synthetic generator's output) and pack it."""
        ts = [torch.from_numpy(a).to(self.device) for a in named.values()]
        self.load_weights(ts)

    # -- forward ---------------------------------------------------------------------------------
    def workspace(self, B: int, T: int) -> torch.Tensor:
        n = self.workspace_bytes(B, T)
        if n == 0:
            raise GPT2Error(ESHAPE, "gpt2_workspace_bytes")
        ws = self._ws.get((B, T))
        if ws is None:
            ws = _aligned_empty(n, self.device)
            self._ws[(B, T)] = ws
        return ws

    def forward(self, tokens: torch.Tensor, logits: torch.Tensor | None = None, argmax: bool | torch.Tensor = True,
                ws: torch.Tensor | None = None, stream=None):
        """tokens int32 [B, T] on the device -> (logits fp32 [B, T, V], argmax int32 [B, T] or None)."""
        _require_cuda(tokens)
        if tokens.dtype != torch.int32 or tokens.dim() != 2 or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 [B, T] device tensor")
        B, T = tokens.shape
        V = self.cfg.n_vocab
        if logits is None:
            logits = torch.empty((B, T, V), dtype=torch.float32, device=self.device)
        if argmax is True:
            argmax = torch.empty((B, T), dtype=torch.int32, device=self.device)
        elif argmax is False:
            argmax = None
        ws = self.workspace(B, T) if ws is None else ws
        _require_cuda(logits, argmax, ws)
        _check(lib().gpt2_forward(self._h, _ptr(tokens), B, T, _ptr(logits), _ptr(argmax), _ptr(ws), ws.numel(),
                                  _stream(stream)), "gpt2_forward")
        return logits, argmax

    def forward_noalloc(self, tokens: torch.Tensor, logits: torch.Tensor, argmax: torch.Tensor | None = None,
                        stream=None):
        """gpt2_forward_noalloc: the forward with the library's fixed scratch as workspace; the
        caller passes every output (nothing is allocated here either)."""
        _require_cuda(tokens, logits, argmax)
        if tokens.dtype != torch.int32 or tokens.dim() != 2 or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 [B, T] device tensor")
        B, T = tokens.shape
        _check(lib().gpt2_forward_noalloc(self._h, _ptr(tokens), B, T, _ptr(logits), _ptr(argmax), _stream(stream)),
               "gpt2_forward_noalloc")
        return logits, argmax

    def forward_loss(self, tokens: torch.Tensor, labels: torch.Tensor | None = None, nll: torch.Tensor | None = None,
                     loss: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
        """tokens int32 [B, T] (and labels int32 [B, T] or None = tokens) on the device ->
        (nll fp32 [B, T], loss fp32 [1]): the shifted next-token cross-entropy, logits never stored."""
        _require_cuda(tokens, labels)
        for t in (tokens, labels):
            if t is not None and (t.dtype != torch.int32 or t.dim() != 2 or not t.is_contiguous()):
                raise ValueError("tokens and labels must be contiguous int32 [B, T] device tensors")
        B, T = tokens.shape
        if labels is not None and tuple(labels.shape) != (B, T):
            raise ValueError("labels must have the shape of tokens")
        if nll is None:
            nll = torch.empty((B, T), dtype=torch.float32, device=self.device)
        if loss is None:
            loss = torch.empty((1,), dtype=torch.float32, device=self.device)
        ws = self.workspace(B, T) if ws is None else ws
        _check(lib().gpt2_forward_loss(self._h, _ptr(tokens), _ptr(labels), B, T, _ptr(nll), _ptr(loss), _ptr(ws),
                                       ws.numel(), _stream(stream)), "gpt2_forward_loss")
        return nll, loss

    # -- cached decoding -------------------------------------------------------------------------
    def kv_cache(self, B: int) -> torch.Tensor:
        """A key/value cache for B sequences (uint8 device buffer, 256-byte aligned)."""
        n = lib().gpt2_kv_cache_bytes(self._h, B)
        if n == 0:
            raise GPT2Error(ESHAPE, "gpt2_kv_cache_bytes")
        return _aligned_empty(n, self.device)

    def _next_outputs(self, B: int, logits, nxt):
        if logits is True:
            logits = torch.empty((B, self.cfg.n_vocab), dtype=torch.float32, device=self.device)
        elif logits is False:
            logits = None
        if nxt is True:
            nxt = torch.empty((B,), dtype=torch.int32, device=self.device)
        elif nxt is False:
            nxt = None
        return logits, nxt

    def prefill(self, tokens: torch.Tensor, cache: torch.Tensor, logits=False, nxt=True, ws=None, stream=None):
        """Forward over the prompt tokens int32 [B, T], filling cache positions 0..T-1; returns the
        last position's (logits [B, V] or None, greedy next token int32 [B] or None)."""
        _require_cuda(tokens, cache)
        if tokens.dtype != torch.int32 or tokens.dim() != 2 or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 [B, T] device tensor")
        B, T = tokens.shape
        logits, nxt = self._next_outputs(B, logits, nxt)
        ws = self.workspace(B, T) if ws is None else ws
        _check(lib().gpt2_prefill(self._h, _ptr(tokens), B, T, _ptr(cache), cache.numel(), _ptr(logits), _ptr(nxt),
                                  _ptr(ws), ws.numel(), _stream(stream)), "gpt2_prefill")
        return logits, nxt

    def decode_step(self, tokens: torch.Tensor, pos: int, cache: torch.Tensor, logits=False, nxt=True, ws=None,
                    stream=None):
        """One step: tokens int32 [B] at position pos (positions 0..pos-1 already cached)."""
        _require_cuda(tokens, cache)
        if tokens.dtype != torch.int32 or tokens.dim() != 1 or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 [B] device tensor")
        B = tokens.shape[0]
        logits, nxt = self._next_outputs(B, logits, nxt)
        ws = self.workspace(B, 1) if ws is None else ws
        _check(lib().gpt2_decode_step(self._h, _ptr(tokens), B, pos, _ptr(cache), cache.numel(), _ptr(logits),
                                      _ptr(nxt), _ptr(ws), ws.numel(), _stream(stream)), "gpt2_decode_step")
        return logits, nxt

    def generate(self, prompt: torch.Tensor, n_new: int, cache: torch.Tensor | None = None, stream=None,
                 do_sample: bool = False, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                 repetition_penalty: float = 1.0, u: torch.Tensor | None = None,
                 generator: torch.Generator | None = None) -> torch.Tensor:
        """Decoding: int32 [B, T] prompt -> int32 [B, T + n_new] (prefill, then one cached step per new
        token; every call is enqueued on the stream without a host synchronisation). Greedy unless
        do_sample; sampling applies the repetition penalty over the whole sequence so far, the
        temperature, top-k and top-p (gpt2_sample), drawing new token i of row b at the uniform
        number u[i, b] (fp32 [n_new, B] on the device; drawn with torch.rand and generator if None)."""
        B, T = prompt.shape
        if T + n_new > self.cfg.n_ctx:
            raise ValueError("prompt plus new tokens exceed n_ctx")
        cache = self.kv_cache(B) if cache is None else cache
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            out = torch.empty((B, T + n_new), dtype=torch.int32, device=self.device)
            out[:, :T] = prompt
            if n_new == 0:
                return out
            if do_sample and u is None:
                u = torch.rand((n_new, B), generator=generator, dtype=torch.float32, device=self.device)
            if do_sample and (u.shape != (n_new, B) or u.dtype != torch.float32 or u.device != out.device):
                raise ValueError("u must be a float32 [n_new, B] tensor on the model's device")
            u = u.contiguous() if do_sample else None
            logits = torch.empty((B, self.cfg.n_vocab), dtype=torch.float32, device=self.device) if do_sample else None
            sws = _aligned_empty(sample_workspace_bytes(B, self.cfg.n_vocab), self.device) if do_sample else None
            toks = [torch.empty((B,), dtype=torch.int32, device=self.device) for _ in range(2)]

            def pick(i, nxt):
                if do_sample:
                    sample(logits, u[i], history=out[:, :T + i], temperature=temperature, top_k=top_k, top_p=top_p,
                           repetition_penalty=repetition_penalty, out=nxt, ws=sws)
                out[:, T + i] = nxt

            self.prefill(prompt, cache, logits=logits if do_sample else False, nxt=False if do_sample else toks[0])
            pick(0, toks[0])
            for i in range(1, n_new):
                cur, nxt = toks[(i - 1) % 2], toks[i % 2]
                self.decode_step(cur, T + i - 1, cache, logits=logits if do_sample else False,
                                 nxt=False if do_sample else nxt)
                pick(i, nxt)
        return out

    def grad_buffer(self) -> torch.Tensor:
        """A zeroed fp32 device buffer for the gradients (gpt2_grad_bytes, 256-byte aligned)."""
        return _aligned_empty(lib().gpt2_grad_bytes(self._h), self.device).zero_()

    def grad_views(self, buf: torch.Tensor, names: list[str] | None = None) -> list[torch.Tensor] | dict:
        """fp32 views of each tensor's gradient inside buf, in source order (a dict when names are given)."""
        views = []
        for i in range(self.n_tensors()):
            off = lib().gpt2_grad_offset(self._h, i)
            shape = self.tensor_shape(i)
            n = int(np.prod(shape))
            views.append(buf[off:off + 4 * n].view(torch.float32).view(shape))
        return dict(zip(names, views)) if names is not None else views

    def train_workspace(self, B: int, T: int) -> torch.Tensor:
        n = lib().gpt2_train_workspace_bytes(self._h, B, T)
        if n == 0:
            raise GPT2Error(ESHAPE, "gpt2_train_workspace_bytes")
        return _aligned_empty(n, self.device)

    def backward(self, tokens: torch.Tensor, labels: torch.Tensor | None = None, grads: torch.Tensor | None = None,
                 loss: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
        """Loss and gradients of the mean shifted cross-entropy: returns (loss fp32 [1], grads buffer)."""
        _require_cuda(tokens, labels, grads, loss, ws)
        if tokens.dtype != torch.int32 or tokens.dim() != 2 or not tokens.is_contiguous():
            raise ValueError("tokens must be a contiguous int32 [B, T] device tensor")
        B, T = tokens.shape
        if labels is not None and (labels.shape != tokens.shape or labels.dtype != torch.int32 or
                                   not labels.is_contiguous()):
            raise ValueError("labels must be a contiguous int32 tensor shaped like tokens")
        grads = self.grad_buffer() if grads is None else grads
        loss = torch.empty((1,), dtype=torch.float32, device=self.device) if loss is None else loss
        ws = self.train_workspace(B, T) if ws is None else ws
        _check(lib().gpt2_backward(self._h, _ptr(tokens), _ptr(labels), B, T, _ptr(grads), grads.numel(), _ptr(loss),
                                   _ptr(ws), ws.numel(), _stream(stream)), "gpt2_backward")
        return loss, grads

    def launches(self, B: int, T: int, with_argmax: bool = True) -> list[str]:
        """Kinds of the kernel launches one forward over B x T tokens enqueues, in order."""
        n = lib().gpt2_forward_launches(self._h, B, T, int(with_argmax), None, 0)
        if n == 0:
            raise ValueError(f"no forward for B={B}, T={T}")
        kinds = (ctypes.c_int32 * n)()
        lib().gpt2_forward_launches(self._h, B, T, int(with_argmax), kinds, n)
        return [KERNEL_KINDS[k] for k in kinds]

    def forward_timed(self, tokens: torch.Tensor, logits: torch.Tensor, argmax: torch.Tensor | None,
                      before: list, after: list, ws: torch.Tensor | None = None, stream=None):
        """forward() that records raw hipEvent_t handles (ints or None) around launch i on the stream."""
        B, T = tokens.shape
        ws = self.workspace(B, T) if ws is None else ws
        n = max(len(before), len(after))
        eb = (ctypes.c_void_p * n)(*[(before[i] if i < len(before) else None) for i in range(n)])
        ea = (ctypes.c_void_p * n)(*[(after[i] if i < len(after) else None) for i in range(n)])
        _check(lib().gpt2_forward_timed(self._h, _ptr(tokens), B, T, _ptr(logits), _ptr(argmax), _ptr(ws), ws.numel(),
                                        _stream(stream), eb, ea, n), "gpt2_forward_timed")
        return logits, argmax

    def forward_repeat(self, tokens: torch.Tensor, logits: torch.Tensor, argmax: torch.Tensor | None, launch: int,
                       repeats: int, before=None, after=None, ws: torch.Tensor | None = None, stream=None):
        """forward() with launch number `launch` enqueued `repeats` times back to back and raw
        hipEvent_t handles (ints or None) recorded around that group."""
        B, T = tokens.shape
        ws = self.workspace(B, T) if ws is None else ws
        _check(lib().gpt2_forward_repeat(self._h, _ptr(tokens), B, T, _ptr(logits), _ptr(argmax), _ptr(ws), ws.numel(),
                                         _stream(stream), launch, repeats, before, after), "gpt2_forward_repeat")
        return logits, argmax

    def forward_debug(self, tokens: torch.Tensor, n_layers: int, ws: torch.Tensor | None = None, stream=None):
        _require_cuda(tokens)
        B, T = tokens.shape
        out = torch.empty((B, T, self.cfg.d_model), dtype=torch.float32, device=self.device)
        ws = self.workspace(B, T) if ws is None else ws
        _check(lib().gpt2_forward_debug(self._h, _ptr(tokens), B, T, n_layers, _ptr(out), _ptr(ws), ws.numel(),
                                        _stream(stream)), "gpt2_forward_debug")
        return out

    def check(self, B: int, T: int, ws: torch.Tensor | None = None, stream=None) -> int:
        ws = self.workspace(B, T) if ws is None else ws
        return lib().gpt2_check(self._h, _ptr(ws), B, T, _stream(stream))


# -- op-level entry points -----------------------------------------------------------------------
def sample(logits: torch.Tensor, u: torch.Tensor, history: torch.Tensor | None = None, temperature: float = 1.0,
           top_k: int = 0, top_p: float = 1.0, repetition_penalty: float = 1.0, out: torch.Tensor | None = None,
           n_kept: torch.Tensor | None = None, ws: torch.Tensor | bool | None = True, stream=None) -> torch.Tensor:
    """Sampled next token per row of fp32 logits [B, V] (row stride logits.stride(0)) at the uniform
    numbers u fp32 [B]; history int32 [B, n] (row stride history.stride(0)) feeds the repetition
    penalty. Returns out int32 [B]; n_kept int32 [B], if given, receives the kept-set sizes. ws: a
    workspace of sample_workspace_bytes(B, V) bytes, True to allocate one, or None / False for the
    one-workgroup-per-row path."""
    _require_cuda(logits, u)
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be a float32 [B, V] device tensor with unit column stride")
    B, V = logits.shape
    if u.dtype != torch.float32 or u.shape != (B,) or not u.is_contiguous():
        raise ValueError("u must be a contiguous float32 [B] device tensor")
    n_hist, hist_ld = 0, 0
    if history is not None:
        _require_cuda(history)
        if history.dtype != torch.int32 or history.dim() != 2 or history.shape[0] != B or history.stride(1) != 1:
            raise ValueError("history must be an int32 [B, n] device tensor with unit column stride")
        n_hist, hist_ld = history.shape[1], history.stride(0)
    out = torch.empty((B,), dtype=torch.int32, device=logits.device) if out is None else out
    if out.dtype != torch.int32 or out.shape != (B,) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [B] device tensor")
    if n_kept is not None and (n_kept.dtype != torch.int32 or n_kept.shape != (B,) or not n_kept.is_contiguous()):
        raise ValueError("n_kept must be a contiguous int32 [B] device tensor")
    if ws is True:
        ws = _aligned_empty(sample_workspace_bytes(B, V), logits.device)
    elif ws is False:
        ws = None
    if ws is not None:
        _require_cuda(ws)
    _check(lib().gpt2_sample(_ptr(logits), logits.stride(0), B, V, _ptr(history) if n_hist else None, hist_ld, n_hist,
                             temperature, top_k, top_p, repetition_penalty, _ptr(u), _ptr(out), _ptr(n_kept), _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "gpt2_sample")
    return out


def sample_workspace_bytes(B: int, V: int) -> int:
    """Bytes of the optional sampler workspace (0 for invalid B, V)."""
    return lib().gpt2_sample_workspace_bytes(B, V)


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None, stream=None):
    """Causal attention of [B, H, T, 64] views (bf16 or fp32); returns o (allocated if None)."""
    _require_cuda(q, k, v, o)
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    dt = BF16 if q.dtype == torch.bfloat16 else F32
    if any(t.dtype != q.dtype for t in (k, v, o)) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v, o must share one dtype, bfloat16 or float32")
    B, H, T, dh = q.shape
    for t in (k, v, o):
        if tuple(t.shape) != (B, H, T, dh):
            raise ValueError("q, k, v, o must have the same shape")
    _check(lib().gpt2_attention(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(o), _strides(o),
                                B, H, T, dh, dt, _stream(stream)), "gpt2_attention")
    return o


def layernorm(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float = 1e-5,
              out_dtype: torch.dtype = torch.bfloat16, stream=None, out: torch.Tensor | None = None):
    """LayerNorm of the rows of fp32 x [M, n]; out (if given) must be a contiguous [M, n] tensor of
    out_dtype."""
    _require_cuda(x, gamma, beta, out)
    M, n = x.shape
    y = torch.empty((M, n), dtype=out_dtype, device=x.device) if out is None else out
    if y.dtype != out_dtype or tuple(y.shape) != (M, n) or not y.is_contiguous():
        raise ValueError("out must be a contiguous [M, n] tensor of out_dtype")
    _check(lib().gpt2_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), M, n, eps,
                                BF16 if out_dtype == torch.bfloat16 else F32, _stream(stream)), "gpt2_layernorm")
    return y


def linear(A: torch.Tensor, W: torch.Tensor, bias: torch.Tensor | None, C: torch.Tensor, M: int, N: int, K: int,
           epilogue: int, gelu: int = GELU_TANH, stream=None):
    """C = epi(A[:M] W[:N]^T + bias); A and W must have their row counts padded to multiples of 256."""
    _require_cuda(A, W, bias, C)
    dt = BF16 if A.dtype == torch.bfloat16 else F32
    if A.shape[0] < -(-M // 256) * 256 or W.shape[0] < -(-N // 256) * 256:
        raise ValueError("A and W need their row counts padded to a multiple of 256")
    _check(lib().gpt2_linear(_ptr(A), _ptr(W), _ptr(bias), _ptr(C), M, N, K, C.stride(0), dt, epilogue, gelu,
                             _stream(stream)), "gpt2_linear")
    return C
