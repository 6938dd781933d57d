"""Python front end of libloop.so.  PyTorch supplies device memory and the
stream; every step of the forward pass runs in the library's kernels."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import _abi as A


@dataclass(frozen=True)
class ModelConfig:
    vocab: int
    hidden: int
    ffn: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_layers: int
    loop_start: int
    loop_end: int
    n_passes: int = 2
    sinkhorn_iters: int = 20
    attn_period: int = 4
    rms_eps: float = 1e-6
    la_eps: float = 1e-6
    dtype: str = "bf16"           # "bf16" or "fp32"

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def qkv_rows(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    def in_loop(self, i: int) -> bool:
        return self.loop_start <= i < self.loop_end

    def to_c(self) -> A.loop_config:
        return A.loop_config(self.vocab, self.hidden, self.ffn, self.n_heads, self.n_kv_heads, self.head_dim,
                             self.n_layers, self.loop_start, self.loop_end, self.n_passes, self.sinkhorn_iters,
                             self.attn_period, self.rms_eps, self.la_eps,
                             A.LOOP_BF16 if self.dtype == "bf16" else A.LOOP_FP32)


def weight_shapes(cfg: ModelConfig) -> Dict[str, tuple]:
    """Name -> shape of every tensor the library reads."""
    C = cfg.hidden
    s = {"embed": (cfg.vocab, C), "head": (cfg.vocab, C), "final_norm": (C,)}
    for i in range(cfg.n_layers):
        p = f"layers.{i}."
        s[p + "attn_norm"] = (C,)
        s[p + "ffn_norm"] = (C,)
        s[p + "qkv"] = (cfg.qkv_rows, C)
        s[p + "o"] = (C, cfg.n_heads * cfg.head_dim)
        s[p + "gate_up"] = (2 * cfg.ffn, C)
        s[p + "down"] = (C, cfg.ffn)
        if cfg.in_loop(i):
            for site in (0, 1):
                s[p + f"mhc_w{site}"] = (8, 2 * C)
                s[p + f"mhc_b{site}"] = (8,)
    return s


def is_fp32_param(name: str) -> bool:
    return name.endswith(("norm", "mhc_w0", "mhc_w1", "mhc_b0", "mhc_b1"))


def random_weights(cfg: ModelConfig, seed: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    """Random-init weights drawn directly in device memory by the seeded
    generator (every matrix and mHC bias ~ N(0, 0.02), norm gains 1)."""
    import synth
    from synth import device as sd
    out = {}
    for name, shape in weight_shapes(cfg).items():
        fp32 = is_fp32_param(name)
        t = torch.empty(shape, dtype=torch.float32 if fp32 else cfg.torch_dtype, device=device)
        if name.endswith("norm"):
            t.fill_(1.0)
        else:
            if name in ("embed", "head"):
                tid = synth.TID_EMBED if name == "embed" else synth.TID_HEAD
            else:
                _, i, what = name.split(".")
                tid = synth.tid_layer(int(i), what)
            sd.fill_tensor_normal(t, seed, tid, synth.WEIGHT_STD)
        out[name] = t
    return out


def weights_from_arrays(cfg: ModelConfig, arrays: Dict[str, "object"], device="cuda") -> Dict[str, torch.Tensor]:
    """Uploads host arrays (name -> numpy) to device tensors of the right dtype."""
    out = {}
    for name, shape in weight_shapes(cfg).items():
        a = torch.as_tensor(arrays[name]).reshape(shape)
        dt = torch.float32 if is_fp32_param(name) else cfg.torch_dtype
        out[name] = a.to(dtype=torch.float32).to(dtype=dt).to(device).contiguous()
    return out


class LoopState:
    """Caller-owned device state (per-(layer, pass) KV caches and linear states)."""

    def __init__(self, model: "LoopModel", batch: int, max_seq: int, n_pages: Optional[int] = None):
        """n_pages: a paged state (every full-attention slot a pool of n_pages
        pages of 64 positions); its block table is ``self.block_table``, int32
        [batch][ceil(max_seq / 64)] on the device, initially page b * blocks + j
        for block j of sequence b (fill it before use if there are fewer pages)."""
        self.model = model
        self.batch = batch
        self.max_seq = max_seq
        self.n_pages = n_pages
        self.block_table = None
        if n_pages is None:
            self.nbytes = A.loop_state_bytes(model.handle, batch, max_seq)
        else:
            self.nbytes = A.loop_state_bytes_paged(model.handle, batch, max_seq, n_pages)
            blocks = (max_seq + 63) // 64
            self.block_table = torch.arange(batch * blocks, dtype=torch.int32,
                                            device=model.device).reshape(batch, blocks) % n_pages
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=model.device)
        self.buf[:256].zero_()
        if n_pages is None:
            self.handle = A.loop_state_create(model.handle, self.buf.data_ptr(), self.nbytes, batch, max_seq)
        else:
            self.handle = A.loop_state_create_paged(model.handle, self.buf.data_ptr(), self.nbytes, batch, max_seq,
                                                    n_pages, self.block_table.data_ptr())

    @property
    def length(self) -> int:
        """The shortest sequence's length (the common one unless ragged)."""
        return A.loop_state_length(self.handle)

    def set_length(self, n: int) -> None:
        A.loop_state_set_length(self.handle, n)

    def seq_length(self, seq: int) -> int:
        return A.loop_state_seq_length(self.handle, seq)

    def set_seq_length(self, seq: int, n: int) -> None:
        A.loop_state_set_seq_length(self.handle, seq, n)

    @property
    def lengths(self):
        return [self.seq_length(i) for i in range(self.batch)]

    def region(self, kind: int, slot: int):
        return A.loop_state_region(self.handle, kind, slot)

    def region_tensor(self, kind: int, slot: int) -> torch.Tensor:
        """View of one region: K/V^T in the model dtype, S/z in float32 (flat)."""
        ptr, nbytes = self.region(kind, slot)
        off = ptr - self.buf.data_ptr()
        dt = self.model.cfg.torch_dtype if kind in (A.REGION_K, A.REGION_VT) else torch.float32
        return self.buf[off:off + nbytes].view(dt)

    def check(self) -> None:
        A.loop_state_check(self.handle, torch.cuda.current_stream(self.model.device).cuda_stream)

    def close(self) -> None:
        if self.handle:
            A.loop_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LoopModel:
    def __init__(self, cfg: ModelConfig, weights: Dict[str, torch.Tensor], device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.weights = weights
        layers = (A.loop_layer_weights * cfg.n_layers)()
        for i in range(cfg.n_layers):
            p = f"layers.{i}."
            L = layers[i]
            L.attn_norm = weights[p + "attn_norm"].data_ptr()
            L.ffn_norm = weights[p + "ffn_norm"].data_ptr()
            L.qkv = weights[p + "qkv"].data_ptr()
            L.o = weights[p + "o"].data_ptr()
            L.gate_up = weights[p + "gate_up"].data_ptr()
            L.down = weights[p + "down"].data_ptr()
            if cfg.in_loop(i):
                for s in (0, 1):
                    L.mhc_w[s] = weights[p + f"mhc_w{s}"].data_ptr()
                    L.mhc_b[s] = weights[p + f"mhc_b{s}"].data_ptr()
        self._layers = layers
        self._cw = A.loop_weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                                  weights["head"].data_ptr(), ctypes.cast(layers, ctypes.POINTER(A.loop_layer_weights)),
                                  cfg.n_layers)
        self._cc = cfg.to_c()
        self.handle = A.loop_model_create(self._cc, self._cw)
        self._ws = None

    def schedule(self):
        return A.loop_model_schedule(self.handle)

    def new_state(self, batch: int, max_seq: int, n_pages: Optional[int] = None) -> LoopState:
        return LoopState(self, batch, max_seq, n_pages)

    def workspace(self, batch: int, max_tokens: int, max_seq: int) -> torch.Tensor:
        n = A.loop_workspace_bytes(self.handle, batch, max_tokens, max_seq)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws

    def _stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def prefill(self, state: LoopState, tokens: Optional[torch.Tensor] = None, embeds: Optional[torch.Tensor] = None,
                all_logits: bool = False, hidden_out: bool = False, cont: bool = False,
                out: Optional[torch.Tensor] = None, seq0: Optional[int] = None) -> torch.Tensor:
        """Prefill of B sequences: [0, B), or [seq0, seq0 + B) of the state
        when seq0 is given (the other sequences keep their lengths)."""
        src = tokens if tokens is not None else embeds
        B, S = int(src.shape[0]), int(src.shape[1])
        flags = (A.LOOP_ALL_LOGITS if all_logits else 0) | (A.LOOP_HIDDEN_OUT if hidden_out else 0) | \
                (A.LOOP_CONTINUE if cont else 0)
        if out is None:
            if hidden_out:
                out = torch.empty(B, S, self.cfg.hidden, dtype=self.cfg.torch_dtype, device=self.device)
            elif all_logits:
                out = torch.empty(B, S, self.cfg.vocab, dtype=torch.float32, device=self.device)
            else:
                out = torch.empty(B, self.cfg.vocab, dtype=torch.float32, device=self.device)
        ws = self.workspace(state.batch, B * S, state.max_seq)
        tok_ptr = tokens.data_ptr() if tokens is not None else None
        emb_ptr = embeds.data_ptr() if embeds is not None else None
        if tokens is not None:
            assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        if embeds is not None:
            assert embeds.dtype == self.cfg.torch_dtype and embeds.is_contiguous()
        if seq0 is None:
            A.loop_prefill(self.handle, state.handle, ws.data_ptr(), ws.numel(), tok_ptr, emb_ptr, B, S, flags,
                           out.data_ptr(), self._stream())
        else:
            A.loop_prefill_rows(self.handle, state.handle, ws.data_ptr(), ws.numel(), seq0, tok_ptr, emb_ptr, B, S,
                                flags, out.data_ptr(), self._stream())
        return out

    def decode_step(self, state: LoopState, tokens: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        B = int(tokens.shape[0])
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        if out is None:
            out = torch.empty(B, self.cfg.vocab, dtype=torch.float32, device=self.device)
        ws = self.workspace(state.batch, B, state.max_seq)
        A.loop_decode_step(self.handle, state.handle, ws.data_ptr(), ws.numel(), tokens.data_ptr(), B,
                           out.data_ptr(), self._stream())
        return out

    def decode_step_noalloc(self, state: LoopState, tokens: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
        """decode_step on the library's own static device workspace: the call
        allocates nothing (the caller passes the logits buffer)."""
        B = int(tokens.shape[0])
        assert tokens.dtype == torch.int32 and tokens.is_contiguous()
        assert out.dtype == torch.float32 and out.is_contiguous() and out.numel() >= B * self.cfg.vocab
        A.loop_decode_step_noalloc(self.handle, state.handle, tokens.data_ptr(), B, out.data_ptr(), self._stream())
        return out

    def decode_pipelined(self, state: LoopState, tokens: Optional[torch.Tensor], out: Optional[torch.Tensor] = None):
        """One call of the pass-pipelined decode (the state holds n_passes
        cohorts of B sequences).  tokens: int32 [B] for the entering cohort, or
        None.  Returns (entered, left, logits): the cohorts that entered and
        left (-1: none) and float32 [B][V] logits of the leaving cohort."""
        G = self.cfg.n_passes
        B = state.batch // G
        if tokens is not None:
            assert tokens.dtype == torch.int32 and tokens.is_contiguous() and int(tokens.shape[0]) == B
        if out is None:
            out = torch.empty(B, self.cfg.vocab, dtype=torch.float32, device=self.device)
        ws = self.workspace(state.batch, state.batch, state.max_seq)
        entered, left = A.loop_decode_pipelined(self.handle, state.handle, ws.data_ptr(), ws.numel(),
                                                tokens.data_ptr() if tokens is not None else None, B,
                                                out.data_ptr(), self._stream())
        return entered, left, out

    def close(self) -> None:
        if self.handle:
            A.loop_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
