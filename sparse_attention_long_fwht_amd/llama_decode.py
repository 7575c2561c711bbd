"""A Llama-3.1-8B-shaped decoder stack around the Adamas decode step.

The pages compare Adamas end to end against dense attention on
Llama-3.1-8B-Instruct (paper abstracts: 4.4x attention-only and 1.5x
end-to-end speedups at 32K; blog section 5.1: the same figures, with memory
bandwidth the limit at 32K and CUDA Graph capture worth 23% at small batch).
This module reproduces that measurement's shape on one MI355X: 32 layers,
hidden 4096, 32 query / 8 KV heads of 128, SwiGLU MLP of 14336, vocabulary
128256, RMSNorm, rotary embeddings (theta 500000) -- with random weights, since
only latency is measured (no checkpoint is loaded and no output quality is
claimed).  Blog section 3.2 keeps the last 3 layers dense; `dense_last` does
the same.

Every attention call goes through libadamas.so (adamas_append_decode_step,
adamas_forced_decode_step or dense_decode_attention).  The model around it:
projections and the vocabulary head are torch bf16 GEMMs (weights stored
[out, in], the layout the GEMV path of the BLAS library is tuned for); the
elementwise work between them is three fused kernels of libllama_glue.so
(residual add + RMSNorm, rotary + cache append, SiLU * up), so that a layer is
about a dozen launches.  One decode step appends one token to every sequence
and is capturable in a HIP graph: token ids and lengths live in device tensors.
"""
from dataclasses import dataclass
from typing import List, Optional

import torch

import torch.nn.functional as F

from . import alloc_workspace, decode_step, decode_workspace_size, dense_decode_attention, dense_workspace_size
from . import llama_glue


@dataclass(frozen=True)
class DecoderShape:
    layers: int = 32
    hidden: int = 4096
    q_heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    ffn: int = 14336
    vocab: int = 128256
    rope_theta: float = 500000.0
    eps: float = 1e-5


LLAMA31_8B = DecoderShape()


class _Layer:
    pass


class LlamaShapedDecoder:
    """Random-weight decoder with per-layer K/V caches and Adamas key codes.

    attention: "adamas" (the Adamas step, the new key encoded inside it) or
    "dense" (dense decode attention over every cached position).  With
    "adamas", the last `dense_last` layers use dense attention and keep no
    codes; sink / recent select adamas_forced_decode_step.
    """

    def __init__(self, shape: DecoderShape, batch: int, capacity: int, attention: str = "adamas",
                 budget: int = 128, dense_last: int = 0, sink: Optional[int] = None, recent: Optional[int] = None,
                 seed: int = 0, device: str = "cuda"):
        if attention not in ("adamas", "dense"):
            raise ValueError("attention must be 'adamas' or 'dense'")
        if shape.head_dim != 128 or shape.hidden != shape.q_heads * shape.head_dim:
            raise ValueError("head_dim 128 and hidden = q_heads * head_dim are required")
        self.shape, self.B, self.cap = shape, batch, capacity
        self.attention, self.budget, self.sink, self.recent = attention, budget, sink, recent
        self.dense_last = shape.layers if attention == "dense" else dense_last
        self.device = device
        self.scale = shape.head_dim ** -0.5
        self.trace: Optional[List[dict]] = None  # set to a list to record each attention call (tests)
        S, dev = shape, device
        g = torch.Generator(device=dev)
        g.manual_seed(seed)

        def w(rows, cols):
            t = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
            for r0 in range(0, rows, 4096):  # (fp32 draws in slices: bounded transient memory)
                r1 = min(rows, r0 + 4096)
                t[r0:r1] = (torch.randn((r1 - r0, cols), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            return t

        nq, nkv, hd = S.q_heads, S.kv_heads, S.head_dim
        self.emb = w(S.vocab, S.hidden)
        self.layers = []
        for i in range(S.layers):
            L = _Layer()
            L.dense = i >= S.layers - self.dense_last
            L.n1 = torch.ones(S.hidden, dtype=torch.bfloat16, device=dev)
            L.n2 = torch.ones(S.hidden, dtype=torch.bfloat16, device=dev)
            L.wqkv = w((nq + 2 * nkv) * hd, S.hidden)  # [out, in]
            L.wo = w(S.hidden, nq * hd)
            L.wgu = w(2 * S.ffn, S.hidden)
            L.wdown = w(S.hidden, S.ffn)
            L.k = torch.zeros((batch, nkv, capacity, hd), dtype=torch.bfloat16, device=dev)
            L.v = torch.zeros((batch, nkv, capacity, hd), dtype=torch.bfloat16, device=dev)
            L.codes = None if L.dense else torch.zeros((batch, nkv, capacity, 32), dtype=torch.uint8, device=dev)
            self.layers.append(L)
        self.norm = torch.ones(S.hidden, dtype=torch.bfloat16, device=dev)
        self.lm_head = w(S.vocab, S.hidden)
        self.inv_freq = 1.0 / (S.rope_theta ** (torch.arange(0, hd, 2, device=dev, dtype=torch.float32) / hd))
        # step state (device): next input token, current length, and scratch
        self.tokens = torch.zeros(batch, dtype=torch.int64, device=dev)
        self.kv_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.new_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        # host-side bound on the longest sequence: a step (or a graph replay)
        # that would append past the capacity is refused before it is issued
        self.len_hi = 0
        self.attn_out = torch.empty((batch, nq, hd), dtype=torch.float32, device=dev)
        self.x = torch.empty((batch, S.hidden), dtype=torch.bfloat16, device=dev)    # residual stream
        self.h = torch.empty((batch, S.hidden), dtype=torch.bfloat16, device=dev)    # normed input of a GEMM
        self.q = torch.empty((batch, nq, hd), dtype=torch.bfloat16, device=dev)
        self.act = torch.empty((batch, S.ffn), dtype=torch.bfloat16, device=dev)
        self.ws = None
        if any(not L.dense for L in self.layers):
            self.ws = alloc_workspace(decode_workspace_size(batch, nq, nkv, capacity, budget), dev)
        self.ws_dense = None
        if any(L.dense for L in self.layers):
            self.ws_dense = alloc_workspace(dense_workspace_size(batch, nq, nkv, capacity), dev)

    # ---- cache set-up (stands in for a prefill: latency does not depend on the values)
    def fill_cache(self, lengths, seed: int = 1):
        """Random K/V for positions < lengths[b] (per-channel log-normal scales,
        as the synthetic workloads draw them) and their codes; sets the lengths."""
        from . import encode_keys
        S = self.shape
        g = torch.Generator(device=self.device)
        g.manual_seed(seed)
        lens = torch.as_tensor(lengths, dtype=torch.int32, device=self.device)
        for L in self.layers:
            for t in (L.k, L.v):
                sc = torch.exp(torch.randn((self.B, S.kv_heads, 1, S.head_dim), generator=g, device=self.device))
                for b in range(self.B):
                    n = int(lengths[b])
                    t[b, :, :n] = (torch.randn((S.kv_heads, n, S.head_dim), generator=g, device=self.device)
                                   * sc[b]).to(torch.bfloat16)
                    t[b, :, n:] = 0
            if L.codes is not None:
                encode_keys(L.k, lens, L.codes, num_q_heads=S.q_heads)
        self.kv_len.copy_(lens)
        self.len_hi = int(max(lengths)) if len(lengths) else 0
        self.tokens.random_(0, S.vocab, generator=g)

    # ---- one decode step
    def use(self, attention: str, dense_last: int = 0):
        """Switch the attention of later steps (same weights and caches): every
        layer keeps its codes, so any mix can be timed on one model."""
        if attention not in ("adamas", "dense"):
            raise ValueError("attention must be 'adamas' or 'dense'")
        if attention == "adamas" and any(L.codes is None for L in self.layers[:self.shape.layers - dense_last]):
            raise ValueError("layers built dense keep no codes")
        self.attention = attention
        self.dense_last = self.shape.layers if attention == "dense" else dense_last
        for i, L in enumerate(self.layers):
            L.dense = i >= self.shape.layers - self.dense_last
        S = self.shape
        if self.ws is None and any(not L.dense for L in self.layers):
            self.ws = alloc_workspace(decode_workspace_size(self.B, S.q_heads, S.kv_heads, self.cap, self.budget),
                                      self.device)
        if self.ws_dense is None and any(L.dense for L in self.layers):
            self.ws_dense = alloc_workspace(dense_workspace_size(self.B, S.q_heads, S.kv_heads, self.cap),
                                            self.device)

    def _attend(self, L, q, sel):
        if L.dense:
            dense_decode_attention(q, L.k, L.v, self.new_len, self.scale, self.attn_out, self.ws_dense)
        elif self.sink is None and self.recent is None:
            decode_step(q, L.k, L.v, L.codes, self.new_len, self.budget, self.scale, self.attn_out, self.ws,
                        sel_idx=sel, append=True)
        else:
            decode_step(q, L.k, L.v, L.codes, self.new_len, self.budget, self.scale, self.attn_out, self.ws,
                        sel_idx=sel, append=True, sink=self.sink, recent=self.recent)

    def reserve(self, n: int):
        """Account for n more appended tokens; raises before any would pass the
        cache capacity (the caches hold positions < capacity)."""
        if self.len_hi + n > self.cap:
            raise RuntimeError("decode past the cache capacity: longest sequence %d + %d tokens > capacity %d"
                               % (self.len_hi, n, self.cap))
        self.len_hi += n

    def state(self):
        """(tokens, lengths, host bound) to restore() later (device copies)."""
        return self.tokens.clone(), self.kv_len.clone(), self.len_hi

    def restore(self, st):
        self.tokens.copy_(st[0])
        self.kv_len.copy_(st[1])
        self.len_hi = st[2]

    def step(self):
        """Append one token to every sequence: returns the next tokens (device, [B])."""
        self.reserve(1)
        return self._step()

    def _step(self):
        S, B = self.shape, self.B
        nq = S.q_heads
        torch.add(self.kv_len, 1, out=self.new_len)
        torch.index_select(self.emb, 0, self.tokens, out=self.x)
        delta = None  # the previous layer's MLP output, added with the next norm
        for L in self.layers:
            llama_glue.add_rmsnorm(self.x, delta, self.x, L.n1, self.h, S.eps)
            qkv = F.linear(self.h, L.wqkv)
            llama_glue.rope_append(qkv, self.kv_len, self.inv_freq, self.q, L.k, L.v)
            sel = None
            if self.trace is not None and not L.dense:
                sel = torch.empty((B, nq, self.budget), dtype=torch.int32, device=self.device)
            self._attend(L, self.q, sel)
            if self.trace is not None:
                self.trace.append(dict(dense=L.dense, q=self.q.clone(), k=L.k.clone(), v=L.v.clone(),
                                       codes=None if L.codes is None else L.codes.clone(),
                                       kv_len=self.new_len.clone(), out=self.attn_out.clone(), sel=sel))
            o = F.linear(self.attn_out.view(B, nq * S.head_dim).to(torch.bfloat16), L.wo)
            llama_glue.add_rmsnorm(self.x, o, self.x, L.n2, self.h, S.eps)
            llama_glue.silu_mul(F.linear(self.h, L.wgu), self.act)
            delta = F.linear(self.act, L.wdown)
        llama_glue.add_rmsnorm(self.x, delta, self.x, self.norm, self.h, S.eps)
        logits = F.linear(self.h, self.lm_head)
        torch.argmax(logits, dim=-1, out=self.tokens)
        self.kv_len.copy_(self.new_len)
        return self.tokens

    def capture(self, steps_per_graph: int = 1):
        """A HIP graph of `steps_per_graph` decode steps (torch.cuda.graph),
        wrapped so that each replay() advances every sequence by that many tokens
        and is refused (RuntimeError) before it would pass the cache capacity."""
        if self.len_hi + steps_per_graph > self.cap:
            raise RuntimeError("a graph of %d steps cannot run: longest sequence %d, capacity %d"
                               % (steps_per_graph, self.len_hi, self.cap))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # warm-up outside the graph (allocator, library handles)
            saved = (self.tokens.clone(), self.kv_len.clone())
            self._step()
            self.tokens.copy_(saved[0])
            self.kv_len.copy_(saved[1])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps_per_graph):
                self._step()
        torch.cuda.synchronize()
        return _GuardedGraph(self, g, steps_per_graph)


class _GuardedGraph:
    """A captured decode graph whose replays are counted against the cache capacity."""

    def __init__(self, model, graph, steps):
        self.model, self.graph, self.steps = model, graph, steps

    def replay(self):
        self.model.reserve(self.steps)
        self.graph.replay()
