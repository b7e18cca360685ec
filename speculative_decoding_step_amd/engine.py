"""Device-memory owner and call sequencer for the EAGLE-3 step (no arithmetic here).

PyTorch allocates the weights, KV caches, workspace and step buffers on the
GPU and provides the stream; every step of the method runs in libeagle3.so,
reached through :mod:`binding`.  The seeded weights are generated directly on
the device by :mod:`synth` (bit-identical to the host twins the oracle uses).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B
from . import configs, synth


@dataclass
class Spec:
    mode: str          # "greedy_tree" | "sample_chain" | "sample_tree"
    depth: int
    topk: int
    n_nodes: int
    temperature: float = 0.0
    draft_greedy: bool = False

    @classmethod
    def of(cls, w: configs.Workload) -> "Spec":
        return cls(w.mode, w.depth, w.topk, w.n_nodes, w.temperature, w.draft_greedy)


def _ptr(t):
    return None if t is None else t.data_ptr()


class Engine:
    def __init__(self, ms: configs.ModelShape, spec: Spec, batch: int, max_seq: int, target_seed: int,
                 head_seed: int, max_rows: int | None = None, device: str = "cuda", sigma: float = 0.02,
                 prefill_chunk: int = 512, weights: dict | None = None, block_size: int = 0, page_seed: int = 0):
        """block_size > 0 makes the KV caches paged: pools of blocks of that many
        positions, each sequence's blocks drawn from a seeded shuffle of the pool
        (three spare blocks), so every K/V access goes through the block table."""
        if not torch.cuda.is_available():
            raise RuntimeError("the EAGLE-3 engine needs a ROCm GPU (gfx950)")
        self.ms, self.spec, self.B, self.max_seq = ms, spec, batch, max_seq
        self.dev = torch.device(device)
        self.bf16 = ms.dtype == "bf16"
        self.tdt = torch.bfloat16 if self.bf16 else torch.float32
        self.rows = spec.n_nodes + 1
        self.W = spec.depth + 1
        self.prefill_chunk = prefill_chunk
        self.max_rows = max_rows or max(batch * self.rows, batch * self.W, batch * spec.topk, prefill_chunk)
        d, V = ms.d, ms.vocab

        # ---- weights (seeded, generated on the device; linear weights are then
        # converted to the library's packed layout, see eagle3_pack_linear).
        # A caller-supplied `weights` dict must already hold packed matrices.
        self.stream = torch.cuda.current_stream(self.dev)
        self.w = weights if weights is not None else {}
        if weights is None:
            for seed, specs in ((target_seed, configs.target_tensor_specs(ms)),
                                (head_seed, configs.head_tensor_specs(ms))):
                for name, shp, kind in specs:
                    t = self._tensor(seed, name, shp, kind, sigma)
                    if kind == "mat" and name != "embed":
                        t = self._pack(t)
                    self.w[name] = t
        w = self.w
        self.shape = B.Shape(ms.n_layers, d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, V, ms.rope_theta,
                             ms.eps, B.BF16 if self.bf16 else B.F32, (C.c_int32 * 3)(*ms.taps), ms.draft_vocab)
        modes = {"greedy_tree": B.GREEDY_TREE, "sample_chain": B.SAMPLE_CHAIN, "sample_tree": B.SAMPLE_TREE}
        self.cfg = B.SpecCfg(modes[spec.mode], spec.depth, spec.topk,
                             spec.n_nodes, spec.temperature, int(spec.draft_greedy))
        self._layers = (B.LayerWeights * ms.n_layers)()
        for l in range(ms.n_layers):
            for f in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down"):
                setattr(self._layers[l], f, w[f"l{l}.{f}"].data_ptr())
        self.tw = B.TargetWeights(w["embed"].data_ptr(), self._layers, w["final_norm"].data_ptr(),
                                  w["lm_head"].data_ptr())
        if ms.draft_vocab > 0:  # reduced draft vocabulary: draft-owned head + ascending map to target ids
            w["h.d2t"] = torch.as_tensor(configs.d2t_np(ms, head_seed), device=self.dev)
        hw = B.HeadWeights()
        for f, _ in B.HeadWeights._fields_:
            t = w.get("h." + f)
            setattr(hw, f, None if t is None else t.data_ptr())
        self.hw = hw

        # ---- caches, workspace, context
        self.block_size = block_size
        if block_size:
            bps = -(-max_seq // block_size)
            max_seq = self.max_seq = bps * block_size
            self.n_blocks = batch * bps + 3
            ids = np.random.default_rng(page_seed).permutation(self.n_blocks)[:batch * bps]
            self.block_table = torch.as_tensor(ids.reshape(batch, bps).astype(np.int32), device=self.dev)
            self.pages = B.KvPages(block_size, self.n_blocks, bps, self.block_table.data_ptr())
            kvt, kvd = B.eagle3_paged_kv_bytes(self.shape, block_size, self.n_blocks)
        else:
            kvt, kvd = B.eagle3_kv_bytes(self.shape, batch, max_seq)
        # zero-filled, so slots no call has written compare equal between engines (and hold finite values)
        self.kv_target = torch.zeros(kvt, dtype=torch.uint8, device=self.dev)
        self.kv_draft = torch.zeros(kvd, dtype=torch.uint8, device=self.dev)
        wsb = B.eagle3_workspace_bytes(self.shape, self.cfg, batch, self.max_rows, max_seq)
        self.workspace = torch.empty(wsb, dtype=torch.uint8, device=self.dev)
        if block_size:
            self.ctx = B.eagle3_create_paged(self.shape, self.cfg, self.tw, self.hw, batch, self.max_rows, self.pages,
                                             self.workspace.data_ptr(), wsb, self.kv_target.data_ptr(),
                                             self.kv_draft.data_ptr(), self.stream.cuda_stream)
        else:
            self.ctx = B.eagle3_create(self.shape, self.cfg, self.tw, self.hw, batch, self.max_rows, max_seq,
                                       self.workspace.data_ptr(), wsb, self.kv_target.data_ptr(),
                                       self.kv_draft.data_ptr(), self.stream.cuda_stream)
        self.n_draft = None

        # ---- step state
        i32 = dict(dtype=torch.int32, device=self.dev)
        R, Wd = self.rows, self.W
        self.seq_lens = torch.zeros(batch, **i32)
        self.new_len = torch.zeros(batch, **i32)
        self.aux_new = torch.zeros(batch, Wd, 3 * d, dtype=self.tdt, device=self.dev)
        self.next_tok = torch.full((batch, Wd), -1, **i32)
        self.tokens = torch.zeros(batch, R, **i32)
        self.parents = torch.zeros(batch, R, **i32)
        self.depth = torch.zeros(batch, R, **i32)
        self.pos = torch.zeros(batch, R, **i32)
        self.mask = torch.zeros(batch, R, dtype=torch.int64, device=self.dev)
        self.score = torch.zeros(batch, R, dtype=torch.float32, device=self.dev)
        self.chain = spec.mode == "sample_chain"
        self.sampling = spec.mode in ("sample_chain", "sample_tree")
        # acceptance uniforms per sequence: one per draft + the final draw (chain), one per (depth, child) + the
        # final draw (tree)
        self.n_u_accept = spec.depth + 1 if self.chain else spec.depth * spec.topk + 1
        self.q = torch.zeros(batch, spec.depth, V, dtype=torch.float32, device=self.dev) if self.chain else None
        self.logits = torch.zeros(batch * R, V, dtype=torch.float32, device=self.dev) if self.sampling else None
        self.argmax = torch.zeros(batch * R, **i32)
        self.margin = torch.zeros(batch * R, dtype=torch.float32, device=self.dev)
        self.aux_tree = torch.zeros(batch, R, 3 * d, dtype=self.tdt, device=self.dev)
        self.path = torch.zeros(batch, Wd, **i32)
        self.path_len = torch.zeros(batch, **i32)
        self.next_root = torch.zeros(batch, **i32)
        self.emitted = torch.zeros(batch, Wd, **i32)
        self.u_draft = torch.zeros(batch, spec.depth, dtype=torch.float32, device=self.dev)
        self.u_accept = torch.zeros(batch, self.n_u_accept, dtype=torch.float32, device=self.dev)
        self.step_idx = 0

    def _tensor(self, seed, name, shape, kind, sigma):
        if kind == "norm":
            return torch.ones(shape, dtype=self.tdt, device=self.dev)
        return synth.normal_t(seed, name, shape, self.dev, sigma, self.ms.dtype)

    def _pack(self, t):
        """The packed copy of a row-major linear weight [out, in] (the original is dropped)."""
        rows = (t.shape[0] + 15) // 16 * 16 if self.bf16 else t.shape[0]
        p = torch.empty((rows, t.shape[1]), dtype=t.dtype, device=t.device)
        B.eagle3_pack_linear(B.BF16 if self.bf16 else B.F32, t.data_ptr(), p.data_ptr(), t.shape[0], t.shape[1],
                             self.stream.cuda_stream)
        return p

    def close(self):
        if getattr(self, "ctx", None):
            torch.cuda.synchronize(self.dev)
            B.eagle3_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def device_status(self) -> int:
        return B.eagle3_device_status(self.ctx)

    def set_draft_lengths(self, n_draft=None):
        """Per-request draft lengths ([B] ints, read at every later step; None = the full budget).

        Once set, the device buffer stays the same (a captured step keeps reading it):
        None then refills it with the full budget."""
        if n_draft is None:
            if self.n_draft is None:
                B.eagle3_set_draft_lengths(self.ctx, None)
            else:
                self.n_draft.fill_(self.spec.n_nodes)
            return
        nd = torch.as_tensor(np.asarray(n_draft, dtype=np.int32), device=self.dev)
        if self.n_draft is None:
            self.n_draft = nd.clone()
            B.eagle3_set_draft_lengths(self.ctx, self.n_draft.data_ptr())
        else:
            self.n_draft.copy_(nd)  # same buffer: a captured step sees the new lengths

    def record_draft_logits(self, on: bool = True):
        """Make every later draft also write its draft-logits table (a parity output,
        eagle3_set_draft_logits_out): self.draft_table [B, 1 + E, V_d] float32, row 0
        the root's draft row, row 1 + r expansion row r in creation order."""
        if on:
            s = self.spec
            e = (s.depth - 1) * s.topk  # a chain has topk 1
            vd = self.ms.draft_vocab or self.ms.vocab
            self.draft_table = torch.full((self.B, 1 + e, vd), float("nan"), dtype=torch.float32, device=self.dev)
            B.eagle3_set_draft_logits_out(self.ctx, self.draft_table.data_ptr())
        else:
            B.eagle3_set_draft_logits_out(self.ctx, None)
            self.draft_table = None

    def kv_logical(self, which: str = "target"):
        """A cache as [L, 2, B, Hkv, max_seq, hd] in position order: a view of a
        contiguous cache, a gather through the block table of a paged one."""
        ms = self.ms
        L = ms.n_layers if which == "target" else 1
        buf = self.kv_target if which == "target" else self.kv_draft
        if not self.block_size:
            return buf.view(self.tdt).view(L, 2, self.B, ms.n_kv_heads, self.max_seq, ms.head_dim)
        bs = self.block_size
        pool = buf.view(self.tdt).view(L, 2, self.n_blocks, ms.n_kv_heads, bs, ms.head_dim)
        g = pool[:, :, self.block_table.long()]                  # [L, 2, B, bps, Hkv, bs, hd]
        return g.permute(0, 1, 2, 4, 3, 5, 6).reshape(L, 2, self.B, ms.n_kv_heads, self.max_seq, ms.head_dim)

    # ------------------------------------------------------------------ prefill
    def prefill(self, prompts, u_root=None):
        """Target prefill (causal, chunked), root draw, draft prefill of positions [0, P-1).

        Leaves the step state ready: seq_lens = P, one catch-up row (position
        P - 1, paired with the root)."""
        d, V = self.ms.d, self.ms.vocab
        i32 = dict(dtype=torch.int32, device=self.dev)
        ch = self.prefill_chunk
        roots = torch.zeros(len(prompts), **i32)
        lm = torch.zeros(1, V, dtype=torch.float32, device=self.dev)
        start = torch.zeros(1, **i32)
        for b, prompt in enumerate(prompts):
            P = len(prompt)
            assert P + self.rows + (self.spec.depth - 1) * self.spec.topk <= self.max_seq
            toks = torch.as_tensor(np.asarray(prompt, dtype=np.int32), device=self.dev)
            aux = torch.empty(P, 3 * d, dtype=self.tdt, device=self.dev)
            for s in range(0, P, ch):
                e = min(P, s + ch)
                start.fill_(s)
                last = e == P
                B.eagle3_verify_tree(self.ctx, b, 1, _ptr(start), e - s, _ptr(toks[s:e]), None, None,
                                     B.LM_LAST if last else B.LM_NONE, _ptr(lm) if last else None, None, None,
                                     _ptr(aux[s:e]))
            if self.spec.temperature == 0:
                B.eagle3_sample(self.ctx, 1, _ptr(lm), 0.0, None, _ptr(roots[b:b + 1]))
            else:
                B.eagle3_sample(self.ctx, 1, _ptr(lm), self.spec.temperature, _ptr(u_root[b:b + 1]),
                                _ptr(roots[b:b + 1]))
            for s in range(0, P - 1, ch):
                e = min(P - 1, s + ch)
                start.fill_(s)
                B.eagle3_draft_prefill(self.ctx, b, 1, _ptr(start), e - s, _ptr(aux[s:e]), _ptr(toks[s + 1:e + 1]))
            self.seq_lens[b] = P
            self.new_len[b] = 1
            self.aux_new[b, 0] = aux[P - 1]
            self.next_tok[b, 0] = roots[b]
        return roots

    # --------------------------------------------------------------------- step
    def set_uniforms(self, u_draft=None, u_accept=None):
        if u_draft is not None:
            self.u_draft.copy_(u_draft)
        if u_accept is not None:
            self.u_accept.copy_(u_accept)

    def draft(self):
        B.eagle3_draft_tree(self.ctx, self.B, _ptr(self.seq_lens), _ptr(self.new_len), _ptr(self.aux_new),
                            _ptr(self.next_tok), _ptr(self.u_draft) if self.chain else None, _ptr(self.tokens),
                            _ptr(self.parents), _ptr(self.depth), _ptr(self.pos), _ptr(self.mask), _ptr(self.score),
                            _ptr(self.q))

    def verify(self):
        B.eagle3_verify_tree(self.ctx, 0, self.B, _ptr(self.seq_lens), self.rows, _ptr(self.tokens), _ptr(self.pos),
                             _ptr(self.mask), B.LM_ALL, _ptr(self.logits), _ptr(self.argmax), _ptr(self.margin),
                             _ptr(self.aux_tree))

    def accept(self):
        B.eagle3_accept(self.ctx, self.B, self.rows, _ptr(self.tokens), _ptr(self.parents), _ptr(self.argmax),
                        _ptr(self.logits), _ptr(self.q), _ptr(self.u_accept) if self.sampling else None,
                        _ptr(self.path), _ptr(self.path_len), _ptr(self.next_root), _ptr(self.emitted))

    def compact(self):
        B.eagle3_compact_kv(self.ctx, self.B, _ptr(self.seq_lens), self.rows, _ptr(self.path), _ptr(self.path_len),
                            _ptr(self.tokens), _ptr(self.next_root), _ptr(self.aux_tree), _ptr(self.aux_new),
                            _ptr(self.next_tok), _ptr(self.new_len))

    def step(self):
        self.draft()
        self.verify()
        self.accept()
        self.compact()
        self.step_idx += 1

    def capture(self):
        """Capture one step (draft, verify, accept, compact) into a HIP graph.

        Replays run the same kernels on the device state current at replay
        time; call replay() instead of step()."""
        cap = torch.cuda.Stream(self.dev)
        cap.wait_stream(self.stream)
        g = torch.cuda.CUDAGraph()
        B.eagle3_set_stream(self.ctx, cap.cuda_stream)
        try:
            with torch.cuda.graph(g, stream=cap):
                self.draft()
                self.verify()
                self.accept()
                self.compact()
        finally:
            B.eagle3_set_stream(self.ctx, self.stream.cuda_stream)
        self.stream.wait_stream(cap)
        self.graph = g
        return g

    def capture_call(self, fn):
        """Capture one call sequence fn() into its own HIP graph (the same way as the
        step); returns the graph.  For timing a part of the step alone, e.g. the
        verify pass, whose replays are idempotent."""
        cap = torch.cuda.Stream(self.dev)
        cap.wait_stream(self.stream)
        g = torch.cuda.CUDAGraph()
        B.eagle3_set_stream(self.ctx, cap.cuda_stream)
        try:
            with torch.cuda.graph(g, stream=cap):
                fn()
        finally:
            B.eagle3_set_stream(self.ctx, self.stream.cuda_stream)
        self.stream.wait_stream(cap)
        return g

    def replay(self):
        self.graph.replay()
        self.step_idx += 1

    # ------------------------------------------------------------------ drivers
    def generate(self, prompts, max_new: int, uniforms=None):
        """Speculative decoding of every sequence until each has max_new tokens.

        uniforms: callable(kind, step) -> tensor for sampling ("root", "draft",
        "accept"), or None for greedy.  Returns (tokens per sequence, path
        lengths per step)."""
        roots = self.prefill(prompts, None if uniforms is None else uniforms("root", 0))
        out = [[] for _ in prompts]
        lens = []
        s = 0
        while min(len(o) for o in out) + 1 < max_new:
            if uniforms is not None:
                self.set_uniforms(uniforms("draft", s), uniforms("accept", s))
            self.step()
            em = self.emitted.cpu().numpy()
            pl = self.path_len.cpu().numpy()
            for b in range(self.B):
                out[b] += [int(t) for t in em[b, :pl[b]]]
            lens.append(pl.copy())
            s += 1
        nr = self.next_tok.cpu().numpy()
        nl = self.new_len.cpu().numpy()
        res = []
        for b in range(self.B):
            last = int(nr[b, nl[b] - 1]) if s else int(roots[b])
            res.append((out[b] + [last])[:max_new])
        return res, lens
