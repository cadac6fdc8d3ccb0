"""One MLA decode step for one layer, as the library calls in order: absorb
the query and append the new tokens to the paged cache (one call), attend over
the latent cache, then merge the key splits and project back to per-head
outputs (one call, mla_combine_up_proj, when the attention was split; else the
up-projection alone).
`run_from_hidden` starts one step earlier, from the hidden states: the
down-projections with the append, and the query up-projection with the
absorb, replace the first two calls.

Buffers are allocated once per shape; `run()` only enqueues library calls on
the current stream.
"""
from __future__ import annotations

import torch

from . import binding as B


class DecodeStep:
    def __init__(self, dims: B.Dims, n_seq: int, q_per_seq: int, max_blocks: int, num_splits: int = 0,
                 device="cuda", keep_latent: bool = True):
        """keep_latent: the merged latent rows are written to o_latent (returned by run);
        without it the fused merge does not write them and run returns None for o_latent."""
        self.d, self.n_seq, self.q_per_seq = dims, n_seq, q_per_seq
        self.keep_latent = keep_latent
        self.max_blocks, self.num_splits = max_blocks, num_splits
        at = B.act_torch_dtype(dims)
        n_tok = n_seq * q_per_seq
        H = dims.n_heads
        self.q_abs = torch.empty((n_seq, q_per_seq, H, dims.d_c + dims.d_rope), dtype=at, device=device)
        self.o_latent = torch.empty((n_seq, q_per_seq, H, dims.d_c), dtype=at, device=device)
        self.lse = torch.empty((n_seq, q_per_seq, H), dtype=torch.float32, device=device)
        self.out = torch.empty((n_tok, H, dims.d_v), dtype=at, device=device)
        ws = B.decode_workspace_bytes(dims, n_seq, q_per_seq, max_blocks, num_splits)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.needs_combine = B.decode_needs_combine(dims, n_seq, q_per_seq, max_blocks, num_splits)
        # the fused merge + up-projection runs one work-group per (head, 32 query rows): it
        # pays off when that fills the chip, else the two calls (many small work-groups) win
        cus = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count \
            if torch.cuda.is_available() else 256
        self.fuse_merge = self.needs_combine and H * ((n_tok + 31) // 32) >= cus

    def _finish(self, seqlens, w_uv, gate, stream):
        """The split merge and the up-projection: one launch (mla_combine_up_proj) when decode
        left partials and the fused kernel fills the chip, else mla_combine (if needed) and
        mla_up_proj."""
        d = self.d
        n_tok = self.n_seq * self.q_per_seq
        if self.fuse_merge:
            B.combine_up_proj(d, seqlens, self.max_blocks, self.workspace, self.o_latent, self.lse, w_uv, out=self.out,
                              num_splits=self.num_splits, gate=gate, write_latent=self.keep_latent, stream=stream)
            return
        if self.needs_combine:
            B.combine(d, seqlens, self.max_blocks, self.workspace, self.o_latent, self.lse, self.num_splits,
                      stream=stream)
        B.up_proj(d, self.o_latent.view(n_tok, d.n_heads, d.d_c), w_uv, out=self.out, stream=stream, gate=gate)

    def _latent(self):
        """o_latent, or None when the merged rows were not written back."""
        return None if self.fuse_merge and not self.keep_latent else self.o_latent

    def run(self, *, q_nope, q_rope, q_pos, new_c_kv, new_k_rope, new_seq_id, new_pos, block_table, seqlens,
            pool, w_uk, w_uv, gate=None, stream=None):
        """q_nope/q_rope [n_seq*q_per_seq, H, *]; q_pos [n_seq*q_per_seq]; new_* the tokens to append;
        gate [n_seq*q_per_seq, H, d_v] (optional): output-gate logits of gated MLA."""
        d = self.d
        n_tok = self.n_seq * self.q_per_seq
        if new_c_kv is not None and new_c_kv.shape[0] > 0:   # the absorb and the append in one launch
            B.absorb_append(d, q_nope, q_rope, q_pos, w_uk, new_c_kv, new_k_rope, new_seq_id, new_pos, block_table,
                            pool, q_abs=self.q_abs.view(n_tok, d.n_heads, -1), stream=stream)
        else:
            B.absorb_q(d, q_nope, q_rope, q_pos, w_uk, q_abs=self.q_abs.view(n_tok, d.n_heads, -1), stream=stream)
        B.decode(d, self.q_abs, pool, block_table, seqlens, self.num_splits, self.workspace, self.o_latent,
                 self.lse, stream=stream)
        self._finish(seqlens, w_uv, gate, stream)
        return self.out, self._latent(), self.lse

    def run_from_hidden(self, *, h, w_down, d_cq, w_uq, q_pos, new_seq_id, new_pos, block_table, seqlens, pool,
                        w_uk, w_uv, gate=None, stream=None):
        """h [n_seq*q_per_seq, d_model] are the hidden states of the new tokens (one per query row);
        w_down [d_cq + d_c + d_rope, d_model] = [W_DQ; W_DKV; W_KR]; w_uq [H, d_nope + d_rope, d_cq]."""
        d = self.d
        n_tok = self.n_seq * self.q_per_seq
        d_model = h.shape[1]
        key = (d_model, d_cq)
        if getattr(self, "_up_key", None) != key:
            dev = h.device
            self._c_q = torch.empty((n_tok, d_cq), dtype=B.act_torch_dtype(d), device=dev)
            self._ws_down = torch.empty(max(B.project_down_workspace_bytes(d, n_tok, d_model, d_cq), 1),
                                        dtype=torch.uint8, device=dev)
            self._ws_q = torch.empty(max(B.absorb_from_latent_workspace_bytes(d, n_tok, d_cq), 1), dtype=torch.uint8,
                                     device=dev)
            self._up_key = key
        B.project_down(d, h, w_down, d_cq, new_seq_id, new_pos, block_table, pool, c_q=self._c_q,
                       workspace=self._ws_down, stream=stream)
        B.absorb_from_latent(d, self._c_q, w_uq, q_pos, w_uk, q_abs=self.q_abs.view(n_tok, d.n_heads, -1),
                             workspace=self._ws_q, stream=stream)
        B.decode(d, self.q_abs, pool, block_table, seqlens, self.num_splits, self.workspace, self.o_latent,
                 self.lse, stream=stream)
        self._finish(seqlens, w_uv, gate, stream)
        return self.out, self._latent(), self.lse
