"""Device set-up of the synthetic decode workloads and the five-call decode step.

Used by the GPU tests, ``bench.py`` and ``__graft_entry__.smoke()``.  All
numbers come from the seeded generator in ``inputs.py`` (filled on the device
by its twin kernel); all compute goes through the C ABI in ``__init__.py``.
"""
from __future__ import annotations

import numpy as np

from . import (make_dims, mla_absorb_out, mla_absorb_q, mla_absorb_q_append, mla_absorb_q_cq,
               mla_absorb_q_append_fp8, mla_absorb_q_append_fp8_workspace_bytes, mla_append_latent,
               mla_append_latent_fp8, mla_append_workspace_bytes, mla_append_workspace_bytes_fp8,
               mla_decode_attention, mla_decode_attention_fp8, mla_decode_attention_fp8_planned,
               mla_decode_attention_planned, mla_decode_plan, mla_fp8_page_bytes, mla_merge_lse,
               mla_merge_lse_planned, mla_merge_absorb_out, mla_merge_absorb_out_workspace_bytes,
               mla_prefill_attention, mla_quantize_rows_fp8, mla_workspace_bytes,
               mla_workspace_bytes_cq)
from . import inputs as I


def fill_fp8_pool(dims, pool, key: int, chunk_rows: int = 1 << 16):
    """Fill every row of an FP8 pool (uint8 [num_pages, page_bytes]) from the fp32
    values of generator stream ``key``: physical row p takes elements
    p*row .. p*row + row-1 (as in a plain pool).  fp32 rows are generated a chunk
    at a time on the device and quantized into their slots by
    mla_quantize_rows_fp8, physical page p addressed as a one-page sequence p."""
    import torch
    P, row = dims.page_size, dims.d_latent + dims.d_rope
    pages = pool.shape[0]
    total = pages * P
    ident = torch.arange(pages, dtype=torch.int32, device=pool.device).reshape(-1, 1)
    buf = torch.empty((min(chunk_rows, total), row), dtype=torch.float32, device=pool.device)
    for r0 in range(0, total, chunk_rows):
        n = min(chunk_rows, total - r0)
        rows = buf[:n]
        I.fill_device(rows, key, 1.0, start=r0 * row)
        phys = torch.arange(r0, r0 + n, dtype=torch.int32, device=pool.device)
        mla_quantize_rows_fp8(dims, rows, (phys // P).contiguous(), (phys % P).contiguous(), ident,
                              pool)
    torch.cuda.synchronize()


class DeviceWorkload:
    """Weights, paged pool, page table, lengths and output buffers of one layer of
    a :class:`inputs.Workload`, resident in device memory."""

    def __init__(self, w: I.Workload, layer: int = 0, num_splits: int | None = None,
                 device: str = "cuda", build_cache: bool = True, outputs_from=None):
        import torch
        self.torch = torch
        self.w, self.layer = w, layer
        self.dev = torch.device(device)
        self.dims = make_dims(w.hidden, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.dtype,
                              w.page_size, w.rope_base, yarn=w.yarn or None)
        self.dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        self.S = num_splits or w.num_splits
        self.lens = I.seq_lengths(w)
        self.bt_host, self.num_pages = I.page_table(w, self.lens)
        B = w.batch
        self.seq_lens = torch.tensor(self.lens, dtype=torch.int32, device=self.dev)
        # the step's tokens: the last position of every sequence (decode), or its last
        # `chunk` positions (prefill); nq of them, token i at (q_seq[i], q_pos[i])
        self.chunk = w.chunk
        if self.chunk:
            qs = np.repeat(np.arange(B, dtype=np.int32), self.chunk)
            qp = np.concatenate([np.arange(int(L) - self.chunk, int(L), dtype=np.int32)
                                 for L in self.lens])
        else:
            qs = np.arange(B, dtype=np.int32)
            qp = (self.lens - 1).astype(np.int32)
        self.q_seq_host, self.q_pos_host = qs, qp
        self.nq = len(qs)
        self.seq_ids = torch.tensor(qs, device=self.dev)
        self.pos = torch.tensor(qp, device=self.dev)
        self.block_table = torch.tensor(self.bt_host, dtype=torch.int32, device=self.dev)
        self.weights = {}
        for name in w.weight_names:
            t = torch.empty(w.weight_shape(name), dtype=self.dt, device=self.dev)
            I.fill_device(t, I.stream_key(w.seed, name, layer), 1.0 / np.sqrt(w.fan_in(name)))
            self.weights[name] = t
        self.fp8 = w.cache == "fp8"
        if self.fp8:
            self.pool = torch.empty((self.num_pages, mla_fp8_page_bytes(self.dims)), dtype=torch.uint8,
                                    device=self.dev)
        else:
            self.pool = torch.empty((self.num_pages, w.page_size, w.row), dtype=self.dt,
                                    device=self.dev)
        if w.cache_from_h:
            L = int(self.lens.max())
            self.h_ctx = torch.empty((B, L, w.hidden), dtype=self.dt, device=self.dev)
            I.fill_device(self.h_ctx, I.stream_key(w.seed, "h_ctx", layer))
            self.h = self.h_ctx[self.seq_ids.long(), self.pos.long()].contiguous()
            self.pool.zero_()
            if build_cache:
                self.build_cache_from_h()
        else:
            self.h_ctx = None
            self.h = torch.empty((self.nq, w.hidden), dtype=self.dt, device=self.dev)
            I.fill_device(self.h, I.stream_key(w.seed, "h_dec", layer))
            if self.fp8:
                self.fill_fp8_pool()
            else:
                I.fill_device(self.pool, I.stream_key(w.seed, "pool", layer))
        nh = w.n_heads
        B = self.nq      # outputs and scratch are per step token
        # decode over a length-proportional plan (host-built, copied to the device)
        self.n_units, self.plan = 0, None
        if w.plan_units and not self.chunk:
            self.n_units, plan = mla_decode_plan(self.lens, w.page_size, w.plan_units)
            self.plan = torch.tensor(plan, dtype=torch.int32, device=self.dev)
        wsa = (mla_append_workspace_bytes_fp8 if self.fp8 else mla_append_workspace_bytes)(self.dims, B)
        self.ws_append = torch.empty(max(1, wsa), dtype=torch.uint8, device=self.dev)
        if outputs_from is not None:     # share scratch/output buffers with another layer
            for k in ("q_lat", "q_pe", "o_part", "lse_part", "o_lat", "lse", "u", "ws"):
                setattr(self, k, getattr(outputs_from, k))
            return
        f32 = torch.float32
        self.q_lat = torch.empty((B, nh, w.d_latent), dtype=f32, device=self.dev)
        self.q_pe = torch.empty((B, nh, w.d_rope), dtype=f32, device=self.dev)
        if self.plan is not None:   # partials per plan unit
            self.o_part = torch.empty((self.n_units, nh, w.d_latent), dtype=f32, device=self.dev)
            self.lse_part = torch.empty((self.n_units, nh), dtype=f32, device=self.dev)
        else:
            self.o_part = torch.empty((B, self.S, nh, w.d_latent), dtype=f32, device=self.dev)
            self.lse_part = torch.empty((B, self.S, nh), dtype=f32, device=self.dev)
        if self.S == 1 and self.plan is None:
            # one split: the merge is the identity, so the split's output (same layout)
            # is the step's o_lat / lse and merge() has nothing to do
            self.o_lat = self.o_part.view(B, nh, w.d_latent)
            self.lse = self.lse_part.view(B, nh)
        else:
            self.o_lat = torch.empty((B, nh, w.d_latent), dtype=f32, device=self.dev)
            self.lse = torch.empty((B, nh), dtype=torch.float32, device=self.dev)
        self.u = torch.empty((B, w.hidden), dtype=f32, device=self.dev)
        ws_bytes = max(mla_workspace_bytes(self.dims, B),
                       mla_merge_absorb_out_workspace_bytes(self.dims, B))
        if w.d_cq:
            ws_bytes = max(ws_bytes, mla_workspace_bytes_cq(self.dims, w.d_cq, B))
        if self.fp8:
            ws_bytes = max(ws_bytes, mla_absorb_q_append_fp8_workspace_bytes(self.dims, B))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.dev)

    def fill_fp8_pool(self):
        """Every row of the FP8 pool from the fp32 values of stream "pool"."""
        fill_fp8_pool(self.dims, self.pool, I.stream_key(self.w.seed, "pool", self.layer))

    def build_cache_from_h(self):
        """Append rows 0..L_b-2 (decode) or 0..L_b-chunk-1 (prefill) of every sequence
        from h_ctx (the context before the step's tokens) through the append call."""
        torch = self.torch
        B, L = self.h_ctx.shape[0], self.h_ctx.shape[1]
        seqs, poss = [], []
        for b in range(B):
            n = int(self.lens[b]) - max(1, self.chunk)
            seqs.append(np.full(n, b, dtype=np.int32))
            poss.append(np.arange(n, dtype=np.int32))
        seq = torch.tensor(np.concatenate(seqs), device=self.dev)
        pos = torch.tensor(np.concatenate(poss), device=self.dev)
        rows = self.h_ctx.reshape(B * L, -1)[(seq.long() * L + pos.long())].contiguous()
        append = mla_append_latent_fp8 if self.fp8 else mla_append_latent
        append(self.dims, rows, self.weights["w_dkv"], self.weights["w_kr"], seq, pos,
               self.block_table, self.pool)

    # ---- the five calls of one decode step ------------------------------
    def absorb_q(self):
        W = self.weights
        if self.w.d_cq:
            mla_absorb_q_cq(self.dims, self.h, W["w_dq"], W["w_uq"], W["w_qr"], W["w_uk"],
                            self.pos, self.q_lat, self.q_pe, self.ws)
        else:
            mla_absorb_q(self.dims, self.h, W["w_q"], W["w_qr"], W["w_uk"], self.pos, self.q_lat,
                         self.q_pe, self.ws)

    def append(self):
        append = mla_append_latent_fp8 if self.fp8 else mla_append_latent
        append(self.dims, self.h, self.weights["w_dkv"], self.weights["w_kr"], self.seq_ids,
               self.pos, self.block_table, self.pool, self.ws_append)

    def absorb_q_append(self):
        """absorb_q and append of the step's tokens in one call (uncompressed
        query; any pool format): one projection reads h for both."""
        W = self.weights
        fused = mla_absorb_q_append_fp8 if self.fp8 else mla_absorb_q_append
        fused(self.dims, self.h, W["w_q"], W["w_qr"], W["w_uk"], W["w_dkv"], W["w_kr"], self.pos,
              self.seq_ids, self.block_table, self.pool, self.q_lat, self.q_pe, self.ws)

    def query_and_append(self):
        """The step's first two calls: fused for the uncompressed query, else
        absorb_q then append."""
        if self.w.d_cq:
            self.absorb_q()
            self.append()
        else:
            self.absorb_q_append()

    def attention(self):
        if self.chunk:
            mla_prefill_attention(self.dims, self.q_lat, self.q_pe, self.pool, self.block_table,
                                  self.seq_ids, self.pos, self.o_part, self.lse_part, fp8=self.fp8)
            return
        if self.plan is not None:
            attend = mla_decode_attention_fp8_planned if self.fp8 else mla_decode_attention_planned
            attend(self.dims, self.q_lat, self.q_pe, self.pool, self.block_table, self.plan,
                   self.n_units, self.o_part, self.lse_part)
            return
        attend = mla_decode_attention_fp8 if self.fp8 else mla_decode_attention
        attend(self.dims, self.q_lat, self.q_pe, self.pool, self.block_table, self.seq_lens,
               self.o_part, self.lse_part)

    def merge(self):
        if self.plan is not None:
            mla_merge_lse_planned(self.dims, self.o_part, self.lse_part, self.plan, self.n_units,
                                  self.o_lat, self.lse)
            return
        if self.S == 1:
            return              # o_lat / lse are the single split's output
        mla_merge_lse(self.dims, self.o_part, self.lse_part, self.o_lat, self.lse)

    def absorb_out(self):
        mla_absorb_out(self.dims, self.o_lat, self.weights["w_uv"], self.weights["w_o"], self.u,
                       self.ws)

    def merge_absorb_out(self):
        """merge then absorb_out as one call (the merged o_lat is not stored; lse is)."""
        if self.plan is not None:
            mla_merge_absorb_out(self.dims, self.o_part, self.lse_part, self.weights["w_uv"],
                                 self.weights["w_o"], self.u, self.ws, lse=self.lse,
                                 plan=self.plan, n_units=self.n_units)
            return
        # one split: lse is the split's own (a view of lse_part), nothing to write
        mla_merge_absorb_out(self.dims, self.o_part, self.lse_part, self.weights["w_uv"],
                             self.weights["w_o"], self.u, self.ws,
                             lse=None if self.S == 1 else self.lse)

    def merge_o_lat(self):
        """Store the merged o_lat of the last attention (the step's fused merge +
        absorb_out does not): mla_merge_lse of the same partials, lse left as the
        step wrote it."""
        if self.plan is not None:
            mla_merge_lse_planned(self.dims, self.o_part, self.lse_part, self.plan, self.n_units,
                                  self.o_lat, None)
        elif self.S > 1:
            mla_merge_lse(self.dims, self.o_part, self.lse_part, self.o_lat, None)

    def step(self):
        """absorb_q -> append (decode token at L-1) -> attention -> merge -> absorb_out
        (the first two as one call where the pool format and query form allow, the
        last two as one call)."""
        self.query_and_append()
        self.attention()
        self.merge_absorb_out()
        return self.u

    # ---- host copies of the same inputs, for the oracle ------------------
    def host_weights(self):
        """fp64 host copies of the weights, regenerated from the seed."""
        return {n: I.to_f64(self.w, I.weight_values(self.w, n, self.layer))
                for n in self.w.weight_names}

    def host_h(self, i: int) -> np.ndarray:
        """fp64 hidden state of step token i (decode: the token of sequence i)."""
        w = self.w
        b, p = int(self.q_seq_host[i]), int(self.q_pos_host[i])
        if w.cache_from_h:
            Lmax = int(self.lens.max())
            v = I.tensor_values(w, "h_ctx", None, 1.0, self.layer,
                                start=(b * Lmax + p) * w.hidden, count=w.hidden)
        else:
            v = I.tensor_values(w, "h_dec", None, 1.0, self.layer, start=i * w.hidden,
                                count=w.hidden)
        return I.to_f64(w, v)

    def host_h_ctx(self, b: int) -> np.ndarray:
        """fp64 hidden states of positions 0..L_b-1 of sequence b (cache-from-h workloads)."""
        w, L, Lmax = self.w, int(self.lens[b]), int(self.lens.max())
        v = I.tensor_values(w, "h_ctx", None, 1.0, self.layer, start=b * Lmax * w.hidden,
                            count=L * w.hidden)
        return I.to_f64(w, v).reshape(L, w.hidden)

    def host_pool_rows(self, b: int, length: int) -> np.ndarray:
        """fp64 generator-filled pool rows of logical positions 0..length-1 of b
        (for an FP8 pool: the fp32 rows before quantization)."""
        if self.fp8:
            return I.pool_rows(self.w, self.bt_host, b, length, self.layer, f32=True).astype(
                np.float64)
        return I.to_f64(self.w, I.pool_rows(self.w, self.bt_host, b, length, self.layer))
