"""Device buffers for one batch of the verification step, and the five calls in order.

Marshalling only: inputs are copied to the GPU once, outputs and workspaces are
allocated once, and `run()` enqueues tree_build -> tree_mask_positions ->
tree_attention -> tree_accept -> kv_compact on one stream through the C ABI.

The batch description is any object with these attributes (numpy arrays):
  mode ('dynamic' | 'static' | 'given'), B, V, K, D, total_tokens, branching,
  T_max, dcap, logprobs [B][R][V] float32 (None for 'given'), root_token [B],
  given_parents / given_tokens [B][T_max], given_size [B] ('given' only),
  prefix_len [B], Hq, Hkv, d, dtype ('bf16' | 'fp32'), S_cap,
  Q [B][T_max][Hq][d], Kc / Vc [B][Hkv][S_cap][d] (uint16 bf16 bits or float32).
In 'given' mode the drafter's tree is an input and the build call is skipped.

With ``paged`` (any object with tokens_per_block, max_blocks, n_blocks,
block_table [B][max_blocks] int32 and K_pool / V_pool [n_blocks][Hkv][tokens_per_block][d])
the cache is that paged pool, and attention and compaction go through
tree_attention_paged, kv_compact_paged and tree_accept_compact_paged.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as tv

_MODES = {"dynamic": tv.MODE_DYNAMIC, "static": tv.MODE_STATIC}


def _t(a, device, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:          # bf16 bit patterns travel as int16 storage
        t = torch.from_numpy(a.view(np.int16)).to(device)
        return t.view(torch.bfloat16)
    t = torch.from_numpy(a).to(device)
    return t if dtype is None else t.to(dtype)


def _copies(t, n):
    return [t] + [t.clone() for _ in range(n - 1)]


class TreeVerifyStep:
    def __init__(self, w, device: str = "cuda", n_copies: int = 1, paged=None, rope_theta=None):
        self.w = w
        self.paged = paged
        self.rope_theta = rope_theta   # set: Q holds pre-rotary queries (tree_attention_rope)
        self.device = device
        B, T_max, dcap = w.B, w.T_max, w.dcap
        self.B, self.T_max, self.dcap = B, T_max, dcap
        W = (T_max + 31) // 32
        i32 = dict(dtype=torch.int32, device=device)
        # inputs
        self.prefix_len = _t(w.prefix_len.astype(np.int32), device)
        self.root_token = _t(w.root_token.astype(np.int32), device)
        self.mode = w.mode
        if w.mode == "given":
            self.logprobs_copies = [None]
            self.draft_tokens = _t(w.given_tokens.astype(np.int32), device)
            self.parents = _t(w.given_parents.astype(np.int32), device)
            self.tree_size = _t(w.given_size.astype(np.int32), device)
        else:
            self.logprobs_copies = _copies(_t(w.logprobs.astype(np.float32), device), n_copies)
            self.draft_tokens = torch.full((B, T_max), -7, **i32)
            self.parents = torch.full((B, T_max), -7, **i32)
            self.tree_size = torch.zeros(B, **i32)
        self.node_score = torch.zeros((B, T_max), dtype=torch.float32, device=device)
        self.status = torch.full((B,), 99, **i32)
        # input copies (more than one lets a benchmark rotate its inputs through HBM
        # so that repeated steps do not run out of the last-level cache)
        has_attn = w.Q is not None   # a tree-only batch has no attention tensors
        self.Q_copies = _copies(_t(w.Q, device), n_copies) if has_attn else [None]
        if not has_attn:
            self.Kc = self.Vc = [None]
            self.S_cap = w.S_cap
        elif paged is None:
            self.Kc = _copies(_t(w.Kc, device), n_copies)
            self.Vc = _copies(_t(w.Vc, device), n_copies)
            self.S_cap = w.S_cap
        else:   # the pools take the linear cache's place
            self.Kc = _copies(_t(paged.K_pool, device), n_copies)
            self.Vc = _copies(_t(paged.V_pool, device), n_copies)
            self.block_table = _t(np.asarray(paged.block_table, np.int32), device)
            self.S_cap = paged.max_blocks * paged.tokens_per_block
        # outputs
        self.tree_mask = torch.full((B, T_max, W), 0x5A5A5A5A, dtype=torch.int32, device=device)
        self.tree_position_ids = torch.full((B, T_max), -7, **i32)
        self.positions = torch.full((B, T_max), -7, **i32)
        self.retrieve_indices = torch.full((B, T_max, dcap + 1), -7, **i32)
        self.leaf_count = torch.full((B,), -7, **i32)
        self.first_child = torch.full((B, T_max), -7, **i32)
        self.next_sibling = torch.full((B, T_max), -7, **i32)
        self.O = torch.zeros_like(self.Q_copies[0]) if has_attn else None
        self.target_predict = torch.full((B, T_max), -1, **i32)
        self.accept_len = torch.full((B,), -7, **i32)
        self.accept_path = torch.full((B, dcap + 1), -7, **i32)
        self.bonus_token = torch.full((B,), -7, **i32)
        self.new_prefix_len = torch.full((B,), -7, **i32)
        # workspaces
        self.dtype_code = tv.DTYPE_BF16 if w.dtype == "bf16" else tv.DTYPE_FP32
        self.elem_bytes = 2 if w.dtype == "bf16" else 4
        if w.mode != "given":
            R = w.logprobs.shape[1]
            K = w.K if w.mode == "dynamic" else max(w.branching)
            nb = tv.tree_build_workspace_bytes(_MODES[w.mode], B, w.V, K, R)
            self.ws_build = torch.zeros(max(nb, 1), dtype=torch.uint8, device=device)
        else:
            self.ws_build = None
        na = tv.tree_attention_workspace_bytes(self.dtype_code, B, T_max, w.Hq, w.Hkv, w.d, self.S_cap) \
            if has_attn else 0
        self.ws_attn = torch.zeros(na, dtype=torch.uint8, device=device) if na else None
        self.copy = 0

    @property
    def logprobs(self):
        return self.logprobs_copies[self.copy % len(self.logprobs_copies)]

    @property
    def Q(self):
        return self.Q_copies[self.copy]

    # ---- the five calls -------------------------------------------------------
    def build(self, stream=None):
        w = self.w
        if w.mode == "given":
            return
        R = w.logprobs.shape[1]
        tv.tree_build(_MODES[w.mode], self.B, w.V, w.K, w.D, w.total_tokens,
                      w.branching if w.mode == "static" else None, self.logprobs, R, self.root_token,
                      self.T_max, self.draft_tokens, self.parents, self.tree_size, self.node_score, self.status,
                      self.ws_build, stream)

    def meta(self, stream=None):
        status_in = None if self.w.mode == "given" else self.status
        tv.tree_mask_positions(self.B, self.T_max, self.dcap, self.parents, self.tree_size, self.prefix_len,
                               self.tree_mask, self.tree_position_ids, self.positions, self.retrieve_indices,
                               self.leaf_count, self.first_child, self.next_sibling, status_in, self.status, stream)

    def attention(self, stream=None, copy=None):
        w = self.w
        c = self.copy if copy is None else copy
        if self.paged is not None:
            pg = self.paged
            tv.tree_attention_paged(self.dtype_code, self.B, self.T_max, w.Hq, w.Hkv, w.d, self.Q_copies[c],
                                    self.Kc[c], self.Vc[c], pg.n_blocks, pg.tokens_per_block, self.block_table,
                                    pg.max_blocks, self.prefix_len, self.tree_size, self.tree_mask, self.status, 0.0,
                                    self.O, self.ws_attn, stream)
            return
        if self.rope_theta is not None:
            tv.tree_attention_rope(self.dtype_code, self.B, self.T_max, w.Hq, w.Hkv, w.d, self.Q_copies[c],
                                   self.Kc[c], self.Vc[c], w.S_cap, self.prefix_len, self.tree_size, self.tree_mask,
                                   self.status, self.rope_theta, 0.0, self.O, self.ws_attn, stream)
            return
        tv.tree_attention(self.dtype_code, self.B, self.T_max, w.Hq, w.Hkv, w.d, self.Q_copies[c], self.Kc[c],
                          self.Vc[c],
                          w.S_cap, self.prefix_len, self.tree_size, self.tree_mask, self.status, 0.0, self.O,
                          self.ws_attn, stream)

    def accept(self, stream=None):
        tv.tree_accept(self.B, self.T_max, self.dcap, self.draft_tokens, self.parents, self.tree_size,
                       self.target_predict, self.status, self.accept_len, self.accept_path, self.bonus_token, stream)

    def compact(self, stream=None, copy=None):
        w = self.w
        c = self.copy if copy is None else copy
        if self.paged is not None:
            pg = self.paged
            tv.kv_compact_paged(self.B, 1, w.Hkv, w.d, self.elem_bytes, self.Kc[c], self.Vc[c], pg.n_blocks,
                                pg.tokens_per_block, self.block_table, pg.max_blocks, 0, self.prefix_len,
                                self.accept_path, self.accept_len, self.dcap, self.new_prefix_len, stream)
            return
        tv.kv_compact(self.B, 1, w.Hkv, w.d, self.elem_bytes, self.Kc[c], self.Vc[c], w.S_cap, 0, self.prefix_len,
                      self.accept_path, self.accept_len, self.dcap, self.new_prefix_len, stream)

    def build_meta(self, stream=None):
        """tree_build and tree_mask_positions in tree_build's launches."""
        w = self.w
        if w.mode == "given":
            return self.meta(stream)
        R = w.logprobs.shape[1]
        tv.tree_build_meta(_MODES[w.mode], self.B, w.V, w.K, w.D, w.total_tokens,
                           w.branching if w.mode == "static" else None, self.logprobs, R, self.root_token,
                           self.T_max, self.draft_tokens, self.parents, self.tree_size, self.node_score, self.status,
                           self.ws_build, self.dcap, self.prefix_len, self.tree_mask, self.tree_position_ids,
                           self.positions, self.retrieve_indices, self.leaf_count, self.first_child,
                           self.next_sibling, stream)

    # ---- the dynamic build one draft layer at a time --------------------------
    def prepare_layers(self, rows=None, logits: bool = False, n_copies: int = 1):
        """Stage one device buffer per draft layer (layer 0: [B][1][V], layer l: [B][K][V])
        from rows [B][1 + D K][V] (default: the batch's log-probs; logits=True: raw
        logits), plus the build state and the per-layer frontier outputs.  n_copies
        copies of the rows are kept (build_layers uses copy `self.copy`)."""
        w = self.w
        assert w.mode == "dynamic"
        src = w.logprobs if rows is None else rows
        B, K, D = self.B, w.K, w.D
        self.layers_logits = bool(logits)
        rows0 = [_t(np.ascontiguousarray(src[:, :1]).astype(np.float32), self.device)]
        for l in range(1, D + 1):
            blk = np.ascontiguousarray(src[:, 1 + (l - 1) * K:1 + l * K]).astype(np.float32)
            rows0.append(_t(blk, self.device))
        self.layer_rows_copies = [rows0] + [[t.clone() for t in rows0] for _ in range(n_copies - 1)]
        n = tv.tree_build_layer_workspace_bytes(B, w.V, K, D)
        if getattr(self, "layer_state", None) is None or self.layer_state.numel() < n:
            self.layer_state = torch.zeros(n, dtype=torch.uint8, device=self.device)
        i32 = dict(dtype=torch.int32, device=self.device)
        self.frontier_tokens = torch.full((D + 1, B, K), -7, **i32)
        self.frontier_parents = torch.full((D + 1, B, K), -7, **i32)

    def build_layers(self, meta: bool = True, stream=None):
        """tree_build_layer for layers 0..D, then tree_build_finish (with the tree
        metadata when meta, as tree_build_meta)."""
        w = self.w
        B, K, D = self.B, w.K, w.D
        rows = self.layer_rows_copies[self.copy % len(self.layer_rows_copies)]
        for l in range(D + 1):
            tv.tree_build_layer(l, B, w.V, K, D, rows[l], self.layers_logits, self.layer_state,
                                self.frontier_tokens[l], self.frontier_parents[l], stream)
        if meta:
            tv.tree_build_finish(B, w.V, K, D, w.total_tokens, self.root_token, self.T_max, self.layer_state,
                                 self.draft_tokens, self.parents, self.tree_size, self.node_score, self.status,
                                 self.dcap, self.prefix_len, self.tree_mask, self.tree_position_ids, self.positions,
                                 self.retrieve_indices, self.leaf_count, self.first_child, self.next_sibling,
                                 stream=stream)
        else:
            tv.tree_build_finish(B, w.V, K, D, w.total_tokens, self.root_token, self.T_max, self.layer_state,
                                 self.draft_tokens, self.parents, self.tree_size, self.node_score, self.status,
                                 stream=stream)

    def frontiers_host(self):
        return self.frontier_tokens.cpu().numpy(), self.frontier_parents.cpu().numpy()

    def accept_compact(self, stream=None, copy=None):
        """tree_accept and kv_compact in one launch."""
        w = self.w
        c = self.copy if copy is None else copy
        if self.paged is not None:
            pg = self.paged
            tv.tree_accept_compact_paged(self.B, self.T_max, self.dcap, self.draft_tokens, self.parents,
                                         self.tree_size, self.target_predict, self.status, self.accept_len,
                                         self.accept_path, self.bonus_token, 1, w.Hkv, w.d, self.elem_bytes,
                                         self.Kc[c], self.Vc[c], pg.n_blocks, pg.tokens_per_block, self.block_table,
                                         pg.max_blocks, 0, self.prefix_len, self.new_prefix_len, stream)
            return
        tv.tree_accept_compact(self.B, self.T_max, self.dcap, self.draft_tokens, self.parents, self.tree_size,
                               self.target_predict, self.status, self.accept_len, self.accept_path,
                               self.bonus_token, 1, w.Hkv, w.d, self.elem_bytes, self.Kc[c], self.Vc[c], w.S_cap, 0,
                               self.prefix_len, self.new_prefix_len, stream)

    def run(self, stream=None, fused=False):
        """One full pass of the step (target_predict must already be set).  With
        fused, the five calls run as tree_build_meta, tree_attention and
        tree_accept_compact (same results, two kernel launches fewer)."""
        if fused:
            self.build_meta(stream)
            self.attention(stream)
            self.accept_compact(stream)
            return
        self.build(stream)
        self.meta(stream)
        self.attention(stream)
        self.accept(stream)
        self.compact(stream)

    # ---- non-greedy acceptance ------------------------------------------------
    def set_target_probs(self, probs: np.ndarray, uniforms: np.ndarray):
        """The target's distribution at every node [B][T_max][V] and the draws [B][T_max]."""
        self.target_probs = _t(np.ascontiguousarray(probs, dtype=np.float32), self.device)
        self.uniforms = _t(np.ascontiguousarray(uniforms, dtype=np.float32), self.device)
        self._alloc_ws_sample()

    def _alloc_ws_sample(self):
        """tree_accept_sample's optional workspace (one float64 per row), allocated once."""
        if getattr(self, "ws_sample", None) is None:
            self.ws_sample = torch.empty(tv.tree_accept_sample_workspace_bytes(self.B, self.T_max),
                                         dtype=torch.uint8, device=self.device)

    def accept_sample(self, stream=None, workspace=True):
        """tree_accept_sample: target-only tree rejection sampling (workspace=False: the
        call without its optional workspace, which sums each visited row on the way)."""
        if workspace:
            self._alloc_ws_sample()
        tv.tree_accept_sample(self.B, self.T_max, self.dcap, self.target_probs.shape[-1], self.draft_tokens,
                              self.parents, self.tree_size, self.target_probs, self.uniforms, self.status,
                              self.accept_len, self.accept_path, self.bonus_token,
                              self.ws_sample if workspace else None, stream)

    def set_sampling_inputs(self, logits: np.ndarray, params, draft_probs=None):
        """Target logits [B][T_max][V] with the per-request (temperature, top_k, top_p,
        min_p), and optionally the drafter's distributions [B][T_max][V]; the probability
        rows that tree_sampling_probs fills are allocated here."""
        self.target_logits = _t(np.ascontiguousarray(logits, dtype=np.float32), self.device)
        temp, top_k, top_p, min_p = params
        self.temperature = _t(np.asarray(temp, np.float32), self.device)
        self.top_k = _t(np.asarray(top_k, np.int32), self.device)
        self.top_p = _t(np.asarray(top_p, np.float32), self.device)
        self.min_p = _t(np.asarray(min_p, np.float32), self.device)
        self.target_probs = torch.zeros_like(self.target_logits)
        self._alloc_ws_sample()
        if draft_probs is not None:
            self.draft_probs = _t(np.ascontiguousarray(draft_probs, dtype=np.float32), self.device)
            V = self.target_logits.shape[-1]
            self.ws_draft = torch.empty(tv.tree_accept_sample_draft_workspace_bytes(self.B, V), dtype=torch.uint8,
                                        device=self.device)

    def sampling_probs(self, stream=None):
        """tree_sampling_probs: the target logits filtered into self.target_probs."""
        tv.tree_sampling_probs(self.B, self.T_max, self.target_logits.shape[-1], self.target_logits, self.tree_size,
                               self.status, self.temperature, self.top_k, self.top_p, self.min_p, self.target_probs,
                               stream)

    def accept_sample_draft(self, without_replacement: bool = True, stream=None):
        """tree_accept_sample_draft: tree rejection sampling with the drafter's q."""
        tv.tree_accept_sample_draft(self.B, self.T_max, self.dcap, self.target_probs.shape[-1], self.draft_tokens,
                                    self.parents, self.tree_size, self.target_probs, self.draft_probs, self.uniforms,
                                    self.status, without_replacement, self.accept_len, self.accept_path,
                                    self.bonus_token, self.ws_draft, stream)

    def set_target_predict(self, tp: np.ndarray):
        self.target_predict.copy_(torch.from_numpy(np.ascontiguousarray(tp.astype(np.int32))))

    # ---- host copies ----------------------------------------------------------
    def tree_host(self):
        return dict(draft_tokens=self.draft_tokens.cpu().numpy(), parents=self.parents.cpu().numpy(),
                    tree_size=self.tree_size.cpu().numpy(), node_score=self.node_score.cpu().numpy(),
                    status=self.status.cpu().numpy())

    def meta_host(self):
        return dict(tree_mask=self.tree_mask.cpu().numpy().view(np.uint32),
                    tree_position_ids=self.tree_position_ids.cpu().numpy(), positions=self.positions.cpu().numpy(),
                    retrieve_indices=self.retrieve_indices.cpu().numpy(), leaf_count=self.leaf_count.cpu().numpy(),
                    first_child=self.first_child.cpu().numpy(), next_sibling=self.next_sibling.cpu().numpy(),
                    status=self.status.cpu().numpy())

    def out_host(self):
        o = self.O.cpu()
        if o.dtype == torch.bfloat16:
            return o.view(torch.int16).numpy().view(np.uint16)
        return o.numpy()

    def kv_host(self, copy=0):
        def h(t):
            t = t.cpu()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
        return h(self.Kc[copy]), h(self.Vc[copy])

    def accept_host(self):
        return dict(accept_len=self.accept_len.cpu().numpy(), accept_path=self.accept_path.cpu().numpy(),
                    bonus_token=self.bonus_token.cpu().numpy(), new_prefix_len=self.new_prefix_len.cpu().numpy())
