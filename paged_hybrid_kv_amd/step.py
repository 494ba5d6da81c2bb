"""The hybrid decode step: every layer of a Gemma 4-style stack appends the
step's new K/V into its family's pool and attends with that family's page
table (pegainfer "Gemma 4" page, intro: five local layers per global one,
the last layer global; Scheduling: one pool and one page budget per family,
local pages before the window freed, global pages kept; prompt rows share
the step with the decode rows).

Each layer owns its pool; all layers of a family share one page table.
The step is plain C-ABI calls on one stream, so it can be captured once as a
HIP graph and replayed.
"""

from __future__ import annotations

import numpy as np
import torch

from . import gw
from .runtime import GLOBAL_THETA, LOCAL_THETA, Pool, Workspace, i32_dev, rope_tables
from .synth import HybridShape, make_page_table, layer_draws, step_tokens, PAGE


class HybridStep:
    def __init__(self, shape: HybridShape | None = None, with_prompts: bool = True, device="cuda",
                 fill_context: bool = True, local_kv_dtype: int = gw.GW_KV_BF16,
                 global_kv_dtype: int = gw.GW_KV_BF16):
        self.shape = sh = shape or HybridShape()
        self.with_prompts = with_prompts
        self.device = device
        # store type of each family's pools (bf16, or e4m3: PR #1012's opt-in fp8 pool)
        self.local_kv_dtype, self.global_kv_dtype = local_kv_dtype, global_kv_dtype
        lens = sh.lens(with_prompts)
        q_len = sh.q_len(with_prompts)
        self.lens, self.q_len = lens, q_len
        self.S = len(lens)
        self.rows = int(q_len.sum())
        self.max_len = int(lens.max())
        self.max_q_len = int(q_len.max())

        # page tables, one per family, drawn once (seed of the shape + 1)
        rng = np.random.default_rng(sh.seed + 1)
        first_local = np.array([max(0, int(L) - int(ql) - sh.window + 1) // PAGE
                                for L, ql in zip(lens, q_len)])
        self.local_seqs = make_page_table(rng, lens, first_local)
        self.global_seqs = make_page_table(rng, lens, None)
        self.local_pt = i32_dev(self.local_seqs.page_table, device)
        self.global_pt = i32_dev(self.global_seqs.page_table, device)
        self.seq_lens = i32_dev(lens, device)
        indptr = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
        self.q_indptr = None if self.max_q_len == 1 else i32_dev(indptr, device)

        self.local_cos, self.local_sin = rope_tables(self.max_len, 256, 256, LOCAL_THETA, device)
        self.global_cos, self.global_sin = rope_tables(self.max_len, 128, 512, GLOBAL_THETA, device)

        # tokens appended in the step, per family
        self.new_tok = {}
        for fam, local in (("local", True), ("global", False)):
            ns, npos, _, _ = step_tokens(sh, with_prompts, local)
            self.new_tok[fam] = (i32_dev(ns, device), i32_dev(npos, device), len(ns))

        self.layers = []
        for l in range(sh.num_layers):
            self.layers.append(self._make_layer(l, fill_context))

        D_l, D_g = sh.local_head_dim, sh.global_head_dim
        self.ws_local = Workspace(device)
        self.ws_global = Workspace(device)
        self.ws_bytes = {
            "local": gw.gw_attn_workspace_bytes(gw.GW_FAMILY_LOCAL, self.S, self.rows, sh.local_q_heads,
                                                D_l, self.max_len, sh.window, self.max_q_len),
            "global": gw.gw_attn_workspace_bytes(gw.GW_FAMILY_GLOBAL_COMPRESSED, self.S, self.rows,
                                                 sh.global_q_heads, D_g, self.max_len, 0, self.max_q_len),
        }
        self.ws_ptr = {"local": self.ws_local.get(self.ws_bytes["local"])[0],
                       "global": self.ws_global.get(self.ws_bytes["global"])[0]}
        self.graph = None

    # ------------------------------------------------------------------ setup
    def _make_layer(self, l, fill_context):
        sh = self.shape
        local = not sh.is_global(l)
        d = layer_draws(sh, l, self.with_prompts, self.device)
        if local:
            pool = Pool(gw.GW_FAMILY_LOCAL, self.local_kv_dtype, self.local_seqs.num_pages,
                        sh.local_kv_heads, 256, self.device)
            pt, stride = self.local_pt, self.local_seqs.page_table.shape[1]
            cos, sin = self.local_cos, self.local_sin
        else:
            pool = Pool(gw.GW_FAMILY_GLOBAL_COMPRESSED, self.global_kv_dtype, self.global_seqs.num_pages,
                        1, 128, self.device)
            pt, stride = self.global_pt, self.global_seqs.page_table.shape[1]
            cos, sin = self.global_cos, self.global_sin
        if fill_context:
            _, _, ps, pp = step_tokens(sh, self.with_prompts, local)
            if len(ps):
                gw.gw_kv_append(pool.desc, d.k_prior, d.v_prior, i32_dev(ps, self.device),
                                i32_dev(pp, self.device), len(ps), pt, stride, cos, sin)
        # each layer writes its own output (the next layer's projection would read it)
        Hq, D = (sh.local_q_heads, sh.local_head_dim) if local else (sh.global_q_heads, sh.global_head_dim)
        out = torch.empty((self.rows, Hq, D), dtype=torch.float32, device=self.device)
        return dict(index=l, local=local, pool=pool, q=d.q, k_new=d.k_new, v_new=d.v_new, pt=pt,
                    stride=stride, cos=cos, sin=sin, out=out)

    # -------------------------------------------------------------- the step
    def append(self, L):
        """Standalone append of the step's new tokens (gw_kv_append)."""
        fam = "local" if L["local"] else "global"
        si, pos, n = self.new_tok[fam]
        gw.gw_kv_append(L["pool"].desc, L["k_new"], L["v_new"], si, pos, n, L["pt"], L["stride"],
                        L["cos"], L["sin"])

    def attend(self, L, out=None, append=False):
        """One layer's attention call; with append=True the call also stores
        every row's own token first (the prep step inside the call)."""
        sh = self.shape
        fam = "local" if L["local"] else "global"
        if L["local"]:
            kn, vn, cs, sn = (L["k_new"], L["v_new"], L["cos"], L["sin"]) if append else (None,) * 4
            gw.gw_decode_attn_local(L["pool"].desc, L["q"], sh.local_q_heads, kn, vn, cs, sn,
                                    self.q_indptr, self.seq_lens,
                                    L["pt"], L["stride"], self.S, self.rows, self.max_q_len, self.max_len,
                                    sh.window, 1.0 / np.sqrt(sh.local_head_dim),
                                    L["out"] if out is None else out,
                                    self.ws_ptr[fam], self.ws_bytes[fam])
        else:
            vn, cs, sn = (L["v_new"], L["cos"], L["sin"]) if append else (None,) * 3
            gw.gw_decode_attn_global(L["pool"].desc, L["q"], sh.global_q_heads, None, vn, cs, sn,
                                     self.q_indptr, self.seq_lens, L["pt"], L["stride"], self.S, self.rows,
                                     self.max_q_len, self.max_len, 1.0 / np.sqrt(sh.global_head_dim),
                                     L["out"] if out is None else out,
                                     self.ws_ptr[fam], self.ws_bytes[fam])

    def layer_out(self, layer: int):
        """fp32 [rows][Hq][D]: layer `layer`'s attention output of the last step."""
        return self.layers[layer]["out"]

    def run(self):
        """One step, eagerly: every layer's attention call appends the step's
        new tokens (decode and prompt rows) and attends, layer by layer."""
        for L in self.layers:
            self.attend(L, append=True)

    def capture(self):
        """Capture the step as one HIP graph (after one eager run)."""
        self.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        self.graph = g
        return g

    def replay(self):
        if self.graph is None:
            self.run()
        else:
            self.graph.replay()

    # ------------------------------------------------------------ accounting
    def _esize(self, local: bool) -> int:
        return 1 if (self.local_kv_dtype if local else self.global_kv_dtype) == gw.GW_KV_E4M3 else 2

    def decode_kv_bytes(self) -> int:
        """Algorithmic KV bytes the decode rows read in one step."""
        sh = self.shape
        dec = sh.decode_lens
        local = sum(min(int(L), sh.window) for L in dec) * sh.local_kv_heads * 256 * 2 * self._esize(True)
        glob = sum(int(L) for L in dec) * (512 + 128) * self._esize(False)
        n_glob = sum(1 for l in range(sh.num_layers) if sh.is_global(l))
        return (sh.num_layers - n_glob) * local + n_glob * glob

    def mixed_step_bytes(self) -> dict:
        """Algorithmic bytes of one step with its prompt rows: every token's
        K/V read once per layer by the rows that attend it (decode rows: the
        window / whole context; prompt rows: the prompt once), the appended
        tokens (raw K/V read, record written), and q read / out written."""
        sh = self.shape
        n_glob = sum(1 for l in range(sh.num_layers) if sh.is_global(l))
        n_loc = sh.num_layers - n_glob
        loc_raw = sh.local_kv_heads * 256 * 2 * 2            # the step's raw K + V (bf16), all KV heads
        loc_tok = sh.local_kv_heads * 256 * 2 * self._esize(True)   # K + V as the pool stores them
        glob_tok = (512 + 128) * self._esize(False)                 # compressed record
        prompts = [int(x) for x in self.q_len[sh.decode_slots:]]
        pre_tok = sum(prompts)
        new_tok = sh.decode_slots + pre_tok
        # a prompt's rows (positions P .. P + n - 1) attend the union
        # [max(0, P - W + 1), P + n - 1] (local) or [0, P + n - 1] (global)
        P = sh.prompt_prefix if self.with_prompts else 0
        loc_rng = sum(P + n - max(0, P - sh.window + 1) for n in prompts)
        glob_rng = sum(P + n for n in prompts)
        kv = self.decode_kv_bytes() + n_loc * loc_rng * loc_tok + n_glob * glob_rng * glob_tok
        app = (n_loc * new_tok * (loc_raw + loc_tok) + n_glob * new_tok * (512 * 2 + glob_tok))
        rows = self.rows
        qo = (n_loc * rows * sh.local_q_heads * 256 * (2 + 4) + n_glob * rows * sh.global_q_heads * 512 * (2 + 4))
        return {"kv_read": kv, "append": app, "q_out": qo, "total": kv + app + qo}

    def prompt_flops(self) -> int:
        """2 x the multiply-adds of the prompt rows' two products (scores and
        weighted values) over the keys each row attends, all layers."""
        sh = self.shape
        n_glob = sum(1 for l in range(sh.num_layers) if sh.is_global(l))
        n_loc = sh.num_layers - n_glob
        P = sh.prompt_prefix if self.with_prompts else 0
        loc = glob = 0
        for n in (int(x) for x in self.q_len[sh.decode_slots:]):
            p = P + np.arange(n, dtype=np.int64)
            loc += int(np.minimum(p + 1, sh.window).sum())
            glob += int((p + 1).sum())
        return (n_loc * loc * sh.local_q_heads * 256 * 4 +
                n_glob * glob * sh.global_q_heads * 512 * 4)

    def local_decode_kv_bytes_per_layer(self) -> int:
        sh = self.shape
        return (sum(min(int(L), sh.window) for L in sh.decode_lens) * sh.local_kv_heads * 256 * 2 *
                self._esize(True))
