"""Seeded synthetic inputs for the paged hybrid-KV decode workloads.

This module only draws random numbers (numpy ``default_rng``); it does none
of the method's arithmetic -- no rotary embedding, no rounding to bf16/e4m3,
no attention.  The HIP path and the CPU oracle each take these fp32 draws and
do their own rounding and rotation, so the two sides share nothing else.

Draw order per case is fixed: lengths -> physical page permutation -> q -> K
-> V (the global family has no separate K draw: its K is tied to V).

The workloads mirror the serving shapes of the Gemma 4 hybrid stack
(pegainfer "Gemma 4" page, Scheduling and Architecture notes: 16 decode
slots, an 8192-token ceiling, 16-token pages, window 1024, local hd256 with
16 q / 8 KV heads, global hd512 with one KV head):

* ``tiny_local``      1 sequence, L=64, W=32, hd256, 2 q / 1 KV head, N(0,1)
* ``local_bf16``      16 slots, L ~ U{1024..8192}, W=1024, 16 q / 8 KV, 0.5*N(0,1)
* ``global_tied``     8 slots, L=131072, hd512, 32 q / 1 KV, N(0,1)
* ``local_fp8``       64 slots, L=8192, W=1024, 16 q / 8 KV, 0.5*N(0,1)
* ``hybrid_step``     shapes of the 60-layer mixed step (see ``HybridShape``)
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 16


def cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


@dataclass
class PagedSeqs:
    """Sequences, their lengths and a permuted page table.

    page_table[s, i] is the physical page of logical page i of sequence s, or
    -1 when that page is not allocated (wholly before a local window, or past
    the sequence).  Allocated pages are a random permutation of
    [0, num_pages).
    """
    lens: np.ndarray            # int64 [S]
    page_table: np.ndarray      # int32 [S, max_pages]
    num_pages: int
    first_page: np.ndarray      # int64 [S]: first allocated logical page

    @property
    def S(self) -> int:
        return int(self.lens.shape[0])


def make_page_table(rng, lens, first_page=None, extra_pages: int = 0) -> PagedSeqs:
    """One shared permutation of all allocated pages, dealt out per sequence.

    Sequence s owns logical pages [first_page[s], cdiv(lens[s], 16)), laid
    out in order over a slice of ``rng.permutation(total + extra_pages)``.
    ``extra_pages`` leaves unused physical pages in the pool.
    """
    lens = np.asarray(lens, dtype=np.int64)
    S = lens.shape[0]
    npg = np.array([cdiv(int(L), PAGE) for L in lens], dtype=np.int64)
    if first_page is None:
        first_page = np.zeros(S, dtype=np.int64)
    first_page = np.asarray(first_page, dtype=np.int64)
    counts = npg - first_page
    total = int(counts.sum())
    perm = rng.permutation(total + extra_pages)
    max_pages = int(npg.max()) if S else 1
    pt = np.full((S, max(1, max_pages)), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        c = int(counts[s])
        pt[s, first_page[s]:npg[s]] = perm[off:off + c]
        off += c
    return PagedSeqs(lens=lens, page_table=pt, num_pages=total + extra_pages,
                     first_page=first_page)


@dataclass
class LocalCase:
    """Local-family attention workload (hd256, sliding window)."""
    name: str
    seqs: PagedSeqs
    window: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_len: np.ndarray           # int64 [S] query rows per sequence (last q_len tokens)
    q: np.ndarray               # fp32 [sum q_len, Hq, D]
    k: np.ndarray               # fp32 [sum stored tokens, Hkv, D] (pre-rotation)
    v: np.ndarray               # fp32 same
    tok_seq: np.ndarray         # int32 [sum stored tokens]: owning sequence
    tok_pos: np.ndarray         # int32 [sum stored tokens]: position in it
    rope: bool                  # rotate K (theta 1e4, all 256 dims)
    fp8: bool                   # store K/V as e4m3
    scale: float

    @property
    def q_indptr(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_len)]).astype(np.int32)


@dataclass
class GlobalCase:
    """Global-family attention workload (hd512, one tied KV head)."""
    name: str
    seqs: PagedSeqs
    num_q_heads: int
    head_dim: int
    rot_dim: int
    q_len: np.ndarray
    q: np.ndarray               # fp32 [sum q_len, Hq, 512]
    v: np.ndarray               # fp32 [sum stored tokens, 512] (K = V before rotation)
    tok_seq: np.ndarray
    tok_pos: np.ndarray
    rope: bool                  # rotate K's first rot_dim dims (theta 1e6, denominator 512)
    scale: float
    # K's per-dim norm weight [512] (K = V * w_k before rotation), None when K = V;
    # every value is 1 + k/64, |k| <= 32, so exact in bf16
    w_k: np.ndarray | None = None
    fp8: bool = False           # e4m3 pool (codes of the bf16 record)

    @property
    def q_indptr(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_len)]).astype(np.int32)


def _stored_tokens(seqs: PagedSeqs, window_fill: int | None):
    """(seq, pos) of every token whose K/V is drawn.

    window_fill None: all tokens 0..L-1.  Otherwise only the tokens of
    allocated pages that also fall in the last ``window_fill`` positions
    (earlier slots of the first such page are left unwritten).
    """
    seq, pos = [], []
    for s in range(seqs.S):
        L = int(seqs.lens[s])
        lo = 0 if window_fill is None else max(0, L - window_fill, int(seqs.first_page[s]) * PAGE)
        seq.append(np.full(L - lo, s, dtype=np.int32))
        pos.append(np.arange(lo, L, dtype=np.int32))
    return np.concatenate(seq), np.concatenate(pos)


def _normal(rng, shape, scale):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def local_case(name, seed, lens, window, num_q_heads, num_kv_heads, q_len=None,
               q_scale=1.0, kv_scale=1.0, rope=True, fp8=False,
               window_only_pages=False, fill_window_only=False, head_dim=256,
               extra_pages=0) -> LocalCase:
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens(rng) if callable(lens) else lens, dtype=np.int64)
    S = lens.shape[0]
    q_len = np.ones(S, dtype=np.int64) if q_len is None else np.asarray(q_len, dtype=np.int64)
    first = None
    if window_only_pages:
        # pages wholly before the window of the first query row are not allocated
        first = np.array([max(0, int(L) - int(ql) - window + 1) // PAGE
                          for L, ql in zip(lens, q_len)], dtype=np.int64)
    seqs = make_page_table(rng, lens, first, extra_pages)
    fill = None
    if fill_window_only:
        fill = window + int(q_len.max()) - 1
    tok_seq, tok_pos = _stored_tokens(seqs, fill)
    n = tok_seq.shape[0]
    q = _normal(rng, (int(q_len.sum()), num_q_heads, head_dim), q_scale)
    k = _normal(rng, (n, num_kv_heads, head_dim), kv_scale)
    v = _normal(rng, (n, num_kv_heads, head_dim), kv_scale)
    return LocalCase(name=name, seqs=seqs, window=window, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, q_len=q_len, q=q,
                     k=k, v=v, tok_seq=tok_seq, tok_pos=tok_pos, rope=rope, fp8=fp8,
                     scale=float(1.0 / np.sqrt(head_dim)))


def global_case(name, seed, lens, num_q_heads=32, q_len=None, q_scale=1.0,
                v_scale=1.0, rope=True, head_dim=512, rot_dim=128,
                extra_pages=0, k_norm=False, fp8=False) -> GlobalCase:
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens(rng) if callable(lens) else lens, dtype=np.int64)
    S = lens.shape[0]
    q_len = np.ones(S, dtype=np.int64) if q_len is None else np.asarray(q_len, dtype=np.int64)
    seqs = make_page_table(rng, lens, None, extra_pages)
    tok_seq, tok_pos = _stored_tokens(seqs, None)
    q = _normal(rng, (int(q_len.sum()), num_q_heads, head_dim), q_scale)
    v = _normal(rng, (tok_seq.shape[0], head_dim), v_scale)
    w_k = (1.0 + rng.integers(-32, 32, size=head_dim, endpoint=True) / 64.0).astype(np.float32) \
        if k_norm else None
    return GlobalCase(name=name, seqs=seqs, num_q_heads=num_q_heads, head_dim=head_dim,
                      rot_dim=rot_dim, q_len=q_len, q=q, v=v, tok_seq=tok_seq,
                      tok_pos=tok_pos, rope=rope, scale=float(1.0 / np.sqrt(head_dim)), w_k=w_k,
                      fp8=fp8)


# ----------------------------------------------------------------------------
# the named workloads
# ----------------------------------------------------------------------------
def tiny_local() -> LocalCase:
    """1 sequence of 64 tokens, window 32, hd256, 2 q heads on 1 KV head,
    4 shuffled physical pages, N(0,1), no rotation, scale 1/16."""
    return local_case("tiny_local", 1, [64], window=32, num_q_heads=2, num_kv_heads=1,
                      rope=False)


def local_bf16(fill_window_only=False) -> LocalCase:
    """16 slots, L ~ U{1024..8192}, window 1024, 16 q / 8 KV heads,
    0.5*N(0,1), K rotated (theta 1e4, positions 0..L-1), all pages allocated."""
    return local_case("local_bf16", 2, lambda r: r.integers(1024, 8192, size=16, endpoint=True),
                      window=1024, num_q_heads=16, num_kv_heads=8, q_scale=0.5,
                      kv_scale=0.5, rope=True, fill_window_only=fill_window_only)


def global_tied(S=8, L=131072, rope=True) -> GlobalCase:
    """8 slots x 131072 tokens, hd512, 32 q heads / 1 KV head, N(0,1)."""
    return global_case("global_tied", 3, [L] * S, num_q_heads=32, rope=rope)


def local_fp8(S=64, L=8192) -> LocalCase:
    """64 slots x 8192 tokens, window 1024, 16 q / 8 KV heads, 0.5*N(0,1),
    e4m3 store; all 32768 pages allocated and permuted, K/V drawn for the
    window's pages only (other slots stay unwritten)."""
    return local_case("local_fp8", 4, [L] * S, window=1024, num_q_heads=16,
                      num_kv_heads=8, q_scale=0.5, kv_scale=0.5, rope=True, fp8=True,
                      fill_window_only=True)


# ----------------------------------------------------------------------------
# the 60-layer hybrid step
# ----------------------------------------------------------------------------
@dataclass
class HybridShape:
    """Shapes of the mixed hybrid step.

    60 layers, layer i global iff (i+1) % 6 == 0 or i is the last layer.
    16 decode slots with contexts drawn in [2048, 8192] (seed 5), each
    advancing one token; 4 new prompts of 512 tokens whose rows are computed
    in the same step (causal within the prompt, no prior context).  With
    prompt_prefix P > 0 the prompt rows are instead a 512-token chunk of
    longer prompts whose first P tokens are already in the cache: rows at
    positions P .. P + 511, each attending its window (local) or everything
    before it (global), cached prefix included.
    """
    num_layers: int = 60
    decode_slots: int = 16
    ctx_lo: int = 2048
    ctx_hi: int = 8192
    prompts: int = 4
    prompt_len: int = 512
    prompt_prefix: int = 0
    window: int = 1024
    local_q_heads: int = 16
    local_kv_heads: int = 8
    local_head_dim: int = 256
    global_q_heads: int = 32
    global_head_dim: int = 512
    global_rot_dim: int = 128
    seed: int = 5
    layer_seed_base: int = 5000
    decode_lens: np.ndarray = field(default=None)

    def __post_init__(self):
        if self.decode_lens is None:
            rng = np.random.default_rng(self.seed)
            self.decode_lens = rng.integers(self.ctx_lo, self.ctx_hi, size=self.decode_slots,
                                            endpoint=True).astype(np.int64)

    def is_global(self, layer: int) -> bool:
        return (layer + 1) % 6 == 0 or layer == self.num_layers - 1

    def lens(self, with_prompts: bool = True) -> np.ndarray:
        """Context length of every sequence in the step (current token included)."""
        extra = [self.prompt_prefix + self.prompt_len] * self.prompts if with_prompts else []
        return np.concatenate([self.decode_lens, np.array(extra, dtype=np.int64)])

    def q_len(self, with_prompts: bool = True) -> np.ndarray:
        extra = [self.prompt_len] * self.prompts if with_prompts else []
        return np.concatenate([np.ones(self.decode_slots, dtype=np.int64),
                               np.array(extra, dtype=np.int64)])


# ----------------------------------------------------------------------------
# per-layer draws of the hybrid step, made on the device (torch's seeded
# generator) so that 60 layers of context can be drawn in seconds; the same
# call on any device returns the same values, so the oracle can re-draw a
# layer on the host side of a test.
# ----------------------------------------------------------------------------
@dataclass
class LayerDraws:
    """Raw N(0,1) draws of one layer (bf16, before any rotation).

    q        [rows][Hq][D]          query rows (decode rows, then prompt rows)
    k_new    [n_new][Hkv][D] | None K of the tokens appended in the step
    v_new    [n_new][Hkv][D] (local) or [n_new][D] (global)
    k_prior, v_prior: the same for the context already in the cache
    """
    q: object
    k_new: object
    v_new: object
    k_prior: object
    v_prior: object


def step_tokens(shape: HybridShape, with_prompts: bool, local: bool):
    """(seq, pos) of the tokens appended in the step and of the prior context.

    Decode slot s appends its current token at L_s - 1; prompt i (sequence
    16 + i) appends positions P..P+511 (P = prompt_prefix).  Prior context:
    positions from the first allocated page (local: the first page of the
    earliest row's window; global: 0) to the position before the first
    appended one; the prompts' prior context follows the decode slots'.
    """
    lens = shape.lens(with_prompts)
    new_s, new_p, pri_s, pri_p = [], [], [], []
    for s in range(shape.decode_slots):
        L = int(lens[s])
        new_s.append([s]); new_p.append([L - 1])
        lo = (max(0, L - shape.window) // PAGE) * PAGE if local else 0
        pri_s.append(np.full(L - 1 - lo, s)); pri_p.append(np.arange(lo, L - 1))
    if with_prompts:
        P = shape.prompt_prefix
        for i in range(shape.prompts):
            s = shape.decode_slots + i
            new_s.append(np.full(shape.prompt_len, s)); new_p.append(P + np.arange(shape.prompt_len))
        for i in range(shape.prompts):
            if P > 0:
                s = shape.decode_slots + i
                lo = (max(0, P - shape.window + 1) // PAGE) * PAGE if local else 0
                pri_s.append(np.full(P - lo, s)); pri_p.append(np.arange(lo, P))
    cat = lambda xs: np.concatenate([np.asarray(x, dtype=np.int32) for x in xs]) if xs else np.zeros(0, np.int32)
    return cat(new_s), cat(new_p), cat(pri_s), cat(pri_p)


def layer_draws(shape: HybridShape, layer: int, with_prompts: bool, device="cuda") -> LayerDraws:
    """Draw layer ``layer``'s inputs with seed layer_seed_base + layer, in the
    fixed order q -> K new -> V new -> K prior -> V prior (global: no K)."""
    import torch
    local = not shape.is_global(layer)
    g = torch.Generator(device=device)
    g.manual_seed(shape.layer_seed_base + layer)
    new_s, _, pri_s, _ = step_tokens(shape, with_prompts, local)
    rows = int(shape.q_len(with_prompts).sum())
    if local:
        Hq, Hkv, D = shape.local_q_heads, shape.local_kv_heads, shape.local_head_dim
        kv = (Hkv, D)
    else:
        Hq, D = shape.global_q_heads, shape.global_head_dim
        kv = (D,)

    def draw(*sz):
        return torch.randn(*sz, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

    q = draw(rows, Hq, D)
    k_new = draw(len(new_s), *kv) if local else None
    v_new = draw(len(new_s), *kv)
    k_prior = draw(len(pri_s), *kv) if local else None
    v_prior = draw(len(pri_s), *kv)
    return LayerDraws(q, k_new, v_new, k_prior, v_prior)
