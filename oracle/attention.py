"""Float64 reference for single-query decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the smoke check and
the benchmark's CPU-baseline leg, never by the library.

What is computed, per sequence s and query head h ("Paged Attention and vLLM", section
"Block Table and Logical-to-Physical Mapping", equation for a_t, with V applied as in the
section "Paged Attention CUDA Kernel"):

    o_{s,h} = softmax( q_{s,h} . [K_tau(0) || K_tau(1) || ...]^T / sqrt(d) ) . [V_tau(0) || ...]

over the L_s stored tokens of sequence s, where token p lives at physical block
tau_s(p div B), offset p mod B ("PagedAttention: Virtual Memory for the KV Cache", section
"A block table preserves token order"). The pages state that paging changes addressing, not
the attention function, so the plain definition is the oracle.

Readings where the pages leave a step open:
  * The garbled equation shows no V and indexes the last block as floor(t/B); we apply V and
    read exactly the ceil(L/B) blocks that hold the L tokens, slots >= L excluded.
  * GQA head mapping: query head h reads KV head h div G, G = H_q / H_kv (contiguous groups).
  * scale defaults to 1/sqrt(head_dim).
  * An empty context (L = 0) yields a zero output.
Layout (the pages leave it to the kernel): k_pool and v_pool both [N][H_kv][B][d].
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _index(pool, phys, kv_head, offset):
    """pool[phys[i], kv_head, offset[i], :] for every i, as float64 [n][d]."""
    try:
        import torch
        if isinstance(pool, torch.Tensor):
            p = torch.from_numpy(np.asarray(phys, dtype=np.int64))
            o = torch.from_numpy(np.asarray(offset, dtype=np.int64))
            return _f64(pool[p, int(kv_head), o])
    except ImportError:  # pragma: no cover
        pass
    return _f64(np.asarray(pool)[phys, int(kv_head), offset])


def token_address(position: int, table_row, block_size: int):
    """Physical block and in-block offset of token ``position``.

    The logical block is position div B and the offset position mod B; the block table maps
    the logical block to a physical one ("PagedAttention: Virtual Memory for the KV Cache",
    sections "A block table preserves token order" and "The indexing rule in code";
    "Paged Attention and vLLM", definition of tau_s).
    """
    logical_block, offset = divmod(int(position), int(block_size))
    return int(table_row[logical_block]), offset


def gather_kv(k_pool, v_pool, table_row, length: int, kv_head: int, block_size: int):
    """Keys and values ``[L][d]`` of one sequence and KV head, in token order, read through
    the block table. Only the first ceil(L/B) table entries are touched."""
    pos = np.arange(int(length))
    logical_block = pos // block_size
    offset = pos % block_size
    phys = np.asarray(table_row, dtype=np.int64)[logical_block]
    K = _index(k_pool, phys, kv_head, offset)
    V = _index(v_pool, phys, kv_head, offset)
    return K, V


def attend(q, K, V, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for one query row over L key/value rows (float64).

    Subtracting the maximum score before exponentiating leaves the softmax unchanged and keeps
    exp in range. L = 0 gives zeros.
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1] if V.ndim == 2 else q.shape[0])
    z = (K @ q) * scale
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def partial_state(q, K, V, scale: float):
    """Per-block partial softmax state (m, l, acc) of "Paged Attention and vLLM", section
    "Paged Attention CUDA Kernel": m = max score, l = sum of exp(score - m),
    acc = sum of exp(score - m) * v. An empty block gives (-inf, 0, 0)."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    if K.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(V.shape[1])
    z = (K @ q) * scale
    m = float(z.max())
    w = np.exp(z - m)
    return m, float(w.sum()), w @ V


def merge_states(states):
    """Combine partial states with the log-sum-exp merge of the same section:
    o = sum_b e^{m_b - m*} acc_b / sum_b e^{m_b - m*} l_b, m* = max_b m_b.
    All-empty input gives zeros."""
    ms = np.array([s[0] for s in states], dtype=np.float64)
    m_star = ms.max()
    d = len(states[0][2])
    if not np.isfinite(m_star):
        return np.zeros(d)
    num = np.zeros(d)
    den = 0.0
    for m, l, acc in states:
        c = math.exp(m - m_star) if np.isfinite(m) else 0.0
        num += c * np.asarray(acc, dtype=np.float64)
        den += c * l
    return num / den


def _heads(q, k_pool):
    S, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return S, Hq, Hkv, Hq // Hkv, d


def paged_decode(q, k_pool, v_pool, tables, lengths, block_size: int, scale=None, seqs=None):
    """Output ``[S][H_q][d]`` (float64) of one decode step over the paged cache.

    ``seqs`` restricts the work to a subset of sequences (rows of other sequences stay NaN).
    """
    S, Hq, Hkv, G, d = _heads(q, k_pool)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((S, Hq, d), np.nan)
    qf = _f64(q)
    for s in (range(S) if seqs is None else seqs):
        L = int(lengths[s])
        for g in range(Hkv):
            K, V = gather_kv(k_pool, v_pool, tables[s], L, g, block_size)
            for i in range(G):
                h = g * G + i
                out[s, h] = attend(qf[s, h], K, V, scale)
    return out


def paged_decode_split(q, k_pool, v_pool, tables, lengths, block_size: int,
                       partition_tokens: int, scale=None):
    """The same output computed the pages' way: partial states over consecutive
    ``partition_tokens``-token chunks, then the log-sum-exp merge."""
    S, Hq, Hkv, G, d = _heads(q, k_pool)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((S, Hq, d))
    qf = _f64(q)
    for s in range(S):
        L = int(lengths[s])
        for g in range(Hkv):
            K, V = gather_kv(k_pool, v_pool, tables[s], L, g, block_size)
            for i in range(G):
                h = g * G + i
                parts = [partial_state(qf[s, h], K[a:a + partition_tokens],
                                       V[a:a + partition_tokens], scale)
                         for a in range(0, max(L, 1), partition_tokens)]
                out[s, h] = merge_states(parts)
    return out


def shared_prefix_decode(q, k_pool, v_pool, prefix_blocks, prefix_len: int, tables, lengths,
                         block_size: int, scale=None):
    """The same output for a batch whose sequences all begin with one shared prefix, computed
    the way prefix sharing allows: the prefix's keys and values are gathered once, through the
    shared block list ("PagedAttention: Virtual Memory for the KV Cache", section "Sharing a
    prefix and copying a partial block": sharers point their tables at the same full blocks),
    each query row's partial state over the prefix and over its own suffix tokens
    [prefix_len, L_s) is taken, and the two merge with the log-sum-exp rule ("Paged Attention
    and vLLM", section "Paged Attention CUDA Kernel").

    Reading: the shared prefix is whole blocks (``prefix_len`` a multiple of ``block_size``,
    ``prefix_blocks`` its ``prefix_len / block_size`` physical ids); every sequence holds at
    least ``prefix_len`` tokens; its suffix token p sits at ``tables[s][p // B]``, offset
    ``p % B`` (table entries before ``prefix_len / B`` are not read)."""
    S, Hq, Hkv, G, d = _heads(q, k_pool)
    B = int(block_size)
    P = int(prefix_len)
    if P % B or len(prefix_blocks) * B < P:
        raise ValueError("the shared prefix must be whole blocks")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qf = _f64(q)
    out = np.zeros((S, Hq, d))
    pos = np.arange(P)
    phys = np.asarray(prefix_blocks, dtype=np.int64)[pos // B]
    for g in range(Hkv):
        Kp = _index(k_pool, phys, g, pos % B)     # gathered once for every sharer
        Vp = _index(v_pool, phys, g, pos % B)
        for s in range(S):
            L = int(lengths[s])
            if L < P:
                raise ValueError(f"sequence {s} is shorter than the shared prefix")
            spos = np.arange(P, L)
            sphys = np.asarray(tables[s], dtype=np.int64)[spos // B]
            Ks = _index(k_pool, sphys, g, spos % B)
            Vs = _index(v_pool, sphys, g, spos % B)
            for i in range(G):
                h = g * G + i
                out[s, h] = merge_states([partial_state(qf[s, h], Kp, Vp, scale),
                                          partial_state(qf[s, h], Ks, Vs, scale)])
    return out


def extend_attention(q, query_start, k_pool, v_pool, tables, lengths, block_size: int,
                     scale=None):
    """Output ``[T][H_q][d]`` (float64) of several new query tokens per sequence over the paged
    cache (chunked prefill, or verification of speculated tokens): the pages' case of a request
    whose cached prefix is reused and only the tokens past it get a fresh prefill pass
    ("KV Cache Optimization and Management", section "RadixAttention: caching, not just
    packing, the prefix"; "PagedAttention: Virtual Memory for the KV Cache", section "Sharing a
    prefix and copying a partial block").

    Reading: sequence s owns query rows ``query_start[s] .. query_start[s+1] - 1`` (n_s rows);
    their keys and values are already stored, so its cache holds L_s = ``lengths[s]`` tokens,
    the last n_s of them the new ones. New token t sits at position L_s - n_s + t and attends
    to positions 0 .. L_s - n_s + t (causal), read through the block table. A row with no
    position to attend (L_s < n_s - t) gives zeros."""
    qf = _f64(q)
    T, Hq, d = qf.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((T, Hq, d))
    starts = [int(x) for x in query_start]
    for s in range(len(starts) - 1):
        n = starts[s + 1] - starts[s]
        L = int(lengths[s])
        for t in range(n):
            upto = L - n + t + 1                 # positions 0 .. L - n + t
            if upto <= 0:
                continue
            for g in range(Hkv):
                K, V = gather_kv(k_pool, v_pool, tables[s], upto, g, block_size)
                for i in range(G):
                    out[starts[s] + t, g * G + i] = attend(qf[starts[s] + t, g * G + i], K, V,
                                                            scale)
    return out


def contiguous_decode(q, k_logical, v_logical, scale=None):
    """The same output from the logical (never paged) per-sequence K/V ``[H_kv][L][d]``."""
    qf = _f64(q)
    S, Hq, d = qf.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((S, Hq, d))
    for s in range(S):
        K_all = _f64(k_logical[s])
        V_all = _f64(v_logical[s])
        Hkv = K_all.shape[0]
        G = Hq // Hkv
        for h in range(Hq):
            out[s, h] = attend(qf[s, h], K_all[h // G], V_all[h // G], scale)
    return out
