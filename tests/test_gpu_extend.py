"""GPU parity of extend (multi-query, causal) attention (paged_attn_extend) against the fp64
oracle: max-abs error <= 2e-3 (16-bit caches, fp32 output) on ragged batches with NaN-poisoned
unused slots; one new token per sequence agrees with the decode; a speculative-verification
batch at the GQA workload's shape and the benchmark's prefill chunk, every row; rejection of
bad calls."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_127_amd as pkv
import workloads as W
from tests.gpu_util import TOL, DeviceBatch, bits, max_err, widened

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load_library()


def _run(db, q, start, out_dtype=torch.float32, ws_fill=255):
    b = db.b
    T, Hq, d = q.shape
    maxq = int(np.diff(start).max())
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    ws = pkv.extend_workspace(b.num_seqs, T, Hq, b.num_kv_heads, d, maxq, db.max_ctx)
    ws.fill_(ws_fill)
    pkv.paged_attn_extend(out, q.cuda(), torch.from_numpy(start).cuda(), maxq, db.k_pool,
                          db.v_pool, db.tables, db.lens, db.max_ctx, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu()


# Runs whose rows per KV head (max new tokens x G) reach 128 take the kernel with
# workgroup-shared key/value tiles, shorter ones the row-state kernel; the first and third cases
# have a twin one token shorter that takes the other kernel.
CASES = [
    # context lengths (including the new tokens), new tokens, Hq, Hkv, d, B, dtype
    ([40, 17, 64, 5, 300], [3, 1, 16, 5, 0], 16, 2, 128, 16, "bf16"),
    ([40, 17, 64, 5, 300], [3, 1, 15, 5, 0], 16, 2, 128, 16, "bf16"),
    ([31, 70, 9, 513], [7, 7, 7, 7], 32, 2, 64, 16, "f16"),
    ([100, 33, 1000], [33, 33, 70], 8, 4, 128, 32, "bf16"),      # whole-sequence prefill
    ([31, 70, 9, 513], [8, 8, 8, 8], 32, 2, 64, 16, "f16"),       # G = 16
    ([2048, 1, 129], [12, 1, 64], 64, 8, 128, 16, "bf16"),
    ([77, 200], [40, 9], 24, 4, 64, 32, "bf16"),                  # G = 6
    ([150, 400, 60], [130, 200, 60], 4, 4, 128, 16, "bf16"),      # G = 1, whole-run prefill
    ([150, 400, 60], [100, 127, 60], 4, 4, 64, 32, "f16"),        # G = 1, one row short
    ([90, 300, 17], [3, 4, 1], 32, 1, 128, 16, "bf16"),           # G = 32 (multi-query): 128 rows
    ([90, 300, 17], [1, 3, 2], 34, 2, 64, 32, "f16"),             # G = 17
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{len(c[0])}-n{max(c[1])}-G{c[2] // c[3]}-d{c[4]}-B{c[5]}-{c[6]}")
def test_parity(case):
    lens, new, hq, hkv, d, B, dt = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    b = W.small_batch(lens, hq, hkv, d, B, DT[dt], seed=seed, poison=True)
    q, start = W.extend_queries(b, new, seed=seed + 1)
    got = _run(DeviceBatch(b), q, start)
    ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, B)
    err = float(np.abs(got.double().numpy() - ref).max())
    print(f"{case[1:]} max-abs {err:.3g}")
    assert np.isfinite(got.numpy()).all()
    assert err <= TOL[DT[dt]], err


def test_one_new_token_is_the_decode():
    b = W.small_batch([1, 15, 16, 17, 33, 100, 511, 1000], 16, 2, 128, 16, torch.bfloat16,
                      seed=12, poison=True)
    db = DeviceBatch(b)
    got = _run(db, b.q, np.arange(b.num_seqs + 1, dtype=np.int32))
    plain = db.decode()
    assert float((plain - got).abs().max()) <= 2e-3
    assert max_err(got, oracle.paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, 16)) <= 2e-3


def test_16bit_output_is_rounded_fp32_output():
    b = W.small_batch([40, 300], 16, 2, 128, 16, torch.bfloat16, seed=13)
    q, start = W.extend_queries(b, [7, 20], seed=14)
    db = DeviceBatch(b)
    f32 = _run(db, q, start)
    b16 = _run(db, q, start, out_dtype=torch.bfloat16)
    assert torch.equal(bits(b16), bits(f32.to(torch.bfloat16)))


def test_result_does_not_depend_on_workspace_contents():
    b = W.small_batch([90, 400], 8, 2, 128, 16, torch.bfloat16, seed=15)
    q, start = W.extend_queries(b, [30, 4], seed=16)
    db = DeviceBatch(b)
    assert torch.equal(bits(_run(db, q, start, ws_fill=0)), bits(_run(db, q, start, ws_fill=255)))


@pytest.mark.parametrize("lens,new,hq,hkv,d,B,dt", [
    ([3000, 40], [3, 5], 8, 1, 128, 16, "bf16"),
    ([2500], [4], 16, 2, 64, 32, "f16"),
    ([4000, 1, 700], [2, 1, 9], 32, 4, 128, 16, "bf16"),
])
def test_few_workgroups_long_contexts(lens, new, hq, hkv, d, B, dt):
    """Few row groups over long contexts: the plan spreads them over many chunk groups, each
    wavefront still gets at least 8 steps, so most chunk groups of the short rows (and the far
    ones of the long rows) have no step at all and write the empty state without loading
    anything. Against the oracle, with the workspace NaN-filled and zero-filled."""
    seed = zlib.crc32(repr((lens, new, hq)).encode()) % 10000
    b = W.small_batch(lens, hq, hkv, d, B, DT[dt], seed=seed, poison=True)
    q, start = W.extend_queries(b, new, seed=seed + 1)
    db = DeviceBatch(b)
    got = _run(db, q, start)
    ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, B)
    err = float(np.abs(got.double().numpy() - ref).max())
    print(f"{lens} {new} max-abs {err:.3g}")
    assert np.isfinite(got.numpy()).all()
    assert err <= TOL[DT[dt]], err
    assert torch.equal(bits(got), bits(_run(db, q, start, ws_fill=0)))


def test_one_chunk_group_writes_the_output_directly():
    """When the row groups alone fill the CUs (96 sequences x 4 KV heads, at most 24 rows each)
    and no row group is long, the plan uses one chunk group and the states kernel writes the
    normalised rows itself: no finish launch (the library's own launch timing shows none),
    parity with the oracle, 16-bit output = RNE of the fp32 output, sequences with no new
    token untouched."""
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(20, 600, size=96)]
    new = [int(x) for x in rng.integers(0, 7, size=96)]
    b = W.small_batch(lens, 16, 4, 128, 16, torch.bfloat16, seed=32, poison=True)
    q, start = W.extend_queries(b, new, seed=33)
    db = DeviceBatch(b)
    pkv.timing_enable(True, every=1)
    try:
        f32 = _run(db, q, start)
        torch.cuda.synchronize()
        _, n_states = pkv.timing_query("extend_states")
        _, n_finish = pkv.timing_query("extend_finish")
    finally:
        pkv.timing_enable(False)
    assert n_states >= 1 and n_finish == 0, (n_states, n_finish)
    ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    err = float(np.abs(f32.double().numpy() - ref).max())
    print(f"one chunk group, {int(start[-1])} query tokens: max-abs {err:.3g}")
    assert np.isfinite(f32.numpy()).all()
    assert err <= 2e-3, err
    b16 = _run(db, q, start, out_dtype=torch.bfloat16)
    assert torch.equal(bits(b16), bits(f32.to(torch.bfloat16)))


@pytest.mark.parametrize("S,hq,hkv,d,B,dt,nmax", [
    (41, 64, 8, 128, 16, "bf16", 4),    # G = 8: up to 32 rows per sequence
    (70, 16, 8, 64, 32, "f16", 16),     # G = 2, head_dim 64, block size 32
])
def test_short_runs_one_row_group(S, hq, hkv, d, B, dt, nmax):
    """Short runs with one row group per sequence and sequences x KV heads filling the CUs
    (one chunk group, streaming key/value loads): a sequence's steps go to as many of its
    workgroup's four wavefronts as get at least 8 steps each. Lengths straddle 256, 512 and
    513 tokens, tie, and include a one-token context; some sequences have no new token. Every
    row against the oracle, the workspace NaN-filled, and the 16-bit output = RNE of the fp32
    output."""
    rng = np.random.default_rng(S)
    lens = [int(x) for x in rng.integers(1, 1500, size=S)]
    lens[:8] = [512, 513, 512, 1, 1000, 1000, 256, 257]
    new = [min(int(x), L) for x, L in zip(rng.integers(0, nmax + 1, size=S), lens)]
    new[3] = 1
    new[7] = 0
    b = W.small_batch(lens, hq, hkv, d, B, DT[dt], seed=S + 1, poison=True)
    q, start = W.extend_queries(b, new, seed=S + 2)
    db = DeviceBatch(b)
    f32 = _run(db, q, start)
    ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, B)
    err = float(np.abs(f32.double().numpy() - ref).max())
    print(f"short runs S={S} G={hq // hkv}: max-abs {err:.3g} over {f32.shape[0]} rows")
    assert np.isfinite(f32.numpy()).all()
    assert err <= TOL[DT[dt]], err
    h16 = _run(db, q, start, out_dtype=DT[dt])
    assert torch.equal(bits(h16), bits(f32.to(DT[dt])))


def test_long_context_chunks():
    """A 32,768-token context with its last 16 tokens new (128 rows per KV head: the tile-sharing
    kernel with 16 chunk groups and the finish kernel) beside a 300-token one with 4 new tokens,
    and a verification-sized run (4 new tokens) at the end of another 32,768-token context on the
    row-state kernel; every row against the oracle."""
    for lens, new in (([32768, 300], [16, 4]), ([32768, 40], [4, 4])):
        b = W.small_batch(lens, 64, 8, 128, 16, torch.bfloat16, seed=32768 + new[0],
                          poison=True)
        q, start = W.extend_queries(b, new, seed=32769 + new[0])
        got = _run(DeviceBatch(b), q, start)
        ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
        err = float(np.abs(got.double().numpy() - ref).max())
        print(f"{lens} {new}: max-abs {err:.3g}")
        assert np.isfinite(got.numpy()).all()
        assert err <= 2e-3, err


def test_speculative_verification_at_gqa_shape():
    """The GQA decode workload (256 sequences, 64/8 heads, bf16, B 16, log-normal lengths), its
    last 4 stored tokens of each sequence taken as the new ones; every row of every sequence
    against the oracle."""
    b = W.config3(16)
    new = np.minimum(4, b.lengths)
    q, start = W.extend_queries(b, new, seed=17)
    got = _run(DeviceBatch(b), q, start)
    assert np.isfinite(got.numpy()).all()
    ref = oracle.extend_attention(q, start, widened(b.k_pool), widened(b.v_pool), b.tables,
                                  b.lengths, 16)
    err = float(np.abs(got.double().numpy() - ref).max())
    print(f"speculative verification: max-abs {err:.3g} over {got.shape[0]} rows")
    assert err <= 2e-3, err


def test_prefill_chunk_at_bench_shape():
    """The prefill chunk the benchmark times: 8 sequences of 1024..4096 stored tokens (64/8
    heads, d 128, bf16, B 16), the last 256 of each new; all 2,048 new tokens (every row group
    of every sequence, so the per-row causal limits and the unmasked steps below every row's
    limit are all covered) against the oracle."""
    b = W.small_batch(W.rng_for(W.SEED_BASE + 9, 0).integers(1024, 4096, size=8, endpoint=True),
                      64, 8, 128, 16, torch.bfloat16, seed=W.SEED_BASE + 9)
    new = np.full(8, 256)
    q, start = W.extend_queries(b, new, seed=72)
    got = _run(DeviceBatch(b), q, start)
    assert np.isfinite(got.numpy()).all()
    ref = oracle.extend_attention(q, start, widened(b.k_pool), widened(b.v_pool), b.tables,
                                  b.lengths, 16)
    err = float(np.abs(got.double().numpy() - ref).max())
    print(f"prefill chunk: max-abs {err:.3g} over {got.shape[0]} rows")
    assert err <= 2e-3, err


def test_rejections_and_validation():
    b = W.small_batch([40, 20], 16, 2, 128, 16, torch.bfloat16, seed=18)
    q, start = W.extend_queries(b, [4, 3], seed=19)
    db = DeviceBatch(b)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    qd, sd = q.cuda(), torch.from_numpy(start).cuda()
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attn_extend(out, qd, sd, 4, db.k_pool, db.v_pool, db.tables, db.lens,
                              db.max_ctx, workspace=small)
    assert e.value.code == -3
    pkv.set_validate(True)
    try:
        bad = sd.clone()
        bad[1] = 5                                     # sequence 0 would own 5 > max 4 rows
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_attn_extend(out, qd, bad, 4, db.k_pool, db.v_pool, db.tables, db.lens,
                                  db.max_ctx)
        assert e.value.code == -7
        short = db.lens.clone()
        short[1] = 2                                   # fewer stored tokens than new ones
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_attn_extend(out, qd, sd, 4, db.k_pool, db.v_pool, db.tables, short,
                                  db.max_ctx)
        assert e.value.code == -7
        pkv.paged_attn_extend(out, qd, sd, 4, db.k_pool, db.v_pool, db.tables, db.lens,
                              db.max_ctx)
        torch.cuda.synchronize()
    finally:
        pkv.set_validate(False)
    ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    assert float(np.abs(out.cpu().double().numpy() - ref).max()) <= 2e-3


@pytest.mark.parametrize("new", [[6, 5, 9], [20, 17, 30]], ids=["row-state", "shared-tile"])
def test_out_of_range_table_entry_gives_nan_rows(new):
    """An out-of-range block id among the blocks a sequence's new tokens attend (its first
    block, which every causal row sees) poisons that sequence's rows (NaN) without any access
    outside the pools; the other sequences match the oracle. Both kernels: 9 x 8 rows per KV
    head take the row-state kernel, 30 x 8 the shared-tile one."""
    b = W.small_batch([300, 90, 500], 16, 2, 128, 16, torch.bfloat16, seed=41)
    q, start = W.extend_queries(b, new, seed=42)
    db = DeviceBatch(b)
    db.tables = db.tables.clone()
    db.tables[1, 0] = b.num_blocks + 7
    got = _run(db, q, start)
    assert torch.isnan(got[int(start[1]):int(start[2])]).all()
    ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    for s in (0, 2):
        r = slice(int(start[s]), int(start[s + 1]))
        assert float(np.abs(got[r].double().numpy() - ref[r]).max()) <= 2e-3


def test_shared_prefix_and_extend_replay_in_a_hip_graph():
    """Both calls allocate nothing, launch only on the caller's stream and record no memset:
    captured together in a HIP graph, three replays (with eager work and synchronisations
    between them) reproduce the eager results bit for bit."""
    b = W.shared_prefix_batch([9, 120, 3, 300], 96, 16, 2, 128, 16, torch.bfloat16, seed=81,
                              poison=True)
    db = DeviceBatch(b)
    # 12 new tokens x G = 8 rows per KV head: the row-state kernel; 20 x 8: the shared-tile one
    q, start = W.extend_queries(b, [5, 9, 3, 12], seed=82)
    q2, start2 = W.extend_queries(b, [20, 17, 3, 18], seed=83)
    qd, sd = q.cuda(), torch.from_numpy(start).cuda()
    qd2, sd2 = q2.cuda(), torch.from_numpy(start2).cuda()
    pre = db.tables[0, :6].contiguous()
    out_sp = torch.empty(db.q.shape, dtype=torch.float32, device="cuda")
    out_ex = torch.empty(qd.shape, dtype=torch.bfloat16, device="cuda")
    out_ex2 = torch.empty(qd2.shape, dtype=torch.float32, device="cuda")
    ws_sp = pkv.shared_prefix_workspace(b.num_seqs, 16, 2, 128, 96)
    ws_ex = pkv.extend_workspace(b.num_seqs, qd.shape[0], 16, 2, 128, 12, db.max_ctx)
    ws_ex2 = pkv.extend_workspace(b.num_seqs, qd2.shape[0], 16, 2, 128, 20, db.max_ctx)

    def step():
        pkv.paged_attn_decode_shared_prefix(out_sp, db.q, db.k_pool, db.v_pool, pre, 96,
                                            db.tables, db.lens, db.max_ctx, workspace=ws_sp)
        pkv.paged_attn_extend(out_ex, qd, sd, 12, db.k_pool, db.v_pool, db.tables, db.lens,
                              db.max_ctx, workspace=ws_ex)
        pkv.paged_attn_extend(out_ex2, qd2, sd2, 20, db.k_pool, db.v_pool, db.tables, db.lens,
                              db.max_ctx, workspace=ws_ex2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref_sp, ref_ex, ref_ex2 = out_sp.clone(), out_ex.clone(), out_ex2.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        out_sp.fill_(float("nan"))
        out_ex.fill_(float("nan"))
        out_ex2.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out_sp.cpu()), bits(ref_sp.cpu()))
        assert torch.equal(bits(out_ex.cpu()), bits(ref_ex.cpu()))
        assert torch.equal(bits(out_ex2.cpu()), bits(ref_ex2.cpu()))
    kw, vw = widened(b.k_pool), widened(b.v_pool)
    assert max_err(ref_sp.cpu(), oracle.paged_decode(b.q, kw, vw, b.tables, b.lengths, 16)) <= 2e-3
    assert max_err(ref_ex2.cpu(), oracle.extend_attention(q2, start2, b.k_pool, b.v_pool, b.tables,
                                                          b.lengths, 16)) <= 2e-3


def test_random_shapes_sweep():
    """Thirty seeded random problems across the supported space -- cache dtype, G from 1 to 16,
    KV heads, head dim, block size, 1 to 12 sequences of 1 to 700 tokens with 0 to 40 new ones
    (both kernels: at least 128 rows per KV head takes the tile-sharing one) -- every row
    against the oracle, with the workspace NaN-filled."""
    rng = np.random.default_rng(78)
    for i in range(30):
        dt = ["bf16", "f16"][i % 2]
        G = int(rng.integers(1, 17))
        hkv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        B = int(rng.choice([16, 32]))
        S = int(rng.integers(1, 13))
        lens = [int(x) for x in rng.integers(1, 701, size=S)]
        new = [int(rng.integers(0, min(L, 40) + 1)) for L in lens]
        j = int(rng.integers(0, S))
        new[j] = max(1, new[j])                                    # at least one new token
        case = (dt, G, hkv, d, B, lens, new)
        print("case", case, flush=True)
        b = W.small_batch(lens, G * hkv, hkv, d, B, DT[dt], seed=6000 + i, poison=True)
        q, start = W.extend_queries(b, new, seed=6100 + i)
        got = _run(DeviceBatch(b), q, start)
        ref = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, B)
        assert np.isfinite(got.numpy()).all(), case
        assert float(np.abs(got.double().numpy() - ref).max()) <= TOL[DT[dt]], case
