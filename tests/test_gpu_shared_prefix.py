"""GPU parity of the shared-prefix decode (paged_attn_decode_shared_prefix) against the plain
fp64 definition, oracle.paged_decode over each sequence's whole block table: max-abs error
<= 2e-3 (16-bit caches, fp32 output) on every output row, on ragged batches whose sequences
share a prefix of whole blocks (unused slots poisoned with NaN) and on the shared-prefix
workload at full size; rejection of bad calls.

The reference is the plain attention over each table, not the prefix/suffix split the kernel
uses: sharing blocks changes addressing only ("PagedAttention: Virtual Memory for the KV
Cache", section "A block table preserves token order"), so the definition is the same as for
the plain decode."""
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


def _ref(b):
    """The plain definition: every sequence's attention through its own table."""
    return oracle.paged_decode(b.q, widened(b.k_pool), widened(b.v_pool), b.tables, b.lengths,
                               b.block_size)


def _run(db, P, out_dtype=torch.float32, workers=0, ws_fill=255):
    b = db.b
    B = b.block_size
    S, Hq, d = b.q.shape
    out = torch.full(db.q.shape, float("nan"), dtype=out_dtype, device="cuda")
    ws = pkv.shared_prefix_workspace(S, Hq, b.num_kv_heads, d, P, workers)
    ws.fill_(ws_fill)
    pre = db.tables[0, :P // B].contiguous()
    pkv.paged_attn_decode_shared_prefix(out, db.q, db.k_pool, db.v_pool, pre, P, db.tables,
                                        db.lens, db.max_ctx, num_workers=workers, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu()


CASES = [
    # suffix lengths, prefix tokens, Hq, Hkv, d, B, dtype
    ([1, 15, 16, 17, 33, 100, 511, 0], 64, 16, 2, 128, 16, "bf16"),
    ([3, 40, 200], 48, 8, 4, 128, 16, "bf16"),          # prefix of 1.5 steps, G = 2
    ([0, 0, 5], 32, 16, 1, 64, 32, "f16"),              # G = 16, head_dim 64
    ([7, 300, 64, 1, 90, 33], 256, 32, 8, 128, 32, "bf16"),
    ([12] * 20, 800, 64, 8, 128, 16, "bf16"),           # 160 rows: three row groups
    ([500, 1, 250, 31], 16, 24, 4, 64, 16, "f16"),      # one prefix block, G = 6
    (list(range(1, 70)), 112, 16, 2, 128, 16, "bf16"),  # 69 sequences, 552 rows per head
    # prefixes past 4096 tokens with at least 128 rows per KV head: the kernel whose four
    # wavefronts share each step's keys and values among four 32-row tiles
    ([3, 0, 40, 1, 17, 9, 2, 100, 5, 6, 7, 8, 11, 13, 64, 31, 1], 4128, 16, 2, 128, 16,
     "bf16"),                                            # 136 rows: a second, ragged row group
    ([1, 2, 3, 0, 50, 7, 9, 33, 12], 4160, 64, 4, 64, 32, "f16"),   # G = 16, 130 blocks of 32
    ([5] * 64, 4112, 4, 2, 128, 16, "bf16"),            # G = 2, 128 rows, a half last step
    # G = 1 (multi-head): the suffix decode on the matrix-core kernel with one real row
    ([1, 15, 16, 17, 33, 100, 511, 0], 64, 4, 4, 128, 16, "bf16"),
    ([3, 0, 250, 40, 9], 96, 8, 8, 64, 32, "f16"),
    ([7] * 130, 4128, 2, 2, 128, 16, "bf16"),           # 130 rows: the tile-sharing prefix kernel
    # more than 16 query heads per KV head: the suffix decode as several schedule heads
    ([1, 15, 16, 17, 33, 100, 0], 64, 32, 1, 128, 16, "bf16"),    # G = 32: two of 16
    ([3, 250, 40, 9], 96, 17, 1, 64, 32, "f16"),                  # G = 17: seventeen of one
    ([2] * 8, 4112, 48, 1, 64, 16, "bf16"),                       # G = 48, the wide prefix kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{len(c[0])}-P{c[1]}-G{c[2] // c[3]}-d{c[4]}-B{c[5]}-{c[6]}")
@pytest.mark.parametrize("workers", [0, 7])
def test_parity(case, workers):
    suf, P, hq, hkv, d, B, dt = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    b = W.shared_prefix_batch(suf, P, hq, hkv, d, B, DT[dt], seed=seed, poison=True)
    db = DeviceBatch(b)
    got = _run(db, P, workers=workers)
    err = max_err(got, _ref(b))
    print(f"{case[1:]} S={len(suf)} workers={workers} max-abs {err:.3g}")
    assert np.isfinite(got.numpy()).all()
    assert err <= TOL[DT[dt]], err


def test_16bit_output_is_rounded_fp32_output():
    b = W.shared_prefix_batch([5, 77, 0, 300], 64, 16, 2, 128, 16, torch.bfloat16, seed=5)
    db = DeviceBatch(b)
    f32 = _run(db, 64)
    b16 = _run(db, 64, out_dtype=torch.bfloat16)
    assert torch.equal(bits(b16), bits(f32.to(torch.bfloat16)))


@pytest.mark.parametrize("prefix_len", [800, 4096, 8192])
def test_shared_prefix_workload_full_size(prefix_len):
    """128 sequences over an 800-, 4096- or 8192-token prefix with U{1..512}-token suffixes
    (64/8 heads, head_dim 128, bf16, block size 16), in the launch configuration the benchmark
    times (800 and 4096: the row-state kernel, one chunk group of up to 32 steps per
    wavefront; 8192: the kernel that shares key/value tiles among row tiles, eight chunk
    groups); every row of all 128 sequences against the oracle."""
    b = W.config4a(prefix_len=prefix_len)
    db = DeviceBatch(b)
    got = _run(db, prefix_len)
    assert np.isfinite(got.numpy()).all()
    err = max_err(got, _ref(b))
    print(f"shared-prefix workload, prefix {prefix_len}: max-abs {err:.3g} on all 128 sequences")
    assert err <= 2e-3, err


@pytest.mark.parametrize("hq,hkv", [(8, 1), (16, 4)])
def test_most_sharers_per_call(hq, hkv):
    """4,096 sequences (the most one call takes) over a 4-block prefix with 0..40-token suffixes,
    G = 8 and G = 4: every row against the plain oracle (4,097 is rejected on the host before
    anything is enqueued: test_library_host)."""
    rng = np.random.default_rng(4096 + hq)
    suf = [int(x) for x in rng.integers(0, 41, size=4096)]
    b = W.shared_prefix_batch(suf, 64, hq, hkv, 64, 16, torch.bfloat16, seed=4096 + hq,
                              poison=True)
    db = DeviceBatch(b)
    got = _run(db, 64)
    assert np.isfinite(got.numpy()).all()
    err = max_err(got, _ref(b))
    print(f"4096 sharers, G = {hq // hkv}: max-abs {err:.3g}")
    assert err <= 2e-3, err


def test_result_does_not_depend_on_workspace_contents():
    b = W.shared_prefix_batch([9, 120, 3], 96, 16, 2, 128, 16, torch.bfloat16, seed=8)
    db = DeviceBatch(b)
    a = _run(db, 96, ws_fill=0)
    c = _run(db, 96, ws_fill=255)
    assert torch.equal(bits(a), bits(c))


def test_rejections_and_validation():
    b = W.shared_prefix_batch([9, 20], 32, 16, 2, 128, 16, torch.bfloat16, seed=4)
    db = DeviceBatch(b)
    out = torch.empty(db.q.shape, dtype=torch.float32, device="cuda")
    pre = db.tables[0, :2].contiguous()
    with pytest.raises(pkv.PagedKVError) as e:     # prefix not whole blocks
        pkv.paged_attn_decode_shared_prefix(out, db.q, db.k_pool, db.v_pool, pre, 24, db.tables,
                                            db.lens, db.max_ctx)
    assert e.value.code == -1
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attn_decode_shared_prefix(out, db.q, db.k_pool, db.v_pool, pre, 32, db.tables,
                                            db.lens, db.max_ctx, workspace=small)
    assert e.value.code == -3
    pkv.set_validate(True)
    try:
        bad = db.tables.clone()
        bad[1, 0] = bad[1, 2]                      # a table that does not share the prefix
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_attn_decode_shared_prefix(out, db.q, db.k_pool, db.v_pool, pre, 32, bad,
                                                db.lens, db.max_ctx)
        assert e.value.code == -7
        short = db.lens.clone()
        short[0] = 20                              # shorter than the prefix
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_attn_decode_shared_prefix(out, db.q, db.k_pool, db.v_pool, pre, 32,
                                                db.tables, short, db.max_ctx)
        assert e.value.code == -7
        pkv.paged_attn_decode_shared_prefix(out, db.q, db.k_pool, db.v_pool, pre, 32, db.tables,
                                            db.lens, db.max_ctx)
        torch.cuda.synchronize()
    finally:
        pkv.set_validate(False)
    assert max_err(out.cpu(), _ref(b)) <= 2e-3


def test_random_shapes_sweep():
    """Twenty-four seeded random problems across the supported space -- cache dtype, G from 1
    to 16, KV heads, head dim, block size, worker count, output dtype, prefix of 1 to 20 blocks,
    ragged suffixes with empty ones -- and four with prefixes past 4096 tokens and at least 128
    rows per KV head (the tile-sharing prefix kernel), every row against the plain oracle; a
    16-bit output is the RNE of the fp32 one."""
    rng = np.random.default_rng(77)
    for i in range(28):
        dt = ["bf16", "f16"][i % 2]
        G = int(rng.integers(1, 17))
        hkv = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        B = int(rng.choice([16, 32]))
        workers = int(rng.choice([0, 7, 64, 2000]))
        if i < 24:
            S = int(rng.integers(1, 41))
            P = B * int(rng.integers(1, 21))
        else:                                     # wide prefix mode: S * G >= 128, P > 4096
            G = int(rng.choice([2, 4, 8, 16]))
            hkv = int(rng.choice([1, 2]))
            S = -(-128 // G) + int(rng.integers(0, 9))
            P = 4096 + B * int(rng.integers(1, 5))
        suf = [int(x) for x in rng.integers(0, 300, size=S)]
        case = (dt, G, hkv, d, B, S, P, workers)
        print("case", case, flush=True)
        b = W.shared_prefix_batch(suf, P, G * hkv, hkv, d, B, DT[dt], seed=5000 + i, poison=True)
        db = DeviceBatch(b)
        got = _run(db, P, workers=workers)
        assert np.isfinite(got.numpy()).all(), case
        assert max_err(got, _ref(b)) <= TOL[DT[dt]], case
        if i % 4 == 0:
            h16 = _run(db, P, out_dtype=DT[dt], workers=workers)
            assert torch.equal(bits(h16), bits(got.to(DT[dt]))), case
