"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Every comparison uses the same seeded inputs on both sides, element by element
over the whole output, at every size: the full-size workloads run with the
same plan the benchmark uses.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import compare, require_gpu, run_gpu, upload
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, va = require_gpu()
    return torch, va


def _oracle(w, heads=None):
    return oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens, w.tree_mask,
                                   w.scale, heads=heads)


def _check(env, w, heads=None, label=None, **kw):
    torch, va = env
    d = upload(w)
    out, lse = run_gpu(va, d, w.scale, **kw)
    ro, rl = _oracle(w, heads)
    if heads is not None:
        out, lse, ro, rl = out[:, :, heads], lse[:, :, heads], ro[:, :, heads], rl[:, :, heads]
    m = compare(out, lse, ro, rl, label or w.name)
    print(f"[parity] {label or w.name}: {m}", flush=True)
    return out, lse


@pytest.mark.parametrize("name", ["tiny", "p4k", "tree32k"])
def test_config_full_oracle(env, name):
    print(f"[parity] start {name}", flush=True)
    _check(env, make_config(name))


@pytest.mark.parametrize("name", ["long185k", "batch8", "long185k_h8"])
def test_config_full_size_whole_output(env, name):
    print(f"[parity] start {name} (all heads)", flush=True)
    _check(env, make_config(name))


def test_batch48_column_plan_whole_output(env):
    """48 sequences of 500 to 8000 keys at 64 heads and 8 verify positions (about
    200k keys; 4 row tiles, so a budget of 64 columns for 48 sequences: the column
    plan at scale: 110 pieces over 64 columns), whole output against
    the oracle."""
    w = make_workload("batch48_mixed", [915, 48], B=48, Q=8, H=64, prefix_range=(500, 8000), mask="tree")
    print(f"[parity] start batch48_mixed: total_kv={w.total_kv}", flush=True)
    _check(env, w, label="batch48_mixed")


EDGE_CASES = {
    "no_prefix": dict(B=1, Q=16, H=8, prefix_lens=[0], mask="chain", num_slots=64),
    "single_query": dict(B=1, Q=1, H=16, prefix_lens=[1000], mask="chain", num_slots=4096),
    "ragged_batch_row_padding": dict(B=5, Q=7, H=5, prefix_lens=[0, 1, 31, 33, 1000], mask="tree",
                                     num_slots=3000),
    "max_q_tree": dict(B=1, Q=64, H=3, prefix_lens=[300], mask="tree", num_slots=1000),
    "wide_rows": dict(B=2, Q=16, H=24, prefix_lens=[777, 2000], mask="tree", num_slots=4000),
    "tail_invisible": dict(B=2, Q=4, H=8, prefix_lens=[40, 3], mask="none", num_slots=100),
}


@pytest.mark.parametrize("case", list(EDGE_CASES))
def test_edge_cases(env, case):
    kw = EDGE_CASES[case]
    w = make_workload(case, [300, len(case)], **kw)
    _check(env, w, label=case)


def test_empty_visible_set(env):
    tm = np.ones((2, 3, 3), np.uint8)
    tm[0, 1, :] = 0                        # sequence 0 has no prefix: query 1 sees nothing
    w = make_workload("empty", [301], B=2, Q=3, H=8, prefix_lens=[0, 10], mask=tm, num_slots=64)
    out, lse = _check(env, w)
    assert np.all(np.isneginf(lse[0, 1])) and np.all(out[0, 1] == 0)


def test_many_small_chunks_cross_the_tail(env):
    """A tiny chunk length puts chunk boundaries inside prefixes and tails and makes
    the merge combine dozens of partials, some of them empty for some rows."""
    torch, va = env
    w = make_workload("chunks", [302], B=6, Q=12, H=4, prefix_lens=[1000, 1001, 1003, 1005, 20, 0],
                      mask="tree", num_slots=5000)
    # one, two, three and four tiles per chunk: the pipeline's prologue and
    # drain at every depth of the tile ring
    for chunk in (32, 64, 96, 128):
        _check(env, w, label=f"chunk{chunk}", chunk_keys=chunk)


def test_chunk_ending_where_the_tail_starts(env):
    """Chunk lengths that divide the prefix, so that a chunk ends exactly where the
    speculative tail starts: that chunk must not need the tail mask (it loads it
    only when it reaches the tail), and the next one holds the whole tail."""
    w = make_workload("tailedge", [310], B=2, Q=8, H=16, prefix_lens=[1024, 512], mask="tree", num_slots=2000)
    for chunk in (32, 256, 512):
        _check(env, w, label=f"tailedge{chunk}", chunk_keys=chunk)


def test_many_chunks_per_sequence_slice_merge(env):
    """32-key chunks over ragged sequences give at least 64 chunks per sequence on
    average, so the merge runs in its slice form (one workgroup per row and 64-dim
    slice, 32 chunk lanes): sequences with 126, 1 and 79 chunks, one without prefix,
    and a query with nothing visible."""
    tm = np.stack([np.tril(np.ones((4, 4), np.uint8))] * 3)
    tm[1, 2, :] = 0                       # sequence 1 has no prefix: query 2 sees nothing
    w = make_workload("slice", [308], B=3, Q=4, H=40, prefix_lens=[4000, 0, 2500], mask=tm, num_slots=8000)
    torch, va = env
    plan = va.query_plan(w.B, w.Q, w.H, w.total_kv, chunk_keys=32)
    assert plan["max_chunks"] >= 64 * w.B
    out, lse = _check(env, w, label="slice_merge", chunk_keys=32)
    assert np.all(np.isneginf(lse[1, 2])) and np.all(out[1, 2] == 0)


def test_prefix_length_past_the_array(env):
    """A prefix length larger than the array holds (prefix_lens[0] + Q > total_kv):
    the header's rule is that positions past total_kv are absent, so every one of
    the total_kv positions counts as prefix and is visible to every query. The plan
    then has a last chunk that lies wholly past the array (it must still get a
    workgroup and leave an empty partial). Expected: the oracle on the same rows
    with the last Q positions as a fully visible tail, which is the same visible
    set."""
    torch, va = env
    w = make_workload("past", [311], B=1, Q=8, H=16, prefix_lens=[3000], mask="chain", num_slots=4096)
    assert w.total_kv == 3008 and w.total_kv % 32 == 0
    d = upload(w)
    d["prefix_lens"].fill_(w.total_kv)    # claims 3008 prefix positions + 8 tail positions
    ref = oracle.verify_attention(w.q, w.kv_pool, w.kv_indices, w.prefix_lens,
                                  np.ones_like(w.tree_mask), w.scale)
    for chunk in (0, 32):                 # the automatic plan, and one chunk per tile
        if chunk:
            plan = va.query_plan(w.B, w.Q, w.H, w.total_kv, chunk_keys=chunk)
            assert plan["grid"] >= (w.total_kv + w.Q + chunk - 1) // chunk
        out, lse = run_gpu(va, d, w.scale, chunk_keys=chunk)
        m = compare(out, lse, *ref, f"past{chunk}")
        print(f"[parity] past{chunk}: {m}", flush=True)


def test_out_of_range_slots_read_as_zero_rows(env):
    w = make_workload("oob", [303], B=2, Q=4, H=8, prefix_lens=[50, 9], mask="tree", num_slots=128)
    bad = w.kv_indices.copy()
    bad[3] = w.num_slots + 7
    bad[60] = -5
    w.kv_indices = bad
    torch, va = env
    out, lse = run_gpu(va, upload(w), w.scale)
    # oracle view: the library reads such entries as all-zero rows
    pool = np.concatenate([w.kv_pool, np.zeros((1, 576), np.uint16)])
    idx = np.where((bad < 0) | (bad >= w.num_slots), w.num_slots, bad).astype(np.int32)
    ro, rl = oracle.verify_attention(w.q, pool, idx, w.prefix_lens, w.tree_mask, w.scale)
    compare(out, lse, ro, rl, "oob")


def test_duplicate_slots(env):
    w = make_workload("dup", [304], B=1, Q=8, H=8, prefix_lens=[200], mask="chain", num_slots=256)
    idx = w.kv_indices.copy()
    idx[100:150] = idx[0:50]
    w.kv_indices = idx
    _check(env, w, label="duplicates")


def test_bf16_dtype_and_side_stream(env):
    torch, va = env
    w = make_workload("dtype", [305], B=2, Q=4, H=16, prefix_lens=[300, 77], mask="tree", num_slots=600)
    d = upload(w)
    d["q"] = d["q"].view(torch.bfloat16)
    d["kv_pool"] = d["kv_pool"].view(torch.bfloat16)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = va.verify_attn(d["q"], d["kv_pool"], d["kv_indices"], d["prefix_lens"],
                                  d["tree_mask"], float(w.scale), stream=s)
    s.synchronize()
    ro, rl = _oracle(w)
    compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl, "dtype")


def test_deterministic_and_relabel_invariant_bitwise(env):
    """Identical inputs give identical bits; so does relabelling the pool (rows and
    kv_indices permuted together), which pins the gather order exactly."""
    torch, va = env
    w = make_workload("relabel", [306], B=3, Q=8, H=16, prefix_lens=[3000, 50, 1200], mask="tree",
                      num_slots=8192)
    d = upload(w)
    o1, l1 = run_gpu(va, d, w.scale)
    o2, l2 = run_gpu(va, d, w.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    perm = np.random.default_rng(9).permutation(w.num_slots)
    pool2 = np.empty_like(w.kv_pool)
    pool2[perm] = w.kv_pool
    d2 = dict(d)
    d2["kv_pool"] = torch.from_numpy(pool2.view(np.int16)).cuda()
    d2["kv_indices"] = torch.from_numpy(perm[w.kv_indices].astype(np.int32)).cuda()
    o3, l3 = run_gpu(va, d2, w.scale)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 1000])
def test_debug_gather_bit_exact(env, n):
    torch, va = env
    rng = np.random.default_rng(n)
    pool = rng.integers(0, 1 << 16, size=(2048, 576), dtype=np.uint16)
    idx = rng.integers(0, 2048, size=n).astype(np.int32)
    if n > 5:
        idx[2] = 5000          # out of range -> zero row
        idx[4] = -1
    dpool = torch.from_numpy(pool.view(np.int16)).cuda()
    rows = va.debug_gather(dpool, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    got = rows.cpu().numpy().view(np.uint16)
    want = np.where(((idx >= 0) & (idx < 2048))[:, None], pool[np.clip(idx, 0, 2047)], 0).astype(np.uint16)
    assert np.array_equal(got, want)


def test_late_max_growth_rescales_some_rows(env):
    """Keys aligned with one query-head row late in the sequence make that row's
    running max jump long after the first tile while its neighbours' maxima stay
    put, so the lazy rescale has to act on a subset of rows only."""
    torch, va = env
    w = make_workload("growth", [307], B=1, Q=4, H=32, prefix_lens=[3000], mask="chain", num_slots=4096)
    qrow = w.q[0, 1, 5].astype(np.uint32) << 16           # query position 1, head 5
    qf = qrow.view(np.float32) * np.float32(0.25)
    from workloads import bf16_from_f32
    for pos in (1500, 2800, 2999):
        w.kv_pool[w.kv_indices[pos]] = bf16_from_f32(qf)
    qrow2 = w.q[0, 3, 30].astype(np.uint32) << 16         # another row grows in a different chunk
    w.kv_pool[w.kv_indices[700]] = bf16_from_f32(qrow2.view(np.float32) * np.float32(0.2))
    for chunk in (0, 1024):
        _check(env, w, label=f"growth_chunk{chunk}", chunk_keys=chunk)


def _sweep_cases(n=24, seed=911):
    """Seeded random shapes: batch, draft length, heads, ragged prefixes (including
    empty ones), mask kind and a forced chunk length, so that plans with one to
    many chunks per sequence and row tiles with padding rows all occur."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        Q = int(rng.integers(1, 17))
        H = int(rng.integers(1, 25))
        prefix = [int(x) for x in rng.integers(0, 1500, size=B)]
        if i % 5 == 0:
            prefix[0] = 0
        mask = ["chain", "tree", "none", "identity"][i % 4]
        chunk = [0, 32, 64, 160][(i // 4) % 4]
        cases.append((i, B, Q, H, prefix, mask, chunk))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"sweep{c[0]}")
def test_random_shape_sweep(env, case):
    i, B, Q, H, prefix, mask, chunk = case
    torch, va = env
    w = make_workload(f"sweep{i}", [912, i], B=B, Q=Q, H=H, prefix_lens=prefix, mask=mask,
                      num_slots=sum(prefix) + B * Q + 64)
    print(f"[parity] sweep{i}: B={B} Q={Q} H={H} prefix={prefix} mask={mask} chunk={chunk}", flush=True)
    _check(env, w, label=f"sweep{i}", chunk_keys=chunk)


def _column_sweep_cases(n=12, seed=913):
    """Seeded random batches under the automatic plan (the column plan): up to 40
    sequences of ragged lengths, some empty and some a single tile, so that columns
    cross sequence boundaries, hold several short sequences, or start inside a
    sequence's start-up units."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(2, 41))
        Q = int(rng.integers(1, 9))
        H = int(rng.integers(1, 33))
        hi = [40, 600, 3000][i % 3]
        prefix = [int(x) for x in rng.integers(0, hi, size=B)]
        prefix[int(rng.integers(0, B))] = 0
        mask = ["chain", "tree"][i % 2]
        cases.append((i, B, Q, H, prefix, mask))
    return cases


@pytest.mark.parametrize("case", _column_sweep_cases(), ids=lambda c: f"columns{c[0]}")
def test_column_plan_sweep(env, case):
    i, B, Q, H, prefix, mask = case
    w = make_workload(f"columns{i}", [914, i], B=B, Q=Q, H=H, prefix_lens=prefix, mask=mask,
                      num_slots=sum(prefix) + B * Q + 64)
    print(f"[parity] columns{i}: B={B} Q={Q} H={H} prefix sum={sum(prefix)} mask={mask}", flush=True)
    _check(env, w, label=f"columns{i}")


def _plan_model(w, plan, ncu):
    """The split plan's piece offsets written out plainly. With fewer sequences than
    the budget of CUs / row_tiles columns (and at most 512): lay every sequence's
    32-key tiles end to end, each preceded by 3 units standing for a piece's
    start-up, cut the axis of U units into columns of ceil(U / C) units (C = the
    budget, at most max_chunks - B + 1 and at most the launched columns), and give
    a sequence one piece per column its tiles meet.
    Otherwise every chunk of the host's length is a piece. Offsets are running sums
    of pieces per sequence, capped at the partial buffers' capacity."""
    n = np.clip(w.prefix_lens.astype(np.int64), 0, w.total_kv) + w.Q
    budget = max(1, ncu // plan["row_tiles"])
    if budget > w.B and w.B <= 512:
        tiles = -(-n // 32)
        units_end = np.cumsum(tiles + 3)
        first_tile = units_end - tiles
        U = int(units_end[-1])
        C = max(1, min(budget, plan["max_chunks"] - w.B + 1, plan["grid"] // plan["row_tiles"]))
        width = -(-U // C)
        pieces = (units_end - 1) // width - first_tile // width + 1
        desc = f"{C} columns"
    else:
        pieces = -(-n // plan["chunk_keys"])
        desc = f"chunks of {plan['chunk_keys']} keys"
    off = np.concatenate([[0], np.cumsum(pieces)])
    return np.minimum(off, plan["max_chunks"]).astype(np.int32), desc


@pytest.mark.parametrize("label,B,Q,H,prefix", [
    ("batch600_two_scan_passes", 600, 2, 4, (0, 60)),    # more sequences than the budget; two scan passes
    ("batch300_over_budget", 300, 3, 4, (0, 80)),         # more sequences than the budget; one pass
    ("batch100_columns", 100, 4, 2, (696, 696)),          # equal sequences, 256 columns
    ("batch8_ragged_columns", 8, 4, 2, (4000, 30000)),    # ragged lengths: columns cross sequences
    ("batch40_short_columns", 40, 4, 64, (0, 300)),       # several short sequences per column
    ("batch2_uneven_columns", 2, 16, 64, (100, 60000)),   # one short, one long sequence
    ("batch250_columns", 250, 4, 2, (0, 60)),             # just under the budget: many pieces per column
    ("batch3_tiny_columns", 3, 1, 8, (0, 10)),            # fewer axis units than columns
])
def test_chunk_plan_batches(env, label, B, Q, H, prefix):
    """Large and ragged batches through the split plan that every split workgroup
    computes for itself: parity with the oracle, and the piece offsets that
    workgroup 0 leaves at the start of the workspace for the merge (int32 [B+1])
    equal the rule's."""
    torch, va = env
    w = make_workload(label, [916, B], B=B, Q=Q, H=H, prefix_range=prefix, mask="tree")
    print(f"[parity] start {label}: B={B} Q={Q} H={H} total_kv={w.total_kv}", flush=True)
    plan = va.query_plan(B, Q, H, w.total_kv)
    ws = va.alloc_workspace(B, Q, H, w.total_kv)
    ws.fill_(0xFF)
    _check(env, w, label=label, workspace=ws)
    got = ws[: 4 * (B + 1)].cpu().numpy().view(np.int32)
    want, desc = _plan_model(w, plan, torch.cuda.get_device_properties(0).multi_processor_count)
    print(f"[parity] {label}: {desc}, {want[-1]} pieces", flush=True)
    assert np.array_equal(got, want), f"{label}: piece offsets differ from the plan rule"


def test_defragmented_cache_full_size_bitwise_equal(env):
    """The 8-head 185k workload over a shuffled pool and over the same rows laid out
    contiguously (what KV defragmentation produces): same q, same rows, only the
    slots differ, so the output must be identical bit for bit."""
    torch, va = env
    w1, w2 = make_config("long185k_h8"), make_config("long185k_h8_contig")
    assert np.array_equal(w1.kv_pool[w1.kv_indices], w2.kv_pool[w2.kv_indices])
    o1, l1 = run_gpu(va, upload(w1), w1.scale)
    o2, l2 = run_gpu(va, upload(w2), w2.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _scale_bf16(bits, s):
    """bf16 bit patterns times a power of two (exact in bf16 for these magnitudes)."""
    f = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(s)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def test_scale_equivariance_large_values(env):
    """Latents times 16 and queries times 1/16 leave every score unchanged and scale
    out by 16 exactly, lse not at all. The relative error must stay within the bar
    and the absolute error may grow with the values (here |v| up to about 100):
    the value operands and the chunk partials are fp16, whose rounding is relative
    to the magnitude."""
    s = 16.0
    w = make_workload("big", [306], B=2, Q=8, H=16, prefix_lens=[700, 1500], mask="tree", num_slots=3000)
    w.kv_pool = _scale_bf16(w.kv_pool, s)
    w.q = _scale_bf16(w.q, 1.0 / s)
    torch, va = env
    out, lse = run_gpu(va, upload(w), w.scale)
    ro, rl = _oracle(w)
    assert np.isfinite(ro).all() and np.isfinite(rl).all()
    rel = float(np.linalg.norm(out - ro) / np.linalg.norm(ro))
    mabs = float(np.abs(out - ro).max())
    labs = float(np.abs(lse - rl).max())
    print(f"[parity] scaled x{s:g}: rel_l2={rel:.3e} max_abs={mabs:.3e} lse_abs={labs:.3e}", flush=True)
    assert rel <= 1e-3 and mabs <= s * 5e-3 and labs <= 1e-3
    # the same inputs unscaled give out / 16 up to rounding of the same size, relatively
    w0 = make_workload("big", [306], B=2, Q=8, H=16, prefix_lens=[700, 1500], mask="tree", num_slots=3000)
    out0, lse0 = run_gpu(va, upload(w0), w0.scale)
    assert float(np.linalg.norm(out / s - out0) / np.linalg.norm(out0)) <= 1e-3
    assert float(np.abs(lse - lse0).max()) <= 1e-3
