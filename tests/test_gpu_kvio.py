"""KV-cache offload / reload and chunked prefill over a reloaded prefix, through the C ABI.

* nf_kv_offload: token-major host rows of arbitrary ranges (unaligned starts, partial last
  blocks, empty ranges, several requests) bit-exact against the oracle's gather, for head
  dims 64 and 128;
* nf_kv_reload: the pool after a reload bit-exact against the oracle's (every slot of the
  ranges set, every other byte unchanged); aliasing ranges and bad block ids rejected on the
  host with the pool untouched;
* a follow-up turn: a prefill chunk is processed, its K/V offloaded, reloaded into other
  pages of a fresh pool, and the request's next chunk runs as a prefill with that cached
  prefix. The GPU's second-turn output against the oracle doing the same on its own first-turn
  K/V.
"""

import numpy as np
import pytest

from oracle import kvio
from oracle import layer as ol
from synth import workloads as sw
from tests.gpu_util import TOL, f64, log_case, rand_bf16, rel_inf

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    from nano_intra_overlap_amd import abi

    c = abi.nf_ctx_create(0)
    yield c
    abi.nf_ctx_destroy(c)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _pinned_u16(shape):
    return torch.empty(shape, dtype=torch.int16, pin_memory=True)


def _ranges_case(rng, num_blocks, n_req, max_blocks):
    """Random ranges over distinct blocks (no slot shared)."""
    perm = rng.permutation(num_blocks)
    table = np.full((n_req, max_blocks), -1, np.int32)
    first, n_tok = [], []
    used = 0
    for r in range(n_req):
        nb = int(rng.integers(1, max_blocks + 1))
        table[r, :nb] = perm[used:used + nb]
        used += nb
        p0 = int(rng.integers(0, nb * 16))
        n = int(rng.integers(0, nb * 16 - p0 + 1))
        first.append(p0)
        n_tok.append(n)
    return np.array(first), np.array(n_tok), table


@pytest.mark.parametrize("name", ["tiny", "llama3_8b_layer"])
def test_kv_offload_and_reload_match_oracle(ctx, name):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool

    shape = sw.WORKLOADS[name].shape
    cfg = abi.make_cfg(shape)
    rng = np.random.default_rng(3)
    nb = 80
    kp, vp = sw.make_kv_pool(shape, nb, 4)
    for trial in range(4):
        first, n_tok, table = _ranges_case(rng, nb, 5, 8)
        hr = abi.HostKvRanges(first, n_tok, table)
        pool = DevicePool.from_host(kp, vp, "cuda")
        rows_d = _pinned_u16((max(hr.n_rows, 1), 2, shape.n_kv, shape.head_dim))
        log_case(f"kv offload {name} trial {trial}: {hr.n_rows} tokens")
        abi.nf_kv_offload(ctx, cfg, pool.desc, hr, rows_d.data_ptr(), _stream())
        torch.cuda.synchronize()
        want = kvio.offload(kp, vp, first, n_tok, table)
        assert np.array_equal(rows_d.numpy().view(np.uint16)[:hr.n_rows], want)
        kg, vg = pool.host_bits()
        assert np.array_equal(kg, kp) and np.array_equal(vg, vp)  # offload leaves the pool alone

        new_rows = rand_bf16(rng, (hr.n_rows, 2, shape.n_kv, shape.head_dim))
        src = _pinned_u16((max(hr.n_rows, 1), 2, shape.n_kv, shape.head_dim))
        src.numpy()[:hr.n_rows] = new_rows.view(np.int16)
        log_case(f"kv reload {name} trial {trial}")
        abi.nf_kv_reload(ctx, cfg, pool.desc, hr, src.data_ptr(), _stream())
        torch.cuda.synchronize()
        k_ref, v_ref = kvio.reload(kp, vp, first, n_tok, table, new_rows)
        kg, vg = pool.host_bits()
        assert np.array_equal(kg, k_ref) and np.array_equal(vg, v_ref)


def test_kv_reload_rejects_bad_ranges_without_touching_the_pool(ctx):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool

    shape = sw.WORKLOADS["tiny"].shape
    cfg = abi.make_cfg(shape)
    kp, vp = sw.make_kv_pool(shape, 10, 5)
    pool = DevicePool.from_host(kp, vp, "cuda")
    src = _pinned_u16((64, 2, shape.n_kv, shape.head_dim))
    cases = [
        ("two ranges on one slot", abi.HostKvRanges([0, 3], [8, 8], [[4, -1], [4, -1]]), abi.NF_E_SLOT_ALIAS),
        ("block id outside the pool", abi.HostKvRanges([0], [20], [[1, 10]]), abi.NF_E_BLOCK_RANGE),
        ("table row too short", abi.HostKvRanges([10], [30], [[1, 2]]), abi.NF_E_BLOCK_TABLE_SHORT),
        ("negative length", abi.HostKvRanges([0], [-1], [[1, 2]]), abi.NF_E_ARG),
    ]
    for name, hr, status in cases:
        log_case(f"kv reload rejects: {name}")
        with pytest.raises(abi.NanoflowError) as e:
            abi.nf_kv_reload(ctx, cfg, pool.desc, hr, src.data_ptr(), _stream())
        assert e.value.status == status, name
    torch.cuda.synchronize()
    kg, vg = pool.host_bits()
    assert np.array_equal(kg, kp) and np.array_equal(vg, vp)


@pytest.mark.parametrize("name,l1,l2", [("tiny", 40, 12), ("tiny", 37, 29), ("llama3_8b_layer", 300, 77)])
def test_follow_up_turn_prefill_over_reloaded_prefix(ctx, name, l1, l2):
    from nano_intra_overlap_amd import abi
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_bits, bf16_tensor

    shape = sw.WORKLOADS[name].shape
    cfg = abi.make_cfg(shape)
    w = sw.make_weights(shape, 8, gain_jitter=0.1)
    dw = DeviceWeights(w, "cuda")
    rng = np.random.default_rng(9)
    dec1 = rng.integers(16, 200, 6)
    # turn 1: decodes + the first chunk of a conversation (no prefix)
    b1 = sw.batch_from_lengths(dec1, [l1], [0], seed=21)
    x1 = sw.make_x(shape, b1.n_tokens, 21)
    kp1, vp1 = sw.make_kv_pool(shape, b1.num_blocks, 21)
    pool1 = DevicePool.from_host(kp1, vp1, "cuda")
    x1d = bf16_tensor(x1, "cuda")
    y1 = torch.empty_like(x1d)
    log_case(f"turn 1 {name}: prefill {l1}")
    abi.nf_layer_forward(ctx, cfg, dw.desc, x1d.data_ptr(), y1.data_ptr(), abi.HostBatch.from_batch(b1), pool1.desc,
                         None, _stream())
    r1 = ol.layer_forward(shape, w, x1, b1, kp1, vp1)
    # offload the conversation's l1 tokens
    conv = b1.n_decode
    hr1 = abi.HostKvRanges([0], [l1], b1.block_table[conv:conv + 1])
    rows_d = _pinned_u16((l1, 2, shape.n_kv, shape.head_dim))
    abi.nf_kv_offload(ctx, cfg, pool1.desc, hr1, rows_d.data_ptr(), _stream())
    torch.cuda.synchronize()
    rows_gpu = rows_d.numpy().view(np.uint16).copy()
    rows_ref = kvio.offload(r1["k_pool"], r1["v_pool"], [0], [l1], b1.block_table[conv:conv + 1])
    assert rel_inf(f64(rows_gpu), f64(rows_ref)) <= TOL

    # turn 2: other decodes, the conversation's next chunk with its l1-token prefix, in a
    # fresh pool with other pages; the prefix comes back by reload
    dec2 = rng.integers(16, 200, 5)
    b2 = sw.batch_from_lengths(dec2, [l2], [l1], seed=22)
    x2 = sw.make_x(shape, b2.n_tokens, 22)
    kp2, vp2 = sw.make_kv_pool(shape, b2.num_blocks, 22)
    conv2 = b2.n_decode
    t2 = b2.block_table[conv2:conv2 + 1]
    pool2 = DevicePool.from_host(kp2, vp2, "cuda")
    hr2 = abi.HostKvRanges([0], [l1], t2)
    src = _pinned_u16((l1, 2, shape.n_kv, shape.head_dim))
    src.numpy()[:] = rows_gpu.view(np.int16)
    log_case(f"turn 2 {name}: reload {l1}, prefill {l2} over the prefix")
    abi.nf_kv_reload(ctx, cfg, pool2.desc, hr2, src.data_ptr(), _stream())
    x2d = bf16_tensor(x2, "cuda")
    y2 = torch.full_like(x2d, float("nan"))
    abi.nf_layer_forward(ctx, cfg, dw.desc, x2d.data_ptr(), y2.data_ptr(), abi.HostBatch.from_batch(b2), pool2.desc,
                         None, _stream())
    torch.cuda.synchronize()
    kr2, vr2 = kvio.reload(kp2, vp2, [0], [l1], t2, rows_ref)
    r2 = ol.layer_forward(shape, w, x2, b2, kr2, vr2)
    y = f64(bf16_bits(y2))
    assert np.isfinite(y).all()
    assert rel_inf(y, r2["y"]) <= TOL, rel_inf(y, r2["y"])
    ranges = ol.request_ranges(b2)
    s0, e0 = ranges[conv2][0], ranges[conv2][1]
    assert rel_inf(y[s0:e0], r2["y"][s0:e0]) <= TOL  # the conversation's rows on their own
