"""Layer-stack parity of nf_stack_forward against the CPU oracle, through the C ABI.

* tiny 3-layer stacks (one pool and one weight set per layer) under the null plan, the
  2- and 4-nano-batch plans, with and without cross-layer pipelining and CU masks: the
  output and every layer's pool against the oracle's layers applied one after another;
* y aliasing x;
* the captured-graph flag is refused (replay is switched off; its replay tests are kept,
  skipped, with the reason);
* argument checks, which fail before anything is enqueued;
* every stacked layer held to 1e-2 against the oracle's layer on the GPU's previous output
  (tiny stacks in full; an 8B-shaped 4-layer stack at the full 2048-token batch, pipelined,
  on sampled requests).
"""

import numpy as np
import pytest

from oracle import layer as ol
from synth import workloads as sw
from tests.gpu_util import TOL, deep_tol, f64, log_case, rel_inf, rel_rms

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


def _hb(b):
    from nano_intra_overlap_amd import abi

    return abi.HostBatch.from_batch(b)


def _tiny_stack(seed, n_layers=3):
    from nano_intra_overlap_amd.device import DeviceWeights, bf16_tensor

    wl = sw.WORKLOADS["tiny"]
    b = sw.make_batch("tiny", seed)
    ws = [sw.make_weights(wl.shape, seed, gain_jitter=0.1, layer=l) for l in range(n_layers)]
    x = sw.make_x(wl.shape, b.n_tokens, seed)
    pools = [sw.make_kv_pool(wl.shape, b.num_blocks, seed, layer=l) for l in range(n_layers)]
    kps, vps = [p[0] for p in pools], [p[1] for p in pools]
    ref = ol.stack_forward(wl.shape, ws, x, b, kps, vps)
    ref["exact"] = ol.stack_forward(wl.shape, ws, x, b, kps, vps, storage="exact")
    dws = [DeviceWeights(w, "cuda") for w in ws]
    return wl.shape, b, x, kps, vps, ref, dws, bf16_tensor(x, "cuda")


def _dev_pools(kps, vps):
    from nano_intra_overlap_amd.device import DevicePool

    return [DevicePool.from_host(k, v, "cuda") for k, v in zip(kps, vps)]


def _run(ctx, shape, dws, x_dev, y_dev, b, pools, plan, flags, sync=True):
    from nano_intra_overlap_amd import abi

    abi.nf_stack_forward(ctx, abi.make_cfg(shape), [w.desc for w in dws], x_dev.data_ptr(), y_dev.data_ptr(),
                         _hb(b), [p.desc for p in pools], plan, flags, _stream())
    if sync:
        torch.cuda.synchronize()


def _check(b, kps, vps, ref, pools, y_dev, rows=None, attn=None):
    """The stack's output (rows: the sampled rows of y_dev; ref computed on those) and the
    slots every layer wrote, against the oracle; every other slot bitwise unchanged (only
    when the whole pool is compared). Deep results are held to deep_tol."""
    from nano_intra_overlap_amd.device import bf16_bits

    ex = ref["exact"]
    y = f64(bf16_bits(y_dev))
    assert np.isfinite(y).all()
    if rows is not None:
        y = y[rows]
    err, rms = rel_inf(y, ref["y"]), rel_rms(y, ref["y"])
    tol_inf, tol_rms = deep_tol(ref["y"], ex["y"]), deep_tol(ref["y"], ex["y"], rel_rms)
    print(f"  y: max rel err {err:.3e} (tol {tol_inf:.3e}), rms rel err {rms:.3e} (tol {tol_rms:.3e})", flush=True)
    assert err <= tol_inf and rms <= tol_rms, (err, rms)
    if attn is not None:  # the last layer's attention output
        e = rel_inf(attn, ref["attns"][-1])
        assert e <= deep_tol(ref["attns"][-1], ex["attns"][-1]), e
    if rows is not None:
        return
    new = np.zeros((b.num_blocks, 16), bool)
    for blk, off in ol.new_token_slots(b, 16):
        new[blk, off] = True
    for l, p in enumerate(pools):
        kg, vg = p.host_bits()
        kp, vp = kps[l], vps[l]
        assert np.array_equal(kg.transpose(0, 3, 1, 2, 4)[~new], kp.transpose(0, 3, 1, 2, 4)[~new]), l
        assert np.array_equal(vg.transpose(0, 3, 1, 2)[~new], vp.transpose(0, 3, 1, 2)[~new]), l
        for got, r, e in ((kg.transpose(0, 3, 1, 2, 4)[new], ref["k_pools"][l].transpose(0, 3, 1, 2, 4)[new],
                           ex["k_pools"][l].transpose(0, 3, 1, 2, 4)[new]),
                          (vg.transpose(0, 3, 1, 2)[new], ref["v_pools"][l].transpose(0, 3, 1, 2)[new],
                           ex["v_pools"][l].transpose(0, 3, 1, 2)[new])):
            assert rel_inf(f64(got), f64(r)) <= deep_tol(f64(r), f64(e)), l


def _plans(hb, T):
    from nano_intra_overlap_amd import abi, plans

    yield "null", None
    yield "seq2", plans.sequential(hb, [0, 39, T])
    yield "overlap2", plans.overlap(hb, [0, 39, T])
    yield "overlap2_masked", plans.overlap(hb, [0, 39, T], abi.cu_mask(per_xcd=24, offset=0),
                                           abi.cu_mask(per_xcd=8, offset=24))
    yield "overlap4_pf_compute", plans.overlap(hb, [0, 10, 20, 50, T], prefill_on_memory=False)


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_stack_plans(ctx, seed):
    from nano_intra_overlap_amd import abi

    shape, b, x, kps, vps, ref, dws, x_dev = _tiny_stack(seed)
    for name, plan in _plans(_hb(b), b.n_tokens):
        for flags in (0, abi.NF_STACK_PIPELINE):
            pools = _dev_pools(kps, vps)
            y_dev = torch.full_like(x_dev, float("nan"))
            log_case(f"tiny 3-layer stack seed={seed} plan={name} flags={flags}")
            _run(ctx, shape, dws, x_dev, y_dev, b, pools, plan, flags)
            _check(b, kps, vps, ref, pools, y_dev)


def test_tiny_stack_in_place(ctx):
    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import bf16_tensor

    shape, b, x, kps, vps, ref, dws, _ = _tiny_stack(2)
    for plan in (None, plans.overlap(_hb(b), [0, 39, b.n_tokens])):
        pools = _dev_pools(kps, vps)
        xy = bf16_tensor(x, "cuda")
        log_case("tiny 3-layer stack in place y=x, pipelined")
        _run(ctx, shape, dws, xy, xy, b, pools, plan, abi.NF_STACK_PIPELINE)
        _check(b, kps, vps, ref, pools, xy)


def _layer_outputs(ctx, shape, dws, x_dev, b, pools, plan, flags):
    """Every layer's output of the stack on the GPU: the stack of the first l + 1 layers run
    for each l (earlier layers rewrite the same slots with the same values)."""
    from nano_intra_overlap_amd.device import bf16_bits

    out = []
    for n in range(1, len(dws) + 1):
        y = torch.full_like(x_dev, float("nan"))
        _run(ctx, shape, dws[:n], x_dev, y, b, pools[:n], plan, flags)
        out.append(bf16_bits(y))
    return out


@pytest.mark.parametrize("plan_name", ["null", "overlap2"])
def test_tiny_stack_each_layer_on_its_own_input(ctx, plan_name):
    """Each stacked layer's output, at the 1e-2 bar, against the oracle's layer applied to
    the GPU's output of the layer before (so rounding noise of earlier layers is not
    charged to later ones); every pool's written slots too, and its other slots unchanged."""
    from nano_intra_overlap_amd import abi

    shape, b, x, kps, vps, ref, dws, x_dev = _tiny_stack(5)
    plan = dict(_plans(_hb(b), b.n_tokens))[plan_name]
    pools = _dev_pools(kps, vps)
    log_case(f"tiny 3-layer stack, every layer, plan={plan_name}")
    ys = _layer_outputs(ctx, shape, dws, x_dev, b, pools, plan, abi.NF_STACK_PIPELINE)
    new = np.zeros((b.num_blocks, 16), bool)
    for blk, off in ol.new_token_slots(b, 16):
        new[blk, off] = True
    ws = [sw.make_weights(shape, 5, gain_jitter=0.1, layer=l) for l in range(3)]
    for l in range(3):
        x_l = x if l == 0 else ys[l - 1]
        r = ol.layer_forward(shape, ws[l], x_l, b, kps[l], vps[l])
        e = rel_inf(f64(ys[l]), r["y"])
        kg, vg = pools[l].host_bits()
        ek = rel_inf(f64(kg.transpose(0, 3, 1, 2, 4)[new]), f64(r["k_pool"].transpose(0, 3, 1, 2, 4)[new]))
        ev = rel_inf(f64(vg.transpose(0, 3, 1, 2)[new]), f64(r["v_pool"].transpose(0, 3, 1, 2)[new]))
        print(f"  layer {l}: y {e:.3e}, written K {ek:.3e}, V {ev:.3e}", flush=True)
        assert e <= TOL and ek <= TOL and ev <= TOL, (l, e, ek, ev)
        assert np.array_equal(kg.transpose(0, 3, 1, 2, 4)[~new], kps[l].transpose(0, 3, 1, 2, 4)[~new]), l
        assert np.array_equal(vg.transpose(0, 3, 1, 2)[~new], vps[l].transpose(0, 3, 1, 2)[~new]), l


GRAPH_OFF = ("captured-graph replay is switched off: its first run ended in a host segmentation fault "
             "inside the capture/replay calls, cause not found")


def test_stack_graph_flag_is_refused(ctx):
    from nano_intra_overlap_amd import abi

    shape, b, x, kps, vps, ref, dws, x_dev = _tiny_stack(3, n_layers=2)
    pools = _dev_pools(kps, vps)
    y = torch.full_like(x_dev, float("nan"))
    log_case("tiny stack with the graph flag (refused on the host)")
    with pytest.raises(abi.NanoflowError) as e:
        _run(ctx, shape, dws, x_dev, y, b, pools, None, abi.NF_STACK_GRAPH)
    assert e.value.status == abi.NF_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()


@pytest.mark.skip(reason=GRAPH_OFF)
def test_tiny_stack_graph_replays(ctx):
    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_bits, bf16_tensor

    shape, b, x, kps, vps, ref, dws, x_dev = _tiny_stack(3)
    # eager work run between replays: a different batch through one layer on the same context
    other = sw.make_batch("tiny", 5)
    ow = DeviceWeights(sw.make_weights(shape, 5), "cuda")
    ox = bf16_tensor(sw.make_x(shape, other.n_tokens, 5), "cuda")
    okp, ovp = sw.make_kv_pool(shape, other.num_blocks, 5)
    for name, plan in (("null", None), ("overlap2", plans.overlap(_hb(b), [0, 39, b.n_tokens]))):
        for flags in (0, abi.NF_STACK_PIPELINE):
            pools = _dev_pools(kps, vps)
            y_eager = torch.full_like(x_dev, float("nan"))
            log_case(f"tiny stack eager plan={name} flags={flags}")
            _run(ctx, shape, dws, x_dev, y_eager, b, pools, plan, flags)
            _check(b, kps, vps, ref, pools, y_eager)
            want_y = bf16_bits(y_eager)
            want_pools = [p.host_bits() for p in pools]
            gpools = _dev_pools(kps, vps)
            y = torch.empty_like(x_dev)
            cap0, launch0 = abi.nf_ctx_graph_stats(ctx)
            for rep in range(4):
                y.fill_(float("nan"))
                log_case(f"tiny stack graph plan={name} flags={flags} call {rep}")
                _run(ctx, shape, dws, x_dev, y, b, gpools, plan, flags | abi.NF_STACK_GRAPH)
                assert np.array_equal(bf16_bits(y), want_y), rep
                for got, want in zip((p.host_bits() for p in gpools), want_pools):
                    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), rep
                # the program's own eager work in between
                opool = DevicePool.from_host(okp, ovp, "cuda")
                oy = torch.empty_like(ox)
                abi.nf_layer_forward(ctx, abi.make_cfg(shape), ow.desc, ox.data_ptr(), oy.data_ptr(), _hb(other),
                                     opool.desc, None, _stream())
                torch.cuda.synchronize()
            cap1, launch1 = abi.nf_ctx_graph_stats(ctx)
            assert cap1 - cap0 == 1 and launch1 - launch0 == 4, (cap1 - cap0, launch1 - launch0)
            # another output pointer: captured again, same result
            y2 = torch.full_like(x_dev, float("nan"))
            _run(ctx, shape, dws, x_dev, y2, b, gpools, plan, flags | abi.NF_STACK_GRAPH)
            assert np.array_equal(bf16_bits(y2), want_y)
            assert abi.nf_ctx_graph_stats(ctx)[0] == cap1 + 1


@pytest.mark.skip(reason=GRAPH_OFF)
def test_tiny_stack_graph_follows_batch_changes(ctx):
    """Same pointers, another batch of the same size: the metadata differs, so the stack is
    captured again and matches that batch's oracle."""
    from nano_intra_overlap_amd import abi

    for seed in (6, 7):
        shape, b, x, kps, vps, ref, dws, x_dev = _tiny_stack(seed)
        pools = _dev_pools(kps, vps)
        y = torch.full_like(x_dev, float("nan"))
        log_case(f"tiny stack graph seed={seed}")
        _run(ctx, shape, dws, x_dev, y, b, pools, None, abi.NF_STACK_GRAPH)
        _check(b, kps, vps, ref, pools, y)


def test_stack_rejects_bad_arguments_without_touching_memory(ctx):
    from nano_intra_overlap_amd import abi, plans

    shape, b, x, kps, vps, ref, dws, x_dev = _tiny_stack(4, n_layers=2)
    pools = _dev_pools(kps, vps)
    y = torch.full_like(x_dev, float("nan"))
    cfg = abi.make_cfg(shape)

    def call(weights, pool_list, plan=None, flags=0):
        abi.nf_stack_forward(ctx, cfg, weights, x_dev.data_ptr(), y.data_ptr(), _hb(b), pool_list, plan, flags,
                             _stream())

    masked = plans.overlap(_hb(b), [0, 39, b.n_tokens], abi.cu_mask(per_xcd=24, offset=0),
                           abi.cu_mask(per_xcd=8, offset=24))
    small = _dev_pools([k[:-1] for k in kps[:1]], [v[:-1] for v in vps[:1]])[0]
    cases = [
        ("no layers", lambda: call([], []), abi.NF_E_ARG),
        ("unknown flag", lambda: call([w.desc for w in dws], [p.desc for p in pools], flags=8), abi.NF_E_ARG),
        ("one pool twice", lambda: call([w.desc for w in dws], [pools[0].desc, pools[0].desc]), abi.NF_E_ARG),
        ("unequal pools", lambda: call([w.desc for w in dws], [pools[0].desc, small.desc]), abi.NF_E_ARG),
        ("graph flag", lambda: call([w.desc for w in dws], [p.desc for p in pools], masked,
                                    abi.NF_STACK_GRAPH), abi.NF_E_UNSUPPORTED),
    ]
    for name, fn, status in cases:
        log_case(f"stack argument check: {name}")
        with pytest.raises(abi.NanoflowError) as e:
            fn()
        assert e.value.status == status, name
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()
    for p, k, v in zip(pools, kps, vps):
        kg, vg = p.host_bits()
        assert np.array_equal(kg, k) and np.array_equal(vg, v)


# ------------------------------------------------------------------------------ full size


def test_full_size_stack_each_layer(ctx):
    """LLaMA-3-8B-shaped layers over the full 2048-token batch, 4 layers, pipelined 2-nano
    overlap plan. Each layer, at the 1e-2 bar, against the oracle's layer applied to the
    GPU's output of the layer before, on sampled requests (every prefill token and 48
    decode requests; rows of different requests are independent), with the written K/V of
    every layer; the 4-layer result against the oracle's stack is reported as well."""
    from nano_intra_overlap_amd import abi, plans
    from nano_intra_overlap_amd.device import DevicePool, DeviceWeights, bf16_tensor
    from synth.workloads import make_kv_pool_torch

    name, seed, n_layers = "llama3_8b_layer", 0, 4
    shape = sw.WORKLOADS[name].shape
    b = sw.make_batch(name, seed)
    ws = [sw.make_weights(shape, seed, layer=l) for l in range(n_layers)]
    x = sw.make_x(shape, b.n_tokens, seed)
    dws = [DeviceWeights(w, "cuda") for w in ws]
    pools = [DevicePool.from_int16(*make_kv_pool_torch(shape, b.num_blocks, seed, layer=l, device="cuda"))
             for l in range(n_layers)]
    x_dev = bf16_tensor(x, "cuda")
    plan = plans.overlap(_hb(b), plans.even_bounds(b.n_tokens, 2))
    log_case(f"full-size {n_layers}-layer stack {name} seed={seed} overlap2 pipelined, every layer")
    ys = _layer_outputs(ctx, shape, dws, x_dev, b, pools, plan, abi.NF_STACK_PIPELINE)
    from tests.test_gpu_layer import _attn_buffer

    attn_last = f64(_attn_buffer(ctx, b.n_tokens, shape.n_q * shape.head_dim))

    rng = np.random.default_rng(seed + 7)
    sample = sorted(rng.choice(b.n_decode, size=48, replace=False).tolist()) + list(range(b.n_decode, b.n_requests))
    sub = b.select(sample)
    ranges = ol.request_ranges(b)
    rows = np.concatenate([np.arange(ranges[r][0], ranges[r][1]) for r in sample])
    need = (sub.cached_lens() + sub.q_lens() + 15) // 16
    used = sorted({int(sub.block_table[i, j]) for i in range(sub.n_requests) for j in range(int(need[i]))})
    remap = {blk: i for i, blk in enumerate(used)}
    bt = np.full_like(sub.block_table, -1)
    for i in range(sub.n_requests):
        for j in range(int(need[i])):
            bt[i, j] = remap[int(sub.block_table[i, j])]
    compact = sw.Batch(sub.decode_ctx, sub.prefill_len, sub.prefill_prefix, bt, len(used))
    kps, vps = zip(*[sw.make_kv_pool_blocks(shape, used, seed, layer=l) for l in range(n_layers)])
    idx = torch.as_tensor(used, device="cuda")
    sl = ol.new_token_slots(compact, 16)
    print(f"[{name} x{n_layers}] {len(rows)} sampled rows, each layer on the GPU's previous output:", flush=True)
    for l in range(n_layers):
        x_l = (x if l == 0 else ys[l - 1])[rows]
        r = ol.layer_forward(shape, ws[l], x_l, compact, kps[l], vps[l])
        e = rel_inf(f64(ys[l][rows]), r["y"])
        kg = pools[l].k[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        vg = pools[l].v[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        kgot = np.stack([kg[blk, :, :, off, :] for blk, off in sl])
        kref = np.stack([r["k_pool"][blk, :, :, off, :] for blk, off in sl])
        vgot = np.stack([vg[blk, :, :, off] for blk, off in sl])
        vref = np.stack([r["v_pool"][blk, :, :, off] for blk, off in sl])
        ek, ev = rel_inf(f64(kgot), f64(kref)), rel_inf(f64(vgot), f64(vref))
        ea = rel_inf(attn_last[rows], r["attn"]) if l == n_layers - 1 else 0.0
        print(f"  layer {l}: y {e:.3e}, written K {ek:.3e}, V {ev:.3e}" + (f", attention {ea:.3e}" if ea else ""),
              flush=True)
        assert e <= TOL and ek <= TOL and ev <= TOL and ea <= TOL, (l, e, ek, ev, ea)
    # end to end, for information (bounded by the oracle's own bf16-vs-exact drift)
    ref = ol.stack_forward(shape, ws, x[rows], compact, list(kps), list(vps))
    ref["exact"] = ol.stack_forward(shape, ws, x[rows], compact, list(kps), list(vps), storage="exact")
    y4 = f64(ys[-1][rows])
    print(f"  4 layers end to end: {rel_inf(y4, ref['y']):.3e} against the oracle's stack "
          f"(bound {deep_tol(ref['y'], ref['exact']['y']):.3e})", flush=True)
    assert rel_inf(y4, ref["y"]) <= deep_tol(ref["y"], ref["exact"]["y"])
