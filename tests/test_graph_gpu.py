"""GPU tests of the whole-step decode graph (astr_decode_graph_create / launch / destroy).

A captured multi-layer step is replayed several times, with the program's own
eager work and synchronisations between replays, and every replay is checked
bit for bit against the same decode calls made eagerly, and against the fp64
oracle after the index arrays change to new sequence lengths.
"""
import numpy as np
import pytest
import torch

from paged_gqa_decode_astr_amd import _lib, tensors
from paged_gqa_decode_astr_amd.workloads import build_paged_inputs

from _gpu_helpers import announce, assert_close, oracle_of

pytestmark = pytest.mark.gpu

DEV = "cuda"
NS = 24          # fixed plan: work groups per kv head


def _layer_inputs(B, n_layers, seed, new_tokens=False, row_stride=1500, lens=None):
    rng = np.random.default_rng(seed)
    out = []
    for l in range(n_layers):
        seq = lens if lens is not None else rng.integers(1, row_stride, size=B)
        out.append(build_paged_inputs(seq, 32, 8, 128, 1 << 15, seed=seed * 100 + l, row_stride=row_stride,
                                      new_tokens=1 if new_tokens else None))
    return out


def _device_layers(inps):
    layers = []
    for inp in inps:
        d = tensors.to_device(inp, DEV)
        B, Hq, D = inp["q"].shape
        d["o"] = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        d["lse"] = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        layers.append(d)
    return layers


def _eager(inps, fused, masks=None):
    """Outputs of the same per-layer calls made eagerly (fresh device copies)."""
    res = []
    for l, inp in enumerate(inps):
        d = tensors.to_device(inp, DEV)
        B, Hq, D = inp["q"].shape
        o = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        ws = tensors.decode_workspace(B, Hq, D, DEV, max_splits=NS)
        run = tensors.run_decode_append if fused else tensors.run_decode
        run(d, o=o, lse=lse, workspace=ws, num_splits=NS, mask=None if masks is None else masks[l])
        res.append((o, lse, d))
    torch.cuda.synchronize()
    return res


def _load(layers, inps):
    """Copy new inputs into the captured (fixed-address) buffers."""
    for d, inp in zip(layers, inps):
        for key in ("q", "k_pool", "v_pool", "k_new", "v_new"):
            if key in d:
                d[key].copy_(tensors.bf16_tensor(inp[key], DEV))
        d["req_to_token"].copy_(torch.from_numpy(inp["req_to_token"]))
        d["kv_indptr"].copy_(torch.from_numpy(inp["kv_indptr"]))
        d["o"].fill_(float("nan"))
        d["lse"].fill_(float("nan"))


def _check_against(layers, ref, what):
    for l, (d, (o, lse, dref)) in enumerate(zip(layers, ref)):
        assert torch.equal(d["o"].view(torch.int16), o.view(torch.int16)), f"{what} layer {l}: O differs from eager"
        assert torch.equal(d["lse"].view(torch.int32), lse.view(torch.int32)), f"{what} layer {l}: lse differs"
        if "k_new" in d:
            assert torch.equal(d["k_pool"].view(torch.int16), dref["k_pool"].view(torch.int16)), f"{what} layer {l}"


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_match_eager(fused):
    B, L = 8, 4
    inps = _layer_inputs(B, L, seed=3 + fused, new_tokens=fused)
    layers = _device_layers(inps)
    ws = tensors.decode_workspace(B, 32, 128, DEV, max_splits=NS)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce(f"graph capture fused={fused} B={B} layers={L}")
    g = _lib.DecodeGraph(layers, ws, num_splits=NS, stream=s)
    s.synchronize()
    ref = _eager(inps, fused)
    _check_against(layers, ref, "live run")
    for rep in range(3):
        for d in layers:
            d["o"].fill_(float("nan"))
            d["lse"].fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        announce(f"graph replay {rep} fused={fused}")
        with torch.cuda.stream(s):
            g.launch()
        s.synchronize()
        _check_against(layers, ref, f"replay {rep}")
        del junk
    g.close()


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_graph_with_pages_and_mask(fused, masked):
    """Layers with a page size of 16 (a 2-D table of page ids) and, optionally, a 2-D mask: the
    captured step carries each layer's page size and mask, bit for bit like the eager calls."""
    B, L, P, stride_keys = 5, 2, 16, 1600
    rng = np.random.default_rng(61 + 2 * fused + masked)
    inps = []
    for l in range(L):
        seq = rng.integers(1, stride_keys, size=B)
        inps.append(build_paged_inputs(seq, 32, 8, 128, 1 << 15, seed=6100 + 10 * l + fused, page_size=P,
                                       new_tokens=1 if fused else None))
    masks = None
    if masked:
        masks = []
        for inp in inps:
            m = (rng.random((B, stride_keys)) < 0.6).astype(np.uint8)
            m[:, 0] = 1
            masks.append(torch.from_numpy(m).to(DEV))
    layers = _device_layers(inps)
    for l, d in enumerate(layers):
        assert d["page_size"] == P
        if masked:
            d["mask"] = masks[l]
    ws = tensors.decode_workspace(B, 32, 128, DEV, max_splits=NS)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce(f"graph capture page_size={P} masked={masked} fused={fused}")
    g = _lib.DecodeGraph(layers, ws, num_splits=NS, stream=s)
    s.synchronize()
    ref = _eager(inps, fused, masks)
    _check_against(layers, ref, "live run")
    for rep in range(2):
        for d in layers:
            d["o"].fill_(float("nan"))
            d["lse"].fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"graph replay {rep} page_size={P} masked={masked} fused={fused}")
        with torch.cuda.stream(s):
            g.launch()
        s.synchronize()
        _check_against(layers, ref, f"replay {rep}")
    g.close()


def test_graph_keeps_its_tensors_alive():
    """The graph object holds the captured tensors: dropping the caller's references and allocating
    new memory does not disturb a replay."""
    B, L = 4, 2
    inps = _layer_inputs(B, L, seed=71)
    layers = _device_layers(inps)
    ws = tensors.decode_workspace(B, 32, 128, DEV, max_splits=NS)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce("graph keeps its tensors alive")
    g = _lib.DecodeGraph(layers, ws, num_splits=NS, stream=s)
    s.synchronize()
    o_ptrs = [d["o"].data_ptr() for d in layers]
    del layers, ws
    filler = [torch.full((1 << 20,), 3.0, device=DEV) for _ in range(8)]   # would reuse freed blocks
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.launch()
    s.synchronize()
    kept = g._keep[0]
    assert [d["o"].data_ptr() for d in kept] == o_ptrs
    ref = _eager(inps, False)
    _check_against(kept, ref, "replay after the caller dropped its references")
    assert all(bool((f == 3.0).all()) for f in filler)
    g.close()


def test_graph_replay_after_new_lengths_matches_oracle():
    B, L = 6, 3
    inps = _layer_inputs(B, L, seed=11)
    layers = _device_layers(inps)
    ws = tensors.decode_workspace(B, 32, 128, DEV, max_splits=NS)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce("graph capture for new lengths")
    g = _lib.DecodeGraph(layers, ws, num_splits=NS, stream=s)
    s.synchronize()
    for trial in range(3):
        lens = np.random.default_rng(100 + trial).integers(1, 1500, size=B)
        lens[trial] = 1
        new = _layer_inputs(B, L, seed=20 + trial, lens=lens)
        _load(layers, new)
        torch.cuda.synchronize()
        announce(f"graph replay with new lengths {lens.tolist()}")
        with torch.cuda.stream(s):
            g.launch()
        s.synchronize()
        _check_against(layers, _eager(new, False), f"new lengths {trial}")
        ref_o, ref_lse = oracle_of(new[0])
        assert_close(layers[0]["o"], ref_o, f"new lengths {trial} O")
        assert_close(layers[0]["lse"], ref_lse, f"new lengths {trial} lse", atol=1e-3, rtol=1e-4)
    g.close()


def test_one_graph_per_batch_size():
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = {}
    for B in (1, 4):
        inps = _layer_inputs(B, 2, seed=40 + B)
        layers = _device_layers(inps)
        ws = tensors.decode_workspace(B, 32, 128, DEV, max_splits=NS)
        announce(f"graph capture B={B}")
        graphs[B] = (_lib.DecodeGraph(layers, ws, num_splits=NS, stream=s), layers, inps, ws)
    s.synchronize()
    for rep in range(2):
        for B, (g, layers, inps, _) in graphs.items():
            for d in layers:
                d["o"].fill_(float("nan"))
            torch.cuda.synchronize()
            announce(f"graph B={B} replay {rep}")
            with torch.cuda.stream(s):
                g.launch()
            s.synchronize()
            _check_against(layers, _eager(inps, False), f"B={B} replay {rep}")
    for g, *_ in graphs.values():
        g.close()


def test_graph_create_reports_layer_errors():
    inps = _layer_inputs(2, 2, seed=5)
    layers = _device_layers(inps)
    layers[1]["sm_scale"] = float("nan")             # rejected on the host, before any capture
    ws = tensors.decode_workspace(2, 32, 128, DEV, max_splits=NS)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce("graph create with a bad layer")
    with pytest.raises(_lib.AstrError) as ei:
        _lib.DecodeGraph(layers, ws, num_splits=NS, stream=s)
    assert "layer 1" in ei.value.message and "sm_scale" in ei.value.message
    s.synchronize()
