"""Every entry point of the library captured into one HIP graph: the calls
allocate, synchronise and clear nothing through the runtime (no memset
nodes), so a replay recomputes what the eager calls computed. The graph
chains them the way a layer does (dynamic per-tensor scales produced inside
the graph feed the products that follow), it is replayed three times with
eager library work and synchronisations between the replays, and every
replay's outputs are compared bit for bit with the eager outputs after the
graph's outputs were overwritten.

Inputs: the seeded activation, weight and KV generators; sizes past one
workgroup tile and one reduction block with ragged tails, so that the
multi-kernel paths (the grid-wide absmax and its tail, the tile product,
the split-K reduce) are the ones captured.
"""
import numpy as np
import pytest
import torch

import int8_scaled_gemm_amd as w8
import workloads
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def _paged(lens, bs, hkv, seed):
    """Shuffled placement of each sequence's blocks, -1 past its length."""
    rng = np.random.default_rng(seed)
    nblk = sum(-(-L // bs) for L in lens) + 2
    perm = rng.permutation(nblk)
    tables = np.full((len(lens), max(-(-L // bs) for L in lens)), -1, np.int32)
    used = 0
    for b, L in enumerate(lens):
        for j in range(-(-L // bs)):
            tables[b, j] = perm[used]
            used += 1
    k = workloads.kv_tensor(seed, "k", shape=(nblk * bs, hkv, 128)).to(DEV)
    v = workloads.kv_tensor(seed, "v", shape=(nblk * bs, hkv, 128)).to(DEV)
    return k, v, torch.from_numpy(tables).to(DEV), nblk


def _layer(ins, outs):
    """One pass over every entry point; outs holds preallocated outputs
    (filled in place), ins the inputs. Returns nothing: the results are
    the contents of outs."""
    o = outs
    # symmetric activations: dynamic per-tensor and per-token, fp8 and int8
    w8.w8a8_quant_per_tensor(ins["x"], "fp8", scale=o["xs8"], dynamic=True, q=o["xq8"])
    w8.w8a8_quant_per_tensor(ins["x"], "int8", scale=o["xsi"], dynamic=True, q=o["xqi"])
    w8.w8a8_quant_per_token(ins["x"], "fp8", q=o["tq8"], scales=o["ts8"])
    # tile products reading the scales computed above
    w8.w8a8_scaled_mm(o["xq8"], ins["w8"].t(), o["xs8"], ins["ws8"], torch.bfloat16, out=o["d8"])
    w8.w8a8_scaled_mm(o["xqi"], ins["wi"].t(), o["xsi"], ins["wsi"], torch.float16, out=o["di"])
    w8.w8a8_scaled_mm(o["tq8"], ins["w8"].t(), o["ts8"], ins["ws8"], torch.float32, out=o["dt"])
    # split K: caller workspace, then the static scratch
    w8.w8a8_scaled_mm(ins["sa"], ins["sb"].t(), ins["ssa"], ins["ssb"], torch.bfloat16,
                      out=o["dsk"], workspace=ins["ws"])
    w8.w8a8_scaled_mm(ins["sa"], ins["sb"].t(), ins["ssa"], ins["ssb"], torch.bfloat16,
                      out=o["dst"], workspace="static")
    # asymmetric int8: per-token and per-tensor, then the zero-point product
    w8.w8a8_quant_per_token_azp(ins["x"], q=o["aq"], scales=o["as"], azp=o["az"])
    w8.w8a8_quant_per_tensor_azp(ins["x"], scale=o["ats"], azp=o["atz"], dynamic=True, q=o["atq"])
    w8.w8a8_colsum(ins["wi"], out=o["cs"])
    w8.w8a8_scaled_mm_azp(o["aq"], ins["wi"].t(), o["as"], o["az"], o["cs"], ins["wsi"],
                          torch.bfloat16, out=o["da"])
    w8.w8a8_scaled_mm_azp(o["atq"], ins["wi"].t(), o["ats"], o["atz"], o["cs"], ins["wsi"],
                          torch.bfloat16, out=o["dat"])
    # merged layers
    w8.w8a8_expand_shard_scales(ins["shs"], ins["rows"], out=o["ex"])
    w8.w8a8_requant_shared_scale(ins["w8"], ins["rows"], ins["shs"], out=o["rq"],
                                 shared_scale=o["rqs"])
    # scaled fp8 KV cache: dynamic quant of a tensor past one block, dequant
    w8.kv_fp8_scaled_quant(ins["kv"], scale=o["kvs"], dynamic=True, q=o["kvq"])
    w8.kv_fp8_scaled_dequant(o["kvq"], o["kvs"], torch.bfloat16, out=o["kvd"])
    # the attention consumer over caches quantised inside the graph
    w8.kv_fp8_scaled_quant(ins["pk"], scale=o["pks"], dynamic=True, q=o["pkq"])
    w8.kv_fp8_scaled_quant(ins["pv"], scale=o["pvs"], dynamic=True, q=o["pvq"])
    w8.kv_fp8_decode_attention(ins["aq_"], o["pkq"].view(-1, 2, 128), o["pvq"].view(-1, 2, 128),
                               ins["starts"], ins["max_len"], o["pks"], o["pvs"],
                               out=o["att"], workspace=ins["aws"])
    w8.kv_fp8_paged_decode_attention(ins["aq_"], o["pkq"], o["pvq"], ins["tables"], ins["lens"],
                                     ins["max_len"], o["pks"], o["pvs"], out=o["patt"],
                                     workspace=ins["aws"])


def _inputs():
    M, N, K = 300, 520, 1040
    x = workloads.activations(M, K, seed=71).to(DEV)
    w = workloads.weights(N, K, seed=72).to(DEV)
    w8_, ws8 = w8.w8a8_quant_per_token(w, "fp8")
    wi, wsi = w8.w8a8_quant_per_token(w, "int8")
    # a split-K decode problem: few rows, long K
    sM, sN, sK = 40, 1000, 8192 + 16
    sx = workloads.activations(sM, sK, seed=73).to(DEV)
    sw = workloads.weights(sN, sK, seed=74).to(DEV)
    sa, ssa = w8.w8a8_quant_per_token(sx, "int8")
    sb, ssb = w8.w8a8_quant_per_token(sw, "int8")
    need = w8.w8a8_scaled_mm_workspace_size(sM, sN, sK)
    assert need > 0, "the decode problem no longer splits K"
    rows = [300, 0, 113, 107]  # shards of the 520 weight rows
    shs = torch.tensor([2e-3, 7e-4, 1.5e-3, 3e-3], dtype=torch.float32, device=DEV)
    lens = [700, 33, 1]
    bs, hkv, hq = 16, 2, 8
    pk, pv, tables, nblk = _paged(lens, bs, hkv, seed=75)
    # the contiguous kernel reads the same cache as rows 0.. of a flat
    # [nblk*bs, hkv, 128] tensor: sequence b starts where its first block is
    starts = torch.tensor([0, 700, 733, 734], dtype=torch.int32, device=DEV)
    max_len = max(lens)
    aws = torch.empty(max(w8.kv_fp8_attention_workspace_size(len(lens), hq, hkv, max_len), 16),
                      dtype=torch.uint8, device=DEV)
    return dict(
        x=x, w8=w8_, ws8=ws8, wi=wi, wsi=wsi, sa=sa, ssa=ssa, sb=sb, ssb=ssb,
        ws=torch.empty(need, dtype=torch.uint8, device=DEV), rows=rows, shs=shs,
        kv=workloads.kv_tensor(76, "k", shape=(1024 + 3, 8, 128)).to(DEV),
        pk=pk.view(nblk, bs, hkv, 128), pv=pv.view(nblk, bs, hkv, 128),
        aq_=workloads.attention_queries(len(lens), hq, 128, seed=77).to(DEV),
        tables=tables, lens=torch.tensor(lens, dtype=torch.int32, device=DEV),
        starts=starts, max_len=max_len, aws=aws)


def _outputs(ins):
    M, K = ins["x"].shape
    N = ins["w8"].shape[0]
    sM, sN = ins["sa"].shape[0], ins["sb"].shape[0]
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=DEV)
    f32, i32, i8, e4 = torch.float32, torch.int32, torch.int8, torch.float8_e4m3fn
    B, hq, _ = ins["aq_"].shape
    return {
        "xq8": e((M, K), e4), "xs8": e(1, f32), "xqi": e((M, K), i8), "xsi": e(1, f32),
        "tq8": e((M, K), e4), "ts8": e(M, f32),
        "d8": e((M, N), torch.bfloat16), "di": e((M, N), torch.float16), "dt": e((M, N), f32),
        "dsk": e((sM, sN), torch.bfloat16), "dst": e((sM, sN), torch.bfloat16),
        "aq": e((M, K), i8), "as": e(M, f32), "az": e(M, i32),
        "atq": e((M, K), i8), "ats": e(1, f32), "atz": e(1, i32), "cs": e(N, i32),
        "da": e((M, N), torch.bfloat16), "dat": e((M, N), torch.bfloat16),
        "ex": e(N, f32), "rq": e((N, K), e4), "rqs": e(1, f32),
        "kvq": e(ins["kv"].shape, e4), "kvs": e(1, f32),
        "kvd": e(ins["kv"].shape, torch.bfloat16),
        "pkq": e(ins["pk"].shape, e4), "pks": e(1, f32),
        "pvq": e(ins["pv"].shape, e4), "pvs": e(1, f32),
        "att": e((B, hq, 128), torch.bfloat16), "patt": e((B, hq, 128), torch.bfloat16)}


def _raw(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(
        {2: torch.int16, 4: torch.int32}[t.element_size()])


def test_every_entry_point_replays_in_one_graph():
    print("graph: every entry point, one capture, three replays", flush=True)
    ins = _inputs()
    eager = _outputs(ins)
    _layer(ins, eager)
    torch.cuda.synchronize()
    # the split-K products agree with each other before any graph exists
    assert torch.equal(_raw(eager["dsk"]), _raw(eager["dst"]))
    outs = _outputs(ins)
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            _layer(ins, outs)
    torch.cuda.synchronize()
    for i in range(3):
        for t in outs.values():
            _raw(t).fill_(0x55 if t.element_size() == 1 else 0x5555)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(_raw(t), _raw(eager[name])), (i, name)
        # eager library work between the replays, on the same static scratch
        # and the same kind of buffers the graph uses
        w8.w8a8_scaled_mm(ins["sa"][:17], ins["sb"][:300].t(), ins["ssa"][:17], ins["ssb"][:300],
                          torch.bfloat16, workspace="static")
        w8.kv_fp8_scaled_quant(ins["kv"][:700])
        torch.cuda.synchronize()
