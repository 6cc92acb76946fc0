"""The decode step (dsa_decode_prolog, dsa_indexer_topk, dsa_sparse_attn)
captured once in a HIP graph and replayed: every replay returns the eager
step's bits.  Between replays the outputs are cleared by eager work and the
device is synchronised, so each replay has to recompute them."""
import pytest
import torch

import numpy as np

from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import DeviceState, bf16_tensor, check_topk_row, say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager(need_gpu):
    say("[graph] decode_8k_needles: prolog + indexer + sparse attention")
    inp = synth.make("decode_8k_needles")
    st = DeviceState(inp)
    dev = st.dev
    R, K = st.R, st.topk
    new_tok = inp["seq_starts"] + inp["seq_lens"] - 1
    k_new = bf16_tensor(inp["k_idx"][new_tok], dev)
    kv_new = bf16_tensor(inp["kv"][new_tok], dev)
    slots = torch.from_numpy(inp["slot_mapping"][new_tok]).to(dev)
    q_bf = bf16_tensor(inp["q_idx"], dev)
    q_fp8 = torch.empty_like(st.q_fp8)
    q_e8 = torch.empty_like(st.q_e8m0)
    out_idx = torch.empty((R, K), dtype=torch.int32, device=dev)
    out_sc = torch.empty((R, K), dtype=torch.float32, device=dev)
    out = torch.empty((R, st.H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((R, st.H), dtype=torch.float32, device=dev)
    ws_i = ops.indexer_workspace(R, st.block_table.shape[1], st.H_I, K, dev)
    ws_s = ops.sparse_attn_workspace(R, st.H, K, dev)
    outs = (out_idx, out_sc, out, lse)

    def step():
        ops.decode_prolog(q_bf, k_new, kv_new, slots, st.k_pool, st.kv_pool, q_out=(q_fp8, q_e8))
        ops.dsa_indexer_topk(q_fp8, q_e8, st.w, st.k_pool, st.block_table, st.row_seq, st.row_pos, K,
                             out_idx=out_idx, out_score=out_sc, workspace=ws_i)
        ops.dsa_sparse_attn(st.q_sfa, st.kv_pool, st.block_table, st.row_seq, out_idx,
                            out=out, lse=lse, workspace=ws_s)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert int((ref[0] >= 0).sum()) == R * K

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()   # once on the capture stream before capture
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "score", "out", "lse"), outs, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        say(f"[graph] replay {rep} equal to eager")
    # the last replay's results against the oracle: the Top-K rule, and the
    # attention over the replay's own indices
    o = Oracle(inp)
    gi, gs = outs[0].cpu().numpy(), outs[1].cpu().numpy()
    for r in range(R):
        ora = o.topk(r)
        check_topk_row(gi[r], gs[r], ora, K, int(inp["row_pos"][r]))
        ref_o, ref_l = o.sfa(r, gi[r])
        got = outs[2][r].cpu().numpy()
        err = float(np.abs(got - ref_o).max())
        bar = 1e-3 * float(np.abs(ref_o).max())
        assert err <= bar, f"row {r}: SFA error {err:.3g} above {bar:.3g}"
        assert np.all(np.abs(outs[3][r].cpu().numpy() - ref_l) <= 1e-3)
    say("[graph] replay results pass the oracle checks")
    # eager again after the replays: the same bits
    step()
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)


def test_graph_of_two_fused_decode_steps(need_gpu):
    """dsa_decode_indexer_topk + dsa_sparse_attn twice in one graph (two
    layers' decode steps over the same inputs, each with its own outputs and
    workspaces, as a model captures several layers in one graph): every
    replay returns the eager bits for both."""
    say("[graph] decode_ragged_b32: two fused decode steps in one graph")
    inp = synth.make("decode_ragged_b32")
    st = DeviceState(inp)
    dev = st.dev
    R, K = st.R, st.topk
    new_tok = inp["seq_starts"] + inp["seq_lens"] - 1
    k_new = bf16_tensor(inp["k_idx"][new_tok], dev)
    kv_new = bf16_tensor(inp["kv"][new_tok], dev)
    slots = torch.from_numpy(inp["slot_mapping"][new_tok]).to(dev)
    q_bf = bf16_tensor(inp["q_idx"], dev)

    def buffers():
        return dict(idx=torch.empty((R, K), dtype=torch.int32, device=dev),
                    score=torch.empty((R, K), dtype=torch.float32, device=dev),
                    out=torch.empty((R, st.H, 512), dtype=torch.float32, device=dev),
                    lse=torch.empty((R, st.H), dtype=torch.float32, device=dev),
                    ws_i=ops.indexer_workspace(R, st.block_table.shape[1], st.H_I, K, dev),
                    ws_s=ops.sparse_attn_workspace(R, st.H, K, dev))

    layers = [buffers(), buffers()]
    names = ("idx", "score", "out", "lse")

    def step(b):
        ops.dsa_decode_indexer_topk(q_bf, st.w, k_new, kv_new, slots, st.k_pool, st.kv_pool,
                                    st.block_table, st.row_seq, st.row_pos, K, out_idx=b["idx"],
                                    out_score=b["score"], workspace=b["ws_i"])
        ops.dsa_sparse_attn(st.q_sfa, st.kv_pool, st.block_table, st.row_seq, b["idx"],
                            out=b["out"], lse=b["lse"], workspace=b["ws_s"])

    for b in layers:
        step(b)
    torch.cuda.synchronize()
    ref = [[b[n].clone() for n in names] for b in layers]
    assert all(torch.equal(x, y) for x, y in zip(ref[0], ref[1]))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for b in layers:
            step(b)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for b in layers:
            step(b)
    torch.cuda.synchronize()
    for rep in range(3):
        for b in layers:
            for n in names:
                b[n].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, b in enumerate(layers):
            for n, r in zip(names, ref[li]):
                assert torch.equal(b[n], r), f"replay {rep}, layer {li}: {n} differs from eager"
        say(f"[graph] replay {rep}: both layers equal to eager")
    # the replay's indices pass the Top-K rule against the oracle on a few rows
    o = Oracle(inp)
    gi, gs = layers[1]["idx"].cpu().numpy(), layers[1]["score"].cpu().numpy()
    for r in (0, R // 2, R - 1):
        check_topk_row(gi[r], gs[r], o.topk(r), K, int(inp["row_pos"][r]))
    say("[graph] replay indices pass the oracle checks")


def test_graph_multi_query_step(need_gpu):
    """The multi-query decode step (dsa_decode_prolog for four query tokens
    per sequence, dsa_indexer_topk_mq, dsa_sparse_attn with split partials
    and the combine launch) captured in one graph: every replay returns the
    eager bits, and the last replay passes the Top-K rule and the attention
    bar against the oracle on every row."""
    say("[graph] multi-query step: prolog + multi-query indexer + sparse attention")
    cfg = synth.Config(97, "mq_graph", batch=3, h_index=64, h_attn=32, topk=512,
                       ragged=(2000, 6000), q_per_seq=4)
    inp = synth.make(cfg)
    st = DeviceState(inp)
    dev = st.dev
    R, K = st.R, st.topk
    new_tok = inp["seq_starts"][inp["row_seq"]].astype(np.int64) + inp["row_pos"].astype(np.int64)
    k_new = bf16_tensor(inp["k_idx"][new_tok], dev)
    kv_new = bf16_tensor(inp["kv"][new_tok], dev)
    slots = torch.from_numpy(inp["slot_mapping"][new_tok].astype(np.int64)).to(dev)
    q_bf = bf16_tensor(inp["q_idx"], dev)
    q_fp8 = torch.empty_like(st.q_fp8)
    q_e8 = torch.empty_like(st.q_e8m0)
    outs = (torch.empty((R, K), dtype=torch.int32, device=dev),
            torch.empty((R, K), dtype=torch.float32, device=dev),
            torch.empty((R, st.H, 512), dtype=torch.float32, device=dev),
            torch.empty((R, st.H), dtype=torch.float32, device=dev))
    ws_i = ops.indexer_workspace(R, st.block_table.shape[1], st.H_I, K, dev)
    ws_s = ops.sparse_attn_workspace(R, st.H, K, dev)

    def step():
        ops.decode_prolog(q_bf, k_new, kv_new, slots, st.k_pool, st.kv_pool, q_out=(q_fp8, q_e8))
        ops.dsa_indexer_topk_mq(q_fp8, q_e8, st.w, st.k_pool, st.block_table, st.row_seq,
                                st.row_pos, cfg.q_per_seq, K, out_idx=outs[0], out_score=outs[1],
                                workspace=ws_i)
        ops.dsa_sparse_attn(st.q_sfa, st.kv_pool, st.block_table, st.row_seq, outs[0],
                            out=outs[2], lse=outs[3], workspace=ws_s)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "score", "out", "lse"), outs, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        say(f"[graph] multi-query replay {rep} equal to eager")
    o = Oracle(inp)
    gi, gs = outs[0].cpu().numpy(), outs[1].cpu().numpy()
    for r in range(R):
        check_topk_row(gi[r], gs[r], o.topk(r), K, int(inp["row_pos"][r]))
        ref_o, ref_l = o.sfa(r, gi[r])
        got = outs[2][r].cpu().numpy()
        err = float(np.abs(got - ref_o).max())
        bar = 1e-3 * float(np.abs(ref_o).max())
        assert err <= bar, f"row {r}: SFA error {err:.3g} above {bar:.3g}"
        assert np.all(np.abs(outs[3][r].cpu().numpy() - ref_l) <= 1e-3)
    say("[graph] multi-query replay results pass the oracle checks")
