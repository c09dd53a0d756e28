"""GPU parity at the Beam block shape (hidden 5120, intermediate 2560, 256
experts in 8 groups of 32, keep 4, top-8, x2.5) in the launch configuration
the benchmark times (automatic schedule):

  * decode batch T=64, prefill chunk T=8192, skewed-load T=16384 (Zipf logit
    offsets): routing of every token against the oracle (ids as sets, counts
    after margin exclusion, weights), outputs on sampled tokens that the
    oracle computes one by one (the block is per-token) -- every token of the
    decode batch, 32 / 24 / 8 evenly spread ones of the others; on the skewed batch
    the sample also holds one token of every token tile of the most loaded
    expert (the blocked tile order of experts with 8 or more token tiles);
  * four stacked sandwich-normed sublayers at T=4096 with independent
    weights, checked per layer with the device's own layer input (teacher
    forcing), since GPU and oracle layer inputs differ by bf16 rounding that
    would legitimately re-route tokens after the first layer.
"""
import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from moe_inputs import bf16_bits

from parity import (check_output, check_routing, expert_fetcher, keep_mask, oracle_block_rows,
                    oracle_route, sample_tokens, sync)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
N_SAMPLE = 8


@pytest.fixture(scope="module")
def bm():
    import sparse_moe_transformer_group_amd as bm
    bm.set_schedule("auto")
    yield bm
    bm.release_workspaces()


@pytest.fixture(scope="module")
def beam_weights(bm):
    s = MI.WORKLOADS["prefill"]
    print("[setup] Beam-shape weights layer 0", flush=True)
    wr = MI.make_router(s.E, s.H).to(DEV)
    wg, wu, wd = MI.make_expert_weights(s.E, s.H, s.I, DEV)
    packed = bm.pack_experts(wg, wu, wd)
    sync()
    yield wr, wg, wu, wd, packed
    del wg, wu, wd, packed
    torch.cuda.empty_cache()


TILE_TOKENS = 320   # token rows per tile of the prefill-size expert GEMMs


def hottest_expert_tile_tokens(ids, keep):
    """One token from every token tile of the most loaded expert.  Its tokens
    (ascending, as the permutation orders them) are split evenly over
    ceil(n / 320) tiles; tile j takes positions [j n / mt, (j + 1) n / mt).
    The sampled position moves inside each tile so that different rows of
    the tile (and of its 32-token blocks) are checked; excluded tokens are
    skipped."""
    counts = np.bincount(ids.reshape(-1), minlength=256)
    e = int(np.argmax(counts))
    toks = np.nonzero((ids == e).any(axis=1))[0]
    n = toks.size
    mt = -(-n // TILE_TOKENS)
    out = []
    for j in range(mt):
        lo, hi = j * n // mt, (j + 1) * n // mt
        for d in range(hi - lo):
            p = lo + (37 * j + d) % (hi - lo)
            if keep[toks[p]]:
                out.append(int(toks[p]))
                break
    return e, mt, np.array(out, dtype=np.int64)


# outputs checked per workload: every token of the decode batch (element by
# element at the headline shape), evenly spread samples elsewhere
N_SAMPLE_OF = {"decode": 64, "verify": 32, "prefill": 24, "skewed": N_SAMPLE}


def beam_case(bm, beam_weights, name, hot_tiles=False):
    shape = MI.WORKLOADS[name]
    print(f"[case] {name} T={shape.T}", flush=True)
    wr, wg, wu, wd, packed = beam_weights
    x = MI.make_x(shape.T, shape.H).to(DEV)
    off = MI.load_zipf_offsets(shape.E).to(DEV) if shape.offset == "zipf" else None
    y, ids, w, counts = bm.block(x, wr, *packed, shape.groups, shape.topk_groups, shape.k,
                                 shape.scale, logit_offset=off)
    sync()
    ref_r = oracle_route(x, wr, shape, off)
    st = check_routing(ids, w, ref_r, shape, counts)
    keep = keep_mask(ref_r)
    toks = sample_tokens(keep, N_SAMPLE_OF[name])
    if hot_tiles:
        e_hot, mt_hot, hot = hottest_expert_tile_tokens(ids.cpu().numpy(), keep)
        assert hot.size == mt_hot >= 8
        st.update(hottest_expert=e_hot, hottest_expert_tiles=mt_hot)
        toks = np.unique(np.concatenate([toks, hot]))
    ref = oracle_block_rows(x, toks, wr, wg, wu, wd, shape, off)
    assert np.array_equal(np.sort(ref["ids"], 1), np.sort(ref_r["ids"][toks], 1))
    st.update(check_output(y[torch.from_numpy(toks).to(DEV)], ref["y"]))
    st["sampled_tokens"] = toks.tolist()
    print({k: v for k, v in st.items() if k not in ("excluded_tokens", "sampled_tokens")},
          flush=True)
    return counts.cpu().numpy()


def test_beam_decode_T64(bm, beam_weights):
    beam_case(bm, beam_weights, "decode")


def test_beam_verify_T256(bm, beam_weights):
    beam_case(bm, beam_weights, "verify")


def test_beam_prefill_T8192(bm, beam_weights):
    beam_case(bm, beam_weights, "prefill")


def test_beam_skewed_T16384(bm, beam_weights):
    counts = beam_case(bm, beam_weights, "skewed", hot_tiles=True)
    # the offsets make the load strongly skewed (Zipf-like)
    assert counts.max() > 20 * counts.mean()
    assert counts.sum() == 16384 * 8


def test_beam_stack_T4096_four_sublayers(bm, beam_weights):
    shape = MI.WORKLOADS["stack"]
    x = MI.make_x(shape.T, shape.H, case=5).to(DEV)
    stream = bm.stream_init(x)
    for layer in range(shape.layers):
        step = layer + 2
        print(f"[case] stack layer {layer} step {step}", flush=True)
        if layer == 0:
            wr, wg, wu, wd, packed = beam_weights
        else:
            wr = MI.make_router(shape.E, shape.H, layer=layer).to(DEV)
            wg, wu, wd = MI.make_expert_weights(shape.E, shape.H, shape.I, DEV, layer=layer)
            packed = bm.pack_experts(wg, wu, wd)
        prev = stream.clone()
        xin, yb, ids, w, counts = bm.sublayer(stream, step, wr, *packed)
        sync()
        prev64 = prev.cpu().numpy().astype(np.float64)
        got_in = O.bf16_bits_to_f64(bf16_bits(xin))
        ref_in = O.rmsnorm(prev64)
        assert np.all(np.abs(got_in - ref_in) <= np.abs(ref_in) * 2.0 ** -7 + 1e-30)
        ref_r = oracle_route(xin, wr, shape)          # teacher-forced layer input
        st = check_routing(ids, w, ref_r, shape, counts)
        toks = sample_tokens(keep_mask(ref_r), 12)
        ref = O.moe_block(bf16_bits(xin)[toks], bf16_bits(wr), expert_fetcher(wg, wu, wd),
                          shape.groups, shape.topk_groups, shape.k, shape.scale)
        st.update(check_output(yb[torch.from_numpy(toks).to(DEV)], ref["y"]))
        ref_stream = O.residual_step(prev64, O.rmsnorm(O.bf16_bits_to_f64(bf16_bits(yb))), step)
        np.testing.assert_allclose(stream.cpu().numpy(), ref_stream, rtol=1e-5, atol=1e-5)
        print({k: v for k, v in st.items() if k != "excluded_tokens"}, flush=True)
        if layer > 0:
            del wg, wu, wd, packed
            torch.cuda.empty_cache()
