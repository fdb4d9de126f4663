"""Streams and graphs: every call enqueues on the stream it is given and
keeps no state between calls (GPU).

  * the whole path on a side stream gives the same bytes as on the default
    stream, also when the stream is only passed as an argument (outputs and
    workspaces the binding allocates belong to that stream, so torch does not
    hand them to other work while the kernels still use them);
  * two codecs on two streams at once give the same bytes as one after the
    other;
  * compress and both receivers captured in a graph and replayed, with new
    inputs copied in between replays and eager work between them, match
    the eager calls on every replay (the kernels clear nothing with memset:
    every output byte is written by a kernel, so the graph holds only
    kernel nodes); the same for the per-shard sender and receiver, and for
    the 16-shard receiver, whose two launches (the second adding to y) sit
    in one graph.
"""
import pytest
import torch

import bit_tensor_activation_amd as B
import workloads as W
from helpers import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
P, T, H, K = 8, 40, 2048, 64
COLS = list(range(3, H, 53))


def draw(seed, T_=T):
    return W.draw(P, T_, H, seed, sigma=0.5, cols=COLS, outlier_factor=60.0, device=DEV)


def full_path(x_calib, x, stream=None):
    """Calibrate, select, compress and decompress, all on `stream`."""
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    for b, xb in enumerate(x_calib):
        B.btq_calib_update(xb, rmin, rmax, 0.9, b == 0, stream=stream)
    sel = B.btq_select_outliers(rmin, rmax, K, stream=stream)
    pk, ol = B.btq_compress_pack(x, K, sel["rscale"], sel["zero_point"], sel["outlier_idx"],
                                 sel["cmap"], stream=stream)
    y = B.btq_decompress_reduce(pk, ol, H, sel["scale"], sel["zero_point"], sel["fmap"],
                                stream=stream)
    return [rmin, rmax, sel["scale"], sel["zero_point"], sel["cmap"], sel["fmap"], pk, ol, y]


def same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_side_stream_matches_default_stream():
    say("case: side stream vs default stream")
    calib = [draw(7000 + b) for b in range(2)]
    x = draw(7100)
    torch.cuda.synchronize()
    ref = full_path(calib, x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)   # default priority
    with torch.cuda.stream(side):
        got = full_path(calib, x, stream=side)
    side.synchronize()
    for a, b in zip(ref, got):
        assert same_bytes(a, b)


def test_stream_argument_alone_orders_the_binding_allocations():
    # The side stream is kept busy, so its calls run late. Their workspaces
    # and outputs are allocated by the binding and (the workspaces) freed
    # when each call returns; the default stream then allocates and fills
    # memory of the same sizes at once. Were the binding's memory tied to the
    # default stream, those fills could land in a workspace or output before
    # the side stream's kernels are done with it.
    say("case: stream passed as an argument only, side stream busy")
    calib = [draw(7000 + b) for b in range(2)]
    x = draw(7100)
    torch.cuda.synchronize()
    ref = full_path(calib, x)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)   # default priority
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)      # a bounded spin: the side stream runs late
    got = full_path(calib, x, stream=side)
    junk = [torch.full((1 << 20,), -7, dtype=torch.int32, device=DEV) for _ in range(64)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for a, b in zip(ref, got):
        assert same_bytes(a, b)


def test_two_streams_at_once_match_one_after_the_other():
    say("case: two codecs on two streams at once")
    inputs = [([draw(7200 + 10 * i + b) for b in range(2)], draw(7300 + i)) for i in range(2)]
    torch.cuda.synchronize()
    seq = [full_path(c, x) for c, x in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]
    outs = []
    for s, (c, x) in zip(streams, inputs):
        with torch.cuda.stream(s):
            outs.append(full_path(c, x, stream=s))
    for s in streams:
        s.synchronize()
    for ref, got in zip(seq, outs):
        for a, b in zip(ref, got):
            assert same_bytes(a, b)


def test_graph_replays_match_eager_calls():
    say("case: graph capture of compress and both receivers, 3 replays")
    calib = [draw(7400 + b) for b in range(2)]
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    for b, xb in enumerate(calib):
        B.btq_calib_update(xb, rmin, rmax, 0.9, b == 0)
    sel = B.btq_select_outliers(rmin, rmax, K)
    pitch = B.btq_packed_pitch(H, K)
    x_static = torch.empty((P, T, H), dtype=torch.int16, device=DEV)
    pk = torch.empty((P, T, pitch), dtype=torch.uint8, device=DEV)
    ol = torch.empty((P, T, K), dtype=torch.int16, device=DEV)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    y16 = torch.empty((T, H), dtype=torch.int16, device=DEV)
    enc = (sel["rscale"], sel["zero_point"], sel["outlier_idx"], sel["cmap"])
    dec = (sel["scale"], sel["zero_point"], sel["fmap"])

    def step(stream=None):
        B.btq_compress_pack_ex(x_static, K, *enc, packed=pk, outliers=ol, stream=stream)
        B.btq_decompress_reduce_ex(pk, ol, H, *dec, y=y, stream=stream)
        B.btq_decompress_reduce_ex(pk, ol, H, *dec, y=y16, bf16=True, stream=stream)

    x_static.copy_(draw(7500))
    step()                      # eager warm-up, on the default stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()                  # calls see the capture stream as the current stream
    for rep in range(3):
        x_new = draw(7600 + rep)
        x_static.copy_(x_new)   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = [pk.clone(), ol.clone(), y.clone(), y16.clone()]
        step()                  # the same inputs, eager
        torch.cuda.synchronize()
        for a, b in zip(got, [pk, ol, y, y16]):
            assert same_bytes(a, b), f"replay {rep}"
        pk.zero_()              # the next replay must write every byte again
        y.zero_()


def test_graph_replays_shard_groups():
    """16 shards: the fp32 receiver runs as two launches (the second adds to
    y), captured in one graph; every replay must equal the eager calls, with
    y cleared in between so the first group has to write it again."""
    say("case: graph capture of the 16-shard receiver (two groups), 3 replays")
    P16 = 16
    draw16 = lambda seed: W.draw(P16, T, H, seed, sigma=0.5, cols=COLS, outlier_factor=60.0,
                                 device=DEV)
    rmin = torch.empty((P16, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    for b in range(2):
        B.btq_calib_update(draw16(7800 + b), rmin, rmax, 0.9, b == 0)
    sel = B.btq_select_outliers(rmin, rmax, K)
    enc = (sel["rscale"], sel["zero_point"], sel["outlier_idx"], sel["cmap"])
    dec = (sel["scale"], sel["zero_point"], sel["fmap"])
    x_static = torch.empty((P16, T, H), dtype=torch.int16, device=DEV)
    pk, ol = B.btq_compress_pack_ex(draw16(7900), K, *enc)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)

    def step():
        B.btq_compress_pack_ex(x_static, K, *enc, packed=pk, outliers=ol)
        B.btq_decompress_reduce_ex(pk, ol, H, *dec, y=y)

    x_static.copy_(draw16(7901))
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        x_static.copy_(draw16(7910 + rep))
        y.fill_(float("nan"))   # the first group must overwrite all of y
        graph.replay()
        torch.cuda.synchronize()
        got = y.clone()
        y.zero_()
        step()
        torch.cuda.synchronize()
        assert same_bytes(got, y), f"replay {rep}"


def test_graph_replays_per_shard_sets():
    say("case: graph capture of the per-shard sender and receiver, 3 replays")
    calib = [draw(7700 + b) for b in range(2)]
    rmin = torch.empty((P, H), dtype=torch.float32, device=DEV)
    rmax = torch.empty_like(rmin)
    for b, xb in enumerate(calib):
        B.btq_calib_update(xb, rmin, rmax, 0.9, b == 0)
    sel = B.btq_select_outliers_per_shard(rmin, rmax, K)
    pitch = B.btq_packed_row_bytes(H, K)
    x_static = torch.empty((P, T, H), dtype=torch.int16, device=DEV)
    pk = torch.empty((P, T, pitch), dtype=torch.uint8, device=DEV)
    ol = torch.empty((P, T, K), dtype=torch.int16, device=DEV)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)

    def step():
        B.btq_compress_pack_per_shard(x_static, K, sel["rscale"], sel["zero_point"],
                                      sel["outlier_idx"], sel["cmap"], packed=pk, outliers=ol)
        B.btq_decompress_reduce_per_shard(pk, ol, H, sel["scale"], sel["zero_point"],
                                          sel["fmap"], y=y)

    x_static.copy_(draw(7800))
    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        x_static.copy_(draw(7900 + rep))
        graph.replay()
        torch.cuda.synchronize()
        got = [pk.clone(), ol.clone(), y.clone()]
        step()
        torch.cuda.synchronize()
        for a, b in zip(got, [pk, ol, y]):
            assert same_bytes(a, b), f"replay {rep}"
        pk.zero_()
        y.zero_()
