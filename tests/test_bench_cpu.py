"""Host-side checks of bench.py's accounting (no GPU): the algorithmic bytes
that every reported GB/s and roofline fraction divides by, counted here
element by element from the tensors each kernel reads and writes."""
import bench

MB = 1e6


def tensor_bytes(*shapes_and_sizes):
    total = 0
    for shape, esize in shapes_and_sizes:
        n = 1
        for d in shape:
            n *= d
        total += n * esize
    return total


def test_linear_step_bytes():
    M, K, N = 4096, 7168, 7168
    ab = bench.algorithmic_bytes(M, K, N)
    # X bf16 in; codes [M][K] and fp32 scales [K/128][M] out
    assert ab["quantize_1x128_x"] == tensor_bytes(((M, K), 2), ((M, K), 1), ((K // 128, M), 4))
    # W bf16 in; both code layouts and one scale per 128x128 tile out
    assert ab["quantize_128x128_w"] == tensor_bytes(((K, N), 2), ((K, N), 1), ((N, K), 1),
                                                    ((K // 128, N // 128), 4))
    # dY bf16 in; 1x128 codes/scales and 128x1 transposed codes/scales out
    assert ab["quantize_dual_dy"] == tensor_bytes(((M, N), 2), ((M, N), 1), ((N // 128, M), 4),
                                                  ((N, M), 1), ((M // 128, N), 4))
    # codes and 1x128 scales in; transposed codes and 128x1 scales out
    assert ab["requant_128x1_x"] == tensor_bytes(((M, K), 1), ((K // 128, M), 4),
                                                 ((K, M), 1), ((M // 128, K), 4))
    # the figures the workload table quotes, to 0.1 MB
    assert round(ab["quantize_1x128_x"] / MB, 1) == 89.0
    assert round((ab["quantize_128x128_w"] - N * K) / MB, 1) == 154.2
    assert round(ab["requant_128x1_x"] / MB, 1) == 60.6


def test_linear_step_bytes_ragged_rows():
    # rows not a multiple of 128: the 128x1 layouts are padded to whole 128-row blocks
    M, K, N = 200, 256, 384
    ab = bench.algorithmic_bytes(M, K, N)
    Mp = 256
    assert ab["quantize_128x1_dy"] == tensor_bytes(((M, N), 2), ((N, Mp), 1), ((Mp // 128, N), 4))


def test_quant_stress_bytes():
    R, C = 16384, 7168
    ab = bench.quant_stress_bytes(R, C)
    one = tensor_bytes(((R, C), 2), ((R, C), 1), ((C // 128, R), 4))
    col = tensor_bytes(((R, C), 2), ((C, R), 1), ((R // 128, C), 4))
    assert ab["quantize_1x128"] == one
    assert ab["quantize_128x1"] == col
    assert ab["quantize_dual"] == one + col - R * C * 2          # one read of X
    assert ab["quantize_128x128"] == tensor_bytes(((R, C), 2), ((R, C), 1), ((C, R), 1),
                                                  ((R // 128, C // 128), 4))
    assert ab["requant_128x1"] == tensor_bytes(((R, C), 1), ((C // 128, R), 4), ((C, R), 1),
                                               ((R // 128, C), 4))
    assert round(ab["quantize_1x128"] / MB, 1) == 356.0


def test_tile_sample_covers_edges_and_fraction():
    import numpy as np
    g = np.random.default_rng(0)
    for n, frac in [(8192, 0.5), (18432, 0.25), (7168, 0.25), (300, 0.5), (128, 0.25), (1, 0.5)]:
        idx, k, nt = bench.tile_sample(n, frac, g)
        assert nt == -(-n // 128)
        assert k == max(1, int(round(frac * nt)))
        tiles = np.unique(idx // 128)
        assert tiles.size == k and tiles[0] == 0 and (k < 2 or tiles[-1] == nt - 1)
        # whole tiles, clipped at n, no duplicates
        assert np.all(np.diff(idx) > 0) and idx[-1] < n
        for t in tiles:
            assert np.sum(idx // 128 == t) == min(128, n - 128 * t)


def test_emit_writes_the_printed_line(tmp_path, capsys):
    """bench.emit prints the JSON line and keeps the same line as
    <workload>[_ue8m0][_sr].json under --results (nothing when it is empty)."""
    import argparse, json
    out = {"metric": "m", "value": 1.5}
    for recipe, rounding, name in (("fp32", "rn", "ffn_dense"), ("ue8m0", "rn", "ffn_dense_ue8m0"),
                                   ("fp32", "sr", "ffn_dense_sr")):
        args = argparse.Namespace(workload="ffn_dense", recipe=recipe, rounding=rounding, results=str(tmp_path))
        bench.emit(args, out)
        printed = capsys.readouterr().out.strip()
        assert json.loads(printed) == out
        assert (tmp_path / f"{name}.json").read_text().strip() == printed
    args = argparse.Namespace(workload="quant_stress", recipe="fp32", rounding="rn", results="")
    bench.emit(args, out)
    assert json.loads(capsys.readouterr().out) == out
    assert not (tmp_path / "quant_stress.json").exists()
