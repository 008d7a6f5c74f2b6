"""The benchmark's algorithmic byte counts against the step totals worked out from the model
shapes by hand (27B-class dense: 64 layers, hidden 5120, 40 q / 8 kv heads of 128, SwiGLU 17408,
vocab 151936): every weight read once, every context K/V row read once per layer, the draft
rows' K/V written. No GPU needed."""
import numpy as np

import bench
import synth


def test_block_and_tree_step_bytes():
    shape = synth.DENSE_27B
    # projections per layer: QKV 7168 x 5120, O 5120 x 5120, gate/up 34816 x 5120, down 5120 x 17408
    per_layer_params = 7168 * 5120 + 5120 * 5120 + 34816 * 5120 + 5120 * 17408
    assert per_layer_params == 330_301_440
    weights_gb = (64 * per_layer_params + 151936 * 5120) * 2 / 1e9          # + output head
    assert abs(weights_gb - 43.83) < 0.01
    block = bench.step_bytes(shape, 1, 16, [4096])
    tree = bench.step_bytes(shape, 1, 64, [8192])
    assert abs(block / 1e9 - 44.91) < 0.01          # + 1.07 GB of context K/V at 4096 positions
    assert abs(tree / 1e9 - 46.00) < 0.01           # + 2.15 GB at 8192
    # context K/V: positions x 8 kv heads x 128 x 2 bytes x (K and V) x 64 layers
    assert abs((tree - block) - (8192 - 4096) * 8 * 128 * 2 * 2 * 64
               - 2 * 5120 * (64 - 16) - (64 - 16) * 8 * 128 * 2 * 2 * 64) < 1


def test_gate_up_launch_bytes():
    shape = synth.DENSE_27B
    # the packed [34816][5120] weight, the [16][5120] operand in, the [16][17408] SwiGLU output out
    assert bench.gate_up_bytes(shape, 16) == 2 * 34816 * 5120 + 2 * 16 * 5120 + 2 * 16 * 17408
    assert bench.gate_up_bytes(shape, 16) == 357_236_736


def test_recurrent_bytes_from_the_shapes():
    """Tree pass: per (request, head) the 128 x 128 fp32 state, q, k, v rows of 64 nodes, gates,
    parents and fp32 outputs; commit: the state read and written plus the accepted rows."""
    tree, commit = bench.rec_bytes(32, 64, 32, 128, np.full(32, 5))
    assert tree == 1024 * (65536 + 49152 + 512 + 32768) == 151_519_232
    assert commit == 1024 * 131072 + 32 * 6 * 32 * 512 + 1024 * 256
