"""Small layer shapes used by the CPU pins and the GPU parity tests.

Each is a variant of the benchmark layers that the oracle (and, for the
smallest, the pure-Python brute force) finishes in seconds."""
from synth import LAYERS, LayerConfig

C0 = LAYERS["tiny_w4a16"]

MINIS = {
    # brute-force sized
    "c0": C0,
    "c0_a8": C0.replace(name="tiny_w4a8", act="a8"),
    "e288": LayerConfig("tiny_e288", 100, T=4, H=64, E=288, k=4, I=32, group=32),
    "k1": LayerConfig("tiny_k1", 101, T=6, H=64, E=5, k=1, I=64, group=32),
    "e1": LayerConfig("tiny_e1", 102, T=5, H=64, E=1, k=1, I=64, group=64),
    "mixed_shared": LayerConfig("tiny_mixed_shared", 103, T=7, H=128, E=6, k=3,
                                I=64, group=32, n_int2=2, group_int2=64,
                                n_shared=1, I_shared=96),
    "mixed_shared_a8": LayerConfig("tiny_mixed_shared_a8", 104, T=5, H=128, E=6,
                                   k=2, I=64, group=64, n_int2=2, group_int2=32,
                                   n_shared=1, I_shared=64, act="a8"),
    "kE": LayerConfig("tiny_kE", 105, T=3, H=64, E=4, k=4, I=32, group=32),
    "norenorm": LayerConfig("tiny_norenorm", 106, T=4, H=64, E=6, k=2, I=32,
                            group=32, renormalize=0),
    # sigmoid-gated shared experts
    "gated_shared": LayerConfig("tiny_gated_shared", 107, T=6, H=128, E=5, k=2, I=64,
                                group=32, n_int2=1, group_int2=64, n_shared=2,
                                I_shared=96, shared_gate=True),
    "gated_shared_a8": LayerConfig("tiny_gated_shared_a8", 108, T=5, H=128, E=4, k=2,
                                   I=64, group=64, n_shared=1, I_shared=64,
                                   shared_gate=True, act="a8"),
}
