"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no Q4 arithmetic: it only draws float32 weights, float32 activations and
token ids with numpy's PCG64, in row-major order.  Shapes follow the model the
pages describe (section *Architecture* of "Implémentation en Rust du modèle
Voxtral Mini 4B Realtime de Mistral pour l'exécuter dans le navigateur"):
decoder width 3072 with GQA 32Q/8KV (head_dim 128), encoder width 1280, a
131072-row vocabulary (the 1.5 GiB float32 embedding table of section
*Solutions techniques*, item 3, is 131072 x 3072 x 4 bytes), and the 38-token
decoder prefix of section *Correction du padding Q4*.

Recipe: W ~ N(0, 0.02^2) float32 (before Q4_0 encoding), X ~ N(0, 1) float32,
ids ~ U[0, 131072) int32; seed = 1000 * workload_index + tensor_index.
"""

from __future__ import annotations

import numpy as np

VOCAB = 131072
DEC_DIM = 3072
ENC_DIM = 1280
PREFIX_TOKENS = 38
W_STD = np.float32(0.02)

# Decoder projections of one layer: (name, N, K).  q/k/v fused: 32*128 + 2*8*128
# = 6144 outputs; gate and up fused along N (2 x 9216).
DECODER_LAYER = (
    ("qkv", 6144, 3072),
    ("o", 3072, 4096),
    ("gate_up", 18432, 3072),
    ("down", 3072, 9216),
)

# Encoder projections (width 1280, 32 heads of 40) plus the adapter after the
# 4x convolutional downsample (4 frames of 1280 concatenated -> 5120 -> 3072).
ENCODER_LAYER = (
    ("qkv", 3840, 1280),
    ("o", 1280, 1280),
    ("up", 5120, 1280),
    ("down", 1280, 5120),
)
ADAPTER = ("adapter", 3072, 5120)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weights(n: int, k: int, seed: int) -> np.ndarray:
    """float32 [n, k] drawn N(0, 0.02^2)."""
    return rng(seed).standard_normal((n, k), dtype=np.float32) * W_STD


def activations(m: int, k: int, seed: int) -> np.ndarray:
    """float32 [m, k] drawn N(0, 1)."""
    return rng(seed).standard_normal((m, k), dtype=np.float32)


def token_ids(count: int, seed: int, vocab: int = VOCAB) -> np.ndarray:
    """int32 [count] drawn uniformly from [0, vocab)."""
    return rng(seed).integers(0, vocab, count, dtype=np.int32)


def seed_for(workload: int, tensor: int) -> int:
    return 1000 * workload + tensor
