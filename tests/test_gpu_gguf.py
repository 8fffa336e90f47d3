"""Q4_0 tensors read from a GGUF file (split into byte pieces, as the pages'
loader does) go straight to the kernels: the bytes the reader returns are the
kernels' weight layout, with no repacking ("Implémentation en Rust du modèle
Voxtral Mini 4B Realtime de Mistral pour l'exécuter dans le navigateur",
sections "Architecture" and "Préparation du modèle et sharding")."""

import numpy as np
import pytest

import gguf_writer as W
import q4_quantized_speech_amd as q4
from gpu_util import announce, assert_within, dev, host, needs_gpu
from oracle import q4_oracle as O
from q4_quantized_speech_amd import synth

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_gguf_tensors_feed_the_kernels(tmp_path):
    rng = np.random.Generator(np.random.PCG64(91))
    shapes = {"blk.0.ffn_down.weight": (300, 640), "token_embd.weight": (513, 96)}
    wq = {k: O.quantize_q4_0((rng.standard_normal(s) * 0.02).astype(np.float32))
          for k, s in shapes.items()}
    tensors = [(k, (s[1], s[0]), W.T_Q4_0, wq[k].tobytes()) for k, s in shapes.items()]
    blob = W.build([("general.architecture", W.STRING, "voxtral")], tensors)[0]
    paths = W.write_shards(blob, str(tmp_path / "m.gguf"), list(range(4096, len(blob), 4096)))
    with q4.Gguf(paths) as g:
        wd = g.read("blk.0.ffn_down.weight")
        emb = g.read("token_embd.weight")
    assert np.array_equal(wd, wq["blk.0.ffn_down.weight"])

    n, k = shapes["blk.0.ffn_down.weight"]
    x = synth.activations(3, k, 17)
    announce("gguf -> matvec 300x640 M=3")
    y = host(q4.matvec(dev(wd), dev(x)))
    ref, b = O.matmul_f64(wd, x, n, k)
    assert_within(y, ref, b, O.MATVEC_REL, O.MATVEC_ABS, "matvec on a GGUF tensor")

    n, k = shapes["token_embd.weight"]
    ids = np.array([0, 512, 7, 300], np.int32)
    announce("gguf -> embed_rows 513x96")
    got = host(q4.embed_rows(dev(emb), dev(ids)))
    assert np.array_equal(got.view(np.uint32), O.embed_rows(emb, ids, n, k).view(np.uint32))
