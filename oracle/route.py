"""Top-k routing (oracle; test infrastructure).

Each token sends its hidden state to k of the E routed experts of the layer
([FTK], the paragraph introducing MoE routing: a router picks a few experts
per token; [FTK], decode paragraph: the router runs on the GPU).  Reading
adopted where the pages are silent:

* rank experts by logit descending, ties to the lower expert index, on the
  float32 logits the caller supplies;
* the gate weights are the softmax over the k kept logits, which equals the
  full softmax renormalised over the picks; computed in float64.
"""
import numpy as np


def topk_softmax(logits, k: int):
    """logits float32 [T, E] -> (ids int32 [T, k] in rank order, w float64 [T, k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("k out of range")
    idx = np.broadcast_to(np.arange(E), lg.shape)
    # lexsort: last key is primary -> (logit descending, index ascending)
    order = np.lexsort((idx, -lg.astype(np.float64)), axis=-1)
    ids = order[:, :k].astype(np.int32)
    z = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    ez = np.exp(z - z.max(axis=1, keepdims=True))
    w = ez / ez.sum(axis=1, keepdims=True)
    return ids, w
