"""Oracle: the prune predicate (test infrastructure).

Restated from the predicate printed on the llama.cpp Gemma 4 prefill page
(section 1, both language versions): pruning of non-output rows before the
first KV-shared layer is allowed only when the output rows can be cropped
(no next-n head needs other rows), the first shared layer index lies
strictly inside (0, n_layer), embeddings are not being extracted, only one
sequence is in flight, and no layer from the first shared one up to and
including index n_layer (the final hidden state) has its input extracted.
"""
from __future__ import annotations


def prune_shared(n_layer: int, n_layer_kv_from_start: int, embeddings: bool, n_seq_max: int,
                 embeddings_layer_inp, crop_before_nextn: bool = True) -> bool:
    ok = (bool(crop_before_nextn) and n_layer_kv_from_start > 0
          and n_layer_kv_from_start < n_layer and not embeddings and n_seq_max == 1)
    il = n_layer_kv_from_start
    while ok and il <= n_layer:
        ok = not embeddings_layer_inp[il]
        il += 1
    return ok
