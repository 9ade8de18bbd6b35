"""Plain fp64 CPU oracle of the pruned prompt prefill -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The engine (prompt_prefill_cross_amd) never does, and
this package imports nothing from the engine: the two share no code.  The
only inputs both sides see are the seeded bytes written by `synth`.

Sources (the pages, by title):
  * "llama.cpp Gemma 4 prefill KV graph optimization" (devotd.net, zh-hans
    and ko versions), section 1: layers from n_layer_kv_from_start on reuse an
    earlier layer's KV cache and write none; non-output token rows are pruned
    before the first such layer; intermediate ubatches skip those layers and
    the last ubatch runs one row; the prune predicate.  Section 3: outputs are
    identical with and without pruning.  Section 5: a unified KV cache (one
    buffer for every sequence) against split caches (one per sequence).
  * "PicoLM KV Cache persistence" (m.xxqk.cn), sections on the cache file
    (magic KVCP, positions / layers / KV dim, then FP16 K then FP16 V), the
    load check, and resuming the prompt loop after N cached positions.

Modules:
  model     -- container parser and Q4_0 dequantisation (closed form)
  forward   -- RMSNorm, RoPE, GELU/SiLU, causal attention, the forward pass,
               the unified cache and its attention masked by sequence
  kvcp      -- KVCP snapshot bytes (writer / reader / validation)
  predicate -- the prune predicate
"""
from .model import OracleModel, parse_model, deq_q4_0  # noqa: F401
from .forward import (KVState, prefill, prefill_multi, rms_norm, rope, gelu_tanh, silu,  # noqa: F401
                      attention, embed_rows, UnifiedKV, attention_cells, prefill_unified)
from .predicate import prune_shared  # noqa: F401
from . import kvcp  # noqa: F401
