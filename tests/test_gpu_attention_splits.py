"""GPU parity of the decode attention's work split: several 64-position
sub-chunks per workgroup (the double-buffered loop), several splits per
(row, kv head) merged by the last workgroup, and the current position ending
part-way through a sub-chunk -- at head dim 64 (tiny decoder) and 128 (the
Llama-3.1-8B layer shapes, four query heads per kv head), for the attention
with the scores on the matrix cores and for the vector-ALU one.

Every decode step is checked stage by stage (tests/teacher_forcing.py): the
attention output of every (row, query head) against the exact softmax over
every position the cache holds, computed in float64 from the stored q and
K/V, and every other stored activation, the exit decisions and the logits
against their exact values from the stored inputs.
"""
import pytest

import synth
from test_gpu_parity_full import parity_run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_w():
    return synth.make_weights(synth.TINY, seed=0, device="cuda")


@pytest.fixture(scope="module")
def w8b_2():
    return synth.make_weights(synth.LLAMA_8B, seed=0, device="cuda", n_layers=2)


# tiny, B=8, a 700-token prompt, 3 steps (positions 700..702, cache of 703):
#   chunk 128  -> 6 splits of 2 sub-chunks; the last split ends inside its
#                 first sub-chunk (640..703);
#   chunk 256  -> 3 splits of 4 sub-chunks; position 700 lies in the third
#                 sub-chunk of the last split;
#   chunk 1024 -> one split that walks all 11 sub-chunks and writes directly.
@pytest.mark.parametrize("attn", ["mfma", "valu"])
@pytest.mark.parametrize("chunk", [128, 256, 1024])
def test_attention_sub_chunks_tiny(tiny_w, chunk, attn):
    parity_run(synth.TINY, tiny_w, B=8, T=700, steps=3, tau=0.5, attn=attn, chunk=chunk,
               check_prefill=False)


# 8B layer shapes (head dim 128, 32 q / 8 kv heads), one row, a 500-token
# prompt (cache of 503): the library's own choice is 8 splits of one
# sub-chunk merged by the last workgroup; chunk 256 gives 2 splits of 4
# sub-chunks with positions 500..502 in the last one; chunk 1024 one split
# (the matrix-core kernel then runs eight wavefronts, 128 positions per
# sub-chunk, no merge).
@pytest.mark.parametrize("attn", ["mfma", "valu"])
@pytest.mark.parametrize("chunk", [0, 256, 1024])
def test_attention_splits_8b_batch1(w8b_2, chunk, attn):
    parity_run(synth.LLAMA_8B, w8b_2, B=1, T=500, steps=3, tau=0.5, attn=attn, chunk=chunk,
               check_prefill=False)


# 8B layer shapes, 32 rows, 1,100-token prompts (cache of 1,102): the
# library's own choice is 2 splits of 576 positions (9 sub-chunks each), the
# configuration of the batch-32 workload.  The float64 oracle cannot prefill
# 35,200 rows at these shapes in seconds, so the decode steps are checked
# against the cache the GPU's prefill wrote.
@pytest.mark.parametrize("attn", ["mfma", "valu"])
def test_attention_default_chunk_8b_batch32(w8b_2, attn):
    parity_run(synth.LLAMA_8B, w8b_2, B=32, T=1100, steps=2, tau=0.5, attn=attn,
               check_prefill=False, free_running=False)


# The long-context workload's shape: 8 rows, 16,384-token prompts, the 8B
# layer shapes (2 layers), the library's own split (about 1,088 positions,
# 17 sub-chunks, per workgroup).  Decode steps checked stage by stage against
# the cache the GPU's prefill wrote (the float64 oracle cannot prefill
# 131,072 rows in seconds).
def test_decode_parity_8b_long_context_batch8(w8b_2):
    parity_run(synth.LLAMA_8B, w8b_2, B=8, T=16384, steps=2, tau=0.5, check_prefill=False,
               free_running=False)


# The 1B workload's prompt length (256 tokens, one row, tied embeddings),
# prefill and decode checked stage by stage, a free-running oracle beside.
def test_parity_1b_layer_shapes_prompt256():
    w = synth.make_weights(synth.LLAMA_1B, seed=0, device="cuda", n_layers=2)
    parity_run(synth.LLAMA_1B, w, B=1, T=256, steps=3, tau=0.5)
