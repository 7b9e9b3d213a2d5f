"""The layer shapes read from the Strata pages, checked against the figures
the pages print (tests/golden/pages_figures.txt).

The pages give no formula for an expert's size; reading taken: each expert is
a SwiGLU FFN of three d x f matrices with d = 2048, f = 768 and 512 experts in
each of 48 layers.  The printed cache figures then imply bits per weight that
must fall in the range of the quantisation levels the pages name (2-bit to
4-bit), and the total must fit the 125B parameter / ~60 GB at 4 bits figure.
"""
import os

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _figures():
    vals = {}
    with open(os.path.join(HERE, "golden", "pages_figures.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("="))
                vals[k] = float(v)
    return vals


def test_layer_count_times_experts_per_layer_is_the_printed_total():
    g = _figures()
    c = synth.CONFIGS["stack"]
    assert c.n_layers == g["n_layers"] == 48
    assert c.n_layers * c.E == g["n_experts_total"]
    assert c.k == g["experts_per_token"]
    assert c.n_resident == g["cached_experts"]


def test_expert_shape_fits_the_printed_model_size():
    g = _figures()
    c = synth.CONFIGS["prefill"]
    params_per_expert = 3 * c.d * c.f
    expert_params = g["n_experts_total"] * params_per_expert
    # all experts together are most of, and not more than, the 125B parameters
    assert 0.85 * g["model_params"] < expert_params <= g["model_params"]
    # four bits per weight: the experts alone take just under the printed ~60 GB
    assert 0.9 * g["model_bytes_4bit"] < expert_params * 4 / 8 <= g["model_bytes_4bit"]
    # the block-32 int4 format adds one fp16 scale per 32 weights: 4.5 bits per weight
    nbytes = oracle.expert_bytes(oracle.WFMT_I4B32, c.d, c.f)
    assert nbytes * 8 == params_per_expert * 4.5


def test_printed_cache_densities_imply_two_to_four_bit_experts():
    g = _figures()
    c = synth.CONFIGS["prefill"]
    params_per_expert = 3 * c.d * c.f
    bpw_700_per_gb = 1e9 / g["experts_per_gb"] * 8 / params_per_expert
    bpw_monitor = g["monitor_bytes"] / g["monitor_experts"] * 8 / params_per_expert
    assert 2.0 <= bpw_700_per_gb <= 3.0
    assert 2.5 <= bpw_monitor <= 4.0


def test_workload_batches_follow_the_printed_draft_and_chunk_sizes():
    g = _figures()
    assert synth.CONFIGS["decode_t4"].T == g["max_draft_tokens"] + 1
    assert synth.CONFIGS["decode_t1"].T == 1
    assert synth.CONFIGS["prefill"].T == g["prefill_chunk"]
