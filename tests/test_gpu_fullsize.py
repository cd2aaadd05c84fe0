"""Parity at the full workload sizes, in the launch configuration bench.py
times: stats and selection compared on every block and row, attention on
256 sampled (KV head, query block) rows that the oracle computes one by one
(every KV head's first, last and two longest rows among them)."""
import pytest

from block_sparse_long_rbs_amd import inputs

import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_mixture_bf16_32k_full_size():
    """32,768 tokens, 64/8 heads, keep-ratio 0.05, compact/high-radius key mixture."""
    H.pipeline_case(inputs.mixture_bf16_32k(), sample_rows=256, seed=1)


@pytest.mark.timeout(900)
def test_mixture_bf16_128k_full_size():
    """131,072 tokens, 32/4 heads, keep-ratio 0.03, sink, the benchmarked workload."""
    H.pipeline_case(inputs.mixture_bf16_128k(), sample_rows=256, seed=2)
