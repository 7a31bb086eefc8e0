"""CPU oracle for paged-attention decode and the KV-cache scatter.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import, call or execute anything in this
package. The library (``paged_attention_decode_amd``) never does, and shares no
code with it: the two sides have independent implementations of the cache
layout, the gather and the arithmetic. The only common code is the seeded
input generator in ``workloads/``, which holds none of the method's arithmetic.

Everything is computed in float64 with numpy, one sequence and one head at a
time, so that each step can be checked against its definition by eye.

Pins (see ``tests/test_oracle.py``): brute force against
``torch.nn.functional.scaled_dot_product_attention`` in float64 on dense K/V;
closed forms (one token returns its value row, equal keys return the mean of
V, hand-derived weights in ``tests/golden/``); invariants (weights sum to one,
relabelling physical blocks changes nothing, key shift, affine values, the
grouped-query head mapping); the split/merge identity against the dense
result; the cache layout against numpy reshape/transpose construction; and
the causal prefill against SDPA with a causal or offset mask and against the
decode definition for one new token.
No oracle function is left unpinned.
"""

from .paged_attention import (  # noqa: F401
    CacheGeometry,
    decode,
    decode_sequence,
    decode_split,
    gather_kv,
    k_index,
    merge_partitions,
    prefill,
    store_kvcache,
    v_index,
    widen,
)
