"""Plain, slow, fp64 CPU oracle for ResidualAttention and the fork bookkeeping.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
calls it and shares no code with it.

What it computes (ForkKV study note, sections "2. Q1 / Q2 / Q3", "3. 架构 / 方法图"
and the "Reconstruction" / "Attention fusion" equations of "4. 作者证明"):
for every agent the full key and value are the base projection plus the
up-projected residual, ``K = RoPE(xW_k + s * xA_k B_k)`` and
``V = xW_v + s * xA_v B_v``; attention is textbook softmax attention over them.
The oracle materialises these merged K/V per agent and KV head and runs a plain
softmax -- it does not follow the pages' fused-kernel algorithm.

Pins (see ``tests/test_oracle_pins.py``): pure-Python brute force on tiny inputs,
the zero-adapter case against ``torch.nn.functional.scaled_dot_product_attention``,
RoPE invariants, the deferred-RoPE and associativity identities, a CPU model of
the fused online-softmax form with split-K merging, and (bookkeeping) the block
counts of the ForkServe README's Results table.  Every function here is pinned;
none is "parity unpinned".
"""
from .storage import decode_values, base_key_rows, base_value_rows, res_key_rows, res_value_rows
from .rope import inv_freq, rope_rotate, rope_unrotate
from .attention import merged_kv, decode_attention, prefill_attention, apply_chunk_write
from .pool_model import PoolModel, PoolError

__all__ = ["decode_values", "base_key_rows", "base_value_rows", "res_key_rows",
           "res_value_rows", "inv_freq", "rope_rotate", "rope_unrotate", "merged_kv",
           "decode_attention", "prefill_attention", "apply_chunk_write", "PoolModel",
           "PoolError"]
