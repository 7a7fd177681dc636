"""fp64 CPU oracle for the FlashAttention forward pass and its gradients.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The library (``flashattention_forward_02_amd``) never imports it, and this package
imports nothing from the library: the two share no code. Inputs come from
``seeded_inputs`` (random draws and storage formats only).

Sources, cited by tag and section throughout:

* [FA-Simplified] "FlashAttention 简化版：Tiling + Online Softmax"
  (forceinjection.github.io, 02_npu_programming/09_flash_attention).
* [FA-Fill] "Flash Attention 代码填空 (Level 2-3)" (boots-coder.github.io, LLM-101-CN).
* [CS349E-L11] "CS349E 第 11 讲 01_online_softmax.py" (semidirectx.com, cs349e/code/lecture11).
* [FA-Scratch] "从零手写 FlashAttention（PyTorch实现 + 原理推导）" (mokono.cn, news/2160643).

What each function is pinned against (tests/test_oracle_pins.py):

* ``attention_fp64`` -- brute force in pure Python on tiny inputs; torch's
  float64 scaled-dot-product attention and scipy's softmax; closed forms (one key,
  constant V, zero scale, two keys, V = I); shift and joint-permutation
  invariance; the one-pass recurrence at the pages' demo size.
* ``online_softmax`` / ``safe_softmax`` -- scipy's softmax; overflow-free on
  shifted inputs where the naive form overflows.
* ``online_attention`` / ``online_attention_row`` -- the three-pass definition at
  the 1e-16 level the lecture-11 demo 1 reports.
* ``partial_state`` / ``merge_states`` / ``merge_*`` -- order independence at the
  1e-16 level the lecture-11 demo 2 reports, on the demo's own draws; empty states.
* ``partial_state_lse`` / ``merge_lse`` (the (lse, o / l) form) -- the merged output against
  full attention and the merged lse against scipy's logsumexp, on demo 2's own draws and
  under the causal mask; order independence; empty and single-part states.
* ``fa1_order_attention`` -- the delayed-normalisation form.
* ``round_to_bf16`` / ``round_to_f16`` -- torch's and numpy's casts; the
  relative P.V error magnitudes the lecture-11 demo 4 reports.
* the causal mask (``attention_fp64(causal=True)``, ``causal_last_key``) -- literal
  loops over the visible keys; torch's float64 attention with is_causal for Nq = Nk;
  each row equals unmasked attention over its key prefix; Nq < Nk equals the last
  rows of the square problem; masked split states merge to the masked result.
* grouped K/V heads (``kv_head_of``, K/V with fewer heads than Q) -- the head map
  written out; torch's float64 attention with enable_gqa; MHA on repeated K/V heads.
* ``attention_backward_fp64`` (dq, dk, dv, log-sum-exp, D) -- central finite differences
  of the forward definition; torch's float64 autograd through its own softmax (causal
  and grouped heads included); closed forms (one key, zero scale, constant V); the
  shift invariance sum_j dK_j = 0; D_i = sum_c dO_ic O_ic; the log-sum-exp against
  scipy's; [FA-Fill Exercise 5]'s blocked recomputation of dV from the stored (m, l),
  on the exercise's own recipe (torch seed 42, N = 64, d = 32, blocks of 16).

Parity unpinned: nothing in this package. (The exact bf16 error of a GPU kernel
depends on where its tiles fall and is bounded by the tolerance, not pinned.)
"""
from .attention import (  # noqa: F401
    scores_fp64,
    causal_last_key,
    kv_head_of,
    attention_fp64,
    attention_rows_fp64,
    safe_softmax,
    naive_softmax,
    online_softmax,
    online_attention_row,
    two_pass_attention_row,
    online_attention,
    fa1_order_attention,
    partial_state,
    merge_states,
    merge_sequential,
    merge_tree,
    finish_state,
    split_bounds,
    split_partial_states,
    partial_state_lse,
    merge_lse,
    split_partial_states_lse,
    brute_force_attention,
    round_to_bf16,
    round_to_f16,
)
from .backward import (  # noqa: F401
    attention_backward_fp64,
    attention_loss_fp64,
    dv_from_statistics_blocked,
)
