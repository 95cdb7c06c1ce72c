"""Writes hand_examples.json: two worked examples derived by hand, evaluated
with nothing but the standard library's exp/log (never with the oracle).

Example 1, block mean selection (SparDA summary, Method: init tokens, sliding
window and top-k mean-pooled blocks; PulseCol §3.1 Eq. (2) for the masked softmax).
  g = 2, n_init = 1, window = 2, k = 2, d = 2, two query heads in one group,
  8 keys, one query at position 7.
  keys  t: 0 (1,0) 1 (1,2) 2 (3,1) 3 (1,1) 4 (2,0) 5 (0,2) 6 (5,5) 7 (1,1)
  pooled blocks: j0 (1,1)  j1 (2,1)  j2 (1,1)  j3 (3,3)
  F(7) = {0} U {6,7}; j3 lies inside F, so the candidates are j0, j1, j2.
  query heads (1,0) and (0,1) sum to (1,1); scores j0 = 2/sqrt2, j1 = 3/sqrt2,
  j2 = 2/sqrt2.  Top-2: j1, then j0 over j2 (equal score, lower index).
  Attended set {0,1} U {2,3} U {0} U {6,7} = {0,1,2,3,6,7}.
  V_t = (1, t).  Head 0 logits = key[0]/sqrt2, head 1 logits = key[1]/sqrt2.

Example 2, shared draft selection (S3R review, sparse drafting: recent window +
top-K, the selection fixed over the drafts, drafts causal among themselves).
  g = 1, n_init = 0, window = 2, k = 2, d = 2, one head; 6 history keys and 2
  drafts at positions 6 and 7; selection position 5.
  keys  t: 0 (1,0) 1 (0,1) 2 (2,2) 3 (-1,0) 4 (3,3) 5 (0,0) 6 (1,1) 7 (2,0)
  draft queries (1,0) and (0,1) sum to (1,1); F(5) = {4,5}; candidates 0..3
  with scores 1, 1, 4, -1 (over sqrt2).  Top-2: t2, then t0 over t1.
  Draft 0 attends {0,2,4,5,6}; draft 1 attends {0,2,4,5,6,7}.
"""
import json
import math
import os

R2 = math.sqrt(2.0)


def softmax_stats(logits, positions):
    z = sum(math.exp(x) for x in logits)
    mean_pos = sum(math.exp(x) * t for x, t in zip(logits, positions)) / z
    return [1.0, mean_pos], math.log(z)


def example1():
    A = [0, 1, 2, 3, 6, 7]
    k0 = {0: 1, 1: 1, 2: 3, 3: 1, 6: 5, 7: 1}
    k1 = {0: 0, 1: 2, 2: 1, 3: 1, 6: 5, 7: 1}
    o0, l0 = softmax_stats([k0[t] / R2 for t in A], A)
    o1, l1 = softmax_stats([k1[t] / R2 for t in A], A)
    return dict(
        name="block_mean_prefill_hand",
        workload=dict(h_q=2, h_kv=1, head_dim=2, seqlens_k=[8], seqlens_q=[1], block=2, topk=2,
                      n_init=1, window=2),
        q=[[[1, 0], [0, 1]]],
        k=[[[1, 0]], [[1, 2]], [[3, 1]], [[1, 1]], [[2, 0]], [[0, 2]], [[5, 5]], [[1, 1]]],
        v=[[[1, t]] for t in range(8)],
        k_cmp=[[1, 1], [2, 1], [1, 1], [3, 3]],
        selected=[[0, 1]], s_k=[2 / R2], s_k1=[2 / R2],
        count=[6, 6], out=[o0, o1], lse=[l0, l1])


def example2():
    kk = {0: (1, 0), 1: (0, 1), 2: (2, 2), 3: (-1, 0), 4: (3, 3), 5: (0, 0), 6: (1, 1), 7: (2, 0)}
    A0 = [0, 2, 4, 5, 6]
    A1 = [0, 2, 4, 5, 6, 7]
    o0, l0 = softmax_stats([kk[t][0] / R2 for t in A0], A0)
    o1, l1 = softmax_stats([kk[t][1] / R2 for t in A1], A1)
    return dict(
        name="shared_draft_hand",
        workload=dict(h_q=1, h_kv=1, head_dim=2, seqlens_k=[8], seqlens_q=[2], block=1, topk=2,
                      n_init=0, window=2, shared_selection=1),
        q=[[[1, 0]], [[0, 1]]],
        k=[[list(kk[t])] for t in range(8)],
        v=[[[1, t]] for t in range(8)],
        k_cmp=[],
        selected=[[0, 2]], s_k=[1 / R2], s_k1=[1 / R2],
        count=[5, 6], out=[o0, o1], lse=[l0, l1])


if __name__ == "__main__":
    out = dict(source="hand-derived; see make_hand_examples.py docstring", cases=[example1(), example2()])
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_examples.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(path)
