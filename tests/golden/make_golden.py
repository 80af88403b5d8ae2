"""Writes the hand-derived fixtures in this folder.

Every expected value is a closed form worked by hand from the rule its
``cite`` field names; ``math.log``/``math.exp`` only evaluate those closed
forms.  Nothing here calls the oracle or the HIP library.
Run: ``python tests/golden/make_golden.py`` from the repository root.
"""
import json
import math
import os

L = math.log
HERE = os.path.dirname(os.path.abspath(__file__))


def _dump(name, about, cases):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump({"about": about, "cases": cases}, f, indent=1)
        f.write("\n")


def transforms_cases():
    Z4 = 3 * math.exp(3.0) + math.exp(2.0)
    return [
        {"name": "inclusive_top_p_keeps_crossing_token",
         "cite": "xorl issue #71, section 3 (transform program: inclusive top-p crossing)",
         "x": [L(5), L(3), L(2)], "tau": 1.0, "top_k": 0, "top_p": 0.75, "min_p": 0.0, "target": 1,
         "expect": {"support_len": 2, "support_ids": [0, 1], "threshold_ties": 1,
                    "logprob": L(3 / 8), "entropy": -(5 / 8 * L(5 / 8) + 3 / 8 * L(3 / 8)), "status": 0},
         "derivation": "masses 0.5, 0.3, 0.2; the mass before rank 1 is 0.5 < 0.75 so rank 1 (which crosses "
                       "0.75) is kept; the mass before rank 2 is 0.8 >= 0.75 so it is dropped; on {0,1} the "
                       "target 1 has probability 3/8"},
        {"name": "top_p_small_gives_singleton",
         "cite": "xorl issue #71, section 3 (inclusive top-p); SkyRL PR #2004 description (singleton support "
                 "has zero entropy)",
         "x": [L(5), L(3), L(2)], "tau": 1.0, "top_k": 0, "top_p": 0.4, "min_p": 0.0, "target": 0,
         "expect": {"support_len": 1, "support_ids": [0], "threshold_ties": 1, "logprob": 0.0, "entropy": 0.0,
                    "status": 0},
         "derivation": "the mass before rank 1 is 0.5 >= 0.4, so only rank 0 stays; a one-token support has "
                       "logprob 0 and entropy 0"},
        {"name": "temperature_applies_before_top_p",
         "cite": "xorl issue #71, section 3 (program starts with temperature)",
         "x": [L(5), L(3), L(2)], "tau": 0.5, "top_k": 0, "top_p": 0.6, "min_p": 0.0, "target": 0,
         "expect": {"support_len": 1, "support_ids": [0], "threshold_ties": 1, "logprob": 0.0, "entropy": 0.0,
                    "status": 0},
         "derivation": "z = 2x gives masses 25/38, 9/38, 4/38; the mass before rank 1 is 25/38 = 0.658 >= 0.6 "
                       "(at tau = 1 it would be 0.5 < 0.6 and two tokens would stay)"},
        {"name": "stable_token_id_top_k_ties",
         "cite": "xorl issue #71, section 3 (stable token-id top-k: equal logits ordered by ascending id)",
         "x": [1.0, 3.0, 3.0, 2.0, 3.0], "tau": 1.0, "top_k": 2, "top_p": 1.0, "min_p": 0.0, "target": 4,
         "expect": {"support_len": 2, "support_ids": [1, 2], "threshold_ties": 2, "threshold_logit": 3.0,
                    "logprob": "-inf", "entropy": L(2), "status": 2},
         "derivation": "rank order (logit desc, id asc) is 1, 2, 4, 3, 0; top-2 is {1, 2}; id 4 ties at logit 3 "
                       "but has the larger id so it is outside; two equal logits give entropy ln 2"},
        {"name": "stable_top_k_threshold_below_tie_run",
         "cite": "xorl issue #71, section 3",
         "x": [1.0, 3.0, 3.0, 2.0, 3.0], "tau": 1.0, "top_k": 4, "top_p": 1.0, "min_p": 0.0, "target": 3,
         "expect": {"support_len": 4, "support_ids": [1, 2, 4, 3], "threshold_ties": 1, "threshold_logit": 2.0,
                    "logprob": 2.0 - L(Z4),
                    "entropy": -(3 * math.exp(3) / Z4 * (3 - L(Z4)) + math.exp(2) / Z4 * (2 - L(Z4))),
                    "status": 0},
         "derivation": "top-4 = ids 1, 2, 4 (logit 3) and 3 (logit 2); LSE = ln(3e^3 + e^2); logprob of id 3 = "
                       "2 - LSE"},
        {"name": "min_p_against_original_max",
         "cite": "xorl issue #71, section 3 (min-p relative to the original row max)",
         "x": [0.0, L(0.5), L(0.04), L(0.06)], "tau": 1.0, "top_k": 0, "top_p": 1.0, "min_p": 0.05, "target": 3,
         "expect": {"support_len": 3, "support_ids": [0, 1, 3], "threshold_ties": 1,
                    "logprob": L(0.06 / 1.56), "entropy": -sum(p / 1.56 * L(p / 1.56) for p in (1, 0.5, 0.06)),
                    "status": 0},
         "derivation": "p / p_max = 1, 0.5, 0.04, 0.06; min-p 0.05 keeps ids 0, 1, 3 (rank order 0, 1, 3); "
                       "total kept weight 1.56"},
        {"name": "top_p_on_top_k_renormalised_masses",
         "cite": "xorl issue #71, section 3 (top-k precedes top-p in the program) -- reading: top-p mass is "
                 "taken after top-k renormalisation",
         "x": [L(0.4), L(0.3), L(0.2), L(0.1)], "tau": 1.0, "top_k": 2, "top_p": 0.5, "min_p": 0.0, "target": 0,
         "expect": {"support_len": 1, "support_ids": [0], "threshold_ties": 1, "logprob": 0.0, "entropy": 0.0,
                    "status": 0},
         "derivation": "top-2 renormalised masses 4/7, 3/7: the mass before rank 1 is 4/7 >= 0.5, so one token "
                       "stays (on the unrenormalised masses it would be 0.4 < 0.5 and two would stay)"},
        {"name": "all_equal_logits_top_k_5",
         "cite": "xorl issue #71, section 3 (stable token-id tie-break)",
         "x": [0.5] * 7, "tau": 1.0, "top_k": 5, "top_p": 1.0, "min_p": 0.0, "target": 2,
         "expect": {"support_len": 5, "support_ids": [0, 1, 2, 3, 4], "threshold_ties": 5, "threshold_logit": 0.5,
                    "logprob": -L(5), "entropy": L(5), "status": 0},
         "derivation": "seven equal logits: rank order is id order; top-5 is ids 0..4, uniform over 5 tokens"},
        {"name": "identity_program_is_full_vocabulary",
         "cite": "xorl issue #71, section 3 (top_p == 1.0 is the full support)",
         "x": [L(5), L(3), L(2)], "tau": 1.0, "top_k": 0, "top_p": 1.0, "min_p": 0.0, "target": 2,
         "expect": {"support_len": 3, "support_ids": [0, 1, 2], "threshold_ties": 1,
                    "logprob": L(0.2), "entropy": -(0.5 * L(0.5) + 0.3 * L(0.3) + 0.2 * L(0.2)), "status": 0},
         "derivation": "no filter active: the support is the whole vocabulary and the scores are plain softmax"},
    ]


def full_cases():
    return [
        {"name": "uniform_logits_V%d" % V,
         "cite": "SkyRL PR #2004 (full-vocabulary entropy path): uniform softmax over V tokens",
         "V": V, "entropy": L(V), "logprob": -L(V), "derivation": "p_v = 1/V: entropy ln V, logprob -ln V"}
        for V in (4096, 129280, 151936)
    ] + [
        {"name": "three_tokens", "cite": "xorl issue #71 section 1 (log-sum-exp, selected logprob)",
         "x": [L(5), L(3), L(2)], "tau": 1.0, "target": 1, "lse": L(10), "logprob": L(0.3),
         "entropy": -(0.5 * L(0.5) + 0.3 * L(0.3) + 0.2 * L(0.2)),
         "derivation": "weights 5, 3, 2: LSE ln 10, p = 0.5, 0.3, 0.2"},
        {"name": "three_tokens_tau_half",
         "cite": "SkyRL PR #2004 review code (divide by temperature after the dot product)",
         "x": [L(5), L(3), L(2)], "tau": 0.5, "target": 0, "lse": L(38), "logprob": L(25 / 38),
         "entropy": -sum(w / 38 * L(w / 38) for w in (25, 9, 4)), "derivation": "z = 2x: weights 25, 9, 4"},
    ]


def l1_cases():
    return [
        {"name": "two_token",
         "cite": "DeepSpec PR #87 (Purpose: per-token L1 distance, accept_rate = clamp(1 - 0.5 L1, 0, 1))",
         "target": [0.0, 0.0], "draft": [L(3), 0.0], "l1": 0.5, "accept_rate": 0.75,
         "derivation": "P = (1/2, 1/2), Q = (3/4, 1/4): |1/2-3/4| + |1/2-1/4| = 1/2"},
        {"name": "identical", "cite": "DeepSpec PR #87", "target": [1.0, -2.0, 0.5, 3.0],
         "draft": [1.0, -2.0, 0.5, 3.0], "l1": 0.0, "accept_rate": 1.0, "derivation": "P = Q"},
        {"name": "three_token", "cite": "DeepSpec PR #87", "target": [L(5), L(3), L(2)],
         "draft": [L(2), L(3), L(5)], "l1": 0.6, "accept_rate": 0.7,
         "derivation": "P = (.5,.3,.2), Q = (.2,.3,.5): 0.3 + 0 + 0.3"},
    ]


if __name__ == "__main__":
    _dump("transforms_cases.json", "Hand-derived cases for the sampling-transform oracle. The pages print no "
          "worked numbers; each case is a closed form worked from the rule its 'cite' names.", transforms_cases())
    _dump("full_cases.json", "Hand-derived full-vocabulary scoring cases (closed forms).", full_cases())
    _dump("l1_cases.json", "Hand-derived softmax-L1 cases.", l1_cases())
