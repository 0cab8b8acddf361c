"""Writes tests/golden/scaling_points.json: the step compression S of the
oracle's lookahead decoding on the two small random-init models whose greedy
continuations of a repeated-motif prompt repeat n-grams (micro: 1 layer,
vocab 8; tiny: 2 layers, vocab 256), for N in {3, 4, 5} and W = G in
{1, 2, 3, 4, 5, 7, 10, 15}, prompt as reference, 16 motif prompts (seeds
0-15) of 128 new tokens each; S = all tokens / all steps.  These are the
points the scaling-law fit of [LD] §4 (Eq. 5 and 7) is checked against.
Calls only oracle/ and synth/ (the seeded inputs).

    python3 tests/golden/make_scaling_points.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import lookahead as la  # noqa: E402
from oracle.model import OracleModel  # noqa: E402

NS = (3, 4, 5)
WS = (1, 2, 3, 4, 5, 7, 10, 15)
PROMPTS = 16
NEW = 128


def main():
    out = {"source": "tests/golden/make_scaling_points.py (oracle lookahead, float64)",
           "recipe": {"N": list(NS), "W=G": list(WS), "prompts": PROMPTS, "new_tokens": NEW,
                      "prompt": "synth.prompt_motif(vocab, seed=k), k < 16",
                      "window": "synth.gen_window(N, W, vocab, seed=2)",
                      "prompt_ref": True, "weights": "synth.gen_weights(shape, 0)"},
           "models": {}}
    for name in ("micro", "tiny"):
        s = synth.SHAPES[name]
        om = OracleModel(s, synth.gen_weights(s, 0))
        prompts = [synth.prompt_motif(s.vocab, seed=k) for k in range(PROMPTS)]
        pts = []
        for N in NS:
            for W in WS:
                win = synth.gen_window(N, W, s.vocab, seed=2)
                toks = steps = 0
                for pr in prompts:
                    r = la.lookahead(om, pr, N, W, W, NEW, win, prompt_ref=True)
                    toks += len(r.tokens)
                    steps += r.steps
                pts.append({"N": N, "W": W, "G": W, "tokens": toks, "steps": steps,
                            "S": toks / steps})
                print(name, N, W, round(toks / steps, 4), flush=True)
        out["models"][name] = pts
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "scaling_points.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
