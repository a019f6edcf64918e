"""Train the four merge lists with the oracle's trainer and store them under workloads/vocabs/.

    python -m oracle.train_vocabs [v1 v2 v3 v4]

Each vocabulary is trained on a seeded synthetic corpus (workloads.textgen.VOCABS): the corpus is
pre-tokenized with the family's rules, and each step merges the most frequent adjacent pair (seen at
least twice), ties to the smallest (left, right), skipping merges whose token would exceed 128
bytes.  If the corpus runs out of pairs before the target count, the corpus is regrown with the same
generator and seed at twice the size.  The stored file records the corpus size and SHA-256.
"""
import os
import sys
import time

import numpy as np

from . import train
from workloads import textgen

OUT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "workloads", "vocabs")


def train_one(name):
    fam, n_merges, gen, size, seed = textgen.VOCABS[name]
    while True:
        t0 = time.time()
        corpus = getattr(textgen, gen)(seed, size).encode("utf-8")
        t1 = time.time()
        merges = train(fam, corpus, n_merges, 128)
        t2 = time.time()
        print(f"{name}: corpus {size} chars ({len(corpus)} bytes, {t1 - t0:.1f}s), "
              f"{merges.shape[0]} merges ({t2 - t1:.1f}s)", flush=True)
        if merges.shape[0] == n_merges:
            break
        size *= 2
    os.makedirs(OUT, exist_ok=True)
    np.savez_compressed(os.path.join(OUT, name + ".npz"), merges=merges,
                        family=np.array(fam), corpus_chars=np.array(size),
                        corpus_sha256=np.array(textgen.sha256(corpus)))


if __name__ == "__main__":
    for n in (sys.argv[1:] or ["v1", "v2", "v3", "v4"]):
        train_one(n)
