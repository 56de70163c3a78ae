"""Writes datagen_sha256.txt: a sha256 of every tensor the seeded input
generator produces for each named workload, shrunk to a size that generates
in well under a second (batch <= 2, seq_len <= 3000, n_q <= 64; block,
m, k, heads, landmarks and mode as named), the small prefill workload at its
full size, and one full-length sequence of the 128k decode workload.

These are fingerprints of inputs, not expected results: the generator holds
none of the method's arithmetic, and nothing here calls the oracle or the
library.  A changed hash means the inputs of every parity test and of the
bench changed (a different numpy/torch stream or rounding, or an edit of
the generator); regenerate only for a deliberate edit of the generator.

Usage: python tests/golden/make_datagen_hashes.py
"""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from hierarchical_index_sparse_amd import datagen  # noqa: E402
from hierarchical_index_sparse_amd.workloads import WORKLOADS  # noqa: E402

OUT = os.path.join(HERE, "datagen_sha256.txt")


def shrunk(w):
    L = min(w.seq_len, 3000)
    kw = dict(batch=min(w.batch, 2), seq_len=L, n_q=min(w.n_q, 64, L))
    if w.varlen_min:
        kw["varlen_min"] = min(w.varlen_min, L)
    return w.with_(**kw)


def cases():
    for name, w in sorted(WORKLOADS.items()):
        yield f"{name}@small", shrunk(w)
    yield "tiny_prefill_4k@full", WORKLOADS["tiny_prefill_4k"]
    # one sequence of the 128k decode cache: K and V span several generator
    # chunks of 2^22 elements, each drawn from its own stream
    yield "decode_128k@batch1", WORKLOADS["decode_128k"].with_(batch=1)


def fingerprint(a):
    h = hashlib.sha256()
    h.update(f"{a.dtype.str}{a.shape}".encode())
    h.update(a.tobytes())
    return h.hexdigest()


def lines():
    for label, w in cases():
        inp = datagen.make_inputs(w)
        for key in sorted(inp):
            if inp[key] is not None:
                yield f"{label} {key} {fingerprint(inp[key])}"


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write("# sha256 of (dtype, shape, bytes) of each generated input tensor; written by\n"
                "# make_datagen_hashes.py from the seeded generator alone\n")
        for ln in lines():
            f.write(ln + "\n")
    print(f"wrote {OUT}")
