"""Write quant_sweep_digests.json: for every chunk of the exhaustive
quantiser-domain sweep (tests/quant_sweep.py), the SHA-256 of the oracle's
fp8 bytes and of its fp32 scales.  Calls only oracle/ for the expected values.

    python tests/golden/make_quant_sweep.py [processes]
"""
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import quant_sweep as S  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402


def one(c):
    x = O.bf16_from_bits(S.chunk_tokens(c))
    qs, ss = [], []
    for r0 in range(0, x.shape[0], 1024):            # bounded memory
        qq, sc = O.quantize_rows(x[r0:r0 + 1024])
        qs.append(qq)
        ss.append(sc)
    import numpy as np
    return c, S.digest(np.concatenate(qs)), S.digest(np.concatenate(ss))


def main():
    procs = int(sys.argv[1]) if len(sys.argv) > 1 else max(1, (os.cpu_count() or 2) // 2)
    n = S.n_chunks()
    res = {}
    with ProcessPoolExecutor(procs) as ex:
        for c, dq, ds in ex.map(one, range(n)):
            res[c] = {"q_sha256": dq, "scale_sha256": ds}
            print(f"chunk {c + 1}/{n} done", flush=True)
    out = {"source": "oracle.moe_oracle.quantize_rows over tests/quant_sweep.chunk_tokens(c); "
                     "written by tests/golden/make_quant_sweep.py",
           "H": S.H, "rows_per_chunk": S.ROWS_PER_CHUNK, "pairs": S.n_pairs(), "chunks": n,
           "digests": [res[c] for c in range(n)]}
    with open(os.path.join(HERE, "quant_sweep_digests.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
