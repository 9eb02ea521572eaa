"""Write config0_oracle.npz: oracle outputs and final states of the tiny fp32
extend followed by one decode token per sequence.  Calls only oracle/ and the
seeded input generators."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle                                    # noqa: E402
from hybrid_model_linear_amd import synth        # noqa: E402


def main():
    ext, dec = synth.config0_tiny()
    out_e, _, fin_e = oracle.gdn_extend(ext.q, ext.k, ext.v, ext.a, ext.b, ext.A_log, ext.dt_bias,
                                        ext.cu_seqlens, ext.slot, ext.has_init, ext.pool, ext.scale)
    pool1 = oracle.apply_final_states(ext.pool, fin_e)
    out_d, _, fin_d = oracle.gdn_decode(dec.q, dec.k, dec.v, dec.a, dec.b, dec.A_log, dec.dt_bias,
                                        dec.slot, pool1, dec.scale)
    pool2 = oracle.apply_final_states(pool1, fin_d)
    touched = np.asarray(ext.slot)
    np.savez_compressed(os.path.join(HERE, "config0_oracle.npz"), extend_out=out_e,
                        decode_out=out_d, slots=touched, state_after_extend=pool1[touched],
                        state_after_decode=pool2[touched])


if __name__ == "__main__":
    main()
