"""MI355X (gfx950) library for the Kimi Delta Attention layer path.

The compute lives in ``libkda.so`` (HIP kernels behind the C ABI of
``include/kda.h``); :mod:`hybrid_recurrent_serving_amd.kda` is its thin
ctypes binding and :mod:`hybrid_recurrent_serving_amd.inputs` draws the
seeded synthetic workloads.  Importing the package loads nothing; the
library is loaded on first use of a binding function.
"""

from .kda import (KDA_BF16, KDA_F32, KDAError, kda_abi_version, kda_args_sizeof,  # noqa: F401
                  kda_ckpt_plan, kda_ckpt_plan_device, kda_conv_short, kda_decode, kda_decode_conv,
                  kda_last_error,
                  kda_prefill_varlen, kda_prefill_workspace_bytes, kda_status_str, kda_verify,
                  kda_verify_conv,
                  load_library, prepare_conv_short, prepare_decode, prepare_decode_conv, Prepared)
