"""Batched speculative-sampling verification on AMD Instinct MI355X (gfx950).

The verification step (accept test, first-rejection scan, residual or bonus
draw, greedy rule) runs in the HIP kernels of libspecverify.so behind a C ABI
(include/spec_verify.h). This package holds the ctypes binding and a small
torch-facing wrapper (`Verifier`) that allocates outputs and passes the current
HIP stream. Torch is used only for device memory and streams.
"""
from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, SV_BF16, SV_EDATA, SV_EHIP, SV_EINVAL, SV_ENOMEM, SV_F32, SV_OK,
    SV_DATA_CONTEXT, SV_DATA_CU_GAMMA, SV_DATA_STATE, SV_DATA_DRAFT_ID, SV_DATA_NONFINITE, SV_DATA_UNIFORM,
    SV_DATA_STALL,
    SV_NGRAM_MAX_N,
    SV_PATH_AUTO, SV_PATH_ONE_LAUNCH, SV_PATH_TWO_LAUNCH, SV_PATH_POOLED, SV_SAMPLE_LOGITS, SV_SAMPLE_WEIGHTS,
    SpecVerifyError, load_library, spec_verify_check_args, spec_verify_create,
    spec_verify_destroy, spec_verify_kernel_times, spec_verify_last_error, spec_verify_last_path,
    spec_verify_run, spec_verify_set_path, spec_verify_set_timing, spec_verify_set_timing_stride,
    spec_verify_status, spec_sample_run, spec_verify_run_onehot, spec_ngram_propose, spec_adapt_gamma,
    spec_vshard_rows, spec_vshard_decide, spec_vshard_finish, vshard_desc, VShardDesc,
    VSHARD_REC_BYTES, VSHARD_PART_DOUBLES, VSHARD_LOCAL_DOUBLES,
    spec_verify_run_static, spec_verify_run_bound, SV_STATIC_MAX_BATCH, SV_STATIC_MAX_ROWS, SV_STATIC_MAX_GAMMA,
)
from .verifier import VocabShard, Verifier, VerifyOutputs  # noqa: F401
