"""MI355X-native segment transform for position-independent caching of
hybrid-attention LLMs: build the cached pair (T_C, S(C|0)) of every prompt
segment, compose cached pairs into running states, and the naive-add
ablation, for the scalar-decay, diagonal-gate, dense gated-delta and KDA
(per-channel gated delta) forms, and the re-rotation of cached pairs to a new
position under rotary embeddings on the keys, and the warm-up of short
causal convolutions at segment starts.

The compute runs in the HIP library ``libpic.so`` (C ABI in
``include/pic.h``); this package is a thin ctypes binding over it.
"""
from ._lib import (DT_BF16, DT_F32, FORM_DENSE, FORM_DIAG, FORM_KDA, FORM_SCALAR, PLAN_BUILD,
                   PLAN_COMPOSE, PREC_FP16, PREC_FP32, ROPE_HALF, ROPE_INTERLEAVED, PicError, load,
                   pic_compose, pic_compose_noalloc, pic_compose_seams, pic_conv_warmup, pic_materialize_T, pic_naive_add,
                   pic_nonfinite_check, pic_plan_dump, pic_rerotate, pic_segment_build,
                   pic_segment_prefill, pic_staging_bytes, pic_staging_release, pic_staging_reserve,
                   pic_split_plan, suggest_split)

__all__ = ["FORM_SCALAR", "FORM_DIAG", "FORM_DENSE", "FORM_KDA", "DT_F32", "DT_BF16", "PREC_FP32",
           "PREC_FP16", "PLAN_BUILD",
           "PLAN_COMPOSE", "PicError", "load", "pic_segment_build", "pic_segment_prefill", "pic_compose", "pic_compose_noalloc",
           "pic_compose_seams", "pic_naive_add", "pic_materialize_T", "pic_plan_dump",
           "pic_rerotate", "ROPE_INTERLEAVED", "ROPE_HALF", "pic_conv_warmup",
           "pic_staging_reserve", "pic_staging_release", "pic_staging_bytes", "pic_nonfinite_check",
           "suggest_split", "pic_split_plan"]
