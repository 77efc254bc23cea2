// The backward dQ kernel's packed-document variants (bwd_dq_kernel with
// DOCS = true, launched through launch_dq_docs): kernels.hip compiled a second
// time with BDATTN_DQ_DOCS_UNIT defined, which keeps its kernels and drops its
// launches, so that these variants get a machine scheduler of their own.
#define BDATTN_DQ_DOCS_UNIT
#include "kernels.hip"
