// The bf16 forward's forms with a skim tier (Triage's low-precision tier, e4m3
// or MXFP4), compiled on their own so that this translation unit can be
// built without LLVM's machine sinking (see the end of fwd_bf16.hip).
#define SA_FWD_SKIM_TU
#include "fwd_bf16.hip"
