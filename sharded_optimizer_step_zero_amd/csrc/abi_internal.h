// abi_internal.h -- helpers shared by the two C-ABI translation units (abi.cpp,
// offload.cpp): workspace layout, error reporting, hyper-parameter checks.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>

#include "../../include/zeroshard.h"
#include "internal.h"
#include "lds.h"

namespace zs {

// Workspace layout of a plan for these init flags (see zs_workspace_bytes).
WorkspaceLayout plan_workspace(const zs_plan* plan, uint32_t flags);
// The thread's last error message (zero_shard_last_error).
void set_error(const std::string& msg);
// Record the message as the thread's last error and return ZS_EINVAL / ZS_EHIP.
int einval(const char* msg);
int ehip(const char* where, hipError_t e);
// ZS_OK or ZS_EINVAL for the AdamW hyper-parameters and the 1-based step.
int check_hparams(float lr, float beta1, float beta2, float eps, float wd, int64_t step);
// The arguments of a loss-scaled step (hyper-parameters, clip threshold, scaler
// state pointer and rules); fills the finalize parameters.  ZS_OK or ZS_EINVAL.
int check_amp_args(const char* who, float lr, float beta1, float beta2, float eps,
                   float weight_decay, float max_grad_norm, const zs_amp_state* state_dev,
                   float growth_factor, float backoff_factor, int32_t growth_interval,
                   AmpParams* p);
// The LDS reservations of a context on the current device (lds.h), checked
// against its limits; ZS_OK, ZS_EINVAL or ZS_EHIP with the message set.
int make_lds_plan(int32_t M, int64_t shard_len, const char* who, LdsPlan* out);

}  // namespace zs
