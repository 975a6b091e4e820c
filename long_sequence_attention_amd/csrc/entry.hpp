// Internal entry points of the C-ABI host code (api.hip) for the other host
// translation units; not exported.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "vdit_attn.h"

namespace vdit {

// Workspace bytes of a live plan and the device it was created on.
vdit_status_t plan_workspace(vdit_attn_t h, size_t* bytes, int* device);

// vdit_attn_fwd with every check, into the given workspace.
vdit_status_t fwd_into_workspace(vdit_attn_t h, const void* q, const void* k, const void* v, int32_t key_len,
                                 void* out, void* workspace, size_t workspace_bytes, void* hip_stream);

}  // namespace vdit
